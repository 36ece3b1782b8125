// issue_probe.hip -- measurement helper for bench.py (not part of the scan library's ABI).
//
// Times long runs of one kind of wave64 fp32 VALU instruction on every SIMD of the GPU, so the
// benchmark can state the issue rates the scan's instruction mix is held to: plain VALU work
// (v_fma_f32), the transcendental v_exp_f32, and a multiply whose operand comes through a DPP row
// broadcast.  The loop is written in assembly with fixed registers: 8 independent chains in
// registers of VGPR banks 2 and 3, the shared operands in banks 0 and 1, so no instruction reads
// two operands from one bank (which costs extra cycles).  One workgroup of 4 waves per CU per
// requested wave per SIMD.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

#define PROBE_REP8(X) X X X X X X X X
#define PROBE_FMA8                                                                                         \
  "v_fma_f32 v42, v42, v48, v49\n v_fma_f32 v43, v43, v48, v49\n v_fma_f32 v46, v46, v48, v49\n"           \
  "v_fma_f32 v47, v47, v48, v49\n v_fma_f32 v50, v50, v48, v49\n v_fma_f32 v51, v51, v48, v49\n"           \
  "v_fma_f32 v54, v54, v48, v49\n v_fma_f32 v55, v55, v48, v49\n"
#define PROBE_EXP8                                                                                         \
  "v_exp_f32 v42, -|v42|\n v_exp_f32 v43, -|v43|\n v_exp_f32 v46, -|v46|\n v_exp_f32 v47, -|v47|\n"       \
  "v_exp_f32 v50, -|v50|\n v_exp_f32 v51, -|v51|\n v_exp_f32 v54, -|v54|\n v_exp_f32 v55, -|v55|\n"
#define PROBE_DPP(r) "v_mul_f32_dpp " r ", " r ", v48 row_newbcast:3 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
#define PROBE_DPP8                                                                                         \
  PROBE_DPP("v42") PROBE_DPP("v43") PROBE_DPP("v46") PROBE_DPP("v47") PROBE_DPP("v50") PROBE_DPP("v51")   \
  PROBE_DPP("v54") PROBE_DPP("v55")
#define PROBE_INIT                                                                                         \
  "v_mov_b32 v42, 0.5\n v_mov_b32 v43, 0.5\n v_mov_b32 v46, 0.5\n v_mov_b32 v47, 0.5\n"                   \
  "v_mov_b32 v50, 0.5\n v_mov_b32 v51, 0.5\n v_mov_b32 v54, 0.5\n v_mov_b32 v55, 0.5\n"                   \
  "v_mov_b32 v48, 0.999\n v_mov_b32 v49, 0.001\n s_mov_b32 s20, %1\n s_nop 1\n"
#define PROBE_LOOP(BODY)                                                                                   \
  asm volatile(PROBE_INIT "1:\n" BODY "s_sub_u32 s20, s20, 1\n s_cmp_lg_u32 s20, 0\n s_cbranch_scc1 1b\n"  \
               "v_add_f32 %0, v42, v55\n"                                                                  \
               : "=v"(r)                                                                                   \
               : "s"(iters)                                                                                \
               : "v42", "v43", "v46", "v47", "v48", "v49", "v50", "v51", "v54", "v55", "s20", "scc")

template <int KIND>
__global__ __launch_bounds__(256) void probe_kernel(float* out, int iters) {
  float r = 0.0f;
  if constexpr (KIND == 0) PROBE_LOOP(PROBE_REP8(PROBE_FMA8));
  if constexpr (KIND == 1) PROBE_LOOP(PROBE_REP8(PROBE_EXP8));
  if constexpr (KIND == 2) PROBE_LOOP(PROBE_REP8(PROBE_DPP8));
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
}

}  // namespace

extern "C" {

// kind 0: v_fma_f32, 1: v_exp_f32, 2: v_mul_f32 with a DPP row-broadcast operand; 64 instructions
// per loop iteration.  waves_per_simd in [1, 8].  On success returns 0 and writes the SIMD cycles per
// wave64 instruction at clock_ghz (event time x clock / instructions per SIMD) and the elapsed
// milliseconds; -1 on bad arguments, -2 on a HIP error.
int ssm_probe_issue(int kind, int waves_per_simd, int iters, double clock_ghz, double* clk_per_instr,
                    double* ms_out) {
  if (kind < 0 || kind > 2 || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 || !clk_per_instr)
    return -1;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return -2;
  const int blocks = prop.multiProcessorCount * waves_per_simd;
  float* out = nullptr;
  if (hipMalloc(&out, sizeof(float) * 256 * (size_t)blocks) != hipSuccess) return -2;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  float ms = 0.0f;
  for (int rep = 0; rep < 3 && err == hipSuccess; ++rep) {  // the last repetition is timed
    err = hipEventRecord(e0, nullptr);
    if (kind == 0) hipLaunchKernelGGL(probe_kernel<0>, dim3(blocks), dim3(256), 0, nullptr, out, iters);
    else if (kind == 1) hipLaunchKernelGGL(probe_kernel<1>, dim3(blocks), dim3(256), 0, nullptr, out, iters);
    else hipLaunchKernelGGL(probe_kernel<2>, dim3(blocks), dim3(256), 0, nullptr, out, iters);
    if (err == hipSuccess) err = hipGetLastError();
    if (err == hipSuccess) err = hipEventRecord(e1, nullptr);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(out);
  if (err != hipSuccess) return -2;
  const double instr_per_simd = 64.0 * iters * waves_per_simd;
  *clk_per_instr = ms * 1e-3 * clock_ghz * 1e9 / instr_per_simd;
  if (ms_out) *ms_out = ms;
  return 0;
}

}  // extern "C"
