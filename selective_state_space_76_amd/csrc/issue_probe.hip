// issue_probe.hip -- measurement helper for bench.py (not part of the scan library's ABI).
//
// Times long runs of one kind of wave64 fp32 VALU instruction on every SIMD of the GPU, so the
// benchmark can state what issue rate the scan's instruction mix is held to: the published fp32
// vector peak counts packed (two-per-lane) FMAs, which this library's kernels are built without.
// Each lane runs 8 independent chains (no dependency stalls); one workgroup of 4 waves per CU and
// per requested wave per SIMD.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

#define PROBE_X8(X) X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7)

template <int KIND>
__global__ __launch_bounds__(256) void probe_kernel(float* out, int iters) {
  float a0 = 0.5f + threadIdx.x * 1e-3f, a1 = a0 + 0.1f, a2 = a0 + 0.2f, a3 = a0 + 0.3f;
  float a4 = a0 + 0.4f, a5 = a0 + 0.5f, a6 = a0 + 0.6f, a7 = a0 + 0.7f;
  const float m = 0.999f, c = 0.001f;
  for (int i = 0; i < iters; ++i) {
    if constexpr (KIND == 0) {  // 64 x v_fma_f32
#define PROBE_F(j) "v_fma_f32 %" #j ", %" #j ", %8, %9\n"
      asm volatile(PROBE_X8(PROBE_F) PROBE_X8(PROBE_F) PROBE_X8(PROBE_F) PROBE_X8(PROBE_F)
                   PROBE_X8(PROBE_F) PROBE_X8(PROBE_F) PROBE_X8(PROBE_F) PROBE_X8(PROBE_F)
                   : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                   : "v"(m), "v"(c));
#undef PROBE_F
    } else {  // 64 x v_exp_f32 (argument kept in (-inf, 0] so values stay bounded)
#define PROBE_F(j) "v_exp_f32 %" #j ", -|%" #j "|\n"
      asm volatile(PROBE_X8(PROBE_F) PROBE_X8(PROBE_F) PROBE_X8(PROBE_F) PROBE_X8(PROBE_F)
                   PROBE_X8(PROBE_F) PROBE_X8(PROBE_F) PROBE_X8(PROBE_F) PROBE_X8(PROBE_F)
                   : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
#undef PROBE_F
    }
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
}

}  // namespace

extern "C" {

// kind 0: v_fma_f32, 1: v_exp_f32.  waves_per_simd in [1, 8].  On success returns 0 and writes
// the SIMD cycles per wave64 instruction at clock_ghz (event time x clock / instructions per SIMD)
// and the elapsed milliseconds; -1 on bad arguments, -2 on a HIP error.
int ssm_probe_issue(int kind, int waves_per_simd, int iters, double clock_ghz, double* clk_per_instr,
                    double* ms_out) {
  if ((kind != 0 && kind != 1) || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 || !clk_per_instr)
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
    else hipLaunchKernelGGL(probe_kernel<1>, dim3(blocks), dim3(256), 0, nullptr, out, iters);
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
