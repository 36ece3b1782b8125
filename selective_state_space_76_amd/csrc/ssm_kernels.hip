// ssm_kernels.hip -- launchers: scan dispatch, carry pass and the decode step.
#include "ssm_device.h"

namespace ssm {

// Chains the segment summaries: carries[s] is the state entering segment s.
__global__ __launch_bounds__(256) void carry_kernel(ScanParams p) {
  const int64_t BDN = p.Bsz * p.Dm * p.N;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= BDN) return;
  const int64_t n = idx % p.N, bd = idx / p.N, d = bd % p.Dm;
  const float Ap = p.A[d * p.N + n] * kLog2e;
  float hc = p.init ? p.init[idx] : 0.0f;
  for (int s = 0; s < p.S; ++s) {
    p.carries[(int64_t)s * BDN + idx] = hc;
    if (s + 1 < p.S) {
      const float decay = exp2_(Ap * p.seg_dsum[(int64_t)s * p.Bsz * p.Dm + bd]);
      hc = __builtin_fmaf(decay, hc, p.seg_state[(int64_t)s * BDN + idx]);
    }
  }
}

hipError_t launch_scan_f32_out(const ScanParams& p, int grid, hipStream_t s);
hipError_t launch_scan_f32_sum(const ScanParams& p, int grid, hipStream_t s);
hipError_t launch_scan_bf16_out(const ScanParams& p, int grid, hipStream_t s);
hipError_t launch_scan_bf16_sum(const ScanParams& p, int grid, hipStream_t s);

hipError_t launch_scan(const ScanParams& p, bool bf16, int mode, hipStream_t s) {
  const int64_t base = p.Bsz * p.nblk;
  const int grid = (int)(base * (mode == 0 ? p.S : p.S - 1));
  if (bf16) return mode == 0 ? launch_scan_bf16_out(p, grid, s) : launch_scan_bf16_sum(p, grid, s);
  return mode == 0 ? launch_scan_f32_out(p, grid, s) : launch_scan_f32_sum(p, grid, s);
}

hipError_t launch_carry(const ScanParams& p, hipStream_t s) {
  const int64_t BDN = p.Bsz * p.Dm * p.N;
  hipLaunchKernelGGL(carry_kernel, dim3((unsigned)((BDN + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename IO, int G>
static hipError_t launch_step_g(const StepParams& p, hipStream_t s) {
  const int64_t threads = p.Bsz * p.Dm * G;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (p.zoh) hipLaunchKernelGGL((step_kernel<IO, G, true>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((step_kernel<IO, G, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename IO, int G>
static hipError_t launch_step4_g(const StepParams& p, hipStream_t s) {
  constexpr int U = 2;  // batch rows per lane (measured best of 2, 4, 8 at 256 x 5120 x 16)
  const int64_t lanes = (p.Bsz + U - 1) / U * p.Dm * G;  // each lane serves U batch rows of one channel
  const dim3 grid((unsigned)((lanes + 255) / 256));
  if (p.zoh) hipLaunchKernelGGL((step4_kernel<IO, G, U, true>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((step4_kernel<IO, G, U, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_step_io(const StepParams& p, hipStream_t s) {
  const int64_t quads = (p.N + 3) / 4;
  if (p.vec) {  // N a multiple of 4: whole 16-byte state quads
    if (quads <= 1) return launch_step4_g<IO, 1>(p, s);
    if (quads <= 2) return launch_step4_g<IO, 2>(p, s);
    if (quads <= 4) return launch_step4_g<IO, 4>(p, s);
    if (quads <= 8) return launch_step4_g<IO, 8>(p, s);
    return launch_step4_g<IO, 16>(p, s);
  }
  if (quads <= 1) return launch_step_g<IO, 1>(p, s);
  if (quads <= 2) return launch_step_g<IO, 2>(p, s);
  if (quads <= 4) return launch_step_g<IO, 4>(p, s);
  if (quads <= 8) return launch_step_g<IO, 8>(p, s);
  return launch_step_g<IO, 16>(p, s);
}

hipError_t launch_step(const StepParams& p, bool bf16, hipStream_t s) {
  return bf16 ? launch_step_io<bf16_t>(p, s) : launch_step_io<float>(p, s);
}

}  // namespace ssm
