// ssm_kernels.hip -- launchers: scan dispatch, carry pass and the decode step; the scratch
// memory of the entry point that allocates nothing.
#include <mutex>

#include "ssm_device.h"

namespace ssm {

// Scratch memory of ssm_scan_fwd_noalloc: a file-scope device array, so the call needs no
// allocation.  Each GPU the library runs on holds its own copy, at its own address, until the
// process ends.  In host code the name `scratch` is only a stand-in for the symbol; its device
// address comes from hipGetSymbolAddress, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_buffer(hipStream_t stream, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {  // the device the work will run on
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;  // the symbol of that device
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// Chains the segment summaries: carries[s] is the state entering segment s.  seg_state may lie in
// the carries' own slots 1 .. S-1 (segment s's end state where the state entering segment s + 1
// goes).  The summaries are read 8 segments at a time before the chain over them runs, so a lane's
// loads are not serialised behind its stores; every slot is read before it is overwritten, so the
// chain also runs in place.
__global__ __launch_bounds__(256) void carry_kernel(ScanParams p) {
  constexpr int G = 8;
  const int64_t BDN = p.Bsz * p.Dm * p.N;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= BDN) return;
  const int64_t n = idx % p.N, bd = idx / p.N, d = bd % p.Dm;
  const float Ap = p.A[d * p.N + n] * kLog2e;
  float hc = p.init ? p.init[idx] : 0.0f;
  for (int s0 = 0; s0 < p.S; s0 += G) {
    float st[G], ds[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {  // the end states and step-size sums of segments s0 .. s0 + G - 1
      const int s = s0 + k;
      st[k] = s + 1 < p.S ? p.seg_state[(int64_t)s * BDN + idx] : 0.0f;
      ds[k] = s + 1 < p.S ? p.seg_dsum[(int64_t)s * p.Bsz * p.Dm + bd] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int s = s0 + k;
      if (s < p.S) {
        p.carries[(int64_t)s * BDN + idx] = hc;
        if (s + 1 < p.S) hc = __builtin_fmaf(exp2_(Ap * ds[k]), hc, st[k]);
      }
    }
  }
}

// The same chain over at most 32 x GR segments, in two levels: a workgroup holds CW = 1024 / GR
// consecutive (b, d, n) chains and GR groups of K consecutive segments; thread (group, chain) folds
// its segments into (P, Q) = (product of the decays, state reached from zero), the groups' pairs go
// through LDS, each thread composes the groups to its left (in order) with the initial state and
// reruns its own segments, writing their carries.  Every summary a workgroup reads is loaded and
// used by the fold before the barrier, and every carry is stored after it, so this also runs in
// place.
template <int K, int GR>
__global__ __launch_bounds__(1024) void carry_tree_kernel(ScanParams p) {
  constexpr int CW = 1024 / GR;
  __shared__ float sp[GR][CW], sq[GR][CW];
  const int c = threadIdx.x % CW, gr = threadIdx.x / CW;
  const int64_t BDN = p.Bsz * p.Dm * p.N;
  const int64_t idx = (int64_t)blockIdx.x * CW + c;
  const bool v = idx < BDN;
  const int64_t ix = v ? idx : 0;
  const int64_t n = ix % p.N, bd = ix / p.N, d = bd % p.Dm;
  const float Ap = p.A[d * p.N + n] * kLog2e;
  const int s0 = gr * K;
  float st[K], dec[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {  // the last segment has no summary: an identity step
    const int s = s0 + k;
    const bool has = s + 1 < p.S;
    st[k] = has ? p.seg_state[(int64_t)s * BDN + ix] : 0.0f;
    const float ds = has ? p.seg_dsum[(int64_t)s * p.Bsz * p.Dm + bd] : 0.0f;
    dec[k] = has ? exp2_(Ap * ds) : 1.0f;
  }
  float P = 1.0f, Q = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    Q = __builtin_fmaf(dec[k], Q, st[k]);
    P *= dec[k];
  }
  sp[gr][c] = P;
  sq[gr][c] = Q;
  __syncthreads();
  float hc = (v && p.init) ? p.init[ix] : 0.0f;
  for (int j = 0; j < gr; ++j) hc = __builtin_fmaf(sp[j][c], hc, sq[j][c]);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int s = s0 + k;
    if (v && s < p.S) p.carries[(int64_t)s * BDN + ix] = hc;
    hc = __builtin_fmaf(dec[k], hc, st[k]);
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

template <int K, int GR>
static void launch_carry_tree(const ScanParams& p, hipStream_t s) {
  constexpr int CW = 1024 / GR;
  const int64_t BDN = p.Bsz * p.Dm * p.N;
  hipLaunchKernelGGL((carry_tree_kernel<K, GR>), dim3((unsigned)((BDN + CW - 1) / CW)), dim3(1024), 0, s, p);
}

hipError_t launch_carry(const ScanParams& p, hipStream_t s) {
  const int64_t BDN = p.Bsz * p.Dm * p.N;
  // two levels up to 1024 segments (each thread's segments in registers); a chain per thread beyond
  if (p.S <= 64) launch_carry_tree<4, 16>(p, s);
  else if (p.S <= 128) launch_carry_tree<8, 16>(p, s);
  else if (p.S <= 256) launch_carry_tree<16, 16>(p, s);
  else if (p.S <= 512) launch_carry_tree<32, 16>(p, s);
  else if (p.S <= 1024) launch_carry_tree<32, 32>(p, s);
  else hipLaunchKernelGGL(carry_kernel, dim3((unsigned)((BDN + 255) / 256)), dim3(256), 0, s, p);
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
