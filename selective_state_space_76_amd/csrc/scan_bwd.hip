// scan_bwd.hip -- launches of the backward pass of the selective scan with the default
// discretisation (B_bar = dt B), and the fixed-order partial-sum pass shared by both
// discretisations.  The kernels and their derivation are in scan_bwd_kernel.h; the
// zero-order-hold variants are compiled in scan_bwd_zoh.hip.
#include "scan_bwd_kernel.h"

namespace ssm {

// out[i] = sum over k of part[k * stride + i], k ascending (the same order on every run).
// V4: 4 consecutive outputs per lane with 16-byte loads (stride and n multiples of 4); the
// loads of 8 consecutive k are issued before their adds, which keep the k order.
template <bool V4>
__global__ __launch_bounds__(256) void reduce_kernel(float* out, const float* part, int64_t count,
                                                     int64_t stride, int64_t n) {
  constexpr int W = V4 ? 4 : 1;
  constexpr int U = 8;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * W;
  if (i >= n) return;
  float acc[W];
#pragma unroll
  for (int e = 0; e < W; ++e) acc[e] = 0.0f;
  int64_t k = 0;
  for (; k + U <= count; k += U) {
    float v[U][W];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* q = part + (k + u) * stride + i;
      if constexpr (V4) {
        const float4 t = *reinterpret_cast<const float4*>(q);
        v[u][0] = t.x; v[u][1] = t.y; v[u][2] = t.z; v[u][3] = t.w;
      } else {
        v[u][0] = *q;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < W; ++e) acc[e] += v[u][e];
  }
  for (; k < count; ++k) {
    const float* q = part + k * stride + i;
#pragma unroll
    for (int e = 0; e < W; ++e) acc[e] += q[e];
  }
  if constexpr (V4) *reinterpret_cast<float4*>(out + i) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  else out[i] = acc[0];
}

hipError_t launch_ckpt(const ScanParams& p, bool bf16, hipStream_t s) {
  return p.zoh ? launch_ckpt_zoh(p, bf16, s) : go_ckpt_all<false>(p, bf16, s);
}

hipError_t launch_bwd(const BwdParams& p, bool bf16, hipStream_t s) {
  return p.zoh ? launch_bwd_zoh(p, bf16, s) : go_bwd_all<false>(p, bf16, s);
}

hipError_t launch_reduce(float* out, const float* part, int64_t count, int64_t stride, int64_t n, hipStream_t s) {
  // 16-byte path when every row start stays 16-byte aligned (bases are 16-byte aligned)
  if (stride % 4 == 0 && n % 4 == 0) {
    const int64_t lanes = n / 4;
    hipLaunchKernelGGL((reduce_kernel<true>), dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, out, part,
                       count, stride, n);
  } else {
    hipLaunchKernelGGL((reduce_kernel<false>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, out, part,
                       count, stride, n);
  }
  return hipGetLastError();
}

}  // namespace ssm
