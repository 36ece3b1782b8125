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

// Adjoint summary of segment s >= 1, for a backward over a split sequence.  The adjoint
// recurrence G_t = dy_t C_t + A_bar_{t+1} G_{t+1} does not involve the state, so what a segment
// passes to its left neighbour is affine in the adjoint X entering it from the right: P X + Q,
// with P = exp(A * (sum of the segment's step sizes)).  This kernel computes Q (X = 0) with the
// backward kernel's layout (rows = channels, lanes = 16 consecutive steps of a 256-step chunk,
// states in a loop, chunks from last to first) and the segment's step-size sum (Kahan per lane,
// lanes added in a fixed order); adj_carry_kernel composes the segments from the right.
template <typename IO, bool REV, bool VEC>
__global__ __launch_bounds__(256) void adj_summary_kernel(BwdParams p) {
  using namespace bwdc;
  constexpr int T = 16;                       // steps per lane (a split segment is whole 256-step chunks)
  constexpr int CH = 16 * T;                  // steps per chunk
  constexpr int KG = T / 4;                   // float4 groups per lane
  constexpr int EPC = 16 / (int)sizeof(IO);   // elements per 16-byte piece
  constexpr int PPR = CH / EPC;               // pieces per C row of a chunk
  constexpr int PPT = 16 * PPR / 256;         // C pieces per thread (16 states)
  __shared__ f32x4 ct[16 * KG * 16];          // [state of the stage][float4 group][lane]
  __shared__ float qacc[16 * 64];             // [channel][state]: Q of the chunks done so far
  __shared__ float a2s[16 * 64];              // [channel][state]: A log2(e)

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int r = lane >> 4, g = lane & 15;
  const int S1 = p.S - 1;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = logical % p.nblk;
  const int rest = logical / p.nblk;
  const int seg = 1 + rest % S1;
  const int64_t b = rest / S1;
  const int64_t L = p.L, N = p.N, Dm = p.Dm;
  const int cl = w * 4 + r;
  const int64_t d = (int64_t)cb * 16 + cl;
  const bool dval = d < Dm;
  const int64_t dd = dval ? d : Dm - 1;
  const bool has_z = p.z != nullptr;
  const float biasd = p.bias ? p.bias[dd] : 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t n = g + 16 * k;
    if (n < N) {
      a2s[cl * 64 + n] = p.A[dd * N + n] * kLog2e;
      qacc[cl * 64 + n] = 0.0f;
    }
  }
  const IO* drow = reinterpret_cast<const IO*>(p.delta) + (b * Dm + dd) * L;
  const IO* zrow = has_z ? reinterpret_cast<const IO*>(p.z) + (b * Dm + dd) * L : nullptr;
  const IO* grow = reinterpret_cast<const IO*>(p.dout) + (b * Dm + dd) * L;
  const int64_t tb = (int64_t)seg * p.seg_len;
  const int64_t te = (tb + p.seg_len < L) ? tb + p.seg_len : L;
  const int64_t nch = (te - tb + CH - 1) / CH;
  float dsum = 0.0f, dcomp = 0.0f;

  for (int64_t ci = nch - 1; ci >= 0; --ci) {
    const int64_t c0 = tb + ci * CH;
    const int64_t t0 = c0 + g * T;
    float dt[T], dy[T];
    float cum = 0.0f;
#pragma unroll
    for (int k = 0; k < T / EPC; ++k) {
      float fd[EPC], fg[EPC], fz[EPC];
      load_piece<IO, REV, VEC>(drow, t0 + k * EPC, L, fd);
      load_piece<IO, REV, VEC>(grow, t0 + k * EPC, L, fg);
      if (has_z) load_piece<IO, REV, VEC>(zrow, t0 + k * EPC, L, fz);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int s = k * EPC + e;
        const float dts = (t0 + s < L) ? softplus_(fd[e] + biasd) : 0.0f;  // past the end: identity step
        const float go = dval ? fg[e] : 0.0f;
        dt[s] = dts;
        dy[s] = has_z ? go * (fz[e] * logistic_(fz[e])) : go;
        cum += dts;
      }
    }
    {
      const float y = cum - dcomp;
      const float t = dsum + y;
      dcomp = (t - dsum) - y;
      dsum = t;
    }

    for (int64_t n0 = 0; n0 < N; n0 += 16) {
      __syncthreads();  // every wave is done with the previous stage's tile
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const int q = tid + 256 * k;
        const int nl = q / PPR, pc = q % PPR;
        const int64_t n = n0 + nl;
        float f[EPC];
        if (n < N) {
          load_piece<IO, REV, VEC>(reinterpret_cast<const IO*>(p.C) + (b * N + n) * L, c0 + pc * EPC, L, f);
        } else {
#pragma unroll
          for (int e = 0; e < EPC; ++e) f[e] = 0.0f;
        }
        const int o = pc * EPC, gl = o / T, s0 = o % T;
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
          const f32x4 v = {f[e], f[e + 1], f[e + 2], f[e + 3]};
          ct[(nl * KG + (s0 + e) / 4) * 16 + gl] = v;
        }
      }
      __syncthreads();

      const int ng = (N - n0) < 16 ? (int)(N - n0) : 16;
#pragma unroll 1
      for (int nl = 0; nl < ng; ++nl) {
        const int64_t n = n0 + nl;
        const float A2 = a2s[cl * 64 + n];
        const f32x4* cq = ct + (nl * KG) * 16 + g;
        float a[T];
#pragma unroll
        for (int s = 0; s < T; ++s) a[s] = exp2_(dt[s] * A2);
        // the lane's steps folded from its last, nothing entering from the right
        float QG = 0.0f;
#pragma unroll
        for (int k = KG - 1; k >= 0; --k) {
          const f32x4 cv = cq[k * 16];
#pragma unroll
          for (int e = 3; e >= 0; --e) {
            const int s = 4 * k + e;
            QG = (s == T - 1) ? dy[s] * cv[e] : __builtin_fmaf(a[s + 1 < T ? s + 1 : 0], QG, dy[s] * cv[e]);
          }
        }
        float Qr = a[0] * QG, Pr = exp2_(cum * A2);
        row_scan_from_right(Qr, Pr);
        if (g == 0) qacc[cl * 64 + n] = __builtin_fmaf(Pr, qacc[cl * 64 + n], Qr);
      }
    }
  }

  if (dval) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t n = g + 16 * k;
      if (n < N) p.adj_q[(((int64_t)seg * p.Bsz + b) * Dm + d) * N + n] = qacc[cl * 64 + n];
    }
  }
  float ds = dsum;  // the row's lanes, rotations by 8, 4, 2, 1 (a fixed order; lane 0 keeps it)
  ds += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ds), 0x128 /* row_ror:8 */, 0xf, 0xf, false));
  ds += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ds), 0x124 /* row_ror:4 */, 0xf, 0xf, false));
  ds += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ds), 0x122 /* row_ror:2 */, 0xf, 0xf, false));
  ds += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ds), 0x121 /* row_ror:1 */, 0xf, 0xf, false));
  if (dval && g == 0) p.adj_dsum[((int64_t)seg * p.Bsz + b) * Dm + d] = ds;
}

// adj_in[s] = adjoint entering segment s from the right: the final-state gradient (or zero)
// for the last segment, then X_{s-1} = exp(A * dsum_s) X_s + Q_s.
__global__ __launch_bounds__(256) void adj_carry_kernel(BwdParams p, float* adj_in) {
  const int64_t BDN = p.Bsz * p.Dm * p.N;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= BDN) return;
  const int64_t n = idx % p.N, bd = idx / p.N, d = bd % p.Dm;
  const float A2 = p.A[d * p.N + n] * kLog2e;
  float x = p.dfinal ? p.dfinal[idx] : 0.0f;
  for (int s = p.S - 1; s >= 0; --s) {
    adj_in[(int64_t)s * BDN + idx] = x;
    if (s > 0) {
      const float decay = exp2_(A2 * p.adj_dsum[(int64_t)s * p.Bsz * p.Dm + bd]);
      x = __builtin_fmaf(decay, x, p.adj_q[(int64_t)s * BDN + idx]);
    }
  }
}

template <typename IO>
static void go_adj_summary(const BwdParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.Bsz * p.nblk * (p.S - 1)));
  const int k = (p.reverse ? 2 : 0) + (p.vec ? 1 : 0);
  switch (k) {
    case 0: hipLaunchKernelGGL((adj_summary_kernel<IO, false, false>), grid, dim3(256), 0, s, p); break;
    case 1: hipLaunchKernelGGL((adj_summary_kernel<IO, false, true>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((adj_summary_kernel<IO, true, false>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((adj_summary_kernel<IO, true, true>), grid, dim3(256), 0, s, p); break;
  }
}

hipError_t launch_adj_summary(const BwdParams& p, bool bf16, hipStream_t s) {
  if (bf16) go_adj_summary<bf16_t>(p, s);
  else go_adj_summary<float>(p, s);
  return hipGetLastError();
}

hipError_t launch_adj_carry(const BwdParams& p, float* adj_in, hipStream_t s) {
  const int64_t BDN = p.Bsz * p.Dm * p.N;
  hipLaunchKernelGGL(adj_carry_kernel, dim3((unsigned)((BDN + 255) / 256)), dim3(256), 0, s, p, adj_in);
  return hipGetLastError();
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
