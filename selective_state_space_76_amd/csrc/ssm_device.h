// ssm_device.h -- gfx950 device code of the selective state-space scan (kernel templates).
//
// Operation (see include/ssm_scan.h for the full statement and its sources):
//   dt = softplus(delta + bias[d]); A_bar = exp(dt*A[d,n]); B_bar = dt*B[n]
//   (or the zero-order-hold B_bar); h = A_bar*h + B_bar*u; y = C.h + D*u;
//   out = y*silu(z).  Selective step: fsdata.site "mamba-state-space-model",
//   section 3.2; bias inside the softplus and per-channel independence:
//   freeguideonline.com Mamba tutorial, sections 4.2 and 4.3; fusing the
//   discretisation into the scan and keeping the expanded state on chip:
//   same tutorial, section 5.2.
//
// Work layout of the scan kernel (one design for every shape):
//   * A workgroup is 4 waves; a wave is 4 rows of 16 lanes; a row owns one
//     channel (b, d), so a workgroup covers 16 consecutive channels of one
//     batch row.  Lane g of a row holds the states n = g + 16*i, i < NL, in
//     registers for the whole sequence (NL = ceil(N/16)).
//   * The sequence is walked in blocks of 64 steps, split in 4 sub-blocks of
//     16.  Lane g owns step g of each sub-block: it loads delta/u/z for that
//     step, computes dt = softplus(.) and dt*u once, and later finishes the
//     output of that step.  Inside a sub-block the row reads step j's dt and
//     dt*u from lane j with a DPP row broadcast (row_newbcast), so each
//     (channel, step) value is computed once, not once per state.
//   * Per state update: one multiply for the exp2 argument, v_exp_f32, one
//     multiply for B_bar*u, one FMA for h and one FMA for C*h.  The sum over
//     n of C*h is a 16 x 16 transpose through LDS (wave-local, no barrier).
//   * Sequences with too few channels to fill the chip are cut into S
//     segments: a summary pass scans each segment from a zero state and keeps
//     its end state and the sum of its step sizes, a carry pass chains the
//     segments (h_in[s+1] = exp(A*sum dt_s)*h_in[s] + h_end[s], the same
//     composition the associative scan uses), and the output pass rescans each
//     segment from its carry.  Exactness follows from associativity of that
//     composition (freeguideonline tutorial, section 5.1).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_launch.h"

namespace ssm {

typedef uint16_t bf16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ void store_io(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_io(bf16_t* p, float v) {
  *p = __builtin_bit_cast(bf16_t, (__bf16)v);  // v_cvt_pk_bf16_f32: round to nearest even
}

// log(1 + e^x).  Above 20 the answer is x to within 2e-9 relative.  Below,
// log1p(e) is formed as log(w) * e / (w - 1) with w = 1 + e, which cancels the
// rounding error of w when e is small (Goldberg, "What every computer
// scientist should know about floating-point arithmetic", theorem 4).
__device__ __forceinline__ float softplus_(float x) {
  const float e = exp2_(x * kLog2e);
  const float w = 1.0f + e;
  const float wm1 = w - 1.0f;
  const float l = log2_(w) * kLn2;
  const float r = (wm1 == 0.0f) ? e : l * (e * rcp_(wm1));
  return x > 20.0f ? x : r;
}

__device__ __forceinline__ float silu_(float z) { return z * rcp_(1.0f + exp2_(-z * kLog2e)); }

// (exp(x) - 1) / x, accurate near 0 (Taylor terms to x^3 when |x| < 0.03).
__device__ __forceinline__ float expm1_over_x(float x, float ex) {
  const float series = 1.0f + x * (0.5f + x * (0.16666667f + x * 0.041666668f));
  return (fabsf(x) < 0.03f) ? series : (ex - 1.0f) * rcp_(x);
}

template <int V> struct IC { static constexpr int value = V; };
template <int I, int E, typename F> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(IC<I>{});
    static_for<I + 1, E>(f);
  }
}

// broadcast lane J of each 16-lane row to the whole row
template <int J> __device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x150 + J, 0xf, 0xf, false));
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroups are dispatched round-robin over the 8 XCDs.  Renumber them so that
// each XCD receives a contiguous range of logical blocks: neighbouring channel
// blocks of one batch row share their B/C rows through that XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int G) {
  const int per = G / 8, rem = G % 8;
  const int xcd = i % 8, k = i / 8;
  return xcd < rem ? xcd * (per + 1) + k : rem * (per + 1) + (xcd - rem) * per + k;
}

// Load the values of 8 consecutive logical steps t..t+7 of one row into v[0..7].
// `vec` means the row length and t are multiples of 8 (bf16) / 4 (fp32) and the
// row is 16-byte aligned.  Steps past the row end are clamped (their values are
// never used: dt is zero there).
template <typename IO, bool REV>
__device__ __forceinline__ void load8(const IO* row, int64_t t, int64_t L, bool vec, float v[8]) {
  if (vec) {
    const int64_t base = t < L - 8 ? t : L - 8;       // logical index of v[0]
    const int64_t pb = REV ? (L - 8 - base) : base;   // physical start of the 8-element run
    float w[8];
    if constexpr (sizeof(IO) == 2) {
      const uint4 q = *reinterpret_cast<const uint4*>(row + pb);
      const uint32_t x[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w[2 * k] = __uint_as_float(x[k] << 16);
        w[2 * k + 1] = __uint_as_float(x[k] & 0xffff0000u);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4*>(row + pb);
      const float4 b = *reinterpret_cast<const float4*>(row + pb + 4);
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
      w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = REV ? w[7 - k] : w[k];
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int64_t tk = t + k;
      tk = tk < L ? tk : L - 1;
      v[k] = to_f32(row[REV ? (L - 1 - tk) : tk]);
    }
  }
}

// ------------------------------------------------------------- scan kernel
//
// MODE 0: output pass (writes out and, for the last segment, final_state).
// MODE 1: summary pass over segments 0..S-2 (writes seg_state and seg_dsum).
template <typename IO, int NL, bool FULLN, int MODE, bool ZOH, bool REV>
__global__ __launch_bounds__(256, MODE == 0 ? 3 : 2) void scan_kernel(ScanParams p) {
  constexpr int RSTRIDE = 20;                   // floats per LDS transpose row (16 + pad, 16 B aligned)
  constexpr int GSTRIDE = 16 * RSTRIDE + 4;     // floats per channel row
  __shared__ float red[MODE == 0 ? 16 * GSTRIDE : 1];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane >> 4, g = lane & 15;
  const int S_launch = MODE == 0 ? p.S : p.S - 1;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = logical % p.nblk;
  const int rest = logical / p.nblk;
  const int seg = rest % S_launch;
  const int64_t b = rest / S_launch;
  const int64_t L = p.L, N = p.N, Dm = p.Dm;
  const int64_t d = (int64_t)cb * 16 + w * 4 + r;
  const bool dval = d < Dm;
  const int64_t dd = dval ? d : Dm - 1;
  const int64_t tb = (int64_t)seg * p.seg_len;
  const int64_t te = (tb + p.seg_len < L) ? tb + p.seg_len : L;
  const bool vec = p.vec != 0;

  const IO* urow = reinterpret_cast<const IO*>(p.u) + (b * Dm + dd) * L;
  const IO* drow = reinterpret_cast<const IO*>(p.delta) + (b * Dm + dd) * L;
  const IO* zrow = p.z ? reinterpret_cast<const IO*>(p.z) + (b * Dm + dd) * L : nullptr;
  IO* orow = MODE == 0 ? reinterpret_cast<IO*>(p.out) + (b * Dm + dd) * L : nullptr;
  const float biasd = p.bias ? p.bias[dd] : 0.0f;
  const float Dd = p.D ? p.D[dd] : 0.0f;

  float Ap[NL], Aln[NL], h[NL];
  bool nval[NL];
  const IO* Brow[NL];
  const IO* Crow[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int64_t n = g + 16 * i;
    nval[i] = FULLN || n < N;
    const int64_t nn = nval[i] ? n : N - 1;
    const float a = p.A[dd * N + nn];
    Aln[i] = nval[i] ? a : 0.0f;
    Ap[i] = Aln[i] * kLog2e;
    float h0 = 0.0f;
    if (MODE == 0) {
      if (p.carries) h0 = p.carries[(((int64_t)seg * p.Bsz + b) * Dm + dd) * N + nn];
      else if (p.init) h0 = p.init[(b * Dm + dd) * N + nn];
    }
    h[i] = nval[i] ? h0 : 0.0f;
    Brow[i] = reinterpret_cast<const IO*>(p.B) + (b * N + nn) * L;
    Crow[i] = reinterpret_cast<const IO*>(p.C) + (b * N + nn) * L;
  }
  float* rb = &red[MODE == 0 ? (w * 4 + r) * GSTRIDE : 0];
  float dsum = 0.0f, dcomp = 0.0f;  // Kahan sum of dt over this lane's steps (summary pass)

  for (int64_t t0 = tb; t0 < te; t0 += 64) {
    // ---- per (channel, step) work for the 4 steps this lane owns in the block
    float dl[4], xu[4], uu[4], zz[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t t = t0 + 16 * s + g;
      const bool tv = t < te;
      const int64_t tc = tv ? t : te - 1;
      const int64_t tp = REV ? (L - 1 - tc) : tc;
      const float dt = tv ? softplus_(to_f32(drow[tp]) + biasd) : 0.0f;
      const float uv = to_f32(urow[tp]);
      dl[s] = dt;
      uu[s] = uv;
      xu[s] = ZOH ? uv : dt * uv;
      zz[s] = (MODE == 0 && zrow) ? to_f32(zrow[tp]) : 0.0f;
      if (MODE == 1) {
        const float yk = dt - dcomp;
        const float tk = dsum + yk;
        dcomp = (tk - dsum) - yk;
        dsum = tk;
      }
    }
    // ---- the recurrence, 16 steps at a time
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float pj[16];
#pragma unroll
      for (int jc = 0; jc < 16; jc += 8) {
        float Bv[NL][8], Cv[NL][8];
        const int64_t tq = t0 + 16 * s + jc;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          load8<IO, REV>(Brow[i], tq, L, vec, Bv[i]);
          if (MODE == 0) load8<IO, REV>(Crow[i], tq, L, vec, Cv[i]);
          if (!FULLN && !nval[i]) {
#pragma unroll
            for (int k = 0; k < 8; ++k) { Bv[i][k] = 0.0f; Cv[i][k] = 0.0f; }
          }
        }
        static_for<0, 8>([&](auto jj_) {
          constexpr int jj = decltype(jj_)::value;
          constexpr int j = jj;  // position within the 8-step chunk; the row lane is jc + jj
          float dj, xj;
          if (jc == 0) { dj = row_bcast<j>(dl[s]); xj = row_bcast<j>(xu[s]); }
          else { dj = row_bcast<j + 8>(dl[s]); xj = row_bcast<j + 8>(xu[s]); }
          float acc = 0.0f;
#pragma unroll
          for (int i = 0; i < NL; ++i) {
            const float a = exp2_(dj * Ap[i]);
            float x;
            if (ZOH) {
              const float arg = dj * Aln[i];
              x = (dj * expm1_over_x(arg, a)) * (xj * Bv[i][jj]);
            } else {
              x = xj * Bv[i][jj];
            }
            h[i] = __builtin_fmaf(a, h[i], x);
            if (MODE == 0) acc = __builtin_fmaf(Cv[i][jj], h[i], acc);
          }
          pj[jc + jj] = acc;
        });
      }
      if (MODE == 0) {
        // ---- sum over states: row g of the [step][state] tile holds step g's terms
#pragma unroll
        for (int j = 0; j < 16; ++j) rb[j * RSTRIDE + g] = pj[j];
        wave_sync();
        const float4 q0 = *reinterpret_cast<const float4*>(rb + g * RSTRIDE + 0);
        const float4 q1 = *reinterpret_cast<const float4*>(rb + g * RSTRIDE + 4);
        const float4 q2 = *reinterpret_cast<const float4*>(rb + g * RSTRIDE + 8);
        const float4 q3 = *reinterpret_cast<const float4*>(rb + g * RSTRIDE + 12);
        wave_sync();
        const float y0 = ((q0.x + q0.y) + (q0.z + q0.w)) + ((q1.x + q1.y) + (q1.z + q1.w));
        const float y1 = ((q2.x + q2.y) + (q2.z + q2.w)) + ((q3.x + q3.y) + (q3.z + q3.w));
        const int64_t t = t0 + 16 * s + g;
        if (dval && t < te) {
          float y = (y0 + y1) + Dd * uu[s];
          if (zrow) y *= silu_(zz[s]);
          store_io(orow + (REV ? (L - 1 - t) : t), y);
        }
      }
    }
  }

  if (MODE == 0) {
    if (p.final_state && seg == p.S - 1 && dval) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (nval[i]) p.final_state[(b * Dm + d) * N + g + 16 * i] = h[i];
    }
  } else {
    // row sum of the lanes' step-size sums
    float ds = dsum;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) ds += __shfl_xor(ds, off, 16);
    const int64_t bd = b * Dm + d;
    if (dval) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (nval[i]) p.seg_state[((int64_t)seg * p.Bsz * Dm) * N + bd * N + g + 16 * i] = h[i];
      if (g == 0) p.seg_dsum[(int64_t)seg * p.Bsz * Dm + bd] = ds;
    }
  }
}

// ----------------------------------------------------------- decode kernel
//
// One generation step.  G lanes per channel, 4 states per lane (N <= 4*G); the
// state row is read and written with 16-byte accesses, so a wave streams
// contiguous memory.  y = sum_n C*h is a butterfly over the G lanes.
template <typename IO, int G, bool ZOH>
__global__ __launch_bounds__(256) void step_kernel(StepParams p) {
  const int64_t BD = p.Bsz * p.Dm;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t c = gid / G;
  const int q = (int)(gid % G);
  const bool cval = c < BD;
  const int64_t cc = cval ? c : BD - 1;
  const int64_t b = cc / p.Dm, d = cc % p.Dm;
  const int64_t N = p.N;
  const float dt = softplus_(to_f32(reinterpret_cast<const IO*>(p.delta)[cc]) + (p.bias ? p.bias[d] : 0.0f));
  const float uv = to_f32(reinterpret_cast<const IO*>(p.u)[cc]);
  const IO* Bp = reinterpret_cast<const IO*>(p.B) + b * N;
  const IO* Cp = reinterpret_cast<const IO*>(p.C) + b * N;
  const int64_t n0 = 4 * (int64_t)q;
  float hv[4] = {0.f, 0.f, 0.f, 0.f}, Av[4] = {0.f, 0.f, 0.f, 0.f};
  float Bv[4] = {0.f, 0.f, 0.f, 0.f}, Cv[4] = {0.f, 0.f, 0.f, 0.f};
  float* st = p.state + cc * N + n0;
  const bool vec4 = p.vec != 0 && n0 < N;  // N % 4 == 0: whole quads
  if (vec4) {
    const float4 hq = *reinterpret_cast<const float4*>(st);
    const float4 aq = *reinterpret_cast<const float4*>(p.A + d * N + n0);
    hv[0] = hq.x; hv[1] = hq.y; hv[2] = hq.z; hv[3] = hq.w;
    Av[0] = aq.x; Av[1] = aq.y; Av[2] = aq.z; Av[3] = aq.w;
#pragma unroll
    for (int k = 0; k < 4; ++k) { Bv[k] = to_f32(Bp[n0 + k]); Cv[k] = to_f32(Cp[n0 + k]); }
  } else if (p.vec == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (n0 + k < N) {
        hv[k] = st[k];
        Av[k] = p.A[d * N + n0 + k];
        Bv[k] = to_f32(Bp[n0 + k]);
        Cv[k] = to_f32(Cp[n0 + k]);
      }
  }
  const float xu = ZOH ? uv : dt * uv;
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = exp2_(dt * Av[k] * kLog2e);
    float x;
    if (ZOH) x = (dt * expm1_over_x(dt * Av[k], a)) * (xu * Bv[k]);
    else x = xu * Bv[k];
    hv[k] = __builtin_fmaf(a, hv[k], x);
    acc = __builtin_fmaf(Cv[k], hv[k], acc);
  }
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, G);
  if (cval && q == 0) {
    float y = acc + (p.D ? p.D[d] : 0.0f) * uv;
    if (p.z) y *= silu_(to_f32(reinterpret_cast<const IO*>(p.z)[cc]));
    store_io(reinterpret_cast<IO*>(p.out) + cc, y);
  }
  if (cval) {
    if (vec4) {
      *reinterpret_cast<float4*>(st) = make_float4(hv[0], hv[1], hv[2], hv[3]);
    } else if (p.vec == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (n0 + k < N) st[k] = hv[k];
    }
  }
}

}  // namespace ssm
