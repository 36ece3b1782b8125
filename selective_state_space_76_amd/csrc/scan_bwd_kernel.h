// scan_bwd_kernel.h -- gradients of the selective scan (either discretisation, either direction).
//
// The pages give only the forward recurrence; the gradients follow from it by the
// chain rule.  Write B_bar = e B: e = dt by default, e = (Abar - 1) / A = dt phi(dt A)
// with phi(x) = (e^x - 1) / x under zero-order hold.  Then de/ddt is 1 by default and
// Abar under ZOH, and de/dA is 0 by default and dt^2 phi'(dt A) under ZOH.  With G the
// gradient reaching the state h after step t (scan order):
//   dy_t  = dout_t * silu(z_t);   dz_t = dout_t * y_t * silu'(z_t)
//   G    += dy_t * C_t            dC_t += dy_t * h_t           (summed over channels)
//   du_t  = dy_t * D + sum_n G_n e_t,n B_t,n
//   ddt_t = sum_n G_n (h_{t-1,n} Abar_t,n A_n + de/ddt u_t B_t,n)
//   dA_n += G_n (h_{t-1,n} Abar_t,n dt_t + de/dA u_t B_t,n);   dB_t += G * e_t * u_t   (over channels)
//   G     = G * Abar_t            (to step t-1)
//   ddelta_t = ddt_t * logistic(delta_t + bias);  dbias += ddelta_t;  dD += dy_t u_t
//   dh0 = G after the first step.
//
// Work layout (lanes over time):
//   * A checkpoint pass (the scan kernel's mode 2) stores the state entering every 64-step
//     block.  A workgroup is 4 waves; a wave is 4 rows of 16 lanes; a row owns one channel
//     (b, d), so the workgroup owns 16 channels of one batch row.  The sequence is walked in
//     chunks of 16 T steps (T = 8 or 16) from last to first; lane g of a row owns the T
//     consecutive steps T g .. T g + T - 1 of the chunk and keeps their per-(channel, step)
//     values (dt, u, dt u, dy, the dz factor) and the sums over states (y, sum G B,
//     sum G h A_bar A) in registers.
//   * The states are a loop (one B/C tile of 16 states per stage).  For state n:
//       forward: each lane folds its steps into (prod A_bar, state from zero), a 16-lane
//       scan composes the pairs with the checkpointed state entering the chunk, and the
//       lane reruns its steps (states h_t in registers) and adds C h_t to y_t;
//       adjoint: G_t = dy_t C_t + A_bar_{t+1} G_{t+1} runs backwards, so each lane folds
//       its steps into (prod A_bar, adjoint from zero) from its last step, a 16-lane scan
//       composes them right to left with the adjoint entering from the next chunk, and the
//       lane reruns its steps backwards, forming the gradient terms of every step.
//     Sums over states are per-lane accumulations (no cross-lane reduction); only dB and
//     dC (sums over channels) are reduced: over the wave's 4 rows with lane swaps, over the
//     4 waves through LDS in a fixed order, and written per workgroup; a separate pass adds
//     the workgroups' partial sums in a fixed order, so every gradient is bitwise
//     reproducible.
//   * Registers do not grow with the number of states, so every N runs at the same
//     occupancy.
#pragma once
#include "ssm_device.h"

namespace ssm {

namespace {

// Sum of x over the 4 rows of the wave, for two vectors at once: returns, in row
// 0 and 2 of the result, the totals of x and y for lanes g (rows 1 and 3 hold
// the totals of x2 and y2 when the pair (x2, y2) is reduced in the same call).
//   row 0: sum_rows x,  row 1: sum_rows x2,  row 2: sum_rows y,  row 3: sum_rows y2
__device__ __forceinline__ float rows4_sum2(float x, float y, float x2, float y2) {
  // halves: lanes 0-31 get x(rows 0,1)+x(rows 2,3), lanes 32-63 the same for y
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  const float P = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x2), __float_as_uint(y2), false, false);
  const float Q = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  // rows: r0 = P(r0)+P(r1), r1 = Q(r0)+Q(r1), r2 = P(r2)+P(r3), r3 = Q(r2)+Q(r3)
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(P), __float_as_uint(Q), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float logistic_(float x) { return rcp_(1.0f + exp2_(-x * kLog2e)); }

// The slope of the softplus at x, logistic(x), from dt = softplus(x) alone (no second read of
// delta): 1 + e^x = e^dt, so logistic(x) = 1 - e^-dt.  Below dt = 1/16 from its Taylor series
// (terms to dt^4; the first dropped term is under 1.3e-7 relative there), above it 1 - e^-dt,
// where the rounding of e^-dt costs under 1e-6 relative.
__device__ __forceinline__ float softplus_slope(float dt) {
  const float series = dt * (1.0f - dt * (0.5f - dt * (0.16666667f - dt * 0.041666668f)));
  return dt < 0.0625f ? series : 1.0f - exp2_(-dt * kLog2e);
}

// d(zoh_e)/dA = (dt a - zoh_e) / A = dt^2 phi'(x), phi'(x) = sum_k (k + 1) x^k / (k + 2)!.
// Below |x| = 1/4 from the series to x^5 (the next term is under 1e-7 relative there); above
// it the closed form, whose difference dt a - zoh_e ~ dt x / 2 is then large enough that
// the rounding of a and zoh_e costs under 1e-5 relative.
__device__ __forceinline__ float zoh_e_dA(float dt, float x, float a, float e, float ia) {
  const float series =
      0.5f + x * (0.33333334f + x * (0.125f + x * (0.033333335f + x * (0.0069444445f + x * 0.0011904762f))));
  return (fabsf(x) < 0.25f) ? (dt * dt) * series : __builtin_fmaf(dt, a, -e) * ia;
}

}  // namespace

namespace bwdc {

// Inclusive scan over the 16 lanes of each row of (P, Q) pairs, the earlier lane first:
// (P1, Q1) then (P2, Q2) gives (P1 P2, P2 Q1 + Q2).  Lanes without a predecessor at a stage
// keep their pair: the fmac reads 0 there (bound_ctrl), the mul is not written.  Each
// stage's DPP reads the VGPR the previous stage wrote two instructions earlier, which with
// the s_nop meets the two wait states DPP needs.
__device__ __forceinline__ void row_scan_from_left(float& Q, float& P) {
  asm volatile(
      "s_nop 1\n"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_mul_f32_dpp %1, %1, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n"
      "s_nop 0\n"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_mul_f32_dpp %1, %1, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n"
      "s_nop 0\n"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_mul_f32_dpp %1, %1, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n"
      "s_nop 0\n"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_mul_f32_dpp %1, %1, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      : "+v"(Q), "+v"(P));
}

// The same composition with the later lane first (row_shl): (P2, Q2) then (P1, Q1) gives
// (P1 P2, P1 Q2 + Q1) for lane 1 left of lane 2.
__device__ __forceinline__ void row_scan_from_right(float& Q, float& P) {
  asm volatile(
      "s_nop 1\n"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_mul_f32_dpp %1, %1, %1 row_shl:1 row_mask:0xf bank_mask:0xf\n"
      "s_nop 0\n"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_mul_f32_dpp %1, %1, %1 row_shl:2 row_mask:0xf bank_mask:0xf\n"
      "s_nop 0\n"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_mul_f32_dpp %1, %1, %1 row_shl:4 row_mask:0xf bank_mask:0xf\n"
      "s_nop 0\n"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "v_mul_f32_dpp %1, %1, %1 row_shl:8 row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      : "+v"(Q), "+v"(P));
}

// v from the previous (next) lane of the row; the row's first (last) lane gets `edge`
__device__ __forceinline__ float from_prev_lane(float edge, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(edge), __float_as_int(v), 0x111 /* row_shr:1 */,
                                                    0xf, 0xf, false));
}
__device__ __forceinline__ float from_next_lane(float edge, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(edge), __float_as_int(v), 0x101 /* row_shl:1 */,
                                                    0xf, 0xf, false));
}

// 16-byte piece -> EPC floats in order
template <typename IO> __device__ __forceinline__ void unpack(const uint4& v, float* f) {
  if constexpr (sizeof(IO) == 2) {
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = __uint_as_float(x[k] << 16);
      f[2 * k + 1] = __uint_as_float(x[k] & 0xffff0000u);
    }
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}

// elements [ts, ts + EPC) of a row in logical step order (logical t is physical L-1-t when
// REV); steps at or past L read 0.  VEC: L is a multiple of EPC, so a piece never straddles L.
template <typename IO, bool REV, bool VEC>
__device__ __forceinline__ void load_piece(const IO* row, int64_t ts, int64_t L, float* f) {
  constexpr int EPC = 16 / (int)sizeof(IO);
  if (VEC) {
    float q[EPC];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ts < L) v = *reinterpret_cast<const uint4*>(row + (REV ? (L - EPC - ts) : ts));
    unpack<IO>(v, q);
#pragma unroll
    for (int e = 0; e < EPC; ++e) f[e] = REV ? q[EPC - 1 - e] : q[e];
  } else {
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const int64_t t = ts + e;
      f[e] = t < L ? to_f32(row[REV ? (L - 1 - t) : t]) : 0.0f;
    }
  }
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// outstanding global loads and stores (the waves of a workgroup exchange data through LDS only).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace bwdc

template <typename IO, int T, bool ZOH, bool REV, bool VEC>
__global__ __launch_bounds__(256, T == 16 ? 2 : 3) void scan_bwd_kernel(BwdParams p) {
  using namespace bwdc;
  // T steps per lane
  constexpr int CH = 16 * T;                  // steps per chunk
  constexpr int KG = T / 4;                   // float4 groups per lane
  constexpr int EPC = 16 / (int)sizeof(IO);   // elements per 16-byte piece
  constexpr int PPR = CH / EPC;               // pieces per coefficient row of a chunk
  constexpr int PPT = 2 * 16 * PPR / 256;     // B and C pieces per thread (16 states)
  // [tensor][state of the stage][float4 group][lane]: step 16 lane + 4 group + component
  __shared__ f32x4 bc[2 * 16 * KG * 16];
  // The default discretisation with 8 steps per lane runs only up to 32 states (more take 16 steps per
  // lane), so its per-state constants need half the LDS; it keeps u and the dz factor of its steps,
  // which the loop over states does not read, in the LDS that frees instead of in registers.
  constexpr bool STASH = T == 8 && !ZOH;
  constexpr int NM = STASH ? 32 : 64;         // states the per-state LDS arrays hold
  // [channel of the workgroup][state]: A log2(e), A, 1/A (ZOH), adjoint entering the chunk from the right
  __shared__ float4 cst[16 * NM];
  __shared__ float dacc[16 * NM];             // [channel][state]: dA summed over the steps done so far
  __shared__ float stash[STASH ? 2 * T * 256 : 1];  // [value][step][thread]: u, dz factor
  __shared__ float red[2][4][2 * CH];         // [parity][wave][dB | dC of the chunk's steps]
  __shared__ float hck[16 * 16];              // [channel][state of the stage]: state entering the chunk

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int r = lane >> 4, g = lane & 15;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = logical % p.nblk;
  const int rest = logical / p.nblk;
  const int seg = rest % p.S;               // segment of the sequence (one when it is not split)
  const int64_t b = rest / p.S;
  const int64_t L = p.L, N = p.N, Dm = p.Dm;
  const int64_t nbk = (L + 63) / 64;
  const int cl = w * 4 + r;
  const int64_t d = (int64_t)cb * 16 + cl;
  const bool dval = d < Dm;
  const int64_t dd = dval ? d : Dm - 1;
  const bool has_z = p.z != nullptr;
  const float biasd = p.bias ? p.bias[dd] : 0.0f;
  const float Dd = p.D ? p.D[dd] : 0.0f;
  float4* cs = cst + cl * NM;
  float* da = dacc + cl * NM;

#pragma unroll
  for (int k = 0; k < NM / 16; ++k) {
    const int64_t n = g + 16 * k;
    if (n < N) {
      const float a = p.A[dd * N + n];
      // adjoint entering the segment's last step from the right: the final-state gradient, or
      // for a split sequence the composition of the segments to the right
      const float gf = !dval ? 0.0f
                             : p.adj_in ? p.adj_in[(((int64_t)seg * p.Bsz + b) * Dm + d) * N + n]
                                        : (p.dfinal ? p.dfinal[(b * Dm + d) * N + n] : 0.0f);
      cs[n] = make_float4(a * kLog2e, a, ZOH ? 1.0f / a : 0.0f, gf);
      da[n] = 0.0f;
    }
  }

  // The seven [B, D, L] streams share this lane's row offset.  Their row pointers are formed from it
  // where they are used (an empty asm hides the offset from loop-invariant hoisting), so the lane keeps
  // one 64-bit offset through the loop over states instead of seven pointers.
  const int64_t roff0 = (b * Dm + dd) * L;
  float dDacc = 0.0f, dbacc = 0.0f;  // this lane's dD and dbias terms
  int par = 0;                       // parity of the dB/dC exchange buffer
  // the segment's chunks (a split segment is a whole number of chunks; the last one may be ragged)
  const int64_t tb = (int64_t)seg * p.seg_len;
  const int64_t te = (tb + p.seg_len < L) ? tb + p.seg_len : L;
  const int64_t nch = (te - tb + CH - 1) / CH;

  for (int64_t ci = nch - 1; ci >= 0; --ci) {
    const int64_t c0 = tb + ci * CH;
    const int64_t t0 = c0 + g * T;
    int64_t roff = roff0;
    asm volatile("" : "+v"(roff));
    const IO* urow = reinterpret_cast<const IO*>(p.u) + roff;
    const IO* drow = reinterpret_cast<const IO*>(p.delta) + roff;
    const IO* zrow = has_z ? reinterpret_cast<const IO*>(p.z) + roff : nullptr;
    const IO* grow = reinterpret_cast<const IO*>(p.dout) + roff;

    // per-(channel, step) values of this lane's 16 steps
    float dt[T], uu[T], xu[T], dy[T], dzf[T];
    float cumlo = 0.0f, cumhi = 0.0f;  // step sizes of the lane's first and second half (kept apart:
                                       // the second as a difference of sums would cancel)
#pragma unroll
    for (int k = 0; k < T / EPC; ++k) {
      float fd[EPC], fu[EPC], fg[EPC], fz[EPC];
      load_piece<IO, REV, VEC>(drow, t0 + k * EPC, L, fd);
      load_piece<IO, REV, VEC>(urow, t0 + k * EPC, L, fu);
      load_piece<IO, REV, VEC>(grow, t0 + k * EPC, L, fg);
      if (has_z) load_piece<IO, REV, VEC>(zrow, t0 + k * EPC, L, fz);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int s = k * EPC + e;
        const bool tv = t0 + s < L;
        const float dts = tv ? softplus_(fd[e] + biasd) : 0.0f;  // past the end: identity step
        const float go = dval ? fg[e] : 0.0f;                     // channels past D contribute nothing
        dt[s] = dts;
        uu[s] = fu[e];
        xu[s] = ZOH ? fu[e] : dts * fu[e];
        if (has_z) {
          const float sg = logistic_(fz[e]);
          dy[s] = go * (fz[e] * sg);
          dzf[s] = go * (sg * __builtin_fmaf(fz[e], 1.0f - sg, 1.0f));  // dz = y * dzf
        } else {
          dy[s] = go;
          dzf[s] = 0.0f;
        }
        if (tv) dDacc = __builtin_fmaf(dy[s], fu[e], dDacc);
        if (s < T / 2) cumlo += dts;
        else cumhi += dts;
        if constexpr (STASH) {  // read back by this thread alone, after the loop over states
          stash[s * 256 + tid] = uu[s];
          stash[(T + s) * 256 + tid] = dzf[s];
        }
      }
    }

    float yv[T], S1[T], S2[T];  // over states: C h; G B (G e B); G A_bar h_{t-1} A (+ G A_bar u B)
#pragma unroll
    for (int s = 0; s < T; ++s) { yv[s] = 0.0f; S1[s] = 0.0f; S2[s] = 0.0f; }

    for (int64_t n0 = 0; n0 < N; n0 += 16) {
      lds_barrier();  // every wave is done with the previous stage's tile
      // the checkpointed states entering the chunk, one (channel tid / 16, state n0 + tid % 16) per
      // thread, loaded with the tile so that no state waits on a global load
      float hcv = 0.0f;
      {
        const int64_t dh = (int64_t)cb * 16 + (tid >> 4), nh = n0 + (tid & 15);
        if (dh < Dm && nh < N) hcv = p.ckpt[((b * nbk + c0 / 64) * Dm + dh) * N + nh];
      }
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const int q = tid + 256 * k;
        const int tt = q / (16 * PPR), nl = (q / PPR) % 16, pc = q % PPR;
        const int64_t n = n0 + nl;
        float f[EPC];
        if (n < N) {
          const IO* src = reinterpret_cast<const IO*>(tt == 0 ? p.B : p.C) + (b * N + n) * L;
          load_piece<IO, REV, VEC>(src, c0 + pc * EPC, L, f);
        } else {
#pragma unroll
          for (int e = 0; e < EPC; ++e) f[e] = 0.0f;
        }
        const int o = pc * EPC, gl = o / T, s0 = o % T;
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
          const f32x4 v = {f[e], f[e + 1], f[e + 2], f[e + 3]};
          bc[((tt * 16 + nl) * KG + (s0 + e) / 4) * 16 + gl] = v;
        }
      }
      hck[tid] = hcv;
      lds_barrier();

      const int ng = (N - n0) < 16 ? (int)(N - n0) : 16;
#pragma unroll 1
      for (int nl = 0; nl < ng; ++nl) {
        const int64_t n = n0 + nl;
        const float4 c4 = cs[n];
        const float A2 = c4.x, Aln = c4.y, Ai = c4.z, Gc = c4.w;
        const float hc = hck[cl * 16 + nl];  // state entering the chunk
        const f32x4* bq = bc + (nl * KG) * 16 + g;
        const f32x4* cq = bc + ((16 + nl) * KG) * 16 + g;

        // forward through the chunk
        float a[T], h[T], ezs[ZOH ? T : 1];  // ezs: the ZOH factor of each step, reused by the adjoint
        float Qa = 0.0f, Qb = 0.0f;
#pragma unroll
        for (int k = 0; k < KG; ++k) {
          const f32x4 bv = bq[k * 16];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = 4 * k + e;
            a[s] = exp2_(dt[s] * A2);
            if constexpr (ZOH) ezs[s] = zoh_e(dt[s], dt[s] * Aln, a[s], Ai);
            const float bb = ZOH ? ezs[ZOH ? s : 0] * (xu[s] * bv[e]) : xu[s] * bv[e];
            h[s] = bb;  // B_bar u for now; the rerun turns it into the state
            if (s < T / 2) Qa = __builtin_fmaf(a[s], Qa, bb);
            else Qb = __builtin_fmaf(a[s], Qb, bb);
          }
        }
        const float Plo = exp2_(cumlo * A2), Phi = exp2_(cumhi * A2);
        const float Pl = Plo * Phi;  // product of the lane's 16 decay factors
        float Q = __builtin_fmaf(Phi, Qa, Qb), P = Pl;
        row_scan_from_left(Q, P);
        const float hs = from_prev_lane(hc, __builtin_fmaf(P, hc, Q));  // state before the lane's first step
        {
          float h1 = hs, h2 = __builtin_fmaf(Plo, hs, Qa);
#pragma unroll
          for (int k = 0; k < KG; ++k) {
            const f32x4 cv = cq[k * 16];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int s = 4 * k + e;
              if (s < T / 2) {
                h1 = __builtin_fmaf(a[s], h1, h[s]);
                h[s] = h1;
              } else {
                h2 = __builtin_fmaf(a[s], h2, h[s]);
                h[s] = h2;
              }
              yv[s] = __builtin_fmaf(cv[e], h[s], yv[s]);
            }
          }
        }

        // adjoint: the lane's steps folded from its last, as if nothing entered from the right
        float QG = 0.0f, dc[T];
#pragma unroll
        for (int k = KG - 1; k >= 0; --k) {
          const f32x4 cv = cq[k * 16];
#pragma unroll
          for (int e = 3; e >= 0; --e) {
            const int s = 4 * k + e;
            dc[s] = dy[s] * cv[e];
            QG = (s == T - 1) ? dc[s] : __builtin_fmaf(a[s + 1 < T ? s + 1 : 0], QG, dc[s]);
          }
        }
        float Qr = a[0] * QG, Pr = Pl;  // adjoint this lane passes to its left neighbour: Qr + Pr X_in
        row_scan_from_right(Qr, Pr);
        const float xout = __builtin_fmaf(Pr, Gc, Qr);
        const float xin = from_next_lane(Gc, xout);  // adjoint entering the lane's last step from the right
        if (g == 0) cs[n].w = xout;                  // into the previous chunk's last step

        // backwards through the lane's steps: G_t, then every gradient term of step t; the dB and
        // dC terms of each pair of steps are summed over the wave's 4 rows as soon as both exist
        float G = xin, dAl = 0.0f;
        float xo = 0.0f, yo = 0.0f;  // dB, dC terms of the odd step of the current pair
        float* rw = red[par][w];
#pragma unroll
        for (int k = KG - 1; k >= 0; --k) {
          const f32x4 bv = bq[k * 16];
#pragma unroll
          for (int e = 3; e >= 0; --e) {
            const int s = 4 * k + e;
            G = (s == T - 1) ? G + dc[s] : __builtin_fmaf(a[s + 1 < T ? s + 1 : 0], G, dc[s]);
            const float hp = s > 0 ? h[s > 0 ? s - 1 : 0] : hs;
            const float tt = G * hp * a[s];
            float vb;  // dB term
            if constexpr (ZOH) {
              const float x = dt[s] * Aln;
              const float ez = ezs[ZOH ? s : 0];
              const float gb = G * bv[e];
              const float gbu = gb * uu[s];
              S1[s] = __builtin_fmaf(gb, ez, S1[s]);
              S2[s] = __builtin_fmaf(tt, Aln, __builtin_fmaf(gbu, a[s], S2[s]));
              dAl = __builtin_fmaf(tt, dt[s], __builtin_fmaf(gbu, zoh_e_dA(dt[s], x, a[s], ez, Ai), dAl));
              vb = G * (ez * uu[s]);
            } else {
              S1[s] = __builtin_fmaf(G, bv[e], S1[s]);
              S2[s] = __builtin_fmaf(tt, Aln, S2[s]);
              dAl = __builtin_fmaf(tt, dt[s], dAl);
              vb = G * xu[s];
            }
            const float vc = dy[s] * h[s];
            if (s % 2 == 1) {
              xo = vb;
              yo = vc;
            } else {
              // rows of the result: 0 = dB step s+1, 1 = dB step s, 2 = dC step s+1, 3 = dC step s
              const float v = rows4_sum2(xo, yo, vb, vc);
              rw[(r >> 1) * CH + T * g + s + ((r & 1) ? 0 : 1)] = v;
            }
          }
        }

        // dA over the row's lanes: rotations by 8, 4, 2, 1 within the row (a fixed order; lane 0 keeps it)
        dAl += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(dAl), 0x128 /* row_ror:8 */, 0xf, 0xf, false));
        dAl += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(dAl), 0x124 /* row_ror:4 */, 0xf, 0xf, false));
        dAl += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(dAl), 0x122 /* row_ror:2 */, 0xf, 0xf, false));
        dAl += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(dAl), 0x121 /* row_ror:1 */, 0xf, 0xf, false));
        if (g == 0) da[n] += dAl;

        // dB, dC over the workgroup's 16 channels: the 4 waves' row sums through LDS, in wave order
        lds_barrier();
#pragma unroll
        for (int e = tid; e < 2 * CH; e += 256) {
          const int qty = e / CH, step = e % CH;
          const int64_t t = c0 + step;
          if (t < L) {
            const float v = ((red[par][0][e] + red[par][1][e]) + red[par][2][e]) + red[par][3][e];
            p.part_bc[((((int64_t)qty * p.nblk + cb) * p.Bsz + b) * N + n) * L + (REV ? L - 1 - t : t)] = v;
          }
        }
        par ^= 1;  // the next state writes the other buffer; this one is free after the next barrier
      }
    }

    // per-step outputs of this lane's steps
    int64_t roffo = roff0;
    asm volatile("" : "+v"(roffo));
    IO* du_row = reinterpret_cast<IO*>(p.du) + roffo;
    IO* dd_row = reinterpret_cast<IO*>(p.ddelta) + roffo;
    IO* dz_row = has_z ? reinterpret_cast<IO*>(p.dz) + roffo : nullptr;
#pragma unroll
    for (int k = 0; k < T / EPC; ++k) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int s = k * EPC + e;
        const int64_t t = t0 + s;
        if constexpr (STASH) {
          uu[s] = stash[s * 256 + tid];
          dzf[s] = stash[(T + s) * 256 + tid];
        }
        const float du = ZOH ? __builtin_fmaf(dy[s], Dd, S1[s]) : __builtin_fmaf(dy[s], Dd, dt[s] * S1[s]);
        const float ddt = ZOH ? S2[s] : __builtin_fmaf(uu[s], S1[s], S2[s]);
        const float ddl = ddt * softplus_slope(dt[s]);
        if (t < L) {
          dbacc += ddl;
          if (dval) {
            const int64_t ph = REV ? (L - 1 - t) : t;
            store_io(du_row + ph, du);
            store_io(dd_row + ph, ddl);
            if (has_z) store_io(dz_row + ph, (yv[s] + Dd * uu[s]) * dzf[s]);
          }
        }
      }
    }
  }

  if (dval) {
#pragma unroll
    for (int k = 0; k < NM / 16; ++k) {
      const int64_t n = g + 16 * k;
      if (n < N) {
        p.part_a[(((int64_t)seg * p.Bsz + b) * Dm + d) * N + n] = da[n];
        if (p.dh0 && seg == 0) p.dh0[(b * Dm + d) * N + n] = cs[n].w;
      }
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    dDacc += __shfl_xor(dDacc, off, 16);
    dbacc += __shfl_xor(dbacc, off, 16);
  }
  if (dval && g == 0) {
    const int64_t SB = (int64_t)p.S * p.Bsz;
    p.part_d[((int64_t)seg * p.Bsz + b) * Dm + d] = dDacc;
    p.part_d[SB * Dm + ((int64_t)seg * p.Bsz + b) * Dm + d] = dbacc;
  }
}


template <typename IO, int T, bool ZOH, bool REV, bool VEC>
void go_bwd(const BwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL((scan_bwd_kernel<IO, T, ZOH, REV, VEC>), dim3((unsigned)(p.Bsz * p.nblk * p.S)), dim3(256), 0, s, p);
}

template <typename IO, int T, bool ZOH>
void go_bwd_flags(const BwdParams& p, hipStream_t s) {
  const int k = (p.reverse ? 2 : 0) + (p.vec ? 1 : 0);
  switch (k) {
    case 0: go_bwd<IO, T, ZOH, false, false>(p, s); break;
    case 1: go_bwd<IO, T, ZOH, false, true>(p, s); break;
    case 2: go_bwd<IO, T, ZOH, true, false>(p, s); break;
    default: go_bwd<IO, T, ZOH, true, true>(p, s); break;
  }
}

// 8 steps per lane (three workgroups per CU) except for the default discretisation with more
// than 32 states, where 16 steps per lane measured faster (5.5 against 6.0 ms per call at
// 4 x 4096 x 64 x 4096; with 16 and 32 states 8 steps win, 0.64 against 0.83 and 1.18 against
// 1.38 ms)
template <bool ZOH>
hipError_t go_bwd_all(const BwdParams& p, bool bf16, hipStream_t s) {
  // the 16-step variant exists for Euler only: with ZOH its extra factors spill
  if constexpr (!ZOH) {
    if (p.N > 32) {
      if (bf16) go_bwd_flags<bf16_t, 16, false>(p, s);
      else go_bwd_flags<float, 16, false>(p, s);
      return hipGetLastError();
    }
  }
  if (bf16) go_bwd_flags<bf16_t, 8, ZOH>(p, s);
  else go_bwd_flags<float, 8, ZOH>(p, s);
  return hipGetLastError();
}

// the checkpoint pass (the scan kernel's mode 2) for one discretisation
template <typename IO, int NL, bool ZOH, bool REV, bool VEC>
void go_ckpt(const ScanParams& p, hipStream_t s) {
  hipLaunchKernelGGL((scan_kernel<IO, NL, 2, ZOH, REV, VEC>), dim3((unsigned)(p.Bsz * p.nblk * p.S)), dim3(256), 0, s, p);
}

template <typename IO, int NL, bool ZOH>
void go_ckpt_flags(const ScanParams& p, hipStream_t s) {
  const int k = (p.reverse ? 2 : 0) + (p.vec ? 1 : 0);
  switch (k) {
    case 0: go_ckpt<IO, NL, ZOH, false, false>(p, s); break;
    case 1: go_ckpt<IO, NL, ZOH, false, true>(p, s); break;
    case 2: go_ckpt<IO, NL, ZOH, true, false>(p, s); break;
    default: go_ckpt<IO, NL, ZOH, true, true>(p, s); break;
  }
}

template <bool ZOH>
hipError_t go_ckpt_all(const ScanParams& p, bool bf16, hipStream_t s) {
  if (bf16) {
    if (p.N <= 16) go_ckpt_flags<bf16_t, 1, ZOH>(p, s);
    else if (p.N <= 32) go_ckpt_flags<bf16_t, 2, ZOH>(p, s);
    else go_ckpt_flags<bf16_t, 4, ZOH>(p, s);
  } else {
    if (p.N <= 16) go_ckpt_flags<float, 1, ZOH>(p, s);
    else if (p.N <= 32) go_ckpt_flags<float, 2, ZOH>(p, s);
    else go_ckpt_flags<float, 4, ZOH>(p, s);
  }
  return hipGetLastError();
}

}  // namespace ssm
