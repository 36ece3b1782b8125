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
// Work layout (up to 16 states; more states run in chunk_bwd_kernel, scan_bwd_chunk.h): the
// forward kernel's (a workgroup = 16 channels of one batch row, a 16-lane row = one
// channel, lane g holds state g).  A checkpoint pass
// (the scan kernel's mode 2) stores the state entering every 64-step block.  This
// kernel walks the blocks from last to first: it restores the block's states from
// the checkpoint by recomputing the forward recurrence in 16-step sub-blocks, then
// runs the adjoint recurrence backwards through each sub-block.  The three sums
// over states per step (y, sum G B, sum G h Abar A) use the in-register 16 x 16
// reduce-scatter of the forward kernel.  dB and dC contributions are summed over
// the wave's 4 channels with lane swaps between 32- and 16-lane halves (VALU only),
// over the 4 waves through LDS in a fixed order, and written per workgroup; a
// separate pass adds the workgroups' partial sums in a fixed order, so every
// gradient is bitwise reproducible.
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

// With one state slice, three workgroups per CU (168 registers, a few spilled): the 130M-class
// shape's 768 workgroups then run in one round instead of one and a half.  The ZOH variant
// holds more live values per step and keeps two.
template <typename IO, int NL, bool ZOH, bool REV, bool VEC>
__global__ __launch_bounds__(256, (NL == 1 && !ZOH) ? 3 : 2) void scan_bwd_kernel(BwdParams p) {
  constexpr int NP = 16 * NL;
  constexpr int TS = 68;                       // LDS tile row: 64 steps + 4 pad
  constexpr int NT = 2;                        // B, C
  constexpr int NS = 4;                        // delta, u, z, dout
  constexpr int EPC = 16 / (int)sizeof(IO);
  constexpr int CPR = 64 / EPC;
  constexpr int NBC = NT * NP * CPR;
  constexpr int NCH = NBC + NS * 16 * CPR;
  constexpr int CPT = (NCH + 255) / 256;
  constexpr int TILE = NT * NP * TS + NS * 16 * TS;
  constexpr int RED = 4 * 2 * 16 * NP;         // per-wave dB/dC sums of one sub-block
  static_assert(NL == 1, "more than 16 states run in chunk_bwd_kernel");
  __shared__ __attribute__((aligned(16))) float tiles[TILE];
  __shared__ float red[2 * RED];               // double-buffered by sub-block parity

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int r = lane >> 4, g = lane & 15;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = logical % p.nblk;
  const int64_t b = logical / p.nblk;
  const int64_t L = p.L, N = p.N, Dm = p.Dm;
  const int64_t nbk = (L + 63) / 64;
  const int cl = w * 4 + r;
  const int64_t d = (int64_t)cb * 16 + cl;
  const bool dval = d < Dm;
  const int64_t dd = dval ? d : Dm - 1;
  const bool has_z = p.z != nullptr;
  const float biasd = p.bias ? p.bias[dd] : 0.0f;
  const float Dd = p.D ? p.D[dd] : 0.0f;

  float Ap[NL], Aln[NL], Ainv[NL], G[NL], dAacc[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int64_t n = g + 16 * i;
    const bool nv = n < N;
    Aln[i] = nv ? p.A[dd * N + n] : 0.0f;
    Ap[i] = Aln[i] * kLog2e;
    Ainv[i] = ZOH ? 1.0f / Aln[i] : 0.0f;  // infinite for A = 0, where zoh_e's series branch is taken
    G[i] = (nv && dval && p.dfinal) ? p.dfinal[(b * Dm + d) * N + n] : 0.0f;
    dAacc[i] = 0.0f;
  }
  float dDacc = 0.0f, dbacc = 0.0f;

  for (int i = tid; i < TILE; i += 256) tiles[i] = 0.0f;

  const IO* src[CPT];
  int dst[CPT];
  bool live[CPT];
  int col[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int c = tid + 256 * k;
    src[k] = nullptr;
    dst[k] = 0;
    live[k] = false;
    col[k] = 0;
    if (c < NBC) {
      const int tt = c / (NP * CPR), n = (c / CPR) % NP;
      col[k] = (c % CPR) * EPC;
      live[k] = n < N;
      src[k] = reinterpret_cast<const IO*>(tt == 0 ? p.B : p.C) + (b * N + (n < N ? n : 0)) * L;
      dst[k] = (tt * NP + n) * TS + col[k];
    } else if (c < NCH) {
      const int e = c - NBC;
      const int st = e / (16 * CPR), row = (e / CPR) % 16;
      col[k] = (e % CPR) * EPC;
      const int64_t dr = (int64_t)cb * 16 + row;
      const void* base = st == 0 ? p.delta : (st == 1 ? p.u : (st == 2 ? p.z : p.dout));
      live[k] = dr < Dm && base != nullptr;
      src[k] = reinterpret_cast<const IO*>(live[k] ? base : p.u) + (b * Dm + (dr < Dm ? dr : 0)) * L;
      dst[k] = NT * NP * TS + (st * 16 + row) * TS + col[k];
    }
  }

  uint4 raw[CPT];
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int64_t ts = t0 + col[k];
      uint4 v = make_uint4(0, 0, 0, 0);
      if (live[k] && ts < L) {
        if (VEC) {
          v = *reinterpret_cast<const uint4*>(src[k] + (REV ? (L - EPC - ts) : ts));
        } else {
          IO e[EPC];
#pragma unroll
          for (int k2 = 0; k2 < EPC; ++k2) {
            const int64_t lt = REV ? (ts + EPC - 1 - k2) : (ts + k2);
            e[k2] = (lt < L) ? src[k][REV ? (L - 1 - lt) : lt] : IO(0);
          }
          v = *reinterpret_cast<const uint4*>(e);
        }
      }
      raw[k] = v;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      if (live[k]) {
        float f[EPC];
        if constexpr (sizeof(IO) == 2) {
          const uint32_t x[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
          for (int k2 = 0; k2 < 4; ++k2) {
            f[2 * k2] = __uint_as_float(x[k2] << 16);
            f[2 * k2 + 1] = __uint_as_float(x[k2] & 0xffff0000u);
          }
        } else {
          f[0] = __uint_as_float(raw[k].x); f[1] = __uint_as_float(raw[k].y);
          f[2] = __uint_as_float(raw[k].z); f[3] = __uint_as_float(raw[k].w);
        }
#pragma unroll
        for (int k2 = 0; k2 < EPC; k2 += 4) {
          float4 o;
          if (REV) o = make_float4(f[EPC - 1 - k2], f[EPC - 2 - k2], f[EPC - 3 - k2], f[EPC - 4 - k2]);
          else o = make_float4(f[k2], f[k2 + 1], f[k2 + 2], f[k2 + 3]);
          *reinterpret_cast<float4*>(tiles + dst[k] + k2) = o;
        }
      }
    }
  };

  IO* du_row = reinterpret_cast<IO*>(p.du) + (b * Dm + dd) * L;
  IO* dd_row = reinterpret_cast<IO*>(p.ddelta) + (b * Dm + dd) * L;
  IO* dz_row = has_z ? reinterpret_cast<IO*>(p.dz) + (b * Dm + dd) * L : nullptr;

  fetch((nbk - 1) * 64);
  int sbp = 0;  // sub-block parity for the reduction buffer
  for (int64_t blk = nbk - 1; blk >= 0; --blk) {
    const int64_t t0 = blk * 64;
    __syncthreads();  // every wave is done with the previous block's tile
    store();
    if (blk > 0) fetch(t0 - 64);
    __syncthreads();

    const float* Bt = tiles;
    const float* Ct = tiles + NP * TS;
    const float* dch = tiles + NT * NP * TS + cl * TS;
    const float* uch = dch + 16 * TS;
    const float* zch = dch + 32 * TS;
    const float* gch = dch + 48 * TS;

    // this lane's own steps 16 s + g
    float dt[4], xu[4], uu[4], xs[4], go[4], zz[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t t = t0 + 16 * s + g;
      const float dl = dch[16 * s + g];
      uu[s] = uch[16 * s + g];
      zz[s] = zch[16 * s + g];
      go[s] = gch[16 * s + g];
      xs[s] = dl + biasd;
      dt[s] = t < L ? softplus_(xs[s]) : 0.0f;  // steps past the end leave the state unchanged
      xu[s] = ZOH ? uu[s] : dt[s] * uu[s];
    }

    // B_bar u of step j of a sub-block for state slice i, given dj = dt, xj = xu of that step,
    // bj = B and a = Abar (under ZOH the factor e depends on the state through A)
    auto bbar_u = [&](float dj, float xj, float bj, float a, int i) -> float {
      if constexpr (ZOH) return zoh_e(dj, dj * Aln[i], a, Ainv[i]) * (xj * bj);
      else return xj * bj;
    };

    // state entering the block, then entering each 16-step sub-block
    float hs[4][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int64_t n = g + 16 * i;
      hs[0][i] = (n < N) ? p.ckpt[((b * nbk + blk) * Dm + dd) * N + n] : 0.0f;
    }
    if constexpr (ZOH) {
      // a rolled loop over the sub-blocks: unrolled, the compiler hoists the ZOH factors of all
      // 48 steps ahead of the state chain and runs out of registers
      float hc[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) hc[i] = hs[0][i];
#pragma unroll 1
      for (int s = 0; s < 3; ++s) {
        const float dts = s == 0 ? dt[0] : (s == 1 ? dt[1] : dt[2]);
        const float xus = s == 0 ? xu[0] : (s == 1 ? xu[1] : xu[2]);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float h = hc[i];
          const float* brow = Bt + (g + 16 * i) * TS + 16 * s;
          static_for<0, 16>([&](auto j_) {
            constexpr int j = decltype(j_)::value;
            const float dj = row_bcast<j>(dts);
            const float a = exp2_(dj * Ap[i]);
            h = __builtin_fmaf(a, h, bbar_u(dj, row_bcast<j>(xus), brow[j], a, i));
          });
          hc[i] = h;
          hs[1][i] = s == 0 ? h : hs[1][i];
          hs[2][i] = s == 1 ? h : hs[2][i];
          hs[3][i] = s == 2 ? h : hs[3][i];
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 3; ++s) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float h = hs[s][i];
          const float* brow = Bt + (g + 16 * i) * TS + 16 * s;
          static_for<0, 16>([&](auto j_) {
            constexpr int j = decltype(j_)::value;
            const float dj = row_bcast<j>(dt[s]);
            const float a = exp2_(dj * Ap[i]);
            h = __builtin_fmaf(a, h, bbar_u(dj, row_bcast<j>(xu[s]), brow[j], a, i));
          });
          hs[s + 1][i] = h;
        }
      }
    }

    float dug[4], ddg[4], dzg[4];
#pragma unroll
    for (int s = 3; s >= 0; --s) {
      auto pick = [&](const float (&v)[4]) { return s == 0 ? v[0] : (s == 1 ? v[1] : (s == 2 ? v[2] : v[3])); };
      const float dt_s = pick(dt), xu_s = pick(xu), uu_s = pick(uu), go_s = pick(go), zz_s = pick(zz),
                  xs_s = pick(xs);
      float hs_s[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) hs_s[i] = s == 0 ? hs[0][i] : (s == 1 ? hs[1][i] : (s == 2 ? hs[2][i] : hs[3][i]));
      float dug_s, ddg_s, dzg_s;
      // The states of the sub-block: a forward pass keeps the states and decay factors for the
      // sweep and gives y (which only dz needs; the sweep needs dy = dout silu(z)).
      float hv[16], av[16];
      float ev[ZOH ? 16 : 1], edv[ZOH ? 16 : 1];  // ZOH: B_bar / B and its A-derivative per step
      float pj[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) pj[j] = 0.0f;
      {
        float h = hs_s[0];
        const float* brow = Bt + g * TS + 16 * s;
        const float* crow = Ct + g * TS + 16 * s;
        static_for<0, 16>([&](auto j_) {
          constexpr int j = decltype(j_)::value;
          const float dj = row_bcast<j>(dt_s);
          const float a = exp2_(dj * Ap[0]);
          if constexpr (ZOH) {
            const float x = dj * Aln[0];
            const float e = zoh_e(dj, x, a, Ainv[0]);
            ev[j] = e;
            edv[j] = zoh_e_dA(dj, x, a, e, Ainv[0]);
            h = __builtin_fmaf(a, h, e * (row_bcast<j>(xu_s) * brow[j]));
          } else {
            h = __builtin_fmaf(a, h, bbar_u(dj, row_bcast<j>(xu_s), brow[j], a, 0));
          }
          av[j] = a;
          hv[j] = h;
          pj[j] = __builtin_fmaf(crow[j], h, pj[j]);
        });
      }
      const float ykeep = row_transpose_sum(pj) + Dd * uu_s;  // y now: pj is not held through the sweep
      float dy = go_s, sg = 0.0f;
      dzg_s = 0.0f;
      if (has_z) {
        sg = logistic_(zz_s);
        dy = go_s * (zz_s * sg);
        dzg_s = go_s * ykeep * (sg * __builtin_fmaf(zz_s, 1.0f - sg, 1.0f));
      }

      // backwards through the sub-block
      float s1[16], s2[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) { s1[j] = 0.0f; s2[j] = 0.0f; }
      float* redw = red + sbp * RED + w * (2 * 16 * NP);  // this wave's [2][16][NP] slice
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float* brow = Bt + (g + 16 * i) * TS + 16 * s;
        const float* crow = Ct + (g + 16 * i) * TS + 16 * s;
        float Gi = G[i], dAi = dAacc[i];
        float xo = 0.0f, yo = 0.0f;  // dB, dC contributions of the odd step of a pair
        static_for<0, 16>([&](auto k_) {
          constexpr int j = 15 - decltype(k_)::value;
          const float dyj = row_bcast<j>(dy);
          Gi = __builtin_fmaf(dyj, crow[j], Gi);
          const float yc = dyj * hv[j];
          const float a = av[j];
          const float hp = j > 0 ? hv[j > 0 ? j - 1 : 0] : hs_s[i];
          const float tt = Gi * hp * a;
          float xb;  // dB contribution
          if constexpr (ZOH) {
            // s1: sum G e B (du);  s2: sum G Abar (h_{t-1} A + u B) (ddt)
            const float dj = row_bcast<j>(dt_s);
            const float uj = row_bcast<j>(xu_s);
            const float e = ev[j];
            const float gb = Gi * brow[j];
            const float gbu = gb * uj;
            s1[j] = __builtin_fmaf(gb, e, s1[j]);
            s2[j] = __builtin_fmaf(tt, Aln[i], __builtin_fmaf(gbu, a, s2[j]));
            dAi = __builtin_fmaf(tt, dj, __builtin_fmaf(gbu, edv[j], dAi));
            xb = Gi * (e * uj);
          } else {
            // s1: sum G B;  s2: sum G Abar h_{t-1} A
            s1[j] = __builtin_fmaf(Gi, brow[j], s1[j]);
            s2[j] = __builtin_fmaf(tt, Aln[i], s2[j]);
            dAi = __builtin_fmaf(tt, row_bcast<j>(dt_s), dAi);
            xb = Gi * row_bcast<j>(xu_s);
          }
          Gi = Gi * a;
          if constexpr (j % 2 == 1) {
            xo = xb;
            yo = yc;
          } else {
            // rows: 0 = dB step j+1, 1 = dB step j, 2 = dC step j+1, 3 = dC step j
            const float v = rows4_sum2(xo, yo, xb, yc);
            const int qty = r >> 1, step = (r & 1) ? j : j + 1;
            redw[(qty * 16 + step) * NP + g + 16 * i] = v;
          }
        });
        G[i] = Gi;
        dAacc[i] = dAi;
      }
      const float S1 = row_transpose_sum(s1);
      const float S2 = row_transpose_sum(s2);
      const int64_t t = t0 + 16 * s + g;
      dug_s = ZOH ? dy * Dd + S1 : dy * Dd + dt_s * S1;
      const float ddt = ZOH ? S2 : uu_s * S1 + S2;
      ddg_s = ddt * logistic_(xs_s);
      if (t < L) {
        dbacc += ddg_s;
        dDacc = __builtin_fmaf(dy, uu_s, dDacc);
      }

      // the workgroup's dB/dC for these 16 steps: add the 4 waves' sums in order
      __syncthreads();
      const float* rb = red + sbp * RED;
      for (int e = tid; e < 2 * 16 * NP; e += 256) {
        const int step = e & 15, n = (e >> 4) % NP, qty = e / (16 * NP);
        const int64_t ts = t0 + 16 * s + step;
        if (n < N && ts < L) {
          const int o = (qty * 16 + step) * NP + n;
          const float v = ((rb[o] + rb[2 * 16 * NP + o]) + rb[2 * 2 * 16 * NP + o]) + rb[3 * 2 * 16 * NP + o];
          p.part_bc[((((int64_t)qty * p.nblk + cb) * p.Bsz + b) * N + n) * L + (REV ? L - 1 - ts : ts)] = v;
        }
      }
      sbp ^= 1;  // the next sub-block writes the other buffer; this one is free after the next barrier
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dug[k] = k == s ? dug_s : dug[k];
        ddg[k] = k == s ? ddg_s : ddg[k];
        dzg[k] = k == s ? dzg_s : dzg[k];
      }
    }
    if (dval) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t t = t0 + 16 * s + g;
        if (t < L) {
          const int64_t ph = REV ? (L - 1 - t) : t;
          store_io(du_row + ph, dug[s]);
          store_io(dd_row + ph, ddg[s]);
          if (has_z) store_io(dz_row + ph, dzg[s]);
        }
      }
    }
  }

  if (dval) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int64_t n = g + 16 * i;
      if (n < N) {
        p.part_a[(b * Dm + d) * N + n] = dAacc[i];
        if (p.dh0) p.dh0[(b * Dm + d) * N + n] = G[i];
      }
    }
  }
  // row sums of the lanes' dD and dbias terms
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    dDacc += __shfl_xor(dDacc, off, 16);
    dbacc += __shfl_xor(dbacc, off, 16);
  }
  if (dval && g == 0) {
    p.part_d[b * Dm + d] = dDacc;
    p.part_d[p.Bsz * Dm + b * Dm + d] = dbacc;
  }
}

// launch of the backward kernel for one discretisation: variants by dtype, state slices
// (N <= 16, 32, 64), direction and whether rows allow 16-byte loads
template <typename IO, int NL, bool ZOH, bool REV, bool VEC>
void go_bwd(const BwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL((scan_bwd_kernel<IO, NL, ZOH, REV, VEC>), dim3((unsigned)(p.Bsz * p.nblk)), dim3(256), 0, s,
                     p);
}

template <typename IO, int NL, bool ZOH>
void go_bwd_flags(const BwdParams& p, hipStream_t s) {
  const int k = (p.reverse ? 2 : 0) + (p.vec ? 1 : 0);
  switch (k) {
    case 0: go_bwd<IO, NL, ZOH, false, false>(p, s); break;
    case 1: go_bwd<IO, NL, ZOH, false, true>(p, s); break;
    case 2: go_bwd<IO, NL, ZOH, true, false>(p, s); break;
    default: go_bwd<IO, NL, ZOH, true, true>(p, s); break;
  }
}

template <bool ZOH>
hipError_t go_bwd_all(const BwdParams& p, bool bf16, hipStream_t s) {
  // up to 16 states (one slice per lane); more states go to chunk_bwd_kernel
  if (bf16) go_bwd_flags<bf16_t, 1, ZOH>(p, s);
  else go_bwd_flags<float, 1, ZOH>(p, s);
  return hipGetLastError();
}

// the checkpoint pass (the scan kernel's mode 2) for one discretisation
template <typename IO, int NL, bool ZOH, bool REV, bool VEC>
void go_ckpt(const ScanParams& p, hipStream_t s) {
  hipLaunchKernelGGL((scan_kernel<IO, NL, 2, ZOH, REV, VEC>), dim3((unsigned)(p.Bsz * p.nblk)), dim3(256), 0, s, p);
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
