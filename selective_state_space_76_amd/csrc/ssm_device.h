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
// Work layout of scan_kernel:
//   * A workgroup is 4 waves; a wave is 4 rows of 16 lanes; a row owns one
//     channel (b, d), so a workgroup covers 16 consecutive channels of one
//     batch row.  Lane g of a row holds the states n = g + 16*i, i < NL, in
//     registers for the whole sequence (NL = ceil(N/16)).
//   * The sequence is walked in blocks of 64 steps, split in 4 sub-blocks of
//     16.  Lane g owns step g of each sub-block: it loads delta/u/z for that
//     step, computes dt = softplus(.) and dt*u once, and later finishes the
//     output of that step.  Inside a sub-block the row reads step j's dt and
//     dt*u from lane j with a DPP row broadcast (row_newbcast); with 2 or 4
//     states per lane, from the channel's LDS rows, where the row writes them
//     over its already-read steps.  Each (channel, step) value is computed
//     once, not once per state.
//   * Per state update: one multiply for the exp2 argument, v_exp_f32, one
//     multiply for B_bar*u, one FMA for h and one FMA for C*h.  The sum over
//     n of C*h is a reduce-scatter of the 16 x 16 (state x step) tile in
//     registers with DPP adds (row_transpose_sum); lane g ends with step g.
//   * Sequences with too few channels to fill the chip are cut into S
//     segments (with bf16 streams and up to 16 states, the passes run in
//     scan_cl.hip's layout instead): a summary pass scans each segment from a
//     zero state and keeps
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
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// log(1 + e^x) = max(x, 0) + log1p(e^-|x|).  With e = e^-|x| <= 1 and w = fl(1 + e) in
// [1, 2], log1p(e) = log(w) + log(1 + d/w) where d = e - (w - 1) is the exact rounding
// error of w (Sterbenz); adding d instead of log(1 + d/w) errs by under |d| (1 - 1/w) <=
// 2^-25 absolute, while it restores the bits of e that w lost when e is small.  (With
// e^x itself, w grows without bound and so does that error: 0.5 at x = 16.)
__device__ __forceinline__ float softplus_(float x) {
  const float e = exp2_(-fabsf(x) * kLog2e);
  const float w = 1.0f + e;
  const float d = e - (w - 1.0f);
  return fmaxf(x, 0.0f) + __builtin_fmaf(log2_(w), kLn2, d);
}

__device__ __forceinline__ float silu_(float z) { return z * rcp_(1.0f + exp2_(-z * kLog2e)); }

// Zero-order hold: B_bar / B = (e^x - 1) / A = dt phi(x) with x = dt A, a = e^x and ia = 1 / A
// (taken once per state where A is fixed, so no division per step), phi(x) = (e^x - 1) / x.
// Below |x| = 0.03 from phi's Taylor series to x^3 (the next term is under 1e-8 relative);
// above it (a - 1) / A, where the rounding of a costs under 4e-6 relative.  A = 0 takes the
// series branch (ia is then infinite and its product discarded).
__device__ __forceinline__ float zoh_e(float dt, float x, float a, float ia) {
  const float series = dt * (1.0f + x * (0.5f + x * (0.16666667f + x * 0.041666668f)));
  return (fabsf(x) < 0.03f) ? series : (a - 1.0f) * ia;
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
  // bound_ctrl set and full masks: every lane is written, so the move can fold
  // into the consuming VALU op as a DPP source operand
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + J, 0xf, 0xf, true));
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

// ------------------------------------------------------------- scan kernel

// Lane g of each 16-lane row returns the sum over the row's lanes n of v_n[g]:
// a reduce-scatter of a 16 x 16 tile entirely in registers.  Four butterfly
// stages exchange half of the remaining values with partner lane g^8
// (row_ror:8), g^7 (row_half_mirror), g^2 and g^1 (quad_perm).  In the first
// two stages the half a lane keeps depends on lane bits 3 and 2, which are
// exactly the DPP banks, so each output is two bank-masked DPP adds into the
// same register; the last two stages select with v_cndmask.  Each asm block
// starts with the two wait states a DPP read of a just-written VGPR needs.
__device__ __forceinline__ float row_transpose_sum(const float (&v)[16]) {
  float a0, a1, a2, a3, a4, a5, a6, a7;
  asm volatile(
      "s_nop 1\n"
      "v_add_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %0, %16, %16 row_ror:8 row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %1, %17, %17 row_ror:8 row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %2, %18, %18 row_ror:8 row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %3, %19, %19 row_ror:8 row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %4, %12, %12 row_ror:8 row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %4, %20, %20 row_ror:8 row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %5, %13, %13 row_ror:8 row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %5, %21, %21 row_ror:8 row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %6, %14, %14 row_ror:8 row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %6, %22, %22 row_ror:8 row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %7, %15, %15 row_ror:8 row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %7, %23, %23 row_ror:8 row_mask:0xf bank_mask:0xc\n"
      : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(a4), "=&v"(a5), "=&v"(a6), "=&v"(a7)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
        "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
  float b0, b1, b2, b3;
  asm volatile(
      "s_nop 1\n"
      "v_add_f32_dpp %0, %4, %4 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %0, %8, %8 row_half_mirror row_mask:0xf bank_mask:0xa\n"
      "v_add_f32_dpp %1, %5, %5 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %1, %9, %9 row_half_mirror row_mask:0xf bank_mask:0xa\n"
      "v_add_f32_dpp %2, %6, %6 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %2, %10, %10 row_half_mirror row_mask:0xf bank_mask:0xa\n"
      "v_add_f32_dpp %3, %7, %7 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %3, %11, %11 row_half_mirror row_mask:0xf bank_mask:0xa\n"
      : "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(a4), "v"(a5), "v"(a6), "v"(a7));
  float out, k0, s0, k1, s1, c0, c1;
  asm volatile(
      "v_cndmask_b32_e64 %1, %7, %9, %11\n"   // lane bit 1 set: keep b2, send b0
      "v_cndmask_b32_e64 %2, %9, %7, %11\n"
      "v_cndmask_b32_e64 %3, %8, %10, %11\n"  // lane bit 1 set: keep b3, send b1
      "v_cndmask_b32_e64 %4, %10, %8, %11\n"
      "s_nop 1\n"
      "v_add_f32_dpp %5, %2, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
      "v_add_f32_dpp %6, %4, %3 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_cndmask_b32_e64 %1, %5, %6, %12\n"   // lane bit 0 set: keep c1, send c0
      "v_cndmask_b32_e64 %2, %6, %5, %12\n"
      "s_nop 1\n"
      "v_add_f32_dpp %0, %2, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
      : "=&v"(out), "=&v"(k0), "=&v"(s0), "=&v"(k1), "=&v"(s1), "=&v"(c0), "=&v"(c1)
      : "v"(b0), "v"(b1), "v"(b2), "v"(b3), "s"(0xCCCCCCCCCCCCCCCCull), "s"(0xAAAAAAAAAAAAAAAAull));
  return out;
}

// MODE 0: output pass (writes out and, for the last segment, final_state; with
//         ckpt set also the state entering every 64-step block, for the backward).
// MODE 1: summary pass over segments 0..S-2 (writes seg_state and seg_dsum).
// MODE 2: checkpoint pass for the backward (writes the state entering every
//         64-step block to ckpt; a split sequence starts each segment from its carry).
// REV: logical step t reads physical position L-1-t.  VEC: rows allow 16-byte
// vector loads (L a multiple of 8 for bf16, of 4 for fp32, 8 <= L < 2^24).
//
// Per 64-step block the workgroup stages, as fp32 in LDS, B (and C) for all
// states (rows >= N stay zero) and delta/u/z of its 16 channels, all fetched
// with coalesced 16-byte loads one block ahead into registers.
// Waves per SIMD the output pass is built for: 4 with one state per lane (3 with
// ZOH), 3 with 64 bf16 states (168 VGPRs, which the buffer-resource staging below
// leaves room for), 2 otherwise.
template <typename IO, int NL, int MODE, bool ZOH, bool REV, bool VEC>
__global__ __launch_bounds__(256, MODE == 0 ? (NL == 1 ? (ZOH ? 3 : 4) : (NL == 4 && !ZOH && sizeof(IO) == 2 ? 3 : 2)) : 2) void scan_kernel(ScanParams p) {
  constexpr int NP = 16 * NL;                  // states padded to the lane grid
  constexpr int TS = 68;                       // LDS tile row: 64 steps + 4 pad (floats)
  constexpr int NT = MODE == 0 ? 2 : 1;        // staged coefficient tensors: B and C, or B only
  constexpr int NS = MODE == 0 ? 3 : 2;        // staged channel streams: delta, u (and z)
  constexpr int EPC = 16 / (int)sizeof(IO);    // elements per 16-byte chunk
  constexpr int CPR = 64 / EPC;                // chunks per 64-step row
  constexpr int NBC = NT * NP * CPR;           // coefficient chunks
  constexpr int NCH = NBC + NS * 16 * CPR;     // + channel-stream chunks
  constexpr int CPT = (NCH + 255) / 256;       // chunks per thread
  // One state per lane: single-buffered tiles (21.8 KB) so 4 workgroups fit a CU -- a fourth wave per
  // SIMD measured faster than double buffering with 3.  The ZOH variant needs more registers than 4
  // waves allow, so it keeps 3 waves and double-buffered tiles (one barrier per block).
  constexpr int NBUF = (NL == 1 && ZOH) ? 2 : 1;
  constexpr int TILE = NT * NP * TS + NS * 16 * TS;
  __shared__ __attribute__((aligned(16))) float tiles[NBUF * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int r = lane >> 4, g = lane & 15;
  const int S_launch = MODE == 1 ? p.S - 1 : p.S;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = logical % p.nblk;
  const int rest = logical / p.nblk;
  const int seg = rest % S_launch;
  const int64_t b = rest / S_launch;
  const int64_t L = p.L, N = p.N, Dm = p.Dm;
  const int cl = w * 4 + r;                    // channel within the workgroup
  const int64_t d = (int64_t)cb * 16 + cl;
  const bool dval = d < Dm;
  const int64_t dd = dval ? d : Dm - 1;
  const int64_t tb = (int64_t)seg * p.seg_len;
  const int64_t te = (tb + p.seg_len < L) ? tb + p.seg_len : L;
  const bool has_z = MODE == 0 && p.z != nullptr;

  IO* orow = MODE == 0 ? reinterpret_cast<IO*>(p.out) + (b * Dm + dd) * L : nullptr;
  const float biasd = p.bias ? p.bias[dd] : 0.0f;
  const float Dd = p.D ? p.D[dd] : 0.0f;

  float Ap[NL], Aln[NL], Ainv[NL], h[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int64_t n = g + 16 * i;
    const bool nv = n < N;
    const int64_t nn = nv ? n : N - 1;
    const float a = p.A[dd * N + nn];
    Aln[i] = nv ? a : 0.0f;
    Ap[i] = Aln[i] * kLog2e;
    Ainv[i] = ZOH ? 1.0f / Aln[i] : 0.0f;
    float h0 = 0.0f;
    if (MODE != 1) {
      if (p.carries) h0 = p.carries[(((int64_t)seg * p.Bsz + b) * Dm + dd) * N + nn];
      else if (p.init) h0 = p.init[(b * Dm + dd) * N + nn];
    }
    h[i] = nv ? h0 : 0.0f;
  }

  // zero the tiles once: padding states, missing channels and steps past the end read 0
  for (int i = tid; i < NBUF * TILE; i += 256) tiles[i] = 0.0f;

  // ---- chunk k of this thread: source row, destination offset in a tile (fixed for the whole kernel)
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
      const void* base = st == 0 ? p.delta : (st == 1 ? p.u : p.z);
      live[k] = dr < Dm && base != nullptr;
      src[k] = reinterpret_cast<const IO*>(live[k] ? base : p.u) + (b * Dm + (dr < Dm ? dr : 0)) * L;
      dst[k] = NT * NP * TS + (st * 16 + row) * TS + col[k];
    }
  }

  // Rows of whole 16-byte pieces (VEC): every region of the chunk slots (B, C, each channel stream) is a
  // whole number of 64-slot groups, so wave w's chunk k -- slots 256 k + 64 w + lane -- lies in one
  // tensor and covers RPC consecutive rows of it (lane: row lane / CPR, piece lane % CPR).  Each such
  // chunk reads through a buffer resource over its valid rows, so rows past N or D read zero, every
  // chunk of a lane takes the same 32-bit lane offset, and the block's step offset is a scalar.  The
  // host keeps L below 2^24 on this path (each resource spans RPC rows of L elements).
  constexpr int RPC = 64 / CPR;
  const int wv = __builtin_amdgcn_readfirstlane(w);
  const int lrow = lane / CPR, lcol = (lane % CPR) * EPC;
  __amdgpu_buffer_rsrc_t rs[CPT];
  int dbase[CPT];
  bool wok[CPT];
  uint32_t voff = 0;
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c0 = 256 * k + 64 * wv;  // the chunk's first slot
      const void* base = p.u;
      int64_t rows = 0;
      dbase[k] = 0;
      wok[k] = c0 < NCH;
      if (c0 < NBC) {
        const int tt = c0 / (NP * CPR), n0 = (c0 / CPR) % NP;
        if (n0 < N) {
          base = reinterpret_cast<const IO*>(tt == 0 ? p.B : p.C) + (b * N + n0) * L;
          rows = N - n0 < RPC ? N - n0 : RPC;
        }
        dbase[k] = (tt * NP + n0) * TS;
      } else if (c0 < NCH) {
        const int e = c0 - NBC;
        const int st = e / (16 * CPR), row0 = (e / CPR) % 16;
        const int64_t dr0 = (int64_t)cb * 16 + row0;
        const void* sb = st == 0 ? p.delta : (st == 1 ? p.u : p.z);
        if (sb != nullptr && dr0 < Dm) {
          base = reinterpret_cast<const IO*>(sb) + (b * Dm + dr0) * L;
          rows = Dm - dr0 < RPC ? Dm - dr0 : RPC;
        }
        dbase[k] = NT * NP * TS + (st * 16 + row0) * TS;
      }
      rs[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                                (int)(rows * L * (int64_t)sizeof(IO)), 0x00020000);
    }
    // lane offset in bytes: forward, row + piece + t0; backward in time, row + (L - EPC - piece) - t0,
    // taken as (row + 64 - EPC - piece) + (L - 64 - t0) for whole blocks
    voff = (uint32_t)(((int64_t)lrow * L + (REV ? 64 - EPC - lcol : lcol)) * (int64_t)sizeof(IO));
  }
  auto vload = [&](int k, uint32_t vo, int so) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs[k], vo, so, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };

  // Other rows: element loads with bounds checks, through the chunks' row pointers.
  uint4 raw[CPT];
  auto fetch = [&](int64_t t0) {
    if constexpr (VEC) {
      if (t0 + 64 <= L) {  // the whole block lies inside the rows
        const int so = (int)((REV ? L - 64 - t0 : t0) * (int64_t)sizeof(IO));
#pragma unroll
        for (int k = 0; k < CPT; ++k)
          if (wok[k]) raw[k] = vload(k, voff, so);
        return;
      }
      // the sequence's ragged last block: pieces at or past L hold zero
      const int64_t ts = t0 + lcol;
      const uint32_t vr = (uint32_t)(((int64_t)lrow * L + (REV ? L - EPC - ts : ts)) * (int64_t)sizeof(IO));
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        raw[k] = make_uint4(0, 0, 0, 0);
        if (wok[k] && ts < L) raw[k] = vload(k, vr, 0);
      }
      return;
    } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int64_t ts = t0 + col[k];  // first logical step of the chunk
      uint4 v = make_uint4(0, 0, 0, 0);
      if (live[k] && ts < L) {
        IO e[EPC];
#pragma unroll
        for (int k2 = 0; k2 < EPC; ++k2) {
          // physical order inside the chunk matches the vector path
          const int64_t lt = REV ? (ts + EPC - 1 - k2) : (ts + k2);
          e[k2] = (lt < L) ? src[k][REV ? (L - 1 - lt) : lt] : IO(0);
        }
        v = *reinterpret_cast<const uint4*>(e);
      }
      raw[k] = v;
    }
    }
  };
  auto store = [&](float* tile) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const bool go = VEC ? wok[k] : live[k];
      if (go) {
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
        float* dp = tile + (VEC ? dbase[k] + lrow * TS + lcol : dst[k]);
#pragma unroll
        for (int k2 = 0; k2 < EPC; k2 += 4) {
          float4 o;
          if (REV) o = make_float4(f[EPC - 1 - k2], f[EPC - 2 - k2], f[EPC - 3 - k2], f[EPC - 4 - k2]);
          else o = make_float4(f[k2], f[k2 + 1], f[k2 + 2], f[k2 + 3]);
          *reinterpret_cast<float4*>(dp + k2) = o;
        }
      }
    }
  };

  float dsum = 0.0f, dcomp = 0.0f;  // Kahan sum of dt over this lane's steps (summary pass)

  fetch(tb);
  if (NBUF == 2) {  // block 0 goes straight into buffer 0; block 1 streams in during block 0
    __syncthreads();  // every thread's share of the zero fill lands before any chunk is stored
    store(tiles);
    fetch(tb + 64);
  }
  int64_t blk = 0;
  for (int64_t t0 = tb; t0 < te; t0 += 64, ++blk) {
    float* tile = tiles + (NBUF == 2 ? (int)(blk & 1) * TILE : 0);
    if (NBUF == 2) {
      // buffer blk&1 holds this block (written during the previous one); the other buffer's last
      // readers finished the previous block before this barrier, so the next block can go there
      __syncthreads();
      if (t0 + 64 < te) {
        store(tiles + (int)((blk + 1) & 1) * TILE);
        if (t0 + 128 < te) fetch(t0 + 128);
      }
    } else {
      __syncthreads();  // every wave is done with the previous block's tile
      store(tile);
      if (t0 + 64 < te) fetch(t0 + 64);  // next block streams in while this one is computed
      __syncthreads();  // tile visible
    }
    if ((MODE == 2 || (MODE == 0 && p.ckpt != nullptr)) && dval) {  // the state entering the block
      const int64_t nbk = (L + 63) / 64;
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (g + 16 * i < N) p.ckpt[((b * nbk + t0 / 64) * Dm + d) * N + g + 16 * i] = h[i];
    }
    const float* Bt = tile;
    const float* Ct = tile + (MODE == 0 ? NP * TS : 0);
    const float* dch = tile + NT * NP * TS + cl * TS;          // this channel's delta row
    const float* uch = tile + NT * NP * TS + (16 + cl) * TS;   // u row
    const float* zch = tile + NT * NP * TS + (32 + cl) * TS;   // z row (output pass)

    // this lane's own steps: issue all LDS reads first, then compute
    float dl[4], xu[4], uu[4], gz[4], zr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      dl[s] = dch[16 * s + g];
      uu[s] = uch[16 * s + g];
      zr[s] = has_z ? zch[16 * s + g] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t t = t0 + 16 * s + g;
      gz[s] = has_z ? silu_(zr[s]) : 1.0f;  // output gate of this step
      const float dt = t < te ? softplus_(dl[s] + biasd) : 0.0f;
      dl[s] = dt;
      xu[s] = ZOH ? uu[s] : dt * uu[s];
      if (MODE == 1) {
        const float yk = dt - dcomp;
        const float tk = dsum + yk;
        dcomp = (tk - dsum) - yk;
        dsum = tk;
      }
    }

    // B and C of a sub-block in registers; with one state per lane the next
    // sub-block's values are read from LDS while this one computes
    constexpr bool PREF = NL == 1;
    float bcur[NL][16], ccur[NL][16], bnxt[NL][16], cnxt[NL][16];
    auto read_bc = [&](int s, float (&bb)[NL][16], float (&cc)[NL][16]) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 vb = *reinterpret_cast<const float4*>(Bt + (g + 16 * i) * TS + 16 * s + 4 * q);
          bb[i][4 * q] = vb.x; bb[i][4 * q + 1] = vb.y; bb[i][4 * q + 2] = vb.z; bb[i][4 * q + 3] = vb.w;
          if (MODE == 0) {
            const float4 vc = *reinterpret_cast<const float4*>(Ct + (g + 16 * i) * TS + 16 * s + 4 * q);
            cc[i][4 * q] = vc.x; cc[i][4 * q + 1] = vc.y; cc[i][4 * q + 2] = vc.z; cc[i][4 * q + 3] = vc.w;
          }
        }
    };
    if (PREF) read_bc(0, bcur, ccur);

    float ys[4];
    if constexpr (ZOH) {
      // The ZOH factor makes phase A larger; fully unrolled, the compiler hoists it across sub-blocks
      // and slices and spills.  So the sub-blocks run in a rolled loop and each state slice fuses its
      // factors with its chain, reading its B/C just before use.
#pragma unroll 1
      for (int s = 0; s < 4; ++s) {
        const float dls = s == 0 ? dl[0] : (s == 1 ? dl[1] : (s == 2 ? dl[2] : dl[3]));
        const float xus = s == 0 ? xu[0] : (s == 1 ? xu[1] : (s == 2 ? xu[2] : xu[3]));
        float pj[16];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          // an empty asm that takes the previous slice's end state and hands on this slice's step
          // values: the slices then run one after the other instead of being hoisted together
          float dli = dls, xui = xus;
          if (i > 0) asm volatile("" : "+v"(dli), "+v"(xui) : "v"(h[i > 0 ? i - 1 : 0]) : "memory");
          float bb[16], cc[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 vb = *reinterpret_cast<const float4*>(Bt + (g + 16 * i) * TS + 16 * s + 4 * q);
            bb[4 * q] = vb.x; bb[4 * q + 1] = vb.y; bb[4 * q + 2] = vb.z; bb[4 * q + 3] = vb.w;
            if (MODE == 0) {
              const float4 vc = *reinterpret_cast<const float4*>(Ct + (g + 16 * i) * TS + 16 * s + 4 * q);
              cc[4 * q] = vc.x; cc[4 * q + 1] = vc.y; cc[4 * q + 2] = vc.z; cc[4 * q + 3] = vc.w;
            }
          }
          float hi = h[i];
          static_for<0, 16>([&](auto j_) {
            constexpr int j = decltype(j_)::value;
            const float dj = row_bcast<j>(dli);
            const float a = exp2_(dj * Ap[i]);
            const float x = zoh_e(dj, dj * Aln[i], a, Ainv[i]) * (row_bcast<j>(xui) * bb[j]);
            hi = __builtin_fmaf(a, hi, x);
            if (MODE == 0) pj[j] = (i == 0) ? cc[j] * hi : __builtin_fmaf(cc[j], hi, pj[j]);
          });
          h[i] = hi;
        }
        if (MODE == 0) {
          const float uus = s == 0 ? uu[0] : (s == 1 ? uu[1] : (s == 2 ? uu[2] : uu[3]));
          const float gzs = s == 0 ? gz[0] : (s == 1 ? gz[1] : (s == 2 ? gz[2] : gz[3]));
          const float yv = (row_transpose_sum(pj) + Dd * uus) * gzs;
          ys[0] = s == 0 ? yv : ys[0];
          ys[1] = s == 1 ? yv : ys[1];
          ys[2] = s == 2 ? yv : ys[2];
          ys[3] = s == 3 ? yv : ys[3];
        }
      }
    } else if constexpr (NL > 1) {
      // Several states per lane: per sub-block the 16 step values are broadcast once, then each state
      // slice reads its own B/C and runs its decay factors, chain and C.h terms before the next slice
      // starts (fewer live registers than all slices' factors at once).
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float dj[16], xj[16], pj[16];
        // the row's 16 lanes have read their steps of this channel's delta and u rows (above), so
        // they overwrite sub-block s with dt and dt u and read all 16 back; only this row reads
        // these two rows and a wave's LDS accesses complete in order, so no barrier is needed
        float* dw = const_cast<float*>(dch) + 16 * s;
        float* xw = const_cast<float*>(uch) + 16 * s;
        dw[g] = dl[s];
        xw[g] = xu[s];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 vd = *reinterpret_cast<const float4*>(dw + 4 * q);
          const float4 vx = *reinterpret_cast<const float4*>(xw + 4 * q);
          dj[4 * q] = vd.x; dj[4 * q + 1] = vd.y; dj[4 * q + 2] = vd.z; dj[4 * q + 3] = vd.w;
          xj[4 * q] = vx.x; xj[4 * q + 1] = vx.y; xj[4 * q + 2] = vx.z; xj[4 * q + 3] = vx.w;
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float hi = h[i];
          // an empty asm that makes this slice's chain start after the previous slice's C.h terms
          if (i > 0) asm volatile("" : "+v"(hi) : "v"(MODE == 0 ? pj[15] : h[i > 0 ? i - 1 : 0]) : "memory");
          float bb[16], cc[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 vb = *reinterpret_cast<const float4*>(Bt + (g + 16 * i) * TS + 16 * s + 4 * q);
            bb[4 * q] = vb.x; bb[4 * q + 1] = vb.y; bb[4 * q + 2] = vb.z; bb[4 * q + 3] = vb.w;
            if (MODE == 0) {
              const float4 vc = *reinterpret_cast<const float4*>(Ct + (g + 16 * i) * TS + 16 * s + 4 * q);
              cc[4 * q] = vc.x; cc[4 * q + 1] = vc.y; cc[4 * q + 2] = vc.z; cc[4 * q + 3] = vc.w;
            }
          }
          float av[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) av[j] = exp2_(dj[j] * Ap[i]);
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            hi = __builtin_fmaf(av[j], hi, xj[j] * bb[j]);
            if (MODE == 0) pj[j] = (i == 0) ? cc[j] * hi : __builtin_fmaf(cc[j], hi, pj[j]);
          }
          h[i] = hi;
        }
        if (MODE == 0) ys[s] = (row_transpose_sum(pj) + Dd * uu[s]) * gz[s];
      }
    } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (PREF) {
        if (s + 1 < 4) read_bc(s + 1, bnxt, cnxt);
      } else {
        read_bc(s, bcur, ccur);
      }
      // phase A: decay factors and inputs of the 16 steps
      float av[16][NL], xv[16][NL];
      static_for<0, 16>([&](auto j_) {
        constexpr int j = decltype(j_)::value;
        const float dj = row_bcast<j>(dl[s]);
        const float xj = row_bcast<j>(xu[s]);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const float bv = bcur[i][j];
          const float a = exp2_(dj * Ap[i]);
          av[j][i] = a;
          if (ZOH) xv[j][i] = zoh_e(dj, dj * Aln[i], a, Ainv[i]) * (xj * bv);
          else xv[j][i] = xj * bv;
        }
      });
      // phase B: the state chain and each step's C.h terms
      float pj[16];
      static_for<0, 16>([&](auto j_) {
        constexpr int j = decltype(j_)::value;
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          h[i] = __builtin_fmaf(av[j][i], h[i], xv[j][i]);
          if (MODE == 0) {
            const float cv = ccur[i][j];
            acc = (i == 0) ? cv * h[i] : __builtin_fmaf(cv, h[i], acc);
          }
        }
        pj[j] = acc;
      });
      if (MODE == 0) ys[s] = (row_transpose_sum(pj) + Dd * uu[s]) * gz[s];
      if (PREF && s + 1 < 4) {
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int j = 0; j < 16; ++j) { bcur[i][j] = bnxt[i][j]; ccur[i][j] = cnxt[i][j]; }
      }
    }
    }
    if (MODE == 0 && dval) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t t = t0 + 16 * s + g;
        if (t < te) store_io(orow + (REV ? (L - 1 - t) : t), ys[s]);
      }
    }
  }

  if (MODE == 0) {
    if (p.final_state && seg == p.S - 1 && dval) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (g + 16 * i < N) p.final_state[(b * Dm + d) * N + g + 16 * i] = h[i];
    }
  } else if (MODE == 1) {
    // row sum of the lanes' step-size sums
    float ds = dsum;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) ds += __shfl_xor(ds, off, 16);
    const int64_t bd = b * Dm + d;
    if (dval) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (g + 16 * i < N) p.seg_state[((int64_t)seg * p.Bsz * Dm) * N + bd * N + g + 16 * i] = h[i];
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
    // the state is streamed once per step: nontemporal accesses keep it from displacing
    // the reused operands (A, B, C) in the caches
    const f32x4 hq = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(st));
    const float4 aq = *reinterpret_cast<const float4*>(p.A + d * N + n0);
    hv[0] = hq.x; hv[1] = hq.y; hv[2] = hq.z; hv[3] = hq.w;
    Av[0] = aq.x; Av[1] = aq.y; Av[2] = aq.z; Av[3] = aq.w;
    if constexpr (sizeof(IO) == 2) {  // 4 bf16 states = one 8-byte load each
      const uint2 bq = *reinterpret_cast<const uint2*>(Bp + n0);
      const uint2 cq = *reinterpret_cast<const uint2*>(Cp + n0);
      Bv[0] = __uint_as_float(bq.x << 16); Bv[1] = __uint_as_float(bq.x & 0xffff0000u);
      Bv[2] = __uint_as_float(bq.y << 16); Bv[3] = __uint_as_float(bq.y & 0xffff0000u);
      Cv[0] = __uint_as_float(cq.x << 16); Cv[1] = __uint_as_float(cq.x & 0xffff0000u);
      Cv[2] = __uint_as_float(cq.y << 16); Cv[3] = __uint_as_float(cq.y & 0xffff0000u);
    } else {
      const float4 bq = *reinterpret_cast<const float4*>(Bp + n0);
      const float4 cq = *reinterpret_cast<const float4*>(Cp + n0);
      Bv[0] = bq.x; Bv[1] = bq.y; Bv[2] = bq.z; Bv[3] = bq.w;
      Cv[0] = cq.x; Cv[1] = cq.y; Cv[2] = cq.z; Cv[3] = cq.w;
    }
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
    if (ZOH) x = zoh_e(dt, dt * Av[k], a, rcp_(Av[k])) * (xu * Bv[k]);
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
      const f32x4 o = {hv[0], hv[1], hv[2], hv[3]};
      __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(st));
    } else if (p.vec == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (n0 + k < N) st[k] = hv[k];
    }
  }
}

// Decode step when N is a multiple of 4: G lanes per channel (G >= N/4, a power of two) with 4
// states each, and U slots per lane: the same channel and state quad in U batch rows ceil(B/U)
// apart, so the lane reads its A quad once for all of them.  Every slot's loads (the state with a
// nontemporal 16-byte access, B, C and the channel's delta/u/z) are issued before any arithmetic,
// so each lane keeps U x 16 bytes of state in flight; each load instruction of a wave still covers
// contiguous memory (consecutive lanes, consecutive channels of one batch row).
template <typename IO, int G, int U, bool ZOH>
__global__ __launch_bounds__(256) void step4_kernel(StepParams p) {
  const int64_t BD = p.Bsz * p.Dm;
  const int64_t N = p.N;
  // Loads are unconditional, from addresses clamped into range, so all slots' loads issue back to
  // back; lanes past the last channel or the last state quad are masked out by selects and by the
  // guarded stores.
  f32x4 hq[U];
  float4 aq[U];
  float Bv[U][4], Cv[U][4];
  float dlv[U], uvv[U], zvv[U], bsv[U], dsv[U];
  int64_t ccs[U], n0s[U];
  int qs[U];
  bool cvs[U], lv[U];
  const void* zsrc = p.z ? p.z : p.u;  // without a gate the loaded value is unused
  // the U slots of a lane are the same channel d and state quad in U batch rows BU apart, so A is
  // read once per lane
  const int64_t BU = (p.Bsz + U - 1) / U;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t c0 = gid / G;
  const int q0 = (int)(gid % G);
  const bool c0v = c0 < BU * p.Dm;
  const int64_t c0c = c0v ? c0 : 0;
  const int64_t b0 = c0c / p.Dm, d0 = c0c - b0 * p.Dm;
  const int64_t n00 = 4 * (int64_t)q0;
  const int64_t nc0 = n00 < N ? n00 : 0;
  const float4 aq0 = *reinterpret_cast<const float4*>(p.A + d0 * N + nc0);
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t bk = b0 + k * BU;
    const bool cval = c0v && bk < p.Bsz;
    const int64_t cc = cval ? bk * p.Dm + d0 : BD - 1;
    const int64_t b = cc / p.Dm;
    const int64_t nc = nc0;
    ccs[k] = cc; n0s[k] = nc; qs[k] = q0; cvs[k] = cval; lv[k] = cval && n00 < N;
    hq[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.state + cc * N + nc));
    aq[k] = aq0;
    const IO* Bp = reinterpret_cast<const IO*>(p.B) + b * N + nc;
    const IO* Cp = reinterpret_cast<const IO*>(p.C) + b * N + nc;
    if constexpr (sizeof(IO) == 2) {  // 4 bf16 states = one 8-byte load each
      const uint2 bq = *reinterpret_cast<const uint2*>(Bp);
      const uint2 cq = *reinterpret_cast<const uint2*>(Cp);
      Bv[k][0] = __uint_as_float(bq.x << 16); Bv[k][1] = __uint_as_float(bq.x & 0xffff0000u);
      Bv[k][2] = __uint_as_float(bq.y << 16); Bv[k][3] = __uint_as_float(bq.y & 0xffff0000u);
      Cv[k][0] = __uint_as_float(cq.x << 16); Cv[k][1] = __uint_as_float(cq.x & 0xffff0000u);
      Cv[k][2] = __uint_as_float(cq.y << 16); Cv[k][3] = __uint_as_float(cq.y & 0xffff0000u);
    } else {
      const float4 bq = *reinterpret_cast<const float4*>(Bp);
      const float4 cq = *reinterpret_cast<const float4*>(Cp);
      Bv[k][0] = bq.x; Bv[k][1] = bq.y; Bv[k][2] = bq.z; Bv[k][3] = bq.w;
      Cv[k][0] = cq.x; Cv[k][1] = cq.y; Cv[k][2] = cq.z; Cv[k][3] = cq.w;
    }
    dlv[k] = to_f32(reinterpret_cast<const IO*>(p.delta)[cc]);
    uvv[k] = to_f32(reinterpret_cast<const IO*>(p.u)[cc]);
    zvv[k] = to_f32(reinterpret_cast<const IO*>(zsrc)[cc]);
    bsv[k] = p.bias ? p.bias[d0] : 0.0f;
    dsv[k] = p.D ? p.D[d0] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t cc = ccs[k];
    const float dt = softplus_(dlv[k] + bsv[k]);
    const float xu = ZOH ? uvv[k] : dt * uvv[k];
    const float hv[4] = {hq[k].x, hq[k].y, hq[k].z, hq[k].w};
    const float Av[4] = {aq[k].x, aq[k].y, aq[k].z, aq[k].w};
    float hn[4];
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = exp2_(dt * Av[e] * kLog2e);
      float x;
      if (ZOH) x = zoh_e(dt, dt * Av[e], a, rcp_(Av[e])) * (xu * Bv[k][e]);
      else x = xu * Bv[k][e];
      hn[e] = __builtin_fmaf(a, hv[e], x);
      acc = __builtin_fmaf(lv[k] ? Cv[k][e] : 0.0f, hn[e], acc);  // padding quads add nothing
    }
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, G);
    if (cvs[k] && qs[k] == 0) {
      float y = acc + dsv[k] * uvv[k];
      if (p.z) y *= silu_(zvv[k]);
      store_io(reinterpret_cast<IO*>(p.out) + cc, y);
    }
    if (lv[k]) {
      const f32x4 o = {hn[0], hn[1], hn[2], hn[3]};
      __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(p.state + cc * N + n0s[k]));
    }
  }
}

}  // namespace ssm
