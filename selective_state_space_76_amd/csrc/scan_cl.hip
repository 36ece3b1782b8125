// scan_cl.hip -- the forward scan of a split sequence with channels on lanes: the summary and output
// passes for bf16 streams and up to 16 states.
//
// The operation is scan_kernel's (ssm_device.h states it, with its sources); this is a second work
// layout for long sequences over few channels, where the sequence split supplies the parallelism.
// A workgroup is 4 waves and owns 64 consecutive channels of one batch row and one segment.  In a
// wave, lane c of every 16-lane row serves channel 16 w + c, and row r holds states 4 r .. 4 r + 3
// of that channel in registers, so the sum over states is mostly a sum inside the lane.
//
// Per 64-step block the workgroup stages B (and C) as fp32, shared by its 64 channels, and delta,
// u (and z) of its channels as raw bf16 in LDS.  Per 16-step sub-block, row r forms dt and dt u
// for steps r, r + 4, r + 8, r + 12 of its channel, each once; the four rows' values pass through a
// small per-wave LDS area, so every row reads 4 consecutive steps at a time, and each lane runs its
// 4 states' recurrences over those steps.  y = sum_n C h: the lane's 4 states in
// order, then the 4 rows' partial sums over two permlane-swap stages (a fixed order), which leave
// row r with steps 4 r .. 4 r + 3 of the sub-block; it finishes them (D skip, gate, bf16 store).
//
// Used for splits with bf16 streams, the default discretisation (the ZOH factor would need more
// registers than 4 waves per SIMD allow), N <= 16, rows of whole 16-byte chunks (L a multiple of 8)
// and L < 2^24 (a buffer resource spans 8 rows, 16 L bytes, and the step offset 2 t0 is a 32-bit
// scalar; both stay far inside their ranges).  Padding states read zero B and C, channels
// past D read zero and are never written, and steps past the end of the sequence take dt = 0
// (identity steps) and are not stored.
#include <type_traits>

#include "ssm_device.h"

namespace ssm {
namespace {

constexpr int kClTS = 68;  // fp32 B/C tile row: 64 steps + 4 pad
constexpr int kClSP = 72;  // bf16 stream tile row: 64 steps + 8 pad (rows stay 16-byte aligned)

__device__ __forceinline__ uint32_t swap_halves(uint32_t v) { return (v >> 16) | (v << 16); }
__device__ __forceinline__ float bf_at(const bf16_t* row, int j) { return __uint_as_float((uint32_t)row[j] << 16); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(bf16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(bf16_t, (__bf16)hi) << 16);
}

// MODE 0: output pass from the carried state (writes out; the last segment also final_state).
// MODE 1: summary pass over segments 0..S-2 (writes seg_state and seg_dsum).
// GATE: the output pass multiplies by silu(z).
// 4 workgroups (waves per SIMD) for the output pass (its chains, C h sums and prefetch registers
// need up to 128 VGPRs), 5 for the summary pass.
template <int MODE, bool REV, bool GATE>
__global__ __launch_bounds__(256, MODE == 0 ? 4 : 5) void scan_cl_kernel(ScanParams p) {
  constexpr int NT = MODE == 0 ? 2 : 1;               // staged coefficient tensors: B (and C)
  constexpr int NS = MODE == 0 && GATE ? 3 : 2;       // staged channel streams: delta, u (and z)
  constexpr int CPT = 1 + 2 * NS;                     // wave-chunks per wave
  __shared__ __attribute__((aligned(16))) float bct[NT * 16 * kClTS];
  __shared__ __attribute__((aligned(16))) bf16_t stt[NS * 64 * kClSP];
  __shared__ __attribute__((aligned(16))) float xch[4 * 2 * 64];  // per wave: dt, dt u as [c][row]

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int ngrp = (int)((p.Dm + 63) / 64);
  const int S_launch = MODE == 1 ? p.S - 1 : p.S;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int cg = logical % ngrp;
  const int rest = logical / ngrp;
  const int seg = rest % S_launch;
  const int64_t b = rest / S_launch;
  const int64_t L = p.L, N = p.N, Dm = p.Dm;
  const int chl = 16 * w + c;  // channel within the workgroup
  const int64_t d = (int64_t)cg * 64 + chl;
  const bool dval = d < Dm;
  const int64_t dd = dval ? d : Dm - 1;
  const int64_t tb = (int64_t)seg * p.seg_len;
  const int64_t te = (tb + p.seg_len < L) ? tb + p.seg_len : L;

  float Ap[4], h[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t n = 4 * r + k;
    const bool nv = n < N;
    Ap[k] = nv ? p.A[dd * N + n] * kLog2e : 0.0f;  // padding states: A = 0, zero B and C
    h[k] = (MODE == 0 && nv) ? p.carries[(((int64_t)seg * p.Bsz + b) * Dm + dd) * N + n] : 0.0f;
  }
  const float biasd = p.bias ? p.bias[dd] : 0.0f;
  const float Dd = p.D ? p.D[dd] : 0.0f;

  // A block is staged in wave-chunks of 64 16-byte pieces: 8 rows x 8 pieces of 8 steps (lane l:
  // row l / 8, steps 8 (l % 8) ..).  Wave w's chunk 0 is 8 rows of B (waves 0, 1) or C (waves 2, 3;
  // output pass only), states 8 (w % 2) ..; its chunks 1 + 2 i and 2 + 2 i are channels 8 w .. and
  // 32 + 8 w .. of stream i (delta, u, z).  Each reads through a buffer resource over its valid rows:
  // rows past N or D read zero, so every chunk of a lane takes the same 32-bit lane offset, the
  // block's step offset is a scalar, and no chunk needs a branch.
  const int wv = __builtin_amdgcn_readfirstlane(w);
  const int col = (lane & 7) * 8;  // this lane's first step within the block
  const int lrow = lane >> 3;
  __amdgpu_buffer_rsrc_t rs[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const void* base = p.u;
    int64_t rows = 0;
    if (k == 0) {
      const int n0 = 8 * (wv & 1);
      if (MODE == 0 || wv < 2) {
        base = reinterpret_cast<const bf16_t*>(wv < 2 ? p.B : p.C) + (b * N + n0) * L;
        rows = N - n0 < 8 ? N - n0 : 8;
      }
    } else {
      const int sti = (k - 1) >> 1;
      const int64_t d0 = (int64_t)cg * 64 + 8 * (wv + 4 * ((k - 1) & 1));
      base = reinterpret_cast<const bf16_t*>(sti == 0 ? p.delta : (sti == 1 ? p.u : p.z)) + (b * Dm + d0) * L;
      rows = Dm - d0 < 8 ? Dm - d0 : 8;
    }
    rs[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                              (int)(rows > 0 ? rows * L * 2 : 0), 0x00020000);
  }
  // lane offset in bytes: forward, row + col + t0; backward in time, row + (L - 8 - col) - t0, taken
  // as (row + 56 - col) + (L - 64 - t0) for whole blocks
  const uint32_t vo = (uint32_t)(((int64_t)lrow * L + (REV ? 56 - col : col)) * 2);
  uint4 raw[CPT];
  auto chunk = [&](int k, uint32_t voff, int soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs[k], voff, soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  auto fetch = [&](int64_t t0) {
    if (t0 + 64 <= L) {  // the whole block lies inside the rows
      const int soff = (int)((REV ? L - 64 - t0 : t0) * 2);
#pragma unroll
      for (int k = 0; k < CPT; ++k) raw[k] = chunk(k, vo, soff);
      return;
    }
    // the sequence's ragged last block: pieces past the end hold zero, except delta's, which hold
    // -inf so that those steps take dt = softplus(-inf) = 0 exactly (identity steps: the state
    // passes through unchanged)
    const uint32_t vp = REV ? (uint32_t)(((int64_t)lrow * L + L - 8 - col - t0) * 2) : vo;
    const int sp = REV ? 0 : (int)(t0 * 2);
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const uint32_t f = (k == 1 || k == 2) ? 0xff80ff80u : 0u;
      raw[k] = make_uint4(f, f, f, f);
      if (t0 + col < L) raw[k] = chunk(k, vp, sp);
    }
  };
  auto store = [&]() {
    if (MODE == 0 || wv < 2) {
      const uint32_t x[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(x[e] << 16);
        f[2 * e + 1] = __uint_as_float(x[e] & 0xffff0000u);
      }
      float4 lo = make_float4(f[0], f[1], f[2], f[3]), hi = make_float4(f[4], f[5], f[6], f[7]);
      if (REV) {  // physical order is logical order reversed
        lo = make_float4(f[7], f[6], f[5], f[4]);
        hi = make_float4(f[3], f[2], f[1], f[0]);
      }
      float* dp = bct + (16 * (wv >> 1) + 8 * (wv & 1) + lrow) * kClTS + col;
      *reinterpret_cast<float4*>(dp) = lo;
      *reinterpret_cast<float4*>(dp + 4) = hi;
    }
#pragma unroll
    for (int k = 1; k < CPT; ++k) {
      uint4 v = raw[k];
      if (REV) v = make_uint4(swap_halves(v.w), swap_halves(v.z), swap_halves(v.y), swap_halves(v.x));
      const int row = 64 * ((k - 1) >> 1) + 8 * (wv + 4 * ((k - 1) & 1)) + lrow;
      *reinterpret_cast<uint4*>(stt + row * kClSP + col) = v;
    }
  };

  const bf16_t* sd = stt + (0 * 64 + chl) * kClSP;  // this channel's delta row
  const bf16_t* su = stt + (1 * 64 + chl) * kClSP;  // u row
  const bf16_t* sz = stt + (MODE == 0 && GATE ? 2 * 64 + chl : 0) * kClSP;  // z row (output pass)
  bf16_t* sdw = stt + (0 * 64 + chl) * kClSP;  // the delta row again: the output pass's outputs
  float dsum = 0.0f, dcomp = 0.0f;  // Kahan sum of this row's step sizes (summary pass)

  // One 64-step block; WHOLE: all 64 steps lie inside the segment, else the sequence's ragged last
  // block, whose steps past the end are identity steps (see fetch) and are not stored
  auto block = [&](int64_t t0, auto whole) {
    constexpr bool WHOLE = decltype(whole)::value;
    const int rem = WHOLE ? 64 : (int)(te - t0);
    __syncthreads();  // the previous block's readers are done
    store();
    if (t0 + 64 < te) fetch(t0 + 64);  // the next block streams in while this one is computed
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // this row's steps of the sub-block: r, r + 4, r + 8, r + 12 (dt and dt u once per step)
      float dq[4], xq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = 16 * s + r + 4 * q;
        const float uu = bf_at(su, j);
        const float dt = softplus_(bf_at(sd, j) + biasd);
        dq[q] = dt;
        xq[q] = dt * uu;
      }
      if (MODE == 1) {  // the row's 4 steps of the sub-block, then one compensated add
        const float part = (dq[0] + dq[1]) + (dq[2] + dq[3]);
        const float yk = part - dcomp, tk = dsum + yk;
        dcomp = (tk - dsum) - yk;
        dsum = tk;
      }
      float acc[16];
      float* xw = xch + 128 * w;  // this wave's exchange slots
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // steps 4 q .. 4 q + 3 of the sub-block: row r's value of step 4 q + r goes to slot 4 c + r,
        // and every lane of column c reads the 4 slots back as one 16-byte load.  Only this wave
        // uses these slots, and a wave's LDS accesses complete in order, so no barrier is needed.
        xw[4 * c + r] = dq[q];
        xw[64 + 4 * c + r] = xq[q];
        const float4 d4 = *reinterpret_cast<const float4*>(xw + 4 * c);
        const float4 x4 = *reinterpret_cast<const float4*>(xw + 64 + 4 * c);
        const float D4[4] = {d4.x, d4.y, d4.z, d4.w};
        const float X4[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 bq = *reinterpret_cast<const float4*>(bct + (4 * r + k) * kClTS + 16 * s + 4 * q);
          float4 cq = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          if (MODE == 0) cq = *reinterpret_cast<const float4*>(bct + (16 + 4 * r + k) * kClTS + 16 * s + 4 * q);
          const float bb[4] = {bq.x, bq.y, bq.z, bq.w};
          const float cc[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = exp2_(D4[e] * Ap[k]);
            h[k] = __builtin_fmaf(a, h[k], X4[e] * bb[e]);
            if (MODE == 0) acc[4 * q + e] = k == 0 ? cc[e] * h[k] : __builtin_fmaf(cc[e], h[k], acc[4 * q + e]);
          }
        }
      }
      if constexpr (MODE == 0) {
        // rows {0,2} and {1,3} first, then the pairs: row r keeps steps 4 r .. 4 r + 3
        float sA[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[j]), __float_as_uint(acc[j + 8]), false, false);
          sA[j] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
        }
        const int jo = 16 * s + 4 * r;  // the row's 4 output steps in the block
        const uint2 uraw = *reinterpret_cast<const uint2*>(su + jo);
        const float uu[4] = {__uint_as_float(uraw.x << 16), __uint_as_float(uraw.x & 0xffff0000u),
                             __uint_as_float(uraw.y << 16), __uint_as_float(uraw.y & 0xffff0000u)};
        float zz[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (GATE) {
          const uint2 zraw = *reinterpret_cast<const uint2*>(sz + jo);
          zz[0] = __uint_as_float(zraw.x << 16);
          zz[1] = __uint_as_float(zraw.x & 0xffff0000u);
          zz[2] = __uint_as_float(zraw.y << 16);
          zz[3] = __uint_as_float(zraw.y & 0xffff0000u);
        }
        float o[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(sA[jj]), __float_as_uint(sA[jj + 4]), false, false);
          const float y = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
          o[jj] = y + Dd * uu[jj];
          if (GATE) o[jj] *= silu_(zz[jj]);
        }
        // into this channel's delta row, whose steps of this sub-block every row has read
        *reinterpret_cast<uint2*>(sdw + jo) = make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
      }
    }
    if constexpr (MODE == 0) {
      // the wave's 16 channels x 64 outputs, whole 16-byte pieces: lanes 8 i .. 8 i + 7 write one
      // channel's row, so every store fills whole lines (pieces past the segment are not stored)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int pc = lane + 64 * i, row = pc >> 3, cp = (pc & 7) * 8;
        const int64_t dw = (int64_t)cg * 64 + 16 * w + row;
        uint4 v = *reinterpret_cast<const uint4*>(stt + (16 * w + row) * kClSP + cp);
        if (dw < Dm && (WHOLE || cp < rem)) {
          bf16_t* op = reinterpret_cast<bf16_t*>(p.out) + (b * Dm + dw) * L;
          if (REV) {
            v = make_uint4(swap_halves(v.w), swap_halves(v.z), swap_halves(v.y), swap_halves(v.x));
            *reinterpret_cast<uint4*>(op + (L - 8 - (t0 + cp))) = v;
          } else {
            *reinterpret_cast<uint4*>(op + t0 + cp) = v;
          }
        }
      }
    }
  };

  fetch(tb);
  int64_t t0 = tb;
  for (; t0 + 64 <= te; t0 += 64) block(t0, std::true_type{});
  if (t0 < te) block(t0, std::false_type{});

  if constexpr (MODE == 0) {
    if (p.final_state && seg == p.S - 1 && dval) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (4 * r + k < N) p.final_state[(b * Dm + d) * N + 4 * r + k] = h[k];
    }
  } else {
    // the channel's step-size sum: rows {0,2} and {1,3} first, then the pairs (every row gets it)
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(dsum), __float_as_uint(dsum), false, false);
    const float pair = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
    const float tot = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
    if (dval) {
      const int64_t BD = p.Bsz * Dm, BDN = BD * N;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (4 * r + k < N) p.seg_state[(int64_t)seg * BDN + (b * Dm + d) * N + 4 * r + k] = h[k];
      if (r == 0) p.seg_dsum[(int64_t)seg * BD + b * Dm + d] = tot;
    }
  }
}

template <int MODE, bool REV, bool GATE>
void go_cl(const ScanParams& p, hipStream_t s) {
  const int64_t ngrp = (p.Dm + 63) / 64;
  const int64_t S_launch = MODE == 1 ? p.S - 1 : p.S;
  hipLaunchKernelGGL((scan_cl_kernel<MODE, REV, GATE>), dim3((unsigned)(p.Bsz * ngrp * S_launch)), dim3(256), 0, s, p);
}

}  // namespace

hipError_t launch_scan_cl(const ScanParams& p, int mode, hipStream_t s) {
  if (mode == 1) {
    if (p.reverse) go_cl<1, true, false>(p, s);
    else go_cl<1, false, false>(p, s);
  } else if (p.z) {
    if (p.reverse) go_cl<0, true, true>(p, s);
    else go_cl<0, false, true>(p, s);
  } else {
    if (p.reverse) go_cl<0, true, false>(p, s);
    else go_cl<0, false, false>(p, s);
  }
  return hipGetLastError();
}

}  // namespace ssm
