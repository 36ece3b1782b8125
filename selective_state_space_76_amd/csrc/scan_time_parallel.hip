// scan_time_parallel.hip -- the selective scan in the time-parallel layout, built beside the library
// (its own shared object, libssmtp.so, not part of the C ABI) so that the library's layout choice can
// be measured against it: bench.py times both on the same inputs, and a GPU test holds this one to
// the oracle.
//
// Operation: the forward scan of ssm_device.h (dt = softplus(delta + bias), A_bar = exp(dt A),
// B_bar u = dt u B, h = A_bar h + B_bar u, y = C.h + D u, out = y silu(z)), bf16 streams, the default
// discretisation, up to 16 states, forward in time, L a multiple of 8.
//
// Layout: the pages' associative scan over time (the pair (A_bar, B_bar u) composes as
// (a, b) o (a', b') = (a a', a' b + b'): freeguideonline.com Mamba tutorial, section 5.1), with the
// expanded state kept on chip (section 5.2).  A workgroup is 4 waves of 4 rows of 16 lanes; a row is
// one channel and lane g owns the T consecutive steps T g .. T g + T - 1 of each chunk of 16 T steps.
// The states run in a loop.  For each state a lane folds its steps into (P, Q) = (product of A_bar,
// state reached from zero), an inclusive scan over the row's 16 lanes composes the pairs (4 stages of
// row_shr DPP moves), the state carried in from the previous chunk enters, and the lane reruns its
// steps from the state entering them, adding C h to its outputs.
#include <stdint.h>

#include "ssm_device.h"

namespace ssm {
namespace {

// row_shr:K within each 16-lane row; lanes without a source keep `old`
template <int K> __device__ __forceinline__ float shr_keep(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                                 0x110 + K, 0xf, 0xf, false));
}

struct TpParams {
  const bf16_t *u, *delta, *B, *C, *z;
  const float *A, *D, *bias, *init;
  bf16_t* out;
  float* final_state;
  int64_t Bsz, Dm, N, L;
  int nblk;  // channel blocks of 16
};

template <int T>
__global__ __launch_bounds__(256, 3) void tp_scan_kernel(TpParams p) {
  constexpr int CH = 16 * T;   // steps per chunk
  constexpr int TSB = CH + 4;  // B/C tile row (floats)
  constexpr int VPL = T / 8;   // 16-byte pieces per lane and stream
  constexpr int BCC = 2 * 16 * (CH / 8) / 256;  // B/C pieces per thread
  __shared__ __attribute__((aligned(16))) float bct[2 * 16 * TSB];
  __shared__ float Atile[16 * 16];
  __shared__ float carry[16 * 16];  // [channel][state]: the state entering the chunk

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane >> 4, g = lane & 15;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = logical % p.nblk;
  const int64_t b = logical / p.nblk;
  const int64_t L = p.L, N = p.N, Dm = p.Dm;
  const int cl = 4 * w + r;  // channel within the workgroup
  const int64_t d = (int64_t)cb * 16 + cl;
  const bool dval = d < Dm;
  const int64_t dd = dval ? d : Dm - 1;
  const float biasd = p.bias ? p.bias[dd] : 0.0f;
  const float Dd = p.D ? p.D[dd] : 0.0f;
  {
    const int c = tid >> 4, n = tid & 15;
    const int64_t dc = (int64_t)cb * 16 + c < Dm ? (int64_t)cb * 16 + c : Dm - 1;
    Atile[tid] = n < N ? p.A[dc * N + n] * kLog2e : 0.0f;
    carry[tid] = (p.init && n < N) ? p.init[(b * Dm + dc) * N + n] : 0.0f;
  }

  // every read goes through a buffer resource over its whole tensor: pieces past the end read zero
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.B), (short)0, (int)(p.Bsz * N * L * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.C), (short)0, (int)(p.Bsz * N * L * 2), 0x00020000);
  const int stream_bytes = (int)(p.Bsz * Dm * L * 2);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.delta), (short)0, stream_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.u), (short)0, stream_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.z ? p.z : p.u), (short)0, stream_bytes, 0x00020000);
  auto ld16 = [](__amdgpu_buffer_rsrc_t rs, int64_t elem) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(elem * 2), 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  // B/C staging: 2 tensors x 16 state rows x CH / 8 pieces, BCC per thread
  int bsrc_row[BCC], bsrc_col[BCC], bdst[BCC];
  bool bliv[BCC], bisc[BCC];
#pragma unroll
  for (int k = 0; k < BCC; ++k) {
    const int c = tid + 256 * k, row = c / (CH / 8), col = (c % (CH / 8)) * 8, tt = row >> 4, n = row & 15;
    bliv[k] = n < N;
    bisc[k] = tt == 1;
    bsrc_row[k] = n < N ? n : 0;
    bsrc_col[k] = col;
    bdst[k] = row * TSB + col;
  }
  const int64_t srow = (b * Dm + dd) * L;  // this row's channel in the [B, D, L] streams

  uint4 braw[BCC], sd[VPL], su[VPL], sz[VPL];
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int k = 0; k < BCC; ++k) {
      const int64_t e = (b * N + bsrc_row[k]) * L + t0 + bsrc_col[k];
      braw[k] = t0 + bsrc_col[k] < L ? ld16(bisc[k] ? rc : rb, e) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int64_t t = t0 + T * g + 8 * v;
      const bool in = t < L;
      sd[v] = in ? ld16(rd, srow + t) : make_uint4(0u, 0u, 0u, 0u);
      su[v] = in ? ld16(ru, srow + t) : make_uint4(0u, 0u, 0u, 0u);
      sz[v] = in ? ld16(rz, srow + t) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto unpack = [&](const uint4 (&src)[VPL], float (&dst)[T]) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const uint32_t x[4] = {src[v].x, src[v].y, src[v].z, src[v].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        dst[8 * v + 2 * q] = __uint_as_float(x[q] << 16);
        dst[8 * v + 2 * q + 1] = __uint_as_float(x[q] & 0xffff0000u);
      }
    }
  };

  fetch(0);
  for (int64_t t0 = 0; t0 < L; t0 += CH) {
    __syncthreads();  // the previous chunk's tile readers are done
#pragma unroll
    for (int k = 0; k < BCC; ++k) {
      if (!bliv[k]) continue;
      const uint32_t x[4] = {braw[k].x, braw[k].y, braw[k].z, braw[k].w};
      float f[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(x[q] << 16);
        f[2 * q + 1] = __uint_as_float(x[q] & 0xffff0000u);
      }
      *reinterpret_cast<float4*>(bct + bdst[k]) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(bct + bdst[k] + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
    // this lane's steps: dt and dt u once; steps past the end of the sequence are identity steps
    float dt[T], du[T], y[T];
    unpack(sd, dt);
    unpack(su, du);
    uint4 zc[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) zc[v] = sz[v];
    float sdt = 0.0f;
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const bool in = t0 + T * g + j < L;
      y[j] = Dd * du[j];
      const float s = in ? softplus_(dt[j] + biasd) : 0.0f;
      dt[j] = s;
      du[j] = in ? s * du[j] : 0.0f;
      sdt += s;
    }
    if (t0 + CH < L) fetch(t0 + CH);  // the next chunk streams in during the state loop
    __syncthreads();
#pragma unroll 1
    for (int n = 0; n < N; ++n) {
      const float Ap = Atile[cl * 16 + n];
      const float* Bt = bct + n * TSB + T * g;
      const float* Ct = bct + (16 + n) * TSB + T * g;
      float a[T], x[T];
      float Q = 0.0f;  // the state these steps reach from zero
#pragma unroll
      for (int j = 0; j < T; j += 4) {
        const float4 bv = *reinterpret_cast<const float4*>(Bt + j);
        const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a[j + q] = exp2_(dt[j + q] * Ap);
          x[j + q] = du[j + q] * bb[q];
          Q = __builtin_fmaf(a[j + q], Q, x[j + q]);
        }
      }
      float P = exp2_(sdt * Ap);  // the product of these steps' A_bar
      // inclusive scan of the pairs over the row: lane g ends with the composition of lanes 0 .. g
#pragma unroll
      for (int k = 1; k < 16; k <<= 1) {
        float Pp, Qp;
        if (k == 1) { Pp = shr_keep<1>(1.0f, P); Qp = shr_keep<1>(0.0f, Q); }
        else if (k == 2) { Pp = shr_keep<2>(1.0f, P); Qp = shr_keep<2>(0.0f, Q); }
        else if (k == 4) { Pp = shr_keep<4>(1.0f, P); Qp = shr_keep<4>(0.0f, Q); }
        else { Pp = shr_keep<8>(1.0f, P); Qp = shr_keep<8>(0.0f, Q); }
        Q = __builtin_fmaf(P, Qp, Q);
        P = P * Pp;
      }
      const float cin = carry[cl * 16 + n];
      const float hend = __builtin_fmaf(P, cin, Q);  // the state after this lane's steps
      float h = shr_keep<1>(cin, hend);               // the state entering them
      const float cnew = row_bcast<15>(hend);
      if (g == 15) carry[cl * 16 + n] = cnew;  // read by this row only, at the next chunk
#pragma unroll
      for (int j = 0; j < T; j += 4) {
        const float4 cv = *reinterpret_cast<const float4*>(Ct + j);
        const float cc[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h = __builtin_fmaf(a[j + q], h, x[j + q]);
          y[j + q] = __builtin_fmaf(cc[q], h, y[j + q]);
        }
      }
    }
    float zf[T];
    unpack(zc, zf);
    if (dval) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int64_t t = t0 + T * g + 8 * v;
        if (t >= L) continue;
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = 8 * v + 2 * q;
          const float y0 = p.z ? y[j] * silu_(zf[j]) : y[j];
          const float y1 = p.z ? y[j + 1] * silu_(zf[j + 1]) : y[j + 1];
          o[q] = (uint32_t)__builtin_bit_cast(bf16_t, (__bf16)y0) | ((uint32_t)__builtin_bit_cast(bf16_t, (__bf16)y1) << 16);
        }
        *reinterpret_cast<uint4*>(p.out + srow + t) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
  if (p.final_state) {
    __syncthreads();
    const int c = tid >> 4, n = tid & 15;
    const int64_t dc = (int64_t)cb * 16 + c;
    if (dc < Dm && n < N) p.final_state[(b * Dm + dc) * N + n] = carry[tid];
  }
}

}  // namespace
}  // namespace ssm

// Returns 0 on success; 1 for an argument the kernel does not take (a null required pointer, N
// outside 1..16, L not a multiple of 8, a stream tensor of 2^31 bytes or more, an unaligned
// pointer); 2 for a failed launch.  Pointers are device memory: u, delta, z, out [B, D, L] bf16;
// B, C [B, N, L] bf16; A [D, N], D and bias [D], init and final_state [B, D, N] fp32 (D, z, bias,
// init and final_state may be null).
extern "C" int ssm_tp_scan_fwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, const void* u,
                               const void* delta, const float* A, const void* B, const void* C, const float* D,
                               const void* z, const float* bias, const float* init, void* out,
                               float* final_state, hipStream_t stream) {
  if (!u || !delta || !A || !B || !C || !out) return 1;
  if (batch < 1 || dim < 1 || seqlen < 1 || dstate < 1 || dstate > 16 || seqlen % 8 != 0) return 1;
  if (batch * dim * seqlen * 2 >= (int64_t(1) << 31) || batch * dstate * seqlen * 2 >= (int64_t(1) << 31)) return 1;
  const void* ptrs[6] = {u, delta, B, C, z, out};
  for (const void* q : ptrs)
    if (q && (reinterpret_cast<uintptr_t>(q) & 15u)) return 1;
  const int64_t nblk = (dim + 15) / 16;
  if (batch * nblk > (int64_t(1) << 31) - 1) return 1;
  ssm::TpParams p;
  p.u = static_cast<const ssm::bf16_t*>(u);
  p.delta = static_cast<const ssm::bf16_t*>(delta);
  p.B = static_cast<const ssm::bf16_t*>(B);
  p.C = static_cast<const ssm::bf16_t*>(C);
  p.z = static_cast<const ssm::bf16_t*>(z);
  p.A = A; p.D = D; p.bias = bias; p.init = init;
  p.out = static_cast<ssm::bf16_t*>(out);
  p.final_state = final_state;
  p.Bsz = batch; p.Dm = dim; p.N = dstate; p.L = seqlen;
  p.nblk = (int)nblk;
  hipLaunchKernelGGL((ssm::tp_scan_kernel<16>), dim3((unsigned)(batch * nblk)), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
