// conv_kernels.hip -- the step that produces u: causal depthwise conv1d + bias + SiLU.
//
// Operation (ai.xwebgame.com Mamba page, PyTorch block step 2): for each batch
// row b and channel d, a convolution of width K over time that only looks back
// (left padding of K-1 zeros, output cut to the sequence length), a per-channel
// bias, then SiLU:
//   u[b,d,t] = silu(bias[d] + sum_k w[d,k] * x[b,d,t-(K-1)+k])
// where steps before 0 come from a carried state of the K-1 previous inputs
// (oldest first) or are zero.  The decode form applies the same formula to one
// new input and shifts the state by one.
//
// Work layout (HBM-bound: one read of x, one write of u):
//   * vector path (a row is a whole number of 16-byte chunks): a wave streams
//     64*P consecutive chunks, one per lane per pass, with all P loads in
//     flight before any arithmetic.  The K-1 inputs before a chunk are the tail
//     of the left lane's chunk, taken with a cross-lane shuffle (lane 0: lane 63
//     of the previous pass, or memory on the first pass, a cache hit on data
//     another wave loads); a row's first chunk takes them from the state.
//   * element path (other lengths): one lane per output element, the K taps
//     read directly (neighbouring lanes share the lines).
//   * decode: a workgroup stages the state of 1024 channels through LDS so
//     HBM sees contiguous pieces, four channels per lane (one channel per lane
//     when the channel count is not a multiple of 4).
#include "ssm_device.h"

namespace ssm {

namespace {

template <typename IO>
__device__ __forceinline__ float ld(const IO* p, int64_t i) { return to_f32(p[i]); }

// Unpacks one 16-byte chunk into V floats (V = 8 for bf16, 4 for fp32).
__device__ __forceinline__ void unpack(const uint4& q, float (&v)[8]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack(const uint4& q, float (&v)[4]) {
  v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
  v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
}

__device__ __forceinline__ uint4 pack(const float (&v)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i]);
    const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i + 1]);
    w[i] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ uint4 pack(const float (&v)[4]) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3]));
}

template <int K>
__device__ __forceinline__ void load_weights(const float* w, int64_t d, float (&wk)[K]) {
  if constexpr (K == 4) {
    const float4 q = *reinterpret_cast<const float4*>(w + d * 4);  // rows of 16 bytes
    wk[0] = q.x; wk[1] = q.y; wk[2] = q.z; wk[3] = q.w;
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = w[d * K + k];
  }
}

}  // namespace

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Vector path.  A wave owns 64*P consecutive chunks (P passes of 64 lanes); all P loads are
// issued before any arithmetic so each lane keeps P * 16 bytes in flight.  The inputs before
// lane l's chunk are the tail of lane l-1's chunk in the same pass; lane 0 takes lane 63's
// tail from the previous pass, or (first pass) the tail of the chunk before the wave's first,
// loaded with the others (so no wave waits on a second round trip to memory; 25.1 -> 24.0 us
// per call at 8 x 1536 x 2048).
template <typename IO, int K, int P, bool NT = true>
__global__ __launch_bounds__(256) void conv_vec_kernel(ConvParams p) {
  constexpr int V = 16 / (int)sizeof(IO);
  constexpr int H = K - 1;
  constexpr int es = (int)sizeof(IO);
  constexpr int W = (H * es + 3) / 4;  // words holding a chunk's last H values
  const int64_t cpr = p.L / V;         // chunks per row
  const int64_t total = p.Bsz * p.Dm * cpr;
  const int lane = threadIdx.x & 63;
  const int64_t wbase = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 * P);
  const IO* x = static_cast<const IO*>(p.x);
  IO* u = static_cast<IO*>(p.u);

  // every load is issued before any arithmetic: the P chunks, lane 0's previous chunk (its tail
  // is the halo of the wave's first chunk) and, at row starts, the carried state
  u32x4 q[P];
  int64_t rows[P], cs[P];
  float sv[P][H > 0 ? H : 1];
  const IO* st = static_cast<const IO*>(p.state_in);
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int64_t gid = wbase + 64 * j + lane;
    const bool valid = gid < total;
    q[j] = u32x4{0u, 0u, 0u, 0u};
    if (valid) {
      const u32x4* src = reinterpret_cast<const u32x4*>(x + gid * V);
      q[j] = NT ? __builtin_nontemporal_load(src) : *src;
    }
    int64_t row, c;
    if (total <= 0xffffffffll) {  // uniform: 32-bit division when the chunk count allows
      const uint32_t g32 = (uint32_t)(valid ? gid : 0), c32 = (uint32_t)cpr;
      row = g32 / c32;
      c = g32 - (uint32_t)row * c32;
    } else {
      row = valid ? gid / cpr : 0;
      c = valid ? gid - row * cpr : 0;
    }
    rows[j] = row;
    cs[j] = c;
#pragma unroll
    for (int k = 0; k < (H > 0 ? H : 1); ++k) sv[j][k] = 0.0f;
    if constexpr (H > 0) {
      if (valid && c == 0 && st) {
#pragma unroll
        for (int k = 0; k < H; ++k) sv[j][k] = ld(st, row * H + k);
      }
    }
  }
  u32x4 qp = u32x4{0u, 0u, 0u, 0u};
  if constexpr (H > 0) {
    if (lane == 0 && wbase > 0 && wbase < total) qp = *reinterpret_cast<const u32x4*>(x + (wbase - 1) * V);
  }

#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int64_t gid = wbase + 64 * j + lane;
    const bool valid = gid < total;
    const int64_t row = rows[j], c = cs[j];
    float xs[V];
    unpack(uint4{q[j].x, q[j].y, q[j].z, q[j].w}, xs);

    float hal[H > 0 ? H : 1];
    if constexpr (H > 0) {
      const uint32_t words[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
      uint32_t tw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 4 - W; i < 4; ++i) {
        tw[i] = (uint32_t)__shfl_up((int)words[i], 1, 64);
        if (j > 0) {
          const uint32_t pw[4] = {q[j - 1].x, q[j - 1].y, q[j - 1].z, q[j - 1].w};
          const uint32_t last = (uint32_t)__builtin_amdgcn_readlane((int)pw[i], 63);
          if (lane == 0) tw[i] = last;
        } else {
          const uint32_t pq[4] = {qp.x, qp.y, qp.z, qp.w};
          if (lane == 0) tw[i] = pq[i];
        }
      }
      float prev[V];
      unpack(uint4{tw[0], tw[1], tw[2], tw[3]}, prev);
#pragma unroll
      for (int k = 0; k < H; ++k) hal[k] = c == 0 ? sv[j][k] : prev[V - H + k];
    }
    if (!valid) continue;

    const int64_t d = row % p.Dm;
    float wk[K];
    load_weights<K>(p.w, d, wk);
    const float b0 = p.bias ? p.bias[d] : 0.0f;
    float us[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float v = b0;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int i = e + k - H;  // index into the chunk; negative reaches into the halo
        v = __builtin_fmaf(wk[k], i >= 0 ? xs[i] : hal[H + i], v);
      }
      us[e] = silu_(v);
    }
    const uint4 o = pack(us);
    u32x4* dst = reinterpret_cast<u32x4*>(u + gid * V);
    if (NT) __builtin_nontemporal_store(u32x4{o.x, o.y, o.z, o.w}, dst);
    else *dst = u32x4{o.x, o.y, o.z, o.w};

    if constexpr (H > 0) {
      if (p.state_out && c == cpr - 1) {  // V >= H: the state is the tail of this chunk
        IO* so = static_cast<IO*>(p.state_out) + row * H;
#pragma unroll
        for (int k = 0; k < H; ++k) store_io(so + k, xs[V - H + k]);
      }
    }
  }
}

template <typename IO, int K>
__global__ __launch_bounds__(256) void conv_elem_kernel(ConvParams p) {
  constexpr int H = K - 1;
  const int64_t total = p.Bsz * p.Dm * p.L;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int64_t row = gid / p.L, t = gid - row * p.L, d = row % p.Dm;
  const IO* xr = static_cast<const IO*>(p.x) + row * p.L;
  const IO* st = static_cast<const IO*>(p.state_in);
  float wk[K];
  load_weights<K>(p.w, d, wk);
  float v = p.bias ? p.bias[d] : 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t s = t - H + k;  // input step; negative reaches into the state
    float xv = 0.0f;
    if (s >= 0) xv = ld(xr, s);
    else if (st) xv = ld(st, row * H + (H + s));
    v = __builtin_fmaf(wk[k], xv, v);
  }
  store_io(static_cast<IO*>(p.u) + gid, silu_(v));
  if (H > 0 && p.state_out && t == p.L - 1) {
    // last H inputs of (state, x): x's tail, reaching into the old state when L < H
    IO* so = static_cast<IO*>(p.state_out) + row * H;
    for (int j = 0; j < H; ++j) {
      const int64_t s = p.L - H + j;
      float xv = 0.0f;
      if (s >= 0) xv = ld(xr, s);
      else if (st) xv = ld(st, row * H + (H + s));
      store_io(so + j, xv);
    }
  }
}

// Decode step, one channel per lane (any channel count).
template <typename IO, int K>
__global__ __launch_bounds__(256) void conv_update_kernel(ConvParams p) {
  constexpr int H = K - 1;
  const int64_t rows = p.Bsz * p.Dm;
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int64_t d = row % p.Dm;
  IO* st = static_cast<IO*>(p.state_out) + row * H;  // read and written in place
  float hv[H > 0 ? H : 1];
#pragma unroll
  for (int j = 0; j < H; ++j) hv[j] = to_f32(st[j]);
  const float xv = ld(static_cast<const IO*>(p.x), row);
  float wk[K];
  load_weights<K>(p.w, d, wk);
  float v = p.bias ? p.bias[d] : 0.0f;
#pragma unroll
  for (int k = 0; k < H; ++k) v = __builtin_fmaf(wk[k], hv[k], v);
  v = __builtin_fmaf(wk[H], xv, v);
  store_io(static_cast<IO*>(p.u) + row, silu_(v));
#pragma unroll
  for (int j = 0; j + 1 < H; ++j) store_io(st + j, hv[j + 1]);
  if constexpr (H > 0) store_io(st + H - 1, xv);
}

// Decode step when the channel count is a multiple of 4: a workgroup owns 1024 consecutive
// channels, 4 per lane.  Their state rows form one contiguous block of 1024*(K-1) elements,
// moved between HBM and LDS with contiguous 8-byte (bf16) or 16-byte (fp32) pieces, so every
// global access is fully coalesced; each lane then reads and rewrites its 4 rows in LDS.
// x, u, the 4 bias values and the 4 weight rows of a lane are contiguous vectors.
template <typename IO, int K>
__global__ __launch_bounds__(256) void conv_update4_kernel(ConvParams p) {
  constexpr int H = K - 1;
  constexpr int es = (int)sizeof(IO);
  constexpr int PB = es == 2 ? 8 : 16;  // bytes per global piece
  constexpr int WPL = H * es;           // LDS words of state per lane (4 rows)
  __shared__ uint32_t sm[H > 0 ? 256 * WPL : 1];
  const int64_t rows = p.Bsz * p.Dm;
  const int64_t rb = (int64_t)blockIdx.x * 1024;
  const int64_t left = rows - rb;
  const int nrows = left < 1024 ? (int)left : 1024;  // a multiple of 4
  char* gst = reinterpret_cast<char*>(static_cast<IO*>(p.state_out) + rb * H);
  const int npieces = nrows * H * es / PB;
  if constexpr (H > 0) {
    for (int i = threadIdx.x; i < npieces; i += 256) {
      if constexpr (PB == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(gst + 8 * i);
        sm[2 * i] = v.x; sm[2 * i + 1] = v.y;
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(gst + 16 * i);
        sm[4 * i] = v.x; sm[4 * i + 1] = v.y; sm[4 * i + 2] = v.z; sm[4 * i + 3] = v.w;
      }
    }
    __syncthreads();
  }
  const int64_t r0 = rb + 4 * (int64_t)threadIdx.x;
  if (r0 < rows) {
    float xv[4];
    if constexpr (es == 2) {
      const uint2 t = *reinterpret_cast<const uint2*>(static_cast<const IO*>(p.x) + r0);
      xv[0] = __uint_as_float(t.x << 16); xv[1] = __uint_as_float(t.x & 0xffff0000u);
      xv[2] = __uint_as_float(t.y << 16); xv[3] = __uint_as_float(t.y & 0xffff0000u);
    } else {
      const float4 t = *reinterpret_cast<const float4*>(static_cast<const IO*>(p.x) + r0);
      xv[0] = t.x; xv[1] = t.y; xv[2] = t.z; xv[3] = t.w;
    }
    uint32_t* my = sm + threadIdx.x * WPL;
    float hv[4][H > 0 ? H : 1];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int k = 0; k < H; ++k) {
        const int e = r * H + k;  // element of the lane's 4 rows
        if constexpr (es == 2)
          hv[r][k] = __uint_as_float((e & 1) ? (my[e >> 1] & 0xffff0000u) : (my[e >> 1] << 16));
        else
          hv[r][k] = __uint_as_float(my[e]);
      }
    const int64_t d0 = r0 % p.Dm;  // a multiple of 4: the lane's channels are d0 .. d0+3
    float bb[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (p.bias) {
      const float4 t = *reinterpret_cast<const float4*>(p.bias + d0);
      bb[0] = t.x; bb[1] = t.y; bb[2] = t.z; bb[3] = t.w;
    }
    float uv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float wk[K];
      load_weights<K>(p.w, d0 + r, wk);
      float v = bb[r];
#pragma unroll
      for (int k = 0; k < H; ++k) v = __builtin_fmaf(wk[k], hv[r][k], v);
      v = __builtin_fmaf(wk[H], xv[r], v);
      uv[r] = silu_(v);
    }
    if constexpr (es == 2) {
      uint2 t;
      t.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)uv[0]) |
            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)uv[1]) << 16);
      t.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)uv[2]) |
            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)uv[3]) << 16);
      *reinterpret_cast<uint2*>(static_cast<IO*>(p.u) + r0) = t;
    } else {
      *reinterpret_cast<float4*>(static_cast<IO*>(p.u) + r0) = make_float4(uv[0], uv[1], uv[2], uv[3]);
    }
    if constexpr (H > 0) {
      // each row drops its oldest input and appends x; the values are widened io elements,
      // so their bits move unchanged
      uint32_t nw[WPL];
#pragma unroll
      for (int i = 0; i < WPL; ++i) nw[i] = 0u;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int k = 0; k < H; ++k) {
          const float nv = (k + 1 < H) ? hv[r][k + 1] : xv[r];
          const int e = r * H + k;
          if constexpr (es == 2) nw[e >> 1] |= (e & 1) ? (__float_as_uint(nv) & 0xffff0000u)
                                                       : (__float_as_uint(nv) >> 16);
          else nw[e] = __float_as_uint(nv);
        }
#pragma unroll
      for (int i = 0; i < WPL; ++i) my[i] = nw[i];
    }
  }
  if constexpr (H > 0) {
    __syncthreads();
    for (int i = threadIdx.x; i < npieces; i += 256) {
      if constexpr (PB == 8)
        *reinterpret_cast<uint2*>(gst + 8 * i) = make_uint2(sm[2 * i], sm[2 * i + 1]);
      else
        *reinterpret_cast<uint4*>(gst + 16 * i) = make_uint4(sm[4 * i], sm[4 * i + 1], sm[4 * i + 2], sm[4 * i + 3]);
    }
  }
}

namespace {

template <typename IO, int K>
hipError_t launch_conv_k(const ConvParams& p, int mode, hipStream_t s) {
  const int64_t rows = p.Bsz * p.Dm;
  if (mode == 2) {
    if (p.Dm % 4 == 0) {
      hipLaunchKernelGGL((conv_update4_kernel<IO, K>), dim3((unsigned)((rows + 1023) / 1024)), dim3(256), 0, s, p);
    } else {
      hipLaunchKernelGGL((conv_update_kernel<IO, K>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, p);
    }
  } else if (mode == 1) {
    constexpr int V = 16 / (int)sizeof(IO);
    constexpr int P = 2;  // chunks per lane (measured best of 1, 2, 4, 8 on gfx950)
    const int64_t chunks = rows * (p.L / V);
    const int64_t per_block = 256 * P;
    hipLaunchKernelGGL((conv_vec_kernel<IO, K, P>), dim3((unsigned)((chunks + per_block - 1) / per_block)),
                       dim3(256), 0, s, p);
  } else {
    const int64_t elems = rows * p.L;
    hipLaunchKernelGGL((conv_elem_kernel<IO, K>), dim3((unsigned)((elems + 255) / 256)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_conv_io(const ConvParams& p, int mode, hipStream_t s) {
  switch (p.K) {
    case 1: return launch_conv_k<IO, 1>(p, mode, s);
    case 2: return launch_conv_k<IO, 2>(p, mode, s);
    case 3: return launch_conv_k<IO, 3>(p, mode, s);
    default: return launch_conv_k<IO, 4>(p, mode, s);
  }
}

}  // namespace

hipError_t launch_conv(const ConvParams& p, bool bf16, int mode, hipStream_t s) {
  return bf16 ? launch_conv_io<bf16_t>(p, mode, s) : launch_conv_io<float>(p, mode, s);
}

}  // namespace ssm
