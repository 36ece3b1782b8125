// ssm_launch.h -- internal interface between the C ABI (ssm_abi.cpp) and the
// gfx950 kernels (ssm_kernels.hip).  Not installed; not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

struct ScanParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  const float* init;     // [B,D,N] state before the first step, or null (zero)
  float* carries;        // [S,B,D,N] state entering each segment (split runs), or null
  void* out;
  float* final_state;
  float* ckpt;           // [B,nb,D,N] state entering each 64-step block (checkpoint pass), or null
  float* seg_state;      // [S-1,B,D,N] end state of each segment scanned from zero (the library
                         // places it at carries + B*D*N; the carry pass overwrites it in place)
  float* seg_dsum;       // [S-1,B,D] sum of the step sizes of each segment
  int64_t Bsz, Dm, N, L;
  int64_t seg_len;       // steps per segment, a multiple of 64
  int S;                 // number of segments (1: no split)
  int nblk;              // channel blocks of 16 = ceil(Dm / 16)
  int vec;               // rows of whole 16-byte pieces, shorter than 2^24 elements (the scan's whole-piece staging)
  int reverse;           // scan from the last step to the first
  int zoh;               // zero-order-hold B_bar
};

struct StepParams {
  float* state;
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  void* out;
  int64_t Bsz, Dm, N;
  int vec;  // N % 4 == 0: state rows read and written as float4
  int zoh;
};

struct BwdParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  const void* dout;       // [B,D,L] gradient of out
  const float* dfinal;    // [B,D,N] gradient of final_state, or null
  const float* ckpt;      // [B,nb,D,N] state entering each 64-step block
  void* du;               // [B,D,L]
  void* ddelta;           // [B,D,L]
  void* dz;               // [B,D,L], written when z is given
  float* dh0;             // [B,D,N] gradient of the initial state, or null
  float* part_bc;         // [2,nblk,B,N,L] dB and dC summed over each workgroup's 16 channels
  float* part_a;          // [S,B,D,N] dA summed over a segment's steps, per batch row
  float* part_d;          // [2,S,B,D] dD and dbias summed over a segment's steps, per batch row
  const float* adj_in;    // [S,B,D,N] adjoint entering each segment from the right (split runs), or null
  float* adj_q;           // [S,B,D,N] adjoint summary of each segment s >= 1 (split runs)
  float* adj_dsum;        // [S,B,D] sum of the step sizes of each segment s >= 1 (split runs)
  int64_t Bsz, Dm, N, L;
  int64_t seg_len;        // steps per segment, a multiple of 256 when S > 1
  int S;                  // number of segments (1: no split)
  int nblk;               // channel blocks of 16
  int vec;                // rows allow 16-byte vector loads
  int reverse;
  int zoh;                // zero-order-hold B_bar
};

struct ConvParams {
  const void* x;          // [B,D,L] (decode: [B,D])
  const float* w;         // [D,K]
  const float* bias;      // [D] or null
  const void* state_in;   // [B,D,K-1] inputs before x, or null (zeros)
  void* u;                // [B,D,L] (decode: [B,D])
  void* state_out;        // [B,D,K-1] or null; decode: the state, read and written
  int64_t Bsz, Dm, L;
  int K;                  // width, 1..4
};

hipError_t launch_scan(const ScanParams& p, bool bf16, int mode, hipStream_t s);
// the split's summary (mode 1) and output (mode 0) passes with channels on lanes: bf16 streams,
// the default discretisation, N <= 16, L a multiple of 8 and below 2^24 (workgroups of 64
// channels, ceil(Dm / 64) per batch row and segment)
hipError_t launch_scan_cl(const ScanParams& p, int mode, hipStream_t s);
// mode 0: per-element prefill, 1: 16-byte-chunk prefill (L a multiple of the chunk), 2: decode step
hipError_t launch_conv(const ConvParams& p, bool bf16, int mode, hipStream_t s);
hipError_t launch_carry(const ScanParams& p, hipStream_t s);
// checkpoint pass (the scan kernel's mode 2), backward pass, and the fixed-order partial sums
hipError_t launch_ckpt(const ScanParams& p, bool bf16, hipStream_t s);
hipError_t launch_bwd(const BwdParams& p, bool bf16, hipStream_t s);
// the zero-order-hold variants of the two (p.zoh set), compiled separately
hipError_t launch_ckpt_zoh(const ScanParams& p, bool bf16, hipStream_t s);
hipError_t launch_bwd_zoh(const BwdParams& p, bool bf16, hipStream_t s);
// sequence split of the backward: the adjoint summary of segments 1..S-1 (adj_q, adj_dsum), then
// the adjoint entering each segment (adj_in), composed from the right
hipError_t launch_adj_summary(const BwdParams& p, bool bf16, hipStream_t s);
hipError_t launch_adj_carry(const BwdParams& p, float* adj_in, hipStream_t s);
// out[i] = sum_k part[k * stride + i] for i < n, k < count (k ascending)
hipError_t launch_reduce(float* out, const float* part, int64_t count, int64_t stride, int64_t n, hipStream_t s);
hipError_t launch_step(const StepParams& p, bool bf16, hipStream_t s);

// Size of the static per-device scratch array behind ssm_scan_fwd_noalloc, and its device address
// on the device `stream` belongs to (the current device for the null stream), looked up once per
// device.
constexpr size_t kScratchBytes = size_t(34) << 20;  // holds the split of 1 x 1024 x 16 x 2^20 (bf16)
hipError_t scratch_buffer(hipStream_t stream, void** ptr);

}  // namespace ssm
