// ssm_abi.cpp -- the C entry points declared in include/ssm_scan.h.
//
// Every argument is validated on the host before anything is enqueued; no HIP
// runtime call is made for an invalid call, so the checks can be exercised on
// a machine without a GPU.  The library allocates no memory; its only state is the
// per-device address of the static scratch array of ssm_scan_fwd_noalloc.
#include <stdint.h>
#include <string.h>

#include "../../include/ssm_scan.h"
#include "ssm_launch.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 40;
constexpr int64_t kMaxElems = int64_t(1) << 61;
constexpr int kTargetBlocks = 1024;    // output-pass workgroups of 4 waves: 4 per CU on 256 CUs
constexpr int64_t kMinSegment = 1024;  // shortest segment worth a summary pass
// A split aims at eight rounds of workgroups: shorter segments balance the passes' workgroups over
// the CUs.  With channels on lanes at most 512 segments (the carry pass is sequential over them)
// unless one round needs more.
constexpr int kRounds = 8;
constexpr int64_t kMaxSegmentsCl = 512;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, int64_t elems, int64_t esize) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + static_cast<uintptr_t>(elems * esize)};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a <= 0 || b <= 0) return false;
  if (a > kMaxElems / b) return false;
  *out = a * b;
  return true;
}

struct Plan {
  int64_t S = 1, seg_len = 0, nblk = 0;
  bool cl = false;  // the split runs with channels on lanes (scan_cl.hip)
  size_t ws_dsum = 0, ws_carry = 0, total = 0;
};

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Shape-only choice of the sequence split, so results never depend on the device.
bool make_plan(const ssm_shape* s, Plan* pl) {
  if (!s) return false;
  if (s->batch < 1 || s->dim < 1 || s->seqlen < 1 || s->dstate < 1 || s->dstate > 64) return false;
  if (s->batch > kMaxDim || s->dim > kMaxDim || s->seqlen > kMaxDim) return false;
  int64_t bd, bdl, bdn;
  if (!mul_ok(s->batch, s->dim, &bd) || !mul_ok(bd, s->seqlen, &bdl) || !mul_ok(bd, s->dstate, &bdn))
    return false;
  int64_t bnl;
  if (!mul_ok(s->batch * s->dstate, s->seqlen, &bnl)) return false;
  pl->nblk = (s->dim + 15) / 16;  // 16 channels (4 waves) per workgroup
  const int64_t base = s->batch * pl->nblk;
  if (base > (int64_t(1) << 30)) return false;
  const int64_t L = s->seqlen;
  pl->S = 1;
  pl->seg_len = ((L + 63) / 64) * 64;
  if (base < kTargetBlocks / 2 && L >= 2 * kMinSegment) {
    // bf16 streams, the default discretisation, up to 16 states and rows of whole 16-byte chunks:
    // the split's passes keep channels on lanes, 64 channels per workgroup, and the segments
    // supply the parallelism (when whole 64-channel groups pad D by at most a fifth)
    const int64_t pad = (s->dim + 63) / 64 * 64 - s->dim;
    pl->cl = s->io_dtype == SSM_BF16 && !(s->flags & SSM_FLAG_ZOH) && s->dstate <= 16 && L % 8 == 0 &&
             L < (int64_t(1) << 24) && 5 * pad <= s->dim;
    const int64_t units = pl->cl ? s->batch * ((s->dim + 63) / 64) : base;  // workgroups per segment
    const int64_t one = (kTargetBlocks + units - 1) / units;                   // segments for one round
    int64_t want = (kRounds * kTargetBlocks + units - 1) / units;
    if (pl->cl && want > kMaxSegmentsCl) want = kMaxSegmentsCl > one ? kMaxSegmentsCl : one;
    int64_t seg = (L + want - 1) / want;
    seg = ((seg + 63) / 64) * 64;
    if (seg < kMinSegment) seg = kMinSegment;
    const int64_t S = (L + seg - 1) / seg;
    if (S > 1) {
      pl->S = S;
      pl->seg_len = seg;
    } else {
      pl->cl = false;
    }
  }
  if (base * pl->S > (int64_t(1) << 31) - 1) return false;
  if (pl->S > 1) {
    // carries [S,B,D,N] (the summary pass writes segment s's end state into slot s + 1, and the
    // carry pass turns it in place into the state entering segment s + 1), then the step-size sums
    pl->ws_carry = round256(sizeof(float) * (size_t)pl->S * (size_t)bdn);
    pl->ws_dsum = round256(sizeof(float) * (size_t)(pl->S - 1) * (size_t)bd);
    pl->total = pl->ws_carry + pl->ws_dsum;
  }
  return true;
}

ssm_status launch_status(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH; }

struct BwdPlan {
  int64_t nblk = 0, nbk = 0, S = 1, seg_len = 0;
  size_t ckpt = 0, bc = 0, a = 0, d = 0;
  size_t seg_dsum = 0, carries = 0, adj_q = 0, adj_dsum = 0, adj_in = 0, total = 0;
};

constexpr int kBwdTargetBlocks = 768;  // 3 backward workgroups per CU on 256 CUs

// Shape-only, like the forward's plan.  Few channels and a long sequence: split the sequence
// into segments (whole 256-step chunks, >= 1024 steps) so that about kRounds x kBwdTargetBlocks
// workgroups run (eight rounds); each segment's checkpoints start from a carried state (summary
// pass + carry) and its adjoint from a carried adjoint (adjoint summary + carry).
bool make_bwd_plan(const ssm_shape* s, BwdPlan* pl, bool saved = false) {
  Plan fp;
  if (!make_plan(s, &fp)) return false;  // same size limits as the forward
  const int64_t Bsz = s->batch, Dm = s->dim, N = s->dstate, L = s->seqlen;
  pl->nblk = (Dm + 15) / 16;
  pl->nbk = (L + 63) / 64;
  const int64_t base = Bsz * pl->nblk;
  pl->S = 1;
  pl->seg_len = ((L + 255) / 256) * 256;
  if (base < kBwdTargetBlocks / 2 && L >= 2 * kMinSegment) {
    const int64_t want = (kRounds * kBwdTargetBlocks + base - 1) / base;
    int64_t seg = (L + want - 1) / want;
    seg = ((seg + 255) / 256) * 256;
    if (seg < kMinSegment) seg = kMinSegment;
    const int64_t S = (L + seg - 1) / seg;
    if (S > 1) {
      pl->S = S;
      pl->seg_len = seg;
    }
  }
  if (base * pl->S > (int64_t(1) << 31) - 1) return false;
  const int64_t BD = Bsz * Dm, BDN = BD * N;
  int64_t x;
  if (!mul_ok(BDN, pl->nbk, &x)) return false;
  pl->ckpt = saved ? 0 : round256(sizeof(float) * (size_t)x);  // saved: the forward wrote them
  if (!mul_ok(2 * pl->nblk * Bsz * N, L, &x)) return false;
  pl->bc = round256(sizeof(float) * (size_t)x);
  if (!mul_ok(BDN, pl->S, &x)) return false;
  pl->a = round256(sizeof(float) * (size_t)x);
  pl->d = round256(sizeof(float) * (size_t)(2 * pl->S * BD));
  if (pl->S > 1) {
    if (!saved) {  // the checkpoints' own split: carries (segment end states in place), step-size sums
      pl->seg_dsum = round256(sizeof(float) * (size_t)((pl->S - 1) * BD));
      pl->carries = round256(sizeof(float) * (size_t)(pl->S * BDN));
    }
    pl->adj_q = round256(sizeof(float) * (size_t)(pl->S * BDN));
    pl->adj_dsum = round256(sizeof(float) * (size_t)(pl->S * BD));
    pl->adj_in = pl->adj_q;
  }
  pl->total = pl->ckpt + pl->bc + pl->a + pl->d + pl->seg_dsum + pl->carries + pl->adj_q +
              pl->adj_dsum + pl->adj_in;
  return true;
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_str(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_SHAPE:
      return "a size is out of range (batch, dim, seqlen >= 1; dstate in [1, 64]; conv width in [1, 4])";
    case SSM_ERR_DTYPE: return "io_dtype must be SSM_F32 or SSM_BF16";
    case SSM_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
    case SSM_ERR_UNSUPPORTED: return "unknown flag bits";
    case SSM_ERR_WORKSPACE: return "workspace smaller than ssm_scan_workspace_size()";
    case SSM_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case SSM_ERR_OVERLAP: return "an output buffer overlaps an input buffer";
    case SSM_ERR_TOO_LARGE: return "the call needs more scratch memory than ssm_scan_fwd_noalloc holds (34 MiB)";
    default: return "unknown status";
  }
}

size_t ssm_scan_workspace_size(const ssm_shape* shape) {
  Plan pl;
  if (!make_plan(shape, &pl)) return 0;
  return pl.total;
}

}  // extern "C"

namespace {

// ssm_scan_fwd, and with ckpt set ssm_scan_fwd_save (the state entering every 64-step block
// is also written, [B, ceil(L/64), D, N] fp32).
ssm_status scan_fwd_impl(const ssm_shape* shape, const void* u, const void* delta, const float* A,
                         const void* B, const void* C, const float* D, const void* z,
                         const float* delta_bias, const float* initial_state, void* out,
                         float* final_state, float* ckpt, void* workspace, size_t workspace_bytes,
                         struct ihipStream_t* stream, bool use_scratch = false) {
  if (!shape) return SSM_ERR_NULL;
  if (shape->io_dtype != SSM_F32 && shape->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (shape->flags & ~(SSM_FLAG_ZOH | SSM_FLAG_REVERSE)) return SSM_ERR_UNSUPPORTED;
  Plan pl;
  if (!make_plan(shape, &pl)) return SSM_ERR_SHAPE;
  if (!u || !delta || !A || !B || !C || !out) return SSM_ERR_NULL;
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, initial_state, out, final_state, ckpt, workspace};
  for (const void* q : ptrs)
    if (misaligned(q)) return SSM_ERR_ALIGN;

  const int64_t Bsz = shape->batch, Dm = shape->dim, N = shape->dstate, L = shape->seqlen;
  const int64_t es = shape->io_dtype == SSM_BF16 ? 2 : 4;
  const Range rc_ = span(ckpt, ckpt ? Bsz * Dm * N * ((L + 63) / 64) : 0, 4);
  const Range ins[] = {span(u, Bsz * Dm * L, es), span(delta, Bsz * Dm * L, es), span(A, Dm * N, 4),
                       span(B, Bsz * N * L, es), span(C, Bsz * N * L, es), span(D, D ? Dm : 0, 4),
                       span(z, z ? Bsz * Dm * L : 0, es), span(delta_bias, delta_bias ? Dm : 0, 4),
                       span(initial_state, initial_state ? Bsz * Dm * N : 0, 4)};
  const Range ro = span(out, Bsz * Dm * L, es);
  const Range rf = span(final_state, final_state ? Bsz * Dm * N : 0, 4);
  for (size_t i = 0; i < sizeof(ins) / sizeof(ins[0]); ++i) {
    if (overlaps(ro, ins[i])) return SSM_ERR_OVERLAP;
    // final_state may be the very buffer initial_state points to (in-place continuation)
    const bool same_state = (i == 8) && final_state && (const void*)final_state == (const void*)initial_state;
    if (!same_state && overlaps(rf, ins[i])) return SSM_ERR_OVERLAP;
  }
  if (overlaps(ro, rf)) return SSM_ERR_OVERLAP;
  for (const Range& r : ins)
    if (overlaps(rc_, r)) return SSM_ERR_OVERLAP;
  if (overlaps(rc_, ro) || overlaps(rc_, rf)) return SSM_ERR_OVERLAP;

  // use_scratch: the split runs in the library's static per-device array (ssm_scan_fwd_noalloc)
  const bool split = pl.S > 1 && (workspace != nullptr || use_scratch);
  if (use_scratch && pl.total > ssm::kScratchBytes) return SSM_ERR_TOO_LARGE;
  if (!use_scratch && pl.S > 1 && workspace != nullptr && workspace_bytes < pl.total) return SSM_ERR_WORKSPACE;
  if (!use_scratch && pl.S > 1 && workspace == nullptr && workspace_bytes != 0) return SSM_ERR_NULL;
  if (split && !use_scratch) {
    const Range rw = span(workspace, (int64_t)pl.total, 1);
    for (const Range& r : ins)
      if (overlaps(rw, r)) return SSM_ERR_OVERLAP;
    if (overlaps(rw, ro) || overlaps(rw, rf) || overlaps(rw, rc_)) return SSM_ERR_OVERLAP;
  }

  ssm::ScanParams p;
  memset(&p, 0, sizeof(p));
  p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.bias = delta_bias;
  p.init = initial_state; p.out = out; p.final_state = final_state; p.ckpt = ckpt;
  p.Bsz = Bsz; p.Dm = Dm; p.N = N; p.L = L;
  p.nblk = (int)pl.nblk;
  // 16-byte chunks stay inside each row; the whole-chunk staging's buffer resources span 8 rows of L
  // elements, so longer rows take the element path
  p.vec = (L % (16 / es)) == 0 && L >= 8 && L < (int64_t(1) << 24) ? 1 : 0;
  p.reverse = (shape->flags & SSM_FLAG_REVERSE) ? 1 : 0;
  p.zoh = (shape->flags & SSM_FLAG_ZOH) ? 1 : 0;
  const bool bf16 = shape->io_dtype == SSM_BF16;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  if (!split) {
    p.S = 1;
    p.seg_len = ((L + 63) / 64) * 64;
    return launch_status(ssm::launch_scan(p, bf16, 0, st));
  }
  if (use_scratch) {  // every argument has been checked; now the device address of the array
    if (ssm::scratch_buffer(st, &workspace) != hipSuccess) return SSM_ERR_LAUNCH;
  }
  char* ws = static_cast<char*>(workspace);
  p.S = (int)pl.S;
  p.seg_len = pl.seg_len;
  float* carries = reinterpret_cast<float*>(ws);
  p.seg_state = carries + Bsz * Dm * N;  // slots 1 .. S-1 of the carries, overwritten in place
  p.seg_dsum = reinterpret_cast<float*>(ws + pl.ws_carry);
  // channels on lanes unless block checkpoints are wanted (the lanes-over-states kernels write them)
  const bool cl = pl.cl && ckpt == nullptr;
  ssm_status rc = launch_status(cl ? ssm::launch_scan_cl(p, 1, st) : ssm::launch_scan(p, bf16, 1, st));
  if (rc != SSM_OK) return rc;
  p.carries = carries;
  rc = launch_status(ssm::launch_carry(p, st));
  if (rc != SSM_OK) return rc;
  return launch_status(cl ? ssm::launch_scan_cl(p, 0, st) : ssm::launch_scan(p, bf16, 0, st));
}

}  // namespace

extern "C" {

ssm_status ssm_scan_fwd(const ssm_shape* shape, const void* u, const void* delta, const float* A,
                        const void* B, const void* C, const float* D, const void* z,
                        const float* delta_bias, const float* initial_state, void* out,
                        float* final_state, void* workspace, size_t workspace_bytes,
                        struct ihipStream_t* stream) {
  return scan_fwd_impl(shape, u, delta, A, B, C, D, z, delta_bias, initial_state, out, final_state, nullptr,
                       workspace, workspace_bytes, stream);
}

ssm_status ssm_scan_fwd_save(const ssm_shape* shape, const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D, const void* z,
                             const float* delta_bias, const float* initial_state, void* out,
                             float* final_state, float* checkpoints, void* workspace,
                             size_t workspace_bytes, struct ihipStream_t* stream) {
  if (!checkpoints) return SSM_ERR_NULL;
  return scan_fwd_impl(shape, u, delta, A, B, C, D, z, delta_bias, initial_state, out, final_state, checkpoints,
                       workspace, workspace_bytes, stream);
}

ssm_status ssm_scan_fwd_noalloc(const ssm_shape* shape, const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D, const void* z,
                                const float* delta_bias, const float* initial_state, void* out,
                                float* final_state, struct ihipStream_t* stream) {
  return scan_fwd_impl(shape, u, delta, A, B, C, D, z, delta_bias, initial_state, out, final_state, nullptr,
                       nullptr, 0, stream, true);
}

ssm_status ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, int32_t io_dtype, uint32_t flags,
                            float* state, const void* u, const void* delta, const float* A, const void* B,
                            const void* C, const float* D, const void* z, const float* delta_bias, void* out,
                            struct ihipStream_t* stream) {
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (flags & ~SSM_FLAG_ZOH) return SSM_ERR_UNSUPPORTED;
  if (batch < 1 || dim < 1 || dstate < 1 || dstate > 64 || batch > kMaxDim || dim > kMaxDim)
    return SSM_ERR_SHAPE;
  int64_t bd, bdn;
  if (!mul_ok(batch, dim, &bd) || !mul_ok(bd, dstate, &bdn)) return SSM_ERR_SHAPE;
  if (bd * 16 > (int64_t(1) << 31) * 256 - 1) return SSM_ERR_SHAPE;
  if (!state || !u || !delta || !A || !B || !C || !out) return SSM_ERR_NULL;
  const void* ptrs[] = {state, u, delta, A, B, C, D, z, delta_bias, out};
  for (const void* q : ptrs)
    if (misaligned(q)) return SSM_ERR_ALIGN;
  const int64_t es = io_dtype == SSM_BF16 ? 2 : 4;
  const Range ins[] = {span(u, bd, es), span(delta, bd, es), span(A, dim * dstate, 4),
                       span(B, batch * dstate, es), span(C, batch * dstate, es), span(D, D ? dim : 0, 4),
                       span(z, z ? bd : 0, es), span(delta_bias, delta_bias ? dim : 0, 4)};
  const Range ro = span(out, bd, es), rs = span(state, bdn, 4);
  for (const Range& r : ins)
    if (overlaps(ro, r) || overlaps(rs, r)) return SSM_ERR_OVERLAP;
  if (overlaps(ro, rs)) return SSM_ERR_OVERLAP;

  ssm::StepParams p;
  memset(&p, 0, sizeof(p));
  p.state = state; p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z;
  p.bias = delta_bias; p.out = out;
  p.Bsz = batch; p.Dm = dim; p.N = dstate;
  p.vec = (dstate % 4) == 0 ? 1 : 0;
  p.zoh = (flags & SSM_FLAG_ZOH) ? 1 : 0;
  return launch_status(ssm::launch_step(p, io_dtype == SSM_BF16, reinterpret_cast<hipStream_t>(stream)));
}

size_t ssm_scan_bwd_workspace_size(const ssm_shape* shape) {
  BwdPlan pl;
  if (!make_bwd_plan(shape, &pl)) return 0;
  return pl.total;
}

size_t ssm_scan_bwd_saved_workspace_size(const ssm_shape* shape) {
  BwdPlan pl;
  if (!make_bwd_plan(shape, &pl, true)) return 0;
  return pl.total;
}

}  // extern "C"

namespace {

// ssm_scan_bwd, and with saved set ssm_scan_bwd_saved (the checkpoints come from
// ssm_scan_fwd_save instead of a checkpoint pass).
ssm_status scan_bwd_impl(const ssm_shape* shape, const void* u, const void* delta, const float* A,
                         const void* B, const void* C, const float* D, const void* z,
                         const float* delta_bias, const float* initial_state, const void* dout,
                         const float* dfinal_state, const float* saved, void* du, void* ddelta, float* dA,
                         float* dB, float* dC, float* dD, void* dz, float* ddelta_bias, float* dinitial_state,
                         void* workspace, size_t workspace_bytes, struct ihipStream_t* stream) {
  if (!shape) return SSM_ERR_NULL;
  if (shape->io_dtype != SSM_F32 && shape->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (shape->flags & ~(SSM_FLAG_ZOH | SSM_FLAG_REVERSE)) return SSM_ERR_UNSUPPORTED;
  BwdPlan pl;
  if (!make_bwd_plan(shape, &pl, saved != nullptr)) return SSM_ERR_SHAPE;
  if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA || !dB || !dC || !workspace)
    return SSM_ERR_NULL;
  if (z && !dz) return SSM_ERR_NULL;
  if (!z) dz = nullptr;
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, initial_state, dout, dfinal_state, saved, du,
                        ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, workspace};
  for (const void* q : ptrs)
    if (misaligned(q)) return SSM_ERR_ALIGN;
  if (workspace_bytes < pl.total) return SSM_ERR_WORKSPACE;

  const int64_t Bsz = shape->batch, Dm = shape->dim, N = shape->dstate, L = shape->seqlen;
  const int64_t es = shape->io_dtype == SSM_BF16 ? 2 : 4;
  const int64_t BDL = Bsz * Dm * L, BNL = Bsz * N * L, BDN = Bsz * Dm * N;
  const Range ins[] = {span(u, BDL, es), span(delta, BDL, es), span(A, Dm * N, 4), span(B, BNL, es),
                       span(C, BNL, es), span(D, D ? Dm : 0, 4), span(z, z ? BDL : 0, es),
                       span(delta_bias, delta_bias ? Dm : 0, 4),
                       span(initial_state, initial_state ? BDN : 0, 4), span(dout, BDL, es),
                       span(dfinal_state, dfinal_state ? BDN : 0, 4),
                       span(saved, saved ? BDN * pl.nbk : 0, 4)};
  const Range outs[] = {span(du, BDL, es), span(ddelta, BDL, es), span(dA, Dm * N, 4), span(dB, BNL, 4),
                        span(dC, BNL, 4), span(dD, dD ? Dm : 0, 4), span(dz, dz ? BDL : 0, es),
                        span(ddelta_bias, ddelta_bias ? Dm : 0, 4),
                        span(dinitial_state, dinitial_state ? BDN : 0, 4),
                        span(workspace, (int64_t)pl.total, 1)};
  const size_t nin = sizeof(ins) / sizeof(ins[0]), nout = sizeof(outs) / sizeof(outs[0]);
  for (size_t i = 0; i < nout; ++i) {
    for (size_t j = 0; j < nin; ++j)
      if (overlaps(outs[i], ins[j])) return SSM_ERR_OVERLAP;
    for (size_t j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outs[j])) return SSM_ERR_OVERLAP;
  }

  const bool bf16 = shape->io_dtype == SSM_BF16;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  size_t off = 0;
  auto take = [&](size_t bytes) { float* q = reinterpret_cast<float*>(ws + off); off += bytes; return q; };
  float* ckpt = saved ? const_cast<float*>(saved) : take(pl.ckpt);  // read only when saved
  float* part_bc = take(pl.bc);
  float* part_a = take(pl.a);
  float* part_d = take(pl.d);
  float* seg_dsum = take(pl.seg_dsum);
  float* carries = take(pl.carries);
  float* seg_state = carries + Bsz * Dm * N;  // slots 1 .. S-1 of the carries, overwritten in place
  float* adj_q = take(pl.adj_q);
  float* adj_dsum = take(pl.adj_dsum);
  float* adj_in = take(pl.adj_in);
  const int vec = (L % (16 / es)) == 0 && L >= 8 ? 1 : 0;
  const int rev = (shape->flags & SSM_FLAG_REVERSE) ? 1 : 0;
  const int zoh = (shape->flags & SSM_FLAG_ZOH) ? 1 : 0;
  const bool split = pl.S > 1;
  const int64_t SB = pl.S * Bsz;

  // checkpoints: the state entering every 64-step block (a split sequence: each segment from
  // its carry, as in the forward's split), unless the forward saved them
  ssm_status rc = SSM_OK;
  if (!saved) {
    ssm::ScanParams fp;
    memset(&fp, 0, sizeof(fp));
    fp.u = u; fp.delta = delta; fp.A = A; fp.B = B; fp.C = C; fp.bias = delta_bias; fp.init = initial_state;
    fp.ckpt = ckpt;
    fp.Bsz = Bsz; fp.Dm = Dm; fp.N = N; fp.L = L;
    fp.S = (int)pl.S;
    fp.seg_len = split ? pl.seg_len : pl.nbk * 64;
    fp.nblk = (int)pl.nblk;
    fp.vec = vec && L < (int64_t(1) << 24) ? 1 : 0;  // the scan kernel's whole-chunk staging (above)
    fp.reverse = rev;
    fp.zoh = zoh;
    if (split) {
      fp.seg_state = seg_state;
      fp.seg_dsum = seg_dsum;
      rc = launch_status(ssm::launch_scan(fp, bf16, 1, st));
      if (rc != SSM_OK) return rc;
      fp.carries = carries;
      rc = launch_status(ssm::launch_carry(fp, st));
      if (rc != SSM_OK) return rc;
    }
    rc = launch_status(ssm::launch_ckpt(fp, bf16, st));
    if (rc != SSM_OK) return rc;
  }

  ssm::BwdParams bp;
  memset(&bp, 0, sizeof(bp));
  bp.u = u; bp.delta = delta; bp.A = A; bp.B = B; bp.C = C; bp.D = D; bp.z = z; bp.bias = delta_bias;
  bp.dout = dout; bp.dfinal = dfinal_state; bp.ckpt = ckpt;
  bp.du = du; bp.ddelta = ddelta; bp.dz = dz; bp.dh0 = dinitial_state;
  bp.part_bc = part_bc; bp.part_a = part_a; bp.part_d = part_d;
  bp.Bsz = Bsz; bp.Dm = Dm; bp.N = N; bp.L = L;
  bp.S = (int)pl.S;
  bp.seg_len = pl.seg_len;
  bp.nblk = (int)pl.nblk;
  bp.vec = vec;
  bp.reverse = rev;
  bp.zoh = zoh;
  if (split) {  // the adjoint entering each segment from the right
    bp.adj_q = adj_q;
    bp.adj_dsum = adj_dsum;
    rc = launch_status(ssm::launch_adj_summary(bp, bf16, st));
    if (rc != SSM_OK) return rc;
    rc = launch_status(ssm::launch_adj_carry(bp, adj_in, st));
    if (rc != SSM_OK) return rc;
    bp.adj_in = adj_in;
  }
  rc = launch_status(ssm::launch_bwd(bp, bf16, st));
  if (rc != SSM_OK) return rc;

  rc = launch_status(ssm::launch_reduce(dB, part_bc, pl.nblk, BNL, BNL, st));
  if (rc != SSM_OK) return rc;
  rc = launch_status(ssm::launch_reduce(dC, part_bc + pl.nblk * BNL, pl.nblk, BNL, BNL, st));
  if (rc != SSM_OK) return rc;
  rc = launch_status(ssm::launch_reduce(dA, part_a, SB, Dm * N, Dm * N, st));
  if (rc != SSM_OK) return rc;
  if (dD) {
    rc = launch_status(ssm::launch_reduce(dD, part_d, SB, Dm, Dm, st));
    if (rc != SSM_OK) return rc;
  }
  if (ddelta_bias) rc = launch_status(ssm::launch_reduce(ddelta_bias, part_d + SB * Dm, SB, Dm, Dm, st));
  return rc;
}

}  // namespace

extern "C" {

ssm_status ssm_scan_bwd(const ssm_shape* shape, const void* u, const void* delta, const float* A,
                        const void* B, const void* C, const float* D, const void* z,
                        const float* delta_bias, const float* initial_state, const void* dout,
                        const float* dfinal_state, void* du, void* ddelta, float* dA, float* dB,
                        float* dC, float* dD, void* dz, float* ddelta_bias, float* dinitial_state,
                        void* workspace, size_t workspace_bytes, struct ihipStream_t* stream) {
  return scan_bwd_impl(shape, u, delta, A, B, C, D, z, delta_bias, initial_state, dout, dfinal_state, nullptr,
                       du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, workspace, workspace_bytes,
                       stream);
}

ssm_status ssm_scan_bwd_saved(const ssm_shape* shape, const void* u, const void* delta, const float* A,
                              const void* B, const void* C, const float* D, const void* z,
                              const float* delta_bias, const float* initial_state, const void* dout,
                              const float* dfinal_state, const float* checkpoints, void* du, void* ddelta,
                              float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias,
                              float* dinitial_state, void* workspace, size_t workspace_bytes,
                              struct ihipStream_t* stream) {
  if (!checkpoints) return SSM_ERR_NULL;
  return scan_bwd_impl(shape, u, delta, A, B, C, D, z, delta_bias, initial_state, dout, dfinal_state,
                       checkpoints, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, workspace,
                       workspace_bytes, stream);
}

ssm_status ssm_conv1d_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int32_t io_dtype,
                          const void* x, const float* weight, const float* bias,
                          const void* initial_conv_state, void* u, void* final_conv_state,
                          struct ihipStream_t* stream) {
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (batch < 1 || dim < 1 || seqlen < 1 || width < 1 || width > 4) return SSM_ERR_SHAPE;
  if (batch > kMaxDim || dim > kMaxDim || seqlen > kMaxDim) return SSM_ERR_SHAPE;
  int64_t bd, bdl;
  if (!mul_ok(batch, dim, &bd) || !mul_ok(bd, seqlen, &bdl)) return SSM_ERR_SHAPE;
  if (bdl > (int64_t(1) << 31) * 255) return SSM_ERR_SHAPE;  // grid of the per-element path
  if (!x || !weight || !u) return SSM_ERR_NULL;
  const int64_t H = width - 1;
  const void* st_in = H > 0 ? initial_conv_state : nullptr;
  void* st_out = H > 0 ? final_conv_state : nullptr;
  const void* ptrs[] = {x, weight, bias, st_in, u, st_out};
  for (const void* q : ptrs)
    if (misaligned(q)) return SSM_ERR_ALIGN;
  const int64_t es = io_dtype == SSM_BF16 ? 2 : 4;
  const Range ins[] = {span(x, bdl, es), span(weight, dim * width, 4), span(bias, bias ? dim : 0, 4),
                       span(st_in, st_in ? bd * H : 0, es)};
  const Range ru = span(u, bdl, es), rs = span(st_out, st_out ? bd * H : 0, es);
  for (const Range& r : ins)
    if (overlaps(ru, r) || overlaps(rs, r)) return SSM_ERR_OVERLAP;
  if (overlaps(ru, rs)) return SSM_ERR_OVERLAP;

  ssm::ConvParams p;
  memset(&p, 0, sizeof(p));
  p.x = x; p.w = weight; p.bias = bias; p.state_in = st_in; p.u = u; p.state_out = st_out;
  p.Bsz = batch; p.Dm = dim; p.L = seqlen; p.K = (int)width;
  const int64_t V = 16 / es;  // elements per 16-byte chunk
  const int mode = (seqlen % V) == 0 ? 1 : 0;
  return launch_status(ssm::launch_conv(p, io_dtype == SSM_BF16, mode, reinterpret_cast<hipStream_t>(stream)));
}

ssm_status ssm_conv1d_update(int64_t batch, int64_t dim, int64_t width, int32_t io_dtype, void* conv_state,
                             const void* x, const float* weight, const float* bias, void* u,
                             struct ihipStream_t* stream) {
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (batch < 1 || dim < 1 || width < 1 || width > 4 || batch > kMaxDim || dim > kMaxDim) return SSM_ERR_SHAPE;
  int64_t bd;
  if (!mul_ok(batch, dim, &bd)) return SSM_ERR_SHAPE;
  if (bd > (int64_t(1) << 31) * 255) return SSM_ERR_SHAPE;
  const int64_t H = width - 1;
  void* st = H > 0 ? conv_state : nullptr;
  if (!x || !weight || !u || (H > 0 && !st)) return SSM_ERR_NULL;
  const void* ptrs[] = {st, x, weight, bias, u};
  for (const void* q : ptrs)
    if (misaligned(q)) return SSM_ERR_ALIGN;
  const int64_t es = io_dtype == SSM_BF16 ? 2 : 4;
  const Range ins[] = {span(x, bd, es), span(weight, dim * width, 4), span(bias, bias ? dim : 0, 4)};
  const Range ru = span(u, bd, es), rs = span(st, st ? bd * H : 0, es);
  for (const Range& r : ins)
    if (overlaps(ru, r) || overlaps(rs, r)) return SSM_ERR_OVERLAP;
  if (overlaps(ru, rs)) return SSM_ERR_OVERLAP;

  ssm::ConvParams p;
  memset(&p, 0, sizeof(p));
  p.x = x; p.w = weight; p.bias = bias; p.state_in = st; p.u = u; p.state_out = st;
  p.Bsz = batch; p.Dm = dim; p.L = 1; p.K = (int)width;
  return launch_status(ssm::launch_conv(p, io_dtype == SSM_BF16, 2, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
