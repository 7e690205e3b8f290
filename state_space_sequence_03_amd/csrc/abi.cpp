// C ABI of the Mamba-3 SSM layer core: argument validation on the host (no
// HIP call happens before every check has passed), workspace sizing and
// dispatch to the gfx950 kernels.  The operations themselves are specified in
// include/mamba3_ssm.h.
#include "../../include/mamba3_ssm.h"

#include <hip/hip_runtime.h>

#include "m3_launch.hpp"

static_assert(M3_TOKEN_PATH_MAX_L <= m3::TOKENS_MAX, "the short-sequence path stages every token in LDS");

namespace {

bool in_set(int64_t v, std::initializer_list<int64_t> s) {
  for (int64_t e : s)
    if (v == e) return true;
  return false;
}

bool aligned(const void* p, uintptr_t a = 16) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Pointers read or written with 16-byte vector accesses must be 16-byte
// aligned; the others only need their element alignment.
bool all_aligned(std::initializer_list<const void*> vec16, std::initializer_list<const void*> elem, uintptr_t esz) {
  for (const void* p : vec16)
    if (p && !aligned(p, 16)) return false;
  for (const void* p : elem)
    if (p && !aligned(p, esz)) return false;
  return true;
}

// Common size checks.  need_chunk: chunked_fwd; need_p: P matters.
m3_status check_dims(const m3_dims* d, bool need_chunk, bool need_p) {
  if (!d) return M3_ERR_NULL;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads < 0) return M3_ERR_SHAPE;
  if (d->dstate <= 0 || d->rank <= 0 || (need_p && d->headdim <= 0)) return M3_ERR_SHAPE;
  if (need_chunk && d->chunk <= 0) return M3_ERR_SHAPE;
  if (d->dstate % 2 != 0) return M3_ERR_SHAPE;
  if (d->io_dtype != M3_F32 && d->io_dtype != M3_BF16) return M3_ERR_UNSUPPORTED;
  if (!in_set(d->dstate, {16, 32, 64, 128})) return M3_ERR_UNSUPPORTED;
  if (need_p && !in_set(d->headdim, {16, 32, 64, 128})) return M3_ERR_UNSUPPORTED;
  if (!in_set(d->rank, {1, 2, 4})) return M3_ERR_UNSUPPORTED;
  if (need_chunk) {
    if (!in_set(d->chunk, {16, 32, 64})) return M3_ERR_UNSUPPORTED;
    if (d->chunk * d->rank > 256) return M3_ERR_UNSUPPORTED;
  }
  // grid limits: (b, h) pairs index 32-bit block ids
  if (d->batch > 65535 || d->nheads > 65535) return M3_ERR_UNSUPPORTED;
  if (d->seqlen > (int64_t(1) << 31) / 64) return M3_ERR_UNSUPPORTED;
  return M3_OK;
}

int io_bf16(const m3_dims* d) { return d->io_dtype == M3_BF16 ? 1 : 0; }

// A launch holds fewer than 2^32 threads: `blocks` blocks of `threads` each.
static bool launch_fits(int64_t blocks, int threads) { return blocks <= ((int64_t(1) << 32) - 1) / threads; }

// Number of sequence segments walked in parallel per (b,h) and their length
// (whole chunks).  Requested through the low 16 bits of flags, else chosen so
// that at least ~512 walkers exist when B*H is small (bf16 io only; each
// segment keeps at least 4 chunks).  Never more segments than chunks.
struct SegPlan {
  int64_t S, seg_len, nchunks;
};
SegPlan seg_plan(const m3_dims* d) {
  SegPlan sp{1, 0, 0};
  sp.nchunks = d->seqlen > 0 ? (d->seqlen + d->chunk - 1) / d->chunk : 0;
  int64_t S = d->flags & 0xffff;
  const int64_t BH = d->batch * d->nheads;
  if (S == 0) {
    S = 1;
    if (d->io_dtype == M3_BF16 && BH > 0 && BH < 256) {
      S = (512 + BH - 1) / BH;
      if (S > sp.nchunks / 4) S = sp.nchunks / 4;
      if (S < 1) S = 1;
    }
  }
  if (S > sp.nchunks) S = sp.nchunks > 0 ? sp.nchunks : 1;
  const int64_t cps = sp.nchunks > 0 ? (sp.nchunks + S - 1) / S : 1;  // chunks per segment
  sp.seg_len = cps * d->chunk;
  sp.S = sp.nchunks > 0 ? (sp.nchunks + cps - 1) / cps : 1;
  return sp;
}

// Segments of the backward: each (b,h) walked as S runs of whole backward
// chunks by separate blocks. Requested through the low 16 bits of flags, else
// chosen so that ~512 blocks exist when B*H is small (each segment keeps at
// least 4 chunks).
struct BwdSegPlan {
  int64_t S, cps, nch;
};
BwdSegPlan bwd_seg_plan(const m3_dims* d) {
  BwdSegPlan sp{1, 0, 0};
  const int64_t q = m3::bwd_chunk_len((int)d->dstate, (int)d->headdim, (int)d->rank);
  sp.nch = d->seqlen > 0 ? (d->seqlen + q - 1) / q : 0;
  int64_t S = d->flags & 0xffff;
  const int64_t BH = d->batch * d->nheads;
  if (S == 0) {
    S = 1;
    if (BH > 0 && BH < 256) {
      S = (512 + BH - 1) / BH;
      if (S > sp.nch / 4) S = sp.nch / 4;
      if (S < 1) S = 1;
    }
  }
  if (S > sp.nch) S = sp.nch > 0 ? sp.nch : 1;
  sp.cps = sp.nch > 0 ? (sp.nch + S - 1) / S : 1;
  sp.S = sp.nch > 0 ? (sp.nch + sp.cps - 1) / sp.cps : 1;
  return sp;
}
// Workspace of the backward: the checkpoints, then (S > 1) the segment arrays,
// each 256-byte aligned.
struct BwdWs {
  size_t ckpt, seg_end, seg_in, dh_loc, dh_end, seg_tot, bnd, bytes;
};
BwdWs bwd_ws(const m3_dims* d, const BwdSegPlan& sp) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t BH = (size_t)(d->batch * d->nheads), NP = (size_t)(d->dstate * d->headdim), K1 = (size_t)(1 + d->dstate / 2);
  BwdWs w{};
  w.ckpt = 0;
  size_t o = up(sizeof(float) * BH * (size_t)(sp.nch + 1) * NP);
  if (sp.S > 1) {
    const size_t st = up(sizeof(float) * BH * (size_t)sp.S * NP);
    w.seg_end = o; o += st;
    w.seg_in = o; o += st;
    w.dh_loc = o; o += st;
    w.dh_end = o; o += st;
    w.seg_tot = o; o += up(sizeof(float) * BH * (size_t)sp.S * K1);
    w.bnd = o; o += up(sizeof(float) * BH * (size_t)sp.S * 4);
  }
  w.bytes = o;
  return w;
}

}  // namespace

extern "C" {

int mamba3_abi_version(void) { return MAMBA3_ABI_VERSION; }

const char* mamba3_status_string(m3_status s) {
  switch (s) {
    case M3_OK: return "ok";
    case M3_ERR_NULL: return "a required pointer is NULL (or only one of prev_B/prev_x was given)";
    case M3_ERR_SHAPE: return "invalid shape (negative size, zero head/state/rank/chunk, or odd dstate)";
    case M3_ERR_UNSUPPORTED: return "size outside the supported set";
    case M3_ERR_ALIGN: return "a pointer is misaligned (16 bytes for vector-accessed buffers, element size otherwise)";
    case M3_ERR_WORKSPACE: return "workspace missing or smaller than the queried size";
    case M3_ERR_HIP: return "a HIP kernel launch failed";
  }
  return "unknown status";
}

// Workspace of a segmented walk (floats): segment end states, incoming
// states, segment totals, per-chunk offsets, each 256-byte aligned.
struct SegWs {
  size_t end, in, tot, meta, bytes;
};
static SegWs seg_ws(const m3_dims* d, const SegPlan& sp) {
  const int64_t BH = d->batch * d->nheads, K = d->dstate / 2, NP = d->dstate * d->headdim;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  SegWs w{};
  size_t o = 0;
  w.end = o; o = up(o + sizeof(float) * (size_t)(BH * sp.S * NP));
  w.in = o; o = up(o + sizeof(float) * (size_t)(BH * sp.S * NP));
  w.tot = o; o = up(o + sizeof(float) * (size_t)(BH * sp.S * (1 + K)));
  w.meta = o; o = up(o + sizeof(float) * (size_t)(BH * sp.nchunks * (1 + K)));
  w.bytes = o;
  return w;
}

// The sizes as walked: the requested dims with the chunk replaced by the one
// the walk uses (m3::walk_chunk; the requested one unless its tiles do not fit
// the LDS).  Segment plans and offsets are kept at this granularity.
static m3_dims walked_dims(const m3_dims* d) {
  m3_dims w = *d;
  w.chunk = m3::walk_chunk(io_bf16(d), (int)d->dstate, (int)d->headdim, (int)d->chunk, (int)d->rank, d->nheads);
  return w;
}

size_t mamba3_ssm_chunked_fwd_workspace_size(const m3_dims* dq) {
  if (check_dims(dq, true, true) != M3_OK) return 0;
  if (dq->batch == 0 || dq->nheads == 0 || dq->seqlen == 0) return 0;
  const m3_dims dw = walked_dims(dq);
  const m3_dims* d = &dw;
  if (d->chunk <= 0) return 0;
  const SegPlan sp = seg_plan(d);
  if (sp.S <= 1) return 0;
  return seg_ws(d, sp).bytes;
}

m3_status mamba3_ssm_chunked_fwd(const m3_dims* dq, const void* x, const void* B, const void* C,
                                 const float* dt, const float* A, const float* lam, const float* theta,
                                 const float* h0, const void* prev_B, const void* prev_x, void* y,
                                 float* h_final, void* workspace, size_t workspace_bytes, void* stream) {
  m3_status st = check_dims(dq, true, true);
  if (st != M3_OK) return st;
  if ((dq->flags & ~(0xffff | M3_FLAG_CHUNK_WALK | M3_FLAG_TOKEN_PATH)) != 0) return M3_ERR_UNSUPPORTED;
  if ((dq->flags & M3_FLAG_CHUNK_WALK) && (dq->flags & M3_FLAG_TOKEN_PATH)) return M3_ERR_UNSUPPORTED;
  if ((dq->flags & M3_FLAG_TOKEN_PATH) && dq->seqlen > M3_TOKEN_PATH_MAX_L) return M3_ERR_UNSUPPORTED;
  // from here on the sizes as walked (a chunk whose tiles do not fit the LDS
  // is walked as shorter chunks)
  const m3_dims dw = walked_dims(dq);
  const m3_dims* d = &dw;
  if (d->chunk <= 0) return M3_ERR_UNSUPPORTED;
  const SegPlan sp = seg_plan(d);
  if (sp.S > 1 && (d->io_dtype != M3_BF16 || d->batch * d->nheads > 65535)) return M3_ERR_UNSUPPORTED;
  if (!launch_fits(d->batch * d->nheads * sp.S, 512)) return M3_ERR_UNSUPPORTED;  // one block per (b, h, segment)
  const bool empty = d->batch == 0 || d->nheads == 0;
  const bool has_tokens = !empty && d->seqlen > 0;
  if ((prev_B == nullptr) != (prev_x == nullptr)) return M3_ERR_NULL;
  if (has_tokens && (!x || !B || !C || !dt || !A || !lam || !theta || !y)) return M3_ERR_NULL;
  const uintptr_t esz = d->io_dtype == M3_BF16 ? 2 : 4;
  if (!all_aligned({x, B, C, y, workspace}, {prev_B, prev_x}, esz) ||
      !all_aligned({theta}, {dt, A, lam, h0, h_final}, 4))
    return M3_ERR_ALIGN;
  const size_t need = mamba3_ssm_chunked_fwd_workspace_size(dq);
  if (need > 0 && (!workspace || workspace_bytes < need)) return M3_ERR_WORKSPACE;
  if (empty) return M3_OK;
  hipStream_t s = (hipStream_t)stream;
  const int64_t BH = d->batch * d->nheads;
  if (d->seqlen == 0) {
    // no token: the final state is h0 (the token before, if any, has no successor)
    if (h_final && h_final != h0)
      return m3::launch_copy_f32(h_final, h0, BH * d->dstate * d->headdim, s) == hipSuccess ? M3_OK : M3_ERR_HIP;
    return M3_OK;
  }
  // the token path wins up to ~8 tokens against the sub-chunk walker and up to
  // 16 against the other walkers (measured at the 1.5B decode shapes)
  const int64_t tok_max =
      m3::subwalk_supported(io_bf16(d), (int)d->dstate, (int)d->headdim, (int)d->chunk, (int)d->rank, d->nheads)
          ? M3_TOKEN_PATH_SUBWALK_L
          : M3_TOKEN_PATH_MAX_L;
  // short calls as one chunk on MFMAs where that kernel covers the sizes
  const bool one_chunk = !(d->flags & (M3_FLAG_TOKEN_PATH | M3_FLAG_CHUNK_WALK)) && sp.S == 1 &&
                         d->seqlen <= M3_TOKEN_PATH_MAX_L &&
                         m3::short_chunk_supported(io_bf16(d), (int)d->dstate, (int)d->headdim, (int)d->rank);
  const bool token_path = !one_chunk && ((d->flags & M3_FLAG_TOKEN_PATH) ||
                                         (d->seqlen <= tok_max && sp.S == 1 && !(d->flags & M3_FLAG_CHUNK_WALK)));
  if (one_chunk || token_path) {
    m3::TokensArgs t{};
    t.h0 = h0; t.h_final = h_final; t.x = x; t.B = B; t.C = C;
    t.dt = dt; t.A = A; t.lam = lam; t.theta = theta; t.prev_B = prev_B; t.prev_x = prev_x; t.y = y;
    t.batch = d->batch; t.L = d->seqlen; t.H = d->nheads; t.R = (int)d->rank;
    // a few tokens: as one chunk on MFMAs, or token by token with the state in registers
    const hipError_t e = one_chunk ? m3::launch_short_chunk((int)d->dstate, t, s)
                                   : m3::launch_decode_tokens(io_bf16(d), (int)d->dstate, (int)d->headdim, t, s);
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
  }
  m3::WalkArgs a{};
  a.x = x; a.B = B; a.C = C; a.dt = dt; a.A = A; a.lam = lam; a.theta = theta;
  a.h0 = h0; a.prev_B = prev_B; a.prev_x = prev_x; a.y = y; a.h_final = h_final;
  a.batch = d->batch; a.L = d->seqlen; a.H = d->nheads;
  a.R = (int)d->rank; a.Q = (int)d->chunk; a.S = (int)sp.S;
  a.seg_len = sp.S > 1 ? sp.seg_len : sp.nchunks * d->chunk;
  if (sp.S > 1) {
    const SegWs w = seg_ws(d, sp);
    char* base = (char*)workspace;
    a.seg_end = (float*)(base + w.end);
    a.seg_in = (float*)(base + w.in);
    a.seg_tot = (float*)(base + w.tot);
    a.chunk_meta = (float*)(base + w.meta);
  }
  hipError_t e = m3::launch_walk(io_bf16(d), (int)d->dstate, (int)d->headdim, a, s);
  if (e == hipSuccess && sp.S > 1) e = m3::launch_segment_fixups(io_bf16(d), (int)d->dstate, (int)d->headdim, a, s);
  return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

size_t mamba3_ssm_chunked_bwd_workspace_size(const m3_dims* d) {
  if (check_dims(d, true, true) != M3_OK) return 0;
  if (d->batch == 0 || d->nheads == 0 || d->seqlen == 0) return 0;
  return bwd_ws(d, bwd_seg_plan(d)).bytes;
}

m3_status mamba3_ssm_chunked_bwd(const m3_dims* d, const void* x, const void* B, const void* C,
                                 const float* dt, const float* A, const float* lam, const float* theta,
                                 const float* h0, const void* prev_B, const void* prev_x,
                                 const void* dy, const float* dh_final,
                                 void* dx, void* dB, void* dC,
                                 float* ddt, float* dA, float* dlam, float* dtheta,
                                 float* dh0, void* dprev_B, void* dprev_x,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  m3_status st = check_dims(d, true, true);
  if (st != M3_OK) return st;
  if ((d->flags & ~0xffff) != 0) return M3_ERR_UNSUPPORTED;
  if (!m3::bwd_supported((int)d->dstate, (int)d->headdim, (int)d->rank)) return M3_ERR_UNSUPPORTED;
  if (d->nheads > 65536) return M3_ERR_UNSUPPORTED;  // 32-bit offsets inside a chunk
  {
    // one block per (b, h, segment); the segment scans run one thread per
    // (b, h, pair, column)
    const BwdSegPlan sp0 = bwd_seg_plan(d);
    if (!launch_fits(d->batch * d->nheads * sp0.S, 512)) return M3_ERR_UNSUPPORTED;
    if (sp0.S > 1 && !launch_fits(d->batch * d->nheads * (d->dstate / 2) * d->headdim, 1)) return M3_ERR_UNSUPPORTED;
  }
  const bool empty = d->batch == 0 || d->nheads == 0;
  const bool has_tokens = !empty && d->seqlen > 0;
  if ((prev_B == nullptr) != (prev_x == nullptr) || (dprev_B == nullptr) != (dprev_x == nullptr)) return M3_ERR_NULL;
  if (has_tokens && (!x || !B || !C || !dt || !A || !lam || !theta || !dy || !dx || !dB || !dC || !ddt || !dA ||
                     !dlam || !dtheta))
    return M3_ERR_NULL;
  const uintptr_t esz = d->io_dtype == M3_BF16 ? 2 : 4;
  if (!all_aligned({x, B, C, dy, dx, dB, dC, workspace}, {prev_B, prev_x, dprev_B, dprev_x}, esz) ||
      !all_aligned({theta, dtheta}, {dt, A, lam, h0, dh_final, ddt, dA, dlam, dh0}, 4))
    return M3_ERR_ALIGN;
  const size_t need = mamba3_ssm_chunked_bwd_workspace_size(d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return M3_ERR_WORKSPACE;
  if (empty) return M3_OK;
  hipStream_t s = (hipStream_t)stream;
  const int64_t BH = d->batch * d->nheads;
  if (d->seqlen == 0) {
    // h_final = h0: dh0 = dh_final; the previous token has no successor
    hipError_t e = hipSuccess;
    if (dh0) e = m3::launch_copy_f32(dh0, dh_final, BH * d->dstate * d->headdim, s);
    if (e == hipSuccess && prev_B && dprev_B) {
      const int64_t nb = BH * d->rank * d->dstate * (int64_t)esz, nx = BH * d->rank * d->headdim * (int64_t)esz;
      // zero fill with a kernel (byte sizes are multiples of 4: N and P are even)
      e = m3::launch_copy_f32((float*)dprev_B, nullptr, nb / 4, s);
      if (e == hipSuccess) e = m3::launch_copy_f32((float*)dprev_x, nullptr, nx / 4, s);
    }
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
  }
  m3::BwdArgs a{};
  a.x = x; a.B = B; a.C = C; a.dt = dt; a.A = A; a.lam = lam; a.theta = theta;
  a.h0 = h0; a.prev_B = prev_B; a.prev_x = prev_x; a.dy = dy; a.dh_final = dh_final;
  a.dx = dx; a.dB = dB; a.dC = dC; a.ddt = ddt; a.dA = dA; a.dlam = dlam; a.dtheta = dtheta;
  a.dh0 = dh0; a.dprev_B = prev_B ? dprev_B : nullptr; a.dprev_x = prev_B ? dprev_x : nullptr;
  a.ckpt = (float*)workspace;
  a.batch = d->batch; a.L = d->seqlen; a.H = d->nheads; a.R = (int)d->rank;
  const BwdSegPlan sp = bwd_seg_plan(d);
  a.S = (int)sp.S;
  a.cps = sp.cps;
  if (sp.S > 1) {
    const BwdWs w = bwd_ws(d, sp);
    char* base = (char*)workspace;
    a.seg_end = (float*)(base + w.seg_end);
    a.seg_in = (float*)(base + w.seg_in);
    a.dh_loc = (float*)(base + w.dh_loc);
    a.dh_end = (float*)(base + w.dh_end);
    a.seg_tot = (float*)(base + w.seg_tot);
    a.bnd = (float*)(base + w.bnd);
  }
  return m3::launch_chunked_bwd(io_bf16(d), (int)d->dstate, (int)d->headdim, a, s) == hipSuccess ? M3_OK : M3_ERR_HIP;
}

m3_status mamba3_ssm_decode_step(const m3_dims* d, float* state, const void* x, const void* B,
                                 const void* C, const float* dt, const float* A, const float* lam,
                                 const float* theta, const void* prev_B, const void* prev_x, void* y,
                                 void* stream) {
  m3_status st = check_dims(d, false, true);
  if (st != M3_OK) return st;
  if (d->flags != 0) return M3_ERR_UNSUPPORTED;
  if (!launch_fits(d->batch * d->nheads, 256)) return M3_ERR_UNSUPPORTED;  // one block per (b, h)
  const bool empty = d->batch == 0 || d->nheads == 0;
  if ((prev_B == nullptr) != (prev_x == nullptr)) return M3_ERR_NULL;
  if (!empty && (!state || !x || !B || !C || !dt || !A || !lam || !theta || !y)) return M3_ERR_NULL;
  const uintptr_t esz = d->io_dtype == M3_BF16 ? 2 : 4;
  if (!all_aligned({state}, {x, B, C, prev_B, prev_x, y}, esz) || !all_aligned({}, {dt, A, lam, theta}, 4))
    return M3_ERR_ALIGN;
  if (empty) return M3_OK;
  m3::DecodeArgs a{};
  a.state = state; a.x = x; a.B = B; a.C = C; a.dt = dt; a.A = A; a.lam = lam; a.theta = theta;
  a.prev_B = prev_B; a.prev_x = prev_x; a.y = y;
  a.BH = d->batch * d->nheads;
  a.R = (int)d->rank;
  hipError_t e = m3::launch_decode(io_bf16(d), (int)d->dstate, (int)d->headdim, a, (hipStream_t)stream);
  return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

size_t mamba3_rope_bc_workspace_size(const m3_dims* d) {
  if (check_dims(d, false, false) != M3_OK) return 0;
  const int64_t nchunks = (d->seqlen + m3::ROPE_CHUNK - 1) / m3::ROPE_CHUNK;
  return sizeof(float) * (size_t)(d->batch * d->nheads * nchunks * (d->dstate / 2));
}

m3_status mamba3_rope_bc(const m3_dims* d, const void* B, const void* C, const float* dt,
                         const float* theta, const float* angle0, void* B_rot, void* C_rot,
                         float* angle_final, void* workspace, size_t workspace_bytes, void* stream) {
  m3_status st = check_dims(d, false, false);
  if (st != M3_OK) return st;
  if (d->flags != 0) return M3_ERR_UNSUPPORTED;
  if ((d->seqlen + m3::ROPE_CHUNK - 1) / m3::ROPE_CHUNK > 65535) return M3_ERR_UNSUPPORTED;  // grid limit
  const bool empty = d->batch == 0 || d->nheads == 0;
  const bool has_tokens = !empty && d->seqlen > 0;
  if (has_tokens && (!B || !C || !dt || !theta || !B_rot || !C_rot)) return M3_ERR_NULL;
  if (!all_aligned({B, C, B_rot, C_rot}, {dt, theta, angle0, angle_final, workspace}, 4)) return M3_ERR_ALIGN;
  const size_t need = mamba3_rope_bc_workspace_size(d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return M3_ERR_WORKSPACE;
  if (empty) return M3_OK;
  m3::RopeArgs a{};
  a.B = B; a.C = C; a.dt = dt; a.theta = theta; a.angle0 = angle0;
  a.B_rot = B_rot; a.C_rot = C_rot; a.angle_final = angle_final; a.totals = (float*)workspace;
  a.batch = d->batch; a.L = d->seqlen; a.H = d->nheads; a.R = (int)d->rank;
  hipError_t e = m3::launch_rope(io_bf16(d), (int)d->dstate, a, (hipStream_t)stream);
  return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

// Workspace of the B/C prologue: the angle chunk totals, then the angles
// (B, L, H, N/2) fp32, each 256-byte aligned.
// prologue workspace: fp32 angle totals per (b, h, 64-token chunk, pair), then
// the fp16 (cos, sin) pair of every (token, head, pair) as one 32-bit word
struct ProWs {
  size_t totals, cs, bytes;
};
static ProWs pro_ws(const m3_dims* d) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t K = (size_t)(d->dstate / 2);
  const size_t nchunks = (size_t)((d->seqlen + m3::ROPE_CHUNK - 1) / m3::ROPE_CHUNK);
  ProWs w{};
  w.totals = 0;
  w.cs = up(sizeof(float) * (size_t)(d->batch * d->nheads) * nchunks * K);
  w.bytes = w.cs + up(sizeof(uint32_t) * (size_t)(d->batch * d->seqlen * d->nheads) * K);
  return w;
}

size_t mamba3_bc_prologue_workspace_size(const m3_dims* d) {
  if (check_dims(d, false, false) != M3_OK) return 0;
  if (d->batch == 0 || d->nheads == 0 || d->seqlen == 0) return 0;
  return pro_ws(d).bytes;
}

m3_status mamba3_bc_prologue(const m3_dims* d, int64_t d_model, const void* u, const void* W, const float* gain,
                             const float* bias, float eps, const float* dt, const float* theta,
                             const float* angle0, void* B_rot, void* C_rot, float* angle_final, void* workspace,
                             size_t workspace_bytes, void* stream) {
  m3_status st = check_dims(d, false, false);
  if (st != M3_OK) return st;
  if (d_model <= 0) return M3_ERR_SHAPE;
  if (d->flags != 0 || d->io_dtype != M3_BF16) return M3_ERR_UNSUPPORTED;
  // 32-bit offsets inside a 256-row operand tile
  if (d_model % 64 != 0 || d_model > (int64_t(1) << 20) || !(eps >= 0.0f) || eps > 3.0e38f) return M3_ERR_UNSUPPORTED;
  if ((d->seqlen + m3::ROPE_CHUNK - 1) / m3::ROPE_CHUNK > 65535) return M3_ERR_UNSUPPORTED;  // grid limit
  {
    // the product's launches: 256 blocks of 512 threads per group of 16 x 16
    // tiles of 256 tokens x 256 features, token rows sliced so that a launch
    // stays under 2^32 work-items; one row of tile groups must fit
    const int64_t nfb = (2 * d->nheads * d->rank * d->dstate + 255) / 256;
    if ((nfb + 15) / 16 > (((int64_t(1) << 32) - 1) / 512) / 256) return M3_ERR_UNSUPPORTED;
  }
  const bool empty = d->batch == 0 || d->nheads == 0;
  const bool has_tokens = !empty && d->seqlen > 0;
  if (has_tokens && (!u || !W || !dt || !theta || !B_rot || !C_rot)) return M3_ERR_NULL;
  if (!all_aligned({u, W, B_rot, C_rot, gain, bias, workspace}, {dt, theta, angle0, angle_final}, 4))
    return M3_ERR_ALIGN;
  const size_t need = mamba3_bc_prologue_workspace_size(d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return M3_ERR_WORKSPACE;
  if (empty) return M3_OK;
  hipStream_t s = (hipStream_t)stream;
  const int N = (int)d->dstate;
  m3::RopeArgs r{};
  r.dt = dt; r.theta = theta; r.angle0 = angle0; r.angle_final = angle_final;
  r.batch = d->batch; r.L = d->seqlen; r.H = d->nheads; r.R = (int)d->rank;
  const ProWs w = pro_ws(d);
  uint32_t* cs = nullptr;
  if (has_tokens) {
    r.totals = (float*)((char*)workspace + w.totals);
    cs = (uint32_t*)((char*)workspace + w.cs);
  }
  hipError_t e = m3::launch_rope_phi(N, r, cs, s);
  if (e != hipSuccess || !has_tokens) return e == hipSuccess ? M3_OK : M3_ERR_HIP;
  m3::ProArgs a{};
  a.u = u; a.W = W; a.gain = gain; a.bias = bias; a.cs = cs; a.B_rot = B_rot; a.C_rot = C_rot; a.eps = eps;
  a.M = d->batch * d->seqlen; a.D = d_model; a.H = (int)d->nheads; a.R = (int)d->rank;
  e = m3::launch_bc_prologue(N, a, s);
  return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

}  // extern "C"
