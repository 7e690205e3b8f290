// Launch entry points of the kernels (host side).  Arguments are already
// validated by the C ABI layer; these functions only pick a template
// instance, size the grid and launch on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m3 {

struct DecodeArgs {
  float* state;
  const void *x, *B, *C;
  const float *dt, *A, *lam, *theta;
  const void *prev_B, *prev_x;
  void* y;
  int64_t BH;
  int R;
};
hipError_t launch_decode(int io_bf16, int N, int P, const DecodeArgs& a, hipStream_t s);

// The chunked forward over a short sequence, token by token (state in
// registers); the ABI layer picks it for short calls.
struct TokensArgs {
  const float* h0;   // nullable (B, H, N, P)
  float* h_final;    // nullable; may alias h0
  const void *x, *B, *C;
  const float *dt, *A, *lam, *theta;
  const void *prev_B, *prev_x;
  void* y;
  int64_t batch, L, H;
  int R;
};
constexpr int TOKENS_MAX = 16;  // at most this many tokens (all staged in LDS)
hipError_t launch_decode_tokens(int io_bf16, int N, int P, const TokensArgs& a, hipStream_t s);
// The same short call as one chunk of the chunked form on bf16 MFMAs (bf16
// io, P = 64, N in {64, 128}; at most TOKENS_MAX tokens).
bool short_chunk_supported(int io_bf16, int N, int P, int R);
hipError_t launch_short_chunk(int N, const TokensArgs& a, hipStream_t s);

struct RopeArgs {
  const void *B, *C;
  const float *dt, *theta, *angle0;
  void *B_rot, *C_rot;
  float* angle_final;
  float* totals;  // workspace: (B*H, nchunks, N/2) fp32
  int64_t batch, L, H;
  int R;
};
constexpr int ROPE_CHUNK = 64;
hipError_t launch_rope(int io_bf16, int N, const RopeArgs& a, hipStream_t s);

// The angles of rope_bc alone, as (cos, sin) pairs rounded to fp16 (one
// 32-bit word per (token, head, pair): cs (B, L, H, N/2)); uses a.totals as
// its workspace and writes a.angle_final when set.
hipError_t launch_rope_phi(int N, const RopeArgs& a, uint32_t* cs, hipStream_t s);

// The B/C prologue: projection, RMS normalisation, bias and rotation.
struct ProArgs {
  const void* u;       // (M, D) bf16, M = B*L tokens
  const void* W;       // (2*H*R*N, D) bf16: rows of W_B, then of W_C
  const float* gain;   // nullable (2*H*R*N), 16-byte aligned
  const float* bias;   // nullable (2*H*R*N), 16-byte aligned
  const uint32_t* cs;  // (M, H, N/2) fp16 (cos, sin) of the angles, from launch_rope_phi
  void *B_rot, *C_rot; // (M, H, R, N) bf16
  float eps;
  int64_t M, D;        // D a multiple of 64, at most 2^20
  int H, R;
};
hipError_t launch_bc_prologue(int N, const ProArgs& a, hipStream_t s);

struct WalkArgs {
  const void *x, *B, *C;
  const float *dt, *A, *lam, *theta;
  const float* h0;
  const void *prev_B, *prev_x;
  void* y;
  float* h_final;     // S == 1: final state (nullable)
  float* seg_end;     // S > 1: (B*H*S, N, P) end state of each segment walked from a zero state
  float* seg_tot;     // S > 1: (B*H*S, 1 + N/2) segment log-decay and angle totals
  float* chunk_meta;  // S > 1: (B*H, nchunks, 1 + N/2) segment-relative log-decay and angle at chunk start
  float* seg_in;      // S > 1: (B*H*S, N, P) true state entering each segment (from the segment scan)
  int64_t batch, L, H;
  int R, Q, S;
  int64_t seg_len;    // tokens per segment, a multiple of Q
};
// LDS bytes the general walker needs for these sizes (0 if they do not fit).
size_t walk_lds_bytes(int io_bf16, int N, int P, int Q, int R);
// The fast walker (bf16 io, N and P <= 64) applies to these sizes.
bool walk_fast_supported(int io_bf16, int N, int P, int Q, int R);
hipError_t launch_walk_fast(int N, int P, const WalkArgs& a, hipStream_t s);
// The sub-chunk walker (bf16 io, P = 64, N = 64 with Q in {32, 64} (Q = 64
// for R = 1), or N = 128 with R in {2, 4}) applies to these sizes; it walks
// sub-chunks of subwalk_qs(N, R) tokens (32 at N = 64, 64 at N = 64 with
// R = 1, 16 at N = 128) and records segment offsets every Q tokens.
bool subwalk_supported(int io_bf16, int N, int P, int Q, int R, int64_t H);
int subwalk_qs(int N, int R);
hipError_t launch_subwalk(int N, const WalkArgs& a, hipStream_t s);
// Chunked forward walk: the sub-chunk walker or the fast walker when one
// applies, the general walker otherwise.
hipError_t launch_walk(int io_bf16, int N, int P, const WalkArgs& a, hipStream_t s);
// The chunk length (tokens) the walk uses for a requested chunk Q: Q itself
// when a walker takes it as it is; the sub-chunk walker's own length when Q is
// shorter and that walker takes the sizes at its length; else the longest of
// Q/2, Q/4, ... (at least 16 virtual rows) whose tiles fit the general
// walker's LDS; 0 if none.  The chunked form is exact for any split, so only
// the rounding order changes.
int walk_chunk(int io_bf16, int N, int P, int Q, int R, int64_t H);

// Backward of the chunked forward: gradients of <dy, y> + <dh_final, h_final>.
struct BwdArgs {
  const void *x, *B, *C;
  const float *dt, *A, *lam, *theta;
  const float* h0;              // nullable
  const void *prev_B, *prev_x;  // nullable pair
  const void* dy;               // (B, L, H, R, P) io dtype
  const float* dh_final;        // nullable (B, H, N, P)
  void *dx, *dB, *dC;           // io dtype
  float *ddt, *dA, *dlam, *dtheta;
  float* dh0;                   // nullable
  void *dprev_B, *dprev_x;      // nullable pair (written when prev is given)
  float* ckpt;                  // workspace: (B*H, nchunks + 1, N, P) fp32 states at chunk starts
  int64_t batch, L, H;
  int R;
  // sequence segments (S > 1: each (b,h) walked as S runs of cps chunks by
  // separate blocks; the workspace arrays below are then set)
  int S;
  int64_t cps;
  float* seg_end;  // (B*H*S, N, P) segment end states walked from a zero state
  float* seg_tot;  // (B*H*S, 1 + N/2) segment log-decay and angle totals
  float* seg_in;   // (B*H*S, N, P) true states entering the segments
  float* dh_loc;   // (B*H*S, N, P) state adjoint at each segment start, walked from zero at its end
  float* dh_end;   // (B*H*S, N, P) true state adjoint at each segment end
  float* bnd;      // (B*H*S, 4) first-token dt / lam gradient parts across segment boundaries
  int ckpt_local;  // checkpoint walk: 1 = end states and totals only (segments from zero)
};
// tokens per chunk of the backward walk: 16, or 8 when N or P is 128 and
// R = 4, or 16 / R (16 virtual rows) when both are 128, so that the chunk's
// tiles fit LDS
constexpr int bwd_chunk_len(int N, int P, int R) {
  return (N > 64 && P > 64) ? 16 / R : (((N > 64 || P > 64) && R == 4) ? 8 : 16);
}
bool bwd_supported(int N, int P, int R);
hipError_t launch_chunked_bwd(int io_bf16, int N, int P, const BwdArgs& a, hipStream_t s);

// After a walk with S > 1 segments: segment scan (true incoming states and
// h_final) and the output fix-up of segments 1..S-1 (bf16 io).
hipError_t launch_segment_fixups(int io_bf16, int N, int P, const WalkArgs& a, hipStream_t s);
// The segment scan alone (seg_end, seg_tot -> seg_in and h_final when set).
hipError_t launch_seg_scan(int N, int P, const WalkArgs& a, hipStream_t s);

// Fill n floats of dst with src (or zeros when src is NULL).
hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t s);

}  // namespace m3
