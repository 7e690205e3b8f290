/*
 * mamba3_ssm.h -- C ABI of the MI355X (gfx950) Mamba-3 SSM layer core.
 *
 * Five operations, all asynchronous on a caller-given HIP stream:
 *
 *   mamba3_ssm_chunked_fwd   whole-sequence forward (prefill / training
 *                            forward) by the chunked parallel form;
 *   mamba3_ssm_chunked_bwd   its backward (training);
 *   mamba3_ssm_decode_step   one-token state update (generation);
 *   mamba3_rope_bc           the cumulative-angle rotation of B and C;
 *   mamba3_bc_prologue       the projection to B and C with their
 *                            normalisation, bias and rotation fused.
 *
 * What they compute (pages cited by title and section):
 *
 *  - linkstar.cloud/article/869, "第一刀：指数梯形离散化": with
 *    alpha_t = exp(dt_t A_t), beta_t = (1 - lam_t) dt_t alpha_t and
 *    gamma_t = lam_t dt_t,
 *        h_t = alpha_t h_{t-1} + beta_t B_{t-1} x_{t-1}^T + gamma_t B_t x_t^T;
 *    the same section gives the parallel form (a 1-semiseparable decay matrix
 *    times a 2-band matrix) that the chunked forward evaluates per chunk.
 *  - same page, "第二刀：复值状态空间": the complex state is a real state whose
 *    transition holds 2x2 rotations R(w) = [[cos w, -sin w], [sin w, cos w]]
 *    with w = dt_t theta_t[k] on pair (2k, 2k+1); equivalently the rotations
 *    move onto B and C as cumulative angles phi_t = sum_{s<=t} dt_s theta_s
 *    (B~ = R(-phi) B, C~ = R(-phi) C: a data-dependent RoPE).
 *  - same page, "第三刀：多输入多输出": B_t is N x R, x_t is P x R, the input
 *    term is the rank-R product B_t x_t^T, and y_t = C_t^T h_t is R x P.
 *  - yetianai.com/news/16273, "榨干硬件算力": chunks are computed in parallel
 *    internally and pass the state from chunk to chunk in order.
 *
 * Notation per (batch b, head h): L tokens, P head dim, N state size (even,
 * N/2 rotation pairs), R MIMO rank, Q chunk length in tokens.
 *
 * Layouts: row-major, contiguous, no strides.
 *   x, y            (B, L, H, R, P)   io dtype
 *   B, C            (B, L, H, R, N)   io dtype
 *   dt, A, lam      (B, L, H)         fp32 (dt > 0, already post-softplus)
 *   theta           (B, L, H, N/2)    fp32, one angle rate per pair
 *   h0, h_final     (B, H, N, P)      fp32, un-rotated ("true") frame
 *   prev_B          (B, H, R, N)      io dtype: raw B of the token before x[:,0]
 *   prev_x          (B, H, R, P)      io dtype: x of that token
 *   angle0/final    (B, H, N/2)       fp32
 *   decode: x, y (B, H, R, P); B, C, prev_B (B, H, R, N); prev_x (B, H, R, P);
 *           dt, A, lam (B, H); theta (B, H, N/2); state (B, H, N, P) fp32.
 * Pair (2k, 2k+1) of B, C and of the state rows is (real, imaginary) of
 * complex component k.
 *
 * Ownership: the caller owns every buffer (device memory unless stated).  The
 * library allocates nothing and, apart from the fixed per-GPU array of
 * mamba3_ssm_chunked_fwd_noalloc, keeps no mutable global state: every other
 * call is reentrant and may run on concurrent streams when its buffers are
 * disjoint from the other calls' buffers.  Alignment: x, B, C, theta, y and the workspace of chunked_fwd,
 * B, C, B_rot and C_rot of rope_bc, and the state of decode_step must be
 * 16-byte aligned; every other pointer must be aligned to its element size.
 *
 * Errors: every entry point validates its arguments on the host and returns a
 * status before any HIP call; nothing is launched on error.  M3_ERR_HIP
 * reports a failed launch.  Device-side faults surface, as usual in HIP, at
 * the caller's next synchronisation.
 *
 * Supported sizes: N in {16,32,64,128}; P in {16,32,64,128}; R in {1,2,4};
 * Q in {16,32,64}; io dtype fp32 or bf16: every combination, for the chunked
 * forward and the backward alike; M3_ERR_UNSUPPORTED outside it.  Where a
 * chunk's tiles would not fit in the 160 KiB of LDS of one compute unit
 * (fp32 io with Q*R = 256, N = P = 128 with long chunks) the chunked forward
 * walks each chunk as 2, 4 or 8 shorter pieces: the chunked form is exact for
 * any split (linkstar.cloud/article/869, "第一刀"), so only the rounding order
 * changes.  batch, seqlen and nheads may be 0 (empty input: nothing is read;
 * h_final receives h0, or zeros).  Size limits (M3_ERR_UNSUPPORTED beyond
 * them): batch and nheads at most 65535 each; the chunked forward and the
 * backward run one block of up to 512 threads per (b, h, segment) and the
 * decode step one of 256 threads per (b, h), and a launch holds fewer than
 * 2^32 threads, so batch * nheads * segments is at most 8,388,607 (16,777,215
 * for decode_step); split larger batches over several calls.
 */
#ifndef MAMBA3_SSM_H
#define MAMBA3_SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAMBA3_ABI_VERSION 1

typedef enum {
  M3_OK = 0,
  M3_ERR_NULL = 1,        /* a required pointer is NULL, or only one of prev_B/prev_x is given */
  M3_ERR_SHAPE = 2,       /* a negative size, or an odd dstate */
  M3_ERR_UNSUPPORTED = 3, /* size outside the supported set listed above */
  M3_ERR_ALIGN = 4,       /* a pointer breaks the alignment rule above */
  M3_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the queried size */
  M3_ERR_HIP = 6          /* a kernel launch failed */
} m3_status;

typedef enum { M3_F32 = 0, M3_BF16 = 1 } m3_dtype;

typedef struct {
  int64_t batch;    /* B */
  int64_t seqlen;   /* L (ignored by decode_step) */
  int64_t nheads;   /* H */
  int64_t headdim;  /* P */
  int64_t dstate;   /* N, even */
  int64_t rank;     /* R */
  int64_t chunk;    /* Q tokens per chunk (chunked_fwd only).  For bf16 io
                       with P = 64 and N = 64 (Q in {32, 64}) or N = 128
                       (R in {2, 4}) the library walks each chunk as 32- or
                       16-token sub-chunks (the chunked form is exact for
                       any split); segments and workspace follow Q.  At
                       N = 64 a chunk of 16 is walked (and segmented) as
                       chunks of 32.  Where Q's tiles do not fit the LDS the
                       walk (and with it segments and workspace) uses Q/2,
                       Q/4 or Q/8. */
  int32_t io_dtype; /* m3_dtype of x, B, C, y, prev_B, prev_x, B_rot, C_rot */
  int32_t flags;    /* chunked_fwd: bits 0..15 = number of sequence segments
                       walked in parallel per (b,h) (0 = chosen by the
                       library: more than one only for bf16 io when B*H <
                       256); M3_FLAG_CHUNK_WALK or M3_FLAG_TOKEN_PATH;
                       other bits must be 0.
                       Segments > 1 need bf16 io and B*H <= 65535.
                       chunked_bwd: bits 0..15 = number of sequence
                       segments (0 = chosen by the library: more than one
                       only when B*H < 256); other bits must be 0.  Other
                       entry points: must be 0. */
} m3_dims;

/* chunked_fwd: short calls (e.g. verifying k draft tokens of a decoder, with
 * the decode state as h0 and h_final) read the state once and write it once.
 * For bf16 io with P = 64 and N = 64 or 128, a call of at most
 * M3_TOKEN_PATH_MAX_L tokens runs as one chunk of the chunked form on bf16
 * MFMAs (two 8-token pieces for R = 4 past 8 tokens).  Other sizes run token
 * by token with the state held on chip (the one-token update of decode_step
 * applied to each token) for seqlen <= M3_TOKEN_PATH_SUBWALK_L when the
 * sub-chunk walker covers the sizes and seqlen <= M3_TOKEN_PATH_MAX_L
 * otherwise.  M3_FLAG_CHUNK_WALK forces the chunk walk; M3_FLAG_TOKEN_PATH
 * forces the token-by-token path (seqlen <= M3_TOKEN_PATH_MAX_L, else
 * M3_ERR_UNSUPPORTED); not both.  Every path computes the same function (the
 * chunked ones to the rounding of their bf16 products). */
#define M3_FLAG_CHUNK_WALK 0x10000
#define M3_FLAG_TOKEN_PATH 0x20000
#define M3_TOKEN_PATH_MAX_L 16
#define M3_TOKEN_PATH_SUBWALK_L 8

/* Whole-sequence forward.
 *   y_t = C_t^T h_t for every token, and h_final = h_L.
 * h0: nullable, the state before x[:,0] (true frame); NULL means zero.
 * prev_B, prev_x: nullable pair, the raw B and x of the token before x[:,0]
 *   (its trapezoid term enters the first update); NULL means none.
 * y: written (must not alias an input).  h_final: nullable; may alias h0.
 * workspace: device scratch of at least
 *   mamba3_ssm_chunked_fwd_workspace_size(d) bytes (may be NULL when that is 0);
 *   its contents on entry do not matter.  It is non-zero only when the
 *   sequence is walked as several segments (see flags): the segments are
 *   walked from a zero state in parallel, then a segment scan supplies the
 *   true incoming states and their contribution is added to y (linearity of
 *   the recurrence).
 * To continue a sequence, pass h_final as h0 and the last token's raw B and x
 * as prev_B / prev_x. */
m3_status mamba3_ssm_chunked_fwd(const m3_dims* d,
                                 const void* x, const void* B, const void* C,
                                 const float* dt, const float* A, const float* lam, const float* theta,
                                 const float* h0, const void* prev_B, const void* prev_x,
                                 void* y, float* h_final,
                                 void* workspace, size_t workspace_bytes, void* stream);
size_t mamba3_ssm_chunked_fwd_workspace_size(const m3_dims* d);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid
 * it): mamba3_ssm_chunked_fwd with no workspace argument.  The workspace comes
 * from a fixed array of M3_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on, until the process ends; this call allocates nothing.
 * Sizes whose workspace (mamba3_ssm_chunked_fwd_workspace_size) exceeds it
 * return M3_ERR_WORKSPACE before any HIP call (48 MiB covers, e.g., one
 * 65,536-token sequence of 32 heads at N = 128, P = 64, R = 4 walked as
 * segments).  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (concurrent streams, or several host threads)
 * race on it and must be serialised by the caller.  The array used is that of
 * the calling thread's current device (hipGetDevice), which must be the
 * device that stream belongs to.  The array's contents carry over between
 * calls; the forward needs none on entry.  Results are those of
 * mamba3_ssm_chunked_fwd with the same arguments. */
#define M3_NOALLOC_SCRATCH_BYTES (48u << 20)
m3_status mamba3_ssm_chunked_fwd_noalloc(const m3_dims* d,
                                         const void* x, const void* B, const void* C,
                                         const float* dt, const float* A, const float* lam, const float* theta,
                                         const float* h0, const void* prev_B, const void* prev_x,
                                         void* y, float* h_final, void* stream);

/* Backward of mamba3_ssm_chunked_fwd: the gradients of
 *     l = sum_t <dy_t, y_t> + <dh_final, h_final>
 * with respect to every input of the forward (the chain rule of the chunked
 * form, chunks walked in reverse order; same pages as the forward).
 *   dy: (B, L, H, R, P) io dtype.  dh_final: nullable (B, H, N, P) fp32; NULL
 *       means zero.
 *   dx (B, L, H, R, P), dB, dC (B, L, H, R, N): io dtype, written.
 *   ddt, dA, dlam (B, L, H), dtheta (B, L, H, N/2): fp32, written.
 *   dh0: nullable (B, H, N, P) fp32, written when given (also when h0 is NULL:
 *        the gradient with respect to a zero initial state).
 *   dprev_B (B, H, R, N), dprev_x (B, H, R, P): nullable pair, io dtype,
 *        written when prev_B/prev_x are given.
 * Supported: N and P in {16, 32, 64, 128}, R in {1, 2, 4}, io fp32 or bf16;
 * d->chunk must be a supported chunk length but the backward walks chunks of
 * its own: 16 tokens, 8 when N or P is 128 and R = 4, 16 / R when both are
 * 128 (the chunked form is exact for any split); nheads
 * at most 65536 (M3_ERR_UNSUPPORTED otherwise: offsets inside a chunk are
 * 32-bit).  Products: fp32 for fp32 io; bf16 MFMAs with fp32 accumulation
 * for bf16 io (operands rounded to bf16; the state product of the checkpoint
 * walk takes w B~ as bf16 hi + lo parts), with fp32 state checkpoints.
 * Segments (flags bits 0..15, for few long sequences): each sequence is cut
 * into runs of whole chunks that separate blocks walk at once.  The states at
 * segment starts come from walks from a zero state and the forward's segment
 * scan; the state adjoints at segment ends from walks of the adjoint from zero
 * and a reverse scan (the adjoint recurrence is linear too); the first token
 * of each segment takes the parts of its dt and lam gradients that the
 * previous segment computes.  The result is the same function; only rounding
 * differs.  The library picks ceil(512 / (B*H)) segments (at most a quarter
 * of the chunks) when B*H < 256 and one otherwise; a count above the number
 * of chunks is clamped to it.
 * workspace: at least
 * mamba3_ssm_chunked_bwd_workspace_size(d) bytes (the states at every chunk
 * start, and with segments four (B, H, S, N, P) fp32 arrays and small
 * per-segment records); its contents on entry do not matter.  Outputs must
 * not alias inputs.
 * Alignment: x, B, C, dy, dx, dB, dC, theta, dtheta and the workspace 16-byte;
 * the others their element size. */
m3_status mamba3_ssm_chunked_bwd(const m3_dims* d,
                                 const void* x, const void* B, const void* C,
                                 const float* dt, const float* A, const float* lam, const float* theta,
                                 const float* h0, const void* prev_B, const void* prev_x,
                                 const void* dy, const float* dh_final,
                                 void* dx, void* dB, void* dC,
                                 float* ddt, float* dA, float* dlam, float* dtheta,
                                 float* dh0, void* dprev_B, void* dprev_x,
                                 void* workspace, size_t workspace_bytes, void* stream);
size_t mamba3_ssm_chunked_bwd_workspace_size(const m3_dims* d);

/* One-token update, in place on the fp32 true-frame state:
 *   h <- alpha R(dt theta) [h + eps prev_B^T prev_x] + gamma B^T x,
 *   y  = C^T h (new state),  eps = (1 - lam) dt.
 * prev_B, prev_x: nullable pair (NULL: no previous token, e.g. the very first
 * token of a sequence).  seqlen and chunk of d are ignored.  y must not alias
 * any input. */
m3_status mamba3_ssm_decode_step(const m3_dims* d, float* state,
                                 const void* x, const void* B, const void* C,
                                 const float* dt, const float* A, const float* lam, const float* theta,
                                 const void* prev_B, const void* prev_x,
                                 void* y, void* stream);

/* Cumulative-angle rotation:
 *   phi_t = angle0 + sum_{s<=t} dt_s theta_s (per pair), B_rot = R(-phi_t) B_t,
 *   C_rot = R(-phi_t) C_t, angle_final = phi_L.
 * angle0, angle_final: nullable.  B_rot / C_rot must not alias B / C.
 * workspace: at least mamba3_rope_bc_workspace_size(d) bytes: the angle
 * totals of every 64-token chunk, which a first pass writes and the rotating
 * pass scans, so that every chunk of a long sequence is rotated in parallel.
 * The library allocates nothing, so the caller provides this array.  chunk
 * of d is ignored.  seqlen is limited to
 * 65535 * 64 tokens (M3_ERR_UNSUPPORTED). */
m3_status mamba3_rope_bc(const m3_dims* d, const void* B, const void* C,
                         const float* dt, const float* theta, const float* angle0,
                         void* B_rot, void* C_rot, float* angle_final,
                         void* workspace, size_t workspace_bytes, void* stream);
size_t mamba3_rope_bc_workspace_size(const m3_dims* d);

/* B/C prologue: the projection of the token activations to B and C with the
 * normalisation, bias and rotation applied on the way out, so that B_rot and
 * C_rot are written once (the input projection of the block,
 * papers.ananclaw.com/promo/explainers__2603-15569, "关键公式与“伪代码”"; RMS
 * normalisation and bias of B and C, linkstar.cloud/article/869,
 * "架构上的其他改动"; the rotation fused with the projection, same page,
 * "第二刀"):
 *   p_t = W u_t  (features ordered (B or C, head, rank, n)),
 *   v = p / sqrt(mean_n p^2 + eps) * gain + bias  (per (token, B or C, head,
 *       rank) vector of N entries),
 *   B_rot, C_rot = R(-phi_t) v with phi_t = angle0 + sum_{s<=t} dt_s theta_s
 *       (as mamba3_rope_bc), angle_final = phi_L.
 * B_rot and C_rot are in the frame that chunked_fwd expects when it is given
 * theta = 0 (then its h_final is in that frame too).
 *   d: batch, seqlen, nheads, dstate (N), rank (R) as for the core; headdim and
 *      chunk are ignored; io_dtype must be M3_BF16; flags 0.
 *   d_model: D, a positive multiple of 64 and at most 2^20
 *      (M3_ERR_UNSUPPORTED otherwise).
 *   u: (B, L, D) bf16.  W: (2*H*R*N, D) bf16, row-major: the H*R*N rows of
 *      W_B, then those of W_C.
 *   gain, bias: nullable (2, H, R, N) fp32 (NULL: 1 and 0).
 *   eps: >= 0 and finite (M3_ERR_UNSUPPORTED otherwise).  With eps = 0 an
 *      all-zero projected vector gives NaN, as the formula does.
 *   dt (B, L, H), theta (B, L, H, N/2), angle0 nullable (B, H, N/2): fp32.
 *   B_rot, C_rot: (B, L, H, R, N) bf16, written (must not alias inputs).
 *   angle_final: nullable (B, H, N/2) fp32, written.
 *   workspace: at least mamba3_bc_prologue_workspace_size(d) bytes (the fp32
 *      angle totals of every 64-token chunk, then the cosine and sine of every
 *      token's angles as fp16 pairs, 4 bytes per (token, head, pair));
 *      contents on entry do not matter.
 * Products: bf16 MFMAs with fp32 accumulation; normalisation, bias and
 * rotation in fp32; outputs rounded to bf16 (nearest even).
 * Alignment: u, W, B_rot, C_rot, gain, bias and the workspace 16-byte; the
 * others 4-byte.  seqlen is limited to 65535 * 64 tokens and 2*H*R*N to
 * 134,213,632 features (M3_ERR_UNSUPPORTED); any number of tokens B*L is taken (the
 * library launches the product in token slices that keep each launch under
 * 2^32 work-items). */
m3_status mamba3_bc_prologue(const m3_dims* d, int64_t d_model, const void* u, const void* W,
                             const float* gain, const float* bias, float eps,
                             const float* dt, const float* theta, const float* angle0,
                             void* B_rot, void* C_rot, float* angle_final,
                             void* workspace, size_t workspace_bytes, void* stream);
size_t mamba3_bc_prologue_workspace_size(const m3_dims* d);

const char* mamba3_status_string(m3_status s);
int mamba3_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA3_SSM_H */
