// Prefill walker for bf16 io with P = 64 and N in {64, 128} (the 1.5B-scale
// and the long-context head shapes): the sequence is walked in sub-chunks of
// QS tokens (32 for N = 64, 64 for N = 64 with R = 1, 16 for N = 128), two
// blocks per compute unit.
//
// Computes what the other walkers compute (chunk.hip, chunk_fast.hip): the
// chunked form of the exponential-trapezoidal recurrence with data-dependent
// RoPE and rank-R inputs (linkstar.cloud/article/869, "第一刀", "第二刀",
// "第三刀"; yetianai.com/news/16273, "榨干硬件算力").  A requested chunk (a
// multiple of QS) is walked as QS-token sub-chunks: the chunked form holds
// for any split of the sequence, because the state carried across a boundary
// is the exact state there.  Segment offsets for the fix-up pass are still
// recorded at the requested chunk boundaries.
//
// gfx950 data flow:
//  * 256 threads and under 80 KB of LDS per block, so two blocks (two (b,h)
//    sequences or segments) share a compute unit and one block's staging and
//    loads overlap the other block's matrix work.  For R = 1 with an even
//    number of (b,h), one 512-thread block walks two adjacent heads instead
//    (each half with its own LDS region): each token's rows of the two heads
//    are then read together, 256 bytes instead of 128.
//  * Coalesced loads.  Staging thread (t, c) owns token t of the sub-chunk (for
//    R = 1: the adjacent tokens 2t, 2t + 1) and the 16-byte column c of each
//    rank row of B (and of x, and of theta's row), so a wave instruction reads
//    whole rows.  Each wave keeps the C rows of its own output tiles in the
//    MFMA operand layout (16 bytes per lane).
//  * Cumulative log-decay and angles: wave scans over the tokens a wave holds
//    (slot_scan: DPP and row swaps, no LDS permutes), plus an exchange of wave
//    totals through LDS.  The wave scans of the next sub-chunk run at the end
//    of the current one, so the exchange shares the sub-chunk's first barrier.
//  * sin/cos are computed once per (token, pair) by the staging thread, which
//    rotates all R ranks of B with them and stores them as a bf16 table for
//    the rotation of C: two bf16 dot products per pair (fp32 sums), the result
//    rounded to bf16 like every MFMA operand.
//  * y leaves the wave as 32 contiguous bytes per lane after a 4 x 4 transpose
//    across the wave's 16-lane rows.
//  * LDS arrays keep their natural row layout with the 16-byte columns
//    XOR-swizzled per row (x rows padded instead), so the 16-byte operand
//    reads and the transpose reads (ds_read_b64_tr_b16) of 16 lanes fall in
//    distinct banks.
//  * Two barriers per sub-chunk: after the previous sub-chunk's last LDS read
//    (and the scan exchange), and after staging.
//  * Wave priorities order the two blocks' waves on a SIMD: matrix phases
//    first, then staging, then the rest.
//
// Precision matches the other bf16 walkers: bf16 MFMA operands with fp32
// accumulation; the chunk state uses w B~ split into bf16 hi + lo parts.
#include "m3_common.hpp"
#include "m3_lanes.hpp"
#include "m3_launch.hpp"
#include "m3_order.hpp"

namespace m3 {

namespace {

// LDS layout of one block
template <int N, int R>
struct SW {
  // sub-chunk length: 32 tokens at N = 64 (64 for R = 1, where a token is one
  // virtual row), 16 at N = 128
  static constexpr int P = 64, K = N / 2, QS = N == 64 ? (R == 1 ? 64 : 32) : 16, V = QS * R;
  static constexpr int CH = N / 8;        // 16-byte columns of a B / C rank row = staging threads per token slot
  static constexpr int TPT = QS * CH / 256;  // tokens per staging thread: 2 (adjacent tokens) for R = 1 at N = 64, else 1
  static constexpr int BROW = 2 * N;      // bytes per row of B~ [V][N]
  static constexpr int XP = 144;          // bytes per row of X [V][64] (128 + 16: transpose reads of 4 rows hit distinct banks)
  static constexpr int WROW = 2 * V;      // bytes per row of (w B~)^T [N][V]
  static constexpr int WCPR = WROW / 16;  // 16-byte columns per row of (w B~)^T
  static constexpr int HROW = 2 * N;      // bytes per row of H'^T [64][N]
  static constexpr int CSROW = 4 * K;     // bytes per row of the (cos, sin) table [QS][K]
  static constexpr int TOTW = K + 4;      // floats per wave in the scan exchange
  static constexpr int OFF_B = 0;
  static constexpr int OFF_X = OFF_B + V * BROW;
  static constexpr int OFF_WH = OFF_X + V * XP;
  static constexpr int OFF_WL = OFF_WH + N * WROW;
  static constexpr int OFF_H = OFF_WL + N * WROW;
  static constexpr int OFF_CS = OFF_H + P * HROW;
  static constexpr int OFF_SC = OFF_CS + QS * CSROW;   // per token: log2 decay, q, gamma, exp(decay)
  static constexpr int OFF_TOT = OFF_SC + QS * 16;
  static constexpr int OFF_TH = OFF_TOT + 4 * TOTW * 4;  // sub-chunk total rotation [K] float2
  static constexpr int BYTES = OFF_TH + K * 8;
};
static_assert(SW<64, 4>::BYTES <= 80 * 1024 && SW<128, 4>::BYTES <= 80 * 1024 && SW<64, 1>::BYTES <= 80 * 1024,
              "two blocks per compute unit");

// rows of (w B~)^T: 16 consecutive rows, and the rows 8 apart that one staging
// instruction writes, spread over the banks
template <int WCPR>
__host__ __device__ constexpr int fW(int n) {
  return WCPR == 4 ? ((n ^ (n >> 2)) & 3) : ((n ^ (n >> 3)) & (WCPR - 1));
}
// The staging thread of column c writes rows n = 8c + e (e < 8); their
// swizzles differ from those of rows 8c and 8c + 4 by e & 3 only, so one
// xor-add per row forms the address.
template <int WCPR>
constexpr bool fW_rows_of_column_ok() {
  for (int c = 0; c < 64; ++c)
    for (int e = 0; e < 8; ++e)
      if (fW<WCPR>(8 * c + e) != (fW<WCPR>(8 * c + 4 * (e >> 2)) ^ (e & 3))) return false;
  return true;
}
static_assert(fW_rows_of_column_ok<4>() && fW_rows_of_column_ok<8>() && fW_rows_of_column_ok<16>(), "row swizzle");

}  // namespace

int subwalk_qs(int N, int R) { return N == 64 ? (R == 1 ? SW<64, 1>::QS : SW<64, 2>::QS) : SW<128, 2>::QS; }

bool subwalk_supported(int io_bf16, int N, int P, int Q, int R, int64_t H) {
  if (!io_bf16 || P != 64) return false;
  // per-thread offsets within a sub-chunk are 32-bit: 32 tokens of (H, R, N or P) bf16
  if (H <= 0 || H * R * (N > P ? N : P) > (int64_t(1) << 24)) return false;
  if (N == 64) return R == 1 ? Q == 64 : ((Q == 32 || Q == 64) && (R == 2 || R == 4));
  if (N == 128) return (Q == 16 || Q == 32 || Q == 64) && (R == 2 || R == 4);
  return false;
}

// HPB heads per block: 1, or 2 adjacent (b,h) sequences walked in lockstep
// by the two halves of a 512-thread block, each with its own LDS region (R =
// 1: each token's 128-byte rows of the two heads are then read together)
template <int N, int R, int HPB>
__global__ __launch_bounds__(256 * HPB, 2 / HPB) void subchunk_walk_kernel(WalkArgs a) {
  typedef SW<N, R> Ly;
  constexpr int P = 64, K = Ly::K, QS = Ly::QS, V = Ly::V, NW = 4, CH = Ly::CH, TPT = Ly::TPT;
  constexpr int RC = TPT * R;               // (w B~)^T columns a staging thread writes: its tokens' ranks
  constexpr int lgR = R == 4 ? 2 : (R == 2 ? 1 : 0);
  constexpr int NKS = N / 32;               // 32-wide slabs of the state dimension (MFMA k steps)
  constexpr int NCT = V / 16;               // column tiles of Y (16 virtual rows each)
  constexpr int NCW = NCT == 8 ? 2 : 1;     // column tiles per wave
  constexpr int PTW = NCT >= 4 ? 4 : 2;     // 16-wide p tiles per wave
  constexpr int NKB = V / 32;               // 32-row slabs of the sub-chunk
  constexpr int NTW = N / 64;               // 16-row state tiles per wave
  constexpr int XIT = R * 8 / CH;           // x row pieces per staging thread
  constexpr int BCPR = N / 8;               // 16-byte columns per row of B~, H'^T and the table
  constexpr float LOG2E = 1.4426950408889634f;
  static_assert(XIT >= 1 && NCT >= 2, "shape");

  __shared__ __align__(16) unsigned char smem_all[HPB * Ly::BYTES];
  const int half = HPB == 1 ? 0 : (int)(threadIdx.x >> 8);
  unsigned char* smem = smem_all + half * Ly::BYTES;
  unsigned char* sB = smem + Ly::OFF_B;
  unsigned char* sX = smem + Ly::OFF_X;
  unsigned char* sWh = smem + Ly::OFF_WH;
  unsigned char* sWl = smem + Ly::OFF_WL;
  unsigned char* sH = smem + Ly::OFF_H;
  unsigned char* sCS = smem + Ly::OFF_CS;
  float4* sSC = (float4*)(smem + Ly::OFF_SC);  // per token: log2 decay, q, gamma, exp(decay)
  float* sTot = (float*)(smem + Ly::OFF_TOT);  // per wave: K angle totals, log-decay total
  float2* sTh = (float2*)(smem + Ly::OFF_TH);

  const int wave = (threadIdx.x >> 6) & 3;
  // lane coordinates; re-derived from an opaque copy of the thread id in every
  // sub-chunk so that the compiler recomputes the LDS addresses next to their
  // uses instead of hoisting dozens of them into registers for the whole walk
  int tid, lane, m16, g, jj, uu, st_t, st_c;
  auto coords = [&](int id) __attribute__((always_inline)) {
    tid = id;
    lane = id & 63;
    m16 = lane & 15;
    g = lane >> 4;
    jj = m16 >> 2;          // transpose-read coordinates
    uu = lane & 3;
    st_t = id / CH;         // staging: token slot (tokens TPT st_t ..), 16-byte column
    st_c = id % CH;
  };
  coords(threadIdx.x & 255);

  const int64_t S = a.S;
  // block order: adjacent heads on one XCD (m3_order.hpp)
  int64_t seg, bh;
  walker_of_block(blockIdx.x, gridDim.x, a.batch * a.H / HPB, S, bh, seg);
  bh = bh * HPB + half;
  const int64_t blk = bh * S + seg;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t L = a.L, H = a.H;
  const int64_t t0 = seg * a.seg_len;
  const int64_t t1 = (t0 + a.seg_len < L) ? t0 + a.seg_len : L;
  auto tokS = [&](int64_t tok) { return (b * L + tok) * H + h; };
  // Global addresses: a block-uniform base at the sub-chunk's first token plus
  // a 32-bit per-thread offset (tokens t < QS of the sub-chunk are t * H rows
  // further; the launch checks that these offsets fit in 32 bits).
  const uint32_t Hu = (uint32_t)H;
  auto rowp = [&](const void* base, int64_t c0, int rowbytes) __attribute__((always_inline)) {
    return (const unsigned char*)base + tokS(c0) * rowbytes;
  };
  const int64_t QM = a.Q;                          // chunk of the segment offsets (a multiple of QS)
  const int64_t nchunks_meta = (L + QM - 1) / QM;
  const int spc = a.Q / QS;                        // sub-chunks per requested chunk: 1, 2 or 4
  int kin = 0;                                     // sub-chunk index within the requested chunk
  int64_t meta_at = (bh * nchunks_meta + t0 / QM) * (1 + K);  // offsets of the current requested chunk

  // output tiles of this wave: the causal work of tiles (w, NCT-1-w) is equal
  int ctl[NCW];
  if constexpr (NCW == 2) {
    ctl[0] = NCT - 1 - wave;  // larger causal range first
    ctl[1] = wave;
  } else if constexpr (NCT == 4) {
    ctl[0] = wave;
  } else {
    ctl[0] = wave & 1;
  }
  const int pt0 = PTW == 4 ? 0 : 2 * (wave >> 1);

  // ---------------- prefetch registers (next sub-chunk) ----------------
  uint4 rB[TPT][R], rX[TPT][XIT];
  float4 rTh[TPT];
  float rdt[TPT], rA[TPT], rlam[TPT], rdt1[TPT], rlam1[TPT];
  uint4 rC[NCW][NKS];

  // Tokens past the end of the segment read the last valid token instead: only
  // their dt, lam (hence q = gamma = 0) are zeroed, which removes them exactly
  // from the scores, the outputs and the state while every operand stays finite.
  auto load_BX = [&](int64_t c0) __attribute__((always_inline)) {
    const int nvalid = (int)((t1 - c0) < QS ? (t1 - c0) : QS);
    const unsigned char* gB = rowp(a.B, c0, R * N * 2);
    const unsigned char* gX = rowp(a.x, c0, R * P * 2);
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int t = TPT * st_t + u;
      const uint32_t tr = (uint32_t)(t < nvalid ? t : nvalid - 1) * Hu;  // token row offset
      const uint32_t ob = tr * (R * N * 2) + 16 * st_c, ox = tr * (R * P * 2);
#pragma unroll
      for (int r = 0; r < R; ++r) rB[u][r] = *(const uint4*)(gB + (ob + r * N * 2));
#pragma unroll
      for (int k = 0; k < XIT; ++k) {
        const int i = st_c + CH * k;  // piece i: rank i / 8, 16-byte column i % 8
        rX[u][k] = *(const uint4*)(gX + (ox + (i >> 3) * P * 2 + 16 * (i & 7)));
      }
    }
  };
  auto load_scal = [&](int64_t c0) __attribute__((always_inline)) {
    const int nvalid = (int)((t1 - c0) < QS ? (t1 - c0) : QS);
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int t = TPT * st_t + u;
      const bool tv = t < nvalid;
      const uint32_t tr = (uint32_t)(tv ? t : nvalid - 1) * Hu;
      rTh[u] = *(const float4*)(rowp(a.theta, c0, K * 4) + (tr * (K * 4) + 16 * st_c));
      const float d = *(const float*)(rowp(a.dt, c0, 4) + tr * 4);
      const float av = *(const float*)(rowp(a.A, c0, 4) + tr * 4);
      const float l = *(const float*)(rowp(a.lam, c0, 4) + tr * 4);
      rdt[u] = tv ? d : 0.0f;
      rA[u] = tv ? av : 0.0f;
      rlam[u] = tv ? l : 0.0f;
      // the following token (its epsilon weights this token's input in the state)
      const bool tv1 = c0 + t + 1 < t1;
      const uint32_t tr1 = tv1 ? tr + Hu : tr;
      const float d1 = *(const float*)(rowp(a.dt, c0, 4) + tr1 * 4);
      const float l1 = *(const float*)(rowp(a.lam, c0, 4) + tr1 * 4);
      rdt1[u] = tv1 ? d1 : 0.0f;
      rlam1[u] = tv1 ? l1 : 0.0f;
    }
  };

  auto load_C = [&](int64_t c0) __attribute__((always_inline)) {
    const int nvalid = (int)((t1 - c0) < QS ? (t1 - c0) : QS);
    const unsigned char* gC = rowp(a.C, c0, R * N * 2);
#pragma unroll
    for (int ci = 0; ci < NCW; ++ci) {
      const int v = ctl[ci] * 16 + m16;
      const int t = (v >> lgR) < nvalid ? (v >> lgR) : nvalid - 1;
      const uint32_t oc = (uint32_t)t * Hu * (R * N * 2) + (v & (R - 1)) * N * 2 + 16 * g;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) rC[ci][ks] = *(const uint4*)(gC + (oc + ks * 64));
    }
  };

  // wave-level inclusive scans over this wave's token slots (lanes CH apart;
  // a slot's TPT adjacent tokens summed in the thread first), for the
  // sub-chunk held in the prefetch registers; wave totals go to LDS
  float sc_l[TPT], sc_p[TPT][4];
  auto local_scan = [&]() __attribute__((always_inline)) {
    float e[TPT][5];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      e[u][0] = rdt[u] * rA[u];
      e[u][1] = rdt[u] * rTh[u].x;
      e[u][2] = rdt[u] * rTh[u].y;
      e[u][3] = rdt[u] * rTh[u].z;
      e[u][4] = rdt[u] * rTh[u].w;
    }
    float v[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      v[i] = e[0][i];
#pragma unroll
      for (int u = 1; u < TPT; ++u) v[i] += e[u][i];
    }
#pragma unroll
    for (int i = 0; i < 5; ++i) v[i] = slot_scan<CH>(v[i], lane);
    // inclusive values of each token of the slot: the slot's last token has v
    float w[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) w[i] = v[i];
#pragma unroll
    for (int u = TPT - 1; u >= 0; --u) {
      sc_l[u] = w[0];
#pragma unroll
      for (int j = 0; j < 4; ++j) sc_p[u][j] = w[1 + j];
#pragma unroll
      for (int i = 0; i < 5; ++i) w[i] -= e[u][i];
    }
    if (lane >= 64 - CH) {  // the wave's last token
      *(float4*)(sTot + wave * Ly::TOTW + 4 * st_c) = make_float4(v[1], v[2], v[3], v[4]);
      if (st_c == 0) sTot[wave * Ly::TOTW + K] = v[0];
    }
  };

  // ---------------- state H' (fp32 registers): n-tiles NTW*wave.., 4 p-tiles ----------------
  f32x4 hst[NTW][4];
  {
    const void* pB = nullptr;
    const void* px = nullptr;
    int64_t pBo = 0, pxo = 0;
    if (seg == 0) {
      if (a.prev_B) { pB = a.prev_B; px = a.prev_x; pBo = bh * (int64_t)(R * N); pxo = bh * (int64_t)(R * P); }
    } else {
      pB = a.B; px = a.x; pBo = tokS(t0 - 1) * (R * N); pxo = tokS(t0 - 1) * (R * P);
    }
    const float eps1 = (t0 < t1) ? (1.0f - a.lam[tokS(t0)]) * a.dt[tokS(t0)] : 0.0f;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int p = pt * 16 + m16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = (wave * NTW + j) * 16 + 4 * g + i;
          float v = 0.0f;
          if (seg == 0 && a.h0) v = a.h0[bh * (int64_t)(N * P) + n * P + p];
          if (pB) {
            float acc = 0.0f;
            for (int r = 0; r < R; ++r)
              acc += bf2f(((const u16*)pB)[pBo + r * N + n]) * bf2f(((const u16*)px)[pxo + r * P + p]);
            v += eps1 * acc;
          }
          hst[j][pt][i] = v;
        }
      }
  }

  float segLam = 0.0f, segPhi[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float sub_lend = 0.0f;  // log-decay total of the current sub-chunk

  if (t0 < t1) {
    load_scal(t0);
    load_BX(t0);
    load_C(t0);
    local_scan();
  }

  for (int64_t c0 = t0; c0 < t1; c0 += QS) {
    {
      int id = tid;
      asm volatile("" : "+v"(id));
      coords(id);
    }
    const int nvalid = (int)((t1 - c0) < QS ? (t1 - c0) : QS);
    const int fm = fsw<BCPR>(m16);  // swizzle of the rows m16 (+ multiples of 16) of B~ and H'^T tiles
    const bool meta = S > 1 && seg > 0 && kin == 0;  // a requested chunk starts here (segments start at one)
    __syncthreads();  // wave totals are in LDS; the previous sub-chunk's LDS reads are done

    // H'^T (bf16) for the inter-chunk output: row p = 16 pt + m16, columns n = 16 nt + 4g ..
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int nt = wave * NTW + j;
      unsigned char* hw = sH + m16 * Ly::HROW + (((2 * nt + (g >> 1)) ^ fm) << 4) + 8 * (g & 1);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
        *(uint2*)(hw + pt * 16 * Ly::HROW) =
            make_uint2(pack_bf2(hst[j][pt][0], hst[j][pt][1]), pack_bf2(hst[j][pt][2], hst[j][pt][3]));
    }

    // Wave priorities: the two blocks of a compute unit share its SIMDs; a
    // wave in the matrix phases (C~, outputs, state) issues first, one in
    // staging next, then the rest.  Measured: 4 % faster at R = 4, 6 % at R = 1.
    __builtin_amdgcn_s_setprio(1);
    // ---------- staging ----------
    {
      // prefix over the lower waves (uniform loop) and the sub-chunk's log-decay total
      float lpre = 0.0f, ppre[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int w2 = 0; w2 < wave; ++w2) {
        const float4 pv = *(const float4*)(sTot + w2 * Ly::TOTW + 4 * st_c);
        lpre += sTot[w2 * Ly::TOTW + K];
        ppre[0] += pv.x;
        ppre[1] += pv.y;
        ppre[2] += pv.z;
        ppre[3] += pv.w;
      }
      const float ltot = sTot[K] + sTot[Ly::TOTW + K] + sTot[2 * Ly::TOTW + K] + sTot[3 * Ly::TOTW + K];
      sub_lend = ltot;
      float wt[TPT], cs[TPT][4], sn[TPT][4];
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int t = TPT * st_t + u;
        const float lam_c = sc_l[u] + lpre;  // Lambda_t, inclusive, from the sub-chunk start
        const float gam = rlam[u] * rdt[u];
        const float q = gam + (1.0f - rlam1[u]) * rdt1[u];  // gamma_t + epsilon_{t+1}
        const float l2 = lam_c * LOG2E;
        wt[u] = __builtin_amdgcn_exp2f((ltot - lam_c) * LOG2E) * q;
        if (st_c == 0) sSC[t] = make_float4(l2, q, gam, __builtin_amdgcn_exp2f(l2));
      }
      // R >= 2: the next sub-chunk's scalars, B and x are requested as soon as
      // this staging has read their registers (measured: slower for R = 1)
      if constexpr (R >= 2)
        if (c0 + QS < t1) load_scal(c0 + QS);
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        uint32_t tab[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sincos_rev(sc_p[u][j] + ppre[j], &sn[u][j], &cs[u][j]);
          tab[j] = pack_bf2(cs[u][j], sn[u][j]);
        }
        *(uint4*)(sCS + swz<BCPR>(TPT * st_t + u, st_c)) = make_uint4(tab[0], tab[1], tab[2], tab[3]);
      }
      if (S > 1) {  // segment-relative offsets at requested chunk starts, for the fix-up pass
        if (meta && tid == 0) a.chunk_meta[meta_at] = segLam;
        segLam += ltot;
      }
      if (st_t == QS / TPT - 1) {  // last token: the sub-chunk's total angles
        float ptot[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ptot[j] = sc_p[TPT - 1][j] + ppre[j];
        if (S > 1) {
          if (meta) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              a.chunk_meta[meta_at + 1 + 4 * st_c + j] = segPhi[j];
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) segPhi[j] += ptot[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // rotation by the total angle, for the state pass
          float s2, c2;
          sincos_rev(ptot[j], &s2, &c2);
          sTh[4 * st_c + j] = make_float2(c2, s2);
        }
      }
      // B~ = R(-phi) B for every rank; w B~ kept in fp32 for the hi/lo split
      // (column u R + r: rank r of the slot's token u)
      float wb[RC][8];
#pragma unroll
      for (int u = 0; u < TPT; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t w4[4] = {rB[u][r].x, rB[u][r].y, rB[u][r].z, rB[u][r].w};
          float bt[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float bu = bf_lo(w4[j]), bw = bf_hi(w4[j]);
            bt[2 * j] = cs[u][j] * bu + sn[u][j] * bw;
            bt[2 * j + 1] = cs[u][j] * bw - sn[u][j] * bu;
          }
          *(uint4*)(sB + swz<BCPR>(RC * st_t + u * R + r, st_c)) =
              make_uint4(pack_bf2(bt[0], bt[1]), pack_bf2(bt[2], bt[3]), pack_bf2(bt[4], bt[5]), pack_bf2(bt[6], bt[7]));
#pragma unroll
          for (int e = 0; e < 8; ++e) wb[u * R + r][e] = wt[u] * bt[e];
        }
#pragma unroll
      for (int u = 0; u < TPT; ++u)
#pragma unroll
        for (int k = 0; k < XIT; ++k) {
          const int i = st_c + CH * k;
          *(uint4*)(sX + (RC * st_t + u * R + (i >> 3)) * Ly::XP + 16 * (i & 7)) =
              make_uint4(rX[u][k].x, rX[u][k].y, rX[u][k].z, rX[u][k].w);
        }
      if constexpr (R >= 2)
        if (c0 + QS < t1) load_BX(c0 + QS);
      // (w B~)^T: row n = 8 st_c + e, columns (token, rank): the R ranks of token t are adjacent.
      // lo = w B~ - hi comes from one dot product per element: hi . (-1, 0) + w B~.
      {
        const int byte = 2 * RC * st_t;
        const int cb = byte >> 4;
        int z0 = (cb ^ fW<Ly::WCPR>(8 * st_c)) << 4, z1 = (cb ^ fW<Ly::WCPR>(8 * st_c + 4)) << 4;
        asm volatile("" : "+v"(z0), "+v"(z1));  // keeps (z ^ 16k) + base as one xor-add per row
        const int base = 8 * st_c * Ly::WROW + (byte & 15);
        // (-1, 0) and (0, -1) as bf16 pairs, held in scalar registers: as an inline
        // constant the compiler would encode (-1, 0) as -1.0, which this operand
        // reads as the fp32 bit pattern, i.e. (0, -1) (measured)
        uint32_t nlo_b = 0x0000bf80u, nhi_b = 0xbf800000u;
        asm volatile("" : "+s"(nlo_b), "+s"(nhi_b));
        const bf16x2 nlo = __builtin_bit_cast(bf16x2, nlo_b), nhi = __builtin_bit_cast(bf16x2, nhi_b);
        auto lo2 = [&](uint32_t hw, float w0, float w1) __attribute__((always_inline)) {
          const bf16x2 hv = __builtin_bit_cast(bf16x2, hw);
          return pack_bf2(__builtin_amdgcn_fdot2_f32_bf16(hv, nlo, w0, false),
                          __builtin_amdgcn_fdot2_f32_bf16(hv, nhi, w1, false));
        };
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int off = (((e < 4 ? z0 : z1) ^ (16 * (e & 3))) + base) + e * Ly::WROW;
          if constexpr (RC == 4) {
            const uint32_t h01 = pack_bf2(wb[0][e], wb[1][e]), h23 = pack_bf2(wb[2][e], wb[3][e]);
            *(uint2*)(sWh + off) = make_uint2(h01, h23);
            *(uint2*)(sWl + off) = make_uint2(lo2(h01, wb[0][e], wb[1][e]), lo2(h23, wb[2][e], wb[3][e]));
          } else if constexpr (RC == 2) {
            const uint32_t h01 = pack_bf2(wb[0][e], wb[1][e]);
            *(uint32_t*)(sWh + off) = h01;
            *(uint32_t*)(sWl + off) = lo2(h01, wb[0][e], wb[1][e]);
          } else {
            const uint32_t h0 = pack_bf2(wb[0][e], 0.0f);
            *(u16*)(sWh + off) = (u16)(h0 & 0xffffu);
            *(u16*)(sWl + off) = (u16)(lo2(h0, wb[0][e], 0.0f) & 0xffffu);
          }
        }
      }
    }
    __syncthreads();  // B~, X, (w B~)^T, H'^T, the cos/sin table and the scalars are in LDS
    __builtin_amdgcn_s_setprio(2);
    const bool more = c0 + QS < t1;
    if constexpr (R == 1) {
      if (more) {
        load_scal(c0 + QS);
        load_BX(c0 + QS);
      }
    }

    // own C~ fragments (operand layout: row v = tile*16 + m16, n = ks*32 + 8g + j)
    uint4 rCt[NCW][NKS];
#pragma unroll
    for (int ci = 0; ci < NCW; ++ci) {
      const int t = (ctl[ci] * 16 + m16) >> lgR;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 tb = *(const uint4*)(sCS + swz<BCPR>(t, 4 * ks + g));
        const uint32_t tw[4] = {tb.x, tb.y, tb.z, tb.w};
        const uint32_t cw[4] = {rC[ci][ks].x, rC[ci][ks].y, rC[ci][ks].z, rC[ci][ks].w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // R(-phi)(u, w) = ((u, w).(cos, sin), (w, u).(cos, -sin)), bf16 pairs, fp32 sums
          const float o0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, cw[j]),
                                                           __builtin_bit_cast(bf16x2, tw[j]), 0.0f, false);
          o[j] = pack_bf2(o0, dot2_bf16_neghi(__builtin_amdgcn_alignbit(cw[j], cw[j], 16), tw[j]));
        }
        rCt[ci][ks] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    if (more) load_C(c0 + QS);

    // ---------- outputs: Y^T = exp(Lam_t) H'^T C~^T + X^T (G o M)^T ----------
    {
      // per-lane bases: the 16-row tiles of B~ and H'^T at n column 32 ks + 8g;
      // the X^T transpose reads at rows 4g + jj and p = pt0*16 + 4uu
      const unsigned char* bB[NKS];
      const unsigned char* bH[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        bB[ks] = sB + m16 * Ly::BROW + (((4 * ks + g) ^ fm) << 4);
        bH[ks] = sH + m16 * Ly::HROW + (((4 * ks + g) ^ fm) << 4);
      }
      const unsigned char* bXt = sX + (4 * g + jj) * Ly::XP + 2 * (pt0 * 16 + 4 * uu);

      f32x4 yacc[NCW][PTW];
      int tcol[NCW];
      float Lt[NCW], gt[NCW];
#pragma unroll
      for (int ci = 0; ci < NCW; ++ci) {
        tcol[ci] = (ctl[ci] * 16 + m16) >> lgR;
        const float4 sc = sSC[tcol[ci]];
        Lt[ci] = sc.x;
        gt[ci] = sc.z;
#pragma unroll
        for (int pp = 0; pp < PTW; ++pp) {
          f32x4 acc = {0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const uint4 hf = *(const uint4*)(bH[ks] + (pt0 + pp) * 16 * Ly::HROW);
            acc = mfma_bf16(as_bf16x8(hf), as_bf16x8(rCt[ci][ks]), acc);
          }
          yacc[ci][pp] = acc * sc.w;
        }
      }
      // shared loop over 32-row source slabs; tile 0 has the larger causal range
      const int nkb0 = ((ctl[0] + 1) * 16 + 31) / 32;
      const int nkb1 = NCW == 2 ? ((ctl[NCW - 1] + 1) * 16 + 31) / 32 : 0;
      for (int kb = 0; kb < nkb0; ++kb) {
        uint4 bfr[2][NKS];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            bfr[sub][ks] = *(const uint4*)(bB[ks] + (kb * 32 + sub * 16) * Ly::BROW);
        const float2* scs = (const float2*)(sSC + kb * 8 + g);  // (log2 decay, q) of the lane's source token (R = 4)
        // X^T fragments of the slab in the score operand's k order (rows 4g..
        // and 16 + 4g..), shared by the wave's column tiles
        uint4 xf[PTW];
        {
          const unsigned char* xk = bXt + kb * 32 * Ly::XP;
#pragma unroll
          for (int pp = 0; pp < PTW; ++pp) {
            const uint2 f0 = lds_tr16(xk + pp * 32);
            const uint2 f1 = lds_tr16(xk + 16 * Ly::XP + pp * 32);
            xf[pp] = make_uint4(f0.x, f0.y, f1.x, f1.y);
          }
        }
#pragma unroll
        for (int ci = 0; ci < NCW; ++ci) {
          if (ci == 1 && kb >= nkb1) continue;
          float gm[2][4];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) acc = mfma_bf16(as_bf16x8(bfr[sub][ks]), as_bf16x8(rCt[ci][ks]), acc);
            // s < t: decay * q_s;  s == t: gamma_t;  else 0 (selected arithmetically)
            if constexpr (R == 4) {
              const int s = kb * 8 + sub * 4 + g;
              const float2 lq = scs[sub * 8];
              const float e = __builtin_amdgcn_exp2f(fminf(Lt[ci] - lq.x, 0.0f)) * lq.y;
              const float m = ((s < tcol[ci]) ? 1.0f : 0.0f) * e + ((s == tcol[ci]) ? gt[ci] : 0.0f);
#pragma unroll
              for (int i = 0; i < 4; ++i) gm[sub][i] = acc[i] * m;
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int s = (kb * 32 + sub * 16 + 4 * g + i) >> lgR;
                const float2 lq = *(const float2*)(sSC + s);
                const float e = __builtin_amdgcn_exp2f(fminf(Lt[ci] - lq.x, 0.0f)) * lq.y;
                const float m = ((s < tcol[ci]) ? 1.0f : 0.0f) * e + ((s == tcol[ci]) ? gt[ci] : 0.0f);
                gm[sub][i] = acc[i] * m;
              }
            }
          }
          const uint4 gfr = make_uint4(pack_bf2(gm[0][0], gm[0][1]), pack_bf2(gm[0][2], gm[0][3]),
                                       pack_bf2(gm[1][0], gm[1][1]), pack_bf2(gm[1][2], gm[1][3]));
#pragma unroll
          for (int pp = 0; pp < PTW; ++pp) {
            yacc[ci][pp] = mfma_bf16(as_bf16x8(xf[pp]), as_bf16x8(gfr), yacc[ci][pp]);
          }
        }
      }
      // store y
#pragma unroll
      for (int ci = 0; ci < NCW; ++ci) {
        const int vcol = ctl[ci] * 16 + m16;
        u16* yrow = (u16*)(rowp(a.y, c0, R * P * 2) + ((uint32_t)(tcol[ci] < nvalid ? tcol[ci] : 0) * Hu * (R * P * 2) +
                                                          (vcol & (R - 1)) * P * 2));
        if constexpr (PTW == 4) {
          // transpose (16-lane row g) x (p tile) so that lane g holds p = 16g .. 16g + 15
          // of its row: 32 contiguous bytes per lane instead of four 8-byte pieces
          uint32_t d0[4], d1[4];
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            d0[pp] = pack_bf2(yacc[ci][pp][0], yacc[ci][pp][1]);
            d1[pp] = pack_bf2(yacc[ci][pp][2], yacc[ci][pp][3]);
          }
          transpose_rows4(d0);
          transpose_rows4(d1);
          if (tcol[ci] < nvalid) {
            *(uint4*)(yrow + 16 * g) = make_uint4(d0[0], d1[0], d0[1], d1[1]);
            *(uint4*)(yrow + 16 * g + 8) = make_uint4(d0[2], d1[2], d0[3], d1[3]);
          }
        } else if (tcol[ci] < nvalid) {
#pragma unroll
          for (int pp = 0; pp < PTW; ++pp)
            *(uint2*)(yrow + (pt0 + pp) * 16 + 4 * g) = make_uint2(pack_bf2(yacc[ci][pp][0], yacc[ci][pp][1]),
                                                                   pack_bf2(yacc[ci][pp][2], yacc[ci][pp][3]));
        }
      }
    }

    // ---------- sub-chunk state S = (w B~)^T X (hi + lo) and the state pass ----------
    {
      f32x4 sacc[NTW][4];
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) sacc[j][pt] = f32x4{0, 0, 0, 0};
      const unsigned char* bXs = sX + (8 * g + jj) * Ly::XP + 8 * uu;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        uint4 xb[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const uint2 f0 = lds_tr16(bXs + kb * 32 * Ly::XP + pt * 32);
          const uint2 f1 = lds_tr16(bXs + (kb * 32 + 4) * Ly::XP + pt * 32);
          xb[pt] = make_uint4(f0.x, f0.y, f1.x, f1.y);
        }
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const int n = (wave * NTW + j) * 16 + m16;
          const int wo = ((4 * kb) ^ g ^ fW<Ly::WCPR>(n)) << 4;
          const unsigned char* bW = sWh + n * Ly::WROW + wo;
          const uint4 ah = *(const uint4*)bW;
          const uint4 al = *(const uint4*)(bW + (Ly::OFF_WL - Ly::OFF_WH));
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            sacc[j][pt] = mfma_bf16(as_bf16x8(ah), as_bf16x8(xb[pt]), sacc[j][pt]);
            sacc[j][pt] = mfma_bf16(as_bf16x8(al), as_bf16x8(xb[pt]), sacc[j][pt]);
          }
        }
      }
      const float eLend = __builtin_amdgcn_exp2f(sub_lend * LOG2E);
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float2 cs = sTh[(wave * NTW + j) * 8 + 2 * g + q];
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            const float u = eLend * hst[j][pt][2 * q] + sacc[j][pt][2 * q];
            const float w = eLend * hst[j][pt][2 * q + 1] + sacc[j][pt][2 * q + 1];
            hst[j][pt][2 * q] = cs.x * u - cs.y * w;
            hst[j][pt][2 * q + 1] = cs.y * u + cs.x * w;
          }
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if (more) local_scan();
    if (++kin == spc) {
      kin = 0;
      meta_at += 1 + K;
    }
  }

  // ---------------- epilogue ----------------
  float* dst = (S == 1) ? a.h_final : a.seg_end + blk * (int64_t)(N * P);
  if (dst) {
    float* base = (S == 1 ? dst + bh * (int64_t)(N * P) : dst);
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          base[((wave * NTW + j) * 16 + 4 * g + i) * P + pt * 16 + m16] = hst[j][pt][i];
  }
  if (S > 1) {
    float* tot = a.seg_tot + blk * (1 + K);
    if (tid == 0) tot[0] = segLam;
    if (st_t == QS / TPT - 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) tot[1 + 4 * st_c + j] = segPhi[j];
    }
  }
}

template <int N, int R>
static hipError_t sw_run(const WalkArgs& a, hipStream_t s) {
  // LDS is static (SW<N, R>::BYTES per head).  R = 1: two adjacent heads per
  // block when B*H is even (the pair shares its segment bounds)
  const int64_t BH = a.batch * a.H;
  if constexpr (R == 1) {
    if (BH % 2 == 0) {
      hipLaunchKernelGGL((subchunk_walk_kernel<N, R, 2>), dim3((unsigned)(BH / 2 * a.S)), dim3(512), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((subchunk_walk_kernel<N, R, 1>), dim3((unsigned)(BH * a.S)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_subwalk(int N, const WalkArgs& a, hipStream_t s) {
  if (N == 64) {
    if (a.Q % SW<64, 1>::QS != 0 && !(a.R > 1 && a.Q % SW<64, 2>::QS == 0)) return hipErrorInvalidValue;
    switch (a.R) {
      case 1: return sw_run<64, 1>(a, s);
      case 2: return sw_run<64, 2>(a, s);
      case 4: return sw_run<64, 4>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (N == 128) {
    if (a.Q % SW<128, 2>::QS != 0) return hipErrorInvalidValue;
    switch (a.R) {
      case 2: return sw_run<128, 2>(a, s);
      case 4: return sw_run<128, 4>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace m3
