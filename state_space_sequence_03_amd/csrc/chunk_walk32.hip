// Prefill walker for bf16 io with N = P = 64 (the 1.5B-scale head shapes):
// 32-token sub-chunks, two blocks per compute unit.
//
// Computes what the other walkers compute (chunk.hip, chunk_fast.hip): the
// chunked form of the exponential-trapezoidal recurrence with data-dependent
// RoPE and rank-R inputs (linkstar.cloud/article/869, "第一刀", "第二刀",
// "第三刀"; yetianai.com/news/16273, "榨干硬件算力").  A requested chunk of 32
// or 64 tokens is walked as 32-token sub-chunks: the chunked form holds for
// any split of the sequence, because the state carried across a boundary is
// the exact state there.
//
// gfx950 data flow:
//  * 256 threads and under 80 KB of LDS per block, so two blocks (two (b,h)
//    sequences) share a compute unit and one block's staging and loads overlap
//    the other block's matrix work.
//  * Coalesced loads.  Staging thread (t, c) owns token t of the sub-chunk and
//    the 16-byte column c of each rank row of B and x and of theta's row, so a
//    wave instruction reads whole 128-byte rows.  Each wave keeps the C rows
//    of its own output tiles in the MFMA operand layout (16 bytes per lane).
//  * Cumulative log-decay and angles: wave scans over the 8 tokens a wave
//    holds, plus an exchange of wave totals through LDS.  The wave scans of
//    the next sub-chunk run at the end of the current one, so the exchange
//    shares the sub-chunk's first barrier.
//  * sin/cos are computed once per (token, pair) by the staging thread, which
//    rotates all R ranks of B with them and stores them as a bf16 table for
//    the rotation of C: two bf16 dot products per pair (fp32 sums), the result
//    rounded to bf16 like every MFMA operand.
//  * y leaves the wave as 32 contiguous bytes per lane after a 4 x 4 transpose
//    across the wave's 16-lane rows.
//  * LDS arrays keep their natural row layout with the 16-byte columns
//    XOR-swizzled per row, so the 16-byte operand reads and the transpose
//    reads (ds_read_b64_tr_b16) of 16 lanes fall in distinct banks.
//  * Two barriers per sub-chunk: after the previous sub-chunk's last LDS read
//    (and the scan exchange), and after staging.
//
// Precision matches the other bf16 walkers: bf16 MFMA operands with fp32
// accumulation; the chunk state uses w B~ split into bf16 hi + lo parts.
#include "m3_common.hpp"
#include "m3_launch.hpp"

namespace m3 {

namespace {

constexpr int W32_QS = 32;  // tokens per sub-chunk

template <int R>
struct W32 {
  static constexpr int N = 64, P = 64, K = 32, QS = W32_QS, V = QS * R;
  static constexpr int XP = 144;          // bytes per X row (128 + 16: transpose reads of 4 rows hit distinct banks)
  static constexpr int WROW = 2 * V;      // bytes per row of (w B~)^T
  static constexpr int WCPR = WROW / 16;  // 16-byte columns per row of (w B~)^T
  static constexpr int OFF_B = 0;                       // B~   [V][64] bf16, swizzled
  static constexpr int OFF_X = OFF_B + V * 128;         // X    [V][64] bf16, padded rows
  static constexpr int OFF_WH = OFF_X + V * XP;         // (w B~)^T hi [64][V] bf16, swizzled
  static constexpr int OFF_WL = OFF_WH + N * WROW;      // (w B~)^T lo
  static constexpr int OFF_H = OFF_WL + N * WROW;       // H'^T [64][64] bf16, swizzled
  static constexpr int OFF_CS = OFF_H + P * 128;        // (cos, sin) [QS][K] bf16 pairs, swizzled
  static constexpr int OFF_SC = OFF_CS + QS * 128;      // per token: log2 decay, q, gamma, exp(decay)
  static constexpr int OFF_TOT = OFF_SC + QS * 16;      // wave totals [4][36] fp32
  static constexpr int OFF_TH = OFF_TOT + 4 * 36 * 4;   // chunk-total rotation [K] float2
  static constexpr int BYTES = OFF_TH + K * 8;
};
static_assert(W32<4>::BYTES <= 80 * 1024, "two blocks per compute unit");

// Swizzle of an array of 128-byte rows: 16-byte column c of row r is stored
// at column c ^ f(r).  f depends only on r mod 16, so the rows of a 16-row
// tile, at any tile offset, share one pattern, and 16 consecutive rows read
// at one logical column fall in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int f16rows(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int sw128(int row, int chunk) { return row * 128 + ((chunk ^ f16rows(row)) << 4); }
// rows of (w B~)^T (WCPR 16-byte columns): 16 consecutive rows, and the 8
// rows 8 apart that one staging instruction writes, both spread over banks
template <int WCPR>
__device__ __forceinline__ int fW(int n) {
  return WCPR == 4 ? ((n ^ (n >> 2)) & 3) : ((n ^ (n >> 3)) & (WCPR - 1));
}

// d[k] of 16-lane row r becomes d[r] of row k: a 4 x 4 transpose of (row of
// the wave) x (register) with the gfx950 row swaps (permlane32_swap exchanges
// rows 2,3 of its first operand with rows 0,1 of its second; permlane16_swap
// the odd rows of the first with the even rows of the second)
__device__ __forceinline__ void transpose_rows4(uint32_t* d) {
  auto s = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
  d[0] = s[0];
  d[2] = s[1];
  s = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
  d[1] = s[0];
  d[3] = s[1];
  s = __builtin_amdgcn_permlane16_swap(d[0], d[1], false, false);
  d[0] = s[0];
  d[1] = s[1];
  s = __builtin_amdgcn_permlane16_swap(d[2], d[3], false, false);
  d[2] = s[0];
  d[3] = s[1];
}

}  // namespace

bool walk32_supported(int io_bf16, int N, int P, int Q, int R) {
  return io_bf16 && N == 64 && P == 64 && (Q == 32 || Q == 64) && (R == 1 || R == 2 || R == 4);
}

int walk_chunk(int io_bf16, int N, int P, int Q, int R) {
  return walk32_supported(io_bf16, N, P, Q, R) ? W32_QS : Q;
}

template <int R>
__global__ __launch_bounds__(256, 2) void walk32_kernel(WalkArgs a) {
  typedef W32<R> Ly;
  constexpr int N = 64, P = 64, K = 32, QS = W32_QS, V = Ly::V, NW = 4;
  constexpr int lgR = R == 4 ? 2 : (R == 2 ? 1 : 0);
  constexpr int NCT = V / 16;               // column tiles of Y (16 virtual rows each)
  constexpr int NCW = NCT == 8 ? 2 : 1;     // column tiles per wave
  constexpr int PTW = NCT >= 4 ? 4 : 2;     // 16-wide p tiles per wave
  constexpr int NKB = V / 32;               // 32-row slabs of the sub-chunk
  constexpr float LOG2E = 1.4426950408889634f;

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* sB = smem + Ly::OFF_B;
  unsigned char* sX = smem + Ly::OFF_X;
  unsigned char* sWh = smem + Ly::OFF_WH;
  unsigned char* sWl = smem + Ly::OFF_WL;
  unsigned char* sH = smem + Ly::OFF_H;
  unsigned char* sCS = smem + Ly::OFF_CS;
  float4* sSC = (float4*)(smem + Ly::OFF_SC);  // per token: log2 decay, q, gamma, exp(decay)
  float* sTot = (float*)(smem + Ly::OFF_TOT);  // per wave: 32 angle totals, log-decay total
  float2* sTh = (float2*)(smem + Ly::OFF_TH);

  const int wave = threadIdx.x >> 6;
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
    st_t = id >> 3;         // staging: token, 16-byte column
    st_c = id & 7;
  };
  coords(threadIdx.x);

  const int64_t S = a.S;
  const int64_t blk = blockIdx.x;
  const int64_t seg = blk % S, bh = blk / S;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t L = a.L, H = a.H;
  const int64_t t0 = seg * a.seg_len;
  const int64_t t1 = (t0 + a.seg_len < L) ? t0 + a.seg_len : L;
  auto tokBC = [&](int64_t tok) { return ((b * L + tok) * H + h) * (int64_t)(R * N); };
  auto tokX = [&](int64_t tok) { return ((b * L + tok) * H + h) * (int64_t)(R * P); };
  auto tokS = [&](int64_t tok) { return (b * L + tok) * H + h; };
  const int64_t nchunks_total = (L + QS - 1) / QS;

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
  uint4 rB[R], rX[R];
  float4 rTh;
  float rdt, rA, rlam, rdt1, rlam1;
  uint4 rC[NCW][2];

  // Tokens past the end of the segment read the last valid token instead: only
  // their dt, lam (hence q = gamma = 0) are zeroed, which removes them exactly
  // from the scores, the outputs and the state while every operand stays finite.
  auto load_BX = [&](int64_t c0) __attribute__((always_inline)) {
    const int nvalid = (int)((t1 - c0) < QS ? (t1 - c0) : QS);
    const int64_t row = tokS(c0 + (st_t < nvalid ? st_t : nvalid - 1));
    const u16* gB = (const u16*)a.B + row * (R * N) + 8 * st_c;
    const u16* gX = (const u16*)a.x + row * (R * P) + 8 * st_c;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      rB[r] = *(const uint4*)(gB + r * N);
      rX[r] = *(const uint4*)(gX + r * P);
    }
  };
  auto load_scal = [&](int64_t c0) __attribute__((always_inline)) {
    const int nvalid = (int)((t1 - c0) < QS ? (t1 - c0) : QS);
    const bool tv = st_t < nvalid;
    const int64_t ts = tokS(c0 + (tv ? st_t : nvalid - 1));
    rTh = *(const float4*)(a.theta + ts * K + 4 * st_c);
    const float d = a.dt[ts], av = a.A[ts], l = a.lam[ts];
    rdt = tv ? d : 0.0f;
    rA = tv ? av : 0.0f;
    rlam = tv ? l : 0.0f;
    // the following token (its epsilon weights this token's input in the state)
    const bool tv1 = c0 + st_t + 1 < t1;
    const int64_t ts1 = tv1 ? ts + H : ts;
    const float d1 = a.dt[ts1], l1 = a.lam[ts1];
    rdt1 = tv1 ? d1 : 0.0f;
    rlam1 = tv1 ? l1 : 0.0f;
  };

  auto load_C = [&](int64_t c0) __attribute__((always_inline)) {
    const int nvalid = (int)((t1 - c0) < QS ? (t1 - c0) : QS);
#pragma unroll
    for (int ci = 0; ci < NCW; ++ci) {
      const int v = ctl[ci] * 16 + m16;
      const int t = (v >> lgR) < nvalid ? (v >> lgR) : nvalid - 1;
      const u16* row = (const u16*)a.C + tokS(c0 + t) * (R * N) + (v & (R - 1)) * N + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) rC[ci][ks] = *(const uint4*)(row + ks * 32);
    }
  };

  // wave-level inclusive scans over this wave's 8 tokens (lanes 8 apart), for
  // the sub-chunk held in the prefetch registers; wave totals go to LDS
  float sc_l, sc_p[4];
  auto local_scan = [&]() __attribute__((always_inline)) {
    float v[5] = {rdt * rA, rdt * rTh.x, rdt * rTh.y, rdt * rTh.z, rdt * rTh.w};
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) {
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const float u = __shfl_up(v[i], o, 64);
        if (lane >= o) v[i] += u;
      }
    }
    sc_l = v[0];
#pragma unroll
    for (int j = 0; j < 4; ++j) sc_p[j] = v[1 + j];
    if (lane >= 56) {
      *(float4*)(sTot + wave * 36 + 4 * st_c) = make_float4(v[1], v[2], v[3], v[4]);
      if (st_c == 0) sTot[wave * 36 + 32] = v[0];
    }
  };

  // ---------------- state H' (fp32 registers): n-tile = wave, 4 p-tiles ----------------
  f32x4 hst[4];
  {
    const void* pB = nullptr;
    const void* px = nullptr;
    int64_t pBo = 0, pxo = 0;
    if (seg == 0) {
      if (a.prev_B) { pB = a.prev_B; px = a.prev_x; pBo = bh * (int64_t)(R * N); pxo = bh * (int64_t)(R * P); }
    } else {
      pB = a.B; px = a.x; pBo = tokBC(t0 - 1); pxo = tokX(t0 - 1);
    }
    const float eps1 = (t0 < t1) ? (1.0f - a.lam[tokS(t0)]) * a.dt[tokS(t0)] : 0.0f;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int p = pt * 16 + m16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = wave * 16 + 4 * g + i;
        float v = 0.0f;
        if (seg == 0 && a.h0) v = a.h0[bh * (int64_t)(N * P) + n * P + p];
        if (pB) {
          float acc = 0.0f;
          for (int r = 0; r < R; ++r)
            acc += bf2f(((const u16*)pB)[pBo + r * N + n]) * bf2f(((const u16*)px)[pxo + r * P + p]);
          v += eps1 * acc;
        }
        hst[pt][i] = v;
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
    const int fm = f16rows(m16);  // swizzle of the rows m16 (+ multiples of 16) of a tile
    __syncthreads();  // wave totals are in LDS; the previous sub-chunk's LDS reads are done

    // H'^T (bf16) for the inter-chunk output: row p = 16 pt + m16, columns n = 16 wave + 4g ..
    {
      unsigned char* hw = sH + m16 * 128 + (((2 * wave + (g >> 1)) ^ fm) << 4) + 8 * (g & 1);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
        *(uint2*)(hw + pt * 2048) = make_uint2(pack_bf2(hst[pt][0], hst[pt][1]), pack_bf2(hst[pt][2], hst[pt][3]));
    }

    // ---------- staging ----------
    {
      // prefix over the lower waves (uniform loop) and the sub-chunk's log-decay total
      float lpre = 0.0f, ppre[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int w2 = 0; w2 < wave; ++w2) {
        const float4 pv = *(const float4*)(sTot + w2 * 36 + 4 * st_c);
        lpre += sTot[w2 * 36 + 32];
        ppre[0] += pv.x;
        ppre[1] += pv.y;
        ppre[2] += pv.z;
        ppre[3] += pv.w;
      }
      const float ltot = sTot[32] + sTot[36 + 32] + sTot[72 + 32] + sTot[108 + 32];
      sub_lend = ltot;
      const float lam_c = sc_l + lpre;  // Lambda_t, inclusive, from the sub-chunk start
      const float gam = rlam * rdt;
      const float q = gam + (1.0f - rlam1) * rdt1;  // gamma_t + epsilon_{t+1}
      const float l2 = lam_c * LOG2E;
      const float wt = __builtin_amdgcn_exp2f((ltot - lam_c) * LOG2E) * q;
      // R >= 2: the next sub-chunk's scalars, B and x are requested as soon as
      // this staging has read their registers (measured: slower for R = 1)
      if constexpr (R >= 2)
        if (c0 + QS < t1) load_scal(c0 + QS);
      if (st_c == 0) sSC[st_t] = make_float4(l2, q, gam, __builtin_amdgcn_exp2f(l2));
      if (S > 1) {  // segment-relative offsets of this sub-chunk, for the fix-up pass
        if (seg > 0 && tid == 0) a.chunk_meta[(bh * nchunks_total + c0 / QS) * (1 + K)] = segLam;
        segLam += ltot;
      }
      if (st_t == QS - 1) {  // last token: the sub-chunk's total angles
        float ptot[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ptot[j] = sc_p[j] + ppre[j];
        if (S > 1) {
          if (seg > 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              a.chunk_meta[(bh * nchunks_total + c0 / QS) * (1 + K) + 1 + 4 * st_c + j] = segPhi[j];
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) segPhi[j] += ptot[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // rotation by the total angle, for the state pass
          float s2, c2;
          fast_sincos(ptot[j], &s2, &c2);
          sTh[4 * st_c + j] = make_float2(c2, s2);
        }
      }
      float cs[4], sn[4];
      uint32_t tab[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        fast_sincos(sc_p[j] + ppre[j], &sn[j], &cs[j]);
        tab[j] = pack_bf2(cs[j], sn[j]);
      }
      *(uint4*)(sCS + sw128(st_t, st_c)) = make_uint4(tab[0], tab[1], tab[2], tab[3]);

      // B~ = R(-phi) B for every rank; w B~ kept in fp32 for the hi/lo split
      float wb[R][8];
      unsigned char* xw = sX + R * st_t * Ly::XP + 16 * st_c;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t w4[4] = {rB[r].x, rB[r].y, rB[r].z, rB[r].w};
        float bt[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float u = bf_lo(w4[j]), w = bf_hi(w4[j]);
          bt[2 * j] = cs[j] * u + sn[j] * w;
          bt[2 * j + 1] = cs[j] * w - sn[j] * u;
        }
        *(uint4*)(sB + sw128(R * st_t + r, st_c)) =
            make_uint4(pack_bf2(bt[0], bt[1]), pack_bf2(bt[2], bt[3]), pack_bf2(bt[4], bt[5]), pack_bf2(bt[6], bt[7]));
#pragma unroll
        for (int e = 0; e < 8; ++e) wb[r][e] = wt * bt[e];
        *(uint4*)(xw + r * Ly::XP) = make_uint4(rX[r].x, rX[r].y, rX[r].z, rX[r].w);
      }
      if constexpr (R >= 2)
        if (c0 + QS < t1) load_BX(c0 + QS);
      // (w B~)^T: row n = 8 st_c + e, columns (token, rank): the R ranks of token t are adjacent
      {
        const int byte = 2 * R * st_t;
        const int cb = byte >> 4;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int n = 8 * st_c + e;
          const int off = n * Ly::WROW + ((cb ^ fW<Ly::WCPR>(n)) << 4) + (byte & 15);
          if constexpr (R == 4) {
            const uint32_t h01 = pack_bf2(wb[0][e], wb[1][e]), h23 = pack_bf2(wb[2][e], wb[3][e]);
            const uint32_t l01 = pack_bf2(wb[0][e] - bf_lo(h01), wb[1][e] - bf_hi(h01));
            const uint32_t l23 = pack_bf2(wb[2][e] - bf_lo(h23), wb[3][e] - bf_hi(h23));
            *(uint2*)(sWh + off) = make_uint2(h01, h23);
            *(uint2*)(sWl + off) = make_uint2(l01, l23);
          } else if constexpr (R == 2) {
            const uint32_t h01 = pack_bf2(wb[0][e], wb[1][e]);
            *(uint32_t*)(sWh + off) = h01;
            *(uint32_t*)(sWl + off) = pack_bf2(wb[0][e] - bf_lo(h01), wb[1][e] - bf_hi(h01));
          } else {
            const uint32_t h0 = pack_bf2(wb[0][e], 0.0f);
            *(u16*)(sWh + off) = (u16)(h0 & 0xffffu);
            *(u16*)(sWl + off) = (u16)(pack_bf2(wb[0][e] - bf_lo(h0), 0.0f) & 0xffffu);
          }
        }
      }
    }
    __syncthreads();  // B~, X, (w B~)^T, H'^T, the cos/sin table and the scalars are in LDS
    // next sub-chunk's loads go out as early as their registers are free: they
    // then have the whole Y and S phases to arrive
    const bool more = c0 + QS < t1;
    if constexpr (R == 1) {
      if (more) {
        load_scal(c0 + QS);
        load_BX(c0 + QS);
      }
    }

    // own C~ fragments (operand layout: row v = tile*16 + m16, n = ks*32 + 8g + j)
    uint4 rCt[NCW][2];
#pragma unroll
    for (int ci = 0; ci < NCW; ++ci) {
      const int t = (ctl[ci] * 16 + m16) >> lgR;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 tb = *(const uint4*)(sCS + sw128(t, 4 * ks + g));
        const uint32_t tw[4] = {tb.x, tb.y, tb.z, tb.w};
        const uint32_t cw[4] = {rC[ci][ks].x, rC[ci][ks].y, rC[ci][ks].z, rC[ci][ks].w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // R(-phi)(u, w) = ((u, w).(cos, sin), (u, w).(-sin, cos)), bf16 pairs, fp32 sums
          const uint32_t ms = __builtin_amdgcn_alignbit(tw[j], tw[j], 16) ^ 0x8000u;  // (-sin, cos)
          const float o0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, cw[j]),
                                                           __builtin_bit_cast(bf16x2, tw[j]), 0.0f, false);
          const float o1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, cw[j]),
                                                           __builtin_bit_cast(bf16x2, ms), 0.0f, false);
          o[j] = pack_bf2(o0, o1);
        }
        rCt[ci][ks] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }

    if (more) load_C(c0 + QS);

    // ---------- outputs: Y^T = exp(Lam_t) H'^T C~^T + X^T (G o M)^T ----------
    {
      // per-lane bases: the 16-row tiles of B~ and H'^T at n column 8g (ks = 0) and
      // 32 + 8g (ks = 1); the X^T transpose reads at rows 4g + jj and p = pt0*16 + 4uu
      const unsigned char* bB[2];
      const unsigned char* bH[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bB[ks] = sB + m16 * 128 + (((4 * ks + g) ^ fm) << 4);
        bH[ks] = sH + m16 * 128 + (((4 * ks + g) ^ fm) << 4);
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
          for (int ks = 0; ks < 2; ++ks) {
            const uint4 hf = *(const uint4*)(bH[ks] + (pt0 + pp) * 2048);
            acc = mfma_bf16(as_bf16x8(hf), as_bf16x8(rCt[ci][ks]), acc);
          }
          yacc[ci][pp] = acc * sc.w;
        }
      }
      // shared loop over 32-row source slabs; tile 0 has the larger causal range
      const int nkb0 = ((ctl[0] + 1) * 16 + 31) / 32;
      const int nkb1 = NCW == 2 ? ((ctl[NCW - 1] + 1) * 16 + 31) / 32 : 0;
      for (int kb = 0; kb < nkb0; ++kb) {
        uint4 bfr[2][2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            bfr[sub][ks] = *(const uint4*)(bB[ks] + (kb * 32 + sub * 16) * 128);
        const float2* scs = (const float2*)(sSC + kb * 8 + g);  // (log2 decay, q) of the lane's source token
#pragma unroll
        for (int ci = 0; ci < NCW; ++ci) {
          if (ci == 1 && kb >= nkb1) continue;
          float gm[2][4];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc = mfma_bf16(as_bf16x8(bfr[sub][ks]), as_bf16x8(rCt[ci][ks]), acc);
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
          // X^T fragments in the score operand's k order (rows 4g.. and 16 + 4g.. of the slab)
          const unsigned char* xk = bXt + kb * 32 * Ly::XP;
#pragma unroll
          for (int pp = 0; pp < PTW; ++pp) {
            const uint2 f0 = lds_tr16(xk + pp * 32);
            const uint2 f1 = lds_tr16(xk + 16 * Ly::XP + pp * 32);
            yacc[ci][pp] = mfma_bf16(as_bf16x8(make_uint4(f0.x, f0.y, f1.x, f1.y)), as_bf16x8(gfr), yacc[ci][pp]);
          }
        }
      }
      // store y
#pragma unroll
      for (int ci = 0; ci < NCW; ++ci) {
        const int vcol = ctl[ci] * 16 + m16;
        u16* yrow = (u16*)a.y + tokX(c0 + (tcol[ci] < nvalid ? tcol[ci] : 0)) + (vcol & (R - 1)) * P;
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
      f32x4 sacc[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) sacc[pt] = f32x4{0, 0, 0, 0};
      const int n = wave * 16 + m16;
      const int gf = g ^ fW<Ly::WCPR>(n);
      const unsigned char* bW = sWh + n * Ly::WROW;
      const unsigned char* bXs = sX + (8 * g + jj) * Ly::XP + 8 * uu;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int wo = ((4 * kb) ^ gf) << 4;
        const uint4 ah = *(const uint4*)(bW + wo);
        const uint4 al = *(const uint4*)(bW + (Ly::OFF_WL - Ly::OFF_WH) + wo);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const uint2 f0 = lds_tr16(bXs + kb * 32 * Ly::XP + pt * 32);
          const uint2 f1 = lds_tr16(bXs + (kb * 32 + 4) * Ly::XP + pt * 32);
          const uint4 xb = make_uint4(f0.x, f0.y, f1.x, f1.y);
          sacc[pt] = mfma_bf16(as_bf16x8(ah), as_bf16x8(xb), sacc[pt]);
          sacc[pt] = mfma_bf16(as_bf16x8(al), as_bf16x8(xb), sacc[pt]);
        }
      }
      const float eLend = __builtin_amdgcn_exp2f(sub_lend * LOG2E);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float2 cs = sTh[wave * 8 + 2 * g + q];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const float u = eLend * hst[pt][2 * q] + sacc[pt][2 * q];
          const float w = eLend * hst[pt][2 * q + 1] + sacc[pt][2 * q + 1];
          hst[pt][2 * q] = cs.x * u - cs.y * w;
          hst[pt][2 * q + 1] = cs.y * u + cs.x * w;
        }
      }
    }
    if (more) local_scan();
  }

  // ---------------- epilogue ----------------
  float* dst = (S == 1) ? a.h_final : a.seg_end + blk * (int64_t)(N * P);
  if (dst) {
    float* base = (S == 1 ? dst + bh * (int64_t)(N * P) : dst);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) base[(wave * 16 + 4 * g + i) * P + pt * 16 + m16] = hst[pt][i];
  }
  if (S > 1) {
    float* tot = a.seg_tot + blk * (1 + K);
    if (tid == 0) tot[0] = segLam;
    if (st_t == QS - 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) tot[1 + 4 * st_c + j] = segPhi[j];
    }
  }
}

template <int R>
static hipError_t w32_run(const WalkArgs& a, hipStream_t s) {
  auto kern = walk32_kernel<R>;
  static bool attr_set = false;  // per instantiation; the attribute is per function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, W32<R>::BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = a.batch * a.H * a.S;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), W32<R>::BYTES, s, a);
  return hipGetLastError();
}

hipError_t launch_walk32(const WalkArgs& a, hipStream_t s) {
  if (a.Q != W32_QS) return hipErrorInvalidValue;
  switch (a.R) {
    case 1: return w32_run<1>(a, s);
    case 2: return w32_run<2>(a, s);
    case 4: return w32_run<4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m3
