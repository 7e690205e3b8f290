// Chunked forward of the Mamba-3 SSM layer core: one fused "chunk walker"
// per (b, h[, sequence segment]).
//
// Method (pages cited by title and section):
//  * linkstar.cloud/article/869, "第一刀：指数梯形离散化": the trapezoidal
//    recurrence unrolls into L = (1-semiseparable decay matrix) x (2-band
//    matrix with gamma on the diagonal and beta below it), i.e. for s < t
//    M[t,s] = exp(Lam_t - Lam_s) q_s with q_s = gamma_s + eps_{s+1},
//    eps = (1 - lam) dt, and M[t,t] = gamma_t;  Lam = cumulative dt*A.
//  * same page, "第二刀": rotations move onto B and C as cumulative angles
//    (B~ = R(-phi) B, C~ = R(-phi) C); the chunk uses chunk-local angles and
//    carries the state between chunks in the un-rotated frame, rotating it by
//    the chunk's total angle.
//  * same page, "第三刀": rank R; a chunk of Q tokens has V = Q*R "virtual rows"
//    (token, rank), and the scores C~ B~^T are V x V.
//  * yetianai.com/news/16273, "榨干硬件算力": parallel matrix work inside a
//    chunk, the state passed from chunk to chunk in order.
//
// Per chunk [c0, c0+Q) of one (b,h), with H' the state entering the chunk
// (un-rotated frame, plus the pending trapezoid term of the token before):
//   y_t     = sum_{c0<=s<=t} M[t,s] (C~_t . B~_s) x_s + exp(Lam_t) C~_t^T H'
//   H'_next = R(Theta) ( exp(Lam_end) H' + sum_s exp(Lam_end - Lam_s) q_s B~_s x_s^T )
// with Lam and phi chunk-local (inclusive), Theta = phi at the chunk end.
//
// gfx950 mapping: NW waves per block, one block per walker, one block per CU
// (LDS bound).  All contractions are MFMA 16x16 tiles (bf16 16x16x32 for bf16
// io, fp32 16x16x4 for fp32 io) with fp32 accumulation.  Everything is
// computed transposed so that results chain in registers:
//   G^T = B~ C~^T          (A: B~ rows from LDS, B: C~ rows in registers)
//   (G o M)^T              masked in registers, becomes the B operand of
//   Y^T  = X^T (G o M)^T   (A: X^T from LDS)
//   Y^T += exp(Lam) (H'^T C~^T)   (A: H'^T from LDS in the io dtype)
//   S    = (w B~)^T X      (A: strided reads of B~, B: X^T rows)
// The fp32 state H' lives in registers of the lanes that own its tiles; an
// io-dtype copy H'^T sits in LDS for the next chunk's inter-chunk term.
// Raw x, B, C, dt, A, lam, theta of the next chunk are loaded into registers
// while the current chunk computes.
#include <type_traits>

#include "m3_common.hpp"
#include "m3_launch.hpp"

namespace m3 {

namespace {

template <typename T>
struct mm;  // MFMA "k-slab" conventions per io dtype

// bf16: one MFMA contracts a slab of 32.  Lane group g holds slab positions
// {4g..4g+3} (elements 0..3) and {16+4g..16+4g+3} (elements 4..7), which is
// exactly where the 16x16 accumulators of two stacked tiles put rows 4g+i and
// 16+4g+i, so a score tile feeds the next product without leaving registers.
template <>
struct mm<bf16_t> {
  static constexpr int SLAB = 32;
  typedef uint4 frag;
  __device__ static frag zero() { return make_uint4(0, 0, 0, 0); }
  // two 8-byte pieces at slab offsets 4g and 16+4g of a contiguous io row
  __device__ static frag lds_row(const u16* row, int g) {
    const uint2 lo = *(const uint2*)(row + 4 * g);
    const uint2 hi = *(const uint2*)(row + 16 + 4 * g);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
  __device__ static f32x4 mac(const frag& a, const frag& b, f32x4 c) {
    return mfma_bf16(as_bf16x8(a), as_bf16x8(b), c);
  }
};

template <>
struct mm<float> {
  static constexpr int SLAB = 16;
  typedef float4 frag;
  __device__ static frag zero() { return make_float4(0, 0, 0, 0); }
  __device__ static frag lds_row(const float* row, int g) { return *(const float4*)(row + 4 * g); }
  __device__ static f32x4 mac(const frag& a, const frag& b, f32x4 c) {
    c = mfma_f32(a.x, b.x, c);
    c = mfma_f32(a.y, b.y, c);
    c = mfma_f32(a.z, b.z, c);
    c = mfma_f32(a.w, b.w, c);
    return c;
  }
};

template <typename T>
struct lds_t { typedef float type; };
template <>
struct lds_t<bf16_t> { typedef u16 type; };

// B~ is kept in LDS as fp32 (rotated once at staging) whenever the tiles fit,
// i.e. for fp32 io and for bf16 io with N, P <= 64; otherwise the raw bf16 B
// is kept and rotated where it is read.
__host__ __device__ constexpr bool b_fp32(int esz, int N, int P) { return esz == 4 || (N <= 64 && P <= 64); }

// LDS layout, shared by host (sizing) and device.  Row pads of 16 bytes.
struct Layout {
  int VP, BLD, XLD, HLD;  // padded virtual rows; leading dims (elements)
  int off_B, off_X, off_H, off_cs, off_sc;
  int bytes;
};

__host__ __device__ inline Layout make_layout(int esz, int N, int P, int Q, int R) {
  Layout L;
  const int slab = esz == 2 ? 32 : 16;
  const int V = Q * R;
  const int bsz = b_fp32(esz, N, P) ? 4 : esz;
  L.VP = ((V + slab - 1) / slab) * slab;
  const int pad = 16 / esz;
  L.BLD = N + 16 / bsz;
  L.XLD = L.VP + pad;
  L.HLD = N + pad;
  int o = 0;
  L.off_B = o; o += L.VP * L.BLD * bsz;
  L.off_X = o; o += P * L.XLD * esz;
  L.off_H = o; o += P * L.HLD * esz;
  o = (o + 15) & ~15;
  L.off_cs = o; o += 64 * (N / 2) * 8;                 // (cos, sin) per (token, pair)
  L.off_sc = o; o += (5 * 64 + 2 + (N / 2)) * 4;       // Lam, eLam, q, gam, w; Lend, spare; Theta
  L.bytes = (o + 15) & ~15;
  return L;
}

constexpr int SC_LAM = 0, SC_EL = 64, SC_Q = 128, SC_GAM = 192, SC_W = 256, SC_LEND = 320, SC_THETA = 322;

}  // namespace

size_t walk_lds_bytes(int io_bf16, int N, int P, int Q, int R) {
  const Layout L = make_layout(io_bf16 ? 2 : 4, N, P, Q, R);
  return L.bytes <= 160 * 1024 ? (size_t)L.bytes : 0;
}

template <typename T, int N, int P, int NW>
__global__ __launch_bounds__(NW * 64, 1) void chunk_walk_kernel(WalkArgs a) {
  typedef typename lds_t<T>::type E;    // LDS element of X^T, H'^T (u16 bits for bf16, float)
  typedef mm<T> M;
  typedef typename M::frag frag;
  constexpr int K = N / 2;
  constexpr int NT = NW * 64;
  constexpr int ESZ = sizeof(E);
  constexpr bool B32 = b_fp32(ESZ, N, P);         // B~ stored rotated in fp32
  typedef typename std::conditional<B32, float, E>::type EB;
  constexpr int VEC = io<T>::VEC;
  constexpr int SLAB = M::SLAB;
  constexpr int NKS = (N + SLAB - 1) / SLAB;      // slabs over n
  constexpr int PT = P / 16;                      // p tiles
  constexpr int NTN = N / 16;                     // n tiles
  constexpr int NST = NTN * PT;                   // state tiles: st -> (nt = st % NTN, pt = st / NTN)
  constexpr int STW = (NST + NW - 1) / NW;        // state tiles per wave
  constexpr int KW = (K + NW - 1) / NW;           // angle pairs scanned per wave
  constexpr int BIT = (256 * N / VEC + NT - 1) / NT;   // B staging vectors per thread (max)
  constexpr int XIT = (256 * P / VEC + NT - 1) / NT;   // x staging vectors per thread (max)
  constexpr float LOG2E = 1.4426950408889634f;

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, g = lane >> 4;
  const int R = a.R, Q = a.Q, V = Q * R;
  const int lgR = R == 4 ? 2 : (R == 2 ? 1 : 0);
  const Layout LY = make_layout(ESZ, N, P, Q, R);
  EB* sB = (EB*)(smem + LY.off_B);     // B~ (fp32) or raw B (io) rows (token, rank) x n
  E* sX = (E*)(smem + LY.off_X);       // X^T: p x (token, rank)
  E* sH = (E*)(smem + LY.off_H);       // H'^T: p x n, io precision
  float2* sCS = (float2*)(smem + LY.off_cs);  // (cos, sin) of the chunk-local angle per (token, pair)
  float* sSC = (float*)(smem + LY.off_sc);

  const int64_t S = a.S;
  const int64_t blk = blockIdx.x;
  const int64_t seg = blk % S, bh = blk / S;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t L = a.L, H = a.H;
  const int64_t t0 = seg * a.seg_len;
  const int64_t t1 = (t0 + a.seg_len < L) ? t0 + a.seg_len : L;
  const int64_t rowsN = (int64_t)R * N, rowsP = (int64_t)R * P;
  // element offset of (token, rank 0) for B/C and x/y, and of token in (B,L,H)
  auto tokBC = [&](int64_t tok) { return ((b * L + tok) * H + h) * rowsN; };
  auto tokX = [&](int64_t tok) { return ((b * L + tok) * H + h) * rowsP; };
  auto tokS = [&](int64_t tok) { return (b * L + tok) * H + h; };
  // in-chunk offsets stay below 2^32 (64 tokens x H x R x max(N, P))
  const uint32_t strBC = (uint32_t)(H * rowsN), strX = (uint32_t)(H * rowsP);

  // column tiles of Y owned by this wave (balanced pairing when NCT == 2 NW)
  const int NCT = V / 16;
  int ctl[2];
  int nct = 0;
  if (NCT == 2 * NW) {
    ctl[0] = wave; ctl[1] = 2 * NW - 1 - wave; nct = 2;
  } else {
    if (wave < NCT) ctl[nct++] = wave;
    if (wave + NW < NCT) ctl[nct++] = wave + NW;
  }

  // zero the padding rows of B and X^T (only when V is not a slab multiple),
  // the scalar arrays and the whole angle table (rows past Q stay zero)
  for (int i = tid; i < (LY.VP - V) * LY.BLD; i += NT) sB[V * LY.BLD + i] = 0;
  for (int i = tid; i < P * (LY.VP - V); i += NT) {
    const int p = i / (LY.VP - V), v = V + i % (LY.VP - V);
    sX[p * LY.XLD + v] = 0;
  }
  for (int i = tid; i < 5 * 64 + 2; i += NT) sSC[i] = 0.0f;
  for (int i = tid; i < 64 * K; i += NT) sCS[i] = make_float2(0.0f, 0.0f);

  // ---------------- raw (prefetch) registers ----------------
  typename io<T>::vec rB[BIT], rX[XIT];
  frag rC[2][NKS];
  float rTh[KW];
  float rdt, rA, rlam, rdt_n, rlam_n;

  auto load_raw = [&](int64_t c0) {
    const int nvalid = (int)((t1 - c0) < Q ? (t1 - c0) : Q);
    const void* gB = (const char*)a.B + tokBC(c0) * io<T>::BYTES;
    const void* gX = (const char*)a.x + tokX(c0) * io<T>::BYTES;
#pragma unroll
    for (int j = 0; j < BIT; ++j) {
      const int i = tid + NT * j;
      const int v = i / (N / VEC), n0 = (i % (N / VEC)) * VEC;
      if (v < V && (v >> lgR) < nvalid)
        rB[j] = ldg16<T>(gB, (uint32_t)(v >> lgR) * strBC + (uint32_t)((v & (R - 1)) * N + n0));
      else
        rB[j] = typename io<T>::vec{};
    }
#pragma unroll
    for (int j = 0; j < XIT; ++j) {
      const int i = tid + NT * j;
      const int v = i / (P / VEC), p0 = (i % (P / VEC)) * VEC;
      if (v < V && (v >> lgR) < nvalid)
        rX[j] = ldg16<T>(gX, (uint32_t)(v >> lgR) * strX + (uint32_t)((v & (R - 1)) * P + p0));
      else
        rX[j] = typename io<T>::vec{};
    }
    const bool tv = lane < nvalid;
    const int64_t ts = tokS(c0 + (tv ? lane : 0));
    rdt = tv ? a.dt[ts] : 0.0f;
    rA = tv ? a.A[ts] : 0.0f;
    rlam = tv ? a.lam[ts] : 0.0f;
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      const int k = wave * KW + j;
      rTh[j] = (tv && k < K) ? a.theta[ts * K + k] : 0.0f;
    }
    // eps of the token after the chunk (0 at the end of the walked range)
    const bool nx = (lane == Q - 1) && (c0 + Q < t1);
    const int64_t tn = tokS(nx ? c0 + Q : c0);
    rdt_n = nx ? a.dt[tn] : 0.0f;
    rlam_n = nx ? a.lam[tn] : 0.0f;
  };

  auto load_raw_C = [&](int64_t c0) {
    const int nvalid = (int)((t1 - c0) < Q ? (t1 - c0) : Q);
    const char* gC = (const char*)a.C + tokBC(c0) * io<T>::BYTES;
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
      const int v = (ci < nct ? ctl[ci] : 0) * 16 + m16;
      const bool ok = ci < nct && (v >> lgR) < nvalid;
      const uint32_t base = ok ? (uint32_t)(v >> lgR) * strBC + (uint32_t)((v & (R - 1)) * N) : 0;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (!ok) { rC[ci][ks] = M::zero(); continue; }
        if constexpr (ESZ == 2) {
          const u16* row = (const u16*)gC + base + ks * 32;
          const uint2 lo = *(const uint2*)(row + 4 * g);
          uint2 hi = make_uint2(0, 0);
          if (ks * 32 + 16 < N) hi = *(const uint2*)(row + 16 + 4 * g);
          rC[ci][ks] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
          rC[ci][ks] = *(const float4*)((const float*)gC + base + ks * 16 + 4 * g);
        }
      }
    }
  };

  // Slab of a B~ row in the MFMA operand layout (see mm<>): from the fp32 B~
  // when B32, else rotated here from the raw bf16 B.
  auto bt_frag = [&](int row, int ks) -> frag {
    if constexpr (B32) {
      const float* rp = (const float*)sB + row * LY.BLD;
      if constexpr (ESZ == 2) {
        const bool two = ks * 32 + 16 < N;
        const float4 lo = *(const float4*)(rp + ks * 32 + 4 * g);
        const float4 hi = two ? *(const float4*)(rp + ks * 32 + 16 + 4 * g) : make_float4(0, 0, 0, 0);
        return make_uint4(pack_bf2(lo.x, lo.y), pack_bf2(lo.z, lo.w), pack_bf2(hi.x, hi.y), pack_bf2(hi.z, hi.w));
      } else {
        return *(const float4*)(rp + ks * 16 + 4 * g);
      }
    } else {
      const int t = row >> lgR;
      const u16* rp = (const u16*)sB + row * LY.BLD + ks * 32;
      const bool two = ks * 32 + 16 < N;
      const uint2 lo = *(const uint2*)(rp + 4 * g);
      const uint2 hi = two ? *(const uint2*)(rp + 16 + 4 * g) : make_uint2(0, 0);
      const float4 ca = *(const float4*)(sCS + t * K + ks * 16 + 2 * g);
      const float4 cb = two ? *(const float4*)(sCS + t * K + ks * 16 + 8 + 2 * g) : make_float4(1, 0, 1, 0);
      const uint32_t w4[4] = {lo.x, lo.y, hi.x, hi.y};
      const float c4[4] = {ca.x, ca.z, cb.x, cb.z}, s4[4] = {ca.y, ca.w, cb.y, cb.w};
      uint32_t o4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float u = bf_lo(w4[q]), w = bf_hi(w4[q]);
        o4[q] = pack_bf2(c4[q] * u + s4[q] * w, c4[q] * w - s4[q] * u);
      }
      return make_uint4(o4[0], o4[1], o4[2], o4[3]);
    }
  };

  // (w B~)^T element for state row n and source row k, in fp32
  auto wbt = [&](int k, int n) -> float {
    const int t = k >> lgR;
    float r;
    if constexpr (B32) {
      r = ((const float*)sB)[k * LY.BLD + n];
    } else {
      const uint32_t wv = *(const uint32_t*)((const u16*)sB + k * LY.BLD + (n & ~1));
      const float be = bf_lo(wv), bo = bf_hi(wv);
      const float2 cs = sCS[t * K + (n >> 1)];
      r = (n & 1) ? (cs.x * bo - cs.y * be) : (cs.x * be + cs.y * bo);
    }
    return r * sSC[SC_W + t];
  };

  // ---------------- state H' (fp32, registers) ----------------
  f32x4 hst[STW];
  {
    // H'_0 = h0 + eps_first * sum_r pB[r] px[r]^T, where (pB, px) is the token
    // before the walked range: prev_B / prev_x for the first segment, the
    // sequence's own token t0-1 for later segments (h0 is then zero: the
    // segment scan adds the true incoming state afterwards).
    const void* pB = nullptr;
    const void* px = nullptr;
    int64_t pBo = 0, pxo = 0;
    if (seg == 0) {
      if (a.prev_B) { pB = a.prev_B; px = a.prev_x; pBo = bh * rowsN; pxo = bh * rowsP; }
    } else {
      pB = a.B; px = a.x; pBo = tokBC(t0 - 1); pxo = tokX(t0 - 1);
    }
    const float eps1 = (t0 < t1) ? (1.0f - a.lam[tokS(t0)]) * a.dt[tokS(t0)] : 0.0f;
#pragma unroll
    for (int j = 0; j < STW; ++j) {
      const int st = wave + NW * j;
      const int nt = st % NTN, pt = st / NTN;
      const int p = pt * 16 + m16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = nt * 16 + 4 * g + i;
        float v = 0.0f;
        if (st < NST) {
          if (seg == 0 && a.h0) v = a.h0[bh * (int64_t)N * P + (int64_t)n * P + p];
          if (pB) {
            float acc = 0.0f;
            for (int r = 0; r < R; ++r) acc += io<T>::load1(pB, pBo + r * N + n) * io<T>::load1(px, pxo + r * P + p);
            v += eps1 * acc;
          }
        }
        hst[j][i] = v;
      }
    }
  }
  auto write_H = [&]() {
#pragma unroll
    for (int j = 0; j < STW; ++j) {
      const int st = wave + NW * j;
      if (st < NST) {
        const int nt = st % NTN, pt = st / NTN;
        E* dst = sH + (pt * 16 + m16) * LY.HLD + nt * 16 + 4 * g;
        if constexpr (ESZ == 2) {
          *(uint2*)dst = make_uint2(pack_bf2(hst[j][0], hst[j][1]), pack_bf2(hst[j][2], hst[j][3]));
        } else {
          *(float4*)dst = make_float4(hst[j][0], hst[j][1], hst[j][2], hst[j][3]);
        }
      }
    }
  };
  write_H();

  // running segment-relative log-decay and angles (only for S > 1), kept by
  // the lanes that scan them
  float segLam = 0.0f;
  float segPhi[KW];
#pragma unroll
  for (int j = 0; j < KW; ++j) segPhi[j] = 0.0f;
  const int64_t nchunks_total = (L + Q - 1) / Q;

  if (t0 < t1) { load_raw(t0); load_raw_C(t0); }

  for (int64_t c0 = t0; c0 < t1; c0 += Q) {
    const int nvalid = (int)((t1 - c0) < Q ? (t1 - c0) : Q);
    // ---------- phase A: scalars, chunk-local scans, X^T ----------
    // LDS scalars per token t: SC_LAM = Lam_t * log2(e) (chunk-local, inclusive),
    // SC_EL = exp(Lam_t), SC_Q = q_t = gamma_t + eps_{t+1}, SC_GAM = gamma_t,
    // SC_W = exp(Lam_end - Lam_t) q_t; SC_LEND = Lam_end * log2(e).
    {
      const bool tv = lane < Q;  // lanes past Q carry zeros
      const float d = tv ? rdt : 0.0f;
      const float eps = (1.0f - rlam) * d;
      const float gam = rlam * d;
      float eps_next = __shfl_down(eps, 1, 64);
      if (lane == Q - 1) eps_next = (1.0f - rlam_n) * rdt_n;
      if (wave == 0) {
        const float lam_c = wave_incl_scan(tv ? d * rA : 0.0f);
        const float lend = __shfl(lam_c, Q - 1, 64);
        const float q = gam + eps_next;
        const float l2 = lam_c * LOG2E, lend2 = lend * LOG2E;
        if (tv) {
          sSC[SC_LAM + lane] = l2;
          sSC[SC_EL + lane] = exp2f(l2);
          sSC[SC_Q + lane] = q;
          sSC[SC_GAM + lane] = gam;
          sSC[SC_W + lane] = exp2f(lend2 - l2) * q;
        }
        if (lane == 0) sSC[SC_LEND] = lend2;
        if (S > 1 && lane == 0) {
          if (seg > 0)
            a.chunk_meta[(bh * nchunks_total + c0 / Q) * (1 + K)] = segLam;
          segLam += lend;
        }
      }
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        const int k = wave * KW + j;
        const float phi = wave_incl_scan(d * rTh[j]);
        if (k < K) {
          if (tv) {
            float s, co;
            sincosf(phi, &s, &co);
            sCS[lane * K + k] = make_float2(co, s);
          }
          if (lane == Q - 1) {
            sSC[SC_THETA + k] = phi;
            if (S > 1) {
              if (seg > 0) a.chunk_meta[(bh * nchunks_total + c0 / Q) * (1 + K) + 1 + k] = segPhi[j];
              segPhi[j] += phi;
            }
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < XIT; ++j) {
      const int i = tid + NT * j;
      const int v = i / (P / VEC), p0 = (i % (P / VEC)) * VEC;
      if (v < V) {
        if constexpr (ESZ == 2) {
          const uint32_t w4[4] = {rX[j].x, rX[j].y, rX[j].z, rX[j].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            sX[(p0 + 2 * q) * LY.XLD + v] = (u16)(w4[q] & 0xffffu);
            sX[(p0 + 2 * q + 1) * LY.XLD + v] = (u16)(w4[q] >> 16);
          }
        } else {
          float f[4];
          io<T>::unpack(rX[j], f);
#pragma unroll
          for (int q = 0; q < 4; ++q) sX[(p0 + q) * LY.XLD + v] = f[q];
        }
      }
    }
    if constexpr (!B32) {
#pragma unroll
      for (int j = 0; j < BIT; ++j) {
        const int i = tid + NT * j;
        const int v = i / (N / VEC), n0 = (i % (N / VEC)) * VEC;
        if (v < V) *(typename io<T>::vec*)((E*)sB + v * LY.BLD + n0) = rB[j];
      }
    }
    __syncthreads();  // angle table, scalars, X^T (raw B) ready
    // ---------- phase B: rotated B~ (fp32) and own C~ ----------
    if constexpr (B32) {
#pragma unroll
      for (int j = 0; j < BIT; ++j) {
        const int i = tid + NT * j;
        const int v = i / (N / VEC), n0 = (i % (N / VEC)) * VEC;
        if (v < V) {
          float f[VEC];
          io<T>::unpack(rB[j], f);
          const int t = v >> lgR;
#pragma unroll
          for (int q = 0; q < VEC / 2; ++q) {
            const float2 cs = sCS[t * K + n0 / 2 + q];
            const float u = f[2 * q], w = f[2 * q + 1];
            f[2 * q] = cs.x * u + cs.y * w;
            f[2 * q + 1] = cs.x * w - cs.y * u;
          }
          float* dst = (float*)sB + v * LY.BLD + n0;
#pragma unroll
          for (int q = 0; q < VEC / 4; ++q) *(float4*)(dst + 4 * q) = make_float4(f[4 * q], f[4 * q + 1], f[4 * q + 2], f[4 * q + 3]);
        }
      }
    }
    frag (&cf)[2][NKS] = rC;  // C~ = R(-phi) C, rotated in place
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
      const int v = (ci < nct ? ctl[ci] : 0) * 16 + m16;
      const int t = (v >> lgR) < Q ? (v >> lgR) : 0;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (ESZ == 2) {
          const uint32_t w4[4] = {rC[ci][ks].x, rC[ci][ks].y, rC[ci][ks].z, rC[ci][ks].w};
          uint32_t o4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = ks * 32 + (q < 2 ? 4 * g + 2 * q : 16 + 4 * g + 2 * (q - 2));
            const float2 cs = n < N ? sCS[t * K + n / 2] : make_float2(1.0f, 0.0f);
            const float u = bf_lo(w4[q]), w = bf_hi(w4[q]);
            o4[q] = pack_bf2(cs.x * u + cs.y * w, cs.x * w - cs.y * u);
          }
          cf[ci][ks] = make_uint4(o4[0], o4[1], o4[2], o4[3]);
        } else {
          float f[4] = {rC[ci][ks].x, rC[ci][ks].y, rC[ci][ks].z, rC[ci][ks].w};
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int n = ks * 16 + 4 * g + 2 * q;
            const float2 cs = sCS[t * K + n / 2];
            const float u = f[2 * q], w = f[2 * q + 1];
            f[2 * q] = cs.x * u + cs.y * w;
            f[2 * q + 1] = cs.x * w - cs.y * u;
          }
          cf[ci][ks] = make_float4(f[0], f[1], f[2], f[3]);
        }
      }
    }
    if constexpr (B32) __syncthreads();  // B~ ready
    // prefetch the next chunk's B, x and scalars (their registers are free now)
    if (c0 + Q < t1) load_raw(c0 + Q);

    // ---------- phase C: outputs ----------
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
      if (ci >= nct) break;
      const int ct = ctl[ci];
      const int vcol = ct * 16 + m16;
      const int tcol = vcol >> lgR;
      const float Lt = sSC[SC_LAM + tcol], gt = sSC[SC_GAM + tcol], eLt = sSC[SC_EL + tcol];
      f32x4 yacc[PT];
      // inter-chunk term: exp(Lam_t) (H'^T C~^T)
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          frag af;
          if constexpr (ESZ == 2) {
            if (ks * 32 + 16 < N) af = M::lds_row((const u16*)sH + (pt * 16 + m16) * LY.HLD + ks * 32, g);
            else { const uint2 lo = *(const uint2*)((const u16*)sH + (pt * 16 + m16) * LY.HLD + ks * 32 + 4 * g); af = make_uint4(lo.x, lo.y, 0, 0); }
          } else {
            af = M::lds_row((const float*)sH + (pt * 16 + m16) * LY.HLD + ks * 16, g);
          }
          acc = M::mac(af, cf[ci][ks], acc);
        }
        yacc[pt] = acc * eLt;
      }
      // intra-chunk term over the causal slabs of source rows
      const int rows_needed = (ct + 1) * 16;
      const int nkb = (rows_needed + SLAB - 1) / SLAB;
      for (int kb = 0; kb < nkb; ++kb) {
        frag gfrag;
        constexpr int SUBS = SLAB / 16;
        float gm[SUBS][4];
#pragma unroll
        for (int sub = 0; sub < SUBS; ++sub) {
          const int srow0 = kb * SLAB + sub * 16;
          f32x4 acc = {0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) acc = M::mac(bt_frag(srow0 + m16, ks), cf[ci][ks], acc);
          // decay x 2-band mask: M[t,s] = exp(Lam_t - Lam_s) q_s (s < t), gamma_t (s == t), 0 (s > t)
          if (R == 4) {  // the four rows of a lane belong to one token
            const int srow = srow0 + 4 * g;
            const int s = srow >> 2;
            const float ls = sSC[SC_LAM + s], qs = sSC[SC_Q + s];
            const float e = exp2f(fminf(Lt - ls, 0.0f)) * qs;
            const float m = srow < V ? (s < tcol ? e : (s == tcol ? gt : 0.0f)) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) gm[sub][i] = acc[i] * m;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int srow = srow0 + 4 * g + i;
              const int s = srow >> lgR;
              const float ls = sSC[SC_LAM + s], qs = sSC[SC_Q + s];
              const float e = exp2f(fminf(Lt - ls, 0.0f)) * qs;
              const float m = srow < V ? (s < tcol ? e : (s == tcol ? gt : 0.0f)) : 0.0f;
              gm[sub][i] = acc[i] * m;
            }
          }
        }
        if constexpr (ESZ == 2) {
          gfrag = make_uint4(pack_bf2(gm[0][0], gm[0][1]), pack_bf2(gm[0][2], gm[0][3]),
                             pack_bf2(gm[SUBS - 1][0], gm[SUBS - 1][1]), pack_bf2(gm[SUBS - 1][2], gm[SUBS - 1][3]));
        } else {
          gfrag = make_float4(gm[0][0], gm[0][1], gm[0][2], gm[0][3]);
        }
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          frag af;
          if constexpr (ESZ == 2) af = M::lds_row((const u16*)sX + (pt * 16 + m16) * LY.XLD + kb * 32, g);
          else af = M::lds_row((const float*)sX + (pt * 16 + m16) * LY.XLD + kb * 16, g);
          yacc[pt] = M::mac(af, gfrag, yacc[pt]);
        }
      }
      // store y (rows p = 16 pt + 4 g + i of column (token, rank) vcol)
      if (tcol < nvalid) {
        const int64_t yo = tokX(c0 + tcol) + (vcol & (R - 1)) * P;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          const int p = pt * 16 + 4 * g;
          if constexpr (ESZ == 2) {
            *(uint2*)((u16*)a.y + yo + p) = make_uint2(pack_bf2(yacc[pt][0], yacc[pt][1]), pack_bf2(yacc[pt][2], yacc[pt][3]));
          } else {
            *(float4*)((float*)a.y + yo + p) = make_float4(yacc[pt][0], yacc[pt][1], yacc[pt][2], yacc[pt][3]);
          }
        }
      }
    }
    if (c0 + Q < t1) load_raw_C(c0 + Q);
    // ---------- chunk state S = (w B~)^T X and the state pass ----------
    // For bf16 the fp32 operand w B~ is split into bf16 hi + lo parts (two
    // MFMAs), so the carried state keeps ~fp32 accuracy; X is exact in bf16.
    {
      const float eLend = exp2f(sSC[SC_LEND]);
      f32x4 sacc[STW];
#pragma unroll
      for (int j = 0; j < STW; ++j) sacc[j] = f32x4{0, 0, 0, 0};
      const int nkb = LY.VP / SLAB;
      for (int kb = 0; kb < nkb; ++kb) {
        frag ahi = M::zero(), alo = M::zero();
        int cur_nt = -1;
#pragma unroll
        for (int j = 0; j < STW; ++j) {
          const int st = wave + NW * j;
          if (st >= NST) continue;
          const int nt = st % NTN, pt = st / NTN;
          if (nt != cur_nt) {
            cur_nt = nt;
            const int n = nt * 16 + m16;
            if constexpr (ESZ == 2) {
              float f[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) f[e] = wbt(kb * 32 + 8 * g + e, n);
              uint32_t h4[4], l4[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const uint32_t hp = pack_bf2(f[2 * q], f[2 * q + 1]);
                h4[q] = hp;
                l4[q] = pack_bf2(f[2 * q] - bf_lo(hp), f[2 * q + 1] - bf_hi(hp));
              }
              ahi = make_uint4(h4[0], h4[1], h4[2], h4[3]);
              alo = make_uint4(l4[0], l4[1], l4[2], l4[3]);
            } else {
              ahi = make_float4(wbt(kb * 16 + 4 * g, n), wbt(kb * 16 + 4 * g + 1, n), wbt(kb * 16 + 4 * g + 2, n),
                                wbt(kb * 16 + 4 * g + 3, n));
            }
          }
          frag bfr;
          if constexpr (ESZ == 2) {
            bfr = *(const uint4*)((const u16*)sX + (pt * 16 + m16) * LY.XLD + kb * 32 + 8 * g);
            sacc[j] = M::mac(ahi, bfr, sacc[j]);
            sacc[j] = M::mac(alo, bfr, sacc[j]);
          } else {
            bfr = *(const float4*)((const float*)sX + (pt * 16 + m16) * LY.XLD + kb * 16 + 4 * g);
            sacc[j] = M::mac(ahi, bfr, sacc[j]);
          }
        }
      }
      // H' <- R(Theta) (exp(Lend) H' + S) on pairs (4g, 4g+1), (4g+2, 4g+3)
#pragma unroll
      for (int j = 0; j < STW; ++j) {
        const int st = wave + NW * j;
        if (st >= NST) continue;
        const int nt = st % NTN;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int k = (nt * 16 + 4 * g) / 2 + q;
          const float2 cs = sCS[(Q - 1) * K + k];
          const float u = eLend * hst[j][2 * q] + sacc[j][2 * q];
          const float w = eLend * hst[j][2 * q + 1] + sacc[j][2 * q + 1];
          hst[j][2 * q] = cs.x * u - cs.y * w;
          hst[j][2 * q + 1] = cs.y * u + cs.x * w;
        }
      }
    }
    __syncthreads();  // every read of this chunk's LDS is done
    write_H();
  }

  // ---------------- epilogue ----------------
  float* dst = (S == 1) ? a.h_final : a.seg_end + blk * (int64_t)N * P;
  if (dst) {
#pragma unroll
    for (int j = 0; j < STW; ++j) {
      const int st = wave + NW * j;
      if (st >= NST) continue;
      const int nt = st % NTN, pt = st / NTN;
      float* base = (S == 1 ? dst + bh * (int64_t)N * P : dst);
#pragma unroll
      for (int i = 0; i < 4; ++i) base[(int64_t)(nt * 16 + 4 * g + i) * P + pt * 16 + m16] = hst[j][i];
    }
  }
  if (S > 1) {
    float* tot = a.seg_tot + blk * (1 + K);
    if (wave == 0 && lane == 0) tot[0] = segLam;
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      const int k = wave * KW + j;
      if (k < K && lane == Q - 1) tot[1 + k] = segPhi[j];
    }
  }
}

template <typename T, int N, int P, int NW>
static hipError_t walk_run(const WalkArgs& a, hipStream_t s) {
  const Layout LY = make_layout(sizeof(typename lds_t<T>::type), N, P, a.Q, a.R);
  auto kern = chunk_walk_kernel<T, N, P, NW>;
  static bool attr_set = false;  // per instantiation; the attribute is per function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = a.batch * a.H * a.S;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NW * 64), LY.bytes, s, a);
  return hipGetLastError();
}

template <typename T, int N, int P>
static hipError_t walk_nw(const WalkArgs& a, hipStream_t s) {
  const int V = a.Q * a.R;
  if (V == 256 || N * P >= 4096) return walk_run<T, N, P, 8>(a, s);
  if constexpr (N * P < 4096) return walk_run<T, N, P, 4>(a, s);
  return hipErrorInvalidValue;
}

template <typename T, int N>
static hipError_t walk_p(int P, const WalkArgs& a, hipStream_t s) {
  switch (P) {
    case 16: return walk_nw<T, N, 16>(a, s);
    case 32: return walk_nw<T, N, 32>(a, s);
    case 64: return walk_nw<T, N, 64>(a, s);
    case 128: return walk_nw<T, N, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t walk_n(int N, int P, const WalkArgs& a, hipStream_t s) {
  switch (N) {
    case 16: return walk_p<T, 16>(P, a, s);
    case 32: return walk_p<T, 32>(P, a, s);
    case 64: return walk_p<T, 64>(P, a, s);
    case 128: return walk_p<T, 128>(P, a, s);
    default: return hipErrorInvalidValue;
  }
}

int walk_chunk(int io_bf16, int N, int P, int Q, int R, int64_t H) {
  if (subwalk_supported(io_bf16, N, P, Q, R, H)) return Q;
  // a chunk shorter than the sub-chunk walker's pieces (e.g. 16 tokens at
  // N = 64) is walked by it at its own length rather than by an older walker
  if (N == 64 || N == 128) {
    const int qs = subwalk_qs(N, R);
    if (Q < qs && subwalk_supported(io_bf16, N, P, qs, R, H)) return qs;
  }
  if (walk_fast_supported(io_bf16, N, P, Q, R)) return Q;
  for (int q = Q; q * R >= 16 && q >= 8; q /= 2)
    if (walk_lds_bytes(io_bf16, N, P, q, R) > 0) return q;
  return 0;
}

hipError_t launch_walk(int io_bf16, int N, int P, const WalkArgs& a, hipStream_t s) {
  if (subwalk_supported(io_bf16, N, P, a.Q, a.R, a.H)) return launch_subwalk(N, a, s);
  if (walk_fast_supported(io_bf16, N, P, a.Q, a.R)) return launch_walk_fast(N, P, a, s);
  return io_bf16 ? walk_n<bf16_t>(N, P, a, s) : walk_n<float>(N, P, a, s);
}

}  // namespace m3
