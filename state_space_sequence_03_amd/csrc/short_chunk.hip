// Short calls of the chunked forward (at most 16 tokens per (b,h), e.g.
// verifying k draft tokens on a decode state): the whole call is one chunk of
// the chunked form, evaluated with bf16 MFMAs (fp32 accumulation) instead of
// token by token on the vector ALUs.  Pages cited by title and section:
//  * linkstar.cloud/article/869, "第一刀：指数梯形离散化": the recurrence over a
//    chunk unrolls into the 1-semiseparable x 2-band form; for s < t
//    M[t,s] = exp(Lam_t - Lam_s) q_s with q_s = gamma_s + eps_{s+1},
//    M[t,t] = gamma_t, Lam the cumulative dt*A;
//  * same page, "第二刀": B~ = R(-phi) B, C~ = R(-phi) C with the cumulative
//    angle phi of dt*theta; the state is carried in the un-rotated frame;
//  * same page, "第三刀": rank R, V = L R virtual rows (token, rank).
// With H' = h0 + eps_1 prev_B^T prev_x (the state entering the call):
//   Y       = diag(exp(Lam)) C~ H' + (G o M) X,        G = C~ B~^T  (V x V)
//   h_final = R(Theta) (exp(Lam_L) H' + (w B~)^T X),   w_s = exp(Lam_L - Lam_s) q_s
// eps_{L+1} = 0: the final state carries no pending trapezoid term, as in the
// other paths.
//
// gfx950 mapping: one block of 256 threads (4 waves) per (b,h).  The state is
// read once (fp32, into the accumulator layout of the N x P tiles) and written
// once; the inputs of every token go to LDS as bf16 tiles (B~, C~ rows, X^T,
// (w B~)^T as bf16 hi + lo parts so that the state keeps ~fp32 accuracy, H'^T,
// G o M).  All five products are 16x16x32 bf16 MFMAs; A and B operands are
// 16-byte reads along the contraction index (rows padded by 16 bytes so the
// 16 lanes of a read fall in distinct banks).
#include "m3_common.hpp"
#include "m3_launch.hpp"

namespace m3 {

namespace {

// VPR: virtual rows held, a multiple of the MFMA k slab (32 or 64): the
// kernel takes calls with L R <= VPR
template <int N, int R, int VPR>
struct SC {
  static constexpr int P = 64, K = N / 2, LMAX = 16;
  static constexpr int VP = VPR;
  static constexpr int LN = N + 8, LV = VP + 8, LP = P + 8;  // padded row lengths (bf16 elements)
  static constexpr int OFF_B = 0;                        // B~ [VP][LN]
  static constexpr int OFF_C = OFF_B + VP * LN * 2;      // C~ [VP][LN]
  static constexpr int OFF_XT = OFF_C + VP * LN * 2;     // X^T [P][LV]
  static constexpr int OFF_WH = OFF_XT + P * LV * 2;     // (w B~)^T hi [N][LV]
  static constexpr int OFF_WL = OFF_WH + N * LV * 2;     // (w B~)^T lo [N][LV]
  static constexpr int OFF_HT = OFF_WL + N * LV * 2;     // H'^T [P][LN]
  static constexpr int OFF_CS = OFF_HT + P * LN * 2;     // (cos, sin) of phi_t [LMAX][K] float2
  static constexpr int OFF_TH = OFF_CS + LMAX * K * 8;   // theta_t [LMAX][K] float, then (cos, sin) of Theta [K]
  // per token: log2 decay, q, gamma, exp(decay), then the total log-decay (entry LMAX); w per token
  static constexpr int OFF_SS = OFF_TH + LMAX * K * 4 + K * 8;
  static constexpr int OFF_W = OFF_SS + (LMAX + 1) * 16;
  static constexpr int OFF_DT = OFF_W + LMAX * 4;  // dt per token
  static constexpr int BYTES = OFF_DT + LMAX * 4;
};

__device__ __forceinline__ bf16x8 ld8(const u16* p) { return as_bf16x8(*(const uint4*)p); }

}  // namespace

bool short_chunk_supported(int io_bf16, int N, int P, int R) {
  return io_bf16 && P == 64 && (N == 64 || N == 128) && (R == 1 || R == 2 || R == 4);
}

// ONE: the call is a single piece (L <= QS), so no next piece is prefetched
template <int N, int R, int VPR, bool ONE>
__global__ __launch_bounds__(256) void short_chunk_kernel(TokensArgs a) {
  typedef SC<N, R, VPR> S;
  constexpr int P = 64, K = S::K, VP = S::VP, LN = S::LN, LV = S::LV;
  constexpr int QS = VP / R < S::LMAX ? VP / R : S::LMAX;  // tokens per piece
  constexpr int NTW = N / 64;  // 16-row state tiles per wave (all 4 p tiles)
  constexpr float LOG2E = 1.4426950408889634f;
  __shared__ __align__(16) unsigned char smem[S::BYTES];
  u16* sB = (u16*)(smem + S::OFF_B);
  u16* sC = (u16*)(smem + S::OFF_C);
  u16* sXT = (u16*)(smem + S::OFF_XT);
  u16* sWh = (u16*)(smem + S::OFF_WH);
  u16* sWl = (u16*)(smem + S::OFF_WL);
  u16* sHT = (u16*)(smem + S::OFF_HT);
  float2* sCS = (float2*)(smem + S::OFF_CS);
  float* sTr = (float*)(smem + S::OFF_TH);
  float2* sTh = (float2*)(smem + S::OFF_TH + S::LMAX * K * 4);
  float4* sSS = (float4*)(smem + S::OFF_SS);
  float* sW = (float*)(smem + S::OFF_W);
  float* sDt = (float*)(smem + S::OFF_DT);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, m16 = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int L = (int)a.L;
  auto tok = [&](int t) { return (b * a.L + t) * a.H + h; };

  constexpr int NBC = VP * (N / 8) / 256, NXP = VP * (P / 8) / 256, NTH = (QS * K + 255) / 256;
  static_assert(NBC >= 1 && NXP >= 1, "whole pieces per thread");
  uint4 rbv[NBC], rcv[NBC], rxv[NXP];
  float rth[NTH];
  float d = 0.0f, av = 0.0f, lm = 0.0f, dn = 0.0f, ln = 0.0f;
  // Global loads of the piece [c0, c0 + nv): rows v >= nv R read the piece's
  // first token and are zeroed; lane t of wave 0 reads the scalars of token
  // t and of the token after it.
  auto load_piece = [&](int c0, int nv) __attribute__((always_inline)) {
    const int V = nv * R;
#pragma unroll
    for (int q = 0; q < NBC; ++q) {
      const int e = tid + 256 * q, v = e / (N / 8), c = e % (N / 8), vv = v < V ? v : 0;
      const int64_t o = tok(c0 + vv / R) * (R * N) + (vv % R) * N + 8 * c;
      const uint32_t keep = v < V ? 0xffffffffu : 0u;
      const uint4 bw = *(const uint4*)((const u16*)a.B + o), cw = *(const uint4*)((const u16*)a.C + o);
      rbv[q] = make_uint4(bw.x & keep, bw.y & keep, bw.z & keep, bw.w & keep);
      rcv[q] = make_uint4(cw.x & keep, cw.y & keep, cw.z & keep, cw.w & keep);
    }
#pragma unroll
    for (int q = 0; q < NXP; ++q) {
      const int e = tid + 256 * q, v = e / (P / 8), c = e % (P / 8), vv = v < V ? v : 0;
      const uint32_t keep = v < V ? 0xffffffffu : 0u;
      const uint4 xw = *(const uint4*)((const u16*)a.x + tok(c0 + vv / R) * (R * P) + (vv % R) * P + 8 * c);
      rxv[q] = make_uint4(xw.x & keep, xw.y & keep, xw.z & keep, xw.w & keep);
    }
#pragma unroll
    for (int q = 0; q < NTH; ++q) {
      const int e = tid + 256 * q, t = e / K;
      rth[q] = a.theta[tok(c0 + (t < nv ? t : 0)) * K + e % K];
    }
    if (wave == 0) {
      const int64_t tl = tok(c0 + (lane < nv ? lane : 0));
      d = a.dt[tl];
      av = a.A[tl];
      lm = a.lam[tl];
      // the token after this one (its epsilon weights this token's input in the state)
      const int64_t tn = tok(c0 + lane + 1 < L ? c0 + lane + 1 : c0);
      dn = a.dt[tn];
      ln = a.lam[tn];
    }
  };

  load_piece(0, L < QS ? L : QS);
  // the state entering the call, fp32, in the accumulator layout of the
  // wave's tiles: rows n = 16 (wave NTW + j) + 4g + i, column p = 16 pt + m16
  f32x4 hs[NTW][4];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = (wave * NTW + j) * 16 + 4 * g + i, p = pt * 16 + m16;
        hs[j][pt][i] = a.h0 ? a.h0[bh * (int64_t)(N * P) + n * P + p] : 0.0f;
      }
  if (a.prev_B) {
    // H' = h0 + eps_1 prev_B^T prev_x
    float pbn[R][NTW][4], pxr[R][4];
    const float eps1 = (1.0f - a.lam[tok(0)]) * a.dt[tok(0)];
    const u16* pB = (const u16*)a.prev_B + bh * (int64_t)(R * N);
    const u16* px = (const u16*)a.prev_x + bh * (int64_t)(R * P);
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) pxr[r][pt] = bf2f(px[r * P + pt * 16 + m16]);
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const u16* pr = pB + r * N + (wave * NTW + j) * 16 + 4 * g;  // prev_B is only 2-byte aligned
#pragma unroll
        for (int i = 0; i < 4; ++i) pbn[r][j][i] = bf2f(pr[i]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int i = 0; i < 4; ++i) hs[j][pt][i] += eps1 * pbn[r][j][i] * pxr[r][pt];
  }

  // ---- the call as pieces of QS tokens (one piece for L <= QS); the state
  // passes from piece to piece in registers
  for (int c0 = 0; c0 < (ONE ? 1 : L); c0 += QS) {
    const int nv = L - c0 < QS ? L - c0 : QS, V = nv * R;
    if (c0 > 0) __syncthreads();  // the previous piece's LDS reads are done
    // raw B, C rows (v = t R + r) and X^T to LDS
#pragma unroll
    for (int q = 0; q < NBC; ++q) {
      const int e = tid + 256 * q, v = e / (N / 8), c = e % (N / 8);
      *(uint4*)(sB + v * LN + 8 * c) = rbv[q];
      *(uint4*)(sC + v * LN + 8 * c) = rcv[q];
    }
#pragma unroll
    for (int q = 0; q < NXP; ++q) {
      const int e = tid + 256 * q, v = e / (P / 8), c = e % (P / 8);
      const uint32_t w4[4] = {rxv[q].x, rxv[q].y, rxv[q].z, rxv[q].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        sXT[(8 * c + 2 * k) * LV + v] = (u16)(w4[k] & 0xffffu);
        sXT[(8 * c + 2 * k + 1) * LV + v] = (u16)(w4[k] >> 16);
      }
    }
#pragma unroll
    for (int q = 0; q < NTH; ++q)
      if (tid + 256 * q < QS * K) sTr[tid + 256 * q] = rth[q];
    // zero the (w B~)^T columns v >= V (the columns v < V are written below)
    for (int e = tid; e < N * VP; e += 256) {
      const int n = e / VP, v = e % VP;
      if (v >= V) {
        sWh[n * LV + v] = 0;
        sWl[n * LV + v] = 0;
      }
    }
    // per-token scalars of the piece (wave 0, lane t): inclusive log-decay, q, gamma, w
    if (wave == 0) {
      const bool tv = lane < nv;
      const float dd = tv ? d : 0.0f, aa = tv ? av : 0.0f, ll = tv ? lm : 0.0f;
      const float lam_c = wave_incl_scan(dd * aa);
      const float lend = __shfl(lam_c, nv - 1, 64);
      // q_t = gamma_t + eps_{t+1}; no pending term past the call's last token
      const bool has_next = c0 + lane + 1 < L;
      const float gam = ll * dd, q = gam + (has_next && tv ? (1.0f - ln) * dn : 0.0f);
      if (tv) {
        sSS[lane] = make_float4(lam_c * LOG2E, q, gam, __builtin_amdgcn_exp2f(lam_c * LOG2E));
        sW[lane] = __builtin_amdgcn_exp2f((lend - lam_c) * LOG2E) * q;
        sDt[lane] = dd;
      }
      if (lane == 0) sSS[S::LMAX] = make_float4(lend, 0.0f, 0.0f, 0.0f);
    }
    // H'^T in bf16 for the inter-piece output (rows p, columns n)
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int n0 = (wave * NTW + j) * 16 + 4 * g, p = pt * 16 + m16;
        *(uint2*)(sHT + p * LN + n0) =
            make_uint2(pack_bf2(hs[j][pt][0], hs[j][pt][1]), pack_bf2(hs[j][pt][2], hs[j][pt][3]));
      }
    __syncthreads();
    // the next piece's inputs are requested now (their registers are free)
    if constexpr (!ONE)
      if (c0 + QS < L) load_piece(c0 + QS, L - c0 - QS < QS ? L - c0 - QS : QS);
    // cumulative angles of every pair within the piece: one thread per pair, in token order
    if (tid < K) {
      float ph = 0.0f;
#pragma unroll
      for (int t = 0; t < QS; ++t) {
        if (t < nv) {
          ph += sDt[t] * sTr[t * K + tid];
          float sn, cs;
          sincos_rev(ph, &sn, &cs);
          sCS[t * K + tid] = make_float2(cs, sn);
        }
      }
      float sn, cs;
      sincos_rev(ph, &sn, &cs);
      sTh[tid] = make_float2(cs, sn);
    }
    __syncthreads();

    // ---- rotation in place: B~ = R(-phi) B, C~ = R(-phi) C; (w B~)^T hi + lo
    for (int e = tid; e < V * (N / 8); e += 256) {
      const int v = e / (N / 8), c = e % (N / 8), t = v / R;
      uint4* pb = (uint4*)(sB + v * LN + 8 * c);
      uint4* pc = (uint4*)(sC + v * LN + 8 * c);
      const uint4 bv = *pb, cv = *pc;
      const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w}, cw[4] = {cv.x, cv.y, cv.z, cv.w};
      const float wt = sW[t];
      uint32_t bo[4], co[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float2 cs = sCS[t * K + 4 * c + q];
        const float b0 = bf_lo(bw[q]), b1 = bf_hi(bw[q]), cc0 = bf_lo(cw[q]), cc1 = bf_hi(cw[q]);
        const float bt0 = cs.x * b0 + cs.y * b1, bt1 = cs.x * b1 - cs.y * b0;
        bo[q] = pack_bf2(bt0, bt1);
        co[q] = pack_bf2(cs.x * cc0 + cs.y * cc1, cs.x * cc1 - cs.y * cc0);
        // w B~ from the fp32 rotation, split into bf16 hi and lo = w B~ - hi
        const float w0 = wt * bt0, w1 = wt * bt1;
        const uint32_t hp = pack_bf2(w0, w1);
        const uint32_t lp = pack_bf2(w0 - bf_lo(hp), w1 - bf_hi(hp));
        const int n = 8 * c + 2 * q;
        sWh[n * LV + v] = (u16)(hp & 0xffffu);
        sWh[(n + 1) * LV + v] = (u16)(hp >> 16);
        sWl[n * LV + v] = (u16)(lp & 0xffffu);
        sWl[(n + 1) * LV + v] = (u16)(lp >> 16);
      }
      *pb = make_uint4(bo[0], bo[1], bo[2], bo[3]);
      *pc = make_uint4(co[0], co[1], co[2], co[3]);
    }
    __syncthreads();

    // ---- G = C~ B~^T, masked: tiles (vt, st) of the VP x VP grid over the
    // waves, kept in registers until every wave has read B~: G o M then takes
    // B~'s place in LDS
    constexpr int NT1 = VP / 16, GPW = (NT1 * NT1 + 3) / 4;
    float gm[GPW][4];
#pragma unroll
    for (int jg = 0; jg < GPW; ++jg) {
      const int ti = wave + 4 * jg;
      const int vt = ti / NT1, st = ti % NT1;
#pragma unroll
      for (int i = 0; i < 4; ++i) gm[jg][i] = 0.0f;
      if (ti >= NT1 * NT1 || vt * 16 >= V || st * 16 >= V) continue;  // an all-zero tile of G o M
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k0 = 0; k0 < N; k0 += 32)
        acc = mfma_bf16(ld8(sC + (vt * 16 + m16) * LN + k0 + 8 * g), ld8(sB + (st * 16 + m16) * LN + k0 + 8 * g),
                        acc);
      // acc[i] = G[v = 16 vt + 4g + i][s = 16 st + m16]
      const int s = st * 16 + m16, ts = s < V ? s / R : 0;
      const float4 ss = sSS[ts];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = vt * 16 + 4 * g + i, t = v < V ? v / R : 0;
        float m = 0.0f;
        if (v < V && s < V) {
          const float4 st4 = sSS[t];
          if (ts < t) m = __builtin_amdgcn_exp2f(fminf(st4.x - ss.x, 0.0f)) * ss.y;
          else if (ts == t) m = st4.z;
        }
        gm[jg][i] = acc[i] * m;
      }
    }
    __syncthreads();  // every read of B~ is done
    u16* sGM = sB;    // G o M [VP][LN] in B~'s place
#pragma unroll
    for (int jg = 0; jg < GPW; ++jg) {
      const int ti = wave + 4 * jg;
      if (ti >= NT1 * NT1) continue;
      const int vt = ti / NT1, st = ti % NT1;
#pragma unroll
      for (int i = 0; i < 4; ++i) sGM[(vt * 16 + 4 * g + i) * LN + st * 16 + m16] = f2bf(gm[jg][i]);
    }
    __syncthreads();

    // ---- y = exp(Lam) C~ H' + (G o M) X: tiles (vt, pt) over the waves
    for (int ti = wave; ti < NT1 * 4; ti += 4) {
      const int vt = ti / 4, pt = ti % 4;
      if (vt * 16 >= V) continue;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k0 = 0; k0 < N; k0 += 32)
        acc = mfma_bf16(ld8(sC + (vt * 16 + m16) * LN + k0 + 8 * g), ld8(sHT + (pt * 16 + m16) * LN + k0 + 8 * g), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = vt * 16 + 4 * g + i;
        acc[i] *= v < V ? sSS[v < V ? v / R : 0].w : 0.0f;
      }
#pragma unroll
      for (int k0 = 0; k0 < VP; k0 += 32)
        acc = mfma_bf16(ld8(sGM + (vt * 16 + m16) * LN + k0 + 8 * g), ld8(sXT + (pt * 16 + m16) * LV + k0 + 8 * g), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = vt * 16 + 4 * g + i;
        if (v < V) ((u16*)a.y)[tok(c0 + v / R) * (R * P) + (v % R) * P + pt * 16 + m16] = f2bf(acc[i]);
      }
    }

    // ---- state after the piece: R(Theta) (exp(Lam_end) H' + (w B~)^T X), fp32
    const float eL = __expf(sSS[S::LMAX].x);
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int nt = wave * NTW + j;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k0 = 0; k0 < VP; k0 += 32) {
          const bf16x8 xb = ld8(sXT + (pt * 16 + m16) * LV + k0 + 8 * g);
          acc = mfma_bf16(ld8(sWh + (nt * 16 + m16) * LV + k0 + 8 * g), xb, acc);
          acc = mfma_bf16(ld8(sWl + (nt * 16 + m16) * LV + k0 + 8 * g), xb, acc);
        }
        // rows 4g + i: pairs (4g, 4g + 1) and (4g + 2, 4g + 3)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float2 cs = sTh[(nt * 16 + 4 * g) / 2 + q];
          const float u = eL * hs[j][pt][2 * q] + acc[2 * q], w = eL * hs[j][pt][2 * q + 1] + acc[2 * q + 1];
          hs[j][pt][2 * q] = cs.x * u - cs.y * w;
          hs[j][pt][2 * q + 1] = cs.y * u + cs.x * w;
        }
      }
    }
  }

  // every read of h0 happened before the first piece: h_final may alias it
  if (a.h_final) {
    float* dst = a.h_final + bh * (int64_t)(N * P);
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[((wave * NTW + j) * 16 + 4 * g + i) * P + pt * 16 + m16] = hs[j][pt][i];
  }
}

template <int N, int R>
static void short_launch(const TokensArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.H)), block(256);
  constexpr int QS = SC<N, R, 32>::VP / R < SC<N, R, 32>::LMAX ? SC<N, R, 32>::VP / R : SC<N, R, 32>::LMAX;
  if (a.L <= QS) hipLaunchKernelGGL((short_chunk_kernel<N, R, 32, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((short_chunk_kernel<N, R, 32, false>), grid, block, 0, s, a);
}

template <int N>
static hipError_t short_run(const TokensArgs& a, hipStream_t s) {
  switch (a.R) {
    case 1: short_launch<N, 1>(a, s); break;
    case 2: short_launch<N, 2>(a, s); break;
    case 4: short_launch<N, 4>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_short_chunk(int N, const TokensArgs& a, hipStream_t s) {
  if (a.batch * a.H == 0 || a.L == 0) return hipSuccess;
  if (a.L > TOKENS_MAX) return hipErrorInvalidValue;
  switch (N) {
    case 64: return short_run<64>(a, s);
    case 128: return short_run<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m3
