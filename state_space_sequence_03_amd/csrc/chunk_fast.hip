// Fast chunk walker for bf16 io with N, P <= 64 (the 1.5B-scale workloads).
//
// Computes exactly what chunk_walk_kernel (chunk.hip) computes -- the chunked
// form of the exponential-trapezoidal recurrence with data-dependent RoPE and
// rank-R inputs (linkstar.cloud/article/869, "第一刀", "第二刀", "第三刀";
// yetianai.com/news/16273, "榨干硬件算力") -- with a gfx950-specific data flow
// that keeps the vector ALU off the inner loops:
//
//  * Staging by token lanes.  Lane t of every wave owns token t of the chunk and
//    wave w owns rotation pairs [w*KW, (w+1)*KW).  The lane scans log-decay and
//    angles over the lanes (wave-level inclusive scans), computes sin/cos once
//    per (token, pair), rotates all R ranks of its B rows and writes
//      - B~ (bf16, rows (token, rank) x n) for the intra-chunk scores, and
//      - w_t B~ split into bf16 hi + lo parts, stored transposed (n x rows),
//        for the chunk state, so its MFMA operands are plain 16-byte reads.
//    w_t = exp(Lam_end - Lam_t) q_t is computed by every wave from the same
//    scan, so no barrier separates the scan from the staging.
//  * X is kept in its natural layout (rows x p); the two operands that need it
//    transposed (X^T for the intra-chunk output, X for the chunk state) are
//    fetched with the gfx950 LDS transpose read ds_read_b64_tr_b16.
//  * Each wave owns two column tiles of Y (16 virtual rows each, paired so all
//    waves do the same causal work) and walks one shared loop over source slabs,
//    reading every B~ and X^T fragment once for both tiles.
//  * The decay x 2-band mask uses the hardware exp2; with R = 4 the four rows a
//    lane holds belong to one token, so one exp covers them.
//
// Precision is that of the general walker: bf16 MFMA operands with fp32
// accumulation; the carried state uses the hi + lo split (~fp32 accuracy).
#include "m3_common.hpp"
#include "m3_launch.hpp"

namespace m3 {

namespace {

struct FLayout {
  int VP, BS, WS, XS, HS;
  int off_B, off_Wh, off_Wl, off_X, off_H, off_phi, off_th, off_sc;
  int bytes;
};

__host__ __device__ inline FLayout make_flayout(int N, int P, int Q, int R) {
  FLayout L;
  const int V = Q * R;
  L.VP = ((V + 31) / 32) * 32;
  L.BS = N + 4;       // bf16 B~ rows: 8-byte aligned, conflict-free 16-lane b64 reads
  L.WS = L.VP + 8;    // bf16 (w B~)^T rows: 16-byte aligned
  L.XS = P + 16;      // bf16 X rows: conflict-free transpose reads
  L.HS = N + 8;       // bf16 H'^T rows
  int o = 0;
  L.off_B = o; o += L.VP * L.BS * 2;
  L.off_Wh = o; o += N * L.WS * 2;
  L.off_Wl = o; o += N * L.WS * 2;
  L.off_X = o; o += L.VP * L.XS * 2;
  L.off_H = o; o += P * L.HS * 2;
  o = (o + 15) & ~15;
  L.off_phi = o; o += 64 * (N / 2) * 4;
  L.off_th = o; o += (N / 2) * 8;
  L.off_sc = o; o += (4 * 64 + 2) * 4;
  L.bytes = (o + 15) & ~15;
  return L;
}

constexpr int F_LAM = 0, F_EL = 64, F_Q = 128, F_GAM = 192, F_LEND = 256;

}  // namespace

bool walk_fast_supported(int io_bf16, int N, int P, int Q, int R) {
  if (!io_bf16 || N > 64 || P > 64) return false;
  return make_flayout(N, P, Q, R).bytes <= 160 * 1024;
}

template <int N, int P, int R>
__global__ __launch_bounds__(512, 1) void chunk_walk_fast_kernel(WalkArgs a) {
  constexpr int NW = 8, NT = 512;
  constexpr int K = N / 2;
  constexpr int KW = K / NW;                  // pairs per wave (1, 2 or 4)
  constexpr int NE = 2 * KW;                  // B elements per rank per lane
  constexpr int NKS = (N + 31) / 32;          // 32-wide slabs over n
  constexpr int PT = P / 16;
  constexpr int NTN = N / 16;
  constexpr int NST = NTN * PT;
  constexpr int STW = (NST + NW - 1) / NW;
  constexpr int XIT = (256 * P / 8 + NT - 1) / NT;
  constexpr float LOG2E = 1.4426950408889634f;

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, g = lane >> 4;
  constexpr int lgR = R == 4 ? 2 : (R == 2 ? 1 : 0);
  const int Q = a.Q, V = Q * R;
  const FLayout LY = make_flayout(N, P, Q, R);
  u16* sB = (u16*)(smem + LY.off_B);
  u16* sWh = (u16*)(smem + LY.off_Wh);
  u16* sWl = (u16*)(smem + LY.off_Wl);
  u16* sX = (u16*)(smem + LY.off_X);
  u16* sH = (u16*)(smem + LY.off_H);
  float* sPhi = (float*)(smem + LY.off_phi);
  float2* sTh = (float2*)(smem + LY.off_th);
  float* sSC = (float*)(smem + LY.off_sc);

  const int64_t S = a.S;
  const int64_t blk = blockIdx.x;
  const int64_t seg = blk % S, bh = blk / S;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t L = a.L, H = a.H;
  const int64_t t0 = seg * a.seg_len;
  const int64_t t1 = (t0 + a.seg_len < L) ? t0 + a.seg_len : L;
  const int64_t rowsN = (int64_t)R * N, rowsP = (int64_t)R * P;
  auto tokBC = [&](int64_t tok) { return ((b * L + tok) * H + h) * rowsN; };
  auto tokX = [&](int64_t tok) { return ((b * L + tok) * H + h) * rowsP; };
  auto tokS = [&](int64_t tok) { return (b * L + tok) * H + h; };
  const uint32_t strBC = (uint32_t)(H * rowsN), strX = (uint32_t)(H * rowsP);

  // column tiles of Y: (w, 2 NW - 1 - w) when there are 16 of them
  const int NCT = V / 16;
  int ctl[2];
  int nct = 0;
  if (NCT == 2 * NW) {
    ctl[0] = 2 * NW - 1 - wave; ctl[1] = wave; nct = 2;   // larger causal range first
  } else {
    if (wave + NW < NCT) ctl[nct++] = wave + NW;
    if (wave < NCT) ctl[nct++] = wave;
  }

  // zero padding rows (V < VP only) and the scalar block
  for (int i = tid; i < (LY.VP - V) * LY.BS; i += NT) sB[V * LY.BS + i] = 0;
  for (int i = tid; i < (LY.VP - V) * LY.XS; i += NT) sX[V * LY.XS + i] = 0;
  for (int i = tid; i < N * (LY.VP - V); i += NT) {
    const int n = i / (LY.VP - V), c = V + i % (LY.VP - V);
    sWh[n * LY.WS + c] = 0;
    sWl[n * LY.WS + c] = 0;
  }
  for (int i = tid; i < 4 * 64 + 2; i += NT) sSC[i] = 0.0f;

  // ---------------- prefetch registers ----------------
  typedef uint32_t bvec[NE / 2];   // NE bf16 of one rank row
  bvec rB[R];
  uint4 rX[XIT];
  uint4 rC[2][NKS];
  float rTh[KW];
  float rdt, rA, rlam, rdt_n, rlam_n;

  auto load_raw = [&](int64_t c0) {
    const int nvalid = (int)((t1 - c0) < Q ? (t1 - c0) : Q);
    const bool tv = lane < nvalid;
    const u16* gB = (const u16*)a.B + tokBC(c0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool ok = tv;
      const u16* src = gB + (uint32_t)lane * strBC + (uint32_t)(r * N + wave * NE);
#pragma unroll
      for (int e = 0; e < NE / 2; ++e) rB[r][e] = 0;
      if (ok) {
        if constexpr (NE == 8) {
          const uint4 v = *(const uint4*)src;
          rB[r][0] = v.x; rB[r][1] = v.y; rB[r][2] = v.z; rB[r][3] = v.w;
        } else if constexpr (NE == 4) {
          const uint2 v = *(const uint2*)src;
          rB[r][0] = v.x; rB[r][1] = v.y;
        } else {
          rB[r][0] = *(const uint32_t*)src;
        }
      }
    }
    const int64_t ts = tokS(c0 + (tv ? lane : 0));
    rdt = tv ? a.dt[ts] : 0.0f;
    rA = tv ? a.A[ts] : 0.0f;
    rlam = tv ? a.lam[ts] : 0.0f;
#pragma unroll
    for (int j = 0; j < KW; ++j) rTh[j] = tv ? a.theta[ts * K + wave * KW + j] : 0.0f;
    const bool nx = (lane == Q - 1) && (c0 + Q < t1);
    const int64_t tn = tokS(nx ? c0 + Q : c0);
    rdt_n = nx ? a.dt[tn] : 0.0f;
    rlam_n = nx ? a.lam[tn] : 0.0f;
  };

  auto load_raw_X = [&](int64_t c0) {
    const int nvalid = (int)((t1 - c0) < Q ? (t1 - c0) : Q);
    const u16* gX = (const u16*)a.x + tokX(c0);
#pragma unroll
    for (int j = 0; j < XIT; ++j) {
      const int i = tid + NT * j;
      const int v = i / (P / 8), p0 = (i % (P / 8)) * 8;
      if (v < V && (v >> lgR) < nvalid)
        rX[j] = *(const uint4*)(gX + (uint32_t)(v >> lgR) * strX + (uint32_t)((v & (R - 1)) * P + p0));
      else
        rX[j] = make_uint4(0, 0, 0, 0);
    }
  };

  auto load_raw_C = [&](int64_t c0) {
    const int nvalid = (int)((t1 - c0) < Q ? (t1 - c0) : Q);
    const u16* gC = (const u16*)a.C + tokBC(c0);
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
      const int v = (ci < nct ? ctl[ci] : 0) * 16 + m16;
      const bool ok = ci < nct && (v >> lgR) < nvalid;
      const u16* row = gC + (ok ? (uint32_t)(v >> lgR) * strBC + (uint32_t)((v & (R - 1)) * N) : 0u);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint2 lo = make_uint2(0, 0), hi = make_uint2(0, 0);
        if (ok) {
          lo = *(const uint2*)(row + ks * 32 + 4 * g);
          if (ks * 32 + 16 < N) hi = *(const uint2*)(row + ks * 32 + 16 + 4 * g);
        }
        rC[ci][ks] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
  };

  // ---------------- state H' (fp32, registers) ----------------
  f32x4 hst[STW];
  {
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
            for (int r = 0; r < R; ++r)
              acc += bf2f(((const u16*)pB)[pBo + r * N + n]) * bf2f(((const u16*)px)[pxo + r * P + p]);
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
        *(uint2*)(sH + (pt * 16 + m16) * LY.HS + nt * 16 + 4 * g) =
            make_uint2(pack_bf2(hst[j][0], hst[j][1]), pack_bf2(hst[j][2], hst[j][3]));
      }
    }
  };
  write_H();

  float segLam = 0.0f;
  float segPhi[KW];
#pragma unroll
  for (int j = 0; j < KW; ++j) segPhi[j] = 0.0f;
  const int64_t nchunks_total = (L + Q - 1) / Q;

  if (t0 < t1) { load_raw(t0); load_raw_X(t0); load_raw_C(t0); }

  for (int64_t c0 = t0; c0 < t1; c0 += Q) {
    const int nvalid = (int)((t1 - c0) < Q ? (t1 - c0) : Q);
    // ---------- staging: scans, rotation, B~ and (w B~)^T hi/lo, X ----------
    {
      const bool tq = lane < Q;
      const float d = tq ? rdt : 0.0f;
      const float eps = (1.0f - rlam) * d;
      const float gam = rlam * d;
      float eps_next = __shfl_down(eps, 1, 64);
      if (lane == Q - 1) eps_next = (1.0f - rlam_n) * rdt_n;
      const float lam_c = wave_incl_scan(tq ? d * rA : 0.0f);   // every wave, same values
      const float lend = __shfl(lam_c, Q - 1, 64);
      const float q = gam + eps_next;
      const float l2 = lam_c * LOG2E, lend2 = lend * LOG2E;
      const float wt = __builtin_amdgcn_exp2f(lend2 - l2) * q;
      if (wave == 0) {
        if (tq) {
          sSC[F_LAM + lane] = l2;
          sSC[F_EL + lane] = __builtin_amdgcn_exp2f(l2);
          sSC[F_Q + lane] = q;
          sSC[F_GAM + lane] = gam;
        }
        if (lane == 0) sSC[F_LEND] = lend2;
        if (S > 1 && lane == 0) {
          if (seg > 0) a.chunk_meta[(bh * nchunks_total + c0 / Q) * (1 + K)] = segLam;
          segLam += lend;
        }
      }
      float cs_c[KW], cs_s[KW];
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        const int k = wave * KW + j;
        const float phi = wave_incl_scan(d * rTh[j]);
        fast_sincos(phi, &cs_s[j], &cs_c[j]);
        if (tq) sPhi[lane * K + k] = phi;
        if (lane == Q - 1) {
          sTh[k] = make_float2(cs_c[j], cs_s[j]);
          if (S > 1) {
            if (seg > 0) a.chunk_meta[(bh * nchunks_total + c0 / Q) * (1 + K) + 1 + k] = segPhi[j];
            segPhi[j] += phi;
          }
        }
      }
      if (tq) {
        // rotate ranks of token `lane`: B~ = R(-phi) B on the wave's pairs
        float wb[R][NE];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float bt[NE];
#pragma unroll
          for (int j = 0; j < KW; ++j) {
            const float u = bf_lo(rB[r][j]), w = bf_hi(rB[r][j]);
            bt[2 * j] = cs_c[j] * u + cs_s[j] * w;
            bt[2 * j + 1] = cs_c[j] * w - cs_s[j] * u;
          }
          u16* dst = sB + (lane * R + r) * LY.BS + wave * NE;
          if constexpr (NE == 8) {
            *(uint2*)dst = make_uint2(pack_bf2(bt[0], bt[1]), pack_bf2(bt[2], bt[3]));
            *(uint2*)(dst + 4) = make_uint2(pack_bf2(bt[4], bt[5]), pack_bf2(bt[6], bt[7]));
          } else if constexpr (NE == 4) {
            *(uint2*)dst = make_uint2(pack_bf2(bt[0], bt[1]), pack_bf2(bt[2], bt[3]));
          } else {
            *(uint32_t*)dst = pack_bf2(bt[0], bt[1]);
          }
#pragma unroll
          for (int e = 0; e < NE; ++e) wb[r][e] = wt * bt[e];
        }
        // (w B~)^T: rows n, columns (token, rank); R consecutive columns per lane
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int n = wave * NE + e;
          u16* dh = sWh + n * LY.WS + lane * R;
          u16* dl = sWl + n * LY.WS + lane * R;
          if constexpr (R == 4) {
            const uint32_t h01 = pack_bf2(wb[0][e], wb[1][e]), h23 = pack_bf2(wb[2][e], wb[3][e]);
            const uint32_t l01 = pack_bf2(wb[0][e] - bf_lo(h01), wb[1][e] - bf_hi(h01));
            const uint32_t l23 = pack_bf2(wb[2][e] - bf_lo(h23), wb[3][e] - bf_hi(h23));
            *(uint2*)dh = make_uint2(h01, h23);
            *(uint2*)dl = make_uint2(l01, l23);
          } else if constexpr (R == 2) {
            const uint32_t h01 = pack_bf2(wb[0][e], wb[1][e]);
            *(uint32_t*)dh = h01;
            *(uint32_t*)dl = pack_bf2(wb[0][e] - bf_lo(h01), wb[1][e] - bf_hi(h01));
          } else {
            const uint32_t h0 = pack_bf2(wb[0][e], 0.0f);
            *dh = (u16)(h0 & 0xffffu);
            *dl = (u16)(pack_bf2(wb[0][e] - bf_lo(h0), 0.0f) & 0xffffu);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < XIT; ++j) {
        const int i = tid + NT * j;
        const int v = i / (P / 8), p0 = (i % (P / 8)) * 8;
        if (v < V) *(uint4*)(sX + v * LY.XS + p0) = rX[j];
      }
    }
    __syncthreads();  // B~, (w B~)^T, X, angles and scalars of this chunk are in LDS
    if (c0 + Q < t1) { load_raw(c0 + Q); load_raw_X(c0 + Q); }

    // own C~ fragments: rotate with the chunk angles
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
      const int v = (ci < nct ? ctl[ci] : 0) * 16 + m16;
      const int t = (v >> lgR) < Q ? (v >> lgR) : 0;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint32_t w4[4] = {rC[ci][ks].x, rC[ci][ks].y, rC[ci][ks].z, rC[ci][ks].w};
        uint32_t o4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = ks * 32 + (q < 2 ? 4 * g + 2 * q : 16 + 4 * g + 2 * (q - 2));
          float sn = 0.0f, cn = 1.0f;
          if (n < N) fast_sincos(sPhi[t * K + n / 2], &sn, &cn);
          const float u = bf_lo(w4[q]), w = bf_hi(w4[q]);
          o4[q] = pack_bf2(cn * u + sn * w, cn * w - sn * u);
        }
        rC[ci][ks] = make_uint4(o4[0], o4[1], o4[2], o4[3]);
      }
    }

    // ---------- outputs: Y^T = exp(Lam_t) H'^T C~^T + X^T (G o M)^T ----------
    {
      f32x4 yacc[2][PT];
      int tcol[2];
      float Lt[2], gt[2];
#pragma unroll
      for (int ci = 0; ci < 2; ++ci) {
        const int ct = ci < nct ? ctl[ci] : 0;
        tcol[ci] = (ct * 16 + m16) >> lgR;
        Lt[ci] = sSC[F_LAM + tcol[ci]];
        gt[ci] = sSC[F_GAM + tcol[ci]];
        const float eLt = sSC[F_EL + tcol[ci]];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          f32x4 acc = {0, 0, 0, 0};
          if (ci < nct) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
              const u16* hr = sH + (pt * 16 + m16) * LY.HS + ks * 32;
              const uint2 lo = *(const uint2*)(hr + 4 * g);
              const uint2 hi = (ks * 32 + 16 < N) ? *(const uint2*)(hr + 16 + 4 * g) : make_uint2(0, 0);
              acc = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), as_bf16x8(rC[ci][ks]), acc);
            }
          }
          yacc[ci][pt] = acc * eLt;
        }
      }
      // shared loop over 32-row source slabs; tile 0 has the larger causal range
      const int nkb0 = nct > 0 ? ((ctl[0] + 1) * 16 + 31) / 32 : 0;
      const int nkb1 = nct > 1 ? ((ctl[1] + 1) * 16 + 31) / 32 : 0;
      for (int kb = 0; kb < nkb0; ++kb) {
        // B~ fragments of the two 16-row halves of the slab
        uint4 bfr[2][NKS];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const u16* br = sB + (kb * 32 + sub * 16 + m16) * LY.BS + ks * 32;
            const uint2 lo = *(const uint2*)(br + 4 * g);
            const uint2 hi = (ks * 32 + 16 < N) ? *(const uint2*)(br + 16 + 4 * g) : make_uint2(0, 0);
            bfr[sub][ks] = make_uint4(lo.x, lo.y, hi.x, hi.y);
          }
#pragma unroll
        for (int ci = 0; ci < 2; ++ci) {
          if (ci >= nct || (ci == 1 && kb >= nkb1)) continue;
          float gm[2][4];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) acc = mfma_bf16(as_bf16x8(bfr[sub][ks]), as_bf16x8(rC[ci][ks]), acc);
            const int srow0 = kb * 32 + sub * 16 + 4 * g;
            // computed for every element (no divergent branches), then selected
            // arithmetically: s < t -> decay * q_s, s == t -> gamma_t, else 0
            if constexpr (R == 4) {
              const int s = srow0 >> 2;
              const float e = __builtin_amdgcn_exp2f(fminf(Lt[ci] - sSC[F_LAM + s], 0.0f)) * sSC[F_Q + s];
              const float m = ((s < tcol[ci]) ? 1.0f : 0.0f) * e + ((s == tcol[ci]) ? gt[ci] : 0.0f);
              const float mv = (srow0 < V) ? m : 0.0f;
#pragma unroll
              for (int i = 0; i < 4; ++i) gm[sub][i] = acc[i] * mv;
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int srow = srow0 + i;
                const int s = srow >> lgR;
                const float e = __builtin_amdgcn_exp2f(fminf(Lt[ci] - sSC[F_LAM + s], 0.0f)) * sSC[F_Q + s];
                const float m = ((s < tcol[ci]) ? 1.0f : 0.0f) * e + ((s == tcol[ci]) ? gt[ci] : 0.0f);
                gm[sub][i] = acc[i] * ((srow < V) ? m : 0.0f);
              }
            }
          }
          const uint4 gfr = make_uint4(pack_bf2(gm[0][0], gm[0][1]), pack_bf2(gm[0][2], gm[0][3]),
                                       pack_bf2(gm[1][0], gm[1][1]), pack_bf2(gm[1][2], gm[1][3]));
          // X^T fragments (rows of the slab in the operand order of the scores)
          const int jj = (lane & 15) >> 2, uu = lane & 3;
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) {
            const uint2 f0 = lds_tr16(sX + (kb * 32 + 4 * g + jj) * LY.XS + pt * 16 + 4 * uu);
            const uint2 f1 = lds_tr16(sX + (kb * 32 + 16 + 4 * g + jj) * LY.XS + pt * 16 + 4 * uu);
            yacc[ci][pt] = mfma_bf16(as_bf16x8(make_uint4(f0.x, f0.y, f1.x, f1.y)), as_bf16x8(gfr), yacc[ci][pt]);
          }
        }
      }
      // store y
#pragma unroll
      for (int ci = 0; ci < 2; ++ci) {
        if (ci >= nct || tcol[ci] >= nvalid) continue;
        const int vcol = ctl[ci] * 16 + m16;
        u16* yrow = (u16*)a.y + tokX(c0 + tcol[ci]) + (vcol & (R - 1)) * P;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
          *(uint2*)(yrow + pt * 16 + 4 * g) = make_uint2(pack_bf2(yacc[ci][pt][0], yacc[ci][pt][1]),
                                                         pack_bf2(yacc[ci][pt][2], yacc[ci][pt][3]));
      }
    }
    if (c0 + Q < t1) load_raw_C(c0 + Q);

    // ---------- chunk state S = (w B~)^T X (hi + lo) and the state pass ----------
    {
      const float eLend = __builtin_amdgcn_exp2f(sSC[F_LEND]);
      f32x4 sacc[STW];
#pragma unroll
      for (int j = 0; j < STW; ++j) sacc[j] = f32x4{0, 0, 0, 0};
      const int nkb = LY.VP / 32;
      const int jj = (lane & 15) >> 2, uu = lane & 3;
      for (int kb = 0; kb < nkb; ++kb) {
#pragma unroll
        for (int j = 0; j < STW; ++j) {
          const int st = wave + NW * j;
          if (st >= NST) continue;
          const int nt = st % NTN, pt = st / NTN;
          const int n = nt * 16 + m16;
          const uint4 ah = *(const uint4*)(sWh + n * LY.WS + kb * 32 + 8 * g);
          const uint4 al = *(const uint4*)(sWl + n * LY.WS + kb * 32 + 8 * g);
          const uint2 f0 = lds_tr16(sX + (kb * 32 + 8 * g + jj) * LY.XS + pt * 16 + 4 * uu);
          const uint2 f1 = lds_tr16(sX + (kb * 32 + 8 * g + 4 + jj) * LY.XS + pt * 16 + 4 * uu);
          const uint4 xb = make_uint4(f0.x, f0.y, f1.x, f1.y);
          sacc[j] = mfma_bf16(as_bf16x8(ah), as_bf16x8(xb), sacc[j]);
          sacc[j] = mfma_bf16(as_bf16x8(al), as_bf16x8(xb), sacc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < STW; ++j) {
        const int st = wave + NW * j;
        if (st >= NST) continue;
        const int nt = st % NTN;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int k = (nt * 16 + 4 * g) / 2 + q;
          const float2 cs = sTh[k];
          const float u = eLend * hst[j][2 * q] + sacc[j][2 * q];
          const float w = eLend * hst[j][2 * q + 1] + sacc[j][2 * q + 1];
          hst[j][2 * q] = cs.x * u - cs.y * w;
          hst[j][2 * q + 1] = cs.y * u + cs.x * w;
        }
      }
    }
    __syncthreads();  // all reads of this chunk's LDS are done
    write_H();
  }

  // ---------------- epilogue ----------------
  float* dst = (S == 1) ? a.h_final : a.seg_end + blk * (int64_t)N * P;
  if (dst) {
    float* base = (S == 1 ? dst + bh * (int64_t)N * P : dst);
#pragma unroll
    for (int j = 0; j < STW; ++j) {
      const int st = wave + NW * j;
      if (st >= NST) continue;
      const int nt = st % NTN, pt = st / NTN;
#pragma unroll
      for (int i = 0; i < 4; ++i) base[(int64_t)(nt * 16 + 4 * g + i) * P + pt * 16 + m16] = hst[j][i];
    }
  }
  if (S > 1) {
    float* tot = a.seg_tot + blk * (1 + K);
    if (wave == 0 && lane == 0) tot[0] = segLam;
#pragma unroll
    for (int j = 0; j < KW; ++j)
      if (lane == Q - 1) tot[1 + wave * KW + j] = segPhi[j];
  }
}

template <int N, int P, int R>
static hipError_t fast_run(const WalkArgs& a, hipStream_t s) {
  const FLayout LY = make_flayout(N, P, a.Q, R);
  auto kern = chunk_walk_fast_kernel<N, P, R>;
  static bool attr_set = false;  // per instantiation; the attribute is per function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = a.batch * a.H * a.S;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(512), LY.bytes, s, a);
  return hipGetLastError();
}

template <int N, int P>
static hipError_t fast_r(const WalkArgs& a, hipStream_t s) {
  switch (a.R) {
    case 1: return fast_run<N, P, 1>(a, s);
    case 2: return fast_run<N, P, 2>(a, s);
    case 4: return fast_run<N, P, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int N>
static hipError_t fast_p(int P, const WalkArgs& a, hipStream_t s) {
  switch (P) {
    case 16: return fast_r<N, 16>(a, s);
    case 32: return fast_r<N, 32>(a, s);
    case 64: return fast_r<N, 64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_walk_fast(int N, int P, const WalkArgs& a, hipStream_t s) {
  switch (N) {
    case 16: return fast_p<16>(P, a, s);
    case 32: return fast_p<32>(P, a, s);
    case 64: return fast_p<64>(P, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m3
