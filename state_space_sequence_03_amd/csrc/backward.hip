// Backward of the chunked forward: the gradients of
//     l = sum_t <dy_t, y_t> + <dh_final, h_final>
// with respect to x, B, C, dt, A, lam, theta, h0 and the previous token's B
// and x.  The forward is the chunked form of the exponential-trapezoidal
// recurrence with data-dependent RoPE and rank-R inputs (linkstar.cloud/
// article/869, "第一刀", "第二刀", "第三刀"; chunks computed in parallel
// inside and passed on in order: yetianai.com/news/16273, "榨干硬件算力").
// The backward of a chunk is the chain rule of that chunk's forward, run over
// the chunks in reverse order.
//
// Per chunk of Q tokens (V = Q R virtual rows (token, rank)), chunk-local
// cumulative log-decay Lam_t and angles phi_t, B~ = R(-phi) B, C~ = R(-phi) C,
// q_s = gamma_s + eps_{s+1}, w_s = e^{Lam_end - Lam_s} q_s and
// M[t,s] = e^{Lam_t - Lam_s} q_s (s < t), gamma_t (s = t), 0 (s > t):
//     y_t   = sum_{s<=t} M[t,s] (C~_t . B~_s) x_s + e^{Lam_t} C~_t^T H_in
//     H_out = R(Theta) (e^{Lam_end} H_in + sum_s w_s B~_s x_s^T)
// With G = C~ B~^T, dGM = dY X^T (both V x V), dZ = R(-Theta) dH_out:
//     dX   = (G o M)^T dY + (w B~) dZ
//     dC~  = (dGM o M) B~ + e^{Lam} dY H_in^T
//     dB~  = (dGM o M)^T C~ + w X dZ^T
//     dH_in = e^{Lam_end} dZ + C~^T (e^{Lam} dY)
// and the scalar adjoints follow from dM = dGM o G (summed over the rank
// blocks), dw_s = B~_s . (X dZ^T)_s, d e^{Lam_t} = C~_t . (dY H_in^T)_t,
// <dZ, H_in> and the rotation adjoints of B~, C~ and H_out.
//
// Two kernels, one block per (b,h) each:
//  1. bwd_ckpt_kernel walks the chunks forward and stores the carried state
//     H' at every chunk start (and the final one) in the workspace;
//  2. bwd_chunk_kernel walks the chunks backward with dH' in registers.
// For fp32 io every product is a fp32 MFMA (16x16x4) over fp32 tiles in LDS,
// so those gradients carry fp32 rounding only. For bf16 io the products are
// bf16 MFMAs (16x16x32) with fp32 accumulation, the precision the forward's
// products have: the reverse walk rounds each operand to bf16, and the
// checkpoint walk, whose states accumulate over the whole sequence, splits
// w B~ into bf16 hi and lo parts (two MFMAs, accurate to ~2^-17). The chunk is
// 16 tokens (8 when N or P is 128 and R = 4, 16 / R when both are, to fit
// LDS), V <= 64, N, P <= 128.  When N = P = 128 leaves no room for the
// chunk's incoming state in LDS, the reverse walk reads it from its
// checkpoint in global memory (L2) instead.
#include "m3_common.hpp"
#include "m3_lanes.hpp"
#include "m3_launch.hpp"
#include "m3_order.hpp"

namespace m3 {

bool bwd_supported(int N, int P, int R) {
  const bool n = N == 16 || N == 32 || N == 64 || N == 128, p = P == 16 || P == 32 || P == 64 || P == 128;
  return n && p && (R == 1 || R == 2 || R == 4);
}

namespace {

// Shapes of one (N, P, R) instance
template <int N, int P, int R>
struct BS {
  static constexpr int QB = bwd_chunk_len(N, P, R);
  static constexpr int K = N / 2, V = QB * R;
  static constexpr int LDN = N + 4, LDP = P + 4, LDV = V + 4;  // fp32 row strides in LDS
  static constexpr int TN = N / 16, TP = P / 16, TV = V / 16;   // 16-wide tiles
  static constexpr int NPT = TN * TP;                           // tiles of an N x P matrix
};

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// acc[j] += A(tr*16 + m16, k) B(k, tc*16 + m16) over k < KD for the wave's
// tiles j of a TM x TN grid (tile ti = wave + NW j, tr = ti / TNC, tc = ti % TNC),
// fp32 MFMA 16x16x4 with scalar operand readers fa(row, k), fb(k, col). The k
// loop is outside the tile loop, so the wave's tiles form independent MFMA
// chains that are issued interleaved.
template <int NW, int TM, int TNC, int KD, typename FA, typename FB>
__device__ __forceinline__ void mm(FA fa, FB fb, f32x4* acc, int wave, int m16, int g) {
  constexpr int NT = TM * TNC, TPW = (NT + NW - 1) / NW;
  if constexpr (NT % NW == 0) {
#pragma unroll 2
    for (int k0 = 0; k0 < KD; k0 += 4) {
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int ti = wave + NW * j, tr = ti / TNC, tc = ti % TNC;
        acc[j] = mfma_f32(fa(tr * 16 + m16, k0 + g), fb(k0 + g, tc * 16 + m16), acc[j]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int ti = wave + NW * j;
      if (ti < NT) {
        const int tr = ti / TNC, tc = ti % TNC;
#pragma unroll 4
        for (int k0 = 0; k0 < KD; k0 += 4) acc[j] = mfma_f32(fa(tr * 16 + m16, k0 + g), fb(k0 + g, tc * 16 + m16), acc[j]);
      }
    }
  }
}

// Operand readers for mmv: IC<E> selects E = 8 (16x16x32) or 4 (16x16x16).
template <int E>
struct IC {
  static constexpr int value = E;
};
template <int E>
struct BV;
template <>
struct BV<8> {
  typedef bf16x8 t;
  typedef f32x8 f;
  typedef uint4 u;
};
template <>
struct BV<4> {
  typedef bf16x4 t;
  typedef f32x4 f;
  typedef uint2 u;
};
// E consecutive bf16 from LDS (one 16- or 8-byte read)
template <int E>
__device__ __forceinline__ typename BV<E>::t lds_bf(const u16* p) {
  return __builtin_bit_cast(typename BV<E>::t, *(const typename BV<E>::u*)p);
}
// E consecutive fp32 from LDS (16-byte reads) times s, rounded to bf16
template <int E>
__device__ __forceinline__ typename BV<E>::t lds_f2bf(const float* p, float s) {
  typename BV<E>::f v;
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    const float4 q = *(const float4*)(p + e);
    v[e] = q.x * s;
    v[e + 1] = q.y * s;
    v[e + 2] = q.z * s;
    v[e + 3] = q.w * s;
  }
  return __builtin_convertvector(v, typename BV<E>::t);
}

// Elements (kk .. kk+E-1, r) down column r of a bf16 tile with row stride ld
// (r = 16 * tile + m16 for lane m16 of a 16-lane group). The transpose read
// gives lane i element (i mod 4) of the 8 bytes that lane 4j + i/4 of its
// group addresses, as its element j: lane m16 addresses row kk + m16/4 at
// columns 16 * tile + 4 (m16 mod 4) .. + 3, so lane m16 receives rows
// kk .. kk+3 of column 16 * tile + m16; a second read gives kk+4 .. kk+7.
template <int E>
__device__ __forceinline__ typename BV<E>::t lds_col(const u16* base, int ld, int r, int kk) {
  auto at = [&](int k) { return base + (k + ((r & 15) >> 2)) * ld + (r & ~15) + 4 * (r & 3); };
  const uint2 f0 = lds_tr16(at(kk));
  if constexpr (E == 4) {
    return __builtin_bit_cast(bf16x4, f0);
  } else {
    const uint2 f1 = lds_tr16(at(kk + 4));
    return __builtin_bit_cast(bf16x8, make_uint4(f0.x, f0.y, f1.x, f1.y));
  }
}

// acc[j] += A(tr*16 + m16, k) B(k, tc*16 + m16) over k < KD with bf16
// operands and fp32 accumulation, the operands given as vectors along k:
// fa(row, kk, IC<E>) = A(row, kk .. kk+E-1), fb(col, kk, IC<E>) =
// B(kk .. kk+E-1, col). Lane group g takes k in [8g, 8g + 8) of each 32-wide
// block (16x16x32), or [4g, 4g + 4) of a last block of 16 (16x16x16).
template <int NW, int TM, int TNC, int KD, typename FA, typename FB>
__device__ __forceinline__ void mmv(FA fa, FB fb, f32x4* acc, int wave, int m16, int g) {
  constexpr int NT = TM * TNC, TPW = (NT + NW - 1) / NW;
  static_assert(KD % 16 == 0, "k in steps of 16");
  constexpr int K32 = KD / 32 * 32;
  if constexpr (NT % NW == 0 && K32 > 0) {
    // every operand of the product first, then the products: the LDS reads
    // are in flight together instead of one MFMA waiting on each pair
    bf16x8 oa[K32 / 32][TPW], ob[K32 / 32][TPW];
#pragma unroll
    for (int k0 = 0; k0 < K32; k0 += 32)
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int ti = wave + NW * j, tr = ti / TNC, tc = ti % TNC, kk = k0 + 8 * g;
        oa[k0 / 32][j] = fa(tr * 16 + m16, kk, IC<8>{});
        ob[k0 / 32][j] = fb(tc * 16 + m16, kk, IC<8>{});
      }
#pragma unroll
    for (int k0 = 0; k0 < K32; k0 += 32)
#pragma unroll
      for (int j = 0; j < TPW; ++j) acc[j] = mfma_bf16(oa[k0 / 32][j], ob[k0 / 32][j], acc[j]);
  } else {
#pragma unroll
  for (int k0 = 0; k0 < K32; k0 += 32) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int ti = wave + NW * j;
      if (NT % NW == 0 || ti < NT) {
        const int tr = ti / TNC, tc = ti % TNC, kk = k0 + 8 * g;
        acc[j] = mfma_bf16(fa(tr * 16 + m16, kk, IC<8>{}), fb(tc * 16 + m16, kk, IC<8>{}), acc[j]);
      }
    }
  }
  }
  if constexpr (KD % 32 == 16) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int ti = wave + NW * j;
      if (NT % NW == 0 || ti < NT) {
        const int tr = ti / TNC, tc = ti % TNC, kk = K32 + 4 * g;
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa(tr * 16 + m16, kk, IC<4>{}), fb(tc * 16 + m16, kk, IC<4>{}),
                                                             acc[j], 0, 0, 0);
      }
    }
  }
}

// Per-token scalars of a chunk (tokens past L are padding with dt = 0, so
// that they change no cumulative quantity and carry no weight).
struct TokScal {
  float d, A, lam, eps_next;
};

template <typename T>
__device__ __forceinline__ float ld_io(const void* p, int64_t i) {
  return io<T>::load1(p, i);
}

// An empty asm makes a per-thread offset look new at every use, so that the
// compiler adds it to the block-uniform base (scalar-base addressing with a
// 32-bit offset) instead of hoisting a 64-bit per-thread address out of the
// chunk loop, where it would occupy (or spill) vector register pairs.
__device__ __forceinline__ void fresh(uint32_t& v) { asm volatile("" : "+v"(v)); }

// Four consecutive gradient elements through a buffer resource whose byte
// count ends at the chunk's last token inside the sequence: the hardware drops
// the rows of tokens past L, so the store needs no branch (a branch splits
// the products phase into blocks the scheduler cannot interleave across).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ void store4_rs(__amdgpu_buffer_rsrc_t r, uint32_t i, const float* f) {
  if constexpr (sizeof(T) == 2) {
    const u32x2_t v = {pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3])};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)(i * 2), 0, 0);
  } else {
    const u32x4 v = {__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)(i * 4), 0, 0);
  }
}

// Raw rows of a chunk held in registers: item e of a thread covers row
// v = e / (W / VEC) (token v / R, rank v % R) and the VEC elements from
// column (e % (W / VEC)) VEC of a row W elements wide. `base` points at the
// chunk's first token (block-uniform), tokens are `tstride` elements apart
// (32-bit offsets), and tokens from `nvalid` on (past L) read as 0.
template <typename T, int W, int V, int TH>
struct RowVecs {
  static constexpr int VEC = io<T>::VEC, PERROW = W / VEC, ITEMS = V * PERROW;
  static constexpr int PER = (ITEMS + TH - 1) / TH;
  typename io<T>::vec r[PER];
  __device__ __forceinline__ void load(const void* base, int tid, int R, uint32_t tstride, int nvalid) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + TH * q;
      const int v = e / PERROW, c = e % PERROW, t = v / R;
      uint32_t off = (uint32_t)t * tstride + (uint32_t)((v % R) * W + c * VEC);
      fresh(off);
      if (e < ITEMS && t < nvalid) r[q] = *(const typename io<T>::vec*)((const char*)base + off * io<T>::BYTES);
      else r[q] = typename io<T>::vec{};
    }
  }
};

// Scalars of a token and of the one after it as loaded (dn = ln = 0 past L);
// the trapezoid weight of the next token is formed when the chunk is staged.
struct TokRaw {
  float d, A, lam, dn, ln;
  __device__ __forceinline__ TokScal scal() const { return TokScal{d, A, lam, (1.0f - ln) * dn}; }
};

}  // namespace

// ---------------------------------------------------------------------------
// 1. forward walk storing H' at every chunk start
// ---------------------------------------------------------------------------
template <typename T, int N, int P, int R>
__global__ __launch_bounds__(256) void bwd_ckpt_kernel(BwdArgs a) {
  typedef BS<N, P, R> S;
  constexpr int QB = S::QB, K = S::K, V = S::V, LDN = S::LDN, LDP = S::LDP;
  constexpr int NW = 4, TH = 64 * NW, NPW = (S::NPT + NW - 1) / NW;
  // block (bh, seg): the chunks [c_begin, c_end) of one segment of a (b,h)
  // sequence (one segment spanning all chunks when NS = 1)
  const int NS = a.S > 1 ? a.S : 1;
  int64_t bh, seg;  // block order: adjacent heads on one XCD (m3_order.hpp)
  walker_of_block(blockIdx.x, gridDim.x, a.batch * a.H, NS, bh, seg);
  const int64_t b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, m16 = lane & 15, g = lane >> 4;
  const int64_t L = a.L, nch = (L + QB - 1) / QB;
  const int64_t c_begin = NS > 1 ? seg * a.cps : 0, c_end = NS > 1 ? (c_begin + a.cps < nch ? c_begin + a.cps : nch) : nch;
  // local pass: segments from a zero state (the first from the true one), end
  // states and totals only; otherwise the checkpoints, segments entering with
  // the states of the segment scan
  const bool local = NS > 1 && a.ckpt_local;
  auto tok_of = [&](int64_t t) { return (b * L + t) * a.H + h; };
  const uint32_t Hu = (uint32_t)a.H;

  // bf16 io: W = w B~ as bf16 hi + lo parts (fp32 accuracy to ~2^-17) and X
  // as loaded, for bf16 MFMAs; fp32 io: fp32 tiles and fp32 MFMAs
  constexpr bool BF = sizeof(T) == 2;
  constexpr int LBN = N + 8, LBP = P + 8;
  __shared__ float sW[BF ? 4 : V * LDN], sX[BF ? 4 : V * LDP];
  __shared__ __attribute__((aligned(16))) u16 tWh[BF ? V * LBN : 8], tWl[BF ? V * LBN : 8], tX[BF ? V * LBP : 8];
  __shared__ float2 sCS[QB][K];
  __shared__ float sLam[QB], sQ[QB], sDA[QB], sOm[QB][K];
  __shared__ TokScal sT[QB];

  // H' in the MFMA accumulator layout: tile j holds rows 16 tr + 4g + i, column 16 tc + m16
  f32x4 Hs[NPW];
  const bool has_prev = a.prev_B != nullptr && seg == 0;
  const float eps1 = (has_prev && L > 0) ? (1.0f - a.lam[tok_of(0)]) * a.dt[tok_of(0)] : 0.0f;
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const int ti = wave + NW * j;
    Hs[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (ti < S::NPT) {
      const int tr = ti / S::TP, tc = ti % S::TP, p = tc * 16 + m16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = tr * 16 + 4 * g + i;
        float v = 0.0f;
        if (seg == 0) {
          if (a.h0) v = a.h0[bh * (int64_t)N * P + n * P + p];
        } else if (!local) {
          v = a.seg_in[(bh * NS + seg) * (int64_t)N * P + n * P + p];
        }
        if (has_prev) {
          float acc = 0.0f;
          for (int r = 0; r < R; ++r)
            acc += ld_io<T>(a.prev_B, (bh * R + r) * N + n) * ld_io<T>(a.prev_x, (bh * R + r) * P + p);
          v += eps1 * acc;
        }
        Hs[j][i] = v;
      }
    }
  }
  float* ck = a.ckpt + bh * (nch + 1) * (int64_t)(N * P);
  auto store_state = [&](int64_t c) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      const int ti = wave + NW * j;
      if (ti < S::NPT) {
        const int tr = ti / S::TP, tc = ti % S::TP, p = tc * 16 + m16;
#pragma unroll
        for (int i = 0; i < 4; ++i) ck[c * (N * P) + (tr * 16 + 4 * g + i) * P + p] = Hs[j][i];
      }
    }
  };

  // The inputs of a chunk are fetched into registers one chunk ahead, as
  // loaded: nothing consumes them before the chunk is staged, so their
  // latency overlaps the current chunk's work.
  constexpr int OMP = (QB * K + TH - 1) / TH;
  RowVecs<T, N, V, TH> rb;
  RowVecs<T, P, V, TH> rx;
  float omd[OMP], omt[OMP];
  TokRaw tsv{0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  auto fetch = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t a0 = c * QB, t0 = tok_of(a0);
    const int nv = (int)(L - a0 < QB ? L - a0 : QB), nv1 = (int)(L - a0 < QB + 1 ? L - a0 : QB + 1);
    rb.load((const char*)a.B + t0 * (R * N * io<T>::BYTES), tid, R, Hu * (R * N), nv);
    rx.load((const char*)a.x + t0 * (R * P * io<T>::BYTES), tid, R, Hu * (R * P), nv);
    if (tid < QB) {
      tsv = TokRaw{0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      uint32_t o = (uint32_t)tid * Hu;
      fresh(o);
      if (tid < nv) {
        tsv.d = (a.dt + t0)[o];
        tsv.A = (a.A + t0)[o];
        tsv.lam = (a.lam + t0)[o];
        if (tid + 1 < nv1) {
          tsv.dn = (a.dt + t0)[o + Hu];
          tsv.ln = (a.lam + t0)[o + Hu];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < OMP; ++q) {
      const int e = tid + TH * q, t = e / K, k = e % K;
      const bool ok = e < QB * K && t < nv;
      uint32_t od = (uint32_t)t * Hu, ot = od * K + k;
      fresh(od);
      fresh(ot);
      omd[q] = ok ? (a.dt + t0)[od] : 0.0f;
      omt[q] = ok ? (a.theta + t0 * K)[ot] : 0.0f;
    }
  };
  if (c_begin < c_end) fetch(c_begin);
  float seg_lam = 0.0f, seg_th[OMP];  // segment totals (local pass)
#pragma unroll
  for (int q = 0; q < OMP; ++q) seg_th[q] = 0.0f;

  for (int64_t c = c_begin; c < c_end; ++c) {
    // This chunk's inputs were requested a chunk ago: wait for them before the
    // state stores.  One counter tracks vector loads and stores alike and the
    // stores are conditional, so a wait placed after them would also wait for
    // the stores.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); expcnt and lgkmcnt left alone
    if (!local) store_state(c);
    if (tid < QB) {
      sT[tid] = tsv.scal();
      sDA[tid] = tsv.d * tsv.A;
    }
#pragma unroll
    for (int q = 0; q < OMP; ++q) {
      const int e = tid + TH * q;
      if (e < QB * K) sOm[e / K][e % K] = omd[q] * omt[q];
    }
    __syncthreads();
    if (tid < QB) {
      float lam_c = 0.0f;
#pragma unroll
      for (int j = 0; j < QB; ++j) lam_c += j <= tid ? sDA[j] : 0.0f;  // all reads issued at once
      sLam[tid] = lam_c;
      sQ[tid] = sT[tid].lam * sT[tid].d + sT[tid].eps_next;
    }
#pragma unroll
    for (int q = 0; q < OMP; ++q) {
      const int e = tid + TH * q, t = e / K, k = e % K;
      if (e < QB * K) {
        float ph = 0.0f;
#pragma unroll
        for (int j = 0; j < QB; ++j) ph += j <= t ? sOm[j][k] : 0.0f;
        float sn, cs;
        // the chunk-local angle: the hardware sine/cosine (in revolutions) for
        // bf16 io, the full-precision library routine for fp32 io
        if constexpr (sizeof(T) == 2) sincos_rev(ph, &sn, &cs);
        else sincosf(ph, &sn, &cs);
        sCS[t][k] = make_float2(cs, sn);
        if (t == QB - 1) seg_th[q] += ph;  // the chunk's total angle of pair k
      }
    }
    __syncthreads();
    const float lamQ = sLam[QB - 1];
    seg_lam += lamQ;
    // W = w B~ (rows v = t R + r), X
    {
      constexpr int VEC = io<T>::VEC;
#pragma unroll
      for (int q = 0; q < RowVecs<T, N, V, TH>::PER; ++q) {
        const int e = tid + TH * q;
        if (e < RowVecs<T, N, V, TH>::ITEMS) {
          const int v = e / (N / VEC), n0 = (e % (N / VEC)) * VEC, t = v / R;
          float f[VEC];
          io<T>::unpack(rb.r[q], f);
          const float w = __expf(lamQ - sLam[t]) * sQ[t];
          uint32_t hi[VEC / 2], lo[VEC / 2];
#pragma unroll
          for (int j = 0; j < VEC / 2; ++j) {
            const float2 cs = sCS[t][n0 / 2 + j];
            const float w0 = w * (cs.x * f[2 * j] + cs.y * f[2 * j + 1]);
            const float w1 = w * (cs.x * f[2 * j + 1] - cs.y * f[2 * j]);
            if constexpr (BF) {
              hi[j] = pack_bf2(w0, w1);
              lo[j] = pack_bf2(w0 - bf_lo(hi[j]), w1 - bf_hi(hi[j]));  // the differences are exact in fp32
            } else {
              sW[v * LDN + n0 + 2 * j] = w0;
              sW[v * LDN + n0 + 2 * j + 1] = w1;
            }
          }
          if constexpr (BF) {
            *(uint4*)&tWh[v * LBN + n0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *(uint4*)&tWl[v * LBN + n0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < RowVecs<T, P, V, TH>::PER; ++q) {
        const int e = tid + TH * q;
        if (e < RowVecs<T, P, V, TH>::ITEMS) {
          const int v = e / (P / VEC), p0 = (e % (P / VEC)) * VEC;
          if constexpr (BF) {
            *(uint4*)&tX[v * LBP + p0] = rx.r[q];
          } else {
            float f[VEC];
            io<T>::unpack(rx.r[q], f);
#pragma unroll
            for (int j = 0; j < VEC; ++j) sX[v * LDP + p0 + j] = f[j];
          }
        }
      }
    }
    if (c + 1 < c_end) fetch(c + 1);
    __syncthreads();
    // S = W^T X, then H' <- R(Theta) (e^{Lam_end} H' + S)
    f32x4 sacc[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j) sacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (BF) {
      // S(n, p) = sum_v W(v, n) X(v, p): both operands run down tile columns
      auto rX = [&](int p, int kk, auto e) { return lds_col<decltype(e)::value>(tX, LBP, p, kk); };
      mmv<NW, S::TN, S::TP, V>([&](int n, int kk, auto e) { return lds_col<decltype(e)::value>(tWh, LBN, n, kk); }, rX,
                               sacc, wave, m16, g);
      mmv<NW, S::TN, S::TP, V>([&](int n, int kk, auto e) { return lds_col<decltype(e)::value>(tWl, LBN, n, kk); }, rX,
                               sacc, wave, m16, g);
    } else {
      mm<NW, S::TN, S::TP, V>([&](int n, int v) { return sW[v * LDN + n]; },
                                     [&](int v, int p) { return sX[v * LDP + p]; }, sacc, wave, m16, g);
    }
    const float eQ = __expf(lamQ);
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      const int ti = wave + NW * j;
      if (ti < S::NPT) {
        const int tr = ti / S::TP;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int k = (tr * 16 + 4 * g) / 2 + q;
          const float2 cs = sCS[QB - 1][k];
          const float u = eQ * Hs[j][2 * q] + sacc[j][2 * q];
          const float w = eQ * Hs[j][2 * q + 1] + sacc[j][2 * q + 1];
          Hs[j][2 * q] = cs.x * u - cs.y * w;
          Hs[j][2 * q + 1] = cs.y * u + cs.x * w;
        }
      }
    }
    __syncthreads();  // LDS reads of this chunk done before the next staging
  }
  if (!local) {
    if (seg == NS - 1) store_state(nch);
  } else {
    float* E = a.seg_end + (bh * NS + seg) * (int64_t)(N * P);
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      const int ti = wave + NW * j;
      if (ti < S::NPT) {
        const int tr = ti / S::TP, tc = ti % S::TP, p = tc * 16 + m16;
#pragma unroll
        for (int i = 0; i < 4; ++i) E[(tr * 16 + 4 * g + i) * P + p] = Hs[j][i];
      }
    }
    float* tot = a.seg_tot + (bh * NS + seg) * (int64_t)(1 + K);
    if (tid == 0) tot[0] = seg_lam;
#pragma unroll
    for (int q = 0; q < OMP; ++q) {
      const int e = tid + TH * q, t = e / K, k = e % K;
      if (e < QB * K && t == QB - 1) tot[1 + k] = seg_th[q];
    }
  }
}

// ---------------------------------------------------------------------------
// 1b. (segments) the state adjoint alone, walked backward over one segment
//     from zero at its end: dH' <- e^{Lam_end} R(-Theta) dH' + C~^T (e^{Lam} dY)
// ---------------------------------------------------------------------------
template <typename T, int N, int P, int R>
__global__ __launch_bounds__(256) void bwd_dh_kernel(BwdArgs a) {
  typedef BS<N, P, R> S;
  constexpr int QB = S::QB, K = S::K, V = S::V, LDN = S::LDN, LDP = S::LDP;
  constexpr int NW = 4, TH = 64 * NW, NPW = (S::NPT + NW - 1) / NW;
  // block (bh, seg): the chunks [c_begin, c_end) of one segment of a (b,h)
  // sequence (one segment spanning all chunks when NS = 1)
  const int NS = a.S > 1 ? a.S : 1;
  int64_t bh, seg;  // block order: adjacent heads on one XCD (m3_order.hpp)
  walker_of_block(blockIdx.x, gridDim.x, a.batch * a.H, NS, bh, seg);
  const int64_t b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, m16 = lane & 15, g = lane >> 4;
  const int64_t L = a.L, nch = (L + QB - 1) / QB;
  const int64_t c_begin = NS > 1 ? seg * a.cps : 0, c_end = NS > 1 ? (c_begin + a.cps < nch ? c_begin + a.cps : nch) : nch;
  if (seg == 0) return;  // the first segment's start adjoint is not needed
  auto tok_of = [&](int64_t t) { return (b * L + t) * a.H + h; };
  const uint32_t Hu = (uint32_t)a.H;

  // bf16 io: W = e^{Lam} C~ as bf16 hi + lo parts (fp32 accuracy to ~2^-17)
  // and dY as loaded, for bf16 MFMAs; fp32 io: fp32 tiles and fp32 MFMAs
  constexpr bool BF = sizeof(T) == 2;
  constexpr int LBN = N + 8, LBP = P + 8;
  __shared__ float sW[BF ? 4 : V * LDN], sX[BF ? 4 : V * LDP];
  __shared__ __attribute__((aligned(16))) u16 tWh[BF ? V * LBN : 8], tWl[BF ? V * LBN : 8], tX[BF ? V * LBP : 8];
  __shared__ float2 sCS[QB][K];
  __shared__ float sLam[QB], sQ[QB], sDA[QB], sOm[QB][K];
  __shared__ TokScal sT[QB];

  // dH' in the MFMA accumulator layout, zero at the segment end (dh_final
  // enters through the segment scan, with the last segment's transition)
  f32x4 Hs[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) Hs[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // The inputs of a chunk are fetched into registers one chunk ahead, as
  // loaded: nothing consumes them before the chunk is staged, so their
  // latency overlaps the current chunk's work.
  constexpr int OMP = (QB * K + TH - 1) / TH;
  RowVecs<T, N, V, TH> rb;
  RowVecs<T, P, V, TH> rx;
  float omd[OMP], omt[OMP];
  TokRaw tsv{0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  auto fetch = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t a0 = c * QB, t0 = tok_of(a0);
    const int nv = (int)(L - a0 < QB ? L - a0 : QB), nv1 = (int)(L - a0 < QB + 1 ? L - a0 : QB + 1);
    rb.load((const char*)a.C + t0 * (R * N * io<T>::BYTES), tid, R, Hu * (R * N), nv);
    rx.load((const char*)a.dy + t0 * (R * P * io<T>::BYTES), tid, R, Hu * (R * P), nv);
    if (tid < QB) {
      tsv = TokRaw{0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      uint32_t o = (uint32_t)tid * Hu;
      fresh(o);
      if (tid < nv) {
        tsv.d = (a.dt + t0)[o];
        tsv.A = (a.A + t0)[o];
        tsv.lam = (a.lam + t0)[o];
        if (tid + 1 < nv1) {
          tsv.dn = (a.dt + t0)[o + Hu];
          tsv.ln = (a.lam + t0)[o + Hu];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < OMP; ++q) {
      const int e = tid + TH * q, t = e / K, k = e % K;
      const bool ok = e < QB * K && t < nv;
      uint32_t od = (uint32_t)t * Hu, ot = od * K + k;
      fresh(od);
      fresh(ot);
      omd[q] = ok ? (a.dt + t0)[od] : 0.0f;
      omt[q] = ok ? (a.theta + t0 * K)[ot] : 0.0f;
    }
  };
  if (c_begin < c_end) fetch(c_end - 1);

  for (int64_t c = c_end - 1; c >= c_begin; --c) {
    if (tid < QB) {
      sT[tid] = tsv.scal();
      sDA[tid] = tsv.d * tsv.A;
    }
#pragma unroll
    for (int q = 0; q < OMP; ++q) {
      const int e = tid + TH * q;
      if (e < QB * K) sOm[e / K][e % K] = omd[q] * omt[q];
    }
    __syncthreads();
    if (tid < QB) {
      float lam_c = 0.0f;
#pragma unroll
      for (int j = 0; j < QB; ++j) lam_c += j <= tid ? sDA[j] : 0.0f;  // all reads issued at once
      sLam[tid] = lam_c;
      sQ[tid] = sT[tid].lam * sT[tid].d + sT[tid].eps_next;
    }
#pragma unroll
    for (int q = 0; q < OMP; ++q) {
      const int e = tid + TH * q, t = e / K, k = e % K;
      if (e < QB * K) {
        float ph = 0.0f;
#pragma unroll
        for (int j = 0; j < QB; ++j) ph += j <= t ? sOm[j][k] : 0.0f;
        float sn, cs;
        // the chunk-local angle: the hardware sine/cosine (in revolutions) for
        // bf16 io, the full-precision library routine for fp32 io
        if constexpr (sizeof(T) == 2) sincos_rev(ph, &sn, &cs);
        else sincosf(ph, &sn, &cs);
        sCS[t][k] = make_float2(cs, sn);
      }
    }
    __syncthreads();
    const float lamQ = sLam[QB - 1];
    // W = e^{Lam} C~ (rows v = t R + r), dY
    {
      constexpr int VEC = io<T>::VEC;
#pragma unroll
      for (int q = 0; q < RowVecs<T, N, V, TH>::PER; ++q) {
        const int e = tid + TH * q;
        if (e < RowVecs<T, N, V, TH>::ITEMS) {
          const int v = e / (N / VEC), n0 = (e % (N / VEC)) * VEC, t = v / R;
          float f[VEC];
          io<T>::unpack(rb.r[q], f);
          const float w = __expf(sLam[t]);
          uint32_t hi[VEC / 2], lo[VEC / 2];
#pragma unroll
          for (int j = 0; j < VEC / 2; ++j) {
            const float2 cs = sCS[t][n0 / 2 + j];
            const float w0 = w * (cs.x * f[2 * j] + cs.y * f[2 * j + 1]);
            const float w1 = w * (cs.x * f[2 * j + 1] - cs.y * f[2 * j]);
            if constexpr (BF) {
              hi[j] = pack_bf2(w0, w1);
              lo[j] = pack_bf2(w0 - bf_lo(hi[j]), w1 - bf_hi(hi[j]));  // the differences are exact in fp32
            } else {
              sW[v * LDN + n0 + 2 * j] = w0;
              sW[v * LDN + n0 + 2 * j + 1] = w1;
            }
          }
          if constexpr (BF) {
            *(uint4*)&tWh[v * LBN + n0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *(uint4*)&tWl[v * LBN + n0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < RowVecs<T, P, V, TH>::PER; ++q) {
        const int e = tid + TH * q;
        if (e < RowVecs<T, P, V, TH>::ITEMS) {
          const int v = e / (P / VEC), p0 = (e % (P / VEC)) * VEC;
          if constexpr (BF) {
            *(uint4*)&tX[v * LBP + p0] = rx.r[q];
          } else {
            float f[VEC];
            io<T>::unpack(rx.r[q], f);
#pragma unroll
            for (int j = 0; j < VEC; ++j) sX[v * LDP + p0 + j] = f[j];
          }
        }
      }
    }
    if (c > c_begin) fetch(c - 1);
    __syncthreads();
    // S = W^T dY = C~^T (e^{Lam} dY), then dH' <- e^{Lam_end} R(-Theta) dH' + S
    f32x4 sacc[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j) sacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (BF) {
      // S(n, p) = sum_v W(v, n) dY(v, p): both operands run down tile columns
      auto rX = [&](int p, int kk, auto e) { return lds_col<decltype(e)::value>(tX, LBP, p, kk); };
      mmv<NW, S::TN, S::TP, V>([&](int n, int kk, auto e) { return lds_col<decltype(e)::value>(tWh, LBN, n, kk); }, rX,
                               sacc, wave, m16, g);
      mmv<NW, S::TN, S::TP, V>([&](int n, int kk, auto e) { return lds_col<decltype(e)::value>(tWl, LBN, n, kk); }, rX,
                               sacc, wave, m16, g);
    } else {
      mm<NW, S::TN, S::TP, V>([&](int n, int v) { return sW[v * LDN + n]; },
                                     [&](int v, int p) { return sX[v * LDP + p]; }, sacc, wave, m16, g);
    }
    const float eQ = __expf(lamQ);
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      const int ti = wave + NW * j;
      if (ti < S::NPT) {
        const int tr = ti / S::TP;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int k = (tr * 16 + 4 * g) / 2 + q;
          const float2 cs = sCS[QB - 1][k];
          const float g0 = Hs[j][2 * q], g1 = Hs[j][2 * q + 1];
          Hs[j][2 * q] = eQ * (cs.x * g0 + cs.y * g1) + sacc[j][2 * q];
          Hs[j][2 * q + 1] = eQ * (cs.x * g1 - cs.y * g0) + sacc[j][2 * q + 1];
        }
      }
    }
    __syncthreads();  // LDS reads of this chunk done before the next staging
  }
  float* E = a.dh_loc + (bh * NS + seg) * (int64_t)(N * P);
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const int ti = wave + NW * j;
    if (ti < S::NPT) {
      const int tr = ti / S::TP, tc = ti % S::TP, p = tc * 16 + m16;
#pragma unroll
      for (int i = 0; i < 4; ++i) E[(tr * 16 + 4 * g + i) * P + p] = Hs[j][i];
    }
  }
}

// ---------------------------------------------------------------------------
// 2. backward walk over the chunks in reverse order
// ---------------------------------------------------------------------------
template <typename T, int N, int P, int R>
__global__ __launch_bounds__(512) void bwd_chunk_kernel(BwdArgs a) {
  typedef BS<N, P, R> S;
  constexpr int QB = S::QB, K = S::K, V = S::V, LDN = S::LDN, LDP = S::LDP, LDV = S::LDV;
  constexpr int TV = S::TV, TN = S::TN, TP = S::TP;
  constexpr int NW = 8, TH = 64 * NW, NPW = (S::NPT + NW - 1) / NW;
  // bf16 io: products with bf16 operands (the gradients are rounded to bf16
  // anyway); fp32 io: fp32 products throughout
  constexpr bool BFO = sizeof(T) == 2;
  constexpr int VVW = (TV * TV + NW - 1) / NW, VNW = (TV * TN + NW - 1) / NW, VPW = (TV * TP + NW - 1) / NW;
  // block (bh, seg): the chunks [c_begin, c_end) of one segment, entered with
  // the true state adjoint at the segment end (one segment when NS = 1)
  const int NS = a.S > 1 ? a.S : 1;
  int64_t bh, seg;  // block order: adjacent heads on one XCD (m3_order.hpp)
  walker_of_block(blockIdx.x, gridDim.x, a.batch * a.H, NS, bh, seg);
  const int64_t b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, m16 = lane & 15, g = lane >> 4;
  const int64_t L = a.L, nch = (L + QB - 1) / QB;
  const int64_t c_begin = NS > 1 ? seg * a.cps : 0, c_end = NS > 1 ? (c_begin + a.cps < nch ? c_begin + a.cps : nch) : nch;
  auto tok_of = [&](int64_t t) { return (b * L + t) * a.H + h; };
  const uint32_t Hu = (uint32_t)a.H;

  // fp32 io: fp32 tiles (rows padded by 4 floats) and fp32 MFMAs. bf16 io
  // (TL): the MFMA operands are bf16 tiles with 16-byte row padding, an
  // operand that runs along a tile's rows read 16 bytes at a time, one that
  // runs down its columns with two transpose reads (ds_read_b64_tr_b16); B~,
  // C~ and H_in are also kept in fp32 for the element-wise adjoints.
  constexpr int LBV = V + 8, LBN = N + 8, LBP = P + 8;
  constexpr int SMALL = K * (QB + 1) * 8 + QB * 16 + QB * 16 + QB * QB * 4 + K * (QB + 1) * 8 + TP * K * 4 + QB * 16 + TN * V * 8 + 4 + 512;
  constexpr int TL_BYTES = 4 * (2 * V * LDN + N * LDP) + 2 * (2 * V * LBV + 2 * V * LBP + 4 * V * LBN + P * LBN) + SMALL;
  constexpr int F32_BYTES = 4 * (2 * V * LDN + 2 * N * LDP + 2 * V * LDP + 2 * V * LDV) + SMALL;
  // HG: the chunk's incoming state H_in is read from its checkpoint in
  // global memory instead of an LDS copy (only where the copy does not fit:
  // N = P = 128 in fp32, and in bf16 with 16-token chunks)
  constexpr bool HG = BFO ? TL_BYTES > 160 * 1024 : F32_BYTES > 160 * 1024;
  constexpr bool TL = BFO && TL_BYTES - (HG ? 4 * N * LDP : 0) <= 160 * 1024;
  static_assert(TL || !BFO, "bf16 io takes the bf16 tile layout at every supported size");
  static_assert(BFO || F32_BYTES - (HG ? 4 * N * LDP : 0) <= 160 * 1024, "fp32 tiles fit the LDS");
  __shared__ __attribute__((aligned(16))) float sB[V * LDN], sC[V * LDN], sH[HG ? 4 : N * LDP];  // 16-byte reads
  __shared__ float sX[TL ? 4 : V * LDP], sDY[TL ? 4 : V * LDP];
  __shared__ float sDZ[TL ? 4 : N * LDP], sGM[TL ? 4 : V * LDV], sDG[TL ? 4 : V * LDV];
  __shared__ __attribute__((aligned(16))) u16 tGMt[TL ? V * LBV : 8];  // (G o M)^T
  __shared__ __attribute__((aligned(16))) u16 tDGt[TL ? V * LBV : 8];  // (dGM o M)^T
  __shared__ __attribute__((aligned(16))) u16 tDY[TL ? V * LBP : 8];  // dY
  __shared__ __attribute__((aligned(16))) u16 tX[TL ? V * LBP : 8];   // X
  __shared__ __attribute__((aligned(16))) u16 tB[TL ? V * LBN : 8];   // B~ (bf16 hi part)
  __shared__ __attribute__((aligned(16))) u16 tC[TL ? V * LBN : 8];   // C~ (bf16 hi part)
  __shared__ __attribute__((aligned(16))) u16 tBl[TL ? V * LBN : 8];  // B~ - hi (lo part)
  __shared__ __attribute__((aligned(16))) u16 tCl[TL ? V * LBN : 8];  // C~ - hi (lo part)
  __shared__ __attribute__((aligned(16))) u16 tDZt[TL ? P * LBN : 8];  // dZ^T
  // per-(pair, token) arrays are stored pair-major with rows of QB + 1: the
  // loops that scan over tokens put the QB tokens of a pair on adjacent
  // lanes, which a token-major row of 32 or 64 words would put in one bank
  constexpr int QT = QB + 1;
  __shared__ float2 sCS[K][QT];
  __shared__ TokScal sT[QB];
  __shared__ float sLam[QB], sEL[QB], sQ[QB], sW[QB];
  // per-tile partial sums, each slot written by one lane and summed in a
  // fixed order by its reader (no atomics: the results do not depend on the
  // order in which waves arrive): the angle adjoint of H_out per column tile
  // and pair, and d e^{Lam}, d w per n-tile and virtual row
  __shared__ float sDM[QB][QB], sDphi[K][QT], sDThP[TP][K], sTh[K][QT], sThP[NW][QB];
  __shared__ float sDLam[QB], sDgam[QB], sColL[4][QB], sColQ[4][QB], sDeP[TN][V], sDwP[TN][V], sRedW[NW];
  __shared__ double sRedD[NW];

  const float* ck = a.ckpt + bh * (nch + 1) * (int64_t)(N * P);
  // dH' (adjoint of the carried state) in the accumulator layout of an N x P matrix
  f32x4 Gb[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const int ti = wave + NW * j;
    Gb[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const float* g0 = seg == NS - 1 ? a.dh_final : a.dh_end + (bh * NS + seg) * (int64_t)N * P;
    if (ti < S::NPT && g0) {
      const int tr = ti / TP, tc = ti % TP;
      if (seg == NS - 1) g0 += bh * (int64_t)N * P;
#pragma unroll
      for (int i = 0; i < 4; ++i) Gb[j][i] = g0[(tr * 16 + 4 * g + i) * P + tc * 16 + m16];
    }
  }
  // the first token of the chunk processed last time: its dt and lam
  // gradients wait for the trapezoid weight of the token before it
  float pend_ddt = 0.0f, pend_dlam = 0.0f;

  // Global inputs of a chunk are fetched into registers one chunk ahead, so
  // that their latency overlaps the previous chunk's products.
  constexpr int THP = (QB * K + TH - 1) / TH, HP = HG ? 1 : (N * P / 4 + TH - 1) / TH;
  RowVecs<T, N, V, TH> rb, rc;
  RowVecs<T, P, V, TH> rx, rdy;
  float thv[THP];
  float4 hv[HP];
  TokRaw tsv{0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  auto fetch = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t a0 = c * QB, t0 = tok_of(a0);
    const int nv = (int)(L - a0 < QB ? L - a0 : QB), nv1 = (int)(L - a0 < QB + 1 ? L - a0 : QB + 1);
    rb.load((const char*)a.B + t0 * (R * N * io<T>::BYTES), tid, R, Hu * (R * N), nv);
    rc.load((const char*)a.C + t0 * (R * N * io<T>::BYTES), tid, R, Hu * (R * N), nv);
    rx.load((const char*)a.x + t0 * (R * P * io<T>::BYTES), tid, R, Hu * (R * P), nv);
    rdy.load((const char*)a.dy + t0 * (R * P * io<T>::BYTES), tid, R, Hu * (R * P), nv);
#pragma unroll
    for (int q = 0; q < THP; ++q) {
      const int e = tid + TH * q, t = e / K, k = e % K;
      uint32_t ot = (uint32_t)t * Hu * K + k;
      fresh(ot);
      thv[q] = (e < QB * K && t < nv) ? (a.theta + t0 * K)[ot] : 0.0f;
    }
    if (tid < QB) {
      tsv = TokRaw{0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      uint32_t o = (uint32_t)tid * Hu;
      fresh(o);
      if (tid < nv) {
        tsv.d = (a.dt + t0)[o];
        tsv.A = (a.A + t0)[o];
        tsv.lam = (a.lam + t0)[o];
        if (tid + 1 < nv1) {
          tsv.dn = (a.dt + t0)[o + Hu];
          tsv.ln = (a.lam + t0)[o + Hu];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < HP; ++q) {
      const int e = tid + TH * q;
      uint32_t o = 4 * e;
      fresh(o);
      if (!HG && e < N * P / 4) hv[q] = *(const float4*)(ck + c * (N * P) + o);
    }
  };
  // H_out of the chunk (the carried state after it) in the layout of Gb: the
  // stored final state for the last chunk, then the H_in of the chunk after
  float ho[NPW][4];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const int ti = wave + NW * j;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ho[j][i] = ti < S::NPT ? ck[c_end * (N * P) + ((ti / TP) * 16 + 4 * g + i) * P + (ti % TP) * 16 + m16] : 0.0f;
  }
  // dt and lam of the first token of the chunk processed last time
  float pend_d = 0.0f, pend_l = 0.0f;
  if (c_begin < c_end) fetch(c_end - 1);
  // the first chunk's inputs are waited for here, as every later chunk's are
  // before the stores (below): the loop then starts with nothing to wait for
  // on either path into it
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  for (int64_t c = c_end - 1; c >= c_begin; --c) {
    const int64_t a0 = c * QB, t0c = tok_of(a0);  // block-uniform
    // The lane coordinates are made opaque once per chunk: the compiler then
    // computes LDS addresses next to their uses instead of hoisting dozens of
    // them out of the loop into registers (where they spill).
    uint32_t tid_f = tid;
    fresh(tid_f);
    {
    const int tid = (int)tid_f, lane = tid & 63, m16 = lane & 15, g = lane >> 4;
    // the chunk's outputs: uniform bases at its first token, 32-bit offsets
    void* const odx = (char*)a.dx + t0c * (R * P * io<T>::BYTES);
    void* const odB = (char*)a.dB + t0c * (R * N * io<T>::BYTES);
    void* const odC = (char*)a.dC + t0c * (R * N * io<T>::BYTES);
    const int nvt = (int)(L - a0 < QB ? L - a0 : QB);  // tokens of the chunk inside the sequence
    const __amdgpu_buffer_rsrc_t rdx = __builtin_amdgcn_make_buffer_rsrc(odx, 0, nvt * (int)Hu * (R * P * io<T>::BYTES), 0x00020000);
    const __amdgpu_buffer_rsrc_t rdB = __builtin_amdgcn_make_buffer_rsrc(odB, 0, nvt * (int)Hu * (R * N * io<T>::BYTES), 0x00020000);
    const __amdgpu_buffer_rsrc_t rdC = __builtin_amdgcn_make_buffer_rsrc(odC, 0, nvt * (int)Hu * (R * N * io<T>::BYTES), 0x00020000);
    // H_in (n, p) of this chunk: the LDS copy, or its checkpoint (HG)
    const float* const hg = ck + c * (N * P);
    auto hin = [&](int n, int p) -> float {
      if constexpr (HG) return hg[n * P + p];
      else return sH[n * LDP + p];
    };
    // ---------------- staging (from the registers fetched ahead) ----------------
#pragma unroll
    for (int q = 0; q < THP; ++q) {
      const int e = tid + TH * q;
      if (e < QB * K) sTh[e % K][e / K] = thv[q];
    }
    if (tid < QB) {
      sT[tid] = tsv.scal();
    }
#pragma unroll
    for (int q = 0; q < HP; ++q) {
      const int e = tid + TH * q;
      if (!HG && e < N * P / 4) {
        float* dst = &sH[((4 * e) / P) * LDP + (4 * e) % P];
        dst[0] = hv[q].x; dst[1] = hv[q].y; dst[2] = hv[q].z; dst[3] = hv[q].w;
      }
    }
    __syncthreads();
    // chunk-local prefix sums over the QB tokens, as 16-lane row scans:
    // the log-decay in wave 0, the angles with lane e = k QB + t
    if (tid < 64) {
      const TokScal ts = sT[tid < QB ? tid : 0];
      float lam_c = tid < QB ? ts.d * ts.A : 0.0f;
      lam_c += row_up<1>(lam_c);
      lam_c += row_up<2>(lam_c);
      lam_c += row_up<4>(lam_c);
      if constexpr (QB > 8) lam_c += row_up<8>(lam_c);
      if (tid < QB) {
        sLam[tid] = lam_c;
        sEL[tid] = __expf(lam_c);
        sQ[tid] = ts.lam * ts.d + ts.eps_next;
      }
    }
    for (int e = tid; e < QB * K; e += TH) {  // QB K is a multiple of 64: whole waves
      const int t = e % QB, k = e / QB;
      float ph = sT[t].d * sTh[k][t];
      {
        float u = row_up<1>(ph);
        if (t >= 1) ph += u;
        u = row_up<2>(ph);
        if (t >= 2) ph += u;
        u = row_up<4>(ph);
        if (t >= 4) ph += u;
        if constexpr (QB > 8) {
          u = row_up<8>(ph);
          if (t >= 8) ph += u;
        }
      }
      float sn, cs;
      // the chunk-local angle: the hardware sine/cosine (in revolutions) for
      // bf16 io, the full-precision library routine for fp32 io
      if constexpr (sizeof(T) == 2) sincos_rev(ph, &sn, &cs);
      else sincosf(ph, &sn, &cs);
      sCS[k][t] = make_float2(cs, sn);
    }
    __syncthreads();
    const float lamQ = sLam[QB - 1], eQ = sEL[QB - 1];
    if (tid < QB) sW[tid] = __expf(lamQ - sLam[tid]) * sQ[tid];
    {
      constexpr int VEC = io<T>::VEC;
#pragma unroll
      for (int q = 0; q < RowVecs<T, N, V, TH>::PER; ++q) {
        const int e = tid + TH * q;
        if (e < RowVecs<T, N, V, TH>::ITEMS) {
          const int v = e / (N / VEC), n0 = (e % (N / VEC)) * VEC, t = v / R;
          float fb[VEC], fc[VEC];
          uint32_t pb[VEC / 2], pc[VEC / 2], lb[VEC / 2], lc[VEC / 2];
          io<T>::unpack(rb.r[q], fb);
          io<T>::unpack(rc.r[q], fc);
#pragma unroll
          for (int j = 0; j < VEC / 2; ++j) {
            const float2 cs = sCS[n0 / 2 + j][t];
            const float b0 = cs.x * fb[2 * j] + cs.y * fb[2 * j + 1], b1 = cs.x * fb[2 * j + 1] - cs.y * fb[2 * j];
            const float c0 = cs.x * fc[2 * j] + cs.y * fc[2 * j + 1], c1 = cs.x * fc[2 * j + 1] - cs.y * fc[2 * j];
            sB[v * LDN + n0 + 2 * j] = b0;
            sB[v * LDN + n0 + 2 * j + 1] = b1;
            sC[v * LDN + n0 + 2 * j] = c0;
            sC[v * LDN + n0 + 2 * j + 1] = c1;
            pb[j] = pack_bf2(b0, b1);
            pc[j] = pack_bf2(c0, c1);
            lb[j] = pack_bf2(b0 - bf_lo(pb[j]), b1 - bf_hi(pb[j]));  // the differences are exact in fp32
            lc[j] = pack_bf2(c0 - bf_lo(pc[j]), c1 - bf_hi(pc[j]));
          }
          if constexpr (TL) {
            *(uint4*)&tB[v * LBN + n0] = make_uint4(pb[0], pb[1], pb[2], pb[3]);
            *(uint4*)&tC[v * LBN + n0] = make_uint4(pc[0], pc[1], pc[2], pc[3]);
            *(uint4*)&tBl[v * LBN + n0] = make_uint4(lb[0], lb[1], lb[2], lb[3]);
            *(uint4*)&tCl[v * LBN + n0] = make_uint4(lc[0], lc[1], lc[2], lc[3]);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < RowVecs<T, P, V, TH>::PER; ++q) {
        const int e = tid + TH * q;
        if (e < RowVecs<T, P, V, TH>::ITEMS) {
          const int v = e / (P / VEC), p0 = (e % (P / VEC)) * VEC;
          if constexpr (TL) {
            // the raw bf16 rows as they came
            *(uint4*)&tX[v * LBP + p0] = rx.r[q];
            *(uint4*)&tDY[v * LBP + p0] = rdy.r[q];
          } else {
            float fx[VEC], fd[VEC];
            io<T>::unpack(rx.r[q], fx);
            io<T>::unpack(rdy.r[q], fd);
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
              sX[v * LDP + p0 + j] = fx[j];
              sDY[v * LDP + p0 + j] = fd[j];
            }
          }
        }
      }
    }
    // dZ = R(-Theta) dH_out; dTheta = <dH_out, J H_out> per pair; <dZ, H_in>
    // The LDS operands first, so that they share one wait: the chunk's total
    // angle of the wave's pairs and H_in at the wave's state elements (also
    // the H_out of the chunk processed next).
    float rh[NPW][4];
    {
      float2 rcs[NPW][2];
#pragma unroll
      for (int j = 0; j < NPW; ++j) {
        const int ti = wave + NW * j;
        if (ti < S::NPT) {
          const int tr = ti / TP, p = (ti % TP) * 16 + m16;
#pragma unroll
          for (int q = 0; q < 2; ++q) rcs[j][q] = sCS[(tr * 16 + 4 * g + 2 * q) / 2][QB - 1];
#pragma unroll
          for (int i = 0; i < 4; ++i) rh[j][i] = hin(tr * 16 + 4 * g + i, p);
        }
      }
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < NPW; ++j) {
        const int ti = wave + NW * j;
        if (ti < S::NPT) {
          const int tr = ti / TP, tc = ti % TP, p = tc * 16 + m16;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int n0 = tr * 16 + 4 * g + 2 * q, k = n0 / 2;
            const float2 cs = rcs[j][q];
            const float g0 = Gb[j][2 * q], g1 = Gb[j][2 * q + 1];
            const float z0 = cs.x * g0 + cs.y * g1, z1 = cs.x * g1 - cs.y * g0;
            if constexpr (TL) {
              *(uint32_t*)&tDZt[p * LBN + n0] = pack_bf2(z0, z1);  // features n0, n0 + 1 of column p
            } else {
              sDZ[n0 * LDP + p] = z0;
              sDZ[(n0 + 1) * LDP + p] = z1;
            }
            const float o0 = ho[j][2 * q], o1 = ho[j][2 * q + 1];
            float dth = -g0 * o1 + g1 * o0;
            dth = lane_sum<1, 16>(dth);
            if (m16 == 0) sDThP[tc][k] = dth;
            part += z0 * rh[j][2 * q] + z1 * rh[j][2 * q + 1];
            // dH_in starts as e^{Lam_end} dZ
            Gb[j][2 * q] = eQ * z0;
            Gb[j][2 * q + 1] = eQ * z1;
          }
        }
      }
      part = lane_sum<1, 64>(part);
      if (lane == 0) sRedW[wave] = part;  // summed over the waves in a fixed order below
    }
    if (c > c_begin) {
      // this chunk's H_in is the H_out of the chunk processed next
#pragma unroll
      for (int j = 0; j < NPW; ++j) {
        const int ti = wave + NW * j;
        if (ti < S::NPT) {
#pragma unroll
          for (int i = 0; i < 4; ++i) ho[j][i] = rh[j][i];
        }
      }
      fetch(c - 1);
    }
    __syncthreads();

    // bf16 io: operand readers along k for mmv (row or column index, first k, IC<E>)
    // (an operand index r = 16 * tile + m16 is a row of the operand's tile
    // for rdT, a column for rdTr)
    auto rdWB = [&](int v, int kk, auto e) { return lds_f2bf<decltype(e)::value>(&sB[v * LDN + kk], sW[v / R]); };
    auto rdH = [&](int n, int kk, auto e) {
      if constexpr (HG) return lds_f2bf<decltype(e)::value>(&hg[n * P + kk], 1.0f);
      else return lds_f2bf<decltype(e)::value>(&sH[n * LDP + kk], 1.0f);
    };
    // along a row: elements (r, kk .. kk+E-1)
    auto rdT = [&](const u16* base, int ld) {
      return [=](int r, int kk, auto e) { return lds_bf<decltype(e)::value>(base + r * ld + kk); };
    };
    // down a column: elements (kk .. kk+E-1, r)
    auto rdTr = [&](const u16* base, int ld) {
      return [=](int r, int kk, auto e) { return lds_col<decltype(e)::value>(base, ld, r, kk); };
    };
    // e^{Lam_v} dY(v, p) down column p: the k range holds E / R whole tokens (R | E)
    auto rdELDY = [&](int p, int kk, auto e) {
      constexpr int E = decltype(e)::value;
      const typename BV<E>::t raw = rdTr(tDY, LBP)(p, kk, e);
      typename BV<E>::f f;
#pragma unroll
      for (int q = 0; q < E; ++q) f[q] = (float)raw[q] * sEL[kk / R + q / R];
      return __builtin_convertvector(f, typename BV<E>::t);
    };

    // ---------------- G = C~ B~^T and dGM = dY X^T (V x V), masked ----------------
    {
      f32x4 gacc[VVW], dacc[VVW];
#pragma unroll
      for (int j = 0; j < VVW; ++j) gacc[j] = dacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (TL) {
        mmv<NW, TV, TV, N>(rdT(tC, LBN), rdT(tB, LBN), gacc, wave, m16, g);
        mmv<NW, TV, TV, P>(rdT(tDY, LBP), rdT(tX, LBP), dacc, wave, m16, g);
      } else {
        mm<NW, TV, TV, N>([&](int v, int n) { return sC[v * LDN + n]; }, [&](int n, int v) { return sB[v * LDN + n]; },
                                 gacc, wave, m16, g);
        mm<NW, TV, TV, P>([&](int v, int p) { return sDY[v * LDP + p]; }, [&](int p, int v) { return sX[v * LDP + p]; },
                                 dacc, wave, m16, g);
      }
#pragma unroll
      for (int j = 0; j < VVW; ++j) {
        const int ti = wave + NW * j;
        if (ti < TV * TV) {
          const int tr = ti / TV, tc = ti % TV;
          const int vc = tc * 16 + m16, s = vc / R, vr0 = tr * 16 + 4 * g;
          float pr[4], gm[4], dg[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int vr = vr0 + i, t = vr / R;
            float m = 0.0f;
            if (s < t) m = __expf(fminf(sLam[t] - sLam[s], 0.0f)) * sQ[s];
            else if (s == t) m = sT[t].lam * sT[t].d;
            gm[i] = gacc[j][i] * m;
            dg[i] = dacc[j][i] * m;
            pr[i] = gacc[j][i] * dacc[j][i];
            if constexpr (!TL) {
              sGM[vr * LDV + vc] = gm[i];
              sDG[vr * LDV + vc] = dg[i];
            }
          }
          if constexpr (TL) {
            // rows vr0 .. vr0+3 of column vc are consecutive in the transposed tiles
            *(uint2*)&tGMt[vc * LBV + vr0] = make_uint2(pack_bf2(gm[0], gm[1]), pack_bf2(gm[2], gm[3]));
            *(uint2*)&tDGt[vc * LBV + vr0] = make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
          }
          // dM[t][s]: sum over the R x R rank block (rows R-groups of i, columns R lanes)
#pragma unroll
          for (int i0 = 0; i0 < 4; i0 += R) {
            float v = 0.0f;
#pragma unroll
            for (int i = 0; i < R; ++i) v += pr[i0 + i];
            v = lane_sum<1, R>(v);
            if (m16 % R == 0) sDM[(tr * 16 + 4 * g + i0) / R][s] = v;
          }
        }
      }
    }
    __syncthreads();
    // The next chunk's inputs were requested at this chunk's start and have
    // had the phases above to land: wait for them here, before this chunk's
    // gradient stores.  One counter tracks vector loads and stores alike, and
    // the stores sit behind branches, so a wait at the next chunk's start
    // would also have to wait for every store still in flight.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); expcnt and lgkmcnt left alone

    // ---------------- products on the masked matrices ----------------
    // dX, dC~ and dB~ are computed transposed (feature rows, virtual-row
    // columns): a lane then holds 4 consecutive features of one (token, rank)
    // row, so each rotation pair sits in one lane and the row is stored with
    // one 8-byte write.
    {
      // dX^T = dY^T GM + dZ^T (w B~)^T  (P x V)
      f32x4 xacc[VPW];
#pragma unroll
      for (int j = 0; j < VPW; ++j) xacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (TL) {
        mmv<NW, TP, TV, V>(rdTr(tDY, LBP), rdT(tGMt, LBV), xacc, wave, m16, g);
        mmv<NW, TP, TV, N>(rdT(tDZt, LBN), rdWB, xacc, wave, m16, g);
      } else {
        mm<NW, TP, TV, V>([&](int p, int t) { return sDY[t * LDP + p]; },
                               [&](int t, int s) { return sGM[t * LDV + s]; }, xacc, wave, m16, g);
        mm<NW, TP, TV, N>([&](int p, int n) { return sDZ[n * LDP + p]; },
                               [&](int n, int v) { return sW[v / R] * sB[v * LDN + n]; }, xacc, wave, m16, g);
      }
#pragma unroll
      for (int j = 0; j < VPW; ++j) {
        const int ti = wave + NW * j;
        if (ti < TP * TV) {
          const int tr = ti / TV, tc = ti % TV, v = tc * 16 + m16, t = v / R, p0 = tr * 16 + 4 * g;
          uint32_t off = (uint32_t)t * Hu * (R * P) + (uint32_t)((v % R) * P + p0);
          fresh(off);
          const float f[4] = {xacc[j][0], xacc[j][1], xacc[j][2], xacc[j][3]};
          store4_rs<T>(rdx, off, f);
        }
      }
    }
    {
      // dC~^T = B~^T DGM^T + e^{Lam} E^T, E^T = H_in dY^T;  dB~^T = C~^T DGM + w F^T, F^T = dZ X^T  (N x V)
      f32x4 cacc[VNW], eacc[VNW], bacc[VNW], facc[VNW];
#pragma unroll
      for (int j = 0; j < VNW; ++j) cacc[j] = eacc[j] = bacc[j] = facc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (TL) {
        // B~ and C~ enter as bf16 hi + lo parts here: the angle adjoints take
        // differences of products that cancel to first order, and one bf16
        // rounding of B~, C~ would leave ~1e-2 relative error in dtheta
        mmv<NW, TN, TV, V>(rdTr(tB, LBN), rdTr(tDGt, LBV), cacc, wave, m16, g);
        mmv<NW, TN, TV, V>(rdTr(tBl, LBN), rdTr(tDGt, LBV), cacc, wave, m16, g);
        mmv<NW, TN, TV, P>(rdH, rdT(tDY, LBP), eacc, wave, m16, g);
        mmv<NW, TN, TV, V>(rdTr(tC, LBN), rdT(tDGt, LBV), bacc, wave, m16, g);
        mmv<NW, TN, TV, V>(rdTr(tCl, LBN), rdT(tDGt, LBV), bacc, wave, m16, g);
        mmv<NW, TN, TV, P>(rdTr(tDZt, LBN), rdT(tX, LBP), facc, wave, m16, g);
      } else {
        mm<NW, TN, TV, V>([&](int n, int s) { return sB[s * LDN + n]; },
                                 [&](int s, int v) { return sDG[v * LDV + s]; }, cacc, wave, m16, g);
        mm<NW, TN, TV, P>([&](int n, int p) { return hin(n, p); },
                               [&](int p, int v) { return sDY[v * LDP + p]; }, eacc, wave, m16, g);
        mm<NW, TN, TV, V>([&](int n, int t) { return sC[t * LDN + n]; },
                                 [&](int t, int s) { return sDG[t * LDV + s]; }, bacc, wave, m16, g);
        mm<NW, TN, TV, P>([&](int n, int p) { return sDZ[n * LDP + p]; },
                               [&](int p, int v) { return sX[v * LDP + p]; }, facc, wave, m16, g);
      }
      // Waves 0-3, while their products run: the masked decay's adjoints
      // (they need only dGM o G and the chunk's scalars, complete since the
      // last barrier; the per-token phase reads them two barriers on).
      if (tid < 256) {
        // dM on s < t and the diagonal; lane (t, s) = t QB + s. Row sums over s
        // (the QB lanes of a row) and partial column sums over the rows a wave
        // holds are formed with shuffles; the waves' column partials are added
        // by the per-token phase below.
        const int t = tid / QB, s = tid % QB;
        // the operands first (one wait), clamped to valid slots past QB x QB
        const int tq = tid < QB * QB ? t : 0;
        const float dm = sDM[tq][s], lam_t = sLam[tq], lam_s = sLam[s], q_s = sQ[s];
        float dmm = 0.0f, dme = 0.0f;
        if (tid < QB * QB) {
          if (s < t) {
            const float e = __expf(fminf(lam_t - lam_s, 0.0f));
            dme = dm * e;
            dmm = dme * q_s;
          } else if (s == t) {
            sDgam[t] = dm;
          }
        }
        float row = dmm, colL = dmm, colQ = dme;
        row = lane_sum<1, QB>(row);
        colL = lane_sum<QB, 64>(colL);
        colQ = lane_sum<QB, 64>(colQ);
        if (tid < QB * QB && s == 0) sDLam[t] = row;
        if (lane < QB) {
          sColL[wave][s] = colL;
          sColQ[wave][s] = colQ;
        }
      }
#pragma unroll
      for (int j = 0; j < VNW; ++j) {
        const int ti = wave + NW * j;
        if (ti < TN * TV) {
          const int tr = ti / TV, tc = ti % TV, v = tc * 16 + m16, t = v / R, n0 = tr * 16 + 4 * g, k0 = n0 / 2;
          const float el = sEL[t], wt = sW[t];
          const float4 bq = *(const float4*)&sB[v * LDN + n0], cq = *(const float4*)&sC[v * LDN + n0];
          const float bS[4] = {bq.x, bq.y, bq.z, bq.w}, cS[4] = {cq.x, cq.y, cq.z, cq.w};
          float dCt[4], dBt[4], de = 0.0f, dw = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dCt[i] = cacc[j][i] + el * eacc[j][i];
            dBt[i] = bacc[j][i] + wt * facc[j][i];
            de += cS[i] * eacc[j][i];
            dw += bS[i] * facc[j][i];
          }
          // sums over n: the lane's 4 features, then the 4 lane groups
          de = lane_sum<16, 64>(de);
          dw = lane_sum<16, 64>(dw);
          if (g == 0) {
            sDeP[tr][v] = de;
            sDwP[tr][v] = dw;
          }
          // per pair (u, w) = features (n0 + 2q, n0 + 2q + 1): the angle
          // adjoint du w - dw u, and the un-rotated gradients
          // R(phi) (du, dw) = (c du - s dw, s du + c dw)
          const float2 cs0 = sCS[k0][t], cs1 = sCS[k0 + 1][t];
          const float cs[2][2] = {{cs0.x, cs0.y}, {cs1.x, cs1.y}};
          float gB[4], gC[4], dph[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int u = 2 * q, w = 2 * q + 1;
            dph[q] = dBt[u] * bS[w] - dBt[w] * bS[u] + dCt[u] * cS[w] - dCt[w] * cS[u];
            gB[u] = cs[q][0] * dBt[u] - cs[q][1] * dBt[w];
            gB[w] = cs[q][1] * dBt[u] + cs[q][0] * dBt[w];
            gC[u] = cs[q][0] * dCt[u] - cs[q][1] * dCt[w];
            gC[w] = cs[q][1] * dCt[u] + cs[q][0] * dCt[w];
          }
          {
            uint32_t off = (uint32_t)t * Hu * (R * N) + (uint32_t)((v % R) * N + n0);
            fresh(off);
            store4_rs<T>(rdB, off, gB);
            store4_rs<T>(rdC, off, gC);
          }
          // the token's angle adjoint sums its R ranks (R adjacent lanes)
          dph[0] = lane_sum<1, R>(dph[0]);
          dph[1] = lane_sum<1, R>(dph[1]);
          if (m16 % R == 0) {
            sDphi[k0][t] = dph[0];
            sDphi[k0 + 1][t] = dph[1];
          }
        }
      }
    }
    {
      // dH_in += C~^T (e^{Lam} dY)
      if constexpr (TL) {
        mmv<NW, TN, TP, V>(rdTr(tC, LBN), rdELDY, Gb, wave, m16, g);
      } else {
        mm<NW, TN, TP, V>([&](int n, int v) { return sC[v * LDN + n]; },
                                 [&](int v, int p) { return sEL[v / R] * sDY[v * LDP + p]; }, Gb, wave, m16, g);
      }
    }
    __syncthreads();

    // ---------------- angle adjoints of the chunk ----------------
    {
      // d omega_t = sum_{i >= t} dphi_i + dTheta; dtheta = dt d omega.
      // Lane e = k QB + t: the suffix sum over t runs within QB lanes with
      // shuffles; theta_t . d omega_t is summed over the wave's pairs k here
      // and over the waves by the per-token phase.
      // Every LDS operand of the wave's items is read before any of them is
      // used, so that the reads share one wait instead of one each.
      constexpr int NIT = (QB * K + TH - 1) / TH;
      float rphi[NIT], rth[NIT], rd[NIT], rtp[NIT][TP];
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        int e = tid + TH * it;
        e = e < QB * K ? e : QB * K - 1;  // past the end: a valid slot, result unused
        const int t = e % QB, k = e / QB;
        rphi[it] = sDphi[k][t];
        rth[it] = sTh[k][t];
        rd[it] = sT[t].d;
#pragma unroll
        for (int tc = 0; tc < TP; ++tc) rtp[it][tc] = sDThP[tc][k];
      }
      float thd = 0.0f;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int e = tid + TH * it;
        if (e >= QB * K) break;  // QB K is a multiple of 64: whole waves
        const int t = e % QB, k = e / QB;
        float dom = rphi[it];
        // suffix sum over the token's QB-lane group
        {
          float u = row_down<1>(dom);
          if (t + 1 < QB) dom += u;
          u = row_down<2>(dom);
          if (t + 2 < QB) dom += u;
          u = row_down<4>(dom);
          if (t + 4 < QB) dom += u;
          if constexpr (QB > 8) {
            u = row_down<8>(dom);
            if (t + 8 < QB) dom += u;
          }
        }
#pragma unroll
        for (int tc = 0; tc < TP; ++tc) dom += rtp[it][tc];
        uint32_t ot = (uint32_t)t * Hu * K + k;
        fresh(ot);
        if (a0 + t < L) (a.dtheta + t0c * K)[ot] = rd[it] * dom;
        thd += rth[it] * dom;
      }
      thd = lane_sum<QB, 64>(thd);
      if (lane < QB) sThP[wave][lane] = thd;  // zero for a wave without items
    }
    __syncthreads();
    // Per-token gradients: lane t < QB of wave 0, sums across tokens with
    // shuffles (no further barrier).
    if (tid < 64) {
      const int t = tid;
      const bool ok = t < QB;
      const int tt = ok ? t : 0;
      // Every LDS operand of the phase is read here, before any is used: the
      // reads then share one wait instead of one each (the sums below keep
      // their order).
      float rwp[R][TN], rep[R][TN], rcl[4], rcq[4], rrw[NW], rthp[NW];
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int tr = 0; tr < TN; ++tr) {
          rwp[r][tr] = sDwP[tr][tt * R + r];
          rep[r][tr] = sDeP[tr][tt * R + r];
        }
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        rcl[w] = sColL[w][tt];
        rcq[w] = sColQ[w][tt];
      }
#pragma unroll
      for (int w = 0; w < NW; ++w) rrw[w] = sRedW[w];
#pragma unroll
      for (int w = 0; w < NW; ++w) rthp[w] = sThP[w][tt];
      const TokScal ts = sT[tt];
      const float r_dlam = sDLam[tt], r_el = sEL[tt], r_w = sW[tt], r_lam = sLam[tt], r_dgam = sDgam[tt];
      float dwt = 0.0f, det = 0.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int tr = 0; tr < TN; ++tr) {
          dwt += rwp[r][tr];
          det += rep[r][tr];
        }
      }
      // w_t = e^{Lam_end - Lam_t} q_t; e^{Lam_t} of the inter-chunk output
      float cl = 0.0f, cq = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        cl += rcl[w];
        cq += rcq[w];
      }
      float dlam_t = ok ? r_dlam - cl + det * r_el - dwt * r_w : 0.0f;
      const float dq_t = ok ? cq + dwt * __expf(lamQ - r_lam) : 0.0f;
      // d Lam_end: e^{Lam_end} <dZ, H_in> plus every token's share through w
      float dlq = ok ? dwt * r_w : 0.0f;
      dlq = lane_sum<1, 16>(dlq);
      float dzh = 0.0f;  // <dZ, H_in>
#pragma unroll
      for (int w = 0; w < NW; ++w) dzh += rrw[w];
      if (t == QB - 1) dlam_t += dlq + eQ * dzh;
      // d(dt A)_t = sum_{i >= t} dLam_i
      float dda = dlam_t;
      {
        float u = row_down<1>(dda);
        if (t + 1 < QB) dda += u;
        u = row_down<2>(dda);
        if (t + 2 < QB) dda += u;
        u = row_down<4>(dda);
        if (t + 4 < QB) dda += u;
        u = row_down<8>(dda);
        if (t + 8 < QB) dda += u;
      }
      const float dq_prev = row_up<1>(dq_t);
      // d eps of the token after this chunk
      const float de_next = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dq_t), QB - 1));
      if (ok) {
        const float dgam = r_dgam + dq_t;           // q_t = gamma_t + eps_{t+1}
        const float deps = t > 0 ? dq_prev : 0.0f;  // eps_t weighs the previous token
        float ddt = ts.A * dda + ts.lam * dgam + (1.0f - ts.lam) * deps;
        const float dlam = ts.d * dgam - ts.d * deps;
        float thd = 0.0f;  // theta_t . d omega_t, the waves' partials in a fixed order
#pragma unroll
        for (int w = 0; w < NW; ++w) thd += rthp[w];
        ddt += thd;
        uint32_t tk = (uint32_t)t * Hu;
        fresh(tk);
        if (a0 + t < L) {
          (a.dA + t0c)[tk] = ts.d * dda;
          if (t > 0) {
            (a.ddt + t0c)[tk] = ddt;
            (a.dlam + t0c)[tk] = dlam;
          }
        }
        if (t == 0) {
          // finish the first token of the chunk processed before (it follows
          // this chunk's last token, whose q carries its eps), then hold this one
          const uint32_t tn = (uint32_t)QB * Hu;
          if (c + 1 < c_end) {
            (a.ddt + t0c)[tn] = pend_ddt + (1.0f - pend_l) * de_next;
            (a.dlam + t0c)[tn] = pend_dlam - pend_d * de_next;
          } else if (c + 1 < nch) {
            // that token opens the next segment, walked by another block: its
            // share from here goes to the boundary record
            const float dn = (a.dt + t0c)[tn], ln = (a.lam + t0c)[tn];
            float* bd = a.bnd + (bh * NS + seg + 1) * 4;
            bd[0] = (1.0f - ln) * de_next;
            bd[1] = -dn * de_next;
          }
          pend_ddt = ddt;
          pend_dlam = dlam;
          pend_d = ts.d;
          pend_l = ts.lam;
        }
      }
    }
    // No barrier here: the next chunk's staging writes the angles, the token
    // scalars and H_in. The per-token phase above (wave 0) reads none of
    // those but the token scalars, whose slot each lane rewrites itself after
    // reading it; every other read of them ended before the last barrier.
    // The other waves therefore stage the next chunk while wave 0 finishes.
    }
  }

  if (seg > 0) {
    // the segment's first token: its parts without the trapezoid weight it
    // gets from the segment before
    if (tid == 0) {
      float* bd = a.bnd + (bh * NS + seg) * 4;
      bd[2] = pend_ddt;
      bd[3] = pend_dlam;
    }
    return;
  }
  // ---------------- the state before the first token ----------------
  // H'_0 = h0 + eps_1 prev_B^T prev_x
  const bool has_prev = a.prev_B != nullptr;
  if (a.dh0) {
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      const int ti = wave + NW * j;
      if (ti < S::NPT) {
        const int tr = ti / TP, tc = ti % TP;
#pragma unroll
        for (int i = 0; i < 4; ++i) a.dh0[bh * (int64_t)N * P + (tr * 16 + 4 * g + i) * P + tc * 16 + m16] = Gb[j][i];
      }
    }
  }
  // dH'_0 to LDS for the prev products (HG: to the first checkpoint's slot in
  // global memory, which nothing reads any more; agent-scope fences around the
  // barrier make the other waves' writes visible past the L1, which may still
  // hold that slot's earlier contents)
  float* const hsc = HG ? a.ckpt + bh * (nch + 1) * (int64_t)(N * P) : sH;
  constexpr int LDH = HG ? P : LDP;
  if (has_prev) {
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      const int ti = wave + NW * j;
      if (ti < S::NPT) {
        const int tr = ti / TP, tc = ti % TP;
#pragma unroll
        for (int i = 0; i < 4; ++i) hsc[(tr * 16 + 4 * g + i) * LDH + tc * 16 + m16] = Gb[j][i];
      }
    }
  }
  if constexpr (HG) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if constexpr (HG) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (L > 0) {
    const float d1 = a.dt[tok_of(0)], l1 = a.lam[tok_of(0)];
    const float eps1 = has_prev ? (1.0f - l1) * d1 : 0.0f;
    if (has_prev) {
      // d eps_1 = <dH'_0, prev_B^T prev_x>; dprev_B = eps_1 dH'_0 prev_x; dprev_x = eps_1 dH'_0^T prev_B.
      // d eps_1 is summed in fp64 and in a fixed order (it can nearly cancel
      // against the first token's other dt and lam terms).
      double part = 0.0;
      for (int e = tid; e < N * P; e += TH) {
        const int n = e / P, p = e % P;
        float q0 = 0.0f;
        for (int r = 0; r < R; ++r)
          q0 += ld_io<T>(a.prev_B, (bh * R + r) * N + n) * ld_io<T>(a.prev_x, (bh * R + r) * P + p);
        part += (double)hsc[n * LDH + p] * (double)q0;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) part += __shfl_xor(part, o, 64);
      if (lane == 0) sRedD[wave] = part;
      if (a.dprev_B) {
        for (int e = tid; e < R * N; e += TH) {
          const int r = e / N, n = e % N;
          float acc = 0.0f;
          for (int p = 0; p < P; ++p) acc += hsc[n * LDH + p] * ld_io<T>(a.prev_x, (bh * R + r) * P + p);
          io<T>::store1(a.dprev_B, (bh * R + r) * N + n, eps1 * acc);
        }
        for (int e = tid; e < R * P; e += TH) {
          const int r = e / P, p = e % P;
          float acc = 0.0f;
          for (int n = 0; n < N; ++n) acc += hsc[n * LDH + p] * ld_io<T>(a.prev_B, (bh * R + r) * N + n);
          io<T>::store1(a.dprev_x, (bh * R + r) * P + p, eps1 * acc);
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      double de1d = 0.0;
      if (has_prev)
        for (int w = 0; w < NW; ++w) de1d += sRedD[w];
      const float de1 = (float)de1d;
      a.ddt[tok_of(0)] = pend_ddt + (1.0f - l1) * de1;
      a.dlam[tok_of(0)] = pend_dlam - d1 * de1;
    }
  }
}

// ---------------------------------------------------------------------------
// 3. (segments) scan of the state adjoint over the segments, last to first:
//    the adjoint at the end of segment j-1 is the one at the start of j, i.e.
//    its local start adjoint plus e^{Lam_j} R(-Theta_j) (adjoint at its end),
//    with Lam_j, Theta_j the segment's total log-decay and angle per pair.
//    One thread per (b,h, pair k, column p).
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(256) void bwd_seg_scan_kernel(BwdArgs a, int P) {
  constexpr int K = N / 2;
  const int64_t NS = a.S;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= a.batch * a.H * K * P) return;
  const int p = (int)(i % P), k = (int)((i / P) % K);
  const int64_t bh = i / ((int64_t)P * K), NP = (int64_t)N * P;
  const int64_t r0 = (int64_t)(2 * k) * P + p, r1 = r0 + P;
  float u = a.dh_final ? a.dh_final[bh * NP + r0] : 0.0f, v = a.dh_final ? a.dh_final[bh * NP + r1] : 0.0f;
  for (int64_t j = NS - 1; j >= 1; --j) {
    const float* tot = a.seg_tot + (bh * NS + j) * (1 + K);
    const float dec = expf(tot[0]);
    float sn, cs;
    sincosf(tot[1 + k], &sn, &cs);
    const float* D = a.dh_loc + (bh * NS + j) * NP;
    const float nu = D[r0] + dec * (cs * u + sn * v);
    const float nv = D[r1] + dec * (cs * v - sn * u);
    u = nu;
    v = nv;
    float* E = a.dh_end + (bh * NS + j - 1) * NP;
    E[r0] = u;
    E[r1] = v;
  }
}

// 4. (segments) the first token of every segment j >= 1: its dt and lam
//    gradients from its own segment plus the part of the segment before.
__global__ __launch_bounds__(256) void bwd_bnd_kernel(BwdArgs a, int QB) {
  const int64_t NS = a.S;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= a.batch * a.H * (NS - 1)) return;
  const int64_t bh = i / (NS - 1), seg = 1 + i % (NS - 1), b = bh / a.H, h = bh % a.H;
  const int64_t t = seg * a.cps * QB;
  if (t >= a.L) return;
  const float* bd = a.bnd + (bh * NS + seg) * 4;
  const int64_t tk = (b * a.L + t) * a.H + h;
  a.ddt[tk] = bd[2] + bd[0];
  a.dlam[tk] = bd[3] + bd[1];
}

template <typename T, int N, int P, int R>
static hipError_t bwd_run(const BwdArgs& a, hipStream_t s) {
  const int64_t BH = a.batch * a.H;
  if (a.S <= 1) {
    const dim3 grid((unsigned)BH);
    hipLaunchKernelGGL((bwd_ckpt_kernel<T, N, P, R>), grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL((bwd_chunk_kernel<T, N, P, R>), grid, dim3(512), 0, s, a);
    return hipGetLastError();
  }
  // segments: the forward states at segment starts (local walks and a scan),
  // the checkpoints, the state adjoint at segment ends (local reverse walks
  // and a scan), then every segment's reverse walk and the boundary tokens
  const dim3 grid((unsigned)(BH * a.S));
  BwdArgs l = a;
  l.ckpt_local = 1;
  hipLaunchKernelGGL((bwd_ckpt_kernel<T, N, P, R>), grid, dim3(256), 0, s, l);
  WalkArgs w{};
  w.batch = a.batch; w.H = a.H; w.S = a.S;
  w.seg_end = a.seg_end; w.seg_tot = a.seg_tot; w.seg_in = a.seg_in; w.h_final = nullptr;
  hipError_t e = launch_seg_scan(N, P, w, s);
  if (e != hipSuccess) return e;
  BwdArgs f = a;
  f.ckpt_local = 0;
  hipLaunchKernelGGL((bwd_ckpt_kernel<T, N, P, R>), grid, dim3(256), 0, s, f);
  hipLaunchKernelGGL((bwd_dh_kernel<T, N, P, R>), grid, dim3(256), 0, s, f);
  const int64_t nt = BH * (N / 2) * P;
  hipLaunchKernelGGL((bwd_seg_scan_kernel<N>), dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, s, f, P);
  hipLaunchKernelGGL((bwd_chunk_kernel<T, N, P, R>), grid, dim3(512), 0, s, f);
  const int64_t nb = BH * (a.S - 1);
  hipLaunchKernelGGL(bwd_bnd_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, f, BS<N, P, R>::QB);
  return hipGetLastError();
}

template <typename T, int N, int P>
static hipError_t bwd_r(const BwdArgs& a, hipStream_t s) {
  switch (a.R) {
    case 1: return bwd_run<T, N, P, 1>(a, s);
    case 2: return bwd_run<T, N, P, 2>(a, s);
    case 4: return bwd_run<T, N, P, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int N>
static hipError_t bwd_p(int P, const BwdArgs& a, hipStream_t s) {
  switch (P) {
    case 16: return bwd_r<T, N, 16>(a, s);
    case 32: return bwd_r<T, N, 32>(a, s);
    case 64: return bwd_r<T, N, 64>(a, s);
    case 128: return bwd_r<T, N, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t bwd_n(int N, int P, const BwdArgs& a, hipStream_t s) {
  switch (N) {
    case 16: return bwd_p<T, 16>(P, a, s);
    case 32: return bwd_p<T, 32>(P, a, s);
    case 64: return bwd_p<T, 64>(P, a, s);
    case 128: return bwd_p<T, 128>(P, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chunked_bwd(int io_bf16, int N, int P, const BwdArgs& a, hipStream_t s) {
  if (a.batch * a.H == 0 || a.L == 0) return hipSuccess;
  if (!bwd_supported(N, P, a.R)) return hipErrorInvalidValue;
  return io_bf16 ? bwd_n<bf16_t>(N, P, a, s) : bwd_n<float>(N, P, a, s);
}

}  // namespace m3
