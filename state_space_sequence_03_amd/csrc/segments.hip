// Sequence segments walked in parallel (one GPU's version of splitting a long
// sequence): when B*H is too small to fill the chip, each (b,h) sequence is cut
// into S segments of whole chunks and every segment is walked from a zero
// state by its own block (chunk.hip / chunk_fast.hip).  The recurrence is
// linear in the state (linkstar.cloud/article/869, "第一刀": h_t = alpha_t
// h_{t-1} + ...), so the true outputs and states follow from two corrections:
//
//  1. segment scan: the true state entering segment j+1 is
//         H_{j+1} = E_j + exp(Lam_j) R(Theta_j) H_j,   H_1 = E_0,
//     with E_j the end state of segment j walked from zero, Lam_j its total
//     log-decay and Theta_j its total angle per pair (the rotation of the
//     complex state, "第二刀").  The last one is h_final.
//  2. fix-up: for a token t of segment j >= 1,
//         y_t += exp(Lam^seg_t) (R(-phi^seg_t) C_t)^T H_j,
//     Lam^seg and phi^seg cumulated from the segment start (chunk offsets
//     stored by the walker plus a chunk-local wave scan).  A chunk whose
//     decay factors are all exactly zero in fp32 adds exactly nothing and is
//     skipped.
//
// The token before each segment (its trapezoid term) is already folded into
// that segment's zero-state walk.
#include "m3_common.hpp"
#include "m3_launch.hpp"

namespace m3 {

// One thread per (b,h, pair k, column p); sequential over segments.
template <int N>
__global__ __launch_bounds__(256) void seg_scan_kernel(WalkArgs a, int P) {
  constexpr int K = N / 2;
  const int64_t S = a.S;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t total = a.batch * a.H * K * P;
  if (i >= total) return;
  const int p = (int)(i % P);
  const int k = (int)((i / P) % K);
  const int64_t bh = i / ((int64_t)P * K);
  const int64_t NP = (int64_t)N * P;
  const int64_t r0 = (int64_t)(2 * k) * P + p, r1 = r0 + P;
  const float* E = a.seg_end + bh * S * NP;
  float u = E[r0], v = E[r1];  // true end of segment 0
  for (int64_t j = 1; j < S; ++j) {
    float* hin = a.seg_in + (bh * S + j) * NP;
    hin[r0] = u;
    hin[r1] = v;
    const float* tot = a.seg_tot + (bh * S + j) * (1 + K);
    const float dec = expf(tot[0]);
    float sn, cs;
    sincosf(tot[1 + k], &sn, &cs);
    const float* Ej = E + j * NP;
    const float nu = Ej[r0] + dec * (cs * u - sn * v);
    const float nv = Ej[r1] + dec * (sn * u + cs * v);
    u = nu;
    v = nv;
  }
  if (a.h_final) {
    a.h_final[bh * NP + r0] = u;
    a.h_final[bh * NP + r1] = v;
  }
}

// One block of 256 threads per chunk of a segment j >= 1.
//   grid.x = chunk index within the sequence, grid.y = b*H + h.
template <typename T, int N, int P>
__global__ __launch_bounds__(256) void seg_fixup_kernel(WalkArgs a) {
  constexpr int K = N / 2;
  constexpr int NKS = (N + 31) / 32;
  constexpr int PT = P / 16;
  const int64_t c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int Q = a.Q, R = a.R, V = Q * R;
  const int lgR = R == 4 ? 2 : (R == 2 ? 1 : 0);
  const int64_t c0 = c * Q;
  const int64_t seg = c0 / a.seg_len;
  if (seg == 0 || c0 >= a.L) return;
  const int64_t L = a.L, H = a.H;
  const int nvalid = (int)((L - c0) < Q ? (L - c0) : Q);
  const int64_t nchunks = (L + Q - 1) / Q;
  const float* meta = a.chunk_meta + (bh * nchunks + c) * (1 + K);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, g = lane >> 4;

  __shared__ float sL[64];               // exp(Lam^seg_t)
  __shared__ float sPhi[64][K + 1];      // phi^seg_t
  __shared__ __align__(16) u16 sHt[P][N + 8];  // H_j^T, bf16
  __shared__ int sAny;

  // chunk-local log-decay scan (wave 0) and decision
  if (wave == 0) {
    const bool tv = lane < nvalid;
    const int64_t ts = (b * L + c0 + (tv ? lane : 0)) * H + h;
    const float la = tv ? a.dt[ts] * a.A[ts] : 0.0f;
    const float lam = wave_incl_scan(la) + meta[0];
    const float e = tv ? expf(lam) : 0.0f;
    sL[lane] = e;
    const unsigned long long nz = __ballot(e != 0.0f);
    if (lane == 0) sAny = nz != 0ull;
  }
  __syncthreads();
  if (!sAny) return;  // every factor is exactly zero: nothing to add

  // angles: wave w scans pairs k = w, w + 4, ...
  for (int k = wave; k < K; k += 4) {
    const bool tv = lane < nvalid;
    const int64_t ts = (b * L + c0 + (tv ? lane : 0)) * H + h;
    const float om = tv ? a.dt[ts] * a.theta[ts * K + k] : 0.0f;
    sPhi[lane][k] = wave_incl_scan(om) + meta[1 + k];
  }
  // incoming true state of the segment, transposed to (p, n), bf16
  const float* hin = a.seg_in + (bh * a.S + seg) * (int64_t)N * P;
  for (int i = tid; i < N * P; i += 256) {
    const int n = i / P, p = i % P;
    sHt[p][n] = f2bf(hin[i]);
  }
  __syncthreads();

  // each wave: column tiles ct = wave, wave + 4, ... of the V virtual rows
  for (int ct = wave; ct < V / 16; ct += 4) {
    const int v = ct * 16 + m16;
    const int t = v >> lgR;
    const bool ok = t < nvalid;
    const int64_t crow = ((b * L + c0 + (ok ? t : 0)) * H + h) * (int64_t)R * N + (v & (R - 1)) * N;
    uint4 cf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float f[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = ks * 32 + (q < 2 ? 4 * g + 2 * q : 16 + 4 * g + 2 * (q - 2));
        float u = 0.0f, w = 0.0f, sn = 0.0f, cs = 1.0f;
        if (ok && n < N) {
          u = io<T>::load1(a.C, crow + n);
          w = io<T>::load1(a.C, crow + n + 1);
          sincosf(sPhi[t][n / 2], &sn, &cs);
        }
        f[2 * q] = cs * u + sn * w;          // R(-phi) applied to (u, w)
        f[2 * q + 1] = cs * w - sn * u;
      }
      cf[ks] = make_uint4(pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]), pack_bf2(f[4], f[5]), pack_bf2(f[6], f[7]));
    }
    const float el = ok ? sL[t] : 0.0f;
    const int64_t yrow = ((b * L + c0 + (ok ? t : 0)) * H + h) * (int64_t)R * P + (v & (R - 1)) * P;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u16* hr = &sHt[pt * 16 + m16][ks * 32];
        const uint2 lo = *(const uint2*)(hr + 4 * g);
        const uint2 hi = (ks * 32 + 16 < N) ? *(const uint2*)(hr + 16 + 4 * g) : make_uint2(0, 0);
        acc = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), as_bf16x8(cf[ks]), acc);
      }
      if (ok && el != 0.0f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t yi = yrow + pt * 16 + 4 * g + i;
          io<T>::store1(a.y, yi, io<T>::load1(a.y, yi) + el * acc[i]);
        }
      }
    }
  }
}


// Fix-up for bf16 io with P = 64 and N in {64, 128} (the shapes of the
// sub-chunk walker): one 256-thread block per (b,h, segment j >= 1) walks the
// segment's chunks in order and stops at the first chunk whose decay factors
// exp(Lam^seg_t) are all exactly zero in fp32: Lam^seg only decreases, so
// every later factor is zero too and adds exactly nothing.  H_j is staged
// once per block as bf16 H_j^T; C is rotated through a per-chunk (cos, sin)
// table with two bf16 dot products per pair, as in the walker; y is updated
// with 32-byte read-modify-writes after a transpose across the wave's rows.
template <int N, int R>
__global__ __launch_bounds__(256) void seg_fixup_walk_kernel(WalkArgs a) {
  constexpr int P = 64, K = N / 2, NKS = N / 32, CPR = N / 8;
  constexpr int lgR = R == 4 ? 2 : (R == 2 ? 1 : 0);
  const int Q = a.Q, V = Q * R;  // Q <= 64
  const int64_t S = a.S;
  const int64_t bh = blockIdx.x / (S - 1), seg = 1 + blockIdx.x % (S - 1);
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t L = a.L, H = a.H;
  const int64_t t0 = seg * a.seg_len;
  const int64_t t1 = (t0 + a.seg_len < L) ? t0 + a.seg_len : L;
  const int64_t nchunks = (L + Q - 1) / Q;
  auto tokS = [&](int64_t tok) { return (b * L + tok) * H + h; };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, g = lane >> 4;

  __shared__ __align__(16) unsigned char sHt[P * 2 * N];   // H_j^T bf16 [P][N], swizzled rows of 2N bytes
  __shared__ __align__(16) unsigned char sCS[64 * 4 * K];  // (cos, sin) bf16 [Q][K], swizzled rows of 2N bytes
  __shared__ float sL[64];                                 // exp(Lam^seg_t)
  __shared__ int sAny;

  // incoming true state of the segment, transposed to (p, n), bf16
  {
    const float* hin = a.seg_in + (bh * S + seg) * (int64_t)(N * P);
    for (int i = tid; i < N * P / 4; i += 256) {
      const int n = (4 * i) / P, p0 = (4 * i) % P;
      const float4 v = *(const float4*)(hin + 4 * i);
      const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(u16*)(sHt + swz<CPR>(p0 + j, n >> 3) + 2 * (n & 7)) = f2bf(f[j]);
    }
  }

  for (int64_t c0 = t0; c0 < t1; c0 += Q) {
    const int nvalid = (int)((t1 - c0) < Q ? (t1 - c0) : Q);
    const float* meta = a.chunk_meta + (bh * nchunks + c0 / Q) * (1 + K);
    if (wave == 0) {  // decay factors from the segment start, lane = token
      const bool tv = lane < nvalid;
      const int64_t ts = tokS(c0 + (tv ? lane : 0));
      const float la = tv ? a.dt[ts] * a.A[ts] : 0.0f;
      const float e = tv ? expf(wave_incl_scan(la) + meta[0]) : 0.0f;
      sL[lane] = e;
      const unsigned long long nz = __ballot(e != 0.0f);
      if (lane == 0) sAny = nz != 0ull;
    }
    // angles from the segment start: waves take pairs k = wave, wave + 4, ...
    for (int k = wave; k < K; k += 4) {
      const bool tv = lane < nvalid;
      const int64_t ts = tokS(c0 + (tv ? lane : 0));
      const float om = tv ? a.dt[ts] * a.theta[ts * K + k] : 0.0f;
      float sn, cs;
      fast_sincos(wave_incl_scan(om) + meta[1 + k], &sn, &cs);
      if (lane < Q) *(uint32_t*)(sCS + swz<CPR>(lane, k >> 2) + 4 * (k & 3)) = pack_bf2(cs, sn);
    }
    __syncthreads();  // H_j^T (first chunk), the table and the factors are in LDS
    if (!sAny) break;  // every factor from here to the segment end is exactly zero

    // waves take column tiles ct = wave, wave + 4, ... of the V virtual rows
    for (int ct = wave; ct < V / 16; ct += 4) {
      const int v = ct * 16 + m16;
      const bool ok = (v >> lgR) < nvalid;
      const int t = ok ? (v >> lgR) : 0;
      const u16* crow = (const u16*)a.C + tokS(c0 + t) * (R * N) + (v & (R - 1)) * N + 8 * g;
      uint4 cf[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 raw = *(const uint4*)(crow + ks * 32);
        const uint4 tb = *(const uint4*)(sCS + swz<CPR>(t, 4 * ks + g));
        const uint32_t tw[4] = {tb.x, tb.y, tb.z, tb.w};
        const uint32_t cw[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t ms = __builtin_amdgcn_alignbit(tw[j], tw[j], 16) ^ 0x8000u;  // (-sin, cos)
          const float o0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, cw[j]),
                                                           __builtin_bit_cast(bf16x2, tw[j]), 0.0f, false);
          const float o1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, cw[j]),
                                                           __builtin_bit_cast(bf16x2, ms), 0.0f, false);
          o[j] = pack_bf2(o0, o1);
        }
        cf[ks] = make_uint4(o[0], o[1], o[2], o[3]);
      }
      // (H_j^T C~^T)[p][v] for the 4 p tiles, scaled by exp(Lam^seg_t)
      const float el = ok ? sL[t] : 0.0f;
      uint32_t d[4][4];  // [i][pt]: p = 16 pt + 4g + i
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint4 hf = *(const uint4*)(sHt + swz<CPR>(pt * 16 + m16, 4 * ks + g));
          acc = mfma_bf16(as_bf16x8(hf), as_bf16x8(cf[ks]), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i][pt] = __float_as_uint(el * acc[i]);
      }
      // after the transpose lane (m16, g) holds p = 16g + 4k + i in d[i][k]
#pragma unroll
      for (int i = 0; i < 4; ++i) transpose_rows4(d[i]);
      if (ok && el != 0.0f) {
        u16* yrow = (u16*)a.y + tokS(c0 + t) * (R * P) + (v & (R - 1)) * P + 16 * g;
        const uint4 y0 = *(const uint4*)yrow, y1 = *(const uint4*)(yrow + 8);
        const uint32_t yw[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
        uint32_t ow[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {  // elements p = 16g + 4k .. 4k + 3
          ow[2 * k] = pack_bf2(bf_lo(yw[2 * k]) + __uint_as_float(d[0][k]), bf_hi(yw[2 * k]) + __uint_as_float(d[1][k]));
          ow[2 * k + 1] = pack_bf2(bf_lo(yw[2 * k + 1]) + __uint_as_float(d[2][k]),
                                   bf_hi(yw[2 * k + 1]) + __uint_as_float(d[3][k]));
        }
        *(uint4*)yrow = make_uint4(ow[0], ow[1], ow[2], ow[3]);
        *(uint4*)(yrow + 8) = make_uint4(ow[4], ow[5], ow[6], ow[7]);
      }
    }
    __syncthreads();  // the table and the factors are rewritten for the next chunk
  }
}

template <int N>
static hipError_t seg_p(int io_bf16, int P, const WalkArgs& a, hipStream_t s) {
  const int64_t nchunks = (a.L + a.Q - 1) / a.Q;
  const dim3 grid((unsigned)nchunks, (unsigned)(a.batch * a.H));
  const int64_t threads = a.batch * a.H * (N / 2) * P;
  hipLaunchKernelGGL((seg_scan_kernel<N>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a, P);
  if constexpr (N == 64 || N == 128) {
    if (io_bf16 && P == 64 && a.Q <= 64 && (a.R == 2 || a.R == 4 || (N == 64 && a.R == 1))) {
      const dim3 g2((unsigned)(a.batch * a.H * (a.S - 1)));
      if (a.R == 4) hipLaunchKernelGGL((seg_fixup_walk_kernel<N, 4>), g2, dim3(256), 0, s, a);
      else if (a.R == 2) hipLaunchKernelGGL((seg_fixup_walk_kernel<N, 2>), g2, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((seg_fixup_walk_kernel<N, 1>), g2, dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
#define M3_FIX(TT, PP) hipLaunchKernelGGL((seg_fixup_kernel<TT, N, PP>), grid, dim3(256), 0, s, a)
  if (io_bf16) {
    switch (P) {
      case 16: M3_FIX(bf16_t, 16); break;
      case 32: M3_FIX(bf16_t, 32); break;
      case 64: M3_FIX(bf16_t, 64); break;
      case 128: M3_FIX(bf16_t, 128); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (P) {
      case 16: M3_FIX(float, 16); break;
      case 32: M3_FIX(float, 32); break;
      case 64: M3_FIX(float, 64); break;
      case 128: M3_FIX(float, 128); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef M3_FIX
  return hipGetLastError();
}

template <int N>
static hipError_t seg_scan_only(int P, const WalkArgs& a, hipStream_t s) {
  const int64_t total = a.batch * a.H * (N / 2) * P;
  hipLaunchKernelGGL((seg_scan_kernel<N>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, P);
  return hipGetLastError();
}

hipError_t launch_seg_scan(int N, int P, const WalkArgs& a, hipStream_t s) {
  switch (N) {
    case 16: return seg_scan_only<16>(P, a, s);
    case 32: return seg_scan_only<32>(P, a, s);
    case 64: return seg_scan_only<64>(P, a, s);
    case 128: return seg_scan_only<128>(P, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_segment_fixups(int io_bf16, int N, int P, const WalkArgs& a, hipStream_t s) {
  switch (N) {
    case 16: return seg_p<16>(io_bf16, P, a, s);
    case 32: return seg_p<32>(io_bf16, P, a, s);
    case 64: return seg_p<64>(io_bf16, P, a, s);
    case 128: return seg_p<128>(io_bf16, P, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m3
