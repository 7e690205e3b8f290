// One-token state update (decode), fused and HBM-streaming.
//
// Per (b,h), with eps = (1 - lam) dt, alpha = exp(dt A), gamma = lam dt and
// w_k = dt theta[k] (linkstar.cloud/article/869, "第一刀" for alpha/beta/gamma,
// "第二刀" for the 2x2 rotations, "第三刀" for the rank-R products):
//     h <- alpha R(w) [h + eps prev_B^T prev_x] + gamma B^T x,   y = C^T h.
// The state stays in the un-rotated ("true") frame, so no angle is carried
// between calls.  The fp32 state (N x P per (b,h)) is read once and written
// once; everything else is small.
//
// Mapping: one 256-thread block per (b,h).  A work item is one rotation pair
// (rows 2k, 2k+1) x 4 consecutive columns; consecutive threads take
// consecutive column groups, so each row is read as one contiguous run and the
// rotation never leaves registers.  The state loads are issued first, before
// the small inputs are staged; y = C^T h is reduced with wave shuffles, then
// across the four waves in LDS.
#include "m3_common.hpp"
#include "m3_lanes.hpp"
#include "m3_launch.hpp"

namespace m3 {

template <typename T, int N, int P, int R>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeArgs a) {
  constexpr int K = N / 2;
  constexpr int CG = P / 4;                 // column groups of 4 (divides 64)
  constexpr int ITEMS = K * CG;
  constexpr int PER = (ITEMS + 255) / 256;  // items per thread
  constexpr int RMAX = R;
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // the state is the only large stream: issue its loads before anything else
  float* st = a.state + bh * (int64_t)N * P;
  const int c = tid % CG;  // items tid + 256 q share the column group (CG divides 256)
  f32x4 h0[PER], h1[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid + 256 * q;
    if (i < ITEMS) {
      const int k = i / CG;
      h0[q] = *(const f32x4*)(st + (2 * k) * P + 4 * c);
      h1[q] = *(const f32x4*)(st + (2 * k + 1) * P + 4 * c);
    }
  }

  __shared__ float sB[RMAX][N], sC[RMAX][N], sPB[RMAX][N];
  __shared__ float2 sCS[K];
  __shared__ float red[4][RMAX * P];

  const float d = a.dt[bh], lam = a.lam[bh];
  const float alpha = expf(d * a.A[bh]);
  // without a previous token its term is absent: weight 0, and the current
  // token's own buffers stand in as (finite) operands so that no load is
  // conditional
  const bool has_prev = a.prev_B != nullptr;
  const float eps = has_prev ? (1.0f - lam) * d : 0.0f, gam = lam * d;
  const void* pB = has_prev ? a.prev_B : a.B;
  const void* px = has_prev ? a.prev_x : a.x;
  for (int k = tid; k < K; k += 256) {
    float s, co;
    sincosf(d * a.theta[bh * K + k], &s, &co);
    sCS[k] = make_float2(co, s);
  }
  for (int i = tid; i < R * N; i += 256) {
    const int r = i / N, n = i % N;
    sB[r][n] = io<T>::load1(a.B, bh * R * N + i);
    sC[r][n] = io<T>::load1(a.C, bh * R * N + i);
    sPB[r][n] = io<T>::load1(pB, bh * R * N + i);
  }
  float xv[RMAX][4], pxv[RMAX][4];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    io<T>::load4(a.x, (bh * R + r) * P + 4 * c, xv[r]);
    io<T>::load4(px, (bh * R + r) * P + 4 * c, pxv[r]);
  }
  __syncthreads();

  float yp[RMAX][4];
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) yp[r][j] = 0.0f;

#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid + 256 * q;
    if (i < ITEMS) {
      const int k = i / CG;
      const float2 cs = sCS[k];
      const float u0[4] = {h0[q][0], h0[q][1], h0[q][2], h0[q][3]};
      const float u1[4] = {h1[q][0], h1[q][1], h1[q][2], h1[q][3]};
      float n0[4], n1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float pin0 = 0.0f, pin1 = 0.0f, cin0 = 0.0f, cin1 = 0.0f;
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
          if (r < R) {
            pin0 += sPB[r][2 * k] * pxv[r][j];
            pin1 += sPB[r][2 * k + 1] * pxv[r][j];
            cin0 += sB[r][2 * k] * xv[r][j];
            cin1 += sB[r][2 * k + 1] * xv[r][j];
          }
        }
        // h <- alpha R(w) [h + eps prev_B^T prev_x] + gamma B^T x
        const float v0 = u0[j] + eps * pin0, v1 = u1[j] + eps * pin1;
        n0[j] = alpha * (cs.x * v0 - cs.y * v1) + gam * cin0;
        n1[j] = alpha * (cs.y * v0 + cs.x * v1) + gam * cin1;
#pragma unroll
        for (int r = 0; r < RMAX; ++r)
          if (r < R) yp[r][j] += sC[r][2 * k] * n0[j] + sC[r][2 * k + 1] * n1[j];
      }
      *(f32x4*)(st + (2 * k) * P + 4 * c) = f32x4{n0[0], n0[1], n0[2], n0[3]};
      *(f32x4*)(st + (2 * k + 1) * P + 4 * c) = f32x4{n1[0], n1[1], n1[2], n1[3]};
    }
  }
  // y[r][p] = sum over pairs: lanes of one wave with the same column group
  // differ in the bits >= log2(CG) of the lane id
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = yp[r][j];
      yp[r][j] = lane_sum<CG, 64>(v);
    }
  if (lane < CG) {
#pragma unroll
    for (int r = 0; r < RMAX; ++r)
      if (r < R)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave][r * P + 4 * c + j] = yp[r][j];
  }
  __syncthreads();
  for (int o = tid; o < R * P; o += 256) {
    const float s = red[0][o] + red[1][o] + red[2][o] + red[3][o];
    io<T>::store1(a.y, bh * R * P + o, s);
  }
}

// Short sequences (the chunked forward with at most TOKENS_MAX tokens per
// call, e.g. the k draft tokens of a verify step): the one-token update above
// applied to each token in turn while the state stays in registers, so the
// fp32 state is read once (h0) and written once (h_final) per call.
//
// Mapping: one 256-thread block per (b,h); wave w owns the columns
// [w P/4, (w+1) P/4) of every state row, lane (pg, cq) the 4 columns 4cq ..
// of that slice in the rotation pairs pg, pg + PG, ...  y_t = C_t^T h_t sums
// over pairs only, i.e. over the lanes of one wave: the token loop has no
// barrier.  Every token's B, C, x (raw, io dtype), (cos, sin) and scalars are
// staged in LDS once, up front, with all their loads in flight together.  The
// input term B_t^T x_t of the lane's elements is kept for the next token,
// whose trapezoid term is exactly that product (prev_B^T prev_x).
template <typename T>
struct lds_elem;
template <>
struct lds_elem<bf16_t> {
  typedef u16 E;
  __device__ static float2 pair(const E* p) {
    const uint32_t v = *(const uint32_t*)p;
    return make_float2(bf_lo(v), bf_hi(v));
  }
  __device__ static void quad(const E* p, float* f) {
    const uint2 v = *(const uint2*)p;
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  }
};
template <>
struct lds_elem<float> {
  typedef float E;
  __device__ static float2 pair(const E* p) { return *(const float2*)p; }
  __device__ static void quad(const E* p, float* f) {
    const float4 v = *(const float4*)p;
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
};

// One exchange step over lane bit M of a reduce-scatter of n values (lanes
// with the bit set keep the upper half), recursing until M reaches 64.
template <int n, int M>
__device__ __forceinline__ void reduce_scatter_step(float* v, int lane, int& base) {
  if constexpr (M < 64) {
    const bool up = (lane & M) != 0;
    if constexpr (n > 1) {
      constexpr int half = n / 2;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const float keep = up ? v[half + i] : v[i], send = up ? v[i] : v[half + i];
        v[i] = keep + __shfl_xor(send, M, 64);
      }
      base += up ? half : 0;
      reduce_scatter_step<half, 2 * M>(v, lane, base);
    } else {
      v[0] += __shfl_xor(v[0], M, 64);
      reduce_scatter_step<1, 2 * M>(v, lane, base);
    }
  }
}

template <typename T, int N, int P, int R>
__global__ __launch_bounds__(256) void decode_tokens_kernel(TokensArgs a) {
  constexpr int K = N / 2;
  constexpr int PW = P / 4;                  // columns per wave
  constexpr int CQ = PW / 4;                 // column quads per wave (1 .. 8)
  constexpr int PG = 64 / CQ;                // pair groups per wave
  constexpr int PPL = (K + PG - 1) / PG;     // pairs per lane
  constexpr int EV = 16 / io<T>::BYTES;      // elements per 16-byte copy
  typedef typename lds_elem<T>::E E;
  const int64_t bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cq = lane % CQ, pg = lane / CQ;
  const int col0 = wave * PW + 4 * cq;
  const int L = (int)a.L;  // 1 .. TOKENS_MAX
  auto tok_of = [&](int t) { return (b * a.L + t) * a.H + h; };

  __shared__ __align__(16) E sB[TOKENS_MAX][R * N], sC[TOKENS_MAX][R * N], sX[TOKENS_MAX][R * P];
  __shared__ float2 sCS[TOKENS_MAX][K];
  __shared__ float4 sS[TOKENS_MAX];  // alpha, eps, gamma

  // state rows 2k, 2k + 1 (k = pg + PG u), columns col0 .. col0 + 3
  f32x4 s0[PPL], s1[PPL];
  const float* st_in = a.h0 ? a.h0 + bh * (int64_t)N * P : nullptr;
#pragma unroll
  for (int u = 0; u < PPL; ++u) {
    const int k = pg + PG * u;
    s0[u] = s1[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (st_in && k < K) {
      s0[u] = *(const f32x4*)(st_in + (2 * k) * P + col0);
      s1[u] = *(const f32x4*)(st_in + (2 * k + 1) * P + col0);
    }
  }

  // stage every token: raw 16-byte copies of B, C and x; (cos, sin); scalars
  {
    constexpr int UB = R * N / EV, UX = R * P / EV;  // 16-byte units per token
    for (int e = tid; e < L * UB; e += 256) {
      const int t = e / UB, o = e % UB;
      const int64_t g = tok_of(t) * (R * N) + o * EV;
      *(uint4*)&sB[t][o * EV] = *(const uint4*)((const E*)a.B + g);
      *(uint4*)&sC[t][o * EV] = *(const uint4*)((const E*)a.C + g);
    }
    for (int e = tid; e < L * UX; e += 256) {
      const int t = e / UX, o = e % UX;
      *(uint4*)&sX[t][o * EV] = *(const uint4*)((const E*)a.x + tok_of(t) * (R * P) + o * EV);
    }
    for (int e = tid; e < L * K; e += 256) {
      const int t = e / K, k = e % K;
      const int64_t tok = tok_of(t);
      float sn, cs;
      sincosf(a.dt[tok] * a.theta[tok * K + k], &sn, &cs);
      sCS[t][k] = make_float2(cs, sn);
    }
    if (tid < L) {
      const int64_t tok = tok_of(tid);
      const float d = a.dt[tok], lm = a.lam[tok];
      const bool first = tid == 0 && a.prev_B == nullptr;  // no previous token: no trapezoid term
      sS[tid] = make_float4(expf(d * a.A[tok]), first ? 0.0f : (1.0f - lm) * d, lm * d, 0.0f);
    }
  }

  // prev_B^T prev_x on the lane's elements (zero without a previous token)
  float pin0[PPL][4], pin1[PPL][4];
#pragma unroll
  for (int u = 0; u < PPL; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) pin0[u][j] = pin1[u][j] = 0.0f;
  if (a.prev_B) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float xr[4];
      io<T>::load4(a.prev_x, (bh * R + r) * P + col0, xr);
#pragma unroll
      for (int u = 0; u < PPL; ++u) {
        const int k = pg + PG * u;
        float b0 = 0.0f, b1 = 0.0f;
        if (k < K) io<T>::load2(a.prev_B, (bh * R + r) * N + 2 * k, b0, b1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pin0[u][j] += b0 * xr[j];
          pin1[u][j] += b1 * xr[j];
        }
      }
    }
  }
  __syncthreads();

  for (int t = 0; t < L; ++t) {
    const float4 sc = sS[t];
    const float alpha = sc.x, eps = sc.y, gam = sc.z;
    float xv[R][4], yp[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      lds_elem<T>::quad(&sX[t][r * P + col0], xv[r]);
#pragma unroll
      for (int j = 0; j < 4; ++j) yp[r][j] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < PPL; ++u) {
      const int k = pg + PG * u;
      if (PPL * PG == K || k < K) {
        float2 bb[R], cc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          bb[r] = lds_elem<T>::pair(&sB[t][r * N + 2 * k]);
          cc[r] = lds_elem<T>::pair(&sC[t][r * N + 2 * k]);
        }
        const float2 csn = sCS[t][k];
        const float acs = alpha * csn.x, asn = alpha * csn.y;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float cin0 = 0.0f, cin1 = 0.0f;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            cin0 += bb[r].x * xv[r][j];
            cin1 += bb[r].y * xv[r][j];
          }
          // h <- alpha R(w) [h + eps prev_B^T prev_x] + gamma B^T x
          const float v0 = s0[u][j] + eps * pin0[u][j], v1 = s1[u][j] + eps * pin1[u][j];
          const float n0 = acs * v0 - asn * v1 + gam * cin0;
          const float n1 = asn * v0 + acs * v1 + gam * cin1;
          s0[u][j] = n0;
          s1[u][j] = n1;
          pin0[u][j] = cin0;
          pin1[u][j] = cin1;
#pragma unroll
          for (int r = 0; r < R; ++r) yp[r][j] += cc[r].x * n0 + cc[r].y * n1;
        }
      }
    }
    // y[r][col0 + j] sums yp over the PG lanes of the column quad (lane bits
    // >= log2 CQ).  Reduce-scatter: each exchange step halves the values a
    // lane holds (it keeps the half picked by its lane bit and adds the
    // partner's copy of that half), so V values need V - 1 shuffles instead of
    // V log2(PG); steps past the last halving sum the single value.
    {
      constexpr int V = 4 * R;
      float v[V];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * r + j] = yp[r][j];
      int base = 0;  // index of the first value this lane keeps
      reduce_scatter_step<V, CQ>(v, lane, base);
      // V >= PG: the lane holds V / PG consecutive outputs from base on;
      // V < PG: lanes whose low log2(V) pair-group bits match hold the same
      // output, and those with the higher bits clear store it
      constexpr int NK = V >= PG ? V / PG : 1;
      if (V >= PG || (pg & ~(V - 1)) == 0) {
        const int r = base >> 2, j = base & 3;
        const int64_t yo = tok_of(t) * (R * P) + r * P + col0 + j;
#pragma unroll
        for (int i = 0; i < NK; ++i) io<T>::store1(a.y, yo + i, v[i]);
      }
    }
  }

  if (a.h_final) {
    float* st_out = a.h_final + bh * (int64_t)N * P;
#pragma unroll
    for (int u = 0; u < PPL; ++u) {
      const int k = pg + PG * u;
      if (k < K) {
        *(f32x4*)(st_out + (2 * k) * P + col0) = s0[u];
        *(f32x4*)(st_out + (2 * k + 1) * P + col0) = s1[u];
      }
    }
  }
}

template <typename T, int N, int P>
static hipError_t tokens_dispatch_r(const TokensArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.H)), block(256);
  switch (a.R) {
    case 1: hipLaunchKernelGGL((decode_tokens_kernel<T, N, P, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_tokens_kernel<T, N, P, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_tokens_kernel<T, N, P, 4>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int N>
static hipError_t tokens_dispatch_p(int P, const TokensArgs& a, hipStream_t s) {
  switch (P) {
    case 16: return tokens_dispatch_r<T, N, 16>(a, s);
    case 32: return tokens_dispatch_r<T, N, 32>(a, s);
    case 64: return tokens_dispatch_r<T, N, 64>(a, s);
    case 128: return tokens_dispatch_r<T, N, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t tokens_dispatch(int N, int P, const TokensArgs& a, hipStream_t s) {
  switch (N) {
    case 16: return tokens_dispatch_p<T, 16>(P, a, s);
    case 32: return tokens_dispatch_p<T, 32>(P, a, s);
    case 64: return tokens_dispatch_p<T, 64>(P, a, s);
    case 128: return tokens_dispatch_p<T, 128>(P, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_tokens(int io_bf16, int N, int P, const TokensArgs& a, hipStream_t s) {
  if (a.batch * a.H == 0 || a.L == 0) return hipSuccess;
  if (a.L > TOKENS_MAX) return hipErrorInvalidValue;  // every token is staged in LDS
  return io_bf16 ? tokens_dispatch<bf16_t>(N, P, a, s) : tokens_dispatch<float>(N, P, a, s);
}

template <typename T, int N, int P>
static hipError_t decode_dispatch_r(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.BH), block(256);
  switch (a.R) {
    case 1: hipLaunchKernelGGL((decode_step_kernel<T, N, P, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_step_kernel<T, N, P, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_step_kernel<T, N, P, 4>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int N>
static hipError_t decode_dispatch_p(int P, const DecodeArgs& a, hipStream_t s) {
  switch (P) {
    case 16: return decode_dispatch_r<T, N, 16>(a, s);
    case 32: return decode_dispatch_r<T, N, 32>(a, s);
    case 64: return decode_dispatch_r<T, N, 64>(a, s);
    case 128: return decode_dispatch_r<T, N, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t decode_dispatch(int N, int P, const DecodeArgs& a, hipStream_t s) {
  switch (N) {
    case 16: return decode_dispatch_p<T, 16>(P, a, s);
    case 32: return decode_dispatch_p<T, 32>(P, a, s);
    case 64: return decode_dispatch_p<T, 64>(P, a, s);
    case 128: return decode_dispatch_p<T, 128>(P, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(int io_bf16, int N, int P, const DecodeArgs& a, hipStream_t s) {
  if (a.BH == 0) return hipSuccess;
  return io_bf16 ? decode_dispatch<bf16_t>(N, P, a, s) : decode_dispatch<float>(N, P, a, s);
}

}  // namespace m3
