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
// rotation never leaves registers.  y = C^T h is reduced through LDS.
#include "m3_common.hpp"
#include "m3_launch.hpp"

namespace m3 {

template <typename T, int N, int P>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeArgs a) {
  constexpr int K = N / 2;
  constexpr int CG = P / 4;                 // column groups of 4 (divides 256)
  constexpr int ITEMS = K * CG;
  constexpr int PER = (ITEMS + 255) / 256;  // items per thread
  constexpr int RMAX = 4;
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int R = a.R;

  __shared__ float sB[RMAX][N], sC[RMAX][N], sPB[RMAX][N];
  __shared__ float2 sCS[K];
  __shared__ float red[256][RMAX * 4 + 1];

  const float d = a.dt[bh], lam = a.lam[bh];
  const float alpha = expf(d * a.A[bh]);
  const float eps = (1.0f - lam) * d, gam = lam * d;
  for (int k = tid; k < K; k += 256) {
    float s, c;
    sincosf(d * a.theta[bh * K + k], &s, &c);
    sCS[k] = make_float2(c, s);
  }
  const bool has_prev = a.prev_B != nullptr;
  for (int i = tid; i < R * N; i += 256) {
    const int r = i / N, n = i % N;
    sB[r][n] = io<T>::load1(a.B, bh * R * N + i);
    sC[r][n] = io<T>::load1(a.C, bh * R * N + i);
    sPB[r][n] = has_prev ? io<T>::load1(a.prev_B, bh * R * N + i) : 0.0f;
  }
  const int c = tid % CG;
  float xv[RMAX][4], pxv[RMAX][4];
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[r][j] = r < R ? io<T>::load1(a.x, (bh * R + r) * P + 4 * c + j) : 0.0f;
      pxv[r][j] = (r < R && has_prev) ? io<T>::load1(a.prev_x, (bh * R + r) * P + 4 * c + j) : 0.0f;
    }
  __syncthreads();

  float* st = a.state + bh * (int64_t)N * P;
  float4 h0[PER], h1[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid + 256 * q;
    if (i < ITEMS) {
      const int k = i / CG;
      h0[q] = *(const float4*)(st + (2 * k) * P + 4 * c);
      h1[q] = *(const float4*)(st + (2 * k + 1) * P + 4 * c);
    }
  }
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
      float u0[4] = {h0[q].x, h0[q].y, h0[q].z, h0[q].w};
      float u1[4] = {h1[q].x, h1[q].y, h1[q].z, h1[q].w};
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
        const float v0 = u0[j] + eps * pin0, v1 = u1[j] + eps * pin1;
        n0[j] = alpha * (cs.x * v0 - cs.y * v1) + gam * cin0;
        n1[j] = alpha * (cs.y * v0 + cs.x * v1) + gam * cin1;
#pragma unroll
        for (int r = 0; r < RMAX; ++r)
          if (r < R) yp[r][j] += sC[r][2 * k] * n0[j] + sC[r][2 * k + 1] * n1[j];
      }
      *(float4*)(st + (2 * k) * P + 4 * c) = make_float4(n0[0], n0[1], n0[2], n0[3]);
      *(float4*)(st + (2 * k + 1) * P + 4 * c) = make_float4(n1[0], n1[1], n1[2], n1[3]);
    }
  }
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[tid][r * 4 + j] = yp[r][j];
  __syncthreads();
  // y[r][p]: sum the partials of the threads that own column group p/4
  constexpr int GROUPS = 256 / CG;
  for (int o = tid; o < R * P; o += 256) {
    const int r = o / P, p = o % P;
    const int cg = p / 4, j = p % 4;
    float s = 0.0f;
#pragma unroll 4
    for (int gi = 0; gi < GROUPS; ++gi) s += red[cg + CG * gi][r * 4 + j];
    io<T>::store1(a.y, bh * R * P + o, s);
  }
}

template <typename T, int N>
static hipError_t decode_dispatch_p(int P, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.BH), block(256);
  switch (P) {
    case 16: hipLaunchKernelGGL((decode_step_kernel<T, N, 16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((decode_step_kernel<T, N, 32>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((decode_step_kernel<T, N, 64>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((decode_step_kernel<T, N, 128>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
