// Cumulative-angle rotation of B and C (the data-dependent RoPE form of the
// complex state, linkstar.cloud/article/869, "第二刀：复值状态空间"):
//     phi_t = angle0 + sum_{s<=t} dt_s theta_s[k],
//     B_rot_t = R(-phi_t) B_t,  C_rot_t = R(-phi_t) C_t,  angle_final = phi_L.
//
// The scan runs along L, which is long (up to 64K tokens) while B*H*N/2 may be
// small, so it is split in three launches over 64-token chunks:
//   1. chunk totals of dt*theta per (b,h,chunk,pair)          -> workspace
//   2. exclusive scan of the totals over chunks (+ angle0)    -> workspace
//   3. per chunk: wave-level inclusive scan in LDS + offset, sincos once per
//      (token, pair), then rotate every rank of B and C with 16-byte accesses.
// Launch 3 moves almost all the bytes (B, C in and out); 1 and 2 read only
// dt and theta once more.
#include "m3_common.hpp"
#include "m3_lanes.hpp"
#include "m3_launch.hpp"

namespace m3 {

template <int N>
__global__ __launch_bounds__(256) void rope_totals_kernel(RopeArgs a, int64_t nchunks) {
  constexpr int K = N / 2;
  constexpr int TG = 256 / K;
  const int64_t h = blockIdx.x, c = blockIdx.y, b = blockIdx.z;  // head fastest
  const int k = threadIdx.x % K, tg = threadIdx.x / K;
  // every load of the thread is issued before the sum (tokens past L read
  // token L - 1 with weight 0)
  constexpr int NT = ROPE_CHUNK / TG;
  float dv[NT], tv[NT];
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    const int64_t tok = c * ROPE_CHUNK + tg + TG * q;
    const int64_t idx = (b * a.L + (tok < a.L ? tok : a.L - 1)) * a.H + h;
    dv[q] = tok < a.L ? a.dt[idx] : 0.0f;
    tv[q] = a.theta[idx * K + k];
  }
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < NT; ++q) s += dv[q] * tv[q];
  __shared__ float red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  if (tg == 0) {
    for (int q = 1; q < TG; ++q) s += red[q * K + k];
    a.totals[((b * a.H + h) * nchunks + c) * K + k] = s;
  }
}

template <int N>
__global__ __launch_bounds__(256) void rope_scan_kernel(RopeArgs a, int64_t nchunks) {
  constexpr int K = N / 2;
  constexpr int SEG = 256 / K;
  const int64_t bh = (int64_t)blockIdx.y * a.H + blockIdx.x;
  const int k = threadIdx.x % K, sg = threadIdx.x / K;
  const int64_t per = (nchunks + SEG - 1) / SEG;
  const int64_t c_begin = sg * per;
  const int64_t c_end = c_begin + per < nchunks ? c_begin + per : nchunks;
  float* tot = a.totals + bh * nchunks * K;
  float s = 0.0f;
  for (int64_t c = c_begin; c < c_end; ++c) s += tot[c * K + k];
  __shared__ float sums[SEG][K];
  sums[sg][k] = s;
  __syncthreads();
  float run = a.angle0 ? a.angle0[bh * K + k] : 0.0f;
  for (int q = 0; q < sg; ++q) run += sums[q][k];
  for (int64_t c = c_begin; c < c_end; ++c) {
    const float v = tot[c * K + k];
    tot[c * K + k] = run;
    run += v;
  }
  if (sg == SEG - 1 && a.angle_final) a.angle_final[bh * K + k] = run;
}

template <typename T, int N>
__global__ __launch_bounds__(256) void rope_apply_kernel(RopeArgs a, int64_t nchunks) {
  constexpr int K = N / 2;
  constexpr int VEC = io<T>::VEC;
  constexpr int VPR = N / VEC;                          // vectors per (token, rank) row
  constexpr int MAXIT = (ROPE_CHUNK * 4 * VPR + 255) / 256;
  constexpr int BATCH = MAXIT < 8 ? MAXIT : 8;          // vectors per tensor kept in flight
  // grid: x = head (fastest: concurrent blocks touch adjacent memory), y = chunk, z = batch
  const int64_t h = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = c * ROPE_CHUNK;
  const int nvalid = (int)((a.L - c0) < ROPE_CHUNK ? (a.L - c0) : ROPE_CHUNK);
  const int R = a.R;
  const int items = nvalid * R * VPR;
  const int64_t e0 = ((b * a.L + c0) * a.H + h) * (int64_t)R * N;  // token c0, rank 0
  auto off = [&](int i) {
    const int row = i / VPR, n0 = (i % VPR) * VEC;
    return e0 + ((int64_t)(row / R) * a.H * R + (row % R)) * N + n0;
  };
  __shared__ float om[ROPE_CHUNK][K + 1];
  __shared__ float2 cs[ROPE_CHUNK][K];
  __shared__ float offs[K];  // the chunk's angle offset per pair (scan of the chunk totals)
  if (tid < K) offs[tid] = a.totals[((b * a.H + h) * nchunks + c) * K + tid];

  // first batch of B and C vectors: in flight while the angles are scanned
  typename io<T>::vec vb[BATCH], vc[BATCH];
#pragma unroll
  for (int j = 0; j < BATCH; ++j) {
    const int i = tid + 256 * j;
    if (i < items) {
      vb[j] = ldg16<T>(a.B, off(i));
      vc[j] = ldg16<T>(a.C, off(i));
    }
  }
  for (int i = tid; i < ROPE_CHUNK * K; i += 256) {
    const int t = i / K, k = i % K;
    float v = 0.0f;
    if (t < nvalid) {
      const int64_t idx = (b * a.L + c0 + t) * a.H + h;
      v = a.dt[idx] * a.theta[idx * K + k];
    }
    om[t][k] = v;
  }
  __syncthreads();
  for (int k = wave; k < K; k += 4) {
    const float v = wave_incl_scan(om[lane][k]) + offs[k];
    float s, co;
    // bf16 io: the hardware sine/cosine (in revolutions; the reduction by the
    // nearest whole revolution is exact); fp32 io: the library routine
    if constexpr (sizeof(T) == 2) sincos_rev(v, &s, &co);
    else sincosf(v, &s, &co);
    cs[lane][k] = make_float2(co, s);
  }
  __syncthreads();

  auto rotate_store = [&](int i, const typename io<T>::vec& bv, const typename io<T>::vec& cv) {
    const int row = i / VPR, n0 = (i % VPR) * VEC;
    const int t = row / R;
    float fb[VEC], fc[VEC];
    io<T>::unpack(bv, fb);
    io<T>::unpack(cv, fc);
#pragma unroll
    for (int q = 0; q < VEC / 2; ++q) {
      const float2 r2 = cs[t][n0 / 2 + q];
      const float b0 = fb[2 * q], b1 = fb[2 * q + 1];
      const float c0v = fc[2 * q], c1v = fc[2 * q + 1];
      // R(-phi) (u, v) = (cos u + sin v, -sin u + cos v)
      fb[2 * q] = r2.x * b0 + r2.y * b1;
      fb[2 * q + 1] = r2.x * b1 - r2.y * b0;
      fc[2 * q] = r2.x * c0v + r2.y * c1v;
      fc[2 * q + 1] = r2.x * c1v - r2.y * c0v;
    }
    stg16_nt<T>(a.B_rot, off(i), io<T>::pack(fb));
    stg16_nt<T>(a.C_rot, off(i), io<T>::pack(fc));
  };
#pragma unroll
  for (int j = 0; j < BATCH; ++j) {
    const int i = tid + 256 * j;
    if (i < items) rotate_store(i, vb[j], vc[j]);
  }
  for (int i = tid + 256 * BATCH; i < items; i += 256) rotate_store(i, ldg16<T>(a.B, off(i)), ldg16<T>(a.C, off(i)));
}

// The angles alone, for a consumer that rotates B and C itself (the B/C
// prologue): cos and sin of phi_t per (token, head, pair), written to cs
// (B, L, H, N/2) as one 32-bit word of two fp16 values.  Per chunk as in
// launch 3: the chunk-local wave scan plus the chunk's offset, then the
// chunk's values written token by token.  A block takes HB adjacent heads,
// so that each token's theta and cs rows are read and written as one piece of
// HB * N/2 * 4 bytes (512 bytes when H allows) instead of one per head.
template <int N, int HB>
__global__ __launch_bounds__(256) void rope_phi_kernel(RopeArgs a, int64_t nchunks, uint32_t* cs) {
  constexpr int K = N / 2, W = HB * K;  // columns of the block: HB heads x K pairs
  constexpr int PER = ROPE_CHUNK * W / 256;
  static_assert(ROPE_CHUNK * W % 256 == 0, "whole passes of the block over the chunk's columns");
  const int64_t h0 = (int64_t)blockIdx.x * HB, c = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = c * ROPE_CHUNK;
  const int nvalid = (int)((a.L - c0) < ROPE_CHUNK ? (a.L - c0) : ROPE_CHUNK);
  __shared__ float om[ROPE_CHUNK][W + 1];
  __shared__ float offs[W];  // the chunk's angle offset per column (scan of the chunk totals)
  if (tid < W) offs[tid] = a.totals[((b * a.H + h0 + tid / K) * nchunks + c) * K + tid % K];
  // every load of the thread is issued before the first product
  float dv[PER], tv[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid + 256 * q, t = i / W, j = i % W;
    const int64_t row = (b * a.L + c0 + t) * a.H + h0;  // (token, first head of the block)
    dv[q] = t < nvalid ? a.dt[row + j / K] : 0.0f;
    tv[q] = t < nvalid ? a.theta[row * K + j] : 0.0f;
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid + 256 * q;
    om[i / W][i % W] = dv[q] * tv[q];
  }
  __syncthreads();
  for (int j = wave; j < W; j += 4) {
    const float v = wave_incl_scan(om[lane][j]) + offs[j];
    om[lane][j] = v;  // each wave reads and writes only its own columns
  }
  __syncthreads();
  // (cos, sin) of the angle, each rounded to fp16 (absolute error <= 2^-12,
  // below the bf16 rounding of the rotated outputs): the consumer rotates
  // every rank of B and C with them and computes no sine itself
  for (int i = tid; i < nvalid * W; i += 256) {
    const int t = i / W, j = i % W;
    float sn, cn;
    sincos_rev(om[t][j], &sn, &cn);
    const f32x2 v = {cn, sn};
    cs[((b * a.L + c0 + t) * a.H + h0) * K + j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
}

template <int N>
static hipError_t rope_phi_run(const RopeArgs& a, uint32_t* cs, hipStream_t s) {
  const int64_t nchunks = (a.L + ROPE_CHUNK - 1) / ROPE_CHUNK;
  const dim3 g3h((unsigned)a.H, (unsigned)nchunks, (unsigned)a.batch);
  hipLaunchKernelGGL((rope_totals_kernel<N>), g3h, dim3(256), 0, s, a, nchunks);
  hipLaunchKernelGGL((rope_scan_kernel<N>), dim3((unsigned)a.H, (unsigned)a.batch), dim3(256), 0, s, a, nchunks);
  constexpr int HB = 256 / N;  // heads whose rows of N/2 floats make 512 bytes
  if (a.H % HB == 0) {
    const dim3 g((unsigned)(a.H / HB), (unsigned)nchunks, (unsigned)a.batch);
    hipLaunchKernelGGL((rope_phi_kernel<N, HB>), g, dim3(256), 0, s, a, nchunks, cs);
  } else {
    hipLaunchKernelGGL((rope_phi_kernel<N, 1>), g3h, dim3(256), 0, s, a, nchunks, cs);
  }
  return hipGetLastError();
}

hipError_t launch_rope_phi(int N, const RopeArgs& a, uint32_t* cs, hipStream_t s) {
  if (a.batch == 0 || a.H == 0) return hipSuccess;
  if (a.L == 0) {
    if (a.angle_final) return launch_copy_f32(a.angle_final, a.angle0, a.batch * a.H * (N / 2), s);
    return hipSuccess;
  }
  switch (N) {
    case 16: return rope_phi_run<16>(a, cs, s);
    case 32: return rope_phi_run<32>(a, cs, s);
    case 64: return rope_phi_run<64>(a, cs, s);
    case 128: return rope_phi_run<128>(a, cs, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int N>
static hipError_t rope_run(const RopeArgs& a, hipStream_t s) {
  const int64_t nchunks = (a.L + ROPE_CHUNK - 1) / ROPE_CHUNK;
  const dim3 g3h((unsigned)a.H, (unsigned)nchunks, (unsigned)a.batch);
  hipLaunchKernelGGL((rope_totals_kernel<N>), g3h, dim3(256), 0, s, a, nchunks);
  hipLaunchKernelGGL((rope_scan_kernel<N>), dim3((unsigned)a.H, (unsigned)a.batch), dim3(256), 0, s, a, nchunks);
  hipLaunchKernelGGL((rope_apply_kernel<T, N>), g3h, dim3(256), 0, s, a, nchunks);
  return hipGetLastError();
}

template <typename T>
static hipError_t rope_dispatch(int N, const RopeArgs& a, hipStream_t s) {
  switch (N) {
    case 16: return rope_run<T, 16>(a, s);
    case 32: return rope_run<T, 32>(a, s);
    case 64: return rope_run<T, 64>(a, s);
    case 128: return rope_run<T, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rope(int io_bf16, int N, const RopeArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.H == 0) return hipSuccess;
  if (a.L == 0) {
    if (a.angle_final) return launch_copy_f32(a.angle_final, a.angle0, a.batch * a.H * (N / 2), s);
    return hipSuccess;
  }
  return io_bf16 ? rope_dispatch<bf16_t>(N, a, s) : rope_dispatch<float>(N, a, s);
}

// grid-stride, so that any n fits one launch of at most 65536 blocks
__global__ void copy_f32_kernel(float* dst, const float* src, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += step) dst[i] = src ? src[i] : 0.0f;
}

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
  hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace m3
