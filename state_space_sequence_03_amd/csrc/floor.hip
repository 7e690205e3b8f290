// Memory-floor probes for the benchmark (not part of the library's
// operations): kernels that move exactly the bytes of a workload with no
// arithmetic beyond what keeps every load alive, so that their time is the
// floor that the access pattern itself sets on this GPU.
//
//  * m3f_stream: nr contiguous input arrays read once and one output array
//    written once (out = xor of the inputs), grid-stride, every load of an
//    iteration issued before its first use.  nr = 3 is the 3:1 read:write mix
//    of the prefill walker (x, B, C in, y out) as one contiguous stream.
//  * m3f_walk: the prefill walker's own global access pattern for bf16 io,
//    P = N = 64, R = 4 or 1 (the 1.5B MIMO and SISO head shapes): one block
//    of 256 threads
//    per (b, h) walking 32-token sub-chunks in order, two blocks per compute
//    unit (64-token sub-chunks, two tokens per staging thread for R = 1), each
//    thread loading the same pieces of B, x, C, theta and the
//    scalars as the walker's staging and output phases (the next sub-chunk's
//    loads issued before the current sub-chunk's stores of y), and storing y
//    as the walker does (32 bytes per lane).  heads_per_block = 2 lets one
//    block of 512 threads walk two adjacent heads together, so that each
//    token's rows of a tensor are read as one 1 KB piece.
//  * m3f_rmw: an in-place read-modify-write of a float array (the decode
//    step's state traffic), for buffers below and above the 256 MB
//    memory-side cache.
//  * m3f_mfma: the achievable bf16 MFMA rate: each wave runs 8 independent
//    accumulator chains of 16x16x32 or 32x32x16 bf16 products with operands
//    held in registers (no memory traffic), two waves per SIMD.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint4 x4(uint4 a, uint4 b) { return make_uint4(a.x ^ b.x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w); }

template <int NR>
__global__ __launch_bounds__(256) void stream_kernel(const uint4* __restrict__ a0, const uint4* __restrict__ a1,
                                                     const uint4* __restrict__ a2, uint4* __restrict__ out, int64_t n) {
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < n; i0 += stride * U) {
    uint4 v[U][NR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n) {
        v[u][0] = a0[i];
        if constexpr (NR > 1) v[u][1] = a1[i];
        if constexpr (NR > 2) v[u][2] = a2[i];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n) {
        uint4 r = v[u][0];
        if constexpr (NR > 1) r = x4(r, v[u][1]);
        if constexpr (NR > 2) r = x4(r, v[u][2]);
        out[i] = r;
      }
    }
  }
}

struct WalkPtrs {
  const unsigned char *x, *B, *C, *theta, *dt, *A, *lam;
  unsigned char* y;
  int64_t batch, L, H;
};

// HPB heads per block (adjacent), 256 threads per head; rank R = 4 (32-token
// sub-chunks, one token per staging thread) or R = 1 (64-token sub-chunks,
// two adjacent tokens per staging thread), as the walker for P = N = 64.
template <int HPB, int R, int N = 64>
__global__ __launch_bounds__(256 * HPB) void walk_kernel(WalkPtrs a) {
  constexpr int P = 64, K = N / 2, QS = N == 128 ? 16 : (R == 1 ? 64 : 32), CH = N / 8, NKS = N / 32;
  constexpr int TPT = QS * CH / 256, XIT = R * 8 / CH;  // x row pieces per thread: rank i / 8, column i % 8
  constexpr int V = QS * R, NCT = V / 16, NCW = NCT == 8 ? 2 : 1;
  constexpr int lgR = R == 4 ? 2 : 0;
  const int tid = threadIdx.x & 255, hsub = threadIdx.x >> 8;
  const int lane = tid & 63, wave = tid >> 6, m16 = lane & 15, g = lane >> 4;
  const int st_t = tid / CH, st_c = tid % CH;
  const int64_t bh = (int64_t)blockIdx.x * HPB + hsub;
  const int64_t b = bh / a.H, h = bh % a.H;
  int ctl[NCW];
  if constexpr (NCW == 2) {
    ctl[0] = 7 - wave;
    ctl[1] = wave;
  } else {
    ctl[0] = wave;
  }
  auto tok = [&](int64_t t) { return (b * a.L + t) * a.H + h; };
  uint4 rB[TPT][R], rX[TPT][XIT], rC[NCW][NKS], rTh[TPT];
  float rd[TPT], ra[TPT], rl[TPT], rd1[TPT], rl1[TPT];
  auto load = [&](int64_t c0) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int64_t t = c0 + TPT * st_t + u;
      const int64_t tt = tok(t);
#pragma unroll
      for (int r = 0; r < R; ++r) rB[u][r] = *(const uint4*)(a.B + (tt * R + r) * N * 2 + 16 * st_c);
#pragma unroll
      for (int k = 0; k < XIT; ++k) {
        const int i = st_c + CH * k;
        rX[u][k] = *(const uint4*)(a.x + (tt * R + (i >> 3)) * P * 2 + 16 * (i & 7));
      }
      rTh[u] = *(const uint4*)(a.theta + tt * K * 4 + 16 * st_c);
      rd[u] = *(const float*)(a.dt + tt * 4);
      ra[u] = *(const float*)(a.A + tt * 4);
      rl[u] = *(const float*)(a.lam + tt * 4);
      const int64_t t1 = t + 1 < a.L ? tok(t + 1) : tt;
      rd1[u] = *(const float*)(a.dt + t1 * 4);
      rl1[u] = *(const float*)(a.lam + t1 * 4);
    }
#pragma unroll
    for (int ci = 0; ci < NCW; ++ci) {
      const int v = ctl[ci] * 16 + m16;
      const int64_t tc = tok(c0 + (v >> lgR));
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        rC[ci][ks] = *(const uint4*)(a.C + (tc * R + (v & (R - 1))) * N * 2 + 16 * g + ks * 64);
    }
  };
  load(0);
  for (int64_t c0 = 0; c0 < a.L; c0 += QS) {
    // fold this sub-chunk's registers into the values stored as y
    uint4 s = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
#pragma unroll
      for (int r = 0; r < R; ++r) s = x4(s, rB[u][r]);
#pragma unroll
      for (int k = 0; k < XIT; ++k) s = x4(s, rX[u][k]);
      s = x4(s, rTh[u]);
      s.x ^= __float_as_uint(rd[u]) ^ __float_as_uint(ra[u]) ^ __float_as_uint(rl[u]);
      s.y ^= __float_as_uint(rd1[u]) ^ __float_as_uint(rl1[u]);
    }
    uint4 yv[NCW];
#pragma unroll
    for (int ci = 0; ci < NCW; ++ci) {
      yv[ci] = s;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) yv[ci] = x4(yv[ci], rC[ci][ks]);
    }
    if (c0 + QS < a.L) load(c0 + QS);
#pragma unroll
    for (int ci = 0; ci < NCW; ++ci) {
      const int v = ctl[ci] * 16 + m16;
      unsigned char* yr = a.y + (tok(c0 + (v >> lgR)) * R + (v & (R - 1))) * P * 2 + 32 * g;
      *(uint4*)yr = yv[ci];
      *(uint4*)(yr + 16) = x4(yv[ci], s);
    }
  }
}

__global__ __launch_bounds__(256) void rmw_kernel(float4* __restrict__ p, int64_t n, float a, float c) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float4 v = p[i];
    v.x = v.x * a + c; v.y = v.y * a + c; v.z = v.z * a + c; v.w = v.w * a + c;
    p[i] = v;
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// KIND 0: 16x16x32 bf16 (16,384 flop), 1: 32x32x16 bf16 (32,768 flop).  The
// operands come from the thread id through an empty asm, so nothing folds;
// the sums are stored only when a flag the host never sets is set.
template <int KIND>
__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(int iters, int store, float* out) {
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v = (float)((threadIdx.x + i) & 7) * 0.125f;
    asm volatile("" : "+v"(v));
    a[i] = (__bf16)v;
    b[i] = (__bf16)(1.0f - v);
  }
  float sum = 0.0f;
  if constexpr (KIND == 0) {
    f32x4_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += acc[j][0] + acc[j][3];
  } else {
    f32x16_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += acc[j][0] + acc[j][15];
  }
  if (store) out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace

extern "C" {

// kind 0: 16x16x32, 1: 32x32x16 bf16; blocks of 256 threads, each wave
// issuing 8 x iters MFMAs; out (blocks * 256 floats) is written only if store.
int m3f_mfma(int kind, int iters, int blocks, int store, float* out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0) hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(blocks), dim3(256), 0, s, iters, store, out);
  else if (kind == 1) hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(blocks), dim3(256), 0, s, iters, store, out);
  else return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// nr in {1, 2, 3} inputs of n16 16-byte vectors each (unused ones may be NULL).
int m3f_stream(int nr, const void* a0, const void* a1, const void* a2, void* out, int64_t n16, int blocks,
               void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const uint4 *p0 = (const uint4*)a0, *p1 = (const uint4*)a1, *p2 = (const uint4*)a2;
  if (nr == 1) hipLaunchKernelGGL(stream_kernel<1>, dim3(blocks), dim3(256), 0, s, p0, p1, p2, (uint4*)out, n16);
  else if (nr == 2) hipLaunchKernelGGL(stream_kernel<2>, dim3(blocks), dim3(256), 0, s, p0, p1, p2, (uint4*)out, n16);
  else if (nr == 3) hipLaunchKernelGGL(stream_kernel<3>, dim3(blocks), dim3(256), 0, s, p0, p1, p2, (uint4*)out, n16);
  else return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The walker's access pattern over (batch, L, H) at P = 64, N = 64 with rank
// R (1 or 4) or N = 128 with R = 4, with L a multiple of the sub-chunk (64
// tokens for R = 1, 32 for N = 64 and R = 4, 16 for N = 128) and H a multiple
// of heads_per_block (1 or 2; 1 at N = 128);
// lds_bytes of dynamic LDS per block sets the number of resident blocks per
// compute unit.
int m3f_walk(const void* x, const void* B, const void* C, const void* theta, const void* dt, const void* A,
             const void* lam, void* y, int64_t batch, int64_t L, int64_t H, int N, int R, int heads_per_block,
             int lds_bytes, void* stream) {
  if ((R != 1 && R != 4) || (N != 64 && N != 128) || (N == 128 && (R != 4 || heads_per_block != 1)) ||
      L % (N == 128 ? 16 : (R == 1 ? 64 : 32)) != 0 || (heads_per_block != 1 && heads_per_block != 2) ||
      H % heads_per_block != 0)
    return 1;
  WalkPtrs a{(const unsigned char*)x, (const unsigned char*)B, (const unsigned char*)C, (const unsigned char*)theta,
             (const unsigned char*)dt, (const unsigned char*)A, (const unsigned char*)lam, (unsigned char*)y,
             batch, L, H};
  hipStream_t s = (hipStream_t)stream;
  const unsigned blocks = (unsigned)(batch * H / heads_per_block);
  if (N == 128) {
    if (hipFuncSetAttribute((const void*)walk_kernel<1, 4, 128>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess) return 2;
    hipLaunchKernelGGL((walk_kernel<1, 4, 128>), dim3(blocks), dim3(256), lds_bytes, s, a);
  } else if (R == 1 && heads_per_block == 1) {
    if (hipFuncSetAttribute((const void*)walk_kernel<1, 1>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess) return 2;
    hipLaunchKernelGGL((walk_kernel<1, 1>), dim3(blocks), dim3(256), lds_bytes, s, a);
  } else if (R == 1) {
    if (hipFuncSetAttribute((const void*)walk_kernel<2, 1>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess) return 2;
    hipLaunchKernelGGL((walk_kernel<2, 1>), dim3(blocks), dim3(512), lds_bytes, s, a);
  } else if (heads_per_block == 1) {
    if (hipFuncSetAttribute((const void*)walk_kernel<1, 4>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess) return 2;
    hipLaunchKernelGGL((walk_kernel<1, 4>), dim3(blocks), dim3(256), lds_bytes, s, a);
  } else {
    if (hipFuncSetAttribute((const void*)walk_kernel<2, 4>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess) return 2;
    hipLaunchKernelGGL((walk_kernel<2, 4>), dim3(blocks), dim3(512), lds_bytes, s, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int m3f_rmw(void* p, int64_t n4, int blocks, void* stream) {
  hipLaunchKernelGGL(rmw_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (float4*)p, n4, 0.999f, 0.001f);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
