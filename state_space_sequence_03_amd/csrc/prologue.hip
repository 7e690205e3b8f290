// The B/C prologue in front of the SSM core, in one pass over its output:
//   p = W u_t                      (projection; the rows of W are those of W_B
//                                   then of W_C; papers.ananclaw.com/promo/
//                                   explainers__2603-15569, "关键公式与“伪代码”")
//   v = p / sqrt(mean_n p^2 + eps) * gain + bias
//                                  (RMS normalisation of every (token, head,
//                                   rank) vector over its N entries, then the
//                                   bias; linkstar.cloud/article/869,
//                                   "架构上的其他改动")
//   B_rot, C_rot = R(-phi_t) v     (the cumulative-angle rotation of rope_bc,
//                                   linkstar.cloud/article/869, "第二刀", which
//                                   notes that it can be fused with the
//                                   projection)
// so that B and C are written once, already normalised and rotated, and never
// read back.  The angles phi_t come from a small pre-pass over dt and theta
// (rope.hip).
//
// The product is computed transposed, D^T = W u^T, on bf16 32x32x16 MFMAs
// with fp32 accumulation: a block owns 256 features x 256 tokens, its eight
// waves 128 features x 64 tokens each (4 x 2 tiles of 32 x 32).  In the MFMA's
// output layout lane l holds token l mod 32 and features 8(v/4) + 4(l/32) +
// (v mod 4) of a tile (v < 16), so
//   * every lane holds runs of 4 consecutive features of one token: each
//     rotation pair sits in one lane and is stored as 8 bytes;
//   * the N features of one (token, head, rank) vector lie in the lane and in
//     lane l ^ 32 only: the sum of squares is the lane's own sum plus one row
//     swap.
// K advances 64 at a time through two LDS stages (the next stage's loads in
// registers while the current one feeds the MFMAs; one barrier per stage).
// Tiles of 256 rows x 128 bytes are swizzled by 16-byte chunks so that the
// 32 rows an operand read touches fall in distinct bank groups.
//
// Block order: workgroups go to the 8 XCDs in turn, so block ids are mapped
// such that each XCD's 32 concurrent blocks cover a 4 x 8 rectangle of
// (token, feature) tiles inside a 16 x 16 super-tile: they share 12 operand
// tiles in that XCD's L2 instead of 64.
#include "m3_common.hpp"
#include "m3_lanes.hpp"
#include "m3_launch.hpp"

namespace m3 {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int PF = 256;   // features per block
constexpr int PT = 256;   // tokens per block
constexpr int PK = 64;    // k per stage (128-byte rows)
constexpr int TILE_BYTES = 256 * PK * 2;

__device__ __forceinline__ int soff(int row, int chunk) { return row * 128 + ((chunk ^ fsw<8>(row)) << 4); }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

template <int N>
__global__ __launch_bounds__(512) void bc_prologue_kernel(ProArgs a, int ntb, int nfb, int nsf) {
  // ---- block -> (token tile, feature tile)
  const int bid = blockIdx.x;
  const int xcd = bid & 7, j = bid >> 3;
  const int sup = j >> 5, w32 = j & 31;
  const int tb = (sup / nsf) * 16 + (xcd >> 1) * 4 + (w32 >> 3);
  const int fb = (sup % nsf) * 16 + (xcd & 1) * 8 + (w32 & 7);
  if (tb >= ntb || fb >= nfb) return;

  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE_BYTES];  // [stage][W, u]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wf = wave & 1, wt = wave >> 1;
  const int64_t F = 2 * (int64_t)a.H * a.R * N;
  const int64_t f0 = (int64_t)fb * PF, m0 = (int64_t)tb * PT;
  const int64_t rowb = a.D * 2;  // bytes per row of u and W

  // ---- global -> register assignments: rows tid/8 + 64 i, 16-byte chunk tid % 8
  const int lrow = tid >> 3, lch = tid & 7;
  const char* pw[4];
  const char* pu[4];
  bool vw[4], vu[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lrow + 64 * i;
    vw[i] = f0 + r < F;
    vu[i] = m0 + r < a.M;
    pw[i] = (const char*)a.W + (vw[i] ? (f0 + r) : 0) * rowb + lch * 16;
    pu[i] = (const char*)a.u + (vu[i] ? (m0 + r) : 0) * rowb + lch * 16;
  }
  uint4 rw[4], ru[4];
  auto load = [&](int64_t kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rw[i] = vw[i] ? *(const uint4*)(pw[i] + kb) : make_uint4(0, 0, 0, 0);
      ru[i] = vu[i] ? *(const uint4*)(pu[i] + kb) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage = [&](int st) {
    char* sw = smem + st * 2 * TILE_BYTES;
    char* su = sw + TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = soff(lrow + 64 * i, lch);
      *(uint4*)(sw + o) = rw[i];
      *(uint4*)(su + o) = ru[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int ft = 0; ft < 4; ++ft)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ft][tt][v] = 0.0f;

  const int nk = (int)(a.D / PK);
  load(0);
  stage(0);
  __syncthreads();
  const int l32 = lane & 31, lh = lane >> 5;
  for (int kk = 0; kk < nk; ++kk) {
    if (kk + 1 < nk) load((int64_t)(kk + 1) * 128);
    const char* sw = smem + (kk & 1) * 2 * TILE_BYTES;
    const char* su = sw + TILE_BYTES;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + lh;
      bf16x8 fa[4], fbv[2];
#pragma unroll
      for (int ft = 0; ft < 4; ++ft) fa[ft] = as_bf16x8(*(const uint4*)(sw + soff(wf * 128 + ft * 32 + l32, ch)));
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) fbv[tt] = as_bf16x8(*(const uint4*)(su + soff(wt * 64 + tt * 32 + l32, ch)));
#pragma unroll
      for (int ft = 0; ft < 4; ++ft)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) acc[ft][tt] = mfma32(fa[ft], fbv[tt], acc[ft][tt]);
    }
    if (kk + 1 < nk) stage((kk + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: RMS over each N-feature vector, gain, bias, rotation, store
  constexpr int G = 128 / N;  // vectors per token in the wave's 128 features
  // feature indices fit 32 bits (F <= 2 * 65535 * 4 * 128)
  const uint32_t HRN = (uint32_t)a.H * (uint32_t)a.R * N;
  const uint32_t shRN = (uint32_t)__builtin_ctz((unsigned)(a.R * N));  // R N is a power of 2
  const uint32_t fw0 = (uint32_t)f0 + wf * 128;  // first feature of the wave
  float inv[2][G];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    float ss[G];
#pragma unroll
    for (int g = 0; g < G; ++g) ss[g] = 0.0f;
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // the lane's feature in the wave is ft*32 + 8(v/4) + 4 lh + (v mod 4);
        // with N >= 16 its vector index does not depend on the lane half lh
        const float x = acc[ft][tt][v];
        ss[(ft * 32 + 8 * (v >> 2)) / N] += x * x;
      }
#pragma unroll
    for (int g = 0; g < G; ++g) inv[tt][g] = rsqrtf(swap_sum32(ss[g]) * (1.0f / N) + a.eps);
  }
  const int K2 = N / 2;
#pragma unroll
  for (int ft = 0; ft < 4; ++ft) {
    if ((int64_t)fw0 + ft * 32 >= F) break;  // F is a multiple of 32: whole tiles are in or out
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t f = fw0 + ft * 32 + 8 * q + 4 * lh;  // first of the lane's 4 features
      const float4 gv = a.gain ? *(const float4*)(a.gain + f) : make_float4(1.f, 1.f, 1.f, 1.f);
      const float4 bv = a.bias ? *(const float4*)(a.bias + f) : make_float4(0.f, 0.f, 0.f, 0.f);
      const bool isC = f >= HRN;
      const uint32_t rem = isC ? f - HRN : f;
      const uint32_t head = rem >> shRN;
      const uint32_t k0 = (rem & (N - 1)) >> 1;
      char* outp = (char*)(isC ? a.C_rot : a.B_rot);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int64_t m = m0 + wt * 64 + tt * 32 + l32;
        if (m >= a.M) continue;
        const float2 ph = *(const float2*)(a.phi + (m * a.H + head) * K2 + k0);
        const float iv = inv[tt][(ft * 32 + 8 * q) / N];
        const float x0 = acc[ft][tt][4 * q + 0] * iv * gv.x + bv.x;
        const float x1 = acc[ft][tt][4 * q + 1] * iv * gv.y + bv.y;
        const float x2 = acc[ft][tt][4 * q + 2] * iv * gv.z + bv.z;
        const float x3 = acc[ft][tt][4 * q + 3] * iv * gv.w + bv.w;
        float s0, c0, s1, c1;
        sincos_rev(ph.x, &s0, &c0);
        sincos_rev(ph.y, &s1, &c1);
        // R(-phi) (x, y) = (cos x + sin y, -sin x + cos y)
        uint2 o;
        o.x = pack_bf2(c0 * x0 + s0 * x1, c0 * x1 - s0 * x0);
        o.y = pack_bf2(c1 * x2 + s1 * x3, c1 * x3 - s1 * x2);
        *(uint2*)(outp + (m * HRN + rem) * 2) = o;
      }
    }
  }
}

template <int N>
static hipError_t prologue_run(const ProArgs& a, hipStream_t s) {
  const int ntb = (int)((a.M + PT - 1) / PT);
  const int nfb = (int)((2 * (int64_t)a.H * a.R * N + PF - 1) / PF);
  const int nst = (ntb + 15) / 16, nsf = (nfb + 15) / 16;
  const int64_t blocks = (int64_t)nst * nsf * 256;
  hipLaunchKernelGGL((bc_prologue_kernel<N>), dim3((unsigned)blocks), dim3(512), 0, s, a, ntb, nfb, nsf);
  return hipGetLastError();
}

hipError_t launch_bc_prologue(int N, const ProArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  switch (N) {
    case 16: return prologue_run<16>(a, s);
    case 32: return prologue_run<32>(a, s);
    case 64: return prologue_run<64>(a, s);
    case 128: return prologue_run<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m3
