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
// read back.  A small pre-pass over dt and theta (rope.hip) writes cos and
// sin of the angles phi_t once per (token, head, pair), as fp16 pairs, which
// every rank of B and C then uses.
//
// The product is computed transposed, D^T = W u^T, on bf16 32x32x16 MFMAs
// with fp32 accumulation: a block owns 256 features x 256 tokens, its eight
// waves (two per SIMD) 128 features x 64 tokens each (4 x 2 tiles of 32 x 32,
// 128 accumulators).  In the MFMA's output layout lane l holds token l mod 32
// and features 8(v/4) + 4(l/32) + (v mod 4) of a tile (v < 16), so
//   * every lane holds runs of 4 consecutive features of one token: each
//     rotation pair sits in one lane and is stored as 8 bytes;
//   * the N features of one (token, head, rank) vector lie in the lane and in
//     lane l ^ 32 only: the sum of squares is the lane's own sum plus one row
//     swap.
// K advances 64 at a time through two LDS stages.  Operands go from global
// memory straight into LDS (buffer_load ... lds: one wave instruction fills
// 1 KB, lane l's 16 bytes at l * 16), one stage ahead: no staging registers
// and no LDS write instructions (4.48 -> 4.24 ms against loads into
// registers two stages ahead, then LDS writes).  With two waves per SIMD one
// wave's operand reads and barrier waits overlap the other's products
// (measured against one wave per SIMD with 128 x 128 per wave: 5.04 ->
// 4.47 ms at the 1.5B shapes; a 128 x 256 tile with two blocks per CU, so
// that one block's epilogue overlaps the other's products, took 5.19 ms:
// the smaller tile's extra operand traffic and barriers cost more).
// Tiles of 256 rows x 128 bytes are swizzled by 16-byte chunks so that the
// 32 rows an operand read touches fall in distinct bank groups; the loads
// apply the swizzle on the global side (each lane fetches the chunk that
// belongs at its LDS slot).
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


__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

// Eight waves per 256 x 256 tile, two per SIMD: wave w owns features
// 128 (w & 1) .. + 127 and tokens 64 (w >> 1) .. + 63 of the tile (4 x 2
// tiles of 32 x 32, 128 accumulators), so that one wave's operand reads,
// barrier waits and epilogue latency overlap the other wave's products on
// the same SIMD.  The epilogue runs in 32-token halves (16 KB of LDS per
// wave), with the gain and bias of the tile's features staged in LDS.
template <int N>
__global__ __launch_bounds__(512) void bc_prologue_kernel(ProArgs a, int ntb, int nfb, int nsf) {
  const int bid = blockIdx.x;
  const int xcd = bid & 7, j = bid >> 3;
  const int sup = j >> 5, w32 = j & 31;
  const int tb = (sup / nsf) * 16 + (xcd >> 1) * 4 + (w32 >> 3);
  const int fb = (sup % nsf) * 16 + (xcd & 1) * 8 + (w32 & 7);
  if (tb >= ntb || fb >= nfb) return;

  constexpr int EPI_GB = 8 * 16384;  // gain and bias of the tile's 256 features after the epilogue rows
  __shared__ __attribute__((aligned(16))) char smem[EPI_GB + 2 * 256 * 4];
  static_assert(2 * 2 * TILE_BYTES <= EPI_GB, "stages fit below the gain/bias rows");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wf = wave & 1, wt = wave >> 1;
  const int64_t F = 2 * (int64_t)a.H * a.R * N;
  const int64_t f0 = (int64_t)fb * PF, m0 = (int64_t)tb * PT;
  const int rowb = (int)(a.D * 2);

  const int nfr = (int)(F - f0 < PF ? F - f0 : PF), ntr = (int)(a.M - m0 < PT ? a.M - m0 : PT);
  const __amdgpu_buffer_rsrc_t rsw =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.W + f0 * rowb), 0, nfr * rowb, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsu =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.u + m0 * rowb), 0, ntr * rowb, 0x00020000);
  // thread rows tid / 8 + 64 i (i < 4), 16-byte chunk tid % 8; rows 64 apart
  // share the swizzle, so they are 8192 bytes apart in LDS
  // stage loads straight into LDS (buffer_load ... lds): instruction i of wave w
  // fills rows 64 i + 8 w .. + 7 of a tile (1 KB, lane l -> 16 bytes at l * 16),
  // so lane l loads the global chunk that the swizzle puts at its slot
  const int wl = lane >> 3, wp = lane & 7;
  const int wch = wp ^ wl ^ (wave & 1);                     // fsw<8>(row) ^ slot
  const int dvoff = (8 * wave + wl) * rowb + wch * 16;
  const int nkb = (int)(a.D / PK), pad = nkb & 1, nst2 = nkb + pad;
  typedef __attribute__((address_space(3))) void lds_void;
  auto dma = [&](int buf, int st) {
    const int kb = st - pad;
    const bool out = kb < 0 || kb >= nkb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int so = out ? 0x40000000 : i * 64 * rowb + kb * 128;
      char* dw = smem + buf * 2 * TILE_BYTES + (64 * i + 8 * wave) * 128;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void*)dw, 16, dvoff, so, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsu, (lds_void*)(dw + TILE_BYTES), 16, dvoff, so, 0, 0);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int ft = 0; ft < 4; ++ft)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ft][tt][v] = 0.0f;

  const int l32 = lane & 31, lh = lane >> 5;
  auto compute = [&](int st) {
    int ll = l32, hh = lh;
    asm volatile("" : "+v"(ll), "+v"(hh));
    const int fsl = fsw<8>(ll);
    const int ba = st * 2 * TILE_BYTES + wf * 16384 + ll * 128;
    const int bb = st * 2 * TILE_BYTES + TILE_BYTES + wt * 8192 + ll * 128;
    bf16x8 fa[2][4], fbv[2][2];
    auto rd = [&](int s, int bsel) {
      const int co = ((2 * s + hh) ^ fsl) << 4;
      const char* pa = smem + ba + co;
      const char* pb = smem + bb + co;
#pragma unroll
      for (int ft = 0; ft < 4; ++ft) fa[bsel][ft] = as_bf16x8(*(const uint4*)(pa + ft * 4096));
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) fbv[bsel][tt] = as_bf16x8(*(const uint4*)(pb + tt * 4096));
    };
    rd(0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) rd(s + 1, (s + 1) & 1);
#pragma unroll
      for (int ft = 0; ft < 4; ++ft)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) acc[ft][tt] = mfma32(fa[s & 1][ft], fbv[s & 1][tt], acc[ft][tt]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < 18) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  dma(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  for (int kk = 0; kk < nst2; kk += 2) {
    dma(1, kk + 1);
    compute(0);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    dma(0, kk + 2);
    compute(1);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  }

  // ---- epilogue: RMS over each N-feature vector, gain, bias, rotation, store
  constexpr int G = 128 / N;
  const uint32_t HRN = (uint32_t)a.H * (uint32_t)a.R * N;
  const uint32_t shRN = (uint32_t)__builtin_ctz((unsigned)(a.R * N));
  const uint32_t fw0 = (uint32_t)f0 + wf * 128;
  const int K2 = N / 2;
  char* phs = smem + wave * 16384;  // angle rows of the half (32 x 256 bytes)
  char* ous = phs + 8192;           // output rows of the half (32 x 256 bytes)
  float* gsh = (float*)(smem + EPI_GB);  // [256] gain, then [256] bias
  if (tid < 64) {
    const uint32_t f = (uint32_t)f0 + 4 * tid;
    const bool ok = (int64_t)f < F;
    const float4 gv = a.gain && ok ? *(const float4*)(a.gain + f) : make_float4(1.f, 1.f, 1.f, 1.f);
    const float4 bv = a.bias && ok ? *(const float4*)(a.bias + f) : make_float4(0.f, 0.f, 0.f, 0.f);
    *(float4*)(gsh + 4 * tid) = gv;
    *(float4*)(gsh + 256 + 4 * tid) = bv;
  }
  auto col = [&](int g) -> int64_t {
    const uint32_t f = fw0 + 8 * g;
    const uint32_t rem = f >= HRN ? f - HRN : f;
    return (int64_t)(rem >> shRN) * K2 + ((rem & (N - 1)) >> 1);
  };
  const int jl = lane >> 4, gl = lane & 15;
  const bool fvalid = (int64_t)fw0 + 8 * gl < F;
  const int64_t colg = fvalid ? col(gl) : 0;
  uint4 phr[2][8];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + wt * 64 + hf * 32 + 4 * i + jl;
      const int64_t mc = m < a.M ? m : a.M - 1;
      const uint4 v = *(const uint4*)(a.cs + mc * (int64_t)a.H * K2 + colg);
      phr[hf][i] = fvalid && m < a.M ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  auto write_phi = [&](int hf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int jj = 4 * i + jl;
      *(uint4*)(phs + jj * 256 + ((gl ^ (jj & 15)) << 4)) = phr[hf][i];
    }
  };
  auto compute_half = [&](int tt) {
    float ss[G];
#pragma unroll
    for (int g = 0; g < G; ++g) ss[g] = 0.0f;
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float x = acc[ft][tt][v];
        ss[(ft * 32 + 8 * (v >> 2)) / N] += x * x;
      }
    float inv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) inv[g] = rsqrtf(swap_sum32(ss[g]) * (1.0f / N) + a.eps);
    const int jr = l32;  // row of the token in the half
#pragma unroll
    for (int ft = 0; ft < 4; ++ft) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = ft * 4 + q;
        const int fo = wf * 128 + 8 * c + 4 * lh;  // the lane's 4 features in the tile
        const float4 gv = *(const float4*)(gsh + fo), bv = *(const float4*)(gsh + 256 + fo);
        // fp16 (cos, sin) of pairs 2(c*2 + lh) and + 1
        const uint2 pc = *(const uint2*)(phs + jr * 256 + ((c ^ (jr & 15)) << 4) + lh * 8);
        const float iv = inv[(ft * 32 + 8 * q) / N];
        const float x0 = acc[ft][tt][4 * q + 0] * iv * gv.x + bv.x;
        const float x1 = acc[ft][tt][4 * q + 1] * iv * gv.y + bv.y;
        const float x2 = acc[ft][tt][4 * q + 2] * iv * gv.z + bv.z;
        const float x3 = acc[ft][tt][4 * q + 3] * iv * gv.w + bv.w;
        const f16x2 h0 = __builtin_bit_cast(f16x2, pc.x), h1 = __builtin_bit_cast(f16x2, pc.y);
        const float c0 = (float)h0[0], s0 = (float)h0[1], c1 = (float)h1[0], s1 = (float)h1[1];
        uint2 o;
        o.x = pack_bf2(c0 * x0 + s0 * x1, c0 * x1 - s0 * x0);
        o.y = pack_bf2(c1 * x2 + s1 * x3, c1 * x3 - s1 * x2);
        *(uint2*)(ous + jr * 256 + ((c ^ (jr & 15)) << 4) + lh * 8) = o;
      }
    }
  };
  const uint32_t fo = fw0 + 8 * gl;
  const bool oc = fo >= HRN;
  char* dst = (char*)(oc ? a.C_rot : a.B_rot) + (int64_t)(oc ? fo - HRN : fo) * 2;
  auto store_half = [&](int hf) {
    const int64_t mh = m0 + wt * 64 + hf * 32;
#pragma unroll 4
    for (int i = 0; i < 8; ++i) {
      const int jj = 4 * i + jl;
      const uint4 v = *(const uint4*)(ous + jj * 256 + ((gl ^ (jj & 15)) << 4));
      if (fvalid && mh + jj < a.M)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), (u32x4*)(dst + (mh + jj) * (int64_t)HRN * 2));
    }
  };
  write_phi(0);
  __syncthreads();
  compute_half(0);
  __syncthreads();
  write_phi(1);
  store_half(0);
  __syncthreads();
  compute_half(1);
  __syncthreads();
  store_half(1);
}



// Blocks of one launch: a dispatch holds fewer than 2^32 work-items.
constexpr int64_t kMaxPrologueBlocks = ((int64_t(1) << 32) - 1) / 512;

template <int N>
static hipError_t prologue_run(const ProArgs& a, hipStream_t s) {
  // Token rows go in slices of whole 16 x 16 tile groups, one launch each, so
  // that every call the ABI accepts stays within the dispatch limit.
  const int nfb = (int)((2 * (int64_t)a.H * a.R * N + PF - 1) / PF);
  const int nsf = (nfb + 15) / 16;
  const int64_t groups = kMaxPrologueBlocks / ((int64_t)nsf * 256);
  if (groups < 1) return hipErrorInvalidValue;  // the ABI rejects such feature counts first
  const int64_t rows = groups * 16 * PT;
  for (int64_t m0 = 0; m0 < a.M; m0 += rows) {
    ProArgs b = a;
    b.M = a.M - m0 < rows ? a.M - m0 : rows;
    b.u = (const char*)a.u + m0 * a.D * 2;
    b.cs = a.cs + m0 * (int64_t)a.H * (N / 2);
    b.B_rot = (char*)a.B_rot + m0 * (int64_t)a.H * a.R * N * 2;
    b.C_rot = (char*)a.C_rot + m0 * (int64_t)a.H * a.R * N * 2;
    const int ntb = (int)((b.M + PT - 1) / PT);
    const int64_t blocks = (int64_t)((ntb + 15) / 16) * nsf * 256;
    hipLaunchKernelGGL((bc_prologue_kernel<N>), dim3((unsigned)blocks), dim3(512), 0, s, b, ntb, nfb, nsf);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
