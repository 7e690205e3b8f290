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
// with fp32 accumulation: a block owns 256 features x 256 tokens, its four
// waves (one per SIMD) 128 features x 128 tokens each (4 x 4 tiles of 32 x 32,
// the 256 accumulators in the AGPRs).  In the MFMA's output layout lane l
// holds token l mod 32 and features 8(v/4) + 4(l/32) + (v mod 4) of a tile
// (v < 16), so
//   * every lane holds runs of 4 consecutive features of one token: each
//     rotation pair sits in one lane and is stored as 8 bytes;
//   * the N features of one (token, head, rank) vector lie in the lane and in
//     lane l ^ 32 only: the sum of squares is the lane's own sum plus one row
//     swap.
// K advances 64 at a time through two LDS stages.  Operands come in through
// buffer loads into two register sets, issued two stages ahead: one wave per
// SIMD cannot hide an L2 miss behind other waves, so each load gets two
// stages of products (~1.7 us) to land.
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
__global__ __launch_bounds__(256) void bc_prologue_kernel(ProArgs a, int ntb, int nfb, int nsf) {
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
  const int rowb = (int)(a.D * 2);  // bytes per row of u and W (D <= 2^20)

  // ---- operand tiles through buffer resources: a uniform base at the tile's
  // first row and a byte count that ends at its last valid row, so rows past
  // F or M read as zeros; thread rows tid/8 + 32 i, 16-byte chunk tid % 8
  const int nfr = (int)(F - f0 < PF ? F - f0 : PF), ntr = (int)(a.M - m0 < PT ? a.M - m0 : PT);
  const __amdgpu_buffer_rsrc_t rsw =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.W + f0 * rowb), 0, nfr * rowb, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsu =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.u + m0 * rowb), 0, ntr * rowb, 0x00020000);
  const int lrow = tid >> 3, lch = tid & 7;
  const int voff = lrow * rowb + lch * 16;
  const int loff = soff(lrow, lch);  // LDS byte offset of row lrow; rows + 32 i add 4096 i
  uint4 xw[8], xu[8], yw[8], yu[8];  // two register sets of one stage each
  // stage s holds k-block s - pad: with an odd number of 64-k blocks a zero
  // stage comes first (its offsets lie past the resource, which reads zeros),
  // so the loop below always runs whole pairs of stages
  const int nkb = (int)(a.D / PK), pad = nkb & 1, nst2 = nkb + pad;
  auto load = [&](uint4* sw_, uint4* su_, int st) {
    const int kb = st - pad;
    const bool out = kb < 0 || kb >= nkb;  // a zero stage (before the first or past the last block)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int so = out ? 0x40000000 : i * 32 * rowb + kb * 128;
      sw_[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsw, voff, so, 0));
      su_[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsu, voff, so, 0));
    }
  };
  auto stage = [&](const uint4* sw_, const uint4* su_, int st) {
    char* bw = smem + st * 2 * TILE_BYTES + loff;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *(uint4*)(bw + i * 4096) = sw_[i];
      *(uint4*)(bw + TILE_BYTES + i * 4096) = su_[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int ft = 0; ft < 4; ++ft)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ft][tt][v] = 0.0f;

  const int l32 = lane & 31, lh = lane >> 5;
  // Operand rows start at multiples of 32, so a row's swizzle depends on the
  // lane only: one base address per 16-k step, the tile offsets (4096 bytes
  // per 32 rows) as immediates.  The lane values pass through an empty asm in
  // every stage so that the compiler recomputes the bases instead of keeping
  // one register per (stage, step, tile) for the whole loop.
  // The products of the stage in LDS buffer st, with the register set (wsrc,
  // usrc) written to the other buffer in between: that buffer was last read
  // before the previous barrier, so only the barrier after this stage remains
  // on the path.
  auto compute = [&](int st, const uint4* wsrc, const uint4* usrc) {
    int ll = l32, hh = lh;
    asm volatile("" : "+v"(ll), "+v"(hh));
    const int fsl = fsw<8>(ll);
    const int ba = st * 2 * TILE_BYTES + wf * 16384 + ll * 128;
    const int bb = st * 2 * TILE_BYTES + TILE_BYTES + wt * 16384 + ll * 128;
    // operands of step s + 1 are read while the products of step s run
    bf16x8 fa[2][4], fbv[2][4];
    auto rd = [&](int s, int bsel) {
      const int co = ((2 * s + hh) ^ fsl) << 4;
      const char* pa = smem + ba + co;
      const char* pb = smem + bb + co;
#pragma unroll
      for (int ft = 0; ft < 4; ++ft) fa[bsel][ft] = as_bf16x8(*(const uint4*)(pa + ft * 4096));
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) fbv[bsel][tt] = as_bf16x8(*(const uint4*)(pb + tt * 4096));
    };
    rd(0, 0);
    stage(wsrc, usrc, st ^ 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) rd(s + 1, (s + 1) & 1);
#pragma unroll
      for (int ft = 0; ft < 4; ++ft)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[ft][tt] = mfma32(fa[s & 1][ft], fbv[s & 1][tt], acc[ft][tt]);
    }
    // instruction order: the first step's 8 operand reads, then for steps
    // 0..2 one read of the next step after every 2 products with the 16 LDS
    // writes of the other buffer spread over the first 16 of those slots,
    // then the last step's 16 products (otherwise each read lands just
    // before its use and the writes pile up at the end)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i < 16) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
  };

  // stage kk sits in LDS buffer kk % 2; the loads of stage kk + 2 are issued
  // before the products of stage kk, so each has two stages of products to
  // land before it is written to LDS.  Every load and LDS write is issued on
  // every pass (stages past the end read zeros): on a single path the
  // compiler's wait counts let the younger loads stay in flight, while a
  // skipped load on one path makes every wait drain all of them.  (An exit in
  // the middle of the pair, or a branch around its second half, also costs
  // hundreds of spilled registers: the accumulators would be live on two
  // paths.)
  load(xw, xu, 0);
  load(yw, yu, 1);
  stage(xw, xu, 0);
  __syncthreads();
  for (int kk = 0; kk < nst2; kk += 2) {
    load(xw, xu, kk + 2);
    compute(0, yw, yu);  // stage kk; stage kk + 1 into buffer 1
    __syncthreads();
    load(yw, yu, kk + 3);
    compute(1, xw, xu);  // stage kk + 1; stage kk + 2 into buffer 0
    __syncthreads();
  }

  // ---- epilogue: RMS over each N-feature vector, gain, bias, rotation, store
  constexpr int G = 128 / N;  // vectors per token in the wave's 128 features
  // feature indices fit 32 bits (F <= 2 * 65535 * 4 * 128)
  const uint32_t HRN = (uint32_t)a.H * (uint32_t)a.R * N;
  const uint32_t shRN = (uint32_t)__builtin_ctz((unsigned)(a.R * N));  // R N is a power of 2
  const uint32_t fw0 = (uint32_t)f0 + wf * 128;  // first feature of the wave
  const int K2 = N / 2;
  // The LDS is free after the last stage: each wave stages, per half of its
  // 128 tokens, the angles of its 64 pairs (16 KB) and its output rows
  // (16 KB), so that global reads and writes are whole 16-byte pieces of
  // contiguous rows instead of 8 bytes from 32 rows per instruction.  Rows are
  // 256 bytes of 16 chunks; chunk c of row j sits at c ^ (j mod 16).
  char* phs = smem + wave * 32768;
  char* ous = phs + 16384;
  // angle column of pair group g (pairs 4g..4g+3 = features fw0 + 8g .. + 7,
  // one vector of one head, consecutive pairs)
  auto col = [&](int g) -> int64_t {
    const uint32_t f = fw0 + 8 * g;
    const uint32_t rem = f >= HRN ? f - HRN : f;
    return (int64_t)(rem >> shRN) * K2 + ((rem & (N - 1)) >> 1);
  };
  const int jl = lane >> 4, gl = lane & 15;  // staging: 4 rows x 16 chunks per instruction
  const bool fvalid = (int64_t)fw0 + 8 * gl < F;
  const int64_t colg = fvalid ? col(gl) : 0;
  // the angles of both halves are requested at once (the staging registers of
  // the main loop are free now): the second half's arrive during the first's
  float4 phr[2][16];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // every lane loads (clamped to a valid token and column) and invalid
      // ones drop the value: a load skipped on one path would make the
      // compiler's waits drain the other half's loads too
      const int64_t m = m0 + wt * 128 + hf * 64 + 4 * i + jl;
      const int64_t mc = m < a.M ? m : a.M - 1;
      const float4 v = *(const float4*)(a.phi + mc * (int64_t)a.H * K2 + colg);
      phr[hf][i] = fvalid && m < a.M ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  auto write_phi = [&](int hf) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int jj = 4 * i + jl;
      *(float4*)(phs + jj * 256 + ((gl ^ (jj & 15)) << 4)) = phr[hf][i];
    }
  };
  // normalisation, gain, bias and rotation of the half's two 32-token tiles
  // into the staged output rows
  float4 gvs[16], bvs[16];
  auto compute_half = [&](int hf) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int tt = 2 * hf + t2;
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
      float inv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) inv[g] = rsqrtf(swap_sum32(ss[g]) * (1.0f / N) + a.eps);
      const int j = t2 * 32 + l32;  // row of the token in the half
#pragma unroll
      for (int ft = 0; ft < 4; ++ft) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = ft * 4 + q;  // 16-byte chunk (8 features) of the lane's 4 features
          const float4 gv = gvs[c], bv = bvs[c];
          // pairs 2(c*2 + lh) and + 1 within group c of the angle row
          const float2 ph = *(const float2*)(phs + j * 256 + ((c ^ (j & 15)) << 4) + lh * 8);
          const float iv = inv[(ft * 32 + 8 * q) / N];
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
          *(uint2*)(ous + j * 256 + ((c ^ (j & 15)) << 4) + lh * 8) = o;
        }
      }
    }
  };
  // whole rows out: chunk gl of row jj holds features fw0 + 8 gl .. + 7 of
  // token mh + jj, all in B_rot or all in C_rot (H R N is a multiple of 8)
  const uint32_t fo = fw0 + 8 * gl;
  const bool oc = fo >= HRN;
  char* dst = (char*)(oc ? a.C_rot : a.B_rot) + (int64_t)(oc ? fo - HRN : fo) * 2;
  auto store_half = [&](int hf) {
    const int64_t mh = m0 + wt * 128 + hf * 64;  // first token of the half
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int jj = 4 * i + jl;
      const uint4 v = *(const uint4*)(ous + jj * 256 + ((gl ^ (jj & 15)) << 4));
      // streamed out: the rows are not read again here, and the operand
      // tiles that later blocks re-read stay in L2
      if (fvalid && mh + jj < a.M)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), (u32x4*)(dst + (mh + jj) * (int64_t)HRN * 2));
    }
  };
  // Order: every load (angles, gain, bias) is requested before the first
  // store.  One counter tracks vector loads and stores alike, and the stores
  // are conditional, so a wait for a load issued after a store would also
  // wait for the store.
  write_phi(0);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const uint32_t f = fw0 + 8 * c + 4 * lh;
    const bool ok = (int64_t)f < F;
    gvs[c] = a.gain && ok ? *(const float4*)(a.gain + f) : make_float4(1.f, 1.f, 1.f, 1.f);
    bvs[c] = a.bias && ok ? *(const float4*)(a.bias + f) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
  compute_half(0);
  __syncthreads();
  write_phi(1);  // the angle rows are free: every wave has finished half 0
  store_half(0);
  __syncthreads();
  compute_half(1);
  __syncthreads();
  store_half(1);
}

template <int N>
static hipError_t prologue_run(const ProArgs& a, hipStream_t s) {
  const int ntb = (int)((a.M + PT - 1) / PT);
  const int nfb = (int)((2 * (int64_t)a.H * a.R * N + PF - 1) / PF);
  const int nst = (ntb + 15) / 16, nsf = (nfb + 15) / 16;
  const int64_t blocks = (int64_t)nst * nsf * 256;
  hipLaunchKernelGGL((bc_prologue_kernel<N>), dim3((unsigned)blocks), dim3(256), 0, s, a, ntb, nfb, nsf);
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
