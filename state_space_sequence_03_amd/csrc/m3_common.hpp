// Shared device helpers for the gfx950 kernels: io-dtype traits, bf16
// rounding, vector loads/stores and the MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace m3 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

struct bf16_t {  // storage tag for bf16 io
  u16 bits;
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950);
// lo goes to bits 0..15.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ u16 f2bf(float f) { return (u16)(pack_bf2(f, 0.0f) & 0xffffu); }
__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// io traits: elements per 16-byte vector and conversions to/from fp32.
// ---------------------------------------------------------------------------
template <typename T>
struct io;

template <>
struct io<float> {
  static constexpr int VEC = 4;       // elements per 16 B
  static constexpr int BYTES = 4;
  typedef float4 vec;
  __device__ static void unpack(const vec& v, float* f) { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
  __device__ static vec pack(const float* f) { return make_float4(f[0], f[1], f[2], f[3]); }
  __device__ static float load1(const void* p, int64_t i) { return ((const float*)p)[i]; }
  __device__ static void store1(void* p, int64_t i, float v) { ((float*)p)[i] = v; }
  // four consecutive elements (one vector access)
  __device__ static void load4(const void* p, int64_t i, float* f) {
    const float4 v = *(const float4*)((const float*)p + i);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
  // two consecutive elements, i even (one 8-byte access)
  __device__ static void load2(const void* p, int64_t i, float& f0, float& f1) {
    const float2 v = *(const float2*)((const float*)p + i);
    f0 = v.x; f1 = v.y;
  }
  // four consecutive elements, i a multiple of 4 (one 16-byte access)
  __device__ static void store4(void* p, int64_t i, const float* f) {
    *(float4*)((float*)p + i) = make_float4(f[0], f[1], f[2], f[3]);
  }
};

template <>
struct io<bf16_t> {
  static constexpr int VEC = 8;
  static constexpr int BYTES = 2;
  typedef uint4 vec;
  __device__ static void unpack(const vec& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static vec pack(const float* f) {
    vec v;
    v.x = pack_bf2(f[0], f[1]);
    v.y = pack_bf2(f[2], f[3]);
    v.z = pack_bf2(f[4], f[5]);
    v.w = pack_bf2(f[6], f[7]);
    return v;
  }
  __device__ static float load1(const void* p, int64_t i) { return bf2f(((const u16*)p)[i]); }
  __device__ static void store1(void* p, int64_t i, float v) { ((u16*)p)[i] = f2bf(v); }
  // four consecutive elements (one 8-byte access; AMDGPU global loads accept
  // 2-byte-aligned addresses)
  __device__ static void load4(const void* p, int64_t i, float* f) {
    const uint2 v = *(const uint2*)((const u16*)p + i);
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  }
  // two consecutive elements, i even (one 4-byte access)
  __device__ static void load2(const void* p, int64_t i, float& f0, float& f1) {
    const uint32_t v = *(const uint32_t*)((const u16*)p + i);
    f0 = bf_lo(v); f1 = bf_hi(v);
  }
  // four consecutive elements, i a multiple of 4 (one 8-byte access)
  __device__ static void store4(void* p, int64_t i, const float* f) {
    *(uint2*)((u16*)p + i) = make_uint2(pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]));
  }
};

// 16-byte global load / store of an io vector.
template <typename T>
__device__ __forceinline__ typename io<T>::vec ldg16(const void* base, int64_t elem) {
  return *(const typename io<T>::vec*)((const char*)base + elem * io<T>::BYTES);
}
template <typename T>
__device__ __forceinline__ void stg16(void* base, int64_t elem, const typename io<T>::vec& v) {
  *(typename io<T>::vec*)((char*)base + elem * io<T>::BYTES) = v;
}
// The same with a non-temporal hint, for outputs that are written once and
// not read again by the kernel (streamed past the caches).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ void stg16_nt(void* base, int64_t elem, const typename io<T>::vec& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), (u32x4*)((char*)base + elem * io<T>::BYTES));
}

// ---------------------------------------------------------------------------
// MFMA wrappers.  Lane l of a wave: m = l % 16, g = l / 16.
//  16x16x32 bf16: A lane holds A[m][8g+j], B lane holds B[8g+j][m] (j < 8);
//  16x16x4 f32:   A lane holds A[m][g],    B lane holds B[g][m];
//  both:          D lane holds D[4g+i][m] (i < 4).
// A contraction only needs A's element j and B's element j of lanes with the
// same g to refer to the same k, so callers may permute k freely as long as
// both operands use the same permutation.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16-byte fp32 loads / stores with a non-temporal hint (streamed data).
__device__ __forceinline__ f32x4 ld_nt(const float* p) { return __builtin_nontemporal_load((const f32x4*)p); }
__device__ __forceinline__ void st_nt(float* p, const f32x4& v) { __builtin_nontemporal_store(v, (f32x4*)p); }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Inclusive prefix sum over the 64 lanes of a wave, on the VALU: row shifts
// by 1, 2, 4, 8 inside each 16-lane row (lanes shifted in from outside the
// row read 0), then the last lane of a row added to the rows after it (row
// broadcasts 15 and 31, masked to the receiving rows).
__device__ __forceinline__ float wave_incl_scan(float v) {
  auto shr = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), decltype(ctrl)::value,
                                                                 0xf, 0xf, true));
  };
  v += shr(v, std::integral_constant<int, 0x111>{});  // row_shr:1
  v += shr(v, std::integral_constant<int, 0x112>{});  // row_shr:2
  v += shr(v, std::integral_constant<int, 0x114>{});  // row_shr:4
  v += shr(v, std::integral_constant<int, 0x118>{});  // row_shr:8
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));
  return v;
}

// 8 bytes per lane from LDS with the gfx950 16-bit transpose read
// (ds_read_b64_tr_b16): within each group of 16 lanes, output lane i holds, as
// element j, element i % 4 of the 8 bytes addressed by input lane 4j + i/4.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ uint2 lds_tr16(const void* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// sin and cos of x after a two-constant reduction by 2*pi (Cody-Waite); the
// reduced argument lies in [-pi, pi] where the hardware sine/cosine are
// accurate to about 1e-6.
__device__ __forceinline__ void fast_sincos(float x, float* s, float* c) {
  const float kInv2Pi = 0.15915494309189535f;
  const float k2PiHi = 6.28318548202514648f;     // float(2 pi)
  const float k2PiLo = -1.7484555314695172e-07f;  // 2 pi - float(2 pi)
  const float n = rintf(x * kInv2Pi);
  float r = fmaf(-n, k2PiHi, x);
  r = fmaf(-n, k2PiLo, r);
  *s = __sinf(r);
  *c = __cosf(r);
}

// sin and cos of x (radians) with the hardware sine/cosine, which take their
// argument in revolutions: x / (2 pi) reduced to [-1/2, 1/2] by subtracting
// the nearest integer (exact), so the only added error is the rounding of the
// product, |x| / (2 pi) * 2^-24 revolutions.
__device__ __forceinline__ void sincos_rev(float x, float* s, float* c) {
  const float y = x * 0.15915494309189535f;
  const float r = y - rintf(y);
  *s = __builtin_amdgcn_sinf(r);
  *c = __builtin_amdgcn_cosf(r);
}

// a.lo * b.lo - a.hi * b.hi over bf16 pairs with an fp32 sum: the dot product
// instruction with the high half of b negated by its operand modifier.
__device__ __forceinline__ float dot2_bf16_neghi(uint32_t a, uint32_t b) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// Swizzle of arrays of rows of CPR 16-byte columns: column c of row r is
// stored at column c ^ f(r), with f depending on r mod 16 only (the pattern
// repeats for every 16-row tile).  With 64 four-byte banks (16 groups of 16
// bytes), 16 consecutive rows read at one logical column fall in 16 distinct
// bank groups: rows of 128 bytes use two rows per bank period, rows of 256
// bytes one.
template <int CPR>
__device__ __forceinline__ int fsw(int row) {
  if constexpr (CPR == 16) return row & 15;
  else return (row & 7) ^ ((row >> 3) & 1);
}
template <int CPR>
__device__ __forceinline__ int swz(int row, int chunk) { return row * (CPR * 16) + ((chunk ^ fsw<CPR>(row)) << 4); }
// d[k] of 16-lane row r becomes d[r] of row k: a 4 x 4 transpose of (row of
// the wave) x (register) with the gfx950 row swaps (permlane32_swap exchanges
// rows 2,3 of its first operand with rows 0,1 of its second; permlane16_swap
// the odd rows of the first with the even rows of the second)
__device__ __forceinline__ void transpose_rows4(uint32_t* d) {
  auto s = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
  d[0] = s[0];
  d[2] = s[1];
  s = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
  d[1] = s[0];
  d[3] = s[1];
  s = __builtin_amdgcn_permlane16_swap(d[0], d[1], false, false);
  d[0] = s[0];
  d[1] = s[1];
  s = __builtin_amdgcn_permlane16_swap(d[2], d[3], false, false);
  d[2] = s[0];
  d[3] = s[1];
}

}  // namespace m3
