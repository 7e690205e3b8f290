// Cross-lane sums and scans for wave64 on gfx950, on the VALU: DPP row
// permutes and the row swaps (v_permlane16_swap / v_permlane32_swap).
#pragma once

#include "m3_common.hpp"

namespace m3 {

// Cross-lane sums and scans on the VALU (DPP and the gfx950 row swaps)
// rather than LDS permutes. dpp<CTRL>(v) is v of the lane the DPP control
// names; lanes outside the 16-lane row read 0 (bound_ctrl).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
// The row swaps exchange rows between their two register operands. Both the
// copy going in and the two results pass through empty asm: without that the
// compiler was seen to treat the two results as one value (the sum came out
// as twice this lane's own value).
__device__ __forceinline__ float swap_sum16(float v) {  // v of lane l plus v of lane l ^ 16
  uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
  asm volatile("" : "+v"(b));
  const auto s = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = s[0];
  b = s[1];
  asm volatile("" : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float swap_sum32(float v) {  // v of lane l plus v of lane l ^ 32
  uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
  asm volatile("" : "+v"(b));
  const auto s = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = s[0];
  b = s[1];
  asm volatile("" : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
// Sum over the lanes whose index differs from this lane's only in bits
// [log2 LO, log2 HI); every lane of such a group receives the group's sum.
// Each step pairs every lane with one holding the sum over the other half of
// its aligned group: lane ^ 1 and lane ^ 2 (quad permutes), the other quad of
// the 8-lane half-row (its mirror, valid once the quads are summed; an LDS
// permute to lane ^ 4 otherwise), lane ^ 8 (row rotation by 8), lane ^ 16 and
// lane ^ 32 (row swaps).
template <int LO, int HI>
__device__ __forceinline__ float lane_sum(float v) {
  if constexpr (LO <= 1 && HI > 1) v += dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  if constexpr (LO <= 2 && HI > 2) v += dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  if constexpr (LO <= 4 && HI > 4) {
    if constexpr (LO == 1) v += dpp<0x141>(v);  // row_half_mirror
    else v += __shfl_xor(v, 4, 64);
  }
  if constexpr (LO <= 8 && HI > 8) v += dpp<0x128>(v);  // row_ror:8
  if constexpr (LO <= 16 && HI > 16) v = swap_sum16(v);
  if constexpr (LO <= 32 && HI > 32) v = swap_sum32(v);
  return v;
}
// v of lane l + O within the 16-lane row (0 past its end), and of lane l - O
template <int O>
__device__ __forceinline__ float row_down(float v) { return dpp<0x100 + O>(v); }  // row_shl:O
template <int O>
__device__ __forceinline__ float row_up(float v) { return dpp<0x110 + O>(v); }    // row_shr:O

// Inclusive scan over the 64 / C slots of C lanes (slot s = lanes C s ..
// C s + C - 1; C = 8 or 16), for each lane position within a slot separately:
// lane l receives v of lanes l, l - C, l - 2C, ... summed.  With C = 8 the
// upper slot of each 16-lane row first adds the lower one (row shift by 8);
// then each row adds the totals of the rows before it, which the row swaps
// bring over: row r ^ 1's total (permlane16_swap) for the odd rows, the total
// of rows 0 and 1 (permlane32_swap of the pair sums) for rows 2 and 3.  Both
// copies going into a swap and its results pass through empty asm, as in
// swap_sum16.
template <int C>
__device__ __forceinline__ float slot_scan(float v, int lane) {
  static_assert(C == 8 || C == 16, "slots of 8 or 16 lanes");
  float tot = v;
  if constexpr (C == 8) {
    v += row_up<8>(v);
    const float rt = dpp<0x128>(v);  // row_ror:8: the lower slot reads the row total of its position
    tot = (lane & 8) ? v : rt;
  }
  uint32_t a = __builtin_bit_cast(uint32_t, tot), b = a;
  asm volatile("" : "+v"(b));
  const auto s = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  uint32_t s0 = s[0], s1 = s[1];
  asm volatile("" : "+v"(s0), "+v"(s1));
  const float prev = __builtin_bit_cast(float, s0);                // odd rows: the total of row r - 1
  uint32_t c = __builtin_bit_cast(uint32_t, prev + __builtin_bit_cast(float, s1)), d = c;  // rows (0, 1) or (2, 3)
  asm volatile("" : "+v"(d));
  const auto q = __builtin_amdgcn_permlane32_swap(c, d, false, false);
  uint32_t q0 = q[0];
  asm volatile("" : "+v"(q0));
  const int row = lane >> 4;
  float add = (row & 1) ? prev : 0.0f;
  if (row >= 2) add += __builtin_bit_cast(float, q0);  // rows 2, 3: the total of rows 0 and 1
  return v + add;
}

}  // namespace m3
