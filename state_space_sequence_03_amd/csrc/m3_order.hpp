// Block order of the walkers (one block per (b,h) sequence or per sequence
// segment).  Workgroups are dispatched to the 8 XCDs in turn, each XCD with
// its own L2.  The per-token scalars dt, A, lam (and their gradients) are laid
// out (B, L, H): the heads of one token are adjacent, 32 bytes for 8 heads.
// When the grid is a multiple of 64 blocks and B*H a multiple of 8, XCD x is
// given, in every group of 64 blocks, 8 adjacent heads at the same segment, so
// that such a 32-byte piece is fetched into (and written from) one L2 for 8
// walkers instead of being fetched by 8 XCDs.  Otherwise blocks map in order
// (block = bh * S + seg).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

__device__ __forceinline__ void walker_of_block(int64_t i, int64_t grid, int64_t BH, int64_t S, int64_t& bh,
                                                int64_t& seg) {
  if (grid % 64 == 0 && BH % 8 == 0) {
    const int64_t slot = i >> 3, lin = (slot >> 3) * 64 + (i & 7) * 8 + (slot & 7);  // a bijection of [0, grid)
    seg = lin / BH;
    bh = lin % BH;
  } else {
    seg = i % S;
    bh = i / S;
  }
}

}  // namespace m3
