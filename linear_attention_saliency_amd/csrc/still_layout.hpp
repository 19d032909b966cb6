// Storage permutations shared by the producer (prep) and consumer (attention) kernels.
//
// A 16x16x32 accumulator leaves lane group g holding rows {4g..4g+3, 16+4g..16+4g+3} of
// each 32-row slice (see the PK assignment in still_common.hpp). When such a result is
// contracted against data staged from memory, the staged operand must hold the same
// 8 indices per lane group. Storing those indices contiguously (position 8g + e for
// index 16*(e/4) + 4g + e%4) lets the consumer fetch each fragment with one 16-byte LDS
// read. The permutation is applied within every 32-element slice.
#pragma once

namespace still {

// position of index k (0..31) inside its 32-slice
__host__ __device__ constexpr int pk_pos32(int k) { return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3); }

// position of index k (any) with the permutation applied per 32-slice
__host__ __device__ constexpr int pk_pos(int k) { return (k & ~31) + pk_pos32(k & 31); }

}  // namespace still
