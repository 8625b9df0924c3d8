// Fragment-major activation layout shared by the batched decoder step's producers (attention,
// residual and activation epilogues, the merge operand) and its weight-streaming products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlt {

// Offset of element [row][k] of a bf16 activation matrix with K columns (K % 64 == 0).  With
// frag == 0 it is row-major.  With frag != 0 it is the fragment-major layout the weight-streaming
// products read as their matrix-core A operand: the 16-byte piece ((i * K/64 + s) * 2 + h) * 64 +
// lane holds X[16 i + lane % 16][64 s + 16 (lane / 16) + 8 h .. + 8], so that one load
// instruction of a wave reads one contiguous kilobyte of a 16-row block.
__device__ __forceinline__ size_t act_offset(int row, int k, int K, int frag) {
  if (!frag) return static_cast<size_t>(row) * K + k;
  const int kk = k & 63;
  const size_t piece =
      ((static_cast<size_t>(row >> 4) * (K >> 6) + (k >> 6)) * 2 + ((kk >> 3) & 1)) * 64 + (row & 15) + 16 * (kk >> 4);
  return piece * 8 + (kk & 7);
}

}  // namespace rlt
