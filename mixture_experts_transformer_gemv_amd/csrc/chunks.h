// Chunks of the f axis for the weight-streaming down-projection (gfx950).
//
// The down-projection y = h W2 (page "A functional bridge between openai/grok and xai-org/grok-1", architecture
// diagram) is split along its f (input) axis into S chunks whose fp32 partial sums are added by the combine.
// Chunk c covers rows [down_chunk_begin(c), down_chunk_begin(c + 1)) of W2: near-equal parts whose boundaries fall
// on multiples of 128 rows (f a multiple of 128 when S > 1), so that a chunk is whole 64-deep steps of the [in, out]
// kernel and whole 128-deep stages of the [out, in] kernel, and both kernels add the same products into the same
// partial sums.
#pragma once

#include <stdint.h>

namespace gm {

__host__ __device__ inline int down_chunk_begin(int c, int f, int S) {
  return c >= S ? f : int(int64_t(c) * (f / 128) / S) * 128;
}

}  // namespace gm
