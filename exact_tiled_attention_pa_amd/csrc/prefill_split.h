// Internal interface of the split-key prefill kernel (prefill_split.hip) and the rule
// that chooses between it and the 128-row tiled prefill kernel (prefill.hip).
#pragma once

#include "kernels.h"

namespace pa {

// 32 query rows per workgroup, shared by its waves (8 at head_dim 64, 5 at 128), which
// divide the key tiles among themselves and merge their softmax states at the end.
constexpr int kPrefillSplitBlockM = 32;
// Its LDS holds one workgroup per CU: the automatic choice takes it when its grid fits
// two rounds of the 256 CUs and a sequence may span more than one key tile.  Measured
// with both kernels forced (causal, d = 128, one sequence): 16 heads x 1024 rows (512
// split workgroups) 22.7 us tiled, 16.1 split; 8 x 2048 (512) 40.3, 21.1; 32 x 1024
// (1024) 23.5, 28.8; 64-row chunks of 8 sequences on 4096-key caches, 32 heads (512)
// 116.6, 120.6.
constexpr int kPrefillSplitMaxWorkgroups = 512;

// Which prefill kernel runs: chosen by launch size, or forced to one of the two.
constexpr int kPrefillPathAuto = 0;
constexpr int kPrefillPathTiles = 1;  // prefill_kernel
constexpr int kPrefillPathSplit = 2;  // prefill_split_kernel

inline bool prefill_takes_split(const PrefillArgs& a, int path) {
  if (path != kPrefillPathAuto) return path == kPrefillPathSplit;
  const long long wgs = (long long)a.num_q_heads * a.batch *
                        ((a.max_q_len + kPrefillSplitBlockM - 1) / kPrefillSplitBlockM);
  const long long keys = (long long)a.max_pages_per_seq << a.log2_page_size;
  return wgs <= kPrefillSplitMaxWorkgroups && keys > kPrefillBlockN;
}

hipError_t launch_prefill_split(const PrefillArgs& a, hipStream_t stream);

}  // namespace pa
