// Internal launch interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* q_start;
  uint16_t* out;
  float scale;
  int causal;
  int batch;
  int num_q_heads;
  int num_kv_heads;
  int head_dim;
  int log2_page_size;
  int max_pages_per_seq;
  int max_q_len;
  int window;  // sliding-window length (0: none); causal only
};

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint16_t* out;
  float* ws_o;        // [batch, num_q_heads, max_splits, head_dim]
  float* ws_ml;       // [batch, num_q_heads, max_splits, 2]  (m in log2 units, l)
  int32_t* plan;      // [2 + batch * max_splits]: claim counter, pair count, pairs
  float scale;
  int batch;
  int num_q_heads;
  int num_kv_heads;
  int head_dim;
  int log2_page_size;
  int max_pages_per_seq;
  int split_tokens;
  int max_splits;
  int window;  // sliding-window length (0: none)
};

// Query heads per K/V head from which decode reads each K/V page once per group.
constexpr int kGqaMinGroup = 4;

inline bool decode_grouped(const DecodeArgs& a) {
  return a.num_q_heads / a.num_kv_heads >= kGqaMinGroup;
}

// Splits of a windowed one-head-per-row decode: laid back from the sequence end, so a
// window of w keys takes ceil(min(w, L) / split_tokens) of them (decode.hip).
__host__ __device__ inline int window_split_count(int seq_len, int window, int split_tokens) {
  const int w = seq_len < window ? seq_len : window;
  return w > 0 ? (w + split_tokens - 1) / split_tokens : 0;
}

// Grid rows of the grouped-head decode (decode_gqa.hip).  Without a window row y is
// split y.  With a sliding window only the splits that can hold keys inside it are
// launched: the splits stay at multiples of split_tokens and the rows count back from
// each sequence's last split (a window of w keys touches at most ceil(w / split_tokens)
// + 1 of them), grid row y walking split (L_b - 1) / split_tokens - y (decode_split_of).
// The one-head-per-row decode takes its work from a list instead (decode.hip).
inline int decode_grid_splits(const DecodeArgs& a) {
  if (a.window <= 0) return a.max_splits;
  const int n = (a.window + a.split_tokens - 1) / a.split_tokens + 1;
  return n < a.max_splits ? n : a.max_splits;
}

struct KvAppendArgs {
  const uint16_t* k_new;  // [num_tokens, num_kv_heads, head_dim]
  const uint16_t* v_new;
  const int32_t* seq_ids;    // [num_tokens]
  const int32_t* positions;  // [num_tokens]
  uint16_t* k_pool;
  uint16_t* v_pool;
  const int32_t* block_table;
  int num_tokens;
  int num_seqs;
  int num_pages;
  int log2_page_size;
  int max_pages_per_seq;
  int row_elems;  // num_kv_heads * head_dim (a multiple of 8)
};

struct CopyPagesArgs {
  uint16_t* k_pool;
  uint16_t* v_pool;
  const int32_t* src_pages;  // [num_copies]
  const int32_t* dst_pages;  // [num_copies]
  int num_copies;
  int num_pages;
  size_t page_bytes;  // page_size * num_kv_heads * head_dim * 2 (a multiple of 16)
};

// Rows of queries per prefill workgroup (4 waves x 32 rows) and keys per tile.
constexpr int kPrefillBlockM = 128;
constexpr int kPrefillBlockN = 64;

// Keys per decode split when pages are at most this long (a split's chunk pages are
// fetched one per lane, so a split holds at most 64 chunks of 16 tokens).
constexpr int kDecodeSplitTokens = 256;
// Keys per decode split with grouped heads (at most 64 groups of 16 keys).
constexpr int kDecodeSplitTokensGrouped = 1024;

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t stream);
// grouped K/V heads (num_q_heads / num_kv_heads >= kGqaMinGroup): same workspace
hipError_t launch_decode_partial_gqa(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream);
// Device address of the current GPU's static decode workspace (PA_NOALLOC_SCRATCH_BYTES
// bytes), looked up on the first call per device and kept.
hipError_t static_decode_workspace(void** ptr);
hipError_t launch_copy_pages(const CopyPagesArgs& a, hipStream_t stream);

}  // namespace pa
