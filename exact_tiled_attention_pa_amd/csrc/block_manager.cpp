// Host-side page manager for the paged KV cache: per-sequence block tables,
// on-demand page allocation, reference counts and copy-on-write prefix sharing.
//
// "FlashAttention and PagedAttention: Two Fixes for Two Different Bottlenecks",
// "How it works" under PagedAttention: the cache is cut into fixed-size blocks
// handed out as a sequence grows, a block table maps each sequence's logical
// blocks to physical ones, and sequences with a common prefix point at the same
// physical blocks, a shared block being copied only when one sharer writes into it.
// "What is Paged FlashAttention?", "Practical example" fixes the mapping
// (logical block = pos / page_size, slot = pos % page_size).
//
// The manager is plain bookkeeping on the host.  It never touches device memory:
// pa_bm_append returns the (source, destination) page pairs that must be copied
// (pa_copy_pages) before the new tokens are written (pa_kv_append), and the caller
// uploads the block table it exports.  Only the page a sequence's next token lands
// in can need a copy: pages wholly before it are full and never written again.

#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "pagedattn.h"
#include "status.h"

struct pa_block_manager {
  int32_t num_pages;
  int32_t page_size;
  int32_t max_seqs;
  int32_t max_pages;
  std::vector<int32_t> table;       // [max_seqs * max_pages]; -1 where unused
  std::vector<int32_t> lens;        // [max_seqs]; -1 marks a free sequence slot
  std::vector<int32_t> refs;        // [num_pages]: table entries naming the page
  std::vector<int32_t> free_pages;  // stack; the back is handed out next
  std::vector<int32_t> free_slots;  // stack of free sequence slots
};

namespace {

using pa::fail;
using pa::ok;

int32_t pages_for(int64_t tokens, int32_t page_size) {
  return (int32_t)((tokens + page_size - 1) / page_size);
}

bool live(const pa_block_manager* bm, int32_t seq) {
  return seq >= 0 && seq < bm->max_seqs && bm->lens[seq] >= 0;
}

int check_live(const pa_block_manager* bm, int32_t seq) {
  if (!bm) return fail(PA_ERR_NULL, "block manager is NULL");
  if (!live(bm, seq))
    return fail(PA_ERR_INVALID_ARG, "sequence %d is not a live sequence of this manager", seq);
  return PA_OK;
}

int32_t* row(pa_block_manager* bm, int32_t seq) {
  return bm->table.data() + (size_t)seq * bm->max_pages;
}

void release_page(pa_block_manager* bm, int32_t page) {
  if (--bm->refs[page] == 0) bm->free_pages.push_back(page);
}

int32_t take_page(pa_block_manager* bm) {
  const int32_t p = bm->free_pages.back();
  bm->free_pages.pop_back();
  bm->refs[p] = 1;
  return p;
}

}  // namespace

extern "C" {

int pa_bm_create(int32_t num_pages, int32_t page_size, int32_t max_seqs,
                 int32_t max_pages_per_seq, pa_block_manager** out) {
  if (!out) return fail(PA_ERR_NULL, "out is NULL");
  *out = nullptr;
  if (num_pages < 1 || page_size < 1 || max_seqs < 1 || max_pages_per_seq < 1)
    return fail(PA_ERR_INVALID_ARG,
                "num_pages=%d page_size=%d max_seqs=%d max_pages_per_seq=%d must be >= 1",
                num_pages, page_size, max_seqs, max_pages_per_seq);
  if ((int64_t)max_pages_per_seq * page_size > ((int64_t)1 << 30))
    return fail(PA_ERR_INVALID_ARG, "max_pages_per_seq * page_size exceeds 2^30 tokens");
  if ((int64_t)max_seqs * max_pages_per_seq > ((int64_t)1 << 31) - 1)
    return fail(PA_ERR_INVALID_ARG, "max_seqs * max_pages_per_seq exceeds 2^31 - 1");
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (!bm) return fail(PA_ERR_CAPACITY, "out of host memory");
  try {
    bm->num_pages = num_pages;
    bm->page_size = page_size;
    bm->max_seqs = max_seqs;
    bm->max_pages = max_pages_per_seq;
    bm->table.assign((size_t)max_seqs * max_pages_per_seq, -1);
    bm->lens.assign(max_seqs, -1);
    bm->refs.assign(num_pages, 0);
    bm->free_pages.resize(num_pages);
    for (int32_t i = 0; i < num_pages; ++i) bm->free_pages[i] = num_pages - 1 - i;
    bm->free_slots.resize(max_seqs);
    for (int32_t i = 0; i < max_seqs; ++i) bm->free_slots[i] = max_seqs - 1 - i;
  } catch (const std::bad_alloc&) {
    delete bm;
    return fail(PA_ERR_CAPACITY, "out of host memory");
  }
  *out = bm;
  return ok();
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_add_sequence(pa_block_manager* bm, int32_t* seq_out) {
  if (!bm || !seq_out) return fail(PA_ERR_NULL, "block manager and seq_out must be non-NULL");
  if (bm->free_slots.empty())
    return fail(PA_ERR_CAPACITY, "all %d sequence slots are in use", bm->max_seqs);
  const int32_t s = bm->free_slots.back();
  bm->free_slots.pop_back();
  bm->lens[s] = 0;
  *seq_out = s;
  return ok();
}

int pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t num_tokens, int32_t* child_out) {
  int st = check_live(bm, parent);
  if (st) return st;
  if (!child_out) return fail(PA_ERR_NULL, "child_out is NULL");
  if (num_tokens < 0 || num_tokens > bm->lens[parent])
    return fail(PA_ERR_INVALID_ARG, "cannot share %d tokens of a %d-token sequence",
                num_tokens, bm->lens[parent]);
  if (bm->free_slots.empty())
    return fail(PA_ERR_CAPACITY, "all %d sequence slots are in use", bm->max_seqs);
  const int32_t c = bm->free_slots.back();
  bm->free_slots.pop_back();
  const int32_t n = pages_for(num_tokens, bm->page_size);
  const int32_t* src = row(bm, parent);
  int32_t* dst = row(bm, c);
  for (int32_t p = 0; p < n; ++p) {
    dst[p] = src[p];
    ++bm->refs[src[p]];
  }
  bm->lens[c] = num_tokens;
  *child_out = c;
  return ok();
}

int pa_bm_free_sequence(pa_block_manager* bm, int32_t seq) {
  int st = check_live(bm, seq);
  if (st) return st;
  int32_t* r = row(bm, seq);
  const int32_t n = pages_for(bm->lens[seq], bm->page_size);
  for (int32_t p = 0; p < n; ++p) {
    release_page(bm, r[p]);
    r[p] = -1;
  }
  bm->lens[seq] = -1;
  bm->free_slots.push_back(seq);
  return ok();
}

int pa_bm_append(pa_block_manager* bm, int32_t seq, int32_t num_tokens, int32_t* copy_src,
                 int32_t* copy_dst, int32_t* num_copies) {
  int st = check_live(bm, seq);
  if (st) return st;
  if (!copy_src || !copy_dst || !num_copies)
    return fail(PA_ERR_NULL, "copy_src, copy_dst and num_copies must be non-NULL");
  *num_copies = 0;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens=%d must be >= 0", num_tokens);
  const int64_t len = bm->lens[seq];
  const int64_t new_len = len + num_tokens;
  if (new_len > (int64_t)bm->max_pages * bm->page_size)
    return fail(PA_ERR_INVALID_ARG, "sequence %d would hold %lld tokens, above the %lld a "
                "table row maps", seq, (long long)new_len,
                (long long)bm->max_pages * bm->page_size);
  if (num_tokens == 0) return ok();
  int32_t* r = row(bm, seq);
  const int32_t have = pages_for(len, bm->page_size);
  const int32_t need = pages_for(new_len, bm->page_size);
  // the next token lands inside a page already in the table: copy it first if shared
  const bool cow = len % bm->page_size != 0 && bm->refs[r[have - 1]] > 1;
  const size_t want = (size_t)(need - have) + (cow ? 1 : 0);
  if (want > bm->free_pages.size())
    return fail(PA_ERR_CAPACITY, "appending %d tokens to sequence %d needs %zu free pages, "
                "%zu left", num_tokens, seq, want, bm->free_pages.size());
  if (cow) {
    const int32_t old = r[have - 1];
    const int32_t fresh = take_page(bm);
    --bm->refs[old];  // still referenced by another sharer, so never freed here
    r[have - 1] = fresh;
    copy_src[0] = old;
    copy_dst[0] = fresh;
    *num_copies = 1;
  }
  for (int32_t p = have; p < need; ++p) r[p] = take_page(bm);
  bm->lens[seq] = (int32_t)new_len;
  return ok();
}

int32_t pa_bm_seq_len(const pa_block_manager* bm, int32_t seq) {
  return bm && live(bm, seq) ? bm->lens[seq] : -1;
}

int32_t pa_bm_free_page_count(const pa_block_manager* bm) {
  return bm ? (int32_t)bm->free_pages.size() : -1;
}

int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t page) {
  return bm && page >= 0 && page < bm->num_pages ? bm->refs[page] : -1;
}

int pa_bm_export(const pa_block_manager* bm, int32_t* block_table, int32_t* seq_lens) {
  if (!bm || !block_table || !seq_lens)
    return fail(PA_ERR_NULL, "block manager, block_table and seq_lens must be non-NULL");
  std::copy(bm->table.begin(), bm->table.end(), block_table);
  for (int32_t s = 0; s < bm->max_seqs; ++s) seq_lens[s] = bm->lens[s] < 0 ? 0 : bm->lens[s];
  return ok();
}

int pa_bm_validate(const pa_block_manager* bm) {
  if (!bm) return fail(PA_ERR_NULL, "block manager is NULL");
  std::vector<int32_t> count(bm->num_pages, 0);
  for (int32_t s = 0; s < bm->max_seqs; ++s) {
    const int32_t* r = bm->table.data() + (size_t)s * bm->max_pages;
    const int32_t n = bm->lens[s] < 0 ? 0 : pages_for(bm->lens[s], bm->page_size);
    for (int32_t p = 0; p < bm->max_pages; ++p) {
      if (p >= n) {
        if (r[p] != -1) return fail(PA_ERR_INVALID_ARG, "seq %d page %d: stale entry", s, p);
        continue;
      }
      if (r[p] < 0 || r[p] >= bm->num_pages)
        return fail(PA_ERR_INVALID_ARG, "seq %d page %d: entry %d out of range", s, p, r[p]);
      ++count[r[p]];
    }
  }
  std::vector<char> is_free(bm->num_pages, 0);
  for (int32_t p : bm->free_pages) {
    if (p < 0 || p >= bm->num_pages || is_free[p])
      return fail(PA_ERR_INVALID_ARG, "free list holds page %d twice or out of range", p);
    is_free[p] = 1;
  }
  for (int32_t p = 0; p < bm->num_pages; ++p) {
    if (count[p] != bm->refs[p])
      return fail(PA_ERR_INVALID_ARG, "page %d: %d references, count says %d", p, count[p],
                  bm->refs[p]);
    if ((count[p] == 0) != (is_free[p] != 0))
      return fail(PA_ERR_INVALID_ARG, "page %d: %d references but %s the free list", p,
                  count[p], is_free[p] ? "on" : "not on");
  }
  int32_t live_slots = 0;
  for (int32_t s = 0; s < bm->max_seqs; ++s) live_slots += bm->lens[s] >= 0;
  if ((size_t)(bm->max_seqs - live_slots) != bm->free_slots.size())
    return fail(PA_ERR_INVALID_ARG, "free sequence slots do not add up");
  return ok();
}

}  // extern "C"
