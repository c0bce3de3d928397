/*
 * libpagedattn: exact attention over a paged KV cache on AMD Instinct MI355X (gfx950).
 *
 * Computes O = softmax(scale * Q K^T) V exactly (up to floating-point rounding)
 * in the FlashAttention manner: K/V tiles are staged on chip, a running row
 * max and row sum implement an online softmax, and the score / probability
 * matrices are never written to device memory.  K and V are read in place from
 * a paged pool through a per-sequence block table.
 *
 * Sources, cited by page title and section:
 *   [FA-PA]  "FlashAttention and PagedAttention: Two Fixes for Two Different
 *            Bottlenecks": "Why attention is costly" (the formula), "How it works"
 *            under FlashAttention (tiling, online softmax, fusion) and under
 *            PagedAttention (fixed-size blocks, block table, a kernel that reads
 *            the scattered blocks), "In code" (causal flag, token-major layout).
 *   [PFA]    "What is Paged FlashAttention?": "How does it work?" (locate pages,
 *            load K/V tiles, online softmax, accumulate) and "Practical example"
 *            (logical = pos / page_size, offset = pos % page_size,
 *            physical = block_table[logical]).
 *   [FA-LLM] "Flash Attention: Fast, Memory-Efficient Attention for LLMs":
 *            "The Algorithm" (running max / sum, per-tile rescale, final division),
 *            "Flash Attention 2" (causal tile skipping), "KV Cache" (decode appends
 *            the new token, then attends over the cache), "Attention Variants"
 *            (grouped K/V heads).
 *
 * Conventions for every entry point
 *   - bf16 values are passed as raw 16-bit patterns (pa_bf16).  Arithmetic is
 *     fp32 (MFMA accumulation, fp32 softmax state); outputs are rounded to
 *     bf16 round-to-nearest-even.
 *   - All array arguments are device pointers owned by the caller (the block
 *     manager's pa_bm_* calls are the exception: host memory only).  The library
 *     never allocates device memory, frees or synchronises; work is enqueued
 *     asynchronously on the given HIP stream (0 = the null stream).
 *   - Layouts are row-major:
 *       q, out          [tokens, num_q_heads, head_dim]
 *       k_pool, v_pool  [num_pages, page_size, num_kv_heads, head_dim]
 *       block_table     int32 [batch, max_pages_per_seq]
 *   - Return value: PA_OK or an error status.  On error nothing is enqueued
 *     and pa_last_error() describes the cause (thread-local).  No call aborts
 *     or throws.
 *   - Device-array contract (not checked on the host, which never reads device
 *     memory): for sequence b with KV length L_b,
 *       0 <= block_table[b, p] < num_pages for p < ceil(L_b / page_size);
 *       table entries past that are never read (any value, e.g. -1);
 *       L_b <= max_pages_per_seq * page_size.
 *     Pool slots past L_b (the tail of the last page) and unused pages may hold
 *     anything, NaN included: they never influence the output.
 *   - Aliased physical pages (several sequences listing the same page, as with
 *     shared prefixes) are allowed: pools are only read.  out must not overlap
 *     any input.
 *   - Thread-safe: no global mutable state other than the thread-local error text
 *     (a block manager object is the caller's state and must not be shared between
 *     threads without a lock).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t pa_bf16; /* raw bf16 bits */

enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,          /* a required pointer is NULL */
  PA_ERR_INVALID_ARG = 2,   /* a size or scalar is out of range */
  PA_ERR_UNSUPPORTED = 3,   /* valid but not implemented (head_dim, page_size) */
  PA_ERR_WORKSPACE = 4,     /* decode workspace missing or too small */
  PA_ERR_HIP = 5,           /* the HIP runtime reported an error at launch */
  PA_ERR_CAPACITY = 6       /* block manager: no free page or sequence slot left */
};

/* Shape of the paged KV pools.  Shared by K and V. */
typedef struct pa_kv_layout {
  int32_t num_pages;          /* physical pages in each pool, >= 1;
                                 num_pages * page_size < 2^31 */
  int32_t page_size;          /* tokens per page: a power of two in [16, 256] */
  int32_t num_kv_heads;       /* heads stored per token in the pools, >= 1;
                                 num_kv_heads * head_dim <= 2^24 */
  int32_t head_dim;           /* 64 or 128 */
  int32_t max_pages_per_seq;  /* row length (int32 elements) of block_table, >= 1 */
} pa_kv_layout;

/*
 * pa_prefill -- attention of a chunk of query rows per sequence over that
 * sequence's paged keys and values ([FA-LLM] "The Algorithm"; [PFA] "How does it
 * work?").  Also serves chunked prefill on top of an existing cache.
 *
 *   q            [q_start[batch], num_q_heads, head_dim] bf16; rows of sequence b
 *                are q_start[b] .. q_start[b+1]-1
 *   k_pool, v_pool  pools described by layout
 *   block_table  int32 [batch, layout->max_pages_per_seq]
 *   seq_lens     int32 [batch]: L_b, KV length of sequence b including this chunk
 *   causal       nonzero: query row i of a chunk of q_len_b rows sits at absolute
 *                position L_b - q_len_b + i and sees keys 0..that position
 *                (bottom-right alignment); zero: every row sees keys 0..L_b-1
 *   scale        multiplies Q K^T; finite and >= 0 (1/sqrt(head_dim) in the usual case)
 *   out          [q_start[batch], num_q_heads, head_dim] bf16
 *   q_start      int32 [batch + 1], non-decreasing, q_start[0] = 0; each
 *                q_len_b = q_start[b+1] - q_start[b] must satisfy q_len_b <= L_b
 *   batch        number of sequences, >= 0 (0: nothing to do)
 *   num_q_heads  multiple of layout->num_kv_heads; query head h reads KV head
 *                h / (num_q_heads / num_kv_heads)
 *   max_q_len    host-side upper bound of every q_len_b (sizes the grid without
 *                reading device memory); rows past q_len_b are never written
 * q, k_pool, v_pool and out must be 16-byte aligned (the kernels move 16-byte pieces).
 * Two kernels compute the same attention: a tiled one (128 query rows per workgroup,
 * their key tiles walked in order) and a split-key one for launches too small to fill
 * the chip (32 query rows per workgroup whose waves, 8 at head_dim 64 and 5 at 128,
 * divide the key tiles and merge their softmax states).  The split-key kernel runs when
 * num_q_heads * batch * ceil(max_q_len / 32) <= 512 and max_pages_per_seq * page_size
 * > 64; the environment variable PA_PREFILL_PATH, read at each call, forces one
 * ("tiles" or "split"; unset, empty or "auto": the rule above).  The two round
 * differently, each within the same tolerance of the exact result.
 * Errors: PA_ERR_NULL, PA_ERR_INVALID_ARG (sizes, scale, max_q_len above
 * max_pages_per_seq * page_size, misaligned arrays, an unknown PA_PREFILL_PATH, a
 * forced split-key launch needing more than 65535 query tiles of 32), PA_ERR_UNSUPPORTED,
 * PA_ERR_HIP.
 */
int pa_prefill(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
               const int32_t* block_table, const int32_t* seq_lens, int causal,
               float scale, pa_bf16* out, const int32_t* q_start, int32_t batch,
               int32_t num_q_heads, int32_t max_q_len, const pa_kv_layout* layout,
               hipStream_t stream);

/*
 * Bytes of device workspace pa_decode needs for `batch` sequences: per
 * (sequence, query head, split) one partial (m, l, O[head_dim]) in fp32, plus
 * the first pass's work list (a counter, a count and one 32-bit entry per
 * (sequence, split)).  Returns 0 for invalid arguments.
 */
size_t pa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                 const pa_kv_layout* layout);

/* Key positions covered by one decode split of a batch of `batch` sequences, with
 * T = max_pages_per_seq * page_size and g = num_q_heads / num_kv_heads:
 *   g >= 4: 1024, halved down to 128 while
 *           batch * ceil(T / split) * num_kv_heads * ceil(g / 32) < 256;
 *   g < 4:  256, halved to 128 and then 64 while
 *           batch * ceil(T / split) * ceil(num_q_heads / h) < 256
 *           (h = 4 heads at head_dim 128, 8 at 64: the heads one 1 KB wave load covers),
 * so that a small batch still gives each of the chip's 256 CUs work.  0 for an invalid
 * layout, head count or batch. */
int32_t pa_decode_split_tokens(int32_t batch, int32_t num_q_heads, const pa_kv_layout* layout);

/*
 * pa_decode -- one new query token per sequence attending over all L_b cached
 * tokens of its sequence, the new token included ([FA-LLM] "KV Cache": the new
 * K_t, V_t are appended before attending).  Memory-bound: each sequence's pages
 * are split into ranges handled by separate workgroups, whose partial
 * (row max, row sum, unnormalised output) triples are merged by a second pass
 * with the same rescaling algebra as the online softmax ([FA-LLM] "The Algorithm").
 *
 *   q         [batch, num_q_heads, head_dim] bf16
 *   seq_lens  int32 [batch], each L_b >= 1 (a sequence with L_b = 0 gets zeros)
 *   scale     finite and >= 0
 *   out       [batch, num_q_heads, head_dim] bf16
 *   workspace device buffer of at least pa_decode_workspace_bytes(...) bytes,
 *             16-byte aligned, any contents; calls that share a workspace must be
 *             ordered on one stream
 * q, k_pool and v_pool must be 16-byte aligned (the kernels move 16-byte pieces).
 * Errors: PA_ERR_NULL, PA_ERR_INVALID_ARG (sizes, scale, misaligned arrays),
 * PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE (missing, too small or misaligned), PA_ERR_HIP.
 */
int pa_decode(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
              const int32_t* block_table, const int32_t* seq_lens, float scale,
              pa_bf16* out, int32_t batch, int32_t num_q_heads, void* workspace,
              size_t workspace_bytes, const pa_kv_layout* layout, hipStream_t stream);

/*
 * The two passes of pa_decode as separate calls, for callers that interleave
 * other work between them or time them separately.  pa_decode(...) is exactly
 * pa_decode_partial(...) followed by pa_decode_combine(...) on the same stream
 * with the same arguments.
 */
int pa_decode_partial(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, float scale,
                      int32_t batch, int32_t num_q_heads, void* workspace,
                      size_t workspace_bytes, const pa_kv_layout* layout,
                      hipStream_t stream);
int pa_decode_combine(const int32_t* seq_lens, pa_bf16* out, int32_t batch,
                      int32_t num_q_heads, const void* workspace, size_t workspace_bytes,
                      const pa_kv_layout* layout, hipStream_t stream);

/*
 * Sliding-window variants ("What do FlashAttention and PagedAttention actually
 * optimize?", section "Sort techniques into the two bins": attention over only the
 * previous w tokens).  window = w >= 1: a query at absolute position p sees only
 * keys p - w + 1 .. p (its own key included); window = 0: no window, identical to
 * pa_prefill / pa_decode.  Key tiles (prefill) and splits (decode) wholly outside
 * the window are skipped, so the work is O(rows * w).  pa_prefill_window needs
 * causal != 0 (PA_ERR_INVALID_ARG otherwise); decode's query sits at L_b - 1.
 * Other arguments, layouts and errors as for pa_prefill / pa_decode.
 */
int pa_prefill_window(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, int causal,
                      float scale, pa_bf16* out, const int32_t* q_start, int32_t batch,
                      int32_t num_q_heads, int32_t max_q_len, int32_t window,
                      const pa_kv_layout* layout, hipStream_t stream);
int pa_decode_window(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
                     const int32_t* block_table, const int32_t* seq_lens, float scale,
                     pa_bf16* out, int32_t batch, int32_t num_q_heads, int32_t window,
                     void* workspace, size_t workspace_bytes, const pa_kv_layout* layout,
                     hipStream_t stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same result, bit for bit, with the split
 * partials kept in a workspace that lives inside the library itself, a static
 * device array of PA_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held from the first
 * call on that GPU until the process ends.  The call allocates nothing, frees
 * nothing and synchronises nothing; its first call on a device looks the array's
 * address up once (hipGetSymbolAddress) with that device current.
 *
 *   arguments  as for pa_decode, without the workspace; the stream must belong
 *              to the current device
 *   limit      pa_decode_workspace_bytes(batch, num_q_heads, layout) must not
 *              exceed PA_NOALLOC_SCRATCH_BYTES (64 MiB: e.g. 64 sequences x 32
 *              heads x 8192 tokens, d = 128); larger requests fail with
 *              PA_ERR_WORKSPACE and enqueue nothing (use pa_decode)
 *   sharing    every call on a GPU uses that GPU's one array: calls whose work
 *              overlaps on one GPU (other streams, other threads) race and give
 *              undefined results; calls ordered on one stream are safe.  The
 *              array keeps the last call's partials; nothing in it needs to start
 *              at zero (each call writes every partial it later reads).
 * Errors: those of pa_decode; PA_ERR_WORKSPACE (request above the limit);
 * PA_ERR_HIP (no current device, or the array's address lookup failed).
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int pa_decode_noalloc(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, float scale,
                      pa_bf16* out, int32_t batch, int32_t num_q_heads,
                      const pa_kv_layout* layout, hipStream_t stream);

/*
 * pa_kv_append -- write the K and V rows of new tokens into their pages, the step
 * before attention in autoregressive decoding ([FA-LLM] "KV Cache": the new K_t,
 * V_t join the cache, then the token attends over it).  Token i of sequence
 * seq_ids[i] at absolute position positions[i] goes to physical page
 * block_table[seq, pos / page_size], slot pos % page_size ([PFA] "Practical
 * example"); every KV head of the token is written.
 *
 *   k_new, v_new  [num_tokens, num_kv_heads, head_dim] bf16 (device)
 *   seq_ids       int32 [num_tokens] (device): row of block_table
 *   positions     int32 [num_tokens] (device): absolute token position
 *   k_pool, v_pool  pools described by layout; written in place
 *   block_table   int32 [num_seqs, layout->max_pages_per_seq] (device)
 *   num_tokens, num_seqs  >= 0 (0: nothing to do)
 * A token whose seq id is outside [0, num_seqs), whose position is negative or
 * at least max_pages_per_seq * page_size, or whose table entry is outside
 * [0, num_pages) is skipped (its slot is not written), so a bad index never
 * writes outside the pools.  Two tokens that map to the same slot race: which one
 * lands is unspecified.  Pages read by other work on the stream must not be
 * written concurrently (order the calls on one stream).  The layout's
 * max_pages_per_seq is block_table's row length; num_q_heads plays no part.
 * k_new, v_new and the pools must be 16-byte aligned (rows move in 16-byte pieces).
 * Errors: PA_ERR_NULL, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP.
 */
int pa_kv_append(const pa_bf16* k_new, const pa_bf16* v_new, const int32_t* seq_ids,
                 const int32_t* positions, int32_t num_tokens, pa_bf16* k_pool,
                 pa_bf16* v_pool, const int32_t* block_table, int32_t num_seqs,
                 const pa_kv_layout* layout, hipStream_t stream);

/*
 * pa_copy_pages -- copy whole pages of both pools, page src_pages[i] to page
 * dst_pages[i]: the copy step of copy-on-write prefix sharing ([FA-PA] "How it
 * works" under PagedAttention: sequences with a common prefix map it to the same
 * physical blocks, and a shared block is copied before one of them writes into
 * it).  Every slot of the page is copied, K and V.
 *
 *   src_pages, dst_pages  int32 [num_copies] (device)
 *   num_copies            >= 0 (0: nothing to do)
 * Pairs with an index outside [0, num_pages), or with src == dst, are skipped.
 * No destination may appear twice or also appear as a source (the copies run
 * concurrently).  The pools must be 16-byte aligned.  Errors: PA_ERR_NULL,
 * PA_ERR_INVALID_ARG (page above 256 MiB, misaligned pool), PA_ERR_UNSUPPORTED,
 * PA_ERR_HIP.
 */
int pa_copy_pages(pa_bf16* k_pool, pa_bf16* v_pool, const int32_t* src_pages,
                  const int32_t* dst_pages, int32_t num_copies, const pa_kv_layout* layout,
                  hipStream_t stream);

/*
 * Block manager: host-side bookkeeping of a paged pool shared by many sequences
 * ([FA-PA] "How it works" under PagedAttention: fixed-size blocks handed out on
 * demand, a block table per sequence, physical blocks shared between sequences with
 * a common prefix and copied when one of them writes into a shared block; [PFA]
 * "Practical example" for the mapping).  It allocates pages only as tokens arrive,
 * counts the table entries naming each page, returns a page to the free list when
 * its count drops to zero, and reports the page copies copy-on-write needs.
 *
 * Unlike the rest of this header these calls take and fill HOST memory and touch
 * no device memory.  A manager is not thread-safe: serialise calls on one manager.
 * Sequences are identified by their row in the exported block table
 * (0 .. max_seqs - 1).  A failing call changes nothing.
 *
 * Typical step for a sequence s that grows by n tokens:
 *   len = pa_bm_seq_len(bm, s);
 *   pa_bm_append(bm, s, n, src, dst, &nc);       -- reserve pages, un-share
 *   pa_copy_pages(k_pool, v_pool, src, dst, nc)  -- (src/dst uploaded to device)
 *   pa_bm_export(bm, table, lens)                -- upload the table
 *   pa_kv_append(..., positions len .. len+n-1)  -- write the new rows
 *   pa_decode / pa_prefill over the exported table and lengths
 */
typedef struct pa_block_manager pa_block_manager;

/* Creates a manager of num_pages pages of page_size tokens for up to max_seqs
 * sequences of up to max_pages_per_seq pages each; every page starts free.
 * *out receives the manager (NULL on error).  Errors: PA_ERR_NULL,
 * PA_ERR_INVALID_ARG (sizes < 1, or a table row mapping above 2^30 tokens),
 * PA_ERR_CAPACITY (host memory). */
int pa_bm_create(int32_t num_pages, int32_t page_size, int32_t max_seqs,
                 int32_t max_pages_per_seq, pa_block_manager** out);

/* Frees the manager (NULL is ignored). */
void pa_bm_destroy(pa_block_manager* bm);

/* Starts an empty sequence; *seq_out receives its table row.  Errors: PA_ERR_NULL,
 * PA_ERR_CAPACITY (every row in use). */
int pa_bm_add_sequence(pa_block_manager* bm, int32_t* seq_out);

/* Starts a sequence whose first num_tokens tokens are those of parent
 * (0 <= num_tokens <= parent's length): it shares the parent's first
 * ceil(num_tokens / page_size) pages, whose counts go up by one; no page is copied
 * now.  *child_out receives its row.  Errors: PA_ERR_NULL, PA_ERR_INVALID_ARG (parent
 * not live, num_tokens out of range), PA_ERR_CAPACITY. */
int pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t num_tokens,
               int32_t* child_out);

/* Ends a sequence: its table row is cleared and each of its pages loses one
 * reference (pages reaching zero become free).  Errors: PA_ERR_NULL,
 * PA_ERR_INVALID_ARG (not live). */
int pa_bm_free_sequence(pa_block_manager* bm, int32_t seq);

/* Grows seq by num_tokens >= 0 tokens, which will sit at positions len .. len+n-1.
 * Allocates the pages those positions need.  If position len falls inside a page
 * shared with another sequence, that page is replaced in seq's row by a fresh page
 * and the pair (old, fresh) is written to copy_src[0], copy_dst[0] with
 * *num_copies = 1 (else 0): the caller must copy it (pa_copy_pages) before writing
 * the new tokens.  copy_src and copy_dst need room for one entry.  All or nothing:
 * with too few free pages nothing changes.  Errors: PA_ERR_NULL, PA_ERR_INVALID_ARG
 * (not live, num_tokens < 0, length above max_pages_per_seq * page_size),
 * PA_ERR_CAPACITY. */
int pa_bm_append(pa_block_manager* bm, int32_t seq, int32_t num_tokens, int32_t* copy_src,
                 int32_t* copy_dst, int32_t* num_copies);

/* Length of a live sequence, -1 otherwise (or for a NULL manager). */
int32_t pa_bm_seq_len(const pa_block_manager* bm, int32_t seq);

/* Number of free pages (-1 for a NULL manager). */
int32_t pa_bm_free_page_count(const pa_block_manager* bm);

/* Table entries naming page (0 if free), -1 if page is out of range. */
int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t page);

/* Copies the block table to block_table (host int32 [max_seqs, max_pages_per_seq],
 * -1 where no page is mapped) and the lengths to seq_lens (host int32 [max_seqs],
 * 0 for unused rows): the arrays pa_kv_append, pa_prefill and pa_decode take.
 * Errors: PA_ERR_NULL. */
int pa_bm_export(const pa_block_manager* bm, int32_t* block_table, int32_t* seq_lens);

/* Checks the manager's invariants (every mapped entry in range, reference counts
 * equal to the table entries naming each page, free list = pages with no
 * reference, no stale entries past a sequence's pages).  PA_OK or
 * PA_ERR_INVALID_ARG with the first violation in pa_last_error(). */
int pa_bm_validate(const pa_block_manager* bm);

/* Static text for a status code. */
const char* pa_status_string(int status);

/* Detail of the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

/* Library version as "major.minor.patch". */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
