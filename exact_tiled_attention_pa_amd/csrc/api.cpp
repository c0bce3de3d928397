// C-ABI layer of libpagedattn: argument validation, workspace layout, grid
// sizing and kernel launch.  Never allocates, frees or synchronises; never reads
// device memory.  See include/pagedattn.h for the contract of every entry point.

#include "pagedattn.h"

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kernels.h"
#include "prefill_split.h"
#include "status.h"

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

namespace pa {

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return PA_OK;
}

}  // namespace pa

namespace {

using pa::fail;
using pa::ok;

int log2_exact(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return (1 << r) == x ? r : -1;
}

// Validates the pool layout and the head counts shared by every entry point.
int check_layout(const pa_kv_layout* layout, int32_t num_q_heads) {
  if (!layout) return fail(PA_ERR_NULL, "layout is NULL");
  if (layout->num_pages < 1 || layout->page_size < 1 || layout->num_kv_heads < 1 ||
      layout->head_dim < 1 || layout->max_pages_per_seq < 1)
    return fail(PA_ERR_INVALID_ARG,
                "layout fields must be >= 1 (num_pages=%d page_size=%d num_kv_heads=%d "
                "head_dim=%d max_pages_per_seq=%d)",
                layout->num_pages, layout->page_size, layout->num_kv_heads, layout->head_dim,
                layout->max_pages_per_seq);
  if (num_q_heads < 1 || num_q_heads % layout->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads=%d must be a positive multiple of num_kv_heads=%d",
                num_q_heads, layout->num_kv_heads);
  if (layout->head_dim != 64 && layout->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim=%d: supported values are 64 and 128",
                layout->head_dim);
  const int lg = log2_exact(layout->page_size);
  if (lg < 4 || lg > 8)
    return fail(PA_ERR_UNSUPPORTED, "page_size=%d: must be a power of two in [16, 256]",
                layout->page_size);
  if ((int64_t)layout->max_pages_per_seq * layout->page_size > (int64_t)1 << 30)
    return fail(PA_ERR_INVALID_ARG, "max_pages_per_seq * page_size exceeds 2^30 tokens");
  if ((int64_t)layout->num_pages * layout->page_size > ((int64_t)1 << 31) - 1)
    return fail(PA_ERR_INVALID_ARG, "num_pages * page_size exceeds 2^31 - 1 token rows");
  // a token row of the pools at most 32 MiB: the kernels' in-page byte offsets (16 rows
  // at most) then stay below 2^31
  if ((int64_t)layout->num_kv_heads * layout->head_dim > (int64_t)1 << 24)
    return fail(PA_ERR_INVALID_ARG, "num_kv_heads * head_dim exceeds 2^24");
  return PA_OK;
}

int check_scale(float scale) {
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(PA_ERR_INVALID_ARG, "scale=%g must be finite and >= 0", (double)scale);
  return PA_OK;
}

// Units of pass-1 work below which the decode shortens its splits: the MI355X has 256
// CUs (the one-head-per-row decode runs one persistent workgroup per CU claiming units;
// the grouped-head decode launches one workgroup per unit).
constexpr int64_t kDecodeFillUnits = 256;
// Query heads per workgroup of the grouped-head decode (kHeadBlock in decode_gqa.hip).
constexpr int kGqaHeadBlock = 32;

// Keys per decode split.  Grouped heads walk longer splits (their workgroups read a
// quarter of the bytes per key that one-head-per-row workgroups do, so a longer split
// keeps the per-workgroup set-up and merge small against the streaming): 1024 keys,
// halved (down to 128) while the batch, each sequence as long as the table allows,
// would launch fewer workgroups (split x K/V head x block of 32 query heads) than there
// are CUs.  The one-head-per-row decode takes 256-key splits, halved (to 128, then 64)
// while the batch would give pass 1 fewer units (split x group of the heads one wave
// load covers) than there are CUs.  Either way a small batch still spreads over the
// chip instead of leaving CUs idle.
// Whether `batch` sequences of `tokens` keys in splits of `st` keys, times `width` work
// items per split, make fewer than kDecodeFillUnits units (batch x splits < 2^40, and
// width only multiplies a count already below the limit, so nothing overflows).
bool too_few_units(int32_t batch, int64_t tokens, int st, int64_t width) {
  const int64_t units = (int64_t)batch * ((tokens + st - 1) / st);
  return units < kDecodeFillUnits && units * width < kDecodeFillUnits;
}

int split_tokens_of(const pa_kv_layout* layout, int32_t num_q_heads, int32_t batch) {
  const int64_t tokens = (int64_t)layout->max_pages_per_seq * layout->page_size;
  const int group = num_q_heads / layout->num_kv_heads;
  if (group >= pa::kGqaMinGroup) {
    const int64_t blocks =
        (int64_t)layout->num_kv_heads * ((group + kGqaHeadBlock - 1) / kGqaHeadBlock);
    int st = pa::kDecodeSplitTokensGrouped;
    while (st > pa::kDecodeSplitTokensGrouped / 8 && too_few_units(batch, tokens, st, blocks))
      st /= 2;
    return st;
  }
  const int heads_per_load = 64 / (layout->head_dim / 8);  // 4 at d = 128, 8 at d = 64
  const int64_t groups = (num_q_heads + heads_per_load - 1) / heads_per_load;
  int st = pa::kDecodeSplitTokens;
  while (st > pa::kDecodeSplitTokens / 4 && too_few_units(batch, tokens, st, groups)) st /= 2;
  return st;
}

int max_splits_of(const pa_kv_layout* layout, int32_t num_q_heads, int32_t batch) {
  const int64_t tokens = (int64_t)layout->max_pages_per_seq * layout->page_size;
  const int st = split_tokens_of(layout, num_q_heads, batch);
  return (int)((tokens + st - 1) / st);
}

// Workspace: fp32 O partials first, then (m, l) pairs, each region 256-byte aligned.
size_t ws_o_bytes(int32_t batch, int32_t num_q_heads, const pa_kv_layout* layout) {
  const size_t n =
      (size_t)batch * num_q_heads * max_splits_of(layout, num_q_heads, batch) * layout->head_dim;
  return (n * sizeof(float) + 255) / 256 * 256;
}

size_t ws_ml_bytes(int32_t batch, int32_t num_q_heads, const pa_kv_layout* layout) {
  const size_t n = (size_t)batch * num_q_heads * max_splits_of(layout, num_q_heads, batch) * 2;
  return (n * sizeof(float) + 255) / 256 * 256;
}

// Pass 1's plan of the one-head-per-row decode: a claim counter, the number of
// (sequence, split) pairs and the pairs themselves.
size_t ws_plan_bytes(int32_t batch, int32_t num_q_heads, const pa_kv_layout* layout) {
  const size_t n = 2 + (size_t)batch * max_splits_of(layout, num_q_heads, batch);
  return (n * sizeof(int32_t) + 255) / 256 * 256;
}

size_t ws_bytes(int32_t batch, int32_t num_q_heads, const pa_kv_layout* layout) {
  return ws_o_bytes(batch, num_q_heads, layout) + ws_ml_bytes(batch, num_q_heads, layout) +
         ws_plan_bytes(batch, num_q_heads, layout);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_decode_common(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
                        const int32_t* block_table, const int32_t* seq_lens, float scale,
                        int32_t batch, int32_t num_q_heads, const void* workspace,
                        size_t workspace_bytes, const pa_kv_layout* layout, bool need_inputs,
                        bool check_workspace = true) {
  int st = check_layout(layout, num_q_heads);
  if (st) return st;
  if (batch < 0) return fail(PA_ERR_INVALID_ARG, "batch=%d must be >= 0", batch);
  if (batch > 65535) return fail(PA_ERR_INVALID_ARG, "batch=%d exceeds 65535", batch);
  if (need_inputs) {
    if (!q || !k_pool || !v_pool || !block_table)
      return fail(PA_ERR_NULL, "q, k_pool, v_pool and block_table must be non-NULL");
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
      return fail(PA_ERR_INVALID_ARG, "q, k_pool and v_pool must be 16-byte aligned");
    st = check_scale(scale);
    if (st) return st;
  }
  if (!seq_lens) return fail(PA_ERR_NULL, "seq_lens must be non-NULL");
  if (max_splits_of(layout, num_q_heads, batch) > 65535)
    return fail(PA_ERR_INVALID_ARG, "max_pages_per_seq * page_size = %lld needs more than 65535 "
                "decode splits", (long long)layout->max_pages_per_seq * layout->page_size);
  // pass 1 numbers its units of work (split x head group) with 32-bit integers
  if ((int64_t)batch * max_splits_of(layout, num_q_heads, batch) * num_q_heads >=
      ((int64_t)1 << 31))
    return fail(PA_ERR_INVALID_ARG, "%d sequences x %d splits x %d query heads exceed 2^31 "
                "decode work units", batch, max_splits_of(layout, num_q_heads, batch),
                num_q_heads);
  if (!check_workspace) return PA_OK;
  const size_t need = ws_bytes(batch, num_q_heads, layout);
  if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (!aligned16(workspace))
    return fail(PA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes is too small (need %zu)",
                workspace_bytes, need);
  return PA_OK;
}

pa::DecodeArgs decode_args(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
                           const int32_t* block_table, const int32_t* seq_lens, float scale,
                           pa_bf16* out, int32_t batch, int32_t num_q_heads,
                           const void* workspace, const pa_kv_layout* layout,
                           int32_t window = 0) {
  pa::DecodeArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  char* ws = static_cast<char*>(const_cast<void*>(workspace));
  a.ws_o = reinterpret_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float*>(ws + ws_o_bytes(batch, num_q_heads, layout));
  a.plan = reinterpret_cast<int32_t*>(ws + ws_o_bytes(batch, num_q_heads, layout) +
                                      ws_ml_bytes(batch, num_q_heads, layout));
  a.scale = scale;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = layout->num_kv_heads;
  a.head_dim = layout->head_dim;
  a.log2_page_size = log2_exact(layout->page_size);
  a.max_pages_per_seq = layout->max_pages_per_seq;
  a.split_tokens = split_tokens_of(layout, num_q_heads, batch);
  a.max_splits = max_splits_of(layout, num_q_heads, batch);
  a.window = window;
  return a;
}

// PA_PREFILL_PATH: unset, empty or "auto" lets the launch size choose the prefill
// kernel; "tiles" or "split" forces one (tests run both at every shape).  -1: unknown.
int prefill_path_from_env() {
  const char* s = std::getenv("PA_PREFILL_PATH");
  if (!s || !*s || !std::strcmp(s, "auto")) return pa::kPrefillPathAuto;
  if (!std::strcmp(s, "tiles")) return pa::kPrefillPathTiles;
  if (!std::strcmp(s, "split")) return pa::kPrefillPathSplit;
  return -1;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(PA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return ok();
}

}  // namespace

extern "C" {

int pa_prefill_window(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, int causal,
                      float scale, pa_bf16* out, const int32_t* q_start, int32_t batch,
                      int32_t num_q_heads, int32_t max_q_len, int32_t window,
                      const pa_kv_layout* layout, hipStream_t stream) {
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "window=%d must be >= 0", window);
  if (window > 0 && !causal)
    return fail(PA_ERR_INVALID_ARG, "a sliding window (window=%d) needs causal attention",
                window);
  int st = check_layout(layout, num_q_heads);
  if (st) return st;
  if (batch < 0) return fail(PA_ERR_INVALID_ARG, "batch=%d must be >= 0", batch);
  if (batch > 65535) return fail(PA_ERR_INVALID_ARG, "batch=%d exceeds 65535", batch);
  if (max_q_len < 0) return fail(PA_ERR_INVALID_ARG, "max_q_len=%d must be >= 0", max_q_len);
  if ((int64_t)max_q_len > (int64_t)layout->max_pages_per_seq * layout->page_size)
    return fail(PA_ERR_INVALID_ARG,
                "max_q_len=%d exceeds the table's capacity of %lld tokens per sequence",
                max_q_len, (long long)layout->max_pages_per_seq * layout->page_size);
  if (num_q_heads > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads=%d exceeds 65535", num_q_heads);
  if ((max_q_len + pa::kPrefillBlockM - 1) / pa::kPrefillBlockM > 65535)
    return fail(PA_ERR_INVALID_ARG, "max_q_len=%d needs more than 65535 query tiles", max_q_len);
  st = check_scale(scale);
  if (st) return st;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !out || !q_start)
    return fail(PA_ERR_NULL, "every array argument of pa_prefill must be non-NULL");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return fail(PA_ERR_INVALID_ARG, "q, k_pool, v_pool and out must be 16-byte aligned");
  const int path = prefill_path_from_env();
  if (path < 0)
    return fail(PA_ERR_INVALID_ARG, "PA_PREFILL_PATH=%s: expected auto, tiles or split",
                std::getenv("PA_PREFILL_PATH"));
  if (batch == 0 || max_q_len == 0) return ok();

  pa::PrefillArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.q_start = q_start;
  a.out = out;
  a.scale = scale;
  a.causal = causal != 0;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = layout->num_kv_heads;
  a.head_dim = layout->head_dim;
  a.log2_page_size = log2_exact(layout->page_size);
  a.max_pages_per_seq = layout->max_pages_per_seq;
  a.max_q_len = max_q_len;
  a.window = window;
  if (pa::prefill_takes_split(a, path)) {
    if ((max_q_len + pa::kPrefillSplitBlockM - 1) / pa::kPrefillSplitBlockM > 65535)
      return fail(PA_ERR_INVALID_ARG,
                  "max_q_len=%d needs more than 65535 split-key query tiles", max_q_len);
    return hip_status(pa::launch_prefill_split(a, stream), "split-key prefill launch");
  }
  return hip_status(pa::launch_prefill(a, stream), "prefill launch");
}

int pa_prefill(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
               const int32_t* block_table, const int32_t* seq_lens, int causal, float scale,
               pa_bf16* out, const int32_t* q_start, int32_t batch, int32_t num_q_heads,
               int32_t max_q_len, const pa_kv_layout* layout, hipStream_t stream) {
  return pa_prefill_window(q, k_pool, v_pool, block_table, seq_lens, causal, scale, out,
                           q_start, batch, num_q_heads, max_q_len, 0, layout, stream);
}

size_t pa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                 const pa_kv_layout* layout) {
  if (check_layout(layout, num_q_heads) != PA_OK || batch < 0) return 0;
  return ws_bytes(batch, num_q_heads, layout);
}

int32_t pa_decode_split_tokens(int32_t batch, int32_t num_q_heads, const pa_kv_layout* layout) {
  if (check_layout(layout, num_q_heads) != PA_OK || batch < 0) return 0;
  return split_tokens_of(layout, num_q_heads, batch);
}

int pa_decode_partial(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, float scale,
                      int32_t batch, int32_t num_q_heads, void* workspace,
                      size_t workspace_bytes, const pa_kv_layout* layout, hipStream_t stream) {
  int st = check_decode_common(q, k_pool, v_pool, block_table, seq_lens, scale, batch,
                               num_q_heads, workspace, workspace_bytes, layout, true);
  if (st) return st;
  if (batch == 0) return ok();
  const pa::DecodeArgs a = decode_args(q, k_pool, v_pool, block_table, seq_lens, scale,
                                       nullptr, batch, num_q_heads, workspace, layout);
  return hip_status(pa::launch_decode_partial(a, stream), "decode partial launch");
}

int pa_decode_combine(const int32_t* seq_lens, pa_bf16* out, int32_t batch,
                      int32_t num_q_heads, const void* workspace, size_t workspace_bytes,
                      const pa_kv_layout* layout, hipStream_t stream) {
  int st = check_decode_common(nullptr, nullptr, nullptr, nullptr, seq_lens, 1.f, batch,
                               num_q_heads, workspace, workspace_bytes, layout, false);
  if (st) return st;
  if (!out) return fail(PA_ERR_NULL, "out must be non-NULL");
  if (batch == 0) return ok();
  const pa::DecodeArgs a = decode_args(nullptr, nullptr, nullptr, nullptr, seq_lens, 1.f, out,
                                       batch, num_q_heads, workspace, layout);
  return hip_status(pa::launch_decode_combine(a, stream), "decode combine launch");
}

int pa_decode_window(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
                     const int32_t* block_table, const int32_t* seq_lens, float scale,
                     pa_bf16* out, int32_t batch, int32_t num_q_heads, int32_t window,
                     void* workspace, size_t workspace_bytes, const pa_kv_layout* layout,
                     hipStream_t stream) {
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "window=%d must be >= 0", window);
  int st = check_decode_common(q, k_pool, v_pool, block_table, seq_lens, scale, batch,
                               num_q_heads, workspace, workspace_bytes, layout, true);
  if (st) return st;
  if (!out) return fail(PA_ERR_NULL, "out must be non-NULL");
  if (batch == 0) return ok();
  const pa::DecodeArgs a = decode_args(q, k_pool, v_pool, block_table, seq_lens, scale, out,
                                       batch, num_q_heads, workspace, layout, window);
  st = hip_status(pa::launch_decode_partial(a, stream), "decode partial launch");
  if (st) return st;
  return hip_status(pa::launch_decode_combine(a, stream), "decode combine launch");
}

int pa_decode(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
              const int32_t* block_table, const int32_t* seq_lens, float scale, pa_bf16* out,
              int32_t batch, int32_t num_q_heads, void* workspace, size_t workspace_bytes,
              const pa_kv_layout* layout, hipStream_t stream) {
  return pa_decode_window(q, k_pool, v_pool, block_table, seq_lens, scale, out, batch,
                          num_q_heads, 0, workspace, workspace_bytes, layout, stream);
}

int pa_decode_noalloc(const pa_bf16* q, const pa_bf16* k_pool, const pa_bf16* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, float scale,
                      pa_bf16* out, int32_t batch, int32_t num_q_heads,
                      const pa_kv_layout* layout, hipStream_t stream) {
  // every argument is checked before any HIP call, so a refused call touches no device
  int st = check_decode_common(q, k_pool, v_pool, block_table, seq_lens, scale, batch,
                               num_q_heads, nullptr, 0, layout, true, false);
  if (st) return st;
  if (!out) return fail(PA_ERR_NULL, "out must be non-NULL");
  const size_t need = ws_bytes(batch, num_q_heads, layout);
  if (need > PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ERR_WORKSPACE,
                "pa_decode_noalloc: %d sequences x %d query heads over up to %lld tokens need "
                "%zu bytes of partials, above the library's static %zu-byte workspace; use "
                "pa_decode with a caller workspace",
                batch, num_q_heads, (long long)layout->max_pages_per_seq * layout->page_size,
                need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
  if (batch == 0) return ok();
  void* scratch = nullptr;
  st = hip_status(pa::static_decode_workspace(&scratch), "static decode workspace lookup");
  if (st) return st;
  return pa_decode_window(q, k_pool, v_pool, block_table, seq_lens, scale, out, batch,
                          num_q_heads, 0, scratch, PA_NOALLOC_SCRATCH_BYTES, layout, stream);
}

int pa_kv_append(const pa_bf16* k_new, const pa_bf16* v_new, const int32_t* seq_ids,
                 const int32_t* positions, int32_t num_tokens, pa_bf16* k_pool,
                 pa_bf16* v_pool, const int32_t* block_table, int32_t num_seqs,
                 const pa_kv_layout* layout, hipStream_t stream) {
  if (!layout) return fail(PA_ERR_NULL, "layout is NULL");
  int st = check_layout(layout, layout->num_kv_heads);
  if (st) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens=%d must be >= 0", num_tokens);
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs=%d must be >= 0", num_seqs);
  if (!k_new || !v_new || !seq_ids || !positions || !k_pool || !v_pool || !block_table)
    return fail(PA_ERR_NULL, "every array argument of pa_kv_append must be non-NULL");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PA_ERR_INVALID_ARG, "k_new, v_new, k_pool and v_pool must be 16-byte aligned");
  if (num_tokens == 0 || num_seqs == 0) return ok();
  pa::KvAppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.seq_ids = seq_ids;
  a.positions = positions;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.num_tokens = num_tokens;
  a.num_seqs = num_seqs;
  a.num_pages = layout->num_pages;
  a.log2_page_size = log2_exact(layout->page_size);
  a.max_pages_per_seq = layout->max_pages_per_seq;
  a.row_elems = layout->num_kv_heads * layout->head_dim;
  return hip_status(pa::launch_kv_append(a, stream), "kv append launch");
}

int pa_copy_pages(pa_bf16* k_pool, pa_bf16* v_pool, const int32_t* src_pages,
                  const int32_t* dst_pages, int32_t num_copies, const pa_kv_layout* layout,
                  hipStream_t stream) {
  if (!layout) return fail(PA_ERR_NULL, "layout is NULL");
  int st = check_layout(layout, layout->num_kv_heads);
  if (st) return st;
  if (num_copies < 0) return fail(PA_ERR_INVALID_ARG, "num_copies=%d must be >= 0", num_copies);
  const size_t page_bytes = (size_t)layout->page_size * layout->num_kv_heads *
                            layout->head_dim * sizeof(pa_bf16);
  if (page_bytes > ((size_t)1 << 28))
    return fail(PA_ERR_INVALID_ARG, "a page of %zu bytes exceeds 256 MiB", page_bytes);
  if (!k_pool || !v_pool || !src_pages || !dst_pages)
    return fail(PA_ERR_NULL, "every array argument of pa_copy_pages must be non-NULL");
  if (!aligned16(k_pool) || !aligned16(v_pool))
    return fail(PA_ERR_INVALID_ARG, "k_pool and v_pool must be 16-byte aligned");
  if (num_copies == 0) return ok();
  pa::CopyPagesArgs a;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.src_pages = src_pages;
  a.dst_pages = dst_pages;
  a.num_copies = num_copies;
  a.num_pages = layout->num_pages;
  a.page_bytes = page_bytes;
  return hip_status(pa::launch_copy_pages(a, stream), "copy pages launch");
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: a size or scalar is out of range";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: head_dim or page_size not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: decode workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: the HIP runtime reported an error";
    case PA_ERR_CAPACITY: return "PA_ERR_CAPACITY: no free page or sequence slot left";
    default: return "unknown pa_status";
  }
}

const char* pa_last_error(void) { return g_last_error; }

const char* pa_version(void) { return "0.1.0"; }

}  // extern "C"
