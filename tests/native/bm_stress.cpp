// Host-only stress test of the block manager (pa_bm_*), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_block_manager_sanitized.py.  Random
// operations are mirrored by a plain model of the page mapping (which logical pages
// each sequence owns and how many table entries name each physical page); after every
// call the manager's own invariant check runs and its exported table is compared with
// the model's reference counts.  Exits non-zero on the first mismatch.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pagedattn.h"

// The library's error-text helpers live in the attention layer; the manager only needs
// their contract (record text, return the status).
namespace pa {
int fail(int status, const char* fmt, ...) {
  (void)fmt;
  return status;
}
int ok() { return PA_OK; }
}  // namespace pa

namespace {

struct Model {
  std::vector<int> len;  // -1: free slot
};

int check(pa_block_manager* bm, int num_pages, int page_size, int max_seqs, int max_pages,
          const Model& m) {
  if (pa_bm_validate(bm) != PA_OK) return 1;
  std::vector<int32_t> table((size_t)max_seqs * max_pages), lens(max_seqs);
  if (pa_bm_export(bm, table.data(), lens.data()) != PA_OK) return 2;
  std::vector<int> refs(num_pages, 0);
  for (int s = 0; s < max_seqs; ++s) {
    const int want = m.len[s] < 0 ? 0 : m.len[s];
    if (lens[s] != want || pa_bm_seq_len(bm, s) != m.len[s]) return 3;
    const int n = (want + page_size - 1) / page_size;
    for (int p = 0; p < max_pages; ++p) {
      const int32_t e = table[(size_t)s * max_pages + p];
      if (p < n) {
        if (e < 0 || e >= num_pages) return 4;
        ++refs[e];
      } else if (e != -1) {
        return 5;
      }
    }
  }
  int free_pages = 0;
  for (int p = 0; p < num_pages; ++p) {
    if (pa_bm_ref_count(bm, p) != refs[p]) return 6;
    free_pages += refs[p] == 0;
  }
  return pa_bm_free_page_count(bm) == free_pages ? 0 : 7;
}

}  // namespace

int main() {
  const int num_pages = 200, page_size = 16, max_seqs = 24, max_pages = 12;
  std::mt19937 rng(12345);
  for (int round = 0; round < 20; ++round) {
    pa_block_manager* bm = nullptr;
    if (pa_bm_create(num_pages, page_size, max_seqs, max_pages, &bm) != PA_OK) return 10;
    Model m;
    m.len.assign(max_seqs, -1);
    for (int step = 0; step < 3000; ++step) {
      std::vector<int> live;
      for (int s = 0; s < max_seqs; ++s)
        if (m.len[s] >= 0) live.push_back(s);
      const int op = (int)(rng() % 8);
      int st = PA_OK;
      if (op == 0 || live.empty()) {
        int32_t s = -1;
        st = pa_bm_add_sequence(bm, &s);
        if (st == PA_OK) m.len[s] = 0;
      } else if (op == 1) {
        const int p = live[rng() % live.size()];
        const int n = (int)(rng() % (m.len[p] + 1));
        int32_t c = -1;
        st = pa_bm_fork(bm, p, n, &c);
        if (st == PA_OK) m.len[c] = n;
      } else if (op == 2 && live.size() > 1) {
        const int s = live[rng() % live.size()];
        st = pa_bm_free_sequence(bm, s);
        if (st == PA_OK) m.len[s] = -1;
      } else {
        const int s = live[rng() % live.size()];
        const int n = (int)(rng() % 40);
        int32_t src = -1, dst = -1, nc = -1;
        st = pa_bm_append(bm, s, n, &src, &dst, &nc);
        if (st == PA_OK) {
          if (nc < 0 || nc > 1) return 11;
          if (nc == 1 && (src == dst || pa_bm_ref_count(bm, src) < 1 ||
                          pa_bm_ref_count(bm, dst) != 1))
            return 12;
          m.len[s] += n;
        }
      }
      // refusals must be the documented ones (capacity, or a length past the table)
      if (st != PA_OK && st != PA_ERR_CAPACITY && st != PA_ERR_INVALID_ARG) return 13;
      const int rc = check(bm, num_pages, page_size, max_seqs, max_pages, m);
      if (rc) {
        std::fprintf(stderr, "round %d step %d op %d: check %d\n", round, step, op, rc);
        return 20 + rc;
      }
    }
    pa_bm_destroy(bm);
  }
  // argument errors on a fresh manager
  pa_block_manager* bm = nullptr;
  if (pa_bm_create(0, 16, 1, 1, &bm) != PA_ERR_INVALID_ARG || bm != nullptr) return 30;
  if (pa_bm_create(8, 16, 2, 2, &bm) != PA_OK) return 31;
  int32_t s = -1, a = 0, b = 0, c = 0;
  if (pa_bm_add_sequence(bm, &s) != PA_OK) return 32;
  if (pa_bm_append(bm, s, 33, &a, &b, &c) != PA_ERR_INVALID_ARG) return 33;
  if (pa_bm_free_sequence(bm, 1) != PA_ERR_INVALID_ARG) return 34;
  if (pa_bm_fork(bm, s, 1, &a) != PA_ERR_INVALID_ARG) return 35;
  pa_bm_destroy(bm);
  pa_bm_destroy(nullptr);
  std::printf("block manager stress: ok\n");
  return 0;
}
