// Paged decode attention for gfx950: one query token per sequence over its whole
// paged KV cache.
//
// Decode reads every cached K/V byte once and does ~1 FLOP per byte, so it is
// bound by HBM bandwidth, not by math ("What is Paged FlashAttention?",
// "Does it change the attention result or complexity?": for single-token decoding
// the cache reads dominate).  The design therefore aims only at moving bytes the
// way HBM likes them:
//
//   pass 1 (decode_plan_kernel, then decode_partial_kernel): the work is a list of
//     (sequence, split) pairs, a split being S = 256 consecutive keys, or 128 or 64
//     for batches too small to give every CU a unit with 256 (with a sliding window the
//     splits are laid back from the sequence end, so a window of w keys takes
//     ceil(w / S) of them), times the head groups: a head group is the heads
//     one wave load covers, 64 lanes x 16 B = 1 KB = one token's row for 4 adjacent
//     heads at d = 128 (8 at d = 64), contiguous in the pool's [page, slot, head, d]
//     layout.  A one-workgroup plan pass lists the pairs and sets a claim counter in
//     the workspace (skipped when the split slots of all sequences, times the head
//     groups, are at most one per workgroup: workgroup i then takes unit i in place).  Pass 1 then runs one persistent workgroup per CU: eight waves
//     stream K/V, one more (the scheduler) claims units (its first two fixed by its
//     index, the rest from the counter), resolves
//     each (its sequence, its table pages "What is Paged FlashAttention?", "Practical
//     example", its query slice) into an LDS descriptor a unit ahead, and merges and
//     stores each finished unit's partial.  The streaming waves take 4 consecutive
//     tokens each of every 32-token step with 16-byte non-temporal buffer loads into
//     registers, one step in flight while the previous one is consumed, and run on
//     from one unit into the next without draining: the scheduler issues every other
//     vector memory operation, so their wait counts cover only their own loads.  A
//     workgroup that streams for the whole launch moves far more bytes per second than
//     a short one per unit, which pays its first loads' latency each time (measured on
//     plain streaming probes: 6.2 TB/s with a 512 KB workgroup each, 7.0 persistent).
//     Dot products run on the VALU and are summed over the 16 lanes of a head with DPP
//     moves; every 16-lane row group keeps its own online-softmax state (running max
//     m, running sum l, output accumulator; "Flash Attention: Fast, Memory-Efficient
//     Attention for LLMs", "The Algorithm"); the waves' states are merged through LDS
//     and the unit's (m, l, unnormalised O) goes to the workspace.
//   pass 2 (decode_combine_kernel): four waves per (sequence, head) each merge every
//     fourth split's partial in order with the same rescaling algebra; their states
//     merge through LDS and one wave writes bf16 O.
//
// Query head h reads K/V head h / (num_q_heads / num_kv_heads).  m is kept in
// log2 units (scores times scale * log2(e)) so every exponential is one v_exp_f32.

#include <atomic>

#include "device_util.h"
#include "kernels.h"
#include "lds_tile.h"

namespace pa {
namespace {

constexpr int kStreamWaves = 8;                       // waves that stream K/V
constexpr int kThreads = (kStreamWaves + 1) * 64;     // plus one scheduler wave
constexpr int kStep = 4;                     // consecutive tokens of a step per wave
constexpr int kChunk = kStep * kStreamWaves; // tokens per step of a split
constexpr int kRing = 2;                     // register slots per streaming wave
constexpr int kAhead = kRing - 1;            // steps in flight ahead of the one consumed
constexpr int kQueue = 4;                    // split descriptors held in LDS
constexpr int kItemPages = 32;               // pages one split may touch (<= 17 here)
// A split is STEPS steps of kChunk keys: 8 (256 keys), or 4 and 2 (128 and 64 keys) for
// batches too small to give every CU a unit of work with 256-key splits.
template <int STEPS>
struct SplitShape {
  static constexpr int kSteps = STEPS;
  static constexpr int kTokens = STEPS * kChunk;
  static constexpr int kMidStep = STEPS / 2;  // step at which the next split is published
  static_assert(kSteps % kRing == 0, "every split starts in ring slot 0");
  static_assert(kSteps - kAhead >= kMidStep, "the next split is known before its loads");
};
constexpr float kEmptyMax = -1e30f;          // running max before any visible key (finite)
constexpr int kPlanThreads = 1024;

template <int D>
struct DecodeGeometry {
  static constexpr int kLanesPerHead = D / 8;          // 16 B (8 bf16) per lane
  static constexpr int kHeads = 64 / kLanesPerHead;    // heads per wave load
};

// One claimed unit of work: a split of one sequence for one head group, resolved by
// the scheduler wave (page numbers and the query slice included) for the streaming
// waves.
struct SplitDesc {
  int valid, b, split, hg;
  int t_begin, t_end, t_lo, page0;
  int pages[kItemPages];  // physical pages page0, page0 + 1, ... of the split
  u32x4 q[64];            // the head group's query rows, lane l's 16 bytes at q[l]
  uint32_t loff[64];      // lane l's byte offset inside a token row (absent head: past it)
};

template <int D>
struct DecodeShared {
  SplitDesc desc[kQueue];
  // each streaming wave's (O, m, l) per head at the end of a split, double-buffered
  float mo[2][kStreamWaves][DecodeGeometry<D>::kHeads][D];
  float mm[2][kStreamWaves][DecodeGeometry<D>::kHeads];
  float ml[2][kStreamWaves][DecodeGeometry<D>::kHeads];
};

// Workgroup barrier that waits only for this wave's LDS traffic: the streaming waves'
// buffer-to-LDS loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// Split key range [t_begin, t_end) of split `split` of a sequence of seq_len keys, splits
// of S keys.  Without a window split s covers keys S s .. S s + S - 1; with a sliding
// window the splits are laid back from the sequence end, so a window of w keys takes
// ceil(min(w, L) / S) splits of at most S keys, the first one reaching back to the
// window's first key (keys before it are masked).
template <int S>
__device__ __forceinline__ void split_range(int seq_len, int split, int window, int& t_begin,
                                            int& t_end) {
  if (window > 0) {
    const int n = window_split_count(seq_len, window, S);
    t_end = seq_len - (n - 1 - split) * S;
    t_begin = max(0, t_end - S);
  } else {
    t_begin = split * S;
    t_end = min(seq_len, t_begin + S);
  }
}

// Splits of a sequence of len keys that hold keys (inside the window, if any), at most
// max_splits: the plan and the partials hold max_splits per sequence.
__device__ inline int sequence_splits(int len, int window, int split_tokens, int max_splits) {
  const int n = window > 0 ? window_split_count(len, window, split_tokens)
                           : (len > 0 ? (len + split_tokens - 1) / split_tokens : 0);
  return min(n, max_splits);
}

// The first claims of each pass-1 workgroup (the split it starts on and the one it
// fetches ahead) are fixed: workgroup i takes units i and grid + i, and the counter
// starts past them.  Through the counter, all workgroups would queue on one address at
// launch.  Later claims stay on the counter: it keeps the workgroups running at one
// moment on neighbouring units (the head groups of one split read the same token rows).
constexpr int kFixedClaims = 2;

// The list of (sequence, split) pairs holding keys, in sequence order, and the claim
// counter of pass 1, both in the workspace: plan[0] = counter (set here to
// counter_start, the first unit no fixed claim takes), plan[1] = number of pairs,
// plan[2 + i] = pair i as the unsigned (sequence << 16) | split.  One workgroup scans the
// sequences' split counts.
__global__ void __launch_bounds__(kPlanThreads)
decode_plan_kernel(const int32_t* __restrict__ seq_lens, int batch, int split_tokens,
                   int max_splits, int window, int counter_start,
                   int32_t* __restrict__ plan) {
  __shared__ int scan[kPlanThreads];
  int base = 0;
  for (int c = 0; c < batch; c += kPlanThreads) {
    const int b = c + (int)threadIdx.x;
    int n = 0;
    if (b < batch) n = sequence_splits(seq_lens[b], window, split_tokens, max_splits);
    scan[threadIdx.x] = n;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
      const int add = threadIdx.x >= (unsigned)off ? scan[threadIdx.x - off] : 0;
      __syncthreads();
      scan[threadIdx.x] += add;
      __syncthreads();
    }
    // the chunk's pairs, written by all threads in order: entry e belongs to the first
    // sequence t of the chunk whose inclusive count exceeds e (a binary search of the
    // scan), as its split e - (count before t); one thread per sequence writing its own
    // pairs would serialise a long sequence's hundreds of splits
    const int total = scan[kPlanThreads - 1];
    for (int e = (int)threadIdx.x; e < total; e += kPlanThreads) {
      int lo = 0, hi = kPlanThreads - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (scan[mid] > e) hi = mid;
        else lo = mid + 1;
      }
      const int split = e - (lo > 0 ? scan[lo - 1] : 0);
      // packed unsigned: sequence indices reach 65534, past the int32 sign bit once shifted
      plan[2 + base + e] = (int32_t)(((uint32_t)(c + lo) << 16) | (uint32_t)split);
    }
    base += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    plan[0] = counter_start;
    plan[1] = base;
  }
}

// Pass 1: one persistent workgroup per CU.  The scheduler wave claims splits (after the
// fixed first two, from the plan's counter) two ahead of the streaming waves, resolves each (sequence, table
// pages, query slice) into an LDS descriptor, and merges and writes the partial of the
// split the streaming waves finished last; it issues every vector memory operation
// besides the K/V stream, so the streaming waves' wait counts cover their own loads
// only and their stream runs on across split boundaries without draining.
template <int D, int STEPS>
__global__ void __launch_bounds__(kThreads)
decode_partial_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
                      const uint16_t* __restrict__ v_pool,
                      const int32_t* __restrict__ block_table,
                      const int32_t* __restrict__ seq_lens, float* __restrict__ ws_o,
                      float* __restrict__ ws_ml, int32_t* __restrict__ plan,
                      float scale_log2, int num_q_heads, int num_kv_heads, int log2_ps,
                      int max_pages, int max_splits, int window, int in_place_batch) {
  using G = DecodeGeometry<D>;
  using SS = SplitShape<STEPS>;
  constexpr uint32_t kOutside = 0x80000000u;   // a load offset past every buffer
  constexpr uint32_t kAllBytes = 0x7fffffffu;  // buffer size: offsets are checked here
  __shared__ __attribute__((aligned(1024))) DecodeShared<D> sh;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_hg = (num_q_heads + G::kHeads - 1) / G::kHeads;
  const int row = lane / G::kLanesPerHead;
  const int col = lane % G::kLanesPerHead;

  if (wave == kStreamWaves) {
    // ------------------------------------------------------------- scheduler wave
    // in place: the units are every (sequence, split slot, head group), at most one
    // per workgroup, and no plan was written
    const int n_items =
        in_place_batch > 0 ? in_place_batch * max_splits * n_hg : plan[1] * n_hg;
    struct Claim { int valid, b, split, hg; };
    int claims = 0;  // made so far; the first kFixedClaims take fixed units
    auto resolve = [&](SplitDesc& d) -> Claim {
      Claim c{0, 0, 0, 0};
      if (in_place_batch > 0) {
        // unit i is workgroup i's only one; a split slot holding no keys of its
        // sequence leaves the workgroup without work
        const int qi = claims++ == 0 ? (int)blockIdx.x : n_items;
        if (qi < n_items) {
          const int p = qi / n_hg;
          c = Claim{0, p / max_splits, p % max_splits, qi % n_hg};
          c.valid = c.split < sequence_splits(seq_lens[c.b], window, SS::kTokens, max_splits);
        }
      } else {
        int qi = (int)blockIdx.x + claims * (int)gridDim.x;
        if (claims >= kFixedClaims) {
          if (lane == 0) qi = atomicAdd(&plan[0], 1);
          qi = __builtin_amdgcn_readfirstlane(qi);
        }
        ++claims;
        if (qi < n_items) {
          const uint32_t pair = (uint32_t)plan[2 + qi / n_hg];
          c = Claim{1, (int)(pair >> 16), (int)(pair & 0xffffu), qi % n_hg};
        }
      }
      if (!c.valid) {
        if (lane == 0) d.valid = 0;
        return c;
      }
      const int seq_len = seq_lens[c.b];
      int t_begin, t_end;
      split_range<SS::kTokens>(seq_len, c.split, window, t_begin, t_end);
      const int page0 = t_begin >> log2_ps;
      if (lane <= ((t_end - 1) >> log2_ps) - page0)
        d.pages[lane] = block_table[(size_t)c.b * max_pages + page0 + lane];
      const int h = c.hg * G::kHeads + row;
      u32x4 w = u32x4{0u, 0u, 0u, 0u};
      if (h < num_q_heads)
        w = *reinterpret_cast<const u32x4*>(q + ((size_t)c.b * num_q_heads + h) * D + col * 8);
      d.q[lane] = w;
      d.loff[lane] = h < num_q_heads
                         ? (uint32_t)(((h / (num_q_heads / num_kv_heads)) * D + col * 8) * 2)
                         : 0x80000000u;
      if (lane == 0) {
        d.valid = 1;
        d.b = c.b;
        d.split = c.split;
        d.hg = c.hg;
        d.t_begin = t_begin;
        d.t_end = t_end;
        d.t_lo = window > 0 ? max(0, seq_len - window) : 0;
        d.page0 = page0;
      }
      return c;
    };
    // the streaming waves' states of a finished split -> its partial in the workspace
    auto merge = [&](const Claim& c, int buf) {
      for (int idx = lane; idx < G::kHeads * D; idx += 64) {
        const int r = idx / D;
        const int d = idx % D;
        const int hh = c.hg * G::kHeads + r;
        if (hh >= num_q_heads) continue;
        float big = sh.mm[buf][0][r];
#pragma unroll
        for (int w = 1; w < kStreamWaves; ++w) big = fmaxf(big, sh.mm[buf][w][r]);
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < kStreamWaves; ++w) {
          const float wt = fast_exp2(sh.mm[buf][w][r] - big);
          acc = fmaf(wt, sh.mo[buf][w][r][d], acc);
          lsum = fmaf(wt, sh.ml[buf][w][r], lsum);
        }
        const size_t slot = ((size_t)c.b * num_q_heads + hh) * max_splits + c.split;
        ws_o[slot * D + d] = acc;
        if (d == 0) {
          ws_ml[slot * 2] = big;
          ws_ml[slot * 2 + 1] = lsum;
        }
      }
    };
    Claim prev{0, 0, 0, 0};
    Claim cur = resolve(sh.desc[0]);
    lds_barrier();  // split 0 published
    for (int k = 0;; ++k) {
      if (!cur.valid) {
        if (prev.valid) merge(prev, (k - 1) & 1);
        break;
      }
      const Claim nxt = resolve(sh.desc[(k + 1) % kQueue]);
      lds_barrier();  // mid-split: split k + 1 published
      if (prev.valid) merge(prev, (k - 1) & 1);
      lds_barrier();  // end of split k: its states are in mo/mm/ml[k & 1]
      prev = cur;
      cur = nxt;
    }
    return;
  }

  // --------------------------------------------------------------- streaming waves
  const int ps_mask = (1 << log2_ps) - 1;
  const int token_bytes = num_kv_heads * D * 2;  // bytes between tokens in the pools

  // split being consumed (c_*) and split being issued ahead (n_*, once published)
  int c_valid, c_tb, c_te, c_tlo, c_page0, c_pages, c_hg;
  int n_valid = 0, n_tb = 0, n_te = 0, n_tlo = 0, n_page0 = 0, n_pages = 0;
  float qf[8];
  uint32_t lane_off = kOutside, n_lane_off = kOutside;
  auto load_desc = [&](const SplitDesc& d, int& valid, int& tb, int& te, int& tlo, int& page0,
                       int& pages, int& hg) {
    valid = __builtin_amdgcn_readfirstlane(d.valid);
    tb = __builtin_amdgcn_readfirstlane(d.t_begin);
    te = __builtin_amdgcn_readfirstlane(d.t_end);
    tlo = __builtin_amdgcn_readfirstlane(d.t_lo);
    page0 = __builtin_amdgcn_readfirstlane(d.page0);
    hg = __builtin_amdgcn_readfirstlane(d.hg);
    pages = d.pages[lane & (kItemPages - 1)];
  };
  auto load_query = [&](const SplitDesc& d) {
    const u32x4 w = d.q[lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qf[2 * i] = bf16_lo(w[i]) * scale_log2;
      qf[2 * i + 1] = bf16_hi(w[i]) * scale_log2;
    }
  };

  // K/V rows of the steps in flight, in registers: step si of a split sits in slot
  // si % kRing (a split is SS::kSteps steps, a multiple of kRing, so each starts in
  // slot 0), token i of
  // the wave's 4 at [slot][i]
  u32x4 kr[kRing][kStep], vr[kRing][kStep];

  // Step si of a split: its tokens t_begin + 32 si + 4 wave + i (i < 4), one 16-byte
  // buffer load per token and pool.  Each token finds its own page (with windowed
  // splits laid back from the sequence end a wave's 4 tokens may straddle two), and
  // tokens outside the split's keys or before the window load with an offset past the
  // buffer: zeros come back and nothing is read.  Branch-free, so that no register of a
  // load still in flight is taken for a temporary on some path.
  auto issue = [&](int valid, int tb, int te, int tlo, int page0, int pages, uint32_t loff,
                   int si, u32x4* kd, u32x4* vd) {
    const int t0 = tb + si * kChunk + wave * kStep;
    const int te_eff = valid ? te : INT_MIN;  // an invalid split loads nothing
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const int t = t0 + i;
      const bool ok = t < te_eff && t >= tlo;
      const int pidx = min(max((t >> log2_ps) - page0, 0), kItemPages - 1);
      const int phys = __builtin_amdgcn_readlane(pages, pidx);
      const size_t row = (((size_t)(uint32_t)phys << log2_ps) + (t & ps_mask)) * (size_t)token_bytes;
      const __amdgpu_buffer_rsrc_t rk =
          make_rsrc(reinterpret_cast<const char*>(k_pool) + row, (int)kAllBytes);
      const __amdgpu_buffer_rsrc_t rv =
          make_rsrc(reinterpret_cast<const char*>(v_pool) + row, (int)kAllBytes);
      const int voff = (int)(ok ? loff : kOutside);
      // non-temporal: every K/V byte is read once
      kd[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, voff, 0, 2));
      vd[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 2));
    }
  };

  float m = kEmptyMax, l = 0.f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;

  auto consume = [&](int si, const u32x4* kc, const u32x4* vc) {
    const int t0 = c_tb + si * kChunk + wave * kStep;
    float sc[kStep];
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = fmaf(qf[2 * w], bf16_lo(kc[i][w]), acc);
        acc = fmaf(qf[2 * w + 1], bf16_hi(kc[i][w]), acc);
      }
      acc = group_sum<G::kLanesPerHead>(acc);
      sc[i] = (t0 + i < c_te && t0 + i >= c_tlo) ? acc : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < kStep; ++i) mx = fmaxf(mx, sc[i]);
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    float psum = 0.f;
    float p[kStep];
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      p[i] = fast_exp2(sc[i] - m_new);
      psum += p[i];
    }
    l = l * alpha + psum;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float lo = o[2 * w] * alpha;
      float hi = o[2 * w + 1] * alpha;
#pragma unroll
      for (int i = 0; i < kStep; ++i) {
        lo = fmaf(p[i], bf16_lo(vc[i][w]), lo);
        hi = fmaf(p[i], bf16_hi(vc[i][w]), hi);
      }
      o[2 * w] = lo;
      o[2 * w + 1] = hi;
    }
    m = m_new;
  };

  lds_barrier();  // split 0 published
  load_desc(sh.desc[0], c_valid, c_tb, c_te, c_tlo, c_page0, c_pages, c_hg);
  if (!c_valid) return;
  load_query(sh.desc[0]);
  lane_off = sh.desc[0].loff[lane];
#pragma unroll
  for (int a = 0; a < kAhead; ++a)
    issue(c_valid, c_tb, c_te, c_tlo, c_page0, c_pages, lane_off, a, kr[a], vr[a]);

  for (int k = 0;; ++k) {
#pragma unroll
    for (int si = 0; si < SS::kSteps; ++si) {
      if (si == SS::kMidStep) {
        lds_barrier();  // split k + 1 published
        int n_hg;
        load_desc(sh.desc[(k + 1) % kQueue], n_valid, n_tb, n_te, n_tlo, n_page0, n_pages, n_hg);
        n_lane_off = sh.desc[(k + 1) % kQueue].loff[lane];
      }
      // step si + kAhead of this split, or one of the next split's first steps, into the
      // slot the previous step was consumed from
      const int ahead = si + kAhead;
      if (ahead < SS::kSteps)
        issue(c_valid, c_tb, c_te, c_tlo, c_page0, c_pages, lane_off, ahead,
              kr[ahead % kRing], vr[ahead % kRing]);
      else
        issue(n_valid, n_tb, n_te, n_tlo, n_page0, n_pages, n_lane_off, ahead - SS::kSteps,
              kr[ahead % kRing], vr[ahead % kRing]);
      consume(si, kr[si % kRing], vr[si % kRing]);
      // keep the steps in program order: hoisting later steps' loads and address work
      // into this one only lengthens register lifetimes
      __builtin_amdgcn_sched_barrier(0);
    }
    // end of split k: its state per head for the scheduler's merge
    const int buf = k & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) sh.mo[buf][wave][row][col * 8 + i] = o[i];
    if (col == 0) {
      sh.mm[buf][wave][row] = m;
      sh.ml[buf][wave][row] = l;
    }
    lds_barrier();
    if (!n_valid) break;
    c_valid = n_valid;
    c_tb = n_tb;
    c_te = n_te;
    c_tlo = n_tlo;
    c_page0 = n_page0;
    c_pages = n_pages;
    lane_off = n_lane_off;
    load_query(sh.desc[(k + 1) % kQueue]);
    m = kEmptyMax;
    l = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.f;
  }
  // the loads issued ahead for a split that does not exist read nothing; let them
  // retire before the wave ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// WAVES waves per (sequence, head): wave w folds splits w, w + WAVES, ... in order with
// the same online rescaling as pass 1 (running max, rescaled sum and output), each lane
// holding D / 64 output columns; the states then merge through LDS with the same
// algebra (weights 2^(m_w - M)) and wave 0 writes O / l as bf16.  The fold is a chain of
// dependent steps, so a long sequence's splits in one chain made the pass
// latency-bound: 4 waves, or 16 when the launch has fewer (sequence, head) pairs than
// the chip has CUs (a small batch, whose splits are short and many).
template <int D, int WAVES>
__global__ void __launch_bounds__(64 * WAVES)
decode_combine_kernel(const int32_t* __restrict__ seq_lens, const float* __restrict__ ws_o,
                      const float* __restrict__ ws_ml, uint16_t* __restrict__ out,
                      int num_q_heads, int split_tokens, int max_splits, int window,
                      int window_aligned) {
  constexpr int kPerLane = D / 64;
  constexpr int kCombineWaves = WAVES;
  __shared__ float st_ml[kCombineWaves][2];
  __shared__ float st_o[kCombineWaves][D];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int seq_len = seq_lens[b];
  // splits holding keys: with a window, the window-aligned splits of the
  // one-head-per-row decode (0 .. count - 1), or the grouped-head decode's splits from
  // the one holding the window's first key
  int s_first = 0;
  int n_splits = seq_len > 0 ? (seq_len + split_tokens - 1) / split_tokens : 0;
  if (window > 0 && window_aligned) n_splits = window_split_count(seq_len, window, split_tokens);
  else if (window > 0) s_first = max(0, seq_len - window) / split_tokens;
  const size_t slot0 = ((size_t)b * num_q_heads + h) * max_splits;

  float m = kEmptyMax, l = 0.f;
  float acc[kPerLane];
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) acc[e] = 0.f;
  // this wave's splits in groups of kGroup: every load of a group is issued before any
  // of its partials is folded in (absent splits of the last group fold in with weight 0)
  constexpr int kGroup = 8;
  for (int s0 = s_first + wave; s0 < n_splits; s0 += kCombineWaves * kGroup) {
    float ms[kGroup], ls[kGroup], os[kGroup][kPerLane];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const int si = s0 + kCombineWaves * i;
      const int s = min(si, n_splits - 1);
      ms[i] = si < n_splits ? ws_ml[(slot0 + s) * 2] : kEmptyMax;
      ls[i] = ws_ml[(slot0 + s) * 2 + 1];
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) os[i][e] = ws_o[(slot0 + s) * D + lane * kPerLane + e];
    }
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const float m_new = fmaxf(m, ms[i]);
      const float a = fast_exp2(m - m_new);
      const float w = fast_exp2(ms[i] - m_new);
      l = fmaf(l, a, w * ls[i]);
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) acc[e] = fmaf(acc[e], a, w * os[i][e]);
      m = m_new;
    }
  }
  // merge: a wave with no split holds m = kEmptyMax, l = 0, O = 0 and gets weight 0
  if (lane == 0) {
    st_ml[wave][0] = m;
    st_ml[wave][1] = l;
  }
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) st_o[wave][lane * kPerLane + e] = acc[e];
  __syncthreads();
  if (wave != 0) return;
  float big = st_ml[0][0];
#pragma unroll
  for (int w = 1; w < kCombineWaves; ++w) big = fmaxf(big, st_ml[w][0]);
  float lt = 0.f;
  float ot[kPerLane];
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) ot[e] = 0.f;
#pragma unroll
  for (int w = 0; w < kCombineWaves; ++w) {
    const float a = fast_exp2(st_ml[w][0] - big);
    lt = fmaf(a, st_ml[w][1], lt);
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) ot[e] = fmaf(a, st_o[w][lane * kPerLane + e], ot[e]);
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* dst = out + ((size_t)b * num_q_heads + h) * D + lane * kPerLane;
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) dst[e] = to_bf16_bits(ot[e] * inv);
}

// Compute units of the current device, looked up once per device (pass 1 runs one
// persistent workgroup per CU).  Calls from several host threads may race to fill an
// entry; they store the same value.
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, int STEPS>
void launch_partial(const DecodeArgs& a, hipStream_t stream) {
  using G = DecodeGeometry<D>;
  const int grid = cu_count();
  // when the (sequence, split slot, head group) space holds at most one unit per
  // workgroup, workgroup i takes unit i in place and the plan pass is not needed.  Not
  // with two per workgroup: the slots holding keys are a prefix of each sequence's
  // range, so by index some workgroups could get two units where the plan gives none
  // more than one
  const int64_t slots = (int64_t)a.batch * a.max_splits *
                        ((a.num_q_heads + G::kHeads - 1) / G::kHeads);
  const int in_place_batch = slots <= grid ? a.batch : 0;
  if (in_place_batch == 0)
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a.seq_lens,
                       a.batch, a.split_tokens, a.max_splits, a.window, kFixedClaims * grid,
                       a.plan);
  hipLaunchKernelGGL((decode_partial_kernel<D, STEPS>), dim3(grid), dim3(kThreads), 0,
                     stream,
                     a.q, a.k_pool, a.v_pool, a.block_table, a.seq_lens, a.ws_o, a.ws_ml,
                     a.plan, score_scale_log2(a.scale), a.num_q_heads, a.num_kv_heads,
                     a.log2_page_size, a.max_pages_per_seq, a.max_splits, a.window,
                     in_place_batch);
}

}  // namespace

hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t stream) {
  if (decode_grouped(a)) return launch_decode_partial_gqa(a, stream);
  // one-head-per-row splits of 256, 128 or 64 keys (the host layer picks the length)
  const bool d128 = a.head_dim == 128;
  switch (a.split_tokens) {
    case 8 * kChunk: d128 ? launch_partial<128, 8>(a, stream) : launch_partial<64, 8>(a, stream); break;
    case 4 * kChunk: d128 ? launch_partial<128, 4>(a, stream) : launch_partial<64, 4>(a, stream); break;
    case 2 * kChunk: d128 ? launch_partial<128, 2>(a, stream) : launch_partial<64, 2>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int WAVES>
void launch_combine(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, a.batch);
  hipLaunchKernelGGL((decode_combine_kernel<D, WAVES>), grid, dim3(64 * WAVES), 0, stream,
                     a.seq_lens, a.ws_o, a.ws_ml, a.out, a.num_q_heads, a.split_tokens,
                     a.max_splits, a.window, decode_grouped(a) ? 0 : 1);
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream) {
  const bool wide = (long long)a.num_q_heads * a.batch < cu_count();
  if (a.head_dim == 128) wide ? launch_combine<128, 16>(a, stream) : launch_combine<128, 4>(a, stream);
  else wide ? launch_combine<64, 16>(a, stream) : launch_combine<64, 4>(a, stream);
  return hipGetLastError();
}

}  // namespace pa
