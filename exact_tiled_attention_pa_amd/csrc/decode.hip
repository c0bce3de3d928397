// Paged decode attention for gfx950: one query token per sequence over its whole
// paged KV cache.
//
// Decode reads every cached K/V byte once and does ~1 FLOP per byte, so it is
// bound by HBM bandwidth, not by math ("What is Paged FlashAttention?",
// "Does it change the attention result or complexity?": for single-token decoding
// the cache reads dominate).  The design therefore aims only at moving bytes the
// way HBM likes them:
//
//   pass 1 (decode_partial_kernel): grid (head group, split, sequence), the two inner
//     coordinates rotated by the sequence index.  A head group is the heads one wave
//     load covers: 64 lanes x 16 B = 1 KB = one token's row for 4 consecutive heads at
//     d = 128 (8 at d = 64), contiguous in the pool's [page, slot, head, d] layout.  Consecutive workgroups are the
//     head groups of the same key range, so concurrently running workgroups read
//     adjacent kilobytes of the same token rows (DRAM row locality), instead of
//     256-byte pieces 8 KB apart.  A split is a range of split_tokens key
//     positions (whole pages); with a sliding window the splits start at the
//     window's first key (rounded down to a multiple of 4), so a window of w keys
//     takes ceil(w / split_tokens) workgroups per head group and none walks keys
//     before it.  Its keys are streamed in steps of 16 tokens, each of the 4 waves
//     taking 4 consecutive tokens of a step, with buffer loads that write straight
//     into a per-wave ring of LDS slots (no VGPR staging, so the kernel needs few
//     registers and the ring, not the register file, sets how many bytes are in
//     flight: 4 steps = 32 KB per wave, 128 KB per CU).  Each lane reads its own 16
//     bytes back from LDS.  The physical page of every page the split touches comes
//     from the block table ("What is Paged FlashAttention?", "Practical example"),
//     one page per lane, fetched for the whole split by one vector load.
//     Dot products run on the VALU and are summed over the 16 lanes of a head
//     with DPP moves; every 16-lane row group keeps its own online-softmax state
//     (running max m, running sum l, output accumulator; "Flash Attention: Fast,
//     Memory-Efficient Attention for LLMs", "The Algorithm"), the 4 waves' states
//     are merged through LDS and the split's (m, l, unnormalised O) goes to the
//     workspace.
//   pass 2 (decode_combine_kernel): one wave per (sequence, head) merges the
//     splits' partials in order with the same rescaling algebra and writes bf16 O.
//
// Query head h reads K/V head h / (num_q_heads / num_kv_heads).  m is kept in
// log2 units (scores times scale * log2(e)) so every exponential is one v_exp_f32.

#include "device_util.h"
#include "kernels.h"
#include "lds_tile.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 16;                   // tokens per chunk (never straddles a page)
constexpr int kStep = kChunk / kWaves;       // consecutive tokens of a chunk per wave
constexpr int kRing = 5;                     // LDS slots per wave: 4 steps in flight
constexpr int kSlotBytes = kStep * 2 * 1024; // the step's K rows, then its V rows
constexpr float kEmptyMax = -1e30f;          // running max before any visible key (finite)

template <int D>
struct DecodeGeometry {
  static constexpr int kLanesPerHead = D / 8;          // 16 B (8 bf16) per lane
  static constexpr int kHeads = 64 / kLanesPerHead;    // heads per wave load
};

template <int D>
__global__ void __launch_bounds__(kThreads)
decode_partial_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
                      const uint16_t* __restrict__ v_pool,
                      const int32_t* __restrict__ block_table,
                      const int32_t* __restrict__ seq_lens, float* __restrict__ ws_o,
                      float* __restrict__ ws_ml, float scale_log2, int num_q_heads,
                      int num_kv_heads, int log2_ps, int max_pages, int split_tokens,
                      int max_splits, int window) {
  using G = DecodeGeometry<D>;
  constexpr int kRingBytes = kWaves * kRing * kSlotBytes;  // 160 KB: one workgroup per CU
  constexpr int kMergeBytes = (kWaves * G::kHeads * D + 2 * kWaves * G::kHeads) * 4;
  static_assert(kMergeBytes <= kRingBytes, "the merge arrays reuse the ring");
  constexpr uint32_t kOutside = 0x80000000u;   // a load offset past every buffer
  constexpr uint32_t kAllBytes = 0x7fffffffu;  // buffer size: offsets are checked here
  __shared__ __attribute__((aligned(1024))) char ring[kRingBytes];

  const int b = blockIdx.z;
  // grid rows and columns rotated by the sequence index: see rotated_grid_index
  const int hg = rotated_grid_index(blockIdx.x, gridDim.x, b);
  const int seq_len = seq_lens[b];
  const int split = rotated_grid_index(blockIdx.y, gridDim.y, b);
  // sliding window: only the last `window` keys count (t_lo on)
  const int t_lo = window > 0 ? max(0, seq_len - window) : 0;
  int t_begin, t_end;
  if (window > 0) {
    // splits laid from t_lo rounded down to a multiple of 4 (a wave's 4 consecutive
    // tokens then never straddle a page); the last one runs to the sequence end and
    // holds up to 3 keys more than split_tokens
    const int n_splits = window_split_count(seq_len, window, split_tokens);
    if (split >= n_splits) return;  // the combine pass never reads this split
    t_begin = (t_lo & ~3) + split * split_tokens;
    t_end = split == n_splits - 1 ? seq_len : t_begin + split_tokens;
  } else {
    t_begin = split * split_tokens;
    if (t_begin >= seq_len) return;  // the combine pass never reads this split
    t_end = min(seq_len, t_begin + split_tokens);
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane / G::kLanesPerHead;
  const int col = lane % G::kLanesPerHead;
  const int h = hg * G::kHeads + row;          // query head of this row group
  const bool active = h < num_q_heads;
  const int hk = (active ? h : 0) / (num_q_heads / num_kv_heads);
  const int ps_mask = (1 << log2_ps) - 1;
  const int token_bytes = num_kv_heads * D * 2;  // bytes between tokens in the pools
  // this lane's 16 bytes inside a token row; rows of absent heads load nothing
  const uint32_t lane_off = active ? (uint32_t)((hk * D + col * 8) * 2) : kOutside;

  // query slice of this lane, pre-multiplied by scale * log2(e)
  float qf[8];
  {
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (active)
      w = *reinterpret_cast<const u32x4*>(q + ((size_t)b * num_q_heads + h) * D + col * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qf[2 * i] = bf16_lo(w[i]) * scale_log2;
      qf[2 * i + 1] = bf16_hi(w[i]) * scale_log2;
    }
  }

  // physical page of each page the split touches, one per lane (a split holds at most
  // split_tokens + 3 <= 259 keys, so at most 18 pages of 16)
  const int n_chunks = (t_end - t_begin + kChunk - 1) / kChunk;
  const int page0 = t_begin >> log2_ps;
  int split_page = 0;
  if (lane <= ((t_end - 1) >> log2_ps) - page0)
    split_page = block_table[(size_t)b * max_pages + page0 + lane];
  // these loads complete here: the ring's loads below are not tracked by the compiler,
  // so no wait it would place for these may be left to count them
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // Step s = chunk s: this wave's tokens t_begin + 16 s + 4 w .. + 3 go to ring slot
  // s % kRing.  Steps past the end are issued too, with every lane out of range (they
  // write zeros to a free slot and read nothing), so each step is 8 loads and the
  // waits below are constants.
  const uint32_t ring_base = lds_address(ring) + (uint32_t)(wave * kRing * kSlotBytes);
  auto issue = [&](int s) {
    const int t0 = t_begin + s * kChunk + wave * kStep;
    const uint32_t slot = ring_base + (uint32_t)((s % kRing) * kSlotBytes);
    const bool live = s < n_chunks;
    const int phys =
        live ? __builtin_amdgcn_readlane(split_page, min((t0 >> log2_ps) - page0, 63)) : 0;
    const size_t row0 = (((size_t)phys << log2_ps) + (t0 & ps_mask)) * (size_t)token_bytes;
    const u32x4 rk = buffer_words(reinterpret_cast<const char*>(k_pool) + row0, kAllBytes);
    const u32x4 rv = buffer_words(reinterpret_cast<const char*>(v_pool) + row0, kAllBytes);
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const bool ok = live && t0 + i < t_end && t0 + i >= t_lo;
      const int voff = (int)(ok ? lane_off + (uint32_t)(i * token_bytes) : kOutside);
      lds_load16(rk, slot + i * 1024, voff);
      lds_load16(rv, slot + (kStep + i) * 1024, voff);
    }
  };

  float m = kEmptyMax, l = 0.f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;

  auto consume = [&](int s) {
    const int t0 = t_begin + s * kChunk + wave * kStep;
    const char* src = ring + wave * kRing * kSlotBytes + (s % kRing) * kSlotBytes + lane * 16;
    u32x4 kc[kStep], vc[kStep];
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      kc[i] = *reinterpret_cast<const u32x4*>(src + i * 1024);
      vc[i] = *reinterpret_cast<const u32x4*>(src + (kStep + i) * 1024);
    }
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
      sc[i] = (t0 + i < t_end && t0 + i >= t_lo) ? acc : -INFINITY;
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

#pragma unroll
  for (int s = 0; s < kRing - 1; ++s) issue(s);
  for (int s = 0; s < n_chunks; ++s) {
    // slot (s - 1) % kRing was read back by the previous consume, whose arithmetic
    // waited for those LDS reads, so it can take step s + kRing - 1 now
    issue(s + kRing - 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kRing - 1) * 2 * kStep));  // step s landed
    consume(s);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();  // every wave is done with the ring, which now holds the merge arrays

  // merge the 4 waves' states per head and write the split's partial
  auto sm_o = reinterpret_cast<float (*)[G::kHeads][D]>(ring);
  auto sm_m = reinterpret_cast<float (*)[G::kHeads]>(ring + kWaves * G::kHeads * D * 4);
  auto sm_l = reinterpret_cast<float (*)[G::kHeads]>(ring + kWaves * G::kHeads * (D + 1) * 4);
#pragma unroll
  for (int i = 0; i < 8; ++i) sm_o[wave][row][col * 8 + i] = o[i];
  if (col == 0) {
    sm_m[wave][row] = m;
    sm_l[wave][row] = l;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G::kHeads * D; idx += kThreads) {
    const int r = idx / D;
    const int d = idx % D;
    const int hh = hg * G::kHeads + r;
    if (hh >= num_q_heads) continue;
    float big = sm_m[0][r];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) big = fmaxf(big, sm_m[w][r]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(sm_m[w][r] - big);
      acc = fmaf(wt, sm_o[w][r][d], acc);
      lsum = fmaf(wt, sm_l[w][r], lsum);
    }
    const size_t slot = ((size_t)b * num_q_heads + hh) * max_splits + split;
    ws_o[slot * D + d] = acc;
    if (d == 0) {
      ws_ml[slot * 2] = big;
      ws_ml[slot * 2 + 1] = lsum;
    }
  }
}

// One wave per (sequence, head), four heads per workgroup: the wave walks the splits
// in order with the same online rescaling as pass 1 (running max, rescaled sum and
// output), each lane holding D / 64 output columns, and writes O / l as bf16.
constexpr int kCombineThreads = 256;
constexpr int kCombineHeads = kCombineThreads / 64;

template <int D>
__global__ void __launch_bounds__(kCombineThreads)
decode_combine_kernel(const int32_t* __restrict__ seq_lens, const float* __restrict__ ws_o,
                      const float* __restrict__ ws_ml, uint16_t* __restrict__ out,
                      int num_q_heads, int split_tokens, int max_splits, int window,
                      int window_aligned) {
  constexpr int kPerLane = D / 64;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * kCombineHeads + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (h >= num_q_heads) return;
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
  // splits in groups of kGroup: every load of a group is issued before any of its
  // partials is folded in (absent splits of the last group fold in with weight 0)
  constexpr int kGroup = 8;
  for (int s0 = s_first; s0 < n_splits; s0 += kGroup) {
    float ms[kGroup], ls[kGroup], os[kGroup][kPerLane];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const int s = min(s0 + i, n_splits - 1);
      ms[i] = s0 + i < n_splits ? ws_ml[(slot0 + s) * 2] : kEmptyMax;
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
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* dst = out + ((size_t)b * num_q_heads + h) * D + lane * kPerLane;
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) dst[e] = to_bf16_bits(acc[e] * inv);
}

template <int D>
void launch_partial(const DecodeArgs& a, hipStream_t stream) {
  using G = DecodeGeometry<D>;
  const dim3 grid((a.num_q_heads + G::kHeads - 1) / G::kHeads, decode_grid_splits(a), a.batch);
  hipLaunchKernelGGL(decode_partial_kernel<D>, grid, dim3(kThreads), 0, stream, a.q, a.k_pool,
                     a.v_pool, a.block_table, a.seq_lens, a.ws_o, a.ws_ml,
                     score_scale_log2(a.scale), a.num_q_heads, a.num_kv_heads,
                     a.log2_page_size, a.max_pages_per_seq, a.split_tokens, a.max_splits,
                     a.window);
}

}  // namespace

hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t stream) {
  if (decode_grouped(a)) return launch_decode_partial_gqa(a, stream);
  if (a.head_dim == 128) launch_partial<128>(a, stream);
  else launch_partial<64>(a, stream);
  return hipGetLastError();
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((a.num_q_heads + kCombineHeads - 1) / kCombineHeads, a.batch);
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(decode_combine_kernel<128>, grid, dim3(kCombineThreads), 0, stream,
                       a.seq_lens, a.ws_o, a.ws_ml, a.out, a.num_q_heads, a.split_tokens,
                       a.max_splits, a.window, decode_grouped(a) ? 0 : 1);
  } else {
    hipLaunchKernelGGL(decode_combine_kernel<64>, grid, dim3(kCombineThreads), 0, stream,
                       a.seq_lens, a.ws_o, a.ws_ml, a.out, a.num_q_heads, a.split_tokens,
                       a.max_splits, a.window, decode_grouped(a) ? 0 : 1);
  }
  return hipGetLastError();
}

}  // namespace pa
