// Paged decode attention for gfx950: one query token per sequence over its whole
// paged KV cache.
//
// Decode reads every cached K/V byte once and does ~1 FLOP per byte, so it is
// bound by HBM bandwidth, not by math ("What is Paged FlashAttention?",
// "Does it change the attention result or complexity?": for single-token decoding
// the cache reads dominate).  The design therefore aims only at keeping enough
// bytes in flight:
//
//   pass 1 (decode_partial_kernel): grid (split, query head, sequence).  A split
//     is a range of split_tokens key positions (whole pages).  Its 4 waves take
//     16-token chunks round-robin; a wave reads a chunk's K and V rows straight
//     into registers (16 B per lane, one 256 B row per 16 lanes at d = 128), with
//     the next chunk's loads issued before the current chunk is consumed.  The
//     physical page of each chunk comes from the block table ("What is Paged
//     FlashAttention?", "Practical example"), fetched for all of the wave's
//     chunks by one vector load up front.  Dot products run on the VALU and are
//     summed across the 16 lanes of a row with DPP moves.  Each 16-lane row group
//     keeps its own online-softmax state (running max m, running sum l, output
//     accumulator; "Flash Attention: Fast, Memory-Efficient Attention for
//     LLMs", "The Algorithm"), so the inner loop needs no cross-row exchange; the
//     16 row-group states of the workgroup are merged once through LDS and the
//     split's (m, l, unnormalised O) is written to the workspace.
//   pass 2 (decode_combine_kernel): per (sequence, head), merges the splits'
//     partials with the same rescaling algebra and writes bf16 O.
//
// m is kept in log2 units (scores times scale * log2(e)) so that every
// exponential is a single v_exp_f32.

#include "device_util.h"
#include "kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 16;           // tokens per wave work unit
constexpr float kEmptyMax = -1e30f;  // running max before any visible key (finite)

template <int D>
__global__ void __launch_bounds__(kThreads)
decode_partial_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
                      const uint16_t* __restrict__ v_pool,
                      const int32_t* __restrict__ block_table,
                      const int32_t* __restrict__ seq_lens, float* __restrict__ ws_o,
                      float* __restrict__ ws_ml, float scale_log2, int num_q_heads,
                      int num_kv_heads, int log2_ps, int max_pages, int split_tokens,
                      int max_splits) {
  constexpr int kLanesPerRow = D / 8;        // 16 B (8 bf16) per lane
  constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  constexpr int kLoads = kChunk / kRowsPerLoad;
  constexpr int kGroups = kWaves * kRowsPerLoad;

  __shared__ float sm_o[kGroups][D];
  __shared__ float sm_m[kGroups];
  __shared__ float sm_l[kGroups];

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int seq_len = seq_lens[b];
  const int t_begin = split * split_tokens;
  if (t_begin >= seq_len) return;  // the combine pass never reads this split
  const int t_end = min(seq_len, t_begin + split_tokens);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane / kLanesPerRow;
  const int col = lane % kLanesPerRow;
  const int hk = h / (num_q_heads / num_kv_heads);
  const int ps_mask = (1 << log2_ps) - 1;
  const size_t token_stride = (size_t)num_kv_heads * D;  // elements between tokens

  // query slice of this lane, pre-multiplied by scale * log2(e)
  float qf[8];
  {
    const u32x4 w = *reinterpret_cast<const u32x4*>(
        q + ((size_t)b * num_q_heads + h) * D + col * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qf[2 * i] = bf16_lo(w[i]) * scale_log2;
      qf[2 * i + 1] = bf16_hi(w[i]) * scale_log2;
    }
  }

  // chunks of this split handled by this wave: wave, wave + 4, ...
  const int n_chunks = (t_end - t_begin + kChunk - 1) / kChunk;
  const int my_chunks = n_chunks > wave ? (n_chunks - wave + kWaves - 1) / kWaves : 0;

  // physical page of each of this wave's chunks, one per lane
  int my_page = 0;
  if (lane < my_chunks) {
    const int t0 = t_begin + (wave + lane * kWaves) * kChunk;
    my_page = block_table[(size_t)b * max_pages + (t0 >> log2_ps)];
  }

  float m = kEmptyMax, l = 0.f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;

  u32x4 kbuf[kLoads], vbuf[kLoads];

  auto issue = [&](int c, u32x4* kd, u32x4* vd) {
    const int t0 = t_begin + (wave + c * kWaves) * kChunk;
    const int phys = __builtin_amdgcn_readlane(my_page, c);
    const size_t base =
        (((size_t)phys << log2_ps) + (t0 & ps_mask)) * token_stride + (size_t)hk * D + col * 8;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int r = i * kRowsPerLoad + row;
      if (t0 + r < t_end) {
        kd[i] = *reinterpret_cast<const u32x4*>(k_pool + base + r * token_stride);
        vd[i] = *reinterpret_cast<const u32x4*>(v_pool + base + r * token_stride);
      } else {
        kd[i] = u32x4{0u, 0u, 0u, 0u};
        vd[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  if (my_chunks > 0) issue(0, kbuf, vbuf);

  for (int c = 0; c < my_chunks; ++c) {
    u32x4 kc[kLoads], vc[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      kc[i] = kbuf[i];
      vc[i] = vbuf[i];
    }
    if (c + 1 < my_chunks) issue(c + 1, kbuf, vbuf);

    const int t0 = t_begin + (wave + c * kWaves) * kChunk;
    float s[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = fmaf(qf[2 * w], bf16_lo(kc[i][w]), acc);
        acc = fmaf(qf[2 * w + 1], bf16_hi(kc[i][w]), acc);
      }
      acc = group_sum<kLanesPerRow>(acc);
      s[i] = (t0 + i * kRowsPerLoad + row < t_end) ? acc : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < kLoads; ++i) mx = fmaxf(mx, s[i]);
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    float psum = 0.f;
    float p[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      p[i] = fast_exp2(s[i] - m_new);
      psum += p[i];
    }
    l = l * alpha + psum;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float lo = o[2 * w] * alpha;
      float hi = o[2 * w + 1] * alpha;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        lo = fmaf(p[i], bf16_lo(vc[i][w]), lo);
        hi = fmaf(p[i], bf16_hi(vc[i][w]), hi);
      }
      o[2 * w] = lo;
      o[2 * w + 1] = hi;
    }
    m = m_new;
  }

  // merge the workgroup's row groups
  const int g = wave * kRowsPerLoad + row;
#pragma unroll
  for (int i = 0; i < 8; ++i) sm_o[g][col * 8 + i] = o[i];
  if (col == 0) {
    sm_m[g] = m;
    sm_l[g] = l;
  }
  __syncthreads();
  const size_t slot = ((size_t)b * num_q_heads + h) * max_splits + split;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float big = sm_m[0];
#pragma unroll
    for (int j = 1; j < kGroups; ++j) big = fmaxf(big, sm_m[j]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
      const float w = fast_exp2(sm_m[j] - big);
      acc = fmaf(w, sm_o[j][d], acc);
      lsum = fmaf(w, sm_l[j], lsum);
    }
    ws_o[slot * D + d] = acc;
    if (d == 0) {
      ws_ml[slot * 2] = big;
      ws_ml[slot * 2 + 1] = lsum;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(D)
decode_combine_kernel(const int32_t* __restrict__ seq_lens, const float* __restrict__ ws_o,
                      const float* __restrict__ ws_ml, uint16_t* __restrict__ out,
                      int num_q_heads, int split_tokens, int max_splits) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int seq_len = seq_lens[b];
  const int n_splits = seq_len > 0 ? (seq_len + split_tokens - 1) / split_tokens : 0;
  const size_t slot0 = ((size_t)b * num_q_heads + h) * max_splits;
  float big = kEmptyMax;
  for (int s = 0; s < n_splits; ++s) big = fmaxf(big, ws_ml[(slot0 + s) * 2]);
  float acc = 0.f, lsum = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const float w = fast_exp2(ws_ml[(slot0 + s) * 2] - big);
    acc = fmaf(w, ws_o[(slot0 + s) * D + d], acc);
    lsum = fmaf(w, ws_ml[(slot0 + s) * 2 + 1], lsum);
  }
  const float r = lsum > 0.f ? acc / lsum : 0.f;
  out[((size_t)b * num_q_heads + h) * D + d] = to_bf16_bits(r);
}

}  // namespace

hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.max_splits, a.num_q_heads, a.batch);
  const float c = score_scale_log2(a.scale);
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(decode_partial_kernel<128>, grid, dim3(kThreads), 0, stream, a.q,
                       a.k_pool, a.v_pool, a.block_table, a.seq_lens, a.ws_o, a.ws_ml, c,
                       a.num_q_heads, a.num_kv_heads, a.log2_page_size, a.max_pages_per_seq,
                       a.split_tokens, a.max_splits);
  } else {
    hipLaunchKernelGGL(decode_partial_kernel<64>, grid, dim3(kThreads), 0, stream, a.q,
                       a.k_pool, a.v_pool, a.block_table, a.seq_lens, a.ws_o, a.ws_ml, c,
                       a.num_q_heads, a.num_kv_heads, a.log2_page_size, a.max_pages_per_seq,
                       a.split_tokens, a.max_splits);
  }
  return hipGetLastError();
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, a.batch);
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(decode_combine_kernel<128>, grid, dim3(128), 0, stream, a.seq_lens,
                       a.ws_o, a.ws_ml, a.out, a.num_q_heads, a.split_tokens, a.max_splits);
  } else {
    hipLaunchKernelGGL(decode_combine_kernel<64>, grid, dim3(64), 0, stream, a.seq_lens,
                       a.ws_o, a.ws_ml, a.out, a.num_q_heads, a.split_tokens, a.max_splits);
  }
  return hipGetLastError();
}

}  // namespace pa
