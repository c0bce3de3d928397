// Paged decode for grouped K/V heads on gfx950: each K/V page is read once for all
// the query heads that share it.
//
// With g = num_q_heads / num_kv_heads > 1 query heads per K/V head ("Flash Attention:
// Fast, Memory-Efficient Attention for LLMs", "Attention Variants": grouped-query and
// multi-query attention), a decode step still reads every cached K/V byte once, but
// each byte now feeds g dot products, g exponentials and g weighted sums.  The
// kernel therefore treats the g query heads of one token like the rows of a small
// query tile and runs both contractions on the matrix cores:
//
//   grid  (K/V head x head block, split, sequence), both inner coordinates rotated by
//         the sequence index.  A head block is up to 32 of the g query heads (one MFMA
//         operand's worth); g > 32 takes several blocks.
//         Splits are the same key ranges as the one-head-per-row decode, and the
//         partials go to the same workspace, so the same combine pass finishes.
//   block 4 waves.  The split's keys come in tiles of 32 positions; wave w takes
//         tiles w, w + 4, ...  Each wave streams its tile straight from the pools
//         into its own LDS region (16-byte buffer loads to LDS, rows past the
//         sequence end read as zeros, pages found through the block table: "What is
//         Paged FlashAttention?", "Practical example").
//   per tile  S^T = K Q^T (v_mfma_f32_32x32x16_bf16, Q of the head block held in
//         VGPRs as the B operand, so each lane holds the scores of one query head),
//         the online-softmax update in fp32 with a lazily raised reference max
//         ("The Algorithm" on the same page), P rounded to bf16 with the row sum
//         taken over the rounded values, then O^T += V^T P^T with V^T read by the
//         transposing LDS read.  Rows of the head block past g hold zero queries and
//         are never written.
//   end   the 4 waves' (m, l, O) are merged through LDS and the split's partial is
//         written to the workspace (m in log2 units, O unnormalised).
//
// The tile layout, swizzles and MFMA operand orders are those of the prefill kernel:
// K chunk c of row r at slot c ^ (r mod chunks), V at slot c ^ v_swizzle(r mod 4);
// register r of the S^T block holds key 8(r/4) + 4(lane/32) + r%4.

#include "device_util.h"
#include "kernels.h"
#include "lds_tile.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 32;               // keys per tile
constexpr int kHeadBlock = 32;          // query heads per workgroup (MFMA columns)
constexpr int kRescaleThreshold = 8;    // log2 units a row max may grow before rescaling
// cache policy of the K/V loads: non-temporal, every byte is read once (227.5 -> 206.3 us
// on a 64-sequence, 8-K/V-head decode against the default policy, same box)
constexpr int kNonTemporal = 2;

template <int D>
struct GqaGeometry {
  static constexpr int kRowBytes = 2 * D;                    // one K or V row in LDS
  static constexpr int kChunks = D / 8;                      // 16-byte chunks per row
  static constexpr int kRowsPerInst = 1024 / kRowBytes;      // rows per 1 KB load
  static constexpr int kInstPerTile = kTile / kRowsPerInst;  // loads per K (or V) tile
  static constexpr int kInstPerGroup = 16 / kRowsPerInst;    // loads per 16-row group
  static constexpr int kTileBytes = kTile * kRowBytes;
  static constexpr int kDK = D / 16;                         // MFMA k-steps over d
  static constexpr int kDB = D / 32;                         // 32-row output blocks
  static constexpr int kOStride = D + 4;                     // merge row stride, floats
  // a wave's LDS region: its K and V tiles, later its [head][d] fp32 partial
  static constexpr int kRegionBytes =
      (2 * kTileBytes > kHeadBlock * kOStride * 4) ? 2 * kTileBytes
                                                   : kHeadBlock * kOStride * 4;
};

template <int D>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
decode_gqa_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
                  const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ block_table,
                  const int32_t* __restrict__ seq_lens, float* __restrict__ ws_o,
                  float* __restrict__ ws_ml, float scale_log2, int num_q_heads,
                  int num_kv_heads, int log2_ps, int max_pages, int split_tokens,
                  int max_splits, int window) {
  using G = GqaGeometry<D>;
  __shared__ __attribute__((aligned(1024))) char lds[kWaves][G::kRegionBytes];
  __shared__ float sm_m[kWaves][kHeadBlock];
  __shared__ float sm_l[kWaves][kHeadBlock];

  const int group = num_q_heads / num_kv_heads;
  const int blocks_per_kv = (group + kHeadBlock - 1) / kHeadBlock;
  const int b = blockIdx.z;
  // grid rows and columns rotated by the sequence index (a bijection per sequence): see
  // rotated_grid_index
  const int col = rotated_grid_index(blockIdx.x, gridDim.x, b);
  const int hk = col / blocks_per_kv;
  const int hb = col % blocks_per_kv;
  const int h0 = hk * group + hb * kHeadBlock;          // first query head of the block
  const int nh = min(kHeadBlock, group - hb * kHeadBlock);
  const int seq_len = seq_lens[b];
  const int split =
      decode_split_of(rotated_grid_index(blockIdx.y, gridDim.y, b), seq_len, split_tokens, window);
  if (split < 0) return;
  const int t_begin = split * split_tokens;
  if (t_begin >= seq_len) return;  // the combine pass never reads this split
  const int t_end = min(seq_len, t_begin + split_tokens);
  const int t_lo = window > 0 ? max(0, seq_len - window) : 0;
  if (t_end <= t_lo) return;       // nor this one (wholly before the window)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int ps_mask = (1 << log2_ps) - 1;
  const int row_bytes_g = num_kv_heads * D * 2;  // token stride in the pools, bytes
  const int32_t* const bt = block_table + (size_t)b * max_pages;
  const int last_page = (seq_len - 1) >> log2_ps;
  char* const k_lds = lds[wave];
  char* const v_lds = lds[wave] + G::kTileBytes;

  // Q fragment (B operand of S^T = K Q^T): head h0 + lane%32, 8 bf16 per k-step
  bf16x8 qf[G::kDK];
  if (l32 < nh) {
    const uint16_t* src = q + ((size_t)b * num_q_heads + h0 + l32) * D + half * 8;
#pragma unroll
    for (int j = 0; j < G::kDK; ++j)
      qf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + j * 16));
  } else {
#pragma unroll
    for (int j = 0; j < G::kDK; ++j) qf[j] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }

  // Physical page of each 16-token group of the split, one group per lane, fetched with
  // one vector load: the tile loads then find their pages with v_readlane instead of
  // waiting for a scalar load of the table before each group.
  static_assert(kDecodeSplitTokensGrouped / 16 <= 64, "a split's groups fit in one wave");
  int group_page = 0;
  if (lane < (t_end - t_begin + 15) / 16)
    group_page = bt[min((t_begin + 16 * lane) >> log2_ps, last_page)];

  // Loads: instruction i fills tile rows kRowsPerInst*i + lane/chunks, slot lane%chunks.
  // The row's place in its 16-row group and its swizzle repeat every kInstPerGroup
  // instructions, so kInstPerGroup byte offsets per lane serve every load.
  int k_voff[G::kInstPerGroup], v_voff[G::kInstPerGroup];
#pragma unroll
  for (int i = 0; i < G::kInstPerGroup; ++i) {
    const int row = G::kRowsPerInst * i + lane / G::kChunks;  // < 16
    const int slot = lane % G::kChunks;
    k_voff[i] = row * row_bytes_g + hk * D * 2 + (slot ^ k_swizzle<D>(row)) * 16;
    v_voff[i] = row * row_bytes_g + hk * D * 2 + (slot ^ v_swizzle<D>(row)) * 16;
  }
  // K reads: row lane%32, chunk 2jj + half
  int k_rd[G::kDK];
#pragma unroll
  for (int jj = 0; jj < G::kDK; ++jj)
    k_rd[jj] = l32 * G::kRowBytes + ((2 * jj + half) ^ k_swizzle<D>(l32)) * 16;
  // V reads (transposing): 16-lane group g reads rows 4*half + (lane%16)/4 (+8) of a
  // 16-key chunk, d columns 32db + 16(g%2) + 4(lane%4) .. +3
  int v_rd[G::kDB];
  {
    const int j16 = lane & 15;
    const int g = lane >> 4;
    const int row = 4 * half + j16 / 4;
#pragma unroll
    for (int db = 0; db < G::kDB; ++db) {
      const int ch = 4 * db + 2 * (g & 1) + (j16 & 3) / 2;
      v_rd[db] = row * G::kRowBytes + (ch ^ v_swizzle<D>(row)) * 16 + 8 * (j16 & 1);
    }
  }

  float m_ref = -INFINITY;  // reference max (log2 units) of O and l
  float l_part = 0.f;       // this lane's share of the row sum (16 keys per tile)
  f32x16 oacc[G::kDB];
#pragma unroll
  for (int i = 0; i < G::kDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;

  // Streams the tile at key kt0 into this wave's region: two 16-row groups, one page
  // each.  The offsets go to the LDS-load builtin as plain scalars: given an array
  // element there, this compiler silently omits the kernel's host-side launch stub.
  auto issue_tile = [&](int kt0) {
#pragma unroll
    for (int i = 0; i < G::kInstPerTile; ++i) {
      const int first_row = G::kRowsPerInst * i;
      const int t0 = kt0 + (first_row & ~15);
      const int phys = __builtin_amdgcn_readlane(group_page, (t0 - t_begin) >> 4);
      const int valid = min(16, t_end - t0);
      const int bytes = valid > 0 ? valid * row_bytes_g : 0;
      const size_t elem =
          (((size_t)phys << log2_ps) + (t0 & ps_mask)) * (size_t)num_kv_heads * D;
      const int koff = k_voff[i % G::kInstPerGroup];
      const int voff = v_voff[i % G::kInstPerGroup];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(k_pool + elem, bytes),
                                               (lds_void*)(k_lds + first_row * G::kRowBytes),
                                               16, koff, 0, 0, kNonTemporal);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(v_pool + elem, bytes),
                                               (lds_void*)(v_lds + first_row * G::kRowBytes),
                                               16, voff, 0, 0, kNonTemporal);
    }
  };

  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  for (int tile = wave; tile < n_tiles; tile += kWaves) {
    const int kt0 = t_begin + tile * kTile;
    if (kt0 + kTile <= t_lo) continue;  // wholly before the window
    issue_tile(kt0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tile is in LDS
    __asm__ __volatile__("" ::: "memory");

    // S^T (keys x heads) = K Q^T
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
    for (int jj = 0; jj < G::kDK; ++jj) {
      const bf16x8 a =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(k_lds + k_rd[jj]));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[jj], sacc, 0, 0, 0);
    }

    // keys past the sequence end or before the window
    if (kt0 + kTile > t_end || kt0 < t_lo) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt0 + (r >> 2) * 8 + half * 4 + (r & 3);
        sacc[r] = (key < t_end && key >= t_lo) ? sacc[r] : -INFINITY;
      }
    }

    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = pair_max(mx) * scale_log2;  // every tile holds at least one visible key

    const bool raise = mx > m_ref + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? fast_exp2(m_ref - mx) : 1.f;
      m_ref = raise ? mx : m_ref;
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < G::kDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }

    // P = exp2(s * c - m_ref) rounded to bf16; the row sum adds the rounded values
    // (two per v_dot2 against (1, 1)).  Packed words stay scalars: building the dot2
    // operands from vector elements is miscompiled by this compiler.
    bf16x8 pb[2];
    float lsum0 = 0.f, lsum1 = 0.f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = fast_exp2(fmaf(sacc[c * 8 + 2 * e], scale_log2, -m_ref));
        const float x1 = fast_exp2(fmaf(sacc[c * 8 + 2 * e + 1], scale_log2, -m_ref));
        w[e] = pack_bf16x2(x0, x1);
      }
      lsum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[0]), ones, lsum0, false);
      lsum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[1]), ones, lsum1, false);
      lsum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[2]), ones, lsum0, false);
      lsum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[3]), ones, lsum1, false);
      pb[c] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
    }
    l_part += lsum0 + lsum1;

    // O^T (d x heads) += V^T P^T, one 16-key chunk at a time
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int db = 0; db < G::kDB; ++db) {
        const char* base = v_lds + c * 16 * G::kRowBytes + v_rd[db];
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base));
        const bf16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 8 * G::kRowBytes));
        const u32x2 wl = __builtin_bit_cast(u32x2, lo);
        const u32x2 wh = __builtin_bit_cast(u32x2, hi);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{wl[0], wl[1], wh[0], wh[1]});
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], oacc[db], 0, 0, 0);
      }
    }
    // every LDS read of this tile has returned before the next tile's loads overwrite it
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __asm__ __volatile__("" ::: "memory");
  }

  // ---- merge the 4 waves' partials and write the split's (m, l, O)
  const float l_row = pair_sum(l_part);
  __syncthreads();  // every wave is done with its tiles: regions become merge buffers
  float* const o_lds = reinterpret_cast<float*>(lds[wave]);  // [head][kOStride]
#pragma unroll
  for (int db = 0; db < G::kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = db * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
      o_lds[l32 * G::kOStride + d] = oacc[db][r];
    }
  if (half == 0) {
    sm_m[wave][l32] = m_ref;
    sm_l[wave][l32] = l_row;
  }
  __syncthreads();
  constexpr int kQuads = D / 4;
  for (int e = tid; e < nh * kQuads; e += kThreads) {
    const int hh = e / kQuads;
    const int d4 = e % kQuads;
    float big = sm_m[0][hh];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) big = fmaxf(big, sm_m[w][hh]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      // a wave without tiles has m = -inf, l = 0, O = 0 and weight exp2(-inf) = 0
      const float wt = fast_exp2(sm_m[w][hh] - big);
      const f32x4 o = *reinterpret_cast<const f32x4*>(
          reinterpret_cast<const float*>(lds[w]) + hh * G::kOStride + d4 * 4);
      acc += wt * o;
      lsum = fmaf(wt, sm_l[w][hh], lsum);
    }
    const size_t slot = ((size_t)b * num_q_heads + h0 + hh) * max_splits + split;
    *reinterpret_cast<f32x4*>(ws_o + slot * D + d4 * 4) = acc;
    if (d4 == 0) {
      ws_ml[slot * 2] = big;
      ws_ml[slot * 2 + 1] = lsum;
    }
  }
}

template <int D>
void launch_gqa(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int blocks_per_kv = (group + kHeadBlock - 1) / kHeadBlock;
  const dim3 grid(a.num_kv_heads * blocks_per_kv, decode_grid_splits(a), a.batch);
  hipLaunchKernelGGL(decode_gqa_kernel<D>, grid, dim3(kThreads), 0, stream, a.q, a.k_pool,
                     a.v_pool, a.block_table, a.seq_lens, a.ws_o, a.ws_ml,
                     score_scale_log2(a.scale), a.num_q_heads, a.num_kv_heads,
                     a.log2_page_size, a.max_pages_per_seq, a.split_tokens, a.max_splits,
                     a.window);
}

}  // namespace

hipError_t launch_decode_partial_gqa(const DecodeArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_gqa<128>(a, stream);
  else launch_gqa<64>(a, stream);
  return hipGetLastError();
}

}  // namespace pa
