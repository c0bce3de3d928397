// Split-key paged prefill for gfx950: the same attention as prefill_kernel, laid out for
// launches too small to fill the chip, where latency rather than throughput counts.
//
// What it computes is unchanged: for each sequence, head and query row, softmax(scale *
// q K^T) V over the row's visible keys, K/V read in place through the block table ("What
// is Paged FlashAttention?", "How does it work?" steps 1-4 and "Practical example").
//
// Why a second layout.  prefill_kernel gives each workgroup 128 query rows and walks
// their key tiles one after another, so a launch's duration is at least its longest key
// loop: for the 600-token example of one head that is 5 workgroups on a chip of 256
// CUs, the last of them walking 10 tiles alone.  Here a workgroup holds only 32 query
// rows and its W waves share them (W = 8 at head_dim 64, 5 at 128: as many as the CU's
// LDS holds): wave w walks key tiles w, w + W, w + 2W, ... of the rows' visible range, each with its own online-softmax state (running max, running
// sum, unnormalised output; "Flash Attention: Fast, Memory-Efficient Attention for
// LLMs", "The Algorithm"), and at the end the W states are merged with the same
// rescaling algebra a split decode uses (states relative to maxima m_w combine as
// sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w with M = max_w m_w).  The key loop is
// 1/W as long, and the launch has four times as many workgroups.
//
// Per wave: one LDS stage of a K and a V tile (16 KB at head_dim 64, 32 KB at 128: 128
// and 160 KB per workgroup, one workgroup per CU), filled by buffer loads straight into LDS with rows past the
// sequence end reading as zero, waited for with the wave's own load counter (no
// workgroup barrier until the merge).  The tile arithmetic is prefill_kernel's: S^T = K
// Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, the transposing LDS read for V^T,
// exp2 softmax with a lazily raised reference max, P rounded to bf16 and the row sum
// taken from the rounded values.  Only tiles crossing the causal diagonal, the sequence
// end or a sliding window's lower edge pay for masks.

#include <climits>

#include "device_util.h"
#include "lds_tile.h"
#include "prefill_split.h"

namespace pa {
namespace {

constexpr int BM = kPrefillSplitBlockM;      // 32 query rows per workgroup
constexpr int BN = kPrefillBlockN;           // 64 key positions per tile
constexpr int kRescaleThreshold = 8;

template <int D>
struct SplitGeometry {
  static constexpr int kRowBytes = 2 * D;                 // one K or V row in LDS
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
  static constexpr int kRowsPerInst = 1024 / kRowBytes;   // rows per 1 KB load
  static constexpr int kInstPerTile = BN / kRowsPerInst;  // loads per K (or V) tile
  static constexpr int kInstPerGroup = 16 / kRowsPerInst; // loads per 16-row group
  static constexpr int kTileBytes = BN * kRowBytes;
  // waves sharing the rows: one stage of 2 * kTileBytes each, as many as the CU's 160 KB
  // of LDS holds (8 x 16 KB at d = 64; 5 x 32 KB at d = 128).  Against 4 waves with two
  // stages at d = 64: the 600-token example 6.5 -> 5.9 us, 33 rows over 9,000 keys 44 ->
  // 23 us; 300 rows over 3,000 keys at d = 128 24.2 -> 20.4 us
  static constexpr int kWaves = D == 64 ? 8 : 5;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kStages = 1;                       // LDS stages per wave
  static constexpr int kWaveBytes = kStages * 2 * kTileBytes;
  static constexpr int kDK = D / 16;                      // MFMA k-steps over d
  static constexpr int kDB = D / 32;                      // 32-wide output blocks
  static constexpr int kMergeRow = D + 4;                 // floats per merged state row
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(SplitGeometry<D>::kThreads)
prefill_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
                     const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ block_table,
                     const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_start,
                     uint16_t* __restrict__ out, float scale_log2, int num_q_heads,
                     int num_kv_heads, int log2_ps, int max_pages, int window) {
  using G = SplitGeometry<D>;
  static_assert(G::kWaves * G::kWaveBytes <= 160 * 1024, "LDS of one CU");
  static_assert(G::kWaves * BM * G::kMergeRow * 4 <= G::kWaves * G::kWaveBytes, "merge fits");
  __shared__ __attribute__((aligned(1024))) char lds[G::kWaves * G::kWaveBytes];

  const int h = blockIdx.x;
  const int b = blockIdx.z;
  const int qt = gridDim.y - 1 - blockIdx.y;  // heaviest causal tiles first
  const int qs = q_start[b];
  const int q_len = q_start[b + 1] - qs;
  const int q0 = qt * BM;
  if (q0 >= q_len) return;  // uniform over the workgroup, before any barrier
  const int seq_len = seq_lens[b];
  const int shift = seq_len - q_len;  // absolute position of local query row 0

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int hk = h / (num_q_heads / num_kv_heads);
  const int ps_mask = (1 << log2_ps) - 1;
  const int row_bytes_g = num_kv_heads * D * 2;  // token stride in the pools, bytes
  const int32_t* const bt = block_table + (size_t)b * max_pages;
  const int last_page = seq_len > 0 ? (seq_len - 1) >> log2_ps : 0;

  // key range of the workgroup's 32 rows and the tiles that need a mask
  int kend = seq_len;
  int full_tiles = seq_len / BN;
  if (CAUSAL) {
    kend = min(seq_len, shift + min(q0 + BM, q_len));
    full_tiles = (shift + q0 + 1) / BN;
  }
  const int n_tiles = (kend + BN - 1) / BN;
  int first_tile = 0;
  int window_masked_tiles = 0;
  if (CAUSAL && window > 0) {
    first_tile = max(0, shift + q0 - window + 1) / BN;
    window_masked_tiles = (max(0, shift + q0 + BM - window) + BN - 1) / BN;
  }

  // ---- Q fragment (B operand of S^T = K Q^T): row q0 + lane%32, the same in every wave
  bf16x8 qf[G::kDK];
  {
    const int r = q0 + l32;
    if (r < q_len) {
      const uint16_t* src = q + ((size_t)(qs + r) * num_q_heads + h) * D + half * 8;
#pragma unroll
      for (int j = 0; j < G::kDK; ++j)
        qf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + j * 16));
    } else {
#pragma unroll
      for (int j = 0; j < G::kDK; ++j) qf[j] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  // ---- per-lane constant offsets
  // Loads: instruction i of a tile fills LDS rows kRowsPerInst * i + lane / chunks, slot
  // lane % chunks; within its 16-row group that row is kRowsPerInst * (i % per-group) +
  // lane / chunks, so each per-group position r has its own source offset: the row inside
  // the group, this K/V head's columns, and the chunk that the row's swizzle puts in this
  // lane's slot.  They are kept as separate scalars and picked by the unrolled r: with an
  // array of them (or a call) as the load's offset operand the host pass of this compiler
  // drops the kernel's launch stub.
  auto voff_of = [&](int r, bool is_k) {
    const int row = G::kRowsPerInst * r + lane / G::kChunks;
    const int slot = lane % G::kChunks;
    const int swz = is_k ? k_swizzle<D>(row) : v_swizzle<D>(row);
    return row * row_bytes_g + hk * D * 2 + (slot ^ swz) * 16;
  };
  // at most 4 positions per group (head_dim 128), kept as separate scalars
  const int k_voff0 = voff_of(0, true), v_voff0 = voff_of(0, false);
  const int k_voff1 = voff_of(1, true), v_voff1 = voff_of(1, false);
  const int k_voff2 = G::kInstPerGroup > 2 ? voff_of(2, true) : 0;
  const int v_voff2 = G::kInstPerGroup > 2 ? voff_of(2, false) : 0;
  const int k_voff3 = G::kInstPerGroup > 3 ? voff_of(3, true) : 0;
  const int v_voff3 = G::kInstPerGroup > 3 ? voff_of(3, false) : 0;
  static_assert(G::kInstPerGroup == 2 || G::kInstPerGroup == 4, "2 or 4 loads per group");
  // K reads: row 32kb + lane%32, chunk 2jj + half
  int k_rd[G::kDK];
#pragma unroll
  for (int jj = 0; jj < G::kDK; ++jj)
    k_rd[jj] = l32 * G::kRowBytes + ((2 * jj + half) ^ k_swizzle<D>(l32)) * 16;
  // V reads (transposing): 16-lane group g reads rows 4*half + 8t + (lane%16)/4 of each
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

  char* const my_lds = lds + wave * G::kWaveBytes;
  auto k_stage = [&](int s) { return my_lds + s * 2 * G::kTileBytes; };
  auto v_stage = [&](int s) { return my_lds + s * 2 * G::kTileBytes + G::kTileBytes; };

  // Physical pages of a tile's four 16-key groups, fetched one tile of this wave ahead of
  // the loads that use them, so that each issue does not wait for its scalar loads.
  int tbl[BN / 16];
  auto fetch_table = [&](int j) {
#pragma unroll
    for (int g = 0; g < BN / 16; ++g) tbl[g] = bt[min((j * BN + 16 * g) >> log2_ps, last_page)];
  };
  // Streams key tile j (64 keys from position 64j; its pages in tbl) of K and V into
  // stage s of this wave: each 16-row group is one page's consecutive rows, one table
  // entry, a buffer resource sized to its rows below seq_len.
  auto issue_tile = [&](int j, int s) {
    const int kt0 = j * BN;
    char* const kd = k_stage(s);
    char* const vd = v_stage(s);
#pragma unroll
    for (int g = 0; g < BN / 16; ++g) {
      const int t0 = kt0 + 16 * g;
      const int phys = tbl[g];
      const int valid = min(16, seq_len - t0);
      const int bytes = valid > 0 ? valid * row_bytes_g : 0;
      const size_t elem =
          (((size_t)phys << log2_ps) + (t0 & ps_mask)) * (size_t)num_kv_heads * D;
#pragma unroll
      for (int r = 0; r < G::kInstPerGroup; ++r) {
        const int i = g * G::kInstPerGroup + r;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(k_pool + elem, bytes),
                                                 (lds_void*)(kd + i * 1024), 16,
                                                 r == 0 ? k_voff0 : r == 1 ? k_voff1
                                                 : r == 2 ? k_voff2 : k_voff3, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(v_pool + elem, bytes),
                                                 (lds_void*)(vd + i * 1024), 16,
                                                 r == 0 ? v_voff0 : r == 1 ? v_voff1
                                                 : r == 2 ? v_voff2 : v_voff3, 0, 0, 0);
      }
    }
  };

  // ---- per-lane softmax state for query row q0 + lane%32
  const int my_pos = shift + q0 + l32;
  const int my_lo = (CAUSAL && window > 0) ? my_pos - window + 1 : INT_MIN;
  float m_ref = -INFINITY;  // reference max (log2 units) of O and l
  float l_part = 0.f;       // this lane's share of the row sum
  f32x16 oacc[G::kDB];
#pragma unroll
  for (int i = 0; i < G::kDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;

  f32x16 sacc[2];
  bf16x8 vfr[4][G::kDB];
  // V^T fragments of the whole tile and the S^T MFMAs (two 32-key blocks alternating)
  auto scores = [&](const char* k_src, const char* v_src) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int db = 0; db < G::kDB; ++db) {
        const char* base = v_src + c * 16 * G::kRowBytes + v_rd[db];
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base));
        const bf16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 8 * G::kRowBytes));
        // whole-vector bit casts, as in prefill_kernel
        const u32x2 wl = __builtin_bit_cast(u32x2, lo);
        const u32x2 wh = __builtin_bit_cast(u32x2, hi);
        vfr[c][db] = __builtin_bit_cast(bf16x8, u32x4{wl[0], wl[1], wh[0], wh[1]});
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int jj = 0; jj < G::kDK; ++jj)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(k_src + kb * 32 * G::kRowBytes + k_rd[jj]));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[jj], sacc[kb], 0, 0, 0);
      }
  };
  // masks, online softmax and O^T += V^T P^T for key tile j
  auto finish_tile = [&](int j) {
    const int kt0 = j * BN;
    // register r of block kb holds key kt0 + 4*half + 32kb + 8(r/4) + r%4
    if (j >= full_tiles) {
      const int lim = CAUSAL ? min(my_pos, seq_len - 1) : seq_len - 1;
      const int hi = lim - kt0 - half * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
          sacc[kb][r] = c <= hi ? sacc[kb][r] : -INFINITY;
        }
    }
    if (j < window_masked_tiles) {
      const int lo = my_lo - kt0 - half * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
          sacc[kb][r] = c >= lo ? sacc[kb][r] : -INFINITY;
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
    mx = pair_max(mx) * scale_log2;

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
    // a row that has seen only masked keys keeps weights exp2(-inf) = 0
    const float m_sub = m_ref == -INFINITY ? 0.f : m_ref;

    bf16x8 pb[4];
    float lsum0 = 0.f, lsum1 = 0.f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = fast_exp2(fmaf(sacc[c >> 1][(c & 1) * 8 + 2 * e], scale_log2, -m_sub));
        const float x1 =
            fast_exp2(fmaf(sacc[c >> 1][(c & 1) * 8 + 2 * e + 1], scale_log2, -m_sub));
        w[e] = pack_bf16x2(x0, x1);
      }
      lsum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[0]), ones, lsum0, false);
      lsum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[1]), ones, lsum1, false);
      lsum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[2]), ones, lsum0, false);
      lsum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[3]), ones, lsum1, false);
      pb[c] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
    }
    l_part += lsum0 + lsum1;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int db = 0; db < G::kDB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[c][db], pb[c], oacc[db], 0, 0, 0);
  };

  // ---- this wave's key tiles: first_tile + wave, + G::kWaves, ... below n_tiles
  const int j0 = first_tile + wave;
  const int count = j0 < n_tiles ? (n_tiles - j0 + G::kWaves - 1) / G::kWaves : 0;
  constexpr int kLoadsPerTile = 2 * G::kInstPerTile;
  static_assert(kLoadsPerTile <= 63, "a tile's loads fit the load counter");
  if (count > 0) {
    fetch_table(j0);
    issue_tile(j0, 0);
    if (count > 1) fetch_table(j0 + G::kWaves);
  }
  for (int it = 0; it < count; ++it) {
    const int j = j0 + it * G::kWaves;
    const int s = it % G::kStages;
    const bool more = it + 1 < count;
    if constexpr (G::kStages == 2) {
      // the other stage was last read by the previous tile; its reads have returned
      // (their values fed that tile's MFMAs), and the wait makes that explicit (it also
      // covers the table entries fetched a tile ago)
      if (more) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __asm__ __volatile__("" ::: "memory");
        issue_tile(j + G::kWaves, 1 - s);
        if (it + 2 < count) fetch_table(j + 2 * G::kWaves);
      }
      if (more) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerTile));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    scores(k_stage(s), v_stage(s));
    if constexpr (G::kStages == 1) {
      if (more) {
        // one stage: every LDS read of this tile must have returned before the next
        // tile's loads overwrite it
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __asm__ __volatile__("" ::: "memory");
        issue_tile(j + G::kWaves, 0);
        if (it + 2 < count) fetch_table(j + 2 * G::kWaves);
      }
    }
    finish_tile(j);
  }

  // ---- merge the waves' states: O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w
  const float l_row = pair_sum(l_part);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();  // every wave is done with its stages
  float* const st = reinterpret_cast<float*>(lds);  // [wave][row][kMergeRow]: O, then m, l
  {
    float* const my = st + (wave * BM + l32) * G::kMergeRow;
#pragma unroll
    for (int db = 0; db < G::kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + half * 4;
        *reinterpret_cast<f32x4*>(my + d) =
            f32x4{oacc[db][g * 4 + 0], oacc[db][g * 4 + 1], oacc[db][g * 4 + 2],
                  oacc[db][g * 4 + 3]};
      }
    if (half == 0) {
      my[D] = m_ref;
      my[D + 1] = l_row;
    }
  }
  __syncthreads();
  constexpr int kPieces = BM * G::kChunks;  // 16-byte output pieces of the 32 rows
#pragma unroll
  for (int p = tid; p < kPieces; p += G::kThreads) {
    const int r = p / G::kChunks;
    const int c = p % G::kChunks;
    const int qrow = q0 + r;
    if (qrow >= q_len) continue;
    float mw[G::kWaves];
    float mmax = -INFINITY;
#pragma unroll
    for (int w = 0; w < G::kWaves; ++w) {
      mw[w] = st[(w * BM + r) * G::kMergeRow + D];
      mmax = fmaxf(mmax, mw[w]);
    }
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < G::kWaves; ++w) {
      // a wave that saw no visible key of this row holds O = 0, l = 0 and m = -inf
      const float a = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - mmax);
      const float* src = st + (w * BM + r) * G::kMergeRow;
      l = fmaf(a, src[D + 1], l);
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + c * 8);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + c * 8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = fmaf(a, x0[e], o[e]);
        o[4 + e] = fmaf(a, x1[e], o[4 + e]);
      }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const u32x4 v = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                     pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
    *reinterpret_cast<u32x4*>(out + ((size_t)(qs + qrow) * num_q_heads + h) * D + c * 8) = v;
  }
}

template <int D, bool CAUSAL>
void launch(const PrefillArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.max_q_len + BM - 1) / BM;
  const dim3 grid(a.num_q_heads, n_qtiles, a.batch);
  hipLaunchKernelGGL((prefill_split_kernel<D, CAUSAL>), grid, dim3(SplitGeometry<D>::kThreads), 0, stream, a.q,
                     a.k_pool, a.v_pool, a.block_table, a.seq_lens, a.q_start, a.out,
                     score_scale_log2(a.scale), a.num_q_heads, a.num_kv_heads,
                     a.log2_page_size, a.max_pages_per_seq, a.window);
}

}  // namespace

hipError_t launch_prefill_split(const PrefillArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) {
    if (a.causal) launch<128, true>(a, stream);
    else launch<128, false>(a, stream);
  } else {
    if (a.causal) launch<64, true>(a, stream);
    else launch<64, false>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace pa
