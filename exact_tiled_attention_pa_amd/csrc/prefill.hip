// Paged prefill attention for gfx950 with bf16 MFMA.
//
// What it computes: for each sequence, head and query row, softmax(scale * q K^T) V
// over the row's visible keys, K/V read in place from the paged pools through the
// block table ("What is Paged FlashAttention?", "How does it work?" steps 1-4 and
// "Practical example").  The score and probability tiles live only in registers
// ("Flash Attention: Fast, Memory-Efficient Attention for LLMs", "The Algorithm":
// running row max and row sum, output rescaled per tile, one final division).
//
// Work decomposition (the FlashAttention-2 split of that page's "Flash Attention 2"
// section, re-shaped for 64-wide waves and MFMA):
//   grid  (query head, query tile, sequence); the query-tile index is reversed so
//         the causally heaviest tiles are dispatched first, and consecutive
//         workgroups differ in head, which round-robins heads over the 8 XCDs so
//         each XCD's L2 holds the K/V of its own heads.
//   block 4 waves; wave w owns 32 query rows; the workgroup walks key tiles of 64
//         positions, skipping tiles entirely in the causal future (same section:
//         masked future tokens are skipped).
//
// K/V tile staging (no VGPR round trip, no per-element address arithmetic):
//   - a 64-key tile is 4 groups of 16 keys; a group never straddles a page (pages
//     hold a power of two >= 16 tokens), so its physical page is one scalar
//     block-table load and its address one scalar base; with pages of 64 tokens or
//     more the whole tile lies in one page, so each wave reads one table entry per
//     tile and derives its groups' bases from that page's address by a scalar add
//     (a separate instantiation: half the scalar work of the tile issue);
//   - each wave issues buffer loads straight into LDS (16 B per lane, 1 KB per
//     instruction) against a buffer resource whose base is the group's first row
//     and whose size covers only the rows below the sequence length: rows past
//     the end read as zero, so stale or NaN bytes in a partly filled last page
//     never reach the MFMAs;
//   - LDS keeps the natural [key][d] layout with the 16-byte chunks of each row
//     XOR-swizzled by the row index, so the K reads (ds_read_b128) and the
//     transposing V reads (ds_read_b64_tr_b16) are free of bank conflicts;
//   - two LDS stages: tile j+1 streams in while tile j is computed; one barrier
//     per tile.  The loads of tile j+1 are issued after tile j's S^T MFMAs, so the
//     scalar work of the issue runs while those MFMAs execute;
//   - the block-table entries of tile j+1 are fetched during tile j-1 and waited for
//     right after tile j's barrier, when no LDS read is outstanding: scalar loads and
//     LDS reads share one completion counter, so a table wait placed after the tile's
//     LDS reads would also hold the softmax until the V^T reads had returned.
//
// Per key tile (per wave, 32 query rows):
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16: Q stays in VGPRs for the whole
//     kernel as the B operand; each lane ends up holding 32 scores of one query
//     row (its query is lane % 32), so row statistics are per lane plus one
//     exchange between lanes l and l ^ 32;
//   - masking only on tiles that cross the causal diagonal, the sequence end or the
//     lower edge of a sliding window (keys p - w + 1 .. p for a row at position p;
//     "What do FlashAttention and PagedAttention actually optimize?", "Sort
//     techniques into the two bins"); tiles wholly below a window are skipped;
//   - online softmax in fp32 with exp2 (scale * log2(e) folded into one FMA).  The
//     reference max is raised only when a row's max grows by more than 8 (log2
//     units); the output and row sum always share the same reference, so the
//     final O / l is unchanged while most tiles skip the rescale of O;
//   - P rounded to bf16 feeds O^T += V^T P^T, again 32x32x16 MFMA with fp32
//     accumulators; V^T fragments come from the transposing LDS read, whose
//     4-key x 16-d block per 16 lanes matches the MFMA operand layout, with the
//     key order of the S^T accumulator registers.  All of a tile's V^T fragments
//     are read at the start of the tile, so those reads overlap S and the softmax.
// Epilogue: O / l, rounded to bf16 (RNE), staged through LDS and written with
// 16-byte coalesced stores.

#include <climits>

#include "device_util.h"
#include "kernels.h"
#include "lds_tile.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int BM = kPrefillBlockM;  // 128 query rows per workgroup
constexpr int BN = kPrefillBlockN;  // 64 key positions per tile
constexpr int kRescaleThreshold = 8;

template <int D>
struct Geometry {
  static constexpr int kRowBytes = 2 * D;                  // one K or V row in LDS
  static constexpr int kChunks = D / 8;                    // 16-byte chunks per row
  static constexpr int kRowsPerInst = 1024 / kRowBytes;    // rows per 1 KB load
  static constexpr int kInstPerWave = BN / kRowsPerInst / kWaves;
  static constexpr int kTileBytes = BN * kRowBytes;
  static constexpr int kDK = D / 16;                       // MFMA k-steps over d
  static constexpr int kDB = D / 32;                       // 32-wide output blocks
  static constexpr int kStageOut = D + 8;                  // epilogue row stride (elements)
};

// LARGE_PAGES: page_size >= BN, so a key tile never straddles a page.
template <int D, bool CAUSAL, bool LARGE_PAGES>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
               const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ block_table,
               const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_start,
               uint16_t* __restrict__ out, float scale_log2, int num_q_heads,
               int num_kv_heads, int log2_ps, int max_pages, int window) {
  using G = Geometry<D>;
  __shared__ __attribute__((aligned(1024))) char k_lds0[G::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_lds1[G::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds0[G::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds1[G::kTileBytes];

  const int h = blockIdx.x;
  const int b = blockIdx.z;
  const int qt = gridDim.y - 1 - blockIdx.y;
  const int qs = q_start[b];
  const int q_len = q_start[b + 1] - qs;
  const int q0 = qt * BM;
  if (q0 >= q_len) return;
  const int seq_len = seq_lens[b];
  const int shift = seq_len - q_len;  // absolute position of local query row 0

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int hk = h / (num_q_heads / num_kv_heads);
  const int ps_mask = (1 << log2_ps) - 1;
  const int row_bytes_g = num_kv_heads * D * 2;  // token stride in the pools, bytes
  const int32_t* const bt = block_table + (size_t)b * max_pages;

  // key range of this workgroup and the tiles that need a mask
  int kend = seq_len;
  int full_tiles = seq_len / BN;
  if (CAUSAL) {
    kend = min(seq_len, shift + min(q0 + BM, q_len));
    full_tiles = (shift + q0 + 1) / BN;
  }
  const int n_tiles = (kend + BN - 1) / BN;
  // sliding window (causal only): row at position p sees keys >= p - window + 1.  The
  // first row's bound gives the first tile; tiles below the last row's bound need masks
  int first_tile = 0;
  int window_masked_tiles = 0;
  if (CAUSAL && window > 0) {
    first_tile = max(0, shift + q0 - window + 1) / BN;
    window_masked_tiles = (max(0, shift + q0 + BM - window) + BN - 1) / BN;
  }
  const int last_page = seq_len > 0 ? (seq_len - 1) >> log2_ps : 0;

  // ---- Q fragment (B operand of S^T = K Q^T): row q0 + 32w + lane%32, 8 bf16 per k-step
  bf16x8 qf[G::kDK];
  {
    const int r = q0 + wave * 32 + l32;
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
  // Loads: instruction i of wave w fills LDS rows kRowsPerInst*(4i + w) + lane/chunks,
  // slot lane%chunks.  Those rows sit at the same offset inside their 16-row group for
  // every i, and have the same swizzle, so one byte offset per lane serves all loads.
  const int ld_row0 = G::kRowsPerInst * wave + lane / G::kChunks;  // row for i = 0
  const int ld_row_in_group = ld_row0 & 15;
  const int ld_slot = lane % G::kChunks;
  const int k_voff = ld_row_in_group * row_bytes_g + hk * D * 2 +
                     (ld_slot ^ k_swizzle<D>(ld_row0)) * 16;
  const int v_voff = ld_row_in_group * row_bytes_g + hk * D * 2 +
                     (ld_slot ^ v_swizzle<D>(ld_row0)) * 16;
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

  // Physical pages of this wave's loads of one tile (with large pages, the tile's one
  // page), fetched one tile ahead of their use so that the scalar loads' wait never
  // lands among outstanding LDS reads.
  constexpr int kTablePerTile = LARGE_PAGES ? 1 : G::kInstPerWave;
  int tbl[kTablePerTile];
#pragma unroll
  for (int i = 0; i < kTablePerTile; ++i) tbl[i] = 0;
  auto fetch_table = [&](int j) {
#pragma unroll
    for (int i = 0; i < kTablePerTile; ++i) {
      const int first_row = G::kRowsPerInst * (kWaves * i + wave);
      const int t0 = j * BN + (LARGE_PAGES ? 0 : (first_row & ~15));
      tbl[i] = bt[min(t0 >> log2_ps, last_page)];
    }
  };
  auto table_ready = [&]() {
#pragma unroll
    for (int i = 0; i < kTablePerTile; ++i) __asm__ __volatile__("" ::"s"(tbl[i]));
  };
  // Streams tile j (64 keys from position 64j) of K and V into one LDS stage.
  auto issue_tile = [&](int j, char* k_dst, char* v_dst) {
    const int kt0 = j * BN;
    if constexpr (LARGE_PAGES) {
      // the tile's 64 rows are consecutive rows of one page: one 64-bit page address,
      // then each 16-row group's base and size (its rows below seq_len) by scalar adds
      const int valid = min(BN, seq_len - kt0);
      const size_t elem =
          (((size_t)tbl[0] << log2_ps) + (kt0 & ps_mask)) * (size_t)num_kv_heads * D;
      const char* const kb = reinterpret_cast<const char*>(k_pool + elem);
      const char* const vb = reinterpret_cast<const char*>(v_pool + elem);
#pragma unroll
      for (int i = 0; i < G::kInstPerWave; ++i) {
        const int first_row = G::kRowsPerInst * (kWaves * i + wave);
        const int g = first_row & ~15;  // first row of the group inside the tile
        const int rows = min(16, valid - g);
        const int bytes = rows > 0 ? rows * row_bytes_g : 0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(kb + g * row_bytes_g, bytes),
                                                 (lds_void*)(k_dst + first_row * G::kRowBytes),
                                                 16, k_voff, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(vb + g * row_bytes_g, bytes),
                                                 (lds_void*)(v_dst + first_row * G::kRowBytes),
                                                 16, v_voff, 0, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < G::kInstPerWave; ++i) {
      const int first_row = G::kRowsPerInst * (kWaves * i + wave);
      const int t0 = kt0 + (first_row & ~15);       // first token of the 16-row group
      const int phys = tbl[i];
      const int valid = min(16, seq_len - t0);      // rows of the group below seq_len
      const int bytes = valid > 0 ? valid * row_bytes_g : 0;
      const size_t elem =
          (((size_t)phys << log2_ps) + (t0 & ps_mask)) * (size_t)num_kv_heads * D;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(k_pool + elem, bytes),
                                               (lds_void*)(k_dst + first_row * G::kRowBytes),
                                               16, k_voff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(v_pool + elem, bytes),
                                               (lds_void*)(v_dst + first_row * G::kRowBytes),
                                               16, v_voff, 0, 0, 0);
    }
  };

  // ---- per-lane softmax state for query row q0 + 32w + lane%32
  const int my_pos = shift + q0 + wave * 32 + l32;  // absolute position of this row
  const int wave_last_pos = shift + q0 + wave * 32 + 31;
  const int my_lo = (CAUSAL && window > 0) ? my_pos - window + 1 : INT_MIN;  // lowest key seen
  const int wave_lo = (CAUSAL && window > 0) ? shift + q0 + wave * 32 - window + 1 : INT_MIN;
  float m_ref = -INFINITY;  // reference max (log2 units) of O and l
  float l_part = 0.f;       // this lane's share of the row sum (its 32 keys per tile)
  f32x16 oacc[G::kDB];
#pragma unroll
  for (int i = 0; i < G::kDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;

  // A tile is computed in two parts: scores() issues the LDS reads of V^T and K and the
  // S^T MFMAs, finish_tile() does the masking, the softmax and P V.  The step issues
  // the next tile's loads in between, so their scalar address work overlaps the MFMAs.
  f32x16 sacc[2];
  bf16x8 vfr[4][G::kDB];
  auto scores = [&](int j, const char* k_src, const char* v_src) {
    // V^T fragments of the whole tile (64 VGPRs), read before the score MFMAs so that the
    // transposing LDS reads complete during S and the softmax instead of stalling P V
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int db = 0; db < G::kDB; ++db) {
        const char* base = v_src + c * 16 * G::kRowBytes + v_rd[db];
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base));
        const bf16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 8 * G::kRowBytes));
        // keep the whole-vector bit casts: element-wise access to these results is not
        // reliable with this compiler
        const u32x2 wl = __builtin_bit_cast(u32x2, lo);
        const u32x2 wh = __builtin_bit_cast(u32x2, hi);
        vfr[c][db] = __builtin_bit_cast(bf16x8, u32x4{wl[0], wl[1], wh[0], wh[1]});
      }

    // S^T (keys x queries) = K Q^T: two 32-key blocks whose MFMA chains alternate, so
    // each pair of K reads feeds two independent MFMAs
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
  auto finish_tile = [&](int j) {
    const int kt0 = j * BN;
    // mask: register r of block kb holds key kt0 + 4*half + c with the constant
    // c = 32kb + 8(r/4) + r%4 (0..59), so each bound is one compare of c against a
    // per-lane threshold: keys past the row's last visible key (tiles crossing the
    // diagonal or the sequence end), and keys before its window (tiles crossing the
    // window's lower edge)
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

    // row max over the tile (32 keys here, 32 in lane ^ 32)
    float mx = sacc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
    mx = pair_max(mx) * scale_log2;

    const bool raise = mx > m_ref + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      // lanes that do not raise keep their reference and scale by exactly 1 (their
      // reference may still be -inf when a window has not started for their row)
      const float alpha = raise ? fast_exp2(m_ref - mx) : 1.f;
      m_ref = raise ? mx : m_ref;
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < G::kDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }

    // a row whose window has not started yet has seen only masked keys: its weights
    // are exp2(-inf) = 0 whatever the reference, so use 0 instead of -inf - -inf
    const float m_sub = m_ref == -INFINITY ? 0.f : m_ref;

    // P = exp2(s * c - m_ref) rounded to bf16 for the MFMA; the row sum adds exactly
    // those rounded values (two per v_dot2 against (1, 1)), so the weights applied to V
    // sum to l.  The packed words are kept as scalars: building the dot2 operands from
    // vector elements is miscompiled by this compiler.
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

    // O^T (d x queries) += V^T P^T
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int db = 0; db < G::kDB; ++db) {
        oacc[db] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[c][db], pb[c], oacc[db], 0, 0, 0);
      }
    }
  };

  auto step = [&](int j, char* k_cur, char* v_cur, char* k_nxt, char* v_nxt) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile j landed
    __syncthreads();                     // everyone's loads landed; tile j-1 fully consumed
    table_ready();                       // tile j+1's pages (no LDS read outstanding here)
    // a tile wholly in this wave's causal future, or wholly before its window, is skipped
    const bool skip = CAUSAL && (j * BN > wave_last_pos || j * BN + BN - 1 < wave_lo);
    if (!skip) scores(j, k_cur, v_cur);
    if (j + 1 < n_tiles) issue_tile(j + 1, k_nxt, v_nxt);
    if (j + 2 < n_tiles) fetch_table(j + 2);
    if (skip) return;
    finish_tile(j);
  };

  if (first_tile < n_tiles) {
    fetch_table(first_tile);
    issue_tile(first_tile, k_lds0, v_lds0);
    if (first_tile + 1 < n_tiles) fetch_table(first_tile + 1);
  }
  for (int j = first_tile; j < n_tiles; j += 2) {
    step(j, k_lds0, v_lds0, k_lds1, v_lds1);
    if (j + 1 < n_tiles) step(j + 1, k_lds1, v_lds1, k_lds0, v_lds0);
  }

  // ---- epilogue: O / l -> bf16, staged through LDS for coalesced stores
  const float l_row = pair_sum(l_part);
  const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // one LDS stage buffer per wave holds that wave's 32 output rows
  static_assert(32 * G::kStageOut * 2 <= G::kTileBytes, "a wave's rows fit in one stage");
  char* const stage = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
  uint16_t* const os = reinterpret_cast<uint16_t*>(stage);
#pragma unroll
  for (int db = 0; db < G::kDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + half * 4;
      const uint32_t w0 = pack_bf16x2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
      const uint32_t w1 = pack_bf16x2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
      *reinterpret_cast<u32x2*>(os + l32 * G::kStageOut + d) = u32x2{w0, w1};
    }
  __syncthreads();
  constexpr int kPieces = 32 * G::kChunks;  // 16-byte pieces of this wave's rows
#pragma unroll
  for (int i = lane; i < kPieces; i += 64) {
    const int r = i / G::kChunks;
    const int cch = i % G::kChunks;
    const int qrow = q0 + wave * 32 + r;
    if (qrow < q_len) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(os + r * G::kStageOut + cch * 8);
      *reinterpret_cast<u32x4*>(out + ((size_t)(qs + qrow) * num_q_heads + h) * D + cch * 8) = v;
    }
  }
}

template <int D, bool CAUSAL, bool LARGE_PAGES>
void launch_pages(const PrefillArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.max_q_len + BM - 1) / BM;
  const dim3 grid(a.num_q_heads, n_qtiles, a.batch);
  hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, LARGE_PAGES>), grid, dim3(kThreads), 0, stream,
                     a.q, a.k_pool, a.v_pool, a.block_table, a.seq_lens, a.q_start, a.out,
                     score_scale_log2(a.scale), a.num_q_heads, a.num_kv_heads,
                     a.log2_page_size, a.max_pages_per_seq, a.window);
}

template <int D, bool CAUSAL>
void launch(const PrefillArgs& a, hipStream_t stream) {
  if ((1 << a.log2_page_size) >= BN) launch_pages<D, CAUSAL, true>(a, stream);
  else launch_pages<D, CAUSAL, false>(a, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
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
