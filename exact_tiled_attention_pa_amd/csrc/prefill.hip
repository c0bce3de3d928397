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
// Per key tile:
//   - the tile's physical pages come from the block table (at most 4 pages of 16);
//     each thread loads its 16-byte pieces of K and V rows into registers one tile
//     ahead (software pipelining), then writes them to LDS: K row-major, V
//     transposed (d-major) with key order permuted inside 16-key groups so the
//     PV MFMA operand of every lane is one 16-byte LDS read;
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16: Q stays in VGPRs for the whole
//     kernel as the B operand; each lane ends up holding 32 scores of one query
//     row (its query is lane % 32), so the row statistics are per lane plus one
//     exchange between lanes l and l ^ 32;
//   - masking only on tiles that cross the causal diagonal or the sequence end;
//     pool slots past the end are never loaded (V rows are zero, scores -inf), so
//     stale or NaN bytes in a partly filled last page cannot leak in;
//   - online softmax in fp32 with exp2 (scale * log2(e) folded into one FMA).  The
//     reference max is raised only when a row's max grows by more than 8 (log2
//     units); the output and row sum always share the same reference, so the
//     final O / l is unchanged while most tiles skip the rescale of O;
//   - P rounded to bf16 feeds O^T += V^T P^T, again 32x32x16 MFMA with fp32
//     accumulators; P never leaves registers.
// Epilogue: O / l, rounded to bf16 (RNE), staged through LDS and written with
// 16-byte coalesced stores.

#include "device_util.h"
#include "kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int BM = kPrefillBlockM;  // 128 query rows per workgroup
constexpr int BN = kPrefillBlockN;  // 64 key positions per tile
constexpr int kRescaleThreshold = 8;

template <int D>
struct PrefillSmem {
  static constexpr int kStrideK = D + 8;   // bf16 elements per K row (16 B pad)
  static constexpr int kStrideV = BN + 8;  // bf16 elements per transposed V row
  static constexpr int kKBytes = BN * kStrideK * 2;
  static constexpr int kVBytes = D * kStrideV * 2;
  static constexpr int kOBytes = BM * kStrideK * 2;  // epilogue staging
  static constexpr int kBytes = (kKBytes + kVBytes) > kOBytes ? (kKBytes + kVBytes) : kOBytes;
};

// position inside a 16-key group at which keys 4q .. 4q+3 are stored, so that
// lanes 0-31 find keys {0-3, 8-11} and lanes 32-63 keys {4-7, 12-15} in one
// 16-byte read: the key order of a 32x32x16 MFMA output column pair
__device__ __forceinline__ int vt_group_pos(int q) { return 4 * (((q & 1) << 1) | (q >> 1)); }

// physical page of the i-th page a key tile touches (i < 4: a 64-key tile spans at
// most four 16-token pages)
__device__ __forceinline__ int pick_page(int i, int p0, int p1, int p2, int p3) {
  const int a = (i & 1) ? p1 : p0;
  const int b = (i & 1) ? p3 : p2;
  return (i & 2) ? b : a;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
               const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ block_table,
               const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_start,
               uint16_t* __restrict__ out, float scale_log2, int num_q_heads,
               int num_kv_heads, int log2_ps, int max_pages) {
  using Smem = PrefillSmem<D>;
  constexpr int kChunksPerRow = D / 8;         // 16-byte pieces per K/V row
  constexpr int kKRowsPerPass = kThreads / kChunksPerRow;
  constexpr int kKLoads = BN / kKRowsPerPass;  // K pieces per thread
  constexpr int kVThreads = 16 * kChunksPerRow;  // threads that load V (4 keys x 8 d each)
  constexpr int kDK = D / 16;                  // MFMA k-steps over d
  constexpr int kDB = D / 32;                  // 32-wide output blocks over d

  __shared__ __attribute__((aligned(16))) char smem[Smem::kBytes];
  uint16_t* const ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* const vt = reinterpret_cast<uint16_t*>(smem + Smem::kKBytes);

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
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int hk = h / (num_q_heads / num_kv_heads);
  const int ps_mask = (1 << log2_ps) - 1;
  const size_t token_stride = (size_t)num_kv_heads * D;
  const int32_t* const bt = block_table + (size_t)b * max_pages;

  // key range of this workgroup and the first tile that needs a mask
  int kend = seq_len;
  int full_tiles = seq_len / BN;
  if (CAUSAL) {
    kend = min(seq_len, shift + min(q0 + BM, q_len));
    full_tiles = (shift + q0 + 1) / BN;
  }
  const int n_tiles = (kend + BN - 1) / BN;
  const int last_page = seq_len > 0 ? (seq_len - 1) >> log2_ps : 0;

  // ---- Q fragment (B operand of S^T = K Q^T): row q0 + 32w + lane%32, 8 bf16 per k-step
  bf16x8 qf[kDK];
  {
    const int r = q0 + wave * 32 + l32;
    if (r < q_len) {
      const uint16_t* src = q + ((size_t)(qs + r) * num_q_heads + h) * D + half * 8;
#pragma unroll
      for (int j = 0; j < kDK; ++j)
        qf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + j * 16));
    } else {
#pragma unroll
      for (int j = 0; j < kDK; ++j) qf[j] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  // ---- register staging of one K/V tile
  u32x4 kreg[kKLoads];
  u32x4 vreg[4];
  const int k_chunk = tid % kChunksPerRow;
  const int k_row0 = tid / kChunksPerRow;
  const int v_group = tid % 16;               // keys 4*v_group .. +3 of the tile
  const int v_chunk = tid / 16;               // d = 8*v_chunk .. +7
  const bool v_loader = tid < kVThreads;

  auto load_tile = [&](int j) {
    const int kt0 = j * BN;
    const int lp0 = kt0 >> log2_ps;
    // physical pages touched by this tile (at most 4 with 16-token pages), clamped to
    // the sequence's last page so no table entry past it is read
    const int p0 = bt[min(lp0, last_page)];
    const int p1 = bt[min(lp0 + 1, last_page)];
    const int p2 = bt[min(lp0 + 2, last_page)];
    const int p3 = bt[min(lp0 + 3, last_page)];
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int t = kt0 + k_row0 + i * kKRowsPerPass;
      if (t < seq_len) {
        const int phys = pick_page((t >> log2_ps) - lp0, p0, p1, p2, p3);
        const size_t off = (((size_t)phys << log2_ps) + (t & ps_mask)) * token_stride +
                           (size_t)hk * D + k_chunk * 8;
        kreg[i] = *reinterpret_cast<const u32x4*>(k_pool + off);
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (v_loader) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = kt0 + v_group * 4 + i;
        if (t < seq_len) {
          const int phys = pick_page((t >> log2_ps) - lp0, p0, p1, p2, p3);
          const size_t off = (((size_t)phys << log2_ps) + (t & ps_mask)) * token_stride +
                             (size_t)hk * D + v_chunk * 8;
          vreg[i] = *reinterpret_cast<const u32x4*>(v_pool + off);
        } else {
          vreg[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i)
      *reinterpret_cast<u32x4*>(ks + (k_row0 + i * kKRowsPerPass) * Smem::kStrideK +
                                k_chunk * 8) = kreg[i];
    if (v_loader) {
      const int col = (v_group >> 2) * 16 + vt_group_pos(v_group & 3);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // d = 8*v_chunk + 2w (low halves) and + 2w + 1 (high halves)
        const uint32_t lo01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x07060302u);
        const int d = v_chunk * 8 + 2 * w;
        *reinterpret_cast<u32x2*>(vt + d * Smem::kStrideV + col) = u32x2{lo01, lo23};
        *reinterpret_cast<u32x2*>(vt + (d + 1) * Smem::kStrideV + col) = u32x2{hi01, hi23};
      }
    }
  };

  // ---- per-lane softmax state for query row q0 + 32w + lane%32
  const int my_pos = shift + q0 + wave * 32 + l32;      // absolute position of this row
  const int wave_last_pos = shift + q0 + wave * 32 + 31;
  float m_ref = -INFINITY;  // reference max (log2 units) of O and l
  float l_part = 0.f;       // this lane's share of the row sum (its 32 keys per tile)
  f32x16 oacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;

  if (n_tiles > 0) load_tile(0);

  for (int j = 0; j < n_tiles; ++j) {
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (j + 1 < n_tiles) load_tile(j + 1);

    const int kt0 = j * BN;
    if (CAUSAL && kt0 > wave_last_pos) continue;  // whole tile in this wave's future

    // S^T (keys x queries) = K Q^T: two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      const uint16_t* krow = ks + (kb * 32 + l32) * Smem::kStrideK + half * 8;
#pragma unroll
      for (int jj = 0; jj < kDK; ++jj) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + jj * 16));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[jj], sacc[kb], 0, 0, 0);
      }
    }

    // mask: register r of block kb holds key kt0 + 32kb + 8(r/4) + 4*half + r%4
    if (j >= full_tiles) {
      const int lim = CAUSAL ? min(my_pos, seq_len - 1) : seq_len - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
          sacc[kb][r] = key <= lim ? sacc[kb][r] : -INFINITY;
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
      const float m_new = raise ? mx : m_ref;
      const float alpha = fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < kDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }

    // P = exp2(s * c - m_ref), bf16 for the MFMA, row-sum partial in fp32
    bf16x8 pb[4];
    float lsum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float x0 = fast_exp2(fmaf(sacc[c >> 1][(c & 1) * 8 + e], scale_log2, -m_ref));
        const float x1 = fast_exp2(fmaf(sacc[c >> 1][(c & 1) * 8 + e + 1], scale_log2, -m_ref));
        lsum += x0 + x1;
        pb[c][e] = (__bf16)x0;
        pb[c][e + 1] = (__bf16)x1;
      }
    }
    l_part += lsum;

    // O^T (d x queries) += V^T P^T
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const uint16_t* vrow = vt + (db * 32 + l32) * Smem::kStrideV + half * 8;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vrow + c * 16));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], oacc[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O / l -> bf16, staged through LDS for coalesced stores
  const float l_row = pair_sum(l_part);
  const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
  __syncthreads();
  uint16_t* const os = reinterpret_cast<uint16_t*>(smem) + wave * 32 * Smem::kStrideK;
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + half * 4;
      const uint32_t w0 = pack_bf16x2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
      const uint32_t w1 = pack_bf16x2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
      *reinterpret_cast<u32x2*>(os + l32 * Smem::kStrideK + d) = u32x2{w0, w1};
    }
  __syncthreads();
  constexpr int kPieces = 32 * kChunksPerRow;  // 16-byte pieces of this wave's rows
#pragma unroll
  for (int i = lane; i < kPieces; i += 64) {
    const int r = i / kChunksPerRow;
    const int cch = i % kChunksPerRow;
    const int qrow = q0 + wave * 32 + r;
    if (qrow < q_len) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(os + r * Smem::kStrideK + cch * 8);
      *reinterpret_cast<u32x4*>(out + ((size_t)(qs + qrow) * num_q_heads + h) * D + cch * 8) = v;
    }
  }
}

template <int D, bool CAUSAL>
void launch(const PrefillArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.max_q_len + BM - 1) / BM;
  const dim3 grid(a.num_q_heads, n_qtiles, a.batch);
  hipLaunchKernelGGL((prefill_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, stream, a.q,
                     a.k_pool, a.v_pool, a.block_table, a.seq_lens, a.q_start, a.out,
                     score_scale_log2(a.scale), a.num_q_heads, a.num_kv_heads, a.log2_page_size,
                     a.max_pages_per_seq);
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
