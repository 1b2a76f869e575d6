// Internal launch interface between the C-ABI host layer (bsattn.cpp) and the
// kernels.  Every function launches asynchronously on `stream` and returns the
// launch status; arguments have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace bsattn {

// Paged K/V (block_table non-null): token t of (b, g) is row t % P of page
// block_table[b * max_pages + t / P] in pools [n_pages, Hkv, P, d], P = 1 << page_shift
// (16, 32 or 64 tokens).  Page numbers are clamped to [0, n_pages).
struct PagedKV {
  const int32_t* block_table;
  int32_t page_shift;
  int32_t max_pages;
  int32_t n_pages;
};

// Row of token t of (b, g) in its K or V pool (or the contiguous cache row).
__host__ __device__ inline size_t paged_row(const PagedKV& p, int b, int g, int n_kv_heads, int t) {
  int page = p.block_table[(size_t)b * p.max_pages + (t >> p.page_shift)];
  page = page < 0 ? 0 : (page >= p.n_pages ? p.n_pages - 1 : page);
  return (((size_t)page * n_kv_heads + g) << p.page_shift) + (t & ((1 << p.page_shift) - 1));
}

struct SummaryArgs {
  const void* K;
  void* mean;       // fp32, or bf16 when mean_bf16
  void* factor;        // fp32 rows [.., rank, e], or FP4 E2M1 codes [.., rank, e / 2] when factor_fp4
  float* factor_scale;  // FP4: one scale per factor row [.., rank]
  const float* basis;   // query-subspace rows [Hkv, sub_dim, d], or null
  int32_t sub_dim;      // e = sub_dim with a basis, else d
  int32_t bh;            // B * Hkv
  int32_t n_kv_heads;    // Hkv (the basis of pair bh is that of K/V head bh % Hkv)
  int32_t kv_capacity;   // token stride
  int32_t nblk_capacity;
  int32_t first_block;
  int32_t n_blocks;
  int32_t rank;
  int32_t head_dim;
  bool bf16;
  bool mean_bf16;  // store the block mean in bfloat16 (round to nearest even)
  bool factor_fp4;  // store factor rows as FP4 E2M1 codes with a float32 scale per row
  PagedKV paged;
};
hipError_t launch_summaries(const SummaryArgs& a, hipStream_t stream);

// One new token per (b, K/V head): rows K_new[bh], V_new[bh] -> K, V row `pos`.
struct AppendArgs {
  const void* K_new;
  const void* V_new;
  void* K;
  void* V;
  int32_t kv_capacity;
  int32_t pos;
  int32_t row_bytes;  // d * element size (a multiple of 16)
  int32_t n_kv_heads;
  PagedKV paged;
};
hipError_t launch_append(const AppendArgs& a, int n_pairs, hipStream_t stream);

struct SelectArgs {
  const void* Q;
  const void* mean;  // fp32, or bf16 when mean_bf16
  const void* factor;        // fp32 rows, or FP4 E2M1 codes when factor_fp4
  const float* factor_scale;  // FP4: one scale per factor row
  const float* basis;         // query-subspace rows [Hkv, sub_dim, d] (FP4 rows of sub_dim), or null
  int32_t sub_dim;
  int32_t* sel;
  float* scores;
  int32_t batch, n_q_heads, n_kv_heads, head_dim;
  int32_t n_blocks;       // complete blocks = n_ctx / 64
  int32_t nblk_capacity;
  int32_t rank;
  int32_t top_k;
  float scale;
  bool bf16;
  ForcedSet forced;
  // scoring split, set by the launcher: each wave scores `per_wave` units (of
  // 4 * PB blocks) of one pair; `n_part` waves per pair
  int32_t per_wave, n_part;
  bool scores_only;  // skip the top-k launch (the fused decode step selects)
  bool mean_bf16;    // the block means are bfloat16
  bool factor_fp4;   // the factor rows are FP4 E2M1 codes + row scales
  // block-sparse prefill (tile_rows > 0): Q is [B, Hq, seq_len, d]; scores and
  // sel hold one row per (b, K/V head, query tile of tile_rows rows); the
  // candidates of tile t are the complete blocks j with 64 j before the window
  // [i - window_left, i] of the tile's last row i, and not inside the sinks
  int32_t tile_rows, n_tiles, seq_len, window_left, n_sink;
  // exact block mass: the keys themselves [B, Hkv, kv_capacity, d] (BF16)
  const void* K;
  int32_t kv_capacity;
};
// Splits `units` per pair over the resident wave slots: as few units per wave
// as keeps every wave resident at once.
inline void split_units(SelectArgs& a, long long units, int slots) {
  const int n_pairs = a.batch * a.n_kv_heads;
  long long c = (n_pairs * units + slots - 1) / slots;
  if (c < 1) c = 1;
  while (c < units && (long long)n_pairs * ((units + c - 1) / c) > slots) ++c;
  a.per_wave = (int)c;
  a.n_part = (int)((units + c - 1) / c);
}
// The VALU scorer (fp32 queries, means or factor rows): scores only, the caller
// launches the top-k.  One object per (head dim, query dtype), select_valu.hip.
template <int D, bool BF16>
hipError_t launch_valu_scores(const SelectArgs& a, hipStream_t stream);
hipError_t launch_prefill_select(const SelectArgs& a, hipStream_t stream);
hipError_t launch_select_exact(const SelectArgs& a, hipStream_t stream);  // K, kv_capacity set
constexpr int kSparseTile = 128;      // query rows per selection tile (the prefill workgroup)
constexpr int kSparseMaxTopK = 256;   // selected blocks per tile
constexpr int kSparseMaxSink = 256;   // sink tokens of the block-sparse prefill
hipError_t launch_select_topk(const SelectArgs& a, hipStream_t stream);

// Forced blocks of a decode step, in the order the decode kernel visits them:
// two block ranges (sinks, window; merged when they touch) and the remaining
// blocks that hold a global token.
struct ForcedBlocks {
  int32_t r0_lo, r0_n;  // blocks [r0_lo, r0_lo + r0_n)
  int32_t r1_lo, r1_n;
  int32_t n_gblk;
  int32_t gblk[256];
};

// Fused decode step limits: 8 scores per lane in registers (with more blocks
// the in-wave selection costs more than the top-k launch it saves: measured at
// 2048 blocks, 32 scores per lane) and the selection table in the wave's V tile.
constexpr int kFusedMaxBlocks = 64 * 8;
constexpr int kFusedMaxTopK = 256;
// Workgroup-selected fused step: 8 scores per thread of a decode workgroup.
constexpr int kFusedWgMaxBlocks = 8 * 64 * 4;

struct DecodeArgs {
  const void* Q;
  const void* K;
  const void* V;
  const int32_t* sel;
  float* O;
  float* lse;
  float* part_o;      // [B*Hq, n_merge, d]  partial numerators
  float* part_ml;     // [B*Hq, n_merge, 2]  partial (max, normaliser), log2 domain
  int32_t batch, n_q_heads, n_kv_heads, head_dim;
  int32_t kv_capacity;
  int32_t top_k;
  int32_t n_items;        // top_k + forced blocks: a pair's item list (selected first)
  int32_t per_wave;       // fp32: items per wave
  int32_t fh_per_wave;    // bf16: forced half items per wave
  int32_t sh_per_wave;    // bf16: selected half items per wave
  int32_t n_part;         // bf16: waves per (b, K/V head), a multiple of kDecodeWaves; fp32: workgroups
  int32_t n_merge;        // partials per query head (workgroups per pair); merged when more than one
  // fused step (bf16): each wave selects its pair's top-k blocks itself from
  // the group scores instead of reading `sel`; the first wave of a pair writes
  // the selection to sel_out.  key_slots: scores per lane (0: not fused, 8:
  // each wave selects alone; -8: each workgroup selects together, 8 scores
  // per thread).
  const float* scores;
  int32_t nblk_capacity;
  int32_t* sel_out;
  int32_t key_slots;
  // scoring in the decode kernel (fused step, bfloat16 means, first order):
  // the means [B, Hkv, nblk_capacity, d]; the scores go to scores_out (may be
  // null).  Null mean: the scores come from `scores`.
  const void* mean;
  float* scores_out;
  uint64_t full_forced[kFusedMaxBlocks / 64];  // bit j % 64 of word j / 64: complete block j has no candidate token
  float scale;
  bool bf16;
  ForcedSet forced;
  ForcedBlocks fblocks;
  PagedKV paged;  // bf16 only
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Split geometry of the decode launch (also sizes the workspace).  bf16: at most
// `half_items` half items per wave and `n_part` waves per pair; fp32: one item
// per wave, `n_part` workgroups per pair.
void decode_split_geometry(int n_items, int n_pairs, int head_dim, bool bf16, int* half_items, int* n_part);
// The allocation-free decode step's scratch (split partials): a device array of
// this many bytes per device; *ptr = its address on the current device.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(void** ptr);
constexpr int kDecodeWaves = 4;  // waves per decode workgroup
// bf16 decode waves resident at once on 256 CUs: 4 per CU at d = 128, 8 at d = 64
constexpr int decode_slots(int head_dim) { return head_dim == 128 ? 1024 : 2048; }

constexpr float kDecodeHeadroom = 8.f;  // log2 units a running max may lag the true max

struct PrefillArgs {
  const void* Q;
  const void* K;
  const void* V;
  float* O;
  float* lse;
  int32_t batch, n_q_heads, n_kv_heads, head_dim;
  int32_t seq_len;
  int32_t kv_capacity;
  int32_t window_left;   // < 0: unbounded
  int32_t window_right;  // < 0: unbounded
  int32_t causal;
  float scale;
  int32_t n_global;
  int32_t gpos[256];
  // block-sparse prefill (sp_sel non-null): the tile's selected blocks
  // [B, Hkv, n_tiles, sp_top_k] and the first sp_n_sink keys join the causal band
  const int32_t* sp_sel;
  int32_t sp_top_k, sp_n_sink, sp_n_tiles;
  // global query rows: key range split over waves, partials in the workspace
  int32_t n_global_wg;        // workgroups (first in the grid) that run global rows
  int32_t g_splits;           // key ranges per global row
  int32_t g_keys_per_split;
  float* g_part_o;            // [B*Hq, ceil(n_global/32), g_splits, 32, d]
  float* g_part_ml;           // [B*Hq, ceil(n_global/32), g_splits, 32, 2] (max, normaliser), log2
  // dilated window (dil > 1): the launch covers the rows and keys of one residue
  // class, physical row dil_off + dil * x for logical row x < seq_len; the
  // windows are in logical rows; Q, O and lse hold seq_phys rows per (b, h)
  int32_t dil, dil_off, seq_phys;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Split geometry of the global query rows (also sizes the prefill workspace).
void prefill_global_geometry(int seq_len, int n_global, int batch, int n_q_heads, int* splits,
                             int* keys_per_split, int* n_wg);

// Gather probe (a measurement aid): loads-only gather of listed K/V blocks, one
// XOR of the loaded words per thread.  blocks [n_pairs, n_blocks] (entries
// clamped into the cache), checksum [n_pairs * wg_per_pair * 256].
struct ProbeArgs {
  const void* K;
  const void* V;
  const int32_t* blocks;
  uint32_t* checksum;
  int32_t n_pairs, n_blocks, kv_capacity, head_dim;
  int32_t wg_per_pair;  // 1 .. 16
  int32_t depth;        // half blocks in flight per wave, 1 .. 4
};
hipError_t launch_gather_probe(const ProbeArgs& a, hipStream_t stream);

}  // namespace bsattn
