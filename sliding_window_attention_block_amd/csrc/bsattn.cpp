// C-ABI entry points: host-side validation, the forced-token description of a
// decode step, workspace sizing, and kernel launches.  Every check runs before
// any launch; the library allocates nothing and keeps no state.
#include "../../include/bsattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "launch.hpp"

static_assert(bsattn::kMaxTopK == BSATTN_MAX_TOP_K, "device top-k limit matches the header");
static_assert(bsattn::kNoAllocScratchBytes == BSATTN_NOALLOC_SCRATCH_BYTES, "scratch size matches the header");
static_assert(bsattn::kMaxBlocks == BSATTN_MAX_BLOCKS, "device block limit matches the header");
static_assert(bsattn::kSparseTile == BSATTN_SPARSE_TILE && bsattn::kSparseMaxTopK == BSATTN_SPARSE_MAX_TOP_K &&
                  bsattn::kSparseMaxSink == BSATTN_SPARSE_MAX_SINK,
              "block-sparse prefill limits match the header");

namespace {

thread_local char g_err[512] = "";

bsattn_status fail(bsattn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

float effective_scale(const bsattn_shape* s) {
  return s->scale != 0.f ? s->scale : 1.0f / std::sqrt((float)s->head_dim);
}

bsattn_status check_shape(const bsattn_shape* s, bool decode) {
  if (s == nullptr) return fail(BSATTN_ERR_INVALID, "shape is NULL");
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1)
    return fail(BSATTN_ERR_INVALID, "batch and head counts must be >= 1");
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(BSATTN_ERR_INVALID, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                s->n_q_heads, s->n_kv_heads);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(BSATTN_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are built", s->head_dim);
  if (s->n_ctx < 1) return fail(BSATTN_ERR_INVALID, "n_ctx must be >= 1");
  if (s->kv_capacity < s->n_ctx) return fail(BSATTN_ERR_INVALID, "kv_capacity < n_ctx");
  if (s->block_size != 64) return fail(BSATTN_ERR_UNSUPPORTED, "block_size %d: only 64 is built", s->block_size);
  if (s->dtype != BSATTN_F32 && s->dtype != BSATTN_BF16) return fail(BSATTN_ERR_INVALID, "unknown dtype %d", s->dtype);
  if (!(s->scale >= 0.f) || !std::isfinite(s->scale)) return fail(BSATTN_ERR_INVALID, "scale must be finite and >= 0");
  if (decode && s->n_q_heads / s->n_kv_heads > BSATTN_MAX_GROUP)
    return fail(BSATTN_ERR_UNSUPPORTED, "query heads per K/V head must be <= %d", BSATTN_MAX_GROUP);
  if ((long long)s->batch * s->n_kv_heads > 65535)
    return fail(BSATTN_ERR_UNSUPPORTED, "batch * n_kv_heads must be <= 65535");
  return BSATTN_OK;
}

bsattn_status check_globals(const int32_t* gpos, int32_t n_global, int32_t n_ctx) {
  if (n_global < 0 || n_global > BSATTN_MAX_GLOBAL)
    return fail(BSATTN_ERR_INVALID, "n_global must be in [0, %d]", BSATTN_MAX_GLOBAL);
  if (n_global > 0 && gpos == nullptr) return fail(BSATTN_ERR_INVALID, "global_pos_host is NULL");
  for (int i = 0; i < n_global; ++i) {
    if (gpos[i] < 0 || gpos[i] >= n_ctx)
      return fail(BSATTN_ERR_INVALID, "global position %d out of [0, %d)", gpos[i], n_ctx);
    if (i > 0 && gpos[i] <= gpos[i - 1])
      return fail(BSATTN_ERR_INVALID, "global positions must be sorted and unique");
  }
  return BSATTN_OK;
}

bsattn::ForcedSet make_forced(int32_t n_ctx, int32_t window, int32_t n_sink, const int32_t* gpos,
                              int32_t n_global) {
  bsattn::ForcedSet f;
  std::memset(&f, 0, sizeof(f));
  f.n_ctx = n_ctx;
  f.sink_end = n_sink < 0 ? 0 : (n_sink > n_ctx ? n_ctx : n_sink);
  const long long t = n_ctx - 1;
  f.win_lo = window > 0 ? (int32_t)(t - window + 1 < 0 ? 0 : t - window + 1) : n_ctx;
  f.n_global = n_global;
  for (int i = 0; i < n_global; ++i) f.gpos[i] = gpos[i];
  return f;
}

// Forced blocks in visiting order: sink range, window range (merged when they
// touch), then blocks holding a global token outside both ranges.
bsattn::ForcedBlocks make_forced_blocks(const bsattn::ForcedSet& f) {
  bsattn::ForcedBlocks fb;
  std::memset(&fb, 0, sizeof(fb));
  const int S = bsattn::kBlock;
  int s_lo = 0, s_hi = (f.sink_end + S - 1) / S;  // [s_lo, s_hi)
  int w_lo = f.win_lo / S, w_hi = f.win_lo < f.n_ctx ? (f.n_ctx - 1) / S + 1 : w_lo;
  if (s_hi > s_lo && w_hi > w_lo && w_lo <= s_hi) {
    fb.r0_lo = 0;
    fb.r0_n = (w_hi > s_hi ? w_hi : s_hi);
  } else {
    if (s_hi > s_lo) { fb.r0_lo = s_lo; fb.r0_n = s_hi - s_lo; }
    if (w_hi > w_lo) {
      if (fb.r0_n == 0) { fb.r0_lo = w_lo; fb.r0_n = w_hi - w_lo; }
      else { fb.r1_lo = w_lo; fb.r1_n = w_hi - w_lo; }
    }
  }
  int last = -1;
  for (int i = 0; i < f.n_global; ++i) {
    const int blk = f.gpos[i] / S;
    const bool in0 = blk >= fb.r0_lo && blk < fb.r0_lo + fb.r0_n;
    const bool in1 = blk >= fb.r1_lo && blk < fb.r1_lo + fb.r1_n;
    if (in0 || in1 || blk == last) continue;
    fb.gblk[fb.n_gblk++] = blk;
    last = blk;
  }
  return fb;
}

// Forced blocks of the sink and window ranges (exact; global tokens add up to
// one block each on top).
int forced_range_blocks(int32_t n_ctx, int32_t window, int32_t n_sink) {
  bsattn::ForcedSet f = make_forced(n_ctx, window, n_sink, nullptr, 0);
  bsattn::ForcedBlocks fb = make_forced_blocks(f);
  return fb.r0_n + fb.r1_n;
}

// Decode launch plan for top_k selected and n_forced forced items per pair:
// n_part waves (bf16) or workgroups (fp32) per pair, n_merge partials per
// query head (one per workgroup; merged when more than one); bf16 waves take
// fh forced and sh selected half items each.
struct DecodePlan {
  int half_items, n_part, n_merge, fh, sh;
};
DecodePlan decode_plan(const bsattn_shape* s, int top_k, int n_forced) {
  DecodePlan p;
  bsattn::decode_split_geometry(top_k + n_forced, s->batch * s->n_kv_heads, s->head_dim,
                                s->dtype == BSATTN_BF16, &p.half_items, &p.n_part);
  p.n_merge = s->dtype == BSATTN_BF16 ? p.n_part / bsattn::kDecodeWaves : p.n_part;
  p.fh = (2 * n_forced + p.n_part - 1) / p.n_part;
  p.sh = (2 * top_k + p.n_part - 1) / p.n_part;
  return p;
}

// Workspace layout: partial numerators [B*Hq, n_merge, d] | partial (max, sum)
// [B*Hq, n_merge, 2], each region 256-byte aligned; nothing when n_merge == 1.
struct WsLayout {
  size_t o_off, ml_off, total;
};
WsLayout workspace_layout(const bsattn_shape* s, int n_merge) {
  const size_t rows = n_merge > 1 ? (size_t)s->batch * s->n_q_heads * n_merge : 0;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WsLayout l;
  l.o_off = 0;
  l.ml_off = up(rows * s->head_dim * sizeof(float));
  l.total = l.ml_off + up(rows * 2 * sizeof(float));
  return l;
}

// Workspace bytes that cover every forced-item count the arguments allow: the
// sink and window blocks plus 0 .. n_global blocks of global tokens (globals
// may share blocks or fall in the ranges, and the split geometry is not
// monotone in the item count).
size_t decode_workspace_bound(const bsattn_shape* s, int top_k, int window, int n_sink, int n_global) {
  const int base = forced_range_blocks(s->n_ctx, window, n_sink);
  size_t most = 0;
  for (int extra = 0; extra <= n_global; ++extra) {
    const size_t t = workspace_layout(s, decode_plan(s, top_k, base + extra).n_merge).total;
    if (t > most) most = t;
  }
  return most;
}

// Prefill workspace (global query rows only): partial numerators
// [B*Hq, ceil(n_global/32), splits, 32, d] | partial (max, sum) [..., 2], 256-byte aligned.
struct PrefillWs {
  int splits, keys_per_split, n_wg;
  size_t o_off, ml_off, total;
};
PrefillWs prefill_workspace_layout(const bsattn_shape* s, int n_global) {
  PrefillWs l;
  bsattn::prefill_global_geometry(s->n_ctx, n_global, s->batch, s->n_q_heads, &l.splits,
                                  &l.keys_per_split, &l.n_wg);
  const size_t rows = (size_t)s->batch * s->n_q_heads * ((n_global + 31) / 32) * l.splits * 32;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  l.o_off = 0;
  l.ml_off = up(rows * s->head_dim * sizeof(float));
  l.total = n_global > 0 ? l.ml_off + up(rows * 2 * sizeof(float)) : 0;
  return l;
}

// Validation of the selector's arguments (bsattn_select_topk, bsattn_decode_step).
bsattn_status check_factor(int32_t rank, const void* factor, int32_t factor_dtype, const float* factor_scale) {
  if (rank > 0 && factor == nullptr) return fail(BSATTN_ERR_INVALID, "factor is NULL with rank > 0");
  if (factor_dtype != BSATTN_F32 && factor_dtype != BSATTN_FP4_E2M1)
    return fail(BSATTN_ERR_INVALID, "factor_dtype %d: must be BSATTN_F32 or BSATTN_FP4_E2M1", factor_dtype);
  if (rank > 0 && factor_dtype == BSATTN_FP4_E2M1 &&
      (factor_scale == nullptr || (reinterpret_cast<uintptr_t>(factor_scale) & 3u) != 0))
    return fail(BSATTN_ERR_INVALID, "FP4 factors need a 4-byte aligned factor_scale");
  return BSATTN_OK;
}

// Paged K/V layout (NULL: contiguous).
bsattn_status paged_args(const bsattn_shape* s, const bsattn_paged_kv* p, bsattn::PagedKV& out) {
  std::memset(&out, 0, sizeof(out));
  if (p == nullptr) return BSATTN_OK;
  if (p->block_table == nullptr || (reinterpret_cast<uintptr_t>(p->block_table) & 3u) != 0)
    return fail(BSATTN_ERR_INVALID, "paged: block_table must be a non-NULL, 4-byte aligned device pointer");
  if (p->page_tokens != 16 && p->page_tokens != 32 && p->page_tokens != 64)
    return fail(BSATTN_ERR_INVALID, "paged: page_tokens %d must be 16, 32 or 64", p->page_tokens);
  if (p->max_pages < 1 || p->n_pages < 1) return fail(BSATTN_ERR_INVALID, "paged: max_pages and n_pages must be >= 1");
  if ((long long)p->max_pages * p->page_tokens != s->kv_capacity)
    return fail(BSATTN_ERR_INVALID, "paged: kv_capacity must equal max_pages * page_tokens");
  out.block_table = p->block_table;
  out.page_shift = p->page_tokens == 16 ? 4 : (p->page_tokens == 32 ? 5 : 6);
  out.max_pages = p->max_pages;
  out.n_pages = p->n_pages;
  return BSATTN_OK;
}

// Query-subspace basis: sub_dim 0 (none), or a multiple of 32 in [32, d] with rank >= 1.
bsattn_status check_basis(const float* basis, int32_t sub_dim, int32_t rank, int32_t head_dim) {
  if (sub_dim == 0) return BSATTN_OK;
  if (sub_dim < 32 || sub_dim > head_dim || sub_dim % 32 != 0)
    return fail(BSATTN_ERR_INVALID, "sub_dim %d: must be 0 or a multiple of 32 in [32, %d]", sub_dim, head_dim);
  if (rank < 1) return fail(BSATTN_ERR_INVALID, "a query-subspace basis needs rank >= 1");
  if (basis == nullptr || !aligned16(basis))
    return fail(BSATTN_ERR_INVALID, "basis must be a non-NULL, 16-byte aligned device pointer");
  return BSATTN_OK;
}

bsattn_status select_args(const bsattn_shape* shape, const void* Q, const void* mean, int32_t mean_dtype,
                          const void* factor, int32_t factor_dtype, const float* factor_scale,
                          const float* basis, int32_t sub_dim, int32_t rank, int32_t nblk_capacity, int32_t top_k, int32_t window, int32_t n_sink,
                          const int32_t* global_pos_host, int32_t n_global, int32_t* sel, float* scores,
                          bsattn::SelectArgs& a) {
  bsattn_status st = check_shape(shape, true);
  if (st != BSATTN_OK) return st;
  if (Q == nullptr || mean == nullptr || sel == nullptr || scores == nullptr)
    return fail(BSATTN_ERR_INVALID, "Q, mean, sel and scores must be non-NULL");
  if (mean_dtype != BSATTN_F32 && mean_dtype != BSATTN_BF16)
    return fail(BSATTN_ERR_INVALID, "mean_dtype %d: must be BSATTN_F32 or BSATTN_BF16", mean_dtype);
  if (rank < 0 || rank > BSATTN_MAX_RANK) return fail(BSATTN_ERR_INVALID, "rank must be in [0, %d]", BSATTN_MAX_RANK);
  st = check_factor(rank, factor, factor_dtype, factor_scale);
  if (st != BSATTN_OK) return st;
  st = check_basis(basis, sub_dim, rank, shape->head_dim);
  if (st != BSATTN_OK) return st;
  if (sub_dim > 0 && (shape->dtype != BSATTN_BF16 || mean_dtype != BSATTN_BF16 || factor_dtype != BSATTN_FP4_E2M1))
    return fail(BSATTN_ERR_UNSUPPORTED, "a query-subspace basis needs BF16 Q, BF16 means and FP4 factors");
  if (top_k < 1 || top_k > BSATTN_MAX_TOP_K) return fail(BSATTN_ERR_INVALID, "top_k must be in [1, %d]", BSATTN_MAX_TOP_K);
  if (window < 0 || n_sink < 0) return fail(BSATTN_ERR_INVALID, "window and n_sink must be >= 0");
  const int nb = shape->n_ctx / shape->block_size;
  if (nb > BSATTN_MAX_BLOCKS) return fail(BSATTN_ERR_UNSUPPORTED, "more than %d complete blocks", BSATTN_MAX_BLOCKS);
  if (nblk_capacity < nb) return fail(BSATTN_ERR_INVALID, "nblk_capacity < n_ctx / block_size");
  st = check_globals(global_pos_host, n_global, shape->n_ctx);
  if (st != BSATTN_OK) return st;
  if (!aligned16(Q) || !aligned16(mean) || (factor && !aligned16(factor)))
    return fail(BSATTN_ERR_INVALID, "device pointers must be 16-byte aligned");
  std::memset(&a, 0, sizeof(a));
  a.Q = Q; a.mean = mean; a.factor = rank > 0 ? factor : nullptr; a.sel = sel; a.scores = scores;
  a.factor_fp4 = rank > 0 && factor_dtype == BSATTN_FP4_E2M1;
  a.factor_scale = a.factor_fp4 ? factor_scale : nullptr;
  a.basis = sub_dim > 0 ? basis : nullptr;
  a.sub_dim = sub_dim;
  a.batch = shape->batch; a.n_q_heads = shape->n_q_heads; a.n_kv_heads = shape->n_kv_heads;
  a.head_dim = shape->head_dim;
  a.n_blocks = nb;
  a.nblk_capacity = nblk_capacity;
  a.rank = rank;
  a.top_k = top_k;
  a.scale = effective_scale(shape);
  a.bf16 = shape->dtype == BSATTN_BF16;
  a.mean_bf16 = mean_dtype == BSATTN_BF16;
  a.forced = make_forced(shape->n_ctx, window, n_sink, global_pos_host, n_global);
  return BSATTN_OK;
}

// Validation of the sparse decode's arguments and its launch plan (bsattn_decode,
// bsattn_decode_step); `sel` is read by the former, written by the latter.
bsattn_status decode_args(const bsattn_shape* shape, const void* Q, const void* K, const void* V,
                          const int32_t* sel, int32_t top_k, int32_t window, int32_t n_sink,
                          const int32_t* global_pos_host, int32_t n_global, float* O, float* lse,
                          void* workspace, size_t ws_bytes, const bsattn_paged_kv* paged,
                          bsattn::DecodeArgs& a) {
  bsattn_status st = check_shape(shape, true);
  if (st != BSATTN_OK) return st;
  bsattn::PagedKV pk;
  st = paged_args(shape, paged, pk);
  if (st != BSATTN_OK) return st;
  if (paged != nullptr && shape->dtype != BSATTN_BF16)
    return fail(BSATTN_ERR_UNSUPPORTED, "paged: the sparse decode reads paged caches in BF16 only");
  if (Q == nullptr || K == nullptr || V == nullptr || sel == nullptr || O == nullptr)
    return fail(BSATTN_ERR_INVALID, "Q, K, V, sel and O must be non-NULL");
  if (top_k < 1 || top_k > BSATTN_MAX_TOP_K) return fail(BSATTN_ERR_INVALID, "top_k must be in [1, %d]", BSATTN_MAX_TOP_K);
  if (window < 0 || n_sink < 0) return fail(BSATTN_ERR_INVALID, "window and n_sink must be >= 0");
  st = check_globals(global_pos_host, n_global, shape->n_ctx);
  if (st != BSATTN_OK) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
    return fail(BSATTN_ERR_INVALID, "device pointers must be 16-byte aligned");
  std::memset(&a, 0, sizeof(a));
  a.forced = make_forced(shape->n_ctx, window, n_sink, global_pos_host, n_global);
  a.fblocks = make_forced_blocks(a.forced);
  const int n_forced = a.fblocks.r0_n + a.fblocks.r1_n + a.fblocks.n_gblk;
  a.n_items = top_k + n_forced;
  const DecodePlan plan = decode_plan(shape, top_k, n_forced);
  const WsLayout lay = workspace_layout(shape, plan.n_merge);
  const size_t need = plan.n_merge > 1 ? lay.total : 0;
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(BSATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(BSATTN_ERR_INVALID, "workspace must be 256-byte aligned");
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.o_off);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.ml_off);
  a.per_wave = 1;
  a.fh_per_wave = plan.fh;
  a.sh_per_wave = plan.sh;
  a.n_part = plan.n_part;
  a.n_merge = plan.n_merge;
  a.Q = Q; a.K = K; a.V = V; a.sel = sel; a.O = O; a.lse = lse;
  a.batch = shape->batch; a.n_q_heads = shape->n_q_heads; a.n_kv_heads = shape->n_kv_heads;
  a.head_dim = shape->head_dim;
  a.kv_capacity = shape->kv_capacity;
  a.top_k = top_k;
  a.scale = effective_scale(shape);
  a.bf16 = shape->dtype == BSATTN_BF16;
  a.paged = pk;
  return BSATTN_OK;
}


}  // namespace

extern "C" {

const char* bsattn_status_string(bsattn_status st) {
  switch (st) {
    case BSATTN_OK: return "ok";
    case BSATTN_ERR_INVALID: return "invalid argument";
    case BSATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case BSATTN_ERR_HIP: return "HIP error";
    case BSATTN_ERR_WORKSPACE: return "workspace too small";
    default: break;
  }
  return "unknown status";
}

const char* bsattn_last_error(void) { return g_err; }

const char* bsattn_version(void) { return "bsattn 0.1.0 gfx950"; }

bsattn_status bsattn_probe_gather(const bsattn_shape* shape, const void* K, const void* V, const int32_t* blocks,
                                  int32_t n_blocks, int32_t wg_per_pair, int32_t depth, uint32_t* checksum,
                                  void* hip_stream) {
  g_err[0] = 0;
  bsattn_status st = check_shape(shape, true);
  if (st != BSATTN_OK) return st;
  if (shape->dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "the gather probe reads BF16 caches");
  if (K == nullptr || V == nullptr || blocks == nullptr || checksum == nullptr)
    return fail(BSATTN_ERR_INVALID, "K, V, blocks and checksum must be non-NULL");
  if (shape->kv_capacity < bsattn::kBlock) return fail(BSATTN_ERR_INVALID, "kv_capacity holds no block");
  if (n_blocks < 1 || n_blocks > bsattn::kMaxBlocks)
    return fail(BSATTN_ERR_INVALID, "n_blocks must be in [1, %d]", bsattn::kMaxBlocks);
  if (wg_per_pair < 1 || wg_per_pair > 16) return fail(BSATTN_ERR_INVALID, "wg_per_pair must be in [1, 16]");
  if (depth < 1 || depth > 4) return fail(BSATTN_ERR_INVALID, "depth must be in [1, 4]");
  bsattn::ProbeArgs a;
  a.K = K;
  a.V = V;
  a.blocks = blocks;
  a.checksum = checksum;
  a.n_pairs = shape->batch * shape->n_kv_heads;
  a.n_blocks = n_blocks;
  a.kv_capacity = shape->kv_capacity;
  a.head_dim = shape->head_dim;
  a.wg_per_pair = wg_per_pair;
  a.depth = depth;
  const hipError_t e = bsattn::launch_gather_probe(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "gather probe launch: %s", hipGetErrorString(e));
  return BSATTN_OK;
}

}  // extern "C"

namespace {

// Validation of the summaries' arguments (bsattn_build_summaries, bsattn_append_kv).
bsattn_status summaries_args(const bsattn_shape* shape, const void* K, int32_t rank, int32_t first_block,
                             int32_t n_blocks, int32_t nblk_capacity, void* mean, int32_t mean_dtype, void* factor,
                             int32_t factor_dtype, float* factor_scale, const float* basis, int32_t sub_dim,
                             const bsattn_paged_kv* paged, bsattn::SummaryArgs& a) {
  bsattn_status st = check_shape(shape, false);
  if (st != BSATTN_OK) return st;
  if (K == nullptr || mean == nullptr) return fail(BSATTN_ERR_INVALID, "K and mean must be non-NULL");
  if (mean_dtype != BSATTN_F32 && mean_dtype != BSATTN_BF16)
    return fail(BSATTN_ERR_INVALID, "mean_dtype %d: must be BSATTN_F32 or BSATTN_BF16", mean_dtype);
  if (rank < 0 || rank > BSATTN_MAX_RANK) return fail(BSATTN_ERR_INVALID, "rank must be in [0, %d]", BSATTN_MAX_RANK);
  st = check_factor(rank, factor, factor_dtype, factor_scale);
  if (st != BSATTN_OK) return st;
  st = check_basis(basis, sub_dim, rank, shape->head_dim);
  if (st != BSATTN_OK) return st;
  if (first_block < 0 || n_blocks < 0) return fail(BSATTN_ERR_INVALID, "negative block range");
  if ((long long)(first_block + (long long)n_blocks) * shape->block_size > shape->n_ctx)
    return fail(BSATTN_ERR_INVALID, "blocks past n_ctx are not complete");
  if ((long long)first_block + n_blocks > nblk_capacity)
    return fail(BSATTN_ERR_INVALID, "block range exceeds nblk_capacity");
  if (!aligned16(K) || !aligned16(mean) || (factor && !aligned16(factor)))
    return fail(BSATTN_ERR_INVALID, "device pointers must be 16-byte aligned");
  std::memset(&a, 0, sizeof(a));
  a.K = K; a.mean = mean; a.factor = factor;
  a.bh = shape->batch * shape->n_kv_heads;
  a.n_kv_heads = shape->n_kv_heads;
  a.kv_capacity = shape->kv_capacity;
  a.nblk_capacity = nblk_capacity;
  a.first_block = first_block;
  a.n_blocks = n_blocks;
  a.rank = rank;
  a.head_dim = shape->head_dim;
  a.bf16 = shape->dtype == BSATTN_BF16;
  a.mean_bf16 = mean_dtype == BSATTN_BF16;
  a.factor_fp4 = rank > 0 && factor_dtype == BSATTN_FP4_E2M1;
  a.factor_scale = factor_scale;
  a.basis = sub_dim > 0 ? basis : nullptr;
  a.sub_dim = sub_dim;
  return paged_args(shape, paged, a.paged);
}

}  // namespace

extern "C" {

bsattn_status bsattn_build_summaries(const bsattn_shape* shape, const void* K, int32_t rank,
                                     int32_t first_block, int32_t n_blocks, int32_t nblk_capacity,
                                     void* mean, int32_t mean_dtype, void* factor, int32_t factor_dtype,
                                     float* factor_scale, const float* basis, int32_t sub_dim,
                                     const bsattn_paged_kv* paged, void* hip_stream) {
  g_err[0] = 0;
  bsattn::SummaryArgs a;
  const bsattn_status st = summaries_args(shape, K, rank, first_block, n_blocks, nblk_capacity, mean, mean_dtype,
                                          factor, factor_dtype, factor_scale, basis, sub_dim, paged, a);
  if (st != BSATTN_OK) return st;
  if (n_blocks == 0) return BSATTN_OK;
  hipError_t e = bsattn::launch_summaries(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "summaries launch: %s", hipGetErrorString(e));
  return BSATTN_OK;
}

bsattn_status bsattn_append_kv(const bsattn_shape* shape, const void* K_new, const void* V_new, void* K, void* V,
                               int32_t rank, int32_t nblk_capacity, void* mean, int32_t mean_dtype, void* factor,
                               int32_t factor_dtype, float* factor_scale, const float* basis, int32_t sub_dim,
                               const bsattn_paged_kv* paged, void* hip_stream) {
  g_err[0] = 0;
  bsattn_status st = check_shape(shape, false);
  if (st != BSATTN_OK) return st;
  bsattn::PagedKV pk;
  st = paged_args(shape, paged, pk);
  if (st != BSATTN_OK) return st;
  if (K_new == nullptr || V_new == nullptr || K == nullptr || V == nullptr)
    return fail(BSATTN_ERR_INVALID, "K_new, V_new, K and V must be non-NULL");
  if (!aligned16(K_new) || !aligned16(V_new) || !aligned16(K) || !aligned16(V))
    return fail(BSATTN_ERR_INVALID, "device pointers must be 16-byte aligned");
  // the new token is t = n_ctx - 1; it completes block n_ctx / S - 1 when n_ctx % S == 0
  const bool completes = shape->n_ctx % shape->block_size == 0;
  bsattn::SummaryArgs sa;
  if (completes) {
    st = summaries_args(shape, K, rank, shape->n_ctx / shape->block_size - 1, 1, nblk_capacity, mean, mean_dtype,
                        factor, factor_dtype, factor_scale, basis, sub_dim, paged, sa);
    if (st != BSATTN_OK) return st;
  }
  bsattn::AppendArgs aa;
  aa.K_new = K_new; aa.V_new = V_new; aa.K = K; aa.V = V;
  aa.kv_capacity = shape->kv_capacity;
  aa.pos = shape->n_ctx - 1;
  aa.row_bytes = shape->head_dim * (shape->dtype == BSATTN_BF16 ? 2 : 4);
  aa.n_kv_heads = shape->n_kv_heads;
  aa.paged = pk;
  hipError_t e = bsattn::launch_append(aa, shape->batch * shape->n_kv_heads, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  if (completes) {
    e = bsattn::launch_summaries(sa, (hipStream_t)hip_stream);
    if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "summaries launch: %s", hipGetErrorString(e));
  }
  return BSATTN_OK;
}

bsattn_status bsattn_select_topk(const bsattn_shape* shape, const void* Q, const void* mean,
                                 int32_t mean_dtype, const void* factor, int32_t factor_dtype,
                                 const float* factor_scale, const float* basis, int32_t sub_dim,
                                 int32_t rank, int32_t nblk_capacity,
                                 int32_t top_k, int32_t window, int32_t n_sink,
                                 const int32_t* global_pos_host, int32_t n_global, int32_t* sel,
                                 float* scores, void* hip_stream) {
  g_err[0] = 0;
  bsattn::SelectArgs a;
  const bsattn_status st = select_args(shape, Q, mean, mean_dtype, factor, factor_dtype, factor_scale, basis,
                                       sub_dim, rank,
                                       nblk_capacity, top_k, window, n_sink, global_pos_host, n_global, sel,
                                       scores, a);
  if (st != BSATTN_OK) return st;
  hipError_t e = bsattn::launch_select_topk(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "select launch: %s", hipGetErrorString(e));
  return BSATTN_OK;
}

bsattn_status bsattn_select_exact(const bsattn_shape* shape, const void* Q, const void* K, int32_t nblk_capacity,
                                  int32_t top_k, int32_t window, int32_t n_sink, const int32_t* global_pos_host,
                                  int32_t n_global, int32_t* sel, float* scores, void* hip_stream) {
  g_err[0] = 0;
  bsattn_status st = check_shape(shape, true);
  if (st != BSATTN_OK) return st;
  if (shape->dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "the exact-mass selector takes BF16 Q/K");
  if (Q == nullptr || K == nullptr || sel == nullptr || scores == nullptr)
    return fail(BSATTN_ERR_INVALID, "Q, K, sel and scores must be non-NULL");
  if (!aligned16(Q) || !aligned16(K)) return fail(BSATTN_ERR_INVALID, "device pointers must be 16-byte aligned");
  if (top_k < 1 || top_k > BSATTN_MAX_TOP_K) return fail(BSATTN_ERR_INVALID, "top_k must be in [1, %d]", BSATTN_MAX_TOP_K);
  if (window < 0 || n_sink < 0) return fail(BSATTN_ERR_INVALID, "window and n_sink must be >= 0");
  const int nb = shape->n_ctx / shape->block_size;
  if (nb > BSATTN_MAX_BLOCKS) return fail(BSATTN_ERR_UNSUPPORTED, "more than %d complete blocks", BSATTN_MAX_BLOCKS);
  if (nblk_capacity < nb) return fail(BSATTN_ERR_INVALID, "nblk_capacity < n_ctx / block_size");
  st = check_globals(global_pos_host, n_global, shape->n_ctx);
  if (st != BSATTN_OK) return st;
  bsattn::SelectArgs a;
  std::memset(&a, 0, sizeof(a));
  a.Q = Q; a.K = K; a.sel = sel; a.scores = scores;
  a.kv_capacity = shape->kv_capacity;
  a.batch = shape->batch; a.n_q_heads = shape->n_q_heads; a.n_kv_heads = shape->n_kv_heads;
  a.head_dim = shape->head_dim;
  a.n_blocks = nb;
  a.nblk_capacity = nblk_capacity;
  a.top_k = top_k;
  a.scale = effective_scale(shape);
  a.bf16 = true;
  a.forced = make_forced(shape->n_ctx, window, n_sink, global_pos_host, n_global);
  hipError_t e = bsattn::launch_select_exact(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "exact selection launch: %s", hipGetErrorString(e));
  return BSATTN_OK;
}

size_t bsattn_decode_workspace_bytes(const bsattn_shape* shape, int32_t top_k, int32_t window,
                                     int32_t n_sink, int32_t n_global) {
  if (check_shape(shape, true) != BSATTN_OK) return 0;
  if (top_k < 1 || top_k > BSATTN_MAX_TOP_K || window < 0 || n_sink < 0 || n_global < 0 ||
      n_global > BSATTN_MAX_GLOBAL)
    return 0;
  return decode_workspace_bound(shape, top_k, window, n_sink, n_global);
}

bsattn_status bsattn_decode(const bsattn_shape* shape, const void* Q, const void* K, const void* V,
                            const int32_t* sel, int32_t top_k, int32_t window, int32_t n_sink,
                            const int32_t* global_pos_host, int32_t n_global, float* O, float* lse,
                            void* workspace, size_t ws_bytes, const bsattn_paged_kv* paged, void* hip_stream) {
  g_err[0] = 0;
  bsattn::DecodeArgs a;
  const bsattn_status st = decode_args(shape, Q, K, V, sel, top_k, window, n_sink, global_pos_host, n_global,
                                       O, lse, workspace, ws_bytes, paged, a);
  if (st != BSATTN_OK) return st;
  hipError_t e = bsattn::launch_decode(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return BSATTN_OK;
}

bsattn_status bsattn_decode_step(const bsattn_shape* shape, const void* Q, const void* K, const void* V,
                                 const void* mean, int32_t mean_dtype, const void* factor,
                                 int32_t factor_dtype, const float* factor_scale, const float* basis,
                                 int32_t sub_dim, int32_t rank, int32_t nblk_capacity,
                                 int32_t top_k, int32_t window, int32_t n_sink, const int32_t* global_pos_host,
                                 int32_t n_global, int32_t* sel, float* scores, float* O, float* lse,
                                 void* workspace, size_t ws_bytes, const bsattn_paged_kv* paged,
                                 void* hip_stream) {
  g_err[0] = 0;
  bsattn::SelectArgs sa;
  bsattn_status st = select_args(shape, Q, mean, mean_dtype, factor, factor_dtype, factor_scale, basis, sub_dim,
                                 rank,
                                 nblk_capacity, top_k, window, n_sink, global_pos_host, n_global, sel, scores,
                                 sa);
  if (st != BSATTN_OK) return st;
  bsattn::DecodeArgs da;
  st = decode_args(shape, Q, K, V, sel, top_k, window, n_sink, global_pos_host, n_global, O, lse, workspace,
                   ws_bytes, paged, da);
  if (st != BSATTN_OK) return st;
  // bf16 with at most 512 complete blocks and top_k <= 256: the decode waves
  // select (each wave alone); up to 2048 blocks the decode workgroups select
  // (together); otherwise the top-k kernel does, then the decode reads sel
  const int nb = sa.n_blocks;
  const bool fused = da.bf16 && nb >= 1 && nb <= bsattn::kFusedMaxBlocks && top_k <= bsattn::kFusedMaxTopK;
  const bool fused_wg = da.bf16 && !fused && nb <= bsattn::kFusedWgMaxBlocks && top_k <= bsattn::kFusedMaxTopK;
  if (fused || fused_wg) {
    sa.scores_only = true;
    da.scores = scores;
    da.nblk_capacity = nblk_capacity;
    da.sel_out = sel;
    da.key_slots = fused ? 8 : -8;
  }
  if (fused) {
    for (int j = 0; j < nb; ++j)
      if (bsattn::forced_mask(da.forced, j) == ~0ull) da.full_forced[j >> 6] |= 1ull << (j & 63);
  }
  // first order with bfloat16 means: the decode workgroups score the blocks
  // themselves (one launch, plus the merge when a pair has several workgroups)
  const bool scored_in_decode = fused && sa.rank == 0 && sa.mean_bf16;
  // a small fp32 step (first order, fp32 means, at most 256 complete blocks
  // and 16 items per pair): one decode workgroup per pair scores, selects and
  // attends, and writes O itself (one launch, no merge)
  const bool fused_f32 = !da.bf16 && sa.rank == 0 && !sa.mean_bf16 && nb >= 1 &&
                         nb <= 64 * bsattn::kDecodeWaves && top_k <= bsattn::kFusedMaxTopK &&
                         da.n_items <= 4 * bsattn::kDecodeWaves;
  hipError_t e = hipSuccess;
  if (fused_f32) {
    da.mean = mean;
    da.scores_out = scores;
    da.sel_out = sel;
    da.nblk_capacity = nblk_capacity;
    da.n_part = 1;
    da.n_merge = 1;
    da.per_wave = (da.n_items + bsattn::kDecodeWaves - 1) / bsattn::kDecodeWaves;
  } else if (scored_in_decode) {
    da.mean = mean;
    da.scores_out = scores;
  } else {
    e = bsattn::launch_select_topk(sa, (hipStream_t)hip_stream);
    if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "select launch: %s", hipGetErrorString(e));
  }
  e = bsattn::launch_decode(da, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return BSATTN_OK;
}

bsattn_status bsattn_decode_step_noalloc(const bsattn_shape* shape, const void* Q, const void* K,
                                         const void* V, const void* mean, int32_t mean_dtype,
                                         const void* factor, int32_t factor_dtype, const float* factor_scale,
                                         const float* basis, int32_t sub_dim, int32_t rank,
                                         int32_t nblk_capacity, int32_t top_k, int32_t window, int32_t n_sink,
                                         const int32_t* global_pos_host, int32_t n_global, int32_t* sel,
                                         float* scores, float* O, float* lse, const bsattn_paged_kv* paged,
                                         void* hip_stream) {
  g_err[0] = 0;
  // the split partials this call needs, checked against the fixed scratch
  // before anything else touches the device
  const bsattn_status st = check_shape(shape, true);
  if (st != BSATTN_OK) return st;
  if (top_k < 1 || top_k > BSATTN_MAX_TOP_K || window < 0 || n_sink < 0 || n_global < 0 ||
      n_global > BSATTN_MAX_GLOBAL)
    return fail(BSATTN_ERR_INVALID, "top_k, window, n_sink or n_global out of range");
  const size_t need = decode_workspace_bound(shape, top_k, window, n_sink, n_global);
  if (need > bsattn::kNoAllocScratchBytes)
    return fail(BSATTN_ERR_WORKSPACE,
                "the split partials need %zu bytes, more than the %zu-byte static scratch of the allocation-free "
                "step: use bsattn_decode_step with a workspace",
                need, bsattn::kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = bsattn::noalloc_scratch(&ws);
    if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "scratch address: %s", hipGetErrorString(e));
  }
  return bsattn_decode_step(shape, Q, K, V, mean, mean_dtype, factor, factor_dtype, factor_scale, basis, sub_dim,
                            rank, nblk_capacity, top_k, window, n_sink, global_pos_host, n_global, sel, scores, O,
                            lse, ws, need, paged, hip_stream);
}

bsattn_status bsattn_select_prefill(const bsattn_shape* shape, const void* Q, const void* mean,
                                    int32_t mean_dtype, int32_t nblk_capacity, int32_t top_k,
                                    int32_t window_left, int32_t n_sink, int32_t* sel, float* scores,
                                    void* hip_stream) {
  g_err[0] = 0;
  bsattn_status st = check_shape(shape, false);
  if (st != BSATTN_OK) return st;
  if (shape->dtype != BSATTN_BF16 || mean_dtype != BSATTN_BF16)
    return fail(BSATTN_ERR_UNSUPPORTED, "the prefill selection takes BF16 queries and BF16 means");
  if (Q == nullptr || mean == nullptr || sel == nullptr || scores == nullptr)
    return fail(BSATTN_ERR_INVALID, "Q, mean, sel and scores must be non-NULL");
  if (!aligned16(Q) || !aligned16(mean)) return fail(BSATTN_ERR_INVALID, "device pointers must be 16-byte aligned");
  if (top_k < 1 || top_k > BSATTN_SPARSE_MAX_TOP_K)
    return fail(BSATTN_ERR_INVALID, "top_k must be in [1, %d]", BSATTN_SPARSE_MAX_TOP_K);
  if (window_left < 0) return fail(BSATTN_ERR_INVALID, "window_left must be >= 0");
  if (n_sink < 0 || n_sink > BSATTN_SPARSE_MAX_SINK)
    return fail(BSATTN_ERR_INVALID, "n_sink must be in [0, %d]", BSATTN_SPARSE_MAX_SINK);
  const int nb = shape->n_ctx / shape->block_size;
  if (nb > BSATTN_MAX_BLOCKS) return fail(BSATTN_ERR_UNSUPPORTED, "more than %d complete blocks", BSATTN_MAX_BLOCKS);
  if (nblk_capacity < nb) return fail(BSATTN_ERR_INVALID, "nblk_capacity < n_ctx / block_size");
  bsattn::SelectArgs a;
  std::memset(&a, 0, sizeof(a));
  a.Q = Q; a.mean = mean; a.sel = sel; a.scores = scores;
  a.batch = shape->batch; a.n_q_heads = shape->n_q_heads; a.n_kv_heads = shape->n_kv_heads;
  a.head_dim = shape->head_dim;
  a.n_blocks = nb;
  a.nblk_capacity = nblk_capacity;
  a.top_k = top_k;
  a.scale = effective_scale(shape);
  a.bf16 = true;
  a.mean_bf16 = true;
  a.tile_rows = bsattn::kSparseTile;
  a.n_tiles = (shape->n_ctx + bsattn::kSparseTile - 1) / bsattn::kSparseTile;
  a.seq_len = shape->n_ctx;
  a.window_left = window_left;
  a.n_sink = n_sink;
  // tile scorer: one workgroup per (pair, tile, 64 blocks); top-k: one per (pair, tile)
  if ((long long)a.batch * a.n_kv_heads * a.n_tiles * ((nb + 63) / 64 > 0 ? (nb + 63) / 64 : 1) > 0x7fffffffLL)
    return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
  hipError_t e = bsattn::launch_prefill_select(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "prefill selection launch: %s", hipGetErrorString(e));
  return BSATTN_OK;
}

bsattn_status bsattn_sparse_prefill(const bsattn_shape* shape, const void* Q, const void* K, const void* V,
                                    const int32_t* sel, int32_t top_k, int32_t window_left, int32_t n_sink,
                                    float* O, float* lse, void* hip_stream) {
  g_err[0] = 0;
  bsattn_status st = check_shape(shape, false);
  if (st != BSATTN_OK) return st;
  if (shape->dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "the sparse prefill takes BF16 Q/K/V only");
  if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr || sel == nullptr)
    return fail(BSATTN_ERR_INVALID, "Q, K, V, sel and O must be non-NULL");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
    return fail(BSATTN_ERR_INVALID, "device pointers must be 16-byte aligned");
  if (top_k < 1 || top_k > BSATTN_SPARSE_MAX_TOP_K)
    return fail(BSATTN_ERR_INVALID, "top_k must be in [1, %d]", BSATTN_SPARSE_MAX_TOP_K);
  if (window_left < 0) return fail(BSATTN_ERR_INVALID, "window_left must be >= 0");
  if (n_sink < 0 || n_sink > BSATTN_SPARSE_MAX_SINK)
    return fail(BSATTN_ERR_INVALID, "n_sink must be in [0, %d]", BSATTN_SPARSE_MAX_SINK);
  const long long n_qt = (shape->n_ctx + 127) / 128;
  if (n_qt * shape->batch * shape->n_q_heads > 0x7fffffffLL) return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
  bsattn::PrefillArgs a;
  std::memset(&a, 0, sizeof(a));
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.lse = lse;
  a.batch = shape->batch; a.n_q_heads = shape->n_q_heads; a.n_kv_heads = shape->n_kv_heads;
  a.head_dim = shape->head_dim;
  a.seq_len = shape->n_ctx;
  a.kv_capacity = shape->kv_capacity;
  a.window_left = window_left;
  a.window_right = 0;
  a.causal = 1;
  a.scale = effective_scale(shape);
  a.sp_sel = sel;
  a.sp_top_k = top_k;
  a.sp_n_sink = n_sink;
  a.sp_n_tiles = (int32_t)n_qt;
  hipError_t e = bsattn::launch_prefill(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "sparse prefill launch: %s", hipGetErrorString(e));
  return BSATTN_OK;
}

size_t bsattn_prefill_workspace_bytes(const bsattn_shape* shape, int32_t n_global) {
  if (check_shape(shape, false) != BSATTN_OK) return 0;
  if (n_global <= 0 || n_global > BSATTN_MAX_GLOBAL) return 0;
  return prefill_workspace_layout(shape, n_global).total;
}

bsattn_status bsattn_prefill(const bsattn_shape* shape, const void* Q, const void* K, const void* V,
                             int32_t window_left, int32_t window_right, int32_t causal,
                             const int32_t* global_pos_host, int32_t n_global, float* O, float* lse,
                             void* workspace, size_t ws_bytes, void* hip_stream) {
  g_err[0] = 0;
  bsattn_status st = check_shape(shape, false);
  if (st != BSATTN_OK) return st;
  if (shape->dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "prefill takes bf16 Q/K/V only");
  if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr)
    return fail(BSATTN_ERR_INVALID, "Q, K, V and O must be non-NULL");
  if (causal != 0 && causal != 1) return fail(BSATTN_ERR_INVALID, "causal must be 0 or 1");
  st = check_globals(global_pos_host, n_global, shape->n_ctx);
  if (st != BSATTN_OK) return st;
  if (causal && n_global > 0)
    return fail(BSATTN_ERR_UNSUPPORTED, "global tokens are bidirectional; causal masks take none");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
    return fail(BSATTN_ERR_INVALID, "device pointers must be 16-byte aligned");
  const PrefillWs lay = prefill_workspace_layout(shape, n_global);
  if (lay.total > 0) {
    if (workspace == nullptr || ws_bytes < lay.total)
      return fail(BSATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", lay.total, ws_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(BSATTN_ERR_INVALID, "workspace must be 256-byte aligned");
  }
  const long long n_qt = (shape->n_ctx + 127) / 128;
  const long long n_wg = n_qt * shape->batch * shape->n_q_heads + lay.n_wg;
  if (n_wg > 0x7fffffffLL) return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
  bsattn::PrefillArgs a;
  std::memset(&a, 0, sizeof(a));
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.lse = lse;
  a.batch = shape->batch; a.n_q_heads = shape->n_q_heads; a.n_kv_heads = shape->n_kv_heads;
  a.head_dim = shape->head_dim;
  a.seq_len = shape->n_ctx;
  a.kv_capacity = shape->kv_capacity;
  a.window_left = window_left < 0 ? -1 : window_left;
  a.window_right = window_right < 0 ? -1 : window_right;
  a.causal = causal;
  a.scale = effective_scale(shape);
  a.n_global = n_global;
  for (int i = 0; i < n_global; ++i) a.gpos[i] = global_pos_host[i];
  if (lay.total > 0) {
    a.n_global_wg = lay.n_wg;
    a.g_splits = lay.splits;
    a.g_keys_per_split = lay.keys_per_split;
    a.g_part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.o_off);
    a.g_part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.ml_off);
  }
  hipError_t e = bsattn::launch_prefill(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return BSATTN_OK;
}

bsattn_status bsattn_prefill_dilated(const bsattn_shape* shape, const void* Q, const void* K, const void* V,
                                     int32_t window_left, int32_t window_right, int32_t causal,
                                     int32_t dilation, float* O, float* lse, void* hip_stream) {
  g_err[0] = 0;
  bsattn_status st = check_shape(shape, false);
  if (st != BSATTN_OK) return st;
  if (shape->dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "prefill takes bf16 Q/K/V only");
  if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr)
    return fail(BSATTN_ERR_INVALID, "Q, K, V and O must be non-NULL");
  if (causal != 0 && causal != 1) return fail(BSATTN_ERR_INVALID, "causal must be 0 or 1");
  if (dilation < 1 || dilation > BSATTN_MAX_DILATION)
    return fail(BSATTN_ERR_INVALID, "dilation must be in [1, %d]", BSATTN_MAX_DILATION);
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
    return fail(BSATTN_ERR_INVALID, "device pointers must be 16-byte aligned");
  const int N = shape->n_ctx;
  // residue class r: logical rows x < ceil((N - r) / s), physical rows r + s x;
  // the dilated band is the plain band of the logical rows with the windows
  // divided by s (rounded down: i - j = s (x_i - x_j))
  const int s = dilation;
  for (int r = 0; r < s && r < N; ++r) {
    const int nr = (N - r + s - 1) / s;
    const long long n_wg = (long long)((nr + 127) / 128) * shape->batch * shape->n_q_heads;
    if (n_wg > 0x7fffffffLL) return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
  }
  bsattn::PrefillArgs a;
  std::memset(&a, 0, sizeof(a));
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.lse = lse;
  a.batch = shape->batch; a.n_q_heads = shape->n_q_heads; a.n_kv_heads = shape->n_kv_heads;
  a.head_dim = shape->head_dim;
  a.kv_capacity = shape->kv_capacity;
  a.window_left = window_left < 0 ? -1 : window_left / s;
  a.window_right = window_right < 0 ? -1 : window_right / s;
  a.causal = causal;
  a.scale = effective_scale(shape);
  a.dil = s;
  a.seq_phys = N;
  for (int r = 0; r < s && r < N; ++r) {
    a.dil_off = r;
    a.seq_len = (N - r + s - 1) / s;
    hipError_t e = bsattn::launch_prefill(a, (hipStream_t)hip_stream);
    if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  }
  return BSATTN_OK;
}

}  // extern "C"
