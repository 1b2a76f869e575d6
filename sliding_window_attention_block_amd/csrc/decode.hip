// Sparse flash-decode over the selected blocks plus the forced tokens
// (window, sinks, globals), split over workgroups, then a log-sum-exp merge.
//
// What is computed: one softmax per query head over the token set
// T = forced tokens  union  tokens of the selected blocks (a set: a token
// reached two ways is attended once), as the COBS explainer's technical
// summary describes block-sparse decode (sections 1 and 2.1: read only the
// chosen contiguous blocks) with the sliding window and sink tokens of the
// SWA glossary ("SWAの拡張手法") and the global tokens of the local-global
// glossary.  Splitting uses the online-softmax identity: partial (m, l, o)
// over disjoint token sets merge exactly after rescaling by 2^(m - M).
//
// Work items: per (b, K/V head) the list is the top_k selected blocks, then
// the forced blocks (sink range, window range, blocks holding a global token).
// A selected block contributes its tokens that are not forced, a forced block
// its forced tokens, so no token is counted twice and no search of `sel` is
// needed.
//
// Fused decode step (bf16): the top-k runs inside the decode waves.  Each
// wave first loads its pair's group scores, then issues the loads of its
// forced half items (which do not depend on the selection), and selects the
// pair's top-k blocks (exact radix select, same keys and tie rule as the
// top-k kernel) while those loads are in flight; its selected half items
// follow.  Every wave of a pair computes the same selection; the pair's first
// wave writes it out.
//
// bf16 path (MFMA, gfx950 v_mfma_f32_16x16x32_bf16): the unit is a half item
// (32 tokens of one block).  Each wave owns a run of half items of one pair
// and pipelines them two deep (next half item's loads in flight while the
// current one is computed); waves never wait for each other until the end,
// where the four waves of a workgroup (one pair) merge in LDS.
//   K goes straight from HBM into MFMA A-operand registers; V is loaded with
//   coalesced 1 KB instructions into registers and, at compute time, written
//   to the wave's LDS tile (XOR-swizzled 16-byte chunks) and read back
//   transposed.
//   S^T = K Q^T: B = Q^T held in registers (16 query heads of the group, zero
//   padded), so lane l holds the logits of query head l%16 for 8 tokens.
//   O^T += V^T P^T: V^T read with ds_read_b64_tr_b16.  P = P_hi + P_lo in
//   bf16 (two products), so the result keeps ~2^-17 of P's precision.  The
//   output tile keeps query head l%16 in lane l, so the rescale is per lane.
// fp32 path (VALU): one token per lane, one item per wave; the 4 waves of a
// workgroup merge in LDS into one partial.
//
// With one workgroup per pair the kernel writes O and lse itself; otherwise
// each workgroup writes one partial and a small second kernel merges them (the
// kernel boundary makes every partial visible; the L2s of the 8 XCDs are not
// coherent with each other, and merging inside the kernel, through agent-scope
// stores and an arrival counter, measured no faster than the extra launch).
#include <mutex>

#include "launch.hpp"

namespace bsattn {
namespace {

constexpr int kW = kDecodeWaves;

struct ItemInfo {
  int blk;
  uint64_t mask;
};

// Block and token mask of item `it` (a selected block: its tokens outside the
// forced set; a forced block: its forced tokens); blk < 0 means nothing to do.
__device__ __forceinline__ ItemInfo item_info(const DecodeArgs& a, const int32_t* selrow, int it) {
  ItemInfo r;
  if (it < a.top_k) {
    const int blk = selrow[it];
    // only complete blocks can be selected; anything else is ignored
    const bool ok = blk >= 0 && blk < a.forced.n_ctx / kBlock;
    r.mask = ok ? ~forced_mask(a.forced, blk) : 0ull;
    r.blk = r.mask ? blk : -1;
    return r;
  }
  const int f = it - a.top_k;
  const ForcedBlocks& fb = a.fblocks;
  int blk;
  if (f < fb.r0_n) blk = fb.r0_lo + f;
  else if (f < fb.r0_n + fb.r1_n) blk = fb.r1_lo + (f - fb.r0_n);
  else blk = fb.gblk[f - fb.r0_n - fb.r1_n];
  r.mask = forced_mask(a.forced, blk);
  r.blk = r.mask ? blk : -1;
  return r;
}

// Swizzle of a per-wave V tile: chunk c of row r lives at physical chunk c ^ f(r).
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  constexpr int RPL = 256 / (D * 2);  // rows per 256-byte bank line
  constexpr int NX = 8 / RPL;         // distinct swizzle values
  return 2 * ((r / RPL) & (NX - 1));
}
template <int D>
__device__ __forceinline__ uint32_t v_off(int r, int c) {
  return (uint32_t)(r * D * 2 + ((c ^ v_swz<D>(r)) << 4));
}

// LDS used for the workgroup merge, overlaid on the V tiles once every wave is done.
template <int D>
struct MergeLds {
  float m[kW][16];
  float l[kW][16];
  float o[kW][16][D + 4];  // padded rows: the 16 heads of a wave hit different banks
};

// Merge the waves' (m, l, o) held in LDS into this workgroup's result: O and lse
// when the pair has one workgroup, else one partial (max and normaliser in the
// log2 domain, unnormalised numerator) for the merge kernel.
template <int D>
__device__ __forceinline__ void write_wg_result(const DecodeArgs& a, const MergeLds<D>* ml, int b, int g) {
  const int G = a.n_q_heads / a.n_kv_heads;
  const int n_wg = a.n_merge, wg = blockIdx.x;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * kW) {
    const int hh = idx / D, dd = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kW; ++w) M = fmaxf(M, ml->m[w][hh]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const float mw = ml->m[w][hh];
        const float sc = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        L = fmaf(sc, ml->l[w][hh], L);
        O = fmaf(sc, ml->o[w][hh][dd], O);
      }
    }
    const size_t qrow = (size_t)b * a.n_q_heads + g * G + hh;
    if (n_wg == 1) {
      a.O[qrow * D + dd] = L > 0.f ? O / L : 0.f;
      if (a.lse != nullptr && dd == 0) a.lse[qrow] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    } else {
      const size_t prow = qrow * n_wg + wg;
      a.part_o[prow * D + dd] = O;
      if (dd == 0) {
        a.part_ml[2 * prow] = M;
        a.part_ml[2 * prow + 1] = L;
      }
    }
  }
}

// bf16 path.  Work unit: a half item (32 tokens of one block) of one
// (b, K/V head) pair.  Each wave owns `per_wave` consecutive half items of one
// pair and runs them through a two-stage register pipeline: while it computes
// one half item, the loads of the next are already in flight.  K is loaded
// straight into MFMA A-operand registers; V is loaded with coalesced 1 KB
// instructions into registers and, at compute time, written to the wave's LDS
// tile and read back transposed.  Only plain vector loads are in flight, so the
// compiler's own waits are exact.  Waves never wait for each other before the
// final merge (no barriers in the loop), so the memory system sees a steady
// stream of requests instead of rounds of workgroups that load, then compute,
// then retire together.
//
// Token set without any search: a selected block contributes its tokens that
// are not forced; a forced block contributes its forced tokens.  Every token of
// T is therefore counted exactly once, whatever `sel` holds.
template <int D>
struct HalfItem {
  static constexpr int DC = D / 32;        // 32-wide d chunks of the QK product
  static constexpr int RB = D * 2;         // bytes per token row
  static constexpr int TILE = 32 * RB;     // V bytes of a half item
  static constexpr int NCH = TILE / 1024;  // 1 KB V load instructions per half item
};

template <int D>
struct Stage {
  u32x4 k[2][HalfItem<D>::DC];  // K A-operands: tokens 16tt + h, dims 32dc + 8grp .. +8
  u32x4 v[HalfItem<D>::NCH];    // V bytes [1024i + 16 lane, +16) of the half item
  uint32_t hmask;               // tokens of T among the 32 (0: nothing to do)
};

// Block and 64-token mask of the f-th forced item, and of a selected block.
// Mask 0: nothing to do (the block index is then 0, so the loads that are
// still issued stay in bounds).
__device__ __forceinline__ void forced_item(const DecodeArgs& a, int f, int& blk, uint64_t& mask) {
  const ForcedBlocks& fb = a.fblocks;
  if (f < fb.r0_n) blk = fb.r0_lo + f;
  else if (f < fb.r0_n + fb.r1_n) blk = fb.r1_lo + (f - fb.r0_n);
  else blk = fb.gblk[f - fb.r0_n - fb.r1_n];
  mask = forced_mask(a.forced, blk);
  if (mask == 0ull) blk = 0;
}
__device__ __forceinline__ void selected_item(const DecodeArgs& a, int sel_blk, int& blk, uint64_t& mask) {
  // only complete blocks can be selected; anything else is ignored
  const bool ok = sel_blk >= 0 && sel_blk < a.forced.n_ctx / kBlock;
  mask = ok ? ~forced_mask(a.forced, sel_blk) : 0ull;
  blk = mask ? sel_blk : 0;
}

// Exact top-k of one pair inside one wave.  Lane l holds the scores of blocks
// 64t + l (t < PL), so (t, lane) order is block order.  Candidates: complete
// blocks with a token outside the forced set; order: score descending, then
// block index ascending.  A radix select (8 bits a pass, 256-bin histogram in
// this wave's LDS `hist`) finds the k-th largest key T and how many keys equal
// to T are taken (the lowest-index ones); bits that every candidate key
// shares are known from the wave's AND / OR, and each pass's 8-bit digit
// starts at the highest bit still undecided.  The selected blocks
// go to tab[0 .. top_k) in ascending order, -1 after the last.
template <int PL>
__device__ __forceinline__ void wave_topk(const DecodeArgs& a, const float (&sv)[PL], uint32_t* hist, int32_t* tab) {
  const int lane = threadIdx.x & 63;
  const int NB = a.forced.n_ctx / kBlock;
  uint32_t key[PL];
  uint32_t cm = 0u;  // bit t: block 64t + lane is a candidate
  uint32_t kand = ~0u, kor = 0u;
#pragma unroll
  for (int t = 0; t < PL; ++t) {
    const int j = 64 * t + lane;
    key[t] = order_key(sv[t]);
    if (j < NB && !((a.full_forced[t] >> lane) & 1ull)) {
      cm |= 1u << t;
      kand &= key[t];
      kor |= key[t];
    }
  }
  const int ncand = __builtin_amdgcn_readlane(wave_incl_scan_dpp(__popc(cm)), 63);
  const int kk = min(a.top_k, ncand);
  uint32_t all_and, all_or;
  wave_and_or(kand, kor, all_and, all_or);  // (all ones / zero when there is no candidate)
  const uint32_t diff = all_and ^ all_or;
  // first pass: the 8 bits from the highest bit on which candidate keys differ
  // down (bits above it are shared by every candidate), then the next 8 below
  const int hb = diff ? 31 - __clz(diff) : -1;
  uint32_t pmask = hb >= 31 ? 0u : ~0u << (hb + 1);
  uint32_t prefix = all_and & pmask;
  int remaining = kk;
  if (kk > 0) {
    for (int hi = hb; hi >= 0;) {
      const int lo = max(hi - 7, 0);
      const uint32_t dmask = (2u << (hi - lo)) - 1u;
      reinterpret_cast<u32x4*>(hist)[lane] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < PL; ++t)
        if (((cm >> t) & 1u) && (key[t] & pmask) == prefix) atomicAdd(&hist[(key[t] >> lo) & dmask], 1u);
      // lane l reads digits 255-4l (c4[3]) down to 252-4l (c4[0])
      const u32x4 c4 = reinterpret_cast<const u32x4*>(hist)[63 - lane];
      const int sum = (int)(c4[0] + c4[1] + c4[2] + c4[3]);
      int cum = wave_incl_scan_dpp(sum) - sum;
      int found = -1, above = 0, inbin = 0;
#pragma unroll
      for (int u = 3; u >= 0; --u) {
        if (found < 0 && cum + (int)c4[u] >= remaining) {
          found = 4 * (63 - lane) + u;
          above = cum;
          inbin = (int)c4[u];
        }
        cum += (int)c4[u];
      }
      const uint64_t hit = __ballot(found >= 0);
      const int src = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
      const int digit = __builtin_amdgcn_readlane(found, src);
      remaining -= __builtin_amdgcn_readlane(above, src);
      prefix |= (uint32_t)digit << lo;
      pmask |= dmask << lo;
      // every key of the bin is taken: the lower bits do not matter
      if (__builtin_amdgcn_readlane(inbin, src) == remaining) break;
      hi = lo - 1;
    }
  }
  // keys above the prefix, then the first `remaining` keys on it, in block order
  int base = 0, eq_before = 0;
  if (kk > 0) {
#pragma unroll
    for (int t = 0; t < PL; ++t) {
      const bool c = (cm >> t) & 1u;
      const uint32_t km = key[t] & pmask;
      const bool eq = c && km == prefix;
      const uint64_t be = __ballot(eq);
      const int er = eq_before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
      const bool take = (c && km > prefix) || (eq && er < remaining);
      const uint64_t bt = __ballot(take);
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bt >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)bt, 0u));
      if (take && pos < a.top_k) tab[pos] = 64 * t + lane;
      base += __popcll(bt);
      eq_before += __popcll(be);
    }
  }
  for (int i = base + lane; i < a.top_k; i += 64) tab[i] = -1;
}

// Exact top-k of one pair by the whole workgroup (kW waves), for up to 64 kW KPT
// blocks: thread t holds the keys of its contiguous block range [t per,
// (t + 1) per) (per <= KPT, loaded into `key` by the caller), so thread order
// is block order.  A radix select over the 256-bin LDS histograms (one per
// pass, cleared up front; one barrier per pass, after which every wave finds
// the pass's digit itself), the same keys, candidates and tie rule as the
// in-wave select; then each thread's taken blocks go to tab[rank] in LDS, the
// ranks from the waves' prefix counts (one barrier), -1 after the last.  Ends
// with a barrier: tab is complete for every wave.
struct WgTopkLds {
  uint32_t hist[4][256];
  uint32_t red[kW][3];  // per wave: candidates, AND, OR of their keys
  int part[kW][2];      // per wave: keys above, keys on the threshold
};
template <int KPT>
__device__ __forceinline__ void wg_topk(const DecodeArgs& a, const uint32_t (&key)[KPT], int j0, int j1,
                                        WgTopkLds& l, int32_t* tab) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t cm = 0u;  // bit t: block j0 + t is a candidate
  uint32_t kand = ~0u, kor = 0u;
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const int j = j0 + t;
    if (j < j1 && forced_mask(a.forced, j) != ~0ull) {
      cm |= 1u << t;
      kand &= key[t];
      kor |= key[t];
    }
  }
  for (int i = tid; i < 4 * 256; i += 64 * kW) (&l.hist[0][0])[i] = 0u;
  {
    const int cnt = __builtin_amdgcn_readlane(wave_incl_scan_dpp(__popc(cm)), 63);
    uint32_t wa, wo;
    wave_and_or(kand, kor, wa, wo);
    if (lane == 0) {
      l.red[wid][0] = (uint32_t)cnt;
      l.red[wid][1] = wa;
      l.red[wid][2] = wo;
    }
  }
  __syncthreads();
  int tot = 0;
  uint32_t all_and = ~0u, all_or = 0u;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    tot += (int)l.red[w][0];
    all_and &= l.red[w][1];
    all_or |= l.red[w][2];
  }
  const int kk = min(a.top_k, tot);
  const uint32_t diff = all_and ^ all_or;
  // 8-bit digits from the highest bit on which candidate keys differ down
  const int hb = diff ? 31 - __clz(diff) : -1;
  uint32_t pmask = hb >= 31 ? 0u : ~0u << (hb + 1);
  uint32_t prefix = all_and & pmask;
  int remaining = kk;
  if (kk > 0) {
    int pass = 0;
    for (int hi = hb; hi >= 0; ++pass) {
      const int lo = max(hi - 7, 0);
      const uint32_t dmask = (2u << (hi - lo)) - 1u;
      uint32_t* h = l.hist[pass];
#pragma unroll
      for (int t = 0; t < KPT; ++t)
        if (((cm >> t) & 1u) && (key[t] & pmask) == prefix) atomicAdd(&h[(key[t] >> lo) & dmask], 1u);
      __syncthreads();
      // every wave: lane l reads digits 255-4l (c4[3]) down to 252-4l (c4[0])
      const u32x4 c4 = reinterpret_cast<const u32x4*>(h)[63 - lane];
      const int sum = (int)(c4[0] + c4[1] + c4[2] + c4[3]);
      int cum = wave_incl_scan_dpp(sum) - sum;
      int found = -1, above = 0, inbin = 0;
#pragma unroll
      for (int u = 3; u >= 0; --u) {
        if (found < 0 && cum + (int)c4[u] >= remaining) {
          found = 4 * (63 - lane) + u;
          above = cum;
          inbin = (int)c4[u];
        }
        cum += (int)c4[u];
      }
      const uint64_t hit = __ballot(found >= 0);
      const int src = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
      const int digit = __builtin_amdgcn_readlane(found, src);
      remaining -= __builtin_amdgcn_readlane(above, src);
      prefix |= (uint32_t)digit << lo;
      pmask |= dmask << lo;
      // the same in every wave: every key of the bin is taken, lower bits do not matter
      if (__builtin_amdgcn_readlane(inbin, src) == remaining) break;
      hi = lo - 1;
    }
  }
  // keys above the prefix, then the first `remaining` keys on it, in block order
  int gt = 0, eq = 0;
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    if (!((cm >> t) & 1u)) continue;
    const uint32_t km = key[t] & pmask;
    gt += km > prefix;
    eq += km == prefix;
  }
  const int igt = wave_incl_scan_dpp(gt), ieq = wave_incl_scan_dpp(eq);
  if (lane == 63) {
    l.part[wid][0] = igt;
    l.part[wid][1] = ieq;
  }
  __syncthreads();
  int gt_before = igt - gt, eq_before = ieq - eq;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    if (w < wid) {
      gt_before += l.part[w][0];
      eq_before += l.part[w][1];
    }
  }
  if (kk > 0) {
    const int take_eq = max(0, min(eq, remaining - eq_before));
    int pos = gt_before + min(eq_before, remaining);
    int taken = 0;
#pragma unroll
    for (int t = 0; t < KPT; ++t) {
      if (!((cm >> t) & 1u)) continue;
      const uint32_t km = key[t] & pmask;
      if (km > prefix || (km == prefix && taken < take_eq)) {
        taken += km == prefix;
        tab[pos++] = j0 + t;
      }
    }
  }
  for (int i = kk + tid; i < a.top_k; i += 64 * kW) tab[i] = -1;
  __syncthreads();
}

template <int D>
__device__ __forceinline__ void load_half(const uint16_t* Kb, const uint16_t* Vb, int tok0, int last,
                                          Stage<D>& st) {
  using H = HalfItem<D>;
  const int lane = threadIdx.x & 63, h = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const size_t row = (size_t)min(tok0 + 16 * tt + h, last);
#pragma unroll
    for (int dc = 0; dc < H::DC; ++dc)
      st.k[tt][dc] = *reinterpret_cast<const u32x4*>(Kb + row * D + 32 * dc + 8 * grp);
  }
#pragma unroll
  for (int i = 0; i < H::NCH; ++i) {
    const int off = 1024 * i + 16 * lane;
    const size_t row = (size_t)min(tok0 + off / H::RB, last);
    st.v[i] = *reinterpret_cast<const u32x4*>(Vb + row * D + (off % H::RB) / 2);
  }
}

// load_half for a paged cache: the item's block has its 64 / P pages p0 .. p3
// (P = 1 << page_shift >= 16, so a 16-row K group or a V chunk never straddles
// two pages); each lane takes the page of its own (clamped) row.
template <int D>
__device__ __forceinline__ void load_half_paged(const DecodeArgs& a, int g, int p0, int p1, int p2, int p3,
                                                int tok0, int last, Stage<D>& st) {
  using H = HalfItem<D>;
  const int lane = threadIdx.x & 63, h = lane & 15, grp = lane >> 4;
  const int sh = a.paged.page_shift;
  auto row_of = [&](int t) __attribute__((always_inline)) {
    const int s = (t & (kBlock - 1)) >> sh;
    const int page = s == 0 ? p0 : (s == 1 ? p1 : (s == 2 ? p2 : p3));
    return (((size_t)page * a.n_kv_heads + g) << sh) + (t & ((1 << sh) - 1));
  };
  const uint16_t* K = reinterpret_cast<const uint16_t*>(a.K);
  const uint16_t* V = reinterpret_cast<const uint16_t*>(a.V);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const size_t row = row_of(min(tok0 + 16 * tt + h, last));
#pragma unroll
    for (int dc = 0; dc < H::DC; ++dc)
      st.k[tt][dc] = *reinterpret_cast<const u32x4*>(K + row * D + 32 * dc + 8 * grp);
  }
#pragma unroll
  for (int i = 0; i < H::NCH; ++i) {
    const int off = 1024 * i + 16 * lane;
    const size_t row = row_of(min(tok0 + off / H::RB, last));
    st.v[i] = *reinterpret_cast<const u32x4*>(V + row * D + (off % H::RB) / 2);
  }
}

// Online-softmax update of one half item whose K and V registers have landed.
template <int D>
__device__ __forceinline__ void compute_half(const Stage<D>& st, uint8_t* vt, const u32x4* qop, float sl2,
                                             float& m_run, float& l_run, f32x4* oacc) {
  using H = HalfItem<D>;
  constexpr int DC = H::DC, DT = D / 16;
  const int lane = threadIdx.x & 63, h = lane & 15, grp = lane >> 4;
  const uint32_t hmask = st.hmask;
  // V rows into the wave's LDS tile (chunk c of row r at physical chunk c ^ swz(r))
#pragma unroll
  for (int i = 0; i < H::NCH; ++i) {
    const int off = 1024 * i + 16 * lane;
    *reinterpret_cast<u32x4*>(vt + v_off<D>(off / H::RB, (off % H::RB) >> 4)) = st.v[i];
  }
  // S^T = K Q^T: lane (h, grp) holds head h's logits of tokens 16tt + 4grp + r
  f32x4 s[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) s[tt] = mfma16x16x32(as_bf16x8(st.k[tt][dc]), as_bf16x8(qop[dc]), s[tt]);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = ((hmask >> (16 * tt + 4 * grp + r)) & 1u) ? s[tt][r] : -INFINITY;
      s[tt][r] = v;
      mx = fmaxf(mx, v);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // the running max moves only when it grows by more than 2^8 (weights stay <= 2^8)
  const float m_cand = mx * sl2;
  const bool need = m_cand > m_run + kDecodeHeadroom;
  if (__ballot(need)) {
    const float m_new = need ? m_cand : m_run;
    const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
    m_run = m_new;
  }
  const float nm = (m_run == -INFINITY) ? 0.f : -m_run;
  // P = P_hi + P_lo, both bf16: the second PV product (free: decode is bound by
  // HBM) keeps the result exact to ~2^-17 of P however few tokens a head sees.
  u32x4 pop, plo;
  float psum = 0.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[tt][r], sl2, nm));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[tt][r + 1], sl2, nm));
      const uint32_t pk = cvt_pk_bf16(p0, p1);
      pop[2 * tt + r / 2] = pk;
      plo[2 * tt + r / 2] = cvt_pk_bf16(p0 - bf16lo(pk), p1 - bf16hi(pk));
      psum += p0 + p1;
    }
  l_run += psum;
  // O^T += V^T P^T.  Lane a of 16-lane group q reads 8 bytes of V row 4q + a/4
  // (+16 for the second half of the k range), columns 16dt + 4(a%4).
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int row = 4 * grp + (h >> 2);
    const int col = 16 * dt + 4 * (h & 3);  // element index
    const u32x2 lo = lds_read_tr16(vt, v_off<D>(row, col >> 3) + ((col & 7) << 1));
    const u32x2 hi = lds_read_tr16(vt, v_off<D>(row + 16, col >> 3) + ((col & 7) << 1));
    const u32x4 vop = u32x4{lo[0], lo[1], hi[0], hi[1]};
    oacc[dt] = mfma16x16x32(as_bf16x8(vop), as_bf16x8(pop), oacc[dt]);
    oacc[dt] = mfma16x16x32(as_bf16x8(vop), as_bf16x8(plo), oacc[dt]);
  }
}

// d = 128: two stages of K and V take 128 registers, so a wave gets the whole
// 512-register budget of a SIMD (one workgroup of 4 waves per CU); d = 64 fits
// two workgroups per CU.  PL > 0: fused step, PL scores per lane for the
// in-wave top-k; PL = 0: the selection comes from `sel`.  PAGED: K and V are
// page pools read through the block table.  SC (with PL > 0): the workgroup
// also scores its pair's blocks (first-order score from bfloat16 block means,
// COBS explainer technical summary 2.1; group score = log of the summed
// exponentials over the group's query heads), so the step needs no scoring
// launch: each wave scores 64 PL / 4 blocks on v_mfma_f32_16x16x32_bf16 (A =
// the group's queries, B = 16 mean rows; products exact in bfloat16, sums in
// fp32, the same operations as the scoring kernel), the scores meet in LDS,
// and every wave then selects from them.  The mean loads are issued before
// the first forced half items' loads, so the scoring waits for the means
// alone while the forced K/V rows stream in.  The workgroups of one pair are
// placed on one XCD (workgroups are dispatched to the 8 XCDs round robin), so
// the second read of the pair's means hits that XCD's L2.
//
// PL < 0: fused step for up to 64 kW (-PL) blocks: the workgroup selects
// together (wg_topk, -PL keys per thread, from `scores`), so a pair's
// selection costs each wave a few barriers instead of a radix select over all
// its blocks.
template <int D, int PL, bool PAGED, bool SC = false>
__global__ __launch_bounds__(64 * kW, D == 128 ? 1 : 2) void decode_bf16_kernel(DecodeArgs args) {
  // The arguments are read in place from the kernel-argument segment (the
  // only explicit argument sits at its offset 0): per-lane lookups into the
  // forced-token tables then stay plain constant-memory loads, where the
  // by-value parameter could be copied to scratch first.
  (void)args;
  const DecodeArgs& a = *(const DecodeArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  using H = HalfItem<D>;
  constexpr int DC = H::DC, DT = D / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kW * H::TILE];

  const int lane = threadIdx.x & 63;
  // wave-uniform (scalar registers): every item index, block and mask below is too
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_pairs = a.batch * a.n_kv_heads;
  int pair, wi;
  if (SC && n_pairs % 8 == 0) {
    // workgroup wg runs on XCD wg % 8: slot wg / 8 of that XCD holds workgroup
    // slot % n_merge of pair 8 (slot / n_merge) + wg % 8
    const int wg = blockIdx.x, xcd = wg & 7, slot = wg >> 3;
    pair = (slot / a.n_merge) * 8 + xcd;
    wi = (slot % a.n_merge) * kW + wid;
  } else {
    const int gw = blockIdx.x * kW + wid;  // global wave index
    pair = gw / a.n_part;
    wi = gw % a.n_part;
  }
  // n_part is a multiple of kW: the four waves of a workgroup share one pair,
  // so this exit is uniform over the workgroup (it meets barriers at the end)
  if (pair >= n_pairs) return;
  const int b = pair / a.n_kv_heads, g = pair % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int h = lane & 15, grp = lane >> 4;
  uint8_t* const vt = smem + wid * H::TILE;

  // fused step: the pair's group scores, loaded before anything else so the
  // selection waits for them alone
  float sv[PL > 0 ? PL : 1];
  if constexpr (PL > 0 && !SC) {
    const float* sc = a.scores + (size_t)pair * a.nblk_capacity;
    const int nb_last = a.forced.n_ctx / kBlock - 1;  // >= 0 on the fused path
#pragma unroll
    for (int t = 0; t < PL; ++t) sv[t] = sc[min(64 * t + lane, nb_last)];
  }
  // PL < 0 (and SC): this thread's keys, blocks [wj0, wj1) of the pair
  constexpr int KPT = PL < 0 ? -PL : (SC ? kFusedMaxBlocks / (64 * kW) : 1);
  uint32_t wkey[KPT];
  int wj0 = 0, wj1 = 0;
  if constexpr (PL < 0) {
    const int NB = a.forced.n_ctx / kBlock;
    const int per = (NB + 64 * kW - 1) / (64 * kW);
    wj0 = min((int)threadIdx.x * per, NB);
    wj1 = min(wj0 + per, NB);
    const float* sc = a.scores + (size_t)pair * a.nblk_capacity;
#pragma unroll
    for (int t = 0; t < KPT; ++t) wkey[t] = order_key(sc[min(wj0 + t, NB - 1)]);
  }

  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.K) + (size_t)pair * a.kv_capacity * D;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(a.V) + (size_t)pair * a.kv_capacity * D;
  const int last = a.forced.n_ctx - 1;  // rows past the context (tail block) are masked; clamp loads
  const float sl2 = a.scale * kLog2e;

  // This wave's half items (32 tokens each): forced halves [f0, f1) of the
  // pair's forced items, then selected halves [s0, s1) of its selected items.
  // Each workgroup of a pair takes an even share of the forced and of the
  // selected half items; inside it the forced ones go in runs to its first
  // kW - 1 waves (the last wave issues no forced load ahead of the selection)
  // and the selected ones are split over all its waves.  With the workgroup
  // selection (PL < 0) the pair's waves take runs of fh / sh half items
  // instead (measured faster there: the selection, not the loads, sets that
  // step's pace).
  const int nf2 = 2 * (a.n_items - a.top_k), ns2 = 2 * a.top_k;
  int f0, f1, s0, s1;
  if constexpr (PL < 0) {
    f0 = min(wi * a.fh_per_wave, nf2);
    f1 = min(f0 + a.fh_per_wave, nf2);
    s0 = min(wi * a.sh_per_wave, ns2);
    s1 = min(s0 + a.sh_per_wave, ns2);
  } else {
    const int M = a.n_merge, wgp = wi / kW, wv = wi % kW;
    const int F0 = nf2 * wgp / M, nF = nf2 * (wgp + 1) / M - F0;
    const int S0 = ns2 * wgp / M, nS = ns2 * (wgp + 1) / M - S0;
    constexpr int kFw = kW - 1;
    f0 = F0 + (wv < kFw ? nF * wv / kFw : nF);
    f1 = F0 + (wv < kFw ? nF * (wv + 1) / kFw : nF);
    s0 = S0 + nS * wv / kW;
    s1 = S0 + nS * (wv + 1) / kW;
  }
  const int nfh = f1 - f0, n = nfh + (s1 - s0);
  const int fi0 = f0 >> 1, si0 = s0 >> 1;
  const int nfi = nfh > 0 ? ((f1 - 1) >> 1) - fi0 + 1 : 0;

  // Item table, one item per lane: lane j < nfi holds forced item fi0 + j,
  // lane nfi + j selected item si0 + j (at most 64 items per wave).
  int blkv = 0;
  uint64_t maskv = 0ull;
  if (lane < nfi) forced_item(a, fi0 + lane, blkv, maskv);
  auto selected_entries = [&](const int32_t* selrow) {
    const int it = si0 + lane - nfi;
    if (lane >= nfi && it < a.top_k && s1 > s0) selected_item(a, selrow[it], blkv, maskv);
  };
  if constexpr (PL == 0) selected_entries(a.sel + (size_t)pair * a.top_k);
  uint32_t mlo = (uint32_t)maskv, mhi = (uint32_t)(maskv >> 32);
  // paged K/V: the pages of lane j's item block (64 / P of them), physical numbers
  int pgv[4] = {0, 0, 0, 0};
  auto item_pages = [&]() __attribute__((always_inline)) {
    if constexpr (PAGED) {
      const int spb = kBlock >> a.paged.page_shift;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (s < spb) {
          const int p = a.paged.block_table[(size_t)b * a.paged.max_pages + min(blkv * spb + s, a.paged.max_pages - 1)];
          pgv[s] = min(max(p, 0), a.paged.n_pages - 1);
        }
    }
  };
  item_pages();

  // Q^T operand: lane (h, grp) holds Q[h][32dc + 8grp .. +8] (zero rows past G)
  u32x4 qop[DC];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.Q) + ((size_t)b * a.n_q_heads + g * G + h) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qop[dc] = h < G ? *reinterpret_cast<const u32x4*>(qrow + 32 * dc + 8 * grp) : u32x4{0u, 0u, 0u, 0u};
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two stages in flight over the wave's half items (stage A: even steps, B:
  // odd).  Loads are issued for every half item (an empty one loads block 0
  // and skips the compute), and every path is written out, so the compiler's
  // waits on the stage registers count exactly the loads issued after them.
  Stage<D> A, B;
  auto load = [&](int hh, Stage<D>& st) {
    int j, odd;
    if (hh < nfh) {
      const int x = f0 + hh;
      j = (x >> 1) - fi0;
      odd = x & 1;
    } else {
      const int x = s0 + (hh - nfh);
      j = nfi + (x >> 1) - si0;
      odd = x & 1;
    }
    const int blk = __builtin_amdgcn_readlane(blkv, j);
    st.hmask = odd ? __builtin_amdgcn_readlane(mhi, j) : __builtin_amdgcn_readlane(mlo, j);
    if constexpr (PAGED)
      load_half_paged<D>(a, g, __builtin_amdgcn_readlane(pgv[0], j), __builtin_amdgcn_readlane(pgv[1], j),
                         __builtin_amdgcn_readlane(pgv[2], j), __builtin_amdgcn_readlane(pgv[3], j),
                         blk * kBlock + 32 * odd, last, st);
    else
      load_half<D>(Kb, Vb, blk * kBlock + 32 * odd, last, st);
  };
  auto comp = [&](const Stage<D>& st) {
    if (st.hmask) compute_half<D>(st, vt, qop, sl2, m_run, l_run, oacc);
  };
  // SC: this wave's 16-block units of the pair's means (unit t = blocks
  // 16 (ST wid + t) .. +15, lane (col, kg) reads dims 32 s + 8 kg .. +7 of block
  // col of the unit; blocks past the last complete one re-read it, unused)
  constexpr int KS = D / 32;
  constexpr int ST = SC ? PL : 1;  // units per wave: 4 waves x PL units x 16 = 64 PL blocks
  __shared__ float s_scores[SC ? 64 * PL : 1];
  u32x4 mv[ST][KS];
  auto issue_means = [&]() __attribute__((always_inline)) {
    if constexpr (SC) {
      const int nb_last = a.forced.n_ctx / kBlock - 1;
      const u32x4* mb = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.mean) +
                                                       (size_t)pair * a.nblk_capacity * D);
#pragma unroll
      for (int t = 0; t < ST; ++t) {
        const int j = min(16 * (ST * wid + t) + h, nb_last);
#pragma unroll
        for (int s = 0; s < KS; ++s) mv[t][s] = mb[(size_t)j * (D / 8) + 4 * s + grp];
      }
    }
  };
  // SC: S^T = Q M^T per unit (lane (col, kg) ends with block col's dot products
  // for heads 4 kg .. +3), scaled; the group score is the log-sum-exp over the
  // G heads; the scores meet in LDS (and the pair's first workgroup writes
  // them out), then every wave takes its PL scores per lane from there
  auto score = [&]() __attribute__((always_inline)) {
    if constexpr (SC) {
      const int NB = a.forced.n_ctx / kBlock;
#pragma unroll
      for (int t = 0; t < ST; ++t) {
        const int j0 = 16 * (ST * wid + t);
        if (j0 < NB) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) acc = mfma16x16x32(as_bf16x8(qop[s]), as_bf16x8(mv[t][s]), acc);
          float sc4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) sc4[i] = acc[i] * a.scale;
          float mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * grp + i < G) mx = fmaxf(mx, sc4[i]);
          if (G > 4) mx = fmaxf(mx, __shfl_xor(mx, 16));
          if (G > 8) mx = fmaxf(mx, __shfl_xor(mx, 32));
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * grp + i < G) sum += __builtin_amdgcn_exp2f((sc4[i] - mx) * kLog2e);
          if (G > 4) sum += __shfl_xor(sum, 16);
          if (G > 8) sum += __shfl_xor(sum, 32);
          const int j = j0 + h;
          // sum >= 1 (the max term is exactly 1): log2 needs no range care
          const float sj = fmaf(__builtin_amdgcn_logf(sum), kLn2, mx);
          if (grp == 0 && j < NB) {
            s_scores[j] = sj;
            if (wi < kW && a.scores_out != nullptr) a.scores_out[(size_t)pair * a.nblk_capacity + j] = sj;
          }
        }
      }
      __syncthreads();
      const int per = (NB + 64 * kW - 1) / (64 * kW);
      wj0 = min((int)threadIdx.x * per, NB);
      wj1 = min(wj0 + per, NB);
#pragma unroll
      for (int t = 0; t < KPT; ++t) wkey[t] = order_key(s_scores[min(wj0 + t, NB - 1)]);
    }
  };
  // fused step: select the pair's blocks (table in this wave's V tile, which
  // the first compute overwrites), write them out from the pair's first wave
  // and fill the selected half of the item table
  __shared__ WgTopkLds wg_lds;  // (PL < 0 only; unused LDS objects are not allocated)
  __shared__ int32_t wg_tab[PL < 0 || SC ? kFusedMaxTopK : 1];
  auto select = [&]() __attribute__((always_inline)) {
    if constexpr (PL < 0 || SC) {
      wg_topk<KPT>(a, wkey, wj0, wj1, wg_lds, wg_tab);
      if (wi < kW)
        for (int i = threadIdx.x; i < a.top_k; i += 64 * kW) a.sel_out[(size_t)pair * a.top_k + i] = wg_tab[i];
      selected_entries(wg_tab);
      mlo = (uint32_t)maskv;
      mhi = (uint32_t)(maskv >> 32);
      item_pages();
    }
    if constexpr (PL > 0 && !SC) {
      int32_t* tab = reinterpret_cast<int32_t*>(vt + 1024);
      wave_topk<PL>(a, sv, reinterpret_cast<uint32_t*>(vt), tab);
      if (wi == 0)
        for (int i = lane; i < a.top_k; i += 64) a.sel_out[(size_t)pair * a.top_k + i] = tab[i];
      selected_entries(tab);
      mlo = (uint32_t)maskv;
      mhi = (uint32_t)(maskv >> 32);
      item_pages();
    }
  };
  // the first nl (<= 2) loads: on the fused step the forced ones among them
  // go before the scoring and selection (so those overlap their latency), the
  // others after; every path runs score() (its barrier) and select() once
  auto prologue = [&](int nl) __attribute__((always_inline)) {
    if constexpr (PL != 0) {
      issue_means();
      const int pre = min(nfh, nl);
      if (pre >= 1) load(0, A);
      if (pre >= 2) load(1, B);
      score();
      select();
      if (nl >= 1 && pre < 1) load(0, A);
      if (nl >= 2 && pre < 2) load(1, B);
    } else {
      if (nl >= 1) load(0, A);
      if (nl >= 2) load(1, B);
    }
  };

  if (n >= 4) {
    prologue(2);
    int s = 0;
    for (; s + 3 < n; s += 2) {
      comp(A);
      load(s + 2, A);
      comp(B);
      load(s + 3, B);
    }
    if (s + 2 < n) {  // three left: s (A), s + 1 (B), s + 2
      comp(A);
      load(s + 2, A);
      comp(B);
      comp(A);
    } else {  // two left
      comp(A);
      comp(B);
    }
  } else if (n == 3) {
    prologue(2);
    comp(A);
    load(2, A);
    comp(B);
    comp(A);
  } else if (n == 2) {
    prologue(2);
    comp(A);
    comp(B);
  } else if (n == 1) {
    prologue(1);
    comp(A);
  } else {
    prologue(0);  // nothing to attend; the pair's first wave still writes the selection
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  // The workgroup's four waves (one pair) merge in LDS: each wave's numerator
  // over its own V tile (16 heads x d floats fill the 64 d bytes exactly), its
  // max and normaliser beside.
  __shared__ float wml[kW][2][16];
  float* const wo = reinterpret_cast<float*>(vt);
  if (h < G) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(wo + h * D + 16 * dt + 4 * grp) = oacc[dt];
    if (grp == 0) {
      wml[wid][0][h] = m_run;
      wml[wid][1][h] = l_run;
    }
  }
  __syncthreads();
  const int n_wg = a.n_merge, wgi = wi / kW;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * kW) {
    const int hh = idx / D, dd = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kW; ++w) M = fmaxf(M, wml[w][0][hh]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const float mw = wml[w][0][hh];
        const float sc = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L = fmaf(sc, wml[w][1][hh], L);
        O = fmaf(sc, reinterpret_cast<const float*>(smem + w * H::TILE)[hh * D + dd], O);
      }
    }
    const size_t qrow = (size_t)b * a.n_q_heads + g * G + hh;
    if (n_wg == 1) {
      a.O[qrow * D + dd] = L > 0.f ? O / L : 0.f;
      if (a.lse != nullptr && dd == 0) a.lse[qrow] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    } else {
      const size_t prow = qrow * n_wg + wgi;
      a.part_o[prow * D + dd] = O;
      if (dd == 0) {
        a.part_ml[2 * prow] = M;
        a.part_ml[2 * prow + 1] = L;
      }
    }
  }
}

// fp32 K/V: one token per lane, VALU dot products.  GM >= G is the padded group size.
// FUSED (the one-call step on a small fp32 problem, one workgroup per pair):
// the workgroup first scores its pair's complete blocks from the fp32 means,
// one block per thread (the selector's first-order score, COBS explainer
// technical summary sections 2.1-2.2: the group log-sum-exp of the scaled
// q . mean), writes them to scores_out, and takes the top-k itself (wg_topk:
// score descending, then block index ascending, the top-k kernel's order),
// which it writes to sel_out and attends.
template <int D, int GM, bool FUSED = false>
__global__ __launch_bounds__(64 * kW) void decode_f32_kernel(DecodeArgs a) {
  constexpr int DL = D / 64;  // output dims per lane
  __shared__ __attribute__((aligned(16))) float qs[GM][D];
  __shared__ float ps[kW][GM][64];
  __shared__ __attribute__((aligned(16))) uint8_t mbuf[sizeof(MergeLds<D>)];
  __shared__ int32_t s_sel[kMaxTopK];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, g = bh % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const float* Kb = reinterpret_cast<const float*>(a.K) + (size_t)bh * a.kv_capacity * D;
  const float* Vb = reinterpret_cast<const float*>(a.V) + (size_t)bh * a.kv_capacity * D;
  if constexpr (!FUSED)
    for (int i = tid; i < a.top_k; i += 64 * kW) s_sel[i] = a.sel[(size_t)bh * a.top_k + i];
  const float sl2 = a.scale * kLog2e;
  for (int i = tid; i < GM * D; i += 64 * kW)
    qs[i / D][i % D] =
        (i / D < G) ? reinterpret_cast<const float*>(a.Q)[((size_t)b * a.n_q_heads + g * G) * D + i] : 0.f;
  __syncthreads();
  if constexpr (FUSED) {
    __shared__ WgTopkLds wl;
    const int NB = a.forced.n_ctx / kBlock;  // <= 64 * kW (host check)
    const int j = tid;
    uint32_t key[1] = {0u};
    if (j < NB) {
      const float4* mr =
          reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.mean) + ((size_t)bh * a.nblk_capacity + j) * D);
      float4 mv[D / 4];
#pragma unroll
      for (int c = 0; c < D / 4; ++c) mv[c] = mr[c];
      float sc[GM];
      float mx = -INFINITY;
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
          const float4 q4 = reinterpret_cast<const float4*>(qs[hh])[c];
          acc = fmaf(mv[c].x, q4.x, acc);
          acc = fmaf(mv[c].y, q4.y, acc);
          acc = fmaf(mv[c].z, q4.z, acc);
          acc = fmaf(mv[c].w, q4.w, acc);
        }
        sc[hh] = acc * a.scale;
        if (hh < G) mx = fmaxf(mx, sc[hh]);
      }
      float sum = 0.f;
#pragma unroll
      for (int hh = 0; hh < GM; ++hh)
        if (hh < G) sum += __builtin_amdgcn_exp2f((sc[hh] - mx) * kLog2e);
      // sum >= 1 (the max term is exactly 1): log2 needs no range care
      const float score = fmaf(__builtin_amdgcn_logf(sum), kLn2, mx);
      if (a.scores_out != nullptr) a.scores_out[(size_t)bh * a.nblk_capacity + j] = score;
      key[0] = order_key(score);
    }
    wg_topk<1>(a, key, min(j, NB), min(j + 1, NB), wl, s_sel);  // ends at a barrier
    for (int i = tid; i < a.top_k; i += 64 * kW) a.sel_out[(size_t)bh * a.top_k + i] = s_sel[i];
  }
  float m_run[GM], l_run[GM], o[GM][DL];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) o[hh][e] = 0.f;
  }
  const int it0 = (blockIdx.x * kW + wid) * a.per_wave;
  const int it1 = min(it0 + a.per_wave, a.n_items);
  const int last = a.forced.n_ctx - 1;  // rows are clamped into the context; masked tokens weigh 0
  for (int it = it0; it < it1; ++it) {
    const ItemInfo inf = item_info(a, s_sel, it);
    if (inf.blk < 0) continue;
    const bool on = (inf.mask >> lane) & 1ull;
    // this lane's K row, loaded once (whole row in flight), then one dot
    // product per query head from registers; at d = 64 the item's 64 V rows
    // are loaded with it (V does not wait for the weights), so an item costs
    // one round trip to memory (at d = 128 the K row alone takes 128 registers
    // and V follows the weights, 16 rows at a time)
    const float4* kr = reinterpret_cast<const float4*>(Kb + (size_t)min(inf.blk * kBlock + lane, last) * D);
    float4 kv[D / 4];
#pragma unroll
    for (int c = 0; c < D / 4; ++c) kv[c] = kr[c];
    constexpr bool EARLY_V = D == 64;
    constexpr int VB = EARLY_V ? 64 : 16;  // V rows per batch: 64 / 32 registers
    float vv[VB][DL];
    auto load_v = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < VB; ++u) {
        const float* vr = Vb + (size_t)min(inf.blk * kBlock + t0 + u, last) * D;
#pragma unroll
        for (int e = 0; e < DL; ++e) vv[u][e] = vr[lane + 64 * e];
      }
    };
    if constexpr (EARLY_V) load_v(0);
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      if (hh >= G) break;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D / 4; ++c) {
        const float4 q4 = reinterpret_cast<const float4*>(qs[hh])[c];
        acc = fmaf(kv[c].x, q4.x, acc);
        acc = fmaf(kv[c].y, q4.y, acc);
        acc = fmaf(kv[c].z, q4.z, acc);
        acc = fmaf(kv[c].w, q4.w, acc);
      }
      const float lg = on ? acc * sl2 : -INFINITY;
      const float mx = wave_max(lg);
      const float m_new = fmaxf(m_run[hh], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run[hh] - m_use);
      const float p = on ? exp2f(lg - m_use) : 0.f;
      l_run[hh] = l_run[hh] * alpha + wave_sum(p);
      m_run[hh] = m_new;
#pragma unroll
      for (int e = 0; e < DL; ++e) o[hh][e] *= alpha;
      ps[wid][hh][lane] = p;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // O += P V over the block's 64 rows, VB rows at a time (a masked token's
    // weight is 0)
#pragma unroll
    for (int t0 = 0; t0 < 64; t0 += VB) {
      if (!EARLY_V || t0 > 0) load_v(t0);
#pragma unroll
      for (int u = 0; u < VB; ++u)
#pragma unroll
        for (int e = 0; e < DL; ++e)
#pragma unroll
          for (int hh = 0; hh < GM; ++hh) o[hh][e] = fmaf(ps[wid][hh][t0 + u], vv[u][e], o[hh][e]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  MergeLds<D>* ml = reinterpret_cast<MergeLds<D>*>(mbuf);
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    if (hh >= G) break;
    if (lane == 0) {
      ml->m[wid][hh] = m_run[hh];
      ml->l[wid][hh] = l_run[hh];
    }
#pragma unroll
    for (int e = 0; e < DL; ++e) ml->o[wid][hh][lane + 64 * e] = o[hh][e];
  }
  __syncthreads();
  write_wg_result<D>(a, ml, b, g);
}

// Merge the partials of every query head: per dim,
// O = sum_s w_s o_s / sum_s w_s l_s with w_s = 2^(m_s - M); lse = ln 2 (M + log2 L).
// One wave per (b, query head); lane owns dims lane + 64e; the partials are read
// CH at a time (all loads of a chunk in flight together; CH the smallest of 2,
// 4, 8, 16, 32 that holds them all, else 32) and folded online.
template <int D, int CH>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int DL = D / 64;
  const size_t qrow = blockIdx.x;  // b * Hq + h
  const int lane = threadIdx.x;
  const int n = a.n_merge;
  const float* pml = a.part_ml + qrow * n * 2;
  const float* po = a.part_o + qrow * n * D + lane;
  float M = -INFINITY, L = 0.f, O[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) O[e] = 0.f;
  for (int j0 = 0; j0 < n; j0 += CH) {
    float ms[CH], ls[CH], os[CH][DL];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int j = min(j0 + u, n - 1);
      ms[u] = j0 + u < n ? pml[2 * j] : -INFINITY;
      ls[u] = pml[2 * j + 1];
#pragma unroll
      for (int e = 0; e < DL; ++e) os[u][e] = po[(size_t)j * D + 64 * e];
    }
    float cm = M;
#pragma unroll
    for (int u = 0; u < CH; ++u) cm = fmaxf(cm, ms[u]);
    if (cm == -INFINITY) continue;
    const float c0 = M == -INFINITY ? 0.f : exp2f(M - cm);
    L *= c0;
#pragma unroll
    for (int e = 0; e < DL; ++e) O[e] *= c0;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const float w = ms[u] == -INFINITY ? 0.f : exp2f(ms[u] - cm);
      L = fmaf(w, ls[u], L);
#pragma unroll
      for (int e = 0; e < DL; ++e) O[e] = fmaf(w, os[u][e], O[e]);
    }
    M = cm;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int e = 0; e < DL; ++e) a.O[qrow * D + lane + 64 * e] = O[e] * inv;
  if (a.lse != nullptr && lane == 0) a.lse[qrow] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int n_pairs = a.batch * a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  if (a.bf16) {
    const long long waves = (long long)n_pairs * a.n_part;
    const dim3 grid((unsigned)((waves + kW - 1) / kW)), block(64 * kW);
    if (a.paged.block_table != nullptr) {
      if (a.key_slots == 0) hipLaunchKernelGGL((decode_bf16_kernel<D, 0, true>), grid, block, 0, stream, a);
      else if (a.key_slots < 0) hipLaunchKernelGGL((decode_bf16_kernel<D, -8, true>), grid, block, 0, stream, a);
      else if (a.mean != nullptr) hipLaunchKernelGGL((decode_bf16_kernel<D, 8, true, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((decode_bf16_kernel<D, 8, true>), grid, block, 0, stream, a);
    } else {
      if (a.key_slots == 0) hipLaunchKernelGGL((decode_bf16_kernel<D, 0, false>), grid, block, 0, stream, a);
      else if (a.key_slots < 0) hipLaunchKernelGGL((decode_bf16_kernel<D, -8, false>), grid, block, 0, stream, a);
      else if (a.mean != nullptr) hipLaunchKernelGGL((decode_bf16_kernel<D, 8, false, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((decode_bf16_kernel<D, 8, false>), grid, block, 0, stream, a);
    }
  } else {
    const dim3 grid(a.n_part, n_pairs);
    const bool fz = a.mean != nullptr;  // the fused fp32 step (one workgroup per pair)
    if (G <= 4) {
      if (fz) hipLaunchKernelGGL((decode_f32_kernel<D, 4, true>), grid, dim3(64 * kW), 0, stream, a);
      else hipLaunchKernelGGL((decode_f32_kernel<D, 4>), grid, dim3(64 * kW), 0, stream, a);
    } else if (G <= 8) {
      if (fz) hipLaunchKernelGGL((decode_f32_kernel<D, 8, true>), grid, dim3(64 * kW), 0, stream, a);
      else hipLaunchKernelGGL((decode_f32_kernel<D, 8>), grid, dim3(64 * kW), 0, stream, a);
    } else {
      if (fz) hipLaunchKernelGGL((decode_f32_kernel<D, 16, true>), grid, dim3(64 * kW), 0, stream, a);
      else hipLaunchKernelGGL((decode_f32_kernel<D, 16>), grid, dim3(64 * kW), 0, stream, a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_merge == 1) return e;
  const dim3 mg(a.batch * a.n_q_heads), mb(64);
  if (a.n_merge <= 2) hipLaunchKernelGGL((decode_merge_kernel<D, 2>), mg, mb, 0, stream, a);
  else if (a.n_merge <= 4) hipLaunchKernelGGL((decode_merge_kernel<D, 4>), mg, mb, 0, stream, a);
  else if (a.n_merge <= 8) hipLaunchKernelGGL((decode_merge_kernel<D, 8>), mg, mb, 0, stream, a);
  else if (a.n_merge <= 16) hipLaunchKernelGGL((decode_merge_kernel<D, 16>), mg, mb, 0, stream, a);
  else hipLaunchKernelGGL((decode_merge_kernel<D, 32>), mg, mb, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// bf16: n_part waves per pair, a multiple of kW (a workgroup's waves share one
// pair and merge in LDS): as many as keep every wave resident at once
// (decode_slots(d) waves over all pairs), at most one per half item and at
// least kW; `half_items` = c = ceil(2 n_items / n_part).  The caller gives each
// wave ceil(2 forced / n_part) forced and ceil(2 top_k / n_part) selected half
// items, at most c + 2 half items spanning at most c / 2 + 3 items, so c <= 120
// (n_part grows past the resident waves when it must) keeps a wave's items
// within one per lane.  fp32: one whole item per wave, 4 waves per workgroup
// merged in LDS, one partial per workgroup.
void decode_split_geometry(int n_items, int n_pairs, int head_dim, bool bf16, int* half_items, int* n_part) {
  if (n_items <= 0 || n_pairs <= 0) {
    *half_items = 1;
    *n_part = bf16 ? kW : 1;
    return;
  }
  if (!bf16) {
    *half_items = 1;
    *n_part = (n_items + kW - 1) / kW;
    return;
  }
  const long long slots = decode_slots(head_dim);
  const long long n_sub = 2LL * n_items;
  long long np = slots / n_pairs / kW * kW;
  const long long cap = (n_sub + kW - 1) / kW * kW;
  if (np > cap) np = cap;
  if (np < kW) np = kW;
  long long c = (n_sub + np - 1) / np;
  if (c > 120) {
    c = 120;
    np = ((n_sub + c - 1) / c + kW - 1) / kW * kW;
  }
  *half_items = (int)c;
  *n_part = (int)np;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_t<64>(a, stream) : launch_t<128>(a, stream);
}

// Scratch of the allocation-free decode step: the split partials live in this
// file-scope device array instead of a caller workspace.  A __device__ variable
// exists once per device the code object is loaded on, at that device's own
// address; host code must never pass the array's name to a kernel (in host code
// it is only a stand-in for the symbol), only the address hipGetSymbolAddress
// returns for the current device, looked up once per device and kept.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace bsattn
