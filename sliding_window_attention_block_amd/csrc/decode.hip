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
// the forced blocks.  A forced block that is also selected is skipped (the
// selected block already covers every token of it); a forced block only
// contributes its forced tokens.
//
// Grid: (workgroups per pair, B * Hkv).  A workgroup has 4 waves; each wave
// owns `items_per_wave` consecutive items.  The 4 waves merge in LDS into one
// partial per workgroup.  With one workgroup per pair the kernel writes O and
// lse itself; otherwise a small second kernel merges the partials (the kernel
// boundary makes every workgroup's partial visible without any L2 write-back
// inside the hot kernel; the L2s of the 8 XCDs are not coherent with each other).
//
// bf16 path (MFMA, gfx950 v_mfma_f32_16x16x32_bf16), per 64-token item:
//   V is copied HBM -> LDS with global_load_lds_dwordx4 (no registers), into
//   a per-wave tile with XOR-swizzled 16-byte chunks; K goes straight from HBM
//   into MFMA A-operand registers.  All of an item's loads are issued at once.
//   S^T = K Q^T: B = Q^T held in registers (16 query heads of the group, zero
//   padded), so lane l holds the logits of query head l%16 for 16 tokens.
//   O^T += V^T P^T: V^T read with ds_read_b64_tr_b16.  P = P_hi + P_lo in
//   bf16 (two products), so the result keeps ~2^-17 of P's precision.  The
//   output tile keeps query head l%16 in lane l, so the rescale is per lane.
// fp32 path (VALU): one token per lane, used when K/V are fp32.
#include "launch.hpp"

namespace bsattn {
namespace {

constexpr int kW = kDecodeWaves;

struct ItemInfo {
  int blk;
  uint64_t mask;
};

// Number of leading non-negative entries of an ascending, -1-padded row.
__device__ __forceinline__ int valid_prefix(const int32_t* sel, int k) {
  int lo = 0, hi = k;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sel[mid] >= 0) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ bool in_sorted(const int32_t* a, int n, int x) {
  const int i = lower_bound_i32(a, n, x);
  return i < n && a[i] == x;
}

// Block and token mask of item `it`; blk < 0 means nothing to do.
__device__ __forceinline__ ItemInfo item_info(const DecodeArgs& a, const int32_t* selrow, int nsel,
                                              int it) {
  ItemInfo r;
  if (it < a.top_k) {
    const int blk = selrow[it];
    // only complete blocks can be selected; anything else is ignored
    r.blk = (blk >= 0 && blk < a.forced.n_ctx / kBlock) ? blk : -1;
    r.mask = ~0ull;
    return r;
  }
  const int f = it - a.top_k;
  const ForcedBlocks& fb = a.fblocks;
  int blk;
  if (f < fb.r0_n) blk = fb.r0_lo + f;
  else if (f < fb.r0_n + fb.r1_n) blk = fb.r1_lo + (f - fb.r0_n);
  else blk = fb.gblk[f - fb.r0_n - fb.r1_n];
  if (in_sorted(selrow, nsel, blk)) { r.blk = -1; r.mask = 0; return r; }
  r.blk = blk;
  r.mask = forced_mask(a.forced, blk);
  if (r.mask == 0ull) r.blk = -1;
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
  const int n_wg = a.n_wg, wg = blockIdx.x;
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

// One wave handles one half of an item (32 tokens): small per-wave footprint (8 KB
// of V in LDS, K in 32 registers) so 16 waves fit on a CU and keep loads in flight
// while others compute.  Sub-item s is half s % 2 of item s / 2.
template <int D>
__global__ __launch_bounds__(64 * kW, 4) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int DC = D / 32;              // d chunks per QK MFMA row
  constexpr int DT = D / 16;              // output d tiles
  constexpr int TILE = 32 * D * 2;        // V of one half item
  constexpr int NCH = TILE / 1024;        // 1 KB LDS-DMA instructions per half item
  constexpr int SEL_OFF = kW * TILE;      // the sel row lives after the V tiles
  constexpr int LDS = SEL_OFF + kMaxTopK * 4;
  static_assert(sizeof(MergeLds<D>) <= LDS, "merge buffer overlays the V tiles and sel row");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  int32_t* s_sel = reinterpret_cast<int32_t*>(smem + SEL_OFF);

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, g = bh % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int h = lane & 15, grp = lane >> 4;
  uint8_t* vt = smem + wid * TILE;
  typedef __attribute__((address_space(3))) void lds_void;

  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.K) + (size_t)bh * a.kv_capacity * D;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(a.V) + (size_t)bh * a.kv_capacity * D;
  // the pair's selected blocks, staged once in LDS (every search below reads LDS)
  for (int i = threadIdx.x; i < a.top_k; i += 64 * kW) s_sel[i] = a.sel[(size_t)bh * a.top_k + i];
  __syncthreads();
  const int nsel = valid_prefix(s_sel, a.top_k);

  const float sl2 = a.scale * kLog2e;
  const int last = a.forced.n_ctx - 1;  // rows past the context (tail block) are masked; clamp loads
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int s0 = (blockIdx.x * kW + wid) * a.items_per_wave;
  const int s1 = min(s0 + a.items_per_wave, 2 * a.n_items);
  for (int sub = s0; sub < s1; ++sub) {
    const ItemInfo inf = item_info(a, s_sel, nsel, sub >> 1);
    const int half = sub & 1;
    const uint32_t hmask = (uint32_t)(inf.mask >> (32 * half));
    if (inf.blk < 0 || hmask == 0u) continue;  // same value in every lane
    const int tok0 = inf.blk * kBlock + 32 * half;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // previous V reads done
    // V: HBM -> LDS.  Instruction k fills tile bytes [1024k, 1024k + 1024); lane l's
    // 16 bytes land at 1024k + 16l, i.e. physical chunk pc of row r, which holds
    // logical chunk pc ^ swz(r).
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int off = 1024 * k + 16 * lane;
      const int r = off / (D * 2), pc = (off % (D * 2)) >> 4;
      const int c = pc ^ v_swz<D>(r);
      const size_t row = (size_t)min(tok0 + r, last);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(Vb + row * D + c * 8),
                                       (lds_void*)(vt + 1024 * k), 16, 0, 0);
    }
    // K operands straight from HBM
    u32x4 kop[2][DC];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const size_t row = (size_t)min(tok0 + 16 * tt + h, last);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        kop[tt][dc] = *reinterpret_cast<const u32x4*>(Kb + row * D + 32 * dc + 8 * grp);
    }
    // Q^T operand: lane (h, grp) holds Q[h][32*dc + 8*grp .. +8] (reloaded per sub-item:
    // an L2 hit, and it keeps 16 registers free across the loop)
    u32x4 qop[DC];
    {
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.Q) + ((size_t)b * a.n_q_heads + g * G + h) * D;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        qop[dc] = h < G ? *reinterpret_cast<const u32x4*>(qrow + 32 * dc + 8 * grp) : u32x4{0u, 0u, 0u, 0u};
    }
    // logits
    f32x4 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) s[tt] = mfma16x16x32(as_bf16x8(kop[tt][dc]), as_bf16x8(qop[dc]), s[tt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = 16 * tt + 4 * grp + r;
        const float v = ((hmask >> tok) & 1u) ? s[tt][r] * sl2 : -INFINITY;
        s[tt][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    // P = P_hi + P_lo, both bf16: the second PV product (free: decode is bound by
    // HBM) keeps the result exact to ~2^-17 of P however few tokens a head sees.
    u32x4 pop, plo;
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = exp2f(s[tt][r] - m_use), p1 = exp2f(s[tt][r + 1] - m_use);
        const uint32_t pk = pack_bf16x2(p0, p1);
        pop[2 * tt + r / 2] = pk;
        plo[2 * tt + r / 2] = pack_bf16x2(p0 - bf16lo(pk), p1 - bf16hi(pk));
        psum += p0 + p1;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // V tile landed in LDS
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
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();  // every wave done with its V tile and the sel row
  MergeLds<D>* ml = reinterpret_cast<MergeLds<D>*>(smem);
  if (grp == 0) {
    ml->m[wid][h] = m_run;
    ml->l[wid][h] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(&ml->o[wid][h][16 * dt + 4 * grp]) = oacc[dt];
  __syncthreads();
  write_wg_result<D>(a, ml, b, g);
}

// fp32 K/V: one token per lane, VALU dot products.  GM >= G is the padded group size.
template <int D, int GM>
__global__ __launch_bounds__(64 * kW) void decode_f32_kernel(DecodeArgs a) {
  constexpr int DL = D / 64;  // output dims per lane
  __shared__ float qs[GM][D];
  __shared__ float ps[kW][GM][64];
  __shared__ __attribute__((aligned(16))) uint8_t mbuf[sizeof(MergeLds<D>)];
  __shared__ int32_t s_sel[kMaxTopK];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, g = bh % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const float* Kb = reinterpret_cast<const float*>(a.K) + (size_t)bh * a.kv_capacity * D;
  const float* Vb = reinterpret_cast<const float*>(a.V) + (size_t)bh * a.kv_capacity * D;
  for (int i = tid; i < a.top_k; i += 64 * kW) s_sel[i] = a.sel[(size_t)bh * a.top_k + i];
  const float sl2 = a.scale * kLog2e;
  for (int i = tid; i < GM * D; i += 64 * kW)
    qs[i / D][i % D] =
        (i / D < G) ? reinterpret_cast<const float*>(a.Q)[((size_t)b * a.n_q_heads + g * G) * D + i] : 0.f;
  __syncthreads();
  const int nsel = valid_prefix(s_sel, a.top_k);
  float m_run[GM], l_run[GM], o[GM][DL];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) o[hh][e] = 0.f;
  }
  const int it0 = (blockIdx.x * kW + wid) * a.items_per_wave;
  const int it1 = min(it0 + a.items_per_wave, a.n_items);
  for (int it = it0; it < it1; ++it) {
    const ItemInfo inf = item_info(a, s_sel, nsel, it);
    if (inf.blk < 0) continue;
    const size_t tok = (size_t)inf.blk * kBlock + lane;
    const bool on = (inf.mask >> lane) & 1ull;
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      if (hh >= G) break;
      float acc = 0.f;
      if (on) {
        const float4* kr = reinterpret_cast<const float4*>(Kb + tok * D);
        for (int c = 0; c < D / 4; ++c) {
          const float4 kv = kr[c];
          acc = fmaf(kv.x, qs[hh][4 * c], acc);
          acc = fmaf(kv.y, qs[hh][4 * c + 1], acc);
          acc = fmaf(kv.z, qs[hh][4 * c + 2], acc);
          acc = fmaf(kv.w, qs[hh][4 * c + 3], acc);
        }
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
    for (int t = 0; t < 64; ++t) {
      if (!((inf.mask >> t) & 1ull)) continue;
      const float* vr = Vb + ((size_t)inf.blk * kBlock + t) * D;
#pragma unroll
      for (int e = 0; e < DL; ++e) {
        const float v = vr[lane + 64 * e];
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) o[hh][e] = fmaf(ps[wid][hh][t], v, o[hh][e]);
      }
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

// Merge the workgroup partials of every query head: per dim,
// O = sum_s w_s o_s / sum_s w_s l_s with w_s = 2^(m_s - M); lse = ln 2 (M + log2 L).
// One workgroup of D threads per (b, query head); 8 partial loads in flight per thread.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  const size_t qrow = blockIdx.x;  // b * Hq + h
  const int dd = threadIdx.x;
  const int n_wg = a.n_wg;
  const float* pml = a.part_ml + qrow * n_wg * 2;
  const float* po = a.part_o + qrow * n_wg * D + dd;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int s0 = 0; s0 < n_wg; s0 += 8) {
    float ms[8], ls[8], os[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u;
      ms[u] = s < n_wg ? pml[2 * s] : -INFINITY;
      ls[u] = s < n_wg ? pml[2 * s + 1] : 0.f;
      os[u] = s < n_wg ? po[(size_t)s * D] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (ms[u] == -INFINITY) continue;
      const float Mn = fmaxf(M, ms[u]);
      const float c0 = exp2f(M - Mn), c1 = exp2f(ms[u] - Mn);
      L = L * c0 + ls[u] * c1;
      O = O * c0 + os[u] * c1;
      M = Mn;
    }
  }
  a.O[qrow * D + dd] = L > 0.f ? O / L : 0.f;
  if (a.lse != nullptr && dd == 0) a.lse[qrow] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.n_wg, a.batch * a.n_kv_heads);
  const int G = a.n_q_heads / a.n_kv_heads;
  if (a.bf16)
    hipLaunchKernelGGL((decode_bf16_kernel<D>), grid, dim3(64 * kW), 0, stream, a);
  else if (G <= 4)
    hipLaunchKernelGGL((decode_f32_kernel<D, 4>), grid, dim3(64 * kW), 0, stream, a);
  else if (G <= 8)
    hipLaunchKernelGGL((decode_f32_kernel<D, 8>), grid, dim3(64 * kW), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_f32_kernel<D, 16>), grid, dim3(64 * kW), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_wg == 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.batch * a.n_q_heads), dim3(D), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// bf16: a wave takes `items_per_wave` half items (32 tokens each); fp32: whole items.
// One geometry serves both, sized for the finer bf16 split.
void decode_split_geometry(int n_items, int* items_per_wave, int* n_wg) {
  const int ipw = 1;
  *items_per_wave = ipw;
  const int per_wg = ipw * kW;
  *n_wg = n_items > 0 ? (2 * n_items + per_wg - 1) / per_wg : 1;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_t<64>(a, stream) : launch_t<128>(a, stream);
}

}  // namespace bsattn
