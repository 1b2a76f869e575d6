// Sparse flash-decode over the selected blocks plus the forced tokens
// (window, sinks, globals), split over workgroups, then a log-sum-exp merge.
//
// What is computed: one softmax per query head over the token set
// T = forced tokens  union  tokens of the selected blocks (a set: a token
// reached two ways is attended once), as the COBS explainer's technical
// summary describes block-sparse decode (sections 1 and 2.1: read only the
// chosen contiguous blocks) with the sliding window and sink tokens of the
// SWA glossary ("SWAの拡張手法") and the global tokens of the local-global
// glossary.  The split-and-merge uses the online-softmax identity: partial
// (m, l, o) over disjoint token sets merge exactly by rescaling with exp(m - M).
//
// Work items: per (b, K/V head) the list is the top_k selected blocks, then
// the forced blocks.  A forced block that is also selected is skipped (the
// selected block already covers every token of it); a forced block only
// contributes its forced tokens.  Each wave owns `items_per_split` items.
//
// bf16 path (MFMA, gfx950 v_mfma_f32_16x16x32_bf16), per 64-token item:
//   S^T = K Q^T: A = K rows straight from HBM (16-byte loads), B = Q^T held in
//   registers (16 query heads of the group, zero padded).  Lane l then holds
//   the logits of query head l%16 for 16 tokens.
//   O^T += V^T P^T: V goes to a per-wave LDS tile (XOR-swizzled 16-byte chunks)
//   and is read back transposed with ds_read_b64_tr_b16; P^T is the softmax
//   numerator of the lane's own logits, rounded to bf16.  The output tile
//   keeps query head l%16 in lane l, so the online-softmax rescale is per lane.
// fp32 path (VALU): one token per lane, used when K/V are fp32.
#include "launch.hpp"

namespace bsattn {
namespace {

constexpr int kWavesPerWg = 2;

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

// Swizzled byte offset of 16-byte chunk `c` of V row `r` in a per-wave tile.
template <int D>
__device__ __forceinline__ uint32_t v_off(int r, int c) {
  constexpr int RB = D * 2;        // bytes per row
  constexpr int RPL = 256 / RB;    // rows per 256-byte bank line
  constexpr int NX = 8 / RPL;      // distinct swizzle values
  const int f = 2 * ((r / RPL) & (NX - 1));
  return (uint32_t)(r * RB + ((c ^ f) << 4));
}

template <int D>
__global__ __launch_bounds__(64 * kWavesPerWg) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int DC = D / 32;  // d chunks per QK MFMA row
  constexpr int DT = D / 16;  // output d tiles
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint8_t vtile[kWavesPerWg][64 * D * 2];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int split = blockIdx.x * kWavesPerWg + wid;
  if (split >= a.n_split) return;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, g = bh % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int h = lane & 15, grp = lane >> 4;
  const uint8_t* vt = vtile[wid];

  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.K) + (size_t)bh * a.kv_capacity * D;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(a.V) + (size_t)bh * a.kv_capacity * D;
  const int32_t* selrow = a.sel + (size_t)bh * a.top_k;
  const int nsel = valid_prefix(selrow, a.top_k);

  // Q^T operand: lane (h, grp) holds Q[h][32*dc + 8*grp .. +8]
  u32x4 qop[DC];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.Q) + ((size_t)b * a.n_q_heads + g * G + h) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      if (h < G) qop[dc] = *reinterpret_cast<const u32x4*>(qrow + 32 * dc + 8 * grp);
      else qop[dc] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  const float sl2 = a.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int it0 = split * a.items_per_split;
  const int it1 = min(it0 + a.items_per_split, a.n_items);
  for (int it = it0; it < it1; ++it) {
    const ItemInfo inf = item_info(a, selrow, nsel, it);
    if (inf.blk < 0) continue;  // wave-uniform
    const int tok0 = inf.blk * kBlock;
    const int last = a.forced.n_ctx - 1;  // rows past the context (tail block) are masked; clamp loads
    // K operands straight from HBM
    u32x4 kop[4][DC];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const size_t row = (size_t)min(tok0 + 16 * tt + h, last);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        kop[tt][dc] = *reinterpret_cast<const u32x4*>(Kb + row * D + 32 * dc + 8 * grp);
    }
    // V -> registers -> swizzled LDS tile
    u32x4 vreg[CPR];
#pragma unroll
    for (int k = 0; k < CPR; ++k) {
      const int c = lane + 64 * k;
      const size_t row = (size_t)min(tok0 + c / CPR, last);
      vreg[k] = *reinterpret_cast<const u32x4*>(Vb + row * D + (c % CPR) * 8);
    }
    // logits
    f32x4 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) s[tt] = mfma16x16x32(as_bf16x8(kop[tt][dc]), as_bf16x8(qop[dc]), s[tt]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // previous item's tr reads done
#pragma unroll
    for (int k = 0; k < CPR; ++k) {
      const int c = lane + 64 * k;
      *reinterpret_cast<u32x4*>(vtile[wid] + v_off<D>(c / CPR, c % CPR)) = vreg[k];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = 16 * tt + 4 * grp + r;
        const float v = ((inf.mask >> tok) & 1ull) ? s[tt][r] * sl2 : -INFINITY;
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
    u32x4 pop[2], plo[2];
    float psum = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const float p0 = exp2f(s[2 * c + half][r] - m_use), p1 = exp2f(s[2 * c + half][r + 1] - m_use);
          const uint32_t pk = pack_bf16x2(p0, p1);
          pop[c][2 * half + r / 2] = pk;
          plo[c][2 * half + r / 2] = pack_bf16x2(p0 - bf16lo(pk), p1 - bf16hi(pk));
          psum += p0 + p1;
        }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // V tile written
    // O^T += V^T P^T.  Lane a of 16-lane group q reads 8 bytes of V row
    // 32c + 4q + a/4 (+16 for the second half), columns 16dt + 4(a%4).
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = 32 * c + 4 * grp + (h >> 2);
        const int col = 16 * dt + 4 * (h & 3);  // element index
        const uint32_t o1 = v_off<D>(row, col >> 3) + ((col & 7) << 1);
        const uint32_t o2 = v_off<D>(row + 16, col >> 3) + ((col & 7) << 1);
        const u32x2 lo = lds_read_tr16(vt, o1);
        const u32x2 hi = lds_read_tr16(vt, o2);
        const u32x4 vop = u32x4{lo[0], lo[1], hi[0], hi[1]};
        oacc[dt] = mfma16x16x32(as_bf16x8(vop), as_bf16x8(pop[c]), oacc[dt]);
        oacc[dt] = mfma16x16x32(as_bf16x8(vop), as_bf16x8(plo[c]), oacc[dt]);
      }
    }
  }
  // partial (m, l, o) of this split for the group's query heads
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (h < G) {
    const size_t row = ((size_t)b * a.n_q_heads + g * G + h) * a.n_split + split;
    if (grp == 0) {
      a.part_ml[2 * row] = m_run;
      a.part_ml[2 * row + 1] = l_run;
    }
    float* po = a.part_o + row * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * grp) = oacc[dt];
  }
}

// fp32 K/V: one token per lane, VALU dot products.  GM >= G is the padded group size.
template <int D, int GM>
__global__ __launch_bounds__(64 * kWavesPerWg) void decode_f32_kernel(DecodeArgs a) {
  constexpr int DL = D / 64;  // output dims per lane
  __shared__ float qs[kWavesPerWg][GM][D];
  __shared__ float ps[kWavesPerWg][GM][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int split = blockIdx.x * kWavesPerWg + wid;
  if (split >= a.n_split) return;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, g = bh % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const float* Kb = reinterpret_cast<const float*>(a.K) + (size_t)bh * a.kv_capacity * D;
  const float* Vb = reinterpret_cast<const float*>(a.V) + (size_t)bh * a.kv_capacity * D;
  const int32_t* selrow = a.sel + (size_t)bh * a.top_k;
  const int nsel = valid_prefix(selrow, a.top_k);
  const float sl2 = a.scale * kLog2e;
  for (int i = lane; i < GM * D; i += 64)
    qs[wid][i / D][i % D] =
        (i / D < G) ? reinterpret_cast<const float*>(a.Q)[((size_t)b * a.n_q_heads + g * G) * D + i] : 0.f;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  float m_run[GM], l_run[GM], o[GM][DL];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) o[hh][e] = 0.f;
  }
  const int it0 = split * a.items_per_split;
  const int it1 = min(it0 + a.items_per_split, a.n_items);
  for (int it = it0; it < it1; ++it) {
    const ItemInfo inf = item_info(a, selrow, nsel, it);
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
          acc = fmaf(kv.x, qs[wid][hh][4 * c], acc);
          acc = fmaf(kv.y, qs[wid][hh][4 * c + 1], acc);
          acc = fmaf(kv.z, qs[wid][hh][4 * c + 2], acc);
          acc = fmaf(kv.w, qs[wid][hh][4 * c + 3], acc);
        }
      }
      const float lg = on ? acc * sl2 : -INFINITY;
      const float mx = wave_max(lg);
      const float m_new = fmaxf(m_run[hh], mx);
      const float alpha = (m_run[hh] == -INFINITY) ? 0.f : exp2f(m_run[hh] - m_new);
      const float p = on ? exp2f(lg - m_new) : 0.f;
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
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    if (hh >= G) break;
    const size_t row = ((size_t)b * a.n_q_heads + g * G + hh) * a.n_split + split;
    if (lane == 0) {
      a.part_ml[2 * row] = m_run[hh];
      a.part_ml[2 * row + 1] = l_run[hh];
    }
#pragma unroll
    for (int e = 0; e < DL; ++e) a.part_o[row * D + lane + 64 * e] = o[hh][e];
  }
}

// Merge the splits of every query head: O = sum_s w_s o_s / sum_s w_s l_s with
// w_s = 2^(m_s - M); lse = ln 2 * (M + log2 sum_s w_s l_s).
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int row = blockIdx.x;  // b * Hq + h
  const int t = threadIdx.x;
  const float* ml = a.part_ml + (size_t)row * a.n_split * 2;
  float M = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f, acc = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < a.n_split; ++s) {
      const float m = ml[2 * s];
      if (m == -INFINITY) continue;
      const float w = exp2f(m - M);
      L = fmaf(w, ml[2 * s + 1], L);
      acc = fmaf(w, a.part_o[((size_t)row * a.n_split + s) * D + t], acc);
    }
  }
  a.O[(size_t)row * D + t] = (L > 0.f) ? acc / L : 0.f;
  if (a.lse != nullptr && t == 0) a.lse[row] = (L > 0.f) ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid((a.n_split + kWavesPerWg - 1) / kWavesPerWg, a.batch * a.n_kv_heads);
  const int G = a.n_q_heads / a.n_kv_heads;
  if (a.bf16)
    hipLaunchKernelGGL((decode_bf16_kernel<D>), grid, dim3(64 * kWavesPerWg), 0, stream, a);
  else if (G <= 4)
    hipLaunchKernelGGL((decode_f32_kernel<D, 4>), grid, dim3(64 * kWavesPerWg), 0, stream, a);
  else if (G <= 8)
    hipLaunchKernelGGL((decode_f32_kernel<D, 8>), grid, dim3(64 * kWavesPerWg), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_f32_kernel<D, 16>), grid, dim3(64 * kWavesPerWg), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.batch * a.n_q_heads), dim3(D), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

void decode_split_geometry(int n_items, int head_dim, bool bf16, int* items_per_split, int* n_split) {
  (void)head_dim;
  (void)bf16;
  const int ips = 1;
  *items_per_split = ips;
  *n_split = n_items > 0 ? (n_items + ips - 1) / ips : 1;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_t<64>(a, stream) : launch_t<128>(a, stream);
}

}  // namespace bsattn
