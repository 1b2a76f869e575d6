// Block selection (COBS explainer, technical summary):
//  * per query head h and complete block j, the first-order score q~.mean_j
//    (section 2.2) or the second-order COBS score q~.mean_j + 1/2 sum_i
//    (factor_ji . q~)^2 (section 2.3, low-rank covariance; with a query
//    subspace the factor rows meet the projected query);
//  * the group score ln sum_h exp(s_hj) over the query heads that share the
//    K/V head (the log of the group's estimated attention mass, section 2.1);
//  * the top-k candidates by (score desc, index asc), written ascending.
// Decode candidates are complete blocks with a token outside the forced set
// (sinks, window, global tokens); prefill tiles have their own rule (below).
//
// Kernels, in file order:
//  * (the VALU scorer for fp32 operands, select_scores_kernel, is in
//    select_valu.hip)
//  * select_scores_mfma_kernel: bf16 queries and means with FP4 factor rows or
//    none, on v_mfma_f32_16x16x32_bf16 (every operand exact in bf16), with the
//    per-workgroup query projection when a subspace basis is given.
//  * topk_kernel: one workgroup per (b, K/V head) or per (b, K/V head, prefill
//    tile), an exact radix select on order-preserving 32-bit keys.
//  * select_exact_kernel: the exact block mass, read from the keys.
//  * prefill_tile_scores_kernel: the block-sparse prefill's tile scores.
#include <type_traits>

#include "launch.hpp"

namespace bsattn {
namespace {


// MFMA scoring, for bfloat16 queries and means with FP4 factor rows or none:
// every operand is exact in bfloat16 (FP4 E2M1 values are), so the products
// are exact and the sums are fp32, as in the VALU kernel above.  One wave
// scores a run of 16-block units of one (b, K/V head) pair with
// v_mfma_f32_16x16x32_bf16: the A operand holds the group's query heads (row m
// = head m, zero past the group), the B operand the 16 blocks' summary rows
// (column n = block n of the unit), so lane l ends with block l % 16's dot
// products for heads 4 (l / 16) .. +3.  The softmax scale, and an FP4 row's
// scale, multiply the fp32 dot products afterwards.
//
// Loads: a mean row is 2D bytes; in k-step s lane (n, kg = l / 16) reads the
// 16 bytes of dims 32 s + 8 kg .. +7 (64 contiguous bytes per row per
// instruction).  An FP4 row of E entries (E = D, or the subspace dimension)
// is E/2 bytes; lane kg reads its E/8 bytes at once (entries kg E/4 .. +E/4)
// and converts 8 codes per k-step, entries kg E/4 + 8 s + t, so the factor
// MFMAs take the query in that order (a second A operand).
//
// With a query-subspace basis P (SK = E / 32 > 0) the factor rows meet the
// projected query P q~ [COBS 2.3].  The four waves of a workgroup share one
// pair and project its queries once: tile T of the projection, MFMAs with 16
// basis rows as A (P split into bfloat16 hi + lo, 16 significant bits) and
// the queries as B, leaves lane (head n, kg) with 4 projected entries; the
// basis rows of tile T = 2 s + u are taken in the order that gives lane kg
// entries kg E/4 + 8 s + 4 u + i, i.e. exactly the 8 entries its FP4 codes
// need in factor k-step s.  Wave w computes k-step w of every tile; the
// partial tiles meet in LDS (one barrier) and each lane sums them and splits
// its projected query into bfloat16 hi + lo (two MFMAs per factor k-step).
// The basis loads are issued before the first summary loads (loads complete
// in issue order, so the projection does not wait on HBM), except for rank 8
// at E = 128, where their registers would not fit.
template <int KF>
struct FacWords {
  uint32_t w[KF];
};
template <>
struct FacWords<4> {
  u32x4 w;
};
template <>
struct FacWords<2> {
  u32x2 w;
};

template <int KF>
__device__ __forceinline__ FacWords<KF> load_fac(const uint8_t* row, int kg) {
  FacWords<KF> r;
  if constexpr (KF == 4) {
    r.w = *reinterpret_cast<const u32x4*>(row + 16 * kg);
  } else if constexpr (KF == 2) {
    r.w = *reinterpret_cast<const u32x2*>(row + 8 * kg);
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(row + 4 * KF * kg);
#pragma unroll
    for (int c = 0; c < KF; ++c) r.w[c] = p[c];
  }
  return r;
}

// x = hi + lo (+ lo2): each part the nearest bfloat16 of what the earlier parts
// leave; two parts hold 16 significant bits, three all 24 of a float.
template <int NP>
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8 (&part)[NP]) {
  float r[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = x[t];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    u32x4 w;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[c] = cvt_pk_bf16(r[2 * c], r[2 * c + 1]);
      r[2 * c] -= bf16lo(w[c]);
      r[2 * c + 1] -= bf16hi(w[c]);
    }
    part[k] = __builtin_bit_cast(bf16x8, w);
  }
}

__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.f, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.f, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.f, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.f, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int D, int RM, int SK>
__global__ __launch_bounds__(256, 2) void select_scores_mfma_kernel(SelectArgs a) {
  constexpr int KS = D / 32;                 // k-steps of the mean
  constexpr int KF = SK > 0 ? SK : D / 32;   // k-steps (dwords per lane) of a factor row
  constexpr int E = 32 * KF;                 // entries of a factor row
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * 4 + wid;
  const int n_pairs = a.batch * a.n_kv_heads;
  const int pair = gw / a.n_part, wi = gw % a.n_part;
  // no barriers unless SK > 0, where n_part % 4 == 0 keeps every wave of the
  // grid (all four of a workgroup) inside [0, n_pairs)
  if (pair >= n_pairs) return;
  const int col = lane & 15, kg = lane >> 4;
  const int b = pair / a.n_kv_heads, g = pair % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int NB = a.n_blocks;
  const int rank = a.rank;

  bf16x8 qm[KS];
  bf16x8 qf[SK > 0 ? 2 * SK : (RM > 0 ? KS : 1)];  // SK > 0: hi, lo per k-step
  {
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(a.Q) + ((size_t)b * a.n_q_heads + g * G + min(col, G - 1)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * kg);
      if (col >= G) v = u32x4{0u, 0u, 0u, 0u};
      qm[s] = __builtin_bit_cast(bf16x8, v);
      if constexpr (RM > 0 && SK == 0) {
        u32x4 w = *reinterpret_cast<const u32x4*>(qrow + kg * (D / 4) + 8 * s);
        if (col >= G) w = u32x4{0u, 0u, 0u, 0u};
        qf[s] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }

  struct Stage {
    u32x4 m[KS];
    FacWords<KF> f[RM > 0 ? RM : 1];
    float fs[RM > 0 ? RM : 1];
  };
  // every load is issued (blocks past the end re-read the last block, factor
  // rows past the rank the last row; both ignored), as in the VALU kernel
  auto load = [&](int u, Stage& st) __attribute__((always_inline)) {
    const int j = min(u * 16 + col, NB - 1);
    const size_t row = (size_t)pair * a.nblk_capacity + j;
    const u32x4* mrow = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.mean) + row * D);
#pragma unroll
    for (int s = 0; s < KS; ++s) st.m[s] = mrow[4 * s + kg];
#pragma unroll
    for (int i = 0; i < RM; ++i) {
      const size_t fr = row * rank + min(i, rank - 1);
      st.f[i] = load_fac<KF>(reinterpret_cast<const uint8_t*>(a.factor) + fr * (E / 2), kg);
      st.fs[i] = a.factor_scale[fr];
    }
  };
  // the pair's projected queries (SK > 0): k-step wid of every tile's basis
  // rows, loaded by project_load() before the first summary loads
  constexpr int NT = 2 * SK;  // projection tiles
  constexpr bool HOIST = SK > 0 && !(RM == 8 && SK == 4);
  float4 pv[HOIST ? NT : 1][2];
  auto basis_row = [&](int T) __attribute__((always_inline)) {
    const int m = lane & 15, s2 = T >> 1, u = T & 1;
    return a.basis + ((size_t)g * E + (m >> 2) * (E / 4) + 8 * s2 + 4 * u + (m & 3)) * D + 32 * wid + 8 * kg;
  };
  auto project_load = [&]() __attribute__((always_inline)) {
    if constexpr (HOIST) {
      if (wid < KS) {
#pragma unroll
        for (int T = 0; T < NT; ++T) {
          const float* prow = basis_row(T);
          pv[T][0] = *reinterpret_cast<const float4*>(prow);
          pv[T][1] = *reinterpret_cast<const float4*>(prow + 4);
        }
      }
    }
  };
  auto project = [&]() __attribute__((always_inline)) {
    if constexpr (SK > 0) {
      __shared__ f32x4 qpart[KS][NT][64];
      // k-step ks = wid, one uniform branch per k-step (constant register indices)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (wid == ks) {
#pragma unroll
          for (int T = 0; T < NT; ++T) {
            float4 x0, x1;
            if constexpr (HOIST) {
              x0 = pv[T][0];
              x1 = pv[T][1];
            } else {
              const float* prow = basis_row(T);
              x0 = *reinterpret_cast<const float4*>(prow);
              x1 = *reinterpret_cast<const float4*>(prow + 4);
            }
            const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            bf16x8 pp[2];
            split_bf16x8<2>(x, pp);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp[0], qm[ks], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp[1], qm[ks], acc, 0, 0, 0);
            qpart[ks][T][lane] = acc;
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int s2 = 0; s2 < SK; ++s2) {
        f32x4 lo4 = qpart[0][2 * s2][lane], hi4 = qpart[0][2 * s2 + 1][lane];
#pragma unroll
        for (int w = 1; w < KS; ++w) {
          lo4 += qpart[w][2 * s2][lane];
          hi4 += qpart[w][2 * s2 + 1][lane];
        }
        lo4 *= a.scale;
        hi4 *= a.scale;
        const float x[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        bf16x8 pp[2];
        split_bf16x8<2>(x, pp);
        qf[2 * s2] = pp[0];
        qf[2 * s2 + 1] = pp[1];
      }
    }
  };
  auto comp = [&](int u, const Stage& st) __attribute__((always_inline)) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qm[s], __builtin_bit_cast(bf16x8, st.m[s]), acc, 0, 0, 0);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = acc[i] * a.scale;
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r < rank) {
        f32x4 pa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KF; ++s) {
          const bf16x8 bv = fp4x8_to_bf16(st.f[r].w[s]);  // 8 codes, entry kg E/4 + 8 s + t in bits 4t ..
          if constexpr (SK > 0) {
            pa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[2 * s], bv, pa, 0, 0, 0);
            pa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[2 * s + 1], bv, pa, 0, 0, 0);
          } else {
            pa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[s], bv, pa, 0, 0, 0);
          }
        }
        // the row's scale (the projected query already carries the softmax scale)
        const float c = SK > 0 ? st.fs[r] : a.scale * st.fs[r];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pr = pa[i] * c;
          sc[i] = fmaf(0.5f * pr, pr, sc[i]);
        }
      }
    }
    // group score: log-sum-exp over the G heads, spread over the lane groups kg
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * kg + i < G) mx = fmaxf(mx, sc[i]);
    if (G > 4) mx = fmaxf(mx, __shfl_xor(mx, 16));
    if (G > 8) mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * kg + i < G) sum += __builtin_amdgcn_exp2f((sc[i] - mx) * kLog2e);
    if (G > 4) sum += __shfl_xor(sum, 16);
    if (G > 8) sum += __shfl_xor(sum, 32);
    const int j = u * 16 + col;
    // sum >= 1 (the max term is exactly 1): log2 needs no range care
    if (kg == 0 && j < NB) a.scores[(size_t)pair * a.nblk_capacity + j] = fmaf(__builtin_amdgcn_logf(sum), kLn2, mx);
  };

  // every path calls project() exactly once (it holds the workgroup's barrier)
  const int n_units = (NB + 15) / 16;
  const int u0 = wi * a.per_wave, u1 = min(u0 + a.per_wave, n_units);
  const int n = u1 - u0;
  Stage A, B;
  project_load();
  if (n >= 4) {
    load(u0, A);
    load(u0 + 1, B);
    project();
    int u = u0;
    for (; u + 3 < u1; u += 2) {
      comp(u, A);
      load(u + 2, A);
      comp(u + 1, B);
      load(u + 3, B);
    }
    if (u + 2 < u1) {
      comp(u, A);
      load(u + 2, A);
      comp(u + 1, B);
      comp(u + 2, A);
    } else {
      comp(u, A);
      comp(u + 1, B);
    }
  } else if (n == 3) {
    load(u0, A);
    load(u0 + 1, B);
    project();
    comp(u0, A);
    load(u0 + 2, A);
    comp(u0 + 1, B);
    comp(u0 + 2, A);
  } else if (n == 2) {
    load(u0, A);
    load(u0 + 1, B);
    project();
    comp(u0, A);
    comp(u0 + 1, B);
  } else if (n == 1) {
    load(u0, A);
    project();
    comp(u0, A);
  } else {
    project();
  }
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// One workgroup of kTopkThreads threads per (b, K/V head).  Thread t owns the contiguous
// block range [t*per, (t+1)*per) (per <= KPT); up to 32 keys per thread stay in
// registers, more (over 32,768 blocks) are read again from the scores on each
// pass, which the L2 holds, so the kernel stays within its 128 registers.
// Barriers: one after the candidate count / AND / OR reduction (which also
// clears the four pass histograms), one per radix pass (every wave then finds
// the pass's digit from the histogram itself), one for the output scan.  Bytes
// on which all candidate keys agree are skipped, and the passes stop once the
// k-th key's bin is taken whole.
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(SelectArgs a) {
  __shared__ uint32_t hist[4][256];
  __shared__ uint32_t red[kTopkWaves][3];  // per wave: candidates, AND, OR of their keys
  __shared__ int part[kTopkWaves][2];      // per wave: keys above, keys on the threshold
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int bh = blockIdx.x;
  const int NB = a.n_blocks;
  const int per = (NB + kTopkThreads - 1) / kTopkThreads;
  const int j0 = min(tid * per, NB), j1 = min(j0 + per, NB);
  const float* sc = a.scores + (size_t)bh * a.nblk_capacity;
  int32_t* out = a.sel + (size_t)bh * a.top_k;

  constexpr bool kRegKeys = KPT <= 32;
  uint32_t key[kRegKeys ? KPT : 1];
  // key of block j0 + t (t < j1 - j0)
  auto key_at = [&](int t) -> uint32_t {
    if constexpr (kRegKeys) return key[t];
    else return order_key(sc[j0 + t]);
  };
  uint64_t cm = 0ull;  // bit t: block j0 + t is a candidate
  uint32_t kand = ~0u, kor = 0u;
  // prefill tiles: blocks starting before the window of the tile's last row
  int tile_klo = 0;
  if (a.tile_rows > 0) {
    const int t = bh % a.n_tiles;
    tile_klo = max(0, min(a.seq_len, (t + 1) * a.tile_rows) - 1 - a.window_left);
  }
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const int j = j0 + t;
    if constexpr (kRegKeys) key[t] = 0u;
    if (j < j1) {
      const uint32_t k = order_key(sc[j]);
      if constexpr (kRegKeys) key[t] = k;
      const bool cand = a.tile_rows > 0 ? (j * kBlock < tile_klo && (j + 1) * kBlock > a.n_sink)
                                        : forced_mask(a.forced, j) != ~0ull;
      if (cand) {
        cm |= 1ull << t;
        kand &= k;
        kor |= k;
      }
    }
  }
  for (int i = tid; i < 4 * 256; i += kTopkThreads) (&hist[0][0])[i] = 0u;
  {
    const int cnt = __builtin_amdgcn_readlane(wave_incl_scan_dpp(__popcll(cm)), 63);
    uint32_t wa, wo;
    wave_and_or(kand, kor, wa, wo);
    if (lane == 0) { red[wid][0] = (uint32_t)cnt; red[wid][1] = wa; red[wid][2] = wo; }
  }
  __syncthreads();
  int tot = 0;
  uint32_t all_and = ~0u, all_or = 0u;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    tot += (int)red[w][0];
    all_and &= red[w][1];
    all_or |= red[w][2];
  }
  const int kk = min(a.top_k, tot);
  const uint32_t diff = all_and ^ all_or;
  // first pass: the 8 bits from the highest bit on which candidate keys differ
  // down (the bits above it are shared by every candidate), then the next 8
  // below, and so on: no pass spends digits on bits every candidate shares
  const int hb = diff ? 31 - __clz(diff) : -1;
  uint32_t pmask = hb >= 31 ? 0u : ~0u << (hb + 1);
  uint32_t prefix = all_and & pmask;
  int remaining = kk;
  if (kk > 0) {
    int pass = 0;
    for (int hi = hb; hi >= 0; ++pass) {
      const int lo = max(hi - 7, 0);
      const uint32_t dmask = (2u << (hi - lo)) - 1u;
      uint32_t* h = hist[pass];
#pragma unroll
      for (int t = 0; t < KPT; ++t)
        if ((cm >> t) & 1ull) {
          const uint32_t k = key_at(t);
          if ((k & pmask) == prefix) atomicAdd(&h[(k >> lo) & dmask], 1u);
        }
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
    if (!((cm >> t) & 1ull)) continue;
    const uint32_t km = key_at(t) & pmask;
    gt += km > prefix;
    eq += km == prefix;
  }
  const int igt = wave_incl_scan_dpp(gt), ieq = wave_incl_scan_dpp(eq);
  if (lane == 63) { part[wid][0] = igt; part[wid][1] = ieq; }
  __syncthreads();
  int gt_before = igt - gt, eq_before = ieq - eq;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    if (w < wid) { gt_before += part[w][0]; eq_before += part[w][1]; }
  }
  if (kk > 0) {
    const int take_eq = max(0, min(eq, remaining - eq_before));
    int pos = gt_before + min(eq_before, remaining);
    int taken = 0;
#pragma unroll
    for (int t = 0; t < KPT; ++t) {
      if (!((cm >> t) & 1ull)) continue;
      const uint32_t km = key_at(t) & pmask;
      if (km > prefix || (km == prefix && taken < take_eq)) {
        taken += km == prefix;
        out[pos++] = j0 + t;
      }
    }
  }
  for (int i = kk + tid; i < a.top_k; i += kTopkThreads) out[i] = -1;
}

hipError_t launch_topk(const SelectArgs& a, hipStream_t stream) {
  const int per = (a.n_blocks + kTopkThreads - 1) / kTopkThreads;
  const dim3 tg(a.batch * a.n_kv_heads * (a.tile_rows > 0 ? a.n_tiles : 1)), tb(kTopkThreads);
  if (per <= 2) hipLaunchKernelGGL(topk_kernel<2>, tg, tb, 0, stream, a);
  else if (per <= 8) hipLaunchKernelGGL(topk_kernel<8>, tg, tb, 0, stream, a);
  else if (per <= 32) hipLaunchKernelGGL(topk_kernel<32>, tg, tb, 0, stream, a);
  else hipLaunchKernelGGL(topk_kernel<64>, tg, tb, 0, stream, a);
  return hipGetLastError();
}

template <int D, int RM, int SK>
hipError_t launch_mfma(const SelectArgs& a0, hipStream_t stream) {
  SelectArgs a = a0;
  if (a.n_blocks > 0) {
    const long long units = (a.n_blocks + 15) / 16;
    // with a query subspace every workgroup projects its pair's queries, so
    // fewer, longer workgroups (half the resident waves) measured faster
    split_units(a, units, SK > 0 ? 256 * 4 : 256 * 8);
    if (SK > 0 && a.n_part % 4 != 0) {
      // the four waves of a workgroup share a pair (one projection, one barrier)
      a.n_part = (a.n_part + 3) / 4 * 4;
      a.per_wave = (int)((units + a.n_part - 1) / a.n_part);
    }
    const long long waves = (long long)a.batch * a.n_kv_heads * a.n_part;
    hipLaunchKernelGGL((select_scores_mfma_kernel<D, RM, SK>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       stream, a);
  }
  if (a.scores_only) return hipGetLastError();
  return launch_topk(a, stream);
}

template <int D, int RM>
hipError_t launch_mfma_s(const SelectArgs& a, hipStream_t stream) {
  switch (a.sub_dim / 32) {
    case 1: return launch_mfma<D, RM, 1>(a, stream);
    case 2: return launch_mfma<D, RM, 2>(a, stream);
    case 3: if constexpr (D >= 96) return launch_mfma<D, RM, 3>(a, stream); else break;
    case 4: if constexpr (D >= 128) return launch_mfma<D, RM, 4>(a, stream); else break;
    default: break;
  }
  return launch_mfma<D, RM, 0>(a, stream);
}

template <int D>
hipError_t launch_mfma_r(const SelectArgs& a, hipStream_t stream) {
  if (a.rank == 0) return launch_mfma<D, 0, 0>(a, stream);
  if (a.rank <= 2) return launch_mfma_s<D, 2>(a, stream);
  if (a.rank <= 4) return launch_mfma_s<D, 4>(a, stream);
  return launch_mfma_s<D, 8>(a, stream);
}


}  // namespace

// Block-sparse prefill selection [COBS 2.1, 2.2; NSA's block selection]: the
// score of block j for query tile t of pair (b, g) is ln sum over the tile's
// rows r and the group's heads h of exp(q~_{r,h} . mean_j), the log of the
// tile's summed estimated mass.  One workgroup per (pair, tile, group of 4
// 16-block units), its 4 waves taking every fourth 16-row slice of the tile's
// (row, head) pairs: v_mfma_f32_16x16x32_bf16 with 16 pairs as A (each A load
// serves the 4 units) and a unit's 16 bf16 means as B (exact products, fp32
// sums), a running log-sum-exp per lane and unit, then across the four lane
// groups and (through LDS, one barrier) the four waves.  Units past the
// tile's candidates are skipped (their scores are not written).
constexpr int kTileUnits = 4;

template <int D>
__global__ __launch_bounds__(256) void prefill_tile_scores_kernel(SelectArgs a) {
  constexpr int KS = D / 32, U = kTileUnits;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NB = a.n_blocks;
  const int n_groups = (NB + 16 * U - 1) / (16 * U);
  const int grp = blockIdx.x % n_groups, rest = blockIdx.x / n_groups;
  const int t = rest % a.n_tiles, pair = rest / a.n_tiles;
  // every exit below depends on the workgroup's indices only (the barrier is reached by all or none)
  if (pair >= a.batch * a.n_kv_heads) return;
  const int N = a.seq_len;
  const int i0 = t * a.tile_rows, rows = min(N, i0 + a.tile_rows) - i0;
  const int klo = max(0, i0 + rows - 1 - a.window_left);
  // units of this group holding a candidate (wave-uniform)
  const int nu = min(U, max(0, (klo + 16 * kBlock - 1) / (16 * kBlock) - grp * U));
  if (nu == 0) return;
  const int col = lane & 15, kg = lane >> 4;
  const int b = pair / a.n_kv_heads, g = pair % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;

  // B operands: unit v's means, lane (block col, kg) holding dims 32 s + 8 kg .. +7
  bf16x8 bm[U][KS];
#pragma unroll
  for (int v = 0; v < U; ++v) {
    const int j = min((grp * U + v) * 16 + col, NB - 1);
    const u32x4* mrow = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.mean) +
                                                       ((size_t)pair * a.nblk_capacity + j) * D);
#pragma unroll
    for (int s = 0; s < KS; ++s) bm[v][s] = __builtin_bit_cast(bf16x8, mrow[4 * s + kg]);
  }
  const uint16_t* Qg = reinterpret_cast<const uint16_t*>(a.Q) + ((size_t)b * a.n_q_heads + g * G) * N * D;
  const float sl2 = a.scale * kLog2e;
  float m[U], l[U];  // per unit: this lane's running max and sum (log2 domain)
#pragma unroll
  for (int v = 0; v < U; ++v) { m[v] = -INFINITY; l[v] = 0.f; }
  const int n_pairs_rows = rows * G;  // (row, head) pairs p = r G + h
  for (int p0 = 16 * wid; p0 < n_pairs_rows; p0 += 64) {
    // A operand: pair p0 + (lane % 16), dims 32 s + 8 kg .. +7
    const int p = min(p0 + col, n_pairs_rows - 1);
    const uint16_t* qrow = Qg + ((size_t)(p % G) * N + i0 + p / G) * D;
    bf16x8 qa[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qa[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * kg));
#pragma unroll
    for (int v = 0; v < U; ++v) {
      if (v < nu) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], bm[v][s], acc, 0, 0, 0);
        // lane (col, kg) holds pairs p0 + 4 kg + i for block (grp U + v) 16 + col
        float x[4], mx = m[v];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = p0 + 4 * kg + i < n_pairs_rows ? acc[i] * sl2 : -INFINITY;
          mx = fmaxf(mx, x[i]);
        }
        if (mx > -INFINITY) {
          l[v] *= __builtin_amdgcn_exp2f(m[v] - mx);  // m = -inf: l is 0
#pragma unroll
          for (int i = 0; i < 4; ++i) l[v] += __builtin_amdgcn_exp2f(x[i] - mx);
          m[v] = mx;
        }
      }
    }
  }
  auto combine = [](float& mm, float& ll, float mo, float lo) __attribute__((always_inline)) {
    const float mn = fmaxf(mm, mo);
    ll = (mm == -INFINITY ? 0.f : ll * __builtin_amdgcn_exp2f(mm - mn)) +
         (mo == -INFINITY ? 0.f : lo * __builtin_amdgcn_exp2f(mo - mn));
    mm = mn;
  };
  __shared__ float part[4][U][16][2];
#pragma unroll
  for (int v = 0; v < U; ++v) {
    // the four lane groups hold disjoint rows of the same block
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) combine(m[v], l[v], __shfl_xor(m[v], o), __shfl_xor(l[v], o));
    if (kg == 0) {
      part[wid][v][col][0] = m[v];
      part[wid][v][col][1] = l[v];
    }
  }
  __syncthreads();
  if (wid == 0 && kg == 0) {
#pragma unroll
    for (int v = 0; v < U; ++v) {
      float mm = part[0][v][col][0], ll = part[0][v][col][1];
#pragma unroll
      for (int w = 1; w < 4; ++w) combine(mm, ll, part[w][v][col][0], part[w][v][col][1]);
      const int j = (grp * U + v) * 16 + col;
      if (v < nu && j < NB && ll > 0.f)
        a.scores[((size_t)pair * a.n_tiles + t) * a.nblk_capacity + j] = (mm + __builtin_amdgcn_logf(ll)) * kLn2;
    }
  }
}

hipError_t launch_select_topk(const SelectArgs& a, hipStream_t stream) {
  // every operand exact in bfloat16: the MFMA scorer
  if (a.bf16 && a.mean_bf16 && (a.rank == 0 || a.factor_fp4))
    return a.head_dim == 64 ? launch_mfma_r<64>(a, stream) : launch_mfma_r<128>(a, stream);
  hipError_t e;
  if (a.head_dim == 64) e = a.bf16 ? launch_valu_scores<64, true>(a, stream) : launch_valu_scores<64, false>(a, stream);
  else e = a.bf16 ? launch_valu_scores<128, true>(a, stream) : launch_valu_scores<128, false>(a, stream);
  if (e != hipSuccess || a.scores_only) return e;
  return launch_topk(a, stream);
}

// Exact block mass [COBS 2.1, the selection oracle]: scores[b,g,j] = ln sum over
// the group's heads h and block j's keys k of exp(q~_h . k), read from the keys
// themselves (a reference selector: it streams every key of the context).  One
// wave per (pair, block): the group's heads as the MFMA A operand (rows past G
// zero), 16 key rows at a time as B (bf16 keys and queries: exact products,
// fp32 sums), the 64 keys x G heads reduced to one log-sum-exp (lane, then the
// 16 lanes of a row group, then the four lane groups).
template <int D>
__global__ __launch_bounds__(256) void select_exact_kernel(SelectArgs a) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long gw = (long long)blockIdx.x * 4 + wid;
  const int NB = a.n_blocks;
  const int pair = (int)(gw / NB), j = (int)(gw % NB);
  if (pair >= a.batch * a.n_kv_heads) return;  // no barriers: waves are independent
  const int col = lane & 15, kg = lane >> 4;
  const int b = pair / a.n_kv_heads, g = pair % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.K) + ((size_t)pair * a.kv_capacity + (size_t)j * kBlock) * D;
  u32x4 kv[4][KS];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int s = 0; s < KS; ++s) kv[c][s] = *reinterpret_cast<const u32x4*>(Kb + (16 * c + col) * D + 32 * s + 8 * kg);
  bf16x8 qm[KS];
  {
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(a.Q) + ((size_t)b * a.n_q_heads + g * G + min(col, G - 1)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * kg);
      if (col >= G) v = u32x4{0u, 0u, 0u, 0u};
      qm[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const float sl2 = a.scale * kLog2e;
  float x[4][4], m = -INFINITY;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qm[s], __builtin_bit_cast(bf16x8, kv[c][s]), acc, 0, 0, 0);
    // lane (key 16 c + col, kg): heads 4 kg .. +3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[c][i] = 4 * kg + i < G ? acc[i] * sl2 : -INFINITY;
      m = fmaxf(m, x[c][i]);
    }
  }
  // the block's max over every lane (the 64 lanes hold disjoint (key, head) pairs)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  float l = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) l += __builtin_amdgcn_exp2f(x[c][i] - m);  // exp2(-inf) = 0
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) l += __shfl_xor(l, o);
  if (lane == 0) a.scores[(size_t)pair * a.nblk_capacity + j] = (m + __builtin_amdgcn_logf(l)) * kLn2;
}

hipError_t launch_select_exact(const SelectArgs& a, hipStream_t stream) {
  if (a.n_blocks > 0) {
    const long long waves = (long long)a.batch * a.n_kv_heads * a.n_blocks;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (a.head_dim == 64) hipLaunchKernelGGL(select_exact_kernel<64>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(select_exact_kernel<128>, grid, block, 0, stream, a);
  }
  return launch_topk(a, stream);
}

hipError_t launch_prefill_select(const SelectArgs& a, hipStream_t stream) {
  if (a.n_blocks > 0) {
    const long long wgs =
        (long long)a.batch * a.n_kv_heads * a.n_tiles * ((a.n_blocks + 16 * kTileUnits - 1) / (16 * kTileUnits));
    const dim3 grid((unsigned)wgs), block(256);
    if (a.head_dim == 64) hipLaunchKernelGGL(prefill_tile_scores_kernel<64>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(prefill_tile_scores_kernel<128>, grid, block, 0, stream, a);
  }
  return launch_topk(a, stream);
}

}  // namespace bsattn
