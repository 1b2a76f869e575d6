// Block selection for a decode query (COBS explainer, technical summary):
//  * per query head h and complete block j, the first-order score q~.mean_j
//    (section 2.2) or the second-order COBS score q~.mean_j + 1/2 sum_i
//    (factor_ji . q~)^2 (section 2.3, low-rank covariance);
//  * the group score ln sum_h exp(s_hj) over the query heads that share the
//    K/V head (the log of the group's estimated attention mass, section 2.1);
//  * the top-k candidates by (score desc, index asc), written ascending.
// Candidates are complete blocks with a token outside the forced set (sinks,
// window, global tokens).
//
// Scoring streams every summary once: 16 lanes (one DPP row) share one block,
// lane l owning the 4-dim chunks l, 16 + l, ... of every query head in
// registers, so each load instruction reads 256 contiguous bytes of a summary
// row; the 16 partial dot products are summed with DPP row rotations.  All of a block's rows
// (mean and up to 8 factor rows) are loaded before any arithmetic, so a wave
// waits on HBM once per block rather than once per row.
//
// Top-k: one wave per (b, K/V head), an exact 4-pass radix select (8 bits a
// pass) on order-preserving 32-bit keys: a 256-bin LDS histogram per pass and
// a wave-wide scan to find the digit of the k-th largest key; then every lane
// emits its candidates above the threshold, and the lowest-index ones equal
// to it, in index order.
#include "launch.hpp"

namespace bsattn {
namespace {

// Sum over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1): every lane gets the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
  return x;
}

template <int D, int GM, int RM, bool BF16>
__global__ __launch_bounds__(256) void select_scores_kernel(SelectArgs a) {
  constexpr int SL = D / 16;               // dims per lane: 4-dim chunks sub, 16 + sub, ...
  constexpr int NC = SL / 4;               // 16-byte chunks per lane per row
  constexpr int PB = RM == 0 ? 4 : (RM <= 4 ? 2 : 1);  // blocks per slot, loaded together
  constexpr int BPW = 16 * PB;             // blocks per workgroup
  const int tid = threadIdx.x;
  const int sub = tid & 15, slot = tid >> 4;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, g = bh % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;

  // lane `sub` owns dims 4(16c + sub) .. +4 for c < NC: each 16-lane row reads
  // 256 contiguous bytes of a summary row per instruction
  float q[GM][SL];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    const size_t off = ((size_t)b * a.n_q_heads + g * G + h) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d0 = 4 * (16 * c + sub);
      if (h < G) {
        if constexpr (BF16) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(a.Q) + off + d0);
          q[h][4 * c] = bf16lo(v[0]) * a.scale;
          q[h][4 * c + 1] = bf16hi(v[0]) * a.scale;
          q[h][4 * c + 2] = bf16lo(v[1]) * a.scale;
          q[h][4 * c + 3] = bf16hi(v[1]) * a.scale;
        } else {
          const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.Q) + off + d0);
          q[h][4 * c] = v.x * a.scale; q[h][4 * c + 1] = v.y * a.scale;
          q[h][4 * c + 2] = v.z * a.scale; q[h][4 * c + 3] = v.w * a.scale;
        }
      } else {
        q[h][4 * c] = q[h][4 * c + 1] = q[h][4 * c + 2] = q[h][4 * c + 3] = 0.f;
      }
    }
  }

  // load phase
  float vec[PB][1 + RM][SL];
  int jj[PB];
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const int j = blockIdx.x * BPW + p * 16 + slot;
    jj[p] = j;
    const int jc = min(j, a.n_blocks - 1);
    const size_t row = (size_t)bh * a.nblk_capacity + jc;
    const float4* src = reinterpret_cast<const float4*>(a.mean + row * D) + sub;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float4 v = src[16 * c];
      vec[p][0][4 * c] = v.x; vec[p][0][4 * c + 1] = v.y; vec[p][0][4 * c + 2] = v.z; vec[p][0][4 * c + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < RM; ++i) {
      if (i < a.rank) {
        const float4* fs = reinterpret_cast<const float4*>(a.factor + (row * a.rank + i) * D) + sub;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const float4 v = fs[16 * c];
          vec[p][1 + i][4 * c] = v.x; vec[p][1 + i][4 * c + 1] = v.y;
          vec[p][1 + i][4 * c + 2] = v.z; vec[p][1 + i][4 * c + 3] = v.w;
        }
      }
    }
  }
  // compute phase
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    float s[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < SL; ++e) acc = fmaf(q[h][e], vec[p][0][e], acc);
      s[h] = acc;
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) s[h] = row16_sum(s[h]);
#pragma unroll
    for (int i = 0; i < RM; ++i) {
      if (i < a.rank) {
        float pr[GM];
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < SL; ++e) acc = fmaf(q[h][e], vec[p][1 + i][e], acc);
          pr[h] = acc;
        }
#pragma unroll
        for (int h = 0; h < GM; ++h) pr[h] = row16_sum(pr[h]);
#pragma unroll
        for (int h = 0; h < GM; ++h) s[h] = fmaf(0.5f * pr[h], pr[h], s[h]);
      }
    }
    if (sub == 0 && jj[p] < a.n_blocks) {
      float mx = s[0];
#pragma unroll
      for (int h = 1; h < GM; ++h)
        if (h < G) mx = fmaxf(mx, s[h]);
      float sum = 0.f;
#pragma unroll
      for (int h = 0; h < GM; ++h)
        if (h < G) sum += __builtin_amdgcn_exp2f((s[h] - mx) * kLog2e);
      // sum >= 1 (the max term is exactly 1): log2 needs no range care
      a.scores[(size_t)bh * a.nblk_capacity + jj[p]] = fmaf(__builtin_amdgcn_logf(sum), kLn2, mx);
    }
  }
}

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Exclusive prefix sum over the workgroup; `tmp` holds kTopkWaves ints.  Returns the
// exclusive prefix and writes the total.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) tmp[wid] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int t = tmp[w];
    before += (w < wid) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

// One workgroup of 1024 threads per (b, K/V head).  Thread t owns the contiguous
// block range [t*per, (t+1)*per); keys stay in registers when per <= KPT.
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(SelectArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ int scan_tmp[kTopkWaves];
  __shared__ int s_digit, s_above;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int bh = blockIdx.x;
  const int NB = a.n_blocks;
  const int per = (NB + kTopkThreads - 1) / kTopkThreads;
  const int j0 = min(tid * per, NB), j1 = min(j0 + per, NB);
  const float* sc = a.scores + (size_t)bh * a.nblk_capacity;
  int32_t* out = a.sel + (size_t)bh * a.top_k;

  // keys of my candidates (non-candidates are never counted); registers if they fit
  uint32_t kreg[KPT];
  uint64_t cmask = 0ull;  // bit t: block j0 + t is a candidate
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const int j = j0 + t;
    kreg[t] = 0u;
    if (j < j1) {
      kreg[t] = order_key(sc[j]);
      if (forced_mask(a.forced, j) != ~0ull) cmask |= 1ull << t;
    }
  }
  int tot;
  const int ncand_dummy = block_excl_scan(__popcll(cmask), scan_tmp, &tot);
  (void)ncand_dummy;
  const int kk = min(a.top_k, tot);

  uint32_t prefix = 0u, pmask = 0u;
  int remaining = kk;
  if (kk > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int t = 0; t < KPT; ++t)
        if (((cmask >> t) & 1ull) && (kreg[t] & pmask) == prefix) atomicAdd(&hist[(kreg[t] >> shift) & 255u], 1u);
      __syncthreads();
      if (wid == 0) {
        // lane l owns digits 255-4l .. 252-4l (descending order)
        int c[4], sum = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          c[t] = (int)hist[255 - 4 * lane - t];
          sum += c[t];
        }
        int cum = wave_incl_scan(sum) - sum;
        int found = -1, above = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (found < 0 && cum + c[t] >= remaining) { found = 255 - 4 * lane - t; above = cum; }
          cum += c[t];
        }
        const uint64_t hit = __ballot(found >= 0);
        const int src = __ffsll((unsigned long long)hit) - 1;
        if (lane == src) { s_digit = found; s_above = above; }
      }
      __syncthreads();
      remaining -= s_above;
      prefix |= (uint32_t)s_digit << shift;
      pmask |= 255u << shift;
    }
  }
  // emit: keys above the threshold, then the lowest-index keys equal to it
  const uint32_t T = prefix;
  int gt = 0, eq = 0;
  if (kk > 0) {
#pragma unroll
    for (int t = 0; t < KPT; ++t) {
      if (!((cmask >> t) & 1ull)) continue;
      gt += kreg[t] > T;
      eq += kreg[t] == T;
    }
  }
  const int eq_before = block_excl_scan(eq, scan_tmp, &tot);
  const int take_eq = max(0, min(eq, remaining - eq_before));
  const int cnt = gt + take_eq;
  int pos = block_excl_scan(cnt, scan_tmp, &tot);
  if (kk > 0 && cnt > 0) {
    int taken = 0;
#pragma unroll
    for (int t = 0; t < KPT; ++t) {
      if (!((cmask >> t) & 1ull)) continue;
      if (kreg[t] > T || (kreg[t] == T && taken < take_eq)) {
        taken += kreg[t] == T;
        out[pos++] = j0 + t;
      }
    }
  }
  for (int i = kk + tid; i < a.top_k; i += kTopkThreads) out[i] = -1;
}

template <int D, int GM, int RM, bool BF16>
hipError_t launch_t(const SelectArgs& a, hipStream_t stream) {
  constexpr int BPW = 16 * (RM == 0 ? 4 : (RM <= 4 ? 2 : 1));
  dim3 grid((a.n_blocks + BPW - 1) / BPW, a.batch * a.n_kv_heads);
  if (a.n_blocks > 0)
    hipLaunchKernelGGL((select_scores_kernel<D, GM, RM, BF16>), grid, dim3(256), 0, stream, a);
  const int per = (a.n_blocks + kTopkThreads - 1) / kTopkThreads;
  const dim3 tg(a.batch * a.n_kv_heads), tb(kTopkThreads);
  if (per <= 2) hipLaunchKernelGGL(topk_kernel<2>, tg, tb, 0, stream, a);
  else if (per <= 8) hipLaunchKernelGGL(topk_kernel<8>, tg, tb, 0, stream, a);
  else if (per <= 32) hipLaunchKernelGGL(topk_kernel<32>, tg, tb, 0, stream, a);
  else hipLaunchKernelGGL(topk_kernel<64>, tg, tb, 0, stream, a);
  return hipGetLastError();
}

template <int D, int GM, bool BF16>
hipError_t launch_r(const SelectArgs& a, hipStream_t stream) {
  if (a.rank == 0) return launch_t<D, GM, 0, BF16>(a, stream);
  if (a.rank <= 4) return launch_t<D, GM, 4, BF16>(a, stream);
  return launch_t<D, GM, 8, BF16>(a, stream);
}

template <int D, bool BF16>
hipError_t launch_g(const SelectArgs& a, hipStream_t stream) {
  const int G = a.n_q_heads / a.n_kv_heads;
  if (G <= 4) return launch_r<D, 4, BF16>(a, stream);
  if (G <= 8) return launch_r<D, 8, BF16>(a, stream);
  return launch_r<D, 16, BF16>(a, stream);
}

}  // namespace

hipError_t launch_select_topk(const SelectArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) return a.bf16 ? launch_g<64, true>(a, stream) : launch_g<64, false>(a, stream);
  return a.bf16 ? launch_g<128, true>(a, stream) : launch_g<128, false>(a, stream);
}

}  // namespace bsattn
