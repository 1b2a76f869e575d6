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
// Scoring streams every summary once: 16 lanes share one block, each lane
// owning d/16 consecutive dims of every query head in registers, so each
// summary row is read with coalesced 16-byte loads.  Top-k is an exact
// 4-pass radix select on order-preserving 32-bit keys in LDS.
#include "launch.hpp"

namespace bsattn {
namespace {

constexpr int kBlocksPerWg = 64;

template <int D, int GM, bool BF16>
__global__ __launch_bounds__(256) void select_scores_kernel(SelectArgs a) {
  constexpr int SL = D / 16;  // dims per lane
  const int tid = threadIdx.x;
  const int sub = tid & 15, slot = tid >> 4;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, g = bh % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;

  float q[GM][SL];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    const int hq = g * G + h;
    const size_t off = ((size_t)b * a.n_q_heads + hq) * D + sub * SL;
#pragma unroll
    for (int e = 0; e < SL; ++e) {
      float v = 0.f;
      if (h < G) {
        if constexpr (BF16) v = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.Q)[off + e]);
        else v = reinterpret_cast<const float*>(a.Q)[off + e];
      }
      q[h][e] = v * a.scale;
    }
  }

  for (int pass = 0; pass < kBlocksPerWg / 16; ++pass) {
    const int j = blockIdx.x * kBlocksPerWg + pass * 16 + slot;
    if (j >= a.n_blocks) break;  // uniform across the 16 lanes of a slot
    const size_t row = (size_t)bh * a.nblk_capacity + j;
    float m[SL];
    {
      const float4* src = reinterpret_cast<const float4*>(a.mean + row * D + sub * SL);
#pragma unroll
      for (int c = 0; c < SL / 4; ++c) {
        const float4 v = src[c];
        m[4 * c] = v.x; m[4 * c + 1] = v.y; m[4 * c + 2] = v.z; m[4 * c + 3] = v.w;
      }
    }
    float s[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < SL; ++e) acc = fmaf(q[h][e], m[e], acc);
      s[h] = acc;
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1)
#pragma unroll
      for (int h = 0; h < GM; ++h) s[h] += __shfl_xor(s[h], o);

    for (int i = 0; i < a.rank; ++i) {
      const float4* src =
          reinterpret_cast<const float4*>(a.factor + (row * a.rank + i) * D + sub * SL);
#pragma unroll
      for (int c = 0; c < SL / 4; ++c) {
        const float4 v = src[c];
        m[4 * c] = v.x; m[4 * c + 1] = v.y; m[4 * c + 2] = v.z; m[4 * c + 3] = v.w;
      }
      float p[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < SL; ++e) acc = fmaf(q[h][e], m[e], acc);
        p[h] = acc;
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1)
#pragma unroll
        for (int h = 0; h < GM; ++h) p[h] += __shfl_xor(p[h], o);
#pragma unroll
      for (int h = 0; h < GM; ++h) s[h] = fmaf(0.5f * p[h], p[h], s[h]);
    }
    if (sub == 0) {
      float mx = s[0];
#pragma unroll
      for (int h = 1; h < GM; ++h)
        if (h < G) mx = fmaxf(mx, s[h]);
      float sum = 0.f;
#pragma unroll
      for (int h = 0; h < GM; ++h)
        if (h < G) sum += expf(s[h] - mx);
      a.scores[row] = mx + logf(sum);
    }
  }
}

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over a 1024-thread workgroup.  `tmp` holds 16 ints.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int w = lane < 16 ? tmp[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(w, o);
      if (lane >= o) w += y;
    }
    if (lane < 16) tmp[16 + lane] = w;  // inclusive wave prefix
  }
  __syncthreads();
  const int before = (wid == 0 ? 0 : tmp[16 + wid - 1]) + x - v;
  *total = tmp[31];
  __syncthreads();
  return before;
}

__global__ __launch_bounds__(1024) void topk_kernel(SelectArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ int scan_tmp[32];
  __shared__ uint32_t s_prefix, s_pmask;
  __shared__ int s_remaining;
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int NB = a.n_blocks;
  const int per = (NB + 1023) / 1024;
  const int j0 = min(tid * per, NB), j1 = min(j0 + per, NB);
  const float* sc = a.scores + (size_t)bh * a.nblk_capacity;
  int32_t* out = a.sel + (size_t)bh * a.top_k;

  uint64_t cand = 0ull;  // bit (j - j0): block j is a candidate
  int ncand_mine = 0;
  for (int j = j0; j < j1; ++j) {
    if (forced_mask(a.forced, j) != ~0ull) {
      cand |= 1ull << (j - j0);
      ++ncand_mine;
    }
  }
  int ncand;
  block_exclusive_scan(ncand_mine, scan_tmp, &ncand);
  const int kk = min(a.top_k, ncand);
  if (kk > 0) {
    if (tid == 0) { s_prefix = 0u; s_pmask = 0u; s_remaining = kk; }
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
      const uint32_t prefix = s_prefix, pmask = s_pmask;
      for (int j = j0; j < j1; ++j) {
        if (!((cand >> (j - j0)) & 1ull)) continue;
        const uint32_t key = order_key(sc[j]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int rem = s_remaining, cum = 0, digit = 0;
        for (int dgt = 255; dgt >= 0; --dgt) {
          const int h = (int)hist[dgt];
          if (cum + h >= rem) { digit = dgt; break; }
          cum += h;
        }
        s_remaining = rem - cum;
        s_prefix = prefix | ((uint32_t)digit << shift);
        s_pmask = pmask | (255u << shift);
      }
      __syncthreads();
    }
  }
  const uint32_t T = s_prefix;
  const int need_eq = kk > 0 ? s_remaining : 0;
  int gt = 0, eq = 0;
  if (kk > 0) {
    for (int j = j0; j < j1; ++j) {
      if (!((cand >> (j - j0)) & 1ull)) continue;
      const uint32_t key = order_key(sc[j]);
      gt += key > T;
      eq += key == T;
    }
  }
  int tot;
  const int eq_before = block_exclusive_scan(eq, scan_tmp, &tot);
  const int take_eq = max(0, min(eq, need_eq - eq_before));
  const int pos0 = block_exclusive_scan(gt + take_eq, scan_tmp, &tot);
  if (kk > 0) {
    int pos = pos0, taken = 0;
    for (int j = j0; j < j1; ++j) {
      if (!((cand >> (j - j0)) & 1ull)) continue;
      const uint32_t key = order_key(sc[j]);
      if (key > T || (key == T && taken < take_eq)) {
        taken += key == T;
        out[pos++] = j;
      }
    }
  }
  for (int i = kk + tid; i < a.top_k; i += 1024) out[i] = -1;
}

template <int D, int GM, bool BF16>
hipError_t launch_t(const SelectArgs& a, hipStream_t stream) {
  dim3 grid((a.n_blocks + kBlocksPerWg - 1) / kBlocksPerWg, a.batch * a.n_kv_heads);
  if (a.n_blocks > 0)
    hipLaunchKernelGGL((select_scores_kernel<D, GM, BF16>), grid, dim3(256), 0, stream, a);
  hipLaunchKernelGGL(topk_kernel, dim3(a.batch * a.n_kv_heads), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_g(const SelectArgs& a, hipStream_t stream) {
  const int G = a.n_q_heads / a.n_kv_heads;
  if (G <= 4) return launch_t<D, 4, BF16>(a, stream);
  if (G <= 8) return launch_t<D, 8, BF16>(a, stream);
  return launch_t<D, 16, BF16>(a, stream);
}

}  // namespace

hipError_t launch_select_topk(const SelectArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) return a.bf16 ? launch_g<64, true>(a, stream) : launch_g<64, false>(a, stream);
  return a.bf16 ? launch_g<128, true>(a, stream) : launch_g<128, false>(a, stream);
}

}  // namespace bsattn
