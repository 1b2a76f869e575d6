// The VALU block scorer, for the dtype mixes the MFMA scorer does not take
// (fp32 queries, fp32 means or fp32 factor rows): per query head h and complete
// block j the first-order score q~.mean_j, plus 1/2 sum_i (factor_ji . q~)^2
// for a rank-r summary (COBS explainer, technical summary 2.2 and 2.3), then
// the group score ln sum_h exp(s_hj) (section 2.1).  16 lanes (one DPP row)
// share one block, lane l owning the 4-dim chunks l, 16 + l, ... of every query
// head, so each load instruction reads 256 contiguous bytes of a summary row;
// DPP row rotations sum the 16 partial dot products.  Waves score runs of
// blocks with the next group's loads in flight.
//
// The kernel has one instantiation per (group size, rank bound, dtype mix);
// this file is compiled once per head dimension and query dtype
// (BSATTN_VALU_D, BSATTN_VALU_BF16), so the objects build in parallel.
#include <type_traits>

#include "launch.hpp"

#ifndef BSATTN_VALU_D
#error "compile with -DBSATTN_VALU_D=64|128 -DBSATTN_VALU_BF16=0|1"
#endif

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

// Scoring waves: 2 per SIMD when a lane's query values and its two stages of
// summary rows take at most 160 registers, else 1 (the whole 512-register budget).
constexpr bool scores_heavy(int GM, int RM, int PB, int D) {
  return GM * (D / 16) + 2 * PB * (1 + RM) * (D / 16) > 160;
}

template <int D, int GM, int RM, int PB, bool BF16, bool MB, bool F4>
__global__ __launch_bounds__(256, scores_heavy(GM, RM, PB, D) ? 1 : 2) void select_scores_kernel(SelectArgs a) {
  constexpr int SL = D / 16;  // dims per lane: 4-dim chunks sub, 16 + sub, ...
  constexpr int NC = SL / 4;  // 16-byte chunks per lane per row
  constexpr int UB = 4 * PB;  // blocks per unit: PB per 16-lane row
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * 4 + wid;
  const int n_pairs = a.batch * a.n_kv_heads;
  const int pair = gw / a.n_part, wi = gw % a.n_part;
  if (pair >= n_pairs) return;  // no barriers: waves are independent
  const int sub = lane & 15, r16 = lane >> 4;
  const int b = pair / a.n_kv_heads, g = pair % a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int NB = a.n_blocks;
  const int rank = a.rank;

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

  // mean rows: 4 dims per 16-byte (fp32) or 8-byte (bf16, widened at compute
  // time so the loads stay plain) chunk
  using MeanChunk = typename std::conditional<MB, u32x2, float4>::type;
  const MeanChunk* mean4 = reinterpret_cast<const MeanChunk*>(a.mean);
  // factor rows: 4 dims per 16-byte fp32 chunk, or per 2 bytes of FP4 codes
  // (dim k of the chunk in bits 4k .. 4k+3) with the row's scale beside them
  using FacChunk = typename std::conditional<F4, uint32_t, float4>::type;
  const float4* fac4 = reinterpret_cast<const float4*>(a.factor);
  const uint16_t* fac2 = reinterpret_cast<const uint16_t*>(a.factor);
  struct Stage {
    MeanChunk m[PB][NC];
    FacChunk v[PB][RM > 0 ? RM : 1][NC];
    float fs[PB][RM > 0 ? RM : 1];  // FP4 row scales
  };
  // Every load is issued unconditionally (blocks past the end re-read the last
  // block, factor rows past the rank re-read the last row, both ignored), so
  // the compiler's waits count exactly the loads issued after each stage.
  auto load = [&](int u, Stage& st) {
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int j = min(u * UB + 4 * p + r16, NB - 1);
      const size_t row = (size_t)pair * a.nblk_capacity + j;
#pragma unroll
      for (int c = 0; c < NC; ++c) st.m[p][c] = mean4[row * (D / 4) + 16 * c + sub];
#pragma unroll
      for (int i = 0; i < RM; ++i) {
        const size_t fr = row * rank + min(i, rank - 1);
        if constexpr (F4) {
#pragma unroll
          for (int c = 0; c < NC; ++c) st.v[p][i][c] = fac2[fr * (D / 4) + 16 * c + sub];
          st.fs[p][i] = a.factor_scale[fr];
        } else {
#pragma unroll
          for (int c = 0; c < NC; ++c) st.v[p][i][c] = fac4[fr * (D / 4) + 16 * c + sub];
        }
      }
    }
  };
  auto dot = [&](const float4* v, int h) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      acc = fmaf(q[h][4 * c], v[c].x, acc);
      acc = fmaf(q[h][4 * c + 1], v[c].y, acc);
      acc = fmaf(q[h][4 * c + 2], v[c].z, acc);
      acc = fmaf(q[h][4 * c + 3], v[c].w, acc);
    }
    return acc;
  };
  auto comp = [&](int u, const Stage& st) {
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int j = u * UB + 4 * p + r16;
      float s[GM];
      float4 mv[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if constexpr (MB) {
          const u32x2 w = st.m[p][c];
          mv[c] = float4{bf16lo(w[0]), bf16hi(w[0]), bf16lo(w[1]), bf16hi(w[1])};
        } else {
          mv[c] = st.m[p][c];
        }
      }
#pragma unroll
      for (int h = 0; h < GM; ++h) s[h] = row16_sum(dot(mv, h));
#pragma unroll
      for (int i = 0; i < RM; ++i) {
        if (i < rank) {
          float4 fv[NC];
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            if constexpr (F4) {
              const uint32_t w = st.v[p][i][c];
              fv[c] = float4{e2m1_value(w), e2m1_value(w >> 4), e2m1_value(w >> 8), e2m1_value(w >> 12)};
            } else {
              fv[c] = st.v[p][i][c];
            }
          }
#pragma unroll
          for (int h = 0; h < GM; ++h) {
            float pr = row16_sum(dot(fv, h));
            if constexpr (F4) pr *= st.fs[p][i];  // the row's scale, once per projection
            s[h] = fmaf(0.5f * pr, pr, s[h]);
          }
        }
      }
      if (sub == 0 && j < NB) {
        float mx = s[0];
#pragma unroll
        for (int h = 1; h < GM; ++h)
          if (h < G) mx = fmaxf(mx, s[h]);
        float sum = 0.f;
#pragma unroll
        for (int h = 0; h < GM; ++h)
          if (h < G) sum += __builtin_amdgcn_exp2f((s[h] - mx) * kLog2e);
        // sum >= 1 (the max term is exactly 1): log2 needs no range care
        a.scores[(size_t)pair * a.nblk_capacity + j] = fmaf(__builtin_amdgcn_logf(sum), kLn2, mx);
      }
    }
  };

  // two units in flight (A: even steps, B: odd), every path written out; one
  // unit when a lane's query values and two stages of summary rows would pass
  // 256 registers (16 query heads with fp32 rank-8 factor rows at D = 128):
  // the second stage would spill
  constexpr int kStageRegs = PB * ((MB ? SL / 2 : SL) + RM * (F4 ? NC + 1 : SL));
  constexpr bool kOneStage = GM * SL + 2 * kStageRegs > 256;
  const int n_units = (NB + UB - 1) / UB;
  const int u0 = wi * a.per_wave, u1 = min(u0 + a.per_wave, n_units);
  const int n = u1 - u0;
  Stage A, B;
  if constexpr (kOneStage) {
    for (int u = u0; u < u1; ++u) {
      load(u, A);
      comp(u, A);
    }
  } else if (n >= 4) {
    load(u0, A);
    load(u0 + 1, B);
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
    comp(u0, A);
    load(u0 + 2, A);
    comp(u0 + 1, B);
    comp(u0 + 2, A);
  } else if (n == 2) {
    load(u0, A);
    load(u0 + 1, B);
    comp(u0, A);
    comp(u0 + 1, B);
  } else if (n == 1) {
    load(u0, A);
    comp(u0, A);
  }
}

template <int D, int GM, int RM, bool BF16>
hipError_t launch_t(const SelectArgs& a0, hipStream_t stream) {
  constexpr int PB = RM == 0 ? 4 : (RM <= 2 ? 2 : 1);  // blocks per 16-lane row per unit
  SelectArgs a = a0;
  const int n_pairs = a.batch * a.n_kv_heads;
  if (a.n_blocks > 0) {
    split_units(a, (a.n_blocks + 4 * PB - 1) / (4 * PB), 256 * (scores_heavy(GM, RM, PB, D) ? 4 : 8));
    const long long waves = (long long)n_pairs * a.n_part;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (RM > 0 && a.factor_fp4) {
      if (a.mean_bf16) hipLaunchKernelGGL((select_scores_kernel<D, GM, RM, PB, BF16, true, RM != 0>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((select_scores_kernel<D, GM, RM, PB, BF16, false, RM != 0>), grid, block, 0, stream, a);
    } else {
      if (a.mean_bf16) hipLaunchKernelGGL((select_scores_kernel<D, GM, RM, PB, BF16, true, false>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((select_scores_kernel<D, GM, RM, PB, BF16, false, false>), grid, block, 0, stream, a);
    }
  }
  return hipGetLastError();
}

template <int D, int GM, bool BF16>
hipError_t launch_r(const SelectArgs& a, hipStream_t stream) {
  if (a.rank == 0) return launch_t<D, GM, 0, BF16>(a, stream);
  if (a.rank <= 2) return launch_t<D, GM, 2, BF16>(a, stream);
  if (a.rank <= 4) return launch_t<D, GM, 4, BF16>(a, stream);
  return launch_t<D, GM, 8, BF16>(a, stream);
}

template <int D, bool BF16>
hipError_t launch_g_impl(const SelectArgs& a, hipStream_t stream) {
  const int G = a.n_q_heads / a.n_kv_heads;
  if (G <= 4) return launch_r<D, 4, BF16>(a, stream);
  if (G <= 8) return launch_r<D, 8, BF16>(a, stream);
  return launch_r<D, 16, BF16>(a, stream);
}

}  // namespace

template <int D, bool BF16>
hipError_t launch_valu_scores(const SelectArgs& a, hipStream_t stream) {
  return launch_g_impl<D, BF16>(a, stream);
}
template hipError_t launch_valu_scores<BSATTN_VALU_D, (BSATTN_VALU_BF16 != 0)>(const SelectArgs&, hipStream_t);

}  // namespace bsattn
