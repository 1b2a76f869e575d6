// Per-block key summaries: the block mean (first cumulant) and a rank-r factor
// of the block covariance (second cumulant), as the COBS explainer's technical
// summary defines them in sections 2.2 and 2.3 (mean key and covariance per
// block; covariance kept as its top-r eigenvectors and eigenvalues).
//
// Covariance normalisation is 1/L (population): the second cumulant of the
// block's empirical key distribution.  The top-r eigenpairs come from the
// L x L centred Gram matrix G = C C^T / L (same non-zero eigenvalues as
// Sigma = C^T C / L): if G w = lambda w with |w| = 1, then sqrt(lambda) v =
// C^T w / sqrt(L).  G is diagonalised by parallel cyclic Jacobi in LDS
// (round-robin pairing: 32 disjoint rotations per round, 63 rounds a sweep).
#include "launch.hpp"

namespace bsattn {
namespace {

// 16-byte chunk c (row c / CH, chunk c % CH of it) of block blk of pair bh's keys:
// contiguous [B*Hkv, kv_capacity, d], or through the block table of a paged cache.
template <int D, bool BF16>
__device__ __forceinline__ const void* key_chunk(const SummaryArgs& a, int bh, int blk, int c) {
  constexpr int CH = D / (BF16 ? 8 : 4);
  constexpr size_t RB = D * (BF16 ? 2 : 4);
  const int t = blk * kBlock + c / CH;
  const size_t row = a.paged.block_table != nullptr
                         ? paged_row(a.paged, bh / a.n_kv_heads, bh % a.n_kv_heads, a.n_kv_heads, t)
                         : (size_t)bh * a.kv_capacity + t;
  return reinterpret_cast<const char*>(a.K) + row * RB + (c % CH) * 16;
}

template <bool BF16>
__device__ __forceinline__ void load_chunk(const void* p, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  if constexpr (BF16) {
    out[0] = bf16lo(v.x); out[1] = bf16hi(v.x); out[2] = bf16lo(v.y); out[3] = bf16hi(v.y);
    out[4] = bf16lo(v.z); out[5] = bf16hi(v.z); out[6] = bf16lo(v.w); out[7] = bf16hi(v.w);
  } else {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  }
}

// ----------------------------------------------------------------- mean only
// One workgroup per (block, b*Hkv).  Streams the block's keys with 16-byte loads.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void summaries_mean_kernel(SummaryArgs a) {
  constexpr int E = BF16 ? 8 : 4;  // elements per 16-byte chunk
  constexpr int CH = D / E;        // chunks per key row
  constexpr int PER = kBlock * CH / 256;
  __shared__ float red[256][E + 1];
  const int tid = threadIdx.x;
  const int blk = a.first_block + blockIdx.x;
  const int bh = blockIdx.y;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    float v[E];
    load_chunk<BF16>(key_chunk<D, BF16>(a, bh, blk, tid + 256 * k), v);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += v[e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[tid][e] = acc[e];
  __syncthreads();
  if (tid < CH) {
    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = 0.f;
    for (int m = tid; m < 256; m += CH) {
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] += red[m][e];
    }
    const size_t off = ((size_t)bh * a.nblk_capacity + blk) * D + tid * E;
    if (a.mean_bf16) {  // round to nearest even, two values per 32-bit store
      uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.mean) + off);
#pragma unroll
      for (int e = 0; e < E; e += 2) dst[e / 2] = cvt_pk_bf16(s[e] * (1.0f / kBlock), s[e + 1] * (1.0f / kBlock));
    } else {
      float* dst = static_cast<float*>(a.mean) + off;
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e] = s[e] * (1.0f / kBlock);
    }
  }
}

// ----------------------------------------------------------------- mean + factor
constexpr int kCtStride = 68;  // floats per row of the transposed block (bank spread, 16-B aligned)
constexpr int kGStride = 65;   // floats per row of the Gram matrix
constexpr int kMaxSweeps = 12;

// Pair i of round r in the round-robin schedule over 64 indices.
__device__ __forceinline__ void rr_pair(int r, int i, int& p, int& q) {
  if (i == 0) { p = r; q = 63; }
  else { p = (r + i) % 63; q = (r - i + 63) % 63; }
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void summaries_factor_kernel(SummaryArgs a) {
  constexpr int E = BF16 ? 8 : 4;
  constexpr int CH = D / E;
  constexpr int PER = kBlock * CH / 256;
  __shared__ __attribute__((aligned(16))) float Ct[D * kCtStride];  // Ct[d][r], centred keys
  __shared__ float G[64 * kGStride];
  __shared__ float W[64 * kGStride];                                // eigenvectors as columns
  __shared__ float mu[D];
  __shared__ float rc[32], rs[32], rt[32];
  __shared__ int rp[32], rq[32];
  __shared__ float red[8];
  __shared__ int pick[8];
  __shared__ float F[8 * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int blk = a.first_block + blockIdx.x;
  const int bh = blockIdx.y;

  // 1. block -> LDS, transposed
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int c = tid + 256 * k;
    const int row = c / CH, col0 = (c % CH) * E;
    float v[E];
    load_chunk<BF16>(key_chunk<D, BF16>(a, bh, blk, c), v);
#pragma unroll
    for (int e = 0; e < E; ++e) Ct[(col0 + e) * kCtStride + row] = v[e];
  }
  __syncthreads();
  // 2. mean
  for (int d = tid; d < D; d += 256) {
    float s = 0.f;
    for (int r = 0; r < kBlock; ++r) s += Ct[d * kCtStride + r];
    s *= (1.0f / kBlock);
    mu[d] = s;  // the covariance is taken about the fp32 mean; only the stored copy is rounded
    const size_t off = ((size_t)bh * a.nblk_capacity + blk) * D + d;
    if (a.mean_bf16) static_cast<uint16_t*>(a.mean)[off] = (uint16_t)(cvt_pk_bf16(s, 0.f) & 0xffffu);
    else static_cast<float*>(a.mean)[off] = s;
  }
  __syncthreads();
  // 3. centre
  for (int i = tid; i < D * kBlock; i += 256) {
    const int d = i / kBlock, r = i % kBlock;
    Ct[d * kCtStride + r] -= mu[d];
  }
  // identity eigenvector matrix
  for (int i = tid; i < 64 * 64; i += 256) W[(i / 64) * kGStride + (i % 64)] = (i / 64 == i % 64) ? 1.f : 0.f;
  __syncthreads();
  // 3b. query-subspace projection [COBS 2.3, compression]: the centred keys
  // become P (k - mean), ED numbers each (rows ED .. D-1 of Ct zeroed), so the
  // steps below factorise the projected covariance P Sigma P^T.  Wave w owns
  // basis rows w, w + 4, ...; lane r owns token r.
  const int ED = a.basis != nullptr ? a.sub_dim : D;
  if (a.basis != nullptr) {
    const float* P = a.basis + (size_t)(bh % a.n_kv_heads) * ED * D;
    float acc[D / 4];
#pragma unroll
    for (int u = 0; u < D / 4; ++u) acc[u] = 0.f;
    for (int d = 0; d < D; ++d) {
      const float c = Ct[d * kCtStride + lane];
#pragma unroll
      for (int u = 0; u < D / 4; ++u) {
        const int j = wid + 4 * u;
        if (j < ED) acc[u] = fmaf(P[(size_t)j * D + d], c, acc[u]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < D / 4; ++u) {
      const int j = wid + 4 * u;
      Ct[j * kCtStride + lane] = j < ED ? acc[u] : 0.f;
    }
    __syncthreads();
  }
  // 4. Gram G = C C^T / L, thread t owns rows 4*(t/16).., cols 4*(t%16)..
  {
    const int x0 = 4 * (tid >> 4), y0 = 4 * (tid & 15);
    float g[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) g[i][j] = 0.f;
    for (int d = 0; d < ED; ++d) {
      const float4 xa = *reinterpret_cast<const float4*>(&Ct[d * kCtStride + x0]);
      const float4 yb = *reinterpret_cast<const float4*>(&Ct[d * kCtStride + y0]);
      const float xs[4] = {xa.x, xa.y, xa.z, xa.w};
      const float ys[4] = {yb.x, yb.y, yb.z, yb.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) g[i][j] = fmaf(xs[i], ys[j], g[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) G[(x0 + i) * kGStride + y0 + j] = g[i][j] * (1.0f / kBlock);
  }
  __syncthreads();

  // 5. Jacobi sweeps
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    for (int r = 0; r < 63; ++r) {
      if (tid < 32) {
        int p, q;
        rr_pair(r, tid, p, q);
        const float app = G[p * kGStride + p], aqq = G[q * kGStride + q], apq = G[p * kGStride + q];
        float c = 1.f, s = 0.f, t = 0.f;
        if (apq != 0.f && fabsf(apq) > 1e-10f * (fabsf(app) + fabsf(aqq))) {
          const float tau = (aqq - app) / (2.f * apq);
          const float sg = tau >= 0.f ? 1.f : -1.f;
          t = fabsf(tau) > 1e18f ? 0.5f / tau : sg / (fabsf(tau) + sqrtf(1.f + tau * tau));
          c = 1.f / sqrtf(1.f + t * t);
          s = t * c;
        }
        rp[tid] = p; rq[tid] = q; rc[tid] = c; rs[tid] = s; rt[tid] = t;
      }
      __syncthreads();
      // G <- J^T G J on 2x2 pair blocks (P rows, Q cols); each block owned by one thread.
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int blkid = tid + 256 * k;  // 0..1023
        const int P = blkid >> 5, Q = blkid & 31;
        const int pP = rp[P], qP = rq[P], pQ = rp[Q], qQ = rq[Q];
        const float cP = rc[P], sP = rs[P], cQ = rc[Q], sQ = rs[Q];
        const float g00 = G[pP * kGStride + pQ], g01 = G[pP * kGStride + qQ];
        const float g10 = G[qP * kGStride + pQ], g11 = G[qP * kGStride + qQ];
        // rows: new_p = c g_p - s g_q ; new_q = s g_p + c g_q
        const float r00 = cP * g00 - sP * g10, r01 = cP * g01 - sP * g11;
        const float r10 = sP * g00 + cP * g10, r11 = sP * g01 + cP * g11;
        float n00 = cQ * r00 - sQ * r01, n01 = sQ * r00 + cQ * r01;
        float n10 = cQ * r10 - sQ * r11, n11 = sQ * r10 + cQ * r11;
        if (P == Q && (sP != 0.f)) {
          const float tP = rt[P];
          n00 = g00 - tP * g01;
          n11 = g11 + tP * g01;
          n01 = 0.f;
          n10 = 0.f;
        }
        G[pP * kGStride + pQ] = n00; G[pP * kGStride + qQ] = n01;
        G[qP * kGStride + pQ] = n10; G[qP * kGStride + qQ] = n11;
      }
      // W <- W J (columns p, q of every row)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int u = tid + 256 * k;  // 0..2047
        const int row = u >> 5, P = u & 31;
        const int p = rp[P], q = rq[P];
        const float c = rc[P], s = rs[P];
        const float wp = W[row * kGStride + p], wq = W[row * kGStride + q];
        W[row * kGStride + p] = c * wp - s * wq;
        W[row * kGStride + q] = s * wp + c * wq;
      }
      __syncthreads();
    }
    // convergence: off-diagonal mass against the diagonal.  In fp32 the sum of
    // squared off-diagonal entries settles near 5e-14 of the diagonal's (the
    // rounding floor of a 64 x 64 rotation sequence), reached after 6 or 7
    // sweeps from a Gram of centred keys; 1e-12 (off-diagonal norm 1e-6 of the
    // diagonal's) stops there instead of running every sweep at the floor.
    float off = 0.f, dia = 0.f;
    for (int i = tid; i < 64 * 64; i += 256) {
      const int x = i >> 6, y = i & 63;
      const float g = G[x * kGStride + y];
      if (x == y) dia += g * g; else off += g * g;
    }
    off = wave_sum(off);
    dia = wave_sum(dia);
    if (lane == 0) { red[wid] = off; red[4 + wid] = dia; }
    __syncthreads();
    const float offt = red[0] + red[1] + red[2] + red[3];
    const float diat = red[4] + red[5] + red[6] + red[7];
    __syncthreads();
    if (offt <= 1e-12f * diat) break;
  }

  // 6. top-r eigenvalues (descending, lower index first on ties)
  if (tid < 64) {
    const float lx = G[tid * kGStride + tid];
    int rank = 0;
    for (int y = 0; y < 64; ++y) {
      const float ly = G[y * kGStride + y];
      rank += (ly > lx) || (ly == lx && y < tid);
    }
    if (rank < a.rank) pick[rank] = tid;
  }
  __syncthreads();
  // 7. factor rows sqrt(lambda_i) v_i = C^T w_i / sqrt(L)
  for (int o = tid; o < a.rank * ED; o += 256) {
    const int i = o / ED, d = o % ED;
    const int x = pick[i];
    float s = 0.f;
    for (int r = 0; r < kBlock; ++r) s = fmaf(Ct[d * kCtStride + r], W[r * kGStride + x], s);
    F[i * D + d] = s * 0.125f;  // 1/sqrt(64)
  }
  __syncthreads();
  // 8. sign: entry of largest magnitude (first on ties) made positive; one wave per row
  for (int i = wid; i < a.rank; i += 4) {
    float best = -1.f;
    int bidx = D;
    for (int d = lane; d < ED; d += 64) {
      const float v = fabsf(F[i * D + d]);
      if (v > best) { best = v; bidx = d; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ob = __shfl_xor(best, o);
      const int oi = __shfl_xor(bidx, o);
      if (ob > best || (ob == best && oi < bidx)) { best = ob; bidx = oi; }
    }
    const float sign = F[i * D + bidx] < 0.f ? -1.f : 1.f;
    const size_t frow = ((size_t)bh * a.nblk_capacity + blk) * a.rank + i;
    if (a.factor_fp4) {
      // FP4 E2M1 with one scale per row: scale = row max / 6, each entry the
      // nearest E2M1 value of entry / scale; lane l packs entries 2l (low
      // nibble) and 2l + 1 into byte l
      const float scale = best / 6.0f;
      for (int l = lane; l < ED / 2; l += 64) {
        const float v0 = scale > 0.f ? (sign * F[i * D + 2 * l]) / scale : 0.f;
        const float v1 = scale > 0.f ? (sign * F[i * D + 2 * l + 1]) / scale : 0.f;
        static_cast<uint8_t*>(a.factor)[frow * (ED / 2) + l] = (uint8_t)(e2m1_code(v0) | (e2m1_code(v1) << 4));
      }
      if (lane == 0) a.factor_scale[frow] = scale;
    } else {
      float* dst = static_cast<float*>(a.factor) + frow * ED;
      for (int d = lane; d < ED; d += 64) dst[d] = sign * F[i * D + d];
    }
  }
}

template <int D, bool BF16>
hipError_t launch_t(const SummaryArgs& a, hipStream_t stream) {
  dim3 grid(a.n_blocks, a.bh);
  if (a.rank == 0)
    hipLaunchKernelGGL((summaries_mean_kernel<D, BF16>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((summaries_factor_kernel<D, BF16>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Append: one workgroup per (b, K/V head) copies the new token's K and V rows
// (16-byte chunks) into row `pos` of the cache.  Paged: a block-table entry
// outside [0, n_pages) (an unallocated page) is not written through: the store is
// skipped, so a stale or missing entry never overwrites another sequence's page.
__global__ __launch_bounds__(64) void append_kv_kernel(AppendArgs a) {
  const size_t bh = blockIdx.x;
  const int n16 = a.row_bytes / 16;
  const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const char*>(a.K_new) + bh * a.row_bytes);
  const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const char*>(a.V_new) + bh * a.row_bytes);
  if (a.paged.block_table != nullptr) {
    const int page = a.paged.block_table[(bh / a.n_kv_heads) * a.paged.max_pages + (a.pos >> a.paged.page_shift)];
    if (page < 0 || page >= a.paged.n_pages) return;  // wave-uniform: the whole workgroup skips
  }
  const size_t row = a.paged.block_table != nullptr
                         ? paged_row(a.paged, (int)bh / a.n_kv_heads, (int)bh % a.n_kv_heads, a.n_kv_heads, a.pos)
                         : bh * a.kv_capacity + a.pos;
  const size_t dst = row * (size_t)a.row_bytes;
  uint4* kd = reinterpret_cast<uint4*>(static_cast<char*>(a.K) + dst);
  uint4* vd = reinterpret_cast<uint4*>(static_cast<char*>(a.V) + dst);
  for (int i = threadIdx.x; i < n16; i += 64) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

hipError_t launch_append(const AppendArgs& a, int n_pairs, hipStream_t stream) {
  hipLaunchKernelGGL(append_kv_kernel, dim3(n_pairs), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_summaries(const SummaryArgs& a, hipStream_t stream) {
  if (a.n_blocks == 0) return hipSuccess;
  if (a.head_dim == 64) return a.bf16 ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
  return a.bf16 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
}

}  // namespace bsattn
