// Per-block key summaries: the block mean (first cumulant) and a rank-r factor
// of the block covariance (second cumulant), as the COBS explainer's technical
// summary defines them in sections 2.2 and 2.3 (mean key and covariance per
// block; covariance kept as its top-r eigenvectors and eigenvalues).
//
// Covariance normalisation is 1/L (population): the second cumulant of the
// block's empirical key distribution.  The top-r eigenpairs come from the
// L x L centred Gram matrix G = C C^T / L (same non-zero eigenvalues as
// Sigma = C^T C / L): if G w = lambda w with |w| = 1, then sqrt(lambda) v =
// C^T w / sqrt(L).  The symmetric eigenproblem is solved the textbook way for
// a few extreme eigenpairs (Golub & Van Loan, the symmetric QR and tridiagonal
// chapters): Householder reduction of G to tridiagonal T in LDS, the top r
// eigenvalues of T by multisection on Sturm counts, their eigenvectors by
// inverse iteration on T (pivoted elimination; the r vectors re-orthonormalised
// after each solve, which also separates close eigenvalues), then the
// reflections applied back.
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
constexpr int kGStride = 65;   // floats per row of the Gram matrix and of the eigenvector work rows

// Sum, min and max over the 64 lanes, the same value in every lane: row_ror
// 8, 4, 2, 1 leave each 16-lane row's total in its lanes, then the four rows'
// first lanes are combined in a fixed order.
#define BSATTN_ROW_ALL(OP, v)                                                                      \
  do {                                                                                             \
    v = OP(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false))); \
    v = OP(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false))); \
    v = OP(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false))); \
    v = OP(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false))); \
  } while (0)
__device__ __forceinline__ float rl(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
__device__ __forceinline__ float f_add(float x, float y) { return x + y; }
__device__ __forceinline__ float wsum(float v) {
  BSATTN_ROW_ALL(f_add, v);
  return (rl(v, 0) + rl(v, 16)) + (rl(v, 32) + rl(v, 48));
}
__device__ __forceinline__ float wmin(float v) {
  BSATTN_ROW_ALL(fminf, v);
  return fminf(fminf(rl(v, 0), rl(v, 16)), fminf(rl(v, 32), rl(v, 48)));
}
__device__ __forceinline__ float wmax(float v) {
  BSATTN_ROW_ALL(fmaxf, v);
  return fmaxf(fmaxf(rl(v, 0), rl(v, 16)), fmaxf(rl(v, 32), rl(v, 48)));
}
#undef BSATTN_ROW_ALL

template <int D, bool BF16>
__global__ __launch_bounds__(256) void summaries_factor_kernel(SummaryArgs a) {
  constexpr int E = BF16 ? 8 : 4;
  constexpr int CH = D / E;
  constexpr int PER = kBlock * CH / 256;
  __shared__ __attribute__((aligned(16))) float Ct[D * kCtStride];  // Ct[d][r], centred keys
  __shared__ float G[64 * kGStride];
  __shared__ __attribute__((aligned(16))) float W[64 * kGStride];  // basis chunks; eigenvector work rows
  __shared__ float mu[D];
  __shared__ float td[64], te[64], tb[64], tp[128];  // T's diagonal, off-diagonal; reflector betas; p
  __shared__ float xc[64], uw[4][128];               // current column; each wave's reflector vector
  __shared__ __attribute__((aligned(16))) float kpart[4];  // each wave's share of u.(beta p)
  __shared__ float lam[8];
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
  __syncthreads();
  // 3b. query-subspace projection [COBS 2.3, compression]: the centred keys
  // become P (k - mean), ED numbers each (rows ED .. D-1 of Ct zeroed), so the
  // steps below factorise the projected covariance P Sigma P^T.  Wave w owns
  // basis rows w, w + 4, ...; lane r owns token r.  P passes through LDS (W,
  // free until the eigenvectors) 32 columns at a time; every lane of a wave
  // reads the same P entries (broadcast), 4 columns per read.
  const int ED = a.basis != nullptr ? a.sub_dim : D;
  if (a.basis != nullptr) {
    const float* P = a.basis + (size_t)(bh % a.n_kv_heads) * ED * D;
    float4* const Pc = reinterpret_cast<float4*>(W);  // [ED][8] float4: columns d0 .. d0 + 31
    float acc[D / 4];
#pragma unroll
    for (int u = 0; u < D / 4; ++u) acc[u] = 0.f;
    for (int d0 = 0; d0 < D; d0 += 32) {
      for (int i = tid; i < ED * 8; i += 256)
        Pc[i] = *reinterpret_cast<const float4*>(P + (size_t)(i >> 3) * D + d0 + 4 * (i & 7));
      __syncthreads();
#pragma unroll 2
      for (int c4 = 0; c4 < 8; ++c4) {
        const float* cr = Ct + (d0 + 4 * c4) * kCtStride + lane;
        const float x0 = cr[0], x1 = cr[kCtStride], x2 = cr[2 * kCtStride], x3 = cr[3 * kCtStride];
#pragma unroll
        for (int u = 0; u < D / 4; ++u) {
          const int j = wid + 4 * u;
          if (j < ED) {
            const float4 p4 = Pc[j * 8 + c4];
            acc[u] = fmaf(p4.w, x3, fmaf(p4.z, x2, fmaf(p4.y, x1, fmaf(p4.x, x0, acc[u]))));
          }
        }
      }
      __syncthreads();
    }
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
#pragma unroll 4
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

  // 5. Householder tridiagonalisation, G = Q T Q^T with Q = H_0 .. H_61: the
  //    reflection H_k = I - beta_k u u^T (u zero in rows 0 .. k) zeroes column
  //    k below the subdiagonal; the trailing block becomes B - u w^T - w u^T
  //    with p = beta B u, w = p - (beta/2)(u.p) u.  Thread t keeps row t / 4,
  //    columns t % 4 + 4 (j + sh) (j < 16), of the matrix in registers for all
  //    62 steps; every 4 steps the row shifts down one register (sh grows; the
  //    column dropped is already reduced), so the column a step hands on
  //    (xc) is always register 0 of its owners: no dynamic register index.
  //    Every wave forms u itself from xc into its own copy uw[wave] (zero
  //    past row 63, like tp), so a step needs two barriers (p and the waves'
  //    shares of u.p complete; the next column complete).  u_k is kept in row k of G for the
  //    back-transformation.
  constexpr int S = kGStride;
  const int grow = tid >> 2, gq = tid & 3;
  float gr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) gr[j] = G[grow * S + gq + 4 * j];
  int sh = 0;
  uw[wid][64 + lane] = 0.f;
  if (tid < 64) tp[64 + tid] = 0.f;
  if (gq == 0) xc[grow] = gr[0];  // column 0
  __syncthreads();  // every row loaded from G (now free for u) and column 0 in xc
  for (int k = 0; k < 62; ++k) {
    float* const uu = uw[wid];
    float beta = 0.f;  // the same in every wave
    {
      const float xl = xc[lane];
      const float xr = lane > k ? xl : 0.f;
      const float x0r = rl(xl, k + 1);
      const float sr = wsum(lane > k + 1 ? xr * xr : 0.f);
      float alpha = x0r, u = 0.f;
      if (sr > 1e-30f && sr < 1e30f) {
        const float mu = sqrtf(fmaf(x0r, x0r, sr));
        const float u0 = x0r >= 0.f ? x0r + mu : x0r - mu;  // no cancellation
        alpha = x0r >= 0.f ? -mu : mu;
        beta = 2.f / fmaf(u0, u0, sr);
        u = lane == k + 1 ? u0 : xr;
      } else if (sr != 0.f) {
        // squares near the ends of the range: u is scale-free, so the column
        // is scaled to max-abs 1 first
        const float xm = wmax(fabsf(xr));
        const float x = xr / xm;
        const float sig = wsum(lane > k + 1 ? x * x : 0.f);
        const float x0 = rl(x, k + 1);
        const float mu = sqrtf(fmaf(x0, x0, sig));
        const float u0 = x0 >= 0.f ? x0 + mu : x0 - mu;
        alpha = (x0 >= 0.f ? -mu : mu) * xm;
        beta = 2.f / fmaf(u0, u0, sig);
        u = lane == k + 1 ? u0 : x;
      }  // sr == 0: the column is already reduced (beta = 0, u = 0)
      uu[lane] = u;  // zero in rows 0 .. k
      if (wid == 0) {
        G[k * S + lane] = u;
        const float dk = rl(xl, k);
        if (lane == 0) {
          td[k] = dk;
          te[k] = alpha;
          tb[k] = beta;
        }
      }
    }
    // p = beta B u for this row (rows 0 .. k get 0, so they stay untouched),
    // and this wave's share of u.(beta p)
    const float* const uc4 = uu + gq + 4 * sh;
    const float* const tc4 = tp + gq + 4 * sh;
    float ucv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) ucv[j] = uc4[4 * j];
    const float ur = uu[grow];
    float pa[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) pa[j & 3] = fmaf(gr[j], ucv[j], pa[j & 3]);
    float pr = (pa[0] + pa[1]) + (pa[2] + pa[3]);
    pr += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(pr), 0xb1, 0xf, 0xf, false));  // quad_perm 1,0,3,2
    pr += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(pr), 0x4e, 0xf, 0xf, false));  // quad_perm 2,3,0,1
    const float tr = grow > k ? beta * pr : 0.f;
    if (gq == 0) tp[grow] = tr;
    const float part = wsum(gq == 0 ? ur * tr : 0.f);
    if (lane == 0) kpart[wid] = part;
    __syncthreads();
    const float4 kp = *reinterpret_cast<const float4*>(kpart);
    const float kk = 0.5f * beta * ((kp.x + kp.y) + (kp.z + kp.w));  // (beta / 2) u.p
    const float wr = tr - kk * ur;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float uc = ucv[j], wc = tc4[4 * j] - kk * uc;
      gr[j] -= fmaf(ur, wc, wr * uc);
    }
    if (((k + 1) & 3) == 0) {
#pragma unroll
      for (int j = 0; j < 15; ++j) gr[j] = gr[j + 1];
      gr[15] = 0.f;
      ++sh;
    }
    if (gq == ((k + 1) & 3)) xc[grow] = gr[0];  // column k + 1
    __syncthreads();
  }
  // the last 2 x 2 block: column 62 is in xc; G[63][63] from its owner
  if (tid == 0) {
    td[62] = xc[62];
    te[62] = xc[63];
    tb[62] = 0.f;
  }
  if (grow == 63 && gq == 3) td[63] = gr[0];  // column 63 = 3 + 4 (0 + 15)
  __syncthreads();

  // 6. top-r eigenvalues of T (d = td, off-diagonal e = te): count(x), the
  //    number of eigenvalues below x, is the number of negative pivots of the
  //    LDL^T factorisation of T - x I (Sturm sequence / Sylvester inertia).
  //    Eigenvalue j (descending) is bracketed by the Gershgorin interval and
  //    narrowed 65-fold per round: lane l counts at the l + 1-th of 64 interior
  //    points.  Wave w takes j = w and w + 4 together.
  const int R = a.rank;
  const float dl = td[lane];
  const float el = lane > 0 ? fabsf(te[lane - 1]) : 0.f, er = lane < 63 ? fabsf(te[lane]) : 0.f;
  const float glo = wmin(dl - el - er), ghi = wmax(dl + el + er);
  const float pivmin = 1e-30f * fmaxf(1.f, wmax(er * er));
  const float tnorm = fmaxf(fabsf(glo), fabsf(ghi));
  auto count_below1 = [&](float x0, int& c0) {
    float q0 = td[0] - x0;
    if (fabsf(q0) < pivmin) q0 = -pivmin;
    c0 = q0 < 0.f;
#pragma unroll 9
    for (int i = 1; i < 64; ++i) {
      const float e = te[i - 1];
      q0 = fmaf(-(e * e), __builtin_amdgcn_rcpf(q0), td[i] - x0);
      if (fabsf(q0) < pivmin) q0 = -pivmin;
      c0 += q0 < 0.f;
    }
  };
  // counts at two points (two independent recurrences side by side)
  auto count_below2 = [&](float x0, float x1, int& c0, int& c1) {
    float q0 = td[0] - x0, q1 = td[0] - x1;
    if (fabsf(q0) < pivmin) q0 = -pivmin;
    if (fabsf(q1) < pivmin) q1 = -pivmin;
    c0 = q0 < 0.f;
    c1 = q1 < 0.f;
#pragma unroll 9
    for (int i = 1; i < 64; ++i) {
      const float e = te[i - 1], d = td[i];
      q0 = fmaf(-(e * e), __builtin_amdgcn_rcpf(q0), d - x0);
      q1 = fmaf(-(e * e), __builtin_amdgcn_rcpf(q1), d - x1);
      if (fabsf(q0) < pivmin) q0 = -pivmin;
      if (fabsf(q1) < pivmin) q1 = -pivmin;
      c0 += q0 < 0.f;
      c1 += q1 < 0.f;
    }
  };
  if (wid < R) {
    const int j0 = wid, j1 = wid + 4;  // ranks from the top; j1 only when r > 4
    const int t0 = 63 - j0, t1 = 63 - j1;
    const float tol = 2e-7f * tnorm;
    float lo0 = glo - 1e-6f * tnorm - pivmin, hi0 = ghi + 1e-6f * tnorm + pivmin;  // count(lo) = 0, count(hi) = 64
    float lo1 = lo0, hi1 = hi0;
    for (int it = 0; it < 8; ++it) {
      const bool go0 = hi0 - lo0 > tol, go1 = j1 < R && hi1 - lo1 > tol;
      if (!go0 && !go1) break;
      const float f = (float)(lane + 1) * (1.f / 65.f);
      const float x0 = fmaf(hi0 - lo0, f, lo0), x1 = fmaf(hi1 - lo1, f, lo1);
      int c0, c1 = 0;
      if (j1 < R) count_below2(x0, x1, c0, c1);
      else count_below1(x0, c0);
      if (go0) {
        const uint64_t above = __ballot(c0 > t0);
        const int L = above ? __ffsll((unsigned long long)above) - 1 : 64;
        const float nhi = L < 64 ? rl(x0, L) : hi0;
        lo0 = L > 0 ? rl(x0, L - 1) : lo0;
        hi0 = nhi;
      }
      if (go1) {
        const uint64_t above = __ballot(c1 > t1);
        const int L = above ? __ffsll((unsigned long long)above) - 1 : 64;
        const float nhi = L < 64 ? rl(x1, L) : hi1;
        lo1 = L > 0 ? rl(x1, L - 1) : lo1;
        hi1 = nhi;
      }
    }
    if (lane == 0) {
      lam[j0] = 0.5f * (lo0 + hi0);
      if (j1 < R) lam[j1] = 0.5f * (lo1 + hi1);
    }
  }
  __syncthreads();

  // 7. eigenvectors of T by inverse iteration: lane j < r of wave 0 factors
  //    T - lambda_j I with partial pivoting (rows i, i + 1; the upper factor
  //    has two superdiagonals), then two solves from a fixed start vector;
  //    after each solve the wave orthonormalises the r vectors in order (lane i
  //    holds entry i).  Work rows (stride S): u0 (reciprocal pivots), u1, u2
  //    (upper factor), ml (multipliers), z (vectors), 8 rows each, in W.
  float* const U0 = W;
  float* const U1 = W + 8 * S;
  float* const U2 = W + 16 * S;
  float* const ML = W + 24 * S;
  float* const Z = W + 32 * S;
  const float tiny = 1e-7f * tnorm + 1e-30f;
  if (wid == 0) {
    uint64_t swp = 0ull;
    if (lane < R) {
      const float lmb = lam[lane];
      float* const u0 = U0 + lane * S;
      float* const u1 = U1 + lane * S;
      float* const u2 = U2 + lane * S;
      float* const ml = ML + lane * S;
      float* const z = Z + lane * S;
      float ad = td[0] - lmb, cu = te[0];
      // u0 keeps the reciprocal pivots
      for (int i = 0; i < 63; ++i) {
        const float b = te[i], an = td[i + 1] - lmb, cn = i < 62 ? te[i + 1] : 0.f;
        const bool keep = fabsf(ad) >= fabsf(b);  // pivot on the current row
        const float pv = keep ? (fabsf(ad) < tiny ? copysignf(tiny, ad) : ad) : b;
        const float ri = 1.f / pv;
        const float mt = (keep ? b : ad) * ri;
        u0[i] = ri;
        u1[i] = keep ? cu : an;
        u2[i] = keep ? 0.f : cn;
        ml[i] = mt;
        swp |= (uint64_t)(!keep) << i;
        const float nad = keep ? fmaf(-mt, cu, an) : fmaf(-mt, an, cu);
        cu = keep ? cn : -mt * cn;
        ad = nad;
      }
      u0[63] = 1.f / (fabsf(ad) < tiny ? copysignf(tiny, ad) : ad);
      for (int i = 0; i < 64; ++i) z[i] = 1.f + (float)((37 * i + 11 * lane) % 17) * (1.f / 34.f);
    }
    for (int it = 0; it < 2; ++it) {
      if (lane < R) {
        const float* const u0 = U0 + lane * S;
        const float* const u1 = U1 + lane * S;
        const float* const u2 = U2 + lane * S;
        const float* const ml = ML + lane * S;
        float* const z = Z + lane * S;
        // forward: the row swaps and multipliers, 9 rows a batch (loads first)
        float yi = z[0];
        for (int i0 = 0; i0 < 63; i0 += 9) {
          float zn[9], mm[9];
#pragma unroll
          for (int t = 0; t < 9; ++t) {
            zn[t] = z[i0 + t + 1];
            mm[t] = ml[i0 + t];
          }
#pragma unroll
          for (int t = 0; t < 9; ++t) {
            const bool sw = (swp >> (i0 + t)) & 1ull;
            const float piv = sw ? zn[t] : yi, oth = sw ? yi : zn[t];
            z[i0 + t] = piv;
            yi = fmaf(-mm[t], piv, oth);
          }
        }
        // back substitution, 9 rows a batch (rows 62 .. 0)
        float x1 = yi * u0[63], x2 = 0.f;
        z[63] = x1;
        for (int i0 = 62; i0 >= 0; i0 -= 9) {
          float zz[9], a0[9], a1[9], a2[9];
#pragma unroll
          for (int t = 0; t < 9; ++t) {
            zz[t] = z[i0 - t];
            a0[t] = u0[i0 - t];
            a1[t] = u1[i0 - t];
            a2[t] = u2[i0 - t];
          }
#pragma unroll
          for (int t = 0; t < 9; ++t) {
            const float x = (zz[t] - a1[t] * x1 - a2[t] * x2) * a0[t];
            z[i0 - t] = x;
            x2 = x1;
            x1 = x;
          }
        }
      }
      // orthonormalise in order (modified Gram-Schmidt; each vector first
      // scaled to max-abs 1 so the squares cannot overflow); lane = entry
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = j < R ? Z[j * S + lane] : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < R) {
          const float mx = wmax(fabsf(v[j]));
          v[j] *= mx > 0.f ? 1.f / mx : 0.f;
#pragma unroll
          for (int jj = 0; jj < j; ++jj) v[j] = fmaf(-wsum(v[j] * v[jj]), v[jj], v[j]);
          const float nn = wsum(v[j] * v[j]);
          v[j] *= nn > 0.f ? rsqrtf(nn) : 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < R) Z[j * S + lane] = v[j];
    }
  }
  __syncthreads();
  // back to G's basis: w = H_0 .. H_61 z (H_61 first); wave w takes vectors
  // w and w + 4, lane = entry
  {
    const int j0 = wid, j1 = wid + 4;
    float y0 = j0 < R ? Z[j0 * S + lane] : 0.f, y1 = j1 < R ? Z[j1 * S + lane] : 0.f;
    if (j0 < R) {
#pragma unroll 2
      for (int k = 61; k >= 0; --k) {
        const float beta = tb[k];
        const float u = G[k * S + lane];  // zero in rows 0 .. k (all zero when beta = 0)
        const float d0 = wsum(u * y0), d1 = wsum(u * y1);
        y0 = fmaf(-beta * d0, u, y0);
        y1 = fmaf(-beta * d1, u, y1);
      }
    }
    __syncthreads();  // every wave has read Z before any writes its result back
    if (j0 < R) Z[j0 * S + lane] = y0;
    if (j1 < R) Z[j1 * S + lane] = y1;
  }
  __syncthreads();
  // 8. factor rows sqrt(lambda_i) v_i = C^T w_i / sqrt(L)
  for (int o = tid; o < R * ED; o += 256) {
    const int i = o / ED, d = o % ED;
    float s = 0.f;
    for (int r = 0; r < kBlock; ++r) s = fmaf(Ct[d * kCtStride + r], Z[i * S + r], s);
    F[i * D + d] = s * 0.125f;  // 1/sqrt(64)
  }
  __syncthreads();
  // 9. sign: entry of largest magnitude (first on ties) made positive; one wave per row
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
