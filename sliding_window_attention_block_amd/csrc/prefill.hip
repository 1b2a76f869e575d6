// Masked prefill attention on MFMA (bf16 in, fp32 accumulate and output).
//
// Mask (query i, key j):  (i - wl <= j <= i + wr) [and j <= i if causal]
//                         or i is global or j is global.
//  * causal band of sliding-window attention (SWA glossary, 概要と動作原理:
//    itself and the w-1 previous tokens; the attention matrix is a band):
//    wl = w - 1, wr = 0, causal;
//  * local window plus bidirectional global tokens (local-global glossary,
//    local attention and global attention sections): wl = wr = 256, globals.
// Key tiles wholly outside the mask are skipped, as the SWA glossary's
// FlashAttention section describes; only tiles on the band edge take a
// per-element mask.  Softmax is the online (flash) form: a running max and
// normaliser per query row, rescaled as tiles arrive.
//
// Layout of the work (gfx950, v_mfma_f32_32x32x16_bf16):
//  * band workgroup: 128 query rows of one (b, h); wave w owns rows 32w..32w+31.
//    K/V tiles of 64 keys are staged in LDS (XOR-swizzled 16-byte chunks) with
//    a register prefetch of the next tile.  Per 32-key sub-tile a wave computes
//    S^T = K Q^T (A = K from LDS, B = Q^T in registers), so lane l holds 16 of
//    the 32 logits of query row l%32, then O^T += V^T P^T with V^T read by
//    ds_read_b64_tr_b16 and P^T taken straight from the logits' registers.
//  * in local+global mode, the global key columns that fall outside a
//    workgroup's band tiles are gathered into extra 64-key tiles, and separate
//    workgroups compute the global query rows against all keys (the 4 waves
//    split the keys, then merge their partial softmax states in LDS).  Band
//    workgroups do not store global rows.
//  * workgroup order: global-row workgroups first, then band workgroups with
//    the K/V head varying fastest (consecutive workgroups land on different
//    XCDs, so each XCD's L2 keeps one head's K/V), heaviest query tiles first.
#include "launch.hpp"

namespace bsattn {
namespace {

constexpr int BM = 128;  // query rows per band workgroup
constexpr int BN = 64;   // keys per LDS stage
// Rows that see fewer keys than this get the compensated (bf16 hi + lo) PV product.
constexpr int kCompKeys = 128;

template <int D>
struct Tile {
  static constexpr int RB = D * 2;       // bytes per row
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int RPL = 256 / RB;   // rows per 256-byte LDS line
  static constexpr int BYTES = BN * RB;  // one K or V stage
  // K tile: read by rows (32 rows x 2 chunks per instruction)
  static __device__ __forceinline__ uint32_t k_off(int r, int c) {
    const int f = (r / RPL) & (16 / RPL - 1);
    return (uint32_t)(r * RB + ((c ^ f) << 4));
  }
  // V tile: read transposed (8 rows x 4 chunks per instruction)
  static __device__ __forceinline__ uint32_t v_off(int r, int c) {
    const int f = 4 * ((r / RPL) & (4 / RPL - 1));
    return (uint32_t)(r * RB + ((c ^ f) << 4));
  }
};

struct Softmax {
  float m, l;
};

// One 32-key sub-tile for a wave: logits, mask, online softmax update, PV.
// `kt` / `vt` are the LDS K/V tiles, `krow0` the sub-tile's first row in them.
// mask_fn(e) returns whether element e (key 8(e/4) + 4(l/32) + e%4) is allowed.
// `comp` (wave-uniform) adds a second PV product with the bf16 residual of P, so
// rows that see only a few keys are not limited by the 2^-9 rounding of P.
template <int D, typename MaskFn>
__device__ __forceinline__ void subtile(const uint8_t* kt, const uint8_t* vt, int krow0,
                                        const u32x4* qop, f32x16* oacc, Softmax& st, float sl2,
                                        bool masked, bool comp, MaskFn mask_fn) {
  using T = Tile<D>;
  const int lane = threadIdx.x & 63;
  const int r32 = lane & 31, h2 = lane >> 5;
  f32x16 s;
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const u32x4 kop = *reinterpret_cast<const u32x4*>(kt + T::k_off(krow0 + r32, 2 * c + h2));
    s = mfma32x32x16(as_bf16x8(kop), as_bf16x8(qop[c]), s);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float v = s[e] * sl2;
    if (masked && !mask_fn(e)) v = -INFINITY;
    s[e] = v;
    mx = fmaxf(mx, v);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  // No branch on m_new: rows with nothing allowed yet keep m = -inf and l = 0 (the
  // MFMAs below must run with every lane active).
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = exp2f(st.m - m_use);
  u32x4 pop[2], plo[2];
  float psum = 0.f;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = exp2f(s[8 * kc + 2 * i] - m_use), p1 = exp2f(s[8 * kc + 2 * i + 1] - m_use);
      const uint32_t pk = pack_bf16x2(p0, p1);
      pop[kc][i] = pk;
      if (comp) {
        plo[kc][i] = pack_bf16x2(p0 - bf16lo(pk), p1 - bf16hi(pk));
        psum += p0 + p1;
      } else {
        psum += bf16lo(pk) + bf16hi(pk);  // normaliser of the rounded weights the MFMA sees
      }
    }
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;
  const int q16 = lane >> 4, a16 = lane & 15;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int row = krow0 + 16 * kc + 4 * h2 + (a16 >> 2);
      const int col = 32 * dt + 16 * (q16 & 1) + 4 * (a16 & 3);  // element
      const u32x2 lo = lds_read_tr16(vt, T::v_off(row, col >> 3) + ((col & 7) << 1));
      const u32x2 hi = lds_read_tr16(vt, T::v_off(row + 8, col >> 3) + ((col & 7) << 1));
      const u32x4 vop = u32x4{lo[0], lo[1], hi[0], hi[1]};
      oacc[dt] = mfma32x32x16(as_bf16x8(vop), as_bf16x8(pop[kc]), oacc[dt]);
      if (comp) oacc[dt] = mfma32x32x16(as_bf16x8(vop), as_bf16x8(plo[kc]), oacc[dt]);
    }
  }
}

template <int D, bool LG>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  using T = Tile<D>;
  constexpr int LDS_BYTES = 2 * T::BYTES > 32 * D * 4 + 1024 ? 2 * T::BYTES : 32 * D * 4 + 1024;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  __shared__ int gcols[256];
  __shared__ int s_ngcols;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r32 = lane & 31, h2 = lane >> 5;
  const int N = a.seq_len;
  const int Hq = a.n_q_heads, Hkv = a.n_kv_heads, G = Hq / Hkv;
  const float sl2 = a.scale * kLog2e;
  const int n_rt = (a.n_global + 31) / 32;
  const int n_grow = LG ? a.batch * Hq * n_rt : 0;

  if (LG && (int)blockIdx.x < n_grow) {
    // ---------------- global query rows against every key
    const int rt = blockIdx.x % n_rt;
    const int bhq = blockIdx.x / n_rt;
    const int b = bhq / Hq, h = bhq % Hq, g = h / G;
    const int slot = rt * 32 + r32;
    const bool row_ok = slot < a.n_global;
    const int row = row_ok ? a.gpos[slot] : a.gpos[0];
    const uint16_t* Qp = reinterpret_cast<const uint16_t*>(a.Q) + ((size_t)(b * Hq + h) * N + row) * D;
    const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.K) + (size_t)(b * Hkv + g) * a.kv_capacity * D;
    const uint16_t* Vb = reinterpret_cast<const uint16_t*>(a.V) + (size_t)(b * Hkv + g) * a.kv_capacity * D;
    u32x4 qop[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qop[c] = *reinterpret_cast<const u32x4*>(Qp + 16 * c + 8 * h2);
    f32x16 oacc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[t][e] = 0.f;
    Softmax st{-INFINITY, 0.f};
    uint8_t* vt = smem + wid * (32 * T::RB);
    const int n_sub = (N + 31) / 32;
    const bool comp = N < kCompKeys;
    for (int kt = wid; kt < n_sub; kt += 4) {
      const int j0 = kt * 32;
      // K rows straight into A operands, V into the wave's LDS tile
      u32x4 kop[D / 16];
      {
        const int key = min(j0 + r32, N - 1);
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
          kop[c] = *reinterpret_cast<const u32x4*>(Kb + (size_t)key * D + 16 * c + 8 * h2);
      }
      constexpr int VPL = 32 * T::CPR / 64;  // V chunks per lane
      u32x4 vreg[VPL];
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        const int c = lane + 64 * k;
        const int key = min(j0 + c / T::CPR, N - 1);
        vreg[k] = *reinterpret_cast<const u32x4*>(Vb + (size_t)key * D + (c % T::CPR) * 8);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        const int c = lane + 64 * k;
        *reinterpret_cast<u32x4*>(vt + T::v_off(c / T::CPR, c % T::CPR)) = vreg[k];
      }
      f32x16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) s = mfma32x32x16(as_bf16x8(kop[c]), as_bf16x8(qop[c]), s);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // online softmax over this sub-tile (keys past N masked)
      float mx = -INFINITY;
      const bool tail = j0 + 32 > N;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = s[e] * sl2;
        if (tail && j0 + 8 * (e >> 2) + 4 * h2 + (e & 3) >= N) v = -INFINITY;
        s[e] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(st.m, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(st.m - m_use);
      u32x4 pop[2], plo[2];
      float psum = 0.f;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = exp2f(s[8 * kc + 2 * i] - m_use), p1 = exp2f(s[8 * kc + 2 * i + 1] - m_use);
          const uint32_t pk = pack_bf16x2(p0, p1);
          pop[kc][i] = pk;
          if (comp) {
            plo[kc][i] = pack_bf16x2(p0 - bf16lo(pk), p1 - bf16hi(pk));
            psum += p0 + p1;
          } else {
            psum += bf16lo(pk) + bf16hi(pk);
          }
        }
      st.l = st.l * alpha + psum;
      st.m = m_new;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;
      const int q16 = lane >> 4, a16 = lane & 15;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const int vr = 16 * kc + 4 * h2 + (a16 >> 2);
          const int col = 32 * dt + 16 * (q16 & 1) + 4 * (a16 & 3);
          const u32x2 lo = lds_read_tr16(vt, T::v_off(vr, col >> 3) + ((col & 7) << 1));
          const u32x2 hi = lds_read_tr16(vt, T::v_off(vr + 8, col >> 3) + ((col & 7) << 1));
          const u32x4 vop = u32x4{lo[0], lo[1], hi[0], hi[1]};
          oacc[dt] = mfma32x32x16(as_bf16x8(vop), as_bf16x8(pop[kc]), oacc[dt]);
          if (comp) oacc[dt] = mfma32x32x16(as_bf16x8(vop), as_bf16x8(plo[kc]), oacc[dt]);
        }
    }
    // merge the 4 waves' states
    st.l += __shfl_xor(st.l, 32);
    __syncthreads();
    float* ml = reinterpret_cast<float*>(smem);          // [4][32][2]
    float* obuf = reinterpret_cast<float*>(smem + 1024);  // [32][D]
    if (lane < 32) { ml[(wid * 32 + r32) * 2] = st.m; ml[(wid * 32 + r32) * 2 + 1] = st.l; }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[(w * 32 + r32) * 2]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = ml[(w * 32 + r32) * 2];
      if (mw != -INFINITY) L += exp2f(mw - M) * ml[(w * 32 + r32) * 2 + 1];
    }
    const float sc = (st.m == -INFINITY) ? 0.f : exp2f(st.m - M);
    for (int w = 0; w < 4; ++w) {
      if (wid == w) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float* dst = obuf + r32 * D + 32 * dt + 8 * j + 4 * h2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float v = oacc[dt][4 * j + i] * sc;
              dst[i] = (w == 0) ? v : dst[i] + v;
            }
          }
      }
      __syncthreads();
    }
    // write the rows: thread t -> row t / (256/32)... 32 rows x D floats
    for (int idx = tid; idx < 32 * D; idx += 256) {
      const int rr = idx / D, d = idx % D;
      const int sl = rt * 32 + rr;
      if (sl >= a.n_global) continue;
      float Lr = 0.f, Mr = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) Mr = fmaxf(Mr, ml[(w * 32 + rr) * 2]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = ml[(w * 32 + rr) * 2];
        if (mw != -INFINITY) Lr += exp2f(mw - Mr) * ml[(w * 32 + rr) * 2 + 1];
      }
      const int grow = a.gpos[sl];
      a.O[((size_t)(b * Hq + h) * N + grow) * D + d] = obuf[rr * D + d] / Lr;
      if (d == 0 && a.lse != nullptr) a.lse[(size_t)(b * Hq + h) * N + grow] = (Mr + log2f(Lr)) * kLn2;
    }
    (void)L;
    return;
  }

  // ---------------- band workgroup
  const int w = blockIdx.x - n_grow;
  const int BHkv = a.batch * Hkv;
  const int kvlin = w % BHkv;
  const int rest = w / BHkv;
  const int hsub = rest % G;
  const int n_qt = (N + BM - 1) / BM;
  const int qt = n_qt - 1 - rest / G;
  const int b = kvlin / Hkv, g = kvlin % Hkv, h = g * G + hsub;
  const int i0 = qt * BM;
  const int wl = a.window_left;
  const int wr = a.causal ? 0 : a.window_right;
  const int klo = wl < 0 ? 0 : max(0, i0 - wl);
  const int khi = wr < 0 ? N : min(N, i0 + BM + wr);
  const int t_lo = klo / BN, t_hi = (khi + BN - 1) / BN;
  const int n_band = max(0, t_hi - t_lo);

  if (LG) {
    if (tid == 0) {
      int n = 0;
      for (int i = 0; i < a.n_global; ++i) {
        const int p = a.gpos[i];
        if (p < t_lo * BN || p >= t_hi * BN) gcols[n++] = p;
      }
      s_ngcols = n;
    }
    __syncthreads();
  }
  const int ngc = LG ? s_ngcols : 0;
  const int n_stage = n_band + (ngc + BN - 1) / BN;

  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.K) + (size_t)(b * Hkv + g) * a.kv_capacity * D;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(a.V) + (size_t)(b * Hkv + g) * a.kv_capacity * D;
  const int r0 = i0 + 32 * wid;
  const int myrow = r0 + r32;
  u32x4 qop[D / 16];
  {
    const uint16_t* Qp = reinterpret_cast<const uint16_t*>(a.Q) + ((size_t)(b * Hq + h) * N + min(myrow, N - 1)) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qop[c] = *reinterpret_cast<const u32x4*>(Qp + 16 * c + 8 * h2);
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[t][e] = 0.f;
  Softmax st{-INFINITY, 0.f};

  // Keys seen by the wave's rows (globals only add keys): the count is piecewise
  // linear in the row, so its minimum over the 32 rows sits at an end row.
  auto band_keys = [&](int i) {
    const int lo = wl < 0 ? 0 : max(0, i - wl);
    const int hi = wr < 0 ? N - 1 : min(N - 1, i + wr);
    return hi - lo + 1;
  };
  const bool comp = __builtin_amdgcn_readfirstlane(
      min(band_keys(min(r0, N - 1)), band_keys(min(r0 + 31, N - 1))) < kCompKeys);

  uint8_t* kt = smem;
  uint8_t* vt = smem + T::BYTES;
  constexpr int PT = BN * T::CPR / 256;  // chunks per thread per tile
  u32x4 kreg[PT], vreg[PT];
  auto load_stage = [&](int stg) {
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      const int c = tid + 256 * k;
      const int rr = c / T::CPR, ch = c % T::CPR;
      int pos;
      bool ok;
      if (stg < n_band) {
        pos = (t_lo + stg) * BN + rr;
        ok = pos < N;
      } else {
        const int slot = (stg - n_band) * BN + rr;
        ok = slot < ngc;
        pos = ok ? gcols[slot] : 0;
      }
      if (ok) {
        kreg[k] = *reinterpret_cast<const u32x4*>(Kb + (size_t)pos * D + ch * 8);
        vreg[k] = *reinterpret_cast<const u32x4*>(Vb + (size_t)pos * D + ch * 8);
      } else {
        kreg[k] = u32x4{0u, 0u, 0u, 0u};
        vreg[k] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  if (n_stage > 0) load_stage(0);
  for (int stg = 0; stg < n_stage; ++stg) {
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      const int c = tid + 256 * k;
      const int rr = c / T::CPR, ch = c % T::CPR;
      *reinterpret_cast<u32x4*>(kt + T::k_off(rr, ch)) = kreg[k];
      *reinterpret_cast<u32x4*>(vt + T::v_off(rr, ch)) = vreg[k];
    }
    __syncthreads();
    if (stg + 1 < n_stage) load_stage(stg + 1);
    const bool band_stage = stg < n_band;
    uint64_t gbits = 0ull;
    if (LG && band_stage) {
      const int base = (t_lo + stg) * BN;
      for (int i = lower_bound_i32(a.gpos, a.n_global, base); i < a.n_global && a.gpos[i] < base + BN; ++i)
        gbits |= 1ull << (a.gpos[i] - base);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      if (band_stage) {
        const int j0 = (t_lo + stg) * BN + 32 * sub;
        if (j0 >= N) continue;
        const uint32_t gsub = (uint32_t)(gbits >> (32 * sub));
        const bool any_lo = wl < 0 || j0 + 31 >= r0 - wl;
        const bool any_hi = wr < 0 || j0 <= r0 + 31 + wr;
        if (!(any_lo && any_hi) && gsub == 0u) continue;  // empty for this wave
        const bool all_lo = wl < 0 || j0 >= r0 + 31 - wl;
        const bool all_hi = wr < 0 || j0 + 31 <= r0 + wr;
        const bool full = all_lo && all_hi && j0 + 31 < N;
        subtile<D>(kt, vt, 32 * sub, qop, oacc, st, sl2, !full, comp, [&](int e) {
          const int jr = 8 * (e >> 2) + 4 * h2 + (e & 3);
          const int j = j0 + jr;
          const bool in_band = (wl < 0 || j >= myrow - wl) && (wr < 0 || j <= myrow + wr);
          return j < N && (in_band || ((gsub >> jr) & 1u));
        });
      } else {
        const int s0 = (stg - n_band) * BN + 32 * sub;
        if (s0 >= ngc) continue;
        const bool full = s0 + 31 < ngc;
        subtile<D>(kt, vt, 32 * sub, qop, oacc, st, sl2, !full, comp, [&](int e) {
          return s0 + 8 * (e >> 2) + 4 * h2 + (e & 3) < ngc;
        });
      }
    }
  }
  // write rows (global rows are written by their own workgroups)
  st.l += __shfl_xor(st.l, 32);
  bool store = myrow < N;
  if (LG && store) {
    const int i = lower_bound_i32(a.gpos, a.n_global, myrow);
    store = !(i < a.n_global && a.gpos[i] == myrow);
  }
  if (store) {
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    float* orow = a.O + ((size_t)(b * Hq + h) * N + myrow) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = oacc[dt][4 * j + i] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * j + 4 * h2) = v;
      }
    if (a.lse != nullptr && h2 == 0)
      a.lse[(size_t)(b * Hq + h) * N + myrow] = st.l > 0.f ? (st.m + log2f(st.l)) * kLn2 : -INFINITY;
  }
}

template <int D, bool LG>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  const int n_qt = (a.seq_len + BM - 1) / BM;
  const int n_rt = (a.n_global + 31) / 32;
  const int n_grow = LG ? a.batch * a.n_q_heads * n_rt : 0;
  const int n_wg = n_grow + n_qt * a.batch * a.n_q_heads;
  hipLaunchKernelGGL((prefill_kernel<D, LG>), dim3(n_wg), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const bool lg = a.n_global > 0;
  if (a.head_dim == 64) return lg ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
  return lg ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
}

}  // namespace bsattn
