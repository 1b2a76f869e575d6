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
// Work layout on gfx950 (v_mfma_f32_32x32x16_bf16):
//  * band workgroup: 128 query rows of one (b, h); wave w owns rows 32w..32w+31.
//    K/V tiles of 64 keys are copied HBM -> LDS with global_load_lds_dwordx4
//    into double-buffered, XOR-swizzled tiles (one barrier per tile).  A wave
//    computes S^T = K Q^T for both 32-key halves of the tile (two independent
//    MFMA chains; A = K from LDS, B = Q^T in registers), so lane l holds 32
//    logits of query row l%32, then O^T += V^T P^T with V^T read by
//    ds_read_b64_tr_b16 and P^T taken straight from the logits' registers.
//    Softmax per tile: one FMA folds the scale into exp2's argument, the row
//    max is only moved (and the accumulator rescaled, wave-uniformly) when it
//    grows by more than 2^8, and P is rounded to bf16 by v_cvt_pk_bf16_f32.
//    Rows that see fewer than 256 keys add the bf16 residual of P in a second
//    product; other rows normalise by the sum of the rounded weights.
//  * local+global: the global key columns outside a workgroup's band tiles are
//    gathered into extra tiles.  The global query rows (every key) are split
//    by key range over many waves (first in the grid); each writes a partial
//    softmax state to the workspace, and a merge kernel combines them.  Band
//    workgroups do not store global rows.
//  * band workgroup order: K/V head varying fastest (consecutive workgroups
//    land on different XCDs, so each XCD's L2 keeps one head's K/V), heaviest
//    query tiles first.
#include <type_traits>

#include "launch.hpp"

namespace bsattn {
namespace {

constexpr int BM = 128;        // query rows per band workgroup
static_assert(BM == kSparseTile, "a block-sparse selection tile is one band workgroup's rows");
constexpr int BN = 64;         // keys per LDS stage
constexpr int kCompKeys = 256; // rows seeing fewer keys take the compensated PV product
constexpr float kHeadroom = 8.f;  // log2 units a row max may grow before the rescale
constexpr bf16x2 kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

template <int D>
struct Tile {
  static constexpr int RB = D * 2;       // bytes per row
  static constexpr int RPL = 256 / RB;   // rows per 256-byte LDS line
  static constexpr int BYTES = BN * RB;  // one K or V stage
  // K tile: read by rows (32 rows x 2 chunks per instruction)
  static __device__ __forceinline__ int k_swz(int r) { return (r / RPL) & (16 / RPL - 1); }
  // V tile: read transposed (8 rows x 4 chunks per instruction)
  static __device__ __forceinline__ int v_swz(int r) { return 4 * ((r / RPL) & (4 / RPL - 1)); }
  static __device__ __forceinline__ uint32_t k_off(int r, int c) { return (uint32_t)(r * RB + ((c ^ k_swz(r)) << 4)); }
  static __device__ __forceinline__ uint32_t v_off(int r, int c) { return (uint32_t)(r * RB + ((c ^ v_swz(r)) << 4)); }
};

struct RowState {
  float m;  // running max in log2 units (may lag the true max by up to kHeadroom)
  float l;  // normaliser relative to m (partial per lane; lanes l, l^32 sum)
};


// Copy rows [0, 64) of a K/V stage into LDS tiles with 1 KB DMA instructions.
// `row_pos(r)` is the token position of tile row r (already clamped into range).
// Wave `wid` of `nw` issues its share of the chunks.
// kt (vt) may be null: that tile is not copied.
template <int D, typename RowPos>
__device__ __forceinline__ void dma_stage(const uint16_t* Kb, const uint16_t* Vb, uint8_t* kt, uint8_t* vt,
                                          int wid, int nw, RowPos row_pos, size_t pitch = D) {
  using T = Tile<D>;
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int NCH = T::BYTES / 1024;
  const int lane = threadIdx.x & 63;
  for (int k = wid; k < NCH; k += nw) {
    const int off = 1024 * k + 16 * lane;
    const int r = off / T::RB, pc = (off % T::RB) >> 4;
    const size_t pos = (size_t)row_pos(r);
    if (kt != nullptr)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(Kb + pos * pitch + (pc ^ T::k_swz(r)) * 8),
                                       (lds_void*)(kt + 1024 * k), 16, 0, 0);
    if (vt != nullptr)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(Vb + pos * pitch + (pc ^ T::v_swz(r)) * 8),
                                       (lds_void*)(vt + 1024 * k), 16, 0, 0);
  }
}

// Per-lane byte offsets, inside a 64-row tile, of the 1 KB DMA chunks a wave
// issues for a contiguous stage (chunks wid, wid + 4, ...): with them a stage's
// copies take one scalar base and no per-lane address arithmetic.
template <int D>
struct DmaLane {
  static constexpr int NW = Tile<D>::BYTES / 1024 / 4;  // chunks per wave per tile
  uint32_t k[NW], v[NW];
  // pitch: bytes between consecutive rows of the copied view (the row size, or
  // a multiple of it for a dilated window's residue class)
  __device__ __forceinline__ void init(int wid, uint32_t pitch = Tile<D>::RB) {
    using T = Tile<D>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int off = 1024 * (wid + 4 * i) + 16 * lane;
      const int r = off / T::RB, pc = (off % T::RB) >> 4;
      k[i] = (uint32_t)(r * pitch + ((pc ^ T::k_swz(r)) << 4));
      v[i] = (uint32_t)(r * pitch + ((pc ^ T::v_swz(r)) << 4));
    }
  }
  // copy rows [row0, row0 + 64) of K and V (all < the sequence length); a null
  // destination tile is not copied
  __device__ __forceinline__ void issue(const uint8_t* Kb, const uint8_t* Vb, int row0, uint8_t* kt, uint8_t* vt,
                                        int wid, size_t pitch = Tile<D>::RB) const {
    typedef __attribute__((address_space(3))) void lds_void;
    const uint8_t* ks = Kb + (size_t)row0 * pitch;
    const uint8_t* vs = Vb + (size_t)row0 * pitch;
    if (kt != nullptr) {
#pragma unroll
      for (int i = 0; i < NW; ++i)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(ks + k[i]), (lds_void*)(kt + 1024 * (wid + 4 * i)),
                                         16, 0, 0);
    }
    if (vt != nullptr) {
#pragma unroll
      for (int i = 0; i < NW; ++i)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(vs + v[i]), (lds_void*)(vt + 1024 * (wid + 4 * i)),
                                         16, 0, 0);
    }
  }
};

// The two 32-lane halves of x, each broadcast to the whole wave, by one
// v_permlane32_swap of two copies of x: a = {x_lo, x_lo}, b = {x_hi, x_hi}.
// Written in asm with both registers read-write: the compiler's builtin for
// this instruction returns its first result twice.  The s_nops cover the
// VALU-write / permlane-read hazards around it.
__device__ __forceinline__ void halves(float x, float& a, float& b) {
  uint32_t u = __builtin_bit_cast(uint32_t, x), v = u;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(u), "+v"(v));
  a = __builtin_bit_cast(float, u);
  b = __builtin_bit_cast(float, v);
}
// Maximum / sum of a value over the two 32-lane halves of the wave.
__device__ __forceinline__ float max_halves(float x) {
  float a, b;
  halves(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_halves(float x) {
  float a, b;
  halves(x, a, b);
  return a + b;
}

// Bits p of [lo, hi] within a 32-bit word (empty when lo > hi).
__device__ __forceinline__ uint32_t range_bits32(int lo, int hi) {
  lo = max(lo, 0);
  hi = max(min(hi, 31), -1);
  const uint32_t upto = hi >= 31 ? ~0u : ((1u << (hi + 1)) - 1u);  // bits <= hi (0 when hi < 0)
  const uint32_t below = (1u << min(lo, 31)) - 1u;                  // bits < lo
  return lo > hi ? 0u : (upto & ~below);
}

// One stage of NH 32-key halves held in LDS for this wave's 32 query rows.
// Bit u of `masked` (wave-uniform) marks a half on a mask edge; only for such a
// half is am(u) evaluated: this lane's allowed keys of half u as bits
// p = key - 32u (the lane's row is l % 32; its elements e hold keys
// 8(e/4) + 4(l/32) + e%4).  COMP adds the product with the bf16 residual of P.
// The MFMAs run unconditionally (a half with nothing allowed only has its
// weights forced to 0), so no accumulator ever sits under a branch, and the mask
// is two ALU ops per element: a signed one-bit field extract (0 or all ones)
// selects, bitwise, between the logit and -inf.
template <int D, int NH, bool COMP, typename AllowedBits>
__device__ __forceinline__ void stage(const uint8_t* kt, const uint8_t* vt, const u32x4* qop,
                                      f32x16* oacc, RowState& st, float sl2, AllowedBits am,
                                      uint32_t masked) {
  using T = Tile<D>;
  const int lane = threadIdx.x & 63;
  const int r32 = lane & 31, h2 = lane >> 5;
  f32x16 s[NH];
#pragma unroll
  for (int u = 0; u < NH; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[u][e] = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
#pragma unroll
    for (int u = 0; u < NH; ++u) {
      const u32x4 k = *reinterpret_cast<const u32x4*>(kt + T::k_off(32 * u + r32, 2 * c + h2));
      s[u] = mfma32x32x16(as_bf16x8(k), as_bf16x8(qop[c]), s[u]);
    }
  // Each 32-key half is its own online-softmax step, in program order
  // QK0 QK1 | softmax0 PV0 | softmax1 PV1: the VALU work of a half runs while
  // the MFMAs issued before it (QK1, then PV0) are still in the matrix pipe.
  const int q16 = lane >> 4, a16 = lane & 15;
#pragma unroll
  for (int u = 0; u < NH; ++u) {
    if ((masked >> u) & 1u) {  // wave-uniform: only halves on a mask edge
      const uint32_t m = am(u) >> (4 * h2);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int p = 8 * (e >> 2) + (e & 3);
        const uint32_t keep = (uint32_t)((int)(m << (31 - p)) >> 31);
        // copied out first: a bit-cast of a vector-element lvalue reads element 0
        const float v = s[u][e];
        const uint32_t x = __builtin_bit_cast(uint32_t, v);
        s[u][e] = __builtin_bit_cast(float, (x & keep) | (0xff800000u & ~keep));
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[u][e]);
    mx = max_halves(mx);
    const float m_cand = mx * sl2;
    const bool need = m_cand > st.m + kHeadroom;
    if (__ballot(need)) {
      const float m_new = need ? m_cand : st.m;
      const float alpha = need ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
      st.l *= alpha;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;
      st.m = m_new;
    }
    const float nm = (st.m == -INFINITY) ? 0.f : -st.m;
    u32x4 pop[2], plo[2];
    float psum = 0.f;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[u][8 * kc + 2 * i], sl2, nm));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[u][8 * kc + 2 * i + 1], sl2, nm));
        const uint32_t pk = cvt_pk_bf16(p0, p1);
        pop[kc][i] = pk;
        if constexpr (COMP) {
          plo[kc][i] = cvt_pk_bf16(p0 - bf16lo(pk), p1 - bf16hi(pk));
          psum += p0 + p1;
        } else {
          // normaliser of the rounded weights the MFMA sees (O stays a convex
          // combination of V rows however peaked the row's softmax is): one
          // v_dot2_f32_bf16 with (1, 1) adds both rounded weights
          psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), kOnesBf16x2, psum, false);
        }
      }
    st.l += psum;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int row = 32 * u + 16 * kc + 4 * h2 + (a16 >> 2);
        const int col = 32 * dt + 16 * (q16 & 1) + 4 * (a16 & 3);  // element
        const u32x2 lo = lds_read_tr16(vt, T::v_off(row, col >> 3) + ((col & 7) << 1));
        const u32x2 hi = lds_read_tr16(vt, T::v_off(row + 8, col >> 3) + ((col & 7) << 1));
        const u32x4 vop = u32x4{lo[0], lo[1], hi[0], hi[1]};
        oacc[dt] = mfma32x32x16(as_bf16x8(vop), as_bf16x8(pop[kc]), oacc[dt]);
        if constexpr (COMP) oacc[dt] = mfma32x32x16(as_bf16x8(vop), as_bf16x8(plo[kc]), oacc[dt]);
      }
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined band stages.  A wave's work per 64-key stage j is: S_j =
// K_j Q^T (16 MFMAs at d = 128), the row max of S_j, P_j = exp2(S_j - m) with
// its row sums (VALU), and O += V_j P_j (16 MFMAs).  Run in that order each
// stage is a chain the MFMA and VALU pipes take in turns.  Here stage j's
// exponentials are issued between the MFMAs of S_{j+1} = K_{j+1} Q^T (region
// A), and S_{j+1}'s row max between the MFMAs of O += V_j P_j (region B), so
// one wave keeps both pipes busy: each region is straight-line code and the
// instruction order inside it is fixed with sched_group_barrier.  A stage on a
// mask edge applies its mask between the two regions (a wave-uniform branch);
// the rescale of O when a row max grows past the headroom follows region B.

#define BSATTN_SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100;

// Region A.  QK: sn = K Q^T from the K tile kt (its first NH 32-key halves:
// both, or the first alone for a gathered-column stage whose second half is
// padding).  Always:
// P of the stage held in s (logits, log2 domain after the fold of sl2 into the
// exponent's argument): bf16 hi parts in pop (lo parts in plo when COMP) and
// the row sums of what the P.V product will see, added to psum.
template <int D, bool COMP, bool QK, bool EXP, int NH = 2>
__device__ __forceinline__ void region_a(const uint8_t* kt, const u32x4* qop, f32x16 (&sn)[2], const f32x16 (&s)[2],
                                         float sl2, float nm, u32x4 (&pop)[2][2], u32x4 (&plo)[2][2], float& psum) {
  using T = Tile<D>;
  const int lane = threadIdx.x & 63;
  const int r32 = lane & 31, h2 = lane >> 5;
  if constexpr (QK) {
#pragma unroll
    for (int u = 0; u < NH; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) sn[u][e] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int u = 0; u < NH; ++u) {
        const u32x4 k = *reinterpret_cast<const u32x4*>(kt + T::k_off(32 * u + r32, 2 * c + h2));
        sn[u] = mfma32x32x16(as_bf16x8(k), as_bf16x8(qop[c]), sn[u]);
      }
  }
  if constexpr (EXP) {
#pragma unroll
  for (int u = 0; u < NH; ++u)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[u][8 * kc + 2 * i], sl2, nm));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[u][8 * kc + 2 * i + 1], sl2, nm));
        const uint32_t pk = cvt_pk_bf16(p0, p1);
        pop[u][kc][i] = pk;
        if constexpr (COMP) {
          plo[u][kc][i] = cvt_pk_bf16(p0 - bf16lo(pk), p1 - bf16hi(pk));
          psum += p0 + p1;
        } else {
          psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), kOnesBf16x2, psum, false);
        }
      }
  }
  if constexpr (QK && EXP) {
    // 16 (d = 128) or 8 (d = 64) MFMAs, each with the next K read and its share
    // of the 96 (non-COMP) or 176 (COMP) VALU instructions of the exponentials
    constexpr int NM = D / 8, NV = COMP ? 176 : 96, PER = (NV + NM - 1) / NM;
    BSATTN_SGB(kSgDsRead, 2);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      BSATTN_SGB(kSgMfma, 1);
      if (i + 2 < NM) BSATTN_SGB(kSgDsRead, 1);
      BSATTN_SGB(kSgValu, PER);
    }
  }
  if constexpr (EXP) {
    // the weights are needed here: otherwise the compiler sinks their
    // computation below the next stage's (branchy) mask, out of this region
#pragma unroll
    for (int u = 0; u < NH; ++u)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        asm volatile("" ::"v"(pop[u][kc]));
        if constexpr (COMP) asm volatile("" ::"v"(plo[u][kc]));
      }
    asm volatile("" ::"v"(psum));
  }
}

// Region B.  O += V P from the V tile vt (P in pop, plo); when MX, the per-lane
// max of sn over both halves (the caller combines the wave's two lane halves).
template <int D, bool COMP, bool PV, bool MX, int NH = 2>
__device__ __forceinline__ float region_b(const uint8_t* vt, const u32x4 (&pop)[2][2], const u32x4 (&plo)[2][2],
                                          f32x16* oacc, const f32x16 (&sn)[2]) {
  using T = Tile<D>;
  const int lane = threadIdx.x & 63;
  const int h2 = lane >> 5, q16 = lane >> 4, a16 = lane & 15;
  if constexpr (PV) {
#pragma unroll
  for (int u = 0; u < NH; ++u)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int row = 32 * u + 16 * kc + 4 * h2 + (a16 >> 2);
        const int col = 32 * dt + 16 * (q16 & 1) + 4 * (a16 & 3);  // element
        const u32x2 lo = lds_read_tr16(vt, T::v_off(row, col >> 3) + ((col & 7) << 1));
        const u32x2 hi = lds_read_tr16(vt, T::v_off(row + 8, col >> 3) + ((col & 7) << 1));
        const u32x4 vop = u32x4{lo[0], lo[1], hi[0], hi[1]};
        oacc[dt] = mfma32x32x16(as_bf16x8(vop), as_bf16x8(pop[u][kc]), oacc[dt]);
        if constexpr (COMP) oacc[dt] = mfma32x32x16(as_bf16x8(vop), as_bf16x8(plo[u][kc]), oacc[dt]);
      }
  }
  float mx = -INFINITY;
  if constexpr (MX) {
#pragma unroll
    for (int u = 0; u < NH; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sn[u][e]);
  }
  if constexpr (PV && MX) {
    constexpr int NM = (D / 32) * 4 * (COMP ? 2 : 1), NR = (D / 32) * 8;
    constexpr int RPER = NR / NM, VPER = (16 + NM - 1) / NM;
    BSATTN_SGB(kSgDsRead, 4);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      BSATTN_SGB(kSgMfma, 1);
      BSATTN_SGB(kSgDsRead, RPER);
      BSATTN_SGB(kSgValu, VPER);
    }
  }
  return mx;
}

// SP: block-sparse causal prefill [NSA block selection; COBS 2.1]: ahead of its
// causal band, a workgroup runs one 64-key stage per block its query tile
// selected and per sink block; a key of such a stage is allowed for row i only
// before i's window (keys in the window come from the band), and only below
// n_sink for a sink block the tile did not select, so no key counts twice.
//
// DIL: dilated causal or bidirectional window [SWA 拡張手法, dilated SWA]: the
// launch takes one residue class r of the rows and keys (physical position
// r + s x for logical position x), where the dilated mask is the plain band
// of the logical positions, so every stage is the band kernel's own (no
// per-element stride test); only the row addressing uses the pitch s d.
// Occupancy: two workgroups (eight waves) per CU, except local+global at
// d = 64, which runs its stages one at a time (no software pipeline, one tile
// of logits live) in at most 128 registers, four workgroups per CU: at
// d = 64 the softmax outweighs the MFMAs, and four waves per SIMD hide each
// stage's dependent chain better than one wave's pipeline with three.
template <int D, bool LG, bool SP = false, bool DIL = false>
__global__ __launch_bounds__(256, (LG && D == 64) ? 4 : 2) void prefill_kernel(PrefillArgs a) {
  using T = Tile<D>;
  constexpr int LDS_BYTES = 4 * T::BYTES;  // K and V, double buffered
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  __shared__ int gcols[256];
  __shared__ int s_ngcols;
  __shared__ int xblk[kSparseMaxTopK + kSparseMaxSink / 64];  // 2 block + (selected)
  __shared__ int s_nx;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform (scalar registers): every tile flag derived from it is too, so
  // the MFMA chains below run under uniform branches, never under exec masks
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h2 = lane >> 5;
  const int N = a.seq_len;
  const int Hq = a.n_q_heads, Hkv = a.n_kv_heads, G = Hq / Hkv;
  const float sl2 = a.scale * kLog2e;
  const int n_gwg = LG ? a.n_global_wg : 0;

  if (LG && (int)blockIdx.x < n_gwg) {
    // ---------------- global query rows: wave = (b, h, row tile, key split)
    const int unit = blockIdx.x * 4 + wid;
    const int n_rt = (a.n_global + 31) / 32;
    const int ks = unit % a.g_splits;
    const int rt = (unit / a.g_splits) % n_rt;
    const int bhq = unit / (a.g_splits * n_rt);
    const bool live = bhq < a.batch * Hq;
    const int b = live ? bhq / Hq : 0, h = live ? bhq % Hq : 0, g = h / G;
    const int slot = min(rt * 32 + r32, a.n_global - 1);
    const int row = a.gpos[slot];
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
    RowState st{-INFINITY, 0.f};
    // this wave's key range, 32 keys at a time, through its own K and V half tiles
    const int kr = a.g_keys_per_split;
    const int k0 = min(N, ks * kr), k1 = min(N, k0 + kr);
    uint8_t* kt = smem + wid * (LDS_BYTES / 4);
    uint8_t* vt = kt + T::BYTES / 2;  // half-height tiles: 32 rows each
    static_assert(T::BYTES % 2048 == 0, "half tiles are whole 1 KB chunks");
    auto rows = [&](auto comp_tag) {
      constexpr bool COMP = decltype(comp_tag)::value;
      for (int j0 = k0; j0 < k1; j0 += 32) {
        typedef __attribute__((address_space(3))) void lds_void;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        constexpr int NCH = T::BYTES / 2048;  // 1 KB chunks per 32-row tile
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
          const int off = 1024 * k + 16 * lane;
          const int r = off / T::RB, pc = (off % T::RB) >> 4;
          const size_t pos = (size_t)min(j0 + r, N - 1);
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(Kb + pos * D + (pc ^ T::k_swz(r)) * 8),
                                           (lds_void*)(kt + 1024 * k), 16, 0, 0);
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(Vb + pos * D + (pc ^ T::v_swz(r)) * 8),
                                           (lds_void*)(vt + 1024 * k), 16, 0, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        stage<D, 1, COMP>(kt, vt, qop, oacc, st, sl2, [&](int) { return range_bits32(0, N - 1 - j0); },
                          j0 + 32 > N ? 1u : 0u);
      }
    };
    if (live) {
      if (N < kCompKeys) rows(std::true_type{});
      else rows(std::false_type{});
    }
    // partial state of this wave -> workspace [b*Hq + h][rt][ks][32 rows]
    st.l = sum_halves(st.l);
    if (live) {
      const size_t prow = (((size_t)bhq * n_rt + rt) * a.g_splits + ks) * 32 + r32;
      if (h2 == 0) {
        a.g_part_ml[2 * prow] = st.m;
        a.g_part_ml[2 * prow + 1] = st.l;
      }
      float* po = a.g_part_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = oacc[dt][4 * j + i];
          *reinterpret_cast<f32x4*>(po + 32 * dt + 8 * j + 4 * h2) = v;
        }
    }
    return;
  }

  // ---------------- band workgroup
  const int w = blockIdx.x - n_gwg;
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
  const int ngc = LG ? __builtin_amdgcn_readfirstlane(s_ngcols) : 0;
  if (SP) {
    if (tid == 0) {
      // merge the tile's ascending selection (-1 padded; entries outside the
      // complete blocks skipped) with the sink blocks 0 .. nsb - 1
      const int32_t* sel = a.sp_sel + ((size_t)kvlin * a.sp_n_tiles + qt) * a.sp_top_k;
      const int nsb = (a.sp_n_sink + BN - 1) / BN, nbc = N / BN;
      int n = 0, i = 0, j = 0;
      while (i < a.sp_top_k || j < nsb) {
        int s = 0x7fffffff;
        while (i < a.sp_top_k) {
          s = sel[i];
          if (s >= 0 && s < nbc) break;
          s = 0x7fffffff;
          ++i;
        }
        const int k = j < nsb ? j : 0x7fffffff;
        if (s == 0x7fffffff && k == 0x7fffffff) break;
        if (s <= k) {
          xblk[n++] = 2 * s + 1;
          ++i;
          if (s == k) ++j;
        } else {
          xblk[n++] = 2 * k;
          ++j;
        }
      }
      s_nx = n;
    }
    __syncthreads();
  }
  const int nx = SP ? __builtin_amdgcn_readfirstlane(s_nx) : 0;  // extra stages, ahead of the band
  const int n_stage = nx + n_band + (ngc + BN - 1) / BN;

  // DIL: logical row x is physical row dil_off + dil * x (Q, K, V, O, lse); the
  // pitches below are then dil rows, else one row
  const int dil = DIL ? a.dil : 1;
  const size_t NP = DIL ? (size_t)a.seq_phys : (size_t)N;              // rows of Q, O, lse per (b, h)
  const size_t roff = DIL ? (size_t)a.dil_off : 0;
  const size_t kpitch = DIL ? (size_t)dil * D : (size_t)D;           // elements between logical rows
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.K) + ((size_t)(b * Hkv + g) * a.kv_capacity + roff) * D;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(a.V) + ((size_t)(b * Hkv + g) * a.kv_capacity + roff) * D;
  const int r0 = i0 + 32 * wid;
  const int myrow = r0 + r32;
  u32x4 qop[D / 16];
  {
    const uint16_t* Qp = reinterpret_cast<const uint16_t*>(a.Q) +
                         ((size_t)(b * Hq + h) * NP + roff + (size_t)dil * min(myrow, N - 1)) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qop[c] = *reinterpret_cast<const u32x4*>(Qp + 16 * c + 8 * h2);
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[t][e] = 0.f;
  RowState st{-INFINITY, 0.f};

  // Keys seen by the wave's rows (globals only add keys): the count is piecewise
  // linear in the row, so its minimum over the 32 rows sits at an end row.
  auto band_keys = [&](int i) {
    const int lo = wl < 0 ? 0 : max(0, i - wl);
    const int hi = wr < 0 ? N - 1 : min(N - 1, i + wr);
    return hi - lo + 1;
  };
  // decided for the whole workgroup (its waves must take the same stage loop:
  // the loops differ in their barriers and copies), from its first and last row
  const bool comp = min(band_keys(min(i0, N - 1)), band_keys(min(i0 + BM - 1, N - 1))) < kCompKeys;

  auto row_pos = [&](int stg, int r) {
    stg -= nx;
    if (stg < n_band) return min((t_lo + stg) * BN + r, N - 1);
    const int slot = (stg - n_band) * BN + r;
    return gcols[min(slot, ngc - 1)];
  };
  DmaLane<D> dl;
  dl.init(wid, (uint32_t)(kpitch * 2));
  const uint8_t* Kb8 = reinterpret_cast<const uint8_t*>(Kb);
  const uint8_t* Vb8 = reinterpret_cast<const uint8_t*>(Vb);
  // copies of stage `stg` into (kt, vt): whole in-range band tiles take the
  // precomputed lane offsets; the sequence's last partial tile and the gathered
  // global columns compute each row's position
  auto issue_stage = [&](int stg, uint8_t* kt, uint8_t* vt) {
    if (SP && stg < nx) {  // a selected block (complete) or a sink block (the last may be partial)
      const int jb = (__builtin_amdgcn_readfirstlane(xblk[stg]) >> 1) * BN;
      if (jb + BN <= N) dl.issue(Kb8, Vb8, jb, kt, vt, wid);
      else dma_stage<D>(Kb, Vb, kt, vt, wid, 4, [&](int r) { return min(jb + r, N - 1); });
      return;
    }
    const int bs = stg - nx;
    const int row0 = (t_lo + bs) * BN;
    if (bs < n_band && row0 + BN <= N) dl.issue(Kb8, Vb8, row0, kt, vt, wid, kpitch * 2);
    else dma_stage<D>(Kb, Vb, kt, vt, wid, 4, [&](int r) { return row_pos(stg, r); }, kpitch);
  };
  // Stage s goes to K tile kb[s % 2] and V tile vb[s % 2]; K of stage s + 2 and
  // V of stage s + 1 are copied while stage s is computed (K runs one stage
  // ahead of V: the QK of stage s + 1 overlaps the exponentials of stage s).
  uint8_t* const kb[2] = {smem, smem + 2 * T::BYTES};
  uint8_t* const vb[2] = {smem + T::BYTES, smem + 3 * T::BYTES};
  // Mask of stage stg on this wave's logits: which halves sit on a mask edge
  // (wave-uniform bits), this lane's allowed keys [lo, hi] plus the global
  // columns among the stage's keys jb .. jb + 63 (position, or gathered-column
  // slot, of its first row); the words of allowed-key bits are built only for
  // the edge halves.  An element is kept by two ALU ops: a signed one-bit field
  // extract (0 or all ones) selects, bitwise, between the logit and -inf.
  auto mask_stage = [&](int stg, f32x16(&sx)[2], int nh = 2) {
    int jb, lo = 0, hi;
    uint32_t masked = 0;
    uint64_t gbits = 0ull;
    if (SP && stg < nx) {
      const int xb = __builtin_amdgcn_readfirstlane(xblk[stg]);
      jb = (xb >> 1) * BN;
      // keys before this row's window (and below n_sink for a sink-only block);
      // the wave's first row allows the fewest
      const int cap = (xb & 1) ? 0x7fffffff : a.sp_n_sink - 1;
      hi = min(myrow - wl - 1, cap);
      const int hi0 = min(r0 - wl - 1, cap);
#pragma unroll
      for (int u = 0; u < 2; ++u) masked |= (jb + 32 * u + 31 > hi0 ? 1u : 0u) << u;
    } else if (stg - nx < n_band) {
      jb = (t_lo + stg - nx) * BN;
      lo = wl < 0 ? 0 : myrow - wl;
      hi = min(N - 1, wr < 0 ? N - 1 : myrow + wr);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j0 = jb + 32 * u;
        // every key of the half allowed for all 32 rows
        const bool all_lo = wl < 0 || j0 >= r0 + 31 - wl;
        const bool all_hi = wr < 0 || j0 + 31 <= r0 + wr;
        masked |= (all_lo && all_hi && j0 + 31 < N ? 0u : 1u) << u;
      }
      if (LG && masked) {
        for (int i = lower_bound_i32(a.gpos, a.n_global, jb); i < a.n_global && a.gpos[i] < jb + BN; ++i)
          gbits |= 1ull << (a.gpos[i] - jb);
      }
    } else {
      jb = (stg - nx - n_band) * BN;
      hi = ngc - 1;
#pragma unroll
      for (int u = 0; u < 2; ++u) masked |= (jb + 32 * u + 32 > ngc ? 1u : 0u) << u;
    }
    if (!masked) return;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u < nh && ((masked >> u) & 1u)) {
        const int j0 = jb + 32 * u;
        const uint32_t m = (range_bits32(lo - j0, hi - j0) | (uint32_t)(gbits >> (32 * u))) >> (4 * h2);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int pbit = 8 * (e >> 2) + (e & 3);
          const uint32_t keep = (uint32_t)((int)(m << (31 - pbit)) >> 31);
          // copied out first: a bit-cast of a vector-element lvalue reads element 0
          const float v = sx[u][e];
          const uint32_t x = __builtin_bit_cast(uint32_t, v);
          sx[u][e] = __builtin_bit_cast(float, (x & keep) | (0xff800000u & ~keep));
        }
      }
    }
  };
  // One stage at a time (K and V of stage s + 1 copied while stage s is
  // computed): for rows that see fewer than 256 keys (the first tiles of a
  // sequence), which take the compensated product (CP) and so keep its extra
  // P registers out of the pipelined loop's budget, and for every local+global
  // workgroup at d = 64 (one tile of logits live: four waves per SIMD).
  auto stages_single = [&](auto comp_tag) {
    constexpr bool CP = decltype(comp_tag)::value;
    if (n_stage == 0) return;
    issue_stage(0, kb[0], vb[0]);
    // stage stg from the tiles kb[cur], vb[cur]: its first NH 32-key halves
    auto body = [&](int stg, int cur, auto nh_tag) {
      constexpr int NH = decltype(nh_tag)::value;
      f32x16 sx[2];
      float unused = 0.f;
      u32x4 pop[2][2], plo[2][2];
      region_a<D, CP, true, false, NH>(kb[cur], qop, sx, sx, sl2, 0.f, pop, plo, unused);
      mask_stage(stg, sx, NH);
      float mx = region_b<D, CP, false, true, NH>(nullptr, pop, plo, oacc, sx);
      mx = max_halves(mx);
      const float m_cand = mx * sl2;
      const bool need = m_cand > st.m + kHeadroom;
      if (__ballot(need)) {
        const float m_new = need ? m_cand : st.m;
        const float alpha = need ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
        st.l *= alpha;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;
        st.m = m_new;
      }
      float psum = 0.f;
      region_a<D, CP, false, true, NH>(nullptr, qop, sx, sx, sl2, (st.m == -INFINITY) ? 0.f : -st.m, pop, plo,
                                      psum);
      st.l += psum;
      region_b<D, CP, true, false, NH>(vb[cur], pop, plo, oacc, sx);
    };
    auto one = [&](int stg, int cur, auto nh_tag) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies for `stg` landed
      __syncthreads();  // every wave's copies landed; every wave is done with the other buffer
      if (stg + 1 < n_stage) issue_stage(stg + 1, kb[cur ^ 1], vb[cur ^ 1]);
      body(stg, cur, nh_tag);
    };
    constexpr std::integral_constant<int, 2> kBoth{};
    // The last stage, when it is a gathered global-column stage holding at
    // most 32 columns, has a second half of padding for every row: the
    // workgroup computes its first half alone (after the loop, so the loop
    // body keeps one shape)
    const int last = n_stage - 1;
    const bool last_half = LG && last - nx >= n_band && (last - nx - n_band) * BN + 32 >= ngc;
    const int n_loop = last_half ? last : n_stage;
    int stg = 0;
    for (; stg + 1 < n_loop; stg += 2) {
      one(stg, 0, kBoth);
      one(stg + 1, 1, kBoth);
    }
    if (stg < n_loop) one(stg, 0, kBoth);
    if (last_half) {
      constexpr std::integral_constant<int, 1> kFirst{};
      if (last & 1) one(last, 1, kFirst);
      else one(last, 0, kFirst);
    }
  };
  auto stages = [&]() {
    constexpr bool COMP = false;
    if (n_stage == 0) return;
    issue_stage(0, kb[0], vb[0]);
    if (n_stage > 1) issue_stage(1, kb[1], nullptr);
    f32x16 sA[2], sB[2];
    u32x4 pop[2][2], plo[2][2];
    float nm = 0.f;
    // the wave's new row max from the per-lane maxima of a stage's logits: the
    // running max moves only when it grows by more than 2^8 (log2 units), and
    // then the normaliser and O are rescaled (wave-uniform branch)
    auto update_max = [&](float mx) {
      mx = max_halves(mx);
      const float m_cand = mx * sl2;
      const bool need = m_cand > st.m + kHeadroom;
      if (__ballot(need)) {
        const float m_new = need ? m_cand : st.m;
        const float alpha = need ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
        st.l *= alpha;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;
        st.m = m_new;
      }
      nm = (st.m == -INFINITY) ? 0.f : -st.m;
    };
    // prologue: S_0 = K_0 Q^T, its mask and max
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    {
      float unused = 0.f;
      region_a<D, COMP, true, false>(kb[0], qop, sA, sA, sl2, nm, pop, plo, unused);
    }
    mask_stage(0, sA);
    update_max(region_b<D, COMP, false, true>(nullptr, pop, plo, oacc, sA));
    // stage j (logits in s) with stage j + 1 (logits into sn): exponentials of j
    // under the MFMAs of S_{j+1}, then O += V_j P_j under the max of S_{j+1}
    auto iter = [&](int j, f32x16(&s)[2], f32x16(&sn)[2], uint8_t* kt_next, uint8_t* vt_cur, uint8_t* k_dst,
                    uint8_t* v_dst) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies of K_{j+1}, V_j landed
      __syncthreads();  // every wave's copies landed; every wave is done with K_j and V_{j-1}
      if (j + 2 < n_stage) issue_stage(j + 2, k_dst, nullptr);
      issue_stage(j + 1, nullptr, v_dst);
      float psum = 0.f;
      region_a<D, COMP, true, true>(kt_next, qop, sn, s, sl2, nm, pop, plo, psum);
      st.l += psum;
      mask_stage(j + 1, sn);
      update_max(region_b<D, COMP, true, true>(vt_cur, pop, plo, oacc, sn));
    };
    // the last stage: its exponentials and O += V P
    auto last = [&](f32x16(&s)[2], uint8_t* vt_cur) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      float psum = 0.f;
      region_a<D, COMP, false, true>(nullptr, qop, s, s, sl2, nm, pop, plo, psum);
      st.l += psum;
      region_b<D, COMP, true, false>(vt_cur, pop, plo, oacc, s);
    };
    // unrolled by two so each buffer's LDS addresses are compile-time offsets
    int j = 0;
    for (; j + 2 < n_stage; j += 2) {
      iter(j, sA, sB, kb[1], vb[0], kb[0], vb[1]);
      iter(j + 1, sB, sA, kb[0], vb[1], kb[1], vb[0]);
    }
    if (j + 1 < n_stage) {
      iter(j, sA, sB, kb[1], vb[0], kb[0], vb[1]);
      last(sB, vb[1]);
    } else {
      last(sA, vb[0]);
    }
  };
  if (comp) stages_single(std::true_type{});
  else if constexpr (LG && D == 64) stages_single(std::false_type{});
  else stages();
  // write rows (global rows are written by the merge of their split partials)
  st.l = sum_halves(st.l);
  bool store = myrow < N;
  if (LG && store) {
    const int i = lower_bound_i32(a.gpos, a.n_global, myrow);
    store = !(i < a.n_global && a.gpos[i] == myrow);
  }
  if (store) {
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    float* orow = a.O + ((size_t)(b * Hq + h) * NP + roff + (size_t)dil * myrow) * D;
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
      a.lse[(size_t)(b * Hq + h) * NP + roff + (size_t)dil * myrow] =
          st.l > 0.f ? (st.m + log2f(st.l)) * kLn2 : -INFINITY;
  }
}

// Merge the key-split partials of every global query row: one wave per
// (b, h, global row); lane owns dims lane + 64e; the partials are read 32 at a
// time (all loads of a chunk in flight together) and folded online.
template <int D>
__global__ __launch_bounds__(64) void prefill_global_merge_kernel(PrefillArgs a) {
  constexpr int DL = D / 64, CH = 32;
  const int n_rt = (a.n_global + 31) / 32;
  const int gi = blockIdx.x % a.n_global;
  const int bhq = blockIdx.x / a.n_global;
  const int rt = gi / 32, r = gi % 32;
  const int lane = threadIdx.x;
  const int KS = a.g_splits;
  const size_t base = ((size_t)bhq * n_rt + rt) * KS;
  float M = -INFINITY, L = 0.f, O[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) O[e] = 0.f;
  for (int j0 = 0; j0 < KS; j0 += CH) {
    float ms[CH], ls[CH], os[CH][DL];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const size_t prow = (base + min(j0 + u, KS - 1)) * 32 + r;
      ms[u] = j0 + u < KS ? a.g_part_ml[2 * prow] : -INFINITY;
      ls[u] = a.g_part_ml[2 * prow + 1];
#pragma unroll
      for (int e = 0; e < DL; ++e) os[u][e] = a.g_part_o[prow * D + lane + 64 * e];
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
  const size_t orow = (size_t)bhq * a.seq_len + a.gpos[gi];
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int e = 0; e < DL; ++e) a.O[orow * D + lane + 64 * e] = O[e] * inv;
  if (a.lse != nullptr && lane == 0) a.lse[orow] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <int D, bool LG>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  const int n_qt = (a.seq_len + BM - 1) / BM;
  const int n_wg = (LG ? a.n_global_wg : 0) + n_qt * a.batch * a.n_q_heads;
  if (!LG && a.dil > 1) {
    hipLaunchKernelGGL((prefill_kernel<D, false, false, true>), dim3(n_wg), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (!LG && a.sp_sel != nullptr) {
    hipLaunchKernelGGL((prefill_kernel<D, false, true>), dim3(n_wg), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((prefill_kernel<D, LG>), dim3(n_wg), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !LG) return e;
  hipLaunchKernelGGL((prefill_global_merge_kernel<D>), dim3(a.batch * a.n_q_heads * a.n_global), dim3(64), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

void prefill_global_geometry(int seq_len, int n_global, int batch, int n_q_heads, int* splits,
                             int* keys_per_split, int* n_wg) {
  if (n_global <= 0) {
    *splits = 0;
    *keys_per_split = 0;
    *n_wg = 0;
    return;
  }
  // about 512 keys per wave: short per-wave chains, many waves in flight
  const int kps = 512;
  const int ks = (seq_len + kps - 1) / kps;
  const int n_rt = (n_global + 31) / 32;
  const long long units = (long long)batch * n_q_heads * n_rt * ks;
  *splits = ks;
  *keys_per_split = kps;
  *n_wg = (int)((units + 3) / 4);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const bool lg = a.n_global > 0;
  if (a.head_dim == 64) return lg ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
  return lg ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
}

}  // namespace bsattn
