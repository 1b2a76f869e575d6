// Device-side helpers shared by the gfx950 kernels: bf16 conversion, MFMA
// wrappers, wave reductions and the forced-token mask of a decode step.
//
// MFMA operand layouts (gfx950, checked on the device with an in-bounds probe):
//  v_mfma_f32_16x16x32_bf16   A[i][k]: lane i + 16*(k/8), element k%8
//                             B[k][j]: lane j + 16*(k/8), element k%8
//                             D[i][j]: lane j + 16*(i/4), element i%4
//  v_mfma_f32_32x32x16_bf16   A[i][k]: lane i + 32*(k/8), element k%8
//                             B[k][j]: lane j + 32*(k/8), element k%8
//                             D[i][j]: lane j + 32*((i/4)%2), element 4*(i/8) + i%4
//  ds_read_b64_tr_b16         within each 16-lane group, lane a supplies an
//                             8-byte row M[a][0..3]; lane i receives
//                             element e of M[4e + i/4][i%4].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBlock = 64;  // tokens per KV block (S)
constexpr int kMaxBlocks = 65536;  // complete blocks per (b, K/V head) the top-k handles
constexpr int kMaxTopK = 1024;     // selected blocks per (b, K/V head)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Low / high bf16 of a packed pair to fp32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 of two values packed into one dword (lo = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  ua = (ua + 0x7fffu + ((ua >> 16) & 1u)) >> 16;
  ub = (ub + 0x7fffu + ((ub >> 16) & 1u)) & 0xffff0000u;
  return ua | ub;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Round-to-nearest-even fp32 -> bf16 of two values in one v_cvt_pk_bf16_f32 (lo = a).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Transposing 8-byte LDS read (gfx950).  `byte_off` is a byte offset into dynamic/static LDS.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_base, uint32_t byte_off) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const __attribute__((address_space(3))) char* p =
      (const __attribute__((address_space(3))) char*)lds_base + byte_off;
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  return __builtin_bit_cast(u32x2, r);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ------------------------------------------------------------------ forced tokens
//
// The tokens every decode step attends regardless of selection: sinks
// [0, n_sink), the window [win_lo, t] with t = n_ctx - 1, and the global
// positions (sorted).  A block whose 64 tokens are all forced is not a
// candidate for selection.
struct ForcedSet {
  int32_t n_ctx;
  int32_t sink_end;  // min(n_sink, n_ctx)
  int32_t win_lo;    // first window token (n_ctx when there is no window)
  int32_t n_global;
  int32_t gpos[256];
};

// 64-bit mask of `lo <= token < hi` within block [base, base + 64).
__host__ __device__ inline uint64_t range_mask64(int base, int lo, int hi) {
  const int a = lo - base > 0 ? lo - base : 0, b = hi - base < 64 ? hi - base : 64;
  if (a >= b) return 0ull;
  uint64_t hiMask = (b == 64) ? ~0ull : ((1ull << b) - 1ull);
  uint64_t loMask = (a == 0) ? 0ull : ((1ull << a) - 1ull);
  return hiMask & ~loMask;
}

// FP4 E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes 0,
// 0.5, 1, 1.5, 2, 3, 4, 6) as a 4-bit code: the value nearest to v, on a tie
// the code whose mantissa bit is 0.  The magnitude code is the number of
// midpoints between neighbouring values below |v|, counting a midpoint that
// |v| equals only when the code above it is even.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return m | ((v < 0.f && m != 0u) ? 8u : 0u);
}
// Value of an E2M1 code (low 4 bits of c), built as float32 bits: exponent
// e > 0 gives 2^(e-1) (1 + m/2); e = 0 gives m/2.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  uint32_t bits = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
  bits |= (c & 8u) << 28;
  return __uint_as_float(bits);
}

// Order-preserving 32-bit key of a float: larger float, larger unsigned key
// (-0 and +0 share the key of +0, as they compare equal).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = f == 0.f ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum across the 64 lanes of a wave with DPP: shifts of 1, 2,
// 4, 8 within each 16-lane row, then lane 15 of rows 0 / 2 added to rows 1 / 3
// (row_bcast:15) and lane 31 to rows 2 and 3 (row_bcast:31).  Lanes whose
// source is outside the row or the row mask take `old` = 0.
__device__ __forceinline__ int wave_incl_scan_dpp(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Bitwise AND of x_and and OR of x_or over the 64 lanes (wave-uniform results).
__device__ __forceinline__ void wave_and_or(uint32_t x_and, uint32_t x_or, uint32_t& all_and, uint32_t& all_or) {
  uint32_t a = x_and, o = x_or;
  // row_ror 8, 4, 2, 1: every lane of a row ends with the row's value
#define BSATTN_AND_OR_STEP(c)                                                  \
  a &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, c, 0xf, 0xf, false); \
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, c, 0xf, 0xf, false);
  BSATTN_AND_OR_STEP(0x128)
  BSATTN_AND_OR_STEP(0x124)
  BSATTN_AND_OR_STEP(0x122)
  BSATTN_AND_OR_STEP(0x121)
#undef BSATTN_AND_OR_STEP
  all_and = __builtin_amdgcn_readlane(a, 0) & __builtin_amdgcn_readlane(a, 16) &
            __builtin_amdgcn_readlane(a, 32) & __builtin_amdgcn_readlane(a, 48);
  all_or = __builtin_amdgcn_readlane(o, 0) | __builtin_amdgcn_readlane(o, 16) |
           __builtin_amdgcn_readlane(o, 32) | __builtin_amdgcn_readlane(o, 48);
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

__host__ __device__ inline int lower_bound_i32(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Forced tokens of block `blk`, restricted to tokens < n_ctx.
__host__ __device__ inline uint64_t forced_mask(const ForcedSet& f, int blk) {
  const int base = blk * kBlock;
  uint64_t m = range_mask64(base, 0, f.sink_end) | range_mask64(base, f.win_lo, f.n_ctx);
  if (f.n_global > 0) {
    int i = lower_bound_i32(f.gpos, f.n_global, base);
    for (; i < f.n_global && f.gpos[i] < base + kBlock; ++i) m |= 1ull << (f.gpos[i] - base);
  }
  return m;
}

}  // namespace bsattn
