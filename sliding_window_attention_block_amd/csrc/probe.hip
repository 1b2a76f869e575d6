// Gather probe: the HBM bandwidth a loads-only gather of listed K/V blocks
// reaches on this GPU, the ceiling the sparse decode's gather is measured
// against (decode is bound by the KV bytes it reads: COBS explainer, technical
// summary section 1).  It is a measurement aid, not a step of the method.
//
// The pair's listed blocks are split into 32-token half blocks (a contiguous
// 32 x d run of K and the same of V, 8 KB each at d = 128), the unit the
// decode waves gather.  Workgroups of four waves, `wg_per_pair` of them per
// (b, K/V head) pair as the decode places them; the pair's half blocks are
// dealt to its waves in even runs, and each wave keeps DEPTH of them in flight
// (16-byte loads, 1 KB per instruction, every byte read once) before folding
// them into one XOR per lane, written out so no load is dead.
#include "launch.hpp"

namespace bsattn {
namespace {

template <int D, int DEPTH>
__global__ __launch_bounds__(256, 1) void gather_probe_kernel(ProbeArgs a) {
  constexpr int HB = 32 * D * 2;   // bytes of a 32-token half block of K (or V)
  constexpr int NL = HB / 1024;    // 16-byte loads per lane per half block and tensor
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wpp = 4 * a.wg_per_pair;
  const int wave = blockIdx.x * 4 + wid;
  const int pair = wave / wpp, wi = wave % wpp;
  const int n_half = 2 * a.n_blocks;
  const int per = (n_half + wpp - 1) / wpp;
  const int h0 = min(n_half, wi * per), h1 = min(n_half, h0 + per);
  const size_t pair_bytes = (size_t)a.kv_capacity * D * 2;
  const uint8_t* Kp = static_cast<const uint8_t*>(a.K) + (size_t)pair * pair_bytes;
  const uint8_t* Vp = static_cast<const uint8_t*>(a.V) + (size_t)pair * pair_bytes;
  const int32_t* bl = a.blocks + (size_t)pair * a.n_blocks;
  const int nbc = a.kv_capacity / kBlock;
  uint32_t acc = 0;
  for (int h = h0; h < h1; h += DEPTH) {
    u32x4 kv[DEPTH][2][NL];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      if (h + i < h1) {  // wave-uniform
        const int blk = min(max(bl[(h + i) >> 1], 0), nbc - 1);
        const size_t off = ((size_t)blk * kBlock + ((h + i) & 1) * 32) * D * 2 + 16 * lane;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          kv[i][0][j] = *reinterpret_cast<const u32x4*>(Kp + off + 1024 * j);
          kv[i][1][j] = *reinterpret_cast<const u32x4*>(Vp + off + 1024 * j);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      if (h + i < h1) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < NL; ++j) acc ^= kv[i][t][j][0] ^ kv[i][t][j][1] ^ kv[i][t][j][2] ^ kv[i][t][j][3];
      }
    }
  }
  a.checksum[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

template <int D>
hipError_t launch_d(const ProbeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.n_pairs * a.wg_per_pair));
  switch (a.depth) {
    case 1: hipLaunchKernelGGL((gather_probe_kernel<D, 1>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((gather_probe_kernel<D, 2>), grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((gather_probe_kernel<D, 3>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((gather_probe_kernel<D, 4>), grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_probe(const ProbeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace bsattn
