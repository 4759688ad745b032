// Threshold-l2 keep-mask: the token-pruning step in front of the ragged path.
//
// "Dispatch-Aware Ragged Attention for Pruned Vision Transformers" evaluates
// its pipeline under four pruning algorithms, Threshold-l2 among them
// (aissential.tech summary, "Summary"); the pages do not define it further.
// Reading used here: CLS (token 0) is always kept; a patch token is kept
// when the L2 norm of its embedding row reaches the per-image keep-quantile
// q of the patch norms (linear interpolation between order statistics).
// In exact arithmetic that is "norm >= the r0-th smallest patch norm",
// r0 = ceil(q (P - 1)) for P = N - 1 patches, and that order-statistic form
// is what the kernel evaluates: patch j is kept when at least r0 + 1 patch
// norms, its own included, are at most its own.
//
// The decision is taken on squared norms in fp64: every square of an fp32 or
// 16-bit value is exact in fp64, and the squares are added in channel order
// c = 0, 1, ..., C - 1, one rounding per addition.  The order is fixed so the
// fp64 value, and with it every keep decision, is unique.
//
// Work decomposition: one workgroup per image, one wave per 64 token rows,
// one lane per token.  A lane must add its own row's channels in order, but
// rows lie C * s bytes apart, so the wave reads its 64 rows 128 bytes at a
// time with coalesced 16-byte loads (8 lanes per row segment), parks the
// 8 KB tile in LDS (16-byte pieces XOR-swizzled by row so that the eight
// lanes of a read phase hit distinct banks) and each lane then walks its
// own row segment.  The next two tiles' loads are in flight while the
// current one is summed.  After a barrier the image's squared norms sit in
// LDS and every thread ranks one patch against all the others.
#include "rva_device.h"
#include "rva_internal.h"

namespace rva {

constexpr int kTileRowBytes = 128;                  // bytes of one row per tile
constexpr int kTileBytes = 64 * kTileRowBytes;      // one wave's tile

// acc += x * x for every element of a 16-byte piece, in element order.
template <int DT>
__device__ __forceinline__ void add_squares(double& acc, u32x4 piece) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = piece[i];
    if constexpr (DT == 0) {
      const double v = (double)__uint_as_float(w);
      acc = __builtin_fma(v, v, acc);
    } else {
#pragma unroll
      for (int half = 0; half < 2; ++half) {  // little-endian: low half is the earlier element
        const uint32_t bits = half ? (w >> 16) : (w & 0xFFFFu);
        float f;
        if constexpr (DT == 1) {
          f = (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
        } else {
          f = __uint_as_float(bits << 16);
        }
        const double v = (double)f;
        acc = __builtin_fma(v, v, acc);
      }
    }
  }
}

template <int DT>
__global__ __launch_bounds__(1024) void threshold_l2_kernel(ThreshParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int ES = DT == 0 ? 4 : 2;
  const int b = blockIdx.x, N = p.N;
  const int lane = lane_id(), w = wave_id(), nw = (int)(blockDim.x >> 6);
  const uint32_t row_bytes = (uint32_t)p.C * ES;
  const Rsrc rx = make_rsrc(static_cast<const char*>(p.x) + (size_t)b * N * row_bytes,
                            (uint32_t)N * row_bytes);
  unsigned char* tile = smem + w * kTileBytes;
  double* sq = reinterpret_cast<double*>(smem + nw * kTileBytes);
  const int nchunks = (int)((row_bytes + kTileRowBytes - 1) / kTileRowBytes);
  const int row0 = w * 64;
  const int lr = lane >> 3, pc = lane & 7;  // load role: rows lr + 8u, piece pc

  // byte offset of piece pc of tile row lr + 8u in chunk k; past the row's
  // end (last chunk, or the look-ahead past the last chunk) or past the
  // image's rows it is kOOB, which loads zeros
  auto offset = [&](int k, int u) -> uint32_t {
    const int r = row0 + lr + 8 * u;
    const uint32_t cb = (uint32_t)k * kTileRowBytes + (uint32_t)pc * 16;
    return (r < N && cb < row_bytes) ? (uint32_t)r * row_bytes + cb : kOOB;
  };

  // Two tiles in flight per wave: tile k is parked and summed while tiles
  // k + 1 and k + 2 load.  A wave reads back only the tile it wrote, and LDS
  // executes one wave's instructions in issue order, so the exchange needs
  // no workgroup barrier, only a compiler barrier that keeps the LDS
  // accesses in program order; the waves of the image run independently.
  auto step = [&](u32x4 (&v)[8], int k, double& acc) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = lr + 8 * u;
      *reinterpret_cast<u32x4*>(tile + r * kTileRowBytes + ((pc ^ (r & 7)) << 4)) = v[u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)offset(k + 2, u), 0, 0);
    asm volatile("" ::: "memory");
    // zero pieces (past the row's end) add exact zeros
#pragma unroll
    for (int q = 0; q < 8; ++q)
      add_squares<DT>(acc, *reinterpret_cast<const u32x4*>(tile + lane * kTileRowBytes + ((q ^ (lane & 7)) << 4)));
    asm volatile("" ::: "memory");
  };
  u32x4 va[8], vb[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) va[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)offset(0, u), 0, 0);
#pragma unroll
  for (int u = 0; u < 8; ++u) vb[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)offset(1, u), 0, 0);
  double acc = 0.0;
  for (int k = 0; k < nchunks; k += 2) {
    step(va, k, acc);
    if (k + 1 < nchunks) step(vb, k + 1, acc);
  }
  if (row0 + lane < N) sq[row0 + lane] = acc;
  __syncthreads();

  uint8_t* mrow = p.mask + (size_t)b * N;
  for (int j = (int)threadIdx.x; j < N; j += (int)blockDim.x) {
    uint8_t keep = 1;  // CLS
    if (j > 0) {
      const double sj = sq[j];
      int at_most = 0;
      for (int i = 1; i < N; ++i) at_most += sq[i] <= sj ? 1 : 0;
      keep = at_most >= p.r0 + 1 ? 1 : 0;
    }
    mrow[j] = keep;
  }
}

size_t threshold_lds_bytes(int N) {
  const int nw = (N + 63) / 64;
  return (size_t)nw * kTileBytes + (size_t)round_up(N * 8, 16);
}

hipError_t threshold_init() {
  const void* fns[3] = {reinterpret_cast<const void*>(&threshold_l2_kernel<0>),
                        reinterpret_cast<const void*>(&threshold_l2_kernel<1>),
                        reinterpret_cast<const void*>(&threshold_l2_kernel<2>)};
  for (const void* f : fns) {
    hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_threshold(const ThreshParams& p, int B, int dtype, hipStream_t s) {
  const dim3 blk(64 * ((p.N + 63) / 64));
  const size_t lds = threshold_lds_bytes(p.N);
  if (dtype == 0) hipLaunchKernelGGL((threshold_l2_kernel<0>), dim3(B), blk, lds, s, p);
  else if (dtype == 1) hipLaunchKernelGGL((threshold_l2_kernel<1>), dim3(B), blk, lds, s, p);
  else hipLaunchKernelGGL((threshold_l2_kernel<2>), dim3(B), blk, lds, s, p);
  return hipGetLastError();
}

}  // namespace rva
