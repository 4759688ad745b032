// Projections on the packed token buffer: y = x W^T + b on kept rows only.
//
// The packer of "Dispatch-Aware Ragged Attention for Pruned Vision
// Transformers" feeds the whole transformer block, not only attention
// (aissential.tech summary, "Method"), and the summary's "In practice" asks
// for attention and the rest of the block to be timed apart.  The rest of
// an attention block is two dense products on the token rows: the QKV
// projection in front of attention and the output projection behind it.
// Here both run on the T kept rows instead of the B*N padded ones, and each
// absorbs a step of the ragged path:
//   * the QKV product reads its input rows straight from the padded
//     embeddings through the kept-index list (the pack's gather) and writes
//     Q, K and V into three packed [T, H, 64] buffers (the column groups of
//     the fused weight);
//   * the output product scatters its rows back to their padded positions
//     and zero-fills the pruned rows (the unpack), optionally adding a
//     residual first.
// T is read on the device (cu_seqlens[B]); the grid is sized for the bound
// B*N and workgroups past T return at once, so nothing waits on the host.
//
// Kernel (gfx950, fp16/bf16 in, fp32 accumulate): 128x128 output tiles,
// four waves of 64x64, K taken 64 at a time through double-buffered LDS
// (16-byte pieces XOR-swizzled by row: conflict-free 16-byte operand reads),
// next K tile loaded into registers while the current one is multiplied.
// The 16x16x32 matrix-core product is taken transposed, D^T = W X^T, so
// that each lane ends with four adjacent output columns of one row: one
// 8-byte store per 16x16 block.  Tiles are ordered so that the workgroups
// of one XCD walk consecutive row blocks through all column tiles, keeping
// each input row block in that XCD's L2 while it is reused.
#include "rva_device.h"
#include "rva_internal.h"

namespace rva {

typedef _Float16 lf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 lbf16x8 __attribute__((ext_vector_type(8)));
typedef float lf32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ lf32x4 mfma16(u32x4 a, u32x4 b, lf32x4 c) {
  if constexpr (DT == 1)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(lf16x8, a),
                                                  __builtin_bit_cast(lf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(lbf16x8, a),
                                                   __builtin_bit_cast(lbf16x8, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ float to_f32(uint32_t bits16) {
  if constexpr (DT == 1) return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  else return __uint_as_float(bits16 << 16);
}

// Four fp32 values -> four 16-bit values (round to nearest even), packed.
template <int DT>
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
  if constexpr (DT == 1) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 h = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
    return __builtin_bit_cast(u32x2, h);
  } else {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    b4 h = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    return __builtin_bit_cast(u32x2, h);
  }
}

constexpr int kLinTile = 128;      // output rows and columns per workgroup
constexpr int kLinK = 64;          // K per stage
constexpr int kLinThreads = 256;
constexpr int kLinZeroRows = 64;   // padded rows per zero-fill workgroup

// byte offset of 16-byte piece p of row r in a [128][64] half tile
__device__ __forceinline__ int lin_swz(int r, int p) { return r * 128 + ((p ^ (r & 7)) << 4); }

template <int DT>
__device__ __forceinline__ void linear_tile(const LinearParams& p, int mb, int nb,
                                            unsigned char* lds, int M) {
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int g = lane >> 4, r16 = lane & 15;
  const int wm = w >> 1, wn = w & 1;  // wave's 64x64 sub-tile
  const int m0 = mb * kLinTile, n0 = nb * kLinTile;
  const uint32_t kbytes = (uint32_t)p.K * 2;
  const Rsrc rx = make_rsrc(p.x, (uint32_t)p.x_rows * kbytes);
  const Rsrc rw = make_rsrc(p.w, (uint32_t)p.Nout * kbytes);

  // load roles: pieces e = tid + 256u (u < 4) of each 128-row x 8-piece tile
  uint32_t arow[4], brow[4];
  int lrow[4], lpc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = tid + kLinThreads * u;
    lrow[u] = e >> 3;
    lpc[u] = e & 7;
    const int m = m0 + lrow[u];
    int src = -1;
    if (m < M) src = p.x_index ? p.x_index[m] : m;
    arow[u] = src >= 0 ? (uint32_t)src * kbytes : kOOB;
    const int n = n0 + lrow[u];
    brow[u] = n < p.Nout ? (uint32_t)n * kbytes : kOOB;
  }
  auto koff = [&](uint32_t row, int kt, int pc) -> uint32_t {
    const uint32_t cb = (uint32_t)kt * (kLinK * 2) + (uint32_t)pc * 16;
    return (row != kOOB && cb < kbytes) ? row + cb : kOOB;
  };

  const int nkt = (p.K + kLinK - 1) / kLinK;
  u32x4 ra[4], rb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ra[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)koff(arow[u], 0, lpc[u]), 0, 0);
    rb[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)koff(brow[u], 0, lpc[u]), 0, 0);
  }
  lf32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = lf32x4{0.f, 0.f, 0.f, 0.f};

  // stage s: A tile at lds + s*32K, W tile at lds + s*32K + 16K
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    *reinterpret_cast<u32x4*>(lds + lin_swz(lrow[u], lpc[u])) = ra[u];
    *reinterpret_cast<u32x4*>(lds + 16384 + lin_swz(lrow[u], lpc[u])) = rb[u];
  }
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int s = kt & 1;
    // next stage's loads (past the last stage they are out of range: zeros)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ra[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)koff(arow[u], kt + 1, lpc[u]), 0, 0);
      rb[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)koff(brow[u], kt + 1, lpc[u]), 0, 0);
    }
    const unsigned char* As = lds + s * 32768;
    const unsigned char* Ws = As + 16384;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 wf[4], xf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wf[i] = *reinterpret_cast<const u32x4*>(Ws + lin_swz(wn * 64 + 16 * i + r16, 4 * ks + g));
        xf[i] = *reinterpret_cast<const u32x4*>(As + lin_swz(wm * 64 + 16 * i + r16, 4 * ks + g));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<DT>(wf[i], xf[j], acc[i][j]);
    }
    unsigned char* Nx = lds + (s ^ 1) * 32768;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<u32x4*>(Nx + lin_swz(lrow[u], lpc[u])) = ra[u];
      *reinterpret_cast<u32x4*>(Nx + 16384 + lin_swz(lrow[u], lpc[u])) = rb[u];
    }
    __syncthreads();
  }

  // epilogue: acc[i][j] lane (r16, g) holds out[m][n .. n+3] with
  // m = m0 + 64 wm + 16 j + r16, n = n0 + 64 wn + 16 i + 4 g
  const int ng = p.Nout / p.y_split;  // columns per output group
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 64 + 16 * j + r16;
    if (m >= M) continue;
    const int orow = p.y_index ? p.y_index[m] : m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + wn * 64 + 16 * i + 4 * g;
      if (n >= p.Nout) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if (p.bias) {
        const u32x2 bb = *reinterpret_cast<const u32x2*>(static_cast<const char*>(p.bias) + (size_t)n * 2);
        v[0] += to_f32<DT>(bb[0] & 0xFFFFu);
        v[1] += to_f32<DT>(bb[0] >> 16);
        v[2] += to_f32<DT>(bb[1] & 0xFFFFu);
        v[3] += to_f32<DT>(bb[1] >> 16);
      }
      const int grp = n / ng, col = n - grp * ng;
      const size_t eoff = ((size_t)orow * ng + col) * 2;
      if (p.residual) {
        const u32x2 rr = *reinterpret_cast<const u32x2*>(static_cast<const char*>(p.residual) + eoff);
        v[0] += to_f32<DT>(rr[0] & 0xFFFFu);
        v[1] += to_f32<DT>(rr[0] >> 16);
        v[2] += to_f32<DT>(rr[1] & 0xFFFFu);
        v[3] += to_f32<DT>(rr[1] >> 16);
      }
      *reinterpret_cast<u32x2*>(static_cast<char*>(p.y[grp]) + eoff) = pack4<DT>(v[0], v[1], v[2], v[3]);
    }
  }
}

// Zero-fill workgroup: padded rows [z * 64, z * 64 + 64) whose mask byte is 0.
__device__ __forceinline__ void linear_zero_rows(const LinearParams& p, int z) {
  const int r0 = z * kLinZeroRows;
  const int rows = min(kLinZeroRows, p.zero_rows - r0);
  const int pieces = p.Nout * 2 / 16;
  char* y = static_cast<char*>(p.y[0]);
  for (int e = threadIdx.x; e < rows * pieces; e += kLinThreads) {
    const int r = r0 + e / pieces, pc = e % pieces;
    if (!p.zero_mask[r])
      *reinterpret_cast<u32x4*>(y + ((size_t)r * p.Nout) * 2 + (size_t)pc * 16) = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int DT>
__global__ __launch_bounds__(kLinThreads, 2) void linear_kernel(LinearParams p) {
  __shared__ __align__(16) unsigned char lds[2 * 32768];
  const int mt = p.m_tiles, nt = p.n_tiles, tiles = mt * nt;
  int bid = blockIdx.x;
  if (bid >= tiles) {
    linear_zero_rows(p, bid - tiles);
    return;
  }
  // XCD-aware order: the workgroups dispatched to one XCD (bid = x mod 8)
  // take consecutive tiles, row block major
  {
    const int q8 = tiles >> 3, r8 = tiles & 7, x = bid & 7, s = bid >> 3;
    bid = (x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8) + s;
  }
  const int mb = bid / nt, nb = bid - mb * nt;
  const int M = p.m_count ? min(*p.m_count, p.M) : p.M;
  if (mb * kLinTile >= M) return;
  linear_tile<DT>(p, mb, nb, lds, M);
}

hipError_t launch_linear(const LinearParams& p, int dtype, hipStream_t s) {
  const int zero_wgs = p.zero_mask ? (p.zero_rows + kLinZeroRows - 1) / kLinZeroRows : 0;
  const dim3 grid(p.m_tiles * p.n_tiles + zero_wgs);
  if (dtype == 1) hipLaunchKernelGGL((linear_kernel<1>), grid, dim3(kLinThreads), 0, s, p);
  else hipLaunchKernelGGL((linear_kernel<2>), grid, dim3(kLinThreads), 0, s, p);
  return hipGetLastError();
}

int linear_tile_size() { return kLinTile; }

}  // namespace rva
