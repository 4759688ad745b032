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
// Kernel (gfx950, fp16/bf16 in, fp32 accumulate): 256x256 output tiles,
// sixteen waves of 64x64 (four per SIMD, so one wave's LDS reads hide behind
// another's matrix-core work), K taken 64 at a time.  Stages reach LDS by
// direct-to-LDS buffer loads (no staging registers), two buffers deep: the
// next stage is in flight while the current one is multiplied, and one
// barrier per stage orders both.  16-byte pieces are XOR-swizzled by row so
// that the 16-byte operand reads are conflict-free.  The 16x16x32
// matrix-core product is taken transposed, D^T = W X^T, so that each lane
// ends with four adjacent output columns of one row; a 16-lane row swap per
// pair of 16x16 blocks gives it eight, so the epilogue reads bias and
// residual and writes output 16 bytes per lane (64 contiguous bytes of a row
// per instruction), with non-temporal stores.  Tiles are dealt to the XCDs in round-robin groups of two row
// blocks (all their column tiles), so a group's input rows are reused from
// one XCD's L2 and the live row blocks (below the device-side row count)
// spread over every XCD.
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

constexpr int kLinBM = 256;        // product rows per workgroup
constexpr int kLinBN = 256;        // output columns per workgroup
constexpr int kLinK = 64;          // K per stage (32 or 64)
constexpr int kLinStages = 2;      // LDS ring depth (2 to 4)
constexpr int kLinWM = 4;          // waves along the rows
constexpr int kLinWN = 4;          // waves along the columns
constexpr int kLinWaves = kLinWM * kLinWN;
constexpr int kLinThreads = 64 * kLinWaves;
constexpr int kLinTM = kLinBM / kLinWM;  // a wave's rows
constexpr int kLinTN = kLinBN / kLinWN;  // a wave's columns
constexpr int kLinZeroRows = 64;   // padded rows per zero-fill workgroup
constexpr int kLinPitch = kLinK * 2;         // bytes of one staged row
constexpr int kLinPieces = kLinK / 8;        // 16-byte pieces per staged row
constexpr int kLinRowsPerLoad = 64 / kLinPieces;  // rows one 1 KB load fills
constexpr int kStageA = kLinBM * kLinPitch;  // bytes of one stage's input tile
constexpr int kStageB = kLinBN * kLinPitch;  // bytes of one stage's weight tile
constexpr int kStageBytes = kStageA + kStageB;
constexpr int kDmaA = kLinBM / kLinRowsPerLoad / kLinWaves;  // 1 KB loads per wave per stage
constexpr int kDmaB = kLinBN / kLinRowsPerLoad / kLinWaves;
static_assert(kLinK == 32 || kLinK == 64, "K per stage");
static_assert(kDmaA * kLinRowsPerLoad * kLinWaves == kLinBM &&
              kDmaB * kLinRowsPerLoad * kLinWaves == kLinBN, "whole loads");
constexpr int kDmaPerStage = kDmaA + kDmaB;  // vector memory ops per lane per stage
static_assert(kLinStages >= 2 && kLinStages <= 4, "ring depth");
static_assert(kDmaPerStage * (kLinStages - 1) < 64, "stages in flight must fit the wait counter");

constexpr int kLinGroupRows = 2;   // row blocks per XCD group

// Workgroup slots for the tiles: whole rounds of 8 XCD groups.
__host__ __device__ inline int linear_tile_slots(int m_tiles, int n_tiles) {
  const int group = kLinGroupRows * n_tiles;
  const int groups = (m_tiles * n_tiles + group - 1) / group;
  return (groups + 7) / 8 * 8 * group;
}

typedef __attribute__((address_space(3))) void* LdsPtr;

// Swizzle key of row r: piece p of the row is stored at slot p ^ key(r).  A
// 16-byte LDS read is served 8 lanes (128 bytes, every bank once) at a time,
// and the 8 lanes of an operand read take the same piece of 8 consecutive
// rows.  A 64-element row fills the 128 bytes of banks, so the key is r mod 8;
// two 32-element rows share them (r and r + 1 in opposite halves), so the key
// is (r / 2) mod 4.  (Hardware counters: no bank conflicts with either; the
// key (r / 4) mod 4 cost four conflict cycles per 32-element read.)
__device__ __forceinline__ int lin_key(int r) { return kLinK == 64 ? (r & 7) : ((r >> 1) & 3); }

// byte offset of 16-byte piece p of row r in a staged [rows][kLinK] half tile
__device__ __forceinline__ int lin_swz(int r, int p) { return r * kLinPitch + ((p ^ lin_key(r)) << 4); }

// Wait until at most N vector memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  // gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt (7) and lgkmcnt (15) left open
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A workgroup barrier without the full memory fence of __syncthreads (which
// would also wait for the stages still in flight).  The caller has already
// waited for the loads other waves must see; this wave's own LDS reads are
// completed first, because after the barrier other waves refill the buffer
// they read.  The clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int DT>
__device__ __forceinline__ void linear_tile(const LinearParams& p, int mb, int nb, int M,
                                            unsigned char* buf0, unsigned char* buf1,
                                            unsigned char* buf2, unsigned char* buf3) {
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, r16 = lane & 15;
  const int wm = w / kLinWN, wn = w - wm * kLinWN;  // wave's kLinTM x kLinTN sub-tile
  const int m0 = mb * kLinBM, n0 = nb * kLinBN;
  const uint32_t kbytes = (uint32_t)p.K * 2;
  const Rsrc rx = make_rsrc(p.x, (uint32_t)p.x_rows * kbytes);
  const Rsrc rw = make_rsrc(p.w, (uint32_t)p.Nout * kbytes);

  // Direct-to-LDS loads: one instruction fills kLinRowsPerLoad rows (1 KB) of a
  // stage, lane L landing at byte 16 L, i.e. row L / kLinPieces, slot
  // L % kLinPieces.  The lane fetches the piece that belongs in that slot
  // under the row swizzle, so LDS ends up in lin_swz order.  Rows past the
  // product (or the weight) read out of range.
  const int nkt = p.K / kLinK;
  uint32_t avoff[kDmaA], bvoff[kDmaB];
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) {
    const int r = w * (kLinBM / kLinWaves) + kLinRowsPerLoad * i + lane / kLinPieces;  // tile row
    const int m = m0 + r;
    int src = -1;
    if (m < M) src = p.x_index ? p.x_index[m] : m;
    avoff[i] = src >= 0 ? (uint32_t)src * kbytes + (((lane % kLinPieces) ^ lin_key(r)) << 4) : kOOB;
  }
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int r = w * (kLinBN / kLinWaves) + kLinRowsPerLoad * i + lane / kLinPieces;
    const int n = n0 + r;
    bvoff[i] = n < p.Nout ? (uint32_t)n * kbytes + (((lane % kLinPieces) ^ lin_key(r)) << 4) : kOOB;
  }
  // Stages past the last one are issued anyway (so that every step has the
  // same loads in flight and the wait counts stay static) through empty
  // descriptors: every lane is out of range and nothing is read.
  const Rsrc rnone = make_rsrc(p.x, 0);
  auto dma = [&](unsigned char* buf, int kt) {
    const bool live = kt < nkt;
    const Rsrc ra = live ? rx : rnone, rb = live ? rw : rnone;
    const int koff = live ? kt * kLinPitch : 0;
#pragma unroll
    for (int i = 0; i < kDmaA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (LdsPtr)(buf + (w * (kLinBM / kLinWaves) + kLinRowsPerLoad * i) * kLinPitch), 16,
          avoff[i], koff, 0, 0);
#pragma unroll
    for (int i = 0; i < kDmaB; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (LdsPtr)(buf + kStageA + (w * (kLinBN / kLinWaves) + kLinRowsPerLoad * i) * kLinPitch),
          16, bvoff[i], koff, 0, 0);
  };

  constexpr int NI = kLinTN / 16, NJ = kLinTM / 16;  // 16x16 blocks of a wave
  lf32x4 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = lf32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const unsigned char* buf) {
    const unsigned char* As = buf;
    const unsigned char* Ws = buf + kStageA;
#pragma unroll
    for (int ks = 0; ks < kLinK / 32; ++ks) {
      u32x4 wf[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i)
        wf[i] = *reinterpret_cast<const u32x4*>(Ws + lin_swz(wn * kLinTN + 16 * i + r16, 4 * ks + g));
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x4 xf = *reinterpret_cast<const u32x4*>(As + lin_swz(wm * kLinTM + 16 * j + r16, 4 * ks + g));
#pragma unroll
        for (int i = 0; i < NI; ++i) acc[i][j] = mfma16<DT>(wf[i], xf, acc[i][j]);
      }
    }
  };

  // Ring of kLinStages buffers, kLinStages - 1 stages in flight.  Step kt:
  // wait for this wave's loads of stage kt (later stages may still be in
  // flight), barrier (every wave's loads of stage kt have landed, every wave
  // is done with stage kt - 1), refill stage kt - 1's buffer with stage
  // kt + kLinStages - 1, multiply stage kt.  The ring is unrolled so that each
  // buffer is a distinct LDS object.
  unsigned char* bufs[4] = {buf0, buf1, buf2, buf3};
#pragma unroll
  for (int st = 0; st < kLinStages - 1; ++st) dma(bufs[st], st);
  for (int kt0 = 0; kt0 < nkt; kt0 += kLinStages) {
#pragma unroll
    for (int j = 0; j < kLinStages; ++j) {
      const int kt = kt0 + j;
      wait_vm<(kLinStages - 2) * kDmaPerStage>();
      bar();
      dma(bufs[(j + kLinStages - 1) % kLinStages], kt + kLinStages - 1);
      if (kt < nkt) compute(bufs[j]);
    }
  }
  wait_vm<0>();

  // epilogue: acc[i][j] lane (r16, g) holds out[m][n .. n+3] with
  // m = m0 + kLinTM wm + 16 j + r16, n = n0 + kLinTN wn + 16 i + 4 g.  One
  // 16-lane row swap per pair of column blocks (2e, 2e + 1) trades lane-row
  // parity g & 1 for the block parity: lane (r16, g) then holds the eight
  // columns 32 e + 16 (g & 1) + 8 (g >> 1) .. + 7 of its row (the first four
  // in acc[2e][j], the next four in acc[2e + 1][j]), so bias, residual and
  // output move 16 bytes per lane and 64 contiguous bytes of a row per
  // instruction.  Every lane takes part in the swaps before any row check.
  static_assert(NI % 2 == 0, "column blocks in pairs");
#pragma unroll
  for (int e = 0; e < NI / 2; ++e)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[2 * e][j][t]),
                                                         __float_as_uint(acc[2 * e + 1][j][t]), false,
                                                         false);
        acc[2 * e][j][t] = __uint_as_float(sw[0]);
        acc[2 * e + 1][j][t] = __uint_as_float(sw[1]);
      }
  const int ng = p.Nout / p.y_split;  // columns per output group (a multiple of 64)
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int m = m0 + wm * kLinTM + 16 * j + r16;
    if (m >= M) continue;
    const int orow = p.y_index ? p.y_index[m] : m;
#pragma unroll
    for (int e = 0; e < NI / 2; ++e) {
      const int n = n0 + wn * kLinTN + 32 * e + 16 * (g & 1) + 8 * (g >> 1);
      if (n >= p.Nout) continue;
      float v[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[t] = acc[2 * e][j][t];
        v[4 + t] = acc[2 * e + 1][j][t];
      }
      if (p.bias) {
        const u32x4 bb = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.bias) + (size_t)n * 2);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[2 * t] += to_f32<DT>(bb[t] & 0xFFFFu);
          v[2 * t + 1] += to_f32<DT>(bb[t] >> 16);
        }
      }
      const int grp = n / ng, col = n - grp * ng;
      const size_t eoff = ((size_t)orow * ng + col) * 2;
      if (p.residual) {
        const u32x4 rr = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.residual) + eoff);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[2 * t] += to_f32<DT>(rr[t] & 0xFFFFu);
          v[2 * t + 1] += to_f32<DT>(rr[t] >> 16);
        }
      }
      const u32x2 lo = pack4<DT>(v[0], v[1], v[2], v[3]), hi = pack4<DT>(v[4], v[5], v[6], v[7]);
      // written once, never read back by the launch: non-temporal
      __builtin_nontemporal_store(u32x4{lo[0], lo[1], hi[0], hi[1]},
                                  reinterpret_cast<u32x4*>(static_cast<char*>(p.y[grp]) + eoff));
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
      __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u},
                                  reinterpret_cast<u32x4*>(y + ((size_t)r * p.Nout) * 2 + (size_t)pc * 16));
  }
}

template <int DT>
__global__ __launch_bounds__(kLinThreads, 1) void linear_kernel(LinearParams p) {
  __shared__ __align__(1024) unsigned char buf0[kStageBytes];
  __shared__ __align__(1024) unsigned char buf1[kStageBytes];
  __shared__ __align__(1024) unsigned char buf2[kLinStages >= 3 ? kStageBytes : 16];
  __shared__ __align__(1024) unsigned char buf3[kLinStages >= 4 ? kStageBytes : 16];
  const int nt = p.n_tiles, tiles = p.m_tiles * nt;
  const int group = kLinGroupRows * nt, slots = linear_tile_slots(p.m_tiles, nt);
  const int bid = blockIdx.x;
  if (bid >= slots) {
    linear_zero_rows(p, bid - slots);
    return;
  }
  // XCD-aware order: tiles are dealt to XCDs (bid = x mod 8) in groups of
  // kLinGroupRows row blocks x all column tiles, round robin.  A group's input
  // rows then stay in one XCD's L2 while its column tiles reuse them, and the
  // live row blocks (those below the device-side row count) spread over all
  // XCDs whatever that count is.
  const int x = bid & 7, s = bid >> 3, q = s / group, o = s - q * group;
  const int t = (q * 8 + x) * group + o;
  if (t >= tiles) return;
  const int mb = t / nt, nb = t - mb * nt;
  const int M = p.m_count ? min(*p.m_count, p.M) : p.M;
  if (mb * kLinBM >= M) return;
  linear_tile<DT>(p, mb, nb, M, buf0, buf1, buf2, buf3);
}

hipError_t launch_linear(const LinearParams& p, int dtype, hipStream_t s) {
  const int zero_wgs = p.zero_mask ? (p.zero_rows + kLinZeroRows - 1) / kLinZeroRows : 0;
  const dim3 grid(linear_tile_slots(p.m_tiles, p.n_tiles) + zero_wgs);
  if (dtype == 1) hipLaunchKernelGGL((linear_kernel<1>), grid, dim3(kLinThreads), 0, s, p);
  else hipLaunchKernelGGL((linear_kernel<2>), grid, dim3(kLinThreads), 0, s, p);
  return hipGetLastError();
}

int linear_tile_rows() { return kLinBM; }
int linear_tile_cols() { return kLinBN; }

}  // namespace rva
