// Internal interface between the host API (rva_host.hip) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rva {

constexpr int kHeadDim = 64;
constexpr int kAttnThreads16 = 256; // 4 waves per attention workgroup (16-bit inputs)
constexpr int kAttnThreads32 = 512; // 8 waves per attention workgroup (fp32 inputs)
constexpr int kQBlock = 16;         // query rows per matrix-core block
constexpr int kQBlocksPerWave = 2;  // query blocks a wave carries through one pass
constexpr int kKeyTile = 32;        // keys per inner step
constexpr int kPackThreads = 256;
constexpr int kScanThreads = 1024;

// 16-bit sequences of up to rc rows are staged whole (K and V of one head
// in one round trip, rows of 64 halves with 16-byte pieces XOR-swizzled by
// row); rc is capped by the registers' query blocks (4 per wave, 4 waves)
// and by the LDS that keeps 3 workgroups per CU.  fp32 stages no keys.
constexpr int kResidentMax16 = 256;
constexpr int kLdsPerCu = 160 * 1024;
constexpr int kAttnWgPerCu16 = 3;
// LDS is given to workgroups in 1280-byte granules (a CU's 160 KB in 128
// of them): 3 workgroups fit a CU at up to 42 granules (53760 bytes) each.
constexpr int kLdsGranule = 1280;
constexpr int kLdsPerWg16 = kLdsPerCu / kAttnWgPerCu16 / kLdsGranule * kLdsGranule;
constexpr int kMaxSeq = 1024;  // longest sequence (= RVA_MAX_TOKENS)
// fp32 attention: the LDS where the waves' partial results of one 16-query
// block are combined: per wave 16 maxima, 16 sums and 16 rows of 64 floats
// (row pitch 68 floats, to spread the rows over the LDS banks).
constexpr int kCombPitch32 = 68;
constexpr int kComb32Bytes = (kAttnThreads32 / 64) * (16 + 16 + 16 * kCombPitch32) * 4;
constexpr int kItemSlotBytes = 16;  // fused 16-bit LDS past the staging area (persistent item slot)
// Key-split form (16-bit): LDS where the 4 waves' partial results of one
// 16-query block are combined (per wave 16 maxima, 16 sums, 16 rows of 64
// floats at a pitch of kCombPitch32), past the staging area.
constexpr int kComb16Bytes = (kAttnThreads16 / 64) * (16 + 16 + 16 * kCombPitch32) * 4;

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* cu;      // packed mode: offsets int32[B+1]
  const uint8_t* mask;    // fused mode: uint8[B,N]
  int32_t* cu_out;        // fused mode: optional offsets output
  int32_t* max_out;       // fused mode: optional max kept count output
  int B, N, H;
  float scale_log2e;      // softmax scale * log2(e)
  int32_t* work;          // persistent form: [next item, workgroups done], zero between launches
  int heads_per_wg;       // fused 16-bit form: heads of one image a workgroup takes in turn (>= 1)
  int rc;                 // 16-bit: longest sequence staged whole (rows, multiple of 16, >= 192); set at launch
  int tail_b;             // fused 16-bit form: last images taken one head per workgroup (0..B)
  int item_slot;          // persistent form: byte offset of its 4-byte item slot in dynamic LDS; set at launch
  int qsplit;             // query tiles per (sequence, head): one workgroup each (>= 1; 1 with head pairs)
  int nbound;             // host: longest sequence the launch is sized for (its length hint)
  int keysplit;           // 16-bit whole sequences: 1 = one query block per workgroup, its key tiles split over the waves
};

struct CopyParams {
  const void* src[3];     // pack: padded q/k/v (NULL = skip); unpack: src[0] = packed o
  void* dst[3];           // pack: packed q/k/v; unpack: dst[0] = padded o
  const uint8_t* mask;
  const int32_t* cu;
  int32_t* kept_index;    // pack only, optional
  int B, N;
  int row_bytes;          // H * d * element size (multiple of 16)
};

struct ThreshParams {
  const void* x;          // token embeddings [B, N, C]
  uint8_t* mask;          // keep-mask output [B, N]
  int N, C;
  int r0;                 // 0-based order statistic a kept patch's norm must reach
};

struct LinearParams {
  const void* x;            // input rows, K halves each
  const int32_t* x_index;   // optional: input row of product row r is x_index[r]
  int x_rows;               // rows addressable through x
  const void* w;            // weight [Nout, K]
  const void* bias;         // [Nout] or NULL
  const void* residual;     // optional, laid out like y[0] (y_split == 1 only)
  void* y[3];               // output column groups, [rows, Nout / y_split] each
  const int32_t* y_index;   // optional: output row of product row r is y_index[r]
  int y_split;              // number of column groups (1 or 3)
  const int32_t* m_count;   // optional device count of product rows (clamped to M)
  int M, K, Nout;           // M: host bound on the product rows
  int m_tiles, n_tiles;
  const uint8_t* zero_mask; // optional: rows r < zero_rows of y[0] with zero_mask[r] == 0 are zeroed
  int zero_rows;
};

__host__ __device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }


// Compaction area at the start of the fused kernel's LDS: the kept
// positions then the pruned ones, uint16[N], then one count (int32) per
// 64-token chunk.
__host__ __device__ inline int attn_chunks(int N) { return (N + 63) >> 6; }
__host__ __device__ inline size_t attn_cnt_off(int N) { return (size_t)round_up(N * 2, 16); }
__host__ __device__ inline size_t attn_compact_bytes(int N) {
  return (size_t)round_up((int)attn_cnt_off(N) + attn_chunks(N) * 4, 16);
}

inline int attn_threads(int dtype) { return dtype == 0 ? kAttnThreads32 : kAttnThreads16; }

// kv_rows: staged key rows of the 16-bit forms (rc); fp32 stages nothing but
// its combine area.
inline size_t attn_lds_bytes(int dtype, bool fused, int N, int kv_rows) {
  size_t kv = dtype == 0 ? (size_t)kComb32Bytes : (size_t)kv_rows * kHeadDim * 2 * 2;
  size_t head = fused ? attn_compact_bytes(N) : 0;
  size_t scan = (size_t)(4 * attn_threads(dtype) + 64) * 4;  // fused scan workgroup reuses LDS
  size_t total = head + kv;
  return total > scan ? total : scan;
}

// Launchers (enqueue only; return the launch status).
hipError_t launch_count_scan(const uint8_t* mask, int B, int N, int32_t* cu, int32_t* max_out,
                             hipStream_t s);
hipError_t launch_pack(const CopyParams& p, int splits, hipStream_t s);
hipError_t launch_unpack(const CopyParams& p, int splits, hipStream_t s);
hipError_t launch_attend(const AttnParams& p, int dtype, bool fused, hipStream_t s);
// Fused 16-bit path as a persistent grid of `grid` workgroups pulling
// (image, head) items from p.work.
hipError_t launch_attend_persistent(const AttnParams& p, int dtype, int grid, hipStream_t s);
int attend_persistent_per_cu(int N);  // resident workgroups per CU
// Longest sequence a 16-bit launch stages whole (rows), as launch_attend sets it.
int attend_resident_rows(int dtype, bool fused, int N);
// Grid positions of a launch's work items (without the offsets workgroup).
long long attend_grid_items(const AttnParams& p, int dtype, bool fused);
hipError_t launch_empty(hipStream_t s);
hipError_t attend_init();  // raises the dynamic-LDS limit of every attention kernel
hipError_t launch_threshold(const ThreshParams& p, int B, int dtype, hipStream_t s);
hipError_t threshold_init();  // raises the dynamic-LDS limit of the keep-mask kernels
hipError_t launch_linear(const LinearParams& p, int dtype, hipStream_t s);
int linear_tile_rows();
int linear_tile_cols();
// Ceiling probes (probe.hip).
hipError_t launch_probe_copy(const void* src, void* dst, long long pieces, int grid, hipStream_t s);
hipError_t launch_probe_read(const void* src, uint32_t* sink, long long pieces, int grid,
                             hipStream_t s);
hipError_t launch_probe_mfma(int iters, float* out, int grid, hipStream_t s);
hipError_t launch_probe_gather(const void* q, const void* k, const void* v, void* o,
                               const uint8_t* mask, const int32_t* cu, const int32_t* kidx, int B,
                               int N, int H, hipStream_t s);
long long probe_mfma_flops(int iters, int grid);

}  // namespace rva
