// Ragged bidirectional attention, packed and fused forms.
//
// What is computed follows "Dispatch-Aware Ragged Attention for Pruned Vision
// Transformers" (sota2.com page, Abstract): non-causal attention over each
// image's kept tokens only, O = softmax(Q K^T * scale) V per image and head.
//
// Work decomposition (CDNA4 / gfx950), 16-bit inputs:
//  * one workgroup of 4 waves per (image, head); on large batches the fused
//    form gives a workgroup two heads of one image, so that its mask row is
//    read and compacted once for both (the images dispatched last keep one
//    head per workgroup, so the launch ends on short workgroups).
//    Post-pruning ViT sequences are short (at most 197 tokens at 224x224,
//    577 at 384x384): a sequence of up to rc rows (208 at N = 197, the most
//    LDS that keeps 3 workgroups per CU) is staged whole, K and V of one or
//    both heads in a single memory round trip by direct-to-LDS loads, with
//    every query block's Q rows loaded alongside; longer sequences are
//    staged in chunks.  V stays row-major and the V^T operand comes from
//    the transposed LDS read;
//  * a wave takes its query blocks of 16 rows one at a time when the
//    sequence is staged whole (two at a time in the chunked form) and walks
//    the keys 32 at a time, reading the next tile's K fragments while the
//    current tile's softmax runs;
//  * scores are formed transposed, S^T = K Q^T, with the 16x16x32 matrix-core
//    product: each lane then holds one query and 4+4 keys, which is exactly
//    the per-lane slice the second product O^T = V^T P^T takes as its B
//    operand, so P never leaves registers;
//  * softmax in fp32 with exp2 (log2 e folded into the scale); row sums come
//    from the matrix cores (an all-ones operand times the rounded
//    probabilities).  A sequence staged whole runs each query block against
//    a fixed reference max, the first key tile's row max (shared by the four
//    lanes of a query with two lane-swap steps), with no rescale and no check
//    in the tile loop; the block is accepted when its row sums stay at or
//    below 2^20 and computed again against its exact max otherwise.  The
//    chunked form keeps a running max and rescales only when it grows by
//    more than 2^8.  Either reference cancels exactly in the final division;
//  * the fused form first compacts the image's keep-mask row in LDS, reads
//    Q/K/V rows straight from the padded tensors through that list, writes
//    O rows straight to padded positions and zero-fills pruned rows (for a
//    sequence staged whole, right after its staging barrier, so that those
//    stores drain during the attention rather than lengthen the wait for
//    the staging loads).  An optional extra workgroup computes cu_seqlens /
//    max_seqlen in the same launch;
//  * O rows leave 64 contiguous bytes per row and store instruction (one
//    16-lane row swap per pair of O blocks) and, like the zero rows, with
//    the non-temporal hint: both are written once and never read back;
//  * launches small enough that one workgroup per 16-query block fits one
//    fill of the device take the key-split form: each workgroup one block,
//    its four waves splitting the block's key tiles, partial results
//    combined through LDS;
//  * the persistent form runs the fused form's items (head pairs, tail
//    heads) in a loop over a device work counter, one resident grid.
// fp32 inputs use the 16x16x4 fp32 matrix-core product (no precision is
// given up) with K and V both staged in LDS and 8-wave workgroups.
#include <math.h>

#include "rva_device.h"
#include "rva_internal.h"

namespace rva {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT>
struct Half16;

template <>
struct Half16<1> {
  typedef _Float16 T;
  typedef f16x8 V8;
  typedef f16x4 V4;
  static __device__ __forceinline__ f32x4 mfma(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Half16<2> {
  typedef __bf16 T;
  typedef bf16x8 V8;
  typedef bf16x4 V4;
  static __device__ __forceinline__ f32x4 mfma(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cache-policy operand of the 16-bit path's global accesses (gfx950 buffer
// instructions: bit 1 is the non-temporal hint).  Q/K/V rows and output
// rows are each touched once per launch.
constexpr int kLoadAux = 0;   // Q loads and K/V staging loads
// Output rows (64 contiguous bytes of a row per store instruction) and the
// zero rows of pruned tokens (whole rows), written once and never read back
// by the launch: non-temporal.
constexpr int kStoreAux = 2;
constexpr int kZeroAux = 2;

// Reductions over the four lanes l, l^16, l^32, l^48 that share a query:
// a lane-swap exchanges 16-lane (resp. 32-lane) rows between two copies of
// the value, after which the elementwise max/sum of the copies is the
// reduction over the pair of rows.
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float quad_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float max8(f32x4 a, f32x4 b) {
  return fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])), fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3])));
}

constexpr float kRescaleSlack = 8.0f;  // log2 units: probabilities stay <= 2^8

// Online-softmax update for one 16-query block and one 32-key tile whose
// scores are s0 (keys 4g..4g+3) and s1 (keys 16+4g..16+4g+3) in this lane:
// writes the (unnormalised) probabilities to pr[8] and rescales the
// accumulators only when some query's max grew by more than kRescaleSlack.
// The row sums are a fifth accumulator block o[4] (computed by the matrix
// cores from an all-ones operand), so only the max is tracked here; a
// rescale multiplies all five blocks.
__device__ __forceinline__ void softmax_step16(f32x4& s0, f32x4& s1, int kvalid, float c, float& m,
                                               f32x4 (&o)[5], float (&pr)[8]) {
  const int g = lane_id() >> 4;
  if (kvalid < kKeyTile) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (4 * g + j >= kvalid) s0[j] = -INFINITY;
      if (16 + 4 * g + j >= kvalid) s1[j] = -INFINITY;
    }
  }
  const float mt = quad_max(max8(s0, s1)) * c;
  if (__any(mt > m + kRescaleSlack)) {
    const float mnew = fmaxf(m, mt);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
#pragma unroll
    for (int db = 0; db < 5; ++db) o[db] *= alpha;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pr[j] = fast_exp2(fmaf(s0[j], c, -m));
    pr[4 + j] = fast_exp2(fmaf(s1[j], c, -m));
  }
}

// ---------------------------------------------------------------- 16-bit

// Staged K and V are row-major [rows][64] halves (128-byte rows) with the
// eight 16-byte pieces of row r stored at slot p ^ (r & 7): the rows one
// fragment read touches then spread over the banks without padding.
__device__ __forceinline__ int kvswz(int row, int piece) { return row * 128 + ((piece ^ (row & 7)) << 4); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 LdsS16x4;

// K fragments of the 32-key tile at k0: lane (r16, g) holds
// K[k0 + 16 kb + r16][32 ks + 8 g .. + 7] (A operand of S^T = K Q^T).
template <int DT>
__device__ __forceinline__ void k_frag16(const unsigned char* __restrict__ Ks, int k0,
                                         typename Half16<DT>::V8 (&kf)[2][2]) {
  typedef typename Half16<DT>::V8 V8;
  const int lane = lane_id(), g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      kf[kb][ks] = *reinterpret_cast<const V8*>(Ks + kvswz(k0 + kb * 16 + r16, ks * 4 + g));
}

// V fragments of the tile at k0 (A operand of O^T = V^T P^T): lane (r16, g)
// holds V[key][16 db + r16] for keys k0 + 4g + j and k0 + 16 + 4g + j
// (j < 4), the keys whose probabilities this lane's column of P^T carries.
// The transposed LDS read hands lane i of a 16-lane group element i % 4 of
// the 8-byte pieces addressed by the group's lanes 4k + i / 4 (k < 4), so
// lane s addresses key row k0 + 4g + s / 4 at dims 16 db + 4 (s % 4) .. + 3.
template <int DT>
__device__ __forceinline__ void v_frag16(const unsigned char* __restrict__ Vs, int k0,
                                         typename Half16<DT>::V8 (&vf)[4]) {
  typedef typename Half16<DT>::V4 V4;
  const int lane = lane_id(), g = lane >> 4, r16 = lane & 15;
  const int trow = k0 + 4 * g + (r16 >> 2), tcol = r16 & 3;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int piece = 2 * db + (tcol >> 1), half = (tcol & 1) << 3;
    const V4 lo = __builtin_bit_cast(V4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LdsS16x4*)(Vs + kvswz(trow, piece) + half)));
    const V4 hi = __builtin_bit_cast(V4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LdsS16x4*)(Vs + kvswz(trow + 16, piece) + half)));
    vf[db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// The per-lane parts of the fragment addresses of a tile.  Tiles start at
// multiples of 32 rows, so a row's swizzle (row & 7) does not depend on the
// tile, and fragment reads of the tile at k0 are (staging base + 128 k0)
// plus these offsets plus constants.  Keeping them apart from the uniform
// tile base lets every query block of a wave share one set of offsets.
struct FragLanes16 {
  uint32_t k[2];  // K: row r16, piece 4 ks + g
  uint32_t v[4];  // V^T: row 4 g + r16 / 4, piece 2 db + (r16 & 3) / 2, half (r16 & 1)
};

__device__ __forceinline__ FragLanes16 frag_lanes16(int lane = lane_id()) {
  const int g = lane >> 4, r16 = lane & 15;
  FragLanes16 L;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) L.k[ks] = (uint32_t)kvswz(r16, ks * 4 + g);
  const int trow = 4 * g + (r16 >> 2), tcol = r16 & 3;
#pragma unroll
  for (int db = 0; db < 4; ++db)
    L.v[db] = (uint32_t)(kvswz(trow, 2 * db + (tcol >> 1)) + ((tcol & 1) << 3));
  return L;
}

// k_frag16 / v_frag16 through precomputed lane offsets; `tile` is the
// tile's first row in the staging area (K or V) and goes through a
// first-lane read so that it stays a uniform scalar added to fixed lane
// offsets, rather than being folded into per-lane induction variables.
template <int DT>
__device__ __forceinline__ void k_frag16(const unsigned char* __restrict__ Ks, int tile,
                                         const FragLanes16& L, typename Half16<DT>::V8 (&kf)[2][2]) {
  typedef typename Half16<DT>::V8 V8;
  const unsigned char* base = Ks + __builtin_amdgcn_readfirstlane(tile * kHeadDim * 2);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      kf[kb][ks] = *reinterpret_cast<const V8*>(base + L.k[ks] + kb * 16 * kHeadDim * 2);
}

// `upper` = the tile's keys 16..31 are staged; otherwise their V operand is
// zero (their probabilities are zero too) and nothing past the staged rows
// is read.
template <int DT>
__device__ __forceinline__ void v_frag16(const unsigned char* __restrict__ Vs, int tile,
                                         const FragLanes16& L, bool upper,
                                         typename Half16<DT>::V8 (&vf)[4]) {
  typedef typename Half16<DT>::V4 V4;
  const unsigned char* base = Vs + __builtin_amdgcn_readfirstlane(tile * kHeadDim * 2);
  V4 hi[4];
  if (upper) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
      hi[db] = __builtin_bit_cast(V4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LdsS16x4*)(base + L.v[db] + 16 * kHeadDim * 2)));
  } else {
#pragma unroll
    for (int db = 0; db < 4; ++db) hi[db] = V4{};
  }
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const V4 lo = __builtin_bit_cast(V4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LdsS16x4*)(base + L.v[db])));
    vf[db] = __builtin_shufflevector(lo, hi[db], 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// LDS fragments of one 32-key tile, shared by every query block that a wave
// runs against that tile.
template <int DT>
struct KVFrag16 {
  typename Half16<DT>::V8 kf[2][2];
  typename Half16<DT>::V8 vf[4];
};

template <int DT>
__device__ __forceinline__ KVFrag16<DT> kv_frag16(const unsigned char* __restrict__ Ks,
                                                  const unsigned char* __restrict__ Vs, int k0) {
  KVFrag16<DT> f;
  k_frag16<DT>(Ks, k0, f.kf);
  v_frag16<DT>(Vs, k0, f.vf);
  return f;
}

// Scores of one 16-query block against one 32-key tile, transposed:
// s0 = keys 4g..4g+3, s1 = keys 16+4g..16+4g+3 of this lane's query.  qf is
// the B operand: lane (r16, g) holds Q[q][32 ks + 8 g .. + 7].
template <int DT>
__device__ __forceinline__ void scores16(const typename Half16<DT>::V8 (&kf)[2][2],
                                         const typename Half16<DT>::V8 (&qf)[2], f32x4& s0,
                                         f32x4& s1) {
  typedef Half16<DT> Tr;
  s0 = f32x4{0.f, 0.f, 0.f, 0.f};
  s1 = f32x4{0.f, 0.f, 0.f, 0.f};
  s0 = Tr::mfma(kf[0][0], qf[0], s0);
  s1 = Tr::mfma(kf[1][0], qf[0], s1);
  s0 = Tr::mfma(kf[0][1], qf[1], s0);
  s1 = Tr::mfma(kf[1][1], qf[1], s1);
}

// Online softmax of the tile's scores and the accumulation of O^T (o[0..3])
// and of the probability row sums (o[4]).
template <int DT>
__device__ __forceinline__ void prob_step16(const typename Half16<DT>::V8 (&vf)[4], f32x4& s0,
                                            f32x4& s1, f32x4 (&o)[5], float& m, int kvalid,
                                            float c) {
  typedef Half16<DT> Tr;
  typedef typename Tr::T T;
  typedef typename Tr::V8 V8;
  float pr[8];
  softmax_step16(s0, s1, kvalid, c, m, o, pr);
  V8 pf;
#pragma unroll
  for (int j = 0; j < 8; ++j) pf[j] = (T)pr[j];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = Tr::mfma(vf[db], pf, o[db]);
  // row sums of the rounded probabilities: every row of an all-ones A
  // operand yields sum_k P[q][k], so each lane ends up holding its query's sum
  V8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (T)1.0f;
  o[4] = Tr::mfma(ones, pf, o[4]);
}

// One 16-query block against one 32-key tile.
template <int DT>
__device__ __forceinline__ void block_step16(const KVFrag16<DT>& f,
                                             const typename Half16<DT>::V8 (&qf)[2], f32x4 (&o)[5],
                                             float& m, int kvalid, float c) {
  f32x4 s0, s1;
  scores16<DT>(f.kf, qf, s0, s1);
  prob_step16<DT>(f.vf, s0, s1, o, m, kvalid, c);
}

// Scores of keys >= kvalid (only a sequence's last tile has any) to -inf.
__device__ __forceinline__ void mask_keys(f32x4& s0, f32x4& s1, int kvalid) {
  if (kvalid >= kKeyTile) return;
  const int g = lane_id() >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (4 * g + j >= kvalid) s0[j] = -INFINITY;
    if (16 + 4 * g + j >= kvalid) s1[j] = -INFINITY;
  }
}

// Largest probability row sum the whole-sequence form's fixed reference max
// accepts for a query block.  Probabilities are non-negative, so every one
// of them is then at most 2^20 as well; an fp16 probability that overflowed
// (2^16 and above round to infinity) makes the sum infinite and fails the
// test, so every accepted fp16 probability is finite.
constexpr float kRefSumLimit = 1048576.0f;  // 2^20

// Probabilities of one tile against a fixed reference max m (scaled by c,
// shared by the four lanes of a query): p = exp2(s c - m), rounded to the
// 16-bit type, accumulated into O^T (o[0..3]) and into the row sums (o[4],
// from an all-ones operand).  FIRST starts the accumulators from zero.
template <int DT, bool FIRST>
__device__ __forceinline__ void fixed_step16(const typename Half16<DT>::V8 (&vf)[4],
                                             const f32x4& s0, const f32x4& s1, f32x4 (&o)[5],
                                             float m, float c) {
  typedef Half16<DT> Tr;
  typedef typename Tr::T T;
  typedef typename Tr::V8 V8;
  V8 pf;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pf[j] = (T)fast_exp2(fmaf(s0[j], c, -m));
    pf[4 + j] = (T)fast_exp2(fmaf(s1[j], c, -m));
  }
  V8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (T)1.0f;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = Tr::mfma(vf[db], pf, FIRST ? z : o[db]);
  o[4] = Tr::mfma(ones, pf, FIRST ? z : o[4]);
}

// Normalise one finished query block and store its rows: O^T block db,
// lane (r16, g) holds O[q][16 db + 4 g .. + 3]; o[4] holds the query's
// probability sum in every element.  Rows at kOOB are dropped.
// Before the stores, one 16-lane row swap per pair of blocks (2 e, 2 e + 1)
// trades lane-row parity g & 1 for the block parity: afterwards lane
// (r16, g) holds O[q][32 e + 16 (g & 1) + 8 (g >> 1) .. + 7] in the pair,
// so each store instruction writes 64 contiguous bytes of every row (two
// per row in all) instead of 32.
template <int DT>
__device__ __forceinline__ void store_block16(const f32x4 (&o)[5], Rsrc ro, uint32_t qoff) {
  typedef Half16<DT> Tr;
  typedef typename Tr::T T;
  typedef typename Tr::V4 V4;
  const int g = lane_id() >> 4;
  // hardware reciprocal (about 1 ulp): ample for 16-bit outputs
  const float inv = __builtin_amdgcn_rcpf(o[4][0]);
  u32x2 out[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    V4 x;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (T)(o[db][j] * inv);
    out[db] = __builtin_bit_cast(u32x2, x);
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      // odd rows of the first operand trade places with even rows of the second
      const auto sw = __builtin_amdgcn_permlane16_swap(out[2 * e][w], out[2 * e + 1][w], false, false);
      out[2 * e][w] = sw[0];
      out[2 * e + 1][w] = sw[1];
    }
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{out[2 * e][0], out[2 * e][1], out[2 * e + 1][0],
                                                 out[2 * e + 1][1]},
                                           ro, (int)(qoff + 64 * e + 32 * (g & 1) + 16 * (g >> 1)), 0,
                                           kStoreAux);
  }
}

// One 16-query block against one 32-key tile of the streamed form, with the
// fixed reference max: `first` (the pass's first tile) sets m to the tile's
// row max, later tiles use m as it is.
template <int DT>
__device__ __forceinline__ void stream_step16(const KVFrag16<DT>& f,
                                              const typename Half16<DT>::V8 (&qf)[2],
                                              f32x4 (&o)[5], float& m, int kvalid, float c,
                                              bool first) {
  f32x4 s0, s1;
  scores16<DT>(f.kf, qf, s0, s1);
  mask_keys(s0, s1, kvalid);
  if (first) {
    m = quad_max(max8(s0, s1)) * c;
    fixed_step16<DT, true>(f.vf, s0, s1, o, m, c);
  } else {
    fixed_step16<DT, false>(f.vf, s0, s1, o, m, c);
  }
}

// Exact fallback of the streamed form for a query block whose probabilities
// against the fixed reference max left range (rare: some later key scores
// far above every key of the block's first tile): the block computed again
// from scratch with a running max and rescaling, reading K and V straight
// from memory, so it needs nothing from the workgroup's other waves.  Rows
// at or past n read as zeros; qf is the block's Q operand, qoff the byte
// offset of its output row (kOOB past n).
template <int DT, typename RowOff>
__device__ __forceinline__ void block_exact16(Rsrc rk, Rsrc rv, Rsrc ro, int n,
                                                        RowOff roff, float c,
                                                        typename Half16<DT>::V8 q0,
                                                        typename Half16<DT>::V8 q1,
                                                        uint32_t qoff) {
  typedef Half16<DT> Tr;
  typedef typename Tr::V8 V8;
  typedef typename Tr::T T;
  const int lane = lane_id(), g = lane >> 4, r16 = lane & 15;
  const V8 qf[2] = {q0, q1};
  f32x4 o[5];
#pragma unroll
  for (int db = 0; db < 5; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  for (int k0 = 0; k0 < n; k0 += kKeyTile) {
    V8 kf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = k0 + kb * 16 + r16;
      const uint32_t base = row < n ? roff(row) : kOOB;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        kf[kb][ks] = __builtin_bit_cast(
            V8, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(base + 64 * ks + 16 * g), 0, 0));
    }
    // V^T operand: lane (r16, g) element j is V[key][16 db + r16] with key
    // 4 g + j (j < 4) or 16 + 4 g + j - 4 (j >= 4) of the tile
    V8 vf[4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = k0 + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
      const uint32_t base = key < n ? roff(key) : kOOB;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        vf[db][j] = __builtin_bit_cast(
            T, __builtin_amdgcn_raw_buffer_load_b16(rv, (int)(base + 2 * (16 * db + r16)), 0, 0));
    }
    f32x4 s0, s1;
    scores16<DT>(kf, qf, s0, s1);
    prob_step16<DT>(vf, s0, s1, o, m, min(kKeyTile, n - k0), c);
  }
  store_block16<DT>(o, ro, qoff);
}

// Global accesses of the 16-bit path go through raw buffer descriptors
// (make_rsrc) whose base is the sequence's head slice and whose size covers
// exactly its rows, so ragged tails need no branches.

// Stage keys [c0, c0 + rows) of the sequence: K and V rows into Ks / Vs by
// direct-to-LDS buffer loads (no registers, no LDS stores by the waves).
// One load instruction fills 8 rows (1 KB), lane L landing at byte 16 L,
// i.e. row L / 8, slot L % 8; the lane fetches the 16-byte piece that the
// row swizzle puts in that slot.  Every row offset is read (through roff)
// before the first load is issued, so no load waits behind another's LDS
// write.  Keys in [rows, round_up(rows, pad)) are out of range and land as
// zeros, so masked probabilities (exact zeros) never meet stale LDS
// contents.  The caller's barrier (with its memory fence) makes the chunk
// visible.  `roff(r)` is the byte offset of sequence row r; MAXROWS bounds
// round_up(rows, pad).
template <int DT, int MAXROWS, typename RowOff>
__device__ __forceinline__ void stage16(Rsrc rk, Rsrc rv, unsigned char* Ks, unsigned char* Vs,
                                        int c0, int rows, int pad, RowOff roff) {
  constexpr int kWaves = kAttnThreads16 / 64;
  constexpr int NI = MAXROWS / 8 / kWaves;  // 8-row loads per wave, at most
  static_assert(MAXROWS % (8 * kWaves) == 0, "whole loads");
  const int lane = lane_id(), w = wave_id();
  const int rpad = round_up(rows, pad);
  const int rl = lane >> 3;                 // row within the load (row & 7 == rl)
  const uint32_t piece16 = (uint32_t)(((lane & 7) ^ rl) << 4);
  uint32_t off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = 8 * (w + kWaves * i) + rl;
    off[i] = r < rows ? roff(c0 + r) + piece16 : kOOB;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r0 = 8 * (w + kWaves * i);
    if (r0 >= rpad) break;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(Ks + r0 * 128),
                                             16, off[i], 0, 0, kLoadAux);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(Vs + r0 * 128),
                                             16, off[i], 0, 0, kLoadAux);
  }
}

// Wait until at most N vector memory operations of this wave are in flight
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left open).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}


// Streamed form (sequences longer than the whole-sequence staging): keys go
// through two LDS buffers of kChunk16 rows, and the next chunk's loads are
// in flight while the current chunk is multiplied.  Every chunk is fetched
// with the same number of loads per wave (rows past the chunk's end are
// out-of-range offsets, which land as zeros), so the wait for a chunk is a
// fixed count of this wave's loads; the last step waits for everything, so
// no load into LDS is left in flight when the sequence is done.
constexpr int kChunk16 = 96;
constexpr int kChunkLoads16 = kChunk16 / 8 / (kAttnThreads16 / 64);  // per wave, K and V each
static_assert(kChunk16 % (8 * (kAttnThreads16 / 64)) == 0 && kChunk16 % kKeyTile == 0, "chunk shape");

// Stage keys [c0, c0 + rows) (rows <= kChunk16) into Ks / Vs as stage16
// does: 2 kChunkLoads16 direct-to-LDS loads per wave, always.
template <typename RowOff>
__device__ __forceinline__ void stage_chunk16(Rsrc rk, Rsrc rv, unsigned char* Ks,
                                              unsigned char* Vs, int c0, int rows, RowOff roff) {
  constexpr int kWaves = kAttnThreads16 / 64;
  const int lane = lane_id(), w = wave_id();
  const int rl = lane >> 3;
  const uint32_t piece16 = (uint32_t)(((lane & 7) ^ rl) << 4);
  uint32_t off[kChunkLoads16];
#pragma unroll
  for (int i = 0; i < kChunkLoads16; ++i) {
    const int r = 8 * (w + kWaves * i) + rl;
    off[i] = r < rows ? roff(c0 + r) + piece16 : kOOB;
  }
#pragma unroll
  for (int i = 0; i < kChunkLoads16; ++i) {
    const int r0 = 8 * (w + kWaves * i);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(Ks + r0 * 128),
                                             16, off[i], 0, 0, kLoadAux);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(Vs + r0 * 128),
                                             16, off[i], 0, 0, kLoadAux);
  }
}

// One sequence (image or packed run), one head, streamed.  rq/rk/rv/ro
// cover the sequence's head slice; roff(r) is the byte offset of its row r.
// Each wave carries two 16-query blocks through a pass over every key
// chunk; the workgroup takes the query blocks qt, qt + qs, qt + 2 qs, ...
// of the sequence (all of them when qs = 1).  Steps (pass, chunk) run as
// one sequence: step s computes on buffer s & 1 while step s + 1's chunk
// lands in the other.  `last_use()` is called by every thread once, after
// the kept-row list (through roff) has been read for the last time.
template <int DT, typename RowOff, typename Hook>
__device__ __forceinline__ void attend_seq16(const AttnParams& p, int n, unsigned char* kvbase,
                                             Rsrc rq, Rsrc rk, Rsrc rv, Rsrc ro, RowOff roff,
                                             Hook last_use, int qt = 0, int qs = 1) {
  typedef Half16<DT> Tr;
  typedef typename Tr::V8 V8;
  const int lane = lane_id(), w = wave_id(), g = lane >> 4, r16 = lane & 15;
  constexpr int kBuf = kChunk16 * kHeadDim * 2;  // bytes of K (or V) in one buffer
  constexpr int kWaves = kAttnThreads16 / 64;
  constexpr int kPerPass = kWaves * kQBlocksPerWave;
  const int nqb = (n + kQBlock - 1) / kQBlock;
  const int nqt = qt < nqb ? (nqb - qt + qs - 1) / qs : 0;  // this workgroup's blocks
  const int npass = (nqt + kPerPass - 1) / kPerPass;
  const int nchunk = (n + kChunk16 - 1) / kChunk16;
  const int nsteps = npass * nchunk;
  const float c = p.scale_log2e;
  if (nsteps == 0) return;
  stage_chunk16(rk, rv, kvbase, kvbase + kBuf, 0, min(kChunk16, n), roff);
  int qb[2];
  bool act[2];
  uint32_t qoff[2];
  V8 qf[2][2];
  f32x4 o[2][5];
  float m[2];
  uint32_t redo = 0;  // blocks to compute again exactly: bit 2 pass + i (at most 8 passes)
  for (int s = 0; s < nsteps; ++s) {
    const int pass = s / nchunk, cc = s - pass * nchunk;
    if (cc == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        qb[i] = pass * kPerPass + w + i * kWaves;
        act[i] = qb[i] < nqt;
        const int q = (qt + qs * qb[i]) * kQBlock + r16;
        qoff[i] = (act[i] && q < n) ? roff(q) : kOOB;
        // B operand of S^T = K Q^T: lane (r16, g) holds Q[q][32 ks + 8 g .. + 7]
        qf[i][0] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(qoff[i] + 16 * g), 0, kLoadAux));
        qf[i][1] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(qoff[i] + 64 + 16 * g), 0, kLoadAux));
        m[i] = -INFINITY;
#pragma unroll
        for (int db = 0; db < 5; ++db) o[i][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // the buffer of step s + 1 was read in step s - 1: every wave is past it
    if (s > 0) lds_barrier();
    if (s + 1 < nsteps) {
      const int c1 = ((s + 1) % nchunk) * kChunk16;
      unsigned char* b = kvbase + ((s + 1) & 1) * 2 * kBuf;
      stage_chunk16(rk, rv, b, b + kBuf, c1, min(kChunk16, n - c1), roff);
      // this wave's loads up to step s are done, step s + 1's still in flight
      wait_vm<2 * kChunkLoads16>();
    } else {
      last_use();
      wait_vm<0>();  // nothing of this wave is left in flight into LDS
    }
    lds_barrier();  // every wave's loads of step s have landed
    const unsigned char* Ks = kvbase + (s & 1) * 2 * kBuf;
    const unsigned char* Vs = Ks + kBuf;
    const int rows = min(kChunk16, n - cc * kChunk16);
    if (act[0]) {
      // softmax against a fixed reference max per query block: the pass's
      // first tile sets it to that tile's row max, later tiles use it as it
      // is, with no running max and no rescale (as the whole-sequence form)
      const int ntile = (rows + kKeyTile - 1) / kKeyTile;
      for (int t = 0; t < ntile; ++t) {
        const int k0 = t * kKeyTile;
        const int kvalid = min(kKeyTile, rows - k0);
        const KVFrag16<DT> f = kv_frag16<DT>(Ks, Vs, k0);
        // two calls, not an unrolled loop over the blocks with an early
        // exit: written that way, the second block's reference max came out
        // wrong with this toolchain (every pass, both forms, GPU tests)
        const bool first = cc == 0 && t == 0;
        stream_step16<DT>(f, qf[0], o[0], m[0], kvalid, c, first);
        if (act[1]) stream_step16<DT>(f, qf[1], o[1], m[1], kvalid, c, first);
      }
    }
    if (cc == nchunk - 1) {
      // rows q >= n went to kOOB; a block whose row sums left the fixed
      // reference's range is computed again exactly once the passes are
      // done (its bit 2 pass + i), when the passes' registers are free
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (!act[i]) continue;
        if (__any(!(o[i][4][0] <= kRefSumLimit)))
          redo |= 1u << (2 * pass + i);
        else
          store_block16<DT>(o[i], ro, qoff[i]);
      }
    }
  }
  while (redo) {
    const int bit = __builtin_ctz(redo);
    redo &= redo - 1;
    const int qbl = (bit >> 1) * kPerPass + w + (bit & 1) * kWaves;
    const int q = (qt + qs * qbl) * kQBlock + r16;
    const uint32_t off = q < n ? roff(q) : kOOB;
    const V8 q0 = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(off + 16 * g), 0, 0));
    const V8 q1 = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(off + 64 + 16 * g), 0, 0));
    block_exact16<DT>(rk, rv, ro, n, roff, c, q0, q1, off);
  }
}

// Whole sequences resident in LDS (n <= rc): the K and V rows of `nh`
// heads of one sequence are staged at once, each head as round_up(n, 16)
// K rows followed by as many V rows (nh * round_up(n, 16) <= rc), each
// wave loads the Q rows of its (head, query block) units before the
// staging barrier, and then runs its units one at a time, storing each as
// soon as it is done.  One memory round trip for all nh heads, however
// many query blocks the sequence has.  Head j of the group lies j * 128
// bytes after head 0 in every token row, so one set of descriptors (over
// head 0's slice, sized to cover the group) and roff serve all of them.
// A wave has at most 4 units (rc <= 256); three Q fragments are held at
// once and the fourth unit's rows are loaded into the first unit's
// registers as soon as that unit is done.
constexpr int kUnitsPerWave = kResidentMax16 / kQBlock / (kAttnThreads16 / 64);
constexpr int kQSlots = 3;

// LANES_PER_TILE: recompute the fragment lane offsets at every tile (behind
// an opaque move, so they are not hoisted) instead of holding them across
// the tile loops; for callers whose own live state leaves no registers for
// them, where they would otherwise be spilled and reloaded every tile.
// The units are the (head, query block) pairs of the workgroup's query
// blocks qt, qt + qs, ... (qt < the sequence's block count).
template <int DT, bool LANES_PER_TILE = false, typename RowOff, typename Hook>
__device__ __forceinline__ void attend_resident16(int n, int nh, float c, unsigned char* kvbase,
                                                  Rsrc rq, Rsrc rk, Rsrc rv, Rsrc ro, RowOff roff,
                                                  Hook last_use, int qt = 0, int qs = 1) {
  typedef Half16<DT> Tr;
  typedef typename Tr::V8 V8;
  constexpr int kWaves = kAttnThreads16 / 64;
  constexpr uint32_t kHeadBytes = kHeadDim * 2;
  static_assert(kUnitsPerWave == kQSlots + 1, "one late Q load per wave");
  // n through an opaque (volatile) move: the unit arithmetic below then
  // cannot be hoisted out of a caller's loop over head groups, where it
  // would stay live across the loop and spill
  asm volatile("" : "+s"(n));
  const int lane = lane_id(), w = wave_id(), g = lane >> 4, r16 = lane & 15;
  const int rows = round_up(n, kQBlock);  // staged rows per head, K and V each
  const int nqb = rows / kQBlock;
  const int nqt = (nqb - qt + qs - 1) / qs;  // the workgroup's query blocks per head
  const int nunits = nh * nqt;
  // every kept-row offset is read before the staging barrier
  uint32_t qoff[kUnitsPerWave];
#pragma unroll
  for (int i = 0; i < kUnitsPerWave; ++i) {
    const int u = w + i * kWaves;
    const int hu = u / nqt;
    const int q = (qt + qs * (u - hu * nqt)) * kQBlock + r16;
    qoff[i] = (u < nunits && q < n) ? roff(q) + (uint32_t)hu * kHeadBytes : kOOB;
  }
  auto load_q = [&](uint32_t off, V8 (&qs)[2]) {
    // B operand of S^T = K Q^T: lane (r16, g) holds Q[q][32 ks + 8 g .. + 7]
    qs[0] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(off + 16 * g), 0, kLoadAux));
    qs[1] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(off + 64 + 16 * g), 0, kLoadAux));
  };
  V8 qf[kQSlots][2];
#pragma unroll
  for (int i = 0; i < kQSlots; ++i) load_q(qoff[i], qf[i]);
  for (int h = 0; h < nh; ++h) {
    unsigned char* Ks = kvbase + h * rows * 2 * kHeadBytes;
    const uint32_t hoff = (uint32_t)h * kHeadBytes;
    stage16<DT, kResidentMax16>(rk, rv, Ks, Ks + rows * kHeadBytes, 0, n, kQBlock,
                                [=](int r) -> uint32_t { return roff(r) + hoff; });
  }
  __syncthreads();
  last_use();
  const int ntile = (n + kKeyTile - 1) / kKeyTile;
  auto lanes_now = [&]() -> FragLanes16 {
    if constexpr (LANES_PER_TILE) {
      int l = lane_id();
      asm volatile("" : "+v"(l));
      return frag_lanes16(l);
    } else {
      return frag_lanes16();
    }
  };
  const FragLanes16 lanes0 = frag_lanes16();
#pragma unroll
  for (int i = 0; i < kUnitsPerWave; ++i) {
    const int u = w + i * kWaves;
    if (u >= nunits) break;
    const int slot = i % kQSlots;
    if (i == 1 && w + kQSlots * kWaves < nunits) load_q(qoff[kQSlots], qf[0]);
    const int hu = u / nqt;
    const unsigned char* Ks = kvbase + hu * rows * 2 * kHeadBytes;
    const unsigned char* Vs = Ks + rows * kHeadBytes;
    // The block's softmax runs against a fixed reference max: the first
    // tile sets it to that tile's row max, and later tiles use it as it is.
    // The tile loop then carries no rescale of the accumulators (whose
    // branch would cost register copies every tile) and no per-tile check:
    // once the block is done, its probability row sums (o[4], from the
    // matrix cores) must stay at or below kRefSumLimit.  A block that fails,
    // some later score far above the first tile's, is computed again from
    // scratch against its exact row max (rare).
    // Every tile loop reads the next tile's K fragments right after the
    // current tile's score products issue.  Every read stays inside the
    // head's staged rows: a last tile with 16 staged rows reads its K rows
    // 16..31 from the head's first V rows (their scores are masked) and
    // skips their V rows.
    f32x4 o[5];
    V8 kf[2][2];
    float m;
    {
      const FragLanes16 lanes = LANES_PER_TILE ? lanes_now() : lanes0;
      k_frag16<DT>(Ks, 0, lanes, kf);
      V8 vf[4];
      v_frag16<DT>(Vs, 0, lanes, kQBlock < rows, vf);
      f32x4 s0, s1;
      scores16<DT>(kf, qf[slot], s0, s1);
      if (ntile > 1) k_frag16<DT>(Ks, kKeyTile, lanes, kf);
      mask_keys(s0, s1, n);
      m = quad_max(max8(s0, s1)) * c;
      fixed_step16<DT, true>(vf, s0, s1, o, m, c);
    }
    // unrolled over the at most kResidentMax16 / kKeyTile tiles, so that a
    // tile's offset in the staging area is a constant of the LDS reads
#pragma unroll
    for (int t = 1; t < kResidentMax16 / kKeyTile; ++t) {
      if (t >= ntile) break;
      const int k0 = t * kKeyTile;
      const FragLanes16 lanes = LANES_PER_TILE ? lanes_now() : lanes0;
      V8 vf[4];
      v_frag16<DT>(Vs, k0, lanes, k0 + kQBlock < rows, vf);
      f32x4 s0, s1;
      scores16<DT>(kf, qf[slot], s0, s1);
      if (t + 1 < ntile) k_frag16<DT>(Ks, k0 + kKeyTile, lanes, kf);
      mask_keys(s0, s1, n - k0);
      fixed_step16<DT, false>(vf, s0, s1, o, m, c);
    }
    if (__any(!(o[4][0] <= kRefSumLimit))) {
      float mx = -INFINITY;
      k_frag16<DT>(Ks, 0, LANES_PER_TILE ? lanes_now() : lanes0, kf);
      for (int t = 0; t < ntile; ++t) {
        const FragLanes16 lanes = LANES_PER_TILE ? lanes_now() : lanes0;
        f32x4 s0, s1;
        scores16<DT>(kf, qf[slot], s0, s1);
        if (t + 1 < ntile) k_frag16<DT>(Ks, (t + 1) * kKeyTile, lanes, kf);
        mask_keys(s0, s1, n - t * kKeyTile);
        mx = fmaxf(mx, max8(s0, s1));
      }
      m = quad_max(mx) * c;
      k_frag16<DT>(Ks, 0, LANES_PER_TILE ? lanes_now() : lanes0, kf);
      for (int t = 0; t < ntile; ++t) {
        const int k0 = t * kKeyTile;
        const FragLanes16 lanes = LANES_PER_TILE ? lanes_now() : lanes0;
        V8 vf[4];
        v_frag16<DT>(Vs, k0, lanes, k0 + kQBlock < rows, vf);
        f32x4 s0, s1;
        scores16<DT>(kf, qf[slot], s0, s1);
        if (t + 1 < ntile) k_frag16<DT>(Ks, k0 + kKeyTile, lanes, kf);
        mask_keys(s0, s1, n - k0);
        if (t == 0)
          fixed_step16<DT, true>(vf, s0, s1, o, m, c);
        else
          fixed_step16<DT, false>(vf, s0, s1, o, m, c);
      }
    }
    store_block16<DT>(o, ro, qoff[i]);
  }
}

// Key-split form of a whole sequence (launches whose one-block-per-workgroup
// grid still fits one slot-fill, so that the workgroup's chain, not its
// share of the device, sets the time): the workgroup stages the sequence's
// K and V as the whole-sequence form does and takes the 16-query blocks qt,
// qt + qs, ... (one, when the launch's length bound holds), and its four
// waves split each block's 32-key tiles (wave w: tiles w, w + 4, ...)
// instead of each walking every tile of blocks of its own.  Each wave keeps
// a running max (rescaling at each of its tiles), its probability row sums
// and a partial O; the partials are combined through LDS (`comb`,
// kComb16Bytes).  A wave may have no tile: it then holds m = -inf, l = 0 and
// O = 0, and weighs nothing in the combine.
template <int DT, typename RowOff, typename Hook>
__device__ __forceinline__ void attend_block_split16(int n, float c, unsigned char* kvbase, Rsrc rq,
                                                     Rsrc rk, Rsrc rv, Rsrc ro, RowOff roff,
                                                     Hook last_use, int qt, int qs,
                                                     unsigned char* comb) {
  typedef Half16<DT> Tr;
  typedef typename Tr::T T;
  typedef typename Tr::V4 V4;
  typedef typename Tr::V8 V8;
  constexpr int kWaves = kAttnThreads16 / 64;
  constexpr uint32_t kHeadBytes = kHeadDim * 2;
  const int lane = lane_id(), w = wave_id(), g = lane >> 4, r16 = lane & 15;
  const int rows = round_up(n, kQBlock);
  const int nqb = rows / kQBlock;
  auto load_q = [&](int qb, V8 (&qf)[2]) {
    const int q = qb * kQBlock + r16;
    const uint32_t off = q < n ? roff(q) : kOOB;
    qf[0] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(off + 16 * g), 0, kLoadAux));
    qf[1] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(off + 64 + 16 * g), 0, kLoadAux));
  };
  V8 qf[2];
  load_q(qt, qf);
  unsigned char* Ks = kvbase;
  unsigned char* Vs = kvbase + rows * kHeadBytes;
  stage16<DT, kResidentMax16>(rk, rv, Ks, Vs, 0, n, kQBlock, roff);
  __syncthreads();
  last_use();
  const int ntile = (n + kKeyTile - 1) / kKeyTile;
  const FragLanes16 lanes = frag_lanes16();
  // the output thread's row within a block (16 threads per row)
  const int qq = (int)threadIdx.x >> 4, d0 = 4 * ((int)threadIdx.x & 15);
  float* cm = reinterpret_cast<float*>(comb);  // [W][16] maxima
  float* cl = cm + kWaves * 16;                 // [W][16] row sums
  float* co = cl + kWaves * 16;                 // [W][16][kCombPitch32] partial O
  for (int qb = qt; qb < nqb; qb += qs) {
    if (qb > qt) {
      load_q(qb, qf);
      __syncthreads();  // the previous block's combine has read the partials
    }
    V8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (T)1.0f;
    f32x4 o[5];
#pragma unroll
    for (int db = 0; db < 5; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
    for (int t = w; t < ntile; t += kWaves) {
      const int k0 = t * kKeyTile;
      V8 kf[2][2], vf[4];
      k_frag16<DT>(Ks, k0, lanes, kf);
      v_frag16<DT>(Vs, k0, lanes, k0 + kQBlock < rows, vf);
      f32x4 s0, s1;
      scores16<DT>(kf, qf, s0, s1);
      mask_keys(s0, s1, n - k0);
      // the tile's first key is valid, so its row max, and m, are finite
      const float mn = fmaxf(m, quad_max(max8(s0, s1)) * c);
      const float alpha = fast_exp2(m - mn);  // 0 at the wave's first tile
      m = mn;
#pragma unroll
      for (int db = 0; db < 5; ++db) o[db] *= alpha;
      V8 pf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[e] = (T)fast_exp2(fmaf(s0[e], c, -m));
        pf[4 + e] = (T)fast_exp2(fmaf(s1[e], c, -m));
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = Tr::mfma(vf[db], pf, o[db]);
      o[4] = Tr::mfma(ones, pf, o[4]);
    }
    if (g == 0) {
      cm[w * 16 + r16] = m;
      cl[w * 16 + r16] = o[4][0];
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
      *reinterpret_cast<f32x4*>(co + (w * 16 + r16) * kCombPitch32 + 16 * db + 4 * g) = o[db];
    __syncthreads();
    const int orow = qb * kQBlock + qq;
    if (orow < n) {
      float M = -INFINITY;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) M = fmaxf(M, cm[i * 16 + qq]);
      float den = 0.f;
      f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        const float mi = cm[i * 16 + qq];
        const float a = mi == -INFINITY ? 0.f : fast_exp2(mi - M);
        den = fmaf(a, cl[i * 16 + qq], den);
        const f32x4 part = *reinterpret_cast<const f32x4*>(co + (i * 16 + qq) * kCombPitch32 + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) num[e] = fmaf(a, part[e], num[e]);
      }
      // hardware reciprocal (about 1 ulp): ample for 16-bit outputs
      const float inv = __builtin_amdgcn_rcpf(den);
      V4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = (T)(num[e] * inv);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, out), ro,
                                            (int)(roff(orow) + 2 * d0), 0, kStoreAux);
    }
  }
}

// ---------------------------------------------------------------- fp32

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max4(f32x4 a) { return fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])); }

// fp32 inputs: one workgroup per (sequence, head, query tile), the tile's
// 16-query blocks taken one at a time.  For one block, the workgroup's
// waves split the keys 16 at a time (wave w: keys 16 w, 16 (w + W), ...),
// each keeping its own running max, row sum and partial O, which are
// combined through LDS once every key is seen.  At these lengths one
// block's keys then take at most a few 16-key steps per wave, so a block
// costs little more than its memory round trips; the fp32 matrix-core rate
// (a quarter of the 16-bit one per cycle and operand) would otherwise make
// a whole sequence per workgroup a long serial chain.
//
// Products, 16x16x4 fp32 matrix cores, scores transposed (S^T = K Q^T):
// step t contracts head dims 16 g + t for lane group g, so lane (r16, g)
// holds K[key r16][16 g .. 16 g + 15] and Q[query r16][16 g .. + 15] as four
// 16-byte pieces each, and ends with S[query r16][keys 4 g .. 4 g + 3].  For
// O^T = V^T P^T, step j contracts keys 4 g + j: lane (r16, g) gives
// V[key 4 g + j][16 db + r16] (one float per lane, 64 contiguous bytes per
// 16 lanes) and its own probability P[r16][4 g + j], and ends with
// O[query r16][16 db + 4 g .. + 3].  K, V and Q come straight from memory
// through buffer descriptors (rows at or past n read as zeros); nothing is
// staged in LDS but the combine.
constexpr int kSlice32 = 16;  // keys per wave step
constexpr int kWaves32 = kAttnThreads32 / 64;

// One 16-query block (rows 16 qb .. 16 qb + 15 of the sequence).  roff(r) is
// the byte offset of sequence row r from the descriptors' base.  Two
// workgroup barriers; every thread must call it.
template <typename RowOff>
__device__ __forceinline__ void block32(Rsrc rq, Rsrc rk, Rsrc rv, Rsrc ro, int n, int qb, float c,
                                        RowOff roff, float* comb) {
  const int lane = lane_id(), w = wave_id(), g = lane >> 4, r16 = lane & 15;
  const int q = qb * kQBlock + r16;
  const uint32_t qoff = q < n ? roff(q) : kOOB;
  f32x4 qf[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4)
    qf[t4] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rq, (int)(qoff + 64 * g + 16 * t4), 0, 0));
  float m = -INFINITY, l = 0.f;
  f32x4 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = w * kSlice32; k0 < n; k0 += kWaves32 * kSlice32) {
    const int kr = k0 + r16;
    const uint32_t koff = kr < n ? roff(kr) : kOOB;
    f32x4 kf[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
      kf[t4] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rk, (int)(koff + 64 * g + 16 * t4), 0, 0));
    float va[4][4];  // [db][j]: V[k0 + 4 g + j][16 db + r16]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vr = k0 + 4 * g + j;
      const uint32_t voff = vr < n ? roff(vr) : kOOB;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        va[db][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  rv, (int)(voff + 4 * (16 * db + r16)), 0, 0));
    }
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 16; ++t) s = mfma_f32(kf[t >> 2][t & 3], qf[t >> 2][t & 3], s);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (k0 + 4 * g + j >= n) s[j] = -INFINITY;
    // key k0 is always valid and lies in lane group 0, so mt is finite
    const float mt = quad_max(max4(s)) * c;
    const float mn = fmaxf(m, mt);
    const float alpha = fast_exp2(m - mn);  // 0 on the first step (m = -inf)
    m = mn;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = fast_exp2(fmaf(s[j], c, -m));
      l += p[j];
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) o[db] = mfma_f32(va[db][j], p[j], o[db]);
  }
  l = quad_sum(l);
  float* cm = comb;                         // [W][16] running maxima
  float* cl = comb + kWaves32 * 16;         // [W][16] row sums
  float* co = comb + 2 * kWaves32 * 16;     // [W][16][kCombPitch32] partial O
  if (g == 0) {
    cm[w * 16 + r16] = m;
    cl[w * 16 + r16] = l;
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
    *reinterpret_cast<f32x4*>(co + (w * 16 + r16) * kCombPitch32 + 16 * db + 4 * g) = o[db];
  __syncthreads();
  // thread: query tid / 32, head dims 2 (tid % 32) and the next
  const int qq = threadIdx.x >> 5, dd = 2 * (threadIdx.x & 31);
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kWaves32; ++i) M = fmaxf(M, cm[i * 16 + qq]);
  float den = 0.f, n0 = 0.f, n1 = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves32; ++i) {
    const float mi = cm[i * 16 + qq];
    // a wave that saw no key holds m = -inf, l = 0 and O = 0
    const float a = mi == -INFINITY ? 0.f : fast_exp2(mi - M);
    const float* row = co + (i * 16 + qq) * kCombPitch32 + dd;
    den = fmaf(a, cl[i * 16 + qq], den);
    n0 = fmaf(a, row[0], n0);
    n1 = fmaf(a, row[1], n1);
  }
  const int qo = qb * kQBlock + qq;
  if (qo < n) {
    const float inv = 1.f / den;
    u32x2 out;
    out[0] = __float_as_uint(n0 * inv);
    out[1] = __float_as_uint(n1 * inv);
    __builtin_amdgcn_raw_buffer_store_b64(out, ro, (int)(roff(qo) + 4 * dd), 0, 0);
  }
  __syncthreads();  // the combine area is free for the next block
}

// ---------------------------------------------------------------- kernels

// Zero the output rows of the pruned tokens of one image for `nh`
// consecutive heads: `ro` covers the image's rows from the first head's
// slice of its first token row (rows `rs` bytes apart), `pruned` lists the
// npruned pruned positions.  The heads' slices of a row are contiguous, so
// a row is nh * 64 elements of 16-byte pieces, each thread keeping one
// piece position and walking the rows.  When `parts` workgroups share the
// image's heads, this one takes every parts-th row from row `part`.
template <int NT, int ESIZE>
__device__ __forceinline__ void zero_pruned(Rsrc ro, const uint16_t* pruned, int npruned, int nh,
                                            uint32_t rs, int part = 0, int parts = 1) {
  const int per = nh * (kHeadDim * ESIZE / 16);  // pieces per row, <= NT
  const int rows = NT / per;                     // rows per sweep of the workgroup
  const int j0 = (int)threadIdx.x / per;
  const uint32_t pc = (uint32_t)((int)threadIdx.x - j0 * per) * 16u;
  if (j0 >= rows) return;
  for (int j = j0 + part * rows; j < npruned; j += parts * rows) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, ro, (int)(pruned[j] * rs + pc), 0,
                                           kZeroAux);
  }
}

// The same parameters with q/k/v/o moved to one sequence's head slice, so
// every per-row address inside is a 32-bit offset from a uniform base (an
// image's rows span at most N * H * 64 * 4 bytes < 2^32).
__device__ __forceinline__ AttnParams rebase(const AttnParams& p, size_t elem0, int esize) {
  AttnParams r = p;
  const size_t off = elem0 * (size_t)esize;
  r.q = static_cast<const char*>(p.q) + off;
  r.k = static_cast<const char*>(p.k) + off;
  r.v = static_cast<const char*>(p.v) + off;
  r.o = static_cast<char*>(p.o) + off;
  return r;
}

// The work of grid position `bid` of the attention launch: in the fused
// form an image's head group (or one head of a tail image), in the packed
// form one (sequence, head); with query tiles (p.qsplit = S > 1, and every
// fp32 launch) one query tile of one (sequence, head).  Tiles are laid out
// so that the S tiles of item i sit at grid positions congruent to i modulo
// 8: workgroups are dealt to the 8 XCDs round robin, so all tiles of a
// sequence run on one XCD and share its K/V rows through that XCD's L2.
// `hook()` is called by every thread at least once after the item's first
// staging barrier, or after its zero fill when the image keeps no token
// (the persistent form, which never splits, hands over its next item index
// there).
// KEYSPLIT: the launch takes the key-split form for sequences staged whole
// (a kernel instance of its own, so that the other instances' registers are
// not shaped by its code).
template <int DT, bool FUSED, bool LANES_PER_TILE = false, bool KEYSPLIT = false, typename Hook>
__device__ __forceinline__ void attend_item(const AttnParams& p, int bid, unsigned char* smem,
                                            Hook hook) {
  constexpr int NT = DT == 0 ? kAttnThreads32 : kAttnThreads16;
  const int S = p.qsplit;
  int HG = (FUSED && DT != 0) ? p.heads_per_wg : 1;
  int b, hg, t = 0;
  if (DT == 0 || S > 1) {
    const int grp = bid / (8 * S), r = bid - grp * 8 * S;
    t = r >> 3;
    const int i = grp * 8 + (r & 7);
    if (i >= p.B * p.H) {  // padding of the last group of 8 items
      hook();
      return;
    }
    b = i / p.H;
    hg = i - b * p.H;
    HG = 1;
  } else {
    // fused 16-bit: a workgroup may take several heads of one image in
    // turn, so that the mask row is read and compacted once for all of
    // them; the last tail_b images of the batch (dispatched last) take one
    // head per workgroup, so the launch ends on short workgroups
    const int ngrp = (p.H + HG - 1) / HG;
    const int lead = (p.B - p.tail_b) * ngrp;
    if (bid < lead) {
      b = bid / ngrp;
      hg = bid - b * ngrp;
    } else {
      const int r = bid - lead, bt = r / p.H;
      b = p.B - p.tail_b + bt;
      hg = r - bt * p.H;
      HG = 1;
    }
  }
  const int H = p.H, N = p.N;
  constexpr int ES = DT == 0 ? 4 : 2;
  const uint32_t rs = (uint32_t)(H * kHeadDim);  // elements between consecutive token rows
  if constexpr (FUSED) {
    uint16_t* idx = reinterpret_cast<uint16_t*>(smem);
    int32_t* cnt = reinterpret_cast<int32_t*>(smem + attn_cnt_off(N));
    const int n = compact_row<NT, uint16_t, true>(p.mask + (size_t)b * N, N, idx, nullptr, nullptr, cnt);
    unsigned char* kvbase = smem + attn_compact_bytes(N);
    const int h0 = hg * HG, h1 = min(H, h0 + HG);
    const uint32_t bytes = (uint32_t)N * rs * ES;
    auto roff = [=](int r) -> uint32_t { return (uint32_t)idx[min(r, n - 1)] * (rs * ES); };
    auto zero_rows = [&] {
      // every head of the group at once: their slices of a row are contiguous
      zero_pruned<NT, ES>(make_rsrc(rebase(p, ((size_t)b * N * H + h0) * kHeadDim, ES).o, bytes),
                          idx + n, N - n, h1 - h0, rs * ES, t, S);
    };
    // A whole sequence (16-bit, not key-split) issues its zero rows right
    // after its staging barrier, so that they drain during the attention:
    // issued before the staging loads, they would be part of the wait for
    // them (the vector-memory counter counts stores too, in order).  A
    // query tile without query rows stages nothing and writes its share at
    // once.
    const bool late_zero = DT != 0 && !KEYSPLIT && n > 0 && n <= p.rc && t * kQBlock < n;
    if (!late_zero) zero_rows();
    if constexpr (DT != 0) {
      if (n > 0 && n <= p.rc) {
        // whole sequence resident: as many of the group's heads at once as
        // their K/V rows fit in the staging area
        const int fit = p.rc / round_up(n, kQBlock);
        for (int h = h0; h < h1;) {
          const int nh = min(fit, h1 - h);
          if (h > h0) __syncthreads();  // the previous heads' staged rows are consumed
          const AttnParams pl = rebase(p, ((size_t)b * N * H + h) * kHeadDim, ES);
          if (t * kQBlock >= n) {  // the tile has no query rows
          } else if constexpr (KEYSPLIT) {
            attend_block_split16<DT>(n, p.scale_log2e, kvbase, make_rsrc(pl.q, bytes),
                                     make_rsrc(pl.k, bytes), make_rsrc(pl.v, bytes),
                                     make_rsrc(pl.o, bytes), roff, hook, t, S,
                                     kvbase + p.rc * (kHeadDim * 2 * 2) + kItemSlotBytes);
          } else {
            attend_resident16<DT, LANES_PER_TILE>(n, nh, p.scale_log2e, kvbase,
                                                  make_rsrc(pl.q, bytes), make_rsrc(pl.k, bytes),
                                                  make_rsrc(pl.v, bytes), make_rsrc(pl.o, bytes),
                                                  roff,
                                                  [&] {
                                                    if (h == h0) zero_rows();
                                                    hook();
                                                  },
                                                  t, S);
          }
          h += nh;
        }
        return;
      }
    }
    for (int h = h0; h < h1; ++h) {
      if (h > hg * HG) __syncthreads();  // the previous head's staged rows are consumed
      if (n <= 0) break;
      const AttnParams pl = rebase(p, ((size_t)b * N * H + h) * kHeadDim, ES);
      if constexpr (DT == 0) {
        float* comb = reinterpret_cast<float*>(kvbase);
        for (int qb = t; qb * kQBlock < n; qb += S)
          block32(make_rsrc(pl.q, bytes), make_rsrc(pl.k, bytes), make_rsrc(pl.v, bytes),
                  make_rsrc(pl.o, bytes), n, qb, p.scale_log2e, roff, comb);
      } else {
        attend_seq16<DT>(pl, n, kvbase, make_rsrc(pl.q, bytes), make_rsrc(pl.k, bytes),
                         make_rsrc(pl.v, bytes), make_rsrc(pl.o, bytes), roff, hook, t, S);
      }
    }
    if (n <= 0) hook();
  } else {
    const int h = hg;
    const int row0 = p.cu[b];
    const int n = p.cu[b + 1] - row0;
    // sequences longer than the ABI's token limit are outside the contract:
    // their rows are left as they are (offsets then stay within 32 bits)
    if (n <= 0 || n > kMaxSeq) return;
    const AttnParams pl = rebase(p, ((size_t)row0 * H + h) * kHeadDim, ES);
    const uint32_t bytes = (uint32_t)n * rs * ES;
    auto roff = [=](int r) -> uint32_t { return (uint32_t)r * (rs * ES); };
    if constexpr (DT == 0) {
      float* comb = reinterpret_cast<float*>(smem);
      for (int qb = t; qb * kQBlock < n; qb += S)
        block32(make_rsrc(pl.q, bytes), make_rsrc(pl.k, bytes), make_rsrc(pl.v, bytes),
                make_rsrc(pl.o, bytes), n, qb, p.scale_log2e, roff, comb);
    } else {
      if (n <= p.rc) {
        if (t * kQBlock >= n) {
        } else if constexpr (KEYSPLIT) {
          attend_block_split16<DT>(n, p.scale_log2e, smem, make_rsrc(pl.q, bytes),
                                   make_rsrc(pl.k, bytes), make_rsrc(pl.v, bytes),
                                   make_rsrc(pl.o, bytes), roff, hook, t, S,
                                   smem + p.rc * (kHeadDim * 2 * 2));
        } else {
          attend_resident16<DT>(n, 1, p.scale_log2e, smem, make_rsrc(pl.q, bytes),
                                make_rsrc(pl.k, bytes), make_rsrc(pl.v, bytes),
                                make_rsrc(pl.o, bytes), roff, hook, t, S);
        }
      } else {
        attend_seq16<DT>(pl, n, smem, make_rsrc(pl.q, bytes), make_rsrc(pl.k, bytes),
                         make_rsrc(pl.v, bytes), make_rsrc(pl.o, bytes), roff, hook, t, S);
      }
    }
  }
}

template <int DT, bool FUSED, bool KEYSPLIT = false>
__device__ __forceinline__ void attend_body(const AttnParams& p, unsigned char* smem) {
  constexpr int NT = DT == 0 ? kAttnThreads32 : kAttnThreads16;
  int bid = blockIdx.x;
  if constexpr (FUSED) {
    if (p.cu_out || p.max_out) {
      if (bid == 0) {
        count_scan_block<NT>(p.mask, p.B, p.N, p.cu_out, p.max_out, reinterpret_cast<int*>(smem));
        return;
      }
      --bid;
    }
  }
  attend_item<DT, FUSED, false, KEYSPLIT>(p, bid, smem, [] {});
}

// 16-bit: 4 waves, register budget for 3 waves per SIMD (3 workgroups per CU).
template <int DT, bool FUSED, bool KEYSPLIT = false>
__global__ __launch_bounds__(kAttnThreads16, 3) void attend16_kernel(AttnParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  attend_body<DT, FUSED, KEYSPLIT>(p, smem);
}

template <bool FUSED>
__global__ __launch_bounds__(kAttnThreads32) void attend32_kernel(AttnParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  attend_body<0, FUSED>(p, smem);
}

// Persistent form of the fused 16-bit kernel: as many workgroups as stay
// resident, each pulling items from a device counter instead of being
// dispatched one item each.  The items are exactly the one-launch kernel's
// grid positions (an image's head pair, or one head of a tail image) and
// run the same per-item code, so registers, staging and results are the
// same bit for bit; what changes is that no workgroup launch separates two
// items of one slot.  Thread 0 fetches the next item's index while the
// current item runs (one atomic ahead) and hands it to the workgroup through
// a 4-byte LDS slot past the staging area: it writes the slot right after
// the item's first staging barrier, where its wave has already waited for
// every earlier load, the atomic included.  The workgroup that leaves last
// returns the counter to zero for the next launch.
template <int DT>
__global__ __launch_bounds__(kAttnThreads16, 3) void attend16_persistent_kernel(AttnParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NT = kAttnThreads16;
  const int tid = threadIdx.x;
  int* slot = reinterpret_cast<int*>(smem + p.item_slot);
  const int HG = p.heads_per_wg;
  const int nitems = (p.B - p.tail_b) * ((p.H + HG - 1) / HG) + p.tail_b * p.H;
  if (blockIdx.x == 0 && (p.cu_out || p.max_out)) {
    count_scan_block<NT>(p.mask, p.B, p.N, p.cu_out, p.max_out, reinterpret_cast<int*>(smem));
    __syncthreads();  // its LDS is reused below
  }
  if (tid == 0) *slot = atomicAdd(p.work, 1);
  __syncthreads();
  int item = *slot;
  while (item < nitems) {
    int next = 0;
    if (tid == 0) next = atomicAdd(p.work, 1);
    attend_item<DT, true, true>(p, item, smem, [&] {
      if (tid == 0) *slot = next;
    });
    // every wave is done with the item's LDS and the slot holds the next index
    lds_barrier();
    item = *slot;
  }
  if (tid == 0) {
    __threadfence();
    if (atomicAdd(p.work + 1, 1) == (int)gridDim.x - 1) {
      atomicExch(p.work, 0);
      atomicExch(p.work + 1, 0);
    }
  }
}

// Rows of the 16-bit staging area, which stages whole sequences of up to
// that many rows: as many 16-row blocks as the LDS left to each of 3
// workgroups per CU holds (after the compaction area and `reserved`
// bytes), at most kResidentMax16.  At N = 197 that is 208 rows: 53248 bytes
// of K/V, 448 of compaction area and the 16-byte item slot; at N = 1024
// still 192, the two key buffers of the streamed form.
static int resident_rows(int dtype, bool fused, int N, int reserved) {
  if (dtype == 0) return 0;
  const long long per_wg = (long long)kLdsPerWg16 - reserved -
                           (fused ? (long long)attn_compact_bytes(N) : 0);
  int rows = (int)(per_wg / (kHeadDim * 2 * 2)) / kQBlock * kQBlock;
  return rows > kResidentMax16 ? kResidentMax16 : rows;
}
static_assert((kLdsPerWg16 - kItemSlotBytes - (2 * 1024 + 16 * 12)) / (kHeadDim * 2 * 2) / kQBlock *
                      kQBlock >= 2 * kChunk16,
              "the streamed form's two key buffers fit the staging area at N = 1024");

int attend_resident_rows(int dtype, bool fused, int N) {
  return resident_rows(dtype, fused, N, (fused && dtype != 0) ? kItemSlotBytes : 0);
}

long long attend_grid_items(const AttnParams& p, int dtype, bool fused) {
  const long long bh = (long long)p.B * p.H;
  if (dtype == 0 || p.qsplit > 1) return (bh + 7) / 8 * 8 * p.qsplit;
  const int hg = (fused && dtype != 0) ? p.heads_per_wg : 1;
  const int tail = (fused && dtype != 0) ? p.tail_b : 0;
  return (long long)(p.B - tail) * ((p.H + hg - 1) / hg) + (long long)tail * p.H;
}

// Dynamic LDS of the fused 16-bit kernels: compaction area, staging area and
// the persistent form's item slot (reserved by both forms, so that both give
// the same sequences the same staging).
static size_t fused16_lds(int N, int rc) {
  return attn_lds_bytes(1, true, N, rc) + kItemSlotBytes;
}

int attend_persistent_per_cu(int N) {
  const int rc = resident_rows(1, true, N, kItemSlotBytes);
  const int by_lds = (int)(kLdsPerCu / fused16_lds(N, rc));
  return by_lds < kAttnWgPerCu16 ? by_lds : kAttnWgPerCu16;  // 3 waves per SIMD by registers
}

hipError_t launch_attend_persistent(const AttnParams& p0, int dtype, int grid, hipStream_t s) {
  AttnParams p = p0;
  p.rc = resident_rows(dtype, true, p.N, kItemSlotBytes);
  const size_t lds = fused16_lds(p.N, p.rc);
  p.item_slot = (int)(lds - kItemSlotBytes);
  if (dtype == 1)
    hipLaunchKernelGGL((attend16_persistent_kernel<1>), dim3(grid), dim3(kAttnThreads16), lds, s, p);
  else
    hipLaunchKernelGGL((attend16_persistent_kernel<2>), dim3(grid), dim3(kAttnThreads16), lds, s, p);
  return hipGetLastError();
}

// Dynamic LDS limit: the 160 KB of a CU.
static hipError_t set_lds_limit(const void* fn) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsPerCu);
}

hipError_t attend_init() {
  const void* fns[12] = {reinterpret_cast<const void*>(&attend16_persistent_kernel<1>),
                        reinterpret_cast<const void*>(&attend16_persistent_kernel<2>),
                        reinterpret_cast<const void*>(&attend32_kernel<false>),
                        reinterpret_cast<const void*>(&attend32_kernel<true>),
                        reinterpret_cast<const void*>(&attend16_kernel<1, false>),
                        reinterpret_cast<const void*>(&attend16_kernel<1, true>),
                        reinterpret_cast<const void*>(&attend16_kernel<2, false>),
                        reinterpret_cast<const void*>(&attend16_kernel<2, true>),
                        reinterpret_cast<const void*>(&attend16_kernel<1, false, true>),
                        reinterpret_cast<const void*>(&attend16_kernel<1, true, true>),
                        reinterpret_cast<const void*>(&attend16_kernel<2, false, true>),
                        reinterpret_cast<const void*>(&attend16_kernel<2, true, true>)};
  for (const void* f : fns) {
    hipError_t e = set_lds_limit(f);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attend(const AttnParams& p0, int dtype, bool fused, hipStream_t s) {
  AttnParams p = p0;
  const bool fused16 = fused && dtype != 0;
  p.rc = resident_rows(dtype, fused, p.N, fused16 ? kItemSlotBytes : 0);
  const size_t lds = (fused16 ? fused16_lds(p.N, p.rc) : attn_lds_bytes(dtype, fused, p.N, p.rc)) +
                     (dtype != 0 && p.keysplit ? kComb16Bytes : 0);
  const int grid = (int)attend_grid_items(p, dtype, fused) +
                   ((fused && (p.cu_out || p.max_out)) ? 1 : 0);
  const dim3 blk(attn_threads(dtype));
  if (dtype == 0) {
    if (fused) hipLaunchKernelGGL((attend32_kernel<true>), dim3(grid), blk, lds, s, p);
    else hipLaunchKernelGGL((attend32_kernel<false>), dim3(grid), blk, lds, s, p);
  } else if (p.keysplit) {
    if (dtype == 1) {
      if (fused) hipLaunchKernelGGL((attend16_kernel<1, true, true>), dim3(grid), blk, lds, s, p);
      else hipLaunchKernelGGL((attend16_kernel<1, false, true>), dim3(grid), blk, lds, s, p);
    } else {
      if (fused) hipLaunchKernelGGL((attend16_kernel<2, true, true>), dim3(grid), blk, lds, s, p);
      else hipLaunchKernelGGL((attend16_kernel<2, false, true>), dim3(grid), blk, lds, s, p);
    }
  } else if (dtype == 1) {
    if (fused) hipLaunchKernelGGL((attend16_kernel<1, true>), dim3(grid), blk, lds, s, p);
    else hipLaunchKernelGGL((attend16_kernel<1, false>), dim3(grid), blk, lds, s, p);
  } else {
    if (fused) hipLaunchKernelGGL((attend16_kernel<2, true>), dim3(grid), blk, lds, s, p);
    else hipLaunchKernelGGL((attend16_kernel<2, false>), dim3(grid), blk, lds, s, p);
  }
  return hipGetLastError();
}

}  // namespace rva
