// Ragged bidirectional attention, packed and fused forms.
//
// What is computed follows "Dispatch-Aware Ragged Attention for Pruned Vision
// Transformers" (sota2.com page, Abstract): non-causal attention over each
// image's kept tokens only, O = softmax(Q K^T * scale) V per image and head.
//
// Work decomposition (CDNA4 / gfx950), 16-bit inputs:
//  * one workgroup of 4 waves per (image, head).  Post-pruning ViT sequences
//    are short (at most 197 tokens at 224x224, 577 at 384x384), so the
//    workgroup stages its sequence's K and V (V transposed) in LDS in one
//    memory round trip; sequences longer than one chunk are staged in chunks;
//  * each wave owns two query blocks of 16 rows at a time and walks the keys
//    32 at a time;
//  * scores are formed transposed, S^T = K Q^T, with the 16x16x32 matrix-core
//    product: each lane then holds one query and 4+4 keys, which is exactly
//    the per-lane slice the second product O^T = V^T P^T takes as its B
//    operand, so P never leaves registers;
//  * softmax in fp32 with exp2 (log2 e folded into the scale).  The running
//    max is shared by the four lanes of a query with two lane-swap steps;
//    row sums come from the matrix cores (an all-ones operand times the
//    rounded probabilities).  The output is rescaled only when
//    the max grows by more than 2^8 (the stale max still bounds every
//    probability by 2^8, far inside fp16/bf16 range, and cancels exactly in
//    the final division);
//  * the fused form first compacts the image's keep-mask row in LDS, reads
//    Q/K/V rows straight from the padded tensors through that list, writes
//    O rows straight to padded positions and zero-fills pruned rows.  An
//    optional extra workgroup computes cu_seqlens / max_seqlen in the same
//    launch.
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
// scores are s0 (keys 4g..4g+3) and s1 (keys 16+4g..16+4g+3) in this lane.
// Writes the (unnormalised) probabilities to pr[8]; rescales `o` and `l`
// only when some query's max grew by more than kRescaleSlack.
__device__ __forceinline__ void softmax_step(f32x4& s0, f32x4& s1, int kvalid, float c, float& m,
                                             float& l, f32x4 (&o)[4], float (&pr)[8]) {
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
    l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pr[j] = fast_exp2(fmaf(s0[j], c, -m));
    pr[4 + j] = fast_exp2(fmaf(s1[j], c, -m));
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += pr[j];
  l += sum;
}

// 16-bit variant: the row sums are a fifth accumulator block o[4] (computed
// by the matrix cores from an all-ones operand), so only the max is tracked
// here; a rescale multiplies all five blocks.
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

// Staged K is [kc][64] halves with the eight 16-byte pieces of row r stored
// at piece index p ^ (r & 7): the 16 rows a b128 fragment read touches then
// spread over all banks without padding.
__device__ __forceinline__ int kswz(int row, int piece) { return row * 64 + ((piece ^ (row & 7)) << 3); }

template <int DT>
__device__ __forceinline__ void tile16(const typename Half16<DT>::T* __restrict__ Ks,
                                       const typename Half16<DT>::T* __restrict__ Vt, int VP, int k0,
                                       int kvalid, const typename Half16<DT>::V8 (&qf)[2][2],
                                       f32x4 (&o)[2][5], float (&m)[2], bool two, float c) {
  typedef Half16<DT> Tr;
  typedef typename Tr::T T;
  typedef typename Tr::V8 V8;
  typedef typename Tr::V4 V4;
  const int lane = lane_id(), g = lane >> 4, r16 = lane & 15;
  // A operand of S^T = K Q^T: lane (r16, g) holds K[k0 + 16 kb + r16][32 ks + 8 g .. + 7]
  V8 kf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      kf[kb][ks] = *reinterpret_cast<const V8*>(Ks + kswz(k0 + kb * 16 + r16, ks * 4 + g));
  V8 vf[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const T* row = Vt + (db * 16 + r16) * VP + k0 + 4 * g;
    const V4 lo = *reinterpret_cast<const V4*>(row);
    const V4 hi = *reinterpret_cast<const V4*>(row + 16);
    vf[db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i == 1 && !two) break;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    s0 = Tr::mfma(kf[0][0], qf[i][0], s0);
    s1 = Tr::mfma(kf[1][0], qf[i][0], s1);
    s0 = Tr::mfma(kf[0][1], qf[i][1], s0);
    s1 = Tr::mfma(kf[1][1], qf[i][1], s1);
    float pr[8];
    softmax_step16(s0, s1, kvalid, c, m[i], o[i], pr);
    V8 pf;
#pragma unroll
    for (int j = 0; j < 8; ++j) pf[j] = (T)pr[j];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[i][db] = Tr::mfma(vf[db], pf, o[i][db]);
    // row sums of the rounded probabilities: every row of an all-ones A
    // operand yields sum_k P[q][k], so each lane ends up holding its query's sum
    V8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (T)1.0f;
    o[i][4] = Tr::mfma(ones, pf, o[i][4]);
  }
}

// Global accesses of the 16-bit path go through raw buffer descriptors
// (make_rsrc) whose base is the sequence's head slice and whose size covers
// exactly its rows, so ragged tails need no branches.

// Stage keys [c0, c0 + rows) of the sequence: K rows into Ks (swizzled
// 16-byte pieces), V transposed into Vt[d][key].  Every load of the chunk is
// issued before the first LDS store, so one memory round trip stages the
// whole chunk.  The V^T block of an item is 4 keys x 4 dims: four 8-byte row
// loads (16 lanes cover one 128-byte row), a 4x4 transpose of 16-bit values
// in registers, four 8-byte LDS stores.  Keys in [rows, round_up(rows, 32))
// load as zeros, so masked probabilities (exact zeros) never meet stale LDS
// contents.  `roff(r)` is the byte offset of sequence row r.
template <int DT, typename RowOff>
__device__ __forceinline__ void stage16(Rsrc rk, Rsrc rv, typename Half16<DT>::T* Ks,
                                        typename Half16<DT>::T* Vt, int VP, int c0, int rows,
                                        RowOff roff) {
  constexpr int NT = kAttnThreads16;
  constexpr int UK = (kKcMax16 * 8 + NT - 1) / NT;       // K pieces per thread at most
  constexpr int UV = (kKcMax16 / 4 * 16 + NT - 1) / NT;  // V^T blocks per thread at most
  static_assert(kKcMax16 % kKeyTile == 0, "chunks are whole key tiles");
  const int tid = threadIdx.x;
  const int rpad = round_up(rows, kKeyTile);
  const int kitems = rpad * 8, vitems = rpad / 4 * 16;
  u32x4 kr[UK];
  u32x2 vr[UV][4];
#pragma unroll
  for (int u = 0; u < UK; ++u) {
    const int e = tid + u * NT;
    const int r = e >> 3, pc = e & 7;
    const uint32_t o = (e < kitems && r < rows) ? roff(c0 + r) + pc * 16 : kOOB;
    kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)o, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < UV; ++u) {
    const int it = tid + u * NT;
    const int kq = it >> 4, dq = it & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = 4 * kq + j;
      const uint32_t o = (it < vitems && key < rows) ? roff(c0 + key) + dq * 8 : kOOB;
      vr[u][j] = __builtin_amdgcn_raw_buffer_load_b64(rv, (int)o, 0, 0);
    }
  }
#pragma unroll
  for (int u = 0; u < UK; ++u) {
    const int e = tid + u * NT;
    if (e < kitems) *reinterpret_cast<u32x4*>(Ks + kswz(e >> 3, e & 7)) = kr[u];
  }
  char* vt = reinterpret_cast<char*>(Vt);
#pragma unroll
  for (int u = 0; u < UV; ++u) {
    const int it = tid + u * NT;
    if (it >= vitems) continue;
    const int kq = it >> 4, dq = it & 15;
    // vr[u][j] holds V[key 4kq+j][dims 4dq..4dq+3]; out holds V^T[dim 4dq+i][keys 4kq..4kq+3]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int w = i >> 1;
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
      u32x2 out;
      out[0] = __builtin_amdgcn_perm(vr[u][1][w], vr[u][0][w], sel);
      out[1] = __builtin_amdgcn_perm(vr[u][3][w], vr[u][2][w], sel);
      *reinterpret_cast<u32x2*>(vt + ((4 * dq + i) * VP + 4 * kq) * 2) = out;
    }
  }
}

// One sequence (image or packed run), one head.  rq/rk/rv/ro cover the
// sequence's head slice; roff(r) is the byte offset of its row r.
template <int DT, typename RowOff>
__device__ __forceinline__ void attend_seq16(const AttnParams& p, int n, unsigned char* kvbase,
                                             Rsrc rq, Rsrc rk, Rsrc rv, Rsrc ro, RowOff roff) {
  typedef Half16<DT> Tr;
  typedef typename Tr::T T;
  typedef typename Tr::V8 V8;
  typedef typename Tr::V4 V4;
  const int lane = lane_id(), w = wave_id(), g = lane >> 4, r16 = lane & 15;
  const int kc = p.kc, VP = kc + kVPad16;
  T* Ks = reinterpret_cast<T*>(kvbase);
  T* Vt = Ks + kc * kHeadDim;
  constexpr int kWaves = kAttnThreads16 / 64;
  constexpr int kPerPass = kWaves * kQBlocksPerWave;
  const int nqb = (n + kQBlock - 1) / kQBlock;
  const int npass = (nqb + kPerPass - 1) / kPerPass;
  const int nchunk = (n + kc - 1) / kc;
  const float c = p.scale_log2e;

  for (int pass = 0; pass < npass; ++pass) {
    int qb[2];
    bool act[2];
    uint32_t qoff[2];
    V8 qf[2][2];
    f32x4 o[2][5];
    float m[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      qb[i] = pass * kPerPass + w + i * kWaves;
      act[i] = qb[i] < nqb;
      const int q = qb[i] * kQBlock + r16;
      qoff[i] = (act[i] && q < n) ? roff(q) : kOOB;
      // B operand of S^T = K Q^T: lane (r16, g) holds Q[q][32 ks + 8 g .. + 7]
      qf[i][0] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(qoff[i] + 16 * g), 0, 0));
      qf[i][1] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(qoff[i] + 64 + 16 * g), 0, 0));
    }
    for (int cc = 0; cc < nchunk; ++cc) {
      // odd passes walk the chunks backwards so the chunk left staged by the
      // previous pass is used first (softmax accumulation is order-free)
      const int ch = (pass & 1) ? nchunk - 1 - cc : cc;
      const int c0 = ch * kc;
      const int rows = min(kc, n - c0);
      if (!(pass > 0 && cc == 0)) {
        if (pass > 0 || cc > 0) __syncthreads();
        stage16<DT>(rk, rv, Ks, Vt, VP, c0, rows, roff);
        __syncthreads();
      }
      if (cc == 0) {  // accumulators come alive only after the first staging
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          m[i] = -INFINITY;
#pragma unroll
          for (int db = 0; db < 5; ++db) o[i][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      if (act[0]) {
        const int ntile = (rows + kKeyTile - 1) / kKeyTile;
        for (int t = 0; t < ntile; ++t) {
          const int k0 = t * kKeyTile;
          tile16<DT>(Ks, Vt, VP, k0, min(kKeyTile, rows - k0), qf, o, m, act[1], c);
        }
      }
    }
    // O^T block db, lane (r16, g) holds O[q][16 db + 4 g .. + 3]; o[i][4] holds
    // the query's probability sum in every element.  Rows q >= n go to kOOB.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (!act[i]) continue;
      const float inv = 1.f / o[i][4][0];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        V4 out;
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = (T)(o[i][db][j] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, out), ro,
                                              (int)(qoff[i] + db * 32 + 8 * g), 0, 0);
      }
    }
  }
}

// ---------------------------------------------------------------- fp32

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// fp32 matrix-core form.  The 16x16x4 product takes one k value per lane
// group; lane group g covers head dims 16g..16g+15 over 16 steps (any
// consistent split of the contraction is valid), so each lane's Q and K
// slices are 64 contiguous bytes.  For P V the k index is the key: step
// (kb, j) uses key 16kb + 4g + j, which is exactly the score this lane holds.
__device__ __forceinline__ void tile32(const float* __restrict__ Ks, const float* __restrict__ Vs,
                                       int k0, int kvalid, const f32x4 (&qf)[2][4],
                                       f32x4 (&o)[2][4], float (&m)[2], float (&l)[2], bool two,
                                       float c) {
  const int lane = lane_id(), g = lane >> 4, r16 = lane & 15;
  f32x4 kf[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
      kf[kb][t4] = *reinterpret_cast<const f32x4*>(Ks + (k0 + kb * 16 + r16) * kPitch32 + 16 * g + 4 * t4);
  float va[4][8];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      va[db][j] = Vs[(k0 + (j >> 2) * 16 + 4 * g + (j & 3)) * kPitch32 + db * 16 + r16];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i == 1 && !two) break;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      s0 = mfma_f32(kf[0][t >> 2][t & 3], qf[i][t >> 2][t & 3], s0);
      s1 = mfma_f32(kf[1][t >> 2][t & 3], qf[i][t >> 2][t & 3], s1);
    }
    float pr[8];
    softmax_step(s0, s1, kvalid, c, m[i], l[i], o[i], pr);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 8; ++j) o[i][db] = mfma_f32(va[db][j], pr[j], o[i][db]);
  }
}

template <typename Elem>
__device__ __forceinline__ void stage32(const float* __restrict__ kg, const float* __restrict__ vg,
                                        float* Ks, float* Vs, int c0, int rows, Elem elem) {
  constexpr int NT = kAttnThreads32;
  const int tid = threadIdx.x;
  const int total = round_up(rows, kKeyTile) * 16;  // <= kKcMax32 * 16
  u32x4 kr[4], vr[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = tid + u * NT;
    kr[u] = u32x4{0u, 0u, 0u, 0u};
    vr[u] = kr[u];
    const int r = e >> 4, pc = e & 15;
    if (e < total && r < rows) {
      const uint32_t el = elem(c0 + r) + pc * 4;
      kr[u] = *reinterpret_cast<const u32x4*>(kg + el);
      vr[u] = *reinterpret_cast<const u32x4*>(vg + el);
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = tid + u * NT;
    if (e < total) {
      const int r = e >> 4, pc = e & 15;
      *reinterpret_cast<u32x4*>(Ks + r * kPitch32 + pc * 4) = kr[u];
      *reinterpret_cast<u32x4*>(Vs + r * kPitch32 + pc * 4) = vr[u];
    }
  }
}

template <typename Elem>
__device__ __forceinline__ void attend_seq32(const AttnParams& p, int n, unsigned char* kvbase,
                                             Elem elem) {
  const int lane = lane_id(), w = wave_id(), g = lane >> 4, r16 = lane & 15;
  const int kc = p.kc;
  float* Ks = reinterpret_cast<float*>(kvbase);
  float* Vs = Ks + kc * kPitch32;
  const float* __restrict__ qg = static_cast<const float*>(p.q);
  const float* __restrict__ kg = static_cast<const float*>(p.k);
  const float* __restrict__ vg = static_cast<const float*>(p.v);
  float* __restrict__ og = static_cast<float*>(p.o);
  constexpr int kWaves = kAttnThreads32 / 64;
  constexpr int kPerPass = kWaves * kQBlocksPerWave;
  const int nqb = (n + kQBlock - 1) / kQBlock;
  const int npass = (nqb + kPerPass - 1) / kPerPass;
  const int nchunk = (n + kc - 1) / kc;
  const float c = p.scale_log2e;

  for (int pass = 0; pass < npass; ++pass) {
    int qb[2];
    bool act[2];
    f32x4 qf[2][4];
    f32x4 o[2][4];
    float m[2], l[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      qb[i] = pass * kPerPass + w + i * kWaves;
      act[i] = qb[i] < nqb;
      m[i] = -INFINITY;
      l[i] = 0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[i][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int q = qb[i] * kQBlock + r16;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) qf[i][t4] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (act[i] && q < n) {
        const uint32_t e = elem(q);
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) qf[i][t4] = *reinterpret_cast<const f32x4*>(qg + e + 16 * g + 4 * t4);
      }
    }
    for (int ch = 0; ch < nchunk; ++ch) {
      const int c0 = ch * kc;
      const int rows = min(kc, n - c0);
      if (nchunk > 1 || pass == 0) {
        if (pass > 0 || ch > 0) __syncthreads();
        stage32(kg, vg, Ks, Vs, c0, rows, elem);
        __syncthreads();
      }
      if (act[0]) {
        const int ntile = (rows + kKeyTile - 1) / kKeyTile;
        for (int t = 0; t < ntile; ++t) {
          const int k0 = t * kKeyTile;
          tile32(Ks, Vs, k0, min(kKeyTile, rows - k0), qf, o, m, l, act[1], c);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (!act[i]) continue;
      const float inv = 1.f / quad_sum(l[i]);
      const int q = qb[i] * kQBlock + r16;
      if (q < n) {
        const uint32_t e = elem(q);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          *reinterpret_cast<f32x4*>(og + e + db * 16 + 4 * g) = o[i][db] * inv;
      }
    }
  }
}

// ---------------------------------------------------------------- kernels

// Zero the output rows of pruned tokens of one (image, head); `o` points at
// the head's slice of the image's first token row.
template <int NT, int ESIZE>
__device__ __forceinline__ void zero_pruned(char* o, const uint64_t* ballots, int N, int H) {
  constexpr int PIECES = kHeadDim * ESIZE / 16;
  const uint32_t rs = (uint32_t)(H * kHeadDim * ESIZE);
  const int total = N * PIECES;
  for (int e = threadIdx.x; e < total; e += NT) {
    const int j = e / PIECES, pc = e - j * PIECES;
    const bool kept = (ballots[j >> 6] >> (j & 63)) & 1ull;
    if (!kept) *reinterpret_cast<u32x4*>(o + (uint32_t)j * rs + pc * 16) = u32x4{0u, 0u, 0u, 0u};
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

template <int DT, bool FUSED>
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
  const int b = bid / p.H, h = bid - b * p.H;
  const int H = p.H, N = p.N;
  constexpr int ES = DT == 0 ? 4 : 2;
  const uint32_t rs = (uint32_t)(H * kHeadDim);  // elements between consecutive token rows
  if constexpr (FUSED) {
    int32_t* idx = reinterpret_cast<int32_t*>(smem);
    const size_t off = (size_t)round_up(N * 4, 16);
    uint64_t* ballots = reinterpret_cast<uint64_t*>(smem + off);
    int32_t* cnt = reinterpret_cast<int32_t*>(smem + off + 16 * 8);
    const int n = compact_row<NT>(p.mask + (size_t)b * N, N, idx, nullptr, ballots, cnt);
    const AttnParams pl = rebase(p, ((size_t)b * N * H + h) * kHeadDim, ES);
    zero_pruned<NT, ES>(static_cast<char*>(pl.o), ballots, N, H);
    if (n <= 0) return;
    unsigned char* kvbase = smem + attn_compact_bytes(N);
    auto elem = [=](int r) -> uint32_t { return (uint32_t)idx[r] * rs; };
    if constexpr (DT == 0) {
      attend_seq32(pl, n, kvbase, elem);
    } else {
      const uint32_t bytes = (uint32_t)N * rs * ES;
      auto roff = [=](int r) -> uint32_t { return (uint32_t)idx[min(r, n - 1)] * (rs * ES); };
      attend_seq16<DT>(pl, n, kvbase, make_rsrc(pl.q, bytes), make_rsrc(pl.k, bytes),
                       make_rsrc(pl.v, bytes), make_rsrc(pl.o, bytes), roff);
    }
  } else {
    const int row0 = p.cu[b];
    const int n = p.cu[b + 1] - row0;
    if (n <= 0) return;
    const AttnParams pl = rebase(p, ((size_t)row0 * H + h) * kHeadDim, ES);
    auto elem = [=](int r) -> uint32_t { return (uint32_t)r * rs; };
    if constexpr (DT == 0) {
      attend_seq32(pl, n, smem, elem);
    } else {
      const uint32_t bytes = (uint32_t)n * rs * ES;
      auto roff = [=](int r) -> uint32_t { return (uint32_t)r * (rs * ES); };
      attend_seq16<DT>(pl, n, smem, make_rsrc(pl.q, bytes), make_rsrc(pl.k, bytes),
                       make_rsrc(pl.v, bytes), make_rsrc(pl.o, bytes), roff);
    }
  }
}

// 16-bit: 4 waves, register budget for 3 waves per SIMD (3 workgroups per CU).
template <int DT, bool FUSED>
__global__ __launch_bounds__(kAttnThreads16, 3) void attend16_kernel(AttnParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  attend_body<DT, FUSED>(p, smem);
}

template <bool FUSED>
__global__ __launch_bounds__(kAttnThreads32) void attend32_kernel(AttnParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  attend_body<0, FUSED>(p, smem);
}

static hipError_t set_lds_limit(const void* fn) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

hipError_t attend_init() {
  const void* fns[6] = {reinterpret_cast<const void*>(&attend32_kernel<false>),
                        reinterpret_cast<const void*>(&attend32_kernel<true>),
                        reinterpret_cast<const void*>(&attend16_kernel<1, false>),
                        reinterpret_cast<const void*>(&attend16_kernel<1, true>),
                        reinterpret_cast<const void*>(&attend16_kernel<2, false>),
                        reinterpret_cast<const void*>(&attend16_kernel<2, true>)};
  for (const void* f : fns) {
    hipError_t e = set_lds_limit(f);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attend(const AttnParams& p, int dtype, bool fused, hipStream_t s) {
  const size_t lds = attn_lds_bytes(dtype, fused, p.N, p.kc);
  const int grid = p.B * p.H + ((fused && (p.cu_out || p.max_out)) ? 1 : 0);
  const dim3 blk(attn_threads(dtype));
  if (dtype == 0) {
    if (fused) hipLaunchKernelGGL((attend32_kernel<true>), dim3(grid), blk, lds, s, p);
    else hipLaunchKernelGGL((attend32_kernel<false>), dim3(grid), blk, lds, s, p);
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
