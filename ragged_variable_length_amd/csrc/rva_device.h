// Device helpers shared by the pack, unpack and attention kernels:
// wave/workgroup reductions and scans, and the per-image row compaction that
// turns a keep-mask row into the ascending list of kept token positions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rva {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer descriptors: a base address and a size in bytes.  Offsets are
// 32-bit, and an offset at or past the size (kOOB is past every size used
// here) reads zeros and drops stores in hardware.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// The wave's index in its workgroup, through a first-lane read: the
// compiler then knows it is the same in every lane, so arithmetic and
// branches on it (unit and row assignments) run on the scalar unit.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// A workgroup barrier that orders LDS only: this wave's LDS accesses
// complete, then s_barrier.  Unlike __syncthreads it does not wait for the
// wave's global loads and stores in flight.  The clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Workgroup-wide inclusive scan of one int per thread.  `tmp` holds at least
// (blockDim.x / 64) ints.  Returns the inclusive prefix; *total receives the
// sum over the workgroup.  Contains two barriers; every thread must call it.
template <int NT>
__device__ int block_inclusive_scan(int v, int* tmp, int* total) {
  constexpr int W = NT / 64;
  const int lane = lane_id(), w = wave_id();
  int incl = wave_inclusive_scan(v);
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    int t = tmp[i];
    before += (i < w) ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl;
}

template <int NT>
__device__ int block_max(int v, int* tmp) {
  constexpr int W = NT / 64;
  v = wave_max(v);
  if (lane_id() == 0) tmp[wave_id()] = v;
  __syncthreads();
  int m = tmp[0];
#pragma unroll
  for (int i = 1; i < W; ++i) m = max(m, tmp[i]);
  __syncthreads();
  return m;
}

// Bit i of the result is set when byte i of the 16-byte chunk is nonzero.
__device__ __forceinline__ uint32_t nonzero_bytes16(u32x4 v) {
  uint32_t out = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t x = v[k];
    // high bit of each byte set iff the byte is nonzero
    const uint32_t hi = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
    // gather the four high bits into a nibble (no carries: distinct bit positions)
    out |= ((((hi >> 7) * 0x00204081u) >> 21) & 0xFu) << (4 * k);
  }
  return out;
}

// Kept counts of every image and their exclusive prefix (cu_seqlens), plus
// the largest count, computed by ONE workgroup of NT threads.  Images are
// taken SEG = 4 * NT at a time.  The segment's mask bytes are read as a flat
// array of 16-byte chunks (all threads, several chunks in flight each); a
// chunk straddles at most one image boundary when N >= 16, and its nonzero
// bytes are credited to the (one or two) images with LDS atomics.  The
// workgroup then scans the SEG counts (4 per thread) and carries the total
// into the next segment.  `lds` holds at least SEG + 64 ints.
template <int NT>
__device__ __forceinline__ void count_scan_block(const uint8_t* __restrict__ mask, int B, int N,
                                 int32_t* __restrict__ cu, int32_t* __restrict__ max_out,
                                 int* lds) {
  constexpr int SEG = 4 * NT;
  const int tid = threadIdx.x;
  int* cnt = lds;
  int* tmp = lds + SEG;
  if (tid == 0 && cu) cu[0] = 0;
  const bool vec = N >= 16 && (reinterpret_cast<uintptr_t>(mask) & 15) == 0;
  const long long total_bytes = (long long)B * N;
  int carry = 0, mx = 0;
  for (int b0 = 0; b0 < B; b0 += SEG) {
    const int nimg = min(SEG, B - b0);
    for (int i = tid; i < SEG; i += NT) cnt[i] = 0;
    __syncthreads();
    const long long lo = (long long)b0 * N, hi = (long long)(b0 + nimg) * N;
    if (vec) {
      // whole 16-byte chunks that lie inside [0, B*N): chunk c covers flat
      // bytes [16c, 16c + 16); bytes outside [lo, hi) are ignored
      const long long c_lo = lo >> 4;
      const long long c_hi = min((hi + 15) >> 4, total_bytes >> 4);
      for (long long c0 = c_lo + tid; c0 < c_hi; c0 += 4 * NT) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const long long c = c0 + (long long)u * NT;
          v[u] = c < c_hi ? *reinterpret_cast<const u32x4*>(mask + 16 * c) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const long long c = c0 + (long long)u * NT;
          if (c >= c_hi) continue;
          uint32_t bits = nonzero_bytes16(v[u]);
          const long long f = 16 * c;  // flat index of byte 0
          if (f < lo) bits &= 0xFFFFu << (int)(lo - f);
          if (f + 16 > hi) bits &= 0xFFFFu >> (int)(f + 16 - hi);
          const int img = (int)(f / N);               // image of byte 0
          const int split = (int)((long long)(img + 1) * N - f);  // bytes of byte 0's image
          const uint32_t first = split >= 16 ? bits : bits & ((1u << split) - 1u);
          const uint32_t rest = bits ^ first;
          if (first) atomicAdd(&cnt[img - b0 < 0 ? 0 : img - b0], __popc(first));
          if (rest) atomicAdd(&cnt[img + 1 - b0], __popc(rest));
        }
      }
      // bytes of a final partial chunk (B*N not a multiple of 16)
      for (long long j = max(lo, (total_bytes >> 4) << 4) + tid; j < hi; j += NT)
        if (mask[j]) atomicAdd(&cnt[(int)(j / N) - b0], 1);
    } else {
      for (long long j = lo + tid; j < hi; j += NT)
        if (mask[j]) atomicAdd(&cnt[(int)(j / N) - b0], 1);
    }
    __syncthreads();
    // scan: thread t owns counts 4t..4t+3
    int v4[4], s = 0, m4 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * tid + k;
      v4[k] = i < nimg ? cnt[i] : 0;
      s += v4[k];
      m4 = max(m4, v4[k]);
    }
    int total;
    const int incl = block_inclusive_scan<NT>(s, tmp, &total);
    int run = carry + incl - s;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * tid + k;
      run += v4[k];
      if (cu && i < nimg) cu[b0 + i + 1] = run;
    }
    mx = max(mx, block_max<NT>(m4, tmp));
    carry += total;
  }
  if (tid == 0 && max_out) *max_out = mx;
}

// Mask bytes a thread contributes to the row compaction below: chunk
// c = wave + i * waves, token j = 64 c + lane, zero past N.  Loading them is
// the compaction's only global access, so a caller can issue it early.
template <int NT>
constexpr int compact_per() { return (16 + NT / 64 - 1) / (NT / 64); }

template <int NT>
__device__ __forceinline__ void mask_row_bytes(const uint8_t* __restrict__ mrow, int N,
                                               uint8_t (&mb)[compact_per<NT>()]) {
  constexpr int W = NT / 64;
  const int lane = lane_id(), w = wave_id();
#pragma unroll
  for (int i = 0; i < compact_per<NT>(); ++i) {
    const int j = (w + i * W) * 64 + lane;
    mb[i] = j < N ? mrow[j] : (uint8_t)0;
  }
}

// Row compaction: for one image's mask row (N <= 1024 bytes, given as the
// bytes of mask_row_bytes) build the ascending list of kept positions
// idx[0..n) in LDS and return n (the same value in every thread).  Each wave
// takes 64-token chunks; a ballot gives every kept lane its rank inside the
// chunk, a prefix over the (at most 16) chunk counts gives the chunk's base.
// With PRUNED_TAIL the pruned positions follow in idx[n..N), ascending (a
// pruned token j with r kept tokens before it goes to n + j - r).
// Optionally stores rank[j] (-1 for a pruned token) and the per-chunk
// ballots.  `cnt` holds one int per 64-token chunk.  Idx is int32_t or
// uint16_t (positions are below 1024).  Contains two LDS-only barriers
// (loads and stores of the caller still in flight are not waited for);
// every thread must call it.
template <int NT, typename Idx = int32_t, bool PRUNED_TAIL = false>
__device__ int compact_bytes(const uint8_t (&mb)[compact_per<NT>()], int N, Idx* idx,
                             int32_t* rank, uint64_t* ballots, int32_t* cnt) {
  constexpr int W = NT / 64;
  constexpr int PER = compact_per<NT>();
  const int lane = lane_id(), w = wave_id();
  const int nchunks = (N + 63) >> 6;
  uint64_t bal[PER];
  bool keep[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = w + i * W;
    keep[i] = (c < nchunks) && (mb[i] != 0);
    bal[i] = __ballot(keep[i]);
    if (c < nchunks && lane == 0) {
      cnt[c] = __popcll(bal[i]);
      if (ballots) ballots[c] = bal[i];
    }
  }
  lds_barrier();
  int n = 0;
  for (int c = 0; c < nchunks; ++c) n += cnt[c];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = w + i * W;
    if (c < nchunks) {
      int base = 0;
      for (int cc = 0; cc < c; ++cc) base += cnt[cc];
      const int j = c * 64 + lane;
      const int r = base + __popcll(bal[i] & lanemask_lt());
      if (keep[i])
        idx[r] = (Idx)j;
      else if (PRUNED_TAIL && j < N)
        idx[n + j - r] = (Idx)j;
      if (rank && j < N) rank[j] = keep[i] ? r : -1;
    }
  }
  lds_barrier();
  return n;
}

template <int NT, typename Idx = int32_t, bool PRUNED_TAIL = false>
__device__ int compact_row(const uint8_t* __restrict__ mrow, int N, Idx* idx, int32_t* rank,
                           uint64_t* ballots, int32_t* cnt) {
  uint8_t mb[compact_per<NT>()];
  mask_row_bytes<NT>(mrow, N, mb);
  return compact_bytes<NT, Idx, PRUNED_TAIL>(mb, N, idx, rank, ballots, cnt);
}

}  // namespace rva
