/*
 * rva_probe.h -- ceiling probes of librva.so (measurement only, not part of
 * the attention path): the bandwidth a plain streaming kernel, the
 * attention's own access pattern without arithmetic, and the matrix-core
 * rate a plain fp16 product loop reach on this device, so that the
 * attention kernels' fractions of "achievable" rest on kernels of known
 * construction.  Same conventions as rva.h: device pointers owned by the
 * caller, stream-ordered, no allocation, status codes, all checks before
 * anything is enqueued.
 */
#ifndef RVA_PROBE_H
#define RVA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * rva_probe_copy -- copy `bytes` (a multiple of 16, > 0) from src to dst
 * (16-byte aligned, not overlapping) with `grid` workgroups of 256 threads,
 * 16-byte non-temporal loads and stores over a grid-stride loop (4
 * workgroups per compute unit measured best).
 */
int rva_probe_copy(const void* src, void* dst, long long bytes, int grid, void* stream);

/*
 * rva_probe_read -- read `bytes` (a multiple of 16, > 0) of src (16-byte
 * aligned) with `grid` workgroups of 256 threads, four 16-byte
 * non-temporal loads in flight per thread (2 workgroups per compute unit
 * measured best); each thread folds what it read into one word written to
 * sink (uint32, grid * 256 entries).
 */
int rva_probe_read(const void* src, uint32_t* sink, long long bytes, int grid, void* stream);

/*
 * rva_probe_mfma -- `iters` rounds of 8 independent 16x16x32 fp16 matrix-core
 * products per wave on register operands, `grid` workgroups of 4 waves
 * (8 workgroups per compute unit, 8 waves per SIMD, measured best);
 * one float per thread to out (grid * 256 entries).  *flops (if not NULL)
 * receives the floating-point operations the launch performs.
 */
int rva_probe_mfma(int iters, float* out, int grid, void* stream, long long* flops);

/*
 * rva_probe_gather -- the HBM traffic of rva_fused with none of its
 * arithmetic, on the same tensors: q, k, v, o padded [B, N, H, 64] with
 * 2-byte elements (16-byte aligned), mask uint8 [B, N], and cu_seqlens
 * (int32 [B + 1]) and kept_index (int32, capacity B * N: entry cu[b] + r
 * holds b * N + j of the r-th kept token of image b) as rva_pack gives them
 * for that mask.  One workgroup of 256 threads per (image, head pair): every
 * kept row's head-pair slice of q, k and v is read, and o's slice of every
 * row written (kept rows: the bitwise XOR of the three; pruned rows: zero),
 * the bytes rva_fused reads and writes, with non-temporal loads and stores
 * (the fastest cache policy for this pattern measured).  Rows and counts outside the tensors are skipped.  Timed
 * beside rva_fused on the same batch it tells how much of the attention's
 * time its access pattern alone takes on this device.  B, N, H as rva_fused.
 */
int rva_probe_gather(const void* q, const void* k, const void* v, void* o, const uint8_t* mask,
                     const int32_t* cu_seqlens, const int32_t* kept_index, int B, int N, int H,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RVA_PROBE_H */
