/*
 * rva_probe.h -- ceiling probes of librva.so (measurement only, not part of
 * the attention path): the bandwidth a plain streaming kernel and the
 * matrix-core rate a plain fp16 product loop reach on this device, so that
 * the attention kernels' fractions of "achievable" rest on kernels of known
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

#ifdef __cplusplus
}
#endif

#endif /* RVA_PROBE_H */
