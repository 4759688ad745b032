/*
 * rva.h -- C ABI of the ragged ViT attention library (librva.so), gfx950 only.
 *
 * The library implements the pack -> ragged bidirectional attention -> unpack
 * path for token-pruned Vision Transformers described in "Dispatch-Aware
 * Ragged Attention for Pruned Vision Transformers" (Abdellatif and Almasri,
 * arXiv 2604.15408).  The sota2.com page's Abstract frames the pipeline:
 * after pruning, each image keeps a different number of tokens; those tokens
 * are packed back to back, attention runs over each image's tokens only, and
 * the result returns to the padded layout.  The aissential.tech summary's
 * "Method" section splits the packer into a small index-building phase and a
 * gather phase.  The same Abstract identifies per-call host dispatch as the
 * dominant cost at these short lengths, which is why this ABI also offers a
 * single fused launch and captured launch plans.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    owned by the caller; the library never allocates or frees them.
 *    Data pointers must be 16-byte aligned, int32 pointers 4-byte aligned.
 *  - Padded layout: [B, N, H, d] row-major (token-major, heads inside a
 *    token row).  Packed layout: [T, H, d] with T = sum of kept counts.
 *    d (head_dim) must be 64.
 *  - mask: uint8 [B, N], nonzero = token kept.  Any image may keep 0..N
 *    tokens.  Kept tokens are packed in ascending token order.
 *  - cu_seqlens: int32 [B+1], cu[0] = 0, cu[b+1] = cu[b] + n_b (the
 *    offsets convention of variable-length attention APIs such as the
 *    FlashAttention-2 varlen interface the Abstract compares against).
 *  - kept_index: int32 [T], entry cu[b] + r holds b*N + j for the r-th kept
 *    token j of image b.
 *  - dtype: RVA_F32 (IEEE binary32), RVA_F16 (binary16) or RVA_BF16
 *    (bfloat16).  Outputs have the input dtype.  Attention accumulates and
 *    normalises in fp32; 16-bit inputs use 16-bit matrix-core products with
 *    fp32 accumulation, fp32 inputs use fp32 matrix-core products.
 *  - stream: a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work: no host synchronisation, no device-to-host
 *    copy, no allocation; results are valid once the stream reaches them.
 *  - softmax_scale <= 0 (or NaN) selects 1/sqrt(d).
 *  - Errors: every function returns an rva_status.  All argument checks run
 *    before anything is enqueued, so a call that fails validation launches
 *    nothing.  RVA_ERR_HIP reports a HIP runtime failure; rva_last_error()
 *    then holds the runtime's message (thread-local).
 *  - Limits: 1 <= B, 1 <= N <= RVA_MAX_TOKENS, 1 <= H <= RVA_MAX_HEADS,
 *    B * N < 2^31.
 */
#ifndef RVA_H
#define RVA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RVA_MAX_TOKENS 1024
#define RVA_MAX_HEADS 64
#define RVA_HEAD_DIM 64
#define RVA_MAX_CHANNELS 65536

typedef enum { RVA_F32 = 0, RVA_F16 = 1, RVA_BF16 = 2 } rva_dtype;

typedef enum {
  RVA_OK = 0,
  RVA_ERR_INVALID = -1,     /* a pointer, size, alignment or dtype is invalid */
  RVA_ERR_UNSUPPORTED = -2, /* valid request outside what is built (d != 64)   */
  RVA_ERR_HIP = -3          /* the HIP runtime reported an error               */
} rva_status;

/*
 * rva_pack -- kept counts, offsets and the packed gather (both packer phases
 * of the aissential.tech summary's "Method").
 *
 * Computes n_b, cu_seqlens and max_seqlen from mask, then copies the kept
 * token rows of each non-NULL padded input into its packed output (bit copy).
 *   q_pad/k_pad/v_pad : [B,N,H,d] inputs; any may be NULL, and then the
 *                       matching *_out must be NULL too (and is skipped).
 *   q_out/k_out/v_out : [T,H,d] outputs; capacity of at least T rows (B*N
 *                       rows always suffices).
 *   cu_seqlens        : int32[B+1] output (required).
 *   max_seqlen        : int32[1] output, may be NULL.
 *   kept_index        : int32[T] output, may be NULL.
 * Two kernel launches: a one-workgroup count/prefix-sum, then the gather.
 */
int rva_pack(const void* q_pad, const void* k_pad, const void* v_pad, const uint8_t* mask,
             int B, int N, int H, int d, int dtype,
             void* q_out, void* k_out, void* v_out,
             int32_t* cu_seqlens, int32_t* max_seqlen, int32_t* kept_index, void* stream);

/*
 * rva_ragged_attend -- bidirectional attention over each packed sequence
 * (the sota2.com Abstract's ragged attention kernel; non-causal).
 *
 * For every image b and head h: O = softmax(Q K^T * scale) V over rows
 * cu[b]..cu[b+1]-1 of q/k/v ([T,H,d]), written to o ([T,H,d], capacity T).
 *   max_seqlen : host-side bound on every n_b, at most RVA_MAX_TOKENS.  It
 *                only sizes the on-chip staging and the launch; any value
 *                >= 1 gives correct results (longer sequences are streamed
 *                in chunks), the true maximum gives the best speed.  <= 0
 *                means RVA_MAX_TOKENS.
 * Every n_b must be at most RVA_MAX_TOKENS (the offsets are device data and
 * are not read on the host): a longer sequence is outside the contract and
 * its output rows are left unwritten.
 * One kernel launch: a workgroup per (sequence, head), or per query tile of
 * one when that leaves compute units idle (rva_set_query_split).
 */
int rva_ragged_attend(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                      int B, int H, int d, int max_seqlen, float softmax_scale, int dtype,
                      void* o, void* stream);

/*
 * rva_unpack -- packed rows back to the padded layout (the Abstract's
 * "unpack").  o_pad[b, j] = o_packed[cu[b] + r] for the r-th kept token j of
 * image b; pruned positions are written as +0.  Every padded row is written
 * exactly once.  One kernel launch.
 */
int rva_unpack(const void* o_packed, const int32_t* cu_seqlens, const uint8_t* mask,
               int B, int N, int H, int d, int dtype, void* o_pad, void* stream);

/*
 * rva_fused -- the whole pack -> attend -> unpack path in ONE kernel launch
 * (the Abstract's dispatch-floor argument taken to its end: padded in,
 * padded out, no packed intermediate in memory).
 *   o_pad      : [B,N,H,d] output; pruned positions are +0.
 *   cu_seqlens : int32[B+1] output or NULL; max_seqlen: int32[1] or NULL.
 *                When either is given, one extra workgroup of the same launch
 *                computes them.
 *   max_seqlen_hint : as rva_ragged_attend's max_seqlen (<= 0 means N).
 * Results are identical to rva_pack + rva_ragged_attend + rva_unpack when
 * both launches take the same work decomposition (rva_set_query_split);
 * otherwise they agree within the same error bounds.
 */
int rva_fused(const void* q_pad, const void* k_pad, const void* v_pad, const uint8_t* mask,
              int B, int N, int H, int d, int max_seqlen_hint, float softmax_scale, int dtype,
              void* o_pad, int32_t* cu_seqlens, int32_t* max_seqlen, void* stream);

/*
 * rva_fused_persistent -- rva_fused as a persistent grid: as many workgroups
 * as stay resident, each pulling rva_fused's work items (an image's head
 * pair, or one head of a tail image) from a device counter, one item ahead,
 * and running them with rva_fused's per-item code.  Same arguments as
 * rva_fused, and the same results bit for bit as rva_fused with one
 * workgroup per (image, head) (16-bit inputs; fp32 falls back to rva_fused
 * itself); small launches that rva_fused runs in the key-split form
 * (rva_set_query_split) agree within the same error bounds.  Plus:
 *   work : int32[2] device scratch, all zero before the first call.  Every
 *          call leaves it zero again when it completes, so one buffer serves
 *          any number of stream-ordered calls.  Only one call may be in
 *          flight on a buffer: two overlapping calls (different streams)
 *          share item indices and the reset, so each computes part of the
 *          items and output rows stay unwritten, silently.  Calls that may
 *          run at the same time need distinct buffers.
 * Limits: as rva_fused, and B * H < 2^30, so that the 32-bit work counter
 * (which reaches the item count plus the resident workgroups) cannot wrap
 * (RVA_ERR_INVALID otherwise, checked before anything is enqueued).
 */
int rva_fused_persistent(const void* q_pad, const void* k_pad, const void* v_pad,
                         const uint8_t* mask, int B, int N, int H, int d, int max_seqlen_hint,
                         float softmax_scale, int dtype, void* o_pad, int32_t* cu_seqlens,
                         int32_t* max_seqlen, int32_t* work, void* stream);

/*
 * rva_fused_persistent_noalloc -- rva_fused_persistent for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * and harnesses that forbid hipMalloc): the same arguments without `work`,
 * and the same results bit for bit.  The work counter pair lives in a
 * 256-byte array of static device memory inside the library (one copy per
 * GPU, held until the process ends), of which a call uses 8 bytes whatever
 * B, N and H are.  Nothing is allocated: no hipMalloc, hipFree or
 * allocating library call.  The first call on a GPU also enqueues a
 * one-workgroup fill kernel that zeroes the counter; every completed call
 * leaves it zero for the next.  All calls on one GPU share that counter, so
 * calls that may overlap on one GPU (different streams, or graphs replayed
 * concurrently) race and leave output rows unwritten: order them on one
 * stream.  Limits: as rva_fused_persistent (B * H < 2^30, RVA_ERR_INVALID
 * otherwise, checked before anything is enqueued, the first call's fill
 * kernel included).
 */
int rva_fused_persistent_noalloc(const void* q_pad, const void* k_pad, const void* v_pad,
                                 const uint8_t* mask, int B, int N, int H, int d,
                                 int max_seqlen_hint, float softmax_scale, int dtype, void* o_pad,
                                 int32_t* cu_seqlens, int32_t* max_seqlen, void* stream);

/*
 * rva_threshold_l2_mask -- the Threshold-l2 keep-mask that feeds the path
 * (one of the four pruning algorithms the aissential.tech summary lists in
 * its "Summary"; the pages give no definition, the reading below is this
 * library's).
 *
 * Per image: token 0 (CLS) is kept; patch token j (1 <= j < N) is kept when
 * the L2 norm of its embedding row x[b, j, :] reaches the keep_quantile-th
 * quantile (linear interpolation) of the image's N - 1 patch norms.  In
 * exact arithmetic that keeps the patches whose norm is at least the r0-th
 * smallest patch norm (0-based), r0 = ceil(keep_quantile * (N - 2)), which is
 * the form evaluated: with distinct norms exactly N - 1 - r0 patches are
 * kept; equal norms are kept or dropped together.  Decisions are taken on
 * squared norms in fp64, summed in channel order c = 0..C-1 (each square is
 * exact in fp64), so they are reproducible bit for bit.
 *   x        : [B, N, C] row-major embeddings in `dtype` (16-byte aligned);
 *              C * element size must be a multiple of 16 bytes,
 *              1 <= C <= RVA_MAX_CHANNELS.
 *   keep_quantile : in [0, 1]; 0 keeps every patch, 1 only the largest.
 *   mask_out : uint8 [B, N] output (1 = keep, 0 = prune).
 * One kernel launch of B workgroups.
 */
int rva_threshold_l2_mask(const void* x, int B, int N, int C, int dtype, double keep_quantile,
                          uint8_t* mask_out, void* stream);

/*
 * Projections on the packed rows -- the two dense products of a ViT attention
 * block, run on the T kept rows only.  The aissential.tech summary's
 * "Method" has the packer feed the whole block, and its "In practice" asks
 * for attention and the rest of the block to be timed apart; the pages give
 * no formula, so these are the standard block's affine maps (nn.Linear
 * layout: weight [out, in], y = x W^T + b).  fp16 and bf16 only (fp32
 * returns RVA_ERR_UNSUPPORTED); 16-bit matrix-core products with fp32
 * accumulation, bias and residual added in fp32, one rounding to the dtype.
 * C = H * 64 with 1 <= H <= RVA_MAX_HEADS; B*N*C*2 < 2^31.  T is read on the
 * device from cu_seqlens[B]: no host synchronisation, and every buffer
 * indexed by packed row has a capacity of B*N rows.
 *
 * rva_qkv_projection: [q | k | v] = x_r W_qkv^T + b_qkv for packed rows r.
 *   x          : with kept_index, padded embeddings [B, N, C] and row r is
 *                x[kept_index[r]] (the pack's gather, fused); with
 *                kept_index NULL, packed rows [T, C].
 *   w_qkv      : [3C, C]; b_qkv: [3C] or NULL.
 *   q, k, v    : packed outputs [T, C] = [T, H, 64] each (weight rows
 *                0..C-1, C..2C-1 and 2C..3C-1).
 * One kernel launch.
 */
int rva_qkv_projection(const void* x, const int32_t* kept_index, const int32_t* cu_seqlens,
                       int B, int N, int C, const void* w_qkv, const void* b_qkv, int dtype,
                       void* q, void* k, void* v, void* stream);

/*
 * rva_out_projection: y_r = o_r W_o^T + b_o (+ residual) for packed rows r.
 *   o          : packed [T, C] (the attention output).
 *   w_o        : [C, C]; b_o: [C] or NULL.
 *   kept_index : with it, y and residual are padded [B, N, C]: row r goes to
 *                y[kept_index[r]] and every row whose mask byte is 0 is
 *                written as +0 (the unpack, fused; mask required); without
 *                it, y and residual are packed [T, C].
 *   residual   : added before rounding, or NULL.  It may be the same buffer
 *                as y (in-place residual update).
 * One kernel launch.
 */
int rva_out_projection(const void* o, const int32_t* kept_index, const int32_t* cu_seqlens,
                       const uint8_t* mask, int B, int N, int C, const void* w_o,
                       const void* b_o, const void* residual, int dtype, void* y, void* stream);

/*
 * Launch plans -- capture once, replay with one graph launch per call (the
 * Abstract's per-call dispatch floor is what this removes).
 *
 * mode RVA_PLAN_STAGED : rva_pack, rva_ragged_attend, rva_unpack (4 kernels).
 *      RVA_PLAN_FUSED  : rva_fused (1 kernel).
 *      RVA_PLAN_EMPTY  : one empty one-workgroup kernel (measures the floor).
 *      RVA_PLAN_L2_FUSED : rva_threshold_l2_mask from x into mask_out, then
 *                        rva_fused reading mask_out (2 kernels); `mask` is
 *                        ignored.
 *      RVA_PLAN_PERSISTENT : rva_fused_persistent (1 kernel); the plan owns
 *                        its work counter (8 bytes of device memory,
 *                        allocated and zeroed at creation, freed at destroy),
 *                        so one launch of the plan may be in flight at a
 *                        time (launches on one stream).
 *      RVA_PLAN_FUSED_DIRECT : rva_fused (1 kernel) without a graph: the
 *                        arguments are validated once at creation and each
 *                        rva_plan_launch enqueues the kernel directly, which
 *                        on ROCm costs less than a one-kernel graph launch.
 *                        Nothing is captured or allocated on the device.
 * Every pointer and size is fixed at creation; the CONTENTS of the inputs
 * (including the mask) may change between launches.  Staged mode needs the
 * packed scratch buffers q/k/v/o_packed (capacity B*N rows each) and
 * cu_seqlens; kept_index and max_seqlen may be NULL.  Fused mode ignores the
 * packed buffers; cu_seqlens and max_seqlen may be NULL.
 * rva_plan_create validates like the direct calls, captures on a private
 * stream and instantiates a HIP graph (host-side allocation by the runtime);
 * rva_plan_launch enqueues one graph launch on `stream` (a direct kernel
 * launch in RVA_PLAN_FUSED_DIRECT mode).
 */
typedef enum {
  RVA_PLAN_STAGED = 0,
  RVA_PLAN_FUSED = 1,
  RVA_PLAN_EMPTY = 2,
  RVA_PLAN_L2_FUSED = 3,
  RVA_PLAN_PERSISTENT = 4,
  RVA_PLAN_FUSED_DIRECT = 5
} rva_plan_mode;

typedef struct {
  int mode;
  int B, N, H, d, dtype;
  int max_seqlen_hint;
  float softmax_scale;
  const void* q_pad;
  const void* k_pad;
  const void* v_pad;
  const uint8_t* mask;
  void* q_packed;
  void* k_packed;
  void* v_packed;
  void* o_packed;
  int32_t* cu_seqlens;
  int32_t* max_seqlen;
  int32_t* kept_index;
  void* o_pad;
  /* keep-mask stage (RVA_PLAN_L2_FUSED): as rva_threshold_l2_mask */
  const void* x;
  int C;
  int x_dtype;
  double keep_quantile;
  uint8_t* mask_out;
} rva_plan_desc;

typedef struct rva_plan_s* rva_plan;

int rva_plan_create(const rva_plan_desc* desc, rva_plan* out);
int rva_plan_launch(rva_plan plan, void* stream);
int rva_plan_destroy(rva_plan plan);

/*
 * Multi-layer plan -- the dispatch argument of the sota2.com Abstract carried
 * over a stack of layers: ONE pack, then for each of `layers` attention
 * sub-layers the QKV projection, the ragged attention and the output
 * projection (residual added in place on the packed stream), then ONE
 * unpack, all captured as a single graph.  Every layer reuses the same
 * cu_seqlens (pruning is fixed across the stack: the pages do not say
 * otherwise).  Layer normalisation and the MLP sub-layer are not part of it.
 *   x_pad      : [B, N, C] embeddings, C = H * 64; mask: [B, N].
 *   w_qkv[l], w_o[l] : host arrays of `layers` device pointers ([3C, C] and
 *                [C, C]); b_qkv / b_o may be NULL, or arrays whose entries
 *                may be NULL.  The arrays are read at creation only.
 *   resid, q, k, v, o : packed scratch, [B*N, C] each (capacity).
 *   cu_seqlens, kept_index : required scratch ([B+1], [B*N]); max_seqlen
 *                may be NULL.
 *   y_pad      : [B, N, C] output: the residual stream after the last layer
 *                at kept positions, +0 at pruned ones.
 * fp16 / bf16 only.  Launch and destroy with rva_plan_launch / rva_plan_destroy.
 */
typedef struct {
  int B, N, H, d, dtype, layers;
  int max_seqlen_hint;
  float softmax_scale;
  const void* x_pad;
  const uint8_t* mask;
  const void* const* w_qkv;
  const void* const* b_qkv;
  const void* const* w_o;
  const void* const* b_o;
  void* resid;
  void* q;
  void* k;
  void* v;
  void* o;
  int32_t* cu_seqlens;
  int32_t* max_seqlen;
  int32_t* kept_index;
  void* y_pad;
} rva_layers_desc;

#define RVA_MAX_LAYERS 64

int rva_layers_plan_create(const rva_layers_desc* desc, rva_plan* out);

/*
 * rva_set_query_split -- how the attention launches of this process split
 * each (sequence, head) into query tiles, one workgroup per tile.  The
 * default, 0, lets every launch choose from the device's compute units and
 * its length bound: fp32 takes one tile per 16-query block; 16-bit launches
 * with fewer (sequence, head) items than resident workgroup slots take as
 * many tiles as fill the slots (at most one 16-query block per wave) or,
 * when one tile per 16-query block still fits one fill of the slots (and
 * the sequences are staged whole), the key-split form: one block per
 * workgroup, its key tiles split over the workgroup's waves and their
 * partial results combined (the same attention in another order of
 * summation); larger launches take one workgroup per (sequence, head), or
 * per head pair.
 * split >= 1 forces that many tiles (at most one per 16-query block of the
 * length bound; 1 also turns head pairing off) on every later launch and
 * plan creation, except the persistent forms.  It exists for tests and
 * tuning (a forced split never takes the key-split form): results stay
 * within the same error bounds, identical bit for bit across forced splits
 * for fp32 and for 16-bit sequences staged whole; a sequence streamed in key
 * chunks may differ in its last bits, because the chunk order of a query
 * block depends on which pass of its workgroup runs it.  RVA_ERR_INVALID
 * for split < 0.
 */
int rva_set_query_split(int split);

/*
 * rva_empty -- enqueue `count` launches of an empty one-workgroup kernel on
 * `stream` through the same launch path as the entry points above; used to
 * measure the per-launch dispatch floor the Abstract discusses.
 */
int rva_empty(int count, void* stream);

/* Static description of a status code; never NULL. */
const char* rva_status_string(int status);
/* Thread-local detail of the last failure on this thread ("" if none). */
const char* rva_last_error(void);
/* Library ABI version (major * 10000 + minor * 100 + patch). */
int rva_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RVA_H */
