/*
 * attn_prefix.h -- C ABI of the prefix-masked / split-KV attention library
 * (libattnprefix.so, HIP kernels for gfx950 / MI355X).
 *
 * The operation.  Each batch element b has a key-padding mask whose valid keys
 * are exactly the first n_b = kv_len[b] rows.  Masking the other keys is the
 * same as cutting k and v down to their first n_b rows and attending with no
 * mask at all (page "Rewrite prefix key-padding masks as k/v truncation to keep
 * SDPA on the flash path (PyTorch)", tabfm PR #80, section Fix; a ragged mask,
 * one n_b per element, equals per-element truncated forwards, section Tests).
 * A prefix mask is therefore carried as one length per batch element instead
 * of a dense mask (page "Add sequence-parallel multi-GPU inference (PyTorch and
 * JAX) and a cuDNN flash attention option", tabfm PR #81, section cuDNN flash
 * attention).  For every (b, h, query row i):
 *
 *     out[b,h,i,:] = sum_{j < n_b} softmax_j(scale * q_i . k_j) * v_j
 *     lse[b,h,i]   = ln sum_{j < n_b} exp(scale * q_i . k_j)       (natural log)
 *
 * and n_b = 0 gives out = 0, lse = -inf.  The kernels read only the first n_b
 * key rows (padded slots cost no bandwidth and their contents, even NaN, never
 * reach a result), keep the softmax in fp32 and never form the [T_q, n] score
 * matrix.  The split-KV form computes normalized partials over fixed key
 * chunks and merges them exactly with log-sum-exp weights (PR #81, section
 * Sequence-parallel inference).
 *
 * Layout.  Row-major, D fastest, no strides:
 *     q, out     [B, H, Tq, D]
 *     k, v       [B, H, S, D]      S = allocated key slots, 0 <= n_b <= S
 *     lse        [B, H, Tq]        fp32
 *     part_out   [B, H, C, Tq, D]  fp32, C = attn_splitkv_num_chunks(S, chunk)
 *     part_lse   [B, H, C, Tq]     fp32
 *     kv_len     [B]               int32
 *
 * Pointers.  Every tensor pointer is a DEVICE pointer (HIP memory of the
 * current device); `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Calls only enqueue work on `stream` and return; buffers must stay
 * alive until that work completes.  The caller owns every buffer: the library
 * allocates no memory, keeps no caller pointer after a call returns and holds no
 * mutable global state, so calls are re-entrant.  The one exception is
 * attn_prefix_bwd_noalloc, whose workspace is a device array of the library
 * shared by every call on a GPU (see there).
 *
 * Errors.  Every call validates its arguments on the host BEFORE any HIP call
 * and returns a status code; no call ever falls back to another algorithm.
 * kv_len values live on the device and cannot be checked without a sync: the
 * kernels clamp n_b into [0, S] (so memory stays safe), and values outside
 * that range are a caller error with unspecified results.  A failed launch
 * returns ATTN_ERR_HIP.
 *
 * Limits.  D in {64, 128, 256}; dtype bf16 or fp32 (inputs and `out` share
 * it); S * D * sizeof(dtype) < 2^31 per (b, h); every launch within the 32-bit
 * work-item count of a 1-D dispatch: B * H * ceil(Tq / 128) [* C] workgroups
 * of 256 threads at most 2^24 - 1 for the forward and split calls (the same
 * bound on ceil(B*H*Tq*D / 1024) for the merge, and on ceil(B*H*Tq*D / 2048),
 * B * H * ceil(Tq / 128) and B * H * ceil(S / 128) for the backward; B at most
 * 2^23 - 1 rows for the mask call; B * H * ceil(Tq / 256) workgroups of 512
 * threads at most 2^23 - 1 where the forward takes eight wavefronts per
 * workgroup).  Larger calls return ATTN_ERR_SHAPE before any launch; size
 * checks come before pointer checks (the eight-wave bound after them, since
 * the kernel is chosen only then).  Zero B, H or Tq is a no-op
 * returning ATTN_OK (then the tensor pointers may be NULL); S = 0 is legal
 * (every n_b is 0) and then k and v may be NULL.
 */
#ifndef ATTN_PREFIX_H
#define ATTN_PREFIX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULLPTR = 1,      /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,        /* a negative size, or a size beyond the limits above */
  ATTN_ERR_DTYPE = 3,        /* dtype is not one of attn_dtype_t */
  ATTN_ERR_UNSUPPORTED = 4,  /* head dim or dtype not supported by this call */
  ATTN_ERR_ALIGN = 5,        /* a tensor pointer is not 16-byte aligned */
  ATTN_ERR_CHUNK = 6,        /* chunk <= 0 or not a multiple of 64 */
  ATTN_ERR_HIP = 7,          /* the HIP runtime reported an error at launch */
  ATTN_ERR_ARG = 8           /* a scalar argument is out of range (e.g. non-finite scale) */
} attn_status_t;

typedef enum { ATTN_BF16 = 0, ATTN_F32 = 1 } attn_dtype_t;

/* Library version as (major << 16) | (minor << 8) | patch. */
int attn_version(void);

/* Fused prefix-masked attention forward.
 * Defined by the truncation identity of tabfm PR #80 (section Fix) and the
 * per-element (ragged) form of its section Tests; kv_len plays the role of the
 * sequence lengths of PR #81 (section cuDNN flash attention).
 *   q, k, v  : device, dtype, layouts above (k, v: only rows j < n_b are read)
 *   kv_len   : device int32 [B]
 *   scale    : softmax scale (e.g. 1/sqrt(D)); must be finite
 *   out      : device, dtype, [B,H,Tq,D]; every element is written
 *   lse      : device fp32 [B,H,Tq] natural-log LSE, or NULL to skip it
 * For bf16 at D = 256 the library picks one of two kernels (32 or 64 query rows
 * per wavefront), or both in one grid, from the launch shape and the device's
 * compute-unit count; results differ only in summation order.  At D = 128 it
 * takes the 32-row kernel, with four or (for launches that fill the GPU) eight
 * wavefronts per workgroup, which give the same bits.  The environment variable
 * ATTN_PREFIX_FWD_ROWS=128, 128x8, 256 or mixed forces a choice (testing; 128x8
 * applies at D = 64 and 128, 256 at D = 128 and 256, mixed only at D = 256).
 * Cost: the bf16 kernels read the valid keys once; a workgroup in which some row's
 * scaled scores climb more than 20 log2 units (about 14 in natural-log units)
 * above that row's maximum over its first key tile reads them a second time
 * (same result; the split-KV partials do the same per chunk).
 */
attn_status_t attn_prefix_fwd(const void* q, const void* k, const void* v, const int32_t* kv_len,
                              int B, int H, int Tq, int S, int D, float scale, attn_dtype_t dtype,
                              void* out, float* lse, void* stream);

/* Split-KV partials: for chunk c the keys [c*chunk, min((c+1)*chunk, n_b)).
 * Each partial is the normalized output O_c (fp32) with its natural-log LSE
 * L_c over that chunk's keys; an empty chunk writes O_c = 0, L_c = -inf.
 * This is one device's share of the inducing attention of tabfm PR #81
 * (section Sequence-parallel inference), cut at fixed key boundaries.
 *   chunk    : keys per chunk, a positive multiple of 64; C = ceil(S / chunk)
 *   part_out : device fp32 [B,H,C,Tq,D], fully written
 *   part_lse : device fp32 [B,H,C,Tq], fully written
 */
attn_status_t attn_splitkv_partial(const void* q, const void* k, const void* v, const int32_t* kv_len,
                                   int B, int H, int Tq, int S, int D, float scale, attn_dtype_t dtype,
                                   int chunk, float* part_out, float* part_lse, void* stream);

/* Split-KV in one launch: the partials of attn_splitkv_partial, then, inside the
 * same kernel, the merge of attn_lse_combine done by the last of the C chunk
 * workgroups of each (b, h, 128-query tile) to finish -- the partial results
 * merged with their log-sum-exp weights (tabfm PR #81, section
 * Sequence-parallel inference), without a second launch.
 *   part_out, part_lse : as for attn_splitkv_partial (caller-provided scratch;
 *                        every element is written)
 *   counters : device int32 [B, H, ceil(Tq / 128)]; must be all zero before the
 *              first call; every call leaves it all zero again.  Calls that share
 *              a counters buffer must not run concurrently.
 *   out, lse : as for attn_lse_combine, out in `dtype` (lse may be NULL)
 * The merged result is bit-identical to attn_splitkv_partial followed by
 * attn_lse_combine.  On MI355X it is slower than those two calls (7.8-8.1 ms
 * against 5.6-6.0 ms on 160 x 4 heads x 100,000 keys in 4,096-key chunks): each
 * merge is one workgroup reading partials that other XCDs' L2 caches just wrote
 * back, while the other chunks' loads stream past, and those merges cost more
 * than the second launch they save.
 * Errors as for attn_splitkv_partial, plus ATTN_ERR_NULLPTR
 * (counters or out NULL) and ATTN_ERR_ALIGN (counters/lse not 4-byte aligned,
 * out not 16-byte aligned). */
attn_status_t attn_splitkv_fwd(const void* q, const void* k, const void* v, const int32_t* kv_len, int B, int H,
                               int Tq, int S, int D, float scale, attn_dtype_t dtype, int chunk, float* part_out,
                               float* part_lse, int32_t* counters, void* out, float* lse, void* stream);

/* Exact log-sum-exp merge of C partials (tabfm PR #81, section
 * Sequence-parallel inference): with M = max_c L_c,
 *     M = -inf  ->  out = 0, lse = -inf
 *     else      ->  w_c = exp(L_c - M), out = sum_c w_c O_c / sum_c w_c,
 *                   lse = M + ln sum_c w_c.
 * Any partition works (chunks of any size, empty ones included).
 *   part_out : device fp32 [B,H,C,Tq,D]; part_lse: device fp32 [B,H,C,Tq]
 *   out      : device, out_dtype, [B,H,Tq,D]
 *   lse      : device fp32 [B,H,Tq], or NULL
 * C = 0 is legal and gives out = 0, lse = -inf.
 */
attn_status_t attn_lse_combine(const float* part_out, const float* part_lse, int B, int H, int C, int Tq,
                               int D, attn_dtype_t out_dtype, void* out, float* lse, void* stream);

/* Prefix-mask detection on the device: the step before a masked attention call
 * that the page on tabfm PR #80 (section Fix) performs on the host, and the
 * mask-to-sequence-lengths mapping of PR #81 (section cuDNN flash attention).
 *   mask       : device, B rows of S bytes (nonzero = attend); row b starts at
 *                mask + b * row_stride (bytes, row_stride >= 0; 0 repeats one row
 *                for every b); a [B,1,1,S] bool tensor is such a layout.  NULL is
 *                allowed when S = 0 (every row is then the empty prefix, n_b = 0).
 *   kv_len     : device int32 [B]; receives n_b when row b is True...True
 *                False...False (n_b = number of True entries, 0 for an all-False
 *                row) and -1 when the row is not a prefix mask.  A -1 must not
 *                reach the attention calls (they would clamp it to 0): callers
 *                check for it, which needs one host synchronization.
 * Errors: ATTN_ERR_SHAPE (negative B, S or row_stride), ATTN_ERR_NULLPTR,
 * ATTN_ERR_ALIGN (kv_len not 4-byte aligned), ATTN_ERR_HIP.  B = 0 is a no-op. */
attn_status_t attn_prefix_mask_to_kv_len(const uint8_t* mask, int B, int S, int64_t row_stride, int32_t* kv_len,
                                         void* stream);

/* Backward pass of attn_prefix_fwd: the exact gradients of the same function,
 * for training on packed batches whose elements have ragged prefix lengths
 * (tabfm PR #80, section Fix, on the masked form at pretraining time; the
 * truncation identity of the same section holds for the derivative too, so
 * padded key slots get zero gradient).  With P = softmax(scale q k^T) over j < n_b, recomputed
 * from `lse`:
 *     delta_i = sum_d dout_id out_id,  dS = P * (dout v^T - delta)
 *     dq = scale dS k,  dk = scale dS^T q,  dv = P^T dout
 *   q, k, v, kv_len, scale : as passed to attn_prefix_fwd (same layouts)
 *   out, lse   : that call's results (device; out [B,H,Tq,D] bf16, lse fp32)
 *   dout       : device bf16 [B,H,Tq,D], the gradient of out
 *   delta      : device fp32 [B,H,Tq], caller-provided workspace; receives delta
 *   dq         : device bf16 [B,H,Tq,D]; dk, dv: device bf16 [B,H,S,D]; every
 *                element is written (dk = dv = 0 on slots j >= n_b; dq = 0 for
 *                batch elements with n_b = 0)
 * Supported: dtype ATTN_BF16 with D in {64, 128, 256} (fp32 inputs return
 * ATTN_ERR_UNSUPPORTED).  Three kernels are enqueued on `stream`
 * (delta, dq, dk/dv); no atomics, so results are deterministic.  Tq = 0 zeroes
 * dk and dv; S = 0 zeroes dq. */
attn_status_t attn_prefix_bwd(const void* q, const void* k, const void* v, const int32_t* kv_len, const void* out,
                              const void* dout, const float* lse, int B, int H, int Tq, int S, int D, float scale,
                              attn_dtype_t dtype, float* delta, void* dq, void* dk, void* dv, void* stream);

/* attn_prefix_bwd without the `delta` workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight training loops, harnesses that
 * forbid hipMalloc.  The same computation, arguments and results as attn_prefix_bwd;
 * delta lives instead in a device array of the library, 16 MiB per GPU, which every
 * GPU the library runs on holds from the library's load to the end of the process.
 * The call allocates nothing and sets no memory (delta is written in full before it
 * is read).  Limit: B * H * Tq <= 4,194,304 rows, else ATTN_ERR_SHAPE before any HIP
 * call.  Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (on different streams, or from different host threads without ordering)
 * race on it and must be serialized by the caller.  The first call on a device looks
 * up the array's device address (ATTN_ERR_HIP if that fails). */
attn_status_t attn_prefix_bwd_noalloc(const void* q, const void* k, const void* v, const int32_t* kv_len,
                                      const void* out, const void* dout, const float* lse, int B, int H, int Tq,
                                      int S, int D, float scale, attn_dtype_t dtype, void* dq, void* dk, void* dv,
                                      void* stream);

/* Host helper: number of chunks ceil(S / chunk); -1 if chunk <= 0 or S < 0. */
int attn_splitkv_num_chunks(int S, int chunk);

/* Host helper: static, human-readable text for a status code. */
const char* attn_status_string(attn_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PREFIX_H */
