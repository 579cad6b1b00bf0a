/*
 * libfa355: fused no-KV-cache multi-head attention forward for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation is mo.mha.no_cache as the "FlashAttentionGPU" API page
 * (max.modular.com) defines it, section "execute", Steps 0-4:
 *
 *     answer = softmax(mask(scale * Q K^T)) V
 *
 * with Q, K, V and the answer read and written in BSHD, the BSHD<->BHSD
 * transposes folded into the kernel's addressing, and the softmax
 * evaluated as an online (FlashAttention-2) reduction over key tiles, so the
 * S x S score matrix is never stored.
 *
 * C ABI only: plain pointers and sizes, no C++ or framework types. All
 * functions are thread-safe; the library keeps no per-call state (only
 * per-device caches of the architecture check and of how many workgroups
 * the device holds at once) and allocates no device memory.
 */
#ifndef FA355_H
#define FA355_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and out (all four share it). */
typedef enum {
    FA355_F32 = 0,  /* IEEE binary32; products and sums in fp32 */
    FA355_BF16 = 1, /* bfloat16; fp32 accumulation */
    FA355_F16 = 2   /* IEEE binary16; fp32 accumulation */
} fa355_dtype;

/*
 * Mask functor applied to the scaled scores (Step 3 of the page's "execute"
 * section; the page's mask_str / dispatch_mask selects it). Key j is
 * visible to query i iff:
 *   FA355_MASK_NONE:            always;
 *   FA355_MASK_CAUSAL:          j <= i;
 *   FA355_MASK_SLIDING_WINDOW:  i - window < j <= i  (the query sees exactly
 *                               `window` keys, itself included; the page's
 *                               local_window_size parameter, read as a causal
 *                               sliding window).
 * Hidden scores get probability exactly 0.
 */
typedef enum {
    FA355_MASK_NONE = 0,
    FA355_MASK_CAUSAL = 1,
    FA355_MASK_SLIDING_WINDOW = 2
} fa355_mask;

typedef enum {
    FA355_OK = 0,
    FA355_ERR_INVALID_ARG = 1, /* bad pointer, size, enum, window or overlap */
    FA355_ERR_UNSUPPORTED = 2, /* valid but not built: head dim, alignment, size */
    FA355_ERR_DEVICE = 3,      /* no current HIP device, or it is not gfx950 */
    FA355_ERR_LAUNCH = 4       /* the HIP launch itself failed */
} fa355_status;

/*
 * mha_no_cache: out = softmax(mask(scale * q k^T)) v, per batch and head.
 *
 * Arguments (all device pointers on the current HIP device, contiguous):
 *   out  [B, S, H,   D]  written; shaped like q (the page's "Args"
 *                        section fixes the shape) and of q's dtype.
 *   q    [B, S, H,   D]  queries, BSHD.
 *   k    [B, S, Hkv, D]  keys, BSHD, or BShD with Hkv < H for grouped
 *                        attention (page, grouped attention, "Step -1").
 *   v    [B, S, Hkv, D]  values, in k's layout: the page's grouped
 *                        attention section requires k and v to carry the
 *                        same head count.
 *   B, S, H, Hkv, D      batch, sequence length (queries and keys: there is
 *                        no cache), query heads, K/V heads, head dim.
 *                        H must be a multiple of Hkv; query head h reads
 *                        K/V head h / (H / Hkv) (contiguous groups, the
 *                        reading taken of the page's "G groups").
 *   scale                multiplies q.k before the mask (page, Step 3);
 *                        any finite value with |scale| * log2(e) within
 *                        the fp32 range (|scale| up to about 2.36e38), 0 and
 *                        negatives included. The kernels form each
 *                        exponent in fp32 as (q.k) * |scale| * log2(e)
 *                        minus the row's running maximum with one fused
 *                        multiply-add, so every |scale * q.k| * log2(e)
 *                        must stay below 2^24 (about 1.7e7): beyond that
 *                        the rounding of the maximum alone exceeds one
 *                        unit of the exponent, and the result is outside
 *                        the contract (undefined).
 *   mask_kind            an fa355_mask value.
 *   window               sliding-window width (>= 1) for
 *                        FA355_MASK_SLIDING_WINDOW; ignored otherwise.
 *   dtype                an fa355_dtype value.
 *   stream               a hipStream_t, or NULL for the null stream; stands
 *                        in for the page's DeviceContext.
 *
 * Supported today: D in {32, 64, 128, 256}; any S >= 1 (ragged tails are
 * masked); all three dtypes. Pointers must be 16-byte aligned; out must not overlap
 * q, k or v. Offsets across tokens, heads and batches are 64-bit, so q, k,
 * v and out may be of any size; only one token's row of q (H * D
 * elements) is limited, to 16 MiB, because offsets inside one tile are
 * 32-bit.
 *
 * Ownership: the caller owns every buffer; the library reads q, k, v and
 * writes every element of out, and allocates nothing.
 *
 * Execution: asynchronous, ordered on `stream`; returns once the kernel is
 * enqueued. The result is deterministic (no atomics): the same inputs give
 * the same bits on every run.
 *
 * Errors: returns an fa355_status and never aborts. Argument checks run
 * before any HIP call, so an invalid call touches no device state:
 * FA355_ERR_INVALID_ARG for a null pointer, a size < 1, H % Hkv != 0, an
 * unknown dtype or mask, window < 1 with the sliding mask, a non-finite
 * scale or one with |scale| * log2(e) beyond the fp32 range, or out
 * overlapping an input; FA355_ERR_UNSUPPORTED for another D, a misaligned
 * pointer, a grid too large to launch (more than 2^31 - 1 work items) or
 * a token row of q over 16 MiB; FA355_ERR_DEVICE if
 * no HIP device is current or it is not gfx950; FA355_ERR_LAUNCH if the
 * launch fails.
 */
int mha_no_cache(void *out, const void *q, const void *k, const void *v, int B, int S, int H,
                 int Hkv, int D, float scale, int mask_kind, int window, int dtype, void *stream);

/* Static text for a status code (never NULL). */
const char *fa355_strerror(int status);

/* Library version string, e.g. "fa355 0.1.0 gfx950". */
const char *fa355_version(void);

/*
 * Work decomposition of one mha_no_cache call, for inspection and tests;
 * pure host arithmetic, no HIP call. The arguments B ... dtype, mask_kind
 * and window are those of the call. A work item computes the same block_m
 * query rows of heads_per_wg consecutive query heads, which share one K/V
 * head (heads_per_wg is the largest of 8, 4, 2, 1 that divides H / Hkv and
 * fits the kernel's waves), against key tiles of block_n keys. fp32 calls
 * at head dim 32 or 64 whose 32-row items number at most 256 use items of
 * 32 rows of one head, the workgroup's four waves each taking every fourth
 * key tile and merging their partial softmax states exactly at the end.
 * 16-bit calls at head dim 256 run 8 waves with 32-key tiles, unless those
 * items would number fewer than 512 under a mask (256 without one): then 4
 * waves with 64-key tiles, so twice the items. Reports the
 * number of work items (num_workgroups), whether the call walks them
 * (walk: 0 or 1) and, for each of the first `n` item indices, what it
 * computes: tiles[3*w + 0] = query tile (rows tile*block_m ...
 * tile*block_m + block_m - 1), tiles[3*w + 1] = b, tiles[3*w + 2] = first
 * head h (heads h ... h + heads_per_wg - 1).
 * Item w runs on XCD w % 8 where the (batch, K/V head) groups split evenly
 * over the 8 XCDs (all of a group's items on one XCD). A call that does not
 * walk launches one workgroup per item. A walking call (16-bit inputs at
 * head dim 64 or 128, items of at most 64 key tiles on average) launches as
 * many workgroups as the device holds at once (a multiple of 8), each
 * taking several items in rounds, when the items outnumber them. Walking
 * calls and unmasked 16-bit calls order each XCD's items group by group
 * (each group's query tiles longest first); other calls put the longest
 * query tiles first. Any output pointer may be NULL; `tiles` NULL queries
 * only the sizes.
 * Returns FA355_OK or FA355_ERR_INVALID_ARG / FA355_ERR_UNSUPPORTED under
 * the same rules as mha_no_cache.
 */
int fa355_plan(int B, int S, int H, int Hkv, int D, int dtype, int mask_kind, int window,
               int *num_workgroups, int *block_m, int *block_n, int *heads_per_wg, int *walk,
               int *tiles, int n);

/*
 * fa355_topk: the top-K token sampler of the recipe page "Custom
 * Operations: Applications in AI Models" (builds.modular.com), section
 * "Optimizing top-K token sampling for GPUs in MAX": each batch row of
 * next-word frequencies is ordered by highest frequency, and the operation
 * returns the ordered values and their positions. Here: the K largest
 * entries of each row in descending order (the page orders the whole row:
 * K = V), equal values by ascending index, -0.0 equal to +0.0.
 *
 * Arguments (device pointers on the current HIP device, contiguous,
 * 4-byte aligned):
 *   values   [B, K] float32   written: values[b*K + i] = in[b*V + indices[b*K + i]],
 *                             bit for bit.
 *   indices  [B, K] int32     written: positions within the row, 0 .. V-1.
 *   in       [B, V] float32   read only; finite values (NaN is outside the
 *                             contract: it is ordered but not tested).
 *   B, V, K                   rows, entries per row, entries kept per row.
 *   stream                    a hipStream_t, or NULL for the null stream.
 * The result is exact and deterministic.
 *
 * Ownership: the caller owns every buffer; the library allocates nothing.
 * Execution: asynchronous on `stream`.
 * Errors: FA355_ERR_INVALID_ARG for a null pointer, B, V or K < 1, K > V,
 * or an output overlapping the input or the other output;
 * FA355_ERR_UNSUPPORTED for K > 1024 or a pointer not 4-byte aligned;
 * FA355_ERR_DEVICE / FA355_ERR_LAUNCH as for mha_no_cache. Checks run
 * before any HIP call.
 */
int fa355_topk(float *values, int *indices, const float *in, int B, int V, int K, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
