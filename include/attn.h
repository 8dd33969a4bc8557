/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * The operation is the attention equation on the page "Shape-Aware Attention"
 * (section "Inspiration"): O = softmax(Q K^T * scale) V, optionally with a causal mask,
 * computed with online softmax -- a running row maximum, running row sum and
 * rescaled fp32 accumulator carried across key/value blocks, so the
 * [B, H, S_q, S_kv] score matrix never exists (page "GPU Kernel for a
 * Transformer Layer", section "What we learned").  Softmax statistics and the
 * accumulator are fp32 (same section: softmax is a reduction and needs fp32).
 * The chunked entry point processes the queries in bounded windows against a
 * key/value cache that holds kv_len valid rows (page "Roofline", section "How
 * we built it": bounded-memory windows against a growing key/value cache, for
 * sequences up to ~100k tokens).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are DEVICE pointers to contiguous row-major arrays:
 *     q, o : [B, H, S_q,  D_h]
 *     k, v : [B, H, S_kv, D_h]
 * all of one element type `dtype` (enum attn_dtype); o is written in that type
 * (round-to-nearest-even from the fp32 accumulator).  Every base pointer must be
 * 16-byte aligned; o must not overlap q, k or v.  D_h must be 64.
 *
 * scale multiplies q.k before the softmax; pass 1/sqrt(D_h) for the equation as printed.  Any
 * finite value is accepted (0 gives the plain mean of the visible values).
 *
 * Causal masking is bottom-right aligned: query row i sits at absolute
 * position p_i = kv_len - S_q + i and sees keys j <= p_i.  With S_q == kv_len
 * this is "key j visible to query i iff j <= i".  A causal call needs
 * S_q <= kv_len so that every row sees at least one key.
 *
 * Arithmetic: Q K^T and P V run on MFMA (bf16/fp16 operands with fp32
 * accumulation for ATTN_BF16/ATTN_F16; true fp32 MFMA for ATTN_F32).  The
 * probabilities P are computed in fp32; on the 16-bit paths they are rounded
 * once to the input type, as the operand of the P V product, and the row sum
 * l adds those rounded values (fp32 accumulation on the matrix cores), so the
 * output is the exact weighted mean with the weights P V applies; each weight
 * differs from the fp32 probability by its rounding (a relative 2^-9 for
 * bf16, 2^-12 for fp16).  ATTN_F32 keeps P and l in fp32.  No [S_q, S_kv]
 * buffer is written anywhere.
 *
 * Ownership and concurrency: the caller allocates and frees every buffer.  The
 * library allocates no device or host memory, keeps no pointer after it
 * returns, and holds no state except a per-device "is gfx950" cache.  Work is
 * enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream);
 * the caller keeps the buffers alive and synchronises the stream before
 * reading o.  Calls are thread-safe.
 *
 * Errors: every entry point returns ATTN_OK (0) once the work is enqueued.
 * Otherwise it returns the first failing check below and enqueues nothing.  No
 * entry point prints, aborts or throws.  Argument checks run before any HIP
 * call, so they behave the same on a machine without a GPU.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_dtype {
    ATTN_F32 = 0,   /* IEEE binary32 */
    ATTN_F16 = 1,   /* IEEE binary16 */
    ATTN_BF16 = 2   /* bfloat16 */
};

enum attn_status {
    ATTN_OK = 0,
    ATTN_E_NULL = 1,     /* q, k, v or o is NULL */
    ATTN_E_SHAPE = 2,    /* B, H, S_q or S_kv < 1; D_h != 64; sizes overflow; one head of K/V >= 4 GiB */
    ATTN_E_DTYPE = 3,    /* dtype not an attn_dtype value */
    ATTN_E_SCALE = 4,    /* scale is NaN or infinite */
    ATTN_E_CAUSAL = 5,   /* causal with S_q > kv_len (a row would see no key) */
    ATTN_E_CHUNK = 6,    /* chunk < 1, or kv_len outside [1, S_kv] */
    ATTN_E_ALIGN = 7,    /* a base pointer is not 16-byte aligned */
    ATTN_E_DEVICE = 8,   /* no current HIP device, or it is not gfx950 */
    ATTN_E_HIP = 9,      /* the HIP runtime reported an error for the launch */
    ATTN_E_OVERLAP = 10, /* o overlaps q, k or v */
    ATTN_E_SPLIT = 11,   /* n_split outside [1, 1024], or the split grid exceeds 2^31 - 1 workgroups */
    ATTN_E_WORKSPACE = 12 /* workspace NULL, not 16-byte aligned, smaller than required, or overlapping q/k/v/o */
};

/*
 * attn_fwd -- O = softmax(Q K^T * scale [+ causal mask]) V over the whole
 * K/V (kv_len = S_kv).  The attention equation of page "Shape-Aware
 * Attention", section "Inspiration"; online softmax as on the page "GPU Kernel for a Transformer
 * Layer", section "What we learned"; causal masking inside the kernel as in
 * that page's section "How we built it".
 *   q, k, v, o : device pointers, layouts above.
 *   B, H       : batch size and number of heads.
 *   S_q, S_kv  : query rows and key/value rows per (b, h).
 *   D_h        : head dimension (must be 64).
 *   causal     : nonzero for the causal mask.
 *   scale      : score multiplier (finite).
 *   dtype      : enum attn_dtype of all four tensors.
 *   stream     : hipStream_t to enqueue on (NULL = null stream).
 * Identical, bit for bit, to attn_fwd_chunked(..., chunk = S_q,
 * kv_len = S_kv).  The launch shape follows attn_sched_rows: 128-row query
 * tiles; when B*H*ceil(S_q/128) is at most twice the number of compute units,
 * each tile's keys are split between two wave groups (even and odd 64-key
 * tiles) and merged at the end, and such small grids take 64-row tiles where
 * 128-row ones would leave compute units idle or unequal, 32-row tiles when
 * S_q <= 32.  The shape depends on B, H, S_q, causal, dtype and the compute
 * unit count, never on chunk or kv_len; a row's arithmetic depends only on
 * whether its keys are split.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *o,
             int B, int H, int S_q, int S_kv, int D_h,
             int causal, float scale, int dtype, void *stream);

/*
 * attn_fwd_chunked -- the same operation with the query rows processed in
 * windows of `chunk` rows against the first kv_len rows of a K/V cache of
 * capacity S_kv (page "Roofline", section "How we built it"; section "What we
 * learned": at ~100k tokens the fix is chunking/streaming).
 *   chunk  : rows per query window, >= 1 (chunk >= S_q is a single window).
 *   kv_len : valid K/V rows, 1 <= kv_len <= S_kv; rows >= kv_len are never read.
 * Windows w = 0 .. ceil(S_q/chunk)-1 cover query rows [w*chunk,
 * min(S_q, (w+1)*chunk)).  Window w reads keys [0, kv_len) when non-causal and
 * [0, kv_len - S_q + min(S_q, (w+1)*chunk)) when causal.  All windows are
 * enqueued as one launch, heaviest window first; memory use is O(S) for any
 * kv_len (no workspace).  The window split changes the schedule, not the
 * result: each output row is bit-identical to attn_fwd's on the same data.
 * A streaming caller appends a window's K/V rows to the cache and calls with
 * S_q = that window's rows and the grown kv_len; its rows equal the single
 * call's bit for bit when both calls make the same key-split choice
 * (attn_sched_rows), and to rounding otherwise.
 */
int attn_fwd_chunked(const void *q, const void *k, const void *v, void *o,
                     int B, int H, int S_q, int S_kv, int D_h,
                     int causal, float scale, int dtype, void *stream,
                     int chunk, int kv_len);

/*
 * attn_fwd_varlen -- attn_fwd for a batch of sequences of different lengths
 * padded to S_kv keys: sequence b (every head h) attends only to its first
 * kv_lens[b] K/V rows (key padding; the case the causal kernel of the page
 * "GPU Kernel for a Transformer Layer", section "How we built it", left to a
 * library call).  Causal masking is bottom-right per sequence:
 * query row i sits at position kv_lens[b] - S_q + i; a row that sees no key
 * (kv_lens[b] = 0, or a causal row before the sequence's first key) gets
 * zeros.
 *   kv_lens : DEVICE pointer to B int32 values, 4-byte aligned; each value is
 *             clamped into [0, S_kv] (rows past S_kv are never read).
 *   Other arguments as attn_fwd.  Rows of K/V at or past kv_lens[b] are never
 *   read.  The key split follows the same rule as attn_fwd.
 * Errors as attn_fwd, except that causal calls with S_q > a sequence's length
 * are allowed; ATTN_E_NULL also for a NULL kv_lens, ATTN_E_ALIGN for a
 * misaligned one.
 */
int attn_fwd_varlen(const void *q, const void *k, const void *v, void *o,
                    int B, int H, int S_q, int S_kv, int D_h,
                    int causal, float scale, int dtype, void *stream,
                    const int *kv_lens);

/*
 * attn_fwd_splitkv -- attn_fwd_chunked with one query window (chunk = S_q)
 * whose keys are also split across workgroups: the first kv_len K/V rows are
 * cut into n_split ranges of whole 64-key tiles; each range is attended on its
 * own with the online-softmax state of the page "GPU Kernel for a Transformer
 * Layer" (section "What we learned": running maximum, running sum, rescaled
 * accumulator), and a second kernel merges the ranges' states exactly as the
 * online update merges two blocks: with M the largest offset, O = sum
 * 2^(m_s - M) acc_s / sum 2^(m_s - M) l_s (one pass over the ranges, eight
 * at a time; a batch that raises M first rescales the running sums; beyond
 * 24 ranges each row's ranges are dealt to sixteen groups of threads whose
 * sums are then combined the same way).  This is the regime of few query
 * tiles against a long cache (a decode step of the growing cache of the page
 * "Roofline", section "How we built it"; small batches, where the page "GPU
 * Kernel for a Transformer Layer", section "What we learned", loses to a
 * library call): more workgroups than query tiles.
 *   kv_len     : valid K/V rows, 1 <= kv_len <= S_kv (as attn_fwd_chunked).
 *   n_split    : 1 .. 1024 key ranges (attn_splitkv_choose picks one); 1 runs
 *                attn_fwd_chunked(..., S_q, kv_len) and needs no workspace.
 *   workspace  : DEVICE memory of at least attn_splitkv_workspace_bytes(B, H,
 *                S_q, n_split) bytes, 16-byte aligned, not overlapping any
 *                tensor; owned by the caller, overwritten by every call (calls
 *                that overlap in time must not share one).  Holds fp32 partial
 *                states only; nothing needs clearing between calls.
 * Same result as attn_fwd_chunked up to fp32 rounding order (the ranges are
 * summed in a different order).  Errors: as attn_fwd_chunked; ATTN_E_SPLIT;
 * ATTN_E_WORKSPACE.
 */
int attn_fwd_splitkv(const void *q, const void *k, const void *v, void *o,
                     int B, int H, int S_q, int S_kv, int D_h,
                     int causal, float scale, int dtype, void *stream,
                     int kv_len, int n_split, void *workspace, size_t workspace_bytes);

/* Size of the device array that attn_fwd_splitkv_noalloc keeps its partial
 * states in: 16 MiB per GPU. */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * attn_fwd_splitkv_noalloc -- attn_fwd_splitkv for callers that cannot
 * allocate device memory (code under stream capture into a HIP graph, tight
 * serving loops, harnesses that forbid allocation).  The partial states
 * live in a device array the library holds instead of a caller workspace;
 * the caller still passes q, k, v and o.  Nothing is allocated or freed.
 *   Arguments as attn_fwd_splitkv without the workspace.  The states take
 *   attn_splitkv_workspace_bytes(B, H, S_q, n_split) bytes, at most
 *   ATTN_NOALLOC_SCRATCH_BYTES (16 MiB: for example n_split = 8 ranges of
 *   7,943 query rows); n_split = 1 needs none.
 * The array is the library's, one per GPU, from the first call on that GPU
 * (which looks up its address) until the process ends.  Every call on a GPU
 * uses the same array: calls that overlap in time on one GPU (two streams,
 * two threads) race and must not be issued; calls one after another on a
 * stream are fine.  The result is bit-identical to attn_fwd_splitkv with the
 * same n_split.  Errors: as attn_fwd_splitkv; ATTN_E_WORKSPACE when the
 * states would exceed ATTN_NOALLOC_SCRATCH_BYTES (checked before any HIP
 * call); ATTN_E_HIP if the array's address cannot be looked up.
 */
int attn_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o,
                             int B, int H, int S_q, int S_kv, int D_h,
                             int causal, float scale, int dtype, void *stream,
                             int kv_len, int n_split);

/* Workspace bytes attn_fwd_splitkv needs (0 for n_split = 1): n_split * B*H*S_q
 * * 264.  Host only.  ATTN_E_SHAPE for sizes < 1 or an overflow, ATTN_E_SPLIT
 * for n_split out of range. */
int attn_splitkv_workspace_bytes(int B, int H, int S_q, int n_split, size_t *bytes);

/* A key-range count for attn_fwd_splitkv on a GPU of n_cu compute units: 1
 * when there are at least two 128-row query tiles per CU or the keys span
 * fewer than 16 64-key tiles; 2 from one to two tiles per CU; below that
 * enough ranges for about one workgroup per CU, keeping at least two key
 * tiles per range.
 * Host only.  ATTN_E_SHAPE for sizes < 1 or a NULL output. */
int attn_splitkv_choose(int B, int H, int S_q, int kv_len, int n_cu, int *n_split);

/*
 * attn_qkv_proj -- the fused Q/K/V projection upstream of attention (page
 * "Roofline", sections "What it does" and "How we built it": the three
 * projections as one larger kernel): y = x W^T (+ bias) as ONE matrix product
 * whose epilogue writes each head's 64 columns straight into q, k, v in the
 * [B, H, S, 64] layout the attention entry points read.
 *   x     : device [B, S, d] (d = 64*H, row-major).
 *   w     : device [3d, d], the three projection weights stacked in the layout
 *           of a linear layer: output feature o is row o; rows [0, d) give q,
 *           [d, 2d) k, [2d, 3d) v, and inside each, head h is rows
 *           [64h, 64h + 64).
 *   bias  : device [3d] or NULL (no bias).
 *   q, k, v : device [B, H, S, 64] outputs: q[b, h, s, e] = y[b*S + s, 64h + e],
 *           k and v from the next two thirds of y.
 *   D_h must be 64.  dtype: ATTN_BF16 or ATTN_F16 (all six tensors); fp32
 *   products accumulate in fp32 (MFMA), the bias is added in fp32, and each
 *   output is rounded once (RNE) to dtype.
 * Conventions as above (16-byte aligned base pointers, asynchronous on
 * `stream`, nothing allocated).  Errors: ATTN_E_NULL (x, w, q, k or v NULL);
 * ATTN_E_SHAPE (B, S or H < 1, D_h != 64, sizes overflow); ATTN_E_DTYPE
 * (ATTN_F32 or unknown); ATTN_E_ALIGN; ATTN_E_OVERLAP (an output overlaps an
 * input or another output); ATTN_E_DEVICE; ATTN_E_HIP.
 */
int attn_qkv_proj(const void *x, const void *w, const void *bias,
                  void *q, void *k, void *v,
                  int B, int S, int H, int D_h, int dtype, void *stream);

/*
 * attn_kv_append -- write n_new new key and value rows into a K/V cache at
 * row kv_len of every (b, h): the append step of a stream of bounded query
 * windows against a growing key/value cache (page "Roofline", section "How
 * we built it").  A streaming caller appends a window's K/V rows, then calls
 * attn_fwd_chunked with S_q = that window's query rows and the grown kv_len
 * (kv_len + n_new).
 *   k_cache, v_cache : device [B, H, S_cap, D_h]; rows [kv_len, kv_len + n_new)
 *                      of every head are overwritten, all other rows are left
 *                      untouched.
 *   k_new, v_new     : device [B, H, n_new, D_h], copied bit for bit.
 *   kv_len           : rows already valid, 0 <= kv_len, kv_len + n_new <= S_cap.
 *   D_h must be 64; dtype (enum attn_dtype) is the element type of all four.
 * Same conventions as above: 16-byte aligned base pointers, asynchronous on
 * `stream`, nothing allocated.  Errors: ATTN_E_NULL; ATTN_E_SHAPE (B, H,
 * S_cap or n_new < 1, kv_len < 0, kv_len + n_new > S_cap, D_h != 64, sizes
 * overflow); ATTN_E_DTYPE; ATTN_E_ALIGN; ATTN_E_OVERLAP (the two caches
 * overlap, or a new-rows buffer overlaps a cache); ATTN_E_DEVICE;
 * ATTN_E_HIP.
 */
int attn_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                   int B, int H, int S_cap, int kv_len, int n_new, int D_h,
                   int dtype, void *stream);

/*
 * Schedule introspection (host only, no GPU needed).
 *
 * attn_sched_rows writes the query rows per workgroup (128, 64 or 32) and
 * whether the keys are split between two wave groups (1 or 2) of an
 * attn_fwd / attn_fwd_chunked / attn_fwd_varlen launch of these sizes,
 * causal flag (0/1) and dtype on a device with n_cu compute units (the launch
 * reads n_cu from the device).  attn_sched_grid writes the number of workgroups one
 * attn_fwd_chunked call with these sizes launches for `rows` query rows per
 * workgroup (attn_fwd: chunk = S_q, kv_len = S_kv; causal as in the call,
 * 0/1); attn_sched_tile writes which head (b*H + h) and which query rows
 * [row0, row1) workgroup `block` computes.  Every (head, row) is covered by
 * exactly one workgroup; windows run heaviest first.  All return ATTN_OK, or
 * ATTN_E_SHAPE for sizes out of range, rows other than 32, 64 and 128, or a NULL
 * output pointer (attn_sched_rows: ATTN_E_DTYPE for an unknown dtype).
 */
int attn_sched_rows(int B, int H, int S_q, int causal, int dtype, int n_cu,
                    int *rows, int *key_split);
int attn_sched_grid(int B, int H, int S_q, int chunk, int kv_len, int causal,
                    int rows, int *grid);
int attn_sched_tile(int B, int H, int S_q, int chunk, int kv_len, int causal,
                    int rows, int block, int *head, int *row0, int *row1);

/* Static, NUL-terminated description of an attn_status value (never NULL). */
const char *attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
