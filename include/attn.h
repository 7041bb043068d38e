/*
 * attn.h - C ABI of the scaled dot-product attention forward for AMD MI355X
 * (gfx950).
 *
 * The operation (learn-cuda-from-scratch Ch. 11 "Attention", section 11.1;
 * AIInfraGuide "3.3 Self-Attention机制深入理解", sections 3.2-3.6):
 *
 *     O[b, h, i, :] = sum_j P[i, j] * V[b, g, j, :]
 *     P[i, :]       = softmax_j( scale * sum_d Q[b, h, i, d] * K[b, g, j, d]  + mask[i, j] )
 *     g             = h / (H_q / H_kv)
 *
 * mask[i, j] is 0 where key j is visible to query row i and -inf elsewhere.
 * Non-causal: every key is visible.  Causal (Ch. 11 page, section 11.1:
 * token i may not see j > i): row i sits at absolute position
 * i + (T_kv - T_q) and sees keys j <= i + (T_kv - T_q).  With T_q == T_kv
 * this is the usual j <= i; with T_q < T_kv it is a chunk of queries placed
 * at the end of the keys; with T_q == 1 (decode) every key is visible.
 *
 * The head mapping covers MHA (H_kv == H_q), MQA (H_kv == 1) and GQA
 * (anything that divides H_q): consecutive query heads share one kv head
 * (Ch. 11 page, sections 11.8.1 and 11.11; AIInfraGuide page, section 9.3).
 *
 * Layout (no strides): Q and O are contiguous row-major [B][H_q][T_q][D];
 * K and V are contiguous row-major [B][H_kv][T_kv][D].  All four tensors
 * have the element type `dtype`.  Pointers are device pointers, 16-byte
 * aligned; O must not overlap Q, K or V.
 *
 * Arithmetic: bf16 tensors are multiplied on bf16 matrix cores with fp32
 * accumulation, the softmax runs in fp32, the weights are rounded to bf16
 * for the P*V product and O is rounded once to bf16 (round-to-nearest-even).
 * fp32 tensors use fp32 arithmetic throughout.  The T_q x T_kv score and
 * weight matrices are never written to memory.
 *
 * Ownership and asynchrony: the caller owns every buffer, including the
 * decode workspace; the library keeps no pointer after a call returns and
 * allocates no device memory (the one static device array it holds, the
 * scratch of attn_fwd_decode_noalloc, comes with the loaded code object).  Calls only enqueue work on `stream` (a
 * hipStream_t; NULL is the null stream) and never synchronise.  Launch
 * failures return ATTN_ERR_HIP (attn_last_hip_error() gives the HIP code
 * of the calling thread's last failure); faults inside a kernel surface at
 * the caller's next synchronisation.
 *
 * Validation: every argument check runs on the host before any HIP call,
 * in this order: shape and parameter values, empty problem, null pointers,
 * alignment, aliasing, workspace.  B == 0 or T_q == 0 is an empty problem:
 * the call returns ATTN_OK, launches nothing and ignores the pointers.
 *
 * Thread safety: all functions are re-entrant; the library holds no mutable
 * host state except the per-thread last HIP error and the per-device
 * address of that scratch array (looked up once, under a lock); calls to
 * attn_fwd_decode_noalloc that overlap on one GPU share the array's
 * contents (see there).  Results are bitwise
 * deterministic for fixed arguments (including the decode split count).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 2

/* Bytes of the static device scratch behind attn_fwd_decode_noalloc. */
#define ATTN_DECODE_SCRATCH_BYTES (16u << 20)

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL_PTR = 1,       /* a tensor pointer (or workspace) is NULL   */
    ATTN_ERR_INVALID_SHAPE = 2,  /* negative size, H <= 0, H_q % H_kv != 0,   */
                                 /* T_kv <= 0, causal with T_q > T_kv, or a   */
                                 /* size too large for the launch grid        */
    ATTN_ERR_UNSUPPORTED = 3,    /* D not 64 or 128; unknown dtype; decode    */
                                 /* with T_q != 1; split count out of range   */
    ATTN_ERR_INVALID_SCALE = 4,  /* scale is NaN or infinite                  */
    ATTN_ERR_ALIGNMENT = 5,      /* a pointer is not 16-byte aligned          */
    ATTN_ERR_ALIAS = 6,          /* O overlaps Q, K or V (or the workspace)   */
    ATTN_ERR_WORKSPACE = 7,      /* decode workspace too small                */
    ATTN_ERR_HIP = 8,            /* a HIP launch call failed                  */
    ATTN_ERR_SCRATCH = 9         /* attn_fwd_decode_noalloc: the split plan   */
                                 /* needs more than ATTN_DECODE_SCRATCH_BYTES */
} attn_status_t;

typedef enum attn_dtype {
    ATTN_F32 = 0,   /* IEEE binary32 */
    ATTN_BF16 = 1   /* bfloat16      */
} attn_dtype_t;

/*
 * Prefill / general forward: any T_q >= 0, T_kv >= 1 (causal needs
 * T_q <= T_kv).  One kernel launch.  bf16: tiled over (query tile, q head,
 * batch) with online softmax (AIInfraGuide page, sections 7.3, 12.2 and
 * 12.3); key tiles wholly above the causal diagonal are skipped and only
 * tiles that cross it are masked element by element (Ch. 11 page, section
 * 11.8.3).  fp32: same math with fp32 FMA instead of matrix cores.
 *
 *   q, k, v  device input tensors (layout above), read only
 *   o        device output tensor, fully overwritten
 *   scale    multiplier of the raw dot product (e.g. 1/sqrt(D)); any finite
 *            value.  Accuracy (bf16): the weights are rounded to bf16
 *            (relative 2^-9) before P*V and O is rounded once, so an element
 *            of O is within 2^-9 * sum_j P_ij |V_jd - O_id| (plus fp32
 *            rounding of the sums) of the exact value before that last
 *            rounding, and within that plus half a bf16 ulp of O after it.
 *            At 1/sqrt(D) with unit-variance inputs this stays below 1.5e-2;
 *            at larger scales rows with |O| >= 4 occur, where half a bf16
 *            ulp alone is 1/64.
 *   causal   0 or nonzero
 *   dtype    ATTN_F32 or ATTN_BF16
 *   stream   hipStream_t to enqueue on
 */
attn_status_t attn_fwd_prefill(const void* q, const void* k, const void* v, void* o,
                               int B, int H_q, int H_kv, int T_q, int T_kv, int D,
                               int causal, float scale, int dtype, void* stream);

/*
 * Causal sliding-window attention (Ch. 11 page, section 11.8.4: attend to
 * the most recent W tokens only, which turns the O(T^2) cost into O(T*W)):
 * as attn_fwd_prefill with causal = 1, except that query row i (absolute
 * position p = i + T_kv - T_q) sees only the keys p - window + 1 ... p.  Key
 * tiles left of every row's window are never visited, tiles that cross a
 * window edge are masked element by element.
 *
 *   window   >= 1 keys; window >= T_kv is plain causal attention
 *   dtype    ATTN_BF16 only
 * Requires T_q <= T_kv.  Other arguments as attn_fwd_prefill.
 */
attn_status_t attn_fwd_prefill_window(const void* q, const void* k, const void* v, void* o,
                                      int B, int H_q, int H_kv, int T_q, int T_kv, int D,
                                      int window, float scale, int dtype, void* stream);

/*
 * Packed variable-length prefill: B sequences of different lengths in one
 * call, the flash_attn_varlen_func form of prefill named on the Ch. 11 page
 * (section 11.8.2).  Layout is token-major and packed:
 *
 *   q, o   [total_q][H_q][D];  k, v  [total_k][H_kv][D]
 *   cu_seqlens_q, cu_seqlens_k   device int32 [B + 1], non-decreasing,
 *          cu[0] = 0, cu[B] = total: sequence b owns query rows
 *          cu_seqlens_q[b] ... cu_seqlens_q[b+1] - 1 and key rows
 *          cu_seqlens_k[b] ... cu_seqlens_k[b+1] - 1
 *   max_seqlen_q, max_seqlen_k   upper bounds of the per-sequence lengths
 *          (they size the grid and the 32-bit offset checks; rows of a
 *          longer sequence beyond max_seqlen_q are not computed)
 *   total_q, total_k   rows of the packed tensors (used for the overlap
 *          checks)
 *   causal, window     per sequence, with bottom-right alignment
 *          (row i at position i + T_kv_b - T_q_b); window 0 = none, window
 *          > 0 needs causal
 *
 * Device values are not checked on the host.  A query row that sees no key
 * (an empty key range, or causal with the row before the first key) gets
 * O = 0.  dtype ATTN_BF16 only; cu arrays 4-byte aligned.  Otherwise as
 * attn_fwd_prefill.
 */
attn_status_t attn_fwd_prefill_varlen(const void* q, const void* k, const void* v, void* o,
                                      const int* cu_seqlens_q, const int* cu_seqlens_k, int B,
                                      int H_q, int H_kv, int D, int total_q, int total_k,
                                      int max_seqlen_q, int max_seqlen_k, int causal, int window,
                                      float scale, int dtype, void* stream);

/*
 * Decode forward: one query token per (batch, q head) against T_kv cached
 * keys (Ch. 11 page, section 11.8.2: decode is a vector against the whole
 * KV cache and is memory-bound).  T_q must be 1; `causal` is accepted and
 * has no effect (the single row sees every key).
 *
 * bf16: the keys are cut into `num_splits` contiguous ranges; one pass
 * writes a partial (running max, exponential sum, unnormalised output) per
 * (batch, q head, split) into `workspace`, a second pass merges them with
 * the block-merge rule of AIInfraGuide section 12.3 and writes O (with one
 * split the first pass writes O directly).  Each kv head's keys and values
 * are read once for all of its query heads.
 * fp32: one pass, no workspace used (workspace may be NULL).
 *
 *   num_splits       0 = library default (attn_fwd_decode_default_splits),
 *                    else 1..1024; clamped to the number of 32-key blocks.
 *                    With one split the split pass writes O itself and no
 *                    workspace is needed.
 *   workspace        device buffer of at least
 *                    attn_fwd_decode_workspace_bytes(...) bytes, 16-byte
 *                    aligned, not overlapping O, Q, K or V; contents on
 *                    entry are ignored and on exit unspecified.  May be NULL
 *                    when that size is 0.
 */
attn_status_t attn_fwd_decode(const void* q, const void* k, const void* v, void* o,
                              int B, int H_q, int H_kv, int T_q, int T_kv, int D,
                              int causal, float scale, int dtype, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode without a workspace argument and without any device allocation,
 * for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments (minus
 * the workspace), checks, split plan, kernels and results, bit for bit, as
 * attn_fwd_decode.  The split partials go to a static device array of
 * ATTN_DECODE_SCRATCH_BYTES (16 MiB) that the library holds on every GPU it
 * runs on until the process ends; the first call on a device looks up that
 * device's copy (hipGetSymbolAddress, with the stream's device current).  A
 * split plan needing more (B * H_q * splits * (D + 2) * 4 bytes; the default
 * plan needs at most about 12.2 MiB) returns ATTN_ERR_SCRATCH before anything
 * is launched.  All calls on one GPU share its array, and nothing in it has
 * to start at zero: calls that may run at the same time on one GPU (other
 * streams, other threads) race on it and must be ordered by the caller.
 */
attn_status_t attn_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                      int B, int H_q, int H_kv, int T_q, int T_kv, int D,
                                      int causal, float scale, int dtype, int num_splits,
                                      void* stream);

/*
 * Decode over a paged KV cache (the serving form of decode; Ch. 11 page,
 * section 11.11: the KV cache is kept in fixed-size pages of 16 tokens, and a
 * block table maps (request, token / 16) to a physical page that the
 * attention kernel loads through one indirection).  Same arithmetic, split
 * plan and workspace rules as attn_fwd_decode (bf16 only).
 *
 *   q            device [B][H_q][D]: one query token per sequence
 *   k_pages,     device [num_pages][H_kv][page_size][D] each: the K and V
 *   v_pages      pools; physical page p holds rows 0..page_size-1 of one
 *                logical page of some sequence, for every kv head
 *   o            device [B][H_q][D], fully overwritten
 *   block_table  device int32 [B][max_pages]: token j of sequence b is row
 *                j % page_size of page block_table[b][j / page_size]; only
 *                entries below ceil(seq_lens[b] / page_size) are read
 *   seq_lens     device int32 [B]: keys of sequence b
 *   page_size    a power of two, 16 ... 65536
 *   num_pages    pages in each pool (>= 1)
 *   max_pages    columns of block_table (>= 1); max_pages * page_size is the
 *                longest sequence (<= 2^30) and sizes the split plan
 *   num_splits, workspace, workspace_bytes: as for attn_fwd_decode, with
 *                T_kv = max_pages * page_size
 *                (attn_fwd_decode_paged_workspace_bytes gives the size)
 *
 * Device-side values are not checked on the host; instead, with no fault in
 * any case: seq_lens[b] is clamped to [0, max_pages * page_size]; a sequence
 * of length 0 gets O = 0; a block id outside [0, num_pages) reads as a page
 * of zeros.  Pages are read only up to the sequence's last key.
 * Pointer checks: q, k_pages, v_pages, o and the workspace 16-byte aligned,
 * block_table and seq_lens 4-byte aligned; o and the workspace may overlap
 * no input.  dtype must be ATTN_BF16.
 */
attn_status_t attn_fwd_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                    void* o, const int* block_table, const int* seq_lens, int B,
                                    int H_q, int H_kv, int D, int page_size, int num_pages,
                                    int max_pages, float scale, int dtype, int num_splits,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_fwd_decode_paged needs (0 if none or invalid sizes). */
size_t attn_fwd_decode_paged_workspace_bytes(int B, int H_q, int H_kv, int D, int page_size,
                                             int max_pages, int num_splits);

/*
 * Fused QKV projection, the step before the attention forward (Ch. 11 page,
 * section 11.2: Q, K and V are three linear maps of the same input X;
 * section 11.8.1: q heads and the fewer kv heads are column blocks of those
 * maps).  One bf16 GEMM Y = X W^T over the concatenated weights; its epilogue
 * splits the columns and writes Q, K, V in the layouts attn_fwd_prefill and
 * attn_fwd_decode take.
 *
 *   x        device [B*T][d_model]: token t of sequence b is row b*T + t
 *   w        device [(H_q + 2*H_kv)*D][d_model]: rows 0 .. H_q*D - 1 are W_Q
 *            (row h*D + d gives feature d of q head h), then H_kv*D rows of
 *            W_K, then H_kv*D rows of W_V (a linear layer's weight layout)
 *   q        device [B][H_q][T][D], fully overwritten
 *   k, v     device [B][H_kv][T][D], fully overwritten
 *   d_model  a multiple of 64
 *   dtype    ATTN_BF16 only
 * Arithmetic: bf16 matrix cores, fp32 accumulation over d_model, each output
 * rounded once to bf16 (round-to-nearest-even).  All pointers 16-byte
 * aligned; the outputs may overlap neither each other nor the inputs.
 * B == 0 or T == 0 is an empty problem (ATTN_OK, nothing launched).
 */
attn_status_t attn_qkv_project(const void* x, const void* w, void* q, void* k, void* v, int B,
                               int T, int d_model, int H_q, int H_kv, int D, int dtype,
                               void* stream);

/* Workspace bytes attn_fwd_decode needs for these sizes (num_splits as
 * passed to attn_fwd_decode, 0 = default).  Returns 0 when no workspace is
 * needed (one split, or dtype ATTN_F32) and for invalid sizes. */
size_t attn_fwd_decode_workspace_bytes(int B, int H_q, int H_kv, int T_kv, int D,
                                       int dtype, int num_splits);

/* Split count attn_fwd_decode uses when num_splits == 0 (>= 1; 0 for
 * invalid sizes): with G = H_q / H_kv, the B * H_kv * ceil(G / 32) groups
 * each get as many splits as fit one round of 768 waves (D = 128) or 1024
 * (D = 64) on the GPU, at least one and at most one per 4 key blocks of
 * 32; after rounding to whole blocks per split the count may come out
 * lower. */
int attn_fwd_decode_default_splits(int B, int H_q, int H_kv, int T_kv, int D);

/* Static, NUL-terminated description of a status code. */
const char* attn_status_string(int status);

/* ATTN_ABI_VERSION of the library. */
int attn_abi_version(void);

/* HIP error code (hipError_t) of the calling thread's last ATTN_ERR_HIP. */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
