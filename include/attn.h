/*
 * attn.h - C ABI of the MI355X (gfx950) exact-attention library (libattn.so).
 *
 * The library computes exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T  [+ causal mask]) V
 * with a fused, tiled forward that keeps per-row online-softmax state (running
 * maximum and sum, rescaling the partial output) and writes only O and the
 * row log-sum-exp, and a backward that recomputes the scores and
 * probabilities from Q, K, V and that log-sum-exp instead of storing them.
 *
 * Sources (pages cited by title and section):
 *   - standard attention, softmax(Q K^T / sqrt(d_k)) V, and the blockwise
 *     online-softmax loop: "FlashAttention in CANN ops-transformer on the
 *     Ascend NPU" (hwcomputing.csdn.net), sections on the memory black hole of
 *     standard attention and on online softmax; mask modes in its tuning
 *     section; usage flash_attention(Q, K, V, mask="causal") with Q, K, V laid
 *     out [batch, heads, N, d] in its usage section.
 *   - tiling, online softmax being exact, backward recomputation: the lpnh.cn
 *     article on FlashAttention-2 in YOLO11, sections 2.1, 2.2 and 2.3.
 *   - GQA/MQA sharing of K/V heads by groups of query heads
 *     (repeat_interleave): "Transformer高效注意力机制实现：Flash Attention与GQA
 *     原理对比与代码实践" (yunthe.com), GQA section.
 *   - one specialised kernel per head dimension and an error (not a silent
 *     fallback) for an unsupported one: "突破FlashAttention性能瓶颈：头维度限制的
 *     技术解析与解决方案" (datacanvas.csdn.net), sections on the origin and the
 *     symptoms of the head-dim limit.
 *
 * Conventions shared by every entry point
 *   Layout: contiguous [B, H, N, d], d innermost ("BHSD"). q, o, dout, dq are
 *     [B, Hq, N, d]; k, v, dk, dv are [B, Hkv, N, d]; lse is [B, Hq, N].
 *     Self-attention: queries and keys have the same length N. The *_ex
 *     entry points take each operand as a strided view instead (attn_tensor),
 *     which covers BSHD ([B, N, H, d], the layout flash_attn_func takes on the
 *     yunthe.com GQA page) and sub-views of larger buffers.
 *   Types: q, k, v, o, dout, dq, dk, dv are bfloat16 (passed as void*), or
 *     float16 through the *_ex entry points ("FlashAttention in CANN
 *     ops-transformer on the Ascend NPU", tuning section on data types); lse
 *     is float32; all accumulation is float32.
 *   GQA: Hq must be a multiple of Hkv; query head h uses KV head
 *     h / (Hq / Hkv) (consecutive groups). Hkv == Hq is MHA, Hkv == 1 is MQA.
 *   Causal (causal != 0): query i attends to keys j <= i; otherwise to all j.
 *   Sliding window (window = W >= 1, the *_window entry points and the
 *     window argument of the pass entry points): query i attends to the W
 *     most recent keys i - W < j <= i, a band inside the causal mask ("FlashAttention in CANN
 *     ops-transformer on the Ascend NPU", tuning section on mask modes).
 *     W >= N allows every key j <= i and so equals the causal mask.
 *   Scale: the factor applied to Q K^T before the softmax, finite and > 0
 *     (callers usually pass 1/sqrt(d)).
 *   Memory: every pointer is a device pointer owned by the caller; the
 *     library never allocates, frees or synchronises (attn_bwd_noalloc uses
 *     a fixed array of its own instead of a caller workspace). Buffers must stay alive
 *     until the stream has run the enqueued work. Outputs are overwritten,
 *     never accumulated into. Device pointers must be 16-byte aligned.
 *   Streams: `stream` is a hipStream_t (NULL means the default stream). All
 *     work is enqueued on it asynchronously; calls return before it runs.
 *   Errors: every argument is checked on the host before anything is
 *     enqueued; on any error nothing is launched and outputs are untouched.
 *     Device-side faults surface at the caller's next synchronisation.
 *   Threads: apart from attn_bwd_noalloc's fixed scratch array (whose
 *     concurrent use races, see there) and a per-thread copy of the last HIP
 *     error string, the library holds no mutable global state; concurrent
 *     calls of every other entry point on different streams are safe.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,       /* a required pointer is NULL */
    ATTN_ERR_SHAPE = 2,      /* B, Hq, Hkv or N < 1, N > ATTN_MAX_SEQ_LEN, or
                                B * Hq * round_up(N, 256) >= 2^31 rows (a kernel grid
                                would pass 2^32 work-items) */
    ATTN_ERR_GQA = 3,        /* Hq is not a multiple of Hkv */
    ATTN_ERR_HEAD_DIM = 4,   /* d is not one of 32, 64, 80, 96, 128, 192, 256 */
    ATTN_ERR_SCALE = 5,      /* scale is not finite or not > 0 */
    ATTN_ERR_ALIGN = 6,      /* a pointer is not 16-byte aligned, or a stride is not a
                                multiple of 8 elements */
    ATTN_ERR_WORKSPACE = 7,  /* workspace NULL or smaller than required */
    ATTN_ERR_HIP = 8,        /* the HIP runtime refused a launch */
    ATTN_ERR_WINDOW = 9,     /* unknown mask kind, window < 0, or a window (>= 1)
                                without the causal mask */
    ATTN_ERR_STRIDE = 10,    /* a stride is negative, or one head's N rows span 2^31
                                elements or more (rows are addressed with 32-bit
                                byte offsets) */
    ATTN_ERR_DTYPE = 11,     /* unknown element type */
    ATTN_ERR_PASSES = 12,    /* passes is 0 or has bits other than ATTN_BWD_ALL */
    ATTN_ERR_DROPOUT = 13,   /* dropout_p is not in [0, 1) */
    ATTN_ERR_SCRATCH = 14    /* attn_bwd_noalloc: B * Hq * N exceeds
                                attn_bwd_noalloc_max_rows() */
} attn_status;

/* Head dimensions with a specialised kernel: 32, 64, 80, 96, 128, 192, 256. */
#define ATTN_NUM_HEAD_DIMS 7
#define ATTN_MAX_SEQ_LEN (1 << 24)

/*
 * Forward pass.
 *   q [B,Hq,N,d] bf16, k and v [B,Hkv,N,d] bf16 (read only).
 *   o [B,Hq,N,d] bf16: softmax(scale*QK^T + mask) V, each element rounded to
 *     nearest even from the float32 result.
 *   lse [B,Hq,N] float32: natural-log log-sum-exp of the row's scaled scores
 *     over its allowed keys, ln sum_j exp(scale * <q_i, k_j>); the backward
 *     pass needs it.
 * Returns ATTN_OK, or an error code with nothing enqueued.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                     hipStream_t stream);

/*
 * Forward pass under the sliding-window mask of W = window keys (query i
 * attends to keys i - W < j <= i). Arguments otherwise as for attn_fwd; lse
 * is the log-sum-exp over the row's band. window < 1 is ATTN_ERR_WINDOW.
 */
attn_status attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int N, int d, float scale, int window,
                            hipStream_t stream);

/*
 * Bytes of device workspace attn_bwd needs: two float32 per query row, the
 * row term D_i = <dO_i, O_i> (stored negated) and the LSE in base 2, each
 * array rounded up to 256 bytes. Two kinds of shapes also keep float32
 * partial dK and dV of two workgroups per key block, 2 * 2 * B * Hkv * N * d
 * * 4 more bytes: d = 128 when B * Hkv * ceil(N / 256) is between 256 and
 * 511 and Hq / Hkv is even (the query heads of each group split over two
 * workgroups), and, among the other shapes with d <= 128 and N >= 512, those
 * with B * Hkv * ceil(N / 128) <= 256 (each key block's query range split
 * over two workgroups; taken for the causal and window masks, and for no
 * mask at <= 128). Returns 0 if the shape is invalid.
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d);

/*
 * Backward pass for the loss gradient dout = dL/dO of a forward call with the
 * same arguments. Recomputes the scores and probabilities from q, k, v and
 * lse (nothing else is kept from the forward).
 *   q, k, v, o, dout bf16 and lse float32 as produced/consumed by attn_fwd.
 *   dq [B,Hq,N,d], dk and dv [B,Hkv,N,d] bf16 outputs; dk and dv sum the
 *     contributions of all query heads that share the KV head.
 *   workspace: device buffer of at least attn_bwd_workspace_bytes(...) bytes,
 *     owned by the caller; its contents on entry do not matter.
 * Returns ATTN_OK, or an error code with nothing enqueued.
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout,
                     void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                     hipStream_t stream);

/*
 * attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc). Arguments, layouts, results and errors are those
 * of attn_bwd; the row terms attn_bwd keeps in the caller's workspace go to
 * a scratch array of fixed size inside the library instead (16 MiB: at most
 * attn_bwd_noalloc_max_rows() = 2^21 query rows B * Hq * N, else
 * ATTN_ERR_SCRATCH with nothing enqueued). Each GPU the library runs on
 * holds its own copy of that array from the library's load until the
 * process ends. The call allocates and frees nothing. Its first call on a
 * device looks up that device's copy (hipGetSymbolAddress), with the device
 * current on the calling thread, which must be the stream's device. The
 * kernels write every scratch entry before reading it, so nothing carries
 * over from a previous call. Calls that overlap on one GPU (concurrent
 * streams, or threads) share the one array and race: serialise them.
 * Shapes for which attn_bwd sums two fp32 halves of dK/dV in its workspace
 * do the same here when the halves fit in the array beside the row terms,
 * else use a single-pass dK/dV kernel, whose dK and dV may differ from
 * attn_bwd's in the last bits; everything else is bitwise identical.
 */
attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout,
                             void* dq, void* dk, void* dv,
                             int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                             hipStream_t stream);

/* Largest B * Hq * N that attn_bwd_noalloc accepts. */
size_t attn_bwd_noalloc_max_rows(void);

/*
 * Backward pass of attn_fwd_window: the gradients of the banded attention,
 * for a forward call with the same arguments. Arguments otherwise as for
 * attn_bwd (same workspace size). window < 1 is ATTN_ERR_WINDOW.
 */
attn_status attn_bwd_window(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout,
                            void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes,
                            int B, int Hq, int Hkv, int N, int d, float scale, int window,
                            hipStream_t stream);

/*
 * The three passes attn_bwd runs, in order, for callers that schedule them
 * separately (for example the dK/dV and dQ passes on two streams after the
 * preprocess, or to time each pass). Arguments mean exactly what they mean
 * for attn_bwd; each validates them the same way and enqueues one kernel.
 * window: 0 for the mask `causal` selects, or W >= 1 (with causal != 0) for
 * the sliding window of attn_bwd_window.
 *   attn_bwd_preprocess: workspace <- -D_i = -<dout_i, o_i> and
 *     lse_i * log2(e) per query row.
 *   attn_bwd_dkdv: dk, dv from q, k, v, lse, dout and the workspace.
 *   attn_bwd_dq:   dq from q, k, v, lse, dout and the workspace.
 * The dK/dV and dQ passes read the workspace the preprocess wrote, so they
 * must run after it completes (same stream, or an event between streams).
 */
attn_status attn_bwd_preprocess(const void* o, const void* dout, const float* lse, void* workspace,
                                size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                                hipStream_t stream);
attn_status attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                          const void* dout, void* dk, void* dv,
                          const void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                          int window, hipStream_t stream);
attn_status attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                        const void* dout, void* dq,
                        const void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                        int window, hipStream_t stream);

/*
 * Strided, typed interface. The entry points above are the special case
 * problem = {B, Hq, Hkv, N, d, scale, causal ? ATTN_MASK_CAUSAL : ATTN_MASK_NONE,
 * 0, ATTN_DTYPE_BF16} with contiguous BHSD tensors.
 */
typedef enum attn_dtype {
    ATTN_DTYPE_BF16 = 0,
    ATTN_DTYPE_FP16 = 1
} attn_dtype;

typedef enum attn_mask_kind {
    ATTN_MASK_NONE = 0,           /* every key */
    ATTN_MASK_CAUSAL = 1,         /* keys j <= i */
    ATTN_MASK_SLIDING_WINDOW = 2  /* keys i - window < j <= i */
} attn_mask_kind;

/*
 * One [B, H, N, d] operand in device memory: element (b, h, n, e) is at
 * data + b*stride_b + h*stride_h + n*stride_n + e, strides counted in
 * elements, the d elements of a row contiguous. Strides must be >= 0 and
 * multiples of 8 (every row starts 16-byte aligned), data 16-byte aligned,
 * and (N - 1) * stride_n + d < 2^31.
 *   contiguous BHSD: stride_b = H*N*d, stride_h = N*d, stride_n = d
 *   contiguous BSHD: stride_b = N*H*d, stride_h = d,   stride_n = H*d
 * Output views must not overlap each other or the inputs.
 */
typedef struct attn_tensor {
    void* data;
    long long stride_b;
    long long stride_h;
    long long stride_n;
} attn_tensor;

typedef struct attn_problem {
    int B, Hq, Hkv, N, d;
    float scale;
    int mask;    /* attn_mask_kind */
    int window;  /* W >= 1 with ATTN_MASK_SLIDING_WINDOW, 0 otherwise */
    int dtype;   /* attn_dtype of q, k, v, o, dout, dq, dk, dv */
    /*
     * Fused dropout on the attention weights (training; "FlashAttention in
     * CANN ops-transformer on the Ascend NPU", tuning section on dropout):
     * O = (P * M / (1 - p')) V with a keep mask M drawn from a
     * counter-based generator, so the backward redraws the same mask from
     * (seed, offset) instead of storing it. Weight (b, h, i, j) is kept when
     * the 16-bit half j % 2 (0: low) of 32-bit word i % 4 of Philox-4x32-10
     * (Salmon et al., SC'11) with counter (j / 2, i / 4, b * Hq + h, offset)
     * and key (seed & 0xffffffff, seed >> 32) is >= T = floor(dropout_p *
     * 2^16), so the realised drop probability is p' = T / 2^16 (dropout_p
     * below 2^-16 drops nothing). lse is that of the softmax (dropout does not
     * change it). 0 turns dropout off; the backward must be given the
     * forward's dropout_p, seed and offset.
     */
    float dropout_p;          /* in [0, 1) */
    unsigned long long seed;
    unsigned int offset;      /* e.g. a per-call counter, so calls draw fresh masks */
} attn_problem;

/*
 * Forward pass of `problem` (q, o: H = Hq; k, v: H = Hkv). lse is contiguous
 * [B, Hq, N] float32. Returns ATTN_OK or an error code with nothing enqueued.
 */
attn_status attn_fwd_ex(const attn_problem* problem, const attn_tensor* q, const attn_tensor* k,
                        const attn_tensor* v, const attn_tensor* o, float* lse, hipStream_t stream);

/*
 * Backward pass of `problem`: the passes selected by the bits of `passes`
 * (ATTN_BWD_PREPROCESS, ATTN_BWD_DKDV, ATTN_BWD_DQ; ATTN_BWD_ALL for the
 * whole backward), in that order. A tensor no selected pass touches may be
 * passed as NULL; workspace as for attn_bwd (attn_bwd_workspace_bytes); the
 * dK/dV and dQ passes read the D_i the preprocess wrote into it.
 */
#define ATTN_BWD_PREPROCESS 1u
#define ATTN_BWD_DKDV 2u
#define ATTN_BWD_DQ 4u
#define ATTN_BWD_ALL 7u
attn_status attn_bwd_ex(const attn_problem* problem, const attn_tensor* q, const attn_tensor* k,
                        const attn_tensor* v, const attn_tensor* o, const float* lse,
                        const attn_tensor* dout, const attn_tensor* dq, const attn_tensor* dk,
                        const attn_tensor* dv, void* workspace, size_t workspace_bytes,
                        unsigned passes, hipStream_t stream);

/*
 * Decoding: Nq new queries per sequence against a key/value cache.
 *   q [B, Hq, Nq, d] and o (same shape) as attn_tensor views; k_cache,
 *   v_cache [B, Hkv, Nk, d] views of a cache with room for Nk rows, of which
 *   the first L_b hold sequence b: L_b = kv_lens[b] clamped to [0, Nk]
 *   (kv_lens: device int32 [B], or NULL for L_b = Nk).
 *   Query i of sequence b is the token at position L_b - Nq + i (the cache
 *   already holds its key and value), so the result equals the last Nq rows
 *   of self-attention over the L_b cached positions under the same mask
 *   (ATTN_MASK_NONE: all L_b keys; CAUSAL: keys j <= L_b - Nq + i;
 *   SLIDING_WINDOW: the W keys ending there). A query that sees no key
 *   (L_b < Nq under a causal mask, or L_b = 0) gets o = 0 and lse = -inf.
 *   lse [B, Hq, Nq] float32 contiguous, natural log.
 *   The KV cache and its GQA sharing are described on "Transformer高效注意力
 *   机制实现：Flash Attention与GQA原理对比与代码实践" (yunthe.com), sections on
 *   the MHA KV cache and on GQA.
 * The cache is split along its length and the partial results are merged by
 * a second kernel; the workspace (attn_decode_workspace_bytes, possibly 0)
 * holds the partials. Returns ATTN_OK or an error code with nothing enqueued.
 */
typedef struct attn_decode_problem {
    int B, Hq, Hkv;
    int Nq;      /* new queries per sequence, >= 1 */
    int Nk;      /* rows the cache views hold, >= 1 */
    int d;
    float scale;
    int mask;    /* attn_mask_kind */
    int window;  /* W >= 1 with ATTN_MASK_SLIDING_WINDOW, 0 otherwise */
    int dtype;   /* attn_dtype of q, k_cache, v_cache, o */
} attn_decode_problem;

/* Workspace bytes attn_decode_fwd needs for `problem` (0 if the shape is
 * invalid or no split is needed). */
size_t attn_decode_workspace_bytes(const attn_decode_problem* problem);

attn_status attn_decode_fwd(const attn_decode_problem* problem, const attn_tensor* q,
                            const attn_tensor* k_cache, const attn_tensor* v_cache,
                            const int* kv_lens, const attn_tensor* o, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static, human-readable description of a status code (never NULL). */
const char* attn_status_string(attn_status status);

/*
 * Text of the last HIP runtime error seen by an entry point on the calling
 * thread ("" if none). Valid until the thread's next call.
 */
const char* attn_last_hip_error(void);

/*
 * Tile plan of the forward kernel for a shape: query rows per wave, rows
 * of Q per workgroup, keys per inner step, threads per workgroup,
 * number of workgroups and bytes of LDS per workgroup. `causal` is nonzero
 * for the causal and sliding-window masks (their workgroups differ in work,
 * which changes the plan for short sequences). Host-only arithmetic (no
 * device call). Returns ATTN_OK or the validation error for that shape.
 */
typedef struct attn_plan {
    int rows_per_wave;
    int block_q;
    int block_kv;
    int threads;
    long long workgroups;
    int lds_bytes;
    int key_splits;  /* > 1: short-sequence plan, each 32-row query tile's keys
                        split over this many waves of one workgroup (64 keys
                        each) and combined in LDS; 1: the step-loop kernel */
    int key_groups;  /* 2: the step-loop kernel with its 4 waves in two groups
                        of 2 over one 64-row query block, each group walking
                        half of the block's key tiles, the two softmax states
                        combined in LDS (small grids, where the longest
                        block's key loop would decide the time); else 1 */
    int products16;  /* 1: the step loop on v_mfma_f32_16x16x32 products
                        (d = 128 without dropout on grids of 512 or more
                        256-row blocks, causal; 256 unmasked); 0: on
                        32x32x16 products */
} attn_plan;

attn_status attn_fwd_plan(int B, int Hq, int Hkv, int N, int d, int causal, attn_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
