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
 *     Self-attention: queries and keys have the same length N.
 *   Types: q, k, v, o, dout, dq, dk, dv are bfloat16 (passed as void*);
 *     lse is float32; all accumulation is float32.
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
 *     library never allocates, frees or synchronises. Buffers must stay alive
 *     until the stream has run the enqueued work. Outputs are overwritten,
 *     never accumulated into. Device pointers must be 16-byte aligned.
 *   Streams: `stream` is a hipStream_t (NULL means the default stream). All
 *     work is enqueued on it asynchronously; calls return before it runs.
 *   Errors: every argument is checked on the host before anything is
 *     enqueued; on any error nothing is launched and outputs are untouched.
 *     Device-side faults surface at the caller's next synchronisation.
 *   Threads: the library holds no mutable global state; concurrent calls on
 *     different streams are safe.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,       /* a required pointer is NULL */
    ATTN_ERR_SHAPE = 2,      /* B, Hq, Hkv or N < 1, or a size overflows */
    ATTN_ERR_GQA = 3,        /* Hq is not a multiple of Hkv */
    ATTN_ERR_HEAD_DIM = 4,   /* d is not one of 64, 80, 128, 256 */
    ATTN_ERR_SCALE = 5,      /* scale is not finite or not > 0 */
    ATTN_ERR_ALIGN = 6,      /* a pointer is not 16-byte aligned */
    ATTN_ERR_WORKSPACE = 7,  /* workspace NULL or smaller than required */
    ATTN_ERR_HIP = 8,        /* the HIP runtime refused a launch */
    ATTN_ERR_WINDOW = 9      /* window < 0, or a window (>= 1) without the causal mask */
} attn_status;

/* Head dimensions with a specialised kernel. */
#define ATTN_NUM_HEAD_DIMS 4
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
                     void* stream);

/*
 * Forward pass under the sliding-window mask of W = window keys (query i
 * attends to keys i - W < j <= i). Arguments otherwise as for attn_fwd; lse
 * is the log-sum-exp over the row's band. window < 1 is ATTN_ERR_WINDOW.
 */
attn_status attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int N, int d, float scale, int window,
                            void* stream);

/*
 * Bytes of device workspace attn_bwd needs: one float32 per query row for the
 * row term D_i = <dO_i, O_i>, rounded up to 256 bytes.
 * Returns 0 if the shape is invalid.
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
                     void* stream);

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
                            void* stream);

/*
 * The three passes attn_bwd runs, in order, for callers that schedule them
 * separately (for example the dK/dV and dQ passes on two streams after the
 * preprocess, or to time each pass). Arguments mean exactly what they mean
 * for attn_bwd; each validates them the same way and enqueues one kernel.
 * window: 0 for the mask `causal` selects, or W >= 1 (with causal != 0) for
 * the sliding window of attn_bwd_window.
 *   attn_bwd_preprocess: workspace <- D_i = <dout_i, o_i> per query row.
 *   attn_bwd_dkdv: dk, dv from q, k, v, lse, dout and the workspace.
 *   attn_bwd_dq:   dq from q, k, v, lse, dout and the workspace.
 * The dK/dV and dQ passes read the workspace the preprocess wrote, so they
 * must run after it completes (same stream, or an event between streams).
 */
attn_status attn_bwd_preprocess(const void* o, const void* dout, void* workspace,
                                size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                                void* stream);
attn_status attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                          const void* dout, void* dk, void* dv,
                          const void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                          int window, void* stream);
attn_status attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                        const void* dout, void* dq,
                        const void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                        int window, void* stream);

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
 * number of workgroups and bytes of LDS per workgroup. Host-only arithmetic
 * (no device call). Returns ATTN_OK or the validation error for that shape.
 */
typedef struct attn_plan {
    int rows_per_wave;
    int block_q;
    int block_kv;
    int threads;
    long long workgroups;
    int lds_bytes;
} attn_plan;

attn_status attn_fwd_plan(int B, int Hq, int Hkv, int N, int d, int causal, attn_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
