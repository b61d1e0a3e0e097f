/*
 * gqa.h - causal grouped-query attention with RoPE for MI355X (gfx950).
 *
 * The operation (web pages on the Qwen2 decoder):
 *   - Qwen2 technical-report walkthrough (aicoding.csdn.net) §4.1.2: h_q query
 *     heads share h_kv K/V heads, g = h_q / h_kv; 0-based query head t reads
 *     KV group u = t / g (the page's 1-based u = floor((t-1)/g) + 1).
 *   - same page §4.1.3 steps 3-4 and §3.5.2: rotate every row of Q and K
 *     (RoPE) at its position, then per head S = Q'K'^T * scale, mask keys
 *     after the query (-inf), row softmax, times V of the group.
 *   - same page §5.2 and "从 Qwen 1 到 Qwen 2 架构演进到底改了什么" (nxmr.cn) §3.2:
 *     RoPE base theta = 1e6 (passed in as `theta`).
 *   RoPE pairs dimension j with j + d/2 and turns the pair by the angle
 *   pos * theta^(-2j/d) (counter-clockwise: x_j' = x_j cos - x_{j+d/2} sin,
 *   x_{j+d/2}' = x_{j+d/2} cos + x_j sin).
 *
 * Layouts: every tensor is dense and row-major, d fastest:
 *   q, o          [B, L, h_q, d]      (prefill)    [B, h_q, d] (decode)
 *   k, v          [B, L, h_kv, d]
 *   k_cache/v_cache [B, cap, h_kv, d] (cached K is stored rotated)
 * The output o is the per-head results side by side, i.e. the "concat"
 * layout before the output projection (walkthrough §4.1.3 step 5).
 *
 * Ownership: every pointer is device memory owned by the caller (16-byte
 * aligned).  The library never allocates, frees or synchronises; it only
 * enqueues kernels on `stream` (a hipStream_t, or NULL for the default
 * stream).  Scratch space is the caller's `workspace`.
 *
 * Errors: arguments are validated on the host before anything is enqueued;
 * on failure nothing is launched, a negative status is returned and
 * gqa_last_error() gives a message (thread-local).  A launch failure
 * reported by the HIP runtime returns GQA_ERR_HIP.  Execution is
 * asynchronous: kernel faults surface at the caller's next synchronisation.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define GQA_F32  0
#define GQA_BF16 1

/* status codes */
#define GQA_OK               0
#define GQA_ERR_INVALID_ARG (-1)  /* bad pointer, size, ratio or range      */
#define GQA_ERR_UNSUPPORTED (-2)  /* valid but not built (d, dtype combo)   */
#define GQA_ERR_WORKSPACE   (-3)  /* workspace missing or too small         */
#define GQA_ERR_HIP         (-4)  /* the HIP runtime refused a launch       */

/*
 * In-place RoPE on x[B, L, h, d] (dtype GQA_F32 or GQA_BF16); row l sits at
 * position pos0 + l.  Angles are formed and reduced in fp64 and rotated in
 * fp32; bf16 results are rounded to nearest even.  d must be even.
 * (Walkthrough §3.5.2 and §4.1.3 step 3; pairing and angle as above.)
 */
int gqa_rope_apply(void* x, int dtype, int64_t B, int64_t L, int h, int d,
                   int64_t pos0, double theta, void* stream);

/* Bytes of workspace gqa_prefill needs for these sizes (0 on bad sizes). */
size_t gqa_prefill_workspace_size(int in_dtype, int64_t B, int64_t L,
                                  int h_kv, int d);

/*
 * Causal GQA prefill with RoPE fused: rows of q, k sit at positions
 * 0 .. L-1; query i sees keys j <= i (all keys if causal == 0).
 *   q [B, L, h_q, d], k/v [B, L, h_kv, d] of in_dtype (GQA_F32 or GQA_BF16);
 *   o [B, L, h_q, d] of out_dtype (GQA_F32 or GQA_BF16).
 *   scale multiplies Q'K'^T (1/sqrt(d) in the walkthrough §4.1.3 step 4).
 *   k_cache / v_cache: both NULL, or both set: then rows 0..L-1 of the
 *   per-layer cache [B, cap, h_kv, d] (in_dtype) receive the rotated K and
 *   the unchanged V (the cache holds only the h_kv groups, §4.1.3 closing
 *   note); cap >= L.
 *   h_q must be a positive multiple of h_kv (a reversed ratio is rejected,
 *   "Qwen2 / Qwen3 的实测配置差异与三个坑" (docs.keinmal.top) pitfall 2).
 *   d must be 64 or 128 (the head sizes of the Qwen2 size table).
 * bf16 inputs run on bf16 matrix cores with fp32 accumulation; f32 inputs
 * run in fp32 throughout.
 */
int gqa_prefill(const void* q, const void* k, const void* v, void* o,
                int in_dtype, int out_dtype,
                int64_t B, int64_t L, int h_q, int h_kv, int d,
                double theta, float scale, int causal,
                void* k_cache, void* v_cache, int64_t cap,
                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace gqa_decode needs for any kv_len <= cap. */
size_t gqa_decode_workspace_size(int64_t B, int h_q, int h_kv, int d,
                                 int64_t cap);

/*
 * One decode step: one new query token per sequence at position q_pos,
 * rotated inside; it attends to cache rows 0 .. kv_len-1, which must hold
 * rotated keys (as gqa_prefill writes them).  Requires 1 <= kv_len <= cap
 * and kv_len <= q_pos + 1.
 *   q [B, h_q, d] and the caches [B, cap, h_kv, d] are in_dtype;
 *   o [B, h_q, d] is out_dtype.
 * The cache is streamed once per KV group, split over key chunks whose
 * partial softmax states are merged exactly (log-sum-exp) in a second pass.
 */
int gqa_decode(const void* q, const void* k_cache, const void* v_cache,
               void* o, int in_dtype, int out_dtype,
               int64_t B, int h_q, int h_kv, int d, int64_t cap,
               int64_t kv_len, int64_t q_pos, double theta, float scale,
               void* workspace, size_t workspace_bytes, void* stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char* gqa_last_error(void);

/* Library build string. */
const char* gqa_version(void);

/*
 * Kernel timing for benchmarks.  While enabled, each gqa_prefill records a
 * HIP event pair around its attention kernel (which = 0) and each
 * gqa_decode around its split-K streaming kernel (which = 1), on the
 * caller's stream.  gqa_timing_read waits for the recorded events, returns
 * the summed milliseconds and the launch count for `which`, and clears
 * them.  Not thread-safe; meant for a single benchmarking thread.
 */
int gqa_timing_enable(int on);
int gqa_timing_read(int which, double* total_ms, int64_t* count);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
