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
 * stream).  Scratch space is the caller's `workspace`.  A workspace serves
 * one call at a time: the call overwrites it (rotated K, transposed V,
 * per-tile norms, work counters, chunk states), so calls that can run at the
 * same time (on different streams) need workspaces of their own; calls
 * ordered on one stream may share one.
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
#define GQA_ERR_UNSUPPORTED (-2)  /* valid but not built: d not 64 or 128,
                                     or sizes past the kernels' index range
                                     (prefill: L or kend > 2^24, h_q or
                                     B*h_kv > 65535)                       */
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
 * bf16 inputs run on the matrix cores with fp32 accumulation: the rotated
 * Q (times scale * log2 e) and K are rounded once to fp16 for Q'K'^T, the
 * probabilities to bf16 for P.V.  fp16 bounds their range: an output row
 * is NaN when its query has such an element of magnitude >= 2^14, or when
 * any key its workgroup visits has a rotated K element >= 2^14 (a group's
 * later rows all see that key).  f32 inputs run in fp32 throughout.
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

/*
 * gqa_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that must not
 * call hipMalloc, harnesses that forbid it).  Arguments, layouts, results and
 * errors are those of gqa_decode; the chunk states live in a static array of
 * GQA_DECODE_NOALLOC_SCRATCH_BYTES that the library's code object reserves on
 * every GPU it runs on (held until the process ends).  A step needs
 *   B * h_q * ceil(kv_len / C) * (d + 2) * 4 bytes (each of its three
 *   parts rounded up to 256) + B * h_q * d * 4 (rounded up to 256),
 *   C = 2048 keys per chunk for GQA_BF16 and 1024 for GQA_F32;
 * a step beyond the limit returns GQA_ERR_UNSUPPORTED before anything is
 * enqueued (for d = 128 about 63,000 pairs of a query head and a chunk:
 * B = 32, h_q = 28 fit up to kv_len = 131072 in bf16, 65536 in fp32).  The
 * call allocates
 * nothing.  All calls on one GPU share its scratch: two calls whose work
 * overlaps on the device (on different streams, or from several threads on
 * one device without ordering) race and give wrong results; calls ordered
 * on one stream are safe.  Outputs equal gqa_decode's bit for bit.  The
 * call only launches kernels, so it can be captured into a HIP graph; its
 * first call on a device looks up the scratch's device address, so make
 * that call before any capture on that device.
 */
#define GQA_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
int gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                       void* o, int in_dtype, int out_dtype,
                       int64_t B, int h_q, int h_kv, int d, int64_t cap,
                       int64_t kv_len, int64_t q_pos, double theta, float scale,
                       void* stream);

/*
 * Autoregressive use around the path (walkthrough §4.1.3 closing note: the
 * per-layer cache keeps only the h_kv groups' K and V, and every step
 * appends the current token's K, V before attending).  The per-sequence
 * arrays below are int64 device memory of B entries; the host cannot read
 * them, so each call takes a host-side bound and the kernels check every
 * entry against it: a sequence whose entries break the stated conditions
 * gets NaN output rows and leaves the cache untouched, and no memory
 * outside the buffers is accessed.
 */

/* Bytes of workspace gqa_prefill_chunk needs when no sequence ends after
 * position kend - 1. */
size_t gqa_prefill_chunk_workspace_size(int in_dtype, int64_t B, int64_t kend,
                                        int h_kv, int d);

/*
 * Chunked causal prefill against the cache.  Sequence b brings len[b] new
 * rows (len NULL: C each) at positions start[b] .. start[b] + len[b] - 1,
 * laid out in q [B, C, h_q, d] and k/v [B, C, h_kv, d] (pre-RoPE, in_dtype);
 * the cache [B, cap, h_kv, d] (in_dtype) already holds rows
 * 0 .. start[b] - 1 (rotated K, as every call here writes it).  The call
 * 1) rotates the new K rows at their positions and writes them with the new
 *    V into cache rows start[b] + i,
 * 2) lets new query i attend to cache rows 0 .. start[b] + i,
 * and writes o [B, C, h_q, d] (out_dtype) rows i < len[b]; other rows are
 * not written.  Conditions: 0 <= start[b], 0 <= len[b] <= C,
 * start[b] + len[b] <= kend <= cap.  Splitting a prompt into chunks gives
 * the rows of the one-shot gqa_prefill (up to rounding).  k and v may both
 * be NULL when the cache already holds the chunk's rows (as written by
 * gqa_qkv_epilogue); step 1 is then skipped.  q_rotated != 0: q holds
 * queries rotated already (gqa_qkv_epilogue's q_out), used as given.
 * bf16 chunks have the operand range of gqa_prefill (NaN rows beyond it).
 */
int gqa_prefill_chunk(const void* q, const void* k, const void* v, void* o,
                      int in_dtype, int out_dtype,
                      int64_t B, int64_t C, int h_q, int h_kv, int d,
                      const int64_t* start, const int64_t* len, int64_t kend,
                      double theta, float scale, int q_rotated,
                      void* k_cache, void* v_cache, int64_t cap,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode with one length and one query position per sequence: q [B, h_q, d]
 * (pre-RoPE) of sequence b, rotated at q_pos[b], attends to its cache rows
 * 0 .. kv_len[b] - 1.  Conditions: 1 <= kv_len[b] <= max_kv_len <= cap and
 * kv_len[b] <= q_pos[b] + 1.  q_rotated != 0: q is rotated already
 * (gqa_qkv_epilogue's q_out) and used as given.  Workspace:
 * gqa_decode_workspace_size(..., cap).
 */
int gqa_decode_ragged(const void* q, const void* k_cache, const void* v_cache,
                      void* o, int in_dtype, int out_dtype,
                      int64_t B, int h_q, int h_kv, int d, int64_t cap,
                      const int64_t* kv_len, const int64_t* q_pos,
                      int64_t max_kv_len, double theta, float scale, int q_rotated,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * One autoregressive step with KV append: the new token of sequence b sits
 * at position pos[b]; its K (k_new [B, h_kv, d], pre-RoPE, rotated at
 * pos[b]) and V (v_new [B, h_kv, d]) are written to cache row pos[b], then
 * its query (q [B, h_q, d], rotated at pos[b]) attends to rows 0 .. pos[b].
 * Conditions: 0 <= pos[b] <= max_pos < cap.  Workspace as gqa_decode.
 */
int gqa_decode_append(const void* q, const void* k_new, const void* v_new,
                      void* k_cache, void* v_cache, void* o,
                      int in_dtype, int out_dtype,
                      int64_t B, int h_q, int h_kv, int d, int64_t cap,
                      const int64_t* pos, int64_t max_pos,
                      double theta, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The step before attention (walkthrough §4.1.3 steps 1-3 and §4.2: the
 * Q, K, V projections keep their bias; the flat outputs are cut into heads;
 * K is rotated at its position; the h_kv groups' K and V go to the cache).
 * qkv [B, C, (h_q + 2 h_kv) d] is the packed projection output without
 * bias: columns [0, h_q d) are the query heads, then h_kv key heads, then
 * h_kv value heads, each head's d columns contiguous; bias
 * [(h_q + 2 h_kv) d] (NULL: none).  Token i < len[b] (len NULL: C) of
 * sequence b sits at position p = start[b] + i:
 *   q_out [B, C, h_q, d] row i = RoPE(its query heads + bias, p),
 *   cache row p = RoPE(K + bias, p) and V + bias.
 * All tensors in `dtype`; sums and rotations in fp32, rounded once.
 * Conditions: 0 <= start[b], 0 <= len[b] <= C, start[b] + len[b] <= kend
 * <= cap; a sequence that breaks them is skipped (q_out rows and cache
 * untouched).  Follow with gqa_prefill_chunk(k = v = NULL, q_rotated = 1)
 * or gqa_decode_ragged(q_rotated = 1).
 */
int gqa_qkv_epilogue(const void* qkv, const void* bias, void* q_out,
                     void* k_cache, void* v_cache, int dtype,
                     int64_t B, int64_t C, int h_q, int h_kv, int d, int64_t cap,
                     const int64_t* start, const int64_t* len, int64_t kend,
                     double theta, void* stream);

/*
 * Decode over a paged cache.  K and V live in page pools
 * k_pool/v_pool [num_pages, h_kv, page_size, d] (in_dtype): a page holds
 * page_size consecutive positions of every KV head (PagedAttention manages
 * memory in blocks per KV head, "从 Qwen 1 到 Qwen 2 架构演进到底改了什么"
 * (nxmr.cn) §2).  block_table [B][max_pages] (int32, device): position j of
 * sequence b is row j % page_size of page block_table[b][j / page_size];
 * q_pos [B] (int64, device) is each query's position.
 *   k_new = v_new = NULL: sequence b attends to positions 0 .. kv_len[b]-1
 *     (kv_len [B] int64 device array, kv_len[b] <= q_pos[b] + 1);
 *   k_new, v_new [B, h_kv, d] set (kv_len NULL): one step with append --
 *     the new token's K (rotated at q_pos[b]) and V are written at position
 *     q_pos[b] first, then it attends to 0 .. q_pos[b].
 * page_size is a power of two; max_kv_len bounds every length and
 * max_kv_len <= max_pages * page_size.  A sequence whose length, position
 * or page ids are out of range gets NaN output (and no cache write).
 * q_rotated as for gqa_decode_ragged.  o [B, h_q, d] in out_dtype.
 */
size_t gqa_decode_paged_workspace_size(int64_t B, int h_q, int h_kv, int d,
                                       int64_t max_kv_len);

int gqa_decode_paged(const void* q, const void* k_new, const void* v_new,
                     void* k_pool, void* v_pool, void* o,
                     int in_dtype, int out_dtype,
                     int64_t B, int h_q, int h_kv, int d,
                     int page_size, int64_t num_pages,
                     const int32_t* block_table, int64_t max_pages,
                     const int64_t* kv_len, const int64_t* q_pos,
                     int64_t max_kv_len, double theta, float scale, int q_rotated,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * YaRN context extension of RoPE for every later call on this thread
 * (like gqa_last_error, the setting is per thread).  Beyond its 32K training
 * window Qwen2 enables YaRN at inference to reach 128K: each pair's
 * frequency is scaled as theta_i' = theta_i / s * alpha_i with a ramp
 * alpha_i over the dimensions ("Qwen-2 详解" (yudonglee.me) §6.2), and the
 * attention logits are rescaled for length extrapolation (walkthrough §5.3).
 * The ramp is the YaRN paper's (Peng et al., 2023): with
 *   D(n) = d ln(original_max_position / (2 pi n)) / (2 ln theta),
 * pair j keeps its frequency for j <= floor(D(beta_fast)), is divided by
 * `factor` for j >= ceil(D(beta_slow)), and is blended linearly in j between
 * (bounds clamped to [0, d-1]); cos and sin are multiplied by
 * 0.1 ln(factor) + 1, so Q'K'^T grows by its square.  factor = 1 restores
 * plain RoPE (the default).  Qwen2's long-context setting is factor 4,
 * original_max_position 32768, beta_fast 32, beta_slow 1.
 * Requires factor >= 1 and, when factor > 1, original_max_position >= 1 and
 * beta_fast > beta_slow > 0.  Cached keys must have been written under the
 * same setting.
 */
int gqa_set_rope_yarn(double factor, double original_max_position,
                      double beta_fast, double beta_slow);

/* Message for the last non-OK status on this thread ("" if none). */
const char* gqa_last_error(void);

/* Library build string. */
const char* gqa_version(void);

/*
 * Kernel timing for benchmarks.  While enabled, each gqa_prefill and
 * gqa_prefill_chunk call, and each decode call (contiguous or paged) except
 * gqa_decode_noalloc, binds HIP events to its own kernel dispatches on the
 * caller's stream (the event takes the dispatch's start or end time; no
 * marker is enqueued between the kernels): the start of its first kernel,
 * the end of its last, and the interval of its main kernel (prefill: the
 * attention kernel; decode: the split-K streaming kernel), which opens at
 * that kernel's start when it is the call's first kernel and otherwise at
 * the end of the kernel launched just before it (so it also holds the
 * launch gap between the two).  gqa_timing_read waits for them and returns
 * the summed milliseconds and the call count for `which`: 0 prefill main
 * kernels, 1 decode main kernels, 2 whole prefill calls (first kernel's
 * start to last kernel's end), 3 whole decode calls.  gqa_timing_enable(1)
 * drops earlier records.  Not thread-safe; meant for a single benchmarking
 * thread.
 */
int gqa_timing_enable(int on);
int gqa_timing_read(int which, double* total_ms, int64_t* count);

/*
 * Streaming-read helper for benchmarks (not part of the attention path): a
 * plain kernel reads `bytes` at device pointer p once, 16 bytes per lane
 * with non-temporal loads, on `stream`, and may write 4 bytes to the device
 * pointer `sink`.  Its rate is the context for the HBM-bound kernels'
 * roofline figures.  p must be 16-byte aligned and bytes a positive
 * multiple of 16 (else GQA_ERR_INVALID_ARG).  `stream` is a hipStream_t
 * (NULL: the default stream), as for every other entry point.  Asynchronous.
 */
int gqa_stream_read(const void* p, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
