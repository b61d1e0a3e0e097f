// Internal launchers behind the C ABI (include/gqa.h).  Every launcher
// assumes the API layer has validated its arguments and enqueues on `st`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace gqa {

constexpr int kPrefillTileK = 64;      // key padding granule of the prepared K/V
constexpr int kPrefillTileV = 32;      // keys per attention tile; V^T is stored per such tile
constexpr int kPrefillRowsWG = 256;    // stacked (position, head) rows per workgroup
constexpr int kDecodeChunk = 1024;     // keys per decode split
constexpr int kDecodeMaxSplitsLds = 8192;  // chunk weights staged by the merge kernel

hipError_t launch_rope_apply(void* x, int dtype, int64_t B, int64_t L, int h, int d, int64_t pos0,
                             RopeParams rp, hipStream_t st);

hipError_t launch_rope_table(float2* cs, int64_t L, int d, int64_t pos0, RopeParams rp,
                             hipStream_t st);

hipError_t launch_kv_prepare_bf16(const uint16_t* k, const uint16_t* v, const float2* cs,
                                  uint16_t* kp, uint16_t* vt, float* kmax, uint16_t* kc,
                                  uint16_t* vc, int64_t B, int64_t L, int64_t Lpad, int h_kv, int d,
                                  int64_t cap, int64_t src_rows, const int64_t* kstart,
                                  const int64_t* klen, int64_t kend, hipStream_t st);

hipError_t launch_kv_prepare_f32(const float* k, const float* v, const float2* cs, float* kp,
                                 float* kc, float* vc, int64_t B, int64_t L, int h_kv, int d,
                                 int64_t cap, hipStream_t st);

// bt != NULL: kc/vc are page pools [num_pages, h_kv, 2^ps_log2, d] addressed
// through the block table bt [B][max_pages]
hipError_t launch_cache_append(const void* k, const void* v, void* kc, void* vc, int bf16,
                               const int64_t* start, const int64_t* len, int64_t B, int64_t C,
                               int h_kv, int d, int64_t cap, int64_t end, RopeParams rp,
                               hipStream_t st, const int32_t* bt = nullptr, int ps_log2 = 0,
                               int64_t max_pages = 0, int64_t num_pages = 0);

hipError_t launch_qkv_epilogue(const void* x, const void* bias, void* q_out, void* kc, void* vc,
                               int bf16, const int64_t* start, const int64_t* len, int64_t B,
                               int64_t C, int h_q, int h_kv, int d, int64_t cap, int64_t end,
                               RopeParams rp, hipStream_t st);

hipError_t launch_prefill_bf16(const uint16_t* q, const uint16_t* kp, const uint16_t* vt,
                               const float* kmax, const float2* cs, void* o, int out_bf16,
                               int64_t B, int64_t L, int64_t Lpad, int h_q, int h_kv, int d,
                               float scale, int causal, const int64_t* qstart,
                               const int64_t* qlen, int64_t kend, hipStream_t st);

// element strides of a K or V operand: sequence b, group u, key j start at
// base + b * batch + u * head + j * row
struct KvStrides {
  int64_t batch, head, row;
};

// cs: the queries' cos/sin table (NULL: q is rotated already); kcs: the
// keys' table, position = key index (NULL: kp holds rotated keys)
hipError_t launch_prefill_f32(const float* q, const float* kp, const float* v, const float2* cs,
                              const float2* kcs, void* o, int out_bf16, int64_t B, int64_t L,
                              int h_q, int h_kv, int d, float scale, int causal, KvStrides ks,
                              KvStrides vs,
                              const int64_t* qstart, const int64_t* qlen, int64_t kend,
                              hipStream_t st);

int decode_num_splits(int64_t kv_len);

hipError_t launch_decode(const void* q, const void* kc, const void* vc, void* o, int in_bf16,
                         int out_bf16, int64_t B, int h_q, int h_kv, int d, int64_t cap,
                         int64_t kv_len, int64_t q_pos, const int64_t* kvl_arr,
                         const int64_t* qpos_arr, int kvl_from_pos, int q_rotated,
                         const int32_t* bt, int ps_log2, int64_t max_pages, int64_t num_pages,
                         RopeParams rp,
                         float scale, float* ws_m, float* ws_l, float* ws_o, hipStream_t st,
                         hipEvent_t ev_begin, hipEvent_t ev_end);

// streaming read of `bytes` (a multiple of 16) at p, for benchmark context
hipError_t launch_stream_read(const void* p, size_t bytes, unsigned* sink, hipStream_t st);

}  // namespace gqa
