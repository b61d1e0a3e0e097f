// Internal launchers behind the C ABI (include/gqa.h).  Every launcher
// assumes the API layer has validated its arguments and enqueues on `st`.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstddef>
#include <tuple>
#include <type_traits>
#include <utility>

#include "common.h"

namespace gqa {

// ---- benchmark timing bound to kernel dispatches
// HIP events that the next launch_kernel of this host thread attaches to its
// dispatch (hipExtLaunchKernel): the start event takes the kernel's start
// time, the stop event its end.  Unlike hipEventRecord, which enqueues a
// marker that the next kernel then waits behind, this adds no packet to the
// stream between the kernels of a call.  Taken (and cleared) by that launch.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& next_launch_events();

// Events of one timed call: its first kernel's start and last kernel's end,
// and the opening and end of its main kernel's interval (call_start may be
// kernel_start, call_stop may be kernel_stop).
struct CallEvents {
  hipEvent_t call_start = nullptr, kernel_start = nullptr, kernel_stop = nullptr,
             call_stop = nullptr;
};

// Launches kernel k on st with the arguments converted to its parameter
// types, binding the pending LaunchEvents (if any) to the dispatch.
template <typename... P, typename... A>
hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, hipStream_t st, A&&... a) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count");
  const LaunchEvents ev = std::exchange(next_launch_events(), LaunchEvents{});
  std::tuple<std::decay_t<P>...> vals{static_cast<std::decay_t<P>>(std::forward<A>(a))...};
  void* args[sizeof...(P) > 0 ? sizeof...(P) : 1];
  std::apply([&](auto&... v) {
    size_t i = 0;
    ((args[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  if (ev.start || ev.stop)
    return hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, 0, st, ev.start,
                              ev.stop, 0);
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, 0, st);
}

constexpr int kPrefillTileK = 64;      // key padding granule of the prepared K/V
constexpr int kPrefillTileV = 32;      // keys per attention tile; V^T is stored per such tile
constexpr int kPrefillRowsWG = 256;    // stacked (position, head) rows per workgroup
constexpr int kPrefillPoolXcds = 8;    // per-XCD shared-tail counters of the attention kernel
constexpr int kPrefillPoolStride = 16; // ints between them (one 64-byte line each)
constexpr int kDecodeChunk = 1024;     // keys per decode split (fp32 cache)
constexpr int kDecodeChunkBf16 = 2048; // keys per decode split (bf16 cache)
constexpr int kDecodeMaxSplits = 8192;  // bound on the chunks of one sequence (8M keys)
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;  // static scratch of gqa_decode_noalloc

hipError_t launch_rope_apply(void* x, int dtype, int64_t B, int64_t L, int h, int d, int64_t pos0,
                             RopeParams rp, hipStream_t st);

hipError_t launch_rope_table(float2* cs, int64_t L, int d, int64_t pos0, RopeParams rp,
                             hipStream_t st);

hipError_t launch_kv_prepare_bf16(const uint16_t* k, const uint16_t* v, const RopeParams* rope,
                                  float2* cs_out, uint16_t* kp, uint16_t* vt, float* kmax, int* kexp,
                                  uint16_t* kc, uint16_t* vc, int64_t B, int64_t L, int64_t Lpad,
                                  int h_kv, int d, int64_t cap, int64_t src_rows,
                                  const int64_t* kstart, const int64_t* klen, int64_t kend,
                                  int* pool_ctr, hipStream_t st);

hipError_t launch_kv_prepare_f32(const float* k, const float* v, RopeParams rp, float* kp,
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

// pool_ctr (nullable): kPrefillPoolXcds workspace ints kPrefillPoolStride
// apart, zeroed by the preparation kernel launched before this one, for the
// tickets of the shared tail of the work
hipError_t launch_prefill_bf16(const uint16_t* q, const uint16_t* kp, const uint16_t* vt,
                               const float* kmax, const int* kexp, const float2* cs, void* o,
                               int out_bf16,
                               int64_t B, int64_t L, int64_t Lpad, int h_q, int h_kv, int d,
                               float scale, int causal, const int64_t* qstart,
                               const int64_t* qlen, int64_t kend, int* pool_ctr,
                               hipStream_t st);

// element strides of a K or V operand: sequence b, group u, key j start at
// base + b * batch + u * head + j * row
struct KvStrides {
  int64_t batch, head, row;
};

// rot_q: rotate the queries at their positions under rp (0: q is rotated
// already); rot_k: rotate the keys at their index (0: kp holds rotated keys)
hipError_t launch_prefill_f32(const float* q, const float* kp, const float* v, int rot_q,
                              int rot_k, RopeParams rp, void* o, int out_bf16, int64_t B, int64_t L,
                              int h_q, int h_kv, int d, float scale, int causal, KvStrides ks,
                              KvStrides vs,
                              const int64_t* qstart, const int64_t* qlen, int64_t kend,
                              hipStream_t st);

// chunks of a sequence of kv_len keys; the fp32 count (the larger) sizes
// workspaces
int decode_num_splits(int64_t kv_len, bool bf16 = false);
// Device address of this library's static decode scratch (kDecodeScratchBytes)
// on the current device, looked up once per device.
hipError_t decode_scratch(void** ptr);

// One decode call.  Scalar kv_len / q_pos, or per-sequence arrays (then
// kv_len bounds every length and sets the chunk count); k_new / v_new set:
// the new token of sequence b is appended at qpos_arr[b] first (if it lies
// in [0, append_end)), and kvl_from_pos makes its length qpos_arr[b] + 1.
// bt set: kc / vc are page pools [num_pages, h_kv, 2^ps_log2, d] addressed
// through the block table bt [B][max_pages].
struct DecodeArgs {
  const void* q;
  const void* kc;
  const void* vc;
  void* o;
  int in_bf16, out_bf16;
  int64_t B;
  int h_q, h_kv, d;
  int64_t cap, kv_len, q_pos;
  const int64_t* kvl_arr;
  const int64_t* qpos_arr;
  int kvl_from_pos, q_rotated;
  const int32_t* bt;
  int ps_log2;
  int64_t max_pages, num_pages;
  const void* k_new;
  const void* v_new;
  int64_t append_end;
  RopeParams rp;
  float scale;
};

// Workspace pieces of a decode call: partial states per (b, u, chunk, head)
// (max m, sum l, unnormalised o[d]) and, for an appending step, the rotated
// queries [B, h_q, d] in the input type.
struct DecodeWsPtrs {
  float* m;
  float* l;
  float* o;
  void* qr;
};

// ev (may be NULL): call_start opens the call's first kernel (the append
// step's preparation, else the split kernel); kernel_start is the split
// kernel's start, or the preparation's end when that precedes it (a start
// event inside the call would delay the split kernel); kernel_stop ends the
// split kernel, call_stop the merge.
hipError_t launch_decode(const DecodeArgs& a, const DecodeWsPtrs& w, hipStream_t st,
                         const CallEvents* ev);

// streaming read of `bytes` (a multiple of 16) at p, for benchmark context
hipError_t launch_stream_read(const void* p, size_t bytes, unsigned* sink, hipStream_t st);

}  // namespace gqa
