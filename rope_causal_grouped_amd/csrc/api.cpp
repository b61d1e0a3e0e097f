// C ABI of the library (declared in include/gqa.h): argument validation,
// workspace carving and kernel dispatch.  Nothing here allocates device
// memory or synchronises the caller's stream.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <utility>
#include <vector>

#include "gqa.h"
#include "launch.h"

namespace gqa {

LaunchEvents& next_launch_events() {
  thread_local LaunchEvents ev;
  return ev;
}

}  // namespace gqa

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(GQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool dtype_ok(int dt) { return dt == GQA_F32 || dt == GQA_BF16; }

// ---- benchmark timing: HIP events bound to the dispatches of a call (its
// first kernel's start, the opening and end of its main kernel's interval,
// its last kernel's end); see gqa::launch_kernel and TimedCall
struct Timing {
  bool on = false;
  std::vector<gqa::CallEvents> rec[2];   // 0: prefill calls, 1: decode calls
  std::vector<hipEvent_t> pool;
  hipEvent_t one() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    return hipEventCreate(&e) == hipSuccess ? e : nullptr;
  }
  // events of one call; own_start / own_stop: the call's first / last
  // kernel is not its main kernel
  bool take(gqa::CallEvents& ev, bool own_start, bool own_stop) {
    ev.kernel_start = one();
    ev.kernel_stop = one();
    ev.call_start = own_start ? one() : ev.kernel_start;
    ev.call_stop = own_stop ? one() : ev.kernel_stop;
    if (ev.kernel_start && ev.kernel_stop && ev.call_start && ev.call_stop) return true;
    release(ev);
    ev = gqa::CallEvents{};
    return false;
  }
  void release(const gqa::CallEvents& ev) {
    for (hipEvent_t e : {ev.kernel_start, ev.kernel_stop})
      if (e) pool.push_back(e);
    if (ev.call_start && ev.call_start != ev.kernel_start) pool.push_back(ev.call_start);
    if (ev.call_stop && ev.call_stop != ev.kernel_stop) pool.push_back(ev.call_stop);
  }
  void clear() {
    for (auto& r : rec) {
      for (auto& ev : r) release(ev);
      r.clear();
    }
  }
};
Timing g_timing;

// Timing of one API call while timing is on.  The call's first kernel takes
// call_start as its start event and its last kernel call_stop as its stop
// event.  The main kernel's interval opens at its own start when it is the
// call's first kernel, else at the end of the kernel launched just before it
// (a stop event: a start event bound inside the call would hold the main
// kernel back by a few microseconds, a stop event does not), so that
// interval also holds the launch gap between the two.  bind() hands events
// to the next launch_kernel; done() keeps the record.  A call that returns
// before done() gives its events back, and no pending binding outlives it.
class TimedCall {
 public:
  TimedCall(int which, bool own_start, bool own_stop, bool allow = true) : which_(which) {
    if (g_timing.on && allow) on_ = g_timing.take(ev_, own_start, own_stop);
  }
  ~TimedCall() {
    gqa::next_launch_events() = gqa::LaunchEvents{};
    if (on_ && !kept_) g_timing.release(ev_);
  }
  TimedCall(const TimedCall&) = delete;
  TimedCall& operator=(const TimedCall&) = delete;
  const gqa::CallEvents* events() const { return on_ ? &ev_ : nullptr; }
  const gqa::CallEvents& ev() const { return ev_; }
  void bind(hipEvent_t start, hipEvent_t stop) {
    if (on_) gqa::next_launch_events() = gqa::LaunchEvents{start, stop};
  }
  void done() {
    if (on_ && !kept_) {
      g_timing.rec[which_].push_back(ev_);
      kept_ = true;
    }
  }

 private:
  int which_;
  bool on_ = false, kept_ = false;
  gqa::CallEvents ev_;
};

// YaRN context extension of RoPE (gqa_set_rope_yarn), per thread like the
// error message; factor 1 is plain RoPE.
struct YarnConfig {
  double factor = 1.0, original_max_position = 0.0, beta_fast = 32.0, beta_slow = 1.0;
};
thread_local YarnConfig g_yarn;

// The call's RoPE parameters: base theta, and the YaRN blend of this thread.
// Pair j keeps its frequency below the correction dimension of beta_fast
// rotations over the original context and is divided by the factor above
// that of beta_slow rotations, linearly in j between; cos and sin carry the
// attention factor 0.1 ln(factor) + 1.
gqa::RopeParams rope_params(double theta, int d) {
  gqa::RopeParams rp{std::log2(theta), 1.0, 0.0, 1.0, 1.0f};
  const YarnConfig& y = g_yarn;
  if (y.factor == 1.0) return rp;
  const double two_ln_theta = 2.0 * std::log(theta);
  auto corr_dim = [&](double rotations) {
    return d * std::log(y.original_max_position / (rotations * 2.0 * M_PI)) / two_ln_theta;
  };
  double lo = std::floor(corr_dim(y.beta_fast));
  double hi = std::ceil(corr_dim(y.beta_slow));
  if (lo < 0.0) lo = 0.0;
  if (hi > d - 1) hi = d - 1;
  if (hi == lo) hi += 0.001;
  rp.inv_factor = 1.0 / y.factor;
  rp.ramp_lo = lo;
  rp.ramp_hi = hi;
  rp.mscale = (float)(0.1 * std::log(y.factor) + 1.0);
  return rp;
}

int check_heads(int h_q, int h_kv) {
  if (h_q < 1 || h_kv < 1)
    return fail(GQA_ERR_INVALID_ARG, "head counts must be >= 1 (h_q=%d, h_kv=%d)", h_q, h_kv);
  if (h_q % h_kv != 0)
    return fail(GQA_ERR_INVALID_ARG,
                "h_q must be a multiple of h_kv (h_q=%d, h_kv=%d): each group of g = h_q/h_kv "
                "query heads shares one K/V head",
                h_q, h_kv);
  return GQA_OK;
}

int check_d(int d) {
  if (d < 2 || (d & 1)) return fail(GQA_ERR_INVALID_ARG, "d=%d: RoPE needs an even head size", d);
  if (d != 64 && d != 128)
    return fail(GQA_ERR_UNSUPPORTED, "d=%d: kernels are built for head sizes 64 and 128", d);
  return GQA_OK;
}

int check_theta_scale(double theta, float scale) {
  if (!(theta > 1.0) || !std::isfinite(theta))
    return fail(GQA_ERR_INVALID_ARG, "theta=%g must be finite and > 1", theta);
  if (!std::isfinite(scale)) return fail(GQA_ERR_INVALID_ARG, "scale must be finite");
  return GQA_OK;
}

int64_t prefill_lpad(int64_t L) { return (L + gqa::kPrefillTileK - 1) / gqa::kPrefillTileK * gqa::kPrefillTileK; }

// workspace pieces of gqa_prefill
struct PrefillWs {
  size_t cs_off, kp_off, vt_off, kmax_off, kexp_off, ctr_off, total;
};

PrefillWs prefill_ws(int in_dtype, int64_t B, int64_t L, int h_kv, int d) {
  PrefillWs w{};
  const size_t cs = align256((size_t)L * (size_t)(d / 2) * sizeof(float2));
  w.cs_off = 0;
  w.kp_off = cs;
  if (in_dtype == GQA_BF16) {
    const size_t kp = align256((size_t)B * h_kv * prefill_lpad(L) * d * 2);
    w.vt_off = cs + kp;
    const size_t tiles = align256((size_t)B * h_kv * (prefill_lpad(L) / gqa::kPrefillTileK) * 4);
    w.kmax_off = cs + 2 * kp;
    w.kexp_off = w.kmax_off + tiles;
    w.ctr_off = w.kexp_off + tiles;     // the attention kernel's ticket counters
    w.total = w.ctr_off + align256(gqa::kPrefillPoolXcds * gqa::kPrefillPoolStride * sizeof(int));
  } else {
    const size_t kp = align256((size_t)B * h_kv * L * d * 4);
    w.vt_off = cs + kp;
    w.kmax_off = cs + kp;
    w.kexp_off = cs + kp;
    w.ctr_off = cs + kp;
    w.total = cs + kp;
  }
  return w;
}

static_assert(GQA_DECODE_NOALLOC_SCRATCH_BYTES == gqa::kDecodeScratchBytes,
              "the header's scratch size is the kernels' one");

struct DecodeWs {
  size_t m_off, l_off, o_off, qr_off, total;
};

// partial states per (b, u, chunk, head); rotated queries [B, h_q, d] of an
// appending step (fp32 size, so one layout serves both input types)
DecodeWs decode_ws(int64_t B, int h_q, int h_kv, int d, int64_t cap, bool bf16 = false) {
  const int g = h_q / h_kv;
  const size_t n = (size_t)B * h_kv * gqa::decode_num_splits(cap, bf16) * g;
  DecodeWs w{};
  w.m_off = 0;
  w.l_off = align256(n * 4);
  w.o_off = w.l_off + align256(n * 4);
  w.qr_off = w.o_off + align256(n * (size_t)d * 4);
  w.total = w.qr_off + align256((size_t)B * h_q * d * 4);
  return w;
}

gqa::DecodeWsPtrs decode_ws_ptrs(void* workspace, const DecodeWs& ws) {
  char* b = (char*)workspace;
  return {(float*)(b + ws.m_off), (float*)(b + ws.l_off), (float*)(b + ws.o_off),
          (void*)(b + ws.qr_off)};
}

}  // namespace

extern "C" {

const char* gqa_last_error(void) { return g_err.c_str(); }

const char* gqa_version(void) { return "gqa-mi355x 0.1 (gfx950)"; }

int gqa_rope_apply(void* x, int dtype, int64_t B, int64_t L, int h, int d, int64_t pos0,
                   double theta, void* stream) {
  g_err.clear();
  if (!x) return fail(GQA_ERR_INVALID_ARG, "x is NULL");
  if (!dtype_ok(dtype)) return fail(GQA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (B < 1 || L < 1 || h < 1) return fail(GQA_ERR_INVALID_ARG, "B, L, h must be >= 1");
  if (d < 2 || (d & 1)) return fail(GQA_ERR_INVALID_ARG, "d=%d: RoPE needs an even head size", d);
  if (pos0 < 0 || pos0 > (INT64_C(1) << 40)) return fail(GQA_ERR_INVALID_ARG, "pos0 out of range");
  if (int rc = check_theta_scale(theta, 1.0f)) return rc;
  if (!aligned16(x)) return fail(GQA_ERR_INVALID_ARG, "x must be 16-byte aligned");
  hipError_t e = gqa::launch_rope_apply(x, dtype, B, L, h, d, pos0, rope_params(theta, d),
                                        (hipStream_t)stream);
  return e == hipSuccess ? GQA_OK : hip_fail(e, "rope_apply launch");
}

size_t gqa_prefill_workspace_size(int in_dtype, int64_t B, int64_t L, int h_kv, int d) {
  if (!dtype_ok(in_dtype) || B < 1 || L < 1 || h_kv < 1 || d < 2) return 0;
  return prefill_ws(in_dtype, B, L, h_kv, d).total;
}

int gqa_prefill(const void* q, const void* k, const void* v, void* o, int in_dtype, int out_dtype,
                int64_t B, int64_t L, int h_q, int h_kv, int d, double theta, float scale,
                int causal, void* k_cache, void* v_cache, int64_t cap, void* workspace,
                size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!q || !k || !v || !o) return fail(GQA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(GQA_ERR_INVALID_ARG, "unknown dtype (in=%d, out=%d)", in_dtype, out_dtype);
  if (B < 1 || L < 1) return fail(GQA_ERR_INVALID_ARG, "B and L must be >= 1");
  if (int rc = check_heads(h_q, h_kv)) return rc;
  if (int rc = check_d(d)) return rc;
  if (int rc = check_theta_scale(theta, scale)) return rc;
  if ((k_cache == nullptr) != (v_cache == nullptr))
    return fail(GQA_ERR_INVALID_ARG, "k_cache and v_cache must both be set or both be NULL");
  if (k_cache && cap < L) return fail(GQA_ERR_INVALID_ARG, "cap=%lld < L=%lld", (long long)cap, (long long)L);
  const int g = h_q / h_kv;
  if (L * g + gqa::kPrefillRowsWG > INT_MAX || B * h_kv > 65535 || h_q > 65535 ||
      L > (INT64_C(1) << 24))
    return fail(GQA_ERR_UNSUPPORTED, "sizes exceed the kernels' index range");
  const int64_t n_rb = (L * g + gqa::kPrefillRowsWG - 1) / gqa::kPrefillRowsWG;
  if (n_rb * B * h_kv > INT_MAX) return fail(GQA_ERR_UNSUPPORTED, "grid too large");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(workspace))
    return fail(GQA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const PrefillWs ws = prefill_ws(in_dtype, B, L, h_kv, d);
  if (!workspace || workspace_bytes < ws.total)
    return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws.total,
                workspace ? workspace_bytes : (size_t)0);

  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)workspace;
  float2* cs = (float2*)(wsb + ws.cs_off);
  const gqa::RopeParams rp = rope_params(theta, d);
  hipError_t e = hipSuccess;
  // timing: the first kernel opens the call; the attention kernel's
  // interval opens at its own start when it is the first kernel, else at
  // the end of the preparation pass before it; the attention kernel ends both
  const bool bf16_in = in_dtype == GQA_BF16;
  TimedCall tc(0, bf16_in || k_cache != nullptr, false);
  const gqa::CallEvents& te = tc.ev();
  if (bf16_in) {   // the preparation kernel also writes the queries' cos/sin table
    const int64_t Lpad = prefill_lpad(L);
    uint16_t* kp = (uint16_t*)(wsb + ws.kp_off);
    uint16_t* vt = (uint16_t*)(wsb + ws.vt_off);
    float* kmax = (float*)(wsb + ws.kmax_off);
    int* kexp = (int*)(wsb + ws.kexp_off);
    tc.bind(te.call_start, te.kernel_start);
    int* ctr = (int*)(wsb + ws.ctr_off);
    e = gqa::launch_kv_prepare_bf16((const uint16_t*)k, (const uint16_t*)v, &rp, cs, kp, vt,
                                    kmax, kexp, (uint16_t*)k_cache, (uint16_t*)v_cache, B, L, Lpad,
                                    h_kv, d, cap, L, nullptr, nullptr, L, ctr, st);
    if (e != hipSuccess) return hip_fail(e, "K/V preparation launch");
    tc.bind(nullptr, te.kernel_stop);
    e = gqa::launch_prefill_bf16((const uint16_t*)q, kp, vt, kmax, kexp, cs, o,
                                 out_dtype == GQA_BF16, B, L, Lpad, h_q, h_kv, d, scale, causal,
                                 nullptr, nullptr, L, ctr, st);
  } else {         // fp32: the kernels form their cos/sin themselves
    const gqa::KvStrides vsd{L * h_kv * d, d, (int64_t)h_kv * d};       // [B, L, h_kv, d]
    if (k_cache) {   // rotated K and V into the cache; attention reads the rotated copy
      float* kp = (float*)(wsb + ws.kp_off);
      tc.bind(te.call_start, te.kernel_start);
      e = gqa::launch_kv_prepare_f32((const float*)k, (const float*)v, rp, kp, (float*)k_cache,
                                     (float*)v_cache, B, L, h_kv, d, cap, st);
      if (e != hipSuccess) return hip_fail(e, "K preparation launch");
      tc.bind(nullptr, te.kernel_stop);
      const gqa::KvStrides ksd{(int64_t)h_kv * L * d, L * d, d};        // [B][h_kv][L][d]
      e = gqa::launch_prefill_f32((const float*)q, kp, (const float*)v, 1, 0, rp, o,
                                  out_dtype == GQA_BF16, B, L, h_q, h_kv, d, scale, causal, ksd,
                                  vsd, nullptr, nullptr, L, st);
    } else {         // no cache: one kernel, which rotates K as it stages each tile
      tc.bind(te.kernel_start, te.kernel_stop);
      e = gqa::launch_prefill_f32((const float*)q, (const float*)k, (const float*)v, 1, 1, rp, o,
                                  out_dtype == GQA_BF16, B, L, h_q, h_kv, d, scale, causal, vsd,
                                  vsd, nullptr, nullptr, L, st);
    }
  }
  if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  tc.done();
  return GQA_OK;
}

size_t gqa_decode_workspace_size(int64_t B, int h_q, int h_kv, int d, int64_t cap) {
  if (B < 1 || h_q < 1 || h_kv < 1 || h_q % h_kv || d < 2 || cap < 1) return 0;
  return decode_ws(B, h_q, h_kv, d, cap).total;
}

}  // extern "C"

namespace {

// gqa_decode with a caller's workspace, or (noalloc) with the library's
// static scratch of the current device.
int decode_call(const void* q, const void* k_cache, const void* v_cache, void* o, int in_dtype,
                int out_dtype, int64_t B, int h_q, int h_kv, int d, int64_t cap, int64_t kv_len,
                int64_t q_pos, double theta, float scale, void* workspace,
                size_t workspace_bytes, void* stream, bool noalloc) {
  g_err.clear();
  if (!q || !k_cache || !v_cache || !o)
    return fail(GQA_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be non-NULL");
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(GQA_ERR_INVALID_ARG, "unknown dtype (in=%d, out=%d)", in_dtype, out_dtype);
  if (B < 1) return fail(GQA_ERR_INVALID_ARG, "B must be >= 1");
  if (int rc = check_heads(h_q, h_kv)) return rc;
  if (int rc = check_d(d)) return rc;
  if (int rc = check_theta_scale(theta, scale)) return rc;
  if (cap < 1) return fail(GQA_ERR_INVALID_ARG, "cap must be >= 1");
  if (kv_len < 1 || kv_len > cap)
    return fail(GQA_ERR_INVALID_ARG, "kv_len=%lld outside [1, cap=%lld]", (long long)kv_len,
                (long long)cap);
  if (q_pos < 0 || kv_len > q_pos + 1)
    return fail(GQA_ERR_INVALID_ARG,
                "kv_len=%lld > q_pos+1=%lld: the query may only see keys at or before its position",
                (long long)kv_len, (long long)(q_pos + 1));
  if (cap > (INT64_C(1) << 30) || q_pos > (INT64_C(1) << 40) || B > 65535 || h_q > 65535 ||
      gqa::decode_num_splits(cap) > gqa::kDecodeMaxSplits)
    return fail(GQA_ERR_UNSUPPORTED, "sizes exceed the kernels' index range");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      !aligned16(workspace))
    return fail(GQA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  // the chunk states are laid out for the chunks of kv_len keys (the caller's
  // workspace is sized by cap, which only leaves room to spare)
  const DecodeWs ws = noalloc ? decode_ws(B, h_q, h_kv, d, kv_len, in_dtype == GQA_BF16)
                               : decode_ws(B, h_q, h_kv, d, cap);
  if (noalloc) {
    if (ws.total > gqa::kDecodeScratchBytes)
      return fail(GQA_ERR_UNSUPPORTED,
                  "this step needs %zu bytes of scratch; the static scratch holds %zu "
                  "(use gqa_decode with a workspace)",
                  ws.total, gqa::kDecodeScratchBytes);
    const hipError_t e = gqa::decode_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, "static decode scratch lookup");
  } else if (!workspace || workspace_bytes < ws.total) {
    return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws.total,
                workspace ? workspace_bytes : (size_t)0);
  }
  gqa::DecodeArgs a{};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.o = o;
  a.in_bf16 = in_dtype == GQA_BF16;
  a.out_bf16 = out_dtype == GQA_BF16;
  a.B = B;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.d = d;
  a.cap = cap;
  a.kv_len = kv_len;
  a.q_pos = q_pos;
  a.rp = rope_params(theta, d);
  a.scale = scale;
  TimedCall tc(1, false, true, !noalloc);
  hipError_t e = gqa::launch_decode(a, decode_ws_ptrs(workspace, ws), (hipStream_t)stream,
                                    tc.events());
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  tc.done();
  return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, int in_dtype,
               int out_dtype, int64_t B, int h_q, int h_kv, int d, int64_t cap, int64_t kv_len,
               int64_t q_pos, double theta, float scale, void* workspace, size_t workspace_bytes,
               void* stream) {
  return decode_call(q, k_cache, v_cache, o, in_dtype, out_dtype, B, h_q, h_kv, d, cap, kv_len,
                     q_pos, theta, scale, workspace, workspace_bytes, stream, false);
}

int gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                       int in_dtype, int out_dtype, int64_t B, int h_q, int h_kv, int d,
                       int64_t cap, int64_t kv_len, int64_t q_pos, double theta, float scale,
                       void* stream) {
  return decode_call(q, k_cache, v_cache, o, in_dtype, out_dtype, B, h_q, h_kv, d, cap, kv_len,
                     q_pos, theta, scale, nullptr, 0, stream, true);
}

size_t gqa_prefill_chunk_workspace_size(int in_dtype, int64_t B, int64_t kend, int h_kv, int d) {
  if (!dtype_ok(in_dtype) || B < 1 || kend < 1 || h_kv < 1 || d < 2) return 0;
  const PrefillWs w = prefill_ws(in_dtype, B, kend, h_kv, d);
  return in_dtype == GQA_BF16 ? w.total : w.kp_off;   // fp32 chunks read K from the cache
}

int gqa_prefill_chunk(const void* q, const void* k, const void* v, void* o, int in_dtype,
                      int out_dtype, int64_t B, int64_t C, int h_q, int h_kv, int d,
                      const int64_t* start, const int64_t* len, int64_t kend, double theta,
                      float scale, int q_rotated, void* k_cache, void* v_cache, int64_t cap,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!q || !o || !start || !k_cache || !v_cache)
    return fail(GQA_ERR_INVALID_ARG, "q, o, start, k_cache and v_cache must be non-NULL");
  if ((k == nullptr) != (v == nullptr))
    return fail(GQA_ERR_INVALID_ARG, "k and v must both be set or both be NULL");
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(GQA_ERR_INVALID_ARG, "unknown dtype (in=%d, out=%d)", in_dtype, out_dtype);
  if (B < 1 || C < 1) return fail(GQA_ERR_INVALID_ARG, "B and C must be >= 1");
  if (int rc = check_heads(h_q, h_kv)) return rc;
  if (int rc = check_d(d)) return rc;
  if (int rc = check_theta_scale(theta, scale)) return rc;
  if (kend < 1 || kend > cap)
    return fail(GQA_ERR_INVALID_ARG, "kend=%lld outside [1, cap=%lld]", (long long)kend,
                (long long)cap);
  const int g = h_q / h_kv;
  if (C * g + gqa::kPrefillRowsWG > INT_MAX || B * h_kv > 65535 || h_q > 65535 ||
      kend > (INT64_C(1) << 24))
    return fail(GQA_ERR_UNSUPPORTED, "sizes exceed the kernels' index range");
  const int64_t n_rb = (C * g + gqa::kPrefillRowsWG - 1) / gqa::kPrefillRowsWG;
  if (n_rb * B * h_kv > INT_MAX) return fail(GQA_ERR_UNSUPPORTED, "grid too large");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(workspace))
    return fail(GQA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const size_t need = gqa_prefill_chunk_workspace_size(in_dtype, B, kend, h_kv, d);
  if (!workspace || workspace_bytes < need)
    return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);

  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)workspace;
  const PrefillWs ws = prefill_ws(in_dtype, B, kend, h_kv, d);
  float2* cs = (float2*)(wsb + ws.cs_off);
  const gqa::RopeParams rp = rope_params(theta, d);
  // timing: the first kernel opens the call; the attention kernel's
  // interval opens at its own start when it is the first kernel, else at
  // the end of the kernel before it; the attention kernel ends both
  const bool bf16_in = in_dtype == GQA_BF16;
  TimedCall tc(0, bf16_in || k != nullptr, false);
  const gqa::CallEvents& te = tc.ev();
  hipError_t e = hipSuccess;
  if (bf16_in) {   // the queries' cos/sin table (the fp32 kernel forms its own)
    tc.bind(te.call_start, nullptr);
    e = gqa::launch_rope_table(cs, kend, d, 0, rp, st);
    if (e != hipSuccess) return hip_fail(e, "rope table launch");
  }
  // 1) the chunk's rotated K and its V into the cache rows start[b] + i
  //    (k, v NULL: an earlier call, e.g. gqa_qkv_epilogue, put them there)
  if (k) {
    tc.bind(bf16_in ? nullptr : te.call_start, bf16_in ? nullptr : te.kernel_start);
    e = gqa::launch_cache_append(k, v, k_cache, v_cache, in_dtype == GQA_BF16, start, len, B, C,
                                 h_kv, d, cap, kend, rp, st);
    if (e != hipSuccess) return hip_fail(e, "cache append launch");
  }

  if (bf16_in) {
    // 2) keys 0 .. start[b] + len[b] - 1 of the cache into the attention layout
    const int64_t Lpad = prefill_lpad(kend);
    uint16_t* kp = (uint16_t*)(wsb + ws.kp_off);
    uint16_t* vt = (uint16_t*)(wsb + ws.vt_off);
    float* kmax = (float*)(wsb + ws.kmax_off);
    int* kexp = (int*)(wsb + ws.kexp_off);
    tc.bind(nullptr, te.kernel_start);
    int* ctr = (int*)(wsb + ws.ctr_off);
    e = gqa::launch_kv_prepare_bf16((const uint16_t*)k_cache, (const uint16_t*)v_cache, nullptr,
                                    nullptr, kp, vt, kmax, kexp, nullptr, nullptr, B, C, Lpad, h_kv,
                                    d, cap, cap, start, len, kend, ctr, st);
    if (e != hipSuccess) return hip_fail(e, "K/V preparation launch");
    // 3) the chunk's queries against them
    tc.bind(nullptr, te.kernel_stop);
    e = gqa::launch_prefill_bf16((const uint16_t*)q, kp, vt, kmax, kexp, q_rotated ? nullptr : cs, o,
                                 out_dtype == GQA_BF16, B, C, Lpad, h_q, h_kv, d, scale, 1, start,
                                 len, kend, ctr, st);
  } else {
    // 2) the chunk's queries against the cache itself
    const gqa::KvStrides csd{cap * h_kv * d, d, (int64_t)h_kv * d};   // [B, cap, h_kv, d]
    tc.bind(k ? nullptr : te.kernel_start, te.kernel_stop);
    e = gqa::launch_prefill_f32((const float*)q, (const float*)k_cache, (const float*)v_cache,
                                q_rotated ? 0 : 1, 0, rp, o, out_dtype == GQA_BF16, B, C, h_q, h_kv,
                                d, scale, 1, csd, csd, start, len, kend, st);
  }
  if (e != hipSuccess) return hip_fail(e, "chunked prefill launch");
  tc.done();
  return GQA_OK;
}

namespace {

// host checks shared by the ragged decode entry points
int decode_ragged_check(const void* q, const void* k_cache, const void* v_cache, void* o,
                        int in_dtype, int out_dtype, int64_t B, int h_q, int h_kv, int d,
                        int64_t cap, int64_t max_kv_len, double theta, float scale,
                        void* workspace, size_t workspace_bytes) {
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(GQA_ERR_INVALID_ARG, "unknown dtype (in=%d, out=%d)", in_dtype, out_dtype);
  if (B < 1) return fail(GQA_ERR_INVALID_ARG, "B must be >= 1");
  if (int rc = check_heads(h_q, h_kv)) return rc;
  if (int rc = check_d(d)) return rc;
  if (int rc = check_theta_scale(theta, scale)) return rc;
  if (cap < 1) return fail(GQA_ERR_INVALID_ARG, "cap must be >= 1");
  if (max_kv_len < 1 || max_kv_len > cap)
    return fail(GQA_ERR_INVALID_ARG, "longest sequence %lld outside [1, cap=%lld]",
                (long long)max_kv_len, (long long)cap);
  if (cap > (INT64_C(1) << 30) || B > 65535 || h_q > 65535 ||
      gqa::decode_num_splits(cap) > gqa::kDecodeMaxSplits)
    return fail(GQA_ERR_UNSUPPORTED, "sizes exceed the kernels' index range");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      !aligned16(workspace))
    return fail(GQA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const DecodeWs ws = decode_ws(B, h_q, h_kv, d, cap);
  if (!workspace || workspace_bytes < ws.total)
    return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws.total,
                workspace ? workspace_bytes : (size_t)0);
  return GQA_OK;
}

// dispatch of a checked ragged decode; k_new / v_new set: the new token is
// appended at q_pos[b] first (if q_pos[b] < append_end)
int decode_ragged_launch(const void* q, const void* k_cache, const void* v_cache, void* o,
                         int in_dtype, int out_dtype, int64_t B, int h_q, int h_kv, int d,
                         int64_t cap, const int64_t* kvl, const int64_t* qpos, int from_pos,
                         int q_rotated, int64_t max_kv_len, double theta, float scale,
                         void* workspace, hipStream_t st, const int32_t* bt = nullptr,
                         int ps_log2 = 0, int64_t max_pages = 0, int64_t num_pages = 0,
                         const void* k_new = nullptr, const void* v_new = nullptr,
                         int64_t append_end = 0) {
  const DecodeWs ws = decode_ws(B, h_q, h_kv, d, cap);
  gqa::DecodeArgs a{};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.o = o;
  a.in_bf16 = in_dtype == GQA_BF16;
  a.out_bf16 = out_dtype == GQA_BF16;
  a.B = B;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.d = d;
  a.cap = cap;
  a.kv_len = max_kv_len;
  a.kvl_arr = kvl;
  a.qpos_arr = qpos;
  a.kvl_from_pos = from_pos;
  a.q_rotated = q_rotated;
  a.bt = bt;
  a.ps_log2 = ps_log2;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.k_new = k_new;
  a.v_new = v_new;
  a.append_end = append_end;
  a.rp = rope_params(theta, d);
  a.scale = scale;
  TimedCall tc(1, k_new != nullptr, true);
  hipError_t e = gqa::launch_decode(a, decode_ws_ptrs(workspace, ws), st, tc.events());
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  tc.done();
  return GQA_OK;
}

}  // namespace

int gqa_decode_ragged(const void* q, const void* k_cache, const void* v_cache, void* o,
                      int in_dtype, int out_dtype, int64_t B, int h_q, int h_kv, int d,
                      int64_t cap, const int64_t* kv_len, const int64_t* q_pos,
                      int64_t max_kv_len, double theta, float scale, int q_rotated,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!q || !k_cache || !v_cache || !o || !kv_len || !q_pos)
    return fail(GQA_ERR_INVALID_ARG, "q, k_cache, v_cache, o, kv_len and q_pos must be non-NULL");
  if (int rc = decode_ragged_check(q, k_cache, v_cache, o, in_dtype, out_dtype, B, h_q, h_kv, d,
                                   cap, max_kv_len, theta, scale, workspace, workspace_bytes))
    return rc;
  return decode_ragged_launch(q, k_cache, v_cache, o, in_dtype, out_dtype, B, h_q, h_kv, d, cap,
                              kv_len, q_pos, 0, q_rotated != 0, max_kv_len, theta, scale,
                              workspace, (hipStream_t)stream);
}

int gqa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, void* o, int in_dtype, int out_dtype, int64_t B, int h_q,
                      int h_kv, int d, int64_t cap, const int64_t* pos, int64_t max_pos,
                      double theta, float scale, void* workspace, size_t workspace_bytes,
                      void* stream) {
  g_err.clear();
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !o || !pos)
    return fail(GQA_ERR_INVALID_ARG,
                "q, k_new, v_new, k_cache, v_cache, o and pos must be non-NULL");
  if (max_pos < 0 || max_pos >= cap)
    return fail(GQA_ERR_INVALID_ARG, "max_pos=%lld outside [0, cap=%lld)", (long long)max_pos,
                (long long)cap);
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(GQA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  // everything the decode checks, before the cache is touched
  if (int rc = decode_ragged_check(q, k_cache, v_cache, o, in_dtype, out_dtype, B, h_q, h_kv, d,
                                   cap, max_pos + 1, theta, scale, workspace, workspace_bytes))
    return rc;
  // the new token's rotated K and its V go to cache row pos[b] (preparation
  // kernel), then it attends to rows 0 .. pos[b]
  return decode_ragged_launch(q, k_cache, v_cache, o, in_dtype, out_dtype, B, h_q, h_kv, d, cap,
                              nullptr, pos, 1, 0, max_pos + 1, theta, scale, workspace,
                              (hipStream_t)stream, nullptr, 0, 0, 0, k_new, v_new, max_pos + 1);
}

size_t gqa_decode_paged_workspace_size(int64_t B, int h_q, int h_kv, int d,
                                       int64_t max_kv_len) {
  return gqa_decode_workspace_size(B, h_q, h_kv, d, max_kv_len);
}

int gqa_decode_paged(const void* q, const void* k_new, const void* v_new, void* k_pool,
                     void* v_pool, void* o, int in_dtype, int out_dtype, int64_t B, int h_q,
                     int h_kv, int d, int page_size, int64_t num_pages,
                     const int32_t* block_table, int64_t max_pages, const int64_t* kv_len,
                     const int64_t* q_pos, int64_t max_kv_len, double theta, float scale,
                     int q_rotated, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!q || !k_pool || !v_pool || !o || !block_table || !q_pos)
    return fail(GQA_ERR_INVALID_ARG,
                "q, k_pool, v_pool, o, block_table and q_pos must be non-NULL");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(GQA_ERR_INVALID_ARG, "k_new and v_new must both be set or both be NULL");
  const bool append = k_new != nullptr;
  if (append == (kv_len != nullptr))
    return fail(GQA_ERR_INVALID_ARG,
                "give kv_len without k_new/v_new, or k_new/v_new (kv_len = q_pos + 1) alone");
  if (page_size < 1 || page_size > (1 << 20) || (page_size & (page_size - 1)))
    return fail(GQA_ERR_INVALID_ARG, "page_size=%d must be a power of two in [1, 2^20]",
                page_size);
  if (num_pages < 1 || num_pages > INT_MAX || max_pages < 1)
    return fail(GQA_ERR_INVALID_ARG, "num_pages and max_pages must be >= 1 (num_pages < 2^31)");
  if (max_kv_len > max_pages * page_size)
    return fail(GQA_ERR_INVALID_ARG, "max_kv_len=%lld exceeds max_pages * page_size = %lld",
                (long long)max_kv_len, (long long)(max_pages * page_size));
  if (append && !(aligned16(k_new) && aligned16(v_new)))
    return fail(GQA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  // the shared checks and the workspace layout see max_kv_len as the cache length
  if (int rc = decode_ragged_check(q, k_pool, v_pool, o, in_dtype, out_dtype, B, h_q, h_kv, d,
                                   max_kv_len, max_kv_len, theta, scale, workspace,
                                   workspace_bytes))
    return rc;
  int ps_log2 = 0;
  while ((1 << ps_log2) < page_size) ++ps_log2;
  // with append, the new token's rotated K and its V go to position q_pos[b]
  // first (preparation kernel)
  return decode_ragged_launch(q, k_pool, v_pool, o, in_dtype, out_dtype, B, h_q, h_kv, d,
                              max_kv_len, kv_len, q_pos, append ? 1 : 0, q_rotated != 0,
                              max_kv_len, theta, scale, workspace, (hipStream_t)stream,
                              block_table, ps_log2, max_pages, num_pages, k_new, v_new,
                              max_kv_len);
}

int gqa_qkv_epilogue(const void* qkv, const void* bias, void* q_out, void* k_cache,
                     void* v_cache, int dtype, int64_t B, int64_t C, int h_q, int h_kv, int d,
                     int64_t cap, const int64_t* start, const int64_t* len, int64_t kend,
                     double theta, void* stream) {
  g_err.clear();
  if (!qkv || !q_out || !k_cache || !v_cache || !start)
    return fail(GQA_ERR_INVALID_ARG, "qkv, q_out, k_cache, v_cache and start must be non-NULL");
  if (!dtype_ok(dtype)) return fail(GQA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (B < 1 || C < 1) return fail(GQA_ERR_INVALID_ARG, "B and C must be >= 1");
  if (int rc = check_heads(h_q, h_kv)) return rc;
  if (int rc = check_d(d)) return rc;
  if (int rc = check_theta_scale(theta, 1.0f)) return rc;
  if (kend < 1 || kend > cap)
    return fail(GQA_ERR_INVALID_ARG, "kend=%lld outside [1, cap=%lld]", (long long)kend,
                (long long)cap);
  if (kend > (INT64_C(1) << 40) || B * C > (INT64_C(1) << 32))
    return fail(GQA_ERR_UNSUPPORTED, "sizes exceed the kernel's index range");
  if (!aligned16(qkv) || !aligned16(bias) || !aligned16(q_out) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return fail(GQA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  hipError_t e = gqa::launch_qkv_epilogue(qkv, bias, q_out, k_cache, v_cache, dtype == GQA_BF16,
                                          start, len, B, C, h_q, h_kv, d, cap, kend,
                                          rope_params(theta, d), (hipStream_t)stream);
  return e == hipSuccess ? GQA_OK : hip_fail(e, "QKV epilogue launch");
}

int gqa_set_rope_yarn(double factor, double original_max_position, double beta_fast,
                      double beta_slow) {
  g_err.clear();
  if (!std::isfinite(factor) || factor < 1.0)
    return fail(GQA_ERR_INVALID_ARG, "factor=%g must be finite and >= 1", factor);
  if (factor > 1.0) {
    if (!(original_max_position >= 1.0) || !std::isfinite(original_max_position))
      return fail(GQA_ERR_INVALID_ARG, "original_max_position must be >= 1");
    if (!(beta_fast > beta_slow) || !(beta_slow > 0.0) || !std::isfinite(beta_fast))
      return fail(GQA_ERR_INVALID_ARG, "need beta_fast > beta_slow > 0");
  }
  g_yarn = YarnConfig{factor, original_max_position, beta_fast, beta_slow};
  return GQA_OK;
}

int gqa_timing_enable(int on) {
  if (on) g_timing.clear();
  g_timing.on = on != 0;
  return GQA_OK;
}

int gqa_timing_read(int which, double* total_ms, int64_t* count) {
  g_err.clear();
  if (which < 0 || which > 3 || !total_ms || !count)
    return fail(GQA_ERR_INVALID_ARG, "bad timing query");
  double tot = 0.0;
  int64_t n = 0;
  for (const auto& ev : g_timing.rec[which & 1]) {
    const hipEvent_t t0 = which < 2 ? ev.kernel_start : ev.call_start;
    const hipEvent_t t1 = which < 2 ? ev.kernel_stop : ev.call_stop;
    hipError_t e = hipEventSynchronize(t1);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, t0, t1);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *count = n;
  return GQA_OK;
}

int gqa_stream_read(const void* p, size_t bytes, void* sink, void* stream) {
  g_err.clear();
  if (!p || !sink || bytes == 0 || bytes % 16 != 0 || (uintptr_t)p % 16 != 0)
    return fail(GQA_ERR_INVALID_ARG, "stream_read: need a 16-byte aligned buffer and a size that is a positive multiple of 16");
  const hipError_t e = gqa::launch_stream_read(p, bytes, (unsigned*)sink, (hipStream_t)stream);
  return e == hipSuccess ? GQA_OK : hip_fail(e, "stream_read launch");
}

}  // extern "C"
