// Causal GQA prefill in fp32 throughout (vector ALU), RoPE fused into the Q
// load; used for fp32 inputs, where the result must match the definition to
// ~1e-4 and the shapes are small (Qwen2-0.5B: 14 query heads over 2 KV heads,
// head size 64).
//
// Same operation as the bf16 kernel (Qwen2 technical-report walkthrough,
// aicoding.csdn.net, §4.1.3 steps 3-4).  A workgroup owns 64 positions of
// one query head; four lanes share a row, each holding a quarter of its dims
// (dims j and j + d/2 of a RoPE pair stay in one lane).  K' (rotated by the
// preparation pass) and V tiles of 64 keys are staged in LDS and shared by
// the 64 rows; the softmax is updated key by key.  Keys and values are read
// through strides, so they may come from the preparation pass (rotated K,
// [B][h_kv][L][d]) and the call's V, or straight from a per-layer cache
// [B, cap, h_kv, d] when a chunk of queries at positions qstart[b] + i
// attends to everything cached so far.

#include "common.h"
#include "launch.h"

namespace gqa {

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kp, const float* __restrict__ v,
    const float2* __restrict__ cs, void* __restrict__ o, int L, int h_q, int h_kv, int g,
    float scale, int causal, KvStrides ks_, KvStrides vs_, const int64_t* __restrict__ qstart,
    const int64_t* __restrict__ qlen, int kend) {
  constexpr int TK = 64;
  constexpr int E = D / 8;  // pair count per lane
  __shared__ float ks[TK][D + 4];
  __shared__ float vs[TK][D + 4];

  const int pbk = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int u = t / g;
  const int row = threadIdx.x >> 2, part = threadIdx.x & 3;

  // queries i < nq of sequence b at positions qs + i; keys 0 .. nk-1
  int qs = 0, nq = L;
  if (qstart) {
    const int64_t s0 = qstart[b], n = qlen ? qlen[b] : L;
    if (!(s0 >= 0 && n >= 0 && n <= L && s0 + n <= kend)) {   // out of range: NaN rows
      const int pr = pbk * TK + row;
      if (pr < L) {
        const int64_t orow = ((int64_t)((int64_t)b * L + pr) * h_q + t) * D;
        for (int e = part; e < D; e += 4) {
          if constexpr (OUT_BF16) ((uint16_t*)o)[orow + e] = 0x7fc0u;
          else ((float*)o)[orow + e] = __builtin_nanf("");
        }
      }
      return;
    }
    qs = (int)s0;
    nq = (int)n;
  }
  if (pbk * TK >= nq) return;
  const int nk = causal ? qs + nq : L;
  const int pl_raw = pbk * TK + row;
  const bool valid = pl_raw < nq;
  const int pl = valid ? pl_raw : nq - 1;   // row of q / o
  const int pos = qs + pl;                  // its position

  // rotated query slice: qr[e] = dim part*E + e, qr[E + e] = dim D/2 + part*E + e
  float qr[2 * E];
  {
    const float* src = q + ((int64_t)((int64_t)b * L + pl) * h_q + t) * D;
    const float2* csr = cs + (int64_t)pos * (D / 2);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = part * E + e;
      const float x1 = src[j], x2 = src[j + D / 2];
      const float2 r2 = cs ? csr[j] : make_float2(1.f, 0.f);   // cs NULL: q is rotated
      qr[e] = fmaf(x1, r2.x, -x2 * r2.y);
      qr[E + e] = fmaf(x2, r2.x, x1 * r2.y);
    }
  }

  float acc[2 * E];
#pragma unroll
  for (int e = 0; e < 2 * E; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int last_row_pos = qs + min(nq - 1, pbk * TK + TK - 1);
  const int n_keys = causal ? last_row_pos + 1 : L;
  const float* kbase = kp + (int64_t)b * ks_.batch + (int64_t)u * ks_.head;
  const float* vbase = v + (int64_t)b * vs_.batch + (int64_t)u * vs_.head;

  for (int k0 = 0; k0 < n_keys; k0 += TK) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < TK * D; idx += 256) {
      const int kk = idx / D, dd = idx % D;
      const int key = k0 + kk;
      float kv = 0.f, vv = 0.f;
      if (key < nk) {
        kv = kbase[(int64_t)key * ks_.row + dd];
        vv = vbase[(int64_t)key * vs_.row + dd];
      }
      ks[kk][dd] = kv;
      vs[kk][dd] = vv;
    }
    __syncthreads();
    const int ntile = min(TK, n_keys - k0);
    for (int jj = 0; jj < ntile; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        dot = fmaf(qr[e], ks[jj][part * E + e], dot);
        dot = fmaf(qr[E + e], ks[jj][D / 2 + part * E + e], dot);
      }
      dot += __shfl_xor(dot, 1, 64);
      dot += __shfl_xor(dot, 2, 64);
      const int key = k0 + jj;
      if (!causal || key <= pos) {
        const float s = dot * scale;
        const float m_new = fmaxf(m, s);
        const float alpha = expf(m - m_new);
        const float p = expf(s - m_new);
        l = fmaf(l, alpha, p);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          acc[e] = fmaf(acc[e], alpha, p * vs[jj][part * E + e]);
          acc[E + e] = fmaf(acc[E + e], alpha, p * vs[jj][D / 2 + part * E + e]);
        }
        m = m_new;
      }
    }
  }

  if (valid) {
    const float inv = 1.0f / l;
    const int64_t orow = ((int64_t)((int64_t)b * L + pl) * h_q + t) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = part * E + e;
      if constexpr (OUT_BF16) {
        ((uint16_t*)o)[orow + j] = f32_to_bf16_bits(acc[e] * inv);
        ((uint16_t*)o)[orow + j + D / 2] = f32_to_bf16_bits(acc[E + e] * inv);
      } else {
        ((float*)o)[orow + j] = acc[e] * inv;
        ((float*)o)[orow + j + D / 2] = acc[E + e] * inv;
      }
    }
  }
}

hipError_t launch_prefill_f32(const float* q, const float* kp, const float* v, const float2* cs,
                              void* o, int out_bf16, int64_t B, int64_t L, int h_q, int h_kv,
                              int d, float scale, int causal, KvStrides ks, KvStrides vs,
                              const int64_t* qstart, const int64_t* qlen, int64_t kend,
                              hipStream_t st) {
  const int g = h_q / h_kv;
  dim3 grid((unsigned)((L + 63) / 64), (unsigned)h_q, (unsigned)B);
#define GQA_LAUNCH(DD, OB)                                                                   \
  prefill_f32_kernel<DD, OB><<<grid, 256, 0, st>>>(q, kp, v, cs, o, (int)L, h_q, h_kv, g, scale, \
                                                   causal, ks, vs, qstart, qlen, (int)kend)
  if (d == 128) {
    if (out_bf16) GQA_LAUNCH(128, true); else GQA_LAUNCH(128, false);
  } else {
    if (out_bf16) GQA_LAUNCH(64, true); else GQA_LAUNCH(64, false);
  }
#undef GQA_LAUNCH
  return hipGetLastError();
}

}  // namespace gqa
