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
// the 64 rows; the softmax is updated key by key.

#include "common.h"
#include "launch.h"

namespace gqa {

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kp, const float* __restrict__ v,
    const float2* __restrict__ cs, void* __restrict__ o, int L, int h_q, int h_kv, int g,
    float scale, int causal) {
  constexpr int TK = 64;
  constexpr int E = D / 8;  // pair count per lane
  __shared__ float ks[TK][D + 4];
  __shared__ float vs[TK][D + 4];

  const int pbk = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int u = t / g;
  const int row = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int pos_raw = pbk * TK + row;
  const bool valid = pos_raw < L;
  const int pos = valid ? pos_raw : L - 1;

  // rotated query slice: qr[e] = dim part*E + e, qr[E + e] = dim D/2 + part*E + e
  float qr[2 * E];
  {
    const float* src = q + ((int64_t)((int64_t)b * L + pos) * h_q + t) * D;
    const float2* csr = cs + (int64_t)pos * (D / 2);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = part * E + e;
      const float x1 = src[j], x2 = src[j + D / 2];
      const float2 r2 = csr[j];
      qr[e] = fmaf(x1, r2.x, -x2 * r2.y);
      qr[E + e] = fmaf(x2, r2.x, x1 * r2.y);
    }
  }

  float acc[2 * E];
#pragma unroll
  for (int e = 0; e < 2 * E; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int last_row_pos = min(L - 1, pbk * TK + TK - 1);
  const int n_keys = causal ? last_row_pos + 1 : L;
  const float* kbase = kp + ((int64_t)b * h_kv + u) * (int64_t)L * D;

  for (int k0 = 0; k0 < n_keys; k0 += TK) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < TK * D; idx += 256) {
      const int kk = idx / D, dd = idx % D;
      const int key = k0 + kk;
      float kv = 0.f, vv = 0.f;
      if (key < L) {
        kv = kbase[(int64_t)key * D + dd];
        vv = v[(((int64_t)b * L + key) * h_kv + u) * D + dd];
      }
      ks[kk][dd] = kv;
      vs[kk][dd] = vv;
    }
    __syncthreads();
    const int nk = min(TK, n_keys - k0);
    for (int jj = 0; jj < nk; ++jj) {
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
    const int64_t orow = ((int64_t)((int64_t)b * L + pos) * h_q + t) * D;
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
                              int d, float scale, int causal, hipStream_t st) {
  const int g = h_q / h_kv;
  dim3 grid((unsigned)((L + 63) / 64), (unsigned)h_q, (unsigned)B);
#define GQA_LAUNCH(DD, OB)                                                                   \
  prefill_f32_kernel<DD, OB><<<grid, 256, 0, st>>>(q, kp, v, cs, o, (int)L, h_q, h_kv, g, scale, \
                                                   causal)
  if (d == 128) {
    if (out_bf16) GQA_LAUNCH(128, true); else GQA_LAUNCH(128, false);
  } else {
    if (out_bf16) GQA_LAUNCH(64, true); else GQA_LAUNCH(64, false);
  }
#undef GQA_LAUNCH
  return hipGetLastError();
}

}  // namespace gqa
