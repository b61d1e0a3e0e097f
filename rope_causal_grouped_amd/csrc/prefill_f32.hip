// Causal GQA prefill in fp32 throughout (vector ALU), RoPE fused into the Q
// load; used for fp32 inputs, where the result must match the definition to
// ~1e-4 and the shapes are small (Qwen2-0.5B: 14 query heads over 2 KV heads,
// head size 64).
//
// Same operation as the bf16 kernel (Qwen2 technical-report walkthrough,
// aicoding.csdn.net, §4.1.3 steps 3-4).  A workgroup owns 16 positions of
// one query head; four lanes share a row, each holding a quarter of its dims
// (dims j and j + d/2 of a RoPE pair stay in one lane).  The workgroup forms
// the pairs' frequencies once (fp64, in LDS) and each lane the cos/sin of
// its own pairs, so the call needs no table kernel.  K' and V tiles of 64
// keys are staged in LDS (K rotated while staging, or rotated already by the
// pass that wrote the cache); each of the
// four waves holds all 16 rows and takes a quarter of every tile's keys,
// updating its own online softmax four keys at a time, and the quarters are
// merged exactly at the end.  The small shapes this serves are latency-
// bound, so the split buys parallelism: four times the workgroups of a
// 64-row layout, and a quarter of the serial key chain per wave.  Keys and
// values are read through strides, so they may be the call's own K and V
// [B, L, h_kv, d], the preparation pass's rotated K [B][h_kv][L][d], or a
// per-layer cache [B, cap, h_kv, d] when a chunk of queries at positions
// qstart[b] + i attends to everything cached so far.

#include "common.h"
#include "launch.h"

namespace gqa {

namespace {

// value of the lane CTRL names within the quad (DPP quad permute)
template <int CTRL>
__device__ __forceinline__ float quad_swap(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

}  // namespace

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kp, const float* __restrict__ v,
    int rot_q, int rot_k, RopeParams rp, void* __restrict__ o, int L, int h_q, int h_kv, int g,
    float scale, int causal, KvStrides ks_, KvStrides vs_, const int64_t* __restrict__ qstart,
    const int64_t* __restrict__ qlen, int kend) {
  constexpr int TK = 64;                 // keys per staged tile
  constexpr int RB = 16;                 // rows (positions) per workgroup
  constexpr int KQ = TK / 4;             // keys of a tile per wave
  constexpr int E = D / 8;               // pair count per lane
  __shared__ __attribute__((aligned(16))) float ks[TK][D + 4];
  __shared__ __attribute__((aligned(16))) float vs[TK][D + 4];
  __shared__ double om[D / 2];           // pair frequencies
  if (rot_q || rot_k) {
    if (threadIdx.x < D / 2) om[threadIdx.x] = rope_omega(threadIdx.x, D, rp);
    __syncthreads();
  }

  const int pbk = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int u = t / g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // key quarter
  const int row = lane >> 2, part = lane & 3;

  // queries i < nq of sequence b at positions qs + i; keys 0 .. nk-1
  int qs = 0, nq = L;
  if (qstart) {
    const int64_t s0 = qstart[b], n = qlen ? qlen[b] : L;
    if (!(s0 >= 0 && n >= 0 && n <= L && s0 + n <= kend)) {   // out of range: NaN rows
      const int pr = pbk * RB + row;
      if (wave == 0 && pr < L) {
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
  if (pbk * RB >= nq) return;
  const int nk = causal ? qs + nq : L;
  const int pl_raw = pbk * RB + row;
  const bool valid = pl_raw < nq;
  const int pl = valid ? pl_raw : nq - 1;   // row of q / o
  const int pos = qs + pl;                  // its position

  // rotated query slice: qr[e] = dim part*E + e, qr[E + e] = dim D/2 + part*E + e
  float qr[2 * E];
  {
    const float* src = q + ((int64_t)((int64_t)b * L + pl) * h_q + t) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = part * E + e;
      const float x1 = src[j], x2 = src[j + D / 2];
      float c = 1.f, sn = 0.f;   // rot_q = 0: q is rotated already
      if (rot_q) {
        rope_cos_sin((double)pos, om[j], c, sn);
        c *= rp.mscale;
        sn *= rp.mscale;
      }
      qr[e] = fmaf(x1, c, -x2 * sn);
      qr[E + e] = fmaf(x2, c, x1 * sn);
    }
  }

  float acc[2 * E];
#pragma unroll
  for (int e = 0; e < 2 * E; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;   // running max in log2 units, sum
  const float sl2 = scale * 1.4426950408889634f;   // scale * log2(e)

  const int last_row_pos = qs + min(nq - 1, pbk * RB + RB - 1);
  const int n_keys = causal ? last_row_pos + 1 : L;
  const float* kbase = kp + (int64_t)b * ks_.batch + (int64_t)u * ks_.head;
  const float* vbase = v + (int64_t)b * vs_.batch + (int64_t)u * vs_.head;

  for (int k0 = 0; k0 < n_keys; k0 += TK) {
    // stage the tile: every 16-byte load issued before the first store.  A
    // thread takes four RoPE pairs (dims j4..j4+3 and j4+d/2..) of a key, so
    // with rot_k set it rotates K here, at the key's position (= its index)
    constexpr int CP = TK * (D / 8) / 256;   // four-pair chunks per thread
    float4 k1[CP], k2[CP], v1[CP], v2[CP];
#pragma unroll
    for (int r = 0; r < CP; ++r) {
      const int idx = threadIdx.x + r * 256;
      const int kk = idx / (D / 8), j4 = (idx % (D / 8)) * 4;
      const int key = k0 + kk;
      k1[r] = k2[r] = v1[r] = v2[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (key < nk) {
        const float* kr = kbase + (int64_t)key * ks_.row + j4;
        const float* vr = vbase + (int64_t)key * vs_.row + j4;
        k1[r] = *(const float4*)kr;
        k2[r] = *(const float4*)(kr + D / 2);
        v1[r] = *(const float4*)vr;
        v2[r] = *(const float4*)(vr + D / 2);
        if (rot_k) {
          float c[4], sn[4];   // (cos, sin) of pairs j4 .. j4+3
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            rope_cos_sin((double)key, om[j4 + e], c[e], sn[e]);
            c[e] *= rp.mscale;
            sn[e] *= rp.mscale;
          }
          float x1[4] = {k1[r].x, k1[r].y, k1[r].z, k1[r].w};
          float x2[4] = {k2[r].x, k2[r].y, k2[r].z, k2[r].w};
          float y1[4], y2[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y1[e] = fmaf(x1[e], c[e], -x2[e] * sn[e]);
            y2[e] = fmaf(x2[e], c[e], x1[e] * sn[e]);
          }
          k1[r] = make_float4(y1[0], y1[1], y1[2], y1[3]);
          k2[r] = make_float4(y2[0], y2[1], y2[2], y2[3]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < CP; ++r) {
      const int idx = threadIdx.x + r * 256;
      const int kk = idx / (D / 8), j4 = (idx % (D / 8)) * 4;
      *(float4*)&ks[kk][j4] = k1[r];
      *(float4*)&ks[kk][j4 + D / 2] = k2[r];
      *(float4*)&vs[kk][j4] = v1[r];
      *(float4*)&vs[kk][j4 + D / 2] = v2[r];
    }
    __syncthreads();
    // this wave's quarter of the tile, four keys per step: their dot
    // products are independent, the quad sums use DPP lane swaps (no LDS
    // round trip), scores are in log2 units with the hardware exp2 (~1
    // ulp), and O is rescaled once per step
    const int ntile = min(TK, n_keys - k0);
    for (int jj = wave * KQ; jj < min(wave * KQ + KQ, ntile); jj += 4) {
      float sv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          d0 = fmaf(qr[e], ks[jj + k][part * E + e], d0);
          d1 = fmaf(qr[E + e], ks[jj + k][D / 2 + part * E + e], d1);
        }
        float dot = d0 + d1;
        dot += quad_swap<0xB1>(dot);   // lanes 0<->1, 2<->3
        dot += quad_swap<0x4E>(dot);   // lanes 0<->2, 1<->3
        const int key = k0 + jj + k;
        sv[k] = (jj + k < ntile && (!causal || key <= pos)) ? dot * sl2 : -INFINITY;
      }
      const float m_new = fmaxf(fmaxf(m, fmaxf(sv[0], sv[1])), fmaxf(sv[2], sv[3]));
      const float mref = m_new == -INFINITY ? 0.f : m_new;   // no visible key yet
      const float alpha = __builtin_amdgcn_exp2f(m - mref);
      float p[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) p[k] = __builtin_amdgcn_exp2f(sv[k] - mref);
      l = fmaf(l, alpha, (p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j1 = part * E + e, j2 = D / 2 + part * E + e;
        float a1 = acc[e] * alpha, a2 = acc[E + e] * alpha;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          a1 = fmaf(p[k], vs[jj + k][j1], a1);
          a2 = fmaf(p[k], vs[jj + k][j2], a2);
        }
        acc[e] = a1;
        acc[E + e] = a2;
      }
      m = m_new;
    }
  }

  // merge the four key quarters (exact log-sum-exp combination): partial
  // sums through LDS (the tile arrays, free once every wave is done), then
  // wave 0 scales each quarter by 2^(m_w - M) and normalises
  __syncthreads();
  float* mb = &ks[0][0];   // [wave][element][lane]
  float* ml = &vs[0][0];   // [wave][m | l][lane]
  static_assert(4 * 2 * E * 64 <= TK * (D + 4), "merge buffer exceeds the tile array");
#pragma unroll
  for (int e = 0; e < 2 * E; ++e) mb[(wave * 2 * E + e) * 64 + lane] = acc[e];
  ml[wave * 128 + lane] = m;
  ml[wave * 128 + 64 + lane] = l;
  __syncthreads();
  if (wave != 0 || !valid) return;
  float mw[4], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = ml[w * 128 + lane];
    M = fmaxf(M, mw[w]);
  }
  // every row sees at least one key (its own position when causal), so M is finite
  float sc[4], lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    sc[w] = __builtin_amdgcn_exp2f(mw[w] - M);   // 0 for a quarter that saw no key
    lsum = fmaf(ml[w * 128 + 64 + lane], sc[w], lsum);
  }
  const float inv = 1.0f / lsum;
  const int64_t orow = ((int64_t)((int64_t)b * L + pl) * h_q + t) * D;
#pragma unroll
  for (int e = 0; e < 2 * E; ++e) {
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) y = fmaf(mb[(w * 2 * E + e) * 64 + lane], sc[w], y);
    y *= inv;
    const int j = e < E ? part * E + e : D / 2 + part * E + (e - E);
    if constexpr (OUT_BF16) ((uint16_t*)o)[orow + j] = f32_to_bf16_bits(y);
    else ((float*)o)[orow + j] = y;
  }
}

hipError_t launch_prefill_f32(const float* q, const float* kp, const float* v, int rot_q,
                              int rot_k, RopeParams rp, void* o, int out_bf16, int64_t B, int64_t L,
                              int h_q, int h_kv, int d, float scale, int causal, KvStrides ks,
                              KvStrides vs, const int64_t* qstart, const int64_t* qlen,
                              int64_t kend, hipStream_t st) {
  const int g = h_q / h_kv;
  dim3 grid((unsigned)((L + 15) / 16), (unsigned)h_q, (unsigned)B);
  hipError_t e;
#define GQA_LAUNCH(DD, OB)                                                                  \
  e = launch_kernel(prefill_f32_kernel<DD, OB>, grid, dim3(256), st, q, kp, v, rot_q, rot_k, rp, o, \
                    (int)L, h_q, h_kv, g, scale, causal, ks, vs, qstart, qlen, (int)kend)
  if (d == 128) {
    if (out_bf16) GQA_LAUNCH(128, true); else GQA_LAUNCH(128, false);
  } else {
    if (out_bf16) GQA_LAUNCH(64, true); else GQA_LAUNCH(64, false);
  }
#undef GQA_LAUNCH
  return e;
}

}  // namespace gqa
