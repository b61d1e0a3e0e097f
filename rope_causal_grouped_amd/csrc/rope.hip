// RoPE kernels: in-place rotation, the per-call cos/sin table, and the
// K/V preparation pass that runs ahead of prefill attention.
//
// RoPE (Qwen2 technical-report walkthrough, aicoding.csdn.net, §3.5.2 and
// §4.1.3 step 3): every row of Q and K is rotated at its position, pair by
// pair, inside the head's d dims.  Pair j couples dims j and j + d/2 and
// turns by pos * theta^(-2j/d); theta = 1e6 for Qwen2 (same page §5.2).

#include "common.h"
#include "launch.h"

namespace gqa {

// ---------------------------------------------------------------------------
// In-place rotation of x[B, L, h, d]; one thread per (row, pair).
template <typename T>
__global__ __launch_bounds__(256) void rope_apply_kernel(T* __restrict__ x, int64_t n_pairs, int64_t L,
                                                         int h, int d, int64_t pos0,
                                                         RopeParams rp) {
  const int half = d >> 1;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n_pairs;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / half;
    const int j = (int)(idx - row * half);
    const int64_t l = (row / h) % L;
    float c, s;
    rope_cs((double)(pos0 + l), j, d, rp, c, s);
    T* p = x + row * d;
    float x1, x2;
    if constexpr (sizeof(T) == 2) {
      x1 = bf16_bits_to_f32(p[j]);
      x2 = bf16_bits_to_f32(p[j + half]);
    } else {
      x1 = p[j];
      x2 = p[j + half];
    }
    const float y1 = fmaf(x1, c, -x2 * s);
    const float y2 = fmaf(x2, c, x1 * s);
    if constexpr (sizeof(T) == 2) {
      p[j] = f32_to_bf16_bits(y1);
      p[j + half] = f32_to_bf16_bits(y2);
    } else {
      p[j] = y1;
      p[j + half] = y2;
    }
  }
}

hipError_t launch_rope_apply(void* x, int dtype, int64_t B, int64_t L, int h, int d, int64_t pos0,
                             RopeParams rp, hipStream_t st) {
  const int64_t n_pairs = B * L * h * (d / 2);
  const int64_t want = (n_pairs + 255) / 256;
  const int grid = (int)(want < 65536 ? want : 65536);
  if (dtype == 1)
    rope_apply_kernel<uint16_t><<<grid, 256, 0, st>>>((uint16_t*)x, n_pairs, L, h, d, pos0,
                                                      rp);
  else
    rope_apply_kernel<float><<<grid, 256, 0, st>>>((float*)x, n_pairs, L, h, d, pos0, rp);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// cs[l][j] = (cos, sin)(pos(l) * omega_j) for l < L, j < d/2, pos(l) = pos0 + l.
// A thread keeps one pair j (d/2 divides the block) and fills kTablePosPerThread
// positions with it, so the fp64 omega_j is formed once per thread.
constexpr int kTablePosPerThread = 4;

__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ cs, int64_t L, int d,
                                                         int64_t pos0, RopeParams rp) {
  const int half = d >> 1;
  const int rows = 256 / half;                       // positions per block and step
  const int j = threadIdx.x % half;
  const double omega = rope_omega(j, d, rp);
  const int64_t l0 = (int64_t)blockIdx.x * rows * kTablePosPerThread + threadIdx.x / half;
#pragma unroll
  for (int i = 0; i < kTablePosPerThread; ++i) {
    const int64_t l = l0 + (int64_t)i * rows;
    if (l >= L) break;
    float c, s;
    rope_cos_sin((double)(pos0 + l), omega, c, s);
    cs[l * half + j] = make_float2(c * rp.mscale, s * rp.mscale);
  }
}

hipError_t launch_rope_table(float2* cs, int64_t L, int d, int64_t pos0, RopeParams rp,
                             hipStream_t st) {
  if (d < 2 || 256 % (d / 2) != 0) return hipErrorInvalidValue;
  const int64_t per_block = (int64_t)(256 / (d / 2)) * kTablePosPerThread;
  const int64_t grid = (L + per_block - 1) / per_block;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  return launch_kernel(rope_table_kernel, dim3((unsigned)grid), dim3(256), st, cs, L, d, pos0, rp);
}

// ---------------------------------------------------------------------------
// K/V preparation for the bf16 prefill.  One workgroup per (64-key tile,
// KV group u, batch b):
//   kp[b][u][key][:]   rotated K as fp16 (the score operand: its 11-bit
//                      significand keeps the logits of large rows within
//                      the bf16 tolerance, where bf16 K' would not), times
//                      2^-kexp of the tile; keys contiguous per group (a
//                      64-key tile is one contiguous 16 KB block, d = 128);
//   kexp[b][u][tile]   0, or the power of two the tile was divided by when
//                      its largest element reached 2^14 (fp16 stays finite);
//   kmax[b][u][tile]   the largest row norm of the tile's stored K' (times
//                      2^kexp): an upper bound on its scores for a given
//                      query norm;
//   vt[b][u][t32][dim][32] V transposed per 32-key attention tile, so the
//                      attention kernel's P.V operand reads consecutive keys
//                      of one dim; inside each 16-key group the keys are
//                      stored in the order 0-3, 8-11, 4-7, 12-15, which is
//                      the order in which one lane of the 32x32 score
//                      accumulator holds them.
// Rows past L are zero.  If kc/vc are set, the rotated K (bf16, rounded once
// from the fp32 rotation) and the V rows are also written to the per-layer
// cache [B, cap, h_kv, d].  The source rows of sequence b start at
// k + b * src_rows * h_kv * d (src_rows = L for the call's own K/V, cap for a
// cache).  With kstart set, sequence b has kstart[b] + klen[b] rows (0 if
// that is not within [0, kend]).  With rotate set, key j is turned at
// position j: the kernel forms each (cos, sin) itself, as the table kernel
// does, and the workgroups of sequence 0, group 0 also store them to
// cs_out[j][pair] (if set) for the attention kernel's queries, so no table
// launch precedes this one; with rotate 0 the source K is taken as already
// rotated (a cache).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void kv_prepare_bf16_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int rotate, RopeParams rp,
    float2* __restrict__ cs_out, uint16_t* __restrict__ kp, uint16_t* __restrict__ vt,
    float* __restrict__ kmax, int* __restrict__ kexp, uint16_t* __restrict__ kc,
    uint16_t* __restrict__ vc, int64_t L, int64_t Lpad, int h_kv, int64_t cap, int64_t src_rows,
    const int64_t* __restrict__ kstart, const int64_t* __restrict__ klen, int64_t kend,
    int* __restrict__ pool_ctr) {
  constexpr int TK = 64;
  constexpr int HALF = D / 2;
  constexpr int PP = HALF / 4;        // RoPE pairs per thread: 4 threads per key row
  constexpr int TV = kPrefillTileV;
  __shared__ __attribute__((aligned(16))) uint16_t vs[TK][D + 8];
  __shared__ float wred[4];
  __shared__ double om[HALF];
  const int tile = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t key0 = (int64_t)tile * TK;
  // the pairs' frequencies, before any load is in flight (so the barrier
  // waits for nothing but them)
  if (rotate) {
    if (tid < HALF) om[tid] = rope_omega(tid, D, rp);
    __syncthreads();
  }
  // the attention kernel's ticket counters for its shared tail start at 0
  if (pool_ctr && tile == 0 && u == 0 && b == 0 && tid < kPrefillPoolXcds)
    __hip_atomic_store(pool_ctr + tid * kPrefillPoolStride, 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (kstart) {   // keys of sequence b: rows 0 .. kstart[b] + klen[b] - 1 of the source
    const int64_t s0 = kstart[b], n = klen ? klen[b] : L;
    L = (s0 >= 0 && n >= 0 && n <= L && s0 + n <= kend) ? s0 + n : 0;
  }
  const int kk = tid >> 2, part = tid & 3;
  const int64_t key = key0 + kk;
  // ---- V rows of the tile, 16 bytes per thread and step: issued first, so
  // that their latency overlaps the K loads and the rotation
  constexpr int VSTEPS = TK * D / 8 / 256;
  u32x4 vval[VSTEPS];
#pragma unroll
  for (int i = 0; i < VSTEPS; ++i) {
    const int c = tid + 256 * i;
    const int64_t vkey = key0 + c / (D / 8);
    vval[i] = u32x4{0u, 0u, 0u, 0u};
    if (vkey < L) vval[i] = *(const u32x4*)(v + (((int64_t)b * src_rows + vkey) * h_kv + u) * D +
                                            (c % (D / 8)) * 8);
  }
  // ---- this thread's quarter of a K row, rotated (or as given), in fp32
  float y1[PP], y2[PP];
  float amax = 0.f;
  if (key < L) {
    const uint16_t* src = k + (((int64_t)b * src_rows + key) * h_kv + u) * D + part * PP;
    uint16_t x1[PP], x2[PP];
#pragma unroll
    for (int c = 0; c < PP / 8; ++c) {
      *(u32x4*)&x1[c * 8] = *(const u32x4*)(src + c * 8);
      *(u32x4*)&x2[c * 8] = *(const u32x4*)(src + HALF + c * 8);
    }
    if (rotate) {   // rotate here; otherwise the source rows are rotated already
      // (cos, sin) of this thread's pairs at position key, formed while the
      // loads are in flight
      float2 r[PP];
#pragma unroll
      for (int e = 0; e < PP; ++e) {
        float c, sn;
        rope_cos_sin((double)key, om[part * PP + e], c, sn);
        r[e] = make_float2(c * rp.mscale, sn * rp.mscale);
      }
      if (cs_out && u == 0 && b == 0) {
        float2* dst = cs_out + key * HALF + part * PP;
#pragma unroll
        for (int e = 0; e < PP; e += 2) *(f32x4*)(dst + e) = f32x4{r[e].x, r[e].y, r[e + 1].x, r[e + 1].y};
      }
#pragma unroll
      for (int e = 0; e < PP; ++e) {
        const float a = bf16_bits_to_f32(x1[e]), bb = bf16_bits_to_f32(x2[e]);
        y1[e] = fmaf(a, r[e].x, -bb * r[e].y);
        y2[e] = fmaf(bb, r[e].x, a * r[e].y);
      }
    } else {
#pragma unroll
      for (int e = 0; e < PP; ++e) {
        y1[e] = bf16_bits_to_f32(x1[e]);
        y2[e] = bf16_bits_to_f32(x2[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < PP; ++e) amax = fmaxf(amax, fmaxf(fabsf(y1[e]), fabsf(y2[e])));
    if (kc) {   // the cache keeps bf16, rounded once from the fp32 rotation
      uint16_t o1[PP], o2[PP];
#pragma unroll
      for (int e = 0; e < PP; ++e) {
        o1[e] = f32_to_bf16_bits(y1[e]);
        o2[e] = f32_to_bf16_bits(y2[e]);
      }
      uint16_t* cdst = kc + (((int64_t)b * cap + key) * h_kv + u) * D + part * PP;
#pragma unroll
      for (int c = 0; c < PP / 8; ++c) {
        *(u32x4*)(cdst + c * 8) = *(const u32x4*)&o1[c * 8];
        *(u32x4*)(cdst + HALF + c * 8) = *(const u32x4*)&o2[c * 8];
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < PP; ++e) y1[e] = y2[e] = 0.f;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if ((tid & 63) == 0) wred[tid >> 6] = amax;

  // ---- V rows into LDS (and the cache copy)
#pragma unroll
  for (int i = 0; i < VSTEPS; ++i) {
    const int c = tid + 256 * i;
    const int vk = c / (D / 8), c8 = c % (D / 8);
    const int64_t vkey = key0 + vk;
    if (vc && vkey < L)
      *(u32x4*)(vc + (((int64_t)b * cap + vkey) * h_kv + u) * D + c8 * 8) = vval[i];
    *(u32x4*)&vs[vk][c8 * 8] = vval[i];
  }
  __syncthreads();

  // ---- the tile's exponent, K' as fp16, and the tile's largest row norm
  const int ex = kexp_of(fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3])));
  const float down = __builtin_ldexpf(1.0f, -ex);
  uint16_t h1[PP], h2[PP];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < PP; ++e) {
    const _Float16 a = (_Float16)(y1[e] * down), bb = (_Float16)(y2[e] * down);
    h1[e] = __builtin_bit_cast(uint16_t, a);
    h2[e] = __builtin_bit_cast(uint16_t, bb);
    ss = fmaf((float)a, (float)a, fmaf((float)bb, (float)bb, ss));
  }
  uint16_t* kdst = kp + (((int64_t)b * h_kv + u) * Lpad + key) * D + part * PP;
#pragma unroll
  for (int c = 0; c < PP / 8; ++c) {
    *(u32x4*)(kdst + c * 8) = *(const u32x4*)&h1[c * 8];
    *(u32x4*)(kdst + HALF + c * 8) = *(const u32x4*)&h2[c * 8];
  }
  // squared row norm (4 threads per row), then the max over the tile's rows
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
#pragma unroll
  for (int m = 4; m < 64; m <<= 1) ss = fmaxf(ss, __shfl_xor(ss, m, 64));
  __syncthreads();   // every thread has read wred
  if ((tid & 63) == 0) wred[tid >> 6] = ss;

  // ---- V^T in tiles of TV keys: vt[b][u][key / TV][dim][TV]; each thread
  // writes 8 consecutive (permuted) keys of one dim
  uint16_t* vdst = vt + (((int64_t)b * h_kv + u) * Lpad + key0) * D;
  for (int c = tid; c < TK * D / 8; c += 256) {
    const int sub = c / (D * TV / 8), rem = c % (D * TV / 8);
    const int dd = rem / (TV / 8), p0 = (rem % (TV / 8)) * 8;
    uint16_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = p0 + e, pp = p & 15;
      const int vk = sub * TV + (p & ~15) + ((pp & 7) >> 2) * 8 + (pp >> 3) * 4 + (pp & 3);
      w[e] = vs[vk][dd];
    }
    *(u32x4*)(vdst + (int64_t)c * 8) = *(const u32x4*)w;
  }
  __syncthreads();
  if (tid == 0) {
    const int64_t t = ((int64_t)b * h_kv + u) * (Lpad / TK) + tile;
    kmax[t] = __builtin_ldexpf(sqrtf(fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]))),
                               ex);
    kexp[t] = ex;
  }
}

// K preparation for the fp32 prefill: kp[b][u][key][:] = rotated K (fp32),
// optional cache copies of rotated K and V.  The pairs' frequencies are
// formed once per workgroup (fp64, in LDS).
template <int D>
__global__ __launch_bounds__(256) void kv_prepare_f32_kernel(
    const float* __restrict__ k, const float* __restrict__ v, RopeParams rp,
    float* __restrict__ kp, float* __restrict__ kc, float* __restrict__ vc, int64_t L, int h_kv,
    int64_t cap) {
  constexpr int TK = 64;
  constexpr int HALF = D / 2;
  __shared__ double om[HALF];
  if (threadIdx.x < HALF) om[threadIdx.x] = rope_omega(threadIdx.x, D, rp);
  __syncthreads();
  const int tile = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
  const int64_t key0 = (int64_t)tile * TK;
  for (int idx = threadIdx.x; idx < TK * HALF; idx += 256) {
    const int kk = idx / HALF, j = idx % HALF;
    const int64_t key = key0 + kk;
    if (key >= L) continue;
    const float* src = k + (((int64_t)b * L + key) * h_kv + u) * D;
    const float x1 = src[j], x2 = src[j + HALF];
    float c, sn;
    rope_cos_sin((double)key, om[j], c, sn);
    c *= rp.mscale;
    sn *= rp.mscale;
    const float o1 = fmaf(x1, c, -x2 * sn);
    const float o2 = fmaf(x2, c, x1 * sn);
    float* kdst = kp + (((int64_t)b * h_kv + u) * L + key) * D;
    kdst[j] = o1;
    kdst[j + HALF] = o2;
    if (kc) {
      float* cdst = kc + (((int64_t)b * cap + key) * h_kv + u) * D;
      cdst[j] = o1;
      cdst[j + HALF] = o2;
    }
  }
  if (vc) {
    for (int idx = threadIdx.x; idx < TK * D; idx += 256) {
      const int kk = idx / D, dd = idx % D;
      const int64_t key = key0 + kk;
      if (key >= L) continue;
      vc[(((int64_t)b * cap + key) * h_kv + u) * D + dd] =
          v[(((int64_t)b * L + key) * h_kv + u) * D + dd];
    }
  }
}

hipError_t launch_kv_prepare_bf16(const uint16_t* k, const uint16_t* v, const RopeParams* rope,
                                  float2* cs_out, uint16_t* kp, uint16_t* vt, float* kmax,
                                  int* kexp, uint16_t* kc, uint16_t* vc, int64_t B, int64_t L,
                                  int64_t Lpad, int h_kv, int d, int64_t cap, int64_t src_rows,
                                  const int64_t* kstart, const int64_t* klen, int64_t kend,
                                  int* pool_ctr, hipStream_t st) {
  if (cs_out && !rope) return hipErrorInvalidValue;
  const int rotate = rope != nullptr;
  const RopeParams rp = rope ? *rope : RopeParams{};
  dim3 grid((unsigned)(Lpad / 64), (unsigned)h_kv, (unsigned)B);
  if (d == 128)
    return launch_kernel(kv_prepare_bf16_kernel<128>, grid, dim3(256), st, k, v, rotate, rp,
                         cs_out, kp, vt, kmax, kexp, kc, vc, L, Lpad, h_kv, cap, src_rows, kstart,
                         klen, kend, pool_ctr);
  return launch_kernel(kv_prepare_bf16_kernel<64>, grid, dim3(256), st, k, v, rotate, rp, cs_out,
                       kp, vt, kmax, kexp, kc, vc, L, Lpad, h_kv, cap, src_rows, kstart, klen,
                       kend, pool_ctr);
}

// ---------------------------------------------------------------------------
// Cache append (the per-layer cache keeps the h_kv groups' rotated K and V,
// appended every step: walkthrough §4.1.3 closing note).  New rows
// k/v[B, C, h_kv, d]; row i < len[b] (len NULL: C) of sequence b sits at
// position p = start[b] + i: kc[b][p][u] = RoPE(k[b][i][u], p) and
// vc[b][p][u] = v[b][i][u].  A sequence whose rows would not lie within
// [0, end) (end <= cap, checked by the caller) is skipped.  With a block
// table bt [B][max_pages] the cache is a pair of page pools
// [num_pages, h_kv, 2^ps_log2, d] and position p goes to page
// bt[b][p >> ps_log2], row p & (page_size - 1); a row whose page id is out
// of range is skipped.  One thread per (row, head, pair j): it rotates dims
// j, j + d/2 and copies them of V.
template <typename T>
__global__ __launch_bounds__(256) void cache_append_kernel(
    const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ kc, T* __restrict__ vc,
    const int64_t* __restrict__ start, const int64_t* __restrict__ len, int64_t n_pairs,
    int64_t C, int h_kv, int d, int64_t cap, int64_t end, RopeParams rp,
    const int32_t* __restrict__ bt, int ps_log2, int64_t max_pages, int64_t num_pages) {
  const int half = d >> 1;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n_pairs;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / half;            // (b, i, u)
    const int j = (int)(idx - row * half);
    const int u = (int)(row % h_kv);
    const int64_t bi = row / h_kv;
    const int64_t i = bi % C, b = bi / C;
    const int64_t s0 = start[b], n = len ? len[b] : C;
    if (!(s0 >= 0 && n >= 0 && n <= C && s0 + n <= end) || i >= n) continue;
    const int64_t p = s0 + i;
    int64_t dst = ((b * cap + p) * h_kv + u) * d;
    if (bt) {
      const int64_t slot = p >> ps_log2;
      const int pid = slot < max_pages ? bt[b * max_pages + slot] : -1;
      if (pid < 0 || pid >= num_pages) continue;
      dst = (((int64_t)pid * h_kv + u) * ((int64_t)1 << ps_log2) + (p & ((1 << ps_log2) - 1))) * d;
    }
    float c, s;
    rope_cs((double)p, j, d, rp, c, s);
    const T* kr = k + row * d;
    const T* vr = v + row * d;
    T* kd = kc + dst;
    T* vd = vc + dst;
    if constexpr (sizeof(T) == 2) {
      const float x1 = bf16_bits_to_f32(kr[j]), x2 = bf16_bits_to_f32(kr[j + half]);
      kd[j] = f32_to_bf16_bits(fmaf(x1, c, -x2 * s));
      kd[j + half] = f32_to_bf16_bits(fmaf(x2, c, x1 * s));
    } else {
      const float x1 = kr[j], x2 = kr[j + half];
      kd[j] = fmaf(x1, c, -x2 * s);
      kd[j + half] = fmaf(x2, c, x1 * s);
    }
    vd[j] = vr[j];
    vd[j + half] = vr[j + half];
  }
}

hipError_t launch_cache_append(const void* k, const void* v, void* kc, void* vc, int bf16,
                               const int64_t* start, const int64_t* len, int64_t B, int64_t C,
                               int h_kv, int d, int64_t cap, int64_t end, RopeParams rp,
                               hipStream_t st, const int32_t* bt, int ps_log2, int64_t max_pages,
                               int64_t num_pages) {
  const int64_t n_pairs = B * C * h_kv * (d / 2);
  const int64_t want = (n_pairs + 255) / 256;
  const int grid = (int)(want < 65536 ? want : 65536);
  if (bf16)
    return launch_kernel(cache_append_kernel<uint16_t>, dim3(grid), dim3(256), st,
                         (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)kc, (uint16_t*)vc,
                         start, len, n_pairs, C, h_kv, d, cap, end, rp, bt, ps_log2, max_pages,
                         num_pages);
  return launch_kernel(cache_append_kernel<float>, dim3(grid), dim3(256), st, (const float*)k,
                       (const float*)v, (float*)kc, (float*)vc, start, len, n_pairs, C, h_kv, d,
                       cap, end, rp, bt, ps_log2, max_pages, num_pages);
}

hipError_t launch_kv_prepare_f32(const float* k, const float* v, RopeParams rp, float* kp,
                                 float* kc, float* vc, int64_t B, int64_t L, int h_kv, int d,
                                 int64_t cap, hipStream_t st) {
  dim3 grid((unsigned)((L + 63) / 64), (unsigned)h_kv, (unsigned)B);
  if (d == 128)
    return launch_kernel(kv_prepare_f32_kernel<128>, grid, dim3(256), st, k, v, rp, kp, kc, vc, L,
                         h_kv, cap);
  return launch_kernel(kv_prepare_f32_kernel<64>, grid, dim3(256), st, k, v, rp, kp, kc, vc, L,
                       h_kv, cap);
}

// ---------------------------------------------------------------------------
// QKV projection epilogue (walkthrough §4.1.3 steps 1-3 and §4.2: each
// projection adds its bias, the flat output is cut into heads, Q and K are
// rotated at their position; the closing note of §4.1.3: the h_kv groups' K
// and V go to the cache).  x[B, C, (h_q + 2 h_kv) d] is the packed
// projection output (query heads, then key heads, then value heads); token
// i < len[b] of sequence b sits at position p = start[b] + i:
//   q_out[b][i][t] = RoPE(x_Q(t) + bias_Q(t), p),
//   kc[b][p][u]    = RoPE(x_K(u) + bias_K(u), p),  vc[b][p][u] = x_V(u) + bias_V(u).
// A workgroup takes kEpiTokens tokens: their cos/sin (one per pair, shared by
// all h_q + h_kv heads) go to LDS first; then one item per pair of Q or K
// chunks (dims c.. and d/2 + c..) that one rotation couples, or per 16-byte
// chunk of a V head.  Sums and rotations in fp32, one rounding to the
// storage type.  Sequences outside [0, end) are skipped.
constexpr int kEpiTokens = 2;

template <typename T>
__global__ __launch_bounds__(256) void qkv_epilogue_kernel(
    const T* __restrict__ x, const T* __restrict__ bias, T* __restrict__ q_out,
    T* __restrict__ kc, T* __restrict__ vc, const int64_t* __restrict__ start,
    const int64_t* __restrict__ len, int64_t n_rows, int64_t C, int h_q, int h_kv, int d,
    int64_t cap, int64_t end, RopeParams rp) {
  constexpr int E = 16 / sizeof(T);             // elements per 16-byte chunk
  __shared__ float2 csl[kEpiTokens][64];        // (cos, sin) per token and pair (d <= 128)
  __shared__ double oml[64];                    // inverse frequency per pair
  const int cpr = d / E;                        // chunks per head row
  const int half = d / 2;
  const int nq = h_q * (cpr / 2), nk = h_kv * (cpr / 2), nv = h_kv * cpr;
  const int per_row = nq + nk + nv;
  const int width = (h_q + 2 * h_kv) * d;
  const int64_t row0 = (int64_t)blockIdx.x * kEpiTokens;
  // position of token `tok` of this workgroup, or -1 if it is not written
  auto token_pos = [&](int tok) -> int64_t {
    const int64_t row = row0 + tok;
    if (row >= n_rows) return -1;
    const int64_t b = row / C, i = row % C;
    const int64_t s0 = start[b], n = len ? len[b] : C;
    if (!(s0 >= 0 && n >= 0 && n <= C && s0 + n <= end) || i >= n) return -1;
    return s0 + i;
  };
  for (int j = threadIdx.x; j < half; j += blockDim.x) oml[j] = rope_omega(j, d, rp);
  __syncthreads();
  for (int idx = threadIdx.x; idx < kEpiTokens * half; idx += blockDim.x) {
    const int tok = idx / half, j = idx % half;
    const int64_t p = token_pos(tok);
    float c = 1.f, sn = 0.f;
    if (p >= 0) {
      rope_cos_sin((double)p, oml[j], c, sn);
      c *= rp.mscale;
      sn *= rp.mscale;
    }
    csl[tok][j] = make_float2(c, sn);
  }
  __syncthreads();
  // the projection output is read once (non-temporal); the bias by every token
  auto load = [&](const T* p, float* f, bool once = true) {
    const u32x4 w = once ? __builtin_nontemporal_load((const u32x4*)p) : *(const u32x4*)p;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = bf16_bits_to_f32((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(w[e]);
    }
  };
  auto store = [&](T* p, const float* f) {
    u32x4 w;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)f32_to_bf16_bits(f[2 * e]) | ((uint32_t)f32_to_bf16_bits(f[2 * e + 1]) << 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(f[e]);
    }
    __builtin_nontemporal_store(w, (u32x4*)p);   // written once
  };
  auto add_bias = [&](float* f, int col) {
    if (!bias) return;
    float bf[E];
    load(bias + col, bf, false);
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] += bf[e];
  };
  for (int it = threadIdx.x; it < kEpiTokens * per_row; it += blockDim.x) {
    const int tok = it / per_row, r = it % per_row;
    const int64_t p = token_pos(tok);
    if (p < 0) continue;
    const int64_t row = row0 + tok;
    const int64_t b = row / C;
    const T* xr = x + row * width;
    float f[E];
    if (r < nq + nk) {                          // Q or K: chunk c of both halves of a head
      const bool is_q = r < nq;
      const int hh = is_q ? r / (cpr / 2) : (r - nq) / (cpr / 2);
      const int c = (is_q ? r : r - nq) % (cpr / 2);
      const int col1 = (is_q ? hh : h_q + hh) * d + c * E, col2 = col1 + half;
      float g[E];
      load(xr + col1, f);
      add_bias(f, col1);
      load(xr + col2, g);
      add_bias(g, col2);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float2 cs = csl[tok][c * E + e];
        const float y1 = fmaf(f[e], cs.x, -g[e] * cs.y);
        const float y2 = fmaf(g[e], cs.x, f[e] * cs.y);
        f[e] = y1;
        g[e] = y2;
      }
      T* dst = is_q ? q_out + (row * h_q + hh) * d : kc + ((b * cap + p) * h_kv + hh) * d;
      store(dst + c * E, f);
      store(dst + half + c * E, g);
    } else {                                    // V chunk
      const int u = (r - nq - nk) / cpr, c = (r - nq - nk) % cpr;
      const int col = (h_q + h_kv + u) * d + c * E;
      load(xr + col, f);
      add_bias(f, col);
      store(vc + ((b * cap + p) * h_kv + u) * d + c * E, f);
    }
  }
}

hipError_t launch_qkv_epilogue(const void* x, const void* bias, void* q_out, void* kc, void* vc,
                               int bf16, const int64_t* start, const int64_t* len, int64_t B,
                               int64_t C, int h_q, int h_kv, int d, int64_t cap, int64_t end,
                               RopeParams rp, hipStream_t st) {
  const int64_t n_rows = B * C;
  const unsigned grid = (unsigned)((n_rows + kEpiTokens - 1) / kEpiTokens);
  if (bf16)
    qkv_epilogue_kernel<uint16_t><<<grid, 256, 0, st>>>(
        (const uint16_t*)x, (const uint16_t*)bias, (uint16_t*)q_out, (uint16_t*)kc, (uint16_t*)vc,
        start, len, n_rows, C, h_q, h_kv, d, cap, end, rp);
  else
    qkv_epilogue_kernel<float><<<grid, 256, 0, st>>>((const float*)x, (const float*)bias,
                                                     (float*)q_out, (float*)kc, (float*)vc, start,
                                                     len, n_rows, C, h_q, h_kv, d, cap, end,
                                                     rp);
  return hipGetLastError();
}

}  // namespace gqa
