// Split-K GQA decode over a contiguous per-layer KV cache.
//
// One new query token per sequence at position q_pos attends to the cached,
// already rotated keys 0 .. kv_len-1 (Qwen2 technical-report walkthrough,
// aicoding.csdn.net, §4.1.3: the cache holds only the h_kv groups' K and V,
// appended every step).  The query is rotated here at q_pos.
//
// The cache of one (batch, group) is cut into chunks of kDecodeChunk keys;
// a workgroup streams one chunk exactly once for all g query heads of the
// group (that single pass over the h_kv-group cache is what GQA saves in
// bandwidth, same page §4.1.1) and leaves an unnormalised partial state
// (row max m, sum l, weighted sum o).  A second kernel merges the chunks:
//   M = max_s m_s,  o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// which equals the unsplit softmax exactly (up to rounding).  Maxima are
// kept in the log2 domain (scores pre-multiplied by scale * log2 e).
//
// Ragged batches: with qpos_arr set, sequence b has its own query position
// qpos_arr[b] and length kvl_arr[b] (or qpos_arr[b] + 1 when the step has
// just appended its own row); kv_len is then the largest allowed length and
// sets the number of chunks.  Chunks past a sequence's length leave an empty
// state (m = -inf, l = 0, o = 0) that the merge weighs with zero.  A
// sequence whose length or position is out of range has no keys at all and
// its output becomes NaN.  With q_rotated set the query arrives rotated
// already (gqa_qkv_epilogue writes it so) and is used as given.
//
// Paged cache: with a block table, position j of sequence b lives in page
// bt[b][j >> ps_log2], row j & (page_size - 1), of the pools
// [num_pages, h_kv, page_size, d] (blocks of page_size positions per KV head,
// as PagedAttention manages memory per KV head: "从 Qwen 1 到 Qwen 2 ..."
// (nxmr.cn) §2).  A workgroup reads its chunk's page ids into LDS once; a
// chunk whose ids fall outside the pool makes the sequence's output NaN.

#include "common.h"
#include "launch.h"

namespace gqa {

namespace {

// K/V row addressing: contiguous [B, cap, h_kv, d] or paged pools
struct KvRows {
  const int32_t* bt;     // block table [B][max_pages], NULL: contiguous cache
  int ps_log2;           // log2(page_size)
  int64_t max_pages, num_pages, cap;
};

// per-sequence (kv_len, q_pos); kv_len = 0 marks an invalid sequence
struct SeqLen {
  int kv_len;
  double q_pos;
};

__device__ __forceinline__ SeqLen seq_len(int b, int kv_len, double q_pos,
                                          const int64_t* __restrict__ kvl_arr,
                                          const int64_t* __restrict__ qpos_arr, int kvl_from_pos) {
  if (!qpos_arr) return {kv_len, q_pos};
  const int64_t qp = qpos_arr[b];
  const int64_t kl = kvl_from_pos ? qp + 1 : kvl_arr[b];
  const bool ok = kl >= 1 && kl <= kv_len && qp >= kl - 1 && qp <= (INT64_C(1) << 40);
  return {ok ? (int)kl : 0, (double)qp};
}

// Page ids of positions [k0, k1) of sequence b into pg[]; false if any id or
// table slot is out of range.  Every thread of the workgroup calls it.
__device__ bool stage_pages(const KvRows& kr, int b, int k0, int k1, int* pg) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int64_t first = (int64_t)k0 >> kr.ps_log2;
  const int n = (int)((((int64_t)k1 - 1) >> kr.ps_log2) - first + 1);
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t slot = first + i;
    int pid = -1;
    if (slot < kr.max_pages) pid = kr.bt[(int64_t)b * kr.max_pages + slot];
    if (pid < 0 || pid >= kr.num_pages) {
      bad = 1;
      pid = 0;
    }
    pg[i] = pid;
  }
  __syncthreads();
  return bad == 0;
}

// element offset of (sequence b, position key, group u) in the K or V store:
// contiguous cache, or row key & (page_size - 1) of the key's page
template <bool PAGED>
__device__ __forceinline__ int64_t kv_row(const KvRows& kr, const int* pg, int k0, int b, int key,
                                          int u, int h_kv, int D) {
  if constexpr (!PAGED) {
    return ((int64_t)b * kr.cap * h_kv + u) * D + (int64_t)key * (h_kv * D);
  } else {
    const int page = pg[(key >> kr.ps_log2) - (k0 >> kr.ps_log2)];
    const int row = key & ((1 << kr.ps_log2) - 1);
    return (((int64_t)page * h_kv + u) * ((int64_t)1 << kr.ps_log2) + row) * D;
  }
}

// partial state of an invalid chunk: the merge turns it into NaN output
__device__ void write_nan_state(float* pm, float* pl, float* po, int64_t out0, int nh, int D) {
  for (int idx = threadIdx.x; idx < 16 * D; idx += blockDim.x) {
    const int cc = idx / D, dim = idx % D;
    if (cc >= nh) continue;
    po[(out0 + cc) * D + dim] = 0.f;
    if (dim == 0) {
      pm[out0 + cc] = __builtin_nanf("");
      pl[out0 + cc] = 0.f;
    }
  }
}

}  // namespace

int decode_num_splits(int64_t kv_len) {
  return (int)((kv_len + kDecodeChunk - 1) / kDecodeChunk);
}

// bf16 cache, matrix cores.  Workgroup = (chunk, group u x head block, b);
// four waves take a quarter of the chunk each.  Per 32-key step a wave
// computes S^T = K q^T (v_mfma_f32_16x16x32_bf16: 16 keys x 16 heads, K
// rows straight from HBM into the A operand), then O^T += V^T P^T with V
// staged through a wave-private LDS slab to turn key-major rows into the
// key-contiguous operand.  Heads beyond 16 per group run as extra head
// blocks (another pass over the chunk).  The cache is read once, so its
// loads are non-temporal (they do not displace reused lines in the caches).
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void decode_split_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ po, int h_q, int h_kv, int g, int n_hb, int64_t cap, int kv_len_max,
    double q_pos_s, RopeParams rp, float sl2, int n_split, const int64_t* __restrict__ kvl_arr,
    const int64_t* __restrict__ qpos_arr, int kvl_from_pos, int q_rotated, KvRows kr) {
  constexpr int CH = kDecodeChunk;
  constexpr int WK = CH / 4;            // keys per wave
  constexpr int NS = D / 32;            // 32-dim k-steps of S^T
  constexpr int NDB = D / 16;           // 16-dim blocks of O^T
  constexpr int VPITCH = D + 8;         // LDS pitch of a staged V row (elements)
  constexpr int VLD = 32 * D / 8 / 64;  // 16-byte V loads per lane per 32-key step
  __shared__ __attribute__((aligned(16))) uint16_t vsh[4][32 * VPITCH];
  __shared__ float cm[4][16], cl[4][16];
  __shared__ float co[4][16][D + 1];
  __shared__ int pg[CH];                // page ids of this chunk (paged cache)

  const int split = blockIdx.x;
  const int u = blockIdx.y / n_hb, hb = blockIdx.y % n_hb;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, h4 = lane >> 4;
  const int c = hb * 16 + col;
  const SeqLen sq = seq_len(b, kv_len_max, q_pos_s, kvl_arr, qpos_arr, kvl_from_pos);
  const int kv_len = sq.kv_len;
  const double q_pos = sq.q_pos;
  if (split * CH >= kv_len) {   // chunk past this sequence's keys: empty state
    for (int idx = tid; idx < 16 * D; idx += 256) {
      const int cc = idx / D, dim = idx % D;
      if (hb * 16 + cc >= g) continue;
      const int64_t out = (((int64_t)b * h_kv + u) * n_split + split) * g + hb * 16 + cc;
      po[out * D + dim] = 0.f;
      if (dim == 0) {
        pm[out] = -INFINITY;
        pl[out] = 0.f;
      }
    }
    return;
  }
  const int chunk0 = split * CH;
  if (PAGED && !stage_pages(kr, b, chunk0, min(chunk0 + CH, kv_len), pg)) {
    write_nan_state(pm, pl, po, (((int64_t)b * h_kv + u) * n_split + split) * g + hb * 16,
                    min(16, g - hb * 16), D);
    return;
  }

  // ---- rotated query, B operand: lane holds head `col`, dims s*32 + h4*8 + e
  bf16x8 qb[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[s][e] = (__bf16)0.f;
  if (c < g) {
    const uint16_t* qrow = q + ((int64_t)b * h_q + (int64_t)u * g + c) * D;
#pragma unroll
    for (int s = 0; s < NS / 2; ++s) {
      const u32x4 r1 = *(const u32x4*)(qrow + s * 32 + h4 * 8);
      const u32x4 r2 = *(const u32x4*)(qrow + s * 32 + h4 * 8 + D / 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = s * 32 + h4 * 8 + e;
        float cs_c = 1.f, cs_s = 0.f;   // q_rotated: the query is used as given
        if (!q_rotated) rope_cs(q_pos, j, D, rp, cs_c, cs_s);
        const float x1 = (e & 1) ? __uint_as_float(r1[e >> 1] & 0xffff0000u)
                                 : __uint_as_float(r1[e >> 1] << 16);
        const float x2 = (e & 1) ? __uint_as_float(r2[e >> 1] & 0xffff0000u)
                                 : __uint_as_float(r2[e >> 1] << 16);
        qb[s][e] = (__bf16)fmaf(x1, cs_c, -x2 * cs_s);
        qb[s + NS / 2][e] = (__bf16)fmaf(x2, cs_c, x1 * cs_s);
      }
    }
  }

  const int kw0 = split * CH + wave * WK;
  const int kw1 = min(kw0 + WK, kv_len);

  float m = -INFINITY, l = 0.f;
  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* vw = vsh[wave];

  for (int k0 = kw0; k0 < kw1; k0 += 32) {
    u32x4 ka[2][NS];
    u32x4 va[VLD];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int key = min(k0 + blk * 16 + col, kv_len - 1);
#pragma unroll
      for (int s = 0; s < NS; ++s)
        ka[blk][s] = __builtin_nontemporal_load(
            (const u32x4*)(kc + kv_row<PAGED>(kr, pg, chunk0, b, key, u, h_kv, D) + s * 32 + h4 * 8));
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int ch = lane + 64 * i;
      const int key = min(k0 + ch / (D / 8), kv_len - 1);
      va[i] = __builtin_nontemporal_load(
          (const u32x4*)(vc + kv_row<PAGED>(kr, pg, chunk0, b, key, u, h_kv, D) + (ch % (D / 8)) * 8));
    }
    // S^T for 2 x 16 keys
    f32x4 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      sacc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        sacc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, ka[blk][s]), qb[s], sacc[blk], 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (k0 + blk * 16 + h4 * 4 + i >= kw1) sacc[blk][i] = -INFINITY;
        mx = fmaxf(mx, sacc[blk][i]);
      }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m, mx * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    bf16x8 pb;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 p = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[e >> 2][e & 3], sl2, -m_new));
      pb[e] = p;
      psum += (float)p;
    }
    l = fmaf(l, alpha, psum);
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;

    // V rows -> wave-private LDS (row-major), then the key-contiguous operand
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int ch = lane + 64 * i;
      *(u32x4*)(vw + (ch / (D / 8)) * VPITCH + (ch % (D / 8)) * 8) = va[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bf16x8 a;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = (e < 4) ? h4 * 4 + e : 16 + h4 * 4 + (e - 4);
        a[e] = __builtin_bit_cast(__bf16, vw[kk * VPITCH + db * 16 + col]);
      }
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, oacc[db], 0, 0, 0);
    }
  }

  // ---- combine the four waves of the workgroup
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (h4 == 0) {
    cm[wave][col] = m;
    cl[wave][col] = l;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) co[wave][col][db * 16 + h4 * 4 + i] = oacc[db][i];
  __syncthreads();
  for (int idx = tid; idx < 16 * D; idx += 256) {
    const int cc = idx / D, dim = idx % D;
    if (hb * 16 + cc >= g) continue;
    float M = cm[0][cc];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, cm[w][cc]);
    float so = 0.f, sl = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(cm[w][cc] - M);
      so = fmaf(f, co[w][cc][dim], so);
      sl = fmaf(f, cl[w][cc], sl);
    }
    const int64_t out = (((int64_t)b * h_kv + u) * n_split + split) * g + hb * 16 + cc;
    po[out * D + dim] = so;
    if (dim == 0) {
      pm[out] = M;
      pl[out] = sl;
    }
  }
}

// fp32 cache, vector ALU (the fp32 parity path).  Workgroup = (chunk, u x
// head block, b); 16 threads per head.  Scores of the chunk go to LDS, then
// each thread reduces one head's max and sum and accumulates 1/16 of its
// output dims.
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void decode_split_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    float* __restrict__ pm, float* __restrict__ pl, float* __restrict__ po, int h_q, int h_kv,
    int g, int n_hb, int64_t cap, int kv_len_max, double q_pos_s, RopeParams rp, float scale,
    int n_split, const int64_t* __restrict__ kvl_arr, const int64_t* __restrict__ qpos_arr,
    int kvl_from_pos, int q_rotated, KvRows kr) {
  constexpr int CH = kDecodeChunk;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ float qs[16][D];
  __shared__ float sc[16][CH];
  __shared__ int pg[CH];                // page ids of this chunk (paged cache)
  const int split = blockIdx.x;
  const int u = blockIdx.y / n_hb, hb = blockIdx.y % n_hb;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int nh = min(16, g - hb * 16);
  const SeqLen sq = seq_len(b, kv_len_max, q_pos_s, kvl_arr, qpos_arr, kvl_from_pos);
  const int kv_len = sq.kv_len;
  const double q_pos = sq.q_pos;
  if (split * CH >= kv_len) {   // chunk past this sequence's keys: empty state
    for (int idx = tid; idx < 16 * D; idx += 256) {
      const int cc = idx / D, dim = idx % D;
      if (cc >= nh) continue;
      const int64_t out = (((int64_t)b * h_kv + u) * n_split + split) * g + hb * 16 + cc;
      po[out * D + dim] = 0.f;
      if (dim == 0) {
        pm[out] = -INFINITY;
        pl[out] = 0.f;
      }
    }
    return;
  }
  if (PAGED && !stage_pages(kr, b, split * CH, min(split * CH + CH, kv_len), pg)) {
    write_nan_state(pm, pl, po, (((int64_t)b * h_kv + u) * n_split + split) * g + hb * 16, nh, D);
    return;
  }

  for (int idx = tid; idx < 16 * (D / 2); idx += 256) {
    const int cc = idx / (D / 2), j = idx % (D / 2);
    float y1 = 0.f, y2 = 0.f;
    if (cc < nh) {
      const float* qrow = q + ((int64_t)b * h_q + (int64_t)u * g + hb * 16 + cc) * D;
      float c = 1.f, s = 0.f;   // q_rotated: the query is used as given
      if (!q_rotated) rope_cs(q_pos, j, D, rp, c, s);
      y1 = fmaf(qrow[j], c, -qrow[j + D / 2] * s);
      y2 = fmaf(qrow[j + D / 2], c, qrow[j] * s);
    }
    qs[cc][j] = y1;
    qs[cc][j + D / 2] = y2;
  }
  __syncthreads();

  const int k0 = split * CH;
  const int nk = min(CH, kv_len - k0);
  for (int kk = tid; kk < nk; kk += 256) {
    const float* krow = kc + kv_row<PAGED>(kr, pg, k0, b, k0 + kk, u, h_kv, D);
    for (int cc = 0; cc < nh; ++cc) {
      float dot = 0.f;
      for (int dd = 0; dd < D; ++dd) dot = fmaf(qs[cc][dd], krow[dd], dot);
      sc[cc][kk] = dot * scale;
    }
  }
  __syncthreads();

  const int cc = tid >> 4, sub = tid & 15;
  float M = -INFINITY;
  if (cc < nh)
    for (int kk = sub; kk < nk; kk += 16) M = fmaxf(M, sc[cc][kk]);
  for (int msk = 1; msk < 16; msk <<= 1) M = fmaxf(M, __shfl_xor(M, msk, 64));
  __syncthreads();
  float Ls = 0.f;
  if (cc < nh)
    for (int kk = sub; kk < nk; kk += 16) {
      const float p = expf(sc[cc][kk] - M);
      sc[cc][kk] = p;
      Ls += p;
    }
  for (int msk = 1; msk < 16; msk <<= 1) Ls += __shfl_xor(Ls, msk, 64);
  __syncthreads();
  if (cc < nh) {
    constexpr int DPT = D / 16;
    float acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
    for (int kk = 0; kk < nk; ++kk) {
      const float p = sc[cc][kk];
      const float* vrow = vc + kv_row<PAGED>(kr, pg, k0, b, k0 + kk, u, h_kv, D) + sub * DPT;
#pragma unroll
      for (int e = 0; e < DPT; ++e) acc[e] = fmaf(p, vrow[e], acc[e]);
    }
    const int64_t out = (((int64_t)b * h_kv + u) * n_split + split) * g + hb * 16 + cc;
#pragma unroll
    for (int e = 0; e < DPT; ++e) po[out * D + sub * DPT + e] = acc[e];
    if (sub == 0) {
      pm[out] = M * kLog2e;
      pl[out] = Ls;
    }
  }
}

// Merge the chunk partials of one (b, query head); one thread per dim.  The
// chunk maxima and sums are staged in LDS once; every thread then issues its
// per-chunk loads independently.
template <bool OUT_BF16>
__global__ __launch_bounds__(128) void decode_merge_kernel(const float* __restrict__ pm,
                                                           const float* __restrict__ pl,
                                                           const float* __restrict__ po,
                                                           void* __restrict__ o, int h_q, int h_kv,
                                                           int g, int d, int n_split) {
  __shared__ float wsc[kDecodeMaxSplitsLds];
  __shared__ float red[2];
  const int t = blockIdx.x, b = blockIdx.y;
  const int u = t / g, c = t % g;
  const int64_t base = (((int64_t)b * h_kv + u) * n_split) * g + c;
  // 1) global max of the chunk maxima (n_split <= kDecodeMaxSplitsLds)
  float M = -INFINITY;
  for (int s = threadIdx.x; s < n_split; s += blockDim.x) M = fmaxf(M, pm[base + (int64_t)s * g]);
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = M;
  __syncthreads();
  M = fmaxf(red[0], blockDim.x > 64 ? red[1] : -INFINITY);
  __syncthreads();
  // 2) chunk weights 2^(m_s - M) and the total sum
  float Ls = 0.f;
  for (int s = threadIdx.x; s < n_split; s += blockDim.x) {
    const float w = __builtin_amdgcn_exp2f(pm[base + (int64_t)s * g] - M);
    wsc[s] = w;
    Ls = fmaf(w, pl[base + (int64_t)s * g], Ls);
  }
  for (int m = 32; m >= 1; m >>= 1) Ls += __shfl_xor(Ls, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = Ls;
  __syncthreads();
  const float inv = 1.0f / (red[0] + (blockDim.x > 64 ? red[1] : 0.f));
  // 3) weighted sum of the chunk outputs
  for (int dim = threadIdx.x; dim < d; dim += blockDim.x) {
    float acc = 0.f;
#pragma unroll 8
    for (int s = 0; s < n_split; ++s)
      acc = fmaf(wsc[s], po[(base + (int64_t)s * g) * d + dim], acc);
    const int64_t oo = ((int64_t)b * h_q + t) * d + dim;
    if constexpr (OUT_BF16)
      ((uint16_t*)o)[oo] = f32_to_bf16_bits(acc * inv);
    else
      ((float*)o)[oo] = acc * inv;
  }
}

hipError_t launch_decode(const void* q, const void* kc, const void* vc, void* o, int in_bf16,
                         int out_bf16, int64_t B, int h_q, int h_kv, int d, int64_t cap,
                         int64_t kv_len, int64_t q_pos, const int64_t* kvl_arr,
                         const int64_t* qpos_arr, int kvl_from_pos, int q_rotated,
                         const int32_t* bt, int ps_log2, int64_t max_pages, int64_t num_pages,
                         RopeParams rp,
                         float scale, float* ws_m, float* ws_l, float* ws_o, hipStream_t st,
                         hipEvent_t ev_begin, hipEvent_t ev_end) {
  const int g = h_q / h_kv;
  const int n_hb = (g + 15) / 16;
  const int n_split = decode_num_splits(kv_len);
  dim3 grid((unsigned)n_split, (unsigned)(h_kv * n_hb), (unsigned)B);
  const float sl2 = scale * 1.4426950408889634f;
  const KvRows kr{bt, ps_log2, max_pages, num_pages, cap};
  if (ev_begin) (void)hipEventRecord(ev_begin, st);
  const bool paged = bt != nullptr;
#define GQA_SPLIT(KERNEL, T, DD, PG, SC)                                                         \
  KERNEL<DD, PG><<<grid, 256, 0, st>>>((const T*)q, (const T*)kc, (const T*)vc, ws_m, ws_l, ws_o, \
                                       h_q, h_kv, g, n_hb, cap, (int)kv_len, (double)q_pos, rp,  \
                                       SC, n_split, kvl_arr, qpos_arr, kvl_from_pos, q_rotated, kr)
  if (in_bf16) {
    if (d == 128) {
      if (paged) GQA_SPLIT(decode_split_bf16_kernel, uint16_t, 128, true, sl2);
      else GQA_SPLIT(decode_split_bf16_kernel, uint16_t, 128, false, sl2);
    } else {
      if (paged) GQA_SPLIT(decode_split_bf16_kernel, uint16_t, 64, true, sl2);
      else GQA_SPLIT(decode_split_bf16_kernel, uint16_t, 64, false, sl2);
    }
  } else {
    if (d == 128) {
      if (paged) GQA_SPLIT(decode_split_f32_kernel, float, 128, true, scale);
      else GQA_SPLIT(decode_split_f32_kernel, float, 128, false, scale);
    } else {
      if (paged) GQA_SPLIT(decode_split_f32_kernel, float, 64, true, scale);
      else GQA_SPLIT(decode_split_f32_kernel, float, 64, false, scale);
    }
  }
#undef GQA_SPLIT
  hipError_t err = hipGetLastError();
  if (ev_end) (void)hipEventRecord(ev_end, st);
  if (err != hipSuccess) return err;
  dim3 mgrid((unsigned)h_q, (unsigned)B);
  if (out_bf16)
    decode_merge_kernel<true><<<mgrid, 128, 0, st>>>(ws_m, ws_l, ws_o, o, h_q, h_kv, g, d, n_split);
  else
    decode_merge_kernel<false><<<mgrid, 128, 0, st>>>(ws_m, ws_l, ws_o, o, h_q, h_kv, g, d,
                                                      n_split);
  return hipGetLastError();
}

}  // namespace gqa
