// Split-K GQA decode over a contiguous per-layer KV cache.
//
// One new query token per sequence at position q_pos attends to the cached,
// already rotated keys 0 .. kv_len-1 (Qwen2 technical-report walkthrough,
// aicoding.csdn.net, §4.1.3: the cache holds only the h_kv groups' K and V,
// appended every step).  The query is rotated here at q_pos.
//
// The cache of one (batch, group) is cut into chunks of kDecodeChunkBf16
// (bf16) or kDecodeChunk (fp32) keys; a workgroup streams one chunk exactly
// once for all g query heads of the group (that single pass over the h_kv-group cache is what GQA saves in
// bandwidth, same page §4.1.1) and leaves an unnormalised partial state
// (row max m, sum l, weighted sum o).  A second kernel merges the chunks:
//   M = max_s m_s,  o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// which equals the unsplit softmax exactly (up to rounding).  Maxima are
// kept in the log2 domain (scores pre-multiplied by scale * log2 e).  (A
// merge by the last-arriving chunk of each group, through an atomic ticket,
// needs a device-scope release in every workgroup; on gfx950 that writes
// back the XCD's L2 each time and made the call four times slower.)
//
// Ragged batches: with qpos_arr set, sequence b has its own query position
// qpos_arr[b] and length kvl_arr[b] (or qpos_arr[b] + 1 when the step has
// just appended its own row); kv_len is then the largest allowed length and
// sets the number of chunks.  Chunks past a sequence's length leave an empty
// state (m = -inf, l = 0, o = 0) that the merge weighs with zero.  A
// sequence whose length or position is out of range has no keys at all and
// its output becomes NaN.  With q_rotated set the query arrives rotated
// already (gqa_qkv_epilogue writes it so) and is used as given.  With an
// appended token (k_new set) a preparation kernel first writes sequence b's
// new row to position qpos_arr[b], if that lies in [0, append_end), and
// rotates the query once into the workspace; the sequence then attends to
// rows 0 .. qpos_arr[b].
//
// Paged cache: with a block table, position j of sequence b lives in page
// bt[b][j >> ps_log2], row j & (page_size - 1), of the pools
// [num_pages, h_kv, page_size, d] (blocks of page_size positions per KV head,
// as PagedAttention manages memory per KV head: "从 Qwen 1 到 Qwen 2 ..."
// (nxmr.cn) §2).  A workgroup reads its chunk's page ids into LDS once; a
// chunk whose ids fall outside the pool makes the sequence's output NaN.

#include <mutex>

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

// Partial state (m, 0, 0) of nh heads starting at partial index out0:
// m = -inf is an empty chunk (weight 0 in the merge), m = NaN an invalid one
// (the merge turns it into NaN output).
__device__ void write_flat_state(float* pm, float* pl, float* po, int64_t out0, int nh, int D,
                                 float m) {
  for (int idx = threadIdx.x; idx < nh * D; idx += blockDim.x) {
    const int cc = idx / D, dim = idx % D;
    po[(out0 + cc) * D + dim] = 0.f;
    if (dim == 0) {
      pm[out0 + cc] = m;
      pl[out0 + cc] = 0.f;
    }
  }
}

}  // namespace

int decode_num_splits(int64_t kv_len, bool bf16) {
  const int ch = bf16 ? kDecodeChunkBf16 : kDecodeChunk;
  return (int)((kv_len + ch - 1) / ch);
}

// Chunk states of an allocation-free decode call, in device memory that the
// code object reserves: each device holds its own copy, at its own address,
// from the library's load until the process ends.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the host-side name of the array is no device address: ask the runtime
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Preparation of an appending step, one workgroup per sequence b: (1) its
// query rows rotated at p = qpos_arr[b] (or used as given when q_rotated)
// and rounded once to T, into qr [B, h_q, d]; (2) the new token's K
// rotated at p and its V written to cache position p (contiguous, or
// through the block table), if 0 <= p < append_end and its page id is in
// range.
template <typename T>
__global__ __launch_bounds__(256) void decode_prep_kernel(
    const T* __restrict__ q, T* __restrict__ qr, const T* __restrict__ k_new,
    const T* __restrict__ v_new, T* __restrict__ kc, T* __restrict__ vc, int h_q, int h_kv,
    int d, int64_t append_end, const int64_t* __restrict__ qpos_arr, int q_rotated,
    RopeParams rp, KvRows kr) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int half = d >> 1;
  const int64_t qp = qpos_arr[b];
  auto ld = [](const T* p) -> float {
    if constexpr (sizeof(T) == 2) return bf16_bits_to_f32(*(const uint16_t*)p);
    else return *p;
  };
  auto st = [](T* p, float y) {
    if constexpr (sizeof(T) == 2) *(uint16_t*)p = f32_to_bf16_bits(y);
    else *p = y;
  };
  for (int idx = tid; idx < h_q * half; idx += blockDim.x) {
    const int t = idx / half, j = idx % half;
    const T* src = q + ((int64_t)b * h_q + t) * d;
    T* dst = qr + ((int64_t)b * h_q + t) * d;
    const float x1 = ld(src + j), x2 = ld(src + j + half);
    float c = 1.f, sn = 0.f;
    if (!q_rotated) rope_cs((double)qp, j, d, rp, c, sn);
    st(dst + j, fmaf(x1, c, -x2 * sn));
    st(dst + j + half, fmaf(x2, c, x1 * sn));
  }
  if (!(qp >= 0 && qp < append_end)) return;
  int64_t row0 = ((int64_t)b * kr.cap + qp) * h_kv * d;   // contiguous: [B, cap, h_kv, d]
  int64_t head_stride = d;
  if (kr.bt) {
    const int64_t slot = qp >> kr.ps_log2;
    const int pid = slot < kr.max_pages ? kr.bt[(int64_t)b * kr.max_pages + slot] : -1;
    if (pid < 0 || pid >= kr.num_pages) return;
    // pools [num_pages, h_kv, page_size, d]
    row0 = (((int64_t)pid * h_kv) << kr.ps_log2) * d + (qp & ((1 << kr.ps_log2) - 1)) * d;
    head_stride = ((int64_t)1 << kr.ps_log2) * d;
  }
  for (int idx = tid; idx < h_kv * half; idx += blockDim.x) {
    const int u = idx / half, j = idx % half;
    const T* ks = k_new + ((int64_t)b * h_kv + u) * d;
    const T* vs = v_new + ((int64_t)b * h_kv + u) * d;
    T* kd = kc + row0 + u * head_stride;
    T* vd = vc + row0 + u * head_stride;
    float c, sn;
    rope_cs((double)qp, j, d, rp, c, sn);
    const float x1 = ld(ks + j), x2 = ld(ks + j + half);
    st(kd + j, fmaf(x1, c, -x2 * sn));
    st(kd + j + half, fmaf(x2, c, x1 * sn));
    vd[j] = vs[j];
    vd[j + half] = vs[j + half];
  }
}


// bf16 cache, matrix cores.  Workgroup = (chunk, group(s) x head block, b).
// Per 32-key step a wave loads the K and V rows of its keys whole (D/8
// lanes to a row, into registers one step ahead) and passes them through a
// wave-private LDS slab in turn: K to form the A operands of S^T = K q^T
// (v_mfma_f32_16x16x32_bf16: 16 keys x 16 heads), V to read it back
// key-contiguous for O^T += V^T P^T.  Heads beyond 16 per group run as extra head blocks
// (another pass over the chunk).  The cache is read once, so its loads are
// non-temporal (they do not displace reused lines in the caches).
// GRP (h_kv a multiple of 4): the workgroup takes one chunk for four KV
// groups, wave w group 4*ub + w over the whole chunk, so that the
// workgroup's loads cover whole cache rows (all groups of a key are
// adjacent in the contiguous cache): 7.0 against 6.6 TB/s for the split's
// load pattern alone.  Each wave then writes its group's state itself.
// Otherwise the four waves take a quarter of the chunk of one group each and
// their states are combined through LDS.
template <int D, bool PAGED, bool GRP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_split_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ po, int h_q, int h_kv, int g, int n_hb, int kv_len_max, double q_pos_s,
    RopeParams rp, float sl2, int n_split, const int64_t* __restrict__ kvl_arr,
    const int64_t* __restrict__ qpos_arr, int kvl_from_pos, int q_rotated, KvRows kr) {
  constexpr int CH = kDecodeChunkBf16;
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
  const int hb = blockIdx.y % n_hb;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u = GRP ? (blockIdx.y / n_hb) * 4 + wave : blockIdx.y / n_hb;
  const int col = lane & 15, h4 = lane >> 4;
  const int c = hb * 16 + col;
  const int nh = min(16, g - hb * 16);
  const SeqLen sq = seq_len(b, kv_len_max, q_pos_s, kvl_arr, qpos_arr, kvl_from_pos);
  const int kv_len = sq.kv_len;
  const int chunk0 = split * CH;
  auto state0 = [&](int uu) { return (((int64_t)b * h_kv + uu) * n_split + split) * g + hb * 16; };
  const int64_t out0 = state0(u);
  // an empty or unreadable chunk: the state of every group of the workgroup
  auto flat_states = [&](float mval) {
    if constexpr (GRP) {
      for (int w = 0; w < 4; ++w)
        write_flat_state(pm, pl, po, state0((blockIdx.y / n_hb) * 4 + w), nh, D, mval);
    } else {
      write_flat_state(pm, pl, po, out0, nh, D, mval);
    }
  };

  if (chunk0 >= kv_len) {   // chunk past this sequence's keys: empty state
    flat_states(-INFINITY);
  } else if (PAGED && !stage_pages(kr, b, chunk0, min(chunk0 + CH, kv_len), pg)) {
    flat_states(__builtin_nanf(""));
  } else {
    const int kw0 = GRP ? chunk0 : chunk0 + wave * WK;
    const int kw1 = min(kw0 + (GRP ? CH : WK), kv_len);
    // one 32-key step's K and V rows, 16 bytes per load, non-temporal; D/8
    // lanes read one whole row, so a load covers a few complete rows (the
    // rows of a group lie at a stride of h_kv rows in the contiguous cache)
    auto load_step = [&](int k0, u32x4 (&ka)[VLD], u32x4 (&va)[VLD]) {
#pragma unroll
      for (int i = 0; i < VLD; ++i) {
        const int ch = lane + 64 * i;
        const int key = min(k0 + ch / (D / 8), kv_len - 1);
        ka[i] = __builtin_nontemporal_load(
            (const u32x4*)(kc + kv_row<PAGED>(kr, pg, chunk0, b, key, u, h_kv, D) +
                           (ch % (D / 8)) * 8));
      }
#pragma unroll
      for (int i = 0; i < VLD; ++i) {
        const int ch = lane + 64 * i;
        const int key = min(k0 + ch / (D / 8), kv_len - 1);
        va[i] = __builtin_nontemporal_load(
            (const u32x4*)(vc + kv_row<PAGED>(kr, pg, chunk0, b, key, u, h_kv, D) +
                           (ch % (D / 8)) * 8));
      }
    };

    // the first step's loads go out before the query rotation; then each
    // step's loads go out before the previous step is computed (two register
    // buffers, the loop unrolled by two so that neither is copied)
    u32x4 kaA[VLD], vaA[VLD], kaB[VLD], vaB[VLD];
    if (kw0 < kw1) load_step(kw0, kaA, vaA);

    // ---- rotated query, B operand: lane holds head `col`, dims
    // s*32 + h4*8 + e (rotated here at the query position unless q_rotated)
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
          if (!q_rotated) rope_cs(sq.q_pos, j, D, rp, cs_c, cs_s);
          const float x1 = (e & 1) ? __uint_as_float(r1[e >> 1] & 0xffff0000u)
                                   : __uint_as_float(r1[e >> 1] << 16);
          const float x2 = (e & 1) ? __uint_as_float(r2[e >> 1] & 0xffff0000u)
                                   : __uint_as_float(r2[e >> 1] << 16);
          qb[s][e] = (__bf16)fmaf(x1, cs_c, -x2 * cs_s);
          qb[s + NS / 2][e] = (__bf16)fmaf(x2, cs_c, x1 * cs_s);
        }
      }
    }

    float m = -INFINITY, l = 0.f;
    f32x4 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint16_t* vw = vsh[wave];

    // scores, online softmax and P.V of the step at k0
    auto compute_step = [&](int k0, const u32x4 (&ka)[VLD], const u32x4 (&va)[VLD]) {
      // K rows -> the wave's LDS slab (row-major), then the A operands of
      // S^T for 2 x 16 keys: lane (col, h4) takes dims s*32 + h4*8 .. +7 of
      // key blk*16 + col
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();   // the previous step's V reads are done
#pragma unroll
      for (int i = 0; i < VLD; ++i) {
        const int ch = lane + 64 * i;
        *(u32x4*)(vw + (ch / (D / 8)) * VPITCH + (ch % (D / 8)) * 8) = ka[i];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      f32x4 sacc[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        sacc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
          sacc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *(const bf16x8*)(vw + (blk * 16 + col) * VPITCH + s * 32 + h4 * 8), qb[s],
              sacc[blk], 0, 0, 0);
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

      // V rows -> the same slab (the K reads are done), then the
      // key-contiguous operand
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
    };

    for (int k0 = kw0; k0 < kw1; k0 += 64) {
      if (k0 + 32 < kw1) load_step(k0 + 32, kaB, vaB);
      compute_step(k0, kaA, vaA);
      if (k0 + 32 >= kw1) break;
      if (k0 + 64 < kw1) load_step(k0 + 64, kaA, vaA);
      compute_step(k0 + 32, kaB, vaB);
    }

    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if constexpr (GRP) {   // this wave's group state (m is the same in the four h4 lanes)
      if (col < nh) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          *(f32x4*)(po + (out0 + col) * D + db * 16 + h4 * 4) = oacc[db];
        if (h4 == 0) {
          pm[out0 + col] = m;
          pl[out0 + col] = l;
        }
      }
      return;
    }
    // ---- combine the four waves of the workgroup
    if (h4 == 0) {
      cm[wave][col] = m;
      cl[wave][col] = l;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) co[wave][col][db * 16 + h4 * 4 + i] = oacc[db][i];
    __syncthreads();
    for (int idx = tid; idx < nh * D; idx += 256) {
      const int cc = idx / D, dim = idx % D;
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
      po[(out0 + cc) * D + dim] = so;
      if (dim == 0) {
        pm[out0 + cc] = M;
        pl[out0 + cc] = sl;
      }
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
    int g, int n_hb, int kv_len_max, double q_pos_s, RopeParams rp, float scale, int n_split,
    const int64_t* __restrict__ kvl_arr, const int64_t* __restrict__ qpos_arr, int kvl_from_pos,
    int q_rotated, KvRows kr) {
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
  const int64_t out0 = (((int64_t)b * h_kv + u) * n_split + split) * g + hb * 16;

  if (split * CH >= kv_len) {   // chunk past this sequence's keys: empty state
    write_flat_state(pm, pl, po, out0, nh, D, -INFINITY);
  } else if (PAGED && !stage_pages(kr, b, split * CH, min(split * CH + CH, kv_len), pg)) {
    write_flat_state(pm, pl, po, out0, nh, D, __builtin_nanf(""));
  } else {
    for (int idx = tid; idx < 16 * (D / 2); idx += 256) {
      const int cc = idx / (D / 2), j = idx % (D / 2);
      float y1 = 0.f, y2 = 0.f;
      if (cc < nh) {
        const float* qrow = q + ((int64_t)b * h_q + (int64_t)u * g + hb * 16 + cc) * D;
        float c = 1.f, s = 0.f;   // q_rotated: the query is used as given
        if (!q_rotated) rope_cs(sq.q_pos, j, D, rp, c, s);
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
#pragma unroll
      for (int e = 0; e < DPT; ++e) po[(out0 + cc) * D + sub * DPT + e] = acc[e];
      if (sub == 0) {
        pm[out0 + cc] = M * kLog2e;
        pl[out0 + cc] = Ls;
      }
    }
  }

}

// Merge of the chunk partials of one (b, query head), one thread per dim.
// Chunk states are folded in batches of 32, every load of a batch issued
// before any of them is used (one memory latency per batch), with an online
// rescale between batches.  Empty chunks (m = -inf) weigh nothing; a NaN
// state, or no non-empty chunk at all, gives NaN.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ pm,
                                                         const float* __restrict__ pl,
                                                         const float* __restrict__ po,
                                                         void* __restrict__ o, int h_q, int h_kv,
                                                         int g, int n_split) {
  constexpr int NB = 32;
  const int t = blockIdx.x, b = blockIdx.y, dim = threadIdx.x;
  const int u = t / g, c = t % g;
  const int64_t base = (((int64_t)b * h_kv + u) * n_split) * g + c;
  float M = -INFINITY, lsum = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < n_split; s0 += NB) {
    float mv[NB], lv[NB], ov[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const bool in = s0 + j < n_split;
      const int64_t e = base + (int64_t)(in ? s0 + j : 0) * g;
      mv[j] = in ? pm[e] : -INFINITY;
      lv[j] = in ? pl[e] : 0.f;
      ov[j] = in ? po[e * D + dim] : 0.f;
    }
    float mn = M;
#pragma unroll
    for (int j = 0; j < NB; ++j) mn = fmaxf(mn, mv[j]);
    const float a = mn == M ? 1.f : __builtin_amdgcn_exp2f(M - mn);
    acc *= a;
    lsum *= a;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float w = mv[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv[j] - mn);
      acc = fmaf(w, ov[j], acc);
      lsum = fmaf(w, lv[j], lsum);
    }
    M = mn;
  }
  const float y = acc / lsum;
  const int64_t oo = ((int64_t)b * h_q + t) * D + dim;
  if constexpr (OUT_BF16) ((uint16_t*)o)[oo] = f32_to_bf16_bits(y);
  else ((float*)o)[oo] = y;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodeWsPtrs& w, hipStream_t st,
                         const CallEvents* ev) {
  const int g = a.h_q / a.h_kv;
  const int n_hb = (g + 15) / 16;
  const int n_split = decode_num_splits(a.kv_len, a.in_bf16);
  const KvRows kr{a.bt, a.ps_log2, a.max_pages, a.num_pages, a.cap};
  const void* q = a.q;
  int q_rotated = a.q_rotated;
  hipError_t err;
  if (a.k_new) {   // 0) append the new token; the query, rotated once, into the workspace
    if (ev) next_launch_events() = LaunchEvents{ev->call_start, ev->kernel_start};
    if (a.in_bf16)
      err = launch_kernel(decode_prep_kernel<uint16_t>, dim3((unsigned)a.B), dim3(256), st,
                          (const uint16_t*)a.q, (uint16_t*)w.qr, (const uint16_t*)a.k_new,
                          (const uint16_t*)a.v_new, (uint16_t*)a.kc, (uint16_t*)a.vc, a.h_q,
                          a.h_kv, a.d, a.append_end, a.qpos_arr, a.q_rotated, a.rp, kr);
    else
      err = launch_kernel(decode_prep_kernel<float>, dim3((unsigned)a.B), dim3(256), st,
                          (const float*)a.q, (float*)w.qr, (const float*)a.k_new,
                          (const float*)a.v_new, (float*)a.kc, (float*)a.vc, a.h_q, a.h_kv, a.d,
                          a.append_end, a.qpos_arr, a.q_rotated, a.rp, kr);
    if (err != hipSuccess) return err;
    q = w.qr;
    q_rotated = 1;
  }
  // 1) split-K streaming (bf16 with h_kv a multiple of 4: a workgroup per
  // four groups of a chunk)
  const bool grp4 = a.in_bf16 && a.h_kv % 4 == 0;
  dim3 grid((unsigned)n_split, (unsigned)((grp4 ? a.h_kv / 4 : a.h_kv) * n_hb), (unsigned)a.B);
  const float sl2 = a.scale * 1.4426950408889634f;
  if (ev) next_launch_events() = LaunchEvents{a.k_new ? nullptr : ev->kernel_start, ev->kernel_stop};
#define GQA_SPLIT(KERNEL, T, TPL, SC)                                                        \
  err = launch_kernel(KERNEL<TPL>, grid, dim3(256), st, (const T*)q, (const T*)a.kc,         \
                      (const T*)a.vc, w.m, w.l, w.o, a.h_q, a.h_kv, g, n_hb, (int)a.kv_len,  \
                      (double)a.q_pos, a.rp, SC, n_split, a.kvl_arr, a.qpos_arr,             \
                      a.kvl_from_pos, q_rotated, kr)
#define GQA_BF16(DD, PG)                                                             \
  do {                                                                               \
    if (grp4) GQA_SPLIT(decode_split_bf16_kernel, uint16_t, GQA_TPL3(DD, PG, true), sl2); \
    else GQA_SPLIT(decode_split_bf16_kernel, uint16_t, GQA_TPL3(DD, PG, false), sl2);     \
  } while (0)
#define GQA_TPL3(DD, PG, GR) DD, PG, GR
#define GQA_F32(DD, PG) GQA_SPLIT(decode_split_f32_kernel, float, GQA_TPL2(DD, PG), a.scale)
#define GQA_TPL2(DD, PG) DD, PG
  if (a.in_bf16) {
    if (a.d == 128) { if (a.bt) GQA_BF16(128, true); else GQA_BF16(128, false); }
    else { if (a.bt) GQA_BF16(64, true); else GQA_BF16(64, false); }
  } else {
    if (a.d == 128) { if (a.bt) GQA_F32(128, true); else GQA_F32(128, false); }
    else { if (a.bt) GQA_F32(64, true); else GQA_F32(64, false); }
  }
#undef GQA_TPL2
#undef GQA_F32
#undef GQA_TPL3
#undef GQA_BF16
#undef GQA_SPLIT
  if (err != hipSuccess) return err;
  // 2) merge of the chunks
  dim3 mgrid((unsigned)a.h_q, (unsigned)a.B);
  if (ev) next_launch_events() = LaunchEvents{nullptr, ev->call_stop};
#define GQA_MERGE(DD, OB)                                                                 \
  err = launch_kernel(decode_merge_kernel<DD, OB>, mgrid, dim3(DD), st, w.m, w.l, w.o, a.o, \
                      a.h_q, a.h_kv, g, n_split)
  if (a.d == 128) {
    if (a.out_bf16) GQA_MERGE(128, true); else GQA_MERGE(128, false);
  } else {
    if (a.out_bf16) GQA_MERGE(64, true); else GQA_MERGE(64, false);
  }
#undef GQA_MERGE
  return err;
}

}  // namespace gqa
