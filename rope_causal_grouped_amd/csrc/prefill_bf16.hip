// Causal GQA prefill on the matrix cores (gfx950) for bf16 inputs, RoPE
// fused into the Q load, fp32 accumulation, online softmax.
//
// What it computes (Qwen2 technical-report walkthrough, aicoding.csdn.net,
// §4.1.3 steps 3-4): for query head t and its KV group u = t / g,
//   O_t = softmax(Q'_t K'_u^T * scale + M) V_u,  M_ij = -inf for j > i,
// with Q', K' the rotated rows.  The same page notes the L x L score matrix
// need not be materialised (flash-style); this kernel keeps it in registers.
//
// Work split.  The g query heads of one KV group read the same K and V, so
// for a fixed (batch b, group u) the rows (position i, head t in the group)
// form one "stacked" query matrix of L*g rows, ordered position-major; that
// matrix is contiguous in q (the g heads of one position are adjacent).  A
// workgroup owns 256 consecutive stacked rows (about 256/g positions, all g
// heads) and streams the K/V tiles of group u through LDS once for all of
// them: the g-fold K/V reuse GQA offers (same page, closing note of §4.1.3).
// Eight waves own 32 rows each, two waves per SIMD.  Which row block a
// workgroup takes follows an XCD-aware order (each XCD works through a few
// groups, heaviest row blocks first) whose lightest items form per-XCD
// pools that faster XCDs may take over (see the work-item comment below).
//
// Per 64-key tile a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_f16
// (K from LDS as the A operand, the wave's rotated Q rows resident in VGPRs
// as the B operand), so each lane holds half of one query row's scores.  The
// rotated rows are rounded once to fp16 for this product: their 11-bit
// significand keeps the logits of large rows (the 32K workload's rows scaled
// by 8) within the bf16 tolerance, where bf16-rounded Q' and K' do not, at
// the same matrix-core rate.  Q' carries scale * log2(e), so scores come out
// in log2 units.  fp16 ends at 65504: a row whose Q' * scale * log2(e) has
// an element of magnitude 2^14 or more, and every row of a workgroup whose
// keys hold such a rotated K element (the preparation pass flags the tile),
// gets NaN operands and so NaN output; nothing is checked inside the loop.
// The probabilities, rounded to bf16, are already in the B-operand layout of
// O^T += V^T P^T on v_mfma_f32_32x32x16_bf16; V arrives pre-transposed (keys
// contiguous, in the accumulator's lane order) from the preparation pass, in
// 32-key sub-tiles.
//
// Ping-pong schedule.  Each wave alternates between a matrix phase (P.V of
// tile i-1, then S^T of tile i) and a vector phase (softmax of tile i).
// Waves 0-3 and waves 4-7 (one of each on every SIMD) run the two phases in
// opposite order and every phase ends at a workgroup barrier, so on each
// SIMD one wave's matrix-core work always runs against the other wave's
// softmax.  Both groups run one loop body (softmax of tile i-1, barrier,
// matrix phase i, barrier), one period apart.  A matrix phase reads 32
// operand fragments from LDS; they are issued a few MFMAs ahead of their use
// so that LDS latency stays hidden.
// The wave group in its vector phase also streams the next tile from HBM
// straight into LDS (global_load_lds_dwordx4, no staging registers): K by
// waves 4-7, V by waves 0-3, each into a two-slot ring.
// LDS rows are unpadded; the 16-byte chunk index is XOR-swizzled with the
// row index, which keeps the operand reads free of bank conflicts.
//
// Softmax without a per-tile max.  |q'| * max|k'| (Cauchy-Schwarz; max over
// the keys this workgroup visits, from the per-tile norms of the preparation
// pass) bounds every score of a row.  Once the row's reference m is within
// 64 (exp2 units) of that bound, probabilities are formed against m directly
// (<= 2^64, far inside fp32 and bf16 range) and the tile max is not needed;
// m is raised only if a tile's probability sum passes 2^32, which keeps O
// and l bounded.  A bound of at most 64 makes m = 0 valid from the start
// (scores lie in [-64, 64]: no probability overflows or underflows).
// Otherwise the tile max is taken first, until m is within reach of the
// bound, and m follows it lazily (raised when the max grows by more than
// 8); m then never exceeds the true running max by more than log2(64), so
// the largest probability cannot underflow.  While every row of a wave has
// m = 0 within its bound and owes no raise, a wave-uniform flag skips the
// per-tile checks altogether.
//
// Output.  O = O / l leaves in whole 128-byte pieces of rows with
// non-temporal stores: each wave turns its rows row-major through LDS the
// loop no longer reads, so O does not sit in the caches as partly written
// dirty lines that the next kernels would have to write back.

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int TK = 64;                      // keys per tile
constexpr int TV = kPrefillTileV;           // keys per prepared V^T sub-tile (32)
constexpr int NW = 8;                       // waves per workgroup
constexpr int RW = 32;                      // rows per wave
constexpr int PF = 4;                       // LDS operand reads kept ahead of the MFMAs
constexpr int kXcds = 8;                    // XCDs (each with its own L2) per MI355X
constexpr int kPoolStride = kPrefillPoolStride;   // ints between the per-XCD tail counters
static_assert(kPrefillPoolXcds == kXcds, "one shared-tail counter per XCD");
constexpr float kRescaleThreshold = 8.0f;   // log2 units, max-first path
constexpr float kBoundHeadroom = 64.0f;     // log2 units, bound-first path
constexpr float kSumCap = 4294967296.0f;    // 2^32

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int P>
using Slot = std::integral_constant<int, P % 2>;

__device__ __forceinline__ float bf16x8_sum(const bf16x8 v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
  return acc;
}

}  // namespace

// PRE: the kernel rotates Q itself (cs set); otherwise Q arrives rotated
// (bf16).  Either way scale * log2(e) is folded into Q' before its one fp16
// rounding; a probability is then a bare exp2 of the score while every row
// of the wave has m = 0, and exp2(s - m) otherwise.
template <int D, bool OUT_BF16, bool PRE>
__global__ __launch_bounds__(NW * 64, 1) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vt, const float* __restrict__ kmax,
    const int* __restrict__ kexp, const float2* __restrict__ cs, void* __restrict__ o, int L,
    int Lpad, int h_q, int h_kv,
    int g, int n_rb, int n_bu, float sl2, int causal, const int64_t* __restrict__ qstart,
    const int64_t* __restrict__ qlen, int kend, int* __restrict__ pool_ctr, int pool_t) {
  constexpr int NS = D / 16;                  // 16-dim k-steps of S^T
  constexpr int NDB = D / 32;                 // 32-dim blocks of O^T
  constexpr int NPV = 4 * NDB;                // P.V MFMAs per tile
  constexpr int NQK = 2 * NS;                 // S^T MFMAs per tile
  constexpr int NR = NPV + NQK;               // operand fragments per matrix phase
  constexpr int ROWS = NW * RW;
  // tile geometry in 16-byte chunks
  constexpr int KCPR = D / 8;                 // chunks per K row (16 for d = 128)
  constexpr int KRPB = KCPR >= 16 ? 1 : 16 / KCPR;   // K rows per 256 bytes
  constexpr int VCPR = TV / 8;                // chunks per V^T row (4)
  constexpr int VRPB = 16 / VCPR;             // V^T rows per 256 bytes
  constexpr int TILE_CH = TK * D / 8;         // chunks per K (or V^T) tile
  constexpr int LPG = TILE_CH / 64 / 4;       // direct loads per wave when 4 waves load a tile
  static_assert(LPG >= 1, "tile too small for the wave count");
  // two-slot rings for K and V^T tiles, one array per slot; the loop below
  // is unrolled by two, so every slot address is a compile-time constant
  // folded into the read instructions' offset fields
  __shared__ __attribute__((aligned(16))) uint16_t ks0[TK * D], ks1[TK * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs0[TK * D], vs1[TK * D];
  __shared__ float wred[NW];
  __shared__ int wexp[NW + 2];               // [NW], [NW + 1]: the shared-tail pick

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int grp = wave >> 2;                  // 0: matrix phase first; 1: vector phase first
  const int hl = lane >> 5, c32 = lane & 31;

  // Work items: row block rb of group bu = (b, u).  Workgroups are
  // dispatched to the eight XCDs round-robin by id, and each XCD has its own
  // L2.  Each group is cut into s strided parts, s = 8 / gcd(groups, 8), so
  // that the parts divide evenly among the XCDs: part r holds row blocks
  // n_rb-1-r, n_rb-1-r-s, ...  XCD x works through parts x*ppx ..
  // (x+1)*ppx-1 in turn: few groups at a time (their K/V stay in its L2),
  // the same share of the work on every XCD (causal row blocks differ in
  // cost), and within a part the heaviest row blocks (latest positions,
  // most keys) first.  Ids past an XCD's items exit at once.
  //
  // Shared tail (pool_t > 0): the last pool_t items of every XCD's list
  // (its lightest) become that XCD's pool, handed out through a
  // device-scope ticket counter per XCD to the workgroups with ids from the
  // XCD's own item count - pool_t on (each XCD also has pool_t extra ids).
  // Such a workgroup takes the next item of its own XCD's pool; once that
  // is empty it takes one from the pool with the most items left (read all
  // counters, then a ticket there; a few bounded retries if another
  // workgroup got there first), and it exits when every pool is empty.  The
  // XCDs do not all run at the same speed, so with a fixed split the faster
  // ones would idle at the end; this way they take over part of the slower
  // ones' tails, and most items still run where their K/V sit in L2.  The
  // counters (kPoolStride ints apart) are zeroed by the preparation kernel
  // that runs before this one.
  int xcd = (int)blockIdx.x % kXcds, j = (int)blockIdx.x / kXcds;
  const int low = n_bu & -n_bu;               // largest power of two dividing n_bu
  const int s_parts = low >= kXcds ? 1 : kXcds / low;
  const int ppx = n_bu * s_parts / kXcds;     // parts per XCD
  auto xcd_items = [&](int x) {
    int c = 0;
    for (int t = 0; t < ppx; ++t) c += (n_rb - (x * ppx + t) % s_parts + s_parts - 1) / s_parts;
    return c;
  };
  if (pool_t > 0 && j >= xcd_items(xcd) - pool_t) {
    if (tid == 0) {
      int sel = -1, tk = 0;
      int t = __hip_atomic_fetch_add(pool_ctr + xcd * kPoolStride, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      if (t < pool_t) {
        sel = xcd;
        tk = t;
      }
      for (int tries = 0; sel < 0 && tries < kXcds; ++tries) {
        int best = -1, left = 0;
        int cnt[kXcds];
#pragma unroll
        for (int y = 0; y < kXcds; ++y)
          cnt[y] = __hip_atomic_load(pool_ctr + y * kPoolStride, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int y = 0; y < kXcds; ++y)
          if (pool_t - cnt[y] > left) {
            left = pool_t - cnt[y];
            best = y;
          }
        if (best < 0) break;                    // every pool is empty
        t = __hip_atomic_fetch_add(pool_ctr + best * kPoolStride, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        if (t < pool_t) {
          sel = best;
          tk = t;
        }
      }
      wexp[NW] = sel;
      wexp[NW + 1] = tk;
    }
    __syncthreads();
    const int sel = wexp[NW];
    if (sel < 0) return;                        // no item left
    xcd = sel;
    j = xcd_items(sel) - pool_t + wexp[NW + 1];
  }
  int part = xcd * ppx, jj = j;
  for (int t = 0; t < ppx; ++t) {
    const int cnt = (n_rb - part % s_parts + s_parts - 1) / s_parts;
    if (jj < cnt) break;
    jj -= cnt;
    ++part;
  }
  if (part >= (xcd + 1) * ppx) return;
  const int bu = part / s_parts;
  const int rb = n_rb - 1 - part % s_parts - s_parts * jj;
  const int b = bu / h_kv, u = bu % h_kv;
  const int R0 = rb * ROWS;

  // Queries of sequence b: rows i < nq of q[b] (row stride L), at positions
  // qs + i.  qs = 0, nq = L for a whole prompt; with qstart set this is a
  // chunk whose keys 0 .. qs + nq - 1 were prepared from the cache (causal
  // only).  A sequence whose chunk is out of range gets NaN rows.
  int qs = 0, nq = L;
  if (qstart) {
    const int64_t s0 = qstart[b], n = qlen ? qlen[b] : L;
    if (!(s0 >= 0 && n >= 0 && n <= L && s0 + n <= kend)) {
      for (int e = tid; e < ROWS * D; e += NW * 64) {
        const int r = R0 + e / D;
        if (r < L * g) {
          const int64_t oo = ((int64_t)((int64_t)b * L + r / g) * h_q + u * g + r % g) * D + e % D;
          if constexpr (OUT_BF16) ((uint16_t*)o)[oo] = 0x7fc0u;
          else ((float*)o)[oo] = __builtin_nanf("");
        }
      }
      return;
    }
    qs = (int)s0;
    nq = (int)n;
  }
  const int nk = causal ? qs + nq : L;   // keys of the sequence
  const int rows_total = nq * g;
  if (R0 >= rows_total) return;          // the whole row block lies past this sequence's rows
  const int row = R0 + wave * RW + c32;
  const bool row_valid = row < rows_total;
  const int rr = row_valid ? row : rows_total - 1;
  const int pl = rr / g;                 // row of q / o
  const int pos = qs + pl;               // its position
  const int head = u * g + (rr - pl * g);

  // ---- key range
  const int rmax = min(R0 + ROWS - 1, rows_total - 1);
  const int n_keys = causal ? qs + rmax / g + 1 : L;
  const int n_tiles = (n_keys + TK - 1) / TK;
  const int wr0 = min(R0 + wave * RW, rows_total - 1);
  const int wr1 = min(R0 + wave * RW + RW - 1, rows_total - 1);
  const int wpos_lo = qs + wr0 / g, wpos_hi = qs + wr1 / g;
  const int lim = causal ? min(pos, nk - 1) : nk - 1;   // last key this row may see
  // tile i has keys this wave may see / needs the element mask
  auto active = [&](int i) { return !causal || i * TK <= wpos_hi; };
  auto masked = [&](int i) { return (causal && i * TK + TK - 1 > wpos_lo) || (i * TK + TK > nk); };

  // ---- direct HBM -> LDS tile loads by one wave group.  Instruction n of
  // wave w (of the group) fills LDS chunks [(w*LPG + n)*64, +64); lane l's
  // chunk P sits at row P / CPR, physical slot P % CPR, and holds logical
  // chunk slot ^ swizzle(row).  Waves 4-7 load K, waves 0-3 load V.
  const int wg4 = wave & 3;
  const uint16_t* src = (grp ? kp : vt) + (int64_t)bu * Lpad * D;
  int loff[LPG];
#pragma unroll
  for (int n = 0; n < LPG; ++n) {
    const int P = (wg4 * LPG + n) * 64 + lane;
    if (grp) {
      const int kr = P / KCPR, kslot = P % KCPR;
      loff[n] = (kr * D + ((kslot ^ ((kr / KRPB) % KCPR)) * 8)) * 2;   // bytes
    } else {
      const int sub = P / (D * VCPR), rem = P % (D * VCPR);
      const int vr = rem / VCPR, vslot = rem % VCPR;
      loff[n] = (sub * D * TV + vr * TV + ((vslot ^ ((vr / VRPB) % VCPR)) * 8)) * 2;
    }
  }
  // the lane's byte offset as a 32-bit value at the load, so that the load
  // takes the uniform tile base in scalar registers (no 64-bit vector add)
  auto lane_off = [](int v) __attribute__((always_inline)) {
    uint32_t u = (uint32_t)v;
    asm volatile("" : "+v"(u));
    return u;
  };
  auto load_tile = [&](uint16_t* ring, int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < LPG; ++n)
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)((const char*)(src + (int64_t)tile * TK * D) +
                                                          lane_off(loff[n])),
          (void __attribute__((address_space(3)))*)&ring[(wg4 * LPG + n) * 64 * 8], 16, 0, 0);
  };
  auto kslot = [&](auto P) -> uint16_t* {
    if constexpr (decltype(P)::value == 0) return ks0;
    else return ks1;
  };
  auto vslot = [&](auto P) -> uint16_t* {
    if constexpr (decltype(P)::value == 0) return vs0;
    else return vs1;
  };
  // Workgroup barrier.  Its release fence makes every LDS write of the
  // wave visible first, the direct tile loads included (the compiler waits
  // for all loads in flight), so a tile issued in a period has landed when
  // that period ends.  Letting the loads stay in flight across the barrier
  // (a bare s_barrier with explicit waits for older tiles) measured slower.
  auto bar = [] { __syncthreads(); };

  // ---- prologue part 1.  Global reads in the order they are needed (the
  // vector-memory counter retires them in order): per-tile K norms, the Q
  // row and its cos/sin, then the first tiles straight into LDS.
  const int n = n_tiles;
  const float* kmax_bu = kmax + (int64_t)bu * (Lpad / TK);
  const int* kexp_bu = kexp + (int64_t)bu * (Lpad / TK);
  float km = tid < n_tiles ? kmax_bu[tid] : 0.f;
  int kx = tid < n_tiles ? kexp_bu[tid] : 0;
  const uint16_t* qrow = q + ((int64_t)((int64_t)b * L + pl) * h_q + head) * D;
  u32x4 raw[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) raw[s] = *(const u32x4*)(qrow + s * 16 + hl * 8);
  f32x4 c4[NS / 2][4];   // PRE: cos/sin of the row's position, two pairs per load
  if constexpr (PRE) {
    const float4* csr = (const float4*)(cs + (int64_t)pos * (D / 2) + hl * 8);
#pragma unroll
    for (int s = 0; s < NS / 2; ++s)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float4 t = csr[s * 8 + e2];
        c4[s][e2] = f32x4{t.x, t.y, t.z, t.w};
      }
  }
  // K(0) by waves 4-7 (the first barrier publishes it)
  if (grp) load_tile(ks0, 0);

  // ---- Q row: rotate at pos, fold in scale * log2(e), divide by 2^eq when
  // the row's largest element reaches 2^14, round to fp16 (B operand
  // layout: lane holds dims s*16 + hl*8 + e of its row; RoPE pairs are
  // (s, s + NS/2)); done after the first barrier, when its reads have long
  // arrived.
  f16x8 qb[NS];
  float qcap;      // bound on |q'| in score units, with a margin for rounding
  bool qbad;       // this row's Q' is outside the fp16 operand range
  auto rotate_q = [&]() __attribute__((always_inline)) {
    float amax = 0.f, ss = 0.f;
    auto put = [&](int s, int e, float y) {
      const _Float16 h = (_Float16)y;
      qb[s][e] = h;
      amax = fmaxf(amax, fabsf(y));
      ss = fmaf((float)h, (float)h, ss);
    };
    auto bf = [](uint32_t w, int e) {
      return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    };
    if constexpr (PRE) {
#pragma unroll
      for (int s = 0; s < NS / 2; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float cr = c4[s][e >> 1][(e & 1) * 2], sr = c4[s][e >> 1][(e & 1) * 2 + 1];
          const float x1 = bf(raw[s][e >> 1], e), x2 = bf(raw[s + NS / 2][e >> 1], e);
          put(s, e, fmaf(x1, cr, -x2 * sr) * sl2);
          put(s + NS / 2, e, fmaf(x2, cr, x1 * sr) * sl2);
        }
      }
    } else {   // rotated already
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) put(s, e, bf(raw[s][e >> 1], e) * sl2);
    }
    qbad = kexp_of(max_xor32(amax)) != 0;
    // |q'| of the row from the fp16 values the matrix cores see
    qcap = sqrtf(sum_xor32(ss)) * 1.01f;
  };

  // ---- operand read offsets (elements), swizzled like the stores
  const int kswz = (c32 / KRPB) % KCPR;       // same for key rows c32 and 32 + c32
  int kread[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) kread[s] = (c32 * D + (((2 * s + hl) ^ kswz) * 8)) * 2;   // bytes
  const int vswz = (c32 / VRPB) % VCPR;       // same for dim rows db*32 + c32
  int vread[2];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) vread[hs] = (c32 * TV + (((2 * hs + hl) ^ vswz) * 8)) * 2;

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const f32x16 zero16 = {};
  f32x16 sacc[2];     // scores of the tile between its matrix and vector phases
  bf16x8 pb[2][2];    // probabilities between the vector and the next matrix phase
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    sacc[kb] = zero16;
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[kb][hs][e] = (__bf16)0.0f;
  }

  // ---- matrix phases.  Fragment j < NPV is V^T block (kb, hs, db) with
  // j = (kb*2 + hs)*NDB + db; fragment NPV + 2s + c is K rows c*32.. at
  // k-step s.  All reads and MFMAs sit in one basic block; the scheduling
  // barriers issue the reads PF fragments ahead of their MFMAs.
  // Lane offsets are in bytes, so that slot base and fragment offset fold
  // into the instruction's offset field.
  auto read_v = [&](const uint16_t* vt0, const int (&vr)[2], int j) {
    const int kb = j / (2 * NDB), hs = (j / NDB) % 2, db = j % NDB;
    return *(const bf16x8*)((const char*)vt0 + (kb * D * TV + db * 32 * TV) * 2 + vr[hs]);
  };
  auto read_k = [&](const uint16_t* kt0, const int (&kr)[NS], int j) {
    const int s = j / 2, c = j % 2;
    return __builtin_bit_cast(bf16x8,
                              *(const f16x8*)((const char*)kt0 + c * 32 * D * 2 + kr[s]));
  };
  auto mma_pv = [&](const bf16x8 a, int j) {
    const int kb = j / (2 * NDB), hs = (j / NDB) % 2, db = j % NDB;
    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][hs], oacc[db], 0, 0, 0);
  };
  auto mma_qk = [&](const bf16x8 a, int j) {   // a: an fp16 K' fragment (16 bytes)
    const int s = j / 2, c = j % 2;
    sacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
        __builtin_bit_cast(f16x8, a), qb[s], s == 0 ? zero16 : sacc[c], 0, 0, 0);
  };
  // P.V of tile i-1 and S^T of tile i (P = i mod 2)
  auto matrix_full = [&](auto P) __attribute__((always_inline)) {
    const uint16_t* vt0 = vslot(Slot<decltype(P)::value + 1>{});
    const uint16_t* kt0 = kslot(P);
    bf16x8 fr[NR];
#pragma unroll
    for (int j = 0; j < NPV; ++j) fr[j] = read_v(vt0, vread, j);
#pragma unroll
    for (int j = 0; j < NQK; ++j) fr[NPV + j] = read_k(kt0, kread, j);
#pragma unroll
    for (int j = 0; j < NPV; ++j) mma_pv(fr[j], j);
#pragma unroll
    for (int j = 0; j < NQK; ++j) mma_qk(fr[NPV + j], j);
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int j = 0; j < NR - PF; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
    __builtin_amdgcn_sched_barrier(0);   // the MFMAs stay in this phase
  };
  // S^T of tile 0 only
  auto matrix_qk = [&]() __attribute__((always_inline)) {
    const uint16_t* kt0 = ks0;
    bf16x8 fr[NQK];
#pragma unroll
    for (int j = 0; j < NQK; ++j) fr[j] = read_k(kt0, kread, j);
#pragma unroll
    for (int j = 0; j < NQK; ++j) mma_qk(fr[j], j);
  };
  // P.V of the last tile only (tile i - 1, slot (i - 1) mod 2)
  auto matrix_pv = [&](int i) __attribute__((always_inline)) {
    const uint16_t* vt0 = (i - 1) % 2 == 0 ? vs0 : vs1;
    bf16x8 fr[NPV];
#pragma unroll
    for (int j = 0; j < NPV; ++j) fr[j] = read_v(vt0, vread, j);
#pragma unroll
    for (int j = 0; j < NPV; ++j) mma_pv(fr[j], j);
  };

  // ---- vector phase i: probabilities of tile i into pb, row sums into l
  auto rescale = [&](float m_new) __attribute__((always_inline)) {
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
  };
  // SH: the reference m of some row in the wave is not 0
  auto probs = [&](const f32x16& s0, const f32x16& s1, auto SH) __attribute__((always_inline)) {
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if constexpr (!decltype(SH)::value) {
        pb[0][e >> 3][e & 7] = (__bf16)__builtin_amdgcn_exp2f(s0[e]);
        pb[1][e >> 3][e & 7] = (__bf16)__builtin_amdgcn_exp2f(s1[e]);
      } else {
        pb[0][e >> 3][e & 7] = (__bf16)__builtin_amdgcn_exp2f(s0[e] - m_run);
        pb[1][e >> 3][e & 7] = (__bf16)__builtin_amdgcn_exp2f(s1[e] - m_run);
      }
    }
    acc0 = bf16x8_sum(pb[0][0], acc0);
    acc1 = bf16x8_sum(pb[0][1], acc1);
    acc0 = bf16x8_sum(pb[1][0], acc0);
    acc1 = bf16x8_sum(pb[1][1], acc1);
    return acc0 + acc1;
  };
  float crow = 0.f;   // bound on this row's scores, score units (set after the prologue)
  float m_raise = 0.f;  // raise of m owed by the previous tile's large sum (applied lazily)
  // fast: every row of the wave has m = 0 within reach of its bound and no
  // raise owed, so a tile needs neither its max nor a rescale; wave-uniform,
  // recomputed only when a tile leaves that state
  bool fast = false;
  auto vector_phase = [&](int i) __attribute__((always_inline)) {
    if (!active(i)) {   // keys beyond this wave's rows: contribute nothing
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[kb][hs][e] = (__bf16)0.0f;
      return;
    }
    // (no AGPR constraint anywhere in this kernel: at two waves per SIMD the
    // compiler then keeps every MFMA accumulator in VGPRs, and the vector
    // ALU reads the scores without copies)
    f32x16 s0 = sacc[0], s1 = sacc[1];
    if (masked(i)) {
      // key of score e: i*TK + (e>>2)*8 + hl*4 + (e&3) (+32 for s1); compared
      // as a constant offset against the row's limit within the tile
      const int t = lim - i * TK - hl * 4;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = (e >> 2) * 8 + (e & 3);
        if (c > t) s0[e] = -INFINITY;
        if (c + 32 > t) s1[e] = -INFINITY;
      }
    }
    // new reference: the owed raise (O and l already hold the tile that
    // caused it), or the tile max while the bound is not yet usable
    const bool was_fast = fast;
    float m_new = m_run + m_raise;
    if (!was_fast && __builtin_amdgcn_ballot_w64(crow > m_run + kBoundHeadroom)) {   // max first
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, fmaxf(s0[e], s1[e]));
      mx = max_xor32(mx);
      if (mx > m_new + kRescaleThreshold) m_new = mx;
    }
    if (!was_fast && __builtin_amdgcn_ballot_w64(m_new != m_run)) rescale(m_new);
    float psum;
    if (!was_fast && __builtin_amdgcn_ballot_w64(m_run != 0.f))
      psum = probs(s0, s1, std::true_type{});
    else
      psum = probs(s0, s1, std::false_type{});
    l_run += psum;
    // probabilities here are <= 2^64; a sum past 2^32 owes a raise of m by
    // its (integral) log2, taken at the next tile once P.V has added it
    m_raise = 0.f;
    if (__builtin_amdgcn_ballot_w64(psum > kSumCap)) {
      m_raise = ceilf(__builtin_amdgcn_logf(fmaxf(max_xor32(psum), 1.0f)));
      fast = false;
    } else if (!was_fast) {
      fast = __builtin_amdgcn_ballot_w64(m_run != 0.f || crow > m_run + kBoundHeadroom) == 0;
    }
  };

  // ---- prologue part 2: largest K norm this workgroup will see (per-tile
  // norms from the preparation pass; more than one per thread only past
  // 32768 keys); K(0) resident, bound known
  for (int t = tid + NW * 64; t < n_tiles; t += NW * 64) {
    km = fmaxf(km, kmax_bu[t]);
    kx = max(kx, kexp_bu[t]);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) km = wave_max_xor(km, m);
  if (__builtin_amdgcn_ballot_w64(kx != 0) != 0 && lane == 0) wexp[wave] = 1;
  else if (lane == 0) wexp[wave] = 0;
  if (lane == 0) wred[wave] = km;
  bar();
  rotate_q();
  {
    float km = wred[0];
    int any = wexp[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      km = fmaxf(km, wred[w]);
      any |= wexp[w];
    }
    crow = qcap * km;
    if (qbad || any != 0) {   // outside the fp16 operand range: NaN scores, NaN row
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[s][e] = (_Float16)__builtin_nanf("");
    }
  }
  // a bound within the headroom makes 0 a valid reference from the start
  // (every score lies in [-crow, crow]), which the scores need no shift for
  if (crow <= kBoundHeadroom) m_run = 0.f;
  fast = __builtin_amdgcn_ballot_w64(crow > kBoundHeadroom) == 0;

  // ---- periods t = 0 .. 2 n_tiles + 1, each but the last ending at a
  // barrier.  Even period 2i: waves 0-3 run matrix phase i (V(i-1), K(i)),
  // waves 4-7 vector phase i-1 and load K(i+1).  Odd period 2i+1: waves 0-3
  // run vector phase i and load V(i), waves 4-7 matrix phase i.  Tile t sits
  // in slot t % 2; a load overwrites the tile read two periods before and
  // has landed at the barrier that ends its period (past the last tile,
  // waves 4-7 load the last K again, into the slot nobody reads any more).
  // The loop runs i = 1 .. n-1 unrolled by two, so every slot is static.
  auto step = [&](auto P, int i) __attribute__((always_inline)) {         // P = i mod 2
    // period 2i-1 (waves 0-3) or 2i (waves 4-7): slot (i-1) mod 2 takes V(i-1)
    // or K(i+1), read by the other group's matrix phase of the next period
    constexpr int Q = decltype(P)::value + 1;
    load_tile(grp ? kslot(Slot<Q>{}) : vslot(Slot<Q>{}), grp ? min(i + 1, n - 1) : i - 1);
    vector_phase(i - 1);
    bar();
    matrix_full(P);                        // period 2i (waves 0-3) or 2i+1
    bar();
  };
  if (grp == 0) {
    matrix_qk();                            // period 0
    bar();
  } else {
    load_tile(ks1, min(1, n - 1));          // period 0
    bar();
    matrix_qk();                            // period 1
    bar();
  }
  {
    int i = 1;
    for (; i + 1 < n; i += 2) {
      step(Slot<1>{}, i);
      step(Slot<0>{}, i + 1);
    }
    if (i < n) step(Slot<1>{}, i);
  }
  if (grp == 0) {
    load_tile(n % 2 == 1 ? vs0 : vs1, n - 1);   // period 2n-1
    vector_phase(n - 1);
    bar();
    matrix_pv(n);                           // period 2n
    bar();
    // period 2n+1: this group's O is final; it is written below while
    // waves 4-7 run the last P.V (no barrier: nothing writes LDS any more)
  } else {
    vector_phase(n - 1);                    // period 2n
    bar();
    matrix_pv(n);                           // period 2n+1
  }

  // ---- epilogue: O = O / l; lane holds dims db*32 + gq*8 + hl*4 + (0..3).
  // O goes out in whole 128-byte pieces of rows with non-temporal stores (so
  // it does not linger in the caches as dirty lines for the next kernel to
  // write back): the wave's 32 rows are turned row-major, 128 bytes of each
  // row at a time (32 dims in fp32, 64 in bf16), through a quarter of a
  // tile slot that nothing reads any more (K slot 0 for waves 0-3; for waves
  // 4-7 the V slot their last P.V does not read), RP rows per pass, with the
  // 16-byte chunks of a row XOR-swizzled by the row.
  const float inv = 1.0f / sum_xor32(l_run);
  {
    constexpr int SB = TK * D / 2;          // bytes per wave: a quarter of a slot
    constexpr int RP = SB / 128;            // rows per pass (32 for d = 128, 16 for d = 64)
    constexpr int NPASS = RW / RP;
    constexpr int TPL = RP / 8;             // chunks per lane per pass
    constexpr int DPB = OUT_BF16 ? 64 : 32; // dims per 128-byte piece
    constexpr int EB = OUT_BF16 ? 2 : 4;    // bytes per element
    char* stage = (grp == 0 ? (char*)ks0 : (char*)(n % 2 == 0 ? vs0 : vs1)) + (wave & 3) * SB;
    int64_t orow_t[NPASS][TPL];
    bool ok_t[NPASS][TPL];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
      for (int t = 0; t < TPL; ++t) {   // row ps*RP + lane/8 + 8t of the wave
        const int r = R0 + wave * RW + ps * RP + lane / 8 + 8 * t;
        ok_t[ps][t] = r < rows_total;
        const int rr = ok_t[ps][t] ? r : 0;
        orow_t[ps][t] = ((int64_t)((int64_t)b * L + rr / g) * h_q + u * g + rr % g) * D;
      }
#pragma unroll
    for (int pc = 0; pc < D / DPB; ++pc)
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
        if (c32 / RP == ps) {
          char* srow = stage + (c32 % RP) * 128;
#pragma unroll
          for (int db2 = 0; db2 < DPB / 32; ++db2) {
            const int db = pc * (DPB / 32) + db2;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              // bytes (db2*32 + gq*8 + hl*4) * EB of the row's piece
              const int byte = (db2 * 32 + gq * 8 + hl * 4) * EB;
              char* dst = srow + (((byte >> 4) ^ (c32 & 7)) << 4) + (byte & 15);
              const float y0 = oacc[db][gq * 4 + 0] * inv, y1 = oacc[db][gq * 4 + 1] * inv;
              const float y2 = oacc[db][gq * 4 + 2] * inv, y3 = oacc[db][gq * 4 + 3] * inv;
              if constexpr (OUT_BF16) {
                u32x2 w;
                w[0] = (uint32_t)f32_to_bf16_bits(y0) | ((uint32_t)f32_to_bf16_bits(y1) << 16);
                w[1] = (uint32_t)f32_to_bf16_bits(y2) | ((uint32_t)f32_to_bf16_bits(y3) << 16);
                *(u32x2*)dst = w;
              } else {
                *(f32x4*)dst = f32x4{y0, y1, y2, y3};
              }
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int t = 0; t < TPL; ++t) {
          const int r = lane / 8 + 8 * t, c = lane % 8;
          const u32x4 w = *(const u32x4*)(stage + r * 128 + ((c ^ (r & 7)) << 4));
          if (ok_t[ps][t])
            __builtin_nontemporal_store(
                w, (u32x4*)((char*)o + (orow_t[ps][t] + pc * DPB) * EB + c * 16));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();   // reads done before the next writes
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
  }
}

hipError_t launch_prefill_bf16(const uint16_t* q, const uint16_t* kp, const uint16_t* vt,
                               const float* kmax, const int* kexp, const float2* cs, void* o,
                               int out_bf16,
                               int64_t B, int64_t L, int64_t Lpad, int h_q, int h_kv, int d,
                               float scale, int causal, const int64_t* qstart,
                               const int64_t* qlen, int64_t kend, int* pool_ctr,
                               hipStream_t st) {
  const int g = h_q / h_kv;
  const int n_rb = (int)((L * g + kPrefillRowsWG - 1) / kPrefillRowsWG);
  const int n_bu = (int)(B * h_kv);
  const float sl2 = scale * 1.4426950408889634f;  // scale * log2(e): exp(x) = exp2(x log2 e)
  // XCD-balanced work order (see the kernel): s strided parts per group
  const int low = n_bu & -n_bu;
  const int s_parts = low >= kXcds ? 1 : kXcds / low;
  const int ppx = n_bu * s_parts / kXcds;
  // shared tail: a quarter of the smallest XCD share, at most 64 items per
  // XCD, and as many extra ids per XCD (56 / 64 / 64 items per XCD at 7B
  // L4096 / 72B L8192 / 7B L32768; measured against 28-32 and 224: the
  // small pools leave most of the tail at the longer shapes, the large one
  // loses it again to the tickets and to the extra ids that exit)
  // Only a causal whole prompt gets one: its row blocks range from one tile
  // to all of them, while a chunk's (or a full mask's) are alike, and
  // moving those off their XCD's L2 cost 4% on the 7B chunk.
  const int min_items = ppx * (n_rb / s_parts);
  const int pool_t = pool_ctr && causal && !qstart ? std::min(64, min_items / 4) : 0;
  const unsigned grid =
      (unsigned)((int64_t)kXcds * (ppx * ((n_rb + s_parts - 1) / s_parts) + pool_t));
  hipError_t e;
#define GQA_LAUNCH(DD, OB, PR)                                                               \
  e = launch_kernel(prefill_bf16_kernel<DD, OB, PR>, dim3(grid), dim3(NW * 64), st, q, kp, vt, \
                    kmax, kexp, cs, o, (int)L, (int)Lpad, h_q, h_kv, g, n_rb, n_bu, sl2,       \
                    causal, qstart, qlen, (int)kend, pool_ctr, pool_t)
#define GQA_LAUNCH_D(DD, OB) \
  do { if (cs) GQA_LAUNCH(DD, OB, true); else GQA_LAUNCH(DD, OB, false); } while (0)
  if (d == 128) {
    if (out_bf16) GQA_LAUNCH_D(128, true); else GQA_LAUNCH_D(128, false);
  } else {
    if (out_bf16) GQA_LAUNCH_D(64, true); else GQA_LAUNCH_D(64, false);
  }
#undef GQA_LAUNCH_D
#undef GQA_LAUNCH
  return e;
}

}  // namespace gqa
