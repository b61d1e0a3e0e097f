// Causal GQA prefill on bf16 matrix cores (gfx950), RoPE fused into the Q
// load, fp32 accumulation, online softmax.
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
// workgroup owns 128 consecutive stacked rows (about 128/g positions, all g
// heads) and streams the K/V tiles of group u through LDS once for all of
// them: the g-fold K/V reuse GQA offers (same page, closing note of §4.1.3).
// Its four waves own 32 rows each.  Two workgroups share a CU, so the two
// waves on each SIMD come from different workgroups, are not tied by a
// common barrier, and overlap one's matrix-core phase with the other's
// softmax.
//
// Per 64-key tile a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (K from LDS as the A operand, the wave's rotated Q rows resident in VGPRs
// as the B operand), so each lane holds one query row's scores and the row
// max needs one exchange with lane ^ 32.  The probabilities, rounded to
// bf16, are already in the B-operand layout of O^T += V^T P^T; V arrives
// pre-transposed (keys contiguous, in the accumulator's lane order) from the
// preparation pass, in 32-key sub-tiles.
//
// K and V^T tiles go from HBM straight into LDS (global_load_lds_dwordx4,
// no staging registers).  That instruction writes 16 bytes per lane at
// consecutive LDS addresses, so the tiles are stored unpadded and bank
// conflicts are avoided instead by XOR-swizzling the 16-byte chunk index of
// each row with bits of the row index; the operand reads apply the same
// swizzle.
//
// The running max is raised only when a row's max grows by more than 2^8
// (exp2 units): probabilities then stay <= 256, exact enough in bf16 and far
// from fp32 overflow, and the O rescale is skipped on almost every tile.
// Waiting for a tile's max before the exponentials would serialise each
// tile, so on the common path the probabilities are formed against the
// running max straight away; that is safe when |q'| * max|k'| over the tile
// (the preparation pass stores max|k'| per 64-key tile) is within 2^64 of
// the running max.  The tile max is then taken alongside P.V, and if it
// grew past the threshold, O and l (which already hold this tile) are
// rescaled together.  The first tile, the diagonal (masked) tiles and tiles
// that fail the bound take the max-first path.

#include "common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int TK = 64;                      // keys per tile
constexpr int TV = kPrefillTileV;           // keys per prepared V^T sub-tile (32)
constexpr int NW = 4;                       // waves per workgroup
constexpr int RW = 32;                      // rows per wave
constexpr float kRescaleThreshold = 8.0f;   // log2 units
constexpr float kStaleMaxHeadroom = 64.0f;  // log2 units: p <= 2^64 against a stale max

}  // namespace

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64, 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vt, const float* __restrict__ kmax,
    const float2* __restrict__ cs, void* __restrict__ o, int L,
    int Lpad, int h_q, int h_kv, int g, int n_rb, int n_bu, float sl2, int causal) {
  constexpr int NS = D / 16;                  // 16-dim k-steps of S^T
  constexpr int NDB = D / 32;                 // 32-dim blocks of O^T
  constexpr int ROWS = NW * RW;
  // tile geometry in 16-byte chunks
  constexpr int KCPR = D / 8;                 // chunks per K row (16 for d = 128)
  constexpr int KRPB = KCPR >= 16 ? 1 : 16 / KCPR;   // K rows per 256 bytes
  constexpr int VCPR = TV / 8;                // chunks per V^T row (4)
  constexpr int VRPB = 16 / VCPR;             // V^T rows per 256 bytes
  constexpr int TILE_CH = TK * D / 8;         // chunks per K (or V^T) tile
  constexpr int LPW = TILE_CH / 64 / NW;      // direct loads per wave per tile and tensor
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][TK * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][TK * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, c32 = lane & 31;

  // Heaviest row blocks (latest positions, most keys) are dispatched first.
  const int id = blockIdx.x;
  const int rb = n_rb - 1 - id / n_bu;
  const int bu = id % n_bu;
  const int b = bu / h_kv, u = bu % h_kv;

  const int rows_total = L * g;
  const int R0 = rb * ROWS;
  const int row = R0 + wave * RW + c32;
  const bool row_valid = row < rows_total;
  const int rr = row_valid ? row : rows_total - 1;
  const int pos = rr / g;
  const int head = u * g + (rr - pos * g);

  // ---- Q row: load, rotate at pos, round to bf16 (B operand layout: lane
  // holds dims s*16 + hl*8 + e of its row; RoPE pairs are (s, s + NS/2)).
  bf16x8 qb[NS];
  {
    const uint16_t* qrow = q + ((int64_t)((int64_t)b * L + pos) * h_q + head) * D;
    u32x4 raw[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) raw[s] = *(const u32x4*)(qrow + s * 16 + hl * 8);
    const float2* csr = cs + (int64_t)pos * (D / 2) + hl * 8;
#pragma unroll
    for (int s = 0; s < NS / 2; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 r2 = csr[s * 16 + e];
        const uint32_t w1 = raw[s][e >> 1], w2 = raw[s + NS / 2][e >> 1];
        const float x1 = (e & 1) ? __uint_as_float(w1 & 0xffff0000u) : __uint_as_float(w1 << 16);
        const float x2 = (e & 1) ? __uint_as_float(w2 & 0xffff0000u) : __uint_as_float(w2 << 16);
        qb[s][e] = (__bf16)fmaf(x1, r2.x, -x2 * r2.y);
        qb[s + NS / 2][e] = (__bf16)fmaf(x2, r2.x, x1 * r2.y);
      }
    }
  }
  // |q'| of the row (from the bf16 values the matrix cores see), times the
  // score scale: |q'| * max|k'| bounds every score of a tile (Cauchy-Schwarz;
  // the rotation keeps norms), with a small margin for fp32 rounding
  float qcap;
  {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)qb[s][e];
        ss = fmaf(x, x, ss);
      }
    qcap = sqrtf(sum_xor32(ss)) * sl2 * 1.01f;
  }
  const float* kmax_bu = kmax + (int64_t)bu * (Lpad / TK);

  // ---- key range
  const int rmax = min(R0 + ROWS - 1, rows_total - 1);
  const int n_keys = causal ? rmax / g + 1 : L;
  const int n_tiles = (n_keys + TK - 1) / TK;
  const int wr0 = min(R0 + wave * RW, rows_total - 1);
  const int wr1 = min(R0 + wave * RW + RW - 1, rows_total - 1);
  const int wpos_lo = wr0 / g, wpos_hi = wr1 / g;
  const int lim = causal ? min(pos, L - 1) : L - 1;   // last key this row may see

  // ---- direct HBM -> LDS tile loads.  Instruction i of wave w fills LDS
  // chunks [(w*LPW + i)*64, +64); lane l's chunk P sits at row P / CPR,
  // physical slot P % CPR, and holds logical chunk slot ^ swizzle(row).
  const uint16_t* kbase = kp + (int64_t)bu * Lpad * D;
  const uint16_t* vbase = vt + (int64_t)bu * Lpad * D;
  int koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int P = (wave * LPW + i) * 64 + lane;
    const int kr = P / KCPR, kslot = P % KCPR;
    koff[i] = kr * D + ((kslot ^ ((kr / KRPB) % KCPR)) * 8);
    const int sub = P / (D * VCPR), rem = P % (D * VCPR);
    const int vr = rem / VCPR, vslot = rem % VCPR;
    voff[i] = sub * D * TV + vr * TV + ((vslot ^ ((vr / VRPB) % VCPR)) * 8);
  }
  // load n of the 2*LPW direct loads a wave issues per tile (K first, then V)
  auto issue_one = [&](int n, int tile, int buf) {
    const int i = n % LPW;
    const int dst = (wave * LPW + i) * 64 * 8;
    if (n < LPW)
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(kbase + (int64_t)tile * TK * D + koff[i]),
          (void __attribute__((address_space(3)))*)&ks[buf][dst], 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(vbase + (int64_t)tile * TK * D + voff[i]),
          (void __attribute__((address_space(3)))*)&vs[buf][dst], 16, 0, 0);
  };
  auto issue_tile = [&](int tile, int buf) {
#pragma unroll
    for (int n = 0; n < 2 * LPW; ++n) issue_one(n, tile, buf);
  };
  auto tile_landed = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // next tile to prefetch; past the last tile the last one is loaded again
  // into the idle buffer (harmless), which keeps the loop body uniform
  auto next_tile = [&](int kt) { return min(kt + 1, n_tiles - 1); };

  // ---- operand read offsets (elements), swizzled like the stores
  const int kswz = (c32 / KRPB) % KCPR;       // same for key rows c32 and 32 + c32
  int kread[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) kread[s] = c32 * D + (((2 * s + hl) ^ kswz) * 8);
  const int vswz = (c32 / VRPB) % VCPR;       // same for dim rows db*32 + c32
  int vread[2];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) vread[hs] = c32 * TV + (((2 * hs + hl) ^ vswz) * 8);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // S^T = K Q^T for two 32-key blocks (independent MFMA chains)
  auto qk = [&](f32x16 (&sacc)[2], int buf) {
    const uint16_t* kt0 = ks[buf];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 a0 = *(const bf16x8*)(kt0 + kread[s]);
      const bf16x8 a1 = *(const bf16x8*)(kt0 + 32 * D + kread[s]);
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qb[s], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qb[s], sacc[1], 0, 0, 0);
    }
  };
  // row max of a tile's scores (exp2 units)
  auto tile_max = [&](const f32x16 (&sacc)[2]) {
    float mx = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(sacc[0][i], sacc[1][i]));
    return max_xor32(mx) * sl2;
  };
  auto rescale = [&](float mx) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      // keep the accumulators in AGPRs outside this rare branch
      asm volatile("" : "+a"(oacc[db]));
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      asm volatile("" : "+a"(oacc[db]));
    }
  };
  // probabilities against the running max (bf16, B operand of P.V); returns
  // their fp32 sum
  auto probs = [&](const f32x16 (&sacc)[2], bf16x8 (&pb)[2][2]) {
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], sl2, -m_run));
        pb[kb][i >> 3][i & 7] = (__bf16)p;
        psum += p;
      }
    return psum;
  };
  // O^T += V^T P^T: per 16-key step, one MFMA per 32-dim block
  auto pv = [&](const bf16x8 (&pb)[2][2], int buf) {
    const uint16_t* vt0 = vs[buf];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 a = *(const bf16x8*)(vt0 + kb * D * TV + db * 32 * TV + vread[hs]);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][hs], oacc[db], 0, 0, 0);
        }
  };

  issue_tile(0, 0);
  tile_landed();
  __syncthreads();

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    const int k0 = kt * TK;
    issue_tile(next_tile(kt), buf ^ 1);
    if (!causal || k0 <= wpos_hi) {
      const bool masked = (causal && k0 + TK - 1 > wpos_lo) || (k0 + TK > L);
      // fast path: no mask on this tile and every score provably within the
      // headroom of the running max, so P can be formed before the tile max
      const bool fast = !masked && !__builtin_amdgcn_ballot_w64(
                                       qcap * kmax_bu[kt] > m_run + kStaleMaxHeadroom);
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
      qk(sacc, buf);
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
            if (key > lim) sacc[kb][i] = -INFINITY;
          }
      }
      if (!fast) {   // max first
        const float mx = tile_max(sacc);
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleThreshold)) rescale(mx);
      }
      bf16x8 pb[2][2];
      l_run += probs(sacc, pb);
      pv(pb, buf);
      if (fast) {    // the tile max off the critical path; rescale what holds it
        const float mx = tile_max(sacc);
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleThreshold)) rescale(mx);
      }
    }
    tile_landed();
    __syncthreads();
  }

  // ---- epilogue: O = O / l; lane holds dims db*32 + grp*8 + hl*4 + (0..3)
  const float inv = 1.0f / sum_xor32(l_run);
  if (row_valid) {
    const int64_t orow = ((int64_t)((int64_t)b * L + pos) * h_q + head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int dim = db * 32 + grp * 8 + hl * 4;
        const float y0 = oacc[db][grp * 4 + 0] * inv, y1 = oacc[db][grp * 4 + 1] * inv;
        const float y2 = oacc[db][grp * 4 + 2] * inv, y3 = oacc[db][grp * 4 + 3] * inv;
        if constexpr (OUT_BF16) {
          u32x2 w;
          w[0] = (uint32_t)f32_to_bf16_bits(y0) | ((uint32_t)f32_to_bf16_bits(y1) << 16);
          w[1] = (uint32_t)f32_to_bf16_bits(y2) | ((uint32_t)f32_to_bf16_bits(y3) << 16);
          *(u32x2*)((uint16_t*)o + orow + dim) = w;
        } else {
          f32x4 w = {y0, y1, y2, y3};
          *(f32x4*)((float*)o + orow + dim) = w;
        }
      }
  }
}

hipError_t launch_prefill_bf16(const uint16_t* q, const uint16_t* kp, const uint16_t* vt,
                               const float* kmax, const float2* cs, void* o, int out_bf16, int64_t B, int64_t L,
                               int64_t Lpad, int h_q, int h_kv, int d, float scale, int causal,
                               hipStream_t st) {
  const int g = h_q / h_kv;
  const int n_rb = (int)((L * g + kPrefillRowsWG - 1) / kPrefillRowsWG);
  const int n_bu = (int)(B * h_kv);
  const float sl2 = scale * 1.4426950408889634f;  // scale * log2(e): exp(x) = exp2(x log2 e)
  const unsigned grid = (unsigned)((int64_t)n_rb * n_bu);
#define GQA_LAUNCH(DD, OB)                                                                    \
  prefill_bf16_kernel<DD, OB><<<grid, NW * 64, 0, st>>>(q, kp, vt, kmax, cs, o, (int)L, (int)Lpad, \
                                                        h_q, h_kv, g, n_rb, n_bu, sl2, causal)
  if (d == 128) {
    if (out_bf16) GQA_LAUNCH(128, true); else GQA_LAUNCH(128, false);
  } else {
    if (out_bf16) GQA_LAUNCH(64, true); else GQA_LAUNCH(64, false);
  }
#undef GQA_LAUNCH
  return hipGetLastError();
}

}  // namespace gqa
