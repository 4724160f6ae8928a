// Transposed grouped matmul on gfx950: the kernels behind tgmm_drhs ("Support
// quantization for tokamax gmm v2", PR #4451, What this does: drhs_tgmm2).
//
//   drhs[g, k, n] = sum over 128-row blocks c meeting group g of
//                   RNE( P_c[k, n] * RNE(s_lhs[c] * s_grad[c]) ),
//   P_c[k, n]     = sum_{m in c, m in g} q(lhs)[m, k] * q(grad)[m, n]   (fp32 MFMA sums)
//
// The contraction runs over the rows of a group, and both operands are stored with
// that axis strided.  The path therefore has four kernels:
//   1. tgmm_plan: per group the first row, the row count and the offset of its
//      "segment" (the 128-row blocks the group meets, laid end to end); per block the
//      scale product sc_c; per segment block the ratio of scale products used below.
//   2. quant_transpose (once per operand): every element quantized exactly once (with
//      its block's scale), or taken as it is when the operand arrives as fp8 codes, and
//      written transposed into the segment, so that each group's rows start on a block
//      boundary and rows of other groups inside a shared block are zero codes.  Columns are stored in pairs: block b of columns 2p, 2p + 1 is 256
//      bytes, [2p: m 0..63][2p + 1: m 0..63][2p: m 64..127][2p + 1: m 64..127], so a
//      half block of two columns is one 128-byte line.
//   3. tgmm_ratio: per (group, 256 k x 256 n) tile, one contraction step per block of
//      the group's segment.  Instead of scaling each block's partial sum and adding it
//      (two vector ops per value per block), the fp32 accumulators are kept in units of
//      the current block's scale product: MFMA adds P_c straight into them, and between
//      blocks each value is multiplied once by sc_prev / sc_next.  The last block's
//      scale product is applied in the epilogue.  A group without rows stores +0.0.
//   4. tgmm_promote: the exact per-block promotion (fresh MFMA partial, then
//      acc += partial * sc_c), for the rare groups whose scale products span more than
//      2^60, where the rescaled accumulators could leave the fp32 range.
//
// A block whose scale product is zero (an all-zero block, a scale whose inverse is not
// finite, or a product that underflows) adds nothing in the method; its codes are
// written as zeros and it keeps the accumulator units unchanged.  For an operand given
// as codes only a zero product counts: its codes are used as they are.
#include "kernels.hpp"

namespace gmm {

namespace {

// tgmm_promote tile
constexpr int TBM = 256;   // k rows of a slab tile
constexpr int TBN = 128;   // n columns of a slab tile
constexpr int NT = 256;
constexpr int A_TILE = TBM * TILE_K;  // [256 k][128 m] fp8
constexpr int B_TILE = TBN * TILE_K;  // [128 n][128 m] fp8
// tgmm_ratio tile
constexpr int RBM = 256;   // k rows
constexpr int RBN = 256;   // n columns
constexpr int RNT = 512;   // 8 waves: 2 (k) x 4 (n), 128 x 64 each
constexpr int RA_TILE = RBM * TILE_K;
constexpr int RB_TILE = RBN * TILE_K;
constexpr int ST_K = 4;    // k-tiles per band of the tile order
constexpr int PLAN_NT = 1024;
constexpr int PAIR_BLOCK = 2 * BLOCK_ROWS;  // bytes of one block of a column pair
static_assert(MAX_GROUPS <= PLAN_NT, "one plan thread per group");
// widest spread of nonzero scale products in a group that the rescaled accumulators
// take: with |P_c| <= 128 * 57344^2 and at most 2^15 blocks the values stay below 2^114
constexpr float RATIO_RANGE = 0x1p60f;

struct Plan {  // views of the plan words (see plan_words)
  const int32_t* off;
  const int32_t* cnt;
  const int32_t* seg;
  const int32_t* wide;
  const float* fin;
  const int32_t* any_wide;
  const int32_t* order;
};
__device__ inline Plan plan_view(const int32_t* w, int G) {
  return Plan{w, w + G, w + 2 * G, w + 3 * G + 1, reinterpret_cast<const float*>(w + 4 * G + 1),
              w + 5 * G + 1, w + 5 * G + 2};
}

// Operand scaling as the plan sees it: per-block scales (blk) or a static scale and
// inverse; `codes` when the operand arrives as fp8 codes.
struct OpScale {
  const float* blk;
  float s, inv;
  int codes;
};

// Block c's scale product RNE(s_a * s_b), and whether the block adds nothing: a zero
// product, or a bf16 operand whose block quantizes to zero codes (inverse 0).  Codes
// given as input are used as they are, so for them only a zero product drops the block.
__device__ inline float scale_product(int64_t c, const OpScale& a, const OpScale& b, bool& dead) {
  const float sa = a.blk ? a.blk[c] : a.s;
  const float sb = b.blk ? b.blk[c] : b.s;
  const float ia = a.codes ? 1.0f : a.blk ? inv_from_scale(sa) : a.inv;
  const float ib = b.codes ? 1.0f : b.blk ? inv_from_scale(sb) : b.inv;
  const float sc = __fmul_rn(sa, sb);
  dead = sc == 0.0f || ia == 0.0f || ib == 0.0f;
  return sc;
}

// inclusive scan over the whole workgroup (all threads call it); op(a, b) associative
template <typename Op>
__device__ inline int block_incl_scan(int v, int* tmp, Op op) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v = op(u, v);
  }
  if (lane == 63) tmp[w] = v;
  __syncthreads();
  for (int i = w - 1; i >= 0; --i) v = op(tmp[i], v);
  __syncthreads();
  return v;
}

// One workgroup.  Plan words: off[G], cnt[G], seg[G + 1], wide[G], fin[G] (float),
// any_wide, order[G] (the groups by segment blocks, most first; ties by index);
// scprod[c] per 128-row block (0 for a block that adds nothing); ratio[b + g] for
// segment block b of group g, and 1 at ratio[seg[g + 1] + g], just past the group's
// blocks.
__global__ __launch_bounds__(PLAN_NT) void tgmm_plan_kernel(
    const int32_t* __restrict__ gs, int g_before, int G, int64_t M, OpScale a_sc, OpScale b_sc,
    int32_t* __restrict__ plan, float* __restrict__ scprod, float* __restrict__ ratio) {
  __shared__ int s_tmp[PLAN_NT / 64];
  __shared__ int s_incl[PLAN_NT];
  __shared__ int s_off[PLAN_NT];
  __shared__ int s_seg[PLAN_NT + 1];
  __shared__ unsigned s_min[PLAN_NT], s_max[PLAN_NT], s_bad[PLAN_NT];
  __shared__ int s_last[PLAN_NT];
  const int t = threadIdx.x;
  const int Mi = (int)M;  // M < 2^31 (and below 2^24 - 128 G, see tgmm_drhs)
  int32_t* off = plan;
  int32_t* cnt = plan + G;
  int32_t* seg = plan + 2 * G;
  int32_t* wide = plan + 3 * G + 1;
  float* fin = reinterpret_cast<float*>(plan + 4 * G + 1);

  // ---- groups of the window (the G after the first g_before): first row, rows,
  // segment offset (sizes outside the contract are clamped so that no access leaves the
  // tensors) ----
  auto add_clamped = [Mi](int x, int y) { return (int)min((int64_t)x + y, (int64_t)Mi); };
  const int mb = t < g_before ? min(max(gs[t], 0), Mi) : 0;
  s_incl[t] = block_incl_scan(mb, s_tmp, add_clamped);
  __syncthreads();
  const int rows_before = s_incl[PLAN_NT - 1];
  __syncthreads();
  const int m = t < G ? min(max(gs[g_before + t], 0), Mi) : 0;
  const int incl = block_incl_scan(m, s_tmp, add_clamped);
  s_incl[t] = incl;
  __syncthreads();
  const int o = add_clamped(rows_before, t > 0 ? s_incl[t - 1] : 0);
  const int c = min(m, Mi - o);
  const int nb = c > 0 ? (o + c - 1) / BLOCK_ROWS - o / BLOCK_ROWS + 1 : 0;
  const int bincl = block_incl_scan(nb, s_tmp, [](int x, int y) { return x + y; });
  if (t < G) {
    off[t] = o;
    cnt[t] = c;
    seg[t] = bincl - nb;
    s_off[t] = o;
    s_seg[t] = bincl - nb;
  }
  if (t == PLAN_NT - 1) {
    seg[G] = bincl;
    s_seg[G] = bincl;
  }
  s_min[t] = 0x7f800000u;
  s_max[t] = 0u;
  s_bad[t] = 0u;

  // ---- per block scale products ----
  const int64_t nblk = (M + BLOCK_ROWS - 1) / BLOCK_ROWS;
  for (int64_t cb = t; cb < nblk; cb += PLAN_NT) {
    bool dead;
    const float sc = scale_product(cb, a_sc, b_sc, dead);
    scprod[cb] = dead ? 0.0f : sc;
  }
  __syncthreads();

  // ---- the order in which the rescaling kernel walks the groups: most segment blocks
  // first, ties by group index (each group's rank counts the groups that go before it) ----
  if (t < G) {
    const int nb_t = s_seg[t + 1] - s_seg[t];
    int rank = 0;
    for (int h = 0; h < G; ++h) {
      const int nb_h = s_seg[h + 1] - s_seg[h];
      rank += (nb_h > nb_t || (nb_h == nb_t && h < t)) ? 1 : 0;
    }
    plan[5 * G + 2 + rank] = t;
  }

  // ---- per segment block ratios: each thread walks a contiguous chunk ----
  const int S = s_seg[G];
  const int chunk = (S + PLAN_NT - 1) / PLAN_NT;
  const int b0 = min(t * chunk, S), b1 = min(b0 + chunk, S);
  auto group_of = [&](int b) {  // s_seg[g] <= b < s_seg[g + 1]
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_seg[mid] <= b) lo = mid; else hi = mid;
    }
    return lo;
  };
  auto block_of = [&](int g, int b) { return (int64_t)(s_off[g] / BLOCK_ROWS + (b - s_seg[g])); };
  // pass 1: the last live block of the chunk
  int last = -1;
  if (b0 < b1) {
    int g = group_of(b0);
    for (int b = b0; b < b1; ++b) {
      while (b >= s_seg[g + 1]) ++g;
      bool dead;
      scale_product(block_of(g, b), a_sc, b_sc, dead);
      if (!dead) last = b;
    }
  }
  const int prev_incl = block_incl_scan(last, s_tmp, [](int x, int y) { return max(x, y); });
  s_last[t] = prev_incl;
  __syncthreads();
  // pass 2: ratios, final scales, per group range of the live scale products
  if (b0 < b1) {
    int g = group_of(b0);
    int prev = t > 0 ? s_last[t - 1] : -1;
    float sc_prev = 0.0f;
    if (prev >= s_seg[g]) {
      bool dead;
      sc_prev = scale_product(block_of(g, prev), a_sc, b_sc, dead);
    } else {
      prev = -1;
    }
    unsigned lmin = 0x7f800000u, lmax = 0u, lbad = 0u;
    auto flush = [&](int gg) {
      if (lmax != 0u || lbad) {
        atomicMin(&s_min[gg], lmin);
        atomicMax(&s_max[gg], lmax);
        if (lbad) atomicOr(&s_bad[gg], 1u);
      }
      lmin = 0x7f800000u; lmax = 0u; lbad = 0u;
    };
    for (int b = b0; b < b1; ++b) {
      if (b >= s_seg[g + 1]) {
        flush(g);
        while (b >= s_seg[g + 1]) ++g;
        prev = -1;
      }
      bool dead;
      const float sc = scale_product(block_of(g, b), a_sc, b_sc, dead);
      float r = 1.0f;
      if (!dead) {
        if (prev >= 0) r = __fdiv_rn(sc_prev, sc);
        prev = b;
        sc_prev = sc;
        if (!__builtin_isfinite(sc)) {
          lbad = 1u;
        } else {
          const unsigned u = __float_as_uint(fabsf(sc));
          lmin = min(lmin, u);
          lmax = max(lmax, u);
        }
      }
      ratio[b + g] = r;
      if (b == s_seg[g + 1] - 1) fin[g] = prev >= 0 ? sc_prev : 1.0f;
    }
    flush(g);
  }
  __syncthreads();
  int w = 0;
  if (t < G) {
    const float lo = __uint_as_float(s_min[t]), hi = __uint_as_float(s_max[t]);
    w = (s_bad[t] != 0u || (s_max[t] != 0u && hi > lo * RATIO_RANGE)) ? 1 : 0;
    wide[t] = w;
    if (s_seg[t + 1] == s_seg[t]) fin[t] = 1.0f;
    ratio[s_seg[t + 1] + t] = 1.0f;
  }
  const int any = __syncthreads_or(w);
  if (t == 0) plan[5 * G + 1] = any;
}

// Quantize an 8 (rows) x 8 (cols) bf16 block held as 8 row vectors into 8 column
// vectors of 8 codes each (rows 0..3 in .x, rows 4..7 in .y): the paired conversion
// packs two rows of one column per instruction, so the transposition is free.
template <int FMT>
__device__ inline void quant_transpose8(const v4u in[8], float inv, v2u out[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t d = c < 2 ? in[r].x : c < 4 ? in[r].y : c < 6 ? in[r].z : in[r].w;
      v[r] = quant_prep<FMT>((c & 1) ? bf16_hi(d) : bf16_lo(d), inv);
    }
    uint32_t lo = cvt_pk<FMT, false>(v[0], v[1], __float_as_uint(v[0]));
    lo = cvt_pk<FMT, true>(v[2], v[3], lo);
    uint32_t hi = cvt_pk<FMT, false>(v[4], v[5], __float_as_uint(v[4]));
    hi = cvt_pk<FMT, true>(v[6], v[7], hi);
    out[c].x = lo;
    out[c].y = hi;
  }
}

// grid (segment blocks upper bound, ceil(C / CW)).  Workgroup (b, ct): segment block b
// (a pair (group g, 128-row block c)) and columns [CW ct, CW ct + CW).  A block whose
// scale product is zero gets zero codes.  x holds bf16 values, quantized here with the
// block's scale (CW = 128: 8 rows x 8 columns per thread), or (CODES) fp8 codes quantized
// beforehand, which are only transposed (CW = 256: 8 rows x 16 columns per thread, so a
// load reads 16 bytes of a row).
template <int FMT, bool CODES>
__global__ __launch_bounds__(256) void quant_transpose_kernel(
    const void* __restrict__ x, int64_t C, const int32_t* __restrict__ plan, int G,
    const float* __restrict__ scale_blk, float inv_static, const float* __restrict__ scprod,
    uint8_t* __restrict__ seg, int64_t seg_row) {
  constexpr int ES = CODES ? 1 : 2;     // bytes per element of x
  constexpr int CW = CODES ? 256 : 128;  // columns per workgroup
  const int32_t* off = plan;
  const int32_t* cnt = plan + G;
  const int32_t* sg = plan + 2 * G;
  const int b = blockIdx.x;
  if (b >= sg[G]) return;
  int lo = 0, hi = G;  // sg[lo] <= b < sg[lo + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sg[mid] <= b) lo = mid; else hi = mid;
  }
  const int g = __builtin_amdgcn_readfirstlane(lo);
  const int o = __builtin_amdgcn_readfirstlane(off[g]);
  const int n = __builtin_amdgcn_readfirstlane(cnt[g]);
  const int c = o / BLOCK_ROWS + (b - __builtin_amdgcn_readfirstlane(sg[g]));
  const int r_lo = max(o, c * BLOCK_ROWS), r_hi = min(o + n, (c + 1) * BLOCK_ROWS);
  const int rel = r_lo - c * BLOCK_ROWS;  // first row of the block that belongs to g
  const int64_t col0 = (int64_t)blockIdx.y * CW;
  // rows [r_lo, r_hi) from column col0 on: later rows read as zero
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc((const uint8_t*)x + ((int64_t)r_lo * C + col0) * ES,
                (uint32_t)(((int64_t)(r_hi - r_lo) * C - col0) * ES));
  const bool dead = scprod[c] == 0.0f;
  const int t = threadIdx.x;
  const int rb = t & 15, cb = t >> 4;  // 8-row block; 8- (bf16) or 16-column (codes) block
  // segment layout by column pairs: pair p, block b holds 256 bytes, [col 2p, m 0..63]
  // [col 2p + 1, m 0..63] [col 2p, m 64..127] [col 2p + 1, m 64..127]
  auto store8 = [&](int64_t col, const v2u (&q)[8]) {
    uint8_t* dst = seg + col * seg_row + (int64_t)b * PAIR_BLOCK + (rb >> 3) * 128 + (rb & 7) * 8;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      *reinterpret_cast<v2u*>(dst + (cc >> 1) * 2 * seg_row + (cc & 1) * 64) = q[cc];
  };
  if constexpr (CODES) {
    if (col0 + cb * 16 >= C) return;  // C is a multiple of 128: whole 16-column blocks
    v4u in[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = rb * 8 + e - rel;  // relative to the first row of g in the block
      uint32_t voff = (uint32_t)row * (uint32_t)C + cb * 16;
      if (row < 0 || dead) voff = 0xfffffff0u;  // previous group's rows, or a dead block: zeros
      in[e] = buf_load16(r, voff);
    }
    v2u lo8[8], hi8[8], q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo8[e].x = in[e].x; lo8[e].y = in[e].y;
      hi8[e].x = in[e].z; hi8[e].y = in[e].w;
    }
    transpose8x8(lo8, q);
    store8(col0 + cb * 16, q);
    transpose8x8(hi8, q);
    store8(col0 + cb * 16 + 8, q);
  } else {
    const float inv = dead ? 0.0f : scale_blk ? inv_from_scale(scale_blk[c]) : inv_static;
    v4u in[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = rb * 8 + e - rel;
      uint32_t voff = (uint32_t)row * (uint32_t)(C * 2) + cb * 16;
      if (row < 0) voff = 0xfffffff0u;  // rows of the previous group: zero codes
      in[e] = buf_load16(r, voff);
    }
    v2u q[8];
    quant_transpose8<FMT>(in, inv, q);
    store8(col0 + cb * 8, q);
  }
}

// One wave fills 8 rows (1 KB) of a swizzled [rows][128 B] tile from global memory.
__device__ inline void load_rows_to_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds_rows,
                                        uint32_t goff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_rows, 16, goff, 0, 0, 0);
}

// Half-block stage of the rescaling kernel: [256 rows][64 contraction bytes] per operand.
// 16-byte chunk c of row r sits at chunk position c ^ (((r >> 1) ^ (r >> 3)) & 3): the
// rows one phase of a fragment read touches (8 rows over 32 banks, or 16 over 64) then
// fall on distinct 16-byte bank groups.
constexpr int HROW = 64;
constexpr int RH_TILE = RBM * HROW;  // 16 KB

// One (group, 256 k x 256 n) tile per workgroup of 8 waves, each wave 128 k x 64 n
// (2 x 4 waves; two waves per SIMD, so one wave's vector work overlaps the other's
// MFMAs).  The contraction runs in half-blocks of 64 rows through a ring of 4 LDS
// stages: half-step h's fp8 tiles are loaded into one of two register staging sets
// three half-steps ahead and written into stage h % 4 two half-steps ahead, and
// half-step h + 1's fragments are read into registers while half-step h's MFMAs run,
// so no step waits on LDS reads when it starts.
template <int A_FMT, int B_FMT>
__global__ __attribute__((amdgpu_flat_work_group_size(RNT, RNT), amdgpu_waves_per_eu(2, 2)))
void tgmm_ratio_kernel(TgmmSegParams p, const float* __restrict__ ratio) {
  // one array for the 4 stages (A tile, then B tile, per stage): every LDS address is
  // then a per-lane register plus a constant that fits the instruction's offset field
  // (two base registers in all), instead of one register per stage and operand
  __shared__ __attribute__((aligned(1024))) uint8_t s_lds[8 * RH_TILE];
  uint8_t* const sA0 = s_lds;
  uint8_t* const sB0 = s_lds + RH_TILE;
  uint8_t* const sA1 = s_lds + 2 * RH_TILE;
  uint8_t* const sB1 = s_lds + 3 * RH_TILE;
  uint8_t* const sA2 = s_lds + 4 * RH_TILE;
  uint8_t* const sB2 = s_lds + 5 * RH_TILE;
  uint8_t* const sA3 = s_lds + 6 * RH_TILE;
  uint8_t* const sB3 = s_lds + 7 * RH_TILE;

  const int n_kt = (p.Kout + RBM - 1) / RBM;
  const int n_nt = (p.Nout + RBN - 1) / RBN;
  // Workgroup i runs on XCD i % 8.  A tile's work grows with its group's row count, and
  // one group may hold a third of the rows, so every group's T tiles are split into 8
  // chunks of csize = ceil(T / 8) consecutive tiles, chunk x on XCD x: every XCD holds an
  // equal share of every group's work.  Each XCD walks its chunks group by group in the
  // plan's order, most blocks first, so the longest tiles start first.  Inside a group,
  // tiles run in bands of ST_K k-tiles, k-tile fastest, so the 32 workgroups an XCD runs
  // together form ST_K k-tiles x 32/ST_K n-tiles: each A block they read is shared by
  // 32/ST_K workgroups and each B block by ST_K of them in the XCD's L2.
  const int T = n_kt * n_nt, csize = (T + 7) / 8;
  const int wg = blockIdx.x, xcd = wg & 7, jx = wg >> 3;
  const int o = jx / csize, t = xcd * csize + (jx - o * csize);
  if (o >= p.G || t >= T) return;
  const Plan pl = plan_view(p.plan, p.G);
  const int g = __builtin_amdgcn_readfirstlane(pl.order[o]);
  const int kt_base = t / (ST_K * n_nt) * ST_K;
  const int band_rows = min(ST_K, n_kt - kt_base);
  const int rt = t - kt_base * n_nt;
  const int kt = kt_base + rt % band_rows, nt = rt / band_rows;

  if (pl.wide[g]) return;  // tgmm_promote takes this group
  const int k0 = kt * RBM, n0 = nt * RBN;
  const int seg0 = __builtin_amdgcn_readfirstlane(pl.seg[g]);
  const int nblk = __builtin_amdgcn_readfirstlane(pl.seg[g + 1]) - seg0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 2, wc = wave & 3;  // wave sub-tile: 128 (k) x 64 (n)
  const int frow = lane & 31, fhalf = lane >> 5;

  v16f acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = v16f{0};
  float fin = 1.0f;

  if (nblk > 0) {
    fin = pl.fin[g];
    const int H = 2 * nblk;  // half-steps
    const uint32_t seg_row = (uint32_t)p.seg_row;
    const int krows = min(p.Kout - k0, RBM), nrows = min(p.Nout - n0, RBN);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(p.a_seg + (int64_t)k0 * p.seg_row + (int64_t)seg0 * PAIR_BLOCK,
                  (uint32_t)((int64_t)krows * p.seg_row - (int64_t)seg0 * PAIR_BLOCK));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(p.b_seg + (int64_t)n0 * p.seg_row + (int64_t)seg0 * PAIR_BLOCK,
                  (uint32_t)((int64_t)nrows * p.seg_row - (int64_t)seg0 * PAIR_BLOCK));
    // The ratio half-step h applies: block (h + 1) / 2's (the tail of the move into
    // block h / 2 for even h, the head of the move into block h / 2 + 1 for odd h).  The
    // group's ratios are followed by a 1 (for the move past its last block); the index
    // stops there.  A uniform read through a restrict pointer: a scalar load, outside
    // the vector-load count the pipeline waits on.
    const float* gratio = ratio + seg0 + g;
    auto ratio_of = [&](int h) -> float { return gratio[min((h + 1) >> 1, nblk)]; };

    // Half-step X of both tiles goes through registers: thread t holds 16-byte chunks t
    // and t + 512 of each tile (row idx / 4, logical chunk idx % 4); in the column-pair
    // layout 8 consecutive threads cover one 128-byte line (rows 2p, 2p + 1).  Past the
    // last half-step the offsets leave the ranges and the loads return zeros.
    auto gload = [&](int X, v4u (&sa)[2], v4u (&sb)[2]) {
      const uint32_t hoff =
          X < H ? (uint32_t)(X >> 1) * PAIR_BLOCK + (uint32_t)(X & 1) * 128 : 0x80000000u;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = q * RNT + tid, row = idx >> 2;
        const uint32_t go = (uint32_t)(row >> 1) * 2 * seg_row + (uint32_t)(row & 1) * 64 + hoff +
                            (uint32_t)(idx & 3) * 16;
        sa[q] = buf_load16(ra, go);
        sb[q] = buf_load16(rb, go);
      }
    };
    uint32_t wo[2];  // the chunks' places in a stage tile
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = q * RNT + tid, row = idx >> 2;
      wo[q] = (uint32_t)row * HROW + ((uint32_t)((idx & 3) ^ (((row >> 1) ^ (row >> 3)) & 3)) << 4);
    }
    auto lwrite = [&](uint8_t* t, const v4u (&sv)[2]) {
#pragma unroll
      for (int q = 0; q < 2; ++q) *reinterpret_cast<v4u*>(t + wo[q]) = sv[q];
    };
    uint32_t fo[2];
    {
      const uint32_t f0 = (uint32_t)(((frow >> 1) ^ (frow >> 3)) & 3);
#pragma unroll
      for (int e = 0; e < 2; ++e) fo[e] = (uint32_t)frow * HROW + ((((uint32_t)(2 * fhalf + e)) ^ f0) << 4);
    }
    auto frag = [&](const uint8_t* tile, int base_row, int i) -> v8i {
      const uint8_t* p0 = tile + (base_row + i * 32) * HROW;
      const v4u lo = *reinterpret_cast<const v4u*>(p0 + fo[0]);
      const v4u hi = *reinterpret_cast<const v4u*>(p0 + fo[1]);
      v8i f;
      f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
      f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
      return f;
    };
    auto rescale = [&](int b, int half, float r) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[b][half * 8 + e] *= r;
    };

    // Half-step h on stage (at, bt).  Unit u: MFMA on sub-block u = 2 i + j (acc[u] holds
    // A rows 32 i.., B rows 32 j..).  B fragments stay in bf for the whole half-step; A
    // fragment i is read into slot i % 2 two units before its first use.  After the
    // first MFMA: this wave's LDS writes of stage h + 1 (made during h - 1) and its reads
    // are done; then the workgroup barrier, after which all of stage h + 1 may be read.
    // Then: the loads of half-step h + 3 into staging set (la, lb); at units 4 and 5
    // staging set (wa, wb), loaded during h - 1, written to stage h + 2 (the four loads
    // of h + 3 may stay in flight); at units 6 and 7 half-step h + 1's first fragments
    // from stage h + 1 (bf[0] and A fragment 0 after the last uses here, bf[1] last).
    // Rescales: the accumulators hold units of the last live block's scale product; the
    // move into block c + 1 multiplies acc[u] by ratio[c + 1] in two halves, at units
    // u + 10 and u + 13 counted from block c's first half-step (after its last MFMA of
    // block c, before its first of block c + 1).  The ratio register r serves
    // half-steps h, h + 4, ...: it is reloaded after its last use here.
    v8i af[2], bf[2];
    auto half = [&](int h, const uint8_t* at, const uint8_t* an, const uint8_t* bn, uint8_t* aw,
                    uint8_t* bw, v4u (&la)[2], v4u (&lb)[2], const v4u (&wa)[2],
                    const v4u (&wb)[2], float& r) {
      const bool second = h & 1;
      float rn = 1.0f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = u >> 1, j = u & 1;
        acc[u] = mfma32x32x64<B_FMT, A_FMT>(bf[j], af[i & 1], acc[u]);
        if (u == 0) {
          __builtin_amdgcn_sched_barrier(0);  // the first MFMA goes out before the wait
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_s_barrier();
          // this half-step's ratio, loaded long ago: taken into a fresh register here,
          // where nothing else is pending, so its uses below wait for nothing
          asm volatile("s_mov_b32 %0, %1" : "=s"(rn) : "s"(r));
          gload(h + 3, la, lb);
        }
        if (!(u & 1) && u < 6) af[(i + 1) & 1] = frag(at, wr * 128, i + 1);
        if (u == 4) {
          asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
          lwrite(aw, wa);
        }
        if (u == 5) lwrite(bw, wb);
        if (u == 6) {
          bf[0] = frag(bn, wc * 64, 0);
          af[0] = frag(an, wr * 128, 0);
        }
        if (u == 7) bf[1] = frag(bn, wc * 64, 1);
        if (!second) {
          if (u == 0) { rescale(6, 0, rn); rescale(3, 1, rn); }
          if (u == 1) { rescale(7, 0, rn); rescale(4, 1, rn); }
          if (u == 2) rescale(5, 1, rn);
          if (u == 3) rescale(6, 1, rn);
          if (u == 4) rescale(7, 1, rn);
        } else {
          if (u >= 2) rescale(u - 2, 0, rn);
          if (u >= 5) rescale(u - 5, 1, rn);
        }
        if (u == 7) r = ratio_of(h + 4);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // prologue: half-steps 0 and 1 into stages 0 and 1, half-step 2 loaded; stage 0's
    // first fragments
    v4u s0a[2], s0b[2], s1a[2], s1b[2];
    gload(0, s0a, s0b);
    gload(1, s1a, s1b);
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    lwrite(sA0, s0a);
    lwrite(sB0, s0b);
    gload(2, s0a, s0b);
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    lwrite(sA1, s1a);
    lwrite(sB1, s1b);
    float r0 = ratio_of(0), r1 = ratio_of(1), r2 = ratio_of(2), r3 = ratio_of(3);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    af[0] = frag(sA0, wr * 128, 0);
    bf[0] = frag(sB0, wc * 64, 0);
    bf[1] = frag(sB0, wc * 64, 1);
    int h = 0;
    for (; h + 4 <= H; h += 4) {
      half(h, sA0, sA1, sB1, sA2, sB2, s1a, s1b, s0a, s0b, r0);
      half(h + 1, sA1, sA2, sB2, sA3, sB3, s0a, s0b, s1a, s1b, r1);
      half(h + 2, sA2, sA3, sB3, sA0, sB0, s1a, s1b, s0a, s0b, r2);
      half(h + 3, sA3, sA0, sB0, sA1, sB1, s0a, s0b, s1a, s1b, r3);
    }
    if (h < H) {  // H is even: two half-steps remain
      half(h, sA0, sA1, sB1, sA2, sB2, s1a, s1b, s0a, s0b, r0);
      half(h + 1, sA1, sA2, sB2, sA3, sB3, s0a, s0b, s1a, s1b, r1);
    }
    // the halves still owed to a next block would multiply by 1
  }

  // ---- store: lane holds out[k = base + lane%32][n = base + 8*(r/4) + 4*(lane/32) + r%4]
  const int64_t slab = (int64_t)g * p.Kout * p.Nout;
  if (!p.out_f32) {
    // bf16: each wave puts its 128 x 64 sub-tile into its own 16 KB of LDS ([row][128 B],
    // 16-byte chunk c of row r at c ^ (r & 7)), then stores whole 128-byte rows, 16 bytes
    // per lane: full lines instead of 16-byte pieces of 32 rows per store.
    __syncthreads();  // every wave is done with the stage tiles
    uint8_t* const wl = s_lds + wave * (128 * 128);
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int i = blk >> 1, j = blk & 1;
      const int row = i * 32 + frow;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int col = j * 64 + r4 * 16 + fhalf * 8;  // byte column
        v2u v;
        v.x = pack_bf16x2(acc[blk][4 * r4] * fin, acc[blk][4 * r4 + 1] * fin);
        v.y = pack_bf16x2(acc[blk][4 * r4 + 2] * fin, acc[blk][4 * r4 + 3] * fin);
        *reinterpret_cast<v2u*>(wl + row * 128 + ((((col >> 4) ^ (row & 7)) << 4) | (col & 15))) = v;
      }
    }
    const bool cols_ok = n0 + wc * 64 < p.Nout;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = q * 8 + (lane >> 3), c = lane & 7;
      const v4u v = *reinterpret_cast<const v4u*>(wl + row * 128 + ((c ^ (row & 7)) << 4));
      const int k = k0 + wr * 128 + row;
      if (cols_ok && k < p.Kout)
        *reinterpret_cast<v4u*>((uint16_t*)p.out + slab + (int64_t)k * p.Nout + n0 + wc * 64 + c * 8) = v;
    }
    return;
  }
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    const int i = blk >> 1, j = blk & 1;
    const int k = k0 + wr * 128 + i * 32 + frow;
    if (k >= p.Kout) continue;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int n = n0 + wc * 64 + j * 32 + 8 * r4 + 4 * fhalf;
      if (n >= p.Nout) continue;
      const int64_t idx = slab + (int64_t)k * p.Nout + n;
      v4f v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[blk][4 * r4 + e] * fin;
      *reinterpret_cast<v4f*>((float*)p.out + idx) = v;
    }
  }
}

// Exact per-block promotion for the groups the plan marks wide.  A grid-stride loop
// over all (group, 256 k x 128 n) tiles that skips every other group, so that the
// launch costs next to nothing when no group is wide.
template <int A_FMT, int B_FMT>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
void tgmm_promote_kernel(TgmmSegParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[A_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[B_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[A_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[B_TILE];

  const Plan pl = plan_view(p.plan, p.G);
  if (*pl.any_wide == 0) return;
  const int n_kt = (p.Kout + TBM - 1) / TBM;
  const int n_nt = p.Nout / TBN;
  const int total = n_kt * n_nt * p.G;
  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    const int g = L % p.G;
    if (pl.wide[g] == 0) continue;
    const int t = L / p.G;
    const int kt = t / n_nt, nt = t - kt * n_nt;
    const int k0 = kt * TBM, n0 = nt * TBN;
    const int32_t* off = p.plan;
    const int32_t* sg = p.plan + 2 * p.G;
    const int seg0 = __builtin_amdgcn_readfirstlane(sg[g]);
    const int nblk = __builtin_amdgcn_readfirstlane(sg[g + 1]) - seg0;
    const int c0 = __builtin_amdgcn_readfirstlane(off[g]) / BLOCK_ROWS;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;  // wave sub-tile: 128 (k) x 64 (n)
    const int frow = lane & 31, fhalf = lane >> 5;

    v16f acc[8];
  #pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = v16f{0};

    if (nblk > 0) {
      const uint32_t seg_row = (uint32_t)p.seg_row;
      const int krows = min(p.Kout - k0, TBM);
      const __amdgpu_buffer_rsrc_t ra =
          make_rsrc(p.a_seg + (int64_t)k0 * p.seg_row + (int64_t)seg0 * PAIR_BLOCK,
                    (uint32_t)((int64_t)krows * p.seg_row - (int64_t)seg0 * PAIR_BLOCK));
      const __amdgpu_buffer_rsrc_t rb =
          make_rsrc(p.b_seg + (int64_t)n0 * p.seg_row + (int64_t)seg0 * PAIR_BLOCK,
                    (uint32_t)((int64_t)TBN * p.seg_row - (int64_t)seg0 * PAIR_BLOCK));

      // direct loads of segment block s: A rows 64w..64w+63 (8 per wave-load),
      // B rows 32w..32w+31
      // byte of (row, logical 16-byte chunk c of the block) from the block's start in the
      // column-pair layout
      auto pair_off = [&](int row, uint32_t c) -> uint32_t {
        return (uint32_t)(row >> 1) * 2 * seg_row + (c >> 2) * 128 + (uint32_t)(row & 1) * 64 +
               (c & 3) * 16;
      };
      auto issue = [&](int s, uint8_t* at, uint8_t* bt) {
        const uint32_t koff = (uint32_t)s * PAIR_BLOCK;
  #pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int row = wave * 64 + q * 8 + (lane >> 3);
          const uint32_t c = (uint32_t)((lane & 7) ^ (row & 7) ^ ((row >> 3) & 7));
          load_rows_to_lds(ra, at + (wave * 64 + q * 8) * TILE_K, pair_off(row, c) + koff);
        }
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wave * 32 + q * 8 + (lane >> 3);
          const uint32_t c = (uint32_t)((lane & 7) ^ (row & 7) ^ ((row >> 3) & 7));
          load_rows_to_lds(rb, bt + (wave * 32 + q * 8) * TILE_K, pair_off(row, c) + koff);
        }
      };
      // fragment addressing, as in the grouped GEMM: two per-lane offsets per half block
      uint32_t fo[2][2];
      {
        const uint32_t f0 = (uint32_t)((frow & 7) ^ (frow >> 3));
  #pragma unroll
        for (int tt = 0; tt < 2; ++tt)
  #pragma unroll
          for (int e = 0; e < 2; ++e)
            fo[tt][e] = (uint32_t)frow * TILE_K + ((((uint32_t)(2 * fhalf + e)) ^ f0 ^ (4u * tt)) << 4);
      }
      auto frag = [&](const uint8_t* tile, int base_row, int i, int ks) -> v8i {
        const int tt = ks ^ (i & 1);
        const uint8_t* p0 = tile + base_row * TILE_K + i * 32 * TILE_K;
        const v4u lo = *reinterpret_cast<const v4u*>(p0 + fo[tt][0]);
        const v4u hi = *reinterpret_cast<const v4u*>(p0 + fo[tt][1]);
        v8i f;
        f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
        f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
        return f;
      };
      auto barrier = [&]() {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      };

      // Partial sums of the current block, one 32x32 sub-block per entry, in block-major
      // MFMA order: unit u = 2b + ks issues half step ks of sub-block b (the two halves are
      // chained accumulations).  Sub-block b is complete after unit 2b + 1; its promotion
      // acc += part * sc runs three units later, 8 values per unit, so every unit pairs
      // one MFMA with 16 VALU instructions, and units 0..2 finish the previous block.
      v16f part[8];
  #pragma unroll
      for (int b = 0; b < 8; ++b) part[b] = v16f{0};
      float sc_prev = 0.0f;
      // scale product of the block a step will multiply, loaded one step ahead so that
      // waiting for it never waits for the direct loads issued after it
      float sc_next = p.scprod[c0];

      auto promote = [&](int b, int half, float sc) {
  #pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[b][half * 8 + e] = __builtin_fmaf(part[b][half * 8 + e], sc, acc[b][half * 8 + e]);
      };

      auto step = [&](int s, const uint8_t* at, const uint8_t* bt, uint8_t* an, uint8_t* bn) {
        const float sc_cur = sc_next;
        sc_next = p.scprod[c0 + min(s + 1, nblk - 1)];
        issue(s + 1, an, bn);
        v8i bf[2][2], af[2][2];  // [j or i parity][ks]
  #pragma unroll
        for (int j = 0; j < 2; ++j)
  #pragma unroll
          for (int ks = 0; ks < 2; ++ks) bf[j][ks] = frag(bt, wc * 64, j, ks);
  #pragma unroll
        for (int ks = 0; ks < 2; ++ks) af[0][ks] = frag(at, wr * 128, 0, ks);
  #pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int b = u >> 1, ks = u & 1, i = b >> 1, j = b & 1;
          part[b] = mfma32x32x64<B_FMT, A_FMT>(bf[j][ks], af[i & 1][ks], ks == 0 ? v16f{0} : part[b]);
          // next A fragments once the previous pair of sub-blocks has used its registers
          if (u == 1 || u == 5 || u == 9) {
  #pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) af[(i + 1) & 1][k2] = frag(at, wr * 128, i + 1, k2);
          }
          const int v = (u + 13) & 15;  // promotion slot: unit u handles value-half v
          if (u < 3) promote(v >> 1, v & 1, sc_prev);
          else promote(v >> 1, v & 1, sc_cur);
          __builtin_amdgcn_sched_barrier(0);
        }
        sc_prev = sc_cur;
        barrier();
      };

      issue(0, sA0, sB0);
      barrier();
      int s = 0;
      for (; s + 1 < nblk; s += 2) {
        step(s, sA0, sB0, sA1, sB1);
        step(s + 1, sA1, sB1, sA0, sB0);
      }
      if (s < nblk) step(s, sA0, sB0, sA1, sB1);
      // the last block's sub-blocks 6 (second half) and 7 are still unpromoted
      promote(6, 1, sc_prev);
      promote(7, 0, sc_prev);
      promote(7, 1, sc_prev);
    }

    // ---- store: lane holds out[k = base + lane%32][n = base + 8*(r/4) + 4*(lane/32) + r%4]
    const int64_t slab = (int64_t)g * p.Kout * p.Nout;
  #pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int i = blk >> 1, j = blk & 1;
      const int k = k0 + wr * 128 + i * 32 + frow;
      if (k >= p.Kout) continue;
  #pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = n0 + wc * 64 + j * 32 + 8 * r4 + 4 * fhalf;
        const int64_t idx = slab + (int64_t)k * p.Nout + n;
        float o[4];
  #pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[blk][4 * r4 + e];
        if (p.out_f32) {
          v4f v = {o[0], o[1], o[2], o[3]};
          *reinterpret_cast<v4f*>((float*)p.out + idx) = v;
        } else {
          v2u v;
          v.x = pack_bf16x2(o[0], o[1]);
          v.y = pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<v2u*>((uint16_t*)p.out + idx) = v;
        }
      }
    }
  }
}

// The transposing quantizer for one operand (bf16 values, or fp8 codes when `codes`).
hipError_t launch_qt(int fmt, bool codes, const void* x, int64_t M, int64_t C,
                     const int32_t* plan, int G, const float* scale_blk, float inv_static,
                     const float* scprod, uint8_t* seg, int64_t seg_row, hipStream_t st) {
  const int64_t max_blocks = (M + BLOCK_ROWS - 1) / BLOCK_ROWS + G;
  const int64_t cw = codes ? 256 : 128;
  dim3 grid((unsigned)max_blocks, (unsigned)((C + cw - 1) / cw));
#define GMM_QT(F, CD)                                                                     \
  if (fmt == F && codes == CD) {                                                          \
    hipLaunchKernelGGL((quant_transpose_kernel<F, CD>), grid, dim3(256), 0, st, x, C, plan, \
                       G, scale_blk, inv_static, scprod, seg, seg_row);                   \
    return hipGetLastError();                                                             \
  }
  GMM_QT(FMT_E4M3, false)
  GMM_QT(FMT_E5M2, false)
  GMM_QT(FMT_E4M3, true)
  GMM_QT(FMT_E5M2, true)
#undef GMM_QT
  return hipErrorInvalidValue;
}

template <int A_FMT, int B_FMT>
hipError_t launch_tgmm_fp8(const TgmmSegParams& p, hipStream_t st) {
  // per group T tiles in 8 chunks of ceil(T / 8), one per XCD
  const int64_t T = (int64_t)((p.Kout + RBM - 1) / RBM) * ((p.Nout + RBN - 1) / RBN);
  const int64_t tiles = 8 * ((T + 7) / 8) * p.G;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((tgmm_ratio_kernel<A_FMT, B_FMT>), dim3((unsigned)tiles), dim3(RNT), 0, st, p,
                     p.ratio);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ptiles = (int64_t)((p.Kout + TBM - 1) / TBM) * (p.Nout / TBN) * p.G;
  hipLaunchKernelGGL((tgmm_promote_kernel<A_FMT, B_FMT>), dim3((unsigned)(ptiles < 1024 ? ptiles : 1024)),
                     dim3(NT), 0, st, p);
  return hipGetLastError();
}

}  // namespace

int64_t tgmm_segment_row_bytes(int64_t M, int G) {
  // every group's rows start on a block boundary: at most ceil(M/128) + G blocks
  return ((M + BLOCK_ROWS - 1) / BLOCK_ROWS + G) * BLOCK_ROWS;
}

hipError_t launch_tgmm(int a_fmt, int b_fmt, const TgmmParams& p, hipStream_t st) {
  const int64_t seg_row = tgmm_segment_row_bytes(p.M, p.G);
  const OpScale a_sc{p.a_scale_blk, p.a_scale_static, p.a_inv_static, p.a_codes};
  const OpScale b_sc{p.b_scale_blk, p.b_scale_static, p.b_inv_static, p.b_codes};
  hipLaunchKernelGGL(tgmm_plan_kernel, dim3(1), dim3(PLAN_NT), 0, st, p.group_sizes, p.g_before,
                     p.G, p.M, a_sc, b_sc, p.plan, p.scprod, p.ratio);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.M > 0) {
    e = launch_qt(a_fmt, p.a_codes != 0, p.a, p.M, p.Kout, p.plan, p.G, p.a_scale_blk,
                  p.a_inv_static, p.scprod, p.a_seg, seg_row, st);
    if (e != hipSuccess) return e;
    e = launch_qt(b_fmt, p.b_codes != 0, p.b, p.M, p.Nout, p.plan, p.G, p.b_scale_blk,
                  p.b_inv_static, p.scprod, p.b_seg, seg_row, st);
    if (e != hipSuccess) return e;
  }
  TgmmSegParams q{};
  q.a_seg = p.a_seg;
  q.b_seg = p.b_seg;
  q.plan = p.plan;
  q.out = p.out;
  q.scprod = p.scprod;
  q.ratio = p.ratio;
  q.Kout = p.Kout;
  q.Nout = p.Nout;
  q.G = p.G;
  q.out_f32 = p.out_f32;
  q.seg_row = seg_row;
  if (a_fmt == FMT_E4M3 && b_fmt == FMT_E5M2) return launch_tgmm_fp8<FMT_E4M3, FMT_E5M2>(q, st);
  if (a_fmt == FMT_E4M3 && b_fmt == FMT_E4M3) return launch_tgmm_fp8<FMT_E4M3, FMT_E4M3>(q, st);
  if (a_fmt == FMT_E5M2 && b_fmt == FMT_E5M2) return launch_tgmm_fp8<FMT_E5M2, FMT_E5M2>(q, st);
  if (a_fmt == FMT_E5M2 && b_fmt == FMT_E4M3) return launch_tgmm_fp8<FMT_E5M2, FMT_E4M3>(q, st);
  return hipErrorInvalidValue;
}

}  // namespace gmm
