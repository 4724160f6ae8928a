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
//      its block's scale) and written transposed, [columns][segment], so that each
//      group's rows start on a 128-byte boundary and rows of other groups inside a
//      shared block are zero codes.
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
// written as zeros and it keeps the accumulator units unchanged.
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
};
__device__ inline Plan plan_view(const int32_t* w, int G) {
  return Plan{w, w + G, w + 2 * G, w + 3 * G + 1, reinterpret_cast<const float*>(w + 4 * G + 1),
              w + 5 * G + 1};
}

__device__ inline float scale_product(int64_t c, const float* a_blk, float a_s, float a_inv,
                                      const float* b_blk, float b_s, float b_inv, bool& dead) {
  const float sa = a_blk ? a_blk[c] : a_s;
  const float sb = b_blk ? b_blk[c] : b_s;
  const float ia = a_blk ? inv_from_scale(sa) : a_inv;
  const float ib = b_blk ? inv_from_scale(sb) : b_inv;
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
// any_wide;
// scprod[c] per 128-row block (0 for a block that adds nothing); ratio[b + g] for
// segment block b of group g, and 1 at ratio[seg[g + 1] + g], just past the group's
// blocks.
__global__ __launch_bounds__(PLAN_NT) void tgmm_plan_kernel(
    const int32_t* __restrict__ gs, int G, int64_t M, const float* __restrict__ a_blk,
    float a_s, float a_inv, const float* __restrict__ b_blk, float b_s, float b_inv,
    int32_t* __restrict__ plan, float* __restrict__ scprod, float* __restrict__ ratio) {
  __shared__ int s_tmp[PLAN_NT / 64];
  __shared__ int s_incl[PLAN_NT];
  __shared__ int s_off[PLAN_NT];
  __shared__ int s_seg[PLAN_NT + 1];
  __shared__ unsigned s_min[PLAN_NT], s_max[PLAN_NT], s_bad[PLAN_NT];
  __shared__ int s_last[PLAN_NT];
  const int t = threadIdx.x;
  const int Mi = (int)M;  // M < 2^23
  int32_t* off = plan;
  int32_t* cnt = plan + G;
  int32_t* seg = plan + 2 * G;
  int32_t* wide = plan + 3 * G + 1;
  float* fin = reinterpret_cast<float*>(plan + 4 * G + 1);

  // ---- groups: first row, rows, segment offset (sizes outside the contract are
  // clamped so that no access leaves the tensors) ----
  const int m = t < G ? min(max(gs[t], 0), Mi) : 0;
  const int incl = block_incl_scan(m, s_tmp, [Mi](int x, int y) { return min(x + y, Mi); });
  s_incl[t] = incl;
  __syncthreads();
  const int o = t > 0 ? s_incl[t - 1] : 0;
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
    const float sc = scale_product(cb, a_blk, a_s, a_inv, b_blk, b_s, b_inv, dead);
    scprod[cb] = dead ? 0.0f : sc;
  }
  __syncthreads();

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
      scale_product(block_of(g, b), a_blk, a_s, a_inv, b_blk, b_s, b_inv, dead);
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
      sc_prev = scale_product(block_of(g, prev), a_blk, a_s, a_inv, b_blk, b_s, b_inv, dead);
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
      const float sc = scale_product(block_of(g, b), a_blk, a_s, a_inv, b_blk, b_s, b_inv, dead);
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

// grid (segment blocks upper bound, C / 128).  Workgroup (b, ct): segment block b (a
// pair (group g, 128-row block c)) and columns [128 ct, 128 ct + 128).  A block whose
// scale product is zero gets zero codes.
template <int FMT>
__global__ __launch_bounds__(256) void quant_transpose_kernel(
    const uint16_t* __restrict__ x, int64_t C, const int32_t* __restrict__ plan, int G,
    const float* __restrict__ scale_blk, float inv_static, const float* __restrict__ scprod,
    uint8_t* __restrict__ seg, int64_t seg_row) {
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
  const int64_t col0 = (int64_t)blockIdx.y * 128;
  // rows [r_lo, r_hi) from column col0 on: later rows read as zero
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(x + (int64_t)r_lo * C + col0, (uint32_t)((int64_t)(r_hi - r_lo) * C * 2 - col0 * 2));
  const float inv = scprod[c] == 0.0f ? 0.0f
                    : scale_blk ? inv_from_scale(scale_blk[c]) : inv_static;
  const int t = threadIdx.x;
  const int rb = t & 15, cb = t >> 4;  // 8-row block, 8-column block
  v4u in[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = rb * 8 + e - rel;  // relative to the first row of g in the block
    uint32_t voff = (uint32_t)row * (uint32_t)(C * 2) + cb * 16;
    if (row < 0) voff = 0xfffffff0u;  // rows of the previous group: zero codes
    in[e] = buf_load16(r, voff);
  }
  v2u q[8];
  quant_transpose8<FMT>(in, inv, q);
  uint8_t* dst = seg + (col0 + cb * 8) * seg_row + (int64_t)b * BLOCK_ROWS + rb * 8;
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) *reinterpret_cast<v2u*>(dst + cc * seg_row) = q[cc];
}

// One wave fills 8 rows (1 KB) of a swizzled [rows][128 B] tile from global memory.
__device__ inline void load_rows_to_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds_rows,
                                        uint32_t goff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_rows, 16, goff, 0, 0, 0);
}

// One (group, 256 k x 256 n) tile per workgroup of 8 waves, each wave 128 k x 64 n
// (2 x 4 waves; two waves per SIMD, so one wave's vector work overlaps the other's
// MFMAs).  Per segment block s: the fp8 tiles of block s + 1 go straight from memory
// into the other LDS stage while block s is contracted.
template <int A_FMT, int B_FMT>
__global__ __attribute__((amdgpu_flat_work_group_size(RNT, RNT), amdgpu_waves_per_eu(2, 2)))
void tgmm_ratio_kernel(TgmmSegParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[RA_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[RB_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[RA_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[RB_TILE];

  const int n_kt = (p.Kout + RBM - 1) / RBM;
  const int n_nt = (p.Nout + RBN - 1) / RBN;
  const int total = n_kt * n_nt * p.G;
  const int wg = blockIdx.x;
  if (wg >= total) return;
  // Workgroup i runs on XCD i % 8 and each XCD owns a contiguous range of the tile
  // order.  That order is made of 32-tile super-tiles (the workgroups one XCD runs at a
  // time), cycling over the groups so that every XCD holds an equal share of every
  // group's work (a tile's work grows with its group's row count).  Inside a group,
  // tiles run in bands of ST_K k-tiles, k-tile fastest, so one super-tile is ST_K k-tiles
  // x 32/ST_K n-tiles: each A block it reads is shared by 32/ST_K workgroups and each
  // B block by ST_K of them while they sit together in the XCD's L2.  Tiles past the
  // last whole super-tile of each group follow, group-fastest.
  const int xcd = wg & 7, jx = wg >> 3, qx = total >> 3, rx = total & 7;
  const int L = xcd * qx + min(xcd, rx) + jx;
  const int T = n_kt * n_nt, T32 = T & ~31;
  int g, t;
  if (L < p.G * T32) {
    const int S = L >> 5;
    g = S % p.G;
    t = (S / p.G) * 32 + (L & 31);
  } else {
    const int r = L - p.G * T32;
    g = r % p.G;
    t = T32 + r / p.G;
  }
  const int kt_base = t / (ST_K * n_nt) * ST_K;
  const int band_rows = min(ST_K, n_kt - kt_base);
  const int rt = t - kt_base * n_nt;
  const int kt = kt_base + rt % band_rows, nt = rt / band_rows;

  const Plan pl = plan_view(p.plan, p.G);
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
    const uint32_t seg_row = (uint32_t)p.seg_row;
    const int krows = min(p.Kout - k0, RBM), nrows = min(p.Nout - n0, RBN);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(p.a_seg + (int64_t)k0 * p.seg_row + (int64_t)seg0 * BLOCK_ROWS,
                  (uint32_t)((int64_t)krows * p.seg_row - (int64_t)seg0 * BLOCK_ROWS));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(p.b_seg + (int64_t)n0 * p.seg_row + (int64_t)seg0 * BLOCK_ROWS,
                  (uint32_t)((int64_t)nrows * p.seg_row - (int64_t)seg0 * BLOCK_ROWS));

    // Direct loads of segment block s: rows 32 w .. 32 w + 31 of both tiles.  Past the
    // group's last block the offset leaves both ranges, so nothing is fetched (the
    // unused stage receives zeros) and the step stays free of branches.
    auto issue = [&](int s, uint8_t* at, uint8_t* bt) {
      const uint32_t koff = s < nblk ? (uint32_t)s * BLOCK_ROWS : 0x80000000u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wave * 32 + q * 8 + (lane >> 3);
        const uint32_t c = (uint32_t)((lane & 7) ^ (row & 7) ^ ((row >> 3) & 7));
        const uint32_t go = (uint32_t)row * seg_row + koff + c * 16;
        load_rows_to_lds(ra, at + (wave * 32 + q * 8) * TILE_K, go);
        load_rows_to_lds(rb, bt + (wave * 32 + q * 8) * TILE_K, go);
      }
    };
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
    auto rescale = [&](int b, int half, float r) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[b][half * 8 + e] *= r;
    };

    // Block s in 16 units u = 8 ks + b: MFMA of half step ks on sub-block b = 2 i + j,
    // chained into acc[b].  The accumulators hold units of the scale product of the
    // last live block; the move to block s + 1 multiplies sub-block b by ratio[s + 1]
    // (in two halves) after its last MFMA of block s (unit 8 + b) has finished and
    // before its first MFMA of block s + 1 (unit b there): halves at units b + 10 and
    // b + 13, counted on into the next block.  ratio of a block that adds nothing is 1.
    // Ratios come through a vector load issued before the step's direct loads, so that
    // waiting for one never waits for those.  The group's ratios are followed by a 1
    // (for the move past its last block); the read one further is out of range and
    // never used.
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(p.ratio + seg0 + g, (uint32_t)(nblk + 1) * 4);
    auto ratio_of = [&](int s) {
      return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rr, (uint32_t)s * 4, 0, 0));
    };
    float rc = ratio_of(0);  // into block s
    float rn = ratio_of(1);  // into block s + 1
    v8i af[4], bf[2][2];
    auto step = [&](int s, const uint8_t* at, const uint8_t* bt, uint8_t* an, uint8_t* bn) {
      const float rnn = ratio_of(s + 2);
      issue(s + 1, an, bn);
      af[0] = frag(at, wr * 128, 0, 0);
      bf[0][0] = frag(bt, wc * 64, 0, 0);
      bf[1][0] = frag(bt, wc * 64, 1, 0);
#pragma unroll
      for (int i = 1; i < 4; ++i) af[i] = frag(at, wr * 128, i, 0);
      bf[0][1] = frag(bt, wc * 64, 0, 1);
      bf[1][1] = frag(bt, wc * 64, 1, 1);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int ks = u >> 3, b = u & 7, i = b >> 1, j = b & 1;
        acc[b] = mfma32x32x64<B_FMT, A_FMT>(bf[j][ks], af[i], acc[b]);
        // the second half step's A fragment once both sub-blocks of row i used the first
        if (u < 8 && (u & 1)) af[u >> 1] = frag(at, wr * 128, u >> 1, 1);
        if (u == 0) { rescale(6, 0, rc); rescale(3, 1, rc); }
        if (u == 1) { rescale(7, 0, rc); rescale(4, 1, rc); }
        if (u == 2) rescale(5, 1, rc);
        if (u == 3) rescale(6, 1, rc);
        if (u == 4) rescale(7, 1, rc);
        if (u >= 10) rescale(u - 10, 0, rn);
        if (u >= 13) rescale(u - 13, 1, rn);
        __builtin_amdgcn_sched_barrier(0);
      }
      rc = rn;
      rn = rnn;
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
    // the halves still owed to a next block would multiply by 1
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
      if (n >= p.Nout) continue;
      const int64_t idx = slab + (int64_t)k * p.Nout + n;
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = acc[blk][4 * r4 + e] * fin;
      if (p.out_f32) {
        v4f v = {o[0], o[1], o[2], o[3]};
        *reinterpret_cast<v4f*>((float*)p.out + idx) = v;
      } else {
        v2u v;
        v.x = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
        v.y = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
        *reinterpret_cast<v2u*>((uint16_t*)p.out + idx) = v;
      }
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
          make_rsrc(p.a_seg + (int64_t)k0 * p.seg_row + (int64_t)seg0 * BLOCK_ROWS,
                    (uint32_t)((int64_t)krows * p.seg_row - (int64_t)seg0 * BLOCK_ROWS));
      const __amdgpu_buffer_rsrc_t rb =
          make_rsrc(p.b_seg + (int64_t)n0 * p.seg_row + (int64_t)seg0 * BLOCK_ROWS,
                    (uint32_t)((int64_t)TBN * p.seg_row - (int64_t)seg0 * BLOCK_ROWS));

      // direct loads of segment block s: A rows 64w..64w+63 (8 per wave-load),
      // B rows 32w..32w+31
      auto issue = [&](int s, uint8_t* at, uint8_t* bt) {
        const uint32_t koff = (uint32_t)s * BLOCK_ROWS;
  #pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int row = wave * 64 + q * 8 + (lane >> 3);
          const uint32_t c = (uint32_t)((lane & 7) ^ (row & 7) ^ ((row >> 3) & 7));
          load_rows_to_lds(ra, at + (wave * 64 + q * 8) * TILE_K, (uint32_t)row * seg_row + koff + c * 16);
        }
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wave * 32 + q * 8 + (lane >> 3);
          const uint32_t c = (uint32_t)((lane & 7) ^ (row & 7) ^ ((row >> 3) & 7));
          load_rows_to_lds(rb, bt + (wave * 32 + q * 8) * TILE_K, (uint32_t)row * seg_row + koff + c * 16);
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
          v.x = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
          v.y = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
          *reinterpret_cast<v2u*>((uint16_t*)p.out + idx) = v;
        }
      }
    }
  }
}

template <int FMT>
hipError_t launch_qt(const uint16_t* x, int64_t M, int64_t C, const int32_t* plan, int G,
                     const float* scale_blk, float inv_static, const float* scprod, uint8_t* seg,
                     int64_t seg_row, hipStream_t st) {
  const int64_t max_blocks = (M + BLOCK_ROWS - 1) / BLOCK_ROWS + G;
  dim3 grid((unsigned)max_blocks, (unsigned)(C / 128));
  hipLaunchKernelGGL(quant_transpose_kernel<FMT>, grid, dim3(256), 0, st, x, C, plan, G,
                     scale_blk, inv_static, scprod, seg, seg_row);
  return hipGetLastError();
}

template <int A_FMT, int B_FMT>
hipError_t launch_tgmm_fp8(const TgmmSegParams& p, hipStream_t st) {
  const int64_t tiles = (int64_t)((p.Kout + RBM - 1) / RBM) * ((p.Nout + RBN - 1) / RBN) * p.G;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((tgmm_ratio_kernel<A_FMT, B_FMT>), dim3((unsigned)tiles), dim3(RNT), 0, st, p);
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
  hipLaunchKernelGGL(tgmm_plan_kernel, dim3(1), dim3(PLAN_NT), 0, st, p.group_sizes, p.G, p.M,
                     p.a_scale_blk, p.a_scale_static, p.a_inv_static, p.b_scale_blk,
                     p.b_scale_static, p.b_inv_static, p.plan, p.scprod, p.ratio);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.M > 0) {
    e = a_fmt == FMT_E4M3
            ? launch_qt<FMT_E4M3>(p.a, p.M, p.Kout, p.plan, p.G, p.a_scale_blk, p.a_inv_static, p.scprod, p.a_seg, seg_row, st)
            : launch_qt<FMT_E5M2>(p.a, p.M, p.Kout, p.plan, p.G, p.a_scale_blk, p.a_inv_static, p.scprod, p.a_seg, seg_row, st);
    if (e != hipSuccess) return e;
    e = b_fmt == FMT_E4M3
            ? launch_qt<FMT_E4M3>(p.b, p.M, p.Nout, p.plan, p.G, p.b_scale_blk, p.b_inv_static, p.scprod, p.b_seg, seg_row, st)
            : launch_qt<FMT_E5M2>(p.b, p.M, p.Nout, p.plan, p.G, p.b_scale_blk, p.b_inv_static, p.scprod, p.b_seg, seg_row, st);
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
