// Transposed grouped matmul on gfx950: the kernels behind tgmm_drhs ("Support
// quantization for tokamax gmm v2", PR #4451, What this does: drhs_tgmm2).
//
//   drhs[g, k, n] = sum over 128-row blocks c meeting group g of  P_c[k, n] * sc_c,
//   P_c[k, n]     = sum_{m in c, m in g} q(lhs)[m, k] * q(grad)[m, n]   (fp32 MFMA sums),
//   sc_c          = RNE(s_lhs[c] * s_grad[c])
//
// The contraction runs over the rows of a group, and both operands are stored row-major
// with that axis strided.  The kernels read the row-major fp8 codes directly: a tile of
// 128 rows x 256 columns is copied into LDS as it lies in memory (whole 128-byte lines
// from global memory), and gfx950's transposing LDS read (ds_read_b64_tr_b8) hands every
// lane the 8 rows of one column that an MFMA operand needs, so no transposed copy of
// either operand is made.  A bf16 operand is quantized once, row-major, into the
// workspace by the stand-alone quantizer (its codes are those every other product uses).
//
//   1. tgmm_plan: per group the first row, the row count and the index of its first
//      "segment block" (the 128-row blocks the group meets, numbered end to end over
//      the groups); per block the scale product sc_c (0 for a block that adds nothing);
//      per segment block the ratio of scale products used below.
//   2. tgmm_main: per (group, 256 k x 256 n) tile, one contraction step per 128-row
//      block of the group.  Instead of scaling each block's partial sum and adding it
//      (two vector ops per value per block), the fp32 accumulators are kept in units of
//      the current block's scale product: MFMA adds P_c straight into them, and between
//      blocks each value is multiplied once by sc_prev / sc_next.  The last block's scale
//      product is applied in the epilogue.  A group without rows stores +0.0.
//   3. tgmm_promote: the per-block promotion as the method states it (fresh MFMA
//      partial P_c, then acc = RNE(acc + RNE(P_c * sc_c))), for the rare groups whose
//      scale products span more than 2^60, where the rescaled accumulators could leave
//      the fp32 range.
//
// A block whose scale product is zero (an all-zero block, a scale whose inverse is not
// finite, or a product that underflows) adds nothing in the method: its rows are read
// as zeros and it leaves the accumulator units unchanged.  For an operand given as codes
// only a zero product counts: its codes are used as they are.
#include "kernels.hpp"

namespace gmm {

namespace {

constexpr int MBK = 256;    // k rows of a tgmm_main tile
constexpr int MBN = 256;    // n columns of a tgmm_main tile
constexpr int MNT = 512;    // 8 waves: 2 (k) x 4 (n), 128 k x 64 n each (two per SIMD)
constexpr int ROWB = 256;   // bytes of one LDS row: 256 k (lhs) or 256 n (grad) codes
constexpr int OPB = BLOCK_ROWS * ROWB;  // one operand's 128-row stage tile: 32 KB
constexpr int ST_K = 4;     // k-tiles per band of the tile order
constexpr int PBK = 128;    // tgmm_promote tile: 128 k x 128 n, 4 waves of 64 x 64
constexpr int PNT = 256;
constexpr int PROWB = 128;  // bytes of one promote LDS row
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

// ---------------------------------------------------------------------------------
// LDS tiles of row-major codes and their transposing reads.
//
// A stage tile is [128 rows m][R bytes] (R = 256 in tgmm_main, 128 in tgmm_promote).
// 16-byte chunk c of row m sits at chunk position c ^ key(m): the 8 rows that one
// 16-lane group of a transposing read touches land on distinct 16-byte bank groups.
//
// ds_read_b64_tr_b8 (measured lane layout): within each group of 16 lanes, lane j
// receives byte b from the address of lane 2b + (j >> 3), plus (j & 7).  So if lane
// 2b + h addresses row m0 + b at column col0 + 8h, lane j receives column col0 + j of
// rows m0 .. m0 + 7, one byte per row: 8 contraction bytes of one MFMA operand row.
// ---------------------------------------------------------------------------------
typedef int32_t v2i __attribute__((ext_vector_type(2)));

__device__ inline v2i lds_read_tr8(const uint8_t* p) {
  typedef __attribute__((address_space(3))) v2i lds_v2i;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)p);
}

// One 32 x 64 MFMA operand from a stage tile: operand row r (0..31) is tile column
// R0 + r, and its 64 contraction bytes are tile rows m0 .. m0 + 63.  Lane l holds row
// l % 32 and contraction bytes 8 q + b = tile row m0 + 32 (l / 32) + 8 q + b: the same
// assignment for both operands of an MFMA, so the products pair up.  `lo` is the lane's
// address of its first read (row part and swizzled column, see tr_lane_offset).
template <int R>
__device__ inline v8i frag_tr8(const uint8_t* lo) {
  v8i f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v2i v = lds_read_tr8(lo + q * 8 * R);
    f[2 * q] = v.x;
    f[2 * q + 1] = v.y;
  }
  return f;
}

// The lane's address (from the tile's start, for m0 = 0) of operand rows R0 .. R0 + 31
// (R0 a multiple of 32) in a tile of R-byte rows whose chunk position is c ^ key(m):
// lane l = 16 g16 + j addresses row 32 (g16 >> 1) + (j >> 1) (+ 8 q per read), column
// R0 + 16 (g16 & 1) + 8 (j & 1).  key(m) depends on m & 7 = (j >> 1) only.
template <int R>
__device__ inline uint32_t tr_lane_offset(int lane, int R0) {
  const int g16 = lane >> 4, j = lane & 15;
  const int row = 32 * (g16 >> 1) + (j >> 1);
  const int chunk = (R0 >> 4) + (g16 & 1);
  const int key = R == 256 ? 2 * (j >> 1) : (j >> 1);
  return (uint32_t)(row * R + ((chunk ^ key) << 4) + 8 * (j & 1));
}

// Row range of block c inside the group [off, off + cnt).
__device__ inline void block_rows(int c, int off, int cnt, int& lo, int& hi) {
  lo = max(off, c * BLOCK_ROWS);
  hi = min(off + cnt, c * BLOCK_ROWS + BLOCK_ROWS);
}

struct TgmmCodesParams {
  const uint8_t* a;      // lhs codes [M, Kout]
  const uint8_t* b;      // grad codes [M, Nout]
  const int32_t* plan;
  const float* scprod;
  const float* ratio;
  void* out;             // [G, Kout, Nout] bf16 or f32
  int32_t Kout, Nout, G, out_f32;
};

// One (group, 256 k x 256 n) tile per workgroup of 8 waves, each 128 k x 64 n (2 x 4
// waves; two per SIMD, so one wave's vector work overlaps the other's MFMAs).  Step s
// contracts the group's rows in its block c_lo + s: two LDS stages of [128 rows][256 B]
// per operand (128 KB), filled from registers that were loaded two steps ahead; one
// barrier per step.
template <int A_FMT, int B_FMT>
__global__ __attribute__((amdgpu_flat_work_group_size(MNT, MNT), amdgpu_waves_per_eu(2, 2)))
void tgmm_main_kernel(TgmmCodesParams p) {
  // stage x: A tile at 2 x OPB, B tile at 2 x OPB + OPB
  __shared__ __attribute__((aligned(1024))) uint8_t s_lds[4 * OPB];
  uint8_t* const sA0 = s_lds;
  uint8_t* const sB0 = s_lds + OPB;
  uint8_t* const sA1 = s_lds + 2 * OPB;
  uint8_t* const sB1 = s_lds + 3 * OPB;

  const int n_kt = (p.Kout + MBK - 1) / MBK;
  const int n_nt = (p.Nout + MBN - 1) / MBN;
  // Workgroup i runs on XCD i % 8.  A tile's work grows with its group's row count, and
  // one group may hold a third of the rows, so every group's T tiles are split into 8
  // chunks of csize = ceil(T / 8) consecutive tiles, chunk x on XCD x: every XCD holds an
  // equal share of every group's work.  Each XCD walks its chunks group by group in the
  // plan's order, most blocks first, so the longest tiles start first.  Inside a group,
  // tiles run in bands of ST_K k-tiles, k-tile fastest, so the 32 workgroups an XCD runs
  // together form ST_K k-tiles x 32/ST_K n-tiles that share lhs and grad rows in its L2.
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
  const int k0 = kt * MBK, n0 = nt * MBN;
  const int seg0 = __builtin_amdgcn_readfirstlane(pl.seg[g]);
  const int nblk = __builtin_amdgcn_readfirstlane(pl.seg[g + 1]) - seg0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 2, wc = wave & 3;  // wave sub-tile: 128 (k) x 64 (n)
  const int frow = lane & 31, fhalf = lane >> 5;

  v16f acc[8];  // acc[2 i + j]: k rows wr 128 + 32 i.., n columns wc 64 + 32 j..
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = v16f{0};
  float fin = 1.0f;

  if (nblk > 0) {
    fin = pl.fin[g];
    const int off = __builtin_amdgcn_readfirstlane(pl.off[g]);
    const int cnt = __builtin_amdgcn_readfirstlane(pl.cnt[g]);
    const int c_lo = off / BLOCK_ROWS;
    const int K = p.Kout, N = p.Nout;
    // ratio(t): the factor of the move into the group's block t (a 1 follows the last)
    const float* gratio = p.ratio + seg0 + g;

    // Global loads: thread t moves 16-byte chunk t & 15 of rows (t >> 4) + 32 q of the
    // step's 128 rows (q = 0..3), of both operands: 16 threads read one row's 256
    // contiguous bytes (two whole lines).  Offsets are relative to the step's first row
    // of the group; rows before it wrap around to offsets past the range and read zeros.
    const int lrow = tid >> 4, lch = tid & 15;
    uint32_t a_off[4], b_off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a_off[q] = (uint32_t)(lrow + 32 * q) * (uint32_t)K + lch * 16;
      b_off[q] = (uint32_t)(lrow + 32 * q) * (uint32_t)N + lch * 16;
    }
    const uint32_t wofs = (uint32_t)lrow * ROWB + ((uint32_t)(lch ^ (2 * (lrow & 7))) << 4);
    v4u sa[4], sb[4];  // staging registers of step s + 2
    // Step x's loads into the staging registers: block c_lo + x's rows of the group;
    // past the group, or in a block whose scale product is zero, everything reads zero.
    // which: 0 = the lhs chunk only, 1 = the grad chunk only
    auto gload = [&](int x, bool live, int q, int which) {
      int lo, hi;
      block_rows(c_lo + x, off, cnt, lo, hi);
      live = live && x < nblk;
      const __amdgpu_buffer_rsrc_t ra =
          make_rsrc(p.a + (int64_t)lo * K + k0, live ? (uint32_t)((hi - lo) * K - k0) : 0u);
      const __amdgpu_buffer_rsrc_t rb =
          make_rsrc(p.b + (int64_t)lo * N + n0, live ? (uint32_t)((hi - lo) * N - n0) : 0u);
      const int skip = lo - (c_lo + x) * BLOCK_ROWS;  // rows of the block before the group
      if (which == 0) sa[q] = buf_load16(ra, a_off[q] - (uint32_t)(skip * K));
      else sb[q] = buf_load16(rb, b_off[q] - (uint32_t)(skip * N));
    };
    // The steps' scalars, 64 steps at a time: lane i holds the ratio of the move into
    // block w0 + i (see gratio) and a ballot mask whether that block adds anything, so a
    // step reads them with readlane and a shift, not with a load it would wait for.
    int w0 = 0;
    float wratio = 1.0f;
    uint64_t wlive = 0;
    auto load_window = [&](int base) {
      w0 = base;
      const int x = base + lane;
      wratio = gratio[min(x, nblk)];
      wlive = __ballot(x < nblk && p.scprod[c_lo + min(x, nblk - 1)] != 0.0f);
      // wait here, once per window, so that no step waits on these loads (vmcnt(0))
      __builtin_amdgcn_s_waitcnt(0x0f70);
    };
    auto ratio_at = [&](int x) {  // w0 <= x < w0 + 64
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wratio), x - w0));
    };
    auto live_of = [&](int x) -> bool { return ((wlive >> (x - w0)) & 1u) != 0u; };
    auto lwrite = [&](uint8_t* at, uint8_t* bt, int q, int which) {
      if (which == 0) *reinterpret_cast<v4u*>(at + q * 32 * ROWB + wofs) = sa[q];
      else *reinterpret_cast<v4u*>(bt + q * 32 * ROWB + wofs) = sb[q];
    };
    // fragment addresses: A operand rows wr 128 + 32 i (k), B operand rows wc 64 + 32 j (n)
    uint32_t fa[4], fb[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = tr_lane_offset<ROWB>(lane, wr * 128 + 32 * i);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = tr_lane_offset<ROWB>(lane, wc * 64 + 32 * j);
    auto fragA = [&](const uint8_t* at, int i, int ks) { return frag_tr8<ROWB>(at + fa[i] + ks * 64 * ROWB); };
    auto fragB = [&](const uint8_t* bt, int j, int ks) { return frag_tr8<ROWB>(bt + fb[j] + ks * 64 * ROWB); };
    auto rescale = [&](int v, int h, float r) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[v][h * 8 + e] *= r;
    };

    // Step s on stage (at, bt); (an, bn) is the next stage.  Unit u issues MFMA
    // (ks = u / 8, i = (u / 2) % 4, j = u % 2) on acc[2 i + j], with the A fragment of
    // linear index L = 4 ks + i in register slot L % 2.  Alongside:
    //   * units 0..7: staging chunk u / 2 of the lhs (u even) or the grad (u odd), step
    //     s + 1, is written to the next stage and refilled with step s + 2's load (one
    //     chunk per unit keeps the LDS writes and the loads from bunching up);
    //   * after odd unit u <= 11, A fragment L = (u + 3) / 2 is read into the slot unit u
    //     has just finished with (two MFMAs before its first use); the ks = 1 B
    //     fragments are read after unit 3;
    //   * before unit 14: this wave's LDS work is done, the workgroup barrier, after which
    //     the next stage is complete and the next step's first fragments are read while
    //     units 14 and 15 (whose fragments are in registers) keep the matrix core busy;
    //     the next step's A fragment 1 follows unit 15;
    //   * the move into block s + 1 multiplies acc[v] by r_next in two halves, half 0 at
    //     unit 10 + v and half 1 at unit 14 + v (two MFMAs after acc[v]'s last one of the
    //     block at unit 8 + v); the halves past unit 15 run in units 0..5 of the next step,
    //     with the same ratio (r_prev there), before acc[v]'s first MFMA at unit v.
    v8i af[2], bf0[2], bf1[2];
    auto step = [&](int s, const uint8_t* at, const uint8_t* bt, uint8_t* an, uint8_t* bn,
                    float r_prev, float r_next, bool live2) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int ks = u >> 3, i = (u >> 1) & 3, j = u & 1;
        if (u == 14) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          bf0[0] = fragB(bn, 0, 0);
          bf0[1] = fragB(bn, 1, 0);
          af[0] = fragA(an, 0, 0);
        }
        acc[2 * i + j] = mfma32x32x64<B_FMT, A_FMT>(ks == 0 ? bf0[j] : bf1[j], af[i & 1], acc[2 * i + j]);
        if (u < 8) {
          // the chunk leaves its registers before they are reloaded (one staging set);
          // one chunk per unit, lhs and grad in turn
          lwrite(an, bn, u >> 1, u & 1);
          __builtin_amdgcn_sched_barrier(0);
          gload(s + 2, live2, u >> 1, u & 1);
        }
        if (u == 3) {
          bf1[0] = fragB(bt, 0, 1);
          bf1[1] = fragB(bt, 1, 1);
        }
        if ((u & 1) && u <= 11) {
          const int L = (u + 3) >> 1;
          af[L & 1] = fragA(at, L & 3, L >> 2);
        }
        if (u == 15) af[1] = fragA(an, 1, 0);
        // the tail of the move into this block
        if (u == 0) { rescale(2, 1, r_prev); rescale(6, 0, r_prev); }
        if (u == 1) { rescale(3, 1, r_prev); rescale(7, 0, r_prev); }
        if (u >= 2 && u <= 5) rescale(u + 2, 1, r_prev);
        // the head of the move into the next block
        if (u >= 10) rescale(u - 10, 0, r_next);
        if (u >= 14) rescale(u - 14, 1, r_next);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // prologue: step 0 into stage 0, step 1 into the staging registers, the first
    // fragments of stage 0.  Step 0's loads go out before the window's and share its
    // wait (one memory round trip, not two): they read block 0 whatever its scale
    // product, and a block that adds nothing has its registers cleared afterwards, as if
    // it had been read as zeros.
#pragma unroll
    for (int q = 0; q < 8; ++q) gload(0, true, q >> 1, q & 1);
    load_window(0);
    bool live0 = live_of(0), live1 = live_of(1), live2 = live_of(2);
    if (!live0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) sa[q] = sb[q] = v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) lwrite(sA0, sB0, q >> 1, q & 1);
#pragma unroll
    for (int q = 0; q < 8; ++q) gload(1, live1, q >> 1, q & 1);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    bf0[0] = fragB(sB0, 0, 0);
    bf0[1] = fragB(sB0, 1, 0);
    af[0] = fragA(sA0, 0, 0);
    af[1] = fragA(sA0, 1, 0);
    float r_prev = 1.0f, r_next = ratio_at(min(1, nblk));
    int s = 0;
    for (; s + 1 < nblk; s += 2) {
      if (s + 4 >= w0 + 64) load_window(s);  // the window holds steps s .. s + 4
      bool live3 = live_of(s + 3);
      float r_n2 = ratio_at(s + 2);  // s + 2 <= nblk here
      step(s, sA0, sB0, sA1, sB1, r_prev, r_next, live2);
      r_prev = r_next;
      r_next = r_n2;
      live2 = live3;
      live3 = live_of(s + 4);
      r_n2 = ratio_at(min(s + 3, nblk));
      step(s + 1, sA1, sB1, sA0, sB0, r_prev, r_next, live2);
      r_prev = r_next;
      r_next = r_n2;
      live2 = live3;
    }
    if (s < nblk) step(s, sA0, sB0, sA1, sB1, r_prev, r_next, live2);
    // the halves still owed to the move past the last block would multiply by 1
  }

  // ---- store: lane holds out[k = base + lane%32][n = base + 8*(r/4) + 4*(lane/32) + r%4]
  const int64_t slab = (int64_t)g * p.Kout * p.Nout;
  if (!p.out_f32) {
    // bf16: each wave puts its 128 x 64 sub-tile into its own 16 KB of LDS ([row][128 B],
    // 16-byte chunk c of row r at c ^ (r & 7)), then stores whole 128-byte rows, 16 bytes
    // per lane: full lines instead of 16-byte pieces of 32 rows.
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
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's region only
    // K and N are multiples of 128: the wave's 128 k rows and 64 n columns lie all inside
    // the output or all outside it
    if (n0 + wc * 64 >= p.Nout || k0 + wr * 128 >= p.Kout) return;
    // stores through a resource over the wave's 128 rows (offsets below 2^30), eight
    // rows' LDS reads in flight before their stores
    const int c = lane & 7;
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc((uint16_t*)p.out + slab + (int64_t)(k0 + wr * 128) * p.Nout, 256u * (uint32_t)p.Nout);
    const uint32_t lane_off = ((uint32_t)(lane >> 3) * (uint32_t)p.Nout + (uint32_t)(n0 + wc * 64 + c * 8)) * 2u;
    const uint32_t q_stride = 16u * (uint32_t)p.Nout;  // 8 rows
#pragma unroll
    for (int q0 = 0; q0 < 16; q0 += 8) {
      v4u v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int row = (q0 + t) * 8 + (lane >> 3);
        v[t] = *reinterpret_cast<const v4u*>(wl + row * 128 + ((c ^ (row & 7)) << 4));
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) buf_store16(ro, lane_off + (uint32_t)(q0 + t) * q_stride, v[t]);
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

// The per-block promotion for the groups the plan marks wide: for each block, a fresh
// MFMA partial P_c, then acc = RNE(acc + RNE(P_c * sc_c)), each rounding on its own.  A
// grid-stride loop over all (group, 128 k x 128 n) tiles that skips every other group,
// so that the launch costs next to nothing when no group is wide.  One LDS stage,
// loaded and consumed in turn: a rare fallback, kept simple.
template <int A_FMT, int B_FMT>
__global__ __attribute__((amdgpu_flat_work_group_size(PNT, PNT), amdgpu_waves_per_eu(1, 1)))
void tgmm_promote_kernel(TgmmCodesParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA[BLOCK_ROWS * PROWB];
  __shared__ __attribute__((aligned(1024))) uint8_t sB[BLOCK_ROWS * PROWB];
  const Plan pl = plan_view(p.plan, p.G);
  if (*pl.any_wide == 0) return;
  const int n_kt = p.Kout / PBK, n_nt = p.Nout / PBK;
  const int total = n_kt * n_nt * p.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;  // wave sub-tile: 64 (k) x 64 (n)
  const int frow = lane & 31, fhalf = lane >> 5;
  uint32_t fa[2], fb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    fa[i] = tr_lane_offset<PROWB>(lane, wr * 64 + 32 * i);
    fb[i] = tr_lane_offset<PROWB>(lane, wc * 64 + 32 * i);
  }
  // thread t moves 16-byte chunk t & 7 of rows (t >> 3) + 32 q (q = 0..3)
  const int lrow = tid >> 3, lch = tid & 7;
  const uint32_t wofs = (uint32_t)lrow * PROWB + ((uint32_t)(lch ^ (lrow & 7)) << 4);
  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    const int g = L % p.G;
    if (pl.wide[g] == 0) continue;
    const int tt = L / p.G;
    const int k0 = (tt / n_nt) * PBK, n0 = (tt % n_nt) * PBK;
    const int off = __builtin_amdgcn_readfirstlane(pl.off[g]);
    const int cnt = __builtin_amdgcn_readfirstlane(pl.cnt[g]);
    const int seg0 = __builtin_amdgcn_readfirstlane(pl.seg[g]);
    const int nblk = __builtin_amdgcn_readfirstlane(pl.seg[g + 1]) - seg0;
    const int c_lo = off / BLOCK_ROWS;
    v16f acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = v16f{0};
    for (int s = 0; s < nblk; ++s) {
      const int c = c_lo + s;
      const float sc = p.scprod[c];
      int lo, hi;
      block_rows(c, off, cnt, lo, hi);
      const bool live = sc != 0.0f;
      const __amdgpu_buffer_rsrc_t ra =
          make_rsrc(p.a + (int64_t)lo * p.Kout + k0, live ? (uint32_t)((hi - lo) * p.Kout - k0) : 0u);
      const __amdgpu_buffer_rsrc_t rb =
          make_rsrc(p.b + (int64_t)lo * p.Nout + n0, live ? (uint32_t)((hi - lo) * p.Nout - n0) : 0u);
      const int skip = lo - c * BLOCK_ROWS;
      v4u va[4], vb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t r = (uint32_t)(lrow + 32 * q - skip);  // wraps for rows before the group
        va[q] = buf_load16(ra, r * (uint32_t)p.Kout + lch * 16);
        vb[q] = buf_load16(rb, r * (uint32_t)p.Nout + lch * 16);
      }
      __syncthreads();  // the previous block's fragment reads are done
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        *reinterpret_cast<v4u*>(sA + q * 32 * PROWB + wofs) = va[q];
        *reinterpret_cast<v4u*>(sB + q * 32 * PROWB + wofs) = vb[q];
      }
      __syncthreads();
      v16f part[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) part[b] = v16f{0};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v8i a2[2], b2[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a2[i] = frag_tr8<PROWB>(sA + fa[i] + ks * 64 * PROWB);
          b2[i] = frag_tr8<PROWB>(sB + fb[i] + ks * 64 * PROWB);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            part[2 * i + j] = mfma32x32x64<B_FMT, A_FMT>(b2[j], a2[i], part[2 * i + j]);
      }
      if (live) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[b][e] = add_rn(acc[b][e], mul_rn(part[b][e], sc));
      }
    }
    __syncthreads();  // the next tile's LDS writes wait for this tile's reads
    // store: lane holds out[k = base + lane%32][n = base + 8*(r/4) + 4*(lane/32) + r%4]
    const int64_t slab = (int64_t)g * p.Kout * p.Nout;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int i = blk >> 1, j = blk & 1;
      const int k = k0 + wr * 64 + i * 32 + frow;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = n0 + wc * 64 + j * 32 + 8 * r4 + 4 * fhalf;
        const int64_t idx = slab + (int64_t)k * p.Nout + n;
        if (p.out_f32) {
          v4f v = {acc[blk][4 * r4], acc[blk][4 * r4 + 1], acc[blk][4 * r4 + 2], acc[blk][4 * r4 + 3]};
          *reinterpret_cast<v4f*>((float*)p.out + idx) = v;
        } else {
          v2u v;
          v.x = pack_bf16x2(acc[blk][4 * r4], acc[blk][4 * r4 + 1]);
          v.y = pack_bf16x2(acc[blk][4 * r4 + 2], acc[blk][4 * r4 + 3]);
          *reinterpret_cast<v2u*>((uint16_t*)p.out + idx) = v;
        }
      }
    }
  }
}

template <int A_FMT, int B_FMT>
hipError_t launch_tgmm_fp8(const TgmmCodesParams& p, hipStream_t st) {
  // per group T tiles in 8 chunks of ceil(T / 8), one per XCD
  const int64_t T = (int64_t)((p.Kout + MBK - 1) / MBK) * ((p.Nout + MBN - 1) / MBN);
  const int64_t tiles = 8 * ((T + 7) / 8) * p.G;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((tgmm_main_kernel<A_FMT, B_FMT>), dim3((unsigned)tiles), dim3(MNT), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one workgroup per CU at most (a grid-stride loop): when no group is wide, every
  // workgroup returns at once and one round of them costs next to nothing
  const int64_t ptiles = (int64_t)(p.Kout / PBK) * (p.Nout / PBK) * p.G;
  hipLaunchKernelGGL((tgmm_promote_kernel<A_FMT, B_FMT>), dim3((unsigned)(ptiles < 256 ? ptiles : 256)),
                     dim3(PNT), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tgmm(int a_fmt, int b_fmt, const TgmmParams& p, hipStream_t st) {
  const OpScale a_sc{p.a_scale_blk, p.a_scale_static, p.a_inv_static, p.a_codes};
  const OpScale b_sc{p.b_scale_blk, p.b_scale_static, p.b_inv_static, p.b_codes};
  hipLaunchKernelGGL(tgmm_plan_kernel, dim3(1), dim3(PLAN_NT), 0, st, p.group_sizes, p.g_before,
                     p.G, p.M, a_sc, b_sc, p.plan, p.scprod, p.ratio);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // a bf16 operand is quantized once, row-major, into the workspace
  if (p.M > 0 && !p.a_codes) {
    e = launch_quantize_rows(a_fmt, p.a, p.M, p.Kout, p.a_scale_blk, p.a_inv_static, p.a_q, st);
    if (e != hipSuccess) return e;
  }
  if (p.M > 0 && !p.b_codes) {
    e = launch_quantize_rows(b_fmt, p.b, p.M, p.Nout, p.b_scale_blk, p.b_inv_static, p.b_q, st);
    if (e != hipSuccess) return e;
  }
  TgmmCodesParams q{};
  q.a = p.a_codes ? (const uint8_t*)p.a : p.a_q;
  q.b = p.b_codes ? (const uint8_t*)p.b : p.b_q;
  q.plan = p.plan;
  q.scprod = p.scprod;
  q.ratio = p.ratio;
  q.out = p.out;
  q.Kout = p.Kout;
  q.Nout = p.Nout;
  q.G = p.G;
  q.out_f32 = p.out_f32;
  if (a_fmt == FMT_E4M3 && b_fmt == FMT_E5M2) return launch_tgmm_fp8<FMT_E4M3, FMT_E5M2>(q, st);
  if (a_fmt == FMT_E4M3 && b_fmt == FMT_E4M3) return launch_tgmm_fp8<FMT_E4M3, FMT_E4M3>(q, st);
  if (a_fmt == FMT_E5M2 && b_fmt == FMT_E5M2) return launch_tgmm_fp8<FMT_E5M2, FMT_E5M2>(q, st);
  if (a_fmt == FMT_E5M2 && b_fmt == FMT_E4M3) return launch_tgmm_fp8<FMT_E5M2, FMT_E4M3>(q, st);
  return hipErrorInvalidValue;
}

}  // namespace gmm
