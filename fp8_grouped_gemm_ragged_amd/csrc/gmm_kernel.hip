// Ragged grouped GEMM with FP8 operands on gfx950: the kernel behind gmm_fwd and
// gmm_dlhs.
//
//   out[m, n] = RNE_out( (sum_k q(A)[m, k] * B_g[k, n]) * s_A(m) * s_B[g, n] )
//
// for every row m of group g.  The forward product (PR #3770 "FP8 Megablox for batch
// split", Description (1)) uses A = lhs, B = rhs[g]; the lhs gradient (PR #4451
// "Support quantization for tokamax gmm v2", the dlhs call with transpose_rhs flipped)
// uses A = grad and B = rhs[g]^T.  Both are this one kernel with different strides.
//
// Work decomposition (one workgroup = one 256 x 256 output tile, 4 waves):
//   * expert-tile scheduler: every workgroup prefix-sums group_sizes into per-group
//     M-tile counts ceil(m_g / 256) (in each wave's registers for up to 64 groups, else in
//     LDS); a tile never spans two groups, empty groups own no tile, and workgroups past
//     the real tile count exit at once;
//   * XCD-aware order: the hardware places workgroup i on XCD i % 8, so workgroup ids
//     are remapped to give each XCD a contiguous range of tiles, ordered in bands of 8
//     M-tiles sweeping the N-tiles: the 32 concurrent tiles of one XCD share A rows and
//     B columns in that XCD's L2;
//   * tail split (with its workspace): when an XCD's last round of tiles is partly
//     empty, those tiles are cut along the contraction into slices run by the idle CUs,
//     and gmm_split_fixup adds the fp32 partial sums in slice order;
//   * K-loop over 128-byte contraction steps with two LDS stages (2 x 64 KB).  Every
//     operand is prefetched two steps ahead into registers with range-checked 16-byte
//     buffer loads (rows past the group end read as zero) and stored into the swizzled
//     LDS tile one step later; a bf16 A operand is quantized in registers on the way;
//   * each wave owns a 128 x 128 sub-tile: 4 x 4 MFMA 32x32x64 fp8 instructions per
//     64-deep half step, fp32 accumulators in AGPRs.  The loop body is one basic block
//     and the quantization of the next step (about 14 VALU instructions per MFMA) is
//     interleaved between the MFMAs, so vector ALU and matrix core run concurrently;
//   * epilogue: (acc * s_A(m)) * s_B(n), RNE to bf16 (or f32), stored only for rows
//     inside the group and columns inside N; bf16 rows are staged through LDS so that
//     every store instruction writes whole 128-byte lines.
#include <algorithm>

#include "kernels.hpp"

namespace gmm {

namespace {

constexpr int BM = 256, BN = 256, BK = TILE_K;
constexpr int NT = 256;
constexpr int A_TILE = BM * BK;                // bytes of one fp8 A tile
constexpr int B_TILE = BN * BK;
constexpr int BAND = 8;                        // M-tiles per band of the tile order

struct TileCoord {
  int g, row0, row_end, n0;
};

// Per-group prefix sums into LDS (first wave) over the window of G groups that starts
// after g_before others: s_tile_cum[g] = M-tiles of window groups < g, s_row_off[g] = the
// first row of window group g (rows of every group before it, inside or outside the
// window), both clamped so that sizes outside the contract never place a tile outside
// rows [0, M).  The caller synchronizes before reading them.
__device__ inline void group_prefix(const int32_t* __restrict__ gs, int g_before, int G, int64_t M,
                                    int* s_tile_cum, int* s_row_off) {
  if (threadIdx.x < 64) {
    const uint32_t Mu = (uint32_t)M;  // M < 2^31
    group_tiles_prefix<BM>(gs + g_before, G, Mu, rows_of_groups(gs, g_before, Mu), s_tile_cum,
                           s_row_off);
  }
}

// Tile L of the tile order: bands of BAND M-tiles, the M-tile index fastest inside a band,
// so the tiles one XCD runs together share A rows and B columns in its L2.  Returns false
// when the tile holds no row (group sizes that overrun M).  Every lane gets the same
// tile; the fields come back wave-uniform (scalar registers).
__device__ inline bool tile_coord(int L, int total_mt, int n_ntiles, int G, int64_t M,
                                  const int* s_tile_cum, const int* s_row_off, TileCoord& tc) {
  const int band = L / (BAND * n_ntiles);
  const int rem = L - band * BAND * n_ntiles;
  const int mt0 = band * BAND;
  const int gm = min(BAND, total_mt - mt0);
  const int nt = rem / gm;
  const int mt = mt0 + (rem - nt * gm);
  // group owning global M-tile mt: s_tile_cum[g] <= mt < s_tile_cum[g + 1]
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_tile_cum[mid] <= mt) lo = mid; else hi = mid;
  }
  tc.g = __builtin_amdgcn_readfirstlane(lo);
  tc.row0 = __builtin_amdgcn_readfirstlane(s_row_off[lo] + (mt - s_tile_cum[lo]) * BM);
  tc.row_end = __builtin_amdgcn_readfirstlane((int)min((int64_t)s_row_off[lo + 1], M));
  tc.n0 = __builtin_amdgcn_readfirstlane(nt * BN);
  return tc.row0 < tc.row_end;
}

// The tail split.  Each XCD works through its range of the tile order in rounds of
// SPLIT_CUS tiles (its CUs).  When at least one round is full and the last one is not,
// the last round's tiles are cut along the contraction into s slices each (s = the most
// that fit the round, at most SPLIT_MAX, at least 2 steps per slice), one workgroup per
// slice: the CUs that would idle through the last round share its work instead.  Only
// when that shortens the round by SPLIT_MIN_SAVED steps or more.  Slices
// store fp32 partial sums, and gmm_split_fixup adds them in slice order and finishes
// the tiles.  The split depends on the shapes and group sizes only, never on the
// device, so every call of a shape gives the same bits.
struct XcdSplit {
  int lo, len;    // the XCD's range of the tile order
  int full;       // tiles in whole rounds (run uncut)
  int tail, s;    // tiles in the last round and slices per tile (s = 1: no split)
};

__device__ inline XcdSplit xcd_split(int total, int xcd, int nk, bool split) {
  XcdSplit x;
  const int q = total >> 3, r = total & 7;
  x.lo = xcd * q + min(xcd, r);
  x.len = q + (xcd < r ? 1 : 0);
  x.full = x.len;
  x.tail = 0;
  x.s = 1;
  if (split && x.len > SPLIT_CUS && x.len % SPLIT_CUS != 0) {
    const int tail = x.len % SPLIT_CUS;
    const int s = min(min(SPLIT_CUS / tail, SPLIT_MAX), nk / 2);
    if (s >= 2 && nk - nk / s >= SPLIT_MIN_SAVED) {
      x.full = x.len - tail;
      x.tail = tail;
      x.s = s;
    }
  }
  return x;
}

// The contraction slice [kb, ke) (of nk steps) of slice `slice` out of s.
__device__ inline void slice_steps(int slice, int s, int nk, int& kb, int& ke) {
  kb = slice * nk / s;
  ke = (slice + 1) * nk / s;
}

// Expert-tile scheduler of the one-tile-per-workgroup kernel.  Returns false for a
// workgroup without work.  Otherwise tc is its tile, [kb, ke) its contraction steps and
// slot the partial-sum slot it stores (-1: the whole contraction, finished here).  The
// two LDS arrays alias the stage buffers: they are dead once the work is known.
__device__ inline bool schedule_tile(const int32_t* __restrict__ gs, int g_before, int G,
                                     int64_t M, int n_ntiles, int nk, bool split,
                                     int* s_tile_cum, int* s_row_off, TileCoord& tc, int& kb,
                                     int& ke, int& slot) {
  // Up to 64 groups, every wave computes the prefix sums itself, lane g holding group g's
  // (the same clamped sums as group_tiles_prefix), and finds its tile's group with a
  // ballot: no LDS and no workgroup barrier before the prologue.  More groups take the
  // prefix sums in LDS and a binary search.
  const bool in_wave = G <= 64;
  const int lane = threadIdx.x & 63;
  uint32_t w_start = 0, w_end = 0;
  int w_cum_ex = 0, total_mt;
  if (in_wave) {
    const uint32_t Mu = (uint32_t)M;  // M < 2^31
    const uint32_t rb = rows_of_groups(gs, g_before, Mu);
    const uint32_t m = lane < G ? (uint32_t)min(max(gs[g_before + lane], 0), (int)Mu) : 0u;
    const uint32_t ir = wave_incl_scan_sat(m, lane, Mu);
    const uint32_t up = (uint32_t)__shfl_up(ir, 1, 64);
    w_end = min(rb + ir, Mu);
    w_start = min(rb + (lane == 0 ? 0u : up), Mu);
    const int tiles = (int)((w_end - w_start + BM - 1) / BM);
    const int it = wave_incl_scan(tiles, lane);
    w_cum_ex = it - tiles;
    total_mt = __builtin_amdgcn_readlane(it, 63);  // lanes past G add no tile
  } else {
    group_prefix(gs, g_before, G, M, s_tile_cum, s_row_off);
    __syncthreads();
    total_mt = s_tile_cum[G];
  }
  // tile L of the order (tile_coord's arithmetic on the wave's sums)
  auto coord = [&](int L) -> bool {
    if (!in_wave) return tile_coord(L, total_mt, n_ntiles, G, M, s_tile_cum, s_row_off, tc);
    const int band = L / (BAND * n_ntiles);
    const int rem = L - band * BAND * n_ntiles;
    const int mt0 = band * BAND;
    const int gm = min(BAND, total_mt - mt0);
    const int nt = rem / gm;
    const int mt = mt0 + (rem - nt * gm);
    // the last group whose first M-tile is at or before mt (lane 0's is 0)
    const uint64_t below = __ballot(lane < G && w_cum_ex <= mt);
    const int lo = 63 - __builtin_clzll(below);
    tc.g = lo;
    tc.row0 = (int)__builtin_amdgcn_readlane(w_start, lo) + (mt - __builtin_amdgcn_readlane(w_cum_ex, lo)) * BM;
    tc.row_end = (int)__builtin_amdgcn_readlane(w_end, lo);
    tc.n0 = nt * BN;
    return tc.row0 < tc.row_end;
  };
  const int total = total_mt * n_ntiles;
  // XCD-aware remap: workgroups of XCD x = wg % 8 take a contiguous range of tiles
  const int wg = blockIdx.x, xcd = wg & 7, j = wg >> 3;
  const XcdSplit x = xcd_split(total, xcd, nk, split);
  bool ok = false;
  kb = 0;
  ke = nk;
  slot = -1;
  if (j < x.full) {
    ok = coord(x.lo + j);
  } else if (j - x.full < x.tail * x.s) {
    const int t = j - x.full;
    ok = coord(x.lo + x.full + t / x.s);
    slice_steps(t % x.s, x.s, nk, kb, ke);
    slot = xcd * SPLIT_CUS + t;
  }
  if (!in_wave) __syncthreads();  // the scheduler arrays alias stage memory
  // every lane computed the same work: make that visible to the compiler, so the buffer
  // resources built from it live in scalar registers
  tc.g = __builtin_amdgcn_readfirstlane(tc.g);
  tc.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
  tc.row_end = __builtin_amdgcn_readfirstlane(tc.row_end);
  tc.n0 = __builtin_amdgcn_readfirstlane(tc.n0);
  kb = __builtin_amdgcn_readfirstlane(kb);
  ke = __builtin_amdgcn_readfirstlane(ke);
  slot = __builtin_amdgcn_readfirstlane(slot);
  return __builtin_amdgcn_readfirstlane((int)ok) != 0;
}

// Thread t's epilogue scales of a tile: row row0 + t and column n0 + t (SW: columns
// 0..127 are the gate channels c0.., 128..255 the up channels I + c0..).
template <bool SW>
__device__ __forceinline__ void tile_scales(const GemmParams& p, const TileCoord& tc, int tid, float& sa_t,
                                   float& sb_t) {
  const int m = max(min(tc.row0 + tid, tc.row_end - 1), 0);
  sa_t = p.a_scale_blk ? p.a_scale_blk[m / BLOCK_ROWS] : p.a_scale_static;
  const int c0 = tc.n0 >> 1;
  const int n = SW ? (tid < 128 ? c0 + tid : (p.Nout >> 1) + c0 + tid - 128)
                   : min(tc.n0 + tid, p.Nout - 1);
  sb_t = p.b_scale[(int64_t)tc.g * p.Nout + n];
}

// Epilogue of a 256 x 256 tile: out = RNE((acc * s_A(m)) * s_B(n)), rows inside the group
// and columns inside N only.  lane holds out[m = base_m + lane%32][n = base_n + 8*(r/4) +
// 4*(lane/32) + r%4].  The scales come from LDS (a global load issued here would also
// wait for every store issued before it: the vector-memory counter retires in order).
// bf16: each wave puts its 128 x 128 sub-tile into its own 32 KB of LDS (`wl`, [row][256
// B], 16-byte chunk c of row r at c ^ (r & 15)), then stores whole rows, 16 lanes per row
// and 16 bytes per lane: every store instruction writes 8 full 128-byte lines instead of
// 16-byte pieces of 32 rows.  Nothing else may touch wl meanwhile.
__device__ __forceinline__ void store_tile(const GemmParams& p, const TileCoord& tc, v16f (&acc)[4][4],
                                  const float* s_sa, const float* s_sb, uint8_t* wl) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1, frow = lane & 31, fhalf = lane >> 5;
  float sa[4];
  v4f sb[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sa[i] = s_sa[wr * 128 + i * 32 + frow];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      sb[j][r4] = *reinterpret_cast<const v4f*>(s_sb + wc * 128 + j * 32 + 8 * r4 + 4 * fhalf);
  if (!p.out_f32) {
    // SwiGLU backward in the epilogue: the first 8 rows' gate and up values are loaded
    // now, so that their latency hides under the conversion below (the wave's columns lie
    // all inside the output or all outside it)
    const bool bwd = p.bwd_gu != nullptr && tc.n0 + wc * 128 < p.Nout;
    const int c = lane & 15;
    const int rows_here = min(tc.row_end - tc.row0, BM);
    __amdgpu_buffer_rsrc_t rg = make_rsrc(nullptr, 0u);
    uint32_t g_off = 0;
    v4u gv[2][8], uv[2][8];
    // gu rows of the tile inside the group: rows past its end read zeros (offsets below
    // 2^31: 256 rows x 2 Nout <= 2^22 columns x 2 bytes)
    const uint32_t two_i = 2u * (uint32_t)p.Nout;
    auto bwd_load = [&](int set, int q0) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t o = g_off + (uint32_t)(q0 + t) * 8u * two_i;
        gv[set][t] = buf_load16(rg, o);
        uv[set][t] = buf_load16(rg, o + 2u * (uint32_t)p.Nout);
      }
    };
    if (bwd) {
      rg = make_rsrc(p.bwd_gu + (int64_t)tc.row0 * two_i, (uint32_t)rows_here * two_i * 2u);
      g_off = ((uint32_t)(wr * 128 + (lane >> 4)) * two_i + (uint32_t)(tc.n0 + wc * 128 + c * 8)) * 2u;
      bwd_load(0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i * 32 + frow;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = __fmul_rn(__fmul_rn(acc[i][j][4 * r4 + e], sa[i]), sb[j][r4][e]);
          v2u v;
          v.x = pack_bf16x2(o[0], o[1]);
          v.y = pack_bf16x2(o[2], o[3]);
          const int chunk = (4 * j + r4) ^ (row & 15);
          *reinterpret_cast<v2u*>(wl + row * 256 + chunk * 16 + fhalf * 8) = v;
        }
      }
    }
    // this wave's LDS writes are done before its own reads (no other wave touches wl)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // the wave's 128 columns lie all inside N or all outside it (N is a multiple of 128)
    if (tc.n0 + wc * 128 >= p.Nout) return;
    if (bwd) {
      // d_gu rows through a resource over the tile's rows of the group (rows past its end
      // are dropped), 4 rows per instruction, 16 lanes per row, 8 channels per lane; the
      // next 8 rows' gate and up loads go out before this batch's stores (the
      // vector-memory counter retires in order)
      const __amdgpu_buffer_rsrc_t rd =
          make_rsrc((uint16_t*)p.out + (int64_t)tc.row0 * two_i, (uint32_t)rows_here * two_i * 2u);
      // block abs-max of the values written: the wave's 128 rows meet at most two
      // 128-row blocks, blk0 and blk0 + 1 (rows past the group's end hold zeros)
      const int wrow0 = tc.row0 + wr * 128;
      const int blk0 = wrow0 >> 7;
      uint32_t am0 = 0u, am1 = 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int set = b & 1;
        if (b < 3) bwd_load(set ^ 1, (b + 1) * 8);
        v4u d[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int row = (b * 8 + t) * 4 + (lane >> 4);
          d[t] = *reinterpret_cast<const v4u*>(wl + row * 256 + ((c ^ (row & 15)) << 4));
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          v4u og, ou;
          swiglu_bwd8(d[t], gv[set][t], uv[set][t], og, ou);
          const uint32_t o = g_off + (uint32_t)(b * 8 + t) * 8u * two_i;
          buf_store16(rd, o, og);
          buf_store16(rd, o + 2u * (uint32_t)p.Nout, ou);
          const uint32_t mm = absmax_bits16(og, absmax_bits16(ou, 0u));
          if (((wrow0 + (b * 8 + t) * 4 + (lane >> 4)) >> 7) == blk0) am0 = max(am0, mm);
          else am1 = max(am1, mm);
        }
      }
      if (p.bwd_amax) {
#pragma unroll
        for (int dd = 32; dd >= 1; dd >>= 1) {
          am0 = max(am0, (uint32_t)__shfl_xor((int)am0, dd, 64));
          am1 = max(am1, (uint32_t)__shfl_xor((int)am1, dd, 64));
        }
        // one vector atomic per block from lane 0; a zero maximum changes nothing
        if (lane == 0) {
          if (am0) atomicMax(p.bwd_amax + blk0, am0);
          if (am1) atomicMax(p.bwd_amax + blk0 + 1, am1);
        }
      }
      return;
    }
    // Stores through a resource over the tile's rows of the group: rows past the group's
    // end fall outside its range and are dropped, so no store needs a per-lane branch.
    // Byte offsets stay below 2^31 (256 rows x N <= 2^22 columns x 2 bytes).
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((uint16_t*)p.out + (int64_t)tc.row0 * p.Nout,
                                                (uint32_t)rows_here * (uint32_t)p.Nout * 2u);
    const uint32_t lane_off =
        ((uint32_t)(wr * 128 + (lane >> 4)) * (uint32_t)p.Nout + (uint32_t)(tc.n0 + wc * 128 + c * 8)) * 2u;
    const uint32_t q_stride = 8u * (uint32_t)p.Nout;  // 4 rows
    // eight rows' LDS reads in flight before their stores
#pragma unroll
    for (int q0 = 0; q0 < 32; q0 += 8) {
      v4u v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int row = (q0 + t) * 4 + (lane >> 4);
        v[t] = *reinterpret_cast<const v4u*>(wl + row * 256 + ((c ^ (row & 15)) << 4));
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) buf_store16(ro, lane_off + (uint32_t)(q0 + t) * q_stride, v[t]);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = tc.row0 + wr * 128 + i * 32 + frow;
    if (m >= tc.row_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = tc.n0 + wc * 128 + j * 32 + 8 * r4 + 4 * fhalf;
        if (n >= p.Nout) continue;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __fmul_rn(__fmul_rn(acc[i][j][4 * r4 + e], sa[i]), sb[j][r4][e]);
        v4f v = {o[0], o[1], o[2], o[3]};
        *reinterpret_cast<v4f*>((float*)p.out + (int64_t)m * p.Nout + n) = v;
      }
    }
  }
}

// A partial-sum slot: one 256 x 256 fp32 tile, [row][column].
__device__ inline float* split_slot(const GemmParams& p, int slot) {
  return p.split_ws + (size_t)slot * (BM * BN);
}

// SwiGLU epilogue of a gate|up tile.  The product values x = (acc * s_A(m)) * s_B(n) are
// the ones gmm_fwd stores (written to gu when given).  The gate and up waves of a row
// half exchange half of their values through LDS, in the lane order every wave's
// accumulators share, and each then stores h = silu(g) * u = (g / (1 + exp(-g))) * u for
// 64 of the 128 rows, all in fp32: in the output dtype, or as fp8 codes
// fp8(clamp(RNE_f32(h * inv), +-qmax)) of a static scale.
__device__ inline void swiglu_epilogue(const GemmParams& p, const TileCoord& tc, int c0, int wr,
                                       int wc, v16f (&acc)[4][4], uint8_t* sA0,
                                       uint8_t* sB0, uint8_t* sA1, uint8_t* sB1,
                                       const float* s_sa, const float* s_sb) {
  // the lane id is recomputed here: cheaper than keeping it live across the main loop
  const int lane = __lane_id();
  const int frow = lane & 31, fhalf = lane >> 5;
  const int I = p.Nout >> 1;
  const int cb = wc == 0 ? c0 : I + c0;  // this wave's first channel
  // the tile's row scales and its gate (0..127) and up (128..255) channel scales, put
  // into LDS by the prologue
  float sa[4];
  v4f sb[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sa[i] = s_sa[wr * 128 + i * 32 + frow];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      sb[j][r4] = *reinterpret_cast<const v4f*>(s_sb + wc * 128 + j * 32 + 8 * r4 + 4 * fhalf);
  auto value = [&](int i, int j, int r4) {
    v4f o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __fmul_rn(__fmul_rn(acc[i][j][4 * r4 + e], sa[i]), sb[j][r4][e]);
    return o;
  };
  // chunk r = 16 i + 4 j + r4 of row half wr, lane-interleaved: the gate wave finishes
  // rows i < 2 and hands over its chunks i >= 2 (region xb); the up wave finishes rows
  // i >= 2 and hands over its chunks i < 2 (region xa)
  uint8_t* const xa = wr == 0 ? sA0 : sA1;
  uint8_t* const xb = wr == 0 ? sB0 : sB1;
  auto chunk = [&](int r) { return reinterpret_cast<v4f*>((r < 32 ? xa : xb) + ((r & 31) * 64 + lane) * 16); };
  __syncthreads();  // every wave is done with the stages
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = tc.row0 + wr * 128 + i * 32 + frow;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const v4f o = value(i, j, r4);
        const int64_t idx = (int64_t)m * p.Nout + cb + j * 32 + 8 * r4 + 4 * fhalf;
        if (p.gu && m < tc.row_end) {
          if (p.out_f32) {
            *reinterpret_cast<v4f*>((float*)p.gu + idx) = o;
          } else {
            v2u v;
            v.x = pack_bf16x2(o[0], o[1]);
            v.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<v2u*>((uint16_t*)p.gu + idx) = v;
          }
        }
        if ((wc == 0) == (i >= 2)) *chunk(i * 16 + j * 4 + r4) = o;
      }
    }
  }
  __syncthreads();  // the handed-over values are in LDS
  // This wave finishes rows i0 .. i0 + 1 of its row half (64 rows x 128 channels), 32
  // rows (one ii) at a time.  Rows of ii come from the 16 KB half ii of the LDS region
  // this wave reads (no other wave touches it now); once read, that half stages the
  // rows' outputs as [32 rows][RB bytes], 16-byte chunk c of row r at c ^ (r & 15), which
  // are then stored as whole rows: every store instruction writes full lines.
  const int i0 = wc == 0 ? 0 : 2;
  uint8_t* const wl = wc == 0 ? xa : xb;
  const bool codes = p.h_codes != 0;
  const int RB = codes ? 128 : 256;             // bytes per staged row (bf16 or codes)
  const int lanes_per_row = RB / 16;            // 16 or 8
  const int rows_per_op = 64 / lanes_per_row;   // 4 or 8
  const int c = lane % lanes_per_row;
  const int swz = codes ? 7 : 15;
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) {
    v4f hv[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        // accumulator rows by constant index only (a computed index would move the
        // accumulators to scratch memory)
        v4f mine, other;
        if (wc == 0) {
          mine = value(ii, j, r4);
          other = *chunk(ii * 16 + j * 4 + r4);
        } else {
          mine = value(2 + ii, j, r4);
          other = *chunk((2 + ii) * 16 + j * 4 + r4);
        }
        const v4f g = wc == 0 ? mine : other;
        const v4f u = wc == 0 ? other : mine;
        // silu(g) = g * sigmoid(g), sigmoid(g) = 1 / (1 + e^-g) through the hardware
        // exp2 and reciprocal (about one ulp each; e^-g = 2^(-g log2 e)): two
        // transcendental instructions per value instead of the library exp and an IEEE
        // division.  Large |g| saturate as the definition does: e^-g = inf gives
        // sigmoid 0, e^-g = 0 gives 1.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float t = __builtin_amdgcn_exp2f(g[e] * -1.44269504088896341f);
          hv[j][r4][e] = (g[e] * __builtin_amdgcn_rcpf(1.0f + t)) * u[e];
        }
      }
    const int mrow = tc.row0 + wr * 128 + (i0 + ii) * 32;  // first row of these 32
    if (p.out_f32 && !codes) {
      const int m = mrow + frow;
      if (m < tc.row_end) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<v4f*>((float*)p.out + (int64_t)m * I + c0 + j * 32 + 8 * r4 + 4 * fhalf) =
                hv[j][r4];
      }
      continue;
    }
    // fp8 codes of h: under the static scale's inverse, or (h_scales) under one dynamic
    // scale per row and 128-channel block.  This tile's 128 channels are one block: the
    // lane holds 64 of its row's values and lane ^ 32 the other 64.
    float h_inv = p.h_inv;
    if (codes && p.h_scales) {
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(hv[j][r4][e]));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      const float sc = __fdiv_rn(amax, p.h_codes == 1 + FMT_E4M3 ? qmax<FMT_E4M3>() : qmax<FMT_E5M2>());
      h_inv = inv_from_scale(sc);
      const int m = mrow + frow;
      if (fhalf == 0 && m < tc.row_end) p.h_scales[(int64_t)m * (I / 128) + c0 / 128] = sc;
    }
    uint8_t* const st = wl + ii * 16384;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this half's reads are done
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const v4f h = hv[j][r4];
        if (codes) {
          // the lhs of the down projection
          const uint32_t q =
              p.h_codes == 1 + FMT_E4M3 ? quant4<FMT_E4M3>(h, h_inv) : quant4<FMT_E5M2>(h, h_inv);
          const int byte = j * 32 + 8 * r4 + 4 * fhalf;
          *reinterpret_cast<uint32_t*>(st + frow * 128 + ((((byte >> 4) ^ frow) & 7) << 4) + (byte & 15)) = q;
        } else {
          v2u v;
          v.x = pack_bf16x2(h[0], h[1]);
          v.y = pack_bf16x2(h[2], h[3]);
          *reinterpret_cast<v2u*>(st + frow * 256 + (((4 * j + r4) ^ (frow & 15)) << 4) + fhalf * 8) = v;
        }
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // stores through a resource over these 32 rows' part inside the group: rows past its
    // end fall outside the range and are dropped (offsets below 2^27)
    const uint32_t row_bytes = (uint32_t)I * (uint32_t)(RB / 128);
    const int rows_valid = max(min(tc.row_end - mrow, 32), 0);
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc((uint8_t*)p.out + ((int64_t)mrow * I + c0) * (RB / 128), (uint32_t)rows_valid * row_bytes);
    for (int q = 0; q < 32 / rows_per_op; ++q) {
      const int row = q * rows_per_op + lane / lanes_per_row;
      const v4u v = *reinterpret_cast<const v4u*>(st + row * RB + ((c ^ (row & swz)) << 4));
      buf_store16(ro, (uint32_t)row * row_bytes + (uint32_t)c * 16u, v);
    }
  }
}

// SW: the merged gate|up forward with the SwiGLU epilogue (fp8 A, contraction-contiguous
// B only).  Its tiles are 256 rows x 128 channel pairs: B rows 0..127 are gate channels
// c0..c0+127 and rows 128..255 the up channels I + c0.., so the waves with wc = 0 hold
// gate values and those with wc = 1 the matching up values of the same outputs.
template <int A_FMT, int B_FMT, bool A_FP8, bool B_TRANS, bool SW = false>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
void gmm_kernel(GemmParams p) {
  static_assert(!SW || (A_FP8 && !B_TRANS), "the SwiGLU epilogue runs on the fp8-A route");
  // one LDS object per stage and operand: the compiler then sees that stores into the
  // next stage never alias fragment reads of the current one
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[A_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[B_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[A_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[B_TILE];
  // the tile's row and column scales (beside the 128 KB of stages: 160 KB of LDS)
  __shared__ float s_sa[BM];
  __shared__ float s_sb[BN];
  int* s_tile_cum = reinterpret_cast<int*>(sA0);
  int* s_row_off = s_tile_cum + (MAX_GROUPS + 1);
  static_assert(2 * (MAX_GROUPS + 1) * sizeof(int) <= A_TILE, "scheduler arrays fit a tile");

  const int n_ntiles = SW ? (p.Nout >> 1) / 128 : (p.Nout + BN - 1) / BN;
  const int Kc = p.Kc;
  const int nk = Kc / BK;
  TileCoord tc;
  int kb, ke, slot;  // contraction steps [kb, ke); slot >= 0: a slice of a split tile
  if (!schedule_tile(p.group_sizes, p.g_before, p.G, p.M, n_ntiles, nk, !SW && p.split_ws,
                     s_tile_cum, s_row_off, tc, kb, ke, slot))
    return;
  const int c0 = SW ? (tc.n0 >> 1) : 0;  // SW: first channel pair of the tile

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  // ---- operand resources (range-checked) ----
  constexpr int AES = A_FP8 ? 1 : 2;  // bytes per A element
  const int rows_here = min(tc.row_end - tc.row0, BM);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(
      (const uint8_t*)p.a + (int64_t)tc.row0 * Kc * AES, (uint32_t)rows_here * Kc * AES);
  __amdgpu_buffer_rsrc_t rb;
  if constexpr (SW) {
    rb = make_rsrc(p.b + (int64_t)tc.g * p.Nout * Kc, (uint32_t)p.Nout * Kc);
  } else if constexpr (!B_TRANS) {
    const int cols_here = min(p.Nout - tc.n0, BN);
    rb = make_rsrc(p.b + ((int64_t)tc.g * p.Nout + tc.n0) * Kc, (uint32_t)cols_here * Kc);
  } else {
    rb = make_rsrc(p.b + (int64_t)tc.g * Kc * p.Nout + tc.n0,
                   (uint32_t)((int64_t)Kc * p.Nout - tc.n0));
  }

  // ---- bf16 A register mapping: piece i -> row i*32 + tid/8, 32-byte pair tid%8 ----
  const int lrow = tid >> 3, lchunk = tid & 7;
  float inv_row[8];
  if constexpr (!A_FP8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = tc.row0 + i * 32 + lrow;
      inv_row[i] = p.a_scale_blk ? inv_from_scale(p.a_scale_blk[min(row, tc.row_end - 1) / BLOCK_ROWS])
                                 : p.a_inv_static;
    }
  }

  // register stage of step kt+2: bf16 A pieces (2 x 16 B), fp8 A pieces (16 B), fp8 B
  // pieces (16 B) or 8x8 blocks of an output-contiguous B
  v4u a_reg[A_FP8 ? 8 : 16];
  v4u bk_reg[B_TRANS ? 1 : 8];
  v2u b_reg[B_TRANS ? 16 : 1];

  // piece i of a tile = rows 32 i .. 32 i + 31, one row per 8 lanes (row 32 i + tid/8),
  // 16 contraction bytes per lane (chunk tid%8)
  auto load_a_piece = [&](int kt, int i) {
    if constexpr (!A_FP8) {
      const uint32_t off = (uint32_t)(i * 32 + lrow) * Kc * 2 + (uint32_t)kt * BK * 2 + lchunk * 32;
      a_reg[2 * i] = buf_load16(ra, off);
      a_reg[2 * i + 1] = buf_load16(ra, off + 16);
    } else {
      a_reg[i] = buf_load16(ra, (uint32_t)(i * 32 + lrow) * Kc + (uint32_t)kt * BK + lchunk * 16);
    }
  };
  auto load_bk_piece = [&](int kt, int i) {
    if constexpr (!B_TRANS) {
      // SW: pieces 0..3 are gate channels c0.., pieces 4..7 the up channels I + c0..
      const uint32_t row = SW ? (uint32_t)((i < 4 ? c0 + i * 32 : (p.Nout >> 1) + c0 + (i - 4) * 32) + lrow)
                              : (uint32_t)(i * 32 + lrow);
      bk_reg[i] = buf_load16(rb, row * Kc + (uint32_t)kt * BK + lchunk * 16);
    }
  };
  auto load_b_block = [&](int kt, int it) {
    if constexpr (B_TRANS) {
      const int q = it * 256 + tid;
      const int nb = (q & 7) | (((q >> 4) & 3) << 3);
      const int kb = ((q >> 3) & 1) | ((q >> 6) << 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t off = (uint32_t)(kt * BK + kb * 8 + e) * p.Nout + nb * 8;
        b_reg[it * 8 + e] = __builtin_amdgcn_raw_buffer_load_b64(rb, off, 0, 0);
      }
    }
  };
  auto store_a_piece = [&](uint8_t* at, int i) {
    if constexpr (!A_FP8) {
      const v2u lo = quant8<A_FMT>(a_reg[2 * i], inv_row[i]);
      const v2u hi = quant8<A_FMT>(a_reg[2 * i + 1], inv_row[i]);
      v4u q;
      q.x = lo.x; q.y = lo.y; q.z = hi.x; q.w = hi.y;
      *reinterpret_cast<v4u*>(at + tile_off(i * 32 + lrow, lchunk)) = q;
    } else {
      *reinterpret_cast<v4u*>(at + tile_off(i * 32 + lrow, lchunk)) = a_reg[i];
    }
  };
  auto store_bk_piece = [&](uint8_t* bt, int i) {
    if constexpr (!B_TRANS) *reinterpret_cast<v4u*>(bt + tile_off(i * 32 + lrow, lchunk)) = bk_reg[i];
  };
  auto store_b_block = [&](uint8_t* bt, int it) {
    if constexpr (B_TRANS) {
      const int q = it * 256 + tid;
      const int nb = (q & 7) | (((q >> 4) & 3) << 3);
      const int kb = ((q >> 3) & 1) | ((q >> 6) << 1);
      v2u t[8];
      transpose8x8(&b_reg[it * 8], t);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<v2u*>(bt + tile_off(nb * 8 + c, kb >> 1) + (kb & 1) * 8) = t[c];
    }
  };
  // This wave's LDS stores of the stage being filled are done; then the workgroup.
  // (Global loads only feed registers, so nothing else needs to land.)
  auto stage_barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{0};

  const int frow = lane & 31, fhalf = lane >> 5;
  // Fragment addressing.  A fragment row is R = base + 32 i + frow (base a multiple of
  // 128), so its swizzle key (R & 7) ^ ((R >> 3) & 7) is f0 ^ 4 (i & 1) with
  // f0 = (frow & 7) ^ (frow >> 3), and the physical chunk of logical chunk
  // 4 ks + 2 fhalf + e is (2 fhalf + e) ^ f0 ^ 4 (ks ^ (i & 1)).  Two per-lane byte
  // offsets per e (t = ks ^ (i & 1)) plus the immediate 4096 i cover every fragment.
  uint32_t fo[2][2];
  {
    const uint32_t f0 = (uint32_t)((frow & 7) ^ (frow >> 3));
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        fo[t][e] = (uint32_t)frow * BK + ((((uint32_t)(2 * fhalf + e)) ^ f0 ^ (4u * t)) << 4);
  }
  auto frag = [&](const uint8_t* tile, int base_row, int i, int ks) -> v8i {
    const int t = ks ^ (i & 1);
    const uint8_t* p0 = tile + base_row * BK + i * 32 * BK;
    const v4u lo = *reinterpret_cast<const v4u*>(p0 + fo[t][0]);
    const v4u hi = *reinterpret_cast<const v4u*>(p0 + fo[t][1]);
    v8i f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
  };
  // Store address of quantized A piece p (row 32 p + lrow): swizzle key
  // g0 ^ 4 (p & 1) with g0 = (lrow & 7) ^ (lrow >> 3).
  uint32_t so[2];
  {
    const uint32_t g0 = (uint32_t)((lrow & 7) ^ (lrow >> 3));
#pragma unroll
    for (int t = 0; t < 2; ++t) so[t] = (uint32_t)lrow * BK + ((((uint32_t)lchunk) ^ g0 ^ (4u * t)) << 4);
  }

  // One quarter of an A piece: the 4 values that make one output dword.
  auto quant_dword = [&](int i, int d) -> uint32_t {
    const v4u w = a_reg[2 * i + (d >> 1)];
    const uint32_t w0 = (d & 1) ? w.z : w.x, w1 = (d & 1) ? w.w : w.y;
    const float inv = inv_row[i];
    uint32_t r = cvt_pk<A_FMT, false>(quant_prep<A_FMT>(bf16_lo(w0), inv),
                                      quant_prep<A_FMT>(bf16_hi(w0), inv), w0);
    return cvt_pk<A_FMT, true>(quant_prep<A_FMT>(bf16_lo(w1), inv),
                               quant_prep<A_FMT>(bf16_hi(w1), inv), r);
  };

  // One contraction step: the 32 MFMAs on stage (at, bt) = step kt, while step kt+1 is
  // completed in stage (an, bn) and step kt+2 is prefetched into registers.  The step
  // is written as 32 units of one MFMA plus one slice of register work each, fenced so
  // that the scheduler keeps the interleaving (the matrix core works through each MFMA
  // while the vector ALU runs the next slice).
  auto step = [&](int kt, const uint8_t* at, const uint8_t* bt, uint8_t* an, uint8_t* bn) {
    v8i af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = frag(at, wr * 128, i, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = frag(bt, wc * 128, j, 0);
    uint32_t qd[4];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int ks = u >> 4, i = (u >> 2) & 3, j = u & 3;
      acc[i][j] = mfma32x32x64<B_FMT, A_FMT>(bf[j], af[i], acc[i][j]);
      // fragments of the second half step, each right after its last use
      if (ks == 0 && j == 3) af[i] = frag(at, wr * 128, i, 1);
      if (ks == 0 && i == 3) bf[j] = frag(bt, wc * 128, j, 1);
      {
        // piece u/4 of step kt+1: A (quantized a quarter per MFMA), then B; each piece is
        // stored to the next stage and its registers refilled with step kt+2
        const int piece = u >> 2, d = u & 3;
        if constexpr (!A_FP8) {
          qd[d] = quant_dword(piece, d);
          if (d == 3) {
            v4u q;
            q.x = qd[0]; q.y = qd[1]; q.z = qd[2]; q.w = qd[3];
            *reinterpret_cast<v4u*>(an + piece * 32 * BK + so[piece & 1]) = q;
            load_a_piece(kt + 2, piece);
          }
        } else if (d == 1) {
          *reinterpret_cast<v4u*>(an + piece * 32 * BK + so[piece & 1]) = a_reg[piece];
          load_a_piece(kt + 2, piece);
        }
        if constexpr (!B_TRANS) {
          if (d == 2) {
            *reinterpret_cast<v4u*>(bn + piece * 32 * BK + so[piece & 1]) = bk_reg[piece];
            load_bk_piece(kt + 2, piece);
          }
        }
      }
      if constexpr (B_TRANS) {
        if (u == 7) { store_b_block(bn, 0); load_b_block(kt + 2, 0); }
        if (u == 23) { store_b_block(bn, 1); load_b_block(kt + 2, 1); }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    stage_barrier();
  };

  // ---- prologue: the tile's scales, step kb into stage 0, step kb + 1 into registers ----
  // The epilogue scales are loaded first (thread t: row row0 + t, column n0 + t) and put
  // into LDS once they land, so the epilogue reads them there instead of waiting for
  // global loads after the last step.
  float sa_t = 1.0f, sb_t = 1.0f;  // (a slice of a split tile stores unscaled sums)
  if (slot < 0) tile_scales<SW>(p, tc, tid, sa_t, sb_t);
#pragma unroll
  for (int i = 0; i < 8; ++i) { load_a_piece(kb, i); load_bk_piece(kb, i); }
  load_b_block(kb, 0);
  load_b_block(kb, 1);
  s_sa[tid] = sa_t;
  s_sb[tid] = sb_t;
#pragma unroll
  for (int i = 0; i < 8; ++i) { store_a_piece(sA0, i); store_bk_piece(sB0, i); }
  store_b_block(sB0, 0);
  store_b_block(sB0, 1);
#pragma unroll
  for (int i = 0; i < 8; ++i) { load_a_piece(kb + 1, i); load_bk_piece(kb + 1, i); }
  load_b_block(kb + 1, 0);
  load_b_block(kb + 1, 1);
  stage_barrier();

  // two steps per trip so that every LDS access names a fixed stage object; past the
  // last step the loads read zeros or in-range bytes that are never used
  int kt = kb;
  for (; kt + 1 < ke; kt += 2) {
    step(kt, sA0, sB0, sA1, sB1);
    step(kt + 1, sA1, sB1, sA0, sB0);
  }
  if (kt < ke) step(kt, sA0, sB0, sA1, sB1);

  if constexpr (SW) {
    swiglu_epilogue(p, tc, c0, wr, wc, acc, sA0, sB0, sA1, sB1, s_sa, s_sb);
  } else {
    // A slice of a split tile stores its fp32 partial sums unscaled (its LDS scales are
    // 1) as a plain [256][256] tile in its slot, for gmm_split_fixup to finish.  The
    // last step ended with a workgroup barrier after every wave's last LDS access, so
    // all stage memory is free: 32 KB per wave.
    GemmParams q = p;
    TileCoord t = tc;
    if (slot >= 0) {
      q.out = split_slot(p, slot);
      q.Nout = BN;
      q.out_f32 = 1;
      t.row0 = 0;
      t.row_end = BM;
      t.n0 = 0;
    }
    store_tile(q, t, acc, s_sa, s_sb, wave == 0 ? sA0 : wave == 1 ? sB0 : wave == 2 ? sA1 : sB1);
  }
}

// Finishes the tiles that the tail split cut into slices.  Workgroup (xcd, t, part) takes
// rows 32 part .. 32 part + 31 of tile t of that XCD's last round: it recomputes the split
// from group_sizes exactly as gmm_kernel did, adds the slices' partial sums in slice
// order, and applies the epilogue's arithmetic (RNE((sum * s_A(m)) * s_B(n)), rows of the
// group and columns inside N only), element by element: thread (r, c) takes 8 consecutive
// columns 8c.. of rows r, r + 8, .., so that every load and store is a contiguous run.
constexpr int FIX_PARTS = BM / 32;

__global__ __launch_bounds__(NT) void gmm_split_fixup_kernel(GemmParams p) {
  __shared__ int s_tile_cum[MAX_GROUPS + 1];
  __shared__ int s_row_off[MAX_GROUPS + 1];
  const int n_ntiles = (p.Nout + BN - 1) / BN;
  const int nk = p.Kc / BK;
  group_prefix(p.group_sizes, p.g_before, p.G, p.M, s_tile_cum, s_row_off);
  __syncthreads();
  const int total_mt = s_tile_cum[p.G];
  const int part = blockIdx.x % FIX_PARTS, tx = blockIdx.x / FIX_PARTS;
  const int xcd = tx & 7, t = tx >> 3;
  const XcdSplit x = xcd_split(total_mt * n_ntiles, xcd, nk, true);
  if (__builtin_amdgcn_readfirstlane((int)(t < x.tail)) == 0) return;
  TileCoord tc;
  if (!tile_coord(x.lo + x.full + t, total_mt, n_ntiles, p.G, p.M, s_tile_cum, s_row_off, tc))
    return;
  const int tid = threadIdx.x, c = tid & 31;
  const int n = tc.n0 + 8 * c;
  if (n >= p.Nout) return;
  v4f sb[2];
  sb[0] = *reinterpret_cast<const v4f*>(p.b_scale + (int64_t)tc.g * p.Nout + n);
  sb[1] = *reinterpret_cast<const v4f*>(p.b_scale + (int64_t)tc.g * p.Nout + n + 4);
  const int slot0 = xcd * SPLIT_CUS + t * x.s;
  for (int rr = 0; rr < 4; ++rr) {
    const int row = part * 32 + rr * 8 + (tid >> 5);  // row of the tile
    const int m = tc.row0 + row;
    if (m >= tc.row_end) break;
    float v[8];
    for (int k = 0; k < x.s; ++k) {
      const float* const src = split_slot(p, slot0 + k) + row * BN + 8 * c;
      const v4f lo = *reinterpret_cast<const v4f*>(src);
      const v4f hi = *reinterpret_cast<const v4f*>(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = k == 0 ? lo[e] : __fadd_rn(v[e], lo[e]);
        v[4 + e] = k == 0 ? hi[e] : __fadd_rn(v[4 + e], hi[e]);
      }
    }
    const float sa = p.a_scale_blk ? p.a_scale_blk[m / BLOCK_ROWS] : p.a_scale_static;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = __fmul_rn(__fmul_rn(v[e], sa), sb[e >> 2][e & 3]);
    if (p.out_f32) {
      float* const dst = (float*)p.out + (int64_t)m * p.Nout + n;
      *reinterpret_cast<v4f*>(dst) = v4f{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<v4f*>(dst + 4) = v4f{o[4], o[5], o[6], o[7]};
    } else {
      v4u w;
      w.x = pack_bf16x2(o[0], o[1]);
      w.y = pack_bf16x2(o[2], o[3]);
      w.z = pack_bf16x2(o[4], o[5]);
      w.w = pack_bf16x2(o[6], o[7]);
      *reinterpret_cast<v4u*>((uint16_t*)p.out + (int64_t)m * p.Nout + n) = w;
    }
  }
}

// Rows outside a group window: [0, first row of the window) and [its end, M), written
// with zeros.  Every workgroup sums the group sizes itself (at most GMM_MAX_GROUPS).
__global__ __launch_bounds__(256) void zero_rows_outside_kernel(uint8_t* __restrict__ out,
                                                                int64_t M, int64_t row_bytes,
                                                                const int32_t* __restrict__ gs,
                                                                int g_before, int G) {
  __shared__ int64_t s_part[2][4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int64_t before = 0, inside = 0;
  for (int g = tid; g < g_before + G; g += 256) {
    const int64_t m = max(gs[g], 0);
    if (g < g_before) before += m; else inside += m;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    before += __shfl_xor(before, d, 64);
    inside += __shfl_xor(inside, d, 64);
  }
  if (lane == 0) {
    s_part[0][w] = before;
    s_part[1][w] = inside;
  }
  __syncthreads();
  const int64_t lo = min(s_part[0][0] + s_part[0][1] + s_part[0][2] + s_part[0][3], M);
  const int64_t hi = min(lo + s_part[1][0] + s_part[1][1] + s_part[1][2] + s_part[1][3], M);
  const int64_t vecs = row_bytes / 16;
  const int64_t total = (lo + (M - hi)) * vecs;
  const v4u z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / vecs, v = i - r * vecs;
    const int64_t row = r < lo ? r : hi + (r - lo);
    *reinterpret_cast<v4u*>(out + row * row_bytes + v * 16) = z;
  }
}

template <int A_FMT, int B_FMT, bool A_FP8, bool B_TRANS>
hipError_t launch_one(const GemmParams& p, hipStream_t st) {
  // upper bound on M-tiles: sum ceil(m_g/BM) <= ceil(M/BM) + G
  const int64_t max_mt = (p.M + BM - 1) / BM + p.G;
  const int64_t n_nt = (p.Nout + BN - 1) / BN;
  const int64_t tiles = max_mt * n_nt;
  if (tiles == 0 || p.M == 0) return hipSuccess;
  // with the tail split, each XCD's slices of its last round may reach SPLIT_CUS - 1
  // workgroups past the end of its range
  const int64_t grid = tiles + (p.split_ws ? SPLIT_SLOTS : 0);
  hipLaunchKernelGGL((gmm_kernel<A_FMT, B_FMT, A_FP8, B_TRANS>), dim3((unsigned)grid), dim3(NT),
                     0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.split_ws) return e;
  hipLaunchKernelGGL(gmm_split_fixup_kernel, dim3(SPLIT_SLOTS * FIX_PARTS), dim3(NT), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_swiglu(int a_fmt, const GemmParams& p, hipStream_t st) {
  const int64_t max_mt = (p.M + BM - 1) / BM + p.G;
  const int64_t grid = max_mt * ((p.Nout / 2) / 128);
  if (grid == 0 || p.M == 0) return hipSuccess;
  if (a_fmt == FMT_E4M3)
    hipLaunchKernelGGL((gmm_kernel<FMT_E4M3, FMT_E4M3, true, false, true>), dim3((unsigned)grid),
                       dim3(NT), 0, st, p);
  else if (a_fmt == FMT_E5M2)
    hipLaunchKernelGGL((gmm_kernel<FMT_E5M2, FMT_E4M3, true, false, true>), dim3((unsigned)grid),
                       dim3(NT), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_zero_rows_outside(void* out, int64_t M, int64_t row_bytes,
                                   const int32_t* gs, int g_before, int G, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const int64_t pieces = M * (row_bytes / 16);
  const int64_t blocks = std::min<int64_t>((pieces + 255) / 256, 256 * 16);
  hipLaunchKernelGGL(zero_rows_outside_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     (uint8_t*)out, M, row_bytes, gs, g_before, G);
  return hipGetLastError();
}

hipError_t launch_gemm(int a_fmt, int b_fmt, bool a_fp8, bool b_trans, const GemmParams& p,
                       hipStream_t st) {
  if (b_fmt != FMT_E4M3) return hipErrorInvalidValue;
#define GMM_DISPATCH(AF, AQ, BT)                                       \
  if (a_fmt == AF && a_fp8 == AQ && b_trans == BT)                     \
    return launch_one<AF, FMT_E4M3, AQ, BT>(p, st);
  GMM_DISPATCH(FMT_E4M3, false, false)
  GMM_DISPATCH(FMT_E4M3, false, true)
  GMM_DISPATCH(FMT_E4M3, true, false)
  GMM_DISPATCH(FMT_E4M3, true, true)
  GMM_DISPATCH(FMT_E5M2, false, false)
  GMM_DISPATCH(FMT_E5M2, false, true)
  GMM_DISPATCH(FMT_E5M2, true, false)
  GMM_DISPATCH(FMT_E5M2, true, true)
#undef GMM_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace gmm
