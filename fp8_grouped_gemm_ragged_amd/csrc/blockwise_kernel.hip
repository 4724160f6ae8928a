// Forward grouped matmul with block-wise scales on gfx950 ("Support quantization for
// tokamax gmm v2", review thread on the ops diff: a 3-D weight scale is block-wise
// quantization; "add static LHS scaling support for GMM v2 FWD", review thread on the
// lhs docstring: lhs scales of shape [M, num_blocks]).
//
// Block kb covers contraction elements [kb bk, (kb + 1) bk); the weight scale is
// sB[g, kb, n] and the lhs scale sA[m, kb].  Because both vary along the contraction,
// every block's partial sum is promoted on its own:
//   out[m, n] = sum_kb partial_kb[m, n] * sA[m, kb] * sB[g, kb, n]
// in fp32 from +0 in increasing kb, each block added with one fused multiply-add by
// RNE(sA * sB) (a rounding order of the same sum; the products are fp32-accurate).
//
// gmm_bs_kernel: 128 x 128 output tiles, four waves of 64 x 64.  Each wave keeps a
// partial accumulator (MFMA target) and an fp32 total; at the end of every block the
// partial is scaled into the total and restarts from zero.  Operands are fp8 codes
// staged through two LDS stages (one register stage ahead); the tile grid is the
// expert-tile schedule of the other products with 128-row tiles.
//
// subchannel_quant_kernel: bf16 [M, K] -> codes and one dynamic scale per row and block
// of bk columns (bk = 128, 256 or 512): bk / 8 lanes share a block and reduce its
// abs-max with lane shuffles.
#include <algorithm>

#include "kernels.hpp"

namespace gmm {

namespace {

constexpr int BS_BM = 128, BS_BN = 128, BS_BK = TILE_K, BS_NT = 256;
constexpr int BS_TILE = BS_BM * BS_BK;  // bytes of one operand tile (A or B)
constexpr int BS_BAND = 8;              // M-tiles per band of the tile order

struct BsTile {
  int g, row0, row_end, n0;
};

// Expert-tile schedule with BS_BM-row tiles (a tile never spans two groups), the tile
// order in bands of BS_BAND M-tiles, XCD-aware: the workgroups of XCD x = wg % 8 take a
// contiguous range of tiles.
__device__ inline bool bs_schedule(const int32_t* __restrict__ gs, int G, int64_t M,
                                   int n_ntiles, int* s_cum, int* s_off, BsTile& tc) {
  const int tid = threadIdx.x;
  // sizes outside the contract are clamped: no tile leaves rows [0, M)
  if (tid < 64) group_tiles_prefix<BS_BM>(gs, G, (uint32_t)M, 0u, s_cum, s_off);
  __syncthreads();
  const int total_mt = s_cum[G];
  const int total = total_mt * n_ntiles;
  const int wg = blockIdx.x;
  bool ok = wg < total;
  if (ok) {
    const int xcd = wg & 7, j = wg >> 3, q = total >> 3, r = total & 7;
    const int L = xcd * q + min(xcd, r) + j;
    const int band = L / (BS_BAND * n_ntiles);
    const int rem = L - band * BS_BAND * n_ntiles;
    const int mt0 = band * BS_BAND;
    const int gm = min(BS_BAND, total_mt - mt0);
    const int nt = rem / gm;
    const int mt = mt0 + (rem - nt * gm);
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_cum[mid] <= mt) lo = mid; else hi = mid;
    }
    tc.g = lo;
    tc.row0 = s_off[lo] + (mt - s_cum[lo]) * BS_BM;
    tc.row_end = (int)min((int64_t)s_off[lo + 1], M);
    tc.n0 = nt * BS_BN;
    ok = tc.row0 < tc.row_end;
  }
  __syncthreads();  // the schedule arrays alias stage memory
  tc.g = __builtin_amdgcn_readfirstlane(tc.g);
  tc.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
  tc.row_end = __builtin_amdgcn_readfirstlane(tc.row_end);
  tc.n0 = __builtin_amdgcn_readfirstlane(tc.n0);
  return __builtin_amdgcn_readfirstlane((int)ok) != 0;
}

// NMAJ: the weight scales are laid out [G, N, K / bk] (p.b_scale_nmajor) instead of
// [G, K / bk, N]; a template parameter so that each instantiation holds one load path
template <int A_FMT, bool NMAJ, bool ONE>
__global__ __attribute__((amdgpu_flat_work_group_size(BS_NT, BS_NT), amdgpu_waves_per_eu(2, 2)))
void gmm_bs_kernel(BsParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[BS_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[BS_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[BS_TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[BS_TILE];
  int* s_cum = reinterpret_cast<int*>(sA0);
  int* s_off = reinterpret_cast<int*>(sB0);
  static_assert((MAX_GROUPS + 1) * sizeof(int) <= BS_TILE, "schedule arrays fit a tile");

  const int n_ntiles = p.N / BS_BN;
  BsTile tc;
  if (!bs_schedule(p.group_sizes, p.G, p.M, n_ntiles, s_cum, s_off, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int K = p.K, nk = K / BS_BK, steps_per_block = p.bk / BS_BK, nkb = K / p.bk;
  const int rows_here = min(tc.row_end - tc.row0, BS_BM);
  // rows past the group's end and columns past N read zeros
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(p.a + (int64_t)tc.row0 * K, (uint32_t)rows_here * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(p.b + ((int64_t)tc.g * p.N + tc.n0) * K, (uint32_t)BS_BN * (uint32_t)K);

  // staging: piece i of a tile = rows 32 i + tid / 8, 16 bytes at chunk tid % 8
  const int lrow = tid >> 3, lchunk = tid & 7;
  v4u a_reg[4], b_reg[4];
  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = (uint32_t)(i * 32 + lrow) * K + (uint32_t)kt * BS_BK + lchunk * 16;
      a_reg[i] = buf_load16(ra, off);
      b_reg[i] = buf_load16(rb, off);
    }
  };
  auto store = [&](uint8_t* at, uint8_t* bt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<v4u*>(at + tile_off(i * 32 + lrow, lchunk)) = a_reg[i];
      *reinterpret_cast<v4u*>(bt + tile_off(i * 32 + lrow, lchunk)) = b_reg[i];
    }
  };

  // lane holds out[m = row0 + 64 wr + 32 i + frow][n = n0 + 64 wc + 32 j + 8 (r/4) +
  // 4 fhalf + r%4] in register r of tile (i, j)
  const int frow = lane & 31, fhalf = lane >> 5;
  v16f part[2][2], total[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      part[i][j] = v16f{0};
      total[i][j] = v16f{0};
    }
  // the lane's rows (clamped inside the group) and its columns' scale offsets
  int64_t sa_row[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    sa_row[i] = (int64_t)max(min(tc.row0 + 64 * wr + 32 * i + frow, tc.row_end - 1), 0) * nkb;
  // NMAJ: scale of (column n, block kb) at (g N + n) nkb + kb, read through a resource
  // over the tile's 128 columns: the lane's offset in a VGPR, the column's in an SGPR
  // (otherwise: at (g nkb + kb) N + n, a resource from the tile's first column, the
  // block's row offset in an SGPR)
  __amdgpu_buffer_rsrc_t rs;
  uint32_t sbt_lane;
  if constexpr (NMAJ) {
    rs = make_rsrc(p.b_scale + ((int64_t)tc.g * p.N + tc.n0) * nkb, (uint32_t)(BS_BN * nkb * 4));
    sbt_lane = (uint32_t)((64 * wc + 4 * fhalf) * nkb) * 4u;
  } else {
    rs = make_rsrc(p.b_scale + (int64_t)tc.g * nkb * p.N + tc.n0,
                   (uint32_t)((nkb * p.N - tc.n0) * 4));
    sbt_lane = (uint32_t)(64 * wc + 4 * fhalf) * 4u;
  }

  // a block's scales are loaded at the start of its last step and used after that
  // step's MFMAs, so their latency hides behind the matrix core
  float sa[2];
  v4f sb[2][4];
  auto load_scales = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 2; ++i) sa[i] = p.a_scale[sa_row[i] + kb];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        if constexpr (!NMAJ) {
          sb[j][r4] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
              rs, sbt_lane + (uint32_t)(32 * j + 8 * r4) * 4u, (uint32_t)(kb * p.N) * 4u, 0));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sb[j][r4][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                rs, sbt_lane + (uint32_t)kb * 4u, (uint32_t)((32 * j + 8 * r4 + e) * nkb) * 4u, 0));
        }
      }
  };
  // total += partial * RNE(sA * sB): one fused multiply-add per value; the partial
  // restarts from zero (ONE: every step is a whole block, whose first MFMAs take a zero
  // accumulator operand instead)
  auto promote = [&]() {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          total[i][j][r] = __builtin_fmaf(part[i][j][r], mul_rn(sa[i], sb[j][r >> 2][r & 3]),
                                          total[i][j][r]);
        if constexpr (!ONE) part[i][j] = v16f{0};
      }
  };

  auto compute = [&](const uint8_t* at, const uint8_t* bt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = lds_read_frag(at, 64 * wr + 32 * i + frow, 4 * ks + 2 * fhalf);
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = lds_read_frag(bt, 64 * wc + 32 * j + frow, 4 * ks + 2 * fhalf);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          part[i][j] = mfma32x32x64<FMT_E4M3, A_FMT>(bf[j], af[i],
                                                     ONE && ks == 0 ? v16f{0} : part[i][j]);
    }
  };

  load(0);
  store(sA0, sB0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool odd = kt & 1;
    const bool block_end = (kt + 1) % steps_per_block == 0;
    if (block_end) load_scales(kt / steps_per_block);
    if (kt + 1 < nk) load(kt + 1);
    compute(odd ? sA1 : sA0, odd ? sB1 : sB0);
    if (block_end) promote();
    if (kt + 1 < nk) store(odd ? sA0 : sA1, odd ? sB0 : sB1);
    __syncthreads();
  }

  // ---- epilogue: rows of the group only ----
  if (!p.out_f32) {
    // bf16: each wave puts its 64 x 64 sub-tile into its own 16 KB stage tile
    // ([row][128 B], 16-byte chunk c of row r at c ^ (r & 7)) and stores whole 128-byte
    // rows, 8 lanes per row: full lines instead of 16-byte pieces of 32 rows.  The loop
    // ended with a barrier after every wave's last LDS access.
    uint8_t* const wl = wave == 0 ? sA0 : wave == 1 ? sB0 : wave == 2 ? sA1 : sB1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 32 * i + frow;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          v2u v;
          v.x = pack_bf16x2(total[i][j][4 * r4], total[i][j][4 * r4 + 1]);
          v.y = pack_bf16x2(total[i][j][4 * r4 + 2], total[i][j][4 * r4 + 3]);
          *reinterpret_cast<v2u*>(wl + row * 128 + (((4 * j + r4) ^ (row & 7)) << 4) + fhalf * 8) = v;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // stores through a resource over the wave's 64 rows inside the group: rows past its
    // end fall outside the range and are dropped (offsets below 2^30); all eight rows'
    // LDS reads in flight before the stores
    const int c = lane & 7;
    const int m0 = tc.row0 + 64 * wr;
    const int rows_valid = max(min(tc.row_end - m0, 64), 0);
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc((uint16_t*)p.out + (int64_t)m0 * p.N, (uint32_t)rows_valid * (uint32_t)p.N * 2u);
    const uint32_t lane_off = ((uint32_t)(lane >> 3) * (uint32_t)p.N + (uint32_t)(tc.n0 + 64 * wc + c * 8)) * 2u;
    v4u v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = q * 8 + (lane >> 3);
      v[q] = *reinterpret_cast<const v4u*>(wl + row * 128 + ((c ^ (row & 7)) << 4));
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) buf_store16(ro, lane_off + (uint32_t)q * 16u * (uint32_t)p.N, v[q]);
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = tc.row0 + 64 * wr + 32 * i + frow;
    if (m >= tc.row_end) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = tc.n0 + 64 * wc + 32 * j + 8 * r4 + 4 * fhalf;
        const int64_t idx = (int64_t)m * p.N + n;
        const v4f o = {total[i][j][4 * r4], total[i][j][4 * r4 + 1], total[i][j][4 * r4 + 2],
                       total[i][j][4 * r4 + 3]};
        *reinterpret_cast<v4f*>((float*)p.out + idx) = o;
      }
    }
  }
}

// One thread per 8 consecutive elements of a row; the bk / 8 lanes of a block (aligned
// within the wave) reduce its abs-max with xor shuffles, then each quantizes its 8.
template <int FMT>
__global__ __launch_bounds__(256) void subchannel_quant_kernel(const uint16_t* __restrict__ x,
                                                               int64_t M, int64_t K, int bk,
                                                               uint8_t* __restrict__ codes,
                                                               float* __restrict__ scales) {
  const int64_t per_row = K / 8, total = M * per_row;
  const int lanes = bk / 8;  // 16, 32 or 64: divides both 64 and per_row
  const int lane = threadIdx.x & 63;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * 256) {
    const v4u w = *reinterpret_cast<const v4u*>(x + t * 8);
    uint32_t m = absmax_bits16(w, 0u);
    for (int d = lanes >> 1; d >= 1; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
    const float s = __fdiv_rn(__uint_as_float(m << 16), qmax<FMT>());
    reinterpret_cast<v2u*>(codes)[t] = quant8<FMT>(w, inv_from_scale(s));
    if ((lane & (lanes - 1)) == 0) {
      const int64_t row = t / per_row, c8 = t - row * per_row;
      scales[row * (K / bk) + c8 / lanes] = s;
    }
  }
}

// ---- the folded gradient of the one-weight-copy dlhs ----
// y[m, n] = RNE(grad[m, n] * s[g(m), n]); its 128-row-block abs-max (as fp32 bits) over
// AMAX_SPLIT row slices per block, then the codes of y.  Every workgroup builds the
// group row offsets in LDS and looks each row's group up once; a thread walks its
// columns and, for each, the slice's rows, so a column's scales are read once per group.
__device__ inline void fold_offsets(const int32_t* __restrict__ gs, int G, int* s_off) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    int carry = 0;
    for (int base = 0; base < G; base += 64) {
      const int g = base + lane;
      const int incl = wave_incl_scan(g < G ? max(gs[g], 0) : 0, lane);
      if (g < G) s_off[g + 1] = carry + incl;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) s_off[0] = 0;
  }
  __syncthreads();
}

// group of row r: the last g with s_off[g] <= r (rows past every group: the last group)
__device__ inline int fold_group(const int* s_off, int G, int64_t r) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_off[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// 8 consecutive bf16 gradient values times their columns' scales, each product rounded
__device__ inline void fold8(v4u w, v4f s0, v4f s1, float (&y)[8]) {
  y[0] = mul_rn(bf16_lo(w.x), s0[0]); y[1] = mul_rn(bf16_hi(w.x), s0[1]);
  y[2] = mul_rn(bf16_lo(w.y), s0[2]); y[3] = mul_rn(bf16_hi(w.y), s0[3]);
  y[4] = mul_rn(bf16_lo(w.z), s1[0]); y[5] = mul_rn(bf16_hi(w.z), s1[1]);
  y[6] = mul_rn(bf16_lo(w.w), s1[2]); y[7] = mul_rn(bf16_hi(w.w), s1[3]);
}

__global__ __launch_bounds__(256) void fold_amax_kernel(const uint16_t* __restrict__ x,
                                                        int64_t M, int64_t N,
                                                        const float* __restrict__ col_scales,
                                                        const int32_t* __restrict__ gs, int G,
                                                        uint32_t* __restrict__ partial) {
  __shared__ int s_off[MAX_GROUPS + 1];
  __shared__ uint32_t red[4];
  fold_offsets(gs, G, s_off);
  const int b = blockIdx.x, sl = blockIdx.y;
  constexpr int rows_per = BLOCK_ROWS / AMAX_SPLIT;
  const int64_t r0 = (int64_t)b * BLOCK_ROWS + (int64_t)sl * rows_per;
  const int64_t r1 = min(r0 + rows_per, M);
  __shared__ int s_grp[BLOCK_ROWS / AMAX_SPLIT];
  if ((int)threadIdx.x < r1 - r0) s_grp[threadIdx.x] = fold_group(s_off, G, r0 + threadIdx.x);
  __syncthreads();
  uint32_t m = 0;
  const int64_t chunks = N / 8;
  const int nrows = (int)(r1 - r0);
  // columns outer, the slice's rows inner: a chunk's 8 scales are loaded once per group
  for (int64_t j = threadIdx.x; j < chunks; j += 256) {
    int gcur = -1;
    v4f s0, s1;
    for (int i0 = 0; i0 < nrows; i0 += 4) {
      v4u w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        w[u] = reinterpret_cast<const v4u*>(x + (r0 + min(i0 + u, nrows - 1)) * N)[j];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (i0 + u >= nrows) break;
        const int gr = s_grp[i0 + u];
        if (gr != gcur) {
          gcur = gr;
          s0 = *reinterpret_cast<const v4f*>(col_scales + (int64_t)gr * N + j * 8);
          s1 = *reinterpret_cast<const v4f*>(col_scales + (int64_t)gr * N + j * 8 + 4);
        }
        float y[8];
        fold8(w[u], s0, s1, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, __float_as_uint(y[e]) & 0x7fffffffu);
      }
    }
  }
  // block maximum
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
  if (lane == 0) red[w] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    partial[b * AMAX_SPLIT + sl] = max(max(red[0], red[1]), max(red[2], red[3]));
}

template <int FMT>
__global__ void fold_scales_kernel(const uint32_t* __restrict__ partial, int nb,
                                   float* __restrict__ scales) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  uint32_t m = 0;
#pragma unroll
  for (int s = 0; s < AMAX_SPLIT; ++s) m = max(m, partial[b * AMAX_SPLIT + s]);
  scales[b] = __fdiv_rn(__uint_as_float(m), qmax<FMT>());
}

template <int FMT>
__global__ __launch_bounds__(256) void fold_quantize_kernel(const uint16_t* __restrict__ x,
                                                            int64_t M, int64_t N,
                                                            const float* __restrict__ col_scales,
                                                            const int32_t* __restrict__ gs, int G,
                                                            const float* __restrict__ scales,
                                                            uint8_t* __restrict__ codes) {
  __shared__ int s_off[MAX_GROUPS + 1];
  fold_offsets(gs, G, s_off);
  const int b = blockIdx.x, sl = blockIdx.y;
  constexpr int rows_per = BLOCK_ROWS / AMAX_SPLIT;
  const int64_t r0 = (int64_t)b * BLOCK_ROWS + (int64_t)sl * rows_per;
  const int64_t r1 = min(r0 + rows_per, M);
  const float inv = inv_from_scale(scales[b]);
  __shared__ int s_grp[BLOCK_ROWS / AMAX_SPLIT];
  if ((int)threadIdx.x < r1 - r0) s_grp[threadIdx.x] = fold_group(s_off, G, r0 + threadIdx.x);
  __syncthreads();
  const int64_t chunks = N / 8;
  const int nrows = (int)(r1 - r0);
  for (int64_t j = threadIdx.x; j < chunks; j += 256) {
    int gcur = -1;
    v4f s0, s1;
    for (int i0 = 0; i0 < nrows; i0 += 4) {
      v4u w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        w[u] = reinterpret_cast<const v4u*>(x + (r0 + min(i0 + u, nrows - 1)) * N)[j];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (i0 + u >= nrows) break;
        const int gr = s_grp[i0 + u];
        if (gr != gcur) {
          gcur = gr;
          s0 = *reinterpret_cast<const v4f*>(col_scales + (int64_t)gr * N + j * 8);
          s1 = *reinterpret_cast<const v4f*>(col_scales + (int64_t)gr * N + j * 8 + 4);
        }
        float y[8];
        fold8(w[u], s0, s1, y);
        uint32_t d0 = cvt_pk<FMT, false>(quant_prep<FMT>(y[0], inv), quant_prep<FMT>(y[1], inv), 0u);
        d0 = cvt_pk<FMT, true>(quant_prep<FMT>(y[2], inv), quant_prep<FMT>(y[3], inv), d0);
        uint32_t d1 = cvt_pk<FMT, false>(quant_prep<FMT>(y[4], inv), quant_prep<FMT>(y[5], inv), 0u);
        d1 = cvt_pk<FMT, true>(quant_prep<FMT>(y[6], inv), quant_prep<FMT>(y[7], inv), d1);
        v2u o;
        o.x = d0;
        o.y = d1;
        reinterpret_cast<v2u*>(codes + (r0 + i0 + u) * N)[j] = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_blockwise(int a_fmt, const BsParams& p, hipStream_t st) {
  const int64_t max_mt = (p.M + BS_BM - 1) / BS_BM + p.G;
  const int64_t grid = max_mt * (p.N / BS_BN);
  if (grid == 0 || p.M == 0) return hipSuccess;
  const dim3 gd((unsigned)grid), bd(BS_NT);
  if (a_fmt != FMT_E4M3 && a_fmt != FMT_E5M2) return hipErrorInvalidValue;
  // one contraction step per scale block (bk = 128) takes the variant without clearing
  const bool one = p.bk == BS_BK;
  if (a_fmt == FMT_E4M3 && !p.b_scale_nmajor) {
    if (one) hipLaunchKernelGGL((gmm_bs_kernel<FMT_E4M3, false, true>), gd, bd, 0, st, p);
    else hipLaunchKernelGGL((gmm_bs_kernel<FMT_E4M3, false, false>), gd, bd, 0, st, p);
  } else if (a_fmt == FMT_E4M3) {
    if (one) hipLaunchKernelGGL((gmm_bs_kernel<FMT_E4M3, true, true>), gd, bd, 0, st, p);
    else hipLaunchKernelGGL((gmm_bs_kernel<FMT_E4M3, true, false>), gd, bd, 0, st, p);
  } else if (!p.b_scale_nmajor) {
    if (one) hipLaunchKernelGGL((gmm_bs_kernel<FMT_E5M2, false, true>), gd, bd, 0, st, p);
    else hipLaunchKernelGGL((gmm_bs_kernel<FMT_E5M2, false, false>), gd, bd, 0, st, p);
  } else {
    if (one) hipLaunchKernelGGL((gmm_bs_kernel<FMT_E5M2, true, true>), gd, bd, 0, st, p);
    else hipLaunchKernelGGL((gmm_bs_kernel<FMT_E5M2, true, false>), gd, bd, 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_subchannel(int fmt, const void* x, int64_t M, int64_t K, int bk,
                                      uint8_t* codes, float* scales, hipStream_t st) {
  const int64_t total = M * (K / 8);
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  if (fmt == FMT_E4M3)
    hipLaunchKernelGGL(subchannel_quant_kernel<FMT_E4M3>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint16_t*)x, M, K, bk, codes, scales);
  else
    hipLaunchKernelGGL(subchannel_quant_kernel<FMT_E5M2>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint16_t*)x, M, K, bk, codes, scales);
  return hipGetLastError();
}

}  // namespace gmm

namespace gmm {

hipError_t launch_quantize_folded(int fmt, const void* x, int64_t M, int64_t N,
                                  const float* col_scales, const int32_t* gs, int G,
                                  uint32_t* partial, float* scales, uint8_t* codes,
                                  hipStream_t st) {
  const int nb = (int)((M + BLOCK_ROWS - 1) / BLOCK_ROWS);
  if (nb == 0) return hipSuccess;
  const uint16_t* xp = (const uint16_t*)x;
  hipLaunchKernelGGL(fold_amax_kernel, dim3(nb, AMAX_SPLIT), dim3(256), 0, st, xp, M, N,
                     col_scales, gs, G, partial);
  const unsigned fb = (unsigned)((nb + 255) / 256);
  if (fmt == FMT_E4M3) {
    hipLaunchKernelGGL(fold_scales_kernel<FMT_E4M3>, dim3(fb), dim3(256), 0, st, partial, nb, scales);
    hipLaunchKernelGGL(fold_quantize_kernel<FMT_E4M3>, dim3(nb, AMAX_SPLIT), dim3(256), 0, st, xp,
                       M, N, col_scales, gs, G, scales, codes);
  } else {
    hipLaunchKernelGGL(fold_scales_kernel<FMT_E5M2>, dim3(fb), dim3(256), 0, st, partial, nb, scales);
    hipLaunchKernelGGL(fold_quantize_kernel<FMT_E5M2>, dim3(nb, AMAX_SPLIT), dim3(256), 0, st, xp,
                       M, N, col_scales, gs, G, scales, codes);
  }
  return hipGetLastError();
}

}  // namespace gmm
