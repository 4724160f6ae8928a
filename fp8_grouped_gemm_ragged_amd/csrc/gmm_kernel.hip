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
// Work decomposition (one workgroup = one 256 x 256 output tile):
//   * expert-tile scheduler: every workgroup prefix-sums group_sizes into per-group
//     M-tile counts ceil(m_g / 256) in LDS; a tile never spans two groups, empty groups
//     own no tile, and workgroups past the real tile count exit at once;
//   * XCD-aware order: the hardware places workgroup i on XCD i % 8, so workgroup ids
//     are remapped to give each XCD a contiguous range of tiles, and tiles are ordered
//     in bands of 8 M-tiles sweeping the N-tiles, so the 32 concurrent tiles of one XCD
//     share A rows and B columns in that XCD's L2;
//   * K-loop over 128-byte contraction steps, double-buffered in LDS (2 x 64 KB): the
//     next step's bf16 A tile is loaded with 16-byte range-checked buffer loads (rows
//     past the group end read as zero), quantized in registers to fp8 and stored to a
//     swizzled LDS tile; the fp8 B tile is copied (or transposed 8x8 in registers
//     when B is stored output-contiguous);
//   * 4 waves, each a 128 x 128 sub-tile of 4 x 4 MFMA 32x32x64 fp8 instructions with
//     fp32 accumulators;
//   * epilogue: (acc * s_A(m)) * s_B(n), RNE to bf16 (or f32), stored only for rows
//     inside the group and columns inside N.
#include "kernels.hpp"

namespace gmm {

namespace {

constexpr int BM = 256, BN = 256, BK = TILE_K;
constexpr int NT = 256;
constexpr int A_TILE = BM * BK;                // bytes of one fp8 A tile
constexpr int B_TILE = BN * BK;
constexpr int STAGE = A_TILE + B_TILE;         // 64 KB
constexpr int BAND = 8;                        // M-tiles per band of the tile order

struct TileCoord {
  int g, row0, row_end, n0;
};

// Expert-tile scheduler.  Returns false for a workgroup without a tile.
__device__ inline bool schedule_tile(const int32_t* __restrict__ gs, int G, int64_t M,
                                     int n_ntiles, int* s_tile_cum, int* s_row_off,
                                     TileCoord& tc) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    int carry_t = 0, carry_r = 0;
    for (int base = 0; base < G; base += 64) {
      const int g = base + lane;
      // sizes outside the contract (negative) are read as 0, and rows past M are
      // dropped below, so no access ever leaves the tensors
      const int m = g < G ? max(gs[g], 0) : 0;
      const int it = wave_incl_scan((m + BM - 1) / BM, lane);
      const int ir = wave_incl_scan(m, lane);
      if (g < G) {
        s_tile_cum[g + 1] = carry_t + it;
        s_row_off[g + 1] = carry_r + ir;
      }
      carry_t += __shfl(it, 63, 64);
      carry_r += __shfl(ir, 63, 64);
    }
    if (lane == 0) {
      s_tile_cum[0] = 0;
      s_row_off[0] = 0;
    }
  }
  __syncthreads();
  const int total_mt = s_tile_cum[G];
  const int total = total_mt * n_ntiles;
  const int wg = blockIdx.x;
  if (wg >= total) return false;
  // XCD-aware remap: workgroups of XCD x = wg % 8 take a contiguous range of tiles.
  const int xcd = wg & 7, j = wg >> 3, q = total >> 3, r = total & 7;
  const int L = xcd * q + min(xcd, r) + j;
  // bands of BAND M-tiles; inside a band the M-tile index runs fastest
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
  tc.g = lo;
  tc.row0 = s_row_off[lo] + (mt - s_tile_cum[lo]) * BM;
  tc.row_end = (int)min((int64_t)s_row_off[lo + 1], M);
  tc.n0 = nt * BN;
  return tc.row0 < tc.row_end;
}

// 8x8 byte transpose: in[r] holds bytes (r, 0..7) as two dwords; out[c] gets bytes
// (0..7, c).  Two rounds of v_perm byte shuffles.
__device__ inline void transpose8x8(const v2u in[8], v2u out[8]) {
  uint32_t x[4][2][2];  // [row pair][dword lo/hi][even/odd column pair]
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t r0 = d ? in[2 * p].y : in[2 * p].x;
      const uint32_t r1 = d ? in[2 * p + 1].y : in[2 * p + 1].x;
      x[p][d][0] = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0c0 r1c0 r0c1 r1c1
      x[p][d][1] = __builtin_amdgcn_perm(r1, r0, 0x07030602u);  // r0c2 r1c2 r0c3 r1c3
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int d = c >> 2, h = (c >> 1) & 1;
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    out[c].x = __builtin_amdgcn_perm(x[1][d][h], x[0][d][h], sel);
    out[c].y = __builtin_amdgcn_perm(x[3][d][h], x[2][d][h], sel);
  }
}

template <int A_FMT, int B_FMT, bool A_FP8, bool B_TRANS>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
void gmm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ int s_tile_cum[MAX_GROUPS + 1];
  __shared__ int s_row_off[MAX_GROUPS + 1];

  const int n_ntiles = (p.Nout + BN - 1) / BN;
  TileCoord tc;
  if (!schedule_tile(p.group_sizes, p.G, p.M, n_ntiles, s_tile_cum, s_row_off, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int Kc = p.Kc;
  const int nk = Kc / BK;

  // ---- operand resources (range-checked) ----
  constexpr int AES = A_FP8 ? 1 : 2;  // bytes per A element
  const int rows_here = min(tc.row_end - tc.row0, BM);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(
      (const uint8_t*)p.a + (int64_t)tc.row0 * Kc * AES, (uint32_t)rows_here * Kc * AES);
  __amdgpu_buffer_rsrc_t rb;
  if constexpr (!B_TRANS) {
    const int cols_here = min(p.Nout - tc.n0, BN);
    rb = make_rsrc(p.b + ((int64_t)tc.g * p.Nout + tc.n0) * Kc, (uint32_t)cols_here * Kc);
  } else {
    rb = make_rsrc(p.b + (int64_t)tc.g * Kc * p.Nout + tc.n0,
                   (uint32_t)((int64_t)Kc * p.Nout - tc.n0));
  }

  // ---- per-thread load mapping ----
  // A: item i -> row i*32 + tid/8, 16-element (bf16) or 16-byte (fp8) chunk tid%8
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

  v4u a_reg[A_FP8 ? 8 : 16];
  v2u b_reg[B_TRANS ? 16 : 1];
  v4u bt_reg[B_TRANS ? 1 : 8];

  auto load_a = [&](int kt) {
    const uint32_t kb = (uint32_t)kt * BK * AES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = (uint32_t)(i * 32 + lrow) * Kc * AES + kb;
      if constexpr (A_FP8) {
        a_reg[i] = buf_load16(ra, off + lchunk * 16);
      } else {
        a_reg[2 * i] = buf_load16(ra, off + lchunk * 32);
        a_reg[2 * i + 1] = buf_load16(ra, off + lchunk * 32 + 16);
      }
    }
  };
  // B (contraction-contiguous): item i -> out column i*32 + tid/8, chunk tid%8
  // B (output-contiguous): 8x8 byte blocks; block q = it*256 + tid, see below
  auto load_b = [&](int kt) {
    if constexpr (!B_TRANS) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        bt_reg[i] = buf_load16(rb, (uint32_t)(i * 32 + lrow) * Kc + kt * BK + lchunk * 16);
    } else {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int q = it * 256 + tid;
        const int nb = (q & 7) | (((q >> 4) & 3) << 3);
        const int kb = ((q >> 3) & 1) | ((q >> 6) << 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t off = (uint32_t)(kt * BK + kb * 8 + e) * p.Nout + nb * 8;
          b_reg[it * 8 + e] = __builtin_amdgcn_raw_buffer_load_b64(rb, off, 0, 0);
        }
      }
    }
  };
  auto store_stage = [&](int stage) {
    uint8_t* at = smem + stage * STAGE;
    uint8_t* bt = at + A_TILE;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 32 + lrow;
      v4u q;
      if constexpr (A_FP8) {
        q = a_reg[i];
      } else {
        const v2u lo = quant8<A_FMT>(a_reg[2 * i], inv_row[i]);
        const v2u hi = quant8<A_FMT>(a_reg[2 * i + 1], inv_row[i]);
        q.x = lo.x; q.y = lo.y; q.z = hi.x; q.w = hi.y;
      }
      *reinterpret_cast<v4u*>(at + tile_off(row, lchunk)) = q;
    }
    if constexpr (!B_TRANS) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<v4u*>(bt + tile_off(i * 32 + lrow, lchunk)) = bt_reg[i];
    } else {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int q = it * 256 + tid;
        const int nb = (q & 7) | (((q >> 4) & 3) << 3);
        const int kb = ((q >> 3) & 1) | ((q >> 6) << 1);
        v2u t[8];
        transpose8x8(&b_reg[it * 8], t);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int n = nb * 8 + c;
          *reinterpret_cast<v2u*>(bt + tile_off(n, kb >> 1) + (kb & 1) * 8) = t[c];
        }
      }
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{0};

  load_a(0);
  load_b(0);
  store_stage(0);
  __syncthreads();

  const int frow = lane & 31, fhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) {
      load_a(kt + 1);
      load_b(kt + 1);
    }
    const uint8_t* at = smem + stage * STAGE;
    const uint8_t* bt = at + A_TILE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = lds_read_frag(at, wr * 128 + i * 32 + frow, ks * 4 + fhalf * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = lds_read_frag(bt, wc * 128 + j * 32 + frow, ks * 4 + fhalf * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x64<B_FMT, A_FMT>(bf[j], af[i], acc[i][j]);
    }
    if (kt + 1 < nk) store_stage(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  // lane holds out[m = base_m + lane%32][n = base_n + 8*(r/4) + 4*(lane/32) + r%4]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = tc.row0 + wr * 128 + i * 32 + frow;
    if (m >= tc.row_end) continue;
    const float sa = p.a_scale_blk ? p.a_scale_blk[m / BLOCK_ROWS] : p.a_scale_static;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = tc.n0 + wc * 128 + j * 32 + 8 * r4 + 4 * fhalf;
        if (n >= p.Nout) continue;
        const v4f sb = *reinterpret_cast<const v4f*>(p.b_scale + (int64_t)tc.g * p.Nout + n);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __fmul_rn(__fmul_rn(acc[i][j][4 * r4 + e], sa), sb[e]);
        const int64_t idx = (int64_t)m * p.Nout + n;
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

template <int A_FMT, int B_FMT, bool A_FP8, bool B_TRANS>
hipError_t launch_one(const GemmParams& p, hipStream_t st) {
  // upper bound on M-tiles: sum ceil(m_g/BM) <= ceil(M/BM) + G
  const int64_t max_mt = (p.M + BM - 1) / BM + p.G;
  const int64_t n_nt = (p.Nout + BN - 1) / BN;
  const int64_t grid = max_mt * n_nt;
  if (grid == 0 || p.M == 0) return hipSuccess;
  hipLaunchKernelGGL((gmm_kernel<A_FMT, B_FMT, A_FP8, B_TRANS>), dim3((unsigned)grid), dim3(NT),
                     0, st, p);
  return hipGetLastError();
}

}  // namespace

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
