// Transposed grouped matmul on gfx950: the kernel behind tgmm_drhs ("Support
// quantization for tokamax gmm v2", PR #4451, What this does: drhs_tgmm2).
//
//   drhs[g, k, n] = sum over 128-row blocks c meeting group g of
//                   RNE( P_c[k, n] * RNE(s_lhs[c] * s_grad[c]) ),
//   P_c[k, n]     = sum_{m in c, m in g} q(lhs)[m, k] * q(grad)[m, n]   (fp32 MFMA sums)
//
// One workgroup computes a 256 (k) x 128 (n) slab tile of one group.  The contraction
// runs over the group's rows, one 128-row block per step; the steps are aligned to the
// global 128-row grid of the dynamic scales, so the first and last blocks of a group
// are partial and rows outside the group read as zero.  Both operands arrive as bf16
// with the contraction (row) axis strided: each thread loads an 8-row x 8-column block
// (eight 16-byte loads), and the paired fp8 conversion packs two rows of one column
// into each half of a dword, so the quantized codes come out row-contiguous per column
// (transposed) without any byte shuffles.  Each step's MFMA result goes to a fresh
// fp32 partial that is scaled and added to the running slab (scale promotion), since a
// dynamic scale changes from block to block.  A group without rows stores +0.0.
#include "kernels.hpp"

namespace gmm {

namespace {

constexpr int TBM = 256;   // k rows of the slab tile
constexpr int TBN = 128;   // n columns of the slab tile
constexpr int NT = 256;
constexpr int A_TILE = TBM * TILE_K;  // [256 k][128 m] fp8
constexpr int B_TILE = TBN * TILE_K;  // [128 n][128 m] fp8
constexpr int STAGE = A_TILE + B_TILE;  // 48 KB

// Quantize an 8 (rows) x 8 (cols) bf16 block held as 8 row vectors into 8 column
// vectors of 8 codes each (rows 0..3 in .x, rows 4..7 in .y).
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
    uint32_t lo = cvt_pk<FMT, false>(v[0], v[1], 0u);
    lo = cvt_pk<FMT, true>(v[2], v[3], lo);
    uint32_t hi = cvt_pk<FMT, false>(v[4], v[5], 0u);
    hi = cvt_pk<FMT, true>(v[6], v[7], hi);
    out[c].x = lo;
    out[c].y = hi;
  }
}

template <int A_FMT, int B_FMT>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
void tgmm_kernel(TgmmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ int s_off[2];

  const int n_kt = (p.Kout + TBM - 1) / TBM;
  const int n_nt = p.Nout / TBN;
  const int tiles_per_group = n_kt * n_nt;
  const int total = tiles_per_group * p.G;
  const int wg = blockIdx.x;
  if (wg >= total) return;
  // Workgroup i runs on XCD i % 8.  Remap so each XCD owns a contiguous range of the
  // tile order, and order tiles group-fastest: every XCD then holds an equal share of
  // every group (the work of a tile grows with its group's row count, so a group-major
  // order would load one XCD with the largest group), while the concurrent tiles of
  // one XCD still cover a few neighbouring slab tiles of each group.
  const int xcd = wg & 7, jx = wg >> 3, qx = total >> 3, rx = total & 7;
  const int L = xcd * qx + min(xcd, rx) + jx;
  const int g = L % p.G;
  const int t = L / p.G;
  const int kt = t / n_nt, nt = t - kt * n_nt;
  const int k0 = kt * TBM, n0 = nt * TBN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) {
    // row offset of group g: prefix sum of group_sizes[0..g)
    int acc = 0;
    for (int base = 0; base < g; base += 64) {
      const int gg = base + lane;
      int v = gg < g ? max(p.group_sizes[gg], 0) : 0;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
      acc += v;
    }
    if (lane == 0) {
      // clamp to [0, M]: sizes outside the contract never move an access out of bounds
      const int64_t lo = min((int64_t)acc, p.M);
      s_off[0] = (int)lo;
      s_off[1] = (int)min(lo + max(p.group_sizes[g], 0), p.M);
    }
  }
  __syncthreads();
  const int off0 = __builtin_amdgcn_readfirstlane(s_off[0]);
  const int off1 = __builtin_amdgcn_readfirstlane(s_off[1]);

  const int wr = wave >> 1, wc = wave & 1;   // wave sub-tile: 128 (k) x 64 (n)
  const int frow = lane & 31, fhalf = lane >> 5;

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{0};

  // load mapping.  A: 512 blocks of 8 rows x 8 k-columns, 2 per thread;
  // block q -> col block cb (k), row block rb (m); lanes 0-7 walk cb so that one load
  // instruction reads 128 contiguous bytes of a row.
  // B: 256 blocks of 8 rows x 8 n-columns, 1 per thread.
  v4u a_reg[16], b_reg[8];

  const int c_first = off0 / BLOCK_ROWS;
  const int c_last = off1 > off0 ? (off1 - 1) / BLOCK_ROWS : c_first - 1;

  auto load_step = [&](int c) {
    const int lo = max(off0, c * BLOCK_ROWS), hi = min(off1, (c + 1) * BLOCK_ROWS);
    const int rlo = lo - c * BLOCK_ROWS;  // first valid row within the block
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(p.a + (int64_t)lo * p.Kout, (uint32_t)(hi - lo) * p.Kout * 2);
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(p.b + (int64_t)lo * p.Nout, (uint32_t)(hi - lo) * p.Nout * 2);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int q = it * 256 + tid;
      const int cb = (q & 7) | (((q >> 4) & 3) << 3);
      const int rb8 = ((q >> 3) & 1) | ((q >> 6) << 1);
      const int col = k0 + cb * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = rb8 * 8 + e - rlo;  // row relative to the first valid row
        uint32_t off = (uint32_t)r * p.Kout * 2 + col * 2;
        if (r < 0 || col >= p.Kout) off = 0xfffffff0u;
        a_reg[it * 8 + e] = buf_load16(ra, off);
      }
    }
    {
      const int q = tid;
      const int cb = (q & 7) | (((q >> 4) & 1) << 3);
      const int rb8 = ((q >> 3) & 1) | ((q >> 5) << 1);
      const int col = n0 + cb * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = rb8 * 8 + e - rlo;
        uint32_t off = (uint32_t)r * p.Nout * 2 + col * 2;
        if (r < 0) off = 0xfffffff0u;
        b_reg[e] = buf_load16(rb, off);
      }
    }
  };
  auto store_step = [&](int c, int stage) {
    uint8_t* at = smem + stage * STAGE;
    uint8_t* bt = at + A_TILE;
    const float ia = p.a_scale_blk ? inv_from_scale(p.a_scale_blk[c]) : p.a_inv_static;
    const float ib = p.b_scale_blk ? inv_from_scale(p.b_scale_blk[c]) : p.b_inv_static;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int q = it * 256 + tid;
      const int cb = (q & 7) | (((q >> 4) & 3) << 3);
      const int rb8 = ((q >> 3) & 1) | ((q >> 6) << 1);
      v2u o[8];
      quant_transpose8<A_FMT>(&a_reg[it * 8], ia, o);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
        *reinterpret_cast<v2u*>(at + tile_off(cb * 8 + cc, rb8 >> 1) + (rb8 & 1) * 8) = o[cc];
    }
    {
      const int q = tid;
      const int cb = (q & 7) | (((q >> 4) & 1) << 3);
      const int rb8 = ((q >> 3) & 1) | ((q >> 5) << 1);
      v2u o[8];
      quant_transpose8<B_FMT>(b_reg, ib, o);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
        *reinterpret_cast<v2u*>(bt + tile_off(cb * 8 + cc, rb8 >> 1) + (rb8 & 1) * 8) = o[cc];
    }
  };

  if (c_first <= c_last) {
    load_step(c_first);
    store_step(c_first, 0);
    __syncthreads();
    for (int c = c_first; c <= c_last; ++c) {
      const int stage = (c - c_first) & 1;
      if (c < c_last) load_step(c + 1);
      const uint8_t* at = smem + stage * STAGE;
      const uint8_t* bt = at + A_TILE;
      v16f part[4][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v8i af[4], bf[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = lds_read_frag(at, wr * 128 + i * 32 + frow, ks * 4 + fhalf * 2);
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = lds_read_frag(bt, wc * 64 + j * 32 + frow, ks * 4 + fhalf * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            part[i][j] = mfma32x32x64<B_FMT, A_FMT>(bf[j], af[i], ks == 0 ? v16f{0} : part[i][j]);
      }
      const float sa = p.a_scale_blk ? p.a_scale_blk[c] : p.a_scale_static;
      const float sb = p.b_scale_blk ? p.b_scale_blk[c] : p.b_scale_static;
      const float sc = __fmul_rn(sa, sb);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = __fadd_rn(acc[i][j][e], __fmul_rn(part[i][j][e], sc));
      if (c < c_last) store_step(c + 1, stage ^ 1);
      __syncthreads();
    }
  }

  // ---- store the slab tile: lane holds out[k = base + lane%32][n = base + 8*(r/4) + 4*(lane/32) + r%4]
  const int64_t slab = (int64_t)g * p.Kout * p.Nout;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = k0 + wr * 128 + i * 32 + frow;
    if (k >= p.Kout) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = n0 + wc * 64 + j * 32 + 8 * r4 + 4 * fhalf;
        const int64_t idx = slab + (int64_t)k * p.Nout + n;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[i][j][4 * r4 + e];
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

template <int A_FMT, int B_FMT>
hipError_t launch_one(const TgmmParams& p, hipStream_t st) {
  const int64_t tiles = (int64_t)((p.Kout + TBM - 1) / TBM) * (p.Nout / TBN) * p.G;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((tgmm_kernel<A_FMT, B_FMT>), dim3((unsigned)tiles), dim3(NT), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tgmm(int a_fmt, int b_fmt, const TgmmParams& p, hipStream_t st) {
  if (a_fmt == FMT_E4M3 && b_fmt == FMT_E5M2) return launch_one<FMT_E4M3, FMT_E5M2>(p, st);
  if (a_fmt == FMT_E4M3 && b_fmt == FMT_E4M3) return launch_one<FMT_E4M3, FMT_E4M3>(p, st);
  if (a_fmt == FMT_E5M2 && b_fmt == FMT_E5M2) return launch_one<FMT_E5M2, FMT_E5M2>(p, st);
  if (a_fmt == FMT_E5M2 && b_fmt == FMT_E4M3) return launch_one<FMT_E5M2, FMT_E4M3>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace gmm
