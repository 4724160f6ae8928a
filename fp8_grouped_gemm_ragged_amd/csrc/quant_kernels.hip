// Quantization kernels: the dynamic-scale prepass, stand-alone quantization of an
// activation matrix and per-channel quantization of a weight.
//
// Dynamic scale (per block of 128 rows over the full row width, blocks aligned to
// row 0): s = RNE_f32(amax / qmax), inv = 0 when s == 0 or 1/s overflows, otherwise
// RNE_f32(1/s).  The zero-inverse rule follows "add static LHS scaling support for
// GMM v2 FWD" (PR #4735, review thread on block_scale_inv); the overflow case extends
// it to blocks whose scale is so small that 1/s is not a finite float32.
#include "kernels.hpp"

namespace gmm {


__device__ inline uint32_t block_reduce_max(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d, 64));
  if (lane == 0) red[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = max(m, red[w]);
    red[0] = m;
  }
  __syncthreads();
  return red[0];
}

// grid (nb, AMAX_SPLIT), 256 threads.  WG (b, s) covers rows
// [b*128 + s*rows_per, +rows_per) of the block and all columns.
template <bool NT>
__global__ __launch_bounds__(256) void absmax_partial_kernel(const uint16_t* __restrict__ x,
                                                             int64_t R, int64_t C,
                                                             uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[4];
  const int b = blockIdx.x, s = blockIdx.y;
  constexpr int rows_per = BLOCK_ROWS / AMAX_SPLIT;
  const int64_t r0 = (int64_t)b * BLOCK_ROWS + (int64_t)s * rows_per;
  const int64_t r1 = min(r0 + rows_per, R);
  // rows r0 .. r1 - 1 are one contiguous range of 16-byte pieces (C % 8 == 0): walked as
  // one range, four loads in flight per thread whatever the row width.  NT: non-temporal
  // loads for a tensor too large to stay in the last-level cache; a smaller one is read
  // normally, so that it is still there when the quantizing pass reads it again.
  const int64_t pieces = r1 > r0 ? (r1 - r0) * (C / 8) : 0;
  const v4u* slice = reinterpret_cast<const v4u*>(x + r0 * C);
  uint32_t m = 0;
  int64_t j = threadIdx.x;
  for (; j + 768 < pieces; j += 1024) {
    v4u w0, w1, w2, w3;
    if constexpr (NT) {
      w0 = __builtin_nontemporal_load(slice + j);
      w1 = __builtin_nontemporal_load(slice + j + 256);
      w2 = __builtin_nontemporal_load(slice + j + 512);
      w3 = __builtin_nontemporal_load(slice + j + 768);
    } else {
      w0 = slice[j];
      w1 = slice[j + 256];
      w2 = slice[j + 512];
      w3 = slice[j + 768];
    }
    m = absmax_bits16(w0, m);
    m = absmax_bits16(w1, m);
    m = absmax_bits16(w2, m);
    m = absmax_bits16(w3, m);
  }
  for (; j < pieces; j += 256) m = absmax_bits16(slice[j], m);
  m = block_reduce_max(m, red);
  if (threadIdx.x == 0) partial[b * AMAX_SPLIT + s] = m;
}

// One thread per block: reduce the partial maxima, s = RNE_f32(amax / qmax).
template <int FMT>
__global__ void finalize_scales_kernel(const uint32_t* __restrict__ partial, int nb,
                                       float* __restrict__ scales_out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  uint32_t m = 0;
#pragma unroll
  for (int s = 0; s < AMAX_SPLIT; ++s) m = max(m, partial[b * AMAX_SPLIT + s]);
  scales_out[b] = __fdiv_rn(__uint_as_float(m << 16), qmax<FMT>());
}

// Stand-alone quantization: one thread per 8 values (16 bytes of bf16).
template <int FMT>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ x,
                                                            int64_t R, int64_t C,
                                                            const float* __restrict__ scale_blk,
                                                            float inv_static,
                                                            uint8_t* __restrict__ codes) {
  const int64_t chunks_per_row = C / 8;
  const int64_t total = R * chunks_per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / chunks_per_row;
    const float inv = scale_blk ? inv_from_scale(scale_blk[r / BLOCK_ROWS]) : inv_static;
    v4u w = reinterpret_cast<const v4u*>(x)[i];
    reinterpret_cast<v2u*>(codes)[i] = quant8<FMT>(w, inv);
  }
}

// ---------------------------------------------------------------------------------
// Per-channel weight quantization, w [G, K, N] bf16.
// axis 0: channel (g, n), reduce over k.  axis 1: channel (g, k), reduce over n.
// ---------------------------------------------------------------------------------

// axis 0 abs-max: one thread per 8 consecutive columns and block of kblk contraction
// rows (kblk = K: the whole column), looping over its k; amax_out [G, K / kblk, N].
__global__ __launch_bounds__(256) void rhs_amax_cols_kernel(const uint16_t* __restrict__ w,
                                                            int64_t G, int64_t K, int64_t N,
                                                            int64_t kblk,
                                                            float* __restrict__ amax_out) {
  const int64_t n8 = N / 8, nkb = K / kblk;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= G * nkb * n8) return;
  const int64_t gb = t / n8, c = t % n8;  // gb = g * nkb + kb
  const int64_t g = gb / nkb, kb = gb % nkb;
  const v4u* p = reinterpret_cast<const v4u*>(w + (g * K + kb * kblk) * N) + c;
  uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t k = 0; k < kblk; ++k) {
    v4u v = p[k * n8];
    uint32_t d[4] = {v.x & 0x7fff7fffu, v.y & 0x7fff7fffu, v.z & 0x7fff7fffu, v.w & 0x7fff7fffu};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m[2 * q] = max(m[2 * q], d[q] & 0xffffu);
      m[2 * q + 1] = max(m[2 * q + 1], d[q] >> 16);
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) amax_out[gb * N + c * 8 + q] = __uint_as_float(m[q] << 16);
}

// axis 1 abs-max: one wave per (g, k) row.
__global__ __launch_bounds__(256) void rhs_amax_rows_kernel(const uint16_t* __restrict__ w,
                                                            int64_t rows, int64_t N,
                                                            float* __restrict__ amax_out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const v4u* p = reinterpret_cast<const v4u*>(w + row * N);
  uint32_t m = 0;
  for (int64_t j = lane; j < N / 8; j += 64) m = absmax_bits16(p[j], m);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
  if (lane == 0) amax_out[row] = __uint_as_float(m << 16);
}

// Quantize a 64(k) x 64(n) tile with per-channel (per block of kblk rows, axis 0)
// inverses computed from the abs-max, writing codes either as [G, K, N] or transposed
// as [G, N, K] through an LDS tile.  kblk is a multiple of 64, so a tile lies in one
// block.
template <int FMT>
__global__ __launch_bounds__(256) void rhs_quantize_kernel(const uint16_t* __restrict__ w,
                                                           int64_t K, int64_t N, int64_t kblk,
                                                           const float* __restrict__ amax,
                                                           int axis, int layout_nk,
                                                           uint8_t* __restrict__ codes) {
  __shared__ float inv_s[64];
  __shared__ uint8_t tile[64][64 + 8];
  const int64_t g = blockIdx.z;
  const int64_t k0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const float a = axis == 0 ? amax[(g * (K / kblk) + k0 / kblk) * N + n0 + tid]
                              : amax[g * K + k0 + tid];
    inv_s[tid] = inv_from_scale(__fdiv_rn(a, qmax<FMT>()));
  }
  __syncthreads();
  // thread -> (k row, 8-column group): 64 rows x 8 groups = 512 items, 2 per thread
  for (int it = 0; it < 2; ++it) {
    const int item = it * 256 + tid;
    const int kr = item >> 3, ng = item & 7;
    const v4u v = *reinterpret_cast<const v4u*>(w + (g * K + k0 + kr) * N + n0 + ng * 8);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint8_t out[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = ng * 8 + 2 * q;
      const float i0 = axis == 0 ? inv_s[nl] : inv_s[kr];
      const float i1 = axis == 0 ? inv_s[nl + 1] : inv_s[kr];
      const uint32_t pk = cvt_pk<FMT, false>(quant_prep<FMT>(bf16_lo(d[q]), i0),
                                      quant_prep<FMT>(bf16_hi(d[q]), i1), 0u);
      out[2 * q] = (uint8_t)(pk & 0xff);
      out[2 * q + 1] = (uint8_t)((pk >> 8) & 0xff);
    }
    if (!layout_nk) {
      v2u o;
      o.x = out[0] | (out[1] << 8) | (out[2] << 16) | ((uint32_t)out[3] << 24);
      o.y = out[4] | (out[5] << 8) | (out[6] << 16) | ((uint32_t)out[7] << 24);
      *reinterpret_cast<v2u*>(codes + (g * K + k0 + kr) * N + n0 + ng * 8) = o;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) tile[ng * 8 + q][kr] = out[q];
    }
  }
  if (layout_nk) {
    __syncthreads();
    // 64 n-rows x 64 k-bytes: 256 threads x 16 bytes
    const int nr = tid >> 2, kc = (tid & 3) * 16;
    v4u o;
    uint32_t* op = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      op[q] = tile[nr][kc + 4 * q] | (tile[nr][kc + 4 * q + 1] << 8) |
              (tile[nr][kc + 4 * q + 2] << 16) | ((uint32_t)tile[nr][kc + 4 * q + 3] << 24);
    *reinterpret_cast<v4u*>(codes + (g * N + n0 + nr) * K + k0 + kc) = o;
  }
}

template <int FMT>
__global__ void rhs_scales_kernel(float* __restrict__ amax_then_scale, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax_then_scale[i] = __fdiv_rn(amax_then_scale[i], qmax<FMT>());
}

// ---------------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------------
hipError_t launch_dynamic_scales(int fmt, const void* x, int64_t R, int64_t C,
                                 uint32_t* partial, float* scales_out, hipStream_t st) {
  const int nb = (int)((R + BLOCK_ROWS - 1) / BLOCK_ROWS);
  if (nb == 0) return hipSuccess;
  // tensors above 128 MiB do not stay in the 256 MB last-level cache until the second pass
  if ((int64_t)R * C * 2 > (int64_t(128) << 20))
    hipLaunchKernelGGL(absmax_partial_kernel<true>, dim3(nb, AMAX_SPLIT), dim3(256), 0, st,
                       (const uint16_t*)x, R, C, partial);
  else
    hipLaunchKernelGGL(absmax_partial_kernel<false>, dim3(nb, AMAX_SPLIT), dim3(256), 0, st,
                       (const uint16_t*)x, R, C, partial);
  const int thr = 256, blocks = (nb + thr - 1) / thr;
  if (fmt == FMT_E4M3)
    hipLaunchKernelGGL(finalize_scales_kernel<FMT_E4M3>, dim3(blocks), dim3(thr), 0, st,
                       partial, nb, scales_out);
  else
    hipLaunchKernelGGL(finalize_scales_kernel<FMT_E5M2>, dim3(blocks), dim3(thr), 0, st,
                       partial, nb, scales_out);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(int fmt, const void* x, int64_t R, int64_t C,
                                const float* scale_blk, float inv_static, uint8_t* codes,
                                hipStream_t st) {
  const int64_t total = R * (C / 8);
  if (total == 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  if (fmt == FMT_E4M3)
    hipLaunchKernelGGL(quantize_rows_kernel<FMT_E4M3>, dim3(blocks), dim3(256), 0, st,
                       (const uint16_t*)x, R, C, scale_blk, inv_static, codes);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<FMT_E5M2>, dim3(blocks), dim3(256), 0, st,
                       (const uint16_t*)x, R, C, scale_blk, inv_static, codes);
  return hipGetLastError();
}

hipError_t launch_quantize_rhs(int fmt, int axis, int layout_nk, int64_t G, int64_t K,
                               int64_t N, int64_t kblk, const void* w, uint8_t* codes,
                               float* scales, hipStream_t st) {
  const uint16_t* wp = (const uint16_t*)w;
  int64_t nch;
  if (axis == 0) {
    nch = G * (K / kblk) * N;
    const int64_t thr = G * (K / kblk) * (N / 8);
    hipLaunchKernelGGL(rhs_amax_cols_kernel, dim3((unsigned)((thr + 255) / 256)), dim3(256), 0,
                       st, wp, G, K, N, kblk, scales);
  } else {
    nch = G * K;
    hipLaunchKernelGGL(rhs_amax_rows_kernel, dim3((unsigned)((G * K + 3) / 4)), dim3(256), 0,
                       st, wp, G * K, N, scales);
  }
  dim3 grid((unsigned)(N / 64), (unsigned)(K / 64), (unsigned)G);
  if (fmt == FMT_E4M3)
    hipLaunchKernelGGL(rhs_quantize_kernel<FMT_E4M3>, grid, dim3(256), 0, st, wp, K, N, kblk,
                       scales, axis, layout_nk, codes);
  else
    hipLaunchKernelGGL(rhs_quantize_kernel<FMT_E5M2>, grid, dim3(256), 0, st, wp, K, N, kblk,
                       scales, axis, layout_nk, codes);
  const unsigned b = (unsigned)((nch + 255) / 256);
  if (fmt == FMT_E4M3)
    hipLaunchKernelGGL(rhs_scales_kernel<FMT_E4M3>, dim3(b), dim3(256), 0, st, scales, nch);
  else
    hipLaunchKernelGGL(rhs_scales_kernel<FMT_E5M2>, dim3(b), dim3(256), 0, st, scales, nch);
  return hipGetLastError();
}

}  // namespace gmm
