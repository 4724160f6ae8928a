// SwiGLU backward on gfx950: the elementwise step between the down projection's dlhs and
// the merged gate|up dlhs of an MoE feed-forward block ("FP8 Megablox for batch split",
// Description (2): the gate and up projections W0 | W1 merged along N).
//
// With gu = [g | u] (the merged forward product, [M, 2 I]) and dh = dL/dh ([M, I]),
// h = silu(g) * u and s = sigmoid(g) = 1 / (1 + exp(-g)):
//   dL/dg = dh * u * s * (1 + g * (1 - s))      dL/du = dh * silu(g) = dh * g * s
// computed in fp32 from the bf16 inputs (s through the hardware exp2 and reciprocal,
// about one ulp each; the other operations rounded to nearest), and stored as
// d_gu = [dL/dg | dL/du] in bf16 (round to nearest even).  HBM-bound: it reads 6 and
// writes 4 bytes per channel and row.
#include <algorithm>

#include "kernels.hpp"

namespace gmm {

namespace {

// 8 channels per thread (16-byte accesses), grid-stride over the M * I / 8 pieces.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t* __restrict__ dh,
                                                         const uint16_t* __restrict__ gu,
                                                         uint16_t* __restrict__ d_gu,
                                                         int64_t M, int64_t I) {
  const int64_t per_row = I / 8;
  const int64_t total = M * per_row;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * 256) {
    const int64_t m = t / per_row, c = (t - m * per_row) * 8;
    const v4u dv = *reinterpret_cast<const v4u*>(dh + m * I + c);
    const v4u gv = *reinterpret_cast<const v4u*>(gu + m * 2 * I + c);
    const v4u uv = *reinterpret_cast<const v4u*>(gu + m * 2 * I + I + c);
    v4u og, ou;
    swiglu_bwd8(dv, gv, uv, og, ou);
    *reinterpret_cast<v4u*>(d_gu + m * 2 * I + c) = og;
    *reinterpret_cast<v4u*>(d_gu + m * 2 * I + I + c) = ou;
  }
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ w, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    w[i] = 0u;
}

// the dynamic-scale rule of the quantizer's prepass: s = RNE_f32(amax / qmax)
template <int FMT>
__global__ __launch_bounds__(256) void amax_bits_to_scales_kernel(uint32_t* __restrict__ w,
                                                                  int64_t nb) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b < nb) w[b] = __float_as_uint(__fdiv_rn(__uint_as_float(w[b] << 16), qmax<FMT>()));
}

}  // namespace

hipError_t launch_zero_words(uint32_t* words, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, st, words, n);
  return hipGetLastError();
}

hipError_t launch_amax_bits_to_scales(int fmt, uint32_t* words, int64_t nb, hipStream_t st) {
  if (nb <= 0) return hipSuccess;
  const dim3 grid((unsigned)((nb + 255) / 256));
  if (fmt == FMT_E4M3)
    hipLaunchKernelGGL(amax_bits_to_scales_kernel<FMT_E4M3>, grid, dim3(256), 0, st, words, nb);
  else
    hipLaunchKernelGGL(amax_bits_to_scales_kernel<FMT_E5M2>, grid, dim3(256), 0, st, words, nb);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* dh, const uint16_t* gu, uint16_t* d_gu, int64_t M,
                             int64_t I, hipStream_t st) {
  const int64_t pieces = M * (I / 8);
  if (pieces == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((pieces + 255) / 256, 256 * 16);
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)blocks), dim3(256), 0, st, dh, gu, d_gu,
                     M, I);
  return hipGetLastError();
}

}  // namespace gmm
