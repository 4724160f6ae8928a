// Kernel launch interface shared by the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace gmm {

constexpr int AMAX_SPLIT = 8;    // row slices per 128-row block in the abs-max prepass
constexpr int MAX_GROUPS = 1024;
constexpr int ROUTE_CHUNK = 256;  // slots per chunk of the routing sort

// Grouped GEMM: out[M, Nout] = A[M, Kc] x B(g) for the rows of group g.
// B is either "contraction-contiguous" codes [G, Nout, Kc] (b_trans == 0) or
// "output-contiguous" codes [G, Kc, Nout] (b_trans == 1).
struct GemmParams {
  const void* a;             // bf16 values or fp8 codes, [M, Kc]
  const uint8_t* b;          // fp8 codes
  const float* b_scale;      // [G, Nout], per output channel
  const int32_t* group_sizes;
  void* out;                 // [M, Nout] bf16 or f32
  const float* a_scale_blk;  // dynamic: per-block scale (inverse derived in-kernel); else null
  float a_inv_static;
  float a_scale_static;
  int64_t M;
  int32_t Kc, Nout, G;
  int32_t g_before;          // group window: the G groups after the first g_before ones
  int32_t out_f32;
  // SwiGLU epilogue (gmm_fwd_swiglu): B holds the merged [W0 | W1] channels (Nout = 2 I),
  // out is h [M, I], gu (optional) the product itself [M, 2 I]
  void* gu;
  // h as fp8 codes (1 + format; 0: h in the output dtype) under a static scale's inverse,
  // or under dynamic scales per row and 128-channel block, written to h_scales [M, I/128]
  int32_t h_codes;
  float h_inv;
  float* h_scales;
  // workspace of SPLIT_SLOTS partial tiles (the tail split of gmm_kernel), or null: no split
  float* split_ws;
  // dlhs of the down projection with the SwiGLU backward in its epilogue: gu = [g | u]
  // bf16 [M, 2 Nout] of the forward; out is then d_gu bf16 [M, 2 Nout] (the product, dh,
  // is rounded to bf16 and used in the epilogue only).  Null: out holds the product.
  const uint16_t* bwd_gu;
  // with bwd_gu, optionally: per 128-row block of d_gu (blocks aligned to row 0) the
  // largest bf16 magnitude bits (absmax_bits16) of its values, by atomic max into words
  // that start at zero; null: none
  uint32_t* bwd_amax;
};

// The tail split of the grouped GEMM: CUs per XCD that one round of tiles fills, the most
// slices per tile, and the partial-sum slots (one 256 x 256 fp32 tile each) it can use.
constexpr int SPLIT_CUS = 32;
constexpr int SPLIT_MAX = 8;
// a tile is cut only when that saves its CU at least this many 128-deep steps: below it,
// the partial sums' stores and the fixup pass cost about what the cut saves
constexpr int SPLIT_MIN_SAVED = 48;
constexpr int SPLIT_SLOTS = 8 * SPLIT_CUS;
constexpr size_t SPLIT_SLOT_BYTES = size_t(256) * 256 * 4;

// tgmm: out[g] = A_g^T [Kout, m] x B_g [m, Nout], contraction over the rows of group g.
struct TgmmParams {
  const void* a;             // [M, Kout]: bf16 values, or fp8 codes when a_codes
  const void* b;             // [M, Nout]: bf16 values, or fp8 codes when b_codes
  const int32_t* group_sizes;
  void* out;                 // [G, Kout, Nout] bf16 or f32
  int32_t* plan;             // workspace: tgmm_plan_words(G) words
  float* scprod;             // workspace: one scale product per 128-row block
  float* ratio;              // workspace: ceil(M / 128) + 2 G floats
  uint8_t* a_q;              // workspace (bf16 a only): its codes, row-major [M, Kout]
  uint8_t* b_q;              // workspace (bf16 b only): its codes, row-major [M, Nout]
  const float* a_scale_blk;  // dynamic: per-block scales; null -> static
  const float* b_scale_blk;
  float a_inv_static, a_scale_static, b_inv_static, b_scale_static;
  int64_t M;
  int32_t Kout, Nout, G;
  int32_t g_before;          // group window: the G groups after the first g_before ones
  int32_t out_f32;
  int32_t a_codes, b_codes;  // the operand is fp8 codes quantized beforehand
};

// forward with block-wise scales: out[M, N] from fp8 A [M, K] (scales [M, K / bk]) and
// fp8 B [G, N, K] (scales [G, K / bk, N])
struct BsParams {
  const uint8_t* a;
  const uint8_t* b;
  const float* a_scale;
  const float* b_scale;
  const int32_t* group_sizes;
  void* out;
  int64_t M;
  int32_t K, N, G, bk;
  int32_t out_f32;
  // b_scale layout: 0 = [G, K / bk, N] (the forward's), 1 = [G, N, K / bk] (per output
  // channel, as the block-wise dlhs's weight copy comes out of the sub-channel quantizer)
  int32_t b_scale_nmajor;
};

// plan words: off, cnt, seg (G + 1), wide, final scale per group, one any-wide flag
inline int64_t tgmm_plan_words(int G) { return 6 * (int64_t)G + 2; }

hipError_t launch_gemm(int a_fmt, int b_fmt, bool a_fp8, bool b_trans, const GemmParams& p,
                       hipStream_t st);
// fp8-A product over merged gate|up channels with the SwiGLU epilogue
hipError_t launch_gemm_swiglu(int a_fmt, const GemmParams& p, hipStream_t st);
// d_gu [M, 2 I] from dh [M, I] and gu [M, 2 I], all bf16
hipError_t launch_swiglu_bwd(const uint16_t* dh, const uint16_t* gu, uint16_t* d_gu, int64_t M,
                             int64_t I, hipStream_t st);
// words[0 .. n) = 0 (a fill kernel: no memset node where a caller captures a graph)
hipError_t launch_zero_words(uint32_t* words, int64_t n, hipStream_t st);
// in place: block magnitude bits (absmax_bits16) -> dynamic scales RNE_f32(amax / qmax)
hipError_t launch_amax_bits_to_scales(int fmt, uint32_t* words, int64_t nb, hipStream_t st);
// routing sort (workspace: counts, route_chunks(n) * (G + 1) ints, and dest_all, the row
// of every slot, n ints) and the row gather
int64_t route_chunks(int64_t n);
hipError_t launch_route(const int32_t* ids, int64_t n, int k, int G, int32_t* counts,
                        int32_t* dest_all, int32_t* gs, int32_t* row_of_slot,
                        int32_t* slot_of_row, const void* x, int64_t row_bytes, void* x_perm,
                        hipStream_t st);
// weighted sum of every token's expert rows (w may be null: weights 1)
hipError_t launch_combine(const uint16_t* y, int64_t T, int k, int64_t H, int64_t rows,
                          const int32_t* row_of_slot, const float* w, uint16_t* out,
                          hipStream_t st);
// zeros into the rows of out [M, row_bytes] outside the window's rows
hipError_t launch_zero_rows_outside(void* out, int64_t M, int64_t row_bytes,
                                   const int32_t* gs, int g_before, int G, hipStream_t st);
hipError_t launch_tgmm(int a_fmt, int b_fmt, const TgmmParams& p, hipStream_t st);
hipError_t launch_dynamic_scales(int fmt, const void* x, int64_t R, int64_t C,
                                 uint32_t* partial, float* scales_out, hipStream_t st);
hipError_t launch_quantize_rows(int fmt, const void* x, int64_t R, int64_t C,
                                const float* scale_blk, float inv_static, uint8_t* codes,
                                hipStream_t st);
// axis 0 scales every (g, block of kblk contraction rows, n): [G, K / kblk, N] (kblk = K is
// per channel); axis 1 every (g, k): [G, K]
hipError_t launch_quantize_rhs(int fmt, int axis, int layout_nk, int64_t G, int64_t K,
                               int64_t N, int64_t kblk, const void* w, uint8_t* codes,
                               float* scales, hipStream_t st);
hipError_t launch_gemm_blockwise(int a_fmt, const BsParams& p, hipStream_t st);
// the folded gradient: codes and 128-row-block scales of grad * s[g(m), n]
// (partial: ceil(M / 128) * AMAX_SPLIT words of workspace)
hipError_t launch_quantize_folded(int fmt, const void* x, int64_t M, int64_t N,
                                  const float* col_scales, const int32_t* gs, int G,
                                  uint32_t* partial, float* scales, uint8_t* codes,
                                  hipStream_t st);
hipError_t launch_quantize_subchannel(int fmt, const void* x, int64_t M, int64_t K, int bk,
                                      uint8_t* codes, float* scales, hipStream_t st);

}  // namespace gmm
