// C-ABI entry points: argument validation, workspace layout and kernel dispatch.
// Every check runs on the host before anything is enqueued.
#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/gmm_fp8.h"
#include "kernels.hpp"

using namespace gmm;

namespace {

constexpr int64_t MAX_DIM = int64_t(1) << 22;  // K, N limit: keeps every tile offset 32-bit

bool env_flag(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && v[0] != '0';
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

int64_t nblocks(int64_t rows) { return (rows + BLOCK_ROWS - 1) / BLOCK_ROWS; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace of one bf16 operand whose dynamic scales the call computes: abs-max
// partials, plus room for the scales when the caller does not ask for them.
size_t dyn_ws_bytes(int64_t rows) {
  const size_t nb = (size_t)nblocks(rows);
  return align256(nb * AMAX_SPLIT * 4) + align256(nb * 4);
}

struct DynWs {
  uint32_t* partial;
  float* scale;
};

DynWs carve(void* base, int64_t rows) {
  const size_t nb = (size_t)nblocks(rows);
  uint8_t* p = (uint8_t*)base;
  DynWs w;
  w.partial = (uint32_t*)p;
  w.scale = (float*)(p + align256(nb * AMAX_SPLIT * 4));
  return w;
}

// The call runs the abs-max prepass itself (and needs workspace) only for a bf16
// operand with GMM_SCALE_DYNAMIC.
// tgmm: plan words, per-block scale products, per-segment-block ratios, and the row-major
// codes of each operand that arrives as bf16 (quantized once by the call).
size_t tgmm_ws_bytes(int64_t M, int64_t K, int64_t N, int32_t G, bool a_codes, bool b_codes) {
  return align256((size_t)tgmm_plan_words(G) * 4) + align256((size_t)nblocks(M) * 4) +
         align256((size_t)(nblocks(M) + 2 * G) * 4) + (a_codes ? 0 : align256((size_t)M * K)) +
         (b_codes ? 0 : align256((size_t)M * N));
}

bool needs_dyn_ws(const gmm_operand_t* op) {
  return op && op->kind == GMM_OPERAND_BF16 && op->scaling == GMM_SCALE_DYNAMIC;
}

// Per-block scales are an input for DYNAMIC_GIVEN and for pre-quantized dynamic codes.
bool scales_are_input(const gmm_operand_t* op) {
  return op->scaling == GMM_SCALE_DYNAMIC_GIVEN ||
         (op->kind == GMM_OPERAND_FP8 && op->scaling == GMM_SCALE_DYNAMIC);
}

// Resolve the scaling of one operand for the kernels: static scale and inverse, or a
// pointer to per-block scales (running the prepass when the call computes them).
struct Scaling {
  const float* blk = nullptr;
  float s = 0.0f, inv = 0.0f;
};

gmm_status_t resolve_scaling(const gmm_operand_t* op, const void* x, int64_t R, int64_t C,
                             float* user_scales, void* ws, hipStream_t st, Scaling& out) {
  if (op->scaling == GMM_SCALE_STATIC) {
    out.s = op->static_scale;
    out.inv = 1.0f / op->static_scale;  // IEEE division on the host: RNE(1/s)
    return GMM_OK;
  }
  if (scales_are_input(op)) {
    out.blk = user_scales;
    return GMM_OK;
  }
  DynWs w = carve(ws, R);
  float* dst = user_scales ? user_scales : w.scale;
  if (R > 0 && launch_dynamic_scales(op->format, x, R, C, w.partial, dst, st) != hipSuccess)
    return GMM_ERR_HIP;
  out.blk = dst;
  return GMM_OK;
}

gmm_status_t check_operand(const gmm_operand_t* op) {
  if (!op) return GMM_ERR_NULL;
  if (op->kind != GMM_OPERAND_BF16 && op->kind != GMM_OPERAND_FP8) return GMM_ERR_RECIPE;
  if (op->format != GMM_FP8_E4M3 && op->format != GMM_FP8_E5M2) return GMM_ERR_RECIPE;
  if (op->scaling != GMM_SCALE_STATIC && op->scaling != GMM_SCALE_DYNAMIC &&
      op->scaling != GMM_SCALE_DYNAMIC_GIVEN)
    return GMM_ERR_RECIPE;
  if (op->scaling == GMM_SCALE_STATIC) {
    const float s = op->static_scale;
    // finite, positive, normal: guards against underflow and scales close to zero
    if (!std::isfinite(s) || !(s >= FLT_MIN)) return GMM_ERR_SCALE;
  }
  return GMM_OK;
}

gmm_status_t check_shape(int64_t M, int64_t K, int64_t N, int32_t G) {
  if (M < 0 || M >= (int64_t(1) << 31)) return GMM_ERR_SHAPE;
  if (G < 1 || G > GMM_MAX_GROUPS) return GMM_ERR_SHAPE;
  if (K <= 0 || N <= 0 || K % 128 || N % 128 || K > MAX_DIM || N > MAX_DIM) return GMM_ERR_SHAPE;
  if (K * N >= (int64_t(1) << 32)) return GMM_ERR_SHAPE;
  return GMM_OK;
}

// GMM_CHECK=1: synchronous validation of group_sizes (debug mode).
gmm_status_t check_group_sizes(const int32_t* gs, int32_t G, int64_t M, hipStream_t st) {
  if (!env_flag("GMM_CHECK")) return GMM_OK;
  std::vector<int32_t> h(G);
  if (hipMemcpyAsync(h.data(), gs, sizeof(int32_t) * G, hipMemcpyDeviceToHost, st) != hipSuccess)
    return GMM_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return GMM_ERR_HIP;
  int64_t sum = 0;
  for (int32_t v : h) {
    if (v < 0) return GMM_ERR_GROUP_SIZES;
    sum += v;
  }
  return sum == M ? GMM_OK : GMM_ERR_GROUP_SIZES;
}

void trace(const char* what, int64_t M, int64_t K, int64_t N, int32_t G) {
  if (env_flag("GMM_TRACE"))
    std::fprintf(stderr, "[gmm_fp8] %s M=%lld K=%lld N=%lld G=%d\n", what, (long long)M,
                 (long long)K, (long long)N, G);
}

// A bf16 operand is quantized once into the workspace, and the product then reads fp8
// codes, when the call has at least this many 256-column output tiles and the workspace
// holds the codes: the in-kernel quantization repeats per output tile, and on gfx950 its
// vector work (about 20 instructions per MFMA) cannot hide under the matrix core.
constexpr int64_t QUANT_ONCE_MIN_TILES = 4;

size_t quant_once_bytes(int64_t M, int64_t Kc) { return align256((size_t)M * Kc); }

bool quant_once_applies(int64_t Nout) { return Nout <= 0 || (Nout + 255) / 256 >= QUANT_ONCE_MIN_TILES; }

// The tail split of gmm_dlhs (partial sums of the last round's tiles) needs SPLIT_SLOTS
// fp32 tiles of workspace.  It can occur when the call has more 256 x 256 tiles than 8
// XCDs x SPLIT_CUS CUs take in one round and a contraction long enough for the split to
// save SPLIT_MIN_SAVED steps (with SPLIT_MAX slices); without that workspace the call
// runs unsplit.
size_t split_ws_bytes(int64_t M, int64_t Kc, int64_t Nout, int32_t G) {
  const int64_t max_tiles = ((M + 255) / 256 + G) * ((Nout + 255) / 256);
  const int64_t nk = Kc / 128;
  return max_tiles > SPLIT_SLOTS && nk - nk / SPLIT_MAX >= SPLIT_MIN_SAVED
             ? SPLIT_SLOTS * SPLIT_SLOT_BYTES : 0;
}

// Shared body of gmm_fwd / gmm_dlhs: out[M, Nout] = A[M, Kc] x B.
// The products run over the window of G groups that follows the first g_before of the
// G_total in group_sizes; output rows outside the window are zero-filled.
gmm_status_t grouped_gemm(const char* name, const gmm_operand_t* aop, int32_t rhs_format,
                          bool b_trans, int32_t out_dtype, int64_t M, int64_t Kc,
                          int64_t Nout, int32_t G_total, int32_t g_before, int32_t G,
                          const void* a, float* a_scales,
                          const uint8_t* rhs, const float* rhs_scales,
                          const int32_t* group_sizes, void* out, void* workspace,
                          size_t workspace_bytes, hipStream_t st, bool swiglu = false,
                          void* gu = nullptr, const gmm_operand_t* h_op = nullptr,
                          float* h_scales = nullptr, const void* bwd_gu = nullptr,
                          float* bwd_scales = nullptr, int32_t bwd_fmt = 0) {
  gmm_status_t s = check_operand(aop);
  if (s != GMM_OK) return s;
  // SwiGLU with fp8 h: codes under a validated static per-tensor scale, or (h_scales)
  // under dynamic scales per row and 128-channel block
  if (h_op) {
    if ((s = check_operand(h_op)) != GMM_OK) return s;
    if (h_op->kind != GMM_OPERAND_FP8 ||
        (h_op->scaling != GMM_SCALE_STATIC && h_op->scaling != GMM_SCALE_DYNAMIC))
      return GMM_ERR_RECIPE;
    if (h_op->scaling == GMM_SCALE_DYNAMIC && M > 0 && !h_scales) return GMM_ERR_NULL;
  }
  if (!h_op || h_op->scaling != GMM_SCALE_DYNAMIC) h_scales = nullptr;
  if (rhs_format != GMM_FP8_E4M3) return GMM_ERR_RECIPE;  // weights are e4m3 codes
  if (out_dtype != GMM_OUT_BF16 && out_dtype != GMM_OUT_F32) return GMM_ERR_RECIPE;
  if ((s = check_shape(M, Kc, Nout, G_total)) != GMM_OK) return s;
  if (g_before < 0 || G < 1 || g_before > G_total - G) return GMM_ERR_SHAPE;
  const bool window = G != G_total;
  // SwiGLU: Nout = 2 I channels, I a multiple of 128, contraction-contiguous weights
  if (swiglu && (Nout % 256 || b_trans)) return swiglu && b_trans ? GMM_ERR_RECIPE : GMM_ERR_SHAPE;
  // SwiGLU backward in the dlhs epilogue: bf16 dh of Nout = I channels, d_gu [M, 2 I]
  if (bwd_gu && (swiglu || h_op || out_dtype != GMM_OUT_BF16)) return GMM_ERR_RECIPE;
  if (bwd_gu && (window || Nout > MAX_DIM / 2)) return GMM_ERR_SHAPE;
  // the kernels number output tiles with 32-bit integers
  if ((M / 256 + 1 + G) * ((Nout + 255) / 256) >= (int64_t(1) << 31)) return GMM_ERR_SHAPE;
  if (!rhs || !rhs_scales || !group_sizes) return GMM_ERR_NULL;
  if (M > 0 && (!a || !out)) return GMM_ERR_NULL;
  const bool a_fp8 = aop->kind == GMM_OPERAND_FP8;
  const bool dyn = aop->scaling != GMM_SCALE_STATIC;
  if (scales_are_input(aop) && M > 0 && !a_scales) return GMM_ERR_NULL;
  for (const void* ptr : {(const void*)a, (const void*)rhs, (const void*)rhs_scales,
                          (const void*)group_sizes, (const void*)out, (const void*)a_scales,
                          (const void*)workspace})
    if (ptr && !aligned16(ptr)) return GMM_ERR_ALIGN;
  const size_t ws_need = needs_dyn_ws(aop) ? dyn_ws_bytes(M) : 0;
  if (ws_need && (!workspace || workspace_bytes < ws_need)) return GMM_ERR_WORKSPACE;
  // Workspace, in order: the dynamic scales' pass, the tail split's partial tiles (dlhs
  // only: a forward stays bit-identical to the SwiGLU forward's product half, whose tiles
  // pair gate and up channels differently), the quantize-once codes.  The split takes
  // its room first, so that the sizes of both routes (GMM_OP_DLHS, GMM_OP_DLHS_FUSED)
  // give both the same split.
  const bool is_dlhs = std::strncmp(name, "gmm_dlhs", 8) == 0;
  // (the fused SwiGLU backward has no tail split: its epilogue needs the whole sum)
  const size_t split_need = is_dlhs && !bwd_gu ? split_ws_bytes(M, Kc, Nout, G) : 0;
  const bool split = split_need && workspace && workspace_bytes >= ws_need + split_need;
  const size_t ws_base = ws_need + (split ? split_need : 0);
  const bool quant_once = !a_fp8 && (swiglu || quant_once_applies(Nout)) && workspace &&
                          workspace_bytes >= ws_base + quant_once_bytes(M, Kc);
  // the SwiGLU epilogue exists on the fp8-A route only: a bf16 lhs is quantized once
  if (swiglu && !a_fp8 && !quant_once) return GMM_ERR_WORKSPACE;
  const size_t ws_used = ws_base + (quant_once ? quant_once_bytes(M, Kc) : 0);
  const size_t a_bytes = (size_t)M * Kc * (a_fp8 ? 1 : 2);
  const size_t esize = out_dtype == GMM_OUT_F32 ? 4 : 2;
  const size_t out_bytes =
      (size_t)M * (swiglu ? Nout / 2 : bwd_gu ? 2 * Nout : Nout) * (h_op ? 1 : esize);
  const size_t gu_bytes = swiglu && gu ? (size_t)M * Nout * esize : 0;
  const size_t b_bytes = (size_t)G * Kc * Nout;
  const size_t as_bytes = (size_t)nblocks(M) * 4;
  if (overlaps(out, out_bytes, a, a_bytes) || overlaps(out, out_bytes, rhs, b_bytes) ||
      overlaps(out, out_bytes, rhs_scales, (size_t)G * Nout * 4) ||
      overlaps(out, out_bytes, group_sizes, (size_t)G_total * 4) ||
      (a_scales && overlaps(out, out_bytes, a_scales, as_bytes)) ||
      (needs_dyn_ws(aop) && overlaps(a_scales, as_bytes, a, a_bytes)) ||
      overlaps(workspace, ws_used, a, a_bytes) || overlaps(workspace, ws_used, out, out_bytes) ||
      overlaps(workspace, ws_used, a_scales, as_bytes))
    return GMM_ERR_ALIAS;
  if (gu_bytes && (overlaps(gu, gu_bytes, a, a_bytes) || overlaps(gu, gu_bytes, rhs, b_bytes) ||
                   overlaps(gu, gu_bytes, rhs_scales, (size_t)G * Nout * 4) ||
                   overlaps(gu, gu_bytes, group_sizes, (size_t)G_total * 4) ||
                   overlaps(gu, gu_bytes, out, out_bytes) ||
                   overlaps(gu, gu_bytes, workspace, ws_used) ||
                   overlaps(gu, gu_bytes, a_scales, as_bytes)))
    return GMM_ERR_ALIAS;
  if (gu && !aligned16(gu)) return GMM_ERR_ALIGN;
  const size_t bg_bytes = bwd_gu ? (size_t)M * 2 * Nout * 2 : 0;
  if (bg_bytes && (overlaps(bwd_gu, bg_bytes, out, out_bytes) ||
                   overlaps(bwd_gu, bg_bytes, workspace, ws_used) ||
                   overlaps(bwd_gu, bg_bytes, a_scales, as_bytes)))
    return GMM_ERR_ALIAS;
  if (bwd_gu && !aligned16(bwd_gu)) return GMM_ERR_ALIGN;
  // d_gu's dynamic block scales, gathered in the same epilogue
  if (!bwd_gu) bwd_scales = nullptr;
  const size_t bs_bytes = bwd_scales ? (size_t)nblocks(M) * 4 : 0;
  if (bs_bytes && (overlaps(bwd_scales, bs_bytes, out, out_bytes) ||
                   overlaps(bwd_scales, bs_bytes, bwd_gu, bg_bytes) ||
                   overlaps(bwd_scales, bs_bytes, a, a_bytes) ||
                   overlaps(bwd_scales, bs_bytes, rhs_scales, (size_t)G * Nout * 4) ||
                   overlaps(bwd_scales, bs_bytes, group_sizes, (size_t)G_total * 4) ||
                   overlaps(bwd_scales, bs_bytes, workspace, ws_used) ||
                   overlaps(bwd_scales, bs_bytes, a_scales, as_bytes)))
    return GMM_ERR_ALIAS;
  if (bwd_scales && !aligned16(bwd_scales)) return GMM_ERR_ALIGN;
  const size_t hs_bytes = h_scales ? (size_t)M * (Nout / 256) * 4 : 0;  // [M, I / 128]
  if (hs_bytes && (overlaps(h_scales, hs_bytes, a, a_bytes) || overlaps(h_scales, hs_bytes, rhs, b_bytes) ||
                   overlaps(h_scales, hs_bytes, rhs_scales, (size_t)G * Nout * 4) ||
                   overlaps(h_scales, hs_bytes, group_sizes, (size_t)G_total * 4) ||
                   overlaps(h_scales, hs_bytes, out, out_bytes) ||
                   (gu_bytes && overlaps(h_scales, hs_bytes, gu, gu_bytes)) ||
                   overlaps(h_scales, hs_bytes, workspace, ws_used) ||
                   overlaps(h_scales, hs_bytes, a_scales, as_bytes)))
    return GMM_ERR_ALIAS;
  if (h_scales && !aligned16(h_scales)) return GMM_ERR_ALIGN;
  if ((s = check_group_sizes(group_sizes, G_total, M, st)) != GMM_OK) return s;
  trace(name, M, Kc, Nout, G);
  if (M == 0) return GMM_OK;
  if (window) {
    // rows of the groups outside the window hold zeros (h and gu of the SwiGLU forward too)
    const int64_t esz = h_op ? 1 : (int64_t)esize;
    if (launch_zero_rows_outside(out, M, (swiglu ? Nout / 2 : Nout) * esz, group_sizes, g_before,
                                 G, st) != hipSuccess ||
        (gu_bytes && launch_zero_rows_outside(gu, M, Nout * (int64_t)esize, group_sizes, g_before,
                                              G, st) != hipSuccess))
      return GMM_ERR_HIP;
  }

  GemmParams p{};
  p.a = a;
  p.b = rhs;
  p.b_scale = rhs_scales;
  p.group_sizes = group_sizes;
  p.out = out;
  p.M = M;
  p.Kc = (int32_t)Kc;
  p.Nout = (int32_t)Nout;
  p.G = G;
  p.g_before = g_before;
  p.out_f32 = out_dtype == GMM_OUT_F32;
  p.gu = gu;
  p.bwd_gu = (const uint16_t*)bwd_gu;
  p.bwd_amax = (uint32_t*)bwd_scales;
  p.split_ws = split ? (float*)((uint8_t*)workspace + ws_need) : nullptr;
  if (h_op) {
    p.h_codes = 1 + h_op->format;
    // the static scale's inverse: IEEE division on the host, RNE(1/s)
    p.h_inv = h_scales ? 0.0f : 1.0f / h_op->static_scale;
    p.h_scales = h_scales;
  }
  Scaling sc;
  if ((s = resolve_scaling(aop, a, M, Kc, a_scales, workspace, st, sc)) != GMM_OK) return s;
  p.a_scale_blk = sc.blk;
  p.a_scale_static = sc.s;
  p.a_inv_static = sc.inv;
  bool a_codes = a_fp8;
  if (quant_once) {
    uint8_t* codes = (uint8_t*)workspace + ws_base;
    if (launch_quantize_rows(aop->format, (const uint16_t*)a, M, Kc, sc.blk, sc.inv, codes, st) !=
        hipSuccess)
      return GMM_ERR_HIP;
    p.a = codes;
    a_codes = true;
  }
  if (bwd_scales && launch_zero_words(p.bwd_amax, nblocks(M), st) != hipSuccess) return GMM_ERR_HIP;
  const hipError_t e = swiglu ? launch_gemm_swiglu(aop->format, p, st)
                              : launch_gemm(aop->format, FMT_E4M3, a_codes, b_trans, p, st);
  if (e != hipSuccess) return GMM_ERR_HIP;
  if (bwd_scales && launch_amax_bits_to_scales(bwd_fmt, p.bwd_amax, nblocks(M), st) != hipSuccess)
    return GMM_ERR_HIP;
  return GMM_OK;
}

// ---- the scratch array of gmm_fwd_noalloc ----
// Its workspace is the dynamic-scale workspace of GMM_NOALLOC_MAX_ROWS rows: abs-max
// partials, then the block scales.
constexpr size_t NOALLOC_SCRATCH_BYTES =
    (size_t((GMM_NOALLOC_MAX_ROWS + BLOCK_ROWS - 1) / BLOCK_ROWS) * AMAX_SPLIT * 4 + 255) / 256 * 256 +
    (size_t((GMM_NOALLOC_MAX_ROWS + BLOCK_ROWS - 1) / BLOCK_ROWS) * 4 + 255) / 256 * 256;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The device address of the current device's copy of `scratch`, looked up on the first
// call with that device current.  In host code the array's name is only a stand-in: the
// kernels are handed this address.
gmm_status_t noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return GMM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GMM_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GMM_OK;
}

// Shared body of gmm_fwd_blockwise and gmm_dlhs_blockwise: out[M, N] from lhs codes
// [M, K] (scales [M, K / bk]) and rhs codes [G, N, K] (contraction contiguous) with scales
// [G, K / bk, N] or, n_major, [G, N, K / bk].
gmm_status_t blockwise_gemm(const char* name, int32_t lhs_format, int32_t out_dtype, int64_t M,
                            int64_t K, int64_t N, int32_t G, int64_t bk, const uint8_t* lhs,
                            const float* lhs_scales, const uint8_t* rhs, const float* rhs_scales,
                            bool n_major, const int32_t* group_sizes, void* out,
                            hipStream_t stream) {
  if (lhs_format != GMM_FP8_E4M3 && lhs_format != GMM_FP8_E5M2) return GMM_ERR_RECIPE;
  if (out_dtype != GMM_OUT_BF16 && out_dtype != GMM_OUT_F32) return GMM_ERR_RECIPE;
  gmm_status_t s = check_shape(M, K, N, G);
  if (s != GMM_OK) return s;
  if (bk < 128 || bk % 128 || K % bk) return GMM_ERR_SHAPE;
  if ((M / 128 + 1 + G) * (N / 128) >= (int64_t(1) << 31)) return GMM_ERR_SHAPE;
  if (!rhs || !rhs_scales || !group_sizes) return GMM_ERR_NULL;
  if (M > 0 && (!lhs || !lhs_scales || !out)) return GMM_ERR_NULL;
  for (const void* ptr : {(const void*)lhs, (const void*)lhs_scales, (const void*)rhs,
                          (const void*)rhs_scales, (const void*)group_sizes, (const void*)out})
    if (ptr && !aligned16(ptr)) return GMM_ERR_ALIGN;
  const int64_t nkb = K / bk;
  const size_t ob = (size_t)M * N * (out_dtype == GMM_OUT_F32 ? 4 : 2);
  if (overlaps(out, ob, lhs, (size_t)M * K) || overlaps(out, ob, lhs_scales, (size_t)M * nkb * 4) ||
      overlaps(out, ob, rhs, (size_t)G * K * N) ||
      overlaps(out, ob, rhs_scales, (size_t)G * nkb * N * 4) ||
      overlaps(out, ob, group_sizes, (size_t)G * 4))
    return GMM_ERR_ALIAS;
  if ((s = check_group_sizes(group_sizes, G, M, stream)) != GMM_OK) return s;
  trace(name, M, K, N, G);
  if (M == 0) return GMM_OK;
  BsParams p{};
  p.a = lhs;
  p.b = rhs;
  p.a_scale = lhs_scales;
  p.b_scale = rhs_scales;
  p.group_sizes = group_sizes;
  p.out = out;
  p.M = M;
  p.K = (int32_t)K;
  p.N = (int32_t)N;
  p.G = G;
  p.bk = (int32_t)bk;
  p.out_f32 = out_dtype == GMM_OUT_F32;
  p.b_scale_nmajor = n_major;
  return launch_gemm_blockwise(lhs_format, p, stream) == hipSuccess ? GMM_OK : GMM_ERR_HIP;
}

}  // namespace

extern "C" {

gmm_status_t gmm_fwd(const gmm_operand_t* lhs_op, int32_t rhs_format, int32_t rhs_layout,
                     int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G,
                     const void* lhs, float* lhs_scales, const uint8_t* rhs,
                     const float* rhs_scales, const int32_t* group_sizes, void* out,
                     void* workspace, size_t workspace_bytes, gmm_stream_t stream) {
  if (rhs_layout != GMM_RHS_KN && rhs_layout != GMM_RHS_NK) return GMM_ERR_RECIPE;
  // forward contracts over K: contiguous when the codes are stored [G, N, K]
  return grouped_gemm("gmm_fwd", lhs_op, rhs_format, rhs_layout == GMM_RHS_KN, out_dtype, M, K,
                      N, G, 0, G, lhs, lhs_scales, rhs, rhs_scales, group_sizes, out, workspace,
                      workspace_bytes, (hipStream_t)stream);
}

gmm_status_t gmm_fwd_noalloc(const gmm_operand_t* lhs_op, int32_t rhs_format, int32_t rhs_layout,
                             int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G,
                             const void* lhs, float* lhs_scales, const uint8_t* rhs,
                             const float* rhs_scales, const int32_t* group_sizes, void* out,
                             gmm_stream_t stream) {
  if (rhs_layout != GMM_RHS_KN && rhs_layout != GMM_RHS_NK) return GMM_ERR_RECIPE;
  if (M > GMM_NOALLOC_MAX_ROWS) return GMM_ERR_WORKSPACE;
  void* ws = nullptr;
  gmm_status_t s = noalloc_scratch(&ws);
  if (s != GMM_OK) return s;
  // only the dynamic-scale workspace fits: a bf16 lhs is quantized inside the product kernel
  const size_t ws_bytes = needs_dyn_ws(lhs_op) ? dyn_ws_bytes(M) : 0;
  return grouped_gemm("gmm_fwd_noalloc", lhs_op, rhs_format, rhs_layout == GMM_RHS_KN, out_dtype,
                      M, K, N, G, 0, G, lhs, lhs_scales, rhs, rhs_scales, group_sizes, out,
                      ws_bytes ? ws : nullptr, ws_bytes, (hipStream_t)stream);
}

gmm_status_t gmm_fwd_local(const gmm_operand_t* lhs_op, int32_t rhs_format, int32_t rhs_layout,
                           int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G_total,
                           int32_t group_offset, int32_t G_local, const void* lhs,
                           float* lhs_scales, const uint8_t* rhs, const float* rhs_scales,
                           const int32_t* group_sizes, void* out, void* workspace,
                           size_t workspace_bytes, gmm_stream_t stream) {
  if (rhs_layout != GMM_RHS_KN && rhs_layout != GMM_RHS_NK) return GMM_ERR_RECIPE;
  return grouped_gemm("gmm_fwd_local", lhs_op, rhs_format, rhs_layout == GMM_RHS_KN, out_dtype,
                      M, K, N, G_total, group_offset, G_local, lhs, lhs_scales, rhs, rhs_scales,
                      group_sizes, out, workspace, workspace_bytes, (hipStream_t)stream);
}

gmm_status_t gmm_dlhs(const gmm_operand_t* grad_op, int32_t rhs_format, int32_t rhs_layout,
                      int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G,
                      const void* grad, float* grad_scales, const uint8_t* rhs,
                      const float* rhs_scales, const int32_t* group_sizes, void* dlhs,
                      void* workspace, size_t workspace_bytes, gmm_stream_t stream) {
  if (rhs_layout != GMM_RHS_KN && rhs_layout != GMM_RHS_NK) return GMM_ERR_RECIPE;
  // dlhs contracts over N: contiguous when the codes are stored [G, K, N]
  return grouped_gemm("gmm_dlhs", grad_op, rhs_format, rhs_layout == GMM_RHS_NK, out_dtype, M,
                      N, K, G, 0, G, grad, grad_scales, rhs, rhs_scales, group_sizes, dlhs,
                      workspace, workspace_bytes, (hipStream_t)stream);
}

gmm_status_t gmm_dlhs_local(const gmm_operand_t* grad_op, int32_t rhs_format, int32_t rhs_layout,
                            int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G_total,
                            int32_t group_offset, int32_t G_local, const void* grad,
                            float* grad_scales, const uint8_t* rhs, const float* rhs_scales,
                            const int32_t* group_sizes, void* dlhs, void* workspace,
                            size_t workspace_bytes, gmm_stream_t stream) {
  if (rhs_layout != GMM_RHS_KN && rhs_layout != GMM_RHS_NK) return GMM_ERR_RECIPE;
  return grouped_gemm("gmm_dlhs_local", grad_op, rhs_format, rhs_layout == GMM_RHS_NK,
                      out_dtype, M, N, K, G_total, group_offset, G_local, grad, grad_scales, rhs,
                      rhs_scales, group_sizes, dlhs, workspace, workspace_bytes,
                      (hipStream_t)stream);
}

gmm_status_t gmm_dlhs_swiglu_bwd(const gmm_operand_t* grad_op, int32_t rhs_format,
                                 int32_t rhs_layout, int64_t M, int64_t I, int64_t N, int32_t G,
                                 const void* grad, float* grad_scales, const uint8_t* rhs,
                                 const float* rhs_scales, const int32_t* group_sizes,
                                 const void* gu, void* d_gu, int32_t d_gu_format,
                                 float* d_gu_scales, void* workspace, size_t workspace_bytes,
                                 gmm_stream_t stream) {
  if (rhs_layout != GMM_RHS_KN && rhs_layout != GMM_RHS_NK) return GMM_ERR_RECIPE;
  if (d_gu_scales && d_gu_format != GMM_FP8_E4M3 && d_gu_format != GMM_FP8_E5M2)
    return GMM_ERR_RECIPE;
  if (I <= 0 || I > MAX_DIM / 2) return GMM_ERR_SHAPE;
  if (M > 0 && !gu) return GMM_ERR_NULL;
  // dlhs of the down projection (contraction over its N = hidden columns, output I)
  return grouped_gemm("gmm_dlhs_swiglu_bwd", grad_op, rhs_format, rhs_layout == GMM_RHS_NK,
                      GMM_OUT_BF16, M, N, I, G, 0, G, grad, grad_scales, rhs, rhs_scales,
                      group_sizes, d_gu, workspace, workspace_bytes, (hipStream_t)stream, false,
                      nullptr, nullptr, nullptr, M > 0 ? gu : nullptr, d_gu_scales,
                      d_gu_format == GMM_FP8_E5M2 ? FMT_E5M2 : FMT_E4M3);
}

gmm_status_t gmm_fwd_swiglu(const gmm_operand_t* lhs_op, int32_t rhs_format, int32_t rhs_layout,
                            int32_t out_dtype, int64_t M, int64_t K, int64_t I, int32_t G,
                            const void* lhs, float* lhs_scales, const uint8_t* rhs,
                            const float* rhs_scales, const int32_t* group_sizes, void* gu,
                            void* h, void* workspace, size_t workspace_bytes,
                            gmm_stream_t stream) {
  if (rhs_layout != GMM_RHS_KN && rhs_layout != GMM_RHS_NK) return GMM_ERR_RECIPE;
  if (I <= 0 || I > MAX_DIM / 2) return GMM_ERR_SHAPE;
  return grouped_gemm("gmm_fwd_swiglu", lhs_op, rhs_format, rhs_layout == GMM_RHS_KN,
                      out_dtype, M, K, 2 * I, G, 0, G, lhs, lhs_scales, rhs, rhs_scales,
                      group_sizes, h, workspace, workspace_bytes, (hipStream_t)stream, true, gu);
}

gmm_status_t gmm_fwd_swiglu_fp8_subchannel(const gmm_operand_t* lhs_op, int32_t rhs_format,
                                           int32_t rhs_layout, int32_t gu_dtype, int64_t M,
                                           int64_t K, int64_t I, int32_t G, const void* lhs,
                                           float* lhs_scales, const uint8_t* rhs,
                                           const float* rhs_scales, const int32_t* group_sizes,
                                           void* gu, int32_t h_format, uint8_t* h_codes,
                                           float* h_scales, void* workspace,
                                           size_t workspace_bytes, gmm_stream_t stream) {
  if (rhs_layout != GMM_RHS_KN && rhs_layout != GMM_RHS_NK) return GMM_ERR_RECIPE;
  if (h_format != GMM_FP8_E4M3 && h_format != GMM_FP8_E5M2) return GMM_ERR_RECIPE;
  if (I <= 0 || I > MAX_DIM / 2) return GMM_ERR_SHAPE;
  const gmm_operand_t h_op{GMM_OPERAND_FP8, h_format, GMM_SCALE_DYNAMIC, 0.0f};
  return grouped_gemm("gmm_fwd_swiglu_fp8_subchannel", lhs_op, rhs_format,
                      rhs_layout == GMM_RHS_KN, gu_dtype, M, K, 2 * I, G, 0, G, lhs, lhs_scales,
                      rhs, rhs_scales, group_sizes, h_codes, workspace, workspace_bytes,
                      (hipStream_t)stream, true, gu, &h_op, h_scales);
}

gmm_status_t gmm_fwd_swiglu_fp8(const gmm_operand_t* lhs_op, int32_t rhs_format,
                                int32_t rhs_layout, int32_t gu_dtype, int64_t M, int64_t K,
                                int64_t I, int32_t G, const void* lhs, float* lhs_scales,
                                const uint8_t* rhs, const float* rhs_scales,
                                const int32_t* group_sizes, void* gu, const gmm_operand_t* h_op,
                                uint8_t* h_codes, void* workspace, size_t workspace_bytes,
                                gmm_stream_t stream) {
  if (!h_op) return GMM_ERR_NULL;
  if (h_op->scaling != GMM_SCALE_STATIC) return GMM_ERR_RECIPE;  // dynamic: the _subchannel call
  if (rhs_layout != GMM_RHS_KN && rhs_layout != GMM_RHS_NK) return GMM_ERR_RECIPE;
  if (I <= 0 || I > MAX_DIM / 2) return GMM_ERR_SHAPE;
  return grouped_gemm("gmm_fwd_swiglu_fp8", lhs_op, rhs_format, rhs_layout == GMM_RHS_KN,
                      gu_dtype, M, K, 2 * I, G, 0, G, lhs, lhs_scales, rhs, rhs_scales,
                      group_sizes, h_codes, workspace, workspace_bytes, (hipStream_t)stream, true,
                      gu, h_op);
}

size_t gmm_permute_workspace_size(int64_t T, int32_t k, int32_t G) {
  if (T < 0 || k < 1 || G < 1) return 0;
  return align256((size_t)route_chunks(T * k) * (G + 1) * 4) + align256((size_t)T * k * 4);
}

gmm_status_t gmm_permute(int64_t T, int32_t k, int32_t G, const int32_t* expert_ids,
                         int64_t row_bytes, const void* x, void* x_perm, int32_t* group_sizes,
                         int32_t* row_of_slot, int32_t* slot_of_row, void* workspace,
                         size_t workspace_bytes, gmm_stream_t stream) {
  if (T < 0 || k < 1 || k > 64 || G < 1 || G > GMM_MAX_GROUPS) return GMM_ERR_SHAPE;
  const int64_t n = T * k;
  if (n >= (int64_t(1) << 31)) return GMM_ERR_SHAPE;
  if (!group_sizes || (n > 0 && (!expert_ids || !row_of_slot || !slot_of_row)))
    return GMM_ERR_NULL;
  if ((x == nullptr) != (x_perm == nullptr)) return GMM_ERR_NULL;
  if (x && (row_bytes <= 0 || row_bytes % 16)) return GMM_ERR_SHAPE;
  for (const void* ptr : {(const void*)expert_ids, x, (const void*)x_perm, (const void*)group_sizes,
                          (const void*)row_of_slot, (const void*)slot_of_row, (const void*)workspace})
    if (ptr && !aligned16(ptr)) return GMM_ERR_ALIGN;
  const size_t ws_need = gmm_permute_workspace_size(T, k, G);
  if (ws_need && (!workspace || workspace_bytes < ws_need)) return GMM_ERR_WORKSPACE;
  const size_t ib = (size_t)n * 4, xb = x ? (size_t)T * row_bytes : 0,
               pb = x ? (size_t)n * row_bytes : 0, gb = (size_t)G * 4;
  // every output against every input and every other output
  const struct { const void* p; size_t n; } outs[] = {
      {x_perm, pb}, {group_sizes, gb}, {row_of_slot, ib}, {slot_of_row, ib}, {workspace, ws_need}};
  for (size_t i = 0; i < 5; ++i) {
    if (overlaps(outs[i].p, outs[i].n, expert_ids, ib) || overlaps(outs[i].p, outs[i].n, x, xb))
      return GMM_ERR_ALIAS;
    for (size_t j = i + 1; j < 5; ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return GMM_ERR_ALIAS;
  }
  trace("gmm_permute", T, k, row_bytes, G);
  int32_t* counts = (int32_t*)workspace;
  int32_t* dest_all =
      n ? (int32_t*)((uint8_t*)workspace + align256((size_t)route_chunks(n) * (G + 1) * 4)) : nullptr;
  return launch_route(expert_ids, n, k, G, counts, dest_all, group_sizes, row_of_slot,
                      slot_of_row, x, row_bytes, x_perm, (hipStream_t)stream) == hipSuccess
             ? GMM_OK
             : GMM_ERR_HIP;
}

gmm_status_t gmm_unpermute(int64_t T, int32_t k, int64_t H, const void* y,
                           const int32_t* row_of_slot, const float* weights, void* out,
                           gmm_stream_t stream) {
  if (T < 0 || k < 1 || k > 64 || H <= 0 || H % 8 || H > MAX_DIM) return GMM_ERR_SHAPE;
  const int64_t n = T * k;
  if (n >= (int64_t(1) << 31)) return GMM_ERR_SHAPE;
  if (T == 0) return GMM_OK;
  if (!y || !row_of_slot || !out) return GMM_ERR_NULL;
  for (const void* ptr : {y, (const void*)row_of_slot, (const void*)weights, (const void*)out})
    if (ptr && !aligned16(ptr)) return GMM_ERR_ALIGN;
  const size_t ob = (size_t)T * H * 2;
  if (overlaps(out, ob, y, (size_t)n * H * 2) || overlaps(out, ob, row_of_slot, (size_t)n * 4) ||
      overlaps(out, ob, weights, weights ? (size_t)n * 4 : 0))
    return GMM_ERR_ALIAS;
  trace("gmm_unpermute", T, k, H, 1);
  return launch_combine((const uint16_t*)y, T, k, H, n, row_of_slot, weights, (uint16_t*)out,
                        (hipStream_t)stream) == hipSuccess
             ? GMM_OK
             : GMM_ERR_HIP;
}

gmm_status_t gmm_swiglu_bwd(int64_t M, int64_t I, const void* dh, const void* gu, void* d_gu,
                            gmm_stream_t stream) {
  if (M < 0 || M >= (int64_t(1) << 31) || I <= 0 || I % 128 || I > MAX_DIM / 2) return GMM_ERR_SHAPE;
  if (M == 0) return GMM_OK;
  if (!dh || !gu || !d_gu) return GMM_ERR_NULL;
  for (const void* ptr : {dh, gu, (const void*)d_gu})
    if (!aligned16(ptr)) return GMM_ERR_ALIGN;
  const size_t hb = (size_t)M * I * 2, gb = 2 * hb;
  if (overlaps(d_gu, gb, dh, hb) || overlaps(d_gu, gb, gu, gb)) return GMM_ERR_ALIAS;
  trace("gmm_swiglu_bwd", M, I, 2 * I, 1);
  return launch_swiglu_bwd((const uint16_t*)dh, (const uint16_t*)gu, (uint16_t*)d_gu, M, I,
                           (hipStream_t)stream) == hipSuccess ? GMM_OK : GMM_ERR_HIP;
}

gmm_status_t tgmm_drhs(const gmm_operand_t* lhs_op, const gmm_operand_t* grad_op,
                       int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G,
                       const void* lhs, float* lhs_scales, const void* grad,
                       float* grad_scales, const int32_t* group_sizes, void* drhs,
                       void* workspace, size_t workspace_bytes, gmm_stream_t stream) {
  return tgmm_drhs_local(lhs_op, grad_op, out_dtype, M, K, N, G, 0, G, lhs, lhs_scales, grad,
                         grad_scales, group_sizes, drhs, workspace, workspace_bytes, stream);
}

gmm_status_t tgmm_drhs_local(const gmm_operand_t* lhs_op, const gmm_operand_t* grad_op,
                             int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G_total,
                             int32_t group_offset, int32_t G, const void* lhs, float* lhs_scales,
                             const void* grad, float* grad_scales, const int32_t* group_sizes,
                             void* drhs, void* workspace, size_t workspace_bytes,
                             gmm_stream_t stream) {
  gmm_status_t s;
  if ((s = check_operand(lhs_op)) != GMM_OK) return s;
  if ((s = check_operand(grad_op)) != GMM_OK) return s;
  if (out_dtype != GMM_OUT_BF16 && out_dtype != GMM_OUT_F32) return GMM_ERR_RECIPE;
  if ((s = check_shape(M, K, N, G_total)) != GMM_OK) return s;
  if (group_offset < 0 || G < 1 || group_offset > G_total - G) return GMM_ERR_SHAPE;
  // 32-bit workgroup numbers (each group's tiles rounded up to a multiple of 8)
  if ((((K + 255) / 256) * ((N + 255) / 256) + 7) / 8 * 8 * G >= (int64_t(1) << 31))
    return GMM_ERR_SHAPE;
  if (!group_sizes || !drhs) return GMM_ERR_NULL;
  if (M > 0 && (!lhs || !grad)) return GMM_ERR_NULL;
  if (M > 0 && ((scales_are_input(lhs_op) && !lhs_scales) || (scales_are_input(grad_op) && !grad_scales)))
    return GMM_ERR_NULL;
  for (const void* ptr : {(const void*)lhs, (const void*)grad, (const void*)group_sizes,
                          (const void*)drhs, (const void*)lhs_scales, (const void*)grad_scales,
                          (const void*)workspace})
    if (ptr && !aligned16(ptr)) return GMM_ERR_ALIGN;
  const size_t wa = needs_dyn_ws(lhs_op) ? dyn_ws_bytes(M) : 0;
  const size_t wb = needs_dyn_ws(grad_op) ? dyn_ws_bytes(M) : 0;
  const bool a_codes = lhs_op->kind == GMM_OPERAND_FP8, g_codes = grad_op->kind == GMM_OPERAND_FP8;
  const size_t wt = tgmm_ws_bytes(M, K, N, G, a_codes, g_codes);
  if (!workspace || workspace_bytes < wa + wb + wt) return GMM_ERR_WORKSPACE;
  const size_t out_bytes = (size_t)G * K * N * (out_dtype == GMM_OUT_F32 ? 4 : 2);
  const size_t lhs_bytes = (size_t)M * K * (a_codes ? 1 : 2);
  const size_t grad_bytes = (size_t)M * N * (g_codes ? 1 : 2);
  const size_t sc_bytes = (size_t)nblocks(M) * 4;
  if (overlaps(drhs, out_bytes, lhs, lhs_bytes) || overlaps(drhs, out_bytes, grad, grad_bytes) ||
      overlaps(drhs, out_bytes, group_sizes, (size_t)G_total * 4) ||
      overlaps(drhs, out_bytes, lhs_scales, sc_bytes) ||
      overlaps(drhs, out_bytes, grad_scales, sc_bytes) ||
      overlaps(workspace, wa + wb + wt, drhs, out_bytes) ||
      overlaps(workspace, wa + wb + wt, lhs, lhs_bytes) ||
      overlaps(workspace, wa + wb + wt, grad, grad_bytes) ||
      overlaps(workspace, wa + wb + wt, lhs_scales, sc_bytes) ||
      overlaps(workspace, wa + wb + wt, grad_scales, sc_bytes))
    return GMM_ERR_ALIAS;
  if ((s = check_group_sizes(group_sizes, G_total, M, (hipStream_t)stream)) != GMM_OK) return s;
  trace("tgmm_drhs", M, K, N, G);
  hipStream_t st = (hipStream_t)stream;

  TgmmParams p{};
  p.a = lhs;
  p.b = grad;
  p.a_codes = a_codes;
  p.b_codes = g_codes;
  p.group_sizes = group_sizes;
  p.out = drhs;
  p.M = M;
  p.Kout = (int32_t)K;
  p.Nout = (int32_t)N;
  p.G = G;
  p.g_before = group_offset;
  p.out_f32 = out_dtype == GMM_OUT_F32;
  {
    uint8_t* base = (uint8_t*)workspace + wa + wb;
    p.plan = (int32_t*)base;
    p.scprod = (float*)(base + align256((size_t)tgmm_plan_words(G) * 4));
    p.ratio = (float*)((uint8_t*)p.scprod + align256((size_t)nblocks(M) * 4));
    uint8_t* codes = (uint8_t*)p.ratio + align256((size_t)(nblocks(M) + 2 * G) * 4);
    p.a_q = a_codes ? nullptr : codes;
    p.b_q = g_codes ? nullptr : codes + (a_codes ? 0 : align256((size_t)M * K));
  }
  if (M > 0) {
    Scaling sa, sg;
    if ((s = resolve_scaling(lhs_op, lhs, M, K, lhs_scales, workspace, st, sa)) != GMM_OK) return s;
    if ((s = resolve_scaling(grad_op, grad, M, N, grad_scales, (uint8_t*)workspace + wa, st, sg)) !=
        GMM_OK)
      return s;
    p.a_scale_blk = sa.blk;
    p.a_scale_static = sa.s;
    p.a_inv_static = sa.inv;
    p.b_scale_blk = sg.blk;
    p.b_scale_static = sg.s;
    p.b_inv_static = sg.inv;
  }
  if (launch_tgmm(lhs_op->format, grad_op->format, p, st) != hipSuccess) return GMM_ERR_HIP;
  return GMM_OK;
}

gmm_status_t gmm_workspace_size(int32_t op, const gmm_operand_t* a, const gmm_operand_t* b,
                                int64_t rows, int64_t cols_a, int64_t cols_b, int32_t G,
                                size_t* bytes) {
  if (!bytes || !a) return GMM_ERR_NULL;
  if (rows < 0 || cols_a < 0 || cols_b < 0 || G < 1 || G > GMM_MAX_GROUPS) return GMM_ERR_SHAPE;
  gmm_status_t s = check_operand(a);
  if (s != GMM_OK) return s;
  size_t n = needs_dyn_ws(a) ? dyn_ws_bytes(rows) : 0;
  if ((op == GMM_OP_FWD || op == GMM_OP_DLHS) && a->kind == GMM_OPERAND_BF16 &&
      quant_once_applies(cols_b))
    n += quant_once_bytes(rows, cols_a);
  if (op == GMM_OP_DLHS || op == GMM_OP_DLHS_FUSED) n += split_ws_bytes(rows, cols_a, cols_b, G);
  if (op == GMM_OP_FWD_SWIGLU && a->kind == GMM_OPERAND_BF16) n += quant_once_bytes(rows, cols_a);
  if (op == GMM_OP_TGMM) {
    if (!b) return GMM_ERR_NULL;
    if ((s = check_operand(b)) != GMM_OK) return s;
    n += needs_dyn_ws(b) ? dyn_ws_bytes(rows) : 0;
    n += tgmm_ws_bytes(rows, cols_a, cols_b, G, a->kind == GMM_OPERAND_FP8,
                       b->kind == GMM_OPERAND_FP8);
  } else if (op != GMM_OP_FWD && op != GMM_OP_DLHS && op != GMM_OP_FWD_FUSED &&
             op != GMM_OP_DLHS_FUSED && op != GMM_OP_QUANTIZE && op != GMM_OP_FWD_SWIGLU) {
    return GMM_ERR_RECIPE;
  }
  *bytes = n;
  return GMM_OK;
}

gmm_status_t gmm_quantize(const gmm_operand_t* op, int64_t R, int64_t C, const void* x,
                          uint8_t* codes, float* scales, void* workspace,
                          size_t workspace_bytes, gmm_stream_t stream) {
  gmm_status_t s = check_operand(op);
  if (s != GMM_OK) return s;
  if (op->kind != GMM_OPERAND_BF16) return GMM_ERR_RECIPE;
  if (R < 0 || R >= (int64_t(1) << 31) || C <= 0 || C % 8 || C > MAX_DIM * 8) return GMM_ERR_SHAPE;
  if (R > 0 && (!x || !codes)) return GMM_ERR_NULL;
  for (const void* ptr : {(const void*)x, (const void*)codes, (const void*)scales, (const void*)workspace})
    if (ptr && !aligned16(ptr)) return GMM_ERR_ALIGN;
  const size_t ws_need = needs_dyn_ws(op) ? dyn_ws_bytes(R) : 0;
  if (ws_need && (!workspace || workspace_bytes < ws_need)) return GMM_ERR_WORKSPACE;
  if (scales_are_input(op) && R > 0 && !scales) return GMM_ERR_NULL;
  if (overlaps(codes, (size_t)R * C, x, (size_t)R * C * 2)) return GMM_ERR_ALIAS;
  if (R == 0) return GMM_OK;
  hipStream_t st = (hipStream_t)stream;
  Scaling sc;
  if ((s = resolve_scaling(op, x, R, C, scales, workspace, st, sc)) != GMM_OK) return s;
  return launch_quantize_rows(op->format, x, R, C, sc.blk, sc.inv, codes, st) == hipSuccess
             ? GMM_OK : GMM_ERR_HIP;
}

gmm_status_t gmm_dynamic_scales(int32_t format, int64_t R, int64_t C, const void* x,
                                float* scales, void* workspace, size_t workspace_bytes,
                                gmm_stream_t stream) {
  if (format != GMM_FP8_E4M3 && format != GMM_FP8_E5M2) return GMM_ERR_RECIPE;
  if (R < 0 || R >= (int64_t(1) << 31) || C <= 0 || C % 8 || C > MAX_DIM * 8) return GMM_ERR_SHAPE;
  if (R > 0 && (!x || !scales)) return GMM_ERR_NULL;
  for (const void* ptr : {(const void*)x, (const void*)scales, (const void*)workspace})
    if (ptr && !aligned16(ptr)) return GMM_ERR_ALIGN;
  const size_t ws_need = dyn_ws_bytes(R);
  if (R > 0 && (!workspace || workspace_bytes < ws_need)) return GMM_ERR_WORKSPACE;
  if (overlaps(scales, (size_t)nblocks(R) * 4, x, (size_t)R * C * 2)) return GMM_ERR_ALIAS;
  if (R == 0) return GMM_OK;
  DynWs w = carve(workspace, R);
  return launch_dynamic_scales(format, x, R, C, w.partial, scales, (hipStream_t)stream) == hipSuccess
             ? GMM_OK : GMM_ERR_HIP;
}

gmm_status_t gmm_quantize_rhs(int32_t format, int32_t channel_axis, int32_t layout, int64_t G,
                              int64_t K, int64_t N, const void* w, uint8_t* codes,
                              float* scales, gmm_stream_t stream) {
  if (format != GMM_FP8_E4M3 && format != GMM_FP8_E5M2) return GMM_ERR_RECIPE;
  if (channel_axis != 0 && channel_axis != 1) return GMM_ERR_RECIPE;
  if (layout != GMM_RHS_KN && layout != GMM_RHS_NK) return GMM_ERR_RECIPE;
  gmm_status_t s = check_shape(0, K, N, (int32_t)std::min<int64_t>(G, GMM_MAX_GROUPS + 1));
  if (s != GMM_OK || G < 1 || G > 65535) return GMM_ERR_SHAPE;
  if (!w || !codes || !scales) return GMM_ERR_NULL;
  for (const void* ptr : {(const void*)w, (const void*)codes, (const void*)scales})
    if (!aligned16(ptr)) return GMM_ERR_ALIGN;
  if (overlaps(codes, (size_t)G * K * N, w, (size_t)G * K * N * 2) ||
      overlaps(scales, (size_t)G * (channel_axis ? K : N) * 4, w, (size_t)G * K * N * 2) ||
      overlaps(scales, (size_t)G * (channel_axis ? K : N) * 4, codes, (size_t)G * K * N))
    return GMM_ERR_ALIAS;
  return launch_quantize_rhs(format, channel_axis, layout == GMM_RHS_NK, G, K, N, K, w, codes,
                             scales, (hipStream_t)stream) == hipSuccess
             ? GMM_OK : GMM_ERR_HIP;
}

gmm_status_t gmm_quantize_rhs_blockwise(int32_t format, int32_t layout, int64_t G, int64_t K,
                                        int64_t N, int64_t bk, const void* w, uint8_t* codes,
                                        float* scales, gmm_stream_t stream) {
  if (format != GMM_FP8_E4M3 && format != GMM_FP8_E5M2) return GMM_ERR_RECIPE;
  if (layout != GMM_RHS_KN && layout != GMM_RHS_NK) return GMM_ERR_RECIPE;
  gmm_status_t s = check_shape(0, K, N, (int32_t)std::min<int64_t>(G, GMM_MAX_GROUPS + 1));
  if (s != GMM_OK || G < 1 || G > 65535 || bk < 128 || bk % 128 || K % bk) return GMM_ERR_SHAPE;
  if (!w || !codes || !scales) return GMM_ERR_NULL;
  for (const void* ptr : {(const void*)w, (const void*)codes, (const void*)scales})
    if (!aligned16(ptr)) return GMM_ERR_ALIGN;
  const size_t sb = (size_t)G * (K / bk) * N * 4;
  if (overlaps(codes, (size_t)G * K * N, w, (size_t)G * K * N * 2) ||
      overlaps(scales, sb, w, (size_t)G * K * N * 2) || overlaps(scales, sb, codes, (size_t)G * K * N))
    return GMM_ERR_ALIAS;
  return launch_quantize_rhs(format, 0, layout == GMM_RHS_NK, G, K, N, bk, w, codes, scales,
                             (hipStream_t)stream) == hipSuccess
             ? GMM_OK : GMM_ERR_HIP;
}

gmm_status_t gmm_quantize_subchannel(int32_t format, int64_t M, int64_t K, int64_t bk,
                                     const void* x, uint8_t* codes, float* scales,
                                     gmm_stream_t stream) {
  if (format != GMM_FP8_E4M3 && format != GMM_FP8_E5M2) return GMM_ERR_RECIPE;
  if (M < 0 || M >= (int64_t(1) << 31) || K <= 0 || K > MAX_DIM) return GMM_ERR_SHAPE;
  if ((bk != 128 && bk != 256 && bk != 512) || K % bk) return GMM_ERR_SHAPE;
  if (M == 0) return GMM_OK;
  if (!x || !codes || !scales) return GMM_ERR_NULL;
  for (const void* ptr : {(const void*)x, (const void*)codes, (const void*)scales})
    if (!aligned16(ptr)) return GMM_ERR_ALIGN;
  const size_t xb = (size_t)M * K * 2, cb = (size_t)M * K, sb = (size_t)M * (K / bk) * 4;
  if (overlaps(codes, cb, x, xb) || overlaps(scales, sb, x, xb) || overlaps(scales, sb, codes, cb))
    return GMM_ERR_ALIAS;
  trace("gmm_quantize_subchannel", M, K, bk, 1);
  return launch_quantize_subchannel(format, x, M, K, (int)bk, codes, scales,
                                    (hipStream_t)stream) == hipSuccess
             ? GMM_OK : GMM_ERR_HIP;
}

gmm_status_t gmm_quantize_folded(int32_t format, int64_t M, int64_t N, int32_t G,
                                 const void* grad, const float* col_scales,
                                 const int32_t* group_sizes, uint8_t* codes, float* scales,
                                 void* workspace, size_t workspace_bytes, gmm_stream_t stream) {
  if (format != GMM_FP8_E4M3 && format != GMM_FP8_E5M2) return GMM_ERR_RECIPE;
  gmm_status_t s = check_shape(M, 128, N, G);
  if (s != GMM_OK) return s;
  if (M == 0) return GMM_OK;
  if (!grad || !col_scales || !group_sizes || !codes || !scales) return GMM_ERR_NULL;
  for (const void* ptr : {grad, (const void*)col_scales, (const void*)group_sizes,
                          (const void*)codes, (const void*)scales, (const void*)workspace})
    if (ptr && !aligned16(ptr)) return GMM_ERR_ALIGN;
  const size_t ws_need = (size_t)nblocks(M) * AMAX_SPLIT * 4;
  if (!workspace || workspace_bytes < ws_need) return GMM_ERR_WORKSPACE;
  const size_t gb = (size_t)M * N * 2, cb = (size_t)M * N, sb = (size_t)nblocks(M) * 4,
               csb = (size_t)G * N * 4, gsb = (size_t)G * 4;
  const struct { const void* p; size_t n; } outs[] = {{codes, cb}, {scales, sb}, {workspace, ws_need}};
  for (size_t i = 0; i < 3; ++i) {
    if (overlaps(outs[i].p, outs[i].n, grad, gb) || overlaps(outs[i].p, outs[i].n, col_scales, csb) ||
        overlaps(outs[i].p, outs[i].n, group_sizes, gsb))
      return GMM_ERR_ALIAS;
    for (size_t j = i + 1; j < 3; ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return GMM_ERR_ALIAS;
  }
  if ((s = check_group_sizes(group_sizes, G, M, (hipStream_t)stream)) != GMM_OK) return s;
  trace("gmm_quantize_folded", M, N, 0, G);
  return launch_quantize_folded(format, grad, M, N, col_scales, group_sizes, G,
                                (uint32_t*)workspace, scales, codes,
                                (hipStream_t)stream) == hipSuccess
             ? GMM_OK
             : GMM_ERR_HIP;
}

gmm_status_t gmm_fwd_blockwise(int32_t lhs_format, int32_t out_dtype, int64_t M, int64_t K,
                               int64_t N, int32_t G, int64_t bk, const uint8_t* lhs,
                               const float* lhs_scales, const uint8_t* rhs,
                               const float* rhs_scales, const int32_t* group_sizes, void* out,
                               gmm_stream_t stream) {
  return blockwise_gemm("gmm_fwd_blockwise", lhs_format, out_dtype, M, K, N, G, bk, lhs,
                        lhs_scales, rhs, rhs_scales, false, group_sizes, out,
                        (hipStream_t)stream);
}

gmm_status_t gmm_dlhs_blockwise(int32_t grad_format, int32_t out_dtype, int64_t M, int64_t K,
                                int64_t N, int32_t G, int64_t bk, const uint8_t* grad,
                                const float* grad_scales, const uint8_t* rhs,
                                const float* rhs_scales, const int32_t* group_sizes, void* dlhs,
                                gmm_stream_t stream) {
  // the block-wise product with contraction N and output K: rhs [G, K, N] is already
  // contraction-contiguous, its scales [G, K, N / bk] per output channel
  return blockwise_gemm("gmm_dlhs_blockwise", grad_format, out_dtype, M, N, K, G, bk, grad,
                        grad_scales, rhs, rhs_scales, true, group_sizes, dlhs,
                        (hipStream_t)stream);
}

gmm_status_t gmm_static_scale_from_bound(float lo, float hi, int32_t format, float* scale) {
  if (!scale) return GMM_ERR_NULL;
  if (format != GMM_FP8_E4M3 && format != GMM_FP8_E5M2) return GMM_ERR_RECIPE;
  if (!std::isfinite(lo) || !std::isfinite(hi) || !(hi > 0.0f) || lo != -hi) return GMM_ERR_SCALE;
  const float s = hi / (format == GMM_FP8_E4M3 ? 448.0f : 57344.0f);
  if (!(s >= FLT_MIN)) return GMM_ERR_SCALE;
  *scale = s;
  return GMM_OK;
}

const char* gmm_status_string(gmm_status_t s) {
  switch (s) {
    case GMM_OK: return "ok";
    case GMM_ERR_NULL: return "a required pointer is NULL";
    case GMM_ERR_SHAPE: return "invalid shape (M, K, N or G)";
    case GMM_ERR_SCALE: return "invalid static scale or calibration range";
    case GMM_ERR_RECIPE: return "unsupported quantization recipe";
    case GMM_ERR_WORKSPACE: return "workspace missing or too small";
    case GMM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case GMM_ERR_GROUP_SIZES: return "group sizes negative or not summing to M";
    case GMM_ERR_HIP: return "HIP runtime error";
    case GMM_ERR_ALIAS: return "an output overlaps an input";
  }
  return "unknown status";
}

const char* gmm_version(void) { return "gmm_fp8 0.1.0 (gfx950)"; }

}  // extern "C"
