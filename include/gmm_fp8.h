/*
 * gmm_fp8.h - C ABI of the MI355X (gfx950) FP8 grouped (ragged) matmul library.
 *
 * The library implements the three products of an MoE expert layer with FP8 operands
 * and fp32 accumulation, as described on the MaxText pull-request pages
 *   "FP8 Megablox for batch split" (PR #3770),
 *   "Support quantization for tokamax gmm v2" (PR #4451) and
 *   "add static LHS scaling support for GMM v2 FWD" (PR #4735):
 *
 *   gmm_fwd    out[m, :]   = lhs[m, :] . rhs[g]          for every row m of group g
 *   gmm_dlhs   dlhs[m, :]  = grad[m, :] . rhs[g]^T       (the gmm against rhs transposed)
 *   tgmm_drhs  drhs[g]     = lhs_g^T . grad_g            (one [K, N] slab per group)
 *
 * and the steps around them in the same MoE layer:
 *
 *   gmm_fwd_swiglu / gmm_fwd_swiglu_fp8 / gmm_fwd_swiglu_fp8_subchannel /
 *   gmm_swiglu_bwd / gmm_dlhs_swiglu_bwd   SwiGLU of the merged gate|up product in the
 *              forward's epilogue (h in bf16/f32, or fp8 codes under a static or
 *              per-row-and-block dynamic scale), and its backward, alone or in the
 *              epilogue of the down projection's dlhs
 *   gmm_fwd_local / gmm_dlhs_local / tgmm_drhs_local   the products over a window of
 *              local experts (group_offset)
 *   gmm_fwd_blockwise, gmm_dlhs_blockwise, gmm_quantize_subchannel,
 *   gmm_quantize_rhs_blockwise, gmm_quantize_folded   block-wise weight scales,
 *              sub-channel lhs scales, and the dlhs on the forward's weight copy
 *   gmm_permute / gmm_unpermute   token routing: the sort of top-k choices by expert
 *              and the weighted combine back
 *
 * Rows of lhs / grad are sorted by group: group g owns rows [off_g, off_g + m_g) with
 * off_0 = 0 and off_{g+1} = off_g + m_g, m_g = group_sizes[g].
 *
 * Common conventions
 * ------------------
 * - Every pointer argument is DEVICE memory owned by the caller, unless marked "host".
 *   The library never allocates, frees or synchronises; all work is enqueued on the
 *   caller's HIP stream and the call returns as soon as it is enqueued.
 * - Tensors are dense, row-major (last index contiguous), 16-byte aligned.
 * - bf16 is IEEE bfloat16 (stored as uint16); fp8 codes are OCP E4M3FN or E5M2 bytes.
 * - group_sizes is int32 [G] in device memory and is never read by the host: the
 *   caller guarantees m_g >= 0 and sum(m_g) == M (checked only when the environment
 *   variable GMM_CHECK=1 is set, which synchronises the stream).
 * - Shapes: 0 <= M < 2^31, 1 <= G <= GMM_MAX_GROUPS, K and N positive multiples of 128
 *   up to 2^22 with K * N < 2^32, and fewer than 2^31 output tiles of 256 x 256
 *   ((M / 256 + 1 + G) * ceil(N_out / 256) for gmm_fwd / gmm_dlhs); tgmm_drhs adds its
 *   own limits.  Anything else is GMM_ERR_SHAPE.
 * - Inputs are read-only; outputs must not overlap inputs.
 * - Errors are returned as gmm_status_t; argument validation happens before any work
 *   is enqueued, so an error return leaves every output untouched.
 * - The functions keep no global state (apart from gmm_fwd_noalloc's device scratch
 *   array, see there) and may be called concurrently on different streams with
 *   different buffers.
 *
 * Quantization recipes
 * --------------------
 * An operand given as bf16 is quantized by the call, inside the product kernel right
 * after it is loaded or, where the entry point says so, once into the workspace (the
 * codes are the same bytes either way):  code = fp8( clamp( RNE_f32(x * inv), -qmax, +qmax ) )  with
 * round-to-nearest-even to fp8 (qmax = 448 for e4m3, 57344 for e5m2), and the fp32
 * product is multiplied back by the scale ("add static LHS scaling support for GMM v2
 * FWD", review thread on the lhs docstring: clip(lhs/scale), result multiplied back by
 * the scale).  The scale s and inv are:
 *   GMM_SCALE_STATIC   one per-tensor scale s (the [1,1] scale of that page, derived
 *                      from a fixed symmetric calibration range, see
 *                      gmm_static_scale_from_bound); inv = RNE_f32(1/s).
 *   GMM_SCALE_DYNAMIC  one scale per block of 128 consecutive rows spanning the full
 *                      row width, blocks aligned to row 0 of the tensor:
 *                      s_b = RNE_f32(amax_b / qmax); inv_b = 0 when s_b == 0 or 1/s_b
 *                      overflows, else RNE_f32(1/s_b) (same page, review thread on
 *                      block_scale_inv: zero inverse for a zero scale).  The call
 *                      computes the scales with an abs-max prepass over the operand.
 *   GMM_SCALE_DYNAMIC_GIVEN  the same per-block recipe with the scales s_b supplied by
 *                      the caller (from gmm_dynamic_scales, or returned by an earlier
 *                      call on the same tensor); the prepass is skipped and inv_b is
 *                      derived from s_b in the kernel by the rule above.
 * An operand given as fp8 codes (GMM_OPERAND_FP8) was quantized beforehand with the
 * same formulas (the pre-quantized activation case of the same page's follow-up
 * commits); its scales are then an input.
 * The rhs of gmm_fwd / gmm_dlhs is always fp8 codes with one scale per output channel
 * ("FP8 Megablox for batch split", Description (1): manually quantized weight;
 * "Support quantization for tokamax gmm v2", review thread on per-channel scales).
 */
#ifndef GMM_FP8_H
#define GMM_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque HIP stream (hipStream_t); NULL is the default stream. */
typedef struct ihipStream_t* gmm_stream_t;

#define GMM_BLOCK_ROWS 128   /* rows per dynamic-scale block */
#define GMM_MAX_GROUPS 1024  /* largest supported number of groups (experts) */
#define GMM_NOALLOC_MAX_ROWS (1 << 20)  /* largest M that gmm_fwd_noalloc accepts */

typedef enum gmm_status {
  GMM_OK = 0,
  GMM_ERR_NULL = 1,        /* a required pointer is NULL */
  GMM_ERR_SHAPE = 2,       /* bad M, K, N or G */
  GMM_ERR_SCALE = 3,       /* static scale not finite, positive and normal; asymmetric range */
  GMM_ERR_RECIPE = 4,      /* unknown or unsupported format / scaling / kind / layout / dtype */
  GMM_ERR_WORKSPACE = 5,   /* workspace missing or smaller than gmm_workspace_size() */
  GMM_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned */
  GMM_ERR_GROUP_SIZES = 7, /* GMM_CHECK=1 only: a negative size or sum != M */
  GMM_ERR_HIP = 8,         /* a HIP runtime call or kernel launch failed */
  GMM_ERR_ALIAS = 9        /* an output buffer overlaps an input buffer */
} gmm_status_t;

typedef enum gmm_fp8_format { GMM_FP8_E4M3 = 0, GMM_FP8_E5M2 = 1 } gmm_fp8_format_t;
/* GMM_SCALE_DYNAMIC_GIVEN: dynamic per-block scales that were computed beforehand (by
 * gmm_dynamic_scales or by an earlier call on the same tensor) and are passed in, so
 * that a tensor used by several products has its block scales computed once. */
typedef enum gmm_scaling {
  GMM_SCALE_STATIC = 0,
  GMM_SCALE_DYNAMIC = 1,
  GMM_SCALE_DYNAMIC_GIVEN = 2
} gmm_scaling_t;
typedef enum gmm_operand_kind { GMM_OPERAND_BF16 = 0, GMM_OPERAND_FP8 = 1 } gmm_operand_kind_t;
typedef enum gmm_out_dtype { GMM_OUT_BF16 = 0, GMM_OUT_F32 = 1 } gmm_out_dtype_t;

/* Physical layout of the rhs codes of gmm_fwd / gmm_dlhs (logical shape [G, K, N]).
 * GMM_RHS_KN: [G, K, N], N contiguous (the layout of the weight itself).
 * GMM_RHS_NK: [G, N, K], K contiguous (the weight stored transposed, the pages'
 *             transpose_rhs).  Both layouts are supported by both calls; the kernel
 *             is fastest when the contraction axis is contiguous: NK for gmm_fwd, KN
 *             for gmm_dlhs. */
typedef enum gmm_rhs_layout { GMM_RHS_KN = 0, GMM_RHS_NK = 1 } gmm_rhs_layout_t;

/* How one operand reaches the kernel and how it is scaled. */
typedef struct gmm_operand {
  int32_t kind;         /* gmm_operand_kind_t */
  int32_t format;       /* gmm_fp8_format_t */
  int32_t scaling;      /* gmm_scaling_t */
  float static_scale;   /* GMM_SCALE_STATIC: the per-tensor scale s (finite, > 0, normal) */
} gmm_operand_t;

/* Operation identifiers for gmm_workspace_size.  The _FUSED variants size the workspace
 * of gmm_fwd / gmm_dlhs calls that quantize a bf16 operand inside the product kernel;
 * GMM_OP_QUANTIZE sizes that of gmm_quantize and gmm_dynamic_scales; GMM_OP_FWD_SWIGLU
 * that of gmm_fwd_swiglu. */
typedef enum gmm_op {
  GMM_OP_FWD = 0,
  GMM_OP_DLHS = 1,
  GMM_OP_TGMM = 2,
  GMM_OP_FWD_FUSED = 3,
  GMM_OP_DLHS_FUSED = 4,
  GMM_OP_QUANTIZE = 5,
  GMM_OP_FWD_SWIGLU = 6
} gmm_op_t;

/*
 * gmm_fwd - forward grouped matmul ("FP8 Megablox for batch split", Description (1);
 * "Support quantization for tokamax gmm v2", What this does: fwd_gmm2).
 *
 *   out[m, n] = RNE_out( (sum_k q(lhs)[m, k] * rhs[g, k, n]) * s_lhs(m) * rhs_scales[g, n] )
 *
 * lhs          [M, K]: bf16 values (lhs_op->kind == GMM_OPERAND_BF16) or fp8 codes.
 * lhs_scales   f32 [ceil(M/128)].  DYNAMIC + BF16: OUTPUT, the block scales the call
 *              computed (may be NULL).  DYNAMIC_GIVEN, or DYNAMIC + FP8: INPUT, the block
 *              scales of the operand.  STATIC: unused (may be NULL); s_lhs is
 *              lhs_op->static_scale.
 * rhs          fp8 codes, layout rhs_layout, format rhs_format.
 * rhs_scales   f32 [G, N]: the dequantization scale of every output channel n.
 * group_sizes  int32 [G].
 * out          [M, N], bf16 or f32 per out_dtype.  Every row is written exactly once.
 * workspace    device scratch; its contents are undefined after the call.  With at least
 *              gmm_workspace_size(GMM_OP_FWD, ...) bytes, a bf16 lhs feeding 4 or more
 *              256-column output tiles is quantized once into the workspace and the
 *              product reads the codes; with at least gmm_workspace_size(
 *              GMM_OP_FWD_FUSED, ...) bytes every workgroup quantizes its lhs tile in
 *              registers (0 bytes unless the call computes dynamic block scales; then
 *              NULL is allowed).  Both routes produce the same codes and outputs.
 * Merged gate|up: pass rhs = concat(W0, W1) along N with concatenated scales; one call
 * produces [gate | up] ("FP8 Megablox for batch split", Description (2)).
 */
gmm_status_t gmm_fwd(const gmm_operand_t* lhs_op, int32_t rhs_format, int32_t rhs_layout,
                     int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G,
                     const void* lhs, float* lhs_scales, const uint8_t* rhs,
                     const float* rhs_scales, const int32_t* group_sizes, void* out,
                     void* workspace, size_t workspace_bytes, gmm_stream_t stream);

/*
 * gmm_fwd_noalloc - gmm_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It takes no
 * workspace: the one scratch buffer the forward needs (the abs-max partials of a dynamic
 * bf16 lhs and, when lhs_scales is NULL, its block scales) is a file-scope device array of
 * the library, about 288 KiB, which each GPU the library runs on holds until the process
 * ends.  Its address is looked up once per device (hipGetSymbolAddress), on the first call
 * with that device current; the call itself makes no allocation.
 * Arguments, outputs and errors as gmm_fwd; a bf16 lhs is quantized inside the product
 * kernel (the codes and outputs equal gmm_fwd's).  M <= GMM_NOALLOC_MAX_ROWS, else
 * GMM_ERR_WORKSPACE.  Every call on one GPU shares that GPU's scratch array, which keeps
 * the last call's contents (the call writes every byte it reads): calls that overlap on
 * one GPU (concurrent streams, or host threads) race, and must be serialized by the
 * caller.  The current device must be the stream's device.
 */
gmm_status_t gmm_fwd_noalloc(const gmm_operand_t* lhs_op, int32_t rhs_format, int32_t rhs_layout,
                             int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G,
                             const void* lhs, float* lhs_scales, const uint8_t* rhs,
                             const float* rhs_scales, const int32_t* group_sizes, void* out,
                             gmm_stream_t stream);

/*
 * gmm_dlhs - lhs gradient: a gmm of grad against rhs transposed ("Support quantization
 * for tokamax gmm v2", review of the dlhs call in ops.py: transpose_rhs flipped).
 *
 *   dlhs[m, k] = RNE_out( (sum_n q(grad)[m, n] * rhs[g, k, n]) * s_grad(m) * rhs_scales[g, k] )
 *
 * grad         [M, N]: bf16 values or fp8 codes (grad_op).  grad_scales as lhs_scales
 *              of gmm_fwd.
 * rhs          the same logical [G, K, N] weight as gmm_fwd, quantized per dlhs output
 *              channel k: rhs_scales f32 [G, K].
 * dlhs         [M, K] bf16 or f32.
 * workspace    as gmm_fwd's (GMM_OP_DLHS / GMM_OP_DLHS_FUSED; output tiles of 256 k).
 *              Both sizes include, for calls of more than 256 output tiles of 256 x 256
 *              and at least 6912 contraction columns, the 64 MiB of the tail split: when
 *              the last round of tiles on the GPU's 8 x 32 CUs is partly empty, its
 *              tiles are cut along the contraction, run by the CUs that would idle,
 *              and their fp32 partial sums added in slice order (only where that saves
 *              48 or more 128-deep steps per tile).  The split takes its room first
 *              (so both sizes give the same split), a bf16 grad's codes what is left; a
 *              smaller workspace runs the call unsplit.  The split depends on the shapes,
 *              group sizes and workspace only; it reorders the fp32 additions of the
 *              tiles it cuts.
 */
gmm_status_t gmm_dlhs(const gmm_operand_t* grad_op, int32_t rhs_format, int32_t rhs_layout,
                      int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G,
                      const void* grad, float* grad_scales, const uint8_t* rhs,
                      const float* rhs_scales, const int32_t* group_sizes, void* dlhs,
                      void* workspace, size_t workspace_bytes, gmm_stream_t stream);

/*
 * Local-expert window ("FP8 Megablox for batch split" follow-up, Description 3: the
 * group_offset argument of the ragged products).  With experts sharded over devices,
 * each device holds G_local of the G_total experts, from group_offset on; the rows stay
 * sorted by global expert, so group_sizes has all G_total entries and only the rows of
 * the local experts are computed.  rhs and rhs_scales hold the G_local local experts
 * (group 0 = expert group_offset).  0 <= group_offset, 1 <= G_local,
 * group_offset + G_local <= G_total <= GMM_MAX_GROUPS (else GMM_ERR_SHAPE).
 *
 * gmm_fwd_local / gmm_dlhs_local - as gmm_fwd / gmm_dlhs; out rows of groups outside the
 * window are written with zeros.  sum(group_sizes) == M over all G_total groups.
 * tgmm_drhs_local - as tgmm_drhs; drhs [G_local, K, N] for the local experts.  Its
 * workspace is gmm_workspace_size(GMM_OP_TGMM, ..., G_local) bytes or more.
 * With group_offset 0 and G_local == G_total each equals its plain entry point.
 */
gmm_status_t gmm_fwd_local(const gmm_operand_t* lhs_op, int32_t rhs_format, int32_t rhs_layout,
                           int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G_total,
                           int32_t group_offset, int32_t G_local, const void* lhs,
                           float* lhs_scales, const uint8_t* rhs, const float* rhs_scales,
                           const int32_t* group_sizes, void* out, void* workspace,
                           size_t workspace_bytes, gmm_stream_t stream);
gmm_status_t gmm_dlhs_local(const gmm_operand_t* grad_op, int32_t rhs_format, int32_t rhs_layout,
                            int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G_total,
                            int32_t group_offset, int32_t G_local, const void* grad,
                            float* grad_scales, const uint8_t* rhs, const float* rhs_scales,
                            const int32_t* group_sizes, void* dlhs, void* workspace,
                            size_t workspace_bytes, gmm_stream_t stream);
gmm_status_t tgmm_drhs_local(const gmm_operand_t* lhs_op, const gmm_operand_t* grad_op,
                             int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G_total,
                             int32_t group_offset, int32_t G_local, const void* lhs,
                             float* lhs_scales, const void* grad, float* grad_scales,
                             const int32_t* group_sizes, void* drhs, void* workspace,
                             size_t workspace_bytes, gmm_stream_t stream);

/*
 * gmm_fwd_swiglu - the merged gate|up forward with SwiGLU in its epilogue ("FP8 Megablox
 * for batch split", Description (2): W0 | W1 merged along N, one call for both).
 *
 *   x[m, n] = (sum_k q(lhs)[m, k] * rhs[g, k, n]) * s_lhs(m) * rhs_scales[g, n]   (fp32,
 *             exactly as gmm_fwd computes it before rounding), n < 2 I;
 *   h[m, c] = silu(x[m, c]) * x[m, I + c],  silu(v) = v / (1 + exp(-v)),  c < I,
 *
 * in fp32 with each operation rounded to nearest, then stored in out_dtype.  rhs holds the
 * merged codes: channels 0..I-1 are the gate (W0), I..2I-1 the up projection (W1); only
 * rhs_layout GMM_RHS_NK ([G, 2I, K]) is accepted (else GMM_ERR_RECIPE), with rhs_scales f32
 * [G, 2I].  I is a positive multiple of 128.  lhs: as gmm_fwd; a bf16 lhs is quantized once
 * into the workspace, which must then hold gmm_workspace_size(GMM_OP_FWD_SWIGLU, ...)
 * bytes (else GMM_ERR_WORKSPACE).
 * gu           optional [M, 2I] in out_dtype: x itself (the values gmm_fwd would store),
 *              which the backward needs; NULL skips it.
 * h            [M, I] in out_dtype.  Rows outside every group are not written.
 */
gmm_status_t gmm_fwd_swiglu(const gmm_operand_t* lhs_op, int32_t rhs_format, int32_t rhs_layout,
                            int32_t out_dtype, int64_t M, int64_t K, int64_t I, int32_t G,
                            const void* lhs, float* lhs_scales, const uint8_t* rhs,
                            const float* rhs_scales, const int32_t* group_sizes, void* gu,
                            void* h, void* workspace, size_t workspace_bytes,
                            gmm_stream_t stream);

/*
 * gmm_fwd_swiglu_fp8 - gmm_fwd_swiglu with h written as fp8 codes, ready to be the lhs of
 * the down projection without a bf16 round trip ("FP8 Megablox for batch split",
 * Description (1) and (2): fp8 operands in the MoE gmms, gate|up merged; "add static LHS
 * scaling support for GMM v2 FWD", Description: a fixed calibration scale per tensor).
 *
 *   h_codes[m, c] = fp8(clamp(RNE_f32(h[m, c] * inv), -qmax, qmax)),  inv = RNE_f32(1/s),
 *
 * with h the fp32 value gmm_fwd_swiglu computes and s = h_op->static_scale.
 * h_op         kind GMM_OPERAND_FP8, scaling GMM_SCALE_STATIC, format e4m3 or e5m2 (else
 *              GMM_ERR_RECIPE), static_scale finite, normal and positive (else
 *              GMM_ERR_SCALE).  The same descriptor, passed as lhs_op of gmm_fwd with
 *              h_codes as lhs, runs the down projection on these codes.
 * h_codes      uint8 [M, I]; rows outside every group are not written.
 * gu, gu_dtype the optional product [M, 2I] as in gmm_fwd_swiglu (gu_dtype bf16 or f32).
 * Everything else, the workspace (GMM_OP_FWD_SWIGLU) included, is as gmm_fwd_swiglu's.
 * h_op->scaling must be GMM_SCALE_STATIC; dynamic scales are gmm_fwd_swiglu_fp8_subchannel's.
 */
gmm_status_t gmm_fwd_swiglu_fp8(const gmm_operand_t* lhs_op, int32_t rhs_format,
                                int32_t rhs_layout, int32_t gu_dtype, int64_t M, int64_t K,
                                int64_t I, int32_t G, const void* lhs, float* lhs_scales,
                                const uint8_t* rhs, const float* rhs_scales,
                                const int32_t* group_sizes, void* gu, const gmm_operand_t* h_op,
                                uint8_t* h_codes, void* workspace, size_t workspace_bytes,
                                gmm_stream_t stream);

/*
 * gmm_fwd_swiglu_fp8_subchannel - gmm_fwd_swiglu with h written as fp8 codes under dynamic
 * scales, one per row and block of 128 channels ("add static LHS scaling support for GMM
 * v2 FWD", review thread on the lhs docstring: lhs scales of shape [M, num_blocks];
 * "FP8 Megablox for batch split", Description (1)):
 *
 *   h_scales[m, b] = RNE_f32(max_{c in block b} |h[m, c]| / qmax),
 *   h_codes[m, c]  = fp8(clamp(RNE_f32(h[m, c] * inv), -qmax, qmax)),
 *   inv = 0 if h_scales[m, b] is 0 or its inverse overflows, else RNE_f32(1 / h_scales[m, b]),
 *
 * with h the fp32 value gmm_fwd_swiglu computes.  Each output tile of the merged product
 * holds the 128 gate and 128 up channels of one block of h, so the block's abs-max is
 * taken inside the tile's epilogue and h never leaves the registers in a wider type.
 * h_format     e4m3 or e5m2 (else GMM_ERR_RECIPE).
 * h_codes      uint8 [M, I]; h_scales f32 [M, I / 128] (NULL only when M = 0); rows
 *              outside every group are not written.  The pair is the sub-channel lhs of
 *              gmm_fwd_blockwise with bk = 128: the down projection on these codes.
 * Everything else (gu, gu_dtype, workspace GMM_OP_FWD_SWIGLU) is as gmm_fwd_swiglu_fp8's.
 */
gmm_status_t gmm_fwd_swiglu_fp8_subchannel(const gmm_operand_t* lhs_op, int32_t rhs_format,
                                           int32_t rhs_layout, int32_t gu_dtype, int64_t M,
                                           int64_t K, int64_t I, int32_t G, const void* lhs,
                                           float* lhs_scales, const uint8_t* rhs,
                                           const float* rhs_scales, const int32_t* group_sizes,
                                           void* gu, int32_t h_format, uint8_t* h_codes,
                                           float* h_scales, void* workspace,
                                           size_t workspace_bytes, gmm_stream_t stream);

/*
 * gmm_swiglu_bwd - the SwiGLU backward between the down projection's dlhs and the merged
 * gate|up dlhs.  From gu = [g | u] (bf16 [M, 2I], as gmm_fwd_swiglu returns it) and
 * dh = dL/dh (bf16 [M, I]), with s = 1 / (1 + exp(-g)):
 *
 *   d_gu[m, c]     = dh * u * s * (1 + g * (1 - s))      (dL/dg)
 *   d_gu[m, I + c] = dh * g * s                          (dL/du = dh * silu(g))
 *
 * in fp32 with each operation rounded to nearest, stored as bf16 [M, 2I].  I is a
 * positive multiple of 128; d_gu must not overlap the inputs.
 */
gmm_status_t gmm_swiglu_bwd(int64_t M, int64_t I, const void* dh, const void* gu, void* d_gu,
                            gmm_stream_t stream);

/*
 * gmm_dlhs_swiglu_bwd - the down projection's dlhs with the SwiGLU backward in its
 * epilogue ("FP8 Megablox for batch split", Description (2): gate and up projections
 * merged, so the backward of h = silu(g) * u meets the merged gu in one pass):
 *
 *   dh   = gmm_dlhs(grad, rhs) in bf16 (the same bits gmm_dlhs returns),
 *   d_gu = gmm_swiglu_bwd(dh, gu)          (the same bits as that call on dh),
 *
 * without dh leaving the product's epilogue: each tile reads gu's gate and up values for
 * its rows and channels and writes both halves of d_gu.
 * grad, grad_op, grad_scales, rhs (the down projection's weight as logical [G, I, N],
 * quantized per output channel i), rhs_scales f32 [G, I], rhs_layout, group_sizes and
 * the workspace are as in gmm_dlhs with K = I (GMM_OP_DLHS or GMM_OP_DLHS_FUSED sizes
 * suffice; there is no tail split).  I is a positive multiple of 128, at most 2^21.
 * gu           bf16 [M, 2I], the merged forward product [g | u] (gmm_fwd_swiglu's gu).
 * d_gu         bf16 [M, 2I] = [dL/dg | dL/du]; rows outside every group are not written.
 *              It must not overlap gu, the workspace or grad_scales (GMM_ERR_ALIAS).
 * d_gu_scales  NULL, or f32 [ceil(M / 128)]: also the dynamic scales of d_gu for its
 *              quantization as the next gradient, in d_gu_format (e4m3 or e5m2, else
 *              GMM_ERR_RECIPE): per block of 128 rows over all 2I columns,
 *              RNE_f32(max |d_gu| / qmax), the values gmm_dynamic_scales gives on d_gu,
 *              gathered in the same epilogue (so a dynamic_given gmm_quantize of d_gu
 *              needs no prepass).  It must not overlap any other buffer of the call.
 */
gmm_status_t gmm_dlhs_swiglu_bwd(const gmm_operand_t* grad_op, int32_t rhs_format,
                                 int32_t rhs_layout, int64_t M, int64_t I, int64_t N, int32_t G,
                                 const void* grad, float* grad_scales, const uint8_t* rhs,
                                 const float* rhs_scales, const int32_t* group_sizes,
                                 const void* gu, void* d_gu, int32_t d_gu_format,
                                 float* d_gu_scales, void* workspace, size_t workspace_bytes,
                                 gmm_stream_t stream);

/*
 * Block-wise scales ("Support quantization for tokamax gmm v2", review thread on the
 * ops diff: a 3-D weight scale is block-wise quantization; "add static LHS scaling
 * support for GMM v2 FWD", review thread on the lhs docstring: lhs scales of shape
 * [M, num_blocks]).  Block kb of the contraction covers k in [kb bk, (kb + 1) bk).
 *
 * gmm_fwd_blockwise - forward grouped matmul with scales that vary along K:
 *
 *   out[m, n] = RNE_out( sum_kb partial_kb[m, n] * lhs_scales[m, kb] * rhs_scales[g, kb, n] ),
 *   partial_kb[m, n] = sum_{k in block kb} lhs[m, k] * rhs[g, n, k]   (fp32),
 *
 * the sum over kb in fp32 from +0 in increasing kb, each block added with one fused
 * multiply-add by RNE(lhs_scales[m, kb] * rhs_scales[g, kb, n]).
 * lhs          fp8 codes [M, K] (lhs_format), lhs_scales f32 [M, K / bk] (from
 *              gmm_quantize_subchannel or any caller).
 * rhs          e4m3 codes [G, N, K] (contraction contiguous), rhs_scales f32
 *              [G, K / bk, N] (from gmm_quantize_rhs_blockwise with layout GMM_RHS_NK).
 * out          [M, N] bf16 or f32; rows outside every group are not written.
 * bk           a multiple of 128 dividing K (else GMM_ERR_SHAPE); K, N, M, G as for
 *              gmm_fwd.  No workspace.
 */
gmm_status_t gmm_fwd_blockwise(int32_t lhs_format, int32_t out_dtype, int64_t M, int64_t K,
                               int64_t N, int32_t G, int64_t bk, const uint8_t* lhs,
                               const float* lhs_scales, const uint8_t* rhs,
                               const float* rhs_scales, const int32_t* group_sizes, void* out,
                               gmm_stream_t stream);

/*
 * gmm_dlhs_blockwise - the lhs gradient with block-wise scales along its contraction n
 * (the dlhs is the gmm against the transposed weight: "Support quantization for tokamax
 * gmm v2", the dlhs call with transpose_rhs flipped, and its review thread on 3-D,
 * block-wise weight scales):
 *
 *   dlhs[m, k] = RNE_out( sum_nb partial_nb[m, k] * grad_scales[m, nb] * rhs_scales[g, k, nb] ),
 *   partial_nb[m, k] = sum_{n in block nb} grad[m, n] * rhs[g, k, n]   (fp32),
 *
 * summed as gmm_fwd_blockwise sums (from +0 in increasing nb, one fused multiply-add per
 * block by RNE(grad_scale * rhs_scale)).
 * grad         fp8 codes [M, N] (grad_format), grad_scales f32 [M, N / bk]
 *              (gmm_quantize_subchannel of the bf16 gradient).
 * rhs          e4m3 codes [G, K, N] (the weight's own layout, GMM_RHS_KN), rhs_scales f32
 *              [G, K, N / bk]: one scale per expert, output channel k and block of bk
 *              columns n, which is gmm_quantize_subchannel of the bf16 weight viewed as
 *              [G * K, N].
 * dlhs         [M, K] bf16 or f32; rows outside every group are not written.
 * bk           a multiple of 128 dividing N; M, K, N, G as for gmm_dlhs.  No workspace.
 */
gmm_status_t gmm_dlhs_blockwise(int32_t grad_format, int32_t out_dtype, int64_t M, int64_t K,
                                int64_t N, int32_t G, int64_t bk, const uint8_t* grad,
                                const float* grad_scales, const uint8_t* rhs,
                                const float* rhs_scales, const int32_t* group_sizes, void* dlhs,
                                gmm_stream_t stream);

/*
 * gmm_quantize_folded - the gradient of the dlhs that runs on the forward's weight copy
 * ("Support quantization for tokamax gmm v2", review threads on the ops diff: per-channel
 * weight scales; the dlhs is a gmm against the transposed rhs).  The forward's scales
 * s[g, n] lie on the dlhs contraction, so they are folded into the gradient first:
 *
 *   y[m, n] = RNE_f32(grad[m, n] * col_scales[g(m), n])       (g(m): the group of row m)
 *
 * then y gets the dynamic 128-row-block recipe (abs-max over the block's full width,
 * s = RNE(amax / qmax), inverse 0 when s is 0 or 1/s overflows, clamp then RNE).
 * grad bf16 [M, N], col_scales f32 [G, N], codes uint8 [M, N], scales f32 [ceil(M/128)].
 * gmm_dlhs on (codes, DYNAMIC_GIVEN-style block scales) with the forward's codes laid out
 * [G, K, N] and all-one rhs_scales [G, K] then computes the lhs gradient.  N a positive
 * multiple of 128; workspace ceil(M/128) * 32 bytes.
 */
gmm_status_t gmm_quantize_folded(int32_t format, int64_t M, int64_t N, int32_t G,
                                 const void* grad, const float* col_scales,
                                 const int32_t* group_sizes, uint8_t* codes, float* scales,
                                 void* workspace, size_t workspace_bytes, gmm_stream_t stream);

/*
 * gmm_quantize_subchannel - dynamic quantization of bf16 x [M, K] with one scale per row
 * and block of bk columns (bk = 128, 256 or 512, dividing K; else GMM_ERR_SHAPE):
 * s = RNE(amax / qmax) over the block, codes as gmm_quantize's dynamic recipe with that
 * block's inverse.  codes uint8 [M, K], scales f32 [M, K / bk].
 */
gmm_status_t gmm_quantize_subchannel(int32_t format, int64_t M, int64_t K, int64_t bk,
                                     const void* x, uint8_t* codes, float* scales,
                                     gmm_stream_t stream);

/*
 * gmm_quantize_rhs_blockwise - quantization of a bf16 weight w [G, K, N] with one scale
 * per expert, block of bk contraction rows and output column: scales f32 [G, K / bk, N]
 * (bk a multiple of 128 dividing K), codes in layout GMM_RHS_KN ([G, K, N]) or
 * GMM_RHS_NK ([G, N, K]).  With bk = K this is gmm_quantize_rhs on channel axis 0.
 */
gmm_status_t gmm_quantize_rhs_blockwise(int32_t format, int32_t layout, int64_t G, int64_t K,
                                        int64_t N, int64_t bk, const void* w, uint8_t* codes,
                                        float* scales, gmm_stream_t stream);

/*
 * Token routing around the grouped products: the MoE layer's permute before them and
 * unpermute after them (the later commits of "add static LHS scaling support for GMM v2
 * FWD": permute()/unpermute() in the MoE layer, activations quantized before the sort so
 * it moves fp8, and the expert outputs gathered back and reduced over the top-k).
 *
 * Slot s = t * k + j is the j-th expert choice of token t (expert_ids int32 [T, k]).
 * Permuted row order: the slots whose id is in [0, G), sorted by expert, slots of one
 * expert in increasing slot order, then the slots with any other id, in slot order: those
 * are dropped (capacity dropping, or a token routed to fewer than k experts).  Every
 * output is fully written.
 */

/* Workspace bytes of gmm_permute (one int per expert, plus one, and chunk of 256 slots,
 * and one int per slot). */
size_t gmm_permute_workspace_size(int64_t T, int32_t k, int32_t G);

/*
 * gmm_permute - sort token slots by expert and gather the rows.
 *
 * expert_ids   int32 [T, k], device.  0 <= T, 1 <= k <= 64, T * k < 2^31, 1 <= G <=
 *              GMM_MAX_GROUPS (else GMM_ERR_SHAPE).
 * group_sizes  OUTPUT int32 [G]: rows per expert, the group_sizes of the grouped
 *              products on x_perm; their sum, the number of routed slots, stays on the
 *              device.
 * row_of_slot  OUTPUT int32 [T * k]: the permuted row of every slot, -1 if dropped.
 * slot_of_row  OUTPUT int32 [T * k]: the slot of every permuted row (the routed rows
 *              first, sum(group_sizes) of them, then the dropped slots).
 * x, x_perm    optional (both or neither): x [T, row_bytes] bytes (bf16 values, fp8 codes
 *              of a static scale, ...), x_perm [T * k, row_bytes]; x_perm[r] = x[slot / k]
 *              for slot = slot_of_row[r].  row_bytes a positive multiple of 16.  A grouped
 *              product over all T * k rows takes the dropped tail as one more group.
 * workspace    gmm_permute_workspace_size(T, k, G) bytes; contents undefined after.
 * Pointers 16-byte aligned; outputs must not overlap inputs or one another.
 */
gmm_status_t gmm_permute(int64_t T, int32_t k, int32_t G, const int32_t* expert_ids,
                         int64_t row_bytes, const void* x, void* x_perm, int32_t* group_sizes,
                         int32_t* row_of_slot, int32_t* slot_of_row, void* workspace,
                         size_t workspace_bytes, gmm_stream_t stream);

/*
 * gmm_unpermute - gather every token's expert outputs back and reduce them:
 *
 *   out[t, c] = RNE_bf16( sum_{j = 0..k-1, row_of_slot[t k + j] >= 0}
 *                         weights[t, j] * y[row_of_slot[t k + j], c] )
 *
 * summed in fp32 in increasing j from +0, each product and each sum rounded to nearest
 * (a token whose slots are all dropped gets +0).  y bf16 [rows, H] (the products' output
 * on the permuted rows, rows = T * k); weights f32 [T, k] or NULL (all 1: then this is the
 * backward of gmm_permute's gather); out bf16 [T, H]; H a positive multiple of 8.
 */
gmm_status_t gmm_unpermute(int64_t T, int32_t k, int64_t H, const void* y,
                           const int32_t* row_of_slot, const float* weights, void* out,
                           gmm_stream_t stream);

/*
 * tgmm_drhs - weight gradient, the transposed grouped matmul ("Support quantization for
 * tokamax gmm v2", What this does: drhs_tgmm2).
 *
 *   drhs[g, k, n] = sum over 128-row blocks c meeting group g of
 *                   RNE( (sum_{m in c, m in g} q(lhs)[m, k] q(grad)[m, n]) * RNE(s_lhs[c] s_grad[c]) )
 *
 * lhs [M, K] and grad [M, N] are each either bf16 values, quantized in-kernel by the
 * operand's recipe (DYNAMIC_GIVEN reuses the block scales of the forward / dlhs calls
 * on the same tensors), or fp8 codes quantized beforehand with that recipe
 * (kind GMM_OPERAND_FP8: for instance the codes gmm_quantize made for gmm_fwd or
 * gmm_dlhs; the codes are used as they are, and must not be NaN or Inf encodings).
 * Because a dynamic scale changes every 128 rows, the contraction over rows is split at
 * block boundaries and each block's partial sum is scaled before it is added.
 * lhs_scales / grad_scales: as gmm_fwd's lhs_scales (outputs for DYNAMIC + BF16, may be
 * NULL; inputs for DYNAMIC_GIVEN and for DYNAMIC + FP8).
 * drhs [G, K, N] bf16 or f32.  A group with m_g == 0 gets a slab of +0.0.
 * Limits beyond the common ones: ceil(K / 256) * ceil(N / 256) * G < 2^31; otherwise
 * GMM_ERR_SHAPE.
 * workspace    required: gmm_workspace_size(GMM_OP_TGMM, lhs_op, grad_op, M, K, N, G)
 *              bytes: the plan of the call (per-group offsets, per-block scale products
 *              and their ratios) and, for an operand given as bf16, its codes quantized
 *              once, row-major.  Operands given as fp8 codes are read where they are.
 */
gmm_status_t tgmm_drhs(const gmm_operand_t* lhs_op, const gmm_operand_t* grad_op,
                       int32_t out_dtype, int64_t M, int64_t K, int64_t N, int32_t G,
                       const void* lhs, float* lhs_scales, const void* grad,
                       float* grad_scales, const int32_t* group_sizes, void* drhs,
                       void* workspace, size_t workspace_bytes, gmm_stream_t stream);

/* Bytes of device workspace the call `op` needs for these operands and sizes.
 * GMM_OP_FWD / GMM_OP_DLHS: `a` is the lhs / grad operand and `b` is ignored; `rows` is
 *   M, `cols_a` the operand's width (the contraction: K for fwd, N for dlhs) and `cols_b`
 *   the output width (N for fwd, K for dlhs; 0 = unknown, counted as wide).  The size
 *   covers the dynamic block scales the call computes, plus, for a bf16 operand of a
 *   wide output, its fp8 codes (rows x cols_a bytes).
 * GMM_OP_FWD_FUSED / GMM_OP_DLHS_FUSED: the same without the codes (0 unless the call
 *   computes dynamic block scales).
 * GMM_OP_QUANTIZE: gmm_quantize / gmm_dynamic_scales on `a` [rows, cols_a].
 * GMM_OP_FWD_SWIGLU: gmm_fwd_swiglu, `a` the lhs, `rows` M, `cols_a` K; a bf16 lhs always
 *   gets room for its codes (the SwiGLU epilogue reads fp8 codes).
 * GMM_OP_TGMM: `a` is the lhs and `b` the grad; tgmm always needs workspace for its plan
 *   (a few bytes per group and per 128-row block), plus rows x cols bytes of codes for
 *   each operand given as bf16.  `rows` is M, `cols_a` / `cols_b` the row widths (K and
 *   N), G the number of groups.
 * Sets *bytes. */
gmm_status_t gmm_workspace_size(int32_t op, const gmm_operand_t* a, const gmm_operand_t* b,
                                int64_t rows, int64_t cols_a, int64_t cols_b, int32_t G,
                                size_t* bytes);

/*
 * gmm_dynamic_scales - the abs-max prepass alone: per-block scales of a bf16 matrix
 * [R, C] for the DYNAMIC recipe of `format`, scales f32 [ceil(R/128)] (output).
 * workspace: gmm_workspace_size(GMM_OP_QUANTIZE, op{BF16, format, DYNAMIC}, NULL, R, C, 0, 1).
 */
gmm_status_t gmm_dynamic_scales(int32_t format, int64_t R, int64_t C, const void* x,
                                float* scales, void* workspace, size_t workspace_bytes,
                                gmm_stream_t stream);

/*
 * gmm_quantize - stand-alone quantization of a bf16 matrix [R, C] into fp8 codes with the
 * static or dynamic recipe above (codes [R, C]; scales f32 [ceil(R/128)]: output for
 * DYNAMIC, input for DYNAMIC_GIVEN, unused for STATIC).  The codes are byte-identical to those the fused
 * kernels form in registers.  Used for the pre-quantized-operand path (hybrid dlhs).
 * workspace: gmm_workspace_size(GMM_OP_QUANTIZE, op, NULL, R, C, 0, 1, &bytes).
 */
gmm_status_t gmm_quantize(const gmm_operand_t* op, int64_t R, int64_t C, const void* x,
                          uint8_t* codes, float* scales, void* workspace,
                          size_t workspace_bytes, gmm_stream_t stream);

/*
 * gmm_quantize_rhs - per-channel quantization of a bf16 weight w [G, K, N] ("FP8
 * Megablox for batch split", Description (1): the weight is quantized manually).
 *   channel_axis 0 -> one scale per (g, n), abs-max over k: scales [G, N]  (gmm_fwd)
 *   channel_axis 1 -> one scale per (g, k), abs-max over n: scales [G, K]  (gmm_dlhs)
 * s = RNE_f32(amax / qmax), inv = 0 if s == 0 or 1/s overflows else RNE_f32(1/s),
 * code = fp8(clamp(RNE_f32(w * inv), +-qmax)).  Codes are written in `layout`.
 */
gmm_status_t gmm_quantize_rhs(int32_t format, int32_t channel_axis, int32_t layout, int64_t G,
                              int64_t K, int64_t N, const void* w, uint8_t* codes,
                              float* scales, gmm_stream_t stream);

/* Host: per-tensor scale from a fixed calibration range [lo, hi]: requires lo == -hi > 0
 * (asymmetric ranges are rejected, "add static LHS scaling support for GMM v2 FWD",
 * review thread on the helper's docstring); *scale = RNE_f32(hi / qmax(format)). */
gmm_status_t gmm_static_scale_from_bound(float lo, float hi, int32_t format, float* scale);

/* Host: static text for a status code. */
const char* gmm_status_string(gmm_status_t status);

/* Host: library version string. */
const char* gmm_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GMM_FP8_H */
