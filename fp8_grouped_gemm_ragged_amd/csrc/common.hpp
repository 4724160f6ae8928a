// Shared device helpers of the gfx950 FP8 grouped matmul kernels.
//
// Nothing here is used by the CPU oracle; the oracle and these kernels share no code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmm {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef int32_t v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// fp8 format selectors: the value is also the MFMA operand-format code of gfx950's
// V_MFMA_*_F8F6F4 instructions (0 = E4M3, 1 = E5M2).
enum : int { FMT_E4M3 = 0, FMT_E5M2 = 1 };

template <int FMT>
__device__ __host__ constexpr float qmax() {
  return FMT == FMT_E4M3 ? 448.0f : 57344.0f;
}

constexpr int BLOCK_ROWS = 128;  // rows per dynamic-scale block
constexpr int TILE_K = 128;      // contraction bytes per LDS row (one fp8 k-step)

// ---------------------------------------------------------------------------------
// Buffer resources: range-checked loads.  A lane whose byte offset lies beyond
// num_records reads zeros without touching memory, which is how rows past the end of
// a group (or past the last output channel) become zero operands.
// ---------------------------------------------------------------------------------
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ inline v4u buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// A range-checked 16-byte store: a lane whose byte offset lies beyond num_records writes
// nothing, which is how rows past the end of a group are left alone.
__device__ inline void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, v4u v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// ---------------------------------------------------------------------------------
// LDS tile layout: a tile is [rows][128 bytes] of fp8 codes, the contraction axis
// contiguous.  16-byte chunk c of row r is stored at chunk position
// c ^ (r & 7) ^ ((r >> 3) & 7): the eight rows an MFMA fragment read touches together
// land in eight different chunk positions, and so do the rows one transposing store
// touches together.
// ---------------------------------------------------------------------------------
__device__ inline uint32_t tile_off(uint32_t row, uint32_t chunk) {
  return row * TILE_K + ((chunk ^ (row & 7u) ^ ((row >> 3) & 7u)) << 4);
}

// ---------------------------------------------------------------------------------
// In-register quantization: code = fp8(clamp(RNE_f32(x * inv), -qmax, qmax)), RNE.
// The multiply is an explicit round-to-nearest fp32 multiply (never fused), the clamp
// is a median of three, and the conversion is gfx950's V_CVT_PK_{FP8,BF8}_F32
// (round to nearest even, OCP encodings).
// ---------------------------------------------------------------------------------
template <int FMT>
__device__ inline float quant_prep(float x, float inv) {
  float y = __fmul_rn(x, inv);
  return __builtin_amdgcn_fmed3f(y, -qmax<FMT>(), qmax<FMT>());
}

// Packs two codes into bytes 0-1 (HI == false) or 2-3 (HI == true) of `old`.
template <int FMT, bool HI>
__device__ inline uint32_t cvt_pk(float a, float b, uint32_t old) {
  if constexpr (FMT == FMT_E4M3)
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
  else
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}

// Abs-max of bf16 values through their bit patterns: for finite bf16, |x| orders like
// the unsigned integer (bits & 0x7fff).  Returns the larger magnitude bits seen.
__device__ inline uint32_t absmax_bits16(v4u w, uint32_t m) {
  const uint32_t mask = 0x7fff7fffu;
  uint32_t a = w.x & mask, b = w.y & mask, c = w.z & mask, d = w.w & mask;
  uint32_t lo = max(max(a & 0xffffu, b & 0xffffu), max(c & 0xffffu, d & 0xffffu));
  uint32_t hi = max(max(a >> 16, b >> 16), max(c >> 16, d >> 16));
  return max(m, max(lo, hi));
}

// An fp32 product and an fp32 sum, each rounded to nearest on its own: never contracted
// into a fused multiply-add (HIP's __fmul_rn / __fadd_rn are plain operators, which the
// compiler fuses under its default contraction).
__device__ inline float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ inline float add_rn(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

// Inverse of a dynamic scale: RNE_f32(1/s), or 0 when s == 0 or 1/s is not finite.
__device__ inline float inv_from_scale(float s) {
  const float r = __fdiv_rn(1.0f, s);
  return (s == 0.0f || !__builtin_isfinite(r)) ? 0.0f : r;
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 4 fp32 values -> 4 fp8 codes (one dword, value e in byte e).
template <int FMT>
__device__ inline uint32_t quant4(v4f v, float inv) {
  const uint32_t d = cvt_pk<FMT, false>(quant_prep<FMT>(v[0], inv), quant_prep<FMT>(v[1], inv), 0u);
  return cvt_pk<FMT, true>(quant_prep<FMT>(v[2], inv), quant_prep<FMT>(v[3], inv), d);
}

// 4 packed bf16 pairs (8 values, one 16-byte load) -> 8 fp8 codes (2 dwords).
template <int FMT>
__device__ inline v2u quant8(v4u w, float inv) {
  v2u r;
  // the first conversion of each dword writes bytes 0-1 and keeps 2-3 of its `old`
  // operand, which the second one overwrites: any register serves as `old`
  uint32_t d0 = cvt_pk<FMT, false>(quant_prep<FMT>(bf16_lo(w.x), inv), quant_prep<FMT>(bf16_hi(w.x), inv), w.x);
  d0 = cvt_pk<FMT, true>(quant_prep<FMT>(bf16_lo(w.y), inv), quant_prep<FMT>(bf16_hi(w.y), inv), d0);
  uint32_t d1 = cvt_pk<FMT, false>(quant_prep<FMT>(bf16_lo(w.z), inv), quant_prep<FMT>(bf16_hi(w.z), inv), w.z);
  d1 = cvt_pk<FMT, true>(quant_prep<FMT>(bf16_lo(w.w), inv), quant_prep<FMT>(bf16_hi(w.w), inv), d1);
  r.x = d0;
  r.y = d1;
  return r;
}

// Two floats -> a packed bf16 pair (a in bits 0-15), each rounded to nearest even:
// gfx950's V_CVT_PK_BF16_F32, one instruction for both.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  const f2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// SwiGLU backward of 8 channels of one row ("FP8 Megablox for batch split", Description
// (2): gate and up projections merged): from bf16 dh (d), gate g and up u, with
// s = sigmoid(g) through the hardware exp2 and reciprocal (about one ulp each) and every
// other operation rounded to nearest in fp32,
//   dL/dg = ((d * u) * s) * (1 + g * (1 - s)),   dL/du = d * (g * s),
// returned as bf16 (RNE) in og and ou.  The elementwise kernel and the dlhs epilogue
// that fuses this step both call it, so the two give the same bits.
__device__ __forceinline__ void swiglu_bwd8(const v4u d, const v4u g8, const v4u u8, v4u& og,
                                            v4u& ou) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float dg[2], du[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float g = h ? bf16_hi(g8[k]) : bf16_lo(g8[k]);
      const float u = h ? bf16_hi(u8[k]) : bf16_lo(u8[k]);
      const float dv = h ? bf16_hi(d[k]) : bf16_lo(d[k]);
      const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
      const float grow = add_rn(1.0f, mul_rn(g, __fsub_rn(1.0f, s)));
      dg[h] = __fmul_rn(__fmul_rn(__fmul_rn(dv, u), s), grow);
      du[h] = __fmul_rn(dv, __fmul_rn(g, s));
    }
    og[k] = pack_bf16x2(dg[0], dg[1]);
    ou[k] = pack_bf16x2(du[0], du[1]);
  }
}

// ---------------------------------------------------------------------------------
// MFMA: D[32x32] += A[32x64] * B[64x32], fp8/bf8 operands, fp32 accumulation.  Lane l
// holds row (l % 32) of A and column (l % 32) of B, 32 contraction bytes each; the
// two operands use the same contraction order, so any consistent assignment of the
// 64 contraction bytes to (lane half, byte) gives the same sum.  The result lane l,
// register r is D[8*(r/4) + 4*(l/32) + r%4][l % 32].
// ---------------------------------------------------------------------------------
template <int FMT_A, int FMT_B>
__device__ inline v16f mfma32x32x64(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT_A, FMT_B, 0, 0, 0, 0);
}

__device__ inline v8i lds_read_frag(const uint8_t* lds, uint32_t row, uint32_t chunk0) {
  v4u lo = *reinterpret_cast<const v4u*>(lds + tile_off(row, chunk0));
  v4u hi = *reinterpret_cast<const v4u*>(lds + tile_off(row, chunk0 + 1));
  v8i f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

// ---------------------------------------------------------------------------------
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

// ---------------------------------------------------------------------------------
// Wave-level inclusive prefix sum (64 lanes).
// ---------------------------------------------------------------------------------
__device__ inline int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Wave-level inclusive prefix sum that saturates at cap: every value lies in [0, cap]
// and cap < 2^31, so no partial sum wraps.
__device__ inline uint32_t wave_incl_scan_sat(uint32_t v, int lane, uint32_t cap) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v = min(v + o, cap);
  }
  return v;
}

// Expert-tile prefix sums, computed by one whole wave.  Groups 0 .. G-1 with sizes gs[g]
// follow `rows_before` rows (<= M).  Every size is read as clamp(gs[g], 0, M) and every
// row offset is clamped to M, so sizes that break the contract (negative, or summing past
// M) can never place a tile outside rows [0, M).  Writes row_off[0 .. G] (row_off[g] =
// first row of group g, row_off[G] = end of the last) and tile_cum[0 .. G] (BM-row tiles
// of the groups before g, each group's count taken from its clamped row range).
template <int BM>
__device__ inline void group_tiles_prefix(const int32_t* __restrict__ gs, int G, uint32_t M,
                                          uint32_t rows_before, int* tile_cum, int* row_off) {
  const int lane = threadIdx.x & 63;
  uint32_t carry_r = rows_before;
  int carry_t = 0;
  if (lane == 0) {
    tile_cum[0] = 0;
    row_off[0] = (int)rows_before;
  }
  for (int base = 0; base < G; base += 64) {
    const int g = base + lane;
    const uint32_t m = g < G ? (uint32_t)min(max(gs[g], 0), (int)M) : 0u;
    const uint32_t ir = wave_incl_scan_sat(m, lane, M);
    // the shuffle runs on every lane (a lane reads another lane's value only while that
    // lane is active), then lane 0 takes 0
    const uint32_t up = (uint32_t)__shfl_up(ir, 1, 64);
    const uint32_t ex = lane == 0 ? 0u : up;
    const uint32_t end = min(carry_r + ir, M), start = min(carry_r + ex, M);
    const int it = wave_incl_scan((int)((end - start + BM - 1) / BM), lane);
    if (g < G) {
      tile_cum[g + 1] = carry_t + it;
      row_off[g + 1] = (int)end;
    }
    carry_t += __shfl(it, 63, 64);
    carry_r = min(carry_r + (uint32_t)__shfl(ir, 63, 64), M);
  }
}

// Rows of the first n groups, clamped as in group_tiles_prefix (one whole wave).
__device__ inline uint32_t rows_of_groups(const int32_t* __restrict__ gs, int n, uint32_t M) {
  const int lane = threadIdx.x & 63;
  uint32_t carry = 0;
  for (int base = 0; base < n; base += 64) {
    const int g = base + lane;
    const uint32_t m = g < n ? (uint32_t)min(max(gs[g], 0), (int)M) : 0u;
    const uint32_t ir = wave_incl_scan_sat(m, lane, M);
    carry = min(carry + (uint32_t)__shfl(ir, 63, 64), M);
  }
  return carry;
}

}  // namespace gmm
