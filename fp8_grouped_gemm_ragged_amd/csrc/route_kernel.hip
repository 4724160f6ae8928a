// Token routing on either side of the grouped products (the MoE layer's permute and
// unpermute; "FP8 Megablox for batch split" and the later commits of "add static LHS
// scaling support for GMM v2 FWD": tokens are sorted by expert before the grouped matmul,
// quantized first so the move carries fp8, and the expert outputs are gathered back and
// reduced over each token's top-k choices).
//
// Routing: slot s = t * k + j holds the j-th expert choice of token t.  The permuted rows
// are the valid slots (0 <= expert < G) sorted by expert, ties kept in slot order (a
// stable counting sort), so every expert's rows are contiguous and group_sizes[e] counts
// them.  Slots with another id are dropped: row_of_slot = -1, and they fill the rows
// after the routed ones in slot order (key G of the sort), so every row is defined.
//   route_count_kernel   per-chunk histogram of the keys (LDS counters)
//   route_scan_kernel    per key, an exclusive scan of its chunk counts; group_sizes
//   route_rank_kernel    one wave per chunk: destination row of every slot, in slot order
//   route_gather_kernel  x_perm[row of slot t k + j] = x[t]: each row read once, k stores
//   route_combine_kernel out[t] = sum_j w[t, j] * y[row_of_slot[t k + j]] in fp32, in
//                        j order, each product and sum rounded to nearest; bf16 out
#include <algorithm>

#include "kernels.hpp"

namespace gmm {

namespace {

__device__ inline bool routed(int e, int G) { return (unsigned)e < (unsigned)G; }
// sort key of a slot: its expert, or G when dropped
__device__ inline int route_key(int e, int G) { return routed(e, G) ? e : G; }

__global__ __launch_bounds__(256) void route_count_kernel(const int32_t* __restrict__ ids,
                                                          int64_t n, int G,
                                                          int32_t* __restrict__ counts) {
  __shared__ int hist[MAX_GROUPS + 1];
  for (int e = threadIdx.x; e <= G; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * ROUTE_CHUNK;
  const int64_t s1 = std::min<int64_t>(s0 + ROUTE_CHUNK, n);
  for (int64_t s = s0 + threadIdx.x; s < s1; s += 256) atomicAdd(&hist[route_key(ids[s], G)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e <= G; e += 256) counts[(int64_t)blockIdx.x * (G + 1) + e] = hist[e];
}

// One workgroup per key (G + 1 of them): counts[b][e] becomes the number of slots of key
// e in the chunks before b; group_sizes[e] the total (key G, the dropped slots, has none).
__global__ __launch_bounds__(256) void route_scan_kernel(int32_t* __restrict__ counts, int nblk,
                                                         int G, int32_t* __restrict__ gs) {
  __shared__ int wsum[4];
  const int e = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    const int b = b0 + threadIdx.x;
    const int c = b < nblk ? counts[(int64_t)b * (G + 1) + e] : 0;
    const int incl = wave_incl_scan(c, lane);
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int before = carry;
    for (int i = 0; i < w; ++i) before += wsum[i];
    if (b < nblk) counts[(int64_t)b * (G + 1) + e] = before + incl - c;
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();  // wsum is rewritten by the next round
  }
  if (threadIdx.x == 0 && e < G) gs[e] = carry;
}

// One wave per chunk of ROUTE_CHUNK slots, taken 64 at a time in slot order.  Lanes that
// share an expert are found with a ballot per distinct expert; each gets the expert's
// running row plus its rank among those lanes, and the lowest lane advances the counter.
__global__ __launch_bounds__(64) void route_rank_kernel(const int32_t* __restrict__ ids,
                                                        int64_t n, int G,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ gs,
                                                        int32_t* __restrict__ row_of_slot,
                                                        int32_t* __restrict__ slot_of_row,
                                                        int32_t* __restrict__ dest_all) {
  __shared__ int run[MAX_GROUPS + 1];
  const int lane = threadIdx.x;
  // run[e] = first row of key e (exclusive prefix of group_sizes; key G starts after
  // every routed slot) + its slots in earlier chunks
  int carry = 0;
  for (int e0 = 0; e0 <= G; e0 += 64) {
    const int e = e0 + lane;
    const int v = e < G ? gs[e] : 0;
    const int incl = wave_incl_scan(v, lane);
    if (e <= G) run[e] = carry + incl - v + counts[(int64_t)blockIdx.x * (G + 1) + e];
    carry += __shfl(incl, 63, 64);
  }
  __syncthreads();
  const uint64_t below = (uint64_t(1) << lane) - 1;
  const int64_t s0 = (int64_t)blockIdx.x * ROUTE_CHUNK;
  const int64_t s1 = std::min<int64_t>(s0 + ROUTE_CHUNK, n);
  for (int64_t p = s0; p < s1; p += 64) {
    const int64_t s = p + lane;
    const bool ok = s < s1;
    const int e = ok ? route_key(ids[s], G) : G;
    uint64_t todo = __ballot(ok);
    int dest = -1;
    while (todo) {
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int le = __builtin_amdgcn_readlane(e, leader);
      const uint64_t same = __ballot(ok && e == le);
      const int start = run[le];
      if (ok && e == le) dest = start + __popcll(same & below);
      if (lane == leader) run[le] = start + __popcll(same);
      todo &= ~same;
    }
    if (ok) {
      row_of_slot[s] = e < G ? dest : -1;
      dest_all[s] = dest;
      if (dest >= 0 && dest < n) slot_of_row[dest] = (int32_t)s;
    }
  }
}

// GATHER_TOKENS tokens per workgroup and iteration: every 16-byte piece of a token's row
// is read once and stored into the rows of its k slots (dest holds the row of every slot,
// dropped ones included).
constexpr int GATHER_TOKENS = 4;

__global__ __launch_bounds__(256) void route_gather_kernel(const uint8_t* __restrict__ x,
                                                           int64_t T, int k, int64_t row_bytes,
                                                           const int32_t* __restrict__ dest,
                                                           uint8_t* __restrict__ xp) {
  const int64_t vecs = row_bytes / 16, n = T * k;
  for (int64_t t0 = (int64_t)blockIdx.x * GATHER_TOKENS; t0 < T;
       t0 += (int64_t)gridDim.x * GATHER_TOKENS) {
    const int64_t pieces = std::min<int64_t>(GATHER_TOKENS, T - t0) * vecs;
    for (int64_t i = threadIdx.x; i < pieces; i += 256) {
      const int64_t tt = i / vecs, c = i - tt * vecs, t = t0 + tt;
      const v4u v = *reinterpret_cast<const v4u*>(x + t * row_bytes + c * 16);
      for (int j = 0; j < k; ++j) {
        const int d = dest[t * k + j];
        if (d >= 0 && d < n) *reinterpret_cast<v4u*>(xp + (int64_t)d * row_bytes + c * 16) = v;
      }
    }
  }
}

// One token per workgroup and iteration; 8 channels per thread.
__global__ __launch_bounds__(256) void route_combine_kernel(const uint16_t* __restrict__ y,
                                                            int64_t T, int k, int64_t H,
                                                            int64_t rows,
                                                            const int32_t* __restrict__ row_of_slot,
                                                            const float* __restrict__ w,
                                                            uint16_t* __restrict__ out) {
  const int64_t vecs = H / 8;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    for (int64_t v = threadIdx.x; v < vecs; v += 256) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
      // four slots at a time: their loads are issued before the sums that use them
      for (int j0 = 0; j0 < k; j0 += 4) {
        v4u q[4];
        float wj[4];
        bool live[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = j0 + u;
          const int r = j < k ? row_of_slot[t * k + j] : -1;
          live[u] = r >= 0 && r < rows;
          wj[u] = live[u] && w ? w[t * k + j] : 1.0f;
          if (live[u]) q[u] = *reinterpret_cast<const v4u*>(y + (int64_t)r * H + v * 8);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (!live[u]) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] = add_rn(acc[2 * i], mul_rn(wj[u], bf16_lo(q[u][i])));
            acc[2 * i + 1] = add_rn(acc[2 * i + 1], mul_rn(wj[u], bf16_hi(q[u][i])));
          }
        }
      }
      v4u o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
      *reinterpret_cast<v4u*>(out + t * H + v * 8) = o;
    }
  }
}

}  // namespace

int64_t route_chunks(int64_t n) { return (n + ROUTE_CHUNK - 1) / ROUTE_CHUNK; }

hipError_t launch_route(const int32_t* ids, int64_t n, int k, int G, int32_t* counts,
                        int32_t* dest_all, int32_t* gs, int32_t* row_of_slot,
                        int32_t* slot_of_row, const void* x, int64_t row_bytes, void* x_perm,
                        hipStream_t st) {
  const int64_t nblk = route_chunks(n);
  if (nblk == 0) {
    // no slots: every expert is empty
    hipLaunchKernelGGL(route_scan_kernel, dim3(G + 1), dim3(256), 0, st, counts, 0, G, gs);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_count_kernel, dim3((unsigned)nblk), dim3(256), 0, st, ids, n, G,
                     counts);
  hipLaunchKernelGGL(route_scan_kernel, dim3(G + 1), dim3(256), 0, st, counts, (int)nblk, G, gs);
  hipLaunchKernelGGL(route_rank_kernel, dim3((unsigned)nblk), dim3(64), 0, st, ids, n, G, counts,
                     gs, row_of_slot, slot_of_row, dest_all);
  if (x && x_perm) {
    const int64_t T = n / k;
    const int64_t blocks = std::min<int64_t>((T + GATHER_TOKENS - 1) / GATHER_TOKENS, 256 * 16);
    hipLaunchKernelGGL(route_gather_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint8_t*)x, T, k, row_bytes, dest_all, (uint8_t*)x_perm);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* y, int64_t T, int k, int64_t H, int64_t rows,
                          const int32_t* row_of_slot, const float* w, uint16_t* out,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(T, 256 * 64);
  hipLaunchKernelGGL(route_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, st, y, T, k, H,
                     rows, row_of_slot, w, out);
  return hipGetLastError();
}

}  // namespace gmm
