// Routing (top-k + softmax weights) and grouping (stable counting sort by local expert).
//
// Routing: the pages ("fix(sm90): support parameterized SwiGLU in FP8 MegaMoE",
// Summary; "Pull Style Cutedsl Megakernel", Layout: top-k reduce) take the top-k
// experts per token; the selection order is (logit descending, expert id
// ascending) and the weights are a softmax over the k chosen logits, computed in
// fp64 and rounded once to fp32.
//
// Grouping: rows of a local expert are contiguous and ordered by slot id
// s = t*k + j; the grouped layout is what the pages' expert GEMMs consume
// ("Optimize sm100 version with token-aware BM240 tiling ...": description).
#include <hip/hip_runtime.h>
#include <climits>
#include <cmath>
#include <cstdint>

#include "device_common.hpp"
#include "moe_internal.hpp"

namespace moe {

// One wave per token; lane l holds logits l, l+64, l+128, ... (VPL of them).
template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + (size_t)t * E;
  float v[VPL];
  unsigned taken = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
    if (e >= E) taken |= 1u << i;
  }
  float sel_v[kMaxTopk];
  int sel_i[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    sel_v[j] = 0.f;
    sel_i[j] = 0;
    if (j < k) {
      float bv = -INFINITY;
      int bi = INT_MAX;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const bool free_ = !((taken >> i) & 1u);
        if (free_ && (bi == INT_MAX || v[i] > bv)) {
          bv = v[i];
          bi = lane + 64 * i;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      sel_v[j] = bv;
      sel_i[j] = bi;
    }
  }
  // softmax over the chosen logits in fp64: e_j = exp(l_j - l_0), S summed in slot order
  double ex[kMaxTopk];
  double S = 0.0;
  const double l0 = (double)sel_v[0];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    ex[j] = 0.0;
    if (j < k) {
      ex[j] = exp((double)sel_v[j] - l0);
      S = (j == 0) ? ex[0] : S + ex[j];
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    if (j < k && lane == j) {
      ids[(size_t)t * k + j] = sel_i[j];
      w[(size_t)t * k + j] = (float)(ex[j] / S);
    }
  }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    route_topk_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 128)
    route_topk_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 256)
    route_topk_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 512)
    route_topk_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else
    route_topk_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

__device__ __forceinline__ int bucket_of(int id, int e0, int EL) {
  const int le = id - e0;
  return (le >= 0 && le < EL) ? le : EL;  // EL = the non-local bucket
}

// Per-chunk bucket histogram (order-free integer counts).
__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ ids, int nslots, int e0, int EL,
                                                           int32_t* __restrict__ chunk_cnt) {
  extern __shared__ int hist[];
  const int NB = EL + 1;
  for (int b = threadIdx.x; b < NB; b += 256) hist[b] = 0;
  __syncthreads();
  const int base = blockIdx.x * kPermChunk;
  for (int i = threadIdx.x; i < kPermChunk; i += 256) {
    const int s = base + i;
    if (s < nslots) atomicAdd(&hist[bucket_of(ids[s], e0, EL)], 1);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < NB; b += 256) chunk_cnt[(size_t)blockIdx.x * NB + b] = hist[b];
}

// One workgroup: per-bucket running sums over chunks, then an exclusive scan over buckets.
__global__ __launch_bounds__(1024) void permute_scan_kernel(const int32_t* __restrict__ chunk_cnt, int nchunks, int EL,
                                                            int32_t* __restrict__ chunk_base,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int tot[2 * 1024 + 2];
  const int NB = EL + 1;
  for (int b = threadIdx.x; b < 2 * 1024; b += blockDim.x) tot[b] = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < NB; b += blockDim.x) {
    int run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const size_t at = (size_t)c * NB + b;
      const int v = chunk_cnt[at];
      chunk_base[at] = run;
      run += v;
    }
    tot[b] = run;
  }
  __syncthreads();
  block_exclusive_scan_2048(tot);  // tot[b] <- sum of tot[0..b)
  for (int b = threadIdx.x; b < NB; b += blockDim.x) {
    offsets[b] = tot[b];
    if (b < EL) counts[b] = tot[b + 1] - tot[b];
  }
}

// Stable scatter: slots in ascending order within each bucket.
__global__ __launch_bounds__(256) void permute_scatter_kernel(const int32_t* __restrict__ ids, int nslots, int e0,
                                                              int EL, const int32_t* __restrict__ chunk_base,
                                                              const int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ row_to_slot,
                                                              int32_t* __restrict__ slot_to_row) {
  extern __shared__ int sm[];
  const int NB = EL + 1;
  int* base = sm;       // [NB]
  int* wcnt = sm + NB;  // [4][NB]
  for (int b = threadIdx.x; b < NB; b += 256) {
    base[b] = offsets[b] + chunk_base[(size_t)blockIdx.x * NB + b];
    wcnt[b] = wcnt[NB + b] = wcnt[2 * NB + b] = wcnt[3 * NB + b] = 0;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int nbits = 1;
  while ((1 << nbits) < NB) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int r = 0; r < kPermChunk / 256; ++r) {
    const int s = blockIdx.x * kPermChunk + r * 256 + threadIdx.x;
    const bool valid = s < nslots;
    const int b = valid ? bucket_of(ids[s], e0, EL) : 0;
    uint64_t match = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (b >> bit) & 1;
      const uint64_t m = __ballot(valid && on);
      match &= on ? m : ~m;
    }
    const int rank = __popcll(match & lt);
    const int cnt = __popcll(match);
    const bool leader = valid && rank == 0;
    if (leader) wcnt[wave * NB + b] = cnt;
    __syncthreads();
    int pos = 0;
    if (valid) {
      pos = base[b] + rank;
      for (int q = 0; q < wave; ++q) pos += wcnt[q * NB + b];
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&base[b], cnt);
      wcnt[wave * NB + b] = 0;
    }
    __syncthreads();
    if (valid) {
      if (b < EL) {
        row_to_slot[pos] = s;
        slot_to_row[s] = pos;
      } else {
        row_to_slot[pos] = -1;
        slot_to_row[s] = -1;
      }
    }
  }
}

hipError_t launch_permute(const int32_t* ids, int nslots, int e0, int EL, int32_t* chunk_cnt, int32_t* chunk_base,
                          int32_t* counts, int32_t* offsets, int32_t* row_to_slot, int32_t* slot_to_row,
                          hipStream_t s) {
  const int NB = EL + 1;
  const int nchunks = (nslots + kPermChunk - 1) / kPermChunk;
  if (nchunks > 0) {
    permute_hist_kernel<<<nchunks, 256, NB * sizeof(int), s>>>(ids, nslots, e0, EL, chunk_cnt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  permute_scan_kernel<<<1, 1024, 0, s>>>(chunk_cnt, nchunks, EL, chunk_base, counts, offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nchunks == 0) return e;
  permute_scatter_kernel<<<nchunks, 256, 5 * NB * sizeof(int), s>>>(ids, nslots, e0, EL, chunk_base, offsets,
                                                                     row_to_slot, slot_to_row);
  return hipGetLastError();
}

}  // namespace moe
