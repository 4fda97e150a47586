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

// Selection keys: the logit's bits mapped so that unsigned order is float order (-0 is
// folded onto +0 first, so equal logits compare equal), above the complemented expert id,
// so the unsigned maximum is the largest logit and, among equal logits, the lowest id.
// 0 is below every finite logit's key and marks a taken (or absent) expert.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)~e;
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}
__device__ __forceinline__ int key_id(uint64_t key) { return (int)~(uint32_t)key; }

template <int CTRL>  // the 64-bit value of the lane the DPP pattern names
__device__ __forceinline__ uint64_t dpp64(uint64_t x) {
  const int lo = (int)(uint32_t)x, hi = (int)(uint32_t)(x >> 32);
  const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xf, 0xf, false);
  const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xf, 0xf, false);
  return ((uint64_t)h2 << 32) | l2;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t readlane64(uint64_t x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
// maximum over the wave: quad xor-1 and xor-2 swaps and row rotations by 4 and 8 reduce each
// 16-lane row, then the four row results are read into scalars (the result is uniform)
__device__ __forceinline__ uint64_t wave_max64(uint64_t x) {
  x = umax64(x, dpp64<0xB1>(x));   // quad_perm [1,0,3,2]
  x = umax64(x, dpp64<0x4E>(x));   // quad_perm [2,3,0,1]
  x = umax64(x, dpp64<0x124>(x));  // row_ror 4
  x = umax64(x, dpp64<0x128>(x));  // row_ror 8
  return umax64(umax64(readlane64(x, 0), readlane64(x, 16)), umax64(readlane64(x, 32), readlane64(x, 48)));
}

// One wave per token; lane l holds the keys of experts l, l+64, l+128, ... (VPL of them).
// Round j takes the wave maximum of the untaken keys; lane j keeps slot j, so the softmax
// needs one exp and one divide per lane, and its sum runs over the slots in order.
template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + (size_t)t * E;
  float v[VPL];  // every load unconditional (index clamped), so all are in flight at once
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = row[min(lane + 64 * i, E - 1)];
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? route_key(v[i], e) : 0ull;
  }
  uint64_t mine = 0;  // lane j: the key of slot j
  for (int j = 0; j < k; ++j) {
    uint64_t b = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) b = umax64(b, key[i]);
    const uint64_t best = wave_max64(b);
    const int id = key_id(best);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (id == lane + 64 * i) key[i] = 0ull;
    if (lane == j) mine = best;
  }
  // softmax over the chosen logits in fp64: e_j = exp(l_j - l_0), S = e_0 + e_1 + ... in
  // slot order, w_j = fp32(e_j / S)
  const double l0 = (double)key_value(readlane64(mine, 0));
  const double ex = lane < k ? exp((double)key_value(mine) - l0) : 0.0;
  const int2 ex2 = *reinterpret_cast<const int2*>(&ex);
  double S = 0.0;
  for (int j = 0; j < k; ++j) {
    const int2 v = make_int2(__builtin_amdgcn_readlane(ex2.x, j), __builtin_amdgcn_readlane(ex2.y, j));
    S = j == 0 ? *reinterpret_cast<const double*>(&v) : S + *reinterpret_cast<const double*>(&v);
  }
  if (lane < k) {
    ids[(size_t)t * k + lane] = key_id(mine);
    w[(size_t)t * k + lane] = (float)(ex / S);
  }
}

// Up to 256 experts: one 16-lane row per token, four tokens per wave; lane l of a row holds
// the keys of experts l, l + 16, l + 32, ... (NK of them).  A round's maximum stays inside
// the row (quad swaps, then rotations by 4 and 8 leave it in all 16 lanes), so no lane has
// to be read out of the wave.  The softmax sum runs through the row one lane at a time
// (row shift by one), so it adds e_0, e_1, ... in slot order like the wave-per-token kernel.
template <int NK>
__global__ __launch_bounds__(256) void route_topk_row_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                             int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63, lr = lane & 15;
  const int t = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  const bool valid = t < T;
  const float* row = logits + (size_t)(valid ? t : 0) * E;
  float v[NK];  // every load unconditional (index clamped), so all are in flight at once
#pragma unroll
  for (int i = 0; i < NK; ++i) v[i] = row[min(lr + 16 * i, E - 1)];
  uint64_t key[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = lr + 16 * i;
    key[i] = valid && e < E ? route_key(v[i], e) : 0ull;
  }
  uint64_t mine = 0, first = 0;  // lane j of the row: the key of slot j; every lane: slot 0's
  for (int j = 0; j < k; ++j) {
    uint64_t b = key[0];
#pragma unroll
    for (int i = 1; i < NK; ++i) b = umax64(b, key[i]);
    b = umax64(b, dpp64<0xB1>(b));   // quad_perm [1,0,3,2]
    b = umax64(b, dpp64<0x4E>(b));   // quad_perm [2,3,0,1]
    b = umax64(b, dpp64<0x124>(b));  // row_ror 4
    b = umax64(b, dpp64<0x128>(b));  // row_ror 8
    const int id = key_id(b);
#pragma unroll
    for (int i = 0; i < NK; ++i)
      if (id == lr + 16 * i) key[i] = 0ull;
    if (lr == j) mine = b;
    if (j == 0) first = b;
  }
  const double l0 = (double)key_value(first);
  const double ex = lr < k ? exp((double)key_value(mine) - l0) : 0.0;
  double acc = ex;  // after step i, lane i holds e_0 + ... + e_i (added in that order)
  for (int i = 1; i < k; ++i) {
    const int2 a = *reinterpret_cast<const int2*>(&acc);
    const int2 p = make_int2(__builtin_amdgcn_update_dpp(0, a.x, 0x111, 0xf, 0xf, false),   // row_shr:1
                             __builtin_amdgcn_update_dpp(0, a.y, 0x111, 0xf, 0xf, false));
    if (lr == i) acc = *reinterpret_cast<const double*>(&p) + ex;
  }
  const double S = __shfl(acc, (lane & ~15) + k - 1);
  if (valid && lr < k) {
    ids[(size_t)t * k + lr] = key_id(mine);
    w[(size_t)t * k + lr] = (float)(ex / S);
  }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // the row kernel launches a quarter of the waves: it wins once the tokens fill the GPU
  // (32768 tokens: 29 against 43 us) and loses while each wave's latency decides (4096
  // tokens: 12.7 against 10.6 us)
  if (E <= 256 && T >= 16384) {
    dim3 rgrid((T + 15) / 16), rblock(256);
    if (E <= 16)
      route_topk_row_kernel<1><<<rgrid, rblock, 0, s>>>(logits, T, E, k, ids, w);
    else if (E <= 32)
      route_topk_row_kernel<2><<<rgrid, rblock, 0, s>>>(logits, T, E, k, ids, w);
    else if (E <= 64)
      route_topk_row_kernel<4><<<rgrid, rblock, 0, s>>>(logits, T, E, k, ids, w);
    else if (E <= 128)
      route_topk_row_kernel<8><<<rgrid, rblock, 0, s>>>(logits, T, E, k, ids, w);
    else
      route_topk_row_kernel<16><<<rgrid, rblock, 0, s>>>(logits, T, E, k, ids, w);
    return hipGetLastError();
  }
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

// ids[s], or ids[n - 1] past the end (n >= 1): the load is unconditional, so a run of them
// is in flight together instead of each waiting behind a branch of its own
__device__ __forceinline__ int load_clamped(const int32_t* __restrict__ ids, int s, int n) {
  return ids[s < n ? s : n - 1];
}

// Per-chunk bucket histogram (order-free integer counts).
__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ ids, int nslots, int e0, int EL,
                                                           int32_t* __restrict__ chunk_cnt) {
  extern __shared__ int hist[];
  const int NB = EL + 1;
  for (int b = threadIdx.x; b < NB; b += 256) hist[b] = 0;
  __syncthreads();
  const int base = blockIdx.x * kPermChunk;
  constexpr int kPer = kPermChunk / 256;
  int id[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) id[r] = load_clamped(ids, base + r * 256 + (int)threadIdx.x, nslots);
#pragma unroll
  for (int r = 0; r < kPer; ++r)
    if (base + r * 256 + (int)threadIdx.x < nslots) atomicAdd(&hist[bucket_of(id[r], e0, EL)], 1);
  __syncthreads();
  for (int b = threadIdx.x; b < NB; b += 256) chunk_cnt[(size_t)blockIdx.x * NB + b] = hist[b];
}

// One workgroup: per-bucket running sums over chunks, then an exclusive scan over buckets.
__global__ __launch_bounds__(1024) void permute_scan_kernel(const int32_t* __restrict__ chunk_cnt, int nchunks, int EL,
                                                            int bm, int32_t* __restrict__ chunk_base,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ plan) {
  __shared__ int tot[2 * 1024 + 2];
  __shared__ int mt[2 * 1024 + 2];
  const int NB = EL + 1;
  for (int b = threadIdx.x; b < 2 * 1024; b += blockDim.x) tot[b] = mt[b] = 0;
  __syncthreads();
  // one wave per bucket: its chunk counts, 64 chunks per pass, become exclusive prefixes
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int b = wave; b < NB; b += 16) {
    int carry = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {  // uniform
      const int c = c0 + lane;
      const size_t at = (size_t)c * NB + b;
      const int v = c < nchunks ? chunk_cnt[at] : 0;
      const int inc = wave_inclusive_scan_dpp(v);
      if (c < nchunks) chunk_base[at] = carry + inc - v;
      carry += __builtin_amdgcn_readlane(inc, 63);
    }
    if (lane == 0) {
      tot[b] = carry;
      if (b < EL) mt[b] = (carry + bm - 1) / bm;  // m-tiles of this expert
    }
  }
  __syncthreads();
  block_exclusive_scan_2048(tot);  // tot[b] <- sum of tot[0..b)
  block_exclusive_scan_2048(mt);
  for (int b = threadIdx.x; b < NB; b += blockDim.x) {
    offsets[b] = tot[b];
    plan[b] = mt[b];
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

// Everything in one workgroup when the slots are few (decode-sized calls): histogram,
// scans, tile plan and the stable scatter, in rounds of 1024 slots.
__global__ __launch_bounds__(1024) void permute_small_kernel(const int32_t* __restrict__ ids, int nslots, int e0,
                                                             int EL, int bm, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ row_to_slot,
                                                             int32_t* __restrict__ slot_to_row,
                                                             int32_t* __restrict__ plan) {
  __shared__ int a[2 * 1024 + 2];
  __shared__ int mt[2 * 1024 + 2];
  __shared__ int base[kPermSmallBuckets];
  __shared__ int wcnt[16][kPermSmallBuckets];
  const int NB = EL + 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // the bucket of each of this thread's slots (slot r * 1024 + tid of round r), loaded once
  // and kept for the scatter; -1 past the last slot
  constexpr int kRounds = kPermSmallSlots / 1024;
  const int nrounds = (nslots + 1023) / 1024;
  int bk[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int s = r * 1024 + tid;
    const int id = load_clamped(ids, s, nslots);
    bk[r] = s < nslots ? bucket_of(id, e0, EL) : -1;
  }
  for (int i = tid; i < 2048; i += 1024) a[i] = mt[i] = 0;
  for (int i = tid; i < 16 * kPermSmallBuckets; i += 1024) (&wcnt[0][0])[i] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
    if (bk[r] >= 0) atomicAdd(&a[bk[r]], 1);
  __syncthreads();
  for (int b = tid; b < EL; b += 1024) {
    counts[b] = a[b];
    mt[b] = (a[b] + bm - 1) / bm;
  }
  __syncthreads();
  if (NB <= 64) {  // one wave scans both (entries past NB are zero and stay unused)
    if (wave == 0) {
      const int v = lane < NB ? a[lane] : 0, m = lane < NB ? mt[lane] : 0;
      const int iv = wave_inclusive_scan(v), im = wave_inclusive_scan(m);
      if (lane < NB) {
        a[lane] = iv - v;
        mt[lane] = im - m;
      }
    }
    __syncthreads();
  } else {
    block_exclusive_scan_2048(a);
    block_exclusive_scan_2048(mt);
  }
  for (int b = tid; b < NB; b += 1024) {
    offsets[b] = a[b];
    plan[b] = mt[b];
    base[b] = a[b];
  }
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) < NB) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    if (r >= nrounds) break;  // uniform
    const int s = r * 1024 + tid;
    const bool valid = bk[r] >= 0;
    const int b = valid ? bk[r] : 0;
    uint64_t match = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (b >> bit) & 1;
      const uint64_t m = __ballot(valid && on);
      match &= on ? m : ~m;
    }
    const int rank = __popcll(match & lt);
    const int cnt = __popcll(match);
    const bool leader = valid && rank == 0;
    if (leader) wcnt[wave][b] = cnt;
    __syncthreads();
    int pos = 0;
    if (valid) {
      pos = base[b] + rank;
      for (int q = 0; q < wave; ++q) pos += wcnt[q][b];
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&base[b], cnt);
      wcnt[wave][b] = 0;
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

// One workgroup, no atomics (up to 8192 slots, up to 63 local experts): the slots form
// chunks of 64 in slot order (round r of wave w is chunk 16 r + w).  Each wave ranks its
// slots among the equal buckets of its chunk with ballots and one lane per bucket stores
// the chunk's count; a wave per bucket turns the counts into exclusive prefixes over the
// chunks; one wave scans the bucket totals.  Position of a slot = bucket offset + prefix of
// its chunk + rank: stable by slot id.
__global__ __launch_bounds__(1024) void permute_tiny_kernel(const int32_t* __restrict__ ids, int nslots, int e0,
                                                            int EL, int bm, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ row_to_slot,
                                                            int32_t* __restrict__ slot_to_row,
                                                            int32_t* __restrict__ plan) {
  constexpr int kChunks = kPermTinySlots / 64;
  constexpr int kRounds = kPermTinySlots / 1024;
  __shared__ int cnt[kPermTinyBuckets][kChunks];  // [bucket][chunk]: count, then prefix
  __shared__ int base[kPermTinyBuckets];
  const int NB = EL + 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nrounds = (nslots + 1023) / 1024, nchunks = (nslots + 63) / 64;
  int bk[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int s = r * 1024 + tid;
    const int id = load_clamped(ids, s, nslots);
    bk[r] = s < nslots ? bucket_of(id, e0, EL) : -1;
  }
  for (int i = tid; i < kPermTinyBuckets * kChunks; i += 1024) (&cnt[0][0])[i] = 0;
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) < NB) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  int rank[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    rank[r] = 0;
    if (r >= nrounds) continue;  // uniform
    const bool valid = bk[r] >= 0;
    const int b = valid ? bk[r] : 0;
    uint64_t match = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (b >> bit) & 1;
      const uint64_t m = __ballot(valid && on);
      match &= on ? m : ~m;
    }
    rank[r] = __popcll(match & lt);
    if (valid && rank[r] == 0) cnt[b][r * 16 + wave] = __popcll(match);
  }
  __syncthreads();
  for (int b = wave; b < NB; b += 16) {
    int carry = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {  // uniform
      const int c = c0 + lane;
      const int v = c < nchunks ? cnt[b][c] : 0;
      const int inc = wave_inclusive_scan_dpp(v);
      if (c < nchunks) cnt[b][c] = carry + inc - v;
      carry += __builtin_amdgcn_readlane(inc, 63);
    }
    if (lane == 0) base[b] = carry;  // bucket total
  }
  __syncthreads();
  if (wave == 0) {
    const int v = lane < NB ? base[lane] : 0;
    const int m = lane < EL ? (v + bm - 1) / bm : 0;  // m-tiles of this expert
    const int iv = wave_inclusive_scan_dpp(v), im = wave_inclusive_scan_dpp(m);
    if (lane < NB) {
      offsets[lane] = iv - v;
      plan[lane] = im - m;
      base[lane] = iv - v;
    }
    if (lane < EL) counts[lane] = v;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    if (r >= nrounds) break;  // uniform
    const int b = bk[r];
    if (b < 0) continue;
    const int s = r * 1024 + tid;
    const int pos = base[b] + cnt[b][r * 16 + wave] + rank[r];
    row_to_slot[pos] = b < EL ? s : -1;
    slot_to_row[s] = b < EL ? pos : -1;
  }
}

// Stable scatter of one chunk (kPermChunk slots) for up to 63 local experts, without
// per-round barriers: every wave ranks its slots of all kPermChunk / 256 rounds by ballot
// matching (sub-chunk 4 r + w holds the chunk's slots [256 r + 64 w, + 64), so sub-chunks are
// in slot order),
// one wave per bucket turns the sub-chunk counts into exclusive prefixes, and each slot's
// position is offset + the chunk's base + the prefix of its sub-chunk + its rank.
__global__ __launch_bounds__(256) void permute_scatter64_kernel(const int32_t* __restrict__ ids, int nslots, int e0,
                                                                int EL, const int32_t* __restrict__ chunk_base,
                                                                const int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ row_to_slot,
                                                                int32_t* __restrict__ slot_to_row) {
  constexpr int kRounds = kPermChunk / 256;
  constexpr int kSub = kRounds * 4;  // sub-chunks of 64 slots (one per wave and round)
  static_assert(kSub <= 64 && kPermChunk % 256 == 0, "one lane per sub-chunk in the prefix");
  __shared__ int sc[kPermTinyBuckets][kSub];  // [bucket][sub-chunk]: count, then prefix
  __shared__ int base[kPermTinyBuckets];
  const int NB = EL + 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int first = blockIdx.x * kPermChunk;
  for (int i = tid; i < kPermTinyBuckets * kSub; i += 256) (&sc[0][0])[i] = 0;
  for (int b = tid; b < NB; b += 256) base[b] = offsets[b] + chunk_base[(size_t)blockIdx.x * NB + b];
  int bk[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int s = first + r * 256 + tid;
    const int id = load_clamped(ids, s, nslots);
    bk[r] = s < nslots ? bucket_of(id, e0, EL) : -1;
  }
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) < NB) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  int rank[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const bool valid = bk[r] >= 0;
    const int b = valid ? bk[r] : 0;
    uint64_t match = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (b >> bit) & 1;
      const uint64_t m = __ballot(valid && on);
      match &= on ? m : ~m;
    }
    rank[r] = __popcll(match & lt);
    if (valid && rank[r] == 0) sc[b][r * 4 + wave] = __popcll(match);
  }
  __syncthreads();
  for (int b = wave; b < NB; b += 4) {
    const int v = lane < kSub ? sc[b][lane] : 0;
    const int ex = wave_inclusive_scan_dpp(v) - v;
    if (lane < kSub) sc[b][lane] = ex;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int b = bk[r];
    if (b < 0) continue;
    const int s = first + r * 256 + tid;
    const int pos = base[b] + sc[b][r * 4 + wave] + rank[r];
    row_to_slot[pos] = b < EL ? s : -1;
    slot_to_row[s] = b < EL ? pos : -1;
  }
}

hipError_t launch_permute(const int32_t* ids, int nslots, int e0, int EL, int32_t* chunk_cnt, int32_t* chunk_base,
                          int32_t* counts, int32_t* offsets, int32_t* row_to_slot, int32_t* slot_to_row, int bm,
                          int32_t* plan, hipStream_t s) {
  const int NB = EL + 1;
  if (nslots <= kPermTinySlots && NB <= kPermTinyBuckets) {
    permute_tiny_kernel<<<1, 1024, 0, s>>>(ids, nslots, e0, EL, bm, counts, offsets, row_to_slot, slot_to_row, plan);
    return hipGetLastError();
  }
  if (nslots <= kPermSmallSlots && NB <= kPermSmallBuckets) {
    permute_small_kernel<<<1, 1024, 0, s>>>(ids, nslots, e0, EL, bm, counts, offsets, row_to_slot, slot_to_row, plan);
    return hipGetLastError();
  }
  const int nchunks = (nslots + kPermChunk - 1) / kPermChunk;
  if (nchunks > 0) {
    permute_hist_kernel<<<nchunks, 256, NB * sizeof(int), s>>>(ids, nslots, e0, EL, chunk_cnt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  permute_scan_kernel<<<1, 1024, 0, s>>>(chunk_cnt, nchunks, EL, bm, chunk_base, counts, offsets, plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nchunks == 0) return e;
  if (NB <= kPermTinyBuckets) {
    permute_scatter64_kernel<<<nchunks, 256, 0, s>>>(ids, nslots, e0, EL, chunk_base, offsets, row_to_slot,
                                                      slot_to_row);
    return hipGetLastError();
  }
  permute_scatter_kernel<<<nchunks, 256, 5 * NB * sizeof(int), s>>>(ids, nslots, e0, EL, chunk_base, offsets,
                                                                     row_to_slot, slot_to_row);
  return hipGetLastError();
}

}  // namespace moe
