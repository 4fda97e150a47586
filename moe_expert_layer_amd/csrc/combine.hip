// Top-k weighted combine back into token order, without atomics.
//
// y[t] = bf16( sum over local slots j = 0..k-1, in slot order, of w[t, j] * Y2[row(t, j)]
//             + sum over shared experts s = 0..S-1 of Y2[R + s T + t] )
// accumulated in fp32 from 0 and rounded once to bfloat16; without shared experts, tokens
// with no local slot get +0.  Sources: "Pull Style Cutedsl Megakernel" (Layout: the top-k reduce after
// the fused FC1/FC2 schedule) and "Optimize sm100 version with token-aware BM240
// tiling, native UE8M0, and direct combine" (description: combine into token order).
// Every output element is written by exactly one thread, so the result does not depend
// on scheduling.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "device_common.hpp"
#include "moe_internal.hpp"

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream(const float* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// grid (ceil(H / 2048), min(T, 65535)): a workgroup owns 2048 columns of one token at a time
// (tokens strided by the grid height); thread i handles columns 4i.. and 1024 + 4i.., so each
// load instruction of the workgroup reads 4 KB of one Y2 row.  The token's slots are taken in
// batches of four whose row loads are all issued before the in-order accumulation.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y2, const int32_t* __restrict__ s2r,
                                                      const float* __restrict__ w, int T, int H, int k,
                                                      const int32_t* __restrict__ r_total, int S,
                                                      uint16_t* __restrict__ y) {
  const int c0 = blockIdx.x * 2048 + threadIdx.x * 4;
  if (c0 >= H) return;
  const bool two = c0 + 1024 < H;
  const int R = S > 0 ? *r_total : 0;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += 4) {
      int rows[4];
      float wt[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {  // slots in slot order; -1 = not local
        const int j = j0 + jj;
        rows[jj] = j < k ? s2r[(long long)t * k + j] : -1;
        wt[jj] = rows[jj] >= 0 ? w[(long long)t * k + j] : 0.f;
      }
      float4 v0[4], v1[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (rows[jj] >= 0) {
          const float* src = y2 + (long long)rows[jj] * H + c0;
          v0[jj] = ld_stream(src);  // Y2 is read once
          if (two) v1[jj] = ld_stream(src + 1024);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (rows[jj] >= 0) {
          acc[0] = fmaf(wt[jj], v0[jj].x, acc[0]);
          acc[1] = fmaf(wt[jj], v0[jj].y, acc[1]);
          acc[2] = fmaf(wt[jj], v0[jj].z, acc[2]);
          acc[3] = fmaf(wt[jj], v0[jj].w, acc[3]);
          if (two) {
            acc[4] = fmaf(wt[jj], v1[jj].x, acc[4]);
            acc[5] = fmaf(wt[jj], v1[jj].y, acc[5]);
            acc[6] = fmaf(wt[jj], v1[jj].z, acc[6]);
            acc[7] = fmaf(wt[jj], v1[jj].w, acc[7]);
          }
        }
      }
    }
    for (int s = 0; s < S; ++s) {  // shared experts, weight 1
      const float* src = y2 + ((long long)R + (long long)s * T + t) * H + c0;
      const float4 a = ld_stream(src);
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      if (two) {
        const float4 b = ld_stream(src + 1024);
        acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
      }
    }
    uint16_t* dst = y + (long long)t * H + c0;
    *reinterpret_cast<uint2*>(dst) =
        make_uint2((uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16),
                   (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16));
    if (two)
      *reinterpret_cast<uint2*>(dst + 1024) =
          make_uint2((uint32_t)f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16),
                     (uint32_t)f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16));
  }
}

hipError_t launch_combine(const float* y2, const int32_t* slot_to_row, const float* topk_w, int T, int H, int k,
                          const int32_t* r_total, int S, uint16_t* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  combine_kernel<<<dim3((H + 2047) / 2048, T < 65535 ? T : 65535), 256, 0, s>>>(y2, slot_to_row, topk_w, T, H, k,
                                                                                r_total, S, y);
  return hipGetLastError();
}

}  // namespace moe
