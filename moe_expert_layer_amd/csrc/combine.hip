// Top-k weighted combine back into token order, without atomics.
//
// y[t] = bf16( sum over local slots j = 0..k-1, in slot order, of w[t, j] * Y2[row(t, j)] )
// accumulated in fp32 from 0 and rounded once to bfloat16; tokens with no local slot
// get +0.  Sources: "Pull Style Cutedsl Megakernel" (Layout: the top-k reduce after
// the fused FC1/FC2 schedule) and "Optimize sm100 version with token-aware BM240
// tiling, native UE8M0, and direct combine" (description: combine into token order).
// One workgroup per token; every output element is written by exactly one thread, so
// the result does not depend on scheduling.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "device_common.hpp"
#include "moe_internal.hpp"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y2, const int32_t* __restrict__ s2r,
                                                      const float* __restrict__ w, int H, int k,
                                                      uint16_t* __restrict__ y) {
  __shared__ int rows[kMaxTopk];
  __shared__ float wt[kMaxTopk];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = s2r[(long long)t * k + threadIdx.x];
    wt[threadIdx.x] = w[(long long)t * k + threadIdx.x];
  }
  __syncthreads();
  uint16_t* yt = y + (long long)t * H;
  for (int c = threadIdx.x * 4; c < H; c += 256 * 4) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = rows[j];
      if (r >= 0) {
        const float4 v = *reinterpret_cast<const float4*>(y2 + (long long)r * H + c);
        const float ww = wt[j];
        a0 = fmaf(ww, v.x, a0);
        a1 = fmaf(ww, v.y, a1);
        a2 = fmaf(ww, v.z, a2);
        a3 = fmaf(ww, v.w, a3);
      }
    }
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(a2) | ((uint32_t)f32_to_bf16_rne(a3) << 16);
    *reinterpret_cast<uint2*>(yt + c) = make_uint2(lo, hi);
  }
}

hipError_t launch_combine(const float* y2, const int32_t* slot_to_row, const float* topk_w, int T, int H, int k,
                          uint16_t* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  combine_kernel<<<T, 256, 0, s>>>(y2, slot_to_row, topk_w, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
