// Device helpers shared by the HIP kernels of the MoE expert layer (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// Inclusive sum over the wave with DPP: shifts by 1, 2, 4, 8 inside each 16-lane row
// (lanes whose source is outside the row add 0), then the last lane of row 0 and row 2 is
// added to rows 1 and 3 (row_bcast:15) and the last lane of row 1 to rows 2 and 3
// (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return v;
}

// Exclusive scan of a[0..2048) (in LDS) by a 1024-thread workgroup; a[] must be
// complete and visible (barrier) on entry.  Ends with a barrier.
__device__ __forceinline__ void block_exclusive_scan_2048(int* a) {
  __shared__ int wsum[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int x0 = a[2 * t], x1 = a[2 * t + 1];
  const int inc = wave_inclusive_scan(x0 + x1);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int v = lane < 16 ? wsum[lane] : 0;
    const int vi = wave_inclusive_scan(v);
    if (lane < 16) wsum[lane] = vi - v;
  }
  __syncthreads();
  const int excl = inc - (x0 + x1) + wsum[wave];
  a[2 * t] = excl;
  a[2 * t + 1] = excl + x0;
  __syncthreads();
}

// float32 -> bfloat16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7f800000u) == 0x7f800000u) return (uint16_t)((b >> 16) | ((b & 0xffffu) ? 0x40u : 0u));
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// UE8M0 byte of the 1x128 requant: smallest e with 448 * 2^e >= amax, byte = e + 127
// clamped to [0, 254]; 127 for amax = 0.  Exact, from the fp32 bits of amax:
// amax = 1.m * 2^(E-127) and 448 = 1.75 * 2^8, so e = E - 135 when 1.m <= 1.75
// (mantissa field <= 0x600000) and E - 134 otherwise.
__device__ __forceinline__ int ue8m0_for_amax(float amax) {
  const uint32_t b = __float_as_uint(amax);
  if (b == 0u) return 127;
  const int E = (int)(b >> 23);
  const int m = (int)(b & 0x7fffff);
  int byte = E - 8 + (m > 0x600000 ? 1 : 0);
  byte = byte < 0 ? 0 : (byte > 254 ? 254 : byte);
  return byte;
}

// 2^(127 - byte) as fp32 for byte in [1, 254]; byte 0 gives 2^127.
__device__ __forceinline__ float inv_scale_of(int byte) {
  return __uint_as_float((uint32_t)(254 - byte) << 23);
}

// logistic function 1 / (1 + e^-z) from the hardware base-2 exponential and reciprocal
// (a few ulp; the result is requantised to E4M3 right after)
__device__ __forceinline__ float sigmoidf_(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

}  // namespace moe
