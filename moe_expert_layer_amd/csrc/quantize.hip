// Input quantisation: bf16 activations -> FP8 E4M3 with one UE8M0 scale per 128 consecutive
// values of a row.  Source: "DSV4 o_proj: fuse fp8/UE8M0 quantize into o_a proj"
// (Description: FP8 E4M3 with 1x128 UE8M0 scales from an amax per block).  The scale rule
// is the one the FC1 epilogue uses for the intermediate: the smallest 2^e with
// 448 * 2^e >= amax (byte e + 127, clamped to [0, 254]; 127 for an all-zero block), codes
// E4M3 round-to-nearest-even of v * 2^-e.  bf16 values are exact in fp32 and the scaling is
// by a power of two, so the result is fully determined.
//
// A thread takes 8 consecutive values (one 16-byte load); the 16 lanes of a DPP row hold one
// 128-value block, so the block amax is a 4-step DPP max and every lane has the scale.
// HBM-bound: 2 bytes read and 1 + 1/128 bytes written per value.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

#include "device_common.hpp"
#include "moe_internal.hpp"

namespace moe {

template <int CTRL>
__device__ __forceinline__ uint32_t umax_dpp(uint32_t m) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, CTRL, 0xf, 0xf, false);
  return m > o ? m : o;
}

__global__ __launch_bounds__(256) void quantize_act_kernel(const uint4* __restrict__ x, long long n8,
                                                           uint2* __restrict__ q, uint8_t* __restrict__ sf) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // group of 8 values
  // n8 is a multiple of 16, so the 16 lanes of a DPP row leave together
  if (i >= n8) return;
  const uint4 v = x[i];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // value 2j in the low half of word j
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
  uint32_t m = 0;  // amax as an unsigned max of the non-negative float bits
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t a = __float_as_uint(f[j]) & 0x7fffffffu;
    m = m > a ? m : a;
  }
  m = umax_dpp<0xB1>(m);   // quad_perm [1,0,3,2]
  m = umax_dpp<0x4E>(m);   // quad_perm [2,3,0,1]
  m = umax_dpp<0x124>(m);  // row_ror 4
  m = umax_dpp<0x128>(m);  // row_ror 8
  const int byte = ue8m0_for_amax(__uint_as_float(m));
  const float inv = inv_scale_of(byte);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] * inv, f[1] * inv, 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] * inv, f[3] * inv, lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4] * inv, f[5] * inv, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6] * inv, f[7] * inv, hi, true);
  q[i] = make_uint2((uint32_t)lo, (uint32_t)hi);
  if ((threadIdx.x & 15) == 0) sf[i >> 4] = (uint8_t)byte;
}

hipError_t launch_quantize_act(const uint16_t* x_bf16, long long n, uint8_t* x, uint8_t* x_sf, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const long long n8 = n / 8;
  const long long blocks = (n8 + 255) / 256;
  quantize_act_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(reinterpret_cast<const uint4*>(x_bf16), n8,
                                                              reinterpret_cast<uint2*>(x), x_sf);
  return hipGetLastError();
}

// Packed UE8M0 scales ("DSV4 o_proj: fuse fp8/UE8M0 quantize into o_a proj": the o_a
// FP8-output tactic checks an int32 scale tensor of shape (M, ceil(G/4)) with MN-major
// stride (1, aligned_M), aligned_M = M rounded up to 4, padding zeroed).  Word (m, j) sits at
// j * aligned_M + m and holds groups 4j .. 4j+3 of row m, group 4j + b in byte b.
// One thread per word: consecutive threads write consecutive words.
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ sf, int M, int G, int AM,
                                                          long long nwords, uint32_t* __restrict__ packed) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
  if (q >= nwords) return;
  const int j = (int)(q / AM), m = (int)(q - (long long)j * AM);
  uint32_t w = 0;
  if (m < M) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (4 * j + b < G) w |= (uint32_t)sf[(long long)m * G + 4 * j + b] << (8 * b);
  }
  packed[q] = w;
}

__global__ __launch_bounds__(256) void unpack_scales_kernel(const uint32_t* __restrict__ packed, int M, int G, int AM,
                                                            long long nwords, uint8_t* __restrict__ sf) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
  if (q >= nwords) return;
  const int j = (int)(q / AM), m = (int)(q - (long long)j * AM);
  if (m >= M) return;
  const uint32_t w = packed[q];
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if (4 * j + b < G) sf[(long long)m * G + 4 * j + b] = (uint8_t)(w >> (8 * b));
}

hipError_t launch_pack_scales(const uint8_t* sf, int M, int G, int32_t* packed, hipStream_t s) {
  const int AM = (M + 3) / 4 * 4;
  const long long nwords = (long long)((G + 3) / 4) * AM;
  if (nwords == 0) return hipSuccess;
  pack_scales_kernel<<<dim3((unsigned)((nwords + 255) / 256)), 256, 0, s>>>(sf, M, G, AM, nwords,
                                                                             reinterpret_cast<uint32_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_unpack_scales(const int32_t* packed, int M, int G, uint8_t* sf, hipStream_t s) {
  const int AM = (M + 3) / 4 * 4;
  const long long nwords = (long long)((G + 3) / 4) * AM;
  if (nwords == 0 || M == 0) return hipSuccess;
  unpack_scales_kernel<<<dim3((unsigned)((nwords + 255) / 256)), 256, 0, s>>>(
      reinterpret_cast<const uint32_t*>(packed), M, G, AM, nwords, sf);
  return hipGetLastError();
}

}  // namespace moe
