// Measurement probes (not part of the layer): matrix-instruction accumulation precision,
// matrix-core rate and HBM read bandwidth on gfx950.  The C interface and its conventions
// are in include/moe_probes.h.
//
// Operand layouts used here (gfx950):
//   scaled 32x32x64 FP8: lane l holds row l%32, K bytes [16*(l/32), +16) and [32 + 16*(l/32), +16)
//     of the 64-wide step; FP4: K elements [32*(l/32), +32) in its first 16 bytes; result lane l,
//     value i is row 8*(i/4) + 4*(l/32) + i%4, column l%32.
//   scaled 16x16x128 FP8: lane l holds row l%16, K bytes [16*(l/16), +16) and [64 + 16*(l/16), +16)
//     of the 128-wide step; FP4: K elements [32*(l/16), +32); result lane l, value i is row
//     4*(l/16) + i, column l%16.
//   32x32x16 FP8 and BF16: lane l holds row l%32, K values [8*(l/32), +8) of the 16-wide step.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "../../include/moe_probes.h"

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

__device__ __forceinline__ v8i pair16(uint4 lo, uint4 hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// E2M1 nibble -> float (OCP MX: sign, 2 exponent bits with bias 1, 1 mantissa bit)
__device__ __forceinline__ float e2m1(uint32_t nib) {
  const uint32_t e = (nib >> 1) & 3u, m = nib & 1u;
  const float mag = e == 0 ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (e - 1));
  return (nib & 8u) ? -mag : mag;
}

// 8 consecutive K values of a row as BF16 (exact conversions: E4M3 and E2M1 fit BF16)
__device__ __forceinline__ bf16x8 bf16_of_fp8(uint2 v) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
__device__ __forceinline__ bf16x8 bf16_of_fp4(uint32_t v) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// result of a 32x32 instruction form: lane l, value i -> row 8*(i/4) + 4*(l/32) + i%4, column l%32
__device__ __forceinline__ void store32(float* c, const v16f& acc, int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) c[(8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)) * 32 + (lane & 31)] = acc[i];
}

template <int BF4>
__global__ __launch_bounds__(64) void probe_gemm_kernel(int form, int K, const uint8_t* __restrict__ a,
                                                        const uint8_t* __restrict__ b, float* __restrict__ c) {
  constexpr bool b_fp4 = BF4 != 0;
  const int p = blockIdx.x, lane = threadIdx.x;
  const int bK = b_fp4 ? K / 2 : K;  // bytes per B row
  const uint8_t* A = a + (long long)p * 32 * K;
  const uint8_t* Bm = b + (long long)p * 32 * bK;
  float* C = c + (long long)p * 1024;
  constexpr int bcode = BF4 ? 4 : 0;  // B operand format of the scaled instructions: E4M3 0, E2M1 4

  if (form == MOE_PROBE_SCALED_32X32X64 || form == MOE_PROBE_SCALED_32X32X64_SPLIT) {
    const int r = lane & 31, kb = lane >> 5;
    v16f acc = {};
    for (int s = 0; s < K / 64; ++s) {
      const uint8_t* ar = A + r * K + 64 * s;
      const v8i av = pair16(ld16(ar + 16 * kb), ld16(ar + 32 + 16 * kb));
      v8i bv;
      if (b_fp4) {
        const uint4 q = ld16(Bm + r * bK + 32 * s + 16 * kb);
        bv = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      } else {
        const uint8_t* br = Bm + r * bK + 64 * s;
        bv = pair16(ld16(br + 16 * kb), ld16(br + 32 + 16 * kb));
      }
      if (form == MOE_PROBE_SCALED_32X32X64) {
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, bcode, 0, 127, 0, 127);
      } else {
        const v16f zero = {};
        const v16f t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, zero, 0, bcode, 0, 127, 0, 127);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += t[i];
      }
    }
    store32(C, acc, lane);
  } else if (form == MOE_PROBE_SCALED_16X16X128) {
    const int r = lane & 15, kb = lane >> 4;
#pragma unroll
    for (int qm = 0; qm < 2; ++qm)
#pragma unroll
      for (int qn = 0; qn < 2; ++qn) {
        v4f acc = {};
        for (int s = 0; s < K / 128; ++s) {
          const uint8_t* ar = A + (16 * qm + r) * K + 128 * s;
          const v8i av = pair16(ld16(ar + 16 * kb), ld16(ar + 64 + 16 * kb));
          v8i bv;
          if (b_fp4) {
            const uint4 q = ld16(Bm + (16 * qn + r) * bK + 64 * s + 16 * kb);
            bv = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
          } else {
            const uint8_t* br = Bm + (16 * qn + r) * bK + 128 * s;
            bv = pair16(ld16(br + 16 * kb), ld16(br + 64 + 16 * kb));
          }
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, bcode, 0, 127, 0, 127);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) C[(16 * qm + 4 * (lane >> 4) + i) * 32 + 16 * qn + (lane & 15)] = acc[i];
      }
  } else if (form == MOE_PROBE_FP8_32X32X16) {
    const int r = lane & 31, kb = lane >> 5;
    v16f acc = {};
    for (int s = 0; s < K / 16; ++s) {
      const uint2 av = ld8(A + r * K + 16 * s + 8 * kb);
      const uint2 bv = ld8(Bm + r * bK + 16 * s + 8 * kb);
      const long al = (long)(((uint64_t)av.y << 32) | av.x), bl = (long)(((uint64_t)bv.y << 32) | bv.x);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(al, bl, acc, 0, 0, 0);
    }
    store32(C, acc, lane);
  } else if (form == MOE_PROBE_BF16_32X32X16) {
    const int r = lane & 31, kb = lane >> 5;
    v16f acc = {};
    for (int s = 0; s < K / 16; ++s) {
      const bf16x8 av = bf16_of_fp8(ld8(A + r * K + 16 * s + 8 * kb));
      const bf16x8 bv = b_fp4 ? bf16_of_fp4(ld4(Bm + r * bK + 8 * s + 4 * kb))
                              : bf16_of_fp8(ld8(Bm + r * bK + 16 * s + 8 * kb));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    }
    store32(C, acc, lane);
  } else if (form == MOE_PROBE_FP32_FMA) {
    for (int e = lane; e < 1024; e += 64) {
      const int m = e >> 5, j = e & 31;
      float acc = 0.f;
      for (int k = 0; k < K; ++k) {
        const float av = __builtin_amdgcn_cvt_f32_fp8((int)A[m * K + k], 0);
        const float bv = b_fp4 ? e2m1((Bm[j * bK + k / 2] >> (4 * (k & 1))) & 15u)
                               : __builtin_amdgcn_cvt_f32_fp8((int)Bm[j * bK + k], 0);
        acc = fmaf(av, bv, acc);
      }
      C[e] = acc;
    }
  }
}

// Four independent accumulators per wave, operands in registers: the instruction issue rate
// is the only limit.  The operand bytes are finite FP8 / FP4 values that differ per lane.
template <int BF4>
__global__ __launch_bounds__(256) void probe_mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int pat = 0x38383838 ^ ((lane & 7) * 0x01010101);  // E4M3 values near 1
  const v8i av = v8i{pat, pat, pat, pat, pat, pat, pat, pat};
  const int fp4pat = 0x22222222 ^ ((lane & 3) * 0x11111111);
  const v8i bv = BF4 ? v8i{fp4pat, fp4pat, fp4pat, fp4pat, 0, 0, 0, 0} : av;
  constexpr int bcode = BF4 ? 4 : 0;
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c0, 0, bcode, 0, 120, 0, 120);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c1, 0, bcode, 0, 120, 0, 120);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c2, 0, bcode, 0, 120, 0, 120);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c3, 0, bcode, 0, 120, 0, 120);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[(long long)blockIdx.x * 256 + threadIdx.x] = s;
}

typedef int v4i_ __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_hbm_read_kernel(const v4i_* __restrict__ src, long long n16,
                                                             float* __restrict__ sink) {
  const long long stride = (long long)gridDim.x * 256;
  int acc = 0;
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {  // four loads in flight per thread
    const v4i_ v0 = __builtin_nontemporal_load(src + i);
    const v4i_ v1 = __builtin_nontemporal_load(src + i + stride);
    const v4i_ v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4i_ v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w ^ v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^
           v3.w;
  }
  for (; i < n16; i += stride) {
    const v4i_ v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(long long)blockIdx.x * 256 + threadIdx.x] = (float)(acc & 0xffff);
}

// direct global-to-LDS load of 16 bytes per lane: LDS address M0 + 16 * lane.  The base sits in
// SGPRs (readfirstlane); a VMEM instruction that reads an SGPR written by a VALU instruction
// needs 5 wait states in between, which the asm provides (s_mov + s_nop 3; this also covers
// the wait between writing M0 and the load that reads it)
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint32_t lds) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const void* b = reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(b), "s"(lds)
               : "memory", "m0");
}

// 64 KB stage t of the panel (bytes [128 (t mod K/128), +128) of its 512 rows) into ring slot
// t % 2: wave w issues 8 loads, load j covering rows 64 w + 8 j .. +8 (8 lanes of 16 bytes a row)
template <int DEPTH>
__global__ __launch_bounds__(512) void probe_dma_stream_kernel(const uint8_t* __restrict__ src, int K, int panels,
                                                               int passes, float* __restrict__ sink) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t ring[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int panel = panels ? (int)(blockIdx.x % panels) : (int)blockIdx.x;
  const uint8_t* base = src + (size_t)panel * 512 * (size_t)K;
  uint32_t off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) off[j] = (uint32_t)((wave * 64 + j * 8 + (lane >> 3)) * K + (lane & 7) * 16);
  const uint32_t ring0 = (uint32_t)(uintptr_t)ring;
  const int nk = K / 128, total = passes * nk;
  auto issue = [&](int t) {
    const uint8_t* b = base + (size_t)(t % nk) * 128;
    const uint32_t st = ring0 + (uint32_t)((t & 1) * 65536 + wave * 8192);
#pragma unroll
    for (int j = 0; j < 8; ++j) dma16(b, off[j], __builtin_amdgcn_readfirstlane(st + j * 1024));
  };
  issue(0);
  if (DEPTH == 2 && total > 1) issue(1);
  for (int t = 0; t < total; ++t) {
    if (DEPTH == 1) {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // stage t landed everywhere
      if (t + 1 < total) issue(t + 1);
    } else {
      if (t + 1 < total) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");  // t landed, t + 1 in flight
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (t + 2 < total) issue(t + 2);  // into the slot of stage t, taken as consumed
    }
  }
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  sink[(size_t)blockIdx.x * 512 + threadIdx.x] = (float)ring[(threadIdx.x * 131) & 131071];
}

// value i of the output: code i (E4M3, E5M2 or E2M1) converted to BF16 with the scale
// 2^(scale_bytes[i / 32] - 127) passed to the conversion instruction as the float whose bits are
// scale_byte << 23 (2^-127 as the denormal 0x00400000 for byte 0)
__global__ __launch_bounds__(256) void probe_cvt_kernel(int fmt, int n, const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ sbytes, uint16_t* __restrict__ out) {
  const int i = (blockIdx.x * 256 + threadIdx.x) * 2;  // two values per thread
  if (i >= n) return;
  const uint32_t sb = sbytes[i / 32];
  const float sc = __uint_as_float(sb == 0 ? 0x00400000u : sb << 23);
  bf16x2 r;
  if (fmt == 2) {  // E2M1: values i, i+1 are the two nibbles of byte i/2
    r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((uint32_t)codes[i / 2], sc, 0);
  } else {
    const uint32_t v = (uint32_t)codes[i] | ((uint32_t)codes[i + 1] << 8);
    r = fmt == 1 ? __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(v, sc, false)
                 : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, sc, false);
  }
  *reinterpret_cast<uint32_t*>(out + i) = __builtin_bit_cast(uint32_t, r);  // i even: value i in the low half
}

}  // namespace

extern "C" {

int moe_probe_cvt_bf16(int fmt, int n, const uint8_t* codes, const uint8_t* scale_bytes, uint16_t* out, void* stream) {
  if (fmt < 0 || fmt > 2 || n < 2 || n % 32 || n > (1 << 28) || !codes || !scale_bytes || !out) return -1;
  probe_cvt_kernel<<<dim3((n / 2 + 255) / 256), 256, 0, (hipStream_t)stream>>>(fmt, n, codes, scale_bytes, out);
  return (int)hipGetLastError();
}


int moe_probe_mfma_gemm(int form, int n, int K, int b_fp4, const uint8_t* a, const uint8_t* b, float* c,
                        void* stream) {
  if (form < 0 || form > 5 || n < 1 || n > 65535 || K < 128 || K % 128 || !a || !b || !c) return -1;
  if (b_fp4 && form == MOE_PROBE_FP8_32X32X16) return -1;
  if (b_fp4) probe_gemm_kernel<1><<<dim3(n), 64, 0, (hipStream_t)stream>>>(form, K, a, b, c);
  else probe_gemm_kernel<0><<<dim3(n), 64, 0, (hipStream_t)stream>>>(form, K, a, b, c);
  return (int)hipGetLastError();
}

int moe_probe_mfma_loop(int blocks, int iters, int b_fp4, float* sink, void* stream) {
  if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 20) || !sink) return -1;
  if (b_fp4) probe_mfma_loop_kernel<1><<<dim3(blocks), 256, 0, (hipStream_t)stream>>>(iters, sink);
  else probe_mfma_loop_kernel<0><<<dim3(blocks), 256, 0, (hipStream_t)stream>>>(iters, sink);
  return (int)hipGetLastError();
}

int moe_probe_hbm_read(const void* src, size_t bytes, int blocks, float* sink, void* stream) {
  if (blocks < 1 || blocks > (1 << 20) || bytes % 16 || !src || !sink) return -1;
  probe_hbm_read_kernel<<<dim3(blocks), 256, 0, (hipStream_t)stream>>>(reinterpret_cast<const v4i_*>(src),
                                                                         (long long)(bytes / 16), sink);
  return (int)hipGetLastError();
}

int moe_probe_dma_stream(const void* src, size_t src_bytes, int K, int blocks, int panels, int passes, int depth,
                         float* sink, void* stream) {
  if (!src || !sink || K < 128 || K > 65536 || K % 128 || blocks < 1 || blocks > 65536 || panels < 0 ||
      panels > blocks || passes < 1 || passes > 65536 || (depth != 1 && depth != 2))
    return -1;
  if (src_bytes < (size_t)(panels ? panels : blocks) * 512 * (size_t)K) return -1;
  const int lds = 2 * 65536;
  hipError_t e = depth == 1 ? hipFuncSetAttribute((const void*)probe_dma_stream_kernel<1>,
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, lds)
                            : hipFuncSetAttribute((const void*)probe_dma_stream_kernel<2>,
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return (int)e;
  const uint8_t* s8 = reinterpret_cast<const uint8_t*>(src);
  if (depth == 1)
    probe_dma_stream_kernel<1><<<dim3(blocks), 512, lds, (hipStream_t)stream>>>(s8, K, panels, passes, sink);
  else
    probe_dma_stream_kernel<2><<<dim3(blocks), 512, lds, (hipStream_t)stream>>>(s8, K, panels, passes, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
