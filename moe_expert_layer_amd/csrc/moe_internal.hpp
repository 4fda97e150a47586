// Internal launch interface between the C-ABI host code and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 16;
constexpr int kMaxShared = 4;  // shared experts per layer
constexpr int kPermChunk = 1024;  // slots per permute workgroup (a multiple of 256, at most 4096)
constexpr int kPermTinySlots = 8192;    // at most this many slots and ...
constexpr int kPermTinyBuckets = 64;    // ... 63 local experts: the one-workgroup permute without atomics
constexpr int kPermSmallSlots = 16384;  // at most this many slots: one-workgroup permute
constexpr int kPermSmallBuckets = 257;  // ... and at most 256 local experts

struct Shape {
  int T, H, I, E, e0, EL, k;
  int wfmt;  // 0 E4M3 block-128, 1 mxfp4, 2 E5M2 block-128
  int S = 0;            // shared experts (weights after the EL routed ones)
  bool tensor = false;  // per-tensor float32 scales instead of UE8M0 blocks
  float h_scale = 1.f;  // per-tensor: static scale of the intermediate
  bool exact_fc1 = false;  // FC1 sums through BF16 MFMAs on operands converted in registers
  bool sf_packed = false;  // x_sf and h_sf are packed int32 MN-major (aligned rows T and T*(k+S))
  int act;   // 0 swiglu, 1 oai
  float clamp, alpha, bias;
};

// route + permute ----------------------------------------------------------
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);
// buckets: EL local experts + 1 trailing bucket for non-local slots.  Also writes the GEMM
// tile plan for tiles of `bm` rows (plan[e] = first m-tile of expert e, plan[EL] = all).
hipError_t launch_permute(const int32_t* ids, int nslots, int e0, int EL, int32_t* chunk_cnt, int32_t* chunk_base,
                          int32_t* counts, int32_t* offsets, int32_t* row_to_slot, int32_t* slot_to_row, int bm,
                          int32_t* plan, hipStream_t s);

// grouped GEMMs ------------------------------------------------------------
// Tile plan: plan[e] = first m-tile of local expert e, plan[EL] = number of m-tiles.
int gemm_block_m(int variant);
// largest contraction the GEMM kernels stage scales for (K / 128 <= 64)
bool gemm_supports(int H, int I);
size_t gemm_max_mtiles(int rows_cap, int EL, int variant, int T, int S);
// plan_ready: `plan` holds the tile plan of these offsets for this variant's tile rows (written
// by launch_permute); otherwise `plan` is ignored and every GEMM workgroup derives the plan
// from `offsets` in its prologue.
hipError_t launch_fc1(const Shape& sh, int variant, const uint8_t* x, const uint8_t* x_sf, const uint8_t* w1,
                      const uint8_t* w1_sf, const int32_t* offsets, const int32_t* row_to_slot, uint8_t* h,
                      uint8_t* h_sf, int32_t* plan, bool plan_ready, hipStream_t s);
hipError_t launch_fc2(const Shape& sh, int variant, const uint8_t* h, const uint8_t* h_sf, const uint8_t* w2,
                      const uint8_t* w2_sf, const int32_t* offsets, float* y2, int32_t* plan, bool plan_ready,
                      hipStream_t s);

// input quantisation --------------------------------------------------------
// n = T * H bf16 values (H % 128 == 0) -> E4M3 codes [n] and UE8M0 bytes [n / 128]
hipError_t launch_quantize_act(const uint16_t* x_bf16, long long n, uint8_t* x, uint8_t* x_sf, hipStream_t s);
// UE8M0 bytes [M, G] <-> packed int32 [ceil(G/4)][pad_up(M, 4)] (MN-major, padding zeroed)
hipError_t launch_pack_scales(const uint8_t* sf, int M, int G, int32_t* packed, hipStream_t s);
hipError_t launch_unpack_scales(const int32_t* packed, int M, int G, uint8_t* sf, hipStream_t s);

// combine --------------------------------------------------------------------
// r_total: device pointer to R (offsets[EL]); shared expert s's rows start at R + s T
hipError_t launch_combine(const float* y2, const int32_t* slot_to_row, const float* topk_w, int T, int H, int k,
                          const int32_t* r_total, int S, uint16_t* y, hipStream_t s);

}  // namespace moe
