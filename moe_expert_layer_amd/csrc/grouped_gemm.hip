// Grouped expert GEMMs on gfx950 scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), or BF16
// MFMA (v_mfma_f32_32x32x16_bf16) for the BF16 layer.
//
// FC1: for every row r of local expert e (token t = row_to_slot[r] / k)
//        g = x_t . W1[e, n],  u = x_t . W1[e, I + n]   (FP8 E4M3 x with 1x128 UE8M0 scales,
//        W1 FP8 E4M3 or E5M2 with 128x128 UE8M0 scales or MXFP4 with 1x32 UE8M0 scales;
//        per-tensor: one float32 scale for x and one per expert)
//      then SwiGLU / OAI-SwiGLU and the 1x128 requant to E4M3 + UE8M0 (fused epilogue;
//      per-tensor: E4M3 of h / h_scale, saturated; BF16 layer: h rounded to BF16).
// FC2: Y2[r, m] = h_r . W2[e, m]  (fp32 rows kept for the combine).
// Shared experts (applied to every token) follow the routed local experts: shared expert s
// owns rows [R + s T, R + (s + 1) T), row R + s T + t being token t.
//
// Sources: "fix(sm90): support parameterized SwiGLU in FP8 MegaMoE" (Summary: the two
// activation formulas, applied in the FC1 epilogue); "Optimize sm100 version with
// token-aware BM240 tiling, native UE8M0, and direct combine" (description: block
// scales consumed natively by the matrix unit); "DSV4 o_proj: fuse fp8/UE8M0 quantize
// into o_a proj" (Description: FP8 + 1x128 UE8M0 emitted from the GEMM epilogue with
// an amax reduction per block).
//
// The MFMA applies the scales: a 128-wide K step is two 32x32x64 instructions that share
// one activation scale per row and one FP8 weight scale per 128-row block; MXFP4 weights
// carry one scale per (row, 32-wide K block).
//
// Operand layout of the scaled 32x32x64 MFMA (measured on gfx950): lane l works on
// row/column l%32 and K half-block kb = l/32 of the 64-wide K block; an FP8 operand holds
// K bytes [16kb, +16) and [32 + 16kb, +16); an FP4 operand holds K elements [32kb, +32)
// (element 2i in the low nibble of byte i); lane l's scale byte covers row/column l%32
// and the 32-wide K block kb; result lane l holds rows 8*(i/4) + 4*(l/32) + i%4, column l%32.
// FC1 feeds the weights as the first operand and the tokens as the second, so a lane's
// results are one token row and runs of 4 consecutive h columns (the epilogue's amax and
// E4M3 packing then stay mostly inside the lane); FC2 keeps tokens first (row-contiguous
// Y2 stores).
//
// Tiles: BM rows x BN weight rows (FC1: BN = 256 = 128 gate + the matching 128 up rows,
// i.e. exactly one 1x128 requant block of h; FC2: BN output columns), in three variants
// chosen per call (launch_variant_w below): 256 rows (8 waves of 64 x 128; MXFP4 FC1: 4 waves
// of 128 x 128; FC2 on persistent workgroups), 128 rows (8 waves; FC2 128 columns wide) and
// 32 rows (4 waves of 32 x 64, the decode tile; its FC1 may sum exactly through BF16 MFMAs on
// operands converted in registers, XA).  K advances BK bytes per stage through a ring of
// NSTAGE LDS stages filled by direct global->LDS loads (global_load_lds_dwordx4): NSTAGE-1
// stages are in flight while one is consumed, and the loads take no registers.  The waits are
// explicit (s_waitcnt vmcnt + s_barrier).  LDS rows are 16-byte-chunk XOR swizzled so the
// operand reads are bank conflict free.  Workgroups map to tiles in an XCD-aware order (consecutive tiles of one
// expert on one XCD, sharing its L2).  Waves whose rows all lie past an expert's last row
// skip their MFMAs (decode-sized experts).
#include <hip/hip_runtime.h>
#include <atomic>
#include <cstdint>
#include <type_traits>

#include "device_common.hpp"
#include "moe_internal.hpp"

namespace moe {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// half q (16 bytes) of a lane's 32-byte operand fragment as 8 BF16 values
__device__ __forceinline__ bf16x8 bf16_half(const v8i& v, int q) {
  const v4i h = q == 0 ? __builtin_shufflevector(v, v, 0, 1, 2, 3) : __builtin_shufflevector(v, v, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, h);
}

// UE8M0 byte -> the float 2^(byte - 127) handed to the scaled conversions (2^-127 is the
// denormal 0x00400000)
__device__ __forceinline__ float scale_f32(int byte) {
  const uint32_t b = (uint32_t)byte & 0xffu;
  return __uint_as_float(b == 0 ? 0x00400000u : b << 23);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 join4(bf16x2 p0, bf16x2 p1, bf16x2 p2, bf16x2 p3) {
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
// group q (8 values, dwords 2q and 2q + 1) of a 32-byte FP8 fragment as BF16 values times sc;
// E4M3 and E5M2 values have at most 3 significant bits, so every conversion is exact
template <bool E5M2>
__device__ __forceinline__ bf16x8 fp8_group_bf16(const v8i& v, int q, float sc) {
  const uint32_t d0 = (uint32_t)v[2 * q], d1 = (uint32_t)v[2 * q + 1];
  if constexpr (E5M2)
    return join4(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, sc, false),
                 __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, sc, true),
                 __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, sc, false),
                 __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, sc, true));
  else
    return join4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, false),
                 __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, true),
                 __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, false),
                 __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, true));
}
// group q (8 values, dword q) of a 16-byte E2M1 fragment as BF16 values times sc
__device__ __forceinline__ bf16x8 fp4_group_bf16(const v8i& v, int q, float sc) {
  const uint32_t d = (uint32_t)v[q];
  return join4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 0), __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 1),
               __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 2), __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 3));
}

constexpr int kGroupN = 8;     // n-tiles per group in the tile order
constexpr int kMaxKSteps = 64; // K <= 8192 (scales of a tile are staged in LDS, one per 128-wide step)

// The tile's activation scales sit in LDS as [row][128-wide K step] bytes.  A row takes whole
// dwords, an odd number of them, so that the 32 rows a wave reads at once (one byte each) fall
// in 32 different banks; with the bare K / 128 bytes (16 or 56: an even number of dwords) rows
// 8 or 16 apart shared a bank.  The table is rounded up to whole 256-byte DMA instructions.
__host__ __device__ constexpr int asf_row_bytes(int nk128) { return nk128 ? ((((nk128 + 3) >> 2) | 1) << 2) : 0; }
__host__ __device__ constexpr int asf_table_bytes(int bm, int nk128) { return (bm * asf_row_bytes(nk128) + 255) & ~255; }

struct GemmArgs {
  const uint8_t* A;      // FC1: x [T, K]; FC2: h [cap, K]
  const uint8_t* A_sf;   // [rows, K/128]
  const int32_t* row_to_slot;
  const uint8_t* B;      // weights of all local experts
  const uint8_t* B_sf;
  const int32_t* offsets;
  const int32_t* plan;
  uint8_t* h;            // FC1 out
  uint8_t* h_sf;
  float* y2;             // FC2 out
  // packed int32 MN-major activation scales (0: row-major bytes): aligned row counts of the A
  // operand's scale tensor and of the FC1 output h_sf; the byte of (row, group g) is at
  // ((g / 4) * aligned + row) * 4 + g % 4
  int asf_am, hsf_am;
  long long b_estride;   // bytes per expert of B
  long long bsf_estride; // bytes per expert of B_sf
  int K;                 // contraction length (H for FC1, I for FC2)
  int N;                 // weight rows per expert (2I for FC1, H for FC2)
  int I;                 // intermediate size (FC1 epilogue)
  int k;                 // top-k (FC1 row -> token)
  int EL;                // routed local experts; shared experts EL .. EL + S - 1 follow them
  int S;                 // shared experts: each has the T rows [offsets[EL] + s T, + T), one per token
  int T;
  int n_tiles;
  int act;
  float clamp, alpha, bias;
  // per-tensor scaling: the MFMAs run with unit scales and the accumulators are multiplied
  // by (x scale or h_scale) * the expert's weight scale; FC1 quantises h with h_inv = 1 / h_scale
  int tensor;
  const float* a_tscale;  // FC1: x scale [1]
  const float* b_tscale;  // weight scale per local expert [EL]
  float h_scale, h_inv;
};

// Tile shape: BM rows x BN weight rows, K advancing BK per stage through an NSTAGE ring,
// NW waves arranged (BM/WTM) x WN, each wave WTM rows x BN/WN weight rows.  PIPE 0: a stage's
// fragments are read, then multiplied; PIPE 2: the half-step pipeline (the fragments of the
// next 64-wide half of a stage are read from LDS while the MFMAs of the current half run).
template <int MODE, int WFMT, int BM, int BN, int BK, int NSTAGE, int NW, int WTM, int PIPE>
struct Cfg {
  static constexpr int NTHR = NW * 64;
  static constexpr int WM = BM / WTM;                       // waves along M
  static constexpr int WN = NW / WM;                        // waves along N
  static constexpr int MI = WTM / 32;                       // 32-row tiles per wave
  // BK is in bytes of an operand row per stage: 128 FP8 or 64 BF16 elements for BK = 128
  static constexpr bool BF16 = WFMT == 3;                   // BF16 operands, unscaled MFMA
  static constexpr int A_ROWB = BK;                         // bytes per activation row per stage
  static constexpr int B_ROWB = WFMT == 1 ? BK / 2 : BK;    // bytes per weight row per stage
  // weight operand format code of the scaled MFMA: E4M3 0, E5M2 1, E2M1 4
  static constexpr int WCODE = WFMT == 1 ? 4 : (WFMT == 2 ? 1 : 0);
  static constexpr int A_BYTES = BM * A_ROWB;
  static constexpr int B_BYTES = BN * B_ROWB;
  static constexpr int S_BYTES = WFMT == 1 ? NW * 256 : 0;  // MXFP4 scale dwords (64 rows per wave)
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int A_INSTR = A_BYTES / 1024;            // 1 KB DMA instructions of the A tile per stage
  // per wave and stage; a tile of fewer instructions than waves is loaded by every wave, wave w
  // repeating instruction w % A_INSTR (same bytes, same place), so all waves count alike
  static constexpr int A_DMA = A_INSTR >= NW ? A_INSTR / NW : 1;
  static constexpr int B_DMA = B_BYTES / 1024 / NW;
  static constexpr int S_DMA = WFMT == 1 ? 1 : 0;           // 4-byte DMA instructions per wave per stage
  static constexpr int PER_STAGE = A_DMA + B_DMA + S_DMA;
  static constexpr int NT = BN / WN / 32;                   // 32-wide column tiles per wave
  static constexpr int NH = BK / 64;  // 64-byte K steps per stage (one FP8 MFMA or two BF16 ones)
  static constexpr int A_CPR = A_ROWB / 16, B_CPR = B_ROWB / 16;  // 16-byte chunks per row
  static_assert(WM * WN == NW && NT >= 1 && (MODE == 2 || NT % 2 == 0), "waves must cover the tile");
  static_assert(A_INSTR >= 1 && B_DMA >= 1 && B_DMA * NW * 1024 == B_BYTES, "");
  static_assert(A_INSTR >= NW ? A_DMA * NW == A_INSTR : NW % A_INSTR == 0, "");
  static_assert(WFMT != 1 || BN <= NW * 64, "one scale DMA per wave covers 64 weight rows");
  static_assert(PIPE == 0 || PIPE == 2, "stage-at-a-time or half-step pipeline");
  static_assert(PIPE != 2 || BK == 128, "the half-step pipeline splits 128-wide stages");
};

// Operand fragments of one stage for one wave (A rows, B columns, their scale bytes).
template <int MI, int NT, int NH>
struct Frags {
  v8i a[NH][MI];
  v8i b[NH][NT];
  int sa[MI];
  int sb[NH][NT];
};

// ---------------------------------------------------------------------------------------
// direct global -> LDS loads (the wave writes 64 lanes x 16 bytes at m0, lane order)

// the source is a uniform 64-bit base plus a 32-bit per-lane offset (the saddr form); the base
// is passed through readfirstlane so it sits in SGPRs even where the compiler cannot prove it
// uniform.  A VMEM instruction that reads an SGPR written by a VALU instruction (readfirstlane,
// an SGPR spill reload) needs 5 wait states in between; the compiler inserts them before its
// own loads but not inside inline asm, so the asm provides them: s_mov + s_nop 3 (this also
// covers the 1 wait state between writing m0 and the LDS DMA that reads it)
__device__ __forceinline__ const void* sbase(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  base = sbase(base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds) {
  base = sbase(base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// XOR swizzles of 16-byte chunks, conflict-free when 8 (or 16) consecutive rows are read at
// one logical chunk: rows of 128, 64 and 32 bytes.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if (CPR == 8) return (r ^ (r >> 3)) & 7;
  if (CPR == 4) return ((r >> 1) ^ (r >> 3)) & 3;
  return ((r >> 2) ^ (r >> 3)) & 1;
}

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ int find_expert(const int32_t* __restrict__ plan, int EL, int mt) {
  int lo = 0, hi = EL - 1;  // last e with plan[e] <= mt (that expert is non-empty)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (plan[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// FC2 epilogue: fp32 rows of Y2 from the accumulators (tokens are the MFMA's first operand:
// lane l of acc[mi][ct] holds rows 8*(i/4) + 4*kb + i%4 of row tile mi, column
// bcol(ct) + l%32), 32 consecutive columns per lane group.  The 256-row tiles (shares with
// hundreds of MB of Y2) store non-temporally so the burst does not evict the operands; the
// smaller tiles' Y2 (tens of MB) stays in the caches for the combine, which reads it next.
template <int BM, int BN, int WTM, int WM, int WN, int MI, int NT>
__device__ __forceinline__ void store_y2_rows(float* __restrict__ y2, int N, const v16f (&acc)[MI][NT], int wave,
                                              int lane, int rb, int nrows, int c0) {
  const int wm = wave % WM, wn = wave / WM;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = wm * WTM + mi * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (r < nrows) {
        float* dst = y2 + (long long)(rb + r) * N;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          const int col = c0 + wn * (BN / WN) + ct * 32 + (lane & 31);
          if (col < N) {
            if constexpr (BM == 256) __builtin_nontemporal_store(acc[mi][ct][i], dst + col);
            else dst[col] = acc[mi][ct][i];
          }
        }
      }
    }
}

// Two workgroups per CU for the tiles whose ring fits twice in LDS (the register budget
// follows from that); one otherwise.
template <int MODE, int WFMT, int BM, int BN, int BK, int NSTAGE, int NW, int WTM, int PIPE>
constexpr int kWgPerCu = NSTAGE * Cfg<MODE, WFMT, BM, BN, BK, NSTAGE, NW, WTM, PIPE>::STAGE <= 80 * 1024 ? 2 : 1;

// XA (FC1 on FP8 / MXFP4 data only): exact-sum FC1.  The scaled FP8 MFMA's sums carry an error
// near 1.5e-5 of their value (measured: the same for every FP8 instruction form, so it comes from
// how the hardware adds the FP8 products, not from chaining), which flips requantised h codes that
// lie that close to an E4M3 rounding midpoint.  XA converts each operand fragment to BF16 in
// registers with its UE8M0 block scale folded in (exact: the codes have at most 3 significant
// bits) and multiplies with the BF16 MFMA, whose fp32 sums match a sequential fp32 sum of the
// exact products.  It costs conversion instructions and half the matrix-core rate, which is
// free where the GEMM streams weights (few rows per expert).
//
// PT (FC2 only): persistent workgroups.  Each workgroup walks its XCD's tile range with a stride
// of the workgroups on that XCD, derives the tile plan once, and stores a tile's Y2 rows in the
// next tile's prologue (after its token rows and scales are set up, just before its first DMA
// stages are issued) instead of at the end of its own K loop.  The tile plan then lives outside
// the stage ring.  The stores precede the DMAs in issue order, so the first stage wait (vector
// memory operations complete in issue order) also covers them.
template <int MODE, int WFMT, int BM, int BN, int BK, int NSTAGE, int NW, int WTM, int PIPE, int XA, int PT>
__global__ __launch_bounds__(NW * 64, (kWgPerCu<MODE, WFMT, BM, BN, BK, NSTAGE, NW, WTM, PIPE>)) void grouped_gemm_kernel(
    GemmArgs g) {
  using C = Cfg<MODE, WFMT, BM, BN, BK, NSTAGE, NW, WTM, PIPE>;
  static_assert(!XA || (MODE == 1 && WFMT != 3), "exact-sum FC1 is for the scaled formats");
  static_assert(!PT || MODE == 2, "persistent workgroups are for FC2");
  using F = Frags<C::MI, C::NT, C::NH>;
  // LDS (dynamic, sized at launch): the stage ring, then the tile's activation scales
  // [row][ks128] and FP8 weight scales [block][ks128].  The token list of the tile rows and
  // the epilogue's amax scratch live inside the ring while it is not in use.
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  uint8_t* ring = lds;
  uint8_t* s_asf = lds + NSTAGE * C::STAGE;
  const int nk128_ = C::BF16 ? 0 : g.K / 128;
  const int asr = asf_row_bytes(nk128_);  // bytes per row of the activation-scale table
  uint8_t* s_bsf = s_asf + asf_table_bytes(BM, nk128_);
  int* s_tok = reinterpret_cast<int*>(ring + NSTAGE * C::STAGE - BM * 4);  // prologue only
  float(*s_amax)[BM] = reinterpret_cast<float(*)[BM]>(ring + BM * 128);      // epilogue only

  // tile plan: plan[e] = m-tiles of the experts before e, plan[EL] = all.  The fused path
  // passes the one the permute wrote; the split entry points pass none and every workgroup
  // scans the offsets itself.  Either way the plan and the expert offsets are put in LDS
  // (inside the ring, which the prologue does not use yet) by loads that are all in flight
  // together, so the expert search below reads LDS instead of chaining dependent global loads
  int* s_plan = PT ? reinterpret_cast<int*>(lds + ((NSTAGE * C::STAGE + asf_table_bytes(BM, nk128_) + 2 * nk128_ + 15) & ~15))
                   : reinterpret_cast<int*>(ring);  // [EL + S + 1]
  int* s_wsum = s_plan + kMaxExperts + 8;      // [NW]
  int* s_offs = s_wsum + 16;                   // [EL + 1]
  static_assert(NSTAGE * C::STAGE >= (2 * kMaxExperts + 32) * 4 + BM * 4, "plan and offsets fit before s_tok");
  if (g.plan != nullptr) {  // no shared experts on this path: the plan has EL + 1 entries
    for (int j = threadIdx.x; j <= g.EL; j += C::NTHR) {
      const int o = g.offsets[j], p = g.plan[j];  // both loads in flight before either store
      s_offs[j] = o;
      s_plan[j] = p;
    }
    __syncthreads();
  } else {
    for (int j = threadIdx.x; j <= g.EL; j += C::NTHR) s_offs[j] = g.offsets[j];
    const int t = threadIdx.x, n = g.EL + g.S + 1, per = (n + C::NTHR - 1) / C::NTHR, beg = t * per;
    int sum = 0;
    for (int j = 0; j < per; ++j) {
      const int ee = beg + j;
      if (ee < n) s_plan[ee] = sum;
      if (ee < g.EL) sum += (g.offsets[ee + 1] - g.offsets[ee] + BM - 1) / BM;
      else if (ee < n - 1) sum += (g.T + BM - 1) / BM;
    }
    const int inc = wave_inclusive_scan(sum);
    if ((t & 63) == 63) s_wsum[t >> 6] = inc;
    __syncthreads();
    int base = inc - sum;
    for (int w = 0; w < (t >> 6); ++w) base += s_wsum[w];
    for (int j = 0; j < per; ++j)
      if (beg + j < n) s_plan[beg + j] += base;
    __syncthreads();
  }
  const int* plan = s_plan;
  const int NE = g.EL + g.S;  // experts with rows: routed, then shared
  const int total = plan[NE] * g.n_tiles;
  const int bid = blockIdx.x;
  // XCD-aware order: dispatch is round-robin over 8 XCDs; each XCD gets a contiguous range of
  // tiles (persistent: workgroup bid >> 3 of XCD bid & 7 takes every (gridDim.x / 8)-th of them)
  int L, pt_p = 0, pt_cnt = 0, pt_base = 0;
  {
    const int x = bid & 7, q = total >> 3, r = total & 7;
    pt_p = bid >> 3;
    pt_cnt = q + (x < r ? 1 : 0);
    pt_base = x * q + (x < r ? x : r);
    if (pt_p >= pt_cnt) return;
    L = pt_base + pt_p;
  }
  // FC2 epilogue: fp32 rows of Y2 from the accumulators (tokens are the MFMA's first operand:
  // lane l of acc[mi][ct] holds rows 8*(i/4) + 4*kb + i%4 of row tile mi, column
  // bcol(ct) + l%32), 32 consecutive columns per lane group.  The 256-row tiles (shares with
  // hundreds of MB of Y2) store non-temporally so the burst does not evict the operands; the
  // smaller tiles' Y2 (tens of MB) stays in the caches for the combine, which reads it next
  v16f acc[C::MI][C::NT];
  int pv_row_begin = 0, pv_rows = 0, pv_n0 = 0;  // the tile whose Y2 stores are pending (PT)
  bool pv_live = false, pv_have = false;
  for (;;) {
  if (PT && pv_have) __syncthreads();  // every wave is past its last LDS read of the previous tile
  const int e = find_expert(plan, NE, L / g.n_tiles);
  const int mt_e = plan[e + 1] - plan[e];
  const int li = L - plan[e] * g.n_tiles;
  const int gn = g.n_tiles < kGroupN ? g.n_tiles : kGroupN;
  const int grp = li / (gn * mt_e);
  const int gsz = (g.n_tiles - grp * gn) < gn ? (g.n_tiles - grp * gn) : gn;
  const int idx = li - grp * gn * mt_e;
  const int m_tile = idx / gsz;
  const int n_tile = grp * gn + idx % gsz;
  // rows of expert e: routed experts from the offsets, shared expert s = e - EL after them
  const bool shared = e >= g.EL;
  const int seg_begin = shared ? s_offs[g.EL] + (e - g.EL) * g.T : s_offs[e];
  const int seg_end = shared ? seg_begin + g.T : s_offs[e + 1];
  const int row_begin = seg_begin + m_tile * BM;
  const int rows = min(BM, seg_end - row_begin);

  // the wave index is made scalar for the 256-row tiles (fewer registers there); the 128-row
  // tiles, whose row-tile skipping switches on it, allocate fewer with it left in a VGPR
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = BM == 256 ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int wm = wave % C::WM, wn = wave / C::WM;
  const int Kb = C::BF16 ? 2 * g.K : g.K;  // bytes per operand row (FP8: K, BF16: 2K)
  const int nk = Kb / BK;                  // stages
  const int nk128 = g.K / 128;             // scale steps (scaled formats)
  const int n0 = MODE == 1 ? n_tile * 128 : n_tile * BN;

  // ---- tile rows: the token (FC1; row i of a shared expert is token i) or h row (FC2) of
  //      each tile row; rows past the expert's last row repeat the first one ----
  for (int i = tid; i < BM; i += C::NTHR) {
    const int r = i < rows ? i : 0;
    s_tok[i] = MODE == 2 ? row_begin + r : shared ? row_begin + r - seg_begin : g.row_to_slot[row_begin + r] / g.k;
  }
  // FP8 weight scales of the tile's two 128-row blocks (FC1: gate n0/128 and up (I+n0)/128;
  // FC2: n0/128 and n0/128 + 1, clamped), loaded now and written to LDS before the first DMA:
  // the compiler cannot count the DMAs (inline asm), so its wait for this load is a full
  // vmcnt(0) and, placed after them, would drain every stage in flight
  const uint8_t* bsf_e = g.B_sf + (long long)e * g.bsf_estride;
  const bool bsf_mine = WFMT != 1 && !C::BF16 && tid < 2 * nk128;
  int bsf_v = 0;
  if (bsf_mine) {
    const int blk = tid / nk128, ks = tid - blk * nk128;
    const int br = MODE == 1 ? (blk == 0 ? n0 / 128 : (g.I + n0) / 128) : min(n0 / 128 + blk, g.N / 128 - 1);
    bsf_v = g.tensor ? 127 : bsf_e[(long long)br * nk128 + ks];
  }
  __syncthreads();
  // activation scales of the tile rows in LDS as [row][k step] (rows asr bytes apart): moved by
  // 4-byte DMA when a row is whole dwords (nk128 % 4 == 0), else by byte loads
  const bool asf_packed = g.asf_am > 0;
  const uint8_t* asf_gbase = MODE == 1 || asf_packed ? g.A_sf : g.A_sf + (long long)row_begin * nk128;
  const bool asf_dma = !C::BF16 && !g.tensor && (nk128 & 3) == 0;
  constexpr int kAsfDma = (asf_table_bytes(BM, kMaxKSteps) / 256 + NW - 1) / NW;  // 64-lane DMAs per wave, at most
  const int asf_n = asf_table_bytes(BM, nk128) / 256;                              // 64-lane DMAs of the tile
  uint32_t asf_off[kAsfDma];
  if (asf_dma) {
    // lane q of the table's DMAs fills dword q: row q / spr, data dword q % spr of it; the pad
    // dword of a row and the rows past the tile (the 256-byte rounding) repeat a valid dword
    const int dpr = nk128 / 4, spr = asr / 4;  // data dwords and table dwords per row
#pragma unroll
    for (int j = 0; j < kAsfDma; ++j) {
      const int q = (wave + NW * j) * 64 + lane, r0 = q / spr;
      const int row = min(r0, BM - 1), dw = min(q - r0 * spr, dpr - 1);
      asf_off[j] = asf_packed ? ((uint32_t)dw * (uint32_t)g.asf_am + (uint32_t)s_tok[row]) * 4u
                              : (uint32_t)(s_tok[row] - (MODE == 1 ? 0 : row_begin)) * (uint32_t)nk128 +
                                    (uint32_t)dw * 4u;
    }
  } else if (!C::BF16) {
    for (int i = tid; i < nk128 * BM; i += C::NTHR) {
      const int r = i / nk128;
      const int ks = i - r * nk128;
      s_asf[r * asr + ks] = g.tensor ? 127
                 : asf_packed ? asf_gbase[((long long)(ks >> 2) * g.asf_am + s_tok[r]) * 4 + (ks & 3)]
                              : asf_gbase[(long long)(s_tok[r] - (MODE == 1 ? 0 : row_begin)) * nk128 + ks];
    }
  }

  // ---- DMA sources of this lane (offsets from uniform bases), swizzled chunk folded in ----
  // FC1 gathers token rows of x (offsets below 2^32: x is smaller than 4 GiB); FC2 reads the
  // tile's rows of h from the tile's first row
  const uint8_t* a_gbase = MODE == 1 ? g.A : g.A + (long long)row_begin * Kb;
  uint32_t a_off[C::A_DMA];
#pragma unroll
  for (int j = 0; j < C::A_DMA; ++j) {
    const int r = ((wave * C::A_DMA + j) % C::A_INSTR) * (64 / C::A_CPR) + lane / C::A_CPR;
    const int c = (lane % C::A_CPR) ^ swz<C::A_CPR>(r);
    a_off[j] = (uint32_t)(s_tok[r] - (MODE == 1 ? 0 : row_begin)) * (uint32_t)Kb + (uint32_t)(c * 16);
  }
  const uint8_t* b_e = g.B + (long long)e * g.b_estride;
  auto b_row = [&](int n) -> int {
    if (MODE == 1) return n < 128 ? n0 + n : g.I + n0 + (n - 128);
    const int rr = n0 + n;
    return rr < g.N ? rr : g.N - 1;
  };
  const uint32_t b_ld = WFMT == 1 ? g.K / 2 : Kb;
  uint32_t b_off[C::B_DMA];
#pragma unroll
  for (int j = 0; j < C::B_DMA; ++j) {
    const int n = (wave * C::B_DMA + j) * (64 / C::B_CPR) + lane / C::B_CPR;
    const int c = (lane % C::B_CPR) ^ swz<C::B_CPR>(n);
    b_off[j] = (uint32_t)b_row(n) * b_ld + (uint32_t)(c * 16);
  }
  // MXFP4: wave w loads the scale dword (4 blocks of 32 = one 128-wide K step) of weight rows
  // (w % (BN/64)) * 64 + lane; waves beyond BN/64 load a second copy that is never read
  uint32_t s_off = 0;
  if (WFMT == 1) s_off = (uint32_t)b_row((wave % (BN / 64)) * 64 + lane) * (uint32_t)(g.K / 32);
  __syncthreads();  // s_tok (inside the ring) is consumed before the ring is filled
  if (bsf_mine) s_bsf[tid] = (uint8_t)bsf_v;  // before any DMA; published by the first wait's barrier
  // every wave, scale lanes or not: no load of the compiler's own is outstanding past this
  // point, so it adds no vmcnt(0) (which would also drain the DMAs) for this load's register
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt not waited for
  // persistent FC2: the previous tile's Y2 stores go out now, ahead of this tile's DMAs
  if (PT && pv_have && pv_live)
    store_y2_rows<BM, BN, WTM, C::WM, C::WN, C::MI, C::NT>(g.y2, g.N, acc, wave, lane, pv_row_begin, pv_rows, pv_n0);
  if (asf_dma) {
#pragma unroll
    for (int j = 0; j < kAsfDma; ++j)
      if (wave + NW * j < asf_n) dma4(asf_gbase, asf_off[j], uniform(lds_addr(s_asf) + (wave + NW * j) * 256));
  }

  const uint32_t ring0 = lds_addr(ring);
  auto issue = [&](int ks) {
    const uint32_t st = ring0 + (uint32_t)((ks % NSTAGE) * C::STAGE);
    const uint8_t* ab = a_gbase + (long long)ks * C::A_ROWB;
    const uint8_t* bb = b_e + (long long)ks * C::B_ROWB;
#pragma unroll
    for (int j = 0; j < C::A_DMA; ++j)
      dma16(ab, a_off[j], uniform(st + ((wave * C::A_DMA + j) % C::A_INSTR) * 1024));
#pragma unroll
    for (int j = 0; j < C::B_DMA; ++j) dma16(bb, b_off[j], uniform(st + C::A_BYTES + (wave * C::B_DMA + j) * 1024));
    if (WFMT == 1)
      dma4(bsf_e + ((ks * BK) / 128) * 4, s_off, uniform(st + C::A_BYTES + C::B_BYTES + wave * 256));
  };
  // wait until at most `ahead` stages of this wave's DMA are in flight, then workgroup barrier
  auto wait_stages = [&](int ahead) {
    if (ahead >= 3) wait_vm_barrier<3 * C::PER_STAGE>();
    else if (ahead == 2) wait_vm_barrier<2 * C::PER_STAGE>();
    else if (ahead == 1) wait_vm_barrier<C::PER_STAGE>();
    else wait_vm_barrier<0>();
  };

#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int ct = 0; ct < C::NT; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][ct][i] = 0.f;

  const int lrow = lane & 31, kb = lane >> 5;
  // a wave whose rows all lie past the expert's last row skips its MFMAs (decode-sized experts);
  // the test is wave-uniform so the MFMA burst stays one straight-line block
  const bool wave_live = wm * WTM < rows;
  // first weight row (tile-local) of column tile ct of this wave, and its offset from tile 0's
  auto bdelta = [](int ct) -> int {
    if (MODE == 1) return ct < C::NT / 2 ? ct * 32 : 128 + (ct - C::NT / 2) * 32;
    return ct * 32;
  };
  const int bcol0 = MODE == 1 ? wn * (128 / C::WN) : wn * (BN / C::WN);
  auto bcol = [&](int ct) -> int { return bcol0 + bdelta(ct); };

  // LDS read addresses.  Rows 32 apart have the same swizzle in 64- and 32-byte rows and
  // differ only in bit 2 of it in 128-byte rows, where bit 2 of the chunk index is the 64-wide
  // K half; so every operand read is a per-lane base (row tile 0, K half 0), possibly with
  // byte 64 (FP8) or 32 (FP4) toggled, plus an immediate row offset.
  const int ra = wm * WTM + lrow, rb = bcol0 + lrow;
  uint32_t a_lds[2], b_lds[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    // exact-sum FC1 on MXFP4 weights reads a token fragment as the contiguous K values
    // [32 kb, +32) of the 64-wide step (chunks 2 kb and 2 kb + 1), the K values of the
    // weight fragment it is multiplied with
    const int achunk = (XA && WFMT == 1) ? 2 * kb + hi : 2 * hi + kb;
    a_lds[hi] = ra * C::A_ROWB + ((achunk ^ swz<C::A_CPR>(ra)) << 4);
    b_lds[hi] = WFMT != 1 ? rb * C::B_ROWB + (((2 * hi + kb) ^ swz<C::B_CPR>(rb)) << 4)
                           : rb * C::B_ROWB + ((kb ^ swz<C::B_CPR>(rb)) << 4);
  }

  // operand fragments of 64-wide K steps h0 .. h0 + NHF - 1 of stage ks from its ring slot
  auto load_into = [&](int ks, int h0, auto& f) {
    constexpr int NHF = sizeof(f.b) / sizeof(f.b[0]);
    const uint8_t* st = ring + (ks % NSTAGE) * C::STAGE;
    const uint8_t* sb_ = st + C::A_BYTES;
    const int k128 = (ks * BK) / 128;
    if (!C::BF16) {
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi) f.sa[mi] = s_asf[(ra + mi * 32) * asr + k128];
    }
    int sbu0 = 0, sbu1 = 0;
    if (WFMT != 1 && !C::BF16) {  // one weight scale per 128x128 block
      if (MODE == 1) { sbu0 = s_bsf[k128]; sbu1 = s_bsf[nk128 + k128]; }
      else { sbu0 = s_bsf[(wn * (BN / C::WN)) / 128 * nk128 + k128]; sbu1 = sbu0; }
    }
#pragma unroll
    for (int hh = 0; hh < NHF; ++hh) {
      const int h = h0 + hh;
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi) {
        const bool flip = C::A_CPR == 8 && ((h ^ mi) & 1);
        const int imm = mi * 32 * C::A_ROWB;
        const uint4 lo = lds16(st + (flip ? a_lds[0] ^ 64u : a_lds[0]) + imm);
        const uint4 hi = lds16(st + (flip ? a_lds[1] ^ 64u : a_lds[1]) + imm);
        f.a[hh][mi] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int ct = 0; ct < C::NT; ++ct) {
        const int d = bdelta(ct);
        if (WFMT != 1) {
          const bool flip = C::B_CPR == 8 && ((h ^ (d / 32)) & 1);
          const int imm = d * C::B_ROWB;
          const uint4 lo = lds16(sb_ + (flip ? b_lds[0] ^ 64u : b_lds[0]) + imm);
          const uint4 hi = lds16(sb_ + (flip ? b_lds[1] ^ 64u : b_lds[1]) + imm);
          f.b[hh][ct] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          f.sb[hh][ct] = (MODE == 1 && ct >= C::NT / 2) ? sbu1 : sbu0;
        } else {
          // chunk 2h + kb of a 64-byte row (bit 1 = K half) or chunk kb of a 32-byte row
          const bool flip = C::B_CPR == 4 && (h & 1);
          const uint4 q = lds16(sb_ + (flip ? b_lds[0] ^ 32u : b_lds[0]) + d * C::B_ROWB);
          f.b[hh][ct] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
          const int dw = *reinterpret_cast<const int*>(st + C::A_BYTES + C::B_BYTES + rb * 4 + d * 4);
          const int blk = ((ks * BK) % 128) / 32 + 2 * h + kb;  // 32-wide block inside the 128-wide step
          f.sb[hh][ct] = dw >> (8 * blk);                         // the MFMA reads the low byte
        }
      }
    }
  };
  // MFMAs of one stage for the first NL row tiles of the wave (row tiles past the expert's last
  // row are skipped; NL is wave-uniform, so each case is one straight-line MFMA burst)
  auto mma_n = [&](const auto& f, auto nl) {
    constexpr int NL = decltype(nl)::value;
    constexpr int NHF = sizeof(f.b) / sizeof(f.b[0]);
    if constexpr (XA) {
      // four BF16 MFMAs per 64-wide K step: group q of the lane's values of both operands (the
      // same K positions in both), scales folded into the conversions
#pragma unroll
      for (int h = 0; h < NHF; ++h) {
        bf16x8 tq[NL][4];
#pragma unroll
        for (int mi = 0; mi < NL; ++mi) {
          const float sc = scale_f32(f.sa[mi]);
#pragma unroll
          for (int q = 0; q < 4; ++q) tq[mi][q] = fp8_group_bf16<false>(f.a[h][mi], q, sc);
        }
#pragma unroll
        for (int ct = 0; ct < C::NT; ++ct) {
          const float sc = scale_f32(f.sb[h][ct]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bf16x8 wq = WFMT == 1 ? fp4_group_bf16(f.b[h][ct], q, sc)
                                        : fp8_group_bf16<WFMT == 2>(f.b[h][ct], q, sc);
#pragma unroll
            for (int mi = 0; mi < NL; ++mi)
              acc[mi][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wq, tq[mi][q], acc[mi][ct], 0, 0, 0);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int h = 0; h < NHF; ++h)
#pragma unroll
      for (int ct = 0; ct < C::NT; ++ct)
#pragma unroll
        for (int mi = 0; mi < NL; ++mi) {
          if constexpr (C::BF16) {
            // the 32 bytes of a lane are two 16-wide K steps of 8 BF16 values each (chunks kb
            // and 2 + kb of the 64-byte step), one unscaled 32x32x16 MFMA each
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const bf16x8 a = bf16_half(f.a[h][mi], q), b = bf16_half(f.b[h][ct], q);
              acc[mi][ct] = MODE == 1 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc[mi][ct], 0, 0, 0)
                                      : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[mi][ct], 0, 0, 0);
            }
          } else {
            acc[mi][ct] = MODE == 1
                              ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[h][ct], f.a[h][mi], acc[mi][ct],
                                                                                C::WCODE, 0, 0, f.sb[h][ct],
                                                                                0, f.sa[mi])
                              : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[h][mi], f.b[h][ct], acc[mi][ct],
                                                                                0, C::WCODE, 0, f.sa[mi], 0,
                                                                                f.sb[h][ct]);
          }
        }
  };
  const int live_tiles = min(C::MI, max(0, (rows - wm * WTM + 31) / 32));
  auto mma = [&](const auto& f) {
    if (BM != 128 || live_tiles >= C::MI) mma_n(f, std::integral_constant<int, C::MI>{});  // 128-row tiles only
    else if (C::MI > 1 && live_tiles == 1) mma_n(f, std::integral_constant<int, 1>{});
    else if (C::MI > 2 && live_tiles == 2) mma_n(f, std::integral_constant<int, (C::MI > 2 ? 2 : 1)>{});
    else if (C::MI > 3 && live_tiles == 3) mma_n(f, std::integral_constant<int, (C::MI > 3 ? 3 : 1)>{});
  };

  // prologue: NSTAGE-1 stages in flight
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < nk) issue(s);

  if (PIPE == 0) {
    for (int ks = 0; ks < nk; ++ks) {
      wait_stages(min(nk - 1 - ks, NSTAGE - 2));
      if (ks + NSTAGE - 1 < nk) issue(ks + NSTAGE - 1);
      if (!wave_live) continue;
      F f;
      load_into(ks, 0, f);
      mma(f);
    }
  } else {
    // half-step pipeline (two 64-wide K steps per stage): the fragments of the next half are
    // read from LDS while the MFMAs of the current one run.  The stage boundary (DMA wait,
    // barrier, next DMA issue) sits between a stage's second-half reads and its MFMAs, when
    // every wave is done reading the stage, so the ring holds NSTAGE stages with NSTAGE - 1
    // of them in flight.
    static_assert(PIPE != 2 || C::NH == 2, "half-step pipeline needs 128-wide stages");
    using FH = Frags<C::MI, C::NT, 1>;
    FH x, y;
    if (NSTAGE - 1 < nk) issue(NSTAGE - 1);
    wait_stages(min(nk - 1, NSTAGE - 1));
    // every part of the loop is straight-line code so the reads of one half and the MFMAs of
    // the other interleave freely; waves with no live rows only take part in the DMA and barriers
    auto run = [&](auto live) {
      constexpr bool L = decltype(live)::value;
      if (L) load_into(0, 0, x);
      int ks = 0;
      for (; ks + NSTAGE < nk; ++ks) {  // steady state: stage ks + NSTAGE goes to the freed slot
        if (L) { load_into(ks, 1, y); mma(x); }
        wait_stages(NSTAGE - 2);
        issue(ks + NSTAGE);
        if (L) { load_into(ks + 1, 0, x); mma(y); }
      }
      for (; ks + 1 < nk; ++ks) {  // drain
        if (L) { load_into(ks, 1, y); mma(x); }
        wait_stages(nk - 2 - ks);
        if (L) { load_into(ks + 1, 0, x); mma(y); }
      }
      if (L) { load_into(ks, 1, y); mma(x); mma(y); }
    };
    if (wave_live) run(std::true_type{});
    else run(std::false_type{});
  }

  if (g.tensor) {  // per-tensor scales: one factor for the whole tile
    const float sc = (MODE == 1 ? g.a_tscale[0] : g.h_scale) * g.b_tscale[e];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int ct = 0; ct < C::NT; ++ct)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mi][ct][i] *= sc;
  }

  if (MODE == 2) {
    if (PT) {  // the next tile of this workgroup, if any; this tile's stores are deferred
      pv_row_begin = row_begin; pv_rows = rows; pv_n0 = n0; pv_live = wave_live; pv_have = true;
      pt_p += gridDim.x >> 3;
      if (pt_p < pt_cnt) {
        L = pt_base + pt_p;
        continue;
      }
    }
    if (wave_live)
      store_y2_rows<BM, BN, WTM, C::WM, C::WN, C::MI, C::NT>(g.y2, g.N, acc, wave, lane, row_begin, rows, n0);
    return;
  }

  // FC1 accumulator layout (weights are the MFMA's first operand, tokens its second, so a
  // lane holds one tile row): lane l of acc[mi][ct] holds tile row wm*WTM + mi*32 + l%32 and,
  // for value i, weight row bcol(ct) + 8*(i/4) + 4*kb + i%4, i.e. runs of 4 consecutive
  // columns.
  const int trow = wm * WTM + lrow;  // tile row of row tile 0 of this lane
  // ---- FC1 epilogue: activation, 1x128 amax, UE8M0 scale, E4M3 codes ----
  // The lane's values of row tile mi all belong to tile row trow + mi*32: gate in
  // acc[mi][c], up in acc[mi][c + NC] at h column wn*128/WN + c*32 + 8*(i/4) + 4*kb + i%4.
  constexpr int NC = C::NT / 2;
  if (g.act == 1) {
    const float cl = g.clamp, al = g.alpha, bi = g.bias;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) {  // clamps as one med3 each; h overwrites the gate
          const float gt = __builtin_amdgcn_fmed3f(acc[mi][c][i], -INFINITY, cl);
          const float up = __builtin_amdgcn_fmed3f(acc[mi][c + NC][i], -cl, cl);
          acc[mi][c][i] = gt * sigmoidf_(al * gt) * (up + bi);
        }
  } else {
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float gt = acc[mi][c][i];
          acc[mi][c][i] = gt * sigmoidf_(gt) * acc[mi][c + NC][i];
        }
  }
  if constexpr (C::BF16) {
    // ---- BF16 layer: h is the activation rounded once to BF16 (no scale).  Four
    //      consecutive columns per lane go to a [BM rows][256 B] tile with 16-byte chunks
    //      XOR-swizzled by row, then whole 16-byte chunks go out row by row ----
    __syncthreads();  // every wave is past its last ring read
    uint8_t* stage_h = ring;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      const int r = trow + mi * 32;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[mi][c][4 * q]) |
                              ((uint32_t)f32_to_bf16_rne(acc[mi][c][4 * q + 1]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[mi][c][4 * q + 2]) |
                              ((uint32_t)f32_to_bf16_rne(acc[mi][c][4 * q + 3]) << 16);
          const int col = wn * (128 / C::WN) + c * 32 + 8 * q + 4 * kb;  // multiple of 4
          *reinterpret_cast<uint2*>(stage_h + r * 256 + ((((col >> 3) ^ (r & 15)) << 4) | ((col & 7) * 2))) =
              make_uint2(lo, hi);
        }
    }
    __syncthreads();
    for (int q = tid; q < BM * 16; q += C::NTHR) {
      const int r = q >> 4, c = q & 15;
      if (r < rows)
        *reinterpret_cast<uint4*>(g.h + (long long)(row_begin + r) * (2 * g.I) + 2 * n0 + c * 16) =
            *reinterpret_cast<const uint4*>(stage_h + r * 256 + ((c ^ (r & 15)) << 4));
    }
    return;
  }
  // amax of each row: over the lane's values (an unsigned max of the non-negative float
  // bits), then with lane l ^ 32 (the other half of the columns), then across the WN waves
  // through LDS.  Both lanes of a pair write the same value to the same place.
  uint32_t rmax[C::MI];
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) {
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t v = __float_as_uint(acc[mi][c][i]) & 0x7fffffffu;
        m = m > v ? m : v;
      }
    const uint32_t o = (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, (int)m);
    rmax[mi] = m > o ? m : o;
  }
  // s_amax lies inside the ring, possibly in the stage the slowest wave still reads: write
  // it once every wave is past its last ring read
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) s_amax[wn][trow + mi * 32] = __uint_as_float(rmax[mi]);
  __syncthreads();  // s_amax complete
  // E4M3 codes, four consecutive columns per dword (two packed conversions), into the
  // [BM rows][128 B] code tile with its 16-byte chunks XOR-swizzled by row (the rows of one
  // wave's writes then spread over the banks); the UE8M0 byte of each row goes to a [BM]
  // array after it.  Every lane of a row computes the same byte.
  uint8_t* stage_h = ring;
  uint8_t* stage_sf = ring + BM * 128 + C::WN * BM * 4;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) {
    const int r = trow + mi * 32;
    uint32_t mx = __float_as_uint(s_amax[0][r]);
#pragma unroll
    for (int w = 1; w < C::WN; ++w) {
      const uint32_t o = __float_as_uint(s_amax[w][r]);
      mx = mx > o ? mx : o;
    }
    const int sfb = ue8m0_for_amax(__uint_as_float(mx));
    stage_sf[r] = (uint8_t)sfb;
    uint8_t* hrow = stage_h + r * 128;
    // block scales keep every value within +-448; the static per-tensor scale saturates
    auto pack = [&](float inv, auto sat) {
      auto v = [&](int c, int j) {
        const float t = acc[mi][c][j] * inv;
        return decltype(sat)::value ? __builtin_amdgcn_fmed3f(t, -448.f, 448.f) : t;
      };
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(v(c, 4 * q), v(c, 4 * q + 1), 0, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(v(c, 4 * q + 2), v(c, 4 * q + 3), word, true);
          const int col = wn * (128 / C::WN) + c * 32 + 8 * q + 4 * kb;  // multiple of 4
          *reinterpret_cast<int*>(hrow + ((((col >> 4) ^ (r & 7)) << 4) | (col & 15))) = word;
        }
    };
    if (g.tensor) pack(g.h_inv, std::true_type{});
    else pack(inv_scale_of(sfb), std::false_type{});
  }
  __syncthreads();
  for (int q = tid; q < BM * 8; q += C::NTHR) {
    const int r = q >> 3, c = q & 7;
    if (r < rows) {
      *reinterpret_cast<uint4*>(g.h + (long long)(row_begin + r) * g.I + n0 + c * 16) =
          *reinterpret_cast<const uint4*>(stage_h + r * 128 + ((c ^ (r & 7)) << 4));
      if (c == 0 && !g.tensor) {
        const long long at = g.hsf_am > 0 ? ((long long)(n_tile >> 2) * g.hsf_am + row_begin + r) * 4 + (n_tile & 3)
                                          : (long long)(row_begin + r) * (g.I / 128) + n_tile;
        g.h_sf[at] = stage_sf[r];
      }
    }
  }
  return;
  }  // tile loop
}

// variant 0: 128-row tiles, 4 waves (FC1: 64-K stages x 3, FC2: 128 columns, 128-K stages
//            x 2), small enough for two workgroups per CU: experts with tens of rows.
// variant 1: 256-row tiles (8 waves of 64x128, 128-K stages x 2): experts with many rows
//            (prefill).  Measured on the prefill share against 64-K x 4 stages, 128x128 wave
//            tiles and fragments read one stage ahead: this shape was fastest.
// variant 2: 32-row tiles, 4 waves side by side along the 256 weight rows, 128-K stages:
//            experts with a handful of rows (decode), where the tile streams weights and
//            the activation rows are a small part of each stage.
int gemm_block_m(int variant) { return variant == 1 ? 256 : variant == 2 ? 32 : 128; }

size_t gemm_max_mtiles(int rows_cap, int EL, int variant, int T, int S) {
  const int bm = gemm_block_m(variant);
  // sum_e ceil(c_e / bm) <= (R + EL * (bm - 1)) / bm with R <= rows_cap, plus the shared
  // experts' ceil(T / bm) each
  return ((size_t)rows_cap + (size_t)EL * (bm - 1)) / bm + (size_t)S * (((size_t)T + bm - 1) / bm);
}

bool gemm_supports(int H, int I) { return H / 128 <= kMaxKSteps && I / 128 <= kMaxKSteps; }

// compute units of the current device (cached per device)
static int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <int MODE, int WFMT, int BM, int BN, int BK, int NSTAGE, int NW, int WTM, int PIPE, int XA, int PT = 0>
static hipError_t launch_one(const GemmArgs& a, size_t grid, hipStream_t s) {
  using C = Cfg<MODE, WFMT, BM, BN, BK, NSTAGE, NW, WTM, PIPE>;
  static_assert(NSTAGE * C::STAGE >= BM * 128 + C::WN * BM * 4 + BM && NSTAGE * C::STAGE >= BM * 4 + BM * 128 &&
                    (!C::BF16 || NSTAGE * C::STAGE >= BM * 256),
                "the ring must hold the epilogue staging and the tile's token list");
  auto kern = grouped_gemm_kernel<MODE, WFMT, BM, BN, BK, NSTAGE, NW, WTM, PIPE, XA, PT>;
  constexpr size_t kPlanBytes = (2 * kMaxExperts + 32) * 4;  // persistent: plan, block sums, offsets
  const size_t nk128 = C::BF16 ? 0 : a.K / 128;
  const size_t tab = (size_t)asf_table_bytes(BM, (int)nk128) + 2 * nk128;  // activation and weight scales
  const size_t lds = PT ? (((size_t)NSTAGE * C::STAGE + tab + 15) & ~(size_t)15) + kPlanBytes
                        : (size_t)NSTAGE * C::STAGE + tab;
  // raise the kernel's dynamic LDS limit to its largest size (K = 8192) once per device
  static std::atomic<uint64_t> ready{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(ready.load(std::memory_order_acquire) & bit)) {
    const size_t most = (size_t)NSTAGE * C::STAGE + (size_t)asf_table_bytes(BM, kMaxKSteps) + 2 * kMaxKSteps +
                        (PT ? 16 + kPlanBytes : 0);
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)most);
    if (e != hipSuccess) return e;
    ready.fetch_or(bit, std::memory_order_acq_rel);
  }
  if (PT) {  // one workgroup per CU (rounded to whole XCD rows of 8), or fewer for a small grid
    const size_t cus = (size_t)device_cus();
    grid = ((grid < cus ? grid : cus) + 7) / 8 * 8;
  }
  kern<<<dim3((unsigned)grid), dim3(NW * 64), lds, s>>>(a);
  return hipGetLastError();
}

template <int MODE, int WFMT, int XA>
static hipError_t launch_variant_w(const GemmArgs& a, int variant, size_t grid, hipStream_t s) {
  // 256-row tiles: eight waves of 64 x 128; MXFP4 FC1 (half the weight bytes per stage, so
  // the MFMAs and LDS reads decide) runs faster as four waves of 128 x 128, accumulators in
  // AGPRs (measured on the 32768-token share: 0.941 against 0.977 ms)
  if (variant == 1) {
    if constexpr (MODE == 1 && WFMT == 1) return launch_one<MODE, WFMT, 256, 256, 128, 2, 4, 128, 2, XA>(a, grid, s);
    else if constexpr (MODE == 2) return launch_one<MODE, WFMT, 256, 256, 128, 2, 8, 64, 2, XA, 1>(a, grid, s);
    else return launch_one<MODE, WFMT, 256, 256, 128, 2, 8, 64, 2, XA>(a, grid, s);
  }
  if (variant == 2) {
    if constexpr (WFMT == 1) return launch_one<MODE, WFMT, 32, 256, 128, 3, 4, 32, 2, XA>(a, grid, s);
    else return launch_one<MODE, WFMT, 32, 256, 128, 2, 4, 32, 2, XA>(a, grid, s);
  }
  // experts with tens of rows: FC2 tiles are 128 columns wide, two workgroups of 8 waves
  // per CU (one streams weights while the other is in its prologue or epilogue); FC1 streams
  // whole 128-byte weight-row segments through a three-stage ring, one workgroup of 8 waves
  // per CU (two per SIMD, so one wave's LDS reads overlap the other's MFMAs), except MXFP4,
  // whose 64-byte stages keep two workgroups per CU
  if constexpr (MODE == 2) return launch_one<MODE, WFMT, 128, 128, 128, 2, 8, 32, 0, XA>(a, grid, s);
  else if constexpr (WFMT == 1) return launch_one<MODE, WFMT, 128, 256, 64, 4, 4, 64, 0, XA>(a, grid, s);
  else return launch_one<MODE, WFMT, 128, 256, 128, 3, 8, 32, 0, XA>(a, grid, s);
}

// weight formats: 0 FP8 E4M3 with 128x128 scales, 1 MXFP4, 2 FP8 E5M2 with 128x128 scales,
// 3 BF16 (activations, weights and the intermediate all BF16, no scales)
template <int MODE>
static hipError_t launch_variant(const GemmArgs& a, int wfmt, int variant, bool exact, size_t grid, hipStream_t s) {
  if constexpr (MODE == 1) {
    if (exact && wfmt != 3) {
      if (wfmt == 1) return launch_variant_w<MODE, 1, 1>(a, variant, grid, s);
      if (wfmt == 2) return launch_variant_w<MODE, 2, 1>(a, variant, grid, s);
      return launch_variant_w<MODE, 0, 1>(a, variant, grid, s);
    }
  }
  if (wfmt == 1) return launch_variant_w<MODE, 1, 0>(a, variant, grid, s);
  if (wfmt == 2) return launch_variant_w<MODE, 2, 0>(a, variant, grid, s);
  if (wfmt == 3) return launch_variant_w<MODE, 3, 0>(a, variant, grid, s);
  return launch_variant_w<MODE, 0, 0>(a, variant, grid, s);
}

// per-tensor scaling: the scale tensors hold float32 values (x: one, weights: one per expert)
static void set_tensor_scales(GemmArgs& a, const Shape& sh, const float* a_scale, const float* b_scale) {
  a.tensor = sh.tensor ? 1 : 0;
  if (!sh.tensor) return;
  a.a_tscale = a_scale;
  a.b_tscale = b_scale;
  a.h_scale = sh.h_scale;
  a.h_inv = 1.0f / sh.h_scale;
}

hipError_t launch_fc1(const Shape& sh, int variant, const uint8_t* x, const uint8_t* x_sf, const uint8_t* w1,
                      const uint8_t* w1_sf, const int32_t* offsets, const int32_t* row_to_slot, uint8_t* h,
                      uint8_t* h_sf, int32_t* plan, bool plan_ready, hipStream_t s) {
  GemmArgs a{};
  a.A = x; a.A_sf = x_sf; a.row_to_slot = row_to_slot; a.B = w1; a.B_sf = w1_sf;
  // the permute's tile plan covers the routed experts only
  a.offsets = offsets; a.plan = plan_ready && sh.S == 0 ? plan : nullptr; a.h = h; a.h_sf = h_sf;
  a.K = sh.H; a.N = 2 * sh.I; a.I = sh.I; a.k = sh.k; a.EL = sh.EL; a.S = sh.S; a.T = sh.T; a.n_tiles = sh.I / 128;
  a.b_estride = sh.wfmt == 3 ? (long long)2 * sh.I * sh.H * 2
                : sh.wfmt != 1 ? (long long)2 * sh.I * sh.H : (long long)2 * sh.I * sh.H / 2;
  a.bsf_estride = sh.wfmt != 1 ? (long long)(2 * sh.I / 128) * (sh.H / 128) : (long long)2 * sh.I * (sh.H / 32);
  a.act = sh.act; a.clamp = sh.clamp; a.alpha = sh.alpha; a.bias = sh.bias;
  if (sh.sf_packed) {
    a.asf_am = (sh.T + 3) & ~3;
    a.hsf_am = (sh.T * (sh.k + sh.S) + 3) & ~3;
  }
  set_tensor_scales(a, sh, reinterpret_cast<const float*>(x_sf), reinterpret_cast<const float*>(w1_sf));
  const size_t grid = gemm_max_mtiles(sh.T * sh.k, sh.EL, variant, sh.T, sh.S) * (size_t)a.n_tiles;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  return launch_variant<1>(a, sh.wfmt, variant, sh.exact_fc1, grid, s);
}

hipError_t launch_fc2(const Shape& sh, int variant, const uint8_t* h, const uint8_t* h_sf, const uint8_t* w2,
                      const uint8_t* w2_sf, const int32_t* offsets, float* y2, int32_t* plan, bool plan_ready,
                      hipStream_t s) {
  GemmArgs a{};
  a.A = h; a.A_sf = h_sf; a.B = w2; a.B_sf = w2_sf; a.offsets = offsets;
  a.plan = plan_ready && sh.S == 0 ? plan : nullptr;
  a.y2 = y2;
  a.K = sh.I; a.N = sh.H; a.I = sh.I; a.k = sh.k; a.EL = sh.EL; a.S = sh.S; a.T = sh.T;
  a.b_estride = sh.wfmt == 3 ? (long long)sh.H * sh.I * 2 : sh.wfmt != 1 ? (long long)sh.H * sh.I : (long long)sh.H * sh.I / 2;
  a.bsf_estride = sh.wfmt != 1 ? (long long)(sh.H / 128) * (sh.I / 128) : (long long)sh.H * (sh.I / 32);
  if (sh.sf_packed) a.asf_am = (sh.T * (sh.k + sh.S) + 3) & ~3;
  set_tensor_scales(a, sh, nullptr, reinterpret_cast<const float*>(w2_sf));
  const int bn = variant == 0 ? 128 : 256;
  a.n_tiles = (sh.H + bn - 1) / bn;
  const size_t grid = gemm_max_mtiles(sh.T * sh.k, sh.EL, variant, sh.T, sh.S) * (size_t)a.n_tiles;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  return launch_variant<2>(a, sh.wfmt, variant, false, grid, s);
}

}  // namespace moe
