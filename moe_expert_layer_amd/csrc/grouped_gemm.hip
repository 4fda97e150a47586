// Grouped expert GEMMs on gfx950 scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// FC1: for every row r of local expert e (token t = row_to_slot[r] / k)
//        g = x_t . W1[e, n],  u = x_t . W1[e, I + n]   (FP8 E4M3 x with 1x128 UE8M0 scales,
//        W1 FP8 E4M3 with 128x128 UE8M0 scales or MXFP4 with 1x32 UE8M0 scales)
//      then SwiGLU / OAI-SwiGLU and the 1x128 requant to E4M3 + UE8M0 (fused epilogue).
// FC2: Y2[r, m] = h_r . W2[e, m]  (fp32 rows kept for the combine).
//
// Sources: "fix(sm90): support parameterized SwiGLU in FP8 MegaMoE" (Summary: the two
// activation formulas, applied in the FC1 epilogue); "Optimize sm100 version with
// token-aware BM240 tiling, native UE8M0, and direct combine" (description: block
// scales consumed natively by the matrix unit); "DSV4 o_proj: fuse fp8/UE8M0 quantize
// into o_a proj" (Description: FP8 + 1x128 UE8M0 emitted from the GEMM epilogue with
// an amax reduction per block).
//
// Scales are applied by the MFMA itself: each 16x16x128 instruction covers exactly one
// 128-wide K block, so the activation scale is one byte per row and the FP8 weight
// scale one byte per 128-row block; MXFP4 weights carry one byte per (row, 32-K block).
//
// Operand layout of the scaled MFMA (measured on gfx950): lane l works on row/column
// l%16; an FP8 operand holds K bytes [16*(l/16), +16) and [64 + 16*(l/16), +16) of the
// 128-wide block; an FP4 operand holds K elements [32*(l/16), +32) (element 2i in the
// low nibble of byte i); the scale byte of lane l covers row/column l%16 and the
// 32-wide K block l/16; the result lane l holds rows 4*(l/16)+i, column l%16.
//
// Tiles: 128 rows x 256 weight rows (FC1: 128 gate + the matching 128 up rows, i.e. one
// 1x128 requant block of h; FC2: 256 output columns), 4 waves in 2x2, each wave 64 rows
// x 8 column tiles of 16.  K advances 128 per step through one LDS buffer with the
// next step prefetched into registers.  LDS rows are 16-byte-chunk XOR swizzled so the
// MFMA operand reads are bank-conflict free.  Workgroups map to tiles through an
// XCD-aware order (consecutive tiles of one expert run on one XCD and share its L2).
#include <hip/hip_runtime.h>
#include <cstdint>

#include "device_common.hpp"
#include "moe_internal.hpp"

namespace moe {

constexpr int kBM = 128;   // rows per tile
constexpr int kBN = 256;   // weight rows per tile
constexpr int kBK = 128;   // K per step
constexpr int kGroupN = 8; // n-tiles per group in the tile order

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
  long long b_estride;   // bytes per expert of B
  long long bsf_estride; // bytes per expert of B_sf
  int K;                 // contraction length (H for FC1, I for FC2)
  int N;                 // weight rows per expert (2I for FC1, H for FC2)
  int I;                 // intermediate size (FC1 epilogue)
  int k;                 // top-k (FC1 row -> token)
  int EL;
  int n_tiles;
  int act;
  float clamp, alpha, bias;
};

__device__ __forceinline__ int find_expert(const int32_t* __restrict__ plan, int EL, int mt) {
  // last e with plan[e] <= mt  (that expert is non-empty)
  int lo = 0, hi = EL - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (plan[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ uint4 lds_load16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void lds_store16(uint8_t* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ uint4 gload16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Swizzled byte offset of 16-byte chunk c of row r in a [rows][128 B] tile.
__device__ __forceinline__ int sw128(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }
// Swizzled byte offset of 16-byte chunk c of row r in a [rows][64 B] tile.
__device__ __forceinline__ int sw64(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 3)) << 4); }

template <int MODE, int WFMT>  // MODE 1 = FC1, 2 = FC2; WFMT 0 = fp8 block-128, 1 = mxfp4
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(GemmArgs g) {
  constexpr int B_ROWB = WFMT == 0 ? 128 : 64;  // bytes of one weight row per K step
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[kBM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[kBN * B_ROWB];
  __shared__ int lds_bsf[WFMT == 1 ? kBN : 1];
  __shared__ float lds_amax[2][kBM];

  const int total_m = g.plan[g.EL];
  const int total = total_m * g.n_tiles;
  const int bid = blockIdx.x;
  if (bid >= total) return;
  // XCD-aware order: dispatch is round-robin over 8 XCDs, give each XCD a contiguous range.
  int L;
  {
    const int x = bid & 7, p = bid >> 3, q = total >> 3, r = total & 7;
    L = x * q + (x < r ? x : r) + p;
  }
  // expert-major order: tiles of expert e are [plan[e]*NT, plan[e+1]*NT)
  const int e = find_expert(g.plan, g.EL, L / g.n_tiles);
  const int mt_e = g.plan[e + 1] - g.plan[e];
  const int li = L - g.plan[e] * g.n_tiles;
  const int gn = g.n_tiles < kGroupN ? g.n_tiles : kGroupN;
  const int grp = li / (gn * mt_e);
  const int gsz = (g.n_tiles - grp * gn) < gn ? (g.n_tiles - grp * gn) : gn;
  const int idx = li - grp * gn * mt_e;
  const int m_tile = idx / gsz;
  const int n_tile = grp * gn + idx % gsz;

  const int row_begin = g.offsets[e] + m_tile * kBM;
  const int rows = min(kBM, g.offsets[e + 1] - row_begin);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int ksteps = g.K / kBK;

  // ---- global source pointers for this thread's share of the tile loads ----
  // A: chunk q = tid + 256 j -> row (tid >> 3) + 32 j, chunk tid & 7
  const uint8_t* a_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int r = (tid >> 3) + 32 * j;
    if (r >= rows) r = 0;
    const int grow = row_begin + r;
    long long arow;
    if (MODE == 1) arow = g.row_to_slot[grow] / g.k; else arow = grow;
    a_src[j] = g.A + arow * (long long)g.K + ((tid & 7) << 4);
  }
  // B rows of the tile: FC1 local n < 128 -> gate row n0 + n, else up row I + n0 + n - 128
  const uint8_t* b_exp = g.B + (long long)e * g.b_estride;
  const int n0 = MODE == 1 ? n_tile * 128 : n_tile * kBN;
  auto b_row = [&](int n) -> int {
    if (MODE == 1) return n < 128 ? n0 + n : g.I + n0 + (n - 128);
    const int rr = n0 + n;
    return rr < g.N ? rr : g.N - 1;
  };
  constexpr int NBL = WFMT == 0 ? 8 : 4;  // 16-byte B loads per thread per step
  const uint8_t* b_src[NBL];
#pragma unroll
  for (int j = 0; j < NBL; ++j) {
    if (WFMT == 0) {
      const int n = (tid >> 3) + 32 * j;
      b_src[j] = b_exp + (long long)b_row(n) * g.K + ((tid & 7) << 4);
    } else {
      const int n = (tid >> 2) + 64 * j;
      b_src[j] = b_exp + (long long)b_row(n) * (g.K / 2) + ((tid & 3) << 4);
    }
  }
  const uint8_t* bsf_exp = g.B_sf + (long long)e * g.bsf_estride;
  // mxfp4 scales: thread tid owns weight row tid of the tile (4 bytes per K step)
  const uint8_t* bsf_src = WFMT == 1 ? bsf_exp + (long long)b_row(tid) * (g.K / 32) : nullptr;

  // ---- MFMA operand rows owned by this lane ----
  const int lrow = lane & 15, kb = lane >> 4;
  const uint8_t* a_sf_row[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    int r = wm * 64 + mi * 16 + lrow;
    if (r >= rows) r = 0;
    const int grow = row_begin + r;
    long long arow;
    if (MODE == 1) arow = g.row_to_slot[grow] / g.k; else arow = grow;
    a_sf_row[mi] = g.A_sf + arow * (long long)ksteps;
  }
  auto bcol = [&](int ct) -> int {  // first weight row (tile-local) of column tile ct for this wave
    if (MODE == 1) return ct < 4 ? wn * 64 + ct * 16 : 128 + wn * 64 + (ct - 4) * 16;
    return wn * 128 + ct * 16;
  };
  // fp8 weight-scale block rows of this wave (uniform): FC1 gate/up, FC2 one block
  int sfb0, sfb1;
  if (MODE == 1) { sfb0 = n0 / 128; sfb1 = (g.I + n0) / 128; }
  else { sfb0 = min((n0 + wn * 128) / 128, g.N / 128 - 1); sfb1 = sfb0; }

  v4f acc[4][8];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[mi][ct] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 pa[4], pb[NBL];
  int pbsf = 0;
  auto gload_step = [&](int ks) {
#pragma unroll
    for (int j = 0; j < 4; ++j) pa[j] = gload16(a_src[j] + ks * kBK);
#pragma unroll
    for (int j = 0; j < NBL; ++j) pb[j] = gload16(b_src[j] + ks * (WFMT == 0 ? kBK : kBK / 2));
    if (WFMT == 1) pbsf = *reinterpret_cast<const int*>(bsf_src + ks * 4);
  };
  auto lds_store_step = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_store16(lds_a + sw128((tid >> 3) + 32 * j, tid & 7), pa[j]);
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
      if (WFMT == 0) lds_store16(lds_b + sw128((tid >> 3) + 32 * j, tid & 7), pb[j]);
      else lds_store16(lds_b + sw64((tid >> 2) + 64 * j, tid & 3), pb[j]);
    }
    if (WFMT == 1) lds_bsf[tid] = pbsf;
  };

  gload_step(0);
  for (int ks = 0; ks < ksteps; ++ks) {
    __syncthreads();  // previous step's LDS reads are done
    lds_store_step();
    __syncthreads();
    if (ks + 1 < ksteps) gload_step(ks + 1);

    int sa[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) sa[mi] = a_sf_row[mi][ks];
    v8i af[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int r = wm * 64 + mi * 16 + lrow;
      const uint4 lo = lds_load16(lds_a + sw128(r, kb));
      const uint4 hi = lds_load16(lds_a + sw128(r, kb + 4));
      af[mi] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    int sbu0 = 0, sbu1 = 0;
    if (WFMT == 0) {
      sbu0 = bsf_exp[(long long)sfb0 * ksteps + ks];
      sbu1 = bsf_exp[(long long)sfb1 * ksteps + ks];
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const int n = bcol(ct) + lrow;
      v8i bf;
      int sb;
      if (WFMT == 0) {
        const uint4 lo = lds_load16(lds_b + sw128(n, kb));
        const uint4 hi = lds_load16(lds_b + sw128(n, kb + 4));
        bf = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sb = (MODE == 1 && ct >= 4) ? sbu1 : sbu0;
      } else {
        const uint4 q = lds_load16(lds_b + sw64(n, kb));
        bf = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
        sb = (lds_bsf[n] >> (8 * kb)) & 0xff;
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        acc[mi][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bf, acc[mi][ct], 0, WFMT == 0 ? 0 : 4,
                                                                       0, sa[mi], 0, sb);
    }
  }

  if (MODE == 2) {
    // ---- FC2 epilogue: fp32 rows of Y2 ----
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + mi * 16 + 4 * kb + i;
        if (r < rows) {
          float* dst = g.y2 + (long long)(row_begin + r) * g.N;
#pragma unroll
          for (int ct = 0; ct < 8; ++ct) {
            const int col = n0 + bcol(ct) + lrow;
            if (col < g.N) dst[col] = acc[mi][ct][i];
          }
        }
      }
    return;
  }

  // ---- FC1 epilogue: activation, 1x128 amax, UE8M0 scale, E4M3 codes ----
  // lane holds, for rows 4*kb+i of each row tile, h columns wn*64 + c*16 + lrow (c = 0..3)
  float hv[4][4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float gt = acc[mi][c][i], up = acc[mi][c + 4][i];
        float hh;
        if (g.act == 1) {
          gt = fminf(gt, g.clamp);
          up = fminf(fmaxf(up, -g.clamp), g.clamp);
          hh = gt * sigmoidf_(g.alpha * gt) * (up + g.bias);
        } else {
          hh = gt * sigmoidf_(gt) * up;
        }
        hv[mi][c][i] = hh;
      }
  float am[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = fmaxf(fmaxf(fabsf(hv[mi][0][i]), fabsf(hv[mi][1][i])), fmaxf(fabsf(hv[mi][2][i]), fabsf(hv[mi][3][i])));
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
      am[mi][i] = m;
    }
  if (lrow == 0) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_amax[wn][wm * 64 + mi * 16 + 4 * kb + i] = am[mi][i];
  }
  __syncthreads();  // also: every wave is past its last LDS operand read
  uint8_t* lds_h = lds_b;  // [128 rows][128 B] staging of the E4M3 codes
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + mi * 16 + 4 * kb + i;
      const float amax = fmaxf(lds_amax[0][r], lds_amax[1][r]);
      const int byte = ue8m0_for_amax(amax);
      const float inv = inv_scale_of(byte);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int code = __builtin_amdgcn_cvt_pk_fp8_f32(hv[mi][c][i] * inv, 0.0f, 0, false) & 0xff;
        lds_h[r * 128 + wn * 64 + c * 16 + lrow] = (uint8_t)code;
      }
      if (wn == 0 && lrow == 0 && r < rows)
        g.h_sf[(long long)(row_begin + r) * (g.I / 128) + n_tile] = (uint8_t)byte;
    }
  __syncthreads();
  // coalesced 16-byte stores of the code tile
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (tid >> 3) + 32 * j, c = tid & 7;
    if (r < rows)
      *reinterpret_cast<uint4*>(g.h + (long long)(row_begin + r) * g.I + n0 + c * 16) =
          *reinterpret_cast<const uint4*>(lds_h + r * 128 + c * 16);
  }
}

// plan[e] = number of m-tiles of experts before e; plan[EL] = all m-tiles
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int EL, int bm,
                                                    int32_t* __restrict__ plan) {
  __shared__ int a[2 * 1024 + 2];
  for (int i = threadIdx.x; i < 2048; i += 1024) a[i] = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < EL; e += 1024) a[e] = (offsets[e + 1] - offsets[e] + bm - 1) / bm;
  __syncthreads();
  block_exclusive_scan_2048(a);
  for (int e = threadIdx.x; e <= EL; e += 1024) plan[e] = a[e];
}

int gemm_block_m(int /*variant*/) { return kBM; }

size_t gemm_max_mtiles(int rows_cap, int EL, int variant) {
  const int bm = gemm_block_m(variant);
  // sum_e ceil(c_e / bm) <= (R + EL * (bm - 1)) / bm with R <= rows_cap
  return ((size_t)rows_cap + (size_t)EL * (bm - 1)) / bm;
}

static hipError_t launch_gemm(const GemmArgs& a, int mode, int wfmt, size_t max_mt, hipStream_t s) {
  const size_t grid = max_mt * (size_t)a.n_tiles;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  dim3 gr((unsigned)grid), bl(256);
  if (mode == 1 && wfmt == 0) grouped_gemm_kernel<1, 0><<<gr, bl, 0, s>>>(a);
  else if (mode == 1) grouped_gemm_kernel<1, 1><<<gr, bl, 0, s>>>(a);
  else if (wfmt == 0) grouped_gemm_kernel<2, 0><<<gr, bl, 0, s>>>(a);
  else grouped_gemm_kernel<2, 1><<<gr, bl, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fc1(const Shape& sh, int variant, const uint8_t* x, const uint8_t* x_sf, const uint8_t* w1,
                      const uint8_t* w1_sf, const int32_t* offsets, const int32_t* row_to_slot, uint8_t* h,
                      uint8_t* h_sf, int32_t* plan, hipStream_t s) {
  plan_kernel<<<1, 1024, 0, s>>>(offsets, sh.EL, gemm_block_m(variant), plan);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  GemmArgs a{};
  a.A = x; a.A_sf = x_sf; a.row_to_slot = row_to_slot; a.B = w1; a.B_sf = w1_sf;
  a.offsets = offsets; a.plan = plan; a.h = h; a.h_sf = h_sf;
  a.K = sh.H; a.N = 2 * sh.I; a.I = sh.I; a.k = sh.k; a.EL = sh.EL; a.n_tiles = sh.I / 128;
  a.b_estride = sh.wfmt == 0 ? (long long)2 * sh.I * sh.H : (long long)2 * sh.I * sh.H / 2;
  a.bsf_estride = sh.wfmt == 0 ? (long long)(2 * sh.I / 128) * (sh.H / 128) : (long long)2 * sh.I * (sh.H / 32);
  a.act = sh.act; a.clamp = sh.clamp; a.alpha = sh.alpha; a.bias = sh.bias;
  return launch_gemm(a, 1, sh.wfmt, gemm_max_mtiles(sh.T * sh.k, sh.EL, variant), s);
}

hipError_t launch_fc2(const Shape& sh, int variant, const uint8_t* h, const uint8_t* h_sf, const uint8_t* w2,
                      const uint8_t* w2_sf, const int32_t* offsets, float* y2, int32_t* plan, hipStream_t s) {
  plan_kernel<<<1, 1024, 0, s>>>(offsets, sh.EL, gemm_block_m(variant), plan);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  GemmArgs a{};
  a.A = h; a.A_sf = h_sf; a.B = w2; a.B_sf = w2_sf; a.offsets = offsets; a.plan = plan; a.y2 = y2;
  a.K = sh.I; a.N = sh.H; a.I = sh.I; a.k = sh.k; a.EL = sh.EL; a.n_tiles = (sh.H + kBN - 1) / kBN;
  a.b_estride = sh.wfmt == 0 ? (long long)sh.H * sh.I : (long long)sh.H * sh.I / 2;
  a.bsf_estride = sh.wfmt == 0 ? (long long)(sh.H / 128) * (sh.I / 128) : (long long)sh.H * (sh.I / 32);
  return launch_gemm(a, 2, sh.wfmt, gemm_max_mtiles(sh.T * sh.k, sh.EL, variant), s);
}

}  // namespace moe
