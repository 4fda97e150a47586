// C ABI of the MoE expert layer: validation, workspace layout and launch sequencing.
//
// The entry points follow the split the pages describe for the fused layer's API: an
// activation kind plus clamp / alpha / up_bias with standard-SwiGLU defaults
// ("fix(sm90): support parameterized SwiGLU in FP8 MegaMoE": Changes, Compatibility),
// a buffer-sizing call next to the execution call (same page, Changes; "Pull Style
// Cutedsl Megakernel": Layout, config -> buffer -> compute entry), and a contract
// check before launching on raw pointers ("DSV4 o_proj: fuse fp8/UE8M0 quantize ...":
// review of the raw-pointer launch).  Every counter a kernel reads is produced inside
// the same call, so a captured graph replays correctly (DeepGEMM PR #451 note on
// resetting combine readiness for graph replay).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/moe_expert_layer.h"
#include "moe_internal.hpp"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace regions (byte offsets from the workspace base).
struct Layout {
  size_t ids, w, counts, offsets, r2s, s2r, chunk_cnt, chunk_base, plan1, h, h_sf, y2, total;
};

Layout make_layout(const moe_layer_desc& d) {
  const size_t cap = (size_t)d.num_tokens * d.topk;
  const size_t NB = (size_t)d.num_local + 1;
  const size_t nchunks = (cap + moe::kPermChunk - 1) / moe::kPermChunk;
  Layout L{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t o = at;
    at = align_up(at + bytes);
    return o;
  };
  L.ids = take(cap * 4);
  L.w = take(cap * 4);
  L.counts = take((size_t)d.num_local * 4);
  L.offsets = take(NB * 4);
  L.r2s = take(cap * 4);
  L.s2r = take(cap * 4);
  L.chunk_cnt = take(nchunks * NB * 4);
  L.chunk_base = take(nchunks * NB * 4);
  L.plan1 = take(NB * 4);
  const size_t hrows = cap + (size_t)d.num_shared * d.num_tokens;  // routed rows, then shared experts' rows
  L.h = take(hrows * (size_t)d.inter * (d.weight_format == MOE_W_BF16 ? 2 : 1));
  // row-major bytes, or packed int32 words [ceil(groups / 4)][rows rounded up to 4]
  L.h_sf = take(d.scale_layout == MOE_SF_PACKED_MN ? (size_t)4 * ((d.inter / 128 + 3) / 4) * ((hrows + 3) / 4 * 4)
                                                    : hrows * (size_t)(d.inter / 128));
  L.y2 = take(hrows * (size_t)d.hidden * 4);
  L.total = at;
  return L;
}

moe_status check_desc(const moe_layer_desc* d) {
  if (!d) return fail(MOE_ERR_NULL, "desc is NULL");
  if (d->num_tokens < 0) return fail(MOE_ERR_INVALID_DESC, "num_tokens %d < 0", d->num_tokens);
  if (d->hidden <= 0 || d->hidden % 128) return fail(MOE_ERR_INVALID_DESC, "hidden %d not a positive multiple of 128", d->hidden);
  if (d->inter <= 0 || d->inter % 128) return fail(MOE_ERR_INVALID_DESC, "inter %d not a positive multiple of 128", d->inter);
  if (d->num_experts < 1 || d->num_experts > moe::kMaxExperts)
    return fail(MOE_ERR_INVALID_DESC, "num_experts %d outside [1, %d]", d->num_experts, moe::kMaxExperts);
  if (d->num_local < 1 || d->local_begin < 0 || (long long)d->local_begin + d->num_local > d->num_experts)
    return fail(MOE_ERR_INVALID_DESC, "local range [%d, %d + %d) not inside [0, %d)", d->local_begin, d->local_begin,
                d->num_local, d->num_experts);
  if (d->topk < 1 || d->topk > moe::kMaxTopk || d->topk > d->num_experts)
    return fail(MOE_ERR_INVALID_DESC, "topk %d outside [1, min(num_experts, %d)]", d->topk, moe::kMaxTopk);
  if ((long long)d->num_tokens * d->topk >= (1LL << 31))
    return fail(MOE_ERR_INVALID_DESC, "num_tokens * topk must be < 2^31");
  if ((long long)d->num_tokens * d->topk * d->hidden >= (1LL << 46))
    return fail(MOE_ERR_INVALID_DESC, "num_tokens * topk * hidden too large");
  if (d->weight_format != MOE_W_FP8_E4M3_B128 && d->weight_format != MOE_W_MXFP4_E2M1_B32 &&
      d->weight_format != MOE_W_FP8_E5M2_B128 && d->weight_format != MOE_W_BF16)
    return fail(MOE_ERR_INVALID_DESC, "weight_format %d unknown", d->weight_format);
  if (d->activation != MOE_ACT_SWIGLU && d->activation != MOE_ACT_SWIGLU_OAI)
    return fail(MOE_ERR_INVALID_DESC, "activation %d unknown", d->activation);
  if (d->activation == MOE_ACT_SWIGLU_OAI) {
    if (std::isnan(d->act_clamp) || !(d->act_clamp > 0.f))
      return fail(MOE_ERR_INVALID_DESC, "act_clamp must be > 0 (or +inf)");
    if (!std::isfinite(d->act_alpha) || !std::isfinite(d->act_up_bias))
      return fail(MOE_ERR_INVALID_DESC, "act_alpha / act_up_bias must be finite");
  }
  if (d->variant < -1 || d->variant > 2) return fail(MOE_ERR_INVALID_DESC, "variant %d unknown", d->variant);
  if (d->num_shared < 0 || d->num_shared > moe::kMaxShared)
    return fail(MOE_ERR_INVALID_DESC, "num_shared %d outside [0, %d]", d->num_shared, moe::kMaxShared);
  if ((long long)d->num_tokens * (d->topk + d->num_shared) >= (1LL << 31))
    return fail(MOE_ERR_INVALID_DESC, "num_tokens * (topk + num_shared) must be < 2^31");
  if (d->scale_mode != MOE_SCALE_BLOCK && d->scale_mode != MOE_SCALE_TENSOR)
    return fail(MOE_ERR_INVALID_DESC, "scale_mode %d unknown", d->scale_mode);
  if (d->scale_mode == MOE_SCALE_TENSOR) {
    if (d->weight_format == MOE_W_MXFP4_E2M1_B32 || d->weight_format == MOE_W_BF16)
      return fail(MOE_ERR_INVALID_DESC, "per-tensor scaling needs FP8 weights");
    if (!std::isfinite(d->h_scale) || !(d->h_scale > 0.f))
      return fail(MOE_ERR_INVALID_DESC, "h_scale must be finite and > 0");
  }
  if (d->scale_layout != MOE_SF_ROW_MAJOR && d->scale_layout != MOE_SF_PACKED_MN)
    return fail(MOE_ERR_INVALID_DESC, "scale_layout %d unknown", d->scale_layout);
  if (d->scale_layout == MOE_SF_PACKED_MN && (d->scale_mode != MOE_SCALE_BLOCK || d->weight_format == MOE_W_BF16))
    return fail(MOE_ERR_INVALID_DESC, "packed scale layout needs blockwise UE8M0 scales");
  if (!moe::gemm_supports(d->hidden, d->inter))
    return fail(MOE_ERR_UNSUPPORTED, "hidden %d / inter %d above the supported 8192", d->hidden, d->inter);
  const long long x_bytes = (long long)d->num_tokens * d->hidden * (d->weight_format == MOE_W_BF16 ? 2 : 1);
  if (x_bytes >= (1LL << 32))
    return fail(MOE_ERR_UNSUPPORTED, "x of %lld bytes is 4 GiB or more", x_bytes);
  return MOE_OK;
}

bool misaligned(const void* p, size_t a) { return ((uintptr_t)p) % a != 0; }

moe_status check_ws(const moe_layer_desc* d, const void* ws, size_t ws_bytes) {
  const Layout L = make_layout(*d);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (misaligned(ws, kAlign)) return fail(MOE_ERR_MISALIGNED, "workspace not 256-byte aligned");
  if (ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L.total);
  return MOE_OK;
}

// Device check: gfx950 only; cached per device.
std::mutex g_dev_mu;
int g_dev_state[64];  // 0 unknown, 1 ok, 2 unsupported

moe_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_dev_state[dev] = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    if (g_dev_state[dev] == 2) return fail(MOE_ERR_UNSUPPORTED, "device arch %s is not gfx950", p.gcnArchName);
  }
  if (g_dev_state[dev] == 2) return fail(MOE_ERR_UNSUPPORTED, "device is not gfx950");
  return MOE_OK;
}

// Whether FC1 sums exactly: BF16 MFMAs on operands converted in registers instead of the scaled
// FP8 MFMA (see the GEMM source).  That costs conversion instructions and half the matrix-core
// rate, which is free where the GEMM streams weights: at most 48 rows per local expert on
// average (the 32-row tile regime, fewer than ~100 FLOPs per weight byte), or a layer whose FC1
// is at most 2^33 FLOPs (a few microseconds of work, launch- and latency-bound).  Larger layers
// keep the scaled FP8 MFMA (measured on the 512-token, 2048-hidden OAI share: the exact FC1 took
// 37.9 instead of 25.3 us).
bool exact_fc1(const moe_layer_desc& d) {
  if (d.weight_format == MOE_W_BF16) return false;
  const long long rows = (long long)d.num_tokens * (d.topk < d.num_local ? d.topk : d.num_local);
  const long long all_rows = rows + (long long)d.num_shared * d.num_tokens;
  const double fc1_flops = 4.0 * (double)all_rows * d.hidden * d.inter;
  return rows <= 48LL * d.num_local || fc1_flops <= 8589934592.0;
}

moe::Shape shape_of(const moe_layer_desc& d) {
  moe::Shape s;
  s.T = d.num_tokens; s.H = d.hidden; s.I = d.inter; s.E = d.num_experts; s.e0 = d.local_begin;
  s.EL = d.num_local; s.k = d.topk; s.wfmt = d.weight_format; s.act = d.activation;
  s.S = d.num_shared;
  s.exact_fc1 = exact_fc1(d);
  s.sf_packed = d.scale_layout == MOE_SF_PACKED_MN;
  s.tensor = d.scale_mode == MOE_SCALE_TENSOR;
  s.h_scale = s.tensor ? d.h_scale : 1.f;
  if (d.activation == MOE_ACT_SWIGLU_OAI) {
    s.clamp = d.act_clamp; s.alpha = d.act_alpha; s.bias = d.act_up_bias;
  } else {
    s.clamp = INFINITY; s.alpha = 1.f; s.bias = 0.f;
  }
  return s;
}

// Tile variant: 256-row tiles once an expert can hold 256 rows on average (T * min(k, E_loc)
// rows spread over E_loc experts is the most the routing can give them), else 128-row tiles.
// Chosen from the descriptor only, so no host synchronisation is needed.
int pick_variant(const moe_layer_desc& d) {
  if (d.variant >= 0) return d.variant;
  // the routing is on the device: the bound T * min(k, E_loc) on the local rows stands in
  // for their count; tiles are sized for its average per local expert
  const long long most_rows = (long long)d.num_tokens * (d.topk < d.num_local ? d.topk : d.num_local);
  if (most_rows >= 256LL * d.num_local) return 1;
  if (most_rows <= 48LL * d.num_local) return 2;
  return 0;
}

#define MOE_TRY_HIP(call)                                                            \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) return fail(MOE_ERR_DEVICE, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

template <typename P>
P* region(void* ws, size_t off) { return reinterpret_cast<P*>(static_cast<uint8_t*>(ws) + off); }

moe_status run_route_permute(const moe_layer_desc& d, const Layout& L, const float* logits, int32_t* ids, float* w,
                             int32_t* counts, int32_t* offsets, int32_t* r2s, int32_t* s2r, void* ws,
                             hipStream_t s) {
  MOE_TRY_HIP(moe::launch_route_topk(logits, d.num_tokens, d.num_experts, d.topk, ids, w, s));
  MOE_TRY_HIP(moe::launch_permute(ids, d.num_tokens * d.topk, d.local_begin, d.num_local,
                                  region<int32_t>(ws, L.chunk_cnt), region<int32_t>(ws, L.chunk_base), counts,
                                  offsets, r2s, s2r, moe::gemm_block_m(pick_variant(d)),
                                  region<int32_t>(ws, L.plan1), s));
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL";
    case MOE_ERR_INVALID_DESC: return "MOE_ERR_INVALID_DESC";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    default: return "MOE_STATUS_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_desc_defaults(moe_layer_desc* d) {
  if (!d) return fail(MOE_ERR_NULL, "desc is NULL");
  std::memset(d, 0, sizeof *d);
  d->weight_format = MOE_W_FP8_E4M3_B128;
  d->activation = MOE_ACT_SWIGLU;
  d->act_clamp = INFINITY;
  d->act_alpha = 1.0f;
  d->act_up_bias = 0.0f;
  d->variant = -1;
  d->scale_mode = MOE_SCALE_BLOCK;
  d->h_scale = 1.0f;
  d->scale_layout = MOE_SF_ROW_MAJOR;
  return ok();
}

moe_status moe_workspace_size(const moe_layer_desc* d, size_t* bytes) {
  if (moe_status st = check_desc(d)) return st;
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  *bytes = make_layout(*d).total;
  return ok();
}

moe_status moe_route_permute(const moe_layer_desc* d, const float* logits, int32_t* ids, float* w, int32_t* counts,
                             int32_t* offsets, int32_t* r2s, int32_t* s2r, void* ws, size_t ws_bytes,
                             void* stream) {
  if (moe_status st = check_desc(d)) return st;
  if (d->num_tokens == 0) return ok();
  if (!logits || !ids || !w || !counts || !offsets || !r2s || !s2r)
    return fail(MOE_ERR_NULL, "logits/topk_ids/topk_w/counts/offsets/row_to_slot/slot_to_row NULL");
  if (misaligned(logits, 16)) return fail(MOE_ERR_MISALIGNED, "logits not 16-byte aligned");
  if (moe_status st = check_ws(d, ws, ws_bytes)) return st;
  if (moe_status st = check_device()) return st;
  const Layout L = make_layout(*d);
  if (moe_status st = run_route_permute(*d, L, logits, ids, w, counts, offsets, r2s, s2r, ws, (hipStream_t)stream))
    return st;
  return ok();
}

moe_status moe_grouped_fc1_swiglu(const moe_layer_desc* d, const uint8_t* x, const uint8_t* x_sf, const uint8_t* w1,
                                  const uint8_t* w1_sf, const int32_t* offsets, const int32_t* r2s, uint8_t* h,
                                  uint8_t* h_sf, void* ws, size_t ws_bytes, void* stream) {
  if (moe_status st = check_desc(d)) return st;
  if (d->num_tokens == 0) return ok();
  const bool tensor = d->scale_mode == MOE_SCALE_TENSOR, bf16 = d->weight_format == MOE_W_BF16;
  if (!x || (!x_sf && !bf16) || !w1 || (!w1_sf && !bf16) || !offsets || !r2s || !h || (!h_sf && !tensor && !bf16))
    return fail(MOE_ERR_NULL, "a required pointer is NULL");
  if (misaligned(x, 16) || misaligned(w1, 16) || misaligned(h, 16) || misaligned(x_sf, 16) || misaligned(w1_sf, 16))
    return fail(MOE_ERR_MISALIGNED, "x / x_sf / w1 / w1_sf / h not 16-byte aligned");
  if (moe_status st = check_ws(d, ws, ws_bytes)) return st;
  if (moe_status st = check_device()) return st;
  const moe::Shape sh = shape_of(*d);
  MOE_TRY_HIP(moe::launch_fc1(sh, pick_variant(*d), x, x_sf, w1, w1_sf, offsets, r2s, h, h_sf,
                              nullptr, false, (hipStream_t)stream));
  return ok();
}

moe_status moe_grouped_fc2_combine(const moe_layer_desc* d, const uint8_t* h, const uint8_t* h_sf, const uint8_t* w2,
                                   const uint8_t* w2_sf, const int32_t* offsets, const int32_t* r2s,
                                   const int32_t* s2r, const float* w, uint16_t* y, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (moe_status st = check_desc(d)) return st;
  if (d->num_tokens == 0) return ok();
  const bool tensor = d->scale_mode == MOE_SCALE_TENSOR, bf16 = d->weight_format == MOE_W_BF16;
  if (!h || (!h_sf && !tensor && !bf16) || !w2 || (!w2_sf && !bf16) || !offsets || !r2s || !s2r || !w || !y)
    return fail(MOE_ERR_NULL, "a required pointer is NULL");
  if (misaligned(h, 16) || misaligned(w2, 16) || misaligned(y, 16) || misaligned(h_sf, 16) || misaligned(w2_sf, 16))
    return fail(MOE_ERR_MISALIGNED, "h / h_sf / w2 / w2_sf / y not 16-byte aligned");
  if (moe_status st = check_ws(d, ws, ws_bytes)) return st;
  if (moe_status st = check_device()) return st;
  const Layout L = make_layout(*d);
  const moe::Shape sh = shape_of(*d);
  float* y2 = region<float>(ws, L.y2);
  MOE_TRY_HIP(moe::launch_fc2(sh, pick_variant(*d), h, h_sf, w2, w2_sf, offsets, y2, nullptr,
                              false, (hipStream_t)stream));
  MOE_TRY_HIP(moe::launch_combine(y2, s2r, w, d->num_tokens, d->hidden, d->topk, offsets + d->num_local,
                                  d->num_shared, y, (hipStream_t)stream));
  return ok();
}

}  // extern "C"

namespace {

moe_status check_layer_args(const moe_layer_desc* d, const float* logits, const uint8_t* x, const uint8_t* x_sf,
                            const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2, const uint8_t* w2_sf,
                            const uint16_t* y) {
  const bool bf16 = d->weight_format == MOE_W_BF16;  // no scale tensors
  if (!logits || !x || (!x_sf && !bf16) || !w1 || (!w1_sf && !bf16) || !w2 || (!w2_sf && !bf16) || !y)
    return fail(MOE_ERR_NULL, "a required pointer is NULL");
  if (misaligned(logits, 16) || misaligned(x, 16) || misaligned(x_sf, 16) || misaligned(w1, 16) ||
      misaligned(w1_sf, 16) || misaligned(w2, 16) || misaligned(w2_sf, 16) || misaligned(y, 16))
    return fail(MOE_ERR_MISALIGNED, "an input/output pointer is not 16-byte aligned");
  return MOE_OK;
}

// The whole layer on a validated descriptor, arguments and workspace.
moe_status run_layer(const moe_layer_desc* d, const float* logits, const uint8_t* x, const uint8_t* x_sf,
                     const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2, const uint8_t* w2_sf, uint16_t* y,
                     int32_t* opt_ids, float* opt_w, int32_t* opt_counts, int32_t* opt_offsets, int32_t* opt_r2s,
                     int32_t* opt_s2r, void* ws, hipStream_t s) {
  const Layout L = make_layout(*d);
  const moe::Shape sh = shape_of(*d);
  int32_t* ids = opt_ids ? opt_ids : region<int32_t>(ws, L.ids);
  float* w = opt_w ? opt_w : region<float>(ws, L.w);
  int32_t* counts = opt_counts ? opt_counts : region<int32_t>(ws, L.counts);
  int32_t* offsets = opt_offsets ? opt_offsets : region<int32_t>(ws, L.offsets);
  int32_t* r2s = opt_r2s ? opt_r2s : region<int32_t>(ws, L.r2s);
  int32_t* s2r = opt_s2r ? opt_s2r : region<int32_t>(ws, L.s2r);
  uint8_t* h = region<uint8_t>(ws, L.h);
  uint8_t* h_sf = region<uint8_t>(ws, L.h_sf);
  float* y2 = region<float>(ws, L.y2);
  const int variant = pick_variant(*d);
  if (moe_status st = run_route_permute(*d, L, logits, ids, w, counts, offsets, r2s, s2r, ws, s)) return st;
  // the permute wrote the tile plan of these offsets (plan1) for this variant's tile rows
  MOE_TRY_HIP(moe::launch_fc1(sh, variant, x, x_sf, w1, w1_sf, offsets, r2s, h, h_sf,
                              region<int32_t>(ws, L.plan1), true, s));
  MOE_TRY_HIP(moe::launch_fc2(sh, variant, h, h_sf, w2, w2_sf, offsets, y2, region<int32_t>(ws, L.plan1), true, s));
  MOE_TRY_HIP(moe::launch_combine(y2, s2r, w, d->num_tokens, d->hidden, d->topk, offsets + d->num_local,
                                  d->num_shared, y, s));
  return ok();
}

}  // namespace

// Scratch of the no-allocation entry point: one array per device, held by the loaded code
// object until the process ends.  In host code `scratch` names a host-side stand-in, not
// the device array; the device address is looked up once per device (with that device
// current) and only that address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr size_t kStaticScratchBytes = MOE_STATIC_SCRATCH_BYTES;
std::mutex g_scratch_mu;
void* g_scratch_dev[64];  // device address of `scratch` per device index, nullptr until looked up

moe_status static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MOE_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer(const moe_layer_desc* d, const float* logits, const uint8_t* x, const uint8_t* x_sf,
                     const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2, const uint8_t* w2_sf, uint16_t* y,
                     int32_t* opt_ids, float* opt_w, int32_t* opt_counts, int32_t* opt_offsets, int32_t* opt_r2s,
                     int32_t* opt_s2r, void* ws, size_t ws_bytes, void* stream) {
  if (moe_status st = check_desc(d)) return st;
  if (d->num_tokens == 0) return ok();
  if (moe_status st = check_layer_args(d, logits, x, x_sf, w1, w1_sf, w2, w2_sf, y)) return st;
  if (moe_status st = check_ws(d, ws, ws_bytes)) return st;
  if (moe_status st = check_device()) return st;
  return run_layer(d, logits, x, x_sf, w1, w1_sf, w2, w2_sf, y, opt_ids, opt_w, opt_counts, opt_offsets, opt_r2s,
                   opt_s2r, ws, (hipStream_t)stream);
}

size_t moe_static_scratch_bytes(void) { return kStaticScratchBytes; }

moe_status moe_layer_static(const moe_layer_desc* d, const float* logits, const uint8_t* x, const uint8_t* x_sf,
                            const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2, const uint8_t* w2_sf,
                            uint16_t* y, int32_t* opt_ids, float* opt_w, int32_t* opt_counts, int32_t* opt_offsets,
                            int32_t* opt_r2s, int32_t* opt_s2r, void* stream) {
  if (moe_status st = check_desc(d)) return st;
  if (d->num_tokens == 0) return ok();
  if (moe_status st = check_layer_args(d, logits, x, x_sf, w1, w1_sf, w2, w2_sf, y)) return st;
  const size_t need = make_layout(*d).total;
  if (need > kStaticScratchBytes)
    return fail(MOE_ERR_WORKSPACE, "layer needs %zu bytes of scratch, more than the static array's %zu; use moe_layer "
                "with a caller-owned workspace", need, kStaticScratchBytes);
  if (moe_status st = check_device()) return st;
  void* ws = nullptr;
  if (moe_status st = static_scratch(&ws)) return st;
  return run_layer(d, logits, x, x_sf, w1, w1_sf, w2, w2_sf, y, opt_ids, opt_w, opt_counts, opt_offsets, opt_r2s,
                   opt_s2r, ws, (hipStream_t)stream);
}

moe_status moe_quantize_act(const moe_layer_desc* d, const uint16_t* x_bf16, uint8_t* x, uint8_t* x_sf,
                            void* stream) {
  if (moe_status st = check_desc(d)) return st;
  if (d->num_tokens == 0) return ok();
  if (d->scale_mode == MOE_SCALE_TENSOR)
    return fail(MOE_ERR_UNSUPPORTED, "moe_quantize_act makes blockwise scales only");
  if (!x_bf16 || !x || !x_sf) return fail(MOE_ERR_NULL, "x_bf16/x/x_sf NULL");
  if (misaligned(x_bf16, 16) || misaligned(x, 16)) return fail(MOE_ERR_MISALIGNED, "x_bf16/x not 16-byte aligned");
  if (moe_status st = check_device()) return st;
  MOE_TRY_HIP(moe::launch_quantize_act(x_bf16, (long long)d->num_tokens * d->hidden, x, x_sf, (hipStream_t)stream));
  return ok();
}

namespace {
moe_status check_pack_args(int32_t rows, int32_t groups, const void* a, const void* b, const void* packed) {
  if (rows < 0 || groups < 1 || (long long)rows * groups >= (1LL << 31))
    return fail(MOE_ERR_INVALID_DESC, "rows %d / groups %d out of range", rows, groups);
  if (rows > 0 && (!a || !b)) return fail(MOE_ERR_NULL, "sf/packed NULL");
  if (misaligned(packed, 4)) return fail(MOE_ERR_MISALIGNED, "packed not 4-byte aligned");
  return MOE_OK;
}
}  // namespace

moe_status moe_pack_scales(int32_t rows, int32_t groups, const uint8_t* sf, int32_t* packed, void* stream) {
  if (moe_status st = check_pack_args(rows, groups, sf, packed, packed)) return st;
  if (rows == 0) return ok();
  if (moe_status st = check_device()) return st;
  MOE_TRY_HIP(moe::launch_pack_scales(sf, rows, groups, packed, (hipStream_t)stream));
  return ok();
}

moe_status moe_unpack_scales(int32_t rows, int32_t groups, const int32_t* packed, uint8_t* sf, void* stream) {
  if (moe_status st = check_pack_args(rows, groups, packed, sf, packed)) return st;
  if (rows == 0) return ok();
  if (moe_status st = check_device()) return st;
  MOE_TRY_HIP(moe::launch_unpack_scales(packed, rows, groups, sf, (hipStream_t)stream));
  return ok();
}

}  // extern "C"
