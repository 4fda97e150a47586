/*
 * moe_expert_layer.h — C ABI of the MI355X (gfx950) MoE expert-layer library.
 *
 * One call of the layer runs, on one GPU's share of the experts:
 *   route    top-k of each token's routing logits + softmax weights over the k chosen
 *   permute  group the local (token, slot) pairs by local expert, stable by slot id
 *   FC1      gate/up grouped GEMM, FP8 E4M3 activations (1x128 UE8M0 scales) against
 *            FP8 E4M3 weights (128x128 UE8M0 scales) or MXFP4 weights (E2M1, UE8M0 per 32)
 *   act      SwiGLU or parameterised OAI-SwiGLU (clamp, sigmoid alpha, up bias)
 *   requant  the intermediate to FP8 E4M3 with one UE8M0 scale per 1x128 block
 *   FC2      down-projection grouped GEMM
 *   combine  top-k weighted sum back into token order (no atomics, fixed slot order)
 *
 * Sources: the fused "Mega MoE" expert layer as described by DeepGEMM PR #445
 * ("fix(sm90): support parameterized SwiGLU in FP8 MegaMoE": Summary, Changes,
 * Compatibility), DeepGEMM PR #386 ("... native UE8M0, and direct combine":
 * description), FlashInfer's "Pull Style Cutedsl Megakernel" (Layout: FC1/FC2 fused
 * scheduling and a top-k reduce), and TensorRT-LLM PR #16346 ("DSV4 o_proj: fuse
 * fp8/UE8M0 quantize ...": Description, 1x128 UE8M0 requant with an amax per block).
 *
 * Conventions for every entry point
 *   - Memory: every tensor pointer is a device pointer owned by the caller; the
 *     library never allocates, frees or keeps pointers after a call returns.  The
 *     workspace (scratch) is caller-owned device memory of at least
 *     moe_workspace_size() bytes, 256-byte aligned; its contents on entry are
 *     ignored (every counter the kernels use is initialised inside the call).
 *   - Layouts are row-major and dense:
 *       logits      float32 [T, E_tot]
 *       x           E4M3 bytes [T, H]            x_sf   UE8M0 bytes [T, H/128] (or packed, see
 *                                                moe_sf_layout)
 *       w1 (fp8)    E4M3 or E5M2 bytes [E_loc, 2I, H]  w1_sf  UE8M0 [E_loc, 2I/128, H/128]
 *       w1 (mxfp4)  E2M1 pairs [E_loc, 2I, H/2]        w1_sf  UE8M0 [E_loc, 2I, H/32]
 *       w2 (fp8)    E4M3 or E5M2 bytes [E_loc, H, I]   w2_sf  UE8M0 [E_loc, H/128, I/128]
 *       w2 (mxfp4)  E2M1 pairs [E_loc, H, I/2]         w2_sf  UE8M0 [E_loc, H, I/32]
 *     W1 rows [0, I) are the gate projection and rows [I, 2I) the up projection.
 *     MXFP4: element 2i of a K-row is the low nibble of byte i.  E4M3 is OCP E4M3FN,
 *     E5M2 is OCP E5M2 (weights only; x and h are always E4M3).
 *     UE8M0 byte b is 2^(b-127); 255 (NaN) is not allowed.
 *       topk_ids    int32 [T, k]  slot j = j-th largest logit (ties: lower expert id)
 *       topk_w      float32 [T, k] softmax over the k chosen logits (computed in fp64)
 *       counts      int32 [E_loc]   rows per local expert
 *       offsets     int32 [E_loc+1] exclusive scan of counts; offsets[E_loc] = R
 *       row_to_slot int32 [T*k]  rows [0, R) hold slot ids s = t*k + j, rest -1
 *       slot_to_row int32 [T*k]  row of slot s, or -1 when expert ids[s] is not local
 *       h           E4M3 bytes [T*k + S*T, I] (rows [0, R + S*T) written), h_sf UE8M0
 *                   [T*k + S*T, I/128]; S = num_shared (0 by default)
 *       y           bfloat16 bits [T, H]; with S = 0, tokens with no local slot get +0
 *   - Requant rule: per 1x128 block, scale 2^e with the smallest integer e such that
 *     448 * 2^e >= amax (byte 127 for an all-zero block), codes = E4M3 round to
 *     nearest even of h * 2^-e.
 *   - Per-tensor scaling (scale_mode = MOE_SCALE_TENSOR; FP8 weight formats only) replaces
 *     every UE8M0 scale tensor with float32 scales (the Hopper kernel's per-tensor mode,
 *     Pull Style Cutedsl Megakernel, Layout section):
 *       x_sf        float32 [1]       x = code * x_sf[0]
 *       w1_sf       float32 [E_loc]   W1[e] = code * w1_sf[e]   (w2_sf likewise)
 *       h           E4M3 codes of h / h_scale, round to nearest even, saturated to +-448;
 *                   h_scale (> 0, finite) is the static scale in the descriptor and
 *                   h_sf is neither read nor written (it may be NULL)
 *     Non-finite or non-positive tensor scales give unspecified results.
 *   - BF16 layer (weight_format = MOE_W_BF16; the pages list BF16 Mega MoE builds beside
 *     the FP8/FP4 ones, "Sync upstream through PR #441"): x is bfloat16 bits [T, H], w1
 *     bfloat16 [E_loc, 2I, H], w2 bfloat16 [E_loc, H, I], h bfloat16 [rows, I] (each
 *     pointer still passed as bytes: rows are 2H, 2I bytes); h is the activation rounded
 *     once to bfloat16 (round to nearest even); x_sf, w1_sf, w2_sf and h_sf are not read
 *     or written (they may be NULL).  Blockwise scaling mode only; x smaller than 4 GiB
 *     means T*H < 2^31 here.
 *   - Shared experts (num_shared = S > 0; the pages list shared-expert builds of the
 *     kernel, "Sync upstream through PR #441", Validation): S more experts that every token
 *     passes through with weight 1.  Their weights follow the routed local experts in
 *     w1/w1_sf/w2/w2_sf, which then hold E_loc + S experts (per-tensor scales: E_loc + S
 *     floats).  Their rows follow the routed rows: shared expert s owns h rows
 *     [R + s*T, R + (s+1)*T), row R + s*T + t being token t, so h and h_sf hold
 *     T*k + S*T rows.  y[t] adds them after the routed slots, in order s = 0..S-1, before
 *     the single bf16 rounding.  counts, offsets, row_to_slot and slot_to_row describe the
 *     routed rows only.
 *   - Logits must be finite; non-finite logits give unspecified routing.
 *   - Validation happens on the host before any launch; on error nothing is
 *     launched and a moe_status is returned (moe_last_error() has details).  A
 *     call with num_tokens = 0 returns MOE_OK without launching anything or
 *     touching any buffer.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream),
 *     do no host synchronisation and no allocation, so they may be captured in a
 *     HIP graph.  Calls on distinct workspaces may run concurrently.
 *   - Alignment: x, x_sf, w1, w1_sf, w2, w2_sf, h, h_sf, logits and y must be
 *     16-byte aligned, the workspace 256-byte aligned (MOE_ERR_MISALIGNED otherwise).
 *   - Limits: H and I multiples of 128 and at most 8192 (MOE_ERR_UNSUPPORTED above);
 *     1 <= E_loc <= E_tot <= 1024;
 *     1 <= k <= min(E_tot, 16); 0 <= S <= 4; T*(k + S) < 2^31; x smaller than 4 GiB (T*H < 2^32,
 *     MOE_ERR_UNSUPPORTED otherwise).
 */
#ifndef MOE_EXPERT_LAYER_H_
#define MOE_EXPERT_LAYER_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,          /* a required pointer is NULL */
  MOE_ERR_INVALID_DESC = 2,  /* a size or parameter in the descriptor is out of range */
  MOE_ERR_MISALIGNED = 3,    /* a pointer violates the alignment rules above */
  MOE_ERR_UNSUPPORTED = 4,   /* valid request the library cannot run (e.g. not a gfx950 device) */
  MOE_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than moe_workspace_size() */
  MOE_ERR_DEVICE = 6         /* a HIP runtime call or launch failed */
} moe_status;

/* Activation names follow the pages' API: "swiglu" and "swigluoai". */
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_SWIGLU_OAI = 1 } moe_act;

/* Scaling: blockwise UE8M0 (the default) or one float32 scale per tensor (see above). */
typedef enum { MOE_SCALE_BLOCK = 0, MOE_SCALE_TENSOR = 1 } moe_scale;

/* Layout of the 1x128 activation scale tensors x_sf and h_sf (blockwise scaling only):
 * MOE_SF_ROW_MAJOR: UE8M0 bytes [rows, groups] (the default; groups = H/128 or I/128);
 * MOE_SF_PACKED_MN: the packed int32 MN-major tensor of "DSV4 o_proj: fuse fp8/UE8M0 quantize
 *   into o_a proj" (Description: shape (rows, ceil(groups/4)), stride (1, aligned_rows),
 *   aligned_rows = rows rounded up to 4): word (m, j) at int32 index j * aligned_rows + m holds
 *   groups 4j..4j+3 of row m, group 4j+b in byte b (the layout moe_pack_scales writes).  The
 *   GEMMs read x_sf (rows = T) and FC1 writes / FC2 reads h_sf (rows = T*k + S*T) in this
 *   layout directly; FC1 writes only the bytes of real groups and rows (padding is not
 *   written and not read). */
typedef enum { MOE_SF_ROW_MAJOR = 0, MOE_SF_PACKED_MN = 1 } moe_sf_layout;

/* Weight formats: FP8 E4M3 or E5M2 with 128x128 UE8M0 block scales, or MXFP4 (E2M1, UE8M0
 * per 32 along K).  The FP8 weight formats are the ones the Hopper CuTeDSL MegaMoE kernel
 * takes (Pull Style Cutedsl Megakernel, Layout section); the activations stay E4M3. */
typedef enum {
  MOE_W_FP8_E4M3_B128 = 0,
  MOE_W_MXFP4_E2M1_B32 = 1,
  MOE_W_FP8_E5M2_B128 = 2,
  MOE_W_BF16 = 3  /* BF16 layer: x, weights and h in BF16, no scales (see above) */
} moe_wfmt;

typedef struct {
  int32_t num_tokens;     /* T >= 0 */
  int32_t hidden;         /* H, multiple of 128 */
  int32_t inter;          /* I, multiple of 128 */
  int32_t num_experts;    /* E_tot: routing width */
  int32_t local_begin;    /* e0: first local expert */
  int32_t num_local;      /* E_loc: local experts are [e0, e0 + E_loc) */
  int32_t topk;           /* k */
  int32_t weight_format;  /* moe_wfmt */
  int32_t activation;     /* moe_act */
  float act_clamp;        /* OAI only: gate <= clamp, |up| <= clamp; +inf = no clamp (must be > 0) */
  float act_alpha;        /* OAI only: sigmoid(alpha * gate); default 1.0 */
  float act_up_bias;      /* OAI only: (up + up_bias); default 0.0 */
  int32_t variant;        /* GEMM tiles: -1 = heuristic; 0 = 128-row tiles; 1 = 256-row tiles;
                             2 = 32-row tiles */
  int32_t scale_mode;     /* moe_scale; default MOE_SCALE_BLOCK */
  float h_scale;          /* MOE_SCALE_TENSOR only: static scale of the intermediate h */
  int32_t num_shared;     /* S in [0, 4]: shared experts applied to every token with weight 1 */
  int32_t scale_layout;   /* moe_sf_layout of x_sf and h_sf; default MOE_SF_ROW_MAJOR */
} moe_layer_desc;

/* ABI version of the loaded library (MOE_ABI_VERSION at build time). */
int moe_abi_version(void);

/* Static string naming a status code. */
const char* moe_status_str(int status);

/* Details of the last error returned on the calling thread ("" when none). */
const char* moe_last_error(void);

/* Fill *desc with defaults: SwiGLU, FP8 weights, blockwise scales, clamp +inf, alpha 1.0,
 * up_bias 0.0, variant -1, h_scale 1.0, all sizes 0 (the pages' Compatibility section: the OAI parameters
 * default to the standard SwiGLU behaviour).  Host only. */
moe_status moe_desc_defaults(moe_layer_desc* desc);

/* Bytes of workspace every entry point below needs for this descriptor.  Host only;
 * validates the descriptor.  The pages split the fused layer's API into a buffer-sizing /
 * allocation call and the execution calls ("fix(sm90): support parameterized SwiGLU in FP8
 * MegaMoE", Changes: buffer allocation and execution APIs), and build the layer as
 * config -> buffer -> compute ("Pull Style Cutedsl Megakernel", Layout); here the caller
 * owns the buffer and this call sizes it.
 * Errors: MOE_ERR_NULL (desc or bytes NULL), MOE_ERR_INVALID_DESC, MOE_ERR_UNSUPPORTED. */
moe_status moe_workspace_size(const moe_layer_desc* desc, size_t* bytes);

/* Route + permute: logits -> topk_ids, topk_w, counts, offsets, row_to_slot, slot_to_row.
 * All outputs are required (caller-owned device buffers of the sizes above).
 * The fused layer consumes tokens grouped by expert (the grouped, "masked/unmasked" expert
 * layouts of "Optimize sm100 version with token-aware BM240 tiling, native UE8M0, and direct
 * combine", description) and its top-k reduce needs each token's k expert ids and weights
 * ("Pull Style Cutedsl Megakernel", Layout: topk_reduce).  The pages do not define the
 * routing function; this call takes the top k logits (ties to the lower expert id) and a
 * float64 softmax over those k, rounded once to float32.  Grouping is stable in the slot id
 * s = t*k + j, so the result is unique.  Reads logits [T, E_tot]; writes every output;
 * uses the workspace for its histograms.  Errors: MOE_ERR_NULL, MOE_ERR_MISALIGNED,
 * MOE_ERR_WORKSPACE, MOE_ERR_INVALID_DESC, MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE. */
moe_status moe_route_permute(const moe_layer_desc* desc, const float* logits, int32_t* topk_ids,
                             float* topk_w, int32_t* counts, int32_t* offsets, int32_t* row_to_slot,
                             int32_t* slot_to_row, void* workspace, size_t workspace_bytes,
                             void* stream);

/* FC1 + activation + 1x128 requant for every row of every local expert.
 * Reads x/x_sf rows of token row_to_slot[r] / k (shared expert rows: every token in
 * order), writes h/h_sf rows [0, R + S*T).
 * Sources: the gate/up GEMM with the activation applied in its epilogue, standard SwiGLU or
 * OAI-SwiGLU with clamp / alpha / up_bias ("fix(sm90): support parameterized SwiGLU in FP8
 * MegaMoE", Summary and Changes: act_type "swiglu" / "swigluoai"); FP8 operands with native
 * UE8M0 block scales ("Optimize sm100 version with token-aware BM240 tiling, native UE8M0,
 * and direct combine", description); the FP8 + 1x128 UE8M0 output emitted from the GEMM
 * epilogue with an amax per block ("DSV4 o_proj: fuse fp8/UE8M0 quantize into o_a proj",
 * Description).  offsets and row_to_slot are this call's inputs (from moe_route_permute);
 * the workspace is not read.  Errors: MOE_ERR_NULL, MOE_ERR_MISALIGNED, MOE_ERR_WORKSPACE,
 * MOE_ERR_INVALID_DESC, MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE. */
moe_status moe_grouped_fc1_swiglu(const moe_layer_desc* desc, const uint8_t* x, const uint8_t* x_sf,
                                  const uint8_t* w1, const uint8_t* w1_sf, const int32_t* offsets,
                                  const int32_t* row_to_slot, uint8_t* h, uint8_t* h_sf,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* FC2 + top-k weighted combine into y (bf16 bits, [T, H]).  The fp32 FC2 rows are
 * kept in the workspace; the sum over a token's local slots runs in slot order
 * j = 0..k-1 in fp32, then adds the shared experts' rows (weight 1), and is rounded
 * once to bf16.  Reads h/h_sf rows [0, R + S*T).
 * Sources: the fused layer ends FC2 -> top-k reduce ("Pull Style Cutedsl Megakernel",
 * Layout: fc1_fc2_fuse_sched, topk_reduce), combining each token's expert outputs back into
 * token order ("Optimize sm100 version with token-aware BM240 tiling, native UE8M0, and
 * direct combine", description), with run-to-run bitwise-identical outputs (same
 * description); this reduce has no atomics and a fixed slot order.  Overwrites the whole
 * of y.  Errors: MOE_ERR_NULL, MOE_ERR_MISALIGNED, MOE_ERR_WORKSPACE, MOE_ERR_INVALID_DESC,
 * MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE. */
moe_status moe_grouped_fc2_combine(const moe_layer_desc* desc, const uint8_t* h, const uint8_t* h_sf,
                                   const uint8_t* w2, const uint8_t* w2_sf, const int32_t* offsets,
                                   const int32_t* row_to_slot, const int32_t* slot_to_row,
                                   const float* topk_w, uint16_t* y, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* The whole layer.  The opt_* outputs may be NULL (then they live in the workspace);
 * when given they receive the routing/grouping results.
 * Sources: the fused "Mega MoE" layer, one call from routed tokens to the combined output
 * ("Pull Style Cutedsl Megakernel", Layout: config -> buffer -> compute, FC1 -> FC2 ->
 * top-k reduce; "fix(sm90): support parameterized SwiGLU in FP8 MegaMoE", Changes: the
 * execution API).  Equal bit for bit to moe_route_permute + moe_grouped_fc1_swiglu +
 * moe_grouped_fc2_combine on the same inputs.  Errors: MOE_ERR_NULL, MOE_ERR_MISALIGNED,
 * MOE_ERR_WORKSPACE, MOE_ERR_INVALID_DESC, MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE. */
moe_status moe_layer(const moe_layer_desc* desc, const float* logits, const uint8_t* x,
                     const uint8_t* x_sf, const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2,
                     const uint8_t* w2_sf, uint16_t* y, int32_t* opt_topk_ids, float* opt_topk_w,
                     int32_t* opt_counts, int32_t* opt_offsets, int32_t* opt_row_to_slot,
                     int32_t* opt_slot_to_row, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Size in bytes of the static per-device scratch array that moe_layer_static uses. */
#define MOE_STATIC_SCRATCH_BYTES (64u * 1024u * 1024u)

/* moe_static_scratch_bytes: MOE_STATIC_SCRATCH_BYTES as built into the loaded library. */
size_t moe_static_scratch_bytes(void);

/* moe_layer without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and errors as moe_layer, except that the scratch comes from a
 * static device array of MOE_STATIC_SCRATCH_BYTES (64 MiB) in the library, one per GPU,
 * held until the process ends; its device address is looked up on the first call on
 * each device (with that device current).  A layer whose moe_workspace_size exceeds that
 * size is rejected with MOE_ERR_WORKSPACE before any launch (decode-sized shares fit:
 * 128 tokens, top-8, hidden 7168, intermediate 2048 need about 33 MB).  The call allocates
 * nothing and needs no zeroed memory.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (other streams, other threads) race and give
 * undefined results; calls ordered on one stream are safe. */
moe_status moe_layer_static(const moe_layer_desc* desc, const float* logits, const uint8_t* x,
                            const uint8_t* x_sf, const uint8_t* w1, const uint8_t* w1_sf,
                            const uint8_t* w2, const uint8_t* w2_sf, uint16_t* y,
                            int32_t* opt_topk_ids, float* opt_topk_w, int32_t* opt_counts,
                            int32_t* opt_offsets, int32_t* opt_row_to_slot, int32_t* opt_slot_to_row,
                            void* stream);

/* Input quantisation (the pages' "DSV4 o_proj: fuse fp8/UE8M0 quantize into o_a proj",
 * Description: FP8 E4M3 with one UE8M0 scale per 1x128 block, from an amax per block).
 * x_bf16 [T, H] bf16 bits -> x [T, H] E4M3 codes and x_sf [T, H/128] UE8M0 bytes, the
 * layout moe_layer and moe_grouped_fc1_swiglu read.  The rule is the one used for the
 * intermediate h: scale 2^e with the smallest e such that 448 * 2^e >= amax of the block
 * (byte e + 127 clamped to [0, 254]; 127 for an all-zero block), codes E4M3
 * round-to-nearest-even of v * 2^-e.  Deterministic and exact for finite inputs.
 * Uses desc->num_tokens and desc->hidden; x_bf16 and x must be 16-byte aligned. No
 * workspace; asynchronous on `stream`.  Blockwise scaling only (MOE_ERR_UNSUPPORTED for
 * MOE_SCALE_TENSOR, whose x scale is the caller's calibration). */
moe_status moe_quantize_act(const moe_layer_desc* desc, const uint16_t* x_bf16, uint8_t* x, uint8_t* x_sf,
                            void* stream);

/* Packed UE8M0 scale interop (the pages' "DSV4 o_proj: fuse fp8/UE8M0 quantize into o_a
 * proj": the FP8-output tactic's int32 scale tensor of shape (M, ceil(G/4)) with MN-major
 * stride (1, aligned_M), aligned_M = M rounded up to 4, padding zeroed).
 * moe_pack_scales: sf [rows, groups] UE8M0 bytes (the layout of x_sf and h_sf) -> packed,
 * an int32 buffer of ceil(groups/4) * aligned_rows words where word (m, j) is at
 * j * aligned_rows + m and holds groups 4j..4j+3 of row m, group 4j+b in byte b
 * (little-endian); every padding row and byte is written as zero.
 * moe_unpack_scales: the inverse (padding is not read).
 * rows >= 0, 1 <= groups, rows * groups < 2^31; packed must be 4-byte aligned.
 * Asynchronous on `stream`. */
moe_status moe_pack_scales(int32_t rows, int32_t groups, const uint8_t* sf, int32_t* packed, void* stream);
moe_status moe_unpack_scales(int32_t rows, int32_t groups, const int32_t* packed, uint8_t* sf, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EXPERT_LAYER_H_ */
