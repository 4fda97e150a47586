"""CPU oracle for the MegaMoE expert layer (test infrastructure only).

ORACLE — TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import or call this module.  The product
path (the HIP library and its Python binding) never touches it.

A plain, slow, obviously correct numpy implementation of one MoE expert layer on
one GPU's share of the experts, written from the pages' description of the fused
"Mega MoE" layer and shared with nothing in the HIP path:

  route      top-k of each token's routing logits, softmax weights over the k chosen
  permute    group the local (token, slot) pairs by expert, stable by slot id
  FC1        gate/up projection of the FP8 E4M3 activations with 1x128 UE8M0 scales
             against FP8 (E4M3 or E5M2) weights with 128x128 UE8M0 block scales (or MXFP4)
  activation SwiGLU, or parameterised OAI-SwiGLU (clamp, sigmoid alpha, up bias)
  requant    the intermediate back to FP8 E4M3 with one UE8M0 scale per 1x128 block
             (per-tensor variant: float32 scales for x and each expert's weights, and a
             static float32 scale for the intermediate, E4M3 codes saturated at 448)
  quantize   (input side) bf16 activations to FP8 E4M3 with the same 1x128 UE8M0 rule
  FC2        down projection of the requantised intermediate
  combine    top-k weighted sum of each token's local rows, back in token order
  shared     (variant) S shared experts that every token passes through with weight 1,
             added after the routed slots
  bf16       (variant) the whole layer in bfloat16: x, weights and the intermediate (the
             activation rounded once to bfloat16), no scales

Sources (pages of the study, cited by title and section):
  * "fix(sm90): support parameterized SwiGLU in FP8 MegaMoE" (DeepGEMM PR #445),
    sections Summary, Root Cause and Compatibility: the two activation formulas,
    the MiniMax-M3 constants (alpha 1.702, up_bias 1.0, clamp 7.0) and the
    defaults alpha 1.0, up_bias 0.0 that reduce OAI-SwiGLU to standard SwiGLU.
  * "Optimize sm100 version with token-aware BM240 tiling, native UE8M0, and
    direct combine" (DeepGEMM PR #386), description: FP8 expert GEMMs with native
    power-of-two (UE8M0) scales and a combine back to token order.
  * "DSV4 o_proj: fuse fp8/UE8M0 quantize into o_a proj" (TensorRT-LLM PR #16346),
    Description: a 1x128 FP8 E4M3 quantisation with UE8M0 scales, amax per block.
  * "Pull Style Cutedsl Megakernel" (FlashInfer skill page), Layout: the fused
    layer is FC1 -> FC2 -> top-k reduce, and the Hopper kernel takes E4M3 or E5M2
    weights.

Readings where the pages are silent (each is listed with its reason in the design
notes): routing is top-k by (logit descending, expert id ascending) with an fp64
softmax over the k chosen logits rounded once to fp32; non-local slots are
dropped after normalisation; W1 rows [0, I) are gate and [I, 2I) are up; the
UE8M0 requant scale is the smallest power of two 2**e with 448 * 2**e >= amax
(byte 127 for an all-zero block) and the codes are E4M3 round-to-nearest-even;
the weight is applied at combine time; the output is bf16 (round to nearest
even) of the weighted sum.

Precision: dequantised operands and both GEMMs in float64 (a library matmul is
the contraction step); the activation in float64; the activation output is then
rounded to float32, and the requant decision is taken on that float32 value, the
precision in which the GPU kernel decides it.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode_e4m3", "decode_e5m2", "decode_ue8m0", "decode_e2m1", "encode_e4m3_rne", "bf16_rne_bits",
    "dequant_act", "dequant_weight", "route", "permute", "activation", "requant_1x128", "requant_tensor",
    "expert_rows", "combine", "layer", "layer_tokens",
]


# ---------------------------------------------------------------------------
# codecs (OCP 8-bit floating point and OCP MX formats)

def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """E4M3FN byte -> float64: sign, 4-bit exponent (bias 7), 3-bit mantissa; S.1111.111 is NaN."""
    c = codes.astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    out = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, out)


def decode_e5m2(codes: np.ndarray) -> np.ndarray:
    """E5M2 byte -> float64: sign, 5-bit exponent (bias 15), 2-bit mantissa; exponent 31 is
    infinity (mantissa 0) or NaN, exponent 0 is subnormal (m/4 * 2**-14)."""
    c = codes.astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 2) & 0x1F
    m = c & 3
    mag = np.where(e == 0, np.ldexp(m / 4.0, -14), np.ldexp(1.0 + m / 4.0, e - 15))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def decode_ue8m0(b: np.ndarray) -> np.ndarray:
    """UE8M0 byte -> 2**(b - 127); 0xFF is NaN."""
    bi = b.astype(np.int64)
    return np.where(bi == 255, np.nan, np.ldexp(1.0, bi - 127))


def decode_e2m1(nib: np.ndarray) -> np.ndarray:
    """E2M1 nibble -> float64: sign, 2-bit exponent (bias 1), 1-bit mantissa."""
    n = nib.astype(np.int64)
    s = (n >> 3) & 1
    e = (n >> 1) & 3
    m = n & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + m / 2.0, e - 1))
    return np.where(s == 1, -mag, mag)


def encode_e4m3_rne(v: np.ndarray) -> np.ndarray:
    """float64 with |v| <= 448 -> E4M3FN byte, round to nearest, ties to even mantissa.

    In the binade [2**ex, 2**(ex+1)) (ex >= -6) the grid spacing is 2**(ex-3); below
    2**-6 the subnormal spacing is 2**-9, which is the same spacing as the ex = -6
    binade.  With n = rint(|v| / spacing) the code is ((ex + 7) << 3) + n - 8, where
    n = 16 carries into the next exponent and, for ex = -6, n < 8 lands on the
    subnormal codes.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if not np.all(a <= 448.0):
        raise ValueError("encode_e4m3_rne: |v| must be <= 448 (and not NaN)")
    _, E = np.frexp(a)  # a = f * 2**E with f in [0.5, 1)
    ex = np.where(a == 0, -6, np.maximum(E - 1, -6))
    n = np.rint(a / np.ldexp(1.0, ex - 3))
    code = ((ex + 7) << 3) + n.astype(np.int64) - 8
    code = np.where(a == 0, 0, code)
    code = code | (np.signbit(v).astype(np.int64) << 7)
    return code.astype(np.uint8)


def bf16_rne_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit pattern, one rounding to nearest even (8 significant bits)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, E = np.frexp(a)
    ex = np.where(a == 0, -126, np.maximum(E - 1, -126))
    r = np.rint(a / np.ldexp(1.0, ex - 7)) * np.ldexp(1.0, ex - 7)
    r = np.where(np.signbit(v), -r, r)
    bits = r.astype(np.float32).view(np.uint32) >> 16  # r is exactly representable in bf16
    return bits.astype(np.uint16)


# ---------------------------------------------------------------------------
# dequantisation of the layer's inputs

def dequant_act(x: np.ndarray, x_sf: np.ndarray) -> np.ndarray:
    """E4M3 rows [n, H] with 1x128 UE8M0 scales [n, H/128] -> float64 [n, H]."""
    n, h = x.shape
    s = decode_ue8m0(x_sf)
    return (decode_e4m3(x).reshape(n, h // 128, 128) * s[:, :, None]).reshape(n, h)


def dequant_weight(w: np.ndarray, sf: np.ndarray, fmt: str, rows: int, cols: int) -> np.ndarray:
    """One expert's weight -> float64 [rows, cols] (K = cols contiguous).

    fp8:     E4M3 bytes [rows, cols], UE8M0 per 128x128 block [rows/128, cols/128].
    fp8e5m2: E5M2 bytes, the same 128x128 block scales.
    mxfp4:   packed E2M1 [rows, cols/2] (element 2i low nibble), UE8M0 per 1x32 [rows, cols/32].
    """
    if fmt in ("fp8", "fp8e5m2"):
        s = decode_ue8m0(sf)
        dec = decode_e4m3 if fmt == "fp8" else decode_e5m2
        v = dec(w).reshape(rows // 128, 128, cols // 128, 128)
        return (v * s[:, None, :, None]).reshape(rows, cols)
    if fmt == "mxfp4":
        vals = np.empty((rows, cols), dtype=np.float64)
        vals[:, 0::2] = decode_e2m1(w & 0xF)
        vals[:, 1::2] = decode_e2m1(w >> 4)
        s = decode_ue8m0(sf)
        return (vals.reshape(rows, cols // 32, 32) * s[:, :, None]).reshape(rows, cols)
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# routing and grouping

def route(logits: np.ndarray, k: int):
    """Top-k experts per token and their softmax weights.

    Slot j of token t holds the j-th largest logit (ties -> lower expert id).  The
    weights are a softmax over the k chosen logits (equal to a softmax over all
    experts renormalised over the chosen ones): d_j = l_j - l_0 and e_j = exp(d_j)
    in float64, S = e_0 + e_1 + ... in slot order, w_j = float32(e_j / S).
    """
    logits = np.asarray(logits, dtype=np.float32)
    if not np.all(np.isfinite(logits)):
        raise ValueError("route: logits must be finite")
    t, e = logits.shape
    ids = np.empty((t, k), dtype=np.int32)
    taken = np.zeros((t, e), dtype=bool)
    ar = np.arange(t)
    for j in range(k):
        cand = np.where(taken, -np.inf, logits.astype(np.float64))
        best = np.argmax(cand, axis=1)  # first maximum -> lowest id among ties
        ids[:, j] = best
        taken[ar, best] = True
    chosen = logits[ar[:, None], ids].astype(np.float64)
    ex = np.exp(chosen - chosen[:, :1])
    s = ex[:, 0].copy()
    for j in range(1, k):
        s = s + ex[:, j]
    w = (ex / s[:, None]).astype(np.float32)
    return ids, w


def permute(ids: np.ndarray, local_begin: int, num_local: int):
    """Group local slots by local expert, ascending slot id inside each expert.

    Slot s = t*k + j is local when local_begin <= ids[t, j] < local_begin + num_local.
    Returns counts [E_loc], offsets [E_loc + 1] (exclusive scan, offsets[-1] = R),
    row_to_slot [T*k] (rows [0, R) hold slot ids, the rest -1) and slot_to_row [T*k]
    (-1 for non-local slots).
    """
    flat = ids.reshape(-1).astype(np.int64)
    le = flat - local_begin
    local = (le >= 0) & (le < num_local)
    counts = np.bincount(le[local], minlength=num_local).astype(np.int32)
    offsets = np.zeros(num_local + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    local_slots = np.nonzero(local)[0]
    order = np.argsort(le[local_slots], kind="stable")
    r = int(offsets[-1])
    row_to_slot = np.full(flat.size, -1, dtype=np.int32)
    row_to_slot[:r] = local_slots[order]
    slot_to_row = np.full(flat.size, -1, dtype=np.int32)
    slot_to_row[row_to_slot[:r]] = np.arange(r, dtype=np.int32)
    return counts, offsets, row_to_slot, slot_to_row


# ---------------------------------------------------------------------------
# expert FFN pieces

def activation(g: np.ndarray, u: np.ndarray, kind: str, clamp: float = np.inf, alpha: float = 1.0,
               up_bias: float = 0.0) -> np.ndarray:
    """SwiGLU: g * sigmoid(g) * u.  OAI-SwiGLU: g' = min(g, clamp), u' = clip(u, -clamp, clamp),
    g' * sigmoid(alpha * g') * (u' + up_bias).  float64."""
    with np.errstate(over="ignore"):
        if kind == "swiglu":
            return g * (1.0 / (1.0 + np.exp(-g))) * u
        if kind == "swigluoai":
            gc = np.minimum(g, clamp)
            uc = np.clip(u, -clamp, clamp)
            return gc * (1.0 / (1.0 + np.exp(-alpha * gc))) * (uc + up_bias)
    raise ValueError(kind)


def requant_1x128(h32: np.ndarray):
    """float32 rows [n, I] -> E4M3 codes [n, I] and UE8M0 bytes [n, I/128].

    Per block of 128 consecutive columns: amax = max |h|; the scale is 2**e for the
    smallest integer e with 448 * 2**e >= amax (byte e + 127, clamped to [0, 254];
    byte 127 when amax = 0); codes = E4M3 RNE of h * 2**-e (never above 448).
    """
    h32 = np.asarray(h32, dtype=np.float32)
    n, i = h32.shape
    blk = h32.astype(np.float64).reshape(n, i // 128, 128)
    amax = np.abs(blk).max(axis=2)
    _, E = np.frexp(amax)
    e = E.astype(np.int64) - 10  # 448 * 2**(E-10) < 2**(E-1) <= amax: below the answer
    for _ in range(4):  # raise e until 448 * 2**e >= amax (at most two steps)
        e = e + (448.0 * np.ldexp(1.0, e) < amax)
    byte = np.clip(e + 127, 0, 254)
    byte = np.where(amax == 0, 127, byte)
    scaled = blk * np.ldexp(1.0, -(byte - 127))[:, :, None]
    codes = encode_e4m3_rne(scaled).reshape(n, i)
    return codes, byte.astype(np.uint8)


def requant_tensor(h32: np.ndarray, h_scale: float) -> np.ndarray:
    """float32 rows -> E4M3 codes of h / h_scale (float64 quotient), saturated to +-448, round
    to nearest even (the per-tensor variant's static-scale quantisation)."""
    v = np.asarray(h32, dtype=np.float32).astype(np.float64) / float(np.float32(h_scale))
    return encode_e4m3_rne(np.clip(v, -448.0, 448.0))


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (the upper half of the float32 pattern; exact)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def quantize_act(x_bf16_bits: np.ndarray):
    """Input quantisation: bf16 rows [T, H] -> E4M3 codes [T, H] and UE8M0 bytes [T, H/128].

    The activations' FP8 E4M3 format with one UE8M0 scale per 128 consecutive values
    ("DSV4 o_proj: fuse fp8/UE8M0 quantize into o_a proj", Description) under the same
    scale rule as the intermediate: bf16 values are exact in float32, so this is
    ``requant_1x128`` of the decoded rows.
    """
    return requant_1x128(decode_bf16(x_bf16_bits))


def pack_ue8m0(sf: np.ndarray) -> np.ndarray:
    """UE8M0 bytes [M, G] -> packed int32 storage [ceil(G/4), aligned_M] (aligned_M = M rounded up to 4).

    The packed scale tensor of "DSV4 o_proj: fuse fp8/UE8M0 quantize into o_a proj" (the
    o_a FP8-output tactic's checks): int32, shape (M, ceil(G/4)), MN-major stride
    (1, aligned_M), padding zeroed.  Word (m, j) holds groups 4j .. 4j+3 of row m, group
    4j + b in byte b (little-endian; the byte order is not printed on the page).  The
    returned array is the storage: element [j, m] is word (m, j).
    """
    sf = np.asarray(sf, dtype=np.uint8)
    m, g = sf.shape
    am, nw = (m + 3) // 4 * 4, (g + 3) // 4
    out = np.zeros((nw, am), dtype=np.uint32)
    for j in range(nw):
        for b in range(4):
            if 4 * j + b < g:
                out[j, :m] |= sf[:, 4 * j + b].astype(np.uint32) << np.uint32(8 * b)
    return out.view(np.int32)


def unpack_ue8m0(packed: np.ndarray, m: int, g: int) -> np.ndarray:
    """Inverse of pack_ue8m0: storage [ceil(G/4), aligned_M] int32 -> UE8M0 bytes [M, G]."""
    w = np.asarray(packed).view(np.uint32)
    sf = np.zeros((m, g), dtype=np.uint8)
    for k in range(g):
        sf[:, k] = (w[k // 4, :m] >> np.uint32(8 * (k % 4))) & np.uint32(0xFF)
    return sf


def expert_rows(d, inputs, e: int, tokens: np.ndarray):
    """FC1 -> activation -> requant -> FC2 for rows of local expert e whose tokens are given.

    Returns (h codes [n, I], h scales [n, I/128], Y2 float64 [n, H]).
    """
    H, I, fmt = d.hidden, d.inter, d.weight_format
    if fmt == "bf16":
        # BF16 layer: operands are bfloat16 bit patterns, no scales; h is the activation's
        # float32 value rounded once to bfloat16 (nearest even); h_sf is not produced (zeros)
        bf = lambda a: decode_bf16(a).astype(np.float64)
        x = bf(inputs["x"][tokens])
        gu = x @ bf(inputs["w1"][e]).T
        h = activation(gu[:, :I], gu[:, I:], d.activation, d.act_clamp, d.act_alpha, d.act_up_bias)
        hq = bf16_rne_bits(h.astype(np.float32).astype(np.float64))
        hs = np.zeros((hq.shape[0], I // 128), np.uint8)
        return hq, hs, bf(hq) @ bf(inputs["w2"][e]).T
    if getattr(d, "scaling", "block") == "tensor":
        # per-tensor: every scale is one float32 (x: [1], weights: one per expert), the
        # intermediate uses the descriptor's static h_scale; h_sf is not produced (zeros)
        dec = decode_e4m3 if fmt == "fp8" else decode_e5m2
        sc = lambda a: float(np.float32(a))
        x = decode_e4m3(inputs["x"][tokens]) * sc(inputs["x_sf"][0])
        w1 = dec(inputs["w1"][e]) * sc(inputs["w1_sf"][e])
        gu = x @ w1.T
        h = activation(gu[:, :I], gu[:, I:], d.activation, d.act_clamp, d.act_alpha, d.act_up_bias)
        hq = requant_tensor(h.astype(np.float32), d.h_scale)
        hs = np.zeros((hq.shape[0], I // 128), np.uint8)
        hd = decode_e4m3(hq) * sc(d.h_scale)
        w2 = dec(inputs["w2"][e]) * sc(inputs["w2_sf"][e])
        return hq, hs, hd @ w2.T
    x = dequant_act(inputs["x"][tokens], inputs["x_sf"][tokens])
    w1 = dequant_weight(inputs["w1"][e], inputs["w1_sf"][e], fmt, 2 * I, H)
    gu = x @ w1.T
    h = activation(gu[:, :I], gu[:, I:], d.activation, d.act_clamp, d.act_alpha, d.act_up_bias)
    hq, hs = requant_1x128(h.astype(np.float32))
    hd = dequant_act(hq, hs)
    w2 = dequant_weight(inputs["w2"][e], inputs["w2_sf"][e], fmt, H, I)
    y2 = hd @ w2.T
    return hq, hs, y2


def combine(w: np.ndarray, slot_to_row: np.ndarray, y2: np.ndarray, tokens: np.ndarray, k: int) -> np.ndarray:
    """y[t] = sum over local slots j (in slot order) of w[t, j] * Y2[row(t, j)], starting from 0."""
    out = np.zeros((tokens.size, y2.shape[1]), dtype=np.float64)
    for j in range(k):
        rows = slot_to_row[tokens * k + j]
        m = rows >= 0
        out[m] = out[m] + w[tokens[m], j].astype(np.float64)[:, None] * y2[rows[m]]
    return out


def layer(d, inputs):
    """The whole layer for every token.  Returns a dict of all outputs."""
    return layer_tokens(d, inputs, None)


def layer_tokens(d, inputs, tokens=None):
    """The layer evaluated for a subset of tokens (all tokens when ``tokens`` is None).

    Routing and grouping always cover every token (they define the row numbering);
    FC1/FC2 are evaluated only for the rows of the requested tokens.  ``h``/``h_sf``
    are indexed by row and hold valid data only for evaluated rows (``h_valid``).
    Shared experts (``num_shared`` = S, weights at indices E_loc .. E_loc + S - 1) own
    rows R + s*T + t after the routed rows and join every token with weight 1.
    """
    T, k, E_loc = d.tokens, d.topk, d.num_local
    S = getattr(d, "num_shared", 0)
    ids, w = route(inputs["logits"], k)
    counts, offsets, r2s, s2r = permute(ids, d.local_begin, E_loc)
    R = int(offsets[-1])
    NR = R + S * T  # rows: routed, then the shared experts' (token order)
    toks = np.arange(T) if tokens is None else np.asarray(sorted(set(int(t) for t in tokens)), dtype=np.int64)
    want = np.zeros(T, dtype=bool)
    want[toks] = True
    y2 = np.zeros((max(NR, 1), d.hidden), dtype=np.float64)
    h = np.zeros((max(NR, 1), d.inter), dtype=np.uint16 if d.weight_format == "bf16" else np.uint8)
    h_sf = np.zeros((max(NR, 1), d.inter // 128), dtype=np.uint8)
    h_valid = np.zeros(max(NR, 1), dtype=bool)
    for e in range(E_loc):
        rows = np.arange(offsets[e], offsets[e + 1])
        if rows.size == 0:
            continue
        rtok = r2s[rows] // k
        sel = want[rtok]
        rows, rtok = rows[sel], rtok[sel]
        if rows.size == 0:
            continue
        hq, hs, yy = expert_rows(d, inputs, e, rtok)
        h[rows], h_sf[rows], y2[rows] = hq, hs, yy
        h_valid[rows] = True
    for s in range(S):
        if toks.size == 0:
            break
        rows = R + s * T + toks
        hq, hs, yy = expert_rows(d, inputs, E_loc + s, toks)
        h[rows], h_sf[rows], y2[rows] = hq, hs, yy
        h_valid[rows] = True
    y64 = combine(w, s2r, y2, toks, k)
    for s in range(S):  # after the routed slots, weight 1
        y64 = y64 + y2[R + s * T + toks]
    return {
        "topk_ids": ids, "topk_w": w, "counts": counts, "offsets": offsets,
        "row_to_slot": r2s, "slot_to_row": s2r, "R": R,
        "h": h[:NR], "h_sf": h_sf[:NR], "h_valid": h_valid[:NR],
        "tokens": toks, "y64": y64, "y_bf16": bf16_rne_bits(y64),
    }
