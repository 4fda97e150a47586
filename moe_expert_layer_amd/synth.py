"""Seeded synthetic inputs for the MoE expert layer.

This module only *makes inputs*: routing logits, FP8 E4M3 activations with 1x128
UE8M0 scales, and expert weights as FP8 E4M3 (or E5M2) with 128x128 UE8M0 block
scales or as MXFP4 (E2M1 nibbles with one UE8M0 scale per 32 elements); variants
with one float32 scale per tensor, with shared experts, or all in BF16.  It holds none of
the layer's arithmetic (routing, grouping, GEMMs, activation, requantisation,
combine); both the HIP path and the CPU oracle consume the bytes it returns.

Encodings of the produced bytes (what both consumers must assume):
  * E4M3 is the OCP 8-bit "E4M3FN" format (bias 7, max 448, no inf); E5M2 is OCP
    E5M2 (bias 15, max 57344).  BF16 values are bit patterns (uint16).
  * UE8M0 byte b means 2**(b - 127).
  * MXFP4: element 2i of a K-row sits in the low nibble of byte i, element 2i+1 in
    the high nibble; nibble = sign<<3 | exp<<1 | mantissa (E2M1, bias 1).
  * W1 of each expert is [2*I, H] row-major: rows [0, I) are the gate projection,
    rows [I, 2I) the up projection.  W2 is [H, I] row-major.

Workloads are the five shapes of the MegaMoE expert-layer study (tiny, OAI-SwiGLU,
decode share, prefill share with a Zipf expert prior, MXFP4 share); the recipe is
restated in each ``Workload``.  Quantising the inputs here uses torch's CPU
float8 cast and a float log2 for the scale exponent: any valid scale byte gives a
valid input, so this choice cannot affect parity between the two consumers.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
from typing import Dict

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "workload", "generate", "shrink", "tensor_scaled"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    hidden: int
    inter: int
    num_experts: int
    local_begin: int
    num_local: int
    topk: int
    activation: str  # "swiglu" | "swigluoai"
    act_clamp: float
    act_alpha: float
    act_up_bias: float
    weight_format: str  # "fp8" (E4M3) | "fp8e5m2" | "mxfp4" | "bf16" (x, weights, h all BF16)
    routing: str  # "normal" | "zipf"
    zipf_s: float
    seed: int
    scaling: str = "block"  # "block" (UE8M0 blocks) | "tensor" (one float32 scale per tensor)
    h_scale: float = 1.0    # "tensor" only: static scale of the intermediate
    num_shared: int = 0     # shared experts (every token, weight 1), stored after the local ones

    @property
    def rows_capacity(self) -> int:
        return self.tokens * (self.topk + self.num_shared)


_INF = float("inf")

WORKLOADS = [
    # 64 tokens, hidden 256, intermediate 128, 8 experts (all local), top-2, SwiGLU
    Workload("tiny", 64, 256, 128, 8, 0, 8, 2, "swiglu", _INF, 1.0, 0.0, "fp8", "normal", 0.0, 1000),
    # 512 tokens, hidden 2048, intermediate 768, 32 experts (all local), top-4, OAI-SwiGLU
    Workload("oai", 512, 2048, 768, 32, 0, 32, 4, "swigluoai", 7.0, 1.702, 1.0, "fp8", "normal", 0.0, 1001),
    # decode share: 128 tokens, top-8 over 256 experts, local experts 0..31
    Workload("decode", 128, 7168, 2048, 256, 0, 32, 8, "swiglu", _INF, 1.0, 0.0, "fp8", "normal", 0.0, 1002),
    # prefill share with a Zipf(1.1) expert prior on the logits, OAI-SwiGLU
    Workload("prefill_zipf", 4096, 7168, 2048, 256, 0, 32, 8, "swigluoai", 7.0, 1.702, 1.0, "fp8", "zipf", 1.1,
             1003),
    # large share with MXFP4 weights, uniform top-8 routing
    Workload("mxfp4_large", 32768, 7168, 2048, 256, 0, 32, 8, "swiglu", _INF, 1.0, 0.0, "mxfp4", "normal", 0.0,
             1004),
]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def shrink(w: Workload, **changes) -> Workload:
    """Same recipe with some sizes replaced (used for small parity cases)."""
    return dataclasses.replace(w, **changes)


def tensor_scaled(w: Workload, h_scale: float | None = None, **changes) -> Workload:
    """The workload with per-tensor float32 scales.  The static intermediate scale is a
    calibration from the input statistics alone: gate and up pre-activations have variance
    about 0.02^2 * H (unit-variance activations against weights of deviation 0.02), and
    16 of those variances map to the E4M3 maximum 448 (larger values saturate)."""
    if h_scale is None:
        h_scale = float(np.float32(16.0 * 0.02 ** 2 * w.hidden / 448.0))
    return dataclasses.replace(w, scaling="tensor", h_scale=h_scale, **changes)


# ---------------------------------------------------------------------------
# input quantisers (input generation only)

def _pow2_exponent_for(amax: np.ndarray, top: float) -> np.ndarray:
    """Integer e with amax / 2**e <= top, from a float log2 (corrected if rounding undershoots)."""
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.maximum(amax, 1e-300) / top))
    e = e.astype(np.int64)
    over = amax / np.ldexp(1.0, e) > top
    e = e + over.astype(np.int64)
    return e


_FP8 = {"e4m3": (torch.float8_e4m3fn, 448.0), "e5m2": (torch.float8_e5m2, 57344.0)}


def _to_fp8_bytes(v: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(_FP8[fmt][0]).view(torch.uint8).numpy()


def _quant_fp8_blocks(v: np.ndarray, br: int, bc: int, fmt: str = "e4m3"):
    """v [N, K] float32 -> FP8 bytes [N, K] and UE8M0 bytes [ceil(N/br), K/bc] (block br x bc).

    The block scale is the smallest power of two that brings the block's amax within the
    format's largest finite value (448 for E4M3, 57344 for E5M2)."""
    n, kk = v.shape
    nb = (n + br - 1) // br
    pad = nb * br - n
    vp = np.pad(v, ((0, pad), (0, 0))) if pad else v
    blk = np.abs(vp.reshape(nb, br, kk // bc, bc)).max(axis=(1, 3)).astype(np.float64)
    e = _pow2_exponent_for(blk, _FP8[fmt][1])
    e = np.where(blk == 0, 0, e)
    e = np.clip(e, -127, 127)
    sf = (e + 127).astype(np.uint8)
    inv = np.ldexp(np.float32(1.0), (-e).astype(np.int32)).astype(np.float32)
    scaled = (vp.reshape(nb, br, kk // bc, bc) * inv[:, None, :, None]).reshape(nb * br, kk)
    q = _to_fp8_bytes(scaled[:n], fmt)
    return q, sf


def _quant_fp8_tensor(v: np.ndarray, fmt: str = "e4m3"):
    """v float32 -> FP8 bytes and one float32 scale amax / (format maximum) (1.0 for all zeros)."""
    amax = float(np.abs(v).max()) if v.size else 0.0
    s = np.float32(amax / _FP8[fmt][1]) if amax > 0 else np.float32(1.0)
    return _to_fp8_bytes(v / s, fmt), s


def _quant_mxfp4(v: np.ndarray):
    """v [N, K] float32 -> packed E2M1 [N, K/2] and UE8M0 [N, K/32] (OCP MX: X = 2^(floor(log2 amax) - 2)).

    Elements round to the nearest of {0, .5, 1, 1.5, 2, 3, 4, 6} (ties to the even code) and
    saturate at 6; the seven threshold compares below encode exactly that.
    """
    n, kk = v.shape
    b = v.reshape(n, kk // 32, 32)
    amax = np.abs(b).max(axis=2)
    _, ex = np.frexp(amax)  # amax = f * 2**ex, f in [0.5, 1): floor(log2 amax) = ex - 1
    e = np.where(amax == 0, 0, ex.astype(np.int64) - 3)
    e = np.clip(e, -127, 127)
    sf = (e + 127).astype(np.uint8)
    a = np.abs(b) * np.ldexp(np.float32(1.0), (-e).astype(np.int32)).astype(np.float32)[:, :, None]
    code = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5)
            + (a > 5.0)).astype(np.uint8)
    code |= (np.signbit(b) & (code > 0)).astype(np.uint8) << 3
    nib = code.reshape(n, kk)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, sf


def _bf16_round(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()


def generate(w: Workload, seed: int | None = None, threads: int = 8, with_bf16: bool = False) -> Dict[str, np.ndarray]:
    """All layer inputs for workload ``w`` as host numpy arrays (seeded, deterministic).

    ``with_bf16`` also returns the bf16 activations before their quantisation, as bit
    patterns ``x_bf16`` [T, H] uint16.

    Seed tree: SeedSequence(seed).spawn(2 + 2 * (E_loc + S)) gives the streams for the
    logits, the activations, then W1 and W2 of each local expert in order, the S shared
    experts last; experts are drawn in a thread pool, which does not change the values.
    """
    seed = w.seed if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(2 + 2 * (w.num_local + w.num_shared))
    rng = lambda i: np.random.Generator(np.random.PCG64(kids[i]))
    T, H, I, E = w.tokens, w.hidden, w.inter, w.num_experts
    EL = w.num_local + w.num_shared  # weight sets: routed local experts, then shared ones
    logits = rng(0).standard_normal((T, E), dtype=np.float32)
    if w.routing == "zipf":
        prior = (-w.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
        logits = (logits + prior[None, :]).astype(np.float32)
    xf = _bf16_round(rng(1).standard_normal((T, H), dtype=np.float32))
    if w.scaling not in ("block", "tensor"):
        raise ValueError(f"unknown scaling {w.scaling}")
    tensor = w.scaling == "tensor"
    if tensor and w.weight_format in ("mxfp4", "bf16"):
        raise ValueError("per-tensor scaling needs FP8 weights")
    bf16 = w.weight_format == "bf16"
    if bf16:  # BF16 layer: bit patterns, no scale tensors
        x = (xf.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        x_sf = np.zeros(0, np.uint8)
    elif tensor:
        x, xs = _quant_fp8_tensor(xf)
        x_sf = np.array([xs], np.float32)
    else:
        x, x_sf = _quant_fp8_blocks(xf, 1, 128)
    out = {"logits": np.ascontiguousarray(logits), "x": x, "x_sf": x_sf}
    if with_bf16:
        out["x_bf16"] = (xf.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    del xf
    if w.weight_format not in ("fp8", "fp8e5m2", "mxfp4", "bf16"):
        raise ValueError(f"unknown weight format {w.weight_format}")
    fp8 = w.weight_format != "mxfp4"
    f8 = "e5m2" if w.weight_format == "fp8e5m2" else "e4m3"
    w1 = np.empty((EL, 2 * I, H if fp8 else H // 2), np.uint8)
    w1_sf = np.empty((EL, 2 * I // 128, H // 128) if fp8 else (EL, 2 * I, H // 32), np.uint8)
    if tensor:
        w1_sf = np.empty(EL, np.float32)
    w2 = np.empty((EL, H, I if fp8 else I // 2), np.uint8)
    w2_sf = np.empty((EL, H // 128, I // 128) if fp8 else (EL, H, I // 32), np.uint8)
    if tensor:
        w2_sf = np.empty(EL, np.float32)

    if bf16:
        w1 = np.empty((EL, 2 * I, H), np.uint16)
        w2 = np.empty((EL, H, I), np.uint16)
        w1_sf = w2_sf = np.zeros(0, np.uint8)

    def one(e):
        for which, shape, dst, dsf in ((0, (2 * I, H), w1, w1_sf), (1, (H, I), w2, w2_sf)):
            a = rng(2 + 2 * e + which).standard_normal(shape, dtype=np.float32)
            a *= np.float32(0.02)
            if bf16:
                dst[e] = (_bf16_round(a).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
                continue
            if tensor:
                q, s = _quant_fp8_tensor(a, f8)
            else:
                q, s = _quant_fp8_blocks(a, 128, 128, f8) if fp8 else _quant_mxfp4(a)
            dst[e], dsf[e] = q, s

    with cf.ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(EL)))
    out.update(w1=w1, w1_sf=w1_sf, w2=w2, w2_sf=w2_sf)
    return out
