"""Seeded synthetic inputs for the MoE expert layer.

This module only *makes inputs*: routing logits, FP8 E4M3 activations with 1x128
UE8M0 scales, and expert weights as FP8 E4M3 with 128x128 UE8M0 block scales or
as MXFP4 (E2M1 nibbles with one UE8M0 scale per 32 elements).  It holds none of
the layer's arithmetic (routing, grouping, GEMMs, activation, requantisation,
combine); both the HIP path and the CPU oracle consume the bytes it returns.

Encodings of the produced bytes (what both consumers must assume):
  * E4M3 is the OCP 8-bit "E4M3FN" format (bias 7, max 448, no inf).
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

import dataclasses
import math
from typing import Dict

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "workload", "generate", "shrink"]


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
    weight_format: str  # "fp8" | "mxfp4"
    routing: str  # "normal" | "zipf"
    zipf_s: float
    seed: int

    @property
    def rows_capacity(self) -> int:
        return self.tokens * self.topk


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


def _to_e4m3_bytes(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _quant_fp8_blocks(v: np.ndarray, br: int, bc: int):
    """v [N, K] float32 -> E4M3 bytes [N, K] and UE8M0 bytes [ceil(N/br), K/bc] (block br x bc)."""
    n, kk = v.shape
    nb = (n + br - 1) // br
    pad = nb * br - n
    vp = np.pad(v, ((0, pad), (0, 0))) if pad else v
    blk = np.abs(vp.reshape(nb, br, kk // bc, bc)).max(axis=(1, 3)).astype(np.float64)
    e = _pow2_exponent_for(blk, 448.0)
    e = np.where(blk == 0, 0, e)
    e = np.clip(e, -127, 127)
    sf = (e + 127).astype(np.uint8)
    inv = np.ldexp(np.float32(1.0), (-e).astype(np.int32)).astype(np.float32)
    scaled = (vp.reshape(nb, br, kk // bc, bc) * inv[:, None, :, None]).reshape(nb * br, kk)
    q = _to_e4m3_bytes(scaled[:n])
    return q, sf


_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MID = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2


def _quant_mxfp4(v: np.ndarray):
    """v [N, K] float32 -> packed E2M1 [N, K/2] and UE8M0 [N, K/32] (OCP MX: X = 2^(floor(log2 amax) - 2))."""
    n, kk = v.shape
    b = v.reshape(n, kk // 32, 32).astype(np.float64)
    amax = np.abs(b).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.maximum(amax, 1e-300))).astype(np.int64) - 2
    e = np.where(amax == 0, 0, e)
    e = np.clip(e, -127, 127)
    sf = (e + 127).astype(np.uint8)
    a = np.abs(b) * np.ldexp(1.0, -e)[:, :, None]
    idx = np.searchsorted(_E2M1_MID, a, side="left")
    tie = np.isin(a, _E2M1_MID)
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)  # ties go to the even mantissa
    idx = np.minimum(idx, 7)  # saturate at 6
    nib = (idx | (np.signbit(b) & (idx > 0)) .astype(np.int64) << 3).astype(np.uint8).reshape(n, kk)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, sf


def _bf16_round(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()


def generate(w: Workload, seed: int | None = None) -> Dict[str, np.ndarray]:
    """All layer inputs for workload ``w`` as host numpy arrays (seeded, deterministic)."""
    seed = w.seed if seed is None else seed
    g_logit, g_x, g_w1, g_w2 = [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(4)]
    T, H, I, E = w.tokens, w.hidden, w.inter, w.num_experts
    logits = g_logit.standard_normal((T, E), dtype=np.float32)
    if w.routing == "zipf":
        prior = (-w.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
        logits = (logits + prior[None, :]).astype(np.float32)
    xf = _bf16_round(g_x.standard_normal((T, H), dtype=np.float32))
    x, x_sf = _quant_fp8_blocks(xf, 1, 128)
    out = {"logits": np.ascontiguousarray(logits), "x": x, "x_sf": x_sf}
    w1s, w1sf, w2s, w2sf = [], [], [], []
    for _ in range(w.num_local):
        a = (0.02 * g_w1.standard_normal((2 * I, H), dtype=np.float32)).astype(np.float32)
        if w.weight_format == "fp8":
            q, s = _quant_fp8_blocks(a, 128, 128)
        else:
            q, s = _quant_mxfp4(a)
        w1s.append(q)
        w1sf.append(s)
        b = (0.02 * g_w2.standard_normal((H, I), dtype=np.float32)).astype(np.float32)
        if w.weight_format == "fp8":
            q, s = _quant_fp8_blocks(b, 128, 128)
        else:
            q, s = _quant_mxfp4(b)
        w2s.append(q)
        w2sf.append(s)
    out["w1"] = np.stack(w1s)
    out["w1_sf"] = np.stack(w1sf)
    out["w2"] = np.stack(w2s)
    out["w2_sf"] = np.stack(w2sf)
    return out
