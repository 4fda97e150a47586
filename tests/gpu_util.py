"""Helpers for the GPU parity tests: upload inputs, call the C ABI, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from moe_expert_layer_amd import binding as B


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(inp):
    # bfloat16 bit patterns travel as int16 (same bytes)
    return {k: torch.from_numpy(np.ascontiguousarray(v.view(np.int16) if v.dtype == np.uint16 else v)).cuda()
            for k, v in inp.items()}


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def i32(*shape):
    return torch.empty(shape, dtype=torch.int32, device="cuda")


def run_layer(w, dev, variant=-1):
    """Fused moe_layer with every optional routing output requested."""
    d = B.desc_from_workload(w, variant)
    ws = B.alloc_workspace(d)
    T, k, EL = w.tokens, w.topk, w.num_local
    y = torch.empty((T, w.hidden), dtype=torch.int16, device="cuda")
    ids, tw = i32(T, k), torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts, offsets, r2s, s2r = i32(EL), i32(EL + 1), i32(T * k), i32(T * k)
    B.moe_layer(d, dev["logits"], dev["x"], dev["x_sf"], dev["w1"], dev["w1_sf"], dev["w2"], dev["w2_sf"], y, ws,
                ids, tw, counts, offsets, r2s, s2r)
    torch.cuda.synchronize()
    return {"y_bf16": y.cpu().numpy().view(np.uint16), "topk_ids": ids.cpu().numpy(), "topk_w": tw.cpu().numpy(),
            "counts": counts.cpu().numpy(), "offsets": offsets.cpu().numpy(), "row_to_slot": r2s.cpu().numpy(),
            "slot_to_row": s2r.cpu().numpy()}


def run_split(w, dev, variant=-1):
    """The three-call path; also returns h / h_sf (per-tensor scaling: h_sf is passed as NULL
    and returned as zeros)."""
    d = B.desc_from_workload(w, variant)
    ws = B.alloc_workspace(d)
    T, k, EL, I = w.tokens, w.topk, w.num_local, w.inter
    S = getattr(w, "num_shared", 0)
    ids, tw = i32(T, k), torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts, offsets, r2s, s2r = i32(EL), i32(EL + 1), i32(T * k), i32(T * k)
    B.moe_route_permute(d, dev["logits"], ids, tw, counts, offsets, r2s, s2r, ws)
    h = torch.empty((T * (k + S), I), dtype=torch.uint8, device="cuda")  # routed rows, then shared
    tensor = getattr(w, "scaling", "block") == "tensor"
    bf16 = w.weight_format == "bf16"
    if bf16:  # h holds bfloat16 values; no scales
        h = torch.empty((T * (k + S), I), dtype=torch.int16, device="cuda")
    h_sf = None if tensor or bf16 else torch.empty((T * (k + S), I // 128), dtype=torch.uint8, device="cuda")
    B.moe_grouped_fc1_swiglu(d, dev["x"], dev["x_sf"], dev["w1"], dev["w1_sf"], offsets, r2s, h, h_sf, ws)
    y = torch.empty((T, w.hidden), dtype=torch.int16, device="cuda")
    B.moe_grouped_fc2_combine(d, h, h_sf, dev["w2"], dev["w2_sf"], offsets, r2s, s2r, tw, y, ws)
    torch.cuda.synchronize()
    R = int(offsets[-1].item())
    NR = R + S * T
    hs = np.zeros((NR, I // 128), np.uint8) if tensor or bf16 else h_sf[:NR].cpu().numpy()
    hh = h[:NR].cpu().numpy()
    return {"y_bf16": y.cpu().numpy().view(np.uint16), "h": hh.view(np.uint16) if bf16 else hh, "h_sf": hs,
            "R": R, "offsets": offsets.cpu().numpy(), "row_to_slot": r2s.cpu().numpy(),
            "slot_to_row": s2r.cpu().numpy(), "topk_ids": ids.cpu().numpy(), "topk_w": tw.cpu().numpy(),
            "counts": counts.cpu().numpy()}


def check_routing(got, ref, R=None):
    assert np.array_equal(got["topk_ids"], ref["topk_ids"]), "topk ids differ"
    assert np.array_equal(got["counts"], ref["counts"]), "counts differ"
    assert np.array_equal(got["offsets"], ref["offsets"]), "offsets differ"
    assert np.array_equal(got["row_to_slot"], ref["row_to_slot"]), "row_to_slot differs"
    assert np.array_equal(got["slot_to_row"], ref["slot_to_row"]), "slot_to_row differs"
    gw, rw = got["topk_w"].view(np.int32), ref["topk_w"].view(np.int32)
    ulps = np.abs(gw.astype(np.int64) - rw.astype(np.int64))
    assert ulps.max() <= 1, f"routing weights differ by {ulps.max()} ulp"


FP8_RANGE_EPS = 3e-5
BF16_ROW_EPS = 1e-5


def _e4m3_value(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int64)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * 2.0 ** (e - 7))
    return np.where(c >> 7, -mag, mag)


def h_agreement(gh, ghs, rh, rhs, valid=None):
    """Fractions of equal E4M3 bytes / scale bytes.

    Where the scale bytes agree, two differing codes must decode to values at most one
    E4M3 grid step (of the larger magnitude) plus FP8_RANGE_EPS * 448 apart: the two sides
    round activation values that differ by the GPU's accumulation error, which the scaled
    MFMA keeps near 1e-5 of the block's range (so in the subnormal range, where the grid
    step is 2^-9, a couple of steps).  Returns (byte_equal_fraction, scale_equal_fraction).
    """
    if valid is not None:
        gh, ghs, rh, rhs = gh[valid], ghs[valid], rh[valid], rhs[valid]
    if gh.dtype == np.uint16:
        # BF16 intermediate: equal, or one bfloat16 step (of the larger magnitude) apart plus
        # the accumulation error, taken as BF16_ROW_EPS of the row's largest magnitude
        a, b = bf16_to_f64(gh), bf16_to_f64(rh)
        big = np.maximum(np.abs(a), np.abs(b))
        _, ex = np.frexp(big)
        step = np.ldexp(1.0, ex - 8)
        floor = BF16_ROW_EPS * np.abs(b).max(axis=-1, keepdims=True) if b.size else 0.0
        bad = np.abs(a - b) > step + floor
        if bad.any():
            rr, cc = np.nonzero(bad)
            detail = [(int(r), int(c), float(a[r, c]), float(b[r, c])) for r, c in zip(rr[:8], cc[:8])]
            raise AssertionError(f"{int(bad.sum())} bfloat16 intermediate values differ by more than one step: {detail}")
        return (float((gh == rh).mean()) if gh.size else 1.0), 1.0
    sf_eq = float((ghs == rhs).mean()) if ghs.size else 1.0
    same_sf = np.repeat(ghs == rhs, 128, axis=1)
    eq = (gh == rh) | (((gh & 0x7F) == 0) & ((rh & 0x7F) == 0))
    byte_eq = float(eq.mean()) if eq.size else 1.0
    bad = (~eq) & same_sf
    if bad.any():
        a, b = _e4m3_value(gh[bad]), _e4m3_value(rh[bad])
        big = np.maximum(np.abs(a), np.abs(b))
        _, ex = np.frexp(big)
        step = np.where(big >= 2.0 ** -6, np.ldexp(1.0, ex - 4), 2.0 ** -9)
        ok = np.abs(a - b) <= step + FP8_RANGE_EPS * 448.0
        if not ok.all():
            rr, cc = np.nonzero(bad)
            i = np.nonzero(~ok)[0][:8]
            detail = [(int(rr[j]), int(cc[j]), hex(int(gh[bad][j])), hex(int(rh[bad][j])), float(a[j]), float(b[j]))
                      for j in i]
            raise AssertionError(f"{int((~ok).sum())} requant codes differ by more than one E4M3 step: {detail}")
    return byte_eq, sf_eq
