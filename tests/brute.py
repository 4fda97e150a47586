"""Independent brute-force references used to pin the oracle (CPU, tiny sizes only).

Nothing here is shared with the oracle: codecs come from torch's float8 dtypes or
from the OCP table fixture, rounding is a nearest-value search over every finite
E4M3 value, scale exponents are searched with exact rationals, and the FFN is
evaluated token by token with explicit loops.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e4m3_table():
    """code -> value for all 256 E4M3FN codes (torch decode; NaN for 0x7F/0xFF)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e5m2_table():
    """code -> value for all 256 E5M2 codes (torch decode; +-inf and NaN at exponent 31)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e5m2).to(torch.float64).numpy()


_E4 = e4m3_table()
_E5 = e5m2_table()
_FINITE = [(c, Fraction(float(_E4[c]))) for c in range(256) if not math.isnan(_E4[c])]


def e2m1_value(nib: int) -> float:
    tab = json.load(open(os.path.join(GOLDEN, "e2m1_values.json")))
    mag = tab["codes_0_to_7"][nib & 7]
    return -mag if nib & tab["sign_bit"] else mag


def e4m3_nearest_code(v: float) -> int:
    """Nearest finite E4M3 value; on a tie the code with even mantissa; sign kept for zero."""
    fv = Fraction(v)
    best = None
    for c, val in _FINITE:
        if (c >> 7) != (1 if math.copysign(1.0, v) < 0 else 0):
            continue  # same sign half of the table only
        dist = abs(val - fv)
        key = (dist, c & 1)  # smaller distance, then even mantissa (lowest mantissa bit 0)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def min_scale_exponent(amax: float) -> int:
    """Smallest integer e with 448 * 2**e >= amax, by exact rational search."""
    a = Fraction(amax)
    e = -200
    while Fraction(448) * Fraction(2) ** e < a:
        e += 1
    return e


def requant_row(h: np.ndarray):
    """float32 row [I] -> (codes [I], scale bytes [I/128]) by brute force."""
    codes, scales = [], []
    for b in range(h.size // 128):
        blk = [float(v) for v in h[b * 128:(b + 1) * 128]]
        amax = max(abs(v) for v in blk)
        if amax == 0:
            byte = 127
        else:
            byte = min(max(min_scale_exponent(amax) + 127, 0), 254)
        scales.append(byte)
        for v in blk:
            codes.append(e4m3_nearest_code(math.ldexp(v, -(byte - 127))))
    return np.array(codes, dtype=np.uint8), np.array(scales, dtype=np.uint8)


def decode_e4m3_torch(codes: np.ndarray) -> np.ndarray:
    return _E4[codes.astype(np.int64)]


def decode_e5m2_torch(codes: np.ndarray) -> np.ndarray:
    return _E5[codes.astype(np.int64)]


def sigmoid(z: float) -> float:
    if z >= 0:
        return 1.0 / (1.0 + math.exp(-z))
    ez = math.exp(z)
    return ez / (1.0 + ez)


def act_scalar(g, u, kind, clamp, alpha, bias):
    if kind == "swiglu":
        return g * sigmoid(g) * u
    gc = min(g, clamp)
    uc = max(-clamp, min(u, clamp))
    return gc * sigmoid(alpha * gc) * (uc + bias)


def weight_dense(w, sf, fmt, rows, cols):
    """Dequantise one expert's weight with explicit loops over blocks."""
    out = np.zeros((rows, cols))
    if fmt in ("fp8", "fp8e5m2"):
        vals = decode_e4m3_torch(w) if fmt == "fp8" else decode_e5m2_torch(w)
        for rb in range(rows // 128):
            for cb in range(cols // 128):
                s = 2.0 ** (int(sf[rb, cb]) - 127)
                out[rb * 128:(rb + 1) * 128, cb * 128:(cb + 1) * 128] = vals[rb * 128:(rb + 1) * 128,
                                                                              cb * 128:(cb + 1) * 128] * s
    else:
        for r in range(rows):
            for c in range(cols):
                byte = int(w[r, c // 2])
                nib = byte & 0xF if c % 2 == 0 else byte >> 4
                out[r, c] = e2m1_value(nib) * 2.0 ** (int(sf[r, c // 32]) - 127)
    return out


def topk_bruteforce(logits_row, k):
    order = sorted(range(len(logits_row)), key=lambda e: (-float(logits_row[e]), e))
    ids = order[:k]
    ls = [Fraction(float(logits_row[i])) for i in ids]
    return ids, ls


def bf16_decode_torch(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 through torch's bfloat16 dtype."""
    return torch.from_numpy(np.ascontiguousarray(bits).astype(np.uint16).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def bf16_round_torch(h32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns by torch's cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(h32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def requant_tensor_row(h: np.ndarray, h_scale: float):
    """float32 row -> E4M3 codes of h / h_scale (exact rational quotient, saturated at 448)."""
    s = Fraction(float(np.float32(h_scale)))
    out = []
    for v in h:
        q = Fraction(float(v)) / s
        q = max(Fraction(-448), min(Fraction(448), q))
        out.append(e4m3_nearest_code(q if q != 0 else math.copysign(0.0, float(v))))
    return np.array(out, dtype=np.uint8)


def layer_bruteforce(d, inputs):
    """Token-by-token dense evaluation: y[t] = sum_j w_tj * FFN_{e_tj}(x_t), float64."""
    T, H, I, k = d.tokens, d.hidden, d.inter, d.topk
    tensor = getattr(d, "scaling", "block") == "tensor"
    bf16 = d.weight_format == "bf16"
    S = getattr(d, "num_shared", 0)
    NE = d.num_local + S  # weight sets: routed local experts, then shared experts
    xs = np.zeros((T, H))
    if bf16:
        xs = bf16_decode_torch(inputs["x"])
    else:
        xv = decode_e4m3_torch(inputs["x"])
        for t in range(T):
            for c in range(H):
                s = float(inputs["x_sf"][0]) if tensor else 2.0 ** (int(inputs["x_sf"][t, c // 128]) - 127)
                xs[t, c] = xv[t, c] * s
    if bf16:
        w1 = [bf16_decode_torch(inputs["w1"][e]) for e in range(NE)]
        w2 = [bf16_decode_torch(inputs["w2"][e]) for e in range(NE)]
    elif tensor:
        dec = decode_e4m3_torch if d.weight_format == "fp8" else decode_e5m2_torch
        w1 = [dec(inputs["w1"][e]) * float(inputs["w1_sf"][e]) for e in range(NE)]
        w2 = [dec(inputs["w2"][e]) * float(inputs["w2_sf"][e]) for e in range(NE)]
    else:
        w1 = [weight_dense(inputs["w1"][e], inputs["w1_sf"][e], d.weight_format, 2 * I, H) for e in range(NE)]
        w2 = [weight_dense(inputs["w2"][e], inputs["w2_sf"][e], d.weight_format, H, I) for e in range(NE)]
    y = np.zeros((T, H))
    for t in range(T):
        ids, ls = topk_bruteforce(inputs["logits"][t], k)
        ex = [math.exp(float(l - ls[0])) for l in ls]
        tot = 0.0
        for v in ex:
            tot += v
        pairs = [(e - d.local_begin, float(np.float32(ex[j] / tot))) for j, e in enumerate(ids)]
        pairs = [(le, wt) for le, wt in pairs if 0 <= le < d.num_local]  # local routed slots
        pairs += [(d.num_local + s, 1.0) for s in range(S)]  # shared experts after them, weight 1
        for le, wt in pairs:
            g = np.array([sum(xs[t, c] * w1[le][n, c] for c in range(H)) for n in range(I)])
            u = np.array([sum(xs[t, c] * w1[le][I + n, c] for c in range(H)) for n in range(I)])
            h = np.array([act_scalar(g[n], u[n], d.activation, d.act_clamp, d.act_alpha, d.act_up_bias)
                          for n in range(I)], dtype=np.float32)
            if bf16:
                hd = bf16_decode_torch(bf16_round_torch(h))
            elif tensor:
                hq = requant_tensor_row(h, d.h_scale)
                hd = np.array([decode_e4m3_torch(hq[n:n + 1])[0] * float(np.float32(d.h_scale)) for n in range(I)])
            else:
                hq, hs = requant_row(h)
                hd = np.array([decode_e4m3_torch(hq[n:n + 1])[0] * 2.0 ** (int(hs[n // 128]) - 127)
                               for n in range(I)])
            for m in range(H):
                y[t, m] += wt * sum(hd[n] * w2[le][m, n] for n in range(I))
    return y
