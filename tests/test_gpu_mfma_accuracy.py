"""Accumulation precision of the gfx950 matrix-instruction forms the layer can use, against an
exact host dot product.

Operands are drawn like the layer's FC1 (activations N(0,1) in bf16, quantised to E4M3 with
1x128 UE8M0 scales; weights N(0, 0.02) quantised to E4M3 with 128x128 UE8M0 scales, or to
MXFP4), over the FC1 contraction length K = 7168.  Only the E4M3 / E2M1 codes enter the probe
GEMMs (all scales 1): the block scales are powers of two and move every product of a block by
the same exact factor.  Every product of two such codes is a multiple of 2^-18 below 2^17 in
magnitude, so the float64 sum is exact in any order.

Measured per form: the error relative to the sum of |products| of each output, the relative
Frobenius error, and the share of E4M3 codes that change when the outputs are requantised with
the layer's 1x128 rule (one scale per 32-output row of a problem here).  A code can only change
where an output lies within the accumulation error of a rounding midpoint, so this share is
what the intermediate requant of FC1 turns accumulation error into.
"""
import numpy as np
import pytest

from moe_expert_layer_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from moe_expert_layer_amd import probe_binding as P
    from tests import gpu_util as G

K = 7168
N = 96  # problems of 32 x 32 outputs


def _operands(seed: int, fp4: bool):
    rng = np.random.default_rng(seed)
    x = synth._bf16_round(rng.standard_normal((N * 32, K), dtype=np.float32))
    a, _ = synth._quant_fp8_blocks(x, 1, 128)
    wv = (0.02 * rng.standard_normal((N * 32, K), dtype=np.float32)).astype(np.float32)
    if fp4:
        b, _ = synth._quant_mxfp4(wv)
    else:
        b, _ = synth._quant_fp8_blocks(wv, 128, 128)
    return a.reshape(N, 32, K), b.reshape(N, 32, -1)


def _decode_e4m3(c):
    return torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


_E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6], np.float64)


def _decode_e2m1(p):
    lo, hi = _E2M1[p & 15], _E2M1[p >> 4]
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.float64)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return out


def _requant_codes(v):
    """E4M3 codes of each 32-value row under the 1x128 rule (smallest 2^e with 448 * 2^e >= amax)."""
    amax = np.abs(v).max(axis=-1, keepdims=True)
    e = np.ceil(np.log2(np.maximum(amax, 1e-300) / 448.0))
    e = np.where(amax / np.ldexp(1.0, e.astype(np.int64)) > 448.0, e + 1, e)
    scaled = (v / np.ldexp(1.0, e.astype(np.int64))).astype(np.float32)
    return torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


FORMS = ["fp32_fma", "scaled_32x32x64", "scaled_32x32x64_split", "scaled_16x16x128", "fp8_32x32x16", "bf16_32x32x16"]


def _measure(fp4: bool, seed: int):
    a, b = _operands(seed, fp4)
    A = _decode_e4m3(a)
    B = _decode_e2m1(b) if fp4 else _decode_e4m3(b)
    exact = np.einsum("pmk,pjk->pmj", A, B)
    sabs = np.einsum("pmk,pjk->pmj", np.abs(A), np.abs(B))
    ref_codes = _requant_codes(exact)
    da, db = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    res = {}
    for form in FORMS:
        if fp4 and form == "fp8_32x32x16":
            continue
        c = torch.zeros((N, 32, 32), dtype=torch.float32, device="cuda")
        P.mfma_gemm(form, da, db, c, b_fp4=fp4)
        torch.cuda.synchronize()
        got = c.cpu().numpy().astype(np.float64)
        err = got - exact
        rel_s = np.abs(err) / np.maximum(sabs, 1e-300)
        flips = float((_requant_codes(got) != ref_codes).mean())
        res[form] = {"rel_fro": float(np.linalg.norm(err) / np.linalg.norm(exact)),
                     "err_over_sabs_median": float(np.median(rel_s)), "err_over_sabs_max": float(rel_s.max()),
                     "bias": float(np.mean(err / np.maximum(sabs, 1e-300))), "code_flips": flips}
        G.say(f"[mfma-accuracy] b={'e2m1' if fp4 else 'e4m3'} seed={seed} {form:24s} rel_fro={res[form]['rel_fro']:.3e} "
              f"|err|/sum|ab| median={res[form]['err_over_sabs_median']:.3e} max={res[form]['err_over_sabs_max']:.3e} "
              f"bias={res[form]['bias']:+.2e} requant code flips={flips:.2e}")
    return res


@pytest.mark.parametrize("fp4", [False, True], ids=["e4m3xe4m3", "e4m3xe2m1"])
def test_mfma_accumulation_precision(fp4):
    res = _measure(fp4, seed=11 + int(fp4))
    # the control (exact products, fp32 fused multiply-add in order) and every instruction form
    # compute the same sums: a wrong operand layout would show as an O(1) error
    assert res["fp32_fma"]["rel_fro"] < 1e-6
    for form, r in res.items():
        assert r["rel_fro"] < 1e-3, (form, r)


def _bf16_bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt", [0, 1, 2], ids=["e4m3", "e5m2", "e2m1"])
def test_scaled_conversion_to_bf16_is_exact(fmt):
    """The scaled conversions (FP8 / FP4 code x 2^(byte - 127) -> BF16) that an exact-sum FC1 can use
    to fold the UE8M0 block scales into its operands: every code under a spread of scale bytes
    gives exactly code * 2^(byte - 127) wherever that value is a normal BF16 number (all E4M3,
    E5M2 and E2M1 values have at most 3 significant bits, so the product is representable)."""
    scales = np.array([1, 40, 100, 120, 127, 128, 135, 160, 200, 240], np.uint8)
    if fmt == 2:
        codes = np.tile(np.arange(256, dtype=np.uint8), 2 * len(scales))  # every pair of nibbles
        n = codes.size * 2
        lo, hi = _E2M1[codes & 15], _E2M1[codes >> 4]
        v = np.empty(n)
        v[0::2], v[1::2] = lo, hi
    else:
        vals = np.array([c for c in range(256) if not ((fmt == 0 and (c & 0x7F) == 0x7F) or (fmt == 1 and (c & 0x7C) == 0x7C))],
                        np.uint8)
        codes = np.resize(vals, 32 * len(scales) * 8)
        n = codes.size
        tt = torch.float8_e4m3fn if fmt == 0 else torch.float8_e5m2
        v = torch.from_numpy(codes.copy()).view(tt).to(torch.float64).numpy()
    sb = np.resize(scales, n // 32).astype(np.uint8)
    expect = v * np.ldexp(1.0, sb.repeat(32).astype(np.int64) - 127)
    out = torch.zeros(n, dtype=torch.int16, device="cuda")
    P.cvt_bf16(fmt, torch.from_numpy(codes).cuda(), torch.from_numpy(sb).cuda(), out)
    torch.cuda.synchronize()
    got = _bf16_bits_to_f64(out.cpu().numpy().view(np.uint16))
    normal = (np.abs(expect) >= 2.0 ** -126) & (np.abs(expect) < 2.0 ** 127) | (expect == 0)
    bad = normal & (got != expect)
    G.say(f"[cvt] fmt={fmt}: {int(normal.sum())} in-range values, {int(bad.sum())} differ")
    assert not bad.any(), list(zip(codes[np.nonzero(bad)[0][:4] // (2 if fmt == 2 else 1)], got[bad][:4], expect[bad][:4]))
    assert normal.mean() > 0.75
