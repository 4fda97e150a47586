"""Pins of the oracle's activation, requantisation and whole-layer evaluation (CPU)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from moe_expert_layer_amd import synth
from oracle import moe_oracle as O
from tests import brute

P = json.load(open(os.path.join(brute.GOLDEN, "oai_swiglu_params.json")))
MM3 = P["minimax_m3"]


def test_activation_closed_forms():
    g = np.array([0.0, 1.0, -3.0])
    u = np.array([5.0, 2.0, 0.5])
    h = O.activation(g, u, "swiglu")
    assert h[0] == 0.0
    assert h[1] == pytest.approx(2.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert h[2] == pytest.approx(-3.0 / (1.0 + math.exp(3.0)) * 0.5, rel=1e-15)


def test_oai_clamps_gate_above_only_and_up_both_sides():
    a, b, c = MM3["alpha"], MM3["up_bias"], MM3["clamp"]
    g = np.array([10.0, -10.0, 3.0, 7.0])
    u = np.array([9.0, -9.0, -2.0, 100.0])
    h = O.activation(g, u, "swigluoai", c, a, b)
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    assert h[0] == pytest.approx(7.0 * sig(a * 7.0) * (7.0 + 1.0), rel=1e-15)   # gate -> 7, up -> 7
    assert h[1] == pytest.approx(-10.0 * sig(-a * 10.0) * (-7.0 + 1.0), rel=1e-15)  # gate not clamped below
    assert h[2] == pytest.approx(3.0 * sig(a * 3.0) * (-2.0 + 1.0), rel=1e-15)
    assert h[3] == pytest.approx(7.0 * sig(a * 7.0) * 8.0, rel=1e-15)


def test_oai_defaults_reduce_to_swiglu_bitwise():
    rng = np.random.default_rng(0)
    g, u = rng.normal(0, 4, 10000), rng.normal(0, 4, 10000)
    dflt = P["defaults_reduce_to_standard_swiglu"]
    a = O.activation(g, u, "swigluoai", np.inf, dflt["alpha"], dflt["up_bias"])
    s = O.activation(g, u, "swiglu")
    assert np.array_equal(a, s)


@pytest.mark.parametrize("amax,byte", [(448.0, 127), (np.nextafter(np.float32(448), np.float32(1e9)), 128),
                                       (224.0, 126), (np.nextafter(np.float32(224), np.float32(1e9)), 127),
                                       (1.0, 119), (0.875, 118), (0.0, 127), (3.0e38, 254 - 0)])
def test_requant_scale_rule(amax, byte):
    h = np.zeros((1, 128), np.float32)
    h[0, 5] = amax
    h[0, 9] = -np.float32(amax) / 3
    codes, sf = O.requant_1x128(h)
    if amax == 3.0e38:
        assert sf[0, 0] == 127 + brute.min_scale_exponent(float(np.float32(amax)))
    else:
        assert sf[0, 0] == byte
    if amax != 0:
        assert brute.decode_e4m3_torch(codes[:, 5])[0] * 2.0 ** (int(sf[0, 0]) - 127) <= float(np.float32(amax)) * (1 + 2 ** -3)


def test_requant_matches_bruteforce_rows():
    rng = np.random.default_rng(5)
    rows = [rng.normal(0, 1, 256), rng.normal(0, 1e-4, 256) * rng.integers(0, 2, 256),
            np.concatenate([np.zeros(128), rng.normal(0, 30, 128)]), rng.standard_cauchy(256)]
    # a row whose values sit exactly on E4M3 rounding ties after scaling
    ties = np.ldexp(1.0 + (2 * rng.integers(0, 8, 256) + 1) / 16.0, rng.integers(-3, 3, 256))
    ties[0] = 448.0
    rows.append(ties)
    h = np.array(rows, dtype=np.float32)
    codes, sf = O.requant_1x128(h)
    for i in range(h.shape[0]):
        bc, bs = brute.requant_row(h[i])
        assert list(sf[i]) == list(bs)
        assert list(codes[i]) == list(bc)


def _tiny(**kw):
    base = synth.shrink(synth.workload("tiny"), tokens=6, hidden=128, inter=128, num_experts=4, num_local=4, topk=2)
    return synth.shrink(base, **kw)


@pytest.mark.parametrize("d", [
    _tiny(),
    _tiny(activation="swigluoai", act_clamp=7.0, act_alpha=1.702, act_up_bias=1.0, seed=11),
    _tiny(num_experts=8, local_begin=2, num_local=3, topk=3, seed=12),
    _tiny(weight_format="mxfp4", seed=13, tokens=4),
    _tiny(weight_format="fp8e5m2", seed=14),
])
def test_layer_matches_token_by_token_bruteforce(d):
    inp = synth.generate(d)
    out = O.layer(d, inp)
    ref = brute.layer_bruteforce(d, inp)
    err = np.abs(out["y64"] - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err < 1e-12
    yb = O.bf16_rne_bits(ref)
    assert np.array_equal(out["y_bf16"], yb)


def test_requant_is_in_effect():
    """Skipping the 1x128 requantisation must move y by about the FP8 quantisation error."""
    d = synth.shrink(synth.workload("tiny"), seed=21)
    inp = synth.generate(d)
    out = O.layer(d, inp)
    ids, w = O.route(inp["logits"], d.topk)
    y = np.zeros_like(out["y64"])
    for t in range(d.tokens):
        x = O.dequant_act(inp["x"][t:t + 1], inp["x_sf"][t:t + 1])
        for j in range(d.topk):
            e = ids[t, j] - d.local_begin
            w1 = O.dequant_weight(inp["w1"][e], inp["w1_sf"][e], "fp8", 2 * d.inter, d.hidden)
            w2 = O.dequant_weight(inp["w2"][e], inp["w2_sf"][e], "fp8", d.hidden, d.inter)
            gu = x @ w1.T
            h = O.activation(gu[:, :d.inter], gu[:, d.inter:], d.activation)
            y[t] += float(w[t, j]) * (h @ w2.T)[0]
    rel = np.linalg.norm(y - out["y64"]) / np.linalg.norm(y)
    assert 3e-3 < rel < 5e-2


def test_exact_integer_layer_bit_exact():
    """Integer-valued operands, unit scales, top-1, OAI with alpha 0: every step is exact."""
    rng = np.random.default_rng(9)
    T, H, I, E = 8, 128, 128, 4
    d = synth.shrink(synth.workload("tiny"), tokens=T, hidden=H, inter=I, num_experts=E, num_local=E, topk=1,
                     activation="swigluoai", act_clamp=np.inf, act_alpha=0.0, act_up_bias=0.0)
    enc = {v: c for c, v in ((c, brute.e4m3_table()[c]) for c in range(0x7F))}
    def ints(shape, lo, hi):
        v = rng.integers(lo, hi + 1, shape)
        return np.vectorize(lambda a: enc[abs(a)] | (0x80 if a < 0 else 0))(v).astype(np.uint8), v
    x, xv = ints((T, H), -3, 3)
    w1, w1v = ints((E, 2 * I, H), -2, 2)
    w2, w2v = ints((E, H, I), -1, 1)
    inp = {"logits": rng.standard_normal((T, E)).astype(np.float32), "x": x,
           "x_sf": np.full((T, H // 128), 127, np.uint8), "w1": w1, "w1_sf": np.full((E, 2 * I // 128, H // 128), 127, np.uint8),
           "w2": w2, "w2_sf": np.full((E, H // 128, I // 128), 127, np.uint8)}
    out = O.layer(d, inp)
    ids = np.argmax(inp["logits"], axis=1)
    for t in range(T):
        e = ids[t]
        g = [int(np.dot(xv[t], w1v[e, n])) for n in range(I)]
        u = [int(np.dot(xv[t], w1v[e, I + n])) for n in range(I)]
        h = [Fraction(gi * ui, 2) for gi, ui in zip(g, u)]  # g * sigmoid(0) * u
        amax = max(abs(v) for v in h)
        byte = 127 if amax == 0 else 127 + brute.min_scale_exponent(float(amax))
        hq = [Fraction(brute.e4m3_table()[brute.e4m3_nearest_code(float(v / Fraction(2) ** (byte - 127)))]) *
              Fraction(2) ** (byte - 127) for v in h]
        y = [sum(hq[n] * int(w2v[e, m, n]) for n in range(I)) for m in range(H)]
        assert [float(v) for v in y] == list(out["y64"][t])
        assert np.array_equal(out["y_bf16"][t], O.bf16_rne_bits(np.array([float(v) for v in y])))


def test_scale_byte_doubling_doubles_output():
    d = synth.shrink(synth.workload("tiny"), seed=31)
    inp = synth.generate(d)
    out = O.layer(d, inp)
    inp2 = dict(inp)
    inp2["w2_sf"] = (inp["w2_sf"].astype(np.int32) + 1).astype(np.uint8)
    out2 = O.layer(d, inp2)
    assert np.array_equal(out2["y64"], 2 * out["y64"])


def test_token_subset_matches_full_layer():
    d = synth.shrink(synth.workload("oai"), tokens=64, hidden=256, inter=256, seed=41)
    inp = synth.generate(d)
    full = O.layer(d, inp)
    toks = np.array([0, 5, 17, 63])
    sub = O.layer_tokens(d, inp, toks)
    assert np.array_equal(sub["y64"], full["y64"][toks])
    assert np.array_equal(sub["h"][sub["h_valid"]], full["h"][sub["h_valid"]])


def test_tokens_without_local_slot_are_zero():
    d = synth.shrink(synth.workload("decode"), tokens=64, hidden=128, inter=128, num_local=4, seed=51)
    inp = synth.generate(d)
    out = O.layer(d, inp)
    loc = (out["slot_to_row"].reshape(d.tokens, d.topk) >= 0).any(1)
    assert (~loc).sum() > 0
    assert np.all(out["y64"][~loc] == 0)


@pytest.mark.parametrize("d", [
    _tiny(num_shared=1, seed=31),
    # shared experts on top of a partial local share (some tokens have no routed local slot)
    _tiny(num_experts=8, local_begin=5, num_local=2, topk=2, num_shared=2, activation="swigluoai", act_clamp=7.0,
          act_alpha=1.702, act_up_bias=1.0, seed=32),
    synth.tensor_scaled(_tiny(num_shared=1, weight_format="fp8e5m2", seed=33)),
])
def test_shared_experts_match_token_by_token_bruteforce(d):
    inp = synth.generate(d)
    assert inp["w1"].shape[0] == d.num_local + d.num_shared
    out = O.layer(d, inp)
    ref = brute.layer_bruteforce(d, inp)
    err = np.abs(out["y64"] - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err < 1e-12
    assert np.array_equal(out["y_bf16"], O.bf16_rne_bits(ref))
    assert out["h"].shape[0] == out["R"] + d.num_shared * d.tokens


def test_shared_expert_equals_routing_every_token_to_it():
    """A shared expert is the same computation as a routed expert that every token picks with
    weight exactly 1 (top-1 over a single local expert whose logit always wins)."""
    d = _tiny(tokens=16, num_local=4, num_shared=1, seed=34)
    inp = synth.generate(d)
    out = O.layer(d, inp)
    # the shared expert alone: zero the routed part by routing every token to a non-local expert
    d1 = synth.shrink(d, num_experts=5, local_begin=4, num_local=1, topk=1, num_shared=0)
    inp1 = dict(inp)
    inp1["logits"] = np.zeros((d.tokens, 5), np.float32)
    inp1["logits"][:, 4] = 10.0  # expert 4 (the only local one) wins for every token
    for key in ("w1", "w1_sf", "w2", "w2_sf"):
        inp1[key] = inp[key][4:5]  # the shared expert's weights as local expert 4
    only_shared = O.layer(d1, inp1)
    assert np.all(only_shared["topk_w"] == 1.0)
    routed = O.layer(synth.shrink(d, num_shared=0), {k: (v[:4] if k.startswith("w") else v) for k, v in inp.items()})
    assert np.allclose(out["y64"], routed["y64"] + only_shared["y64"], rtol=0, atol=1e-12 * np.abs(out["y64"]).max())


@pytest.mark.parametrize("d", [
    _tiny(weight_format="bf16", seed=41),
    _tiny(weight_format="bf16", activation="swigluoai", act_clamp=7.0, act_alpha=1.702, act_up_bias=1.0,
          num_shared=1, seed=42),
])
def test_bf16_layer_matches_token_by_token_bruteforce(d):
    inp = synth.generate(d)
    assert inp["x"].dtype == np.uint16 and inp["w1"].dtype == np.uint16
    out = O.layer(d, inp)
    ref = brute.layer_bruteforce(d, inp)
    err = np.abs(out["y64"] - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err < 1e-12
    assert np.array_equal(out["y_bf16"], O.bf16_rne_bits(ref))


def test_bf16_intermediate_is_one_rounding_of_the_activation():
    """h of the BF16 layer equals torch's bfloat16 cast of the float32 activation of the
    float64 gate/up products (computed here from torch's bfloat16 decode of the operands)."""
    d = _tiny(weight_format="bf16", tokens=8, seed=43)
    inp = synth.generate(d)
    out = O.layer(d, inp)
    e = 0
    rows = np.arange(out["offsets"][e], out["offsets"][e + 1])
    toks = out["row_to_slot"][rows] // d.topk
    x = brute.bf16_decode_torch(inp["x"][toks])
    gu = x @ brute.bf16_decode_torch(inp["w1"][e]).T
    g, u = gu[:, :d.inter], gu[:, d.inter:]
    h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    assert np.array_equal(out["h"][rows], brute.bf16_round_torch(h))
