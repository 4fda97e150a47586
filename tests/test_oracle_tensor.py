"""Pins of the oracle's per-tensor scaling variant (CPU): float32 scales for x and each
expert's weights, a static float32 scale for the intermediate with E4M3 saturation."""
import numpy as np
import pytest
import torch

from moe_expert_layer_amd import synth
from oracle import moe_oracle as O
from tests import brute


def _tiny(**kw):
    base = synth.shrink(synth.workload("tiny"), tokens=6, hidden=128, inter=128, num_experts=4, num_local=4, topk=2)
    return synth.shrink(base, **kw)


def test_requant_tensor_grid_ties_and_saturation():
    s = 0.375  # any positive float32
    grid = brute.e4m3_table()[:0x7F]  # non-negative finite E4M3 values
    # exact multiples of grid values land on their codes
    assert np.array_equal(O.requant_tensor((grid * s).astype(np.float32), s), np.arange(0x7F, dtype=np.uint8))
    # midway between 1.0 (0x38) and 1.125 (0x39) goes to the even mantissa, 1.0
    assert O.requant_tensor(np.float32([1.0625 * s]), s)[0] == 0x38
    # beyond the E4M3 range: saturate to +-448 (0x7E / 0xFE), never NaN
    got = O.requant_tensor(np.float32([500 * s, -1e6 * s, 464 * s]), s)
    assert list(got) == [0x7E, 0xFE, 0x7E]
    # agrees with torch's E4M3 cast of the in-range quotient
    rng = np.random.default_rng(3)
    h = (rng.standard_normal(4096) * 40).astype(np.float32)
    q = np.clip(h.astype(np.float64) / np.float64(np.float32(s)), -448, 448)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.requant_tensor(h, s), ref)


@pytest.mark.parametrize("d", [
    synth.tensor_scaled(_tiny(seed=21)),
    # OAI with a small static scale: values above 448 * h_scale = 0.224 saturate
    synth.tensor_scaled(_tiny(activation="swigluoai", act_clamp=7.0, act_alpha=1.702, act_up_bias=1.0, seed=22),
                        h_scale=5e-4),
    synth.tensor_scaled(_tiny(weight_format="fp8e5m2", num_experts=8, local_begin=3, num_local=4, topk=3, seed=23)),
])
def test_tensor_layer_matches_token_by_token_bruteforce(d):
    inp = synth.generate(d)
    assert inp["x_sf"].shape == (1,) and inp["w1_sf"].shape == (d.num_local,)
    out = O.layer(d, inp)
    ref = brute.layer_bruteforce(d, inp)
    err = np.abs(out["y64"] - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err < 1e-12
    assert np.array_equal(out["y_bf16"], O.bf16_rne_bits(ref))
    if d.h_scale == 5e-4:
        assert np.isin(out["h"], [0x7E, 0xFE]).any()  # the saturation is exercised


def test_tensor_w2_scale_is_linear():
    """Doubling every expert's W2 scale doubles the output exactly (a power-of-two factor)."""
    d = synth.tensor_scaled(synth.shrink(synth.workload("tiny"), tokens=32, seed=24))
    inp = synth.generate(d)
    a = O.layer(d, inp)
    inp2 = dict(inp)
    inp2["w2_sf"] = (inp["w2_sf"] * 2).astype(np.float32)
    b = O.layer(d, inp2)
    assert np.array_equal(b["y64"], 2 * a["y64"])
