"""Seeded random layer configurations against the oracle, over the descriptor's valid range at
small sizes: token counts, hidden and intermediate sizes, routing width, local share, top-k,
weight formats, activations, scaling modes, shared experts and forced tile variants.

Checks, for the three-call path and the one-call entry point:
* routing (ids, counts, offsets, row<->slot maps) bit-exact, weights within one fp32 ulp;
* the intermediate h: every differing code within one grid step of the oracle's (the
  h_agreement rule), and at least 99% of codes equal;
* every token whose intermediate rows all equal the oracle's bit for bit: y within one
  bfloat16 step plus 1e-4 of the token's largest |y| (FC2 runs on identical inputs there,
  so only the MFMA's own rounding and the final bf16 rounding remain);
* the relative Frobenius error of y within the 2e-3 bar, for every draw (layers of this size
  sum FC1 exactly, so requantised h codes flip only where fp32 rounding itself decides).
"""
import os

import numpy as np
import pytest

from moe_expert_layer_amd import synth
from oracle import moe_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_util as G

TOL = 2e-3
N_CASES = int(os.environ.get("MOE_RANDOM_CASES", "32"))  # a longer sweep: MOE_RANDOM_CASES=300


def random_case(i: int):
    """Configuration i: drawn from its own seed, within the library's limits."""
    rng = np.random.default_rng(5000 + i)
    fmt = ["fp8", "fp8e5m2", "mxfp4", "bf16"][int(rng.integers(4))]
    E = int(rng.choice([1, 2, 3, 8, 16, 33, 64, 200]))
    EL = int(rng.integers(1, min(E, 16) + 1))
    e0 = int(rng.integers(0, E - EL + 1))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1, 300))
    H = 128 * int(rng.integers(1, 7))
    I = 128 * int(rng.integers(1, 5))
    oai = bool(rng.integers(2))
    S = int(rng.integers(1, 3)) if rng.random() < 0.3 else 0
    variant = int(rng.integers(-1, 3))
    tensor = fmt in ("fp8", "fp8e5m2") and rng.random() < 0.3
    base = synth.workload("oai" if oai else "tiny")
    w = synth.shrink(base, name=f"random{i}", tokens=T, hidden=H, inter=I, num_experts=E, local_begin=e0,
                     num_local=EL, topk=k, weight_format=fmt, num_shared=S, seed=7000 + i)
    if tensor:
        w = synth.tensor_scaled(w)
    return w, variant


def _token_rows(slot_to_row, T, k, R, S):
    rows = [list(r[r >= 0]) for r in slot_to_row.reshape(T, k)]
    for t in range(T):
        rows[t] += [R + s * T + t for s in range(S)]
    return rows


def _check(name, w, got, ref):
    G.check_routing(got, ref)
    be, se = G.h_agreement(got["h"], got["h_sf"], ref["h"], ref["h_sf"])
    assert be >= 0.99 and se >= 0.99, (name, be, se)
    T, k, S, R = w.tokens, w.topk, w.num_shared, got["R"]
    same = np.all(got["h"] == ref["h"], axis=1) & np.all(got["h_sf"] == ref["h_sf"], axis=1)
    a, b = G.bf16_to_f64(got["y_bf16"]), G.bf16_to_f64(ref["y_bf16"])
    clean = 0
    for t, rows in enumerate(_token_rows(ref["slot_to_row"], T, k, R, S)):
        if not all(same[r] for r in rows):
            continue
        clean += 1
        big = np.maximum(np.abs(a[t]), np.abs(b[t]))
        _, ex = np.frexp(big)
        step = np.ldexp(1.0, ex - 8)  # one bfloat16 step at the larger magnitude
        floor = 1e-4 * np.abs(b[t]).max() if b[t].size else 0.0
        bad = np.abs(a[t] - b[t]) > step + floor
        assert not bad.any(), (name, t, np.nonzero(bad)[0][:8], a[t][bad][:4], b[t][bad][:4])
    err = G.rel_fro(a, b)
    G.say(f"[random] {name}: R={R} clean tokens {clean}/{T} rel_fro={err:.3e} h_bytes_equal={be:.5f}")
    assert err <= TOL, (name, err)
    return err


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_config_against_oracle(i):
    w, variant = random_case(i)
    G.say(f"[random] case {i}: T={w.tokens} H={w.hidden} I={w.inter} E={w.num_experts} e0={w.local_begin} "
          f"EL={w.num_local} k={w.topk} fmt={w.weight_format} act={w.activation} scaling={w.scaling} "
          f"S={w.num_shared} variant={variant}")
    inp = synth.generate(w)
    ref = O.layer(w, inp)
    dev = G.upload(inp)
    got = G.run_split(w, dev, variant=variant)
    _check(f"case {i}", w, got, ref)
    one = G.run_layer(w, dev, variant=variant)
    assert np.array_equal(one["y_bf16"], got["y_bf16"])


@pytest.mark.parametrize("i", [171, 216])
def test_named_sweep_draws(i):
    """Two draws of the 300-draw sweep that once missed the 2e-3 bar (2.03e-3: MXFP4, T = 288,
    H = 640, I = 256, a two-expert share every token reaches; 2.22e-3: FP8, T = 209, H = 512,
    I = 128).  Their excess came from requantised h codes flipped by the FP8 matrix
    instructions' summation error; layers of this size now sum FC1 exactly."""
    w, variant = random_case(i)
    G.say(f"[random] named draw {i}: T={w.tokens} H={w.hidden} I={w.inter} E={w.num_experts} EL={w.num_local} "
          f"k={w.topk} fmt={w.weight_format} variant={variant}")
    inp = synth.generate(w)
    ref = O.layer(w, inp)
    dev = G.upload(inp)
    got = G.run_split(w, dev, variant=variant)
    err = _check(f"draw {i}", w, got, ref)
    assert err <= TOL, err
