"""Pins of the oracle's routing and grouping: brute force, closed forms, invariants (CPU)."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import brute


def _logits(rng, t, e, ties=False):
    l = rng.standard_normal((t, e)).astype(np.float32)
    if ties:  # coarse values force many exact ties, including +0.0 / -0.0
        l = (np.round(l * 2) / 2).astype(np.float32)
        l[:, ::7] = -0.0
        l[:, 3::11] = 0.0
    return l


@pytest.mark.parametrize("t,e,k,ties", [(50, 8, 2, False), (40, 32, 4, True), (30, 256, 8, True), (5, 5, 5, True)])
def test_topk_ids_match_bruteforce(t, e, k, ties):
    rng = np.random.default_rng(t * 1000 + e)
    l = _logits(rng, t, e, ties)
    ids, w = O.route(l, k)
    for i in range(t):
        ref_ids, _ = brute.topk_bruteforce(l[i], k)
        assert list(ids[i]) == ref_ids


def test_weights_closed_form_and_invariants():
    rng = np.random.default_rng(7)
    l = _logits(rng, 200, 64)
    k = 6
    ids, w = O.route(l, k)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)  # non-increasing with slot index
    for i in range(0, 200, 17):
        ch = [float(l[i, e]) for e in ids[i]]
        # softmax over the chosen logits, evaluated with math.fsum at float64 precision
        den = math.fsum(math.exp(c - ch[0]) for c in ch)
        for j in range(k):
            exact = math.exp(ch[j] - ch[0]) / den
            assert abs(float(w[i, j]) - exact) <= np.spacing(np.float32(exact))


def test_k1_weight_is_exactly_one():
    rng = np.random.default_rng(8)
    ids, w = O.route(_logits(rng, 100, 16), 1)
    assert np.all(w == 1.0)


def test_route_rejects_non_finite():
    l = np.zeros((2, 4), np.float32)
    l[1, 2] = np.inf
    with pytest.raises(ValueError):
        O.route(l, 2)


def _perm_bruteforce(ids, e0, el):
    t, k = ids.shape
    pairs = sorted((int(ids[i, j]) - e0, i * k + j) for i in range(t) for j in range(k)
                   if 0 <= int(ids[i, j]) - e0 < el)
    counts = [0] * el
    for le, _ in pairs:
        counts[le] += 1
    return counts, [s for _, s in pairs]


@pytest.mark.parametrize("t,e,k,e0,el", [(64, 8, 2, 0, 8), (100, 256, 8, 0, 32), (100, 256, 8, 96, 32),
                                         (17, 16, 3, 5, 1), (30, 64, 4, 60, 4)])
def test_permute_matches_bruteforce(t, e, k, e0, el):
    rng = np.random.default_rng(t + e + e0)
    ids, _ = O.route(_logits(rng, t, e), k)
    counts, offsets, r2s, s2r = O.permute(ids, e0, el)
    bc, bslots = _perm_bruteforce(ids, e0, el)
    R = len(bslots)
    assert list(counts) == bc
    assert offsets[0] == 0 and offsets[-1] == R and np.all(np.diff(offsets) == counts)
    assert list(r2s[:R]) == bslots and np.all(r2s[R:] == -1)
    # bijection between rows [0, R) and local slots
    assert np.all(s2r[r2s[:R]] == np.arange(R))
    local = np.array([0 <= int(v) - e0 < el for v in ids.reshape(-1)])
    assert np.all((s2r >= 0) == local)
    # ascending slot id within each expert
    for le in range(el):
        seg = r2s[offsets[le]:offsets[le + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(ids.reshape(-1)[seg] - e0 == le)


def test_permute_no_local_slots():
    ids = np.array([[40, 41], [42, 43]], np.int32)
    counts, offsets, r2s, s2r = O.permute(ids, 0, 32)
    assert counts.sum() == 0 and offsets[-1] == 0 and np.all(r2s == -1) and np.all(s2r == -1)
