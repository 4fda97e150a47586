"""Full-size workloads on the GPU (the bench's launch configuration: fused moe_layer,
heuristic kernel variant): routing and grouping bit-exact over every token, layer output
checked against the oracle on a seeded sample of tokens evaluated one by one."""
import numpy as np
import pytest

from moe_expert_layer_amd import synth
from oracle import moe_oracle as O

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if torch.cuda.is_available():
    from tests import gpu_util as G

TOL = 2e-3


def _sample_tokens(ref, w, n=12, seed=0):
    """Seeded sample: tokens with the most local slots, one with none, the rest random."""
    loc = (ref["slot_to_row"].reshape(w.tokens, w.topk) >= 0).sum(1)
    rng = np.random.default_rng(seed)
    pick = set(np.argsort(-loc, kind="stable")[:3].tolist())
    none = np.nonzero(loc == 0)[0]
    if none.size:
        pick.add(int(none[0]))
    pick.add(w.tokens - 1)
    while len(pick) < n:
        pick.add(int(rng.integers(0, w.tokens)))
    return np.array(sorted(pick))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "prefill_zipf", "mxfp4_large"])
def test_fullsize_sampled_parity(name):
    w = synth.workload(name)
    G.say(f"[fullsize] {name}: generating inputs")
    inp = synth.generate(w)
    ids, tw = O.route(inp["logits"], w.topk)
    counts, offsets, r2s, s2r = O.permute(ids, w.local_begin, w.num_local)
    ref_route = {"topk_ids": ids, "topk_w": tw, "counts": counts, "offsets": offsets, "row_to_slot": r2s,
                 "slot_to_row": s2r}
    G.say(f"[fullsize] {name}: R={int(offsets[-1])} rows, running moe_layer on the GPU")
    dev = G.upload(inp)
    got = G.run_layer(w, dev)
    G.check_routing(got, ref_route)
    toks = _sample_tokens(ref_route, w)
    G.say(f"[fullsize] {name}: oracle on {toks.size} sampled tokens")
    ref = O.layer_tokens(w, inp, toks)
    yg = G.bf16_to_f64(got["y_bf16"][toks])
    yr = G.bf16_to_f64(ref["y_bf16"])
    err = G.rel_fro(yg, yr)
    per_tok = [G.rel_fro(yg[i], yr[i]) for i in range(toks.size) if np.any(yr[i] != 0)]
    G.say(f"[fullsize] {name}: sampled rel_fro={err:.3e} worst token {max(per_tok):.3e}")
    assert err <= TOL
    assert max(per_tok) <= 2 * TOL
    nol = (ref_route["slot_to_row"].reshape(w.tokens, w.topk) >= 0).sum(1) == 0
    assert np.all(got["y_bf16"][nol] == 0)
    del dev
    torch.cuda.empty_cache()
