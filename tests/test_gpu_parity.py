"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: routing ids, counts, offsets and both maps bit-exact; routing weights within
1 fp32 ulp (fp64 exp on two platforms); layer output bf16 within a relative Frobenius
error of 2e-3; requantised intermediate codes equal or one E4M3 step apart.
"""
import numpy as np
import pytest

from moe_expert_layer_amd import synth
from oracle import moe_oracle as O
from tests import brute

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_util as G

TOL = 2e-3


def _small_cases():
    tiny = synth.workload("tiny")
    oai = synth.workload("oai")
    return [
        ("tiny", tiny),
        ("oai_full", oai),
        # several tiles per expert, ragged row and column tails, OAI
        ("ragged_oai", synth.shrink(oai, tokens=600, hidden=1024, inter=384, num_experts=8, num_local=8, topk=2,
                                    seed=7)),
        # FC2 column tile half outside H, partial local share
        ("ragged_h384_share", synth.shrink(tiny, tokens=300, hidden=384, inter=256, num_experts=24, local_begin=5,
                                           num_local=7, topk=5, seed=8)),
        # skewed routing with empty experts
        ("zipf_small", synth.shrink(synth.workload("prefill_zipf"), tokens=256, hidden=512, inter=256,
                                    num_experts=64, num_local=16, topk=6, seed=9)),
        ("mxfp4_small", synth.shrink(synth.workload("mxfp4_large"), tokens=200, hidden=512, inter=384,
                                     num_experts=16, num_local=8, topk=4, seed=10)),
        # E5M2 weights (activations stay E4M3): MFMA weight-operand format 1
        ("e5m2_small", synth.shrink(oai, tokens=300, hidden=768, inter=384, num_experts=16, num_local=8, topk=4,
                                    weight_format="fp8e5m2", seed=15)),
        # per-tensor float32 scales; the second case saturates about 4.5% of h at 448 * h_scale
        ("tensor_oai", synth.tensor_scaled(synth.shrink(oai, tokens=600, hidden=1024, inter=384, num_experts=8,
                                                        num_local=8, topk=2, seed=16))),
        ("tensor_e5m2_sat", synth.tensor_scaled(synth.shrink(oai, tokens=200, hidden=512, inter=256, num_experts=16,
                                                             local_begin=4, num_local=8, topk=4,
                                                             weight_format="fp8e5m2", seed=17), h_scale=0.0015)),
        # shared experts after the routed ones (weight 1 for every token)
        ("shared_oai", synth.shrink(oai, tokens=300, hidden=768, inter=384, num_experts=16, local_begin=4,
                                    num_local=8, topk=4, num_shared=1, seed=18)),
        ("shared2_partial", synth.shrink(tiny, tokens=40, hidden=512, inter=256, num_experts=64, local_begin=10,
                                         num_local=8, topk=4, num_shared=2, seed=19)),
        # shared experts whose exact row count (every token) picks another tile shape than the
        # routed experts' heuristic: routed 32-row tiles with 128-row shared tiles (the decode
        # regime; MXFP4 with two shared experts), routed 32-row with 256-row shared tiles
        ("shared_tiles_v2_v0", synth.shrink(tiny, tokens=100, hidden=512, inter=256, num_experts=64, local_begin=8,
                                            num_local=16, topk=4, num_shared=1, seed=34)),
        ("shared_tiles_v2_v0_mxfp4", synth.shrink(synth.workload("mxfp4_large"), tokens=90, hidden=512, inter=384,
                                                  num_experts=64, num_local=16, topk=4, num_shared=2, seed=35)),
        ("shared_tiles_v2_v1", synth.shrink(oai, tokens=300, hidden=512, inter=256, num_experts=64, num_local=32,
                                            topk=4, num_shared=1, seed=36)),
        # the whole layer in bfloat16 (x, weights, h), with a shared expert in the second case
        ("bf16_oai", synth.shrink(oai, tokens=300, hidden=768, inter=384, num_experts=16, local_begin=2,
                                  num_local=8, topk=4, weight_format="bf16", seed=25)),
        ("bf16_shared", synth.shrink(tiny, tokens=100, hidden=512, inter=256, num_experts=32, num_local=8, topk=4,
                                     weight_format="bf16", num_shared=1, seed=26)),
        ("top1", synth.shrink(tiny, tokens=130, topk=1, seed=11)),
        ("k16_e1024", synth.shrink(tiny, tokens=40, num_experts=1024, local_begin=1000, num_local=24, topk=16,
                                   seed=12)),
        # more than 16384 slots: chunked multi-workgroup permute
        ("many_slots", synth.shrink(tiny, tokens=2100, hidden=256, inter=128, num_experts=64, num_local=16, topk=8,
                                    seed=13)),
        # more than 256 local experts: chunked permute as well
        ("many_local", synth.shrink(tiny, tokens=96, hidden=256, inter=128, num_experts=1024, local_begin=100,
                                    num_local=300, topk=8, seed=14)),
        # the largest contraction the kernels take (K = 8192: 64 scale steps staged in LDS),
        # in FC1 (hidden) and in FC2 (intermediate)
        ("max_k_fc1", synth.shrink(tiny, tokens=40, hidden=8192, inter=256, num_experts=4, num_local=4, topk=2,
                                   seed=29)),
        ("max_k_fc2", synth.shrink(tiny, tokens=40, hidden=256, inter=8192, num_experts=4, num_local=4, topk=2,
                                   seed=30)),
        # every token routed to every expert (k = E); a share of one expert
        ("k_equals_e", synth.shrink(tiny, tokens=50, num_experts=4, num_local=4, topk=4, seed=31)),
        ("one_local", synth.shrink(tiny, tokens=70, num_experts=16, local_begin=15, num_local=1, topk=3, seed=32)),
        # the most local experts (1024): the GEMM prologue's plan and offsets in LDS fill
        # their whole regions over several passes of the workgroup's threads
        ("max_local", synth.shrink(tiny, tokens=64, hidden=256, inter=128, num_experts=1024, num_local=1024,
                                   topk=4, seed=33)),
    ]


@pytest.mark.parametrize("name,w", _small_cases(), ids=[c[0] for c in _small_cases()])
def test_layer_parity_small(name, w):
    G.say(f"[parity] {name}: T={w.tokens} H={w.hidden} I={w.inter} E={w.num_experts} EL={w.num_local} k={w.topk}")
    inp = synth.generate(w)
    ref = O.layer(w, inp)
    dev = G.upload(inp)
    got = G.run_split(w, dev)
    G.check_routing(got, ref)
    be, se = G.h_agreement(got["h"], got["h_sf"], ref["h"], ref["h_sf"])
    err = G.rel_fro(G.bf16_to_f64(got["y_bf16"]), G.bf16_to_f64(ref["y_bf16"]))
    G.say(f"[parity] {name}: R={got['R']} rel_fro={err:.3e} h_bytes_equal={be:.5f} h_sf_equal={se:.5f}")
    # MFMA sums carry ~1e-5 of sum|products| absolute error, so values near an E4M3
    # midpoint may round the other way; a wrong index or scale gives far lower agreement
    assert be >= 0.99 and se >= 0.99
    assert err <= TOL
    # the fused entry point gives the same bits as the three-call path
    fused = G.run_layer(w, dev)
    assert np.array_equal(fused["y_bf16"], got["y_bf16"])
    G.check_routing(fused, ref)
    # without shared experts, tokens without a local slot are exactly +0
    nol = ~(ref["slot_to_row"].reshape(w.tokens, w.topk) >= 0).any(1)
    if w.num_shared == 0:
        assert np.all(fused["y_bf16"][nol] == 0)
    else:
        assert nol.any() or name != "shared2_partial"


@pytest.mark.parametrize("variant", [0, 1, 2])
@pytest.mark.parametrize("name", ["ragged_oai", "ragged_h384_share", "zipf_small", "mxfp4_small", "e5m2_small",
                                  "tensor_oai", "shared_oai", "bf16_oai", "k16_e1024", "max_k_fc1", "max_k_fc2",
                                  "max_local"])
def test_layer_parity_forced_variant(name, variant):
    """Each tile shape against the oracle (three-call path, whose GEMMs derive the tile plan
    themselves), and the one-call entry point (the permute's plan) bit-identical to it."""
    w = dict(_small_cases())[name]
    G.say(f"[variant] {name} variant={variant}")
    inp = synth.generate(w)
    ref = O.layer(w, inp)
    dev = G.upload(inp)
    got = G.run_split(w, dev, variant=variant)
    assert np.array_equal(G.run_layer(w, dev, variant=variant)["y_bf16"], got["y_bf16"])
    G.check_routing(got, ref)
    be, se = G.h_agreement(got["h"], got["h_sf"], ref["h"], ref["h_sf"])
    err = G.rel_fro(G.bf16_to_f64(got["y_bf16"]), G.bf16_to_f64(ref["y_bf16"]))
    G.say(f"[variant] {name} variant={variant}: rel_fro={err:.3e} h_bytes_equal={be:.5f}")
    assert be >= 0.99 and se >= 0.99 and err <= TOL


def test_run_twice_bit_identical():
    w = synth.shrink(synth.workload("oai"), tokens=300, hidden=768, inter=256, seed=20)
    inp = synth.generate(w)
    dev = G.upload(inp)
    a = G.run_layer(w, dev)
    b = G.run_layer(w, dev)
    assert np.array_equal(a["y_bf16"], b["y_bf16"])


@pytest.mark.parametrize("scaling", ["block", "tensor"])
@pytest.mark.parametrize("fmt", ["fp8", "fp8e5m2"])
@pytest.mark.parametrize("variant", [-1, 0, 1, 2])
def test_exact_integer_layer_bit_exact(variant, fmt, scaling):
    """Small-integer operands, unit scales, top-1, OAI with alpha 0: every partial sum is exact in
    fp32 (x, W2 in {-1, 0, 1}; W1 rows with at most 4 non-zeros so |g|, |u| <= 4 and h = g*u/2 is a
    half-integer <= 8 that the requant reproduces exactly), so the GPU output equals the oracle bit for bit.
    With per-tensor scaling every scale is 1.0 (h_scale too)."""
    rng = np.random.default_rng(9)
    T, H, I, E = 200, 256, 256, 4
    w = synth.shrink(synth.workload("tiny"), tokens=T, hidden=H, inter=I, num_experts=E, num_local=E, topk=1,
                     activation="swigluoai", act_clamp=np.inf, act_alpha=0.0, act_up_bias=0.0, weight_format=fmt)
    ONE, MONE = 0x38, 0xB8  # E4M3 codes of +1 and -1
    WONE, WMONE = (0x38, 0xB8) if fmt == "fp8" else (0x3C, 0xBC)  # the weights' codes of +1 and -1

    def pm1(shape, p_zero, one=ONE, mone=MONE):
        v = rng.choice([mone, 0, one], size=shape, p=[(1 - p_zero) / 2, p_zero, (1 - p_zero) / 2])
        return v.astype(np.uint8)

    w1 = np.zeros((E, 2 * I, H), np.uint8)
    for e in range(E):
        for n in range(2 * I):
            cols = rng.choice(H, size=4, replace=False)
            w1[e, n, cols] = rng.choice([WMONE, WONE], size=4)
    inp = {"logits": rng.standard_normal((T, E)).astype(np.float32), "x": pm1((T, H), 0.3),
           "x_sf": np.full((T, H // 128), 127, np.uint8), "w1": w1,
           "w1_sf": np.full((E, 2 * I // 128, H // 128), 127, np.uint8), "w2": pm1((E, H, I), 0.3, WONE, WMONE),
           "w2_sf": np.full((E, H // 128, I // 128), 127, np.uint8)}
    if scaling == "tensor":
        w = synth.tensor_scaled(w, h_scale=1.0)
        inp.update(x_sf=np.ones(1, np.float32), w1_sf=np.ones(E, np.float32), w2_sf=np.ones(E, np.float32))
    ref = O.layer(w, inp)
    got = G.run_split(w, G.upload(inp), variant=variant)
    assert np.array_equal(got["h"], ref["h"]) and np.array_equal(got["h_sf"], ref["h_sf"])
    assert np.array_equal(got["y_bf16"], ref["y_bf16"])


def test_w2_scale_plus_one_doubles_output():
    w = synth.shrink(synth.workload("oai"), tokens=200, hidden=512, inter=256, seed=22)
    inp = synth.generate(w)
    a = G.run_layer(w, G.upload(inp))
    inp2 = dict(inp)
    inp2["w2_sf"] = (inp["w2_sf"].astype(np.int32) + 1).astype(np.uint8)
    b = G.run_layer(w, G.upload(inp2))
    ya, yb = G.bf16_to_f64(a["y_bf16"]), G.bf16_to_f64(b["y_bf16"])
    assert np.array_equal(yb, 2 * ya)


def test_token_permutation_equivariance():
    w = synth.shrink(synth.workload("oai"), tokens=256, hidden=512, inter=256, seed=23)
    inp = synth.generate(w)
    a = G.run_layer(w, G.upload(inp))
    perm = np.random.default_rng(1).permutation(w.tokens)
    inp2 = dict(inp)
    for key in ("logits", "x", "x_sf"):
        inp2[key] = np.ascontiguousarray(inp[key][perm])
    b = G.run_layer(w, G.upload(inp2))
    assert np.array_equal(b["y_bf16"], a["y_bf16"][perm])


def test_zero_tokens_noop():
    w = synth.shrink(synth.workload("tiny"), tokens=0)
    from moe_expert_layer_amd import binding as B
    d = B.desc_from_workload(w)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    y = torch.empty((0, w.hidden), dtype=torch.int16, device="cuda")
    e = torch.empty(0, dtype=torch.uint8, device="cuda")
    B.moe_layer(d, e, e, e, e, e, e, e, y, ws)
    torch.cuda.synchronize()


def test_no_local_rows_gives_zero_output():
    """Routing that never picks a local expert: no rows, both GEMMs have no tiles, and y is
    exactly zero (the oracle agrees bit for bit)."""
    w = synth.shrink(synth.workload("tiny"), tokens=90, num_experts=16, local_begin=4, num_local=6, topk=3,
                     seed=33)
    inp = synth.generate(w)
    logits = inp["logits"].copy()
    logits[:, w.local_begin:w.local_begin + w.num_local] = -1e30  # finite, below every other logit
    inp["logits"] = logits
    ref = O.layer(w, inp)
    assert not (ref["slot_to_row"] >= 0).any()
    dev = G.upload(inp)
    for got in (G.run_split(w, dev), G.run_layer(w, dev)):
        G.check_routing(got, ref)
        assert got.get("R", 0) == 0
        assert np.all(got["y_bf16"] == 0) and np.array_equal(got["y_bf16"], ref["y_bf16"])


def _graph_cases():
    oai = synth.shrink(synth.workload("oai"), tokens=256, hidden=512, inter=256, seed=24)
    return [("fp8", oai),
            ("tensor_shared", synth.tensor_scaled(synth.shrink(oai, num_shared=1, seed=27))),
            ("bf16", synth.shrink(oai, weight_format="bf16", seed=28))]


@pytest.mark.parametrize("name,w", _graph_cases(), ids=[c[0] for c in _graph_cases()])
def test_graph_capture_replay(name, w):
    """moe_layer captured in a HIP graph replays to the eager result every time."""
    inp = synth.generate(w)
    dev = G.upload(inp)
    eager = G.run_layer(w, dev)
    from moe_expert_layer_amd import binding as B
    d = B.desc_from_workload(w)
    ws = B.alloc_workspace(d)
    y = torch.zeros((w.tokens, w.hidden), dtype=torch.int16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.moe_layer(d, dev["logits"], dev["x"], dev["x_sf"], dev["w1"], dev["w1_sf"], dev["w2"], dev["w2_sf"], y, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.moe_layer(d, dev["logits"], dev["x"], dev["x_sf"], dev["w1"], dev["w1_sf"], dev["w2"], dev["w2_sf"], y, ws)
    for i in range(3):
        y.zero_()
        ws.fill_(0xAB)  # poison the workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint16), eager["y_bf16"]), f"replay {i}"


@pytest.mark.parametrize("name,w", [
    ("oai", synth.shrink(synth.workload("oai"), tokens=256, hidden=512, inter=256, seed=36)),
    # 16800 slots: the chunked permute (histogram, chunk scan, scatter) inside the graph
    ("chunked", synth.shrink(synth.workload("tiny"), tokens=2100, hidden=256, inter=128, num_experts=64,
                             num_local=16, topk=8, seed=37))], ids=["oai", "chunked"])
def test_graph_capture_replay_split_calls(name, w):
    """The three split calls (route/permute, FC1, FC2 + combine) captured in one HIP graph
    replay to the eager result every time, with the workspace poisoned between replays."""
    from moe_expert_layer_amd import binding as B
    dev = G.upload(synth.generate(w))
    eager = G.run_split(w, dev)
    d = B.desc_from_workload(w)
    ws = B.alloc_workspace(d)
    T, k, EL, I = w.tokens, w.topk, w.num_local, w.inter
    ids, tw = G.i32(T, k), torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts, offsets, r2s, s2r = G.i32(EL), G.i32(EL + 1), G.i32(T * k), G.i32(T * k)
    h = torch.empty((T * k, I), dtype=torch.uint8, device="cuda")
    h_sf = torch.empty((T * k, I // 128), dtype=torch.uint8, device="cuda")
    y = torch.zeros((T, w.hidden), dtype=torch.int16, device="cuda")

    def calls():
        B.moe_route_permute(d, dev["logits"], ids, tw, counts, offsets, r2s, s2r, ws)
        B.moe_grouped_fc1_swiglu(d, dev["x"], dev["x_sf"], dev["w1"], dev["w1_sf"], offsets, r2s, h, h_sf, ws)
        B.moe_grouped_fc2_combine(d, h, h_sf, dev["w2"], dev["w2_sf"], offsets, r2s, s2r, tw, y, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for i in range(3):
        y.zero_()
        ws.fill_(0xAB)  # poison the workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint16), eager["y_bf16"]), f"{name} replay {i}"
        assert np.array_equal(offsets.cpu().numpy(), eager["offsets"]), f"{name} replay {i}"


def test_zero_shared_expert_leaves_routed_output_bit_exact():
    """A shared expert whose W2 is all zero adds exactly +0 to every token: the output equals
    the layer without shared experts bit for bit (and the routed rows are unaffected)."""
    w = synth.shrink(synth.workload("oai"), tokens=200, hidden=512, inter=256, num_experts=16, num_local=8,
                     topk=4, num_shared=1, seed=29)
    inp = synth.generate(w)
    inp["w2"][w.num_local:] = 0
    with_shared = G.run_layer(w, G.upload(inp))
    w0 = synth.shrink(w, num_shared=0)
    inp0 = {k: (v[:w.num_local] if k in ("w1", "w1_sf", "w2", "w2_sf") else v) for k, v in inp.items()}
    without = G.run_layer(w0, G.upload(inp0))
    assert np.array_equal(with_shared["y_bf16"], without["y_bf16"])


def test_concurrent_streams_with_distinct_workspaces():
    """Layers on two streams at once, each with its own workspace (the header allows this):
    every result equals the same layer run alone, bit for bit."""
    from moe_expert_layer_amd import binding as B
    cases = [synth.shrink(synth.workload("oai"), tokens=400, hidden=1024, inter=512, num_experts=16, num_local=8,
                          topk=4, seed=34),
             synth.shrink(synth.workload("tiny"), tokens=300, hidden=768, inter=256, num_experts=24, local_begin=3,
                          num_local=9, topk=5, seed=35, weight_format="mxfp4")]
    runs = []
    for w in cases:
        dev = G.upload(synth.generate(w))
        alone = G.run_layer(w, dev)["y_bf16"]
        d = B.desc_from_workload(w)
        ws = B.alloc_workspace(d)
        ys = [torch.empty((w.tokens, w.hidden), dtype=torch.int16, device="cuda") for _ in range(3)]
        runs.append((w, dev, d, ws, ys, alone))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    torch.cuda.synchronize()
    for it in range(3):  # three layer calls per stream, interleaved at issue
        for (w, dev, d, ws, ys, _), st in zip(runs, streams):
            with torch.cuda.stream(st):
                B.moe_layer(d, dev["logits"], dev["x"], dev["x_sf"], dev["w1"], dev["w1_sf"], dev["w2"],
                            dev["w2_sf"], ys[it], ws, stream=st)
    torch.cuda.synchronize()
    for w, dev, d, ws, ys, alone in runs:
        for y in ys:
            assert np.array_equal(y.cpu().numpy().view(np.uint16), alone)
