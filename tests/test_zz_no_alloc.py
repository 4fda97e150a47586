"""moe_layer_static (the entry point that allocates nothing: its scratch is a static device
array in the library) against moe_layer with a caller-owned workspace: same routing outputs
and the same y, bit for bit, on two calls in a row, the second with a smaller layer (the
array keeps the first call's contents, which the second must not depend on)."""
import ctypes

import numpy as np
import pytest

from moe_expert_layer_amd import binding as B
from moe_expert_layer_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_util as G


def _static_call(w, dev):
    d = B.desc_from_workload(w)
    T, k, EL = w.tokens, w.topk, w.num_local
    y = torch.empty((T, w.hidden), dtype=torch.int16, device="cuda")
    ids, tw = G.i32(T, k), torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts, offsets, r2s, s2r = G.i32(EL), G.i32(EL + 1), G.i32(T * k), G.i32(T * k)
    B.moe_layer_static(d, dev["logits"], dev["x"], dev["x_sf"], dev["w1"], dev["w1_sf"], dev["w2"], dev["w2_sf"], y,
                       ids, tw, counts, offsets, r2s, s2r)
    torch.cuda.synchronize()
    return {"y_bf16": y.cpu().numpy().view(np.uint16), "topk_ids": ids.cpu().numpy(), "topk_w": tw.cpu().numpy(),
            "counts": counts.cpu().numpy(), "offsets": offsets.cpu().numpy(), "row_to_slot": r2s.cpu().numpy(),
            "slot_to_row": s2r.cpu().numpy()}


def _same(a, b):
    for key in ("y_bf16", "topk_ids", "counts", "offsets", "row_to_slot", "slot_to_row"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["topk_w"].view(np.int32), b["topk_w"].view(np.int32))


def test_static_scratch_layer_equals_workspace_layer():
    assert B.lib().moe_static_scratch_bytes() == 64 * 2 ** 20
    big = synth.workload("decode")  # about 33 MB of scratch: the largest graded share that fits
    small = synth.shrink(synth.workload("oai"), tokens=200, hidden=1024, inter=512, num_experts=16, local_begin=3,
                         num_local=10, topk=3, name="oai-small")
    for w in (big, small):  # two calls in a row, the second smaller
        G.say(f"[no-alloc] {w.name}: T={w.tokens} H={w.hidden} I={w.inter} E={w.num_experts} k={w.topk}")
        inp = synth.generate(w)
        dev = G.upload(inp)
        got = _static_call(w, dev)
        ref = G.run_layer(w, dev)
        _same(got, ref)
        again = _static_call(w, dev)  # run-to-run bit identity through the shared array
        _same(again, ref)
        G.say(f"[no-alloc] {w.name}: moe_layer_static == moe_layer bit for bit")
        del dev
    torch.cuda.empty_cache()


def test_static_scratch_rejects_a_layer_too_large():
    w = synth.workload("prefill_zipf")  # needs gigabytes of scratch
    d = B.desc_from_workload(w)
    assert B.moe_workspace_size(d) > B.lib().moe_static_scratch_bytes()
    t = torch.zeros(16, dtype=torch.uint8, device="cuda")
    y = torch.zeros(16, dtype=torch.int16, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer_static(d, t, t, t, t, t, t, t, y)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    assert "static" in str(ei.value)


def test_static_entry_replays_under_graph_capture():
    """moe_layer_static captured in a HIP graph (the case it exists for: a caller that cannot
    allocate) replays to the eager result every time, with an eager call of another layer
    shape between the replays overwriting the shared static array."""
    w = synth.shrink(synth.workload("oai"), tokens=240, hidden=512, inter=256, num_experts=16, local_begin=2,
                     num_local=12, topk=4, seed=44, name="oai-graph")
    other = synth.shrink(synth.workload("tiny"), tokens=300, hidden=768, inter=384, num_experts=8, num_local=8,
                         topk=2, seed=45, name="tiny-between")
    dev, dev_other = G.upload(synth.generate(w)), G.upload(synth.generate(other))
    eager = _static_call(w, dev)
    d = B.desc_from_workload(w)
    T, k, EL = w.tokens, w.topk, w.num_local
    y = torch.zeros((T, w.hidden), dtype=torch.int16, device="cuda")
    ids, tw = G.i32(T, k), torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts, offsets, r2s, s2r = G.i32(EL), G.i32(EL + 1), G.i32(T * k), G.i32(T * k)

    def call():
        B.moe_layer_static(d, dev["logits"], dev["x"], dev["x_sf"], dev["w1"], dev["w1_sf"], dev["w2"], dev["w2_sf"],
                           y, ids, tw, counts, offsets, r2s, s2r)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        y.zero_()
        _static_call(other, dev_other)  # eager work through the same static array
        g.replay()
        torch.cuda.synchronize()
        got = {"y_bf16": y.cpu().numpy().view(np.uint16), "topk_ids": ids.cpu().numpy(), "topk_w": tw.cpu().numpy(),
               "counts": counts.cpu().numpy(), "offsets": offsets.cpu().numpy(), "row_to_slot": r2s.cpu().numpy(),
               "slot_to_row": s2r.cpu().numpy()}
        _same(got, eager)
        G.say(f"[no-alloc] graph replay {i}: equal to the eager call bit for bit")
