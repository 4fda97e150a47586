"""The packed int32 MN-major scale layout ("DSV4 o_proj: fuse fp8/UE8M0 quantize into o_a proj",
Description: shape (rows, ceil(groups/4)), stride (1, aligned rows)) consumed in place by the
GEMMs: x_sf given packed, h_sf written packed by FC1 and read packed by FC2.

The packed x_sf is made on the host by the oracle's packer (pinned against a worked example of
the layout); the layer must give the oracle's result, and the same bits as with row-major scale
bytes; the packed h_sf, unpacked on the host, must equal the row-major run's h_sf byte for byte.
"""
import numpy as np
import pytest

from moe_expert_layer_amd import binding as B
from moe_expert_layer_amd import synth
from oracle import moe_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_util as G

TOL = 2e-3


def _cases():
    tiny, oai = synth.workload("tiny"), synth.workload("oai")
    return {
        # several tiles per expert, ragged tails (row count not a multiple of 4: padded words)
        "ragged_oai": synth.shrink(oai, tokens=601, hidden=1024, inter=384, num_experts=8, num_local=8, topk=2, seed=7),
        # groups per row not a multiple of 4 (H/128 = 5, I/128 = 3): partial last words
        "odd_groups": synth.shrink(tiny, tokens=203, hidden=640, inter=384, num_experts=16, local_begin=3,
                                   num_local=9, topk=3, seed=40),
        "mxfp4": synth.shrink(synth.workload("mxfp4_large"), tokens=250, hidden=512, inter=512, num_experts=16,
                              num_local=8, topk=4, seed=41),
        "shared": synth.shrink(oai, tokens=130, hidden=768, inter=256, num_experts=32, local_begin=4, num_local=12,
                               topk=4, num_shared=1, seed=42),
    }


def _run(w, dev, x_sf, packed, variant):
    d = B.desc_from_workload(w, variant, scale_layout="packed" if packed else "rows")
    ws = B.alloc_workspace(d)
    T, k, EL, I, S = w.tokens, w.topk, w.num_local, w.inter, w.num_shared
    rows = T * (k + S)
    ids, tw = G.i32(T, k), torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts, offsets, r2s, s2r = G.i32(EL), G.i32(EL + 1), G.i32(T * k), G.i32(T * k)
    B.moe_route_permute(d, dev["logits"], ids, tw, counts, offsets, r2s, s2r, ws)
    h = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
    if packed:
        h_sf = torch.zeros(((I // 128 + 3) // 4) * ((rows + 3) // 4 * 4), dtype=torch.int32, device="cuda")
    else:
        h_sf = torch.empty((rows, I // 128), dtype=torch.uint8, device="cuda")
    B.moe_grouped_fc1_swiglu(d, dev["x"], x_sf, dev["w1"], dev["w1_sf"], offsets, r2s, h, h_sf, ws)
    y = torch.empty((T, w.hidden), dtype=torch.int16, device="cuda")
    B.moe_grouped_fc2_combine(d, h, h_sf, dev["w2"], dev["w2_sf"], offsets, r2s, s2r, tw, y, ws)
    y1 = torch.empty_like(y)
    B.moe_layer(d, dev["logits"], dev["x"], x_sf, dev["w1"], dev["w1_sf"], dev["w2"], dev["w2_sf"], y1, ws)
    torch.cuda.synchronize()
    R = int(offsets[-1].item())
    NR = R + S * T
    hs = h_sf.cpu().numpy()
    hs = O.unpack_ue8m0(hs.reshape((I // 128 + 3) // 4, -1), rows, I // 128) if packed else hs
    return {"y": y.cpu().numpy().view(np.uint16), "y_fused": y1.cpu().numpy().view(np.uint16),
            "h": h[:NR].cpu().numpy(), "h_sf": hs[:NR]}


@pytest.mark.parametrize("variant", [-1, 0, 1, 2])
@pytest.mark.parametrize("name", sorted(_cases()))
def test_packed_scales_consumed_in_place(name, variant):
    w = _cases()[name]
    G.say(f"[packed] {name} variant={variant}: T={w.tokens} H={w.hidden} I={w.inter} k={w.topk} S={w.num_shared}")
    inp = synth.generate(w)
    ref = O.layer(w, inp)
    dev = G.upload(inp)
    x_sf_packed = torch.from_numpy(np.ascontiguousarray(O.pack_ue8m0(inp["x_sf"]))).cuda()
    rows = _run(w, dev, dev["x_sf"], False, variant)
    pk = _run(w, dev, x_sf_packed, True, variant)
    assert np.array_equal(pk["y"], rows["y"]) and np.array_equal(pk["y_fused"], rows["y"])
    assert np.array_equal(pk["h"], rows["h"]) and np.array_equal(pk["h_sf"], rows["h_sf"])
    err = G.rel_fro(G.bf16_to_f64(pk["y"]), G.bf16_to_f64(ref["y_bf16"]))
    be, se = G.h_agreement(pk["h"], pk["h_sf"], ref["h"], ref["h_sf"])
    G.say(f"[packed] {name} variant={variant}: equal to the row-major run; rel_fro={err:.3e} h_bytes_equal={be:.5f}")
    assert err <= TOL and be >= 0.99 and se >= 0.99
