"""GPU parity of the input quantisation (moe_quantize_act) against the oracle, bit for bit.

bf16 values are exact in fp32 and the scaling is by a power of two, so codes and scale
bytes are fully determined: the bar is equality of every byte.
"""
import numpy as np
import pytest

from moe_expert_layer_amd import synth
from oracle import moe_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from moe_expert_layer_amd import binding as B
    from tests import gpu_util as G


def _bits(v32):
    return (np.asarray(v32, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _run(bits):
    T, H = bits.shape
    d = B.make_desc(num_tokens=T, hidden=H, inter=128, num_experts=1, topk=1)
    xb = torch.from_numpy(bits.view(np.int16)).cuda()
    x = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    sf = torch.empty((T, H // 128), dtype=torch.uint8, device="cuda")
    B.moe_quantize_act(d, xb, x, sf)
    torch.cuda.synchronize()
    return x.cpu().numpy(), sf.cpu().numpy()


def _ties():
    """Blocks whose largest magnitude is 448 (scale byte 127: codes are the values rounded
    directly) filled with every midpoint between adjacent positive E4M3 values, normal and
    subnormal, with both signs: round-to-nearest-even decides each one (all are exact in bf16)."""
    grid = np.sort(np.unique(np.abs(O.decode_e4m3(np.arange(256, dtype=np.uint8)))))
    grid = grid[np.isfinite(grid)]
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([mids, -mids])
    n = -(-len(vals) // 127) * 127
    vals = np.concatenate([vals, np.zeros(n - len(vals))]).reshape(-1, 127)
    blocks = np.concatenate([np.full((len(vals), 1), 448.0), vals], 1)  # one block per row
    return blocks.astype(np.float32)


def _cases():
    rng = np.random.default_rng(40)
    n = lambda *s: rng.standard_normal(s).astype(np.float32)
    special = np.concatenate([np.zeros((1, 256)), -np.zeros((1, 256)), n(1, 256) * 1e-38, n(1, 256) * 8e37,
                              np.concatenate([np.zeros((1, 128)), n(1, 128)], 1)]).astype(np.float32)
    return [("n01_1x128", n(1, 128)), ("n01_37x384", n(37, 384)), ("n01_300x2048", n(300, 2048)),
            ("cauchy_129x7168", rng.standard_cauchy((129, 7168)).astype(np.float32)),
            ("tiny_8x1024", n(8, 1024) * 1e-30), ("large_8x1024", n(8, 1024) * 1e30), ("special", special),
            ("e4m3_ties", _ties())]


@pytest.mark.parametrize("name,v", _cases(), ids=[c[0] for c in _cases()])
def test_quantize_bit_exact(name, v):
    bits = _bits(synth._bf16_round(np.asarray(v, np.float32)))
    G.say(f"[quant] {name}: {bits.shape}")
    q, sf = _run(bits)
    rq, rsf = O.quantize_act(bits)
    assert np.array_equal(sf, rsf)
    assert np.array_equal(q, rq)


def test_quantize_zero_tokens_is_a_noop():
    d = B.make_desc(num_tokens=0, hidden=256, inter=128, num_experts=1, topk=1)
    B.moe_quantize_act(d, None, None, None)


@pytest.mark.parametrize("cfg", ["decode", "mxfp4_large"])
def test_quantize_fullsize(cfg):
    """Full-size activations: every byte against the seeded inputs (which the CPU tests pin to
    the oracle), and 16 sampled rows against the oracle directly."""
    w = synth.workload(cfg)
    inp = synth.generate(w, with_bf16=True)
    G.say(f"[quant] fullsize {cfg}: T={w.tokens} H={w.hidden}")
    q, sf = _run(inp["x_bf16"])
    assert np.array_equal(sf, inp["x_sf"]) and np.array_equal(q, inp["x"])
    rows = np.random.default_rng(41).choice(w.tokens, size=min(16, w.tokens), replace=False)
    rq, rsf = O.quantize_act(inp["x_bf16"][rows])
    assert np.array_equal(q[rows], rq) and np.array_equal(sf[rows], rsf)


@pytest.mark.parametrize("m,g", [(1, 1), (3, 4), (5, 6), (37, 3), (130, 16), (4096, 56)])
def test_pack_unpack_scales_bit_exact(m, g):
    sf = np.random.default_rng(m + 7 * g).integers(0, 255, (m, g)).astype(np.uint8)
    ref = O.pack_ue8m0(sf)
    dsf = torch.from_numpy(sf).cuda()
    packed = torch.full((ref.size,), -1, dtype=torch.int32, device="cuda")  # poisoned: padding must be written
    B.moe_pack_scales(m, g, dsf, packed)
    back = torch.full((m, g), 0xAB, dtype=torch.uint8, device="cuda")
    B.moe_unpack_scales(m, g, packed, back)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), ref.ravel())
    assert np.array_equal(back.cpu().numpy(), sf)


def test_quantize_then_pack_matches_oracle():
    w = synth.shrink(synth.workload("decode"), tokens=61)
    inp = synth.generate(w, with_bf16=True)
    q, sf = _run(inp["x_bf16"])
    g = w.hidden // 128
    packed = torch.empty(((g + 3) // 4) * ((w.tokens + 3) // 4 * 4), dtype=torch.int32, device="cuda")
    B.moe_pack_scales(w.tokens, g, torch.from_numpy(sf).cuda(), packed)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), O.pack_ue8m0(O.quantize_act(inp["x_bf16"])[1]).ravel())
