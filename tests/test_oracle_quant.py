"""Pins of the oracle's input quantisation (bf16 -> E4M3 + 1x128 UE8M0) on the CPU."""
import numpy as np
import pytest
import torch

from moe_expert_layer_amd import synth
from oracle import moe_oracle as O
from tests import brute


def _bits(v32: np.ndarray) -> np.ndarray:
    """float32 values that are exact in bf16 -> bf16 bit patterns."""
    return (np.asarray(v32, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def test_decode_bf16_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, 200000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite patterns (inf / NaN excluded)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = O.decode_bf16(bits)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("shape,scale", [((7, 128), 1.0), ((33, 384), 1.0), ((5, 1024), 1e-30), ((4, 256), 1e30)])
def test_quantize_matches_the_generators_torch_cast(shape, scale):
    # the input generator quantises with torch's E4M3 cast (independent of the oracle's encoder)
    rng = np.random.default_rng(2)
    v = synth._bf16_round((rng.standard_normal(shape) * scale).astype(np.float32))
    q_ref, sf_ref = synth._quant_fp8_blocks(v, 1, 128)
    q, sf = O.quantize_act(_bits(v))
    assert np.array_equal(q, q_ref) and np.array_equal(sf, sf_ref)


def test_quantize_matches_bruteforce_rows():
    rng = np.random.default_rng(3)
    rows = [rng.standard_normal(256), np.zeros(256), rng.standard_normal(256) * 1e-38,  # bf16 subnormals
            np.concatenate([np.zeros(128), rng.standard_normal(128) * 3e38 / 4]),      # near the bf16 maximum
            np.concatenate([-np.zeros(128), rng.standard_cauchy(128)])]
    v = synth._bf16_round(np.array(rows, dtype=np.float32))
    q, sf = O.quantize_act(_bits(v))
    for i in range(v.shape[0]):
        bc, bs = brute.requant_row(v[i])
        assert list(sf[i]) == list(bs)
        assert list(q[i]) == list(bc)


def test_generator_bf16_is_the_quantised_input():
    w = synth.shrink(synth.workload("oai"), tokens=40, hidden=512)
    inp = synth.generate(w, with_bf16=True)
    q, sf = O.quantize_act(inp["x_bf16"])
    assert np.array_equal(q, inp["x"]) and np.array_equal(sf, inp["x_sf"])


def test_pack_ue8m0_worked_example():
    # M = 5 rows, G = 6 groups: aligned M = 8, two words per row; rows 5..7 and the upper
    # half of each row's second word are padding (zero)
    sf = np.arange(30, dtype=np.uint8).reshape(5, 6) + 100
    st = O.pack_ue8m0(sf)
    assert st.shape == (2, 8) and st.dtype == np.int32
    for m in range(5):
        w0 = int(sf[m, 0]) | int(sf[m, 1]) << 8 | int(sf[m, 2]) << 16 | int(sf[m, 3]) << 24
        w1 = int(sf[m, 4]) | int(sf[m, 5]) << 8
        assert int(st[0, m].view(np.uint32)) == w0 and int(st[1, m].view(np.uint32)) == w1
    assert not st[:, 5:].any()
    # the storage viewed with the printed shape (M, ceil(G/4)) and stride (1, aligned_M)
    t = torch.as_strided(torch.from_numpy(st.ravel().copy()), (5, 2), (1, 8))
    assert int(t[3, 1]) == int(st[1, 3]) and int(t[4, 0]) == int(st[0, 4])


@pytest.mark.parametrize("m,g", [(1, 1), (3, 4), (4, 5), (7, 56), (130, 16)])
def test_pack_unpack_round_trip(m, g):
    sf = np.random.default_rng(m * 100 + g).integers(0, 255, (m, g)).astype(np.uint8)
    st = O.pack_ue8m0(sf)
    assert st.shape == ((g + 3) // 4, (m + 3) // 4 * 4)
    assert np.array_equal(O.unpack_ue8m0(st, m, g), sf)
    w = st.view(np.uint32)
    assert not w[:, m:].any()  # padding rows
    if g % 4:
        assert not (w[-1, :m] >> np.uint32(8 * (g % 4))).any()  # padding bytes
