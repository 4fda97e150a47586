"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before touching a GPU (no compute calls here)."""
import ctypes
import math
import os
import re

import pytest

from moe_expert_layer_amd import binding as B
from moe_expert_layer_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return B.lib()


# header -> the library that exports its functions
HEADERS = {"moe_expert_layer.h": "libmoe_expert_layer.so", "moe_probes.h": "libmoe_probes.so"}


def declared_functions(header):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\s*\(", src, flags=re.M)))


def test_every_header_has_a_library():
    assert sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")) == sorted(HEADERS)


@pytest.mark.parametrize("header", sorted(HEADERS))
def test_exports_every_declared_symbol(L, header):
    names = declared_functions(header)
    assert len(names) >= (9 if header == "moe_expert_layer.h" else 3)
    lib = ctypes.CDLL(os.path.join(ROOT, "moe_expert_layer_amd", HEADERS[header]))
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(L):
    assert L.moe_abi_version() == 3
    assert B.status_str(0) == "MOE_OK" and B.status_str(5) == "MOE_ERR_WORKSPACE"
    assert B.status_str(99) == "MOE_STATUS_UNKNOWN"


def test_defaults_follow_standard_swiglu(L):
    d = B.MoeLayerDesc()
    assert L.moe_desc_defaults(ctypes.byref(d)) == 0
    assert d.activation == B.MOE_ACT_SWIGLU and d.weight_format == B.MOE_W_FP8_E4M3_B128
    assert math.isinf(d.act_clamp) and d.act_alpha == 1.0 and d.act_up_bias == 0.0 and d.variant == -1
    assert d.scale_mode == B.MOE_SCALE_BLOCK and d.h_scale == 1.0 and d.scale_layout == B.MOE_SF_ROW_MAJOR


@pytest.mark.parametrize("i", range(5))
def test_workspace_size_covers_capacity(L, i):
    w = synth.workload(i)
    n = B.moe_workspace_size(B.desc_from_workload(w))
    cap = w.tokens * w.topk
    assert n >= cap * (w.hidden * 4 + w.inter + w.inter // 128 + 16)
    assert n % 256 == 0


@pytest.mark.parametrize("field,value", [("hidden", 100), ("inter", 0), ("num_experts", 0), ("num_experts", 2000),
                                         ("topk", 0), ("topk", 17), ("num_local", 0), ("local_begin", -1),
                                         ("num_tokens", -5), ("weight_format", 7), ("activation", 3),
                                         ("variant", 5), ("scale_mode", 2), ("num_shared", 5),
                                         ("num_shared", -1)])
def test_invalid_descriptor_rejected(L, field, value):
    d = B.desc_from_workload(synth.workload("tiny"))
    setattr(d, field, value)
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_ERR_INVALID_DESC
    assert L.moe_last_error()


def test_local_range_must_fit(L):
    d = B.desc_from_workload(synth.workload("decode"))
    d.local_begin = 240  # 240 + 32 > 256
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_ERR_INVALID_DESC


def test_oai_parameters_validated(L):
    d = B.desc_from_workload(synth.workload("oai"))
    n = ctypes.c_size_t(0)
    d.act_clamp = 0.0
    assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_ERR_INVALID_DESC
    d.act_clamp, d.act_alpha = 7.0, float("nan")
    assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_ERR_INVALID_DESC


def test_null_and_misaligned_pointers_rejected_before_launch(L):
    d = B.desc_from_workload(synth.workload("tiny"))
    P = ctypes.c_void_p
    # NULL inputs
    st = L.moe_layer(ctypes.byref(d), *([None] * 15), 0, None)
    assert st == B.MOE_ERR_NULL
    # misaligned inputs (never dereferenced: validation fails first)
    bad = [P(0x1001)] * 8 + [None] * 6
    st = L.moe_layer(ctypes.byref(d), *bad, P(0x100000), 1 << 30, None)
    assert st == B.MOE_ERR_MISALIGNED
    # small workspace
    good = [P(0x10000)] * 8 + [None] * 6
    st = L.moe_layer(ctypes.byref(d), *good, P(0x100000), 16, None)
    assert st == B.MOE_ERR_WORKSPACE
    st = L.moe_layer(ctypes.byref(d), *good, P(0x100010), 1 << 30, None)
    assert st == B.MOE_ERR_MISALIGNED  # workspace must be 256-byte aligned


def test_zero_tokens_is_a_noop_without_device(L):
    d = B.desc_from_workload(synth.shrink(synth.workload("tiny"), tokens=0))
    assert L.moe_layer(ctypes.byref(d), *([None] * 15), 0, None) == B.MOE_OK
    assert L.moe_route_permute(ctypes.byref(d), *([None] * 7), None, 0, None) == B.MOE_OK


def test_oversized_activation_matrix_unsupported(L):
    # the FC1 loads address x with 32-bit offsets: T * H must stay below 2^32 bytes
    d = B.desc_from_workload(synth.workload("decode"))
    n = ctypes.c_size_t(0)
    d.num_tokens = (1 << 32) // d.hidden + 1
    d.topk = 1
    assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_ERR_UNSUPPORTED
    d.num_tokens = (1 << 32) // d.hidden - 1
    assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_OK


def test_quantize_act_validation(L):
    d = B.desc_from_workload(synth.workload("tiny"))
    P = ctypes.c_void_p
    assert L.moe_quantize_act(ctypes.byref(d), None, None, None, None) == B.MOE_ERR_NULL
    assert L.moe_quantize_act(ctypes.byref(d), P(0x1008), P(0x2000), P(0x3000), None) == B.MOE_ERR_MISALIGNED
    d.hidden = 100
    assert L.moe_quantize_act(ctypes.byref(d), P(0x1000), P(0x2000), P(0x3000), None) == B.MOE_ERR_INVALID_DESC


def test_pack_scales_validation(L):
    P = ctypes.c_void_p
    assert L.moe_pack_scales(-1, 4, P(0x1000), P(0x2000), None) == B.MOE_ERR_INVALID_DESC
    assert L.moe_pack_scales(4, 0, P(0x1000), P(0x2000), None) == B.MOE_ERR_INVALID_DESC
    assert L.moe_pack_scales(4, 4, None, P(0x2000), None) == B.MOE_ERR_NULL
    assert L.moe_unpack_scales(4, 4, P(0x2002), P(0x1000), None) == B.MOE_ERR_MISALIGNED
    assert L.moe_pack_scales(0, 4, None, None, None) == B.MOE_OK


def test_per_tensor_scaling_validated(L):
    n = ctypes.c_size_t(0)
    d = B.desc_from_workload(synth.tensor_scaled(synth.workload("tiny")))
    assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_OK
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        d.h_scale = bad
        assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_ERR_INVALID_DESC
    d.h_scale = 0.5
    d.weight_format = B.MOE_W_MXFP4_E2M1_B32
    assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_ERR_INVALID_DESC
    d.weight_format = B.MOE_W_FP8_E5M2_B128
    assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_OK
    # the input quantiser makes blockwise scales only
    P = ctypes.c_void_p
    assert L.moe_quantize_act(ctypes.byref(d), P(0x1000), P(0x2000), P(0x3000), None) == B.MOE_ERR_UNSUPPORTED


def test_h_sf_optional_only_with_per_tensor_scaling(L):
    P = ctypes.c_void_p
    args = [P(0x10000)] * 6 + [P(0x20000), None]  # x, x_sf, w1, w1_sf, offsets, row_to_slot, h, h_sf
    d = B.desc_from_workload(synth.workload("tiny"))
    assert L.moe_grouped_fc1_swiglu(ctypes.byref(d), *args, P(0x100000), 16, None) == B.MOE_ERR_NULL
    d = B.desc_from_workload(synth.tensor_scaled(synth.workload("tiny")))
    # past the pointer checks: the undersized workspace is what is reported
    assert L.moe_grouped_fc1_swiglu(ctypes.byref(d), *args, P(0x100000), 16, None) == B.MOE_ERR_WORKSPACE


def test_probe_arguments_rejected_before_launch():
    """The probe entry points check their arguments on the host (-1) before any launch."""
    lib = ctypes.CDLL(os.path.join(ROOT, "moe_expert_layer_amd", "libmoe_probes.so"))
    P = ctypes.c_void_p
    lib.moe_probe_mfma_gemm.argtypes = [ctypes.c_int] * 4 + [P] * 4
    lib.moe_probe_mfma_loop.argtypes = [ctypes.c_int] * 3 + [P] * 2
    lib.moe_probe_hbm_read.argtypes = [P, ctypes.c_size_t, ctypes.c_int, P, P]
    fake = P(256)  # never dereferenced: every call below fails its argument check
    assert lib.moe_probe_mfma_gemm(6, 1, 128, 0, fake, fake, fake, None) == -1   # unknown form
    assert lib.moe_probe_mfma_gemm(0, 0, 128, 0, fake, fake, fake, None) == -1   # no problems
    assert lib.moe_probe_mfma_gemm(0, 1, 96, 0, fake, fake, fake, None) == -1    # K not a multiple of 128
    assert lib.moe_probe_mfma_gemm(2, 1, 128, 1, fake, fake, fake, None) == -1   # FP4 with the FP8-only form
    assert lib.moe_probe_mfma_gemm(0, 1, 128, 0, None, fake, fake, None) == -1   # NULL operand
    assert lib.moe_probe_mfma_loop(0, 10, 0, fake, None) == -1
    assert lib.moe_probe_hbm_read(fake, 17, 1, fake, None) == -1                 # not whole 16-byte loads
    lib.moe_probe_dma_stream.argtypes = [P, ctypes.c_size_t] + [ctypes.c_int] * 5 + [P, P]
    one = 512 * 1024  # one panel of 512 rows of K = 1024 bytes
    assert lib.moe_probe_dma_stream(fake, one, 1000, 1, 0, 1, 1, fake, None) == -1   # K not a multiple of 128
    assert lib.moe_probe_dma_stream(fake, one, 1024, 2, 0, 1, 1, fake, None) == -1   # two panels, one in src
    assert lib.moe_probe_dma_stream(fake, one, 1024, 2, 3, 1, 1, fake, None) == -1   # more panels than workgroups
    assert lib.moe_probe_dma_stream(fake, one, 1024, 1, 0, 1, 3, fake, None) == -1   # depth 3
    assert lib.moe_probe_dma_stream(fake, one, 1024, 1, 0, 0, 1, fake, None) == -1   # no pass
    assert lib.moe_probe_dma_stream(fake, one, 1024, 1, 0, 1, 1, None, None) == -1   # no sink


def test_static_scratch_entry_rejects_large_layers_before_launch(L):
    """moe_layer_static refuses a layer whose scratch exceeds the static array, on the host,
    before any device call (fake, never dereferenced pointers)."""
    d = B.desc_from_workload(synth.workload("prefill_zipf"))
    assert B.moe_workspace_size(d) > L.moe_static_scratch_bytes() == 64 * 2 ** 20
    fake = ctypes.c_void_p(4096)
    st = L.moe_layer_static(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, fake, None, None, None, None,
                            None, None, None)
    assert st == B.MOE_ERR_WORKSPACE
    assert b"static" in L.moe_last_error()
