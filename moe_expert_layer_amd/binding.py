"""Thin ctypes binding over the C ABI in include/moe_expert_layer.h.

Argument marshalling only: every step of the layer runs in the HIP library.  Tensors
are torch device tensors (torch provides device memory and the current HIP stream);
the functions carry the C names.  If the shared library is missing or fails to load,
every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_expert_layer.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_INVALID_DESC, MOE_ERR_MISALIGNED, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, \
    MOE_ERR_DEVICE = range(7)
MOE_ACT_SWIGLU, MOE_ACT_SWIGLU_OAI = 0, 1
MOE_W_FP8_E4M3_B128, MOE_W_MXFP4_E2M1_B32, MOE_W_FP8_E5M2_B128, MOE_W_BF16 = 0, 1, 2, 3
ACTIVATIONS = {"swiglu": MOE_ACT_SWIGLU, "swigluoai": MOE_ACT_SWIGLU_OAI}
MOE_SCALE_BLOCK, MOE_SCALE_TENSOR = 0, 1
MOE_SF_ROW_MAJOR, MOE_SF_PACKED_MN = 0, 1
SCALE_LAYOUTS = {"rows": MOE_SF_ROW_MAJOR, "packed": MOE_SF_PACKED_MN}
SCALINGS = {"block": MOE_SCALE_BLOCK, "tensor": MOE_SCALE_TENSOR}
WEIGHT_FORMATS = {"fp8": MOE_W_FP8_E4M3_B128, "mxfp4": MOE_W_MXFP4_E2M1_B32, "fp8e5m2": MOE_W_FP8_E5M2_B128, "bf16": MOE_W_BF16}


class MoeLayerDesc(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
        ("num_experts", ctypes.c_int32), ("local_begin", ctypes.c_int32), ("num_local", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("weight_format", ctypes.c_int32), ("activation", ctypes.c_int32),
        ("act_clamp", ctypes.c_float), ("act_alpha", ctypes.c_float), ("act_up_bias", ctypes.c_float),
        ("variant", ctypes.c_int32), ("scale_mode", ctypes.c_int32), ("h_scale", ctypes.c_float),
        ("num_shared", ctypes.c_int32), ("scale_layout", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_str(status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded C library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, S, I32, VP = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p
        D = ctypes.POINTER(MoeLayerDesc)
        L.moe_abi_version.restype = ctypes.c_int
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [I32]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_desc_defaults.restype = I32
        L.moe_desc_defaults.argtypes = [D]
        L.moe_workspace_size.restype = I32
        L.moe_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_route_permute.restype = I32
        L.moe_route_permute.argtypes = [D, P, P, P, P, P, P, P, P, S, VP]
        L.moe_grouped_fc1_swiglu.restype = I32
        L.moe_grouped_fc1_swiglu.argtypes = [D, P, P, P, P, P, P, P, P, P, S, VP]
        L.moe_grouped_fc2_combine.restype = I32
        L.moe_grouped_fc2_combine.argtypes = [D, P, P, P, P, P, P, P, P, P, P, S, VP]
        L.moe_layer.restype = I32
        L.moe_layer.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, S, VP]
        L.moe_static_scratch_bytes.restype = ctypes.c_size_t
        L.moe_static_scratch_bytes.argtypes = []
        L.moe_layer_static.restype = I32
        L.moe_layer_static.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, VP]
        L.moe_quantize_act.restype = I32
        L.moe_quantize_act.argtypes = [D, P, P, P, VP]
        L.moe_pack_scales.restype = I32
        L.moe_pack_scales.argtypes = [I32, I32, P, P, VP]
        L.moe_unpack_scales.restype = I32
        L.moe_unpack_scales.argtypes = [I32, I32, P, P, VP]
        _lib = L
    return _lib


def status_str(st: int) -> str:
    return lib().moe_status_str(st).decode()


def _check(st: int):
    if st != MOE_OK:
        raise MoeError(st, lib().moe_last_error().decode())


def make_desc(num_tokens: int, hidden: int, inter: int, num_experts: int, topk: int, local_begin: int = 0,
              num_local: Optional[int] = None, weight_format: str = "fp8", activation: str = "swiglu",
              activation_clamp: Optional[float] = None, activation_alpha: float = 1.0,
              activation_up_bias: float = 0.0, variant: int = -1, scaling: str = "block",
              h_scale: float = 1.0, num_shared: int = 0, scale_layout: str = "rows") -> MoeLayerDesc:
    """Descriptor with the pages' keyword names (activation, activation_clamp/alpha/up_bias).

    weight_format: "fp8" (E4M3), "fp8e5m2", "mxfp4" or "bf16" (the whole layer in BF16);
    scaling: "block" (UE8M0 scale tensors) or "tensor" (float32 scales, static h_scale);
    num_shared: shared experts after the local ones in the weight tensors;
    scale_layout: "rows" (UE8M0 bytes [rows, groups]) or "packed" (int32 MN-major words) for x_sf / h_sf."""
    d = MoeLayerDesc()
    _check(lib().moe_desc_defaults(ctypes.byref(d)))
    d.num_tokens, d.hidden, d.inter = num_tokens, hidden, inter
    d.num_experts, d.topk = num_experts, topk
    d.local_begin = local_begin
    d.num_local = num_experts if num_local is None else num_local
    d.weight_format = WEIGHT_FORMATS[weight_format]
    d.activation = ACTIVATIONS[activation]
    d.act_clamp = math.inf if activation_clamp is None else activation_clamp
    d.act_alpha, d.act_up_bias = activation_alpha, activation_up_bias
    d.variant = variant
    d.scale_mode = SCALINGS[scaling]
    d.h_scale = h_scale
    d.num_shared = num_shared
    d.scale_layout = SCALE_LAYOUTS[scale_layout]
    return d


def desc_from_workload(w, variant: int = -1, scale_layout: str = "rows") -> MoeLayerDesc:
    return make_desc(w.tokens, w.hidden, w.inter, w.num_experts, w.topk, w.local_begin, w.num_local,
                     w.weight_format, w.activation, w.act_clamp, w.act_alpha, w.act_up_bias, variant,
                     getattr(w, "scaling", "block"), getattr(w, "h_scale", 1.0), getattr(w, "num_shared", 0),
                     scale_layout)


def moe_workspace_size(desc: MoeLayerDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def moe_route_permute(desc, logits, topk_ids, topk_w, counts, offsets, row_to_slot, slot_to_row, workspace,
                      stream=None):
    _check(lib().moe_route_permute(ctypes.byref(desc), _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(counts),
                                   _ptr(offsets), _ptr(row_to_slot), _ptr(slot_to_row), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_grouped_fc1_swiglu(desc, x, x_sf, w1, w1_sf, offsets, row_to_slot, h, h_sf, workspace, stream=None):
    _check(lib().moe_grouped_fc1_swiglu(ctypes.byref(desc), _ptr(x), _ptr(x_sf), _ptr(w1), _ptr(w1_sf),
                                        _ptr(offsets), _ptr(row_to_slot), _ptr(h), _ptr(h_sf), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_grouped_fc2_combine(desc, h, h_sf, w2, w2_sf, offsets, row_to_slot, slot_to_row, topk_w, y, workspace,
                            stream=None):
    _check(lib().moe_grouped_fc2_combine(ctypes.byref(desc), _ptr(h), _ptr(h_sf), _ptr(w2), _ptr(w2_sf),
                                         _ptr(offsets), _ptr(row_to_slot), _ptr(slot_to_row), _ptr(topk_w), _ptr(y),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(stream)))


def moe_layer(desc, logits, x, x_sf, w1, w1_sf, w2, w2_sf, y, workspace, topk_ids=None, topk_w=None, counts=None,
              offsets=None, row_to_slot=None, slot_to_row=None, stream=None):
    _check(lib().moe_layer(ctypes.byref(desc), _ptr(logits), _ptr(x), _ptr(x_sf), _ptr(w1), _ptr(w1_sf), _ptr(w2),
                           _ptr(w2_sf), _ptr(y), _ptr(topk_ids), _ptr(topk_w), _ptr(counts), _ptr(offsets),
                           _ptr(row_to_slot), _ptr(slot_to_row), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_layer_static(desc, logits, x, x_sf, w1, w1_sf, w2, w2_sf, y, topk_ids=None, topk_w=None, counts=None,
                     offsets=None, row_to_slot=None, slot_to_row=None, stream=None):
    """moe_layer with the library's static scratch array instead of a workspace (allocates nothing)."""
    _check(lib().moe_layer_static(ctypes.byref(desc), _ptr(logits), _ptr(x), _ptr(x_sf), _ptr(w1), _ptr(w1_sf),
                                  _ptr(w2), _ptr(w2_sf), _ptr(y), _ptr(topk_ids), _ptr(topk_w), _ptr(counts),
                                  _ptr(offsets), _ptr(row_to_slot), _ptr(slot_to_row), _stream(stream)))


def moe_quantize_act(desc, x_bf16, x, x_sf, stream=None):
    """bf16 activations [T, H] (int16/uint16/bfloat16 tensor) -> E4M3 codes x [T, H] and UE8M0 x_sf [T, H/128]."""
    _check(lib().moe_quantize_act(ctypes.byref(desc), _ptr(x_bf16), _ptr(x), _ptr(x_sf), _stream(stream)))


def moe_pack_scales(rows, groups, sf, packed, stream=None):
    """UE8M0 bytes [rows, groups] -> packed int32 words [ceil(groups/4) * pad_up(rows, 4)] (MN-major)."""
    _check(lib().moe_pack_scales(rows, groups, _ptr(sf), _ptr(packed), _stream(stream)))


def moe_unpack_scales(rows, groups, packed, sf, stream=None):
    """Inverse of moe_pack_scales."""
    _check(lib().moe_unpack_scales(rows, groups, _ptr(packed), _ptr(sf), _stream(stream)))


def alloc_workspace(desc, device="cuda"):
    """A uint8 device tensor of moe_workspace_size(desc) bytes (torch allocations are 256-byte aligned)."""
    import torch
    return torch.empty(max(moe_workspace_size(desc), 256), dtype=torch.uint8, device=device)
