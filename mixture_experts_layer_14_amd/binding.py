"""Thin Python binding of libmoe_mi355x.so (the C ABI in include/moe.h).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the library function of the same name; every step
of the layer runs in the library's HIP kernels.  PyTorch provides device
memory and streams.  There is no fallback: if the library is missing, or no
GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
SOFTMAX, SIGMOID = 0, 1
F32, BF16, FP8_E4M3 = 0, 1, 2
LAYOUT_ROW_MAJOR, LAYOUT_PACKED = 0, 1

# every entry point that include/moe.h declares
ENTRY_POINTS = (
    "moe_workspace_size", "moe_status_string", "moe_pack_weights", "moe_topk",
    "moe_align_permute", "moe_quant_act_fp8", "moe_grouped_gemm_w13_act",
    "moe_grouped_gemm_w2_combine", "moe_forward", "moe_router_gemm",
    "moe_peak_mfma_bf16", "moe_peak_read", "moe_forward_noalloc", "moe_router_topk",
)


class MoeParams(ctypes.Structure):
    """Mirror of `moe_params` in include/moe.h."""
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("hidden_size", ctypes.c_int32),
        ("intermediate_size", ctypes.c_int32),
        ("scoring_func", ctypes.c_int32),
        ("renormalize", ctypes.c_int32),
        ("num_expert_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float),
        ("act_dtype", ctypes.c_int32),
        ("weight_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("num_shared_experts", ctypes.c_int32),
        ("non_gated", ctypes.c_int32),
        ("swiglu_alpha", ctypes.c_float),
        ("swiglu_limit", ctypes.c_float),
        ("router_weight_on_input", ctypes.c_int32),
        ("weight_layout", ctypes.c_int32),
        ("shared_intermediate", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))
        self.status = status


_lib = None
_VP = ctypes.c_void_p
_P = ctypes.POINTER(MoeParams)


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libmoe_mi355x.so is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(path)
    L.moe_workspace_size.restype = ctypes.c_size_t
    L.moe_workspace_size.argtypes = [_P]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_pack_weights.argtypes = [_VP, _VP, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _VP]
    L.moe_topk.argtypes = [_P, _VP, _VP, _VP, _VP, _VP]
    L.moe_align_permute.argtypes = [_P, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]
    L.moe_quant_act_fp8.argtypes = [_P, _VP, _VP, _VP, _VP]
    L.moe_grouped_gemm_w13_act.argtypes = [_P] + [_VP] * 12 + [ctypes.c_size_t, _VP]
    L.moe_grouped_gemm_w2_combine.argtypes = [_P] + [_VP] * 12 + [ctypes.c_size_t, _VP]
    L.moe_forward.argtypes = [_P] + [_VP] * 15 + [ctypes.c_size_t, _VP]
    L.moe_forward_noalloc.argtypes = [_P] + [_VP] * 14 + [_VP]
    L.moe_router_gemm.argtypes = [_P, _VP, _VP, ctypes.c_int32, _VP, _VP, ctypes.c_size_t, _VP]
    L.moe_router_topk.argtypes = [_P, _VP, _VP, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP,
                                  ctypes.c_size_t, _VP]
    L.moe_peak_mfma_bf16.argtypes = [ctypes.c_int64, ctypes.c_int32, _VP, _VP]
    L.moe_peak_read.argtypes = [_VP, ctypes.c_int64, ctypes.c_int32, _VP, _VP]
    # every entry point taking pointers must declare them (a bare Python int
    # would be passed as a 32-bit C int)
    for name in ENTRY_POINTS[2:]:
        assert getattr(L, name).argtypes, name
    for name in ENTRY_POINTS[2:]:
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def make_params(*, num_tokens, num_experts, top_k, hidden_size, intermediate_size,
                scoring_func=SOFTMAX, renormalize=True, num_expert_group=0, topk_group=0,
                routed_scaling_factor=1.0, act_dtype=BF16, weight_dtype=BF16, out_dtype=BF16,
                num_shared_experts=0, non_gated=False, swiglu_alpha=0.0, swiglu_limit=0.0,
                router_weight_on_input=False, weight_layout=LAYOUT_ROW_MAJOR,
                shared_intermediate=0) -> MoeParams:
    """moe_params; weight_layout defaults to row-major like a zero-initialised
    C struct (the GEMM calls then refuse the weights: pass LAYOUT_PACKED with
    weights from pack_weights)."""
    return MoeParams(int(num_tokens), int(num_experts), int(top_k), int(hidden_size),
                     int(intermediate_size), int(scoring_func), int(bool(renormalize)),
                     int(num_expert_group), int(topk_group), float(routed_scaling_factor),
                     int(act_dtype), int(weight_dtype), int(out_dtype), int(num_shared_experts),
                     int(bool(non_gated)), float(swiglu_alpha), float(swiglu_limit),
                     int(bool(router_weight_on_input)), int(weight_layout),
                     int(shared_intermediate))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn, status, raise_on_error):
    if status != MOE_OK and raise_on_error:
        raise MoeError(fn, status)
    return status


def moe_workspace_size(p: MoeParams) -> int:
    return int(load().moe_workspace_size(ctypes.byref(p)))


def moe_topk(p, router_logits, e_score_correction_bias, topk_ids, topk_weights, stream=None,
             raise_on_error=True):
    st = load().moe_topk(ctypes.byref(p), _ptr(router_logits), _ptr(e_score_correction_bias),
                         _ptr(topk_ids), _ptr(topk_weights), _stream(stream))
    return _check("moe_topk", st, raise_on_error)


def moe_align_permute(p, topk_ids, expert_offsets, sorted_slots, slot_to_row, workspace,
                      stream=None, raise_on_error=True):
    st = load().moe_align_permute(ctypes.byref(p), _ptr(topk_ids), _ptr(expert_offsets),
                                  _ptr(sorted_slots), _ptr(slot_to_row), _ptr(workspace),
                                  _nbytes(workspace), _stream(stream))
    return _check("moe_align_permute", st, raise_on_error)


def moe_pack_weights(src, dst, matrices, rows, row_bytes, stream=None, raise_on_error=True):
    st = load().moe_pack_weights(_ptr(src), _ptr(dst), int(matrices), int(rows), int(row_bytes),
                                 _stream(stream))
    return _check("moe_pack_weights", st, raise_on_error)


def pack_weights(w, stream=None):
    """Packed copy of an expert weight tensor [..., rows, cols] (any dtype):
    every trailing [rows, cols] matrix re-laid out for the GEMM calls."""
    w = w.contiguous()
    out = torch.empty_like(w)
    rows, cols = w.shape[-2], w.shape[-1]
    matrices = w.numel() // (rows * cols) if w.numel() else 0
    moe_pack_weights(w, out, matrices, rows, cols * w.element_size(), stream)
    return out


def moe_quant_act_fp8(p, hidden, q, scale, stream=None, raise_on_error=True):
    st = load().moe_quant_act_fp8(ctypes.byref(p), _ptr(hidden), _ptr(q), _ptr(scale),
                                  _stream(stream))
    return _check("moe_quant_act_fp8", st, raise_on_error)


def moe_grouped_gemm_w13_act(p, hidden, hidden_scale, w13, w13_scale, shared_w13,
                             shared_w13_scale, expert_offsets, sorted_slots, topk_weights, act,
                             act_scale, workspace, stream=None, raise_on_error=True):
    st = load().moe_grouped_gemm_w13_act(
        ctypes.byref(p), _ptr(hidden), _ptr(hidden_scale), _ptr(w13), _ptr(w13_scale),
        _ptr(shared_w13), _ptr(shared_w13_scale), _ptr(expert_offsets), _ptr(sorted_slots),
        _ptr(topk_weights), _ptr(act), _ptr(act_scale), _ptr(workspace), _nbytes(workspace),
        _stream(stream))
    return _check("moe_grouped_gemm_w13_act", st, raise_on_error)


def moe_grouped_gemm_w2_combine(p, act, act_scale, w2, w2_scale, shared_w2, shared_w2_scale,
                                expert_offsets, sorted_slots, slot_to_row, topk_weights, out,
                                workspace, stream=None, raise_on_error=True):
    st = load().moe_grouped_gemm_w2_combine(
        ctypes.byref(p), _ptr(act), _ptr(act_scale), _ptr(w2), _ptr(w2_scale), _ptr(shared_w2),
        _ptr(shared_w2_scale), _ptr(expert_offsets), _ptr(sorted_slots), _ptr(slot_to_row),
        _ptr(topk_weights), _ptr(out), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return _check("moe_grouped_gemm_w2_combine", st, raise_on_error)


def moe_router_gemm(p, hidden, gate_w, router_logits, workspace, gate_dtype=None, stream=None,
                    raise_on_error=True):
    """Router gate logits hidden W_g^T (fp32) into ``router_logits`` [T, E];
    the gate dtype follows the tensor (bfloat16 or float32) unless given."""
    if gate_dtype is None:
        gate_dtype = F32 if gate_w is not None and gate_w.dtype == torch.float32 else BF16
    st = load().moe_router_gemm(ctypes.byref(p), _ptr(hidden), _ptr(gate_w), int(gate_dtype),
                                _ptr(router_logits), _ptr(workspace), _nbytes(workspace),
                                _stream(stream))
    return _check("moe_router_gemm", st, raise_on_error)


def moe_router_topk(p, hidden, gate_w, e_score_correction_bias, topk_ids, topk_weights,
                    router_logits, workspace, gate_dtype=None, stream=None, raise_on_error=True):
    """Router gate GEMM and top-k in one call: ids and weights into topk_ids /
    topk_weights, the logits into router_logits unless it is None."""
    if gate_dtype is None:
        gate_dtype = F32 if gate_w is not None and gate_w.dtype == torch.float32 else BF16
    st = load().moe_router_topk(ctypes.byref(p), _ptr(hidden), _ptr(gate_w), int(gate_dtype),
                                _ptr(e_score_correction_bias), _ptr(topk_ids), _ptr(topk_weights),
                                _ptr(router_logits), _ptr(workspace), _nbytes(workspace),
                                _stream(stream))
    return _check("moe_router_topk", st, raise_on_error)


def moe_forward(p, hidden, router_logits, e_score_correction_bias, w13, w13_scale, w2, w2_scale,
                shared_w13, shared_w13_scale, shared_w2, shared_w2_scale, out, topk_ids_out,
                topk_weights_out, workspace, stream=None, raise_on_error=True):
    st = load().moe_forward(
        ctypes.byref(p), _ptr(hidden), _ptr(router_logits), _ptr(e_score_correction_bias),
        _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(shared_w13),
        _ptr(shared_w13_scale), _ptr(shared_w2), _ptr(shared_w2_scale), _ptr(out),
        _ptr(topk_ids_out), _ptr(topk_weights_out), _ptr(workspace), _nbytes(workspace),
        _stream(stream))
    return _check("moe_forward", st, raise_on_error)


def moe_forward_noalloc(p, hidden, router_logits, e_score_correction_bias, w13, w13_scale, w2,
                        w2_scale, shared_w13, shared_w13_scale, shared_w2, shared_w2_scale, out,
                        topk_ids_out, topk_weights_out, stream=None, raise_on_error=True):
    st = load().moe_forward_noalloc(
        ctypes.byref(p), _ptr(hidden), _ptr(router_logits), _ptr(e_score_correction_bias),
        _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(shared_w13),
        _ptr(shared_w13_scale), _ptr(shared_w2), _ptr(shared_w2_scale), _ptr(out),
        _ptr(topk_ids_out), _ptr(topk_weights_out), _stream(stream))
    return _check("moe_forward_noalloc", st, raise_on_error)


def moe_peak_mfma_bf16(iters, blocks, sink, stream=None, raise_on_error=True):
    st = load().moe_peak_mfma_bf16(int(iters), int(blocks), _ptr(sink), _stream(stream))
    return _check("moe_peak_mfma_bf16", st, raise_on_error)


def moe_peak_read(buf, blocks, sink, stream=None, raise_on_error=True):
    st = load().moe_peak_read(_ptr(buf), _nbytes(buf), int(blocks), _ptr(sink), _stream(stream))
    return _check("moe_peak_read", st, raise_on_error)


def _nbytes(t):
    if t is None:
        return 0
    return t.numel() * t.element_size()
