"""ctypes front of the CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The product path never imports
this module.  It shares no code with the HIP library and takes every input as
plain numpy arrays (bf16 as uint16 bit patterns, e4m3 as uint8 codes).

Sources: vLLM API docs page "vllm.model_executor.layers.fused_moe.layer"
(FusedMoE.select_experts, weight layout in _load_w13/_load_w2); SGLang page
"srt/layers/moe/fused_moe_triton/layer.py" (FusedMoE.forward_impl); SGLang
page "srt/models/deepseek_v2.py" (DeepseekV2MLP, MoEGate, DeepseekV2MoE).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")

F32, BF16, E4M3 = 0, 1, 2
SOFTMAX, SIGMOID = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, -O2, no fast-math)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
             "-pthread", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


class _Layer(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("E", ctypes.c_int64), ("K", ctypes.c_int64),
        ("H", ctypes.c_int64), ("I", ctypes.c_int64),
        ("scoring", ctypes.c_int), ("renormalize", ctypes.c_int),
        ("n_group", ctypes.c_int), ("topk_group", ctypes.c_int),
        ("routed_scaling_factor", ctypes.c_double),
        ("x_dtype", ctypes.c_int), ("w_dtype", ctypes.c_int),
        ("act_fp8", ctypes.c_int),
        ("hidden", ctypes.c_void_p), ("logits", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
        ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
        ("shared_w13", ctypes.c_void_p), ("shared_w13_scale", ctypes.c_void_p),
        ("shared_w2", ctypes.c_void_p), ("shared_w2_scale", ctypes.c_void_p),
        ("gated", ctypes.c_int), ("act_alpha", ctypes.c_double),
        ("clamp_limit", ctypes.c_double), ("weight_on_input", ctypes.c_int),
        ("shared_I", ctypes.c_int64),
    ]


def _bind(path):
    L = ctypes.CDLL(path)
    L.or_bf16_to_f64.restype = ctypes.c_double
    L.or_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.or_e4m3_to_f64.restype = ctypes.c_double
    L.or_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    L.or_e4m3_from_f32.restype = ctypes.c_uint8
    L.or_e4m3_from_f32.argtypes = [ctypes.c_float]
    L.or_quant_fp8_groups.restype = None
    L.or_quant_fp8_groups.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 3
    L.or_route.restype = ctypes.c_int
    L.or_route.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                           ctypes.c_int, ctypes.c_int, ctypes.c_int,
                           ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
    L.or_permute.restype = ctypes.c_int
    L.or_permute.argtypes = [ctypes.c_int64, ctypes.c_int] + [ctypes.c_void_p] * 4
    L.or_router_logits.restype = None
    L.or_router_logits.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_void_p, ctypes.c_int,
                                                          ctypes.c_void_p, ctypes.c_int,
                                                          ctypes.c_void_p]
    L.or_moe_forward_tokens.restype = ctypes.c_int
    L.or_moe_forward_tokens.argtypes = [ctypes.POINTER(_Layer), ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int]
    return L


def lib():
    """The oracle library built from oracle/moe_oracle.c (built on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        _lib = _bind(LIB)
    return _lib


def load_variant(path):
    """Bind another build of the oracle source (used by the planted-mistake
    tests, which compile edited copies to prove that the pins catch them)."""
    return _bind(path)


def _ptr(a):
    return None if a is None else a.ctypes.data


def bf16_to_f64(bits: np.ndarray, lib_=None) -> np.ndarray:
    L = lib_ or lib()
    f = np.vectorize(lambda v: L.or_bf16_to_f64(int(v)), otypes=[np.float64])
    return f(np.asarray(bits, dtype=np.uint16))


def e4m3_to_f64(codes: np.ndarray, lib_=None) -> np.ndarray:
    L = lib_ or lib()
    f = np.vectorize(lambda v: L.or_e4m3_to_f64(int(v)), otypes=[np.float64])
    return f(np.asarray(codes, dtype=np.uint8))


def e4m3_from_f32(x: np.ndarray, lib_=None) -> np.ndarray:
    L = lib_ or lib()
    f = np.vectorize(lambda v: L.or_e4m3_from_f32(float(v)), otypes=[np.uint8])
    return f(np.asarray(x, dtype=np.float32))


def quant_fp8_groups(x: np.ndarray, group: int = 128, lib_=None):
    """Per-row, per-group fp8 quantisation; returns (codes uint8, scales f32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    assert cols % group == 0
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // group), np.float32)
    (lib_ or lib()).or_quant_fp8_groups(rows, cols, group, _ptr(x), _ptr(q), _ptr(s))
    return q, s


def route(logits: np.ndarray, K: int, *, bias=None, scoring: int = SOFTMAX,
          renormalize: bool = True, n_group: int = 0, topk_group: int = 0,
          routed_scaling_factor: float = 1.0, lib_=None):
    """Top-k routing of every row; returns (ids int32 [T,K], weights f64 [T,K])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    rc = (lib_ or lib()).or_route(T, E, K, _ptr(logits), _ptr(b), scoring, int(renormalize),
                        n_group, topk_group, routed_scaling_factor, _ptr(ids), _ptr(w))
    if rc:
        raise ValueError("oracle routing rejected the arguments")
    return ids, w


def permute(ids: np.ndarray, E: int, lib_=None):
    """Stable expert-major permutation of the flat slots t*K+k."""
    flat = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    n = flat.size
    offsets = np.empty(E + 1, np.int32)
    sorted_slots = np.empty(n, np.int32)
    slot_to_row = np.empty(n, np.int32)
    rc = (lib_ or lib()).or_permute(n, E, _ptr(flat), _ptr(offsets), _ptr(sorted_slots),
                          _ptr(slot_to_row))
    if rc:
        raise ValueError("oracle permutation rejected the ids")
    return offsets, sorted_slots, slot_to_row


def router_logits(hidden: np.ndarray, x_dtype: int, gate: np.ndarray, g_dtype: int,
                  lib_=None) -> np.ndarray:
    """Router gate logits x W_g^T in float64 ([T, E]); hidden [T, H] and gate
    [E, H] as float32 arrays (F32) or bf16 bit patterns (BF16)."""
    hidden = np.ascontiguousarray(hidden)
    gate = np.ascontiguousarray(gate)
    T, H = hidden.shape
    E = gate.shape[0]
    assert gate.shape[1] == H
    out = np.empty((T, E), np.float64)
    (lib_ or lib()).or_router_logits(T, E, H, _ptr(hidden), x_dtype, _ptr(gate), g_dtype,
                                     _ptr(out))
    return out


def _expert_ptrs(per_expert, E):
    """Array of E pointers from either one [E, ...] array or a dict e -> array."""
    arr = (ctypes.c_void_p * E)()
    keep = []
    for e in range(E):
        a = None
        if isinstance(per_expert, dict):
            a = per_expert.get(e)
        elif per_expert is not None:
            a = per_expert[e]
        if a is not None:
            a = np.ascontiguousarray(a)
            keep.append(a)
            arr[e] = a.ctypes.data
    return arr, keep


def moe_forward_tokens(layer: dict, tokens, nthreads: int = 1, lib_=None) -> np.ndarray:
    """Layer output (float64, [len(tokens), H]) for the listed token indices.

    ``layer`` keys: T E K H I, scoring, renormalize, n_group, topk_group,
    routed_scaling_factor, x_dtype, w_dtype, act_fp8, hidden, logits, bias,
    w13, w13_scale, w2, w2_scale, shared_w13, shared_w13_scale, shared_w2,
    shared_w2_scale, shared_I (the shared expert's intermediate size; 0 or
    absent: I), and the activation variants gated (True), act_alpha
    (1.0), clamp_limit (0.0: none), weight_on_input (False).  Weight entries
    are [E, ...] arrays or dicts e -> array (only the experts the listed
    tokens use need to be present).
    """
    E = int(layer["E"])
    keep = []

    def arr(key, dtype=None):
        a = layer.get(key)
        if a is None:
            return None
        a = np.ascontiguousarray(a) if dtype is None else np.ascontiguousarray(a, dtype=dtype)
        keep.append(a)
        return a

    st = _Layer()
    for k in ("T", "E", "K", "H", "I"):
        setattr(st, k, int(layer[k]))
    st.scoring = int(layer.get("scoring", SOFTMAX))
    st.renormalize = int(bool(layer.get("renormalize", True)))
    st.n_group = int(layer.get("n_group", 0))
    st.topk_group = int(layer.get("topk_group", 0))
    st.routed_scaling_factor = float(layer.get("routed_scaling_factor", 1.0))
    st.x_dtype = int(layer["x_dtype"])
    st.w_dtype = int(layer["w_dtype"])
    st.act_fp8 = int(bool(layer.get("act_fp8", False)))
    st.gated = int(bool(layer.get("gated", True)))
    st.act_alpha = float(layer.get("act_alpha", 1.0))
    st.clamp_limit = float(layer.get("clamp_limit", 0.0))
    st.weight_on_input = int(bool(layer.get("weight_on_input", False)))
    st.shared_I = int(layer.get("shared_I", 0))
    st.hidden = _ptr(arr("hidden"))
    st.logits = _ptr(arr("logits", np.float32))
    st.bias = _ptr(arr("bias", np.float32))
    p13, k13 = _expert_ptrs(layer["w13"], E)
    p2, k2 = _expert_ptrs(layer["w2"], E)
    keep += [p13, k13, p2, k2]
    st.w13 = ctypes.addressof(p13)
    st.w2 = ctypes.addressof(p2)
    if layer.get("w13_scale") is not None:
        s13, ks13 = _expert_ptrs(layer["w13_scale"], E)
        s2, ks2 = _expert_ptrs(layer["w2_scale"], E)
        keep += [s13, ks13, s2, ks2]
        st.w13_scale = ctypes.addressof(s13)
        st.w2_scale = ctypes.addressof(s2)
    st.shared_w13 = _ptr(arr("shared_w13"))
    st.shared_w13_scale = _ptr(arr("shared_w13_scale", np.float32))
    st.shared_w2 = _ptr(arr("shared_w2"))
    st.shared_w2_scale = _ptr(arr("shared_w2_scale", np.float32))
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    out = np.empty((tok.size, int(layer["H"])), np.float64)
    rc = (lib_ or lib()).or_moe_forward_tokens(ctypes.byref(st), tok.size, _ptr(tok), _ptr(out),
                                     int(nthreads))
    if rc:
        raise ValueError("oracle forward failed (status %d)" % rc)
    return out
