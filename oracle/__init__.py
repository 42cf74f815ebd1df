"""CPU oracle of the fused MoE layer (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``moe_oracle.c`` (plain C,
float64) with ctypes and numpy; it shares no code with the HIP library and
never imports it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16, FP8 = 0, 1, 2
SOFTMAX, SIGMOID = 0, 1
STANDARD, BATCHED = 0, 1
SILU, GELU = 0, 1


def compile_source(src: str, out: str) -> str:
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


_lib = None


def load_library(path: str):
    """Load a compiled oracle (the real one, or a test's mutated copy) with its signatures."""
    L = C.CDLL(path)
    i64, i32, vp, dp = C.c_int64, C.c_int, C.c_void_p, C.c_void_p
    L.oracle_e4m3_decode.restype = C.c_double
    L.oracle_e4m3_decode.argtypes = [C.c_uint8]
    L.oracle_e4m3_encode.restype = C.c_uint8
    L.oracle_e4m3_encode.argtypes = [C.c_float]
    L.oracle_e4m3_encode_array.argtypes = [i64, vp, vp]
    L.oracle_e4m3_decode_array.argtypes = [i64, vp, vp]
    L.oracle_quant_g128.argtypes = [i64, i64, vp, vp, vp]
    L.oracle_route.argtypes = [i64, i64, i64, vp, i32, i32, vp, dp]
    L.oracle_count.argtypes = [i64, vp, i64, vp]
    L.oracle_permute_standard.restype = i64
    L.oracle_permute_standard.argtypes = [i64, vp, i64, i64, vp, vp, vp, i64, vp]
    L.oracle_permute_batched.argtypes = [i64, vp, i64, i64, vp, vp]
    L.oracle_expert_row.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, i32, dp, i32, dp, dp]
    L.oracle_input_row.argtypes = [i32, i32, vp, i64, i64, i32, C.c_float, dp]
    L.oracle_combine.argtypes = [i64, i64, i64, dp, dp, vp, dp]
    L.oracle_moe_tokens.restype = i32
    L.oracle_moe_tokens.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                    i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp, dp, vp, dp]
    L.oracle_dense_mlp_tokens.restype = i32
    L.oracle_dense_mlp_tokens.argtypes = [i64, i64, i64, i32, i32, vp, vp, vp, i64, vp, dp]
    return L


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = load_library(_LIB)
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _np(t, dtype=None) -> Optional[np.ndarray]:
    """A C-contiguous host numpy view of a tensor / array (bf16 -> uint16 bits, fp8 -> uint8)."""
    if t is None:
        return None
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            if t.dtype in (torch.float8_e4m3fn,):
                return t.view(torch.uint8).numpy()
            t = t.numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(t)
    if dtype is not None:
        a = np.ascontiguousarray(a, dtype=dtype)
    return a


# ------------------------------------------------------------------- API

def host_array(t) -> Optional[np.ndarray]:
    """A host copy of a tensor in the form the calls below take (bf16 as uint16
    bits, fp8 as uint8 codes), to hand the same large tensor to many calls."""
    return _np(t)


def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().oracle_e4m3_decode_array(c.size, _p(c), _p(out))
    return out


def e4m3_encode(values) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_encode_array(v.size, _p(v), _p(out))
    return out


def quant_g128(x) -> tuple[np.ndarray, np.ndarray]:
    """Token-group-128 fp8 quantisation of fp32 rows -> (codes uint8, scales fp32)."""
    x = _np(x, np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    assert cols % 128 == 0
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    lib().oracle_quant_g128(rows, cols, _p(x), _p(q), _p(s))
    return q, s


def route(logits, k: int, scoring: int = SOFTMAX, renormalize: bool = False):
    lg = np.ascontiguousarray(_np(logits), dtype=np.float32)
    M, E = lg.shape
    ids = np.empty((M, k), np.int32)
    w = np.empty((M, k), np.float64)
    lib().oracle_route(M, E, k, _p(lg), scoring, int(renormalize), _p(ids), _p(w))
    return ids, w


def count(ids, E: int) -> np.ndarray:
    ids = np.ascontiguousarray(_np(ids), dtype=np.int32).ravel()
    c = np.empty(E, np.int32)
    lib().oracle_count(ids.size, _p(ids), E, _p(c))
    return c


def perm_len_bound(n: int, E: int, align: int) -> int:
    return n + E * (align - 1)


def permute_standard(ids, E: int, align: int = 1, perm_len: Optional[int] = None):
    """Returns (counts, offsets[E+1], perm[perm_len], inv[n])."""
    ids = np.ascontiguousarray(_np(ids), dtype=np.int32).ravel()
    n = ids.size
    if perm_len is None:
        perm_len = perm_len_bound(n, E, align)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(perm_len, np.int32)
    inv = np.empty(n, np.int32)
    lib().oracle_permute_standard(n, _p(ids), E, align, _p(counts), _p(offsets), _p(perm),
                                  perm_len, _p(inv))
    return counts, offsets, perm, inv


def permute_batched(ids, E: int, cap: int):
    """Returns (counts[E], inv[n]); inv = e*cap + rank, or -1 when rank >= cap."""
    ids = np.ascontiguousarray(_np(ids), dtype=np.int32).ravel()
    counts = np.empty(E, np.int32)
    inv = np.empty(ids.size, np.int32)
    lib().oracle_permute_batched(ids.size, _p(ids), E, cap, _p(counts), _p(inv))
    return counts, inv


def input_row(x, m: int, act_dtype: int, act_quant: int = 0, weight: Optional[float] = None) -> np.ndarray:
    """Token m's input row as the experts see it; weight: router weight applied on the input."""
    xa = _np(x)
    K = xa.shape[-1]
    a = np.empty(K, np.float64)
    lib().oracle_input_row(act_dtype, act_quant, _p(xa), K, m, int(weight is not None),
                           0.0 if weight is None else float(weight), _p(a))
    return a


def expert_row(a, e: int, w1, w2, w_dtype: int, I: int, w1_scale=None, w2_scale=None,
               requant_fp8: bool = False, activation: int = SILU):
    """Returns (act[I] before any re-quantisation, y[K])."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    K = a.size
    w1a, w2a = _np(w1), _np(w2)
    s1 = _np(w1_scale, np.float32)
    s2 = _np(w2_scale, np.float32)
    act = np.empty(I, np.float64)
    y = np.empty(K, np.float64)
    lib().oracle_expert_row(w_dtype, _p(w1a), _p(s1), _p(w2a), _p(s2), e, K, I, activation, _p(a),
                            int(requant_fp8), _p(act), _p(y))
    return act, y


def combine(w, y, keep=None) -> np.ndarray:
    """w [M, k], y [M, k, K] -> out [M, K]."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    M, k = w.shape
    K = y.shape[-1]
    kp = None if keep is None else np.ascontiguousarray(keep, dtype=np.int32).ravel()
    out = np.empty((M, K), np.float64)
    lib().oracle_combine(M, k, K, _p(w), _p(y), _p(kp), _p(out))
    return out


def moe_tokens(wl, inputs: dict, tokens=None):
    """The whole layer for the given token rows of a workload.

    inputs may hold "expert_map" (int32 [global experts], local index or -1)
    for one expert-parallel shard; wl.global_E (0: wl.E) is the router width.
    Returns (out [ntok, K] float64, ids [ntok, k] global, weights [ntok, k])."""
    logits = np.ascontiguousarray(_np(inputs["logits"]), dtype=np.float32)
    x = _np(inputs["x"])
    w1, w2 = _np(inputs["w1"]), _np(inputs["w2"])
    s1, s2 = _np(inputs.get("w1_scale"), np.float32), _np(inputs.get("w2_scale"), np.float32)
    M = logits.shape[0]
    if tokens is None:
        tokens = list(range(M))
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    out = np.empty((tok.size, wl.K), np.float64)
    ids = np.empty((tok.size, wl.topk), np.int32)
    wts = np.empty((tok.size, wl.topk), np.float64)
    emap = _np(inputs.get("expert_map"), np.int32)
    Eg = getattr(wl, "global_E", 0) or wl.E
    assert logits.shape[1] == Eg and (emap is None or emap.size == Eg)
    rc = lib().oracle_moe_tokens(M, wl.K, wl.I, wl.E, Eg, wl.topk, wl.scoring, int(wl.renormalize),
                                 wl.act_dtype, wl.w_dtype, wl.act_quant, wl.format,
                                 wl.capacity, getattr(wl, "activation", SILU),
                                 int(getattr(wl, "router_weight_on_input", False)), _p(emap),
                                 _p(logits), _p(x), _p(w1), _p(s1), _p(w2), _p(s2),
                                 tok.size, _p(tok), _p(out), _p(ids), _p(wts))
    if rc == -2:
        raise ValueError("router weight on the input needs topk == 1")
    if rc != 0:
        raise ValueError("token index out of range")
    return out, ids, wts


def dense_mlp_tokens(x, w1, w2, I: int, dtype: int, tokens=None, activation: int = SILU) -> np.ndarray:
    xa, w1a, w2a = _np(x), _np(w1), _np(w2)
    M, K = xa.shape
    if tokens is None:
        tokens = list(range(M))
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    out = np.empty((tok.size, K), np.float64)
    rc = lib().oracle_dense_mlp_tokens(M, K, I, dtype, activation, _p(xa), _p(w1a), _p(w2a), tok.size,
                                       _p(tok), _p(out))
    if rc != 0:
        raise ValueError("token index out of range")
    return out
