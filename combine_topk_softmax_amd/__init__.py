"""Fused MoE layer for AMD Instinct MI355X (gfx950): Python binding.

A thin ctypes layer over ``libmoe_gfx950.so`` (see ``include/moe.h``): it only
marshals torch tensors, streams and events into the C ABI.  Every step of the
layer runs in the library's HIP kernels; there is no fallback of any kind, and
importing the binding without the built library raises.

Build the library in-tree with ``python -m combine_topk_softmax_amd.build``.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIBRARY may name another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(_HERE, "libmoe_gfx950.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
FORMAT_STANDARD, FORMAT_BATCHED_EXPERTS = 0, 1
DTYPE_F32, DTYPE_BF16, DTYPE_FP8_E4M3 = 0, 1, 2
QUANT_NONE, QUANT_FP8_TOKEN_GROUP_128 = 0, 1
SCORING_SOFTMAX, SCORING_SIGMOID = 0, 1
ACTIVATION_SILU, ACTIVATION_GELU = 0, 1
DEVICE_BAD_EXPERT_ID, DEVICE_CAPACITY_OVERFLOW = 1, 2
WEIGHTS_ROW_MAJOR, WEIGHTS_PACKED = 0, 1
NUM_STAGE_EVENTS = 6


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} ({status})")
        self.status = status


class Problem(C.Structure):
    _fields_ = [
        ("E", C.c_int64), ("M", C.c_int64), ("N", C.c_int64), ("K", C.c_int64),
        ("topk", C.c_int64), ("max_tokens_per_expert", C.c_int64), ("align", C.c_int64),
        ("shared_N", C.c_int64), ("global_E", C.c_int64), ("chunk_tokens", C.c_int64),
        ("format", C.c_int32), ("act_dtype", C.c_int32), ("w_dtype", C.c_int32),
        ("act_quant", C.c_int32), ("scoring", C.c_int32), ("renormalize", C.c_int32),
        ("activation", C.c_int32), ("apply_router_weight_on_input", C.c_int32),
        ("weight_layout", C.c_int32), ("reserved", C.c_int32),
        ("expert_map", C.c_void_p),
    ]


class Weights(C.Structure):
    _fields_ = [("w1", C.c_void_p), ("w1_scale", C.c_void_p), ("w2", C.c_void_p), ("w2_scale", C.c_void_p)]


class Shared(C.Structure):
    _fields_ = [("w1", C.c_void_p), ("w2", C.c_void_p), ("out", C.c_void_p), ("aux_stream", C.c_void_p),
                ("input_ready", C.c_void_p), ("output_ready", C.c_void_p)]


class StageEvents(C.Structure):
    _fields_ = [("ev", C.c_void_p * NUM_STAGE_EVENTS)]


class DboEventsStruct(C.Structure):
    _fields_ = [("prepared", C.c_void_p * 2), ("computed", C.c_void_p * 2), ("finalized", C.c_void_p * 2)]


class WsLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in (
        "total_bytes", "status", "counts", "offsets", "chunk_hist", "tiles", "perm", "inv", "act",
        "act_q", "act_scale", "topk_weights", "topk_ids", "a_q", "a_scale", "fused_out", "shared_act")]
    _fields_ += [(n, C.c_int64) for n in ("perm_len", "n_chunks", "chunk", "max_tiles", "tile_rows", "act_rows")]
    _fields_ += [("down_partial", C.c_size_t), ("down_split", C.c_int64)]


EXPORTS = ("moe_status_str", "moe_version", "moe_validate", "moe_workspace_size", "moe_workspace_layout",
           "moe_pack_weights", "moe_route", "moe_prepare", "moe_experts", "moe_finalize", "moe_shared_expert", "moe_forward",
           "moe_forward_noalloc", "moe_prepare_async", "moe_finalize_async", "moe_receive", "moe_forward_dbo")

_lib = None
ABI_VERSION = 5   # the struct layouts and calls mirrored here
STATIC_SCRATCH_BYTES = 64 << 20   # MOE_STATIC_SCRATCH_BYTES of moe_forward_noalloc


def load_library(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m combine_topk_softmax_amd.build`")
    L = C.CDLL(path)
    vp, P = C.c_void_p, C.POINTER
    L.moe_status_str.restype = C.c_char_p
    L.moe_status_str.argtypes = [C.c_int]
    L.moe_version.restype = C.c_int
    if L.moe_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {L.moe_version()}, this binding expects {ABI_VERSION}: rebuild it")
    for name, args in {
        "moe_validate": [P(Problem)],
        "moe_workspace_size": [P(Problem), P(C.c_size_t)],
        "moe_workspace_layout": [P(Problem), P(WsLayout)],
        "moe_pack_weights": [P(Problem), P(Weights), vp, vp, vp],
        "moe_route": [P(Problem), vp, vp, vp, vp],
        "moe_prepare": [P(Problem), vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp],
        "moe_experts": [P(Problem), vp, vp, P(Weights), vp, vp, vp, C.c_size_t, vp],
        "moe_finalize": [P(Problem), vp, vp, vp, vp, C.c_size_t, vp],
        "moe_shared_expert": [P(Problem), vp, vp, vp, vp, vp, C.c_size_t, vp],
        "moe_forward": [P(Problem), vp, vp, P(Weights), vp, P(Shared), vp, C.c_size_t, vp, P(StageEvents)],
        "moe_forward_noalloc": [P(Problem), vp, vp, P(Weights), vp, P(Shared), vp, P(StageEvents), vp],
        "moe_prepare_async": [P(Problem), vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp, vp],
        "moe_finalize_async": [P(Problem), vp, vp, vp, vp, C.c_size_t, vp, vp],
        "moe_receive": [vp, vp],
        "moe_forward_dbo": [P(Problem), vp, vp, P(Weights), vp, P(Shared), vp, vp, C.c_size_t, vp, vp,
                            P(DboEventsStruct)],
    }.items():
        f = getattr(L, name)
        f.restype = C.c_int
        f.argtypes = args
    _lib = L
    return L


def status_str(status: int) -> str:
    return load_library().moe_status_str(status).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the HIP library must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ws(ws: torch.Tensor):
    return _ptr(ws), ws.numel() * ws.element_size()


def make_problem(E, M, N, K, topk, *, format=FORMAT_STANDARD, act_dtype=DTYPE_BF16, w_dtype=DTYPE_BF16,
                 act_quant=QUANT_NONE, scoring=SCORING_SOFTMAX, renormalize=False,
                 max_tokens_per_expert=0, align=0, shared_N=0, weight_layout=WEIGHTS_ROW_MAJOR,
                 activation=ACTIVATION_SILU, apply_router_weight_on_input=False, global_E=0,
                 expert_map: Optional[torch.Tensor] = None, chunk_tokens=0) -> Problem:
    """expert_map: device int32 tensor [global_E] (local expert or -1); the
    caller keeps it alive while the problem is in use."""
    if expert_map is not None and (expert_map.dtype != torch.int32 or expert_map.numel() != (global_E or E)):
        raise ValueError("expert_map must be an int32 tensor of global_E entries")
    return Problem(E=E, M=M, N=N, K=K, topk=topk, max_tokens_per_expert=max_tokens_per_expert, align=align,
                   shared_N=shared_N, global_E=global_E, chunk_tokens=chunk_tokens, format=format, act_dtype=act_dtype, w_dtype=w_dtype,
                   act_quant=act_quant, scoring=scoring, renormalize=int(renormalize), activation=activation,
                   apply_router_weight_on_input=int(apply_router_weight_on_input), weight_layout=weight_layout,
                   reserved=0, expert_map=_ptr(expert_map))


def validate(p: Problem) -> int:
    return load_library().moe_validate(C.byref(p))


def workspace_size(p: Problem) -> int:
    n = C.c_size_t()
    _check(load_library().moe_workspace_size(C.byref(p), C.byref(n)), "moe_workspace_size")
    return n.value


def workspace_layout(p: Problem) -> WsLayout:
    L = WsLayout()
    _check(load_library().moe_workspace_layout(C.byref(p), C.byref(L)), "moe_workspace_layout")
    return L


def empty_workspace(p: Problem, device="cuda") -> torch.Tensor:
    return torch.empty(workspace_size(p), dtype=torch.uint8, device=device)


def moe_pack_weights(p: Problem, w1, w2, w1_packed, w2_packed, stream=None):
    """One-time reordering of row-major w1 / w2 into the packed layout."""
    src = _weights(w1, None, w2, None)
    _check(load_library().moe_pack_weights(C.byref(p), C.byref(src), _ptr(w1_packed), _ptr(w2_packed),
                                           _stream(stream)), "moe_pack_weights")


def pack_weights(p: Problem, w1, w2, stream=None):
    """Packed copies of w1 / w2 (new tensors of the same shape and dtype)."""
    w1p, w2p = torch.empty_like(w1), torch.empty_like(w2)
    moe_pack_weights(p, w1, w2, w1p, w2p, stream)
    return w1p, w2p


def moe_route(p: Problem, logits, topk_weights, topk_ids, stream=None):
    _check(load_library().moe_route(C.byref(p), _ptr(logits), _ptr(topk_weights), _ptr(topk_ids),
                                    _stream(stream)), "moe_route")


def moe_prepare(p: Problem, x, topk_ids, a_out, a_scale_out, expert_num_tokens, workspace, stream=None,
                topk_weights=None):
    """topk_weights is read only with apply_router_weight_on_input."""
    wp, wn = _ws(workspace)
    _check(load_library().moe_prepare(C.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(a_out),
                                      _ptr(a_scale_out), _ptr(expert_num_tokens), wp, wn, _stream(stream)),
           "moe_prepare")


def _weights(w1, w1_scale, w2, w2_scale) -> Weights:
    return Weights(_ptr(w1), _ptr(w1_scale), _ptr(w2), _ptr(w2_scale))


def moe_experts(p: Problem, a, a_scale, w1, w1_scale, w2, w2_scale, expert_num_tokens, fused_out, workspace,
                stream=None):
    wp, wn = _ws(workspace)
    w = _weights(w1, w1_scale, w2, w2_scale)
    _check(load_library().moe_experts(C.byref(p), _ptr(a), _ptr(a_scale), C.byref(w), _ptr(expert_num_tokens),
                                      _ptr(fused_out), wp, wn, _stream(stream)), "moe_experts")


def moe_finalize(p: Problem, fused_out, topk_weights, out, workspace, stream=None):
    wp, wn = _ws(workspace)
    _check(load_library().moe_finalize(C.byref(p), _ptr(fused_out), _ptr(topk_weights), _ptr(out), wp, wn,
                                       _stream(stream)), "moe_finalize")


def moe_shared_expert(p: Problem, x, w1, w2, out, workspace, stream=None):
    wp, wn = _ws(workspace)
    _check(load_library().moe_shared_expert(C.byref(p), _ptr(x), _ptr(w1), _ptr(w2), _ptr(out), wp, wn,
                                            _stream(stream)), "moe_shared_expert")


def _event_handle(ev: torch.cuda.Event) -> int:
    if ev.cuda_event == 0:            # torch creates events lazily
        ev.record()
    return ev.cuda_event


class SharedExpertStreams:
    """The aux stream and the two events the shared expert overlaps with."""

    def __init__(self, device=None):
        self.stream = torch.cuda.Stream(device=device)
        self.input_ready = torch.cuda.Event()
        self.output_ready = torch.cuda.Event()


def _shared_and_events(shared, shared_streams, events):
    sh = None
    if shared is not None:
        if shared_streams is None:
            raise ValueError("a shared expert needs SharedExpertStreams")
        w1s, w2s, sout = shared
        sh = Shared(_ptr(w1s), _ptr(w2s), _ptr(sout), shared_streams.stream.cuda_stream,
                    _event_handle(shared_streams.input_ready), _event_handle(shared_streams.output_ready))
    ev = None
    if events is not None:
        ev = StageEvents()
        for i, e in enumerate(events[:NUM_STAGE_EVENTS]):
            ev.ev[i] = _event_handle(e) if e is not None else None
    return (C.byref(sh) if sh is not None else None), (C.byref(ev) if ev is not None else None)


def moe_forward(p: Problem, logits, x, w1, w1_scale, w2, w2_scale, out, workspace, stream=None,
                shared=None, shared_streams: Optional[SharedExpertStreams] = None, events=None):
    """shared = (w1s, w2s, shared_out); events = list of torch.cuda.Event (timing) or None."""
    L = load_library()
    wp, wn = _ws(workspace)
    w = _weights(w1, w1_scale, w2, w2_scale)
    sh, ev = _shared_and_events(shared, shared_streams, events)
    _check(L.moe_forward(C.byref(p), _ptr(logits), _ptr(x), C.byref(w), _ptr(out), sh, wp, wn, _stream(stream),
                         ev), "moe_forward")


def moe_forward_noalloc(p: Problem, logits, x, w1, w1_scale, w2, w2_scale, out, stream=None, shared=None,
                        shared_streams: Optional[SharedExpertStreams] = None, events=None, status_out=None):
    """moe_forward on the library's own static workspace (no caller workspace,
    no allocation); status_out: optional device int32 tensor of one element
    that receives the call's device status word."""
    L = load_library()
    w = _weights(w1, w1_scale, w2, w2_scale)
    sh, ev = _shared_and_events(shared, shared_streams, events)
    _check(L.moe_forward_noalloc(C.byref(p), _ptr(logits), _ptr(x), C.byref(w), _ptr(out), sh, _stream(stream),
                                 ev, _ptr(status_out)), "moe_forward_noalloc")


# ------------------------------------------- asynchronous prepare / finalize

def moe_prepare_async(p: Problem, x, topk_ids, a_out, a_scale_out, expert_num_tokens, workspace, stream, done,
                      topk_weights=None):
    """moe_prepare enqueued on `stream`, `done` (torch.cuda.Event) recorded after it."""
    wp, wn = _ws(workspace)
    _check(load_library().moe_prepare_async(C.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(a_out),
                                            _ptr(a_scale_out), _ptr(expert_num_tokens), wp, wn, _stream(stream),
                                            _event_handle(done)), "moe_prepare_async")


def moe_finalize_async(p: Problem, fused_out, topk_weights, out, workspace, stream, done):
    wp, wn = _ws(workspace)
    _check(load_library().moe_finalize_async(C.byref(p), _ptr(fused_out), _ptr(topk_weights), _ptr(out), wp, wn,
                                             _stream(stream), _event_handle(done)), "moe_finalize_async")


def moe_receive(stream, done):
    """`stream` waits on the device for the work `done` marks."""
    _check(load_library().moe_receive(_stream(stream), _event_handle(done)), "moe_receive")


class DboEvents:
    """The six events of moe_forward_dbo."""

    def __init__(self):
        self.events = [torch.cuda.Event() for _ in range(6)]

    def struct(self) -> DboEventsStruct:
        h = [_event_handle(e) for e in self.events]
        return DboEventsStruct((C.c_void_p * 2)(h[0], h[1]), (C.c_void_p * 2)(h[2], h[3]),
                               (C.c_void_p * 2)(h[4], h[5]))


def dbo_microbatch_problem(p: Problem) -> Problem:
    """The problem each moe_forward_dbo workspace is sized for ((M + 1) / 2 tokens)."""
    q = Problem.from_buffer_copy(p)
    q.M = (p.M + 1) // 2
    return q


def moe_forward_dbo(p: Problem, logits, x, w1, w1_scale, w2, w2_scale, out, workspaces, comm_stream,
                    events: DboEvents, stream=None, shared=None, shared_streams=None):
    """Two-microbatch layer.  workspaces: two tensors of at least
    workspace_size(dbo_microbatch_problem(p)) bytes; shared = (w1s, w2s,
    shared_out) with shared_streams a pair of SharedExpertStreams (one per
    microbatch)."""
    L = load_library()
    w0, n0 = _ws(workspaces[0])
    w1p, n1 = _ws(workspaces[1])
    w = _weights(w1, w1_scale, w2, w2_scale)
    sh = None
    if shared is not None:
        if shared_streams is None or len(shared_streams) != 2:
            raise ValueError("a shared expert needs one SharedExpertStreams per microbatch")
        w1s, w2s, sout = shared
        m0 = (p.M + 1) // 2
        halves = (sout[:m0], sout[m0:])
        sh = (Shared * 2)(*[Shared(_ptr(w1s), _ptr(w2s), _ptr(halves[u]) if halves[u].numel() else None,
                                   shared_streams[u].stream.cuda_stream,
                                   _event_handle(shared_streams[u].input_ready),
                                   _event_handle(shared_streams[u].output_ready)) for u in range(2)])
    ev = events.struct()
    _check(L.moe_forward_dbo(C.byref(p), _ptr(logits), _ptr(x), C.byref(w), _ptr(out), sh, w0, w1p, min(n0, n1),
                             _stream(stream), _stream(comm_stream), C.byref(ev)), "moe_forward_dbo")
