"""Shared helpers of the GPU tests: problem structs from workloads, running the
HIP path through the C ABI, reading workspace regions, error measures."""
import numpy as np
import torch

import combine_topk_softmax_amd as moe
from workloads import DTYPE_BF16, DTYPE_F32, FORMAT_BATCHED

# Output bounds: max|got - ref| / max|ref| per tensor.  bf16 operands with
# fp32 accumulation and fp8 come from the layer's stated accuracy; fp32 is
# derived: fp32 rounding of K- and I-long sums and of exp stays near 1e-6, so
# 1e-4 leaves a wide margin while still catching any real error.
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
WEIGHT_RTOL = 1e-5


def tol_for(wl) -> float:
    if wl.w_dtype == 2:
        return TOL["fp8"]
    return TOL["f32"] if wl.act_dtype == DTYPE_F32 else TOL["bf16"]


def torch_act_dtype(wl):
    return torch.float32 if wl.act_dtype == DTYPE_F32 else torch.bfloat16


def problem(wl, **over) -> moe.Problem:
    kw = dict(format=wl.format, act_dtype=wl.act_dtype, w_dtype=wl.w_dtype, act_quant=wl.act_quant,
              scoring=wl.scoring, renormalize=wl.renormalize, max_tokens_per_expert=wl.capacity,
              shared_N=2 * wl.shared_I, activation=wl.activation,
              apply_router_weight_on_input=wl.router_weight_on_input, global_E=wl.global_E)
    kw.update(over)
    return moe.make_problem(wl.E, wl.M, 2 * wl.I, wl.K, wl.topk, **kw)


def ws_view(ws: torch.Tensor, off: int, n: int, dtype=torch.int32) -> torch.Tensor:
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return ws[off: off + nbytes].view(dtype)


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def run_forward(wl, d, ws=None, p=None, out=None, shared_out=None, streams=None):
    """Whole layer through moe_forward; returns (out, shared_out or None, ws, problem).
    d may hold "expert_map" (device int32 [global_E]) for an expert-parallel shard."""
    p = p or problem(wl, expert_map=d.get("expert_map"))
    if ws is None:
        ws = moe.empty_workspace(p)
    if out is None:
        out = torch.empty(wl.M, wl.K, dtype=torch_act_dtype(wl), device="cuda")
    shared = None
    if wl.shared_I:
        if shared_out is None:
            shared_out = torch.empty(wl.M, wl.K, dtype=torch_act_dtype(wl), device="cuda")
        streams = streams or moe.SharedExpertStreams()
        shared = (d["w1s"], d["w2s"], shared_out)
    moe.moe_forward(p, d["logits"], d["x"], d["w1"], d.get("w1_scale"), d["w2"], d.get("w2_scale"), out, ws,
                    shared=shared, shared_streams=streams)
    return out, shared_out, ws, p


def to_cuda(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def batched(wl) -> bool:
    return wl.format == FORMAT_BATCHED
