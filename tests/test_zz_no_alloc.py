"""moe_forward_noalloc: the layer on the library's own static workspace gives
bit for bit what moe_forward gives with a caller workspace, call after call
(the second call smaller than the first, so it runs on what the first left in
the shared array)."""
import numpy as np
import pytest
import torch

import combine_topk_softmax_amd as moe
import oracle
from tests import gpu_util as U
from workloads import FORMAT_BATCHED, WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

# in call order: each later problem is smaller than the one before it
CALLS = [
    # 128 x 256 MFMA tiles (about 600 rows per expert)
    ("bf16_mfma", WORKLOADS["mixtral_bf16"].replace(M=1200, K=512, I=256, E=4, topk=2, renormalize=False,
                                                    logits_dist="normal")),
    # weight streaming, with the shared expert on its aux stream
    ("bf16_shared", WORKLOADS["dsv3_bf16"].replace(M=256, E=32, I=256, K=512, shared_I=256)),
    # fp8 worst-tokens layout, capacity overflow flagged in the status word
    ("fp8_batched_overflow", WORKLOADS["decode_fp8_m64"].replace(M=60, K=256, I=256, E=5, topk=2, capacity=20)),
    ("fp32_tiny", WORKLOADS["tiny_fp32"].replace(M=17)),
]


def test_noalloc_forward_matches_forward_call_after_call():
    sizes = []
    for name, wl in CALLS:
        print(f"[no-alloc] {name}: M={wl.M} K={wl.K} I={wl.I} E={wl.E} top-{wl.topk}", flush=True)
        d = U.to_cuda(make_inputs(wl, seed=41, device="cpu"))
        ref, sref, ws, p = U.run_forward(wl, d)
        assert moe.workspace_size(p) <= moe.STATIC_SCRATCH_BYTES
        sizes.append(moe.workspace_size(p))
        torch.cuda.synchronize()
        ref_status = U.ws_view(ws, moe.workspace_layout(p).status, 1).item()
        out = torch.full_like(ref, float("nan"))
        shared = streams = sout = None
        if wl.shared_I:
            sout = torch.full_like(ref, float("nan"))
            shared, streams = (d["w1s"], d["w2s"], sout), moe.SharedExpertStreams()
        status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        moe.moe_forward_noalloc(p, d["logits"], d["x"], d["w1"], d.get("w1_scale"), d["w2"], d.get("w2_scale"),
                                out, shared=shared, shared_streams=streams, status_out=status)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), name
        if wl.shared_I:
            assert torch.equal(sout, sref), name
        assert status.item() == ref_status, name
        if wl.format == FORMAT_BATCHED and wl.capacity < wl.M:
            assert status.item() == moe.DEVICE_CAPACITY_OVERFLOW
        # and within the bar of the oracle on a few tokens
        toks = [0, wl.M // 2, wl.M - 1]
        oref, _, _ = oracle.moe_tokens(wl, d, toks)
        assert U.rel_err(out.float().cpu().numpy()[toks], oref) <= U.tol_for(wl), name
    assert sizes == sorted(sizes, reverse=True) and sizes[-1] < sizes[0]
