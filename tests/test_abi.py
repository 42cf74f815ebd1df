"""The C ABI without a GPU: the library loads, exports every entry point that
include/moe.h declares, the ctypes structs match the C layout, and host-side
validation returns the documented status codes (no kernel is launched)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import combine_topk_softmax_amd as moe
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char \*|int)\s*\*?\s*(moe_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    L = moe.load_library()
    names = _declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(moe.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, re.M), n


def test_version_and_status_strings():
    L = moe.load_library()
    assert L.moe_version() == 5
    assert moe.status_str(moe.MOE_OK) == "ok"
    assert "workspace" in moe.status_str(moe.MOE_ERR_WORKSPACE)


_LAYOUT_PROBE = r"""
#include <stdio.h>
#include <stddef.h>
#include "moe.h"
#define F(T, f) printf(#T "." #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("moe_problem %zu\n", sizeof(moe_problem));
  F(moe_problem, E) F(moe_problem, max_tokens_per_expert) F(moe_problem, shared_N) F(moe_problem, global_E)
  F(moe_problem, chunk_tokens)
  F(moe_problem, format)
  F(moe_problem, apply_router_weight_on_input) F(moe_problem, weight_layout) F(moe_problem, expert_map)
  printf("moe_weights %zu\n", sizeof(moe_weights));
  printf("moe_shared %zu\n", sizeof(moe_shared));
  F(moe_shared, output_ready)
  printf("moe_stage_events %zu\n", sizeof(moe_stage_events));
  printf("moe_ws_layout %zu\n", sizeof(moe_ws_layout));
  F(moe_ws_layout, shared_act) F(moe_ws_layout, perm_len) F(moe_ws_layout, act_rows)
  return 0;
}
"""


def test_ctypes_structs_match_c_layout(tmp_path):
    src = tmp_path / "probe.c"
    src.write_text(_LAYOUT_PROBE)
    exe = tmp_path / "probe"
    subprocess.check_call(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                           "-I", "/opt/rocm/include", str(src), "-o", str(exe)])
    got = dict(line.rsplit(" ", 1) for line in subprocess.check_output([str(exe)], text=True).splitlines())
    py = {
        "moe_problem": C.sizeof(moe.Problem), "moe_weights": C.sizeof(moe.Weights),
        "moe_shared": C.sizeof(moe.Shared), "moe_stage_events": C.sizeof(moe.StageEvents),
        "moe_ws_layout": C.sizeof(moe.WsLayout),
    }
    for k, v in py.items():
        assert int(got[k]) == v, k
    for key, val in got.items():
        if "." in key:
            struct, field = key.split(".")
            cls = {"moe_problem": moe.Problem, "moe_shared": moe.Shared, "moe_ws_layout": moe.WsLayout}[struct]
            assert getattr(cls, field).offset == int(val), key


def _prob(wl):
    return moe.make_problem(wl.E, wl.M, 2 * wl.I, wl.K, wl.topk, format=wl.format, act_dtype=wl.act_dtype,
                            w_dtype=wl.w_dtype, act_quant=wl.act_quant, scoring=wl.scoring,
                            renormalize=wl.renormalize, max_tokens_per_expert=wl.capacity,
                            shared_N=2 * wl.shared_I)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workloads_validate_and_layout(name):
    wl = WORKLOADS[name]
    p = _prob(wl)
    assert moe.validate(p) == moe.MOE_OK
    L = moe.workspace_layout(p)
    assert L.total_bytes == moe.workspace_size(p)
    n = wl.M * wl.topk
    offs = sorted((getattr(L, f), f) for f, _ in moe.WsLayout._fields_[1:17] + [("down_partial", None)])
    assert all(o % 256 == 0 for o, _ in offs)
    assert offs[-1][0] <= L.total_bytes
    if wl.format == moe.FORMAT_STANDARD:
        assert L.perm_len == n and L.act_rows == n
    else:
        assert L.act_rows == wl.E * wl.capacity
    assert L.max_tiles >= -(-n // 128)
    assert L.n_chunks * L.chunk >= n and L.n_chunks <= 256


def test_validation_status_codes():
    base = dict(E=8, M=16, N=256, K=256, topk=2)
    ok = moe.make_problem(**base)
    assert moe.validate(ok) == moe.MOE_OK
    bad = [
        (dict(base, topk=9), moe.MOE_ERR_INVALID_ARG),                 # topk > E
        (dict(base, N=255), moe.MOE_ERR_INVALID_ARG),                  # odd N (activation halves it)
        (dict(base, M=-1), moe.MOE_ERR_INVALID_ARG),
        (dict(base, E=0), moe.MOE_ERR_INVALID_ARG),
        (dict(base, K=200), moe.MOE_ERR_UNSUPPORTED),                  # K % 128
        (dict(base, N=2 * 96), moe.MOE_ERR_UNSUPPORTED),               # I % 64
        (dict(base, E=2048, topk=2), moe.MOE_ERR_UNSUPPORTED),
    ]
    for kw, code in bad:
        assert moe.validate(moe.make_problem(**kw)) == code, kw
    p = moe.make_problem(**base, format=moe.FORMAT_BATCHED_EXPERTS)          # capacity missing
    assert moe.validate(p) == moe.MOE_ERR_INVALID_ARG
    p = moe.make_problem(**base, w_dtype=moe.DTYPE_FP8_E4M3)                  # fp8 weights need fp8 acts
    assert moe.validate(p) == moe.MOE_ERR_UNSUPPORTED
    p = moe.make_problem(**base, act_dtype=moe.DTYPE_F32)                     # mixed f32 x bf16
    assert moe.validate(p) == moe.MOE_ERR_UNSUPPORTED
    p = moe.make_problem(**base)
    p.activation = 2                                                          # silu or gelu only
    assert moe.validate(p) == moe.MOE_ERR_UNSUPPORTED
    assert moe.validate(moe.make_problem(**base, activation=moe.ACTIVATION_GELU)) == moe.MOE_OK
    p = moe.make_problem(**base, apply_router_weight_on_input=True)          # needs topk == 1
    assert moe.validate(p) == moe.MOE_ERR_INVALID_ARG
    p = moe.make_problem(**dict(base, topk=1), apply_router_weight_on_input=True)
    assert moe.validate(p) == moe.MOE_OK
    p = moe.make_problem(**base)
    p.apply_router_weight_on_input = 2
    assert moe.validate(p) == moe.MOE_ERR_INVALID_ARG
    # expert-parallel shard: global_E without a map, local experts above global
    assert moe.validate(moe.make_problem(**base, global_E=16)) == moe.MOE_ERR_INVALID_ARG
    p = moe.make_problem(**base, global_E=16)
    p.expert_map = 0x1000                                                     # any device pointer
    assert moe.validate(p) == moe.MOE_OK
    p = moe.make_problem(**dict(base, E=20), global_E=16)
    p.expert_map = 0x1000
    assert moe.validate(p) == moe.MOE_ERR_INVALID_ARG
    p = moe.make_problem(**dict(base, E=4, topk=6), global_E=16)             # topk bounded by global_E
    p.expert_map = 0x1000
    assert moe.validate(p) == moe.MOE_OK
    p = moe.make_problem(**base, global_E=2048)
    p.expert_map = 0x1000
    assert moe.validate(p) == moe.MOE_ERR_UNSUPPORTED
    assert moe.validate(moe.make_problem(**base, global_E=-1)) == moe.MOE_ERR_INVALID_ARG
    # activation chunking: Standard format only
    assert moe.validate(moe.make_problem(**base, chunk_tokens=-1)) == moe.MOE_ERR_INVALID_ARG
    assert moe.validate(moe.make_problem(**base, chunk_tokens=4)) == moe.MOE_OK
    assert moe.validate(moe.make_problem(**base, chunk_tokens=4, format=moe.FORMAT_BATCHED_EXPERTS,
                                         max_tokens_per_expert=16)) == moe.MOE_ERR_UNSUPPORTED
    p = moe.make_problem(**base)
    p.scoring = 7
    assert moe.validate(p) == moe.MOE_ERR_INVALID_ARG
    p = moe.make_problem(**base, weight_layout=5)
    assert moe.validate(p) == moe.MOE_ERR_INVALID_ARG
    p = moe.make_problem(**dict(base, N=2 * 192), weight_layout=moe.WEIGHTS_PACKED)   # packed panels need I % 128
    assert moe.validate(p) == moe.MOE_ERR_UNSUPPORTED
    assert moe.validate(moe.make_problem(**dict(base, N=2 * 192))) == moe.MOE_OK


def test_host_errors_need_no_gpu():
    """Calls that fail validation, or have M == 0, return before touching the device."""
    L = moe.load_library()
    p = moe.make_problem(E=8, M=16, N=256, K=256, topk=2)
    ws_size = moe.workspace_size(p)
    assert L.moe_route(C.byref(p), None, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_prepare(C.byref(p), None, None, None, None, None, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    fake = C.c_void_p(0x1000)
    assert L.moe_prepare(C.byref(p), fake, fake, None, None, None, fake, fake, ws_size - 1, None) \
        == moe.MOE_ERR_WORKSPACE
    # router weight on the input: prepare needs the weights and an a_out
    p1 = moe.make_problem(E=8, M=16, N=256, K=256, topk=1, apply_router_weight_on_input=True)
    ws1 = moe.workspace_size(p1)
    assert L.moe_prepare(C.byref(p1), fake, fake, None, fake, None, fake, fake, ws1, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_prepare(C.byref(p1), fake, fake, fake, None, None, fake, fake, ws1, None) == moe.MOE_ERR_INVALID_ARG
    w = moe.Weights(None, None, None, None)
    assert L.moe_experts(C.byref(p), fake, None, C.byref(w), fake, fake, fake, ws_size, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_finalize(C.byref(p), None, None, None, fake, ws_size, None) == moe.MOE_ERR_INVALID_ARG
    # shared expert requested by the problem but not given
    ps = moe.make_problem(E=8, M=16, N=256, K=256, topk=2, shared_N=256)
    assert L.moe_forward(C.byref(ps), fake, fake, C.byref(w), fake, None, fake, 1 << 40, None, None) \
        == moe.MOE_ERR_INVALID_ARG
    assert L.moe_shared_expert(C.byref(p), fake, fake, fake, fake, fake, ws_size, None) == moe.MOE_ERR_INVALID_ARG
    src = moe.Weights(0x1000, None, 0x2000, None)
    assert L.moe_pack_weights(C.byref(p), C.byref(src), None, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(C.byref(p), C.byref(src), C.c_void_p(0x1000), C.c_void_p(0x3000), None) \
        == moe.MOE_ERR_INVALID_ARG                                                   # in place
    # chunking belongs to moe_forward: the stage calls refuse a chunked problem
    pc = moe.make_problem(E=8, M=16, N=256, K=256, topk=2, chunk_tokens=4)
    wsc = moe.workspace_size(pc)
    assert L.moe_prepare(C.byref(pc), fake, fake, None, None, None, fake, fake, wsc, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_experts(C.byref(pc), fake, None, C.byref(moe.Weights(0x1000, None, 0x2000, None)), fake, fake,
                         fake, wsc, None) == moe.MOE_ERR_UNSUPPORTED
    # M == 0: nothing to do, nothing launched
    p0 = moe.make_problem(E=8, M=0, N=256, K=256, topk=2)
    assert L.moe_route(C.byref(p0), None, None, None, None) == moe.MOE_OK
    assert L.moe_forward(C.byref(p0), None, None, None, None, None, None, 0, None, None) == moe.MOE_OK


def test_chunked_workspace_holds_one_chunk():
    wl = WORKLOADS["dsv3_bf16"]
    full = moe.workspace_layout(_prob(wl))
    p = _prob(wl)
    p.chunk_tokens = 512
    ch = moe.workspace_layout(p)
    assert ch.perm_len == 512 * wl.topk and ch.act_rows == 512 * wl.topk
    assert ch.total_bytes < full.total_bytes
    # the batch-wide regions keep their size: the pair -> slot map (read by the
    # combine) and the (M, topk, K) expert output
    assert ch.act - ch.inv == full.act - full.inv
    assert ch.shared_act - ch.fused_out == full.shared_act - full.fused_out
    assert moe.validate(p) == moe.MOE_OK


def test_down_gemm_k_split_layout():
    # few experts and wide K in bf16 (the Mixtral shape): the streaming down
    # GEMM splits K in two and the workspace holds both fp32 partial slices
    wl = WORKLOADS["mixtral_bf16"]
    L = moe.workspace_layout(_prob(wl))
    assert L.down_split == 2
    assert L.down_partial % 256 == 0 and L.down_partial >= L.shared_act
    assert L.total_bytes >= L.down_partial + 2 * L.perm_len * wl.K * 4
    # many experts (DeepSeek-V3 shape), fp8 weights, or rows past one
    # streaming tile: no split and no partial slices
    for name in ("dsv3_bf16", "decode_fp8_m256", "skewed_bf16"):
        L = moe.workspace_layout(_prob(WORKLOADS[name]))
        assert L.down_split == 1 and L.total_bytes <= L.down_partial + 256
    # a chunked call reserves the split of one chunk
    p = _prob(wl)
    p.chunk_tokens = 128
    ch = moe.workspace_layout(p)
    assert ch.down_split in (1, 2)
    if ch.down_split == 2:
        assert ch.total_bytes >= ch.down_partial + 2 * ch.perm_len * wl.K * 4


def test_noalloc_forward_rejects_problems_beyond_its_scratch():
    """moe_forward_noalloc checks the problem's workspace against the static
    array on the host, before any launch or pointer use."""
    L = moe.load_library()
    wl = WORKLOADS["skewed_bf16"]
    p = moe.make_problem(wl.E, wl.M, 2 * wl.I, wl.K, wl.topk)
    assert moe.workspace_size(p) > moe.STATIC_SCRATCH_BYTES
    w = moe.Weights()
    assert L.moe_forward_noalloc(C.byref(p), None, None, C.byref(w), None, None, None, None, None) == \
        moe.MOE_ERR_WORKSPACE
    small = moe.make_problem(8, 64, 256, 256, 2, act_dtype=moe.DTYPE_F32, w_dtype=moe.DTYPE_F32)
    assert moe.workspace_size(small) <= moe.STATIC_SCRATCH_BYTES
    # within the limit, the usual argument checks apply (null inputs)
    assert L.moe_forward_noalloc(C.byref(small), None, None, C.byref(w), None, None, None, None, None) == \
        moe.MOE_ERR_INVALID_ARG


def test_dbo_forward_host_checks():
    """moe_forward_dbo refuses, before any launch: one workspace for both
    microbatches, a workspace smaller than a microbatch's, chunking, and
    missing events."""
    L = moe.load_library()
    p = moe.make_problem(8, 64, 256, 256, 2, act_dtype=moe.DTYPE_F32, w_dtype=moe.DTYPE_F32)
    q = moe.dbo_microbatch_problem(p)
    assert q.M == 32 and p.M == 64
    need = moe.workspace_size(q)
    assert need < moe.workspace_size(p)
    w = moe.Weights(1, None, 2, None)
    ev = moe.DboEventsStruct((C.c_void_p * 2)(1, 2), (C.c_void_p * 2)(3, 4), (C.c_void_p * 2)(5, 6))
    args = lambda ws0, ws1, n, e: (C.byref(p), 8, 16, C.byref(w), 24, None, ws0, ws1, n, None, None, e)
    assert L.moe_forward_dbo(*args(4096, 4096, need, C.byref(ev))) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_forward_dbo(*args(4096, 8192, need - 1, C.byref(ev))) == moe.MOE_ERR_WORKSPACE
    assert L.moe_forward_dbo(*args(4096, 8192, need, None)) == moe.MOE_ERR_INVALID_ARG
    pc = moe.Problem.from_buffer_copy(p)
    pc.chunk_tokens = 16
    assert L.moe_forward_dbo(C.byref(pc), 8, 16, C.byref(w), 24, None, 4096, 8192, need, None, None,
                             C.byref(ev)) == moe.MOE_ERR_UNSUPPORTED
