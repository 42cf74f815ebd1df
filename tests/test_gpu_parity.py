"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Integer results (routing ids, counts, offsets, permutation, batched slots, fp8
codes and scales of the first quantisation) must match bit for bit; float
outputs within the bounds of tests/gpu_util.TOL.  Small shapes compare every
element and span several tiles with ragged tails; full workload sizes compare
every routing / permutation entry and a seeded sample of output rows.
"""
import numpy as np
import pytest
import torch

import combine_topk_softmax_amd as moe
import oracle
from tests import gpu_util as U
from workloads import (DTYPE_BF16, DTYPE_F32, DTYPE_FP8, FORMAT_BATCHED, FORMAT_STANDARD, QUANT_FP8_G128,
                       SCORING_SIGMOID, WORKLOADS, make_inputs, make_logits, sample_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- router

ROUTE_CASES = [(n, None) for n in WORKLOADS] + [
    ("ties", dict(M=333, E=16, topk=4)), ("k_equals_E", dict(M=77, E=8, topk=8)),
    ("E1", dict(M=5, E=1, topk=1)), ("E1024", dict(M=65, E=1024, topk=6)),
    ("E200_sigmoid", dict(M=129, E=200, topk=8, scoring=SCORING_SIGMOID, renormalize=True)),
]


@pytest.mark.parametrize("name,over", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_parity(name, over):
    wl = WORKLOADS.get(name, WORKLOADS["tiny_fp32"])
    if over:
        wl = wl.replace(**over)
    logits = make_logits(wl, seed=11)
    if name == "ties":
        logits = torch.round(logits * 2) / 2       # many exact ties
        logits[0, :] = -0.0
        logits[0, 3] = 0.0
    p = U.problem(wl)
    lg = logits.cuda()
    w = torch.empty(wl.M, wl.topk, device="cuda")
    ids = torch.empty(wl.M, wl.topk, dtype=torch.int32, device="cuda")
    moe.moe_route(p, lg, w, ids)
    torch.cuda.synchronize()
    rids, rw = oracle.route(logits, wl.topk, wl.scoring, wl.renormalize)
    np.testing.assert_array_equal(ids.cpu().numpy(), rids)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=U.WEIGHT_RTOL, atol=1e-7)


# ---------------------------------------------------------------- prepare

def _ids_from_oracle(wl, seed=12):
    ids, w = oracle.route(make_logits(wl, seed=seed), wl.topk, wl.scoring, wl.renormalize)
    return ids, w


STD_CASES = [("tiny_fp32", 1), ("mixtral_bf16", 1), ("dsv3_bf16", 1), ("skewed_bf16", 1),
             ("tiny_fp32", 16), ("dsv3_bf16", 128), ("skewed_bf16", 7)]


@pytest.mark.parametrize("name,align", STD_CASES)
def test_prepare_standard_parity(name, align):
    wl = WORKLOADS[name]
    ids, _ = _ids_from_oracle(wl)
    p = U.problem(wl, align=align)
    L = moe.workspace_layout(p)
    ws = moe.empty_workspace(p)
    ws.fill_(0xAB)                                      # poison
    counts = torch.empty(wl.E, dtype=torch.int32, device="cuda")
    x = torch.zeros(wl.M, wl.K, dtype=U.torch_act_dtype(wl), device="cuda")
    moe.moe_prepare(p, x, torch.from_numpy(ids).cuda(), None, None, counts, ws)
    torch.cuda.synchronize()
    rc, roff, rperm, rinv = oracle.permute_standard(ids, wl.E, align)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc)
    np.testing.assert_array_equal(U.ws_view(ws, L.counts, wl.E).cpu().numpy(), rc)
    np.testing.assert_array_equal(U.ws_view(ws, L.offsets, wl.E + 1).cpu().numpy(), roff)
    np.testing.assert_array_equal(U.ws_view(ws, L.perm, L.perm_len).cpu().numpy(), rperm)
    np.testing.assert_array_equal(U.ws_view(ws, L.inv, wl.M * wl.topk).cpu().numpy(), rinv)
    assert U.ws_view(ws, L.status, 1).item() == 0


BATCH_CASES = ["decode_fp8_m64", "decode_fp8_m256", "bf16_batched", "fp8_overflow"]


def _batched_wl(name):
    if name == "bf16_batched":
        return WORKLOADS["dsv3_bf16"].replace(M=300, K=512, I=256, E=16, topk=4, format=FORMAT_BATCHED,
                                               capacity=300, shared_I=0)
    if name == "fp8_overflow":
        return WORKLOADS["decode_fp8_m64"].replace(M=200, K=256, I=256, capacity=40)
    return WORKLOADS[name]


@pytest.mark.parametrize("name", BATCH_CASES)
def test_prepare_batched_parity(name):
    wl = _batched_wl(name)
    ids, _ = _ids_from_oracle(wl)
    d = make_inputs(wl.replace(E=1, I=128), seed=13, device="cpu")   # only x is used
    x = d["x"]
    p = U.problem(wl)
    L = moe.workspace_layout(p)
    ws = moe.empty_workspace(p)
    fp8 = wl.act_quant == QUANT_FP8_G128
    cap, E, K = wl.capacity, wl.E, wl.K
    a_out = torch.full((E, cap, K), 0x7F if fp8 else 0, dtype=torch.uint8 if fp8 else U.torch_act_dtype(wl),
                       device="cuda")
    a_scale = torch.full((E, cap, K // 128), -1.0, device="cuda") if fp8 else None
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    moe.moe_prepare(p, x.cuda(), torch.from_numpy(ids).cuda(), a_out, a_scale, counts, ws)
    torch.cuda.synchronize()
    rc, rinv = oracle.permute_batched(ids, E, cap)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc)
    np.testing.assert_array_equal(U.ws_view(ws, L.inv, wl.M * wl.topk).cpu().numpy(), rinv)
    status = U.ws_view(ws, L.status, 1).item()
    assert status == (moe.DEVICE_CAPACITY_OVERFLOW if (rc > cap).any() else 0)
    a_cpu = a_out.cpu().reshape(E * cap, K)
    flat = np.arange(wl.M * wl.topk)
    kept = rinv >= 0
    rows, toks = rinv[kept], flat[kept] // wl.topk
    if fp8:
        q, s = oracle.quant_g128(x.float().numpy())
        np.testing.assert_array_equal(a_cpu.numpy()[rows], q[toks])
        np.testing.assert_array_equal(a_scale.cpu().reshape(E * cap, K // 128).numpy()[rows], s[toks])
    else:
        np.testing.assert_array_equal(a_cpu.float().numpy()[rows], x.float().numpy()[toks])


def _e4m3_rounding_edges() -> np.ndarray:
    """Every positive e4m3 value (codes 1..0x7e) and every midpoint between
    consecutive ones: the normal midpoints have 4 significant bits and the
    subnormal ones are odd multiples of 2^-10, so all are exact in bf16."""
    vals = oracle.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    return np.concatenate([vals, mids, [vals[0] / 2]])


def test_fp8_quantiser_rounding_edges():
    """The token-group-128 quantiser at its rounding edges, bit for bit against
    the oracle: groups whose scale is exactly 1 or 2^-3 (amax 448 and 56), so
    that x / scale lands on every e4m3 value and every tie between two (ties go
    to the even code, subnormals included), with both signs; a group at a
    scale that is not a power of two; a group of zeros (scale from the 1e-10
    floor); and tiny values (per-token-group quantisation, modular_kernel.py
    page, and the worst-tokens page's batched rows)."""
    wl = WORKLOADS["decode_fp8_m64"].replace(M=64, K=512, I=128, E=4, topk=1, capacity=64)
    edges = _e4m3_rounding_edges()
    rng = np.random.default_rng(5)
    x = np.zeros((wl.M, wl.K), np.float32)
    for m in range(wl.M):
        sel = rng.permutation(edges.size)[:127]
        sign = np.where(rng.random(127) < 0.5, -1.0, 1.0)
        x[m, 0:127] = edges[sel] * sign                        # group 0: scale 1
        x[m, 127] = 448.0
        x[m, 128:255] = edges[sel] * sign / 8.0                # group 1: scale 2^-3
        x[m, 255] = -56.0
        x[m, 256:384] = rng.standard_normal(128) * 37.0        # group 2: any scale
        if m % 2 == 0:
            x[m, 384:512] = 0.0                                # group 3: all zero ...
        else:
            x[m, 384:512] = rng.standard_normal(128) * 1e-5    # ... or tiny
    xb = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(xb.float().numpy()[:, :256], x[:, :256])   # the edges are exact in bf16
    ids, _ = _ids_from_oracle(wl)
    p = U.problem(wl)
    L = moe.workspace_layout(p)
    ws = moe.empty_workspace(p)
    cap, E, K = wl.capacity, wl.E, wl.K
    a_out = torch.full((E, cap, K), 0x7F, dtype=torch.uint8, device="cuda")
    a_scale = torch.full((E, cap, K // 128), -1.0, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    print(f"  fp8 quantiser edges: M={wl.M} K={K}", flush=True)
    moe.moe_prepare(p, xb.cuda(), torch.from_numpy(ids).cuda(), a_out, a_scale, counts, ws)
    torch.cuda.synchronize()
    rinv = U.ws_view(ws, L.inv, wl.M * wl.topk).cpu().numpy()
    kept = rinv >= 0
    assert kept.all()
    rows, toks = rinv, np.arange(wl.M * wl.topk) // wl.topk
    q, sc = oracle.quant_g128(xb.float().numpy())
    assert (sc[:, 0] == 1.0).all() and (sc[:, 1] == 0.125).all()
    np.testing.assert_array_equal(a_out.cpu().reshape(E * cap, K).numpy()[rows], q[toks])
    np.testing.assert_array_equal(a_scale.cpu().reshape(E * cap, K // 128).numpy()[rows], sc[toks])


def test_prepare_flags_bad_ids():
    wl = WORKLOADS["tiny_fp32"]
    ids, _ = _ids_from_oracle(wl)
    ids[3, 1] = wl.E          # out of range
    ids[10, 0] = -5
    p = U.problem(wl)
    L = moe.workspace_layout(p)
    ws = moe.empty_workspace(p)
    counts = torch.empty(wl.E, dtype=torch.int32, device="cuda")
    x = torch.zeros(wl.M, wl.K, device="cuda")
    moe.moe_prepare(p, x, torch.from_numpy(ids).cuda(), None, None, counts, ws)
    torch.cuda.synchronize()
    assert U.ws_view(ws, L.status, 1).item() & moe.DEVICE_BAD_EXPERT_ID
    inv = U.ws_view(ws, L.inv, wl.M * wl.topk).cpu().numpy()
    assert inv[3 * wl.topk + 1] == -1 and inv[10 * wl.topk] == -1
    good = (ids >= 0) & (ids < wl.E)
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(ids[good], minlength=wl.E))


# ---------------------------------------------------------------- experts

SMALL = {
    "tiny_fp32": WORKLOADS["tiny_fp32"],
    "bf16_ragged": WORKLOADS["mixtral_bf16"].replace(M=300, K=384, I=192, E=7, topk=3, renormalize=False,
                                                     logits_dist="normal"),
    "bf16_batched": WORKLOADS["mixtral_bf16"].replace(M=150, K=256, I=128, E=5, topk=2, format=FORMAT_BATCHED,
                                                      capacity=150, logits_dist="normal"),
    "fp8_batched": WORKLOADS["decode_fp8_m64"].replace(M=90, K=384, I=256, E=5, topk=2, capacity=90),
    "fp8_standard": WORKLOADS["decode_fp8_m64"].replace(M=90, K=256, I=256, E=6, topk=3,
                                                        format=FORMAT_STANDARD, capacity=0),
    # more rows per expert than one weight-streaming tile: 128 x 256 MFMA tiles,
    # several row tiles per expert plus a ragged last one, 2 column tiles
    "bf16_mfma": WORKLOADS["mixtral_bf16"].replace(M=700, K=512, I=256, E=4, topk=2, renormalize=False,
                                                   logits_dist="normal"),
    "bf16_mfma_batched": WORKLOADS["mixtral_bf16"].replace(M=600, K=256, I=128, E=3, topk=2,
                                                           format=FORMAT_BATCHED, capacity=600,
                                                           logits_dist="normal"),
    # 128 x 256 MFMA tiles past one L2 group of row tiles (16 for the gated,
    # 6 for the down GEMM): about 20 row tiles (a whole gated group and a
    # partial one; three whole down groups and a partial one) x 2 column
    # tiles, and about 33 row tiles (two whole gated groups, five whole down
    # groups, and a partial one of each)
    "bf16_mfma_groups": WORKLOADS["mixtral_bf16"].replace(M=1200, K=512, I=256, E=4, topk=2, renormalize=False,
                                                          logits_dist="normal"),
    "bf16_mfma_18tiles": WORKLOADS["mixtral_bf16"].replace(M=2000, K=256, I=256, E=3, topk=2, renormalize=False,
                                                           logits_dist="normal"),
    "bf16_mfma_zipf": WORKLOADS["skewed_bf16"].replace(M=1500, K=256, I=256, E=16, topk=4),
    # weight streaming with enough (expert, column tile) items that the down
    # GEMM gives each wavefront two 16-row weight blocks
    "bf16_down2": WORKLOADS["mixtral_bf16"].replace(M=256, K=2048, I=128, E=64, topk=4, renormalize=False,
                                                    logits_dist="normal"),
    "fp8_batched_down2": WORKLOADS["decode_fp8_m64"].replace(M=96, K=2048, I=256, E=64, topk=4, capacity=96),
    # fp8 weight streaming with 32-80 rows per expert and at least 256 wide
    # items: wide gated panels (2 gate + 2 up blocks per wavefront, 256 act
    # columns = two quantisation groups per item, row tiles of at most 96
    # rows); the Zipf case puts more than 96 rows on some experts, which then
    # take several row tiles
    "fp8_wide": WORKLOADS["decode_fp8_m64"].replace(M=192, K=256, I=2048, E=32, topk=8, capacity=192),
    "fp8_wide_two_tiles": WORKLOADS["decode_fp8_m64"].replace(M=300, K=256, I=2048, E=32, topk=8, capacity=300,
                                                              logits_dist="zipf"),
    # the same with K a multiple of 512: the down GEMM also takes four weight
    # blocks per wavefront (512 output columns per item)
    "fp8_wide_down4": WORKLOADS["decode_fp8_m64"].replace(M=192, K=512, I=2048, E=32, topk=8, capacity=192),
    # fp8 down GEMM with two-block panels whose last round of items would be
    # part-empty (32 experts x 20 panels = 640 items on 256 compute units):
    # the balanced plan deals each row tile's 40 column units out as 8 items
    # of three blocks per wavefront, then 8 of two; Zipf logits put up to 128
    # rows on some experts (eight 16-row blocks) and none on others, so the
    # device's tile count differs from the plan's expectation
    "fp8_balanced_down": WORKLOADS["decode_fp8_m64"].replace(M=128, K=5120, I=256, E=32, topk=8, capacity=128,
                                                             logits_dist="zipf"),
    # too few experts for a wide item per compute unit (an expert-parallel
    # shard's share): narrow panels
    "fp8_few_experts": WORKLOADS["decode_fp8_m64"].replace(M=96, K=256, I=256, E=4, topk=2, capacity=96),
    # bf16 weight streaming with few experts and wide K: two-block down panels
    # would leave too few work items, so the down GEMM splits K in two and a
    # reduce sums the fp32 partials into the pair rows; the Zipf case puts
    # several row tiles on one expert and none on others
    "bf16_split_k": WORKLOADS["mixtral_bf16"].replace(M=64, K=4096, I=512, E=8, topk=2, renormalize=False,
                                                      logits_dist="normal"),
    "bf16_split_k_zipf": WORKLOADS["mixtral_bf16"].replace(M=200, K=4096, I=512, E=8, topk=2,
                                                           logits_dist="zipf"),
    # bf16 weight streaming with 36 column panels per expert (288 items: one
    # whole round per XCD plus 4 items, which run as two row halves each)
    "bf16_split_tail": WORKLOADS["mixtral_bf16"].replace(M=64, K=256, I=4608, E=8, topk=2, renormalize=False,
                                                         logits_dist="normal"),
    # the same regime with I % 128 != 0: the general 128 x 128 tile kernel
    "bf16_tiled_I192": WORKLOADS["mixtral_bf16"].replace(M=700, K=384, I=192, E=4, topk=2, renormalize=False,
                                                         logits_dist="normal"),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_experts_parity_every_pair(name):
    wl = SMALL[name]
    d = make_inputs(wl, seed=14, device="cpu")
    ids, _ = _ids_from_oracle(wl)
    p = U.problem(wl)
    ws = moe.empty_workspace(p)
    g = U.to_cuda(d)
    counts = torch.empty(wl.E, dtype=torch.int32, device="cuda")
    fp8 = wl.act_quant == QUANT_FP8_G128
    bat = U.batched(wl)
    a_out = a_scale = None
    if bat:
        a_out = torch.empty(wl.E, wl.capacity, wl.K, dtype=torch.uint8 if fp8 else U.torch_act_dtype(wl),
                            device="cuda")
    elif fp8:
        a_out = torch.empty(wl.M, wl.K, dtype=torch.uint8, device="cuda")
    if fp8:
        a_scale = torch.empty(a_out.shape[0] * (a_out.shape[1] if bat else 1), wl.K // 128, device="cuda")
    moe.moe_prepare(p, g["x"], torch.from_numpy(ids).cuda(), a_out, a_scale, counts, ws)
    rows = wl.E * wl.capacity if bat else wl.M * wl.topk
    fused = torch.full((rows, wl.K), float("nan"), dtype=U.torch_act_dtype(wl), device="cuda")
    moe.moe_experts(p, a_out if a_out is not None else g["x"], a_scale, g["w1"], g.get("w1_scale"), g["w2"],
                    g.get("w2_scale"), counts, fused, ws)
    if wl.I % 128 == 0:
        # the packed weight layout reorders bytes only: bitwise the same rows
        pp = U.problem(wl, weight_layout=moe.WEIGHTS_PACKED)
        w1p, w2p = moe.pack_weights(pp, g["w1"], g["w2"])
        fused_p = torch.full_like(fused, float("nan"))
        moe.moe_experts(pp, a_out if a_out is not None else g["x"], a_scale, w1p, g.get("w1_scale"), w2p,
                        g.get("w2_scale"), counts, fused_p, ws)
        torch.cuda.synchronize()
        assert torch.equal(fused_p.view(torch.int16), fused.view(torch.int16))
    torch.cuda.synchronize()
    got = fused.float().cpu().numpy()
    L = moe.workspace_layout(p)
    inv = U.ws_view(ws, L.inv, wl.M * wl.topk).cpu().numpy()
    ref = np.zeros((wl.M * wl.topk, wl.K))
    mine = np.zeros_like(ref)
    for m in range(wl.M):
        a = oracle.input_row(d["x"], m, wl.act_dtype, wl.act_quant)
        for j in range(wl.topk):
            f = m * wl.topk + j
            _, y = oracle.expert_row(a, int(ids[m, j]), d["w1"], d["w2"], wl.w_dtype, wl.I,
                                     d.get("w1_scale"), d.get("w2_scale"), requant_fp8=fp8)
            ref[f] = y
            mine[f] = got[inv[f]] if bat else got[f]
    assert np.all(np.isfinite(mine))
    err = U.rel_err(mine, ref)
    print(f"  {name}: max rel err {err:.3e}", flush=True)
    assert err <= U.tol_for(wl)


@pytest.mark.parametrize("M,K,Is", [(300, 512, 256), (64, 256, 128), (513, 768, 384)])
def test_shared_expert_parity(M, K, Is):
    """The always-on shared expert alone (dense gated MLP over all M tokens),
    with M not a multiple of the row tile."""
    wl = WORKLOADS["dsv3_bf16"].replace(M=M, K=K, I=128, E=4, topk=2, shared_I=Is)
    d = make_inputs(wl, seed=16, device="cpu")
    p = U.problem(wl)
    ws = moe.empty_workspace(p)
    g = U.to_cuda(d)
    out = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_shared_expert(p, g["x"], g["w1s"], g["w2s"], out, ws)
    torch.cuda.synchronize()
    toks = list(range(M))
    ref = oracle.dense_mlp_tokens(d["x"], d["w1s"], d["w2s"], Is, wl.act_dtype, toks)
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    err = U.rel_err(got, ref)
    print(f"  shared M={M} K={K} Is={Is}: max rel err {err:.3e}", flush=True)
    assert err <= U.tol_for(wl)


@pytest.mark.parametrize("name", ["fp8_batched", "fp8_standard", "fp8_wide"])
def test_act_requant_group_invariants(name):
    """fp8: the gated GEMM writes act as e4m3 codes with one scale per row and
    128 columns, the scale being the group's max magnitude / 448.  So every
    group of a real row holds a code of magnitude exactly 448 and no larger
    one, and every scale is positive."""
    wl = SMALL[name]
    d = make_inputs(wl, seed=17, device="cpu")
    ids, _ = _ids_from_oracle(wl)
    p = U.problem(wl)
    ws = moe.empty_workspace(p)
    g = U.to_cuda(d)
    counts = torch.empty(wl.E, dtype=torch.int32, device="cuda")
    bat = U.batched(wl)
    rows_a = wl.E * wl.capacity if bat else wl.M
    a_out = torch.empty(*((wl.E, wl.capacity) if bat else (wl.M,)), wl.K, dtype=torch.uint8, device="cuda")
    a_scale = torch.empty(rows_a, wl.K // 128, device="cuda")
    moe.moe_prepare(p, g["x"], torch.from_numpy(ids).cuda(), a_out, a_scale, counts, ws)
    rows = wl.E * wl.capacity if bat else wl.M * wl.topk
    fused = torch.empty(rows, wl.K, dtype=torch.bfloat16, device="cuda")
    moe.moe_experts(p, a_out, a_scale, g["w1"], g["w1_scale"], g["w2"], g["w2_scale"], counts, fused, ws)
    torch.cuda.synchronize()
    L = moe.workspace_layout(p)
    G = wl.I // 128
    codes = U.ws_view(ws, L.act_q, L.act_rows * wl.I, torch.uint8).cpu().numpy().reshape(L.act_rows, G, 128)
    scales = U.ws_view(ws, L.act_scale, L.act_rows * G, torch.float32).cpu().numpy().reshape(L.act_rows, G)
    c = counts.cpu().numpy()
    if bat:
        real = np.concatenate([e * wl.capacity + np.arange(c[e]) for e in range(wl.E)])
    else:
        real = np.arange(wl.M * wl.topk)       # every slot of the permutation is a real pair (align 1)
    mags = np.abs(oracle.e4m3_decode(codes[real].ravel()).reshape(len(real), G, 128))
    assert len(real) > 0
    np.testing.assert_array_equal(mags.max(axis=2), 448.0)
    assert np.all(scales[real] > 0)


def test_finalize_parity():
    for wl, bat in ((WORKLOADS["tiny_fp32"], False), (SMALL["bf16_ragged"], False), (SMALL["fp8_batched"], True)):
        gen = torch.Generator().manual_seed(15)
        p = U.problem(wl)
        ws = moe.empty_workspace(p)
        ids, w = _ids_from_oracle(wl)
        rows = wl.E * wl.capacity if bat else wl.M * wl.topk
        y = torch.randn(rows, wl.K, generator=gen).to(U.torch_act_dtype(wl))
        # the combine reads the pair -> row map that prepare leaves in the workspace
        counts = torch.empty(wl.E, dtype=torch.int32, device="cuda")
        x = torch.zeros(wl.M, wl.K, dtype=U.torch_act_dtype(wl), device="cuda")
        if bat:
            a_out = torch.empty(wl.E, wl.capacity, wl.K, dtype=torch.uint8, device="cuda")
            a_s = torch.empty(wl.E * wl.capacity, wl.K // 128, device="cuda")
            moe.moe_prepare(p, x, torch.from_numpy(ids).cuda(), a_out, a_s, counts, ws)
            _, inv = oracle.permute_batched(ids, wl.E, wl.capacity)
            ypairs = y.float().numpy()[np.maximum(inv, 0)]
            keep = (inv >= 0).astype(np.int32)
        else:
            moe.moe_prepare(p, x, torch.from_numpy(ids).cuda(), None, None, counts, ws)
            ypairs, keep = y.float().numpy(), None
        out = torch.empty(wl.M, wl.K, dtype=U.torch_act_dtype(wl), device="cuda")
        wt = torch.from_numpy(w.astype(np.float32))
        moe.moe_finalize(p, y.cuda(), wt.cuda(), out, ws)
        torch.cuda.synchronize()
        ref = oracle.combine(wt.double().numpy(), ypairs.reshape(wl.M, wl.topk, wl.K), keep)
        assert U.rel_err(out.float().cpu().numpy(), ref) <= U.tol_for(wl)


def test_finalize_ignores_bad_id_pairs():
    """A pick with an out-of-range expert id is flagged by prepare and adds
    nothing in finalize: its row of the expert output (left NaN here, as the
    experts step never writes it) is not read."""
    wl = SMALL["bf16_ragged"]
    d = U.to_cuda(make_inputs(wl, seed=24, device="cpu"))
    p = U.problem(wl)
    ws = moe.empty_workspace(p)
    w = torch.empty(wl.M, wl.topk, device="cuda")
    ids = torch.empty(wl.M, wl.topk, dtype=torch.int32, device="cuda")
    moe.moe_route(p, d["logits"], w, ids)
    bad = [(3, 1), (wl.M - 1, 0)]
    ids[3, 1] = wl.E
    ids[wl.M - 1, 0] = -7
    counts = torch.empty(wl.E, dtype=torch.int32, device="cuda")
    moe.moe_prepare(p, d["x"], ids, None, None, counts, ws)
    fused = torch.full((wl.M * wl.topk, wl.K), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_experts(p, d["x"], None, d["w1"], None, d["w2"], None, counts, fused, ws)
    out = torch.empty(wl.M, wl.K, dtype=torch.bfloat16, device="cuda")
    moe.moe_finalize(p, fused, w, out, ws)
    torch.cuda.synchronize()
    L = moe.workspace_layout(p)
    assert U.ws_view(ws, L.status, 1).item() & moe.DEVICE_BAD_EXPERT_ID
    keep = np.ones((wl.M, wl.topk), np.int32)
    for m, j in bad:
        keep[m, j] = 0
    y = fused.float().cpu().numpy().reshape(wl.M, wl.topk, wl.K)
    assert np.isnan(y[keep == 0]).all() and np.isfinite(y[keep == 1]).all()
    ref = oracle.combine(w.cpu().double().numpy(), np.where(keep[..., None] == 1, y, 0.0), keep)
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    assert U.rel_err(got, ref) <= U.tol_for(wl)


# ---------------------------------------------------------------- whole layer

FULL = list(WORKLOADS)
# token rows whose whole layer output the full-size test compares (all of
# them where the oracle finishes in seconds); the larger workloads compare a
# sample of tokens plus expert-output rows covering every 32-row block of every
# expert segment (below)
FULL_ALL_TOKENS = {"tiny_fp32", "mixtral_bf16", "decode_fp8_m64", "decode_fp8_m256"}


def _segment_block_pairs(counts, offsets, perm, block=32, seed=0):
    """One pair from every `block`-row block of every expert's segment of the
    Standard permutation, plus each segment's last row: every row tile of any
    grouped-GEMM tiling by multiples of `block` (and every column tile of it,
    as each row is compared in full) holds a checked pair."""
    rng = np.random.default_rng(seed)
    picks = set()
    for e in range(len(counts)):
        c, base = int(counts[e]), int(offsets[e])
        for b0 in range(0, c, block):
            picks.add(base + b0 + int(rng.integers(min(block, c - b0))))
        if c:
            picks.add(base + c - 1)
    return sorted(int(perm[s]) for s in picks)


def _check_pair_rows(wl, d, ws, L, rids, pairs):
    """Unweighted expert output rows (M, k, K) that moe_forward left in its
    workspace, against the oracle's expert MLP of each pair."""
    fused = U.ws_view(ws, L.fused_out, wl.M * wl.topk * wl.K, torch.bfloat16)
    got = fused.view(wl.M * wl.topk, wl.K)[torch.tensor(pairs, device="cuda")].float().cpu().numpy()
    x, w1, w2 = (oracle.host_array(d[k]) for k in ("x", "w1", "w2"))
    ref = np.empty_like(got, dtype=np.float64)
    last_m, a = -1, None
    for i, f in enumerate(pairs):
        m, j = divmod(f, wl.topk)
        if m != last_m:
            a, last_m = oracle.input_row(x, m, wl.act_dtype), m
        _, ref[i] = oracle.expert_row(a, int(rids[m, j]), w1, w2, wl.w_dtype, wl.I)
    assert np.all(np.isfinite(got))
    return U.rel_err(got, ref)


@pytest.mark.parametrize("name", FULL)
def test_forward_parity_full_size(name):
    """Every workload at full size, in the launch configuration the benchmark
    times (packed expert weights where the shape allows)."""
    wl = WORKLOADS[name]
    small = wl.M * wl.K * wl.I * wl.E < 2 ** 28
    d = make_inputs(wl, seed=0, device="cpu" if small else "cuda")
    g = U.to_cuda(d)
    p = None
    if wl.I % 128 == 0:
        p = U.problem(wl, weight_layout=moe.WEIGHTS_PACKED)
        g["w1"], g["w2"] = moe.pack_weights(p, g["w1"], g["w2"])
    out, sout, ws, p = U.run_forward(wl, g, p=p)
    torch.cuda.synchronize()
    del g
    L = moe.workspace_layout(p)
    # every routing / counting / permutation entry
    rids, rw = oracle.route(d["logits"], wl.topk, wl.scoring, wl.renormalize)
    np.testing.assert_array_equal(U.ws_view(ws, L.topk_ids, wl.M * wl.topk).cpu().numpy().reshape(wl.M, -1), rids)
    tw = U.ws_view(ws, L.topk_weights, wl.M * wl.topk, torch.float32).cpu().numpy().reshape(wl.M, -1)
    np.testing.assert_allclose(tw, rw, rtol=U.WEIGHT_RTOL, atol=1e-7)
    if U.batched(wl):
        rc, rinv = oracle.permute_batched(rids, wl.E, wl.capacity)
        np.testing.assert_array_equal(U.ws_view(ws, L.inv, wl.M * wl.topk).cpu().numpy(), rinv)
    else:
        rc, roff, rperm, rinv = oracle.permute_standard(rids, wl.E, 1)
        np.testing.assert_array_equal(U.ws_view(ws, L.perm, L.perm_len).cpu().numpy(), rperm)
        np.testing.assert_array_equal(U.ws_view(ws, L.offsets, wl.E + 1).cpu().numpy(), roff)
    np.testing.assert_array_equal(U.ws_view(ws, L.counts, wl.E).cpu().numpy(), rc)
    assert U.ws_view(ws, L.status, 1).item() == 0
    if name not in FULL_ALL_TOKENS:
        # expert-output rows from every 32-row block of every expert segment
        assert not U.batched(wl) and L.down_split == 1
        pairs = _segment_block_pairs(rc, roff, rperm, seed=9)
        perr = _check_pair_rows(wl, d, ws, L, rids, pairs)
        print(f"  {name}: {len(pairs)} expert-output rows, max rel err {perr:.3e}", flush=True)
        assert perr <= U.tol_for(wl)
    toks = list(range(wl.M)) if name in FULL_ALL_TOKENS else sample_tokens(wl.M, 10, seed=1)
    ref, _, _ = oracle.moe_tokens(wl, d, toks)
    got = out.float().cpu().numpy()[toks]
    assert np.all(np.isfinite(got))
    err = U.rel_err(got, ref)
    print(f"  {name}: {len(toks)} token rows, max rel err {err:.3e}", flush=True)
    assert err <= U.tol_for(wl)
    if wl.shared_I:
        sref = oracle.dense_mlp_tokens(d["x"], d["w1s"], d["w2s"], wl.shared_I, wl.act_dtype, toks)
        serr = U.rel_err(sout.float().cpu().numpy()[toks], sref)
        print(f"  {name}: shared expert max rel err {serr:.3e}", flush=True)
        assert serr <= U.tol_for(wl)


# ---------------------------------------------------------------- edge cases

EDGE = {
    "M1": WORKLOADS["mixtral_bf16"].replace(M=1, K=256, I=128, E=8, topk=2),
    "k_eq_E": WORKLOADS["mixtral_bf16"].replace(M=37, K=256, I=128, E=4, topk=4, logits_dist="normal"),
    "E1_k1": WORKLOADS["tiny_fp32"].replace(M=130, E=1, topk=1),
    "fp8_M1": WORKLOADS["decode_fp8_m64"].replace(M=1, K=256, I=128, E=8, capacity=8),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_forward_edge_shapes(name):
    wl = EDGE[name]
    d = make_inputs(wl, seed=16, device="cpu")
    out, _, ws, _ = U.run_forward(wl, U.to_cuda(d))
    torch.cuda.synchronize()
    ref, _, _ = oracle.moe_tokens(wl, d)
    assert U.rel_err(out.float().cpu().numpy(), ref) <= U.tol_for(wl)


def test_forward_empty_batch_is_noop():
    wl = WORKLOADS["tiny_fp32"].replace(M=0)
    p = U.problem(wl)
    out = torch.empty(0, wl.K, device="cuda")
    d = make_inputs(wl.replace(M=1), seed=0, device="cuda")
    moe.moe_forward(p, d["logits"][:0], d["x"][:0], d["w1"], None, d["w2"], None, out,
                    torch.empty(16, dtype=torch.uint8, device="cuda"))


def test_zero_count_expert_nan_weights_change_nothing():
    wl = SMALL["bf16_ragged"]
    d = make_inputs(wl, seed=17, device="cpu")
    d["logits"][:, 2] = -1e4                      # expert 2 never routed
    g = U.to_cuda(d)
    base, _, _, _ = U.run_forward(wl, g)
    g["w1"][2] = float("nan")
    g["w2"][2] = float("nan")
    poisoned, _, ws, p = U.run_forward(wl, g)
    torch.cuda.synchronize()
    assert U.ws_view(ws, moe.workspace_layout(p).counts, wl.E)[2].item() == 0
    assert torch.isfinite(poisoned.float()).all()
    assert torch.equal(base, poisoned)


def test_maximal_skew_all_tokens_same_experts():
    wl = SMALL["bf16_ragged"].replace(M=700)
    d = make_inputs(wl, seed=18, device="cpu")
    d["logits"][:, :wl.topk] += 100.0             # every token picks experts 0..k-1
    out, _, ws, p = U.run_forward(wl, U.to_cuda(d))
    torch.cuda.synchronize()
    counts = U.ws_view(ws, moe.workspace_layout(p).counts, wl.E).cpu().numpy()
    assert counts[:wl.topk].tolist() == [wl.M] * wl.topk and counts[wl.topk:].sum() == 0
    toks = sample_tokens(wl.M, 40, seed=2)
    ref, _, _ = oracle.moe_tokens(wl, d, toks)
    assert U.rel_err(out.float().cpu().numpy()[toks], ref) <= U.tol_for(wl)


def test_batched_capacity_overflow_drops_and_flags():
    wl = SMALL["fp8_batched"].replace(M=120, capacity=20)
    d = make_inputs(wl, seed=19, device="cpu")
    out, _, ws, p = U.run_forward(wl, U.to_cuda(d))
    torch.cuda.synchronize()
    assert U.ws_view(ws, moe.workspace_layout(p).status, 1).item() == moe.DEVICE_CAPACITY_OVERFLOW
    ref, _, _ = oracle.moe_tokens(wl, d)        # the oracle drops the same pairs
    assert U.rel_err(out.float().cpu().numpy(), ref) <= U.tol_for(wl)


def test_standard_and_batched_agree_bitwise():
    wl = SMALL["bf16_ragged"]
    d = U.to_cuda(make_inputs(wl, seed=20, device="cpu"))
    a, _, _, _ = U.run_forward(wl, d)
    b, _, _, _ = U.run_forward(wl.replace(format=FORMAT_BATCHED, capacity=wl.M), d)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_forward_is_deterministic():
    wl = WORKLOADS["dsv3_bf16"].replace(M=512, E=64, I=256, K=512, shared_I=256)
    d = U.to_cuda(make_inputs(wl, seed=21, device="cpu"))
    a, sa, _, _ = U.run_forward(wl, d)
    b, sb, _, _ = U.run_forward(wl, d)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(sa, sb)


def test_stage_calls_equal_forward():
    """route -> prepare -> experts -> finalize through the separate calls
    gives exactly what moe_forward gives (same kernels, same order; with the
    down GEMM split over K, moe_experts reduces the partial sums into the pair
    rows and moe_forward's combine reads them directly, bit for bit the same)."""
    for wl in (SMALL["bf16_ragged"], SMALL["fp8_batched"], SMALL["bf16_split_k"], SMALL["bf16_split_k_zipf"]):
        d = U.to_cuda(make_inputs(wl, seed=22, device="cpu"))
        ref, _, _, p = U.run_forward(wl, d)
        ws = moe.empty_workspace(p)
        w = torch.empty(wl.M, wl.topk, device="cuda")
        ids = torch.empty(wl.M, wl.topk, dtype=torch.int32, device="cuda")
        moe.moe_route(p, d["logits"], w, ids)
        counts = torch.empty(wl.E, dtype=torch.int32, device="cuda")
        fp8 = wl.act_quant == QUANT_FP8_G128
        bat = U.batched(wl)
        a_out = a_s = None
        if bat:
            a_out = torch.empty(wl.E, wl.capacity, wl.K, dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
            if fp8:
                a_s = torch.empty(wl.E * wl.capacity, wl.K // 128, device="cuda")
        moe.moe_prepare(p, d["x"], ids, a_out, a_s, counts, ws)
        rows = wl.E * wl.capacity if bat else wl.M * wl.topk
        fused = torch.empty(rows, wl.K, dtype=torch.bfloat16, device="cuda")
        moe.moe_experts(p, a_out if bat else d["x"], a_s, d["w1"], d.get("w1_scale"), d["w2"], d.get("w2_scale"),
                        counts, fused, ws)
        out = torch.empty_like(ref)
        moe.moe_finalize(p, fused, w, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


def test_graph_replay_matches_eager():
    """Capture the whole layer (with the shared expert on its aux stream) in one
    graph; replay it with fresh inputs copied into the captured buffers and
    compare every replay with an eager run on the same inputs."""
    wl = WORKLOADS["dsv3_bf16"].replace(M=256, E=32, I=256, K=512, shared_I=256)
    d = U.to_cuda(make_inputs(wl, seed=23, device="cpu"))
    p = U.problem(wl)
    ws = moe.empty_workspace(p)
    out = torch.empty(wl.M, wl.K, dtype=torch.bfloat16, device="cuda")
    sout = torch.empty_like(out)
    streams = moe.SharedExpertStreams()
    U.run_forward(wl, d, ws=ws, p=p, out=out, shared_out=sout, streams=streams)   # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            moe.moe_forward(p, d["logits"], d["x"], d["w1"], None, d["w2"], None, out, ws,
                            shared=(d["w1s"], d["w2s"], sout), shared_streams=streams)
    torch.cuda.synchronize()
    ews = moe.empty_workspace(p)
    for it in range(5):
        fresh = make_inputs(wl, seed=100 + it, device="cpu")
        d["logits"].copy_(fresh["logits"].cuda())
        d["x"].copy_(fresh["x"].cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e_out, e_sout, _, _ = U.run_forward(wl, d, ws=ews, p=p)
        torch.cuda.synchronize()
        assert torch.equal(out, e_out), it
        assert torch.equal(sout, e_sout), it


def test_graph_replay_split_paths():
    """The same for a layer whose gated GEMM runs its items as row halves (fewer
    than half a round of items) and whose down GEMM splits K into fp32 partial
    sums and a reduce: every replay bitwise equal to an eager run."""
    wl = SMALL["bf16_split_k"]
    d = U.to_cuda(make_inputs(wl, seed=24, device="cpu"))
    p = U.problem(wl)
    assert moe.workspace_layout(p).down_split == 2
    ws = moe.empty_workspace(p)
    out = torch.empty(wl.M, wl.K, dtype=torch.bfloat16, device="cuda")
    U.run_forward(wl, d, ws=ws, p=p, out=out)   # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            moe.moe_forward(p, d["logits"], d["x"], d["w1"], None, d["w2"], None, out, ws)
    torch.cuda.synchronize()
    ews = moe.empty_workspace(p)
    for it in range(3):
        fresh = make_inputs(wl, seed=200 + it, device="cpu")
        d["logits"].copy_(fresh["logits"].cuda())
        d["x"].copy_(fresh["x"].cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e_out, _, _, _ = U.run_forward(wl, d, ws=ews, p=p)
        torch.cuda.synchronize()
        assert torch.equal(out, e_out), it


# ---------------------------------------------------------------- packed weights

PACK_CASES = {
    "bf16_stream": WORKLOADS["mixtral_bf16"].replace(M=300, K=384, I=256, E=7, topk=3, renormalize=False,
                                                     logits_dist="normal"),
    "bf16_tiled": WORKLOADS["mixtral_bf16"].replace(M=1200, K=256, I=256, E=4, topk=2, renormalize=False,
                                                    logits_dist="normal"),
    "fp8_batched_stream": SMALL["fp8_batched"],
    "fp8_standard_stream": SMALL["fp8_standard"],
    "fp32_tiled": WORKLOADS["tiny_fp32"],
}


@pytest.mark.parametrize("name", list(PACK_CASES))
def test_packed_weights_give_identical_results(name):
    """The packed layout only moves bytes: the layer's output is bitwise the same."""
    wl = PACK_CASES[name]
    d = U.to_cuda(make_inputs(wl, seed=24, device="cpu"))
    ref, _, _, p = U.run_forward(wl, d)
    pp = U.problem(wl, weight_layout=moe.WEIGHTS_PACKED)
    w1p, w2p = moe.pack_weights(pp, d["w1"], d["w2"])
    torch.cuda.synchronize()
    # packing permutes bytes within each tensor
    for a, b in ((d["w1"], w1p), (d["w2"], w2p)):
        va, vb = a.view(torch.uint8).flatten(), b.view(torch.uint8).flatten()
        assert torch.equal(torch.bincount(va.long(), minlength=256), torch.bincount(vb.long(), minlength=256))
        assert not torch.equal(va, vb) or va.numel() <= 16
    dp = dict(d, w1=w1p, w2=w2p)
    got, _, _, _ = U.run_forward(wl, dp, p=pp)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


@pytest.mark.parametrize("name", ["mixtral_bf16", "dsv3_bf16", "decode_fp8_m64", "decode_fp8_m256", "skewed_bf16"])
def test_packed_weights_full_size(name):
    """The configuration the benchmark times (packed weights, full size):
    bitwise equal to the row-major run and within the bar of the oracle."""
    wl = WORKLOADS[name]
    d = make_inputs(wl, seed=0, device="cuda")
    ref, sref, _, _ = U.run_forward(wl, d)
    pp = U.problem(wl, weight_layout=moe.WEIGHTS_PACKED)
    w1p, w2p = moe.pack_weights(pp, d["w1"], d["w2"])
    got, sgot, _, _ = U.run_forward(wl, dict(d, w1=w1p, w2=w2p), p=pp)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    del w1p, w2p
    toks = sample_tokens(wl.M, 6, seed=3)
    oref, _, _ = oracle.moe_tokens(wl, d, toks)
    err = U.rel_err(got.float().cpu().numpy()[toks], oref)
    print(f"  {name} packed: max rel err {err:.3e}", flush=True)
    assert err <= U.tol_for(wl)


# ----------------------------------------- GELU, expert-parallel shard, router weight on input

GELU_CASES = {
    "f32_tiled": WORKLOADS["tiny_fp32"].replace(activation=1),
    "bf16_stream": WORKLOADS["mixtral_bf16"].replace(M=300, K=384, I=256, E=7, topk=3, renormalize=False,
                                                     logits_dist="normal", activation=1),
    "bf16_mfma_shared": WORKLOADS["dsv3_bf16"].replace(M=520, K=512, I=256, E=4, topk=2, shared_I=256,
                                                       activation=1),
    "fp8_batched": WORKLOADS["decode_fp8_m64"].replace(M=90, K=384, I=256, E=5, topk=2, capacity=90,
                                                       activation=1),
}


@pytest.mark.parametrize("name", list(GELU_CASES))
def test_gelu_forward_parity(name):
    """gelu_and_mul in every gated epilogue (tiled, streaming with fp8
    re-quantisation, 128x256 MFMA, shared expert)."""
    wl = GELU_CASES[name]
    d = make_inputs(wl, seed=31, device="cpu")
    out, sout, _, _ = U.run_forward(wl, U.to_cuda(d))
    torch.cuda.synchronize()
    toks = sample_tokens(wl.M, 24, seed=5)
    ref, _, _ = oracle.moe_tokens(wl, d, toks)
    err = U.rel_err(out.float().cpu().numpy()[toks], ref)
    print(f"  gelu {name}: max rel err {err:.3e}", flush=True)
    assert err <= U.tol_for(wl)
    if wl.shared_I:
        sref = oracle.dense_mlp_tokens(d["x"], d["w1s"], d["w2s"], wl.shared_I, wl.act_dtype, toks,
                                       activation=1)
        serr = U.rel_err(sout.float().cpu().numpy()[toks], sref)
        print(f"  gelu {name} shared: max rel err {serr:.3e}", flush=True)
        assert serr <= U.tol_for(wl)


SHARD_CASES = {
    "bf16_standard": WORKLOADS["mixtral_bf16"].replace(M=200, K=384, I=256, E=12, topk=3, renormalize=True,
                                                       logits_dist="normal"),
    "bf16_batched": WORKLOADS["mixtral_bf16"].replace(M=150, K=256, I=128, E=12, topk=2, format=FORMAT_BATCHED,
                                                      capacity=150, logits_dist="normal"),
    "fp8_batched": WORKLOADS["decode_fp8_m64"].replace(M=80, K=256, I=256, E=12, topk=4, capacity=80),
    # few experts and wide K (8 local of 24): the unsharded layer and every
    # shard split the down GEMM over K, and a shard's permutation holds only
    # its own picks
    "bf16_split_k": WORKLOADS["mixtral_bf16"].replace(M=96, K=4096, I=512, E=24, topk=2, renormalize=True,
                                                      logits_dist="normal"),
}


def _shard_inputs(d, Eg, n_shards, s):
    """Shard s of n: global experts g with g % n == s, local index g // n."""
    glob = torch.arange(Eg)[torch.arange(Eg) % n_shards == s]
    emap = torch.full((Eg,), -1, dtype=torch.int32)
    emap[glob] = torch.arange(glob.numel(), dtype=torch.int32)
    out = dict(d, w1=d["w1"][glob].contiguous(), w2=d["w2"][glob].contiguous(), expert_map=emap)
    for k in ("w1_scale", "w2_scale"):
        if d.get(k) is not None:
            out[k] = d[k][glob].contiguous()
    return out, glob.numel()


@pytest.mark.parametrize("name", list(SHARD_CASES))
def test_expert_parallel_shards(name):
    """Three expert-parallel shards (expert_map): each matches the oracle's
    shard; the routing ids are global; the shards' outputs sum to the
    unsharded layer's."""
    wl = SHARD_CASES[name]
    Eg = wl.E
    d = make_inputs(wl, seed=32, device="cpu")
    full, _, fws, _ = U.run_forward(wl, U.to_cuda(d))
    torch.cuda.synchronize()
    total = torch.zeros_like(full, dtype=torch.float32)
    toks = sample_tokens(wl.M, 20, seed=6)
    for s in range(3):
        ds, El = _shard_inputs(d, Eg, 3, s)
        wls = wl.replace(E=El, global_E=Eg)
        out, _, ws, p = U.run_forward(wls, U.to_cuda(ds))
        torch.cuda.synchronize()
        L = moe.workspace_layout(p)
        if name == "bf16_split_k":
            assert L.down_split == 2
        ids = U.ws_view(ws, L.topk_ids, wl.M * wl.topk).cpu().numpy()
        fids = U.ws_view(fws, moe.workspace_layout(U.problem(wl)).topk_ids, wl.M * wl.topk).cpu().numpy()
        np.testing.assert_array_equal(ids, fids)
        counts = U.ws_view(ws, L.counts, El).cpu().numpy()
        local = ds["expert_map"].numpy()[ids]
        np.testing.assert_array_equal(counts, np.bincount(local[local >= 0], minlength=El))
        assert (U.ws_view(ws, L.status, 1).item() & moe.DEVICE_BAD_EXPERT_ID) == 0
        ref, _, _ = oracle.moe_tokens(wls, ds, toks)
        err = U.rel_err(out.float().cpu().numpy()[toks], ref)
        print(f"  shard {name} {s}: max rel err {err:.3e}", flush=True)
        assert err <= U.tol_for(wl)
        total += out.float()
    err = U.rel_err(total.cpu().numpy(), full.float().cpu().numpy())
    print(f"  shards {name} sum vs unsharded: max rel err {err:.3e}", flush=True)
    assert err <= U.tol_for(wl)


WOI_CASES = {
    "f32": WORKLOADS["tiny_fp32"].replace(topk=1, renormalize=False, router_weight_on_input=True),
    "bf16_stream": WORKLOADS["mixtral_bf16"].replace(M=300, K=384, I=256, E=6, topk=1, renormalize=False,
                                                     logits_dist="normal", router_weight_on_input=True),
    "bf16_batched": WORKLOADS["mixtral_bf16"].replace(M=150, K=256, I=128, E=5, topk=1, format=FORMAT_BATCHED,
                                                      capacity=150, logits_dist="normal", renormalize=False,
                                                      router_weight_on_input=True),
    "fp8_batched": WORKLOADS["decode_fp8_m64"].replace(M=90, K=384, I=256, E=5, topk=1, capacity=90,
                                                       renormalize=False, router_weight_on_input=True),
}


@pytest.mark.parametrize("name", list(WOI_CASES))
def test_router_weight_on_input_parity(name):
    """topk = 1 with the router weight applied to the input before
    quantisation / dispatch, and not again in the combine."""
    wl = WOI_CASES[name]
    d = make_inputs(wl, seed=33, device="cpu")
    out, _, _, _ = U.run_forward(wl, U.to_cuda(d))
    torch.cuda.synchronize()
    toks = sample_tokens(wl.M, 24, seed=7)
    ref, _, w = oracle.moe_tokens(wl, d, toks)
    assert np.all(w < 1.0)
    err = U.rel_err(out.float().cpu().numpy()[toks], ref)
    print(f"  weight on input {name}: max rel err {err:.3e}", flush=True)
    assert err <= U.tol_for(wl)
    # the weight is applied once: against the plain layer the output differs
    plain, _, _ = oracle.moe_tokens(wl.replace(router_weight_on_input=False), d, toks)
    assert U.rel_err(plain, ref) > 10 * U.tol_for(wl)


# ----------------------------------------------------------------- activation chunking

CHUNK_CASES = {
    # streaming kernel for the batch and for every chunk: bitwise equal to unchunked
    "bf16_stream": (WORKLOADS["mixtral_bf16"].replace(M=300, K=384, I=256, E=7, topk=3, renormalize=False,
                                                      logits_dist="normal"), 128, True),
    "fp8_standard": (WORKLOADS["decode_fp8_m64"].replace(M=200, K=256, I=256, E=6, topk=3,
                                                         format=FORMAT_STANDARD, capacity=0), 64, True),
    "weight_on_input": (WORKLOADS["mixtral_bf16"].replace(M=300, K=384, I=256, E=6, topk=1, renormalize=False,
                                                          logits_dist="normal", router_weight_on_input=True),
                        100, True),
    # MFMA tiles for the batch, weight streaming for each chunk: same result within the bar
    "bf16_mfma_to_stream": (WORKLOADS["mixtral_bf16"].replace(M=1200, K=256, I=256, E=4, topk=2,
                                                              renormalize=False, logits_dist="normal"), 500, False),
}


@pytest.mark.parametrize("name", list(CHUNK_CASES))
def test_chunked_forward(name):
    """The experts step in chunks of tokens (per-chunk recount, permutation,
    tile plan and GEMMs): each token's result is unchanged."""
    wl, chunk, bitwise = CHUNK_CASES[name]
    dcpu = make_inputs(wl, seed=34, device="cpu")
    d = U.to_cuda(dcpu)
    ref, _, _, _ = U.run_forward(wl, d)
    pc = U.problem(wl, chunk_tokens=chunk)
    assert moe.workspace_size(pc) < moe.workspace_size(U.problem(wl))
    got, _, ws, _ = U.run_forward(wl, d, p=pc)
    torch.cuda.synchronize()
    L = moe.workspace_layout(pc)
    assert U.ws_view(ws, L.status, 1).item() == 0
    if bitwise:
        assert torch.equal(got, ref)
    toks = sample_tokens(wl.M, 16, seed=8)
    oref, _, _ = oracle.moe_tokens(wl, dcpu, toks)
    err = U.rel_err(got.float().cpu().numpy()[toks], oref)
    print(f"  chunked {name}: max rel err {err:.3e}", flush=True)
    assert err <= U.tol_for(wl)


def test_chunked_forward_split_k_and_short_last_chunk():
    """Few experts and wide K in bf16: the down GEMM splits K into fp32 partial
    sums for the batch and for the 64-token chunks, whose workspace reserves
    the split of one chunk; the last chunk of 3 tokens (6 picks on at most 6
    experts) is below the split's item count and takes unsplit panels.  Every
    token is compared with the oracle."""
    wl = SMALL["bf16_split_k"].replace(M=131)
    pc = U.problem(wl, chunk_tokens=64)
    full, ch = moe.workspace_layout(U.problem(wl)), moe.workspace_layout(pc)
    assert full.down_split == 2 and ch.down_split == 2
    dcpu = make_inputs(wl, seed=35, device="cpu")
    d = U.to_cuda(dcpu)
    ref, _, _, _ = U.run_forward(wl, d)
    got, _, ws, _ = U.run_forward(wl, d, p=pc)
    torch.cuda.synchronize()
    assert U.ws_view(ws, ch.status, 1).item() == 0
    # the full chunks split K exactly as the whole batch does
    assert torch.equal(got[:128], ref[:128])
    toks = np.arange(wl.M)
    oref, _, _ = oracle.moe_tokens(wl, dcpu, toks)
    for name, out in (("batch", ref), ("chunked", got)):
        err = U.rel_err(out.float().cpu().numpy(), oref)
        print(f"  split-K {name}: max rel err {err:.3e}", flush=True)
        assert err <= U.tol_for(wl)


def test_chunked_forward_with_shard_map_and_bad_ids_flag():
    """Chunks of an expert-parallel shard; a bad id in the first chunk stays
    flagged after the later chunks run."""
    wl = SHARD_CASES["bf16_standard"]
    d = make_inputs(wl, seed=35, device="cpu")
    ds, El = _shard_inputs(d, wl.E, 3, 1)
    wls = wl.replace(E=El, global_E=wl.E)
    g = U.to_cuda(ds)
    ref, _, _, _ = U.run_forward(wls, g)
    pc = U.problem(wls, expert_map=g["expert_map"], chunk_tokens=64)
    got, _, _, _ = U.run_forward(wls, g, p=pc)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    # a map entry outside [-1, E) on a picked expert: flagged, and kept across chunks
    bad_map = g["expert_map"].clone()
    picked = oracle.route(ds["logits"], wl.topk, wl.scoring, wl.renormalize)[0][0, 0]
    bad_map[int(picked)] = El + 5
    pb = U.problem(wls, expert_map=bad_map, chunk_tokens=64)
    _, _, ws, _ = U.run_forward(wls, g, p=pb)
    torch.cuda.synchronize()
    assert U.ws_view(ws, moe.workspace_layout(pb).status, 1).item() & moe.DEVICE_BAD_EXPERT_ID


# ------------------------------------------------------- random shapes

def _random_cases(n=24, seed=2024):
    """Seeded random small layers over dtype, format, scoring, activation and
    ragged sizes, so that every grouped-GEMM kernel (weight streaming, 128x256
    MFMA tiles, 128x128 tiles) meets shapes the named cases do not."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        kind = ["f32", "bf16", "bf16", "fp8"][int(rng.integers(4))]
        E = int(rng.integers(1, 41))
        k = int(rng.integers(1, min(E, 8) + 1))
        M = int(rng.integers(1, 400))
        K = 128 * int(rng.integers(1, 7))
        I = (128 if kind == "fp8" else 64) * int(rng.integers(1, 7))
        if M * k * I * K > 2e8:
            continue
        batched = kind != "f32" and rng.random() < 0.4
        base = dict(tiny_fp32="tiny_fp32", bf16="mixtral_bf16", fp8="decode_fp8_m64")
        wl = WORKLOADS[base.get(kind, "tiny_fp32")].replace(
            M=M, K=K, I=I, E=E, topk=k, logits_dist="normal",
            scoring=SCORING_SIGMOID if rng.random() < 0.3 else 0,
            renormalize=bool(rng.random() < 0.5), activation=int(rng.random() < 0.3),
            format=FORMAT_BATCHED if (batched or kind == "fp8") else FORMAT_STANDARD,
            capacity=M if (batched or kind == "fp8") else 0)
        cases.append((f"{kind}_E{E}_k{k}_M{M}_K{K}_I{I}_{'bat' if wl.format else 'std'}", wl))
    return cases


RANDOM_CASES = _random_cases()


@pytest.mark.parametrize("name,wl", RANDOM_CASES, ids=[c[0] for c in RANDOM_CASES])
def test_forward_random_shapes(name, wl):
    d = make_inputs(wl, seed=21, device="cpu")
    out, _, ws, p = U.run_forward(wl, U.to_cuda(d))
    torch.cuda.synchronize()
    L = moe.workspace_layout(p)
    assert int(U.ws_view(ws, L.status, 1).cpu()[0]) == 0
    ref, _, _ = oracle.moe_tokens(wl, d)
    err = U.rel_err(out.float().cpu().numpy(), ref)
    print(f"  {name}: max rel err {err:.3e}", flush=True)
    assert err <= U.tol_for(wl)


# ------------------------------- asynchronous prepare / finalize, two microbatches

def test_async_prepare_finalize_equal_the_stage_calls():
    """prepare_async / finalize_async on a dispatch stream, received on the
    compute stream, give exactly what the synchronous stage calls give (the
    hook / receiver pair is equivalent to prepare / finalize)."""
    for wl in (SMALL["bf16_ragged"], SMALL["fp8_batched"], SMALL["bf16_split_k"]):
        d = U.to_cuda(make_inputs(wl, seed=33, device="cpu"))
        ref, _, _, p = U.run_forward(wl, d)
        ws = moe.empty_workspace(p)
        w = torch.empty(wl.M, wl.topk, device="cuda")
        ids = torch.empty(wl.M, wl.topk, dtype=torch.int32, device="cuda")
        moe.moe_route(p, d["logits"], w, ids)
        fp8 = wl.act_quant == QUANT_FP8_G128
        bat = U.batched(wl)
        counts = torch.full((wl.E,), -1, dtype=torch.int32, device="cuda")
        a_out = a_s = None
        if bat:
            a_out = torch.empty(wl.E, wl.capacity, wl.K, dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
            if fp8:
                a_s = torch.empty(wl.E * wl.capacity, wl.K // 128, device="cuda")
        comm = torch.cuda.Stream()
        comm.wait_stream(torch.cuda.current_stream())
        prepared, combined = torch.cuda.Event(), torch.cuda.Event()
        moe.moe_prepare_async(p, d["x"], ids, a_out, a_s, counts, ws, comm, prepared)
        moe.moe_receive(torch.cuda.current_stream(), prepared)
        rows = wl.E * wl.capacity if bat else wl.M * wl.topk
        fused = torch.empty(rows, wl.K, dtype=torch.bfloat16, device="cuda")
        moe.moe_experts(p, a_out if bat else d["x"], a_s, d["w1"], d.get("w1_scale"), d["w2"], d.get("w2_scale"),
                        counts, fused, ws)
        out = torch.empty_like(ref)
        comm.wait_stream(torch.cuda.current_stream())
        moe.moe_finalize_async(p, fused, w, out, ws, comm, combined)
        moe.moe_receive(torch.cuda.current_stream(), combined)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


DBO_CASES = {
    # the same GEMM kernels for the batch and its halves: bitwise equal to moe_forward
    "fp8_batched": (WORKLOADS["decode_fp8_m64"].replace(M=96, K=512, I=256, E=16, topk=4, capacity=96), True),
    "bf16_split_k": (SMALL["bf16_split_k"], True),
    "bf16_mfma": (SMALL["bf16_mfma_groups"], True),
    "bf16_shared": (WORKLOADS["dsv3_bf16"].replace(M=256, E=32, I=256, K=512, shared_I=256), True),
    "odd_M": (SMALL["bf16_ragged"].replace(M=301), True),
    "M1": (SMALL["bf16_ragged"].replace(M=1), True),
    # halves of 300 rows per expert stream where the batch takes MFMA tiles:
    # within the bar of the oracle
    "bf16_mfma_to_stream": (WORKLOADS["mixtral_bf16"].replace(M=600, K=512, I=256, E=4, topk=2, renormalize=False,
                                                              logits_dist="normal"), False),
}


def _run_dbo(wl, d, p=None, wss=None, out=None, sout=None, comm=None, events=None, streams=None):
    p = p or U.problem(wl)
    if wss is None:
        q = moe.dbo_microbatch_problem(p)
        wss = [moe.empty_workspace(q), moe.empty_workspace(q)]
    out = out if out is not None else torch.empty(wl.M, wl.K, dtype=U.torch_act_dtype(wl), device="cuda")
    comm = comm or torch.cuda.Stream()
    events = events or moe.DboEvents()
    shared = None
    if wl.shared_I:
        sout = sout if sout is not None else torch.empty_like(out)
        streams = streams or (moe.SharedExpertStreams(), moe.SharedExpertStreams())
        shared = (d["w1s"], d["w2s"], sout)
    moe.moe_forward_dbo(p, d["logits"], d["x"], d["w1"], d.get("w1_scale"), d["w2"], d.get("w2_scale"), out, wss,
                        comm, events, shared=shared, shared_streams=streams)
    return out, sout, wss


@pytest.mark.parametrize("name", list(DBO_CASES))
def test_dbo_forward(name):
    """moe_forward_dbo (two microbatches, dispatch and combine on a second
    stream) against moe_forward, and against the oracle."""
    wl, bitwise = DBO_CASES[name]
    d = make_inputs(wl, seed=34, device="cpu")
    g = U.to_cuda(d)
    ref, sref, _, p = U.run_forward(wl, g)
    out, sout, wss = _run_dbo(wl, g, p=p)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    if bitwise:
        assert torch.equal(out, ref)
        if wl.shared_I:
            assert torch.equal(sout, sref)
    toks = sample_tokens(wl.M, 24, seed=6)
    oref, _, _ = oracle.moe_tokens(wl, d, toks)
    err = U.rel_err(got[toks], oref)
    print(f"  dbo {name}: max rel err {err:.3e}", flush=True)
    assert err <= U.tol_for(wl)
    # each microbatch's status word is clear
    q = moe.dbo_microbatch_problem(p)
    for ws in wss[: 2 if wl.M > 1 else 1]:
        assert U.ws_view(ws, moe.workspace_layout(q).status, 1).item() == 0


def test_dbo_graph_replay_matches_eager():
    """The two-microbatch layer captured in one graph (the dispatch stream and
    the shared expert's aux streams fork from and join the capture stream);
    every replay with fresh inputs is bitwise equal to an eager run."""
    wl = DBO_CASES["bf16_shared"][0]
    d = U.to_cuda(make_inputs(wl, seed=35, device="cpu"))
    p = U.problem(wl)
    q = moe.dbo_microbatch_problem(p)
    wss = [moe.empty_workspace(q), moe.empty_workspace(q)]
    out = torch.empty(wl.M, wl.K, dtype=torch.bfloat16, device="cuda")
    sout = torch.empty_like(out)
    comm, events = torch.cuda.Stream(), moe.DboEvents()
    streams = (moe.SharedExpertStreams(), moe.SharedExpertStreams())
    _run_dbo(wl, d, p, wss, out, sout, comm, events, streams)   # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            _run_dbo(wl, d, p, wss, out, sout, comm, events, streams)
    torch.cuda.synchronize()
    for r in range(3):
        fresh = make_inputs(wl, seed=36 + r, device="cpu")
        d["logits"].copy_(fresh["logits"].cuda())
        d["x"].copy_(fresh["x"].cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got, sgot = out.clone(), sout.clone()
        ref, sref, _ = _run_dbo(wl, d, p)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), r
        assert torch.equal(sgot, sref), r


PLAN_CASES = {
    # the large-batch counting (up to 256 chunks) and plan kernels: 131K Zipf
    # pairs whose largest expert has about 130 row tiles, and 32K pairs over
    # 256 experts
    # (K and I cut down: the routing and so the plan do not depend on them)
    "skewed_full": WORKLOADS["skewed_bf16"].replace(K=256, I=128),
    "dsv3_full": WORKLOADS["dsv3_bf16"].replace(K=256, I=128, shared_I=0),
    # a small batch: the one-block counting kernel writes the plan
    "mixtral_small": WORKLOADS["mixtral_bf16"].replace(M=300, K=256, I=128, logits_dist="normal"),
    # BatchedExperts rows (segment e * capacity)
    "decode_m256": WORKLOADS["decode_fp8_m256"].replace(K=512, I=256),
    # experts without pairs first, in the middle and last (their logits pushed
    # down), past the small-batch size
    "empty_experts": WORKLOADS["mixtral_bf16"].replace(M=3000, K=256, I=256, E=16, topk=2,
                                                       renormalize=False, logits_dist="normal"),
}


@pytest.mark.parametrize("name", list(PLAN_CASES))
def test_tile_plan_matches_counts(name):
    """The grouped GEMMs' tile plan, read from the workspace after a forward
    pass, against the one the counts define: for every expert in order,
    ceil(count / rows) tiles of (expert, segment start, first row, rows), with
    rows the plan's tile height (the largest tile) and the count clipped to
    the capacity in the batched format; the tile count after them."""
    wl = PLAN_CASES[name]
    d = make_inputs(wl, seed=23, device="cpu")
    if name == "empty_experts":
        for e in (0, 1, 7, wl.E - 2, wl.E - 1):
            d["logits"][:, e] = -1e4
    out, _, ws, p = U.run_forward(wl, U.to_cuda(d))
    torch.cuda.synchronize()
    L = moe.workspace_layout(p)
    ids = U.ws_view(ws, L.topk_ids, wl.M * wl.topk).cpu().numpy()
    counts = np.bincount(ids, minlength=wl.E)[: wl.E]
    if name == "empty_experts":
        assert counts[[0, 1, 7, wl.E - 2, wl.E - 1]].sum() == 0 and counts.sum() == wl.M * wl.topk
    ntile = U.ws_view(ws, L.tiles + 4 * 4 * L.max_tiles, 1).item()
    tiles = U.ws_view(ws, L.tiles, 4 * ntile).cpu().numpy().reshape(ntile, 4)
    rows = int(tiles[:, 3].max())
    if U.batched(wl):
        seg = np.arange(wl.E) * wl.capacity
        cnt = np.minimum(counts, wl.capacity)
    else:
        seg = U.ws_view(ws, L.offsets, wl.E).cpu().numpy()
        cnt = counts
    ref = [(e, seg[e], i * rows, min(rows, cnt[e] - i * rows))
           for e in range(wl.E) for i in range(-(-int(cnt[e]) // rows))]
    print(f"  plan {name}: {ntile} tiles of {rows} rows, largest expert {cnt.max()} rows", flush=True)
    assert ntile == len(ref) <= L.max_tiles
    np.testing.assert_array_equal(tiles, np.array(ref, dtype=np.int64).reshape(-1, 4))
