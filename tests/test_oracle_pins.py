"""Pins of the CPU oracle against things other than itself (CPU only).

Each check ties one oracle function to a closed form, a library routine, a
dense brute force or an invariant of the method, chosen so that a plausible
mistake (dropped term, wrong sign or index, transposed operand, wrong tie
order) fails at least one of them; test_planted_mistakes builds mutated copies
of the oracle and shows each is caught.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
from tests import bruteforce as bf
from workloads import WORKLOADS, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tied_logits(M, E, rng):
    """Small-integer logits so that ties are frequent."""
    return rng.integers(-2, 3, size=(M, E)).astype(np.float32)


# ------------------------------------------------------------------ router

@pytest.mark.parametrize("M,E,k", [(1, 1, 1), (7, 4, 4), (33, 8, 2), (64, 32, 8), (17, 256, 8)])
def test_route_ids_match_stable_argsort(M, E, k):
    for logits in (RNG.standard_normal((M, E)).astype(np.float32), _tied_logits(M, E, RNG)):
        ids, _ = oracle.route(logits, k)
        np.testing.assert_array_equal(ids, bf.topk_select(logits, k))
        assert all(len(set(r)) == k for r in ids.tolist())


@pytest.mark.parametrize("sigmoid", [False, True])
@pytest.mark.parametrize("renorm", [False, True])
def test_route_weights_match_scipy(sigmoid, renorm):
    logits = RNG.standard_normal((50, 16)).astype(np.float32) * 3
    ids, w = oracle.route(logits, 4, oracle.SIGMOID if sigmoid else oracle.SOFTMAX, renorm)
    ref = bf.router_weights(logits, ids, sigmoid, renorm)
    np.testing.assert_allclose(w, ref, rtol=1e-13, atol=0)
    if renorm:
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-13)


def test_route_full_softmax_when_k_equals_E():
    logits = RNG.standard_normal((9, 6)).astype(np.float32)
    ids, w = oracle.route(logits, 6)
    P = sps.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(np.take_along_axis(P, ids, 1), w, rtol=1e-13)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-13)
    assert np.all(np.diff(w, axis=1) <= 0)       # emitted in descending order


def test_route_golden_closed_forms():
    for case in _load("router_closed_form.json")["cases"]:
        if "probs" in case:
            logits = np.log(np.array(case["probs"], np.float64)).astype(np.float32)
            tol = 1e-6                           # fp32 rounding of the logs
        else:
            logits = np.array(case["logits"], np.float32)
            tol = 1e-15
        scoring = oracle.SIGMOID if case["scoring"] == "sigmoid" else oracle.SOFTMAX
        ids, w = oracle.route(logits[None, :], case["k"], scoring, case["renormalize"])
        assert ids[0].tolist() == case["ids"], case["name"]
        np.testing.assert_allclose(w[0], case["weights"], rtol=tol, err_msg=case["name"])


# --------------------------------------------------- counting / permutation

@pytest.mark.parametrize("M,E,k,align", [(64, 8, 2, 1), (64, 8, 2, 32), (300, 32, 8, 16),
                                         (5, 256, 8, 128), (1000, 3, 3, 7)])
def test_counts_and_standard_permutation(M, E, k, align):
    ids, _ = oracle.route(RNG.standard_normal((M, E)).astype(np.float32), k)
    flat = ids.ravel()
    counts, offsets, perm, inv = oracle.permute_standard(ids, E, align)
    # counts: library routine, and they sum to M*k
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    assert counts.sum() == M * k
    np.testing.assert_array_equal(oracle.count(ids, E), counts)
    # offsets: padded exclusive prefix sum, within the host bound
    assert offsets[0] == 0 and np.all(np.diff(offsets) % align == 0)
    np.testing.assert_array_equal(np.diff(offsets), -(-counts // align) * align)
    assert offsets[-1] <= M * k + E * (align - 1) == perm.size
    # valid slots are a bijection onto [0, M*k); pads are -1
    valid = perm >= 0
    assert valid.sum() == M * k
    np.testing.assert_array_equal(np.sort(perm[valid]), np.arange(M * k))
    np.testing.assert_array_equal(perm[inv], np.arange(M * k))      # perm o inv = id
    np.testing.assert_array_equal(inv[perm[valid]], np.nonzero(valid)[0])
    # stable order inside each segment == numpy's stable argsort by expert
    order = np.argsort(flat, kind="stable")
    got = np.concatenate([perm[offsets[e]: offsets[e] + counts[e]] for e in range(E)])
    np.testing.assert_array_equal(got, order)
    for e in range(E):
        seg = perm[offsets[e]: offsets[e + 1]]
        assert np.all(seg[counts[e]:] == -1)
        assert np.all(np.diff(seg[: counts[e]]) > 0)
        assert np.all(flat[seg[: counts[e]]] == e)


@pytest.mark.parametrize("cap", [1, 5, 64, 10_000])
def test_batched_slots(cap):
    M, E, k = 200, 16, 4
    ids, _ = oracle.route(RNG.standard_normal((M, E)).astype(np.float32), k)
    flat = ids.ravel()
    counts, inv = oracle.permute_batched(ids, E, cap)
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    for e in range(E):
        f_e = np.nonzero(flat == e)[0]                  # ascending pair order
        r = np.arange(f_e.size)
        expect = np.where(r < cap, e * cap + r, -1)
        np.testing.assert_array_equal(inv[f_e], expect)
    kept = inv[inv >= 0]
    assert len(np.unique(kept)) == kept.size            # no two pairs share a row


# ------------------------------------------------------------------ fp8

def test_e4m3_golden_codes():
    g = _load("e4m3_codes.json")
    for v, code, exact in g["encode"]:
        assert int(oracle.e4m3_encode([v])[0]) == code, v
        if exact:
            assert oracle.e4m3_decode([code])[0] == v, v
    for c in g["decode_nan"]:
        assert math.isnan(oracle.e4m3_decode([c])[0])


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def _encoder_probe_values():
    # every bf16-representable finite value below 448 in magnitude, plus values
    # whose low 16 bits sit on and beside every rounding boundary
    hi = np.arange(0, 1 << 16, dtype=np.uint32)
    vals = []
    for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
        vals.append(((hi << 16) | lo).view(np.float32))
    v = np.concatenate(vals)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    return v


def test_e4m3_encoder_matches_torch_cast_dense():
    v = _encoder_probe_values()
    ours = oracle.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_error_bound_and_roundtrip():
    x = (RNG.standard_normal(20000) * 50).astype(np.float32)
    x = x[np.abs(x) <= 448]
    q = oracle.e4m3_decode(oracle.e4m3_encode(x))
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(np.abs(q - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])
    assert np.all(np.abs(q - x)[~normal] <= 2.0 ** -10)
    reps = oracle.e4m3_decode(np.arange(0, 127, dtype=np.uint8)).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_decode(oracle.e4m3_encode(reps)), reps)


def test_quant_g128_matches_torch_and_bounds():
    x = (RNG.standard_normal((5, 384)) * RNG.uniform(1e-3, 1e3, (5, 1))).astype(np.float32)
    x[2, 128:256] = 0.0                                  # an all-zero group
    q, s = oracle.quant_g128(x)
    deq = oracle.e4m3_decode(q) * np.repeat(s, 128, axis=1)
    np.testing.assert_array_equal(deq, bf.fp8_group_quant_torch(x))
    amax = np.abs(x).reshape(5, 3, 128).max(2)
    np.testing.assert_array_equal(s, (np.maximum(amax, np.float32(1e-10)) / np.float32(448)).astype(np.float32))
    assert np.all(deq[2, 128:256] == 0)
    # each group's max element lands on +-448 * s
    grp = np.abs(oracle.e4m3_decode(q)).reshape(5, 3, 128).max(2)
    assert np.all((grp == 448) | (amax == 0))


# ------------------------------------------------------- expert MLP / layer

def _tiny(M, K, I, E, k, seed):
    rng = np.random.default_rng(seed)
    return dict(logits=rng.standard_normal((M, E)).astype(np.float32),
                x=rng.standard_normal((M, K)).astype(np.float32),
                w1=(rng.standard_normal((E, 2 * I, K)) * 0.2).astype(np.float32),
                w2=(rng.standard_normal((E, K, I)) * 0.2).astype(np.float32))


def _wl(M, K, I, E, k, **kw):
    return WORKLOADS["tiny_fp32"].replace(M=M, K=K, I=I, E=E, topk=k, **kw)


@pytest.mark.parametrize("M,K,I,E,k,sig,ren", [(5, 8, 4, 3, 2, False, False), (9, 16, 8, 6, 3, True, True),
                                               (4, 12, 6, 5, 5, False, True), (3, 8, 2, 1, 1, False, False)])
def test_layer_matches_dense_brute_force(M, K, I, E, k, sig, ren):
    d = _tiny(M, K, I, E, k, seed=M * 131 + E)
    wl = _wl(M, K, I, E, k, scoring=int(sig), renormalize=ren)
    out, ids, w = oracle.moe_tokens(wl, d)
    ref, rids, rw = bf.dense_moe(d["logits"], d["x"], d["w1"], d["w2"], k, sig, ren)
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=1e-13)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_tiny_fp32_workload_matches_dense_brute_force():
    wl = WORKLOADS["tiny_fp32"]
    d = make_inputs(wl, seed=0, device="cpu")
    out, _, _ = oracle.moe_tokens(wl, d)
    ref, _, _ = bf.dense_moe(d["logits"].numpy(), d["x"].numpy(), d["w1"].numpy(), d["w2"].numpy(),
                             wl.topk)
    rel = np.abs(out - ref).max() / np.abs(ref).max()
    assert rel <= 1e-12


def test_fp8_layer_matches_dense_brute_force():
    # tiny fp8 batched layer: token-group quantisation of x and of act
    wl = WORKLOADS["decode_fp8_m64"].replace(M=6, K=256, I=128, E=4, topk=2, capacity=48)
    d = make_inputs(wl, seed=3, device="cpu")
    out, _, _ = oracle.moe_tokens(wl, d)
    w1 = (d["w1"].view(torch.float8_e4m3fn).to(torch.float64)
          * torch.repeat_interleave(torch.repeat_interleave(d["w1_scale"].double(), 128, 1), 128, 2)).numpy()
    w2 = (d["w2"].view(torch.float8_e4m3fn).to(torch.float64)
          * torch.repeat_interleave(torch.repeat_interleave(d["w2_scale"].double(), 128, 1), 128, 2)).numpy()
    ref, _, _ = bf.dense_moe(d["logits"].numpy(), d["x"].float().numpy(), w1, w2, wl.topk, fp8_act=True)
    # same quantisation decisions on both sides except where fp64 sums of act
    # land on a different side of an fp32 rounding -- allow that rare flip
    rel = np.abs(out - ref).max() / np.abs(ref).max()
    assert rel <= 1e-3


@pytest.mark.parametrize("cap", [1, 3, 7])
def test_batched_capacity_drop_matches_brute_force(cap):
    """Worst-tokens layout with fewer rows per expert than some experts
    receive: the picks whose rank in their expert (token order) reaches the
    capacity are dropped and add nothing to their token's output."""
    M, K, I, E, k = 24, 8, 4, 4, 2
    d = _tiny(M, K, I, E, k, seed=77 + cap)
    wl = _wl(M, K, I, E, k, format=oracle.BATCHED, capacity=cap)
    out, ids, _ = oracle.moe_tokens(wl, d)
    keep = bf.capacity_keep(ids, cap)
    # the rank rule itself, counted pick by pick in token order
    seen = {}
    for m in range(M):
        for j in range(k):
            e = int(ids[m, j])
            assert keep[m, j] == (seen.get(e, 0) < cap)
            seen[e] = seen.get(e, 0) + 1
    assert keep.any() and not keep.all()
    ref, _, _ = bf.dense_moe(d["logits"], d["x"], d["w1"], d["w2"], k, capacity=cap)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    undropped, _, _ = bf.dense_moe(d["logits"], d["x"], d["w1"], d["w2"], k)
    assert np.abs(out - undropped).max() > 1e-3 * np.abs(undropped).max()


def test_fp8_capacity_drop_matches_dense_brute_force():
    # the tiny fp8 batched layer with 2 rows per expert buffer: most picks dropped
    wl = WORKLOADS["decode_fp8_m64"].replace(M=6, K=256, I=128, E=4, topk=2, capacity=2)
    d = make_inputs(wl, seed=3, device="cpu")
    out, ids, _ = oracle.moe_tokens(wl, d)
    assert not bf.capacity_keep(ids, 2).all()
    w1 = (d["w1"].view(torch.float8_e4m3fn).to(torch.float64)
          * torch.repeat_interleave(torch.repeat_interleave(d["w1_scale"].double(), 128, 1), 128, 2)).numpy()
    w2 = (d["w2"].view(torch.float8_e4m3fn).to(torch.float64)
          * torch.repeat_interleave(torch.repeat_interleave(d["w2_scale"].double(), 128, 1), 128, 2)).numpy()
    ref, _, _ = bf.dense_moe(d["logits"].numpy(), d["x"].float().numpy(), w1, w2, wl.topk, fp8_act=True,
                             capacity=2)
    rel = np.abs(out - ref).max() / np.abs(ref).max()
    assert rel <= 1e-3


def test_golden_expert_closed_form():
    g = _load("expert_closed_form.json")
    x = np.array(g["x"], np.float32)
    w1 = np.array(g["w1"], np.float32)
    w2 = np.array(g["w2"], np.float32)
    for e in range(g["E"]):
        act, y = oracle.expert_row(x[0].astype(np.float64), e, w1, w2, oracle.F32, g["I"])
        np.testing.assert_allclose(act, [g["act"][e]], rtol=1e-15)
        np.testing.assert_allclose(y, g["y"][e], rtol=1e-15)
    logits = np.log(np.array(g["probs"]))[None, :].astype(np.float32)
    wl = _wl(1, g["K"], g["I"], g["E"], g["topk"])
    out, ids, w = oracle.moe_tokens(wl, dict(logits=logits, x=x, w1=w1, w2=w2))
    np.testing.assert_allclose(out, g["out"], rtol=1e-7)    # fp32 rounding of the log-probs


def test_single_expert_is_textbook_gated_mlp():
    # E = 1, k = 1: the layer is silu(x Wg^T) * (x Wu^T) W2^T with weight 1
    d = _tiny(7, 16, 8, 1, 1, seed=5)
    out, _, w = oracle.moe_tokens(_wl(7, 16, 8, 1, 1), d)
    x, w1, w2 = (torch.from_numpy(d[k]).double() for k in ("x", "w1", "w2"))
    ref = (torch.nn.functional.silu(x @ w1[0, :8].T) * (x @ w1[0, 8:].T)) @ w2[0].T
    np.testing.assert_allclose(w, 1.0)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.dense_mlp_tokens(d["x"], d["w1"][0], d["w2"][0], 8, oracle.F32),
                               ref.numpy(), rtol=1e-12, atol=1e-14)


def test_identical_experts_with_renorm_is_dense_mlp():
    d = _tiny(6, 16, 8, 4, 3, seed=6)
    d["w1"][:] = d["w1"][0]
    d["w2"][:] = d["w2"][0]
    out, _, _ = oracle.moe_tokens(_wl(6, 16, 8, 4, 3, renormalize=True), d)
    ref = bf.dense_mlp(d["x"], d["w1"][0], d["w2"][0])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_zero_count_expert_contributes_nothing():
    d = _tiny(16, 16, 8, 6, 2, seed=7)
    d["logits"][:, 4] = -30.0                       # expert 4 is never picked
    wl = _wl(16, 16, 8, 6, 2)
    base, ids, _ = oracle.moe_tokens(wl, d)
    assert not np.any(ids == 4)
    d["w1"][4] = np.nan
    d["w2"][4] = np.nan
    poisoned, _, _ = oracle.moe_tokens(wl, d)
    assert np.all(np.isfinite(poisoned))
    np.testing.assert_array_equal(poisoned, base)


def test_identity_expert_dispatch_combine_returns_x():
    # dispatch the rows, let each "expert" return its input unchanged, combine
    # with renormalised weights: the layer is the identity
    M, E, k, K = 40, 8, 3, 5
    logits = RNG.standard_normal((M, E)).astype(np.float32)
    x = RNG.standard_normal((M, K))
    ids, w = oracle.route(logits, k, oracle.SOFTMAX, True)
    counts, offsets, perm, inv = oracle.permute_standard(ids, E, align=4)
    dispatched = np.full((perm.size, K), np.nan)
    dispatched[perm >= 0] = x[perm[perm >= 0] // k]        # permute: slot <- token row
    y = dispatched[inv].reshape(M, k, K)                   # unpermute: pair <- slot
    np.testing.assert_allclose(oracle.combine(w, y), x, rtol=1e-14, atol=1e-15)
    for cap in (1000, 7):
        counts_b, inv_b = oracle.permute_batched(ids, E, cap)
        buf = np.full((E * cap, K), np.nan)
        keep = inv_b >= 0
        buf[inv_b[keep]] = x[np.nonzero(keep)[0] // k]
        yb = np.zeros((M * k, K))
        yb[keep] = buf[inv_b[keep]]
        out = oracle.combine(w, yb.reshape(M, k, K), keep.astype(np.int32))
        if cap == 1000:
            np.testing.assert_allclose(out, x, rtol=1e-14, atol=1e-15)
        else:
            dropped = ~keep.reshape(M, k)
            ref = x * (w * ~dropped).sum(1, keepdims=True)
            np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


def test_metamorphic_relations():
    M, K, I, E, k = 12, 16, 8, 5, 2
    d = _tiny(M, K, I, E, k, seed=8)
    wl = _wl(M, K, I, E, k)
    out, _, _ = oracle.moe_tokens(wl, d)
    # permuting tokens permutes the output
    p = RNG.permutation(M)
    d2 = dict(d, logits=d["logits"][p], x=d["x"][p])
    np.testing.assert_allclose(oracle.moe_tokens(wl, d2)[0], out[p], rtol=1e-13, atol=1e-15)
    # relabelling experts (logit columns and weight slices together) changes nothing
    q = RNG.permutation(E)
    d3 = dict(d, logits=np.ascontiguousarray(d["logits"][:, q]), w1=d["w1"][q], w2=d["w2"][q])
    np.testing.assert_allclose(oracle.moe_tokens(wl, d3)[0], out, rtol=1e-13, atol=1e-15)
    # linear in w2 (no renormalisation): doubling w2 doubles the output
    d4 = dict(d, w2=d["w2"] * 2)
    np.testing.assert_allclose(oracle.moe_tokens(wl, d4)[0], 2 * out, rtol=1e-13, atol=1e-15)
    # Standard == BatchedExperts when nothing overflows
    wlb = wl.replace(format=oracle.BATCHED, capacity=M)
    np.testing.assert_array_equal(oracle.moe_tokens(wlb, d)[0], out)


def test_combine_is_weighted_sum():
    M, k, K = 7, 3, 4
    w = RNG.standard_normal((M, k))
    y = RNG.standard_normal((M, k, K))
    np.testing.assert_allclose(oracle.combine(w, y), np.einsum("mj,mjk->mk", w, y), rtol=1e-13)


# ------------------------------------------ GELU, expert-parallel shard, router weight on input

def test_gelu_expert_closed_form():
    """gelu_and_mul: with a = [1], gate rows g_j and up rows 1, act_j = gelu(g_j)
    = g_j * Phi(g_j).  Checked against textbook values of the normal CDF,
    scipy's ndtr and the odd-symmetry identity gelu(x) - gelu(-x) = x."""
    g = np.array([-3.0, -2.0, -1.0, -0.5, 0.0, 0.5, 1.0, 2.0, 3.0])
    I = g.size
    w1 = np.concatenate([g, np.ones(I)]).reshape(1, 2 * I, 1).astype(np.float32)
    w2 = np.ones((1, 1, I), np.float32)
    act, _ = oracle.expert_row(np.array([1.0]), 0, w1, w2, oracle.F32, I, activation=oracle.GELU)
    np.testing.assert_allclose(act, g * sps.ndtr(g), rtol=1e-14, atol=1e-16)
    # Phi(1) = 0.8413447460685429, Phi(2) = 0.9772498680518208 (tables of the normal CDF)
    np.testing.assert_allclose(act[g == 1.0], 0.8413447460685429, rtol=1e-14)
    np.testing.assert_allclose(act[g == 2.0], 2 * 0.9772498680518208, rtol=1e-14)
    np.testing.assert_allclose(act[g == -1.0], -(1 - 0.8413447460685429), rtol=1e-13)
    np.testing.assert_allclose(act[g > 0] - act[g < 0][::-1], g[g > 0], rtol=1e-14)
    assert act[g == 0.0] == 0.0
    silu, _ = oracle.expert_row(np.array([1.0]), 0, w1, w2, oracle.F32, I)
    np.testing.assert_allclose(silu, g * sps.expit(g), rtol=1e-14, atol=1e-16)


@pytest.mark.parametrize("M,K,I,E,k", [(6, 8, 4, 3, 2), (9, 16, 8, 6, 3)])
def test_gelu_layer_matches_dense_brute_force(M, K, I, E, k):
    d = _tiny(M, K, I, E, k, seed=M * 17 + E)
    out, _, _ = oracle.moe_tokens(_wl(M, K, I, E, k, activation=oracle.GELU), d)
    ref, _, _ = bf.dense_moe(d["logits"], d["x"], d["w1"], d["w2"], k, gelu=True)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.dense_mlp_tokens(d["x"], d["w1"][0], d["w2"][0], I, oracle.F32,
                                                       activation=oracle.GELU),
                               _dense_gelu(d["x"], d["w1"][0], d["w2"][0]), rtol=1e-12, atol=1e-14)


def _dense_gelu(x, w1, w2):
    x, w1, w2 = (np.asarray(a, np.float64) for a in (x, w1, w2))
    I = w1.shape[0] // 2
    H = x @ w1.T
    return bf.gated(H[:, :I], H[:, I:], gelu=True) @ w2.T


def _shard(d, Eg, n_shards, s):
    """Shard s of n: global experts g with g % n == s, local index g // n."""
    glob = np.arange(Eg)[np.arange(Eg) % n_shards == s]
    emap = np.full(Eg, -1, np.int32)
    emap[glob] = np.arange(glob.size, dtype=np.int32)
    return dict(d, w1=np.ascontiguousarray(d["w1"][glob]), w2=np.ascontiguousarray(d["w2"][glob]),
                expert_map=emap), glob.size


@pytest.mark.parametrize("fmt", [oracle.STANDARD, oracle.BATCHED])
def test_expert_shards_sum_to_the_full_layer(fmt):
    """One expert-parallel shard computes only its experts' picks; the shards'
    outputs add up to the unsharded layer (and each matches a dense brute force
    over its experts)."""
    M, K, I, Eg, k = 20, 16, 8, 8, 3
    d = _tiny(M, K, I, Eg, k, seed=21)
    full, fids, _ = oracle.moe_tokens(_wl(M, K, I, Eg, k, format=fmt, capacity=M), d)
    total = np.zeros_like(full)
    for s in range(3):
        ds, El = _shard(d, Eg, 3, s)
        wl = _wl(M, K, I, El, k, global_E=Eg, format=fmt, capacity=M)
        out, ids, _ = oracle.moe_tokens(wl, ds)
        np.testing.assert_array_equal(ids, fids)                     # routing is global
        ref, _, _ = bf.dense_moe(d["logits"], d["x"], ds["w1"], ds["w2"], k, expert_map=ds["expert_map"])
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
        total += out
    np.testing.assert_allclose(total, full, rtol=1e-12, atol=1e-14)


def test_identity_and_empty_expert_maps():
    M, K, I, E, k = 10, 8, 4, 5, 2
    d = _tiny(M, K, I, E, k, seed=22)
    base, _, _ = oracle.moe_tokens(_wl(M, K, I, E, k), d)
    ident = dict(d, expert_map=np.arange(E, dtype=np.int32))
    np.testing.assert_array_equal(oracle.moe_tokens(_wl(M, K, I, E, k, global_E=E), ident)[0], base)
    none_local = dict(d, expert_map=np.full(E, -1, np.int32))
    np.testing.assert_array_equal(oracle.moe_tokens(_wl(M, K, I, E, k, global_E=E), none_local)[0], 0.0)


def test_count_and_permutations_skip_other_shards_pairs():
    ids = np.array([[2, -1], [0, 2], [-1, -1], [1, 0]], np.int32)
    np.testing.assert_array_equal(oracle.count(ids, 3), [2, 1, 2])
    counts, offsets, perm, inv = oracle.permute_standard(ids, 3, align=2)
    flat = ids.ravel()
    assert np.all(inv[flat < 0] == -1)
    np.testing.assert_array_equal(np.sort(perm[perm >= 0]), np.nonzero(flat >= 0)[0])
    np.testing.assert_array_equal(flat[perm[perm >= 0]], np.sort(flat[flat >= 0], kind="stable"))
    cb, invb = oracle.permute_batched(ids, 3, cap=4)
    np.testing.assert_array_equal(cb, counts)
    assert np.all(invb[flat < 0] == -1)
    np.testing.assert_array_equal(invb[flat >= 0] // 4, flat[flat >= 0])


@pytest.mark.parametrize("act_dtype", [oracle.F32, oracle.BF16])
def test_router_weight_on_input_matches_brute_force(act_dtype):
    """topk = 1: the expert sees w * x (held in the activation dtype) and its
    output is added unweighted."""
    M, K, I, E = 12, 16, 8, 4
    d = _tiny(M, K, I, E, 1, seed=23)
    wl = _wl(M, K, I, E, 1, router_weight_on_input=True, act_dtype=act_dtype)
    if act_dtype == oracle.BF16:
        xb = torch.from_numpy(d["x"]).to(torch.bfloat16)
        d = dict(d, x=xb)
        xin = xb.float().numpy()
    else:
        xin = d["x"]
    out, _, w = oracle.moe_tokens(wl, d)
    assert np.all(w < 1.0)
    ref, _, _ = bf.dense_moe(d["logits"], xin, d["w1"], d["w2"], 1, weight_on_input=True,
                             bf16_input=act_dtype == oracle.BF16)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    # a renormalised single pick has weight 1: exactly the unweighted-input layer
    wl1 = wl.replace(renormalize=True)
    np.testing.assert_array_equal(oracle.moe_tokens(wl1, d)[0],
                                  oracle.moe_tokens(wl1.replace(router_weight_on_input=False), d)[0])
    with pytest.raises(ValueError):
        oracle.moe_tokens(_wl(M, K, I, E, 2, router_weight_on_input=True), _tiny(M, K, I, E, 2, seed=1))


# ------------------------------------------------------- planted mistakes

# (name, text in moe_oracle.c, replacement, the pin test(s) that must catch it)
MUTANTS = [
    ("ties to the higher index", "l[e] > l[best]", "l[e] >= l[best]",
     [lambda: test_route_ids_match_stable_argsort(33, 8, 2)]),
    ("softmax denominator misses expert 0",
     "for (int64_t e = 0; e < E; ++e) den += exp", "for (int64_t e = 1; e < E; ++e) den += exp",
     [lambda: test_route_weights_match_scipy(False, False)]),
    ("renormalisation dropped", "if (renormalize)\n", "if (0)\n",
     [lambda: test_route_weights_match_scipy(True, True)]),
    ("unstable permutation", "perm[s] = (int32_t)f;\n    inv[f] = s;",
     "perm[s] = (int32_t)(n - 1 - f);\n    inv[n - 1 - f] = s;",
     [lambda: test_counts_and_standard_permutation(64, 8, 2, 1)]),
    ("padding rounds down", "((counts[e] + align - 1) / align) * align", "(counts[e] / align) * align",
     [lambda: test_counts_and_standard_permutation(64, 8, 2, 32)]),
    ("silu sign", "act[j] = g / (1.0 + exp(-g)) * u;", "act[j] = g / (1.0 + exp(g)) * u;",
     [lambda: test_layer_matches_dense_brute_force(5, 8, 4, 3, 2, False, False)]),
    ("gate and up swapped", "act[j] = g / (1.0 + exp(-g)) * u;", "act[j] = u / (1.0 + exp(-u)) * g;",
     [lambda: test_layer_matches_dense_brute_force(5, 8, 4, 3, 2, False, False),
      test_golden_expert_closed_form]),
    ("w2 read transposed", "weight_at(w_dtype, w2, w2_scale, e, K, I, r, j)",
     "weight_at(w_dtype, w2, w2_scale, e, I, K, j % I, (r * I + j) % K)",
     [lambda: test_layer_matches_dense_brute_force(9, 16, 8, 6, 3, True, True)]),
    ("fp8 ties away from even", "(d == bestd && (c & 1) == 0)", "(d == bestd && (c & 1) == 1)",
     [test_e4m3_encoder_matches_torch_cast_dense]),
    ("fnuz maximum in the scale", "fmaxf(amax, 1e-10f) / 448.0f", "fmaxf(amax, 1e-10f) / 240.0f",
     [test_quant_g128_matches_torch_and_bounds]),
    ("combine ignores the slot weight", "out[m * K + c] += w[m * k + j] * y", "out[m * K + c] += w[m * k] * y",
     [lambda: test_layer_matches_dense_brute_force(9, 16, 8, 6, 3, True, True), test_combine_is_weighted_sum]),
    ("sigmoid scoring uses softmax", "double p = scoring == OR_SOFTMAX ?", "double p = 1 ?",
     [lambda: test_route_weights_match_scipy(True, False)]),
    ("gelu in its tanh form", "0.5 * g * (1.0 + erf(g / sqrt(2.0)))",
     "0.5 * g * (1.0 + tanh(0.7978845608028654 * (g + 0.044715 * g * g * g)))",
     [test_gelu_expert_closed_form, lambda: test_gelu_layer_matches_dense_brute_force(6, 8, 4, 3, 2)]),
    ("expert map ignored", "lids[f] = expert_map ? expert_map[ids[f]] : ids[f];",
     "lids[f] = ids[f] % E;",
     [lambda: test_expert_shards_sum_to_the_full_layer(oracle.STANDARD)]),
    ("router weight applied twice", "wc[j] = weight_on_input ? 1.0 : wts[m * k + j];",
     "wc[j] = wts[m * k + j];",
     [lambda: test_router_weight_on_input_matches_brute_force(oracle.F32)]),
    ("router weight on input ignored", "oracle_input_row(act_dtype, act_quant, x, K, m, weight_on_input,",
     "oracle_input_row(act_dtype, act_quant, x, K, m, 0,",
     [lambda: test_router_weight_on_input_matches_brute_force(oracle.F32)]),
    ("weighted bf16 input not rounded to bf16", "return act_dtype == OR_BF16 ? (double)round_bf16(p) : (double)p;",
     "return (double)p;",
     [lambda: test_router_weight_on_input_matches_brute_force(oracle.BF16)]),
    ("fp8 weight block scales read transposed", "scale[(e * (R / 128) + r / 128) * (C / 128) + c / 128]",
     "scale[(e * (C / 128) + c / 128) * (R / 128) + r / 128]",
     [test_fp8_layer_matches_dense_brute_force]),
    ("act not re-quantised before the down GEMM", "  if (requant_fp8) {\n", "  if (0) {\n",
     [test_fp8_layer_matches_dense_brute_force]),
    ("batched capacity check off by one", "inv[f] = r < cap ? (int32_t)(e * cap + r) : -1;",
     "inv[f] = r <= cap ? (int32_t)(e * cap + r) : -1;",
     [lambda: test_batched_slots(5)]),
    ("batched capacity drop ignored", "keep[j] = lids[m * k + j] >= 0 && !(inv && inv[m * k + j] < 0);",
     "keep[j] = lids[m * k + j] >= 0;",
     [lambda: test_batched_capacity_drop_matches_brute_force(3), test_fp8_capacity_drop_matches_dense_brute_force]),
    ("group maximum taken over signed values", "float a = fabsf(xg[i]);", "float a = xg[i];",
     [test_quant_g128_matches_torch_and_bounds]),
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistakes_are_caught(mutant, tmp_path, monkeypatch):
    name, old, new, checks = mutant
    src = open(oracle._SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name!r} not found"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = oracle.compile_source(str(path), str(tmp_path / "mutant.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.load_library(so))
    for check in checks:
        with pytest.raises(AssertionError):
            check()
