"""Dense float64 brute force of the MoE layer, used only to pin the oracle.

It shares nothing with the oracle's code path: routing uses numpy's stable
argsort and scipy's softmax / expit, every expert is applied densely to every
token (no counting, permutation or combine step), SiLU is written as
g * sigmoid(g) and GELU as g * Phi(g) with scipy's normal CDF, and the fp8
token-group quantiser uses torch's float8_e4m3fn cast.  Only suitable for tiny shapes.
"""
import numpy as np
import scipy.special as sps
import torch


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    # stable sort of the negated fp32 logits: larger first, lower index on ties
    return np.argsort(-logits.astype(np.float32), axis=1, kind="stable")[:, :k]


def router_weights(logits: np.ndarray, ids: np.ndarray, sigmoid: bool, renorm: bool) -> np.ndarray:
    L = logits.astype(np.float64)
    P = sps.expit(L) if sigmoid else sps.softmax(L, axis=1)
    w = np.take_along_axis(P, ids, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def fp8_group_quant_torch(x: np.ndarray) -> np.ndarray:
    """Dequantised token-group-128 fp8 of fp32 rows via torch's e4m3fn cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    rows, cols = t.shape
    g = t.reshape(rows, cols // 128, 128)
    s = torch.clamp(g.abs().amax(dim=2, keepdim=True), min=1e-10) / 448.0
    q = torch.clamp(g / s, -448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * s.to(torch.float64)).reshape(rows, cols).numpy()


def gated(G, U, gelu=False):
    """silu(G) * U, written as G * sigmoid(G) * U; or gelu(G) * U as G * Phi(G) * U
    with scipy's normal CDF."""
    return G * (sps.ndtr(G) if gelu else sps.expit(G)) * U


def capacity_keep(ids: np.ndarray, capacity: int) -> np.ndarray:
    """Batched (worst-tokens) layout with `capacity` rows per expert: a pick is
    kept when fewer than `capacity` earlier picks (in token order) went to the
    same expert.  Ranks come from numpy's stable argsort of the flat ids, so
    ties in expert keep their token order."""
    flat = np.asarray(ids).ravel()
    order = np.argsort(flat, kind="stable")
    rank = np.empty(flat.size, np.int64)
    sorted_ids = flat[order]
    starts = np.searchsorted(sorted_ids, sorted_ids, side="left")
    rank[order] = np.arange(flat.size) - starts
    return (rank < capacity).reshape(np.asarray(ids).shape)


def dense_moe(logits, x, w1, w2, k, sigmoid=False, renorm=False, fp8_act=False, gelu=False,
              expert_map=None, weight_on_input=False, bf16_input=False, capacity=None):
    """out[m] = sum_j w[m,j] * expert_{id[m,j]}(x[m]) with every expert evaluated densely.

    x [M, K], w1 [E, 2I, K], w2 [E, K, I] as float64 arrays (already dequantised).
    expert_map [global E]: local expert of each global one, -1 for another shard's
    (those picks add nothing).  weight_on_input (k = 1): the input row is w * x,
    rounded to fp32 (numpy's float32 product) and to bf16 (torch's cast) when
    bf16_input, and the expert output is added unweighted.  capacity: the
    batched layout's rows per expert; picks past it (capacity_keep) add nothing."""
    x = np.asarray(x, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    E, N, K = w1.shape
    I = N // 2
    ids = topk_select(np.asarray(logits), k)
    wts = router_weights(np.asarray(logits), ids, sigmoid, renorm)
    M = x.shape[0]
    if weight_on_input:
        assert k == 1
        p = np.float32(1.0) * wts[:, :1].astype(np.float32) * x.astype(np.float32)   # fp32 products
        if bf16_input:
            p = torch.from_numpy(p).to(torch.bfloat16).to(torch.float32).numpy()
        x = p.astype(np.float64)
    if fp8_act:
        x = fp8_group_quant_torch(x.astype(np.float32))
    H = np.einsum("mc,enc->emn", x, w1)                # [E, M, 2I]
    A = gated(H[..., :I], H[..., I:], gelu)
    if fp8_act:
        A = np.stack([fp8_group_quant_torch(A[e].astype(np.float32)) for e in range(E)])
    Y = np.einsum("emi,eki->emk", A, w2)               # [E, M, K]
    keep = np.ones(ids.shape, bool) if capacity is None else capacity_keep(ids, capacity)
    out = np.zeros((M, K))
    for m in range(M):
        for j in range(k):
            e = ids[m, j] if expert_map is None else expert_map[ids[m, j]]
            if e < 0 or not keep[m, j]:
                continue
            out[m] += (1.0 if weight_on_input else wts[m, j]) * Y[e, m]
    return out, ids, wts


def dense_mlp(x, w1, w2):
    """The one-expert gated MLP applied to all rows (shared expert)."""
    x = np.asarray(x, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    I = w1.shape[0] // 2
    H = x @ w1.T
    return gated(H[:, :I], H[:, I:]) @ w2.T
