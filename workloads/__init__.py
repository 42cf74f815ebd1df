"""Seeded synthetic inputs for the fused MoE layer.

This module only draws random tensors of the right shapes, dtypes and
distributions.  It holds none of the layer's arithmetic (no routing, counting,
permutation, GEMM or combine) and is the one piece of code that both the CPU
oracle (``oracle/``) and the HIP path (``combine_topk_softmax_amd``) are fed
from.

Workloads (sizes follow the fused-MoE problem tuple ``(E, M, N, K, topk)`` of
the modular-kernel page, ``_moe_problem_size``; N = 2*I, gate rows first):

===================  =====  ====  =====  ===  ==  ========================  =========
name                 M      K     I      E    k   routing                   precision
===================  =====  ====  =====  ===  ==  ========================  =========
tiny_fp32            64     256   128    8    2   softmax, N(0,1) logits    fp32
mixtral_bf16         512    4096  14336  8    2   softmax+renorm, U[0,1)    bf16
dsv3_bf16            4096   7168  2048   256  8   sigmoid+renorm, N(0,1)    bf16 (+ shared expert I=2048)
decode_fp8_m64       64     7168  2048   32   8   softmax, N(0,1)           fp8 batched, cap = 8*M
decode_fp8_m256      256    7168  2048   32   8   softmax, N(0,1)           fp8 batched, cap = 8*M
skewed_bf16          16384  4096  1536   128  8   softmax, Zipf(1.2) bias   bf16
===================  =====  ====  =====  ===  ==  ========================  =========

x ~ N(0, 1); expert weights ~ N(0, 0.02) (0.02 is the standard deviation).
bf16 tensors are fp32 draws rounded to nearest-even.  fp8 weights are the
same draws stored as OCP e4m3fn codes with one fp32 scale per 128x128 block
(scale = block amax / 448), encoded with torch's own float8_e4m3fn cast.

Each tensor has its own generator, seeded from (seed, tensor name), so a tensor
does not change when another one is added or resized.  Generators are torch's:
the CPU stream for small workloads and tests, the device stream when the
tensors are made on the GPU (large weights); either way the same tensor object
is handed to both sides of a parity check.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional

import torch

# Values of the problem-struct enums (mirrored by include/moe.h).
FORMAT_STANDARD, FORMAT_BATCHED = 0, 1
DTYPE_F32, DTYPE_BF16, DTYPE_FP8 = 0, 1, 2
QUANT_NONE, QUANT_FP8_G128 = 0, 1
SCORING_SOFTMAX, SCORING_SIGMOID = 0, 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    I: int
    E: int
    topk: int
    scoring: int = SCORING_SOFTMAX
    renormalize: bool = False
    act_dtype: int = DTYPE_BF16
    w_dtype: int = DTYPE_BF16
    act_quant: int = QUANT_NONE
    format: int = FORMAT_STANDARD
    capacity: int = 0            # batched: max tokens per expert
    logits_dist: str = "normal"  # normal | uniform | zipf
    zipf_s: float = 1.2
    shared_I: int = 0            # >0: one always-on shared expert of this size
    global_E: int = 0            # >0: experts in the global space (router width); E are local
    activation: int = 0          # 0 silu_and_mul, 1 gelu_and_mul
    router_weight_on_input: bool = False   # topk == 1 only

    @property
    def N(self) -> int:
        return 2 * self.I

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def gemm_flops(self) -> int:
        """Flops of the two routed expert GEMMs over the M*topk real rows."""
        return 2 * self.M * self.topk * 3 * self.I * self.K

    def shared_flops(self) -> int:
        return 2 * self.M * 3 * self.shared_I * self.K if self.shared_I else 0


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_fp32", M=64, K=256, I=128, E=8, topk=2,
                 act_dtype=DTYPE_F32, w_dtype=DTYPE_F32),
        Workload("mixtral_bf16", M=512, K=4096, I=14336, E=8, topk=2,
                 renormalize=True, logits_dist="uniform"),
        Workload("dsv3_bf16", M=4096, K=7168, I=2048, E=256, topk=8,
                 scoring=SCORING_SIGMOID, renormalize=True, shared_I=2048),
        Workload("decode_fp8_m64", M=64, K=7168, I=2048, E=32, topk=8,
                 w_dtype=DTYPE_FP8, act_quant=QUANT_FP8_G128,
                 format=FORMAT_BATCHED, capacity=64 * 8),
        Workload("decode_fp8_m256", M=256, K=7168, I=2048, E=32, topk=8,
                 w_dtype=DTYPE_FP8, act_quant=QUANT_FP8_G128,
                 format=FORMAT_BATCHED, capacity=256 * 8),
        Workload("skewed_bf16", M=16384, K=4096, I=1536, E=128, topk=8,
                 logits_dist="zipf"),
    ]
}


def _seed_for(seed: int, name: str) -> int:
    h = hashlib.sha256(f"{seed}/{name}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 62) - 1)


def generator(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed_for(seed, name))
    return g


def _torch_dtype(code: int):
    return {DTYPE_F32: torch.float32, DTYPE_BF16: torch.bfloat16}[code]


def make_logits(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """Router logits [M, router width], fp32 (the router width is global_E when set, else E)."""
    g = generator(seed, "logits", device)
    E = w.global_E or w.E
    if w.logits_dist == "normal":
        return torch.randn(w.M, E, generator=g, device=device)
    if w.logits_dist == "uniform":
        return torch.rand(w.M, E, generator=g, device=device)
    if w.logits_dist == "zipf":
        # Gumbel noise plus log-popularity: with p_r proportional to r^-s over a
        # seeded ranking of the experts, the arg-max of each row is distributed
        # exactly as p (Gumbel-max), so expert load follows Zipf(s).
        gp = generator(seed, "zipf-rank", "cpu")
        rank = torch.randperm(E, generator=gp).to(torch.float64) + 1.0
        p = rank ** (-w.zipf_s)
        logp = torch.log(p / p.sum()).to(torch.float32).to(device)
        u = torch.rand(w.M, E, generator=g, device=device)
        u = u.clamp_min(torch.finfo(torch.float32).tiny)
        gumbel = -torch.log(-torch.log(u))
        return (gumbel + logp[None, :]).contiguous()
    raise ValueError(w.logits_dist)


def make_x(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    g = generator(seed, "x", device)
    x = torch.randn(w.M, w.K, generator=g, device=device)
    return x.to(_torch_dtype(w.act_dtype))


def _expert_draws(n_exp: int, rows: int, cols: int, name: str, seed: int, device,
                  out_dtype) -> torch.Tensor:
    """N(0, 0.02) draws, one expert at a time (bounded fp32 temporaries)."""
    g = generator(seed, name, device)
    out = torch.empty(n_exp, rows, cols, dtype=out_dtype, device=device)
    for e in range(n_exp):
        out[e] = (torch.randn(rows, cols, generator=g, device=device) * 0.02).to(out_dtype)
    return out


def _fp8_block_encode(wf: torch.Tensor):
    """Store fp32 weights [n, R, C] as e4m3fn codes + one fp32 scale per 128x128 block."""
    n, R, C = wf.shape
    assert R % 128 == 0 and C % 128 == 0
    blk = wf.reshape(n, R // 128, 128, C // 128, 128)
    amax = blk.abs().amax(dim=(2, 4))                       # [n, R/128, C/128]
    scale = torch.clamp(amax, min=1e-10) / 448.0
    q = (blk / scale[:, :, None, :, None]).clamp(-448.0, 448.0)
    q = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, R, C)
    return q.contiguous(), scale.to(torch.float32).contiguous()


def _fp8_expert_draws(n_exp, rows, cols, name, seed, device):
    g = generator(seed, name, device)
    q = torch.empty(n_exp, rows, cols, dtype=torch.uint8, device=device)
    s = torch.empty(n_exp, rows // 128, cols // 128, dtype=torch.float32, device=device)
    for e in range(n_exp):
        wf = torch.randn(1, rows, cols, generator=g, device=device) * 0.02
        qe, se = _fp8_block_encode(wf)
        q[e], s[e] = qe[0], se[0]
    return q, s


def make_weights(w: Workload, seed: int = 0, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    """w1 [E, 2I, K] (gate rows then up rows), w2 [E, K, I]; fp8 adds block scales."""
    out: Dict[str, Optional[torch.Tensor]] = {"w1_scale": None, "w2_scale": None}
    if w.w_dtype == DTYPE_FP8:
        out["w1"], out["w1_scale"] = _fp8_expert_draws(w.E, w.N, w.K, "w1", seed, device)
        out["w2"], out["w2_scale"] = _fp8_expert_draws(w.E, w.K, w.I, "w2", seed, device)
    else:
        dt = _torch_dtype(w.w_dtype)
        out["w1"] = _expert_draws(w.E, w.N, w.K, "w1", seed, device, dt)
        out["w2"] = _expert_draws(w.E, w.K, w.I, "w2", seed, device, dt)
    if w.shared_I:
        dt = _torch_dtype(w.act_dtype)
        out["w1s"] = _expert_draws(1, 2 * w.shared_I, w.K, "w1s", seed, device, dt)[0]
        out["w2s"] = _expert_draws(1, w.K, w.shared_I, "w2s", seed, device, dt)[0]
    return out


def make_inputs(w: Workload, seed: int = 0, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    d = {"logits": make_logits(w, seed, device), "x": make_x(w, seed, device)}
    d.update(make_weights(w, seed, device))
    return d


def sample_tokens(M: int, n: int, seed: int = 0):
    """A seeded sorted sample of token rows that always includes the first and last."""
    if n >= M:
        return list(range(M))
    g = generator(seed, "sample", "cpu")
    idx = set(torch.randperm(M, generator=g)[: max(n - 2, 0)].tolist())
    idx.update({0, M - 1})
    return sorted(idx)
