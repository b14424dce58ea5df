"""Seeded synthetic inputs for KDA chunked prefill and decode (test and bench infrastructure).

This module only draws random tensors with the shapes and value distributions of
the KDA prefill workloads; it holds no step of the delta-rule arithmetic, so both
the HIP path and the oracle may take their inputs from it.

Value recipe (the reading of the workloads; the pages fix only the gate floor):
  * q, k ~ N(0, 1), L2-normalised over the key channels per (token, head) in
    float32, then rounded to the compute dtype (bf16 round-to-nearest-even);
  * v ~ N(0, 1), rounded to the compute dtype;
  * g = -5 * sigmoid(N(0, 1)) in float32: a per-token, per-channel log decay in
    [-5, 0].  -5 is the production ``gate_lower_bound`` the cudnn-frontend
    Hopper KDA prefill PR (#1056, description and "Correctness") measures at;
  * beta = sigmoid(N(0, 1)) in float32, already a value in (0, 1) (the
    TensorRT-LLM KDA prefill fix PR #19826 names a beta-sigmoid test);
  * initial state ~ N(0, 0.1^2) in float32 (sigma = 0.1), or zeros;
  * the long-sequence workload pins 13 of 128 channels of every head at exactly
    g = -5 for every token (10% of channels at the gate floor).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

GATE_LOWER_BOUND = -5.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    lengths: tuple          # per-sequence token counts
    H: int
    D: int                  # d_k == d_v
    dtype: str              # "bf16" or "f32" for q, k, v, out
    dense: bool             # [B, T, H, D] tensors (equal lengths) or packed + cu_seqlens
    zero_state: bool = False
    floor_channels: int = 0  # channels per head pinned at g = -5
    seed: int = 0

    @property
    def n_seq(self) -> int:
        return len(self.lengths)

    @property
    def tokens(self) -> int:
        return int(sum(self.lengths))

    def describe(self) -> dict:
        return {"workload": self.name, "n_seq": self.n_seq, "tokens": self.tokens,
                "H": self.H, "d_k": self.D, "d_v": self.D, "dtype": self.dtype,
                "layout": "dense" if self.dense else "packed",
                "initial_state": "zeros" if self.zero_state else "N(0,0.1^2)",
                "seed": self.seed}


def varlen_lengths(seed: int = 14, n: int = 8, hi: int = 8192) -> List[int]:
    """Eight lengths uniform in [1, 8192]; seed 14 gives a ~32K-token total."""
    return [int(x) for x in np.random.default_rng(seed).integers(1, hi + 1, n)]


WORKLOADS = {
    "tiny": Workload("tiny", (256,), H=2, D=64, dtype="f32", dense=True, zero_state=True),
    "eqlen": Workload("eqlen", (4096,) * 2, H=16, D=128, dtype="bf16", dense=True),
    "varlen": Workload("varlen", tuple(varlen_lengths()), H=32, D=128, dtype="bf16", dense=False),
    "varlen_padded": Workload("varlen_padded", (4000,) * 8, H=32, D=128, dtype="bf16", dense=True),
    # the varlen lengths at 64 heads: 512 chains on 256 CUs, where the chain order matters
    "varlen_h64": Workload("varlen_h64", tuple(varlen_lengths()), H=64, D=128, dtype="bf16", dense=False),
    "long": Workload("long", (65536,), H=8, D=128, dtype="bf16", dense=True, floor_channels=13),
    "large": Workload("large", (8192,) * 16, H=64, D=128, dtype="bf16", dense=True),
    # 256 and 288 equal chains: one full round of the CUs, and a full round plus 32 chains
    # (the planner then segments only those 32)
    "eqlen256": Workload("eqlen256", (4096,) * 8, H=32, D=128, dtype="bf16", dense=True),
    "eqlen288": Workload("eqlen288", (4096,) * 9, H=32, D=128, dtype="bf16", dense=True),
}


def custom(lengths, H=2, D=128, dtype="bf16", dense=False, zero_state=False,
           floor_channels=0, seed=0, name="custom") -> Workload:
    return Workload(name, tuple(int(x) for x in lengths), H=H, D=D, dtype=dtype, dense=dense,
                    zero_state=zero_state, floor_channels=floor_channels, seed=seed)


def _torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def make_inputs(w: Workload, device="cpu", gate: Optional[str] = None) -> dict:
    """Draw the inputs of workload ``w`` on ``device`` from a torch generator seeded
    with ``w.seed``.  Returns a dict with q, k, v, g, beta, initial_state (or None),
    cu_seqlens (int32, or None in dense layout) and lengths.

    ``gate`` overrides the gate distribution for edge cases: "floor" sets every g
    to -5, "zero" sets every g to 0, "mild" scales the drawn g by 0.01 (slow decay,
    so a state carries across many chunks).

    ``g_logits`` and ``beta_logits`` hold the normal draws the gates and betas are
    the activations of (g = -5 sigmoid(g_logits), beta = sigmoid(beta_logits)); a
    gate pinned at -5 has the logit 30 and a zero gate -1e4, whose fp32 activations
    are exactly -5 and 0.  Under "mild" there is no such logit and g_logits is None.
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    N, H, D = w.n_seq, w.H, w.D
    T_tot = w.tokens
    dt = _torch_dtype(w.dtype)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)

    def unit_rows(x):
        return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)

    q = unit_rows(randn(T_tot, H, D)).to(dt)
    k = unit_rows(randn(T_tot, H, D)).to(dt)
    v = randn(T_tot, H, D).to(dt)
    g_logits = randn(T_tot, H, D)
    g = GATE_LOWER_BOUND * torch.sigmoid(g_logits)
    beta_logits = randn(T_tot, H)
    beta = torch.sigmoid(beta_logits)
    # logits whose fp32 activation lands on the bound or on zero exactly
    LOGIT_AT_BOUND, LOGIT_AT_ZERO = 30.0, -1.0e4
    if w.floor_channels:
        for h in range(H):
            ch = torch.randperm(D, generator=gen, device=dev)[: w.floor_channels]
            g[:, h, ch] = GATE_LOWER_BOUND
            g_logits[:, h, ch] = LOGIT_AT_BOUND
    if gate == "floor":
        g.fill_(GATE_LOWER_BOUND)
        g_logits.fill_(LOGIT_AT_BOUND)
    elif gate == "zero":
        g.zero_()
        g_logits.fill_(LOGIT_AT_ZERO)
    elif gate == "mild":
        g.mul_(0.01)
        g_logits = None
    s0 = None if w.zero_state else 0.1 * randn(N, H, D, D)

    out = {"lengths": list(w.lengths), "initial_state": s0}
    if w.dense:
        L = w.lengths[0]
        assert all(x == L for x in w.lengths), "dense layout needs equal lengths"
        out.update(q=q.view(N, L, H, D), k=k.view(N, L, H, D), v=v.view(N, L, H, D),
                   g=g.view(N, L, H, D), beta=beta.view(N, L, H), cu_seqlens=None,
                   g_logits=None if g_logits is None else g_logits.view(N, L, H, D),
                   beta_logits=beta_logits.view(N, L, H))
    else:
        cu = torch.zeros(N + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(w.lengths, dtype=torch.int64), 0).to(torch.int32)
        out.update(q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu.to(dev), g_logits=g_logits, beta_logits=beta_logits)
    return out


def to_packed(x: torch.Tensor) -> torch.Tensor:
    """[B, T, ...] -> [B*T, ...] (a view change only)."""
    return x.reshape(x.shape[0] * x.shape[1], *x.shape[2:])


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """R requests of T tokens each against a pool of P state slots (every request
    names its own slot), the decode / draft-verify shape of KDA serving."""
    name: str
    R: int
    T: int
    H: int
    D: int
    pool_dtype: str         # "f32" or "bf16"
    P: int
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.R * self.T

    def describe(self) -> dict:
        return {"workload": self.name, "requests": self.R, "tokens_per_request": self.T, "H": self.H,
                "d_k": self.D, "d_v": self.D, "dtype": "bf16", "state_pool": self.pool_dtype,
                "pool_slots": self.P, "state_update": True, "seed": self.seed}


DECODE_WORKLOADS = {
    "decode": DecodeWorkload("decode", R=256, T=1, H=32, D=128, pool_dtype="f32", P=512),
    "decode_bf16": DecodeWorkload("decode_bf16", R=256, T=1, H=32, D=128, pool_dtype="bf16", P=512),
    "verify4": DecodeWorkload("verify4", R=256, T=4, H=32, D=128, pool_dtype="f32", P=512),
}


def make_decode_inputs(w: DecodeWorkload, device="cpu") -> dict:
    """q, k, v, g, beta [R, T, H, D] in the prefill recipe (a dense workload of R
    equal-length sequences), a pool of P states ~ N(0, 0.1^2) in the pool dtype,
    and a seeded permutation of slots as int32 state indices."""
    x = make_inputs(custom([w.T] * w.R, H=w.H, D=w.D, dtype="bf16", dense=True, seed=w.seed), device=device)
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 1)
    pool = 0.1 * torch.randn(w.P, w.H, w.D, w.D, generator=gen, device=dev, dtype=torch.float32)
    pool = pool.to(_torch_dtype(w.pool_dtype))
    idx = torch.randperm(w.P, generator=gen, device=dev)[: w.R].to(torch.int32)
    return {"q": x["q"], "k": x["k"], "v": x["v"], "g": x["g"], "beta": x["beta"], "pool": pool, "idx": idx}
