"""KDA prefill oracle: plain, slow, obviously correct float64 CPU code.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  It
shares no code with the HIP path (``gated_delta_rule_38_amd``) and neither
imports the other.

Contents
  * ``recurrence``      -- numpy float64 token-by-token gated delta rule;
  * ``run_c``           -- the same recurrence in C (``kda_oracle.c``), OpenMP
                           over (sequence, head) chains, for the large workloads;
  * ``chunked.chunked`` -- a brute-force float64 chunked (WY/UT) form used only
                           to pin the oracle and the chunk algebra (pin P7);
  * ``activations``     -- float64 gate and beta activations for inputs given
                           as logits (g = lower_bound * sigmoid(x), beta =
                           sigmoid(b)), applied before the recurrence;
  * ``gated_rmsnorm``   -- the float64 output epilogue: RMS normalisation of
                           each (token, head) output row, a per-channel weight
                           and a sigmoid output gate;
  * ``rel_l2``          -- the parity metric, ||x - ref||_2 / ||ref||_2 over the
                           whole tensor in float64.

The method (the reading of the pages, which name Kimi Delta Attention and its
a WY-form chunk but never print the recurrence): per sequence n and head h,
    S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = S_t^T q_t,
S_{-1} = initial state (zeros if None); the final state is S after the last
token.  Zero-length sequences give no output rows and a final state equal to
the initial state.

Every function here is pinned by ``tests/test_oracle.py`` (closed forms, the
textbook delta rule, linearity, split invariance, the chunked twin, packing
independence, the dense [B, T, H, D] layout against hand-built packed input;
the metric against hand-worked values), and each group of pins is shown to
catch planted mistakes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile kda_oracle.c with gcc (IEEE float64, no fast-math) into oracle/."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.kda_oracle_f64.restype = ctypes.c_int
        P = ctypes.c_void_p
        lib.kda_oracle_f64.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       P, P, P, P, P, P, P, P, P, ctypes.c_int, P]
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Host float64 copy of a numpy array or a (CPU) torch tensor, any dtype."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _cu(cu_seqlens, T: int) -> np.ndarray:
    if cu_seqlens is None:
        return np.array([0, T], dtype=np.int64)
    if hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))


def _packed(q, k, v, g, beta, s0, cu_seqlens):
    """Accept dense [B, T, H, D] (cu_seqlens None) or packed [T, H, D] inputs."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    if q.ndim == 4:
        B, T = q.shape[:2]
        q, k, v, g = (x.reshape(B * T, *x.shape[2:]) for x in (q, k, v, g))
        beta = beta.reshape(B * T, beta.shape[-1])
        cu = np.arange(B + 1, dtype=np.int64) * T if cu_seqlens is None else _cu(cu_seqlens, B * T)
    else:
        cu = _cu(cu_seqlens, q.shape[0])
    s0 = None if s0 is None else _f64(s0)
    return q, k, v, g, beta, s0, cu


def recurrence(q, k, v, g, beta, initial_state=None, cu_seqlens=None):
    """numpy float64 token loop.  Returns (o [T, H, DV], final_state [N, H, DK, DV])
    in packed layout (dense inputs are flattened to [B*T, H, D])."""
    q, k, v, g, beta, s0, cu = _packed(q, k, v, g, beta, initial_state, cu_seqlens)
    T, H, DK = q.shape
    DV = v.shape[-1]
    N = len(cu) - 1
    o = np.zeros((T, H, DV))
    sT = np.zeros((N, H, DK, DV))
    for n in range(N):
        for h in range(H):
            S = np.zeros((DK, DV)) if s0 is None else s0[n, h].copy()
            for t in range(cu[n], cu[n + 1]):
                S = np.exp(g[t, h])[:, None] * S                       # Diag(exp g_t) S_{t-1}
                r = k[t, h] @ S                                         # k_t^T D S_{t-1}
                S = S + beta[t, h] * np.outer(k[t, h], v[t, h] - r)     # (I - b k k^T) D S + b k v^T
                o[t, h] = S.T @ q[t, h]                                 # o_t = S_t^T q_t
            sT[n, h] = S
    return o, sT


def run_c(q, k, v, g, beta, initial_state=None, cu_seqlens=None, threads: int = 0,
          return_threads: bool = False):
    """The C float64 oracle (same recurrence), OpenMP over chains."""
    q, k, v, g, beta, s0, cu = _packed(q, k, v, g, beta, initial_state, cu_seqlens)
    T, H, DK = q.shape
    DV = v.shape[-1]
    N = len(cu) - 1
    o = np.zeros((T, H, DV))
    sT = np.zeros((N, H, DK, DV))
    used = ctypes.c_int(0)
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = _load().kda_oracle_f64(N, H, DK, DV, ptr(cu), ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta),
                                ptr(s0), ptr(o), ptr(sT), int(threads), ctypes.byref(used))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_f64 failed with code {rc}")
    if return_threads:
        return o, sT, used.value
    return o, sT


def activations(g_logits=None, beta_logits=None, lower_bound: float = -5.0):
    """Float64 activations for gate and beta inputs given as logits.

    The pages name a production gate lower bound of -5 (cudnn-frontend PR #1056,
    correctness section: its fp64 oracle runs at that production bound) and a
    beta-sigmoid prefill test (TensorRT-LLM PR #19826, description) but print
    no formula; the reading taken here is the plainest one consistent with a
    lower bound: the per-token, per-channel log decay is lower_bound * sigmoid(x),
    so it lies in [lower_bound, 0], and beta = sigmoid(b) lies in (0, 1).
    Returns (g, beta) as float64 arrays (None where the input is None).
    """
    def sigmoid(x):
        x = _f64(x)
        return 1.0 / (1.0 + np.exp(-x))
    g = None if g_logits is None else float(lower_bound) * sigmoid(g_logits)
    beta = None if beta_logits is None else sigmoid(beta_logits)
    return g, beta


def gated_rmsnorm(o, z, weight, eps: float):
    """Float64 gated RMS normalisation of output rows.

    TensorRT-LLM PR #19960 lists a fused attention epilogue with a gated RMSNorm
    on the KDA output but prints no formula; the reading taken here is the plain
    gated RMSNorm: for every token and head, over the value channels c,
        y_c = o_c / sqrt(mean_c(o_c^2) + eps) * weight_c * sigmoid(z_c).
    o, z: [..., V] (any leading shape); weight: [V].  Returns float64 [..., V].
    """
    o, z, w = _f64(o), _f64(z), _f64(weight)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + float(eps))
    return o * r * w * (1.0 / (1.0 + np.exp(-z)))


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole tensor, accumulated in float64."""
    x = _f64(x).ravel()
    ref = _f64(ref).ravel()
    den = float(np.sqrt(np.dot(ref, ref)))
    num = float(np.sqrt(np.dot(x - ref, x - ref)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
