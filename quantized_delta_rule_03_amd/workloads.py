"""Seeded synthetic inputs for the five workloads of the decode path.

This module is shared by the tests, the benchmark and the oracle-side checks. It
only draws random numbers and shapes them; it holds none of the method's
arithmetic (no state update, no quantization, no bit assignment). The gate values
it derives from drawn half-lives (a = 2^(-1/tau)) and drawn logits
(a = exp(-softplus(x))) are inputs of the method, not steps of it.

Seeding: every array comes from ``numpy.random.default_rng(SeedSequence(key))``
with ``key = [seed, workload_id, stream, ...]``; stream 0 = static draws
(half-lives: [..., 0, 0]; outlier masks: [..., 0, 1, request]), 1 = decode-step
inputs ([..., 1, step, request]), 2 = pre-warm inputs ([..., 2, step, request]).
Inside a request's step the draw order is k, q, v, b, x.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

GDN = 0
KDA = 1

DK = 128
DV = 128


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    n_req: int
    n_head: int
    steps: int
    gate: int
    bits_policy: str        # "uniform8" or "quartile"
    tau_max: Optional[float]  # half-life range upper end (log-uniform in [1, tau_max])
    per_step_gate: bool      # gate drawn per step (exp(-softplus(x))) vs fixed from tau
    prewarm_steps: int = 0
    outlier_frac: float = 0.0
    window: int = 0

    @property
    def n_unit(self):
        return self.n_req * self.n_head


WORKLOADS = {
    0: Workload(0, "gdn_single_head_8bit", 1, 1, 64, GDN, "uniform8", None, True),
    1: Workload(1, "gdn_32h_b64_mixed", 64, 32, 256, GDN, "quartile", 4096.0, False),
    2: Workload(2, "kda_32h_b256_mixed_prewarm", 256, 32, 256, KDA, "quartile", 8192.0, False,
                prewarm_steps=512, outlier_frac=0.01),
    3: Workload(3, "gdn_serving_1024req_32h_mixed", 1024, 32, 128, GDN, "quartile", 4096.0,
                False),
    4: Workload(4, "kda_window64_b256_8bit", 256, 32, 1024, KDA, "uniform8", 8192.0, False,
                prewarm_steps=512, outlier_frac=0.01, window=64),
}


def _rng(seed, wid, stream, *index):
    key = [int(seed), int(wid), int(stream)] + [int(i) for i in index]
    return np.random.default_rng(np.random.SeedSequence(key))


def _unit_normal_rows(rng, shape):
    """N(0,1) vectors along the last axis, L2-normalised in fp64, rounded to fp32."""
    x = rng.standard_normal(shape)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x.astype(np.float32)


def halflives(w: Workload, seed: int = 0) -> Optional[np.ndarray]:
    """Gate half-lives (tokens), log-uniform in [1, tau_max].

    GDN: one per head [n_head]; KDA: one per key channel [n_head, DK]. Fixed across
    requests and steps. None for a per-step gate.
    """
    if w.per_step_gate:
        return None
    rng = _rng(seed, w.wid, 0, 0)
    shape = (w.n_head,) if w.gate == GDN else (w.n_head, DK)
    return np.exp(rng.uniform(0.0, np.log(w.tau_max), size=shape))


def gate_from_halflife(tau: np.ndarray) -> np.ndarray:
    """a = 2^(-1/tau) (so that a^tau = 1/2), computed in fp64, stored as fp32."""
    return np.power(2.0, -1.0 / np.asarray(tau, np.float64)).astype(np.float32)


def static_gate(w: Workload, seed: int = 0, n_req: Optional[int] = None) -> Optional[np.ndarray]:
    """The fixed gate tensor as the decode call takes it: GDN [n_req, n_head], KDA
    [n_req, n_head, DK] (the same values for every request)."""
    tau = halflives(w, seed)
    if tau is None:
        return None
    n_req = w.n_req if n_req is None else n_req
    a = gate_from_halflife(tau)
    return np.ascontiguousarray(np.broadcast_to(a, (n_req,) + a.shape))


def uniform_bits(n_head: int, width: int = 8) -> np.ndarray:
    return np.full((n_head, DK), width, np.uint8)


def step_inputs(w: Workload, step: int, seed: int = 0, n_req: Optional[int] = None,
                stream: int = 1, r0: int = 0) -> dict:
    """Inputs of decode step ``step`` for requests [r0, r0 + n_req).

    q, k: [n_req, n_head, DK] unit-norm; v: [n_req, n_head, DV] ~ N(0,1);
    b: [n_req, n_head] ~ U(0,1); a: the gate (per-step exp(-softplus(x)) for a
    per-step-gate workload, else the fixed gate). Each request draws from its own
    seed key [seed, workload, stream, step, request], so any subset of requests gets
    exactly the values it has in the full-size run.
    """
    n = (w.n_req - r0) if n_req is None else n_req
    H = w.n_head
    out = {"q": np.empty((n, H, DK), np.float32), "k": np.empty((n, H, DK), np.float32),
           "v": np.empty((n, H, DV), np.float32), "b": np.empty((n, H), np.float32)}
    x = np.empty((n, H), np.float64)
    for i in range(n):
        rng = _rng(seed, w.wid, stream, step, r0 + i)
        out["k"][i] = _unit_normal_rows(rng, (H, DK))
        out["q"][i] = _unit_normal_rows(rng, (H, DK))
        out["v"][i] = rng.standard_normal((H, DV))
        out["b"][i] = rng.uniform(0.0, 1.0, size=H)
        x[i] = rng.standard_normal(H)
    if w.per_step_gate:
        # a = exp(-softplus(x)) = 1 / (1 + e^x), evaluated in fp64
        out["a"] = np.exp(-np.logaddexp(0.0, x)).astype(np.float32)
    else:
        out["a"] = static_gate(w, seed, n)
    return {kk: np.ascontiguousarray(vv) for kk, vv in out.items()}


def prewarm_inputs(w: Workload, step: int, seed: int = 0, n_req: Optional[int] = None,
                   r0: int = 0) -> dict:
    """Inputs of pre-warm step ``step`` (same distributions, stream 2)."""
    return step_inputs(w, step, seed, n_req, stream=2, r0=r0)


def outlier_masks(w: Workload, seed: int = 0, n_req: Optional[int] = None, r0: int = 0):
    """Boolean masks selecting outlier key channels [n_req, n_head, DK] and value rows
    [n_req, n_head, DV], each entry independently with probability outlier_frac."""
    n = (w.n_req - r0) if n_req is None else n_req
    key_sel = np.empty((n, w.n_head, DK), bool)
    val_sel = np.empty((n, w.n_head, DV), bool)
    for i in range(n):
        rng = _rng(seed, w.wid, 0, 1, r0 + i)
        key_sel[i] = rng.uniform(size=(w.n_head, DK)) < w.outlier_frac
        val_sel[i] = rng.uniform(size=(w.n_head, DV)) < w.outlier_frac
    return key_sel, val_sel


def device_step_inputs(w: Workload, step: int, device, seed: int = 0):
    """Full-size step inputs drawn on the GPU with a seeded torch generator (for the
    timed benchmark, where host generation of many steps would dominate set-up).
    Same distributions as ``step_inputs``; not bit-identical to it."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1000003 + w.wid * 7919 + int(step)) & 0x7FFFFFFFFFFF)
    full = (w.n_req, w.n_head)

    def unit(shape):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float64)
        x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x.to(torch.float32).contiguous()

    k = unit(full + (DK,))
    q = unit(full + (DK,))
    v = torch.randn(full + (DV,), generator=g, device=device, dtype=torch.float32)
    b = torch.rand(full, generator=g, device=device, dtype=torch.float32)
    return {"q": q, "k": k, "v": v, "b": b}
