"""Seeded synthetic inputs for the SSD forward scan and the decode step.

This module only draws random numbers and rounds them to their storage type;
it holds none of the scan's arithmetic.  The same draws feed the GPU library
and the CPU checks, so both sides consume bit-identical inputs.

Distributions (the N(mu, s) of the workload descriptions is read with s the
variance, so B and C have standard deviation 1/sqrt(N) and the initial state
standard deviation sqrt(0.1)):

    x ~ N(0, 1)                    dt = softplus(z + dt_shift), z ~ N(0, 1)
    A = -exp(U(0, a_hi)) per head  B, C ~ N(0, 1/N)       D ~ N(0, 1)
    init ~ N(0, init_var) or absent

Inputs of the block around the scan (``make_layer_inputs``):

    xbc ~ N(0, 1) over the H P + 2 G N channels   z ~ N(0, 1)
    conv_w ~ N(0, 1/K), conv_b ~ N(0, 0.1)       dt_raw ~ N(dt_shift, 1)
    dt_bias ~ N(0, 0.1); A, D as above

Seeding: the per-head parameters and the initial state come from
``numpy.random.default_rng(seed)``; the per-token arrays are drawn in slabs of
at most 65,536 tokens, slab ``s`` of batch row ``b`` from
``default_rng([seed, b, s])``, in the order x, z, B, C.  Values are drawn in
fp64, rounded once to fp32 and then, for bf16 storage, to bf16 with
round-to-nearest-even (torch's conversion).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

SLAB = 65536


@dataclass(frozen=True)
class ForwardSpec:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str            # "f32" or "bf16": storage type of x, B, C and y
    dt_shift: float = -2.0
    a_hi: float = 1.5
    init_var: float = 0.0
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def with_(self, **kw) -> "ForwardSpec":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeSpec:
    name: str
    batch: int
    steps: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    dtype: str
    dt_shift: float = -2.0
    a_hi: float = 1.5
    init_var: float = 0.1
    seed: int = 0

    def with_(self, **kw) -> "DecodeSpec":
        return replace(self, **kw)


# The five workloads: a tiny fp32 case, a Mamba-2-130M-shaped layer, a
# Mamba-2-2.7B-shaped layer (the headline throughput workload), a one-million
# token long-context layer with 8 B/C groups, and batch-256 decode.
TINY_F32 = ForwardSpec("tiny_f32_b1_l256_h1_p16_n16", 1, 256, 1, 16, 16, 1, 64, "f32",
                       seed=1001)
MAMBA2_130M = ForwardSpec("mamba2_130m_b8_l2048_h24_p64_n128", 8, 2048, 24, 64, 128, 1, 256,
                          "bf16", seed=1002)
MAMBA2_2P7B = ForwardSpec("mamba2_2p7b_b4_l8192_h80_p64_n128", 4, 8192, 80, 64, 128, 1, 256,
                          "bf16", init_var=0.1, seed=1003)
LONG_1M = ForwardSpec("long_b1_l1048576_h32_p64_n128_g8", 1, 1 << 20, 32, 64, 128, 8, 256,
                      "bf16", dt_shift=-4.0, a_hi=1.0, seed=1004)
DECODE_B256 = DecodeSpec("decode_b256_s64_h80_p64_n128", 256, 64, 80, 64, 128, 1, "bf16",
                         init_var=0.1, seed=1005)

FORWARD_SPECS = {s.name: s for s in (TINY_F32, MAMBA2_130M, MAMBA2_2P7B, LONG_1M)}


def _softplus(z):
    return np.log1p(np.exp(z))


def _store(a64: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(f"unknown storage type {dtype!r}")


def _head_params(rng, H, a_hi):
    u = rng.uniform(0.0, a_hi, size=H)
    A = -np.exp(u)
    D = rng.standard_normal(H)
    return A, D


def make_forward_inputs(spec: ForwardSpec) -> dict:
    """CPU tensors: x [B,L,H,P], dt [B,L,H] f32, A [H] f32, B, C [B,L,G,N],
    D [H] f32, init [B,H,P,N] f32 or None."""
    Bt, L, H, P, N, G = spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate, spec.ngroups
    sd = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    rng = np.random.default_rng(spec.seed)
    A, D = _head_params(rng, H, spec.a_hi)
    init = None
    if spec.init_var > 0:
        init = _store(rng.standard_normal((Bt, H, P, N)) * math.sqrt(spec.init_var), "f32")
    x = torch.empty((Bt, L, H, P), dtype=sd)
    dt = torch.empty((Bt, L, H), dtype=torch.float32)
    Bm = torch.empty((Bt, L, G, N), dtype=sd)
    Cm = torch.empty((Bt, L, G, N), dtype=sd)
    bc_std = math.sqrt(1.0 / N)
    for b in range(Bt):
        for s, t0 in enumerate(range(0, L, SLAB)):
            n = min(SLAB, L - t0)
            r = np.random.default_rng([spec.seed, b, s])
            x[b, t0:t0 + n] = _store(r.standard_normal((n, H, P)), spec.dtype)
            dt[b, t0:t0 + n] = _store(_softplus(r.standard_normal((n, H)) + spec.dt_shift), "f32")
            Bm[b, t0:t0 + n] = _store(r.standard_normal((n, G, N)) * bc_std, spec.dtype)
            Cm[b, t0:t0 + n] = _store(r.standard_normal((n, G, N)) * bc_std, spec.dtype)
    return dict(x=x, dt=dt, A=_store(A, "f32"), B=Bm, C=Cm, D=_store(D, "f32"), init=init)


def make_decode_static(spec: DecodeSpec) -> dict:
    """A [H], D [H] (f32) and the initial state [batch,H,P,N] f32."""
    rng = np.random.default_rng(spec.seed)
    A, D = _head_params(rng, spec.nheads, spec.a_hi)
    state = rng.standard_normal((spec.batch, spec.nheads, spec.headdim, spec.dstate))
    state = _store(state * math.sqrt(spec.init_var), "f32")
    return dict(A=_store(A, "f32"), D=_store(D, "f32"), state=state)


def make_decode_step(spec: DecodeSpec, t: int) -> dict:
    """Per-step inputs of step t: x_t [batch,H,P], dt_t [batch,H] f32,
    B_t, C_t [batch,G,N]; drawn from default_rng([seed, t])."""
    r = np.random.default_rng([spec.seed, t])
    Bt, H, P, N, G = spec.batch, spec.nheads, spec.headdim, spec.dstate, spec.ngroups
    bc_std = math.sqrt(1.0 / N)
    return dict(
        x=_store(r.standard_normal((Bt, H, P)), spec.dtype),
        dt=_store(_softplus(r.standard_normal((Bt, H)) + spec.dt_shift), "f32"),
        B=_store(r.standard_normal((Bt, G, N)) * bc_std, spec.dtype),
        C=_store(r.standard_normal((Bt, G, N)) * bc_std, spec.dtype),
    )


def make_layer_inputs(spec: ForwardSpec, kernel_width: int = 4) -> dict:
    """CPU tensors for the block around the scan: xbc [B,L,H*P+2*G*N] and
    z [B,L,H,P] in the storage type; conv_w [Cd,K], conv_b [Cd], dt_raw [B,L,H],
    dt_bias [H], A [H], D [H] (f32); init [B,H,P,N] f32 or None.

    Per-head and per-channel parameters come from default_rng([seed, K]) in
    the order A, D, dt_bias, conv_w, conv_b, init; per-token arrays in slabs
    from default_rng([seed, K, b, s]) in the order xbc, dt_raw, z."""
    Bt, L, H, P, N, G = spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate, spec.ngroups
    K = int(kernel_width)
    Cd = H * P + 2 * G * N
    sd = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    rng = np.random.default_rng([spec.seed, K])
    A, D = _head_params(rng, H, spec.a_hi)
    dt_bias = rng.standard_normal(H) * math.sqrt(0.1)
    conv_w = rng.standard_normal((Cd, K)) * math.sqrt(1.0 / K)
    conv_b = rng.standard_normal(Cd) * math.sqrt(0.1)
    init = None
    if spec.init_var > 0:
        init = _store(rng.standard_normal((Bt, H, P, N)) * math.sqrt(spec.init_var), "f32")
    xbc = torch.empty((Bt, L, Cd), dtype=sd)
    dt_raw = torch.empty((Bt, L, H), dtype=torch.float32)
    z = torch.empty((Bt, L, H, P), dtype=sd)
    for b in range(Bt):
        for s, t0 in enumerate(range(0, L, SLAB)):
            n = min(SLAB, L - t0)
            r = np.random.default_rng([spec.seed, K, b, s])
            xbc[b, t0:t0 + n] = _store(r.standard_normal((n, Cd)), spec.dtype)
            dt_raw[b, t0:t0 + n] = _store(r.standard_normal((n, H)) + spec.dt_shift, "f32")
            z[b, t0:t0 + n] = _store(r.standard_normal((n, H, P)), spec.dtype)
    return dict(xbc=xbc, z=z, conv_w=_store(conv_w, "f32"), conv_b=_store(conv_b, "f32"),
                dt_raw=dt_raw, dt_bias=_store(dt_bias, "f32"), A=_store(A, "f32"),
                D=_store(D, "f32"), init=init)
