"""Seeded synthetic inputs shaped like the workloads on the ManifoldKV and OjaKV
pages (long-context KV caches of a Llama-3.1-8B-shaped model: 32 layers, 8 KV
heads, 32 query heads, head dim 128).

This module only draws inputs.  It holds none of the method's arithmetic and
is shared by the oracle side and the HIP side of every test and benchmark; the
two sides never exchange values through it.

Every tensor is drawn slice by slice from a torch generator seeded with
``mix(seed, tag, slice)``, on whatever device the caller names, so any slice can
be regenerated alone.  bf16 tensors are produced by rounding fp32 draws to
nearest-even.  Distribution conventions: N(m, v) takes a variance (the per-channel
offsets use sigma = sqrt(2)); LogNormal(0, 0.25) is parameterised by the
underlying normal's mean and standard deviation.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BASE_SEED = 20261202
D_HEAD = 128

_TAGS = {"muK": 1, "muV": 2, "tok": 3, "scale": 4, "plant": 5, "seg": 6, "K": 7, "V": 8,
         "Q": 9, "muQ": 10, "U": 11, "Xt": 12, "dec": 13, "score": 14}


def mix(*parts: int) -> int:
    """SplitMix64-style mixing of integers into a 63-bit seed."""
    h = 0x9E3779B97F4A7C15
    for p in parts:
        h = (h ^ (int(p) & 0xFFFFFFFFFFFFFFFF)) * 0xBF58476D1CE4E5B9 & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 31
        h = h * 0x94D049BB133111EB & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 29
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(device, seed, tag, *idx):
    g = torch.Generator(device=device)
    g.manual_seed(mix(seed, _TAGS[tag], *idx))
    return g


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_bits(a: np.ndarray, device="cpu") -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).to(device)


# --------------------------------------------------------------- ManifoldKV


def manifold_global(L, B, H, S, D=D_HEAD, planted=16, seed=BASE_SEED, device="cpu"):
    """Key/value cache for global ManifoldKV scoring, [L*B*H, S, D] bf16 each.

    Per (layer, kv head): channel offsets mu^K, mu^V ~ N(0, 2).  Per token:
    a norm scale s_t ~ LogNormal(0, 0.25) shared by k_t and v_t and
    z ~ N(0, I); k_t = s_t (mu^K + z^K), v_t = s_t (mu^V + z^V).  ``planted``
    token positions per slice, uniform without replacement, are scaled x4 in
    both K and V.  Returns (K, V, planted_idx int64 [G, planted])."""
    G = L * B * H
    K = torch.empty((G, S, D), dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    plant = torch.empty((G, planted), dtype=torch.int64)
    sq2 = math.sqrt(2.0)
    for l in range(L):
        for h in range(H):
            muK = torch.randn(D, generator=_gen(device, seed, "muK", l, h), device=device) * sq2
            muV = torch.randn(D, generator=_gen(device, seed, "muV", l, h), device=device) * sq2
            for b in range(B):
                g = (l * B + b) * H + h
                gs = _gen(device, seed, "scale", g)
                s = torch.empty(S, device=device).log_normal_(0.0, 0.25, generator=gs)
                gt = _gen(device, seed, "tok", g)
                zk = torch.randn((S, D), generator=gt, device=device)
                zv = torch.randn((S, D), generator=gt, device=device)
                gp = _gen("cpu", seed, "plant", g)
                p = torch.randperm(S, generator=gp)[:planted].sort().values
                plant[g] = p
                mult = torch.ones(S, device=device)
                mult[p.to(device)] = 4.0
                sc = (s * mult)[:, None]
                K[g] = ((muK[None, :] + zk) * sc).to(torch.bfloat16)
                V[g] = ((muV[None, :] + zv) * sc).to(torch.bfloat16)
    return K, V, plant


def manifold_drifting(L, B, H, S, D=D_HEAD, segment=8192, seed=BASE_SEED, device="cpu"):
    """Drifting-mixture cache for windowed ManifoldKV, [L*B*H, S, D] bf16 each.

    Per (layer, kv head) the channel mean is redrawn, mu^(j) ~ N(0, 2), for every
    ``segment``-token stretch j; k_t ~ N(mu^(seg(t)), I), v_t likewise with its
    own means.  No norm scales and no planted outliers."""
    G = L * B * H
    K = torch.empty((G, S, D), dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    nseg = -(-S // segment)
    sq2 = math.sqrt(2.0)
    for l in range(L):
        for h in range(H):
            gm = _gen(device, seed, "seg", l, h)
            muK = torch.randn((nseg, D), generator=gm, device=device) * sq2
            muV = torch.randn((nseg, D), generator=gm, device=device) * sq2
            seg_of = torch.arange(S, device=device) // segment
            for b in range(B):
                g = (l * B + b) * H + h
                gt = _gen(device, seed, "tok", g)
                K[g] = (muK[seg_of] + torch.randn((S, D), generator=gt, device=device)).to(
                    torch.bfloat16)
                V[g] = (muV[seg_of] + torch.randn((S, D), generator=gt, device=device)).to(
                    torch.bfloat16)
    return K, V


# -------------------------------------------------------------------- OjaKV


def orthonormal_basis(D, R, seed, *idx):
    """Q factor (positive diagonal of R) of a seeded N(0,1) D x R matrix, fp32.
    Drawn on the host in float64 so that it is identical everywhere."""
    rng = np.random.Generator(np.random.Philox(mix(seed, _TAGS["U"], *idx)))
    A = rng.standard_normal((D, R))
    Q, Rm = np.linalg.qr(A)
    Q = Q * np.sign(np.diag(Rm))[None, :]
    return Q.astype(np.float32)


@dataclass
class OjaInputs:
    L: int
    B: int
    Hkv: int
    Hq: int
    S: int
    D: int
    R: int
    Wq: int
    K: torch.Tensor          # [L*B*Hkv, S_cap, D] bf16
    V: torch.Tensor
    Q: torch.Tensor          # [L, B, Hq, Wq, D] bf16: the query window
    Uk: torch.Tensor         # [L, Hkv, D, R] fp32
    Uv: torch.Tensor
    muQ: torch.Tensor = field(default=None)   # [L, Hq, D] fp32 per-head query offsets
    muK: torch.Tensor = field(default=None)   # [L, Hkv, D]
    muV: torch.Tensor = field(default=None)


def oja_inputs(L, B, Hkv, Hq, S, D=D_HEAD, R=64, Wq=32, S_cap=None, seed=BASE_SEED,
               device="cpu"):
    """Hybrid low-rank workload: K, V ~ N(mu, I) with per-(layer, kv head) offsets
    mu ~ N(0, 2); the query window Q ~ N(mu^Q, I) with per-(layer, query head)
    offsets; U_k, U_v seeded-QR orthonormal D x R.  Only the window's Wq most
    recent queries are drawn.  ``S_cap`` >= S reserves token rows for decode
    appends (left zero)."""
    S_cap = S if S_cap is None else S_cap
    G = L * B * Hkv
    K = torch.zeros((G, S_cap, D), dtype=torch.bfloat16, device=device)
    V = torch.zeros_like(K)
    Q = torch.empty((L, B, Hq, Wq, D), dtype=torch.bfloat16, device=device)
    sq2 = math.sqrt(2.0)
    muK = torch.empty((L, Hkv, D), device=device)
    muV = torch.empty((L, Hkv, D), device=device)
    muQ = torch.empty((L, Hq, D), device=device)
    for l in range(L):
        for h in range(Hkv):
            muK[l, h] = torch.randn(D, generator=_gen(device, seed, "muK", l, h), device=device) * sq2
            muV[l, h] = torch.randn(D, generator=_gen(device, seed, "muV", l, h), device=device) * sq2
        for hq in range(Hq):
            muQ[l, hq] = torch.randn(D, generator=_gen(device, seed, "muQ", l, hq), device=device) * sq2
    for l in range(L):
        for b in range(B):
            for h in range(Hkv):
                g = (l * B + b) * Hkv + h
                gk = _gen(device, seed, "K", g)
                K[g, :S] = (muK[l, h][None] + torch.randn((S, D), generator=gk, device=device)).to(
                    torch.bfloat16)
                gv = _gen(device, seed, "V", g)
                V[g, :S] = (muV[l, h][None] + torch.randn((S, D), generator=gv, device=device)).to(
                    torch.bfloat16)
            for hq in range(Hq):
                gq = _gen(device, seed, "Q", l, b, hq)
                Q[l, b, hq] = (muQ[l, hq][None] + torch.randn((Wq, D), generator=gq, device=device)
                               ).to(torch.bfloat16)
    Uk = torch.empty((L, Hkv, D, R), dtype=torch.float32)
    Uv = torch.empty_like(Uk)
    for l in range(L):
        for h in range(Hkv):
            Uk[l, h] = torch.from_numpy(orthonormal_basis(D, R, seed, 0, l, h))
            Uv[l, h] = torch.from_numpy(orthonormal_basis(D, R, seed, 1, l, h))
    return OjaInputs(L, B, Hkv, Hq, S, D, R, Wq, K, V, Q, Uk.to(device), Uv.to(device),
                     muQ=muQ, muK=muK, muV=muV)


def decode_token(inp: OjaInputs, step, seed=BASE_SEED):
    """New (k, v) per slice and q per query head for decode step ``step``, from
    the same per-head offsets: k [G, D], v [G, D], q [L, B, Hq, D] (bf16)."""
    dev = inp.K.device
    gen = _gen(dev, seed, "dec", step)
    G = inp.L * inp.B * inp.Hkv
    offK = inp.muK[:, None].expand(inp.L, inp.B, inp.Hkv, inp.D).reshape(G, inp.D)
    offV = inp.muV[:, None].expand(inp.L, inp.B, inp.Hkv, inp.D).reshape(G, inp.D)
    k = (offK + torch.randn((G, inp.D), generator=gen, device=dev)).to(torch.bfloat16)
    v = (offV + torch.randn((G, inp.D), generator=gen, device=dev)).to(torch.bfloat16)
    q = (inp.muQ[:, None] + torch.randn((inp.L, inp.B, inp.Hq, inp.D), generator=gen, device=dev)
         ).to(torch.bfloat16)
    return k, v, q


def random_scores(G, S, seed=BASE_SEED, device="cpu", kind="normal"):
    """fp32 score rows for selection tests: 'normal' (|N(0,1)|*10), 'ties'
    (few distinct values), 'signed' (N(0,1), both signs and +-0)."""
    g = _gen(device, seed, "score", G, S)
    if kind == "normal":
        return torch.randn((G, S), generator=g, device=device).abs() * 10.0
    if kind == "ties":
        return torch.randint(0, 7, (G, S), generator=g, device=device).to(torch.float32) * 0.5
    if kind == "signed":
        x = torch.randn((G, S), generator=g, device=device)
        x[:, ::17] = 0.0
        x[:, 5::17] = -0.0
        return x
    raise ValueError(kind)


def random_lowrank(G, S, R, seed=BASE_SEED, device="cpu"):
    """fp32 compressed rows X~ ~ N(0, 4) for reconstruction tests, [G, S, R]."""
    g = _gen(device, seed, "Xt", G, S, R)
    return torch.randn((G, S, R), generator=g, device=device) * 2.0
