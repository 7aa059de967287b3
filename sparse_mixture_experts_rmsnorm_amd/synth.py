"""Seeded synthetic inputs for the MoE layer (no arithmetic of the method).

Recipe (same for every workload):
  x        ~ N(0, 1)                         [T, d]
  weights  ~ N(0, w_std^2), w_std = 0.02     router, experts, shared, tables
  gamma    = 1 (omitted) unless the workload asks for a gain; then N(1, 0.1^2)
  bias     none | N(0, 1) per expert | Zipf: b_e = -s * ln(rank_e) with rank a
           seeded permutation of 1..E (expert popularity ~ rank^-s)
Values are drawn in float32 and stored as float32 (fp32 workloads) or as
bf16 with round-to-nearest-even (bf16 workloads).

Two generators produce the bytes:
  * numpy  (PCG64, seed = workload seed): host arrays; bf16 arrives as uint16
    bit patterns.  Used for every size the CPU handles quickly.
  * torch  (device generator, same seed): device tensors, for the multi-GB
    weight tables of the full-size layers.  The oracle receives the very same
    bytes copied back to the host.

Weight layouts are those of the "Variable-size experts" nanoMOE notes
(weight-allocation section): w1, w3 are [d, sum f] with one column slice per
expert, w2 is [sum f, d]; the router is [d, E]; the Cartesian keys are
[d, Nr] and [d, Nc]; atomic tables W, V are [N, d] (OmniMoE summary 2.1).
"""
from __future__ import annotations

import numpy as np

from .workloads import Workload


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _shapes(wl: Workload) -> dict:
    d = wl.d
    shp = {"x": (wl.T, d)}
    if wl.router == "cartesian":
        shp["k_rows"] = (d, wl.Nr)
        shp["k_cols"] = (d, wl.Nc)
        shp["W"] = (wl.Nr * wl.Nc, d)
        shp["V"] = (wl.Nr * wl.Nc, d)
    else:
        F = sum(wl.sizes)
        shp["w_router"] = (d, wl.E)
        shp["w1"] = (d, F)
        if wl.act == "swiglu":
            shp["w3"] = (d, F)
        shp["w2"] = (F, d)
    if wl.shared_ffn:
        shp["ws1"] = (d, wl.shared_ffn)
        if wl.shared_act == "swiglu":
            shp["ws3"] = (d, wl.shared_ffn)
        shp["ws2"] = (wl.shared_ffn, d)
    return shp


def _bias_numpy(wl: Workload, rng) -> np.ndarray | None:
    if wl.bias == "normal":
        return rng.standard_normal(wl.E, dtype=np.float32)
    if wl.bias == "zipf":
        rank = rng.permutation(wl.E).astype(np.float64) + 1.0
        return (-wl.zipf_s * np.log(rank)).astype(np.float32)
    return None


def make_numpy(wl: Workload, seed: int | None = None) -> dict:
    """Host inputs: float32 arrays, or uint16 bf16 bits for bf16 workloads.

    Tensors are drawn in a fixed order (x, then weights in the order of
    _shapes, then gamma, then bias) from one PCG64 stream.
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    out = {}
    for name, shape in _shapes(wl).items():
        a = rng.standard_normal(shape, dtype=np.float32)
        if name != "x":
            a *= np.float32(wl.w_std)
        out[name] = _to_bf16_bits(a) if wl.dtype == "bf16" else a
    if wl.gamma:
        g = (1.0 + 0.1 * rng.standard_normal(wl.d)).astype(np.float32)
        out["gamma"] = _to_bf16_bits(g) if wl.dtype == "bf16" else g
    b = _bias_numpy(wl, rng)
    if b is not None:
        out["bias"] = b  # router bias stays float32 (it is added to fp32 logits)
    return out


def make_torch(wl: Workload, device="cuda", seed: int | None = None) -> dict:
    """Device inputs from a seeded torch generator (float32 or bfloat16)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed if seed is None else seed)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    out = {}
    for name, shape in _shapes(wl).items():
        # fill in row chunks to bound the float32 staging buffer
        t = torch.empty(shape, dtype=dt, device=device)
        rows = shape[0]
        step = max(1, (1 << 26) // max(1, int(np.prod(shape[1:]))))
        for r0 in range(0, rows, step):
            r1 = min(rows, r0 + step)
            chunk = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                                dtype=torch.float32)
            if name != "x":
                chunk.mul_(wl.w_std)
            t[r0:r1].copy_(chunk)
        out[name] = t
    if wl.gamma:
        gg = 1.0 + 0.1 * torch.randn(wl.d, generator=g, device=device, dtype=torch.float32)
        out["gamma"] = gg.to(dt)
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    b = _bias_numpy(wl, rng)
    if b is not None:
        out["bias"] = torch.from_numpy(b).to(device)
    return out


def to_host(t) -> np.ndarray:
    """Device tensor -> host numpy with bf16 returned as uint16 bits."""
    import torch
    c = t.detach().cpu()
    if c.dtype == torch.bfloat16:
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def to_device(a: np.ndarray, device="cuda"):
    """Host array -> device tensor (uint16 bit patterns become bfloat16)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def make_integer_routing(T: int, d: int, E: int, seed: int, dup_pairs=(), bias_int=None) -> dict:
    """Router inputs on which every fp32 sum is exact, whatever its order.

    x      entries +-1 (bf16), feature 0 is +1 for every token;
    w_r    small integers in [-3, 3] times 2^-6 (bf16), [d, E];
    row 0 of w_r holds bias_int[e] * 2^-6 (|bias_int| <= 256, so still exact
    in bf16): with feature 0 fixed at +1 it acts as a per-expert bias inside
    the product, skewing the load so that the capacity rule drops slots;
    dup_pairs (a, b): column b is a copy of column a, so experts a and b tie
    exactly on every token.
    Returns bf16 bit patterns (uint16) for both.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=(T, d))
    x[:, 0] = 1.0
    w = rng.integers(-3, 4, size=(d, E)).astype(np.float32)
    if bias_int is not None:
        b = np.asarray(bias_int, dtype=np.float32)
        if b.shape != (E,) or np.max(np.abs(b)) > 256:
            raise ValueError("bias_int must hold E integers of magnitude <= 256")
        w[0, :] = b
    for a, c in dup_pairs:
        w[:, c] = w[:, a]
    w *= np.float32(2.0 ** -6)
    return dict(x=_to_bf16_bits(x), w_router=_to_bf16_bits(w))


def zipf_bias_int(E: int, s: float, seed: int, unit: float = 0.5) -> np.ndarray:
    """Zipf-shaped integer bias for make_integer_routing: round(-s ln(rank_e)
    * unit / 2^-6), rank a seeded permutation of 1..E, i.e. the bias
    -s ln(rank_e) * unit in multiples of 2^-6."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rank = rng.permutation(E).astype(np.float64) + 1.0
    return np.rint(-s * np.log(rank) * unit / 2.0 ** -6).astype(np.int64)
