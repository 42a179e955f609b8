"""Seeded synthetic inputs for the routed-expert layer.

This module produces the tensors a caller hands to the layer: activations,
the full-precision router, the frozen int4 base experts and the trainable
low-rank adapters, plus an upstream gradient.  It holds none of the layer's
own arithmetic (routing, expert products, combine, backward); it only draws
random numbers, rounds them to their storage types and packs the frozen base
into the int4 storage format, which is offline preparation of an input.

Distributions (N(mu, var): the second argument is a variance):
  x, dY ~ N(0, 1); router W_r ~ N(0, 1/d); router bias ~ N(0, var) when used;
  gate/up base and A_gate/A_up ~ N(0, 1/d); down base and A_down ~ N(0, 1/f);
  every B ~ N(0, 0.02).

Seeding: SeedSequence([seed, cfg_id]) spawns, in this order, the streams for
x, W_r, bias, dY and then one child per expert, which spawns nine streams in
the order W_gate, W_up, W_down, A_gate, B_gate, A_up, B_up, A_down, B_down.
Draws are PCG64 float32 standard normals scaled by the standard deviation.

Storage formats (these are the library's input formats):
  * adapters are stored out x in like the base: A [r][K], B [N][r], so the
    adapter term of a row x is (x A^T) B^T.
  * bf16 tensors are carried as uint16 bit patterns, rounded to nearest even.
  * int4 base matrix W[N, K] (out x in) -> q: uint8 [N, K/2] and
    scale: bf16 [N, K/group].  Symmetric per-group quantisation along K:
    s = bf16(max|w| / 7), q = clamp(round_half_even(w / s), -8, 7), q = 0 when
    s = 0.  Nibbles are two's complement.  Each aligned 32-bit little-endian
    word holds the eight values k0..k7 of one 8-wide block of K; nibble slot j
    (bits 4j..4j+3) holds k_{2j} for j < 4 and k_{2(j-4)+1} for j >= 4, so a
    word unpacks into the bf16 pairs (k0,k1), (k2,k3), (k4,k5), (k6,k7) with
    one shift and one mask per pair.
  * int8 base matrix (bits = 8) -> q: uint8 [N, K] holding the two's-complement
    bytes in k order, scale: bf16 [N, K/group]; s = bf16(max|w| / 127),
    q = clamp(round_half_even(w / s), -128, 127), q = 0 when s = 0.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import LayerConfig

MATS = ("gate", "up", "down")


# ---------------------------------------------------------------- dtypes --

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def to_storage(a32: np.ndarray, act: str) -> np.ndarray:
    if act == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if act == "bf16":
        return bf16_bits(a32)
    raise ValueError(f"unknown activation dtype {act!r}")


def storage_to_f32(a: np.ndarray, act: str) -> np.ndarray:
    return a.astype(np.float32) if act == "f32" else bf16_to_f32(a)


# ------------------------------------------------------------ int4 base --

def pack_int4(q: np.ndarray) -> np.ndarray:
    """int8 values in [-8, 7], shape [..., K] (K % 8 == 0) -> uint8 [..., K/2]
    in the interleaved word layout described in the module docstring."""
    q = np.asarray(q)
    if q.shape[-1] % 8:
        raise ValueError("K must be a multiple of 8")
    n = (q.astype(np.int16) & 0xF).astype(np.uint8)
    n = n.reshape(q.shape[:-1] + (q.shape[-1] // 8, 8))
    b0 = n[..., 0] | (n[..., 2] << 4)
    b1 = n[..., 4] | (n[..., 6] << 4)
    b2 = n[..., 1] | (n[..., 3] << 4)
    b3 = n[..., 5] | (n[..., 7] << 4)
    out = np.stack([b0, b1, b2, b3], axis=-1)
    return np.ascontiguousarray(out.reshape(q.shape[:-1] + (q.shape[-1] // 2,)))


def quantize_int4(w: np.ndarray, group: int):
    """w float32 [N, K] -> (q uint8 [N, K/2], scale bf16 bits [N, K/group])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    wg = w.reshape(N, K // group, group)
    amax = np.abs(wg).max(axis=2)
    s_bits = bf16_bits(amax / np.float32(7.0))
    s = bf16_to_f32(s_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = wg / s[:, :, None]
    ratio = np.where(s[:, :, None] == 0, np.float32(0), ratio)
    q = np.clip(np.rint(ratio), -8, 7).astype(np.int8).reshape(N, K)
    return pack_int4(q), s_bits


def quantize_int8(w: np.ndarray, group: int):
    """w float32 [N, K] -> (q uint8 [N, K] two's-complement bytes,
    scale bf16 bits [N, K/group])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    wg = w.reshape(N, K // group, group)
    amax = np.abs(wg).max(axis=2)
    s_bits = bf16_bits(amax / np.float32(127.0))
    s = bf16_to_f32(s_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = wg / s[:, :, None]
    ratio = np.where(s[:, :, None] == 0, np.float32(0), ratio)
    q = np.clip(np.rint(ratio), -128, 127).astype(np.int8).reshape(N, K)
    return np.ascontiguousarray(q.view(np.uint8)), s_bits


def quantize(w: np.ndarray, group: int, bits: int):
    if bits == 4:
        return quantize_int4(w, group)
    if bits == 8:
        return quantize_int8(w, group)
    raise ValueError(f"unsupported base width {bits}")


# ------------------------------------------------------------ generator --

def _normal(ss: np.random.SeedSequence, shape, var: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    a = g.standard_normal(shape, dtype=np.float32)
    a *= np.float32(np.sqrt(var))
    return a


def _expert(cfg: LayerConfig, ss: np.random.SeedSequence):
    d, f, r, g = cfg.d, cfg.f, cfg.r, cfg.group
    s = ss.spawn(9)
    wg = _normal(s[0], (f, d), 1.0 / d)
    wu = _normal(s[1], (f, d), 1.0 / d)
    wd = _normal(s[2], (d, f), 1.0 / f)
    out = {}
    for name, w in (("gate", wg), ("up", wu), ("down", wd)):
        out[name] = quantize(w, g, cfg.bits)
    out["A_gate"] = to_storage(_normal(s[3], (r, d), 1.0 / d), cfg.act)
    out["B_gate"] = to_storage(_normal(s[4], (f, r), 0.02), cfg.act)
    out["A_up"] = to_storage(_normal(s[5], (r, d), 1.0 / d), cfg.act)
    out["B_up"] = to_storage(_normal(s[6], (f, r), 0.02), cfg.act)
    out["A_down"] = to_storage(_normal(s[7], (r, f), 1.0 / f), cfg.act)
    out["B_down"] = to_storage(_normal(s[8], (d, r), 0.02), cfg.act)
    return out


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(cfg: LayerConfig, seed: int = 0, threads: int | None = None) -> dict:
    """All inputs of one layer call as numpy arrays (see module docstring).

    Keys: x [T,d], dy [T,d] (act storage); w_router [d,E] f32; b_router [E]
    f32 or None; for m in gate/up/down: q_m [E,N,K/2] u8 (int4; [E,N,K] for int8), s_m [E,N,K/g] u16,
    A_m [E,r,K], B_m [E,N,r] (act storage; out x in like the base).
    N,K = (f,d) for gate/up and (d,f) for down.
    """
    root = np.random.SeedSequence([seed, cfg.cfg_id])
    s_x, s_wr, s_b, s_dy, *s_exp = root.spawn(4 + cfg.E)
    T, d, E, f, r, g = cfg.T, cfg.d, cfg.E, cfg.f, cfg.r, cfg.group
    out = {
        "x": to_storage(_normal(s_x, (T, d), 1.0), cfg.act),
        "w_router": _normal(s_wr, (d, E), 1.0 / d),
        "b_router": (_normal(s_b, (E,), cfg.router_bias_var)
                     if cfg.router_bias_var > 0 else None),
        "dy": to_storage(_normal(s_dy, (T, d), 1.0), cfg.act),
    }
    adt = np.float32 if cfg.act == "f32" else np.uint16
    shapes = {"gate": (f, d), "up": (f, d), "down": (d, f)}
    for m, (N, K) in shapes.items():
        out[f"q_{m}"] = np.empty((E, N, K * cfg.bits // 8), np.uint8)
        out[f"s_{m}"] = np.empty((E, N, K // g), np.uint16)
        out[f"A_{m}"] = np.empty((E, r, K), adt)
        out[f"B_{m}"] = np.empty((E, N, r), adt)

    def fill(e):
        ex = _expert(cfg, s_exp[e])
        for m in MATS:
            out[f"q_{m}"][e], out[f"s_{m}"][e] = ex[m]
            out[f"A_{m}"][e] = ex[f"A_{m}"]
            out[f"B_{m}"][e] = ex[f"B_{m}"]

    n = threads or default_threads()
    if n == 1 or E == 1:
        for e in range(E):
            fill(e)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(fill, range(E)))
    return out


def checksums(inputs: dict) -> dict:
    """SHA-256 of every generated array, for the record of a run."""
    import hashlib
    return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
            for k, v in inputs.items() if v is not None}
