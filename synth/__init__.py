"""Seeded synthetic workloads for the rotated residual-VQ KV cache.

This module only draws inputs: KV tensors, queries, fp16 recency windows and
codebooks.  It holds none of the method's arithmetic (no rotation, no
quantisation, no attention), so both the CPU oracle and the HIP path may take
their inputs from here without sharing computation.

Five workloads are defined, named by what they are:

  1 tiny        1 layer, 1 KV head, 1 query head, head_dim 64, 1024 tokens,
                fp32 K/V ~ N(0,1), 2 stages of full-vector codebooks
                (C=256 x 64), no window, seed 0.
  2 llama8b     Llama-3-8B-shaped layer: 8 KV / 32 query heads, head_dim 128,
                32768 tokens, bf16 K/V ~ N(0,1) with 4 outlier channels per
                head scaled x10, RoPE (theta 5e5) on K, 16 groups x 8 dims,
                1 stage, 128-token fp16 window, seed 1.
  3 qwen7b      Qwen2.5-7B-shaped decode batch: 16 sequences x 8192 tokens,
                4 KV / 28 query heads, RoPE (theta 1e6) on K, 16x8 groups,
                2 stages, 64-token window, seed 2.
  4 longctx     1 sequence x 131072 tokens, 8 KV / 32 query heads, K/V =
                per-(head, channel) scale x Laplace(0,1), scales log-uniform in
                [0.5, 8], 16x8 groups, 4 stages, 256-token window, seed 3.
  5 prefill     32 layers x 8 KV heads x 32768 tokens, bf16 K/V ~ N(0,1),
                RoPE (theta 5e5) on K, 16x8 groups, 2 stages, encode only,
                seed 4.

Readings taken where the workload descriptions are silent (each is listed in
the design notes): codebook entries of stage s are i.i.d.
N(0, sigma_x^2 / dsub) * 0.5**s, with sigma_x^2 the per-coordinate variance of
that (layer, K|V) source under its generator law; RoPE is the rotate-half
convention applied to every key (window included) before the bf16 cast; the
window holds the last W tokens, cast from bf16 to fp16; every tensor draws
from its own child of ``SeedSequence(seed)``.

Encode input layout: ``x[book][seq][t][d]`` where for decode workloads book 0
is K and book 1 is V (seq = b * Hkv + kv), and for the prefill workload book
2*layer + {0: K, 1: V}.  Codebooks: ``cb[book][S][G][C][dsub]`` float32.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "make_inputs", "bf16_bits",
           "bf16_bits_to_f32", "make_codebooks", "code_bytes_per_vector"]


@dataclasses.dataclass(frozen=True)
class Workload:
    key: int
    name: str
    batch: int
    layers: int
    n_kv_heads: int
    n_q_heads: int          # 0 = encode-only workload
    head_dim: int
    tokens: int
    window: int
    n_groups: int
    n_stages: int
    n_codewords: int
    x_dtype: str            # "f32" or "bf16"
    seed: int
    rope_theta: float | None
    source: str             # "normal", "normal_outliers", "laplace_scaled"
    n_outliers: int = 0
    outlier_scale: float = 1.0

    @property
    def dsub(self) -> int:
        return self.head_dim // self.n_groups

    @property
    def code_tokens(self) -> int:
        return self.tokens - self.window

    @property
    def n_books(self) -> int:
        return 2 * self.layers

    @property
    def n_seq(self) -> int:
        return self.batch * self.n_kv_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny", 1, 1, 1, 1, 64, 1024, 0, 1, 2, 256, "f32", 0, None, "normal"),
    2: Workload(2, "llama8b", 1, 1, 8, 32, 128, 32768, 128, 16, 1, 256, "bf16", 1, 5.0e5,
                "normal_outliers", n_outliers=4, outlier_scale=10.0),
    3: Workload(3, "qwen7b", 16, 1, 4, 28, 128, 8192, 64, 16, 2, 256, "bf16", 2, 1.0e6, "normal"),
    4: Workload(4, "longctx", 1, 1, 8, 32, 128, 131072, 256, 16, 4, 256, "bf16", 3, None,
                "laplace_scaled"),
    5: Workload(5, "prefill", 1, 32, 8, 0, 128, 32768, 0, 16, 2, 256, "bf16", 4, 5.0e5, "normal"),
}


def workload(key: int, **overrides) -> Workload:
    """The named workload, optionally resized (batch, tokens, window, layers,
    heads) for tests that need the same distributions at smaller sizes."""
    return WORKLOADS[key].replace(**overrides) if overrides else WORKLOADS[key]


def code_bytes_per_vector(w: Workload) -> int:
    """One uint8 code per (stage, group): C <= 256 codewords fit one byte."""
    return w.n_stages * w.n_groups


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only: round-to-nearest-even of float32 bits)
# ----------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------
def _children(w: Workload):
    ss = np.random.SeedSequence(w.seed)
    # fixed order: K, V, per-head params, K codebooks, V codebooks, queries, spare, spare
    return ss.spawn(8)


def _rope_k(x: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding on the last axis, positions 0..T-1 along
    axis -2.  Workload synthesis only (the keys a RoPE model would cache)."""
    T, D = x.shape[-2], x.shape[-1]
    half = D // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1 = x[..., :half].astype(np.float64)
    x2 = x[..., half:].astype(np.float64)
    out = np.empty(x.shape, dtype=np.float32)
    out[..., :half] = x1 * c - x2 * s
    out[..., half:] = x2 * c + x1 * s
    return out


def _source_params(w: Workload):
    """Per-(kv-head, channel) multipliers for K and V of every layer, and the
    per-coordinate source variance sigma_x^2 of each (layer, K|V)."""
    rng = np.random.default_rng(_children(w)[2])
    L, H, D = w.layers, w.n_kv_heads, w.head_dim
    mult = np.ones((L, 2, H, D), dtype=np.float32)
    var = np.ones((L, 2), dtype=np.float64)
    for l in range(L):
        if w.source == "normal_outliers":
            for h in range(H):
                ch = rng.choice(D, size=w.n_outliers, replace=False)
                mult[l, :, h, ch] = w.outlier_scale     # same channels on K and V
            var[l, :] = ((D - w.n_outliers) + w.n_outliers * w.outlier_scale ** 2) / D
        elif w.source == "laplace_scaled":
            for kv in range(2):
                s = np.exp(rng.uniform(np.log(0.5), np.log(8.0), size=(H, D)))
                mult[l, kv] = s.astype(np.float32)
                var[l, kv] = float(np.mean(2.0 * s.astype(np.float64) ** 2))  # Laplace(0,1) var = 2
    return mult, var


def make_codebooks(w: Workload) -> np.ndarray:
    """cb[book][S][G][C][dsub] float32; stage s ~ N(0, sigma_x^2/dsub) * 0.5**s."""
    ch = _children(w)
    _, var = _source_params(w)
    L, S, G, C, ds = w.layers, w.n_stages, w.n_groups, w.n_codewords, w.dsub
    out = np.empty((2 * L, S, G, C, ds), dtype=np.float32)
    k_ss, v_ss = ch[3].spawn(L), ch[4].spawn(L)
    for l in range(L):
        for kv, ss in ((0, k_ss[l]), (1, v_ss[l])):
            rng = np.random.default_rng(ss)
            std = np.sqrt(var[l, kv] / ds)
            z = rng.standard_normal((S, G, C, ds), dtype=np.float64) * std
            z *= (0.5 ** np.arange(S, dtype=np.float64))[:, None, None, None]
            out[2 * l + kv] = z.astype(np.float32)
    return out


def make_layer_kv(w: Workload, layer: int):
    """Float32 K and V of one layer, [B*Hkv][T][D], after outliers/scales and
    RoPE on K (before any bf16 cast)."""
    ch = _children(w)
    mult, _ = _source_params(w)
    shape = (w.batch, w.n_kv_heads, w.tokens, w.head_dim)
    out = []
    for kv, ss in ((0, ch[0].spawn(w.layers)[layer]), (1, ch[1].spawn(w.layers)[layer])):
        rng = np.random.default_rng(ss)
        if w.source == "laplace_scaled":
            x = rng.laplace(0.0, 1.0, size=shape).astype(np.float32)
        else:
            x = rng.standard_normal(shape, dtype=np.float32)
        x *= mult[layer, kv][None, :, None, :]
        if kv == 0 and w.rope_theta is not None:
            x = _rope_k(x, w.rope_theta)
        out.append(x.reshape(w.n_seq, w.tokens, w.head_dim))
    return out[0], out[1]


def make_inputs(w: Workload, *, layers=None) -> dict:
    """All inputs of a workload.

    Returns a dict with
      x        encode input [n_books][n_seq][T][D]: float32, or uint16 bf16 bits
      x_f32    the same values as float32 (exact widening of bf16)
      cb       codebooks [n_books][S][G][C][dsub] float32
      q        queries [B][Hq][D] float32 (decode workloads)
      k_win, v_win   fp16 [B][Hkv][W][D] (decode workloads with W > 0)
    ``layers`` restricts a multi-layer workload to the listed layers (books
    2l and 2l+1 of each listed layer, in order).
    """
    layers = list(range(w.layers)) if layers is None else list(layers)
    cb_all = make_codebooks(w)
    xs, cbs = [], []
    for l in layers:
        k, v = make_layer_kv(w, l)
        xs += [k, v]
        cbs += [cb_all[2 * l], cb_all[2 * l + 1]]
    x32 = np.stack(xs)
    if w.x_dtype == "bf16":
        xb = bf16_bits(x32)
        x_f32 = bf16_bits_to_f32(xb)
        x = xb
    else:
        x = x32
        x_f32 = x32
    out = {"workload": w, "x": x, "x_f32": x_f32, "cb": np.stack(cbs)}
    if w.n_q_heads > 0:
        rng = np.random.default_rng(_children(w)[5])
        out["q"] = rng.standard_normal((w.batch, w.n_q_heads, w.head_dim), dtype=np.float32)
        Tc, W = w.code_tokens, w.window
        shp = (w.batch, w.n_kv_heads, W, w.head_dim)
        out["k_win"] = x_f32[0][:, Tc:, :].astype(np.float16).reshape(shp)
        out["v_win"] = x_f32[1][:, Tc:, :].astype(np.float16).reshape(shp)
    return out
