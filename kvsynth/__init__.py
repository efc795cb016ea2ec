"""Seeded synthetic KV caches shaped like long-context LLaMA/Mistral layers.

This module is the only code shared by the oracle side and the HIP side: it
draws inputs and holds none of the pruning method's arithmetic.  Everything
is produced on the host with NumPy's PCG64 from a fixed base seed and a
per-tensor spawn key, then stored as float32 or as bf16 bit patterns (uint16,
round-to-nearest-even from float32).

Why these shapes and distributions: "ThinK: Thinner Key Cache by Query-Driven
Pruning" (original abstract) evaluates LLaMA and Mistral models on long
sequences and attributes the channel redundancy to an uneven magnitude
distribution and low-rank structure of the attention weights (Method details
-> Core idea).  No dataset or weights are available here, so each
configuration draws keys with log-normal per-channel scales, a few x8 outlier
channels and a rank-32 component plus small noise; values are N(0, 1).

Spawn keys: (config id, layer, tensor id, sub-index) with tensor ids
  0 channel scales, 1 outlier picks, 2 low-rank factor U, 3 low-rank basis W_r,
  4 key noise, 5 observation-window queries, 6 values, 7 ragged lengths,
  100+s decode query of step s, 200+s and 300+s the key and value that step appends.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Optional, Tuple

import numpy as np

BASE_SEED = 240721018
BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_capacity: int
    obs_window: int
    keep: int
    prune_ratio: float
    dtype: str                      # "f32" or "bf16"
    sigma: Tuple[float, float]      # log-normal sigma, spread linearly over the layers
    n_outliers: int                 # x8 outlier channels per kv head
    lowrank: int                    # 0: plain Gaussian keys; r: rank-r part plus noise
    noise: float
    ragged: Optional[Tuple[int, int]] = None   # inclusive length range, else full capacity
    decode_steps: int = 1

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def layer_sigma(self, layer: int) -> float:
        lo, hi = self.sigma
        if self.layers == 1:
            return lo
        return float(np.linspace(lo, hi, self.layers)[layer])


CONFIGS = {
    "tiny": Config("tiny", 1, 1, 1, 2, 2, 16, 256, 8, 8, 0.5, "f32", (1.0, 1.0), 2, 0, 0.0),
    "llama2-7b-layer-4k": Config("llama2-7b-layer-4k", 2, 1, 1, 32, 32, 128, 4096, 32, 77, 0.4,
                                 "bf16", (1.0, 1.0), 4, 32, 0.1),
    "mistral-7b-gqa-32k": Config("mistral-7b-gqa-32k", 3, 1, 1, 32, 8, 128, 32768, 32, 64, 0.5,
                                 "bf16", (1.0, 1.0), 4, 32, 0.1),
    "batched-ragged-16k": Config("batched-ragged-16k", 4, 1, 8, 32, 8, 128, 16384, 32, 51, 0.6,
                                 "bf16", (1.0, 1.0), 4, 32, 0.1, ragged=(8192, 16384)),
    "llama3-8b-128k": Config("llama3-8b-128k", 5, 32, 1, 32, 8, 128, 131072, 64, 64, 0.5,
                             "bf16", (0.5, 1.5), 4, 32, 0.1, decode_steps=128),
}


def custom(name="custom", *, batch=1, n_q_heads=2, n_kv_heads=2, head_dim=16, seq_capacity=64,
           obs_window=4, keep=8, dtype="f32", sigma=1.0, n_outliers=2, lowrank=0, noise=0.1,
           ragged=None, layers=1, cfg_id=0) -> Config:
    """A configuration with arbitrary sizes for tests (config id 0 unless given)."""
    return Config(name, cfg_id, layers, batch, n_q_heads, n_kv_heads, head_dim, seq_capacity,
                  obs_window, keep, 1.0 - keep / head_dim, dtype, (sigma, sigma), n_outliers,
                  lowrank, noise, ragged)


# ---------------------------------------------------------------------------
# bf16 storage
# ---------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def storage_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def nan_value(dtype: str):
    return BF16_NAN if dtype == "bf16" else np.float32(np.nan)


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------
def _rng(cfg: Config, layer: int, tensor: int, sub: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(BASE_SEED, spawn_key=(cfg.cfg_id, layer, tensor, sub))
    return np.random.Generator(np.random.PCG64(ss))


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    out = np.empty(shape, np.float32)
    rng.standard_normal(out=out, dtype=np.float32)
    return out


def seq_lens(cfg: Config, layer: int = 0) -> np.ndarray:
    """Valid tokens per sequence: full capacity, or uniform over cfg.ragged (inclusive)."""
    if cfg.ragged is None:
        return np.full(cfg.batch, cfg.seq_capacity, np.int32)
    lo, hi = cfg.ragged
    return _rng(cfg, 0, 7).integers(lo, hi + 1, size=cfg.batch).astype(np.int32)


def channel_scale(cfg: Config, layer: int) -> np.ndarray:
    """Per-(kv head, channel) scale exp(sigma*N(0,1)) with n_outliers channels x8. [Hkv, D]."""
    Hkv, D = cfg.n_kv_heads, cfg.head_dim
    sigma = cfg.layer_sigma(layer)
    scale = np.exp(np.float32(sigma) * _normal(_rng(cfg, layer, 0), (Hkv, D))).astype(np.float32)
    for kv in range(Hkv):
        if cfg.n_outliers > 0:
            picks = _rng(cfg, layer, 1, kv).choice(D, size=cfg.n_outliers, replace=False)
            scale[kv, picks] *= np.float32(8.0)
    return scale


def _keys_slab(cfg: Config, layer: int, b: int, kv: int, n: int, scale_row: np.ndarray,
               w_r: Optional[np.ndarray]) -> np.ndarray:
    sub = b * cfg.n_kv_heads + kv
    D = cfg.head_dim
    if cfg.lowrank == 0:
        return _normal(_rng(cfg, layer, 4, sub), (n, D)) * scale_row
    u = _normal(_rng(cfg, layer, 2, sub), (n, cfg.lowrank))
    base = u @ w_r
    base += np.float32(cfg.noise) * _normal(_rng(cfg, layer, 4, sub), (n, D))
    base *= scale_row
    return base


def _pool(threads):
    n = threads or min(16, os.cpu_count() or 1)
    return _cf.ThreadPoolExecutor(max_workers=max(1, n))


def make_layer(cfg: Config, layer: int = 0, *, with_v: bool = True, nan_pad: bool = True,
               threads: Optional[int] = None) -> dict:
    """One layer's cache and observation window.

    Returns dict with
      k_cache [B,S_cap,Hkv,D], v_cache [B,S_cap,Hkv,D] (if with_v),
      q_obs [B,W,Hq,D] (the last W prompt queries of each sequence),
      seq_lens int32 [B], channel_scale float32 [Hkv,D];
    stored as float32 or bf16 bits.  Rows t >= len_b hold a NaN sentinel when
    nan_pad, so that any read of padding poisons the result."""
    B, S, Hq, Hkv, D, W = (cfg.batch, cfg.seq_capacity, cfg.n_q_heads, cfg.n_kv_heads,
                           cfg.head_dim, cfg.obs_window)
    lens = seq_lens(cfg, layer)
    scale = channel_scale(cfg, layer)
    sdt = storage_dtype(cfg.dtype)
    fill = nan_value(cfg.dtype) if nan_pad else sdt(0)
    k = np.empty((B, S, Hkv, D), sdt)
    v = np.empty((B, S, Hkv, D), sdt) if with_v else None
    w_bases = None
    if cfg.lowrank:
        w_bases = [(_normal(_rng(cfg, layer, 3, kv), (cfg.lowrank, D)) /
                    np.float32(np.sqrt(cfg.lowrank))).astype(np.float32) for kv in range(Hkv)]

    def k_task(b, kv):
        n = int(lens[b])
        slab = _keys_slab(cfg, layer, b, kv, n, scale[kv], w_bases[kv] if w_bases else None)
        k[b, :n, kv, :] = _store(slab, cfg.dtype)
        k[b, n:, kv, :] = fill

    def v_task(b, kv):
        n = int(lens[b])
        slab = _normal(_rng(cfg, layer, 6, b * Hkv + kv), (n, D))
        v[b, :n, kv, :] = _store(slab, cfg.dtype)
        v[b, n:, kv, :] = fill

    jobs = [(k_task, b, kv) for b in range(B) for kv in range(Hkv)]
    if with_v:
        jobs += [(v_task, b, kv) for b in range(B) for kv in range(Hkv)]
    if len(jobs) == 1 or B * S * Hkv * D < (1 << 20):
        for fn, b, kv in jobs:
            fn(b, kv)
    else:
        with _pool(threads) as ex:
            list(ex.map(lambda j: j[0](j[1], j[2]), jobs))

    head_scale = np.repeat(scale, cfg.group, axis=0)          # [Hq, D], q head h -> kv h // G
    q_obs = np.empty((B, W, Hq, D), sdt)
    for b in range(B):
        q_obs[b] = _store(_normal(_rng(cfg, layer, 5, b), (W, Hq, D)) * head_scale, cfg.dtype)
    out = dict(k_cache=k, q_obs=q_obs, seq_lens=lens, channel_scale=scale)
    if with_v:
        out["v_cache"] = v
    return out


def decode_q(cfg: Config, layer: int, step: int, scale: Optional[np.ndarray] = None) -> np.ndarray:
    """The query of decode step `step`: [B,Hq,D], N(0,1) times the layer's channel scale."""
    if scale is None:
        scale = channel_scale(cfg, layer)
    head_scale = np.repeat(scale, cfg.group, axis=0)
    x = _normal(_rng(cfg, layer, 100 + step), (cfg.batch, cfg.n_q_heads, cfg.head_dim))
    return _store(x * head_scale, cfg.dtype)


def decode_kv(cfg: Config, layer: int, step: int, scale: Optional[np.ndarray] = None):
    """The key and value a decode step appends: [B,Hkv,D] each; the key is
    N(0,1) times the layer's channel scale (tensor id 200+step), the value
    N(0,1) (tensor id 300+step)."""
    if scale is None:
        scale = channel_scale(cfg, layer)
    shape = (cfg.batch, cfg.n_kv_heads, cfg.head_dim)
    k = _normal(_rng(cfg, layer, 200 + step), shape) * scale
    v = _normal(_rng(cfg, layer, 300 + step), shape)
    return _store(k, cfg.dtype), _store(v, cfg.dtype)


def as_float(a: np.ndarray) -> np.ndarray:
    """Stored array -> float32 values (bf16 bits are widened exactly)."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)
