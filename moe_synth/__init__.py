"""Seeded synthetic inputs for the MoE layer: shapes, value distributions and
routing skew of the workloads the pages measure.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no routing, no products, no combine).  Both the CPU oracle
and the HIP library are fed from here, and nothing else is shared by the two.

Shapes (COMET paper review, §5.1 model table: Mixtral 8x7B, Qwen2-MoE-2.7B,
Phi-3.5-MoE; PTO MoE article, measured-performance paragraph, for the
expert-parallel share: hidden 7168, expert width 4096, top-8, 16 local
experts, 2048 tokens per source):

    name      M      H     F      E   k  S  dtype  skew (token-fraction std)
    tiny      256    256   512    8   2  1  f32    0
    qwen2     4096   2048  1408   64  4  1  bf16   0
    mixtral   8192   4096  14336  8   2  1  bf16   0.032
    phi35     16384  4096  6400   16  2  1  bf16   0.05
    epshare   16384  7168  4096   16  8  8  bf16   0  (8 source blocks x 2048 rows)
    epshare_b 16384  7168  4096  128  8  8  bf16   0  (same blocks; experts 0..15 held)

The two expert-parallel readings of the PTO measured case: in epshare the 8
source blocks are routed among the 16 local experts only; in epshare_b they
are routed among 8 x 16 = 128 experts (one group of 16 per card) and this
call holds experts 0..15, so it keeps about 1/8 of the routed pairs (about
1024 per held expert) and its combine is the partial one.

Distributions: x ~ N(0,1); gate logits ~ N(0,1) in f32 plus, for the skewed
layers, a per-expert bias s * z_e (z drawn N(0,1), then standardised) whose
scale s makes the standard deviation of the per-expert token fractions equal
the target (COMET review §5.6.2: std 0 is uniform, 0.05 leaves the lightest
expert a few hundred tokens, 0.032 is the production average).  s is
calibrated once against the oracle's routing and stored in
``skew_scales.json``.  Weights ~ N(0, 0.02^2).  bf16 layers round x and the
weights to bf16 (torch's round-to-nearest-even conversion); logits stay f32.

Storage: x [M,H]; logits [M,E] f32; W_gate, W_up [E,F,H]; W_down [E,H,F]
(each stored matrix row is one output column of the math matrix, so the
reduction index is contiguous); src_block [M] int32 (token t of the
expert-parallel share comes from block t // 2048).  bf16 arrays are returned
as uint16 bit patterns.

Every tensor has its own PCG64 stream, keyed by (seed, tensor tag[, expert]),
so tensors and experts can be drawn independently and in parallel.
"""
from __future__ import annotations

import json
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SKEW_FILE = os.path.join(_HERE, "skew_scales.json")

WEIGHT_STD = 0.02

# stream tags
_T_X, _T_LOGITS, _T_SKEW, _T_WG, _T_WU, _T_WD = 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class Config:
    name: str
    M: int
    H: int
    F: int
    E: int
    k: int
    S: int = 1
    dtype: str = "bf16"  # "bf16" or "f32"
    seed: int = 0
    skew: float = 0.0
    block: int = 0  # tokens per source block (S > 1)
    base: int = 0   # first expert held
    local: int = 0  # experts held (0: all E); the weights hold these only

    @property
    def EL(self) -> int:
        return self.local if self.local else self.E

    @property
    def R(self) -> int:
        return self.M * self.k

    @property
    def flops(self) -> int:
        """Multiply-adds x2 of the three expert products: 6 * R * H * F."""
        return 6 * self.R * self.H * self.F


CONFIGS = {
    "tiny": Config("tiny", 256, 256, 512, 8, 2, 1, "f32", 101),
    "qwen2": Config("qwen2", 4096, 2048, 1408, 64, 4, 1, "bf16", 102),
    "mixtral": Config("mixtral", 8192, 4096, 14336, 8, 2, 1, "bf16", 103, 0.032),
    "phi35": Config("phi35", 16384, 4096, 6400, 16, 2, 1, "bf16", 104, 0.05),
    "epshare": Config("epshare", 16384, 7168, 4096, 16, 8, 8, "bf16", 105, 0.0, 2048),
    "epshare_b": Config("epshare_b", 16384, 7168, 4096, 128, 8, 8, "bf16", 106, 0.0, 2048, 0, 16),
}


def config(name: str, **overrides) -> Config:
    return replace(CONFIGS[name], **overrides) if overrides else CONFIGS[name]


def _rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *tags])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns via torch's conversion (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _finish(a: np.ndarray, dtype: str) -> np.ndarray:
    return a if dtype == "f32" else to_bf16_bits(a)


def draw_logits_raw(cfg: Config) -> np.ndarray:
    return _rng(cfg.seed, _T_LOGITS).standard_normal((cfg.M, cfg.E), dtype=np.float32)


def draw_skew_direction(cfg: Config) -> np.ndarray:
    """z [E], standardised to mean 0 and population std 1 (float64)."""
    z = _rng(cfg.seed, _T_SKEW).standard_normal(cfg.E)
    return (z - z.mean()) / z.std()


def skew_scale(cfg: Config) -> float:
    if cfg.skew == 0.0:
        return 0.0
    with open(SKEW_FILE) as fh:
        table = json.load(fh)
    key = f"{cfg.name}:{cfg.seed}:{cfg.M}:{cfg.E}:{cfg.k}:{cfg.skew}"
    if key not in table:
        raise KeyError(f"no calibrated skew scale for {key}; run tests/golden/make_skew_scales.py")
    return float(table[key]["scale"])


def logits_with_scale(cfg: Config, scale: float) -> np.ndarray:
    raw = draw_logits_raw(cfg)
    if scale == 0.0:
        return raw
    bias = (scale * draw_skew_direction(cfg)).astype(np.float32)
    return raw + bias[None, :]


def make_logits(cfg: Config) -> np.ndarray:
    return logits_with_scale(cfg, skew_scale(cfg))


def make_x(cfg: Config) -> np.ndarray:
    x = _rng(cfg.seed, _T_X).standard_normal((cfg.M, cfg.H), dtype=np.float32)
    return _finish(x, cfg.dtype)


def make_src_block(cfg: Config):
    if cfg.S == 1:
        return None
    block = cfg.block or (cfg.M // cfg.S)
    return (np.arange(cfg.M, dtype=np.int64) // block).astype(np.int32)


def _weight(cfg: Config, tag: int, e: int, rows: int, cols: int) -> np.ndarray:
    w = _rng(cfg.seed, tag, e).standard_normal((rows, cols), dtype=np.float32)
    w *= np.float32(WEIGHT_STD)
    return _finish(w, cfg.dtype)


def make_weights(cfg: Config, threads: int = 8):
    """(W_gate [EL,F,H], W_up [EL,F,H], W_down [EL,H,F]) of the held experts
    base .. base + EL - 1 (each drawn from its expert's own stream, so a
    held slice equals the same slice of the full stack)."""
    dt = np.float32 if cfg.dtype == "f32" else np.uint16
    EL = cfg.EL
    wg = np.empty((EL, cfg.F, cfg.H), dt)
    wu = np.empty((EL, cfg.F, cfg.H), dt)
    wd = np.empty((EL, cfg.H, cfg.F), dt)
    jobs = []
    for slot in range(EL):
        jobs.append((wg, _T_WG, slot, cfg.F, cfg.H))
        jobs.append((wu, _T_WU, slot, cfg.F, cfg.H))
        jobs.append((wd, _T_WD, slot, cfg.H, cfg.F))

    def run(job):
        dst, tag, slot, r, c = job
        dst[slot] = _weight(cfg, tag, cfg.base + slot, r, c)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(run, jobs))
    return wg, wu, wd


def make_inputs(cfg: Config, weights: bool = True, threads: int = 8) -> dict:
    d = dict(x=make_x(cfg), logits=make_logits(cfg), src_block=make_src_block(cfg))
    if weights:
        d["w_gate"], d["w_up"], d["w_down"] = make_weights(cfg, threads)
    return d


def token_sample(cfg: Config, n: int, seed_tag: int = 7) -> np.ndarray:
    """A seeded, sorted sample of n distinct token indices; for S > 1 it is
    spread evenly over the source blocks."""
    rng = _rng(cfg.seed, 100 + seed_tag)
    if n >= cfg.M:
        return np.arange(cfg.M, dtype=np.int64)
    if cfg.S > 1:
        block = cfg.block or (cfg.M // cfg.S)
        per = max(1, n // cfg.S)
        parts = [b * block + rng.choice(block, size=per, replace=False) for b in range(cfg.S)]
        return np.sort(np.concatenate(parts)).astype(np.int64)
    return np.sort(rng.choice(cfg.M, size=n, replace=False)).astype(np.int64)
