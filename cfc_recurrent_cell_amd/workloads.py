"""Seeded synthetic inputs for the CfC K-loop and the axis-0 reducer.

This module only draws random numbers and lays them out; it holds none of the
cell's arithmetic, so both the HIP path and the float64 oracle can consume its
arrays without sharing any of the method's code.

Shapes follow the workloads the pages describe:
  * the smoke / cluster shape of the K-loop Parallelization Implementation
    Plan (B=32, seq_len=64, HIDDEN_DIM=128; Task 7 and the launch configs of
    Task 5), scaled to B=256 for the training-scale case;
  * the GRN grad_w1 scratch tail of the same plan (Task "GRN bwd", ~40K floats
    at B=32) for the standalone reduce;
  * batch=8192, K=8, width 256 from the Custom Kernel Optimization
    Implementation Plan ("Dimensions" line) for the large-batch case.
The pages' CfC input is a LayerNorm output, so x ~ N(0, 1) is the faithful
distribution.

Conventions (all stated, none printed by the pages):
  * N(0, v) names the VARIANCE v; W ~ N(0, 1/fan_in) is LeCun-normal.
  * numpy PCG64 with a fixed seed per workload and a fixed draw order:
    W_in, W_rec, (b), w_tau, x (then the per-feature scale), h0, y.
    Arrays specified as zero are not drawn.
  * every array is cast to float32 after drawing; dt is a float32 scalar.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class CfcConfig:
    name: str
    B: int
    K: int
    n_in: int
    n_hid: int
    dt: float
    seed: int
    h0_var: float = 0.0          # 0 => h0 = 0 (not drawn)
    x_feature_scale: bool = False  # x = s_f * z, s_f ~ U[0.5, 2] per feature
    steps: int = 1               # repeated steps over the same inputs
    cell: str = "gated"          # "gated" or "tau_decay" (w_tau then holds tau ~ U[0.05, 2])


@dataclasses.dataclass(frozen=True)
class ReduceConfig:
    name: str
    B: int
    N: int
    seed: int
    integer_seed: int


# The five named workloads.
TINY = CfcConfig("tiny_B4_K8_n16_H32", B=4, K=8, n_in=16, n_hid=32, dt=1.0, seed=0)
REDUCE = ReduceConfig("reduce_B32_N40960", B=32, N=40960, seed=1, integer_seed=11)
SMOKE = CfcConfig("smoke_B32_K64_H128", B=32, K=64, n_in=128, n_hid=128, dt=1.0, seed=2,
                  h0_var=0.1)
TRAIN = CfcConfig("train_B256_K64_H128", B=256, K=64, n_in=128, n_hid=128, dt=0.5, seed=3,
                  x_feature_scale=True, steps=10)
LARGE = CfcConfig("large_B8192_K8_H256", B=8192, K=8, n_in=256, n_hid=256, dt=1.0, seed=4,
                  h0_var=0.1)

# A sequence four times the training length, beyond the one-call backward's
# on-chip bound at this width (76 steps): run in windows.
LONG = CfcConfig("long_B256_K256_H128", B=256, K=256, n_in=128, n_hid=128, dt=0.5, seed=5,
                 x_feature_scale=True)

# The tau-decay cell: the shape and dt of the pages' B=1 backward test (n_in=8,
# n_hid=16, dt=0.02, tau ~ U[0.05, 2]) over a few rows and steps, and the
# training-scale shape with the same dt and tau range.
TAU_TINY = CfcConfig("tau_tiny_B4_K8_n8_H16", B=4, K=8, n_in=8, n_hid=16, dt=0.02, seed=20,
                     h0_var=0.1, cell="tau_decay")
TAU_TRAIN = CfcConfig("tau_train_B256_K64_H128", B=256, K=64, n_in=128, n_hid=128, dt=0.02, seed=21,
                      x_feature_scale=True, cell="tau_decay")

CFC_CONFIGS = {c.name: c for c in (TINY, SMOKE, TRAIN, LARGE, LONG, TAU_TINY, TAU_TRAIN)}


def scratch_row_len(n_in: int, n_hid: int) -> int:
    """Length of one per-batch gradient row: W_in, W_rec, b, w_tau concatenated."""
    return n_hid * (n_in + n_hid + 2)


@dataclasses.dataclass
class CfcInputs:
    w_in: np.ndarray    # [H, n_in]
    w_rec: np.ndarray   # [H, H]
    b: np.ndarray       # [H]
    w_tau: np.ndarray   # [H]
    x: np.ndarray       # [B, K, n_in]
    h0: np.ndarray      # [B, H]
    y: np.ndarray       # [B, H]
    dt: np.float32
    cell: str = "gated"


def make_cfc_inputs(cfg: CfcConfig, B: Optional[int] = None) -> CfcInputs:
    """Draw one workload's inputs.  ``B`` overrides the batch size (same draw order)."""
    B = cfg.B if B is None else B
    K, n_in, H = cfg.K, cfg.n_in, cfg.n_hid
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    w_in = rng.standard_normal((H, n_in)) * np.sqrt(1.0 / n_in)
    w_rec = rng.standard_normal((H, H)) * np.sqrt(1.0 / H)
    b = np.zeros(H)
    w_tau = _draw_w_tau(rng, H, cfg.cell)
    x = rng.standard_normal((B, K, n_in))
    if cfg.x_feature_scale:
        s = rng.uniform(0.5, 2.0, size=n_in)
        x = x * s[None, None, :]
    if cfg.h0_var > 0:
        h0 = rng.standard_normal((B, H)) * np.sqrt(cfg.h0_var)
    else:
        h0 = np.zeros((B, H))
    y = rng.standard_normal((B, H))
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return CfcInputs(f(w_in), f(w_rec), f(b), f(w_tau), f(x), f(h0), f(y), np.float32(cfg.dt), cfg.cell)


def _draw_w_tau(rng, H: int, cell: str) -> np.ndarray:
    """The gated cell's w_tau ~ N(0, 0.1); the tau-decay cell's time constants
    tau ~ U[0.05, 2] (the range of the pages' B=1 backward test)."""
    if cell == "tau_decay":
        return rng.uniform(0.05, 2.0, size=H)
    if cell != "gated":
        raise ValueError(f"unknown cell {cell!r}")
    return rng.standard_normal(H) * np.sqrt(0.1)


def make_random_cfc_inputs(B: int, K: int, n_in: int, n_hid: int, dt: float, seed: int,
                           w_scale: float = 1.0, b_std: float = 0.1,
                           h0_std: float = 0.3, cell: str = "gated") -> CfcInputs:
    """Generic seeded inputs for ragged / edge-case shapes (nonzero b and h0)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w_in = rng.standard_normal((n_hid, n_in)) * (w_scale / np.sqrt(max(n_in, 1)))
    w_rec = rng.standard_normal((n_hid, n_hid)) * (w_scale / np.sqrt(max(n_hid, 1)))
    b = rng.standard_normal(n_hid) * b_std
    w_tau = _draw_w_tau(rng, n_hid, cell)
    x = rng.standard_normal((B, K, n_in))
    h0 = rng.standard_normal((B, n_hid)) * h0_std
    y = rng.standard_normal((B, n_hid))
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return CfcInputs(f(w_in), f(w_rec), f(b), f(w_tau), f(x), f(h0), f(y), np.float32(dt), cell)


def make_reduce_input(cfg: ReduceConfig = REDUCE, integer: bool = False) -> np.ndarray:
    """[B, N] float32; the integer variant draws integers uniform in [-8, 8]."""
    if integer:
        rng = np.random.Generator(np.random.PCG64(cfg.integer_seed))
        a = rng.integers(-8, 9, size=(cfg.B, cfg.N))
    else:
        rng = np.random.Generator(np.random.PCG64(cfg.seed))
        a = rng.standard_normal((cfg.B, cfg.N))
    return np.ascontiguousarray(a, dtype=np.float32)


def make_random_matrix(B: int, N: int, seed: int, integer: bool = False) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    if integer:
        a = rng.integers(-8, 9, size=(B, N))
    else:
        a = rng.standard_normal((B, N))
    return np.ascontiguousarray(a, dtype=np.float32)
