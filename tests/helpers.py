"""Shared test utilities: conversions and error metrics (no decoder arithmetic)."""

from __future__ import annotations

import numpy as np
import torch


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a (bf16) tensor to a float64 NumPy array on the host."""
    return t.detach().to("cpu", torch.float64).numpy()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def max_abs(got, ref) -> float:
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


def report(name, got, ref):
    r, m = rel_l2(got, ref), max_abs(got, ref)
    print(f"{name}: rel_l2={r:.3e} max_abs={m:.3e} ref_max={np.max(np.abs(ref)):.3e}", flush=True)
    return r, m


def perm16_tokens(sp: int) -> np.ndarray:
    """Token stored at each physical column of the V^T layout (groups of 16:
    0 1 2 3 8 9 10 11 4 5 6 7 12 13 14 15)."""
    p = np.arange(sp) % 16
    inner = (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1)
    return (np.arange(sp) // 16) * 16 + inner


def oracle_dims(d):
    import oracle
    return oracle.ModelDims(hidden=d.hidden, n_heads=d.n_heads, n_kv_heads=d.n_kv_heads,
                            head_dim=d.head_dim, intermediate=d.intermediate,
                            rms_eps=d.rms_eps, rope_theta=d.rope_theta,
                            mrope_section=tuple(d.mrope_section))


def oracle_layer(weights: dict):
    import oracle
    return oracle.LayerWeights(**{k: f64(v) for k, v in weights.items()})


def row_rel_max(got, ref, row_len: int) -> float:
    """Largest relative L2 error over rows of `row_len` consecutive values
    (e.g. one (token, head) vector of a head_dim): a single wrong row shows up
    here even when the whole-tensor rel-L2 hides it."""
    g = np.asarray(got, np.float64).reshape(-1, row_len)
    r = np.asarray(ref, np.float64).reshape(-1, row_len)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    # rows whose reference is (numerically) zero are judged by the absolute error
    rel = np.where(den > 1e-12, num / np.where(den > 1e-12, den, 1.0), num)
    return float(np.max(rel)) if rel.size else 0.0


def report_rows(name, got, ref, row_len: int):
    """Whole-tensor rel-L2 and max-abs as `report`, plus the worst row's rel-L2."""
    r, m = rel_l2(got, ref), max_abs(got, ref)
    w = row_rel_max(got, ref, row_len)
    print(f"{name}: rel_l2={r:.3e} max_abs={m:.3e} worst_row_rel={w:.3e}", flush=True)
    return r, m, w
