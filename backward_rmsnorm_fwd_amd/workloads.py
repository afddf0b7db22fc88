"""Seeded synthetic workloads (inputs only; no RMSNorm arithmetic here).

This module is the one piece shared by the HIP path's tests and benchmark and
by the oracle's checks: it draws the input tensors.  It computes nothing of
the method itself.

Recipe (the pages use synthetic data only; page "Check an AI model calculation
before accelerating it", section "Docker and GPU prerequisites", and the
torchtitan page's test cases):

* NumPy ``Generator(PCG64(seed))`` draws in float32, in a fixed order
  (x, then gamma or w, then dy, then any row permutation), followed by one
  round-to-nearest-even cast to the target dtype with ``torch.Tensor.to``.
* ``N(0, s)`` means mean 0 and standard deviation s.

Workloads (sizes are LLM hidden-state shapes):

=====  =======================================================================
c1a    fp32 65 x 128: 64 rows x, dy ~ N(0,1), gamma ~ U(0.5,1.5), + 1 zero row
c1b    fp32 1 x 2, the worked example x=[3,4], gamma=[1,1], dy=[1,2]
c1c    fp32 1 x 2, x=[3,4], gamma=[2,0.5], dy=[1,2]
c2     bf16 32768 x 4096 (8 sequences x 4096 tokens): x ~ N(0,1),
       gamma ~ U(0.5,1.5), dy ~ N(0,1e-2)
c3     fp16 262144 x 1024: x ~ N(0,1) with 1% of rows x1e3, 1% x1e-3 and 0.1%
       all-zero, gamma ~ U(0.5,1.5), dy ~ N(0,1)
c4     bf16 2048 x 65536: as c2
c5     bf16 65536 x 5120, offset weight: x ~ N(0,1), w ~ N(0,0.02),
       dy ~ N(0,1e-2)
=====  =======================================================================

Every recipe can also be drawn at another (M, N) -- the parity tests use that
to run each recipe at sizes the oracle finishes quickly.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: torch.dtype
    M: int
    N: int
    offset: bool
    recipe: str
    eps: float = 1e-6
    seed: int = 0
    description: str = ""


WORKLOADS = {
    "c1a": Workload("c1a", torch.float32, 65, 128, False, "c1a",
                    description="fp32 64x128 random rows plus one all-zero row"),
    "c1b": Workload("c1b", torch.float32, 1, 2, False, "c1b",
                    description="fp32 worked example x=[3,4], gamma=[1,1], dy=[1,2]"),
    "c1c": Workload("c1c", torch.float32, 1, 2, False, "c1c",
                    description="fp32 worked example x=[3,4], gamma=[2,0.5], dy=[1,2]"),
    "c2": Workload("c2", torch.bfloat16, 32768, 4096, False, "llm",
                   description="bf16 hidden states, 8 sequences x 4096 tokens, hidden 4096"),
    "c3": Workload("c3", torch.float16, 262144, 1024, False, "scaled_rows",
                   description="fp16 many short rows with 1e3/1e-3-scaled and all-zero rows"),
    "c4": Workload("c4", torch.bfloat16, 2048, 65536, False, "llm",
                   description="bf16 long rows, hidden 65536"),
    "c5": Workload("c5", torch.bfloat16, 65536, 5120, True, "offset",
                   description="bf16 offset weight (1+w), hidden 5120"),
}


def _normal(rng, shape, std=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _uniform(rng, shape, lo, hi):
    return (rng.random(size=shape, dtype=np.float32) * np.float32(hi - lo)
            + np.float32(lo))


def _cast(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype)


def special_rows_c3(M):
    """Row counts of the c3 recipe: (x1e3, x1e-3, zero)."""
    return M // 100, M // 100, M // 1000


def make_inputs(name, M=None, N=None, seed=None, dtype=None):
    """Draw the inputs of workload ``name`` (optionally at another M, N).

    Returns a dict with CPU tensors ``x`` [M, N], ``w`` [N] (gamma, or the
    offset weight w when ``offset``), ``dy`` [M, N], plus ``offset``, ``eps``,
    ``dtype`` and, for the scaled-rows recipe, the row index sets.
    """
    out, arrays, _ = _draw(name, M, N, seed, dtype)
    x, g, dy = arrays
    out.update(x=_cast(x, out["dtype"]), w=_cast(g, out["dtype"]), dy=_cast(dy, out["dtype"]))
    return out


def make_layernorm_inputs(name, M=None, N=None, seed=None, dtype=None):
    """LayerNorm inputs for workload ``name``: the RMSNorm recipe's x, weight
    and dy (same draws), then, from the same generator, a bias
    ``b ~ U(-0.5, 0.5)`` [N] and a per-row shift ``s_i ~ N(0, 1)`` added to
    every element of row i before the cast, so rows have non-zero means (the
    c3 recipe's all-zero rows become constant rows).  The worked examples
    (c1b, c1c) keep x = [3, 4] and take b = [0, 0] and [0.5, -0.25].
    The offset recipe's weight is used as gamma directly (LayerNorm has no
    offset mode).  Returns the dict of ``make_inputs`` plus ``b``.
    """
    out, arrays, rng = _draw(name, M, N, seed, dtype)
    x, g, dy = arrays
    M, N = out["M"], out["N"]
    if rng is None:
        b = np.array([0.0, 0.0] if name == "c1b" else [0.5, -0.25], dtype=np.float32)
    else:
        b = _uniform(rng, (N,), -0.5, 0.5)
        x = x + _normal(rng, (M, 1))
    T = out["dtype"]
    out.update(x=_cast(x, T), w=_cast(g, T), dy=_cast(dy, T), b=_cast(b, T), offset=False)
    return out


def _draw(name, M, N, seed, dtype):
    """The float32 arrays (x, weight, dy) of a recipe, its metadata, and the
    generator after the draws (None for the fixed worked examples)."""
    wl = WORKLOADS[name]
    M = wl.M if M is None else int(M)
    N = wl.N if N is None else int(N)
    seed = wl.seed if seed is None else int(seed)
    dtype = wl.dtype if dtype is None else dtype
    out = {"offset": wl.offset, "eps": wl.eps, "dtype": dtype, "M": M, "N": N,
           "name": name, "seed": seed}
    if wl.recipe in ("c1b", "c1c"):
        x = np.array([[3.0, 4.0]], dtype=np.float32)
        g = np.array([1.0, 1.0] if wl.recipe == "c1b" else [2.0, 0.5],
                     dtype=np.float32)
        dy = np.array([[1.0, 2.0]], dtype=np.float32)
        return out, (x, g, dy), None
    rng = np.random.Generator(np.random.PCG64(seed))
    if wl.recipe == "c1a":
        x = np.zeros((M, N), dtype=np.float32)
        x[:M - 1] = _normal(rng, (M - 1, N))
        g = _uniform(rng, (N,), 0.5, 1.5)
        dy = _normal(rng, (M, N))
        out["zero_rows"] = np.array([M - 1])
    elif wl.recipe == "llm":
        x = _normal(rng, (M, N))
        g = _uniform(rng, (N,), 0.5, 1.5)
        dy = _normal(rng, (M, N), 1e-2)
    elif wl.recipe == "offset":
        x = _normal(rng, (M, N))
        g = _normal(rng, (N,), 0.02)
        dy = _normal(rng, (M, N), 1e-2)
    elif wl.recipe == "scaled_rows":
        x = _normal(rng, (M, N))
        g = _uniform(rng, (N,), 0.5, 1.5)
        dy = _normal(rng, (M, N))
        perm = rng.permutation(M)
        n_big, n_small, n_zero = special_rows_c3(M)
        big = perm[:n_big]
        small = perm[n_big:n_big + n_small]
        zero = perm[n_big + n_small:n_big + n_small + n_zero]
        x[big] *= np.float32(1e3)
        x[small] *= np.float32(1e-3)
        x[zero] = 0.0
        out.update(big_rows=np.sort(big), small_rows=np.sort(small),
                   zero_rows=np.sort(zero))
    else:  # pragma: no cover
        raise KeyError(wl.recipe)
    return out, (x, g, dy), rng


def make_tile_case(shape, dtype, seed, scale=1.0):
    """Tile-boundary and adversarial-variance cases of the torchtitan page
    (section "形状选择": 255/256/257, 4095/4096/4097, 5120, a 3-D input;
    section "对抗样本": near-zero and zero variance via ``scale``).

    x ~ N(0,1)*scale, gamma ~ U(0.5,1.5), dy ~ N(0,1); any leading dims.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n = shape[-1]
    x = _normal(rng, shape) * np.float32(scale)
    g = _uniform(rng, (n,), 0.5, 1.5)
    dy = _normal(rng, shape)
    return {"x": _cast(x, dtype), "w": _cast(g, dtype), "dy": _cast(dy, dtype),
            "offset": False, "eps": 1e-6, "dtype": dtype}


def make_layernorm_tile_case(shape, dtype, seed, scale=1.0, shift_std=1.0):
    """LayerNorm version of ``make_tile_case``: the same draws, then a bias
    b ~ U(-0.5, 0.5) and a per-row shift ~ N(0, shift_std) added before the
    cast.  A small ``scale`` with a large ``shift_std`` gives rows whose
    spread is tiny against their mean (the variance then comes from a
    cancelling difference)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = shape[-1]
    x = _normal(rng, shape) * np.float32(scale)
    g = _uniform(rng, (n,), 0.5, 1.5)
    dy = _normal(rng, shape)
    b = _uniform(rng, (n,), -0.5, 0.5)
    x = x + _normal(rng, shape[:-1] + (1,), shift_std)
    return {"x": _cast(x, dtype), "w": _cast(g, dtype), "dy": _cast(dy, dtype),
            "b": _cast(b, dtype), "offset": False, "eps": 1e-6, "dtype": dtype}


def make_add_inputs(name, M=None, N=None, seed=None, dtype=None):
    """Inputs of the residual add fused with RMSNorm for workload ``name``:
    the recipe's x, weight and dy (same draws), then from the same generator
    a residual stream ``res ~ N(0, 1)`` [M, N] and the gradient arriving on
    it ``dh`` [M, N], drawn like the recipe's dy (N(0, 1e-2) for the LLM
    recipes, N(0, 1) otherwise).  Returns the dict of ``make_inputs`` plus
    ``res`` and ``dh``."""
    out, arrays, rng = _draw(name, M, N, seed, dtype)
    x, g, dy = arrays
    M, N = out["M"], out["N"]
    if rng is None:
        res = np.array([[0.5, -1.0]], dtype=np.float32)
        dh = np.array([[0.25, 0.5]], dtype=np.float32)
    else:
        res = _normal(rng, (M, N))
        dh = _normal(rng, (M, N), 1e-2 if WORKLOADS[name].recipe in ("llm", "offset") else 1.0)
    T = out["dtype"]
    out.update(x=_cast(x, T), w=_cast(g, T), dy=_cast(dy, T), res=_cast(res, T), dh=_cast(dh, T))
    return out


def make_cast_inputs(name, M=None, N=None, seed=None, out_dtype=torch.bfloat16):
    """Inputs of RMSNorm with its output cast to ``out_dtype`` for workload
    ``name``: the recipe's draws (x, weight, dy, in that order), with x and
    the weight in float32 (the wide input) and dy in ``out_dtype`` (the
    gradient arrives in the dtype the forward wrote).  Returns the dict of
    ``make_inputs`` with ``dtype`` float32 plus ``out_dtype``."""
    out, arrays, _ = _draw(name, M, N, seed, torch.float32)
    x, g, dy = arrays
    out.update(x=_cast(x, torch.float32), w=_cast(g, torch.float32), dy=_cast(dy, out_dtype),
               out_dtype=out_dtype)
    return out


def make_cast_tile_case(shape, out_dtype, seed, scale=1.0):
    """``make_tile_case`` for the cast path: float32 x and gamma, dy in
    ``out_dtype``."""
    case = make_tile_case(shape, torch.float32, seed, scale)
    case["dy"] = case["dy"].to(out_dtype)
    case["out_dtype"] = out_dtype
    return case
