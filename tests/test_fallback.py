"""The fallback analysis for outputs the gate cannot decide (oracle.fallback,
the torchtitan page's section "gate 失效时的三步替代分析"), on the CPU.

The sweep is the one the LayerNorm GPU test runs for dx at short rows: row
lengths T in {2, 3, 4, 8, 16, 64, 256}, three seeds, 64 rows each, float32 and
bfloat16.  Targets are CPU stand-ins: a correct float32 evaluation in a third
order (must end PASS WITH LIMITATIONS), and variants with one planted mistake
each: truncation instead of rounding (bias: FAIL), an error that grows like T
(growth: FAIL in float32; in bfloat16 the output rounding hides it at small T,
so it must at least not pass), and noise ten envelope units wide
(INCONCLUSIVE).
"""
import numpy as np
import pytest
import torch

from backward_rmsnorm_fwd_amd import workloads
from oracle import fallback
from oracle import layernorm as lnref

TS = (2, 3, 4, 8, 16, 64, 256)
SEEDS = (0, 1, 2)


def _third_order(dy, x, g, eps, cast=True):
    """A correct float32 dx in another legal order: xhat by division by the
    standard deviation, means as sums times 1/N (rounded to x's dtype unless
    ``cast`` is false)."""
    xf, dyf = x.float(), dy.float()
    n = xf.shape[-1]
    inv = 1.0 / n
    mean = xf.sum(-1, keepdim=True) * inv
    d = xf - mean
    sd = torch.sqrt((d * d).sum(-1, keepdim=True) * inv + eps)
    xhat = d / sd
    u = dyf * g.float()
    c1 = u.sum(-1, keepdim=True) * inv
    c2 = (u * xhat).sum(-1, keepdim=True) * inv
    dx = (u - c1 - xhat * c2) / sd
    return dx.to(x.dtype) if cast else dx


def _truncate(t, dtype):
    if dtype != torch.bfloat16:
        return t
    bits = t.float().contiguous().view(torch.int32) & ~0xFFFF
    return bits.view(torch.float32).to(dtype)


def _cases(dtype, mutation=None):
    cases = []
    for T in TS:
        for seed in SEEDS:
            inp = workloads.make_layernorm_tile_case((64, T), dtype, 100 + seed)
            x, w, dy, eps = inp["x"], inp["w"], inp["dy"], inp["eps"]
            golden = lnref.golden_ln_dx(dy, x, w, eps)
            mag = lnref.ln_dx_magnitude(dy, x, w, eps)
            ref_a = lnref.reference_ln_backward(dy, x, w, eps)[0]
            ref_b = lnref.reference_ln_dx_reordered(dy, x, w, eps)
            if mutation == "truncate":
                # the third order computed in float32, then cut to bf16
                tgt = _truncate(_third_order(dy, x, w, eps, cast=False), dtype)
            else:
                tgt = _third_order(dy, x, w, eps)
            t64 = tgt.double().numpy()
            rng = np.random.default_rng(seed + 17 * T)
            if mutation == "grows_with_T":
                t64 = t64 + 0.5 * T * fallback.U32 * mag * rng.choice([-1.0, 1.0], size=mag.shape)
            elif mutation == "noise":
                env = fallback.U32 * mag
                t64 = t64 + 10.0 * env * rng.choice([-1.0, 1.0], size=mag.shape)
            cases.append(fallback.Case(T, seed, t64, ref_a, ref_b, golden, mag, dtype))
    return cases


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_correct_target_passes_with_limitations(dtype):
    res = fallback.analyse(_cases(dtype))
    print(fallback.report(res, f"third order {dtype}"))
    assert res.verdict == "PASS WITH LIMITATIONS", res.reasons


def test_truncation_fails_on_bias():
    res = fallback.analyse(_cases(torch.bfloat16, "truncate"))
    assert res.verdict == "FAIL"
    assert any("bias" in r for r in res.reasons)


def test_error_growing_with_T_fails():
    res = fallback.analyse(_cases(torch.float32, "grows_with_T"))
    assert res.verdict == "FAIL"
    assert any("grows" in r for r in res.reasons)


def test_error_growing_with_T_never_passes_in_bf16():
    """In bfloat16 the output's rounding hides most of the planted growth at
    small T; the analysis must still not pass it."""
    res = fallback.analyse(_cases(torch.bfloat16, "grows_with_T"))
    assert res.verdict in ("FAIL", "INCONCLUSIVE")


def test_wide_noise_is_inconclusive():
    res = fallback.analyse(_cases(torch.float32, "noise"))
    assert res.verdict == "INCONCLUSIVE"


def test_legal_column_sums_are_float32_sums_in_other_orders():
    g = np.random.default_rng(5)
    terms = torch.from_numpy(g.standard_normal((64, 7)).astype(np.float32))
    sums = fallback.legal_column_sums(terms, k=4, seed=3)
    exact = terms.double().sum(0).numpy()
    bound = 63 * fallback.U32 * terms.double().abs().sum(0).numpy()
    seq = torch.zeros(7)
    for i in range(63, -1, -1):
        seq = seq + terms[i]
    assert torch.equal(sums[0], seq)                      # back to front
    for s_ in sums:
        assert np.all(np.abs(s_.double().numpy() - exact) <= bound)
    assert len({tuple(s_.tolist()) for s_ in sums}) > 1    # orders differ


def test_the_gate_rejects_legal_orders_of_small_column_sums():
    """What step 1 measures, shown on the CPU: for 64-row column sums of 2
    columns, the gate (2x the float32 reference's error) rejects some plain
    float32 sums taken in other row orders -- it cannot decide there."""
    from oracle import gate
    inp = workloads.make_layernorm_tile_case((64, 2), torch.bfloat16, 100)
    x, w, dy, eps = inp["x"], inp["w"], inp["dy"], inp["eps"]
    dg_g, _ = lnref.golden_ln_param_grads(dy, x, eps)
    dg_r = lnref.reference_ln_backward(dy, x, w, eps)[1]
    terms, _ = lnref.reference_ln_param_terms(dy, x, eps)
    verdicts = [gate.gate_tensor("dgamma", c, dg_r, dg_g, torch.float32).verdict
                for c in fallback.legal_column_sums(terms, k=16, seed=1)]
    assert "FAIL" in verdicts
