"""The analysis that replaces the gate where the gate is invalid (test
infrastructure only).

The torchtitan kernel-numerics-verifier page (section "gate 失效时的三步替代
分析") prescribes three steps for an output whose same-precision reference is
too inaccurate to calibrate the gate (reference relative error above its 10%
trigger):

1. compare two legal float32 evaluation orders of the formula, which measures
   how sensitive the result is to the order of the arithmetic;
2. repeat over several reduction lengths T and random seeds: an error that
   grows about like sqrt(T) is zero-mean rounding noise, one that grows like
   T is a systematic bias; record the conditioning at each T and compare the
   error distributions and bias of the reference and the target;
3. a bias, scaling or mismatch of the target that the references do not
   share is a FAIL.

It ends in PASS WITH LIMITATIONS when the target and the references follow one
conditioning-driven noise envelope, INCONCLUSIVE when the evidence cannot
separate rounding noise from a bug.

The envelope is written per element: ``env_i = u * S_i + floor_i``, where u =
2^-24 is the float32 unit roundoff, ``S_i`` the sum of the magnitudes of the
terms the formula adds for element i (the numerator of its condition number),
and ``floor_i`` the rounding of the float64 golden to the output dtype.  Any
float32 evaluation of the formula is off by a modest multiple of ``u * S_i``
before the output is rounded; dividing errors by ``env_i`` puts target and
references on one scale.

Checks (constants fixed here with the gate's, before any target is looked
at):

* envelope: at every (T, seed), the target's largest normalised error is at
  most FUDGE_FACTOR times the larger of the two references' largest
  normalised errors and their mutual distance (step 1's order sensitivity),
  and at least one envelope unit;
* growth: across the T sweep, the slope of log(rms normalised error)
  against log(T) of the target exceeds max(0, the references' slope) by at
  most GROWTH_SLOPE_SLACK (0.5: the distance between sqrt(T) and T growth).
  In envelope units an error that is rounding noise does not grow with T;
  one that grows like T is systematic.  The root mean square over all
  elements and seeds of a T is used rather than the maximum, which a few
  cancelling elements decide; raw errors would mislead where the references
  are far less accurate than the target at small T;
* bias: over every element of the sweep, the target's signed error along the
  golden's sign, sum(e*sign(g))/sum|e|, stays within ROUNDING_BIAS_MAX (or
  twice the references', if larger), once ROUNDING_BIAS_MIN_ELEMENTS errors
  are non-zero.

Verdict: FAIL if the growth or bias check fails; PASS WITH LIMITATIONS if the
envelope check holds everywhere; INCONCLUSIVE otherwise.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from .gate import FUDGE_FACTOR, ROUNDING_BIAS_MAX, ROUNDING_BIAS_MIN_ELEMENTS, _as_torch_dtype

U32 = 2.0 ** -24
GROWTH_SLOPE_SLACK = 0.5


@dataclass
class Case:
    """One (T, seed) point of the sweep: the target, two float32 references
    in different legal orders, the float64 golden and the per-element
    magnitude sum S of the formula's terms (all the same shape)."""
    T: int
    seed: int
    target: np.ndarray
    ref_a: np.ndarray
    ref_b: np.ndarray
    golden: np.ndarray
    magnitude: np.ndarray
    out_dtype: object


@dataclass
class CaseRow:
    T: int
    seed: int
    target_norm: float
    ref_norm: float
    order_gap_norm: float
    envelope_ok: bool
    target_max_err: float
    ref_max_err: float
    condition_max: float


@dataclass
class FallbackResult:
    rows: list
    target_slope: float
    ref_slope: float
    bias_target: float | None
    bias_reference: float | None
    verdict: str
    reasons: list = field(default_factory=list)


def _f64(a):
    if hasattr(a, "detach"):
        return a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def _envelope(case):
    g = np.asarray(case.golden, dtype=np.float64)
    rounded = torch.from_numpy(g).to(_as_torch_dtype(case.out_dtype)).double().numpy()
    return U32 * np.asarray(case.magnitude, dtype=np.float64) + np.abs(rounded - g)


def _slope(Ts, errs):
    """Least-squares slope of log(err) against log(T) (errors floored at the
    smallest positive one, so an exact result does not dominate)."""
    Ts, errs = np.asarray(Ts, dtype=np.float64), np.asarray(errs, dtype=np.float64)
    pos = errs[errs > 0]
    if Ts.size < 2 or pos.size == 0:
        return 0.0
    e = np.maximum(errs, pos.min())
    return float(np.polyfit(np.log(Ts), np.log(e), 1)[0])


def _bias_sums(err_signed, g, acc):
    s = np.sign(g)
    keep = (err_signed != 0) & (s != 0) & np.isfinite(err_signed)
    acc[0] += float(np.sum(err_signed[keep] * s[keep]))
    acc[1] += float(np.sum(np.abs(err_signed[keep])))
    acc[2] += int(np.count_nonzero(keep))


def analyse(cases):
    """Run the three steps over the sweep ``cases`` and return the verdict."""
    rows = []
    per_T_t, per_T_r = {}, {}
    bt, br = [0.0, 0.0, 0], [0.0, 0.0, 0]
    envelope_ok = True
    for c in cases:
        g = np.asarray(c.golden, dtype=np.float64)
        t, ra, rb = _f64(c.target), _f64(c.ref_a), _f64(c.ref_b)
        env = _envelope(c)
        env = np.where(env > 0, env, np.finfo(np.float64).tiny)
        et, ea, eb = np.abs(t - g), np.abs(ra - g), np.abs(rb - g)
        tn = float(np.max(et / env))
        rn = float(max(np.max(ea / env), np.max(eb / env)))
        gn = float(np.max(np.abs(ra - rb) / env))
        ok = tn <= FUDGE_FACTOR * max(rn, gn, 1.0)
        envelope_ok &= ok
        mag = np.asarray(c.magnitude, dtype=np.float64)
        cond = float(np.max(mag / np.maximum(np.abs(g), np.finfo(np.float64).tiny)))
        rows.append(CaseRow(c.T, c.seed, tn, rn, gn, ok, float(et.max()),
                            float(max(ea.max(), eb.max())), cond))
        qt, qr = per_T_t.setdefault(c.T, [0.0, 0]), per_T_r.setdefault(c.T, [0.0, 0])
        qt[0] += float(np.sum((et / env) ** 2))
        qt[1] += et.size
        qr[0] += float(np.sum((ea / env) ** 2) + np.sum((eb / env) ** 2))
        qr[1] += ea.size + eb.size
        _bias_sums(t - g, g, bt)
        _bias_sums(ra - g, g, br)
        _bias_sums(rb - g, g, br)
    Ts = sorted(per_T_t)
    ts = _slope(Ts, [np.sqrt(per_T_t[T][0] / per_T_t[T][1]) for T in Ts])
    rs = _slope(Ts, [np.sqrt(per_T_r[T][0] / per_T_r[T][1]) for T in Ts])
    bias_t = bt[0] / bt[1] if bt[2] >= ROUNDING_BIAS_MIN_ELEMENTS else None
    bias_r = br[0] / br[1] if br[2] >= ROUNDING_BIAS_MIN_ELEMENTS else None
    reasons = []
    fail = False
    if ts > max(rs, 0.0) + GROWTH_SLOPE_SLACK:
        fail = True
        reasons.append(f"target error (envelope units) grows with T at slope {ts:.2f} "
                       f"against {rs:.2f} for the references")
    if bias_t is not None:
        lim = ROUNDING_BIAS_MAX if bias_r is None else max(ROUNDING_BIAS_MAX, 2 * abs(bias_r))
        if abs(bias_t) > lim:
            fail = True
            reasons.append(f"target rounding bias {bias_t:+.3f} beyond {lim:.3f}")
    if fail:
        verdict = "FAIL"
    elif envelope_ok:
        verdict = "PASS WITH LIMITATIONS"
    else:
        verdict = "INCONCLUSIVE"
        reasons.append("target outside the references' noise envelope at some (T, seed)")
    return FallbackResult(rows, ts, rs, bias_t, bias_r, verdict, reasons)


def legal_column_sums(terms, k=8, seed=0):
    """``k`` legal float32 evaluations of the column sums of ``terms`` (an
    [M, N] float32 tensor of per-row contributions): plain sequential
    accumulations over the rows, the first back to front, the others in
    random row orders drawn from ``seed``.  Step 1 of the analysis uses them
    to test whether the gate can decide a column sum at all: a gate that
    rejects one of them rejects correct float32 arithmetic, and cannot tell a
    bug from rounding order (the gate is then invalid for that tensor)."""
    t = terms.detach().to("cpu").float()
    rng = np.random.default_rng(seed)
    orders = [np.arange(t.shape[0])[::-1]] + [rng.permutation(t.shape[0]) for _ in range(k - 1)]
    out = []
    for order in orders:
        acc = torch.zeros(t.shape[1], dtype=torch.float32)
        for i in order:
            acc = acc + t[int(i)]
        out.append(acc)
    return out


def report(res, title=""):
    """Markdown table of the sweep and the verdict."""
    lines = [f"### {title}"] if title else []
    lines.append("| T | seed | target / env | refs / env | order gap / env | within envelope "
                 "| target max err | refs max err | max condition |")
    lines.append("|---|---|---|---|---|---|---|---|---|")
    for r in res.rows:
        lines.append(f"| {r.T} | {r.seed} | {r.target_norm:.2f} | {r.ref_norm:.2f} | "
                     f"{r.order_gap_norm:.2f} | {r.envelope_ok} | {r.target_max_err:.3e} | "
                     f"{r.ref_max_err:.3e} | {r.condition_max:.3g} |")
    bt = "-" if res.bias_target is None else f"{res.bias_target:+.3f}"
    br = "-" if res.bias_reference is None else f"{res.bias_reference:+.3f}"
    lines.append(f"\nGrowth slope in T of the rms error in envelope units: target "
                 f"{res.target_slope:.2f}, "
                 f"references {res.ref_slope:.2f}.  Rounding bias: target {bt}, "
                 f"references {br}.")
    lines.append(f"Verdict: **{res.verdict}**" + (" — " + "; ".join(res.reasons)
                                                   if res.reasons else ""))
    return "\n".join(lines)
