"""Numerics gate for target (kernel) outputs (test infrastructure only).

Follows the torchtitan kernel-numerics-verifier page:

* section "正确性判据" (correctness gate).  For each output tensor, in the
  golden's float64::

      reference_error = max|reference - golden|
      target_error    = max|target - golden|
      rounding_floor  = max|golden.to(target dtype).to(float64) - golden|
      absolute_floor  = max(project_atol, rounding_floor)
      threshold       = fudge_factor * reference_error + absolute_floor
      PASS  iff  target_error <= threshold

  The page's text lost its operators in extraction; the reading used here is
  the one its prose supports ("the kernel error is at most fudge_factor times
  the reference's, with the rounding floor added on top").
* workflow step 3: structure first -- shape, dtype and the positions of NaN,
  +Inf and -Inf must match before any number is compared.
* section "先检查条件数" (conditioning first):
  ``reference_error / max(max|golden|, absolute_floor)`` above
  MAX_REFERENCE_RELATIVE_ERROR makes the gate invalid: no PASS/FAIL is given,
  the verdict is INCONCLUSIVE.
* section "结果报告规范" (report format): one row per tensor and one overall
  verdict.

The constants below were fixed before any kernel existed and are never raised
to let a failing kernel through (same section of the page).

Two checks are added on top of the page's gate and declared here with it:

* rstd (the per-row inverse RMS the forward stores for the backward) must be
  within RSTD_MAX_REL_ERROR of the golden r, relative, elementwise.
* rounding bias: for bfloat16/float16 outputs the max-error gate cannot tell
  round-to-nearest-even from truncation (truncation stays within one unit in
  the last place), so the signed error measured along the sign of the golden,
  ``sum(e * sign(golden)) / sum|e|``, must stay within ROUNDING_BIAS_MAX in
  magnitude (truncation toward zero gives exactly -1; unbiased rounding ~0).
"""
from __future__ import annotations

from dataclasses import dataclass, field, asdict

import numpy as np
import torch

# ---- constants, declared before any kernel ran -------------------------------
FUDGE_FACTOR = 2.0
PROJECT_ATOL = 0.0
MAX_REFERENCE_RELATIVE_ERROR = 0.1
RSTD_MAX_REL_ERROR = 1e-6
ROUNDING_BIAS_MAX = 0.25
ROUNDING_BIAS_MIN_ELEMENTS = 4096
# ------------------------------------------------------------------------------

# The page "Check an AI model calculation before accelerating it" (section
# "Three distinct numerical comparisons") declares allclose tolerances for the
# kernel against its same-dtype reference: |target - reference| <= atol +
# rtol*|reference| elementwise, atol 1e-5 and rtol 1e-4 in float32, atol =
# rtol = 3e-3 in float16.  They are logged beside each gate row as
# information only (the gate decides); the page declares none for bfloat16.
PAGE_ALLCLOSE = {"float32": (1e-5, 1e-4), "float16": (3e-3, 3e-3)}

_TORCH_DTYPES = {
    "float32": torch.float32, "fp32": torch.float32, torch.float32: torch.float32,
    "float16": torch.float16, "fp16": torch.float16, torch.float16: torch.float16,
    "bfloat16": torch.bfloat16, "bf16": torch.bfloat16, torch.bfloat16: torch.bfloat16,
}


def _as_torch_dtype(d):
    return _TORCH_DTYPES[d]


def _to_f64(a):
    if hasattr(a, "detach"):
        return a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def _dtype_name(a):
    if hasattr(a, "dtype") and isinstance(a.dtype, torch.dtype):
        return str(a.dtype).replace("torch.", "")
    return str(np.asarray(a).dtype)


def rounding_floor(golden, out_dtype):
    """max|golden.to(out_dtype).to(float64) - golden| over finite elements."""
    g = torch.from_numpy(np.ascontiguousarray(golden, dtype=np.float64))
    finite = torch.isfinite(g)
    if not bool(finite.any()):
        return 0.0
    rt = g.to(_as_torch_dtype(out_dtype)).double()
    return float((rt - g).abs()[finite].max())


def structure_mismatch(target, golden, expected_dtype=None):
    """Returns None when the structure matches, else a description."""
    t = _to_f64(target)
    if t.shape != golden.shape:
        return f"shape {t.shape} != golden {golden.shape}"
    if expected_dtype is not None:
        want = str(_as_torch_dtype(expected_dtype)).replace("torch.", "")
        have = _dtype_name(target)
        if have != want:
            return f"dtype {have} != expected {want}"
    for what, fn in (("NaN", np.isnan),
                     ("+Inf", lambda a: np.isposinf(a)),
                     ("-Inf", lambda a: np.isneginf(a))):
        mt, mg = fn(t), fn(golden)
        if not np.array_equal(mt, mg):
            bad = int(np.count_nonzero(mt != mg))
            return f"{what} positions differ at {bad} element(s)"
    return None


def _max_abs_err(a, golden):
    mask = np.isfinite(golden)
    if not mask.any():
        return 0.0
    return float(np.max(np.abs(a[mask] - golden[mask])))


def rounding_bias(target, golden):
    """sum(e*sign(golden))/sum|e| with e = target - golden (finite, e != 0)."""
    t = _to_f64(target).ravel()
    g = np.asarray(golden, dtype=np.float64).ravel()
    mask = np.isfinite(g) & np.isfinite(t)
    e = t[mask] - g[mask]
    s = np.sign(g[mask])
    keep = (e != 0) & (s != 0)
    if np.count_nonzero(keep) < ROUNDING_BIAS_MIN_ELEMENTS:
        return None
    e, s = e[keep], s[keep]
    return float(np.sum(e * s) / np.sum(np.abs(e)))


@dataclass
class GateRow:
    tensor: str
    dtype: str
    shape: tuple
    reference_error: float = float("nan")
    target_error: float = float("nan")
    rounding_floor: float = float("nan")
    absolute_floor: float = float("nan")
    threshold: float = float("nan")
    golden_scale: float = float("nan")
    reference_relative_error: float = float("nan")
    condition: float | None = None
    bias_target: float | None = None
    bias_reference: float | None = None
    gate_valid: bool = False
    verdict: str = "FAIL"
    note: str = ""
    extra: dict = field(default_factory=dict)

    def as_dict(self):
        d = asdict(self)
        d["shape"] = list(self.shape)
        return d


class TensorGate:
    """The gate of one output tensor, fed in row chunks.

    ``add(target, reference, golden)`` takes one chunk of rows (the golden
    float64 NumPy); ``finish()`` returns the GateRow.  Every quantity of the
    gate is a maximum (reference and target error, rounding floor, golden
    scale) or a sum (the rounding-bias numerator and denominator), so a tensor
    fed in chunks gets the row it would get whole: full-size tensors can be
    gated on every element without holding them in float64 at once."""

    def __init__(self, name, out_dtype, shape, condition=None, fudge=FUDGE_FACTOR,
                 project_atol=PROJECT_ATOL, max_ref_rel=MAX_REFERENCE_RELATIVE_ERROR):
        self.out_dtype = out_dtype
        self.want = str(_as_torch_dtype(out_dtype)).replace("torch.", "")
        self.row = GateRow(tensor=name, dtype=self.want, shape=tuple(shape), condition=condition)
        self.fudge, self.project_atol, self.max_ref_rel = fudge, project_atol, max_ref_rel
        self.failed = None      # structure failure of the target
        self.ref_failed = None  # structure failure of the reference
        self.ref_err = self.tgt_err = self.floor = self.scale = 0.0
        self.bias = {"t": [0.0, 0.0, 0], "r": [0.0, 0.0, 0]}  # sum(e*s), sum|e|, count
        self.any_finite = False
        self.allclose_bad = 0   # elements outside the page's allclose rule
        self.allclose_n = 0

    @staticmethod
    def _bias_terms(a, g, acc):
        mask = np.isfinite(g) & np.isfinite(a)
        e = a[mask] - g[mask]
        sg = np.sign(g[mask])
        keep = (e != 0) & (sg != 0)
        e, sg = e[keep], sg[keep]
        acc[0] += float(np.sum(e * sg))
        acc[1] += float(np.sum(np.abs(e)))
        acc[2] += int(e.size)

    def add(self, target, reference, golden):
        golden = np.asarray(golden, dtype=np.float64)
        if self.failed is not None:
            return
        why = structure_mismatch(target, golden, self.out_dtype)
        if why is not None:
            self.failed = why
            return
        if self.ref_failed is None:
            why = structure_mismatch(reference, golden, self.out_dtype)
            if why is not None:
                self.ref_failed = why
                return
        t = _to_f64(target)
        r = _to_f64(reference)
        self.ref_err = max(self.ref_err, _max_abs_err(r, golden))
        self.tgt_err = max(self.tgt_err, _max_abs_err(t, golden))
        self.floor = max(self.floor, rounding_floor(golden, self.out_dtype))
        fin = np.isfinite(golden)
        if fin.any():
            self.any_finite = True
            self.scale = max(self.scale, float(np.max(np.abs(golden[fin]))))
        if self.want in ("bfloat16", "float16"):
            self._bias_terms(t.ravel(), golden.ravel(), self.bias["t"])
            self._bias_terms(r.ravel(), golden.ravel(), self.bias["r"])
        if self.want in PAGE_ALLCLOSE:
            atol, rtol = PAGE_ALLCLOSE[self.want]
            both = np.isfinite(t) & np.isfinite(r)
            bad = np.abs(t[both] - r[both]) > atol + rtol * np.abs(r[both])
            self.allclose_bad += int(np.count_nonzero(bad))
            self.allclose_n += int(np.count_nonzero(both))

    @staticmethod
    def _bias(acc):
        if acc[2] < ROUNDING_BIAS_MIN_ELEMENTS:
            return None
        return acc[0] / acc[1]

    def finish(self):
        row = self.row
        if self.want in PAGE_ALLCLOSE and self.failed is None and self.ref_failed is None:
            atol, rtol = PAGE_ALLCLOSE[self.want]
            row.extra["allclose"] = {"atol": atol, "rtol": rtol, "outside": self.allclose_bad,
                                     "elements": self.allclose_n,
                                     "verdict": self.allclose_bad == 0}
        if self.failed is not None:
            row.verdict = "FAIL"
            row.note = "structure: " + self.failed
            return row
        if self.ref_failed is not None:
            row.verdict = "INCONCLUSIVE"
            row.note = "reference structure: " + self.ref_failed
            return row
        row.reference_error = self.ref_err
        row.target_error = self.tgt_err
        row.rounding_floor = self.floor
        row.absolute_floor = max(self.project_atol, row.rounding_floor)
        row.threshold = self.fudge * row.reference_error + row.absolute_floor
        row.golden_scale = self.scale if self.any_finite else 0.0
        denom = max(row.golden_scale, row.absolute_floor)
        if denom > 0:
            row.reference_relative_error = row.reference_error / denom
        else:
            row.reference_relative_error = 0.0 if row.reference_error == 0 else float("inf")
        row.gate_valid = row.reference_relative_error <= self.max_ref_rel
        if not row.gate_valid:
            row.verdict = "INCONCLUSIVE"
            row.note = "reference is too inaccurate to gate the target"
            return row
        ok = row.target_error <= row.threshold
        notes = []
        if self.want in ("bfloat16", "float16"):
            row.bias_target = self._bias(self.bias["t"])
            row.bias_reference = self._bias(self.bias["r"])
            if row.bias_target is not None:
                lim = ROUNDING_BIAS_MAX
                if row.bias_reference is not None:
                    lim = max(lim, 2.0 * abs(row.bias_reference))
                if abs(row.bias_target) > lim:
                    ok = False
                    notes.append(f"rounding bias {row.bias_target:+.3f} beyond {lim:.3f}")
        if row.target_error > row.threshold:
            notes.append("target_error above threshold")
        row.verdict = "PASS" if ok else "FAIL"
        row.note = "; ".join(notes)
        return row


def gate_tensor(name, target, reference, golden, out_dtype, condition=None,
                fudge=FUDGE_FACTOR, project_atol=PROJECT_ATOL,
                max_ref_rel=MAX_REFERENCE_RELATIVE_ERROR):
    """Gate one output tensor.  ``golden`` is float64 NumPy."""
    golden = np.asarray(golden, dtype=np.float64)
    g = TensorGate(name, out_dtype, golden.shape, condition, fudge, project_atol, max_ref_rel)
    g.add(target, reference, golden)
    return g.finish()


def gate_rstd(target_rstd, golden_r, reference_rstd=None,
              max_rel=RSTD_MAX_REL_ERROR):
    """rstd check: max_i |rstd_i - r_i| / r_i <= max_rel (float32 output)."""
    g = np.asarray(golden_r, dtype=np.float64).ravel()
    row = GateRow(tensor="rstd", dtype="float32", shape=tuple(g.shape))
    why = structure_mismatch(np.asarray(_to_f64(target_rstd)).ravel(), g)
    if why is None and _dtype_name(target_rstd) != "float32":
        why = f"dtype {_dtype_name(target_rstd)} != expected float32"
    if why is not None:
        row.verdict, row.note = "FAIL", "structure: " + why
        return row
    t = _to_f64(target_rstd).ravel()
    row.target_error = float(np.max(np.abs(t - g) / g)) if g.size else 0.0
    if reference_rstd is not None and g.size:
        rr = _to_f64(reference_rstd).ravel()
        row.reference_error = float(np.max(np.abs(rr - g) / g))
        atol, rtol = PAGE_ALLCLOSE["float32"]
        bad = int(np.count_nonzero(np.abs(t - rr) > atol + rtol * np.abs(rr)))
        row.extra["allclose"] = {"atol": atol, "rtol": rtol, "outside": bad,
                                 "elements": int(g.size), "verdict": bad == 0}
    row.threshold = max_rel
    row.absolute_floor = 0.0
    row.golden_scale = float(np.max(np.abs(g))) if g.size else 0.0
    row.gate_valid = True
    row.verdict = "PASS" if row.target_error <= max_rel else "FAIL"
    row.note = "relative error, elementwise"
    return row


# LayerNorm row statistics.  A row's mean and inverse standard deviation are
# each one sum over the row, so comparing two float32 evaluations of them
# compares rounding luck, not correctness: they are checked against the
# float64 golden with fixed bounds instead.  The mean: one float32 unit in the
# last place of the exact mean plus 2^-36 of the row's largest |x| (room for
# the rounding of a float64 accumulation over up to 2^14 terms).  rstd: the
# RMSNorm bound, RSTD_MAX_REL_ERROR relative.
MEAN_ROW_ABS_SLACK = 2.0 ** -36


def gate_mean(target_mean, golden_mean, row_absmax):
    """|mean_i - mu_i| <= 2^-23 |mu_i| + 2^-36 max_j |x_ij| for every row."""
    g = np.asarray(golden_mean, dtype=np.float64).ravel()
    a = np.asarray(row_absmax, dtype=np.float64).ravel()
    row = GateRow(tensor="mean", dtype="float32", shape=tuple(g.shape))
    why = structure_mismatch(np.asarray(_to_f64(target_mean)).ravel(), g)
    if why is None and _dtype_name(target_mean) != "float32":
        why = f"dtype {_dtype_name(target_mean)} != expected float32"
    if why is not None:
        row.verdict, row.note = "FAIL", "structure: " + why
        return row
    t = _to_f64(target_mean).ravel()
    bound = 2.0 ** -23 * np.abs(g) + MEAN_ROW_ABS_SLACK * a
    err = np.abs(t - g)
    row.target_error = float(np.max(err)) if g.size else 0.0
    row.threshold = float(np.max(err / np.where(bound > 0, bound, 1.0))) if g.size else 0.0
    row.absolute_floor = 0.0
    row.golden_scale = float(np.max(np.abs(g))) if g.size else 0.0
    row.gate_valid = True
    row.verdict = "PASS" if bool(np.all(err <= bound)) else "FAIL"
    row.note = "per-row bound 2^-23|mu| + 2^-36 max|x| (threshold column: worst error/bound)"
    return row


def overall_verdict(rows):
    """One verdict for the report (torchtitan page, report section): FAIL if
    any row fails, else INCONCLUSIVE if any row is, else PASS WITH
    LIMITATIONS if any row is, else PASS."""
    verdicts = [r.verdict for r in rows]
    if any(v == "FAIL" for v in verdicts):
        return "FAIL"
    if any(v == "INCONCLUSIVE" for v in verdicts):
        return "INCONCLUSIVE"
    if any(v == "PASS WITH LIMITATIONS" for v in verdicts):
        return "PASS WITH LIMITATIONS"
    return "PASS"


def report(rows, title=""):
    """Markdown table in the page's report layout plus the overall verdict."""
    lines = []
    if title:
        lines.append(f"### {title}")
    lines.append("| Tensor | Ref/golden | Condition | Target error | Threshold | Gate valid | Verdict |")
    lines.append("|---|---|---|---|---|---|---|")
    for r in rows:
        cond = "-" if r.condition is None else f"{r.condition:.3g}"
        lines.append(
            f"| {r.tensor} ({r.dtype}) | {r.reference_error:.3e} | {cond} | "
            f"{r.target_error:.3e} | {r.threshold:.3e} | {r.gate_valid} | "
            f"{r.verdict}{' — ' + r.note if r.note else ''} |")
    lines.append(f"\nOverall: **{overall_verdict(rows)}**")
    info = []
    for r in rows:
        a = r.extra.get("allclose") if r.extra else None
        if a is not None:
            info.append(f"{r.tensor} {a['verdict']} ({a['outside']} of {a['elements']} outside "
                        f"atol {a['atol']:g}, rtol {a['rtol']:g})")
    if info:
        lines.append("Page allclose against the reference (information only): " + "; ".join(info))
    return "\n".join(lines)
