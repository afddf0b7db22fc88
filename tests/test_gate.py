"""The same-dtype reference and the numerics gate, exercised on the CPU.

Targets here are CPU stand-ins: a correct float32 implementation (must PASS)
and variants carrying one mistake each (must FAIL), so the gate is shown to
catch them before any kernel is judged by it.  Mistakes (torchtitan page,
"九步工作流" step 9 lists where bugs hide; page "Check an AI model
calculation before accelerating it" gives the N-vs-BLOCK and sum-vs-mean
traps): padded denominator, mean instead of sum for dgamma, r^2 instead of r^3,
squaring fp16 before the upcast, truncating instead of rounding to nearest
even, and an output element never written.
"""
import numpy as np
import pytest
import torch

from oracle import gate, golden, reference
from backward_rmsnorm_fwd_amd import workloads

EPS = 1e-6


def _next_pow2(n):
    return 1 << (n - 1).bit_length()


def stand_in(x, w, dy, eps=EPS, offset=False, mutation=None):
    """A CPU target with float32 intermediates and optional planted mistake.

    Returns y, rstd, dx, dgamma in the kernel's output dtypes."""
    T = x.dtype
    n = x.shape[-1]
    den = _next_pow2(n) if mutation == "padded_denominator" else n
    if mutation == "square_before_upcast":
        ss = (x * x).float().sum(-1, keepdim=True)  # squares in T: may overflow
    else:
        xf0 = x.float()
        ss = (xf0 * xf0).sum(-1, keepdim=True)
    xf = x.float()
    g = w.float()
    if offset:
        g = 1.0 + g
    r = torch.rsqrt(ss / den + eps)
    y32 = xf * r * g
    u = dy.float() * g
    p = 2 if mutation == "r_squared" else 3
    dx32 = r * u - xf * r.pow(p) * (u * xf).sum(-1, keepdim=True) / den
    contrib = dy.float() * xf * r
    dgamma = contrib.mean(0) if mutation == "dgamma_mean" else contrib.sum(0)

    def cast(v):
        if mutation == "truncate" and T == torch.bfloat16:
            bits = v.contiguous().view(torch.int32) & ~0xFFFF
            return bits.view(torch.float32).to(T)  # exact: low bits are zero
        return v.to(T)

    y, dx = cast(y32), cast(dx32)
    if mutation == "unwritten":
        y = y.clone()
        y.view(-1)[7] = float("nan")  # stands for a never-written, NaN-poisoned slot
    return y, r.squeeze(-1), dx, dgamma


def run_gate(inp, mutation=None):
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    off, eps = inp["offset"], inp["eps"]
    T = x.dtype
    y_t, r_t, dx_t, dg_t = stand_in(x, w, dy, eps, off, mutation)
    y_r, r_r = reference.reference_forward(x, w, eps, off)
    dx_r, dg_r = reference.reference_backward(dy, x, w, eps, off)
    y_g, r_g = golden.golden_forward(x, w, eps, off)
    dx_g, dg_g = golden.golden_backward(dy, x, w, eps, off)
    n = x.shape[-1]
    rows = [
        gate.gate_tensor("y", y_t.reshape(-1, n), y_r, y_g, T),
        gate.gate_rstd(r_t.reshape(-1), r_g, r_r),
        gate.gate_tensor("dx", dx_t.reshape(-1, n), dx_r, dx_g, T),
        gate.gate_tensor("dgamma", dg_t, dg_r, dg_g, torch.float32),
    ]
    return rows


def verdicts(rows):
    return {r.tensor: r.verdict for r in rows}


@pytest.mark.parametrize("name", ["c1a", "c1b", "c1c"])
def test_correct_stand_in_passes_small_configs(name):
    rows = run_gate(workloads.make_inputs(name))
    assert gate.overall_verdict(rows) == "PASS", gate.report(rows)


@pytest.mark.parametrize("name,M,N", [("c2", 96, 4096), ("c3", 3000, 1024),
                                      ("c4", 6, 65536), ("c5", 80, 5120)])
def test_correct_stand_in_passes_scaled_down_configs(name, M, N):
    rows = run_gate(workloads.make_inputs(name, M=M, N=N))
    assert gate.overall_verdict(rows) == "PASS", gate.report(rows)


def test_padded_denominator_caught_at_257_not_at_256():
    bad = run_gate(workloads.make_tile_case((3, 257), torch.float32, 1), "padded_denominator")
    assert verdicts(bad)["y"] == "FAIL" and verdicts(bad)["dx"] == "FAIL"
    same = run_gate(workloads.make_tile_case((3, 256), torch.float32, 1), "padded_denominator")
    assert gate.overall_verdict(same) == "PASS"


def test_dgamma_mean_caught_at_m17_not_at_m1():
    inp17 = workloads.make_tile_case((17, 64), torch.float32, 2)
    assert verdicts(run_gate(inp17, "dgamma_mean"))["dgamma"] == "FAIL"
    inp1 = workloads.make_tile_case((1, 64), torch.float32, 2)
    assert verdicts(run_gate(inp1, "dgamma_mean"))["dgamma"] == "PASS"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_r_squared_caught(dtype):
    # rows with rms ~4, so that r^2 and r^3 differ by a factor of ~4
    inp = workloads.make_tile_case((8, 512), dtype, 3, scale=4.0)
    assert verdicts(run_gate(inp, "r_squared"))["dx"] == "FAIL"


def test_square_before_upcast_caught_on_scaled_fp16_rows():
    inp = workloads.make_inputs("c3", M=1000, N=256)
    v = verdicts(run_gate(inp, "square_before_upcast"))
    assert v["y"] == "FAIL" and v["rstd"] == "FAIL"


def test_truncation_caught_by_rounding_bias():
    inp = workloads.make_inputs("c2", M=32, N=4096)
    rows = run_gate(inp, "truncate")
    v = verdicts(rows)
    assert v["y"] == "FAIL" and v["dx"] == "FAIL"
    y_row = [r for r in rows if r.tensor == "y"][0]
    # the max-error gate alone would let truncation through
    assert y_row.target_error <= y_row.threshold
    assert y_row.bias_target < -0.9


def test_unwritten_element_caught_by_structure_check():
    rows = run_gate(workloads.make_inputs("c1a"), "unwritten")
    y_row = [r for r in rows if r.tensor == "y"][0]
    assert y_row.verdict == "FAIL" and "NaN" in y_row.note


def test_gate_inconclusive_when_reference_is_too_inaccurate():
    g = np.linspace(-1, 1, 64)
    ref = torch.tensor(g * 1.5, dtype=torch.float32)  # 50% relative error
    row = gate.gate_tensor("t", torch.tensor(g, dtype=torch.float32), ref, g, torch.float32)
    assert row.verdict == "INCONCLUSIVE" and not row.gate_valid


def test_gate_rstd_threshold():
    r = np.linspace(0.5, 1000.0, 50)
    ok = gate.gate_rstd(torch.tensor(r * (1 + 5e-7), dtype=torch.float32), r)
    bad = gate.gate_rstd(torch.tensor(r * (1 + 3e-6), dtype=torch.float32), r)
    assert ok.verdict == "PASS" and bad.verdict == "FAIL"
    wrong_dtype = gate.gate_rstd(torch.tensor(r, dtype=torch.float64), r)
    assert wrong_dtype.verdict == "FAIL"


def test_gate_dtype_mismatch_fails():
    g = np.linspace(-1, 1, 64)
    t = torch.tensor(g, dtype=torch.float32)
    row = gate.gate_tensor("t", t, t.to(torch.bfloat16), g, torch.bfloat16)
    assert row.verdict == "FAIL" and "dtype" in row.note


def test_rounding_floor_is_half_ulp_scale():
    g = np.array([1.0 + 2.0 ** -9, 3.0])  # halfway between bf16 neighbours of 1
    assert gate.rounding_floor(g, torch.bfloat16) == pytest.approx(2.0 ** -9)


def test_reference_matches_its_own_autograd():
    inp = workloads.make_tile_case((8, 300), torch.float32, 4)
    for off in (False, True):
        dx, dg = reference.reference_backward(inp["dy"], inp["x"], inp["w"], EPS, off)
        dxa, dga = reference.reference_backward_autograd(inp["dy"], inp["x"], inp["w"], EPS, off)
        assert torch.allclose(dx, dxa, rtol=1e-5, atol=1e-6)
        assert torch.allclose(dg, dga, rtol=1e-5, atol=1e-6)


def test_reference_close_to_golden_in_fp32():
    inp = workloads.make_tile_case((16, 1000), torch.float32, 5)
    y, r = reference.reference_forward(inp["x"], inp["w"], EPS)
    yg, rg = golden.golden_forward(inp["x"], inp["w"], EPS)
    assert np.allclose(y.double().numpy(), yg, rtol=1e-5, atol=1e-6)
    assert np.allclose(r.double().numpy(), rg, rtol=1e-6, atol=0)


def test_report_layout():
    rows = run_gate(workloads.make_inputs("c1b"))
    text = gate.report(rows, "c1b")
    assert "| Tensor | Ref/golden | Condition | Target error | Threshold | Gate valid | Verdict |" in text
    assert "Overall: **PASS**" in text


def test_gate_mean_bounds():
    """The LayerNorm mean check: a correctly rounded float32 mean passes, one
    four float32 ulps away fails; a zero mean is held to the 2^-36 max|x|
    slack only."""
    g = np.array([1.0 / 3.0, -12.5 + 1e-9, 0.0])
    absmax = np.array([2.0, 20.0, 1.0])
    t = torch.tensor(g, dtype=torch.float32)
    assert gate.gate_mean(t, g, absmax).verdict == "PASS"
    bad = t.clone()
    bad[0] = float(np.float32(g[0]) + 4 * np.spacing(np.float32(g[0])))
    assert gate.gate_mean(bad, g, absmax).verdict == "FAIL"
    bad = t.clone()
    bad[2] = 2.0 ** -30
    assert gate.gate_mean(bad, g, absmax).verdict == "FAIL"
    bad[2] = 2.0 ** -38
    assert gate.gate_mean(bad, g, absmax).verdict == "PASS"
    assert gate.gate_mean(t.double(), g, absmax).verdict == "FAIL"  # must be float32


@pytest.mark.parametrize("mutation", [None, "truncate", "r_squared", "unwritten"])
def test_chunked_gate_equals_whole_gate(mutation):
    """TensorGate fed in row chunks gives the row gate_tensor gives on the
    whole tensor (same errors, floor, threshold, bias within float64 sum
    order, verdict), so full-size tensors can be gated chunk by chunk."""
    inp = workloads.make_inputs("c2", M=96, N=256)
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    y_t, _, dx_t, _ = stand_in(x, w, dy, EPS, False, mutation)
    y_r, _ = reference.reference_forward(x, w, EPS)
    dx_r, _ = reference.reference_backward(dy, x, w, EPS)
    y_g, _ = golden.golden_forward(x, w, EPS)
    dx_g = golden.golden_dx(dy, x, w, EPS)
    for name, t, r, g in (("y", y_t, y_r, y_g), ("dx", dx_t, dx_r, dx_g)):
        whole = gate.gate_tensor(name, t, r, g, torch.bfloat16)
        acc = gate.TensorGate(name, torch.bfloat16, g.shape)
        for a in range(0, 96, 40):
            acc.add(t[a:a + 40], r[a:a + 40], g[a:a + 40])
        part = acc.finish()
        assert part.verdict == whole.verdict, (name, mutation)
        for k in ("reference_error", "target_error", "rounding_floor", "threshold",
                  "golden_scale", "gate_valid", "note"):
            a_, b_ = getattr(part, k), getattr(whole, k)
            assert a_ == b_ or (a_ != a_ and b_ != b_), (k, a_, b_)
        if whole.bias_target is not None:
            assert abs(part.bias_target - whole.bias_target) < 1e-12


def test_page_allclose_logged_as_information():
    """The page's allclose rule (|t - ref| <= atol + rtol*|ref|, float32
    1e-5/1e-4, float16 3e-3/3e-3) is reported beside the gate row and never
    changes the verdict; bfloat16 has no declared tolerance."""
    g = np.array([1.0, 100.0, -3.0])
    ref = torch.tensor(g, dtype=torch.float32)
    near = ref.clone()
    near[0] += 1e-4                    # within 1e-5 + 1e-4*1
    far = ref.clone()
    far[1] += 0.02                     # beyond 1e-5 + 1e-4*100
    a = gate.gate_tensor("t", near, ref, g, torch.float32).extra["allclose"]
    assert a["verdict"] and a["outside"] == 0 and a["elements"] == 3
    row = gate.gate_tensor("t", far, ref, g, torch.float32)
    assert row.extra["allclose"]["outside"] == 1 and not row.extra["allclose"]["verdict"]
    assert row.verdict == "FAIL"       # the gate, not allclose, decides
    h = torch.tensor(g, dtype=torch.float16)
    assert gate.gate_tensor("t", h, h, g, torch.float16).extra["allclose"]["atol"] == 3e-3
    b = torch.tensor(g, dtype=torch.bfloat16)
    assert "allclose" not in gate.gate_tensor("t", b, b, g, torch.bfloat16).extra
    assert "Page allclose" in gate.report([row])


@pytest.mark.parametrize("mutation", [None, "dx_scaled", "y_unwritten"])
def test_layernorm_chunked_gate_equals_whole_gate(mutation):
    """The row-chunked LayerNorm gate (y and dx a block of rows at a time)
    gives the same rows as the whole-tensor gate: same verdicts and errors."""
    from oracle import layernorm as lnref
    from parity import gate_ln_full, gate_ln_full_chunked
    inp = workloads.make_layernorm_inputs("c2", M=50, N=512)
    x, w, b, dy, eps = inp["x"], inp["w"], inp["b"], inp["dy"], inp["eps"]
    y, mu, r = lnref.reference_ln_forward(x, w, b, eps)
    dx, dg, db = lnref.reference_ln_backward(dy, x, w, eps)
    if mutation == "dx_scaled":
        dx = (dx.float() * 1.01).to(dx.dtype)
    elif mutation == "y_unwritten":
        y = y.clone()
        y[13, 7] = float("nan")
    out = {"y": y, "mean": mu, "rstd": r, "dx": dx, "dgamma": dg, "dbeta": db}
    whole = gate_ln_full(inp, out)
    part = gate_ln_full_chunked(inp, out, chunk_rows=7)
    assert [p.tensor for p in part] == [w_.tensor for w_ in whole]
    for p, w_ in zip(part, whole):
        assert p.verdict == w_.verdict, (p.tensor, mutation)
        a_, b_ = p.target_error, w_.target_error
        assert a_ == b_ or (a_ != a_ and b_ != b_), (p.tensor, a_, b_)
    if mutation:
        assert gate.overall_verdict(part) == "FAIL"
