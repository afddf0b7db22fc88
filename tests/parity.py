"""Helpers that run the HIP path through the C ABI and gate it against the
oracle (golden + reference) on the same seeded inputs."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import backward_rmsnorm_fwd_amd as rn
from oracle import gate, golden, reference
from oracle import fused as fusedref
from oracle import layernorm as lnref


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_target(inp, device, offset=None, poison=True):
    """Forward + backward on the GPU (outputs pre-poisoned with NaN)."""
    off = inp["offset"] if offset is None else offset
    x = inp["x"].to(device)
    w = inp["w"].to(device)
    dy = inp["dy"].to(device)
    y, rstd = rn.fwd(x, w, inp["eps"], off, poison=poison)
    dx, dg = rn.bwd(dy, x, w, rstd, off, poison=poison)
    torch.cuda.synchronize()
    return {"y": y, "rstd": rstd, "dx": dx, "dgamma": dg}


def gate_full(inp, out):
    """Gate every element (small inputs)."""
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    off, eps, T = inp["offset"], inp["eps"], inp["x"].dtype
    n = x.shape[-1]
    y_r, r_r = reference.reference_forward(x, w, eps, off)
    dx_r, dg_r = reference.reference_backward(dy, x, w, eps, off)
    y_g, r_g = golden.golden_forward(x, w, eps, off)
    dx_g, dg_g = golden.golden_backward(dy, x, w, eps, off)
    worst = int(np.argmax(np.abs(out["dgamma"].double().cpu().numpy() - dg_g))) if n else 0
    cond = golden.dgamma_condition(dy, x, eps, worst) if x.numel() else None
    return [
        gate.gate_tensor("y", out["y"].cpu().reshape(-1, n), y_r, y_g, T),
        gate.gate_rstd(out["rstd"].cpu(), r_g, r_r),
        gate.gate_tensor("dx", out["dx"].cpu().reshape(-1, n), dx_r, dx_g, T),
        gate.gate_tensor("dgamma", out["dgamma"].cpu(), dg_r, dg_g, torch.float32,
                         condition=cond),
    ]


def blocks_in_order(M, chunk_rows, work, workers=4):
    """Yield (a, b, work(a, b)) for the row blocks [a, b) of [0, M) in
    order.  The blocks' oracle work runs a few at a time in threads (NumPy
    and torch release the interpreter lock in their array loops), and at
    most `workers` blocks' results are held; the caller consumes them in
    block order, so everything it accumulates is as in a serial loop."""
    spans = [(a, min(M, a + chunk_rows)) for a in range(0, M, chunk_rows)]
    with ThreadPoolExecutor(workers) as ex:
        for i in range(0, len(spans), workers):
            futures = [(a, b, ex.submit(work, a, b)) for a, b in spans[i:i + workers]]
            for a, b, f in futures:
                yield a, b, f.result()


def add_together(*feeds):
    """Feed independent TensorGates one block each at the same time, each in
    a thread of its own (every gate still sees its blocks in order)."""
    with ThreadPoolExecutor(len(feeds)) as ex:
        for f in [ex.submit(g.add, *args) for g, args in feeds]:
            f.result()


def gate_full_chunked(inp, out, chunk_rows=8192):
    """Gate every element of a full-size run, a block of rows at a time.

    y and dx are gated through gate.TensorGate, fed one row block at a time
    (golden and reference computed for that block only, the target's block
    copied from the device), so no tensor is held in float64 whole; rstd and
    dgamma are gated whole (dgamma's golden and reference are column sums
    over all rows, themselves accumulated in row blocks)."""
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    off, eps, T = inp["offset"], inp["eps"], inp["x"].dtype
    M, n = x.shape[0], x.shape[-1]
    gy = gate.TensorGate("y", T, (M, n))
    gdx = gate.TensorGate("dx", T, (M, n))
    r_g = np.empty(M)
    r_r = torch.empty(M, dtype=torch.float32)

    def work(a, b):
        xs, dys = x[a:b], dy[a:b]
        y_r, rr = reference.reference_forward(xs, w, eps, off)
        dx_r, _ = reference.reference_backward(dys, xs, w, eps, off)
        y_g, rg = golden.golden_forward(xs, w, eps, off)
        return y_r, rr, dx_r, y_g, rg, golden.golden_dx(dys, xs, w, eps, off)

    with ThreadPoolExecutor(1) as side:  # the column sums meanwhile
        dg = side.submit(lambda: (golden.golden_dgamma(dy, x, eps),
                                  reference.reference_dgamma(dy, x, eps)))
        for a, b, (y_r, rr, dx_r, y_g, rg, dx_g) in blocks_in_order(M, chunk_rows, work):
            r_r[a:b], r_g[a:b] = rr, rg
            add_together((gy, (out["y"][a:b].cpu(), y_r, y_g)),
                         (gdx, (out["dx"][a:b].cpu(), dx_r, dx_g)))
        dg_g, dg_r = dg.result()
    dg_t = out["dgamma"].cpu()
    worst = int(np.argmax(np.abs(dg_t.double().numpy() - dg_g)))
    cond = golden.dgamma_condition(dy, x, eps, worst)
    return [gy.finish(), gate.gate_rstd(out["rstd"].cpu(), r_g, r_r), gdx.finish(),
            gate.gate_tensor("dgamma", dg_t, dg_r, dg_g, torch.float32, condition=cond)]


def sample_rows(inp, count, seed=1234):
    """Random rows plus the first/last rows and any special rows of the recipe."""
    M = inp["x"].shape[0]
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(count, M), replace=False).tolist())
    rows.update([0, M - 1])
    for key in ("zero_rows", "big_rows", "small_rows"):
        if key in inp:
            rows.update(np.asarray(inp[key])[:32].tolist())
    return np.array(sorted(rows))


def sample_cols(N, count, seed=4321):
    rng = np.random.default_rng(seed)
    cols = set(rng.choice(N, size=min(count, N), replace=False).tolist())
    cols.update([0, N - 1])
    return np.array(sorted(cols))


def gate_sampled(inp, out, rows, cols):
    """Gate sampled rows of y, rstd, dx and sampled columns of dgamma (the
    dgamma columns are still sums over all M rows)."""
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    off, eps, T = inp["offset"], inp["eps"], inp["x"].dtype
    rt = torch.as_tensor(rows, dtype=torch.long)
    xs, dys = x[rt], dy[rt]
    y_r, r_r = reference.reference_forward(xs, w, eps, off)
    dx_r, _ = reference.reference_backward(dys, xs, w, eps, off)
    y_g, r_g = golden.golden_forward(xs, w, eps, off)
    dx_g = golden.golden_dx(dys, xs, w, eps, off)
    dg_g = golden.golden_dgamma(dy, x, eps, cols=cols)
    dg_r = reference.reference_dgamma(dy, x, eps, cols=cols)
    dev_rows = rt.to(out["y"].device)
    dev_cols = torch.as_tensor(cols, dtype=torch.long, device=out["y"].device)
    return [
        gate.gate_tensor("y[rows]", out["y"][dev_rows].cpu(), y_r, y_g, T),
        gate.gate_rstd(out["rstd"][dev_rows].cpu(), r_g, r_r),
        gate.gate_tensor("dx[rows]", out["dx"][dev_rows].cpu(), dx_r, dx_g, T),
        gate.gate_tensor("dgamma[cols]", out["dgamma"][dev_cols].cpu(), dg_r, dg_g,
                         torch.float32),
    ]


def assert_pass(rows, title):
    text = gate.report(rows, title)
    log(text)
    assert gate.overall_verdict(rows) == "PASS", text


# ---- LayerNorm ------------------------------------------------------------------

def run_ln_target(inp, device, poison=True, bias=True):
    """LayerNorm forward + backward on the GPU (outputs pre-poisoned with NaN)."""
    x = inp["x"].to(device)
    w = inp["w"].to(device)
    b = inp["b"].to(device) if bias else None
    dy = inp["dy"].to(device)
    y, mean, rstd = rn.ln_fwd(x, w, b, inp["eps"], poison=poison)
    dx, dg, db = rn.ln_bwd(dy, x, w, mean, rstd, poison=poison, bias=bias)
    torch.cuda.synchronize()
    return {"y": y, "mean": mean, "rstd": rstd, "dx": dx, "dgamma": dg, "dbeta": db}


def gate_ln_full(inp, out, bias=True):
    """Gate every element of y, mean, rstd, dx, dgamma and dbeta."""
    x, w, dy, eps, T = inp["x"], inp["w"], inp["dy"], inp["eps"], inp["x"].dtype
    b = inp["b"] if bias else None
    n = x.shape[-1]
    y_r, mu_r, r_r = lnref.reference_ln_forward(x, w, b, eps)
    dx_r, dg_r, db_r = lnref.reference_ln_backward(dy, x, w, eps)
    y_g, mu_g, r_g = lnref.golden_ln_forward(x, w, b, eps)
    dx_g, dg_g, db_g = lnref.golden_ln_backward(dy, x, w, eps)
    worst = int(np.argmax(np.abs(out["dgamma"].double().cpu().numpy() - dg_g))) if n else 0
    cg, cb = lnref.ln_param_condition(dy, x, eps, worst) if x.numel() else (None, None)
    rows = [
        gate.gate_tensor("y", out["y"].cpu().reshape(-1, n), y_r, y_g, T),
        gate.gate_mean(out["mean"].cpu(), mu_g, x.reshape(-1, n).abs().amax(1).double()
                       if x.numel() else np.zeros(0)),
        gate.gate_rstd(out["rstd"].cpu(), r_g, r_r),
        gate.gate_tensor("dx", out["dx"].cpu().reshape(-1, n), dx_r, dx_g, T),
        gate.gate_tensor("dgamma", out["dgamma"].cpu(), dg_r, dg_g, torch.float32, condition=cg),
    ]
    if out.get("dbeta") is not None:
        rows.append(gate.gate_tensor("dbeta", out["dbeta"].cpu(), db_r, db_g, torch.float32))
    return rows


def gate_ln_full_chunked(inp, out, chunk_rows=8192):
    """Gate every element of a full-size LayerNorm run, a block of rows at a
    time: y and dx through gate.TensorGate (golden and reference computed
    per block), mean and rstd whole from the per-block statistics, dgamma
    and dbeta whole (their golden accumulated in row blocks)."""
    x, w, b, dy, eps, T = inp["x"], inp["w"], inp["b"], inp["dy"], inp["eps"], inp["x"].dtype
    M, n = x.shape[0], x.shape[-1]
    gy = gate.TensorGate("y", T, (M, n))
    gdx = gate.TensorGate("dx", T, (M, n))
    mu_g, r_g, xmax = np.empty(M), np.empty(M), np.empty(M)
    r_r = torch.empty(M, dtype=torch.float32)

    def work(a, e):
        xs, dys = x[a:e], dy[a:e]
        y_r, _, rr = lnref.reference_ln_forward(xs, w, b, eps)
        dx_r, _, _ = lnref.reference_ln_backward(dys, xs, w, eps)
        y_g, mg, rg = lnref.golden_ln_forward(xs, w, b, eps)
        dx_g = lnref.golden_ln_dx(dys, xs, w, eps)
        return y_r, rr, dx_r, y_g, mg, rg, dx_g, xs.abs().amax(1).double().numpy()

    with ThreadPoolExecutor(1) as side:  # the column sums meanwhile
        pg = side.submit(lambda: (lnref.golden_ln_param_grads(dy, x, eps),
                                  lnref.reference_ln_param_grads(dy, x, eps)))
        for a, e, (y_r, rr, dx_r, y_g, mg, rg, dx_g, xm) in blocks_in_order(M, chunk_rows,
                                                                             work):
            r_r[a:e], mu_g[a:e], r_g[a:e], xmax[a:e] = rr, mg, rg, xm
            add_together((gy, (out["y"][a:e].cpu(), y_r, y_g)),
                         (gdx, (out["dx"][a:e].cpu(), dx_r, dx_g)))
        (dg_g, db_g), (dg_r, db_r) = pg.result()
    dg_t = out["dgamma"].cpu()
    worst = int(np.argmax(np.abs(dg_t.double().numpy() - dg_g)))
    cg, _ = lnref.ln_param_condition(dy, x, eps, worst)
    return [gy.finish(), gate.gate_mean(out["mean"].cpu(), mu_g, xmax),
            gate.gate_rstd(out["rstd"].cpu(), r_g, r_r), gdx.finish(),
            gate.gate_tensor("dgamma", dg_t, dg_r, dg_g, torch.float32, condition=cg),
            gate.gate_tensor("dbeta", out["dbeta"].cpu(), db_r, db_g, torch.float32)]


def gate_ln_sampled(inp, out, rows, cols):
    """Sampled rows of y, mean, rstd, dx; sampled columns of dgamma and dbeta
    (still sums over all M rows)."""
    x, w, b, dy, eps, T = inp["x"], inp["w"], inp["b"], inp["dy"], inp["eps"], inp["x"].dtype
    rt = torch.as_tensor(rows, dtype=torch.long)
    xs, dys = x[rt], dy[rt]
    y_r, mu_r, r_r = lnref.reference_ln_forward(xs, w, b, eps)
    dx_r, _, _ = lnref.reference_ln_backward(dys, xs, w, eps)
    y_g, mu_g, r_g = lnref.golden_ln_forward(xs, w, b, eps)
    dx_g = lnref.golden_ln_dx(dys, xs, w, eps)
    dg_g, db_g = lnref.golden_ln_param_grads(dy, x, eps, cols=cols)
    dg_r, db_r = lnref.reference_ln_param_grads(dy, x, eps, cols=cols)
    dr = rt.to(out["y"].device)
    dc = torch.as_tensor(cols, dtype=torch.long, device=out["y"].device)
    return [
        gate.gate_tensor("y[rows]", out["y"][dr].cpu(), y_r, y_g, T),
        gate.gate_mean(out["mean"][dr].cpu(), mu_g, xs.abs().amax(1).double()),
        gate.gate_rstd(out["rstd"][dr].cpu(), r_g, r_r),
        gate.gate_tensor("dx[rows]", out["dx"][dr].cpu(), dx_r, dx_g, T),
        gate.gate_tensor("dgamma[cols]", out["dgamma"][dc].cpu(), dg_r, dg_g, torch.float32),
        gate.gate_tensor("dbeta[cols]", out["dbeta"][dc].cpu(), db_r, db_g, torch.float32),
    ]


# ---- residual add fused with RMSNorm -----------------------------------------------

def run_add_target(inp, device, poison=True, with_dh=True):
    x, res, w, dy = (inp[k].to(device) for k in ("x", "res", "w", "dy"))
    dh = inp["dh"].to(device) if with_dh else None
    off, eps = inp["offset"], inp["eps"]
    y, h, rstd = rn.add_fwd(x, res, w, eps, off, poison=poison)
    dx, dg = rn.add_bwd(dy, dh, h, w, rstd, off, poison=poison)
    torch.cuda.synchronize()
    return {"y": y, "h": h, "rstd": rstd, "dx": dx, "dgamma": dg}


def gate_add_full(inp, out, with_dh=True):
    """h bit-exact (the dtype's add, taken in the same precision on both
    sides); y, rstd, dx and dgamma through the gate."""
    x, res, w, dy, eps, off = inp["x"], inp["res"], inp["w"], inp["dy"], inp["eps"], inp["offset"]
    dh = inp["dh"] if with_dh else None
    T, n = x.dtype, x.shape[-1]
    h_o = fusedref.residual_sum(x, res)
    h_t = out["h"].cpu()
    h_row = gate.GateRow(tensor="h", dtype=str(T).replace("torch.", ""), shape=tuple(h_o.shape))
    h_row.gate_valid = True
    h_row.target_error = float((h_t.double() - h_o.double()).abs().max()) if h_o.numel() else 0.0
    h_row.verdict = "PASS" if torch.equal(h_t, h_o) else "FAIL"
    h_row.note = "bitwise equal to the dtype's add"
    _, y_r, r_r = fusedref.reference_add_forward(x, res, w, eps, off)
    _, y_g, r_g = fusedref.golden_add_forward(x, res, w, eps, off)
    dx_r, dg_r = fusedref.reference_add_backward(dy, dh, h_o, w, eps, off)
    dx_g, dg_g = fusedref.golden_add_backward(dy, dh, h_o, w, eps, off)
    worst = int(np.argmax(np.abs(out["dgamma"].double().cpu().numpy() - dg_g))) if n else 0
    cond = golden.dgamma_condition(dy, h_o, eps, worst) if x.numel() else None
    return [
        h_row,
        gate.gate_tensor("y", out["y"].cpu().reshape(-1, n), y_r, y_g, T),
        gate.gate_rstd(out["rstd"].cpu(), r_g, r_r),
        gate.gate_tensor("dx", out["dx"].cpu().reshape(-1, n), dx_r, dx_g, T),
        gate.gate_tensor("dgamma", out["dgamma"].cpu(), dg_r, dg_g, torch.float32, condition=cond),
    ]


def gate_add_full_chunked(inp, out, chunk_rows=8192):
    """Every element of a full-size fused-add run: h bit-exact whole, y and
    dx a block of rows at a time (gate.TensorGate), rstd and dgamma whole."""
    x, res, w, dy, dh = inp["x"], inp["res"], inp["w"], inp["dy"], inp["dh"]
    eps, off, T = inp["eps"], inp["offset"], inp["x"].dtype
    M, n = x.shape[0], x.shape[-1]
    h_o = fusedref.residual_sum(x, res)
    h_t = out["h"].cpu()
    h_row = gate.GateRow(tensor="h", dtype=str(T).replace("torch.", ""), shape=tuple(h_o.shape))
    h_row.gate_valid = True
    h_row.target_error = float((h_t.double() - h_o.double()).abs().max())
    h_row.verdict = "PASS" if torch.equal(h_t, h_o) else "FAIL"
    h_row.note = "bitwise equal to the dtype's add"
    gy = gate.TensorGate("y", T, (M, n))
    gdx = gate.TensorGate("dx", T, (M, n))
    r_g = np.empty(M)
    r_r = torch.empty(M, dtype=torch.float32)

    def work(a, e):
        xs, rs, dys, dhs, hs = x[a:e], res[a:e], dy[a:e], dh[a:e], h_o[a:e]
        _, y_r, rr = fusedref.reference_add_forward(xs, rs, w, eps, off)
        _, y_g, rg = fusedref.golden_add_forward(xs, rs, w, eps, off)
        dx_r, _ = fusedref.reference_add_backward(dys, dhs, hs, w, eps, off)
        return y_r, rr, y_g, rg, dx_r, fusedref.golden_add_dx(dys, dhs, hs, w, eps, off)

    with ThreadPoolExecutor(1) as side:  # the column sums meanwhile
        dg = side.submit(lambda: (golden.golden_dgamma(dy, h_o, eps),
                                  reference.reference_dgamma(dy, h_o, eps)))
        for a, e, (y_r, rr, y_g, rg, dx_r, dx_g) in blocks_in_order(M, chunk_rows, work):
            r_r[a:e], r_g[a:e] = rr, rg
            add_together((gy, (out["y"][a:e].cpu(), y_r, y_g)),
                         (gdx, (out["dx"][a:e].cpu(), dx_r, dx_g)))
        dg_g, dg_r = dg.result()
    dg_t = out["dgamma"].cpu()
    worst = int(np.argmax(np.abs(dg_t.double().numpy() - dg_g)))
    cond = golden.dgamma_condition(dy, h_o, eps, worst)
    return [h_row, gy.finish(), gate.gate_rstd(out["rstd"].cpu(), r_g, r_r), gdx.finish(),
            gate.gate_tensor("dgamma", dg_t, dg_r, dg_g, torch.float32, condition=cond)]


def gate_add_sampled(inp, out, rows, cols):
    """Sampled rows of h (bit-exact), y, rstd and dx, and sampled columns of
    dgamma (sums over all rows), against the fused-add oracle."""
    x, res, w, dy, dh = inp["x"], inp["res"], inp["w"], inp["dy"], inp["dh"]
    eps, off, T = inp["eps"], inp["offset"], inp["x"].dtype
    rt = torch.as_tensor(rows, dtype=torch.long)
    xs, rs, dys, dhs = x[rt], res[rt], dy[rt], dh[rt]
    dev_rows = rt.to(out["y"].device)
    dev_cols = torch.as_tensor(cols, dtype=torch.long, device=out["y"].device)
    h_o = fusedref.residual_sum(xs, rs)
    h_t = out["h"][dev_rows].cpu()
    h_row = gate.GateRow(tensor="h[rows]", dtype=str(T).replace("torch.", ""),
                         shape=tuple(h_o.shape))
    h_row.gate_valid = True
    h_row.target_error = float((h_t.double() - h_o.double()).abs().max())
    h_row.verdict = "PASS" if torch.equal(h_t, h_o) else "FAIL"
    h_row.note = "bitwise equal to the dtype's add"
    _, y_r, r_r = fusedref.reference_add_forward(xs, rs, w, eps, off)
    _, y_g, r_g = fusedref.golden_add_forward(xs, rs, w, eps, off)
    dx_r, _ = fusedref.reference_add_backward(dys, dhs, h_o, w, eps, off)
    dx_g = fusedref.golden_add_dx(dys, dhs, h_o, w, eps, off)
    h_all = fusedref.residual_sum(x, res)
    dg_g = golden.golden_dgamma(dy, h_all, eps, cols=cols)
    dg_r = reference.reference_dgamma(dy, h_all, eps, cols=cols)
    return [
        h_row,
        gate.gate_tensor("y[rows]", out["y"][dev_rows].cpu(), y_r, y_g, T),
        gate.gate_rstd(out["rstd"][dev_rows].cpu(), r_g, r_r),
        gate.gate_tensor("dx[rows]", out["dx"][dev_rows].cpu(), dx_r, dx_g, T),
        gate.gate_tensor("dgamma[cols]", out["dgamma"][dev_cols].cpu(), dg_r, dg_g,
                         torch.float32),
    ]


def run_cast_target(inp, device, poison=True):
    x, w, dy = (inp[k].to(device) for k in ("x", "w", "dy"))
    off, eps = inp["offset"], inp["eps"]
    y, rstd = rn.cast_fwd(x, w, inp["out_dtype"], eps, off, poison=poison)
    dx, dg = rn.cast_bwd(dy, x, w, rstd, off, poison=poison)
    torch.cuda.synchronize()
    return {"y": y, "rstd": rstd, "dx": dx, "dgamma": dg}


def gate_cast_full(inp, out):
    """y (in the narrow dtype: its rounding floor), rstd, dx and dgamma
    (float32) through the gate against the cast oracle."""
    x, w, dy, eps, off = inp["x"], inp["w"], inp["dy"], inp["eps"], inp["offset"]
    To, n = inp["out_dtype"], x.shape[-1]
    y_r, r_r = fusedref.reference_cast_forward(x, w, To, eps, off)
    y_g, r_g = fusedref.golden_cast_forward(x, w, eps, off)
    dx_r, dg_r = fusedref.reference_cast_backward(dy, x, w, eps, off)
    dx_g, dg_g = fusedref.golden_cast_backward(dy, x, w, eps, off)
    worst = int(np.argmax(np.abs(out["dgamma"].double().cpu().numpy() - dg_g))) if n else 0
    cond = golden.dgamma_condition(dy, x, eps, worst) if x.numel() else None
    return [
        gate.gate_tensor("y", out["y"].cpu().reshape(-1, n), y_r, y_g, To),
        gate.gate_rstd(out["rstd"].cpu(), r_g, r_r),
        gate.gate_tensor("dx", out["dx"].cpu().reshape(-1, n), dx_r, dx_g, torch.float32),
        gate.gate_tensor("dgamma", out["dgamma"].cpu(), dg_r, dg_g, torch.float32,
                         condition=cond),
    ]


def gate_cast_full_chunked(inp, out, chunk_rows=8192):
    """Every element of a full-size cast run, y and dx a block of rows at a
    time (gate.TensorGate), rstd and dgamma whole."""
    x, w, dy, eps, off = inp["x"], inp["w"], inp["dy"], inp["eps"], inp["offset"]
    To = inp["out_dtype"]
    M, n = x.shape[0], x.shape[-1]
    gy = gate.TensorGate("y", To, (M, n))
    gdx = gate.TensorGate("dx", torch.float32, (M, n))
    r_g = np.empty(M)
    r_r = torch.empty(M, dtype=torch.float32)

    def work(a, e):
        xs, dys = x[a:e], dy[a:e]
        y_r, rr = fusedref.reference_cast_forward(xs, w, To, eps, off)
        y_g, rg = fusedref.golden_cast_forward(xs, w, eps, off)
        dx_r, _ = fusedref.reference_cast_backward(dys, xs, w, eps, off)
        return y_r, rr, y_g, rg, dx_r, fusedref.golden_cast_dx(dys, xs, w, eps, off)

    with ThreadPoolExecutor(1) as side:  # the column sums meanwhile
        dg = side.submit(lambda: (golden.golden_dgamma(dy, x, eps),
                                  reference.reference_dgamma(dy.float(), x, eps)))
        for a, e, (y_r, rr, y_g, rg, dx_r, dx_g) in blocks_in_order(M, chunk_rows, work):
            r_r[a:e], r_g[a:e] = rr, rg
            add_together((gy, (out["y"][a:e].cpu(), y_r, y_g)),
                         (gdx, (out["dx"][a:e].cpu(), dx_r, dx_g)))
        dg_g, dg_r = dg.result()
    dg_t = out["dgamma"].cpu()
    worst = int(np.argmax(np.abs(dg_t.double().numpy() - dg_g)))
    cond = golden.dgamma_condition(dy, x, eps, worst)
    return [gy.finish(), gate.gate_rstd(out["rstd"].cpu(), r_g, r_r), gdx.finish(),
            gate.gate_tensor("dgamma", dg_t, dg_r, dg_g, torch.float32, condition=cond)]


def gate_cast_sampled(inp, out, rows, cols):
    """Sampled rows of y, rstd and dx and sampled columns of dgamma (sums
    over all rows) against the cast oracle."""
    x, w, dy, eps, off = inp["x"], inp["w"], inp["dy"], inp["eps"], inp["offset"]
    To = inp["out_dtype"]
    rt = torch.as_tensor(rows, dtype=torch.long)
    xs, dys = x[rt], dy[rt]
    y_r, r_r = fusedref.reference_cast_forward(xs, w, To, eps, off)
    dx_r, _ = fusedref.reference_cast_backward(dys, xs, w, eps, off)
    y_g, r_g = fusedref.golden_cast_forward(xs, w, eps, off)
    dx_g = fusedref.golden_cast_dx(dys, xs, w, eps, off)
    dg_g = golden.golden_dgamma(dy, x, eps, cols=cols)
    dg_r = reference.reference_dgamma(dy.float(), x, eps, cols=cols)
    dev_rows = rt.to(out["y"].device)
    dev_cols = torch.as_tensor(cols, dtype=torch.long, device=out["y"].device)
    return [
        gate.gate_tensor("y[rows]", out["y"][dev_rows].cpu(), y_r, y_g, To),
        gate.gate_rstd(out["rstd"][dev_rows].cpu(), r_g, r_r),
        gate.gate_tensor("dx[rows]", out["dx"][dev_rows].cpu(), dx_r, dx_g, torch.float32),
        gate.gate_tensor("dgamma[cols]", out["dgamma"][dev_cols].cpu(), dg_r, dg_g,
                         torch.float32),
    ]
