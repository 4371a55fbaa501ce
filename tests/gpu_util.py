"""Helpers shared by the GPU parity tests: the tolerance bar, margin records,
top-K validity, host/device staging."""
import os
import sys

import numpy as np
import torch

import oracle as O
from block_diffusion_drafter_step_amd import pipeline as P

# Per element: |gpu - ref| <= atol + rtol * |ref| (+ a rounding-point term
# where a check declares one), bf16 workloads (2e-2, 1e-2), fp32 (1e-4, 1e-4).
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
GAP = 1e-3          # a ranking is unique where the score gap exceeds this

# one record per float comparison, written out by conftest.py when asked
MARGINS = []


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else \
        t.detach().cpu().double().numpy()


def _case() -> str:
    cur = os.environ.get("PYTEST_CURRENT_TEST", "")
    return cur.split(" (")[0].split("::", 1)[-1] if cur else "?"


def assert_close(gpu, ref, act: str, what: str, term=None):
    """Every element within atol + rtol |ref| + term (term: a per-element
    allowance for a declared rounding point, broadcast against ref; None =
    none).  Records the largest error, the largest error / bar and how many
    elements were beyond the plain bar (inside the term)."""
    atol, rtol = TOL[act]
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    both_inf = np.isinf(gpu) & np.isinf(ref) & (np.sign(gpu) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(gpu - ref))
    fin = np.where(np.isfinite(ref), ref, 0.0)
    plain = atol + rtol * np.abs(fin)
    t = np.zeros_like(plain) if term is None else np.broadcast_to(np.asarray(term, dtype=np.float64),
                                                                 plain.shape)
    lim = plain + t
    bad = ~(err <= lim)
    beyond_plain = int(np.sum((err > plain) & ~bad))
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = float(np.nanmax(np.where(bad, np.inf, err / lim))) if err.size else 0.0
    MARGINS.append({"case": _case(), "check": what, "elements": int(err.size),
                    "max_err": float(np.nanmax(err)) if err.size else 0.0, "max_ratio": ratio,
                    "beyond_plain": beyond_plain, "term": term is not None})
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - lim, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} elements off; worst at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r} (atol {atol}, rtol {rtol}, term {t[i]!r})")
    say(f"  {what}: max |err| {float(err.max()) if err.size else 0.0:.3g}, max err/bar {ratio:.3g} over "
        f"{err.size} elements" + (f"; {beyond_plain} inside the rounding-point term" if term is not None
                                  else ""))
    return beyond_plain


def act_np(a, act):
    return O.act_to_f64(a, act)


def dev(a, act):
    return P.act_tensor(a, act)


def check_topk(gpu_idx, gpu_unary, logits, K, act, what, drift=None):
    """Top-K of each row against the oracle's logits.

    Every row: K distinct indices in [0, V); the oracle's logits along the
    GPU's order non-increasing within the margin; every pick at least the
    oracle's K-th logit minus the margin.  Rows whose K-th gap exceeds the
    margin: the index set exact, and the order exact where adjacent gaps
    exceed it.  Unary within tolerance of the oracle's value at the GPU's
    picks.  The margin is GAP plus twice `drift` (a bound on how far the
    GPU's logits can sit from the oracle's when the two ran on different
    inputs)."""
    gpu_idx = np.asarray(gpu_idx)
    r = O.topk_unary_from_logits(logits, K)
    gaps = O.topk_gaps(logits, K)
    nrow, V = logits.shape
    drift = np.zeros(nrow) if drift is None else np.asarray(drift, dtype=np.float64)
    ref_idx = r["idx"]
    assert gpu_idx.shape == (nrow, K), (what, gpu_idx.shape)
    assert np.all((gpu_idx >= 0) & (gpu_idx < V)), (what, "index out of range")
    unique_rows = 0
    for i in range(nrow):
        margin = GAP + 2 * drift[i]
        gi = gpu_idx[i]
        assert len(set(gi.tolist())) == K, (what, i, "repeated index", gi)
        picked = logits[i][gi]
        assert np.all(picked[:-1] >= picked[1:] - margin), (what, i, "not in descending order", picked)
        kth = -np.sort(-logits[i])[K - 1]
        assert np.all(picked >= kth - margin), (what, i, "a pick below the K-th logit")
        if gaps["kth_gap"][i] > margin:
            unique_rows += 1
            assert set(gi.tolist()) == set(ref_idx[i].tolist()), (what, i, gi, ref_idx[i])
            for k in range(K - 1):
                if gaps["adj_gap"][i][k] > margin:
                    assert gi[k] == ref_idx[i][k], (what, i, k, gi, ref_idx[i])
    ref_unary_at_gpu = logits[np.arange(nrow)[:, None], gpu_idx] - r["lse"][:, None]
    assert_close(gpu_unary, ref_unary_at_gpu, act, what + " unary",
                 term=2 * drift[:, None] if np.any(drift) else None)
    say(f"  {what}: {unique_rows}/{nrow} rows with a unique top-{K}")
    return unique_rows


def _command(argv) -> str:
    """The pytest command line as typed (python -m pytest for the module's path)."""
    argv = list(argv)
    if argv and argv[0] == "python":
        argv = argv[1:]
    if argv and argv[0].endswith(os.path.join("pytest", "__main__.py")):
        argv = ["-m", "pytest"] + argv[1:]
    return "python " + " ".join(argv)


def write_margins(path: str, argv, records=None) -> None:
    """The parity margins of this session as markdown: one row per test (its
    checks, elements compared and worst error / bar), then every check that
    used a rounding-point term."""
    records = MARGINS if records is None else records
    lines = ["# Parity margins of the GPU tests", "",
             "Every float comparison of `tests/test_gpu_parity.py`: the bar is "
             "`atol + rtol * |ref|` per element (bf16 workloads 2e-2 / 1e-2, fp32 1e-4 / 1e-4), "
             "plus, where the check names one, a rounding-point term. `max err / bar` below 1 "
             "passes; `beyond plain bar` counts the elements that needed the term.", "",
             "Command: `DFLASH_PARITY_MARGINS=" + path + " " + _command(argv) + "`", "",
             "| test | checks | elements | worst check | max err / bar |", "|---|---|---|---|---|"]
    by = {}
    for m in records:
        by.setdefault(m["case"], []).append(m)
    for case, ms in by.items():
        w = max(ms, key=lambda m: m["max_ratio"])
        lines.append(f"| {case} | {len(ms)} | {sum(m['elements'] for m in ms)} | {w['check']} | "
                     f"{w['max_ratio']:.3g} |")
    lines += ["", "Checks with a rounding-point term:", "",
              "| test | check | elements | max abs err | max err / bar | beyond plain bar |",
              "|---|---|---|---|---|---|"]
    for m in records:
        if m["term"]:
            lines.append(f"| {m['case']} | {m['check']} | {m['elements']} | {m['max_err']:.3g} | "
                         f"{m['max_ratio']:.3g} | {m['beyond_plain']} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
