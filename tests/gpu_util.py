"""Helpers shared by the GPU parity tests: tolerances, host/device staging."""
import sys

import numpy as np
import torch

import oracle as O
from block_diffusion_drafter_step_amd import pipeline as P

# per element |gpu - ref| <= atol + rtol * max(|ref|, rms of ref's row): the
# relative bar is taken against the row's scale, because an output of a long
# dot product that cancels to near zero has no meaningful elementwise
# relative error (its error scales with the terms, not with the result)
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
GAP = 1e-3          # a ranking is unique where the score gap exceeds this


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else \
        t.detach().cpu().double().numpy()


def assert_close(gpu, ref, act: str, what: str, extra_atol=0.0):
    atol, rtol = TOL[act]
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    both_inf = np.isinf(gpu) & np.isinf(ref) & (np.sign(gpu) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(gpu - ref))
    fin = np.where(np.isfinite(ref), ref, 0.0)
    row_rms = np.sqrt(np.mean(fin * fin, axis=-1, keepdims=True)) if fin.ndim else np.abs(fin)
    lim = atol + extra_atol + rtol * np.maximum(np.abs(fin), row_rms)
    bad = ~(err <= lim)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - lim, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} elements off; worst at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r} (atol {atol}, rtol {rtol})")
    say(f"  {what}: max |err| {float(err.max()) if err.size else 0.0:.3g} over {err.size} elements")


def act_np(a, act):
    return O.act_to_f64(a, act)


def dev(a, act):
    return P.act_tensor(a, act)


def check_topk(gpu_idx, gpu_unary, logits, K, act, what, drift=None):
    """Index sets exact where the K-th gap exceeds the margin, order exact where
    the adjacent gaps do; unary within tolerance of the oracle at the GPU's
    picks.  The margin is GAP, plus twice `drift` (a bound on how far the GPU's
    logits can sit from the oracle's when the two ran on different inputs)."""
    r = O.topk_unary_from_logits(logits, K)
    gaps = O.topk_gaps(logits, K)
    nrow = logits.shape[0]
    drift = np.zeros(nrow) if drift is None else np.asarray(drift, dtype=np.float64)
    ref_idx = r["idx"]
    unique_rows = 0
    for i in range(nrow):
        margin = GAP + 2 * drift[i]
        if gaps["kth_gap"][i] > margin:
            unique_rows += 1
            assert set(gpu_idx[i]) == set(ref_idx[i]), (what, i, gpu_idx[i], ref_idx[i])
            for k in range(K - 1):
                if gaps["adj_gap"][i][k] > margin:
                    assert gpu_idx[i][k] == ref_idx[i][k], (what, i, k, gpu_idx[i], ref_idx[i])
        else:
            # several answers are right: the GPU's picks must still be a valid top-K
            kth = -np.sort(-logits[i])[K - 1]
            assert np.all(logits[i][gpu_idx[i]] >= kth - margin), (what, i)
    ref_unary_at_gpu = logits[np.arange(nrow)[:, None], gpu_idx] - r["lse"][:, None]
    assert_close(gpu_unary, ref_unary_at_gpu, act, what + " unary", extra_atol=2 * drift[:, None])
    say(f"  {what}: {unique_rows}/{nrow} rows with a unique top-{K}")
    return unique_rows
