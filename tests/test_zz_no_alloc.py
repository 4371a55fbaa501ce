"""The no-allocation LM-head call against the workspace one, through the C ABI.

dflash_topk_unary_noalloc runs the same kernels as dflash_topk_unary on the
library's static scratch, so its outputs must equal the workspace call's bit
for bit.  Two calls in a row, the second on a smaller input (another head
type, fewer rows, a wider K), then the first shape again: the static array
keeps the previous call's contents and no call may depend on them.
"""
import ctypes

import numpy as np
import pytest
import torch

from block_diffusion_drafter_step_amd import configs, synth
from block_diffusion_drafter_step_amd import dflash as D
from block_diffusion_drafter_step_amd import pipeline as P

pytestmark = pytest.mark.gpu


def both(cfg, tag):
    """(workspace call, no-allocation call) outputs on the same seeded inputs."""
    w = synth.Workload(cfg)
    h = P.act_tensor(synth.normal(cfg.seed, tag + ".h", (cfg.B, cfg.d), 1.0, cfg.act), cfg.act)
    wl = P.weight_tensor(w.w_lm())
    outs = []
    for noalloc in (False, True):
        idx = torch.full((cfg.B, cfg.K), -1, dtype=torch.int32, device="cuda")
        un = torch.full((cfg.B, cfg.K), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            D.dflash_topk_unary_noalloc(h, wl, cfg.K, idx, un)
        else:
            ws = D.workspace(D.dflash_topk_unary_workspace(cfg.B, cfg.V, cfg.K))
            D.dflash_topk_unary(h, wl, cfg.K, idx, un, ws)
        torch.cuda.synchronize()
        outs.append((idx.cpu().numpy(), un.cpu().numpy()))
    return outs


def check(cfg, tag):
    print(f"noalloc {cfg.name} V={cfg.V} d={cfg.d} B={cfg.B} K={cfg.K} weight={cfg.weight}", flush=True)
    (i0, u0), (i1, u1) = both(cfg, tag)
    assert np.all(i0 >= 0) and np.all(i0 < cfg.V)
    assert np.array_equal(i0, i1), (i0, i1)
    assert np.array_equal(u0.view(np.uint32), u1.view(np.uint32))


def test_noalloc_matches_workspace_call_twice_then_smaller():
    big = configs.shrink(configs.get(1), V=151936, d=512, B=16, K=8)          # resident path
    small = configs.shrink(configs.get(4), V=20011, d=256, B=5, K=32)         # Q8_0, streaming path
    check(big, "na1")
    check(small, "na2")
    check(big, "na3")


def test_noalloc_rejects_a_vocabulary_beyond_its_scratch():
    h = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    data = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((16, 32), dtype=torch.int32, device="cuda")
    un = torch.empty((16, 32), dtype=torch.float32, device="cuda")
    w = D._Weight(D.BF16, 0, (1 << 20) + 16, 64, data.data_ptr(), None)   # never read: rejected first
    st = D.load().dflash_topk_unary_noalloc(h.data_ptr(), 16, D.BF16, ctypes.byref(w), 32, idx.data_ptr(),
                                            un.data_ptr(), None)
    assert st == 2, D.load().dflash_last_error()
    assert b"static array" in D.load().dflash_last_error()
