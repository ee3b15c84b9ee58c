"""lct_group_run_noalloc (the library's fixed per-GPU scratch array, no
allocation) against lct_group_run (caller workspace), both through the C ABI,
on the MI355X: two calls in a row, the second on a smaller step.  Index sets
must be bit-exact and outputs within the attention tolerance."""

import numpy as np
import pytest
import torch

import long_context_top_amd as lct
import synth.device as sd
from synth import configs as C
from tests.gpu_util import announce, host

pytestmark = pytest.mark.gpu

ATOL = 1e-2


def _inputs(cfg):
    qi = [sd.make(cfg, cfg.qi_spec(g)) for g in range(cfg.n_groups)]
    ki = [sd.make(cfg, cfg.ki_spec(g)) for g in range(cfg.n_groups)]
    q = [sd.make(cfg, cfg.q_spec(l)) for l in range(cfg.n_layers)]
    k = [sd.make(cfg, cfg.k_spec(l)) for l in range(cfg.n_layers)]
    v = [sd.make(cfg, cfg.v_spec(l)) for l in range(cfg.n_layers)]
    return qi, ki, q, k, v


def _outputs(cfg, fill):
    out = [torch.full((cfg.B, cfg.Lq, cfg.Hq, cfg.D), fill, dtype=torch.float32, device="cuda")
           for _ in range(cfg.n_layers)]
    idx = [torch.full((cfg.B, cfg.Lq, cfg.topk), -7, dtype=torch.int32, device="cuda")
           for _ in range(cfg.n_groups)]
    return out, idx


def _compare(cfg):
    announce(f"group_run_noalloc {cfg.name}: B={cfg.B} L={cfg.L} k={cfg.topk} layers={cfg.n_layers}")
    qi, ki, q, k, v = _inputs(cfg)
    out_a, idx_a = _outputs(cfg, 0.0)
    out_b, idx_b = _outputs(cfg, float("nan"))
    run_a = lct.GroupRun(qi, ki, q, k, v, out_a, cfg.topk, cfg.group, cfg.scale, idx_out=idx_a)
    run_b = lct.GroupRun(qi, ki, q, k, v, out_b, cfg.topk, cfg.group, cfg.scale, idx_out=idx_b)
    assert run_a.ws_bytes <= lct.NOALLOC_SCRATCH_BYTES
    run_a()
    run_b.call_noalloc()
    torch.cuda.synchronize()
    for g in range(cfg.n_groups):
        assert np.array_equal(host(idx_a[g]), host(idx_b[g])), g
    err = max(float(np.abs(host(a) - host(b)).max()) for a, b in zip(out_a, out_b))
    print(f"  max |noalloc - workspace| = {err:.2e}", flush=True)
    assert err < ATOL


def test_noalloc_matches_workspace_call_twice():
    big = C.DecodeConfig("noalloc_big", 4141, B=8, Lq=1, L=40000, n_layers=8, group=4, Hq=32, Hkv=4,
                         D=128, H_idx=4, d_idx=64, topk=2048)
    small = big.with_(name="noalloc_small", seed=4242, B=2, L=9000, topk=512, n_layers=4)
    _compare(big)      # few long rows: multi-workgroup select, split attention
    _compare(small)    # shorter rows: one workgroup per row; the array keeps the first call's data
