"""The allocation-free entry point (hs2_block_forward_static) against
hs2_block_forward, through the C ABI, on calls in a row of shrinking size:
the static workspace keeps what the previous call left, and each call must
still give exactly what the workspace-taking entry point gives."""
import sys

import pytest
import torch

from synth import Workload, make_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    Workload(0, "static_prefill", "bf16", batch=1, n_q=600, n_kv=3000, h_q=16, h_kv=2, d=128,
             top_k=256, window=32, n_sparse=3),
    Workload(0, "static_smaller", "bf16", batch=2, n_q=100, n_kv=700, h_q=8, h_kv=2, d=128,
             top_k=64, window=16, n_sparse=2),
    Workload(0, "static_decode", "bf16", batch=3, n_q=1, n_kv=2500, h_q=16, h_kv=2, d=128,
             top_k=256, window=64, n_sparse=2),
]


def test_static_workspace_matches_block_forward(gpu_lib):
    for case in CASES:
        say("case", case)
        inp = make_inputs(case, device="cuda")
        args = (inp["q_full"], inp["q_sparse"], inp["k"], inp["v"])
        kw = dict(top_k=case.top_k, window=case.window)
        ref = gpu_lib.block_forward(*args, **kw)
        out = {n: torch.full_like(t, -7 if t.dtype == torch.int32 else 3.0)
               for n, t in ref.items()}
        gpu_lib.block_forward_static(*args, out=out, **kw)
        torch.cuda.synchronize()
        for key in ("o_full", "o_sparse", "idx", "lse"):
            assert torch.equal(out[key], ref[key]), (case.name, key)
        say("  identical:", ", ".join(f"{k} {tuple(out[k].shape)}" for k in out))
