"""Parity of the backward pass (through the C ABI) with the fp64 oracle.

The GPU backward takes the forward's outputs (O, LSE) from the GPU forward
and the index sets from the oracle or from the seeded random generator; the
oracle recomputes everything from Q, K, V, idx and dO alone. Every gradient
element is compared against a bound derived from the arithmetic:

    |gpu - ref| <= eps * (|ref| + mag)

where mag is the sum of the magnitudes of the summands behind that element
(the oracle's with_mag output: P^T |dO| for dV, scale * W |K| for dQ and
scale * W^T |Q| for dK, W = P (|dP| + rowsum(|dO| |O|))). In bf16 the GPU
rounds P and dS to bf16 for its products, forms Delta from the bf16 O, and
stores the gradient in bf16: each rounding is at most 2^-9 relative, and
fp32 accumulation over up to 2^15 terms adds at most about 2^-9 of mag, so
eps = 2^-7 (four half-ulps). In fp32 the products take fp32 operands; the
error is the exp2 argument's rounding (about 2^-20 relative in P for
logits below 16) plus fp32 accumulation over a few hundred terms, so
eps = 2^-15.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import hs2_oracle as O
from synth import Workload, grad_inputs, make_inputs, random_index_rows, to_host

pytestmark = pytest.mark.gpu

EPS = {"bf16": 2.0 ** -7, "fp32": 2.0 ** -15}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name, dtype, B, nq, nkv, hq, hkv, d, top_k, window, L=2, cid=0):
    return Workload(cid, name, dtype, batch=B, n_q=nq, n_kv=nkv, h_q=hq, h_kv=hkv, d=d,
                    top_k=top_k, window=window, n_sparse=L)


def as_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got, want):
    return float(np.abs(got - want).max() / max(1.0, np.abs(want).max()))


def check_grad(name, got, want, mag, dtype):
    """Per-element bound |got - want| <= eps (|want| + mag); prints the
    worst ratio of the error to the bound's scale and the normalised max
    error as diagnostics."""
    scale = np.abs(want) + mag
    ratio = np.abs(got - want) / np.maximum(scale, 1e-300)
    worst = float(ratio.max())
    say(name, f"max err / (|ref| + mag) = {worst:.3e} (eps {EPS[dtype]:.3e}),",
        f"normalised max err {rel_err(got, want):.3e}")
    assert np.all(np.abs(got - want) <= EPS[dtype] * scale), name


def gpu_forward_outputs(lib, inp, idx, case, select="token"):
    """O_full and LSE from the GPU full layer; O_sparse from the GPU sparse
    layers over the given index sets."""
    kw = dict(top_k=case.top_k, window=case.window, select=select, block_size=16, top_blocks=4)
    o_full, _, lse, _ = lib.full_attn_select(inp["q_full"], inp["k"], inp["v"], **kw)
    o_sparse = lib.sparse_attn(inp["q_sparse"], inp["k"], inp["v"], idx, **kw) \
        if case.n_sparse else None
    return o_full, lse, o_sparse


def run_backward(lib, case, idx_source="oracle", select="token", deterministic=False):
    inp = make_inputs(case, device="cuda")
    grads = grad_inputs(case, device="cuda")
    host = {n: to_host(inp[n]) for n in ("q_full", "k", "v", "q_sparse")}
    if idx_source == "oracle":
        ref_fwd = O.block_forward(host["q_full"], host["q_sparse"], host["k"], host["v"],
                                  top_k=case.top_k, window=case.window, select=select,
                                  block_size=16, top_blocks=4)
        idx = torch.from_numpy(ref_fwd["idx"].astype(np.int32)).cuda()
    else:
        idx = random_index_rows(case, device="cuda")
    kw = dict(top_k=case.top_k, window=case.window, select=select, block_size=16, top_blocks=4)
    o_full, lse, o_sparse = gpu_forward_outputs(lib, inp, idx, case, select)
    L = case.n_sparse
    out = lib.block_backward(inp["q_full"], inp["q_sparse"] if L else None, inp["k"], inp["v"],
                             o_full, o_sparse, lse, idx if L else None, grads["do_full"],
                             grads["do_sparse"] if L else None, deterministic=deterministic, **kw)
    torch.cuda.synchronize()
    return inp, grads, host, idx, out


BWD_CASES = [
    small("b_fp32_d64", "fp32", 2, 300, 300, 4, 1, 64, 32, 16, L=3),
    small("b_bf16_d128", "bf16", 1, 700, 700, 8, 2, 128, 64, 32, L=2),
    small("b_bf16_chunk_g8", "bf16", 1, 200, 650, 16, 2, 128, 48, 16, L=3),
    small("b_bf16_d64_ragged", "bf16", 2, 157, 411, 4, 2, 64, 40, 13, L=2),
    small("b_fp32_d128_chunk", "fp32", 1, 130, 333, 8, 4, 128, 30, 8, L=2),
    small("b_bf16_no_sparse", "bf16", 1, 300, 500, 8, 2, 128, 32, 16, L=0),
    small("b_bf16_decode", "bf16", 3, 1, 900, 8, 2, 128, 64, 32, L=2),
    # 64 rows per work-group in the sparse backward: 8 layers x 8 heads
    small("b_bf16_64rows", "bf16", 1, 90, 300, 16, 2, 128, 40, 16, L=8),
    # six heads per KV head: 64-row tiles start mid-query (64 = 10 * 6 + 4)
    small("b_bf16_g6_chunk", "bf16", 2, 150, 420, 12, 2, 128, 40, 16, L=2),
    # one query head per KV head, and a single partial 64-row tile (15 rows)
    small("b_bf16_g1", "bf16", 1, 100, 260, 4, 4, 128, 40, 16, L=2),
    small("b_bf16_g3_tiny", "bf16", 1, 5, 70, 6, 2, 128, 16, 8, L=1),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: c.name)
def test_backward_small(gpu_lib, case):
    say("case", case)
    inp, grads, host, idx, out = run_backward(gpu_lib, case)
    L = case.n_sparse
    ref = O.block_backward(host["q_full"], host["q_sparse"], host["k"], host["v"],
                           to_host(idx) if L else np.full((case.batch, case.n_q, 1), -1),
                           to_host(grads["do_full"]), to_host(grads["do_sparse"]), with_mag=True)
    for name in ("dq_full", "dk", "dv") + (("dq_sparse",) if L else ()):
        check_grad(name, as_np(out[name]), ref[name], ref["mag"][name], case.dtype)


@pytest.mark.parametrize("case", [
    small("b_rand_bf16", "bf16", 2, 400, 1400, 8, 2, 128, 96, 32, L=3),
    small("b_rand_fp32", "fp32", 1, 260, 260, 8, 8, 64, 50, 10, L=2),
], ids=lambda c: c.name)
def test_backward_random_index_sets(gpu_lib, case):
    say("case", case)
    inp, grads, host, idx, out = run_backward(gpu_lib, case, idx_source="random")
    ref = O.block_backward(host["q_full"], host["q_sparse"], host["k"], host["v"], to_host(idx),
                           to_host(grads["do_full"]), to_host(grads["do_sparse"]), with_mag=True)
    for name in ("dq_full", "dq_sparse", "dk", "dv"):
        check_grad(name, as_np(out[name]), ref[name], ref["mag"][name], case.dtype)


def test_backward_block_mode_indices(gpu_lib):
    case = small("b_block", "bf16", 1, 260, 500, 8, 2, 128, 0, 16, L=2)
    inp, grads, host, idx, out = run_backward(gpu_lib, case, select="block")
    ref = O.block_backward(host["q_full"], host["q_sparse"], host["k"], host["v"], to_host(idx),
                           to_host(grads["do_full"]), to_host(grads["do_sparse"]), with_mag=True)
    for name in ("dq_full", "dq_sparse", "dk", "dv"):
        check_grad(name, as_np(out[name]), ref[name], ref["mag"][name], "bf16")


@pytest.mark.parametrize("L", [0, 3], ids=["full_layer", "with_sparse_layers"])
def test_backward_deterministic(gpu_lib, L):
    """Two runs of the deterministic entry point give bit-identical
    gradients. With sparse layers the K/V sums come from atomics landing in
    any order; 1024 queries with 128-key windows make many of them add into
    the same keys."""
    case = small("b_det", "bf16", 1, 1024, 1024, 16, 2, 128, 128, 32, L=L)
    a = run_backward(gpu_lib, case, deterministic=True)[4]
    b = run_backward(gpu_lib, case, deterministic=True)[4]
    for name in ("dq_full", "dk", "dv") + (("dq_sparse",) if L else ()):
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("case", [BWD_CASES[0], BWD_CASES[1], BWD_CASES[2], BWD_CASES[7]],
                         ids=lambda c: c.name)
def test_backward_deterministic_parity(gpu_lib, case):
    """The deterministic entry point (fixed-point K/V sums) meets the same
    per-element bound as the default one."""
    say("case", case)
    inp, grads, host, idx, out = run_backward(gpu_lib, case, deterministic=True)
    L = case.n_sparse
    ref = O.block_backward(host["q_full"], host["q_sparse"], host["k"], host["v"], to_host(idx),
                           to_host(grads["do_full"]), to_host(grads["do_sparse"]), with_mag=True)
    for name in ("dq_full", "dk", "dv") + (("dq_sparse",) if L else ()):
        check_grad(name, as_np(out[name]), ref[name], ref["mag"][name], case.dtype)


@pytest.mark.parametrize("mul", [1e-6, 1e3], ids=["tiny_grads", "large_grads"])
def test_backward_gradient_magnitudes(gpu_lib, mul):
    """The sparse layers' K/V sums are fixed point with a scale derived from
    the inputs: gradients scaled by 1e-6 or 1e3 keep the same relative
    accuracy (the oracle is linear in dO)."""
    case = small("b_mag", "bf16", 1, 400, 900, 8, 2, 128, 96, 32, L=3)
    inp = make_inputs(case, device="cuda")
    grads = grad_inputs(case, device="cuda")
    grads = {n: (g.float() * mul).to(g.dtype) for n, g in grads.items()}
    host = {n: to_host(inp[n]) for n in ("q_full", "k", "v", "q_sparse")}
    idx = random_index_rows(case, device="cuda")
    kw = dict(top_k=case.top_k, window=case.window)
    o_full, lse, o_sparse = gpu_forward_outputs(gpu_lib, inp, idx, case)
    out = gpu_lib.block_backward(inp["q_full"], inp["q_sparse"], inp["k"], inp["v"], o_full,
                                 o_sparse, lse, idx, grads["do_full"], grads["do_sparse"],
                                 deterministic=True, **kw)
    torch.cuda.synchronize()
    ref = O.block_backward(host["q_full"], host["q_sparse"], host["k"], host["v"], to_host(idx),
                           to_host(grads["do_full"]), to_host(grads["do_sparse"]), with_mag=True)
    for name in ("dq_full", "dq_sparse", "dk", "dv"):
        check_grad(name, as_np(out[name]), ref[name], ref["mag"][name], "bf16")


def test_backward_32k_prefill_tail_and_invariants(gpu_lib):
    """The 32K-token prefill shape (32 query heads, 4 KV heads, 3 sparse
    layers) in the configuration the benchmark times, on random index sets:
    the oracle gives every gradient a tail of 256 keys decides (dK, dV of
    those keys, dQ of the queries at or after them) exactly; over all keys,
    the V gradients of a KV group must add up to the group's output
    gradients and the K gradients to zero."""
    case = Workload(2, "prefill_bf16_32k_needles", "bf16", batch=1, n_q=32768, n_kv=32768,
                    h_q=32, h_kv=4, d=128, n_sparse=3)
    say("case", case.name)
    inp, grads, host, idx, out = run_backward(gpu_lib, case, idx_source="random")
    j_lo = case.n_kv - 256
    say("tail oracle from key", j_lo)
    t = O.block_backward_tail(host["q_full"], host["q_sparse"], host["k"], host["v"],
                              to_host(idx), to_host(grads["do_full"]),
                              to_host(grads["do_sparse"]), 0, j_lo, with_mag=True)
    rows = torch.from_numpy(t["rows"]).cuda()
    checks = [("dq_full", as_np(out["dq_full"][0, rows])),
              ("dq_sparse", as_np(out["dq_sparse"][:, 0, rows])),
              ("dk", as_np(out["dk"][0, j_lo:])),
              ("dv", as_np(out["dv"][0, j_lo:]))]
    for name, got in checks:
        check_grad("tail " + name, got, t[name], t["mag"][name], "bf16")
    # sums over all keys, per KV group (fp64 on the host)
    G = case.h_q // case.h_kv
    dv_sum = as_np(out["dv"][0].sum(dim=0, dtype=torch.float64))          # [h_kv, d]
    dk_sum = as_np(out["dk"][0].sum(dim=0, dtype=torch.float64))
    do_all = grads["do_full"][0].double().sum(dim=0) + grads["do_sparse"][:, 0].double().sum(
        dim=(0, 1))                                                        # [h_q, d]
    want_dv = as_np(do_all.view(case.h_kv, G, case.d).sum(dim=1))
    e_dv = float(np.abs(dv_sum - want_dv).max() / np.abs(want_dv).max())
    dk_scale = float(out["dk"][0].double().abs().sum(dim=0).max())
    e_dk = float(np.abs(dk_sum).max() / dk_scale)
    say("sum dV rel err", e_dv, "sum dK / sum |dK|", e_dk)
    assert e_dv <= 1e-2
    assert e_dk <= 1e-2
