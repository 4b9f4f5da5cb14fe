"""Host checks of the seeded input generators that drive the backward pass."""
import numpy as np
import pytest

from synth import Workload, grad_inputs, random_index_rows


def _w(nq, nkv, top_k, window, B=2):
    return Workload(0, "idx", "bf16", batch=B, n_q=nq, n_kv=nkv, h_q=4, h_kv=2, d=64,
                    top_k=top_k, window=window, n_sparse=2)


@pytest.mark.parametrize("nq,nkv,top_k,window", [(50, 50, 8, 4), (30, 300, 16, 8),
                                                 (7, 7, 1, 1), (64, 1000, 100, 128)])
def test_random_index_rows_are_valid_sets(nq, nkv, top_k, window):
    w = _w(nq, nkv, top_k, window)
    idx = random_index_rows(w, rows_per_chunk=13).numpy()
    assert idx.shape == (2, nq, top_k + window)
    for b in range(2):
        for i in range(nq):
            p = nkv - nq + i
            row = idx[b, i]
            n = int((row >= 0).sum())
            assert np.all(row[:n] >= 0) and np.all(row[n:] == -1)     # packed, -1 tail
            sel = row[:n]
            assert np.all(np.diff(sel) > 0) and sel[-1] == p           # ascending, ends at p
            win = np.arange(max(0, p - window + 1), p + 1)
            assert np.array_equal(sel[len(sel) - len(win):], win)     # window present
            n_cand = max(0, p - window + 1)
            assert n == min(top_k, n_cand) + len(win)
            assert np.all(sel[:n - len(win)] <= p - window)


def test_random_index_rows_are_seeded_and_spread():
    w = _w(40, 4000, 64, 16, B=1)
    a, b = random_index_rows(w).numpy(), random_index_rows(w).numpy()
    assert np.array_equal(a, b)
    row = a[0, -1]
    picks = row[:64]
    # one pick in each of the 64 integer ranges [t C / 64, (t + 1) C / 64)
    C = 4000 - 1 - 16 + 1
    t = np.arange(64)
    assert np.all((picks >= t * C // 64) & (picks < (t + 1) * C // 64))


def test_grad_inputs_shapes():
    w = _w(5, 9, 2, 2)
    g = grad_inputs(w)
    assert tuple(g["do_full"].shape) == (2, 5, 4, 64)
    assert tuple(g["do_sparse"].shape) == (2, 2, 5, 4, 64)
