"""Pins for the CPU oracle: checks against facts fixed independently of it.

Each test ties the oracle to something other than its own formulas: a library
attention routine, closed forms worked out by hand, brute-force enumeration,
invariants that follow from the definition, or special cases that reduce to
a simpler problem. All run on the CPU.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import hs2_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa_reference(q, k, v):
    """torch's fp64 CPU attention with an explicit end-aligned causal mask."""
    B, nq, hq, d = q.shape
    nkv = k.shape[1]
    pos = torch.arange(nq) + (nkv - nq)
    mask = torch.arange(nkv)[None, :] <= pos[:, None]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, enable_gqa=True)
    return o.permute(0, 2, 1, 3).numpy()


# --------------------------------------------------------------------------
# full layer: library routine and closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("B,nq,nkv,hq,hkv,d", [(1, 9, 9, 4, 1, 8), (2, 5, 13, 6, 2, 4),
                                               (1, 1, 17, 8, 4, 16), (1, 33, 40, 4, 4, 8)])
def test_full_layer_matches_torch_sdpa(B, nq, nkv, hq, hkv, d):
    q, k, v = rand((B, nq, hq, d), 1), rand((B, nkv, hkv, d), 2), rand((B, nkv, hkv, d), 3)
    o, _ = O.full_layer(q, k, v)
    np.testing.assert_allclose(o, sdpa_reference(q, k, v), rtol=0, atol=1e-12)


def test_lse_closed_form_zero_keys():
    # all logits are 0, so LSE at position p is log(p + 1)
    B, nq, nkv, hq, hkv, d = 1, 7, 10, 2, 1, 4
    q = rand((B, nq, hq, d), 4)
    k = np.zeros((B, nkv, hkv, d))
    v = rand((B, nkv, hkv, d), 5)
    _, lse = O.full_layer(q, k, v)
    pos = np.arange(nq) + nkv - nq
    np.testing.assert_allclose(lse[0, 0], np.log(pos + 1.0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 1], np.log(pos + 1.0), rtol=0, atol=1e-14)


def test_first_token_output_is_its_value():
    # position 0 sees only key 0: softmax weight 1
    q, k, v = rand((1, 6, 4, 8), 6), rand((1, 6, 2, 8), 7), rand((1, 6, 2, 8), 8)
    o, lse = O.full_layer(q, k, v)
    for h in range(4):
        np.testing.assert_allclose(o[0, 0, h], v[0, 0, h // 2], atol=1e-15)
        assert abs(lse[0, h, 0] - (q[0, 0, h] @ k[0, 0, h // 2]) / math.sqrt(8)) < 1e-14


def test_constant_values_give_constant_outputs():
    B, n, hq, hkv, d = 1, 40, 4, 2, 8
    q, k = rand((B, n, hq, d), 9), rand((B, n, hkv, d), 10)
    row = rand((hkv, d), 11)
    v = np.broadcast_to(row, (B, n, hkv, d)).copy()
    o, _ = O.full_layer(q, k, v)
    res = O.block_forward(q, rand((2, B, n, hq, d), 12), k, v, top_k=5, window=3)
    for h in range(hq):
        np.testing.assert_allclose(o[0, :, h], np.broadcast_to(row[h // 2], (n, d)), atol=1e-13)
        np.testing.assert_allclose(res["o_sparse"][:, 0, :, h],
                                   np.broadcast_to(row[h // 2], (2, n, d)), atol=1e-13)


# --------------------------------------------------------------------------
# worked example with rational scores (hand-derived; see the golden file)
# --------------------------------------------------------------------------
def test_worked_example_d1():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_d1.json")))
    a = [Fraction(x) for x in ex["a"]]
    n = len(a)
    c = ex["query_exponents"]           # head h has logit c_h * ln(a_j)
    # inputs: d = 1, scale 1, q = c_h, k_j = ln(a_j) so exp(logit) = a_j ** c_h
    q = np.array(c, dtype=np.float64).reshape(1, 1, len(c), 1).repeat(n, axis=1)
    k = np.log(np.array([float(x) for x in a])).reshape(1, n, 1, 1)
    v = np.array(ex["v"], dtype=np.float64).reshape(1, n, 1, 1)
    res = O.block_forward(q, q[None], k, v, top_k=ex["top_k"], window=ex["window"],
                          scale=1.0)
    for p_str, want in ex["expected"].items():
        p = int(p_str)
        # hand-derived scores from the golden file, as exact fractions
        for j_str, frac in want["S"].items():
            assert abs(res["S"][0, p, int(j_str)] - float(Fraction(frac))) < 1e-14
        got = res["idx"][0, p]
        assert list(got[got >= 0]) == want["idx"]
        assert abs(res["o_sparse"][0, 0, p, 0, 0] - float(Fraction(want["o_sparse_h0"]))) < 1e-13
        # the selection threshold, hand-derived as the top_k-th candidate score
        tau = float(want["tau"]) if want["tau"] == "inf" else float(Fraction(want["tau"]))
        assert res["tau"][0, p] == tau or abs(res["tau"][0, p] - tau) < 1e-14
        assert O.kth_candidate_score(res["S"][0, p], p, ex["top_k"], ex["window"]) == \
            res["tau"][0, p]

    # block mode on the same inputs: hand-derived block scores (candidates
    # only), thresholds and index sets
    bm = ex["block_mode"]
    res = O.block_forward(q, q[None], k, v, top_k=ex["top_k"], window=ex["window"],
                          select="block", block_size=bm["block_size"],
                          top_blocks=bm["top_blocks"], scale=1.0)
    for p_str, want in bm["expected"].items():
        p = int(p_str)
        bs = O.block_scores(res["S"][0, p], p, bm["block_size"], ex["window"])
        np.testing.assert_allclose(bs, [float(Fraction(x)) for x in want["block_scores"]],
                                   rtol=0, atol=1e-14)
        tau = float(Fraction(want["tau"]))
        assert abs(O.kth_block_score(res["S"][0, p], p, bm["block_size"], bm["top_blocks"],
                                     ex["window"]) - tau) < 1e-14
        assert abs(res["tau"][0, p] - tau) < 1e-14
        got = res["idx"][0, p]
        assert list(got[got >= 0]) == want["idx"]
    for p in (0, 1):                    # no candidates: no block, no threshold
        assert len(O.block_scores(res["S"][0, p], p, bm["block_size"], ex["window"])) == 0
        assert res["tau"][0, p] == np.inf


# --------------------------------------------------------------------------
# selection: brute force, rank counting, ties
# --------------------------------------------------------------------------
def brute_force_topk(S, k):
    """All k-subsets; keep the best score multiset, then the smallest indices."""
    n = len(S)
    best = None
    for sub in itertools.combinations(range(n), min(k, n)):
        key = (tuple(sorted((-S[i] for i in sub))), sub)
        if best is None or key < best:
            best = key
    return list(best[1])


@pytest.mark.parametrize("seed", range(40))
def test_token_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n_cand = int(rng.integers(0, 12))
    k = int(rng.integers(1, 5))
    w = int(rng.integers(1, 4))
    p = n_cand + w - 1
    # small integer scores make ties frequent
    S = rng.integers(0, 4, size=p + 1).astype(np.float64) / 4
    got = O.select_token(S, p, k, w)
    want = brute_force_topk(S[:n_cand], k) + list(range(max(0, p - w + 1), p + 1))
    assert list(got) == want
    # rank-count characterisation
    cand = np.arange(n_cand)
    for j in cand:
        rank = np.sum(S[:n_cand] > S[j]) + np.sum((S[:n_cand] == S[j]) & (cand < j))
        assert (j in got) == (rank < k)


@pytest.mark.parametrize("seed", range(40))
def test_threshold_is_lowest_score_of_the_brute_force_set(seed):
    # tau is fixed by the chosen set itself: the lowest score in the top-k
    # subset found by enumeration, at least the best score left out; +inf when
    # there is no candidate. Distinct scores make the k-th and (k+1)-th differ.
    rng = np.random.default_rng(500 + seed)
    n_cand = int(rng.integers(0, 12))
    k = int(rng.integers(1, 5))
    w = int(rng.integers(1, 4))
    p = n_cand + w - 1
    S = rng.permutation(p + 1).astype(np.float64) / 16 if seed % 2 else \
        rng.integers(0, 4, size=p + 1).astype(np.float64) / 4
    tau = O.kth_candidate_score(S, p, k, w)
    if n_cand == 0:
        assert tau == np.inf
        return
    chosen = brute_force_topk(S[:n_cand], k)
    assert tau == min(S[j] for j in chosen)
    rest = [j for j in range(n_cand) if j not in chosen]
    if rest:
        assert tau >= max(S[j] for j in rest)


def test_threshold_literal_values():
    # hand-written rows: the threshold is the k-th largest candidate score,
    # not the (k+1)-th, and window scores never count
    S = np.array([0.1, 0.7, 0.4, 0.9, 0.2, 0.05, 5.0, 6.0])   # p = 7, window 2: j <= 5
    assert O.kth_candidate_score(S, 7, 1, 2) == 0.9
    assert O.kth_candidate_score(S, 7, 2, 2) == 0.7
    assert O.kth_candidate_score(S, 7, 3, 2) == 0.4
    assert O.kth_candidate_score(S, 7, 6, 2) == 0.05
    assert O.kth_candidate_score(S, 7, 9, 2) == 0.05            # fewer than k: lowest
    assert O.kth_candidate_score(S, 1, 3, 2) == np.inf          # no candidate
    assert O.kth_candidate_score(np.array([2.0, 2.0, 1.0, 0.0]), 3, 2, 1) == 2.0


def test_exact_ties_take_lowest_indices():
    # K = 0: every logit equal, every score equal -> the first k candidates
    B, n, hq, hkv, d = 1, 30, 4, 1, 8
    q, v = rand((B, n, hq, d), 13), rand((B, n, hkv, d), 14)
    k = np.zeros((B, n, hkv, d))
    res = O.block_forward(q, np.zeros((0, B, n, hq, d)), k, v, top_k=5, window=4)
    for p in range(n):
        row = res["idx"][0, p]
        row = list(row[row >= 0])
        n_cand = max(0, p - 3)
        assert row == list(range(min(5, n_cand))) + list(range(max(0, p - 3), p + 1))


def test_single_head_selection_is_topk_of_dot_products():
    # one head: P is increasing in the logit, so the score order is the order
    # of the raw dot products and no exp/LSE is involved
    B, n, d, k, w = 1, 200, 16, 20, 8
    q, kk, v = rand((B, n, 1, d), 15), rand((B, n, 1, d), 16), rand((B, n, 1, d), 17)
    res = O.block_forward(q, np.zeros((0, B, n, 1, d)), kk, v, top_k=k, window=w)
    for p in range(n):
        n_cand = max(0, p - w + 1)
        dots = kk[0, :n_cand, 0] @ q[0, p, 0]
        order = sorted(range(n_cand), key=lambda j: (-dots[j], j))[:k]
        want = sorted(order) + list(range(max(0, p - w + 1), p + 1))
        row = res["idx"][0, p]
        assert list(row[row >= 0]) == want


def test_scores_sum_to_head_count():
    B, n, hq, hkv, d = 2, 50, 8, 2, 8
    q, k, v = rand((B, n, hq, d), 18), rand((B, n, hkv, d), 19), rand((B, n, hkv, d), 20)
    _, lse = O.full_layer(q, k, v)
    S = O.scores(q, k, lse)
    np.testing.assert_allclose(S.sum(axis=2), hq, rtol=0, atol=1e-12)
    assert np.all(S >= 0)
    assert np.all(S[:, np.arange(n)[:, None] < np.arange(n)[None, :]] == 0)


def test_index_set_invariants():
    B, nq, nkv, hq, hkv, d, k, w = 1, 60, 90, 4, 2, 8, 10, 6
    q, kk, v = rand((B, nq, hq, d), 21), rand((B, nkv, hkv, d), 22), rand((B, nkv, hkv, d), 23)
    res = O.block_forward(q, np.zeros((0, B, nq, hq, d)), kk, v, top_k=k, window=w)
    for i in range(nq):
        p = nkv - nq + i
        row = res["idx"][0, i]
        valid = row[row >= 0]
        assert len(valid) == min(p + 1, k + w)
        assert np.all(np.diff(valid) > 0)
        assert valid[-1] == p and np.all(valid <= p)
        assert set(range(max(0, p - w + 1), p + 1)) <= set(valid.tolist())
        assert np.all(row[len(valid):] == -1)


# --------------------------------------------------------------------------
# dense reduction: when k + w covers the whole prefix, sparse == dense
# --------------------------------------------------------------------------
@pytest.mark.parametrize("hq,hkv", [(4, 1), (6, 3)])
def test_dense_reduction(hq, hkv):
    B, n, d = 1, 24, 8
    q, k, v = rand((B, n, hq, d), 24), rand((B, n, hkv, d), 25), rand((B, n, hkv, d), 26)
    qs = rand((2, B, n, hq, d), 27)
    res = O.block_forward(q, qs, k, v, top_k=16, window=8)
    for i in range(n):
        row = res["idx"][0, i]
        assert list(row[row >= 0]) == list(range(i + 1))
    for layer in range(2):
        np.testing.assert_allclose(res["o_sparse"][layer], sdpa_reference(qs[layer], k, v),
                                   rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# block selection
# --------------------------------------------------------------------------
def test_block_mode_with_unit_blocks_is_token_mode():
    B, n, hq, hkv, d = 1, 70, 4, 2, 8
    q, k, v = rand((B, n, hq, d), 28), rand((B, n, hkv, d), 29), rand((B, n, hkv, d), 30)
    qs = rand((1, B, n, hq, d), 31)
    t = O.block_forward(q, qs, k, v, top_k=9, window=5)
    b = O.block_forward(q, qs, k, v, top_k=9, window=5, select="block",
                        block_size=1, top_blocks=9)
    np.testing.assert_array_equal(t["idx"], b["idx"])
    np.testing.assert_allclose(t["o_sparse"], b["o_sparse"], atol=0)


@pytest.mark.parametrize("seed", range(20))
def test_block_selection_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    bsz = int(rng.integers(1, 5))
    tb = int(rng.integers(1, 4))
    w = int(rng.integers(1, 4))
    n_cand = int(rng.integers(0, 14))
    p = n_cand + w - 1
    S = rng.integers(0, 5, size=p + 1).astype(np.float64)
    got = O.select_block(S, p, bsz, tb, w)
    n_blocks = (n_cand + bsz - 1) // bsz
    bmax = [max(S[b * bsz:min(n_cand, (b + 1) * bsz)]) for b in range(n_blocks)]
    chosen = brute_force_topk(np.array(bmax), tb) if n_blocks else []
    toks = [j for b in chosen for j in range(b * bsz, min(n_cand, (b + 1) * bsz))]
    assert list(got) == toks + list(range(max(0, p - w + 1), p + 1))
    # block scores are the per-block maxima over candidates, and the block
    # threshold is the lowest score among the enumerated best blocks
    assert list(O.block_scores(S, p, bsz, w)) == bmax
    tau = O.kth_block_score(S, p, bsz, tb, w)
    assert tau == (min(bmax[b] for b in chosen) if n_blocks else np.inf)


def test_block_scores_literal_values():
    # block 2 reaches into the window (p = 10, window 2: candidates j <= 8);
    # its window key 9 has the row's largest score and must not count
    S = np.array([0.1, 0.3, 0.2, 0.0,  0.5, 0.4, 0.45, 0.6,  0.05, 0.9, 0.8])
    np.testing.assert_array_equal(O.block_scores(S, 10, 4, 2), [0.3, 0.6, 0.05])
    assert O.kth_block_score(S, 10, 4, 1, 2) == 0.6
    assert O.kth_block_score(S, 10, 4, 2, 2) == 0.3
    assert O.kth_block_score(S, 10, 4, 3, 2) == 0.05
    assert O.kth_block_score(S, 10, 4, 5, 2) == 0.05
    assert list(O.select_block(S, 10, 4, 1, 2)) == [4, 5, 6, 7, 9, 10]
    assert list(O.select_block(S, 10, 4, 3, 2)) == [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10]


# --------------------------------------------------------------------------
# streamed sampled-row oracle agrees with the dense one
# --------------------------------------------------------------------------
@pytest.mark.parametrize("select", ["token", "block"])
def test_streamed_rows_match_dense(select):
    B, nq, nkv, hq, hkv, d = 2, 20, 75, 4, 2, 8
    q, k, v = rand((B, nq, hq, d), 32), rand((B, nkv, hkv, d), 33), rand((B, nkv, hkv, d), 34)
    qs = rand((2, B, nq, hq, d), 35)
    kw = dict(top_k=12, window=5, select=select, block_size=4, top_blocks=3)
    dense = O.block_forward(q, qs, k, v, **kw)
    rows = [0, 3, 19]
    for b in range(B):
        s = O.block_rows(q, qs, k, v, b, rows, chunk=16, **kw)
        np.testing.assert_allclose(s["lse"], dense["lse"][b][:, rows].T, atol=1e-12)
        np.testing.assert_allclose(s["o_full"], dense["o_full"][b, rows], atol=1e-12)
        np.testing.assert_allclose(s["S"], dense["S"][b, rows], atol=1e-13)
        np.testing.assert_array_equal(s["idx"], dense["idx"][b, rows])
        np.testing.assert_allclose(s["o_sparse"], dense["o_sparse"][:, b, rows], atol=1e-12)


def test_bf16_bits_widen_exactly():
    vals = np.array([1.0, -2.5, 0.1015625, 2.0 ** 100, 0.0], dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(O.widen(bits), vals.astype(np.float64))


# --------------------------------------------------------------------------
# near-tie agreement rule
# --------------------------------------------------------------------------
def test_compare_selection_rule():
    p, w, k = 9, 2, 3
    S = np.array([0.5, 0.3, 0.3 * (1 - 4e-7), 0.1, 0.3 * (1 - 5e-6), 0.05, 0.0, 0.0, 0.0, 0.0])
    ref = O.select_token(S, p, k, w)
    tau = O.kth_candidate_score(S, p, k, w)
    assert list(ref) == [0, 1, 2, 8, 9]
    ok, n, _ = O.compare_selection(ref, ref, S, p, w, tau)
    assert ok and n == 0
    swapped_tie = [0, 1, 4, 8, 9]      # index 4 is 5e-6 below tau: not a tie
    ok, _, why = O.compare_selection(swapped_tie, ref, S, p, w, tau)
    assert not ok and why == "beyond-tie"
    S2 = S.copy()
    S2[4] = 0.3 * (1 - 9e-7)
    ref2 = O.select_token(S2, p, k, w)
    ok, n, _ = O.compare_selection([0, 1, 4, 8, 9], ref2, S2, p, w,
                                   O.kth_candidate_score(S2, p, k, w))
    assert ok and n == 2
    ok, _, why = O.compare_selection([0, 1, 2, 7, 9], ref, S, p, w, tau)
    assert not ok and why == "window"


def test_compare_selection_band_sits_on_the_kth_score():
    # candidates 0..4 (p = 6, window 2), k = 3. Key 1 sits 9e-7 above the
    # k-th score 0.3 (key 2) and key 3 sits 9e-7 below it: both are within
    # 1e-6 of tau = 0.3, so a row that keeps 3 instead of 1 is an excused
    # near-tie. A band around the (k+1)-th score (key 3) would reject it.
    p, w, k = 6, 2, 3
    S = np.array([0.5, 0.3 * (1 + 9e-7), 0.3, 0.3 * (1 - 9e-7), 0.1, 0.0, 0.0])
    ref = O.select_token(S, p, k, w)
    assert list(ref) == [0, 1, 2, 5, 6]
    tau = O.kth_candidate_score(S, p, k, w)
    assert tau == 0.3
    ok, n, _ = O.compare_selection([0, 2, 3, 5, 6], ref, S, p, w, tau)
    assert ok and n == 2
    ok, _, why = O.compare_selection([0, 2, 3, 5, 6], ref, S, p, w, S[3])
    assert not ok and why == "beyond-tie"
    # a swap with key 4, far below tau, is never excused
    ok, _, why = O.compare_selection([0, 1, 4, 5, 6], ref, S, p, w, tau)
    assert not ok and why == "beyond-tie"


def test_compare_selection_block_rule():
    # blocks of 4. First p = 12, window 2: candidates j <= 10, so block 2
    # holds candidates 8..10 only; window key 11 (score 0.9) lies in its span
    # and must not raise its score.
    w, bsz, tb = 2, 4, 2
    S = np.full(14, 0.01)
    S[1] = 0.5                         # block 0: max 0.5
    S[5] = 0.3 * (1 + 6e-7)            # block 1: max 0.3(1 + 6e-7)
    S[9] = 0.3                         # block 2: max 0.3, its other keys 0.01
    S[11] = 0.9
    ref = O.select_block(S, 12, bsz, tb, w)
    assert list(ref) == [0, 1, 2, 3, 4, 5, 6, 7, 11, 12]
    assert O.kth_block_score(S, 12, bsz, tb, w) == S[5]
    # Then p = 13: block 2 = keys 8..11, all candidates, with key 11 lowered.
    S[11] = 0.2
    p = 13
    ref = O.select_block(S, p, bsz, tb, w)
    assert list(ref) == [0, 1, 2, 3, 4, 5, 6, 7, 12, 13]
    tau = O.kth_block_score(S, p, bsz, tb, w)
    assert tau == S[5]
    # blocks 0 and 2 instead of 0 and 1: block 2's max (not its min) is
    # within 1e-6 of tau, so the swap is an excused near-tie
    gpu = [0, 1, 2, 3, 8, 9, 10, 11, 12, 13]
    ok, n, _ = O.compare_selection(gpu, ref, S, p, w, tau, block_size=bsz)
    assert ok and n == 8
    # the same swap when block 2's max is far from tau is not excused
    S3 = S.copy()
    S3[9] = 0.2
    ok, _, why = O.compare_selection(gpu, O.select_block(S3, p, bsz, tb, w), S3, p, w,
                                     O.kth_block_score(S3, p, bsz, tb, w), block_size=bsz)
    assert not ok and why == "beyond-tie"
    # a row of another size (a block cut at the window edge) never agrees
    ok, _, why = O.compare_selection(gpu[:-3] + [13], ref, S, p, w, tau, block_size=bsz)
    assert not ok and why == "size"


def test_pages_constants():
    c = json.load(open(os.path.join(GOLDEN, "pages_constants.json")))
    from synth import CONFIGS
    for w in CONFIGS.values():
        assert w.top_k == c["top_k_global_tokens"]["value"]
        assert w.window == c["recent_window_tokens"]["value"]
        assert w.block_size == c["previous_generation_block_tokens"]["value"]


# ----------------------------------------------------------------------------
# one decode step over a growing cache
# ----------------------------------------------------------------------------
def _decode_case(seed, lens, cap=40, hq=4, hkv=2, d=8, L=2):
    B = len(lens)
    return dict(q_full=rand((B, 1, hq, d), seed), q_sparse=rand((L, B, 1, hq, d), seed + 1),
                k_new=rand((B, 1, hkv, d), seed + 2), v_new=rand((B, 1, hkv, d), seed + 3),
                k_cache=rand((B, cap, hkv, d), seed + 4), v_cache=rand((B, cap, hkv, d), seed + 5),
                lens=lens)


def test_decode_step_is_last_row_of_prefill():
    # the step's query sees keys 0..lens[b] with its own row last: the same
    # as the last row of the causal prefill over that prefix
    c = _decode_case(40, [20, 33, 3])
    got = O.decode_step(**c, top_k=5, window=4)
    for b, n in enumerate(c["lens"]):
        k = np.concatenate([c["k_cache"][b, :n], c["k_new"][b]])[None]
        v = np.concatenate([c["v_cache"][b, :n], c["v_new"][b]])[None]
        q = np.concatenate([rand((n, 4, 8), 90 + b), c["q_full"][b]])[None]
        qs = np.concatenate([rand((2, n, 4, 8), 95 + b), c["q_sparse"][:, b]], axis=1)[:, None]
        ref = O.block_forward(q, qs, k, v, top_k=5, window=4)
        np.testing.assert_allclose(got["o_full"][b, 0], ref["o_full"][0, -1], atol=1e-12)
        np.testing.assert_allclose(got["lse"][b, :, 0], ref["lse"][0, :, -1], atol=1e-12)
        np.testing.assert_array_equal(got["idx"][b, 0], ref["idx"][0, -1])
        np.testing.assert_allclose(got["o_sparse"][:, b, 0], ref["o_sparse"][:, 0, -1], atol=1e-12)


def test_decode_step_ignores_rows_past_length():
    c = _decode_case(50, [7, 25])
    base = O.decode_step(**c, top_k=4, window=3)
    for b, n in enumerate(c["lens"]):
        c["k_cache"][b, n:] = 1e6
        c["v_cache"][b, n:] = -1e6
    again = O.decode_step(**c, top_k=4, window=3)
    for key in ("o_full", "lse", "idx", "o_sparse"):
        np.testing.assert_array_equal(base[key], again[key])


def test_decode_step_zero_keys_closed_form():
    # every logit 0: LSE = log(n + 1) over the n + 1 keys, and ties take the
    # lowest candidate indices before the window
    c = _decode_case(60, [30, 10, 0])
    c["k_cache"][:] = 0
    c["k_new"][:] = 0
    got = O.decode_step(**c, top_k=6, window=5)
    for b, n in enumerate(c["lens"]):
        np.testing.assert_allclose(got["lse"][b, :, 0], math.log(n + 1), atol=1e-12)
        n_c = max(0, n - 5 + 1)
        want = list(range(min(6, n_c))) + list(range(max(0, n - 4), n + 1))
        row = got["idx"][b, 0]
        assert list(row[row >= 0]) == want


def test_paged_decode_step_matches_contiguous():
    # a pool whose pages hold the same rows in shuffled order gives the same
    # step as the contiguous cache
    c = _decode_case(70, [37, 64, 5], cap=64)
    ps, mp = 16, 4
    B = 3
    rng = np.random.default_rng(7)
    perm = rng.permutation(B * mp + 2)[:B * mp]       # pool of 14 pages, 12 used
    table = perm.reshape(B, mp).astype(np.int32)
    k_pool = rand(((B * mp + 2) * ps, 2, 8), 71)
    v_pool = rand(((B * mp + 2) * ps, 2, 8), 72)
    for b in range(B):
        rows = O.pool_rows(table, ps, b, mp * ps)
        k_pool[rows] = c["k_cache"][b]
        v_pool[rows] = c["v_cache"][b]
    want = O.decode_step(**c, top_k=5, window=4)
    got = O.decode_step_paged(c["q_full"], c["q_sparse"], c["k_new"], c["v_new"], k_pool, v_pool,
                              table, ps, c["lens"], top_k=5, window=4)
    for key in ("o_full", "lse", "idx", "o_sparse"):
        np.testing.assert_array_equal(want[key], got[key])
    # pool rows: position j of sequence b sits in page table[b, j // ps]
    assert list(O.pool_rows(table, ps, 1, 20)[15:18]) == [
        table[1, 0] * ps + 15, table[1, 1] * ps + 0, table[1, 1] * ps + 1]


# ----------------------------------------------------------------------------
# KV Bridging projection
# ----------------------------------------------------------------------------
def test_kv_bridge_brute_force():
    h = rand((2, 3, 5), 80)
    w = rand((2, 6, 5), 81)
    k, v = O.kv_bridge(h, w, h_kv=2)
    for b in range(2):
        for t in range(3):
            for f in range(6):
                want_k = sum(h[b, t, c] * w[0, f, c] for c in range(5))
                want_v = sum(h[b, t, c] * w[1, f, c] for c in range(5))
                assert abs(k[b, t, f // 3, f % 3] - want_k) < 1e-12
                assert abs(v[b, t, f // 3, f % 3] - want_v) < 1e-12


def test_kv_bridge_feature_selection():
    # weight rows that are unit vectors copy hidden features: exact
    h = rand((1, 4, 8), 82)
    perm = np.random.default_rng(83).permutation(8)
    w = np.zeros((2, 8, 8))
    w[0, np.arange(8), perm] = 1.0
    w[1, np.arange(8), perm[::-1]] = 2.0
    k, v = O.kv_bridge(h, w, h_kv=2)
    np.testing.assert_array_equal(k.reshape(1, 4, 8), h[:, :, perm])
    np.testing.assert_array_equal(v.reshape(1, 4, 8), 2.0 * h[:, :, perm[::-1]])


# ----------------------------------------------------------------------------
# backward pass (index sets held fixed)
# ----------------------------------------------------------------------------
def _bwd_case(seed, B=1, nq=6, nkv=9, hq=4, hkv=2, d=3, L=2, top_k=2, window=2):
    q, qs = rand((B, nq, hq, d), seed), rand((L, B, nq, hq, d), seed + 1)
    k, v = rand((B, nkv, hkv, d), seed + 2), rand((B, nkv, hkv, d), seed + 3)
    dof, dos = rand((B, nq, hq, d), seed + 4), rand((L, B, nq, hq, d), seed + 5)
    idx = O.block_forward(q, qs, k, v, top_k=top_k, window=window)["idx"]
    return dict(q_full=q, q_sparse=qs, k=k, v=v, idx=idx, do_full=dof, do_sparse=dos)


def _block_loss(c):
    """sum(dO * O) over the full layer and every sparse layer: its gradient
    with respect to any input is what the backward pass returns."""
    o, _ = O.full_layer(c["q_full"], c["k"], c["v"])
    total = float((c["do_full"] * o).sum())
    for l in range(c["q_sparse"].shape[0]):
        ol = O.sparse_layer(c["q_sparse"][l], c["k"], c["v"], c["idx"])
        total += float((c["do_sparse"][l] * ol).sum())
    return total


def test_backward_matches_finite_differences():
    # central differences of the (separately pinned) forward pass, for every
    # input element; the idx sets stay fixed while inputs move
    c = _bwd_case(100)
    g = O.block_backward(**c)
    eps = 1e-6
    for name, gname in (("q_full", "dq_full"), ("q_sparse", "dq_sparse"), ("k", "dk"),
                        ("v", "dv")):
        x = c[name]
        num = np.zeros_like(x)
        for pos in np.ndindex(*x.shape):
            old = x[pos]
            x[pos] = old + eps
            up = _block_loss(c)
            x[pos] = old - eps
            down = _block_loss(c)
            x[pos] = old
            num[pos] = (up - down) / (2 * eps)
        np.testing.assert_allclose(g[gname], num, rtol=0, atol=2e-7, err_msg=name)


def test_backward_matches_torch_autograd():
    # torch's fp64 attention differentiated by autograd: the full layer with
    # an end-aligned causal mask, the sparse layers with the idx sets as mask
    B, nq, nkv, hq, hkv, d, L = 2, 7, 11, 6, 2, 8, 2
    c = _bwd_case(110, B=B, nq=nq, nkv=nkv, hq=hq, hkv=hkv, d=d, L=L, top_k=3, window=3)
    got = O.block_backward(**c)
    t = {n: torch.from_numpy(c[n].copy()).requires_grad_(True)
         for n in ("q_full", "q_sparse", "k", "v")}
    pos = torch.arange(nq) + (nkv - nq)
    causal = torch.arange(nkv)[None, :] <= pos[:, None]
    kt, vt = t["k"].permute(0, 2, 1, 3), t["v"].permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(t["q_full"].permute(0, 2, 1, 3), kt, vt, attn_mask=causal,
                                       enable_gqa=True)
    loss = (o * torch.from_numpy(c["do_full"]).permute(0, 2, 1, 3)).sum()
    chosen = torch.zeros((B, 1, nq, nkv), dtype=torch.bool)
    for b in range(B):
        for i in range(nq):
            sel = c["idx"][b, i][c["idx"][b, i] >= 0]
            chosen[b, 0, i, torch.from_numpy(sel)] = True
    for l in range(L):
        ol = F.scaled_dot_product_attention(t["q_sparse"][l].permute(0, 2, 1, 3), kt, vt,
                                            attn_mask=chosen, enable_gqa=True)
        loss = loss + (ol * torch.from_numpy(c["do_sparse"][l]).permute(0, 2, 1, 3)).sum()
    loss.backward()
    for n, gn in (("q_full", "dq_full"), ("q_sparse", "dq_sparse"), ("k", "dk"), ("v", "dv")):
        np.testing.assert_allclose(got[gn], t[n].grad.numpy(), rtol=0, atol=1e-11, err_msg=n)


def test_backward_sum_invariants():
    # every softmax row sums to 1, so the V gradients of a KV group add up to
    # the group's output gradients; the softmax Jacobian kills constants, so
    # the K gradients of a group sum to zero
    c = _bwd_case(120, B=2, nq=10, nkv=16, hq=6, hkv=3, d=5, L=3, top_k=4, window=3)
    g = O.block_backward(**c)
    G = 2
    for b in range(2):
        for kv in range(3):
            heads = slice(kv * G, (kv + 1) * G)
            want = c["do_full"][b, :, heads].sum(axis=(0, 1)) + \
                c["do_sparse"][:, b, :, heads].sum(axis=(0, 1, 2))
            np.testing.assert_allclose(g["dv"][b, :, kv].sum(axis=0), want, atol=1e-12)
            np.testing.assert_allclose(g["dk"][b, :, kv].sum(axis=0), 0.0, atol=1e-12)


def test_backward_constant_values_closed_form():
    # V rows all equal: every output is that row whatever the weights, so Q
    # and K get no gradient and dV spreads dO by the probabilities
    c = _bwd_case(130, nq=8, nkv=8, top_k=3, window=2)
    c["v"][:] = rand((1, 1, 2, 3), 131)
    g = O.block_backward(**c)
    np.testing.assert_allclose(g["dq_full"], 0.0, atol=1e-13)
    np.testing.assert_allclose(g["dq_sparse"], 0.0, atol=1e-13)
    np.testing.assert_allclose(g["dk"], 0.0, atol=1e-13)
    # the first query sees only key 0 in the full layer: P = 1
    d0 = O.block_backward(**{**c, "do_sparse": np.zeros_like(c["do_sparse"]),
                             "do_full": np.where(np.arange(8)[None, :, None, None] == 0,
                                                 c["do_full"], 0.0)})
    np.testing.assert_allclose(d0["dv"][0, 0, 0], c["do_full"][0, 0, :2].sum(axis=0), atol=1e-13)
    np.testing.assert_allclose(d0["dv"][0, 1:], 0.0, atol=1e-13)


@pytest.mark.parametrize("j_lo", [0, 9, 15])
def test_backward_tail_matches_dense(j_lo):
    c = _bwd_case(140, B=2, nq=8, nkv=17, hq=4, hkv=2, d=6, L=2, top_k=3, window=3)
    dense = O.block_backward(**c)
    for b in range(2):
        t = O.block_backward_tail(c["q_full"], c["q_sparse"], c["k"], c["v"], c["idx"],
                                  c["do_full"], c["do_sparse"], b, j_lo)
        rows = t["rows"]
        assert list(rows) == list(range(max(0, j_lo - 9), 8))
        np.testing.assert_allclose(t["dq_full"], dense["dq_full"][b, rows], atol=1e-12)
        np.testing.assert_allclose(t["dq_sparse"], dense["dq_sparse"][:, b, rows], atol=1e-12)
        np.testing.assert_allclose(t["dk"], dense["dk"][b, j_lo:], atol=1e-12)
        np.testing.assert_allclose(t["dv"], dense["dv"][b, j_lo:], atol=1e-12)
    # the summand magnitudes agree the same way
    dense = O.block_backward(**c, with_mag=True)["mag"]
    t = O.block_backward_tail(c["q_full"], c["q_sparse"], c["k"], c["v"], c["idx"],
                              c["do_full"], c["do_sparse"], 1, j_lo, with_mag=True)
    m, rows = t["mag"], t["rows"]
    np.testing.assert_allclose(m["dq_full"], dense["dq_full"][1, rows], atol=1e-12)
    np.testing.assert_allclose(m["dq_sparse"], dense["dq_sparse"][:, 1, rows], atol=1e-12)
    np.testing.assert_allclose(m["dk"], dense["dk"][1, j_lo:], atol=1e-12)
    np.testing.assert_allclose(m["dv"], dense["dv"][1, j_lo:], atol=1e-12)


def test_backward_summand_magnitudes():
    # the per-element error bound of the GPU comparison scales with these:
    # every gradient element is at most its magnitude (triangle inequality),
    # dV equals its magnitude when every output gradient is nonnegative (all
    # its summands P * dO are then >= 0), magnitudes are linear in |dO|, and
    # the gradients themselves do not change when magnitudes are requested
    c = _bwd_case(150, B=2, nq=7, nkv=11, hq=4, hkv=2, d=5, L=2, top_k=3, window=2)
    plain = O.block_backward(**c)
    r = O.block_backward(**c, with_mag=True)
    for n in ("dq_full", "dq_sparse", "dk", "dv"):
        np.testing.assert_array_equal(r[n], plain[n])
        assert np.all(np.abs(r[n]) <= r["mag"][n] + 1e-13), n
        assert np.all(r["mag"][n] >= 0), n
    c2 = dict(c, do_full=np.abs(c["do_full"]), do_sparse=np.abs(c["do_sparse"]))
    r2 = O.block_backward(**c2, with_mag=True)
    np.testing.assert_allclose(r2["mag"]["dv"], r2["dv"], rtol=1e-13, atol=1e-14)
    c3 = dict(c, do_full=-3 * c["do_full"], do_sparse=-3 * c["do_sparse"])
    r3 = O.block_backward(**c3, with_mag=True)
    for n in ("dq_full", "dq_sparse", "dk", "dv"):
        np.testing.assert_allclose(r3["mag"][n], 3 * r["mag"][n], rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# variable-length batches
# ----------------------------------------------------------------------------
def test_varlen_equal_lengths_is_the_batched_block():
    B, nq, nkv, hq, hkv, d, L = 3, 6, 14, 4, 2, 8, 2
    q, qs = rand((B, nq, hq, d), 150), rand((L, B, nq, hq, d), 151)
    k, v = rand((B, nkv, hkv, d), 152), rand((B, nkv, hkv, d), 153)
    want = O.block_forward(q, qs, k, v, top_k=3, window=4)
    cu_q, cu_kv = np.arange(B + 1) * nq, np.arange(B + 1) * nkv
    got = O.block_forward_varlen(q.reshape(B * nq, hq, d), qs.reshape(L, B * nq, hq, d),
                                 k.reshape(B * nkv, hkv, d), v.reshape(B * nkv, hkv, d),
                                 cu_q, cu_kv, top_k=3, window=4)
    np.testing.assert_array_equal(got["o_full"], want["o_full"].reshape(B * nq, hq, d))
    np.testing.assert_array_equal(got["o_sparse"], want["o_sparse"].reshape(L, B * nq, hq, d))
    np.testing.assert_array_equal(got["idx"], want["idx"].reshape(B * nq, -1))
    for b in range(B):
        np.testing.assert_array_equal(got["lse"][b], want["lse"][b])


def test_varlen_sequences_are_independent():
    # changing one sequence's data leaves every other sequence's results alone
    cu_q, cu_kv = [0, 5, 5, 6, 10], [0, 9, 12, 20, 24]
    hq, hkv, d, L = 4, 1, 8, 2
    q, qs = rand((10, hq, d), 160), rand((L, 10, hq, d), 161)
    k, v = rand((24, hkv, d), 162), rand((24, hkv, d), 163)
    a = O.block_forward_varlen(q, qs, k, v, cu_q, cu_kv, top_k=2, window=3)
    k2 = k.copy()
    k2[12:20] = rand((8, hkv, d), 164)             # sequence 2's keys
    b = O.block_forward_varlen(q, qs, k2, v, cu_q, cu_kv, top_k=2, window=3)
    other = np.r_[0:5, 6:10]
    np.testing.assert_array_equal(a["o_full"][other], b["o_full"][other])
    np.testing.assert_array_equal(a["idx"][other], b["idx"][other])
    assert not np.array_equal(a["o_full"][5], b["o_full"][5])
    assert a["lse"][1] is None                     # the empty sequence
    # the one-query sequence sits at the last position of its 8 keys
    assert a["idx"][5][a["idx"][5] >= 0][-1] == 7


# ----------------------------------------------------------------------------
# chunked prefill over a paged pool
# ----------------------------------------------------------------------------
def _paged_prefill_case(seed, lens, chunks, ps=8, mp=6, hq=4, hkv=2, d=8, L=2):
    B = len(lens)
    n_pages = B * mp + 3
    table = np.random.default_rng(seed).permutation(n_pages)[:B * mp].reshape(B, mp)
    cu_q = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    tq = int(cu_q[-1])
    return dict(q_full=rand((tq, hq, d), seed + 1), q_sparse=rand((L, tq, hq, d), seed + 2),
                k_new=rand((tq, hkv, d), seed + 3), v_new=rand((tq, hkv, d), seed + 4),
                k_pool=rand((n_pages * ps, hkv, d), seed + 5),
                v_pool=rand((n_pages * ps, hkv, d), seed + 6),
                page_table=table.astype(np.int32), page_size=ps, cu_q=cu_q, lens=lens)


def test_paged_prefill_chunk_is_tail_of_full_prefill():
    # a chunk appended after n cached tokens gives its queries the results
    # they get as the last rows of a causal prefill over all n + chunk tokens
    # (earlier queries change nothing for later ones)
    c = _paged_prefill_case(200, [13, 0, 30], [7, 5, 1])
    got = O.block_forward_paged(**c, top_k=4, window=3)
    for b, n in enumerate(c["lens"]):
        q0, q1 = int(c["cu_q"][b]), int(c["cu_q"][b + 1])
        rows = O.pool_rows(c["page_table"], c["page_size"], b, n)
        k = np.concatenate([c["k_pool"][rows], c["k_new"][q0:q1]])[None]
        v = np.concatenate([c["v_pool"][rows], c["v_new"][q0:q1]])[None]
        q = np.concatenate([rand((n, 4, 8), 210 + b), c["q_full"][q0:q1]])[None]
        qs = np.concatenate([rand((2, n, 4, 8), 220 + b), c["q_sparse"][:, q0:q1]], axis=1)[:, None]
        ref = O.block_forward(q, qs, k, v, top_k=4, window=3)
        m = q1 - q0
        np.testing.assert_allclose(got["o_full"][q0:q1], ref["o_full"][0, n:], atol=1e-12)
        np.testing.assert_allclose(got["lse"][b], ref["lse"][0, :, n:], atol=1e-12)
        np.testing.assert_array_equal(got["idx"][q0:q1], ref["idx"][0, n:])
        np.testing.assert_allclose(got["o_sparse"][:, q0:q1], ref["o_sparse"][:, 0, n:],
                                   atol=1e-12)
        assert len(got["new_rows"][b]) == m


def test_paged_prefill_one_token_is_the_paged_decode_step():
    # one new token per sequence: the paged decode step
    c = _paged_prefill_case(230, [9, 40, 0], [1, 1, 1])
    got = O.block_forward_paged(**c, top_k=3, window=5)
    want = O.decode_step_paged(c["q_full"][:, None], c["q_sparse"][:, :, None],
                               c["k_new"][:, None], c["v_new"][:, None], c["k_pool"],
                               c["v_pool"], c["page_table"], c["page_size"], c["lens"],
                               top_k=3, window=5)
    np.testing.assert_array_equal(got["o_full"], want["o_full"][:, 0])
    np.testing.assert_array_equal(got["idx"], want["idx"][:, 0])
    np.testing.assert_array_equal(got["o_sparse"], want["o_sparse"][:, :, 0])
    # the new token of sequence b lands at position lens[b] of its pages
    for b, n in enumerate(c["lens"]):
        ps = c["page_size"]
        assert got["new_rows"][b][0] == c["page_table"][b, n // ps] * ps + n % ps
