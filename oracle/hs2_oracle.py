"""CPU oracle for the HySparse2 Hybrid Block: plain fp64 NumPy, slow on purpose.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run this module; the library's
product path never does, and this module shares no code with it.

What it computes, step by step (the pages describe the method in prose only):

1. Full layer ("Two-Level KV Sharing: ..." on the openai-hub.net page, section
   "From Hybrid SWA to HySparse2"): causal attention of every query head over
   the shared K/V, s_h(p, j) = <Q[p, h], K[j, g(h)]> * scale for j <= p, with
   grouped-query heads g(h) = floor(h * h_kv / h_q) and scale 1/sqrt(d).
   Outputs O_full and the per-head natural-log LSE.
2. Importance score: the same page says the full layer also decides which
   tokens matter. Reading used: S(p, j) = sum over all query heads of the full
   layer's softmax probability P_h(p, j), one score row per query.
3. Token-level selection ("Xiaomi Unveils HySparse2", section "Token-Level
   Selection and Unified Local Access"; bibibi.cc, section "Article"): the 128
   most recent tokens are always kept; up to 1024 further tokens are chosen
   from outside that window. Candidates are C_p = {0 <= j <= p - w}; the
   chosen set is the first min(k, |C_p|) candidates in the order of
   (-S(p, j), j), i.e. ties go to the lower index.
4. Block selection, the previous generation's variant (bibibi.cc, section
   "Article": 64-token groups kept whole): block score = max candidate score
   in the block, top blocks ordered by (-score, block id), expanded to their
   candidate tokens.
5. Sparse layers ("Xiaomi Unveils HySparse2", section "Two-Level KV Sharing",
   KV Reuse; and section "Token-Level Selection and Unified Local Access"):
   every sparse layer attends, with one softmax, over window + selected
   tokens, reading the same K/V and the same index set as the full layer.

6. Backward pass, for fine-tuning ("Xiaomi Unveils HySparse2", section
   "Performance Gains: Cost, Speed, and Long-Context Capabilities": the
   compared models are fine-tuned alike before evaluation). Reading used: the
   index sets are held fixed (a discrete choice has no gradient, so the score
   and selection steps pass none back); the full layer and every sparse layer
   are differentiated as ordinary softmax attention, and because all of them
   read the one K/V buffer (KV Reuse) their K and V gradients add up.

Inputs may be float32/float64 arrays or raw bf16 bit patterns (uint16); they
are widened exactly to fp64.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# input widening
# ----------------------------------------------------------------------------
def widen(x) -> np.ndarray:
    """Exact fp64 copy of an fp32/fp64 array or of raw bf16 bits (uint16)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def group_of(h: int, h_q: int, h_kv: int) -> int:
    """KV head read by query head h: consecutive query heads share one."""
    return (h * h_kv) // h_q


# ----------------------------------------------------------------------------
# step 1: full causal attention + per-head LSE (dense, small shapes)
# ----------------------------------------------------------------------------
def full_layer(q, k, v, scale=None):
    """Dense causal GQA attention.

    q [B, n_q, h_q, d], k/v [B, n_kv, h_kv, d]; query i is at position
    n_kv - n_q + i. Returns (O [B, n_q, h_q, d], lse [B, h_q, n_q]) in fp64.
    """
    q, k, v = widen(q), widen(k), widen(v)
    B, nq, hq, d = q.shape
    nkv, hkv = k.shape[1], k.shape[2]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    pos = np.arange(nq) + (nkv - nq)
    keep = np.arange(nkv)[None, :] <= pos[:, None]          # causal mask
    out = np.zeros((B, nq, hq, d))
    lse = np.zeros((B, hq, nq))
    for b in range(B):
        for h in range(hq):
            g = group_of(h, hq, hkv)
            s = (q[b, :, h, :] @ k[b, :, g, :].T) * scale
            s = np.where(keep, s, NEG_INF)
            m = s.max(axis=1, keepdims=True)
            l = np.exp(s - m).sum(axis=1, keepdims=True)
            row_lse = m + np.log(l)
            p = np.exp(s - row_lse)
            out[b, :, h, :] = p @ v[b, :, g, :]
            lse[b, h, :] = row_lse[:, 0]
    return out, lse


# ----------------------------------------------------------------------------
# step 2: head-summed importance score
# ----------------------------------------------------------------------------
def scores(q, k, lse, scale=None):
    """S[b, i, j] = sum_h exp(s_h(p, j) - lse_h(p)) for j <= p, 0 beyond p.

    `lse` is the full layer's per-head LSE [B, h_q, n_q] (natural log), so the
    normaliser covers every key j <= p, window keys included.
    """
    q, k = widen(q), widen(k)
    B, nq, hq, d = q.shape
    nkv, hkv = k.shape[1], k.shape[2]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    pos = np.arange(nq) + (nkv - nq)
    keep = np.arange(nkv)[None, :] <= pos[:, None]
    S = np.zeros((B, nq, nkv))
    for b in range(B):
        for h in range(hq):
            g = group_of(h, hq, hkv)
            s = (q[b, :, h, :] @ k[b, :, g, :].T) * scale
            p = np.where(keep, np.exp(np.where(keep, s, 0.0) - lse[b, h][:, None]), 0.0)
            S[b] += p
    return S


# ----------------------------------------------------------------------------
# step 3/4: selection
# ----------------------------------------------------------------------------
def window_of(p: int, window: int) -> np.ndarray:
    return np.arange(max(0, p - window + 1), p + 1)


def select_token(S_row, p: int, top_k: int, window: int) -> np.ndarray:
    """Ascending index set: top-k candidates by (-S, j) plus the window."""
    S_row = np.asarray(S_row, dtype=np.float64)
    n_cand = max(0, p - window + 1)
    cand = np.arange(n_cand)
    order = np.lexsort((cand, -S_row[:n_cand]))       # primary -S, then index
    chosen = np.sort(cand[order[:min(top_k, n_cand)]])
    return np.concatenate([chosen, window_of(p, window)]).astype(np.int64)


def select_block(S_row, p: int, block_size: int, top_blocks: int,
                 window: int) -> np.ndarray:
    """Block-level variant: blocks of candidates ranked by their max score."""
    S_row = np.asarray(S_row, dtype=np.float64)
    n_cand = max(0, p - window + 1)
    n_blocks = (n_cand + block_size - 1) // block_size
    bscore = np.array([S_row[bi * block_size:min(n_cand, (bi + 1) * block_size)].max()
                       for bi in range(n_blocks)]) if n_blocks else np.zeros(0)
    bid = np.arange(n_blocks)
    order = np.lexsort((bid, -bscore))
    chosen_blocks = np.sort(bid[order[:min(top_blocks, n_blocks)]])
    toks = [np.arange(bi * block_size, min(n_cand, (bi + 1) * block_size))
            for bi in chosen_blocks]
    chosen = np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)
    return np.concatenate([chosen, window_of(p, window)]).astype(np.int64)


def block_scores(S_row, p: int, block_size: int, window: int) -> np.ndarray:
    """Score of each block of candidates: the largest candidate score in it.

    Block b holds keys b*block_size .. (b+1)*block_size - 1; only its keys
    j <= p - window count (a block that reaches into the window is scored on
    its candidate keys alone)."""
    n_cand = max(0, p - window + 1)
    n_blocks = (n_cand + block_size - 1) // block_size
    return np.array([np.asarray(S_row[bi * block_size:min(n_cand, (bi + 1) * block_size)],
                                dtype=np.float64).max() for bi in range(n_blocks)])


def kth_candidate_score(S_row, p: int, top_k: int, window: int) -> float:
    """tau_p: the score of the k-th ranked candidate (the selection threshold).

    With fewer than k candidates it is the lowest candidate score; with none,
    +inf."""
    n_cand = max(0, p - window + 1)
    if n_cand == 0:
        return np.inf
    vals = np.sort(np.asarray(S_row[:n_cand], dtype=np.float64))[::-1]
    return float(vals[min(top_k, n_cand) - 1])


def kth_block_score(S_row, p: int, block_size: int, top_blocks: int, window: int) -> float:
    """Block-mode threshold: the block score of the top_blocks-th ranked block
    (the lowest one when fewer blocks exist; +inf with no candidates)."""
    bs = block_scores(S_row, p, block_size, window)
    if len(bs) == 0:
        return np.inf
    return float(np.sort(bs)[::-1][min(top_blocks, len(bs)) - 1])


def pad_index_row(idx_row, width: int) -> np.ndarray:
    out = np.full(width, -1, dtype=np.int64)
    out[:len(idx_row)] = idx_row
    return out


# ----------------------------------------------------------------------------
# step 5: sparse layers over a given index set
# ----------------------------------------------------------------------------
def sparse_layer(q_l, k, v, idx, scale=None):
    """One sparse layer. q_l [B, n_q, h_q, d]; idx [B, n_q, W] (-1 = unused).

    For each query and head: softmax over the listed keys only, then the
    probability-weighted sum of their values.
    """
    q_l, k, v = widen(q_l), widen(k), widen(v)
    B, nq, hq, d = q_l.shape
    hkv = k.shape[2]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    idx = np.asarray(idx)
    out = np.zeros((B, nq, hq, d))
    for b in range(B):
        for i in range(nq):
            sel = idx[b, i][idx[b, i] >= 0]
            for h in range(hq):
                g = group_of(h, hq, hkv)
                s = (k[b, sel, g, :] @ q_l[b, i, h, :]) * scale
                e = np.exp(s - s.max())
                out[b, i, h, :] = (e / e.sum()) @ v[b, sel, g, :]
    return out


# ----------------------------------------------------------------------------
# the whole block, dense (small shapes)
# ----------------------------------------------------------------------------
def block_forward(q_full, q_sparse, k, v, top_k=1024, window=128,
                  select="token", block_size=64, top_blocks=16, scale=None):
    """Full layer -> scores -> selection -> every sparse layer, all in fp64.

    q_sparse [L, B, n_q, h_q, d]. Returns dict(o_full, lse, S, idx, tau,
    o_sparse) with idx [B, n_q, W] padded with -1, W = top_k + window in token
    mode and top_blocks * block_size + window in block mode.
    """
    o_full, lse = full_layer(q_full, k, v, scale)
    S = scores(q_full, k, lse, scale)
    B, nq = S.shape[0], S.shape[1]
    nkv = np.asarray(k).shape[1]
    width = top_k + window if select == "token" else top_blocks * block_size + window
    idx = np.full((B, nq, width), -1, dtype=np.int64)
    tau = np.zeros((B, nq))
    for b in range(B):
        for i in range(nq):
            p = nkv - nq + i
            if select == "token":
                row = select_token(S[b, i], p, top_k, window)
                tau[b, i] = kth_candidate_score(S[b, i], p, top_k, window)
            else:
                row = select_block(S[b, i], p, block_size, top_blocks, window)
                tau[b, i] = kth_block_score(S[b, i], p, block_size, top_blocks, window)
            idx[b, i, :len(row)] = row
    q_sparse = np.asarray(q_sparse)
    o_sparse = np.stack([sparse_layer(q_sparse[l], k, v, idx, scale)
                         for l in range(q_sparse.shape[0])]) if q_sparse.shape[0] else \
        np.zeros((0,) + o_full.shape)
    return dict(o_full=o_full, lse=lse, S=S, idx=idx, tau=tau, o_sparse=o_sparse)


def decode_step(q_full, q_sparse, k_new, v_new, k_cache, v_cache, lens, top_k=1024, window=128,
                select="token", block_size=64, top_blocks=16, scale=None):
    """One decode step over a growing cache, per sequence (batch rows may
    hold different lengths).

    For sequence b the new token's K/V row joins the first lens[b] cached
    rows, so the cache the full layer and every sparse layer read ("Two-Level
    KV Sharing", KV Reuse) holds keys 0..lens[b], and the new query sits at
    position lens[b]; the block is then exactly block_forward on that prefix
    with one query. q_full [B, 1, h_q, d], q_sparse [L, B, 1, h_q, d], k_new /
    v_new [B, 1, h_kv, d], k_cache / v_cache [B, cap, h_kv, d] (rows past
    lens[b] are never read). Returns dict(o_full [B, 1, h_q, d], lse
    [B, h_q, 1], S (list of B score rows), idx [B, 1, W], tau [B, 1],
    o_sparse [L, B, 1, h_q, d]).
    """
    q_full, q_sparse = np.asarray(q_full), np.asarray(q_sparse)
    k_new, v_new = np.asarray(k_new), np.asarray(v_new)
    k_cache, v_cache = np.asarray(k_cache), np.asarray(v_cache)
    outs = []
    for b in range(q_full.shape[0]):
        n = int(lens[b])
        kb = np.concatenate([k_cache[b, :n], k_new[b]], axis=0)[None]
        vb = np.concatenate([v_cache[b, :n], v_new[b]], axis=0)[None]
        outs.append(block_forward(q_full[b:b + 1], q_sparse[:, b:b + 1], kb, vb, top_k=top_k,
                                  window=window, select=select, block_size=block_size,
                                  top_blocks=top_blocks, scale=scale))
    return dict(o_full=np.concatenate([o["o_full"] for o in outs]),
                lse=np.concatenate([o["lse"] for o in outs]),
                S=[o["S"][0, 0] for o in outs],
                idx=np.concatenate([o["idx"] for o in outs]),
                tau=np.concatenate([o["tau"] for o in outs]),
                o_sparse=np.concatenate([o["o_sparse"] for o in outs], axis=1))


def block_forward_varlen(q_full, q_sparse, k, v, cu_q, cu_kv, **kw):
    """The block over a packed batch of sequences of different lengths:
    sequence b owns queries cu_q[b]..cu_q[b+1] and keys cu_kv[b]..cu_kv[b+1]
    of the packed tensors (q_full [total_q, h_q, d], q_sparse
    [L, total_q, h_q, d], k/v [total_kv, h_kv, d]) and is exactly
    block_forward of batch 1 on its slices. Returns dict(o_full, o_sparse,
    idx [total_q, W], lse list of [h_q, n_q(b)] arrays, S list, tau list)."""
    q_full, q_sparse = np.asarray(q_full), np.asarray(q_sparse)
    k, v = np.asarray(k), np.asarray(v)
    outs = []
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_kv[b]), int(cu_kv[b + 1])
        if q1 == q0:
            outs.append(None)
            continue
        outs.append(block_forward(q_full[None, q0:q1], q_sparse[:, None, q0:q1],
                                  k[None, k0:k1], v[None, k0:k1], **kw))
    live = [o for o in outs if o is not None]
    L, hq, d = q_sparse.shape[0], q_full.shape[1], q_full.shape[2]
    width = live[0]["idx"].shape[-1] if live else 0
    return dict(
        o_full=np.concatenate([o["o_full"][0] for o in live]) if live else np.zeros((0, hq, d)),
        o_sparse=np.concatenate([o["o_sparse"][:, 0] for o in live], axis=1) if live
        else np.zeros((L, 0, hq, d)),
        idx=np.concatenate([o["idx"][0] for o in live]) if live else np.zeros((0, width)),
        lse=[None if o is None else o["lse"][0] for o in outs],
        S=[None if o is None else o["S"][0] for o in outs],
        tau=[None if o is None else o["tau"][0] for o in outs])


def kv_bridge(hidden, w_kv, h_kv: int):
    """KV Bridging ("Architectural Innovation: Two-Level KV Sharing" on
    blog.lynxflow.co; "Two-Level KV Sharing" on hitechexpert.top): a
    Cross-Decoder full layer's K and V are linear projections of the hidden
    states of its Self-Decoder full layer, token by token:
    k[b, t] = hidden[b, t] . W_k^T, v[b, t] = hidden[b, t] . W_v^T.
    hidden [B, n, d_model], w_kv [2, h_kv * d, d_model] (W_k, W_v; one row per
    output feature). Returns fp64 (k, v), each [B, n, h_kv, d]."""
    h, w = widen(hidden), widen(w_kv)
    B, n, dm = h.shape
    d = w.shape[1] // h_kv
    flat = h.reshape(B * n, dm)
    k = (flat @ w[0].T).reshape(B, n, h_kv, d)
    v = (flat @ w[1].T).reshape(B, n, h_kv, d)
    return k, v


def pool_rows(page_table, page_size: int, b: int, n: int) -> np.ndarray:
    """Pool rows of positions 0..n-1 of sequence b in a paged KV pool."""
    j = np.arange(n)
    return np.asarray(page_table)[b, j // page_size].astype(np.int64) * page_size + j % page_size


def decode_step_paged(q_full, q_sparse, k_new, v_new, k_pool, v_pool, page_table, page_size,
                      lens, **kw):
    """decode_step with the cache in a paged pool: each sequence's first
    lens[b] rows are read through its page-table row (position j at pool row
    page_table[b, j // page_size] * page_size + j % page_size), then the step
    is decode_step on that prefix. The pool's layout changes nothing else."""
    k_pool, v_pool = np.asarray(k_pool), np.asarray(v_pool)
    B = np.asarray(q_full).shape[0]
    n_max = max(1, max(int(x) for x in lens))
    kc = np.zeros((B, n_max) + k_pool.shape[1:], dtype=k_pool.dtype)
    vc = np.zeros((B, n_max) + v_pool.shape[1:], dtype=v_pool.dtype)
    for b in range(B):
        rows = pool_rows(page_table, page_size, b, int(lens[b]))
        kc[b, :len(rows)] = k_pool[rows]
        vc[b, :len(rows)] = v_pool[rows]
    return decode_step(q_full, q_sparse, k_new, v_new, kc, vc, lens, **kw)


def block_forward_paged(q_full, q_sparse, k_new, v_new, k_pool, v_pool, page_table, page_size,
                        cu_q, lens, **kw):
    """Chunked prefill over a paged pool ("Two-Level KV Sharing": one cache
    serves every layer of the block). Sequence b holds lens[b] tokens, read
    through its page-table row as in decode_step_paged, and appends its new
    tokens, packed rows cu_q[b]..cu_q[b+1] of k_new / v_new; its queries sit
    at positions lens[b] .. lens[b] + n_q(b) - 1. The block is then
    block_forward_varlen over those logical K/V rows. Returns that dict, plus
    the pool rows the new tokens land in ("new_rows", one array per
    sequence)."""
    k_pool, v_pool = np.asarray(k_pool), np.asarray(v_pool)
    k_new, v_new = np.asarray(k_new), np.asarray(v_new)
    ks, vs, cu_kv, new_rows = [], [], [0], []
    for b in range(len(cu_q) - 1):
        n, q0, q1 = int(lens[b]), int(cu_q[b]), int(cu_q[b + 1])
        rows = pool_rows(page_table, page_size, b, n + (q1 - q0))
        ks += [k_pool[rows[:n]], k_new[q0:q1]]
        vs += [v_pool[rows[:n]], v_new[q0:q1]]
        cu_kv.append(cu_kv[-1] + n + (q1 - q0))
        new_rows.append(rows[n:])
    out = block_forward_varlen(q_full, q_sparse, np.concatenate(ks), np.concatenate(vs), cu_q,
                               np.asarray(cu_kv), **kw)
    out["new_rows"] = new_rows
    return out


# ----------------------------------------------------------------------------
# the same definitions, streamed over K/V chunks for a few sampled query rows
# (large contexts: the full score matrix never exists)
# ----------------------------------------------------------------------------
def block_rows(q_full, q_sparse, k, v, b: int, rows, top_k=1024, window=128,
               select="token", block_size=64, top_blocks=16, scale=None,
               chunk=1 << 16):
    """Oracle for selected query indices `rows` of batch entry `b`.

    Two sweeps over K/V in chunks of `chunk` keys: the first accumulates each
    row's per-head LSE with the identity lse(A u B) = logaddexp(lse(A), lse(B));
    the second forms P = exp(s - lse), accumulating O_full and the score row.
    Returns dict of per-row results (o_full [R, h_q, d], lse [R, h_q],
    S [R, n_kv] (0 beyond p), idx [R, W], tau [R], o_sparse [L, R, h_q, d]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    nq, hq, d = q_full.shape[1], q_full.shape[2], q_full.shape[3]
    nkv, hkv = k.shape[1], k.shape[2]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    pos = rows + (nkv - nq)
    R = len(rows)
    Q = widen(q_full[b, rows])                               # [R, hq, d]
    groups = np.array([group_of(h, hq, hkv) for h in range(hq)])
    lse = np.full((R, hq), NEG_INF)
    o_full = np.zeros((R, hq, d))
    S = np.zeros((R, nkv))
    last = int(pos.max()) + 1 if R else 0
    first = int(pos.min()) if R else 0

    def chunk_logits(hs, c0, c1):
        # s_h = scale * Q_h K_g^T for the heads hs of one group over keys
        # c0..c1-1, as one matrix product over (row, head) pairs: [R, G, c];
        # keys past a row's position get -inf (a chunk that lies wholly at or
        # before every row's position needs no mask)
        g = groups[hs[0]]
        s = (Q[:, hs, :].reshape(R * len(hs), d) @ widen(k[b, c0:c1, g]).T) * scale
        s = s.reshape(R, len(hs), c1 - c0)
        if c1 - 1 > first:
            keep = (np.arange(c0, c1)[None, :] <= pos[:, None])[:, None, :]
            s = np.where(keep, s, NEG_INF)
        return s

    def group_rows(g):
        # both sweeps for the heads of KV group g: their LSE, O and their
        # share of the score rows (groups are independent until S is summed)
        hs = np.nonzero(groups == g)[0]
        lse_g = np.full((R, len(hs)), NEG_INF)
        for c0 in range(0, last, chunk):
            s = chunk_logits(hs, c0, min(last, c0 + chunk))
            m = s.max(axis=2)                                       # [R, G]
            ok = np.isfinite(m)
            part = np.full(m.shape, NEG_INF)
            e = np.exp(s - np.where(ok, m, 0.0)[:, :, None])       # exp(-inf) = 0
            part[ok] = m[ok] + np.log(e.sum(axis=2)[ok])
            lse_g = np.logaddexp(lse_g, part)
        o_g = np.zeros((R, len(hs), d))
        S_g = np.zeros((R, last))
        for c0 in range(0, last, chunk):
            c1 = min(last, c0 + chunk)
            p = np.exp(chunk_logits(hs, c0, c1) - lse_g[:, :, None])  # 0 past each row's p
            o_g += (p.reshape(-1, c1 - c0) @ widen(v[b, c0:c1, g])).reshape(R, len(hs), d)
            S_g[:, c0:c1] = p.sum(axis=1)
        return hs, lse_g, o_g, S_g

    # one thread per group, each running single-threaded BLAS
    with threadpool_limits(limits=1, user_api="blas"), \
            ThreadPoolExecutor(max_workers=max(1, min(hkv, os.cpu_count() or 1))) as ex:
        parts = list(ex.map(group_rows, range(hkv)))
    for hs, lse_g, o_g, S_g in parts:                      # fixed group order
        lse[:, hs] = lse_g
        o_full[:, hs] = o_g
        S[:, :last] += S_g
    width = top_k + window if select == "token" else top_blocks * block_size + window
    idx = np.full((R, width), -1, dtype=np.int64)
    tau = np.zeros(R)
    for r in range(R):
        p = int(pos[r])
        if select == "token":
            row = select_token(S[r], p, top_k, window)
            tau[r] = kth_candidate_score(S[r], p, top_k, window)
        else:
            row = select_block(S[r], p, block_size, top_blocks, window)
            tau[r] = kth_block_score(S[r], p, block_size, top_blocks, window)
        idx[r, :len(row)] = row
    L = q_sparse.shape[0]
    o_sparse = np.zeros((L, R, hq, d))
    for r in range(R):
        sel = idx[r][idx[r] >= 0]
        Ks, Vs = widen(k[b, sel]), widen(v[b, sel])
        for l in range(L):
            ql = widen(q_sparse[l, b, rows[r]])
            for h in range(hq):
                g = groups[h]
                s = (Ks[:, g, :] @ ql[h]) * scale
                e = np.exp(s - s.max())
                o_sparse[l, r, h] = (e / e.sum()) @ Vs[:, g, :]
    return dict(o_full=o_full, lse=lse, S=S, idx=idx, tau=tau, o_sparse=o_sparse,
                pos=pos)


def sparse_rows(q_sparse, k, v, b: int, rows, idx_rows, scale=None):
    """Sparse layers for sampled rows over GIVEN index rows [R, W] (-1 pad)."""
    rows = np.asarray(rows, dtype=np.int64)
    L, hq, d = q_sparse.shape[0], q_sparse.shape[3], q_sparse.shape[4]
    hkv = k.shape[2]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((L, len(rows), hq, d))
    for r in range(len(rows)):
        sel = np.asarray(idx_rows[r])
        sel = sel[sel >= 0]
        Ks, Vs = widen(k[b, sel]), widen(v[b, sel])
        for l in range(L):
            ql = widen(q_sparse[l, b, rows[r]])
            for h in range(hq):
                g = group_of(h, hq, hkv)
                s = (Ks[:, g, :] @ ql[h]) * scale
                e = np.exp(s - s.max())
                out[l, r, h] = (e / e.sum()) @ Vs[:, g, :]
    return out


# ----------------------------------------------------------------------------
# step 6: backward pass with the index sets held fixed
# ----------------------------------------------------------------------------
def attention_grads(q, k, v, keep, dout, scale, with_mag=False):
    """Gradients of one softmax-attention head, the textbook way.

    q [n, d], k/v [m, d], keep [n, m] bool (which keys each query sees; every
    query sees at least one), dout [n, d] = dLoss/dO. With s = scale q k^T
    (masked), P = softmax(s) per row and O = P v:
      dv = P^T dout
      dP = dout v^T
      ds = P * (dP - rowsum(P * dP))     (the softmax Jacobian applied to dP)
      dq = scale ds k,   dk = scale ds^T q.
    Returns (dq, dk, dv) in fp64.

    with_mag=True also returns, as a fourth item, the magnitudes of the
    summands behind every gradient element (an error-bound helper for
    comparisons, not part of the method): with Delta = rowsum(P * dP) =
    rowsum(dout * O) and A = rowsum(|dout| * |O|) >= |Delta|, the weight
    W = P * (|dP| + A) bounds |ds| termwise, and
      mag_dq = scale W |k|,  mag_dk = scale W^T |q|,  mag_dv = P^T |dout|,
    so |dq| <= mag_dq, |dk| <= mag_dk, |dv| <= mag_dv elementwise, with
    equality for dv when dout >= 0.
    """
    s = np.where(keep, (q @ k.T) * scale, NEG_INF)
    m = s.max(axis=1, keepdims=True)
    e = np.where(keep, np.exp(s - m), 0.0)
    P = e / e.sum(axis=1, keepdims=True)
    dv = P.T @ dout
    dP = dout @ v.T
    ds = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    grads = (scale * ds @ k, scale * ds.T @ q, dv)
    if not with_mag:
        return grads
    A = (np.abs(dout) * np.abs(P @ v)).sum(axis=1, keepdims=True)
    W = P * (np.abs(dP) + A)
    return grads + ((scale * W @ np.abs(k), scale * W.T @ np.abs(q), P.T @ np.abs(dout)),)


def block_backward(q_full, q_sparse, k, v, idx, do_full, do_sparse, scale=None,
                   with_mag=False):
    """Backward of the whole block for given output gradients, dense.

    q_full / do_full [B, n_q, h_q, d], q_sparse / do_sparse [L, B, n_q, h_q, d],
    k/v [B, n_kv, h_kv, d], idx [B, n_q, W] (-1 padded; the sparse layers'
    index sets, held fixed). Returns dict(dq_full, dq_sparse, dk, dv) in fp64;
    dk and dv sum the full layer's and every sparse layer's contributions.
    with_mag=True adds "mag", a dict of the same four keys holding each
    element's summand magnitude (attention_grads), summed like the gradients.
    """
    qf, kk, vv, dof = widen(q_full), widen(k), widen(v), widen(do_full)
    qs, dos = widen(q_sparse), widen(do_sparse)
    B, nq, hq, d = qf.shape
    nkv, hkv = kk.shape[1], kk.shape[2]
    L = qs.shape[0]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    idx = np.asarray(idx)
    pos = np.arange(nq) + (nkv - nq)
    causal = np.arange(nkv)[None, :] <= pos[:, None]
    out = dict(dq_full=np.zeros_like(qf), dq_sparse=np.zeros_like(qs), dk=np.zeros_like(kk),
               dv=np.zeros_like(vv))
    mag = {n: np.zeros_like(a) for n, a in out.items()}

    def add(dst, res, b, h, g, layer):
        # res = (dq, dk, dv): dq belongs to (layer, b, :, h), dk/dv sum into group g
        if layer is None:
            dst["dq_full"][b, :, h] = res[0]
        else:
            dst["dq_sparse"][layer, b, :, h] = res[0]
        dst["dk"][b, :, g] += res[1]
        dst["dv"][b, :, g] += res[2]

    for b in range(B):
        chosen = np.zeros((nq, nkv), dtype=bool)
        for i in range(nq):
            sel = idx[b, i][idx[b, i] >= 0]
            chosen[i, sel] = True
        for h in range(hq):
            g = group_of(h, hq, hkv)
            passes = [(None, qf[b, :, h], causal, dof[b, :, h])] + \
                [(l, qs[l, b, :, h], chosen, dos[l, b, :, h]) for l in range(L)]
            for layer, qh, keep, doh in passes:
                res = attention_grads(qh, kk[b, :, g], vv[b, :, g], keep, doh, scale, with_mag)
                add(out, res[:3], b, h, g, layer)
                if with_mag:
                    add(mag, res[3], b, h, g, layer)
    if with_mag:
        out["mag"] = mag
    return out


def block_backward_tail(q_full, q_sparse, k, v, idx, do_full, do_sparse, b: int, j_lo: int,
                        scale=None, with_mag=False):
    """block_backward for large contexts, restricted to what a tail of keys
    decides: the K/V gradient rows j >= j_lo and the query gradients of every
    query at position p >= j_lo. Only those queries can reach such a key
    (causality, and index entries never exceed p), so summing their
    contributions alone gives those K/V rows exactly; nothing of size
    n_q x n_kv is formed, only (queries in the tail) x n_kv per KV group.

    Returns dict(rows (query indices i), dq_full [R, h_q, d],
    dq_sparse [L, R, h_q, d], dk, dv [n_kv - j_lo, h_kv, d]); with_mag=True
    adds "mag" with the summand magnitudes of the same elements.
    """
    nq, hq, d = q_full.shape[1], q_full.shape[2], q_full.shape[3]
    nkv, hkv = k.shape[1], k.shape[2]
    L = np.asarray(q_sparse).shape[0]
    G = hq // hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    q_off = nkv - nq
    rows = np.arange(max(0, j_lo - q_off), nq)
    R = len(rows)
    pos = rows + q_off
    causal = np.arange(nkv)[None, :] <= pos[:, None]                 # [R, n_kv]
    idx = np.asarray(idx)
    chosen = np.zeros((R, nkv), dtype=bool)
    for r, i in enumerate(rows):
        sel = idx[b, i][idx[b, i] >= 0]
        chosen[r, sel] = True
    def zeros():
        return dict(dq_full=np.zeros((R, hq, d)), dq_sparse=np.zeros((L, R, hq, d)),
                    dk=np.zeros((nkv - j_lo, hkv, d)), dv=np.zeros((nkv - j_lo, hkv, d)))
    out, mag = zeros(), zeros()

    def add(dst, res, layer, heads, g):
        a, bk, bv = res
        if layer is None:
            dst["dq_full"][:, heads] = a.reshape(R, G, d)
        else:
            dst["dq_sparse"][layer][:, heads] = a.reshape(R, G, d)
        dst["dk"][:, g] += bk[j_lo:]
        dst["dv"][:, g] += bv[j_lo:]

    for g in range(hkv):
        heads = [h for h in range(hq) if group_of(h, hq, hkv) == g]
        Kg, Vg = widen(k[b, :, g]), widen(v[b, :, g])
        # every (query, head of the group) pair is one attention row
        passes = [(None, causal)] + [(l, chosen) for l in range(L)]
        for layer, keep in passes:
            qsrc = q_full[b, rows] if layer is None else np.asarray(q_sparse)[layer, b, rows]
            dsrc = do_full[b, rows] if layer is None else np.asarray(do_sparse)[layer, b, rows]
            Q = widen(qsrc)[:, heads].reshape(R * G, d)
            dO = widen(dsrc)[:, heads].reshape(R * G, d)
            res = attention_grads(Q, Kg, Vg, np.repeat(keep, G, axis=0), dO, scale, with_mag)
            add(out, res[:3], layer, heads, g)
            if with_mag:
                add(mag, res[3], layer, heads, g)
    out["rows"] = rows
    if with_mag:
        out["mag"] = mag
    return out


# ----------------------------------------------------------------------------
# agreement rule for index sets at near-ties
# ----------------------------------------------------------------------------
TIE_REL = 1e-6
TIE_ABS = 2.0 ** -126


def compare_selection(gpu_row, ref_row, S_row, p: int, window: int, tau: float,
                      rel: float = TIE_REL, block_size: int = 0):
    """Compare one GPU index row with the oracle's.

    Both rows are -1 padded. They agree when the window parts are equal, the
    sizes are equal and every index in the symmetric difference is
    tie-eligible: |S(p, j) - tau| <= max(rel * tau, 2^-126). In block mode
    (block_size > 0) the rule is applied to the block scores of the blocks
    that differ. Returns (ok, n_differing, reason).
    """
    g = np.asarray(gpu_row)
    r = np.asarray(ref_row)
    g = g[g >= 0]
    r = r[r >= 0]
    if len(g) != len(r):
        return False, abs(len(g) - len(r)), "size"
    if len(g) and (np.any(np.diff(g) <= 0)):
        return False, 0, "order"
    w = window_of(p, window)
    if not np.array_equal(g[len(g) - len(w):], w):
        return False, 0, "window"
    diff = np.setxor1d(g, r)
    if len(diff) == 0:
        return True, 0, ""
    band = max(rel * tau, TIE_ABS)
    if block_size:
        blocks = np.unique(diff // block_size)
        bs = block_scores(S_row, p, block_size, window)
        ok = bool(np.all(np.abs(bs[blocks] - tau) <= band))
    else:
        ok = bool(np.all(np.abs(np.asarray(S_row, np.float64)[diff] - tau) <= band))
    return ok, len(diff), "" if ok else "beyond-tie"
