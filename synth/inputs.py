"""Seeded input tensors for a workload.

Every tensor is drawn i.i.d. N(0,1) in fp32 from a torch generator seeded by
(workload number, stream id), rounded once to the workload dtype (bf16 with
round-to-nearest-even), and then, where the workload asks for it, given a
planted retrieval structure:

* needles  - K rows at random positions set to a fixed-norm copy of the unit
             direction of a later "target" query, per KV group;
* boost    - a random 1 % of key positions get a common direction added;
* clusters - 32 runs of 32 consecutive keys get that common direction added.

Streams: 0 = full-layer Q, 1 = K, 2 = V, 3 = structure, 10 + l = sparse Q of
layer l, 20/21 = bridging hidden states / weights, 40 = full-layer output
gradient, 41 + l = sparse-layer output gradient of layer l, 60 = random index
sets, 1000 + 16 * step + 0..3 = the new token of decode step `step`. The same bits go to the GPU library and (as a host copy) to the
oracle. Nothing here computes attention, scores or selections.
"""
import math

import numpy as np
import torch

from .configs import Workload

_CHUNK_ELEMS = 1 << 25     # draw in bounded pieces so fp32 temporaries stay small


def _seed(cid: int, stream: int) -> int:
    return 0x5EED_0000 + 1_000_003 * cid + stream


def _torch_dtype(w: Workload):
    return torch.float32 if w.dtype == "fp32" else torch.bfloat16


def _randn(shape, w: Workload, stream: int, device) -> torch.Tensor:
    """N(0,1) draws of `shape`, rounded to the workload dtype, chunked."""
    g = torch.Generator(device=device)
    g.manual_seed(_seed(w.cid, stream))
    out = torch.empty(shape, dtype=_torch_dtype(w), device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK_ELEMS):
        e = min(n, s + _CHUNK_ELEMS)
        flat[s:e] = torch.randn(e - s, generator=g, device=device,
                                dtype=torch.float32).to(out.dtype)
    return out


def _unit_direction(rng: np.random.Generator, d: int) -> np.ndarray:
    u = rng.standard_normal(d)
    return (u / np.linalg.norm(u)).astype(np.float32)


def make_inputs(w: Workload, device="cpu", sparse_layers=None) -> dict:
    """Build all inputs of workload `w` on `device`.

    Returns a dict with torch tensors
      q_full   [B, n_q, h_q, d]
      k, v     [B, n_kv, h_kv, d]
      q_sparse [L, B, n_q, h_q, d]
    and `meta`, a dict describing the planted structure.
    `sparse_layers` optionally overrides the number of sparse layers drawn.
    """
    B, nq, nkv, hq, hkv, d = w.batch, w.n_q, w.n_kv, w.h_q, w.h_kv, w.d
    L = w.n_sparse if sparse_layers is None else sparse_layers
    q_full = _randn((B, nq, hq, d), w, 0, device)
    k = _randn((B, nkv, hkv, d), w, 1, device)
    v = _randn((B, nkv, hkv, d), w, 2, device)
    q_sparse = torch.empty((L, B, nq, hq, d), dtype=q_full.dtype, device=device)
    for layer in range(L):
        q_sparse[layer] = _randn((B, nq, hq, d), w, 10 + layer, device)
    meta = {"structure": w.structure}
    rng = np.random.default_rng([w.cid, 3])
    G = hq // hkv
    if w.structure == "needles":
        n_needles = int(w.extra["n_needles"])
        norm = float(w.extra["needle_norm"])
        # needle positions in [0, n_kv - window) and a target query position at
        # least one window later; targets must lie inside the query chunk
        pos = np.sort(rng.choice(nkv - w.window, size=n_needles, replace=False))
        lo = np.maximum(pos + w.window, w.q_off)
        tgt = rng.integers(lo, nkv)
        for b in range(B):
            for j, p in zip(pos.tolist(), tgt.tolist()):
                for g in range(hkv):
                    qv = q_full[b, p - w.q_off, g * G].float()
                    k[b, j, g] = (norm * qv / qv.norm()).to(k.dtype)
        meta.update(needle_pos=pos, needle_target=tgt)
    elif w.structure == "boost":
        u = torch.from_numpy(_unit_direction(rng, d)).to(device)
        n_boost = int(round(w.extra["boost_frac"] * nkv))
        shift = float(w.extra["boost_scale"]) * math.sqrt(d) * u
        positions = []
        for b in range(B):
            pos = np.sort(rng.choice(nkv, size=n_boost, replace=False))
            idx = torch.from_numpy(pos).to(device)
            k[b, idx] = (k[b, idx].float() + shift).to(k.dtype)
            positions.append(pos)
        meta.update(boost_pos=positions, direction=u.cpu().numpy())
    elif w.structure == "clusters":
        u = torch.from_numpy(_unit_direction(rng, d)).to(device)
        nc, cl = int(w.extra["n_clusters"]), int(w.extra["cluster_len"])
        shift = float(w.extra["boost_scale"]) * math.sqrt(d) * u
        span = w.q_off - w.window - cl + 1          # admissible start offsets
        seg = span // nc
        starts = np.array([c * seg + int(rng.integers(0, seg - cl + 1))
                           for c in range(nc)])
        pos = (starts[:, None] + np.arange(cl)[None, :]).reshape(-1)
        for b in range(B):
            idx = torch.from_numpy(pos).to(device)
            k[b, idx] = (k[b, idx].float() + shift).to(k.dtype)
        meta.update(cluster_start=starts, cluster_pos=pos,
                    direction=u.cpu().numpy())
    return {"q_full": q_full, "k": k, "v": v, "q_sparse": q_sparse, "meta": meta}


def decode_step_inputs(w: Workload, step: int, device="cpu", sparse_layers=None) -> dict:
    """The new token's tensors for decode step `step` of workload `w`.

    Returns q_full [B, 1, h_q, d], q_sparse [L, B, 1, h_q, d] and the new
    cache rows k_new, v_new [B, 1, h_kv, d]; streams 1000 + 16 * step + 0..3,
    so every step draws fresh, reproducible values.
    """
    B, hq, hkv, d = w.batch, w.h_q, w.h_kv, w.d
    L = w.n_sparse if sparse_layers is None else sparse_layers
    base = 1000 + 16 * step
    return dict(q_full=_randn((B, 1, hq, d), w, base, device),
                q_sparse=_randn((L, B, 1, hq, d), w, base + 1, device),
                k_new=_randn((B, 1, hkv, d), w, base + 2, device),
                v_new=_randn((B, 1, hkv, d), w, base + 3, device))


def bridge_inputs(w: Workload, d_model: int, device="cpu") -> dict:
    """Hidden states [B, n_kv, d_model] (N(0,1)) and bridging weights
    [2, h_kv * d, d_model] (N(0, 1/d_model), so projections come out near
    unit scale) for the KV Bridging projection; streams 20 and 21."""
    B, n, F = w.batch, w.n_kv, w.h_kv * w.d
    hidden = _randn((B, n, d_model), w, 20, device)
    g = torch.Generator(device=device)
    g.manual_seed(_seed(w.cid, 21))
    wk = torch.empty((2, F, d_model), dtype=_torch_dtype(w), device=device)
    flat = wk.view(-1)
    for s in range(0, flat.numel(), _CHUNK_ELEMS):
        e = min(flat.numel(), s + _CHUNK_ELEMS)
        flat[s:e] = (torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
                     * d_model ** -0.5).to(wk.dtype)
    return dict(hidden=hidden, w_kv=wk)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor: float32 values for fp32, raw uint16 bits for bf16."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def grad_inputs(w: Workload, device="cpu", sparse_layers=None) -> dict:
    """Output gradients for the backward pass: do_full [B, n_q, h_q, d]
    (stream 40) and do_sparse [L, B, n_q, h_q, d] (streams 41 + l), N(0,1)."""
    B, nq, hq, d = w.batch, w.n_q, w.h_q, w.d
    L = w.n_sparse if sparse_layers is None else sparse_layers
    do_full = _randn((B, nq, hq, d), w, 40, device)
    do_sparse = torch.empty((L, B, nq, hq, d), dtype=do_full.dtype, device=device)
    for layer in range(L):
        do_sparse[layer] = _randn((B, nq, hq, d), w, 41 + layer, device)
    return {"do_full": do_full, "do_sparse": do_sparse}


def random_index_rows(w: Workload, device="cpu", rows_per_chunk=4096) -> torch.Tensor:
    """Valid index sets drawn at random (stream 60), to drive the backward
    pass independently of any selection: for query i at position
    p = q_off + i, the window max(0, p - window + 1) .. p plus min(top_k, C)
    of the C = p - window + 1 candidates 0 .. p - window, one drawn uniformly
    from each of min(top_k, C) consecutive, disjoint integer ranges that tile
    0 .. C - 1 (so the picks are distinct and ascending). Rows are
    ascending and -1 padded to top_k + window; int32 [B, n_q, top_k + window].
    """
    B, nq, k, win = w.batch, w.n_q, w.top_k, w.window
    width = k + win
    g = torch.Generator(device=device)
    g.manual_seed(_seed(w.cid, 60))
    out = torch.full((B, nq, width), -1, dtype=torch.int32, device=device)
    t = torch.arange(k, device=device, dtype=torch.int64)
    wj = torch.arange(win, device=device, dtype=torch.int64)
    for b in range(B):
        for i0 in range(0, nq, rows_per_chunk):
            i1 = min(nq, i0 + rows_per_chunk)
            p = torch.arange(i0, i1, device=device, dtype=torch.int64) + (w.n_kv - nq)
            C = torch.clamp(p - win + 1, min=0)                        # candidates
            n_pick = torch.clamp(C, max=k)
            lo = (t[None, :] * C[:, None]) // k                        # range t starts
            hi = ((t[None, :] + 1) * C[:, None]) // k                  # and ends
            u = torch.rand((i1 - i0, k), generator=g, device=device, dtype=torch.float64)
            pick = lo + torch.minimum((u * (hi - lo)).to(torch.int64), hi - lo - 1)
            # fewer candidates than top_k: take them all
            pick = torch.where((C < k)[:, None], t[None, :], pick)
            valid = t[None, :] < n_pick[:, None]
            wpos = torch.clamp(p - win + 1, min=0)[:, None] + wj[None, :]
            wvalid = wpos <= p[:, None]
            # candidates first (ascending), then the window (also ascending and
            # above every candidate); valid entries are packed to the front
            vals = torch.cat([torch.where(valid, pick, -1), torch.where(wvalid, wpos, -1)], 1)
            order = torch.argsort((vals < 0).to(torch.int8), dim=1, stable=True)
            rows = torch.gather(vals, 1, order)
            out[b, i0:i1] = rows.to(torch.int32)
    return out
