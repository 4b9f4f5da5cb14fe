"""C-ABI checks that need no GPU: the library loads, exports every declared
entry point, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

from token_level_sparse_pass_amd import hs2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hs2.h")

if not os.path.exists(hs2.LIB_PATH):
    pytest.skip("libhs2.so not built", allow_module_level=True)

FAKE = 0x10000          # aligned, non-null: never dereferenced by failing calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hs2_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = hs2.load()
    names = declared_functions()
    assert {"hs2_full_attn_select", "hs2_sparse_attn", "hs2_block_forward",
            "hs2_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    lib = hs2.load()
    assert lib.hs2_abi_version() == hs2.ABI_VERSION
    for s, text in hs2.STATUS.items():
        assert lib.hs2_status_string(s).decode() == text


def base_problem(**kw):
    args = dict(dtype=hs2.BF16, batch=1, n_q=256, n_kv=1024, h_q=8, h_kv=2, head_dim=128,
                top_k=64, window=16)
    args.update(kw)
    return hs2.problem(**args)


def full_call(p, q=FAKE, k=FAKE, v=FAKE, o=FAKE, idx=FAKE, lse=None, ws=FAKE, ws_bytes=None):
    lib = hs2.load()
    if ws_bytes is None:
        ws_bytes = hs2.workspace_size(p)[1]
    vp = ctypes.c_void_p
    return lib.hs2_full_attn_select(ctypes.byref(p), vp(q), vp(k), vp(v), vp(o), vp(idx),
                                    vp(lse), None, vp(ws), ws_bytes, None)


def test_index_width():
    assert hs2.index_width(base_problem()) == 64 + 16
    assert hs2.index_width(base_problem(select="block", block_size=8, top_blocks=4)) == 32 + 16
    assert hs2.index_width(base_problem(top_k=1024, window=128)) == 1152


def test_workspace_sizes():
    p = base_problem()
    mn, pref = hs2.workspace_size(p)
    stats = 3 * 1 * 8 * 256 * 4                   # m2, l, 1/l per (query, head)
    row = (1024 - 16 + 255) // 256 * 256 * 4
    vt = 1 * 2 * 128 * 1024 * 2                     # transposed V (bf16, d = 128)
    assert mn >= stats + row + vt
    assert pref >= mn
    assert pref >= stats + 256 * row         # one chunk holds every query row
    # decode needs its logits and partials
    d = base_problem(n_q=1, batch=4)
    mn_d, pref_d = hs2.workspace_size(d)
    assert mn_d == pref_d and mn_d >= 4 * 8 * 1024 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 3), (dict(h_q=6, h_kv=4), 2), (dict(n_q=2048), 2),
    (dict(batch=0), 2), (dict(window=0), 2), (dict(top_k=5000), 3),
    (dict(select="block", top_blocks=300), 3), (dict(dtype=7), 3),
    (dict(softmax_scale=0.0), 2), (dict(h_q=128, h_kv=1), 3),
])
def test_problem_rejected(kw, status):
    p = base_problem(**kw)
    assert full_call(p, ws_bytes=1 << 30) == status
    assert hs2.load().hs2_last_error().decode() != ""


def test_abi_version_mismatch():
    p = base_problem()
    p.abi_version = 99
    assert full_call(p, ws_bytes=1 << 30) == 3


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "idx", "ws"])
def test_null_pointers(name):
    p = base_problem()
    assert full_call(p, **{name: None}) == 1


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "idx", "ws", "lse"])
def test_misaligned_pointers(name):
    p = base_problem()
    assert full_call(p, **{name: FAKE + 4}) == 5


def test_workspace_too_small():
    p = base_problem()
    mn, _ = hs2.workspace_size(p)
    assert full_call(p, ws_bytes=mn - 1) == 4
    assert "workspace" in hs2.load().hs2_last_error().decode()


def test_sparse_rejections():
    lib = hs2.load()
    p = base_problem()
    vp = ctypes.c_void_p
    assert lib.hs2_sparse_attn(ctypes.byref(p), -1, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                               vp(FAKE), None) == 2
    assert lib.hs2_sparse_attn(ctypes.byref(p), 2, None, vp(FAKE), vp(FAKE), vp(FAKE),
                               vp(FAKE), None) == 1
    assert lib.hs2_sparse_attn(ctypes.byref(p), 2, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE + 8),
                               vp(FAKE), None) == 5
    # zero layers is a valid no-op that touches nothing
    assert lib.hs2_sparse_attn(ctypes.byref(p), 0, None, None, None, None, None, None) == 0


def test_block_forward_rejections():
    lib = hs2.load()
    p = base_problem()
    vp = ctypes.c_void_p
    mn, _ = hs2.workspace_size(p)
    args = [vp(FAKE)] * 8
    assert lib.hs2_block_forward(ctypes.byref(p), 3, *args[:6], vp(FAKE), None, vp(FAKE),
                                 mn - 16, None) == 4
    assert lib.hs2_block_forward(None, 3, *args[:6], vp(FAKE), None, vp(FAKE), mn, None) == 1


def test_debug_rows_validated():
    lib = hs2.load()
    p = base_problem()
    rows = (ctypes.c_int32 * 1)(256)             # out of range: batch * n_q = 256
    dbg = hs2.Debug(rows, 1, FAKE)
    vp = ctypes.c_void_p
    st = lib.hs2_full_attn_select(ctypes.byref(p), *([vp(FAKE)] * 5), None, ctypes.byref(dbg),
                                  vp(FAKE), hs2.workspace_size(p)[1], None)
    assert st == 2


def decode_call(p, lens, n_layers=2, ptrs=None, ws_bytes=None):
    lib = hs2.load()
    vp = ctypes.c_void_p
    P = dict(q=FAKE, qs=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, o=FAKE, os=FAKE, idx=FAKE,
             ws=FAKE)
    P.update(ptrs or {})
    if ws_bytes is None:
        ws_bytes = hs2.workspace_size(p)[1]
    arr = None if lens is None else (ctypes.c_int32 * len(lens))(*lens)
    return lib.hs2_decode_step(ctypes.byref(p), n_layers, vp(P["q"]), vp(P["qs"]), vp(P["kn"]),
                               vp(P["vn"]), vp(P["kc"]), vp(P["vc"]), arr, vp(P["o"]),
                               vp(P["os"]), vp(P["idx"]), None, vp(P["ws"]), ws_bytes, None)


def test_decode_step_rejections():
    p = base_problem(n_q=1, batch=3, n_kv=4096)
    assert decode_call(base_problem(), [1]) == 2                   # n_q != 1
    assert decode_call(p, None) == 1                               # no lengths
    assert decode_call(p, [10, 4096, 3]) == 2                      # no room left
    assert "no room" in hs2.load().hs2_last_error().decode()
    assert decode_call(p, [10, -1, 3]) == 2
    assert decode_call(p, [10, 20, 3], ptrs=dict(kn=None)) == 1
    assert decode_call(p, [10, 20, 3], ptrs=dict(vc=FAKE + 4)) == 5
    mn, _ = hs2.workspace_size(p)
    assert decode_call(p, [10, 20, 3], ws_bytes=mn - 1) == 4


def test_decode_step_paged_rejections():
    lib = hs2.load()
    vp = ctypes.c_void_p

    def call(p, pages, lens=(10, 20, 3)):
        arr = (ctypes.c_int32 * len(lens))(*lens)
        return lib.hs2_decode_step_paged(ctypes.byref(p), None if pages is None else
                                         ctypes.byref(pages), 2, *([vp(FAKE)] * 6), arr,
                                         *([vp(FAKE)] * 3), None, vp(FAKE),
                                         hs2.workspace_size(p)[1], None)
    p = base_problem(n_q=1, batch=3, n_kv=64 * 50)
    assert call(p, None) == 1
    assert call(p, hs2.KvPages(None, 64, 50, 200)) == 1            # no table
    assert call(p, hs2.KvPages(FAKE, 48, 50, 200)) == 2            # not a power of two
    assert call(p, hs2.KvPages(FAKE, 16, 200, 200)) == 2           # pages below 32 rows
    assert call(p, hs2.KvPages(FAKE, 64, 40, 200)) == 2            # n_kv != max_pages * page_size
    assert "max_pages" in lib.hs2_last_error().decode()
    assert call(p, hs2.KvPages(FAKE, 64, 50, 0)) == 2              # empty pool
    assert call(p, hs2.KvPages(FAKE, 64, 50, 200), lens=(10, 3200, 3)) == 2


def test_kv_bridge_rejections():
    lib = hs2.load()
    vp = ctypes.c_void_p
    p = base_problem(n_kv=1000)
    args = [vp(FAKE)] * 4
    assert lib.hs2_kv_bridge(ctypes.byref(base_problem(dtype=hs2.FP32)), 256, *args, None) == 3
    assert lib.hs2_kv_bridge(ctypes.byref(p), 100, *args, None) == 2       # not a multiple of 64
    assert lib.hs2_kv_bridge(ctypes.byref(p), 0, *args, None) == 2
    assert lib.hs2_kv_bridge(ctypes.byref(p), 256, None, *args[1:], None) == 1
    assert lib.hs2_kv_bridge(ctypes.byref(p), 256, vp(FAKE), vp(FAKE), vp(FAKE + 2), vp(FAKE),
                             None) == 5


def test_backward_workspace_and_rejections():
    lib = hs2.load()
    vp = ctypes.c_void_p
    p = base_problem()
    # Delta rows; for bf16 at head dim 128 a K^T copy and the Q / dO rows in
    # transposed 64-row tiles with their statistics; then, when there are
    # sparse layers, two K/V accumulators sized for 64-bit fixed point (the
    # deterministic entry point; the default one uses their first half as
    # fp32) and a 256-byte block for their bounds and scales
    delta = 1 * 8 * 256 * 4
    tiles = 2 * (256 * 4 // 64)                      # KV heads x 64-row tiles
    kt = 1 * 2 * 1024 * 128 * 2 + 2 * tiles * 64 * 128 * 2 + tiles * 128 * 4
    acc = 1 * 1024 * 2 * 128 * 8
    assert hs2.backward_workspace_size(p, 0) == delta + kt
    assert hs2.backward_workspace_size(p, 3) == delta + kt + 2 * acc + 256
    # the K^T copy serves only the bf16, head-dim-128 dQ kernel
    assert hs2.backward_workspace_size(base_problem(head_dim=64), 0) == 1 * 8 * 256 * 4
    assert hs2.backward_workspace_size(base_problem(dtype=hs2.FP32), 0) == delta
    ws = hs2.backward_workspace_size(p, 2)

    # both entry points validate alike (the deterministic one shares the code)
    for fn in (lib.hs2_block_backward, lib.hs2_block_backward_deterministic):
        def call(L=2, ws_bytes=ws, **over):
            names = ["q_full", "q_sparse", "k", "v", "o_full", "o_sparse", "lse", "idx",
                     "do_full", "do_sparse", "dq_full", "dq_sparse", "dk", "dv", "ws"]
            a = {n: FAKE for n in names}
            a.update(over)
            ptrs = [vp(a[n]) for n in names]
            return fn(ctypes.byref(p), L, *ptrs[:-1], ptrs[-1], ws_bytes, None)

        assert call(L=-1) == 2
        for n in ("q_full", "k", "v", "o_full", "lse", "do_full", "dq_full", "dk", "dv", "ws"):
            assert call(**{n: None}) == 1, n
            assert call(**{n: FAKE + 4}) == 5, n
        for n in ("q_sparse", "o_sparse", "idx", "do_sparse", "dq_sparse"):
            assert call(**{n: None}) == 1, n
        assert call(ws_bytes=ws - 1) == 4
        assert b"workspace" in lib.hs2_last_error()
    bad = base_problem(h_q=6, h_kv=4)
    assert lib.hs2_backward_workspace_size(ctypes.byref(bad), 1, ctypes.byref(ctypes.c_size_t())) == 2


def test_varlen_checks_and_workspace():
    lib = hs2.load()
    vp = ctypes.c_void_p
    p = base_problem(batch=3)
    cq = (ctypes.c_int32 * 4)(0, 100, 101, 301)
    ck = (ctypes.c_int32 * 4)(0, 500, 1500, 1700)
    mn, pref = hs2.workspace_size_varlen(p, cq, ck)
    # bf16 / head_dim 128: the prefill-shaped sequences (100 x 500, 200 x 200)
    # share one full-attention launch, so their statistics (3 x h_q floats per
    # query), transposed V copies (h_kv x 64-key tiles x 128 x 2 B) and a score
    # chunk (rows of the longest score row) coexist; the one-query sequence
    # (decode path) reuses the same bytes afterwards
    up = lambda x: (x + 255) // 256 * 256
    fixed = up(3 * 8 * 301 * 4) + up(2 * (8 + 4) * 64 * 128 * 2)
    row = (500 - 16 + 255) // 256 * 256 * 4
    dec = hs2.workspace_size(base_problem(batch=1, n_q=1, n_kv=1000))
    assert mn == max(fixed + up(row), dec[0])
    assert pref == max(fixed + up(256 * row), dec[1])      # rows: 200 rounded up to 128s
    # other dtypes run sequence by sequence: the largest single need
    p32 = base_problem(batch=3, dtype=hs2.FP32)
    mn32, pref32 = hs2.workspace_size_varlen(p32, cq, ck)
    want = [hs2.workspace_size(base_problem(batch=1, n_q=a, n_kv=b, dtype=hs2.FP32))
            for a, b in ((100, 500), (1, 1000), (200, 200))]
    assert mn32 == max(w[0] for w in want) and pref32 == max(w[1] for w in want)

    def call(cq, ck, ws_bytes=pref, **over):
        a = dict(q_full=FAKE, q_sparse=FAKE, k=FAKE, v=FAKE, o_full=FAKE, o_sparse=FAKE,
                 idx=FAKE, lse=None, ws=FAKE)
        a.update(over)
        arr = lambda x: (ctypes.c_int32 * len(x))(*x)
        return lib.hs2_block_forward_varlen(
            ctypes.byref(p), 2, arr(cq), arr(ck), vp(a["q_full"]), vp(a["q_sparse"]), vp(a["k"]),
            vp(a["v"]), vp(a["o_full"]), vp(a["o_sparse"]), vp(a["idx"]), vp(a["lse"]),
            vp(a["ws"]), ws_bytes, None)

    ok_q, ok_k = [0, 100, 101, 301], [0, 500, 1500, 1700]
    assert call([1, 100, 101, 301], ok_k) == 2                  # must start at 0
    assert call([0, 100, 99, 301], ok_k) == 2                   # decreasing
    assert call([0, 600, 601, 801], ok_k) == 2                  # more queries than keys
    assert call(ok_q, ok_k, ws_bytes=mn - 1) == 4
    assert call(ok_q, ok_k, q_full=None) == 1
    assert call(ok_q, ok_k, k=FAKE + 8) == 5
    assert lib.hs2_block_forward_varlen(ctypes.byref(p), 2, None, None, *[vp(FAKE)] * 9,
                                        pref, None) == 1
    # a one-query sequence takes the decode path, which caps h_q / h_kv at 32
    wide = base_problem(batch=1, h_q=64, h_kv=1)
    one = (ctypes.c_int32 * 2)(0, 1)
    keys = (ctypes.c_int32 * 2)(0, 300)
    assert lib.hs2_workspace_size_varlen(ctypes.byref(wide), one, keys,
                                         ctypes.byref(ctypes.c_size_t()), None) == 3


def test_paged_prefill_workspace_and_rejections():
    lib = hs2.load()
    vp = ctypes.c_void_p
    ps, mp = 64, 50
    p = base_problem(batch=3, n_kv=ps * mp)
    pages = hs2.KvPages(FAKE, ps, mp, 200)
    cu_q, lens = [0, 100, 101, 301], [400, 999, 0]
    mn, pref = hs2.workspace_size_paged(p, pages, cu_q, lens)
    # two staging buffers hold the rows of the sequences with two or more new
    # tokens (500 + 200 rows of 2 * 128 bf16), then the variable-length
    # batch of the logical lengths (n_kv(b) = lens[b] + n_q(b))
    up = lambda x: (x + 255) // 256 * 256
    stage = up((500 + 200) * 2 * 128 * 2)
    vmn, vpref = hs2.workspace_size_varlen(p, cu_q, [0, 500, 1500, 1700])
    assert (mn, pref) == (2 * stage + vmn, 2 * stage + vpref)
    # one-token sequences are not staged
    mn1, _ = hs2.workspace_size_paged(p, pages, [0, 1, 2, 3], lens)
    assert mn1 == hs2.workspace_size_varlen(p, [0, 1, 2, 3], [0, 401, 1401, 1402])[0]

    def call(cq=cu_q, ln=lens, pg=pages, ws_bytes=pref, **over):
        a = dict(q_full=FAKE, q_sparse=FAKE, k_new=FAKE, v_new=FAKE, k_pool=FAKE, v_pool=FAKE,
                 o_full=FAKE, o_sparse=FAKE, idx=FAKE, lse=None, ws=FAKE)
        a.update(over)
        arr = lambda x: None if x is None else (ctypes.c_int32 * len(x))(*x)
        return lib.hs2_block_forward_paged(
            ctypes.byref(p), None if pg is None else ctypes.byref(pg), 2, arr(cq), arr(ln),
            *[vp(a[n]) for n in ("q_full", "q_sparse", "k_new", "v_new", "k_pool", "v_pool",
                                 "o_full", "o_sparse", "idx", "lse", "ws")], ws_bytes, None)

    assert call(pg=None) == 1
    assert call(pg=hs2.KvPages(FAKE, 48, mp, 200)) == 2           # page size
    assert call(pg=hs2.KvPages(FAKE, ps, mp - 1, 200)) == 2       # capacity != n_kv
    assert call(cq=None) == 1 and call(ln=None) == 1
    assert call(cq=[1, 100, 101, 301]) == 2                       # must start at 0
    assert call(cq=[0, 100, 99, 301]) == 2                        # decreasing
    assert call(ln=[3150, 999, 0]) == 2                           # 3150 + 100 > 3200
    assert "capacity" in lib.hs2_last_error().decode()
    assert call(ln=[-1, 999, 0]) == 2
    assert call(ws_bytes=mn - 1) == 4
    assert call(k_new=None) == 1 and call(v_pool=None) == 1
    assert call(idx=FAKE + 4) == 5
    assert call(ws=FAKE + 8) == 5


def test_paged_prefill_without_new_tokens_launches_nothing():
    # a batch where no sequence appends anything is a no-op: OK without a
    # workspace, before any device work
    lib = hs2.load()
    vp = ctypes.c_void_p
    p = base_problem(batch=2, n_kv=64 * 10)
    pages = hs2.KvPages(FAKE, 64, 10, 20)
    cu_q = (ctypes.c_int32 * 3)(0, 0, 0)
    lens = (ctypes.c_int32 * 2)(100, 0)
    assert hs2.workspace_size_paged(p, pages, [0, 0, 0], [100, 0]) == (0, 0)
    st = lib.hs2_block_forward_paged(ctypes.byref(p), ctypes.byref(pages), 2, cu_q, lens,
                                     *[vp(FAKE)] * 9, None, None, 0, None)
    assert st == 0, lib.hs2_last_error().decode()


# --------------------------------------------------------------------------
# the Python binding checks every tensor's shape before any device call (the
# C ABI sees raw pointers only); CPU tensors reach these checks, then fail as
# non-device tensors, so nothing here touches a GPU
# --------------------------------------------------------------------------
def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def _shape_error(fn, *args, match="shape", **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def test_binding_rejects_mis_shaped_block_forward():
    import torch
    B, nq, nkv, hq, hkv, d, L = 1, 8, 32, 4, 2, 64, 2
    q, qs = _t(B, nq, hq, d), _t(L, B, nq, hq, d)
    k, v = _t(B, nkv, hkv, d), _t(B, nkv, hkv, d)
    kw = dict(top_k=4, window=4)
    _shape_error(hs2.block_forward, q, _t(L, B, nq, hq + 1, d), k, v, **kw)     # q_sparse heads
    _shape_error(hs2.block_forward, q, _t(L, B, nq - 1, hq, d), k, v, **kw)     # q_sparse rows
    _shape_error(hs2.block_forward, q, qs, k, _t(B, nkv - 1, hkv, d), **kw)     # v != k
    _shape_error(hs2.block_forward, q, qs, _t(B, nkv, hkv, d // 2), v, **kw)    # head dim
    out = dict(o_full=_t(B, nq, hq, d), o_sparse=_t(L, B, nq, hq, d),
               idx=torch.zeros((B, nq, 7), dtype=torch.int32), lse=None)
    _shape_error(hs2.block_forward, q, qs, k, v, out=out, **kw)                 # idx width
    out["idx"] = torch.zeros((B, nq, 8), dtype=torch.int64)
    _shape_error(hs2.block_forward, q, qs, k, v, out=out, match="int32", **kw)  # idx dtype
    # every shape right: the next check is the device
    _shape_error(hs2.block_forward, q, qs, k, v, match="device tensor", **kw)


def test_binding_rejects_mis_shaped_sparse_and_full_calls():
    import torch
    B, nq, nkv, hq, hkv, d, L = 2, 8, 32, 4, 2, 64, 3
    qs, k, v = _t(L, B, nq, hq, d), _t(B, nkv, hkv, d), _t(B, nkv, hkv, d)
    kw = dict(top_k=4, window=4)
    idx = torch.zeros((B, nq, 8), dtype=torch.int32)
    _shape_error(hs2.sparse_attn, qs, k, v, torch.zeros((B, nq - 1, 8), dtype=torch.int32), **kw)
    _shape_error(hs2.sparse_attn, qs, k, v, torch.zeros((1, nq, 8), dtype=torch.int32), **kw)
    _shape_error(hs2.sparse_attn, qs, _t(B + 1, nkv, hkv, d), v, idx, **kw)
    _shape_error(hs2.sparse_attn, qs, k, v, idx, match="device tensor", **kw)
    _shape_error(hs2.full_attn_select, _t(B, nq, hq, d), k, _t(B, nkv, hkv + 1, d), **kw)
    _shape_error(hs2.full_attn_select, _t(B, nq, hq, d), _t(B, nkv, hkv, d + 1), v, **kw)


def test_binding_rejects_mis_shaped_decode_and_bridge_calls():
    import torch
    B, cap, hq, hkv, d, L = 2, 64, 4, 2, 64, 2
    q, qs = _t(B, 1, hq, d), _t(L, B, 1, hq, d)
    kn, vn = _t(B, 1, hkv, d), _t(B, 1, hkv, d)
    kc, vc = _t(B, cap, hkv, d), _t(B, cap, hkv, d)
    kw = dict(top_k=4, window=4)
    _shape_error(hs2.decode_step, q, qs, kn, _t(B, 2, hkv, d), kc, vc, [3, 4], **kw)
    _shape_error(hs2.decode_step, q, qs, kn, vn, kc, _t(B, cap, hkv, d + 8), [3, 4], **kw)
    _shape_error(hs2.decode_step, q, qs, kn, vn, kc, vc, [3], match="lens", **kw)
    pool = _t(4 * 32, hkv, d)
    table = torch.zeros((B, 2), dtype=torch.int32)
    _shape_error(hs2.decode_step_paged, q, qs, kn, vn, pool, _t(4 * 32, hkv, d // 2), table, 32,
                 [3, 4], **kw)
    _shape_error(hs2.decode_step_paged, q, qs, kn, vn, pool, pool.clone(),
                 torch.zeros((B + 1, 2), dtype=torch.int32), 32, [3, 4], **kw)
    _shape_error(hs2.kv_bridge, _t(1, 16, 256), _t(2, 128, 255), 2)
    _shape_error(hs2.kv_bridge, _t(1, 16, 256), _t(3, 128, 256), 2)
    _shape_error(hs2.kv_bridge, _t(1, 16, 256), _t(2, 128, 256), 3, match="multiple")


def test_binding_rejects_mis_shaped_packed_and_backward_calls():
    import torch
    hq, hkv, d, L = 4, 2, 64, 2
    q, qs = _t(10, hq, d), _t(L, 10, hq, d)
    k, v = _t(40, hkv, d), _t(40, hkv, d)
    kw = dict(top_k=4, window=4)
    _shape_error(hs2.block_forward_varlen, q, qs, k, _t(41, hkv, d), [0, 4, 10], [0, 20, 40],
                 **kw)
    _shape_error(hs2.block_forward_varlen, q, _t(L, 10, hq + 2, d), k, v, [0, 4, 10],
                 [0, 20, 40], **kw)
    _shape_error(hs2.block_forward_varlen, q, qs, k, v, [0, 4, 10], [0, 40], match="cu_seqlens",
                 **kw)
    pool = _t(4 * 32, hkv, d)
    table = torch.zeros((2, 4), dtype=torch.int32)
    _shape_error(hs2.block_forward_paged, q, qs, _t(10, hkv, d), _t(9, hkv, d), pool, pool.clone(),
                 table, 32, [0, 4, 10], [5, 6], **kw)
    B, nq, nkv = 1, 8, 32
    qf, kk, vv = _t(B, nq, hq, d), _t(B, nkv, hkv, d), _t(B, nkv, hkv, d)
    qsp = _t(L, B, nq, hq, d)
    lse = torch.zeros((B, hq, nq), dtype=torch.float32)
    idx = torch.zeros((B, nq, 8), dtype=torch.int32)
    args = [qf, qsp, kk, vv, qf.clone(), qsp.clone(), lse, idx, qf.clone(), qsp.clone()]
    bad = list(args)
    bad[6] = torch.zeros((B, hq, nq + 1), dtype=torch.float32)            # lse
    _shape_error(hs2.block_backward, *bad, **kw)
    bad = list(args)
    bad[9] = _t(L + 1, B, nq, hq, d)                                     # do_sparse
    _shape_error(hs2.block_backward, *bad, **kw)
    _shape_error(hs2.block_backward, *args, match="device tensor", **kw)


def test_static_workspace_entry_point_rejects_on_the_host():
    lib = hs2.load()
    vp = ctypes.c_void_p

    def call(p, ptrs=None):
        a = dict(q=FAKE, qs=FAKE, k=FAKE, v=FAKE, o=FAKE, os=FAKE, idx=FAKE, lse=None)
        a.update(ptrs or {})
        return lib.hs2_block_forward_static(ctypes.byref(p), 2, vp(a["q"]), vp(a["qs"]),
                                            vp(a["k"]), vp(a["v"]), vp(a["o"]), vp(a["os"]),
                                            vp(a["idx"]), vp(a["lse"]), None)
    # the 1M-token context needs far more than the static workspace's 64 MiB
    big = base_problem(n_q=16384, n_kv=1048576, h_q=64, h_kv=8, top_k=1024, window=128)
    assert hs2.workspace_size(big)[0] > hs2.STATIC_WORKSPACE_BYTES
    assert call(big) == 4                                      # HS2_ERR_WORKSPACE
    assert "static" in lib.hs2_last_error().decode()
    small = base_problem()
    assert hs2.workspace_size(small)[0] <= hs2.STATIC_WORKSPACE_BYTES
    assert call(small, dict(q=None)) == 1                      # HS2_ERR_NULL
    assert call(small, dict(os=None)) == 1
    assert call(small, dict(idx=FAKE + 4)) == 5                # HS2_ERR_ALIGN
    assert call(base_problem(h_q=6, h_kv=4)) == 2              # HS2_ERR_SHAPE
