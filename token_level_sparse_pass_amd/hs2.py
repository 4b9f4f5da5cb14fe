"""Python binding of libhs2.so (the C ABI in include/hs2.h).

Argument marshalling only: tensors are passed as raw device pointers and
every step of the Hybrid Block runs in the library's HIP kernels. PyTorch
provides device memory and the current stream. If the library has not been
built, every call raises; there is no fallback path.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhs2.so")

ABI_VERSION = 1
FP32, BF16 = 0, 1
SELECT_TOKEN, SELECT_BLOCK = 0, 1
STATUS = {0: "ok", 1: "null pointer", 2: "invalid shape", 3: "unsupported",
          4: "workspace too small", 5: "misaligned pointer", 6: "device error"}


class Problem(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("window", ctypes.c_int32), ("select", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("top_blocks", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class Debug(ctypes.Structure):
    _fields_ = [("rows", ctypes.POINTER(ctypes.c_int32)), ("n_rows", ctypes.c_int32),
                ("scores_out", ctypes.c_void_p)]


class KvPages(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


class HS2Error(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"hs2 status {status} ({STATUS.get(status, '?')}): {detail}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libhs2.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with "
                           "`python -m token_level_sparse_pass_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER(Problem)
    lib.hs2_abi_version.restype = i32
    lib.hs2_index_width.argtypes = [P]
    lib.hs2_index_width.restype = i32
    lib.hs2_workspace_size.argtypes = [P, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.hs2_workspace_size.restype = i32
    lib.hs2_full_attn_select.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Debug),
                                         vp, sz, vp]
    lib.hs2_full_attn_select.restype = i32
    lib.hs2_sparse_attn.argtypes = [P, i32, vp, vp, vp, vp, vp, vp]
    lib.hs2_sparse_attn.restype = i32
    lib.hs2_block_forward.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_block_forward.restype = i32
    lib.hs2_block_forward_static.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hs2_block_forward_static.restype = i32
    lib.hs2_decode_step.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(i32), vp, vp,
                                    vp, vp, vp, sz, vp]
    lib.hs2_decode_step.restype = i32
    lib.hs2_decode_step_paged.argtypes = [P, ctypes.POINTER(KvPages), i32, vp, vp, vp, vp, vp, vp,
                                          ctypes.POINTER(i32), vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_decode_step_paged.restype = i32
    lib.hs2_kv_bridge.argtypes = [P, i32, vp, vp, vp, vp, vp]
    lib.hs2_kv_bridge.restype = i32
    pi = ctypes.POINTER(i32)
    lib.hs2_workspace_size_varlen.argtypes = [P, pi, pi, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.hs2_workspace_size_varlen.restype = i32
    lib.hs2_block_forward_varlen.argtypes = [P, i32, pi, pi] + [vp] * 9 + [sz, vp]
    lib.hs2_block_forward_varlen.restype = i32
    KP = ctypes.POINTER(KvPages)
    lib.hs2_workspace_size_paged.argtypes = [P, KP, pi, pi, ctypes.POINTER(sz),
                                             ctypes.POINTER(sz)]
    lib.hs2_workspace_size_paged.restype = i32
    lib.hs2_block_forward_paged.argtypes = [P, KP, i32, pi, pi] + [vp] * 11 + [sz, vp]
    lib.hs2_block_forward_paged.restype = i32
    lib.hs2_backward_workspace_size.argtypes = [P, i32, ctypes.POINTER(sz)]
    lib.hs2_backward_workspace_size.restype = i32
    lib.hs2_block_backward.argtypes = [P, i32] + [vp] * 14 + [vp, sz, vp]
    lib.hs2_block_backward.restype = i32
    lib.hs2_block_backward_deterministic.argtypes = [P, i32] + [vp] * 14 + [vp, sz, vp]
    lib.hs2_block_backward_deterministic.restype = i32
    lib.hs2_status_string.argtypes = [i32]
    lib.hs2_status_string.restype = ctypes.c_char_p
    lib.hs2_last_error.restype = ctypes.c_char_p
    lib.hs2_profile_enable.argtypes = [i32]
    lib.hs2_profile_enable.restype = i32
    lib.hs2_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64)]
    lib.hs2_profile_read.restype = i32
    if lib.hs2_abi_version() != ABI_VERSION:
        raise RuntimeError("libhs2.so ABI version mismatch")
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise HS2Error(status, _lib.hs2_last_error().decode())


def problem(dtype, batch, n_q, n_kv, h_q, h_kv, head_dim, top_k=1024, window=128,
            select="token", block_size=64, top_blocks=16, softmax_scale=None) -> Problem:
    if isinstance(dtype, torch.dtype):
        dtype = BF16 if dtype == torch.bfloat16 else FP32 if dtype == torch.float32 else -1
    sel = SELECT_TOKEN if select == "token" else SELECT_BLOCK if select == "block" else select
    scale = head_dim ** -0.5 if softmax_scale is None else softmax_scale
    return Problem(ABI_VERSION, dtype, batch, n_q, n_kv, h_q, h_kv, head_dim, top_k, window,
                   sel, block_size, top_blocks, scale)


def index_width(p: Problem) -> int:
    w = load().hs2_index_width(ctypes.byref(p))
    if w < 0:
        raise HS2Error(2, load().hs2_last_error().decode())
    return w


def workspace_size(p: Problem):
    lib = load()
    mn, pref = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.hs2_workspace_size(ctypes.byref(p), ctypes.byref(mn), ctypes.byref(pref)))
    return mn.value, pref.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _problem_from(q, k, kw):
    B, nq, hq, d = q.shape
    _, nkv, hkv, _ = k.shape
    return problem(q.dtype, B, nq, nkv, hq, hkv, d, **kw)


def _check_tensor(t, name, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")


def _validate(specs):
    """Check every tensor argument against the shape the call implies.

    specs: (tensor or None, name, expected shape, dtype or None) tuples; a
    None tensor is skipped. The C ABI receives raw pointers and cannot see a
    mis-shaped tensor, which would become an out-of-bounds device access, so
    every shape, dtype and device is checked here first: shapes and dtypes
    before anything touches a device (so these checks also run without a
    GPU), then that all tensors are contiguous device tensors on one device.
    """
    live = [s for s in specs if s[0] is not None]
    for t, name, shape, dtype in live:
        if tuple(t.shape) != tuple(int(x) for x in shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} is {t.dtype}, expected {dtype}")
    dev = live[0][0].device if live else None
    for t, name, _, _ in live:
        _check_tensor(t, name)
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _ws_bytes(ws, device):
    """Byte size of a caller workspace (any dtype), after checking it."""
    if not ws.is_cuda or ws.device != device:
        raise ValueError(f"workspace must be a device tensor on {device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws.numel() * ws.element_size()


def alloc_workspace(p: Problem, device, nbytes=None):
    mn, pref = workspace_size(p)
    n = pref if nbytes is None else max(nbytes, mn)
    return torch.empty(n, dtype=torch.uint8, device=device)


def full_attn_select(q, k, v, *, workspace=None, debug_rows=None, want_lse=True, **kw):
    """Full layer + scoring + selection. Returns (o, idx, lse, scores|None)."""
    lib = load()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, n_q, h_q, d] and k [B, n_kv, h_kv, d]")
    B, nq, hq, d = q.shape
    _validate([(q, "q", q.shape, q.dtype), (k, "k", (B, k.shape[1], k.shape[2], d), q.dtype),
               (v, "v", k.shape, q.dtype)])
    p = _problem_from(q, k, kw)
    width = index_width(p)
    o = torch.empty_like(q)
    idx = torch.empty((B, nq, width), dtype=torch.int32, device=q.device)
    lse = torch.empty((B, hq, nq), dtype=torch.float32, device=q.device) if want_lse else None
    ws = alloc_workspace(p, q.device) if workspace is None else workspace
    dbg_ref, scores = None, None
    if debug_rows is not None:
        rows = (ctypes.c_int32 * len(debug_rows))(*[int(r) for r in debug_rows])
        scores = torch.empty((len(debug_rows), k.shape[1]), dtype=torch.float32, device=q.device)
        dbg = Debug(rows, len(debug_rows), scores.data_ptr())
        dbg_ref = ctypes.byref(dbg)
    _check(lib.hs2_full_attn_select(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                    _ptr(idx), _ptr(lse), dbg_ref, _ptr(ws),
                                    _ws_bytes(ws, q.device), _stream(q.device)))
    return o, idx, lse, scores


def sparse_attn(q_layers, k, v, idx, **kw):
    """Sparse layers over the given index rows. q_layers [L, B, n_q, h_q, d]."""
    lib = load()
    if q_layers.dim() != 5 or k.dim() != 4:
        raise ValueError("q_layers must be [L, B, n_q, h_q, d] and k [B, n_kv, h_kv, d]")
    L, B, nq, hq, d = q_layers.shape
    p = problem(q_layers.dtype, B, nq, k.shape[1], hq, k.shape[2], d, **kw)
    width = index_width(p)
    _validate([(q_layers, "q_layers", q_layers.shape, q_layers.dtype),
               (k, "k", (B, k.shape[1], k.shape[2], d), q_layers.dtype),
               (v, "v", k.shape, q_layers.dtype), (idx, "idx", (B, nq, width), torch.int32)])
    o = torch.empty_like(q_layers)
    _check(lib.hs2_sparse_attn(ctypes.byref(p), L, _ptr(q_layers), _ptr(k), _ptr(v),
                               _ptr(idx), _ptr(o), _stream(k.device)))
    return o


def block_forward(q_full, q_sparse, k, v, *, workspace=None, want_lse=True, out=None, **kw):
    """The whole Hybrid Block. Returns dict(o_full, o_sparse, idx, lse)."""
    lib = load()
    if q_full.dim() != 4 or k.dim() != 4 or q_sparse.dim() != 5:
        raise ValueError("q_full must be [B, n_q, h_q, d], q_sparse [L, B, n_q, h_q, d] "
                         "and k [B, n_kv, h_kv, d]")
    B, nq, hq, d = q_full.shape
    L = q_sparse.shape[0]
    p = _problem_from(q_full, k, kw)
    width = index_width(p)
    kshape = (B, k.shape[1], k.shape[2], d)
    specs = [(q_full, "q_full", q_full.shape, q_full.dtype),
             (q_sparse, "q_sparse", (L,) + tuple(q_full.shape), q_full.dtype),
             (k, "k", kshape, q_full.dtype), (v, "v", kshape, q_full.dtype)]
    if out is not None:
        specs += [(out["o_full"], "o_full", q_full.shape, q_full.dtype),
                  (out["o_sparse"], "o_sparse", q_sparse.shape, q_full.dtype),
                  (out["idx"], "idx", (B, nq, width), torch.int32),
                  (out.get("lse"), "lse", (B, hq, nq), torch.float32)]
    _validate(specs)
    if out is None:
        out = dict(o_full=torch.empty_like(q_full), o_sparse=torch.empty_like(q_sparse),
                   idx=torch.empty((B, nq, width), dtype=torch.int32, device=q_full.device),
                   lse=torch.empty((B, hq, nq), dtype=torch.float32, device=q_full.device)
                   if want_lse else None)
    ws = alloc_workspace(p, q_full.device) if workspace is None else workspace
    _check(lib.hs2_block_forward(ctypes.byref(p), L, _ptr(q_full),
                                 _ptr(q_sparse), _ptr(k), _ptr(v), _ptr(out["o_full"]),
                                 _ptr(out["o_sparse"]), _ptr(out["idx"]), _ptr(out.get("lse")),
                                 _ptr(ws), _ws_bytes(ws, q_full.device), _stream(q_full.device)))
    return out


STATIC_WORKSPACE_BYTES = 64 << 20      # HS2_STATIC_WORKSPACE_BYTES


def block_forward_static(q_full, q_sparse, k, v, *, out, **kw):
    """hs2_block_forward_static: the whole block with the library's static
    device workspace, for callers that cannot allocate. `out` holds the
    caller's output tensors (o_full, o_sparse, idx, lse or None); the call
    allocates nothing. Calls that overlap in time on one GPU race."""
    lib = load()
    if q_full.dim() != 4 or k.dim() != 4 or q_sparse.dim() != 5:
        raise ValueError("q_full must be [B, n_q, h_q, d], q_sparse [L, B, n_q, h_q, d] "
                         "and k [B, n_kv, h_kv, d]")
    B, nq, hq, d = q_full.shape
    L = q_sparse.shape[0]
    p = _problem_from(q_full, k, kw)
    width = index_width(p)
    kshape = (B, k.shape[1], k.shape[2], d)
    _validate([(q_full, "q_full", q_full.shape, q_full.dtype),
               (q_sparse, "q_sparse", (L,) + tuple(q_full.shape), q_full.dtype),
               (k, "k", kshape, q_full.dtype), (v, "v", kshape, q_full.dtype),
               (out["o_full"], "o_full", q_full.shape, q_full.dtype),
               (out["o_sparse"], "o_sparse", q_sparse.shape, q_full.dtype),
               (out["idx"], "idx", (B, nq, width), torch.int32),
               (out.get("lse"), "lse", (B, hq, nq), torch.float32)])
    _check(lib.hs2_block_forward_static(ctypes.byref(p), L, _ptr(q_full), _ptr(q_sparse),
                                        _ptr(k), _ptr(v), _ptr(out["o_full"]),
                                        _ptr(out["o_sparse"]), _ptr(out["idx"]),
                                        _ptr(out.get("lse")), _stream(q_full.device)))
    return out


def decode_step(q_full, q_sparse, k_new, v_new, k_cache, v_cache, lens, *, workspace=None,
                want_lse=True, out=None, **kw):
    """One decode step over a growing cache (hs2_decode_step).

    q_full [B, 1, h_q, d], q_sparse [L, B, 1, h_q, d], k_new / v_new
    [B, 1, h_kv, d], k_cache / v_cache [B, capacity, h_kv, d] (modified in
    place: the new rows land at row lens[b]); lens: the B lengths before the
    step (a sequence of ints, kept on the host). Returns dict(o_full,
    o_sparse, idx, lse); the caller advances lens.
    """
    lib = load()
    if q_full.dim() != 4 or k_cache.dim() != 4 or q_sparse.dim() != 5:
        raise ValueError("q_full must be [B, 1, h_q, d], q_sparse [L, B, 1, h_q, d] and "
                         "k_cache [B, capacity, h_kv, d]")
    B, nq, hq, d = q_full.shape
    hkv = k_cache.shape[2]
    if len(lens) != B:
        raise ValueError(f"lens has {len(lens)} entries, expected {B}")
    p = _problem_from(q_full, k_cache, kw)
    width = index_width(p)
    cshape = (B, k_cache.shape[1], hkv, d)
    specs = [(q_full, "q_full", q_full.shape, q_full.dtype),
             (q_sparse, "q_sparse", (q_sparse.shape[0],) + tuple(q_full.shape), q_full.dtype),
             (k_new, "k_new", (B, nq, hkv, d), q_full.dtype),
             (v_new, "v_new", (B, nq, hkv, d), q_full.dtype),
             (k_cache, "k_cache", cshape, q_full.dtype), (v_cache, "v_cache", cshape, q_full.dtype)]
    if out is not None:
        specs += [(out["o_full"], "o_full", q_full.shape, q_full.dtype),
                  (out["o_sparse"], "o_sparse", q_sparse.shape, q_full.dtype),
                  (out["idx"], "idx", (B, nq, width), torch.int32),
                  (out.get("lse"), "lse", (B, hq, nq), torch.float32)]
    _validate(specs)
    lens_h = (ctypes.c_int32 * B)(*[int(x) for x in lens])
    if out is None:
        out = dict(o_full=torch.empty_like(q_full), o_sparse=torch.empty_like(q_sparse),
                   idx=torch.empty((B, nq, width), dtype=torch.int32, device=q_full.device),
                   lse=torch.empty((B, hq, nq), dtype=torch.float32, device=q_full.device)
                   if want_lse else None)
    ws = alloc_workspace(p, q_full.device) if workspace is None else workspace
    _check(lib.hs2_decode_step(ctypes.byref(p), q_sparse.shape[0], _ptr(q_full), _ptr(q_sparse),
                               _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), lens_h,
                               _ptr(out["o_full"]), _ptr(out["o_sparse"]), _ptr(out["idx"]),
                               _ptr(out.get("lse")), _ptr(ws), _ws_bytes(ws, q_full.device),
                               _stream(q_full.device)))
    return out


def decode_step_paged(q_full, q_sparse, k_new, v_new, k_pool, v_pool, page_table, page_size,
                      lens, *, workspace=None, want_lse=True, out=None, **kw):
    """hs2_decode_step_paged: decode_step over a paged KV pool.

    k_pool / v_pool [n_pages * page_size, h_kv, d] (modified in place),
    page_table int32 device tensor [B, max_pages]; row j of sequence b is
    pool row page_table[b, j // page_size] * page_size + j % page_size.
    """
    lib = load()
    if q_full.dim() != 4 or k_pool.dim() != 3 or q_sparse.dim() != 5 or page_table.dim() != 2:
        raise ValueError("q_full must be [B, 1, h_q, d], q_sparse [L, B, 1, h_q, d], k_pool "
                         "[rows, h_kv, d] and page_table [B, max_pages]")
    B, nq, hq, d = q_full.shape
    hkv = k_pool.shape[1]
    if len(lens) != B:
        raise ValueError(f"lens has {len(lens)} entries, expected {B}")
    max_pages = page_table.shape[1]
    n_pages = k_pool.shape[0] // page_size
    p = problem(q_full.dtype, B, nq, max_pages * page_size, hq, hkv, d, **kw)
    width = index_width(p)
    pshape = (k_pool.shape[0], hkv, d)
    specs = [(q_full, "q_full", q_full.shape, q_full.dtype),
             (q_sparse, "q_sparse", (q_sparse.shape[0],) + tuple(q_full.shape), q_full.dtype),
             (k_new, "k_new", (B, nq, hkv, d), q_full.dtype),
             (v_new, "v_new", (B, nq, hkv, d), q_full.dtype),
             (k_pool, "k_pool", pshape, q_full.dtype), (v_pool, "v_pool", pshape, q_full.dtype),
             (page_table, "page_table", (B, max_pages), torch.int32)]
    if out is not None:
        specs += [(out["o_full"], "o_full", q_full.shape, q_full.dtype),
                  (out["o_sparse"], "o_sparse", q_sparse.shape, q_full.dtype),
                  (out["idx"], "idx", (B, nq, width), torch.int32),
                  (out.get("lse"), "lse", (B, hq, nq), torch.float32)]
    _validate(specs)
    pages = KvPages(page_table.data_ptr(), page_size, max_pages, n_pages)
    lens_h = (ctypes.c_int32 * B)(*[int(x) for x in lens])
    if out is None:
        out = dict(o_full=torch.empty_like(q_full), o_sparse=torch.empty_like(q_sparse),
                   idx=torch.empty((B, nq, width), dtype=torch.int32, device=q_full.device),
                   lse=torch.empty((B, hq, nq), dtype=torch.float32, device=q_full.device)
                   if want_lse else None)
    ws = alloc_workspace(p, q_full.device) if workspace is None else workspace
    _check(lib.hs2_decode_step_paged(ctypes.byref(p), ctypes.byref(pages), q_sparse.shape[0],
                                     _ptr(q_full), _ptr(q_sparse), _ptr(k_new), _ptr(v_new),
                                     _ptr(k_pool), _ptr(v_pool), lens_h, _ptr(out["o_full"]),
                                     _ptr(out["o_sparse"]), _ptr(out["idx"]),
                                     _ptr(out.get("lse")), _ptr(ws), _ws_bytes(ws, q_full.device),
                                     _stream(q_full.device)))
    return out


def kv_bridge(hidden, w_kv, h_kv, *, out=None):
    """hs2_kv_bridge: K, V [B, n, h_kv, d] from hidden [B, n, d_model] and
    w_kv [2, h_kv * d, d_model] (bf16). Returns (k, v)."""
    lib = load()
    if hidden.dim() != 3 or w_kv.dim() != 3:
        raise ValueError("hidden must be [B, n, d_model] and w_kv [2, h_kv * d, d_model]")
    B, n, dm = hidden.shape
    feats = w_kv.shape[1]
    if h_kv <= 0 or feats % h_kv:
        raise ValueError(f"w_kv has {feats} output features, not a multiple of h_kv = {h_kv}")
    d = feats // h_kv
    specs = [(hidden, "hidden", hidden.shape, torch.bfloat16),
             (w_kv, "w_kv", (2, feats, dm), torch.bfloat16)]
    if out is not None:
        specs += [(out[0], "k", (B, n, h_kv, d), torch.bfloat16),
                  (out[1], "v", (B, n, h_kv, d), torch.bfloat16)]
    _validate(specs)
    p = problem(torch.bfloat16, B, 1, n, h_kv, h_kv, d, top_k=1, window=1)
    if out is None:
        out = (torch.empty((B, n, h_kv, d), dtype=torch.bfloat16, device=hidden.device),
               torch.empty((B, n, h_kv, d), dtype=torch.bfloat16, device=hidden.device))
    _check(lib.hs2_kv_bridge(ctypes.byref(p), dm, _ptr(hidden), _ptr(w_kv), _ptr(out[0]),
                             _ptr(out[1]), _stream(hidden.device)))
    return out


def backward_workspace_size(p: Problem, n_sparse_layers: int) -> int:
    n = ctypes.c_size_t()
    _check(load().hs2_backward_workspace_size(ctypes.byref(p), int(n_sparse_layers),
                                              ctypes.byref(n)))
    return n.value


def block_backward(q_full, q_sparse, k, v, o_full, o_sparse, lse, idx, do_full, do_sparse, *,
                   workspace=None, out=None, deterministic=False, **kw):
    """Backward of the whole block with the index sets held fixed. Takes the
    forward's inputs and outputs (lse: natural log, required) and the output
    gradients; returns dict(dq_full, dq_sparse, dk, dv). deterministic=True
    calls hs2_block_backward_deterministic (bit-reproducible K/V sums)."""
    lib = load()
    dt = q_full.dtype
    if q_full.dim() != 4 or k.dim() != 4:
        raise ValueError("q_full must be [B, n_q, h_q, d] and k [B, n_kv, h_kv, d]")
    B, nq, hq, d = q_full.shape
    L = 0 if q_sparse is None else q_sparse.shape[0]
    p = _problem_from(q_full, k, kw)
    kshape = (B, k.shape[1], k.shape[2], d)
    specs = [(q_full, "q_full", q_full.shape, dt), (k, "k", kshape, dt), (v, "v", kshape, dt),
             (o_full, "o_full", q_full.shape, dt), (do_full, "do_full", q_full.shape, dt),
             (lse, "lse", (B, hq, nq), torch.float32)]
    if L:
        lshape = (L,) + tuple(q_full.shape)
        specs += [(q_sparse, "q_sparse", lshape, dt), (o_sparse, "o_sparse", lshape, dt),
                  (do_sparse, "do_sparse", lshape, dt),
                  (idx, "idx", (B, nq, index_width(p)), torch.int32)]
    if out is not None:
        specs += [(out["dq_full"], "dq_full", q_full.shape, dt),
                  (out["dq_sparse"] if L else None, "dq_sparse", (L,) + tuple(q_full.shape), dt),
                  (out["dk"], "dk", kshape, dt), (out["dv"], "dv", kshape, dt)]
    _validate(specs)
    if out is None:
        out = dict(dq_full=torch.empty_like(q_full),
                   dq_sparse=torch.empty_like(q_sparse) if L else None,
                   dk=torch.empty_like(k), dv=torch.empty_like(v))
    if workspace is None:
        workspace = torch.empty(max(16, backward_workspace_size(p, L)), dtype=torch.uint8,
                                device=q_full.device)
    fn = lib.hs2_block_backward_deterministic if deterministic else lib.hs2_block_backward
    _check(fn(
        ctypes.byref(p), L, _ptr(q_full), _ptr(q_sparse if L else None), _ptr(k), _ptr(v),
        _ptr(o_full), _ptr(o_sparse if L else None), _ptr(lse), _ptr(idx if L else None),
        _ptr(do_full), _ptr(do_sparse if L else None), _ptr(out["dq_full"]),
        _ptr(out["dq_sparse"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(workspace),
        _ws_bytes(workspace, q_full.device), _stream(q_full.device)))
    return out


def _cu(x):
    vals = [int(t) for t in (x.tolist() if hasattr(x, "tolist") else x)]
    return (ctypes.c_int32 * len(vals))(*vals), vals


def workspace_size_varlen(p: Problem, cu_q, cu_kv):
    cq, _ = _cu(cu_q)
    ck, _ = _cu(cu_kv)
    mn, pref = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().hs2_workspace_size_varlen(ctypes.byref(p), cq, ck, ctypes.byref(mn),
                                            ctypes.byref(pref)))
    return mn.value, pref.value


def block_forward_varlen(q_full, q_sparse, k, v, cu_q, cu_kv, *, workspace=None, want_lse=True,
                         **kw):
    """The block over a packed batch of sequences of different lengths.
    q_full [total_q, h_q, d], q_sparse [L, total_q, h_q, d], k/v
    [total_kv, h_kv, d]; cu_q / cu_kv: host sequences of batch + 1 offsets.
    Returns dict(o_full, o_sparse, idx [total_q, W], lse (h_q * total_q
    floats, sequence b's [h_q][n_q(b)] block at h_q * cu_q[b]))."""
    lib = load()
    if q_full.dim() != 3 or k.dim() != 3 or q_sparse.dim() != 4:
        raise ValueError("q_full must be [total_q, h_q, d], q_sparse [L, total_q, h_q, d] and "
                         "k [total_kv, h_kv, d]")
    cq, vq = _cu(cu_q)
    ck, vk = _cu(cu_kv)
    batch = len(vq) - 1
    total_q, hq, d = q_full.shape
    hkv = k.shape[1]
    if len(vk) != len(vq) or vq[-1] != total_q or vk[-1] != k.shape[0]:
        raise ValueError("cu_seqlens do not match the packed tensors")
    kshape = (k.shape[0], hkv, d)
    _validate([(q_full, "q_full", q_full.shape, q_full.dtype),
               (q_sparse, "q_sparse", (q_sparse.shape[0],) + tuple(q_full.shape), q_full.dtype),
               (k, "k", kshape, q_full.dtype), (v, "v", kshape, q_full.dtype)])
    p = problem(q_full.dtype, batch, 1, 1, hq, hkv, d, **kw)
    width = index_width(p)
    mn, pref = workspace_size_varlen(p, cq, ck)
    if workspace is None:
        workspace = torch.empty(max(16, pref), dtype=torch.uint8, device=q_full.device)
    out = dict(o_full=torch.empty_like(q_full), o_sparse=torch.empty_like(q_sparse),
               idx=torch.empty((total_q, width), dtype=torch.int32, device=q_full.device),
               lse=torch.empty((hq * total_q,), dtype=torch.float32, device=q_full.device)
               if want_lse else None)
    _check(lib.hs2_block_forward_varlen(
        ctypes.byref(p), q_sparse.shape[0], cq, ck, _ptr(q_full), _ptr(q_sparse), _ptr(k),
        _ptr(v), _ptr(out["o_full"]), _ptr(out["o_sparse"]), _ptr(out["idx"]), _ptr(out["lse"]),
        _ptr(workspace), _ws_bytes(workspace, q_full.device), _stream(q_full.device)))
    return out


def _paged_problem(q_full, k_pool, page_table, page_size, batch, kw):
    max_pages = page_table.shape[1]
    p = problem(q_full.dtype, batch, 1, max_pages * page_size, q_full.shape[1], k_pool.shape[1],
                q_full.shape[2], **kw)
    pages = KvPages(page_table.data_ptr(), page_size, max_pages, k_pool.shape[0] // page_size)
    return p, pages


def workspace_size_paged(p: Problem, pages: KvPages, cu_q, lens):
    cq, _ = _cu(cu_q)
    ln, _ = _cu(lens)
    mn, pref = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().hs2_workspace_size_paged(ctypes.byref(p), ctypes.byref(pages), cq, ln,
                                           ctypes.byref(mn), ctypes.byref(pref)))
    return mn.value, pref.value


def block_forward_paged(q_full, q_sparse, k_new, v_new, k_pool, v_pool, page_table, page_size,
                        cu_q, lens, *, workspace=None, want_lse=True, **kw):
    """hs2_block_forward_paged: chunked prefill over a paged KV pool.

    q_full [total_q, h_q, d], q_sparse [L, total_q, h_q, d], k_new / v_new
    [total_q, h_kv, d] (sequence b's new tokens are rows cu_q[b] ..
    cu_q[b+1]), k_pool / v_pool [n_pages * page_size, h_kv, d] (modified in
    place), page_table int32 device tensor [B, max_pages]; lens: the B
    lengths before the call (host ints; the caller advances them). Returns
    dict(o_full, o_sparse, idx [total_q, W], lse) as block_forward_varlen."""
    lib = load()
    if q_full.dim() != 3 or k_pool.dim() != 3 or q_sparse.dim() != 4 or page_table.dim() != 2:
        raise ValueError("q_full must be [total_q, h_q, d], q_sparse [L, total_q, h_q, d], "
                         "k_pool [rows, h_kv, d] and page_table [B, max_pages]")
    cq, vq = _cu(cu_q)
    ln, vl = _cu(lens)
    batch = len(vq) - 1
    total_q, hq, d = q_full.shape
    hkv = k_pool.shape[1]
    if vq[-1] != total_q or len(vl) != batch:
        raise ValueError("cu_q / lens do not match the packed tensors")
    if page_table.shape[0] != batch:
        raise ValueError("page_table needs one row per sequence")
    pshape = (k_pool.shape[0], hkv, d)
    _validate([(q_full, "q_full", q_full.shape, q_full.dtype),
               (q_sparse, "q_sparse", (q_sparse.shape[0],) + tuple(q_full.shape), q_full.dtype),
               (k_new, "k_new", (total_q, hkv, d), q_full.dtype),
               (v_new, "v_new", (total_q, hkv, d), q_full.dtype),
               (k_pool, "k_pool", pshape, q_full.dtype), (v_pool, "v_pool", pshape, q_full.dtype),
               (page_table, "page_table", page_table.shape, torch.int32)])
    p, pages = _paged_problem(q_full, k_pool, page_table, page_size, batch, kw)
    width = index_width(p)
    if workspace is None:
        _, pref = workspace_size_paged(p, pages, vq, vl)
        workspace = torch.empty(max(16, pref), dtype=torch.uint8, device=q_full.device)
    out = dict(o_full=torch.empty_like(q_full), o_sparse=torch.empty_like(q_sparse),
               idx=torch.empty((total_q, width), dtype=torch.int32, device=q_full.device),
               lse=torch.empty((hq * total_q,), dtype=torch.float32, device=q_full.device)
               if want_lse else None)
    _check(lib.hs2_block_forward_paged(
        ctypes.byref(p), ctypes.byref(pages), q_sparse.shape[0], cq, ln, _ptr(q_full),
        _ptr(q_sparse), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(out["o_full"]),
        _ptr(out["o_sparse"]), _ptr(out["idx"]), _ptr(out["lse"]), _ptr(workspace),
        _ws_bytes(workspace, q_full.device), _stream(q_full.device)))
    return out
