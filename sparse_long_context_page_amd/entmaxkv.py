"""Python binding of libentmaxkv.so (the C ABI in include/entmaxkv.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the decode runs in the library's HIP
kernels. Importing this module loads the library and raises if it is not
built (there is no fallback path).

The function names match the C ABI:
    entmaxkv_build_page_meta, entmaxkv_append_page_meta, entmaxkv_score_select,
    entmaxkv_score_select_noalloc, entmaxkv_decode_sparse, entmaxkv_decode_topk,
    entmaxkv_decode_full, entmaxkv_build_page_moments,
    entmaxkv_append_page_moments, entmaxkv_gauss_select, entmaxkv_workspace_bytes,
    entmaxkv_topk_kernels, entmaxkv_strerror
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libentmaxkv.so")

ENTMAXKV_OK = 0
ENTMAXKV_ERR_INVALID = -1
ENTMAXKV_ERR_UNSUPPORTED = -2
ENTMAXKV_ERR_WORKSPACE = -3
ENTMAXKV_ERR_HIP = -4

ENTMAXKV_F32 = 0
ENTMAXKV_BF16 = 1

ENTMAXKV_WS_SELECT = 0
ENTMAXKV_WS_SPARSE = 1
ENTMAXKV_WS_FULL = 2
ENTMAXKV_WS_GAUSS = 3
ENTMAXKV_WS_TOPK = 4

# kernels each entry point launches (for per-kernel event timing)
KERNELS = {"build_page_meta": 1, "append_page_meta": 1, "score_select": 2,
           "score_select_noalloc": 2, "decode_sparse": 2, "decode_topk": 4,
           "decode_full": 2, "build_page_moments": 1, "append_page_moments": 1,
           "gauss_select": 2}


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
    ]


class EntmaxKVError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {entmaxkv_strerror(code)} (code {code})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m sparse_long_context_page_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    SP = ctypes.POINTER(Shape)
    lib.entmaxkv_build_page_meta.argtypes = [SP, P, P, P, P, P, P]
    lib.entmaxkv_append_page_meta.argtypes = [SP, P, P, P, P, I32, P, P, P]
    lib.entmaxkv_score_select.argtypes = [SP, P, P, P, P, I32, P, P, P, SZ, P, P]
    lib.entmaxkv_score_select_noalloc.argtypes = [SP, P, P, P, P, I32, P, P, P, P]
    lib.entmaxkv_decode_sparse.argtypes = [SP, P, P, P, P, P, P, I32, F32, P, P, P, P, SZ, P, P]
    lib.entmaxkv_decode_topk.argtypes = [SP, P, P, P, P, P, P, I32, F32, P, P, P, P, P, P, SZ,
                                         P, P]
    lib.entmaxkv_decode_full.argtypes = [SP, P, P, P, P, P, F32, P, P, P, P, SZ, P, P]
    lib.entmaxkv_build_page_moments.argtypes = [SP, P, P, P, P, P, P]
    lib.entmaxkv_append_page_moments.argtypes = [SP, P, P, P, P, I32, P, P, P]
    lib.entmaxkv_gauss_select.argtypes = [SP, P, P, P, P, F32, F32, I32, P, P, P, SZ, P, P]
    lib.entmaxkv_workspace_bytes.argtypes = [SP, I32, I32, ctypes.POINTER(SZ)]
    lib.entmaxkv_topk_kernels.argtypes = [SP, I32, ctypes.POINTER(I32)]
    lib.entmaxkv_strerror.argtypes = [ctypes.c_int]
    lib.entmaxkv_strerror.restype = ctypes.c_char_p
    lib.entmaxkv_version.argtypes = []
    for name in ("entmaxkv_build_page_meta", "entmaxkv_append_page_meta",
                 "entmaxkv_score_select", "entmaxkv_score_select_noalloc",
                 "entmaxkv_decode_sparse", "entmaxkv_decode_topk", "entmaxkv_decode_full",
                 "entmaxkv_build_page_moments", "entmaxkv_append_page_moments",
                 "entmaxkv_gauss_select", "entmaxkv_workspace_bytes", "entmaxkv_topk_kernels",
                 "entmaxkv_version"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()


def entmaxkv_strerror(code: int) -> str:
    return lib.entmaxkv_strerror(int(code)).decode()


def make_shape(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq,
               num_phys_pages, kv_dtype) -> Shape:
    if isinstance(kv_dtype, str):
        kv_dtype = {"f32": ENTMAXKV_F32, "bf16": ENTMAXKV_BF16}[kv_dtype]
    return Shape(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim), int(page_size),
                 int(max_pages_per_seq), int(num_phys_pages), int(kv_dtype))


# ---------------------------------------------------------------------------
# marshalling helpers


def _ptr(t, name, dtypes=None, nullable=False, numel=None):
    """Pointer of tensor `t` after host-side checks: its dtype, at least
    `numel` elements (the count the shape implies: a shorter tensor would
    make the kernels read or write past its end) and contiguity. Raises
    TypeError / ValueError before any library call. That every tensor lives
    on the GPU is checked afterwards, for all arguments at once
    (_on_device)."""
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements; the shape needs {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _on_device(**tensors):
    """Every given tensor (None allowed) must be a device tensor."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


class _Sizes:
    """Element counts the shape implies for each array argument."""

    def __init__(self, shape: Shape):
        B, H, Hkv = shape.batch, shape.num_q_heads, shape.num_kv_heads
        D, ps = shape.head_dim, shape.page_size
        self.q = B * H * D
        self.out = B * H * D
        self.heads = B * H
        self.pool = shape.num_phys_pages * Hkv * ps * D
        self.meta = shape.num_phys_pages * Hkv * 2 * D
        self.block_table = B * shape.max_pages_per_seq
        self.batch = B

    def sel(self, budget):
        return self.heads * max(int(budget), 0)


def _kv_dtypes(shape: Shape):
    return (torch.float32,) if shape.kv_dtype == ENTMAXKV_F32 else (torch.bfloat16, torch.int16)


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def _events(events):
    if events is None:
        return None
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(int(e)) for e in events])
    return ctypes.cast(arr, ctypes.c_void_p), arr


def _check(rc: int, where: str):
    if rc != ENTMAXKV_OK:
        raise EntmaxKVError(rc, where)


def entmaxkv_workspace_bytes(shape: Shape, budget_pages: int, which: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.entmaxkv_workspace_bytes(ctypes.byref(shape), int(budget_pages), int(which),
                                        ctypes.byref(out)), "entmaxkv_workspace_bytes")
    return int(out.value)


def entmaxkv_topk_kernels(shape: Shape, budget_pages: int) -> int:
    """Kernels entmaxkv_decode_topk launches here: 2 (per-head path) or 4."""
    out = ctypes.c_int32(0)
    _check(lib.entmaxkv_topk_kernels(ctypes.byref(shape), int(budget_pages), ctypes.byref(out)),
           "entmaxkv_topk_kernels")
    return int(out.value)


def workspace(shape: Shape, budget_pages: int, which: int, device) -> torch.Tensor:
    """Allocate a workspace tensor of the size the library asks for."""
    n = entmaxkv_workspace_bytes(shape, budget_pages, which)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# entry points


def _args_build_page_meta(shape: Shape, k_pool, block_table, seq_lens, meta, stream=None):
    n = _Sizes(shape)
    ptrs = [_ptr(k_pool, "k_pool", _kv_dtypes(shape), numel=n.pool),
            _ptr(block_table, "block_table", (torch.int32,), numel=n.block_table),
            _ptr(seq_lens, "seq_lens", (torch.int32,), numel=n.batch),
            _ptr(meta, "meta", _kv_dtypes(shape), numel=n.meta)]
    _on_device(k_pool=k_pool, block_table=block_table, seq_lens=seq_lens, meta=meta)
    return lib.entmaxkv_build_page_meta, [ctypes.byref(shape), *ptrs,
                                          _stream(stream, k_pool.device), None]


def _args_append(fn, what, shape: Shape, k_pool, block_table, old_lens, new_lens,
                 max_new_tokens, meta, stream=None):
    n = _Sizes(shape)
    ptrs = [_ptr(k_pool, "k_pool", _kv_dtypes(shape), numel=n.pool),
            _ptr(block_table, "block_table", (torch.int32,), numel=n.block_table),
            _ptr(old_lens, "old_lens", (torch.int32,), numel=n.batch),
            _ptr(new_lens, "new_lens", (torch.int32,), numel=n.batch)]
    mp = _ptr(meta, what, _kv_dtypes(shape), numel=n.meta)
    _on_device(k_pool=k_pool, block_table=block_table, old_lens=old_lens, new_lens=new_lens,
               **{what: meta})
    return fn, [ctypes.byref(shape), *ptrs, int(max_new_tokens), mp,
                _stream(stream, k_pool.device), None]


def _args_append_page_meta(shape: Shape, k_pool, block_table, old_lens, new_lens,
                           max_new_tokens, meta, stream=None):
    return _args_append(lib.entmaxkv_append_page_meta, "meta", shape, k_pool, block_table,
                        old_lens, new_lens, max_new_tokens, meta, stream)


def _args_append_page_moments(shape: Shape, k_pool, block_table, old_lens, new_lens,
                              max_new_tokens, moments, stream=None):
    return _args_append(lib.entmaxkv_append_page_moments, "moments", shape, k_pool,
                        block_table, old_lens, new_lens, max_new_tokens, moments, stream)


def _args_build_page_moments(shape: Shape, k_pool, block_table, seq_lens, moments, stream=None):
    n = _Sizes(shape)
    ptrs = [_ptr(k_pool, "k_pool", _kv_dtypes(shape), numel=n.pool),
            _ptr(block_table, "block_table", (torch.int32,), numel=n.block_table),
            _ptr(seq_lens, "seq_lens", (torch.int32,), numel=n.batch),
            _ptr(moments, "moments", _kv_dtypes(shape), numel=n.meta)]
    _on_device(k_pool=k_pool, block_table=block_table, seq_lens=seq_lens, moments=moments)
    return lib.entmaxkv_build_page_moments, [ctypes.byref(shape), *ptrs,
                                             _stream(stream, k_pool.device), None]


def _ws_args(ws, shape, budget, which, device):
    """(pointer, bytes, tensor) of the workspace, allocated when not given."""
    if ws is None:
        ws = workspace(shape, budget, which, device)
    else:
        _ptr(ws, "ws")
        _on_device(ws=ws)
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), ws


def _args_gauss_select(shape: Shape, q, moments, block_table, seq_lens, alpha, delta, cap_pages,
                       sel, tau_hat=None, ws=None, stream=None):
    n = _Sizes(shape)
    pq = _ptr(q, "q", (torch.float32,), numel=n.q)
    pm = _ptr(moments, "moments", _kv_dtypes(shape), numel=n.meta)
    pbt = _ptr(block_table, "block_table", (torch.int32,), numel=n.block_table)
    pl = _ptr(seq_lens, "seq_lens", (torch.int32,), numel=n.batch)
    ps_ = _ptr(sel, "sel", (torch.int32,), numel=n.sel(cap_pages))
    pt = _ptr(tau_hat, "tau_hat", (torch.float32,), nullable=True, numel=n.heads)
    _on_device(q=q, moments=moments, block_table=block_table, seq_lens=seq_lens, sel=sel,
               tau_hat=tau_hat)
    pw, nw, ws = _ws_args(ws, shape, cap_pages, ENTMAXKV_WS_GAUSS, q.device)
    return lib.entmaxkv_gauss_select, [
        ctypes.byref(shape), pq, pm, pbt, pl, float(alpha), float(delta), int(cap_pages), ps_,
        pt, pw, nw, _stream(stream, q.device), None], ws


def _args_score_select(shape: Shape, q, meta, block_table, seq_lens, budget_pages, sel,
                       sel_ub=None, ws=None, stream=None):
    n = _Sizes(shape)
    pq = _ptr(q, "q", (torch.float32,), numel=n.q)
    pm = _ptr(meta, "meta", _kv_dtypes(shape), numel=n.meta)
    pbt = _ptr(block_table, "block_table", (torch.int32,), numel=n.block_table)
    pl = _ptr(seq_lens, "seq_lens", (torch.int32,), numel=n.batch)
    ps_ = _ptr(sel, "sel", (torch.int32,), numel=n.sel(budget_pages))
    pu = _ptr(sel_ub, "sel_ub", (torch.float32,), nullable=True, numel=n.sel(budget_pages))
    _on_device(q=q, meta=meta, block_table=block_table, seq_lens=seq_lens, sel=sel,
               sel_ub=sel_ub)
    pw, nw, ws = _ws_args(ws, shape, budget_pages, ENTMAXKV_WS_SELECT, q.device)
    return lib.entmaxkv_score_select, [
        ctypes.byref(shape), pq, pm, pbt, pl, int(budget_pages), ps_, pu, pw, nw,
        _stream(stream, q.device), None], ws


def _args_score_select_noalloc(shape: Shape, q, meta, block_table, seq_lens, budget_pages, sel,
                               sel_ub=None, stream=None):
    n = _Sizes(shape)
    pq = _ptr(q, "q", (torch.float32,), numel=n.q)
    pm = _ptr(meta, "meta", _kv_dtypes(shape), numel=n.meta)
    pbt = _ptr(block_table, "block_table", (torch.int32,), numel=n.block_table)
    pl = _ptr(seq_lens, "seq_lens", (torch.int32,), numel=n.batch)
    ps_ = _ptr(sel, "sel", (torch.int32,), numel=n.sel(budget_pages))
    pu = _ptr(sel_ub, "sel_ub", (torch.float32,), nullable=True, numel=n.sel(budget_pages))
    _on_device(q=q, meta=meta, block_table=block_table, seq_lens=seq_lens, sel=sel,
               sel_ub=sel_ub)
    return lib.entmaxkv_score_select_noalloc, [
        ctypes.byref(shape), pq, pm, pbt, pl, int(budget_pages), ps_, pu,
        _stream(stream, q.device), None]


def _decode_ptrs(shape: Shape, q, k_pool, v_pool, block_table, seq_lens, out, tau, support):
    n = _Sizes(shape)
    return (_ptr(q, "q", (torch.float32,), numel=n.q),
            _ptr(k_pool, "k_pool", _kv_dtypes(shape), numel=n.pool),
            _ptr(v_pool, "v_pool", _kv_dtypes(shape), numel=n.pool),
            _ptr(block_table, "block_table", (torch.int32,), numel=n.block_table),
            _ptr(seq_lens, "seq_lens", (torch.int32,), numel=n.batch),
            _ptr(out, "out", (torch.float32,), numel=n.out),
            _ptr(tau, "tau", (torch.float32,), nullable=True, numel=n.heads),
            _ptr(support, "support", (torch.int32,), nullable=True, numel=n.heads))


def _args_decode_sparse(shape: Shape, q, k_pool, v_pool, block_table, seq_lens, sel,
                        budget_pages, alpha, out, tau=None, support=None, ws=None, stream=None):
    pq, pk, pv, pbt, pl, po, pt, psu = _decode_ptrs(shape, q, k_pool, v_pool, block_table,
                                                     seq_lens, out, tau, support)
    ps_ = _ptr(sel, "sel", (torch.int32,), numel=_Sizes(shape).sel(budget_pages))
    _on_device(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table, seq_lens=seq_lens,
               sel=sel, out=out, tau=tau, support=support)
    pw, nw, ws = _ws_args(ws, shape, budget_pages, ENTMAXKV_WS_SPARSE, q.device)
    return lib.entmaxkv_decode_sparse, [
        ctypes.byref(shape), pq, pk, pv, pbt, pl, ps_, int(budget_pages), float(alpha), po, pt,
        psu, pw, nw, _stream(stream, q.device), None], ws


def _args_decode_topk(shape: Shape, q, meta, k_pool, v_pool, block_table, seq_lens,
                      budget_pages, alpha, sel, out, sel_ub=None, tau=None, support=None,
                      ws=None, stream=None):
    pq, pk, pv, pbt, pl, po, pt, psu = _decode_ptrs(shape, q, k_pool, v_pool, block_table,
                                                     seq_lens, out, tau, support)
    n = _Sizes(shape)
    pm = _ptr(meta, "meta", _kv_dtypes(shape), numel=n.meta)
    ps_ = _ptr(sel, "sel", (torch.int32,), numel=n.sel(budget_pages))
    pu = _ptr(sel_ub, "sel_ub", (torch.float32,), nullable=True, numel=n.sel(budget_pages))
    _on_device(q=q, meta=meta, k_pool=k_pool, v_pool=v_pool, block_table=block_table,
               seq_lens=seq_lens, sel=sel, sel_ub=sel_ub, out=out, tau=tau, support=support)
    pw, nw, ws = _ws_args(ws, shape, budget_pages, ENTMAXKV_WS_TOPK, q.device)
    return lib.entmaxkv_decode_topk, [
        ctypes.byref(shape), pq, pm, pk, pv, pbt, pl, int(budget_pages), float(alpha), ps_, pu,
        po, pt, psu, pw, nw, _stream(stream, q.device), None], ws


def _args_decode_full(shape: Shape, q, k_pool, v_pool, block_table, seq_lens, alpha, out,
                      tau=None, support=None, ws=None, stream=None):
    pq, pk, pv, pbt, pl, po, pt, psu = _decode_ptrs(shape, q, k_pool, v_pool, block_table,
                                                     seq_lens, out, tau, support)
    _on_device(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table, seq_lens=seq_lens,
               out=out, tau=tau, support=support)
    pw, nw, ws = _ws_args(ws, shape, 0, ENTMAXKV_WS_FULL, q.device)
    return lib.entmaxkv_decode_full, [
        ctypes.byref(shape), pq, pk, pv, pbt, pl, float(alpha), po, pt, psu, pw, nw,
        _stream(stream, q.device), None], ws


def _run(name, fn, args, events):
    if events is not None:
        ev = _events(events)
        args = list(args)
        args[-1] = ev[0]
    _check(fn(*args), name)


def entmaxkv_build_page_meta(shape: Shape, k_pool, block_table, seq_lens, meta, stream=None,
                             events=None):
    fn, args = _args_build_page_meta(shape, k_pool, block_table, seq_lens, meta, stream)
    _run("entmaxkv_build_page_meta", fn, args, events)


def entmaxkv_append_page_meta(shape: Shape, k_pool, block_table, old_lens, new_lens,
                              max_new_tokens, meta, stream=None, events=None):
    fn, args = _args_append_page_meta(shape, k_pool, block_table, old_lens, new_lens,
                                      max_new_tokens, meta, stream)
    _run("entmaxkv_append_page_meta", fn, args, events)


def entmaxkv_build_page_moments(shape: Shape, k_pool, block_table, seq_lens, moments,
                                stream=None, events=None):
    fn, args = _args_build_page_moments(shape, k_pool, block_table, seq_lens, moments, stream)
    _run("entmaxkv_build_page_moments", fn, args, events)


def entmaxkv_append_page_moments(shape: Shape, k_pool, block_table, old_lens, new_lens,
                                 max_new_tokens, moments, stream=None, events=None):
    fn, args = _args_append_page_moments(shape, k_pool, block_table, old_lens, new_lens,
                                         max_new_tokens, moments, stream)
    _run("entmaxkv_append_page_moments", fn, args, events)


def entmaxkv_gauss_select(shape: Shape, q, moments, block_table, seq_lens, alpha, delta,
                          cap_pages, sel, tau_hat=None, ws=None, stream=None, events=None):
    fn, args, _ = _args_gauss_select(shape, q, moments, block_table, seq_lens, alpha, delta,
                                     cap_pages, sel, tau_hat, ws, stream)
    _run("entmaxkv_gauss_select", fn, args, events)


def entmaxkv_score_select(shape: Shape, q, meta, block_table, seq_lens, budget_pages, sel,
                          sel_ub=None, ws=None, stream=None, events=None):
    fn, args, _ = _args_score_select(shape, q, meta, block_table, seq_lens, budget_pages, sel,
                                     sel_ub, ws, stream)
    _run("entmaxkv_score_select", fn, args, events)


def entmaxkv_score_select_noalloc(shape: Shape, q, meta, block_table, seq_lens, budget_pages,
                                  sel, sel_ub=None, stream=None, events=None):
    """entmaxkv_score_select with the library's static scratch in place of a
    workspace (allocates nothing; calls overlapping on one GPU race)."""
    fn, args = _args_score_select_noalloc(shape, q, meta, block_table, seq_lens, budget_pages,
                                          sel, sel_ub, stream)
    _run("entmaxkv_score_select_noalloc", fn, args, events)


def entmaxkv_decode_sparse(shape: Shape, q, k_pool, v_pool, block_table, seq_lens, sel,
                           budget_pages, alpha, out, tau=None, support=None, ws=None,
                           stream=None, events=None):
    fn, args, _ = _args_decode_sparse(shape, q, k_pool, v_pool, block_table, seq_lens, sel,
                                      budget_pages, alpha, out, tau, support, ws, stream)
    _run("entmaxkv_decode_sparse", fn, args, events)


def entmaxkv_decode_topk(shape: Shape, q, meta, k_pool, v_pool, block_table, seq_lens,
                         budget_pages, alpha, sel, out, sel_ub=None, tau=None, support=None,
                         ws=None, stream=None, events=None):
    """Bounds, top-k selection and sparse decode in one call (sel is written)."""
    fn, args, _ = _args_decode_topk(shape, q, meta, k_pool, v_pool, block_table, seq_lens,
                                    budget_pages, alpha, sel, out, sel_ub, tau, support, ws,
                                    stream)
    _run("entmaxkv_decode_topk", fn, args, events)


def entmaxkv_decode_full(shape: Shape, q, k_pool, v_pool, block_table, seq_lens, alpha, out,
                         tau=None, support=None, ws=None, stream=None, events=None):
    fn, args, _ = _args_decode_full(shape, q, k_pool, v_pool, block_table, seq_lens, alpha, out,
                                    tau, support, ws, stream)
    _run("entmaxkv_decode_full", fn, args, events)


class Prepared:
    """An entry point with its arguments marshalled once, for tight loops.
    The tensors must stay alive and unchanged in place while it is used.

        call = Prepared("decode_full", shape, q, k, v, bt, lens, 1.5, out, ws=ws)
        call()                 # or call(events=[e0, e1, e2, e3])
    """

    _makers = {"build_page_meta": _args_build_page_meta,
               "append_page_meta": _args_append_page_meta, "score_select": _args_score_select,
               "decode_sparse": _args_decode_sparse, "decode_topk": _args_decode_topk,
               "decode_full": _args_decode_full,
               "build_page_moments": _args_build_page_moments,
               "append_page_moments": _args_append_page_moments,
               "gauss_select": _args_gauss_select}

    def __init__(self, name: str, *args, **kwargs):
        r = Prepared._makers[name](*args, **kwargs)
        self.name = "entmaxkv_" + name
        self.fn, self.args = r[0], r[1]
        self.keep = (args, kwargs, r[2:] if len(r) > 2 else ())  # keep tensors alive
        self._ev_cache = {}

    def __call__(self, events=None):
        if events is None:
            rc = self.fn(*self.args)
        else:
            key = tuple(events)
            ev = self._ev_cache.get(key)
            if ev is None:
                ev = self._ev_cache[key] = _events(events)
            self.args[-1] = ev[0]
            rc = self.fn(*self.args)
            self.args[-1] = None
        if rc != ENTMAXKV_OK:
            raise EntmaxKVError(rc, self.name)


# ---------------------------------------------------------------------------
# HIP events for per-kernel timing (plumbing around hipEvent_t)


class HipEvents:
    """A set of timing-enabled hipEvent_t handles, passed as `events=`."""

    _hip = None

    def __init__(self, n: int):
        if HipEvents._hip is None:
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            HipEvents._hip = h
        self.handles = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = HipEvents._hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.handles.append(e.value)

    def record(self, i: int, stream) -> None:
        """Record event i on `stream` (a torch stream or a raw handle)."""
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        rc = HipEvents._hip.hipEventRecord(ctypes.c_void_p(self.handles[i]), ctypes.c_void_p(handle))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def __len__(self):
        return len(self.handles)

    def __iter__(self):
        return iter(self.handles)

    def elapsed_ms(self, i: int, j: int) -> float:
        out = ctypes.c_float()
        HipEvents._hip.hipEventSynchronize(ctypes.c_void_p(self.handles[j]))
        rc = HipEvents._hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.handles[i]),
                                                ctypes.c_void_p(self.handles[j]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def close(self):
        for e in self.handles:
            HipEvents._hip.hipEventDestroy(ctypes.c_void_p(e))
        self.handles = []
