"""HSTU jagged SiLU attention on AMD MI355X (gfx950).

A thin ctypes binding over ``libhstu.so`` (C ABI in ``include/hstu.h``). Every
function here only marshals arguments: it checks tensor placement, dtypes and
shapes, allocates the output and workspace through PyTorch, and calls the
library on the current HIP stream. All arithmetic runs in the library's HIP
kernels. If the library is missing, importing this package raises.

Functions mirror the C entry points by name:

* ``hstu_attn_fwd``        full causal path over jagged sequences
* ``hstu_kv_append``       paged KV append
* ``hstu_attn_fwd_cached`` new tokens against a cached, paged prefix
* ``hstu_mfalcon_fwd``     M-FALCON candidate scoring
* ``hstu_workspace_size``  workspace bytes of one call
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhstu.so")

HSTU_F32, HSTU_BF16 = 0, 1
HSTU_FN_FULL, HSTU_FN_CACHED, HSTU_FN_MFALCON, HSTU_FN_MFALCON_CACHED, HSTU_FN_FULL_BWD = 0, 1, 2, 3, 4
PAGE_SIZE = 64
HSTU_FLAG_FP32_NORM_INPUT = 1
HSTU_FLAG_SAVED_FORWARD = 2

EXPORTED_SYMBOLS = (
    "hstu_status_string", "hstu_version", "hstu_workspace_size", "hstu_attn_fwd",
    "hstu_kv_append", "hstu_attn_fwd_cached", "hstu_attn_fwd_cached_noalloc", "hstu_mfalcon_fwd",
    "hstu_mfalcon_fwd_cached", "hstu_attn_bwd",
    "hstu_layer_workspace_size", "hstu_matmul_bf16",
    "hstu_layer_fwd", "hstu_pm_create", "hstu_pm_destroy", "hstu_pm_reserve", "hstu_pm_commit", "hstu_pm_lookup",
    "hstu_pm_evict", "hstu_pm_stats",
)


class HstuError(RuntimeError):
    pass


class _Params(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("alpha", ctypes.c_float), ("norm_n", ctypes.c_int32),
        ("pos_tab", ctypes.c_void_p), ("n_pos", ctypes.c_int32), ("pos_head_stride", ctypes.c_int32),
        ("time_tab", ctypes.c_void_p), ("n_time", ctypes.c_int32), ("time_head_stride", ctypes.c_int32),
        ("ln_w", ctypes.c_void_p), ("ln_b", ctypes.c_void_p), ("ln_eps", ctypes.c_float),
        ("timing_events", ctypes.c_void_p * 4), ("flags", ctypes.c_int32),
    ]


class _KVCache(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p), ("ts_pages", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p), ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
    ]


class _Grads(ctypes.Structure):
    _fields_ = [("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p), ("du", ctypes.c_void_p),
                ("d_pos_tab", ctypes.c_void_p), ("d_time_tab", ctypes.c_void_p), ("d_ln_w", ctypes.c_void_p),
                ("d_ln_b", ctypes.c_void_p)]


class _LayerWeights(ctypes.Structure):
    _fields_ = [("embed_dim", ctypes.c_int32), ("w1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("products", ctypes.c_int32)]


HSTU_PRODUCTS_HIPBLASLT, HSTU_PRODUCTS_OWN, HSTU_PRODUCTS_AUTO = 0, 1, 2


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                          "or `python hstu_jagged_silu_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(_Params)
    K = ctypes.POINTER(_KVCache)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.hstu_status_string.restype = ctypes.c_char_p
    lib.hstu_status_string.argtypes = [ctypes.c_int]
    lib.hstu_version.restype = i32
    lib.hstu_version.argtypes = []
    lib.hstu_workspace_size.restype = sz
    lib.hstu_workspace_size.argtypes = [i32, P, i32, i64, i32]
    lib.hstu_attn_fwd.restype = ctypes.c_int
    lib.hstu_attn_fwd.argtypes = [P, i32, vp, i32, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hstu_attn_bwd.restype = ctypes.c_int
    lib.hstu_attn_bwd.argtypes = [P, i32, vp, i32, i64, vp, vp, vp, vp, vp, vp, ctypes.POINTER(_Grads), vp, sz, vp]
    lib.hstu_matmul_bf16.restype = ctypes.c_int
    lib.hstu_matmul_bf16.argtypes = [i64, i32, i32, vp, vp, vp, i32, i32, vp]
    lib.hstu_kv_append.restype = ctypes.c_int
    lib.hstu_kv_append.argtypes = [K, P, i32, vp, vp, i64, vp, vp, vp, vp]
    lib.hstu_attn_fwd_cached.restype = ctypes.c_int
    lib.hstu_attn_fwd_cached.argtypes = [P, i32, vp, vp, i32, i32, i64, vp, vp, vp, K, vp, vp, sz, vp]
    lib.hstu_attn_fwd_cached_noalloc.restype = ctypes.c_int
    lib.hstu_attn_fwd_cached_noalloc.argtypes = [P, i32, vp, vp, i32, i32, i64, vp, vp, vp, K, vp, vp]
    lib.hstu_mfalcon_fwd.restype = ctypes.c_int
    lib.hstu_mfalcon_fwd.argtypes = [P, i32, vp, vp, i32, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hstu_mfalcon_fwd_cached.restype = ctypes.c_int
    lib.hstu_mfalcon_fwd_cached.argtypes = [P, i32, vp, vp, i32, i32, i64, vp, vp, vp, vp, vp, K, vp, vp, sz, vp]
    lib.hstu_pm_create.restype = vp
    lib.hstu_pm_create.argtypes = [i32, i32, i32]
    lib.hstu_pm_destroy.restype = None
    lib.hstu_pm_destroy.argtypes = [vp]
    lib.hstu_pm_reserve.restype = ctypes.c_int
    lib.hstu_pm_reserve.argtypes = [vp, i32, vp, vp, vp, vp, ctypes.POINTER(i32)]
    lib.hstu_pm_commit.restype = ctypes.c_int
    lib.hstu_pm_commit.argtypes = [vp, i32, vp, vp]
    lib.hstu_pm_lookup.restype = i32
    lib.hstu_pm_lookup.argtypes = [vp, i64]
    lib.hstu_pm_evict.restype = ctypes.c_int
    lib.hstu_pm_evict.argtypes = [vp, i64]
    lib.hstu_pm_stats.restype = ctypes.c_int
    lib.hstu_pm_stats.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i64)]
    W = ctypes.POINTER(_LayerWeights)
    lib.hstu_layer_workspace_size.restype = sz
    lib.hstu_layer_workspace_size.argtypes = [P, i32, i32, i64, i32]
    lib.hstu_layer_fwd.restype = ctypes.c_int
    lib.hstu_layer_fwd.argtypes = [P, W, i32, vp, i32, i64, vp, vp, vp, vp, sz, vp]
    return lib


_lib = _load()


def lib():
    """The loaded ctypes library handle."""
    return _lib


def version() -> int:
    return int(_lib.hstu_version())


def status_string(code: int) -> str:
    return _lib.hstu_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise HstuError(f"{what}: {status_string(code)}")


# ---------------------------------------------------------------------------
# argument marshalling
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class LayerParams:
    """Layer parameters (C struct hstu_params_t). Tables are fp32 device tensors,
    shape [n] (shared by all heads) or [H, n] (one per head)."""
    num_heads: int
    head_dim: int
    dtype: torch.dtype = torch.bfloat16
    alpha: float = 1.0
    norm_n: int = 0
    pos_tab: Optional[torch.Tensor] = None
    time_tab: Optional[torch.Tensor] = None
    ln_w: Optional[torch.Tensor] = None
    ln_b: Optional[torch.Tensor] = None
    ln_eps: float = 1e-5
    flags: int = 0   # HSTU_FLAG_FP32_NORM_INPUT: fp32 attention output round trip instead of the norm-ready store;
    #                  HSTU_FLAG_SAVED_FORWARD: hstu_attn_bwd reuses the matching forward's workspace

    def c_struct(self, timing_events=None) -> _Params:
        p = _Params()
        p.num_heads = self.num_heads
        p.head_dim = self.head_dim
        p.dtype = {torch.bfloat16: HSTU_BF16, torch.float32: HSTU_F32}.get(self.dtype, -1)
        p.alpha = self.alpha
        p.norm_n = self.norm_n
        for name in ("pos_tab", "time_tab"):
            t = getattr(self, name)
            n_field = "n_pos" if name == "pos_tab" else "n_time"
            s_field = "pos_head_stride" if name == "pos_tab" else "time_head_stride"
            if t is None:
                setattr(p, name, None)
                setattr(p, n_field, 0)
                setattr(p, s_field, 0)
                continue
            _device_tensor(t, torch.float32, name)
            if t.dim() == 1:
                setattr(p, n_field, t.shape[0])
                setattr(p, s_field, 0)
            elif t.dim() == 2 and t.shape[0] == self.num_heads:
                setattr(p, n_field, t.shape[1])
                setattr(p, s_field, t.stride(0))
            else:
                raise ValueError(f"{name} must be [n] or [H, n]")
            setattr(p, name, t.data_ptr())
        for name in ("ln_w", "ln_b"):
            t = getattr(self, name)
            if t is not None:
                _device_tensor(t, torch.float32, name)
                if t.numel() != self.num_heads * self.head_dim:
                    raise ValueError(f"{name} must have H*d elements")
            setattr(p, name, None if t is None else t.data_ptr())
        p.ln_eps = self.ln_eps
        p.flags = self.flags
        if timing_events is not None:
            for i, ev in enumerate(timing_events[:4]):
                p.timing_events[i] = None if ev is None else ev.cuda_event
        return p


def _device_tensor(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def hstu_workspace_size(fn: int, params: LayerParams, batch: int, total_q_tokens: int, max_len: int) -> int:
    """Workspace bytes for one call of entry point ``fn`` (HSTU_FN_*)."""
    p = params.c_struct()
    n = int(_lib.hstu_workspace_size(fn, ctypes.byref(p), batch, total_q_tokens, max_len))
    if n == 0:
        raise HstuError("hstu_workspace_size: invalid arguments")
    return n


def _workspace(ws, nbytes, device):
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    _device_tensor(ws, torch.uint8, "workspace")
    if ws.numel() < nbytes:
        raise HstuError(f"workspace has {ws.numel()} bytes, {nbytes} needed")
    return ws


# Debug mode (HSTU_DEBUG=1 in the environment): content-check result word in
# the workspace header and its bits (include/hstu.h).
HSTU_WS_DEBUG_FLAG_OFFSET = 128
(HSTU_DEBUG_BAD_OFFSETS, HSTU_DEBUG_BAD_LENGTH, HSTU_DEBUG_BAD_CANDIDATES, HSTU_DEBUG_BAD_CACHE_LEN,
 HSTU_DEBUG_BAD_PAGE) = 1, 2, 4, 8, 16


def debug_flag(workspace) -> int:
    """The content-check bits the last debug-mode call wrote into `workspace`
    (waits for the current stream first); 0 means the content was valid."""
    torch.cuda.current_stream().synchronize()
    w = workspace[HSTU_WS_DEBUG_FLAG_OFFSET:HSTU_WS_DEBUG_FLAG_OFFSET + 4].cpu()
    return int(w.view(torch.int32)[0])


def _jagged_checks(params, q, k, v, u, ts, seq_offsets):
    H, d = params.num_heads, params.head_dim
    for name, t in (("q", q), ("k", k), ("v", v)):
        _device_tensor(t, params.dtype, name)
        if t.dim() != 3 or t.shape[1:] != (H, d):
            raise ValueError(f"{name} must be [T, {H}, {d}]")
    _device_tensor(u, params.dtype, "u")
    if u.shape != (q.shape[0], H * d):
        raise ValueError(f"u must be [T, {H * d}]")
    _device_tensor(ts, torch.int64, "ts")
    _device_tensor(seq_offsets, torch.int32, "seq_offsets")
    if ts.shape != (q.shape[0],):
        raise ValueError("ts must be [T]")


def hstu_attn_fwd(q, k, v, u, ts, seq_offsets, max_len: int, params: LayerParams, *, y=None,
                  workspace=None, timing_events=None):
    """Full causal path. q, k, v: [T, H, d]; u: [T, H*d]; ts int64 [T];
    seq_offsets int32 [B+1] on the GPU. Returns y [T, H*d]."""
    _jagged_checks(params, q, k, v, u, ts, seq_offsets)
    T, B = q.shape[0], seq_offsets.shape[0] - 1
    y = torch.empty_like(u) if y is None else y
    _device_tensor(y, params.dtype, "y")
    nbytes = hstu_workspace_size(HSTU_FN_FULL, params, B, T, max_len)
    ws = _workspace(workspace, nbytes, q.device)
    p = params.c_struct(timing_events)
    _check(_lib.hstu_attn_fwd(ctypes.byref(p), B, seq_offsets.data_ptr(), max_len, T, q.data_ptr(), k.data_ptr(),
                              v.data_ptr(), u.data_ptr(), ts.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(),
                              _stream()), "hstu_attn_fwd")
    return y


def hstu_attn_bwd(q, k, v, u, ts, seq_offsets, max_len: int, dy, params: LayerParams, *, workspace=None,
                  timing_events=None, table_grads: bool = True, affine_grads: bool = True):
    """Backward of hstu_attn_fwd for the upstream gradient dy [T, H*d].

    Returns a dict with dq, dk, dv ([T, H, d], bf16), du ([T, H*d], bf16),
    d_pos_tab / d_time_tab (fp32, shaped like the tables; None without a
    table or when table_grads is False) and d_ln_w / d_ln_b (fp32 [H*d]; None
    without the affine term or when affine_grads is False).

    With HSTU_FLAG_SAVED_FORWARD in params.flags, workspace must be the one
    that hstu_attn_fwd used with these same arguments (allocate it with
    hstu_workspace_size(HSTU_FN_FULL_BWD, ...) and pass it to both calls,
    with nothing else using it in between): the backward then reuses that
    forward's norm-ready output instead of recomputing the attention."""
    if (params.flags & HSTU_FLAG_SAVED_FORWARD) and workspace is None:
        raise ValueError("HSTU_FLAG_SAVED_FORWARD needs the forward call's workspace")
    _jagged_checks(params, q, k, v, u, ts, seq_offsets)
    _device_tensor(dy, params.dtype, "dy")
    if dy.shape != u.shape:
        raise ValueError("dy must have the shape of u")
    T, B = q.shape[0], seq_offsets.shape[0] - 1
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v), "du": torch.empty_like(u)}
    for name, src, want in (("d_pos_tab", params.pos_tab, table_grads), ("d_time_tab", params.time_tab, table_grads),
                            ("d_ln_w", params.ln_w, affine_grads), ("d_ln_b", params.ln_b, affine_grads)):
        out[name] = torch.empty_like(src) if (src is not None and want) else None
    g = _Grads(out["dq"].data_ptr(), out["dk"].data_ptr(), out["dv"].data_ptr(), out["du"].data_ptr(),
               _ptr(out["d_pos_tab"]), _ptr(out["d_time_tab"]), _ptr(out["d_ln_w"]), _ptr(out["d_ln_b"]))
    nbytes = hstu_workspace_size(HSTU_FN_FULL_BWD, params, B, T, max_len)
    ws = _workspace(workspace, nbytes, q.device)
    p = params.c_struct(timing_events)
    _check(_lib.hstu_attn_bwd(ctypes.byref(p), B, seq_offsets.data_ptr(), max_len, T, q.data_ptr(), k.data_ptr(),
                              v.data_ptr(), u.data_ptr(), ts.data_ptr(), dy.data_ptr(), ctypes.byref(g),
                              ws.data_ptr(), ws.numel(), _stream()), "hstu_attn_bwd")
    return out


def hstu_mfalcon_fwd(q, k, v, u, ts, seq_offsets, num_candidates, max_len: int, params: LayerParams, *, y=None,
                     workspace=None, timing_events=None):
    """M-FALCON: each user's rows are [history | candidates]; num_candidates int32 [B]."""
    _jagged_checks(params, q, k, v, u, ts, seq_offsets)
    _device_tensor(num_candidates, torch.int32, "num_candidates")
    T, B = q.shape[0], seq_offsets.shape[0] - 1
    y = torch.empty_like(u) if y is None else y
    _device_tensor(y, params.dtype, "y")
    nbytes = hstu_workspace_size(HSTU_FN_MFALCON, params, B, T, max_len)
    ws = _workspace(workspace, nbytes, q.device)
    p = params.c_struct(timing_events)
    _check(_lib.hstu_mfalcon_fwd(ctypes.byref(p), B, seq_offsets.data_ptr(), num_candidates.data_ptr(), max_len, T,
                                 q.data_ptr(), k.data_ptr(), v.data_ptr(), u.data_ptr(), ts.data_ptr(),
                                 y.data_ptr(), ws.data_ptr(), ws.numel(), _stream()), "hstu_mfalcon_fwd")
    return y


HSTU_EPI_NONE, HSTU_EPI_SILU_SPLIT = 0, 1


def hstu_matmul_bf16(a, b, *, epilogue: int = HSTU_EPI_NONE, split_width: int = 0, out=None):
    """C = A B on the library's MFMA kernel (bf16). a [M, K], b [K, N].
    HSTU_EPI_NONE returns [M, N]; HSTU_EPI_SILU_SPLIT returns [N / w, M, w]
    (SiLU, then column blocks of width w = split_width)."""
    _device_tensor(a, torch.bfloat16, "a")
    _device_tensor(b, torch.bfloat16, "b")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("a must be [M, K] and b [K, N]")
    M, K = a.shape
    N = b.shape[1]
    shape = (M, N) if epilogue == HSTU_EPI_NONE else (N // max(split_width, 1), M, split_width)
    out = torch.empty(shape, dtype=torch.bfloat16, device=a.device) if out is None else out
    _device_tensor(out, torch.bfloat16, "out")
    if out.numel() != M * N:
        raise ValueError("out has the wrong size")
    _check(_lib.hstu_matmul_bf16(M, N, K, a.data_ptr(), b.data_ptr(), out.data_ptr(), epilogue, split_width,
                                 _stream()), "hstu_matmul_bf16")
    return out


def hstu_layer_workspace_size(params: LayerParams, embed_dim: int, batch: int, total_tokens: int,
                              max_len: int) -> int:
    """Workspace bytes of one hstu_layer_fwd call."""
    p = params.c_struct()
    n = int(_lib.hstu_layer_workspace_size(ctypes.byref(p), embed_dim, batch, total_tokens, max_len))
    if n == 0:
        raise HstuError("hstu_layer_workspace_size: invalid arguments")
    return n


def hstu_layer_fwd(x, w1, w2, ts, seq_offsets, max_len: int, params: LayerParams, *, out=None,
                   workspace=None, timing_events=None, products: int = HSTU_PRODUCTS_AUTO):
    """Full layer: [U|V|Q|K] = SiLU(x w1), attention, out = A w2.

    x [T, E], w1 [E, 4*H*d], w2 [H*d, E], all bf16 on the GPU; ts int64 [T];
    seq_offsets int32 [B+1]. products: HSTU_PRODUCTS_AUTO (default: f1 on the
    library's MFMA kernel where it fits, f2 on hipBLASLt), HSTU_PRODUCTS_OWN
    (both on the library's kernel) or HSTU_PRODUCTS_HIPBLASLT. Returns out [T, E]."""
    H, d = params.num_heads, params.head_dim
    for name, t in (("x", x), ("w1", w1), ("w2", w2)):
        _device_tensor(t, params.dtype, name)
        if t.dim() != 2:
            raise ValueError(f"{name} must be 2-D")
    T, E = x.shape
    if w1.shape != (E, 4 * H * d) or w2.shape != (H * d, E):
        raise ValueError(f"w1 must be [{E}, {4 * H * d}] and w2 [{H * d}, {E}]")
    _device_tensor(ts, torch.int64, "ts")
    _device_tensor(seq_offsets, torch.int32, "seq_offsets")
    if ts.shape != (T,):
        raise ValueError("ts must be [T]")
    B = seq_offsets.shape[0] - 1
    out = torch.empty_like(x) if out is None else out
    _device_tensor(out, params.dtype, "out")
    nbytes = hstu_layer_workspace_size(params, E, B, T, max_len)
    ws = _workspace(workspace, nbytes, x.device)
    p = params.c_struct(timing_events)
    wts = _LayerWeights(E, w1.data_ptr(), w2.data_ptr(), products)
    _check(_lib.hstu_layer_fwd(ctypes.byref(p), ctypes.byref(wts), B, seq_offsets.data_ptr(), max_len, T,
                               x.data_ptr(), ts.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(), _stream()),
           "hstu_layer_fwd")
    return out


@dataclasses.dataclass
class PagedKVCache:
    """Caller-owned paged KV cache (C struct hstu_kv_cache_t).

    k_pages, v_pages: [num_pages, H, 64, d]; ts_pages: int64 [num_pages, 64];
    page_table: int32 [B, max_pages_per_seq] (-1 = none)."""
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    ts_pages: torch.Tensor
    page_table: torch.Tensor

    @staticmethod
    def empty(num_pages, num_heads, head_dim, page_table, dtype=torch.bfloat16, device="cuda"):
        k = torch.zeros(num_pages, num_heads, PAGE_SIZE, head_dim, dtype=dtype, device=device)
        v = torch.zeros_like(k)
        ts = torch.zeros(num_pages, PAGE_SIZE, dtype=torch.int64, device=device)
        return PagedKVCache(k, v, ts, page_table)

    def c_struct(self, params: LayerParams) -> _KVCache:
        H, d = params.num_heads, params.head_dim
        for name in ("k_pages", "v_pages"):
            t = getattr(self, name)
            _device_tensor(t, params.dtype, name)
            if t.dim() != 4 or t.shape[1:] != (H, PAGE_SIZE, d):
                raise ValueError(f"{name} must be [P, {H}, {PAGE_SIZE}, {d}]")
        _device_tensor(self.ts_pages, torch.int64, "ts_pages")
        _device_tensor(self.page_table, torch.int32, "page_table")
        if self.page_table.dim() != 2:
            raise ValueError("page_table must be [B, max_pages_per_seq]")
        c = _KVCache()
        c.k_pages, c.v_pages = self.k_pages.data_ptr(), self.v_pages.data_ptr()
        c.ts_pages, c.page_table = self.ts_pages.data_ptr(), self.page_table.data_ptr()
        c.num_pages = self.k_pages.shape[0]
        c.page_size = PAGE_SIZE
        c.max_pages_per_seq = self.page_table.shape[1]
        return c


def hstu_kv_append(cache: PagedKVCache, new_offsets, cache_lens, k_new, v_new, ts_new, params: LayerParams):
    """Write new tokens' K, V, ts at positions cache_lens[b] + m of each user's pages."""
    H, d = params.num_heads, params.head_dim
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _device_tensor(t, params.dtype, name)
        if t.dim() != 3 or t.shape[1:] != (H, d):
            raise ValueError(f"{name} must be [T, {H}, {d}]")
    _device_tensor(ts_new, torch.int64, "ts_new")
    _device_tensor(new_offsets, torch.int32, "new_offsets")
    _device_tensor(cache_lens, torch.int32, "cache_lens")
    c = cache.c_struct(params)
    p = params.c_struct()
    B = new_offsets.shape[0] - 1
    _check(_lib.hstu_kv_append(ctypes.byref(c), ctypes.byref(p), B, new_offsets.data_ptr(), cache_lens.data_ptr(),
                               k_new.shape[0], k_new.data_ptr(), v_new.data_ptr(), ts_new.data_ptr(), _stream()),
           "hstu_kv_append")


def hstu_attn_fwd_cached(q_new, u_new, ts_new, new_offsets, cache_lens, max_new: int, max_total: int,
                         cache: PagedKVCache, params: LayerParams, *, y=None, workspace=None,
                         timing_events=None):
    """New tokens (already appended) attend causally to the cached prefix and themselves."""
    H, d = params.num_heads, params.head_dim
    _device_tensor(q_new, params.dtype, "q_new")
    if q_new.dim() != 3 or q_new.shape[1:] != (H, d):
        raise ValueError(f"q_new must be [T, {H}, {d}]")
    _device_tensor(u_new, params.dtype, "u_new")
    _device_tensor(ts_new, torch.int64, "ts_new")
    _device_tensor(new_offsets, torch.int32, "new_offsets")
    _device_tensor(cache_lens, torch.int32, "cache_lens")
    T, B = q_new.shape[0], new_offsets.shape[0] - 1
    y = torch.empty_like(u_new) if y is None else y
    _device_tensor(y, params.dtype, "y")
    nbytes = hstu_workspace_size(HSTU_FN_CACHED, params, B, T, max_total)
    ws = _workspace(workspace, nbytes, q_new.device)
    c = cache.c_struct(params)
    p = params.c_struct(timing_events)
    _check(_lib.hstu_attn_fwd_cached(ctypes.byref(p), B, new_offsets.data_ptr(), cache_lens.data_ptr(), max_new,
                                     max_total, T, q_new.data_ptr(), u_new.data_ptr(), ts_new.data_ptr(),
                                     ctypes.byref(c), y.data_ptr(), ws.data_ptr(), ws.numel(), _stream()),
           "hstu_attn_fwd_cached")
    return y


def hstu_attn_fwd_cached_noalloc(q_new, u_new, ts_new, new_offsets, cache_lens, max_new: int, max_total: int,
                                 cache: PagedKVCache, params: LayerParams, y, *, timing_events=None):
    """hstu_attn_fwd_cached for callers that cannot allocate: no workspace
    argument (the library's per-GPU scratch of HSTU_NOALLOC_SCRATCH_BYTES is
    used) and the output y is required. Calls on one GPU must be ordered on
    one stream."""
    H, d = params.num_heads, params.head_dim
    _device_tensor(q_new, params.dtype, "q_new")
    if q_new.dim() != 3 or q_new.shape[1:] != (H, d):
        raise ValueError(f"q_new must be [T, {H}, {d}]")
    _device_tensor(u_new, params.dtype, "u_new")
    _device_tensor(ts_new, torch.int64, "ts_new")
    _device_tensor(new_offsets, torch.int32, "new_offsets")
    _device_tensor(cache_lens, torch.int32, "cache_lens")
    _device_tensor(y, params.dtype, "y")
    T, B = q_new.shape[0], new_offsets.shape[0] - 1
    c = cache.c_struct(params)
    p = params.c_struct(timing_events)
    _check(_lib.hstu_attn_fwd_cached_noalloc(ctypes.byref(p), B, new_offsets.data_ptr(), cache_lens.data_ptr(),
                                             max_new, max_total, T, q_new.data_ptr(), u_new.data_ptr(),
                                             ts_new.data_ptr(), ctypes.byref(c), y.data_ptr(), _stream()),
           "hstu_attn_fwd_cached_noalloc")
    return y


HSTU_NOALLOC_SCRATCH_BYTES = 64 << 20


def hstu_mfalcon_fwd_cached(q, k, v, u, ts, cand_offsets, hist_lens, max_cand: int, max_hist: int,
                            cache: PagedKVCache, params: LayerParams, *, y=None, workspace=None,
                            timing_events=None):
    """Candidates score against the users' paged histories (hist_lens int32 [B])
    and themselves. q, k, v: [T_cand, H, d]; u: [T_cand, H*d]; ts int64 [T_cand]."""
    H, d = params.num_heads, params.head_dim
    for name, t in (("q", q), ("k", k), ("v", v)):
        _device_tensor(t, params.dtype, name)
        if t.dim() != 3 or t.shape[1:] != (H, d):
            raise ValueError(f"{name} must be [T, {H}, {d}]")
    _device_tensor(u, params.dtype, "u")
    _device_tensor(ts, torch.int64, "ts")
    _device_tensor(cand_offsets, torch.int32, "cand_offsets")
    _device_tensor(hist_lens, torch.int32, "hist_lens")
    T, B = q.shape[0], cand_offsets.shape[0] - 1
    y = torch.empty_like(u) if y is None else y
    _device_tensor(y, params.dtype, "y")
    nbytes = hstu_workspace_size(HSTU_FN_MFALCON_CACHED, params, B, T, max_hist)
    ws = _workspace(workspace, nbytes, q.device)
    c = cache.c_struct(params)
    p = params.c_struct(timing_events)
    _check(_lib.hstu_mfalcon_fwd_cached(ctypes.byref(p), B, cand_offsets.data_ptr(), hist_lens.data_ptr(),
                                        max_cand, max_hist, T, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        u.data_ptr(), ts.data_ptr(), ctypes.byref(c), y.data_ptr(), ws.data_ptr(),
                                        ws.numel(), _stream()), "hstu_mfalcon_fwd_cached")
    return y


class PageManager:
    """Host-side page manager of the paged KV cache (hstu_pm_*): which pool
    pages hold which user's history, with LRU eviction. Page ids only; the
    bytes live in PagedKVCache pools (one per layer, same page ids)."""

    def __init__(self, num_pages: int, max_pages_per_seq: int, max_users: int):
        self._h = _lib.hstu_pm_create(num_pages, max_pages_per_seq, max_users)
        if not self._h:
            raise HstuError("hstu_pm_create: invalid arguments")
        self.num_pages, self.max_pages_per_seq, self.max_users = num_pages, max_pages_per_seq, max_users

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            try:
                _lib.hstu_pm_destroy(h)
            except Exception:  # interpreter shutdown
                pass
            self._h = None

    def reserve(self, user_ids, n_new):
        """Returns (cache_lens int32 [B], page_table int32 [B, max_pages], evicted)."""
        import numpy as np
        ids = np.ascontiguousarray(user_ids, dtype=np.int64)
        n = np.ascontiguousarray(n_new, dtype=np.int32)
        if ids.shape != n.shape or ids.ndim != 1:
            raise ValueError("user_ids and n_new must be 1-D of equal length")
        lens = np.zeros(len(ids), np.int32)
        table = np.full((len(ids), self.max_pages_per_seq), -1, np.int32)
        ev = ctypes.c_int32(0)
        _check(_lib.hstu_pm_reserve(self._h, len(ids), ids.ctypes.data, n.ctypes.data, lens.ctypes.data,
                                    table.ctypes.data, ctypes.byref(ev)), "hstu_pm_reserve")
        return lens, table, int(ev.value)

    def commit(self, user_ids, n_new):
        import numpy as np
        ids = np.ascontiguousarray(user_ids, dtype=np.int64)
        n = np.ascontiguousarray(n_new, dtype=np.int32)
        _check(_lib.hstu_pm_commit(self._h, len(ids), ids.ctypes.data, n.ctypes.data), "hstu_pm_commit")

    def lookup(self, user_id: int) -> int:
        return int(_lib.hstu_pm_lookup(self._h, int(user_id)))

    def evict(self, user_id: int):
        _check(_lib.hstu_pm_evict(self._h, int(user_id)), "hstu_pm_evict")

    def stats(self):
        fp, us, ev = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int64(0)
        _check(_lib.hstu_pm_stats(self._h, ctypes.byref(fp), ctypes.byref(us), ctypes.byref(ev)), "hstu_pm_stats")
        return {"free_pages": fp.value, "users": us.value, "evictions": ev.value}


class HipEvent:
    """A raw HIP event for the library's timing_events slots (torch's Event
    refuses elapsed times of events it did not record itself)."""
    _hip = None

    def __init__(self):
        if HipEvent._hip is None:
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            HipEvent._hip = h
        ev = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise HstuError("hipEventCreate failed")
        self.cuda_event = ev.value

    def record(self):
        if HipEvent._hip.hipEventRecord(self.cuda_event, _stream()) != 0:
            raise HstuError("hipEventRecord failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        if HipEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, end.cuda_event) != 0:
            raise HstuError("hipEventElapsedTime failed (events not recorded or not complete)")
        return float(ms.value)

    def __del__(self):
        hip = getattr(HipEvent, "_hip", None)
        if getattr(self, "cuda_event", None) and hip is not None:
            try:
                hip.hipEventDestroy(self.cuda_event)
            except Exception:  # interpreter shutdown
                pass
            self.cuda_event = None


def pair_count(kind: str, lengths: Sequence[int], extra: Optional[Sequence[int]] = None) -> int:
    """Allowed (query, key) pairs per head: the unit of algorithmic work (4*d FLOP each).

    full: sum L(L+1)/2; cached (lengths = new tokens, extra = cached prefix):
    sum M*C + M(M+1)/2; mfalcon (lengths = history, extra = candidates):
    sum n(n+1)/2 + m(n+1)."""
    tot = 0
    if kind == "full":
        for L in lengths:
            tot += L * (L + 1) // 2
    elif kind == "cached":
        for M, C in zip(lengths, extra):
            tot += M * C + M * (M + 1) // 2
    elif kind == "mfalcon":
        for n, m in zip(lengths, extra):
            tot += n * (n + 1) // 2 + m * (n + 1)
    else:
        raise ValueError(kind)
    return int(tot)
