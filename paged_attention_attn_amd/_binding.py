"""ctypes binding over ``libpaged_attention_attn.so``: argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it checks dtypes/devices/contiguity (an unsupported
input raises, it is never copied or routed elsewhere), allocates outputs with
torch when the caller passes none, and hands raw device pointers plus the
current HIP stream to the library.  If the library has not been built, every
call raises.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpaged_attention_attn.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "paged_attention_attn.h")

_lib = None


class DecodeCall(ctypes.Structure):
    """The C struct attn_decode_call: the arguments of one paged_attn_decode call."""
    _fields_ = [("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("num_seqs", ctypes.c_int), ("H", ctypes.c_int), ("Hkv", ctypes.c_int),
                ("d", ctypes.c_int), ("page_size", ctypes.c_int), ("max_pages_per_seq", ctypes.c_int),
                ("num_pages", ctypes.c_int), ("scale", ctypes.c_float), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("kv_fp8", ctypes.c_int), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float)]


def lib() -> ctypes.CDLL:
    """The loaded HIP library (loaded on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run `python -m paged_attention_attn_amd.build`)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
        L.attn_fwd.restype = i
        L.attn_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
        L.attn_fwd_f32.restype = i
        L.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
        L.attn_fwd_window.restype = i
        L.paged_attn_decode_workspace_size.argtypes = [i, i, i, i, i]
        L.paged_attn_decode_workspace_size.restype = sz
        L.paged_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, sz, vp]
        L.paged_attn_decode.restype = i
        L.paged_attn_decode_no_alloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
        L.paged_attn_decode_no_alloc.restype = i
        L.paged_attn_decode_fp8.argtypes = [vp, vp, vp, f, f, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, sz, vp]
        L.paged_attn_decode_fp8.restype = i
        L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, f, f, vp]
        L.attn_fwd_fp8.restype = i
        L.paged_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
        L.paged_prefill.restype = i
        L.paged_attn_decode_graph_create.argtypes = [ctypes.POINTER(DecodeCall), i, vp, ctypes.POINTER(ctypes.c_void_p)]
        L.paged_attn_decode_graph_create.restype = i
        L.paged_attn_decode_graph_launch.argtypes = [vp, vp]
        L.paged_attn_decode_graph_launch.restype = i
        L.paged_attn_decode_graph_destroy.argtypes = [vp]
        L.paged_attn_decode_graph_destroy.restype = i
        L.attn_status_string.argtypes = [i]
        L.attn_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions the public header declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:ATTN_API\s+)?(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise RuntimeError(f"paged_attention_attn error {rc}: {attn_status_string(rc)}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape(t, name, shape):
    """Raises ValueError unless t is a tensor of exactly this shape.  Shapes are checked before dtype and
    device, and the library sizes every write from q's shape, so an output of any other shape is refused
    rather than written past its end."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _dims(t, name, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")


def _require(t, name, dtype, ndim, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (no implicit copies)")


def _prefill(entry, dtype, q, k, v, causal, scale, out, lse, mask_args=None):
    _dims(q, "q", 4)
    _dims(k, "k", 4)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    _shape(k, "k", (B, Hkv, N, d))
    _shape(v, "v", (B, Hkv, N, d))
    if out is not None:
        _shape(out, "out", (B, H, N, d))
    if lse is not None:
        _shape(lse, "lse", (B, H, N))
    _require(q, "q", dtype, 4)
    _require(k, "k", dtype, 4, q.device)
    _require(v, "v", dtype, 4, q.device)
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", dtype, 4, q.device)
    if lse is not None:
        _require(lse, "lse", torch.float32, 3, q.device)
    if scale is None:
        scale = d ** -0.5
    mask = [int(bool(causal))] if mask_args is None else [int(x) for x in mask_args]
    _check(entry(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, N, d, *mask, float(scale),
                 _stream(q.device)))
    return out, lse


def attn_fwd(q, k, v, causal: bool, scale: float | None = None, out=None, lse=None):
    """bf16 attention forward: q [B,H,N,d], k/v [B,Hkv,N,d] -> (out [B,H,N,d] bf16, lse [B,H,N] fp32 or None)."""
    return _prefill(lib().attn_fwd, torch.bfloat16, q, k, v, causal, scale, out, lse)


def attn_fwd_window(q, k, v, window: int, n_global: int = 0, scale: float | None = None, out=None, lse=None):
    """bf16 causal attention where key j is visible to query i iff j <= i and (i - j < window or j < n_global)."""
    return _prefill(lib().attn_fwd_window, torch.bfloat16, q, k, v, True, scale, out, lse,
                    mask_args=(window, n_global))


def attn_fwd_fp8(q, k, v_t, causal: bool, scale: float | None = None, q_scale: float = 1.0, k_scale: float = 1.0,
                 v_scale: float = 1.0, out=None, lse=None):
    """FP8 attention (C: attn_fwd_fp8).  q [B,H,N,d], k [B,Hkv,N,d] and v_t [B,Hkv,d,N] (V transposed) hold
    E4M3 bytes (torch.uint8 or torch.float8_e4m3fn); the inputs are their values times the scales.
    Returns (O bf16 [B,H,N,d], LSE)."""
    fp8 = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
    _dims(q, "q", 4)
    _dims(k, "k", 4)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    _shape(k, "k", (B, Hkv, N, d))
    _shape(v_t, "v_t", (B, Hkv, d, N))
    if out is not None:
        _shape(out, "out", (B, H, N, d))
    if lse is not None:
        _shape(lse, "lse", (B, H, N))
    for t, name, nd in ((q, "q", 4), (k, "k", 4), (v_t, "v_t", 4)):
        if t.dtype not in fp8:
            raise TypeError(f"{name} must hold E4M3 bytes (torch.uint8 or torch.float8_e4m3fn)")
        _require(t, name, t.dtype, nd, q.device)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    _require(out, "out", torch.bfloat16, 4, q.device)
    if lse is not None:
        _require(lse, "lse", torch.float32, 3, q.device)
    if scale is None:
        scale = d ** -0.5
    _check(lib().attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v_t), _ptr(out), _ptr(lse), B, H, Hkv, N, d, int(bool(causal)),
                              float(scale), float(q_scale), float(k_scale), float(v_scale), _stream(q.device)))
    return out, lse


def attn_fwd_f32(q, k, v, causal: bool, scale: float | None = None, out=None, lse=None):
    """fp32 attention forward with the same shapes as :func:`attn_fwd`."""
    return _prefill(lib().attn_fwd_f32, torch.float32, q, k, v, causal, scale, out, lse)


def paged_prefill(q, k_new, v_new, k_cache, v_cache, block_table, ctx_lens, q_start, max_q_len: int | None = None,
                  scale: float | None = None, num_pages=None, out=None, lse=None):
    """Chunked prefill over a paged cache, appending the chunk (C: paged_prefill).

    q [T, H, d], k_new / v_new [T, Hkv, d] bf16 hold the chunks back to back (sequence s owns rows
    q_start[s] .. q_start[s+1]-1); k_cache / v_cache [num_pages, 16, Hkv, d] bf16 are updated in place;
    block_table [S, max_pages], ctx_lens [S], q_start [S + 1] int32 on the same device.  max_q_len
    bounds every chunk length (default T, known without reading the device).  Returns (O, LSE).
    """
    for t, name, nd in ((q, "q", 3), (k_cache, "k_cache", 4), (ctx_lens, "ctx_lens", 1),
                        (block_table, "block_table", 2)):
        _dims(t, name, nd)
    T, H, d = q.shape
    P, page_size, Hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError(f"k_cache's head dim {dk} differs from q's {d}")
    S = ctx_lens.shape[0]
    _shape(v_cache, "v_cache", tuple(k_cache.shape))
    _shape(k_new, "k_new", (T, Hkv, d))
    _shape(v_new, "v_new", (T, Hkv, d))
    _shape(block_table, "block_table", (S, block_table.shape[1]))
    _shape(q_start, "q_start", (S + 1,))
    if out is not None:
        _shape(out, "out", (T, H, d))
    if lse is not None:
        _shape(lse, "lse", (T, H))
    _require(q, "q", torch.bfloat16, 3)
    dev = q.device
    _require(k_new, "k_new", torch.bfloat16, 3, dev)
    _require(v_new, "v_new", torch.bfloat16, 3, dev)
    _require(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _require(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(ctx_lens, "ctx_lens", torch.int32, 1, dev)
    _require(q_start, "q_start", torch.int32, 1, dev)
    if max_q_len is None:
        max_q_len = T
    if num_pages is None:
        num_pages = P
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", torch.bfloat16, 3, dev)
    if lse is not None:
        _require(lse, "lse", torch.float32, 2, dev)
    if scale is None:
        scale = d ** -0.5
    _check(lib().paged_prefill(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                               _ptr(ctx_lens), _ptr(q_start), _ptr(out), _ptr(lse), S, H, Hkv, d, page_size,
                               block_table.shape[1], int(num_pages), int(max_q_len), float(scale), _stream(dev)))
    return out, lse


def paged_attn_decode_workspace_size(num_seqs: int, H: int, d: int, page_size: int, max_pages_per_seq: int) -> int:
    return int(lib().paged_attn_decode_workspace_size(num_seqs, H, d, page_size, max_pages_per_seq))


def _decode_args(q, k_cache, v_cache, block_table, seq_lens, scale, num_pages, workspace, out, lse,
                 cache_dtype=torch.bfloat16, need_workspace=True):
    """Checks the decode tensors and fills in the defaults; returns the C argument list (without a stream)."""
    for t, name, nd in ((q, "q", 3), (k_cache, "k_cache", 4), (block_table, "block_table", 2)):
        _dims(t, name, nd)
    S, H, d = q.shape
    P, page_size, Hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError(f"k_cache's head dim {dk} differs from q's {d}")
    max_pages = block_table.shape[1]
    _shape(v_cache, "v_cache", tuple(k_cache.shape))
    _shape(block_table, "block_table", (S, max_pages))
    _shape(seq_lens, "seq_lens", (S,))
    if out is not None:
        _shape(out, "out", (S, H, d))
    if lse is not None:
        _shape(lse, "lse", (S, H))
    _require(q, "q", torch.bfloat16, 3)
    dev = q.device
    _require(k_cache, "k_cache", cache_dtype, 4, dev)
    _require(v_cache, "v_cache", cache_dtype, 4, dev)
    _require(block_table, "block_table", torch.int32, 2, dev)
    _require(seq_lens, "seq_lens", torch.int32, 1, dev)
    if num_pages is None:
        num_pages = P
    if need_workspace:
        need = paged_attn_decode_workspace_size(S, H, d, page_size, max_pages)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        _require(workspace, "workspace", torch.uint8, 1, dev)
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", torch.bfloat16, 3, dev)
    if lse is not None:
        _require(lse, "lse", torch.float32, 2, dev)
    if scale is None:
        scale = d ** -0.5
    args = [_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse), S, H,
            Hkv, d, page_size, max_pages, int(num_pages), float(scale), _ptr(workspace),
            workspace.numel() if workspace is not None else 0]
    return args, workspace, out, lse


def paged_attn_decode(q, k_cache, v_cache, block_table, seq_lens, scale: float | None = None, num_pages=None,
                      workspace=None, out=None, lse=None):
    """Paged decode: q [S,H,d] bf16, caches [P,16,Hkv,d] bf16, block_table [S,max_pages] int32, seq_lens [S] int32.

    Returns (out [S,H,d] bf16, lse [S,H] fp32 or None).  ``workspace`` is a
    uint8 device tensor of at least paged_attn_decode_workspace_size() bytes
    (allocated here when not given).
    """
    args, _, out, lse = _decode_args(q, k_cache, v_cache, block_table, seq_lens, scale, num_pages, workspace, out,
                                     lse)
    _check(lib().paged_attn_decode(*args, _stream(q.device)))
    return out, lse


def paged_attn_decode_no_alloc(q, k_cache, v_cache, block_table, seq_lens, scale: float | None = None,
                               num_pages=None, out=None, lse=None):
    """:func:`paged_attn_decode` with the library's fixed per-GPU scratch as its workspace (C:
    paged_attn_decode_no_alloc): the C call allocates nothing.  Pass ``out`` (and ``lse``) to keep this
    wrapper from allocating them.  Calls that overlap on one GPU race on that scratch."""
    args, _, out, lse = _decode_args(q, k_cache, v_cache, block_table, seq_lens, scale, num_pages, None, out, lse,
                                     need_workspace=False)
    _check(lib().paged_attn_decode_no_alloc(*args[:15], _stream(q.device)))
    return out, lse


def paged_attn_decode_fp8(q, k_cache, v_cache, block_table, seq_lens, k_scale: float, v_scale: float,
                          scale: float | None = None, num_pages=None, workspace=None, out=None, lse=None):
    """Paged decode over an FP8 cache: caches [P,16,Hkv,d] uint8 holding E4M3 codes of the keys / values divided
    by k_scale / v_scale; q, block_table, seq_lens, workspace, out and lse as in :func:`paged_attn_decode`."""
    args, _, out, lse = _decode_args(q, k_cache, v_cache, block_table, seq_lens, scale, num_pages, workspace, out,
                                     lse, cache_dtype=torch.uint8)
    args = args[:3] + [float(k_scale), float(v_scale)] + args[3:]
    _check(lib().paged_attn_decode_fp8(*args, _stream(q.device)))
    return out, lse


class PagedDecodeGraph:
    """Decode calls captured once as a hipGraph (paged_attn_decode_graph_create) and replayed as one submission.

    ``calls`` is a list of dicts, one per paged_attn_decode call in order (say one per layer of a
    model's decode step), with the keyword names of :func:`paged_attn_decode` (q, k_cache, v_cache,
    block_table, seq_lens, and optionally scale, num_pages, workspace, out, lse).  Caches of dtype uint8 make
    the call a :func:`paged_attn_decode_fp8` call, whose k_scale and v_scale the dict then gives.  Tensors are
    the graph's fixed buffers: update the inputs in place between replays; every replay rewrites the
    outputs (``self.outputs[i]`` is call i's (out, lse)).  Missing workspaces and outputs are
    allocated here, at creation; a replay allocates nothing.
    """

    def __init__(self, calls, capture_stream=None):
        structs, self.outputs, self._keep = [], [], []
        for c in calls:
            fp8 = c["k_cache"].dtype == torch.uint8
            args, ws, out, lse = _decode_args(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"],
                                              c.get("scale"), c.get("num_pages"), c.get("workspace"), c.get("out"),
                                              c.get("lse"), cache_dtype=torch.uint8 if fp8 else torch.bfloat16)
            extra = [1, float(c["k_scale"]), float(c["v_scale"])] if fp8 else [0, 1.0, 1.0]
            structs.append(DecodeCall(*[a.value if isinstance(a, ctypes.c_void_p) else a for a in args], *extra))
            self.outputs.append((out, lse))
            self._keep.append((c, ws, out, lse))  # the graph holds their addresses
        if not structs:
            raise ValueError("at least one decode call is needed")
        self.device = calls[0]["q"].device
        self._stream = capture_stream if capture_stream is not None else torch.cuda.Stream(self.device)
        arr = (DecodeCall * len(structs))(*structs)
        handle = ctypes.c_void_p()
        self._handle = None
        _check(lib().paged_attn_decode_graph_create(arr, len(structs), ctypes.c_void_p(self._stream.cuda_stream),
                                                    ctypes.byref(handle)))
        self._handle = handle

    def replay(self, stream=None):
        """Enqueue one replay on ``stream`` (default: the current stream); returns the list of (out, lse)."""
        if self._handle is None:
            raise RuntimeError("graph not available")
        s = _stream(self.device) if stream is None else ctypes.c_void_p(stream.cuda_stream)
        _check(lib().paged_attn_decode_graph_launch(self._handle, s))
        return self.outputs

    def close(self):
        if self._handle is not None:
            torch.cuda.synchronize(self.device)
            _check(lib().paged_attn_decode_graph_destroy(self._handle))
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass
