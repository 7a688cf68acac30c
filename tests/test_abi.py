"""CPU tests of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments on the host before anything is launched (no GPU needed,
and no call here reaches a launch)."""

from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import pytest
import torch

import paged_attention_attn_amd as paa
from paged_attention_attn_amd import _binding

ATTN_OK, NULL, SHAPE, HEAD_DIM, PAGE, WS, ALIGN, LARGE, GROUP, LAUNCH, SCALE, SCRATCH = range(12)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(paa.LIB_PATH):
        from paged_attention_attn_amd import build
        build.build()
    return paa.lib()


def test_exports_every_declared_symbol(L):
    names = paa.declared_functions()
    assert set(names) == {"attn_fwd", "attn_fwd_f32", "attn_fwd_fp8", "attn_fwd_window", "paged_attn_decode_workspace_size", "paged_prefill",
                          "paged_attn_decode", "paged_attn_decode_fp8", "paged_attn_decode_no_alloc",
                          "paged_attn_decode_graph_create",
                          "paged_attn_decode_graph_launch",
                          "paged_attn_decode_graph_destroy", "attn_status_string"}
    for n in names:
        assert hasattr(L, n), n


def test_exports_exactly_the_declared_symbols(L):
    """The library's dynamic symbol table defines the declared entry points and nothing else: no helper,
    no C++ internal, no compiler-generated global."""
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not installed")
    out = subprocess.run([nm, "-D", "--defined-only", paa.LIB_PATH], check=True, capture_output=True,
                         text=True).stdout
    defined = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert defined == set(paa.declared_functions())


def test_status_strings(L):
    for code in range(12):
        assert paa.attn_status_string(code) != "unknown status code"
    assert paa.attn_status_string(12345) == "unknown status code"


P = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,code", [
    ((None, P, P, P, None, 1, 2, 2, 8, 64, 1, 0.1), NULL),
    ((P, P, P, P, None, 1, 4, 3, 8, 64, 1, 0.1), SHAPE),
    ((P, P, P, P, None, -1, 2, 2, 8, 64, 1, 0.1), SHAPE),
    ((P, P, P, P, None, 1, 2, 2, 8, 96, 1, 0.1), HEAD_DIM),
    ((ctypes.c_void_p(0x10008), P, P, P, None, 1, 2, 2, 8, 64, 1, 0.1), ALIGN),
    ((P, P, P, P, None, 70000, 30000, 1, 100000, 128, 1, 0.1), LARGE),
    ((P, P, P, P, None, 1, 1, 1, 1 << 23, 128, 1, 0.1), LARGE),  # one K head of 2 GiB
    ((P, P, P, P, None, 0, 2, 2, 8, 64, 1, 0.1), ATTN_OK),   # empty batch: nothing to launch
    ((None, None, None, None, None, 0, 2, 2, 8, 64, 1, 0.1), ATTN_OK),  # empty: pointers unused
    ((P, P, P, P, None, 1, 2, 2, 0, 64, 1, 0.1), ATTN_OK),   # empty sequence
    ((P, P, P, P, None, 1, 2, 2, 8, 64, 1, 0.0), SCALE),
    ((P, P, P, P, None, 1, 2, 2, 8, 64, 1, -0.125), SCALE),
    ((P, P, P, P, None, 1, 2, 2, 8, 64, 1, float("nan")), SCALE),
    ((P, P, P, P, None, 1, 2, 2, 8, 64, 1, float("inf")), SCALE),
])
def test_prefill_validation(L, args, code):
    assert L.attn_fwd(*args, None) == code
    assert L.attn_fwd_f32(*args, None) == code


def test_window_validation(L):
    base = (P, P, P, P, None, 1, 2, 2, 8, 64)
    assert L.attn_fwd_window(*base, 0, 0, 0.1, None) == SHAPE       # window must be >= 1
    assert L.attn_fwd_window(*base, 4, -1, 0.1, None) == SHAPE      # n_global must be >= 0
    assert L.attn_fwd_window(*base, 4, 0, 0.0, None) == SCALE
    assert L.attn_fwd_window(None, P, P, P, None, 1, 2, 2, 8, 64, 4, 0, 0.1, None) == NULL
    assert L.attn_fwd_window(P, P, P, P, None, 0, 2, 2, 8, 64, 4, 0, 0.1, None) == ATTN_OK  # empty batch


def test_decode_validation(L):
    ws = paa.paged_attn_decode_workspace_size(4, 8, 128, 16, 10)
    base = dict(q=P, kc=P, vc=P, bt=P, lens=P, o=P, lse=None, S=4, H=8, Hkv=2, d=128, ps=16, mp=10, np_=100,
                scale=0.1, ws=P, wsb=ws)

    def call(**kw):
        a = dict(base, **kw)
        return L.paged_attn_decode(a["q"], a["kc"], a["vc"], a["bt"], a["lens"], a["o"], a["lse"], a["S"], a["H"],
                                   a["Hkv"], a["d"], a["ps"], a["mp"], a["np_"], a["scale"], a["ws"], a["wsb"], None)

    assert call(bt=None) == NULL
    assert call(ws=None) == NULL
    assert call(Hkv=3) == SHAPE
    assert call(d=80) == HEAD_DIM
    assert call(ps=32) == PAGE
    assert call(wsb=ws - 1) == WS
    assert call(H=64, Hkv=2, wsb=10 ** 9) == GROUP
    assert call(q=ctypes.c_void_p(0x10004)) == ALIGN
    assert call(scale=0.0) == SCALE
    assert call(scale=float("nan")) == SCALE
    assert call(S=0) == ATTN_OK
    assert call(S=0, q=None, ws=None) == ATTN_OK  # empty: pointers unused


def test_decode_no_alloc_validation(L):
    """The no-allocation decode checks what paged_attn_decode checks and refuses, before anything is
    launched, a call whose workspace would not fit its fixed 32 MiB scratch (no GPU needed)."""
    base = dict(q=P, kc=P, vc=P, bt=P, lens=P, o=P, lse=None, S=4, H=8, Hkv=2, d=128, ps=16, mp=10, np_=100,
                scale=0.1)

    def call(**kw):
        a = dict(base, **kw)
        return L.paged_attn_decode_no_alloc(a["q"], a["kc"], a["vc"], a["bt"], a["lens"], a["o"], a["lse"], a["S"],
                                            a["H"], a["Hkv"], a["d"], a["ps"], a["mp"], a["np_"], a["scale"], None)

    assert call(bt=None) == NULL
    assert call(Hkv=3) == SHAPE
    assert call(d=80) == HEAD_DIM
    assert call(ps=32) == PAGE
    assert call(H=64, Hkv=2) == GROUP
    assert call(q=ctypes.c_void_p(0x10004)) == ALIGN
    assert call(scale=0.0) == SCALE
    assert call(S=0) == ATTN_OK and call(S=0, q=None) == ATTN_OK
    limit = 32 << 20
    # the largest batch of 32-head sequences whose workspace fits, and one more sequence
    fits = max(S for S in range(1, 2000) if paa.paged_attn_decode_workspace_size(S, 32, 128, 16, 1024) <= limit)
    assert fits * 32 >= 31000
    assert call(S=fits + 1, H=32, Hkv=8, mp=1024, np_=40000) == SCRATCH
    assert call(S=100000, H=32, Hkv=8, mp=1024, np_=40000) == SCRATCH


def test_decode_fp8_validation(L):
    """The FP8 decode checks what the bf16 decode checks, plus both cache scales (no GPU needed)."""
    ws = paa.paged_attn_decode_workspace_size(4, 8, 128, 16, 10)
    base = dict(q=P, kc=P, vc=P, ks=0.5, vs=0.25, bt=P, lens=P, o=P, lse=None, S=4, H=8, Hkv=2, d=128, ps=16,
                mp=10, np_=100, scale=0.1, ws=P, wsb=ws)

    def call(**kw):
        a = dict(base, **kw)
        return L.paged_attn_decode_fp8(a["q"], a["kc"], a["vc"], a["ks"], a["vs"], a["bt"], a["lens"], a["o"],
                                       a["lse"], a["S"], a["H"], a["Hkv"], a["d"], a["ps"], a["mp"], a["np_"],
                                       a["scale"], a["ws"], a["wsb"], None)

    assert call(kc=None) == NULL
    assert call(Hkv=3) == SHAPE
    assert call(d=96) == HEAD_DIM
    assert call(ps=8) == PAGE
    assert call(wsb=ws - 1) == WS
    assert call(vc=ctypes.c_void_p(0x10008)) == ALIGN
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert call(ks=bad) == SCALE and call(vs=bad) == SCALE
    assert call(S=0) == ATTN_OK


def test_decode_graph_validation(L):
    """Argument errors come back before any capture begins (no GPU needed)."""
    ws = paa.paged_attn_decode_workspace_size(4, 8, 128, 16, 10)
    handle = ctypes.c_void_p(0x1234)
    S = ctypes.c_void_p(0x20000)  # a stand-in stream handle: never used, every call fails validation first

    def call(**kw):
        a = dict(q=0x10000, k_cache=0x10000, v_cache=0x10000, block_table=0x10000, seq_lens=0x10000, o=0x10000,
                 lse=None, num_seqs=4, H=8, Hkv=2, d=128, page_size=16, max_pages_per_seq=10, num_pages=100,
                 scale=0.1, workspace=0x10000, workspace_bytes=ws)
        a.update(kw)
        return _binding.DecodeCall(**a)

    def create(calls, stream=S):
        arr = (_binding.DecodeCall * len(calls))(*calls)
        return L.paged_attn_decode_graph_create(arr, len(calls), stream, ctypes.byref(handle))

    assert create([call()], stream=None) == NULL
    assert handle.value is None  # cleared on error
    assert create([call(), call(page_size=32)]) == PAGE  # every call is checked
    assert create([call(d=96)]) == HEAD_DIM
    assert create([call(workspace_bytes=ws - 1)]) == WS
    assert create([call(scale=-1.0)]) == SCALE
    assert create([call(block_table=None)]) == NULL
    assert create([call(kv_fp8=2)]) == SHAPE
    assert create([call(q=0x10004)]) == ALIGN  # the graph checks exactly what an eager call checks
    assert create([call(max_pages_per_seq=1 << 28)]) == LARGE  # token positions past 2^31
    assert create([call(kv_fp8=1, k_scale=0.0, v_scale=1.0)]) == SCALE  # an FP8 call's scales are checked
    assert create([call(kv_fp8=1, k_scale=1.0, v_scale=float("nan"))]) == SCALE
    assert create([call(kv_fp8=0, k_scale=0.0, v_scale=0.0), call(d=96)]) == HEAD_DIM  # ... a bf16 call's are not
    arr = (_binding.DecodeCall * 1)(call())
    assert L.paged_attn_decode_graph_create(arr, 0, S, ctypes.byref(handle)) == SHAPE
    assert L.paged_attn_decode_graph_create(None, 1, S, ctypes.byref(handle)) == NULL
    assert L.paged_attn_decode_graph_create(arr, 1, S, None) == NULL
    assert L.paged_attn_decode_graph_launch(None, None) == NULL
    assert L.paged_attn_decode_graph_destroy(None) == ATTN_OK


def test_workspace_linear_in_length(L):
    """Workspace memory grows linearly with the longest sequence, never quadratically."""
    sizes = [paa.paged_attn_decode_workspace_size(64, 32, 128, 16, mp) for mp in (64, 128, 256, 512, 1024)]
    for a, b in zip(sizes, sizes[1:]):
        assert b <= 2.0 * a + 512
    assert paa.paged_attn_decode_workspace_size(64, 32, 96, 16, 10) == 0


def test_product_path_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _binding.lib()


def test_paged_prefill_validation(L):
    """Argument errors of the chunked paged prefill come back on the host; empty calls are valid."""
    # q, k_new, v_new, k_cache, v_cache, block_table, ctx_lens, q_start, o, lse
    ptrs = [P] * 8 + [P, None]

    def call(num_seqs=2, H=8, Hkv=2, d=128, page_size=16, max_pages=4, num_pages=10, max_q_len=33, scale=0.1,
             p=None):
        return L.paged_prefill(*(p or ptrs), num_seqs, H, Hkv, d, page_size, max_pages, num_pages, max_q_len, scale,
                               None)

    assert call(H=6, Hkv=4) == SHAPE
    assert call(num_seqs=-1) == SHAPE
    assert call(max_q_len=-1) == SHAPE
    assert call(max_pages=0) == SHAPE
    assert call(num_pages=0) == SHAPE
    assert call(d=96) == HEAD_DIM
    assert call(page_size=32) == PAGE
    assert call(scale=float("nan")) == SCALE
    assert call(p=[None] * 10, num_seqs=0) == ATTN_OK  # empty batch
    assert call(p=[None] * 10, max_q_len=0) == ATTN_OK  # empty chunks
    for i in range(9):  # every pointer but lse is required
        p = list(ptrs)
        p[i] = None
        assert call(p=p) == NULL, i
    p = list(ptrs)
    p[3] = ctypes.c_void_p(0x10008)  # k_cache not 16-byte aligned
    assert call(p=p) == ALIGN
    assert call(max_pages=1 << 28) == LARGE
    assert call(Hkv=8, max_q_len=1 << 20) == LARGE  # one sequence's chunk rows of k_new: 2 GiB


def test_fp8_validation(L):
    """FP8 prefill: the bf16 rules, plus N a multiple of 16 and three finite positive tensor scales."""
    base = (P, P, P, P, None, 1, 8, 2, 64, 128, 1, 0.1)
    assert L.attn_fwd_fp8(P, P, P, P, None, 1, 8, 2, 40, 128, 1, 0.1, 1.0, 1.0, 1.0, None) == SHAPE  # N % 16
    assert L.attn_fwd_fp8(P, P, P, P, None, 1, 8, 3, 64, 128, 1, 0.1, 1.0, 1.0, 1.0, None) == SHAPE
    assert L.attn_fwd_fp8(P, P, P, P, None, 1, 8, 2, 64, 96, 1, 0.1, 1.0, 1.0, 1.0, None) == HEAD_DIM
    for bad in ((0.0, 1.0, 1.0), (1.0, -1.0, 1.0), (1.0, 1.0, float("inf"))):
        assert L.attn_fwd_fp8(*base, *bad, None) == SCALE
    assert L.attn_fwd_fp8(None, P, P, P, None, 1, 8, 2, 64, 128, 1, 0.1, 1.0, 1.0, 1.0, None) == NULL
    assert L.attn_fwd_fp8(None, None, None, None, None, 0, 8, 2, 64, 128, 1, 0.1, 1.0, 1.0, 1.0, None) == ATTN_OK


# ---- the Python binding refuses output buffers of the wrong shape (before any device check) ----

def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _expect_shape_error(fn, name):
    with pytest.raises(ValueError, match=f"{name} must have shape"):
        fn()


def _expect_device_error(fn):
    with pytest.raises(ValueError, match="must be on a GPU"):
        fn()


def test_binding_prefill_output_shapes():
    q, k, v = _bf(1, 4, 8, 64), _bf(1, 2, 8, 64), _bf(1, 2, 8, 64)
    for entry in (paa.attn_fwd, lambda *a, **kw: paa.attn_fwd_window(*a[:3], 4, 0, **kw)):
        call = lambda **kw: entry(q, k, v, True, **kw) if entry is paa.attn_fwd else entry(q, k, v, **kw)  # noqa
        _expect_shape_error(lambda: call(out=_bf(1, 4, 7, 64)), "out")
        _expect_shape_error(lambda: call(lse=torch.zeros(1, 4, 7)), "lse")
        _expect_shape_error(lambda: call(lse=torch.zeros(4, 8)), "lse")
        _expect_device_error(lambda: call(out=_bf(1, 4, 8, 64), lse=torch.zeros(1, 4, 8)))
    _expect_shape_error(lambda: paa.attn_fwd(q, _bf(1, 2, 9, 64), v, True), "k")
    _expect_shape_error(lambda: paa.attn_fwd(q, k, _bf(1, 2, 8, 32), True), "v")
    f = lambda t: torch.zeros(t, dtype=torch.float32)  # noqa: E731
    _expect_shape_error(lambda: paa.attn_fwd_f32(f((1, 4, 8, 64)), f((1, 2, 8, 64)), f((1, 2, 8, 64)), True,
                                                 out=f((1, 4, 8, 32))), "out")


def test_binding_fp8_output_shapes():
    u = lambda *s: torch.zeros(s, dtype=torch.uint8)  # noqa: E731
    q, k, vt = u(1, 4, 16, 64), u(1, 2, 16, 64), u(1, 2, 64, 16)
    _expect_shape_error(lambda: paa.attn_fwd_fp8(q, k, vt, True, out=_bf(1, 4, 15, 64)), "out")
    _expect_shape_error(lambda: paa.attn_fwd_fp8(q, k, vt, True, lse=torch.zeros(1, 4, 15)), "lse")
    _expect_shape_error(lambda: paa.attn_fwd_fp8(q, k, u(1, 2, 16, 64), True), "v_t")
    _expect_device_error(lambda: paa.attn_fwd_fp8(q, k, vt, True, out=_bf(1, 4, 16, 64),
                                                  lse=torch.zeros(1, 4, 16)))


def test_binding_decode_output_shapes():
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)  # noqa: E731
    q, kc, vc, bt, lens = _bf(3, 8, 128), _bf(10, 16, 2, 128), _bf(10, 16, 2, 128), i32(3, 4), i32(3)
    for entry, extra in ((paa.paged_attn_decode, ()), ):
        _expect_shape_error(lambda: entry(q, kc, vc, bt, lens, *extra, out=_bf(2, 8, 128)), "out")
        _expect_shape_error(lambda: entry(q, kc, vc, bt, lens, *extra, lse=torch.zeros(3, 4)), "lse")
        _expect_shape_error(lambda: entry(q, kc, vc, bt, i32(2), *extra), "seq_lens")
        _expect_shape_error(lambda: entry(q, kc, vc, i32(2, 4), lens, *extra), "block_table")
        _expect_shape_error(lambda: entry(q, kc, _bf(10, 16, 2, 64), bt, lens, *extra), "v_cache")
        _expect_device_error(lambda: entry(q, kc, vc, bt, lens, *extra, out=_bf(3, 8, 128),
                                           lse=torch.zeros(3, 8)))
    u8 = torch.zeros((10, 16, 2, 128), dtype=torch.uint8)
    _expect_shape_error(lambda: paa.paged_attn_decode_fp8(q, u8, u8, bt, lens, 1.0, 1.0, out=_bf(3, 8, 64)), "out")
    _expect_shape_error(lambda: paa.paged_attn_decode_fp8(q, u8, u8, bt, lens, 1.0, 1.0,
                                                          lse=torch.zeros(8, 3)), "lse")
    with pytest.raises(ValueError, match="out must have shape"):  # a graph call is checked the same way
        paa.PagedDecodeGraph([dict(q=q, k_cache=kc, v_cache=vc, block_table=bt, seq_lens=lens, out=_bf(3, 8, 64))])


def test_binding_paged_prefill_output_shapes():
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)  # noqa: E731
    q, kn, vn = _bf(20, 8, 64), _bf(20, 2, 64), _bf(20, 2, 64)
    kc, vc, bt, ctx, qs = _bf(10, 16, 2, 64), _bf(10, 16, 2, 64), i32(2, 5), i32(2), i32(3)
    call = lambda **kw: paa.paged_prefill(q, kn, vn, kc, vc, bt, ctx, qs, **kw)  # noqa: E731
    _expect_shape_error(lambda: call(out=_bf(20, 8, 32)), "out")
    _expect_shape_error(lambda: call(lse=torch.zeros(20, 4)), "lse")
    _expect_shape_error(lambda: paa.paged_prefill(q, kn, vn, kc, vc, bt, ctx, i32(2)), "q_start")
    _expect_shape_error(lambda: paa.paged_prefill(q, _bf(19, 2, 64), vn, kc, vc, bt, ctx, qs), "k_new")
    _expect_device_error(lambda: call(out=_bf(20, 8, 64), lse=torch.zeros(20, 8)))


# ---- host-side sanitizer build of the C ABI ----

HERE = os.path.dirname(os.path.abspath(__file__))
ROCM = "/opt/rocm"
# instrumentation for the host pass of abi.hip only (device code is compiled as usual)
HOST_SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()
LINK_SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def test_abi_host_code_under_asan_and_ubsan(L, tmp_path):
    """abi.hip's host code built with AddressSanitizer and UndefinedBehaviorSanitizer, driven through every
    entry point's argument checks (tests/abi_host_check.cpp), including size arithmetic near its overflow
    limits: no report, no leak, and every status as expected.  Nothing is launched."""
    from paged_attention_attn_amd import build as B
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(B.HIPCC) and os.path.exists(clangxx)):
        pytest.skip("ROCm compilers not installed")
    objs = [os.path.join(B.BUILD, n + ".o") for n in ("prefill_bf16", "prefill_fp8", "prefill_f32", "paged_decode")]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    abi_o = str(tmp_path / "abi_sanitized.o")
    exe = str(tmp_path / "abi_host_check")
    compile_cmd = [B.HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SANITIZE,
                   "-c", os.path.join(B.CSRC, "abi.hip"), "-o", abi_o]
    r = subprocess.run(compile_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    link_cmd = [clangxx, "-std=c++17", "-O1", "-g", *LINK_SANITIZE, "-I" + os.path.join(ROCM, "include"),
                "-D__HIP_PLATFORM_AMD__", os.path.join(HERE, "abi_host_check.cpp"), abi_o, *objs,
                "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    r = subprocess.run(link_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "abi host checks passed" in r.stdout, r.stdout + r.stderr
