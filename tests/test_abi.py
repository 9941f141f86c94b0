"""The C-ABI library on a host without a GPU: it loads, exports every
function include/attn_decode.h declares, and rejects bad arguments on the
host before any HIP call (no kernel is launched by these tests).

The argument checks are called with a stand-in device address (FAKE) that
is never dereferenced while a check refuses the call.  Should a check ever
let such a call through, it would launch on an unmapped address, so those
tests are host-only: they are skipped where a GPU is visible."""
import ctypes
import os
import re
import subprocess
import sys

import pytest
import torch

import decode_attention_kv_seq_amd as ad

host_only = pytest.mark.skipif(torch.cuda.device_count() > 0,
                               reason="stand-in device addresses: host-only")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_decode.h")

OK, NULL, DIM, ALIGN, WS, HIP = range(6)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return ad.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 20, names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(6):
        assert lib.attn_status_string(s)
    assert lib.attn_status_string(99) == b"unknown status"


def test_workspace_bytes(lib):
    assert ad.workspace_bytes(0, 4, 64, 128) == 0
    assert ad.workspace_bytes(1, 0, 64, 128) == 0
    assert ad.workspace_bytes(1, 4, 257, 128) == 0
    assert ad.workspace_bytes(1, 4, 64, 0) == 0
    for (B, H, D, S) in [(1, 4, 64, 128), (1, 32, 128, 32768), (64, 32, 128, 8192),
                         (1, 64, 64, 131072), (3, 5, 7, 11)]:
        n = ad.workspace_bytes(B, H, D, S)
        assert n > 0 and n % 256 == 0
        # room for at least one partial (m, l, o[D]) per (sequence, head)
        assert n >= B * H * (D + 2) * 4
        assert ad.workspace_bytes(B, H, D, S + 1000) >= n or S + 1000 > 2 ** 32
    # bounded: a few MiB for the largest single-GPU shapes here
    assert ad.workspace_bytes(1, 64, 64, 131072) < 16 << 20


FAKE = 0x100000  # a nonzero, 256-byte aligned address; never dereferenced


def call_single(lib, q=FAKE, k=FAKE, v=FAKE, out=FAKE, H=4, D=64, S=128, cp=100, dump=None,
                ws=FAKE, ws_bytes=1 << 30):
    return lib.attn_decode_f16(q, k, v, out, H, D, S, cp, dump, ws, ws_bytes, None)


@host_only
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(out=None), NULL),
    (dict(H=0), DIM), (dict(D=0), DIM), (dict(S=0), DIM), (dict(D=257), DIM),
    (dict(q=FAKE + 1), ALIGN), (dict(k=FAKE + 1), ALIGN), (dict(out=FAKE + 1), ALIGN),
    (dict(dump=FAKE + 2), ALIGN), (dict(ws=FAKE + 8), ALIGN),
    (dict(ws=None), WS), (dict(ws_bytes=16), WS),
])
def test_single_rejects_bad_arguments(lib, kw, code):
    assert call_single(lib, **kw) == code
    assert lib.attn_last_error().decode()


@host_only
def test_batched_rejects_bad_arguments(lib):
    f = lib.attn_decode_f16_batched
    assert f(FAKE, FAKE, FAKE, FAKE, None, 2, 4, 64, 128, None, FAKE, 1 << 30, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE + 2, 2, 4, 64, 128, None, FAKE, 1 << 30, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 64, 128, None, FAKE, 1 << 30, None) == DIM
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 70000, 4, 64, 128, None, FAKE, 1 << 40, None) == DIM
    need = ad.workspace_bytes(2, 4, 64, 128)
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 64, 128, None, FAKE, need - 1, None) == WS
    assert b"smaller" in lib.attn_last_error()


@host_only
def test_split_and_combine_reject_bad_arguments(lib):
    assert lib.attn_decode_f16_split(None, FAKE, FAKE, None, 5, 1, 4, 64, 128, None, FAKE,
                                     1 << 30, None) == NULL
    assert lib.attn_decode_f16_split(FAKE, FAKE, FAKE, None, 5, 1, 4, 300, 128, None, FAKE,
                                     1 << 30, None) == DIM
    assert lib.attn_decode_f16_combine(None, None, 5, 1, 4, 64, 128, FAKE, 1 << 30, None) == NULL
    assert lib.attn_decode_f16_combine(FAKE, None, 5, 1, 4, 64, 128, None, 1 << 30, None) == WS
    assert lib.attn_decode_f16_combine(FAKE + 1, None, 5, 1, 4, 64, 128, FAKE, 1 << 30,
                                       None) == ALIGN


@host_only
def test_error_text_is_per_call(lib):
    call_single(lib, D=0)
    a = lib.attn_last_error().decode()
    call_single(lib, ws=None)
    b = lib.attn_last_error().decode()
    assert "nonzero" in a and "workspace" in b


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(4, 64, dtype=torch.float16)
    k = torch.zeros(128, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        ad.decode(q, k, k, 100)
    with pytest.raises(TypeError):
        ad.decode(q, k.float(), k, 100)


@host_only
def test_paged_rejects_bad_arguments(lib):
    f = lib.attn_decode_f16_paged
    ok_args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, bt=FAKE, cp=FAKE, B=2, H=4, D=64, P=16,
                   MB=8, NB=16, dump=None, ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = dict(ok_args, **kw)
        return f(a["q"], a["k"], a["v"], a["out"], a["bt"], a["cp"], a["B"], a["H"], a["D"],
                 a["P"], a["MB"], a["NB"], a["dump"], a["ws"], a["wsb"], None)

    assert call(bt=None) == NULL
    assert call(cp=None) == NULL
    assert call(bt=FAKE + 2) == ALIGN
    assert call(P=12) == DIM
    assert call(P=0) == DIM
    assert call(MB=0) == DIM
    assert call(NB=0) == DIM
    assert call(P=65536, MB=1 << 16) == DIM        # capacity 2^32
    assert call(wsb=16) == WS
    assert call(D=300) == DIM


@host_only
def test_noalloc_rejects_bad_arguments(lib):
    """The allocation-free call: the usual checks, and sizes whose workspace
    exceeds the library's per-GPU array (ATTN_NOALLOC_SCRATCH_BYTES) refused
    with ATTN_ERR_WORKSPACE before any HIP call."""
    f = lib.attn_decode_f16_batched_noalloc
    assert f(FAKE, FAKE, FAKE, FAKE, None, 2, 4, 64, 128, None, None) == NULL
    assert f(None, FAKE, FAKE, FAKE, FAKE, 2, 4, 64, 128, None, None) == NULL
    assert f(FAKE, FAKE, FAKE, None, FAKE, 2, 4, 64, 128, None, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE + 1, FAKE, 2, 4, 64, 128, None, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE + 2, 2, 4, 64, 128, None, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 64, 128, None, None) == DIM
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 300, 128, None, None) == DIM
    assert ad.workspace_bytes(1024, 64, 128, 131072) > ad.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1024, 64, 128, 131072, None, None) == WS
    assert b"allocation-free" in lib.attn_last_error()
    # the workloads here fit
    for (B, H, D, S) in [(64, 32, 128, 8192), (1, 32, 128, 32768), (1, 64, 64, 131072),
                         (1024, 32, 128, 8192)]:
        assert 0 < ad.workspace_bytes(B, H, D, S) <= ad.NOALLOC_SCRATCH_BYTES


@host_only
def test_table_check_rejects_bad_arguments(lib):
    f = lib.attn_paged_table_check
    assert f(None, FAKE, 2, 16, 8, 16, FAKE, None) == NULL
    assert f(FAKE, None, 2, 16, 8, 16, FAKE, None) == NULL
    assert f(FAKE, FAKE, 2, 16, 8, 16, None, None) == NULL
    assert f(FAKE + 2, FAKE, 2, 16, 8, 16, FAKE, None) == ALIGN
    assert f(FAKE, FAKE, 2, 16, 8, 16, FAKE + 2, None) == ALIGN
    assert f(FAKE, FAKE, 0, 16, 8, 16, FAKE, None) == DIM
    assert f(FAKE, FAKE, 2, 12, 8, 16, FAKE, None) == DIM
    assert f(FAKE, FAKE, 2, 16, 0, 16, FAKE, None) == DIM
    assert f(FAKE, FAKE, 2, 16, 8, 0, FAKE, None) == DIM
    assert f(FAKE, FAKE, 2, 65536, 1 << 16, 16, FAKE, None) == DIM


def test_paged_generator_gathers_the_pool():
    from decode_attention_kv_seq_amd import workloads as wl
    import torch
    w = wl.Workload("t", n_heads=3, head_dim=8, seq_len=64, cur_pos=None, seed=9, batch=4,
                    page_size=8)
    kp, vp = wl.make_kv_paged(w)
    bt = w.block_table()
    assert sorted(bt.view(-1).tolist()) == list(range(w.num_blocks))
    for b in range(4):
        for h in range(3):
            _, k, v = wl.head_slice_paged(w, b, h)
            L = w.valid_len(b)
            dk = torch.stack([kp[bt[b, p // 8], p % 8, h] for p in range(L)])
            dv = torch.stack([vp[bt[b, p // 8], p % 8, h] for p in range(L)])
            assert torch.equal(dk, k.view(L, 8)) and torch.equal(dv, v.view(L, 8))


@host_only
def test_two_dispatch_rejects_bad_arguments(lib):
    assert lib.attn_qk_f16(None, FAKE, FAKE, 4, 64, 128, 5, None) == NULL
    assert lib.attn_qk_f16(FAKE, FAKE, FAKE + 1, 4, 64, 128, 5, None) == ALIGN
    assert lib.attn_qk_f16(FAKE, FAKE, FAKE, 4, 0, 128, 5, None) == DIM
    assert lib.attn_pv_f16(FAKE, FAKE, None, 4, 64, 128, 5, FAKE, 1 << 30, None) == NULL
    assert lib.attn_pv_f16(FAKE, FAKE, FAKE, 4, 64, 128, 5, None, 1 << 30, None) == WS
    assert lib.attn_pv_f16(FAKE, FAKE + 1, FAKE, 4, 64, 128, 5, FAKE, 1 << 30, None) == ALIGN


@host_only
def test_decode_step_rejects_bad_arguments(lib):
    f = lib.attn_decode_step_f16
    ok = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, out=FAKE, H=4, D=64, S=128, cp=100,
              dims=64, base=10000.0, trad=0, ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["out"], a["H"], a["D"], a["S"],
                 a["cp"], a["dims"], a["base"], a["trad"], a["ws"], a["wsb"], None)

    for name in ("q", "kn", "vn", "kc", "vc", "out"):
        assert call(**{name: None}) == NULL, name
        assert call(**{name: FAKE + 1}) == ALIGN, name
    assert call(dims=63) == DIM                     # odd
    assert call(dims=66) == DIM                     # past head_dim
    assert call(base=0.0) == DIM
    assert call(base=-2.0) == DIM
    assert call(base=float("nan")) == DIM
    assert call(base=float("inf")) == DIM
    assert call(cp=128) == DIM                      # the slot must exist
    assert b"slot" in lib.attn_last_error()
    assert call(D=0) == DIM
    assert call(ws=None) == WS
    assert call(wsb=16) == WS
    g = lib.attn_decode_step_f16_batched
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 2, 4, 64, 128, 64, 1e4, 0, FAKE, 1 << 30,
             None) == NULL
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, 2, 4, 64, 128, 64, 1e4, 0, FAKE,
             1 << 30, None) == ALIGN
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 64, 128, 65, 1e4, 0, FAKE, 1 << 30,
             None) == DIM


@host_only
def test_rope_rejects_bad_arguments(lib):
    f = lib.attn_rope_f16
    assert f(None, FAKE, FAKE, 2, 4, 64, 64, 1e4, 0, None) == NULL
    assert f(FAKE, FAKE, None, 2, 4, 64, 64, 1e4, 0, None) == NULL
    assert f(FAKE, FAKE + 1, FAKE, 2, 4, 64, 64, 1e4, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE + 2, 2, 4, 64, 64, 1e4, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, 2, 4, 64, 3, 1e4, 0, None) == DIM
    assert f(FAKE, FAKE, FAKE, 2, 4, 64, 64, 0.0, 0, None) == DIM
    assert f(FAKE, FAKE, FAKE, 0, 4, 64, 64, 1e4, 0, None) == DIM


@host_only
def test_softmax_rejects_bad_arguments(lib):
    f = lib.attn_softmax_f32
    need = ad.softmax_workspace_bytes(8, 5000)
    assert need >= 8 * 2 * 8 and need % 256 == 0
    assert ad.softmax_workspace_bytes(0, 5) == 0 and ad.softmax_workspace_bytes(5, 0) == 0
    assert f(None, FAKE, 8, 5000, FAKE, need, None) == NULL
    assert f(FAKE, None, 8, 5000, FAKE, need, None) == NULL
    assert f(FAKE, FAKE, 0, 5000, FAKE, need, None) == DIM
    assert f(FAKE, FAKE, 8, 0, FAKE, need, None) == DIM
    assert f(FAKE + 2, FAKE, 8, 5000, FAKE, need, None) == ALIGN
    assert f(FAKE, FAKE + 2, 8, 5000, FAKE, need, None) == ALIGN
    assert f(FAKE, FAKE, 8, 5000, FAKE + 8, need, None) == ALIGN
    assert f(FAKE, FAKE, 8, 5000, None, need, None) == WS
    assert f(FAKE, FAKE, 8, 5000, FAKE, need - 1, None) == WS
    assert f(FAKE, FAKE, 1 << 20, 1 << 31, FAKE, 1 << 40, None) == DIM


@host_only
def test_dispatch_limits(lib):
    """Calls whose launch would exceed the GPU's dispatch limit (2^32 - 1
    work-items per grid dimension) are refused with ATTN_ERR_DIM before any
    HIP call, though every other check passes: a paged batch that declares a
    2^31-position capacity over a small pool, more than 67108860 sequences x
    heads (the merge's grid), a softmax of 70 million one-column rows (one
    wave per row), the scores pass over 65536 heads x 2^31 positions; the
    plan query refuses the same sizes."""
    big = 1 << 62
    # paged, 1100 sequences (chunked grid) x 512 heads, capacity 65536 x 32768
    assert lib.attn_decode_f16_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1100, 512, 128, 65536, 32768,
                                     1, None, FAKE, big, None) == DIM
    assert b"dispatch limit" in lib.attn_last_error()
    # 64 heads stay within the limit per sequence, 9.2e9 workgroups in all
    assert ad.plan(1100, 64, 128, 1 << 31, 0, ad.PLAN_PAGED)["workgroups"] > 1 << 32
    with pytest.raises(ad.AttnError):
        ad.plan(1100, 512, 128, 1 << 31, 0, ad.PLAN_PAGED)
    # sequences x heads
    assert lib.attn_decode_workspace_bytes(65535, 1025, 8, 1) == 0
    assert lib.attn_decode_workspace_bytes(65535, 1024, 8, 1) > 0
    assert lib.attn_decode_f16_batched(FAKE, FAKE, FAKE, FAKE, FAKE, 65535, 1025, 8, 1, None,
                                       FAKE, big, None) == DIM
    # softmax: 70M rows of one column take a wave each
    assert lib.attn_softmax_f32(FAKE, FAKE, 70000000, 1, FAKE, big, None) == DIM
    assert b"dispatch limit" in lib.attn_last_error()
    # the scores pass and a single-sequence plan over 65536 heads x 2^31 positions
    assert lib.attn_qk_f16(FAKE, FAKE, FAKE, 65536, 1, 1 << 31, (1 << 31) - 1, None) == DIM
    with pytest.raises(ad.AttnError):
        ad.plan(1, 65536, 1, 1 << 31, (1 << 31) - 1, 0)


@host_only
def test_paged_step_rejects_bad_arguments(lib):
    f = lib.attn_decode_step_f16_paged

    def call(**kw):
        a = dict(q=FAKE, kn=FAKE, vn=FAKE, kp=FAKE, vp=FAKE, out=FAKE, bt=FAKE, cp=FAKE, B=2, H=4,
                 D=64, P=16, MB=8, NB=16, dims=64, base=1e4, trad=0, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return f(a["q"], a["kn"], a["vn"], a["kp"], a["vp"], a["out"], a["bt"], a["cp"], a["B"],
                 a["H"], a["D"], a["P"], a["MB"], a["NB"], a["dims"], a["base"], a["trad"],
                 a["ws"], a["wsb"], None)

    assert call(bt=None) == NULL
    assert call(cp=None) == NULL
    assert call(kn=None) == NULL
    assert call(P=12) == DIM
    assert call(dims=65) == DIM
    assert call(base=-1.0) == DIM
    assert call(out=FAKE + 1) == ALIGN
    assert call(wsb=16) == WS


@host_only
def test_header_and_library_from_c(tmp_path):
    """tests/c/abi_from_c.c, a strict C99 program (gcc -std=c99 -pedantic
    -Werror) that includes the header, links the library and checks its
    host-side answers; none of its calls reaches the GPU."""
    lib_dir = os.path.dirname(ad.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_from_c.c"),
           "-o", exe, "-L", lib_dir, "-lattn_decode", "-Wl,-rpath," + lib_dir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def test_missing_library_is_an_error():
    """No fallback: without the built library the binding raises ImportError."""
    saved = ad._lib
    ad._lib = None
    try:
        with pytest.raises(ImportError, match="not built"):
            ad.load_library(os.path.join(ROOT, "no_such_dir", "libattn_decode.so"))
    finally:
        ad._lib = saved


def test_host_tensors_are_refused():
    """Every call needs GPU tensors; host tensors are an error, never
    computed some other way."""
    import torch
    q = torch.zeros((4, 64), dtype=torch.float16)
    k = torch.zeros((128, 4, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensor"):
        ad.decode(q, k, k, 100)
    with pytest.raises(ValueError, match="GPU tensor"):
        ad.softmax(torch.zeros((2, 8), dtype=torch.float32))
