"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from hybrid_linear_attention_gdn_amd import _lib as L
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "sanawm_gdn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libsanawm_gdn.so is not built (run __graft_entry__.build())")
    return L.load()


def test_exports_every_declared_symbol(lib):
    decl = _declared_functions()
    assert set(decl) == set(L.EXPORTED), decl
    for name in decl:
        assert hasattr(lib, name), name
    assert lib.gdn_version() == 1
    assert lib.gdn_chunk_len() == 80
    assert lib.gdn_status_string(L.GDN_ERR_WORKSPACE) == b"GDN_ERR_WORKSPACE"


def _p(**kw):
    d = dict(batch=1, seq_len=160, num_heads=20, head_dim_k=112, head_dim_v=112, qkv_dtype=L.GDN_BF16,
             o_dtype=L.GDN_F32, flags=0)
    d.update(kw)
    return L.Problem(**d)


def _ws(lib, p):
    n = ctypes.c_size_t(123)
    st = lib.gdn_workspace_bytes(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


def test_workspace_bytes(lib):
    st, n = _ws(lib, _p())
    assert st == L.GDN_OK and n > 0 and n % 256 == 0
    st0, n0 = _ws(lib, _p(seq_len=0))
    assert st0 == L.GDN_OK and n0 == 0
    st2, n2 = _ws(lib, _p(seq_len=320))
    assert n2 > n
    stp, np_ = _ws(lib, _p(qkv_dtype=L.GDN_F32, head_dim_k=64, head_dim_v=32))
    assert stp == L.GDN_OK and np_ > 0
    lay = L.WorkspaceLayout()
    assert lib.gdn_workspace_layout(ctypes.byref(_p()), ctypes.byref(lay)) == L.GDN_OK
    # MFMA path: a ring of two chunk ranges of records per head, then the carried state
    assert lay.total == n and lay.mfma == 1 and lay.rec < lay.carry < lay.total
    assert lay.range_cap == 2 and lay.first_range == 2  # T = 160: two chunks
    assert lay.carry - lay.rec >= 2 * lay.range_cap * 20 * lay.rec_bytes
    assert lay.total - lay.carry >= 20 * 112 * 112 * 4
    lay_l = L.WorkspaceLayout()
    assert lib.gdn_workspace_layout(ctypes.byref(_p(seq_len=80 * 500)), ctypes.byref(lay_l)) == 0
    assert lay_l.range_cap == 48 and lay_l.first_range == 25
    assert lay_l.total < 2 * 48 * 20 * lay.rec_bytes + 20 * 112 * 112 * 4 + 4096  # bounded in T
    lay_p = L.WorkspaceLayout()
    assert lib.gdn_workspace_layout(ctypes.byref(_p(qkv_dtype=L.GDN_F32)), ctypes.byref(lay_p)) == 0
    assert lay_p.mfma == 0 and lay_p.beta < lay_p.rq < lay_p.rk < lay_p.gcum < lay_p.total


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), L.GDN_ERR_INVALID_ARGUMENT),
    (dict(seq_len=-1), L.GDN_ERR_INVALID_ARGUMENT),
    (dict(num_heads=0), L.GDN_ERR_INVALID_ARGUMENT),
    (dict(head_dim_k=0), L.GDN_ERR_INVALID_ARGUMENT),
    (dict(qkv_dtype=7), L.GDN_ERR_INVALID_ARGUMENT),
    (dict(o_dtype=-1), L.GDN_ERR_INVALID_ARGUMENT),
    (dict(flags=64), L.GDN_ERR_INVALID_ARGUMENT),
    (dict(qkv_dtype=L.GDN_F32, head_dim_k=129), L.GDN_ERR_UNSUPPORTED),
    (dict(qkv_dtype=L.GDN_F32, head_dim_v=200), L.GDN_ERR_UNSUPPORTED),
    (dict(flags=4), L.GDN_ERR_INVALID_ARGUMENT),  # the retired portable-kernel bit
    (dict(batch=1 << 20, num_heads=1 << 10), L.GDN_ERR_UNSUPPORTED),
])
def test_bad_problems(lib, kw, status):
    st, _ = _ws(lib, _p(**kw))
    assert st == status
    assert lib.gdn_last_error()


def test_null_problem_and_outputs(lib):
    n = ctypes.c_size_t(0)
    assert lib.gdn_workspace_bytes(None, ctypes.byref(n)) == L.GDN_ERR_INVALID_ARGUMENT
    assert lib.gdn_workspace_bytes(ctypes.byref(_p()), None) == L.GDN_ERR_INVALID_ARGUMENT
    assert lib.gdn_workspace_layout(ctypes.byref(_p()), None) == L.GDN_ERR_INVALID_ARGUMENT


def _call(lib, fn, p, ptrs=None, ws_bytes=None, **over):
    # Fake, well-aligned addresses: every call here must fail host validation
    # before touching them (no HIP call is made on this path).
    base = dict(q=0x10000, k=0x20000, v=0x30000, g=0x40000, beta=0x50000, state_in=0x60000, state_out=0x70000,
                o=0x80000, ws=0x100000)
    base.update(over)
    st, need = _ws(lib, p)
    wsb = need if ws_bytes is None else ws_bytes
    return getattr(lib, fn)(ctypes.byref(p), *(ctypes.c_void_p(base[n]) for n in
                                               ("q", "k", "v", "g", "beta", "state_in", "state_out", "o", "ws")),
                            ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("fn", ["gdn_fwd", "gdn_chunk_step"])
def test_argument_errors_before_launch(lib, fn):
    p = _p()
    for name in ("q", "k", "v", "g", "beta", "o"):
        assert _call(lib, fn, p, **{name: None}) == L.GDN_ERR_INVALID_ARGUMENT
        assert name.encode() in lib.gdn_last_error()
        assert _call(lib, fn, p, **{name: 0x10008}) == L.GDN_ERR_INVALID_ARGUMENT  # misaligned
    assert _call(lib, fn, p, state_out=0x70004) == L.GDN_ERR_INVALID_ARGUMENT
    assert _call(lib, fn, p, ws=None) == L.GDN_ERR_WORKSPACE
    _, need = _ws(lib, p)
    assert _call(lib, fn, p, ws_bytes=need - 1) == L.GDN_ERR_WORKSPACE
    assert b"too small" in lib.gdn_last_error()
    assert _call(lib, fn, p, ws=0x100010) == L.GDN_ERR_INVALID_ARGUMENT  # workspace alignment


def test_chunk_step_contract(lib):
    assert _call(lib, "gdn_chunk_step", _p(), state_in=None) == L.GDN_ERR_INVALID_ARGUMENT
    assert b"state_in" in lib.gdn_last_error()
    assert _call(lib, "gdn_chunk_step", _p(seq_len=170), q=None) == L.GDN_ERR_INVALID_ARGUMENT
    assert _call(lib, "gdn_chunk_step", _p(seq_len=170)) == L.GDN_ERR_INVALID_ARGUMENT
    assert b"seq_len" in lib.gdn_last_error()


def test_fp8_problems(lib):
    # E4M3FN q, k, v: the MFMA kernels only (d = 112), same workspace as bf16
    st, n = _ws(lib, _p(qkv_dtype=L.GDN_FP8_E4M3))
    assert st == L.GDN_OK and n == _ws(lib, _p())[1]
    lay = L.WorkspaceLayout()
    assert lib.gdn_workspace_layout(ctypes.byref(_p(qkv_dtype=L.GDN_FP8_E4M3)), ctypes.byref(lay)) == L.GDN_OK
    assert lay.mfma == 1
    assert _ws(lib, _p(qkv_dtype=L.GDN_FP8_E4M3, head_dim_k=64, head_dim_v=64))[0] == L.GDN_ERR_UNSUPPORTED
    assert _ws(lib, _p(qkv_dtype=3))[0] == L.GDN_ERR_INVALID_ARGUMENT


def test_reverse_flag_and_bidirectional_host_checks(lib):
    # the reverse scan: a gdn_fwd flag, same workspace; gdn_chunk_step rejects it
    rev = _p(flags=L.GDN_FLAG_REVERSE)
    assert _ws(lib, rev) == _ws(lib, _p())
    assert _call(lib, "gdn_chunk_step", rev) == L.GDN_ERR_INVALID_ARGUMENT
    assert b"REVERSE" in lib.gdn_last_error()
    # the bidirectional layer: one scan's workspace (the two scans run one
    # after the other) + the reverse scan's fp32 o (+ the forward scan's for
    # bf16 o), each 256-byte aligned
    o_bytes = 1 * 160 * 20 * 112 * 4
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    n = ctypes.c_size_t(0)
    for o_dtype, qkv, copies in ((L.GDN_F32, L.GDN_BF16, 1), (L.GDN_BF16, L.GDN_BF16, 2),
                                 (L.GDN_F32, L.GDN_F32, 1), (L.GDN_BF16, L.GDN_F32, 2)):
        p = _p(o_dtype=o_dtype, qkv_dtype=qkv)
        assert lib.gdn_bidir_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == L.GDN_OK
        assert n.value == up(_ws(lib, p)[1]) + copies * up(o_bytes)
    assert lib.gdn_bidir_workspace_bytes(ctypes.byref(rev), ctypes.byref(n)) == L.GDN_ERR_INVALID_ARGUMENT
    assert lib.gdn_bidir_workspace_bytes(ctypes.byref(_p(seq_len=0)), ctypes.byref(n)) == L.GDN_OK and n.value == 0
    vp = lambda x: ctypes.c_void_p(x)  # noqa: E731
    p = _p()
    lib.gdn_bidir_workspace_bytes(ctypes.byref(p), ctypes.byref(n))
    good = dict(q=0x10000, k=0x20000, v=0x30000, g=0x40000, beta=0x50000, o=0x80000, ws=0x100000)

    def bidir(**over):
        a = dict(good, **over)
        return lib.gdn_bidir_fwd(ctypes.byref(p), *(vp(a[x]) for x in ("q", "k", "v", "g", "beta", "o", "ws")),
                                 ctypes.c_size_t(over.get("bytes", n.value)), None)
    assert bidir(q=None) == L.GDN_ERR_INVALID_ARGUMENT and b"q" in lib.gdn_last_error()
    assert bidir(o=0x80008) == L.GDN_ERR_INVALID_ARGUMENT
    assert bidir(bytes=n.value - 1) == L.GDN_ERR_WORKSPACE
    assert bidir(ws=None) == L.GDN_ERR_WORKSPACE


def test_no_alloc_size_checks_before_any_hip_call(lib):
    # the fixed 64 MiB workspace: B * H = 355 units do not fit even one-chunk
    # ranges (two 69,632 B records and the 50,176 B carried state per unit);
    # the fp32 kernels' workspace grows with T
    assert L.GDN_NO_ALLOC_SCRATCH_BYTES == 64 << 20
    vp = ctypes.c_void_p

    def call(p):
        return lib.gdn_fwd_no_alloc(ctypes.byref(p), *(vp(0x10000 * (i + 1)) for i in range(8)), None)
    assert call(_p(num_heads=355)) == L.GDN_ERR_WORKSPACE
    assert call(_p(batch=5, num_heads=71)) == L.GDN_ERR_WORKSPACE
    assert b"workspace" in lib.gdn_last_error()
    assert call(_p(qkv_dtype=L.GDN_F32, seq_len=27280)) == L.GDN_ERR_WORKSPACE
    assert call(_p(batch=0)) == L.GDN_ERR_INVALID_ARGUMENT
    assert call(_p(flags=64)) == L.GDN_ERR_INVALID_ARGUMENT


def test_unsupported_head_dim_on_mfma_path(lib):
    p = _p(head_dim_k=128, head_dim_v=128)
    st, _ = _ws(lib, p)
    mfma = L.WorkspaceLayout()
    lib.gdn_workspace_layout(ctypes.byref(_p()), ctypes.byref(mfma))
    if mfma.mfma:
        assert st == L.GDN_ERR_UNSUPPORTED
    else:
        assert st == L.GDN_OK


ATTN_HEADER = os.path.join(ROOT, "include", "sanawm_attn.h")


def test_attention_exports_and_host_checks(lib):
    text = re.sub(r"/\*.*?\*/", "", open(ATTN_HEADER).read(), flags=re.S)
    decl = sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))
    assert set(decl) == set(L.EXPORTED_ATTN), decl
    for name in decl:
        assert hasattr(lib, name), name
    # the page geometry: 880-token frames, 3 per block, 2 cached blocks, 1 sink frame
    p = L.AttnProblem(1, 20, 112, 880, 3, 2, 1, L.GDN_F32)
    n = ctypes.c_size_t(0)
    assert lib.attn_cache_bytes(ctypes.byref(p), ctypes.byref(n)) == L.GDN_OK
    keys = 880 + 3 * 2640
    vt_keys = 896 + 3 * 2688  # V^T rows padded to multiples of 64 keys
    assert n.value == 20 * ((224 * (keys + vt_keys) + 255) // 256 * 256)
    bad = L.AttnProblem(1, 20, 128, 880, 3, 2, 1, L.GDN_F32)
    assert lib.attn_cache_bytes(ctypes.byref(bad), ctypes.byref(n)) == L.GDN_ERR_UNSUPPORTED and n.value == 0
    bad = L.AttnProblem(1, 20, 112, 880, 0, 2, 1, L.GDN_F32)
    assert lib.attn_cache_bytes(ctypes.byref(bad), ctypes.byref(n)) == L.GDN_ERR_INVALID_ARGUMENT
    # argument errors come back before any device call
    fake = ctypes.c_void_p(256)
    assert lib.attn_block_fwd(ctypes.byref(p), -1, fake, fake, fake, fake, 1 << 40, fake, None) == \
        L.GDN_ERR_INVALID_ARGUMENT
    assert lib.attn_block_fwd(ctypes.byref(p), 0, None, fake, fake, fake, 1 << 40, fake, None) == \
        L.GDN_ERR_INVALID_ARGUMENT
    assert b"q is NULL" in lib.gdn_last_error()
    assert lib.attn_block_fwd(ctypes.byref(p), 0, fake, fake, fake, fake, 16, fake, None) == L.GDN_ERR_WORKSPACE
