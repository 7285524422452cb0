"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU.

No call here reaches a kernel launch: every call either fails validation or
has an empty batch, both of which return before any HIP call.  Pointers are
fake device addresses that are never dereferenced.
"""

import ctypes
import os
import re

import pytest

import gated_delta_rule_causal_amd as gd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")

LA_OK, LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_DTYPE, LA_ERR_UNSUPPORTED, LA_ERR_ALIGN, \
    LA_ERR_WORKSPACE, LA_ERR_HIP, LA_ERR_ARG = range(9)
F32, BF16 = 0, 1
CHUNKED, RECURRENT, PARALLEL = 0, 1, 2
NORMALIZED, GATED = 0, 1

BASE = 0x7F0000000000  # fake, 16-byte aligned, never dereferenced
GiB = 1 << 30


def P(i):
    """A distinct fake device pointer, 1 GiB apart so buffers never overlap."""
    return ctypes.c_void_p(BASE + i * GiB)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gd.library_path()):
        pytest.skip("liblinattn.so not built")
    return gd._load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == sorted(["lin_attn_prefill", "gdn_prefill", "gdn_prefill_noalloc", "gla_prefill",
                            "gdn_prefill_prep", "gdn_prefill_scan", "gdn_preprocess", "gdn_preprocess_varlen",
                            "kda_prefill", "gdn_prefill_varlen", "lin_attn_prefill_varlen",
                            "lin_attn_decode_step", "la_workspace_bytes",
                            "la_status_str", "la_abi_version"])


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(gd.library_path())
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_version_and_status_strings(lib):
    assert gd.la_abi_version() == 1
    for s in range(9):
        assert gd.la_status_str(s).startswith(
            ["LA_OK", "LA_ERR_NULL", "LA_ERR_SHAPE", "LA_ERR_DTYPE", "LA_ERR_UNSUPPORTED",
             "LA_ERR_ALIGN", "LA_ERR_WORKSPACE", "LA_ERR_HIP", "LA_ERR_ARG"][s])
    assert "unknown" in gd.la_status_str(99)


def prefill(lib, dtype=F32, B=1, H=2, T=8, dk=16, dv=16, q=1, k=2, v=3, S0=None, z0=None, o=4,
            S_out=None, z_out=None, form=CHUNKED, chunk=16, ws=None, ws_bytes=0):
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))
    return lib.lin_attn_prefill(dtype, B, H, T, dk, dv, f(q), f(k), f(v), f(S0), f(z0), f(o), f(S_out),
                                f(z_out), form, chunk, f(ws), ws_bytes, None)


def gdn(lib, dtype=F32, B=1, H=2, T=8, dk=16, dv=16, q=1, k=2, v=3, a=5, b=6, S0=None, o=4, S_out=None,
        form=CHUNKED, chunk=16, ws=None, ws_bytes=0):
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))
    return lib.gdn_prefill(dtype, B, H, T, dk, dv, f(q), f(k), f(v), f(a), f(b), f(S0), f(o), f(S_out),
                           form, chunk, f(ws), ws_bytes, None)


def decode(lib, kind=GATED, dtype=BF16, N=2, H=2, dk=16, dv=16, q=1, k=2, v=3, a=5, b=6, S=7, z=None, o=4):
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))
    return lib.lin_attn_decode_step(kind, dtype, N, H, dk, dv, f(q), f(k), f(v), f(a), f(b), f(S), f(z),
                                    f(o), None)


def test_prefill_validation(lib):
    assert prefill(lib, dtype=7) == LA_ERR_DTYPE
    assert prefill(lib, form=9) == LA_ERR_ARG
    assert prefill(lib, dk=48) == LA_ERR_SHAPE
    assert prefill(lib, dv=256) == LA_ERR_SHAPE
    assert prefill(lib, chunk=24) == LA_ERR_SHAPE
    assert prefill(lib, B=-1) == LA_ERR_SHAPE
    assert prefill(lib, T=-3) == LA_ERR_SHAPE
    assert prefill(lib, q=None) == LA_ERR_NULL
    assert prefill(lib, o=None) == LA_ERR_NULL
    assert prefill(lib, v=ctypes.c_void_p(BASE + 3 * GiB + 8)) == LA_ERR_ALIGN
    assert prefill(lib, S_out=ctypes.c_void_p(BASE + 9 * GiB + 4)) == LA_ERR_ALIGN
    assert prefill(lib, form=PARALLEL, S0=8) == LA_ERR_ARG
    assert prefill(lib, form=PARALLEL, T=8193) == LA_ERR_SHAPE
    # output overlapping an input
    assert prefill(lib, o=1) == LA_ERR_ARG
    assert prefill(lib, o=ctypes.c_void_p(BASE + 3 * GiB + 256)) == LA_ERR_ARG
    # S_out partially overlapping S0 is an error; S_out == S0 is the in-place update
    assert prefill(lib, S0=8, S_out=ctypes.c_void_p(BASE + 8 * GiB + 16)) == LA_ERR_ARG
    # too large: B*H beyond a grid dimension
    assert prefill(lib, B=1 << 20, H=1 << 12) == LA_ERR_SHAPE
    # empty batch: nothing to do, nothing launched
    assert prefill(lib, B=0) == LA_OK
    assert prefill(lib, H=0, q=None, k=None, v=None, o=None) == LA_OK


def test_gdn_validation(lib):
    assert gdn(lib, dtype=2) == LA_ERR_DTYPE
    assert gdn(lib, form=PARALLEL) == LA_ERR_ARG
    assert gdn(lib, dk=8) == LA_ERR_SHAPE
    assert gdn(lib, chunk=0) == LA_ERR_SHAPE
    assert gdn(lib, a=None) == LA_ERR_NULL
    assert gdn(lib, b=None) == LA_ERR_NULL
    assert gdn(lib, a=ctypes.c_void_p(BASE + 5 * GiB + 4)) == LA_ERR_ALIGN
    assert gdn(lib, o=5) == LA_ERR_ARG  # o on top of alpha
    assert gdn(lib, S0=8, S_out=ctypes.c_void_p(BASE + 8 * GiB + 64)) == LA_ERR_ARG
    assert gdn(lib, B=0) == LA_OK


def gdn_noalloc(lib, dtype=BF16, B=2, H=16, T=8192, dk=128, dv=128, q=1, k=2, v=3, a=5, b=6, S0=None, o=4,
                S_out=None, form=CHUNKED, chunk=64):
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))
    return lib.gdn_prefill_noalloc(dtype, B, H, T, dk, dv, f(q), f(k), f(v), f(a), f(b), f(S0), f(o), f(S_out),
                                   form, chunk, None)


def test_gdn_noalloc_validation(lib):
    """The allocation-free variant reports argument errors exactly as
    gdn_prefill does, before it looks up the library's device array (which
    needs a device): these calls never reach HIP."""
    assert gdn_noalloc(lib, dtype=2) == LA_ERR_DTYPE
    assert gdn_noalloc(lib, form=PARALLEL) == LA_ERR_ARG
    assert gdn_noalloc(lib, dk=8) == LA_ERR_SHAPE
    assert gdn_noalloc(lib, chunk=0) == LA_ERR_SHAPE
    assert gdn_noalloc(lib, q=None) == LA_ERR_NULL
    assert gdn_noalloc(lib, a=None) == LA_ERR_NULL
    assert gdn_noalloc(lib, a=ctypes.c_void_p(BASE + 5 * GiB + 4)) == LA_ERR_ALIGN
    assert gdn_noalloc(lib, o=5) == LA_ERR_ARG
    assert gdn_noalloc(lib, S0=8, S_out=ctypes.c_void_p(BASE + 8 * GiB + 64)) == LA_ERR_ARG
    assert gdn_noalloc(lib, B=0) == LA_OK
    # the workspace a uniform call needs never exceeds the library's 72 MiB array
    for B, H, T in ((1, 1, 1 << 20), (2, 16, 8192), (1, 16, 262144), (4, 64, 4096), (1, 257, 100000)):
        assert gd.la_workspace_bytes("gdn_prefill", "bf16", B, H, T, 128, 128, "chunked", 64) <= 72 << 20


def test_decode_validation(lib):
    assert decode(lib, kind=9) == LA_ERR_ARG
    assert decode(lib, dtype=9) == LA_ERR_DTYPE
    assert decode(lib, dk=100) == LA_ERR_SHAPE
    assert decode(lib, S=None) == LA_ERR_NULL
    assert decode(lib, a=None) == LA_ERR_NULL             # gated delta needs gates
    assert decode(lib, z=8) == LA_ERR_ARG                 # ... and takes no z
    assert decode(lib, kind=NORMALIZED) == LA_ERR_NULL    # normalized needs z
    assert decode(lib, kind=NORMALIZED, z=8) == LA_ERR_ARG  # ... and takes no gates
    assert decode(lib, o=7) == LA_ERR_ARG                 # o on top of S
    assert decode(lib, q=ctypes.c_void_p(BASE + GiB + 2)) == LA_ERR_ALIGN
    assert decode(lib, N=0) == LA_OK


def test_grid_beyond_one_launch_is_a_shape_error(lib):
    """Sizes within every bound whose launch would hold 2^32 or more
    work-items are refused before anything is launched (so no device is
    needed to see it, and no call here launches anything): a decode step
    over 2^24 heads of d = 16 (1 KiB of state each, 16 GiB in all) and the
    fp32 chunked kernels, one workgroup per head, over as many heads."""
    W = lambda i: ctypes.c_void_p(BASE + i * 32 * GiB)
    many = dict(N=1 << 19, H=32)
    assert decode(lib, q=W(1), k=W(2), v=W(3), a=W(5), b=W(6), S=W(7), o=W(4), **many) == LA_ERR_SHAPE
    assert prefill(lib, B=1 << 19, H=32, T=1, q=W(1), k=W(2), v=W(3), o=W(4)) == LA_ERR_SHAPE
    assert gdn(lib, B=1 << 19, H=32, T=1, q=W(1), k=W(2), v=W(3), a=W(5), b=W(6), o=W(4)) == LA_ERR_SHAPE


def test_workspace_query(lib):
    big = ctypes.c_size_t(-1).value
    assert lib.la_workspace_bytes(9, F32, 1, 1, 8, 16, 16, CHUNKED, 16) == big
    assert lib.la_workspace_bytes(0, 5, 1, 1, 8, 16, 16, CHUNKED, 16) == big
    assert lib.la_workspace_bytes(1, F32, 1, 1, 8, 16, 16, PARALLEL, 16) == big
    assert lib.la_workspace_bytes(0, F32, 1, 1, 8, 16, 16, CHUNKED, 17) == big
    assert lib.la_workspace_bytes(2, BF16, 4, 4, 1, 128, 128, 0, 0) == 0
    assert lib.la_workspace_bytes(0, F32, 1, 2, 256, 16, 16, RECURRENT, 0) == 0
    assert lib.la_workspace_bytes(1, F32, 1, 2, 256, 16, 16, RECURRENT, 0) == 0
    # fp32 chunked at dk = dv = 128 with chunk 128 does not fit any kernel
    assert lib.la_workspace_bytes(1, F32, 1, 1, 256, 128, 128, CHUNKED, 128) == big
    assert gdn(lib, dk=128, dv=128, chunk=128) == LA_ERR_UNSUPPORTED


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gd, "_lib", None)
    monkeypatch.setattr(gd, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="build the HIP library"):
        gd.la_abi_version()


def test_split_gdn_validation(lib):
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))

    def prep(dtype=BF16, B=1, H=2, T=100, dk=128, dv=128, q=1, k=2, v=3, a=5, b=6, chunk=64, ws=9,
             ws_bytes=1 << 40):
        return lib.gdn_prefill_prep(dtype, B, H, T, dk, dv, f(q), f(k), f(v), f(a), f(b), chunk, f(ws), ws_bytes,
                                    None)

    def scan(dtype=BF16, B=1, H=2, T=100, dk=128, dv=128, q=1, k=2, v=3, a=5, b=6, S0=None, o=4, S_out=None,
             chunk=64, ws=9, ws_bytes=1 << 40):
        return lib.gdn_prefill_scan(dtype, B, H, T, dk, dv, f(q), f(k), f(v), f(a), f(b), f(S0), f(o), f(S_out),
                                    chunk, f(ws), ws_bytes, None)

    assert prep(dtype=F32) == LA_ERR_UNSUPPORTED
    assert prep(dk=64, dv=64) == LA_ERR_UNSUPPORTED
    assert prep(chunk=32, ws=None) == LA_ERR_WORKSPACE   # any valid chunk: the kernels' 64-token blocks
    assert prep(chunk=33) == LA_ERR_SHAPE
    assert prep(ws=None) == LA_ERR_WORKSPACE
    assert prep(ws_bytes=1000) == LA_ERR_WORKSPACE
    assert prep(a=None) == LA_ERR_NULL
    assert prep(ws=2) == LA_ERR_ARG          # workspace on top of k
    assert prep(B=0) == LA_OK
    assert scan(o=None) == LA_ERR_NULL
    assert scan(o=9) == LA_ERR_ARG           # output on top of the workspace
    assert scan(o=1) == LA_ERR_ARG           # output on top of q
    assert scan(S0=7, S_out=ctypes.c_void_p(BASE + 7 * GiB + 32)) == LA_ERR_ARG
    assert scan(ws=ctypes.c_void_p(BASE + 9 * GiB + 8)) == LA_ERR_ALIGN
    assert scan(a=None) == LA_ERR_NULL
    n = lib.la_workspace_bytes(1, BF16, 1, 2, 1000, 128, 128, CHUNKED, 64)
    assert n > 0 and scan(T=1000, ws_bytes=n - 1) == LA_ERR_WORKSPACE
    # one segment per head needs no workspace (many heads, short sequence)
    assert lib.la_workspace_bytes(1, BF16, 64, 8, 64, 128, 128, CHUNKED, 64) == 0


def test_segmented_linear_attention_workspace(lib):
    """The bf16 chunked linear-attention path cuts long sequences into segments
    and needs a workspace; it must not overlap any tensor."""
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))

    def la(T=1000, ws=9, ws_bytes=1 << 40, q=1, o=4):
        return lib.lin_attn_prefill(BF16, 1, 2, T, 128, 128, f(q), P(2), P(3), None, None, f(o), None, None,
                                    CHUNKED, 64, f(ws), ws_bytes, None)

    n = lib.la_workspace_bytes(0, BF16, 1, 2, 1000, 128, 128, CHUNKED, 64)
    assert n > 0
    assert la(ws=None) == LA_ERR_WORKSPACE
    assert la(ws_bytes=n - 1) == LA_ERR_WORKSPACE
    assert la(ws=1) == LA_ERR_ARG            # workspace on top of q
    assert la(ws=4) == LA_ERR_ARG            # workspace on top of o
    # one segment (short sequence, many heads): no workspace
    assert lib.la_workspace_bytes(0, BF16, 64, 8, 64, 128, 128, CHUNKED, 64) == 0


def test_gla_validation(lib):
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))
    GLA = 3

    def gla(dtype=BF16, T=1000, dk=128, dv=128, q=1, k=2, v=3, a=5, S0=None, o=4, S_out=None, form=CHUNKED,
            chunk=64, ws=9, ws_bytes=1 << 40):
        return lib.gla_prefill(dtype, 1, 2, T, dk, dv, f(q), f(k), f(v), f(a), f(S0), f(o), f(S_out), form, chunk,
                               f(ws), ws_bytes, None)

    assert gla(a=None) == LA_ERR_NULL
    assert gla(form=PARALLEL) == LA_ERR_ARG
    assert gla(dtype=F32) == LA_ERR_UNSUPPORTED            # chunked: bf16, d = 128, chunk 64 only
    assert gla(ws=None) == LA_ERR_WORKSPACE
    assert gla(ws=5) == LA_ERR_ARG                         # workspace on top of alpha
    assert gla(o=5) == LA_ERR_ARG                          # output on top of alpha
    assert gla(S0=7, S_out=ctypes.c_void_p(BASE + 7 * GiB + 32)) == LA_ERR_ARG
    n = lib.la_workspace_bytes(GLA, BF16, 1, 2, 1000, 128, 128, CHUNKED, 64)
    assert n > 0 and gla(ws_bytes=n - 1) == LA_ERR_WORKSPACE
    assert lib.la_workspace_bytes(GLA, F32, 1, 2, 1000, 16, 16, RECURRENT, 0) == 0
    assert lib.la_workspace_bytes(GLA, F32, 1, 2, 1000, 16, 16, CHUNKED, 16) == ctypes.c_size_t(-1).value
    # decode: the gated kind needs alpha, no beta, no z
    dec = lambda a=5, b=None, z=None: lib.lin_attn_decode_step(2, BF16, 4, 2, 128, 128, P(1), P(2), P(3), f(a), f(b),
                                                               P(6), f(z), P(4), None)
    assert dec(a=None) == LA_ERR_NULL
    assert dec(b=8) == LA_ERR_ARG
    assert dec(z=8) == LA_ERR_ARG


def test_preprocess_validation(lib):
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))

    def pre(dtype=BF16, B=2, T=100, H=4, dk=128, dv=128, x=1, w=2, a=3, b=4, st=None, st_out=None, q=5, k=6, v=7,
            al=8, be=9):
        return lib.gdn_preprocess(dtype, B, T, H, dk, dv, f(x), f(w), f(a), f(b), f(st), f(st_out), f(q), f(k),
                                  f(v), f(al), f(be), None)

    assert pre(dtype=3) == LA_ERR_DTYPE
    assert pre(dk=48) == LA_ERR_SHAPE
    assert pre(dv=256) == LA_ERR_SHAPE
    assert pre(T=-1) == LA_ERR_SHAPE
    assert pre(x=None) == LA_ERR_NULL
    assert pre(w=None) == LA_ERR_NULL
    assert pre(be=None) == LA_ERR_NULL
    assert pre(q=ctypes.c_void_p(BASE + 5 * GiB + 8)) == LA_ERR_ALIGN
    assert pre(q=1) == LA_ERR_ARG                          # output on top of x
    assert pre(k=5) == LA_ERR_ARG                          # two outputs on the same memory
    assert pre(st=10, st_out=10) == LA_ERR_ARG             # the conv state is not updated in place
    assert pre(al=4) == LA_ERR_ARG                         # alpha on top of b_logit
    assert pre(B=0) == LA_OK                               # empty batch: nothing to do
    assert pre(T=0, st=10) == LA_OK                        # no tokens and no state to write


def test_kda_validation(lib):
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))
    KDA = 4

    def kda(dtype=BF16, T=100, dk=128, dv=128, q=1, k=2, v=3, a=5, b=6, S0=None, o=4, S_out=None, form=RECURRENT):
        return lib.kda_prefill(dtype, 1, 2, T, dk, dv, f(q), f(k), f(v), f(a), f(b), f(S0), f(o), f(S_out), form, 64,
                               None, 0, None)

    assert kda(a=None) == LA_ERR_NULL
    assert kda(b=None) == LA_ERR_NULL
    assert kda(form=PARALLEL) == LA_ERR_ARG
    assert kda(form=CHUNKED, dtype=F32) == LA_ERR_UNSUPPORTED      # block form: bf16, d = 128, chunk 64
    assert kda(form=CHUNKED) == LA_ERR_WORKSPACE                   # ... with its workspace
    assert kda(dk=48) == LA_ERR_SHAPE
    assert kda(o=5) == LA_ERR_ARG                          # output on top of alpha
    assert kda(S0=7, S_out=ctypes.c_void_p(BASE + 7 * GiB + 32)) == LA_ERR_ARG
    assert kda(q=ctypes.c_void_p(BASE + GiB + 4)) == LA_ERR_ALIGN
    assert lib.la_workspace_bytes(KDA, BF16, 1, 2, 100, 128, 128, RECURRENT, 0) == 0
    assert lib.la_workspace_bytes(KDA, BF16, 1, 2, 100, 128, 128, CHUNKED, 64) == 2 * 2 * 74240
    assert lib.la_workspace_bytes(KDA, F32, 1, 2, 100, 128, 128, CHUNKED, 64) == ctypes.c_size_t(-1).value
    # decode: KDA needs alpha (per channel) and beta, no z
    dec = lambda a=5, b=6, z=None: lib.lin_attn_decode_step(3, BF16, 4, 2, 128, 128, P(1), P(2), P(3), f(a), f(b),
                                                            P(7), f(z), P(4), None)
    assert dec(a=None) == LA_ERR_NULL
    assert dec(b=None) == LA_ERR_NULL
    assert dec(z=8) == LA_ERR_ARG
    # alpha spans N*H*dk floats: an output placed inside it is an overlap
    assert lib.lin_attn_decode_step(3, BF16, 4, 2, 128, 128, P(1), P(2), P(3), P(5), P(6), P(7), None,
                                    ctypes.c_void_p(BASE + 5 * GiB + 2048), None) == LA_ERR_ARG


def test_varlen_validation(lib):
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))
    VARLEN = 5

    def vl(dtype=BF16, N=3, H=2, T=500, dk=128, dv=128, cu=10, q=1, k=2, v=3, a=5, b=6, S0=None, o=4, S_out=None,
           snap=0, nsnap=0, S_snap=None, form=CHUNKED, chunk=64, ws=9, ws_bytes=1 << 40):
        return lib.gdn_prefill_varlen(dtype, N, H, T, dk, dv, f(cu), f(q), f(k), f(v), f(a), f(b), f(S0), f(o),
                                      f(S_out), snap, nsnap, f(S_snap), form, chunk, f(ws), ws_bytes, None)

    assert vl(dtype=7) == LA_ERR_DTYPE
    assert vl(form=PARALLEL) == LA_ERR_ARG
    assert vl(dtype=F32) == LA_ERR_UNSUPPORTED             # chunked: bf16, d = 128, chunk 64 only
    assert vl(snap=100, nsnap=4, S_snap=11) == LA_ERR_SHAPE  # chunked snapshots at whole chunks
    assert vl(snap=-1) == LA_ERR_SHAPE
    assert vl(cu=None) == LA_ERR_NULL
    assert vl(a=None) == LA_ERR_NULL
    assert vl(snap=128, nsnap=4, S_snap=None) == LA_ERR_NULL
    assert vl(cu=ctypes.c_void_p(BASE + 10 * GiB + 2)) == LA_ERR_ALIGN
    assert vl(ws=None) == LA_ERR_WORKSPACE
    assert vl(ws=5) == LA_ERR_ARG                          # workspace on top of alpha
    assert vl(o=10) == LA_ERR_ARG                          # output on top of cu_seqlens
    assert vl(snap=128, nsnap=4, S_snap=4) == LA_ERR_ARG   # snapshots on top of o
    need = lib.la_workspace_bytes(VARLEN, BF16, 3, 2, 500, 128, 128, CHUNKED, 64)
    assert need > 0 and vl(ws_bytes=need - 1) == LA_ERR_WORKSPACE
    rec = lib.la_workspace_bytes(VARLEN, F32, 3, 2, 500, 64, 64, RECURRENT, 0)
    assert 0 < rec < need
    assert vl(N=0) == LA_OK


def test_varlen_kinds_validation(lib):
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))
    K_NORM, K_GDN, K_GATED, K_KDA = 0, 1, 2, 3
    PREFILL_VARLEN = 6

    def vl(kind=K_KDA, dtype=BF16, N=3, H=2, T=500, dk=128, dv=128, cu=10, q=1, k=2, v=3, a=5, b=6, S0=None,
           z0=None, o=4, S_out=None, z_out=None, snap=0, nsnap=0, S_snap=None, z_snap=None, form=RECURRENT,
           chunk=64, ws=9, ws_bytes=1 << 40):
        return lib.lin_attn_prefill_varlen(kind, dtype, N, H, T, dk, dv, f(cu), f(q), f(k), f(v), f(a), f(b), f(S0),
                                           f(z0), f(o), f(S_out), f(z_out), snap, nsnap, f(S_snap), f(z_snap), form,
                                           chunk, f(ws), ws_bytes, None)

    assert vl(kind=9) == LA_ERR_ARG
    assert vl(dtype=7) == LA_ERR_DTYPE
    assert vl(form=PARALLEL) == LA_ERR_ARG
    # block form of every kind on the matrix cores: bf16, d = 128
    assert vl(form=CHUNKED, ws=None) == LA_ERR_WORKSPACE
    assert vl(form=CHUNKED, dtype=F32) == LA_ERR_UNSUPPORTED
    assert vl(form=CHUNKED, dk=64, dv=64) == LA_ERR_UNSUPPORTED
    assert vl(form=CHUNKED, kind=K_GATED, b=None, ws=None) == LA_ERR_WORKSPACE
    assert vl(form=CHUNKED, kind=K_NORM, a=None, b=None, ws=None) == LA_ERR_WORKSPACE
    assert vl(form=CHUNKED, kind=K_GATED, b=None, dtype=F32) == LA_ERR_UNSUPPORTED
    assert vl(form=CHUNKED, kind=K_NORM, a=None, b=None, dk=64, dv=64) == LA_ERR_UNSUPPORTED
    assert vl(form=CHUNKED, snap=100, nsnap=4, S_snap=11) == LA_ERR_SHAPE   # snapshots at whole 64-token blocks
    assert vl(form=CHUNKED, kind=K_NORM, a=None, b=None, snap=100, nsnap=4, S_snap=11, z_snap=12) == LA_ERR_SHAPE
    kneed = lib.la_workspace_bytes(PREFILL_VARLEN, BF16, 3, 2, 500, 128, 128, CHUNKED, 64)
    assert kneed >= lib.la_workspace_bytes(5, BF16, 3, 2, 500, 128, 128, CHUNKED, 64)
    assert vl(form=CHUNKED, ws_bytes=1000) == LA_ERR_WORKSPACE
    assert vl(form=CHUNKED, kind=K_GATED, b=None, ws_bytes=1000) == LA_ERR_WORKSPACE
    assert vl(form=CHUNKED, kind=K_NORM, a=None, b=None, ws_bytes=1000) == LA_ERR_WORKSPACE
    assert vl(form=CHUNKED, chunk=48) == LA_ERR_SHAPE
    assert vl(dk=48) == LA_ERR_SHAPE
    assert vl(snap=-1) == LA_ERR_SHAPE
    assert vl(z0=12) == LA_ERR_ARG                         # no normaliser outside the normalised kind
    assert vl(kind=K_GATED, z_out=12) == LA_ERR_ARG
    assert vl(kind=K_GDN, z_snap=12) == LA_ERR_ARG
    assert vl(kind=K_NORM) == LA_ERR_ARG                   # the normalised kind takes no gates
    assert vl(kind=K_NORM, a=None) == LA_ERR_ARG
    assert vl(kind=K_GATED) == LA_ERR_ARG                  # ... and the scalar-gated kind no beta
    assert vl(cu=None) == LA_ERR_NULL
    assert vl(a=None) == LA_ERR_NULL
    assert vl(b=None) == LA_ERR_NULL
    assert vl(kind=K_GATED, b=None, a=None) == LA_ERR_NULL
    assert vl(o=None) == LA_ERR_NULL
    assert vl(snap=128, nsnap=4, S_snap=None) == LA_ERR_NULL
    assert vl(kind=K_NORM, a=None, b=None, snap=128, nsnap=4, S_snap=11) == LA_ERR_NULL   # z snapshots needed
    assert vl(cu=ctypes.c_void_p(BASE + 10 * GiB + 2)) == LA_ERR_ALIGN
    assert vl(z_snap=ctypes.c_void_p(BASE + 12 * GiB + 4), kind=K_NORM, a=None, b=None) == LA_ERR_ALIGN
    assert vl(ws=None) == LA_ERR_WORKSPACE
    need = lib.la_workspace_bytes(PREFILL_VARLEN, BF16, 3, 2, 500, 128, 128, RECURRENT, 0)
    assert need == lib.la_workspace_bytes(5, BF16, 3, 2, 500, 128, 128, RECURRENT, 0) > 0
    assert vl(ws_bytes=need - 1) == LA_ERR_WORKSPACE
    assert vl(ws=5) == LA_ERR_ARG                          # workspace on top of alpha
    assert vl(o=10) == LA_ERR_ARG                          # output on top of cu_seqlens
    assert vl(snap=128, nsnap=4, S_snap=4) == LA_ERR_ARG   # snapshots on top of o
    # KDA's alpha holds H*T*dk floats (512 000 bytes here), the scalar gate H*T
    # (4 000 bytes): an output state 300 000 bytes past alpha overlaps only the first
    inside = ctypes.c_void_p(BASE + 5 * GiB + 300000)
    assert vl(S_out=inside) == LA_ERR_ARG
    assert vl(kind=K_GATED, b=None, S_out=inside, ws=None) == LA_ERR_WORKSPACE
    # in-place state update is allowed (stopped here by the missing workspace, checked last)
    assert vl(kind=K_NORM, a=None, b=None, S0=11, S_out=11, z0=12, z_out=12, ws=None) == LA_ERR_WORKSPACE
    assert vl(kind=K_NORM, a=None, b=None, S_out=12, z_out=12) == LA_ERR_ARG
    assert vl(kind=K_NORM, a=None, b=None, snap=128, nsnap=4, S_snap=11, z_snap=11) == LA_ERR_ARG
    # the gated-delta kind forwards to gdn_prefill_varlen (chunked: bf16, d = 128, chunk 64)
    assert vl(kind=K_GDN, dtype=F32, form=CHUNKED) == LA_ERR_UNSUPPORTED
    assert vl(N=0) == LA_OK
    assert vl(H=0) == LA_OK


def test_preprocess_varlen_validation(lib):
    f = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else P(x))

    def pre(dtype=BF16, N=3, T=100, H=4, dk=128, dv=128, cu=10, x=1, w=2, a=3, b=4, st=None, st_out=None, q=5, k=6,
            v=7, al=8, be=9):
        return lib.gdn_preprocess_varlen(dtype, N, T, H, dk, dv, f(cu), f(x), f(w), f(a), f(b), f(st), f(st_out),
                                         f(q), f(k), f(v), f(al), f(be), None)

    assert pre(dtype=3) == LA_ERR_DTYPE
    assert pre(dk=48) == LA_ERR_SHAPE
    assert pre(cu=None) == LA_ERR_NULL
    assert pre(x=None) == LA_ERR_NULL
    assert pre(cu=ctypes.c_void_p(BASE + 10 * GiB + 2)) == LA_ERR_ALIGN
    assert pre(q=10) == LA_ERR_ARG                         # output on top of cu_seqlens
    assert pre(st=11, st_out=11) == LA_ERR_ARG
    assert pre(N=0) == LA_OK
