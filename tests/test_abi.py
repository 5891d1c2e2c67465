"""The C ABI library: it loads, exports every symbol include/ikbo.h declares, and rejects bad
arguments before touching the GPU. Runs without a GPU: no call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

import request_candidate_broadcast_amd as ikbo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ikbo.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ikbo.LIB_PATH):
        from request_candidate_broadcast_amd import _build
        _build.build(verbose=False)
    return ikbo.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ikbo_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("ikbo_dca_forward", "ikbo_lcb_forward", "ikbo_glm_mlp_forward", "ikbo_check_index",
              "ikbo_dca_workspace_size", "ikbo_lcb_workspace_size", "ikbo_glm_mlp_workspace_size",
              "ikbo_status_string", "ikbo_last_error_message", "ikbo_version"):
        assert n in names
    assert sorted(ikbo.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", ikbo.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = set(re.findall(r"\bT (ikbo_[a-z_0-9]+)\b", out))
    for n in declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_version_and_status_strings(lib):
    assert lib.ikbo_version() == 100
    assert lib.ikbo_status_string(0) == b"IKBO_OK"
    assert lib.ikbo_status_string(4) == b"IKBO_WORKSPACE_TOO_SMALL"
    assert lib.ikbo_status_string(99) == b"IKBO_UNKNOWN_STATUS"


def test_workspace_sizes(lib):
    assert lib.ikbo_dca_workspace_size(1000, 10) >= 4 * (1000 + 3 * 11)
    assert lib.ikbo_dca_workspace_size(-1, 10) == 0
    # Z in fp32 [R, N_c] at least
    assert lib.ikbo_lcb_workspace_size(100, 8, 64, 64, 32, 48, 1) >= 4 * 8 * 48
    assert lib.ikbo_lcb_workspace_size(100, 8, 64, 64, 32, 48, 7) == 0
    # a misaligned bf16 K width adds zero-padded copies of the operands it multiplies
    aligned = lib.ikbo_lcb_workspace_size(100, 8, 64, 64, 32, 48, 1)
    padded = lib.ikbo_lcb_workspace_size(100, 8, 64, 61, 32, 48, 1)
    assert padded >= aligned + 2 * 64 * (100 + 48)
    assert lib.ikbo_lcb_workspace_size(100, 8, 64, 61, 32, 48, 0) == lib.ikbo_lcb_workspace_size(100, 8, 64, 64, 32, 48, 0)
    layers = (ikbo.GlmLayer * 2)()
    layers[0] = ikbo.GlmLayer(None, None, None, None, None, 64, 32, 48, 40, 1)
    layers[1] = ikbo.GlmLayer(None, None, None, None, None, 48, 40, 16, 24, 0)
    n = lib.ikbo_glm_mlp_workspace_size(100, 8, 2, layers, 1)
    assert n >= 2 * 2 * 100 * 40      # two bf16 hidden candidate buffers


FAKE = 0x10000          # a 16-byte-aligned address that is never dereferenced: calls fail first
MIS = 0x10008           # 8-byte aligned only


def dca(lib, **kw):
    a = dict(q=FAKE, C=64, Lq=1, k=FAKE, v=FAKE, R=4, cu=None, L=16, m=FAKE, off=None, flags=0, H=2, d=128,
             scale=0.0, ind=1, outd=0, out=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.ikbo_dca_forward(a["q"], a["C"], a["Lq"], a["k"], a["v"], a["R"], a["cu"], a["L"], a["m"], a["off"],
                                a["flags"], a["H"], a["d"], a["scale"], a["ind"], a["outd"], a["out"], a["ws"],
                                a["wsb"], a["stream"])


def test_dca_argument_errors(lib):
    assert dca(lib, m=None, off=None) == ikbo.IKBO_INVALID_ARGUMENT
    assert b"cand_to_req" in lib.ikbo_last_error_message()
    assert dca(lib, C=-1) == ikbo.IKBO_INVALID_ARGUMENT
    assert dca(lib, H=0) == ikbo.IKBO_INVALID_ARGUMENT
    assert dca(lib, flags=4) == ikbo.IKBO_INVALID_ARGUMENT
    assert dca(lib, d=96) == ikbo.IKBO_UNSUPPORTED
    assert dca(lib, ind=0, d=130) == ikbo.IKBO_UNSUPPORTED
    assert dca(lib, ind=7) == ikbo.IKBO_UNSUPPORTED
    # a request's bf16 K block must span fewer than 2^31 bytes: 1M keys x 8 heads x 128 x 2 B does not
    assert dca(lib, L=1 << 20, H=8) == ikbo.IKBO_UNSUPPORTED
    assert b"2^31" in lib.ikbo_last_error_message()
    assert dca(lib, q=MIS) == ikbo.IKBO_MISALIGNED
    assert dca(lib, m=MIS) == ikbo.IKBO_MISALIGNED
    assert dca(lib, q=None) == ikbo.IKBO_INVALID_ARGUMENT
    assert dca(lib, wsb=16) == ikbo.IKBO_WORKSPACE_TOO_SMALL
    assert dca(lib, ws=None, wsb=1 << 30) == ikbo.IKBO_WORKSPACE_TOO_SMALL
    # nothing to do: succeeds without any GPU work
    assert dca(lib, C=0) == ikbo.IKBO_OK


def lcb(lib, **kw):
    a = dict(xr=FAKE, R=4, kr=64, xc=FAKE, C=32, kc=64, m=FAKE, off=None, flags=0, wrr=FAKE, wcr=FAKE, wcc=FAKE,
             br=None, bc=None, nr=32, nc=32, act=0, ind=1, outd=1, yr=FAKE, yc=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.ikbo_lcb_forward(a["xr"], a["R"], a["kr"], a["xc"], a["C"], a["kc"], a["m"], a["off"], a["flags"],
                                a["wrr"], a["wcr"], a["wcc"], a["br"], a["bc"], a["nr"], a["nc"], a["act"], a["ind"],
                                a["outd"], a["yr"], a["yc"], a["ws"], a["wsb"], a["stream"])


def test_lcb_argument_errors(lib):
    assert lcb(lib, m=None, off=None) == ikbo.IKBO_INVALID_ARGUMENT
    # misaligned K widths are padded in the workspace: its size, not the width, is checked
    need = lib.ikbo_lcb_workspace_size(32, 4, 60, 64, 32, 32, 1)
    assert lcb(lib, kr=60, wsb=need - 1) == ikbo.IKBO_WORKSPACE_TOO_SMALL
    assert lcb(lib, act=5) == ikbo.IKBO_INVALID_ARGUMENT
    assert lcb(lib, nr=-1) == ikbo.IKBO_INVALID_ARGUMENT
    assert lcb(lib, wcc=None) == ikbo.IKBO_INVALID_ARGUMENT
    assert lcb(lib, yc=None) == ikbo.IKBO_INVALID_ARGUMENT
    assert lcb(lib, xc=MIS) == ikbo.IKBO_MISALIGNED
    assert lcb(lib, wsb=8) == ikbo.IKBO_WORKSPACE_TOO_SMALL
    assert lcb(lib, outd=3) == ikbo.IKBO_UNSUPPORTED


def test_glm_mlp_argument_errors(lib):
    layers = (ikbo.GlmLayer * 2)()
    layers[0] = ikbo.GlmLayer(FAKE, FAKE, FAKE, None, None, 64, 32, 48, 40, 1)
    layers[1] = ikbo.GlmLayer(FAKE, FAKE, FAKE, None, None, 48, 40, 16, 24, 0)
    f = lambda n=2, ly=layers, wsb=1 << 30, m=FAKE: lib.ikbo_glm_mlp_forward(
        FAKE, 4, FAKE, 32, m, None, 0, n, ly, 1, 1, FAKE, FAKE, FAKE, wsb, None)
    assert f(n=0) == ikbo.IKBO_INVALID_ARGUMENT
    assert f(m=None) == ikbo.IKBO_INVALID_ARGUMENT
    assert f(wsb=64) == ikbo.IKBO_WORKSPACE_TOO_SMALL
    bad = (ikbo.GlmLayer * 2)()
    bad[0] = layers[0]
    bad[1] = ikbo.GlmLayer(FAKE, FAKE, FAKE, None, None, 40, 40, 16, 24, 0)   # k_req != previous n_req
    assert f(ly=bad) == ikbo.IKBO_INVALID_ARGUMENT
    assert b"do not match" in lib.ikbo_last_error_message()
    odd = (ikbo.GlmLayer * 2)()
    odd[0] = ikbo.GlmLayer(FAKE, FAKE, FAKE, None, None, 64, 32, 44, 40, 1)   # hidden width not a multiple of 8
    odd[1] = ikbo.GlmLayer(FAKE, FAKE, FAKE, None, None, 44, 40, 16, 24, 0)
    need_odd = lib.ikbo_glm_mlp_workspace_size(32, 4, 2, odd, 1)
    assert need_odd > lib.ikbo_glm_mlp_workspace_size(32, 4, 2, layers, 1)   # room for the padded copies
    assert f(ly=odd, wsb=need_odd - 1) == ikbo.IKBO_WORKSPACE_TOO_SMALL


def test_check_index_argument_errors(lib):
    assert lib.ikbo_check_index(None, None, 4, 2, 0, FAKE, None) == ikbo.IKBO_INVALID_ARGUMENT
    assert lib.ikbo_check_index(FAKE, None, 4, 2, 0, None, None) == ikbo.IKBO_INVALID_ARGUMENT
    assert lib.ikbo_check_index(FAKE, None, 4, 2, 0, FAKE + 4, None) == ikbo.IKBO_MISALIGNED


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("request_candidate_broadcast_amd")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            mod.load_library(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved


def kvp(lib, **kw):
    a = dict(s=FAKE, rows=1024, d_in=256, wk=FAKE, wv=FAKE, d_out=128, ind=1, outd=1, k=FAKE, v=FAKE, stream=None)
    a.update(kw)
    return lib.ikbo_kv_project(a["s"], a["rows"], a["d_in"], a["wk"], a["wv"], a["d_out"], a["ind"], a["outd"],
                               a["k"], a["v"], a["stream"])


def test_kv_project_argument_errors(lib):
    assert kvp(lib, rows=-1) == ikbo.IKBO_INVALID_ARGUMENT
    assert kvp(lib, ind=7) == ikbo.IKBO_UNSUPPORTED
    assert kvp(lib, wv=None) == ikbo.IKBO_INVALID_ARGUMENT
    assert kvp(lib, k=MIS) == ikbo.IKBO_MISALIGNED
    assert kvp(lib, d_in=100) == ikbo.IKBO_MISALIGNED          # bf16 rows need d_in % 8 == 0
    assert b"d_in" in lib.ikbo_last_error_message()
    # nothing to compute: OK without touching the GPU
    assert kvp(lib, rows=0) == ikbo.IKBO_OK
    assert kvp(lib, d_out=0) == ikbo.IKBO_OK


def rattn(lib, **kw):
    a = dict(q=FAKE, R=8, Lq=4, k=FAKE, v=FAKE, cu=None, L=64, H=2, d=128, scale=0.0, ind=1, outd=0, out=FAKE,
             ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.ikbo_request_attention(a["q"], a["R"], a["Lq"], a["k"], a["v"], a["cu"], a["L"], a["H"], a["d"],
                                      a["scale"], a["ind"], a["outd"], a["out"], a["ws"], a["wsb"], a["stream"])


def test_request_attention_argument_errors(lib):
    need = lib.ikbo_request_attention_workspace_size(8)
    assert need >= 4 * 9 + lib.ikbo_dca_workspace_size(8, 8)
    assert lib.ikbo_request_attention_workspace_size(-1) == 0
    assert rattn(lib, R=-1) == ikbo.IKBO_INVALID_ARGUMENT
    assert rattn(lib, wsb=need - 1) == ikbo.IKBO_WORKSPACE_TOO_SMALL
    assert rattn(lib, d=96) == ikbo.IKBO_UNSUPPORTED
    assert rattn(lib, L=1 << 20, H=8) == ikbo.IKBO_UNSUPPORTED
    assert b"2^31" in lib.ikbo_last_error_message()
    assert rattn(lib, q=MIS) == ikbo.IKBO_MISALIGNED
    assert rattn(lib, Lq=0) == ikbo.IKBO_INVALID_ARGUMENT
    assert rattn(lib, R=0) == ikbo.IKBO_OK


def fm(lib, **kw):
    a = dict(xr=FAKE, R=4, nr=32, xc=FAKE, C=64, nc=32, d=64, m=FAKE, off=None, flags=0, ind=1, outd=1, yr=FAKE,
             yc=FAKE, stream=None)
    a.update(kw)
    return lib.ikbo_fm_forward(a["xr"], a["R"], a["nr"], a["xc"], a["C"], a["nc"], a["d"], a["m"], a["off"], a["flags"],
                               a["ind"], a["outd"], a["yr"], a["yc"], a["stream"])


def test_fm_argument_errors(lib):
    assert fm(lib, d=0) == ikbo.IKBO_INVALID_ARGUMENT
    assert fm(lib, nr=30) == ikbo.IKBO_UNSUPPORTED
    assert b"multiples of 4" in lib.ikbo_last_error_message()
    assert fm(lib, ind=5) == ikbo.IKBO_UNSUPPORTED
    assert fm(lib, m=None, off=None) == ikbo.IKBO_INVALID_ARGUMENT
    assert fm(lib, yc=None) == ikbo.IKBO_INVALID_ARGUMENT
    assert fm(lib, xr=None) == ikbo.IKBO_INVALID_ARGUMENT
    assert fm(lib, yc=MIS) == ikbo.IKBO_MISALIGNED
    assert fm(lib, C=0, yr=None) == ikbo.IKBO_OK       # nothing to compute


def lcbe(lib, **kw):
    a = dict(xr=FAKE, R=4, nr=32, xc=FAKE, C=64, nc=32, d=64, wrr=FAKE, kr=16, wcr=FAKE, wcc=FAKE, kc=32, m=FAKE,
             off=None, flags=0, norm=1, gr=None, br=None, gc=FAKE, bc=FAKE, eps=1e-5, ind=1, outd=1, yr=FAKE, yc=FAKE,
             ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.ikbo_lcb_emb_forward(a["xr"], a["R"], a["nr"], a["xc"], a["C"], a["nc"], a["d"], a["wrr"], a["kr"],
                                    a["wcr"], a["wcc"], a["kc"], a["m"], a["off"], a["flags"], a["norm"], a["gr"],
                                    a["br"], a["gc"], a["bc"], a["eps"], a["ind"], a["outd"], a["yr"], a["yc"], a["ws"],
                                    a["wsb"], a["stream"])


def test_lcb_emb_argument_errors(lib):
    # Z in fp32 [R, k_c, d]
    assert lib.ikbo_lcb_emb_workspace_size(4, 32, 64) >= 4 * 4 * 32 * 64
    assert lib.ikbo_lcb_emb_workspace_size(-1, 32, 64) == 0
    assert lcbe(lib, d=0) == ikbo.IKBO_INVALID_ARGUMENT
    assert lcbe(lib, nc=0) == ikbo.IKBO_INVALID_ARGUMENT
    assert lcbe(lib, kc=-1) == ikbo.IKBO_INVALID_ARGUMENT
    assert lcbe(lib, d=257) == ikbo.IKBO_UNSUPPORTED
    assert lcbe(lib, ind=7) == ikbo.IKBO_UNSUPPORTED
    assert lcbe(lib, norm=3) == ikbo.IKBO_INVALID_ARGUMENT
    assert lcbe(lib, eps=-1.0) == ikbo.IKBO_INVALID_ARGUMENT
    assert lcbe(lib, eps=float("nan")) == ikbo.IKBO_INVALID_ARGUMENT
    assert lcbe(lib, m=None, off=None) == ikbo.IKBO_INVALID_ARGUMENT
    assert lcbe(lib, flags=4) == ikbo.IKBO_INVALID_ARGUMENT
    for k in ("xc", "yc", "wcc", "wcr", "xr"):
        assert lcbe(lib, **{k: None}) == ikbo.IKBO_INVALID_ARGUMENT, k
    assert lcbe(lib, wrr=None) == ikbo.IKBO_INVALID_ARGUMENT
    for k in ("xr", "xc", "wrr", "wcr", "wcc", "gc", "bc", "yr", "yc", "ws"):
        assert lcbe(lib, **{k: MIS}) == ikbo.IKBO_MISALIGNED, k
    assert lcbe(lib, wsb=4 * 4 * 32 * 64 - 1) == ikbo.IKBO_WORKSPACE_TOO_SMALL
    assert lcbe(lib, ws=None) == ikbo.IKBO_WORKSPACE_TOO_SMALL
    assert lcbe(lib, C=0, yr=None) == ikbo.IKBO_OK        # nothing to compute
    assert lcbe(lib, kc=0, yr=None, ws=None, wsb=0) == ikbo.IKBO_OK


def test_probe_library_exports_and_rejects_bad_arguments():
    """The ceiling probes (include/ikbo_probe.h) load, export their one entry point, and refuse bad
    arguments before launching anything."""
    probe_h = os.path.join(os.path.dirname(HEADER), "ikbo_probe.h")
    names = set(re.findall(r"^\s*int\s+(ikbo_probe_[a-z_]+)\s*\(", open(probe_h).read(), re.M))
    assert names == {"ikbo_probe_launch"}
    if not os.path.exists(ikbo.PROBE_PATH):
        from request_candidate_broadcast_amd import _build
        _build.build_probe(verbose=False)
    out = subprocess.run(["nm", "-D", "--defined-only", ikbo.PROBE_PATH], stdout=subprocess.PIPE, text=True).stdout
    assert re.search(r"\bT ikbo_probe_launch\b", out)
    lib = ikbo.load_probe()
    assert lib.ikbo_probe_launch(0, None, 1 << 20, 10, 4, None) == 1          # NULL buffer
    assert lib.ikbo_probe_launch(0, FAKE, 1 << 20, 10, 0, None) == 1          # no blocks
    assert lib.ikbo_probe_launch(0, FAKE, 1000, 10, 4, None) == 1             # output too small
    assert lib.ikbo_probe_launch(9, FAKE, 1 << 20, 10, 4, None) == 1          # unknown probe
    assert lib.ikbo_probe_launch(2, FAKE + 4, 1 << 20, 0, 4, None) == 1       # misaligned copy


def test_dca_layer_checks_every_stage_before_launching(lib):
    # bf16 attention is built for head_dim 64 and 128. With 96 the call must fail before the query
    # generator is launched; without a GPU a launch would report IKBO_HIP_ERROR instead.
    W = 4 * 2 * 96
    layers = (ikbo.GlmLayer * 1)()
    layers[0] = ikbo.GlmLayer(FAKE, FAKE, FAKE, None, None, 64, 64, W, W, 0)
    need = lib.ikbo_dca_layer_workspace_size(32, 4, 1, layers, 64, 2, 96, 1)
    assert need > 0
    rc = lib.ikbo_dca_layer_forward(FAKE, 4, FAKE, 32, FAKE, None, 0, 1, layers, FAKE, 64, 128, None, 16, FAKE, FAKE,
                                    FAKE, FAKE, 4, 2, 96, 0.0, 1, FAKE, FAKE, FAKE, need, None)
    assert rc == ikbo.IKBO_UNSUPPORTED, lib.ikbo_last_error_message()
    assert b"head_dim" in lib.ikbo_last_error_message()
