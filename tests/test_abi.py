"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
entry point include/glance.h declares with the binding's signatures, and
rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

from tree_verified_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "glance.h")

OK_PTR = 0x100000  # 16-byte aligned stand-in; every call below fails validation first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(glance_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from tree_verified_block_amd import build
        build.build(verbose=False)
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(_lib.SIGNATURES), (names, sorted(_lib.SIGNATURES))
    for n in names:
        assert hasattr(lib, n), n


def test_helpers(lib):
    assert lib.glance_abi_version() == 1
    assert lib.glance_status_string(0) == b"ok"
    assert b"workspace" in lib.glance_status_string(-3)
    assert lib.glance_build_tree_ws(1, 15, 151936, 63) > 0
    assert lib.glance_build_tree_ws(0, 15, 151936, 63) == 0
    off = lib.glance_build_tree_flag_offset(1, 15, 151936, 63)
    assert 0 < off and off % 4 == 0 and off + 4 <= lib.glance_build_tree_ws(1, 15, 151936, 63)
    assert lib.glance_build_tree_flag_offset(1, 0, 151936, 63) == 0
    assert lib.glance_verify_head_ws(64, 151936, 4096, 1) >= 64 * 5 * 4
    assert lib.glance_tree_attn_ws(1, 64, 1024, 4096, 32, 8, 128) > 0


def _tree(lib, **kw):
    a = dict(logits=OK_PTR, dtype=1, root=OK_PTR, nseq=1, L=15, V=151936, N=63, out=OK_PTR,
             ws=OK_PTR * 16, ws_bytes=1 << 40)
    a.update(kw)
    o = a["out"]
    return lib.glance_build_tree(a["logits"], a["dtype"], a["root"], a["nseq"], a["L"], a["V"],
                                 a["N"], o, o, o, o, o, o, a["ws"], a["ws_bytes"], None)


def test_build_tree_rejects_bad_arguments(lib):
    assert _tree(lib, nseq=0) == -1
    assert _tree(lib, L=0) == -1
    assert _tree(lib, L=17) == -1
    assert _tree(lib, V=1) == -1
    assert _tree(lib, N=64) == -1
    assert _tree(lib, N=-1) == -1
    assert _tree(lib, dtype=7) == -1
    assert _tree(lib, logits=None) == -1
    assert b"draft_logits" in lib.glance_last_error()
    assert _tree(lib, logits=OK_PTR + 2) == -2
    assert _tree(lib, out=OK_PTR + 4) == -2
    assert _tree(lib, ws=None) == -3
    assert _tree(lib, ws=OK_PTR + 16) == -3          # not 256-byte aligned
    assert _tree(lib, ws_bytes=16) == -3
    assert b"needed" in lib.glance_last_error()


def test_build_tree_shared_rejects_bad_arguments(lib):
    p = OK_PTR

    def call(**kw):
        a = dict(logits=p, dtype=1, root=p, w=p, nseq=4, L=15, V=151936, n_max=63, budget=126,
                 tau=float("-inf"), out=p, ws=p * 16, ws_bytes=1 << 40)
        a.update(kw)
        o = a["out"]
        return lib.glance_build_tree_shared(a["logits"], a["dtype"], a["root"], a["w"], a["nseq"],
                                            a["L"], a["V"], a["n_max"], a["budget"], a["tau"], o, o,
                                            o, o, o, o, a["ws"], a["ws_bytes"], None)

    assert call(nseq=0) == -1
    assert call(nseq=17) == -1
    assert call(n_max=64) == -1
    assert call(n_max=-1) == -1
    assert call(budget=-1) == -1
    assert call(tau=float("nan")) == -1
    assert call(w=None) == -1
    assert call(w=p + 4) == -2
    assert call(L=17) == -1
    assert call(ws_bytes=64) == -3
    assert call(dtype=0, V=200000) == -4


def _head(lib, **kw):
    a = dict(h=OK_PTR, w=OK_PTR, dtype=1, R=64, d=4096, V=151936, out=OK_PTR, ws=OK_PTR * 16,
             ws_bytes=1 << 40)
    a.update(kw)
    o = a["out"]
    return lib.glance_verify_head(a["h"], a["w"], a["dtype"], a["R"], a["d"], a["V"], o, o, o, o,
                                  None, a["ws"], a["ws_bytes"], None)


def test_verify_head_rejects_bad_arguments(lib):
    assert _head(lib, R=0) == -1
    assert _head(lib, V=1) == -1
    assert _head(lib, d=4000) == -4       # bf16 needs d_model % 256 == 0
    assert _head(lib, w=OK_PTR + 8) == -2
    assert _head(lib, ws_bytes=100) == -3


def _head_sampled(lib, **kw):
    a = dict(h=OK_PTR, w=OK_PTR, dtype=1, R=64, d=4096, V=151936, T=1.0, out=OK_PTR,
             tok=OK_PTR, sgap=OK_PTR, ws=OK_PTR * 16, ws_bytes=1 << 40)
    a.update(kw)
    o = a["out"]
    return lib.glance_verify_head_sampled(a["h"], a["w"], a["dtype"], a["R"], a["d"], a["V"],
                                          a["T"], (1 << 63) + 5, (1 << 40) + 3, o, o, o, o,
                                          a["tok"], a["sgap"], None, a["ws"], a["ws_bytes"], None)


def test_verify_head_sampled_rejects_bad_arguments(lib):
    assert _head_sampled(lib, T=0.0) == -1
    assert _head_sampled(lib, T=-1.0) == -1
    assert _head_sampled(lib, T=float("nan")) == -1
    assert _head_sampled(lib, T=float("inf")) == -1
    assert _head_sampled(lib, tok=None) == -1
    assert _head_sampled(lib, sgap=None) == -1
    assert _head_sampled(lib, tok=OK_PTR + 2) == -2
    assert _head_sampled(lib, R=0) == -1
    assert _head_sampled(lib, d=4000) == -4
    assert _head_sampled(lib, ws_bytes=100) == -3
    # the workspace holds the sampled partials as well
    assert lib.glance_verify_head_ws(64, 151936, 4096, 1) >= 64 * 8 * 4


def test_head_pack_rejects_bad_arguments(lib):
    p = OK_PTR
    assert lib.glance_head_pack_bytes(151936, 4096) >= 151936 * 4096 * 2
    assert lib.glance_head_pack_bytes(151936, 4000) == 0
    assert lib.glance_head_pack_bytes(1, 4096) == 0
    assert lib.glance_head_pack(p, 1, 4096, p, None) == -1
    assert lib.glance_head_pack(p, 1000, 4000, p, None) == -4
    assert lib.glance_head_pack(None, 1000, 256, p, None) == -1
    assert lib.glance_head_pack(p, 1000, 256, p + 8, None) == -2

    def packed(**kw):
        a = dict(h=p, w=p, R=64, d=4096, V=151936, T=1.0, tok=None, sgap=None, ws=p * 16,
                 ws_bytes=1 << 40)
        a.update(kw)
        return lib.glance_verify_head_packed(a["h"], a["w"], a["R"], a["d"], a["V"], a["T"], 1, 2,
                                             p, p, p, p, a["tok"], a["sgap"], None, a["ws"],
                                             a["ws_bytes"], None)

    assert packed(w=None) == -1
    assert packed(w=p + 4) == -2
    assert packed(R=0) == -1
    assert packed(d=4000) == -4
    assert packed(ws_bytes=100) == -3
    assert packed(tok=p, sgap=p, T=0.0) == -1      # sampling needs T > 0
    assert packed(tok=p) == -1                     # both draw outputs or neither

    def noalloc(R):
        return lib.glance_verify_head_packed_noalloc(p, p, R, 4096, 151936, 1.0, 1, 2, p, p, p, p,
                                                     None, None, None, None)

    # rows are checked, and sizes beyond the fixed scratch rejected, before any device call
    assert noalloc(0) == -1
    assert lib.glance_verify_head_ws(551, 151936, 4096, 1) <= 8 << 20
    assert lib.glance_verify_head_ws(552, 151936, 4096, 1) > 8 << 20
    assert noalloc(552) == -4
    assert b"scratch" in lib.glance_last_error()


def test_entropy_log_value_rejects_bad_arguments(lib):
    p = OK_PTR
    assert lib.glance_entropy_log_value(p, 0, 1, 0.96, 0.63, 15, p, None) == -1
    assert lib.glance_entropy_log_value(p, 4, 0, 0.96, 0.63, 15, p, None) == -1
    assert lib.glance_entropy_log_value(p, 4, 1, 0.96, 0.63, 0, p, None) == -1
    assert lib.glance_entropy_log_value(p, 4, 1, float("nan"), 0.63, 15, p, None) == -1
    assert lib.glance_entropy_log_value(p, 4, 1, 0.96, float("inf"), 15, p, None) == -1
    assert lib.glance_entropy_log_value(None, 4, 1, 0.96, 0.63, 15, p, None) == -1
    assert lib.glance_entropy_log_value(p, 4, 1, 0.96, 0.63, 15, None, None) == -1
    assert lib.glance_entropy_log_value(p + 2, 4, 1, 0.96, 0.63, 15, p, None) == -2


def test_attn_pack_rejects_bad_arguments(lib):
    p = OK_PTR
    qkv = ((32 + 16) * 128 // 16) * (4096 // 64) * 2048
    wo = (4096 // 16) * (32 * 128 // 64) * 2048
    assert lib.glance_attn_pack_bytes(4096, 32, 8, 128) == ((qkv + 255) // 256) * 256 + wo
    assert lib.glance_attn_pack_bytes(4000, 32, 8, 128) == 0
    assert lib.glance_attn_pack_bytes(4096, 32, 8, 64) == 0
    assert lib.glance_attn_pack_bytes(4096, 30, 8, 128) == 0
    assert lib.glance_attn_pack(p, p, p, p, 4096, 32, 8, 64, p, None) == -4
    assert lib.glance_attn_pack(None, p, p, p, 4096, 32, 8, 128, p, None) == -1
    assert lib.glance_attn_pack(p, p, p, p + 8, 4096, 32, 8, 128, p, None) == -2
    assert lib.glance_attn_pack(p, p, p, p, 4096, 32, 8, 128, None, None) == -1
    # a packed copy is bf16 only, and replaces the four row-major pointers
    assert _attn(lib, dtype=0, D=64, packed=p) == -4
    assert _attn(lib, layer=None, packed=p, ws_bytes=100) == -3


def _attn(lib, **kw):
    a = dict(dtype=1, embed=OK_PTR, h_in=None, nseq=1, n_rows=64, d=4096, Hq=32, Hkv=8, D=128,
             max_prefix=1024, n_pos=2048, ws=OK_PTR * 16, ws_bytes=1 << 40, layer=OK_PTR,
             packed=None)
    a.update(kw)
    lay = _lib.GlanceAttnLayer(*(a["layer"],) * 4, OK_PTR, OK_PTR, a["packed"])
    p = OK_PTR
    return lib.glance_tree_attn(ctypes.byref(lay), a["dtype"], a["embed"], p, a["h_in"], p, p,
                                a["max_prefix"], p, p, p, p, a["n_pos"], a["nseq"], a["n_rows"],
                                a["d"], a["Hq"], a["Hkv"], a["D"], None, None, None, a["ws"],
                                a["ws_bytes"], None)


def test_tree_layer_rejects_bad_arguments(lib):
    p = OK_PTR

    def call(inter=12288, eps=1e-6, D=128, d=4096, gate=p, ws_bytes=1 << 40):
        attn = _lib.GlanceAttnLayer(*(p,) * 6)
        full = _lib.GlanceFullLayer(attn, p, p, p, p, gate, p, p, inter, eps)
        return lib.glance_tree_layer(ctypes.byref(full), p, p, None, p, p, 1024, p, p, p, p, 2048,
                                     1, 64, d, 32, 8, D, None, None, None, p * 16, ws_bytes, None)

    assert lib.glance_tree_layer_ws(1, 64, 1024, 4096, 32, 8, 128, 12288) > \
        lib.glance_tree_attn_ws(1, 64, 1024, 4096, 32, 8, 128)
    assert lib.glance_tree_layer_ws(1, 64, 1024, 4096, 32, 8, 64, 12288) == 0
    assert call(inter=1000) == -4
    assert call(D=64) == -4
    assert call(d=4000) == -4
    assert call(eps=float("nan")) == -1
    assert call(eps=-1.0) == -1
    assert call(gate=None) == -1
    assert call(gate=p + 2) == -2
    assert call(ws_bytes=1000) == -3


def test_mlp_pack_rejects_bad_arguments(lib):
    p = OK_PTR
    assert lib.glance_mlp_pack_bytes(4096, 12288) >= 3 * 4096 * 12288 * 2
    assert lib.glance_mlp_pack_bytes(4096, 1000) == 0
    assert lib.glance_mlp_pack(p, p, p, 4096, 1000, p, None) == -4
    assert lib.glance_mlp_pack(None, p, p, 4096, 12288, p, None) == -1
    assert lib.glance_mlp_pack(p, p, p, 4096, 12288, p + 8, None) == -2


def test_tree_attn_rejects_bad_arguments(lib):
    assert _attn(lib, n_rows=65) == -1
    assert _attn(lib, Hq=30) == -1            # not a multiple of Hkv
    assert _attn(lib, D=64) == -4             # bf16 path is head_dim 128
    assert _attn(lib, embed=None) == -1       # neither embed nor h_in
    assert _attn(lib, n_pos=100) == -1
    # every row's position P + depth (depth < n_rows) needs a table row
    assert _attn(lib, max_prefix=1024, n_pos=1024 + 63) == -1
    assert _attn(lib, max_prefix=1024, n_pos=1024 + 64, ws_bytes=1000) == -3
    assert _attn(lib, layer=OK_PTR + 2) == -2
    assert _attn(lib, dtype=0, max_prefix=9000, n_pos=10000) == -4
    assert _attn(lib, ws_bytes=1000) == -3


def test_accept_walk_rejects_bad_arguments(lib):
    p = OK_PTR
    assert lib.glance_accept_walk(p, p, p, p, p, 0, 64, 15, 1e-3, p, p, p, p, None) == -1
    assert lib.glance_accept_walk(p, p, p, p, p, 1, 65, 15, 1e-3, p, p, p, p, None) == -1
    assert lib.glance_accept_walk(p, p, p, p, p, 1, 64, 0, 1e-3, p, p, p, p, None) == -1
    assert lib.glance_accept_walk(None, p, p, p, p, 1, 64, 15, 1e-3, p, p, p, p, None) == -1
    assert lib.glance_accept_walk(p, p, p, p, p + 4, 1, 64, 15, 1e-3, p, p, p, p, None) == -2


def test_commit_and_advance_reject_bad_arguments(lib):
    p = OK_PTR
    ok = dict(tk=p, tv=p, dtype=1, path=p, na=p, nseq=1, L=15, Hkv=8, D=128, kvo=p, kc=p, vc=p,
              cap=2048)

    def commit(**kw):
        a = {**ok, **kw}
        return lib.glance_commit_kv(a["tk"], a["tv"], a["dtype"], a["path"], a["na"], a["nseq"],
                                    a["L"], a["Hkv"], a["D"], a["kvo"], a["kc"], a["vc"], a["cap"],
                                    None)

    assert commit(nseq=2) == -4
    assert commit(dtype=7) == -1
    assert commit(L=0) == -1
    assert commit(L=17) == -1
    assert commit(Hkv=1, D=2, dtype=0) == -1  # 8-byte rows
    assert commit(cap=-1) == -1
    assert commit(kc=None) == -1
    assert commit(vc=p + 8) == -2
    assert lib.glance_advance_round(p, p, 2, p, p, None) == -4
    assert lib.glance_advance_round(p, None, 1, p, p, None) == -1
    assert lib.glance_advance_round(p, p, 1, p + 4, p, None) == -2


def test_binding_requires_built_library(tmp_path):
    """The binding never falls back: a missing library raises."""
    with pytest.raises(RuntimeError, match="missing"):
        saved = _lib._lib
        _lib._lib = None
        try:
            _lib.load(str(tmp_path / "nope.so"))
        finally:
            _lib._lib = saved


def test_tree_outputs_start_as_an_empty_tree():
    """The binding allocates the tree outputs as a tree of padding rows, so that
    a layer call made before any tree build (the layer gathers embed[token]
    without a bound on the token) reads only the padding marker."""
    from tree_verified_block_amd import api
    out = api.tree_outputs(3, 7, "cpu")
    assert set(out) == {"parent", "depth", "token", "anc", "score", "n_valid"}
    assert out["token"].shape == (3, 8) and bool((out["token"] == -1).all())
    assert bool((out["parent"] == -1).all()) and bool((out["depth"] == 0).all())
    assert bool((out["anc"] == 0).all()) and bool((out["n_valid"] == 0).all())


def test_head_timing_rejects_a_single_event(lib):
    p = ctypes.c_void_p(64)
    assert lib.glance_head_timing(p, None) == -1
    assert lib.glance_head_timing(None, p) == -1
    assert lib.glance_head_timing(None, None) == 0


def test_read_probe_rejects_bad_arguments(lib):
    p = ctypes.c_void_p(256)
    assert lib.glance_read_probe(p, 0, 1, p, None) == -1
    assert lib.glance_read_probe(p, 24, 1, p, None) == -1
    assert lib.glance_read_probe(p, 32, 0, p, None) == -1
    assert lib.glance_read_probe(p, 32, 65537, p, None) == -1
    assert lib.glance_read_probe(None, 32, 1, p, None) == -1
    assert lib.glance_read_probe(p, 32, 1, None, None) == -1
    assert lib.glance_read_probe(ctypes.c_void_p(264), 32, 1, p, None) == -2

