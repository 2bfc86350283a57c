"""C ABI of libw8a8 without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

from w8a8_int8_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")

OK, ENULL, ESHAPE, EALIGN, EDTYPE, EARG = 0, 1, 2, 3, 4, 5

# Fake, never dereferenced device addresses: every call below must fail its
# host-side checks.  With a GPU present these tests are skipped (a validation
# bug would then launch a kernel on them); the GPU suite covers error paths
# with real buffers.
P = 1 << 20  # 16-byte aligned, non-null
PODD = P + 4  # 4-byte aligned only

cpu_only = pytest.mark.skipif(torch.cuda.is_available(),
                              reason="fake pointers are only safe without a GPU")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_header_symbols():
    lib = _lib.load()
    syms = declared_symbols()
    assert len(syms) == 20
    for s in syms:
        assert hasattr(lib, s), s
        assert s in _lib.PROTOTYPES, s
    assert lib.w8a8_abi_version() == 7


def declared_prototypes():
    """name -> list of parameter declarations, from the header's prototypes."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(w8a8_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        params = [p.strip() for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
        out[m.group(1)] = params
    return out


def test_binding_prototypes_match_the_header():
    """The binding's argument lists follow the header: same count, and the
    pointer / integer / floating kind of every parameter."""
    def kind_decl(p):
        if "*" in p or "hipStream_t" in p:
            return "ptr"
        if p.startswith("double") or p.startswith("float"):
            return "fp"
        return "int"

    def kind_ct(t):
        if t is ctypes.c_void_p:
            return "ptr"
        if t in (ctypes.c_double, ctypes.c_float):
            return "fp"
        return "int"

    decl = declared_prototypes()
    assert sorted(decl) == sorted(_lib.PROTOTYPES)
    for name, params in decl.items():
        args = _lib.PROTOTYPES[name][1]
        assert [kind_decl(p) for p in params] == [kind_ct(t) for t in args], name
    # the two calls whose form departs from the first sketch of the boundary:
    # device-side smoothing factors on a stream, and a workspace size that
    # depends on N (the split-K partial sums are S x M x N)
    assert decl["w8a8_smooth_factors"][-1].startswith("hipStream_t")
    assert [p.split()[-1] for p in decl["w8a8_linear_workspace_bytes"]] == ["M", "N", "K"]


def test_status_strings():
    lib = _lib.load()
    for code in range(0, 8):
        s = lib.w8a8_status_str(code)
        assert s and s.decode()
    assert lib.w8a8_status_str(99).decode() == "unknown status"


def test_workspace_bytes():
    lib = _lib.load()
    assert lib.w8a8_linear_workspace_bytes(0, 0, 0) == 0
    assert lib.w8a8_linear_workspace_bytes(1, 8, 16) == 256 + 256  # one split: no partials
    assert lib.w8a8_linear_workspace_bytes(2048, 4096, 4096) == 2048 * 4096 + 2048 * 4
    assert lib.w8a8_linear_workspace_bytes(-1, 8, 16) == 0
    # The runtime forward splits K at 17-32 tokens below 12288 output channels
    # when rows have 32 or more 256-byte pieces, and at 3-16 tokens below 2048
    # channels when they have 64 or more: blocks of 64 channels, about 256
    # blocks, at least 8 pieces per split, at most 16 splits.  The workspace
    # adds the int32 slices (splits x M x N) and one 4-byte counter per
    # 64-channel group, each rounded up to 256 bytes.
    # 1024 channels: 16 groups; K = 16384 is 64 pieces: 8 splits
    assert lib.w8a8_linear_workspace_bytes(32, 1024, 16384) == 32 * 16384 + 256 + 8 * 32 * 1024 * 4 + 256
    assert lib.w8a8_linear_workspace_bytes(24, 1024, 16384) == 24 * 16384 + 256 + 8 * 24 * 1024 * 4 + 256
    assert lib.w8a8_linear_workspace_bytes(8, 1024, 16384) == 8 * 16384 + 256 + 8 * 8 * 1024 * 4 + 256
    assert lib.w8a8_linear_workspace_bytes(3, 1024, 16384) == 3 * 16384 + 256 + (8 * 3 * 1024 * 4) + 256
    # 4096 channels: 64 groups, 4 splits; 2048: 32 groups, 8 splits
    assert lib.w8a8_linear_workspace_bytes(32, 4096, 16384) == 32 * 16384 + 256 + 4 * 32 * 4096 * 4 + 256
    assert lib.w8a8_linear_workspace_bytes(32, 2048, 16384) == 32 * 16384 + 256 + 8 * 32 * 2048 * 4 + 256
    # (slices rounded up to 256 bytes): 2040 channels, 32 pieces: 32 groups, 4 splits
    assert lib.w8a8_linear_workspace_bytes(17, 2040, 8192) == 17 * 8192 + 256 + (4 * 17 * 2040 * 4 + 128) + 256
    # unsplit: rows of 16 pieces at 17-32 tokens, at 3-16 tokens rows of fewer
    # than 64 pieces or 2048 channels or more, 12288 channels or more, 1-2 tokens
    assert lib.w8a8_linear_workspace_bytes(32, 1024, 4096) == 32 * 4096 + 256
    assert lib.w8a8_linear_workspace_bytes(17, 2040, 4096) == 17 * 4096 + 256
    assert lib.w8a8_linear_workspace_bytes(32, 4096, 4096) == 32 * 4096 + 256
    assert lib.w8a8_linear_workspace_bytes(16, 1024, 8192) == 16 * 8192 + 256
    assert lib.w8a8_linear_workspace_bytes(16, 2048, 16384) == 16 * 16384 + 256
    assert lib.w8a8_linear_workspace_bytes(32, 16384, 4096) == 32 * 4096 + 256
    assert lib.w8a8_linear_workspace_bytes(32, 12288, 16384) == 32 * 16384 + 256
    assert lib.w8a8_linear_workspace_bytes(2, 1024, 16384) == 2 * 16384 + 256


@cpu_only
def test_channel_amax_rejects():
    f = _lib.load().w8a8_channel_amax
    assert f(0, 0, 4, 8, P, 0) == ENULL
    assert f(0, 0, 0, 8, 0, 0) == ENULL  # amax is always required
    assert f(P, 0, 4, 8, 0, 0) == ENULL
    assert f(P, 7, 4, 8, P, 0) == EDTYPE
    assert f(P, 0, -1, 8, P, 0) == ESHAPE
    assert f(P, 0, 4, 0, P, 0) == ESHAPE
    assert f(P, 0, 4, 12, P, 0) == ESHAPE
    assert f(PODD, 0, 4, 8, P, 0) == EALIGN
    assert f(P, 1, 4, 8, P + 2, 0) == EALIGN


@cpu_only
def test_smooth_factors_rejects():
    f = _lib.load().w8a8_smooth_factors
    assert f(0, P, 8, 0.5, P, P, 0) == ENULL
    assert f(P, P, 8, 0.5, P, 0, 0) == ENULL
    assert f(0, 0, 0, 0.5, 0, 0, 0) == OK  # K == 0: nothing to do, no launch
    assert f(P, P, -1, 0.5, P, P, 0) == ESHAPE
    assert f(P, P, 8, -0.01, P, P, 0) == EARG
    assert f(P, P, 8, 1.5, P, P, 0) == EARG
    assert f(P, P, 8, float("nan"), P, P, 0) == EARG
    assert f(P + 2, P, 8, 0.5, P, P, 0) == EALIGN


@cpu_only
def test_scale_quant_rows_rejects():
    f = _lib.load().w8a8_scale_quant_rows
    assert f(0, 0, 4, 16, P, P, P, 0) == ENULL
    assert f(P, 0, 4, 16, P, P, 0, 0) == ENULL
    assert f(0, 0, 0, 16, P, 0, 0, 0) == OK  # no rows: nothing to do, no launch
    assert f(P, 2, 4, 16, P, P, P, 0) == EDTYPE
    assert f(P, 0, -4, 16, P, P, P, 0) == ESHAPE
    assert f(P, 0, 4, 24, P, P, P, 0) == ESHAPE  # cols % 16
    assert f(P, 0, 4, 65536 + 16, P, P, P, 0) == ESHAPE
    assert f(PODD, 0, 4, 16, P, P, P, 0) == EALIGN
    assert f(P, 0, 4, 16, PODD, P, P, 0) == EALIGN
    assert f(P, 0, 4, 16, P, PODD, P, 0) == EALIGN
    assert f(P, 0, 4, 16, P, P, P + 2, 0) == EALIGN


@cpu_only
def test_scale_quant_pair_rejects():
    """Each matrix is checked as w8a8_scale_quant_rows checks it, before any launch."""
    f = _lib.load().w8a8_scale_quant_pair
    # w, N, s, qw, sw, x, M, inv_s, qx, sx, dtype, K, stream
    assert f(0, 4, P, P, P, P, 4, P, P, P, 0, 16, 0) == ENULL
    assert f(P, 4, P, P, P, P, 4, P, P, 0, 0, 16, 0) == ENULL
    assert f(0, 0, P, 0, 0, 0, 0, P, 0, 0, 0, 16, 0) == OK  # no rows: no launch
    assert f(P, 4, P, P, P, P, 4, P, P, P, 2, 16, 0) == EDTYPE
    assert f(P, -4, P, P, P, P, 4, P, P, P, 0, 16, 0) == ESHAPE
    assert f(P, 4, P, P, P, P, -4, P, P, P, 0, 16, 0) == ESHAPE
    assert f(P, 4, P, P, P, P, 4, P, P, P, 0, 24, 0) == ESHAPE  # K % 16
    assert f(P, 4, P, P, P, P, 4, P, P, P, 0, 65536 + 16, 0) == ESHAPE
    assert f(P, 1 << 30, P, P, P, P, 1 << 30, P, P, P, 0, 16, 0) == ESHAPE  # M + N
    assert f(PODD, 4, P, P, P, P, 4, P, P, P, 0, 16, 0) == EALIGN
    assert f(P, 4, P, P, P, PODD, 4, P, P, P, 0, 16, 0) == EALIGN
    assert f(P, 4, P, P, P, P, 4, PODD, P, P, 0, 16, 0) == EALIGN
    assert f(P, 4, P, P, P, P, 4, P, P, P + 2, 0, 16, 0) == EALIGN


@cpu_only
def test_gemm_rejects():
    lib = _lib.load()
    g = lib.w8a8_gemm_i32
    assert g(0, P, P, 4, 8, 16, 0) == ENULL
    assert g(P, P, 0, 4, 8, 16, 0) == ENULL
    assert g(0, P, 0, 0, 8, 16, 0) == OK  # empty output: no launch
    assert g(P, P, P, -1, 8, 16, 0) == ESHAPE
    assert g(P, P, P, 4, 12, 16, 0) == ESHAPE  # N % 8
    assert g(P, P, P, 4, 8, 24, 0) == ESHAPE  # K % 16
    assert g(P, P, P, 4, 8, 131072 + 16, 0) == ESHAPE  # int32 exactness bound
    assert g(PODD, P, P, 4, 8, 16, 0) == EALIGN
    assert g(P, P, PODD, 4, 8, 16, 0) == EALIGN
    d = lib.w8a8_gemm_dequant
    assert d(P, 0, P, P, P, 0, 4, 8, 16, 0) == ENULL
    assert d(P, P, P, P, P, 3, 4, 8, 16, 0) == EDTYPE
    assert d(P, P, P, PODD, P, 0, 4, 8, 16, 0) == EALIGN
    assert d(P, P, P, P, P, 0, 4, 9, 16, 0) == ESHAPE


def test_calibrate_smooth_scratch_bytes():
    f = _lib.load().w8a8_calibrate_smooth_scratch_bytes
    assert f(4096) == 4 * 4096 + 4 * 16
    assert f(4104) == 4 * 4160 + 4 * 17  # 64-float padding, one counter per 256 channels
    assert f(8) == 256 + 4
    assert f(0) == 0 and f(12) == 0 and f(-8) == 0


@cpu_only
def test_calibrate_smooth_rejects():
    lib = _lib.load()
    f = lib.w8a8_calibrate_smooth
    need = lib.w8a8_calibrate_smooth_scratch_bytes(64)
    args = [P, 4, P, 8, 0, 64, 0.5, P, P, P, P, P, need, 0]

    def call(**kw):
        a = list(args)
        names = ["x", "cal_rows", "w", "N", "dtype", "K", "alpha", "ax", "aw", "s", "inv_s",
                 "scratch", "nbytes", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(dtype=2) == EDTYPE
    assert call(K=12) == ESHAPE and call(K=0) == ESHAPE and call(N=-1) == ESHAPE
    assert call(cal_rows=-1) == ESHAPE
    assert call(x=0) == ENULL and call(w=0) == ENULL and call(scratch=0) == ENULL
    assert call(ax=0) == ENULL and call(inv_s=0) == ENULL
    assert call(alpha=1.5) == EARG and call(alpha=float("nan")) == EARG
    assert call(nbytes=need - 1) == EARG
    assert call(x=PODD) == EALIGN and call(scratch=P + 4) == EALIGN and call(s=P + 2) == EALIGN


def test_calib_layer_struct_matches_the_header():
    """The binding's w8a8_calib_layer_t has the header's fields, in order, with
    the pointer / integer / floating kind of each, and no padding."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\}\s*w8a8_calib_layer_t;", text, flags=re.S).group(1)
    decls = [d.strip() for d in body.split(";") if d.strip()]
    names = [d.split()[-1].lstrip("*") for d in decls]
    assert names == [f[0] for f in _lib.CalibLayer._fields_]
    for d, (_, t) in zip(decls, _lib.CalibLayer._fields_):
        kind = "ptr" if "*" in d else "fp" if d.startswith("double") else "int"
        assert kind == ("ptr" if t is ctypes.c_void_p else "fp" if t is ctypes.c_double else "int"), d
    assert ctypes.sizeof(_lib.CalibLayer) == 8 * len(names)


@cpu_only
def test_calibrate_smooth_layers_rejects():
    """Every entry is checked before anything is enqueued; a bad entry
    anywhere in the array fails the whole call."""
    lib = _lib.load()
    f = lib.w8a8_calibrate_smooth_layers
    need = lib.w8a8_calibrate_smooth_scratch_bytes(64)

    def entry(**kw):
        e = dict(x_cal=P, cal_rows=4, w=P, N=8, K=64, alpha=0.5, amax_x=P, amax_w=P, s=P, inv_s=P,
                 scratch=P, scratch_bytes=need)
        e.update(kw)
        return _lib.CalibLayer(**e)

    def call(entries, dtype=0, n=None):
        arr = (_lib.CalibLayer * max(1, len(entries)))(*entries)
        return f(ctypes.addressof(arr), len(entries) if n is None else n, dtype, 0)

    assert f(None, 0, 0, 0) == 0  # nothing to do
    assert f(None, 1, 0, 0) == ENULL
    assert call([entry()], n=-1) == ESHAPE
    assert call([entry()], dtype=2) == EDTYPE
    for bad, code in ((dict(K=12), ESHAPE), (dict(N=-1), ESHAPE), (dict(cal_rows=-1), ESHAPE),
                      (dict(x_cal=0), ENULL), (dict(scratch=0), ENULL), (dict(inv_s=0), ENULL),
                      (dict(alpha=1.5), EARG), (dict(alpha=float("nan")), EARG),
                      (dict(scratch_bytes=need - 1), EARG), (dict(w=PODD), EALIGN),
                      (dict(s=P + 2), EALIGN)):
        # the bad entry last, after good ones: still rejected before any launch
        assert call([entry(), entry(), entry(**bad)]) == code, bad
    # entries past 8 are checked too (they would go to a second launch)
    assert call([entry()] * 9 + [entry(K=0)]) == ESHAPE


@cpu_only
def test_linear_rejects():
    lin = _lib.load().w8a8_linear
    need = _lib.load().w8a8_linear_workspace_bytes(4, 8, 16)
    assert lin(P, 0, P, P, P, P, 4, 8, 16, 0, need, 0) == ENULL
    assert lin(P, 5, P, P, P, P, 4, 8, 16, P, need, 0) == EDTYPE
    assert lin(P, 0, P, P, P, P, 4, 8, 16, P, need - 1, 0) == EARG
    assert lin(P, 0, P, P, P, P, 4, 8, 16, P + 16, need, 0) == EALIGN  # workspace 256 B
    assert lin(P, 0, P, P, P, P, 4, 8, 24, P, 1 << 20, 0) == ESHAPE
    assert lin(P, 0, P, P, P, P, 4, 12, 16, P, need, 0) == ESHAPE


@cpu_only
def test_linear_noalloc_rejects():
    f = _lib.load().w8a8_linear_noalloc
    assert f(P, 0, P, P, P, P, 4096, 16, 16384, 0) == 7  # more than the static scratch
    assert f(P, 0, P, P, P, P, -1, 8, 16, 0) == ESHAPE
    assert f(P, 5, P, P, P, P, 4, 8, 16, 0) == EDTYPE
    assert f(P, 0, P, P, 0, P, 4, 8, 16, 0) == ENULL
    assert f(P, 0, P, P, P, P, 4, 8, 24, 0) == ESHAPE
    assert f(PODD, 0, P, P, P, P, 4, 8, 16, 0) == EALIGN
    assert f(P, 0, P, P, PODD, P, 4, 8, 16, 0) == EALIGN


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError, match="no fallback"):
        _lib.load()


@cpu_only
def test_gemm_float_rejects():
    g = _lib.load().w8a8_gemm_float
    assert g(0, P, P, 0, 4, 8, 16, 0) == ENULL
    assert g(P, P, P, 2, 4, 8, 16, 0) == EDTYPE
    assert g(P, P, P, 0, 4, 8, 12, 0) == ESHAPE  # K % 8
    assert g(P, P, P, 0, 4, 12, 16, 0) == ESHAPE  # N % 8
    assert g(P, P, P, 0, 4, 8, (1 << 20) + 8, 0) == ESHAPE
    assert g(PODD, P, P, 0, 4, 8, 16, 0) == EALIGN
    assert g(0, P, 0, 0, 0, 8, 16, 0) == OK  # empty output: no launch


@cpu_only
def test_e4m3_entry_points_reject():
    lib = _lib.load()
    f = lib.w8a8_scale_quant_rows_e4m3
    assert f(0, 0, 4, 16, P, P, P, 0) == ENULL
    assert f(0, 0, 0, 16, P, 0, 0, 0) == OK  # no rows: nothing to do, no launch
    assert f(P, 2, 4, 16, P, P, P, 0) == EDTYPE
    assert f(P, 0, 4, 24, P, P, P, 0) == ESHAPE  # cols % 16
    assert f(P, 0, 4, 16, P, PODD, P, 0) == EALIGN
    d = lib.w8a8_gemm_dequant_e4m3
    assert d(P, 0, P, P, P, 0, 4, 8, 16, 0) == ENULL
    assert d(P, P, P, P, P, 3, 4, 8, 16, 0) == EDTYPE
    assert d(P, P, P, P, P, 0, 4, 8, 24, 0) == ESHAPE  # K % 16
    assert d(P, P, P, P, P, 0, 4, 9, 16, 0) == ESHAPE  # N % 8
    assert d(PODD, P, P, P, P, 0, 4, 8, 16, 0) == EALIGN
    assert d(P, P, P, PODD, P, 0, 4, 8, 16, 0) == EALIGN
    assert d(0, 0, P, P, 0, 0, 0, 8, 16, 0) == OK  # no tokens: no launch


@cpu_only
def test_rmsnorm_quant_rows_rejects():
    lib = _lib.load()
    f = lib.w8a8_rmsnorm_quant_rows
    assert f(P, 0, 4, 16, 0, 1e-5, P, P, 0) == ENULL  # g
    assert f(P, 3, 4, 16, P, 1e-5, P, P, 0) == EDTYPE
    assert f(P, 0, 4, 24, P, 1e-5, P, P, 0) == ESHAPE
    assert f(P, 0, 4, 0, P, 1e-5, P, P, 0) == ESHAPE  # empty rows have no mean
    assert f(P, 0, 4, 16, PODD, 1e-5, P, P, 0) == EALIGN
    assert f(P, 0, 4, 16, P, -1e-5, P, P, 0) == EARG
    assert f(P, 0, 4, 16, P, float("nan"), P, P, 0) == EARG
    assert f(P, 0, 4, 16, P, float("inf"), P, P, 0) == EARG
    assert f(0, 0, 0, 16, P, 1e-5, 0, 0, 0) == OK  # no rows: no launch
    fold = lib.w8a8_fold_norm_weight
    assert fold(P, 0, 8, P, 0) == ENULL
    assert fold(P, P, -1, P, 0) == ESHAPE
    assert fold(P, P, 8, P + 2, 0) == EALIGN
    assert fold(0, 0, 0, 0, 0) == OK


@cpu_only
def test_layernorm_quant_rows_rejects():
    lib = _lib.load()
    f = lib.w8a8_layernorm_quant_rows
    assert f(P, 0, 4, 16, P, 0, 1e-5, P, P, 0) == ENULL  # b
    assert f(P, 0, 4, 16, 0, P, 1e-5, P, P, 0) == ENULL  # g
    assert f(P, 1, 4, 16, P, P, 1e-5, P, P, 0) == EDTYPE  # bf16: no exact row sums
    assert f(P, 3, 4, 16, P, P, 1e-5, P, P, 0) == EDTYPE
    assert f(P, 0, 4, 24, P, P, 1e-5, P, P, 0) == ESHAPE
    assert f(P, 0, 4, 0, P, P, 1e-5, P, P, 0) == ESHAPE  # empty rows have no mean
    assert f(P, 0, 4, 65552, P, P, 1e-5, P, P, 0) == ESHAPE
    assert f(P, 0, 4, 16, P, PODD, 1e-5, P, P, 0) == EALIGN
    assert f(P, 0, 4, 16, P, P, -1e-5, P, P, 0) == EARG
    assert f(P, 0, 4, 16, P, P, float("nan"), P, P, 0) == EARG
    assert f(0, 0, 0, 16, P, P, 1e-5, 0, 0, 0) == OK  # no rows: no launch
