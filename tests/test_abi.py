"""The C ABI: every symbol include/mxsg.h declares is exported by libmxsg.so,
and argument errors are reported on the host before any HIP call (so these
run without a GPU)."""
import ctypes
import os
import re

import pytest

from mx_scaled_grouped_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxsg.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libmxsg.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxsg_[a-z_]+)\s*\(", text)))


def test_header_matches_binding():
    assert _declared() == sorted(_lib.SIGNATURES)


def _declared_arity():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(mxsg_[a-z_]+)\s*\(([^)]*)\)\s*;", text):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_header_arity_matches_binding():
    arity = _declared_arity()
    for name, (_, argtypes) in _lib.SIGNATURES.items():
        assert arity[name] == len(argtypes), (name, arity[name], len(argtypes))


def test_status_bits_match_header():
    from mx_scaled_grouped_amd import api
    text = open(HEADER).read()
    bits = {k: int(v) for k, v in re.findall(r"#define MXSG_STATUS_(\w+) (\d+)", text)}
    assert bits == {"ENDS_DECREASING": api.STATUS_ENDS_DECREASING, "ENDS_RANGE": api.STATUS_ENDS_RANGE,
                    "ENDS_TOTAL": api.STATUS_ENDS_TOTAL, "NONFINITE": api.STATUS_NONFINITE,
                    "BAD_EXPERT": api.STATUS_BAD_EXPERT}
    assert len(set(bits.values())) == 5 and all(v & (v - 1) == 0 for v in bits.values())


def test_all_symbols_exported():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = _lib.load()
    assert lib.mxsg_status_str(0) == b"ok"
    assert lib.mxsg_status_str(2) == b"bad shape"
    assert lib.mxsg_status_str(99) == b"unknown status"
    assert lib.mxsg_version() >= 100


def test_padded_capacity():
    lib = _lib.load()
    for M, E in [(0, 1), (1, 1), (1024, 4), (16384, 8), (98304, 64), (5, 3)]:
        cap = lib.mxsg_padded_capacity(M, E)
        assert cap % 128 == 0
        # the worst case: every group holds 1 mod 128 tokens
        assert cap >= M + 127 * E - 127 * 0 - ((M + 127 * E) % 128)
        assert cap >= ((M + 127 * E) // 128) * 128
    assert lib.mxsg_padded_capacity(-1, 1) == -1


FAKE = 0x1000  # a non-null pointer that is never dereferenced: validation fails first


def _qact(**kw):
    args = dict(x=FAKE, M=16, C=256, recipe=0, fmt=0, E=1, ends=FAKE, rc=FAKE, rs=FAKE, cc=None,
                cs=None, ld=0, ps=None, amax=FAKE, dls=None, dli=None)
    args.update(kw)
    return _lib.status_of("mxsg_quantize_act", *args.values(), None, None)


def test_quantize_act_validation():
    assert _qact(recipe=7) == _lib.INVALID_ARGUMENT
    assert _qact(fmt=5) == _lib.INVALID_ARGUMENT
    assert _qact(fmt=2) == _lib.UNSUPPORTED                 # e2m1 only with MX
    assert _qact(C=200) == _lib.BAD_SHAPE                   # feature dim % 128
    assert _qact(M=-1) == _lib.INVALID_ARGUMENT
    assert _qact(rc=None) == _lib.INVALID_ARGUMENT          # no output at all
    assert _qact(amax=None) == _lib.INVALID_ARGUMENT        # tensorwise needs amax
    assert _qact(recipe=1, dls=None) == _lib.INVALID_ARGUMENT
    assert _qact(recipe=2, rs=None) == _lib.INVALID_ARGUMENT
    # column-wise: needs groups, padded starts and a large enough ld
    assert _qact(cc=FAKE, cs=FAKE, E=0, ps=FAKE, ld=256) == _lib.INVALID_ARGUMENT
    assert _qact(cc=FAKE, cs=FAKE, ps=None, ld=256) == _lib.INVALID_ARGUMENT
    assert _qact(cc=FAKE, cs=FAKE, ps=FAKE, ld=100) == _lib.BAD_SHAPE
    assert _qact(cc=FAKE, cs=FAKE, ps=FAKE, ld=128, M=200) == _lib.BAD_SHAPE
    assert b"ld" in _lib.load().mxsg_last_error()


def _qag(**kw):
    args = dict(x=FAKE, T=100, idx=FAKE, M=16, C=256, recipe=0, fmt=0, E=1, ends=FAKE, rc=FAKE,
                rs=FAKE, cc=None, cs=None, ld=0, ps=None, amax=FAKE, dls=None, dli=None)
    args.update(kw)
    return _lib.status_of("mxsg_quantize_act_gather", *args.values(), None, None)


def test_quantize_act_gather_validation():
    assert _qag(idx=None) == _lib.INVALID_ARGUMENT          # routed rows need an index
    assert _qag(T=0) == _lib.BAD_SHAPE                      # nothing to gather from
    assert _qag(T=-3) == _lib.BAD_SHAPE
    assert _qag(C=200) == _lib.BAD_SHAPE
    assert _qag(recipe=7) == _lib.INVALID_ARGUMENT
    assert _qag(cc=FAKE, cs=FAKE, ps=FAKE, ld=100) == _lib.BAD_SHAPE
    assert b"quantize_act_gather" in _lib.load().mxsg_last_error()


def _qw(**kw):
    args = dict(w=FAKE, E=2, K=256, N=256, recipe=0, fmt=0, kc=FAKE, ks=FAKE, nc=FAKE, ns=FAKE,
                amax=FAKE, dls=None, dli=None)
    args.update(kw)
    return _lib.status_of("mxsg_quantize_weight", *args.values(), None, None)


def test_quantize_weight_validation():
    assert _qw(K=130) == _lib.BAD_SHAPE
    assert _qw(N=64) == _lib.BAD_SHAPE
    assert _qw(E=0) == _lib.INVALID_ARGUMENT
    assert _qw(kc=None, nc=None) == _lib.INVALID_ARGUMENT
    assert _qw(ks=None) == _lib.INVALID_ARGUMENT
    assert _qw(recipe=3, amax=None, ns=None) == _lib.INVALID_ARGUMENT
    assert _qw(recipe=9) == _lib.INVALID_ARGUMENT


def _mm(**kw):
    args = dict(mode=0, recipe=0, fa=0, fb=0, E=4, M=64, K=256, N=256, ends=FAKE, ps=None,
                a=FAKE, sa=FAKE, lda=256, b=FAKE, sb=FAKE, ldb=256, out=FAKE, acc=0)
    args.update(kw)
    return _lib.status_of("mxsg_grouped_mm", *args.values(), None, None)


def test_grouped_mm_validation():
    assert _mm(mode=3) == _lib.INVALID_ARGUMENT
    assert _mm(fa=1, fb=1) == _lib.UNSUPPORTED             # e5m2 x e5m2 not built
    assert _mm(K=200) == _lib.BAD_SHAPE
    assert _mm(lda=128) == _lib.BAD_SHAPE                  # lda < K
    assert _mm(ldb=512) == _lib.BAD_SHAPE                  # ldb must equal K
    assert _mm(out=None) == _lib.INVALID_ARGUMENT
    assert _mm(acc=1) == _lib.INVALID_ARGUMENT             # accumulate is wgrad-only
    assert _mm(mode=2, ps=None, lda=640, ldb=640) == _lib.INVALID_ARGUMENT  # needs padded starts
    assert _mm(mode=2, ps=FAKE, lda=128, ldb=128) == _lib.BAD_SHAPE  # ld below capacity


def _act_sizes(M, C, recipe, E, fmt=0):
    out = (ctypes.c_int64 * 5)()
    st = _lib.status_of("mxsg_quantize_act_sizes", M, C, recipe, fmt, E, ctypes.addressof(out))
    return st, list(out)


def _w_sizes(E, K, N, recipe, fmt=0):
    out = (ctypes.c_int64 * 4)()
    st = _lib.status_of("mxsg_quantize_weight_sizes", E, K, N, recipe, fmt, ctypes.addressof(out))
    return st, list(out)


@pytest.mark.parametrize("M,C,E", [(0, 128, 1), (1, 128, 1), (7, 256, 3), (1000, 384, 8),
                                   (65536, 4096, 64), (5, 128, 0)])
def test_quantize_act_sizes(M, C, E):
    lib = _lib.load()
    ld = lib.mxsg_padded_capacity(M, E) if E else 0
    rows = M + (M % 2)                                  # rows are stored in pairs
    for recipe, row_s, col_s in [(0, 4, 4), (1, 4, 4),
                                 (2, 4 * M * (C // 128), 4 * C * (ld // 128)),
                                 (3, M * (C // 32), C * (ld // 32))]:
        st, b = _act_sizes(M, C, recipe, E)
        assert st == _lib.OK
        assert b[0] == rows * C and b[1] == row_s
        if E:
            assert b[2:] == [C * ld, col_s, 4 * (E + 1)]
        else:
            assert b[2:] == [0, 0, 0]


def test_quantize_act_sizes_validation():
    assert _act_sizes(16, 200, 0, 1)[0] == _lib.BAD_SHAPE
    assert _act_sizes(-1, 128, 0, 1)[0] == _lib.INVALID_ARGUMENT
    assert _act_sizes(16, 128, 5, 1)[0] == _lib.INVALID_ARGUMENT      # no recipe 5
    assert _act_sizes(16, 128, 4, 1)[0] == _lib.UNSUPPORTED           # NVFP4 takes e2m1 elements only
    assert _act_sizes(16, 128, 0, -1)[0] == _lib.INVALID_ARGUMENT
    assert _act_sizes(1 << 31, 128, 0, 1)[0] == _lib.BAD_SHAPE
    assert _lib.status_of("mxsg_quantize_act_sizes", 16, 128, 0, 0, 1, None) == _lib.INVALID_ARGUMENT
    # 4-bit codes: MX only, half the code bytes, same scales
    assert _act_sizes(16, 128, 0, 1, fmt=2)[0] == _lib.UNSUPPORTED
    assert _act_sizes(16, 128, 3, 1, fmt=5)[0] == _lib.INVALID_ARGUMENT
    st, b4 = _act_sizes(7, 256, 3, 3, fmt=2)
    st8, b8 = _act_sizes(7, 256, 3, 3, fmt=0)
    assert st == st8 == _lib.OK
    assert [b4[0], b4[2]] == [b8[0] // 2, b8[2] // 2] and [b4[1], b4[3], b4[4]] == [b8[1], b8[3], b8[4]]
    # the same shape rule answers the launching call the same way
    assert _qact(C=200) == _act_sizes(16, 200, 0, 1)[0]


@pytest.mark.parametrize("E,K,N", [(1, 128, 128), (8, 4096, 14336), (3, 256, 640)])
def test_quantize_weight_sizes(E, K, N):
    for recipe, sc in [(0, 4 * E), (1, 4 * E), (2, 4 * E * (K // 128) * (N // 128)),
                       (3, E * K * N // 32)]:
        st, b = _w_sizes(E, K, N, recipe)
        assert st == _lib.OK
        assert b == [E * K * N, sc, E * K * N, sc]


def test_quantize_weight_sizes_validation():
    assert _w_sizes(2, 130, 256, 0)[0] == _lib.BAD_SHAPE
    assert _w_sizes(0, 128, 128, 0)[0] == _lib.INVALID_ARGUMENT
    assert _w_sizes(1 << 16, 128, 128, 0)[0] == _lib.BAD_SHAPE
    assert _w_sizes(2, 128, 128, 5)[0] == _lib.INVALID_ARGUMENT
    assert _qw(K=130) == _w_sizes(2, 130, 256, 0)[0]
    assert _w_sizes(2, 256, 256, 2, fmt=2)[0] == _lib.UNSUPPORTED
    assert _w_sizes(2, 256, 384, 3, fmt=2)[1] == [2 * 256 * 384 // 2, 2 * 256 * 384 // 32] * 2
    # NVFP4: half-byte codes; e4m3 block codes per 16 elements, then one fp32 tensor scale per expert
    assert _w_sizes(2, 256, 384, 4, fmt=2)[1] == [2 * 256 * 384 // 2, 2 * 256 * 384 // 16 + 8] * 2
    assert _w_sizes(2, 256, 384, 4, fmt=0)[0] == _lib.UNSUPPORTED


def test_nvfp4_act_sizes():
    M, C, E = 7, 256, 3
    ld = _lib.load().mxsg_padded_capacity(M, E)
    st, b = _act_sizes(M, C, 4, E, fmt=2)
    assert st == _lib.OK
    assert b == [(M + 1) * C // 2, M * C // 16 + 4, C * ld // 2, C * ld // 16 + 4, 4 * (E + 1)]
    # grouped GEMM: NVFP4 needs e2m1 on both sides, and e2m1 no other recipe than MX / NVFP4
    assert _mm_check(recipe=4, fa=2, fb=2, lda=128, ldb=128) == _lib.OK
    assert _mm_check(recipe=4, fa=0, fb=0) == _lib.UNSUPPORTED
    assert _mm_check(recipe=2, fa=2, fb=2, lda=128, ldb=128) == _lib.UNSUPPORTED


def _mm_check(**kw):
    args = dict(mode=0, recipe=0, fa=0, fb=0, E=4, M=64, K=256, N=256, lda=256, ldb=256, acc=0)
    args.update(kw)
    return _lib.status_of("mxsg_grouped_mm_check", *args.values())


def test_grouped_mm_check_agrees_with_launcher():
    """Over a grid of shape arguments (pointers all valid), the host-only
    check and the launching call return the same status; every case here
    fails validation or would launch, so only failing ones go to the
    launcher."""
    lib = _lib.load()
    seen = set()
    for mode in (0, 1, 2, 3):
        for recipe in (0, 2, 3, 5):
            for fa, fb in ((0, 0), (1, 0), (1, 1)):
                for K, N in ((256, 256), (200, 256), (256, 384)):
                    for lda, ldb in ((256, 256), (128, 256), (384, 384), (1024, 1024)):
                        for acc in (0, 1):
                            kw = dict(mode=mode, recipe=recipe, fa=fa, fb=fb, K=K, N=N, lda=lda,
                                      ldb=ldb, acc=acc)
                            st = _mm_check(**kw)
                            seen.add(st)
                            if st != _lib.OK:
                                msg = lib.mxsg_last_error()
                                assert _mm(ps=FAKE, **kw) == st, kw
                                assert lib.mxsg_last_error() == msg
    assert seen == {_lib.OK, _lib.INVALID_ARGUMENT, _lib.BAD_SHAPE, _lib.UNSUPPORTED}
    assert _mm_check(mode=2, lda=128, ldb=128) == _lib.BAD_SHAPE
    assert _mm_check(mode=2, lda=1024, ldb=1024) == _lib.OK
    assert _mm_check(mode=1, recipe=2, N=65536 + 128, lda=65536 + 128, ldb=65536 + 128) == _lib.UNSUPPORTED
    # 4-bit operands: MX, both sides, row lengths in code bytes
    assert _mm_check(recipe=3, fa=2, fb=2, lda=128, ldb=128) == _lib.OK
    assert _mm_check(recipe=3, fa=2, fb=2, lda=256, ldb=256) == _lib.BAD_SHAPE   # ldb must be K/2
    assert _mm_check(recipe=3, fa=2, fb=0, lda=128, ldb=128) == _lib.UNSUPPORTED
    assert _mm_check(recipe=0, fa=2, fb=2, lda=128, ldb=128) == _lib.UNSUPPORTED
    assert _mm_check(mode=2, recipe=3, fa=2, fb=2, lda=320, ldb=320) == _lib.OK   # capacity 640 / 2
    assert _mm_check(mode=2, recipe=3, fa=2, fb=2, lda=288, ldb=320) == _lib.BAD_SHAPE


def test_delayed_and_sweep_validation():
    assert _lib.status_of("mxsg_delayed_update", FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0, 0, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_delayed_update", None, FAKE, FAKE, FAKE, FAKE, 2, 16, 0, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_delayed_update", FAKE, FAKE, FAKE, FAKE, FAKE, 2, 16, 2, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_cast_sweep", 0, 16, 5, FAKE, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_cast_sweep", 0, 16, 0, None, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_stream_copy", FAKE, FAKE, 24, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_stream_copy", None, FAKE, 32, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_stream_copy", FAKE + 8, FAKE, 32, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_clock_probe", -1, 10, FAKE, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_clock_probe", 4, -1, FAKE, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_clock_probe", 4, 10, None, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_clock_probe", (1 << 20) + 1, 10, FAKE, None) == _lib.INVALID_ARGUMENT
    assert _lib.status_of("mxsg_wall_clock_rate_khz", None) == _lib.INVALID_ARGUMENT


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_blockwise_contraction_limit():
    """Blockwise forward / dgrad accept a contraction of up to 65536 (the
    per-tile weight-scale table) and report UNSUPPORTED beyond it; wgrad's
    contraction (the tokens of a group) has no such limit."""
    assert _mm_check(recipe=2, K=65536, lda=65536, ldb=65536) == _lib.OK
    assert _mm_check(recipe=2, K=65536 + 128, lda=65536 + 128, ldb=65536 + 128) == _lib.UNSUPPORTED
    assert _mm_check(mode=1, recipe=2, N=65536, lda=65536, ldb=65536) == _lib.OK
    assert _mm_check(mode=1, recipe=2, N=65536 + 128, lda=65536 + 128, ldb=65536 + 128) == _lib.UNSUPPORTED


def test_route_validation():
    """mxsg_route rejects bad sizes and missing outputs before any launch."""
    st = _lib.status_of
    p = ctypes.c_void_p(16)
    assert st("mxsg_route", p, 10, 0, 4, p, p, None, None, None) == _lib.INVALID_ARGUMENT      # k = 0
    assert st("mxsg_route", p, 10, 2, 0, p, p, None, None, None) == _lib.INVALID_ARGUMENT      # E = 0
    assert st("mxsg_route", p, -1, 2, 4, p, p, None, None, None) == _lib.INVALID_ARGUMENT      # T < 0
    assert st("mxsg_route", p, 1 << 30, 2, 4, p, p, None, None, None) == _lib.BAD_SHAPE        # T k >= 2^31
    assert st("mxsg_route", p, 10, 2, 4, None, p, None, None, None) == _lib.INVALID_ARGUMENT   # no group_ends
    assert st("mxsg_route", None, 10, 2, 4, p, p, None, None, None) == _lib.INVALID_ARGUMENT   # no ids
    assert st("mxsg_route", p, 10, 2, 4, p, None, None, None, None) == _lib.INVALID_ARGUMENT   # no row_index


def test_swiglu_and_sweep_validation():
    st = _lib.status_of
    p = ctypes.c_void_p(16)
    assert st("mxsg_swiglu", p, 4, 12, p, None) == _lib.BAD_SHAPE             # C not a multiple of 8
    assert st("mxsg_swiglu", p, -1, 8, p, None) == _lib.BAD_SHAPE
    assert st("mxsg_swiglu", None, 4, 8, p, None) == _lib.INVALID_ARGUMENT
    assert st("mxsg_swiglu", ctypes.c_void_p(8), 4, 8, p, None) == _lib.INVALID_ARGUMENT   # misaligned
    assert st("mxsg_sigmoid_sweep", None, None) == _lib.INVALID_ARGUMENT
