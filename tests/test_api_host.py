"""The C-ABI library on the host: it loads, exports every declared entry point, and rejects bad
arguments before touching the GPU (so these run without one). Fake device addresses are never
dereferenced: every call here fails its host-side checks, or has M = 0 and enqueues nothing.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dq.h")
LIB = os.path.join(ROOT, "fp8_dynamic_quant_amd", "libdq.so")

OK, NULL, SHAPE, ALIGN, ALIAS, EPI, HIP, WORKSPACE, VALUE = range(9)
BIAS, GELU, GATED = 0, 1, 2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libdq.so is not built (python fp8_dynamic_quant_amd/build.py)")
    L = ctypes.CDLL(LIB)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.dq_quantize_fp8.argtypes = [vp, i64, i64, vp, vp, vp]
    L.dq_quantize_weight_fp8.argtypes = [vp, i64, i64, vp, vp, vp]
    L.dq_linear_fp8.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, i32, vp, vp, vp, vp,
                                ctypes.c_uint64, vp]
    L.dq_linear_fp8_noalloc.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, i32, vp, vp, vp, vp]
    L.dq_linear_fp8_segmented.argtypes = [vp, vp, i64, i64, vp, vp, vp, i64, vp, i32, vp, vp, vp,
                                          vp, ctypes.c_uint64, vp]
    L.dq_linear_fp8_segmented_workspace_size.argtypes = [i64, vp, i64, i64]
    L.dq_linear_fp8_segmented_workspace_size.restype = ctypes.c_uint64
    L.dq_layernorm_modulate_quantize_fp8.argtypes = [vp, i64, i64, vp, vp, ctypes.c_float, vp,
                                                     vp, vp, vp]
    L.dq_linear_qkv_fp8.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, vp, vp, ctypes.c_float,
                                    vp, vp, vp, vp, ctypes.c_uint64, vp]
    L.dq_linear_qkv_fp8_attn.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, vp, vp,
                                         ctypes.c_float, vp, vp, vp, vp, vp, vp, vp,
                                         ctypes.c_uint64, vp]
    L.dq_quantize_v_fp8.argtypes = [vp, i64, i64, vp, vp, vp]
    L.dq_attention_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, ctypes.c_uint64,
                                   i64, vp]
    L.dq_attention_fp8_workspace_size.argtypes = [i64, i64]
    L.dq_attention_fp8_workspace_size.restype = ctypes.c_uint64
    L.dq_quantize_mx_fp8.argtypes = [vp, i64, i64, vp, vp, vp]
    L.dq_linear_mx_fp8.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, i32, vp, vp]
    L.dq_quantize_mxfp4.argtypes = [vp, i64, i64, vp, vp, vp]
    L.dq_linear_mxfp4.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, i32, vp, vp, vp, vp]
    L.dq_linear_mxfp4_segmented.argtypes = [vp, vp, i64, i64, vp, vp, vp, i64, vp, i32, vp, vp,
                                            vp, vp]
    L.dq_linear_fp8_workspace_size.argtypes = [i64, i64, i64]
    L.dq_linear_fp8_workspace_size.restype = ctypes.c_uint64
    L.dq_status_string.restype = ctypes.c_char_p
    L.dq_status_string.argtypes = [i32]
    return L


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(dq_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("dq_quantize_fp8", "dq_quantize_weight_fp8", "dq_linear_fp8",
              "dq_layernorm_modulate_quantize_fp8", "dq_linear_qkv_fp8", "dq_linear_qkv_fp8_attn",
              "dq_quantize_v_fp8", "dq_attention_fp8", "dq_attention_fp8_workspace_size",
              "dq_quantize_mx_fp8", "dq_linear_mx_fp8", "dq_quantize_mxfp4", "dq_linear_mxfp4",
              "dq_linear_mxfp4_segmented",
              "dq_linear_fp8_workspace_size", "dq_status_string", "dq_last_hip_error",
              "dq_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.dq_abi_version() == 11
    for st in range(9):
        s = lib.dq_status_string(st)
        assert s and len(s) > 1
    assert lib.dq_status_string(12345) == b"unknown status"
    assert lib.dq_last_hip_error() == 0


X, Q, S = 0x10000000, 0x20000000, 0x30000000          # fake, 16-byte aligned, far apart


@pytest.mark.parametrize("fn", ["dq_quantize_fp8", "dq_quantize_weight_fp8"])
def test_quantize_argument_checks(lib, fn):
    f = getattr(lib, fn)
    assert f(X, 0, 64, Q, S, None) == OK                    # empty: nothing to do
    assert f(None, 4, 64, Q, S, None) == NULL
    assert f(X, 4, 64, None, S, None) == NULL
    assert f(X, 4, 64, Q, None, None) == NULL
    assert f(X, -1, 64, Q, S, None) == SHAPE
    assert f(X, 4, 0, Q, S, None) == SHAPE
    assert f(X, 4, 12, Q, S, None) == SHAPE                 # K % 8
    assert f(X, 4, 4, Q, S, None) == SHAPE                  # K < 8
    assert f(X, 1 << 31, 64, Q, S, None) == SHAPE           # M too large
    assert f(X + 2, 4, 64, Q, S, None) == ALIGN
    assert f(X, 4, 64, Q + 8, S, None) == ALIGN
    assert f(X, 4, 64, Q, S + 4, None) == ALIGN
    assert f(X, 4, 64, X + 64, S, None) == ALIAS            # codes inside x
    assert f(X, 4, 64, Q, X, None) == ALIAS                 # scales inside x
    assert f(X, 4, 64, Q, Q + 128, None) == ALIAS           # scales inside codes


def test_quantize_adjacent_buffers_are_not_aliases(lib):
    # x occupies [X, X + 2*4*64); codes right after it do not overlap
    # (the call is rejected for another reason so that nothing is launched)
    assert lib.dq_quantize_fp8(X, 4, 64, X + 2 * 4 * 64, None, None) == NULL


MS, MT, Y = 0x40000000, 0x50000000, 0x60000000          # fake modulation vectors and y


def lnmq(lib, M=4, K=64, x=X, ms=MS, mt=MT, eps=1e-6, y=Y, q=Q, s=S):
    return lib.dq_layernorm_modulate_quantize_fp8(x, M, K, ms, mt, eps, y, q, s, None)


def test_layernorm_modulate_argument_checks(lib):
    assert lnmq(lib, M=0) == OK                             # empty: nothing to do
    assert lnmq(lib, M=0, x=None, q=None) == OK
    assert lnmq(lib, M=-1) == SHAPE
    assert lnmq(lib, M=1 << 31) == SHAPE
    assert lnmq(lib, K=0) == SHAPE
    assert lnmq(lib, K=4) == SHAPE                          # K < 8
    assert lnmq(lib, K=12) == SHAPE                         # K % 8
    assert lnmq(lib, K=8192 + 8) == SHAPE                   # one row must fit the registers
    assert lnmq(lib, M=0, K=12) == SHAPE                    # shapes are checked even when empty
    assert lnmq(lib, eps=-1e-6) == VALUE
    assert lnmq(lib, eps=0.0) == VALUE                      # 0/0 on a row of equal values
    assert lnmq(lib, eps=float("nan")) == VALUE
    assert lnmq(lib, eps=float("inf")) == VALUE
    assert lnmq(lib, M=0, eps=-1.0) == VALUE
    for name in ("x", "ms", "mt", "q", "s"):
        assert lnmq(lib, **{name: None}) == NULL, name
    for name in ("x", "ms", "mt", "y", "q"):
        assert lnmq(lib, **{name: {"x": X, "ms": MS, "mt": MT, "y": Y, "q": Q}[name] + 8}) \
            == ALIGN, name
    assert lnmq(lib, s=S + 4) == ALIGN
    assert lnmq(lib, q=X + 64) == ALIAS                     # codes inside x
    assert lnmq(lib, y=X) == ALIAS                          # y over x (no in-place form)
    assert lnmq(lib, s=MS) == ALIAS                         # scales over mod_scale
    assert lnmq(lib, q=MT - 16) == ALIAS                    # codes run into mod_shift
    assert lnmq(lib, s=Q + 64) == ALIAS                     # scales inside codes
    assert lnmq(lib, q=Y + 2 * 4 * 64 - 16) == ALIAS        # codes inside y
    # adjacent, non-overlapping buffers are fine; y = NULL is allowed (the call then fails on
    # a NULL scale so that nothing is launched)
    assert lnmq(lib, y=None, q=X + 2 * 4 * 64, s=None) == NULL
    assert lnmq(lib, y=Y, q=Y + 2 * 4 * 64, s=None) == NULL
    assert lib.dq_last_hip_error() == 0


Aq, As, Wq, Ws, Bi, Ga, Re, Ou = (0x1000000 * i for i in range(1, 9))


Wk = 0x9000000                                             # fake workspace, 256-byte aligned


def lin(lib, M=64, K=256, N=128, q=Aq, sa=As, qw=Wq, sw=Ws, bias=Bi, epi=BIAS, gate=Ga,
        res=Re, out=Ou, ws=None, ws_bytes=0):
    return lib.dq_linear_fp8(q, sa, M, K, qw, sw, N, bias, epi, gate, res, out, ws, ws_bytes,
                             None)


def test_linear_argument_checks(lib):
    assert lin(lib, M=0) == OK
    assert lin(lib, M=0, epi=7) == EPI                       # epilogue is checked even when empty
    assert lin(lib, K=192) == SHAPE                          # K % 128
    assert lin(lib, K=0) == SHAPE
    assert lin(lib, K=1 << 24) == SHAPE                      # one tile must fit a 32-bit range
    assert lin(lib, N=96) == SHAPE                           # N % 64
    assert lin(lib, N=0) == SHAPE
    assert lin(lib, M=-3) == SHAPE
    assert lin(lib, epi=3) == EPI
    assert lin(lib, epi=-1) == EPI
    assert lin(lib, epi=GATED, gate=None) == EPI
    assert lin(lib, epi=GATED, res=None) == EPI
    assert lin(lib, q=None) == NULL
    assert lin(lib, sa=None) == NULL
    assert lin(lib, qw=None) == NULL
    assert lin(lib, sw=None) == NULL
    assert lin(lib, out=None) == NULL
    assert lin(lib, q=Aq + 1) == ALIGN
    assert lin(lib, bias=Bi + 2) == ALIGN
    assert lin(lib, epi=GATED, gate=Ga + 2) == ALIGN
    assert lin(lib, epi=GATED, res=Re + 2) == ALIGN
    assert lin(lib, out=Ou + 8) == ALIGN
    assert lin(lib, out=Aq) == ALIAS                         # out over the codes
    assert lin(lib, out=Ws) == ALIAS
    assert lin(lib, out=Bi) == ALIAS
    assert lin(lib, epi=GATED, out=Ga) == ALIAS
    assert lin(lib, epi=GATED, out=Re + 64) == ALIAS         # partial overlap with residual


NQ, CS, SN, OQ, OK_, OV = (0x10000000 * i for i in range(10, 16))   # fake, far from the others


def qkv(lib, M=64, K=256, heads=1, q=Aq, sa=As, qw=Wq, sw=Ws, bias=Bi, nqk=NQ, cos=CS, sin=SN,
        eps=1e-6, oq=OQ, ok=OK_, ov=OV, ws=None, ws_bytes=0):
    return lib.dq_linear_qkv_fp8(q, sa, M, K, qw, sw, heads, bias, nqk, cos, sin, eps, oq, ok, ov,
                                 ws, ws_bytes, None)


def test_linear_qkv_argument_checks(lib):
    assert qkv(lib, M=0) == OK
    assert qkv(lib, M=0, q=None, oq=None) == OK               # empty: pointers are not checked
    assert qkv(lib, heads=0) == SHAPE
    assert qkv(lib, heads=-2) == SHAPE
    assert qkv(lib, heads=1 << 30) == SHAPE
    assert qkv(lib, K=192) == SHAPE                          # K % 128
    assert qkv(lib, M=-1) == SHAPE
    assert qkv(lib, M=0, K=100) == SHAPE
    assert qkv(lib, eps=0.0) == VALUE
    assert qkv(lib, eps=-1.0) == VALUE
    assert qkv(lib, eps=float("nan")) == VALUE
    assert qkv(lib, M=0, eps=float("inf")) == VALUE
    for name in ("q", "sa", "qw", "sw", "nqk", "cos", "sin", "oq", "ok", "ov"):
        assert qkv(lib, **{name: None}) == NULL, name
    base = dict(q=Aq, sa=As, qw=Wq, sw=Ws, bias=Bi, nqk=NQ, cos=CS, sin=SN, oq=OQ, ok=OK_, ov=OV)
    for name, val in base.items():
        assert qkv(lib, **{name: val + 8}) == ALIGN, name
    # outputs are [heads, M, 128] bf16 = 16 KiB here; the fake inputs are far apart
    assert qkv(lib, oq=Aq) == ALIAS                           # query output over the codes
    assert qkv(lib, ok=CS + 64) == ALIAS                      # key output over the cosines
    assert qkv(lib, ov=NQ - 1024) == ALIAS                    # value output runs into the weights
    assert qkv(lib, ok=OQ + 16384 - 16) == ALIAS              # two outputs overlap
    assert qkv(lib, ov=Bi) == ALIAS
    # adjacent outputs are fine (the call then fails on the NULL codes, launching nothing)
    assert qkv(lib, ok=OQ + 16384, ov=OQ + 32768, q=None) == NULL


def test_linear_qkv_workspace_checks(lib):
    need = 4096 + 4 * 256 * 256 * 4                           # a budget of four partial tiles
    assert qkv(lib, ws=Wk + 16, ws_bytes=need) == WORKSPACE
    assert qkv(lib, ws=Wk, ws_bytes=need, oq=Wk + 4096) == ALIAS
    assert qkv(lib, ws=Wk, ws_bytes=need, cos=Wk + (1 << 20)) == ALIAS
    assert qkv(lib, ws=Wk, ws_bytes=need, q=None) == NULL
    assert lib.dq_last_hip_error() == 0


Q8, SQ8, K8, SK8, SV8 = (0x10000000 * i for i in range(16, 21))   # fake, far from the others


def qkv8(lib, M=64, K=256, heads=1, q=Aq, sa=As, qw=Wq, sw=Ws, bias=Bi, nqk=NQ, cos=CS, sin=SN,
         eps=1e-6, q8=Q8, sq=SQ8, k8=K8, sk=SK8, ov=OV, sv=SV8, ws=None, ws_bytes=0):
    return lib.dq_linear_qkv_fp8_attn(q, sa, M, K, qw, sw, heads, bias, nqk, cos, sin, eps, q8, sq,
                                      k8, sk, ov, sv, ws, ws_bytes, None)


def test_linear_qkv_attn_argument_checks(lib):
    assert qkv8(lib, M=0) == OK
    assert qkv8(lib, M=0, q=None, q8=None) == OK              # empty: pointers are not checked
    assert qkv8(lib, heads=0) == SHAPE
    assert qkv8(lib, heads=1 << 30) == SHAPE
    assert qkv8(lib, K=192) == SHAPE
    assert qkv8(lib, M=-1) == SHAPE
    assert qkv8(lib, M=72) == SHAPE                           # M % 16 (the transposed values)
    assert qkv8(lib, eps=0.0) == VALUE
    assert qkv8(lib, eps=float("nan")) == VALUE
    for name in ("q", "sa", "qw", "sw", "nqk", "cos", "sin", "q8", "sq", "k8", "sk", "ov", "sv"):
        assert qkv8(lib, **{name: None}) == NULL, name
    base = dict(q=Aq, sa=As, qw=Wq, sw=Ws, bias=Bi, nqk=NQ, cos=CS, sin=SN, q8=Q8, sq=SQ8, k8=K8,
                sk=SK8, ov=OV, sv=SV8)
    for name, val in base.items():
        assert qkv8(lib, **{name: val + 8}) == ALIGN, name
    # codes [heads, M, 128] = 8 KiB here (the values' too), scales [heads, M] = 256 bytes
    assert qkv8(lib, q8=Aq) == ALIAS                          # query codes over the input codes
    assert qkv8(lib, sk=CS + 64) == ALIAS                     # key scales over the cosines
    assert qkv8(lib, k8=Q8 + 8192 - 16) == ALIAS              # two code outputs overlap
    assert qkv8(lib, sq=Q8 + 4096) == ALIAS                   # scales inside the query codes
    assert qkv8(lib, ov=K8 - 8192 + 16) == ALIAS              # value codes run into the key codes
    assert qkv8(lib, sv=SK8 + 128) == ALIAS                   # two scale outputs overlap
    assert qkv8(lib, k8=Q8 + 8192, sq=Q8 + 16384, sk=Q8 + 16640, ov=Q8 + 16896,
                sv=Q8 + 25088, q=None) == NULL                # adjacent outputs are fine


def test_linear_qkv_attn_workspace_checks(lib):
    need = 4096 + 4 * 256 * 256 * 4
    assert qkv8(lib, ws=Wk + 16, ws_bytes=need) == WORKSPACE
    assert qkv8(lib, ws=Wk, ws_bytes=need, sq=Wk + 4096) == ALIAS
    assert qkv8(lib, ws=Wk, ws_bytes=need, q=None) == NULL
    assert lib.dq_last_hip_error() == 0


AQ, ASQ, AK, ASK, AV, ASV, AO = (0x20000000 * i for i in range(20, 27))   # fake, far apart


def attn(lib, H=2, S=64, q=AQ, sq=ASQ, k=AK, sk=ASK, vt=AV, sv=ASV, out=AO, ws=None, ws_bytes=0,
         max_wg=0):
    return lib.dq_attention_fp8(q, sq, k, sk, vt, sv, H, S, out, ws, ws_bytes, max_wg, None)


def test_attention_argument_checks(lib):
    assert attn(lib, S=0) == OK
    assert attn(lib, H=0, q=None) == OK                      # empty: pointers are not checked
    assert attn(lib, S=24) == SHAPE                          # S % 16
    assert attn(lib, S=-16) == SHAPE
    assert attn(lib, H=-1) == SHAPE
    assert attn(lib, H=65536) == SHAPE
    assert attn(lib, S=1 << 24) == SHAPE
    assert attn(lib, S=0, H=3) == OK
    for name in ("q", "sq", "k", "sk", "vt", "sv", "out"):
        assert attn(lib, **{name: None}) == NULL, name
    base = dict(q=AQ, sq=ASQ, k=AK, sk=ASK, vt=AV, sv=ASV, out=AO)
    for name, val in base.items():
        assert attn(lib, **{name: val + 4}) == ALIGN, name
    # out is S H 128 bf16 = 32 KiB here
    assert attn(lib, out=AQ) == ALIAS
    assert attn(lib, out=ASV - 1024) == ALIAS
    assert attn(lib, out=AV + 16) == ALIAS
    assert attn(lib, out=AQ + 2 * 64 * 128, sq=None) == NULL        # right after q: no alias
    assert attn(lib, max_wg=-1) == VALUE
    assert attn(lib, max_wg=-1, S=0) == VALUE                       # checked before the size


AW = 0x20000000 * 30


def test_attention_workspace(lib):
    size = lib.dq_attention_fp8_workspace_size
    part = 12 * 64 * 66 * 4                             # one workgroup's partial result
    assert part == 202752
    assert size(4, 4608) == 4096 + 2 * 48 * part        # 4 heads x 12 query tiles of 384
    assert size(24, 4608) == 4096 + 2 * 256 * part      # at most 256 workgroups
    assert size(2, 64) == 4096 + 2 * 2 * part
    assert size(64, 1 << 16) == 4096 + 2 * 256 * part
    assert size(0, 64) == 4096 and size(3, 0) == 4096
    assert size(2, 24) == 0 and size(-1, 64) == 0
    need = size(2, 64)
    assert attn(lib, ws=AW, ws_bytes=need - 1) == WORKSPACE
    assert attn(lib, ws=AW + 16, ws_bytes=need) == WORKSPACE     # not 256-byte aligned
    assert attn(lib, ws=AQ, ws_bytes=need) == ALIAS              # over the query codes
    assert attn(lib, ws=AO - 256, ws_bytes=need) == ALIAS        # into the output
    assert attn(lib, ws=AW, ws_bytes=need, q=None) == NULL
    assert attn(lib, S=0, ws=AW + 16, ws_bytes=0) == OK          # empty: nothing is checked
    assert lib.dq_last_hip_error() == 0


MX_X, MX_Q, MX_S, MX_W, MX_SW, MX_O, MX_G, MX_R = (0x20000000 * i for i in range(40, 48))  # fake


def test_quantize_mx_argument_checks(lib):
    f = lib.dq_quantize_mx_fp8
    assert f(MX_X, 0, 64, MX_Q, MX_S, None) == OK                # empty
    assert f(MX_X, 4, 48, MX_Q, MX_S, None) == SHAPE             # K % 32
    assert f(MX_X, 4, 16, MX_Q, MX_S, None) == SHAPE             # K < 32
    assert f(MX_X, -1, 64, MX_Q, MX_S, None) == SHAPE
    assert f(None, 4, 64, MX_Q, MX_S, None) == NULL
    assert f(MX_X, 4, 64, None, MX_S, None) == NULL
    assert f(MX_X, 4, 64, MX_Q, None, None) == NULL
    assert f(MX_X + 8, 4, 64, MX_Q, MX_S, None) == ALIGN
    assert f(MX_X, 4, 64, MX_Q + 8, MX_S, None) == ALIGN
    assert f(MX_X, 4, 64, MX_X + 256, MX_S, None) == ALIAS       # codes inside x
    assert f(MX_X, 4, 64, MX_Q, MX_Q + 16, None) == ALIAS        # scales inside the codes
    assert lib.dq_last_hip_error() == 0


def mxlin(lib, M=64, K=256, N=128, qa=MX_Q, sa=MX_S, qw=MX_W, sw=MX_SW, bias=None, epi=0, out=MX_O):
    return lib.dq_linear_mx_fp8(qa, sa, M, K, qw, sw, N, bias, epi, out, None)


def test_linear_mx_argument_checks(lib):
    assert mxlin(lib, M=0) == OK
    assert mxlin(lib, K=96) == SHAPE                             # K % 128
    assert mxlin(lib, K=1 << 24) == SHAPE
    assert mxlin(lib, N=96) == SHAPE                             # N % 64
    assert mxlin(lib, M=-1) == SHAPE
    # one 512-thread workgroup per 256 x 256 tile: fewer than 2^23 tiles
    assert mxlin(lib, M=1 << 20, K=128, N=1 << 19) == SHAPE        # 4096 x 2048 tiles
    assert mxlin(lib, M=1 << 20, K=128, N=(1 << 19) - 256, qa=None) == NULL  # one tile column less
    assert mxlin(lib, epi=2) == EPI                              # gated residual: not offered
    assert mxlin(lib, epi=7) == EPI
    for name in ("qa", "sa", "qw", "sw", "out"):
        assert mxlin(lib, **{name: None}) == NULL, name
    assert mxlin(lib, qa=MX_Q + 8) == ALIGN
    assert mxlin(lib, sa=MX_S + 2) == ALIGN                      # scale dwords: 4-byte aligned
    assert mxlin(lib, out=MX_O + 8) == ALIGN
    assert mxlin(lib, bias=MX_O + 0x100000 + 8) == ALIGN
    assert mxlin(lib, out=MX_Q) == ALIAS                         # output over the codes
    assert mxlin(lib, out=MX_SW - 64) == ALIAS                   # output into the weight scales
    assert lib.dq_last_hip_error() == 0


def test_quantize_mxfp4_argument_checks(lib):
    f = lib.dq_quantize_mxfp4
    assert f(MX_X, 0, 64, MX_Q, MX_S, None) == OK                # empty
    assert f(MX_X, 4, 48, MX_Q, MX_S, None) == SHAPE             # K % 32
    assert f(MX_X, 4, 16, MX_Q, MX_S, None) == SHAPE             # K < 32
    assert f(MX_X, -1, 64, MX_Q, MX_S, None) == SHAPE
    assert f(None, 4, 64, MX_Q, MX_S, None) == NULL
    assert f(MX_X, 4, 64, None, MX_S, None) == NULL
    assert f(MX_X, 4, 64, MX_Q, None, None) == NULL
    assert f(MX_X + 8, 4, 64, MX_Q, MX_S, None) == ALIGN
    assert f(MX_X, 4, 64, MX_Q + 8, MX_S, None) == ALIGN
    assert f(MX_X, 4, 64, MX_X + 256, MX_S, None) == ALIAS       # codes inside x
    assert f(MX_X, 4, 64, MX_Q, MX_Q + 127, None) == ALIAS       # 4 rows x 32 code bytes


def mx4lin(lib, M=64, K=256, N=128, qa=MX_Q, sa=MX_S, qw=MX_W, sw=MX_SW, bias=None, epi=0,
           gate=None, res=None, out=MX_O):
    return lib.dq_linear_mxfp4(qa, sa, M, K, qw, sw, N, bias, epi, gate, res, out, None)


def test_linear_mxfp4_argument_checks(lib):
    assert mx4lin(lib, M=0) == OK
    assert mx4lin(lib, K=128) == SHAPE                           # K % 256
    assert mx4lin(lib, K=384) == SHAPE
    assert mx4lin(lib, K=1 << 24) == SHAPE
    assert mx4lin(lib, N=96) == SHAPE                            # N % 64
    assert mx4lin(lib, M=-1) == SHAPE
    assert mx4lin(lib, M=1 << 20, K=256, N=1 << 19) == SHAPE      # 4096 x 2048 tiles
    assert mx4lin(lib, epi=3) == EPI                             # the QKV epilogue: not offered
    assert mx4lin(lib, epi=2) == EPI                             # gated without gate/residual
    assert mx4lin(lib, epi=2, gate=MX_G) == EPI
    assert mx4lin(lib, epi=2, res=MX_R) == EPI
    assert mx4lin(lib, epi=2, gate=MX_G + 8, res=MX_R) == ALIGN
    assert mx4lin(lib, epi=2, gate=MX_G, res=MX_R + 8) == ALIGN
    assert mx4lin(lib, epi=2, gate=MX_O + 64, res=MX_R) == ALIAS  # gate inside the output
    assert mx4lin(lib, epi=2, gate=MX_G, res=MX_O + 64) == ALIAS  # residual shifted over it
    for name in ("qa", "sa", "qw", "sw", "out"):
        assert mx4lin(lib, **{name: None}) == NULL, name
    assert mx4lin(lib, qa=MX_Q + 8) == ALIGN
    assert mx4lin(lib, sa=MX_S + 4) == ALIGN                     # scale pairs: 8-byte aligned
    assert mx4lin(lib, sw=MX_SW + 4) == ALIGN
    assert mx4lin(lib, out=MX_O + 8) == ALIGN
    assert mx4lin(lib, out=MX_Q) == ALIAS                        # output over the codes
    assert mx4lin(lib, out=MX_SW - 64) == ALIAS                  # output into the weight scales
    assert lib.dq_last_hip_error() == 0


def test_linear_mxfp4_segmented_argument_checks(lib):
    """Row segments of one MXFP4 activation matrix, each with its own weights: the per-call rules
    hold for every segment, and the segment list itself is checked."""
    Arr = ctypes.c_void_p * 4
    rows = (ctypes.c_int64 * 4)(64, 0, 37, 256)
    qw = Arr(MX_W, MX_W + 0x100000, MX_W + 0x200000, MX_W + 0x300000)
    sw = Arr(MX_SW, MX_SW + 0x100000, MX_SW + 0x200000, MX_SW + 0x300000)
    nob = Arr(None, None, None, None)
    gates = Arr(MX_G, MX_G + 4096, MX_G + 8192, MX_G + 12288)
    f = lib.dq_linear_mxfp4_segmented

    def call(nseg=4, seg=rows, w=qw, s=sw, b=nob, epi=0, g=None, res=None, out=MX_O, K=256):
        return f(MX_Q, MX_S, K, nseg, seg, w, s, 128, b, epi, g, res, out, None)
    zero = (ctypes.c_int64 * 2)(0, 0)
    assert call(nseg=2, seg=zero) == OK                          # every segment empty
    assert call(nseg=0) == SHAPE
    assert call(nseg=65) == SHAPE
    assert call(nseg=2, seg=(ctypes.c_int64 * 2)(64, -1)) == SHAPE
    assert call(K=128) == SHAPE
    assert call(seg=None) == NULL
    assert call(w=None) == NULL
    assert call(s=None) == NULL
    assert call(b=None) == NULL
    assert call(w=Arr(MX_W, None, MX_W, MX_W)) == NULL           # a NULL weight in the list
    assert call(s=Arr(MX_SW, MX_SW, MX_SW + 4, MX_SW)) == ALIGN  # a misaligned scale array
    assert call(epi=2, res=MX_R) == EPI                          # gated, no gate list
    assert call(epi=2, g=Arr(MX_G, MX_G, None, MX_G), res=MX_R) == EPI
    assert call(epi=2, g=gates) == EPI                           # no residual
    assert call(epi=2, g=Arr(MX_G, MX_G, MX_G + 8, MX_G), res=MX_R) == ALIGN
    assert call(b=Arr(None, MX_O + 32, None, None)) == ALIAS     # a bias inside the output
    assert lib.dq_last_hip_error() == 0



def test_quantize_v_argument_checks(lib):
    f = lib.dq_quantize_v_fp8
    V, VT, SV = 0x30000000, 0x40000000, 0x50000000
    assert f(V, 0, 64, VT, SV, None) == OK
    assert f(V, 2, 0, VT, SV, None) == OK
    assert f(V, 2, 40, VT, SV, None) == SHAPE                # S % 16
    assert f(None, 2, 64, VT, SV, None) == NULL
    assert f(V, 2, 64, None, SV, None) == NULL
    assert f(V, 2, 64, VT, None, None) == NULL
    assert f(V + 2, 2, 64, VT, SV, None) == ALIGN
    assert f(V, 2, 64, VT + 8, SV, None) == ALIGN
    assert f(V, 2, 64, V + 1024, SV, None) == ALIAS          # codes inside v
    assert f(V, 2, 64, VT, VT + 256, None) == ALIAS          # scales inside codes
    assert lib.dq_last_hip_error() == 0


def test_workspace_size(lib):
    """The workspace of the schedule dq_linear_fp8 prefers: 0 when it cuts no tile, else 4096
    bytes of arrival counters plus one 256 x 256 fp32 partial tile (256 KiB) per part. With no
    GPU visible the query assumes 256 compute units."""
    size = lib.dq_linear_fp8_workspace_size
    part = 256 * 256 * 4
    # 24 tiles of 96 steps: each cut into 4 parts (96 partial tiles)
    assert size(512, 12288, 3072) == 4096 + 96 * part
    # 864 tiles: 96 left over after three rounds run as narrow halves, no cut
    assert size(4608, 3072, 12288) == 0
    assert size(64, 256, 512) == 0                                # 2 tiles of 2 steps
    assert size(16896, 3072, 12288) == 0                          # 3168 tiles, 96 left over
    assert size(256, 8192, 256) == 4096 + 4 * part                # one tile of 64 steps, 4 parts
    for M, K, N in [(40, 4096, 192), (600, 5120, 448), (256, 6400, 768), (2304, 3072, 2560)]:
        s = size(M, K, N)
        assert s == 0 or (s > 4096 and (s - 4096) % part == 0), (M, K, N, s)
    assert size(64, 192, 512) == 0                                # K % 128
    assert size(64, 256, 96) == 0                                 # N % 64
    assert size(-1, 256, 512) == 0
    assert size(0, 256, 512) == 0                                 # empty problems need none


def test_linear_workspace_checks(lib):
    need = lib.dq_linear_fp8_workspace_size(256, 8192, 256)
    # the size is a budget (a smaller workspace runs a schedule that fits), so only its
    # alignment and its overlap with the other arguments are errors
    assert lin(lib, ws=Wk + 16, ws_bytes=need) == WORKSPACE      # not 256-byte aligned
    assert lin(lib, ws=Aq, ws_bytes=need) == ALIAS               # workspace over the codes
    assert lin(lib, ws=Ou, ws_bytes=need) == ALIAS               # workspace over the output
    assert lin(lib, ws=Aq - 4096, ws_bytes=4097) == ALIAS        # its last byte on the codes
    assert lin(lib, ws=Wk, ws_bytes=need, q=None) == NULL
    assert lin(lib, M=0, ws=Wk, ws_bytes=0) == OK                # empty: nothing is checked


def noalloc(lib, M=64, K=256, N=128, q=Aq, sa=As, qw=Wq, sw=Ws, bias=Bi, epi=BIAS, gate=Ga,
            res=Re, out=Ou):
    return lib.dq_linear_fp8_noalloc(q, sa, M, K, qw, sw, N, bias, epi, gate, res, out, None)


def test_noalloc_argument_checks(lib):
    """The allocation-free linear refuses exactly what dq_linear_fp8 refuses, before any HIP
    call (its scratch limits the schedule, never the problem)."""
    assert noalloc(lib, M=0) == OK
    assert noalloc(lib, K=192) == SHAPE
    assert noalloc(lib, K=1 << 24) == SHAPE
    assert noalloc(lib, N=96) == SHAPE
    assert noalloc(lib, M=-1) == SHAPE
    assert noalloc(lib, epi=3) == EPI
    assert noalloc(lib, epi=GATED, gate=None) == EPI
    assert noalloc(lib, q=None) == NULL
    assert noalloc(lib, out=None) == NULL
    assert noalloc(lib, qw=Wq + 8) == ALIGN
    assert noalloc(lib, out=Aq) == ALIAS
    assert noalloc(lib, epi=GATED, res=Ou + 2) == ALIGN
    assert noalloc(lib, epi=GATED, res=Ou + 16) == ALIAS        # residual overlaps out, not equal
    assert lib.dq_last_hip_error() == 0


W2q, W2s, B2, G2 = (0x1000000 * i for i in range(10, 14))   # the second segment's tensors


def seg(lib, rows=(64, 32), K=256, N=128, q=Aq, sa=As, qw=(Wq, W2q), sw=(Ws, W2s), bias=(Bi, B2),
        epi=BIAS, gate=(Ga, G2), res=Re, out=Ou, ws=None, ws_bytes=0, arrays=True):
    n = len(rows)
    R = ctypes.c_int64 * max(n, 1)
    arr = lambda t: (ctypes.c_void_p * len(t))(*t) if (arrays and t is not None) else None
    return lib.dq_linear_fp8_segmented(q, sa, K, n, R(*rows) if arrays else None, arr(qw),
                                       arr(sw), N, arr(bias), epi, arr(gate), res, out, ws,
                                       ws_bytes, None)


def test_segmented_argument_checks(lib):
    """Every segment's tensors are checked as dq_linear_fp8 checks its weight, before any HIP
    call; rows are counted per segment."""
    assert seg(lib, rows=(0, 0)) == OK                           # empty: nothing launched
    assert seg(lib, rows=()) == SHAPE                            # no segment
    assert seg(lib, rows=(1,) * 5, qw=(Wq,) * 5, sw=(Ws,) * 5, bias=(Bi,) * 5,
               gate=(Ga,) * 5) == SHAPE                          # more than four
    assert seg(lib, rows=(64, -1)) == SHAPE
    assert seg(lib, K=192) == SHAPE
    assert seg(lib, N=96) == SHAPE
    assert seg(lib, arrays=False) == NULL                        # host arrays missing
    assert seg(lib, epi=5) == EPI
    assert seg(lib, epi=GATED, gate=(Ga, None)) == EPI           # a segment without a gate
    assert seg(lib, epi=GATED, res=None) == EPI
    assert seg(lib, qw=(Wq, None)) == NULL
    assert seg(lib, sw=(Ws + 4, W2s)) == ALIGN
    assert seg(lib, bias=(Bi, B2 + 2)) == ALIGN
    assert seg(lib, out=W2q) == ALIAS                            # out over the second weight
    assert seg(lib, ws=Wk + 64, ws_bytes=4096) == WORKSPACE
    assert seg(lib, ws=Ou - 256, ws_bytes=4096) == ALIAS
    assert lib.dq_last_hip_error() == 0


def test_segmented_workspace_size(lib):
    size = lib.dq_linear_fp8_segmented_workspace_size
    R = ctypes.c_int64 * 2
    part = 256 * 256 * 4
    # 512 text rows + 4096 image rows: 18 tile rows, as one 4608-row problem
    assert size(2, R(512, 4096), 12288, 3072) == lib.dq_linear_fp8_workspace_size(4608, 12288, 3072)
    # two segments of 256 rows and one tile each: 2 tiles of 64 steps
    assert size(2, R(256, 256), 8192, 256) == lib.dq_linear_fp8_workspace_size(512, 8192, 256)
    # segments round up to whole tile rows of their own: 257 + 1 rows are 3 tile rows, not 2
    s = size(2, R(257, 1), 8192, 256)
    assert s == lib.dq_linear_fp8_workspace_size(768, 8192, 256) and (s - 4096) % part == 0
    assert size(0, R(1, 1), 256, 128) == 0
    assert size(2, None, 256, 128) == 0
    assert size(2, R(64, 64), 192, 128) == 0


def test_last_hip_error_untouched_by_argument_errors(lib):
    assert lin(lib, K=100) == SHAPE
    assert lib.dq_last_hip_error() == 0


def test_python_binding_names_match_the_c_entry_points():
    import fp8_dynamic_quant_amd as dq
    for name in ("dq_quantize_fp8", "dq_quantize_weight_fp8", "dq_linear_fp8",
                 "dq_linear_fp8_noalloc", "dq_linear_fp8_segmented",
                 "dq_linear_fp8_segmented_workspace_size", "dq_layernorm_modulate_quantize_fp8", "dq_linear_qkv_fp8",
                 "dq_linear_qkv_fp8_attn", "dq_quantize_v_fp8", "dq_attention_fp8", "dq_attention_fp8_workspace_size",
                 "dq_quantize_mx_fp8", "dq_linear_mx_fp8", "dq_quantize_mxfp4", "dq_linear_mxfp4",
                 "dq_linear_mxfp4_segmented", "dq_linear_fp8_workspace_size"):
        assert callable(getattr(dq, name))
    assert dq.lib().dq_abi_version() == 11
    assert dq.dq_linear_fp8_workspace_size(512, 12288, 3072) == 4096 + 96 * 262144


def test_python_binding_rejects_cpu_tensors():
    import torch
    import fp8_dynamic_quant_amd as dq
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dq.dq_quantize_fp8(x)
    with pytest.raises(ValueError):
        dq.dq_layernorm_modulate_quantize_fp8(x, torch.zeros(64, dtype=torch.bfloat16),
                                              torch.zeros(64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        dq.dq_linear_fp8(torch.zeros(4, 128, dtype=torch.uint8), torch.zeros(4),
                         torch.zeros(64, 128, dtype=torch.uint8), torch.zeros(64))
