"""The C ABI loads, exports what include/fa.h declares, and validates on the host (CPU only).

Every call here is rejected by the host-side checks (or is an empty problem),
so nothing is launched and no GPU is needed.
"""
import math
import os
import re

import pytest

from exact_attention_48_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

A = 0x100000   # a 16-byte aligned fake device address (never dereferenced: validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(capi.LIB_PATH):
        pytest.skip("libfa.so not built")
    return capi.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(capi.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_status_strings(lib):
    for st in (capi.FA_OK, capi.FA_ERR_INVALID_ARGUMENT, capi.FA_ERR_UNSUPPORTED, capi.FA_ERR_WORKSPACE,
               capi.FA_ERR_HIP):
        assert capi.fa_status_string(st).startswith("FA_")
    assert "unknown" in capi.fa_status_string(99)
    assert "gfx950" in capi.fa_version()


def fwd(*, q=A, k=A, v=A, o=A, lse=A, B=1, Hq=2, Hkv=2, N=16, d=128, causal=0, scale=0.1, cu=None, opt=None):
    return capi.fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, cu, opt, stream=0, check=False)


# Every case is invalid, so validation returns before any HIP call.
@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(lse=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(d=96), capi.FA_ERR_UNSUPPORTED),
    (dict(d=256), capi.FA_ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(Hkv=0), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(B=-1), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(N=-5), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(causal=2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=-0.1), capi.FA_ERR_INVALID_ARGUMENT),          # row maxima are taken on the raw Q K^T
    (dict(scale=-1e-30), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(q=A + 8), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(o=A + 2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(lse=A + 2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(cu=A + 1), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(B=1 << 20, N=1 << 20), capi.FA_ERR_UNSUPPORTED),
    (dict(Hq=257, Hkv=257), capi.FA_ERR_UNSUPPORTED),        # Hkv * d > 32768
    (dict(Hq=513, Hkv=513, d=64), capi.FA_ERR_UNSUPPORTED),
    (dict(Hq=256, Hkv=256, q=None), capi.FA_ERR_INVALID_ARGUMENT),   # at the limit: the pointer check decides
    (dict(opt=capi.FaOptions(7, 8.0, 1)), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(opt=capi.FaOptions(0, -1.0, 1)), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(opt=capi.FaOptions(0, 8.0, 2)), capi.FA_ERR_INVALID_ARGUMENT),
])
def test_forward_rejects(lib, kw, expect):
    assert fwd(**kw) == expect


def test_empty_forward_is_ok_without_pointers(lib):
    assert fwd(q=None, k=None, v=None, o=None, lse=None, B=0) == capi.FA_OK
    assert fwd(q=None, k=None, v=None, o=None, lse=None, N=0) == capi.FA_OK


def bwd(*, ws=A, ws_bytes=1 << 30, stages=capi.FA_BWD_ALL, **kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A, B=1, Hq=2, Hkv=2, N=16, d=128, causal=0,
                scale=0.1, cu=None)
    args.update(kw)
    return capi.fa_bwd_ex(args["q"], args["k"], args["v"], args["o"], args["lse"], args["do"], args["dq"],
                          args["dk"], args["dv"], args["B"], args["Hq"], args["Hkv"], args["N"], args["d"],
                          args["causal"], args["scale"], args["cu"], ws, ws_bytes, stages, stream=0, check=False)


@pytest.mark.parametrize("kw,expect", [
    (dict(ws=None, ws_bytes=0), capi.FA_ERR_WORKSPACE),
    (dict(ws_bytes=1), capi.FA_ERR_WORKSPACE),
    (dict(ws=A + 16), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(dq=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(dv=A + 4), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(d=32), capi.FA_ERR_UNSUPPORTED),
    (dict(Hq=4, Hkv=3), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(stages=0), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(stages=8), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=-0.1), capi.FA_ERR_INVALID_ARGUMENT),
])
def test_backward_rejects(lib, kw, expect):
    assert bwd(**kw) == expect


def test_workspace_size(lib):
    assert capi.fa_bwd_workspace_size(0, 2, 2, 128, 128, 1, 0) == 0
    # D_i and LSE_i * log2(e), fp32 each, laid out like the LSE
    assert capi.fa_bwd_workspace_size(2, 16, 16, 8192, 128, 1, 0) == 2 * (2 * 8192 * 16 * 4)
    n = capi.fa_bwd_workspace_size(3, 5, 5, 7, 64, 0, 1)
    assert n >= 2 * 3 * 7 * 5 * 4 and n % 256 == 0


def split(*, q=A, k=A, v=A, o=A, lse=A, B=1, Hq=2, Hkv=2, Nq=16, Nk=64, d=128, causal=1, scale=0.1, n=4, opt=None):
    if opt is not None:
        return capi.fa_fwd_split_ex(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, n, opt, stream=0,
                                    check=False)
    return capi.fa_fwd_split(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, n, stream=0, check=False)


@pytest.mark.parametrize("kw,expect", [
    (dict(n=0), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(n=1025), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(Nq=65, Nk=64), capi.FA_ERR_INVALID_ARGUMENT),       # causal needs Nq <= Nk
    (dict(Nk=-1), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(d=96), capi.FA_ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(q=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(o=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(o=A + 4), capi.FA_ERR_INVALID_ARGUMENT),            # fp32 partial rows need 16-byte alignment
    (dict(causal=2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=math.nan), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=-0.5), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(opt=capi.FaOptions(capi.FA_EXP_POLY, 8.0, 1)), capi.FA_ERR_UNSUPPORTED),   # split kernel: v_exp_f32
    (dict(opt=capi.FaOptions(0, 65.0, 1)), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(opt=capi.FaOptions(0, 8.0, 1), B=0), capi.FA_OK),
    (dict(B=0), capi.FA_OK),                                   # empty: nothing to do
    (dict(Nq=0), capi.FA_OK),
])
def test_split_rejects(lib, kw, expect):
    assert split(**kw) == expect


def merge(*, op=A, lp=A, o=A, lse=A, n=2, B=1, H=2, N=16, d=128):
    return capi.fa_merge(op, lp, o, lse, n, B, H, N, d, stream=0, check=False)


@pytest.mark.parametrize("kw,expect", [
    (dict(n=0), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(n=1025), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(H=0), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(N=-1), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(d=96), capi.FA_ERR_UNSUPPORTED),
    (dict(op=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(lse=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(o=A + 2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(B=0), capi.FA_OK),
    (dict(N=0), capi.FA_OK),
])
def test_merge_rejects(lib, kw, expect):
    assert merge(**kw) == expect


def fp8(*, q=A, k=A, v=A, qd=A, kd=A, o=A, lse=A, B=1, Hq=2, Hkv=2, N=16, d=128, causal=0, scale=0.1, cu=None,
        opt=None):
    if opt is not None:
        return capi.fa_fwd_fp8_ex(q, k, v, qd, kd, o, lse, B, Hq, Hkv, N, d, causal, scale, cu, opt, stream=0,
                                  check=False)
    return capi.fa_fwd_fp8(q, k, v, qd, kd, o, lse, B, Hq, Hkv, N, d, causal, scale, cu, stream=0, check=False)


@pytest.mark.parametrize("kw,expect", [
    (dict(d=64), capi.FA_ERR_UNSUPPORTED),                    # 8-bit Q/K: d = 128 only
    (dict(d=96), capi.FA_ERR_UNSUPPORTED),
    (dict(qd=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(kd=A + 2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(q=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(Hq=3, Hkv=2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(causal=3), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=-0.1), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(opt=capi.FaOptions(capi.FA_EXP_POLY, 8.0, 1)), capi.FA_ERR_UNSUPPORTED),   # 8-bit kernel: v_exp_f32
    (dict(opt=capi.FaOptions(0, 8.0, 3)), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(opt=capi.FaOptions(0, 8.0, 0), B=0), capi.FA_OK),
    (dict(B=0), capi.FA_OK),
])
def test_fp8_rejects(lib, kw, expect):
    assert fp8(**kw) == expect


def fp8_blocks(*, q=A, k=A, v=A, qd=A, kd=A, o=A, lse=A, B=1, Hq=2, Hkv=2, N=16, d=128, causal=0, scale=0.1,
               cu=None, opt=None):
    return capi.fa_fwd_fp8_blockscale(q, k, v, qd, kd, o, lse, B, Hq, Hkv, N, d, causal, scale, cu, opt, stream=0,
                                      check=False)


@pytest.mark.parametrize("kw,expect", [
    (dict(N=64 * 4096 + 1), capi.FA_ERR_UNSUPPORTED),         # more than 4096 descale blocks
    (dict(N=64 * 4096 + 1, B=0), capi.FA_ERR_UNSUPPORTED),    # the block limit comes before the empty check
    (dict(d=64), capi.FA_ERR_UNSUPPORTED),
    (dict(qd=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(kd=A + 2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(opt=capi.FaOptions(capi.FA_EXP_POLY, 8.0, 1)), capi.FA_ERR_UNSUPPORTED),
    (dict(B=0), capi.FA_OK),
    (dict(N=0), capi.FA_OK),
])
def test_fp8_blockscale_rejects(lib, kw, expect):
    assert fp8_blocks(**kw) == expect


def exp2_eval(*, x=A, y=A + 4096, n=16, mode=capi.FA_EXP_HW):
    return capi.fa_exp2_eval(x, y, n, mode, stream=0, check=False)


@pytest.mark.parametrize("kw,expect", [
    (dict(mode=2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(mode=-1), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(n=-1), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(x=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(y=A + 2), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(n=0), capi.FA_OK),
    (dict(n=0, mode=capi.FA_EXP_POLY), capi.FA_OK),
])
def test_exp2_eval_rejects(lib, kw, expect):
    assert exp2_eval(**kw) == expect


def bwd_noalloc(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A, B=1, Hq=2, Hkv=2, N=16, d=128, causal=0,
                scale=0.1, cu=None)
    args.update(kw)
    return capi.fa_bwd_noalloc(args["q"], args["k"], args["v"], args["o"], args["lse"], args["do"], args["dq"],
                               args["dk"], args["dv"], args["B"], args["Hq"], args["Hkv"], args["N"], args["d"],
                               args["causal"], args["scale"], args["cu"], stream=0, check=False)


@pytest.mark.parametrize("kw,expect", [
    (dict(dq=None), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(dk=A + 4), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(d=32), capi.FA_ERR_UNSUPPORTED),
    (dict(scale=-1.0), capi.FA_ERR_INVALID_ARGUMENT),
    (dict(Hq=4, Hkv=3), capi.FA_ERR_INVALID_ARGUMENT),
    # 2 x 4 x 65536 x 64 x 4 bytes of D and LSE*log2(e) = 128 MiB > the fixed 64 MiB array
    (dict(B=4, N=65536, Hq=64, Hkv=64), capi.FA_ERR_WORKSPACE),
    (dict(B=0), capi.FA_OK),
])
def test_bwd_noalloc_rejects_before_launch(lib, kw, expect):
    assert bwd_noalloc(**kw) == expect


def test_bwd_noalloc_limit(lib):
    assert capi.fa_bwd_noalloc_max_workspace() == 64 << 20
    # the largest workloads here fit: the causal 8192-token backward and the packed GQA one (B * N bound)
    assert capi.fa_bwd_workspace_size(2, 16, 16, 8192, 128, 1, 0) <= 64 << 20
    assert capi.fa_bwd_workspace_size(16, 32, 8, 16007, 128, 1, 1) <= 64 << 20
