"""Host checks of the C ABI: the library loads, exports every entry point
include/dbf.h declares, and rejects bad arguments with the documented status
before making any HIP call (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "dbf.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    lib = D.library()
    names = declared_functions()
    assert set(names) == set(D.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_versions():
    assert D.dbf_abi_version() == 1
    assert D.dbf_layout_version() == 1


@pytest.mark.parametrize("rows,k", [(1, 1), (3, 31), (64, 32), (65, 33),
                                    (70, 97), (130, 300), (16, 4096), (4096, 16),
                                    (11008, 2048), (8192, 6144)])
def test_packed_bytes_matches_oracle_layout(rows, k):
    assert D.dbf_packed_bytes(rows, k) == 4 * O.default().packed_words(rows, k)


def test_packed_bytes_edges():
    assert D.dbf_packed_bytes(0, 5) == 0
    assert D.dbf_packed_bytes(5, 0) == 0
    # full tiles are whole 128-byte lines
    assert D.dbf_packed_bytes(64, 128) == 1024


def test_workspace_bytes():
    assert D.dbf_workspace_bytes(512, 512, 256, 1, 0) == 0
    assert D.dbf_workspace_bytes(512, 512, 256, 1, 1, D.DBF_PATH_DECODE) > 0
    assert D.dbf_workspace_bytes(512, 512, 256, 1, 1, D.DBF_PATH_MFMA) > 0


# (N, M, R, terms, tokens, path): decode while T <= 4 or the sign work
# terms * ceil(T / 4) * R * (N + M) is at most 8.0e7
AUTO_CASES = [(4096, 4096, 2048, 1, 1, "decode"), (4096, 4096, 2048, 1, 16, "decode"),
              (4096, 4096, 2048, 1, 17, "mfma"), (4096, 4096, 2048, 1, 20, "mfma"),
              (4096, 4096, 2048, 1, 32, "mfma"),
              (4096, 4096, 2048, 2, 8, "decode"), (4096, 4096, 2048, 2, 9, "mfma"),
              (4096, 4096, 2048, 2, 16, "mfma"), (11008, 4096, 2048, 3, 4, "decode"),
              (11008, 4096, 2048, 3, 5, "mfma"), (8192, 8192, 6144, 1, 4, "decode"),
              (8192, 8192, 6144, 1, 5, "mfma"), (512, 512, 256, 1, 64, "decode"),
              (512, 512, 256, 8, 64, "decode"), (16384, 16384, 8192, 8, 1, "decode"),
              (4096, 4096, 2048, 1, 4096, "mfma")]


@pytest.mark.parametrize("N,M,R,L,T,path", AUTO_CASES)
def test_auto_path_rule(N, M, R, L, T, path):
    want = D.DBF_PATH_DECODE if path == "decode" else D.DBF_PATH_MFMA
    # the rule itself, written out
    work = L * -(-T // 4) * R * (N + M)
    assert (T <= 4 or work <= 8.0e7) == (path == "decode")
    auto = D.dbf_workspace_bytes(N, M, R, L, T, D.DBF_PATH_AUTO)
    assert auto == D.dbf_workspace_bytes(N, M, R, L, T, want)
    other = D.DBF_PATH_MFMA if want == D.DBF_PATH_DECODE else D.DBF_PATH_DECODE
    assert auto != D.dbf_workspace_bytes(N, M, R, L, T, other)


L = D.library()
FAKE = 1 << 20            # a 16-byte aligned non-NULL address, never touched
MIS = FAKE + 8            # misaligned


def _terms(n=1, **over):
    arr = (D._CTerm * max(n, 1))()
    for i in range(n):
        f = dict(b1=FAKE, b2=FAKE, alpha=FAKE, beta=FAKE, gamma=FAKE)
        f.update(over)
        arr[i] = D._CTerm(**f)
    return arr


def fwd(terms=None, n=1, N=8, M=8, R=8, x=FAKE, xdt=D.DBF_BF16, T=1, ldx=8,
        y=FAKE, ydt=D.DBF_F32, ldy=8, acc=0, ws=FAKE, wsb=1 << 30, path=0):
    if terms is None:
        terms = _terms(n)
    return L.dbf_linear_forward(terms, n, N, M, R, x, xdt, T, ldx, y, ydt, ldy,
                                acc, ws, wsb, path, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), D.DBF_EINVAL), (dict(n=9), D.DBF_EINVAL),
    (dict(terms=_terms(1, b1=None)), D.DBF_EINVAL),
    (dict(terms=_terms(1, gamma=None)), D.DBF_EINVAL),
    (dict(terms=_terms(1, b2=MIS)), D.DBF_EALIGN),
    (dict(terms=_terms(1, alpha=FAKE + 1)), D.DBF_EALIGN),
    (dict(N=0), D.DBF_EINVAL), (dict(R=0), D.DBF_EINVAL), (dict(T=-1), D.DBF_EINVAL),
    (dict(xdt=D.DBF_F32), D.DBF_EDTYPE), (dict(ydt=D.DBF_I8), D.DBF_EDTYPE),
    (dict(acc=2), D.DBF_EINVAL), (dict(path=7), D.DBF_EINVAL),
    (dict(ldx=7), D.DBF_EINVAL), (dict(ldy=7), D.DBF_EINVAL),
    (dict(x=None), D.DBF_EINVAL), (dict(y=MIS), D.DBF_EALIGN),
    (dict(ws=None), D.DBF_EWORKSPACE), (dict(wsb=16), D.DBF_EWORKSPACE),
    (dict(ws=MIS), D.DBF_EALIGN),
])
def test_forward_validation(kw, code):
    assert fwd(**kw) == code
    assert D.dbf_last_error()


def fwd_noalloc(terms=None, n=1, N=8, M=8, R=8, x=FAKE, xdt=D.DBF_BF16, T=1, ldx=8,
                y=FAKE, ydt=D.DBF_F32, ldy=8, acc=0, path=0):
    if terms is None:
        terms = _terms(n)
    return L.dbf_linear_forward_noalloc(terms, n, N, M, R, x, xdt, T, ldx, y, ydt, ldy, acc,
                                        path, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), D.DBF_EINVAL), (dict(terms=_terms(1, b2=MIS)), D.DBF_EALIGN),
    (dict(N=0), D.DBF_EINVAL), (dict(T=-1), D.DBF_EINVAL),
    (dict(xdt=D.DBF_F32), D.DBF_EDTYPE), (dict(ydt=D.DBF_I8), D.DBF_EDTYPE),
    (dict(acc=2), D.DBF_EINVAL), (dict(path=7), D.DBF_EINVAL),
    (dict(ldx=7), D.DBF_EINVAL), (dict(x=None), D.DBF_EINVAL), (dict(y=MIS), D.DBF_EALIGN),
    # the 8192 x 8192, R 6144 layer at 4096 tokens needs more workspace than
    # the library's scratch: refused before any HIP call
    (dict(N=8192, M=8192, R=6144, T=4096, ldx=8192, ldy=8192), D.DBF_EWORKSPACE),
])
def test_forward_noalloc_validation(kw, code):
    assert fwd_noalloc(**kw) == code
    assert D.dbf_last_error()


def test_forward_noalloc_limit():
    # the limit is the scratch size: sizes just above it are refused, and the
    # workspace of the one-token 4096 x 4096 layer fits
    assert L.dbf_workspace_bytes(8192, 8192, 6144, 1, 4096, 0) > D.DBF_NOALLOC_SCRATCH_BYTES
    assert L.dbf_workspace_bytes(4096, 4096, 2048, 1, 1, 0) <= D.DBF_NOALLOC_SCRATCH_BYTES
    assert fwd_noalloc(T=0, x=None, y=None) == D.DBF_OK


def test_forward_zero_tokens_is_a_noop():
    assert fwd(T=0, x=None, y=None, ws=None) == D.DBF_OK


def i8(terms=None, n=1, N=8, M=8, R=8, x=FAKE, T=1, ldx=8, s1=None, s2=None,
       y=None, ydt=D.DBF_F32, ldy=8, ws=FAKE, wsb=1 << 30):
    if terms is None:
        terms = _terms(n, gamma=None)
    return L.dbf_linear_forward_i8(terms, n, N, M, R, x, T, ldx, s1, s2, y, ydt,
                                   ldy, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(terms=_terms(1)), D.DBF_EINVAL),                       # gamma given
    (dict(s2=FAKE), D.DBF_EINVAL),                               # s2 with beta
    (dict(n=2, terms=(lambda a: (setattr(a[1], "beta", None), a)[1])(_terms(2, gamma=None))),
     D.DBF_EINVAL),                                              # mixed beta
    (dict(terms=_terms(1, gamma=None, beta=None), R=65536, M=65536),
     D.DBF_EUNSUPPORTED),                                        # int32 overflow
    (dict(y=FAKE, ydt=D.DBF_I32), D.DBF_EDTYPE),
    (dict(s1=MIS), D.DBF_EALIGN),
    (dict(wsb=4), D.DBF_EWORKSPACE),
])
def test_i8_validation(kw, code):
    assert i8(**kw) == code


def ad(w0=FAKE, ldw=8, terms=None, n=1, N=8, M=8, R=8, x=FAKE, T=1, ldx=8,
       y=FAKE, ydt=D.DBF_F32, ldy=8, ws=FAKE, wsb=1 << 30):
    if terms is None and n > 0:
        terms = _terms(n)
    return L.lordba_adapter_forward(w0, ldw, terms, n, N, M, R, x, T, ldx, y, ydt,
                                    ldy, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), D.DBF_EINVAL), (dict(n=9), D.DBF_EINVAL),
    (dict(ldw=4), D.DBF_EINVAL), (dict(w0=None), D.DBF_EINVAL),
    (dict(w0=MIS), D.DBF_EALIGN), (dict(ydt=7), D.DBF_EDTYPE),
    (dict(ws=None), D.DBF_EWORKSPACE), (dict(R=0), D.DBF_EINVAL),
])
def test_adapter_validation(kw, code):
    assert ad(**kw) == code


def _bools(n=1, **over):
    arr = (D._CBool * max(n, 1))()
    for i in range(n):
        f = dict(w=FAKE, s_in=FAKE, s_out=FAKE)
        f.update(over)
        arr[i] = D._CBool(**f)
    return arr


def bfwd(kernels=None, n=1, N=8, M=8, x=FAKE, xdt=D.DBF_BF16, T=1, ldx=8,
         y=FAKE, ydt=D.DBF_F32, ldy=8, acc=0, ws=FAKE, wsb=1 << 30, path=0):
    if kernels is None:
        kernels = _bools(n)
    return L.dbf_bool_forward(kernels, n, N, M, x, xdt, T, ldx, y, ydt, ldy, acc,
                              ws, wsb, path, None)


@pytest.mark.parametrize("kw,code", [
    (dict(kernels=None, n=0), D.DBF_EINVAL), (dict(n=0), D.DBF_EINVAL),
    (dict(n=9), D.DBF_EINVAL),
    (dict(kernels=_bools(1, w=None)), D.DBF_EINVAL),
    (dict(kernels=_bools(1, s_in=None)), D.DBF_EINVAL),
    (dict(kernels=_bools(1, s_out=None)), D.DBF_EINVAL),
    (dict(kernels=_bools(1, w=MIS)), D.DBF_EALIGN),
    (dict(kernels=_bools(1, s_out=FAKE + 1)), D.DBF_EALIGN),
    (dict(N=0), D.DBF_EINVAL), (dict(M=0), D.DBF_EINVAL), (dict(T=-1), D.DBF_EINVAL),
    (dict(xdt=D.DBF_I8), D.DBF_EDTYPE), (dict(ydt=D.DBF_I32), D.DBF_EDTYPE),
    (dict(acc=3), D.DBF_EINVAL), (dict(path=5), D.DBF_EINVAL),
    (dict(ldx=7), D.DBF_EINVAL), (dict(ldy=7), D.DBF_EINVAL),
    (dict(y=None), D.DBF_EINVAL), (dict(x=MIS), D.DBF_EALIGN),
    (dict(ws=None), D.DBF_EWORKSPACE), (dict(wsb=100), D.DBF_EWORKSPACE),
    (dict(ws=MIS), D.DBF_EALIGN),
])
def test_bool_forward_validation(kw, code):
    assert bfwd(**kw) == code
    assert D.dbf_last_error()


def test_bool_zero_tokens_is_a_noop():
    assert bfwd(T=0, x=None, y=None, ws=None, wsb=0) == D.DBF_OK


def test_bool_workspace_bytes():
    assert D.dbf_bool_workspace_bytes(4096, 4096, 2, 0) == 0
    assert D.dbf_bool_workspace_bytes(0, 4096, 2, 1) == 0
    # decode: the head plus fp32 partials of every kernel and K-split
    dec = D.dbf_bool_workspace_bytes(4096, 4096, 2, 1, D.DBF_PATH_DECODE)
    assert dec > D.DBF_WS_HEAD_BYTES and (dec - D.DBF_WS_HEAD_BYTES) % (2 * 4096 * 4) == 0
    # MFMA: at least the fp16 u of every kernel and token
    assert D.dbf_bool_workspace_bytes(4096, 4096, 2, 512, D.DBF_PATH_MFMA) >= 2 * 512 * 4096 * 2
    assert (D.dbf_bool_workspace_bytes(4096, 4096, 2, 1) == dec)


@pytest.mark.parametrize("T,K,path", [(1, 2, "decode"), (2, 8, "decode"), (4, 2, "decode"),
                                      (3, 3, "mfma"), (4, 3, "mfma"), (8, 2, "decode"),
                                      (9, 2, "mfma"), (5, 3, "mfma"), (16, 1, "decode"),
                                      (17, 1, "mfma"), (4, 8, "mfma")])
def test_bool_auto_path_rule(T, K, path):
    # decode while the decode launch has one token block (T <= 2) or
    # n_kernels times its blocks (ceil(T / 2) to 4 tokens, ceil(T / 4)
    # above) is at most 4
    want = D.DBF_PATH_DECODE if path == "decode" else D.DBF_PATH_MFMA
    auto = D.dbf_bool_workspace_bytes(4096, 4096, K, T, D.DBF_PATH_AUTO)
    assert auto == D.dbf_bool_workspace_bytes(4096, 4096, K, T, want)
    other = D.DBF_PATH_MFMA if want == D.DBF_PATH_DECODE else D.DBF_PATH_DECODE
    assert auto != D.dbf_bool_workspace_bytes(4096, 4096, K, T, other)


def _tts(n=1, **over):
    arr = (D._CTermT * max(n, 1))()
    for i in range(n):
        f = dict(b1t=FAKE, b2t=FAKE)
        f.update(over)
        arr[i] = D._CTermT(**f)
    return arr


def bwd(terms=None, tterms=None, n=1, N=8, M=8, R=8, x=FAKE, xdt=D.DBF_BF16, ldx=8,
        dy=FAKE, dydt=D.DBF_F32, lddy=8, T=1, dx=FAKE, dxdt=D.DBF_F32, lddx=8,
        da=FAKE, db=FAKE, dg=FAKE, ws=FAKE, wsb=1 << 30, path=0):
    terms = _terms(n) if terms is None else terms
    tterms = _tts(n) if tterms is None else tterms
    return L.dbf_linear_backward(terms, tterms, n, N, M, R, x, xdt, ldx, dy, dydt, lddy, T,
                                 dx, dxdt, lddx, da, db, dg, ws, wsb, path, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), D.DBF_EINVAL), (dict(n=9), D.DBF_EINVAL),
    (dict(terms=_terms(1, gamma=None)), D.DBF_EINVAL),
    (dict(tterms=_tts(1, b1t=None)), D.DBF_EINVAL),
    (dict(tterms=_tts(1, b2t=MIS)), D.DBF_EALIGN),
    (dict(R=0), D.DBF_EINVAL), (dict(T=-1), D.DBF_EINVAL),
    (dict(xdt=D.DBF_F32), D.DBF_EDTYPE), (dict(dydt=D.DBF_I8), D.DBF_EDTYPE),
    (dict(dxdt=D.DBF_I32), D.DBF_EDTYPE), (dict(path=4), D.DBF_EINVAL),
    (dict(ldx=7), D.DBF_EINVAL), (dict(lddy=7), D.DBF_EINVAL), (dict(lddx=7), D.DBF_EINVAL),
    (dict(dy=None), D.DBF_EINVAL), (dict(dx=MIS), D.DBF_EALIGN),
    (dict(db=FAKE + 2), D.DBF_EALIGN),
    (dict(ws=None), D.DBF_EWORKSPACE), (dict(wsb=64), D.DBF_EWORKSPACE),
])
def test_backward_validation(kw, code):
    assert bwd(**kw) == code
    assert D.dbf_last_error()


def test_backward_optional_outputs_and_zero_tokens():
    # every output may be NULL; T = 0 does nothing
    assert bwd(T=0, x=None, dy=None, ws=None, wsb=0) == D.DBF_OK
    assert bwd(dx=None, lddx=0, da=None, db=None, dg=None, dxdt=99, T=0) == D.DBF_OK


def test_transpose_packed_validation():
    assert L.dbf_transpose_packed(None, 4, 4, FAKE, None) == D.DBF_EINVAL
    assert L.dbf_transpose_packed(MIS, 4, 4, FAKE, None) == D.DBF_EALIGN
    assert L.dbf_transpose_packed(FAKE, -1, 4, FAKE, None) == D.DBF_EINVAL
    assert L.dbf_transpose_packed(FAKE, 0, 4, FAKE, None) == D.DBF_OK


def test_backward_workspace_bytes():
    assert D.dbf_backward_workspace_bytes(64, 64, 32, 1, 0) == 0
    small = D.dbf_backward_workspace_bytes(512, 512, 256, 1, 8)
    # at least the four fp32 intermediates
    assert small >= 4 * 8 * (256 + 512 + 256 + 512)
    assert D.dbf_backward_workspace_bytes(512, 512, 256, 2, 8) > small


def madd(w0=FAKE, ldw=8, adapters=None, n=2, N=8, M=8, R=8, idx=FAKE, x=FAKE, T=1, ldx=8,
         y=FAKE, ydt=D.DBF_F32, ldy=8, ws=FAKE, wsb=1 << 30):
    adapters = _terms(max(n, 1)) if adapters is None else adapters
    return L.lordba_multi_adapter_forward(w0, ldw, adapters, n, N, M, R, idx, x, T, ldx, y,
                                          ydt, ldy, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), D.DBF_EINVAL), (dict(n=33), D.DBF_EINVAL),
    (dict(adapters=_terms(2, beta=None)), D.DBF_EINVAL),
    (dict(adapters=_terms(2, b1=MIS)), D.DBF_EALIGN),
    (dict(w0=None), D.DBF_EINVAL), (dict(w0=MIS), D.DBF_EALIGN), (dict(ldw=7), D.DBF_EINVAL),
    (dict(R=0), D.DBF_EINVAL), (dict(T=-1), D.DBF_EINVAL), (dict(ydt=D.DBF_I8), D.DBF_EDTYPE),
    (dict(idx=None), D.DBF_EINVAL), (dict(idx=FAKE + 2), D.DBF_EALIGN),
    (dict(ldx=7), D.DBF_EINVAL), (dict(ldy=7), D.DBF_EINVAL), (dict(x=MIS), D.DBF_EALIGN),
    (dict(ws=None), D.DBF_EWORKSPACE),
])
def test_multi_adapter_validation(kw, code):
    assert madd(**kw) == code
    assert D.dbf_last_error()


def test_multi_adapter_oracle_composition():
    # several adapters beside one base, composed from the pinned oracle
    # functions: all -1 is the base, one adapter for all is adapter mode,
    # and each token matches its own single-token evaluation
    o = O.default()
    from bit_adapters_amd import synth as S
    ads = [S.make_custom(24, 40, 8, 1, 1, seed=s)[0]["terms"][0] for s in range(3)]
    layer, x = S.make_custom(24, 40, 8, 1, 7, seed=9, base=True)
    w0 = O.widen_bf16(layer["w0"])
    xx = O.widen_bf16(x)
    ads64 = [dict(b1=a["b1"], b2=a["b2"], alpha=a["alpha"].astype(np.float64),
                  beta=a["beta"].astype(np.float64), gamma=a["gamma"].astype(np.float64))
             for a in ads]
    assert np.array_equal(o.multi_adapter(w0, ads64, [-1] * 7, xx), o.dense(w0, xx))
    assert np.allclose(o.multi_adapter(w0, ads64, [1] * 7, xx), o.adapter(w0, [ads64[1]], xx),
                       rtol=1e-13, atol=1e-15)
    idx = [0, -1, 2, 2, 1, -1, 0]
    y = o.multi_adapter(w0, ads64, idx, xx)
    for t, a in enumerate(idx):
        ref = o.dense(w0, xx[t:t + 1]) + (o.forward([ads64[a]], xx[t:t + 1]) if a >= 0 else 0)
        assert np.allclose(y[t], ref[0], rtol=1e-13, atol=1e-15)


def test_header_compiles_as_c(tmp_path):
    # the ABI header is plain C: no HIP or C++ type in any declaration
    src = tmp_path / "h.c"
    src.write_text('#include "dbf.h"\nint main(void) { return 0; }\n')
    inc = os.path.dirname(HEADER)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", inc, "-c", str(src), "-o", str(tmp_path / "h.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_workspace_check_validation():
    assert L.dbf_workspace_check(None, None) == D.DBF_EINVAL
    assert L.dbf_workspace_check(MIS, None) == D.DBF_EALIGN
    m = re.search(r"#define DBF_WS_HEAD_BYTES (\d+)", open(HEADER).read())
    assert D.DBF_WS_HEAD_BYTES == int(m.group(1))


def test_pack_validation():
    assert L.dbf_pack(FAKE, 9, 4, 4, 4, FAKE, None) == D.DBF_EDTYPE
    assert L.dbf_pack(None, D.DBF_I8, 4, 4, 4, FAKE, None) == D.DBF_EINVAL
    assert L.dbf_pack(FAKE, D.DBF_I8, 4, 4, 3, FAKE, None) == D.DBF_EINVAL
    assert L.dbf_pack(FAKE, D.DBF_I8, 4, 4, 4, MIS, None) == D.DBF_EALIGN
    assert L.dbf_pack(FAKE, D.DBF_I8, 0, 4, 4, FAKE, None) == D.DBF_OK
    assert L.dbf_unpack(FAKE, 4, 4, FAKE, 3, None) == D.DBF_EINVAL
    assert L.dbf_unpack(MIS, 4, 4, FAKE, 4, None) == D.DBF_EALIGN


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device error")
def test_valid_call_without_device_reports_edevice():
    assert fwd() == D.DBF_EDEVICE
    assert "device" in D.dbf_last_error()


def svid(w=FAKE, dt=D.DBF_F32, N=8, M=8, ldw=8, n=1, outs=None, iters=8, res=None, ws=FAKE,
         wsb=1 << 30):
    if outs is None:
        outs = (D._CBoolOut * max(n, 1))()
        for i in range(n):
            outs[i] = D._CBoolOut(FAKE, FAKE, FAKE)
    return L.dbf_svid_extract(w, dt, N, M, ldw, n, outs, iters, res, ws, wsb, None)


def _souts(**over):
    a = (D._CBoolOut * 1)()
    f = dict(w=FAKE, s_in=FAKE, s_out=FAKE)
    f.update(over)
    a[0] = D._CBoolOut(**f)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), D.DBF_EINVAL), (dict(dt=D.DBF_I8), D.DBF_EDTYPE), (dict(w=None), D.DBF_EINVAL),
    (dict(ldw=7), D.DBF_EINVAL), (dict(w=FAKE + 2), D.DBF_EALIGN),
    (dict(n=0), D.DBF_EINVAL), (dict(n=9), D.DBF_EINVAL),
    (dict(iters=0), D.DBF_EINVAL), (dict(iters=1001), D.DBF_EINVAL),
    (dict(outs=_souts(w=None)), D.DBF_EINVAL), (dict(outs=_souts(w=MIS)), D.DBF_EALIGN),
    (dict(outs=_souts(s_in=FAKE + 1)), D.DBF_EALIGN), (dict(res=FAKE + 2), D.DBF_EALIGN),
    (dict(ws=None), D.DBF_EWORKSPACE), (dict(wsb=16), D.DBF_EWORKSPACE),
])
def test_svid_validation(kw, code):
    assert svid(**kw) == code
    assert D.dbf_last_error()


def test_svid_workspace_bytes():
    # the fp32 residual dominates: at least N * M * 4 bytes
    assert L.dbf_svid_workspace_bytes(0, 8) == 0
    assert L.dbf_svid_workspace_bytes(300, 1000) >= 300 * 1000 * 4
