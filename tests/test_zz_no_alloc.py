"""dbf_linear_forward_noalloc, the workspace-free forward (its workspace is
the library's own scratch array on each device), against dbf_linear_forward
with a caller workspace.  Both run the same kernels, so the outputs must be
bitwise equal; each is also checked against the fp64 oracle.  Two calls run
in a row on the scratch, the second with a smaller input, on both paths."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import DEV, assert_close, device_terms, to_np, x64, x_dev

pytestmark = pytest.mark.gpu


def noalloc(terms, N, M, R, x, path):
    """The entry point called through the C ABI (no workspace argument)."""
    y = torch.empty((x.shape[0], N), dtype=torch.float32, device=DEV)
    ct = (D._CTerm * len(terms))()
    for i, t in enumerate(terms):
        ct[i] = D._CTerm(*(v.data_ptr() for v in t))
    st = D.library().dbf_linear_forward_noalloc(
        ct, len(terms), N, M, R, x.data_ptr(), D.DBF_BF16 if x.dtype == torch.bfloat16 else D.DBF_F16,
        x.shape[0], x.stride(0), y.data_ptr(), D.DBF_F32, y.stride(0), 0, path,
        torch.cuda.current_stream().cuda_stream)
    assert st == D.DBF_OK, D.dbf_last_error()
    return y


def with_ws(terms, N, M, R, x, path):
    nb = D.dbf_workspace_bytes(N, M, R, len(terms), x.shape[0], path)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device=DEV)
    return D.dbf_linear_forward(terms, N, M, R, x, ws=ws, path=path)


CASES = [
    # (path, first shape, second smaller shape): N, M, R, L, T
    (D.DBF_PATH_DECODE, (4096, 4096, 2048, 1, 16), (4096, 4096, 2048, 1, 1)),
    (D.DBF_PATH_DECODE, (700, 1500, 300, 3, 9), (130, 300, 70, 2, 2)),
    (D.DBF_PATH_MFMA, (1000, 2048, 512, 2, 200), (300, 500, 200, 1, 20)),
    (D.DBF_PATH_AUTO, (4096, 4096, 2048, 1, 64), (4096, 4096, 2048, 1, 4)),
]


@pytest.mark.parametrize("path,first,second", CASES)
def test_noalloc_matches_workspace_entry(path, first, second):
    for (N, M, R, L, T) in (first, second):
        print("noalloc", path, N, M, R, L, T, flush=True)
        layer, x = S.make_custom(N, M, R, L, T, seed=N + M + R + T)
        terms = device_terms(layer)
        xd = x_dev(x)
        a = noalloc(terms, N, M, R, xd, path)
        b = with_ws(terms, N, M, R, xd, path)
        torch.cuda.synchronize()
        assert torch.equal(a, b), "noalloc output differs from dbf_linear_forward"
        assert_close(to_np(a), O.default().forward(O.terms64(layer), x64(x)))


def test_noalloc_refuses_oversize_and_keeps_working():
    layer, x = S.make_custom(300, 500, 200, 1, 3, seed=7)
    terms = device_terms(layer)
    big = torch.zeros((4096, 8192), dtype=torch.bfloat16, device=DEV)
    ct = (D._CTerm * 1)()
    ct[0] = D._CTerm(*(v.data_ptr() for v in terms[0]))
    y = torch.empty((4096, 8192), dtype=torch.float32, device=DEV)
    st = D.library().dbf_linear_forward_noalloc(
        ct, 1, 8192, 8192, 6144, big.data_ptr(), D.DBF_BF16, 4096, 8192, y.data_ptr(),
        D.DBF_F32, 8192, 0, D.DBF_PATH_AUTO, torch.cuda.current_stream().cuda_stream)
    assert st == D.DBF_EWORKSPACE
    a = noalloc(terms, 300, 500, 200, x_dev(x), D.DBF_PATH_DECODE)
    torch.cuda.synchronize()
    assert_close(to_np(a), O.default().forward(O.terms64(layer), x64(x)))
