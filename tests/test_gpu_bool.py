"""dbf_bool_forward (the Multi-Boolean form: y = sum_k s_out_k . (Wb_k
(s_in_k . x))) on the decode and MFMA paths against the fp64 oracle."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import (DEV, assert_close, assert_close_bf16, f16_dev, pack_signs, to_np, x64,
                     x_dev)

pytestmark = pytest.mark.gpu

DEC, MF, AUTO = D.DBF_PATH_DECODE, D.DBF_PATH_MFMA, D.DBF_PATH_AUTO


def dev_kernels(layer):
    out = [D.DbfBoolKernel(pack_signs(k["w"]), f16_dev(k["s_in"]), f16_dev(k["s_out"]))
           for k in layer["kernels"]]
    torch.cuda.synchronize()
    return out


def oracle_kernels(layer):
    return [dict(w=k["w"], s_in=np.asarray(k["s_in"], np.float64),
                 s_out=np.asarray(k["s_out"], np.float64)) for k in layer["kernels"]]


def run(layer, x, path=AUTO, kernels=None, **kw):
    kernels = kernels or dev_kernels(layer)
    y = D.dbf_bool_forward(kernels, layer["N"], layer["M"], x_dev(x), path=path, **kw)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("config,T,path", [(6, 1, DEC), (6, 4, DEC), (6, 16, DEC),
                                           (6, 1, MF), (6, 16, MF), (6, 256, AUTO),
                                           (7, 1, AUTO), (7, 8, DEC), (7, 8, MF),
                                           (7, 64, AUTO)])
def test_configs(config, T, path):
    print("bool config", config, "T", T, "path", path, flush=True)
    layer = S.make_bool_layer(config)
    x = S.make_x(config, T)
    y = to_np(run(layer, x, path))
    # every token against the oracle, over the whole output and per token
    ref = O.default().bool_forward(oracle_kernels(layer), x64(x))
    assert_close(y, ref)
    num = np.linalg.norm(y - ref, axis=1)
    assert np.all(num <= 2e-3 * np.linalg.norm(ref, axis=1))


@pytest.mark.parametrize("path", [DEC, MF])
@pytest.mark.parametrize("scale", [2.0 ** 20, 2.0 ** -20])
def test_extreme_activation_scale(path, scale):
    # |s_in . x| far above the fp16 range, or far below its normal range: the
    # MFMA path's per-token power of two keeps the fp16 operand in range
    layer, x = S.make_custom_bool(300, 1000, 2, 40, seed=41)
    xs = S.f32_to_bf16_bits((x64(x) * scale).astype(np.float32))
    assert np.array_equal(x64(xs), x64(x) * scale)  # a power of two: exact
    y = to_np(run(layer, xs, path))
    assert np.all(np.isfinite(y))
    ref = O.default().bool_forward(oracle_kernels(layer), x64(xs))
    assert_close(y, ref)


# ragged N and M (not multiples of 4, 32, 64 or 128), M < 128, one to four
# kernels; on the MFMA path the few-tile shapes split K
ODD = [(1, 1, 1, 1), (65, 33, 3, 1), (130, 300, 2, 5), (300, 129, 3, 20),
       (77, 1000, 2, 40), (513, 64, 1, 17), (40, 4100, 1, 33), (700, 3000, 4, 9),
       (2000, 2048, 2, 130), (77, 9000, 2, 40)]


@pytest.mark.parametrize("N,M,K,T", ODD)
@pytest.mark.parametrize("path", [DEC, MF])
def test_odd_shapes(N, M, K, T, path):
    print("bool odd", N, M, K, T, path, flush=True)
    layer, x = S.make_custom_bool(N, M, K, T, seed=N + 3 * M + K)
    y = to_np(run(layer, x, path))
    ref = O.default().bool_forward(oracle_kernels(layer), x64(x))
    assert_close(y, ref)


# one column tile at one to three tokens: K split 6, 5, 10 and 16 ways on
# the MFMA path (the split sums are instantiated per count)
SPLITS = [(100, 768, 2, 3), (128, 1280, 1, 1), (128, 896, 3, 1), (128, 4096, 2, 1)]


@pytest.mark.parametrize("N,M,K,T", SPLITS)
def test_split_counts(N, M, K, T):
    print("bool split", N, M, K, T, flush=True)
    layer, x = S.make_custom_bool(N, M, K, T, seed=5 * N + M + K)
    y = to_np(run(layer, x, MF))
    ref = O.default().bool_forward(oracle_kernels(layer), x64(x))
    assert_close(y, ref)


@pytest.mark.parametrize("path", [DEC, MF])
def test_output_dtypes_accumulate_strides(path):
    N, M, K, T = 301, 900, 2, 12
    layer, x = S.make_custom_bool(N, M, K, T, seed=17, x_kind="f16")
    ref = O.default().bool_forward(oracle_kernels(layer), x64(x))
    kernels = dev_kernels(layer)
    xd = torch.zeros((T, 904), dtype=torch.float16, device=DEV)
    xd[:, :M] = x_dev(x)
    big = torch.full((T, 320), 7.0, dtype=torch.float32, device=DEV)
    base = torch.randn((T, N), dtype=torch.float32, device=DEV)
    big[:, :N] = base
    D.dbf_bool_forward(kernels, N, M, xd[:, :M], y=big[:, :N], accumulate=True, path=path)
    torch.cuda.synchronize()
    assert_close(to_np(big[:, :N]), ref + to_np(base))
    assert torch.all(big[:, N:] == 7.0)
    yb = torch.full((T, 310), 3.0, dtype=torch.bfloat16, device=DEV)
    D.dbf_bool_forward(kernels, N, M, xd[:, :M], y=yb[:, :N], path=path)
    torch.cuda.synchronize()
    assert_close_bf16(to_np(yb[:, :N]), ref)
    assert torch.all(yb[:, N:] == 3.0)


def test_deterministic_and_paths_agree():
    layer = S.make_bool_layer(6)
    x = S.make_x(6, 16)
    kernels = dev_kernels(layer)
    a = to_np(run(layer, x, DEC, kernels=kernels))
    assert np.array_equal(a, to_np(run(layer, x, DEC, kernels=kernels)))
    b = to_np(run(layer, x, MF, kernels=kernels))
    assert np.array_equal(b, to_np(run(layer, x, MF, kernels=kernels)))
    assert_close(a, b)


def test_row_flip_on_gpu():
    # flipping row 9 of one kernel's signs changes output 9 only
    layer, x = S.make_custom_bool(128, 512, 2, 3, seed=23)
    y = to_np(run(layer, x, DEC))
    layer["kernels"][1]["w"][9, :] *= -1
    y2 = to_np(run(layer, x, DEC))
    rest = [n for n in range(128) if n != 9]
    assert np.array_equal(y2[:, rest], y[:, rest])
    assert not np.allclose(y2[:, 9], y[:, 9])


def test_shared_workspace_with_the_double_binary_layer():
    # one workspace serves boolean-kernel and double-binary calls in turn; the
    # handoff head is zero after each and no wait gave up
    layer, x = S.make_custom_bool(256, 1024, 2, 3, seed=5)
    dlayer, dx = S.make_custom(256, 1024, 96, 2, 3, seed=6)
    nb = max(D.dbf_bool_workspace_bytes(256, 1024, 2, 3, DEC),
             D.dbf_workspace_bytes(256, 1024, 96, 2, 3, DEC))
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    from dbfutil import device_terms
    dterms = device_terms(dlayer)
    o = O.default()
    ref = o.bool_forward(oracle_kernels(layer), x64(x))
    dref = o.forward(O.terms64(dlayer), x64(dx))
    kernels = dev_kernels(layer)
    for _ in range(2):
        y = D.dbf_bool_forward(kernels, 256, 1024, x_dev(x), ws=ws, path=DEC)
        D.dbf_workspace_check(ws)
        assert not ws[:D.DBF_WS_HEAD_BYTES].any()
        assert_close(to_np(y), ref)
        y = D.dbf_linear_forward(dterms, 256, 1024, 96, x_dev(dx), ws=ws, path=DEC)
        D.dbf_workspace_check(ws)
        assert not ws[:D.DBF_WS_HEAD_BYTES].any()
        assert_close(to_np(y), dref)


def test_zero_tokens():
    layer, _ = S.make_custom_bool(8, 8, 1, 1, seed=1)
    x = torch.empty((0, 8), dtype=torch.bfloat16, device=DEV)
    y = D.dbf_bool_forward(dev_kernels(layer), 8, 8, x)
    assert y.shape == (0, 8)


@pytest.mark.parametrize("path", [DEC, MF])
def test_maximum_kernels(path):
    layer, x = S.make_custom_bool(150, 700, D.DBF_MAX_TERMS, 5, seed=99)
    y = to_np(run(layer, x, path))
    assert_close(y, O.default().bool_forward(oracle_kernels(layer), x64(x)))
