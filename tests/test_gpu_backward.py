"""dbf_transpose_packed and dbf_linear_backward against the oracle: the
transpose bit for bit, the gradients (dx and the three scale vectors of
every term) to the float tolerance."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import DEV, assert_close, assert_close_bf16, device_terms, to_np, x64, x_dev

pytestmark = pytest.mark.gpu

DEC, MF, AUTO = D.DBF_PATH_DECODE, D.DBF_PATH_MFMA, D.DBF_PATH_AUTO


@pytest.mark.parametrize("rows,k", [(1, 1), (3, 70), (64, 128), (130, 33), (200, 513),
                                    (4096, 2048), (11008, 2048), (97, 4100)])
def test_transpose_packed_bit_exact(rows, k):
    v = S.random_values(rows, k, seed=rows + k)
    o = O.default()
    packed = D.dbf_pack(torch.from_numpy(v).to(DEV))
    got = D.dbf_transpose_packed(packed, rows, k)
    torch.cuda.synchronize()
    want = o.transpose_packed(o.pack(v.astype(np.float64)), rows, k)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want)


def _dy(T, N, seed, kind="f32"):
    v = np.random.default_rng([0xDBF, 105, seed, T, N]).standard_normal((T, N)).astype(np.float32)
    if kind == "bf16":
        bits = S.f32_to_bf16_bits(v)
        return x_dev(bits), O.widen_bf16(bits)
    return torch.from_numpy(v).to(DEV), v.astype(np.float64)


def _run(layer, x, dy, path, **kw):
    N, M, R = layer["N"], layer["M"], layer["R"]
    terms = device_terms(layer)
    tts = [D.dbf_term_t(t, N, M, R) for t in terms]
    out = D.dbf_linear_backward(terms, tts, N, M, R, x_dev(x), dy, path=path, **kw)
    torch.cuda.synchronize()
    return out


def _check(layer, x, dy_np, got):
    dx, scales = got
    rdx, rda, rdb, rdg = O.default().backward(O.terms64(layer), x64(x), dy_np)
    if dx is not None:
        assert_close(to_np(dx), rdx, what="dx")
    if scales is not None:
        for i, (da, db, dg) in enumerate(scales):
            assert_close(to_np(da), rda[i], what="dalpha %d" % i)
            assert_close(to_np(db), rdb[i], what="dbeta %d" % i)
            assert_close(to_np(dg), rdg[i], what="dgamma %d" % i)


ODD = [(1, 1, 1, 1, 1), (65, 33, 17, 2, 3), (130, 300, 70, 3, 5), (300, 129, 257, 1, 40),
       (77, 1000, 96, 2, 130), (40, 4100, 130, 1, 33)]


@pytest.mark.parametrize("N,M,R,L,T", ODD)
@pytest.mark.parametrize("path", [DEC, MF])
def test_backward_odd_shapes(N, M, R, L, T, path):
    print("backward odd", N, M, R, L, T, path, flush=True)
    layer, x = S.make_custom(N, M, R, L, T, seed=N + M + R)
    dy, dy_np = _dy(T, N, seed=N)
    _check(layer, x, dy_np, _run(layer, x, dy, path))


@pytest.mark.parametrize("config,T,path", [(2, 4, AUTO), (2, 64, AUTO), (4, 8, DEC), (4, 8, MF)])
def test_backward_configs(config, T, path):
    print("backward config", config, T, path, flush=True)
    layer = S.make_layer(config)
    x = S.make_x(config, T)
    dy, dy_np = _dy(T, layer["N"], seed=config, kind="bf16")
    _check(layer, x, dy_np, _run(layer, x, dy, path))


@pytest.mark.parametrize("scale", [1e-4, 1e-7])
@pytest.mark.parametrize("path", [DEC, MF])
def test_backward_small_gradients(scale, path):
    # realistic gradient magnitudes: alpha . dy lies far below fp16's normal
    # range, where an unscaled fp16 operand would lose most of its bits; the
    # MFMA products' per-token power of two keeps them at full precision
    N, M, R, L, T = 300, 700, 130, 2, 48
    layer, x = S.make_custom(N, M, R, L, T, seed=59)
    v = np.random.default_rng([0xDBF, 107, T, N]).standard_normal((T, N)) * scale
    dy_np = v.astype(np.float32).astype(np.float64)
    dy = torch.from_numpy(dy_np.astype(np.float32)).to(DEV)
    _check(layer, x, dy_np, _run(layer, x, dy, path))


def test_backward_dtypes_optional_outputs_deterministic():
    N, M, R, L, T = 200, 700, 96, 2, 24
    layer, x = S.make_custom(N, M, R, L, T, seed=31, x_kind="f16")
    dy, dy_np = _dy(T, N, seed=31)
    rdx, _, _, _ = O.default().backward(O.terms64(layer), x64(x), dy_np)
    # bf16 dx
    dx, scales = _run(layer, x, dy, MF, dx_dtype=torch.bfloat16, want_scales=False)
    assert scales is None
    assert_close_bf16(to_np(dx), rdx)
    # scale gradients only, twice: bitwise equal
    a = _run(layer, x, dy, DEC, want_dx=False)
    b = _run(layer, x, dy, DEC, want_dx=False)
    assert a[0] is None
    for sa, sb in zip(a[1], b[1]):
        for u, v in zip(sa, sb):
            assert torch.equal(u, v)
    _check(layer, x, dy_np, a)
