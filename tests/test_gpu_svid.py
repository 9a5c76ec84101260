"""dbf_svid_extract (successive SVID of a real weight into boolean kernels,
on the GPU) against oracle.svid_extract (numpy, fp64 SVD).

The signs of the first kernel are those of W: bit-exact.  The scales come
from a leading singular pair found by fp32 power iteration instead of an
fp64 SVD, so they meet the float tolerance rather than bit equality; a
later kernel's signs are those of a residual that differs from the oracle's
by those roundings, so they may differ only where the oracle's residual is
near zero.  The residual norms the GPU reports are checked against its own
kernels recomputed in fp64, and against the oracle's."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import DEV, assert_close, to_np, x64, x_dev

pytestmark = pytest.mark.gpu


def weight(N, M, seed, kind):
    v = np.random.default_rng([0xDBF, 108, seed, N, M]).standard_normal((N, M)).astype(np.float32)
    v *= np.float32(0.02)
    if kind == "bf16":
        bits = S.f32_to_bf16_bits(v)
        return x_dev(bits), O.widen_bf16(bits)
    if kind == "f16":
        h = v.astype(np.float16)
        return torch.from_numpy(h).to(DEV), h.astype(np.float64)
    return torch.from_numpy(v).to(DEV), v.astype(np.float64)


def unpack_signs(k, N, M):
    o = O.default()
    return o.unpack(k.w.cpu().numpy().view(np.uint32), N, M)


def f16(t):
    return t.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("N,M,K,kind", [(300, 1000, 3, "bf16"), (1024, 768, 3, "f32"),
                                        (97, 4100, 2, "f16"), (2048, 2048, 2, "bf16")])
def test_against_oracle(N, M, K, kind):
    print("svid", N, M, K, kind, flush=True)
    w, w64 = weight(N, M, N + M, kind)
    ks, res = D.dbf_svid_extract(w, K, residual=True)
    torch.cuda.synchronize()
    ref = O.svid_extract(w64, K)
    r_ref = w64.copy()
    r_gpu = w64.copy()
    for i, (k, kr) in enumerate(zip(ks, ref)):
        signs = unpack_signs(k, N, M)
        if i == 0:
            assert np.array_equal(signs, kr["w"]), "first kernel: signs of W"
        else:
            # any disagreement sits where the oracle's residual is ~0
            diff = signs != kr["w"]
            assert diff.mean() <= 1e-3, diff.mean()
            assert np.all(np.abs(r_ref[diff]) <= 1e-3 * np.abs(r_ref).max())
        # the signs are those of the residual the GPU's own kernels leave (it
        # keeps it in fp32: a sign may differ only within a few fp32 steps of 0)
        off = signs != np.where(r_gpu >= 0, 1, -1)
        assert np.all(np.abs(r_gpu[off]) <= 1e-6 * np.abs(r_gpu).max())
        assert np.all(f16(k.s_in) >= 0) and np.all(f16(k.s_out) >= 0)
        assert_close(f16(k.s_in), kr["s_in"].astype(np.float64), what="s_in %d" % i)
        assert_close(f16(k.s_out), kr["s_out"].astype(np.float64), what="s_out %d" % i)
        r_ref = r_ref - kr["w"] * np.outer(kr["s_out"].astype(np.float64), kr["s_in"].astype(np.float64))
        r_gpu = r_gpu - signs * np.outer(f16(k.s_out), f16(k.s_in))
        got = float(res[i])
        assert np.isclose(got, np.sum(r_gpu ** 2), rtol=1e-4), (got, np.sum(r_gpu ** 2))
        assert np.isclose(got, np.sum(r_ref ** 2), rtol=1e-3), (got, np.sum(r_ref ** 2))
    # the kernels run as they are on the boolean-kernel forward
    x = S.f32_to_bf16_bits(np.random.default_rng(5).standard_normal((4, M)).astype(np.float32))
    y = D.dbf_bool_forward(ks, N, M, x_dev(x))
    torch.cuda.synchronize()
    refk = [dict(w=k["w"], s_in=k["s_in"].astype(np.float64), s_out=k["s_out"].astype(np.float64))
            for k in ref]
    assert_close(to_np(y), O.default().bool_forward(refk, x64(x)))


def test_rank_one_scaled_signs():
    # W = S . (a b^T) with a, b > 0: the first kernel is S and a b^T, up to
    # the fp16 rounding of the scales; the residual is that rounding
    g = np.random.default_rng(61)
    N, M = 200, 333
    Sg = (g.integers(0, 2, (N, M)) * 2 - 1).astype(np.int8)
    a, b = g.uniform(0.5, 2.0, N), g.uniform(0.5, 2.0, M)
    W = (Sg * np.outer(a, b)).astype(np.float32)
    ks = D.dbf_svid_extract(torch.from_numpy(W).to(DEV), 1)
    torch.cuda.synchronize()
    assert np.array_equal(unpack_signs(ks[0], N, M), Sg)
    rel = np.abs(np.outer(f16(ks[0].s_out), f16(ks[0].s_in)) / np.outer(a, b) - 1)
    assert rel.max() <= 2.0 ** -9


def test_deterministic_and_zero_matrix():
    w, _ = weight(500, 700, 3, "f32")
    a = D.dbf_svid_extract(w, 2)
    b = D.dbf_svid_extract(w, 2)
    torch.cuda.synchronize()
    for ka, kb in zip(a, b):
        for u, v in zip(ka, kb):
            assert torch.equal(u, v)
    z = torch.zeros((64, 96), dtype=torch.float32, device=DEV)
    ks, res = D.dbf_svid_extract(z, 2, residual=True)
    torch.cuda.synchronize()
    for k in ks:
        assert np.all(unpack_signs(k, 64, 96) == 1)  # sign(0) = +1
        assert not k.s_in.any() and not k.s_out.any()
    assert not res.any()
