"""Pins of the fp64 oracle against things other than itself.

None of the pages prints a worked numerical example, so every pin is
mathematics the parametrization fixes:

* brute force: Delta W materialised with numpy matrix products (a library
  primitive) from the LoRDBA parametrization (section 2, "Arquitetura
  Central") and applied to x; on small-integer data both sides are exact and
  must agree bit for bit;
* the DBF page's own Hadamard form (technical summary, section 2),
  (a . A . m^T)(B . b^T), evaluated with broadcasting;
* closed forms: all-ones signs, rank 1;
* invariants: flipping a row of B1 negates exactly that output, the gauge
  flip (row r of B2 with column r of B1) and the column flip (column m of B2
  against -x_m) change nothing, a consistent permutation of the inner index,
  power-of-two homogeneity, additivity over terms;
* the integer path against Python big integers;
* the dense base against numpy;
* the bit layout against hand-derived fixtures (tests/golden/) and
  counting invariants.

``test_mutants_are_caught`` plants plausible mistakes in a copy of the
oracle's C source, on the CPU, and checks that some pin fails for each.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_layer(N, M, R, L, seed, integer=False):
    g = np.random.default_rng([7, seed, N, M, R, L])
    terms = []
    for _ in range(L):
        b1 = (g.integers(0, 2, (N, R)) * 2 - 1).astype(np.int8)
        b2 = (g.integers(0, 2, (R, M)) * 2 - 1).astype(np.int8)
        if integer:
            a, b, c = (g.integers(1, 4, n).astype(np.float64) for n in (N, R, M))
        else:
            a = g.uniform(0.5, 1.5, N).astype(np.float16).astype(np.float64)
            b = g.uniform(0.5, 1.5, R).astype(np.float16).astype(np.float64)
            c = g.uniform(0.5, 1.5, M).astype(np.float16).astype(np.float64)
        terms.append(dict(b1=b1, b2=b2, alpha=a, beta=b, gamma=c))
    return terms


def _rand_x(T, M, seed, integer=False):
    g = np.random.default_rng([8, seed, T, M])
    if integer:
        return g.integers(-3, 4, (T, M)).astype(np.float64)
    return g.standard_normal((T, M))


def _dense_delta_w(terms):
    """Delta W = sum_i diag(alpha) B1 diag(beta) B2 diag(gamma), materialised
    with numpy matrix products."""
    dw = 0.0
    for t in terms:
        left = t["alpha"][:, None] * t["b1"].astype(np.float64)
        mid = t["beta"][:, None] * t["b2"].astype(np.float64)
        dw = dw + (left @ mid) * t["gamma"][None, :]
    return dw


SHAPES = [(1, 1, 1, 1), (2, 3, 5, 1), (8, 5, 3, 2), (33, 65, 32, 3),
          (64, 33, 65, 1), (5, 8, 2, 3)]


# --------------------------------------------------------------------------
# pins; each takes an Oracle and raises AssertionError on a mismatch
# --------------------------------------------------------------------------
def pin_bruteforce_real(o):
    for k, (N, M, R, L) in enumerate(SHAPES):
        terms = _rand_layer(N, M, R, L, k)
        x = _rand_x(3, M, k)
        y = o.forward(terms, x)
        ref = x @ _dense_delta_w(terms).T
        err = np.abs(y - ref).max() / max(np.abs(ref).max(), 1e-300)
        assert err <= 1e-12, (N, M, R, L, err)


def pin_bruteforce_exact(o):
    for k, (N, M, R, L) in enumerate(SHAPES):
        terms = _rand_layer(N, M, R, L, 100 + k, integer=True)
        x = _rand_x(2, M, 100 + k, integer=True)
        y = o.forward(terms, x)
        ref = x @ _dense_delta_w(terms).T
        assert np.array_equal(y, ref), (N, M, R, L)


def pin_dbf_hadamard_form(o):
    # DBF: W ~ (a . A . m^T)(B . b^T) with a = alpha, A = B1, m = beta,
    # B = B2, b = gamma; broadcasting products, one term.
    for k, (N, M, R, _) in enumerate(SHAPES):
        t = _rand_layer(N, M, R, 1, 200 + k)[0]
        a, A, m = t["alpha"], t["b1"].astype(np.float64), t["beta"]
        B, b = t["b2"].astype(np.float64), t["gamma"]
        W = (a[:, None] * A * m[None, :]) @ (B * b[None, :])
        x = _rand_x(2, M, 200 + k)
        y = o.forward([t], x)
        ref = x @ W.T
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def pin_all_ones(o):
    # B1 = B2 = 1:  y_n = sum_i alpha_n (sum_r beta_r) (sum_m gamma_m x_m)
    for integer in (True, False):
        terms = _rand_layer(7, 9, 4, 3, 300, integer=integer)
        for t in terms:
            t["b1"][:] = 1
            t["b2"][:] = 1
        x = _rand_x(2, 9, 300, integer=integer)
        y = o.forward(terms, x)
        ref = sum(t["alpha"][None, :] * t["beta"].sum()
                  * (x * t["gamma"][None, :]).sum(axis=1)[:, None]
                  for t in terms)
        if integer:
            assert np.array_equal(y, ref)
        else:
            assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)


def pin_rank_one(o):
    # R = 1: Delta W = (alpha . b1) beta (b2 . gamma)^T, an outer product
    terms = _rand_layer(6, 11, 1, 1, 400)
    t = terms[0]
    x = _rand_x(3, 11, 400)
    y = o.forward(terms, x)
    left = t["alpha"] * t["b1"][:, 0]
    right = t["b2"][0, :] * t["gamma"]
    ref = (x @ right)[:, None] * t["beta"][0] * left[None, :]
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


def pin_row_flip(o):
    # flipping row n0 of every B1 negates y[:, n0] exactly, nothing else moves
    terms = _rand_layer(9, 13, 5, 2, 500)
    x = _rand_x(2, 13, 500)
    y = o.forward(terms, x)
    n0 = 4
    for t in terms:
        t["b1"][n0, :] *= -1
    y2 = o.forward(terms, x)
    assert np.array_equal(y2[:, n0], -y[:, n0])
    rest = [n for n in range(9) if n != n0]
    assert np.array_equal(y2[:, rest], y[:, rest])


def pin_gauge(o):
    # flipping row r0 of B2 together with column r0 of B1 leaves y unchanged
    terms = _rand_layer(9, 13, 5, 2, 600)
    x = _rand_x(2, 13, 600)
    y = o.forward(terms, x)
    r0 = 2
    terms[1]["b2"][r0, :] *= -1
    terms[1]["b1"][:, r0] *= -1
    assert np.array_equal(o.forward(terms, x), y)


def pin_column_flip(o):
    # flipping column m0 of every B2 is the same as negating x[:, m0]
    terms = _rand_layer(9, 13, 5, 2, 700)
    x = _rand_x(2, 13, 700)
    m0 = 6
    x2 = x.copy()
    x2[:, m0] *= -1
    y = o.forward(terms, x2)
    for t in terms:
        t["b2"][:, m0] *= -1
    assert np.array_equal(o.forward(terms, x), y)


def pin_permutation(o):
    terms = _rand_layer(10, 12, 7, 2, 800)
    x = _rand_x(2, 12, 800)
    y = o.forward(terms, x)
    p = np.random.default_rng(1).permutation(7)
    for t in terms:
        t["b1"] = t["b1"][:, p].copy()
        t["b2"] = t["b2"][p, :].copy()
        t["beta"] = t["beta"][p].copy()
    y2 = o.forward(terms, x)
    assert np.allclose(y2, y, rtol=1e-13, atol=1e-13 * np.abs(y).max())


def pin_homogeneity(o):
    terms = _rand_layer(10, 12, 7, 2, 900)
    x = _rand_x(2, 12, 900)
    y = o.forward(terms, x)
    for t in terms:
        t["alpha"] = t["alpha"] * 2.0
        t["beta"] = t["beta"] * 4.0
        t["gamma"] = t["gamma"] * 0.5
    y2 = o.forward(terms, x * 8.0)
    assert np.array_equal(y2, y * 32.0)


def pin_additivity(o):
    terms = _rand_layer(10, 12, 7, 3, 1000)
    x = _rand_x(3, 12, 1000)
    y = o.forward(terms, x)
    parts = [o.forward([t], x) for t in terms]
    assert np.allclose(y, sum(parts), rtol=1e-14, atol=1e-14 * np.abs(y).max())
    # and each part is really there: dropping one term changes the result
    assert not np.allclose(o.forward(terms[:2], x), y)


def pin_int_bigint(o):
    for k, (N, M, R, L) in enumerate(SHAPES):
        terms = _rand_layer(N, M, R, L, 1100 + k)
        g = np.random.default_rng([9, k])
        xq = g.integers(-127, 128, (2, M)).astype(np.int8)
        s1, s2 = o.forward_int(terms, xq)
        for i, t in enumerate(terms):
            for tok in range(2):
                xs = [int(v) for v in xq[tok]]
                ref1 = [sum(int(t["b2"][r, m]) * xs[m] for m in range(M))
                        for r in range(R)]
                ref2 = [sum(int(t["b1"][n, r]) * ref1[r] for r in range(R))
                        for n in range(N)]
                assert list(s1[i, tok]) == ref1
                assert list(s2[i, tok]) == ref2


def pin_int_all_ones(o):
    terms = _rand_layer(5, 9, 3, 1, 1200)
    terms[0]["b1"][:] = 1
    terms[0]["b2"][:] = 1
    xq = np.random.default_rng(3).integers(-127, 128, (2, 9)).astype(np.int8)
    s1, s2 = o.forward_int(terms, xq)
    tot = xq.astype(np.int64).sum(axis=1)
    assert np.array_equal(s1[0], np.repeat(tot[:, None], 3, axis=1))
    assert np.array_equal(s2[0], np.repeat(3 * tot[:, None], 5, axis=1))


def pin_dense(o):
    g = np.random.default_rng(11)
    w0 = g.standard_normal((13, 17)) * 0.02
    x = g.standard_normal((3, 17))
    ref = x @ w0.T
    assert np.allclose(o.dense(w0, x), ref, rtol=1e-13, atol=1e-15)
    wi = g.integers(-5, 6, (13, 17)).astype(np.float64)
    xi = g.integers(-5, 6, (3, 17)).astype(np.float64)
    assert np.array_equal(o.dense(wi, xi), xi @ wi.T)


def _read_fixture(name):
    rows = K = None
    plus, plusrows, words = [], [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if not line:
                continue
            if line[0] == "shape":
                rows, K = int(line[1]), int(line[2])
            elif line[0] == "plus":
                plus.append((int(line[1]), int(line[2])))
            elif line[0] == "plusrow":
                plusrows.append(int(line[1]))
            elif line[0] == "word":
                words[int(line[1])] = int(line[2], 16)
    S = -np.ones((rows, K))
    for r, k in plus:
        S[r, k] = 1.0
    for r in plusrows:
        S[r, :] = 1.0
    return S, words


FIXTURES = ["pack_2x40.txt", "pack_65x130.txt", "pack_3x16.txt"]
FIXTURE_WORDS = {"pack_2x40.txt": 128, "pack_65x130.txt": 1024,
                 "pack_3x16.txt": 64}


def pin_pack_golden(o):
    for name in FIXTURES:
        S, words = _read_fixture(name)
        got = o.pack(S)
        assert got.size == FIXTURE_WORDS[name], name
        exp = np.zeros(got.size, dtype=np.uint32)
        for i, v in words.items():
            exp[i] = v
        assert np.array_equal(got, exp), name
        assert np.array_equal(o.unpack(exp, *S.shape), S.astype(np.int8)), name


def pin_pack_counts(o):
    g = np.random.default_rng(12)
    for rows, K in [(1, 1), (3, 31), (64, 32), (65, 33), (70, 97), (130, 300),
                    (16, 4096), (4096, 16)]:
        v = g.standard_normal((rows, K))
        w = o.pack(v)
        pop = int(np.unpackbits(w.view(np.uint8)).sum())
        assert pop == int((v >= 0).sum()), (rows, K)
        # all +1: exactly rows*K set bits, the padding stays 0
        assert int(np.unpackbits(o.pack(np.ones((rows, K))).view(np.uint8)).sum()) == rows * K
        assert np.array_equal(o.unpack(w, rows, K), np.where(v >= 0, 1, -1))
    # sign convention: 0 and -0.0 are +1, NaN and negatives are -1
    v = np.array([[0.0, -0.0, np.nan, -1e-300, 1e-300, -np.inf, np.inf]])
    assert np.array_equal(o.unpack(o.pack(v), 1, 7), [[1, 1, -1, -1, 1, -1, 1]])


def _rand_bool(N, M, K, seed, integer=False):
    g = np.random.default_rng([9, seed, N, M, K])
    ks = []
    for _ in range(K):
        w = (g.integers(0, 2, (N, M)) * 2 - 1).astype(np.int8)
        if integer:
            si = g.integers(1, 4, M).astype(np.float64)
            so = g.integers(1, 4, N).astype(np.float64)
        else:
            si = g.uniform(0.5, 1.5, M).astype(np.float16).astype(np.float64)
            so = g.uniform(0.5, 1.5, N).astype(np.float16).astype(np.float64)
        ks.append(dict(w=w, s_in=si, s_out=so))
    return ks


def _bool_dense(ks):
    # the Multi-Boolean weight, sum_k Wb_k . (s_out_k s_in_k^T), with numpy
    return sum(k["w"] * np.outer(k["s_out"], k["s_in"]) for k in ks)


def pin_bool_bruteforce(o):
    ks = _rand_bool(37, 53, 3, 1)
    x = _rand_x(4, 53, 1)
    ref = x @ _bool_dense(ks).T
    y = o.bool_forward(ks, x)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    # small integers: both sides are exact
    ks = _rand_bool(29, 41, 2, 2, integer=True)
    x = _rand_x(3, 41, 2, integer=True)
    assert np.array_equal(o.bool_forward(ks, x), x @ _bool_dense(ks).T)


def pin_bool_all_ones(o):
    # all signs +1: y[t, n] = sum_k s_out_k[n] (s_in_k . x[t])
    ks = _rand_bool(20, 30, 2, 3)
    for k in ks:
        k["w"][:] = 1
    x = _rand_x(2, 30, 3)
    ref = sum(np.outer(x @ k["s_in"], k["s_out"]) for k in ks)
    assert np.allclose(o.bool_forward(ks, x), ref, rtol=1e-12, atol=1e-12)


def pin_bool_row_flip(o):
    # flipping row 5 of one kernel's signs negates that kernel's output 5
    # and leaves every other output of the sum unchanged, exactly
    ks = _rand_bool(16, 24, 2, 4)
    x = _rand_x(3, 24, 4)
    flipped = [ks[0], dict(ks[1], w=ks[1]["w"].copy())]
    flipped[1]["w"][5] *= -1
    y, y1 = o.bool_forward(ks, x), o.bool_forward(flipped, x)
    rest = [n for n in range(16) if n != 5]
    assert np.array_equal(y1[:, rest], y[:, rest])
    assert np.array_equal(o.bool_forward(flipped[1:], x)[:, 5],
                          -o.bool_forward(ks[1:], x)[:, 5])


def pin_bool_additivity(o):
    ks = _rand_bool(18, 26, 3, 5, integer=True)
    x = _rand_x(2, 26, 5, integer=True)
    parts = sum(o.bool_forward([k], x) for k in ks)
    assert np.array_equal(o.bool_forward(ks, x), parts)


def pin_backward_adjoint(o):
    # the layer is linear in x: <dy, F x> = <dx, x> (exact on small integers)
    terms = _rand_layer(9, 11, 6, 2, 1400, integer=True)
    x = _rand_x(3, 11, 1400, integer=True)
    dy = _rand_x(3, 9, 1401, integer=True)
    dx, _, _, _ = o.backward(terms, x, dy)
    assert np.sum(dy * o.forward(terms, x)) == np.sum(dx * x)
    # and dx = dy Delta W with Delta W materialised by numpy products
    terms = _rand_layer(13, 17, 7, 2, 1402)
    x = _rand_x(2, 17, 1402)
    dy = _rand_x(2, 13, 1403)
    W = sum(np.diag(t["alpha"]) @ t["b1"] @ np.diag(t["beta"]) @ t["b2"] @ np.diag(t["gamma"])
            for t in terms)
    dx, _, _, _ = o.backward(terms, x, dy)
    assert np.max(np.abs(dx - dy @ W)) <= 1e-12 * np.max(np.abs(dy @ W))


def pin_backward_scale_steps(o):
    # the layer is linear in every single scale entry, so a unit step of
    # alpha_i[n] (beta_i[r], gamma_i[m]) changes <dy, y> by exactly that
    # entry's gradient; small integers keep both sides exact
    terms = _rand_layer(5, 7, 4, 2, 1410, integer=True)
    x = _rand_x(3, 7, 1410, integer=True)
    dy = _rand_x(3, 5, 1411, integer=True)
    _, da, db, dg = o.backward(terms, x, dy)
    base = np.sum(dy * o.forward(terms, x))
    for i in range(2):
        for key, grad in (("alpha", da), ("beta", db), ("gamma", dg)):
            for j in range(len(terms[i][key])):
                v = terms[i][key].copy()
                v[j] += 1.0
                stepped = list(terms)
                stepped[i] = dict(terms[i], **{key: v})
                assert np.sum(dy * o.forward(stepped, x)) - base == grad[i, j], (key, i, j)


PINS = [pin_bruteforce_real, pin_bruteforce_exact, pin_dbf_hadamard_form,
        pin_all_ones, pin_rank_one, pin_row_flip, pin_gauge, pin_column_flip,
        pin_permutation, pin_homogeneity, pin_additivity, pin_int_bigint,
        pin_int_all_ones, pin_dense, pin_pack_golden, pin_pack_counts,
        pin_bool_bruteforce, pin_bool_all_ones, pin_bool_row_flip, pin_bool_additivity,
        pin_backward_adjoint, pin_backward_scale_steps]


@pytest.fixture(scope="module")
def orc():
    return O.default()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_thread_count_does_not_change_result(orc):
    terms = _rand_layer(40, 70, 33, 2, 1300)
    x = _rand_x(3, 70, 1300)
    y = orc.forward(terms, x)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    code = ("import numpy as np, sys; sys.path.insert(0, %r); import oracle as O;"
            "d = np.load(sys.argv[1]); terms=[dict(b1=d['b1%%d'%%i], b2=d['b2%%d'%%i],"
            "alpha=d['a%%d'%%i], beta=d['b%%d'%%i], gamma=d['g%%d'%%i]) for i in range(2)];"
            "np.save(sys.argv[2], O.Oracle().forward(terms, d['x']))"
            % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    with tempfile.TemporaryDirectory() as td:
        arrs = {"x": x}
        for i, t in enumerate(terms):
            arrs.update({"b1%d" % i: t["b1"], "b2%d" % i: t["b2"],
                         "a%d" % i: t["alpha"], "b%d" % i: t["beta"],
                         "g%d" % i: t["gamma"]})
        np.savez(os.path.join(td, "in.npz"), **arrs)
        subprocess.run(["python", "-c", code, os.path.join(td, "in.npz"),
                        os.path.join(td, "out.npy")], check=True, env=env)
        y1 = np.load(os.path.join(td, "out.npy"))
    assert np.array_equal(y, y1)


# (description, original text, planted mistake)
MUTANTS = [
    ("gamma dropped", "u[m] = g[m] * xt[m];", "u[m] = xt[m];"),
    ("beta dropped", "v[r] = be[r] * s;", "v[r] = s;"),
    ("alpha dropped", "yt[n] += a[n] * s;", "yt[n] += s;"),
    ("stage-1 sign", "s += (row[m] > 0) ? u[m] : -u[m];",
     "s += (row[m] > 0) ? u[m] : u[m];"),
    ("stage-2 sign", "s += (row[r] > 0) ? v[r] : -v[r];",
     "s += (row[r] > 0) ? -v[r] : v[r];"),
    ("B2 read transposed", "s += (row[m] > 0) ? u[m] : -u[m];",
     "s += (b2[m * R + r] > 0) ? u[m] : -u[m];"),
    ("B1 read transposed", "s += (row[r] > 0) ? v[r] : -v[r];",
     "s += (b1[r * N + n] > 0) ? v[r] : -v[r];"),
    ("terms overwrite", "yt[n] += a[n] * s;", "yt[n] = a[n] * s;"),
    ("last term dropped", "for (i = 0; i < L; ++i)", "for (i = 0; i + 1 < L; ++i)"),
    ("dense index", "s += row[m] * xt[m];", "s += row[m] * xt[M - 1 - m];"),
    ("int sign ignored", "s += (row[m] > 0) ? (int64_t)xt[m] : -(int64_t)xt[m];",
     "s += (int64_t)xt[m];"),
    ("int stage-2 transposed", "s += (row[q] > 0) ? o1[q] : -o1[q];",
     "s += (b1[i][q * N + n] > 0) ? o1[q] : -o1[q];"),
    ("bit order reversed", "|= (uint32_t)1u << (k % 32);",
     "|= (uint32_t)1u << (31 - k % 32);"),
    ("sign of zero", "if (v[r * K + k] >= 0.0)", "if (v[r * K + k] > 0.0)"),
    ("tile column-major", "return tile * 64 * kw + (r % 64) * kw + w;",
     "return tile * 64 * kw + w * 64 + (r % 64);"),
    ("unpack inverted", "& 1u) ? 1 : -1;", "& 1u) ? -1 : 1;"),
    ("bool s_in dropped", "xs[m] = s_in[k][m] * x[t * M + m];", "xs[m] = x[t * M + m];"),
    ("bool s_out dropped", "yt[o] += s_out[k][o] * acc;", "yt[o] += acc;"),
    ("bool sign", "acc += (wrow[q] > 0) ? xs[q] : -xs[q];",
     "acc += (wrow[q] > 0) ? xs[q] : xs[q];"),
    ("bool read transposed", "acc += (wrow[q] > 0) ? xs[q] : -xs[q];",
     "acc += (wb[k][q * N + o] > 0) ? xs[q] : -xs[q];"),
    ("bool kernels overwrite", "yt[o] += s_out[k][o] * acc;", "yt[o] = s_out[k][o] * acc;"),
    ("bool last kernel dropped", "for (k = 0; k < K; ++k)", "for (k = 0; k + 1 < K; ++k)"),
    ("bwd alpha dropped", "acc += (B1[n * R + r] > 0) ? al[n] * dyt[n] : -(al[n] * dyt[n]);",
     "acc += (B1[n * R + r] > 0) ? dyt[n] : -dyt[n];"),
    ("bwd B1 read untransposed", "acc += (B1[n * R + r] > 0) ? al[n] * dyt[n] : -(al[n] * dyt[n]);",
     "acc += (B1[r * N + n] > 0) ? al[n] * dyt[n] : -(al[n] * dyt[n]);"),
    ("bwd beta dropped", "acc += (B2[r * M + m] > 0) ? be[r] * g[r] : -(be[r] * g[r]);",
     "acc += (B2[r * M + m] > 0) ? g[r] : -g[r];"),
    ("bwd dgamma with gamma", "dgamma[(int64_t)i * M + m] += xt[m] * h[m];",
     "dgamma[(int64_t)i * M + m] += ga[m] * h[m];"),
    ("bwd dx without gamma", "dx[t * M + m] += ga[m] * h[m];", "dx[t * M + m] += h[m];"),
    ("bwd dbeta with beta", "dbeta[(int64_t)i * R + r] += sv[r] * g[r];",
     "dbeta[(int64_t)i * R + r] += be[r] * sv[r] * g[r];"),
    ("bwd dalpha with alpha", "dalpha[(int64_t)i * N + n] += dyt[n] * z[n];",
     "dalpha[(int64_t)i * N + n] += dyt[n] * al[n] * z[n];"),
]


def test_mutants_are_caught():
    src = open(O.SOURCE).read()
    with tempfile.TemporaryDirectory() as td:
        for desc, old, new in MUTANTS:
            assert src.count(old) >= 1, desc
            msrc = os.path.join(td, "m.c")
            with open(msrc, "w") as f:
                f.write(src.replace(old, new))
            lib = os.path.join(td, "m_%d.so" % MUTANTS.index((desc, old, new)))
            O.build(msrc, lib)
            mo = O.Oracle(lib)
            failed = []
            for pin in PINS:
                try:
                    pin(mo)
                except AssertionError:
                    failed.append(pin.__name__)
            assert failed, "planted mistake not caught: " + desc
    assert shutil.which("gcc")


# -- successive SVID (Multi-Boolean page, technical summary, section 2) ----
def test_svid_recovers_rank_one_scaled_signs():
    # W = S . (a b^T) with a, b > 0: one kernel recovers S and a b^T
    g = np.random.default_rng(41)
    S = (g.integers(0, 2, (24, 40)) * 2 - 1).astype(np.int8)
    a, b = g.uniform(0.5, 2.0, 24), g.uniform(0.5, 2.0, 40)
    W = S * np.outer(a, b)
    k = O.svid_extract(W, 1, round_fp16=False)[0]
    assert np.array_equal(k["w"], S)
    assert np.allclose(np.outer(k["s_out"], k["s_in"]), np.outer(a, b), rtol=1e-12)
    # the fp16 storage of the scales costs at most their rounding
    k = O.svid_extract(W, 1)[0]
    assert k["s_in"].dtype == np.float16 and k["s_out"].dtype == np.float16
    assert np.array_equal(k["w"], S)
    rel = np.abs(np.outer(k["s_out"].astype(np.float64), k["s_in"].astype(np.float64))
                 / np.outer(a, b) - 1)
    assert rel.max() <= 2.0 ** -10


def test_svid_residual_is_the_eckart_young_tail():
    # |W - Wb . P| = ||W| - P| elementwise (|Wb| = 1), and the best rank-one
    # P leaves the sum of the other squared singular values of |W|
    g = np.random.default_rng(42)
    W = g.standard_normal((30, 50))
    k = O.svid_extract(W, 1, round_fp16=False)[0]
    assert np.array_equal(k["w"], np.where(W >= 0, 1, -1))
    res = W - k["w"] * np.outer(k["s_out"], k["s_in"])
    sv = np.linalg.svd(np.abs(W), compute_uv=False)
    assert np.isclose(np.sum(res ** 2), np.sum(sv[1:] ** 2), rtol=1e-10)
    # the even split: s_out and s_in carry the same norm
    assert np.isclose(np.linalg.norm(k["s_out"]), np.linalg.norm(k["s_in"]), rtol=1e-12)


def test_svid_successive_kernels():
    g = np.random.default_rng(43)
    W = g.standard_normal((40, 64)) * 0.02
    ks = O.svid_extract(W, 4)
    r = W.copy()
    x = g.standard_normal((3, 64))
    o = O.default()
    prev_err = np.linalg.norm(x @ W.T)
    for i, k in enumerate(ks):
        # each kernel takes the signs of what the earlier ones left
        assert np.array_equal(k["w"], np.where(r >= 0, 1, -1))
        assert np.all(k["s_in"] >= 0) and np.all(k["s_out"] >= 0)
        nxt = r - k["w"] * np.outer(k["s_out"].astype(np.float64), k["s_in"].astype(np.float64))
        assert np.linalg.norm(nxt) < np.linalg.norm(r)
        r = nxt
        # and the forward of the first i + 1 kernels approaches W x
        err = np.linalg.norm(o.bool_forward(ks[:i + 1], x) - x @ W.T)
        assert err < prev_err
        prev_err = err


def test_transpose_packed_round_trip():
    o = O.default()
    for rows, K in [(1, 1), (3, 70), (64, 128), (130, 33), (200, 513)]:
        v = np.random.default_rng([44, rows, K]).standard_normal((rows, K))
        w = o.pack(v)
        wt = o.transpose_packed(w, rows, K)
        assert np.array_equal(o.unpack(wt, K, rows), np.where(v >= 0, 1, -1).T)
        assert np.array_equal(o.transpose_packed(wt, K, rows), w)
