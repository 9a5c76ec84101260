"""fp64 CPU oracle of the double-binary factorized linear layer.

TEST INFRASTRUCTURE ONLY.  Tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it; the library in ``bit_adapters_amd``
never imports, links or runs anything here, and nothing here imports the
library.  Inputs come from ``bit_adapters_amd.synth`` (random draws only).

The arithmetic lives in ``dbf_oracle.c`` (plain C, fp64, fixed summation
order); this module only widens the stored types to fp64 and calls it:

* ``forward``   -- y = sum_i diag(alpha_i) B1_i diag(beta_i) B2_i diag(gamma_i) x,
  the parametrization of Delta W on the LoRDBA page (section 2, "Arquitetura
  Central"), which is the DBF approximation (DBF technical summary,
  section 2) for one term and the multi-kernel sum of the Multi-Boolean page
  (technical summary, section 2, item 2) for several terms;
* ``dense``     -- the frozen base W0 x of LoRDBA's unmerged adapter mode
  (LoRDBA sections 1 and 5);
* ``forward_int`` -- exact integer sign sums for int8 activations;
* ``backward`` -- the chain rule through the layer: dx and the gradients of
  the three scale vectors of every term;
* ``bool_forward`` -- the Multi-Boolean form itself (technical summary,
  section 2, items 1 and 2): y = sum_k s_out_k . (Wb_k (s_in_k . x)), each
  kernel a full N x M sign matrix with a rank-one scale;
* ``svid_extract`` -- successive SVID of a real matrix into such kernels
  (same section, items 1 and 3), in numpy;
* ``pack`` / ``unpack`` -- the uint32 bit layout written out from its
  definition, one bit at a time.

Every function is pinned by tests/test_oracle_pins.py against closed forms,
invariants and brute force; the pack layout is additionally pinned by a
hand-derived fixture under tests/golden/.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "dbf_oracle.c")
LIBRARY = os.path.join(_HERE, "libdbf_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_i8p = ctypes.POINTER(ctypes.c_int8)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i64 = ctypes.c_int64


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (no fast-math, OpenMP for the outer
    loops)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", source, "-o", output + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


class Oracle:
    """A loaded oracle library (the default one, or a variant built from
    another source file, which the mutation tests use)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build(SOURCE, path)
        lib = ctypes.CDLL(path)
        lib.dbf_oracle_forward.restype = ctypes.c_int
        lib.dbf_oracle_forward.argtypes = [
            ctypes.c_int, _i64, _i64, _i64, _i64,
            ctypes.POINTER(_i8p), ctypes.POINTER(_i8p),
            ctypes.POINTER(_dp), ctypes.POINTER(_dp), ctypes.POINTER(_dp),
            _dp, _dp]
        lib.dbf_oracle_dense.restype = None
        lib.dbf_oracle_dense.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp]
        lib.dbf_oracle_forward_int.restype = None
        lib.dbf_oracle_forward_int.argtypes = [
            ctypes.c_int, _i64, _i64, _i64, _i64,
            ctypes.POINTER(_i8p), ctypes.POINTER(_i8p), _i8p, _i64p, _i64p]
        lib.dbf_oracle_packed_words.restype = _i64
        lib.dbf_oracle_packed_words.argtypes = [_i64, _i64]
        lib.dbf_oracle_pack.restype = None
        lib.dbf_oracle_pack.argtypes = [_dp, _i64, _i64, _u32p]
        lib.dbf_oracle_unpack.restype = None
        lib.dbf_oracle_unpack.argtypes = [_u32p, _i64, _i64, _i8p]
        lib.dbf_oracle_bool_forward.restype = ctypes.c_int
        lib.dbf_oracle_bool_forward.argtypes = [
            ctypes.c_int, _i64, _i64, _i64, ctypes.POINTER(_i8p),
            ctypes.POINTER(_dp), ctypes.POINTER(_dp), _dp, _dp]
        lib.dbf_oracle_backward.restype = ctypes.c_int
        lib.dbf_oracle_backward.argtypes = [
            ctypes.c_int, _i64, _i64, _i64, _i64,
            ctypes.POINTER(_i8p), ctypes.POINTER(_i8p),
            ctypes.POINTER(_dp), ctypes.POINTER(_dp), ctypes.POINTER(_dp),
            _dp, _dp, _dp, _dp, _dp, _dp]
        lib.dbf_oracle_threads.restype = ctypes.c_int
        lib.dbf_oracle_set_threads.restype = None
        lib.dbf_oracle_set_threads.argtypes = [ctypes.c_int]
        self.lib = lib
        self.path = path

    # -- the layer -------------------------------------------------------
    def forward(self, terms, x) -> np.ndarray:
        """y [T x N] in fp64 for fp64 activations x [T x M] and a list of
        terms (dicts with int8 b1 [N x R], b2 [R x M] and alpha, beta, gamma
        convertible to fp64)."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        T, M = x.shape
        L = len(terms)
        N, R = terms[0]["b1"].shape
        keep = []

        def arr(a, dt):
            a = np.ascontiguousarray(a, dtype=dt)
            keep.append(a)
            return a

        b1 = [arr(t["b1"], np.int8) for t in terms]
        b2 = [arr(t["b2"], np.int8) for t in terms]
        for t in terms:
            assert t["b1"].shape == (N, R) and t["b2"].shape == (R, M)
        al = [arr(t["alpha"], np.float64) for t in terms]
        be = [arr(t["beta"], np.float64) for t in terms]
        ga = [arr(t["gamma"], np.float64) for t in terms]
        y = np.empty((T, N), dtype=np.float64)
        P8 = (_i8p * L)(*[a.ctypes.data_as(_i8p) for a in b1])
        Q8 = (_i8p * L)(*[a.ctypes.data_as(_i8p) for a in b2])
        A = (_dp * L)(*[a.ctypes.data_as(_dp) for a in al])
        B = (_dp * L)(*[a.ctypes.data_as(_dp) for a in be])
        G = (_dp * L)(*[a.ctypes.data_as(_dp) for a in ga])
        rc = self.lib.dbf_oracle_forward(L, N, M, R, T, P8, Q8, A, B, G,
                                         x.ctypes.data_as(_dp),
                                         y.ctypes.data_as(_dp))
        if rc != 0:
            raise MemoryError("oracle scratch allocation failed")
        return y

    def backward(self, terms, x, dy):
        """Gradients of a loss with dL/dy = dy [T x N] through the layer:
        (dx [T x M], dalpha [L x N], dbeta [L x R], dgamma [L x M]), fp64."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        dy = np.ascontiguousarray(dy, dtype=np.float64)
        T, M = x.shape
        L = len(terms)
        N, R = terms[0]["b1"].shape
        assert dy.shape == (T, N)
        keep = []

        def arr(a, dt):
            a = np.ascontiguousarray(a, dtype=dt)
            keep.append(a)
            return a

        b1 = [arr(t["b1"], np.int8) for t in terms]
        b2 = [arr(t["b2"], np.int8) for t in terms]
        al = [arr(t["alpha"], np.float64) for t in terms]
        be = [arr(t["beta"], np.float64) for t in terms]
        ga = [arr(t["gamma"], np.float64) for t in terms]
        dx = np.empty((T, M)); da = np.empty((L, N)); db = np.empty((L, R)); dg = np.empty((L, M))
        P8 = (_i8p * L)(*[a.ctypes.data_as(_i8p) for a in b1])
        Q8 = (_i8p * L)(*[a.ctypes.data_as(_i8p) for a in b2])
        A = (_dp * L)(*[a.ctypes.data_as(_dp) for a in al])
        B = (_dp * L)(*[a.ctypes.data_as(_dp) for a in be])
        G = (_dp * L)(*[a.ctypes.data_as(_dp) for a in ga])
        rc = self.lib.dbf_oracle_backward(
            L, N, M, R, T, P8, Q8, A, B, G, x.ctypes.data_as(_dp), dy.ctypes.data_as(_dp),
            dx.ctypes.data_as(_dp), da.ctypes.data_as(_dp), db.ctypes.data_as(_dp),
            dg.ctypes.data_as(_dp))
        if rc != 0:
            raise MemoryError("oracle scratch allocation failed")
        return dx, da, db, dg

    def transpose_packed(self, words, rows: int, K: int) -> np.ndarray:
        """The packed layout of S^T for the packed S (rows x K)."""
        return self.pack(self.unpack(words, rows, K).T.astype(np.float64))

    def multi_adapter(self, w0, adapters, idx, x) -> np.ndarray:
        """Several adapters beside one base: y[t] = W0 x[t] + Delta W_a x[t]
        with a = idx[t] (-1: the base alone), from dense and forward."""
        y = self.dense(w0, x)
        idx = np.asarray(idx)
        for a in sorted(set(int(v) for v in idx if v >= 0)):
            rows = np.nonzero(idx == a)[0]
            y[rows] += self.forward([adapters[a]], x[rows])
        return y

    def dense(self, w0, x) -> np.ndarray:
        """W0 x for every token: [T x N] fp64."""
        w0 = np.ascontiguousarray(w0, dtype=np.float64)
        x = np.ascontiguousarray(x, dtype=np.float64)
        N, M = w0.shape
        T = x.shape[0]
        y = np.zeros((T, N), dtype=np.float64)
        self.lib.dbf_oracle_dense(N, M, T, w0.ctypes.data_as(_dp),
                                  x.ctypes.data_as(_dp), y.ctypes.data_as(_dp))
        return y

    def adapter(self, w0, terms, x) -> np.ndarray:
        """Unmerged adapter mode: Delta W x first, then W0 x added."""
        y = self.forward(terms, x) if terms else np.zeros(
            (x.shape[0], w0.shape[0]))
        return y + self.dense(w0, x)

    def forward_int(self, terms, xq):
        """Exact int64 sign sums (s1 [L x T x R], s2 [L x T x N]) for int8
        activations."""
        xq = np.ascontiguousarray(xq, dtype=np.int8)
        T, M = xq.shape
        L = len(terms)
        N, R = terms[0]["b1"].shape
        b1 = [np.ascontiguousarray(t["b1"], dtype=np.int8) for t in terms]
        b2 = [np.ascontiguousarray(t["b2"], dtype=np.int8) for t in terms]
        s1 = np.empty((L, T, R), dtype=np.int64)
        s2 = np.empty((L, T, N), dtype=np.int64)
        P8 = (_i8p * L)(*[a.ctypes.data_as(_i8p) for a in b1])
        Q8 = (_i8p * L)(*[a.ctypes.data_as(_i8p) for a in b2])
        self.lib.dbf_oracle_forward_int(L, N, M, R, T, P8, Q8,
                                        xq.ctypes.data_as(_i8p),
                                        s1.ctypes.data_as(_i64p),
                                        s2.ctypes.data_as(_i64p))
        return s1, s2

    def bool_forward(self, kernels, x) -> np.ndarray:
        """y [T x N] in fp64 for fp64 activations x [T x M] and a list of
        boolean kernels (dicts with int8 w [N x M] and s_in [M], s_out [N]
        convertible to fp64)."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        T, M = x.shape
        K = len(kernels)
        N = kernels[0]["w"].shape[0]
        w = [np.ascontiguousarray(k["w"], dtype=np.int8) for k in kernels]
        si = [np.ascontiguousarray(k["s_in"], dtype=np.float64) for k in kernels]
        so = [np.ascontiguousarray(k["s_out"], dtype=np.float64) for k in kernels]
        for a, b, c in zip(w, si, so):
            assert a.shape == (N, M) and b.shape == (M,) and c.shape == (N,)
        y = np.empty((T, N), dtype=np.float64)
        W = (_i8p * K)(*[a.ctypes.data_as(_i8p) for a in w])
        SI = (_dp * K)(*[a.ctypes.data_as(_dp) for a in si])
        SO = (_dp * K)(*[a.ctypes.data_as(_dp) for a in so])
        rc = self.lib.dbf_oracle_bool_forward(K, N, M, T, W, SI, SO,
                                              x.ctypes.data_as(_dp),
                                              y.ctypes.data_as(_dp))
        if rc != 0:
            raise MemoryError("oracle scratch allocation failed")
        return y

    # -- the bit layout -------------------------------------------------
    def packed_words(self, rows: int, K: int) -> int:
        return int(self.lib.dbf_oracle_packed_words(rows, K))

    def pack(self, values) -> np.ndarray:
        """uint32 words of the sign layout; bit = (value >= 0)."""
        v = np.ascontiguousarray(values, dtype=np.float64)
        rows, K = v.shape
        out = np.empty(self.packed_words(rows, K), dtype=np.uint32)
        self.lib.dbf_oracle_pack(v.ctypes.data_as(_dp), rows, K,
                                 out.ctypes.data_as(_u32p))
        return out

    def unpack(self, words, rows: int, K: int) -> np.ndarray:
        w = np.ascontiguousarray(words, dtype=np.uint32)
        assert w.size == self.packed_words(rows, K)
        s = np.empty((rows, K), dtype=np.int8)
        self.lib.dbf_oracle_unpack(w.ctypes.data_as(_u32p), rows, K,
                                   s.ctypes.data_as(_i8p))
        return s

    def threads(self) -> int:
        return int(self.lib.dbf_oracle_threads())

    def set_threads(self, n: int) -> None:
        """Threads of the parallel loops from now on (results do not depend
        on it)."""
        self.lib.dbf_oracle_set_threads(int(n))


# -- successive SVID (numpy) ---------------------------------------------
def svid_extract(w, n_kernels: int, round_fp16: bool = True) -> list:
    """Successive sign-value-independent decomposition of a real N x M
    matrix into boolean kernels, as the Multi-Boolean page describes it
    (technical summary, section 2): item 1, Wb = sign(W) and a rank-one fit
    W ~ Wb . (s_out s_in^T); item 3, each later kernel is extracted the same
    way from the residual the earlier ones leave.

    Readings where the page is silent: sign(0) is +1 (the bit rule of the
    packed layout); the rank-one fit of |W| is its leading singular pair
    (sigma, u, v), taken with the nonnegative sign (|W| is nonnegative, so
    such a pair exists) and split evenly, s_out = sqrt(sigma) u and
    s_in = sqrt(sigma) v; the scales are rounded to fp16 (their storage
    type) before the residual is formed, so later kernels absorb that
    rounding.  Returns [dict(w=int8 [N x M], s_in=fp16 [M], s_out=fp16 [N])].
    """
    r = np.array(w, dtype=np.float64)
    out = []
    for _ in range(n_kernels):
        wb = np.where(r >= 0, 1, -1).astype(np.int8)
        u, sv, vt = np.linalg.svd(np.abs(r), full_matrices=False)
        lu, lv = u[:, 0], vt[0]
        if lu.sum() + lv.sum() < 0:
            lu, lv = -lu, -lv
        s_out = np.sqrt(sv[0]) * lu
        s_in = np.sqrt(sv[0]) * lv
        if round_fp16:
            s_out = s_out.astype(np.float16)
            s_in = s_in.astype(np.float16)
        r = r - wb * np.outer(np.asarray(s_out, np.float64), np.asarray(s_in, np.float64))
        out.append(dict(w=wb, s_in=s_in, s_out=s_out))
    return out


# -- widening of the stored types to fp64 (exact) ------------------------
def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) to fp64: a bf16 value is the upper half of
    the fp32 with the same bits."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def widen(a, kind: str) -> np.ndarray:
    """Stored activations or weights to fp64: kind is 'bf16' (uint16 bit
    patterns), 'f16', 'f32' or 'i8'."""
    if kind == "bf16":
        return widen_bf16(a)
    return np.asarray(a).astype(np.float64)


def terms64(layer) -> list:
    """The layer's terms with the fp16 scales widened to fp64 (exact)."""
    return [dict(b1=t["b1"], b2=t["b2"],
                 alpha=np.asarray(t["alpha"], dtype=np.float64),
                 beta=np.asarray(t["beta"], dtype=np.float64),
                 gamma=np.asarray(t["gamma"], dtype=np.float64))
            for t in layer["terms"]]


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
