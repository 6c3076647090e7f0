"""Pins for the CPU oracle: hand-worked fixtures, brute force, invariants.

None of these checks calls the HIP library.  Each pins an oracle function to
something other than itself: values worked out by hand (tests/golden/),
scalar-loop brute force written from the definitions, closed forms, and the
invariants the method guarantees (a superset of the firing set reproduces the
dense layer; partial results over a partition of the active set add up to the
result over the whole set; compaction lists exactly the marked positions).
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.reference import Q4_0Matrix

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


# ---------------------------------------------------------------------------
# Scalar brute force, one neuron and one output at a time.
# ---------------------------------------------------------------------------

def _dot(row, x):
    s = 0.0
    for a, b in zip(row, x):
        s += float(a) * float(b)
    return s


def _bf_neuron(x, i, act, w_up, b_up, w_gate, b_gate):
    if act in ("relu", "relu2"):
        z = _dot(w_up[i], x) + (float(b_up[i]) if b_up is not None else 0.0)
        h = z if z > 0 else 0.0
        if act == "relu2":
            h = h * h
        return h, z > 0
    g = _dot(w_gate[i], x) + (float(b_gate[i]) if b_gate is not None else 0.0)
    u = _dot(w_up[i], x)
    return (g if g > 0 else 0.0) * u, g > 0


def _bf_ffn(xs, neurons, act, w_up, w_down_t, b_up=None, w_gate=None, b_gate=None):
    d = len(w_down_t[0])
    ys = []
    for x in xs:
        y = [0.0] * d
        for i in neurons:
            h, _ = _bf_neuron(x, i, act, w_up, b_up, w_gate, b_gate)
            for j in range(d):
                y[j] += float(w_down_t[i][j]) * h
        ys.append(y)
    return np.array(ys)


def _random_ffn(rng, d, f, act, dtype=np.float64):
    w_up = rng.standard_normal((f, d)).astype(dtype)
    w_dt = rng.standard_normal((f, d)).astype(dtype)
    b = (0.5 * rng.standard_normal(f)).astype(np.float32)
    w_gate = rng.standard_normal((f, d)).astype(dtype) if act == "reglu" else None
    kw = dict(b_up=None if act == "reglu" else b, w_gate=w_gate, b_gate=b if act == "reglu" else None)
    return w_up, w_dt, kw


# ---------------------------------------------------------------------------
# Hand-worked example around the pages' predicted set {3, 4, 5}
# ---------------------------------------------------------------------------

class TestWorkedExample:
    g = _gold("worked_example_345.json")

    def _relu(self):
        r = self.g["relu"]
        return np.array(r["w_up"], float), np.array(self.g["w_down_t"], float), np.array(r["b_up"], float)

    def test_dense_relu(self):
        w_up, w_dt, b = self._relu()
        y, fired = oracle.dense_ffn(np.array(self.g["x"], float), w_up, w_dt, "relu", b_up=b)
        assert np.array_equal(y, np.array(self.g["relu"]["y_dense"], float))
        for t, expect in enumerate(self.g["relu"]["fired"]):
            assert list(np.flatnonzero(fired[t])) == expect

    def test_dense_relu2(self):
        w_up, w_dt, b = self._relu()
        y, _ = oracle.dense_ffn(np.array(self.g["x"], float), w_up, w_dt, "relu2", b_up=b)
        assert np.array_equal(y, np.array(self.g["relu2"]["y_dense"], float))

    def test_dense_reglu(self):
        r = self.g["reglu"]
        y, fired = oracle.dense_ffn(np.array(self.g["x"], float), np.array(r["w_up"], float),
                                    np.array(self.g["w_down_t"], float), "reglu",
                                    w_gate=np.array(r["w_gate"], float), b_gate=np.array(r["b_gate"], float))
        assert np.array_equal(y, np.array(r["y_dense"], float))
        for t, expect in enumerate(r["fired"]):
            assert list(np.flatnonzero(fired[t])) == expect

    def test_partition_superset_single(self):
        w_up, w_dt, b = self._relu()
        x0 = np.array(self.g["x"][0], float)
        part = self.g["relu"]["partition_token0"]
        ya = oracle.sparse_ffn(x0, part["set_a"], w_up, w_dt, "relu", b_up=b)
        yb = oracle.sparse_ffn(x0, part["set_b"], w_up, w_dt, "relu", b_up=b)
        assert np.array_equal(ya[0], part["y_a"])
        assert np.array_equal(yb[0], part["y_b"])
        yall = oracle.sparse_ffn(x0, [3, 4, 5], w_up, w_dt, "relu", b_up=b)
        assert np.array_equal(ya + yb, yall)
        assert np.array_equal(yall[0], self.g["relu"]["y_dense"][0])
        sup = self.g["relu"]["superset_token0"]
        assert np.array_equal(oracle.sparse_ffn(x0, sup["set"], w_up, w_dt, "relu", b_up=b)[0], sup["y"])
        assert np.array_equal(oracle.sparse_ffn(x0, [3], w_up, w_dt, "relu", b_up=b)[0],
                              self.g["relu"]["single_3_token0"])

    @pytest.mark.parametrize("tau", ["0.5", "0.75", "0.25"])
    def test_predictor(self, tau):
        p = self.g["predictor"]
        logits, mask = oracle.predict(np.array(self.g["x"], float), np.array(p["p1"], float),
                                      np.array(p["p2"], float), np.array(p["c"], float), float(tau))
        assert np.array_equal(logits, np.array(p["logits"], float))
        for t, expect in enumerate(p["masks"][tau]):
            assert list(np.flatnonzero(mask[t])) == expect

    def test_layer(self):
        p = self.g["predictor"]
        w_up, w_dt, b = self._relu()
        out = oracle.layer(np.array(self.g["x"], float), np.array(p["p1"], float), np.array(p["p2"], float),
                           np.array(p["c"], float), 0.5, w_up, w_dt, "relu", b_up=b)
        ref = self.g["layer_relu_tau_0.5_both_tokens"]
        assert list(out["idx"]) == ref["idx"] and out["count"] == len(ref["idx"])
        assert np.array_equal(out["y"], np.array(ref["y"], float))
        out = oracle.layer(np.array(self.g["x"][0], float), np.array(p["p1"], float), np.array(p["p2"], float),
                           np.array(p["c"], float), 0.75, w_up, w_dt, "relu", b_up=b)
        ref = self.g["layer_relu_tau_0.75_token0"]
        assert list(out["idx"]) == ref["idx"]
        assert np.array_equal(out["y"], np.array(ref["y"], float))


# ---------------------------------------------------------------------------
# Q4_0 blocks written by hand
# ---------------------------------------------------------------------------

class TestQ4_0:
    g = _gold("q4_0_blocks.json")

    def _block(self, name):
        return np.frombuffer(bytes.fromhex(self.g["blocks"][name]["hex"]), dtype=np.uint8)

    @pytest.mark.parametrize("name", ["A", "B", "C"])
    def test_block(self, name):
        w = oracle.q4_0_dequant(self._block(name)[None, :], 32)
        assert np.array_equal(w[0], np.array(self.g["blocks"][name]["weights"], float))

    def test_matrix(self):
        m = self.g["matrix"]
        rows = np.stack([np.concatenate([self._block(n) for n in r]) for r in m["rows"]])
        w = oracle.q4_0_dequant(rows, m["cols"])
        expect = np.stack([np.concatenate([self.g["blocks"][n]["weights"] for n in r]) for r in m["rows"]])
        assert np.array_equal(w, expect.astype(float))
        qm = Q4_0Matrix(rows, m["cols"])
        assert np.array_equal(qm.rows([1]), expect[1:2].astype(float))

    def test_random_codes(self):
        # Bytes assembled here one nibble at a time from random scales/codes.
        rng = np.random.default_rng(5)
        rows, nb = 3, 4
        scales = (rng.standard_normal((rows, nb)) * 0.1).astype(np.float16)
        codes = rng.integers(0, 16, size=(rows, nb, 32))
        raw = bytearray()
        for r in range(rows):
            for b in range(nb):
                raw += scales[r, b].tobytes()
                for j in range(16):
                    raw.append(int(codes[r, b, j]) | (int(codes[r, b, j + 16]) << 4))
        blocks = np.frombuffer(bytes(raw), np.uint8).reshape(rows, nb * 18)
        w = oracle.q4_0_dequant(blocks, nb * 32)
        for r in range(rows):
            for b in range(nb):
                for j in range(32):
                    assert w[r, 32 * b + j] == float(scales[r, b]) * (int(codes[r, b, j]) - 8)

    def test_bad_shapes(self):
        with pytest.raises(ValueError):
            oracle.q4_0_dequant(np.zeros((1, 18), np.uint8), 33)
        with pytest.raises(ValueError):
            oracle.q4_0_dequant(np.zeros((1, 17), np.uint8), 32)


# ---------------------------------------------------------------------------
# Brute force on tiny random inputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["relu", "relu2", "reglu"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_dense_and_sparse(act, seed):
    rng = np.random.default_rng(100 + seed)
    d, f, n = 7 + seed, 13 + 2 * seed, 1 + seed
    w_up, w_dt, kw = _random_ffn(rng, d, f, act)
    xs = rng.standard_normal((n, d))
    y, fired = oracle.dense_ffn(xs, w_up, w_dt, act, **kw)
    ref = _bf_ffn(xs, range(f), act, w_up, w_dt, **kw)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    for t in range(n):
        for i in range(f):
            assert fired[t, i] == _bf_neuron(xs[t], i, act, w_up, kw["b_up"], kw["w_gate"], kw["b_gate"])[1]
    sub = sorted(rng.choice(f, size=f // 2, replace=False).tolist())
    ys = oracle.sparse_ffn(xs, sub, w_up, w_dt, act, **kw)
    ref = _bf_ffn(xs, sub, act, w_up, w_dt, **kw)
    assert np.allclose(ys, ref, rtol=1e-12, atol=1e-12 * max(1.0, np.abs(ref).max()))


def test_bruteforce_predict():
    rng = np.random.default_rng(7)
    d, r, f, n = 9, 3, 17, 2
    p1 = rng.standard_normal((r, d))
    p2 = rng.standard_normal((f, r))
    c = rng.standard_normal(f)
    xs = rng.standard_normal((n, d))
    tau = 0.3
    logits, mask = oracle.predict(xs, p1, p2, c, tau)
    for t in range(n):
        tt = [_dot(p1[k], xs[t]) for k in range(r)]
        for i in range(f):
            l = _dot(p2[i], tt) + c[i]
            assert math.isclose(logits[t, i], l, rel_tol=1e-12, abs_tol=1e-12)
            # sigmoid evaluated directly; far from the band both rules agree
            s = 1.0 / (1.0 + math.exp(-l))
            if abs(s - tau) > 1e-9:
                assert bool(mask[t, i]) == (s > tau)


def test_predict_nan_is_inactive():
    logits, mask = oracle.predict(np.array([1.0]), np.array([[1.0]]), np.array([[1.0], [1.0]]),
                                  np.array([np.nan, 0.5]), 0.5)
    assert not mask[0, 0] and mask[0, 1]


# ---------------------------------------------------------------------------
# Invariants of the method
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["relu", "relu2", "reglu"])
def test_superset_reproduces_dense(act):
    rng = np.random.default_rng(11)
    d, f, n = 96, 300, 3
    w_up, w_dt, kw = _random_ffn(rng, d, f, act, dtype=np.float16)
    xs = rng.standard_normal((n, d)).astype(np.float16)
    y, fired = oracle.dense_ffn(xs, w_up, w_dt, act, **kw)
    extra = rng.random(f) < 0.2
    for t in range(n):
        sup = np.flatnonzero(fired[t] | extra)
        ys = oracle.sparse_ffn(xs[t], sup, w_up, w_dt, act, **kw)
        assert np.max(np.abs(ys[0] - y[t])) <= 1e-12 * np.abs(y[t]).max()
    # one list for all tokens: the union of the firing sets
    union = np.flatnonzero(fired.any(axis=0))
    yu = oracle.sparse_ffn(xs, union, w_up, w_dt, act, **kw)
    assert np.max(np.abs(yu - y)) <= 1e-12 * np.abs(y).max()
    # a strict subset of the firing set misses something
    if fired[0].sum() > 1:
        missing = np.flatnonzero(fired[0])[1:]
        assert np.max(np.abs(oracle.sparse_ffn(xs[0], missing, w_up, w_dt, act, **kw)[0] - y[0])) > 0


def test_all_ones_and_empty():
    rng = np.random.default_rng(12)
    d, f = 40, 70
    w_up, w_dt, kw = _random_ffn(rng, d, f, "relu", dtype=np.float32)
    x = rng.standard_normal(d).astype(np.float32)
    y, _ = oracle.dense_ffn(x, w_up, w_dt, "relu", **kw)
    idx, count = oracle.compact(np.ones(f, np.uint8))
    assert count == f
    assert np.max(np.abs(oracle.sparse_ffn(x, idx, w_up, w_dt, "relu", **kw) - y)) <= 1e-12 * np.abs(y).max()
    idx, count = oracle.compact(np.zeros(f, np.uint8))
    assert count == 0 and idx.size == 0
    y0 = oracle.sparse_ffn(x, idx, w_up, w_dt, "relu", **kw)
    assert y0.shape == (1, d) and np.all(y0 == 0.0)


def test_partition_adds_up():
    rng = np.random.default_rng(13)
    d, f = 33, 90
    for act in ("relu", "reglu", "relu2"):
        w_up, w_dt, kw = _random_ffn(rng, d, f, act)
        xs = rng.standard_normal((2, d))
        s = np.flatnonzero(rng.random(f) < 0.5)
        side = rng.random(s.size) < 0.5
        ya = oracle.sparse_ffn(xs, s[side], w_up, w_dt, act, **kw)
        yb = oracle.sparse_ffn(xs, s[~side], w_up, w_dt, act, **kw)
        yall = oracle.sparse_ffn(xs, s, w_up, w_dt, act, **kw)
        assert np.max(np.abs(ya + yb - yall)) <= 1e-12 * max(1.0, np.abs(yall).max())


# ---------------------------------------------------------------------------
# Compaction
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_ff", [1, 2, 15, 16, 17, 1000, 4099])
def test_compact_matches_flatnonzero(d_ff):
    rng = np.random.default_rng(d_ff)
    for density in (0.0, 0.03, 0.5, 1.0):
        m = (rng.random(d_ff) < density).astype(np.uint8)
        idx, count = oracle.compact(m)
        assert idx.dtype == np.int32
        assert np.array_equal(idx, np.flatnonzero(m))
        assert count == int(m.sum())
        assert np.all(np.diff(idx) > 0)


def test_compact_union_and_nonzero_bytes():
    rng = np.random.default_rng(3)
    m = (rng.random((5, 257)) < 0.1).astype(np.uint8)
    m[2, 7] = 200          # any nonzero byte marks the neuron
    idx, count = oracle.compact(m)
    assert np.array_equal(idx, np.flatnonzero(m.any(axis=0)))
    assert 7 in idx.tolist()


# ---------------------------------------------------------------------------
# Predictor special cases
# ---------------------------------------------------------------------------

def test_identity_predictor_recovers_firing_set():
    # r = d, p1 = I, p2 = w_up, c = b_up, tau = 1/2: the logits are the
    # pre-activations, the mask is the true firing set and the layer is dense.
    rng = np.random.default_rng(21)
    d, f, n = 48, 160, 4
    w_up, w_dt, kw = _random_ffn(rng, d, f, "relu", dtype=np.float32)
    xs = rng.standard_normal((n, d)).astype(np.float32)
    y, fired = oracle.dense_ffn(xs, w_up, w_dt, "relu", **kw)
    logits, mask = oracle.predict(xs, np.eye(d), w_up, kw["b_up"], 0.5)
    assert np.array_equal(mask, fired)
    out = oracle.layer(xs, np.eye(d), w_up, kw["b_up"], 0.5, w_up, w_dt, "relu", **kw)
    assert np.max(np.abs(out["y"] - y)) <= 1e-12 * np.abs(y).max()


@pytest.mark.parametrize("tau", [1e-6, 0.01, 0.2, 0.5, 0.6, 0.9, 0.999])
def test_threshold_closed_form(tau):
    theta = oracle.logit_threshold(tau)
    assert math.isclose(1.0 / (1.0 + math.exp(-theta)), tau, rel_tol=1e-12)
    ls = theta + np.concatenate([-np.logspace(-6, 2, 50), np.logspace(-6, 2, 50)])
    s = oracle.sigmoid(ls)
    assert np.array_equal(s > tau, ls > theta)


def test_threshold_rejects_out_of_range():
    for tau in (0.0, 1.0, -0.1, 2.0):
        with pytest.raises(ValueError):
            oracle.logit_threshold(tau)
