"""Shared test helpers: tolerance checks and small random inputs.  No method arithmetic."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rand_problem(seed, P, R, Hq, Hkv, d, dv=None):
    g = np.random.default_rng(seed)
    dv = d if dv is None else dv
    return dict(q=g.standard_normal((R, Hq, d)), k_p=g.standard_normal((P, Hkv, d)),
                v_p=g.standard_normal((P, Hkv, dv)), k_r=g.standard_normal((R, Hkv, d)),
                v_r=g.standard_normal((R, Hkv, dv)), d_o=g.standard_normal((R, Hq, dv)))


def rel_l2(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    return float(np.linalg.norm((x - y).ravel()) / max(np.linalg.norm(y.ravel()), 1e-300))


def max_abs(x, y):
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(y, np.float64)))) if np.size(x) else 0.0


def assert_bf16_close(name, got, ref, rl2=5e-3, mabs=2e-2):
    r, m = rel_l2(got, ref), max_abs(got, ref)
    assert r <= rl2 and m <= mabs, f"{name}: rel-L2 {r:.3e} (<= {rl2}), max-abs {m:.3e} (<= {mabs})"
    return r, m


def assert_f32_close(name, got, ref, mabs=1e-5):
    m = max_abs(got, ref)
    assert m <= mabs, f"{name}: max-abs {m:.3e} (<= {mabs})"
    return m


def assert_D_close(name, got, ref, dtype):
    """D = dO . O (the backward's preprocess) against the oracle's.  D is a d_v-term dot
    product of dO with O, so it carries O's error weighted by dO: the element bound is the
    O bound (bf16: 2e-2, fp32: 1e-5) scaled by max(1, |D|), and bf16 also keeps the
    rel-L2 bound of 5e-3."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    tol = (2e-2 if dtype == "bf16" else 1e-5) * np.maximum(1.0, np.abs(ref))
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"{name}: worst |dD|/bound {float(np.max(err / tol)):.3f}"
    if dtype == "bf16":
        r = rel_l2(got, ref)
        assert r <= 5e-3, f"{name}: rel-L2 {r:.3e}"
