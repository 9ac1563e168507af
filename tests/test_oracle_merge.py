"""Pins of the oracle's chunk partials, merge and serial accumulation (CPU only)."""
import numpy as np
import pytest

from oracle import dense
from tests._helpers import load_golden, rand_problem


@pytest.mark.parametrize("chunk", [64, 32, 22, 16, 4, 15, 17])
def test_chunked_merge_is_exact(chunk):
    # 64 keys: chunk counts 1, 2, 3, 4, 16 and uneven boundaries C-1, C, C+1 around 16
    x = rand_problem(11, 64, 10, 4, 2, 8)
    o, lse = dense.attend(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], 0.35)
    bounds = dense.chunk_bounds(64, chunk)
    po, pl = dense.chunk_partials(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], 0.35, bounds)
    assert po.shape[0] == len(bounds) + 1
    mo, ml = dense.merge(po, pl)
    np.testing.assert_allclose(mo, o, atol=1e-13)
    np.testing.assert_allclose(ml, lse, atol=1e-13)


def test_merge_identities():
    x = rand_problem(12, 40, 8, 2, 1, 4)
    po, pl = dense.chunk_partials(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], 0.5,
                                  dense.chunk_bounds(40, 13))
    o, lse = dense.merge(po, pl)
    # single part
    o1, l1 = dense.merge(po[:1], pl[:1])
    np.testing.assert_array_equal(o1, po[0])
    np.testing.assert_array_equal(l1, pl[0])
    # an empty part (-inf) changes nothing
    po2 = np.concatenate([po, np.zeros_like(po[:1])])
    pl2 = np.concatenate([pl, np.full_like(pl[:1], -np.inf)])
    o2, l2 = dense.merge(po2, pl2)
    np.testing.assert_allclose(o2, o, atol=1e-14)
    np.testing.assert_allclose(l2, lse, atol=1e-14)
    # order does not matter
    perm = np.random.default_rng(0).permutation(po.shape[0])
    o3, l3 = dense.merge(po[perm], pl[perm])
    np.testing.assert_allclose(o3, o, atol=1e-13)
    np.testing.assert_allclose(l3, lse, atol=1e-13)
    # two equal parts: lse + ln 2, same output
    o4, l4 = dense.merge(np.stack([po[0], po[0]]), np.stack([pl[0], pl[0]]))
    np.testing.assert_allclose(o4, po[0], atol=1e-14)
    np.testing.assert_allclose(l4, pl[0] + np.log(2.0), atol=1e-14)
    # all parts empty: O = 0, lse = -inf
    o5, l5 = dense.merge(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o5 == 0) and np.all(np.isneginf(l5))


def test_merge_golden():
    gd = load_golden("merge_closed_form.json")
    pl = np.array([[float(v) for v in r] for r in gd["parts_lse"]])
    po = np.array(gd["parts_o"], dtype=np.float64)
    o, lse = dense.merge(po, pl)
    np.testing.assert_allclose(o, gd["expect"]["o"], atol=1e-14)
    np.testing.assert_allclose(lse, gd["expect"]["lse"], atol=1e-14)


def test_response_part_is_causal_and_prompt_parts_see_all_rows():
    x = rand_problem(13, 8, 6, 2, 2, 4)
    po, pl = dense.chunk_partials(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], 1.0,
                                  dense.chunk_bounds(8, 8))
    # response part of row 0 sees only key 0: O = v_r[0], lse = tau q_0 . k_r[0]
    for h in range(2):
        np.testing.assert_allclose(po[1, 0, h], x["v_r"][0, h], atol=1e-14)
        np.testing.assert_allclose(pl[1, 0, h], x["q"][0, h] @ x["k_r"][0, h], atol=1e-14)


def test_accumulate_counts_members_per_position():
    # G members of ones with lengths R_g: position r accumulates #{g : R_g > r}
    lens = [5, 3, 8, 1, 8, 2, 6, 4]
    acc = dense.accumulate([np.ones((n, 2, 3)) for n in lens], 8)
    expect = np.array([sum(1 for n in lens if n > r) for r in range(8)], dtype=np.float64)
    np.testing.assert_array_equal(acc, np.broadcast_to(expect[:, None, None], acc.shape))


def test_serial_replay_sum_equals_independent_replays():
    # the gradient of a sum of G replayed losses is the sum of G independent gradients
    base = rand_problem(14, 20, 9, 2, 1, 4)
    members = [rand_problem(100 + g, 20, 9, 2, 1, 4) for g in range(8)]
    grads = []
    for m in members:
        grads.append(dense.attend_bwd(m["q"], base["k_p"], base["v_p"], m["k_r"], m["v_r"],
                                      m["d_o"], 0.5)["dk_r"])
    acc = dense.accumulate(grads, 9)
    # linearity check through the loss: scaling member 0's d_o by 2 doubles its term
    m0 = members[0]
    g2 = dense.attend_bwd(m0["q"], base["k_p"], base["v_p"], m0["k_r"], m0["v_r"],
                          2 * m0["d_o"], 0.5)["dk_r"]
    np.testing.assert_allclose(g2, 2 * grads[0], atol=1e-12)
    np.testing.assert_allclose(acc, np.sum(grads, axis=0), atol=1e-12)
