"""Pins for the oracle's MoE combine (the reading: out[t] = sum_k w[t,k] *
y[row_of_slot[t,k]] over live slots, fp64, rounded once to bf16) -- closed
forms, exact small-integer sums, power-of-two scaling and order invariance."""
import numpy as np

import oracle


def bf16(v):
    return oracle.bf16_round_array(np.asarray(v, np.float64))


def test_single_slot_unit_weight_copies_the_row():
    rng = np.random.default_rng(1)
    y = bf16(rng.standard_normal((9, 40)) * 10)
    ros = np.array([4, 0, 8, 2], np.int32)
    res = oracle.combine(y, ros, np.ones(4, np.float32), 4)
    assert np.array_equal(res["out"], y[ros])


def test_hand_example_and_dropped_slots():
    y = bf16([[1.0, -2.0], [0.5, 3.0], [7.0, 7.0]])
    # token 0: rows 0 and 1 with weights 1/4 and 1/2; token 1: dropped slots
    # (-1 and past the rows) and row 2 with weight 2; token 2: nothing live
    ros = np.array([0, 1, -1, -1, 2, 3, -1, 99, 5], np.int32)
    w = np.array([0.25, 0.5, 9.0, 9.0, 2.0, 9.0, 9.0, 9.0, 9.0], np.float32)
    res = oracle.combine(y, ros, w, 3)
    e = res["exact"]
    assert np.array_equal(e[0], [0.25 * 1.0 + 0.5 * 0.5, 0.25 * -2.0 + 0.5 * 3.0])  # [0.5, 1.0]
    assert np.array_equal(e[1], [14.0, 14.0])
    assert np.array_equal(e[2], [0.0, 0.0])
    assert np.array_equal(res["out"], bf16(e))
    assert np.array_equal(res["bound"][0], [0.25 + 0.25, 0.5 + 1.5])


def test_power_of_two_weight_scaling_is_exact():
    rng = np.random.default_rng(2)
    y = bf16(rng.standard_normal((30, 24)))
    ros = rng.integers(0, 30, 10 * 4).astype(np.int32)
    w = (rng.random(40) + 0.1).astype(np.float32)
    a = oracle.combine(y, ros, w, 10)
    b = oracle.combine(y, ros, (w * np.float32(8.0)).astype(np.float32), 10)
    assert np.array_equal(b["exact"], a["exact"] * 8.0)
    assert np.array_equal(oracle.bf16_round_array(b["exact"] / 8.0), a["out"])


def test_slot_order_does_not_matter_for_exact_sums():
    # small integers: every partial sum is exact, so the k order cannot change anything
    rng = np.random.default_rng(3)
    y = bf16(rng.integers(-50, 50, (12, 16)))
    ntok, k = 6, 5
    ros = rng.integers(0, 12, ntok * k).astype(np.int32)
    w = rng.integers(1, 8, ntok * k).astype(np.float32)
    a = oracle.combine(y, ros, w, ntok)
    perm = np.concatenate([t * k + rng.permutation(k) for t in range(ntok)])
    b = oracle.combine(y, ros[perm], w[perm], ntok)
    assert np.array_equal(a["exact"], b["exact"]) and np.array_equal(a["out"], b["out"])
    # and the sums are the plain integer sums
    yi = oracle.bf16_value_array(y).astype(np.int64)
    expect = np.zeros((ntok, 16), np.int64)
    for t in range(ntok):
        for j in range(k):
            expect[t] += int(w[t * k + j]) * yi[ros[t * k + j]]
    assert np.array_equal(a["exact"], expect.astype(np.float64))


def test_bound_dominates_and_equals_for_nonnegative_terms():
    rng = np.random.default_rng(4)
    y = bf16(np.abs(rng.standard_normal((20, 8))))
    ros = rng.integers(0, 20, 7 * 3).astype(np.int32)
    w = rng.random(21).astype(np.float32)
    res = oracle.combine(y, ros, w, 7)
    assert np.array_equal(res["bound"], res["exact"])
    y2 = bf16(rng.standard_normal((20, 8)))
    res2 = oracle.combine(y2, ros, w, 7)
    assert np.all(res2["bound"] >= np.abs(res2["exact"]))
