"""Pins of the oracle's QKV projection (reading R8: [Q | K | V] = x W^T + b,
rounded once to fp16) against cases whose result is fixed by the definition
alone: one-hot inputs pick out a weight column, stacked identity weights
reproduce the input in the Q, K, V order, exact halfway sums round to even,
and small integer sums equal Python's exact integer arithmetic."""
import numpy as np

import oracle as O


def test_one_hot_rows_select_weight_columns():
    # x row n = e_{j(n)}: output row n = W[:, j(n)] + b exactly (x W^T, not x W)
    rng = np.random.default_rng(1)
    C, R = 64, 48
    w = (rng.integers(-64, 65, (R, C)) / 32).astype(np.float16)
    b = (rng.integers(-16, 17, R) / 16).astype(np.float16)
    js = rng.integers(0, C, 10)
    x = np.zeros((10, C), np.float16)
    x[np.arange(10), js] = 1
    y = O.qkv_projection(x, w, b)
    want = (w[:, js].T.astype(np.float64) + b.astype(np.float64)).astype(np.float16)
    assert np.array_equal(y, want)
    assert np.array_equal(O.qkv_projection(x, w), w[:, js].T)


def test_stacked_identity_gives_q_k_v_in_order():
    # W = [I; 2I; -I] (3 H D x H D): Q = x, K = 2x, V = -x, head h = channels h D..h D+D-1
    rng = np.random.default_rng(2)
    H, D, n = 3, 8, 5
    C = H * D
    x = rng.standard_normal((n, C)).astype(np.float16)
    eye = np.eye(C)
    w = np.concatenate([eye, 2 * eye, -eye]).astype(np.float16)
    q, k, v = O.split_qkv(O.qkv_projection(x, w), H, D)
    for h in range(H):
        xs = x[:, h * D:(h + 1) * D]
        assert np.array_equal(q[h], xs)
        assert np.array_equal(k[h], (2 * xs.astype(np.float64)).astype(np.float16))
        assert np.array_equal(v[h], -xs)


def test_halfway_sums_round_to_even_once():
    # 1 + 2^-11 lies halfway between fp16 1 and 1 + 2^-10: to 1 (even);
    # 1 + 3 * 2^-11 halfway between 1 + 2^-10 and 1 + 2^-9: to 1 + 2^-9 (even)
    x = np.array([[1.0, 2.0 ** -11], [1.0, 3 * 2.0 ** -11], [1.0, 2.0 ** -11 + 2.0 ** -20]],
                 np.float16)
    w = np.ones((1, 2), np.float16)
    y = O.qkv_projection(x, w)[:, 0].astype(np.float64)
    assert y[0] == 1.0
    assert y[1] == 1.0 + 2.0 ** -9
    assert y[2] == 1.0 + 2.0 ** -10          # just above halfway: up


def test_small_integer_sums_are_exact():
    rng = np.random.default_rng(3)
    n, C, R = 7, 40, 9
    xi = rng.integers(-20, 21, (n, C))
    wi = rng.integers(-20, 21, (R, C))
    bi = rng.integers(-100, 101, R)
    y = O.qkv_projection(xi.astype(np.float16), wi.astype(np.float16), bi.astype(np.float16))
    for i in range(n):
        for r in range(R):
            exact = sum(int(xi[i, c]) * int(wi[r, c]) for c in range(C)) + int(bi[r])
            assert float(y[i, r]) == float(np.float16(exact))
