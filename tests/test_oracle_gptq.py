"""Pins for the GPTQ oracle (aiwing.uk ch.22 sec.22.3).

Q-1  with H proportional to the identity there is nothing to compensate (U is diagonal),
     so GPTQ is round-to-nearest: the same codes, scales and zero points as ``quantize``;
Q-2  the page's objective: on correlated calibration data ||W X - W_hat X||_F^2 of GPTQ is
     below that of round-to-nearest on the same X (with and without AWQ s);
Q-3  the objective is invariant to scaling X by a power of two, bit for bit;
Q-4  U is upper triangular with U^T U = (H + damping)^-1;
Q-5  the compensated weights in closed form: when column k is reached, the row's
     remaining weights are those that minimise the page's objective (with the damped
     H) given the codes already chosen for columns 0..k-1, i.e. the least-squares
     continuation v = w[k:] + (w[:k] - w_hat[:k]) H[:k, k:] H[k:, k:]^-1.  Every group's
     scale and zero point are the R3-R5 values of v over the group at its first
     column (checked in exact rationals), and every code is the nearest code to v_k;
and mutations (error propagated with the wrong sign; group parameters formed from
the uncompensated W') that fail Q-2 and Q-5.
"""
from fractions import Fraction
import numpy as np
import pytest

import oracle
from oracle import gptq
from oracle.exact import nearest_code, smallest_fp16_at_least


def _data(seed, N, K, n, awq):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    s = np.exp(rng.standard_normal(K) * 0.5).astype(np.float16) if awq else None
    # correlated features: a low-rank mix plus noise (real activations are correlated)
    B = rng.standard_normal((K // 8, K)).astype(np.float32)
    Xc = (rng.standard_normal((n, K // 8)).astype(np.float32) @ B / np.sqrt(K / 8)
          + 0.3 * rng.standard_normal((n, K)).astype(np.float32)).astype(np.float16)
    return W, s, Xc


def _same(a, b):
    return (np.array_equal(a.q, b.q) and np.array_equal(a.scales.view(np.uint16), b.scales.view(np.uint16))
            and np.array_equal(a.zeros.view(np.uint16), b.zeros.view(np.uint16)))


def test_q1_identity_hessian_is_round_to_nearest():
    rng = np.random.default_rng(60)
    N, K = 32, 256
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = (np.eye(K) * 3.0).astype(np.float16)          # H = 18 I
    assert _same(gptq.quantize_gptq(W, None, X), oracle.quantize(W, None))


@pytest.mark.parametrize("awq", [False, True])
def test_q2_gptq_beats_round_to_nearest(awq):
    W, s, X = _data(61 + awq, 48, 512, 1024, awq)
    g = gptq.quantize_gptq(W, s, X)
    r = oracle.quantize(W, s)
    lg, lr = gptq.layer_loss(W, s, g, X), gptq.layer_loss(W, s, r, X)
    assert lg < 0.9 * lr, (lg, lr)


def test_q3_scaling_x_by_two_changes_nothing():
    W, s, X = _data(63, 16, 256, 512, True)
    a = gptq.quantize_gptq(W, s, X)
    b = gptq.quantize_gptq(W, s, (X.astype(np.float32) * 2).astype(np.float16))
    assert _same(a, b)


def test_q4_factor():
    _, s, X = _data(64, 16, 256, 512, True)
    H = gptq.hessian(X, s)
    U = gptq.inverse_cholesky_upper(H)
    assert np.allclose(np.tril(U, -1), 0)
    Hd = H + gptq.DAMP * np.mean(np.diag(H)) * np.eye(256)
    assert np.allclose(U.T @ U @ Hd, np.eye(256), atol=1e-8)


def test_mutation_wrong_sign_fails_q2(monkeypatch):
    W, s, X = _data(65, 32, 384, 768, False)
    lr = gptq.layer_loss(W, s, oracle.quantize(W, s), X)
    real = gptq.inverse_cholesky_upper
    monkeypatch.setattr(gptq, "inverse_cholesky_upper",
                        lambda H, damp=gptq.DAMP: -real(H, damp) + 2 * np.diag(np.diag(real(H, damp))))
    lm = gptq.layer_loss(W, s, gptq.quantize_gptq(W, s, X), X)
    assert not lm < 0.9 * lr


def _near_boundary(x: float, tol: float = 1e-9) -> bool:
    """True when x lies within tol (relative) of a rounding boundary of rint."""
    f = x - np.floor(x)
    return abs(f - 0.5) < tol * max(1.0, abs(x))


def _check_q5(W, s, X, damp=gptq.DAMP):
    """Q-5 on the oracle's result: group parameters and codes against the least-squares
    continuation of the already-quantized columns.  Returns how many (row, group) pairs
    were skipped because v sits within rounding noise of a boundary (the closed form
    and the sequential updates agree to ~1e-12, not bit for bit)."""
    N, K = W.shape
    res = gptq.quantize_gptq(W, s, X, damp)
    Wp = W.astype(np.float64)
    Xs = X.astype(np.float64)
    if s is not None:
        Wp = Wp / s.astype(np.float64)[None, :]
        Xs = Xs * s.astype(np.float64)[None, :]
    H = 2.0 * Xs.T @ Xs
    Hd = H + damp * np.mean(np.diag(H)) * np.eye(K)
    g_of = np.arange(K) // 128
    sc = res.scales.astype(np.float64)[:, g_of]
    zp = res.zeros.astype(np.float64)[:, g_of]
    What = (res.q.astype(np.float64) - zp) * sc            # dequantized, in W' units
    skipped = 0
    for k in range(K):
        a = Wp[:, :k] - What[:, :k]
        v = Wp[:, k:] + (a @ Hd[:k, k:]) @ np.linalg.inv(Hd[k:, k:]) if k else Wp.copy()
        g = k // 128
        for n in range(N):
            if k % 128 == 0:                                 # the group's parameters
                grp = v[n, :128]
                mn, mx = min(grp.min(), 0.0), max(grp.max(), 0.0)
                want, _ = smallest_fp16_at_least(Fraction(mx - mn) / 15)
                lo, _ = smallest_fp16_at_least(Fraction(mx - mn) * (1 - 1e-9) / 15)
                hi, _ = smallest_fp16_at_least(Fraction(mx - mn) * (1 + 1e-9) / 15)
                if lo != hi or _near_boundary(-mn / float(want)):
                    skipped += 1
                    continue
                assert Fraction(float(res.scales[n, g])) == want, (n, g)
                assert float(res.zeros[n, g]) == np.rint(-mn / float(want)), (n, g)
            t = v[n, 0] / float(res.scales[n, g])
            if _near_boundary(t):
                continue
            assert res.q[n, k] == nearest_code(Fraction(t), int(res.zeros[n, g])), (n, k)
    return skipped


def test_q5_least_squares_continuation():
    W, s, X = _data(66, 6, 384, 768, True)
    assert _check_q5(W, s, X) <= 1


def test_mutation_uncompensated_group_parameters_fails_q5(monkeypatch):
    W, s, X = _data(66, 6, 384, 768, True)
    orig = W.astype(np.float64) / s.astype(np.float64)[None, :]
    real = gptq.group_params
    calls = []

    def planted(wg):                     # the g-th call sees the original W' of group g
        g = len(calls)
        calls.append(g)
        return real(orig[:, 128 * g:128 * g + 128])
    monkeypatch.setattr(gptq, "group_params", planted)
    with pytest.raises(AssertionError):
        _check_q5(W, s, X)
