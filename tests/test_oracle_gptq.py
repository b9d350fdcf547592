"""Pins for the GPTQ oracle (aiwing.uk ch.22 sec.22.3).

Q-1  with H proportional to the identity there is nothing to compensate (U is diagonal),
     so GPTQ is round-to-nearest: the same codes, scales and zero points as ``quantize``;
Q-2  the page's objective: on correlated calibration data ||W X - W_hat X||_F^2 of GPTQ is
     below that of round-to-nearest on the same X (with and without AWQ s);
Q-3  the objective is invariant to scaling X by a power of two, bit for bit;
Q-4  U is upper triangular with U^T U = (H + damping)^-1;
and a mutation (error propagated with the wrong sign) that fails Q-2.
"""
import numpy as np
import pytest

import oracle
from oracle import gptq


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
