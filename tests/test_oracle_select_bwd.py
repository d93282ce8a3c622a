"""Pins of the oracle's selector-side backward (CPU).

The gate log g = s - LSE(s) of the [SAS] review (§4.2.2; "How it works",
step 5: the loss reaches the selector through g) is differentiated
numerically: with the selection of every row held fixed, the loss
L = sum over rows and selected slots of dg * g(q, kbar) is evaluated through
the oracle's forward (score_select) at q +- h and kbar +- h, and the central
differences must equal oracle.select_bwd.  Inputs are dyadic with few bits so
that x +- h is exact in fp32 (h = 2^-10)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle

H = 2.0 ** -10


def _dyadic(rng, shape, scale=64.0):
    return (np.round(rng.standard_normal(shape) * scale) / scale).astype(np.float32)


def _case(seed, Hq, Hkv, share_group, d=8, b=4, nq=24, K=2):
    rng = np.random.default_rng(seed)
    q = _dyadic(rng, (1, Hq, nq, d))
    C = nq // b
    kbar = _dyadic(rng, (1, Hkv, C, d))
    zeros = np.zeros((1, Hkv, C), np.float32)
    kw = dict(Hkv=Hkv, b=b, K=K, q_pos0=0, gate=True, share_group=share_group)
    ora = oracle.score_select(q, kbar, zeros, np.zeros(C, np.float32), **kw)
    idx = ora["idx"]
    dg = np.where(idx >= 0, rng.standard_normal(idx.shape), 0.0)
    return q, kbar, zeros, idx, dg, kw


def _loss(q, kbar, zeros, idx, dg, kw):
    ora = oracle.score_select(q, kbar, zeros, np.zeros(kbar.shape[2], np.float32), **kw)
    assert np.array_equal(ora["idx"], idx), "selection moved under the perturbation"
    return float(np.sum(np.where(idx >= 0, dg * np.exp(ora["logg"]), 0.0)))


@pytest.mark.parametrize("Hq,Hkv,share_group,seed", [(4, 2, True, 61), (2, 2, False, 62), (4, 1, True, 63)])
def test_select_bwd_matches_finite_differences(Hq, Hkv, share_group, seed):
    q, kbar, zeros, idx, dg, kw = _case(seed, Hq, Hkv, share_group)
    dq, dkbar = oracle.select_bwd(q, kbar, idx, dg, Hkv=Hkv, b=kw["b"], K=kw["K"], q_pos0=0,
                                  share_group=share_group)
    num_q = np.zeros_like(dq)
    for i in np.ndindex(q.shape):
        qp, qm = q.copy(), q.copy()
        qp[i] += H
        qm[i] -= H
        num_q[i] = (_loss(qp, kbar, zeros, idx, dg, kw) - _loss(qm, kbar, zeros, idx, dg, kw)) / (2 * H)
    num_k = np.zeros_like(dkbar)
    for i in np.ndindex(kbar.shape):
        kp, km = kbar.copy(), kbar.copy()
        kp[i] += H
        km[i] -= H
        num_k[i] = (_loss(q, kp, zeros, idx, dg, kw) - _loss(q, km, zeros, idx, dg, kw)) / (2 * H)
    scale = max(np.abs(num_q).max(), np.abs(num_k).max())
    assert scale > 1e-3
    assert np.abs(dq - num_q).max() <= 1e-5 * scale, np.abs(dq - num_q).max()
    assert np.abs(dkbar - num_k).max() <= 1e-5 * scale, np.abs(dkbar - num_k).max()


def test_select_bwd_score_gradient_sums_to_zero():
    """Adding one constant to every score of a row leaves its gate unchanged,
    so the score gradients of a row sum to zero; for a single query row the
    summary gradients of its candidates (ds_c q_hat / sqrt(d)) then sum to
    the zero vector."""
    rng = np.random.default_rng(64)
    d, b = 8, 4
    q = _dyadic(rng, (1, 1, 1, d))
    kbar = _dyadic(rng, (1, 1, 6, d))
    zeros = np.zeros((1, 1, 6), np.float32)
    kw = dict(Hkv=1, b=b, K=3, q_pos0=24, gate=True, share_group=True)
    ora = oracle.score_select(q, kbar, zeros, np.zeros(6, np.float32), **kw)
    dg = np.where(ora["idx"] >= 0, rng.standard_normal(ora["idx"].shape), 0.0)
    dq, dkbar = oracle.select_bwd(q, kbar, ora["idx"], dg, Hkv=1, b=b, K=3, q_pos0=24)
    total = dkbar[0, 0].sum(axis=0)
    assert np.abs(total).max() <= 1e-12 * max(1.0, np.abs(dkbar).max())
    assert np.abs(dq).max() > 0
