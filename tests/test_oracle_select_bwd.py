"""Pins of the oracle's selector-side backward (CPU).

The gate log g = s - LSE(s) of the [SAS] review (§4.2.2; "How it works",
step 5: the loss reaches the selector through g) is differentiated
numerically: with the selection of every row held fixed, the loss
L = sum over rows and selected slots of dg * g(q, kbar) is evaluated through
the oracle's forward (score_select) at q +- h and kbar +- h, and the central
differences must equal oracle.select_bwd.  Inputs are dyadic with few bits so
that x +- h is exact in fp32 (h = 2^-10).  The same holds through the learned
projection ktilde = W kbar (perturbing W gives dW), and the block mean's
backward is checked against torch autograd of the mean."""
from __future__ import annotations

import numpy as np
import pytest
import torch

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


def _loss(q, kbar, zeros, idx, dg, kw, W=None):
    ora = oracle.score_select(q, kbar, zeros, np.zeros(kbar.shape[2], np.float32), proj_w=W, **kw)
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


@pytest.mark.parametrize("Hq,Hkv,share_group,seed", [(4, 2, True, 65), (2, 1, False, 66)])
def test_select_bwd_through_projection_matches_finite_differences(Hq, Hkv, share_group, seed):
    q, kbar, zeros, _, _, kw = _case(seed, Hq, Hkv, share_group)
    d = q.shape[-1]
    rng = np.random.default_rng(seed + 100)
    W = _dyadic(rng, (d, d), scale=32.0)
    ora = oracle.score_select(q, kbar, zeros, np.zeros(kbar.shape[2], np.float32), proj_w=W, **kw)
    idx = ora["idx"]
    dg = np.where(idx >= 0, rng.standard_normal(idx.shape), 0.0)
    dq, dkbar, dW = oracle.select_bwd(q, kbar, idx, dg, Hkv=Hkv, b=kw["b"], K=kw["K"], q_pos0=0,
                                      share_group=share_group, proj_w=W)

    def numeric(x, loss_at):
        out = np.zeros(x.shape)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += H
            xm[i] -= H
            out[i] = (loss_at(xp) - loss_at(xm)) / (2 * H)
        return out

    num_q = numeric(q, lambda x: _loss(x, kbar, zeros, idx, dg, kw, W=W))
    num_k = numeric(kbar, lambda x: _loss(q, x, zeros, idx, dg, kw, W=W))
    num_w = numeric(W, lambda x: _loss(q, kbar, zeros, idx, dg, kw, W=x))
    scale = max(np.abs(num_q).max(), np.abs(num_k).max(), np.abs(num_w).max())
    assert scale > 1e-3
    for got, num in ((dq, num_q), (dkbar, num_k), (dW, num_w)):
        assert np.abs(got - num).max() <= 1e-5 * scale, np.abs(got - num).max()


def test_select_bwd_identity_projection_is_plain():
    """W = I reduces the projected backward to the plain one (and dW to the
    sum of dkbar_c kbar_c^T)."""
    q, kbar, zeros, idx, dg, kw = _case(67, 4, 2, True)
    d = q.shape[-1]
    a = oracle.select_bwd(q, kbar, idx, dg, Hkv=2, b=kw["b"], K=kw["K"], q_pos0=0)
    dq, dkbar, dW = oracle.select_bwd(q, kbar, idx, dg, Hkv=2, b=kw["b"], K=kw["K"], q_pos0=0,
                                      proj_w=np.eye(d, dtype=np.float32))
    assert np.allclose(dq, a[0], rtol=0, atol=1e-14) and np.allclose(dkbar, a[1], rtol=0, atol=1e-14)
    ref = np.einsum("bhce,bhcf->ef", a[1], kbar.astype(np.float64))
    assert np.allclose(dW, ref, rtol=1e-12, atol=1e-14)


def test_mean_bwd_matches_autograd_of_the_block_mean():
    rng = np.random.default_rng(68)
    B, Hkv, b, ccap, L, d = 2, 3, 4, 5, 23, 6          # 3 trailing tokens are in no summary
    k = torch.tensor(rng.standard_normal((B, Hkv, L, d)), dtype=torch.float64, requires_grad=True)
    up = rng.standard_normal((B, Hkv, ccap, d))
    kbar = k[:, :, :ccap * b].reshape(B, Hkv, ccap, b, d).mean(dim=3)
    (kbar * torch.tensor(up)).sum().backward()
    assert np.allclose(oracle.mean_bwd(up, b, L), k.grad.numpy(), rtol=0, atol=1e-15)
