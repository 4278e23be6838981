"""Pins of the oracle's AdamW step against closed forms and an independent library.

The pages ("Paged optimizers, and QLoRA end to end", zerotofrontier.app "sft/peft")
keep the adapters' Adam states in paged memory and give the learning rates; the
update is Kingma & Ba (2015) Algorithm 1 with Loshchilov & Hutter (2019) decoupled
weight decay.  Each test below fails for a plausible slip in the oracle: a missing or
wrong bias correction, a sign error, decay coupled into the gradient, a dropped term.
"""
import numpy as np
import pytest
import torch

import oracle

B1, B2, EPS = 0.9, 0.999, 1e-8


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def test_first_step_closed_form():
    # from zero moments, step 1: m = (1-b1) g, v = (1-b2) g^2, and the bias-corrected
    # update is g / (|g| + eps), so p moves by lr * sign(g) up to eps
    rng = _rng(1)
    n = 1000
    p = rng.normal(0, 1, n).astype(np.float32)
    g = rng.normal(0, 1e-3, n).astype(np.float32)
    z = np.zeros(n, np.float32)
    lr, wd = 2e-4, 0.01
    po, mo, vo = oracle.adamw_step(p, g, z, z, lr, B1, B2, EPS, wd, 1)
    gd = g.astype(np.float64)
    np.testing.assert_allclose(mo, (1 - B1) * gd, rtol=1e-14, atol=0)
    np.testing.assert_allclose(vo, (1 - B2) * gd * gd, rtol=1e-14, atol=0)
    expect = p.astype(np.float64) * (1 - lr * wd) - lr * gd / (np.abs(gd) + EPS)
    np.testing.assert_allclose(po, expect, rtol=1e-14, atol=1e-18)


@pytest.mark.parametrize("t_end", [1, 7, 200])
def test_constant_gradient_steps(t_end):
    # a constant gradient g from zero moments gives m_t = (1-b1^t) g and
    # v_t = (1-b2^t) g^2, so every bias-corrected step is lr * g / (|g| + eps)
    rng = _rng(2)
    n = 257
    p0 = rng.normal(0, 1, n).astype(np.float32)
    g = rng.normal(0, 1, n).astype(np.float32)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    lr = 1e-4
    for t in range(1, t_end + 1):
        po, mo, vo = oracle.adamw_step(p, g, m, v, lr, B1, B2, EPS, 0.0, t)
        p, m, v = po.astype(np.float32), mo.astype(np.float32), vo.astype(np.float32)
    gd = g.astype(np.float64)
    np.testing.assert_allclose(mo, (1 - B1 ** t_end) * gd, rtol=2e-6, atol=0)
    np.testing.assert_allclose(vo, (1 - B2 ** t_end) * gd * gd, rtol=2e-6, atol=0)
    expect = p0.astype(np.float64) - t_end * lr * gd / (np.abs(gd) + EPS)
    # the state passes through fp32 between steps: one rounding of p per step
    assert np.all(np.abs(po - expect) <= t_end * 2.0 ** -23 * np.abs(expect))


def test_weight_decay_only():
    # zero gradient and zero moments: the update term vanishes and p decays
    # geometrically by (1 - lr wd) per step (decoupled decay, not through m or v)
    n = 64
    p = np.linspace(-3, 3, n).astype(np.float32)
    z = np.zeros(n, np.float32)
    lr, wd = 1e-3, 0.1
    cur = p.copy()
    for t in range(1, 6):
        po, mo, vo = oracle.adamw_step(cur, z, z, z, lr, B1, B2, EPS, wd, t)
        assert not mo.any() and not vo.any()
        np.testing.assert_allclose(po, cur.astype(np.float64) * (1 - lr * wd), rtol=1e-15, atol=0)
        cur = po.astype(np.float32)


@pytest.mark.parametrize("t", [1, 2, 10, 1000])
@pytest.mark.parametrize("wd", [0.0, 0.05])
def test_matches_torch_adamw_float64(t, wd):
    # one step from a given state at step t, against torch.optim.AdamW in float64
    rng = _rng(3 + t)
    n = 513
    p = rng.normal(0, 0.02, n).astype(np.float32)
    g = rng.normal(0, 1e-2, n).astype(np.float32)
    m = rng.normal(0, 1e-3, n).astype(np.float32)
    v = (rng.normal(0, 1e-2, n) ** 2).astype(np.float32)
    lr = 1e-4
    po, mo, vo = oracle.adamw_step(p, g, m, v, lr, B1, B2, EPS, wd, t)

    tp = torch.nn.Parameter(torch.from_numpy(p.astype(np.float64)))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(B1, B2), eps=EPS, weight_decay=wd, foreach=False)
    tp.grad = torch.from_numpy(g.astype(np.float64))
    opt.state[tp] = {"step": torch.tensor(float(t - 1), dtype=torch.float64),
                     "exp_avg": torch.from_numpy(m.astype(np.float64)),
                     "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    opt.step()
    st = opt.state[tp]
    np.testing.assert_allclose(mo, st["exp_avg"].numpy(), rtol=1e-13, atol=1e-20)
    np.testing.assert_allclose(vo, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=1e-24)
    np.testing.assert_allclose(po, tp.detach().numpy(), rtol=1e-13, atol=1e-18)
