"""GPU parity of the adapter optimizer step against the oracle.

"Paged optimizers, and QLoRA end to end" (zerotofrontier.app "sft/peft"): the adapters'
Adam states are paged between GPU and host memory.  The kernel computes the AdamW update
in fp32, the oracle in float64 from the same fp32 state.  The tolerance is the error
bound of the kernel's fp32 arithmetic, propagated per element from the oracle's exact
values (u = 2^-24, each fp32 operation within one rounding):
  |dm| <= 6u (b1|m| + (1-b1)|g|),   |dv| <= 6u (b2 v + (1-b2) g^2)
  the update step*m/denom, denom = sqrt(v)/sqrt(bc2) + eps, moves by at most
    step (|dm| + 6u|m|) / denom + step |m| ddenom / denom^2,
    ddenom <= min(|dv| / (2 sqrt(v)), sqrt(|dv|)) / sqrt(bc2) + 6u denom
  |dp| <= 4u |p| + (update bound) + u |p'|
and the whole bound is doubled.  A wrong bias correction, sign or decay term moves p by
a sizeable fraction of lr and fails it.  The bf16 copy must equal round-to-nearest-even
of the kernel's own fp32 p bit for bit, and the paged path must equal the device path
bit for bit.
"""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_09_amd as nf4
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
U = 2.0 ** -24
F32 = lambda x: float(np.float32(x))      # hyperparameters as the kernel receives them


def _state(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    p = rng.normal(0, 0.02, n).astype(np.float32)
    g = rng.normal(0, 1e-2, n).astype(np.float32)
    m = rng.normal(0, 1e-3, n).astype(np.float32)
    v = (rng.normal(0, 1e-2, n) ** 2).astype(np.float32)
    if n > 8:
        g[:3] = 0.0                       # zero gradient
        m[3], v[3] = 0.0, 0.0             # fresh moments
        g[4] = 1e4                        # large gradient
        v[5] = 0.0                        # sqrt(0)
    return p, g, m, v


def _bound(p0, g, m0, v0, po, mo, vo, lr, b1, b2, eps, t):
    p0, g, m0, v0 = (a.astype(np.float64) for a in (p0, g, m0, v0))
    bc1, bc2 = 1.0 - b1 ** t, 1.0 - b2 ** t
    step = lr / bc1
    dm = 6 * U * (b1 * np.abs(m0) + (1 - b1) * np.abs(g))
    dv = 6 * U * (b2 * v0 + (1 - b2) * g * g)
    sv = np.sqrt(vo)
    denom = sv / np.sqrt(bc2) + eps
    with np.errstate(divide="ignore", invalid="ignore"):
        dsq = np.where(sv > 0, np.minimum(dv / (2 * np.where(sv > 0, sv, 1)), np.sqrt(dv)), np.sqrt(dv))
    ddenom = dsq / np.sqrt(bc2) + 6 * U * denom
    dupd = step * (dm + 6 * U * np.abs(mo)) / denom + step * np.abs(mo) * ddenom / denom ** 2
    dp = 4 * U * np.abs(p0) + dupd + U * np.abs(po)
    return 2 * dp, 2 * dm, 2 * dv


def _run_gpu(p, g, m, v, lr, t, b1, b2, eps, wd, paged=False, stage_bytes=None):
    gd = torch.from_numpy(g).to(DEV)
    pbf = torch.empty(p.size, dtype=torch.bfloat16, device=DEV)
    if paged:
        ph, mh, vh = (torch.from_numpy(a.copy()).pin_memory() for a in (p, m, v))
        stage = None
        if stage_bytes is not None:
            stage = nf4._workspace(stage_bytes, torch.device(DEV))
        nf4.adamw_step_paged(ph, gd, mh, vh, lr, t, b1, b2, eps, wd, p_bf16=pbf, stage=stage)
        torch.cuda.synchronize()
        return ph.numpy().copy(), mh.numpy().copy(), vh.numpy().copy(), pbf
    pd, md, vd = (torch.from_numpy(a).to(DEV) for a in (p, m, v))
    nf4.adamw_step(pd, gd, md, vd, lr, t, b1, b2, eps, wd, p_bf16=pbf)
    torch.cuda.synchronize()
    return pd.cpu().numpy(), md.cpu().numpy(), vd.cpu().numpy(), pbf


@pytest.mark.parametrize("n", [1, 3, 4, 7, 1000, 65537, (1 << 20) + 3])
@pytest.mark.parametrize("t,wd", [(1, 0.0), (3, 0.01), (1000, 0.1)])
def test_adamw_step_matches_oracle(n, t, wd):
    print("adamw", n, t, wd, flush=True)
    p, g, m, v = _state(n, seed=n * 7 + t)
    lr, b1, b2, eps = F32(1e-4), F32(0.9), F32(0.999), F32(1e-8)
    pg, mg, vg, pbf = _run_gpu(p, g, m, v, lr, t, b1, b2, eps, F32(wd))
    po, mo, vo = oracle.adamw_step(p, g, m, v, lr, b1, b2, eps, F32(wd), t)
    bp, bm, bv = _bound(p, g, m, v, po, mo, vo, lr, b1, b2, eps, t)
    assert np.all(np.abs(mg - mo) <= bm), "m"
    assert np.all(np.abs(vg - vo) <= bv), "v"
    assert np.all(np.abs(pg - po) <= bp), "p: max excess %g" % np.max(np.abs(pg - po) - bp)
    expect_bf = torch.from_numpy(pg).bfloat16().view(torch.int16).numpy()
    assert np.array_equal(pbf.cpu().view(torch.int16).numpy(), expect_bf), "bf16 copy"


@pytest.mark.parametrize("n,stage_bytes", [(1000, 1536), (1000, 3 * 1536), (65537, 1 << 16), (5, 1 << 20),
                                           (64 * 5, 1536)])
def test_paged_step_equals_device_step(n, stage_bytes):
    # the paged path (host-resident state through a staging buffer, several chunks and a
    # partial last chunk) gives the device path's bits
    p, g, m, v = _state(n, seed=99 + n)
    args = (F32(2e-4), 7, F32(0.9), F32(0.999), F32(1e-8), F32(0.05))
    a = _run_gpu(p, g, m, v, *args)
    b = _run_gpu(p, g, m, v, *args, paged=True, stage_bytes=stage_bytes)
    for x, y, name in zip(a[:3], b[:3], "pmv"):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), name
    assert torch.equal(a[3].view(torch.int16), b[3].view(torch.int16)), "bf16 copy"


def test_paged_adamw_optimizer():
    # adapter tensors of two projections (A r x K, B N x r), three steps; a budget that
    # keeps only the first on the GPU, one tensor paged out and back mid-run: same bits
    # as keeping everything on the GPU, and the first step agrees with the oracle
    torch.manual_seed(0)
    shapes = [(64, 512), (384, 64), (64, 1088), (200, 64)]
    params_a = [(torch.randn(s, device=DEV) * 0.02).bfloat16() for s in shapes]
    params_b = [q.clone() for q in params_a]
    opt_a = nf4.PagedAdamW(params_a, lr=1e-4, weight_decay=0.01)
    opt_b = nf4.PagedAdamW(params_b, lr=1e-4, weight_decay=0.01,
                           device_budget_bytes=shapes[0][0] * shapes[0][1] * 12, stage_bytes=4096)
    assert not opt_b.on_host(0) and all(opt_b.on_host(i) for i in range(1, 4))
    p_first = [q.float().cpu().numpy().ravel() for q in params_a]
    for it in range(3):
        grads = [torch.randn(s, device=DEV) * 1e-2 for s in shapes]
        if it == 0:
            g_first = [x.cpu().numpy().ravel() for x in grads]
        opt_a.step(grads)
        opt_b.step(grads)
        if it == 0:
            opt_b.page_in(2)
            opt_b.page_out(0)
            torch.cuda.synchronize()
            for i in range(4):
                z = np.zeros_like(p_first[i])
                po, _, _ = oracle.adamw_step(p_first[i], g_first[i], z, z, F32(1e-4), F32(0.9), F32(0.999),
                                             F32(1e-8), F32(0.01), 1)
                got = params_a[i].float().cpu().numpy().ravel()
                # bf16 copy of the updated master: within half a bf16 ulp of the exact step
                assert np.all(np.abs(got - po) <= 2.0 ** -8 * np.abs(po) + 1e-30), i
    torch.cuda.synchronize()
    for qa, qb in zip(params_a, params_b):
        assert torch.equal(qa.view(torch.int16), qb.view(torch.int16))
    for sa, sb in zip(opt_a.state, opt_b.state):
        for k in ("p", "m", "v"):
            assert torch.equal(sa[k].cpu().view(torch.int32), sb[k].cpu().view(torch.int32)), k
