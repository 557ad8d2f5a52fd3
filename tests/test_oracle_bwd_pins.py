"""Pins of the oracle's gradients against facts fixed outside their own code.

The gradient functions are checked against central finite differences of
the (separately pinned) forward oracle, against torch autograd of the
library LayerNorm, and against identities the chain rule must satisfy.  A
dropped term (the bias gradient of one table, the alpha factor, the slope of
SiLU), a transposed operand (dQ from Q instead of K) or a mask slip fails at
least one of them.
"""
import numpy as np
import pytest

import oracle

STEP = 1e-6


def _case(kind, seed=0):
    """Tiny jagged batch: (q, k, v, offsets, ts, rab_pos, rab_time, alpha, lengths, ncand)."""
    rng = np.random.default_rng(seed)
    H, dqk, dv = 2, 3, 2
    lengths = ncand = None
    if kind == "mfalcon":
        offsets = np.array([0, 6, 10], dtype=np.int32)
        ncand = np.array([2, 3], dtype=np.int32)
    elif kind == "padded":
        offsets = np.array([0, 7, 11], dtype=np.int32)
        lengths = np.array([5, 3], dtype=np.int32)
    else:
        offsets = np.array([0, 6, 9], dtype=np.int32)
    T = int(offsets[-1])
    q = rng.normal(0, 0.7, size=(T, H, dqk))
    k = rng.normal(0, 0.7, size=(T, H, dqk))
    v = rng.normal(0, 0.7, size=(T, H, dv))
    # gaps spanning several log2 buckets; 3 of the 5 buckets, the last clamped
    ts = np.cumsum(rng.integers(1, 40, size=T)).astype(np.int64)
    if kind == "per_head":
        rp = rng.normal(0, 0.3, size=(H, 4))
        rt = rng.normal(0, 0.3, size=(H, 5))
    else:
        rp = rng.normal(0, 0.3, size=4)     # P = 4: offsets >= 3 clamp
        rt = rng.normal(0, 0.3, size=5)
    return q, k, v, offsets, ts, rp, rt, 0.37, lengths, ncand


def _loss(args, dout, act, **over):
    q, k, v, offsets, ts, rp, rt, alpha, lengths, ncand = args
    x = dict(q=q, k=k, v=v, rp=rp, rt=rt)
    x.update(over)
    o = oracle.attn(x["q"], x["k"], x["v"], offsets, ts, x["rp"], x["rt"], alpha,
                    lengths=lengths, num_candidates=ncand, act=act)
    return float(np.sum(o * dout))


def _fd(args, dout, act, name, arr):
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        a1 = arr.copy(); a1[idx] += STEP
        a0 = arr.copy(); a0[idx] -= STEP
        g[idx] = (_loss(args, dout, act, **{name: a1}) - _loss(args, dout, act, **{name: a0})) / (2 * STEP)
    return g


@pytest.mark.parametrize("kind,act", [("causal", oracle.ACT_SILU), ("mfalcon", oracle.ACT_SILU),
                                      ("padded", oracle.ACT_SILU), ("per_head", oracle.ACT_SILU),
                                      ("causal", oracle.ACT_IDENTITY)])
def test_attn_bwd_matches_finite_differences(kind, act):
    args = _case(kind)
    q, k, v, offsets, ts, rp, rt, alpha, lengths, ncand = args
    rng = np.random.default_rng(9)
    dout = rng.normal(0, 1.0, size=v.shape)
    dq, dk, dv, drp, drt = oracle.attn_bwd(q, k, v, offsets, ts, rp, rt, alpha, dout,
                                           lengths=lengths, num_candidates=ncand, act=act)
    for name, got, arr in [("q", dq, q), ("k", dk, k), ("v", dv, v), ("rp", drp, rp), ("rt", drt, rt)]:
        ref = _fd(args, dout, act, name, arr)
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-8, err_msg=f"{kind} d{name}")
    # every table entry the batch reaches gets a gradient (the clamped buckets included)
    assert np.count_nonzero(drp) >= 3 and np.count_nonzero(drt) >= 3


def test_attn_bwd_table_gradients_have_equal_totals():
    """Every visible pair adds its dLoss/dS once to a position bucket and once
    to a time bucket, so both tables' gradients sum to the same total; a
    batch with all biases zero and identity activation has dLoss/dS = alpha
    <dO_i, V_j>, whose total is checked directly."""
    args = _case("mfalcon", seed=3)
    q, k, v, offsets, ts, rp, rt, alpha, lengths, ncand = args
    dout = np.random.default_rng(4).normal(size=v.shape)
    _, _, _, drp, drt = oracle.attn_bwd(q, k, v, offsets, ts, rp, rt, alpha, dout,
                                        num_candidates=ncand)
    assert abs(drp.sum() - drt.sum()) <= 1e-12 * max(1.0, abs(drp.sum()))
    _, _, _, drp0, _ = oracle.attn_bwd(q, k, v, offsets, ts, 0 * rp, 0 * rt, alpha, dout,
                                       num_candidates=ncand, act=oracle.ACT_IDENTITY)
    total = 0.0
    for b in range(len(offsets) - 1):
        s0, L = int(offsets[b]), int(offsets[b + 1] - offsets[b])
        for i in range(L):
            for j in range(L):
                if oracle.visible(i, j, L, L - int(ncand[b])):
                    total += alpha * float(np.sum(dout[s0 + i] * v[s0 + j]))
    assert abs(drp0.sum() - total) <= 1e-12 * max(1.0, abs(total))


def test_attn_bwd_is_linear_in_the_upstream_gradient():
    args = _case("causal", seed=5)
    q, k, v, offsets, ts, rp, rt, alpha, _, _ = args
    rng = np.random.default_rng(6)
    g1, g2 = rng.normal(size=v.shape), rng.normal(size=v.shape)
    a = oracle.attn_bwd(q, k, v, offsets, ts, rp, rt, alpha, g1)
    b = oracle.attn_bwd(q, k, v, offsets, ts, rp, rt, alpha, g2)
    c = oracle.attn_bwd(q, k, v, offsets, ts, rp, rt, alpha, 2.0 * g1 - g2)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(z, 2.0 * x - y, rtol=1e-12, atol=1e-12)


def test_ln_gate_bwd_matches_finite_differences_and_torch():
    import torch
    rng = np.random.default_rng(8)
    o = rng.normal(0, 0.2, size=(3, 6))
    u = rng.normal(0, 1.0, size=(3, 6))
    dy = rng.normal(0, 1.0, size=(3, 6))
    eps = 1e-3
    do, du = oracle.ln_gate_bwd(o, u, dy, eps=eps)

    def f(oo, uu):
        return float(np.sum(oracle.ln_gate(oo, uu, eps=eps) * dy))

    for got, which in [(do, 0), (du, 1)]:
        ref = np.zeros_like(o)
        for idx in np.ndindex(o.shape):
            args1 = [o.copy(), u.copy()]
            args0 = [o.copy(), u.copy()]
            args1[which][idx] += STEP
            args0[which][idx] -= STEP
            ref[idx] = (f(*args1) - f(*args0)) / (2 * STEP)
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-8)
    # the same gradients from torch autograd of the library layer_norm
    ot = torch.tensor(o, requires_grad=True)
    ut = torch.tensor(u, requires_grad=True)
    y = torch.nn.functional.layer_norm(ot, (6,), eps=eps) * ut
    y.backward(torch.tensor(dy))
    np.testing.assert_allclose(do, ot.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(du, ut.grad.numpy(), rtol=1e-10, atol=1e-12)
