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

import hstu_synth as synth
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


def _layer_case(seed=0, with_bias=True, mfalcon=False):
    rng = np.random.default_rng(seed)
    H, d, D = 2, 2, 4
    offsets = np.array([0, 5, 8], dtype=np.int32)
    T = int(offsets[-1])
    x = rng.normal(0, 0.7, size=(T, D))
    w1 = rng.normal(0, 0.5, size=(4 * H * d, D))
    w2 = rng.normal(0, 0.5, size=(D, H * d))
    b1 = rng.normal(0, 0.2, size=4 * H * d) if with_bias else None
    b2 = rng.normal(0, 0.2, size=D) if with_bias else None
    ts = np.cumsum(rng.integers(1, 40, size=T)).astype(np.int64)
    rp = rng.normal(0, 0.3, size=4)
    rt = rng.normal(0, 0.3, size=5)
    nc = np.array([2, 1], dtype=np.int32) if mfalcon else None
    return dict(x=x, w1=w1, w2=w2, b1=b1, b2=b2, offsets=offsets, ts=ts, rp=rp, rt=rt, H=H, d=d,
                alpha=0.41, eps=1e-3, nc=nc)


def _layer_loss(c, g, **over):
    a = dict(c)
    a.update(over)
    y = oracle.layer(a["x"], a["w1"], a["w2"], a["offsets"], a["ts"], a["rp"], a["rt"], a["alpha"],
                     a["H"], a["d"], b1=a["b1"], b2=a["b2"], eps=a["eps"], num_candidates=a["nc"])
    return float(np.sum(y * g))


@pytest.mark.parametrize("mfalcon", [False, True])
def test_layer_bwd_matches_finite_differences(mfalcon):
    c = _layer_case(1, mfalcon=mfalcon)
    g = np.random.default_rng(2).normal(size=c["x"].shape)
    got = oracle.layer_bwd(c["x"], c["w1"], c["w2"], c["offsets"], c["ts"], c["rp"], c["rt"],
                           c["alpha"], c["H"], c["d"], g, b1=c["b1"], b2=c["b2"], eps=c["eps"],
                           num_candidates=c["nc"])
    for name, key in [("x", "dx"), ("w1", "dw1"), ("b1", "db1"), ("w2", "dw2"), ("b2", "db2"),
                      ("rp", "drab_pos"), ("rt", "drab_time")]:
        arr = c[name]
        ref = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1 = arr.copy(); a1[idx] += STEP
            a0 = arr.copy(); a0[idx] -= STEP
            ref[idx] = (_layer_loss(c, g, **{name: a1}) - _layer_loss(c, g, **{name: a0})) / (2 * STEP)
        np.testing.assert_allclose(got[key], ref, rtol=1e-6, atol=1e-8, err_msg=f"layer d{name}")


def test_layer_bwd_residual_and_bias_identities():
    """dX - dX_out is the part through f1 alone, and the bias gradients are the
    token sums of the pre-activation gradients: db2 = sum_t dX_out, and with
    x = 0 rows db1 equals the gradient through a constant input column."""
    c = _layer_case(3)
    g = np.random.default_rng(4).normal(size=c["x"].shape)
    got = oracle.layer_bwd(c["x"], c["w1"], c["w2"], c["offsets"], c["ts"], c["rp"], c["rt"],
                           c["alpha"], c["H"], c["d"], g, b1=c["b1"], b2=c["b2"], eps=c["eps"])
    np.testing.assert_allclose(got["db2"], g.sum(axis=0), rtol=1e-12, atol=1e-12)
    # a bias is a weight on an all-ones input column: extend X with ones and W1 with b1
    x1 = np.concatenate([c["x"], np.ones((c["x"].shape[0], 1))], axis=1)
    w11 = np.concatenate([c["w1"], c["b1"][:, None]], axis=1)
    g1 = np.concatenate([g, np.zeros((g.shape[0], 1))], axis=1)
    w21 = np.concatenate([c["w2"], np.zeros((1, c["w2"].shape[1]))], axis=0)
    b21 = np.concatenate([c["b2"], [0.0]])
    ext = oracle.layer_bwd(x1, w11, w21, c["offsets"], c["ts"], c["rp"], c["rt"], c["alpha"],
                           c["H"], c["d"], g1, b2=b21, eps=c["eps"])
    np.testing.assert_allclose(ext["dw1"][:, -1], got["db1"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ext["dw1"][:, :-1], got["dw1"], rtol=1e-10, atol=1e-12)


def test_attn_bwd_rows_equals_full_oracle_at_those_rows():
    """The row-by-row gradient entry gives exactly the full oracle's dQ at the
    selected query rows and dK, dV at the selected key rows: candidates, a
    sequence of candidates only, per-head tables, identity activation."""
    x = synth.make_attn(83, [37, 1, 90, 64], H=2, d=16, P=40, NT=12, alpha=0.125, dtype="f32",
                        num_candidates=[5, 0, 30, 64])
    rng = np.random.default_rng(84)
    rp = rng.normal(0, 0.1, size=(2, 40))
    rt = rng.normal(0, 0.1, size=(2, 12))
    dout = rng.normal(0, 1.0, size=x.v.shape)
    qrows = np.array([0, 36, 37, 38, 50, 127, 128, 191])
    krows = np.array([1, 37, 40, 100, 127, 130, 191, 0])
    for act in (oracle.ACT_SILU, oracle.ACT_IDENTITY):
        dq, dk, dv, _, _ = oracle.attn_bwd(x.q, x.k, x.v, x.offsets, x.ts, rp, rt, x.alpha, dout,
                                           num_candidates=x.num_candidates, act=act)
        rq, rk, rv = oracle.attn_bwd_rows(x.q, x.k, x.v, x.offsets, x.ts, rp, rt, x.alpha, dout,
                                          qrows, krows, num_candidates=x.num_candidates, act=act)
        assert np.array_equal(rq, dq[qrows])
        assert np.array_equal(rk, dk[krows])
        assert np.array_equal(rv, dv[krows])
