"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each test fixes the oracle to something other than its own code: values
worked by hand from the pages' definitions (tests/golden), closed forms,
textbook reductions computed with library routines (numpy matmul, scipy's
logistic, torch's layer_norm), and invariants the method must satisfy.
A plausible mistake (a dropped bias term, a sign or index slip, a transposed
operand, a wrong candidate position, an off-by-one mask) fails at least one.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import hstu_synth as synth
from hstu_sequential_transducer_causal_amd import flops

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _num(x):
    """Golden numbers: plain numbers, or expressions in ln3 = ln(3) and sqrt()."""
    if not isinstance(x, str):
        return float(x)
    s = x.replace("ln3", "LN3")
    if s.startswith("LN3"):
        s = "1*" + s
    elif s.startswith("-LN3"):
        s = "-1*" + s[1:]
    else:
        s = s.replace("LN3", "*LN3")
    return float(eval(s, {"LN3": math.log(3), "sqrt": math.sqrt}))


def _run_golden(g):
    T = g["offsets"][-1]
    q = np.array(g["q"], dtype=np.float64).reshape(T, g["H"], g["d_qk"])
    k = np.array(g["k"], dtype=np.float64).reshape(T, g["H"], g["d_qk"])
    v = np.array(g["v"], dtype=np.float64).reshape(T, g["H"], g["d_v"])
    rp = np.array([_num(x) for x in g["rab_pos"]])
    rt = np.array([_num(x) for x in g["rab_time"]])
    act = oracle.ACT_IDENTITY if g["act"] == "identity" else oracle.ACT_SILU
    o = oracle.attn(q, k, v, g["offsets"], np.array(g["ts"], dtype=np.int64), rp, rt,
                    g["alpha"], num_candidates=g["num_candidates"], act=act)
    exp = np.array([[_num(x) for x in row] for row in g["expected_o"]])
    return o.reshape(T, -1), exp


# ---------------------------------------------------------------------------
# scalar definitions
# ---------------------------------------------------------------------------
def test_time_bucket_closed_form():
    # bucket = min(NT-1, bit_length(|gap|)); bit_length(2^k) = k+1, bit_length(2^k-1) = k
    cases = [(0, 0), (1, 1), (2, 2), (3, 2), (4, 3), (7, 3), (8, 4), (60, 6), (3600, 12),
             (86400, 17), (2**30 - 1, 30), (2**30, 31), (2**40, 31), (2**62, 31)]
    for gap, want in cases:
        assert oracle.time_bucket(TS := synth.TS_EPOCH + gap, synth.TS_EPOCH, 32) == want, gap
        assert oracle.time_bucket(synth.TS_EPOCH, TS, 32) == want, -gap   # |gap|
    assert oracle.time_bucket(-(2**62), 2**62, 32) == 31                 # no int64 overflow
    assert oracle.time_bucket(100, 0, 4) == 3                              # saturation at NT-1


def test_position_bucket_and_candidate_positions():
    P = 5
    assert [oracle.pos_bucket(i, 0, 100, P) for i in range(8)] == [0, 1, 2, 3, 4, 4, 4, 4]
    assert oracle.pos_bucket(7, 7, 100, P) == 0
    # candidates (rows >= n_hist = 4) all sit at position 4
    assert oracle.pos_bucket(6, 0, 4, 100) == 4
    assert oracle.pos_bucket(9, 3, 4, 100) == 1
    assert oracle.pos_bucket(9, 9, 4, 100) == 0


def test_gradient_block_count_brute_force():
    """The gradient kernels store G for every 32x32 block that holds a
    visible pair; flops.grad_blocks counts them in closed form."""
    for L, c in [(1, 0), (32, 0), (33, 0), (70, 0), (70, 6), (70, 38), (64, 64), (95, 31)]:
        n = L - c
        want = 0
        for q in range(-(-L // 32)):
            for k in range(q + 1):
                if any(oracle.visible(i, j, L, n)
                       for i in range(32 * q, min(L, 32 * q + 32))
                       for j in range(32 * k, min(L, 32 * k + 32))):
                    want += 1
        assert flops.grad_blocks([L], [c]) == want, (L, c)


def test_mask_pair_counts_closed_form():
    # causal: L(L+1)/2 pairs; M-FALCON: n(n+1)/2 + c(n+1)
    for L in [1, 2, 7, 33]:
        assert oracle.count_visible([0, L]) == L * (L + 1) // 2
    for n, c in [(1, 1), (5, 3), (20, 7), (0, 4)]:
        got = oracle.count_visible([0, n + c], num_candidates=[c])
        assert got == n * (n + 1) // 2 + c * (n + 1)
        assert got == flops.visible_pairs([n + c], [c])
    # candidates never see each other, history never sees candidates
    L, n = 9, 5
    for i in range(L):
        for j in range(L):
            vis = oracle.visible(i, j, L, n)
            if i < n:
                assert vis == (j <= i)
            else:
                assert vis == (j < n or j == i)


def test_silu_properties_and_library_logistic():
    from scipy.special import expit
    xs = [-30.0, -5.0, -1.0, -1e-3, 0.0, 1e-3, 0.5, 1.0, 3.0, 20.0]
    for x in xs:
        assert oracle.silu(x) == pytest.approx(x * expit(x), rel=1e-14, abs=1e-300)
        assert oracle.silu(x) - oracle.silu(-x) == pytest.approx(x, rel=1e-13, abs=1e-15)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(math.log(3)) == pytest.approx(0.75 * math.log(3), rel=1e-15)
    assert oracle.silu(-800.0) == 0.0 or abs(oracle.silu(-800.0)) < 1e-300


# ---------------------------------------------------------------------------
# hand-computed golden cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["attn_identity_causal_4x2.json", "attn_identity_mfalcon_4x2.json"])
def test_golden_identity_exact(name):
    o, exp = _run_golden(_load(name))
    assert np.array_equal(o, exp), (o, exp)


def test_golden_silu_closed_form():
    o, exp = _run_golden(_load("attn_silu_ln3.json"))
    np.testing.assert_allclose(o, exp, rtol=1e-15, atol=0)


def test_golden_ln_gate():
    g = _load("ln_gate_1234.json")
    y = oracle.ln_gate(np.array(g["o"], float), np.array(g["u"], float), eps=g["eps"])
    exp = np.array([[_num(x) for x in r] for r in g["expected_y"]])
    np.testing.assert_allclose(y, exp, rtol=1e-15)


def test_golden_tiles():
    g = _load("tiles_small.json")
    for case in g["cases"]:
        got = oracle.tiles(case["offsets"], case["tile_m"], case["tile_n"],
                           num_candidates=case["num_candidates"])
        assert got.tolist() == case["tiles"], case["why"]


def test_flop_convention_matches_worked_example():
    g = _load("flops_worked_example.json")
    dense = flops.dense_attn_flops(g["T"], g["d"])
    assert abs(dense - g["printed_flops"]) <= g["printed_rel_precision"] * g["printed_flops"]
    # the causal count keeps L(L+1)/2 of the T^2 pairs
    assert flops.attn_flops([g["T"]], 1, g["d"], g["d"]) * 2 == pytest.approx(dense, rel=2e-4)


# ---------------------------------------------------------------------------
# textbook reductions via library routines
# ---------------------------------------------------------------------------
def _rand_batch(seed, lengths, H, d, dv=None, ints=False):
    rng = np.random.default_rng(seed)
    dv = dv or d
    T = int(sum(lengths))
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    if ints:
        q = rng.integers(-3, 4, size=(T, H, d)).astype(np.float64)
        k = rng.integers(-3, 4, size=(T, H, d)).astype(np.float64)
        v = rng.integers(-3, 4, size=(T, H, dv)).astype(np.float64)
    else:
        q = rng.normal(0, 0.5, size=(T, H, d))
        k = rng.normal(0, 0.5, size=(T, H, d))
        v = rng.normal(0, 0.5, size=(T, H, dv))
    ts = np.concatenate([np.cumsum(rng.integers(1, 200, size=L)) for L in lengths]).astype(np.int64)
    return off, q, k, v, ts


def test_identity_zero_bias_is_masked_matmul():
    """act = identity, zero tables: O = alpha * tril(Q K^T) V (numpy matmul)."""
    lengths = [5, 17, 1, 30]
    off, q, k, v, ts = _rand_batch(1, lengths, 3, 8, dv=6)
    alpha = 0.37
    o = oracle.attn(q, k, v, off, ts, np.zeros(16), np.zeros(32), alpha, act=oracle.ACT_IDENTITY)
    for b, L in enumerate(lengths):
        s0, s1 = off[b], off[b + 1]
        for h in range(3):
            S = q[s0:s1, h, :] @ k[s0:s1, h, :].T
            ref = alpha * (np.tril(S) @ v[s0:s1, h, :])
            np.testing.assert_allclose(o[s0:s1, h, :], ref, rtol=1e-12, atol=1e-12)


def test_identity_mfalcon_zero_bias_is_masked_matmul():
    n, c = 11, 6
    off, q, k, v, ts = _rand_batch(2, [n + c], 2, 4)
    o = oracle.attn(q, k, v, off, ts, np.zeros(8), np.zeros(32), 1.0,
                    num_candidates=[c], act=oracle.ACT_IDENTITY)
    M = np.zeros((n + c, n + c))
    M[:n, :n] = np.tril(np.ones((n, n)))
    M[n:, :n] = 1.0
    M[np.arange(n, n + c), np.arange(n, n + c)] = 1.0
    for h in range(2):
        ref = (M * (q[:, h] @ k[:, h].T)) @ v[:, h]
        np.testing.assert_allclose(o[:, h], ref, rtol=1e-12, atol=1e-12)


def test_position_bias_decodes_clamped_offsets():
    """Q = K = 0, V = 1, rab_pos[p] = 2^p: O_i = sum_{j<=i} 2^min(i-j, P-1)."""
    L, P = 12, 5
    q = np.zeros((L, 1, 1)); k = np.zeros((L, 1, 1)); v = np.ones((L, 1, 1))
    ts = np.arange(L, dtype=np.int64)
    o = oracle.attn(q, k, v, [0, L], ts, 2.0 ** np.arange(P), np.zeros(32), 1.0,
                    act=oracle.ACT_IDENTITY)[:, 0, 0]
    for i in range(L):
        want = (2 ** (i + 1) - 1) if i < P - 1 else (2 ** (P - 1) - 1) + (i - (P - 2)) * 2 ** (P - 1)
        assert o[i] == want, i


@pytest.mark.parametrize("sign", [1, -1])
def test_time_bias_decodes_log2_buckets(sign):
    """ts_j = sign * 2^j: for j < i, |t_i - t_j| = 2^i - 2^j has bit length i,
    so row i sees i keys in bucket min(NT-1, i) and itself in bucket 0."""
    L, NT = 12, 8
    rt = 3.0 ** np.arange(NT)
    q = np.zeros((L, 1, 1)); k = np.zeros((L, 1, 1)); v = np.ones((L, 1, 1))
    ts = sign * (2 ** np.arange(L, dtype=np.int64))
    o = oracle.attn(q, k, v, [0, L], ts, np.zeros(4), rt, 1.0, act=oracle.ACT_IDENTITY)[:, 0, 0]
    for i in range(L):
        assert o[i] == i * rt[min(NT - 1, i)] + rt[0], i


def test_integer_inputs_exact_against_rational_arithmetic():
    """Identity activation, integer inputs, power-of-two alpha: the oracle's
    result equals exact rational arithmetic of alpha * (M . (QK^T + R)) V,
    with R assembled from the (separately pinned) bucket functions."""
    lengths = [6, 9]
    off, q, k, v, ts = _rand_batch(3, lengths, 2, 3, ints=True)
    rp = np.array([1, -2, 3, 5, -7, 11], dtype=np.float64)
    rt = np.array([0, 1, -1, 2, -2, 4, -4, 8] * 4, dtype=np.float64)
    alpha = 0.25
    o = oracle.attn(q, k, v, off, ts, rp, rt, alpha, act=oracle.ACT_IDENTITY)
    for b, L in enumerate(lengths):
        base = int(off[b])
        for h in range(2):
            for i in range(L):
                acc = [Fraction(0)] * 3
                for j in range(i + 1):
                    s = sum(Fraction(int(q[base + i, h, c])) * int(k[base + j, h, c]) for c in range(3))
                    s += Fraction(rp[oracle.pos_bucket(i, j, L, len(rp))])
                    s += Fraction(rt[oracle.time_bucket(ts[base + i], ts[base + j], len(rt))])
                    for c in range(3):
                        acc[c] += s * int(v[base + j, h, c])
                for c in range(3):
                    assert o[base + i, h, c] == float(Fraction(1, 4) * acc[c])


def test_per_head_tables():
    lengths = [7]
    off, q, k, v, ts = _rand_batch(4, lengths, 2, 4)
    rp = np.random.default_rng(0).normal(size=(2, 8))
    rt = np.random.default_rng(1).normal(size=(2, 32))
    both = oracle.attn(q, k, v, off, ts, rp, rt, 0.5)
    for h in range(2):
        one = oracle.attn(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], off, ts, rp[h], rt[h], 0.5)
        np.testing.assert_array_equal(both[:, h:h + 1], one)


# ---------------------------------------------------------------------------
# invariants named by the method
# ---------------------------------------------------------------------------
def test_causality_future_rows_do_not_matter():
    x = synth.config(1)
    o = oracle.attn(x.q, x.k, x.v, x.offsets, x.ts, x.rab_pos, x.rab_time, x.alpha)
    rng = np.random.default_rng(9)
    for b in range(x.B):
        L = int(x.offsets[b + 1] - x.offsets[b])
        cut = L // 2
        lo = int(x.offsets[b]) + cut + 1
        hi = int(x.offsets[b + 1])
        q2, k2, v2, ts2 = x.q.copy(), x.k.copy(), x.v.copy(), x.ts.copy()
        q2[lo:hi] = rng.normal(size=q2[lo:hi].shape)
        k2[lo:hi] = rng.normal(size=k2[lo:hi].shape)
        v2[lo:hi] = rng.normal(size=v2[lo:hi].shape)
        ts2[lo:hi] += 10_000
        o2 = oracle.attn(q2, k2, v2, x.offsets, ts2, x.rab_pos, x.rab_time, x.alpha)
        assert np.array_equal(o[:lo], o2[:lo])


def test_mfalcon_candidate_equals_single_candidate_run():
    x = synth.config(4, batch=2, max_len=24)
    o = oracle.attn(x.q, x.k, x.v, x.offsets, x.ts, x.rab_pos, x.rab_time, x.alpha,
                    num_candidates=x.num_candidates)
    sc = oracle.mfalcon_score(x.q, x.k, x.v, x.u, x.offsets, x.num_candidates, x.ts,
                              x.rab_pos, x.rab_time, x.alpha, x.w)
    for b in range(x.B):
        s0 = int(x.offsets[b]); L = int(x.offsets[b + 1]) - s0
        c = int(x.num_candidates[b]); n = L - c
        for cand in range(c):
            rows = list(range(s0, s0 + n)) + [s0 + n + cand]
            sub = lambda a: a[rows]
            o1 = oracle.attn(sub(x.q), sub(x.k), sub(x.v), [0, n + 1], sub(x.ts), x.rab_pos,
                             x.rab_time, x.alpha, num_candidates=[1])
            assert np.array_equal(o1[n], o[s0 + n + cand])
            assert np.array_equal(o1[:n], o[s0:s0 + n])    # history unaffected by candidates
            s1 = oracle.mfalcon_score(sub(x.q), sub(x.k), sub(x.v), sub(x.u), [0, n + 1], [1],
                                      sub(x.ts), x.rab_pos, x.rab_time, x.alpha, x.w)
            assert s1[0, 0] == sc[b, cand]


def test_padding_invariance():
    x = synth.config(1)
    o = oracle.attn(x.q, x.k, x.v, x.offsets, x.ts, x.rab_pos, x.rab_time, x.alpha)
    L = np.diff(x.offsets)
    pad = np.array([3, 0, 5, 1])
    off_p = np.concatenate([[0], np.cumsum(L + pad)]).astype(np.int32)
    Tp = int(off_p[-1])

    def padded(a, fill):
        out = np.full((Tp,) + a.shape[1:], fill, dtype=a.dtype)
        for b in range(x.B):
            out[off_p[b]:off_p[b] + L[b]] = a[x.offsets[b]:x.offsets[b + 1]]
        return out
    sentinel = np.full((Tp, x.H, x.d), 123.0)
    op = oracle.attn(padded(x.q, np.nan), padded(x.k, np.nan), padded(x.v, np.nan), off_p,
                     padded(x.ts, -(2**62)), x.rab_pos, x.rab_time, x.alpha, lengths=L,
                     out=sentinel)
    for b in range(x.B):
        assert np.array_equal(op[off_p[b]:off_p[b] + L[b]], o[x.offsets[b]:x.offsets[b + 1]])
        assert np.all(op[off_p[b] + L[b]:off_p[b + 1]] == 123.0)


def test_batch_is_concatenation_of_sequences():
    x = synth.config(1)
    o = oracle.attn(x.q, x.k, x.v, x.offsets, x.ts, x.rab_pos, x.rab_time, x.alpha)
    for b in range(x.B):
        s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
        ob = oracle.attn(x.q[s0:s1], x.k[s0:s1], x.v[s0:s1], [0, s1 - s0], x.ts[s0:s1],
                         x.rab_pos, x.rab_time, x.alpha)
        assert np.array_equal(ob, o[s0:s1])


# ---------------------------------------------------------------------------
# LayerNorm gate and the layer
# ---------------------------------------------------------------------------
def test_ln_gate_matches_torch_layer_norm():
    import torch
    rng = np.random.default_rng(5)
    o = rng.normal(0, 0.01, size=(40, 512))
    u = rng.normal(0, 0.5, size=(40, 512))
    y = oracle.ln_gate(o, u, eps=1e-5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(o), (512,), eps=1e-5).numpy() * u
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)
    # U = 1: zero mean and variance var/(var+eps) per row
    y1 = oracle.ln_gate(o, np.ones_like(o), eps=1e-5)
    var = o.var(axis=1)
    np.testing.assert_allclose(y1.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose(y1.var(axis=1), var / (var + 1e-5), rtol=1e-10)
    assert np.all(oracle.ln_gate(np.full((2, 8), 3.0), np.ones((2, 8))) == 0.0)


def test_layer_is_composition_of_library_routines():
    """f1 by numpy matmul, SiLU by scipy's logistic, attention by the pinned
    oracle attention, LayerNorm by torch, f2 by numpy matmul."""
    import torch
    from scipy.special import expit
    x = synth.config(5, batch=3, max_len=20)
    l = 1
    H, d, D = x.H, x.d, x.D
    out = oracle.layer(x.x, x.w1[l], x.w2[l], x.offsets, x.ts, x.rab_pos[l], x.rab_time[l],
                       x.alpha, H, d)
    X = x.x.astype(np.float64)
    z = X @ x.w1[l].astype(np.float64).T
    z = z * expit(z)
    hd = H * d
    U, V, Q, K = (z[:, i * hd:(i + 1) * hd] for i in range(4))
    T = X.shape[0]
    O = oracle.attn(Q.reshape(T, H, d), K.reshape(T, H, d), V.reshape(T, H, d), x.offsets, x.ts,
                    x.rab_pos[l], x.rab_time[l], x.alpha).reshape(T, hd)
    Y = torch.nn.functional.layer_norm(torch.from_numpy(O), (hd,), eps=x.eps).numpy() * U
    ref = X + Y @ x.w2[l].astype(np.float64).T
    np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-9)


def test_layer_biases():
    x = synth.config(5, batch=2, max_len=10)
    rng = np.random.default_rng(3)
    b1 = rng.normal(size=4 * x.H * x.d); b2 = rng.normal(size=x.D)
    out = oracle.layer(x.x, x.w1[0], x.w2[0], x.offsets, x.ts, x.rab_pos[0], x.rab_time[0],
                       x.alpha, x.H, x.d, b1=b1, b2=b2)
    # zeroing W2 leaves X + b2
    out0 = oracle.layer(x.x, x.w1[0], np.zeros_like(x.w2[0]), x.offsets, x.ts, x.rab_pos[0],
                        x.rab_time[0], x.alpha, x.H, x.d, b1=b1, b2=b2)
    np.testing.assert_allclose(out0, x.x + b2[None, :], rtol=0, atol=0)
    assert not np.allclose(out, out0)


# ---------------------------------------------------------------------------
# tiles
# ---------------------------------------------------------------------------
def test_tiles_cover_every_visible_pair_and_nothing_else():
    x = synth.config(4, batch=2, max_len=40)
    BM, BN = 16, 8
    t = oracle.tiles(x.offsets, BM, BN, num_candidates=x.num_candidates)
    got = set(map(tuple, t.tolist()))
    want = set()
    for b in range(x.B):
        L = int(x.offsets[b + 1] - x.offsets[b]); n = L - int(x.num_candidates[b])
        for i in range(L):
            for j in range(L):
                if (i < n and j <= i) or (i >= n and (j < n or j == i)):
                    want.add((b, i // BM, j // BN))
    assert got == want


def test_attn_rows_equals_full_oracle_at_those_rows():
    """The row-by-row entry (for batches too large for the full oracle) gives
    exactly the full oracle's values at the selected rows: padded rows,
    candidates, per-head tables, rows from every sequence, repeated rows."""
    x = synth.make_attn(81, [37, 1, 90, 64], H=2, d=16, P=40, NT=12, alpha=0.125, dtype="f32",
                        num_candidates=[5, 0, 30, 64])
    rng = np.random.default_rng(82)
    rp = rng.normal(0, 0.1, size=(2, 40))
    rt = rng.normal(0, 0.1, size=(2, 12))
    full = oracle.attn(x.q, x.k, x.v, x.offsets, x.ts, rp, rt, x.alpha,
                       num_candidates=x.num_candidates)
    rows = np.array([0, 36, 37, 38, 50, 127, 128, 191, 60, 0])
    got = oracle.attn_rows(x.q, x.k, x.v, x.offsets, x.ts, rp, rt, x.alpha, rows,
                           num_candidates=x.num_candidates)
    assert np.array_equal(got, full[rows])
    got_id = oracle.attn_rows(x.q, x.k, x.v, x.offsets, x.ts, rp, rt, x.alpha, rows,
                              num_candidates=x.num_candidates, act=oracle.ACT_IDENTITY)
    full_id = oracle.attn(x.q, x.k, x.v, x.offsets, x.ts, rp, rt, x.alpha,
                          num_candidates=x.num_candidates, act=oracle.ACT_IDENTITY)
    assert np.array_equal(got_id, full_id[rows])


def test_layer_scores_are_composition_of_library_routines():
    """The scoring layer: f1 (+ b1) by numpy matmul, SiLU by scipy's
    logistic, the split U | V | Q | K, then the scores by the library route
    (pinned attention, torch's layer_norm, the gate, numpy's dot with w); a
    sequence without candidates and one of candidates only included."""
    from scipy.special import expit
    rng = np.random.default_rng(85)
    H, d, D = 2, 16, 32
    lengths, cands = [20, 9, 6, 13], [4, 0, 6, 1]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(off[-1])
    X = rng.normal(0, 0.5, size=(T, D))
    w1 = rng.uniform(-0.3, 0.3, size=(4 * H * d, D))
    b1 = rng.normal(0, 0.1, size=4 * H * d)
    ts = np.concatenate([np.cumsum(rng.integers(1, 500, size=L)) for L in lengths]).astype(np.int64)
    rp = rng.normal(0, 0.1, size=24)
    rt = rng.normal(0, 0.1, size=16)
    w = rng.normal(0, 1.0 / np.sqrt(H * d), size=H * d)
    got = oracle.layer_scores(X, w1, off, cands, ts, rp, rt, 0.05, w, H, d, b1=b1)
    z = X @ w1.T + b1
    z = z * expit(z)
    hd = H * d
    U, V, Q, K = (z[:, i * hd:(i + 1) * hd].reshape(T, H, d) for i in range(4))
    ref = _scores_by_library_route(Q, K, V, U, off, cands, ts, rp, rt, 0.05, w, 1e-5)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    assert got.shape == (4, 6)


# ---------------------------------------------------------------------------
# M-FALCON scores
# ---------------------------------------------------------------------------
def _scores_by_library_route(q, k, v, u, off, cands, ts, rp, rt, alpha, w, eps):
    """Scores without the oracle's score step: the pinned attention, torch's
    layer_norm over the H*d_v values of a row, the U gate, then numpy's dot
    with w at each candidate row n_b + c."""
    import torch
    T, H, d = q.shape
    O = oracle.attn(q, k, v, off, ts, rp, rt, alpha, num_candidates=cands).reshape(T, H * d)
    Y = torch.nn.functional.layer_norm(torch.from_numpy(O), (H * d,), eps=eps).numpy()
    Y = Y * u.reshape(T, H * d)
    B = len(off) - 1
    ref = np.zeros((B, max(1, int(np.max(cands)))))
    for b in range(B):
        n = int(off[b + 1] - off[b]) - int(cands[b])
        for c in range(int(cands[b])):
            ref[b, c] = Y[int(off[b]) + n + c] @ w
    return ref[:, :int(np.max(cands))]


def test_golden_mfalcon_score():
    """Hand-worked scores (closed forms in ln 3 through sigma(ln 3) = 3/4)."""
    g = _load("mfalcon_score_ln3_4x4.json")
    env = {"ln3": math.log(3), "sqrt": math.sqrt}
    T, H, d = g["offsets"][-1], g["H"], g["d"]
    arr = lambda key: np.array(g[key], dtype=np.float64).reshape(T, H, d)
    rp = np.array([eval(str(x), env) for x in g["rab_pos"]], dtype=np.float64)
    rt = np.array(g["rab_time"], dtype=np.float64)
    got = oracle.mfalcon_score(arr("q"), arr("k"), arr("v"), arr("u"), g["offsets"],
                               g["num_candidates"], np.array(g["ts"], dtype=np.int64), rp, rt,
                               g["alpha"], np.array(g["w"], dtype=np.float64), eps=g["eps"])
    exp = np.array([[eval(s, env) for s in g["expected_scores"]]])
    np.testing.assert_allclose(got, exp, rtol=1e-13, atol=0)


def test_mfalcon_score_matches_library_route():
    """Users with no candidates, only candidates, one candidate, and
    candidates that start inside a 32- or 128-row block; per-row U and an
    asymmetric w, so a dropped gate, a reversed or rescaled w, or a score
    read at the wrong row changes the result."""
    rng = np.random.default_rng(86)
    H, d = 2, 8
    lengths = [45, 9, 6, 140, 1, 33]
    cands = [6, 0, 6, 12, 1, 1]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(off[-1])
    q, k, v, u = (rng.normal(0, 0.5, size=(T, H, d)) for _ in range(4))
    ts = np.zeros(T, dtype=np.int64)
    for b, L in enumerate(lengths):
        n = L - cands[b]
        t = np.cumsum(rng.integers(1, 400, size=L)).astype(np.int64)
        if cands[b] and n:
            t[n:] = t[n - 1]
        ts[off[b]:off[b + 1]] = t
    rp = rng.normal(0, 0.1, size=64)
    rt = rng.normal(0, 0.1, size=32)
    w = rng.normal(0, 1.0 / np.sqrt(H * d), size=H * d)
    got = oracle.mfalcon_score(q, k, v, u, off, cands, ts, rp, rt, 1 / 160, w)
    ref = _scores_by_library_route(q, k, v, u, off, cands, ts, rp, rt, 1 / 160, w, 1e-5)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)
    # entries past a user's candidate count are never written
    assert np.all(got[1] == 0.0) and np.all(got[4, 1:] == 0.0)
