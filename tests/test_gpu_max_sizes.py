"""GPU parity at the largest supported sizes: a sequence of the maximum length
(65 536 rows) beside a short one, checked on sampled rows against the oracle
evaluated row by row (each row depends on its own sequence's earlier rows
only), plus the LN * U gate on those rows."""
import numpy as np
import pytest

import hstu_synth as synth
import oracle
from hstu_testlib import DeviceAttn, assert_close, host_f32, log

pytestmark = pytest.mark.gpu

MAX_LEN = 65536   # the library's maximum sequence length


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _sample_rows(x, rng, per_seq=12):
    rows = []
    L = np.diff(x.offsets)
    for b in range(x.B):
        r0, n = int(x.offsets[b]), int(L[b])
        fixed = [0, 1, 31, 32, 127, 128, n // 2, n - 2, n - 1]
        rand = rng.choice(n, size=min(per_seq, n), replace=False)
        rows += [r0 + int(i) for i in fixed + list(rand) if 0 <= i < n]
    return np.unique(np.array(rows, dtype=np.int64))


@pytest.mark.parametrize("ncand", [None, [1024, 7]])
def test_max_length_sequence_sampled_rows(ncand):
    """One maximum-length sequence and a short one: causal, or with M-FALCON
    candidates (1024 on the long sequence).  Clamped positions (P = 1024 of
    65 535 possible offsets), the widest time buckets, split row blocks."""
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    x = synth.make_attn(91, [MAX_LEN, 300], H=2, d=128, P=1024, NT=32, alpha=1.0 / MAX_LEN,
                        dtype="bf16", num_candidates=ncand, mean_gap=600.0)
    log(f"max length: T = {x.T}, candidates {ncand}")
    d = DeviceAttn(x)
    o, y = ops.hstu_attn_fwd(d.q, d.k, d.v, d.offsets, d.ts, d.rab_pos, d.rab_time, x.alpha,
                             max_seq_len=MAX_LEN, num_candidates=d.ncand, u=d.u, ln_eps=x.eps)
    torch.cuda.synchronize()
    rows = _sample_rows(x, np.random.default_rng(92))
    ref = oracle.attn_rows(x.q, x.k, x.v, x.offsets, x.ts, x.rab_pos, x.rab_time, x.alpha, rows,
                           num_candidates=x.num_candidates)
    got = host_f32(o)[rows]
    assert_close(got, ref, "bf16", f"max length O ({len(rows)} rows)")
    yref = oracle.ln_gate(ref, x.u[rows], eps=x.eps)
    assert_close(host_f32(y)[rows].reshape(len(rows), -1), yref, "bf16", "max length Y")


@pytest.mark.parametrize("ncand", [None, [1024, 7]])
def test_max_length_gradients_sampled_rows(ncand):
    """Gradients (from dLoss/dO) of the same maximum-length batch: dQ at
    sampled query rows and dK, dV at sampled key rows against the oracle
    evaluated row by row.  (The table gradients sum over every pair of the
    sequence; they are checked at the smaller sizes.)"""
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    from hstu_testlib import dev_tensor
    x = synth.make_attn(93, [MAX_LEN, 300], H=2, d=128, P=1024, NT=32, alpha=1.0 / MAX_LEN,
                        dtype="bf16", num_candidates=ncand, mean_gap=600.0)
    g = synth.upstream_grad(94, x.v.shape)
    d = DeviceAttn(x)
    dq, dk, dv, _, _, _ = ops.hstu_attn_bwd(d.q, d.k, d.v, d.offsets, d.ts, d.rab_pos, d.rab_time,
                                            x.alpha, max_seq_len=MAX_LEN, dout=dev_tensor(g, "bf16"),
                                            num_candidates=d.ncand, want_rab=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(95)
    qrows = _sample_rows(x, rng)
    krows = _sample_rows(x, rng)
    rq, rk, rv = oracle.attn_bwd_rows(x.q, x.k, x.v, x.offsets, x.ts, x.rab_pos, x.rab_time, x.alpha,
                                      g, qrows, krows, num_candidates=x.num_candidates)
    assert_close(host_f32(dq)[qrows], rq, "bf16", f"max length dQ ({len(qrows)} rows)")
    assert_close(host_f32(dk)[krows], rk, "bf16", f"max length dK ({len(krows)} rows)")
    assert_close(host_f32(dv)[krows], rv, "bf16", f"max length dV ({len(krows)} rows)")
