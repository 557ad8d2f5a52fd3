"""GPU parity of the attention gradients (hstu_attn_bwd, bf16, d = 128)
against the fp64 oracle's chain rule on the same seeded bf16 inputs."""
import numpy as np
import pytest

import hstu_synth as synth
import oracle
from hstu_testlib import DeviceAttn, assert_close, dev_tensor, host_f32, log, valid_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hstu_sequential_transducer_causal_amd import _lib
    _lib.load()


def _run_bwd(d: DeviceAttn, g, act=0, **kw):
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    out = ops.hstu_attn_bwd(d.q, d.k, d.v, d.offsets, d.ts, d.rab_pos, d.rab_time, d.x.alpha,
                            max_seq_len=d.max_seq_len, dout=g, seq_lengths=d.lengths,
                            num_candidates=d.ncand, act=act, **kw)
    torch.cuda.synchronize()
    return out


def _check(x, what, act=0, seed=101):
    log(f"{what}: B={x.B} T={x.T} H={x.H}")
    d = DeviceAttn(x)
    gnp = synth.upstream_grad(seed, x.v.shape)
    g = dev_tensor(gnp, "bf16")
    dq, dk, dv, _, drp, drt = _run_bwd(d, g, act=act)
    rq, rk, rv, rrp, rrt = oracle.attn_bwd(x.q, x.k, x.v, x.offsets, x.ts, x.rab_pos, x.rab_time,
                                           x.alpha, gnp, lengths=x.lengths,
                                           num_candidates=x.num_candidates, act=act)
    rows = valid_rows(x)
    assert_close(host_f32(dq)[rows], rq[rows], "bf16", f"{what} dQ")
    assert_close(host_f32(dk)[rows], rk[rows], "bf16", f"{what} dK")
    assert_close(host_f32(dv)[rows], rv[rows], "bf16", f"{what} dV")
    assert_close(host_f32(drp), rrp, "bf16", f"{what} d rab_pos")
    assert_close(host_f32(drt), rrt, "bf16", f"{what} d rab_time")
    return dq, dk, dv, drp, drt


def test_bwd_ragged_causal_clamped_positions():
    x = synth.make_attn(61, [1, 63, 64, 65, 130, 300], H=2, d=128, P=70, NT=32, alpha=1 / 256,
                        dtype="bf16")
    _check(x, "bwd ragged causal P=70")


def test_bwd_more_sequences_than_the_scheduler_keeps_in_lds():
    """4200 short sequences (1..48 rows): both work lists and the G-block
    prefix past the scheduler's LDS copies."""
    rng = np.random.default_rng(79)
    lengths = rng.integers(1, 49, size=4200).tolist()
    x = synth.make_attn(80, lengths, H=1, d=128, P=64, NT=32, alpha=1 / 128, dtype="bf16")
    _check(x, "bwd 4200 short sequences")


def test_bwd_three_heads():
    """An odd head count: entries of the work list spread over the eight
    per-die queues with the head rotated by the sequence; every head's
    outputs and the per-head tables' gradients against the oracle."""
    x = synth.make_attn(64, [50, 130, 7, 260, 1], H=3, d=128, P=256, NT=32, alpha=1 / 256,
                        dtype="bf16")
    x.rab_pos = np.stack([x.rab_pos, x.rab_pos[::-1].copy(), 0.5 * x.rab_pos]).astype(np.float32)
    _check(x, "bwd three heads, per-head position tables")


def test_bwd_mfalcon_edge_counts():
    x = synth.make_attn(62, [70, 70, 200, 129, 64, 300], H=2, d=128, P=1024, NT=32, alpha=1 / 256,
                        dtype="bf16", num_candidates=[0, 70, 1, 65, 63, 150])
    _check(x, "bwd M-FALCON edge counts")


def test_bwd_identity_activation():
    x = synth.make_attn(63, [5, 200, 131], H=2, d=128, P=300, NT=32, alpha=1 / 256, dtype="bf16",
                        qkv_std=0.1)
    _check(x, "bwd identity", act=1)


def test_bwd_per_head_tables_and_wide_timestamps():
    x = synth.make_attn(64, [150, 260], H=3, d=128, P=200, NT=32, alpha=1 / 256, dtype="bf16",
                        mean_gap=float(2 ** 26))
    x.ts[x.offsets[1] + 100:] += 2 ** 31     # a jump inside the second sequence
    rng = np.random.default_rng(1)
    x.rab_pos = rng.normal(0, 0.1, size=(3, 200)).astype(np.float32)
    x.rab_time = rng.normal(0, 0.1, size=(3, 32)).astype(np.float32)
    _check(x, "bwd per-head tables, wide timestamps")


def test_bwd_padding_rows_untouched_and_never_read():
    import torch
    x = synth.make_attn(65, [200, 90, 129], H=2, d=128, P=64, NT=32, alpha=1 / 64, dtype="bf16")
    x.lengths = np.array([150, 0, 129], dtype=np.int32)
    pads = np.setdiff1d(np.arange(x.T), valid_rows(x))
    for a in (x.q, x.k, x.v):
        a[pads] = np.nan
    d = DeviceAttn(x)
    gnp = synth.upstream_grad(7, x.v.shape)
    gnp[pads] = np.nan
    g = dev_tensor(gnp, "bf16")
    sentinel = [torch.full_like(d.q, 3.0) for _ in range(3)]
    dq, dk, dv, _, drp, drt = _run_bwd(d, g, dq=sentinel[0], dk=sentinel[1], dv=sentinel[2])
    for t, name in [(dq, "dQ"), (dk, "dK"), (dv, "dV")]:
        h = host_f32(t)
        assert np.all(h[pads] == 3.0), f"{name} pad rows written"
        assert np.all(np.isfinite(h[valid_rows(x)])), f"{name} NaN leaked"
    gz = np.nan_to_num(gnp)
    xz = synth.make_attn(65, [200, 90, 129], H=2, d=128, P=64, NT=32, alpha=1 / 64, dtype="bf16")
    rq, rk, rv, rrp, rrt = oracle.attn_bwd(xz.q, xz.k, xz.v, xz.offsets, xz.ts, xz.rab_pos,
                                           xz.rab_time, xz.alpha, gz, lengths=x.lengths)
    rows = valid_rows(x)
    assert_close(host_f32(dq)[rows], rq[rows], "bf16", "padded dQ")
    assert_close(host_f32(dk)[rows], rk[rows], "bf16", "padded dK")
    assert_close(host_f32(dv)[rows], rv[rows], "bf16", "padded dV")
    assert_close(host_f32(drp), rrp, "bf16", "padded d rab_pos")
    assert_close(host_f32(drt), rrt, "bf16", "padded d rab_time")


def test_bwd_through_the_gate():
    """Upstream gradient of Y = LN(O) * U: dO and dU come from the gate's
    derivative first (O here is a seeded stand-in for the forward's output)."""
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    x = synth.make_attn(66, [100, 257, 33], H=4, d=128, P=1024, NT=32, alpha=1 / 512, dtype="bf16")
    d = DeviceAttn(x)
    onp = synth.upstream_grad(8, x.v.shape, std=0.02)
    dynp = synth.upstream_grad(9, x.v.shape)
    o, dy = dev_tensor(onp, "bf16"), dev_tensor(dynp, "bf16")
    dq, dk, dv, du, drp, drt = ops.hstu_attn_bwd(
        d.q, d.k, d.v, d.offsets, d.ts, d.rab_pos, d.rab_time, x.alpha, max_seq_len=d.max_seq_len,
        dy=dy, o=o, u=d.u, ln_eps=x.eps)
    torch.cuda.synchronize()
    T = x.T
    rdo, rdu = oracle.ln_gate_bwd(onp.reshape(T, -1), x.u.reshape(T, -1), dynp.reshape(T, -1),
                                  eps=x.eps)
    assert_close(host_f32(du).reshape(T, -1), rdu, "bf16", "gate dU")
    rq, rk, rv, rrp, rrt = oracle.attn_bwd(x.q, x.k, x.v, x.offsets, x.ts, x.rab_pos, x.rab_time,
                                           x.alpha, rdo.reshape(x.v.shape))
    assert_close(host_f32(dq), rq, "bf16", "gate path dQ")
    assert_close(host_f32(dk), rk, "bf16", "gate path dK")
    assert_close(host_f32(dv), rv, "bf16", "gate path dV")
    assert_close(host_f32(drp), rrp, "bf16", "gate path d rab_pos")
    assert_close(host_f32(drt), rrt, "bf16", "gate path d rab_time")


def test_bwd_run_to_run_identical():
    x = synth.config(2, batch=5, max_len=400)
    d = DeviceAttn(x)
    g = dev_tensor(synth.upstream_grad(10, x.v.shape), "bf16")
    a = [host_f32(t) for t in _run_bwd(d, g) if t is not None]
    b = [host_f32(t) for t in _run_bwd(d, g) if t is not None]
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


@pytest.mark.parametrize("cfg", [3, 4])
def test_bwd_full_size(cfg):
    """The full long-sequence (3) and M-FALCON (4) workloads, every output
    against the oracle."""
    x = synth.config(cfg)
    _check(x, f"bwd cfg{cfg} full size", seed=200 + cfg)


def test_bwd_table_gradients_bucket_by_bucket():
    """M-FALCON users of many shapes (so that workgroups take candidate-row
    blocks and history-row blocks one after the other), no clamped bucket to
    dominate, and the table gradients checked bucket by bucket.  G reaches
    the histograms to within 2^-17 of itself (two bf16 halves) from exact
    bf16 inputs and is summed in fp32, so every bucket must match the oracle
    far below the bf16 output bound: a stale scratch cell from a previous
    block would show in its bucket."""
    rng = np.random.default_rng(107)
    B = 24
    lengths = rng.integers(40, 420, size=B)
    cands = np.minimum(lengths, rng.integers(1, 200, size=B))
    cands[::5] = lengths[::5]          # users with candidates only
    x = synth.make_attn(108, lengths.tolist(), H=2, d=128, P=1024, NT=32, alpha=1 / 512,
                        dtype="bf16", num_candidates=cands.tolist())
    d = DeviceAttn(x)
    gnp = synth.upstream_grad(109, x.v.shape)
    g = dev_tensor(gnp, "bf16")
    _, _, _, _, drp, drt = _run_bwd(d, g)
    _, _, _, rrp, rrt = oracle.attn_bwd(x.q, x.k, x.v, x.offsets, x.ts, x.rab_pos, x.rab_time,
                                        x.alpha, gnp, num_candidates=x.num_candidates)
    for got, ref, name in ((host_f32(drp), rrp, "d rab_pos"), (host_f32(drt), rrt, "d rab_time")):
        scale = float(np.abs(ref).max())
        err = np.abs(got.astype(np.float64) - ref)
        worst = int(err.argmax())
        log(f"{name} bucket by bucket: max err / max|ref| = {err.max() / scale:.3e} at bucket {worst}"
            f" (ref {ref[worst]:.4e}, got {got[worst]:.4e})")
        assert np.all(err <= 1e-3 * scale + 1e-3 * np.abs(ref)), name
