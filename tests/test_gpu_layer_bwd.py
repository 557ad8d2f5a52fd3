"""GPU parity of the layer gradients (hstu_layer_bwd: f2 + residual, gate,
attention, f1 + SiLU) against the fp64 oracle on the same seeded bf16
inputs."""
import numpy as np
import pytest

import hstu_synth as synth
import oracle
from hstu_testlib import assert_close, dev_tensor, host_f32, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hstu_sequential_transducer_causal_amd import _lib
    _lib.load()


def _biases(x: synth.LayerInputs, seed: int):
    zw = 4 * x.H * x.d
    return (synth.upstream_grad(seed, (zw,), std=0.1, dtype="f32"),
            synth.upstream_grad(seed + 1, (x.D,), std=0.1, dtype="f32"))


def _run(x: synth.LayerInputs, g: np.ndarray, l=0, biases=None):
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    xd = dev_tensor(x.x, "bf16")
    gd = dev_tensor(g, "bf16")
    off = torch.from_numpy(x.offsets.astype(np.int32)).cuda()
    ts = torch.from_numpy(x.ts).cuda()
    b1 = b2 = None
    if biases is not None:
        b1, b2 = (torch.from_numpy(b.astype(np.float32)).cuda() for b in biases)
    out = ops.hstu_layer_bwd(xd, dev_tensor(x.w1[l], "bf16"), dev_tensor(x.w2[l], "bf16"), off, ts,
                             torch.from_numpy(x.rab_pos[l]).cuda(),
                             torch.from_numpy(x.rab_time[l]).cuda(), x.alpha, gd, H=x.H, d=x.d,
                             max_seq_len=int(np.diff(x.offsets).max()), b1=b1, b2=b2, ln_eps=x.eps)
    torch.cuda.synchronize()
    return {k: (None if v is None else host_f32(v)) for k, v in out.items()}


def _check(x, what, l=0, seed=300, biases=None):
    log(f"{what}: B={x.B} T={x.T} D={x.D} H={x.H}")
    g = synth.upstream_grad(seed, x.x.shape)
    got = _run(x, g, l, biases)
    b1, b2 = biases if biases is not None else (None, None)
    ref = oracle.layer_bwd(x.x, x.w1[l], x.w2[l], x.offsets, x.ts, x.rab_pos[l], x.rab_time[l],
                           x.alpha, x.H, x.d, g, b1=b1, b2=b2, eps=x.eps)
    for k in ("dx", "dw1", "db1", "dw2", "db2", "drab_pos", "drab_time"):
        assert_close(got[k], ref[k], "bf16", f"{what} {k}")
    return got


def test_layer_bwd_ragged_rows():
    x = synth.make_layer_stack(71, [1, 77, 130], H=4, d=128, D=512, layers=1, P=1024, NT=32,
                               alpha=1 / 256)
    _check(x, "layer bwd ragged")


def test_layer_bwd_with_biases():
    x = synth.make_layer_stack(72, [200, 33, 300], H=4, d=128, D=512, layers=1, P=1024, NT=32,
                               alpha=1 / 512)
    _check(x, "layer bwd biases", biases=_biases(x, 5))


def test_layer_bwd_cfg5_reduced_second_layer():
    x = synth.config(5, batch=3, max_len=400)
    _check(x, "layer bwd cfg5 reduced, layer 1", l=1)


def test_layer_bwd_run_to_run_identical():
    x = synth.make_layer_stack(73, [150, 260], H=4, d=128, D=512, layers=1, P=1024, NT=32,
                               alpha=1 / 256)
    g = synth.upstream_grad(9, x.x.shape)
    a, b = _run(x, g), _run(x, g)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


def _subset(x: synth.LayerInputs, seqs):
    """The layer inputs of sequences ``seqs`` alone (packed, offsets rebased)."""
    import dataclasses
    rows = np.concatenate([np.arange(x.offsets[b], x.offsets[b + 1]) for b in seqs])
    L = [int(x.offsets[b + 1] - x.offsets[b]) for b in seqs]
    off = np.zeros(len(seqs) + 1, dtype=np.int32)
    off[1:] = np.cumsum(L)
    return dataclasses.replace(x, B=len(seqs), offsets=off, x=x.x[rows], ts=x.ts[rows]), rows


def test_layer_bwd_full_size_first_layer():
    """Workload 5 at full size (32 sequences of 512..4096 rows), first layer.
    Three full-length sequences (the shortest, the longest and one more) as a
    batch of their own against the oracle, every output: dX and the parameter
    and table gradients, which sum over the batch's tokens.  In the full
    batch, dX of a sequence depends on that sequence alone (the same three
    against the same oracle run); the parameter gradients sum over sequences,
    so the full batch's equal the sum of its two halves', and db2 is the token
    sum of dX_out."""
    x = synth.config(5)
    g = synth.upstream_grad(310, x.x.shape)
    log(f"layer bwd cfg5 full size: B={x.B} T={x.T}")
    full = _run(x, g)
    L = np.diff(x.offsets)
    seqs = sorted({int(np.argmin(L)), int(np.argmax(L)), 3})
    xs, rows = _subset(x, seqs)
    sub = _run(xs, g[rows])
    ref = oracle.layer_bwd(xs.x, xs.w1[0], xs.w2[0], xs.offsets, xs.ts, xs.rab_pos[0], xs.rab_time[0],
                           xs.alpha, xs.H, xs.d, g[rows], eps=xs.eps)
    what = f"cfg5 sequences {seqs} (L={[int(L[b]) for b in seqs]})"
    for k in ("dx", "dw1", "db1", "dw2", "db2", "drab_pos", "drab_time"):
        assert_close(sub[k], ref[k], "bf16", f"{what} {k}")
    assert_close(full["dx"][rows], ref["dx"], "bf16", f"{what} dx in the full batch")
    np.testing.assert_allclose(full["db2"], g.astype(np.float64).sum(axis=0),
                               rtol=1e-4, atol=1e-3 * float(np.abs(g).sum(axis=0).max()))
    half = x.B // 2
    xa, ra = _subset(x, list(range(half)))
    xb, rb = _subset(x, list(range(half, x.B)))
    pa, pb = _run(xa, g[ra]), _run(xb, g[rb])
    for k in ("dw1", "db1", "dw2", "db2", "drab_pos", "drab_time"):
        assert_close(full[k], pa[k].astype(np.float64) + pb[k], "bf16", f"cfg5 {k} = sum of halves")


def test_layer_saved_pair_equals_recomputation():
    """hstu_layer_fwd_saved gives hstu_layer_fwd's X_out bit for bit, and
    hstu_layer_bwd_saved (reading the kept Z, pre-activation, O, Y) gives
    hstu_layer_bwd's gradients bit for bit (both run the same kernels on the
    same inputs; the saved pair only skips the recomputation)."""
    import torch
    from hstu_sequential_transducer_causal_amd import _lib, ops
    x = synth.make_layer_stack(75, [1, 300, 77, 512], H=4, d=128, D=512, layers=1, P=1024, NT=32,
                               alpha=1 / 512)
    b1, b2 = (torch.from_numpy(b.astype(np.float32)).cuda() for b in _biases(x, 76))
    g = synth.upstream_grad(77, x.x.shape)
    xd = dev_tensor(x.x, "bf16")
    w1, w2 = dev_tensor(x.w1[0], "bf16"), dev_tensor(x.w2[0], "bf16")
    off = torch.from_numpy(x.offsets.astype(np.int32)).cuda()
    ts = torch.from_numpy(x.ts).cuda()
    rp, rt = torch.from_numpy(x.rab_pos[0]).cuda(), torch.from_numpy(x.rab_time[0]).cuda()
    kw = dict(H=x.H, d=x.d, max_seq_len=int(np.diff(x.offsets).max()))
    need = ops.layer_saved_bytes(xd, w1, w2, off, ts, rp, rt, x.alpha, **kw)
    T, hd = x.x.shape[0], x.H * x.d
    assert need >= 2 * T * 4 * hd * 2 + 2 * T * hd * 2
    saved = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")   # stale bytes everywhere
    plain = ops.hstu_layer_fwd(xd, w1, w2, off, ts, rp, rt, x.alpha, b1=b1, b2=b2, ln_eps=x.eps, **kw)
    kept = ops.hstu_layer_fwd(xd, w1, w2, off, ts, rp, rt, x.alpha, b1=b1, b2=b2, ln_eps=x.eps, saved=saved,
                              **kw)
    torch.cuda.synchronize()
    assert torch.equal(plain, kept)
    # X_out written over X would leave the gradients a wrong X: refused before any launch
    with pytest.raises(_lib.HstuError, match="overlap"):
        ops.hstu_layer_fwd(xd, w1, w2, off, ts, rp, rt, x.alpha, b1=b1, b2=b2, ln_eps=x.eps, saved=saved,
                           x_out=xd, **kw)
    gd = dev_tensor(g, "bf16")
    ref = ops.hstu_layer_bwd(xd, w1, w2, off, ts, rp, rt, x.alpha, gd, b1=b1, b2=b2, ln_eps=x.eps, **kw)
    got = ops.hstu_layer_bwd(xd, w1, w2, off, ts, rp, rt, x.alpha, gd, b1=b1, b2=b2, ln_eps=x.eps,
                             saved=saved, **kw)
    torch.cuda.synchronize()
    for k in ("dx", "dw1", "db1", "dw2", "db2", "drab_pos", "drab_time"):
        assert torch.equal(ref[k], got[k]), k
    log(f"saved pair: {need / 2**20:.1f} MiB kept, X_out and all gradients identical")
