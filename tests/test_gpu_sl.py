"""GPU parity of stochastic length (hstu_stochastic_length): the kept rows
and packed offsets bit-exact against the oracle's Philox-keyed selection,
and the gathered rows bit-exact against a plain index gather."""
import numpy as np
import pytest

import hstu_synth as synth
from oracle import stochastic_length as sl
from hstu_testlib import dev_tensor, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hstu_sequential_transducer_causal_amd import _lib
    _lib.load()


def _run(offsets, cap, seed, step, caps=None, tensors=()):
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    off = torch.from_numpy(np.asarray(offsets, dtype=np.int32)).cuda()
    cd = None if caps is None else torch.from_numpy(np.asarray(caps, dtype=np.int32)).cuda()
    oo, idx, outs = ops.stochastic_length(off, cap, seed=seed, step=step, caps=cd, tensors=tensors)
    torch.cuda.synchronize()
    oo = oo.cpu().numpy()
    return oo, idx.cpu().numpy()[:int(oo[-1])], outs


def _check(offsets, cap, seed, step, caps=None, what=""):
    oo, idx, _ = _run(offsets, cap, seed, step, caps)
    ref_off, ref_idx = sl.select(offsets, cap if caps is None else caps, seed=seed, step=step)
    assert np.array_equal(oo, ref_off), f"{what} offsets"
    assert np.array_equal(idx, ref_idx), f"{what} kept rows"
    log(f"{what}: {len(idx)} of {offsets[-1]} rows kept, bit-exact")


def test_sl_ragged_lengths_around_the_cap():
    L = [0, 1, 5, 6, 7, 31, 32, 33, 255, 256, 257, 600]
    off = np.concatenate([[0], np.cumsum(L)])
    for cap in (1, 6, 32, 256):
        _check(off, cap, seed=77, step=3, what=f"ragged cap {cap}")


def test_sl_per_sequence_caps_and_zero_cap():
    L = [50, 300, 1000, 17]
    off = np.concatenate([[0], np.cumsum(L)])
    _check(off, 0, seed=5, step=0, caps=[0, 299, 10, 17], what="per-sequence caps")
    _check(off, 0, seed=5, step=0, what="cap 0")


def test_sl_long_history_workload():
    """The long-sequence workload's raw lengths (lognormal, clipped to
    [1024, 8192]) under its cap floor(8192^0.85) = 2120, and the cap of
    another exponent (alpha = 1.6: floor(8192^0.8) = 1351)."""
    rng = np.random.default_rng(3)
    L = np.clip(np.round(rng.lognormal(np.log(3000), 0.5, size=16)), 1024, 8192).astype(int)
    off = np.concatenate([[0], np.cumsum(L)])
    for cap in (2120, 1351):
        _check(off, cap, seed=2024, step=17, what=f"long histories cap {cap}")


def test_sl_ties_on_the_threshold_key():
    """Equal 32-bit keys with the threshold on them: in a 65536-event sequence
    a seed with two equal keys is found on the CPU, and the cap is set to the
    rank of the first, so exactly one of the pair is kept -- the lower index,
    as the oracle's (key, index) order says."""
    L = 65536
    for seed in range(1, 40):
        u = sl.event_keys(L, 0, seed, 1)
        vals, counts = np.unique(u, return_counts=True)
        if np.any(counts > 1):
            break
    else:
        pytest.skip("no equal keys found")
    tied = vals[np.argmax(counts > 1)]
    cap = int(np.sum(u < tied)) + 1          # keeps exactly one of the tied events
    off = np.array([0, L], dtype=np.int64)
    log(f"seed {seed}: key {int(tied):#x} occurs {int(counts.max())} times; cap {cap}")
    _check(off, cap, seed=seed, step=1, what="threshold on equal keys")
    _, idx, _ = _run(off, cap, seed, 1)
    pair = np.nonzero(u == tied)[0]
    assert pair[0] in idx and pair[1] not in idx


def test_sl_gather_rows_and_timestamps():
    import torch
    x = synth.make_layer_stack(81, [900, 40, 3000, 2500], H=4, d=128, D=512, layers=1, P=1024,
                               NT=32, alpha=1 / 256)
    xd = dev_tensor(x.x, "bf16")
    ts = torch.from_numpy(x.ts).cuda()
    extra = torch.arange(x.T * 3, dtype=torch.float32, device="cuda").reshape(x.T, 3)   # 12-byte rows
    oo, idx, (gx, gts, gex) = _run(x.offsets, 1000, 11, 2, tensors=(xd, ts, extra))
    n = int(oo[-1])
    ref_off, ref_idx = sl.select(x.offsets, 1000, seed=11, step=2)
    assert np.array_equal(idx, ref_idx)
    xb = xd.view(torch.int16).cpu().numpy()
    assert np.array_equal(gx.view(torch.int16).cpu().numpy()[:n], xb[ref_idx])
    assert np.array_equal(gts.cpu().numpy()[:n], x.ts[ref_idx])
    assert np.array_equal(gex.cpu().numpy()[:n], extra.cpu().numpy()[ref_idx])


def test_sl_run_to_run_identical_and_seeded():
    off = np.array([0, 5000, 9000], dtype=np.int32)
    a = _run(off, 1200, 1, 1)[1]
    assert np.array_equal(a, _run(off, 1200, 1, 1)[1])
    assert not np.array_equal(a, _run(off, 1200, 1, 2)[1])
