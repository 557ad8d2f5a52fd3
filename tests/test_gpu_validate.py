"""hstu_validate_offsets and the HSTU_VALIDATE=1 switch: the device check of
the batch structure the attention calls trust (the jagged layout of "Meta
HSTU: как действия пользователя стали основой большой рекомендательной
модели", section "Разная длина истории превращается в выигрыш по ресурсам";
the candidate counts of "生成式推荐（一）：HSTU", section "M-FALCON").
Malformed batches reach only the validator: no attention kernel is launched
on them."""
import os

import numpy as np
import pytest

import hstu_synth as synth
from hstu_testlib import DeviceAttn, log, run_attn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hstu_sequential_transducer_causal_amd import _lib
    _lib.load()


def _check(offsets, *, num_rows, max_seq_len, lengths=None, ncand=None):
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    t = lambda a: None if a is None else torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")
    ops.hstu_validate_offsets(t(offsets), num_rows=num_rows, max_seq_len=max_seq_len,
                              seq_lengths=t(lengths), num_candidates=t(ncand))


def _fails(what, b, **kw):
    from hstu_sequential_transducer_causal_amd import _lib
    with pytest.raises(_lib.HstuError) as e:
        _check(**kw)
    log(f"{what}: {e.value}")
    assert e.value.status == _lib.HSTU_ERR_ARG
    assert f"sequence {b}:" in str(e.value) and what in str(e.value)


def test_valid_batches_pass():
    rng = np.random.default_rng(5)
    for B in (1, 7, 300, 2500):   # one pass of the workgroup, and several
        L = rng.integers(0, 90, size=B)
        off = np.concatenate([[0], np.cumsum(L)])
        c = np.minimum(L, rng.integers(0, 20, size=B))
        _check(off, num_rows=int(off[-1]), max_seq_len=int(max(1, L.max())), ncand=c)
        # padded layout: each slot 100 rows, L_b of them used
        offp = np.arange(B + 1) * 100
        _check(offp, num_rows=int(offp[-1]) + 5, max_seq_len=100, lengths=L, ncand=c)


def test_each_violation_named():
    off = [0, 10, 25, 25, 60]
    _fails("offsets[0] < 0", 0, offsets=[-1, 10, 25, 25, 60], num_rows=60, max_seq_len=64)
    _fails("offsets decrease", 2, offsets=[0, 10, 25, 20, 60], num_rows=60, max_seq_len=64)
    _fails("offsets[B] > num_rows", 3, offsets=off, num_rows=59, max_seq_len=64)
    _fails("seq_lengths[b] outside", 1, offsets=off, num_rows=60, max_seq_len=64, lengths=[10, 16, 0, 35])
    _fails("seq_lengths[b] outside", 3, offsets=off, num_rows=60, max_seq_len=64, lengths=[10, 15, 0, -1])
    _fails("length > max_seq_len", 3, offsets=off, num_rows=60, max_seq_len=34)
    _fails("num_candidates[b] outside", 2, offsets=off, num_rows=60, max_seq_len=64, ncand=[0, 15, 1, 0])
    _fails("num_candidates[b] outside", 0, offsets=off, num_rows=60, max_seq_len=64, ncand=[-1, 0, 0, 0])


def test_first_failure_is_reported():
    # violations at sequences 700 and 1200 (different workgroup passes): the lower one is named
    B = 1500
    L = np.full(B, 5)
    off = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    c = np.zeros(B, dtype=np.int64)
    c[1200] = 9
    off[701] = off[700] - 1   # sequence 700's end lies before its start
    _fails("offsets decrease", 700, offsets=off, num_rows=int(off[-1]), max_seq_len=5, ncand=c)


def test_hstu_validate_env_guards_the_calls():
    from hstu_sequential_transducer_causal_amd import _lib
    x = synth.make_attn(31, [40, 70, 33], H=2, d=128, P=128, NT=32, alpha=1 / 128, dtype="bf16")
    d = DeviceAttn(x)
    old = os.environ.get("HSTU_VALIDATE")
    try:
        os.environ["HSTU_VALIDATE"] = "1"
        run_attn(d)   # a well-formed batch runs as usual
        bad = d.offsets.clone()
        bad[2] = bad[1] - 1
        d.offsets = bad
        with pytest.raises(_lib.HstuError) as e:
            run_attn(d)
        log(f"guarded forward: {e.value}")
        assert e.value.status == _lib.HSTU_ERR_ARG and "sequence 1:" in str(e.value)
        # the gradients are guarded the same way
        import torch
        from hstu_sequential_transducer_causal_amd import ops
        g = torch.zeros_like(d.v)
        with pytest.raises(_lib.HstuError) as e:
            ops.hstu_attn_bwd(d.q, d.k, d.v, d.offsets, d.ts, d.rab_pos, d.rab_time, d.x.alpha,
                              max_seq_len=d.max_seq_len, dout=g)
        log(f"guarded gradients: {e.value}")
        assert e.value.status == _lib.HSTU_ERR_ARG and "sequence 1:" in str(e.value)
    finally:
        if old is None:
            os.environ.pop("HSTU_VALIDATE", None)
        else:
            os.environ["HSTU_VALIDATE"] = old


def test_hstu_validate_layer_needs_packed_rows():
    """A layer's gradients sum over every row, so its batch must be packed:
    with HSTU_VALIDATE=1 a layer call whose offsets end before num_rows is
    refused, the same batch packed runs."""
    import torch
    from hstu_sequential_transducer_causal_amd import _lib, ops
    from hstu_testlib import dev_tensor
    x = synth.make_layer_stack(33, [40, 70, 33], H=2, d=128, D=256, layers=1, P=128, NT=32,
                               alpha=1 / 128)
    xd = dev_tensor(x.x, "bf16")
    w1, w2 = dev_tensor(x.w1[0], "bf16"), dev_tensor(x.w2[0], "bf16")
    ts = torch.from_numpy(x.ts).cuda()
    rp, rt = torch.from_numpy(x.rab_pos[0]).cuda(), torch.from_numpy(x.rab_time[0]).cuda()
    run = lambda off: ops.hstu_layer_fwd(xd, w1, w2, torch.from_numpy(off.astype(np.int32)).cuda(), ts, rp,
                                         rt, x.alpha, H=x.H, d=x.d, max_seq_len=70, ln_eps=x.eps)
    old = os.environ.get("HSTU_VALIDATE")
    try:
        os.environ["HSTU_VALIDATE"] = "1"
        run(x.offsets)
        short = np.array([0, 40, 110], dtype=np.int64)   # the last 33 rows in no sequence
        with pytest.raises(_lib.HstuError) as e:
            run(short)
        log(f"guarded layer: {e.value}")
        assert e.value.status == _lib.HSTU_ERR_ARG and "packed" in str(e.value)
        torch.cuda.synchronize()
    finally:
        if old is None:
            os.environ.pop("HSTU_VALIDATE", None)
        else:
            os.environ["HSTU_VALIDATE"] = old
