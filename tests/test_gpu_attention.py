"""GPU parity of the attention path (scheduler + attention core + LN*U
epilogue) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import hstu_synth as synth
import oracle
from hstu_testlib import (DeviceAttn, assert_close, host_f32, log, oracle_attn, rel_errors,
                          run_attn, valid_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hstu_sequential_transducer_causal_amd import _lib
    _lib.load()


def _check_full(x, what, act=0, with_u=True):
    log(f"{what}: B={x.B} T={x.T} H={x.H} d={x.d} dtype={x.dtype}")
    d = DeviceAttn(x)
    o, y = run_attn(d, with_u=with_u, act=act)
    import torch
    torch.cuda.synchronize()
    ref = oracle_attn(x, act=act)
    rows = valid_rows(x)
    og = host_f32(o)[rows]
    assert_close(og, ref[rows], x.dtype, f"{what} O")
    if with_u:
        yr = oracle.ln_gate(ref[rows].reshape(len(rows), -1), x.u[rows].reshape(len(rows), -1),
                            eps=x.eps)
        assert_close(host_f32(y)[rows].reshape(len(rows), -1), yr, x.dtype, f"{what} Y")


def test_cfg1_fp32_full():
    _check_full(synth.config(1), "cfg1 fp32")


@pytest.mark.parametrize("seed", [11, 12])
def test_cfg1_fp32_other_seeds(seed):
    _check_full(synth.config(1, seed=seed, batch=7), f"cfg1 fp32 seed {seed}")


def test_cfg1_fp32_d64():
    x = synth.make_attn(5, [1, 64, 65, 130, 3], H=3, d=64, P=40, NT=32, alpha=1 / 128, dtype="f32")
    _check_full(x, "fp32 d64 ragged")


def test_bf16_more_sequences_than_the_scheduler_keeps_in_lds():
    """4500 short sequences (1..100 rows): past the 4096 the scheduler keeps
    in LDS, so the list and the sequence data beside each item come from the
    workspace copies; every row against the oracle."""
    rng = np.random.default_rng(77)
    lengths = rng.integers(1, 101, size=4500).tolist()
    x = synth.make_attn(78, lengths, H=1, d=128, P=128, NT=32, alpha=1 / 128, dtype="bf16")
    _check_full(x, "bf16 4500 short sequences")


def test_bf16_three_heads():
    """An odd head count through the per-die work queues (head rotated by the
    sequence)."""
    x = synth.make_attn(65, [50, 130, 7, 260, 1, 129], H=3, d=128, P=256, NT=32, alpha=1 / 256,
                        dtype="bf16")
    _check_full(x, "bf16 three heads")


def test_cfg2_bf16_small():
    _check_full(synth.config(2, batch=6, max_len=300), "cfg2 bf16 reduced")


def test_cfg3_bf16_small():
    _check_full(synth.config(3, batch=3, max_len=1200), "cfg3 bf16 reduced")


def test_cfg4_bf16_small_attention():
    _check_full(synth.config(4, batch=2, max_len=256), "cfg4 bf16 reduced (attention rows)")


def test_bf16_clamped_positions_ragged():
    """Small P so that most tiles use the clamped position bucket; ragged tails."""
    x = synth.make_attn(21, [1, 63, 64, 65, 127, 128, 129, 400], H=2, d=128, P=70, NT=32,
                        alpha=1 / 512, dtype="bf16")
    _check_full(x, "bf16 P=70 ragged")


def test_bf16_identity_activation():
    x = synth.make_attn(22, [5, 200, 131], H=2, d=128, P=300, NT=32, alpha=1 / 256, dtype="bf16",
                        qkv_std=0.1)
    _check_full(x, "bf16 identity act", act=1, with_u=False)


def test_bf16_wide_timestamps():
    """Gaps of up to 2^27 s push the time span past 2^30 s: the 64-bit path."""
    x = synth.make_attn(23, [150, 260], H=2, d=128, P=1024, NT=32, alpha=1 / 256, dtype="bf16",
                        mean_gap=float(2 ** 26))
    span = [int(x.ts[x.offsets[b + 1] - 1] - x.ts[x.offsets[b]]) for b in range(x.B)]
    assert max(span) > 2 ** 31
    _check_full(x, "bf16 wide timestamps")


def test_bf16_mixed_narrow_and_wide_tiles():
    x = synth.make_attn(24, [300], H=1, d=128, P=1024, NT=32, alpha=1 / 256, dtype="bf16")
    x.ts[200:] += 2 ** 31          # a jump in the middle of the sequence
    _check_full(x, "bf16 jump in timestamps")


def test_bf16_per_head_tables():
    x = synth.make_attn(25, [100, 170], H=3, d=128, P=200, NT=32, alpha=1 / 256, dtype="bf16")
    rng = np.random.default_rng(0)
    x.rab_pos = rng.normal(0, 0.1, size=(3, 200)).astype(np.float32)
    x.rab_time = rng.normal(0, 0.1, size=(3, 32)).astype(np.float32)
    _check_full(x, "bf16 per-head tables")


def test_bf16_empty_and_single_sequences():
    x = synth.make_attn(26, [0, 1, 0, 2, 129, 0], H=2, d=128, P=64, NT=32, alpha=1 / 64,
                        dtype="bf16")
    _check_full(x, "bf16 empty/single rows")


def test_bf16_mfalcon_edge_counts():
    """Candidate counts 0 (causal), all rows (no history), 1, and a ragged mix."""
    lengths = [70, 70, 200, 129, 64]
    nc = [0, 70, 1, 65, 63]
    x = synth.make_attn(27, lengths, H=2, d=128, P=1024, NT=32, alpha=1 / 256, dtype="bf16",
                        num_candidates=nc, with_w=True)
    _check_full(x, "bf16 M-FALCON edge counts")


@pytest.mark.parametrize("with_u", [True, False])
def test_bf16_split_row_blocks(with_u):
    """Few, long row blocks: the scheduler splits them over their key tiles.
    The partial sums are added up by the LN*U epilogue when it runs, else by
    the combine pass; O (and Y) must match the oracle either way."""
    from hstu_sequential_transducer_causal_amd import ops
    x = synth.config(3, batch=2, max_len=1200)
    d = DeviceAttn(x)
    items, _, _ = ops.hstu_attn_schedule(d.q, d.k, d.v, d.offsets, d.ts, d.rab_pos, d.rab_time,
                                         max_seq_len=d.max_seq_len)
    assert (items[:, 5] >= 0).any(), "this case is meant to split row blocks"
    _check_full(x, f"bf16 split blocks, {'epilogue' if with_u else 'combine pass'}", with_u=with_u)


@pytest.mark.parametrize("cfg,seqs", [(2, [0, 17, 63]), (3, [0, 5, 15])])
def test_full_size_sampled_sequences(cfg, seqs):
    """The full workload on the GPU, checked on whole sampled sequences (each
    sequence's output depends on that sequence alone)."""
    x = synth.config(cfg)
    log(f"cfg{cfg} full size: B={x.B} T={x.T}")
    d = DeviceAttn(x)
    o, y = run_attn(d)
    import torch
    torch.cuda.synchronize()
    og, yg = host_f32(o), host_f32(y)
    refs = oracle_attn(x, seqs=seqs)
    for b in seqs:
        s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
        assert_close(og[s0:s1], refs[b], x.dtype, f"cfg{cfg} seq {b} (L={s1 - s0}) O")
        yr = oracle.ln_gate(refs[b].reshape(s1 - s0, -1), x.u[s0:s1].reshape(s1 - s0, -1), eps=x.eps)
        assert_close(yg[s0:s1].reshape(s1 - s0, -1), yr, x.dtype, f"cfg{cfg} seq {b} Y")


def test_identity_integer_inputs_bit_exact():
    """Integer inputs, identity activation, power-of-two alpha: every product
    and sum is exact in fp32, so the GPU must equal the oracle rounded to
    bf16 bit for bit."""
    rng = np.random.default_rng(31)
    lengths = [1, 40, 64, 65, 190]
    x = synth.make_attn(31, lengths, H=2, d=128, P=100, NT=32, alpha=1 / 64, dtype="bf16")
    T = x.T
    x.q = rng.integers(-1, 2, size=(T, 2, 128)).astype(np.float32)
    x.k = (rng.random((T, 2, 128)) < 0.1).astype(np.float32)
    x.v = rng.integers(-2, 3, size=(T, 2, 128)).astype(np.float32)
    x.rab_pos = rng.integers(-3, 4, size=100).astype(np.float32)
    x.rab_time = rng.integers(-3, 4, size=32).astype(np.float32)
    d = DeviceAttn(x)
    o, _ = run_attn(d, with_u=False, act=1)
    import torch
    torch.cuda.synchronize()
    ref = oracle_attn(x, act=1)
    # |S| <= 128 + 6 fits bf16 exactly; sums stay far below 2^24
    want = synth.bf16_round(ref.astype(np.float32))
    got = host_f32(o)
    assert np.array_equal(got, want), f"max diff {np.abs(got - want).max()}"


def _two_bucket_blocks(x, NT):
    """Counts of (32-row block, 32-key block) pairs at or below the diagonal
    whose time-difference range [nearest, farthest] spans exactly two
    neighbouring log2 buckets (bucket = bit length of |dt|): those with
    every key at or before every row, and those whose ranges overlap."""
    def bucket(dt):
        return min(int(dt).bit_length(), NT - 1)
    keys_first = overlap = 0
    for b in range(x.B):
        t = x.ts[x.offsets[b]:x.offsets[b + 1]]
        L = len(t)
        for r0 in range(0, L, 32):
            rt = t[r0:min(r0 + 32, L)]
            for k0 in range(0, r0 + 1, 32):
                kt = t[k0:min(k0 + 32, L)]
                lo = max(0, rt.min() - kt.max(), kt.min() - rt.max())
                hi = max(rt.max() - kt.min(), kt.max() - rt.min())
                if bucket(hi) - bucket(lo) == 1:
                    if kt.max() <= rt.min():
                        keys_first += 1
                    else:
                        overlap += 1
    return keys_first, overlap


def test_identity_two_bucket_time_blocks_bit_exact():
    """Integer inputs and identity activation over timestamps whose 32x32
    blocks often span exactly two log2 time buckets, both with every key
    before the block's rows (the compare-and-select path) and overlapping
    them (the sad-and-shift path): the GPU equals the oracle bit for bit."""
    rng = np.random.default_rng(37)
    lengths = [700, 260, 97]
    x = synth.make_attn(37, lengths, H=2, d=128, P=1024, NT=32, alpha=1 / 64, dtype="bf16")
    T = x.T
    # regular 10 s steps; random 1-49 s steps; simultaneous events with a 1 s
    # step at events 40 and 80 (32-row blocks spanning one second: buckets 0
    # and 1 on the diagonal)
    gaps = [np.full(700, 10, np.int64), rng.integers(1, 50, 260).astype(np.int64),
            np.isin(np.arange(97), (40, 80)).astype(np.int64)]
    for b in range(x.B):
        s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
        x.ts[s0:s1] = 1_700_000_000 + np.cumsum(gaps[b][: s1 - s0])
    keys_first, overlap = _two_bucket_blocks(x, 32)
    log(f"two-bucket blocks: {keys_first} with keys first, {overlap} overlapping")
    assert keys_first >= 20 and overlap >= 2
    x.q = rng.integers(-1, 2, size=(T, 2, 128)).astype(np.float32)
    x.k = (rng.random((T, 2, 128)) < 0.1).astype(np.float32)
    x.v = rng.integers(-2, 3, size=(T, 2, 128)).astype(np.float32)
    x.rab_pos = rng.integers(-3, 4, size=1024).astype(np.float32)
    x.rab_time = rng.integers(-3, 4, size=32).astype(np.float32)
    d = DeviceAttn(x)
    o, _ = run_attn(d, with_u=False, act=1)
    import torch
    torch.cuda.synchronize()
    ref = oracle_attn(x, act=1)
    want = synth.bf16_round(ref.astype(np.float32))
    got = host_f32(o)
    assert np.array_equal(got, want), f"max diff {np.abs(got - want).max()}"


def test_fp32_identity_integer_inputs_exact():
    rng = np.random.default_rng(32)
    x = synth.make_attn(32, [3, 64, 65, 100], H=2, d=32, P=50, NT=32, alpha=1 / 64, dtype="f32")
    T = x.T
    x.q = rng.integers(-2, 3, size=(T, 2, 32)).astype(np.float32)
    x.k = rng.integers(-2, 3, size=(T, 2, 32)).astype(np.float32)
    x.v = rng.integers(-2, 3, size=(T, 2, 32)).astype(np.float32)
    x.rab_pos = rng.integers(-3, 4, size=50).astype(np.float32)
    x.rab_time = rng.integers(-3, 4, size=32).astype(np.float32)
    d = DeviceAttn(x)
    o, _ = run_attn(d, with_u=False, act=1)
    import torch
    torch.cuda.synchronize()
    ref = oracle_attn(x, act=1)
    assert np.array_equal(host_f32(o), ref.astype(np.float32))
