"""GPU invariants of the method (through the C ABI): causality, M-FALCON
candidate independence, padding invariance, batch = concatenation of its
sequences, run-to-run determinism, and the scheduler's work list against the
oracle's brute-force tile set (bit-exact)."""
import numpy as np
import pytest

import hstu_synth as synth
import oracle
from hstu_testlib import DeviceAttn, assert_close, host_f32, log, oracle_attn, run_attn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _sync():
    import torch
    torch.cuda.synchronize()


def _tile_list(a_end, kb):
    return list(range(a_end)) + list(range(kb & 0xFFFF, kb >> 16))


def _items_to_tiles(items):
    """Tiles covered by the pieces, checking that the pieces of each row block
    split its tile list into disjoint, complete position ranges."""
    tiles = set()
    cover = {}
    for b, qt, a_end, kb, pr, slot, k, n in items.tolist():
        lst = _tile_list(a_end, kb)
        p0, p1 = pr & 0xFFFF, pr >> 16
        assert 0 <= p0 < p1 <= len(lst)
        for kt in lst[p0:p1]:
            tiles.add((b, qt, kt))
        cover.setdefault((b, qt), []).append((p0, p1, slot, k, len(lst), n))
    for key, parts in cover.items():
        parts.sort()
        assert parts[0][0] == 0 and parts[-1][1] == parts[-1][4], key
        assert all(parts[i][1] == parts[i + 1][0] for i in range(len(parts) - 1)), key
        assert all(p[5] == len(parts) for p in parts), key     # every piece knows the count
        if len(parts) == 1:
            assert parts[0][2] == -1 and parts[0][3] == 0, key     # not split
        else:
            assert len({p[2] for p in parts}) == 1 and parts[0][2] >= 0, key
            assert sorted(p[3] for p in parts) == list(range(len(parts))), key
    return tiles


@pytest.mark.parametrize("case", ["causal", "mfalcon", "padded", "empty", "cfg3", "cfg4", "f32"])
def test_schedule_matches_bruteforce_tiles(case):
    from hstu_sequential_transducer_causal_amd import ops
    if case == "causal":
        x = synth.config(2, batch=9, max_len=700)
    elif case == "mfalcon":
        x = synth.make_attn(3, [130, 70, 300, 64, 1], H=1, d=128, P=64, NT=32, alpha=1.0,
                            dtype="bf16", num_candidates=[40, 70, 1, 0, 1])
    elif case == "padded":
        x = synth.make_attn(4, [200, 90, 129], H=1, d=128, P=64, NT=32, alpha=1.0, dtype="bf16")
        x.lengths = np.array([150, 0, 129], dtype=np.int32)
    elif case == "empty":
        x = synth.make_attn(5, [0, 0, 5, 0], H=1, d=128, P=64, NT=32, alpha=1.0, dtype="bf16")
    elif case == "cfg3":
        x = synth.config(3)
    elif case == "cfg4":
        x = synth.config(4)   # long row blocks next to the work per workgroup: split pieces
    else:
        x = synth.config(1, batch=11)
    d = DeviceAttn(x)
    items, tm, tn = ops.hstu_attn_schedule(d.q, d.k, d.v, d.offsets, d.ts, d.rab_pos, d.rab_time,
                                           max_seq_len=d.max_seq_len, seq_lengths=d.lengths,
                                           num_candidates=d.ncand)
    got = _items_to_tiles(items)
    want = set(map(tuple, oracle.tiles(x.offsets, tm, tn, lengths=x.lengths,
                                       num_candidates=x.num_candidates).tolist()))
    log(f"schedule {case}: {len(items)} items, {len(got)} tiles (tile {tm}x{tn})")
    assert got == want
    # no duplicate pieces
    keys = [(int(r[0]), int(r[1]), int(r[6])) for r in items.tolist()]
    assert len(keys) == len(set(keys))
    # longest piece first
    cost = [(r[4] >> 16) - (r[4] & 0xFFFF) for r in items.tolist()]
    assert cost == sorted(cost, reverse=True)


@pytest.mark.parametrize("B,max_len", [(9000, 128), (5000, 400)])
def test_schedule_beyond_the_lds_copies(B, max_len):
    """More sequences than the scheduler keeps in LDS (4096), and more row
    blocks than it keeps costs for (8192): the list is built from its
    workspace copies (searches over the global prefix, costs recomputed).
    9000 sequences of 1..128 rows are 9000 row blocks; 5000 of up to 400 rows
    about 10 000."""
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    rng = np.random.default_rng(B)
    lengths = rng.integers(1, max_len + 1, size=B).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(off[-1])
    dev = torch.device("cuda:0")
    q = torch.zeros((T, 1, 128), dtype=torch.bfloat16, device=dev)   # (the list reads no rows)
    ts = torch.zeros(T, dtype=torch.int64, device=dev)
    items, tm, tn = ops.hstu_attn_schedule(q, q, q, torch.from_numpy(off).to(dev), ts,
                                           torch.zeros(64, device=dev), torch.zeros(32, device=dev),
                                           max_seq_len=int(lengths.max()))
    got = _items_to_tiles(items)
    want = set(map(tuple, oracle.tiles(off, tm, tn).tolist()))
    log(f"schedule B={B}: {len(items)} items, {len(got)} tiles")
    assert len(items) > 8192 and got == want
    cost = [(r[4] >> 16) - (r[4] & 0xFFFF) for r in items.tolist()]
    assert cost == sorted(cost, reverse=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causality_future_rows_do_not_change_past_rows(dtype):
    if dtype == "bf16":
        x = synth.make_attn(41, [300, 257], H=2, d=128, P=1024, NT=32, alpha=1 / 512, dtype="bf16")
    else:
        x = synth.make_attn(41, [60, 45], H=2, d=32, P=128, NT=32, alpha=1 / 64, dtype="f32")
    o1, y1 = run_attn(DeviceAttn(x))
    _sync()
    o1 = host_f32(o1)
    rng = np.random.default_rng(1)
    x2 = synth.AttnInputs(**{**x.__dict__})
    x2.q, x2.k, x2.v, x2.ts = x.q.copy(), x.k.copy(), x.v.copy(), x.ts.copy()
    cut = {}
    for b in range(x.B):
        s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
        c = s0 + (s1 - s0) // 3
        cut[b] = c
        for arr in (x2.q, x2.k, x2.v):
            arr[c + 1:s1] = synth.bf16_round(rng.normal(0, 2.0, size=arr[c + 1:s1].shape).astype(np.float32))
        x2.ts[c + 1:s1] += 12345
    o2, _ = run_attn(DeviceAttn(x2))
    _sync()
    o2 = host_f32(o2)
    for b in range(x.B):
        s0 = int(x.offsets[b])
        assert np.array_equal(o1[s0:cut[b] + 1], o2[s0:cut[b] + 1]), b


def test_mfalcon_candidate_equals_single_candidate_run():
    x = synth.config(4, batch=2, max_len=192)
    d = DeviceAttn(x)
    o, _ = run_attn(d, with_u=False)
    _sync()
    o = host_f32(o)
    for b in range(x.B):
        s0 = int(x.offsets[b]); L = int(x.offsets[b + 1]) - s0
        c = int(x.num_candidates[b]); n = L - c
        for cand in [0, 1, c // 2, c - 1]:
            rows = list(range(s0, s0 + n)) + [s0 + n + cand]
            xs = synth.AttnInputs(B=1, H=x.H, d=x.d, offsets=np.array([0, n + 1], np.int32),
                                  q=x.q[rows], k=x.k[rows], v=x.v[rows], u=x.u[rows], ts=x.ts[rows],
                                  rab_pos=x.rab_pos, rab_time=x.rab_time, alpha=x.alpha,
                                  dtype=x.dtype, num_candidates=np.array([1], np.int32))
            o1, _ = run_attn(DeviceAttn(xs), with_u=False)
            _sync()
            o1 = host_f32(o1)
            ref = oracle_attn(xs)[n]
            # the batched candidate row and the single-candidate row agree within
            # the bf16 tolerance of the oracle value (different tile paths)
            assert_close(o[s0 + n + cand], ref, "bf16", f"batched candidate {cand}")
            assert_close(o1[n], ref, "bf16", f"single candidate {cand}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padding_invariance(dtype):
    import torch
    if dtype == "bf16":
        x = synth.make_attn(43, [130, 64, 7, 250], H=2, d=128, P=512, NT=32, alpha=1 / 256,
                            dtype="bf16", num_candidates=[10, 0, 3, 50])
    else:
        x = synth.make_attn(43, [50, 64, 7], H=2, d=32, P=128, NT=32, alpha=1 / 64, dtype="f32")
    o_packed, y_packed = run_attn(DeviceAttn(x))
    _sync()
    o_packed, y_packed = host_f32(o_packed), host_f32(y_packed)
    L = np.diff(x.offsets)
    pad = np.array([5, 64, 1, 3])[:x.B]
    off_p = np.concatenate([[0], np.cumsum(L + pad)]).astype(np.int32)
    Tp = int(off_p[-1])

    def padded(a, fill):
        out = np.full((Tp,) + a.shape[1:], fill, dtype=a.dtype)
        for b in range(x.B):
            out[off_p[b]:off_p[b] + L[b]] = a[x.offsets[b]:x.offsets[b + 1]]
        return out
    xp = synth.AttnInputs(B=x.B, H=x.H, d=x.d, offsets=off_p, q=padded(x.q, np.nan),
                          k=padded(x.k, np.nan), v=padded(x.v, np.nan), u=padded(x.u, np.nan),
                          ts=padded(x.ts, -(2 ** 62)), rab_pos=x.rab_pos, rab_time=x.rab_time,
                          alpha=x.alpha, dtype=x.dtype, lengths=L.astype(np.int32),
                          num_candidates=x.num_candidates)
    dp = DeviceAttn(xp)
    sentinel = 7.0
    o = torch.full((Tp, x.H, x.d), sentinel, dtype=dp.q.dtype, device="cuda")
    y = torch.full((Tp, x.H, x.d), sentinel, dtype=dp.q.dtype, device="cuda")
    run_attn(dp, o=o, y=y)
    _sync()
    o, y = host_f32(o), host_f32(y)
    for b in range(x.B):
        a0, a1 = int(x.offsets[b]), int(x.offsets[b + 1])
        p0 = int(off_p[b])
        assert np.array_equal(o[p0:p0 + L[b]], o_packed[a0:a1]), b
        assert np.array_equal(y[p0:p0 + L[b]], y_packed[a0:a1]), b
        assert np.all(o[p0 + L[b]:off_p[b + 1]] == sentinel)
        assert np.all(y[p0 + L[b]:off_p[b + 1]] == sentinel)


def test_batch_is_concatenation_and_runs_are_deterministic():
    x = synth.config(2, batch=5, max_len=400)
    d = DeviceAttn(x)
    o1, y1 = run_attn(d)
    o2, y2 = run_attn(d)
    _sync()
    o1, o2 = host_f32(o1), host_f32(o2)
    assert np.array_equal(o1, o2)
    assert np.array_equal(host_f32(y1), host_f32(y2))
    for b in [0, 3]:
        s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
        xb = synth.AttnInputs(B=1, H=x.H, d=x.d, offsets=np.array([0, s1 - s0], np.int32),
                              q=x.q[s0:s1], k=x.k[s0:s1], v=x.v[s0:s1], u=x.u[s0:s1],
                              ts=x.ts[s0:s1], rab_pos=x.rab_pos, rab_time=x.rab_time,
                              alpha=x.alpha, dtype=x.dtype)
        ob, _ = run_attn(DeviceAttn(xb))
        _sync()
        assert np.array_equal(host_f32(ob), o1[s0:s1])
