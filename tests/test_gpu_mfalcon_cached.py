"""GPU parity of M-FALCON against a history KV cache (mfalcon_score_cached).

The cached pass reads each user's history keys and values from a cache and
the candidates from their own buffers; every candidate sees the whole
history at position n_b plus itself.  Its outputs must equal the oracle's
M-FALCON pass over the combined [history | candidates] sequence: the
candidates' attention rows, and the scores <LN(O) * U, w>."""
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


def _run_cached(x, sp, rab_pos, rab_time, *, with_o=True, workspace=None, score_stride=None):
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    dev = "cuda"
    hr, cr = sp.hist_rows, sp.cand_rows
    k_hist = dev_tensor(x.k[hr], "bf16")
    v_hist = dev_tensor(x.v[hr], "bf16")
    q = dev_tensor(x.q[cr], "bf16")
    k = dev_tensor(x.k[cr], "bf16")
    v = dev_tensor(x.v[cr], "bf16")
    u = dev_tensor(x.u[cr], "bf16")
    ts_hist = torch.from_numpy(np.ascontiguousarray(sp.ts[hr])).to(dev)
    ts_cand = torch.from_numpy(np.ascontiguousarray(sp.ts[cr])).to(dev)
    hoff = torch.from_numpy(sp.hist_offsets.astype(np.int32)).to(dev)
    coff = torch.from_numpy(sp.cand_offsets.astype(np.int32)).to(dev)
    rp = torch.from_numpy(np.ascontiguousarray(rab_pos, dtype=np.float32)).to(dev)
    rt = torch.from_numpy(np.ascontiguousarray(rab_time, dtype=np.float32)).to(dev)
    w = torch.from_numpy(x.w.astype(np.float32)).to(dev)
    max_hist = int(max(1, np.diff(sp.hist_offsets).max())) if x.B else 1
    max_cands = int(max(1, np.diff(sp.cand_offsets).max())) if x.B else 1
    o = torch.empty_like(q) if with_o else None
    scores, o = ops.mfalcon_score_cached(k_hist, v_hist, hoff, ts_hist, q, k, v, u, coff, ts_cand,
                                         rp, rt, x.alpha, w, max_hist_len=max_hist,
                                         max_cands=max_cands,
                                         score_stride=score_stride or max_cands, ln_eps=x.eps,
                                         o=o, workspace=workspace)
    torch.cuda.synchronize()
    return host_f32(scores), (host_f32(o) if with_o else None)


def _oracle(x, sp, rab_pos, rab_time):
    """Oracle O and scores of every candidate row (combined layout)."""
    o = oracle.attn(x.q, x.k, x.v, x.offsets, sp.ts, rab_pos, rab_time, x.alpha,
                    num_candidates=x.num_candidates)
    cr = sp.cand_rows
    y = oracle.ln_gate(o[cr], x.u[cr], eps=x.eps)
    return o[cr], y @ x.w.astype(np.float64)


def _check(x, sp, rab_pos, rab_time, what):
    s, o = _run_cached(x, sp, rab_pos, rab_time)
    o_ref, s_ref = _oracle(x, sp, rab_pos, rab_time)
    assert_close(o, o_ref, "bf16", f"{what}: candidates' O")
    got = np.concatenate([s[b, :int(x.num_candidates[b])] for b in range(x.B)])
    assert_close(got, s_ref, "bf16", f"{what}: scores")
    return s, o


def test_cached_ragged_users_and_empty_history():
    """Ragged histories and candidate counts, a user without history (its
    candidates see only themselves), users without candidates, candidates
    that start mid-tile, request times after the last event."""
    hist = [100, 300, 129, 0, 40, 64, 0]
    cands = [1, 200, 65, 3, 0, 64, 0]
    x = synth.make_attn(61, [h + c for h, c in zip(hist, cands)], H=4, d=128, P=1024, NT=32,
                        alpha=1 / 512, dtype="bf16", num_candidates=cands, with_w=True)
    sp = synth.split_cached(x, seed=62, max_gap=3_000_000)
    _check(x, sp, x.rab_pos, x.rab_time, "cached ragged")
    # the same pass through the combined layout agrees with the cached one
    from hstu_testlib import DeviceAttn
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    x2 = synth.make_attn(61, [h + c for h, c in zip(hist, cands)], H=4, d=128, P=1024, NT=32,
                         alpha=1 / 512, dtype="bf16", num_candidates=cands, with_w=True)
    x2.ts = sp.ts
    d = DeviceAttn(x2)
    full, _, _ = ops.mfalcon_score(d.q, d.k, d.v, d.u, d.offsets, d.ncand, d.ts, d.rab_pos,
                                   d.rab_time, x2.alpha, d.w, max_seq_len=d.max_seq_len,
                                   score_stride=max(cands), ln_eps=x2.eps)
    torch.cuda.synchronize()
    s, _ = _run_cached(x, sp, x.rab_pos, x.rab_time)
    full = host_f32(full)
    got = np.concatenate([s[b, :c] for b, c in enumerate(cands)])
    ref = np.concatenate([full[b, :c] for b, c in enumerate(cands)])
    assert_close(got, ref, "bf16", "cached vs combined layout")


def test_cached_per_head_tables_and_wide_time_gaps():
    """Per-head bias tables, time gaps past the widest bucket, positions past
    the last position bucket (history longer than P)."""
    hist = [700, 33, 257]
    cands = [130, 7, 64]
    x = synth.make_attn(63, [h + c for h, c in zip(hist, cands)], H=3, d=128, P=200, NT=24,
                        alpha=1 / 256, dtype="bf16", num_candidates=cands, with_w=True,
                        mean_gap=5e5)
    rng = np.random.default_rng(64)
    rp = rng.normal(0, 0.1, size=(3, 200)).astype(np.float32)
    rt = rng.normal(0, 0.1, size=(3, 24)).astype(np.float32)
    sp = synth.split_cached(x, seed=65, max_gap=1 << 26)
    _check(x, sp, rp, rt, "cached per-head tables")


def test_cached_many_candidates_split_blocks():
    """Few users with many candidates and a long history: every row block
    reads every history tile, and with few blocks per head the long ones are
    split over their key tiles (fp32 partials combined in the epilogue)."""
    hist = [2048, 1500]
    cands = [1000, 333]
    x = synth.make_attn(66, [h + c for h, c in zip(hist, cands)], H=4, d=128, P=1024, NT=32,
                        alpha=1 / 2560, dtype="bf16", num_candidates=cands, with_w=True)
    sp = synth.split_cached(x, seed=67, max_gap=100_000)
    _check(x, sp, x.rab_pos, x.rab_time, "cached many candidates")


def test_cached_workspace_reuse_is_deterministic():
    """Two calls in a row on one workspace, the second smaller: each gives
    the same scores as a call on a fresh workspace, bit for bit."""
    import torch
    hist = [300, 129, 512]
    cands = [200, 65, 96]
    x = synth.make_attn(68, [h + c for h, c in zip(hist, cands)], H=4, d=128, P=1024, NT=32,
                        alpha=1 / 512, dtype="bf16", num_candidates=cands, with_w=True)
    sp = synth.split_cached(x, seed=69, max_gap=10_000)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    s1, o1 = _run_cached(x, sp, x.rab_pos, x.rab_time, workspace=ws)
    s1b, o1b = _run_cached(x, sp, x.rab_pos, x.rab_time)
    assert np.array_equal(s1, s1b) and np.array_equal(o1, o1b)
    hs, cs = [40], [17]
    y = synth.make_attn(70, [hs[0] + cs[0]], H=4, d=128, P=1024, NT=32, alpha=1 / 512,
                        dtype="bf16", num_candidates=cs, with_w=True)
    spy = synth.split_cached(y, seed=71, max_gap=10_000)
    s2, o2 = _run_cached(y, spy, y.rab_pos, y.rab_time, workspace=ws)
    s2b, o2b = _run_cached(y, spy, y.rab_pos, y.rab_time)
    assert np.array_equal(s2, s2b) and np.array_equal(o2, o2b)
    o_ref, s_ref = _oracle(y, spy, y.rab_pos, y.rab_time)
    assert_close(s2[0, :17], s_ref, "bf16", "second, smaller call")
    log("workspace reuse: identical results")


def test_cached_full_size_sampled_candidates():
    """8 users x (2048 history + 4096 candidates) scored in one call; for two
    users the oracle checks a random sample of 48 candidates (each candidate
    depends on the history and itself alone, so the sample is scored as a
    short [history | sampled candidates] sequence)."""
    B, n, c = 8, 2048, 4096
    x = synth.make_attn(72, [n + c] * B, H=4, d=128, P=1024, NT=32, alpha=1 / (n + 512),
                        dtype="bf16", num_candidates=[c] * B, with_w=True)
    sp = synth.split_cached(x, seed=73, max_gap=86_400)
    s, o = _run_cached(x, sp, x.rab_pos, x.rab_time)
    rng = np.random.default_rng(74)
    for b in [0, 7]:
        pick = np.sort(rng.choice(c, size=48, replace=False))
        r0 = int(x.offsets[b])
        rows = np.concatenate([np.arange(r0, r0 + n), r0 + n + pick])
        o_ref = oracle.attn(x.q[rows], x.k[rows], x.v[rows], [0, len(rows)], sp.ts[rows],
                            x.rab_pos, x.rab_time, x.alpha, num_candidates=[48])[n:]
        s_ref = oracle.ln_gate(o_ref, x.u[rows][n:], eps=x.eps) @ x.w.astype(np.float64)
        o_got = o[int(sp.cand_offsets[b]) + pick]
        assert_close(o_got, o_ref, "bf16", f"full size user {b}: sampled O")
        assert_close(s[b, pick], s_ref, "bf16", f"full size user {b}: sampled scores")
