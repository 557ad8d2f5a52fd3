"""GPU parity of the M-FALCON ranking pass (scores) and of the HSTU layer
stack (f1 + SiLU, attention, LN * U, f2 + residual) against the oracle."""
import numpy as np
import pytest

import hstu_synth as synth
import oracle
from hstu_testlib import DeviceAttn, assert_close, dev_tensor, host_f32, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _scores_gpu(x):
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    d = DeviceAttn(x)
    cmax = int(x.num_candidates.max())
    y = torch.empty_like(d.q)
    scores, o, y = ops.mfalcon_score(d.q, d.k, d.v, d.u, d.offsets, d.ncand, d.ts, d.rab_pos,
                                     d.rab_time, x.alpha, d.w, max_seq_len=d.max_seq_len,
                                     score_stride=cmax, ln_eps=x.eps, y=y)
    torch.cuda.synchronize()
    return host_f32(scores), host_f32(o), host_f32(y)


def _scores_candidates_only(x):
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    d = DeviceAttn(x)
    cmax = int(x.num_candidates.max())
    scores, _, _ = ops.mfalcon_score(d.q, d.k, d.v, d.u, d.offsets, d.ncand, d.ts, d.rab_pos,
                                     d.rab_time, x.alpha, d.w, max_seq_len=d.max_seq_len,
                                     score_stride=cmax, ln_eps=x.eps, candidates_only=True)
    torch.cuda.synchronize()
    return host_f32(scores)


@pytest.mark.parametrize("case", ["ragged", "cfg4"])
def test_mfalcon_candidates_only_scores(case):
    """Computing only the query tiles that hold candidate rows (candidates read
    history K/V, never history outputs) gives the oracle's scores, including
    users whose candidates start mid-tile or who have none.  With few row
    blocks left the long ones are split over their key tiles (partial sums
    added in fp32), so the result matches the full pass within tolerance, and
    exactly where neither pass split."""
    if case == "ragged":
        x = synth.make_attn(52, [100, 300, 129, 256, 40], H=4, d=128, P=1024, NT=32,
                            alpha=1 / 512, dtype="bf16", num_candidates=[1, 200, 65, 0, 40],
                            with_w=True)
        users = list(range(x.B))
    else:
        x = synth.config(4)
        users = [0, 7]
    full, _, _ = _scores_gpu(x)
    part = _scores_candidates_only(x)
    for b in users:
        c = int(x.num_candidates[b])
        if c == 0:
            continue
        s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
        sl = slice(s0, s1)
        ref = oracle.mfalcon_score(x.q[sl], x.k[sl], x.v[sl], x.u[sl], [0, s1 - s0], [c],
                                   x.ts[sl], x.rab_pos, x.rab_time, x.alpha, x.w, eps=x.eps)
        assert_close(part[b, :c], ref[0, :c], "bf16", f"candidates-only scores {case} user {b}")
    for b in range(x.B):
        c = int(x.num_candidates[b])
        assert_close(part[b, :c], full[b, :c], "bf16", f"candidates-only vs full pass user {b}")
    log(f"candidates-only scores ({case}, B={x.B}) match the oracle and the full pass")


def test_mfalcon_scores_small():
    x = synth.config(4, batch=3, max_len=256)
    log(f"cfg4 reduced: B={x.B} T={x.T}")
    s, o, y = _scores_gpu(x)
    ref = oracle.mfalcon_score(x.q, x.k, x.v, x.u, x.offsets, x.num_candidates, x.ts, x.rab_pos,
                               x.rab_time, x.alpha, x.w, eps=x.eps)
    assert_close(s, ref, "bf16", "cfg4 reduced scores")


def test_mfalcon_scores_ragged_candidates():
    x = synth.make_attn(51, [100, 300, 129], H=4, d=128, P=1024, NT=32, alpha=1 / 512,
                        dtype="bf16", num_candidates=[1, 200, 65], with_w=True)
    s, _, _ = _scores_gpu(x)
    ref = oracle.mfalcon_score(x.q, x.k, x.v, x.u, x.offsets, x.num_candidates, x.ts, x.rab_pos,
                               x.rab_time, x.alpha, x.w, eps=x.eps)
    for b in range(x.B):
        c = int(x.num_candidates[b])
        assert_close(s[b, :c], ref[b, :c], "bf16", f"ragged scores seq {b}")


def test_mfalcon_scores_full_size_sampled_user():
    """Full workload (8 users x (2048 + 512)) on the GPU; the oracle scores two
    users (each user's scores depend on that user's rows alone)."""
    x = synth.config(4)
    log(f"cfg4 full: B={x.B} T={x.T}")
    s, _, _ = _scores_gpu(x)
    for b in [0, 7]:
        s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
        sl = slice(s0, s1)
        ref = oracle.mfalcon_score(x.q[sl], x.k[sl], x.v[sl], x.u[sl], [0, s1 - s0],
                                   [int(x.num_candidates[b])], x.ts[sl], x.rab_pos, x.rab_time,
                                   x.alpha, x.w, eps=x.eps)
        assert_close(s[b], ref[0], "bf16", f"cfg4 user {b} scores")


def _layer_stack_gpu(x: synth.LayerInputs):
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    xd = dev_tensor(x.x, "bf16")
    off = torch.from_numpy(x.offsets.astype(np.int32)).cuda()
    ts = torch.from_numpy(x.ts).cuda()
    max_len = int(np.diff(x.offsets).max())
    cur = xd
    for l in range(x.layers):
        w1 = dev_tensor(x.w1[l], "bf16")
        w2 = dev_tensor(x.w2[l], "bf16")
        rp = torch.from_numpy(x.rab_pos[l]).cuda()
        rt = torch.from_numpy(x.rab_time[l]).cuda()
        cur = ops.hstu_layer_fwd(cur, w1, w2, off, ts, rp, rt, x.alpha, H=x.H, d=x.d,
                                 max_seq_len=max_len, ln_eps=x.eps)
    torch.cuda.synchronize()
    return host_f32(cur)


def _layer_stack_oracle(x: synth.LayerInputs, seqs=None):
    if seqs is None:
        cur = x.x.astype(np.float64)
        for l in range(x.layers):
            cur = oracle.layer(cur, x.w1[l], x.w2[l], x.offsets, x.ts, x.rab_pos[l],
                               x.rab_time[l], x.alpha, x.H, x.d, eps=x.eps)
        return cur
    out = {}
    for b in seqs:
        s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
        cur = x.x[s0:s1].astype(np.float64)
        for l in range(x.layers):
            cur = oracle.layer(cur, x.w1[l], x.w2[l], [0, s1 - s0], x.ts[s0:s1], x.rab_pos[l],
                               x.rab_time[l], x.alpha, x.H, x.d, eps=x.eps)
        out[b] = cur
    return out


def test_layer_stack_small():
    x = synth.config(5, batch=3, max_len=300)
    log(f"cfg5 reduced: B={x.B} T={x.T}")
    got = _layer_stack_gpu(x)
    ref = _layer_stack_oracle(x)
    assert_close(got, ref, "bf16", "cfg5 reduced 4-layer X_out")


def test_single_layer_ragged_rows():
    """M not a multiple of the GEMM tile; one layer."""
    x = synth.make_layer_stack(52, [1, 77, 130], H=4, d=128, D=512, layers=1, P=1024, NT=32,
                               alpha=1 / 256)
    got = _layer_stack_gpu(x)
    ref = _layer_stack_oracle(x)
    assert_close(got, ref, "bf16", "1-layer ragged X_out")


def test_single_layer_biases_in_place():
    """f1 and f2 with their biases, X_out written over X (the f2 epilogue reads
    each residual element before it writes that element); rows span two GEMM
    row tiles with a ragged tail."""
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    x = synth.make_layer_stack(53, [1, 300, 77], H=4, d=128, D=512, layers=1, P=1024, NT=32,
                               alpha=1 / 256)
    rng = np.random.default_rng(54)
    b1 = rng.normal(0, 0.2, size=4 * x.H * x.d).astype(np.float32)
    b2 = rng.normal(0, 0.2, size=x.x.shape[1]).astype(np.float32)
    xd = dev_tensor(x.x, "bf16")
    out = ops.hstu_layer_fwd(xd, dev_tensor(x.w1[0], "bf16"), dev_tensor(x.w2[0], "bf16"),
                             torch.from_numpy(x.offsets.astype(np.int32)).cuda(),
                             torch.from_numpy(x.ts).cuda(), torch.from_numpy(x.rab_pos[0]).cuda(),
                             torch.from_numpy(x.rab_time[0]).cuda(), x.alpha, H=x.H, d=x.d,
                             max_seq_len=int(np.diff(x.offsets).max()), b1=torch.from_numpy(b1).cuda(),
                             b2=torch.from_numpy(b2).cuda(), ln_eps=x.eps, x_out=xd)
    torch.cuda.synchronize()
    assert out.data_ptr() == xd.data_ptr()
    ref = oracle.layer(x.x, x.w1[0], x.w2[0], x.offsets, x.ts, x.rab_pos[0], x.rab_time[0], x.alpha,
                       x.H, x.d, b1=b1, b2=b2, eps=x.eps)
    assert_close(host_f32(xd), ref, "bf16", "1-layer biases, in place")


def test_layer_stack_full_size_sampled_sequences():
    x = synth.config(5)
    log(f"cfg5 full: B={x.B} T={x.T}")
    got = _layer_stack_gpu(x)
    L = np.diff(x.offsets)
    seqs = [int(np.argmin(L)), 3]
    refs = _layer_stack_oracle(x, seqs)
    for b in seqs:
        s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
        assert_close(got[s0:s1], refs[b], "bf16", f"cfg5 seq {b} (L={s1 - s0}) X_out")


def _layer_scores_gpu(x, ncand, w, candidates_only):
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    xd = dev_tensor(x.x, "bf16")
    w1 = dev_tensor(x.w1[0], "bf16")
    off = torch.from_numpy(x.offsets.astype(np.int32)).cuda()
    nc = torch.from_numpy(np.asarray(ncand, dtype=np.int32)).cuda()
    ts = torch.from_numpy(x.ts).cuda()
    rp = torch.from_numpy(x.rab_pos[0]).cuda()
    rt = torch.from_numpy(x.rab_time[0]).cuda()
    wd = torch.from_numpy(w.astype(np.float32)).cuda()
    cmax = max(1, int(max(ncand)))
    s = ops.mfalcon_layer_score(xd, w1, off, nc, ts, rp, rt, x.alpha, wd, H=x.H, d=x.d,
                                max_seq_len=int(np.diff(x.offsets).max()), score_stride=cmax,
                                ln_eps=x.eps, candidates_only=candidates_only)
    torch.cuda.synchronize()
    return host_f32(s)


@pytest.mark.parametrize("candidates_only", [True, False])
def test_mfalcon_last_layer_scores_ragged(candidates_only):
    """The last layer of an M-FALCON stack, candidate rows only: f1 + SiLU
    over every row, attention (only the query tiles holding candidates, or
    all), LN * U and the score -- against the oracle's scoring layer; users
    without candidates, of candidates only, and with candidates mid-tile."""
    lengths = [300, 129, 64, 520, 200]
    ncand = [40, 0, 64, 257, 1]
    x = synth.make_layer_stack(96, lengths, H=4, d=128, D=512, layers=1, P=1024, NT=32,
                               alpha=1 / 1024)
    w = np.random.default_rng(97).normal(0, 1 / np.sqrt(512), size=512)
    got = _layer_scores_gpu(x, ncand, w, candidates_only)
    ref = oracle.layer_scores(x.x, x.w1[0], x.offsets, ncand, x.ts, x.rab_pos[0], x.rab_time[0],
                              x.alpha, w, x.H, x.d, eps=x.eps)
    g = np.concatenate([got[b, :c] for b, c in enumerate(ncand)])
    r = np.concatenate([ref[b, :c] for b, c in enumerate(ncand)])
    assert_close(g, r, "bf16", f"last-layer scores (candidates_only={candidates_only})")


def test_mfalcon_last_layer_scores_full_size_sampled_users():
    """8 users x (2048 history + 512 candidates), D = 512, 4 heads of 128, in
    one call; the oracle's scoring layer checks two users (a user's scores
    depend on that user's rows alone)."""
    n, c, B = 2048, 512, 8
    x = synth.make_layer_stack(98, [n + c] * B, H=4, d=128, D=512, layers=1, P=1024, NT=32,
                               alpha=1 / (n + c))
    w = np.random.default_rng(99).normal(0, 1 / np.sqrt(512), size=512)
    got = _layer_scores_gpu(x, [c] * B, w, True)
    for b in (0, 7):
        s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
        ref = oracle.layer_scores(x.x[s0:s1], x.w1[0], [0, s1 - s0], [c], x.ts[s0:s1], x.rab_pos[0],
                                  x.rab_time[0], x.alpha, w, x.H, x.d, eps=x.eps)
        assert_close(got[b], ref[0], "bf16", f"full-size last-layer scores user {b}")
