"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, run the oracle on the same inputs, compare."""
from __future__ import annotations

import sys
import time

import numpy as np

import hstu_synth as synth

# Tolerances, relative to max |reference| over the compared outputs.
TOL_F32_MAX = 1e-4
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 2e-3


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def dev_tensor(a: np.ndarray, dtype: str, device="cuda"):
    """Upload a float32 array as float32 or bfloat16 (values already bf16-exact)."""
    import torch
    if dtype == "bf16":
        bits = synth.bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits.copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host_f32(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


class DeviceAttn:
    """Device copies of an AttnInputs batch."""

    def __init__(self, x: synth.AttnInputs, device="cuda"):
        import torch
        self.x = x
        self.q = dev_tensor(x.q, x.dtype, device)
        self.k = dev_tensor(x.k, x.dtype, device)
        self.v = dev_tensor(x.v, x.dtype, device)
        self.u = dev_tensor(x.u, x.dtype, device)
        self.offsets = torch.from_numpy(x.offsets.astype(np.int32)).to(device)
        self.ts = torch.from_numpy(x.ts.astype(np.int64)).to(device)
        self.rab_pos = torch.from_numpy(x.rab_pos.astype(np.float32)).to(device)
        self.rab_time = torch.from_numpy(x.rab_time.astype(np.float32)).to(device)
        self.lengths = None if x.lengths is None else torch.from_numpy(x.lengths.astype(np.int32)).to(device)
        self.ncand = (None if x.num_candidates is None
                      else torch.from_numpy(x.num_candidates.astype(np.int32)).to(device))
        self.w = None if x.w is None else torch.from_numpy(x.w.astype(np.float32)).to(device)
        self.max_seq_len = int(max(1, x.seq_lengths().max() if x.B else 1))


def run_attn(d: DeviceAttn, *, with_u=True, act=0, o=None, y=None):
    from hstu_sequential_transducer_causal_amd import ops
    return ops.hstu_attn_fwd(d.q, d.k, d.v, d.offsets, d.ts, d.rab_pos, d.rab_time, d.x.alpha,
                             max_seq_len=d.max_seq_len, seq_lengths=d.lengths,
                             num_candidates=d.ncand, u=d.u if with_u else None, ln_eps=d.x.eps,
                             act=act, o=o, y=y)


def oracle_attn(x: synth.AttnInputs, act=0, seqs=None):
    """Oracle O [T, H, d] (all rows, or only the rows of sequences ``seqs``)."""
    import oracle
    if seqs is None:
        return oracle.attn(x.q, x.k, x.v, x.offsets, x.ts, x.rab_pos, x.rab_time, x.alpha,
                           lengths=x.lengths, num_candidates=x.num_candidates, act=act)
    out = {}
    for b in seqs:
        s0 = int(x.offsets[b])
        L = int(x.seq_lengths()[b])
        sl = slice(s0, s0 + L)
        nc = None if x.num_candidates is None else [int(x.num_candidates[b])]
        out[b] = oracle.attn(x.q[sl], x.k[sl], x.v[sl], [0, L], x.ts[sl], x.rab_pos, x.rab_time,
                             x.alpha, num_candidates=nc, act=act)
    return out


def rel_errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    scale = scale if scale > 0 else 1.0
    err = np.abs(got - ref)
    return float(err.max() / scale) if err.size else 0.0, float(err.mean() / scale) if err.size else 0.0


def assert_close(got, ref, dtype: str, what: str = ""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    mx, mean = rel_errors(got, ref)
    log(f"{what}: max_err/max|ref| = {mx:.3e}, mean_err/max|ref| = {mean:.3e}")
    if dtype == "f32":
        assert mx <= TOL_F32_MAX, f"{what}: max rel err {mx:.3e} > {TOL_F32_MAX}"
    else:
        assert mx <= TOL_BF16_MAX, f"{what}: max rel err {mx:.3e} > {TOL_BF16_MAX}"
        assert mean <= TOL_BF16_MEAN, f"{what}: mean rel err {mean:.3e} > {TOL_BF16_MEAN}"
    return mx, mean


def valid_rows(x: synth.AttnInputs) -> np.ndarray:
    L = x.seq_lengths()
    return np.concatenate([np.arange(x.offsets[b], x.offsets[b] + L[b]) for b in range(x.B)]
                          ).astype(np.int64) if x.B else np.zeros(0, np.int64)
