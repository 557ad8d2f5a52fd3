"""Benchmark of the HSTU attention hot path on one MI355X.

A step is one pass of the hot path over one batch of the long-sequence
workload (16 jagged sequences, lognormal lengths clipped to [1024, 8192],
stochastic length capped at 8192**0.85 = 2120, 8 heads, d = 128, bf16):
the device-side jagged tile scheduler, the bf16 MFMA attention core and the
LayerNorm(O) * U epilogue, all through hstu_attn_fwd.  Inputs are resident
in HBM before the timed region.

Prints ONE JSON line.  `value` is unmasked attention TFLOP/s of the whole
step; `roofline` is the attention-core kernel alone, timed with HIP events
recorded around its launch on the same stream; `cpu_baseline` is the fp64
oracle on a bounded sample of the same workload (host cores of this machine);
`parity` is one step of the same call checked against that oracle run (max
and mean |err| / max|ref|).  Order: the parity check and the CPU baseline,
the other workloads (each with its own sampled parity check), then the
headline's W warm-up and K timed steps.
Other workloads (bf16 batch of 64, M-FALCON ranking, the 4-layer stack) and
the gradients (hstu_attn_bwd from dLoss/dY on the long-sequence and M-FALCON
workloads; hstu_layer_bwd on one layer of the stack) and stochastic length
with its gather (the long-sequence workload's raw batch) are timed briefly
and reported under "other_workloads".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=400)
    p.add_argument("--settle", type=float, default=SETTLE_S,
                   help="seconds of untimed back-to-back steps before each case's warm-up (0: none)")
    p.add_argument("--workload", type=int, default=3, help="workload number 2..5 for the main line")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-others", action="store_true")
    p.add_argument("--cpu-sample-seqs", type=int, default=0, help="0: all sequences")
    p.add_argument("--only-bwd", action="store_true",
                   help="only time the attention gradients on --workload (for kernel traces)")
    p.add_argument("--only-sl-sweep", action="store_true",
                   help="only the stochastic-length exponent sweep")
    p.add_argument("--only-cached", action="store_true",
                   help="only the M-FALCON pass against a history KV cache")
    p.add_argument("--only-layer-bwd", action="store_true",
                   help="only time the gradients of one layer of the stack workload (for kernel traces)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device copy (reference for the HBM byte counters)")
    return p.parse_args()


def up(a, dtype, dev):
    import torch
    import hstu_synth as synth
    if dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(a).view(np.int16).copy()).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)


class AttnCase:
    def __init__(self, x, dev, with_scores=False, candidates_only=False):
        import torch
        from hstu_sequential_transducer_causal_amd import ops
        self.x = x
        self.q, self.k, self.v, self.u = (up(a, x.dtype, dev) for a in (x.q, x.k, x.v, x.u))
        self.off = torch.from_numpy(x.offsets).to(dev)
        self.ts = torch.from_numpy(x.ts).to(dev)
        self.rp = torch.from_numpy(x.rab_pos).to(dev)
        self.rt = torch.from_numpy(x.rab_time).to(dev)
        self.nc = None if x.num_candidates is None else torch.from_numpy(x.num_candidates).to(dev)
        self.w = None if x.w is None else torch.from_numpy(x.w).to(dev)
        self.max_len = int(np.diff(x.offsets).max())
        self.o = torch.empty_like(self.q)
        self.y = torch.empty_like(self.q)
        self.with_scores = with_scores
        self.candidates_only = candidates_only
        if with_scores:
            self.cmax = int(x.num_candidates.max())
            self.scores = torch.zeros(x.B, self.cmax, dtype=torch.float32, device=dev)
        args = ops.make_attn_args(self.q, self.k, self.v, self.off, self.ts, self.rp, self.rt,
                                  x.alpha, max_seq_len=self.max_len, o=self.o,
                                  num_candidates=self.nc, u=self.u, y=self.y)
        self.ws = torch.empty(max(1, ops.attn_workspace_bytes(args)), dtype=torch.uint8, device=dev)

    def step(self, ev0=None, ev1=None, ev2=None, ev3=None):
        from hstu_sequential_transducer_causal_amd import ops
        if self.with_scores:
            ops.mfalcon_score(self.q, self.k, self.v, self.u, self.off, self.nc, self.ts, self.rp,
                              self.rt, self.x.alpha, self.w, max_seq_len=self.max_len,
                              score_stride=self.cmax, ln_eps=self.x.eps, o=self.o, y=None,
                              scores=self.scores, workspace=self.ws, ev_core_begin=ev0,
                              ev_core_end=ev1, candidates_only=self.candidates_only)
        else:
            ops.hstu_attn_fwd(self.q, self.k, self.v, self.off, self.ts, self.rp, self.rt,
                              self.x.alpha, max_seq_len=self.max_len, num_candidates=self.nc,
                              u=self.u, ln_eps=self.x.eps, o=self.o, y=self.y, workspace=self.ws,
                              ev_core_begin=ev0, ev_core_end=ev1, ev_epi_begin=ev2, ev_epi_end=ev3)


class StackCase:
    def __init__(self, x, dev):
        import torch
        from hstu_sequential_transducer_causal_amd import ops
        self.x = x
        self.xin = up(x.x, "bf16", dev)
        self.bufs = [torch.empty_like(self.xin), torch.empty_like(self.xin)]
        self.w1 = [up(w, "bf16", dev) for w in x.w1]
        self.w2 = [up(w, "bf16", dev) for w in x.w2]
        self.rp = [torch.from_numpy(r).to(dev) for r in x.rab_pos]
        self.rt = [torch.from_numpy(r).to(dev) for r in x.rab_time]
        self.off = torch.from_numpy(x.offsets).to(dev)
        self.ts = torch.from_numpy(x.ts).to(dev)
        self.max_len = int(np.diff(x.offsets).max())
        l = ops.make_layer_args(self.xin, self.w1[0], self.w2[0], self.off, self.ts, self.rp[0],
                                self.rt[0], x.alpha, H=x.H, d=x.d, max_seq_len=self.max_len,
                                x_out=self.bufs[0])
        self.ws = torch.empty(ops.layer_workspace_bytes(l), dtype=torch.uint8, device=dev)

    def step(self, ev0=None, ev1=None):
        from hstu_sequential_transducer_causal_amd import ops
        cur = self.xin
        for l in range(self.x.layers):
            out = self.bufs[l % 2]
            ops.hstu_layer_fwd(cur, self.w1[l], self.w2[l], self.off, self.ts, self.rp[l],
                               self.rt[l], self.x.alpha, H=self.x.H, d=self.x.d,
                               max_seq_len=self.max_len, ln_eps=self.x.eps, x_out=out,
                               workspace=self.ws)
            cur = out


class BwdCase:
    """Gradients of the attention path from dLoss/dY (gate derivative, both
    work lists, the dQ and dK/dV kernels, the table-gradient reduction)."""

    def __init__(self, x, dev):
        import torch
        import hstu_synth as synth
        from hstu_sequential_transducer_causal_amd import ops
        self.x = x
        self.q, self.k, self.v, self.u = (up(a, "bf16", dev) for a in (x.q, x.k, x.v, x.u))
        self.o = up(synth.upstream_grad(8, x.v.shape, std=0.02), "bf16", dev)
        self.dy = up(synth.upstream_grad(9, x.v.shape), "bf16", dev)
        self.off = torch.from_numpy(x.offsets).to(dev)
        self.ts = torch.from_numpy(x.ts).to(dev)
        self.rp = torch.from_numpy(x.rab_pos).to(dev)
        self.rt = torch.from_numpy(x.rab_time).to(dev)
        self.nc = None if x.num_candidates is None else torch.from_numpy(x.num_candidates).to(dev)
        self.max_len = int(np.diff(x.offsets).max())
        self.out = [torch.empty_like(self.q) for _ in range(4)]
        self.drp = torch.empty_like(self.rp)
        self.drt = torch.empty_like(self.rt)
        a = ops.make_attn_bwd_args(self.q, self.k, self.v, self.off, self.ts, self.rp, self.rt,
                                   x.alpha, max_seq_len=self.max_len, dq=self.out[0],
                                   dk=self.out[1], dv=self.out[2], dy=self.dy, o=self.o, u=self.u,
                                   du=self.out[3], ln_eps=x.eps, num_candidates=self.nc,
                                   drab_pos=self.drp, drab_time=self.drt)
        self.ws = torch.empty(max(1, ops.attn_bwd_workspace_bytes(a)), dtype=torch.uint8, device=dev)

    def step(self, events=None):
        from hstu_sequential_transducer_causal_amd import ops
        ops.hstu_attn_bwd(
            self.q, self.k, self.v, self.off, self.ts, self.rp, self.rt, self.x.alpha,
            max_seq_len=self.max_len, dy=self.dy, o=self.o, u=self.u, ln_eps=self.x.eps,
            num_candidates=self.nc, dq=self.out[0], dk=self.out[1], dv=self.out[2],
            du=self.out[3], drab_pos=self.drp, drab_time=self.drt, workspace=self.ws,
            events=events)


# Kernel times come from HIP events that the timed launches themselves carry.
# Each event pair costs the stream a few microseconds between kernels, so only
# every EVENT_STRIDE-th timed step carries them; the others run bare.
EVENT_STRIDE = 10

# Before its warm-up steps every timed case first runs untimed steps back to
# back for SETTLE_S seconds of wall time (--settle): after the host-side work
# between cases (input generation, the oracle) the GPU's clocks have dropped,
# and a short timed window (20 steps of 0.25 ms) would otherwise measure their
# ramp, not the sustained rate.  The count of those steps is reported.
SETTLE_S = 0.25
SETTLE_LOG = []


def settle(step, label=""):
    """Run step() back to back, untimed, until SETTLE_S seconds have passed
    (synchronising every 16 steps to read the clock); returns the count."""
    import torch
    n = 0
    if SETTLE_S > 0:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S:
            for _ in range(16):
                step()
            n += 16
            torch.cuda.synchronize()
    SETTLE_LOG.append((label, n))
    return n


def time_bwd(case, steps, warmup):
    """Wall time per step and the mean dQ / dK-dV kernel times (HIP events
    carried by those launches on every EVENT_STRIDE-th timed step)."""
    import torch
    settle(case.step, "bwd")
    for _ in range(warmup):
        case.step()
    torch.cuda.synchronize()
    evs = []
    for _ in range(0, steps, EVENT_STRIDE):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for ev in e:
            ev.record()
        evs.append(e)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i % EVENT_STRIDE == 0:
            case.step(tuple(ev.cuda_event for ev in evs[i // EVENT_STRIDE]))
        else:
            case.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    dq = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dkv = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    return ms, dq, dkv


def bwd_record(x, dev, steps):
    from hstu_sequential_transducer_causal_amd import flops
    c = BwdCase(x, dev)
    ms, dq, dkv = time_bwd(c, steps, 2)
    L = np.diff(x.offsets)
    pairs = flops.visible_pairs(L, x.num_candidates)
    alg = flops.attn_bwd_flops(L, x.H, x.d, x.num_candidates)
    gblk = flops.grad_blocks(L, x.num_candidates) * x.H
    ex_dq = pairs * x.H * 2 * x.d + gblk * 2 * 32768   # G K, and the transpose of each G block
    ex_dkv = pairs * x.H * 8 * x.d     # S, dO V^T, dV, dK
    g_bytes = gblk * 32 * 32 * 4       # G blocks, fp32: written by dK/dV, read by dQ
    rec = {"ms_per_step": round(ms, 4), "tflops": round(alg / (ms * 1e-3) / 1e12, 2),
           "tokens_per_s": round(x.T / (ms * 1e-3), 1), "tokens": x.T,
           "dq_kernel_ms": round(dq, 4), "dkv_kernel_ms": round(dkv, 4),
           "dq_kernel_tflops_executed": round(ex_dq / (dq * 1e-3) / 1e12, 2),
           "dkv_kernel_tflops_executed": round(ex_dkv / (dkv * 1e-3) / 1e12, 2),
           "dkv_kernel_frac_bf16_peak": round(ex_dkv / (dkv * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "g_blocks_bytes": g_bytes, "dq_kernel_g_read_gbs": round(g_bytes / (dq * 1e-3) / 1e9, 1),
           "flop_convention": "tflops: 8*d per visible pair and head (dV, dO V^T, dQ, dK); "
                              "executed: dK/dV 8*d per pair (S recomputed), dQ 2*d per pair (G K from "
                              "the stored G) plus 2 32x32x16 MFMAs per stored block (its transpose)"}
    del c
    return rec


class LayerBwdCase:
    """Gradients of one layer (layer 0 of the stack workload) from dLoss/dX_out."""

    def __init__(self, x, dev, saved=False):
        import torch
        import hstu_synth as synth
        from hstu_sequential_transducer_causal_amd import ops
        self.x = x
        self.xin = up(x.x, "bf16", dev)
        self.g = up(synth.upstream_grad(310, x.x.shape), "bf16", dev)
        self.w1, self.w2 = up(x.w1[0], "bf16", dev), up(x.w2[0], "bf16", dev)
        self.rp = torch.from_numpy(x.rab_pos[0]).to(dev)
        self.rt = torch.from_numpy(x.rab_time[0]).to(dev)
        self.off = torch.from_numpy(x.offsets).to(dev)
        self.ts = torch.from_numpy(x.ts).to(dev)
        self.max_len = int(np.diff(x.offsets).max())
        f32 = dict(dtype=torch.float32, device=dev)
        zw = 4 * x.H * x.d
        self.out = dict(dx=torch.empty_like(self.xin), dw1=torch.empty(zw, x.D, **f32),
                        dw2=torch.empty(x.D, x.H * x.d, **f32), drab_pos=torch.empty_like(self.rp),
                        drab_time=torch.empty_like(self.rt))
        a = ops.make_layer_bwd_args(self.xin, self.w1, self.w2, self.off, self.ts, self.rp, self.rt,
                                    x.alpha, self.g, H=x.H, d=x.d, max_seq_len=self.max_len,
                                    dx=self.out["dx"], dw1=self.out["dw1"], dw2=self.out["dw2"],
                                    drab_pos=self.out["drab_pos"], drab_time=self.out["drab_time"])
        self.args = a
        self.ws = torch.empty(max(1, ops.layer_bwd_workspace_bytes(a, saved=saved)), dtype=torch.uint8, device=dev)
        self.saved = None
        if saved:
            # the training forward keeps Z, the pre-activation, O and Y (untimed)
            kw = dict(H=x.H, d=x.d, max_seq_len=self.max_len)
            need = ops.layer_saved_bytes(self.xin, self.w1, self.w2, self.off, self.ts, self.rp, self.rt,
                                         x.alpha, **kw)
            self.saved = torch.empty(need, dtype=torch.uint8, device=dev)
            ops.hstu_layer_fwd(self.xin, self.w1, self.w2, self.off, self.ts, self.rp, self.rt, x.alpha,
                               saved=self.saved, **kw)
            torch.cuda.synchronize()

    def step(self, ev0=None, ev1=None):
        import ctypes
        import torch
        from hstu_sequential_transducer_causal_amd import _lib
        lib = _lib.load()
        stream = torch.cuda.current_stream().cuda_stream
        if self.saved is None:
            _lib.check(lib.hstu_layer_bwd(ctypes.byref(self.args), self.ws.data_ptr(), self.ws.numel(), stream))
        else:
            _lib.check(lib.hstu_layer_bwd_saved(ctypes.byref(self.args), self.saved.data_ptr(), self.saved.numel(),
                                                self.ws.data_ptr(), self.ws.numel(), stream))


class CachedCase:
    """M-FALCON against a history KV cache: every user's candidates scored
    over the cached history keys/values (mfalcon_score_cached)."""

    def __init__(self, dev, B=4, n=2048, c=16384, seed=41):
        import torch
        import hstu_synth as synth
        from hstu_sequential_transducer_causal_amd import ops
        x = synth.make_attn(seed, [n + c] * B, H=4, d=128, P=1024, NT=32, alpha=1.0 / (n + 512),
                            dtype="bf16", num_candidates=[c] * B, with_w=True)
        sp = synth.split_cached(x, seed=seed + 1, max_gap=86_400)
        self.name = f"mfalcon_cached_bf16_b{B}_n{n}_c{c}_h4_d128"
        self.B, self.n, self.c, self.H, self.d = B, n, c, x.H, x.d
        hr, cr = sp.hist_rows, sp.cand_rows
        self.k_hist, self.v_hist = up(x.k[hr], "bf16", dev), up(x.v[hr], "bf16", dev)
        self.q, self.k, self.v, self.u = (up(a[cr], "bf16", dev) for a in (x.q, x.k, x.v, x.u))
        self.ts_hist = torch.from_numpy(np.ascontiguousarray(sp.ts[hr])).to(dev)
        self.ts_cand = torch.from_numpy(np.ascontiguousarray(sp.ts[cr])).to(dev)
        self.hoff = torch.from_numpy(sp.hist_offsets).to(dev)
        self.coff = torch.from_numpy(sp.cand_offsets).to(dev)
        self.rp = torch.from_numpy(x.rab_pos).to(dev)
        self.rt = torch.from_numpy(x.rab_time).to(dev)
        self.w = torch.from_numpy(x.w).to(dev)
        self.alpha, self.eps = x.alpha, x.eps
        self.o = torch.empty_like(self.q)
        self.scores = torch.zeros(B, c, dtype=torch.float32, device=dev)
        m = ops.make_mfalcon_cached_args(self.k_hist, self.v_hist, self.hoff, self.ts_hist, self.q,
                                         self.k, self.v, self.u, self.coff, self.ts_cand, self.rp,
                                         self.rt, self.alpha, self.w, max_hist_len=n, max_cands=c,
                                         scores=self.scores, score_stride=c, o=self.o)
        self.ws = torch.empty(max(1, ops.mfalcon_cached_workspace_bytes(m)), dtype=torch.uint8,
                              device=dev)
        self.x, self.dev = x, dev

    def step(self, ev0=None, ev1=None):
        from hstu_sequential_transducer_causal_amd import ops
        ops.mfalcon_score_cached(self.k_hist, self.v_hist, self.hoff, self.ts_hist, self.q, self.k,
                                 self.v, self.u, self.coff, self.ts_cand, self.rp, self.rt,
                                 self.alpha, self.w, max_hist_len=self.n, max_cands=self.c,
                                 score_stride=self.c, ln_eps=self.eps, o=self.o,
                                 scores=self.scores, workspace=self.ws, ev_core_begin=ev0,
                                 ev_core_end=ev1)

    def record(self, steps):
        st, ce = time_case(self, steps, 2)
        ncand = self.B * self.c
        # unmasked pairs: every candidate with the n history keys and itself
        fc = float(ncand) * (self.n + 1) * 4 * self.d * self.H
        rec = {"ms_per_step": round(st, 4), "candidates_per_s": round(ncand / (st * 1e-3), 1),
               "candidate_pair_tflops": round(fc / (st * 1e-3) / 1e12, 2)}
        if ce:
            rec["core_ms"] = round(ce, 4)
            rec["core_tflops"] = round(fc / (ce * 1e-3) / 1e12, 2)
        # the same scores from the combined [history | candidates] layout,
        # computing only the query tiles that hold candidates
        import torch
        comb = AttnCase(self.x, self.dev, with_scores=True, candidates_only=True)
        st2, _ = time_case(comb, steps, 2)
        rec["combined_layout_candidates_only_ms"] = round(st2, 4)
        del comb
        torch.cuda.empty_cache()
        return rec


class LastLayerCase:
    """The last layer of an M-FALCON stack, scores only (mfalcon_layer_score):
    8 users x (2048 history + 512 candidates), D = 512, 4 heads of 128."""

    def __init__(self, dev, candidates_only=True, B=8, n=2048, c=512, seed=43):
        import torch
        import hstu_synth as synth
        x = synth.make_layer_stack(seed, [n + c] * B, H=4, d=128, D=512, layers=1, P=1024, NT=32,
                                   alpha=1.0 / (n + c))
        self.name = f"mfalcon_last_layer_bf16_b{B}_n{n}_bm{c}_D512_h4_d128"
        self.B, self.n, self.c, self.H, self.d = B, n, c, x.H, x.d
        self.T = x.T
        self.x = up(x.x, "bf16", dev)
        self.w1 = up(x.w1[0], "bf16", dev)
        self.off = torch.from_numpy(x.offsets).to(dev)
        self.nc = torch.full((B,), c, dtype=torch.int32, device=dev)
        self.ts = torch.from_numpy(x.ts).to(dev)
        self.rp = torch.from_numpy(x.rab_pos[0]).to(dev)
        self.rt = torch.from_numpy(x.rab_time[0]).to(dev)
        self.w = torch.from_numpy(np.random.default_rng(seed + 1).normal(
            0, 1 / np.sqrt(512), size=512).astype(np.float32)).to(dev)
        self.alpha, self.eps = x.alpha, x.eps
        self.scores = torch.zeros(B, c, dtype=torch.float32, device=dev)
        self.candidates_only = candidates_only

    def step(self, ev0=None, ev1=None):
        from hstu_sequential_transducer_causal_amd import ops
        ops.mfalcon_layer_score(self.x, self.w1, self.off, self.nc, self.ts, self.rp, self.rt,
                                self.alpha, self.w, H=self.H, d=self.d, max_seq_len=self.n + self.c,
                                score_stride=self.c, ln_eps=self.eps,
                                candidates_only=self.candidates_only, scores=self.scores)


def sl_record(dev, steps):
    """Stochastic length with the gather of the rows of Q, K, V, U (8 heads of
    128, bf16) and timestamps, on the long-sequence workload's raw batch."""
    import torch
    import hstu_synth as synth
    from hstu_sequential_transducer_causal_amd import ops
    L = synth.longseq_raw_lengths()
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(L)]).astype(np.int32)).to(dev)
    T = int(L.sum())
    g = torch.Generator(device=dev).manual_seed(5)
    rows = [torch.randn(T, 1024, generator=g, device=dev).to(torch.bfloat16) for _ in range(4)]
    ts = torch.arange(T, dtype=torch.int64, device=dev) * 60
    tensors = (*rows, ts)
    settle(lambda: ops.stochastic_length(off, synth.SL_CAP, seed=1, step=0, tensors=tensors), "sl")
    for _ in range(2):
        ops.stochastic_length(off, synth.SL_CAP, seed=1, step=0, tensors=tensors)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        oo, _, _ = ops.stochastic_length(off, synth.SL_CAP, seed=1, step=i, tensors=tensors)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    kept = int(oo[-1].item())
    moved = 2 * kept * (4 * 1024 * 2 + 8)   # read + write of every kept row
    return {"ms_per_step": round(ms, 4), "raw_rows": T, "kept_rows": kept,
            "gbytes_per_s": round(moved / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(moved / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def sl_sweep_record(dev, steps):
    """Stochastic-length exponent sweep on the long-sequence workload's raw
    batch (16 sequences, 8 heads of 128): per alpha the cap is
    floor(8192 ** (alpha / 2)); a step is the seeded subsampling with the
    gather of Q, K, V, U and timestamps, then hstu_attn_fwd (with LN * U)
    on the kept rows."""
    import torch
    import hstu_synth as synth
    from hstu_sequential_transducer_causal_amd import flops, ops
    L = synth.longseq_raw_lengths()
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(L)]).astype(np.int32)).to(dev)
    T = int(L.sum())
    H, d = 8, 128
    g = torch.Generator(device=dev).manual_seed(6)
    rows = [(0.5 * torch.randn(T, H * d, generator=g, device=dev)).to(torch.bfloat16) for _ in range(4)]
    ts = torch.cumsum(torch.randint(1, 120, (T,), generator=g, device=dev), 0).to(torch.int64)
    rp = (0.1 * torch.randn(1024, generator=g, device=dev)).float()
    rt = (0.1 * torch.randn(32, generator=g, device=dev)).float()
    out = {}
    for alpha in (1.6, 1.7, 1.8, 1.9, 2.0):
        cap = int(math.floor(synth.SL_MAX_RAW ** (alpha / 2)))
        kept = np.minimum(L, cap)
        o = torch.empty(T, H, d, dtype=torch.bfloat16, device=dev)
        y = torch.empty_like(o)

        def step(i):
            oo, _, (q, k, v, u, t) = ops.stochastic_length(off, cap, seed=7, step=i,
                                                           tensors=(*rows, ts))
            ops.hstu_attn_fwd(q.view(T, H, d), k.view(T, H, d), v.view(T, H, d), oo, t, rp, rt,
                              1.0 / synth.SL_MAX_RAW, max_seq_len=cap, u=u.view(T, H, d), o=o, y=y)

        settle(lambda: step(0), f"sl alpha {alpha}")
        for i in range(2):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        fl = flops.attn_flops(kept, H, d, d)
        out[f"alpha_{alpha}"] = {"cap": cap, "kept_tokens": int(kept.sum()), "ms_per_step": round(ms, 4),
                                 "attn_gflop": round(fl / 1e9, 1),
                                 "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}
        log(f"stochastic length alpha {alpha}: {out[f'alpha_{alpha}']}")
        del o, y
        torch.cuda.empty_cache()
    return out


def time_case(case, steps, warmup, core_events=True, epi_events=False):
    """Wall time per step (synchronised bracket) and mean core-kernel time (HIP
    events carried by the core launch on every EVENT_STRIDE-th timed step);
    with epi_events also the epilogue launch's mean time, left in
    case.epi_ms."""
    import torch
    settle(case.step, getattr(case, "name", ""))
    for _ in range(warmup):
        case.step()
    torch.cuda.synchronize()
    evs = []
    nev = 4 if epi_events else 2
    if core_events:
        for _ in range(0, steps, EVENT_STRIDE):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
            for ev in e:
                ev.record()                  # materialise the HIP events
            evs.append(e)
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if core_events and i % EVENT_STRIDE == 0:
            case.step(*(ev.cuda_event for ev in evs[i // EVENT_STRIDE]))
        else:
            case.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    core_ms = None
    if core_events:
        core_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        if epi_events:
            case.epi_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    return ms_step, core_ms


TRAFFIC_FILES = [os.path.join(ROOT, "profiles", f)
                 for f in ("attn_bf16_longseq_traffic.json", "attn_bf16_b64_traffic.json")]
KERNEL_SRCS = [os.path.join(ROOT, "hstu_sequential_transducer_causal_amd", "csrc", f)
               for f in ("attn_bf16.hip", "tile_ops.h", "hstu_device.h")]


def _code_only(text: str) -> str:
    """C++ source without its comments, blank lines and runs of spaces
    (string literals in these sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(" ".join(l.split()) for l in text.splitlines() if l.strip())


def kernel_hash() -> str:
    """Hash of the code (comments left out) of the sources the attention-core
    kernel is compiled from and of its compiler flags."""
    import hashlib
    from hstu_sequential_transducer_causal_amd import build
    h = hashlib.sha256()
    for src in KERNEL_SRCS:
        with open(src, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    flags = [f for f in build.CXXFLAGS if f != "-I" and not os.path.isabs(f)]   # (no paths)
    h.update(repr(flags + build.EXTRA_FLAGS.get("attn_bf16.hip", [])).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the attention core on `workload` from the
    committed counter runs (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    factor), or None when none covers that workload or the kernel source
    changed since they were taken."""
    for path in TRAFFIC_FILES:
        try:
            with open(path) as f:
                t = json.load(f)
        except (OSError, ValueError):
            continue
        if t.get("workload", "").split(" ")[0] != workload:
            continue
        if t.get("kernel_sha256_16") != kernel_hash():
            return None
        return int(t["bytes_per_launch"])
    return None


def copy_calibration():
    import torch
    n = 256 * 1024 * 1024
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(x, nseq):
    """The oracle as it stands, on the first nseq sequences of the workload
    (all when nseq <= 0); returns the record and the oracle's O of those rows."""
    import oracle
    from hstu_sequential_transducer_causal_amd import flops
    seqs = list(range(x.B if nseq <= 0 else min(nseq, x.B)))
    L = np.diff(x.offsets)
    s1 = int(x.offsets[seqs[-1] + 1])
    nc = None if x.num_candidates is None else x.num_candidates[:len(seqs)]
    t0 = time.perf_counter()
    ref = oracle.attn(x.q[:s1], x.k[:s1], x.v[:s1], x.offsets[:len(seqs) + 1], x.ts[:s1], x.rab_pos,
                      x.rab_time, x.alpha, num_candidates=nc)
    dt = time.perf_counter() - t0
    fl = flops.attn_flops(L[seqs], x.H, x.d, x.d, nc)
    rec = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
           "cpu_model": cpu_model(), "kind": "oracle", "seconds": dt,
           "sample": f"fp64 oracle attention (no epilogue) on sequences {seqs} of the same "
                     f"workload (lengths {[int(v) for v in L[seqs]]}, {x.H} heads), "
                     f"{fl / 1e9:.1f} GFLOP"}
    return rec, ref


def _err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = float(np.abs(ref).max()) or 1.0
    e = np.abs(got - ref)
    return {"max_err_rel": float(f"{e.max() / scale:.3e}"), "mean_err_rel": float(f"{e.mean() / scale:.3e}")}


def parity_record(case, x, ref_o=None, nseq=0):
    """One step of `case` against the oracle on its first nseq sequences (all
    when nseq <= 0; ref_o: the oracle's O of those rows if already computed):
    max and mean |err| / max|ref| of O, and of Y (or, for M-FALCON, of the
    scores); bf16 bounds 2e-2 (max) and 2e-3 (mean)."""
    import torch
    import oracle
    case.step()
    torch.cuda.synchronize()
    seqs = list(range(x.B if nseq <= 0 else min(nseq, x.B)))
    s1 = int(x.offsets[seqs[-1] + 1])
    nc = None if x.num_candidates is None else x.num_candidates[:len(seqs)]
    if ref_o is None:
        ref_o = oracle.attn(x.q[:s1], x.k[:s1], x.v[:s1], x.offsets[:len(seqs) + 1], x.ts[:s1],
                            x.rab_pos, x.rab_time, x.alpha, num_candidates=nc)
    o = case.o[:s1].float().cpu().numpy()
    rec = {"sample": f"sequences {seqs[0]}..{seqs[-1]} of {x.B} ({s1} rows)", "O": _err(o, ref_o)}
    if case.with_scores:
        ref_s = oracle.mfalcon_score(x.q[:s1], x.k[:s1], x.v[:s1], x.u[:s1], x.offsets[:len(seqs) + 1], nc,
                                     x.ts[:s1], x.rab_pos, x.rab_time, x.alpha, x.w, eps=x.eps)
        got_s = case.scores[:len(seqs), :ref_s.shape[1]].cpu().numpy()
        rec["scores"] = _err(got_s, ref_s)
    else:
        ref_y = oracle.ln_gate(ref_o.reshape(s1, -1), x.u[:s1].reshape(s1, -1), eps=x.eps)
        rec["Y"] = _err(case.y[:s1].float().cpu().numpy().reshape(s1, -1), ref_y)
    rec["pass"] = all(v["max_err_rel"] <= 2e-2 and v["mean_err_rel"] <= 2e-3
                      for k, v in rec.items() if isinstance(v, dict))
    return rec


def main():
    args = parse()
    global SETTLE_S
    SETTLE_S = max(0.0, args.settle)
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    import hstu_synth as synth
    from hstu_sequential_transducer_causal_amd import _lib, flops

    _lib.load()
    dev = torch.device("cuda:0")
    wl = args.workload
    log(f"generating workload {wl}")
    x = synth.config(wl)
    if args.only_sl_sweep:
        print(json.dumps({"workload": "hstu_sl_alpha_sweep_longseq_raw_b16_h8_d128",
                          **sl_sweep_record(dev, args.steps)}), flush=True)
        return
    if args.only_cached:
        c = CachedCase(dev)
        print(json.dumps({"workload": c.name, **c.record(args.steps)}), flush=True)
        return
    if args.only_layer_bwd:
        xl = synth.config(5)
        c = LayerBwdCase(xl, dev)
        st, _ = time_case(c, args.steps, args.warmup, core_events=False)
        lf = flops.layer_bwd_flops(np.diff(xl.offsets), xl.H, xl.d, xl.D)
        print(json.dumps({"workload": xl.name + "_layer0_bwd", "ms_per_step": round(st, 4),
                          "tflops": round(lf / (st * 1e-3) / 1e12, 2)}), flush=True)
        return
    if args.only_bwd:
        rec = bwd_record(x, dev, args.steps)
        print(json.dumps({"workload": x.name + "_bwd", **rec}), flush=True)
        return
    L = np.diff(x.offsets)
    if wl == 5:
        case = StackCase(x, dev)
        fl = 0
        for _ in range(x.layers):
            lf = flops.layer_flops(L, x.H, x.d, x.D)
            fl += lf["f1"] + lf["attn"] + lf["f2"]
        attn_fl_core = flops.attn_flops(L, x.H, x.d, x.d)
    else:
        case = AttnCase(x, dev, with_scores=(wl == 4))
        fl = flops.attn_flops(L, x.H, x.d, x.d, x.num_candidates)
        attn_fl_core = fl
    log(f"workload {x.name}: B={x.B} T={x.T} GFLOP/step={fl / 1e9:.2f}")

    # correctness of this very call path first: one step against the oracle
    # (the oracle's run on the host cores is also the CPU baseline)
    cpu_rec, parity = None, None
    if wl != 5:
        if not args.no_cpu_baseline:
            log("timing the oracle (CPU baseline) and checking one step against it")
            cpu_rec, ref_o = cpu_baseline(x, args.cpu_sample_seqs)
            parity = parity_record(case, x, ref_o, args.cpu_sample_seqs)
        else:
            parity = parity_record(case, x, None, 2)
        log(f"parity: {parity}")

    others = None
    if not args.no_others:
        others = {}
        for w in (2, 4, 5):
            if w == wl:
                continue
            xo = synth.config(w)
            Lo = np.diff(xo.offsets)
            if w == 5:
                c = StackCase(xo, dev)
                flo = sum(sum(flops.layer_flops(Lo, xo.H, xo.d, xo.D).values()) for _ in range(xo.layers))
                st, ce = time_case(c, max(2, args.steps // 10), 1, core_events=False)
            else:
                c = AttnCase(xo, dev, with_scores=(w == 4))
                flo = flops.attn_flops(Lo, xo.H, xo.d, xo.d, xo.num_candidates)
                st, ce = time_case(c, max(3, args.steps // 3), 2)
            rec = {"ms_per_step": round(st, 4), "tflops": round(flo / (st * 1e-3) / 1e12, 2),
                   "tokens_per_s": round(xo.T / (st * 1e-3), 1), "tokens": xo.T}
            if w != 5:
                rec["parity"] = parity_record(c, xo, None, 4 if w == 2 else 2)
            if ce:
                rec["core_ms"] = round(ce, 4)
                rec["core_tflops"] = round(flo / (ce * 1e-3) / 1e12, 2)
            if w == 4:
                rec["candidates_per_s"] = round(int(xo.num_candidates.sum()) / (st * 1e-3), 1)
            others[xo.name] = rec
            log(f"{xo.name}: {rec}")
            del c
            torch.cuda.empty_cache()
            if w == 4:
                # scores only: the query tiles holding candidate rows (their
                # unmasked pairs: b_m (n + 1) per user); same scores
                c = AttnCase(xo, dev, with_scores=True, candidates_only=True)
                st, ce = time_case(c, max(3, args.steps // 3), 2)
                n_hist = Lo - xo.num_candidates
                fc = float(np.sum(xo.num_candidates * (n_hist + 1))) * 4 * xo.d * xo.H
                rec = {"ms_per_step": round(st, 4),
                       "candidates_per_s": round(int(xo.num_candidates.sum()) / (st * 1e-3), 1),
                       "candidate_pair_tflops": round(fc / (st * 1e-3) / 1e12, 2),
                       "speedup_vs_full_pass": round(others[xo.name]["ms_per_step"] / st, 2)}
                if ce:
                    rec["core_ms"] = round(ce, 4)
                others[xo.name + "_candidates_only"] = rec
                log(f"{xo.name} candidates only: {rec}")
                del c
                torch.cuda.empty_cache()
                # the last layer of an M-FALCON stack, scores only
                recs = {}
                for co in (True, False):
                    c = LastLayerCase(dev, candidates_only=co)
                    st, _ = time_case(c, max(3, args.steps // 3), 2, core_events=False)
                    recs[co] = st
                    name = c.name
                    del c
                    torch.cuda.empty_cache()
                others[name] = {"ms_per_step": round(recs[True], 4),
                                "candidates_per_s": round(8 * 512 / (recs[True] * 1e-3), 1),
                                "all_rows_attention_ms": round(recs[False], 4)}
                log(f"{name}: {others[name]}")
                # many candidates per user against a cached history
                c = CachedCase(dev)
                rec = c.record(max(3, args.steps // 3))
                others[c.name] = rec
                log(f"{c.name}: {rec}")
                del c
                torch.cuda.empty_cache()
        sl_rec = sl_record(dev, max(3, args.steps // 3))
        others["hstu_sl_gather_longseq_raw_b16_cap2120"] = sl_rec
        log(f"stochastic length + gather: {sl_rec}")
        others["hstu_sl_alpha_sweep_longseq_raw_b16_h8_d128"] = sl_sweep_record(dev, max(3, args.steps // 6))
        xl = synth.config(5)
        c = LayerBwdCase(xl, dev)
        st, _ = time_case(c, max(2, args.steps // 10), 1, core_events=False)
        lf = flops.layer_bwd_flops(np.diff(xl.offsets), xl.H, xl.d, xl.D)
        rec = {"ms_per_step": round(st, 4), "tflops": round(lf / (st * 1e-3) / 1e12, 2),
               "tokens_per_s": round(xl.T / (st * 1e-3), 1), "tokens": xl.T,
               "flop_convention": "attention gradients at 8*d per visible pair and head plus the four "
                                  "weight/data products of f1 and f2; the recomputed forward not counted"}
        others[xl.name + "_layer0_bwd"] = rec
        log(f"{xl.name} layer-0 gradients: {rec}")
        del c
        torch.cuda.empty_cache()
        c = LayerBwdCase(xl, dev, saved=True)
        st, _ = time_case(c, max(2, args.steps // 10), 1, core_events=False)
        rec = {"ms_per_step": round(st, 4), "tflops": round(lf / (st * 1e-3) / 1e12, 2),
               "saved_mib": round(c.saved.numel() / 2**20, 1),
               "flop_convention": "as the recomputing gradients; Z, the pre-activation, O and Y kept by "
                                  "hstu_layer_fwd_saved instead of recomputed"}
        others[xl.name + "_layer0_bwd_saved"] = rec
        log(f"{xl.name} layer-0 gradients from saved activations: {rec}")
        del c
        torch.cuda.empty_cache()
        for w in (3, 4):
            xb = x if w == wl else synth.config(w)
            rec = bwd_record(xb, dev, max(3, args.steps // 3))
            others[xb.name + "_bwd"] = rec
            log(f"{xb.name} gradients: {rec}")
            torch.cuda.empty_cache()

    # the headline: untimed settle steps, W untimed warm-up steps, then K timed steps
    ms_step, core_ms = time_case(case, args.steps, args.warmup, core_events=(wl != 5),
                                 epi_events=(wl in (2, 3)))
    settle_steps = SETTLE_LOG[-1][1]
    value = fl / (ms_step * 1e-3) / 1e12
    tokens_s = x.T / (ms_step * 1e-3)
    log(f"step {ms_step:.3f} ms, core {core_ms} ms, {value:.1f} TFLOP/s")

    roofline = None
    if core_ms:
        ach = attn_fl_core / (core_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(x.name),
                    "kernel": "attn_bf16_kernel", "core_ms": round(core_ms, 4)}

    epilogue = None
    if getattr(case, "epi_ms", None):
        # LayerNorm(O) * U: O and U read once, Y written once (bf16)
        eb = 3 * x.T * x.H * x.d * 2
        gbs = eb / (case.epi_ms * 1e-3) / 1e9
        epilogue = {"bound": "hbm", "kernel": "ln_gate_rows_kernel", "ms": round(case.epi_ms, 4),
                    "bytes": eb, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4)}

    line = {
        "metric": "HSTU attention fwd TFLOP/s (unmasked) + jagged tokens/s; % bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle": {"seconds": SETTLE_S, "steps": settle_steps},
        "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": x.name, "global_batch": x.B, "tokens": x.T,
                   "max_seq_len": int(L.max()), "heads": x.H, "head_dim": x.d},
        "tokens_per_s": round(tokens_s, 1),
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "epilogue": epilogue,
        "parity": parity,
    }
    if others is not None:
        line["other_workloads"] = others
    line["cpu_baseline"] = cpu_rec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
