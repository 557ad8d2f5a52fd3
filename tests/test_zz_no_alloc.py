"""hstu_attn_fwd_noalloc (the entry point that allocates nothing, for callers
that cannot allocate) against hstu_attn_fwd on the same inputs: two calls in
a row, the second on a smaller batch (the library's scratch buffer keeps the
first call's contents), plus a batch whose long row blocks are split over
their key tiles (partial sums in the scratch buffer)."""
import numpy as np
import pytest

import hstu_synth as synth
from hstu_testlib import DeviceAttn, assert_close, host_f32, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hstu_sequential_transducer_causal_amd import _lib
    _lib.load()


def _both(x):
    import torch
    from hstu_sequential_transducer_causal_amd import ops
    d = DeviceAttn(x)
    kw = dict(max_seq_len=d.max_seq_len, seq_lengths=d.lengths, num_candidates=d.ncand, u=d.u,
              ln_eps=x.eps)
    o_ref, y_ref = ops.hstu_attn_fwd(d.q, d.k, d.v, d.offsets, d.ts, d.rab_pos, d.rab_time, x.alpha, **kw)
    o = torch.full_like(o_ref, float("nan"))
    y = torch.full_like(y_ref, float("nan"))
    ops.hstu_attn_fwd_noalloc(d.q, d.k, d.v, d.offsets, d.ts, d.rab_pos, d.rab_time, x.alpha, o=o, y=y, **kw)
    torch.cuda.synchronize()
    return host_f32(o), host_f32(o_ref), host_f32(y), host_f32(y_ref)


@pytest.mark.parametrize("case", ["split blocks then a small batch", "M-FALCON then a small batch"])
def test_noalloc_matches_hstu_attn_fwd_twice(case):
    if case.startswith("split"):
        first = synth.config(3, batch=2, max_len=1200)   # long row blocks: split over key tiles
    else:
        first = synth.config(4, batch=3, max_len=700)
    second = synth.config(2, batch=3, max_len=200)        # smaller: stale scratch must not leak
    for k, x in enumerate((first, second)):
        o, o_ref, y, y_ref = _both(x)
        same = np.array_equal(o, o_ref) and np.array_equal(y, y_ref)
        log(f"noalloc {case}, call {k + 1} (T={x.T}): bit-identical to hstu_attn_fwd: {same}")
        assert_close(o, o_ref, "bf16", f"noalloc call {k + 1} O")
        assert_close(y, y_ref, "bf16", f"noalloc call {k + 1} Y")
