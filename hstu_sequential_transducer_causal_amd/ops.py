"""Python binding of libhstu.so: torch tensors in, torch tensors out.

Argument marshalling only -- every step of the path runs in the HIP kernels
behind include/hstu.h.  PyTorch provides device memory and the stream.
Names follow the C ABI: hstu_attn_fwd, hstu_attn_bwd, mfalcon_score, mfalcon_score_cached,
mfalcon_layer_score, hstu_layer_fwd, hstu_layer_bwd, hstu_stochastic_length, hstu_attn_schedule,
hstu_validate_offsets.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.HSTU_F32, torch.bfloat16: _lib.HSTU_BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _head_view_stride(t: torch.Tensor, H: int, d: int) -> int:
    """Row stride of a [rows, H, d] (or [rows, H*d]) view with dense heads."""
    if t.dim() == 3:
        if t.shape[1:] != (H, d) or t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError(f"expected [rows, {H}, {d}] with dense heads, got {tuple(t.shape)} "
                             f"strides {t.stride()}")
        return t.stride(0)
    if t.dim() == 2:
        if t.shape[1] != H * d or t.stride(1) != 1:
            raise ValueError(f"expected [rows, {H * d}] with unit column stride")
        return t.stride(0)
    raise ValueError("expected a 2-D or 3-D tensor")


def _empty_ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def make_attn_args(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, alpha, *,
                   max_seq_len: int, o: torch.Tensor, seq_lengths=None, num_candidates=None,
                   u=None, y=None, ln_eps: float = 1e-5, act: int = _lib.HSTU_ACT_SILU,
                   ev_core_begin=None, ev_core_end=None, ev_epi_begin=None,
                   ev_epi_end=None) -> _lib.AttnArgs:
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    H, d_qk = (q.shape[1], q.shape[2]) if q.dim() == 3 else (None, None)
    if H is None:
        raise ValueError("q must be [rows, H, d_qk]")
    d_v = v.shape[2] if v.dim() == 3 else v.shape[1] // H
    rp_hs = rab_pos.shape[-1] if rab_pos.dim() == 2 else 0
    rt_hs = rab_time.shape[-1] if rab_time.dim() == 2 else 0
    a = _lib.AttnArgs()
    a.struct_size = ctypes.sizeof(_lib.AttnArgs)
    a.B = seq_offsets.numel() - 1
    a.H = H
    a.d_qk = d_qk
    a.d_v = d_v
    a.max_seq_len = int(max_seq_len)
    a.num_rows = q.shape[0]
    a.seq_offsets = _ptr(seq_offsets)
    a.seq_lengths = _ptr(seq_lengths)
    a.num_candidates = _ptr(num_candidates)
    a.dtype = _DTYPES[q.dtype]
    a.act = act
    a.q, a.q_stride = q.data_ptr(), _head_view_stride(q, H, d_qk)
    a.k, a.k_stride = k.data_ptr(), _head_view_stride(k, H, d_qk)
    a.v, a.v_stride = v.data_ptr(), _head_view_stride(v, H, d_v)
    a.timestamps = timestamps.data_ptr()
    a.rab_pos = rab_pos.data_ptr()
    a.num_pos_buckets = rab_pos.shape[-1]
    a.rab_pos_head_stride = rp_hs
    a.rab_time = rab_time.data_ptr()
    a.num_time_buckets = rab_time.shape[-1]
    a.rab_time_head_stride = rt_hs
    a.alpha = float(alpha)
    a.o, a.o_stride = o.data_ptr(), _head_view_stride(o, H, d_v)
    if u is not None:
        a.u, a.u_stride = u.data_ptr(), _head_view_stride(u, H, d_v)
    if y is not None:
        a.y, a.y_stride = y.data_ptr(), _head_view_stride(y, H, d_v)
    a.ln_eps = float(ln_eps)
    a.ev_core_begin = ev_core_begin
    a.ev_core_end = ev_core_end
    a.ev_epi_begin = ev_epi_begin
    a.ev_epi_end = ev_epi_end
    return a


def hstu_attn_fwd(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, alpha, *,
                  max_seq_len: int, seq_lengths=None, num_candidates=None, u=None,
                  ln_eps: float = 1e-5, act: int = _lib.HSTU_ACT_SILU, o=None, y=None,
                  workspace=None, stream=None, ev_core_begin=None, ev_core_end=None,
                  ev_epi_begin=None, ev_epi_end=None):
    """O (and Y = LayerNorm(O) * U when ``u`` is given) of the jagged batch.

    q, k: [rows, H, d_qk]; v, u: [rows, H, d_v]; seq_offsets int32 [B+1];
    timestamps int64 [rows]; rab_pos float32 [P] or [H, P]; rab_time float32
    [NT] or [H, NT].  Returns (o, y) with y None when u is None.
    """
    lib = _lib.load()
    if o is None:
        o = torch.empty(q.shape[0], q.shape[1], v.shape[2], dtype=q.dtype, device=q.device)
    if u is not None and y is None:
        y = torch.empty_like(o)
    args = make_attn_args(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, alpha,
                          max_seq_len=max_seq_len, o=o, seq_lengths=seq_lengths,
                          num_candidates=num_candidates, u=u, y=y if u is not None else None,
                          ln_eps=ln_eps, act=act, ev_core_begin=ev_core_begin,
                          ev_core_end=ev_core_end, ev_epi_begin=ev_epi_begin, ev_epi_end=ev_epi_end)
    need = lib.hstu_attn_workspace_bytes(ctypes.byref(args))
    if workspace is None:
        workspace = _empty_ws(need, q.device)
    _lib.check(lib.hstu_attn_fwd(ctypes.byref(args), workspace.data_ptr(), workspace.numel(),
                                 _stream_ptr(stream)))
    return o, (y if u is not None else None)


def hstu_attn_fwd_noalloc(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, alpha, *,
                          max_seq_len: int, seq_lengths=None, num_candidates=None, u=None,
                          ln_eps: float = 1e-5, act: int = _lib.HSTU_ACT_SILU, o=None, y=None,
                          stream=None):
    """hstu_attn_fwd without a workspace (the library's own scratch buffer;
    for callers that cannot allocate).  o and y must be given: the call
    allocates nothing."""
    lib = _lib.load()
    if o is None or (u is not None and y is None):
        raise ValueError("hstu_attn_fwd_noalloc allocates nothing: pass o (and y with u)")
    args = make_attn_args(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, alpha,
                          max_seq_len=max_seq_len, o=o, seq_lengths=seq_lengths,
                          num_candidates=num_candidates, u=u, y=y if u is not None else None,
                          ln_eps=ln_eps, act=act)
    _lib.check(lib.hstu_attn_fwd_noalloc(ctypes.byref(args), _stream_ptr(stream)))
    return o, (y if u is not None else None)


def make_attn_bwd_args(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, alpha, *,
                       max_seq_len: int, dq, dk, dv, dout=None, dy=None, o=None, u=None,
                       du=None, ln_eps: float = 1e-5, seq_lengths=None, num_candidates=None,
                       act: int = _lib.HSTU_ACT_SILU, drab_pos=None, drab_time=None,
                       events=None) -> _lib.AttnBwdArgs:
    if (dout is None) == (dy is None):
        raise ValueError("give exactly one of dout and dy")
    args = _lib.AttnBwdArgs()
    args.struct_size = ctypes.sizeof(_lib.AttnBwdArgs)
    H, d = q.shape[1], v.shape[2]
    args.attn = make_attn_args(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, alpha,
                               max_seq_len=max_seq_len, o=o if o is not None else v,
                               seq_lengths=seq_lengths, num_candidates=num_candidates, u=u,
                               ln_eps=ln_eps, act=act)
    if o is None:
        args.attn.o = None
    if dy is not None:
        args.dy, args.dy_stride = dy.data_ptr(), _head_view_stride(dy, H, d)
        if du is not None:
            args.du, args.du_stride = du.data_ptr(), _head_view_stride(du, H, d)
    else:
        args.dout, args.dout_stride = dout.data_ptr(), _head_view_stride(dout, H, d)
    args.dq, args.dq_stride = dq.data_ptr(), _head_view_stride(dq, H, q.shape[2])
    args.dk, args.dk_stride = dk.data_ptr(), _head_view_stride(dk, H, q.shape[2])
    args.dv, args.dv_stride = dv.data_ptr(), _head_view_stride(dv, H, d)
    args.drab_pos = _ptr(drab_pos)
    args.drab_time = _ptr(drab_time)
    if events is not None:
        args.ev_dq_begin, args.ev_dq_end, args.ev_dkv_begin, args.ev_dkv_end = events
    return args


def attn_bwd_workspace_bytes(args: _lib.AttnBwdArgs) -> int:
    return int(_lib.load().hstu_attn_bwd_workspace_bytes(ctypes.byref(args)))


def hstu_attn_bwd(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, alpha, *,
                  max_seq_len: int, dout=None, dy=None, o=None, u=None, ln_eps: float = 1e-5,
                  seq_lengths=None, num_candidates=None, act: int = _lib.HSTU_ACT_SILU,
                  want_rab: bool = True, dq=None, dk=None, dv=None, du=None, drab_pos=None,
                  drab_time=None, workspace=None, stream=None, events=None):
    """Gradients of the attention path (bf16, d = 128).

    The upstream gradient is ``dout`` = dLoss/dO, or ``dy`` = dLoss/dY of
    Y = LayerNorm(O) * U (then ``o`` = the forward's O and ``u`` are
    required).  Returns (dq, dk, dv, du, drab_pos, drab_time): du is None
    without dy, the table gradients (float32, shaped like the tables) None
    unless ``want_rab``.  ``events`` = (dq begin, dq end, dkv begin, dkv end)
    raw hipEvent_t handles or None.
    """
    lib = _lib.load()
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dy is not None and du is None:
        du = torch.empty_like(v)
    if dy is None:
        du = None
    if want_rab:
        if drab_pos is None:
            drab_pos = torch.empty(rab_pos.shape, dtype=torch.float32, device=q.device)
        if drab_time is None:
            drab_time = torch.empty(rab_time.shape, dtype=torch.float32, device=q.device)
    else:
        drab_pos = drab_time = None
    args = make_attn_bwd_args(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, alpha,
                              max_seq_len=max_seq_len, dq=dq, dk=dk, dv=dv, dout=dout, dy=dy,
                              o=o, u=u, du=du, ln_eps=ln_eps, seq_lengths=seq_lengths,
                              num_candidates=num_candidates, act=act, drab_pos=drab_pos,
                              drab_time=drab_time, events=events)
    need = lib.hstu_attn_bwd_workspace_bytes(ctypes.byref(args))
    if need == 0:
        # invalid arguments: let the call itself report why
        _lib.check(lib.hstu_attn_bwd(ctypes.byref(args), None, 0, _stream_ptr(stream)))
    if workspace is None:
        workspace = _empty_ws(need, q.device)
    _lib.check(lib.hstu_attn_bwd(ctypes.byref(args), workspace.data_ptr(), workspace.numel(),
                                 _stream_ptr(stream)))
    return dq, dk, dv, du, drab_pos, drab_time


def attn_workspace_bytes(args: _lib.AttnArgs) -> int:
    return int(_lib.load().hstu_attn_workspace_bytes(ctypes.byref(args)))


def mfalcon_score(q, k, v, u, seq_offsets, num_candidates, timestamps, rab_pos, rab_time, alpha,
                  w, *, max_seq_len: int, score_stride: int, ln_eps: float = 1e-5, o=None,
                  y=None, scores=None, workspace=None, stream=None, ev_core_begin=None,
                  ev_core_end=None, candidates_only: bool = False):
    """M-FALCON ranking scores [B, score_stride] (fp32) of every candidate.

    candidates_only: compute only the query tiles that hold candidate rows
    (y must be None; history rows of `o` outside those tiles stay unwritten)."""
    lib = _lib.load()
    B = seq_offsets.numel() - 1
    if o is None:
        o = torch.empty(q.shape[0], q.shape[1], v.shape[2], dtype=q.dtype, device=q.device)
    if scores is None:
        scores = torch.zeros(B, score_stride, dtype=torch.float32, device=q.device)
    m = _lib.MfalconArgs()
    m.struct_size = ctypes.sizeof(_lib.MfalconArgs)
    m.attn = make_attn_args(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, alpha,
                            max_seq_len=max_seq_len, o=o, num_candidates=num_candidates, u=u,
                            y=y, ln_eps=ln_eps, ev_core_begin=ev_core_begin,
                            ev_core_end=ev_core_end)
    m.w = w.data_ptr()
    m.scores = scores.data_ptr()
    m.score_stride = int(score_stride)
    m.candidates_only = 1 if candidates_only else 0
    need = lib.hstu_mfalcon_workspace_bytes(ctypes.byref(m))
    if workspace is None:
        workspace = _empty_ws(need, q.device)
    _lib.check(lib.mfalcon_score(ctypes.byref(m), workspace.data_ptr(), workspace.numel(),
                                 _stream_ptr(stream)))
    return scores, o, y


def make_mfalcon_cached_args(k_hist, v_hist, hist_offsets, ts_hist, q, k, v, u, cand_offsets,
                             ts_cand, rab_pos, rab_time, alpha, w, *, max_hist_len: int,
                             max_cands: int, scores, score_stride: int, o=None,
                             ln_eps: float = 1e-5, ev_core_begin=None,
                             ev_core_end=None) -> _lib.MfalconCachedArgs:
    if q.dim() != 3:
        raise ValueError("q must be [candidate rows, H, d]")
    H, d = q.shape[1], q.shape[2]
    m = _lib.MfalconCachedArgs()
    m.struct_size = ctypes.sizeof(_lib.MfalconCachedArgs)
    m.B = hist_offsets.numel() - 1
    m.H, m.d = H, d
    m.max_hist_len, m.max_cands = int(max_hist_len), int(max_cands)
    m.hist_offsets, m.num_hist_rows = hist_offsets.data_ptr(), k_hist.shape[0]
    m.k_hist, m.k_hist_stride = _ptr(k_hist), _head_view_stride(k_hist, H, d)
    m.v_hist, m.v_hist_stride = _ptr(v_hist), _head_view_stride(v_hist, H, d)
    m.ts_hist = ts_hist.data_ptr()
    m.cand_offsets, m.num_cand_rows = cand_offsets.data_ptr(), q.shape[0]
    m.q, m.q_stride = _ptr(q), _head_view_stride(q, H, d)
    m.k, m.k_stride = _ptr(k), _head_view_stride(k, H, d)
    m.v, m.v_stride = _ptr(v), _head_view_stride(v, H, d)
    m.u, m.u_stride = _ptr(u), _head_view_stride(u, H, d)
    m.ts_cand = ts_cand.data_ptr()
    m.rab_pos, m.num_pos_buckets = rab_pos.data_ptr(), rab_pos.shape[-1]
    m.rab_pos_head_stride = rab_pos.shape[-1] if rab_pos.dim() == 2 else 0
    m.rab_time, m.num_time_buckets = rab_time.data_ptr(), rab_time.shape[-1]
    m.rab_time_head_stride = rab_time.shape[-1] if rab_time.dim() == 2 else 0
    m.alpha, m.ln_eps = float(alpha), float(ln_eps)
    m.w, m.scores, m.score_stride = w.data_ptr(), scores.data_ptr(), int(score_stride)
    m.o, m.o_stride = (_ptr(o), _head_view_stride(o, H, d)) if o is not None else (None, 0)
    m.ev_core_begin, m.ev_core_end = ev_core_begin, ev_core_end
    return m


def mfalcon_cached_workspace_bytes(m: _lib.MfalconCachedArgs) -> int:
    return int(_lib.load().hstu_mfalcon_cached_workspace_bytes(ctypes.byref(m)))


def mfalcon_score_cached(k_hist, v_hist, hist_offsets, ts_hist, q, k, v, u, cand_offsets,
                         ts_cand, rab_pos, rab_time, alpha, w, *, max_hist_len: int,
                         max_cands: int, score_stride: int, ln_eps: float = 1e-5, o=None,
                         scores=None, workspace=None, stream=None, ev_core_begin=None,
                         ev_core_end=None):
    """Scores [B, score_stride] (fp32) of every candidate against a cached
    history (keys/values [hist rows, H, d]); returns (scores, o) where o is
    the candidates' attention output when given, else None."""
    lib = _lib.load()
    B = hist_offsets.numel() - 1
    if scores is None:
        scores = torch.zeros(B, score_stride, dtype=torch.float32, device=q.device)
    m = make_mfalcon_cached_args(k_hist, v_hist, hist_offsets, ts_hist, q, k, v, u, cand_offsets,
                                 ts_cand, rab_pos, rab_time, alpha, w, max_hist_len=max_hist_len,
                                 max_cands=max_cands, scores=scores, score_stride=score_stride,
                                 o=o, ln_eps=ln_eps, ev_core_begin=ev_core_begin,
                                 ev_core_end=ev_core_end)
    need = lib.hstu_mfalcon_cached_workspace_bytes(ctypes.byref(m))
    if workspace is None:
        workspace = _empty_ws(need, q.device)
    _lib.check(lib.mfalcon_score_cached(ctypes.byref(m), workspace.data_ptr(), workspace.numel(),
                                        _stream_ptr(stream)))
    return scores, o


def make_layer_args(x, w1, w2, seq_offsets, timestamps, rab_pos, rab_time, alpha, *, H: int,
                    d: int, max_seq_len: int, x_out, b1=None, b2=None, num_candidates=None,
                    ln_eps: float = 1e-5) -> _lib.LayerArgs:
    """Argument struct of one layer; w2 and x_out may be None for the scoring
    layer (mfalcon_layer_score)."""
    l = _lib.LayerArgs()
    l.struct_size = ctypes.sizeof(_lib.LayerArgs)
    l.B = seq_offsets.numel() - 1
    l.H, l.d, l.D = H, d, x.shape[1]
    l.max_seq_len = int(max_seq_len)
    l.num_rows = x.shape[0]
    l.seq_offsets = seq_offsets.data_ptr()
    l.num_candidates = _ptr(num_candidates)
    for name, t in (("x", x), ("w1", w1), ("w2", w2), ("x_out", x_out)):
        if t is not None and (t.dtype != torch.bfloat16 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor")
    l.x, l.w1, l.w2, l.x_out = x.data_ptr(), w1.data_ptr(), _ptr(w2), _ptr(x_out)
    l.b1, l.b2 = _ptr(b1), _ptr(b2)
    l.timestamps = timestamps.data_ptr()
    l.rab_pos, l.num_pos_buckets = rab_pos.data_ptr(), rab_pos.shape[-1]
    l.rab_time, l.num_time_buckets = rab_time.data_ptr(), rab_time.shape[-1]
    l.alpha = float(alpha)
    l.ln_eps = float(ln_eps)
    return l


def mfalcon_layer_score(x, w1, seq_offsets, num_candidates, timestamps, rab_pos, rab_time, alpha,
                        w, *, H: int, d: int, max_seq_len: int, score_stride: int, b1=None,
                        ln_eps: float = 1e-5, candidates_only: bool = True, scores=None,
                        workspace=None, stream=None):
    """Scores [B, score_stride] (fp32) of every candidate after the last layer
    (f1 + SiLU over all rows, attention, LN * U on the candidate rows)."""
    lib = _lib.load()
    B = seq_offsets.numel() - 1
    if scores is None:
        scores = torch.zeros(B, score_stride, dtype=torch.float32, device=x.device)
    m = _lib.MfalconLayerArgs()
    m.struct_size = ctypes.sizeof(_lib.MfalconLayerArgs)
    m.layer = make_layer_args(x, w1, None, seq_offsets, timestamps, rab_pos, rab_time, alpha, H=H,
                              d=d, max_seq_len=max_seq_len, x_out=None, b1=b1,
                              num_candidates=num_candidates, ln_eps=ln_eps)
    m.w, m.scores, m.score_stride = w.data_ptr(), scores.data_ptr(), int(score_stride)
    m.candidates_only = 1 if candidates_only else 0
    need = lib.hstu_mfalcon_layer_workspace_bytes(ctypes.byref(m))
    if workspace is None:
        workspace = _empty_ws(need, x.device)
    _lib.check(lib.mfalcon_layer_score(ctypes.byref(m), workspace.data_ptr(), workspace.numel(),
                                       _stream_ptr(stream)))
    return scores


def hstu_layer_fwd(x, w1, w2, seq_offsets, timestamps, rab_pos, rab_time, alpha, *, H: int,
                   d: int, max_seq_len: int, b1=None, b2=None, num_candidates=None,
                   ln_eps: float = 1e-5, x_out=None, workspace=None, saved=None, stream=None):
    """One HSTU layer (f1 + SiLU, attention, LN * U, f2 + residual); returns X_out.
    With `saved` (a uint8 device tensor of layer_saved_bytes() bytes) the
    activations the gradients need are kept there (hstu_layer_fwd_saved)."""
    lib = _lib.load()
    if x_out is None:
        x_out = torch.empty_like(x)
    l = make_layer_args(x, w1, w2, seq_offsets, timestamps, rab_pos, rab_time, alpha, H=H, d=d,
                        max_seq_len=max_seq_len, x_out=x_out, b1=b1, b2=b2,
                        num_candidates=num_candidates, ln_eps=ln_eps)
    need = lib.hstu_layer_workspace_bytes(ctypes.byref(l))
    if workspace is None:
        workspace = _empty_ws(need, x.device)
    if saved is None:
        _lib.check(lib.hstu_layer_fwd(ctypes.byref(l), workspace.data_ptr(), workspace.numel(),
                                      _stream_ptr(stream)))
    else:
        _lib.check(lib.hstu_layer_fwd_saved(ctypes.byref(l), saved.data_ptr(), saved.numel(),
                                            workspace.data_ptr(), workspace.numel(), _stream_ptr(stream)))
    return x_out


def layer_saved_bytes(x, w1, w2, seq_offsets, timestamps, rab_pos, rab_time, alpha, *, H: int, d: int,
                      max_seq_len: int, num_candidates=None) -> int:
    """Bytes of the buffer hstu_layer_fwd_saved keeps the activations in."""
    l = make_layer_args(x, w1, w2, seq_offsets, timestamps, rab_pos, rab_time, alpha, H=H, d=d,
                        max_seq_len=max_seq_len, x_out=x, num_candidates=num_candidates)
    return int(_lib.load().hstu_layer_saved_bytes(ctypes.byref(l)))


def make_layer_bwd_args(x, w1, w2, seq_offsets, timestamps, rab_pos, rab_time, alpha, dx_out, *,
                        H: int, d: int, max_seq_len: int, dx, dw1, dw2, b1=None, b2=None, db1=None,
                        db2=None, drab_pos=None, drab_time=None, num_candidates=None,
                        ln_eps: float = 1e-5) -> _lib.LayerBwdArgs:
    g = _lib.LayerBwdArgs()
    g.struct_size = ctypes.sizeof(_lib.LayerBwdArgs)
    g.layer = make_layer_args(x, w1, w2, seq_offsets, timestamps, rab_pos, rab_time, alpha, H=H, d=d,
                              max_seq_len=max_seq_len, x_out=x, b1=b1, b2=b2,
                              num_candidates=num_candidates, ln_eps=ln_eps)
    g.layer.x_out = None
    g.dx_out, g.dx = dx_out.data_ptr(), dx.data_ptr()
    g.dw1, g.dw2 = dw1.data_ptr(), dw2.data_ptr()
    g.db1, g.db2 = _ptr(db1), _ptr(db2)
    g.drab_pos, g.drab_time = _ptr(drab_pos), _ptr(drab_time)
    return g


def layer_bwd_workspace_bytes(g: _lib.LayerBwdArgs, saved: bool = False) -> int:
    """Workspace of hstu_layer_bwd, or (saved) of hstu_layer_bwd_saved."""
    lib = _lib.load()
    f = lib.hstu_layer_bwd_saved_workspace_bytes if saved else lib.hstu_layer_bwd_workspace_bytes
    return int(f(ctypes.byref(g)))


def hstu_layer_bwd(x, w1, w2, seq_offsets, timestamps, rab_pos, rab_time, alpha, dx_out, *, H: int,
                   d: int, max_seq_len: int, b1=None, b2=None, num_candidates=None,
                   ln_eps: float = 1e-5, want_bias: bool = True, want_rab: bool = True, dx=None,
                   workspace=None, saved=None, stream=None):
    """Gradients of one HSTU layer for dLoss/dX_out: returns a dict with dx
    (bf16 [rows, D]), dw1 [4Hd, D], dw2 [D, Hd] and, if asked for, db1, db2,
    drab_pos, drab_time (all float32)."""
    lib = _lib.load()
    dev = x.device
    zw, D = 4 * H * d, x.shape[1]
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty_like(x) if dx is None else dx,
           "dw1": torch.empty(zw, D, **f32), "dw2": torch.empty(D, H * d, **f32),
           "db1": torch.empty(zw, **f32) if want_bias else None,
           "db2": torch.empty(D, **f32) if want_bias else None,
           "drab_pos": torch.empty(rab_pos.shape, **f32) if want_rab else None,
           "drab_time": torch.empty(rab_time.shape, **f32) if want_rab else None}
    g = make_layer_bwd_args(x, w1, w2, seq_offsets, timestamps, rab_pos, rab_time, alpha, dx_out,
                            H=H, d=d, max_seq_len=max_seq_len, dx=out["dx"], dw1=out["dw1"],
                            dw2=out["dw2"], b1=b1, b2=b2, db1=out["db1"], db2=out["db2"],
                            drab_pos=out["drab_pos"], drab_time=out["drab_time"],
                            num_candidates=num_candidates, ln_eps=ln_eps)
    need = layer_bwd_workspace_bytes(g, saved=saved is not None)
    if need == 0:
        _lib.check(lib.hstu_layer_bwd(ctypes.byref(g), None, 0, _stream_ptr(stream)))
    if workspace is None:
        workspace = _empty_ws(need, dev)
    if saved is None:
        _lib.check(lib.hstu_layer_bwd(ctypes.byref(g), workspace.data_ptr(), workspace.numel(),
                                      _stream_ptr(stream)))
    else:   # the activations a training forward kept (hstu_layer_bwd_saved)
        _lib.check(lib.hstu_layer_bwd_saved(ctypes.byref(g), saved.data_ptr(), saved.numel(),
                                            workspace.data_ptr(), workspace.numel(), _stream_ptr(stream)))
    return out


def stochastic_length(seq_offsets, cap, *, seed: int, step: int = 0, caps=None, tensors=(),
                      out_index=None, stream=None):
    """Seeded order-preserving subsampling of every sequence to at most
    ``cap`` (or ``caps[b]``) rows, with the kept rows of ``tensors`` (each
    [rows, ...] with contiguous rows) gathered into packed outputs.

    Returns (out_offsets int32 [B+1], out_index int64 [rows] -- valid up to
    out_offsets[B] -- and the list of gathered tensors, each with as many
    rows as its source; rows past out_offsets[B] are left unwritten).
    """
    lib = _lib.load()
    dev = seq_offsets.device
    B = seq_offsets.numel() - 1
    rows = tensors[0].shape[0] if tensors else None
    a = _lib.SlArgs()
    a.struct_size = ctypes.sizeof(_lib.SlArgs)
    a.B = B
    out_off = torch.empty(B + 1, dtype=torch.int32, device=dev)
    if rows is None:
        rows = int(seq_offsets[-1].item()) if B > 0 else 0
    a.num_rows = rows
    out_index = torch.empty(max(rows, 1), dtype=torch.int64, device=dev) if out_index is None else out_index
    a.seq_offsets = seq_offsets.data_ptr()
    a.cap = int(cap)
    a.caps = _ptr(caps)
    a.seed = int(seed) & ((1 << 64) - 1)
    a.step = int(step) & ((1 << 64) - 1)
    a.out_offsets = out_off.data_ptr()
    a.out_index = out_index.data_ptr()
    if len(tensors) > _lib.SL_MAX_TENSORS:
        raise ValueError(f"at most {_lib.SL_MAX_TENSORS} tensors")
    outs = []
    a.num_tensors = len(tensors)
    for t, x in enumerate(tensors):
        if x.shape[0] != rows or not x[0].is_contiguous():
            raise ValueError("tensors need the same row count and contiguous rows")
        y = torch.empty_like(x)
        rb = x[0].numel() * x.element_size()
        a.src[t], a.src_stride[t] = x.data_ptr(), x.stride(0) * x.element_size()
        a.dst[t], a.dst_stride[t] = y.data_ptr(), y.stride(0) * y.element_size()
        a.row_bytes[t] = rb
        outs.append(y)
    _lib.check(lib.hstu_stochastic_length(ctypes.byref(a), _stream_ptr(stream)))
    return out_off, out_index, outs


def layer_workspace_bytes(l: _lib.LayerArgs) -> int:
    return int(_lib.load().hstu_layer_workspace_bytes(ctypes.byref(l)))


def hstu_attn_schedule(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, *, max_seq_len: int,
                       seq_lengths=None, num_candidates=None, stream=None):
    """The device-built work list as a host int32 array [count, 8] plus (tile_m, tile_n)."""
    import numpy as np
    lib = _lib.load()
    args = make_attn_args(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, 1.0,
                          max_seq_len=max_seq_len, o=torch.empty_like(v),
                          seq_lengths=seq_lengths, num_candidates=num_candidates)
    need = lib.hstu_attn_workspace_bytes(ctypes.byref(args))
    ws = _empty_ws(need, q.device)
    B = seq_offsets.numel() - 1
    cap = max(1, B * ((max_seq_len + 63) // 64)) + 1024   # row blocks + split pieces
    items = np.zeros((cap, 8), dtype=np.int32)
    count = ctypes.c_int64(0)
    tm, tn = ctypes.c_int32(0), ctypes.c_int32(0)
    _lib.check(lib.hstu_attn_schedule(ctypes.byref(args), ws.data_ptr(), ws.numel(),
                                      items.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), cap,
                                      ctypes.byref(count), ctypes.byref(tm), ctypes.byref(tn),
                                      _stream_ptr(stream)))
    return items[:count.value], tm.value, tn.value


def hstu_validate_offsets(seq_offsets, *, num_rows: int, max_seq_len: int, seq_lengths=None,
                          num_candidates=None, stream=None) -> None:
    """Checks the device batch structure (offsets, lengths, candidate counts);
    raises HstuError (HSTU_ERR_ARG) naming the first failing sequence."""
    lib = _lib.load()
    a = _lib.AttnArgs()
    a.struct_size = ctypes.sizeof(_lib.AttnArgs)
    a.B = seq_offsets.numel() - 1
    a.num_rows = num_rows
    a.max_seq_len = max_seq_len
    a.seq_offsets = seq_offsets.data_ptr()
    a.seq_lengths = seq_lengths.data_ptr() if seq_lengths is not None else None
    a.num_candidates = num_candidates.data_ptr() if num_candidates is not None else None
    _lib.check(lib.hstu_validate_offsets(ctypes.byref(a), _stream_ptr(stream)))
