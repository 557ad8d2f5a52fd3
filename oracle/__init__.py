"""fp64 CPU oracle of the HSTU attention path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``hstu_oracle.c`` (plain fp64
loops, OpenMP over independent (sequence, head) units) through ctypes and
shares nothing with the HIP library.

Functions take numpy arrays; floating inputs are upcast to float64 exactly
(bf16/fp32 values are exact in fp64).  Parity status of each function is
stated in its docstring; all are pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

ACT_SILU = 0
ACT_IDENTITY = 1

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.library_path()
        if not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        lib.hstu_oracle_time_bucket.restype = ctypes.c_int32
        lib.hstu_oracle_time_bucket.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
        lib.hstu_oracle_pos_bucket.restype = ctypes.c_int32
        lib.hstu_oracle_pos_bucket.argtypes = [ctypes.c_int32] * 4
        lib.hstu_oracle_visible.restype = ctypes.c_int32
        lib.hstu_oracle_visible.argtypes = [ctypes.c_int32] * 4
        lib.hstu_oracle_silu.restype = ctypes.c_double
        lib.hstu_oracle_silu.argtypes = [ctypes.c_double]
        lib.hstu_oracle_max_threads.restype = ctypes.c_int32
        lib.hstu_oracle_attn.restype = None
        lib.hstu_oracle_attn_rows.restype = None
        lib.hstu_oracle_ln_gate.restype = None
        lib.hstu_oracle_attn_bwd.restype = None
        lib.hstu_oracle_attn_bwd_rows.restype = None
        lib.hstu_oracle_ln_gate_bwd.restype = None
        lib.hstu_oracle_layer_bwd.restype = None
        lib.hstu_oracle_layer.restype = None
        lib.hstu_oracle_mfalcon_score.restype = None
        lib.hstu_oracle_layer_scores.restype = None
        lib.hstu_oracle_tiles.restype = ctypes.c_int64
        lib.hstu_oracle_count_visible.restype = ctypes.c_int64
        _LIB = lib
    return _LIB


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray], typ):
    if a is None:
        return ctypes.cast(None, typ)
    return a.ctypes.data_as(typ)


def _i32(a) -> Optional[np.ndarray]:
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def max_threads() -> int:
    return int(_lib().hstu_oracle_max_threads())


# ---------------------------------------------------------------------------
# scalar definitions
# ---------------------------------------------------------------------------
def time_bucket(t_i: int, t_j: int, num_time_buckets: int = 32) -> int:
    return int(_lib().hstu_oracle_time_bucket(int(t_i), int(t_j), int(num_time_buckets)))


def pos_bucket(i: int, j: int, n_hist: int, num_pos_buckets: int) -> int:
    return int(_lib().hstu_oracle_pos_bucket(int(i), int(j), int(n_hist), int(num_pos_buckets)))


def visible(i: int, j: int, L: int, n_hist: int) -> bool:
    return bool(_lib().hstu_oracle_visible(int(i), int(j), int(L), int(n_hist)))


def silu(x: float) -> float:
    return float(_lib().hstu_oracle_silu(float(x)))


# ---------------------------------------------------------------------------
# array functions
# ---------------------------------------------------------------------------
def attn(q, k, v, offsets, ts, rab_pos, rab_time, alpha, *, lengths=None,
         num_candidates=None, act=ACT_SILU, num_threads=0, out=None) -> np.ndarray:
    """O[T, H, d_v] = alpha * sum_j act(QK^T + rab_pos + rab_time) V over visible pairs.

    q, k: [T, H, d_qk]; v: [T, H, d_v]; ts: int64 [T]; rab_* : [P] / [NT]
    shared, or [H, P] / [H, NT] per head.  Padding rows (lengths given) of
    the result are left at 0 (or at ``out``'s values).
    """
    q = _f64(q); k = _f64(k); v = _f64(v)
    T, H, dqk = q.shape
    dv = v.shape[2]
    off = _i32(offsets)
    B = len(off) - 1
    rp = _f64(rab_pos); rt = _f64(rab_time)
    P = rp.shape[-1]; NT = rt.shape[-1]
    rps = P if rp.ndim == 2 else 0
    rts = NT if rt.ndim == 2 else 0
    o = np.zeros((T, H, dv), dtype=np.float64) if out is None else out
    tsa = np.ascontiguousarray(ts, dtype=np.int64)
    ln = _i32(lengths); nc = _i32(num_candidates)
    _lib().hstu_oracle_attn(
        ctypes.c_int32(B), ctypes.c_int32(H), ctypes.c_int32(dqk), ctypes.c_int32(dv),
        _ptr(off, _i32p), _ptr(ln, _i32p), _ptr(nc, _i32p),
        _ptr(q, _f64p), ctypes.c_int64(H * dqk), _ptr(k, _f64p), ctypes.c_int64(H * dqk),
        _ptr(v, _f64p), ctypes.c_int64(H * dv), _ptr(tsa, _i64p),
        _ptr(rp, _f64p), ctypes.c_int32(P), _ptr(rt, _f64p), ctypes.c_int32(NT),
        ctypes.c_int64(rps), ctypes.c_int64(rts), ctypes.c_double(alpha), ctypes.c_int32(act),
        _ptr(o, _f64p), ctypes.c_int64(H * dv), ctypes.c_int32(num_threads))
    return o


def attn_rows(q, k, v, offsets, ts, rab_pos, rab_time, alpha, rows, *, lengths=None,
              num_candidates=None, act=ACT_SILU, num_threads=0) -> np.ndarray:
    """O[rows[r], H, d_v] of selected rows of the jagged batch (the definition
    of ``attn``, evaluated row by row: O(L d) per row)."""
    q = _f64(q); k = _f64(k); v = _f64(v)
    T, H, dqk = q.shape
    dv = v.shape[2]
    off = _i32(offsets)
    B = len(off) - 1
    rp = _f64(rab_pos); rt = _f64(rab_time)
    P = rp.shape[-1]; NT = rt.shape[-1]
    rps = P if rp.ndim == 2 else 0
    rts = NT if rt.ndim == 2 else 0
    rw = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((len(rw), H, dv), dtype=np.float64)
    tsa = np.ascontiguousarray(ts, dtype=np.int64)
    ln = _i32(lengths); nc = _i32(num_candidates)
    _lib().hstu_oracle_attn_rows(
        ctypes.c_int32(B), ctypes.c_int32(H), ctypes.c_int32(dqk), ctypes.c_int32(dv),
        _ptr(off, _i32p), _ptr(ln, _i32p), _ptr(nc, _i32p),
        _ptr(q, _f64p), ctypes.c_int64(H * dqk), _ptr(k, _f64p), ctypes.c_int64(H * dqk),
        _ptr(v, _f64p), ctypes.c_int64(H * dv), _ptr(tsa, _i64p),
        _ptr(rp, _f64p), ctypes.c_int32(P), _ptr(rt, _f64p), ctypes.c_int32(NT),
        ctypes.c_int64(rps), ctypes.c_int64(rts), ctypes.c_double(alpha), ctypes.c_int32(act),
        ctypes.c_int64(len(rw)), _ptr(rw, _i64p), _ptr(out, _f64p), ctypes.c_int32(num_threads))
    return out


def ln_gate(o, u, eps=1e-5, num_threads=0) -> np.ndarray:
    """Y[r, :] = LayerNorm(o[r, :]) * u[r, :] over the whole row (biased var)."""
    o2 = _f64(o).reshape(o.shape[0], -1)
    u2 = _f64(u).reshape(u.shape[0], -1)
    rows, width = o2.shape
    y = np.empty_like(o2)
    _lib().hstu_oracle_ln_gate(
        ctypes.c_int64(rows), ctypes.c_int32(width), _ptr(o2, _f64p), ctypes.c_int64(width),
        _ptr(u2, _f64p), ctypes.c_int64(width), ctypes.c_double(eps), _ptr(y, _f64p),
        ctypes.c_int64(width), ctypes.c_int32(num_threads))
    return y


def attn_bwd(q, k, v, offsets, ts, rab_pos, rab_time, alpha, dout, *, lengths=None,
             num_candidates=None, act=ACT_SILU, num_threads=0):
    """Gradients of the attention core for an upstream gradient ``dout`` of O.

    Returns (dq, dk, dv, drab_pos, drab_time): dq, dk [T, H, d_qk], dv
    [T, H, d_v] (padding rows 0), and the table gradients shaped like the
    tables ([P] / [NT] summed over heads when shared, [H, P] / [H, NT] per
    head).  Chain rule through the forward definition, one (sequence, head)
    at a time, i then j ascending.  Pinned by central finite differences of
    ``attn`` (tests/test_oracle_pins.py).
    """
    q = _f64(q); k = _f64(k); v = _f64(v); g = _f64(dout)
    T, H, dqk = q.shape
    dv_ = v.shape[2]
    off = _i32(offsets)
    B = len(off) - 1
    rp = _f64(rab_pos); rt = _f64(rab_time)
    P = rp.shape[-1]; NT = rt.shape[-1]
    rps = P if rp.ndim == 2 else 0
    rts = NT if rt.ndim == 2 else 0
    dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
    drp = np.zeros_like(rp); drt = np.zeros_like(rt)
    tsa = np.ascontiguousarray(ts, dtype=np.int64)
    ln = _i32(lengths); nc = _i32(num_candidates)
    _lib().hstu_oracle_attn_bwd(
        ctypes.c_int32(B), ctypes.c_int32(H), ctypes.c_int32(dqk), ctypes.c_int32(dv_),
        _ptr(off, _i32p), _ptr(ln, _i32p), _ptr(nc, _i32p),
        _ptr(q, _f64p), _ptr(k, _f64p), _ptr(v, _f64p), ctypes.c_int64(H * dqk),
        ctypes.c_int64(H * dv_), _ptr(tsa, _i64p),
        _ptr(rp, _f64p), ctypes.c_int32(P), _ptr(rt, _f64p), ctypes.c_int32(NT),
        ctypes.c_int64(rps), ctypes.c_int64(rts), ctypes.c_double(alpha), ctypes.c_int32(act),
        _ptr(g, _f64p), _ptr(dq, _f64p), _ptr(dk, _f64p), _ptr(dv, _f64p),
        _ptr(drp, _f64p), _ptr(drt, _f64p), ctypes.c_int32(num_threads))
    return dq, dk, dv, drp, drt


def attn_bwd_rows(q, k, v, offsets, ts, rab_pos, rab_time, alpha, dout, qrows, krows, *,
                  lengths=None, num_candidates=None, act=ACT_SILU, num_threads=0):
    """dQ at the query rows ``qrows`` and dK, dV at the key rows ``krows`` of
    the jagged batch: the sums of ``attn_bwd``, in its order, per row
    (O(L d) each; no table gradients).  Returns (dq [nq, H, d_qk],
    dk [nk, H, d_qk], dv [nk, H, d_v])."""
    q = _f64(q); k = _f64(k); v = _f64(v); g = _f64(dout)
    T, H, dqk = q.shape
    dv_ = v.shape[2]
    off = _i32(offsets)
    B = len(off) - 1
    rp = _f64(rab_pos); rt = _f64(rab_time)
    P = rp.shape[-1]; NT = rt.shape[-1]
    rps = P if rp.ndim == 2 else 0
    rts = NT if rt.ndim == 2 else 0
    qr = np.ascontiguousarray(qrows, dtype=np.int64)
    kr = np.ascontiguousarray(krows, dtype=np.int64)
    dq = np.zeros((len(qr), H, dqk)); dk = np.zeros((len(kr), H, dqk)); dvo = np.zeros((len(kr), H, dv_))
    tsa = np.ascontiguousarray(ts, dtype=np.int64)
    ln = _i32(lengths); nc = _i32(num_candidates)
    _lib().hstu_oracle_attn_bwd_rows(
        ctypes.c_int32(B), ctypes.c_int32(H), ctypes.c_int32(dqk), ctypes.c_int32(dv_),
        _ptr(off, _i32p), _ptr(ln, _i32p), _ptr(nc, _i32p),
        _ptr(q, _f64p), _ptr(k, _f64p), _ptr(v, _f64p), ctypes.c_int64(H * dqk),
        ctypes.c_int64(H * dv_), _ptr(tsa, _i64p),
        _ptr(rp, _f64p), ctypes.c_int32(P), _ptr(rt, _f64p), ctypes.c_int32(NT),
        ctypes.c_int64(rps), ctypes.c_int64(rts), ctypes.c_double(alpha), ctypes.c_int32(act),
        _ptr(g, _f64p), ctypes.c_int64(len(qr)), _ptr(qr, _i64p), _ptr(dq, _f64p),
        ctypes.c_int64(len(kr)), _ptr(kr, _i64p), _ptr(dk, _f64p), _ptr(dvo, _f64p),
        ctypes.c_int32(num_threads))
    return dq, dk, dvo


def ln_gate_bwd(o, u, dy, eps=1e-5, num_threads=0):
    """Gradients (dO, dU) of Y = LayerNorm(o) * u for an upstream gradient dy
    (rows of any width; closed form of the LayerNorm derivative, pinned by
    finite differences of ``ln_gate``)."""
    o2 = _f64(o).reshape(o.shape[0], -1)
    u2 = _f64(u).reshape(u.shape[0], -1)
    g2 = _f64(dy).reshape(dy.shape[0], -1)
    rows, width = o2.shape
    do = np.empty_like(o2)
    du = np.empty_like(o2)
    _lib().hstu_oracle_ln_gate_bwd(
        ctypes.c_int64(rows), ctypes.c_int32(width), _ptr(o2, _f64p), ctypes.c_int64(width),
        _ptr(u2, _f64p), ctypes.c_int64(width), _ptr(g2, _f64p), ctypes.c_int64(width),
        ctypes.c_double(eps), _ptr(do, _f64p), ctypes.c_int64(width), _ptr(du, _f64p),
        ctypes.c_int64(width), ctypes.c_int32(num_threads))
    return do, du


def layer(x, w1, w2, offsets, ts, rab_pos, rab_time, alpha, H, d, *, b1=None, b2=None,
          eps=1e-5, num_candidates=None, num_threads=0) -> np.ndarray:
    """One HSTU layer: X + (LN(attn(split(SiLU(X W1^T + b1)))) * U) W2^T + b2."""
    x = _f64(x)
    T, D = x.shape
    off = _i32(offsets)
    B = len(off) - 1
    w1 = _f64(w1); w2 = _f64(w2)
    assert w1.shape == (4 * H * d, D) and w2.shape == (D, H * d)
    b1a = None if b1 is None else _f64(b1)
    b2a = None if b2 is None else _f64(b2)
    rp = _f64(rab_pos); rt = _f64(rab_time)
    out = np.zeros_like(x)
    tsa = np.ascontiguousarray(ts, dtype=np.int64)
    nc = _i32(num_candidates)
    _lib().hstu_oracle_layer(
        ctypes.c_int32(B), ctypes.c_int32(H), ctypes.c_int32(d), ctypes.c_int32(D),
        _ptr(off, _i32p), _ptr(nc, _i32p), _ptr(x, _f64p), _ptr(w1, _f64p), _ptr(b1a, _f64p),
        _ptr(w2, _f64p), _ptr(b2a, _f64p), _ptr(tsa, _i64p),
        _ptr(rp, _f64p), ctypes.c_int32(rp.shape[-1]), _ptr(rt, _f64p), ctypes.c_int32(rt.shape[-1]),
        ctypes.c_double(alpha), ctypes.c_double(eps), _ptr(out, _f64p), ctypes.c_int32(num_threads))
    return out


def layer_bwd(x, w1, w2, offsets, ts, rab_pos, rab_time, alpha, H, d, dx_out, *, b1=None,
              b2=None, eps=1e-5, num_candidates=None, num_threads=0) -> dict:
    """Gradients of one HSTU layer (``layer``) for an upstream gradient dx_out.

    Returns a dict with dx [T, D], dw1 [4Hd, D], db1 [4Hd], dw2 [D, Hd],
    db2 [D], drab_pos [P], drab_time [NT] (shared tables).  Chain rule through
    f2, the gate, the attention and f1 + SiLU (pinned by central finite
    differences of ``layer``).
    """
    x = _f64(x)
    T, D = x.shape
    off = _i32(offsets)
    B = len(off) - 1
    w1 = _f64(w1); w2 = _f64(w2)
    zw, hd = 4 * H * d, H * d
    assert w1.shape == (zw, D) and w2.shape == (D, hd)
    b1a = None if b1 is None else _f64(b1)
    b2a = None if b2 is None else _f64(b2)
    rp = _f64(rab_pos); rt = _f64(rab_time)
    g = _f64(dx_out)
    out = {"dx": np.zeros_like(x), "dw1": np.zeros((zw, D)), "db1": np.zeros(zw),
           "dw2": np.zeros((D, hd)), "db2": np.zeros(D), "drab_pos": np.zeros_like(rp),
           "drab_time": np.zeros_like(rt)}
    tsa = np.ascontiguousarray(ts, dtype=np.int64)
    nc = _i32(num_candidates)
    _lib().hstu_oracle_layer_bwd(
        ctypes.c_int32(B), ctypes.c_int32(H), ctypes.c_int32(d), ctypes.c_int32(D),
        _ptr(off, _i32p), _ptr(nc, _i32p), _ptr(x, _f64p), _ptr(w1, _f64p), _ptr(b1a, _f64p),
        _ptr(w2, _f64p), _ptr(b2a, _f64p), _ptr(tsa, _i64p),
        _ptr(rp, _f64p), ctypes.c_int32(rp.shape[-1]), _ptr(rt, _f64p), ctypes.c_int32(rt.shape[-1]),
        ctypes.c_double(alpha), ctypes.c_double(eps), _ptr(g, _f64p),
        _ptr(out["dx"], _f64p), _ptr(out["dw1"], _f64p), _ptr(out["db1"], _f64p),
        _ptr(out["dw2"], _f64p), _ptr(out["db2"], _f64p), _ptr(out["drab_pos"], _f64p),
        _ptr(out["drab_time"], _f64p), ctypes.c_int32(num_threads))
    return out


def mfalcon_score(q, k, v, u, offsets, num_candidates, ts, rab_pos, rab_time, alpha, w,
                  *, eps=1e-5, num_threads=0) -> np.ndarray:
    """scores[b, c] = < LN(O[n_b + c]) * U[n_b + c], w > for every candidate c."""
    q = _f64(q); k = _f64(k); v = _f64(v); u = _f64(u)
    T, H, d = q.shape
    off = _i32(offsets)
    nc = _i32(num_candidates)
    B = len(off) - 1
    cmax = int(nc.max()) if B else 0
    scores = np.zeros((B, max(cmax, 1)), dtype=np.float64)
    rp = _f64(rab_pos); rt = _f64(rab_time); wa = _f64(w)
    tsa = np.ascontiguousarray(ts, dtype=np.int64)
    _lib().hstu_oracle_mfalcon_score(
        ctypes.c_int32(B), ctypes.c_int32(H), ctypes.c_int32(d), _ptr(off, _i32p), _ptr(nc, _i32p),
        _ptr(q, _f64p), _ptr(k, _f64p), _ptr(v, _f64p), _ptr(u, _f64p), ctypes.c_int64(H * d),
        _ptr(tsa, _i64p), _ptr(rp, _f64p), ctypes.c_int32(rp.shape[-1]), _ptr(rt, _f64p),
        ctypes.c_int32(rt.shape[-1]), ctypes.c_double(alpha), ctypes.c_double(eps),
        _ptr(wa, _f64p), _ptr(scores, _f64p), ctypes.c_int32(scores.shape[1]),
        ctypes.c_int32(num_threads))
    return scores[:, :cmax]


def layer_scores(x, w1, offsets, num_candidates, ts, rab_pos, rab_time, alpha, w, H, d, *,
                 b1=None, eps=1e-5, num_threads=0) -> np.ndarray:
    """scores[b, c] after the last layer: Z = SiLU(X W1^T + b1) split into
    U | V | Q | K, then ``mfalcon_score`` of that attention."""
    x = _f64(x)
    T, D = x.shape
    off = _i32(offsets)
    nc = _i32(num_candidates)
    B = len(off) - 1
    w1 = _f64(w1)
    assert w1.shape == (4 * H * d, D)
    b1a = None if b1 is None else _f64(b1)
    cmax = int(nc.max()) if B else 0
    scores = np.zeros((B, max(cmax, 1)), dtype=np.float64)
    rp = _f64(rab_pos); rt = _f64(rab_time); wa = _f64(w)
    tsa = np.ascontiguousarray(ts, dtype=np.int64)
    _lib().hstu_oracle_layer_scores(
        ctypes.c_int32(B), ctypes.c_int32(H), ctypes.c_int32(d), ctypes.c_int32(D),
        _ptr(off, _i32p), _ptr(nc, _i32p), _ptr(x, _f64p), _ptr(w1, _f64p), _ptr(b1a, _f64p),
        _ptr(tsa, _i64p), _ptr(rp, _f64p), ctypes.c_int32(rp.shape[-1]), _ptr(rt, _f64p),
        ctypes.c_int32(rt.shape[-1]), ctypes.c_double(alpha), ctypes.c_double(eps), _ptr(wa, _f64p),
        _ptr(scores, _f64p), ctypes.c_int32(scores.shape[1]), ctypes.c_int32(num_threads))
    return scores[:, :cmax]


def tiles(offsets, tile_m, tile_n, *, lengths=None, num_candidates=None) -> np.ndarray:
    """Brute-force non-empty tiles as an int32 array of (b, qt, kt) rows, ascending."""
    off = _i32(offsets)
    B = len(off) - 1
    ln = _i32(lengths); nc = _i32(num_candidates)
    lib = _lib()
    args = (ctypes.c_int32(B), _ptr(off, _i32p), _ptr(ln, _i32p), _ptr(nc, _i32p),
            ctypes.c_int32(tile_m), ctypes.c_int32(tile_n))
    n = lib.hstu_oracle_tiles(*args, ctypes.cast(None, _i32p), ctypes.c_int64(0))
    out = np.zeros((max(n, 1), 3), dtype=np.int32)
    lib.hstu_oracle_tiles(*args, _ptr(out, _i32p), ctypes.c_int64(n))
    return out[:n]


def count_visible(offsets, *, lengths=None, num_candidates=None) -> int:
    off = _i32(offsets)
    return int(_lib().hstu_oracle_count_visible(
        ctypes.c_int32(len(off) - 1), _ptr(off, _i32p), _ptr(_i32(lengths), _i32p),
        _ptr(_i32(num_candidates), _i32p)))
