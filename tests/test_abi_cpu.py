"""CPU-only checks of the C ABI boundary: the library loads, exports every
symbol include/hstu.h declares, the ctypes structs match the C layout, and
every host-side validation error is returned before any launch (no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from hstu_sequential_transducer_causal_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hstu.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from hstu_sequential_transducer_causal_amd import build
        build.build()
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\([^;{]*\)\s*;", text)
    return sorted(set(n for n in names if n not in ("sizeof",)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    for name in declared:
        assert name in exported, name
    # no other C-linkage symbol leaks out (internal C++ names are mangled)
    plain = set(n for n in exported if not n.startswith("_Z"))
    assert plain == set(declared), sorted(plain - set(declared))


def test_abi_version_and_status_strings(lib):
    assert lib.hstu_abi_version() == 11
    for s in [0, -1, -2, -3, -4, 99]:
        assert lib.hstu_status_string(s)


_STRUCTS = {
    "hstu_attn_args": _lib.AttnArgs,
    "hstu_mfalcon_args": _lib.MfalconArgs,
    "hstu_mfalcon_cached_args": _lib.MfalconCachedArgs,
    "hstu_mfalcon_layer_args": _lib.MfalconLayerArgs,
    "hstu_layer_args": _lib.LayerArgs,
    "hstu_attn_bwd_args": _lib.AttnBwdArgs,
    "hstu_layer_bwd_args": _lib.LayerBwdArgs,
    "hstu_sl_args": _lib.SlArgs,
}


def test_ctypes_layout_matches_c(tmp_path):
    src = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for cname, cls in _STRUCTS.items():
        src.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            src.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    src.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-o", str(exe), str(c)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    for line in out.splitlines():
        cname, fname, val = line.split()
        cls = _STRUCTS[cname]
        want = ctypes.sizeof(cls) if fname == "size" else getattr(cls, fname).offset
        assert int(val) == want, line


def _valid_args():
    """A fully valid bf16 argument set with fake (never dereferenced) device pointers."""
    a = _lib.AttnArgs()
    a.struct_size = ctypes.sizeof(_lib.AttnArgs)
    a.B, a.H, a.d_qk, a.d_v, a.max_seq_len, a.num_rows = 2, 4, 128, 128, 100, 200
    fake = 0x10000
    a.seq_offsets = fake
    a.dtype, a.act = _lib.HSTU_BF16, _lib.HSTU_ACT_SILU
    a.q = a.k = a.v = a.o = fake
    a.q_stride = a.k_stride = a.v_stride = a.o_stride = 512
    a.timestamps = a.rab_pos = a.rab_time = fake
    a.num_pos_buckets, a.num_time_buckets = 1024, 32
    a.alpha = 1.0 / 1024
    a.ln_eps = 1e-5
    return a


def _call(lib, a, ws=None, nbytes=0):
    return lib.hstu_attn_fwd(ctypes.byref(a), ws, nbytes, None)


MUTATIONS = [
    ("struct_size", lambda a: setattr(a, "struct_size", 8), _lib.HSTU_ERR_ARG),
    ("B<0", lambda a: setattr(a, "B", -1), _lib.HSTU_ERR_ARG),
    ("H<1", lambda a: setattr(a, "H", 0), _lib.HSTU_ERR_ARG),
    ("dtype", lambda a: setattr(a, "dtype", 7), _lib.HSTU_ERR_ARG),
    ("act", lambda a: setattr(a, "act", 5), _lib.HSTU_ERR_ARG),
    ("bf16 d=64", lambda a: (setattr(a, "d_qk", 64), setattr(a, "d_v", 64)), _lib.HSTU_ERR_UNSUPPORTED),
    ("f32 d=128", lambda a: setattr(a, "dtype", _lib.HSTU_F32), _lib.HSTU_ERR_UNSUPPORTED),
    ("P=0", lambda a: setattr(a, "num_pos_buckets", 0), _lib.HSTU_ERR_ARG),
    ("P too big", lambda a: setattr(a, "num_pos_buckets", 100000), _lib.HSTU_ERR_ARG),
    ("NT=0", lambda a: setattr(a, "num_time_buckets", 0), _lib.HSTU_ERR_ARG),
    ("alpha nan", lambda a: setattr(a, "alpha", float("nan")), _lib.HSTU_ERR_ARG),
    ("alpha inf", lambda a: setattr(a, "alpha", float("inf")), _lib.HSTU_ERR_ARG),
    ("max_seq_len", lambda a: setattr(a, "max_seq_len", 1 << 20), _lib.HSTU_ERR_ARG),
    ("offsets NULL", lambda a: setattr(a, "seq_offsets", None), _lib.HSTU_ERR_ARG),
    ("q NULL", lambda a: setattr(a, "q", None), _lib.HSTU_ERR_ARG),
    ("ts NULL", lambda a: setattr(a, "timestamps", None), _lib.HSTU_ERR_ARG),
    ("tables NULL", lambda a: setattr(a, "rab_time", None), _lib.HSTU_ERR_ARG),
    ("q stride small", lambda a: setattr(a, "q_stride", 100), _lib.HSTU_ERR_ARG),
    ("misaligned q", lambda a: setattr(a, "q", 0x10002), _lib.HSTU_ERR_UNSUPPORTED),
    ("y without u", lambda a: setattr(a, "y", 0x10000), _lib.HSTU_ERR_ARG),
    ("eps<=0", lambda a: (setattr(a, "y", 0x10000), setattr(a, "u", 0x10000),
                          setattr(a, "u_stride", 512), setattr(a, "y_stride", 512),
                          setattr(a, "ln_eps", 0.0)), _lib.HSTU_ERR_ARG),
]


@pytest.mark.parametrize("name,mut,status", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_validation_errors_before_any_launch(lib, name, mut, status):
    a = _valid_args()
    mut(a)
    assert _call(lib, a) == status
    assert lib.hstu_last_error()
    assert lib.hstu_attn_workspace_bytes(ctypes.byref(a)) == 0


def test_null_args_and_workspace_errors(lib):
    assert lib.hstu_attn_fwd(None, None, 0, None) == _lib.HSTU_ERR_ARG
    a = _valid_args()
    need = lib.hstu_attn_workspace_bytes(ctypes.byref(a))
    assert need > 0
    assert _call(lib, a, None, 0) == _lib.HSTU_ERR_WORKSPACE
    assert _call(lib, a, 0x20000, need - 1) == _lib.HSTU_ERR_WORKSPACE
    assert _call(lib, a, 0x20001, need) == _lib.HSTU_ERR_WORKSPACE   # misaligned
    assert b"workspace" in lib.hstu_last_error()


def test_empty_batch_is_a_no_op(lib):
    a = _valid_args()
    a.B = 0
    assert _call(lib, a) == _lib.HSTU_OK


def test_mfalcon_and_layer_validation(lib):
    m = _lib.MfalconArgs()
    m.struct_size = ctypes.sizeof(_lib.MfalconArgs)
    m.attn = _valid_args()
    m.score_stride = 4
    # u required for the scores' LayerNorm
    assert lib.mfalcon_score(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_ARG
    m.attn.u, m.attn.u_stride = 0x10000, 512
    assert lib.mfalcon_score(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_ARG  # no candidates
    m.attn.num_candidates = 0x10000
    m.w = m.scores = 0x10000
    need = lib.hstu_mfalcon_workspace_bytes(ctypes.byref(m))
    assert need > 0
    assert lib.mfalcon_score(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_WORKSPACE
    # candidates only: Y would be incomplete, so it must not be requested
    m.candidates_only = 1
    m.attn.y, m.attn.y_stride = 0x10000, 512
    assert lib.mfalcon_score(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_ARG
    assert b"candidates_only" in lib.hstu_last_error()
    m.struct_size = 4
    assert lib.mfalcon_score(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_ARG

    l = _lib.LayerArgs()
    l.struct_size = ctypes.sizeof(_lib.LayerArgs)
    l.B, l.H, l.d, l.D, l.max_seq_len, l.num_rows = 2, 4, 128, 512, 100, 200
    fake = 0x10000
    l.seq_offsets = l.x = l.w1 = l.w2 = l.x_out = l.timestamps = l.rab_pos = l.rab_time = fake
    l.num_pos_buckets, l.num_time_buckets = 1024, 32
    l.alpha, l.ln_eps = 1.0 / 4096, 1e-5
    need = lib.hstu_layer_workspace_bytes(ctypes.byref(l))
    assert need >= 200 * (4 * 512 + 2 * 512) * 2
    assert lib.hstu_layer_fwd(ctypes.byref(l), None, 0, None) == _lib.HSTU_ERR_WORKSPACE
    l.d = 64
    assert lib.hstu_layer_fwd(ctypes.byref(l), None, 0, None) == _lib.HSTU_ERR_UNSUPPORTED
    l.d, l.D = 128, 100
    assert lib.hstu_layer_fwd(ctypes.byref(l), None, 0, None) == _lib.HSTU_ERR_UNSUPPORTED


def _valid_bwd():
    g = _lib.AttnBwdArgs()
    g.struct_size = ctypes.sizeof(_lib.AttnBwdArgs)
    g.attn = _valid_args()
    fake = 0x10000
    g.dout, g.dout_stride = fake, 512
    g.dq = g.dk = g.dv = fake
    g.dq_stride = g.dk_stride = g.dv_stride = 512
    return g


BWD_MUTATIONS = [
    ("struct_size", lambda g: setattr(g, "struct_size", 8), _lib.HSTU_ERR_ARG),
    ("fp32", lambda g: (setattr(g.attn, "dtype", _lib.HSTU_F32), setattr(g.attn, "d_qk", 64),
                        setattr(g.attn, "d_v", 64)), _lib.HSTU_ERR_UNSUPPORTED),
    ("no upstream gradient", lambda g: setattr(g, "dout", None), _lib.HSTU_ERR_ARG),
    ("dq NULL", lambda g: setattr(g, "dq", None), _lib.HSTU_ERR_ARG),
    ("dk stride small", lambda g: setattr(g, "dk_stride", 100), _lib.HSTU_ERR_ARG),
    ("misaligned dv", lambda g: setattr(g, "dv", 0x10004), _lib.HSTU_ERR_UNSUPPORTED),
    ("dy without u", lambda g: (setattr(g, "dy", 0x10000), setattr(g, "dy_stride", 512)),
     _lib.HSTU_ERR_ARG),
    ("dy without o", lambda g: (setattr(g, "dy", 0x10000), setattr(g, "dy_stride", 512),
                                setattr(g.attn, "u", 0x10000), setattr(g.attn, "u_stride", 512),
                                setattr(g.attn, "o", None)), _lib.HSTU_ERR_ARG),
    ("forward args", lambda g: setattr(g.attn, "H", 0), _lib.HSTU_ERR_ARG),
    ("tables too long", lambda g: setattr(g.attn, "num_pos_buckets", 8192), _lib.HSTU_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,mut,status", BWD_MUTATIONS, ids=[m[0] for m in BWD_MUTATIONS])
def test_bwd_validation_errors_before_any_launch(lib, name, mut, status):
    g = _valid_bwd()
    mut(g)
    assert lib.hstu_attn_bwd(ctypes.byref(g), None, 0, None) == status
    assert lib.hstu_last_error()
    assert lib.hstu_attn_bwd_workspace_bytes(ctypes.byref(g)) == 0


def test_bwd_workspace_errors_and_size(lib):
    assert lib.hstu_attn_bwd(None, None, 0, None) == _lib.HSTU_ERR_ARG
    g = _valid_bwd()
    g.attn.o = None      # not read without dy
    need = lib.hstu_attn_bwd_workspace_bytes(ctypes.byref(g))
    assert need > 0
    assert lib.hstu_attn_bwd(ctypes.byref(g), None, 0, None) == _lib.HSTU_ERR_WORKSPACE
    assert lib.hstu_attn_bwd(ctypes.byref(g), 0x20000, need - 1, None) == _lib.HSTU_ERR_WORKSPACE
    # with dy the workspace also holds dO: rows x H x 128 bf16
    g.dy, g.dy_stride = 0x10000, 512
    g.attn.o = g.attn.u = 0x10000
    g.attn.u_stride = 512
    need_dy = lib.hstu_attn_bwd_workspace_bytes(ctypes.byref(g))
    assert need_dy >= need + g.attn.num_rows * 512 * 2


def _valid_layer_bwd():
    g = _lib.LayerBwdArgs()
    g.struct_size = ctypes.sizeof(_lib.LayerBwdArgs)
    l = g.layer
    l.struct_size = ctypes.sizeof(_lib.LayerArgs)
    l.B, l.H, l.d, l.D, l.max_seq_len, l.num_rows = 2, 4, 128, 512, 100, 200
    fake = 0x10000
    l.seq_offsets = l.x = l.w1 = l.w2 = l.timestamps = l.rab_pos = l.rab_time = fake
    l.num_pos_buckets, l.num_time_buckets = 1024, 32
    l.alpha, l.ln_eps = 1.0 / 4096, 1e-5
    g.dx_out = g.dx = g.dw1 = g.dw2 = fake
    return g


LAYER_BWD_MUTATIONS = [
    ("struct_size", lambda g: setattr(g, "struct_size", 4), _lib.HSTU_ERR_ARG),
    ("dw1 NULL", lambda g: setattr(g, "dw1", None), _lib.HSTU_ERR_ARG),
    ("dx_out NULL", lambda g: setattr(g, "dx_out", None), _lib.HSTU_ERR_ARG),
    ("misaligned dx", lambda g: setattr(g, "dx", 0x10002), _lib.HSTU_ERR_UNSUPPORTED),
    ("D % 128", lambda g: setattr(g.layer, "D", 448), _lib.HSTU_ERR_UNSUPPORTED),
    ("d != 128", lambda g: setattr(g.layer, "d", 64), _lib.HSTU_ERR_UNSUPPORTED),
    ("tables too long", lambda g: setattr(g.layer, "num_pos_buckets", 8000), _lib.HSTU_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,mut,status", LAYER_BWD_MUTATIONS, ids=[m[0] for m in LAYER_BWD_MUTATIONS])
def test_layer_bwd_validation_errors_before_any_launch(lib, name, mut, status):
    g = _valid_layer_bwd()
    mut(g)
    assert lib.hstu_layer_bwd(ctypes.byref(g), None, 0, None) == status
    assert lib.hstu_last_error()
    assert lib.hstu_layer_bwd_workspace_bytes(ctypes.byref(g)) == 0


def test_layer_bwd_workspace_errors(lib):
    g = _valid_layer_bwd()
    need = lib.hstu_layer_bwd_workspace_bytes(ctypes.byref(g))
    # at least Z, its pre-activation and dZ (rows x 4Hd bf16 each)
    assert need >= 3 * 200 * 2048 * 2
    assert lib.hstu_layer_bwd(ctypes.byref(g), None, 0, None) == _lib.HSTU_ERR_WORKSPACE
    assert lib.hstu_layer_bwd(ctypes.byref(g), 0x20000, need - 1, None) == _lib.HSTU_ERR_WORKSPACE


def test_layer_saved_pair_errors(lib):
    """The training pair checks its saved-activation buffer before any launch:
    Z and the pre-activation (rows x 4Hd bf16), O and Y (rows x Hd bf16)."""
    g = _valid_layer_bwd()
    l = g.layer
    l.x_out = 0x100000          # past x's 200 x 512 bf16 rows at 0x10000
    need_saved = lib.hstu_layer_saved_bytes(ctypes.byref(l))
    assert need_saved == 2 * 200 * 2048 * 2 + 2 * 200 * 512 * 2
    ws_f = lib.hstu_layer_workspace_bytes(ctypes.byref(l))
    ws_b = lib.hstu_layer_bwd_saved_workspace_bytes(ctypes.byref(g))
    # the saved gradients need no room for a recomputed forward
    assert ws_b == lib.hstu_layer_bwd_workspace_bytes(ctypes.byref(g)) - need_saved
    # X_out over X would leave the gradients a wrong X: rejected (whole or partial overlap)
    for xo in (0x10000, 0x10000 + 200 * 512 * 2 - 16, 0x10000 - 16):
        l.x_out = xo
        assert lib.hstu_layer_fwd_saved(ctypes.byref(l), 0x30000, need_saved, 0x20000, ws_f,
                                        None) == _lib.HSTU_ERR_ARG
        assert b"overlap" in lib.hstu_last_error()
    l.x_out = 0x10000 + 200 * 512 * 2          # adjacent, not overlapping
    assert lib.hstu_layer_fwd_saved(ctypes.byref(l), 0x30000, need_saved - 1, 0x20000, ws_f,
                                    None) == _lib.HSTU_ERR_WORKSPACE
    l.x_out = 0x100000
    assert lib.hstu_layer_fwd_saved(ctypes.byref(l), None, 0, 0x20000, ws_f, None) == _lib.HSTU_ERR_ARG
    assert lib.hstu_layer_fwd_saved(ctypes.byref(l), 0x30000, need_saved - 1, 0x20000, ws_f,
                                    None) == _lib.HSTU_ERR_WORKSPACE
    assert lib.hstu_layer_fwd_saved(ctypes.byref(l), 0x30008, need_saved, 0x20000, ws_f,
                                    None) == _lib.HSTU_ERR_WORKSPACE   # misaligned
    assert lib.hstu_layer_bwd_saved(ctypes.byref(g), None, 0, 0x20000, ws_b, None) == _lib.HSTU_ERR_ARG
    assert lib.hstu_layer_bwd_saved(ctypes.byref(g), 0x30000, need_saved - 1, 0x20000, ws_b,
                                    None) == _lib.HSTU_ERR_WORKSPACE
    assert lib.hstu_layer_bwd_saved(ctypes.byref(g), 0x30000, need_saved, 0x20000, ws_b - 1,
                                    None) == _lib.HSTU_ERR_WORKSPACE
    # invalid layer arguments: no size, and the plain calls' errors
    l.struct_size = 4
    assert lib.hstu_layer_saved_bytes(ctypes.byref(l)) == 0
    assert lib.hstu_layer_fwd_saved(ctypes.byref(l), 0x30000, need_saved, 0x20000, ws_f,
                                    None) == _lib.HSTU_ERR_ARG


def _valid_sl():
    a = _lib.SlArgs()
    a.struct_size = ctypes.sizeof(_lib.SlArgs)
    a.B, a.num_rows, a.cap = 3, 100, 10
    a.seq_offsets = a.out_offsets = a.out_index = 0x10000
    a.num_tensors = 1
    a.src[0] = a.dst[0] = 0x10000
    a.src_stride[0] = a.dst_stride[0] = 1024
    a.row_bytes[0] = 1024
    return a


SL_MUTATIONS = [
    ("struct_size", lambda a: setattr(a, "struct_size", 4)),
    ("B<0", lambda a: setattr(a, "B", -1)),
    ("cap<0", lambda a: setattr(a, "cap", -1)),
    ("too many tensors", lambda a: setattr(a, "num_tensors", 9)),
    ("offsets NULL", lambda a: setattr(a, "seq_offsets", None)),
    ("row_bytes % 4", lambda a: a.row_bytes.__setitem__(0, 6)),
    ("stride < row", lambda a: a.src_stride.__setitem__(0, 512)),
    ("misaligned dst", lambda a: a.dst.__setitem__(0, 0x10002)),
    ("NULL src", lambda a: a.src.__setitem__(0, None)),
]


@pytest.mark.parametrize("name,mut", SL_MUTATIONS, ids=[m[0] for m in SL_MUTATIONS])
def test_sl_validation_errors_before_any_launch(lib, name, mut):
    a = _valid_sl()
    mut(a)
    assert lib.hstu_stochastic_length(ctypes.byref(a), None) == _lib.HSTU_ERR_ARG
    assert lib.hstu_last_error()


def _valid_cached():
    m = _lib.MfalconCachedArgs()
    m.struct_size = ctypes.sizeof(_lib.MfalconCachedArgs)
    m.B, m.H, m.d, m.max_hist_len, m.max_cands = 2, 4, 128, 1000, 300
    fake = 0x10000
    m.hist_offsets = m.cand_offsets = m.ts_hist = m.ts_cand = fake
    m.num_hist_rows, m.num_cand_rows = 2000, 600
    m.k_hist = m.v_hist = m.q = m.k = m.v = m.u = fake
    m.k_hist_stride = m.v_hist_stride = m.q_stride = m.k_stride = m.v_stride = m.u_stride = 512
    m.rab_pos, m.num_pos_buckets = fake, 1024
    m.rab_time, m.num_time_buckets = fake, 32
    m.alpha, m.ln_eps = 1.0 / 1000, 1e-5
    m.w = m.scores = fake
    m.score_stride = 300
    return m


CACHED_MUTATIONS = [
    ("struct_size", lambda m: setattr(m, "struct_size", 4), _lib.HSTU_ERR_ARG),
    ("H<1", lambda m: setattr(m, "H", 0), _lib.HSTU_ERR_ARG),
    ("d=64", lambda m: setattr(m, "d", 64), _lib.HSTU_ERR_UNSUPPORTED),
    ("max_hist_len<0", lambda m: setattr(m, "max_hist_len", -1), _lib.HSTU_ERR_ARG),
    ("max_cands too big", lambda m: setattr(m, "max_cands", 1 << 30), _lib.HSTU_ERR_ARG),
    ("score_stride<max_cands", lambda m: setattr(m, "score_stride", 299), _lib.HSTU_ERR_ARG),
    ("P=0", lambda m: setattr(m, "num_pos_buckets", 0), _lib.HSTU_ERR_ARG),
    ("NT=0", lambda m: setattr(m, "num_time_buckets", 0), _lib.HSTU_ERR_ARG),
    ("alpha inf", lambda m: setattr(m, "alpha", float("inf")), _lib.HSTU_ERR_ARG),
    ("eps 0", lambda m: setattr(m, "ln_eps", 0.0), _lib.HSTU_ERR_ARG),
    ("k_hist stride", lambda m: setattr(m, "k_hist_stride", 500), _lib.HSTU_ERR_ARG),
    ("u stride % 8", lambda m: setattr(m, "u_stride", 516), _lib.HSTU_ERR_ARG),
    ("H*d > 4096", lambda m: setattr(m, "H", 64), _lib.HSTU_ERR_UNSUPPORTED),
    ("v_hist NULL", lambda m: setattr(m, "v_hist", None), _lib.HSTU_ERR_ARG),
    ("ts_cand NULL", lambda m: setattr(m, "ts_cand", None), _lib.HSTU_ERR_ARG),
    ("w NULL", lambda m: setattr(m, "w", None), _lib.HSTU_ERR_ARG),
    ("misaligned q", lambda m: setattr(m, "q", 0x10008), _lib.HSTU_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,mut,status", CACHED_MUTATIONS, ids=[m[0] for m in CACHED_MUTATIONS])
def test_cached_validation_errors_before_any_launch(lib, name, mut, status):
    m = _valid_cached()
    mut(m)
    assert lib.mfalcon_score_cached(ctypes.byref(m), None, 0, None) == status
    assert lib.hstu_last_error()
    assert lib.hstu_mfalcon_cached_workspace_bytes(ctypes.byref(m)) == 0


def test_cached_workspace_errors_and_size(lib):
    m = _valid_cached()
    need = lib.hstu_mfalcon_cached_workspace_bytes(ctypes.byref(m))
    # at least the candidates' O (no o given) and the history's row codes
    assert need >= 600 * 512 * 2 + 2000 * 4
    assert lib.mfalcon_score_cached(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_WORKSPACE
    assert lib.mfalcon_score_cached(ctypes.byref(m), 0x20000, need - 1, None) == _lib.HSTU_ERR_WORKSPACE
    m.o, m.o_stride = 0x10000, 512
    assert lib.hstu_mfalcon_cached_workspace_bytes(ctypes.byref(m)) == need - 600 * 512 * 2
    # nothing to score: no launch, no workspace needed
    m.num_cand_rows = 0
    assert lib.mfalcon_score_cached(ctypes.byref(m), None, 0, None) == _lib.HSTU_OK
    m.num_cand_rows, m.B = 600, 0
    assert lib.mfalcon_score_cached(ctypes.byref(m), None, 0, None) == _lib.HSTU_OK


def test_mfalcon_layer_validation(lib):
    m = _lib.MfalconLayerArgs()
    m.struct_size = ctypes.sizeof(_lib.MfalconLayerArgs)
    l = m.layer
    l.struct_size = ctypes.sizeof(_lib.LayerArgs)
    l.B, l.H, l.d, l.D, l.max_seq_len, l.num_rows = 2, 4, 128, 512, 100, 200
    fake = 0x10000
    l.seq_offsets = l.x = l.w1 = l.timestamps = l.rab_pos = l.rab_time = fake
    l.num_pos_buckets, l.num_time_buckets = 1024, 32
    l.alpha, l.ln_eps = 1.0 / 4096, 1e-5
    m.score_stride = 16
    # candidates, w and scores are required; w2 and x_out are not
    assert lib.mfalcon_layer_score(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_ARG
    assert b"num_candidates" in lib.hstu_last_error()
    l.num_candidates = fake
    assert lib.mfalcon_layer_score(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_ARG
    m.w = m.scores = fake
    need = lib.hstu_mfalcon_layer_workspace_bytes(ctypes.byref(m))
    assert need >= 200 * (4 * 512 + 512) * 2
    assert lib.mfalcon_layer_score(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_WORKSPACE
    m.score_stride = 0
    assert lib.mfalcon_layer_score(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_ARG
    m.score_stride = 16
    l.d = 64
    assert lib.mfalcon_layer_score(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_UNSUPPORTED
    l.d = 128
    m.struct_size = 4
    assert lib.mfalcon_layer_score(ctypes.byref(m), None, 0, None) == _lib.HSTU_ERR_ARG
    assert lib.hstu_mfalcon_layer_workspace_bytes(ctypes.byref(m)) == 0


def test_noalloc_entry_point_host_checks(lib):
    """hstu_attn_fwd_noalloc: the same argument checks as hstu_attn_fwd, and a
    call needing more scratch than the library's fixed buffer is refused
    before any launch (no GPU here: every case must fail on the host)."""
    assert lib.hstu_attn_noalloc_scratch_bytes() == 32 << 20
    for name, mut, status in MUTATIONS:
        a = _valid_args()
        mut(a)
        assert lib.hstu_attn_fwd_noalloc(ctypes.byref(a), None) == status, name
    a = _valid_args()
    a.num_rows = 5_000_000            # 8 bytes of codes and split map per row: 40 MB
    assert lib.hstu_attn_fwd_noalloc(ctypes.byref(a), None) == _lib.HSTU_ERR_WORKSPACE
    assert b"noalloc" in lib.hstu_last_error()


def test_validate_offsets_host_checks(lib):
    """hstu_validate_offsets: the host-side argument errors, returned before
    any device work (an empty batch is valid and touches nothing)."""
    assert lib.hstu_validate_offsets(None, None) == _lib.HSTU_ERR_ARG
    a = _lib.AttnArgs()
    a.struct_size = ctypes.sizeof(_lib.AttnArgs) + 8
    assert lib.hstu_validate_offsets(ctypes.byref(a), None) == _lib.HSTU_ERR_ARG
    a.struct_size = ctypes.sizeof(_lib.AttnArgs)
    a.B, a.num_rows, a.max_seq_len = 0, 0, 0
    assert lib.hstu_validate_offsets(ctypes.byref(a), None) == _lib.HSTU_OK
    a.B = -1
    assert lib.hstu_validate_offsets(ctypes.byref(a), None) == _lib.HSTU_ERR_ARG
    a.B, a.num_rows, a.max_seq_len = 3, 100, 64
    a.seq_offsets = None
    assert lib.hstu_validate_offsets(ctypes.byref(a), None) == _lib.HSTU_ERR_ARG
    assert b"seq_offsets" in lib.hstu_last_error()
