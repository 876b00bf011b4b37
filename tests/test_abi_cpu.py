"""The C-ABI library loads, exports what include/*.h declares, and refuses bad
arguments on the host before any launch (no GPU needed: every call here
returns during argument checking)."""

import ctypes
import glob
import os
import re

import pytest

from mxfp4_mixture_experts_router_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(moe_mxfp4_\w+)\s*\(", text))
    return names


def test_every_declared_symbol_is_exported():
    decl = _declared()
    assert decl == set(_lib.EXPORTED), decl ^ set(_lib.EXPORTED)
    handle = _lib.lib()
    for name in decl:
        assert getattr(handle, name) is not None


def test_version_and_status_strings():
    L = _lib.lib()
    assert b"gfx950" in L.moe_mxfp4_version()
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert L.moe_mxfp4_status_string(st).startswith(b"MOE_")
    assert L.moe_mxfp4_status_string(12345) == b"unknown status"


def _desc(**kw):
    d = dict(T=4, K=256, I=256, E_global=8, E_local=8, expert_offset=0, top_k=2, scoring=0,
             activation=0, swiglu_alpha=1.702, swiglu_limit=7.0, weight_layout=0, down_pairing=0, w13_order=0,
             mma=0)
    d.update(kw)
    return _lib.MoeDesc(**d)


def _ws_bytes(d):
    n = ctypes.c_size_t(0)
    st = _lib.lib().moe_mxfp4_workspace_bytes(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_workspace_query():
    st, n = _ws_bytes(_desc())
    assert st == 0 and n > 0 and n % 256 == 0
    st2, n2 = _ws_bytes(_desc(T=8))
    assert n2 > n
    assert _lib.lib().moe_mxfp4_workspace_bytes(None, ctypes.byref(ctypes.c_size_t())) == _lib.MOE_ERR_NULL
    assert _lib.lib().moe_mxfp4_workspace_bytes(ctypes.byref(_desc()), None) == _lib.MOE_ERR_NULL


@pytest.mark.parametrize("bad,code", [
    (dict(K=250), _lib.MOE_ERR_SHAPE),
    (dict(K=0), _lib.MOE_ERR_SHAPE),
    (dict(K=8192 + 32), _lib.MOE_ERR_SHAPE),
    (dict(I=48), _lib.MOE_ERR_SHAPE),
    (dict(T=-1), _lib.MOE_ERR_SHAPE),
    (dict(E_local=9), _lib.MOE_ERR_SHAPE),
    (dict(E_local=4, expert_offset=5), _lib.MOE_ERR_SHAPE),
    (dict(expert_offset=-1), _lib.MOE_ERR_SHAPE),
    (dict(top_k=0), _lib.MOE_ERR_SHAPE),
    (dict(top_k=9), _lib.MOE_ERR_SHAPE),
    (dict(E_global=600, E_local=513), _lib.MOE_ERR_SHAPE),
    (dict(T=131072, K=8192), _lib.MOE_ERR_SHAPE),           # x reaches 2 GiB
    (dict(T=32768, top_k=8, I=4096), _lib.MOE_ERR_SHAPE),   # the intermediate reaches 2 GiB
    (dict(scoring=2), _lib.MOE_ERR_MODE),
    (dict(activation=-1), _lib.MOE_ERR_MODE),
    (dict(w13_order=2), _lib.MOE_ERR_MODE),
    (dict(w13_order=-1), _lib.MOE_ERR_MODE),
    (dict(mma=2), _lib.MOE_ERR_MODE),
    (dict(mma=-1), _lib.MOE_ERR_MODE),
    # split rows of the scaled-FP4 path: whole 256-byte chunks per 128 values,
    # so I = 32 needs 8x the bf16 bytes (2^19 routes x 256 B = 128 MiB is fine,
    # T * top_k = 2^23 routes x 256 B = 2 GiB is not)
    (dict(mma=1, T=1 << 20, top_k=8, I=32, K=32), _lib.MOE_ERR_SHAPE),
])
def test_bad_descriptors_are_refused(bad, code):
    st, _ = _ws_bytes(_desc(**bad))
    assert st == code


def test_scaled_fp4_workspace_holds_the_split_rows():
    # the split activations (x by token, the intermediate by route) exist only
    # when the MFMA lists can run (T > 2): 256 bytes per 128 values, plus one
    # scale word per row, each region 256-byte aligned
    def split(T, K=256, I=256, top_k=2):
        def up(n):
            return (n + 255) // 256 * 256
        return (up(T * ((K + 127) // 128) * 256) + up(T * 4) +
                up(T * top_k * ((I + 127) // 128) * 256) + up(T * top_k * 4))
    for T in (1, 2):
        assert _ws_bytes(_desc(T=T, mma=1)) == _ws_bytes(_desc(T=T, mma=0))
    for T, K, I in ((3, 256, 256), (40, 96, 224), (100, 7168, 2048)):
        st0, n0 = _ws_bytes(_desc(T=T, K=K, I=I, mma=0))
        st1, n1 = _ws_bytes(_desc(T=T, K=K, I=I, mma=1))
        assert st0 == st1 == _lib.MOE_OK
        assert n1 - n0 == split(T, K, I), (T, K, I)
    assert _ws_bytes(_desc(mma=1, T=1 << 16, top_k=8, I=32, K=32))[0] == _lib.MOE_OK


def test_largest_activation_buffers_are_accepted():
    assert _ws_bytes(_desc(T=131071, K=8192))[0] == _lib.MOE_OK
    assert _ws_bytes(_desc(T=32767, top_k=8, I=4096))[0] == _lib.MOE_OK


# fake, never-dereferenced addresses: every call below must fail in the host checks
A = 0x10000
A_MIS = 0x10008


def _decode(d, **kw):
    args = dict(x=A, logits=A, ids=None, wts=None, w13p=A, w13s=A, b13=None, w2p=A, w2s=A, b2=None,
                out=A, ws=A, ws_bytes=1 << 40)
    args.update(kw)
    return _lib.lib().moe_mxfp4_decode(
        ctypes.byref(d), args["x"], args["logits"], args["ids"], args["wts"], args["w13p"], args["w13s"],
        args["b13"], args["w2p"], args["w2s"], args["b2"], args["out"], args["ws"], args["ws_bytes"], None)


def test_decode_error_paths():
    d = _desc()
    E = _lib
    assert _decode(d, logits=None) == E.MOE_ERR_MODE                      # neither routing input
    assert _decode(d, ids=A, wts=A) == E.MOE_ERR_MODE                     # both
    assert _decode(d, logits=None, ids=A) == E.MOE_ERR_MODE               # ids without weights
    assert _decode(d, x=None) == E.MOE_ERR_NULL
    assert _decode(d, w2s=None) == E.MOE_ERR_NULL
    assert _decode(d, out=None) == E.MOE_ERR_NULL
    assert _decode(d, x=A_MIS) == E.MOE_ERR_ALIGN
    assert _decode(d, w13p=A_MIS) == E.MOE_ERR_ALIGN
    assert _decode(d, w2s=A_MIS) == E.MOE_ERR_ALIGN
    assert _decode(d, out=A_MIS) == E.MOE_ERR_ALIGN
    assert _decode(d, b13=A_MIS) == E.MOE_ERR_ALIGN                      # biases are copied 16 B at a time
    assert _decode(d, b2=A_MIS) == E.MOE_ERR_ALIGN
    assert _decode(d, ws=None) == E.MOE_ERR_WORKSPACE
    assert _decode(d, ws=A_MIS) == E.MOE_ERR_ALIGN
    _, need = _ws_bytes(d)
    assert _decode(d, ws_bytes=need - 1) == E.MOE_ERR_WORKSPACE
    assert _decode(_desc(E_global=2048, E_local=8)) == E.MOE_ERR_SHAPE   # too many experts to route
    assert _decode(_desc(T=0)) == E.MOE_OK                               # T = 0: nothing to do
    assert _decode(_desc(T=0), x=None, out=None) == E.MOE_OK


def _decode_routes(d, **kw):
    args = dict(x=A, logits=A, ids=None, wts=None, w13p=A, w13s=A, b13=None, w2p=A, w2s=A, b2=None,
                out=A, ws=A, ws_bytes=1 << 40)
    args.update(kw)
    return _lib.lib().moe_mxfp4_decode_routes(
        ctypes.byref(d), args["x"], args["logits"], args["ids"], args["wts"], args["w13p"], args["w13s"],
        args["b13"], args["w2p"], args["w2s"], args["b2"], args["out"], args["ws"], args["ws_bytes"], None)


def test_route_output_error_paths():
    d = _desc()
    E, L = _lib, _lib.lib()
    assert _decode_routes(d, logits=None) == E.MOE_ERR_MODE
    assert _decode_routes(d, out=None) == E.MOE_ERR_NULL
    assert _decode_routes(d, w13p=None) == E.MOE_ERR_NULL
    assert _decode_routes(d, out=A_MIS) == E.MOE_ERR_ALIGN
    assert _decode_routes(d, b2=A_MIS) == E.MOE_ERR_ALIGN
    _, need = _ws_bytes(d)
    assert _decode_routes(d, ws_bytes=need - 1) == E.MOE_ERR_WORKSPACE
    assert _decode_routes(_desc(w13_order=5)) == E.MOE_ERR_MODE
    assert _decode_routes(_desc(T=0), x=None, out=None) == E.MOE_OK
    down = L.moe_mxfp4_down_routes
    assert down(ctypes.byref(d), None, A, A, None, None, A, 1 << 40, None) == E.MOE_ERR_NULL
    assert down(ctypes.byref(d), None, A, A, None, A_MIS, A, 1 << 40, None) == E.MOE_ERR_ALIGN
    assert down(ctypes.byref(d), A_MIS, A, A, None, A, A, 1 << 40, None) == E.MOE_ERR_ALIGN
    assert down(ctypes.byref(d), None, A, A, None, A, A, need - 1, None) == E.MOE_ERR_WORKSPACE
    assert down(ctypes.byref(_desc(T=0)), None, A, A, None, None, A, 1 << 40, None) == E.MOE_OK


def test_prefill_and_unpack_error_paths():
    d = _desc()
    E, L = _lib, _lib.lib()
    n = ctypes.c_size_t(0)
    assert L.moe_mxfp4_prefill_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == E.MOE_OK
    _, dec = _ws_bytes(d)
    assert n.value >= dec + d.E_local * 3 * d.I * d.K * 2
    pf = L.moe_mxfp4_prefill

    def call(**kw):
        a = dict(x=A, logits=A, ids=None, wts=None, w13p=A, w13s=A, b13=None, w2p=A, w2s=A, b2=None,
                 out=A, ws=A, ws_bytes=n.value)
        a.update(kw)
        return pf(ctypes.byref(kw.pop("desc", d)), a["x"], a["logits"], a["ids"], a["wts"], a["w13p"], a["w13s"],
                  a["b13"], a["w2p"], a["w2s"], a["b2"], a["out"], a["ws"], a["ws_bytes"], None)

    assert call(ws_bytes=dec) == E.MOE_ERR_WORKSPACE          # the decode workspace is too small here
    assert call(ws=None) == E.MOE_ERR_WORKSPACE
    assert call(ws=A_MIS) == E.MOE_ERR_ALIGN
    assert call(logits=None) == E.MOE_ERR_MODE
    assert call(out=None) == E.MOE_ERR_NULL
    assert call(w2p=A_MIS) == E.MOE_ERR_ALIGN
    un = L.moe_mxfp4_unpack
    assert un(ctypes.byref(d), A, A, A, A, None, A, A, 1 << 40, None) == E.MOE_ERR_NULL
    assert un(ctypes.byref(d), A, A, A, A, A_MIS, A, A, 1 << 40, None) == E.MOE_ERR_ALIGN
    assert un(ctypes.byref(d), A, A, A, A, A, A, A, dec - 1, None) == E.MOE_ERR_WORKSPACE
    assert un(ctypes.byref(_desc(T=0)), None, None, None, None, None, None, None, 0, None) == E.MOE_OK


def test_tile_weights_error_paths():
    L, E = _lib.lib(), _lib
    assert L.moe_mxfp4_tile_weights(A, 24, 64, 0, None) == E.MOE_ERR_SHAPE      # rows not a multiple of 16
    assert L.moe_mxfp4_tile_weights(A, 32, 48, 0, None) == E.MOE_ERR_SHAPE      # cols not a multiple of 32
    assert L.moe_mxfp4_tile_weights(A, 32, 16384, 0, None) == E.MOE_ERR_SHAPE   # cols above 8192
    assert L.moe_mxfp4_tile_weights(A, 32, 64, 2, None) == E.MOE_ERR_MODE
    assert L.moe_mxfp4_tile_weights(None, 32, 64, 0, None) == E.MOE_ERR_NULL
    assert L.moe_mxfp4_tile_weights(A_MIS, 32, 64, 0, None) == E.MOE_ERR_ALIGN
    assert L.moe_mxfp4_tile_weights(None, 0, 64, 0, None) == E.MOE_OK           # nothing to do
    assert _decode(_desc(weight_layout=2)) == E.MOE_ERR_MODE
    assert _decode(_desc(down_pairing=3)) == E.MOE_ERR_MODE
    assert _decode(_desc(down_pairing=-1)) == E.MOE_ERR_MODE


def test_encode_error_paths():
    L, E = _lib.lib(), _lib
    assert L.moe_mxfp4_encode(A, 0, 4, 48, 0, A, A, None) == E.MOE_ERR_SHAPE      # cols not a multiple of 32
    assert L.moe_mxfp4_encode(A, 2, 4, 64, 0, A, A, None) == E.MOE_ERR_MODE       # dtype
    assert L.moe_mxfp4_encode(A, 0, 4, 64, 2, A, A, None) == E.MOE_ERR_MODE       # rule
    assert L.moe_mxfp4_encode(None, 0, 4, 64, 0, A, A, None) == E.MOE_ERR_NULL
    assert L.moe_mxfp4_encode(A, 0, 4, 64, 0, A, None, None) == E.MOE_ERR_NULL
    assert L.moe_mxfp4_encode(A_MIS, 1, 4, 64, 1, A, A, None) == E.MOE_ERR_ALIGN
    assert L.moe_mxfp4_encode(A, 1, 4, 64, 1, A_MIS, A, None) == E.MOE_ERR_ALIGN
    assert L.moe_mxfp4_encode(None, 0, 0, 64, 0, None, None, None) == E.MOE_OK    # nothing to do


def test_hook_error_paths():
    L = _lib.lib()
    d = _desc()
    E = _lib
    assert L.moe_mxfp4_route(ctypes.byref(d), None, A, A, None) == E.MOE_ERR_NULL
    assert L.moe_mxfp4_route(ctypes.byref(_desc(E_global=1100, E_local=8)), A, A, A, None) == E.MOE_ERR_SHAPE
    assert L.moe_mxfp4_bucket(ctypes.byref(d), A, A, A, None, A, 1 << 40, None) == E.MOE_ERR_NULL
    assert L.moe_mxfp4_bucket(ctypes.byref(d), A, A, A, A, A, 16, None) == E.MOE_ERR_WORKSPACE
    assert L.moe_mxfp4_plan(ctypes.byref(d), None, None, None, A, 1 << 40, None) == E.MOE_ERR_MODE
    assert L.moe_mxfp4_plan(ctypes.byref(d), A, A, A, A, 1 << 40, None) == E.MOE_ERR_MODE
    assert L.moe_mxfp4_plan(ctypes.byref(d), None, A, None, A, 1 << 40, None) == E.MOE_ERR_MODE
    assert L.moe_mxfp4_plan(ctypes.byref(d), A, None, None, A, 16, None) == E.MOE_ERR_WORKSPACE
    assert L.moe_mxfp4_plan(ctypes.byref(_desc(T=0)), A, None, None, None, 0, None) == E.MOE_OK
    assert L.moe_mxfp4_gate_up(ctypes.byref(d), A, A, A, None, A_MIS, A, 1 << 40, None) == E.MOE_ERR_ALIGN
    assert L.moe_mxfp4_gate_up(ctypes.byref(d), None, A, A, None, None, A, 1 << 40, None) == E.MOE_ERR_NULL
    assert L.moe_mxfp4_gate_up(ctypes.byref(d), A, A, A, None, None, None, 1 << 40, None) == E.MOE_ERR_WORKSPACE
    assert L.moe_mxfp4_down(ctypes.byref(d), None, A, None, None, A, A, 1 << 40, None) == E.MOE_ERR_NULL
    assert L.moe_mxfp4_down(ctypes.byref(d), A_MIS, A, A, None, A, A, 1 << 40, None) == E.MOE_ERR_ALIGN
    assert L.moe_mxfp4_down(ctypes.byref(d), None, A, A, None, A, A, 8, None) == E.MOE_ERR_WORKSPACE
    assert L.moe_mxfp4_dequant(A, A, 4, 48, 0, A, None) == E.MOE_ERR_SHAPE
    assert L.moe_mxfp4_dequant(A, A, 4, 64, 7, A, None) == E.MOE_ERR_MODE
    assert L.moe_mxfp4_dequant(A_MIS, A, 4, 64, 0, A, None) == E.MOE_ERR_ALIGN
    assert L.moe_mxfp4_dequant(None, A, 4, 64, 0, A, None) == E.MOE_ERR_NULL
    assert L.moe_mxfp4_dequant(A, A, 0, 64, 0, A, None) == E.MOE_OK
    assert L.moe_mxfp4_plan_read(ctypes.byref(d), None, 1 << 40, A, A, A, A, A, None) == E.MOE_ERR_WORKSPACE
    assert L.moe_mxfp4_plan_read(ctypes.byref(d), A_MIS, 1 << 40, A, A, A, A, A, None) == E.MOE_ERR_ALIGN
    assert L.moe_mxfp4_plan_read(ctypes.byref(d), A, 16, A, A, A, A, A, None) == E.MOE_ERR_WORKSPACE
    assert L.moe_mxfp4_plan_read(ctypes.byref(_desc(top_k=0)), A, 1 << 40, A, A, A, A, A, None) == E.MOE_ERR_SHAPE
    assert L.moe_mxfp4_plan_read(ctypes.byref(_desc(T=0)), None, 0, None, None, None, None, None, None) == E.MOE_OK


def test_noalloc_refuses_calls_beyond_its_workspace_before_any_launch():
    L = _lib.lib()
    E = _lib
    d = _desc(T=4096, K=7168, I=2048, E_global=384, E_local=48, top_k=8)
    n = ctypes.c_size_t(0)
    assert L.moe_mxfp4_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == E.MOE_OK
    assert n.value > E.MOE_SCRATCH_BYTES
    assert L.moe_mxfp4_decode_noalloc(ctypes.byref(d), A, A, None, None, A, A, None, A, A, None, A, None) == \
        E.MOE_ERR_WORKSPACE
    assert L.moe_mxfp4_decode_noalloc(ctypes.byref(d), A, None, None, None, A, A, None, A, A, None, A, None) == \
        E.MOE_ERR_MODE
    assert L.moe_mxfp4_decode_noalloc(ctypes.byref(d), A_MIS, A, None, None, A, A, None, A, A, None, A, None) == \
        E.MOE_ERR_ALIGN
    assert L.moe_mxfp4_decode_noalloc(ctypes.byref(_desc(T=0)), None, A, None, None, None, None, None, None, None,
                                      None, None, None) == E.MOE_OK


def test_binding_steps_need_a_planned_workspace():
    # the steps that read a plan refuse to run on a workspace the binding would
    # have to allocate (it would hold no plan); checked before any device work
    torch = pytest.importorskip("torch")
    import mxfp4_mixture_experts_router_amd as m
    d = m.make_desc(T=4, K=256, I=256, E_global=8, E_local=8, top_k=2)
    fake = torch.zeros(4)
    for fn, args in ((m.moe_mxfp4_gate_up, (d, fake, fake, fake, None)),
                     (m.moe_mxfp4_down, (d, fake, fake, fake, None)),
                     (m.moe_mxfp4_down_routes, (d, fake, fake, fake, None)),
                     (m.moe_mxfp4_unpack, (d, fake, fake, fake, fake, fake, fake, None)),
                     (m.moe_mxfp4_plan_read, (d, None))):
        with pytest.raises(ValueError, match="reads the plan"):
            fn(*args)


def test_binding_rejects_unexpected_dtypes():
    torch = pytest.importorskip("torch")
    import mxfp4_mixture_experts_router_amd as m
    with pytest.raises(TypeError):
        m._ptr(torch.zeros(4, 256, dtype=torch.float16), torch.bfloat16, (4, 256), "x")
    with pytest.raises(ValueError):
        m._ptr(torch.zeros(4, 255, dtype=torch.bfloat16), torch.bfloat16, (4, 256), "x")
    with pytest.raises(ValueError):
        m._ptr(torch.zeros(4, 256, dtype=torch.bfloat16), torch.bfloat16, (4, 256), "x")  # host tensor
