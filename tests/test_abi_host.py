"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/gdn.h declares, and rejects bad arguments with the
documented status before touching the HIP runtime. Pointers here are host
addresses that the library never dereferences, because validation fails (or,
for empty work, returns) before any launch."""
import ctypes
import os
import re

import pytest

from gated_deltanet_linear_step_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, NULL, SHAPE, UNSUPPORTED, OVERFLOW, ALIGN, WORKSPACE = 0, 1, 2, 3, 4, 5, 6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_exported_set():
    assert declared_functions() == sorted(ops.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ops.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = ops.load()
    for s in range(8):
        assert len(ops.status_string(s)) > 0
    assert ops.status_string(99) == "unknown status"
    assert lib.gdn_version() >= 100


# Host buffers standing in for device arrays (never dereferenced on these paths).
_BUF = (ctypes.c_float * 4096)()
P = ctypes.addressof(_BUF)
P16 = (P + 255) // 256 * 256  # 256-byte aligned address inside the buffer


def vp(x):
    return ctypes.c_void_p(x)


def dims(**kw):
    d = dict(Hk=2, Hv=4, dk=128, dv=128, head_map=ops.MAP_TILED, flags=0)
    d.update(kw)
    return ops.make_dims(d["Hk"], d["Hv"], d["dk"], d["dv"], d["head_map"], d["flags"],
                         d.get("decay", 0), d.get("scale", 0.0))


def inputs(**kw):
    inp = ops.Inputs(q=vp(P16), k=vp(P16), v=vp(P16), q_stride=1024, k_stride=1024,
                     v_stride=1024, qkv_dtype=ops.BF16, g=vp(P16), beta=vp(P16))
    for key, val in kw.items():
        setattr(inp, key, val)
    return inp


def decode(d=None, inp=None, batch=2, T=1, state=P16, slots=None, num_slots=2, out_dtype=0,
           out=P16):
    lib = ops.load()
    d = dims() if d is None else d
    inp = inputs() if inp is None else inp
    return lib.gdn_decode_step(ctypes.byref(d), batch, T, ctypes.byref(inp), vp(state),
                               vp(slots) if slots else None, num_slots, out_dtype, vp(out), None)


def test_decode_validation():
    lib = ops.load()
    assert lib.gdn_decode_step(None, 1, 1, None, None, None, 1, 0, None, None) == NULL
    assert decode(out=0) == NULL
    assert decode(state=0) == NULL
    assert decode(d=dims(Hk=3)) == SHAPE                    # Hv % Hk != 0
    assert decode(d=dims(Hk=0)) == SHAPE
    assert decode(d=dims(dk=96, dv=128)) == UNSUPPORTED     # not built
    assert decode(d=dims(dk=256, dv=64)) == UNSUPPORTED
    assert decode(d=dims(dk=128, dv=32)) == UNSUPPORTED
    assert decode(d=dims(flags=16)) == UNSUPPORTED          # unknown flag bit
    assert decode(d=dims(head_map=2)) == SHAPE
    assert decode(d=dims(scale=-1.0)) == SHAPE
    assert decode(out_dtype=7) == UNSUPPORTED
    assert decode(inp=inputs(qkv_dtype=5)) == UNSUPPORTED
    assert decode(inp=inputs(q=None)) == NULL
    assert decode(inp=inputs(g=None)) == NULL               # gates needed without RAW_GATES
    assert decode(d=dims(flags=ops.RAW_GATES)) == NULL      # a, b, decay, dt_bias missing
    assert decode(d=dims(flags=ops.GATED_NORM)) == NULL     # z, norm weight missing
    assert decode(d=dims(flags=ops.GATED_NORM),
                  inp=inputs(z=vp(P16 + 2), norm_weight=vp(P16))) == ALIGN  # z read as words
    assert decode(inp=inputs(q_stride=100)) == SHAPE        # narrower than Hk*dk
    assert decode(inp=inputs(q=vp(P16 + 2))) == ALIGN       # not 4-element aligned
    assert decode(inp=inputs(k_stride=1026)) == ALIGN
    assert decode(inp=inputs(v=vp(P16 + 2))) == ALIGN       # v is read in groups of 4 too
    assert decode(inp=inputs(v_stride=2050)) == ALIGN
    assert decode(state=P16 + 4) == ALIGN                   # state needs 16 bytes
    assert decode(T=0) == SHAPE
    assert decode(batch=-1) == SHAPE
    assert decode(batch=3, num_slots=2) == SHAPE            # identity slots need num_slots >= B
    assert decode(batch=2 ** 30, T=4, num_slots=2 ** 30) == OVERFLOW
    assert decode(batch=0) == OK                            # nothing to launch


def conv(C=64, K=4, N=2, cu=None, total=4, x_dtype=ops.BF16, x=P16, xs=64, w=P16, st=P16,
         y_dtype=ops.F32, y=P16, ys=64):
    return ops.load().gdn_conv_update(C, K, N, vp(cu) if cu else None, total, x_dtype, vp(x), xs,
                                      vp(w), vp(st), y_dtype, vp(y), ys, None)


def test_conv_validation():
    assert conv(K=1) == UNSUPPORTED and conv(K=9) == UNSUPPORTED
    assert conv(C=0) == SHAPE
    assert conv(x=0) == NULL and conv(y=0) == NULL and conv(st=0) == NULL
    assert conv(xs=10) == SHAPE
    assert conv(total=5) == SHAPE          # uniform lengths need N | total
    assert conv(N=0, total=3) == SHAPE
    assert conv(N=0, total=0) == OK
    assert conv(total=0) == OK
    assert conv(x_dtype=3) == UNSUPPORTED


def test_prefill_validation():
    lib = ops.load()
    cu_ok = (ctypes.c_int32 * 3)(0, 100, 230)
    cu_bad = (ctypes.c_int32 * 3)(0, 150, 100)
    cu_tot = (ctypes.c_int32 * 3)(0, 100, 200)
    d = dims(head_map=ops.MAP_GROUPED)
    need = lib.gdn_prefill_workspace_bytes(ctypes.byref(d), 2, 230)
    if need == 0:
        pytest.skip("this build has no prefill kernels yet")
    # upper bound over splits: more sequences or tokens never need less
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(d), 3, 230) >= need
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(d), 2, 300) >= need
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(dims(Hk=3)), 2, 230) == 0

    def call(cu=cu_ok, ws=P16, ws_bytes=None, d=d, total=230, N=2, inp=None):
        inp = inputs() if inp is None else inp
        wsb = need if ws_bytes is None else ws_bytes
        return lib.gdn_prefill_chunked(ctypes.byref(d), N, cu, vp(P16), total,
                                       ctypes.byref(inp), vp(P16), 0, vp(P16), vp(ws) if ws else None,
                                       wsb, None)

    assert call(cu=cu_bad) == SHAPE        # not monotone
    assert call(cu=cu_tot) == SHAPE        # cu[N] != total
    assert call(ws=0) == WORKSPACE
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert call(ws=P16 + 16) == ALIGN
    assert call(d=dims(Hk=3)) == SHAPE
    assert call(d=dims(dk=96, dv=96)) == UNSUPPORTED
    assert call(d=dims(flags=8)) == UNSUPPORTED            # GDN_STREAM_STATE: decode only
    assert lib.gdn_prefill_chunked(ctypes.byref(d), 2, None, vp(P16), 230,
                                   ctypes.byref(inputs()), vp(P16), 0, vp(P16), vp(P16), need,
                                   None) == NULL
    zero = (ctypes.c_int32 * 3)(0, 0, 0)
    assert call(cu=zero, total=0) == OK    # all sequences empty: nothing launched


def test_layer_validation():
    lib = ops.load()
    sbytes = 2 * (2 * 2 * 128 + 4 * 128) * 3 * 2  # num_slots=2, channels, K-1, bf16

    def layer(d=None, K=4, w=P16, cin=P16, cout=P16 + sbytes, batch=0, T=1, num_slots=2,
              inp=None, state=P16, out=P16):
        d = dims() if d is None else d
        inp = inputs() if inp is None else inp
        ca = ops.ConvArgs(K, vp(w) if w else None, vp(cin) if cin else None,
                          vp(cout) if cout else None)
        return lib.gdn_decode_layer(ctypes.byref(d), batch, T, ctypes.byref(ca), ctypes.byref(inp),
                                    vp(state), None, num_slots, 0, vp(out), None)

    assert layer() == OK                                    # batch 0: nothing launched
    assert layer(w=0) == NULL and layer(cin=0) == NULL and layer(cout=0) == NULL
    assert lib.gdn_decode_layer(ctypes.byref(dims()), 0, 1, None, ctypes.byref(inputs()),
                                vp(P16), None, 2, 0, vp(P16), None) == NULL
    assert layer(K=3) == UNSUPPORTED and layer(K=5) == UNSUPPORTED  # built for K = 4
    assert layer(cin=P16 + 2) == ALIGN and layer(w=P16 + 6) == ALIGN
    assert layer(cout=P16 + 256) == SHAPE                   # overlaps the input window
    assert layer(cout=P16 - sbytes + 8) == SHAPE
    assert layer(d=dims(Hk=3)) == SHAPE                     # the decode step's own checks
    assert layer(T=0) == SHAPE
    assert layer(inp=inputs(v_stride=2050)) == ALIGN
