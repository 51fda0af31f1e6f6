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
    for s in range(9):
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
    assert need > 0
    # the gated norm keeps an f32 core output in the workspace: the query must say so
    dn = dims(head_map=ops.MAP_GROUPED, flags=ops.GATED_NORM)
    need_norm = lib.gdn_prefill_workspace_bytes(ctypes.byref(dn), 2, 230)
    assert need_norm >= need + 230 * 4 * 128 * 4
    assert ops.prefill_workspace_bytes(Hk=2, Hv=4, dk=128, dv=128, num_seqs=2, total_tokens=230,
                                       gated_norm=True) == need_norm
    assert ops.prefill_workspace_bytes(Hk=2, Hv=4, dk=128, dv=128, num_seqs=2,
                                       total_tokens=230) == need
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
    assert call(d=dims(dk=96, dv=128)) == UNSUPPORTED       # not built
    assert call(d=dims(dk=32, dv=64)) == UNSUPPORTED
    assert call(d=dims(flags=8)) == UNSUPPORTED            # GDN_STREAM_STATE: decode only
    # a gated-norm call with the plain workspace size is refused, not overrun
    assert call(d=dn, inp=inputs(z=vp(P16), norm_weight=vp(P16))) == WORKSPACE
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


# ------------------------------------------------------------------ kernel selection
# Which kernel runs is a function of the shape, the flags and the device, checked
# here on the host the way the ferrum-kernels tests page checks its specialisation
# predicates (`simd_delta_specialization_is_shape_and_device_capability_driven`,
# `chunk_k_gram_specialization_requires_repeated_k128_heads`).

DECODE_SHAPES = {  # (dk, dv): (waves, lanes per row)
    (32, 32): (4, 8), (64, 64): (4, 16), (96, 96): (6, 8), (128, 128): (8, 16),
    (64, 128): (8, 16), (128, 64): (8, 16), (128, 256): (8, 16), (256, 128): (16, 32),
    (256, 256): (16, 32)}


@pytest.mark.parametrize("dk,dv", sorted(DECODE_SHAPES))
def test_decode_kernel_choice_per_head_shape(dk, dv):
    waves, lpr = DECODE_SHAPES[(dk, dv)]
    for fused in (False, True):
        for T, mode in ((1, 2), (4, 1 if fused else 0)):
            i = ops.decode_launch_info(Hk=4, Hv=8, dk=dk, dv=dv, batch=3, tokens_per_seq=T,
                                       fused_conv=fused)
            assert (i["waves"], i["lanes_per_row"], i["token_mode"]) == (waves, lpr, mode)
            assert i["workgroups"] == 3 * 8 and i["threads"] == 64 * waves
            assert i["nontemporal"] == 0
    # the geometry the kernel template asserts: a row's pieces tile dk, rows tile a wave
    rows_per_load = 64 // lpr
    assert 64 % lpr == 0 and dk % (4 * lpr) == 0
    assert (dv // waves) % rows_per_load == 0 and dv // waves <= 64
    assert 2 * dk + dv <= 64 * waves  # the fused layer gives every conv channel a thread


def test_decode_stream_hint_selects_the_nontemporal_kernel():
    f = ops.L2NORM_QK | ops.RAW_GATES | ops.GATED_NORM
    one = ops.decode_launch_info(Hk=16, Hv=32, dk=128, dv=128, batch=64, flags=f | ops.STREAM_STATE)
    assert (one["waves"], one["nontemporal"], one["token_mode"]) == (16, 1, 2)
    multi = ops.decode_launch_info(Hk=16, Hv=32, dk=128, dv=128, batch=64, tokens_per_seq=4,
                                   flags=f | ops.STREAM_STATE)
    assert (multi["waves"], multi["nontemporal"], multi["token_mode"]) == (8, 1, 1)
    other = ops.decode_launch_info(Hk=16, Hv=32, dk=64, dv=64, batch=64, flags=f | ops.STREAM_STATE)
    assert (other["waves"], other["nontemporal"]) == (4, 1)
    plain = ops.decode_launch_info(Hk=16, Hv=32, dk=128, dv=128, batch=64, flags=f)
    assert (plain["waves"], plain["nontemporal"]) == (8, 0)


def test_decode_launch_info_rejects_what_the_entry_points_reject():
    with pytest.raises(ops.GdnError) as e:
        ops.decode_launch_info(Hk=4, Hv=8, dk=128, dv=32, batch=1)
    assert e.value.status == UNSUPPORTED
    with pytest.raises(ops.GdnError) as e:
        ops.decode_launch_info(Hk=3, Hv=8, dk=128, dv=128, batch=1)
    assert e.value.status == SHAPE
    with pytest.raises(ops.GdnError) as e:
        ops.decode_launch_info(Hk=4, Hv=8, dk=128, dv=128, batch=1, tokens_per_seq=0)
    assert e.value.status == SHAPE


def test_prefill_carry_choice_follows_sequences_and_compute_units():
    kw = dict(Hk=16, Hv=32, dk=128, dv=128)
    # one 4096-token sequence: 32 heads x 8 one-slice workgroups fill 256 CUs once
    i = ops.prefill_launch_info([4096], compute_units=256, **kw)
    assert (i["carry_kind"], i["slices_per_workgroup"]) == (0, 1)
    assert i["workgroups"] == 256 and i["threads"] == 64 * 4 and i["prep_workgroups"] == 64 * 16
    # two sequences: one-slice workgroups would need two rounds, two-slice ones fit
    i = ops.prefill_launch_info([4096, 4096], compute_units=256, **kw)
    assert (i["carry_kind"], i["slices_per_workgroup"], i["workgroups"]) == (0, 2, 256)
    assert i["threads"] == 64 * 6
    # the eight varlen sequences: throughput bound, four slices per workgroup
    i = ops.prefill_launch_info([512, 1024, 2048, 3072, 4096, 5120, 6144, 8192],
                                compute_units=256, **kw)
    assert (i["carry_kind"], i["slices_per_workgroup"]) == (1, 4)
    assert i["workgroups"] == 256 * 2 and i["threads"] == 64 * 6
    assert i["prep_workgroups"] == sum((n + 63) // 64 for n in
                                       (512, 1024, 2048, 3072, 4096, 5120, 6144, 8192)) * 16
    # the same single sequence on a device with fewer CUs takes the two-slice split
    i = ops.prefill_launch_info([4096], compute_units=200, **kw)
    assert (i["carry_kind"], i["slices_per_workgroup"]) == (0, 2)
    # workgroups of one head share blockIdx % 8 (one XCD): groups padded to 8
    i = ops.prefill_launch_info([100] * 3, Hk=2, Hv=4, dk=128, dv=128, compute_units=256)
    assert i["workgroups"] == 16 * 8  # 12 groups -> 16, eight slices each


def test_prefill_launch_info_validates_like_the_entry_point():
    kw = dict(Hk=16, Hv=32, dk=128, dv=128, compute_units=256)
    with pytest.raises(ops.GdnError) as e:
        ops.prefill_launch_info([10, 20], **dict(kw, Hk=5))
    assert e.value.status == SHAPE
    with pytest.raises(ops.GdnError) as e:
        ops.prefill_launch_info([10, 20], **dict(kw, compute_units=0))
    assert e.value.status == SHAPE


def test_noalloc_prefill_rejects_what_its_scratch_cannot_hold():
    """gdn_prefill_chunked_noalloc validates like gdn_prefill_chunked and refuses a call
    whose workspace would exceed its static scratch, before any HIP call."""
    lib = ops.load()
    d = dims(head_map=ops.MAP_GROUPED)
    Hk, Hv = 16, 32
    big = dims(Hk=Hk, Hv=Hv, head_map=ops.MAP_GROUPED)
    T = 4096
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(big), 1, T) > ops.NOALLOC_SCRATCH_BYTES
    cu = (ctypes.c_int32 * 2)(0, T)

    def call(dd, cu_h, total, N):
        return lib.gdn_prefill_chunked_noalloc(ctypes.byref(dd), N, cu_h, vp(P16), total,
                                               ctypes.byref(inputs(q_stride=4096, k_stride=4096,
                                                                   v_stride=4096)),
                                               vp(P16), 0, vp(P16), None)
    assert call(big, cu, T, 1) == 8  # GDN_ERR_SCRATCH
    assert ops.status_string(8).startswith("the call needs more")
    small = (ctypes.c_int32 * 3)(0, 100, 230)
    bad = (ctypes.c_int32 * 3)(0, 150, 100)
    assert call(d, bad, 230, 2) == SHAPE
    assert call(dims(Hk=3), small, 230, 2) == SHAPE
    assert call(dims(dk=96, dv=128), small, 230, 2) == UNSUPPORTED
    zero = (ctypes.c_int32 * 3)(0, 0, 0)
    assert call(d, zero, 0, 2) == OK  # nothing to do: no HIP call, nothing launched


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 64), (96, 96), (64, 128), (128, 64), (128, 256),
                                   (256, 128), (256, 256)])
def test_prefill_other_head_shapes_take_the_one_kernel_path(dk, dv):
    """Head shapes other than 128 x 128 run the f32 path: a preparation kernel per
    (chunk, k-head) and a carry per (sequence, v-head, 32 dv rows), with 64-token
    chunks (32 at dk = 256); 128 x 128 keeps the f16-operand MFMA kernels."""
    lengths = [100, 0, 37]
    clen = 32 if dk == 256 else 64
    chunks = sum((n + clen - 1) // clen for n in lengths)
    i = ops.prefill_launch_info(lengths, Hk=2, Hv=4, dk=dk, dv=dv, compute_units=256)
    assert (i["carry_kind"], i["slices_per_workgroup"]) == (2, 2)
    assert i["prep_workgroups"] == chunks * 2
    assert i["workgroups"] == len(lengths) * 4 * (dv // 32) and i["threads"] == 512
    # the workspace: per (chunk, k-head) q, per (chunk, v-head) diag(e) K, W, U,
    # Aqk and decay rows, f32; the gated norm adds its f32 core output
    d = dims(dk=dk, dv=dv)
    mc = 137 // clen + 3
    floor = 4 * mc * (2 * clen * dk + 4 * (2 * clen * dk + clen * dv + clen * clen + 3 * clen))
    need = ops.load().gdn_prefill_workspace_bytes(ctypes.byref(d), 3, 137)
    assert floor <= need <= floor + 16 * 256
    dn = dims(dk=dk, dv=dv, flags=ops.GATED_NORM)
    assert ops.load().gdn_prefill_workspace_bytes(ctypes.byref(dn), 3, 137) >= need + 137 * 4 * dv * 4
    i = ops.prefill_launch_info(lengths, Hk=2, Hv=4, dk=128, dv=128, compute_units=256)
    assert i["carry_kind"] in (0, 1) and i["prep_workgroups"] > 0
