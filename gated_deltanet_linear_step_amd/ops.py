"""Thin ctypes binding over libgdn.so (the C ABI in include/gdn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libgdn.so. Tensors must already live on the GPU; the current torch
stream is passed to the library. If the library has not been built, the first
call raises -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIB_PATH selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("GDN_LIB_PATH") or os.path.join(HERE, "libgdn.so")

GDN_OK = 0
STATUS_NAMES = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_UNSUPPORTED",
                4: "GDN_ERR_OVERFLOW", 5: "GDN_ERR_ALIGN", 6: "GDN_ERR_WORKSPACE",
                7: "GDN_ERR_LAUNCH", 8: "GDN_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20
F32, F16, BF16 = 0, 1, 2
MAP_GROUPED, MAP_TILED = 0, 1
DECAY_LOG_RATE, DECAY_NEGATIVE_RATE = 0, 1
L2NORM_QK, RAW_GATES, GATED_NORM, STREAM_STATE = 1, 2, 4, 8
CHUNK = 64

EXPORTED = ["gdn_conv_update", "gdn_decode_step", "gdn_prefill_workspace_bytes",
            "gdn_prefill_chunked", "gdn_status_string", "gdn_version", "gdn_decode_layer",
            "gdn_decode_launch_info", "gdn_prefill_launch_info", "gdn_prefill_chunked_noalloc"]

_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_VP = ctypes.c_void_p


class Dims(ctypes.Structure):
    _fields_ = [("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("head_map", ctypes.c_int32), ("decay", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("scale", ctypes.c_float),
                ("l2_eps", ctypes.c_float), ("norm_eps", ctypes.c_float)]


class Inputs(ctypes.Structure):
    _fields_ = [("q", _VP), ("k", _VP), ("v", _VP),
                ("q_stride", ctypes.c_int64), ("k_stride", ctypes.c_int64),
                ("v_stride", ctypes.c_int64), ("qkv_dtype", ctypes.c_int32),
                ("a", _VP), ("b", _VP), ("ab_dtype", ctypes.c_int32),
                ("decay_param", _VP), ("dt_bias", _VP),
                ("g", _VP), ("beta", _VP),
                ("z", _VP), ("z_dtype", ctypes.c_int32), ("norm_weight", _VP)]


class ConvArgs(ctypes.Structure):
    _fields_ = [("kernel_size", ctypes.c_int32), ("weight", _VP), ("state_in", _VP),
                ("state_out", _VP)]


class LaunchInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("waves", "lanes_per_row", "token_mode", "nontemporal", "carry_kind",
                 "slices_per_workgroup", "workgroups", "threads", "prep_workgroups")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_LIB = None


def load() -> ctypes.CDLL:
    """Load libgdn.so from the package directory (raises if it is not built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_version.restype = ctypes.c_int32
    lib.gdn_conv_update.restype = ctypes.c_int
    lib.gdn_conv_update.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _VP,
                                    ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_int64, _VP, _VP,
                                    ctypes.c_int32, _VP, ctypes.c_int64, _VP]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32,
                                    ctypes.POINTER(Inputs), _VP, _VP, ctypes.c_int32,
                                    ctypes.c_int32, _VP, _VP]
    lib.gdn_decode_layer.restype = ctypes.c_int
    lib.gdn_decode_layer.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32,
                                     ctypes.POINTER(ConvArgs), ctypes.POINTER(Inputs), _VP, _VP,
                                     ctypes.c_int32, ctypes.c_int32, _VP, _VP]
    lib.gdn_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_prefill_workspace_bytes.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32,
                                                ctypes.c_int32]
    lib.gdn_prefill_chunked.restype = ctypes.c_int
    lib.gdn_prefill_chunked.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32, _VP, _VP,
                                        ctypes.c_int32, ctypes.POINTER(Inputs), _VP,
                                        ctypes.c_int32, _VP, _VP, ctypes.c_size_t, _VP]
    lib.gdn_prefill_chunked_noalloc.restype = ctypes.c_int
    lib.gdn_prefill_chunked_noalloc.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32, _VP, _VP,
                                                ctypes.c_int32, ctypes.POINTER(Inputs), _VP,
                                                ctypes.c_int32, _VP, _VP]
    lib.gdn_decode_launch_info.restype = ctypes.c_int
    lib.gdn_decode_launch_info.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.POINTER(LaunchInfo)]
    lib.gdn_prefill_launch_info.restype = ctypes.c_int
    lib.gdn_prefill_launch_info.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32, _VP,
                                            ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(LaunchInfo)]
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load().gdn_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != GDN_OK:
        raise GdnError(status, what)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _dt(t) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _stream(stream=None) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _row_view(t, width: int, name: str):
    """(tensor, row stride in elements) for a [rows, ..., width-elements] activation."""
    if t.dim() < 2:
        raise ValueError(f"{name}: need at least 2 dims")
    flat_inner = 1
    for s in t.shape[1:]:
        flat_inner *= s
    if flat_inner != width:
        raise ValueError(f"{name}: inner size {flat_inner} != {width}")
    # inner dims must be contiguous; the row stride may be larger (views into a mixed row)
    exp = 1
    for d in range(t.dim() - 1, 0, -1):
        if t.shape[d] != 1 and t.stride(d) != exp:
            raise ValueError(f"{name}: inner dims must be contiguous")
        exp *= t.shape[d]
    return t, t.stride(0)


def _cu_device(cu, device):
    """cu_seqlens as the device int32 [N+1] tensor the kernels read (a copy when the
    caller's tensor has another dtype or lives elsewhere)."""
    if cu is None:
        return None
    if cu.dtype.is_floating_point or cu.dim() != 1:
        raise TypeError("cu_seqlens must be a 1-d integer tensor")
    return cu.to(device=device, dtype=torch.int32).contiguous()


def _cu_host(cu):
    """cu_seqlens as a host int32 [N+1] tensor (the prefill validates it there)."""
    if cu.dtype.is_floating_point or cu.dim() != 1:
        raise TypeError("cu_seqlens must be a 1-d integer tensor")
    return cu.to(device="cpu", dtype=torch.int32).contiguous()


def _check_state(state, Hv, dv, dk):
    if state.dtype != torch.float32 or not state.is_contiguous():
        raise ValueError("state must be contiguous float32")
    if state.dim() != 4 or tuple(state.shape[1:]) != (Hv, dv, dk):
        raise ValueError(f"state must be [slots][{Hv}][{dv}][{dk}], got {tuple(state.shape)}")


def _check_out(out, rows, Hv, dv):
    if out.dtype not in _DT or not out.is_contiguous():
        raise ValueError("out must be contiguous f32, f16 or bf16")
    if out.numel() != rows * Hv * dv or out.shape[0] != rows:
        raise ValueError(f"out must be [{rows}][{Hv}][{dv}], got {tuple(out.shape)}")


def _check_conv(conv_weight, conv_state_in, conv_state_out, qdtype, slots, channels):
    K = conv_weight.shape[1] if conv_weight.dim() == 2 else -1
    if tuple(conv_weight.shape) != (channels, K):
        raise ValueError(f"conv_weight must be [{channels}][K]")
    for name, t in (("conv_weight", conv_weight), ("conv_state_in", conv_state_in),
                    ("conv_state_out", conv_state_out)):
        if t.dtype != qdtype or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous in q's dtype")
    for name, t in (("conv_state_in", conv_state_in), ("conv_state_out", conv_state_out)):
        if tuple(t.shape) != (slots, channels, K - 1):
            raise ValueError(f"{name} must be [{slots}][{channels}][{K - 1}]")


def _check_slots(state_slots, batch):
    if state_slots is None:
        return
    if state_slots.dtype != torch.int32 or not state_slots.is_contiguous() or \
            state_slots.numel() != batch:
        raise ValueError(f"state_slots must be a contiguous int32 [{batch}] tensor")


def make_dims(Hk, Hv, dk, dv, head_map, flags, decay=DECAY_LOG_RATE, scale=0.0, l2_eps=0.0,
              norm_eps=0.0) -> Dims:
    return Dims(Hk, Hv, dk, dv, head_map, decay, flags, scale, l2_eps, norm_eps)


def make_inputs(q, k, v, *, Hk, Hv, dk, dv, a=None, b=None, decay_param=None, dt_bias=None,
                g=None, beta=None, z=None, norm_weight=None):
    q, qs = _row_view(q, Hk * dk, "q")
    k, ks = _row_view(k, Hk * dk, "k")
    v, vs = _row_view(v, Hv * dv, "v")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    keep = [q, k, v]
    inp = Inputs(q=_ptr(q), k=_ptr(k), v=_ptr(v), q_stride=qs, k_stride=ks, v_stride=vs,
                 qkv_dtype=_dt(q))
    if a is not None:
        for t in (a, b):
            if not t.is_contiguous():
                raise ValueError("a, b must be contiguous [tokens][Hv]")
        if decay_param.dtype != torch.float32 or dt_bias.dtype != torch.float32:
            raise TypeError("decay_param and dt_bias must be float32")
        inp.a, inp.b, inp.ab_dtype = _ptr(a), _ptr(b), _dt(a)
        inp.decay_param, inp.dt_bias = _ptr(decay_param), _ptr(dt_bias)
        keep += [a, b, decay_param, dt_bias]
    if g is not None:
        if g.dtype != torch.float32 or beta.dtype != torch.float32:
            raise TypeError("g and beta must be float32")
        if not (g.is_contiguous() and beta.is_contiguous()):
            raise ValueError("g, beta must be contiguous [tokens][Hv]")
        inp.g, inp.beta = _ptr(g), _ptr(beta)
        keep += [g, beta]
    if z is not None:
        if not z.is_contiguous():
            raise ValueError("z must be contiguous [tokens][Hv][dv]")
        if norm_weight.dtype != torch.float32:
            raise TypeError("norm_weight must be float32")
        inp.z, inp.z_dtype, inp.norm_weight = _ptr(z), _dt(z), _ptr(norm_weight)
        keep += [z, norm_weight]
    return inp, keep


def decode_launch_info(*, Hk, Hv, dk, dv, batch, tokens_per_seq=1, fused_conv=True,
                       head_map=MAP_TILED, flags=L2NORM_QK | RAW_GATES | GATED_NORM) -> dict:
    """The decode kernel gdn_decode_layer (fused_conv) or gdn_decode_step would run."""
    dims = make_dims(Hk, Hv, dk, dv, head_map, flags)
    info = LaunchInfo()
    _check(load().gdn_decode_launch_info(ctypes.byref(dims), batch, tokens_per_seq,
                                         int(fused_conv), ctypes.byref(info)),
           "gdn_decode_launch_info")
    return info.as_dict()


def prefill_launch_info(lengths, *, Hk, Hv, dk, dv, compute_units, head_map=MAP_GROUPED,
                        flags=L2NORM_QK | RAW_GATES) -> dict:
    """The prefill kernels gdn_prefill_chunked would run for these sequence lengths
    on a device with `compute_units` CUs."""
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    arr = (ctypes.c_int32 * len(cu))(*cu)
    dims = make_dims(Hk, Hv, dk, dv, head_map, flags)
    info = LaunchInfo()
    _check(load().gdn_prefill_launch_info(ctypes.byref(dims), len(lengths), arr, cu[-1],
                                          compute_units, ctypes.byref(info)),
           "gdn_prefill_launch_info")
    return info.as_dict()


def conv_update(x, weight, conv_state, *, cu_seqlens=None, num_seqs=None, y=None,
                y_dtype=torch.float32, stream=None):
    """Causal depthwise conv + SiLU over x [tokens][C] (rows may be strided),
    weight [C][K], conv_state [N][C][K-1] (updated in place). Returns y."""
    total, C = x.shape
    if x.stride(1) != 1:
        raise ValueError("x channels must be contiguous")
    K = weight.shape[1]
    N = conv_state.shape[0] if num_seqs is None else num_seqs
    if weight.dtype != x.dtype or conv_state.dtype != x.dtype:
        raise TypeError("weight and conv_state must have x's dtype")
    if not (weight.is_contiguous() and conv_state.is_contiguous()):
        raise ValueError("weight and conv_state must be contiguous")
    if tuple(weight.shape) != (C, K) or tuple(conv_state.shape[1:]) != (C, K - 1) or \
            conv_state.shape[0] < N:
        raise ValueError("weight must be [C][K] and conv_state [N][C][K-1]")
    cu_seqlens = _cu_device(cu_seqlens, x.device)
    if cu_seqlens is not None and cu_seqlens.numel() != N + 1:
        raise ValueError("cu_seqlens must hold N + 1 offsets")
    if y is None:
        y = torch.empty((total, C), dtype=y_dtype, device=x.device)
    if y.dim() != 2 or y.shape[0] != total or y.shape[1] < C or y.stride(1) != 1:
        raise ValueError("y must be [tokens][>= C] with contiguous channels")
    st = load().gdn_conv_update(C, K, N, _ptr(cu_seqlens), total, _dt(x), _ptr(x), x.stride(0),
                                _ptr(weight), _ptr(conv_state), _dt(y), _ptr(y), y.stride(0),
                                _stream(stream))
    _check(st, "gdn_conv_update")
    return y


def decode_step(q, k, v, state, *, Hk, Hv, dk, dv, head_map, batch, tokens_per_seq=1,
                a=None, b=None, decay_param=None, dt_bias=None, g=None, beta=None, z=None,
                norm_weight=None, l2norm_qk=True, decay=DECAY_LOG_RATE, scale=0.0,
                state_slots=None, out=None, out_dtype=torch.float32, stream_state=False,
                stream=None):
    """One call of gdn_decode_step. q, k [B*T][Hk*dk] (views allowed), v [B*T][Hv*dv],
    state [slots][Hv][dv][dk] f32 updated in place. Returns out [B*T][Hv][dv].
    stream_state sets GDN_STREAM_STATE (non-temporal state loads and stores)."""
    flags = (L2NORM_QK if l2norm_qk else 0) | (RAW_GATES if a is not None else 0) | \
        (GATED_NORM if z is not None else 0) | (STREAM_STATE if stream_state else 0)
    dims = make_dims(Hk, Hv, dk, dv, head_map, flags, decay, scale)
    inp, keep = make_inputs(q, k, v, Hk=Hk, Hv=Hv, dk=dk, dv=dv, a=a, b=b,
                            decay_param=decay_param, dt_bias=dt_bias, g=g, beta=beta, z=z,
                            norm_weight=norm_weight)
    _check_state(state, Hv, dv, dk)
    rows = batch * tokens_per_seq
    if out is None:
        out = torch.empty((rows, Hv, dv), dtype=out_dtype, device=state.device)
    _check_out(out, rows, Hv, dv)
    _check_slots(state_slots, batch)
    num_slots = state.shape[0]
    st = load().gdn_decode_step(ctypes.byref(dims), batch, tokens_per_seq, ctypes.byref(inp),
                                _ptr(state), _ptr(state_slots), num_slots, _dt(out), _ptr(out),
                                _stream(stream))
    _check(st, "gdn_decode_step")
    del keep
    return out


def decode_layer(q, k, v, state, conv_weight, conv_state_in, conv_state_out, *, Hk, Hv, dk, dv,
                 head_map, batch, tokens_per_seq=1, a=None, b=None, decay_param=None,
                 dt_bias=None, g=None, beta=None, z=None, norm_weight=None, l2norm_qk=True,
                 decay=DECAY_LOG_RATE, scale=0.0, state_slots=None, out=None,
                 out_dtype=torch.float32, stream_state=False, stream=None):
    """One call of gdn_decode_layer: q, k, v are the pre-conv projections (views of
    the mixed row allowed); conv_weight [channels][4], conv states [slots][channels][3]
    in q's dtype (read from conv_state_in, the new window written to conv_state_out);
    state [slots][Hv][dv][dk] f32 updated in place. Returns out [B*T][Hv][dv].
    stream_state sets GDN_STREAM_STATE (non-temporal state loads and stores)."""
    flags = (L2NORM_QK if l2norm_qk else 0) | (RAW_GATES if a is not None else 0) | \
        (GATED_NORM if z is not None else 0) | (STREAM_STATE if stream_state else 0)
    dims = make_dims(Hk, Hv, dk, dv, head_map, flags, decay, scale)
    inp, keep = make_inputs(q, k, v, Hk=Hk, Hv=Hv, dk=dk, dv=dv, a=a, b=b,
                            decay_param=decay_param, dt_bias=dt_bias, g=g, beta=beta, z=z,
                            norm_weight=norm_weight)
    _check_state(state, Hv, dv, dk)
    _check_conv(conv_weight, conv_state_in, conv_state_out, q.dtype, state.shape[0],
                2 * Hk * dk + Hv * dv)
    conv = ConvArgs(conv_weight.shape[1], _ptr(conv_weight), _ptr(conv_state_in),
                    _ptr(conv_state_out))
    rows = batch * tokens_per_seq
    if out is None:
        out = torch.empty((rows, Hv, dv), dtype=out_dtype, device=state.device)
    _check_out(out, rows, Hv, dv)
    _check_slots(state_slots, batch)
    st = load().gdn_decode_layer(ctypes.byref(dims), batch, tokens_per_seq, ctypes.byref(conv),
                                 ctypes.byref(inp), _ptr(state), _ptr(state_slots), state.shape[0],
                                 _dt(out), _ptr(out), _stream(stream))
    _check(st, "gdn_decode_layer")
    del keep
    return out


def prefill_workspace_bytes(*, Hk, Hv, dk, dv, head_map=MAP_GROUPED, num_seqs, total_tokens,
                            gated_norm=False, flags=None):
    """Workspace gdn_prefill_chunked needs; the gated norm needs more, so pass
    gated_norm=True (or the call's flags) for calls that apply it."""
    if flags is None:
        flags = GATED_NORM if gated_norm else 0
    dims = make_dims(Hk, Hv, dk, dv, head_map, flags)
    return int(load().gdn_prefill_workspace_bytes(ctypes.byref(dims), num_seqs, total_tokens))


def prefill_chunked(q, k, v, state, cu_seqlens, *, Hk, Hv, dk, dv, head_map, a=None, b=None,
                    decay_param=None, dt_bias=None, g=None, beta=None, z=None, norm_weight=None,
                    l2norm_qk=True, decay=DECAY_LOG_RATE, scale=0.0, out=None,
                    out_dtype=torch.float32, workspace=None, cu_seqlens_host=None, stream=None):
    """One call of gdn_prefill_chunked over packed sequences (cu_seqlens int32 [N+1]).
    state [N][Hv][dv][dk] f32: initial in, final out. Returns out [tokens][Hv][dv]."""
    flags = (L2NORM_QK if l2norm_qk else 0) | (RAW_GATES if a is not None else 0) | \
        (GATED_NORM if z is not None else 0)
    dims = make_dims(Hk, Hv, dk, dv, head_map, flags, decay, scale)
    inp, keep = make_inputs(q, k, v, Hk=Hk, Hv=Hv, dk=dk, dv=dv, a=a, b=b,
                            decay_param=decay_param, dt_bias=dt_bias, g=g, beta=beta, z=z,
                            norm_weight=norm_weight)
    cu_seqlens_host = _cu_host(cu_seqlens if cu_seqlens_host is None else cu_seqlens_host)
    cu_dev = _cu_device(cu_seqlens, state.device)
    if cu_dev.numel() != cu_seqlens_host.numel():
        raise ValueError("cu_seqlens and cu_seqlens_host differ in length")
    N = cu_seqlens_host.numel() - 1
    total = int(cu_seqlens_host[-1])
    _check_state(state, Hv, dv, dk)
    if state.shape[0] != N:
        raise ValueError(f"state must hold one slot per sequence ({N})")
    if out is None:
        out = torch.empty((total, Hv, dv), dtype=out_dtype, device=state.device)
    _check_out(out, total, Hv, dv)
    need = load().gdn_prefill_workspace_bytes(ctypes.byref(dims), N, total)
    if workspace is None:
        workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=state.device)
    host_ptr = ctypes.c_void_p(cu_seqlens_host.data_ptr())
    st = load().gdn_prefill_chunked(ctypes.byref(dims), N, host_ptr, _ptr(cu_dev), total,
                                    ctypes.byref(inp), _ptr(state), _dt(out), _ptr(out),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    _check(st, "gdn_prefill_chunked")
    del keep
    return out


def prefill_chunked_noalloc(q, k, v, state, cu_seqlens, out, *, cu_seqlens_host, Hk, Hv, dk, dv,
                            head_map, a=None, b=None, decay_param=None, dt_bias=None, g=None,
                            beta=None, z=None, norm_weight=None, l2norm_qk=True,
                            decay=DECAY_LOG_RATE, scale=0.0, stream=None):
    """One call of gdn_prefill_chunked_noalloc: the prefill with the library's static
    scratch as its workspace. The caller passes every buffer, out included, and the
    offsets on both sides (int32 [N+1] on the GPU and on the host), so the binding
    itself allocates nothing. Returns out."""
    flags = (L2NORM_QK if l2norm_qk else 0) | (RAW_GATES if a is not None else 0) | \
        (GATED_NORM if z is not None else 0)
    dims = make_dims(Hk, Hv, dk, dv, head_map, flags, decay, scale)
    inp, keep = make_inputs(q, k, v, Hk=Hk, Hv=Hv, dk=dk, dv=dv, a=a, b=b,
                            decay_param=decay_param, dt_bias=dt_bias, g=g, beta=beta, z=z,
                            norm_weight=norm_weight)
    for name, t, dev in (("cu_seqlens", cu_seqlens, True), ("cu_seqlens_host", cu_seqlens_host, False)):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.is_cuda != dev:
            raise ValueError(f"{name} must be a contiguous int32 tensor on the "
                             f"{'GPU' if dev else 'host'}")
    N = cu_seqlens_host.numel() - 1
    total = int(cu_seqlens_host[-1])
    _check_state(state, Hv, dv, dk)
    _check_out(out, total, Hv, dv)
    st = load().gdn_prefill_chunked_noalloc(ctypes.byref(dims), N,
                                            ctypes.c_void_p(cu_seqlens_host.data_ptr()),
                                            _ptr(cu_seqlens), total, ctypes.byref(inp),
                                            _ptr(state), _dt(out), _ptr(out), _stream(stream))
    _check(st, "gdn_prefill_chunked_noalloc")
    del keep
    return out


class PreparedCall:
    """A library call with its ctypes arguments built once; ``launch()`` re-issues
    it on the stream captured at preparation time (for tight timing loops and
    graph capture, where per-call Python marshalling would dominate)."""

    def __init__(self, fn, args, what, keep):
        self._fn, self._args, self._what, self._keep = fn, args, what, keep

    def launch(self):
        st = self._fn(*self._args)
        if st != GDN_OK:
            raise GdnError(st, self._what)


def prepare_conv_update(x, weight, conv_state, y, *, cu_seqlens=None, num_seqs=None,
                        stream=None) -> PreparedCall:
    total, C = x.shape
    N = conv_state.shape[0] if num_seqs is None else num_seqs
    cu_seqlens = _cu_device(cu_seqlens, x.device)
    args = (C, weight.shape[1], N, _ptr(cu_seqlens), total, _dt(x), _ptr(x), x.stride(0),
            _ptr(weight), _ptr(conv_state), _dt(y), _ptr(y), y.stride(0), _stream(stream))
    return PreparedCall(load().gdn_conv_update, args, "gdn_conv_update",
                        [x, weight, conv_state, y, cu_seqlens])


def prepare_decode_step(q, k, v, state, out, *, Hk, Hv, dk, dv, head_map, batch,
                        tokens_per_seq=1, a=None, b=None, decay_param=None, dt_bias=None,
                        g=None, beta=None, z=None, norm_weight=None, l2norm_qk=True,
                        decay=DECAY_LOG_RATE, scale=0.0, state_slots=None,
                        stream_state=False, stream=None) -> PreparedCall:
    flags = (L2NORM_QK if l2norm_qk else 0) | (RAW_GATES if a is not None else 0) | \
        (GATED_NORM if z is not None else 0) | (STREAM_STATE if stream_state else 0)
    dims = make_dims(Hk, Hv, dk, dv, head_map, flags, decay, scale)
    inp, keep = make_inputs(q, k, v, Hk=Hk, Hv=Hv, dk=dk, dv=dv, a=a, b=b,
                            decay_param=decay_param, dt_bias=dt_bias, g=g, beta=beta, z=z,
                            norm_weight=norm_weight)
    _check_state(state, Hv, dv, dk)
    _check_out(out, batch * tokens_per_seq, Hv, dv)
    _check_slots(state_slots, batch)
    args = (ctypes.byref(dims), batch, tokens_per_seq, ctypes.byref(inp), _ptr(state),
            _ptr(state_slots), state.shape[0], _dt(out), _ptr(out), _stream(stream))
    return PreparedCall(load().gdn_decode_step, args, "gdn_decode_step",
                        keep + [dims, inp, state, out, state_slots])


def prepare_decode_layer(q, k, v, state, conv_weight, conv_state_in, conv_state_out, out, *, Hk,
                         Hv, dk, dv, head_map, batch, tokens_per_seq=1, a=None, b=None,
                         decay_param=None, dt_bias=None, g=None, beta=None, z=None,
                         norm_weight=None, l2norm_qk=True, decay=DECAY_LOG_RATE, scale=0.0,
                         state_slots=None, stream_state=False, stream=None) -> PreparedCall:
    flags = (L2NORM_QK if l2norm_qk else 0) | (RAW_GATES if a is not None else 0) | \
        (GATED_NORM if z is not None else 0) | (STREAM_STATE if stream_state else 0)
    dims = make_dims(Hk, Hv, dk, dv, head_map, flags, decay, scale)
    inp, keep = make_inputs(q, k, v, Hk=Hk, Hv=Hv, dk=dk, dv=dv, a=a, b=b,
                            decay_param=decay_param, dt_bias=dt_bias, g=g, beta=beta, z=z,
                            norm_weight=norm_weight)
    _check_state(state, Hv, dv, dk)
    _check_conv(conv_weight, conv_state_in, conv_state_out, q.dtype, state.shape[0],
                2 * Hk * dk + Hv * dv)
    _check_out(out, batch * tokens_per_seq, Hv, dv)
    _check_slots(state_slots, batch)
    conv = ConvArgs(conv_weight.shape[1], _ptr(conv_weight), _ptr(conv_state_in),
                    _ptr(conv_state_out))
    args = (ctypes.byref(dims), batch, tokens_per_seq, ctypes.byref(conv), ctypes.byref(inp),
            _ptr(state), _ptr(state_slots), state.shape[0], _dt(out), _ptr(out), _stream(stream))
    return PreparedCall(load().gdn_decode_layer, args, "gdn_decode_layer",
                        keep + [dims, inp, conv, state, out, state_slots, conv_weight,
                                conv_state_in, conv_state_out])


def prepare_prefill_chunked(q, k, v, state, cu_seqlens_dev, cu_seqlens_host, out, workspace, *,
                            Hk, Hv, dk, dv, head_map, a=None, b=None, decay_param=None,
                            dt_bias=None, g=None, beta=None, z=None, norm_weight=None,
                            l2norm_qk=True, decay=DECAY_LOG_RATE, scale=0.0,
                            stream=None) -> PreparedCall:
    flags = (L2NORM_QK if l2norm_qk else 0) | (RAW_GATES if a is not None else 0) | \
        (GATED_NORM if z is not None else 0)
    dims = make_dims(Hk, Hv, dk, dv, head_map, flags, decay, scale)
    inp, keep = make_inputs(q, k, v, Hk=Hk, Hv=Hv, dk=dk, dv=dv, a=a, b=b,
                            decay_param=decay_param, dt_bias=dt_bias, g=g, beta=beta, z=z,
                            norm_weight=norm_weight)
    if cu_seqlens_host.device.type != "cpu" or cu_seqlens_host.dtype != torch.int32:
        raise ValueError("cu_seqlens_host must be a CPU int32 tensor")
    cu_seqlens_dev = _cu_device(cu_seqlens_dev, state.device)
    N = cu_seqlens_host.numel() - 1
    total = int(cu_seqlens_host[-1])
    _check_state(state, Hv, dv, dk)
    _check_out(out, total, Hv, dv)
    args = (ctypes.byref(dims), N, ctypes.c_void_p(cu_seqlens_host.data_ptr()),
            _ptr(cu_seqlens_dev), total, ctypes.byref(inp), _ptr(state), _dt(out), _ptr(out),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    return PreparedCall(load().gdn_prefill_chunked, args, "gdn_prefill_chunked",
                        keep + [dims, inp, state, out, workspace, cu_seqlens_dev,
                                cu_seqlens_host])
