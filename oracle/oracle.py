"""ctypes wrapper over the f64 C oracle (TEST INFRASTRUCTURE ONLY).

Every function takes and returns float64 numpy arrays. Callers widen f16/bf16
inputs to float64 before the call (exactly), and round outputs themselves.

Sources, as cited in ``gdn_oracle.c``:
  [FK] docs.rs ferrum-kernels 0.8.0, src/backend/metal/vnext_ops/gated_delta_attention_tests.rs
  [LM] docs.rs libmir-metal 0.1.0, src/engine/gated_delta_layer/decode/mod.rs
  [FC] docs.rs ferrox-core 0.24.0, src/gdn.rs
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "lib_path", "load", "sigmoid", "silu", "softplus", "k_head", "l2norm", "gates",
    "conv", "recurrence", "gated_rmsnorm", "core", "segment", "batch", "packed",
    "MAP_GROUPED", "MAP_TILED", "DECAY_LOG_RATE", "DECAY_NEGATIVE_RATE",
]

MAP_GROUPED, MAP_TILED = 0, 1
DECAY_LOG_RATE, DECAY_NEGATIVE_RATE = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_D = ctypes.POINTER(ctypes.c_double)


class _CoreCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("T", "Hk", "Hv", "dk", "dv", "map", "decay_kind", "l2norm", "raw_gates",
                 "gated_norm")] + \
               [("scale", ctypes.c_double), ("l2_eps", ctypes.c_double),
                ("norm_eps", ctypes.c_double), ("h_begin", ctypes.c_int), ("h_end", ctypes.c_int)]


def lib_path() -> str:
    # GDN_ORACLE_LIB selects another build of the same source (the sanitized one)
    return os.environ.get("GDN_ORACLE_LIB") or os.path.join(_HERE, "liboracle_gdn.so")


def load():
    """Load (building first if absent) the oracle library."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(path)
    for name in ("gdn_oracle_sigmoid", "gdn_oracle_silu", "gdn_oracle_softplus"):
        f = getattr(lib, name)
        f.restype, f.argtypes = ctypes.c_double, [ctypes.c_double]
    lib.gdn_oracle_k_head.restype = ctypes.c_int
    lib.gdn_oracle_k_head.argtypes = [ctypes.c_int] * 4
    lib.gdn_oracle_l2norm.restype = None
    lib.gdn_oracle_l2norm.argtypes = [_D, ctypes.c_int, ctypes.c_double]
    lib.gdn_oracle_gates.restype = None
    lib.gdn_oracle_gates.argtypes = [ctypes.c_int] * 3 + [_D] * 6
    lib.gdn_oracle_conv.restype = None
    lib.gdn_oracle_conv.argtypes = [ctypes.c_int] * 3 + [_D] * 4
    lib.gdn_oracle_recurrence.restype = None
    lib.gdn_oracle_recurrence.argtypes = [ctypes.c_int] * 6 + [ctypes.c_double] + [_D] * 7 + \
        [ctypes.c_int] * 2
    lib.gdn_oracle_gated_rmsnorm.restype = None
    lib.gdn_oracle_gated_rmsnorm.argtypes = [ctypes.c_int, ctypes.c_int, _D, _D, _D,
                                             ctypes.c_double, _D]
    lib.gdn_oracle_core.restype = ctypes.c_int
    lib.gdn_oracle_core.argtypes = [ctypes.POINTER(_CoreCfg)] + [_D] * 13
    lib.gdn_oracle_segment.restype = ctypes.c_int
    lib.gdn_oracle_segment.argtypes = [ctypes.POINTER(_CoreCfg), ctypes.c_int] + [_D] * 11
    lib.gdn_oracle_batch.restype = ctypes.c_int
    lib.gdn_oracle_batch.argtypes = [ctypes.POINTER(_CoreCfg)] + [ctypes.c_int] * 3 + [_D] * 14
    _LIB = lib
    return lib


def _f64(x, shape=None):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if shape is not None:
        a = a.reshape(shape)
    return a


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(_D)


def sigmoid(x: float) -> float:
    return load().gdn_oracle_sigmoid(float(x))


def silu(x: float) -> float:
    return load().gdn_oracle_silu(float(x))


def softplus(x: float) -> float:
    return load().gdn_oracle_softplus(float(x))


def k_head(head_map: int, h: int, num_k_heads: int, num_v_heads: int) -> int:
    return load().gdn_oracle_k_head(head_map, h, num_k_heads, num_v_heads)


def l2norm(x, eps: float = 1e-6):
    """Normalise each last-axis row of x (returns a new array)."""
    a = _f64(x).copy()
    n = a.shape[-1]
    flat = a.reshape(-1, n)
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        load().gdn_oracle_l2norm(_p(row), n, eps)
        flat[r] = row
    return flat.reshape(a.shape)


def gates(a, b, decay_param, dt_bias, decay_kind: int = DECAY_LOG_RATE):
    """(g, beta) from raw a, b [T][Hv] and per-head decay_param, dt_bias [Hv]."""
    a, b = _f64(a), _f64(b)
    T, Hv = a.shape
    dp, db = _f64(decay_param, (Hv,)), _f64(dt_bias, (Hv,))
    g = np.zeros((T, Hv))
    beta = np.zeros((T, Hv))
    load().gdn_oracle_gates(T, Hv, decay_kind, _p(dp), _p(db), _p(a), _p(b), _p(g), _p(beta))
    return g, beta


def conv(x, w, state):
    """Causal depthwise conv + SiLU. x [T][C], w [C][K], state [C][K-1] -> (y, new_state)."""
    x, w = _f64(x), _f64(w)
    T, C = x.shape
    K = w.shape[1]
    st = _f64(state, (C, K - 1)).copy()
    y = np.zeros((T, C))
    load().gdn_oracle_conv(T, C, K, _p(x), _p(w), _p(st), _p(y))
    return y, st


def recurrence(q, k, v, g, beta, S0, head_map: int, scale=None, heads=None):
    """The token-by-token rule. q, k [T][Hk][dk]; v [T][Hv][dv]; g, beta [T][Hv];
    S0 [Hv][dv][dk]. Returns (o [T][Hv][dv], S [Hv][dv][dk]). ``heads`` = (h0, h1)
    restricts the work to v-heads [h0, h1); other heads' o stay 0 and S unchanged."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    g, beta = _f64(g, (T, Hv)), _f64(beta, (T, Hv))
    S = _f64(S0, (Hv, dv, dk)).copy()
    o = np.zeros((T, Hv, dv))
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    h0, h1 = heads if heads is not None else (0, Hv)
    load().gdn_oracle_recurrence(T, Hk, Hv, dk, dv, head_map, float(scale), _p(q), _p(k), _p(v),
                                 _p(g), _p(beta), _p(S), _p(o), h0, h1)
    return o, S


def gated_rmsnorm(o, z, w, eps: float = 1e-6):
    o = _f64(o)
    dv = o.shape[-1]
    rows = o.size // dv
    z = _f64(z, o.shape)
    w = _f64(w, (dv,))
    y = np.zeros(o.shape)
    load().gdn_oracle_gated_rmsnorm(rows, dv, _p(o), _p(z), _p(w), eps, _p(y))
    return y


def _cfg(T, Hk, Hv, dk, dv, head_map, decay_kind, l2norm_qk, raw_gates, gated_norm, scale,
         l2_eps, norm_eps, heads):
    h0, h1 = heads if heads is not None else (0, Hv)
    return _CoreCfg(T, Hk, Hv, dk, dv, head_map, decay_kind, int(l2norm_qk), int(raw_gates),
                    int(gated_norm), float(1.0 / np.sqrt(dk) if scale is None else scale),
                    float(l2_eps), float(norm_eps), h0, h1)


def core(q, k, v, S0, head_map, *, a=None, b=None, decay_param=None, dt_bias=None, g=None,
         beta=None, z=None, norm_w=None, l2norm_qk=True, decay_kind=DECAY_LOG_RATE,
         scale=None, l2_eps=1e-6, norm_eps=1e-6, heads=None):
    """One sequence: [L2 norm q,k] -> gates (raw a/b, or given g/beta) -> recurrence
    -> [gated RMS norm when z is given]. Returns (y [T][Hv][dv], S)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    raw = a is not None
    gn = z is not None
    S = _f64(S0, (Hv, dv, dk)).copy()
    y = np.zeros((T, Hv, dv))
    cfg = _cfg(T, Hk, Hv, dk, dv, head_map, decay_kind, l2norm_qk, raw, gn, scale, l2_eps,
               norm_eps, heads)
    arrs = dict(
        a=_f64(a, (T, Hv)) if raw else None, b=_f64(b, (T, Hv)) if raw else None,
        dp=_f64(decay_param, (Hv,)) if raw else None, db=_f64(dt_bias, (Hv,)) if raw else None,
        g=None if raw else _f64(g, (T, Hv)), beta=None if raw else _f64(beta, (T, Hv)),
        z=_f64(z, (T, Hv, dv)) if gn else None, w=_f64(norm_w, (dv,)) if gn else None)
    rc = load().gdn_oracle_core(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(arrs["a"]),
                                _p(arrs["b"]), _p(arrs["dp"]), _p(arrs["db"]), _p(arrs["g"]),
                                _p(arrs["beta"]), _p(arrs["z"]), _p(arrs["w"]), _p(S), _p(y))
    if rc != 0:
        raise ValueError("oracle core: bad shape")
    return y, S


def segment(x, conv_w, conv_state, S0, *, Hk, Hv, dk, dv, head_map, a, b, decay_param,
            dt_bias, z, norm_w, decay_kind=DECAY_LOG_RATE, scale=None, l2_eps=1e-6,
            norm_eps=1e-6):
    """One sequence through the whole layer ([FK] `cpu_segment`): conv + SiLU over the
    mixed [q|k|v] channels, split, L2 norm, gates, recurrence, gated RMS norm.
    Returns (y [T][Hv][dv], conv_state', S')."""
    x = _f64(x)
    T = x.shape[0]
    Kc = _f64(conv_w).shape[1]
    QKV = 2 * Hk * dk + Hv * dv
    cw = _f64(conv_w, (QKV, Kc))
    cs = _f64(conv_state, (QKV, Kc - 1)).copy()
    S = _f64(S0, (Hv, dv, dk)).copy()
    y = np.zeros((T, Hv, dv))
    cfg = _cfg(T, Hk, Hv, dk, dv, head_map, decay_kind, True, True, True, scale, l2_eps,
               norm_eps, None)
    rc = load().gdn_oracle_segment(
        ctypes.byref(cfg), Kc, _p(x), _p(cw), _p(cs), _p(_f64(a, (T, Hv))),
        _p(_f64(b, (T, Hv))), _p(_f64(decay_param, (Hv,))), _p(_f64(dt_bias, (Hv,))),
        _p(_f64(z, (T, Hv, dv))), _p(_f64(norm_w, (dv,))), _p(S), _p(y))
    if rc != 0:
        raise ValueError("oracle segment: bad shape")
    return y, cs, S


def batch(*, B, T, Hk, Hv, dk, dv, head_map, S0, a, b, decay_param, dt_bias, z, norm_w,
          x=None, conv_w=None, conv_state=None, q=None, k=None, v=None, nthreads=1,
          decay_kind=DECAY_LOG_RATE):
    """B independent sequences of T tokens each, spread over host threads.
    With x/conv_w/conv_state: the whole layer per sequence; else q/k/v core
    (L2 norm, raw gates, gated norm). Arrays are batched along a leading B axis.
    Returns (y [B][T][Hv][dv], conv_state' or None, S')."""
    S = _f64(S0, (B, Hv, dv, dk)).copy()
    y = np.zeros((B, T, Hv, dv))
    cfg = _cfg(T, Hk, Hv, dk, dv, head_map, decay_kind, True, True, True, None, 1e-6, 1e-6,
               None)
    QKV = 2 * Hk * dk + Hv * dv
    if x is not None:
        Kc = _f64(conv_w).shape[1]
        xs = _f64(x, (B, T, QKV))
        cw = _f64(conv_w, (QKV, Kc))
        cs = _f64(conv_state, (B, QKV, Kc - 1)).copy()
        qq = kk = vv = None
    else:
        Kc = 0
        xs = cw = cs = None
        qq, kk = _f64(q, (B, T, Hk, dk)), _f64(k, (B, T, Hk, dk))
        vv = _f64(v, (B, T, Hv, dv))
    load().gdn_oracle_batch(
        ctypes.byref(cfg), Kc, B, int(nthreads), _p(xs), _p(cw), _p(cs), _p(qq), _p(kk), _p(vv),
        _p(_f64(a, (B, T, Hv))), _p(_f64(b, (B, T, Hv))), _p(_f64(decay_param, (Hv,))),
        _p(_f64(dt_bias, (Hv,))), _p(_f64(z, (B, T, Hv, dv))), _p(_f64(norm_w, (dv,))), _p(S),
        _p(y))
    return y, cs, S


def packed(q, k, v, S0, head_map, cu_seqlens, *, nthreads=1, heads=None, a=None, b=None,
           decay_param=None, dt_bias=None, g=None, beta=None, z=None, norm_w=None,
           l2norm_qk=True, decay_kind=DECAY_LOG_RATE, scale=None, l2_eps=1e-6, norm_eps=1e-6):
    """Packed variable-length sequences (cu_seqlens [N+1]) through ``core``, token by
    token. Each (sequence, v-head) pair is an independent problem: it is handed to
    ``core`` as a one-k-head, one-v-head call on its own slices (the k-head the map
    gives, that head's gates and parameters), and the pairs are spread over
    ``nthreads`` host threads. This driver adds no arithmetic.
    q, k [T][Hk][dk]; v [T][Hv][dv]; S0 [N][Hv][dv][dk]. Returns (y [T][Hv][dv],
    S [N][Hv][dv][dk]); v-heads outside ``heads`` keep y = 0 and S = S0."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    N = len(cu) - 1
    S = _f64(S0, (N, Hv, dv, dk)).copy()
    y = np.zeros((T, Hv, dv))
    raw = a is not None
    if raw:
        a, b = _f64(a, (T, Hv)), _f64(b, (T, Hv))
        dp, db = _f64(decay_param, (Hv,)), _f64(dt_bias, (Hv,))
    else:
        g, beta = _f64(g, (T, Hv)), _f64(beta, (T, Hv))
    if z is not None:
        z = _f64(z, (T, Hv, dv))
    heads = range(Hv) if heads is None else heads
    units = [(i, h) for i in range(N) if cu[i + 1] > cu[i] for h in heads]

    def one(unit):
        i, h = unit
        lo, hi = cu[i], cu[i + 1]
        kh = k_head(head_map, h, Hk, Hv)
        kw = dict(l2norm_qk=l2norm_qk, decay_kind=decay_kind, l2_eps=l2_eps, norm_eps=norm_eps,
                  scale=1.0 / np.sqrt(dk) if scale is None else scale)
        if raw:
            kw.update(a=a[lo:hi, h:h + 1], b=b[lo:hi, h:h + 1], decay_param=dp[h:h + 1],
                      dt_bias=db[h:h + 1])
        else:
            kw.update(g=g[lo:hi, h:h + 1], beta=beta[lo:hi, h:h + 1])
        if z is not None:
            kw.update(z=z[lo:hi, h:h + 1], norm_w=norm_w)
        yh, Sh = core(q[lo:hi, kh:kh + 1], k[lo:hi, kh:kh + 1], v[lo:hi, h:h + 1],
                      S[i, h:h + 1], MAP_GROUPED, **kw)
        return unit, yh, Sh

    with ThreadPoolExecutor(max_workers=max(1, int(nthreads))) as ex:
        for (i, h), yh, Sh in ex.map(one, units):
            y[cu[i]:cu[i + 1], h] = yh[:, 0]
            S[i, h] = Sh[0]
    return y, S
