"""GPU parity of gdn_conv_update + gdn_decode_step against the CPU oracle.

Both sides consume the same seeded inputs (synth); the oracle widens them to
float64. Tolerances: max-abs 1e-3 on decode outputs and states (the
ferrum-kernels tests page's split-continuity diagnostic, adopted for the
decode contract); conv states are raw carried inputs and must match exactly;
a T-token call and its 3+1 split must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_linear_step_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 1e-3


def f64(t):
    return t.detach().cpu().double().numpy()


def maxabs(a, b):
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


def ulp16(x, dtype):
    """Spacing of the 16-bit format at |x|."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    mant = 10 if dtype == torch.float16 else 7
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
    return 2.0 ** (e - mant)


def run_layer(W, *, T, B, out_dtype=torch.float32, state=None, conv_state=None, x=None,
              slots=None, num_slots=None):
    """conv_update + decode_step on the GPU for workload W (tensors already on DEV)."""
    Hk, Hv, dk, dv = W["Hk"], W["Hv"], W["dk"], W["dv"]
    QK = Hk * dk
    y = ops.conv_update(W["x_d"] if x is None else x, W["conv_w_d"],
                        W["conv_state_d"] if conv_state is None else conv_state)
    out = ops.decode_step(y[:, :QK], y[:, QK:2 * QK], y[:, 2 * QK:],
                          W["state_d"] if state is None else state, Hk=Hk, Hv=Hv, dk=dk, dv=dv,
                          head_map=W["head_map"], batch=B, tokens_per_seq=T, a=W["a_d"],
                          b=W["b_d"], decay_param=W["A_log_d"], dt_bias=W["dt_bias_d"],
                          z=W["z_d"], norm_weight=W["norm_w_d"], out_dtype=out_dtype,
                          state_slots=slots)
    return out


def to_dev(W):
    for key in ("x", "z", "a", "b", "conv_w", "A_log", "dt_bias", "norm_w", "conv_state", "state"):
        W[key + "_d"] = W[key].to(DEV).contiguous()
    return W


def oracle_layer(W, B, T, state=None, conv_state=None):
    Hk, Hv, dk, dv = W["Hk"], W["Hv"], W["dk"], W["dv"]
    S0 = f64(W["state"]) if state is None else state
    cs0 = f64(W["conv_state"]) if conv_state is None else conv_state
    return oracle.batch(B=B, T=T, Hk=Hk, Hv=Hv, dk=dk, dv=dv, head_map=W["head_map"],
                        S0=S0.reshape(B, Hv, dv, dk), a=f64(W["a"]), b=f64(W["b"]),
                        decay_param=f64(W["A_log"]), dt_bias=f64(W["dt_bias"]), z=f64(W["z"]),
                        norm_w=f64(W["norm_w"]), x=f64(W["x"]), conv_w=f64(W["conv_w"]),
                        conv_state=cs0.reshape(B, -1, W["conv_k"] - 1), nthreads=8)


# ------------------------------------------------------------------ layer conformance (T=4, fp16)

def layer_conformance_workload():
    W = synth.layer_conformance()
    W["x"] = W["x"]
    W["z"] = W["z"].reshape(4, -1)
    W["state"] = W["state"].unsqueeze(0)
    W["conv_state"] = W["conv_state"].unsqueeze(0)
    return to_dev(W)


def test_layer_conformance_fp16_full_split_and_oracle():
    W = layer_conformance_workload()
    st_full, cs_full = W["state_d"].clone(), W["conv_state_d"].clone()
    out_full = run_layer(W, T=4, B=1, state=st_full, conv_state=cs_full)
    out16 = run_layer(W, T=4, B=1, out_dtype=torch.float16, state=W["state_d"].clone(),
                      conv_state=W["conv_state_d"].clone())
    # 3 + 1 split
    st_split, cs_split = W["state_d"].clone(), W["conv_state_d"].clone()
    Ws = dict(W)
    parts = []
    for lo, hi in ((0, 3), (3, 4)):
        for key in ("x", "z", "a", "b"):
            Ws[key + "_d"] = W[key + "_d"][lo:hi].contiguous()
        parts.append(run_layer(Ws, T=hi - lo, B=1, state=st_split, conv_state=cs_split))
    torch.cuda.synchronize()
    out_split = torch.cat(parts)
    assert torch.equal(out_full, out_split), "4-token call and 3+1 split differ"
    assert torch.equal(st_full, st_split) and torch.equal(cs_full, cs_split)

    y, cs, S = oracle_layer(W, B=1, T=4)
    o = f64(out_full).reshape(y.shape)
    assert np.any(np.abs(o) > 1e-4)
    assert maxabs(o, y) <= TOL
    assert maxabs(f64(st_full), S) <= TOL
    assert maxabs(f64(cs_full), cs) == 0.0
    o16 = f64(out16).reshape(y.shape)
    assert np.all(np.abs(o16 - y) <= ulp16(y, torch.float16) + TOL)


# ------------------------------------------------------------------ batched decode (B=64, bf16)

def test_batched_decode_b64_steps_1_and_8():
    B = 64
    W = to_dev(synth.decode_batch(seed=2, B=B, head_map=synth.TILED))
    S_ref, cs_ref = f64(W["state"]), f64(W["conv_state"])
    for step in range(1, 9):
        out = run_layer(W, T=1, B=B)
        y, cs_ref, S_ref = oracle_layer(W, B=B, T=1, state=S_ref, conv_state=cs_ref)
        if step in (1, 8):
            torch.cuda.synchronize()
            assert maxabs(f64(out).reshape(y.shape), y) <= TOL, f"out at step {step}"
            assert maxabs(f64(W["state_d"]), S_ref) <= TOL, f"state at step {step}"
            assert maxabs(f64(W["conv_state_d"]), cs_ref) == 0.0


@pytest.mark.parametrize("B", [1, 32])
def test_deep_model_layer_shapes_hv48(B):
    # Hk=16, Hv=48: two of the independently seeded layers of the 48-layer stack
    for layer in (0, 47):
        W = to_dev(synth.decode_batch(seed=4 * 1000 + layer, B=B, Hk=16, Hv=48,
                                      head_map=synth.TILED))
        out = run_layer(W, T=1, B=B)
        torch.cuda.synchronize()
        y, cs, S = oracle_layer(W, B=B, T=1)
        assert maxabs(f64(out).reshape(y.shape), y) <= TOL
        assert maxabs(f64(W["state_d"]), S) <= TOL
        assert maxabs(f64(W["conv_state_d"]), cs) == 0.0


# ------------------------------------------------------------------ small shapes, maps, dtypes

# every built (dk, dv) head shape
HEAD_SHAPES = [(32, 32), (64, 64), (128, 128), (64, 128), (128, 64), (128, 256), (256, 128),
               (96, 96), (256, 256)]


@pytest.mark.parametrize("dk,dv", HEAD_SHAPES)
@pytest.mark.parametrize("head_map", [synth.GROUPED, synth.TILED])
@pytest.mark.parametrize("T", [1, 11])
def test_core_given_gates_shapes(dk, dv, head_map, T):
    rng = np.random.default_rng(100 + dk + 3 * dv + T + head_map)
    B, Hk, Hv = 3, 2, 4
    q = torch.from_numpy(rng.normal(size=(B * T, Hk, dk)).astype(np.float32))
    k = torch.from_numpy(rng.normal(size=(B * T, Hk, dk)).astype(np.float32))
    v = torch.from_numpy(rng.normal(size=(B * T, Hv, dv)).astype(np.float32))
    g = torch.from_numpy(-np.abs(rng.normal(size=(B * T, Hv))).astype(np.float32))
    beta = torch.from_numpy(rng.uniform(0, 1, size=(B * T, Hv)).astype(np.float32))
    S0 = torch.from_numpy(rng.normal(0, 0.1, size=(B, Hv, dv, dk)).astype(np.float32))
    st = S0.to(DEV)
    out = ops.decode_step(q.to(DEV), k.to(DEV), v.to(DEV), st, Hk=Hk, Hv=Hv, dk=dk, dv=dv,
                          head_map=head_map, batch=B, tokens_per_seq=T, g=g.to(DEV),
                          beta=beta.to(DEV), l2norm_qk=True)
    torch.cuda.synchronize()
    for bi in range(B):
        sl = slice(bi * T, (bi + 1) * T)
        yo, So = oracle.core(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(S0[bi]), head_map,
                             g=f64(g[sl]), beta=f64(beta[sl]), l2norm_qk=True)
        assert maxabs(f64(out[sl]), yo) <= TOL
        assert maxabs(f64(st[bi]), So) <= TOL


@pytest.mark.parametrize("dk,dv", HEAD_SHAPES[3:])
@pytest.mark.parametrize("T", [1, 3])
def test_two_launch_layer_head_shapes(dk, dv, T):
    """conv update + decode step with L2 norm, raw gates and the gated norm at the
    non-square and 256-wide head shapes."""
    B = 2
    W = to_dev(synth.decode_batch(seed=60 + dk + dv + T, B=B, Hk=2, Hv=4, dk=dk, dv=dv, T=T))
    out = run_layer(W, T=T, B=B)
    torch.cuda.synchronize()
    y, cs, S = oracle_layer(W, B=B, T=T)
    assert maxabs(f64(out).reshape(y.shape), y) <= TOL
    assert maxabs(f64(W["state_d"]), S) <= TOL
    assert maxabs(f64(W["conv_state_d"]), cs) == 0.0


@pytest.mark.parametrize("act", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T", [1, 2])
def test_activation_and_output_dtypes(act, out_dtype, T):
    B = 4
    W = to_dev(synth.decode_batch(seed=7, B=B, T=T, Hk=2, Hv=4, head_map=synth.GROUPED,
                                  dtype=act))
    out = run_layer(W, T=T, B=B, out_dtype=out_dtype)
    torch.cuda.synchronize()
    y, cs, S = oracle_layer(W, B=B, T=T)
    o = f64(out).reshape(y.shape)
    if out_dtype == torch.float32:
        assert maxabs(o, y) <= TOL
    else:
        assert np.all(np.abs(o - y) <= ulp16(y, out_dtype) + TOL)
    assert maxabs(f64(W["state_d"]), S) <= TOL
    assert maxabs(f64(W["conv_state_d"]), cs) == 0.0


def test_state_slots_and_out_of_range_slot():
    # slot 99 is past the pool and -1 is a sentinel: neither sequence touches memory
    B, Hk, Hv, d = 5, 2, 4, 64
    rng = np.random.default_rng(21)
    q = torch.from_numpy(rng.normal(size=(B, Hk, d)).astype(np.float32)).to(DEV)
    k = torch.from_numpy(rng.normal(size=(B, Hk, d)).astype(np.float32)).to(DEV)
    v = torch.from_numpy(rng.normal(size=(B, Hv, d)).astype(np.float32)).to(DEV)
    g = torch.full((B, Hv), -0.1, device=DEV)
    beta = torch.full((B, Hv), 0.5, device=DEV)
    pool = torch.from_numpy(rng.normal(0, 0.1, size=(6, Hv, d, d)).astype(np.float32)).to(DEV)
    slot_list = [5, 0, 99, 2, -1]
    slots = torch.tensor(slot_list, dtype=torch.int32, device=DEV)
    before = pool.clone()
    out = torch.full((B, Hv, d), 7.0, device=DEV)
    ops.decode_step(q, k, v, pool, Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=synth.TILED, batch=B,
                    g=g, beta=beta, state_slots=slots, out=out)
    torch.cuda.synchronize()
    for bi, s in enumerate(slot_list):
        if s < 0 or s >= pool.shape[0]:
            assert torch.all(out[bi] == 7.0)
            continue
        yo, So = oracle.core(f64(q[bi:bi + 1]), f64(k[bi:bi + 1]), f64(v[bi:bi + 1]),
                             f64(before[s]), synth.TILED, g=f64(g[bi:bi + 1]),
                             beta=f64(beta[bi:bi + 1]))
        assert maxabs(f64(out[bi:bi + 1]), yo) <= TOL
        assert maxabs(f64(pool[s]), So) <= TOL
    for s in (1, 3, 4):  # slots no sequence named are untouched
        assert torch.equal(pool[s], before[s])


def test_sentinels_around_state_and_determinism():
    B, Hk, Hv, d = 8, 16, 32, 128
    W = to_dev(synth.decode_batch(seed=9, B=B, T=3, Hk=Hk, Hv=Hv, head_map=synth.TILED))
    n = B * Hv * d * d
    guard = torch.full((n + 64,), 73.25, device=DEV)
    guard[32:32 + n] = W["state_d"].reshape(-1)
    st = guard[32:32 + n].view(B, Hv, d, d)
    cs1 = W["conv_state_d"].clone()
    out1 = run_layer(W, T=3, B=B, state=st, conv_state=cs1)
    st2, cs2 = W["state_d"].clone(), W["conv_state_d"].clone()
    out2 = run_layer(W, T=3, B=B, state=st2, conv_state=cs2)
    torch.cuda.synchronize()
    assert torch.all(guard[:32] == 73.25) and torch.all(guard[32 + n:] == 73.25)
    assert torch.equal(out1, out2) and torch.equal(st, st2) and torch.equal(cs1, cs2)


def test_error_leaves_buffers_untouched():
    import ctypes
    W = to_dev(synth.decode_batch(seed=10, B=2, Hk=2, Hv=4, head_map=synth.TILED))
    st = W["state_d"].clone()
    before = st.clone()
    out = torch.full((2, 4, 128), 3.0, device=DEV)
    y = ops.conv_update(W["x_d"], W["conv_w_d"], W["conv_state_d"].clone())
    g = torch.zeros(2, 4, device=DEV)
    inp, keep = ops.make_inputs(y[:, :256], y[:, 256:512], y[:, 512:], Hk=2, Hv=4, dk=128,
                                dv=128, g=g, beta=g)
    lib = ops.load()
    for Hk, flags, status in ((3, 0, 2), (2, 64, 3)):  # Hv % Hk != 0; unknown flag bit
        dims = ops.make_dims(Hk, 4, 128, 128, synth.TILED, flags)
        rc = lib.gdn_decode_step(ctypes.byref(dims), 2, 1, ctypes.byref(inp),
                                 ctypes.c_void_p(st.data_ptr()), None, 2, ops.F32,
                                 ctypes.c_void_p(out.data_ptr()), None)
        assert rc == status
    torch.cuda.synchronize()
    assert torch.equal(st, before) and torch.all(out == 3.0)


@pytest.mark.parametrize("K", [2, 4, 6])
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.float16])
def test_conv_update_varlen_matches_oracle(K, y_dtype):
    rng = np.random.default_rng(22 + K)
    lengths = [5, 0, 1, 2, 9, 3]
    C = 300
    total = sum(lengths)
    x = torch.from_numpy(rng.normal(size=(total, C)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.normal(0, 0.5, size=(C, K)).astype(np.float32)).to(torch.bfloat16)
    cs = torch.from_numpy(rng.normal(size=(len(lengths), C, K - 1)).astype(np.float32)).to(
        torch.bfloat16)
    cu = synth.cu_seqlens(lengths)
    cs_d = cs.to(DEV)
    y = ops.conv_update(x.to(DEV), w.to(DEV), cs_d, cu_seqlens=cu.to(DEV), y_dtype=y_dtype)
    torch.cuda.synchronize()
    for i, n in enumerate(lengths):
        lo = int(cu[i])
        yo, so = oracle.conv(f64(x[lo:lo + n]).reshape(n, C), f64(w), f64(cs[i]))
        if n:
            err = np.abs(f64(y[lo:lo + n]) - yo)
            bound = 1e-5 if y_dtype == torch.float32 else ulp16(yo, y_dtype) + 1e-5
            assert np.all(err <= bound)
        assert maxabs(f64(cs_d[i]), so) == 0.0


@pytest.mark.parametrize("act", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("C", [8192, 300, 302])
def test_conv_update_one_token_per_sequence(act, y_dtype, C):
    # the decode shape (vectorised when C % 4 == 0, the generic kernel otherwise)
    rng = np.random.default_rng(23)
    N, K = 5, 4
    x = torch.from_numpy(rng.normal(size=(N, C)).astype(np.float32)).to(act)
    w = torch.from_numpy(rng.normal(0, 0.5, size=(C, K)).astype(np.float32)).to(act)
    cs = torch.from_numpy(rng.normal(size=(N, C, K - 1)).astype(np.float32)).to(act)
    cs_d = cs.to(DEV)
    y = ops.conv_update(x.to(DEV), w.to(DEV), cs_d, y_dtype=y_dtype)
    torch.cuda.synchronize()
    for i in range(N):
        yo, so = oracle.conv(f64(x[i:i + 1]), f64(w), f64(cs[i]))
        err = np.abs(f64(y[i:i + 1]) - yo)
        bound = 1e-5 if y_dtype == torch.float32 else ulp16(yo, y_dtype) + 1e-5
        assert np.all(err <= bound)
        assert maxabs(f64(cs_d[i]), so) == 0.0


def test_negative_rate_decay_matches_oracle():
    # decay parameter given as -exp(A_log) (the NegativeRate parameterisation)
    B, T = 3, 2
    W = to_dev(synth.decode_batch(seed=31, B=B, T=T, Hk=2, Hv=4, head_map=synth.TILED))
    neg = -torch.exp(W["A_log"])
    Hk, Hv, d = 2, 4, 128
    QK = Hk * d
    y = ops.conv_update(W["x_d"], W["conv_w_d"], W["conv_state_d"])
    out = ops.decode_step(y[:, :QK], y[:, QK:2 * QK], y[:, 2 * QK:], W["state_d"], Hk=Hk, Hv=Hv,
                          dk=d, dv=d, head_map=synth.TILED, batch=B, tokens_per_seq=T,
                          a=W["a_d"], b=W["b_d"], decay_param=neg.to(DEV),
                          dt_bias=W["dt_bias_d"], z=W["z_d"], norm_weight=W["norm_w_d"],
                          decay=ops.DECAY_NEGATIVE_RATE)
    torch.cuda.synchronize()
    yo, cs, S = oracle.batch(B=B, T=T, Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=synth.TILED,
                             S0=f64(W["state"]), a=f64(W["a"]), b=f64(W["b"]),
                             decay_param=f64(neg), dt_bias=f64(W["dt_bias"]), z=f64(W["z"]),
                             norm_w=f64(W["norm_w"]), x=f64(W["x"]), conv_w=f64(W["conv_w"]),
                             conv_state=f64(W["conv_state"]), nthreads=8,
                             decay_kind=oracle.DECAY_NEGATIVE_RATE)
    assert maxabs(f64(out).reshape(yo.shape), yo) <= TOL
    assert maxabs(f64(W["state_d"]), S) <= TOL


@pytest.mark.parametrize("T", [2, 4, 8])
def test_multi_token_verify_decode_b64(T):
    # several tokens per sequence in one call: the state is read and written once
    B = 64
    W = to_dev(synth.decode_batch(seed=40 + T, B=B, T=T, head_map=synth.TILED))
    out = run_layer(W, T=T, B=B)
    torch.cuda.synchronize()
    y, cs, S = oracle_layer(W, B=B, T=T)
    assert maxabs(f64(out).reshape(y.shape), y) <= TOL
    assert maxabs(f64(W["state_d"]), S) <= TOL
    assert maxabs(f64(W["conv_state_d"]), cs) == 0.0


# ------------------------------------------------------------------ the ferrox-core device-step shapes

def within_device_step_bound(a, b):
    """The ferrox-core device-step test's bound, |a - b| <= 2e-4 max(|b|, 1), element
    by element (checked beside this contract's 1e-3 max-abs)."""
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return bool(np.all(np.abs(a - b) <= 2e-4 * np.maximum(np.abs(b), 1.0)))


@pytest.mark.parametrize("head_map", [synth.TILED, synth.GROUPED])
def test_device_step_shapes_4_48_128(head_map):
    """(n_k, n_v, S) = (4, 48, 128), tiled and grouped (a 12:1 head map), one token
    of one sequence with the ferrox-core test's LCG draws: un-normalised uniform q
    and k, g = -|u|, beta = 0.5 + 0.25 u, state uniform in [-0.5, 0.5), no L2 norm,
    given gates, the core output (ferrox-core gdn.rs,
    `the_device_delta_step_matches_this_one`)."""
    n_k, n_v, s = 4, 48, 128
    W = synth.device_step(n_k, n_v, s)
    state = W["state"].unsqueeze(0).to(DEV).contiguous()
    out = ops.decode_step(W["q"].reshape(1, -1).to(DEV), W["k"].reshape(1, -1).to(DEV),
                          W["v"].reshape(1, -1).to(DEV), state, Hk=n_k, Hv=n_v, dk=s, dv=s,
                          head_map=head_map, batch=1, g=W["g"].to(DEV), beta=W["beta"].to(DEV),
                          l2norm_qk=False)
    torch.cuda.synchronize()
    y, S = oracle.core(f64(W["q"]), f64(W["k"]), f64(W["v"]), f64(W["state"]), head_map,
                       g=f64(W["g"]), beta=f64(W["beta"]), l2norm_qk=False)
    o = f64(out).reshape(y.shape)
    assert np.max(np.abs(y)) > 1.0  # un-normalised keys: outputs well above 1
    assert maxabs(o, y) <= TOL and maxabs(f64(state[0]), S) <= TOL
    assert within_device_step_bound(o, y) and within_device_step_bound(f64(state[0]), S)


def test_device_step_d4_is_not_built():
    """The ferrox-core test's third shape, (2, 2, 4), has 4-wide heads, which no
    kernel here is built for: the call is refused, and the oracle alone covers
    d = 4 (exact-rational and hand-worked pins)."""
    W = synth.device_step(2, 2, 4)
    state = W["state"].unsqueeze(0).to(DEV).contiguous()
    before = state.clone()
    with pytest.raises(ops.GdnError) as e:
        ops.decode_step(W["q"].reshape(1, -1).to(DEV), W["k"].reshape(1, -1).to(DEV),
                        W["v"].reshape(1, -1).to(DEV), state, Hk=2, Hv=2, dk=4, dv=4,
                        head_map=synth.TILED, batch=1, g=W["g"].to(DEV), beta=W["beta"].to(DEV),
                        l2norm_qk=False)
    assert e.value.status == 3  # GDN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(state, before)
