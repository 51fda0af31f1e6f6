"""GPU parity of gdn_decode_layer (conv + the whole decode step in one launch)
against the CPU oracle, and against the two-launch path it replaces.

Same bars as the decode contract: max-abs 1e-3 on outputs and states; the conv
window is a carry of raw inputs and must match exactly; a T-token call and its
3+1 split agree bit for bit; the call never writes its input conv state.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_step_amd import ops, synth
from test_gpu_decode import DEV, TOL, f64, maxabs, oracle_layer, run_layer, to_dev, ulp16, \
    layer_conformance_workload

pytestmark = pytest.mark.gpu


def run_fused(W, *, T, B, cs_in, cs_out, out_dtype=torch.float32, state=None, x=None, z=None,
              a=None, b=None, slots=None, out=None, stream_state=False):
    Hk, Hv, dk, dv = W["Hk"], W["Hv"], W["dk"], W["dv"]
    QK = Hk * dk
    x = W["x_d"] if x is None else x
    return ops.decode_layer(x[:, :QK], x[:, QK:2 * QK], x[:, 2 * QK:],
                            W["state_d"] if state is None else state, W["conv_w_d"], cs_in,
                            cs_out, Hk=Hk, Hv=Hv, dk=dk, dv=dv, head_map=W["head_map"],
                            batch=B, tokens_per_seq=T, a=W["a_d"] if a is None else a,
                            b=W["b_d"] if b is None else b, decay_param=W["A_log_d"],
                            dt_bias=W["dt_bias_d"], z=W["z_d"] if z is None else z,
                            norm_weight=W["norm_w_d"], out_dtype=out_dtype, state_slots=slots,
                            out=out, stream_state=stream_state)


def test_fused_layer_conformance_fp16_split_and_oracle():
    W = layer_conformance_workload()
    cs0 = W["conv_state_d"].clone()
    st_full, cs_out = W["state_d"].clone(), torch.empty_like(cs0)
    out_full = run_fused(W, T=4, B=1, cs_in=cs0, cs_out=cs_out, state=st_full)
    # 3 + 1 split, alternating the conv buffers
    st_split, cs_a, cs_b = W["state_d"].clone(), cs0.clone(), torch.empty_like(cs0)
    parts = []
    for (lo, hi), (ci, co) in zip(((0, 3), (3, 4)), ((cs_a, cs_b), (cs_b, cs_a))):
        sl = lambda t: t[lo:hi].contiguous()  # noqa: E731
        parts.append(run_fused(W, T=hi - lo, B=1, cs_in=ci, cs_out=co, state=st_split,
                               x=sl(W["x_d"]), z=sl(W["z_d"]), a=sl(W["a_d"]), b=sl(W["b_d"])))
    torch.cuda.synchronize()
    assert torch.equal(cs0, W["conv_state_d"]), "the input conv state was written"
    assert torch.equal(out_full, torch.cat(parts)), "4-token call and 3+1 split differ"
    assert torch.equal(st_full, st_split) and torch.equal(cs_out, cs_a)

    y, cs, S = oracle_layer(W, B=1, T=4)
    o = f64(out_full).reshape(y.shape)
    assert np.any(np.abs(o) > 1e-4)
    assert maxabs(o, y) <= TOL
    assert maxabs(f64(st_full), S) <= TOL
    assert maxabs(f64(cs_out), cs) == 0.0
    # the two-launch path (conv_update + decode_step) on the same inputs
    st2 = W["state_d"].clone()
    out2 = run_layer(W, T=4, B=1, state=st2, conv_state=cs0.clone())
    torch.cuda.synchronize()
    assert maxabs(f64(out_full), f64(out2)) <= 1e-5
    assert maxabs(f64(st_full), f64(st2)) <= 1e-6


@pytest.mark.parametrize("stream_state", [False, True])
def test_fused_layer_b64_steps_1_and_8(stream_state):
    # the headline step, and (with the cache hint) the rotating leg's launch
    B = 64
    W = to_dev(synth.decode_batch(seed=2, B=B, head_map=synth.TILED))
    S_ref, cs_ref = f64(W["state"]), f64(W["conv_state"])
    bufs = [W["conv_state_d"].clone(), torch.empty_like(W["conv_state_d"])]
    for step in range(1, 9):
        out = run_fused(W, T=1, B=B, cs_in=bufs[0], cs_out=bufs[1], out_dtype=torch.float32,
                        stream_state=stream_state)
        bufs.reverse()
        y, cs_ref, S_ref = oracle_layer(W, B=B, T=1, state=S_ref, conv_state=cs_ref)
        if step in (1, 8):
            torch.cuda.synchronize()
            assert maxabs(f64(out).reshape(y.shape), y) <= TOL, f"step {step} output"
            assert maxabs(f64(W["state_d"]), S_ref) <= TOL, f"step {step} state"
            assert maxabs(f64(bufs[0]), cs_ref) == 0.0, f"step {step} conv state"


@pytest.mark.parametrize("dk,dv,Hk,Hv", [(128, 128, 2, 4), (64, 64, 2, 2), (32, 32, 1, 4),
                                         (64, 128, 2, 2), (128, 64, 2, 4), (128, 256, 2, 4),
                                         (256, 128, 1, 2), (96, 96, 2, 4), (256, 256, 1, 2)])
@pytest.mark.parametrize("head_map", [synth.GROUPED, synth.TILED])
@pytest.mark.parametrize("T", [1, 3, 9, 17])
def test_fused_layer_shapes_maps_tokens(dk, dv, Hk, Hv, head_map, T):
    B = 3
    W = to_dev(synth.decode_batch(seed=40 + T + dk + 2 * dv, B=B, Hk=Hk, Hv=Hv, dk=dk, dv=dv,
                                  T=T, head_map=head_map))
    cs_out = torch.full_like(W["conv_state_d"], 9.0)
    out = run_fused(W, T=T, B=B, cs_in=W["conv_state_d"], cs_out=cs_out)
    torch.cuda.synchronize()
    y, cs, S = oracle_layer(W, B=B, T=T)
    assert maxabs(f64(out).reshape(y.shape), y) <= TOL
    assert maxabs(f64(W["state_d"]), S) <= TOL
    assert maxabs(f64(cs_out), cs) == 0.0


@pytest.mark.parametrize("act", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fused_layer_dtypes(act, out_dtype):
    B, T = 4, 2
    W = to_dev(synth.decode_batch(seed=51, B=B, Hk=2, Hv=4, T=T, dtype=act))
    cs_out = torch.empty_like(W["conv_state_d"])
    out = run_fused(W, T=T, B=B, cs_in=W["conv_state_d"], cs_out=cs_out, out_dtype=out_dtype)
    torch.cuda.synchronize()
    y, cs, S = oracle_layer(W, B=B, T=T)
    o = f64(out).reshape(y.shape)
    bound = TOL if out_dtype == torch.float32 else ulp16(y, out_dtype) + TOL
    assert np.all(np.abs(o - y) <= bound)
    assert maxabs(f64(W["state_d"]), S) <= TOL
    assert maxabs(f64(cs_out), cs) == 0.0


def test_fused_layer_slots_and_out_of_range_slot():
    B, Hk, Hv, d, nslots = 4, 2, 4, 64, 5
    W = to_dev(synth.decode_batch(seed=61, B=nslots, Hk=Hk, Hv=Hv, dk=d, dv=d))
    slots = [4, 77, 1, -1]  # 77: past the pool; -1: a sentinel
    # activations of the three sequences; states and conv windows live in a pool of 5
    x = W["x_d"][:B].contiguous()
    z, a, b = W["z_d"][:B].contiguous(), W["a_d"][:B].contiguous(), W["b_d"][:B].contiguous()
    pool0, cs_pool0 = W["state_d"].clone(), W["conv_state_d"].clone()
    pool, cs_out = W["state_d"], torch.full_like(cs_pool0, 5.0)
    out = torch.full((B, Hv, d), 7.0, device=DEV)
    run_fused(W, T=1, B=B, cs_in=cs_pool0, cs_out=cs_out, x=x, z=z, a=a, b=b,
              slots=torch.tensor(slots, dtype=torch.int32, device=DEV), out=out)
    torch.cuda.synchronize()
    for bi, s in enumerate(slots):
        if s < 0 or s >= nslots:
            assert torch.all(out[bi] == 7.0)
            continue
        Wi = dict(W)
        for key in ("x", "z", "a", "b"):
            Wi[key] = W[key][bi:bi + 1]
        y, cs, S = oracle_layer(Wi, B=1, T=1, state=f64(pool0[s:s + 1]),
                                conv_state=f64(cs_pool0[s:s + 1]))
        assert maxabs(f64(out[bi:bi + 1]).reshape(y.shape), y) <= TOL
        assert maxabs(f64(pool[s]), S[0]) <= TOL
        assert maxabs(f64(cs_out[s]), cs[0]) == 0.0
    for s in (0, 2, 3):  # slots no sequence named: both states untouched
        assert torch.equal(pool[s], pool0[s])
        assert torch.all(cs_out[s] == 5.0)


@pytest.mark.parametrize("B", [1, 32])
def test_fused_layer_deep_model_shapes_hv48(B):
    # Hk=16, Hv=48: two of the independently seeded layers of the 48-layer stack,
    # through the launch the 48-layer benchmark leg uses (with the cache hint at
    # B=32, whose stack holds 4.8 GB of state)
    for layer in (0, 47):
        W = to_dev(synth.decode_batch(seed=4 * 1000 + layer, B=B, Hk=16, Hv=48,
                                      head_map=synth.TILED))
        cs_out = torch.empty_like(W["conv_state_d"])
        out = run_fused(W, T=1, B=B, cs_in=W["conv_state_d"], cs_out=cs_out,
                        out_dtype=torch.float32, stream_state=B == 32)
        torch.cuda.synchronize()
        y, cs, S = oracle_layer(W, B=B, T=1)
        assert maxabs(f64(out).reshape(y.shape), y) <= TOL
        assert maxabs(f64(W["state_d"]), S) <= TOL
        assert maxabs(f64(cs_out), cs) == 0.0


@pytest.mark.parametrize("T", [2, 4, 8])
def test_fused_layer_multi_token_verify_b64(T):
    # the benchmark's multi-token leg: B=64 sequences, T tokens each in one call
    B = 64
    W = to_dev(synth.decode_batch(seed=20 + T, B=B, T=T, head_map=synth.TILED))
    cs_out = torch.empty_like(W["conv_state_d"])
    out = run_fused(W, T=T, B=B, cs_in=W["conv_state_d"], cs_out=cs_out)
    torch.cuda.synchronize()
    y, cs, S = oracle_layer(W, B=B, T=T)
    assert maxabs(f64(out).reshape(y.shape), y) <= TOL
    assert maxabs(f64(W["state_d"]), S) <= TOL
    assert maxabs(f64(cs_out), cs) == 0.0


@pytest.mark.parametrize("T", [1, 3])
def test_stream_state_hint_is_bitwise_neutral(T):
    """GDN_STREAM_STATE only changes the cache hints of the state loads and stores:
    both decode entry points give the same bits with and without it, and match the
    oracle."""
    B = 4
    W = to_dev(synth.decode_batch(seed=71 + T, B=B, Hk=2, Hv=4, T=T, head_map=synth.TILED))
    Hk, Hv, dk, dv = W["Hk"], W["Hv"], W["dk"], W["dv"]
    QK = Hk * dk
    x = W["x_d"]
    res = []
    for hint in (False, True):
        st, cs_out = W["state_d"].clone(), torch.empty_like(W["conv_state_d"])
        out = ops.decode_layer(x[:, :QK], x[:, QK:2 * QK], x[:, 2 * QK:], st, W["conv_w_d"],
                               W["conv_state_d"], cs_out, Hk=Hk, Hv=Hv, dk=dk, dv=dv,
                               head_map=W["head_map"], batch=B, tokens_per_seq=T, a=W["a_d"],
                               b=W["b_d"], decay_param=W["A_log_d"], dt_bias=W["dt_bias_d"],
                               z=W["z_d"], norm_weight=W["norm_w_d"], stream_state=hint)
        y = ops.conv_update(x, W["conv_w_d"], W["conv_state_d"].clone(), num_seqs=B)
        st2 = W["state_d"].clone()
        out2 = ops.decode_step(y[:, :QK], y[:, QK:2 * QK], y[:, 2 * QK:], st2, Hk=Hk, Hv=Hv,
                               dk=dk, dv=dv, head_map=W["head_map"], batch=B,
                               tokens_per_seq=T, a=W["a_d"], b=W["b_d"],
                               decay_param=W["A_log_d"], dt_bias=W["dt_bias_d"], z=W["z_d"],
                               norm_weight=W["norm_w_d"], stream_state=hint)
        res.append((out, st, cs_out, out2, st2))
    torch.cuda.synchronize()
    for plain, hinted in zip(*res):
        assert torch.equal(plain, hinted)
    y, cs, S = oracle_layer(W, B=B, T=T)
    assert maxabs(f64(res[1][0]).reshape(y.shape), y) <= TOL
    assert maxabs(f64(res[1][1]), S) <= TOL
    assert maxabs(f64(res[1][2]), cs) == 0.0


# ------------------------------------------------------------------ the ferrox-core device-step shapes

@pytest.mark.parametrize("head_map", [synth.TILED, synth.GROUPED])
def test_fused_layer_device_step_shapes_4_48_128(head_map):
    """The ferrox-core device-step shapes (4, 48, 128) through the one-launch layer.
    The layer convolves its inputs first, so the LCG draws are its pre-conv rows,
    and the taps (scale 0.5) and the window (scale 1) continue the same stream. No
    L2 norm, given gates, the core output; the oracle runs its conv, the split and
    the core in turn."""
    from test_gpu_decode import within_device_step_bound
    import oracle
    n_k, n_v, s = 4, 48, 128
    W = synth.device_step(n_k, n_v, s)
    QK, QKV = n_k * s, 2 * n_k * s + n_v * s
    x = torch.cat([W["q"].reshape(1, -1), W["k"].reshape(1, -1), W["v"].reshape(1, -1)], 1)
    conv_w = torch.from_numpy(W["rng"].draw(QKV * 4, 0.5).reshape(QKV, 4))
    window = torch.from_numpy(W["rng"].draw(QKV * 3, 1.0).reshape(1, QKV, 3))
    xd = x.to(DEV).contiguous()
    state = W["state"].unsqueeze(0).to(DEV).contiguous()
    cs_in, cs_out = window.to(DEV), torch.empty_like(window, device=DEV)
    out = ops.decode_layer(xd[:, :QK], xd[:, QK:2 * QK], xd[:, 2 * QK:], state, conv_w.to(DEV),
                           cs_in, cs_out, Hk=n_k, Hv=n_v, dk=s, dv=s, head_map=head_map, batch=1,
                           g=W["g"].to(DEV), beta=W["beta"].to(DEV), l2norm_qk=False)
    torch.cuda.synchronize()
    ycv, cs = oracle.conv(f64(x), f64(conv_w), f64(window[0]))
    q = ycv[:, :QK].reshape(1, n_k, s)
    k = ycv[:, QK:2 * QK].reshape(1, n_k, s)
    v = ycv[:, 2 * QK:].reshape(1, n_v, s)
    y, S = oracle.core(q, k, v, f64(W["state"]), head_map, g=f64(W["g"]), beta=f64(W["beta"]),
                       l2norm_qk=False)
    o = f64(out).reshape(y.shape)
    assert maxabs(o, y) <= TOL and maxabs(f64(state[0]), S) <= TOL
    assert within_device_step_bound(o, y) and within_device_step_bound(f64(state[0]), S)
    assert maxabs(f64(cs_out[0]), cs) == 0.0


# ------------------------------------------------------------------ slot pools across calls

def test_pool_slot_sits_out_a_step_and_rejoins():
    """Three pooled sequences over three steps with alternating conv buffers; slot 1
    sits out the middle step. The caller carries that slot's window into the buffer
    the next call reads (the contract gdn.h states for pools), and every output,
    state and window then matches the oracle run per sequence. Without the carry
    the buffer would hold the slot's stale window, which the test also shows."""
    Hk, Hv, d, nslots = 2, 4, 64, 3
    W = to_dev(synth.decode_batch(seed=71, B=nslots, Hk=Hk, Hv=Hv, dk=d, dv=d))
    pool, bufs = W["state_d"], [W["conv_state_d"].clone(), torch.zeros_like(W["conv_state_d"])]
    S_ref = {s: f64(W["state"][s:s + 1]) for s in range(nslots)}
    cs_ref = {s: f64(W["conv_state"][s:s + 1]) for s in range(nslots)}
    schedule = [[0, 1, 2], [2, 0], [1, 0, 2]]
    par = 0
    for step, slots in enumerate(schedule):
        Ws = synth.decode_batch(seed=700 + step, B=len(slots), Hk=Hk, Hv=Hv, dk=d, dv=d)
        Ws = to_dev(dict(Ws, conv_w=W["conv_w"], A_log=W["A_log"]))
        cs_in, cs_out = bufs[par], bufs[1 - par]
        out = run_fused(Ws, T=1, B=len(slots), cs_in=cs_in, cs_out=cs_out, state=pool,
                        slots=torch.tensor(slots, dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        for bi, s in enumerate(slots):
            Wi = dict(Ws)
            for key in ("x", "z", "a", "b"):
                Wi[key] = Ws[key][bi:bi + 1]
            y, cs_ref[s], S_ref[s] = oracle_layer(Wi, B=1, T=1, state=S_ref[s],
                                                 conv_state=cs_ref[s])
            assert maxabs(f64(out[bi:bi + 1]).reshape(y.shape), y) <= TOL, f"step {step} slot {s}"
        left_out = [s for s in range(nslots) if s not in slots]
        for s in left_out:
            # the slot's latest window is in the buffer this call read; the one the
            # next call reads holds an older one until the caller carries it over
            assert not torch.equal(cs_out[s], cs_in[s])
            cs_out[s].copy_(cs_in[s])
        par = 1 - par
    torch.cuda.synchronize()
    for s in range(nslots):
        assert maxabs(f64(pool[s]), S_ref[s][0]) <= TOL
        assert maxabs(f64(bufs[par][s]), cs_ref[s][0]) == 0.0
