"""GPU parity of gdn_prefill_chunked against the token-by-token CPU oracle.

The chunked prefill reaches the recurrence's result in another summation order,
so its oracle is the sequential recurrence itself. Tolerances (max-abs): 0.012
on outputs and 1e-3 on carried states, the chunk-core diagnostics of the
ferrum-kernels tests page, which this contract adopts.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_linear_step_amd import ops, synth
from helpers import f64, maxabs, oracle_core_heads, ulp16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL_OUT, TOL_STATE = 0.012, 1e-3


def run_prefill(P, *, state=None, out_dtype=torch.float32, raw=True, gated=False, lo=None, hi=None,
                cu=None):
    """Prefill over P's packed tokens [lo, hi) (default: all) with cu_seqlens cu."""
    Hk, Hv, d = P["Hk"], P["Hv"], P["dk"]
    lo = 0 if lo is None else lo
    hi = P["q"].shape[0] if hi is None else hi
    cu = P["cu_seqlens"] if cu is None else cu
    dv = lambda t: t[lo:hi].reshape(hi - lo, -1).to(DEV).contiguous()  # noqa: E731
    kw = {}
    if raw:
        kw.update(a=dv(P["a"]), b=dv(P["b"]), decay_param=P["A_log"].to(DEV),
                  dt_bias=P["dt_bias"].to(DEV))
    else:
        kw.update(g=dv(P["g"]), beta=dv(P["beta"]))
    if gated:
        kw.update(z=P["z"][lo:hi].to(DEV).contiguous(), norm_weight=P["norm_w"].to(DEV))
    st = P["state"].to(DEV).contiguous() if state is None else state
    out = ops.prefill_chunked(dv(P["q"]), dv(P["k"]), dv(P["v"]), st, cu, Hk=Hk, Hv=Hv, dk=d,
                              dv=d, head_map=P["head_map"], out_dtype=out_dtype, **kw)
    return out, st


def oracle_seq(P, i, S0, heads=None, raw=True, gated=False):
    cu = P["cu_seqlens"]
    lo, hi = int(cu[i]), int(cu[i + 1])
    kw = {}
    if raw:
        kw.update(a=f64(P["a"][lo:hi]), b=f64(P["b"][lo:hi]), decay_param=f64(P["A_log"]),
                  dt_bias=f64(P["dt_bias"]))
    else:
        kw.update(g=f64(P["g"][lo:hi]), beta=f64(P["beta"][lo:hi]))
    if gated:
        kw.update(z=f64(P["z"][lo:hi]), norm_w=f64(P["norm_w"]))
    heads = range(P["Hv"]) if heads is None else heads
    return oracle_core_heads(f64(P["q"][lo:hi]), f64(P["k"][lo:hi]), f64(P["v"][lo:hi]), S0,
                             P["head_map"], heads, **kw)


# ------------------------------------------------------------------ the chunk-core workload

def core_workload(T, Hk, Hv, d, head_map):
    W = synth.core_sin(T, Hk, Hv, d, d)
    return dict(Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=head_map, q=W["q"], k=W["k"], v=W["v"],
                g=W["g"], beta=W["beta"], state=W["state"].unsqueeze(0),
                cu_seqlens=synth.cu_seqlens([T]))


@pytest.mark.parametrize("Hk,Hv", [(2, 4), (2, 2)])
@pytest.mark.parametrize("head_map", [synth.GROUPED, synth.TILED])
def test_chunk_core_145_tokens_split_73_with_sentinel(Hk, Hv, head_map):
    T, d, split = 145, 128, 73
    P = core_workload(T, Hk, Hv, d, head_map)
    n = Hv * d * d
    guard = torch.full((n + 16,), 73.25, device=DEV)
    guard[:n] = P["state"].reshape(-1).to(DEV)
    st = guard[:n].view(1, Hv, d, d)
    out, _ = run_prefill(P, state=st, raw=False)
    torch.cuda.synchronize()
    y, S = oracle_seq(P, 0, f64(P["state"][0]), raw=False)
    assert np.any(np.abs(f64(out)) > 1e-4)
    assert maxabs(f64(out), y) <= TOL_OUT
    assert maxabs(f64(st[0]), S) <= TOL_STATE
    assert torch.all(guard[n:] == 73.25)
    # the same tokens in two calls, split at a token that is not chunk-aligned
    g2 = torch.full((n + 16,), 73.25, device=DEV)
    g2[:n] = P["state"].reshape(-1).to(DEV)
    st2 = g2[:n].view(1, Hv, d, d)
    o1, _ = run_prefill(P, state=st2, raw=False, lo=0, hi=split, cu=synth.cu_seqlens([split]))
    assert torch.all(g2[n:] == 73.25)
    o2, _ = run_prefill(P, state=st2, raw=False, lo=split, hi=T,
                        cu=synth.cu_seqlens([T - split]))
    torch.cuda.synchronize()
    assert torch.all(g2[n:] == 73.25)
    assert maxabs(f64(torch.cat([o1, o2])), f64(out)) <= TOL_OUT
    assert maxabs(f64(st2), f64(st)) <= TOL_STATE


# ------------------------------------------------------------------ single long sequence (T=4096)

def test_prefill_t4096_grouped_bf16_matches_oracle():
    P = synth.prefill(seed=3, lengths=[4096], head_map=synth.GROUPED)
    out, st = run_prefill(P)
    torch.cuda.synchronize()
    y, S = oracle_seq(P, 0, f64(P["state"][0]))
    assert maxabs(f64(out), y) <= TOL_OUT
    assert maxabs(f64(st[0]), S) <= TOL_STATE


# ------------------------------------------------------------------ varlen prefill then decode

def test_varlen_prefill_then_64_decode_steps():
    lengths = [512, 1024, 2048, 3072, 4096, 5120, 6144, 8192]
    P = synth.prefill(seed=5, lengths=lengths, head_map=synth.TILED, state_std=0.02)
    Hk, Hv, d = P["Hk"], P["Hv"], P["dk"]
    out, st = run_prefill(P)
    torch.cuda.synchronize()
    heads = [0, 13, 31]  # sampled v-heads, all sequences, every token
    S_ref = {}
    for i in range(len(lengths)):
        lo, hi = int(P["cu_seqlens"][i]), int(P["cu_seqlens"][i + 1])
        y, S = oracle_seq(P, i, f64(P["state"][i]), heads=heads)
        assert maxabs(f64(out[lo:hi, heads]), y[:, heads]) <= TOL_OUT, f"seq {i} out"
        assert maxabs(f64(st[i, heads]), S[heads]) <= TOL_STATE, f"seq {i} state"
        S_ref[i] = S
    # 64 batched decode steps (B=8) with fresh inputs, the state carried on both sides
    for step in range(64):
        D = synth.prefill(seed=5000 + step, lengths=[1] * 8, head_map=synth.TILED)
        o = ops.decode_step(D["q"].reshape(8, -1).to(DEV), D["k"].reshape(8, -1).to(DEV),
                            D["v"].reshape(8, -1).to(DEV), st, Hk=Hk, Hv=Hv, dk=d, dv=d,
                            head_map=synth.TILED, batch=8, a=D["a"].to(DEV), b=D["b"].to(DEV),
                            decay_param=P["A_log"].to(DEV), dt_bias=P["dt_bias"].to(DEV))
        if step in (0, 63):
            torch.cuda.synchronize()
        for i in range(8):
            yo, So = oracle.core(f64(D["q"][i:i + 1]), f64(D["k"][i:i + 1]),
                                 f64(D["v"][i:i + 1]), S_ref[i], synth.TILED,
                                 a=f64(D["a"][i:i + 1]), b=f64(D["b"][i:i + 1]),
                                 decay_param=f64(P["A_log"]), dt_bias=f64(P["dt_bias"]),
                                 heads=(heads[0], heads[-1] + 1))
            S_ref[i] = So
            if step in (0, 63):
                assert maxabs(f64(o[i, heads]), yo[0, heads]) <= TOL_OUT
    for i in range(8):
        assert maxabs(f64(st[i, heads]), S_ref[i][heads]) <= TOL_STATE


# ------------------------------------------------------------------ edges, dtypes, gated norm

@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_one_sequence_chunk_bounds(T):
    """One sequence: its chunk bounds come from the token count alone (no chunk
    table), including a lone partial chunk and an exact multiple of 64."""
    P = synth.prefill(seed=20 + T, lengths=[T], Hk=2, Hv=4, head_map=synth.TILED, state_std=0.05)
    out, st = run_prefill(P)
    torch.cuda.synchronize()
    y, S = oracle_seq(P, 0, f64(P["state"][0]))
    assert maxabs(f64(out), y) <= TOL_OUT
    assert maxabs(f64(st[0]), S) <= TOL_STATE


@pytest.mark.parametrize("head_map", [synth.GROUPED, synth.TILED])
def test_ragged_lengths_including_empty(head_map):
    lengths = [0, 1, 63, 64, 65, 130, 0, 7]
    P = synth.prefill(seed=11, lengths=lengths, Hk=2, Hv=4, head_map=head_map, state_std=0.05)
    out, st = run_prefill(P)
    torch.cuda.synchronize()
    for i, n in enumerate(lengths):
        lo = int(P["cu_seqlens"][i])
        if n == 0:
            assert torch.equal(st[i].cpu(), P["state"][i]), "empty sequence changed its state"
            continue
        y, S = oracle_seq(P, i, f64(P["state"][i]))
        assert maxabs(f64(out[lo:lo + n]), y) <= TOL_OUT
        assert maxabs(f64(st[i]), S) <= TOL_STATE


@pytest.mark.parametrize("gated", [False, True])
def test_many_sequences_four_slice_carry_workgroups(gated):
    """Enough (sequence, head) pairs that the carry packs 4 dv slices per workgroup
    (the split carry's 2-slice workgroups would need more than one round of CUs);
    ragged lengths, empty ones included, every head compared."""
    lengths = [(37 * i) % 150 for i in range(24)]  # 0 .. 148, two empties
    P = synth.prefill(seed=15, lengths=lengths, Hk=2, Hv=4, head_map=synth.TILED,
                      state_std=0.05, with_z=gated)
    assert len(lengths) * 4 * (128 // 32) > 256  # past one round of 2-slice workgroups
    out, st = run_prefill(P, gated=gated)
    torch.cuda.synchronize()
    for i, n in enumerate(lengths):
        lo = int(P["cu_seqlens"][i])
        if n == 0:
            assert torch.equal(st[i].cpu(), P["state"][i]), "empty sequence changed its state"
            continue
        y, S = oracle_seq(P, i, f64(P["state"][i]), gated=gated)
        assert maxabs(f64(out[lo:lo + n]), y) <= TOL_OUT
        assert maxabs(f64(st[i]), S) <= TOL_STATE


@pytest.mark.parametrize("gated", [False, True])
def test_two_slice_split_carry_workgroups(gated):
    """Between 33 and 64 (sequence, head) pairs: the split carry with 2 dv slices
    per workgroup (1-slice workgroups would need two rounds of CUs); ragged
    lengths across several chunks, an empty sequence, every head compared."""
    lengths = [(53 * i + 40) % 300 for i in range(12)]  # 5 .. 270 tokens
    lengths[3] = 192  # whole chunks only
    lengths[5] = 0
    P = synth.prefill(seed=16, lengths=lengths, Hk=2, Hv=4, head_map=synth.GROUPED,
                      state_std=0.05, with_z=gated)
    groups = len(lengths) * 4
    assert groups * (128 // 16) > 256 >= groups * (128 // 32)
    out, st = run_prefill(P, gated=gated)
    torch.cuda.synchronize()
    for i, n in enumerate(lengths):
        lo = int(P["cu_seqlens"][i])
        if n == 0:
            assert torch.equal(st[i].cpu(), P["state"][i]), "empty sequence changed its state"
            continue
        y, S = oracle_seq(P, i, f64(P["state"][i]), gated=gated)
        assert maxabs(f64(out[lo:lo + n]), y) <= TOL_OUT
        assert maxabs(f64(st[i]), S) <= TOL_STATE


def test_more_than_256_sequences():
    """300 short ragged sequences (empty ones included): the chunk table is built in
    blocks of 256 sequences, and past 256 the carry keeps the sequences' order."""
    rng = np.random.default_rng(17)
    lengths = [int(x) for x in rng.choice([0, 1, 5, 63, 64, 65, 100], size=300)]
    P = synth.prefill(seed=17, lengths=lengths, Hk=1, Hv=2, head_map=synth.TILED,
                      state_std=0.05)
    out, st = run_prefill(P)
    torch.cuda.synchronize()
    for i, n in enumerate(lengths):
        lo = int(P["cu_seqlens"][i])
        if n == 0:
            assert torch.equal(st[i].cpu(), P["state"][i]), "empty sequence changed its state"
            continue
        y, S = oracle_seq(P, i, f64(P["state"][i]))
        assert maxabs(f64(out[lo:lo + n]), y) <= TOL_OUT
        assert maxabs(f64(st[i]), S) <= TOL_STATE


@pytest.mark.parametrize("act", [torch.float32, torch.float16])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("lengths", [[100, 37], [137]])  # [137]: the one-sequence path
def test_prefill_dtypes_and_gated_norm(act, out_dtype, lengths):
    P = synth.prefill(seed=12, lengths=lengths, Hk=2, Hv=4, head_map=synth.GROUPED, dtype=act,
                      state_std=0.02, with_z=True)
    out, st = run_prefill(P, out_dtype=out_dtype, gated=True)
    torch.cuda.synchronize()
    for i, n in enumerate(lengths):
        lo = int(P["cu_seqlens"][i])
        y, S = oracle_seq(P, i, f64(P["state"][i]), gated=True)
        o = f64(out[lo:lo + n])
        bound = TOL_OUT if out_dtype == torch.float32 else ulp16(y, out_dtype) + TOL_OUT
        assert np.all(np.abs(o - y) <= bound)
        assert maxabs(f64(st[i]), S) <= TOL_STATE


def test_prefill_is_deterministic():
    P = synth.prefill(seed=13, lengths=[300, 77], Hk=2, Hv=4, head_map=synth.TILED,
                      state_std=0.02)
    o1, s1 = run_prefill(P)
    o2, s2 = run_prefill(P)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_prefill_bad_offsets_leave_state_untouched():
    P = synth.prefill(seed=14, lengths=[10, 20], Hk=2, Hv=4, head_map=synth.TILED,
                      state_std=0.02)
    st = P["state"].to(DEV)
    before = st.clone()
    bad = torch.tensor([0, 25, 20], dtype=torch.int32)  # not monotone
    with pytest.raises(ops.GdnError) as e:
        run_prefill(P, state=st, cu=bad)
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert torch.equal(st, before)
