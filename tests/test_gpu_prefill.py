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
from helpers import f64, maxabs, oracle_core_heads, threads, ulp16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL_OUT, TOL_STATE = 0.012, 1e-3
TOL_DECODE = 1e-3  # decode outputs and states


def run_prefill(P, *, state=None, out_dtype=torch.float32, raw=True, gated=False, lo=None, hi=None,
                cu=None, decay=ops.DECAY_LOG_RATE, l2norm_qk=True):
    """Prefill over P's packed tokens [lo, hi) (default: all) with cu_seqlens cu."""
    Hk, Hv, dk, dv_ = P["Hk"], P["Hv"], P["dk"], P["dv"]
    lo = 0 if lo is None else lo
    hi = P["q"].shape[0] if hi is None else hi
    cu = P["cu_seqlens"] if cu is None else cu
    dv = lambda t: t[lo:hi].reshape(hi - lo, -1).to(DEV).contiguous()  # noqa: E731
    kw = {}
    if raw:
        kw.update(a=dv(P["a"]), b=dv(P["b"]), decay_param=P["A_log"].to(DEV),
                  dt_bias=P["dt_bias"].to(DEV), decay=decay)
    else:
        kw.update(g=dv(P["g"]), beta=dv(P["beta"]))
    if gated:
        kw.update(z=P["z"][lo:hi].to(DEV).contiguous(), norm_weight=P["norm_w"].to(DEV))
    st = P["state"].to(DEV).contiguous() if state is None else state
    out = ops.prefill_chunked(dv(P["q"]), dv(P["k"]), dv(P["v"]), st, cu, Hk=Hk, Hv=Hv, dk=dk,
                              dv=dv_, head_map=P["head_map"], out_dtype=out_dtype,
                              l2norm_qk=l2norm_qk, **kw)
    return out, st


def oracle_seq(P, i, S0, heads=None, raw=True, gated=False, decay=ops.DECAY_LOG_RATE,
               l2norm_qk=True):
    cu = P["cu_seqlens"]
    lo, hi = int(cu[i]), int(cu[i + 1])
    kw = dict(l2norm_qk=l2norm_qk)
    if raw:
        kw.update(a=f64(P["a"][lo:hi]), b=f64(P["b"][lo:hi]), decay_param=f64(P["A_log"]),
                  dt_bias=f64(P["dt_bias"]), decay_kind=decay)
    else:
        kw.update(g=f64(P["g"][lo:hi]), beta=f64(P["beta"][lo:hi]))
    if gated:
        kw.update(z=f64(P["z"][lo:hi]), norm_w=f64(P["norm_w"]))
    heads = range(P["Hv"]) if heads is None else heads
    return oracle_core_heads(f64(P["q"][lo:hi]), f64(P["k"][lo:hi]), f64(P["v"][lo:hi]), S0,
                             P["head_map"], heads, **kw)


def split_with_sentinel(P, split, **kw):
    """The whole sequence in one call and in two calls split at a token that is not
    chunk-aligned, each on a state with sentinels on both sides. Returns the two
    outputs and the two final states; asserts that no sentinel moved."""
    T = P["q"].shape[0]
    Hv, dv, dk = P["Hv"], P["dv"], P["dk"]
    n = Hv * dv * dk
    states = []
    for _ in range(2):
        guard = torch.full((n + 32,), 73.25, device=DEV)
        guard[16:16 + n] = P["state"].reshape(-1).to(DEV)
        states.append((guard, guard[16:16 + n].view(1, Hv, dv, dk)))
    out, _ = run_prefill(P, state=states[0][1], **kw)
    o1, _ = run_prefill(P, state=states[1][1], lo=0, hi=split, cu=synth.cu_seqlens([split]), **kw)
    o2, _ = run_prefill(P, state=states[1][1], lo=split, hi=T, cu=synth.cu_seqlens([T - split]),
                        **kw)
    torch.cuda.synchronize()
    for guard, _ in states:
        assert torch.all(guard[:16] == 73.25) and torch.all(guard[16 + n:] == 73.25)
    return out, torch.cat([o1, o2]), states[0][1], states[1][1]


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


# ------------------------------------------------------------------ decay and normalisation variants

@pytest.mark.parametrize("head_map", [synth.GROUPED, synth.TILED])
def test_negative_rate_decay_145_tokens_split_73_with_sentinel(head_map):
    """GDN_DECAY_NEGATIVE_RATE through the prefill: the rate multiplying softplus is
    passed as is (the ferrum-kernels tests page's NegativeRate parameterisation)."""
    P = synth.prefill(seed=41, lengths=[145], Hk=2, Hv=4, head_map=head_map, state_std=0.05)
    P["A_log"] = synth.negative_rates(41, P["Hv"])  # the decay parameter, here a rate
    dec = ops.DECAY_NEGATIVE_RATE
    out, out_split, st, st_split = split_with_sentinel(P, 73, decay=dec)
    y, S = oracle_seq(P, 0, f64(P["state"][0]), decay=dec)
    assert np.any(np.abs(f64(out)) > 1e-3)
    assert maxabs(f64(out), y) <= TOL_OUT and maxabs(f64(out_split), y) <= TOL_OUT
    assert maxabs(f64(st[0]), S) <= TOL_STATE and maxabs(f64(st_split[0]), S) <= TOL_STATE
    # the same rates given as A_log = log(-rate) under the log-rate form agree
    yl, Sl = oracle_seq(dict(P, A_log=torch.log(-P["A_log"].double())), 0, f64(P["state"][0]))
    assert maxabs(yl, y) <= 1e-9 and maxabs(Sl, S) <= 1e-9


@pytest.mark.parametrize("head_map", [synth.GROUPED, synth.TILED])
def test_unnormalised_qk_145_tokens_split_73_with_sentinel(head_map):
    """No in-op L2 norm: the ferrox-core generator's un-normalised uniform q and k
    (scaled so |k|^2 stays near 1 and the rule is stable), given g and beta."""
    P = synth.lcg_prefill(T=145, Hk=2, Hv=4, dk=128, dv=128)
    P["head_map"] = head_map
    out, out_split, st, st_split = split_with_sentinel(P, 73, raw=False, l2norm_qk=False)
    y, S = oracle_seq(P, 0, f64(P["state"][0]), raw=False, l2norm_qk=False)
    assert np.any(np.abs(f64(out)) > 1e-2)
    assert maxabs(f64(out), y) <= TOL_OUT and maxabs(f64(out_split), y) <= TOL_OUT
    assert maxabs(f64(st[0]), S) <= TOL_STATE and maxabs(f64(st_split[0]), S) <= TOL_STATE


@pytest.mark.parametrize("nseq,Hv", [(1, 2), (12, 4), (24, 4)])
def test_zero_beta_decays_the_state_by_the_summed_gates(nseq, Hv):
    """beta = 0 writes nothing, so after T tokens of weak decay the state is exactly
    exp(sum g) S0 and o_t = scale exp(G_t) S0 q_t (closed forms of the rule). The
    state check is tight (1e-5 on |S0| <= 0.5): a decay factor taken from the
    wrong token of a chunk is off by several percent. Sequence and head counts
    select the three carry shapes (one-slice split, two-slice split, four-slice)."""
    lengths = [200 - 7 * i for i in range(nseq)]  # 3 full chunks + a partial one, ragged
    T, Hk, d = sum(lengths), 1, 128
    r = synth.Lcg(91)
    P = dict(Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=synth.TILED, cu_seqlens=synth.cu_seqlens(lengths),
             state=torch.from_numpy(r.draw(nseq * Hv * d * d, 0.5).reshape(nseq, Hv, d, d)),
             q=torch.from_numpy(r.draw(T * Hk * d, 1.0).reshape(T, Hk, d)),
             k=torch.from_numpy(r.draw(T * Hk * d, 1.0).reshape(T, Hk, d)),
             v=torch.from_numpy(r.draw(T * Hv * d, 1.0).reshape(T, Hv, d)),
             g=torch.from_numpy((np.float32(-0.05) * np.abs(r.draw(T * Hv, 1.0))).reshape(T, Hv)),
             beta=torch.zeros(T, Hv))
    groups = nseq * Hv
    info = ops.prefill_launch_info(lengths, Hk=Hk, Hv=Hv, dk=d, dv=d, compute_units=256,
                                   head_map=synth.TILED, flags=ops.L2NORM_QK)
    assert (info["carry_kind"], info["slices_per_workgroup"]) == \
        ((0, 1) if groups <= 32 else (0, 2) if groups <= 64 else (1, 4))
    out, st = run_prefill(P, raw=False)
    torch.cuda.synchronize()
    cu = P["cu_seqlens"].tolist()
    g = f64(P["g"])
    qn = f64(P["q"]) / np.linalg.norm(f64(P["q"]), axis=-1, keepdims=True)
    for i in range(nseq):
        G = np.cumsum(g[cu[i]:cu[i + 1]], axis=0)  # [t][h]
        S0 = f64(P["state"][i])
        S_exact = np.exp(G[-1])[:, None, None] * S0
        assert np.max(np.abs(f64(st[i]) - S_exact)) <= 1e-5, f"seq {i} state"
        o_exact = np.exp(G)[:, :, None] * np.einsum("hji,ti->thj", S0, qn[cu[i]:cu[i + 1], 0]) / \
            np.sqrt(d)
        assert maxabs(f64(out[cu[i]:cu[i + 1]]), o_exact) <= TOL_OUT, f"seq {i} out"


def test_int64_cu_seqlens_through_the_binding():
    """A torch int64 cu_seqlens (torch's default integer type) reaches the kernels as
    the int32 [N+1] array they read, on the device as on the host."""
    lengths = [70, 0, 129]
    P = synth.prefill(seed=42, lengths=lengths, Hk=2, Hv=4, head_map=synth.TILED, state_std=0.05)
    cu64 = P["cu_seqlens"].to(torch.int64)
    o_dev, s_dev = run_prefill(P, cu=cu64.to(DEV))
    o_host, s_host = run_prefill(P, cu=cu64)
    o_ref, s_ref = run_prefill(P)
    torch.cuda.synchronize()
    assert torch.equal(o_dev, o_ref) and torch.equal(s_dev, s_ref)
    assert torch.equal(o_host, o_ref) and torch.equal(s_host, s_ref)
    y, S = oracle.packed(f64(P["q"]), f64(P["k"]), f64(P["v"]), f64(P["state"]), P["head_map"],
                         P["cu_seqlens"], a=f64(P["a"]), b=f64(P["b"]),
                         decay_param=f64(P["A_log"]), dt_bias=f64(P["dt_bias"]), nthreads=4)
    assert maxabs(f64(o_ref), y) <= TOL_OUT and maxabs(f64(s_ref), S) <= TOL_STATE


def test_binding_rejects_misshaped_buffers_before_any_launch():
    P = synth.prefill(seed=43, lengths=[10, 20], Hk=2, Hv=4, head_map=synth.TILED,
                      state_std=0.02)
    st = P["state"].to(DEV)
    before = st.clone()
    with pytest.raises(ValueError):  # state of another head shape
        run_prefill(P, state=st.view(2, 4, 64, 256))
    with pytest.raises(ValueError):  # fewer state slots than sequences
        run_prefill(P, state=st[:1].contiguous())
    with pytest.raises(TypeError):  # offsets as floats
        run_prefill(P, state=st, cu=P["cu_seqlens"].float())
    with pytest.raises(ValueError):  # an output too small for the tokens
        ops.prefill_chunked(*(P[x][:30].reshape(30, -1).to(DEV) for x in ("q", "k", "v")), st,
                            P["cu_seqlens"], Hk=2, Hv=4, dk=128, dv=128, head_map=synth.TILED,
                            g=torch.zeros(30, 4, device=DEV), beta=torch.zeros(30, 4, device=DEV),
                            out=torch.empty(29, 4, 128, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(st, before)


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
    """The packed eight-sequence prefill (512..8192 tokens, tiled, nonzero initial
    states), then 64 batched decode steps with fresh inputs. Every output of every
    v-head and every final state is compared with the token-by-token oracle:
    (A) the whole pipeline at the prefill tolerances, the GPU's state carried from
    the prefill into the decode; (B) the decode steps from the oracle's own
    post-prefill state (rounded to f32) at the decode tolerances."""
    lengths = [512, 1024, 2048, 3072, 4096, 5120, 6144, 8192]
    P = synth.prefill(seed=5, lengths=lengths, head_map=synth.TILED, state_std=0.02)
    Hk, Hv, d = P["Hk"], P["Hv"], P["dk"]
    out, st = run_prefill(P)
    torch.cuda.synchronize()
    y, S = oracle.packed(f64(P["q"]), f64(P["k"]), f64(P["v"]), f64(P["state"]), synth.TILED,
                         P["cu_seqlens"], a=f64(P["a"]), b=f64(P["b"]),
                         decay_param=f64(P["A_log"]), dt_bias=f64(P["dt_bias"]),
                         nthreads=threads())
    for i in range(len(lengths)):
        lo, hi = int(P["cu_seqlens"][i]), int(P["cu_seqlens"][i + 1])
        assert maxabs(f64(out[lo:hi]), y[lo:hi]) <= TOL_OUT, f"seq {i} out"
        assert maxabs(f64(st[i]), S[i]) <= TOL_STATE, f"seq {i} state"
    stB = torch.from_numpy(S).float().to(DEV)  # (B): the oracle's state, in f32
    S_A, S_B = S, f64(stB)
    common = dict(Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=synth.TILED, batch=8,
                  decay_param=P["A_log"].to(DEV), dt_bias=P["dt_bias"].to(DEV))
    for step in range(64):
        D = synth.prefill(seed=5000 + step, lengths=[1] * 8, head_map=synth.TILED)
        args = [D[x].reshape(8, -1).to(DEV) for x in ("q", "k", "v")]
        gates = dict(a=D["a"].to(DEV), b=D["b"].to(DEV))
        oA = ops.decode_step(*args, st, **common, **gates)
        oB = ops.decode_step(*args, stB, **common, **gates)
        torch.cuda.synchronize()
        kw = dict(a=f64(D["a"]), b=f64(D["b"]), decay_param=f64(P["A_log"]),
                  dt_bias=f64(P["dt_bias"]), nthreads=8)
        cu1 = np.arange(9)
        yA, S_A = oracle.packed(f64(D["q"]), f64(D["k"]), f64(D["v"]), S_A, synth.TILED, cu1, **kw)
        yB, S_B = oracle.packed(f64(D["q"]), f64(D["k"]), f64(D["v"]), S_B, synth.TILED, cu1, **kw)
        assert maxabs(f64(oA), yA) <= TOL_OUT, f"step {step} (A)"
        assert maxabs(f64(oB), yB) <= TOL_DECODE, f"step {step} (B)"
    assert maxabs(f64(st), S_A) <= TOL_STATE
    assert maxabs(f64(stB), S_B) <= TOL_DECODE


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


# ------------------------------------------------------------------ other head shapes (the f32 path)

OTHER_SHAPES = [(32, 32), (64, 64), (96, 96), (64, 128), (128, 64), (128, 256), (256, 128),
                (256, 256)]


@pytest.mark.parametrize("Hk,Hv", [(2, 4), (2, 2)])
@pytest.mark.parametrize("head_map", [synth.GROUPED, synth.TILED])
def test_page_chunk_core_d32_145_tokens_split_73_with_sentinel(Hk, Hv, head_map):
    """The ferrum-kernels page's own chunked-core shape, (Hk, Hv, dk, dv) = (2, 4, 32,
    32) (and (2, 2, 32, 32)), on that test's sin-pattern inputs: T = 145 against the
    token-by-token oracle, and split at token 73 (not chunk-aligned) across two
    calls, with sentinels around the state
    (`chunked_c64_matches_recurrent_oracle_and_non_aligned_state_continuity`)."""
    P = core_workload(145, Hk, Hv, 32, head_map)
    out, out_split, st, st_split = split_with_sentinel(P, 73, raw=False)
    y, S = oracle_seq(P, 0, f64(P["state"][0]), raw=False)
    assert np.any(np.abs(f64(out)) > 1e-4)
    assert maxabs(f64(out), y) <= TOL_OUT and maxabs(f64(out_split), y) <= TOL_OUT
    assert maxabs(f64(st[0]), S) <= TOL_STATE and maxabs(f64(st_split[0]), S) <= TOL_STATE
    assert maxabs(f64(st_split), f64(st)) <= TOL_STATE


@pytest.mark.parametrize("dk,dv", OTHER_SHAPES)
@pytest.mark.parametrize("head_map", [synth.GROUPED, synth.TILED])
def test_other_head_shapes_ragged_varlen(dk, dv, head_map):
    """Ragged packed sequences (an empty one, a single token, lengths around the 32-
    and 64-token chunk edges) with nonzero initial states, raw gates and bf16 N(0,1)
    inputs, every head and state compared with the oracle."""
    lengths = [0, 1, 31, 33, 64, 65, 150]
    P = synth.prefill(seed=60 + dk + dv, lengths=lengths, Hk=2, Hv=4, dk=dk, dv=dv,
                      head_map=head_map, state_std=0.05)
    out, st = run_prefill(P)
    torch.cuda.synchronize()
    y, S = oracle.packed(f64(P["q"]), f64(P["k"]), f64(P["v"]), f64(P["state"]), head_map,
                         P["cu_seqlens"], a=f64(P["a"]), b=f64(P["b"]),
                         decay_param=f64(P["A_log"]), dt_bias=f64(P["dt_bias"]),
                         nthreads=threads())
    assert torch.equal(st[0].cpu(), P["state"][0]), "empty sequence changed its state"
    assert maxabs(f64(out), y) <= TOL_OUT
    assert maxabs(f64(st), S) <= TOL_STATE


@pytest.mark.parametrize("dk,dv", [(32, 32), (96, 96), (256, 128)])
@pytest.mark.parametrize("act", [torch.float32, torch.float16])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_other_head_shapes_dtypes_and_gated_norm(dk, dv, act, out_dtype):
    lengths = [100, 37]
    P = synth.prefill(seed=70 + dk, lengths=lengths, Hk=2, Hv=4, dk=dk, dv=dv,
                      head_map=synth.GROUPED, dtype=act, state_std=0.02, with_z=True)
    out, st = run_prefill(P, out_dtype=out_dtype, gated=True)
    torch.cuda.synchronize()
    y, S = oracle.packed(f64(P["q"]), f64(P["k"]), f64(P["v"]), f64(P["state"]), synth.GROUPED,
                         P["cu_seqlens"], a=f64(P["a"]), b=f64(P["b"]),
                         decay_param=f64(P["A_log"]), dt_bias=f64(P["dt_bias"]), z=f64(P["z"]),
                         norm_w=f64(P["norm_w"]), nthreads=threads())
    bound = TOL_OUT if out_dtype == torch.float32 else ulp16(y, out_dtype) + TOL_OUT
    assert np.all(np.abs(f64(out) - y) <= bound)
    assert maxabs(f64(st), S) <= TOL_STATE


@pytest.mark.parametrize("dk,dv", [(64, 64), (256, 256)])
def test_other_head_shapes_negative_rate_and_unnormalised(dk, dv):
    """NegativeRate decay with the in-op L2 norm, then un-normalised LCG inputs with
    given gates and weak decay (the regime where the carried state matters most)."""
    P = synth.prefill(seed=75, lengths=[145], Hk=2, Hv=4, dk=dk, dv=dv, head_map=synth.TILED,
                      state_std=0.05)
    P["A_log"] = synth.negative_rates(75, 4)
    dec = ops.DECAY_NEGATIVE_RATE
    out, out_split, st, st_split = split_with_sentinel(P, 73, decay=dec)
    y, S = oracle_seq(P, 0, f64(P["state"][0]), decay=dec)
    assert maxabs(f64(out), y) <= TOL_OUT and maxabs(f64(out_split), y) <= TOL_OUT
    assert maxabs(f64(st[0]), S) <= TOL_STATE and maxabs(f64(st_split[0]), S) <= TOL_STATE
    L = synth.lcg_prefill(T=145, Hk=2, Hv=4, dk=dk, dv=dv, qk_scale=0.15 * (128 / dk) ** 0.5)
    L["head_map"] = synth.GROUPED
    out, out_split, st, st_split = split_with_sentinel(L, 73, raw=False, l2norm_qk=False)
    y, S = oracle_seq(L, 0, f64(L["state"][0]), raw=False, l2norm_qk=False)
    assert maxabs(f64(out), y) <= TOL_OUT and maxabs(f64(out_split), y) <= TOL_OUT
    assert maxabs(f64(st[0]), S) <= TOL_STATE and maxabs(f64(st_split[0]), S) <= TOL_STATE


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (256, 128)])
def test_other_head_shapes_long_sequence(dk, dv):
    """T = 2048 (32 chunks; 64 of 32 tokens at dk = 256) at the config-3 statistics
    (bf16 N(0,1), zero state)."""
    P = synth.prefill(seed=77, lengths=[2048], Hk=4, Hv=8, dk=dk, dv=dv, head_map=synth.GROUPED)
    out, st = run_prefill(P)
    torch.cuda.synchronize()
    y, S = oracle.packed(f64(P["q"]), f64(P["k"]), f64(P["v"]), f64(P["state"]), synth.GROUPED,
                         P["cu_seqlens"], a=f64(P["a"]), b=f64(P["b"]),
                         decay_param=f64(P["A_log"]), dt_bias=f64(P["dt_bias"]),
                         nthreads=threads())
    assert maxabs(f64(out), y) <= TOL_OUT and maxabs(f64(st), S) <= TOL_STATE


@pytest.mark.parametrize("n_seqs", [300, 1100])
def test_other_head_shapes_many_short_sequences(n_seqs):
    """Hundreds of short sequences (0-5 tokens, empty ones included) through the f32
    path: the carry takes up to 1024 sequences longest first and more in their
    packed order, the chunk table spans several plan passes; every head, output and
    state against the oracle."""
    rng = np.random.default_rng(n_seqs)
    lengths = [int(x) for x in rng.integers(0, 6, size=n_seqs)]
    P = synth.prefill(seed=80, lengths=lengths, Hk=1, Hv=2, dk=32, dv=32, head_map=synth.GROUPED,
                      state_std=0.05)
    out, st = run_prefill(P)
    torch.cuda.synchronize()
    y, S = oracle.packed(f64(P["q"]), f64(P["k"]), f64(P["v"]), f64(P["state"]), synth.GROUPED,
                         P["cu_seqlens"], a=f64(P["a"]), b=f64(P["b"]),
                         decay_param=f64(P["A_log"]), dt_bias=f64(P["dt_bias"]),
                         nthreads=threads())
    empty = [i for i, n in enumerate(lengths) if n == 0]
    assert empty and torch.equal(st[empty].cpu(), P["state"][empty])
    assert maxabs(f64(out), y) <= TOL_OUT
    assert maxabs(f64(st), S) <= TOL_STATE
