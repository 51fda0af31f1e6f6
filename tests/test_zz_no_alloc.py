"""GPU check of gdn_prefill_chunked_noalloc, the no-allocation prefill entry point,
against gdn_prefill_chunked on the same inputs.

Both run the same kernels; the no-allocation call takes its workspace from the
library's static per-GPU scratch instead of a caller buffer, so the two must agree
bit for bit. Two calls in a row, the second smaller than the first, show that the
second call does not depend on what the first one left in the shared scratch.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_step_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def inputs(P, gated):
    T = P["q"].shape[0]
    d = lambda t: t.reshape(T, -1).to(DEV).contiguous()  # noqa: E731
    kw = dict(a=d(P["a"]), b=d(P["b"]), decay_param=P["A_log"].to(DEV),
              dt_bias=P["dt_bias"].to(DEV))
    if gated:
        kw.update(z=P["z"].to(DEV).contiguous(), norm_weight=P["norm_w"].to(DEV))
    return (d(P["q"]), d(P["k"]), d(P["v"])), kw


def both(P, gated, out_dtype):
    (q, k, v), kw = inputs(P, gated)
    cu_h = P["cu_seqlens"].to(torch.int32).contiguous()
    cu_d = cu_h.to(DEV)
    T = int(cu_h[-1])
    dims = dict(Hk=P["Hk"], Hv=P["Hv"], dk=P["dk"], dv=P["dv"], head_map=P["head_map"])
    st_ref = P["state"].to(DEV).contiguous()
    o_ref = ops.prefill_chunked(q, k, v, st_ref, cu_d, cu_seqlens_host=cu_h, out_dtype=out_dtype,
                                **dims, **kw)
    st = P["state"].to(DEV).contiguous()
    out = torch.full((T, P["Hv"], P["dv"]), 7.0, dtype=out_dtype, device=DEV)
    ops.prefill_chunked_noalloc(q, k, v, st, cu_d, out, cu_seqlens_host=cu_h, **dims, **kw)
    torch.cuda.synchronize()
    return o_ref, st_ref, out, st


def test_noalloc_prefill_matches_the_workspace_entry_point_two_calls():
    # first call: three ragged sequences with the gated norm (the larger workspace)
    P1 = synth.prefill(seed=81, lengths=[150, 64, 229], Hk=2, Hv=4, head_map=synth.TILED,
                       state_std=0.05, with_z=True)
    o_ref, st_ref, out, st = both(P1, gated=True, out_dtype=torch.float32)
    assert torch.equal(out, o_ref) and torch.equal(st, st_ref)
    # second call, smaller: one 70-token sequence, no norm, bf16 out; the scratch
    # still holds the first call's contents
    P2 = synth.prefill(seed=82, lengths=[70], Hk=2, Hv=4, head_map=synth.GROUPED,
                       state_std=0.05)
    o_ref, st_ref, out, st = both(P2, gated=False, out_dtype=torch.bfloat16)
    assert torch.equal(out, o_ref) and torch.equal(st, st_ref)
    assert np.any(np.abs(out.float().cpu().numpy()) > 1e-3)


@pytest.mark.parametrize("dk,dv", [(32, 32), (256, 128)])
def test_noalloc_prefill_other_head_shapes_two_calls(dk, dv):
    """The f32 path (its own workspace layout, 32-token chunks at dk = 256): the
    same two calls in a row, bit for bit against the workspace entry point."""
    P1 = synth.prefill(seed=84, lengths=[150, 0, 97], Hk=2, Hv=4, dk=dk, dv=dv,
                       head_map=synth.TILED, state_std=0.05, with_z=True)
    o_ref, st_ref, out, st = both(P1, gated=True, out_dtype=torch.float32)
    assert torch.equal(out, o_ref) and torch.equal(st, st_ref)
    P2 = synth.prefill(seed=85, lengths=[45], Hk=2, Hv=4, dk=dk, dv=dv, head_map=synth.GROUPED,
                       state_std=0.05)
    o_ref, st_ref, out, st = both(P2, gated=False, out_dtype=torch.bfloat16)
    assert torch.equal(out, o_ref) and torch.equal(st, st_ref)
    assert np.any(np.abs(out.float().cpu().numpy()) > 1e-3)


def test_noalloc_prefill_refuses_more_than_its_scratch():
    P = synth.prefill(seed=83, lengths=[4096], Hk=16, Hv=32, head_map=synth.GROUPED)
    need = ops.prefill_workspace_bytes(Hk=16, Hv=32, dk=128, dv=128, num_seqs=1, total_tokens=4096)
    assert need > ops.NOALLOC_SCRATCH_BYTES
    (q, k, v), kw = inputs(P, gated=False)
    st = P["state"].to(DEV).contiguous()
    out = torch.full((4096, 32, 128), 7.0, device=DEV)
    cu_h = P["cu_seqlens"]
    with pytest.raises(ops.GdnError) as e:
        ops.prefill_chunked_noalloc(q, k, v, st, cu_h.to(DEV), out, cu_seqlens_host=cu_h, Hk=16,
                                    Hv=32, dk=128, dv=128, head_map=synth.GROUPED, **kw)
    assert e.value.status == 8  # GDN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(st == 0)
