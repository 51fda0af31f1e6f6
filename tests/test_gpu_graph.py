"""gdn_decode_layer launches captured in a HIP graph (the 48-layer token step
of the deep-model workload) replay exactly what eager launches compute.

Every replay is checked against eager results, with eager work and
synchronizations between replays; the comparison is bitwise (the same kernels
on the same inputs in the same order).
"""
import pytest
import torch

from gated_deltanet_linear_step_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def make_layers(n, B, Hk, Hv, d, stream=None):
    QK = Hk * d
    Ls = []
    for layer in range(n):
        W = synth.decode_batch(seed=4 * 1000 + layer, B=B, Hk=Hk, Hv=Hv, dk=d, dv=d,
                               head_map=synth.TILED)
        S = {k: (v.to(DEV).contiguous() if hasattr(v, "to") else v) for k, v in W.items()}
        S["state0"], S["cs0"] = S["state"].clone(), S["conv_state"].clone()
        S["cb"] = torch.zeros_like(S["conv_state"])
        S["out"] = torch.zeros((B, Hv, d), dtype=torch.float32, device=DEV)
        x = S["x"]
        kw = dict(Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=synth.TILED, batch=B, a=S["a"], b=S["b"],
                  decay_param=S["A_log"], dt_bias=S["dt_bias"], z=S["z"], norm_weight=S["norm_w"])
        S["calls"] = [ops.prepare_decode_layer(x[:, :QK], x[:, QK:2 * QK], x[:, 2 * QK:],
                                               S["state"], S["conv_w"], ci, co, S["out"],
                                               stream=stream, **kw)
                      for ci, co in ((S["conv_state"], S["cb"]), (S["cb"], S["conv_state"]))]
        Ls.append(S)
    return Ls


def token(Ls, par):
    for S in Ls:
        S["calls"][par].launch()


def snapshot(Ls):
    return [(S["state"].clone(), S["conv_state"].clone(), S["out"].clone()) for S in Ls]


def test_graph_replays_match_eager_steps():
    n, B, Hk, Hv, d = 3, 2, 2, 4, 128
    eager = make_layers(n, B, Hk, Hv, d)
    refs = []
    for step in range(6):
        token(eager, step & 1)
        if step & 1:
            torch.cuda.synchronize()
            refs.append(snapshot(eager))

    cap = torch.cuda.Stream()
    Ls = make_layers(n, B, Hk, Hv, d, stream=cap)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        token(Ls, 0)
        token(Ls, 1)
    torch.cuda.synchronize()
    # capturing launched nothing: the states are still the initial ones
    for S in Ls:
        assert torch.equal(S["state"], S["state0"]) and torch.equal(S["conv_state"], S["cs0"])
    scratch = torch.zeros(1 << 20, device=DEV)
    for r in range(3):
        graph.replay()
        scratch.add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        for (st, cs, out), S in zip(refs[r], Ls):
            assert torch.equal(S["state"], st), f"replay {r}: state"
            assert torch.equal(S["conv_state"], cs), f"replay {r}: conv state"
            assert torch.equal(S["out"], out), f"replay {r}: output"
