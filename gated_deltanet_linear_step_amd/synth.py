"""Seeded synthetic workloads for the gated delta-rule step.

This module only draws numbers: it holds none of the method's arithmetic, and
both the HIP path's tests/benchmark and the CPU oracle consume what it returns.
Every array comes back as a torch CPU tensor in its storage dtype (f16, bf16,
f32, int32); callers widen to float64 for the oracle and copy to the GPU for
the HIP library.

Three recipes:

* ``sin_values`` -- f16/f32(sin(i * f) * amp), the deterministic patterns of the
  ferrum-kernels 0.8.0 test page (``half_values`` / ``float_values``), used for
  the T=4 layer conformance workload with the frequencies and amplitudes that
  page prints.
* ``Lcg`` -- the 32-bit linear congruential draws of the ferrox-core 0.24.0
  gdn.rs tests (``the_device_delta_step_matches_this_one``): un-normalised
  uniform q, k, v and states, used for that test's device-step shapes.
* numpy ``default_rng(seed)`` normals/uniforms rounded to bf16 (round to nearest
  even, via torch) for the batched-decode, prefill and deep-model workloads;
  draw order is parameters, then states, then per-step inputs.
"""
from __future__ import annotations

import numpy as np
import torch

GROUPED, TILED = 0, 1


def sin_values(n: int, freq: float, amp: float, dtype=torch.float16) -> torch.Tensor:
    """dtype(sin(i * freq) * amp) for i in [0, n), evaluated in float32."""
    i = np.arange(n, dtype=np.float32)
    vals = np.sin(i * np.float32(freq)).astype(np.float32) * np.float32(amp)
    return torch.from_numpy(vals.astype(np.float32)).to(dtype)


def _t(a: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)


def qkv_features(Hk: int, Hv: int, dk: int, dv: int) -> int:
    return 2 * Hk * dk + Hv * dv


def default_dt_bias(Hv: int) -> torch.Tensor:
    """dt_bias[h] = -0.25 + 0.04 h (the layer-conformance workload's formula)."""
    return torch.tensor([-0.25 + h * 0.04 for h in range(Hv)], dtype=torch.float32)


def default_norm(dv: int) -> torch.Tensor:
    """norm[j] = 0.82 + 0.013 j (the layer-conformance workload's formula)."""
    return torch.tensor([0.82 + j * 0.013 for j in range(dv)], dtype=torch.float32)


def layer_conformance(T: int = 4, Hk: int = 16, Hv: int = 32, dk: int = 128, dv: int = 128,
                      conv_k: int = 4, head_map: int = GROUPED) -> dict:
    """The T=4 fp16 layer workload of the ferrum-kernels test page
    (``assert_recurrent_conformance``): sin patterns with the printed
    frequencies/amplitudes, A_log[h] = -1.7 + 0.07 h."""
    QKV = qkv_features(Hk, Hv, dk, dv)
    return dict(
        T=T, Hk=Hk, Hv=Hv, dk=dk, dv=dv, conv_k=conv_k, head_map=head_map,
        x=sin_values(T * QKV, 0.017, 0.21).reshape(T, QKV),
        a=sin_values(T * Hv, 0.071, 0.18).reshape(T, Hv),
        b=sin_values(T * Hv, 0.053, 0.24).reshape(T, Hv),
        z=sin_values(T * Hv * dv, 0.029, 0.31).reshape(T, Hv, dv),
        conv_w=sin_values(QKV * conv_k, 0.011, 0.16).reshape(QKV, conv_k),
        A_log=torch.tensor([-1.7 + h * 0.07 for h in range(Hv)], dtype=torch.float32),
        dt_bias=default_dt_bias(Hv),
        norm_w=default_norm(dv),
        conv_state=sin_values(QKV * (conv_k - 1), 0.023, 0.04).reshape(QKV, conv_k - 1),
        state=sin_values(Hv * dv * dk, 0.007, 0.025, torch.float32).reshape(Hv, dv, dk),
    )


def decode_batch(seed: int, B: int, Hk: int = 16, Hv: int = 32, dk: int = 128, dv: int = 128,
                 T: int = 1, conv_k: int = 4, head_map: int = TILED, dtype=torch.bfloat16,
                 state_std: float = 0.02) -> dict:
    """Batched decode workload: B sequences of T tokens, every activation N(0, 1)
    in ``dtype``; fp32 state N(0, state_std^2); conv state N(0, 1); conv taps
    N(0, 0.5^2); A_log ~ U[-2, 0]; dt_bias and norm by formula.
    Mixed [q|k|v] inputs are [B*T][QKV] (token-major, sequence outer)."""
    rng = np.random.default_rng(seed)
    QKV = qkv_features(Hk, Hv, dk, dv)
    conv_w = _t(rng.normal(0.0, 0.5, (QKV, conv_k)), dtype)
    A_log = torch.from_numpy(rng.uniform(-2.0, 0.0, Hv).astype(np.float32))
    state = torch.from_numpy(rng.normal(0.0, state_std, (B, Hv, dv, dk)).astype(np.float32))
    conv_state = _t(rng.normal(0.0, 1.0, (B, QKV, conv_k - 1)), dtype)
    x = _t(rng.normal(0.0, 1.0, (B * T, QKV)), dtype)
    z = _t(rng.normal(0.0, 1.0, (B * T, Hv, dv)), dtype)
    a = _t(rng.normal(0.0, 1.0, (B * T, Hv)), dtype)
    b = _t(rng.normal(0.0, 1.0, (B * T, Hv)), dtype)
    return dict(B=B, T=T, Hk=Hk, Hv=Hv, dk=dk, dv=dv, conv_k=conv_k, head_map=head_map,
                x=x, z=z, a=a, b=b, conv_w=conv_w, A_log=A_log, dt_bias=default_dt_bias(Hv),
                norm_w=default_norm(dv), conv_state=conv_state, state=state)


def fresh_decode_inputs(seed: int, B: int, Hk: int, Hv: int, dk: int, dv: int, T: int = 1,
                        dtype=torch.bfloat16) -> dict:
    """New per-step activations (x, z, a, b) N(0, 1) for a further decode step."""
    rng = np.random.default_rng(seed)
    QKV = qkv_features(Hk, Hv, dk, dv)
    return dict(x=_t(rng.normal(0.0, 1.0, (B * T, QKV)), dtype),
                z=_t(rng.normal(0.0, 1.0, (B * T, Hv, dv)), dtype),
                a=_t(rng.normal(0.0, 1.0, (B * T, Hv)), dtype),
                b=_t(rng.normal(0.0, 1.0, (B * T, Hv)), dtype))


def cu_seqlens(lengths) -> torch.Tensor:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def prefill(seed: int, lengths, Hk: int = 16, Hv: int = 32, dk: int = 128, dv: int = 128,
            head_map: int = GROUPED, dtype=torch.bfloat16, state_std: float = 0.0,
            with_z: bool = False) -> dict:
    """Packed prefill workload: sequences of the given lengths back to back.
    q, k [tok][Hk][dk], v [tok][Hv][dv], a, b [tok][Hv] all N(0, 1) in ``dtype``;
    A_log ~ U[-2, 0]; dt_bias by formula; initial states N(0, state_std^2)
    (zeros when state_std == 0)."""
    rng = np.random.default_rng(seed)
    N = len(lengths)
    tok = int(sum(lengths))
    A_log = torch.from_numpy(rng.uniform(-2.0, 0.0, Hv).astype(np.float32))
    if state_std > 0:
        state = torch.from_numpy(rng.normal(0.0, state_std, (N, Hv, dv, dk)).astype(np.float32))
    else:
        state = torch.zeros((N, Hv, dv, dk), dtype=torch.float32)
    q = _t(rng.normal(0.0, 1.0, (tok, Hk, dk)), dtype)
    k = _t(rng.normal(0.0, 1.0, (tok, Hk, dk)), dtype)
    v = _t(rng.normal(0.0, 1.0, (tok, Hv, dv)), dtype)
    a = _t(rng.normal(0.0, 1.0, (tok, Hv)), dtype)
    b = _t(rng.normal(0.0, 1.0, (tok, Hv)), dtype)
    out = dict(N=N, lengths=list(lengths), cu_seqlens=cu_seqlens(lengths), Hk=Hk, Hv=Hv, dk=dk,
               dv=dv, head_map=head_map, q=q, k=k, v=v, a=a, b=b, A_log=A_log,
               dt_bias=default_dt_bias(Hv), state=state)
    if with_z:
        out["z"] = _t(rng.normal(0.0, 1.0, (tok, Hv, dv)), dtype)
        out["norm_w"] = default_norm(dv)
    return out


def core_sin(T: int, Hk: int, Hv: int, dk: int, dv: int) -> dict:
    """The chunk-core workload of the ferrum-kernels test page
    (``chunked_c64_matches_recurrent_oracle_and_non_aligned_state_continuity``):
    f32 q, k, v from sin patterns (q, k normalised by the caller's L2 norm),
    g = -0.008 - |sin(0.017 i)| * 0.025, beta = 0.2 + |sin(0.013 i)| * 0.6,
    initial state sin(0.011 i) * 0.025."""
    i = np.arange(T * Hv, dtype=np.float32)
    g = (np.float32(-0.008) - np.abs(np.sin(i * np.float32(0.017))) * np.float32(0.025))
    beta = np.float32(0.2) + np.abs(np.sin(i * np.float32(0.013))) * np.float32(0.6)
    return dict(
        T=T, Hk=Hk, Hv=Hv, dk=dk, dv=dv,
        q=sin_values(T * Hk * dk, 0.019, 0.4, torch.float32).reshape(T, Hk, dk),
        k=sin_values(T * Hk * dk, 0.031, 0.35, torch.float32).reshape(T, Hk, dk),
        v=sin_values(T * Hv * dv, 0.023, 0.2, torch.float32).reshape(T, Hv, dv),
        g=torch.from_numpy(g.astype(np.float32)).reshape(T, Hv),
        beta=torch.from_numpy(beta.astype(np.float32)).reshape(T, Hv),
        state=sin_values(Hv * dv * dk, 0.011, 0.025, torch.float32).reshape(Hv, dv, dk),
    )


class Lcg:
    """The ferrox-core gdn.rs test generator: seed <- seed * 1664525 + 1013904223
    (mod 2^32); each draw is ((seed >> 8) / 2^23 - 1) * scale in f32, uniform in
    [-scale, scale). Draws continue one stream in call order."""

    def __init__(self, seed: int):
        self.seed = seed & 0xFFFFFFFF

    def draw(self, n: int, scale: float) -> np.ndarray:
        out = np.empty(n, dtype=np.float32)
        s = self.seed
        for i in range(n):
            s = (s * 1664525 + 1013904223) & 0xFFFFFFFF
            out[i] = np.float32(s >> 8)
        self.seed = s
        return (out / np.float32(8388608.0) - np.float32(1.0)) * np.float32(scale)


def device_step(n_k: int, n_v: int, s: int, seed: int = 12345) -> dict:
    """The inputs of the ferrox-core device-step test for one token of one
    sequence, drawn in that test's order: state [n_v][s][s] (scale 0.5), q, k
    [n_k][s] and v [n_v][s] (scale 1), g = -|u| and beta = 0.5 + 0.25 u with u
    uniform in [-1, 1). q and k are not normalised. f32 throughout."""
    r = Lcg(seed)
    state = r.draw(n_v * s * s, 0.5).reshape(n_v, s, s)
    q = r.draw(n_k * s, 1.0).reshape(1, n_k, s)
    k = r.draw(n_k * s, 1.0).reshape(1, n_k, s)
    v = r.draw(n_v * s, 1.0).reshape(1, n_v, s)
    g = -np.abs(r.draw(n_v, 1.0)).reshape(1, n_v)
    beta = (np.float32(0.5) + np.float32(0.25) * r.draw(n_v, 1.0)).reshape(1, n_v)
    t = torch.from_numpy
    return dict(state=t(np.ascontiguousarray(state)), q=t(q), k=t(k), v=t(v),
                g=t(np.ascontiguousarray(g, dtype=np.float32)),
                beta=t(np.ascontiguousarray(beta, dtype=np.float32)), rng=r)


def lcg_prefill(T: int, Hk: int, Hv: int, dk: int, dv: int, seed: int = 777,
                qk_scale: float = 0.15) -> dict:
    """An un-normalised prefill workload from the same LCG stream: q, k uniform in
    [-qk_scale, qk_scale) (so |k|^2 is about dk * qk_scale^2 / 3, below 1 at
    dk = 128 and the default scale: a stable delta rule without the in-op L2
    norm), v in [-1, 1), g = -0.05 |u|, beta = 0.5 + 0.25 u, initial state in
    [-0.05, 0.05). f32, one sequence."""
    r = Lcg(seed)
    state = r.draw(Hv * dv * dk, 0.05).reshape(1, Hv, dv, dk)
    q = r.draw(T * Hk * dk, qk_scale).reshape(T, Hk, dk)
    k = r.draw(T * Hk * dk, qk_scale).reshape(T, Hk, dk)
    v = r.draw(T * Hv * dv, 1.0).reshape(T, Hv, dv)
    g = np.float32(-0.05) * np.abs(r.draw(T * Hv, 1.0)).reshape(T, Hv)
    beta = (np.float32(0.5) + np.float32(0.25) * r.draw(T * Hv, 1.0)).reshape(T, Hv)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))  # noqa: E731
    return dict(T=T, Hk=Hk, Hv=Hv, dk=dk, dv=dv, q=t(q), k=t(k), v=t(v), g=t(g), beta=t(beta),
                state=t(state), cu_seqlens=cu_seqlens([T]))


def negative_rates(seed: int, Hv: int) -> torch.Tensor:
    """Per-head decay rates for the negative-rate parameterisation (the rate that
    multiplies softplus, passed as is): uniform in [-1, -0.135], the range that
    A_log ~ U[-2, 0] gives under the log-rate form."""
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.uniform(-1.0, -0.135, Hv).astype(np.float32))
