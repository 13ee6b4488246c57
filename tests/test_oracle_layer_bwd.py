"""Pins of the oracle's layer gradients ("Actions Speak Louder than Words" §3.1 eqs. (1)-(3)):
float64 autograd of an independent torch composition of the layer (linear, SiLU, split, dense
masked attention with the bias, LayerNorm, gate, linear, residual), and central finite
differences of the forward oracle for L = sum(Y * dY) at sampled coordinates of every input."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from hstu_sequential_transduction_jagged_amd import synth


def _params(seed, D, H, dqk, dv, P=8, NT=6, kind=oracle.BIAS_RAB_PT):
    rng = np.random.default_rng(seed)
    N1 = 2 * H * (dqk + dv)
    HV = H * dv
    p = dict(w1=rng.standard_normal((N1, D)) * 0.4, b1=rng.standard_normal(N1) * 0.2,
             gamma=1 + 0.3 * rng.standard_normal(HV), beta=0.3 * rng.standard_normal(HV),
             w2=rng.standard_normal((D, HV)) * 0.4, b2=rng.standard_normal(D) * 0.2)
    if kind == oracle.BIAS_RAB_PT:
        p["w_pos"] = rng.standard_normal(P) * 0.5
        p["w_time"] = rng.standard_normal(NT) * 0.5
    return p


def _torch_layer(offs, x, p, ts, kind, H, dqk, dv, alpha, residual, eps):
    t = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    X = torch.tensor(x, requires_grad=True)
    HV, HQ = H * dv, H * dqk
    Z = F.silu(X @ t["w1"].T + t["b1"])
    U, V, Q, K = torch.split(Z, [HV, HV, HQ, HQ], dim=1)
    outs = []
    for b in range(len(offs) - 1):
        s, e = int(offs[b]), int(offs[b + 1])
        n = e - s
        if n == 0:
            continue
        i = torch.arange(n)[:, None]
        j = torch.arange(n)[None, :]
        heads = []
        for h in range(H):
            S = alpha * (Q[s:e, h * dqk:(h + 1) * dqk] @ K[s:e, h * dqk:(h + 1) * dqk].T)
            if kind == oracle.BIAS_RAB_PT:
                P, NT = p["w_pos"].shape[0], p["w_time"].shape[0]
                dt = torch.tensor(ts[s:e])[:, None] - torch.tensor(ts[s:e])[None, :]
                tb = torch.clamp(torch.floor(torch.log2(torch.clamp(dt, min=0).double() + 1)).long(),
                                 max=NT - 1)
                S = S + t["w_pos"][torch.clamp(i - j, 0, P - 1)] + t["w_time"][tb]
            A = torch.where(i >= j, F.silu(S), torch.zeros_like(S))
            heads.append(A @ V[s:e, h * dv:(h + 1) * dv])
        outs.append(torch.cat(heads, dim=1))
    O = torch.cat(outs)
    G = F.layer_norm(O, (HV,), t["gamma"], t["beta"], eps) * U
    Y = G @ t["w2"].T + t["b2"]
    if residual:
        Y = Y + X
    return Y, X, t


@pytest.mark.parametrize("residual", [False, True])
@pytest.mark.parametrize("kind", [oracle.BIAS_RAB_PT, oracle.BIAS_NONE])
def test_layer_grads_against_torch_autograd(residual, kind):
    D, H, dqk, dv = 6, 2, 3, 4
    lengths = [4, 0, 9, 1]
    rng = np.random.default_rng(60)
    offs = synth.offsets_from_lengths(lengths).astype(np.int64)
    T = int(offs[-1])
    x = rng.standard_normal((T, D))
    ts = np.concatenate([100 + np.cumsum(rng.integers(0, 20, size=n)) for n in lengths])
    p = _params(61, D, H, dqk, dv, kind=kind)
    dY = rng.standard_normal((T, D))
    alpha, eps = 0.6, 1e-5
    bias = oracle.Bias(kind, ts, p.get("w_pos"), p.get("w_time")) if kind == oracle.BIAS_RAB_PT \
        else oracle.Bias(oracle.BIAS_NONE)
    got = oracle.layer_bwd(offs, x, p["w1"], p["b1"], p["gamma"], p["beta"], p["w2"], p["b2"], bias,
                           alpha, H, dqk, dv, dY, residual=residual, ln_eps=eps)
    Y, X, t = _torch_layer(offs, x, p, ts, kind, H, dqk, dv, alpha, residual, eps)
    (Y * torch.tensor(dY)).sum().backward()
    pairs = [("dx", X), ("dw1", t["w1"]), ("db1", t["b1"]), ("dgamma", t["gamma"]),
             ("dbeta", t["beta"]), ("dw2", t["w2"]), ("db2", t["b2"])]
    if kind == oracle.BIAS_RAB_PT:
        pairs += [("dw_pos", t["w_pos"]), ("dw_time", t["w_time"])]
    for name, leaf in pairs:
        np.testing.assert_allclose(got[name], leaf.grad.numpy(), rtol=1e-10, atol=1e-10,
                                   err_msg=name)


def test_layer_grads_finite_differences():
    D, H, dqk, dv = 5, 2, 3, 3
    lengths = [6, 3]
    rng = np.random.default_rng(62)
    offs = synth.offsets_from_lengths(lengths).astype(np.int64)
    T = int(offs[-1])
    x = rng.standard_normal((T, D))
    ts = np.concatenate([100 + np.cumsum(rng.integers(0, 20, size=n)) for n in lengths])
    p = _params(63, D, H, dqk, dv)
    dY = rng.standard_normal((T, D))
    alpha, eps = 0.5, 1e-5
    bias = oracle.Bias(oracle.BIAS_RAB_PT, ts, p["w_pos"], p["w_time"])
    got = oracle.layer_bwd(offs, x, p["w1"], p["b1"], p["gamma"], p["beta"], p["w2"], p["b2"], bias,
                           alpha, H, dqk, dv, dY, residual=True, ln_eps=eps)

    def L():
        y = oracle.layer(offs, x, p["w1"], p["b1"], p["gamma"], p["beta"], p["w2"], p["b2"], bias,
                         alpha, H, dqk, dv, residual=True, ln_eps=eps)
        return float(np.sum(y * dY))

    eps_fd = 1e-6
    checks = [("dx", x), ("dw1", p["w1"]), ("db1", p["b1"]), ("dgamma", p["gamma"]),
              ("dbeta", p["beta"]), ("dw2", p["w2"]), ("db2", p["b2"]), ("dw_pos", p["w_pos"]),
              ("dw_time", p["w_time"])]
    for name, arr in checks:
        for _ in range(4):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            a0 = arr[idx]
            arr[idx] = a0 + eps_fd
            lp = L()
            arr[idx] = a0 - eps_fd
            lm = L()
            arr[idx] = a0
            fd = (lp - lm) / (2 * eps_fd)
            assert abs(fd - got[name][idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, fd, got[name][idx])


def test_round_bf16_against_torch_and_ties():
    """The mirror mode's bf16 rounding: ties go to the even neighbour (1 + 2^-8 lies halfway
    between 1 and 1 + 2^-7; 1 + 3 2^-8 halfway between 1 + 2^-7 and 1 + 2^-6), and on float32
    inputs it agrees with torch's own float32 -> bfloat16 conversion."""
    got = oracle.round_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20,
                                      -(1 + 2.0 ** -8), 0.0]))
    assert list(got) == [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.0, 0.0]
    rng = np.random.default_rng(70)
    r = (rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000)).astype(np.float32)
    ref = torch.from_numpy(r).to(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.round_bf16(r.astype(np.float64)), ref)


def test_mirror_mode_rounds_only_where_named():
    """Nothing rounded gives the exact gradients; rounding only G changes only dW2 = dY^T G
    (G feeds nothing else); rounding Y in the forward is the exact Y rounded once."""
    D, H, dqk, dv = 6, 2, 3, 4
    lengths = [5, 7]
    rng = np.random.default_rng(71)
    offs = synth.offsets_from_lengths(lengths).astype(np.int64)
    T = int(offs[-1])
    x = rng.standard_normal((T, D))
    ts = np.concatenate([100 + np.cumsum(rng.integers(0, 20, size=n)) for n in lengths])
    p = _params(72, D, H, dqk, dv)
    dY = rng.standard_normal((T, D))
    bias = oracle.Bias(oracle.BIAS_RAB_PT, ts, p["w_pos"], p["w_time"])
    args = (offs, x, p["w1"], p["b1"], p["gamma"], p["beta"], p["w2"], p["b2"], bias, 0.6, H, dqk,
            dv)
    exact = oracle.layer_bwd(*args, dY, residual=True)
    g = oracle.layer_bwd(*args, dY, residual=True, round_at=("G",))
    for name in ("dx", "dw1", "db1", "dgamma", "dbeta", "db2", "dw_pos", "dw_time"):
        np.testing.assert_allclose(g[name], exact[name], rtol=1e-12, atol=1e-12, err_msg=name)
    assert np.max(np.abs(g["dw2"] - exact["dw2"])) > 0
    y = oracle.layer(*args, residual=True)
    ym, _, _ = oracle.layer_mirror(*args, residual=True, round_at=("Y",))
    np.testing.assert_array_equal(ym, oracle.round_bf16(oracle.layer_mirror(*args, residual=True)[0]))
    np.testing.assert_allclose(oracle.layer_mirror(*args, residual=True)[0], y, rtol=1e-12, atol=1e-12)
