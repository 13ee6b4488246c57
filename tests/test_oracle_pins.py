"""Pins of the fp64 CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: hand-worked
bucket indices, closed forms (prefix sums, single-token sequences, bucket
histograms, limits of SiLU), invariants (causality, jagged vs per-user,
permutations, scaling), a dense brute force on tiny inputs and a float64
PyTorch composition of the layer.  The inputs are chosen so that a plausible
mistake (a dropped bias term, i-j for j-i, a dropped diagonal, a transposed
weight, a wrong chunk order) fails at least one of them.

Sources: "Actions Speak Louder than Words" reading notes §3.1 eqs. (1)-(3) and
§3.2; "4.4 推荐模型的 Scaling", "HSTU 层" and the toy HSTULayer; GenRank article
part (2) (ALiBi).
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from hstu_sequential_transduction_jagged_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _silu_t(x):
    return F.silu(torch.as_tensor(x, dtype=torch.float64)).numpy()


def _rand_case(seed, lengths, H=2, d=8, dv=None, kind=oracle.BIAS_RAB_PT, P=16, NT=8,
               table_std=0.5, per_head=False):
    rng = np.random.default_rng(seed)
    dv = dv or d
    offs = synth.offsets_from_lengths(lengths).astype(np.int64)
    T = int(offs[-1])
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, dv))
    ts = np.concatenate([1000 + np.cumsum(rng.integers(0, 300, size=n)) for n in lengths]) \
        if T else np.zeros(0, np.int64)
    shape_p = (H, P) if per_head else (P,)
    shape_t = (H, NT) if per_head else (NT,)
    if kind == oracle.BIAS_RAB_PT:
        bias = oracle.Bias(kind, ts, rng.standard_normal(shape_p) * table_std,
                           rng.standard_normal(shape_t) * table_std)
    elif kind == oracle.BIAS_ALIBI:
        bias = oracle.Bias(kind, slopes=oracle.alibi_slopes(H))
    else:
        bias = oracle.Bias(oracle.BIAS_NONE)
    return offs, q, k, v, ts, bias


# ----------------------------------------------------------------------------------------------
# bucket indices: hand-worked values


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_bucket_golden():
    rows = _golden_rows("buckets.txt")
    assert len(rows) >= 20
    for kind, arg, size, expected in rows:
        fn = oracle.time_bucket if kind == "time" else oracle.pos_bucket
        assert fn(int(arg), int(size)) == int(expected), (kind, arg, size)


def test_time_bucket_matches_power_of_two_brackets():
    # bucket m <=> 2^m <= 1 + dt < 2^(m+1), for every dt in a range (before clipping)
    for dt in list(range(0, 5000)) + [2 ** e - 2 for e in range(2, 34)] + [2 ** e - 1 for e in range(1, 34)]:
        m = oracle.time_bucket(dt, 64)
        assert 2 ** m <= 1 + dt < 2 ** (m + 1), dt


# ----------------------------------------------------------------------------------------------
# SiLU itself (through a length-1 sequence: O = SiLU(w_p[0] + w_t[0]) * v)


def test_silu_golden_points():
    rows = _golden_rows("silu.txt")
    for xs, ys in rows:
        x, y = float(xs), float(ys)
        offs = np.array([0, 1])
        q = np.zeros((1, 1, 4))
        v = np.ones((1, 1, 1))
        bias = oracle.Bias(oracle.BIAS_RAB_PT, np.array([5], np.int64), np.array([x, 0.0]),
                           np.array([0.0, 7.0]))
        o = oracle.attention(offs, q, q, v, bias, alpha=1.0)
        assert abs(o[0, 0, 0] - y) <= 1e-15 * max(1.0, abs(y)), (x, o[0, 0, 0], y)


def test_silu_saturation_has_no_nan():
    # ALiBi-style very negative arguments: SiLU -> -0, never NaN
    offs = np.array([0, 1])
    q = np.zeros((1, 1, 4))
    v = np.ones((1, 1, 2))
    for x in [-800.0, -2000.0, -1e6]:
        bias = oracle.Bias(oracle.BIAS_RAB_PT, np.array([0], np.int64), np.array([x]),
                           np.array([0.0]))
        o = oracle.attention(offs, q, q, v, bias, alpha=1.0)
        assert np.all(np.isfinite(o)) and np.all(np.abs(o) < 1e-300)
    for x in [40.0, 700.0]:
        bias = oracle.Bias(oracle.BIAS_RAB_PT, np.array([0], np.int64), np.array([x]),
                           np.array([0.0]))
        o = oracle.attention(offs, q, q, v, bias, alpha=1.0)
        assert abs(o[0, 0, 0] - x) <= 1e-15 * x


# ----------------------------------------------------------------------------------------------
# closed forms


@pytest.mark.parametrize("out_scale", [1.0, 0.125])
def test_constant_bias_is_scaled_prefix_sum(out_scale):
    # alpha = 0 and constant tables: every weight is SiLU(c1 + c2), so
    # O_i = out_scale * SiLU(c1 + c2) * sum_{j <= i} v_j  (mask includes the diagonal)
    lengths = [0, 1, 5, 37, 2]
    offs, q, k, v, ts, _ = _rand_case(1, lengths, H=3, d=4, dv=6)
    c1, c2 = 0.7, -0.2
    bias = oracle.Bias(oracle.BIAS_RAB_PT, ts, np.full(16, c1), np.full(8, c2))
    o = oracle.attention(offs, q, k, v, bias, alpha=0.0, out_scale=out_scale)
    w = _silu_t(c1 + c2)
    for b in range(len(lengths)):
        s, e = offs[b], offs[b + 1]
        ref = out_scale * w * np.cumsum(v[s:e], axis=0)
        np.testing.assert_allclose(o[s:e], ref, rtol=1e-13, atol=1e-13)


def test_single_token_users():
    # n = 1: O_0 = SiLU(alpha <q,k> + w_p[0] + w_t[0]) v_0
    lengths = [1] * 7
    offs, q, k, v, ts, bias = _rand_case(2, lengths, H=2, d=8, P=4, NT=4)
    alpha = 0.3
    o = oracle.attention(offs, q, k, v, bias, alpha)
    x = alpha * np.einsum("thd,thd->th", q, k) + bias.w_pos[0] + bias.w_time[0]
    ref = _silu_t(x)[..., None] * v
    np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("m", [0, 1, 3, 5, 7])
def test_time_bucket_histogram(m):
    # K = 0, V = 1, w_p = 0, w_t = nu * e_m: O_i = SiLU(nu) * #{j <= i : bucket(t_i - t_j) = m}
    lengths = [40, 13, 1]
    offs, q, k, v, ts, _ = _rand_case(3, lengths, H=1, d=4)
    k[:] = 0.0
    v = np.ones((offs[-1], 1, 1))
    NT = 8
    nu = 1.3
    wt = np.zeros(NT)
    wt[m] = nu
    bias = oracle.Bias(oracle.BIAS_RAB_PT, ts, np.zeros(16), wt)
    o = oracle.attention(offs, q, k, v, bias, alpha=0.9)
    for b in range(len(lengths)):
        s = offs[b]
        for i in range(lengths[b]):
            cnt = 0
            for j in range(i + 1):
                u = 1 + max(int(ts[s + i]) - int(ts[s + j]), 0)
                lo, hi = 2 ** m, 2 ** (m + 1)
                inside = (lo <= u < hi) if m < NT - 1 else (u >= lo)
                cnt += inside
            assert abs(o[s + i, 0, 0] - _silu_t(nu) * cnt) < 1e-12, (b, i, cnt)


@pytest.mark.parametrize("p", [0, 1, 6, 15])
def test_position_bucket_histogram(p):
    # w_p = nu * e_p, w_t = 0, K = 0, V = 1: O_i = SiLU(nu) * #{j <= i : min(i - j, P-1) = p}
    P = 16
    lengths = [40, 9]
    offs, q, k, v, ts, _ = _rand_case(4, lengths, H=2, d=4, P=P)
    k[:] = 0.0
    v = np.ones((offs[-1], 2, 1))
    wp = np.zeros(P)
    wp[p] = -0.8
    bias = oracle.Bias(oracle.BIAS_RAB_PT, ts, wp, np.zeros(8))
    o = oracle.attention(offs, q, k, v, bias, alpha=0.5)
    for b, n in enumerate(lengths):
        for i in range(n):
            if p < P - 1:
                cnt = 1 if i >= p else 0
            else:
                cnt = max(0, i - (P - 1) + 1)
            assert abs(o[offs[b] + i, :, 0] - _silu_t(-0.8) * cnt).max() < 1e-12


def test_alibi_series():
    # alpha = 0, V = 1: O_i(h) = sum_{m=0}^{i} SiLU(-slope_h * m)
    H = 4
    lengths = [30, 3]
    offs, q, k, v, ts, _ = _rand_case(5, lengths, H=H, d=4)
    v = np.ones((offs[-1], H, 1))
    slopes = oracle.alibi_slopes(H)
    np.testing.assert_allclose(slopes, [2 ** -2, 2 ** -4, 2 ** -6, 2 ** -8])
    bias = oracle.Bias(oracle.BIAS_ALIBI, slopes=slopes)
    o = oracle.attention(offs, q, k, v, bias, alpha=0.0)
    for b, n in enumerate(lengths):
        for h in range(H):
            series = np.cumsum(_silu_t(-slopes[h] * np.arange(n)))
            np.testing.assert_allclose(o[offs[b]:offs[b + 1], h, 0], series, rtol=1e-13,
                                       atol=1e-14)


def test_large_argument_limit_is_masked_linear_attention():
    # SiLU(x) = x - x e^-x/(1+e^-x) ~ x when x >> 0: with a constant +40 bias and
    # small alpha q.k, O = tril(alpha Q K^T + 40) V up to 40 e^-39 relative
    lengths = [23, 1, 9]
    offs, q, k, v, ts, _ = _rand_case(6, lengths, H=2, d=8, dv=5)
    bias = oracle.Bias(oracle.BIAS_RAB_PT, ts, np.full(16, 25.0), np.full(8, 15.0))
    alpha = 0.02
    o = oracle.attention(offs, q, k, v, bias, alpha)
    for b, n in enumerate(lengths):
        s, e = offs[b], offs[b + 1]
        for h in range(2):
            S = alpha * q[s:e, h] @ k[s:e, h].T + 40.0
            ref = np.tril(S) @ v[s:e, h]
            np.testing.assert_allclose(o[s:e, h], ref, rtol=1e-12, atol=1e-12)


def test_small_argument_limit_is_half_masked_linear_attention():
    # SiLU(x) = x/2 + x^2/4 + O(x^4): with |x| <= ~1e-4, O = 0.5 tril(alpha QK^T - slope(i-j)) V
    # to relative accuracy ~1e-4 (ALiBi bias: a plain Toeplitz matrix)
    H = 2
    lengths = [31, 4]
    offs, q, k, v, ts, _ = _rand_case(7, lengths, H=H, d=8)
    slopes = np.array([1e-6, 3e-6])
    bias = oracle.Bias(oracle.BIAS_ALIBI, slopes=slopes)
    alpha = 1e-5
    o = oracle.attention(offs, q, k, v, bias, alpha)
    for b, n in enumerate(lengths):
        s, e = offs[b], offs[b + 1]
        ij = np.subtract.outer(np.arange(n), np.arange(n))
        for h in range(H):
            X = alpha * q[s:e, h] @ k[s:e, h].T - slopes[h] * ij
            ref = np.tril(0.5 * X + 0.25 * X * X) @ v[s:e, h]
            err = np.abs(o[s:e, h] - ref).max() / np.abs(ref).max()
            assert err < 1e-6, err


# ----------------------------------------------------------------------------------------------
# invariants


def test_zero_queries_and_keys_give_zero():
    lengths = [5, 0, 17]
    offs, q, k, v, ts, _ = _rand_case(8, lengths)
    z = np.zeros_like(q)
    o = oracle.attention(offs, z, z, v, oracle.Bias(oracle.BIAS_NONE), alpha=1.0)
    assert np.all(o == 0.0)
    bias0 = oracle.Bias(oracle.BIAS_RAB_PT, ts, np.zeros(16), np.zeros(8))
    assert np.all(oracle.attention(offs, z, z, v, bias0, alpha=1.0) == 0.0)


def test_causality():
    lengths = [25, 12]
    offs, q, k, v, ts, bias = _rand_case(9, lengths)
    o = oracle.attention(offs, q, k, v, bias, 0.4)
    j = offs[0] + 17
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[j] += 3.0
    k2[j] -= 2.0
    v2[j] *= -5.0
    ts2 = ts.copy()
    ts2[j:offs[1]] += 10 ** 7  # later events moved further into the future (still ordered)
    bias2 = oracle.Bias(oracle.BIAS_RAB_PT, ts2, bias.w_pos, bias.w_time)
    o2 = oracle.attention(offs, q2, k2, v2, bias2, 0.4)
    assert np.array_equal(o[:j], o2[:j])
    assert not np.allclose(o[j:offs[1]], o2[j:offs[1]])
    assert np.array_equal(o[offs[1]:], o2[offs[1]:])


@pytest.mark.parametrize("kind", [oracle.BIAS_RAB_PT, oracle.BIAS_ALIBI, oracle.BIAS_NONE])
def test_jagged_equals_per_user(kind):
    lengths = [7, 0, 19, 1, 4]
    offs, q, k, v, ts, bias = _rand_case(10, lengths, H=3, kind=kind)
    o = oracle.attention(offs, q, k, v, bias, 0.25)
    for b, n in enumerate(lengths):
        s, e = offs[b], offs[b + 1]
        sub = oracle.Bias(kind, None if ts is None else ts[s:e], bias.w_pos, bias.w_time,
                          bias.slopes)
        ob = oracle.attention(np.array([0, n]), q[s:e], k[s:e], v[s:e], sub, 0.25)
        assert np.array_equal(o[s:e], ob)


def test_user_permutation_permutes_outputs():
    lengths = [6, 11, 3, 8]
    offs, q, k, v, ts, bias = _rand_case(11, lengths)
    o = oracle.attention(offs, q, k, v, bias, 0.3)
    perm = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(offs[b], offs[b + 1]) for b in perm])
    offs_p = synth.offsets_from_lengths([lengths[b] for b in perm])
    bias_p = oracle.Bias(oracle.BIAS_RAB_PT, ts[idx], bias.w_pos, bias.w_time)
    op = oracle.attention(offs_p, q[idx], k[idx], v[idx], bias_p, 0.3)
    assert np.array_equal(op, o[idx])


def test_head_permutation_with_shared_tables():
    lengths = [9, 14]
    offs, q, k, v, ts, bias = _rand_case(12, lengths, H=4)
    o = oracle.attention(offs, q, k, v, bias, 0.3)
    perm = [3, 1, 0, 2]
    op = oracle.attention(offs, q[:, perm], k[:, perm], v[:, perm], bias, 0.3)
    assert np.array_equal(op, o[:, perm])


def test_per_head_tables_select_their_head():
    lengths = [12, 5]
    offs, q, k, v, ts, bias = _rand_case(13, lengths, H=3, per_head=True)
    o = oracle.attention(offs, q, k, v, bias, 0.3)
    for h in range(3):
        bh = oracle.Bias(oracle.BIAS_RAB_PT, ts, bias.w_pos[h], bias.w_time[h])
        oh = oracle.attention(offs, q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], bh, 0.3)
        assert np.array_equal(oh[:, 0], o[:, h])


def test_power_of_two_scaling_of_v_is_exact():
    lengths = [10, 3]
    offs, q, k, v, ts, bias = _rand_case(14, lengths)
    o = oracle.attention(offs, q, k, v, bias, 0.3)
    o8 = oracle.attention(offs, q, k, v * 8.0, bias, 0.3)
    assert np.array_equal(o8, o * 8.0)


def test_linearity_in_v_and_table_shift():
    lengths = [15, 6]
    offs, q, k, v, ts, bias = _rand_case(15, lengths)
    v2 = np.random.default_rng(0).standard_normal(v.shape)
    o1 = oracle.attention(offs, q, k, v, bias, 0.3)
    o2 = oracle.attention(offs, q, k, v2, bias, 0.3)
    o12 = oracle.attention(offs, q, k, 2.0 * v - v2, bias, 0.3)
    np.testing.assert_allclose(o12, 2.0 * o1 - o2, rtol=1e-12, atol=1e-12)
    shifted = oracle.Bias(oracle.BIAS_RAB_PT, ts, bias.w_pos + 0.375, bias.w_time - 0.375)
    np.testing.assert_allclose(oracle.attention(offs, q, k, v, shifted, 0.3), o1, rtol=1e-12,
                               atol=1e-12)


def test_rows_entry_matches_full():
    lengths = [13, 0, 29, 2]
    offs, q, k, v, ts, bias = _rand_case(16, lengths, H=3)
    o = oracle.attention(offs, q, k, v, bias, 0.2)
    rng = np.random.default_rng(1)
    toks = rng.integers(0, offs[-1], size=40)
    heads = rng.integers(0, 3, size=40)
    r = oracle.attention_rows(offs, q, k, v, bias, 0.2, toks, heads)
    assert np.array_equal(r, o[toks, heads])


# ----------------------------------------------------------------------------------------------
# dense brute force on tiny inputs (materialises the n x n score, bias and mask)


def _dense(offs, q, k, v, ts, kind, wp, wt, slopes, alpha, out_scale=1.0, weight_unit=0.0):
    T, H, _ = q.shape
    out = np.zeros((T, H, v.shape[2]))
    for b in range(len(offs) - 1):
        s, e = offs[b], offs[b + 1]
        n = e - s
        if n == 0:
            continue
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        mask = (j <= i)
        for h in range(H):
            if kind == oracle.BIAS_RAB_PT:
                pb = np.minimum(np.maximum(i - j, 0), len(wp) - 1)
                dt = np.maximum(ts[s:e][:, None] - ts[s:e][None, :], 0) + 1
                tb = np.array([[int(u).bit_length() - 1 for u in row] for row in dt])
                tb = np.minimum(tb, len(wt) - 1)
                Bm = wp[pb] + wt[tb]
            elif kind == oracle.BIAS_ALIBI:
                Bm = -slopes[h] * (i - j)
            else:
                Bm = 0.0
            S = alpha * (q[s:e, h] @ k[s:e, h].T) + Bm
            A = np.where(mask, _silu_t(S), 0.0)
            if weight_unit:
                A = weight_unit * torch.from_numpy(A / weight_unit).to(torch.bfloat16).double().numpy()
            out[s:e, h] = out_scale * (A @ v[s:e, h])
    return out


@pytest.mark.parametrize("kind", [oracle.BIAS_RAB_PT, oracle.BIAS_ALIBI, oracle.BIAS_NONE])
@pytest.mark.parametrize("seed", [20, 21])
def test_dense_brute_force(kind, seed):
    lengths = [0, 1, 2, 37, 5]
    offs, q, k, v, ts, bias = _rand_case(seed, lengths, H=2, d=6, dv=3, kind=kind, P=8, NT=12)
    o = oracle.attention(offs, q, k, v, bias, 0.7, out_scale=0.5)
    ref = _dense(offs, q, k, v, ts, kind, bias.w_pos, bias.w_time, bias.slopes, 0.7, 0.5)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_mirror_weights_against_dense():
    """The oracle's mirror mode (SiLU weights kept as bf16 multiples of a unit) against the
    dense brute force with the weights rounded by torch's own bfloat16 conversion, and a unit of
    0 is the exact result."""
    lengths = [0, 1, 2, 37, 5]
    offs, q, k, v, ts, bias = _rand_case(22, lengths, H=2, d=6, dv=3, kind=oracle.BIAS_RAB_PT,
                                         P=8, NT=12)
    unit = 0.5 * math.log(2.0)
    o = oracle.attention(offs, q, k, v, bias, 0.7, weight_unit=unit)
    ref = _dense(offs, q, k, v, ts, oracle.BIAS_RAB_PT, bias.w_pos, bias.w_time, None, 0.7,
                 weight_unit=unit)
    exact = oracle.attention(offs, q, k, v, bias, 0.7)
    assert np.max(np.abs(o - exact)) > 0
    np.testing.assert_allclose(o, ref, rtol=1e-6, atol=1e-6 * np.abs(exact).max())
    np.testing.assert_array_equal(oracle.attention(offs, q, k, v, bias, 0.7, weight_unit=0.0),
                                  exact)


# ----------------------------------------------------------------------------------------------
# the layer (eqs. 1-3) against a float64 PyTorch composition


def _torch_layer(offs, x, L, H, dqk, dv, alpha, residual, eps, ts, kind):
    X = torch.as_tensor(x, dtype=torch.float64)
    Z = F.silu(F.linear(X, torch.as_tensor(L.w1, dtype=torch.float64),
                        torch.as_tensor(L.b1, dtype=torch.float64)))
    HV, HQ = H * dv, H * dqk
    U, V, Q, K = torch.split(Z, [HV, HV, HQ, HQ], dim=-1)
    T = x.shape[0]
    O = _dense(offs, Q.reshape(T, H, dqk).numpy(), K.reshape(T, H, dqk).numpy(),
               V.reshape(T, H, dv).numpy(), ts, kind,
               None if L.bias.w_pos is None else L.bias.w_pos.astype(np.float64),
               None if L.bias.w_time is None else L.bias.w_time.astype(np.float64),
               oracle.alibi_slopes(H), alpha)
    O = torch.as_tensor(O.reshape(T, HV))
    G = F.layer_norm(O, (HV,), torch.as_tensor(L.gamma, dtype=torch.float64),
                     torch.as_tensor(L.beta, dtype=torch.float64), eps) * U
    Y = F.linear(G, torch.as_tensor(L.w2, dtype=torch.float64),
                 torch.as_tensor(L.b2, dtype=torch.float64))
    if residual:
        Y = Y + X
    return Y.numpy()


def _oracle_layer(inp, L, x=None, residual=None):
    b = L.bias
    ob = oracle.Bias(b.kind, inp.ts, b.w_pos, b.w_time,
                     oracle.alibi_slopes(inp.H) if b.kind == oracle.BIAS_ALIBI else None)
    return oracle.layer(inp.offsets, inp.x if x is None else x, L.w1, L.b1, L.gamma, L.beta,
                        L.w2, L.b2, ob, inp.alpha, inp.H, inp.dqk, inp.dv,
                        residual=inp.residual if residual is None else residual,
                        ln_eps=inp.ln_eps)


@pytest.mark.parametrize("kind", [oracle.BIAS_RAB_PT, oracle.BIAS_ALIBI])
@pytest.mark.parametrize("residual", [False, True])
def test_layer_matches_torch_composition(kind, residual):
    rng = np.random.default_rng(30)
    lengths = [0, 3, 17, 1]
    inp = synth.make_layer("t", 30, lengths, D=16, H=2, d=8, alpha=0.3, residual=residual,
                           bias_kind=kind, P=8, NT=16, table_std=0.5, randomize_affine=True,
                           rng=rng, dtype="f32")
    L = inp.layers[0]
    y = _oracle_layer(inp, L)
    ref = _torch_layer(inp.offsets, inp.x, L, inp.H, inp.dqk, inp.dv, inp.alpha, residual,
                       inp.ln_eps, inp.ts, kind)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11)


def test_layer_with_zero_values_reduces_to_beta_gate():
    # V = SiLU(0) = 0 (zero V block of W1 and b1) => O = 0 => LayerNorm(O) = beta
    # => Y = (beta * U) W2^T + b2
    inp = synth.make_layer("t", 31, [6, 9], D=16, H=2, d=8, alpha=0.3, P=8, NT=16,
                           randomize_affine=True, dtype="f32")
    L = inp.layers[0]
    HV = inp.H * inp.dv
    L.w1[HV:2 * HV] = 0.0
    L.b1[HV:2 * HV] = 0.0
    y, z, o = oracle.layer(inp.offsets, inp.x, L.w1, L.b1, L.gamma, L.beta, L.w2, L.b2,
                           oracle.Bias(oracle.BIAS_RAB_PT, inp.ts, L.bias.w_pos, L.bias.w_time),
                           inp.alpha, inp.H, inp.dqk, inp.dv, return_intermediates=True)
    assert np.all(o == 0.0)
    x = inp.x.astype(np.float64)
    U = _silu_t(x @ L.w1[:HV].astype(np.float64).T + L.b1[:HV])
    ref = (L.beta.astype(np.float64) * U) @ L.w2.astype(np.float64).T + L.b2
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_layer_split_order_u_v_q_k():
    # The intermediates must follow U | V | Q | K: Q and K blocks feed the scores,
    # V the values, U the gate.  Swapping any two blocks of W1 changes Y.
    inp = synth.make_layer("t", 32, [11], D=16, H=2, d=8, alpha=0.5, P=8, NT=16,
                           randomize_affine=True, dtype="f32", table_std=0.3)
    L = inp.layers[0]
    y = _oracle_layer(inp, L)
    HV = 16
    for a, b in [(0, 1), (1, 2), (2, 3)]:
        w1 = L.w1.copy()
        w1[a * HV:(a + 1) * HV], w1[b * HV:(b + 1) * HV] = L.w1[b * HV:(b + 1) * HV], L.w1[a * HV:(a + 1) * HV]
        L2 = synth.LayerParams(w1, L.b1, L.gamma, L.beta, L.w2, L.b2, L.bias)
        assert not np.allclose(_oracle_layer(inp, L2), y)


def test_length_normalised_variant_single_user():
    """The length-normalised variant of the layer: "4.4 推荐模型的 Scaling" (remarks on the HSTU
    layer) divides each pointwise weight by the sequence length, eqs. (1)-(3) of "Actions Speak
    Louder than Words" §3.1 otherwise.  Written here as explicit sums over the causal pairs
    (position-only bias indexed by i - j, residual), it must equal the oracle's attention with
    alpha = 1 and out_scale = 1/n, and the oracle layer (which has no division) up to the
    LayerNorm's eps: LN(c o; eps) = LN(o; eps / c^2)."""
    rng = np.random.default_rng(33)
    n, d, h = 12, 8, 2
    dh = d // h
    x = rng.standard_normal((n, d))
    w1 = rng.standard_normal((4 * d, d)) * 0.3
    b1 = rng.standard_normal(4 * d) * 0.1
    w2 = rng.standard_normal((d, d)) * 0.3
    b2 = rng.standard_normal(d) * 0.1
    wp = rng.standard_normal(n) * 0.5
    # eq. (1): four blocks of d columns of SiLU(x W1^T + b1): gate, values, queries, keys
    z = x @ w1.T + b1
    z = z / (1.0 + np.exp(-z))
    U, V, Q, K = z[:, :d], z[:, d:2 * d], z[:, 2 * d:3 * d], z[:, 3 * d:]
    # eq. (2), one head (a block of dh columns) and one row at a time, each weight divided by n
    O = np.zeros((n, d))
    for hh in range(h):
        c = slice(hh * dh, (hh + 1) * dh)
        for i in range(n):
            for j in range(i + 1):
                sc = float(Q[i, c] @ K[j, c]) + wp[i - j]
                O[i, c] += sc / (1.0 + math.exp(-sc)) / n * V[j, c]

    # eq. (3): LayerNorm over the d features (biased variance), gate, f2, residual
    def out(o_rows, eps):
        y = np.zeros((n, d))
        for i in range(n):
            r = o_rows[i]
            mu = r.mean()
            g = (r - mu) / math.sqrt(((r - mu) ** 2).mean() + eps) * U[i]
            y[i] = x[i] + w2 @ g + b2
        return y

    offs = np.array([0, n])
    sh = lambda a: a.reshape(n, h, dh)
    bias = oracle.Bias(oracle.BIAS_RAB_PT, np.zeros(n, np.int64), wp, np.zeros(1))
    o = oracle.attention(offs, sh(Q), sh(K), sh(V), bias, alpha=1.0, out_scale=1.0 / n)
    np.testing.assert_allclose(o.reshape(n, d), O, rtol=1e-12, atol=1e-13)
    # no division, eps -> 0: the oracle layer equals the normalised form
    y = oracle.layer(offs, x, w1, b1, np.ones(d), np.zeros(d), w2, b2, bias, 1.0, h, dh, dh,
                     residual=True, ln_eps=1e-30)
    np.testing.assert_allclose(y, out(O, 1e-30), rtol=1e-10, atol=1e-10)
    # and with eps scaled by n^2 it equals the normalised form with eps
    y_eps = oracle.layer(offs, x, w1, b1, np.ones(d), np.zeros(d), w2, b2, bias, 1.0, h, dh, dh,
                         residual=True, ln_eps=1e-5 * n * n)
    np.testing.assert_allclose(y_eps, out(O, 1e-5), rtol=1e-10, atol=1e-10)


def test_stack_is_composition_of_residual_layers():
    inp = synth.make_layer("t", 34, [5, 8], D=16, H=2, d=8, alpha=0.3, n_layers=3,
                           residual=True, P=8, NT=16, randomize_affine=True, dtype="f32")
    biases = [oracle.Bias(oracle.BIAS_RAB_PT, inp.ts, L.bias.w_pos, L.bias.w_time)
              for L in inp.layers]
    layers = [dict(w1=L.w1, b1=L.b1, gamma=L.gamma, beta=L.beta, w2=L.w2, b2=L.b2)
              for L in inp.layers]
    y = oracle.stack(inp.offsets, inp.x, layers, biases, inp.alpha, inp.H, inp.dqk, inp.dv)
    h = inp.x.astype(np.float64)
    for L in inp.layers:
        h = _torch_layer(inp.offsets, h, L, inp.H, inp.dqk, inp.dv, inp.alpha, True, 1e-5,
                         inp.ts, oracle.BIAS_RAB_PT)
    np.testing.assert_allclose(y, h, rtol=1e-10, atol=1e-10)


def test_embed_sum():
    rng = np.random.default_rng(35)
    it = rng.standard_normal((50, 8))
    ac = rng.standard_normal((4, 8))
    ids = rng.integers(0, 50, size=20)
    acts = rng.integers(0, 4, size=20)
    x = oracle.embed_sum(it, ac, ids, acts)
    for t in range(20):
        np.testing.assert_array_equal(x[t], it[ids[t]] + ac[acts[t]])


def test_bucket_counts_brute_force():
    """The per-row bucket histograms equal a count over the pairs with the scalar bucket
    functions (pinned by the golden bucket table), on ragged users with unsorted, equal and
    far-apart timestamps."""
    lengths = [0, 1, 7, 40]
    offs = synth.offsets_from_lengths(lengths).astype(np.int64)
    rng = np.random.default_rng(80)
    ts = np.concatenate([np.zeros(0, np.int64), np.array([5], np.int64),
                         np.array([3, 3, 2, 10, 1 << 33, (1 << 33) + 1, 0], np.int64),
                         np.cumsum(rng.integers(0, 1 << 12, size=40)).astype(np.int64)])
    P, NT = 6, 9
    pc, tc = oracle.bucket_counts(offs, ts, P, NT)
    for b in range(len(lengths)):
        s = int(offs[b])
        for i in range(lengths[b]):
            ep, et = np.zeros(P, np.int64), np.zeros(NT, np.int64)
            for j in range(i + 1):
                ep[oracle.pos_bucket(i - j, P)] += 1
                et[oracle.time_bucket(int(ts[s + i] - ts[s + j]), NT)] += 1
            assert np.array_equal(pc[s + i], ep) and np.array_equal(tc[s + i], et), (b, i)
