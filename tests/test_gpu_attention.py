"""GPU parity of the attention (eq. (2)) against the fp64 oracle, through the C ABI.

Tolerances: max_k |y_k - ref_k| / rms(ref) <= 1e-4 for fp32 outputs; for bf16
outputs the same bound, 2e-2, after allowing each element its own bf16 rounding
(2^-8 |ref_k|), see tests/hstu_testutil.err_stored; bucket indices and the
scheduler's work list bit-exact.  Cases span several query and
key tiles with ragged tails, empty and single-token users, the benchmark's
near-linear SiLU regime (alpha = 1/N_max, tables N(0, 0.02)) and a strongly
nonlinear one (alpha = 1/sqrt(d), tables N(0, 1)).
"""
import numpy as np
import pytest
import torch

import oracle
from hstu_sequential_transduction_jagged_amd import binding, synth
from tests.hstu_testutil import (TOL, DevAttn, err_rms, err_stored, oracle_attn, oracle_attn_rows,
                                 run_attn, schedule_reference, to_dev)

pytestmark = pytest.mark.gpu

RAGGED = [0, 1, 2, 31, 32, 33, 63, 64, 65, 255, 256, 257, 700, 1500]


def _case(dtype, lengths, H=2, d=64, kind=synth.BIAS_RAB_PT, alpha=None, table_std=0.02, P=256,
          NT=32, seed=7, per_head=False):
    alpha = alpha if alpha is not None else 1.0 / max(1, max(lengths))
    return synth.make_attn("case", seed, dtype, lengths, H=H, d=d, alpha=alpha, bias_kind=kind,
                           P=P, NT=NT, table_std=table_std, per_head_tables=per_head)


def _check(inp, tol=None):
    o = run_attn(inp)
    ref = oracle_attn(inp)
    e = err_stored(o, ref, inp.dtype)
    print("%s dtype=%s T=%d H=%d err=%.3g (without storage allowance %.3g)"
          % (inp.name, inp.dtype, inp.T, inp.H, e, err_rms(o, ref)), flush=True)
    assert e <= (tol or TOL[inp.dtype]), e
    return o, ref


def test_attn_small_fp32_workload():
    _check(synth.attn_small())


def test_attn_small_fp32_nonlinear():
    inp = synth.attn_small(seed=2000)
    inp.alpha = 1.0 / np.sqrt(32)
    inp.bias.w_pos = inp.bias.w_pos * 50.0  # std 1
    inp.bias.w_time = inp.bias.w_time * 50.0
    _check(inp)


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("kind", [synth.BIAS_RAB_PT, synth.BIAS_ALIBI, synth.BIAS_NONE])
def test_fp32_ragged(d, kind):
    inp = _case("f32", [0, 1, 31, 32, 33, 127, 128, 129, 300], H=3, d=d, kind=kind,
                alpha=1.0 / np.sqrt(d), table_std=1.0, P=64, NT=16, per_head=True)
    _check(inp)


@pytest.mark.parametrize("regime", ["workload", "nonlinear"])
@pytest.mark.parametrize("kind", [synth.BIAS_RAB_PT, synth.BIAS_ALIBI, synth.BIAS_NONE])
def test_bf16_ragged(kind, regime):
    if regime == "workload":
        inp = _case("bf16", RAGGED, kind=kind, alpha=1.0 / 2048, table_std=0.02)
    else:
        inp = _case("bf16", RAGGED, kind=kind, alpha=1.0 / 8.0, table_std=1.0)
    _check(inp)


@pytest.mark.parametrize("regime", ["workload", "nonlinear"])
@pytest.mark.parametrize("kind", [synth.BIAS_RAB_PT, synth.BIAS_ALIBI, synth.BIAS_NONE])
def test_bf16_d32_ragged(kind, regime):
    # head dim 32 in bf16: two k-steps of the score product and one 32-column output block on
    # the stages' 128-byte rows; H = 3 so the last head's row ends inside the token's row
    if regime == "workload":
        inp = _case("bf16", RAGGED, H=3, d=32, kind=kind, alpha=1.0 / 2048, table_std=0.02)
    else:
        inp = _case("bf16", RAGGED, H=3, d=32, kind=kind, alpha=1.0 / np.sqrt(32), table_std=1.0,
                    P=64, NT=16, per_head=True)
    _check(inp)


def test_bf16_d32_strided_views_bitwise():
    """Q, K, V as column blocks of one [T, 3 H d + 8] bf16 buffer (row stride 3 H d + 8, as the
    layer's Z views are) give exactly the contiguous result; the columns between and after the
    blocks hold large values that must never be read."""
    inp = _case("bf16", [700, 0, 33, 257], H=3, d=32, alpha=0.05, table_std=0.5)
    d = DevAttn(inp)
    ref = d.run()
    T, H = inp.T, inp.H
    z = torch.full((T, 3 * H * 32 + 8), 3.0e38, dtype=torch.bfloat16, device="cuda")
    z[:, 0:H * 32] = d.q.reshape(T, -1)
    z[:, H * 32:2 * H * 32] = d.k.reshape(T, -1)
    z[:, 2 * H * 32:3 * H * 32] = d.v.reshape(T, -1)
    views = [z[:, i * H * 32:(i + 1) * H * 32].view(T, H, 32) for i in range(3)]
    o = binding.hstu_attn_fwd(views[0], views[1], views[2], d.offsets, inp.max_seqlen, d.bias,
                              inp.alpha, inp.out_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    assert torch.isfinite(o.float()).all()


def test_bf16_d32_long_users_sampled_rows():
    """Users of 8 192 and 3 000 rows (every query tile, far key tiles on the Taylor path), H = 4,
    d = 32, position + time bias; 600 sampled (token, head) rows against the oracle."""
    inp = _case("bf16", [8192, 3000], H=4, d=32, alpha=1.0 / 8192, table_std=0.02, seed=11)
    o = run_attn(inp)
    rng = np.random.default_rng(5)
    toks = rng.integers(0, inp.T, size=600)
    heads = rng.integers(0, inp.H, size=600)
    ref = oracle_attn_rows(inp, toks, heads)
    e = err_stored(o[toks, heads], ref, "bf16")
    print("d32 long err=%.3g" % e, flush=True)
    assert e <= TOL["bf16"], e


@pytest.mark.parametrize("kind", [synth.BIAS_RAB_PT, synth.BIAS_ALIBI])
def test_bf16_maximum_sizes_sampled_rows(kind):
    """The largest inputs the entry points accept: a user of 65 536 rows (max_seqlen's limit:
    512 query tiles, 2 048 key blocks) beside a one-row user, position tables of 1 024 buckets
    and 64 time buckets (both limits), tables of std 0.5 and alpha = 1/64 so that every SiLU
    path occurs; 300 sampled (token, head) rows (the last rows, tile and bucket edges, random
    rows) against the oracle."""
    inp = _case("bf16", [65536, 1], H=2, d=64, kind=kind, alpha=1.0 / 64, table_std=0.5,
                P=1024, NT=64, seed=13)
    o = run_attn(inp)
    rng = np.random.default_rng(8)
    toks = [65535, 65534, 65536, 0, 127, 128, 1023, 1024, 1025, 32767, 32768]
    toks += list(rng.integers(0, inp.T, size=300 - len(toks)))
    toks = np.array(toks)
    heads = rng.integers(0, inp.H, size=len(toks))
    ref = oracle_attn_rows(inp, toks, heads)
    e = err_stored(o[toks, heads], ref, "bf16")
    print("max sizes kind=%d err=%.3g (without storage allowance %.3g)"
          % (kind, e, err_rms(o[toks, heads], ref)), flush=True)
    assert e <= TOL["bf16"], e
    assert np.all(np.isfinite(o))


def test_bf16_per_head_tables_and_small_buckets():
    inp = _case("bf16", [5, 300, 129], H=3, alpha=0.1, table_std=1.0, P=16, NT=6, per_head=True)
    _check(inp)


def test_bf16_out_scale_and_toy_normalisation():
    inp = _case("bf16", [40, 250], alpha=1.0, table_std=0.5)
    inp.q = synth.round_bf16(inp.q * 0.125)
    inp.out_scale = 1.0 / 250
    _check(inp)


def test_bf16_unsorted_timestamps_and_huge_gaps():
    inp = _case("bf16", [300, 200], alpha=0.1, table_std=1.0)
    rng = np.random.default_rng(3)
    ts = inp.ts.copy()
    ts[:300] = rng.permutation(ts[:300])           # not monotone
    ts[300:] = np.cumsum(rng.integers(0, 2 ** 34, size=200))  # deltas beyond 2^31
    inp.ts = ts
    _check(inp)



@pytest.mark.parametrize("slopes", ["default", "mixed"])
@pytest.mark.parametrize("alpha", [1.0 / 4096, 1.0 / 8.0])
def test_bf16_alibi_far_cut(alpha, slopes):
    """ALiBi with users long enough that most key blocks lie where the bias alone puts the
    base-2 SiLU argument beyond 64 (the kernel skips those pairs: each weighs < 7e-18).  The
    nonlinear alpha makes the score part of the bound large (D up to ~20), so a cut that ignored
    it would drop pairs that matter; the mixed slopes include 0 and a negative slope (nothing may
    be cut), 2 and 4 (everything beyond ~45 / ~23 keys is cut).  A quarter of the keys carry
    values 8 times the others', so a pair cut too early shows in the output.
    Bound: 2e-2 for the default slopes; with a zero or negative slope thousands of same-sign
    weights of order one add up, and rounding the weights alone to bf16 (the matrix cores'
    operand) costs more than 2e-2, so the mixed case is held to max(2e-2, 1.5 e_m), e_m the
    error of the oracle with only its weights rounded so (oracle.attention(weight_unit=...))."""
    inp = _case("bf16", [1200, 700, 300, 65, 1] if slopes == "mixed" else [3000, 1500, 700, 65, 1],
                H=8, kind=synth.BIAS_ALIBI, alpha=alpha)
    rng = np.random.default_rng(11)
    inp.v = synth.round_bf16(inp.v * rng.choice([1.0, 8.0], size=(inp.T, 1, 1)).astype(np.float32))
    if slopes == "default":
        _check(inp)
        return
    inp.bias.slopes = np.array([4.0, 0.5, 0.0, -0.002, 2.0, 0.03, 1.0, 0.125], np.float32)
    o = run_attn(inp)
    ref = oracle_attn(inp)
    b = oracle.Bias(oracle.BIAS_ALIBI, slopes=inp.bias.slopes)
    mir = oracle.attention(inp.offsets, inp.q, inp.k, inp.v, b, inp.alpha,
                           weight_unit=-np.log(2.0) / 2.0)
    e, em = err_stored(o, ref, "bf16"), err_stored(mir, ref, "bf16")
    bound = max(TOL["bf16"], 1.5 * em)
    print("alibi mixed slopes T=%d err=%.3g (bf16 weights alone %.3g, bound %.3g)"
          % (inp.T, e, em, bound), flush=True)
    assert e <= bound, (e, bound)

def test_attn_long_workload_sampled_rows():
    """The long-sequence bf16 workload at full size (16 users up to 8192 tokens, H=8), checked
    on sampled rows: the last rows of every user (longest causal sums), tile edges, and
    random rows."""
    inp = synth.attn_long()
    d = DevAttn(inp)
    o = d.run()
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    rng = np.random.default_rng(5)
    toks, heads = [], []
    for b in range(inp.B):
        s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
        for i in [e - 1, e - 2, s, s + 255, s + 256, min(e - 1, s + 4095)]:
            if s <= i < e:
                toks.append(i)
                heads.append(int(rng.integers(0, inp.H)))
    toks += list(rng.integers(0, inp.T, size=400))
    heads += list(rng.integers(0, inp.H, size=400))
    toks, heads = np.array(toks), np.array(heads)
    ref = oracle_attn_rows(inp, toks, heads)
    e = err_stored(o[toks, heads], ref, "bf16")
    print("attn_long sampled rows=%d err=%.3g (without storage allowance %.3g)"
          % (len(toks), e, err_rms(o[toks, heads], ref)), flush=True)
    assert e <= TOL["bf16"]
    assert np.all(np.isfinite(o))


# ---------------------------------------------------------------------------------------------
# bitwise invariants of the GPU path


def test_gpu_jagged_equals_per_user_bitwise():
    inp = _case("bf16", [300, 0, 129, 1, 64], alpha=0.05, table_std=0.5)
    full = run_attn(inp)
    for b in range(inp.B):
        s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
        if e == s:
            continue
        sub = synth.AttnInputs("sub", 0, "bf16", 1, inp.H, inp.dqk, inp.dv,
                               np.array([0, e - s], np.int32), e - s, inp.ts[s:e], inp.q[s:e],
                               inp.k[s:e], inp.v[s:e], inp.bias, inp.alpha)
        ob = run_attn(sub)
        assert np.array_equal(ob, full[s:e]), b


def test_gpu_user_permutation_bitwise():
    lengths = [260, 7, 513, 64]
    inp = _case("bf16", lengths, alpha=0.05, table_std=0.5)
    full = run_attn(inp)
    perm = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(inp.offsets[b], inp.offsets[b + 1]) for b in perm])
    p = synth.AttnInputs("perm", 0, "bf16", 4, inp.H, 64, 64,
                         synth.offsets_from_lengths([lengths[b] for b in perm]), inp.max_seqlen,
                         inp.ts[idx], inp.q[idx], inp.k[idx], inp.v[idx], inp.bias, inp.alpha)
    assert np.array_equal(run_attn(p), full[idx])


def test_gpu_causality_bitwise():
    inp = _case("bf16", [600], alpha=0.05, table_std=0.5)
    full = run_attn(inp)
    j = 333
    inp2 = synth.AttnInputs("c", 0, "bf16", 1, inp.H, 64, 64, inp.offsets, inp.max_seqlen,
                            inp.ts.copy(), inp.q.copy(), inp.k.copy(), inp.v.copy(), inp.bias,
                            inp.alpha)
    inp2.q[j:] = synth.round_bf16(inp2.q[j:] * 3.0)
    inp2.k[j:] = synth.round_bf16(-inp2.k[j:])
    inp2.v[j:] = 0.0
    inp2.ts[j:] += 10 ** 6
    out2 = run_attn(inp2)
    assert np.array_equal(out2[:j], full[:j])
    assert not np.array_equal(out2[j:], full[j:])


def test_gpu_v_power_of_two_scaling_bitwise():
    inp = _case("bf16", [500, 77], alpha=0.05, table_std=0.5)
    full = run_attn(inp)
    inp.v = inp.v * 4.0
    assert np.array_equal(run_attn(inp), full * 4.0)


def test_gpu_zero_queries_keys_and_bias():
    inp = _case("bf16", [300, 5], kind=synth.BIAS_NONE)
    inp.q[:] = 0.0
    inp.k[:] = 0.0
    assert np.all(run_attn(inp) == 0.0)


@pytest.mark.parametrize("kind", [synth.BIAS_RAB_PT, synth.BIAS_ALIBI, synth.BIAS_NONE])
def test_gpu_empty_batch(kind):
    """Three empty users (T = 0, no timestamps): the call succeeds and returns an empty output."""
    inp = _case("bf16", [0, 0, 0], kind=kind)
    o = run_attn(inp)
    assert o.shape == (0, inp.H, inp.dv)


def test_gpu_repeat_calls_identical():
    inp = _case("bf16", RAGGED, alpha=0.05, table_std=0.5)
    d = DevAttn(inp)
    a = d.run().clone()
    b = d.run()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("kind", [synth.BIAS_RAB_PT, synth.BIAS_NONE, synth.BIAS_ALIBI])
def test_gpu_prepare_then_prepared_equals_one_call(kind):
    # hstu_attn_plan + hstu_attn_prepare + hstu_attn_fwd_prepared is hstu_attn_fwd in parts
    inp = _case("bf16", RAGGED, kind=kind, alpha=0.05, table_std=0.5)
    d = DevAttn(inp)
    ref = d.run().clone()
    ws = torch.empty(binding.attn_workspace_bytes(inp.B, inp.H, inp.max_seqlen, inp.T),
                     dtype=torch.uint8, device="cuda")
    binding.hstu_attn_plan(binding.DTYPE_BF16, inp.B, inp.H, inp.dqk, d.offsets, inp.max_seqlen, ws)
    binding.hstu_attn_prepare(d.k, d.offsets, inp.max_seqlen, ws, d.bias)
    o = binding.hstu_attn_fwd_prepared(d.q, d.k, d.v, d.offsets, inp.max_seqlen, ws, d.bias,
                                       inp.alpha, inp.out_scale)
    # a second kernel-only call on the same prepared workspace
    o2 = binding.hstu_attn_fwd_prepared(d.q, d.k, d.v, d.offsets, inp.max_seqlen, ws, d.bias,
                                        inp.alpha, inp.out_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref) and torch.equal(o2, ref)


# ---------------------------------------------------------------------------------------------
# integer paths: bucket indices and the work list, bit-exact


def test_bucket_indices_bit_exact():
    import oracle
    rng = np.random.default_rng(11)
    lengths = [50, 1, 300]
    offs = synth.offsets_from_lengths(lengths)
    ts = np.concatenate([np.cumsum(rng.integers(0, 2 ** 20, size=50)),
                         np.array([7]),
                         np.cumsum(rng.integers(0, 2 ** 33, size=300))]).astype(np.int64)
    ts[5] = ts[4] - 3  # a negative delta
    ti, tj = [], []
    for b, n in enumerate(lengths):
        s = offs[b]
        for _ in range(400):
            i = int(rng.integers(0, n))
            j = int(rng.integers(0, i + 1))
            ti.append(s + i)
            tj.append(s + j)
    ti, tj = np.array(ti, np.int64), np.array(tj, np.int64)
    for P, NT in [(256, 32), (128, 32), (7, 5), (1, 1), (1024, 64)]:
        pb, tb = binding.hstu_debug_buckets(to_dev(offs.astype(np.int32)), to_dev(ts), P, NT,
                                            to_dev(ti), to_dev(tj))
        torch.cuda.synchronize()
        pb, tb = pb.cpu().numpy(), tb.cpu().numpy()
        b_of = np.searchsorted(offs, ti, side="right") - 1
        for r in range(len(ti)):
            base = offs[b_of[r]]
            assert pb[r] == oracle.pos_bucket((ti[r] - base) - (tj[r] - base), P)
            assert tb[r] == oracle.time_bucket(int(ts[ti[r]]) - int(ts[tj[r]]), NT)


def test_prepass_key_norms_and_block_time_stats():
    """The bf16 forward's prepass outputs, read back from the workspace: per (32-key block, head)
    the largest squared norm of the block's key rows (fp32 sums of the bf16 squares, within 1e-5
    of the exact value, relative), and for the position + time bias each block's (min, max)
    timestamp at its first token and every token's time minus its block's minimum (exact
    integers).  300 users (more than 64: the row-to-user search takes two steps), among them
    empty, single-token and multi-block ones, and H = 3 (one head pair with a single head)."""
    rng = np.random.default_rng(21)
    lengths = rng.integers(0, 90, size=300)
    lengths[:6] = [0, 1, 32, 33, 700, 0]
    H = 3
    inp = _case("bf16", lengths.tolist(), H=H, d=64)
    dev = DevAttn(inp)
    B, T, ms = inp.B, inp.T, inp.max_seqlen
    ws = torch.zeros(binding.attn_workspace_bytes(B, H, ms, T), dtype=torch.uint8, device="cuda")
    dev.run(workspace=ws)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()

    def al(x):
        return (x + 255) // 256 * 256
    # regions: header + work list (32 B per item, 128-row tiles), TimeStat x T, int32 x T,
    # tile classes (8 B per row and column), key norms (4 B per row and head)
    rows = (T + 31 * B) // 32 + 1
    p_stats = 256 + al(B * H * ((ms + 127) // 128) * 32)
    p_rel = p_stats + al(16 * T)
    p_cls = p_rel + al(4 * T)
    p_kn = p_cls + al(rows * ((ms + 31) // 32) * 8)
    stats = w[p_stats:p_stats + 16 * T].view(np.int64).reshape(T, 2)
    rel = w[p_rel:p_rel + 4 * T].view(np.int32)
    kn = w[p_kn:p_kn + 4 * rows * H].view(np.float32).reshape(rows, H)
    offs = inp.offsets.astype(np.int64)
    k = inp.k.astype(np.float64)
    n_checked = 0
    for b in range(B):
        t0, n = int(offs[b]), int(offs[b + 1] - offs[b])
        row0 = (t0 + 31 * b) // 32
        for blk in range((n + 31) // 32):
            a, e = t0 + 32 * blk, t0 + min(32 * blk + 32, n)
            exact = np.max(np.sum(k[a:e] ** 2, axis=2), axis=0)  # [H]
            got = kn[row0 + blk].astype(np.float64)
            assert np.all(np.abs(got - exact) <= 1e-5 * exact), (b, blk, got, exact)
            tb = inp.ts[a:e]
            assert tuple(stats[a]) == (tb.min(), tb.max()), (b, blk)
            assert np.array_equal(rel[a:e], np.minimum(tb - tb.min(), 0x7fffffff)), (b, blk)
            n_checked += 1
    print("prepass: %d blocks of %d users, %d heads" % (n_checked, B, H), flush=True)


@pytest.mark.parametrize("B", [300, 5000])
def test_schedule_many_users_bit_exact(B):
    """The scheduler alone (hstu_attn_plan) on batches of more than 64 users (several ballot
    chunks per cost class) and of more than 4 096 (offsets read from global memory instead of
    LDS), with empty users and users longer than max_seqlen (cut at its tiles)."""
    rng = np.random.default_rng(B)
    lengths = rng.integers(0, 1200, size=B)
    lengths[rng.random(B) < 0.1] = 0
    lengths[:3] = [5000, 0, 1]
    ms, H = 1000, 3
    offs = synth.offsets_from_lengths(lengths)
    ws = torch.zeros(binding.attn_workspace_bytes(B, H, ms, int(offs[-1])), dtype=torch.uint8,
                     device="cuda")
    binding.hstu_attn_plan(binding.DTYPE_BF16, B, H, 64, to_dev(offs), ms, ws)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    count = int(w[:4].view(np.int32)[0])
    ref = schedule_reference(lengths, H, binding.attn_block_rows(binding.DTYPE_BF16, 64), ms)
    assert count == len(ref)
    items = w[256:256 + 32 * count].view(np.int32).reshape(count, 8)
    assert [tuple(x[:3]) for x in items] == ref
    b = items[:, 0]
    assert np.array_equal(items[:, 3], offs[b + 1].astype(np.int64) - offs[b])
    assert np.array_equal(items[:, 4:6].copy().view(np.int64)[:, 0], offs[b])


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 32)])
def test_schedule_bit_exact(dtype, d):
    lengths = [0, 1, 700, 256, 257, 1500, 3, 128, 129, 1024]
    H = 3
    inp = _case(dtype, lengths, H=H, d=d)
    dev = DevAttn(inp)
    ws = torch.zeros(binding.attn_workspace_bytes(inp.B, H, inp.max_seqlen, inp.T),
                     dtype=torch.uint8, device="cuda")
    dev.run(workspace=ws)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    count = int(w[:4].view(np.int32)[0])
    br = binding.attn_block_rows(binding.DTYPE_BF16 if dtype == "bf16" else binding.DTYPE_F32, d)
    ref = schedule_reference(lengths, H, br, inp.max_seqlen)
    assert count == len(ref)
    # 32-byte entries: b, h, q_tile, the user's length (int32), its first token (int64), pad
    items = w[256:256 + 32 * count].view(np.int32).reshape(count, 8)
    assert [tuple(x[:3]) for x in items] == ref
    offs = inp.offsets.astype(np.int64)
    b = items[:, 0]
    assert np.array_equal(items[:, 3], offs[b + 1] - offs[b])
    assert np.array_equal(items[:, 4:6].copy().view(np.int64)[:, 0], offs[b])


def test_validate_offsets_flags():
    offs = to_dev(np.array([0, 5, 3, 9], np.int32))
    f = binding.hstu_validate_offsets(offs, 10, 4)
    torch.cuda.synchronize()
    # decreasing (5 -> 3), offsets[B] != T (9 != 10), a length above 4 (5, 6)
    assert int(f.item()) == (2 | 4 | 8)
    ok = binding.hstu_validate_offsets(to_dev(np.array([0, 2, 2, 6], np.int32)), 6, 4)
    torch.cuda.synchronize()
    assert int(ok.item()) == 0
