"""GPU parity of the full layer (eqs. (1)-(3)), the GenRank token construction and the
residual stack against the fp64 oracle, through the C ABI.  bf16 outputs: max error
<= 2e-2 of the reference RMS beyond each element's own bf16 rounding (err_stored)."""
import numpy as np
import pytest
import torch

import oracle
from hstu_sequential_transduction_jagged_amd import binding, synth
from tests.hstu_testutil import TOL, DevLayer, err_rms, err_stored, oracle_bias, oracle_layer, to_dev

pytestmark = pytest.mark.gpu


def _run_layer(inp, x=None, **kw):
    d = DevLayer(inp)
    xx = d.x if x is None else x
    y = d.run_layer(xx, **kw)
    torch.cuda.synchronize()
    return d, y


@pytest.mark.parametrize("affine", [False, True])
def test_layer_small_workload(affine):
    inp = synth.layer_small(randomize_affine=affine)
    d, y = _run_layer(inp)
    ref = oracle_layer(inp)
    yy = y.float().cpu().numpy()
    e = err_stored(yy, ref, "bf16")
    print("layer_small T=%d affine=%s err=%.3g (without storage allowance %.3g)"
          % (inp.T, affine, e, err_rms(yy, ref)), flush=True)
    assert e <= TOL["bf16"]


def test_layer_intermediates():
    """Z = SiLU(X W1^T + b1) with its U | V | Q | K blocks, and O (stored between the attention
    and the LayerNorm as a per (token, head) fp32 offset plus bf16 deviations), checked
    separately; the per-head statistics stored with O describe the represented values."""
    inp = synth.make_layer("t", 40, [0, 1, 300, 257, 64], D=256, H=4, d=64, alpha=1.0 / 300,
                           P=128, NT=32, table_std=0.5, randomize_affine=True)
    d = DevLayer(inp)
    ws = torch.zeros(binding.layer_workspace_bytes(inp.B, inp.T, 256, 4, 64, 64, inp.max_seqlen),
                     dtype=torch.uint8, device="cuda")
    y = d.run_layer(d.x, workspace=ws)
    torch.cuda.synchronize()
    zo, oo, so, _ = binding.layer_workspace_offsets(inp.T, 4, 64, 64)
    z = ws[zo:zo + inp.T * 1024 * 2].view(torch.bfloat16).view(inp.T, 1024).float().cpu().numpy()
    # O is stored per (token, head) as an fp32 offset (first of four statistics) + bf16 values
    dev = ws[oo:oo + inp.T * 256 * 2].view(torch.bfloat16).view(inp.T, 4, 64).float().cpu().numpy()
    st = ws[so:so + inp.T * 4 * 16].view(torch.float32).view(inp.T, 4, 4).cpu().numpy()
    o = (dev.astype(np.float64) + st[:, :, :1]).reshape(inp.T, 256)
    o3 = o.reshape(inp.T, 4, 64)
    mean = o3.mean(axis=2)
    np.testing.assert_allclose(st[:, :, 1], mean, rtol=0, atol=1e-6 * np.abs(o3).max())
    np.testing.assert_allclose(st[:, :, 2], ((o3 - mean[:, :, None]) ** 2).sum(axis=2), rtol=1e-4,
                               atol=1e-6 * (o3 ** 2).sum(axis=2).max())
    yr, zr, orf = oracle_layer(inp, return_intermediates=True)
    for name, a, r in [("U", z[:, :256], zr[:, :256]), ("V", z[:, 256:512], zr[:, 256:512]),
                       ("Q", z[:, 512:768], zr[:, 512:768]), ("K", z[:, 768:], zr[:, 768:]),
                       ("O", o, orf), ("Y", y.float().cpu().numpy(), yr)]:
        e = err_stored(a, r, "bf16")
        print(name, "err=%.3g (without storage allowance %.3g)" % (e, err_rms(a, r)), flush=True)
        assert e <= TOL["bf16"], name


def test_layer_residual_and_alibi():
    inp = synth.make_layer("t", 41, [200, 3, 129], D=512, H=8, d=64, alpha=1.0 / 200,
                           residual=True, bias_kind=synth.BIAS_ALIBI, randomize_affine=True)
    d, y = _run_layer(inp)
    e = err_stored(y.float().cpu().numpy(), oracle_layer(inp), "bf16")
    assert e <= TOL["bf16"], e


def test_embed_sum_exact():
    g = synth.genrank(B=3, lo=40, hi=90, n_items=2000)
    it = to_dev(g.item_table, torch.bfloat16)
    ac = to_dev(g.action_table, torch.bfloat16)
    ids = to_dev(g.item_ids.astype(np.int32))
    aids = to_dev(g.action_ids.astype(np.int32))
    x = binding.hstu_embed_sum_fwd(it, ac, ids, aids)
    torch.cuda.synchronize()
    # fp32 sum of the two bf16 rows, rounded once to bf16
    ref = (torch.from_numpy(g.item_table[g.item_ids]) + torch.from_numpy(g.action_table[g.action_ids])
           ).to(torch.bfloat16)
    assert torch.equal(x.cpu(), ref)
    ro = oracle.embed_sum(g.item_table, g.action_table, g.item_ids, g.action_ids)
    assert err_stored(x.float().cpu().numpy(), ro, "bf16") <= 1e-6


def test_genrank_layer_small():
    g = synth.genrank(B=4, lo=100, hi=600, n_items=5000, randomize_affine=True)
    it = to_dev(g.item_table, torch.bfloat16)
    ac = to_dev(g.action_table, torch.bfloat16)
    x = binding.hstu_embed_sum_fwd(it, ac, to_dev(g.item_ids.astype(np.int32)),
                                   to_dev(g.action_ids.astype(np.int32)))
    d = DevLayer(g)
    y = d.run_layer(x)
    torch.cuda.synchronize()
    # the layer's input is the bf16-stored token sum (checked bit-exact in test_embed_sum_exact);
    # the oracle takes the same rounding of its own fp64 sum
    xr = synth.round_bf16(oracle.embed_sum(g.item_table, g.action_table, g.item_ids,
                                           g.action_ids).astype(np.float32))
    ref = oracle_layer(g, x=xr)
    yy = y.float().cpu().numpy()
    e = err_stored(yy, ref, "bf16")
    print("genrank small T=%d err=%.3g (without storage allowance %.3g)" % (g.T, e, err_rms(yy, ref)),
          flush=True)
    assert e <= TOL["bf16"]



def test_genrank_full_size_sampled_users():
    """The GenRank configuration at its full size, as its benchmark runs it: 64 users of
    512..4096 events, tokens = item_emb[id] + action_emb[a] over 10^6 items (Zipf(1.1) ids) and
    4 actions, rows of 512; then one layer with the ALiBi bias (D = 512, H = 8, d = 64).  The
    token sums are compared bit for bit on every row with the fp32 sum of the two bf16 rows
    rounded once; the layer output on three users (the shortest, a median one, the longest)
    with the oracle run on those users alone (a layer acts on each user independently)."""
    g = synth.genrank(randomize_affine=True)
    it = to_dev(g.item_table, torch.bfloat16)
    ac = to_dev(g.action_table, torch.bfloat16)
    x = binding.hstu_embed_sum_fwd(it, ac, to_dev(g.item_ids.astype(np.int32)),
                                   to_dev(g.action_ids.astype(np.int32)))
    d = DevLayer(g)
    y = d.run_layer(x)
    torch.cuda.synchronize()
    xs = (torch.from_numpy(g.item_table[g.item_ids]) +
          torch.from_numpy(g.action_table[g.action_ids])).to(torch.bfloat16)
    assert torch.equal(x.cpu(), xs)
    print("genrank tokens: %d x %d bit-exact" % tuple(xs.shape), flush=True)
    xr = xs.float().numpy()
    del it, xs
    yy = y.float().cpu().numpy()
    lengths = np.diff(g.offsets.astype(np.int64))
    order = np.argsort(lengths, kind="stable")
    L = g.layers[0]
    for b in sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])}):
        s, e = int(g.offsets[b]), int(g.offsets[b + 1])
        ref = oracle.layer(np.array([0, e - s]), xr[s:e], L.w1, L.b1, L.gamma, L.beta, L.w2,
                           L.b2, oracle_bias(L.bias, g.ts[s:e], g.H), g.alpha, g.H, g.dqk, g.dv,
                           residual=g.residual, ln_eps=g.ln_eps)
        err = err_stored(yy[s:e], ref, "bf16")
        print("genrank user %d (%d rows): err=%.3g (without storage allowance %.3g)"
              % (b, e - s, err, err_rms(yy[s:e], ref)), flush=True)
        assert err <= TOL["bf16"], (b, err)


def test_stack_small():
    inp = synth.stack8(B=12, n_layers=3, hi=1500, randomize_affine=True)
    d = DevLayer(inp)
    h = d.x
    for li in range(len(inp.layers)):
        h = d.run_layer(h, li=li)
    torch.cuda.synchronize()
    x = inp.x.astype(np.float64)
    for li in range(len(inp.layers)):
        x = oracle_layer(inp, x=x, li=li)
    hh = h.float().cpu().numpy()
    e = err_stored(hh, x, "bf16")
    print("stack T=%d layers=%d err=%.3g (without storage allowance %.3g)"
          % (inp.T, len(inp.layers), e, err_rms(hh, x)), flush=True)
    assert e <= TOL["bf16"]



def _stack(d, fuse):
    inp = d.inp
    y = binding.hstu_stack_fwd(d.x, d.offsets, inp.max_seqlen, d.layers, inp.H, inp.dqk, inp.dv,
                               inp.alpha, inp.residual, inp.ln_eps, fuse_boundaries=fuse)
    torch.cuda.synchronize()
    return y


def test_stack_fused_boundaries_bitwise_and_oracle():
    """The layer stack entry point with the f2 / next-f1 boundary fused into one kernel
    ("Actions Speak Louder than Words" reading notes §3.5, the single operator between two
    attentions): its output equals the three-kernel stack bit for bit (the fused kernel takes
    f1's products in f1's order) and hstu_layer_fwd applied layer by layer, and is held to the
    oracle like test_stack_small (3 layers, 12 users with ragged 64-token tiles, residual)."""
    inp = synth.stack8(B=12, n_layers=3, hi=1500, randomize_affine=True)
    d = DevLayer(inp)
    y_fused = _stack(d, True)
    y_plain = _stack(d, False)
    h = d.x
    for li in range(len(inp.layers)):
        h = d.run_layer(h, li=li)
    torch.cuda.synchronize()
    assert torch.equal(y_fused, y_plain)
    assert torch.equal(y_plain, h)
    x = inp.x.astype(np.float64)
    for li in range(len(inp.layers)):
        x = oracle_layer(inp, x=x, li=li)
    yy = y_fused.float().cpu().numpy()
    e = err_stored(yy, x, "bf16")
    print("fused stack T=%d layers=%d err=%.3g (without storage allowance %.3g)"
          % (inp.T, len(inp.layers), e, err_rms(yy, x)), flush=True)
    assert e <= TOL["bf16"]


def test_stack_mixed_biases_reuses_plan_bitwise():
    """The stack entry point plans the batch once and keeps the tile classes while the layers'
    position + time bias keeps its timestamps and bucket counts.  Four layers whose biases are
    rab (P = 256, NT = 32), ALiBi, rab as the first, and rab with other bucket counts (P = 64,
    NT = 16: the classes are made again) give, fused and unfused, exactly what hstu_layer_fwd
    gives layer by layer."""
    inp = synth.stack8(B=12, n_layers=4, hi=1500, randomize_affine=True)
    d = DevLayer(inp)
    d.layers[1]["bias"] = binding.make_bias(binding.BIAS_ALIBI)
    rng = np.random.default_rng(21)
    d.layers[3]["bias"] = binding.make_bias(
        binding.BIAS_RAB_PT, d.ts,
        to_dev((rng.standard_normal(64) * 0.5).astype(np.float32)),
        to_dev((rng.standard_normal(16) * 0.5).astype(np.float32)))
    h = d.x
    for li in range(len(inp.layers)):
        h = d.run_layer(h, li=li)
    torch.cuda.synchronize()
    assert torch.equal(_stack(d, False), h)
    assert torch.equal(_stack(d, True), h)
    assert torch.isfinite(h.float()).all()


def test_stack8_full_size_all_layers_sampled_users():
    """The whole 8-layer stack at full size (128 users, T = 80 405, residual, position + time
    bias), fused and three-kernel boundaries giving identical bits, and its output checked on
    three sampled users (the shortest, a median one, the one cut to 1 024 rows by Stochastic
    Length): no layer mixes users, so the oracle runs the 8 layers on each user alone.
    Reference: the exact fp64 chain.  Rounding alone compounds over eight residual layers: the
    oracle with the path's storage points rounded (Z, P, O as offset + deviations, G, and every
    layer's Y, oracle.layer_mirror) already differs from the exact chain by up to ~0.04 on these
    users, so the bound is max(2e-2, 2 e_m) with e_m that mirror's error (the same convention as
    the layer backward's)."""
    inp = synth.stack8()
    d = DevLayer(inp)
    y = _stack(d, True)
    assert torch.equal(y, _stack(d, False))
    yy = y.float().cpu().numpy()
    lengths = np.diff(inp.offsets.astype(np.int64))
    order = np.argsort(lengths, kind="stable")
    for b in sorted({int(order[0]), int(order[len(order) // 2]),
                     int(np.argmin(np.abs(lengths - 1024)))}):
        s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
        ref = inp.x[s:e].astype(np.float64)
        mir = ref.copy()
        for L in inp.layers:
            bias = oracle_bias(L.bias, inp.ts[s:e], inp.H)
            args = (L.w1, L.b1, L.gamma, L.beta, L.w2, L.b2, bias, inp.alpha, inp.H, inp.dqk, inp.dv)
            ref = oracle.layer(np.array([0, e - s]), ref, *args, residual=inp.residual,
                               ln_eps=inp.ln_eps)
            mir = oracle.layer_mirror(np.array([0, e - s]), mir, *args, residual=inp.residual,
                                      ln_eps=inp.ln_eps, round_at=("Z", "P", "Oc", "G", "Y"))[0]
        err, em = err_stored(yy[s:e], ref, "bf16"), err_stored(mir, ref, "bf16")
        bound = max(TOL["bf16"], 2.0 * em)
        print("stack8, 8 layers, user %d (%d rows): err=%.3g (without storage allowance %.3g; "
              "storage rounding alone %.3g, bound %.3g)"
              % (b, e - s, err, err_rms(yy[s:e], ref), em, bound), flush=True)
        assert err <= bound, (b, err, bound)


@pytest.mark.parametrize("D,H", [(640, 12), (384, 2)])
def test_layer_uneven_widths(D, H):
    """Model widths whose f2 output is not a whole number of 512-feature chunks (640 = 512 + 128,
    384 = 3 x 128) and a LayerNorm width above 512 (H dv = 768), with residual; 380 tokens cover
    one full and one ragged 256-token f1 tile and six 64-token f2 tiles."""
    inp = synth.make_layer("t", 42 + H, [130, 250], D=D, H=H, d=64, alpha=1.0 / 250,
                           residual=True, randomize_affine=True)
    d, y = _run_layer(inp)
    yy = y.float().cpu().numpy()
    ref = oracle_layer(inp)
    e = err_stored(yy, ref, "bf16")
    print("layer D=%d H=%d err=%.3g (without storage allowance %.3g)" % (D, H, e, err_rms(yy, ref)),
          flush=True)
    assert e <= TOL["bf16"]


def test_stack_layer_full_size_sampled_users():
    """The first layer of the 8-layer stack workload at its full size (128 users, T = 80 405,
    D = 512, H = 8, position + time bias, residual), in the launch configuration the stack
    benchmark uses.  A layer acts on each user's rows independently, so the oracle recomputes it
    for four sampled users (the shortest, a median one, one cut to 1 024 rows by Stochastic
    Length and the longest, 4 096 rows) and their Y rows are compared with the GPU's."""
    inp = synth.stack8()
    d, y = _run_layer(inp)
    yy = y.float().cpu().numpy()
    lengths = np.diff(inp.offsets.astype(np.int64))
    order = np.argsort(lengths, kind="stable")
    picks = {int(order[0]), int(order[len(order) // 2]), int(np.argmin(np.abs(lengths - 1024))),
             int(order[-1])}
    L = inp.layers[0]
    for b in sorted(picks):
        s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
        ref = oracle.layer(np.array([0, e - s]), inp.x[s:e], L.w1, L.b1, L.gamma, L.beta, L.w2,
                           L.b2, oracle_bias(L.bias, inp.ts[s:e], inp.H), inp.alpha, inp.H,
                           inp.dqk, inp.dv, residual=inp.residual, ln_eps=inp.ln_eps)
        err = err_stored(yy[s:e], ref, "bf16")
        print("stack8 layer 0, user %d (%d rows): err=%.3g (without storage allowance %.3g)"
              % (b, e - s, err, err_rms(yy[s:e], ref)), flush=True)
        assert err <= TOL["bf16"], (b, err)
