"""GPU gradients of one HSTU layer ("Actions Speak Louder than Words" §3.1 eqs. (1)-(3)) against
the fp64 oracle, through the C ABI.

Where the error comes from.  The path keeps Z (U, V, Q, K) in bf16, hands the attention's SiLU
weights P to the matrix cores in bf16 (as multiples of ln(2)/2), stores O per (token, head) as
an fp32 offset plus bf16 deviations, and keeps G = LN(O) * U, dG, dZ and dZpre in bf16 between
its kernels.  The oracle's mirror mode (``oracle.layer_bwd(round_at=...)``) rounds exactly those
intermediates of the fp64 computation and nothing else, which measures how much error the
storage format alone causes.  Rounded one at a time (plain bf16 O, no P) on the f1-dX case below
(position + time bias, T = 1 306), the table gradients move by up to 0.10 (dw_pos) and 0.12
(dw_time) from dO's rounding alone, 0.05 / 0.065 from O's and 0.034 / 0.040 from Z's: they are
sums over ~10^5 pairs whose terms largely cancel (sum |g| is up to ~900 times the RMS of the
table gradient), so a relative perturbation of 2^-9 per term shows at the several-percent
level.  The path therefore
  - keeps dO to about 16 bits in the dO V^T product (the LayerNorm backward also writes the bf16
    remainder of dO and the dK/dV kernel adds its product), so dA, dK and the table gradients no
    longer see dO's rounding (dV and dQ still use bf16 dO);
  - stores O relative to each head row's mean, so O's rounding scales with the row's spread,
    which the LayerNorm divides by, not with its magnitude.
With the mirror rounding at the path's own points (Z, P, Oc, G, dG, dZ, dZpre) its errors match
the GPU's to within ~20 % on every gradient of these cases.
Bound: every gradient's max-abs error relative to the RMS of the exact fp64 gradient (dx, a
bf16 output, after its own rounding is allowed) must stay within max(2e-2, 2 e_m), where e_m is
the same metric for that mirror: the kernels' own arithmetic (fp32 summation order, bounded
SiLU expansions, bf16 dO in dV and dQ, bf16 G in dK) may add at most as much again.
Cases: ragged users (empty, single token, several 32/64/256-row tiles), with and without
residual, position + time bias and none, a case with enough tokens for the f1-kernel dX path,
a wider model (D = 512, H = 16), and the 8-layer stack's first layer at full size.
"""
import numpy as np
import pytest
import torch

import oracle
from hstu_sequential_transduction_jagged_amd import binding, synth
from tests.hstu_testutil import DevLayer, err_rms, err_stored, oracle_bias, to_dev

pytestmark = pytest.mark.gpu

FLOOR = 2e-2
MIRROR = ("Z", "P", "Oc", "G", "dG", "dZ", "dZpre")
NAMES = ("dx", "dw1", "db1", "dgamma", "dbeta", "dw2", "db2", "dw_pos", "dw_time")


def _gpu_bwd(inp, dY):
    d = DevLayer(inp)
    L = d.layers[0]
    ws = torch.empty(binding.layer_workspace_bytes(inp.B, inp.T, inp.D, inp.H, inp.dqk, inp.dv,
                                                   inp.max_seqlen), dtype=torch.uint8, device="cuda")
    d.run_layer(d.x, workspace=ws)
    got = binding.hstu_layer_bwd(d.x, d.offsets, inp.max_seqlen, L["w1"], L["b1"], L["gamma"],
                                 L["beta"], L["w2"], inp.H, inp.dqk, inp.dv, L["bias"], inp.alpha,
                                 inp.residual, inp.ln_eps, ws, to_dev(dY, torch.bfloat16))
    torch.cuda.synchronize()
    return {k: (None if v is None else v.float().cpu().numpy().astype(np.float64))
            for k, v in got.items()}


def _oracle_bwd(inp, dY, offsets=None, x=None, ts=None, round_at=()):
    P = inp.layers[0]
    offsets = inp.offsets if offsets is None else offsets
    x = inp.x if x is None else x
    ts = inp.ts if ts is None else ts
    return oracle.layer_bwd(offsets, x, P.w1, P.b1, P.gamma, P.beta, P.w2, P.b2,
                            oracle_bias(P.bias, ts, inp.H), inp.alpha, inp.H, inp.dqk, inp.dv, dY,
                            residual=inp.residual, ln_eps=inp.ln_eps, round_at=round_at)


def _compare(label, got, ref, mir, rows=None):
    for name in NAMES:
        if ref[name] is None:
            assert got[name] is None
            continue
        y = got[name] if rows is None or name != "dx" else got[name][rows]
        e = err_stored(y, ref[name], "bf16") if name == "dx" else err_rms(y, ref[name])
        em = err_rms(mir[name], ref[name])
        bound = max(FLOOR, 2.0 * em)
        print("%s %s err=%.3g (storage alone %.3g, bound %.3g)" % (label, name, e, em, bound),
              flush=True)
        assert e <= bound, (name, e, bound)


def _check(inp, seed=3):
    rng = np.random.default_rng(seed)
    dY = synth.round_bf16(rng.standard_normal((inp.T, inp.D)).astype(np.float32))
    got = _gpu_bwd(inp, dY)
    ref = _oracle_bwd(inp, dY)
    mir = _oracle_bwd(inp, dY, round_at=MIRROR)
    _compare(inp.name, got, ref, mir)


@pytest.mark.parametrize("residual", [False, True])
@pytest.mark.parametrize("kind", [synth.BIAS_RAB_PT, synth.BIAS_NONE])
def test_layer_bwd_ragged(kind, residual):
    inp = synth.make_layer("lbwd", 40, [0, 1, 33, 130, 300], D=256, H=2, d=64, alpha=1.0 / 64,
                           residual=residual, bias_kind=kind, P=64, NT=16, table_std=0.5,
                           randomize_affine=True)
    _check(inp)


@pytest.mark.parametrize("residual", [False, True])
def test_layer_bwd_enough_tokens_for_the_f1_dx_path(residual):
    # T H d_v >= D N1 (1 306 x 128 >= 256 x 512): dX = dZpre W1 (+ dY) runs on the f1 kernel with
    # W1^T staged in the freed dG buffer; position + time bias with tables of std 0.5
    inp = synth.make_layer("lbwd_f1dx", 43, [1, 300, 555, 450], D=256, H=2, d=64,
                           alpha=1.0 / 128, residual=residual, bias_kind=synth.BIAS_RAB_PT, P=64,
                           NT=16, table_std=0.5, randomize_affine=True)
    assert inp.T * inp.H * inp.dv >= inp.D * 2 * inp.H * (inp.dqk + inp.dv)
    _check(inp, seed=5)


def test_layer_bwd_wide():
    inp = synth.make_layer("lbwd_wide", 41, [70, 257], D=512, H=16, d=64, alpha=1.0 / 128,
                           residual=True, P=128, NT=32, table_std=0.2, randomize_affine=True)
    _check(inp, seed=4)


def test_layer_empty_batch():
    """Three empty users (T = 0, no timestamps): the forward returns an empty output and the
    backward's weight, bias, LayerNorm and table gradients, sums over no tokens, are zeros."""
    inp = synth.make_layer("lempty", 44, [0, 0, 0], D=256, H=2, d=64, alpha=1.0 / 64,
                           residual=True, bias_kind=synth.BIAS_RAB_PT, P=64, NT=16,
                           table_std=0.5, randomize_affine=True)
    d = DevLayer(inp)
    L = d.layers[0]
    ws = torch.empty(max(256, binding.layer_workspace_bytes(inp.B, inp.T, inp.D, inp.H, inp.dqk,
                                                            inp.dv, inp.max_seqlen)),
                     dtype=torch.uint8, device="cuda")
    y = d.run_layer(d.x, workspace=ws)
    got = binding.hstu_layer_bwd(d.x, d.offsets, inp.max_seqlen, L["w1"], L["b1"], L["gamma"],
                                 L["beta"], L["w2"], inp.H, inp.dqk, inp.dv, L["bias"], inp.alpha,
                                 inp.residual, inp.ln_eps, ws,
                                 torch.empty((0, inp.D), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert y.shape == (0, inp.D)
    assert got["dx"].shape == (0, inp.D)
    for name in NAMES[1:]:
        assert got[name] is not None and torch.all(got[name] == 0).item(), name


def test_layer_bwd_full_size_sampled_users():
    """The first layer of the 8-layer stack workload at its full size (128 users, T = 80 405,
    D = 512, H = 8, position + time bias, residual), forward and backward as the layer benchmark
    runs them, every kernel over the whole batch.  The upstream gradient is nonzero only on
    three sampled users (a median one, one cut to 1 024 rows by Stochastic Length, the longest,
    4 096 rows): users do not interact, so every gradient of the batch -- the weight, bias,
    LayerNorm and table gradients summed over all 80 405 tokens, and dX -- equals those three
    users' gradients, which the oracle computes on its own.  dX of every other user is exactly
    zero."""
    inp = synth.stack8(n_layers=1)
    lengths = np.diff(inp.offsets.astype(np.int64))
    order = np.argsort(lengths, kind="stable")
    picks = sorted({int(order[len(order) // 2]), int(np.argmin(np.abs(lengths - 1024))),
                    int(order[-1])})
    rows = np.concatenate([np.arange(inp.offsets[b], inp.offsets[b + 1]) for b in picks])
    rng = np.random.default_rng(12)
    dY = np.zeros((inp.T, inp.D), np.float32)
    dY[rows] = synth.round_bf16(rng.standard_normal((len(rows), inp.D)).astype(np.float32))
    got = _gpu_bwd(inp, dY)
    mask = np.ones(inp.T, bool)
    mask[rows] = False
    assert np.all(got["dx"][mask] == 0.0)
    offs = synth.offsets_from_lengths([int(lengths[b]) for b in picks])
    sub = dict(offsets=offs, x=inp.x[rows], ts=inp.ts[rows])
    ref = _oracle_bwd(inp, dY[rows], **sub)
    mir = _oracle_bwd(inp, dY[rows], round_at=MIRROR, **sub)
    _compare("stack8 layer 0, users %s (%s rows)" % (picks, [int(lengths[b]) for b in picks]),
             got, ref, mir, rows=rows)
