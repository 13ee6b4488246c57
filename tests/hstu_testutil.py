"""Shared helpers of the tests: device copies of synthetic inputs, the error metric,
and oracle calls on the same inputs."""
import numpy as np
import torch

import oracle
from hstu_sequential_transduction_jagged_amd import binding, synth

TOL = {"f32": 1e-4, "bf16": 2e-2}

# Unit roundoff of the output storage format: |RNE(x) - x| <= u |x|.  bf16 keeps 8
# significant bits, so u = 2^-8.
UNIT_ROUNDOFF = {"f32": 0.0, "bf16": 2.0 ** -8}


def err_rms(y, ref):
    """max_k |y_k - ref_k| / sqrt(mean_k ref_k^2) over the whole tensor."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(y - ref)) / max(rms, 1e-300))


def err_stored(y, ref, dtype):
    """The parity metric for an output stored in `dtype`:
        max_k max(0, |y_k - ref_k| - u |ref_k|) / sqrt(mean_k ref_k^2),
    i.e. the max-abs error relative to the reference RMS after allowing each element the
    rounding of its own storage format (u = 2^-8 for bf16, 0 for fp32).  The exact
    result rounded to nearest in the output format scores 0; without the allowance it
    alone scores about 0.02 on bf16 tensors with max/rms of 5-8."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(ref * ref))
    ex = np.maximum(np.abs(y - ref) - UNIT_ROUNDOFF[dtype] * np.abs(ref), 0.0)
    return float(np.max(ex) / max(rms, 1e-300))


def torch_dtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_dev(a, dtype=None, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device=device, dtype=dtype) if dtype is not None else t.to(device)


def oracle_bias(spec: synth.BiasSpec, ts, H):
    if spec.kind == synth.BIAS_RAB_PT:
        return oracle.Bias(oracle.BIAS_RAB_PT, ts, spec.w_pos, spec.w_time)
    if spec.kind == synth.BIAS_ALIBI:
        slopes = spec.slopes if spec.slopes is not None else oracle.alibi_slopes(H)
        return oracle.Bias(oracle.BIAS_ALIBI, slopes=slopes)
    return oracle.Bias(oracle.BIAS_NONE)


def device_bias(spec: synth.BiasSpec, ts_dev, device="cuda"):
    if spec.kind == synth.BIAS_RAB_PT:
        return binding.make_bias(binding.BIAS_RAB_PT, ts_dev, to_dev(spec.w_pos, device=device),
                                 to_dev(spec.w_time, device=device))
    if spec.kind == synth.BIAS_ALIBI:
        sl = None if spec.slopes is None else to_dev(spec.slopes.astype(np.float32), device=device)
        return binding.make_bias(binding.BIAS_ALIBI, alibi_slopes=sl)
    return binding.make_bias(binding.BIAS_NONE)


class DevAttn:
    """Device copies of an AttnInputs case."""

    def __init__(self, inp: synth.AttnInputs, device="cuda"):
        dt = torch_dtype(inp.dtype)
        self.inp = inp
        self.q = to_dev(inp.q, dt, device)
        self.k = to_dev(inp.k, dt, device)
        self.v = to_dev(inp.v, dt, device)
        self.offsets = to_dev(inp.offsets.astype(np.int32), device=device)
        self.ts = to_dev(inp.ts.astype(np.int64), device=device)
        self.bias = device_bias(inp.bias, self.ts, device)

    def run(self, **kw):
        o = binding.hstu_attn_fwd(self.q, self.k, self.v, self.offsets, self.inp.max_seqlen,
                                  self.bias, self.inp.alpha, self.inp.out_scale, **kw)
        return o


def run_attn(inp, **kw):
    d = DevAttn(inp)
    o = d.run(**kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64)


def oracle_attn(inp: synth.AttnInputs):
    return oracle.attention(inp.offsets, inp.q, inp.k, inp.v, oracle_bias(inp.bias, inp.ts, inp.H),
                            inp.alpha, inp.out_scale)


def oracle_attn_rows(inp: synth.AttnInputs, tokens, heads):
    return oracle.attention_rows(inp.offsets, inp.q, inp.k, inp.v,
                                 oracle_bias(inp.bias, inp.ts, inp.H), inp.alpha, tokens, heads,
                                 inp.out_scale)


class DevCand:
    """Device copies of a CandInputs case (bf16)."""

    def __init__(self, inp: synth.CandInputs, device="cuda"):
        bf = torch.bfloat16
        self.inp = inp
        self.qc, self.kc, self.vc = (to_dev(a, bf, device) for a in (inp.qc, inp.kc, inp.vc))
        self.kh, self.vh = to_dev(inp.kh, bf, device), to_dev(inp.vh, bf, device)
        self.ho = to_dev(inp.hist_offsets.astype(np.int32), device=device)
        self.co = to_dev(inp.cand_offsets.astype(np.int32), device=device)
        self.ts_h = to_dev(inp.ts_h.astype(np.int64), device=device)
        self.ts_c = to_dev(inp.ts_c.astype(np.int64), device=device)
        self.bias = device_bias(inp.bias, self.ts_h, device)

    def run(self, **kw):
        i = self.inp
        return binding.hstu_attn_candidates_fwd(self.qc, self.kc, self.vc, self.co, i.max_cand,
                                                self.kh, self.vh, self.ho, i.max_hist, self.bias,
                                                self.ts_c, i.alpha, i.out_scale, **kw)


def oracle_cand(inp: synth.CandInputs):
    return oracle.attention_candidates(inp.hist_offsets, inp.cand_offsets, inp.qc, inp.kc, inp.vc,
                                       inp.kh, inp.vh, oracle_bias(inp.bias, inp.ts_h, inp.H),
                                       inp.ts_c, inp.alpha, inp.out_scale)


class DevLayer:
    """Device copies of a LayerInputs case (one or more layers)."""

    def __init__(self, inp: synth.LayerInputs, device="cuda"):
        self.inp = inp
        bf = torch.bfloat16
        self.offsets = to_dev(inp.offsets.astype(np.int32), device=device)
        self.ts = to_dev(inp.ts.astype(np.int64), device=device)
        self.x = None if inp.x is None else to_dev(inp.x, bf, device)
        self.layers = []
        for L in inp.layers:
            self.layers.append(dict(
                w1=to_dev(L.w1, bf, device), b1=to_dev(L.b1, device=device),
                gamma=to_dev(L.gamma, device=device), beta=to_dev(L.beta, device=device),
                w2=to_dev(L.w2, bf, device), b2=to_dev(L.b2, device=device),
                bias=device_bias(L.bias, self.ts, device)))

    def run_layer(self, x, li=0, residual=None, **kw):
        L = self.layers[li]
        inp = self.inp
        return binding.hstu_layer_fwd(x, self.offsets, inp.max_seqlen, L["w1"], L["b1"],
                                      L["gamma"], L["beta"], L["w2"], L["b2"], inp.H, inp.dqk,
                                      inp.dv, L["bias"], inp.alpha,
                                      inp.residual if residual is None else residual,
                                      inp.ln_eps, **kw)


def oracle_layer(inp: synth.LayerInputs, x=None, li=0, residual=None, **kw):
    L = inp.layers[li]
    return oracle.layer(inp.offsets, inp.x if x is None else x, L.w1, L.b1, L.gamma, L.beta, L.w2,
                        L.b2, oracle_bias(L.bias, inp.ts, inp.H), inp.alpha, inp.H, inp.dqk,
                        inp.dv, residual=inp.residual if residual is None else residual,
                        ln_eps=inp.ln_eps, **kw)


def schedule_reference(lengths, H, block_rows, max_seqlen):
    """The scheduler's list order written out on the host: cost (= q_tile + 1) descending,
    then user, then head ascending; users longer than max_seqlen are cut at its tiles."""
    max_tiles = -(-max_seqlen // block_rows)
    ntiles = [min(-(-int(n) // block_rows), max_tiles) if n > 0 else 0 for n in lengths]
    items = []
    for c in range(max_tiles, 0, -1):
        for b, m in enumerate(ntiles):
            if m >= c:
                for h in range(H):
                    items.append((b, h, c - 1))
    return items
