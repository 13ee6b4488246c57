"""The attention forward without allocation (hstu_attn_fwd_noalloc: the workspace is the
library's static device array) against hstu_attn_fwd with a caller workspace, through the C ABI:
two calls in a row on one stream, the second with a smaller batch, each equal bit for bit (the
same kernels on the same inputs, every output element computed by one workgroup)."""
import numpy as np
import pytest
import torch

from hstu_sequential_transduction_jagged_amd import binding, synth
from tests.hstu_testutil import DevAttn

pytestmark = pytest.mark.gpu


def _case(name, seed, lengths, H, kind):
    return synth.make_attn(name, seed, "bf16", lengths, H=H, d=64, alpha=1.0 / 512,
                           P=128, NT=32, table_std=0.5, bias_kind=kind)


@pytest.mark.parametrize("kind", [synth.BIAS_RAB_PT, synth.BIAS_ALIBI])
def test_noalloc_equals_workspace_call_twice(kind):
    big = _case("noalloc_big", 70, [3000, 0, 1, 777, 2049, 64], 4, kind)
    small = _case("noalloc_small", 71, [5, 300, 129], 2, kind)
    for inp in (big, small):
        d = DevAttn(inp)
        ref = d.run()
        out = torch.full_like(ref, float("nan"))
        binding.hstu_attn_fwd_noalloc(d.q, d.k, d.v, d.offsets, inp.max_seqlen, out, d.bias,
                                      inp.alpha, inp.out_scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), inp.name
        print("%s: T=%d, noalloc output equals the workspace call" % (inp.name, inp.T), flush=True)
