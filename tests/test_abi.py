"""The C-ABI library loads on the host and exports every symbol include/hstu.h declares;
host-side argument checks answer without touching a GPU."""
import ctypes
import os
import re

import pytest

from hstu_sequential_transduction_jagged_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hstu.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hstu_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "hstu_attn_fwd" in names and "hstu_layer_fwd" in names
    L = binding.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(binding.SIGNATURES), set(names) ^ set(binding.SIGNATURES)


def test_status_strings():
    L = binding.lib()
    assert L.hstu_status_string(0) == b"ok"
    assert L.hstu_status_string(-3).startswith(b"workspace")
    assert L.hstu_status_string(12345) == b"unknown status"


def test_workspace_sizes():
    L = binding.lib()
    # 256-byte header + one 32-byte item per (user, head, 128-row tile), 256-aligned
    # + per-token timestamp statistics (16 B) and offsets (4 B), each region 256-aligned
    # + tile classes: 8 B per (query block row, key block), (T + 31 B) / 32 + 1 rows of
    #   ceil(max_seqlen / 32) entries
    # + key norm bounds: 4 B per (key block row, head), rows as the tile classes
    def al(x):
        return (x + 255) // 256 * 256

    def tclass(B, ms, T):
        return ((T + 31 * B) // 32 + 1) * ((ms + 31) // 32) * 8

    def knorm(B, H, T):
        return al(((T + 31 * B) // 32 + 1) * H * 4)
    assert L.hstu_attn_workspace_bytes(16, 8, 8192, 0) == \
        256 + 16 * 8 * 64 * 32 + tclass(16, 8192, 0) + knorm(16, 8, 0)
    assert L.hstu_attn_workspace_bytes(0, 8, 8192, 0) == 256 + tclass(0, 8192, 0) + knorm(0, 8, 0)
    assert L.hstu_attn_workspace_bytes(16, 8, 8192, 1000) == \
        256 + 16 * 8 * 64 * 32 + 16128 + 4096 + tclass(16, 8192, 1000) + knorm(16, 8, 1000)
    assert L.hstu_attn_block_rows(1, 64) == 128
    assert L.hstu_attn_block_rows(1, 32) == 128
    assert L.hstu_attn_block_rows(0, 32) == 128
    assert L.hstu_attn_block_rows(1, 48) == 0
    z, o, st, a = binding.layer_workspace_offsets(1000, 4, 64, 64)
    # Z | O | per (token, head) O statistics (4 fp32) | attention workspace, 256-byte aligned
    assert z == 0 and o == 1000 * 1024 * 2 and st == o + 1000 * 256 * 2 and a == st + 1000 * 4 * 16
    aw = L.hstu_attn_workspace_bytes(3, 4, 300, 1000)
    assert L.hstu_layer_workspace_bytes(3, 1000, 384, 4, 64, 64, 300) == a + (aw + 255) // 256 * 256


def _attn(**kw):
    L = binding.lib()
    args = dict(dt=1, B=2, H=2, dqk=64, dv=64, offsets=None, max_seqlen=16, T=20, q=None, qs=128,
                k=None, ks=128, v=None, vs=128, bias=None, alpha=1.0, out_scale=1.0, o=None,
                ws=None, wsb=0, stream=None)
    args.update(kw)
    return L.hstu_attn_fwd(args["dt"], args["B"], args["H"], args["dqk"], args["dv"],
                           args["offsets"], args["max_seqlen"], args["T"], args["q"], args["qs"],
                           args["k"], args["ks"], args["v"], args["vs"], args["bias"],
                           args["alpha"], args["out_scale"], args["o"], args["ws"], args["wsb"],
                           args["stream"])


def test_host_side_errors_need_no_gpu():
    L = binding.lib()
    assert _attn(dt=7) == -1
    assert _attn(H=0) == -1
    assert _attn(dqk=64, dv=32) == -2
    assert _attn(dt=1, dqk=48, dv=48) == -2      # head dims are 32 and 64
    assert _attn(dt=1, dqk=32, dv=32) == -1      # d = 32 is supported; null pointers
    assert _attn(max_seqlen=70000) == -2
    bad = binding.HstuBias()
    bad.kind = 9
    assert _attn(bias=ctypes.byref(bad)) == -1
    rab = binding.HstuBias()
    rab.kind = binding.BIAS_RAB_PT            # missing tables
    assert _attn(bias=ctypes.byref(rab)) == -1
    assert b"timestamps" in L.hstu_last_error()
    # empty problems return OK without launching anything
    assert _attn(B=0) == 0
    assert _attn(T=0) == 0
    # null pointers with work to do are rejected before any launch
    assert _attn() == -1
    fake = ctypes.c_void_p(0x100000)
    assert _attn(offsets=fake, q=fake, k=fake, v=fake, o=fake, ws=fake, wsb=16) == -3
    assert _attn(offsets=fake, q=fake, k=fake, v=fake, o=fake, ws=fake, wsb=1 << 20, qs=100) == -1
    assert _attn(offsets=fake, q=fake, k=fake, v=fake, o=fake, ws=ctypes.c_void_p(0x100010),
                 wsb=1 << 20) == -3
    # the forward in parts: same checks, no launches without work
    assert L.hstu_attn_prepare(7, 2, 2, 64, None, 16, 20, None, 128, None, None, 0, None) == -1
    assert L.hstu_attn_prepare(1, 0, 2, 64, None, 16, 20, None, 128, None, None, 0, None) == 0
    assert L.hstu_attn_prepare(1, 2, 2, 64, None, 16, 20, None, 128, None, None, 0, None) == -1
    assert L.hstu_attn_prepare(1, 2, 2, 64, fake, 16, 20, fake, 128, None, fake, 16, None) == -3
    assert L.hstu_attn_fwd_prepared(1, 2, 2, 64, 32, None, 16, 20, None, 128, None, 128, None,
                                    128, None, 1.0, 1.0, None, None, 0, None) == -2
    assert L.hstu_layer_fwd(0, 1, 256, 4, 64, 64, None, 8, 8, None, None, None, None, None, 1e-5,
                            None, None, None, 1.0, 0, None, None, 0, None) == -2
    assert L.hstu_layer_fwd(1, 1, 256, 4, 64, 64, None, 8, 8, None, None, None, None, None, 0.0,
                            None, None, None, 1.0, 0, None, None, 0, None) == -1
    assert L.hstu_embed_sum_fwd(4, 12, None, 1, None, 1, None, None, None, None) == -2
    # the layer stack: per-layer argument arrays required; the fused boundary needs d_model 512
    P2 = ctypes.c_void_p * 2
    nul = P2(None, None)
    bias_none = (ctypes.POINTER(binding.HstuBias) * 2)(ctypes.pointer(binding.make_bias(binding.BIAS_NONE)),
                                                       ctypes.pointer(binding.make_bias(binding.BIAS_NONE)))
    def stack(n=2, D=512, fuse=1, arrays=True, w=nul, bias=bias_none, B=1):
        a = (lambda v: v) if arrays else (lambda v: None)
        return L.hstu_stack_fwd(1, B, n, D, 8, 64, 64, None, 8, 8, None, a(w), a(nul), a(nul), a(nul),
                                1e-5, a(w), a(nul), a(bias), 1.0, 1, fuse, None, None, 0, None)
    assert stack(n=0) == -1
    assert stack(arrays=False) == -1
    assert stack(D=256) == -2
    assert stack(D=256, fuse=0) == -1          # null weights
    assert stack(w=P2(fake, fake), B=0) == 0   # no work
    assert stack(w=P2(fake, fake)) == -1       # null x / y / offsets
    assert L.hstu_stack_workspace_bytes(2, 100, 512, 8, 64, 64, 60) == (
        L.hstu_layer_workspace_bytes(2, 100, 512, 8, 64, 64, 60) + 2 * 102400)
    # candidate scoring: bf16 and d = 64 only; empty work is OK; strides and pointers checked
    def cand(dt=1, B=1, H=2, d=64, mh=8, mc=4, tc=4, p=None, s=128, s_h=128, ts=None):
        return L.hstu_attn_candidates_fwd(dt, B, H, d, d, p, mh, 100, p, mc, tc, p, s, p, s, p, s,
                                          p, s_h, p, s_h, None, ts, 1.0, 1.0, p, None, 0, None)
    assert cand(dt=0) == -2
    assert cand(d=32) == -2
    assert cand(tc=0) == 0 and cand(mc=0) == 0 and cand(B=0) == 0
    assert cand() == -1
    assert cand(p=fake, s=64) == -1                        # stride below H * d
    assert cand(p=ctypes.c_void_p(0x100008)) == -1         # rows not 16-byte aligned
    assert cand(p=fake, mh=1 << 20, s_h=1 << 12) == -2     # history past 32-bit offsets
    assert cand(p=fake, s=132) == -1                       # stride leaves rows misaligned
    assert cand(p=fake) == -3                              # no workspace
    ws = L.hstu_attn_candidates_workspace_bytes
    assert ws(3, 2, 1024, 0, 100) == 256 + 256            # unit list header + 6 entries
    assert ws(3, 2, 1024, 100, 100) == 1792 + 512 + 256 + 256
    assert ws(1, 2, 1025, 0, 100) == 2 * 100 * 2 * 64 * 4 + 256 + 256
    assert ws(16, 8, 8192, 37425, 16384) == \
        8 * 16384 * 8 * 64 * 4 + 599040 + 149760 + 256 + 4096


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="libhstu.so not found"):
        binding.lib()


def test_noalloc_rejects_batches_beyond_its_scratch():
    """The no-allocation attention (a 32 MiB static workspace) refuses, before anything is
    enqueued, a batch whose workspace would exceed it: one user of 65 536 rows needs tile
    classes of (65 536 / 32 + 1) x 2 048 x 8 bytes alone."""
    L = binding.lib()
    need = L.hstu_attn_workspace_bytes(1, 1, 65536, 65536)
    assert need > 32 << 20
    st = L.hstu_attn_fwd_noalloc(1, 1, 1, 64, 64, None, 65536, 65536, None, 64, None, 64, None,
                                 64, None, 1.0, 1.0, None, None)
    assert st == -2
    assert b"no-allocation" in L.hstu_last_error()
