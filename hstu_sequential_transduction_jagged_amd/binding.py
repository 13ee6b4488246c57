"""ctypes binding of libhstu (declared in include/hstu.h).

Argument marshalling only: tensors are PyTorch device tensors, their data
pointers and the current HIP stream are passed through the C ABI, and every
step of the computation runs in the library's kernels.  Workspaces are
allocated here with PyTorch (the library itself never allocates).  If the
shared library is missing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhstu.so")

DTYPE_F32, DTYPE_BF16, DTYPE_BF16_OUT_F32 = 0, 1, 2
BIAS_NONE, BIAS_RAB_PT, BIAS_ALIBI = 0, 1, 2

_P = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class HstuBias(ctypes.Structure):
    _fields_ = [("kind", _i32), ("timestamps", _P), ("w_pos", _P), ("w_time", _P),
                ("num_pos_buckets", _i32), ("num_time_buckets", _i32),
                ("pos_head_stride", _i32), ("time_head_stride", _i32), ("alibi_slopes", _P)]


# name -> (restype, argtypes)
SIGNATURES = {
    "hstu_attn_workspace_bytes": (_sz, [_i32, _i32, _i32, _i64]),
    "hstu_attn_fwd": (_i32, [_i32, _i32, _i32, _i32, _i32, _P, _i32, _i64, _P, _i64, _P, _i64, _P,
                             _i64, ctypes.POINTER(HstuBias), _f32, _f32, _P, _P, _sz, _P]),
    "hstu_attn_fwd_noalloc": (_i32, [_i32, _i32, _i32, _i32, _i32, _P, _i32, _i64, _P, _i64, _P,
                                     _i64, _P, _i64, ctypes.POINTER(HstuBias), _f32, _f32, _P,
                                     _P]),
    "hstu_attn_block_rows": (_i32, [_i32, _i32]),
    "hstu_attn_plan": (_i32, [_i32, _i32, _i32, _i32, _P, _i32, _P, _sz, _P]),
    "hstu_attn_fwd_planned": (_i32, [_i32, _i32, _i32, _i32, _i32, _P, _i32, _i64, _P, _i64, _P,
                                     _i64, _P, _i64, ctypes.POINTER(HstuBias), _f32, _f32, _P, _P,
                                     _sz, _P]),
    "hstu_attn_prepare": (_i32, [_i32, _i32, _i32, _i32, _P, _i32, _i64, _P, _i64,
                                 ctypes.POINTER(HstuBias), _P, _sz, _P]),
    "hstu_attn_fwd_prepared": (_i32, [_i32, _i32, _i32, _i32, _i32, _P, _i32, _i64, _P, _i64, _P,
                                      _i64, _P, _i64, ctypes.POINTER(HstuBias), _f32, _f32, _P, _P,
                                      _sz, _P]),
    "hstu_attn_bwd": (_i32, [_i32, _i32, _i32, _i32, _i32, _P, _i32, _i64, _P, _i64, _P, _i64, _P,
                             _i64, _P, _i64, ctypes.POINTER(HstuBias), _f32, _f32, _P, _P, _P, _P,
                             _P, _P, _sz, _P]),
    "hstu_layer_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32, _i32]),
    "hstu_layer_fwd": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _P, _i32, _i64, _P, _P, _P, _P,
                              _P, _f32, _P, _P, ctypes.POINTER(HstuBias), _f32, _i32, _P, _P, _sz,
                              _P]),
    "hstu_stack_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32, _i32]),
    "hstu_stack_fwd": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _P, _i32, _i64, _P, _P, _P,
                              _P, _P, _f32, _P, _P, _P, _f32, _i32, _i32, _P, _P, _sz, _P]),
    "hstu_layer_workspace_offsets": (None, [_i64, _i32, _i32, _i32, ctypes.POINTER(_sz),
                                            ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                            ctypes.POINTER(_sz)]),
    "hstu_attn_candidates_fwd": (_i32, [_i32, _i32, _i32, _i32, _i32, _P, _i32, _i64, _P, _i32,
                                        _i64, _P, _i64, _P, _i64, _P, _i64, _P, _i64, _P, _i64,
                                        ctypes.POINTER(HstuBias), _P, _f32, _f32, _P, _P, _sz,
                                        _P]),
    "hstu_attn_candidates_workspace_bytes": (_sz, [_i32, _i32, _i32, _i64, _i64]),
    "hstu_layer_bwd": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _P, _i32, _i64, _P, _P, _P, _P, _P,
                              _f32, _P, ctypes.POINTER(HstuBias), _f32, _i32, _P, _P, _P, _P, _P,
                              _P, _P, _P, _P, _P, _P, _P, _sz, _P]),
    "hstu_layer_bwd_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32]),
    "hstu_stochastic_length": (_i32, [_i32, _P, _i32, _i64, _i32, ctypes.c_double, _P, _P, _P,
                                      _i64, _P, _P, _P, _P, _P, _P, _sz, _P]),
    "hstu_stochastic_length_workspace_bytes": (_sz, [_i32, _i64]),
    "hstu_embed_sum_fwd": (_i32, [_i64, _i32, _P, _i64, _P, _i32, _P, _P, _P, _P]),
    "hstu_validate_offsets": (_i32, [_i32, _P, _i64, _i32, _P, _P]),
    "hstu_debug_buckets": (_i32, [_i32, _P, _P, _i32, _i32, _i64, _P, _P, _P, _P, _P]),
    "hstu_status_string": (ctypes.c_char_p, [_i32]),
    "hstu_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """Load libhstu.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libhstu.so not found at %s: build it with "
                               "hstu_sequential_transduction_jagged_amd/build.py" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class HstuError(RuntimeError):
    pass


def _check(name, status):
    if status != 0:
        L = lib()
        raise HstuError("%s failed: %s (%s)" % (name, L.hstu_status_string(status).decode(),
                                                L.hstu_last_error().decode()))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise HstuError("unsupported dtype %s" % t.dtype)


def make_bias(kind=BIAS_NONE, timestamps=None, w_pos=None, w_time=None, alibi_slopes=None):
    """Build the hstu_bias struct from device tensors.  w_pos/w_time may be [P] (shared
    across heads) or [H, P] (per head)."""
    b = HstuBias()
    b.kind = kind
    keep = []
    if kind == BIAS_RAB_PT:
        for t in (timestamps, w_pos, w_time):
            if t is None or not t.is_cuda:
                raise HstuError("rab_pt bias needs device timestamps, w_pos and w_time")
        if timestamps.dtype != torch.int64 or w_pos.dtype != torch.float32 or \
                w_time.dtype != torch.float32:
            raise HstuError("timestamps must be int64, tables float32")
        w_pos, w_time, timestamps = w_pos.contiguous(), w_time.contiguous(), timestamps.contiguous()
        b.timestamps, b.w_pos, b.w_time = _ptr(timestamps), _ptr(w_pos), _ptr(w_time)
        b.num_pos_buckets = w_pos.shape[-1]
        b.num_time_buckets = w_time.shape[-1]
        b.pos_head_stride = w_pos.shape[-1] if w_pos.dim() == 2 else 0
        b.time_head_stride = w_time.shape[-1] if w_time.dim() == 2 else 0
        keep = [timestamps, w_pos, w_time]
    elif kind == BIAS_ALIBI:
        if alibi_slopes is not None:
            alibi_slopes = alibi_slopes.contiguous()
            if alibi_slopes.dtype != torch.float32:
                raise HstuError("alibi slopes must be float32")
            b.alibi_slopes = _ptr(alibi_slopes)
            keep = [alibi_slopes]
    b._keep = keep  # keep tensors alive as long as the struct
    return b


def attn_workspace_bytes(B, H, max_seqlen, total_tokens):
    return int(lib().hstu_attn_workspace_bytes(B, H, max_seqlen, total_tokens))


def attn_block_rows(dtype_code, d):
    return int(lib().hstu_attn_block_rows(dtype_code, d))


def _rows(t: torch.Tensor, name: str):
    """[T, H, d] tensor (possibly a strided view) -> (row stride, H, d)."""
    if t.dim() == 3 and t.numel() == 0:
        return t.shape[1] * t.shape[2], t.shape[1], t.shape[2]
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise HstuError("%s must be [T, H, d] with contiguous heads" % name)
    return t.stride(0), t.shape[1], t.shape[2]


def hstu_attn_fwd(q, k, v, offsets, max_seqlen, bias: Optional[HstuBias] = None, alpha=1.0,
                  out_scale=1.0, out=None, workspace=None, out_f32=False):
    """Jagged causal pointwise attention.  q, k, v: [T, H, d] device tensors (bf16 or fp32,
    row-strided views allowed); offsets: int32 [B+1] on the device.  Returns o [T, H, d]
    (fp32 when out_f32 is set for bf16 inputs)."""
    if not q.is_cuda:
        raise HstuError("inputs must be device tensors")
    dt = _dtype_code(q)
    if out_f32:
        if dt != DTYPE_BF16:
            raise HstuError("out_f32 needs bf16 inputs")
        dt = DTYPE_BF16_OUT_F32
    qs, H, d = _rows(q, "q")
    ks, _, _ = _rows(k, "k")
    vs, _, dv = _rows(v, "v")
    T = q.shape[0]
    B = offsets.numel() - 1
    if offsets.dtype != torch.int32:
        raise HstuError("offsets must be int32")
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.float32 if out_f32 else q.dtype,
                          device=q.device)
    need = attn_workspace_bytes(B, H, max_seqlen, T)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    bias = bias if bias is not None else make_bias(BIAS_NONE)
    st = lib().hstu_attn_fwd(dt, B, H, d, dv, _ptr(offsets), int(max_seqlen), T, _ptr(q), qs,
                             _ptr(k), ks, _ptr(v), vs, ctypes.byref(bias), float(alpha),
                             float(out_scale), _ptr(out), _ptr(workspace), workspace.numel(),
                             _stream(q.device))
    _check("hstu_attn_fwd", st)
    return out


def hstu_attn_fwd_noalloc(q, k, v, offsets, max_seqlen, out, bias: Optional[HstuBias] = None,
                          alpha=1.0, out_scale=1.0):
    """hstu_attn_fwd without a workspace argument (the library's static device scratch); the
    caller passes the output tensor."""
    if not q.is_cuda or not out.is_cuda:
        raise HstuError("inputs and output must be device tensors")
    dt = _dtype_code(q)
    if out.dtype == torch.float32 and dt == DTYPE_BF16:
        dt = DTYPE_BF16_OUT_F32
    qs, H, d = _rows(q, "q")
    ks, _, _ = _rows(k, "k")
    vs, _, dv = _rows(v, "v")
    if offsets.dtype != torch.int32:
        raise HstuError("offsets must be int32")
    bias = bias if bias is not None else make_bias(BIAS_NONE)
    st = lib().hstu_attn_fwd_noalloc(dt, offsets.numel() - 1, H, d, dv, _ptr(offsets),
                                     int(max_seqlen), q.shape[0], _ptr(q), qs, _ptr(k), ks,
                                     _ptr(v), vs, ctypes.byref(bias), float(alpha),
                                     float(out_scale), _ptr(out), _stream(q.device))
    _check("hstu_attn_fwd_noalloc", st)
    return out


def hstu_attn_plan(dtype_code, B, H, d, offsets, max_seqlen, workspace):
    """Run the jagged scheduler only, writing the work list into `workspace`."""
    st = lib().hstu_attn_plan(dtype_code, B, H, d, _ptr(offsets), int(max_seqlen), _ptr(workspace),
                              workspace.numel(), _stream(workspace.device))
    _check("hstu_attn_plan", st)
    return workspace


def hstu_attn_prepare(k, offsets, max_seqlen, workspace, bias=None, T=None):
    """The per-batch prepasses of the attention (key norm bounds; timestamp statistics and tile
    classes of the position + time bias) into `workspace`, after hstu_attn_plan."""
    dt = _dtype_code(k)
    ks, H, d = _rows(k, "k")
    T = k.shape[0] if T is None else T
    B = offsets.numel() - 1
    bias = bias if bias is not None else make_bias(BIAS_NONE)
    st = lib().hstu_attn_prepare(dt, B, H, d, _ptr(offsets), int(max_seqlen), T, _ptr(k), ks,
                                 ctypes.byref(bias), _ptr(workspace), workspace.numel(),
                                 _stream(k.device))
    _check("hstu_attn_prepare", st)


def hstu_attn_fwd_prepared(q, k, v, offsets, max_seqlen, workspace, bias=None, alpha=1.0,
                           out_scale=1.0, out=None):
    """The attention kernel alone, on a workspace that hstu_attn_plan and hstu_attn_prepare
    filled."""
    return hstu_attn_fwd_planned(q, k, v, offsets, max_seqlen, workspace, bias, alpha, out_scale,
                                 out, _entry="hstu_attn_fwd_prepared")


def hstu_attn_fwd_planned(q, k, v, offsets, max_seqlen, workspace, bias=None, alpha=1.0,
                          out_scale=1.0, out=None, _entry="hstu_attn_fwd_planned"):
    """Attention on a work list that hstu_attn_plan wrote into `workspace`."""
    dt = _dtype_code(q)
    qs, H, d = _rows(q, "q")
    ks, _, _ = _rows(k, "k")
    vs, _, dv = _rows(v, "v")
    T = q.shape[0]
    B = offsets.numel() - 1
    if out is None:
        out = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    bias = bias if bias is not None else make_bias(BIAS_NONE)
    st = getattr(lib(), _entry)(dt, B, H, d, dv, _ptr(offsets), int(max_seqlen), T, _ptr(q), qs,
                                _ptr(k), ks, _ptr(v), vs, ctypes.byref(bias), float(alpha),
                                float(out_scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                _stream(q.device))
    _check(_entry, st)
    return out


def layer_workspace_bytes(B, T, D, H, dqk, dv, max_seqlen):
    return int(lib().hstu_layer_workspace_bytes(B, T, D, H, dqk, dv, max_seqlen))


def layer_workspace_offsets(T, H, dqk, dv):
    """Byte offsets of Z, O, the O statistics and the attention workspace in the layer
    workspace."""
    z, o, st, a = _sz(), _sz(), _sz(), _sz()
    lib().hstu_layer_workspace_offsets(T, H, dqk, dv, ctypes.byref(z), ctypes.byref(o),
                                       ctypes.byref(st), ctypes.byref(a))
    return z.value, o.value, st.value, a.value


def hstu_layer_fwd(x, offsets, max_seqlen, w1, b1, ln_gamma, ln_beta, w2, b2, H, dqk, dv,
                   bias: Optional[HstuBias] = None, alpha=1.0, residual=False, ln_eps=1e-5,
                   out=None, workspace=None):
    """One HSTU layer forward (bf16).  x: [T, D]; w1: [2H(dqk+dv), D]; w2: [D, H dv];
    b1, b2, ln_gamma, ln_beta: fp32 or None.  Returns y [T, D]."""
    if x.dtype != torch.bfloat16:
        raise HstuError("the layer runs in bf16")
    T, D = x.shape
    B = offsets.numel() - 1
    if out is None:
        out = torch.empty((T, D), dtype=x.dtype, device=x.device)
    need = layer_workspace_bytes(B, T, D, H, dqk, dv, max_seqlen)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    bias = bias if bias is not None else make_bias(BIAS_NONE)
    for name, t in (("x", x), ("w1", w1), ("w2", w2), ("b1", b1), ("b2", b2),
                    ("ln_gamma", ln_gamma), ("ln_beta", ln_beta)):
        if t is not None and not t.is_contiguous():
            raise HstuError("%s must be contiguous" % name)
    st = lib().hstu_layer_fwd(DTYPE_BF16, B, D, H, dqk, dv, _ptr(offsets), int(max_seqlen), T,
                              _ptr(x), _ptr(w1), _ptr(b1),
                              _ptr(ln_gamma), _ptr(ln_beta), float(ln_eps), _ptr(w2),
                              _ptr(b2), ctypes.byref(bias), float(alpha), int(bool(residual)),
                              _ptr(out), _ptr(workspace), workspace.numel(), _stream(x.device))
    _check("hstu_layer_fwd", st)
    return out


def stack_workspace_bytes(B, T, D, H, dqk, dv, max_seqlen):
    return int(lib().hstu_stack_workspace_bytes(B, T, D, H, dqk, dv, max_seqlen))


def hstu_stack_fwd(x, offsets, max_seqlen, layers, H, dqk, dv, alpha=1.0, residual=False,
                   ln_eps=1e-5, fuse_boundaries=False, out=None, workspace=None):
    """A stack of HSTU layers (bf16).  layers: a list of dicts with w1, b1, gamma, beta, w2, b2
    (device tensors or None as for hstu_layer_fwd) and bias (HstuBias or None).  With
    fuse_boundaries, each f2 and the next layer's f1 run as one kernel (d_model = 512).
    Returns y [T, D]."""
    if x.dtype != torch.bfloat16:
        raise HstuError("the layer runs in bf16")
    T, D = x.shape
    B = offsets.numel() - 1
    n = len(layers)
    if out is None:
        out = torch.empty((T, D), dtype=x.dtype, device=x.device)
    need = stack_workspace_bytes(B, T, D, H, dqk, dv, max_seqlen)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    biases = [L.get("bias") if L.get("bias") is not None else make_bias(BIAS_NONE) for L in layers]
    for L in layers:
        for name in ("w1", "w2", "b1", "b2", "gamma", "beta"):
            t = L.get(name)
            if t is not None and not t.is_contiguous():
                raise HstuError("%s must be contiguous" % name)
    arr = lambda key: (_P * n)(*[_ptr(L.get(key)) for L in layers])
    bias_arr = (ctypes.POINTER(HstuBias) * n)(*[ctypes.pointer(b) for b in biases])
    st = lib().hstu_stack_fwd(DTYPE_BF16, B, n, D, H, dqk, dv, _ptr(offsets), int(max_seqlen), T,
                              _ptr(x), arr("w1"), arr("b1"), arr("gamma"), arr("beta"),
                              float(ln_eps), arr("w2"), arr("b2"), bias_arr, float(alpha),
                              int(bool(residual)), int(bool(fuse_boundaries)), _ptr(out),
                              _ptr(workspace), workspace.numel(), _stream(x.device))
    _check("hstu_stack_fwd", st)
    return out


def hstu_attn_candidates_fwd(q_cand, k_cand, v_cand, cand_offsets, max_cand, k_hist, v_hist,
                             hist_offsets, max_hist, bias: Optional[HstuBias] = None,
                             cand_timestamps=None, alpha=1.0, out_scale=1.0, out=None,
                             workspace=None):
    """Candidate scoring over a cached history (bf16, d = 64): every candidate of user b sees
    the user's history and itself.  q/k/v_cand: [Tc, H, 64]; k/v_hist: [Th, H, 64] (row-strided
    views allowed); offsets int32 [B+1] on the device; bias.timestamps are the history's and
    cand_timestamps the candidates'.  Returns o [Tc, H, 64]."""
    if q_cand.dtype != torch.bfloat16:
        raise HstuError("candidate scoring runs in bf16")
    qs, H, d = _rows(q_cand, "q_cand")
    kcs, _, _ = _rows(k_cand, "k_cand")
    vcs, _, dv = _rows(v_cand, "v_cand")
    khs, _, _ = _rows(k_hist, "k_hist")
    vhs, _, _ = _rows(v_hist, "v_hist")
    Tc = q_cand.shape[0]
    B = cand_offsets.numel() - 1
    if hist_offsets.numel() != B + 1:
        raise HstuError("hist_offsets and cand_offsets must have the same length")
    if cand_offsets.dtype != torch.int32 or hist_offsets.dtype != torch.int32:
        raise HstuError("offsets must be int32")
    if out is None:
        out = torch.empty((Tc, H, dv), dtype=q_cand.dtype, device=q_cand.device)
    bias = bias if bias is not None else make_bias(BIAS_NONE)
    Th = k_hist.shape[0]
    need = candidates_workspace_bytes(B, H, max_hist, Th, Tc)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q_cand.device)
    st = lib().hstu_attn_candidates_fwd(
        DTYPE_BF16, B, H, d, dv, _ptr(hist_offsets), int(max_hist), Th, _ptr(cand_offsets),
        int(max_cand), Tc, _ptr(q_cand), qs, _ptr(k_cand), kcs, _ptr(v_cand), vcs, _ptr(k_hist),
        khs, _ptr(v_hist), vhs, ctypes.byref(bias), _ptr(cand_timestamps), float(alpha),
        float(out_scale), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q_cand.device))
    _check("hstu_attn_candidates_fwd", st)
    return out


def candidates_workspace_bytes(B, H, max_hist, total_hist, total_cand):
    return int(lib().hstu_attn_candidates_workspace_bytes(int(B), int(H), int(max_hist),
                                                          int(total_hist), int(total_cand)))


def hstu_attn_bwd(q, k, v, d_o, offsets, max_seqlen, bias: Optional[HstuBias] = None, alpha=1.0,
                  out_scale=1.0, workspace=None, dw_out=None):
    """Gradients of hstu_attn_fwd for the upstream gradient d_o (bf16, d = 64).  Returns
    (dq, dk, dv, dw_pos, dw_time); the table gradients are fp32 tensors shaped like the bias
    tables (None without the position + time bias), written into dw_out = (dw_pos, dw_time)
    when given."""
    if q.dtype != torch.bfloat16:
        raise HstuError("the backward pass runs in bf16")
    qs, H, d = _rows(q, "q")
    ks, _, _ = _rows(k, "k")
    vs, _, dv_ = _rows(v, "v")
    dos, _, _ = _rows(d_o, "d_o")
    T = q.shape[0]
    B = offsets.numel() - 1
    if offsets.dtype != torch.int32:
        raise HstuError("offsets must be int32")
    bias = bias if bias is not None else make_bias(BIAS_NONE)
    dq = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
    dk = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
    dv = torch.empty((T, H, dv_), dtype=q.dtype, device=q.device)
    dwp = dwt = None
    if bias.kind == BIAS_RAB_PT:
        ts, wp, wt = bias._keep
        if dw_out is not None:
            dwp, dwt = dw_out
            if dwp.shape != wp.shape or dwt.shape != wt.shape or dwp.dtype != torch.float32 \
                    or dwt.dtype != torch.float32:
                raise HstuError("dw_out must be fp32 tensors shaped like the bias tables")
        else:
            dwp = torch.empty(wp.shape, dtype=torch.float32, device=q.device)
            dwt = torch.empty(wt.shape, dtype=torch.float32, device=q.device)
    need = attn_workspace_bytes(B, H, max_seqlen, T)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib().hstu_attn_bwd(DTYPE_BF16, B, H, d, dv_, _ptr(offsets), int(max_seqlen), T, _ptr(q),
                             qs, _ptr(k), ks, _ptr(v), vs, _ptr(d_o), dos, ctypes.byref(bias),
                             float(alpha), float(out_scale), _ptr(dq), _ptr(dk), _ptr(dv),
                             _ptr(dwp), _ptr(dwt), _ptr(workspace), workspace.numel(),
                             _stream(q.device))
    _check("hstu_attn_bwd", st)
    return dq, dk, dv, dwp, dwt


def hstu_layer_bwd(x, offsets, max_seqlen, w1, b1, gamma, beta, w2, H, dqk, dv, bias, alpha,
                   residual, ln_eps, fwd_workspace, dy, workspace=None):
    """Gradients of hstu_layer_fwd (called before with the same inputs and fwd_workspace).
    Returns a dict: dx (bf16), dw1, db1, dgamma, dbeta, dw2, db2, dw_pos, dw_time (fp32)."""
    T, D = x.shape
    B = offsets.numel() - 1
    N1 = w1.shape[0]
    HV = H * dv
    dev = x.device
    f = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    out = dict(dx=torch.empty_like(x), dw1=f(N1, D), db1=f(N1), dgamma=f(HV), dbeta=f(HV),
               dw2=f(D, HV), db2=f(D), dw_pos=None, dw_time=None)
    bias = bias if bias is not None else make_bias(BIAS_NONE)
    if bias.kind == BIAS_RAB_PT:
        ts, wp, wt = bias._keep
        out["dw_pos"] = torch.empty(wp.shape, dtype=torch.float32, device=dev)
        out["dw_time"] = torch.empty(wt.shape, dtype=torch.float32, device=dev)
    need = int(lib().hstu_layer_bwd_workspace_bytes(B, T, H, dqk, dv, int(max_seqlen)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib().hstu_layer_bwd(DTYPE_BF16, B, D, H, dqk, dv, _ptr(offsets), int(max_seqlen), T,
                              _ptr(x), _ptr(w1), _ptr(b1), _ptr(gamma), _ptr(beta), float(ln_eps),
                              _ptr(w2), ctypes.byref(bias), float(alpha), int(bool(residual)),
                              _ptr(fwd_workspace), _ptr(dy), _ptr(out["dx"]), _ptr(out["dw1"]),
                              _ptr(out["db1"]), _ptr(out["dgamma"]), _ptr(out["dbeta"]),
                              _ptr(out["dw2"]), _ptr(out["db2"]), _ptr(out["dw_pos"]),
                              _ptr(out["dw_time"]), _ptr(workspace), workspace.numel(),
                              _stream(dev))
    _check("hstu_layer_bwd", st)
    return out


def hstu_stochastic_length(offsets, max_seqlen, N_c, alpha, u_user, key_tok, x=None, ts=None):
    """Stochastic Length on the device.  Returns (out_offsets int32 [B+1], src_index int32 [T],
    x_out, ts_out); outputs are sized like the inputs, the first out_offsets[B] rows valid."""
    B = offsets.numel() - 1
    T = key_tok.numel()
    dev = offsets.device
    out_offsets = torch.empty(B + 1, dtype=torch.int32, device=dev)
    src_index = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    x_out = torch.empty_like(x) if x is not None else None
    ts_out = torch.empty_like(ts) if ts is not None else None
    row_bytes = x[0].numel() * x.element_size() if x is not None and T else 0
    ws = torch.empty(max(int(lib().hstu_stochastic_length_workspace_bytes(B, T)), 256),
                     dtype=torch.uint8, device=dev)
    st = lib().hstu_stochastic_length(B, _ptr(offsets), int(max_seqlen), T, int(N_c), float(alpha),
                                      _ptr(u_user), _ptr(key_tok), _ptr(x), row_bytes, _ptr(ts),
                                      _ptr(out_offsets), _ptr(src_index), _ptr(x_out),
                                      _ptr(ts_out), _ptr(ws), ws.numel(), _stream(dev))
    _check("hstu_stochastic_length", st)
    return out_offsets, src_index[:T], x_out, ts_out


def hstu_embed_sum_fwd(item_table, action_table, item_ids, action_ids, out=None):
    """GenRank action-oriented tokens: x[t] = item_table[item_ids[t]] + action_table[action_ids[t]]."""
    T = item_ids.numel()
    dim = item_table.shape[1]
    if out is None:
        out = torch.empty((T, dim), dtype=torch.bfloat16, device=item_table.device)
    st = lib().hstu_embed_sum_fwd(T, dim, _ptr(item_table), item_table.shape[0],
                                  _ptr(action_table), action_table.shape[0], _ptr(item_ids),
                                  _ptr(action_ids), _ptr(out), _stream(item_table.device))
    _check("hstu_embed_sum_fwd", st)
    return out


def hstu_validate_offsets(offsets, total_tokens, max_seqlen):
    flags = torch.zeros(1, dtype=torch.int32, device=offsets.device)
    st = lib().hstu_validate_offsets(offsets.numel() - 1, _ptr(offsets), int(total_tokens),
                                     int(max_seqlen), _ptr(flags), _stream(offsets.device))
    _check("hstu_validate_offsets", st)
    return flags


def hstu_debug_buckets(offsets, timestamps, num_pos, num_time, token_i, token_j):
    R = token_i.numel()
    pb = torch.empty(R, dtype=torch.int32, device=offsets.device)
    tb = torch.empty(R, dtype=torch.int32, device=offsets.device)
    st = lib().hstu_debug_buckets(offsets.numel() - 1, _ptr(offsets), _ptr(timestamps), num_pos,
                                  num_time, R, _ptr(token_i), _ptr(token_j), _ptr(pb), _ptr(tb),
                                  _stream(offsets.device))
    _check("hstu_debug_buckets", st)
    return pb, tb


def status_string(code):
    return lib().hstu_status_string(code).decode()
