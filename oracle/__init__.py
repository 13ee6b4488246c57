"""fp64 CPU oracle for the HSTU layer forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports, links or calls it, and it shares no code with that
path.  The arithmetic lives in ``hstu_oracle.c`` (plain loops in double); this
module only marshals numpy arrays into it and adds the two pieces that are a
single line of numpy (the embedding sum and the layer stack loop).

Sources, by page title and section:
  "Actions Speak Louder than Words" reading notes, §3.1 eqs. (1)-(3), §3.2,
  §3.3 (Stochastic Length), §3.6 (M-FALCON candidate scoring); the gradients of eq. (2)
  (backward pass);
  "4.4 推荐模型的 Scaling", section "HSTU 层" and the toy HSTULayer ("代码");
  GenRank article (joto.ai), "(1) item-action组织" and "(2) 位置 & 时间偏差".
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hstu_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BIAS_NONE, BIAS_RAB_PT, BIAS_ALIBI = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile hstu_oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        _lib.oracle_pos_bucket.argtypes = [i64, i32]
        _lib.oracle_pos_bucket.restype = i32
        _lib.oracle_time_bucket.argtypes = [i64, i32]
        _lib.oracle_time_bucket.restype = i32
        _lib.oracle_attention.argtypes = [i32, i32, i32, i32, P, P, i64, P, i64, P, i64, i32, P,
                                          P, i32, i64, P, i32, i64, P, f64, f64, P]
        _lib.oracle_attention.restype = None
        _lib.oracle_attention_mirror.argtypes = [i32, i32, i32, i32, P, P, i64, P, i64, P, i64,
                                                 i32, P, P, i32, i64, P, i32, i64, P, f64, f64,
                                                 f64, P]
        _lib.oracle_attention_mirror.restype = None
        _lib.oracle_attention_rows.argtypes = [i32, i32, i32, i32, P, P, i64, P, i64, P, i64, i32,
                                               P, P, i32, i64, P, i32, i64, P, f64, f64, i64, P, P,
                                               P]
        _lib.oracle_attention_rows.restype = None
        _lib.oracle_attention_bwd.argtypes = [i32, i32, i32, i32, P, P, P, P, P, i32, P, P, i32,
                                              i64, P, i32, i64, P, f64, f64, P, P, P, P, P]
        _lib.oracle_attention_bwd.restype = None
        _lib.oracle_attention_candidates.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P, i32,
                                                     P, P, P, i32, i64, P, i32, i64, P, f64, f64,
                                                     P]
        _lib.oracle_attention_candidates.restype = None
        _lib.oracle_layer.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, f64, P, P, i32, P,
                                      P, i32, i64, P, i32, i64, P, f64, i32, P, P, P]
        _lib.oracle_layer.restype = None
        _lib.oracle_bucket_counts.argtypes = [i32, P, P, i32, i32, P, P]
        _lib.oracle_bucket_counts.restype = None
        _lib.oracle_num_threads.restype = i32
        _lib.oracle_num_threads.argtypes = []
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(_L().oracle_num_threads())


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def pos_bucket(i_minus_j: int, num_pos: int) -> int:
    return int(_L().oracle_pos_bucket(int(i_minus_j), int(num_pos)))


def time_bucket(dt: int, num_time: int) -> int:
    return int(_L().oracle_time_bucket(int(dt), int(num_time)))


def bucket_counts(offsets, ts, num_pos: int, num_time: int):
    """For every row i of every user: how many keys j <= i fall in each position bucket and in
    each time bucket (the integer part of the bias, as the rab^{p,t} form defines it).
    Returns int32 arrays [T, num_pos] and [T, num_time]."""
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    ts = np.ascontiguousarray(ts, dtype=np.int64)
    T = int(offs[-1]) if len(offs) else 0
    pc = np.zeros((T, num_pos), np.int32)
    tc = np.zeros((T, num_time), np.int32)
    if T:
        _L().oracle_bucket_counts(len(offs) - 1, _ptr(offs), _ptr(ts), int(num_pos),
                                  int(num_time), _ptr(pc), _ptr(tc))
    return pc, tc


class Bias:
    """Relative attention bias description (host numpy arrays).

    kind: BIAS_NONE, BIAS_RAB_PT (position + log2 time-delta tables) or
    BIAS_ALIBI (per-head slopes, bias = -slope_h * (i - j)).
    w_pos is [P] (shared over heads) or [H, P]; likewise w_time.
    """

    def __init__(self, kind=BIAS_NONE, timestamps=None, w_pos=None, w_time=None, slopes=None):
        self.kind = kind
        self.ts = None if timestamps is None else np.ascontiguousarray(timestamps, dtype=np.int64)
        self.w_pos = None if w_pos is None else _f64(w_pos)
        self.w_time = None if w_time is None else _f64(w_time)
        self.slopes = None if slopes is None else _f64(slopes)

    def args(self):
        if self.kind == BIAS_RAB_PT:
            wp, wt = self.w_pos, self.w_time
            P = wp.shape[-1]
            NT = wt.shape[-1]
            sp = P if wp.ndim == 2 else 0
            st = NT if wt.ndim == 2 else 0
            return (self.kind, _ptr(self.ts), _ptr(wp), P, sp, _ptr(wt), NT, st, None)
        if self.kind == BIAS_ALIBI:
            return (self.kind, None, None, 0, 0, None, 0, 0, _ptr(self.slopes))
        return (BIAS_NONE, None, None, 0, 0, None, 0, 0, None)


def alibi_slopes(H: int) -> np.ndarray:
    """Slopes 2^(-8 (h+1) / H) for 0-based head h (the ALiBi geometric series
    2^-8/H ... 2^-8); GenRank article, part (2) names ALiBi without a formula."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float64)


def attention(offsets, q, k, v, bias: Bias, alpha: float, out_scale: float = 1.0,
              weight_unit: float = 0.0):
    """Eq. (2) on a jagged batch. q, k: [T, H, dqk]; v: [T, H, dv]. Returns [T, H, dv] fp64.
    weight_unit != 0 is the mirror mode: every SiLU weight is kept as weight_unit times a bf16
    value before it multiplies v (a bf16 path's weight operand)."""
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, dqk = q.shape
    dv = v.shape[2]
    B = len(offs) - 1
    o = np.zeros((T, H, dv), dtype=np.float64)
    if T == 0 or B == 0:
        return o
    _L().oracle_attention_mirror(B, H, dqk, dv, _ptr(offs), _ptr(q), H * dqk, _ptr(k), H * dqk,
                                 _ptr(v), H * dv, *bias.args(), float(alpha), float(out_scale),
                                 float(weight_unit), _ptr(o))
    return o


def attention_rows(offsets, q, k, v, bias: Bias, alpha: float, tokens, heads,
                   out_scale: float = 1.0):
    """Eq. (2) for selected (token, head) rows only; returns [R, dv] fp64."""
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, dqk = q.shape
    dv = v.shape[2]
    B = len(offs) - 1
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    hd = np.ascontiguousarray(heads, dtype=np.int32)
    R = len(tok)
    out = np.zeros((R, dv), dtype=np.float64)
    if R == 0:
        return out
    _L().oracle_attention_rows(B, H, dqk, dv, _ptr(offs), _ptr(q), H * dqk, _ptr(k), H * dqk,
                               _ptr(v), H * dv, *bias.args(), float(alpha), float(out_scale), R,
                               _ptr(tok), _ptr(hd), _ptr(out))
    return out


def attention_bwd(offsets, q, k, v, dO, bias: Bias, alpha: float, out_scale: float = 1.0):
    """Gradients of eq. (2) ("Actions Speak Louder than Words" §3.1 eq. (2)) for the upstream
    gradient dO: returns (dq, dk, dv, dw_pos, dw_time) in float64; the table gradients have
    the tables' shapes (None without the position + time bias)."""
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    T, H, dqk = q.shape
    dv = v.shape[2]
    B = len(offs) - 1
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    rab = bias.kind == BIAS_RAB_PT
    dwp = np.zeros_like(bias.w_pos) if rab else np.zeros(1)
    dwt = np.zeros_like(bias.w_time) if rab else np.zeros(1)
    if T and B:
        _L().oracle_attention_bwd(B, H, dqk, dv, _ptr(offs), _ptr(q), _ptr(k), _ptr(v), _ptr(dO),
                                  *bias.args(), float(alpha), float(out_scale), _ptr(dq), _ptr(dk),
                                  _ptr(dvv), _ptr(dwp), _ptr(dwt))
    return dq, dk, dvv, (dwp if rab else None), (dwt if rab else None)


def attention_candidates(hist_offsets, cand_offsets, q_c, k_c, v_c, k_h, v_h, bias: Bias,
                         cand_ts, alpha: float, out_scale: float = 1.0):
    """Candidate scoring over a user history ("Actions Speak Louder than Words" §3.6, M-FALCON;
    GenRank article part (2): candidates of one request share one position): candidate c of
    user b sits at position n_b and attends to the whole history and to itself only.
    q_c, k_c, v_c: [Tc, H, d]; k_h, v_h: [Th, H, d]; bias.timestamps are the history's and
    cand_ts the candidates'.  Returns [Tc, H, dv] in float64."""
    hist_offsets = np.ascontiguousarray(hist_offsets, np.int64)
    cand_offsets = np.ascontiguousarray(cand_offsets, np.int64)
    B = len(cand_offsets) - 1
    Tc, H, dqk = q_c.shape
    dv = v_c.shape[2]
    q_c, k_c, v_c = _f64(q_c), _f64(k_c), _f64(v_c)
    k_h = _f64(k_h).reshape(-1, H, dqk)
    v_h = _f64(v_h).reshape(-1, H, dv)
    cts = np.ascontiguousarray(cand_ts if cand_ts is not None else np.zeros(Tc), np.int64)
    o = np.zeros((Tc, H, dv), np.float64)
    a = bias.args()
    _L().oracle_attention_candidates(B, H, dqk, dv, _ptr(hist_offsets), _ptr(cand_offsets),
                                     _ptr(q_c), _ptr(k_c), _ptr(v_c), _ptr(k_h), _ptr(v_h), a[0],
                                     a[1], _ptr(cts), *a[2:], float(alpha), float(out_scale),
                                     _ptr(o))
    return o


def layer(offsets, x, w1, b1, gamma, beta, w2, b2, bias: Bias, alpha: float, H: int, dqk: int,
          dv: int, residual: bool = False, ln_eps: float = 1e-5, return_intermediates=False):
    """One HSTU layer, eqs. (1)-(3). x: [T, D]; w1: [2H(dqk+dv), D]; w2: [D, H dv]."""
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    x = _f64(x)
    T, D = x.shape
    B = len(offs) - 1
    N1 = 2 * H * (dqk + dv)
    y = np.zeros((T, D), dtype=np.float64)
    z = np.zeros((T, N1), dtype=np.float64)
    o = np.zeros((T, H * dv), dtype=np.float64)
    if T > 0 and B > 0:
        w1, b1, w2, b2 = _f64(w1), _f64(b1), _f64(w2), _f64(b2)
        gamma, beta = _f64(gamma), _f64(beta)
        _L().oracle_layer(B, D, H, dqk, dv, _ptr(offs), _ptr(x), _ptr(w1), _ptr(b1), _ptr(gamma),
                          _ptr(beta), float(ln_eps), _ptr(w2), _ptr(b2), *bias.args(),
                          float(alpha), int(bool(residual)), _ptr(y), _ptr(z), _ptr(o))
    if return_intermediates:
        return y, z, o
    return y


def round_bf16(a):
    """Each value rounded to the nearest bfloat16 (8 significant bits, ties to even), returned
    as float64.  Used only by the mirror mode of ``layer`` / ``layer_bwd``, which rounds named
    intermediates to bf16 storage to measure how much of a bf16 path's error its storage
    format alone explains.  (No bf16 subnormals or overflow: the magnitudes here are moderate.)"""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)                       # a = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)  # np.rint rounds halves to even


# intermediates of the layer a mirror run may round to bf16 (forward, then backward):
#   Z, G, Y, dG, dO, dZ, dZpre  the tensor, each element to the nearest bf16;
#   O    each element to the nearest bf16;  Oc  each (token, head) row as its mean plus bf16
#        deviations from it (a storage form that keeps the row's spread to 8 bits);
#   P    the attention's SiLU weights, as bf16 multiples of ln(2)/2 (the weights a path that
#        evaluates SiLU in base-2 units hands to the matrix product).
MIRROR_POINTS = ("Z", "P", "O", "Oc", "G", "Y", "dG", "dO", "dZ", "dZpre")


def _round_rows_centred(o, H):
    T = o.shape[0]
    o3 = o.reshape(T, H, -1)
    m = o3.mean(axis=2, keepdims=True)
    return (m + round_bf16(o3 - m)).reshape(o.shape)


def layer_mirror(offsets, x, w1, b1, gamma, beta, w2, b2, bias: Bias, alpha: float, H: int,
                 dqk: int, dv: int, residual: bool = False, ln_eps: float = 1e-5, round_at=()):
    """``layer`` composed step by step in float64 (eqs. (1)-(3)), with the intermediates named in
    `round_at` (Z, P, O or Oc, G, Y; see MIRROR_POINTS) rounded where they are formed.  With
    nothing rounded it is the exact layer.  Returns (y, z, o)."""
    for p in round_at:
        assert p in MIRROR_POINTS, p
    R = lambda name, a: round_bf16(a) if name in round_at else a
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    x, w1, b1, w2, b2 = _f64(x), _f64(w1), _f64(b1), _f64(w2), _f64(b2)
    gamma, beta = _f64(gamma), _f64(beta)
    T = x.shape[0]
    HV, HQ = H * dv, H * dqk
    zpre = x @ w1.T + b1
    z = R("Z", zpre / (1.0 + np.exp(-zpre)))
    V, Q, K = z[:, HV:2 * HV], z[:, 2 * HV:2 * HV + HQ], z[:, 2 * HV + HQ:]
    o = R("O", attention(offs, Q.reshape(T, H, dqk), K.reshape(T, H, dqk), V.reshape(T, H, dv),
                         bias, alpha, weight_unit=0.5 * math.log(2.0) if "P" in round_at else 0.0
                         ).reshape(T, HV))
    if "Oc" in round_at:
        o = _round_rows_centred(o, H)
    xc = o - o.mean(axis=1, keepdims=True)
    xhat = xc / np.sqrt((xc * xc).mean(axis=1, keepdims=True) + ln_eps)
    G = R("G", (xhat * gamma + beta) * z[:, :HV])
    y = R("Y", G @ w2.T + b2 + (x if residual else 0.0))
    return y, z, o


def layer_bwd(offsets, x, w1, b1, gamma, beta, w2, b2, bias: Bias, alpha: float, H: int,
              dqk: int, dv: int, dY, residual: bool = False, ln_eps: float = 1e-5, round_at=()):
    """Gradients of one HSTU layer ("Actions Speak Louder than Words" §3.1 eqs. (1)-(3)) for the
    upstream gradient dY, by the chain rule through each equation in reverse:
      eq. (3)  Y = (LN(O) * U) W2^T + b2 (+ X):  dW2 = dY^T G, db2 = sum_t dY, dG = dY W2,
               dU = dG * LN(O), d(LN) = dG * U, dgamma = sum_t d(LN) * xhat, dbeta = sum_t d(LN),
               dO = rstd (dxhat - mean(dxhat) - xhat mean(dxhat * xhat)), dxhat = d(LN) * gamma;
      eq. (2)  attention_bwd (dQ, dK, dV, table gradients);
      eq. (1)  Z = SiLU(X W1^T + b1), split U | V | Q | K:  dZpre = dZ * SiLU'(Zpre),
               dW1 = dZpre^T X, db1 = sum_t dZpre, dX = dZpre W1 (+ dY).
    `round_at` (mirror mode, see ``layer_mirror`` and MIRROR_POINTS) rounds the named
    intermediates where they are formed; empty gives the exact gradients.
    Returns a dict of float64 arrays: dx, dw1, db1, dgamma, dbeta, dw2, db2, dw_pos, dw_time."""
    for p in round_at:
        assert p in MIRROR_POINTS, p
    R = lambda name, a: round_bf16(a) if name in round_at else a
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    x, w1, b1, w2, b2 = _f64(x), _f64(w1), _f64(b1), _f64(w2), _f64(b2)
    gamma, beta, dY = _f64(gamma), _f64(beta), _f64(dY)
    T, D = x.shape
    HV, HQ = H * dv, H * dqk
    if round_at:
        _, z, o = layer_mirror(offs, x, w1, b1, gamma, beta, w2, b2, bias, alpha, H, dqk, dv,
                               residual, ln_eps,
                               tuple(p for p in round_at if p in ("Z", "P", "O", "Oc")))
    else:
        _, z, o = layer(offs, x, w1, b1, gamma, beta, w2, b2, bias, alpha, H, dqk, dv,
                        residual=residual, ln_eps=ln_eps, return_intermediates=True)
    zpre = x @ w1.T + b1
    U = z[:, :HV]
    V, Q, K = z[:, HV:2 * HV], z[:, 2 * HV:2 * HV + HQ], z[:, 2 * HV + HQ:]
    mean = o.mean(axis=1, keepdims=True)
    xc = o - mean
    rstd = 1.0 / np.sqrt((xc * xc).mean(axis=1, keepdims=True) + ln_eps)
    xhat = xc * rstd
    ln = xhat * gamma + beta
    G = R("G", ln * U)
    dw2 = dY.T @ G
    db2 = dY.sum(axis=0)
    dG = R("dG", dY @ w2)
    dU = dG * ln
    dln = dG * U
    dgamma = (dln * xhat).sum(axis=0)
    dbeta = dln.sum(axis=0)
    dxhat = dln * gamma
    dO = R("dO", rstd * (dxhat - dxhat.mean(axis=1, keepdims=True)
                         - xhat * (dxhat * xhat).mean(axis=1, keepdims=True)))
    dq, dk, dvv, dwp, dwt = attention_bwd(offs, Q.reshape(T, H, dqk), K.reshape(T, H, dqk),
                                          V.reshape(T, H, dv), dO.reshape(T, H, dv), bias, alpha)
    dZ = R("dZ", np.concatenate([dU, dvv.reshape(T, HV), dq.reshape(T, HQ), dk.reshape(T, HQ)],
                                axis=1))
    sg = 1.0 / (1.0 + np.exp(-zpre))
    dzpre = R("dZpre", dZ * sg * (1.0 + zpre * (1.0 - sg)))
    dw1 = dzpre.T @ x
    db1 = dzpre.sum(axis=0)
    dx = dzpre @ w1 + (dY if residual else 0.0)
    return dict(dx=dx, dw1=dw1, db1=db1, dgamma=dgamma, dbeta=dbeta, dw2=dw2, db2=db2,
                dw_pos=dwp, dw_time=dwt, dzpre=dzpre, dO=dO, G=G)


def sl_length(N_c: int, alpha: float) -> int:
    """Target length of Stochastic Length ("Actions Speak Louder than Words" §3.3): the
    subsequence has N_c^(alpha/2) elements, taken as the integer part."""
    return int(math.floor(float(N_c) ** (alpha / 2.0)))


def stochastic_length(offsets, N_c: int, alpha: float, u_user, key_tok):
    """Stochastic Length ("Actions Speak Louder than Words" §3.3) on a jagged batch.

    For user b with n_b events and L = sl_length(N_c, alpha): n_b <= L keeps the sequence;
    n_b > L replaces it, with probability 1 - N_c^alpha / n_b^2, by L of its events, else keeps
    it.  The random draws are inputs: user b is subsampled iff u_user[b] < 1 - N_c^alpha / n_b^2
    (in float64), and the L events kept are those with the smallest key_tok (ties by lower
    index), in their original order (a uniform random L-subset when the keys are i.i.d.).
    Returns (out_offsets int64 [B+1], src_index int64 [T_out]: the input token of each output
    token)."""
    offs = np.asarray(offsets, dtype=np.int64)
    u_user = np.asarray(u_user, dtype=np.float32)
    key_tok = np.asarray(key_tok, dtype=np.float32)
    L = sl_length(N_c, alpha)
    c = float(N_c) ** float(alpha)
    out_off = [0]
    src = []
    for b in range(len(offs) - 1):
        s, e = int(offs[b]), int(offs[b + 1])
        n = e - s
        idx = np.arange(s, e, dtype=np.int64)
        if n > L and float(u_user[b]) < 1.0 - c / float(n * n):
            order = np.argsort(key_tok[s:e], kind="stable")[:L]
            idx = s + np.sort(order).astype(np.int64)
        src.append(idx)
        out_off.append(out_off[-1] + len(idx))
    return (np.asarray(out_off, dtype=np.int64),
            np.concatenate(src) if src else np.zeros(0, np.int64))


def embed_sum(item_table, action_table, item_ids, action_ids):
    """GenRank action-oriented token: item embedding + action embedding
    (GenRank article, part (1))."""
    return _f64(item_table)[np.asarray(item_ids)] + _f64(action_table)[np.asarray(action_ids)]


def stack(offsets, x, layers, bias_per_layer, alpha, H, dqk, dv, ln_eps=1e-5):
    """Layers stacked with residual connections ("Actions Speak Louder than
    Words" §3.1: identical layers joined by residuals). layers: list of dicts
    with w1, b1, gamma, beta, w2, b2."""
    h = _f64(x)
    for L, bias in zip(layers, bias_per_layer):
        h = layer(offsets, h, L["w1"], L["b1"], L["gamma"], L["beta"], L["w2"], L["b2"], bias,
                  alpha, H, dqk, dv, residual=True, ln_eps=ln_eps)
    return h
