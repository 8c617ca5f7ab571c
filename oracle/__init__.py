"""fp64 CPU oracle of Orthros attention: TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package. The product path (the HIP library and its Python
binding) never imports, links or calls it, and the two share no code.

The arithmetic lives in ``orthros_oracle.c`` (plain C, fp64, two-pass
softmax per row); this module only marshals numpy arrays. Each function
names the passage of the pages it follows:

* ``swa``         base-stream sliding-window attention, o_t
                  (Orthros: Phase-Aware Heterogeneous Attention for
                  Efficient Transformers, paper text §3.1, the o_t equation)
* ``xattn``       output-stream full cross-attention, o'_t
                  (same page, §3.1, the o'_t equation; rows t = T_in + r)
* ``row_weights`` normalised weights of one row (support / sum checks)
* ``Cache``       incremental prefill-then-decode, the decode pair step
                  (same page, §3.2 Decoding)
* ``attn_backward`` gradients of both streams (q_pre, qx_pre, K, V and the
                  four scale-offset vectors) for training (paper text §3.2,
                  pre-training and SFT), row by row in numpy fp64
* ``attn_backward_sampled`` selected rows' dq and selected keys' dK, dV of
                  the same gradients, in matrix form over the rows that see
                  each key (for full-size checks)
* ``layer``       one attention layer with its projections: k, v = x W_K,
                  x W_V for the base rows, q = alpha (.) (x W_Q) + beta and
                  q' = alpha' (.) (x' W_Q) + beta', the two streams, their
                  outputs in input row order, then W_O (same page, §3.1,
                  the description of Algorithm 1 and Figure 1(b)); numpy
                  fp64 matrix products, attention through ``swa``/``xattn``

Parity pins (tests/test_oracle_pins.py) tie every function to something
other than itself: torch's scaled_dot_product_attention for the cases that
reduce to standard causal or masked attention, closed forms, exact index
supports, and incremental == batched.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liborthros_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # noqa: WPS433 (build on first use)
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    c_int, c_i64, c_void = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    lib.oracle_swa.argtypes = [c_int, c_int, c_int, c_int, c_int, c_i64, _i32p,
                               _dp, _dp, _dp, _dp, _dp, _dp, _dp, c_i64, _i64p]
    lib.oracle_swa.restype = c_int
    lib.oracle_xattn.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int,
                                 _i32p, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                 c_i64, _i64p]
    lib.oracle_xattn.restype = c_int
    lib.oracle_row_weights.argtypes = [c_int, c_int, c_int, c_i64, c_i64,
                                       c_int, _dp, _dp, _dp, _dp, _dp, _dp]
    lib.oracle_row_weights.restype = c_int
    lib.oracle_cache_new.argtypes = [c_int, c_int, c_int, c_i64]
    lib.oracle_cache_new.restype = c_void
    lib.oracle_cache_free.argtypes = [c_void]
    lib.oracle_cache_free.restype = None
    lib.oracle_cache_len.argtypes = [c_void, c_int]
    lib.oracle_cache_len.restype = c_i64
    lib.oracle_cache_append.argtypes = [c_void, c_int, _dp, _dp]
    lib.oracle_cache_append.restype = c_int
    lib.oracle_cache_decode_pair.argtypes = [c_void, c_int, c_i64, _i32p,
                                             _dp, _dp, _dp, _dp, _dp, _dp,
                                             _dp, _dp, _dp, _dp]
    lib.oracle_cache_decode_pair.restype = c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = c_int
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, typ=_dp):
    return None if a is None else a.ctypes.data_as(typ)


def _map(head_map):
    if head_map is None:
        return None
    return np.ascontiguousarray(head_map, dtype=np.int32)


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
    return r, r.shape[0]


def num_threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().oracle_num_threads())


def swa(q_pre, alpha, beta, k, v, W, head_map=None, rows=None):
    """Base-stream SWA, every position t: keys [max(0, t-W+1), t].

    q_pre [B,T,Hq,D]; alpha, beta [Hq*D] (or [Hq,D]); k, v [B,T,Hkv,D].
    rows: optional (n,2) int array of (b, t) to evaluate; outputs are then
    [n, Hq, D] / [n, Hq] instead of [B,T,Hq,D] / [B,T,Hq].
    Returns (o, lse) as float64.
    """
    lib = _load()
    q_pre, k, v = _f64(q_pre), _f64(k), _f64(v)
    alpha, beta = _f64(alpha).reshape(-1), _f64(beta).reshape(-1)
    B, T, Hq, D = q_pre.shape
    Hkv = k.shape[2]
    assert k.shape == (B, T, Hkv, D) and v.shape == k.shape
    assert alpha.size == Hq * D and beta.size == Hq * D
    hm = _map(head_map)
    r, n = _rows(rows)
    lead = (n,) if r is not None else (B, T)
    o = np.empty(lead + (Hq, D))
    lse = np.empty(lead + (Hq,))
    rc = lib.oracle_swa(B, T, Hq, Hkv, D, int(W), _ptr(hm, _i32p),
                        _ptr(q_pre), _ptr(alpha), _ptr(beta), _ptr(k),
                        _ptr(v), _ptr(o), _ptr(lse), n, _ptr(r, _i64p))
    if rc:
        raise ValueError("oracle_swa: invalid arguments")
    return o, lse


def xattn(qx_pre, alpha_x, beta_x, k, v, T_in, head_map=None, rows=None):
    """Output-stream cross-attention: row r sits at t = T_in + r and attends
    keys [0, t]. qx_pre [B,T_out,Hq,D]; k, v [B,T,Hkv,D] with T >= T_in+T_out
    (only the first T_in + T_out keys are visible).
    rows: optional (n,2) array of (b, r). Returns (o_x, lse)."""
    lib = _load()
    qx_pre = _f64(qx_pre)
    alpha_x, beta_x = _f64(alpha_x).reshape(-1), _f64(beta_x).reshape(-1)
    B, T_out, Hq, D = qx_pre.shape
    T = T_in + T_out
    k = _f64(k[:, :T])
    v = _f64(v[:, :T])
    Hkv = k.shape[2]
    assert k.shape == (B, T, Hkv, D)
    hm = _map(head_map)
    r, n = _rows(rows)
    lead = (n,) if r is not None else (B, T_out)
    o = np.empty(lead + (Hq, D))
    lse = np.empty(lead + (Hq,))
    rc = lib.oracle_xattn(B, int(T_in), T_out, Hq, Hkv, D, _ptr(hm, _i32p),
                          _ptr(qx_pre), _ptr(alpha_x), _ptr(beta_x), _ptr(k),
                          _ptr(v), _ptr(o), _ptr(lse), n, _ptr(r, _i64p))
    if rc:
        raise ValueError("oracle_xattn: invalid arguments")
    return o, lse


def row_weights(q_pre_row, alpha_h, beta_h, k_b, v_b, t, W, g):
    """Normalised weights over all T keys for one query row at position t
    (W <= 0: unbounded window). k_b, v_b [T,Hkv,D] of one batch entry."""
    lib = _load()
    k_b, v_b = _f64(k_b), _f64(v_b)
    T, Hkv, D = k_b.shape
    w = np.empty(T)
    rc = lib.oracle_row_weights(T, Hkv, D, int(t), int(W), int(g),
                                _ptr(_f64(q_pre_row)), _ptr(_f64(alpha_h)),
                                _ptr(_f64(beta_h)), _ptr(k_b), _ptr(v_b),
                                _ptr(w))
    if rc:
        raise ValueError("oracle_row_weights: invalid arguments")
    return w


class Cache:
    """Growing per-layer K/V cache of the base stream (incremental mode)."""

    def __init__(self, B, Hkv, D, cap):
        self._lib = _load()
        self.B, self.Hkv, self.D, self.cap = B, Hkv, D, cap
        self._h = self._lib.oracle_cache_new(B, Hkv, D, int(cap))
        if not self._h:
            raise MemoryError("oracle cache allocation failed")

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.oracle_cache_free(h)

    def length(self, b):
        return int(self._lib.oracle_cache_len(self._h, b))

    def append(self, k_new, v_new):
        """k_new, v_new [B, n, Hkv, D]."""
        k_new, v_new = _f64(k_new), _f64(v_new)
        n = k_new.shape[1]
        assert k_new.shape == (self.B, n, self.Hkv, self.D)
        if self._lib.oracle_cache_append(self._h, n, _ptr(k_new), _ptr(v_new)):
            raise ValueError("oracle cache append: capacity exceeded")

    def decode_pair(self, q_pre, qx_pre, alpha, beta, alpha_x, beta_x,
                    k_new, v_new, W, head_map=None):
        """Append one base token, then base SWA + output full attention.
        q_pre, qx_pre [B,Hq,D]; k_new, v_new [B,Hkv,D]. Returns (o, o_x)."""
        q_pre, qx_pre = _f64(q_pre), _f64(qx_pre)
        B, Hq, D = q_pre.shape
        o = np.empty((B, Hq, D))
        o_x = np.empty((B, Hq, D))
        hm = _map(head_map)
        rc = self._lib.oracle_cache_decode_pair(
            self._h, Hq, int(W), _ptr(hm, _i32p), _ptr(q_pre), _ptr(qx_pre),
            _ptr(_f64(alpha).reshape(-1)), _ptr(_f64(beta).reshape(-1)),
            _ptr(_f64(alpha_x).reshape(-1)), _ptr(_f64(beta_x).reshape(-1)),
            _ptr(_f64(k_new)), _ptr(_f64(v_new)), _ptr(o), _ptr(o_x))
        if rc:
            raise ValueError("oracle decode_pair: invalid arguments")
        return o, o_x


def layer(x, w_q, w_k, w_v, w_o, alpha, beta, alpha_x, beta_x, T_out, W,
          Hkv, D, rows=None):
    """One Orthros attention layer, fp64.

    x [B, T + T_out, d_model]: the T base rows, then the T_out
    output-specific rows (row T + r is the output token at position
    T_in + r, T_in = T - T_out). Weights as in x W: w_q [d_model, Hq*D],
    w_k, w_v [d_model, Hkv*D], w_o [Hq*D, d_model].
    Returns y [B, T + T_out, d_model], or with `rows` (row indices into the
    T + T_out rows) y[:, rows] only; a base row t is then evaluated over its
    key slice [max(0, t-W+1), t] and an output row over [0, T_in + r].
    """
    x = _f64(x)
    w_q, w_k, w_v, w_o = (_f64(w) for w in (w_q, w_k, w_v, w_o))
    B, M, _ = x.shape
    T = M - T_out
    T_in = T - T_out
    Hq = w_q.shape[1] // D
    k = (x[:, :T] @ w_k).reshape(B, T, Hkv, D)
    v = (x[:, :T] @ w_v).reshape(B, T, Hkv, D)
    if rows is None:
        q_all = (x @ w_q).reshape(B, M, Hq, D)
        o, _ = swa(q_all[:, :T], alpha, beta, k, v, W)
        parts = [o]
        if T_out:
            ox, _ = xattn(q_all[:, T:], alpha_x, beta_x, k, v, T_in)
            parts.append(ox)
        o_cat = np.concatenate(parts, axis=1).reshape(B, M, Hq * D)
        return o_cat @ w_o
    out = []
    for i in rows:
        q_i = (x[:, i] @ w_q).reshape(B, 1, Hq, D)
        if i < T:
            lo = max(0, i - W + 1)
            o_i, _ = xattn(q_i, alpha, beta, k[:, lo:i + 1], v[:, lo:i + 1],
                           i - lo)
        else:
            t = T_in + (i - T)
            o_i, _ = xattn(q_i, alpha_x, beta_x, k[:, :t + 1], v[:, :t + 1], t)
        out.append(o_i.reshape(B, Hq * D) @ w_o)
    return np.stack(out, axis=1)


def attn_backward(q_pre, qx_pre, alpha, beta, alpha_x, beta_x, k, v, d_o,
                  d_ox, W, head_map=None, heads=None, with_kv=True):
    """Gradients of both streams' outputs, fp64, row by row.

    Inputs as for ``swa`` and ``xattn`` (k, v [B, T, Hkv, D]; qx_pre
    [B, T_out, Hq, D] with row r at position T - T_out + r; qx_pre may have
    T_out = 0), plus the upstream gradients d_o [B, T, Hq, D] and d_ox
    [B, T_out, Hq, D] of o and o'. For a row with query q over keys R:
    p = softmax(K_R q / sqrt(D)), dp = V_R dO, ds = p (dp - p.dp),
    dq = K_R^T ds / sqrt(D), dK_R += ds q^T / sqrt(D), dV_R += p dO^T
    (the chain rule through the o_t and o'_t equations of paper text §3.1),
    then through the scale-offset q = alpha (.) q_pre + beta:
    dq_pre = alpha (.) dq, d_alpha = sum of dq (.) q_pre, d_beta = sum of dq.
    Returns a dict of dq_pre, dqx_pre, dk, dv, d_alpha, d_beta, d_alpha_x,
    d_beta_x (alpha/beta gradients [Hq*D]).

    heads: optional list of query heads to evaluate (the entries of the
    other heads stay zero); with_kv=False skips the dK, dV sums (left zero).
    Each head's rows are independent of the others', so a subset gives that
    subset's exact entries.
    """
    q_pre, qx_pre = _f64(q_pre), _f64(qx_pre)
    k, v, d_o, d_ox = _f64(k), _f64(v), _f64(d_o), _f64(d_ox)
    B, T, Hq, D = q_pre.shape
    Hkv = k.shape[2]
    T_out = qx_pre.shape[1]
    T_in = T - T_out
    kv_of = (np.arange(Hq) // (Hq // Hkv) if head_map is None
             else np.asarray(head_map, dtype=np.int64))
    scale = 1.0 / np.sqrt(D)
    g = {"dq_pre": np.zeros_like(q_pre), "dqx_pre": np.zeros_like(qx_pre),
         "dk": np.zeros_like(k), "dv": np.zeros_like(v)}
    for name in ("d_alpha", "d_beta", "d_alpha_x", "d_beta_x"):
        g[name] = np.zeros((Hq, D))

    def row(b, h, qp, a, be, lo, hi, dO):
        gkv = kv_of[h]
        q = a * qp + be
        K, V = k[b, lo:hi + 1, gkv], v[b, lo:hi + 1, gkv]
        s = K @ q * scale
        p = np.exp(s - s.max())
        p /= p.sum()
        dp = V @ dO
        ds = p * (dp - p @ dp)
        dq = K.T @ ds * scale
        if with_kv:
            g["dk"][b, lo:hi + 1, gkv] += np.outer(ds, q) * scale
            g["dv"][b, lo:hi + 1, gkv] += np.outer(p, dO)
        return dq

    a2 = _f64(alpha).reshape(Hq, D)
    b2 = _f64(beta).reshape(Hq, D)
    ax2 = _f64(alpha_x).reshape(Hq, D)
    bx2 = _f64(beta_x).reshape(Hq, D)
    for b in range(B):
        for h in (range(Hq) if heads is None else heads):
            for t in range(T):
                dq = row(b, h, q_pre[b, t, h], a2[h], b2[h],
                         max(0, t - W + 1), t, d_o[b, t, h])
                g["dq_pre"][b, t, h] = a2[h] * dq
                g["d_alpha"][h] += dq * q_pre[b, t, h]
                g["d_beta"][h] += dq
            for r in range(T_out):
                dq = row(b, h, qx_pre[b, r, h], ax2[h], bx2[h], 0, T_in + r,
                         d_ox[b, r, h])
                g["dqx_pre"][b, r, h] = ax2[h] * dq
                g["d_alpha_x"][h] += dq * qx_pre[b, r, h]
                g["d_beta_x"][h] += dq
    for name in ("d_alpha", "d_beta", "d_alpha_x", "d_beta_x"):
        g[name] = g[name].reshape(-1)
    return g


def attn_backward_sampled(q_pre, qx_pre, alpha, beta, alpha_x, beta_x, k, v,
                          d_o, d_ox, W, b, rows, out_rows, keys, g):
    """Selected entries of ``attn_backward`` for one batch entry b, fp64.

    rows / out_rows: base positions t / output rows r whose dq_pre / dqx_pre
    (all heads) are returned; keys: key positions j whose dK, dV for KV head
    g (contiguous head grouping) are returned. Every gradient is the same
    chain rule; a row's softmax is taken over its whole key range (matrix
    products over the rows that see the sampled keys, masked).
    Returns (dq [len(rows), Hq, D], dqx [len(out_rows), Hq, D],
    dk [len(keys), D], dv [len(keys), D]).
    """
    q_pre, qx_pre = _f64(q_pre[b]), _f64(qx_pre[b])
    kb, vb = _f64(k[b]), _f64(v[b])
    d_o, d_ox = _f64(d_o[b]), _f64(d_ox[b])
    T, Hq, D = q_pre.shape
    Hkv = kb.shape[1]
    T_out = qx_pre.shape[0]
    T_in = T - T_out
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D)
    A, Bv = _f64(alpha).reshape(Hq, D), _f64(beta).reshape(Hq, D)
    AX, BX = _f64(alpha_x).reshape(Hq, D), _f64(beta_x).reshape(Hq, D)
    pos = np.arange(T)

    def grads(Q, dO, p_row, lo_row, kv):
        """Rows Q [n, D] at positions p_row with ranges [lo_row, p_row]
        against all keys of KV head kv: P, dS [n, T] (zero outside)."""
        K, V = kb[:, kv], vb[:, kv]
        s = Q @ K.T * scale
        inside = (pos[None, :] >= lo_row[:, None]) & (pos[None, :] <= p_row[:, None])
        s = np.where(inside, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = dO @ V.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        return p, ds

    dq = np.zeros((len(rows), Hq, D))
    dqx = np.zeros((len(out_rows), Hq, D))
    for h in range(Hq):
        kv = h // G
        if len(rows):
            t = np.asarray(rows)
            Q = A[h] * q_pre[t, h] + Bv[h]
            _, ds = grads(Q, d_o[t, h], t, np.maximum(t - W + 1, 0), kv)
            dq[:, h] = A[h] * (ds @ kb[:, kv] * scale)
        if len(out_rows):
            r = np.asarray(out_rows)
            Q = AX[h] * qx_pre[r, h] + BX[h]
            p_ = T_in + r
            _, ds = grads(Q, d_ox[r, h], p_, np.zeros_like(p_), kv)
            dqx[:, h] = AX[h] * (ds @ kb[:, kv] * scale)
    dk = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    for h in range(g * G, (g + 1) * G):
        for n, j in enumerate(keys):
            t = np.arange(j, min(T, j + W))          # base rows that see j
            if len(t):
                Q = A[h] * q_pre[t, h] + Bv[h]
                p, ds = grads(Q, d_o[t, h], t, np.maximum(t - W + 1, 0), g)
                dk[n] += ds[:, j] @ Q * scale
                dv[n] += p[:, j] @ d_o[t, h]
            r = np.arange(max(0, j - T_in), T_out)   # output rows that see j
            if len(r):
                Q = AX[h] * qx_pre[r, h] + BX[h]
                p_ = T_in + r
                p, ds = grads(Q, d_ox[r, h], p_, np.zeros_like(p_), g)
                dk[n] += ds[:, j] @ Q * scale
                dv[n] += p[:, j] @ d_ox[r, h]
    return dq, dqx, dk, dv
