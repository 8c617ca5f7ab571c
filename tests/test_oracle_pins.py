"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test ties the oracle to something the pages or the mathematics fix:
  * standard causal / masked attention computed by torch's
    scaled_dot_product_attention (a library routine) in the special cases
    where the method reduces to it (identity affine with W >= T, reproduction
    note "Orthros：阶段异构注意力", local reproduction section; a band mask for
    W < T, paper text §3.1 of "Orthros: Phase-Aware Heterogeneous Attention
    for Efficient Transformers", o_t equation index range);
  * exact supports and unit sums of the softmax weights (same equations);
  * closed forms (W = 1, zero query, constant V, two keys, spike keys);
  * incremental prefill-then-decode == batched (reproduction note, 1e-4 gate);
  * symmetries (channel / head permutation, GQA replication, batch
    independence).
A plausible slip in the oracle (window off by one, missing beta, wrong
sqrt(D), wrong head map, T_in offset, attend-before-append) fails at least
one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import prefill_inputs, workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def sdpa(q, k, v, mask=None, causal=False, scale=None, head_map=None):
    """torch fp64 CPU scaled_dot_product_attention.
    q [B,T,Hq,D], k,v [B,S,Hkv,D] -> [B,T,Hq,D]. KV heads are expanded to
    the query heads by head_map (default h // (Hq/Hkv))."""
    q = torch.from_numpy(np.ascontiguousarray(q)).double()
    k = torch.from_numpy(np.ascontiguousarray(k)).double()
    v = torch.from_numpy(np.ascontiguousarray(v)).double()
    Hq, Hkv = q.shape[2], k.shape[2]
    idx = (torch.arange(Hq) // (Hq // Hkv) if head_map is None
           else torch.as_tensor(head_map, dtype=torch.long))
    k = k.index_select(2, idx)
    v = v.index_select(2, idx)
    qt, kt, vt = (x.permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                         is_causal=causal, scale=scale)
    return out.permute(0, 2, 1, 3).numpy()


def band_mask(T, W, q_offset=0, nrows=None):
    """Boolean [nrows, T]: key j visible to the row at position t iff
    t - W + 1 <= j <= t, built from triangular masks (not from lo/hi)."""
    nrows = T - q_offset if nrows is None else nrows
    ones = np.ones((T, T), dtype=bool)
    m = np.tril(ones) & np.triu(ones, -(W - 1))
    return m[q_offset:q_offset + nrows]


def ident(Hq, D):
    return np.ones(Hq * D), np.zeros(Hq * D)


# --- P1: identity affine, W >= T  ==  standard causal attention -----------

@pytest.mark.parametrize("B,T,Hq,Hkv,D,W", [
    (1, 64, 2, 2, 16, 64),     # tiny fp32 configuration, identity run
    (2, 37, 4, 2, 8, 37),
    (1, 50, 8, 2, 32, 1000),   # W far above T
])
def test_identity_affine_full_window_is_causal_attention(B, T, Hq, Hkv, D, W):
    q, k, v = rnd((B, T, Hq, D), 1), rnd((B, T, Hkv, D), 2), rnd((B, T, Hkv, D), 3)
    a, b = ident(Hq, D)
    o, _ = oracle.swa(q, a, b, k, v, W)
    ref = sdpa(q, k, v, causal=True)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_tiny_config_identity_run_matches_causal():
    tiny, tiny_id = workload("tiny_f32")
    cfg = tiny.with_(W=64, identity_affine=True)
    x = prefill_inputs(cfg, tiny_id)
    q, k, v = (t.double().numpy() for t in (x.q_pre, x.k, x.v))
    o, _ = oracle.swa(q, x.alpha.numpy(), x.beta.numpy(), k, v, cfg.W)
    np.testing.assert_allclose(o, sdpa(q, k, v, causal=True), atol=1e-12)


# --- P1b: band window == masked attention --------------------------------

@pytest.mark.parametrize("W", [1, 2, 15, 16, 17, 63, 64, 65])
def test_window_equals_band_masked_attention(W):
    B, T, Hq, Hkv, D = 2, 64, 4, 2, 16
    q, k, v = rnd((B, T, Hq, D), 4), rnd((B, T, Hkv, D), 5), rnd((B, T, Hkv, D), 6)
    a, b = ident(Hq, D)
    o, _ = oracle.swa(q, a, b, k, v, W)
    ref = sdpa(q, k, v, mask=band_mask(T, W))
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


# --- output stream vs causal attention ------------------------------------

def _paradigms(T):
    with open(os.path.join(GOLDEN, "paradigms.json")) as f:
        spec = json.load(f)["paradigms"]
    out = []
    for p in spec:
        if p["name"] == "decoding":
            continue  # single-token step: covered by the cache tests
        T_out_sft = max(1, T // 3)
        env = {"T": T, "T_out_sft": T_out_sft}
        out.append((p["name"], eval(p["T_in"], {}, env),  # noqa: S307
                    eval(p["T_out"], {}, env)))
    return out


@pytest.mark.parametrize("name,T_in,T_out", _paradigms(48))
def test_output_stream_is_causal_attention_at_output_rows(name, T_in, T_out):
    """Each (T_in, T_out) paradigm of the pages: the output rows t = T_in+r
    see keys [0, t]; with identity affine that is causal attention whose
    queries at rows t are the output-stream queries."""
    B, T, Hq, Hkv, D = 2, T_in + T_out, 4, 2, 16
    assert T == 48
    qx = rnd((B, T_out, Hq, D), 7)
    k, v = rnd((B, T, Hkv, D), 8), rnd((B, T, Hkv, D), 9)
    a, b = ident(Hq, D)
    ox, _ = oracle.xattn(qx, a, b, k, v, T_in)
    qfull = np.concatenate([np.zeros((B, T_in, Hq, D)), qx], axis=1)
    ref = sdpa(qfull, k, v, causal=True)[:, T_in:]
    np.testing.assert_allclose(ox, ref, atol=1e-12, rtol=0)


# --- affine pins ------------------------------------------------------------

def test_scalar_scale_equals_attention_scale():
    """alpha = c (all channels), beta = 0: scores scale by c."""
    B, T, Hq, Hkv, D, W, c = 1, 40, 4, 4, 16, 9, 1.7
    q, k, v = rnd((B, T, Hq, D), 10), rnd((B, T, Hkv, D), 11), rnd((B, T, Hkv, D), 12)
    o, _ = oracle.swa(q, np.full(Hq * D, c), np.zeros(Hq * D), k, v, W)
    ref = sdpa(q, k, v, mask=band_mask(T, W), scale=c / math.sqrt(D))
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_zero_scale_makes_query_the_offset():
    """alpha = 0: every base query equals beta of its head."""
    B, T, Hq, Hkv, D, W = 2, 33, 4, 2, 8, 7
    q, k, v = rnd((B, T, Hq, D), 13), rnd((B, T, Hkv, D), 14), rnd((B, T, Hkv, D), 15)
    beta = rnd((Hq, D), 16)
    o, _ = oracle.swa(q, np.zeros(Hq * D), beta, k, v, W)
    qb = np.broadcast_to(beta, (B, T, Hq, D))
    np.testing.assert_allclose(o, sdpa(qb, k, v, mask=band_mask(T, W)),
                               atol=1e-12)
    ox, _ = oracle.xattn(q[:, -5:], np.zeros(Hq * D), beta, k, v, T - 5)
    ref = sdpa(qb, k, v, causal=True)[:, -5:]
    np.testing.assert_allclose(ox, ref, atol=1e-12)


def test_channel_permutation_equivariance():
    """Permuting channels of q_pre, alpha, beta and K together leaves o
    unchanged; permuting V's channels permutes o. Catches per-channel
    alpha/beta indexed by the wrong channel or head."""
    B, T, Hq, Hkv, D, W = 1, 30, 4, 2, 16, 6
    rng = np.random.default_rng(17)
    q, k, v = rnd((B, T, Hq, D), 18), rnd((B, T, Hkv, D), 19), rnd((B, T, Hkv, D), 20)
    a, b = 1 + 0.3 * rnd((Hq, D), 21), 0.5 * rnd((Hq, D), 22)
    o, _ = oracle.swa(q, a, b, k, v, W)
    p = rng.permutation(D)
    pv = rng.permutation(D)
    o2, _ = oracle.swa(q[..., p], a[:, p], b[:, p], k[..., p], v[..., pv], W)
    np.testing.assert_allclose(o2, o[..., pv], atol=1e-12)


def test_head_permutation_and_map():
    """Permuting q heads (with their alpha/beta rows and a head map that
    follows them) permutes the outputs; GQA == KV heads replicated."""
    B, T, Hq, Hkv, D, W = 2, 25, 8, 2, 8, 5
    q, k, v = rnd((B, T, Hq, D), 23), rnd((B, T, Hkv, D), 24), rnd((B, T, Hkv, D), 25)
    a, b = 1 + 0.2 * rnd((Hq, D), 26), 0.2 * rnd((Hq, D), 27)
    o, _ = oracle.swa(q, a, b, k, v, W)
    # replicated KV heads, Hkv = Hq
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    o_rep, _ = oracle.swa(q, a, b, kr, vr, W)
    np.testing.assert_allclose(o_rep, o, atol=1e-12)
    # explicit permuted map
    perm = np.random.default_rng(28).permutation(Hq)
    hmap = (perm // G).astype(np.int32)
    o_p, _ = oracle.swa(q[:, :, perm], a[perm], b[perm], k, v, W,
                        head_map=hmap)
    np.testing.assert_allclose(o_p, o[:, :, perm], atol=1e-12)
    # explicit map vs torch with the same map
    hm2 = np.array([1, 0, 1, 1, 0, 0, 1, 0], dtype=np.int32)
    o_m, _ = oracle.swa(q, np.ones(Hq * D), np.zeros(Hq * D), k, v, W,
                        head_map=hm2)
    ref = sdpa(q, k, v, mask=band_mask(T, W), head_map=hm2)
    np.testing.assert_allclose(o_m, ref, atol=1e-12)


def test_batch_independence():
    B, T, Hq, Hkv, D, W = 3, 20, 2, 1, 8, 4
    q, k, v = rnd((B, T, Hq, D), 29), rnd((B, T, Hkv, D), 30), rnd((B, T, Hkv, D), 31)
    a, b = ident(Hq, D)
    o, _ = oracle.swa(q, a, b, k, v, W)
    k2 = k.copy()
    k2[1] += rnd(k2[1].shape, 99)  # (a constant shift would cancel)
    o2, _ = oracle.swa(q, a, b, k2, v, W)
    np.testing.assert_array_equal(o2[0], o[0])
    np.testing.assert_array_equal(o2[2], o[2])
    assert np.abs(o2[1] - o[1]).max() > 1e-3


# --- P2: weights sum to one over exactly the stated ranges -----------------

@pytest.mark.parametrize("W", [1, 3, 16, 64, 0])
def test_weight_support_and_sum(W):
    """W = 0 means the unbounded output-stream range [0, t]."""
    T, Hkv, D = 40, 2, 8
    k, v = rnd((T, Hkv, D), 32), rnd((T, Hkv, D), 33)
    qrow = rnd((D,), 34)
    a, b = 1 + 0.1 * rnd((D,), 35), 0.1 * rnd((D,), 36)
    for t in range(T):
        w = oracle.row_weights(qrow, a, b, k, v, t, W, g=1)
        lo = 0 if W <= 0 else max(0, t - W + 1)
        nz = np.flatnonzero(w)
        assert nz[0] == lo and nz[-1] == t and nz.size == t - lo + 1
        assert abs(w.sum() - 1.0) <= 1e-12
        assert (w[lo:t + 1] > 0).all()


# --- P5: closed forms -------------------------------------------------------

def test_window_one_returns_own_value():
    B, T, Hq, Hkv, D = 2, 17, 4, 2, 8
    q, k, v = rnd((B, T, Hq, D), 37), rnd((B, T, Hkv, D), 38), rnd((B, T, Hkv, D), 39)
    a, b = 1 + 0.1 * rnd(Hq * D, 40), 0.1 * rnd(Hq * D, 41)
    o, _ = oracle.swa(q, a, b, k, v, 1)
    np.testing.assert_array_equal(o, np.repeat(v, Hq // Hkv, axis=2))


def test_zero_query_gives_window_mean():
    B, T, Hq, Hkv, D, W = 1, 23, 2, 1, 4, 5
    q, k, v = rnd((B, T, Hq, D), 42), rnd((B, T, Hkv, D), 43), rnd((B, T, Hkv, D), 44)
    o, _ = oracle.swa(q, np.zeros(Hq * D), np.zeros(Hq * D), k, v, W)
    for t in range(T):
        mean = v[0, max(0, t - W + 1):t + 1, 0].mean(axis=0)
        for h in range(Hq):
            np.testing.assert_allclose(o[0, t, h], mean, atol=1e-14)


def test_constant_values_and_single_position():
    B, T, Hq, Hkv, D, W = 1, 12, 2, 2, 8, 4
    q, k = rnd((B, T, Hq, D), 45), rnd((B, T, Hkv, D), 46)
    c = rnd((D,), 47)
    v = np.broadcast_to(c, (B, T, Hkv, D)).copy()
    a, b = 1 + 0.1 * rnd(Hq * D, 48), 0.1 * rnd(Hq * D, 49)
    o, _ = oracle.swa(q, a, b, k, v, W)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-14)
    # V == 1 gives exactly 1 everywhere
    o1, _ = oracle.swa(q, a, b, k, np.ones_like(v), W)
    np.testing.assert_allclose(o1, 1.0, atol=1e-15)
    # T = 1: both streams return v_0
    o_t1, _ = oracle.swa(q[:, :1], a, b, k[:, :1], v[:, :1] + 1.5, 8)
    np.testing.assert_allclose(o_t1[0, 0, 0], c + 1.5, atol=1e-15)
    ox_t1, _ = oracle.xattn(q[:, :1], a, b, k[:, :1], v[:, :1] - 2.0, 0)
    np.testing.assert_allclose(ox_t1[0, 0, 1], c - 2.0, atol=1e-15)


def test_two_keys_logistic_closed_form():
    """t = 1, window 2: o = v0 + sigmoid(s1 - s0) (v1 - v0), s_j =
    q.k_j/sqrt(D) with q = alpha q_pre + beta; lse = logaddexp(s0, s1)."""
    D = 8
    q = rnd((1, 2, 1, D), 50)
    k, v = rnd((1, 2, 1, D), 51), rnd((1, 2, 1, D), 52)
    a, b = 1 + 0.3 * rnd(D, 53), 0.3 * rnd(D, 54)
    o, lse = oracle.swa(q, a, b, k, v, 2)
    qq = a * q[0, 1, 0] + b
    s0, s1 = (qq @ k[0, 0, 0]) / math.sqrt(D), (qq @ k[0, 1, 0]) / math.sqrt(D)
    sig = 1.0 / (1.0 + math.exp(-(s1 - s0)))
    np.testing.assert_allclose(o[0, 1, 0], v[0, 0, 0] + sig * (v[0, 1, 0] - v[0, 0, 0]),
                               atol=1e-14)
    np.testing.assert_allclose(lse[0, 1, 0], np.logaddexp(s0, s1), atol=1e-14)


def test_same_query_full_window_both_streams_agree():
    """alpha' = alpha, beta' = beta, q' = q and W >= t+1: o'_t == o_t."""
    B, T, Hq, Hkv, D = 2, 30, 4, 2, 8
    q, k, v = rnd((B, T, Hq, D), 55), rnd((B, T, Hkv, D), 56), rnd((B, T, Hkv, D), 57)
    a, b = 1 + 0.1 * rnd(Hq * D, 58), 0.1 * rnd(Hq * D, 59)
    o, _ = oracle.swa(q, a, b, k, v, T)
    T_in = 11
    ox, _ = oracle.xattn(q[:, T_in:], a, b, k, v, T_in)
    np.testing.assert_allclose(ox, o[:, T_in:], atol=1e-13)


@pytest.mark.parametrize("T,W", [(64, 16), (70, 16), (33, 1), (40, 13)])
def test_spike_probe_membership(T, W):
    """alpha = 0, beta = s e_0: every query is s e_0. K = 0 except spikes
    with k = s' e_0 (score 20), V = 0 except v_spike = e_c. Then o_t[c] =
    e^20 / (e^20 + n - 1) exactly when the spike lies in the row's range
    (n = range size), else 0."""
    D, Hq, Hkv = 8, 1, 1
    s_q, score = 4.0, 20.0
    s_k = score * math.sqrt(D) / s_q
    spikes = [0, W - 1, W, T - 1] + list(range(3, T, 2 * W + 3))
    spikes = sorted(set(j for j in spikes if 0 <= j < T))
    for j_star in spikes:
        k = np.zeros((1, T, Hkv, D))
        v = np.zeros((1, T, Hkv, D))
        k[0, j_star, 0, 0] = s_k
        c = 1 + j_star % (D - 1)
        v[0, j_star, 0, c] = 1.0
        beta = np.zeros(D)
        beta[0] = s_q
        q = rnd((1, T, Hq, D), 60)
        o, _ = oracle.swa(q, np.zeros(D), beta, k, v, W)
        ox, _ = oracle.xattn(q, np.zeros(D), beta, k, v, 0)
        for t in range(T):
            for (out, lo) in ((o, max(0, t - W + 1)), (ox, 0)):
                n = t - lo + 1
                inside = lo <= j_star <= t
                expect = (math.exp(score) / (math.exp(score) + n - 1)
                          if inside else 0.0)
                assert abs(out[0, t, 0, c] - expect) <= 1e-12, (t, j_star)


# --- P3: incremental == batched --------------------------------------------

def _gate():
    with open(os.path.join(GOLDEN, "paradigms.json")) as f:
        return json.load(f)["consistency_gate"]["gate_max_abs"]


@pytest.mark.parametrize("B,Hq,Hkv,D,T0,steps,W", [
    (2, 4, 2, 16, 20, 12, 8),
    (1, 2, 2, 16, 64, 5, 16),   # tiny configuration shape
    (3, 8, 2, 8, 5, 9, 100),    # window larger than the sequence
])
def test_incremental_prefill_then_decode_equals_batched(B, Hq, Hkv, D, T0,
                                                        steps, W):
    T = T0 + steps
    q, qx = rnd((B, T, Hq, D), 61), rnd((B, T, Hq, D), 62)
    k, v = rnd((B, T, Hkv, D), 63), rnd((B, T, Hkv, D), 64)
    a, b = 1 + 0.1 * rnd(Hq * D, 65), 0.1 * rnd(Hq * D, 66)
    ax, bx = 1 + 0.1 * rnd(Hq * D, 67), 0.1 * rnd(Hq * D, 68)
    o_b, _ = oracle.swa(q, a, b, k, v, W)
    ox_b, _ = oracle.xattn(qx[:, T0:], ax, bx, k, v, T0)

    cache = oracle.Cache(B, Hkv, D, cap=T + 3)
    cache.append(k[:, :T0], v[:, :T0])
    assert all(cache.length(bi) == T0 for bi in range(B))
    for s in range(steps):
        t = T0 + s
        o_i, ox_i = cache.decode_pair(q[:, t], qx[:, t], a, b, ax, bx,
                                      k[:, t], v[:, t], W)
        assert np.abs(o_i - o_b[:, t]).max() <= _gate()
        assert np.abs(ox_i - ox_b[:, s]).max() <= _gate()
        np.testing.assert_allclose(o_i, o_b[:, t], atol=1e-12)
        np.testing.assert_allclose(ox_i, ox_b[:, s], atol=1e-12)
    assert all(cache.length(bi) == T for bi in range(B))


def test_decode_appends_before_attending():
    """The base query of a decode step sees its own new key: with W = 1 the
    base output is exactly the new value."""
    B, Hq, Hkv, D = 1, 2, 1, 8
    cache = oracle.Cache(B, Hkv, D, cap=8)
    cache.append(rnd((B, 3, Hkv, D), 69), rnd((B, 3, Hkv, D), 70))
    kn, vn = rnd((B, Hkv, D), 71), rnd((B, Hkv, D), 72)
    o, ox = cache.decode_pair(rnd((B, Hq, D), 73), rnd((B, Hq, D), 74),
                              np.ones(Hq * D), np.zeros(Hq * D),
                              np.ones(Hq * D), np.zeros(Hq * D), kn, vn, 1)
    np.testing.assert_array_equal(o[0, 0], vn[0, 0])
    assert cache.length(0) == 4


def test_cache_capacity_is_enforced():
    cache = oracle.Cache(1, 1, 4, cap=2)
    cache.append(np.zeros((1, 2, 1, 4)), np.zeros((1, 2, 1, 4)))
    with pytest.raises(ValueError):
        cache.append(np.zeros((1, 1, 1, 4)), np.zeros((1, 1, 1, 4)))


def test_row_sample_matches_full_evaluation():
    B, T, Hq, Hkv, D, W = 2, 50, 4, 2, 8, 7
    q, k, v = rnd((B, T, Hq, D), 75), rnd((B, T, Hkv, D), 76), rnd((B, T, Hkv, D), 77)
    a, b = 1 + 0.1 * rnd(Hq * D, 78), 0.1 * rnd(Hq * D, 79)
    o, lse = oracle.swa(q, a, b, k, v, W)
    rows = np.array([[0, 0], [1, 49], [0, 6], [1, 7], [1, 20]])
    o_s, lse_s = oracle.swa(q, a, b, k, v, W, rows=rows)
    for i, (bb, t) in enumerate(rows):
        np.testing.assert_array_equal(o_s[i], o[bb, t])
        np.testing.assert_array_equal(lse_s[i], lse[bb, t])
    ox, _ = oracle.xattn(q[:, 40:], a, b, k, v, 40)
    ox_s, _ = oracle.xattn(q[:, 40:], a, b, k, v, 40, rows=[[1, 3], [0, 9]])
    np.testing.assert_array_equal(ox_s[0], ox[1, 3])
    np.testing.assert_array_equal(ox_s[1], ox[0, 9])


def test_invalid_arguments_raise():
    q = np.zeros((1, 4, 2, 4))
    k = np.zeros((1, 4, 1, 4))
    with pytest.raises(ValueError):
        oracle.swa(q, np.ones(8), np.zeros(8), k, k, 0)          # W < 1
    with pytest.raises(ValueError):
        oracle.swa(q, np.ones(8), np.zeros(8), k, k, 2,
                   head_map=np.array([0, 1], dtype=np.int32))     # map >= Hkv


# --- the layer with its projections (oracle.layer) ---------------------------

def torch_layer(x, w_q, w_k, w_v, w_o, a, b, ax, bx, T_out, W, Hkv, D):
    """Independent fp64 evaluation of one layer: torch matmuls, the affine
    written out, and scaled_dot_product_attention with triangular band masks
    (base rows) and causal rows (output rows)."""
    X = torch.from_numpy(x).double()
    B, M, _ = X.shape
    T = M - T_out
    Hq = w_q.shape[1] // D
    t = lambda z: torch.from_numpy(np.ascontiguousarray(z)).double()  # noqa
    q_all = X @ t(w_q)
    q = t(a) * q_all[:, :T] + t(b)
    k = (X[:, :T] @ t(w_k)).reshape(B, T, Hkv, D).numpy()
    v = (X[:, :T] @ t(w_v)).reshape(B, T, Hkv, D).numpy()
    o = sdpa(q.reshape(B, T, Hq, D).numpy(), k, v, mask=band_mask(T, W))
    parts = [o]
    if T_out:
        qx = (t(ax) * q_all[:, T:] + t(bx)).reshape(B, T_out, Hq, D).numpy()
        rows = band_mask(T, T, q_offset=T - T_out)   # causal rows T_in..T-1
        parts.append(sdpa(qx, k, v, mask=rows))
    o_cat = np.concatenate(parts, axis=1).reshape(B, M, Hq * D)
    return o_cat @ w_o


def layer_case(B, T, T_out, dm, Hq, Hkv, D, seed):
    x = rnd((B, T + T_out, dm), seed)
    w = [rnd(s, seed + i + 1, 1 / math.sqrt(s[0])) for i, s in
         enumerate([(dm, Hq * D), (dm, Hkv * D), (dm, Hkv * D), (Hq * D, dm)])]
    a, b = 1 + 0.1 * rnd(Hq * D, seed + 5), 0.1 * rnd(Hq * D, seed + 6)
    ax, bx = 1 + 0.1 * rnd(Hq * D, seed + 7), 0.1 * rnd(Hq * D, seed + 8)
    return x, w, (a, b, ax, bx)


@pytest.mark.parametrize("B,T,T_out,dm,Hq,Hkv,D,W", [
    (2, 30, 3, 24, 4, 2, 8, 7),
    (1, 40, 40, 16, 2, 1, 8, 5),     # every position also an output row (PT)
    (1, 25, 0, 16, 2, 2, 8, 100),    # no output rows; W above T
    (2, 33, 1, 32, 4, 4, 8, 1),      # window of one
])
def test_layer_equals_masked_attention_with_projections(B, T, T_out, dm, Hq,
                                                         Hkv, D, W):
    x, w, aff = layer_case(B, T, T_out, dm, Hq, Hkv, D, 300 + T)
    got = oracle.layer(x, *w, *aff, T_out, W, Hkv, D)
    ref = torch_layer(x, *w, *aff, T_out, W, Hkv, D)
    assert got.shape == (B, T + T_out, dm)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_layer_rows_mode_equals_full_mode():
    B, T, T_out, dm, Hq, Hkv, D, W = 2, 50, 4, 16, 4, 2, 8, 9
    x, w, aff = layer_case(B, T, T_out, dm, Hq, Hkv, D, 401)
    full = oracle.layer(x, *w, *aff, T_out, W, Hkv, D)
    rows = [0, 1, 8, 9, 10, 49, 50, 53]
    part = oracle.layer(x, *w, *aff, T_out, W, Hkv, D, rows=rows)
    np.testing.assert_allclose(part, full[:, rows], rtol=1e-12, atol=1e-13)


def test_layer_output_row_order_and_causality():
    """Output rows depend only on their own hidden row and on base rows up
    to their position; base rows never see the output rows."""
    B, T, T_out, dm, Hq, Hkv, D, W = 1, 20, 3, 16, 2, 1, 8, 6
    x, w, aff = layer_case(B, T, T_out, dm, Hq, Hkv, D, 501)
    y0 = oracle.layer(x, *w, *aff, T_out, W, Hkv, D)
    x1 = x.copy()
    x1[:, T + 1] += 1.0                      # output row of position T_in+1
    y1 = oracle.layer(x1, *w, *aff, T_out, W, Hkv, D)
    changed = np.abs(y1 - y0).max(axis=(0, 2)) > 0
    assert changed.tolist() == [i == T + 1 for i in range(T + T_out)]
    x2 = x.copy()
    x2[:, T - 1] += 1.0                      # the last base row (position T-1)
    y2 = oracle.layer(x2, *w, *aff, T_out, W, Hkv, D)
    changed = np.abs(y2 - y0).max(axis=(0, 2)) > 0
    T_in = T - T_out
    expect = [T - 1 <= i < T or i == T + T_out - 1
              for i in range(T + T_out)]
    assert changed.tolist() == expect, (changed, T_in)


# --- training gradients (oracle.attn_backward) --------------------------------

def torch_streams_grad(q_pre, qx_pre, a, b, ax, bx, k, v, d_o, d_ox, W,
                       head_map=None):
    """torch autograd (fp64) of <o, d_o> + <o', d_ox> through the affine and
    scaled_dot_product_attention with triangular masks."""
    t = lambda z: torch.from_numpy(np.ascontiguousarray(z)).double().requires_grad_()  # noqa
    qp, qxp, A, Bt, AX, BX, K, V = (t(z) for z in
                                    (q_pre, qx_pre, a, b, ax, bx, k, v))
    B, T, Hq, D = q_pre.shape
    T_out = qx_pre.shape[1]
    Hkv = k.shape[2]
    idx = (torch.arange(Hq) // (Hq // Hkv) if head_map is None
           else torch.as_tensor(head_map, dtype=torch.long))
    Kh = K.index_select(2, idx).permute(0, 2, 1, 3)
    Vh = V.index_select(2, idx).permute(0, 2, 1, 3)
    q = (A.reshape(Hq, D) * qp + Bt.reshape(Hq, D)).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(q, Kh, Vh, attn_mask=torch.from_numpy(
        band_mask(T, W)))
    loss = (o.permute(0, 2, 1, 3) * torch.from_numpy(d_o)).sum()
    if T_out:
        qx = (AX.reshape(Hq, D) * qxp + BX.reshape(Hq, D)).permute(0, 2, 1, 3)
        ox = F.scaled_dot_product_attention(qx, Kh, Vh, attn_mask=torch.from_numpy(
            band_mask(T, T, q_offset=T - T_out)))
        loss = loss + (ox.permute(0, 2, 1, 3) * torch.from_numpy(d_ox)).sum()
    loss.backward()
    grad = lambda z: np.zeros(z.shape) if z.grad is None else z.grad.numpy()  # noqa
    return {"dq_pre": grad(qp), "dqx_pre": grad(qxp), "dk": grad(K),
            "dv": grad(V), "d_alpha": grad(A), "d_beta": grad(Bt),
            "d_alpha_x": grad(AX), "d_beta_x": grad(BX)}


def grad_case(B, T, T_out, Hq, Hkv, D, seed):
    q, qx = rnd((B, T, Hq, D), seed), rnd((B, T_out, Hq, D), seed + 1)
    k, v = rnd((B, T, Hkv, D), seed + 2), rnd((B, T, Hkv, D), seed + 3)
    a, b = 1 + 0.1 * rnd(Hq * D, seed + 4), 0.1 * rnd(Hq * D, seed + 5)
    ax, bx = 1 + 0.1 * rnd(Hq * D, seed + 6), 0.1 * rnd(Hq * D, seed + 7)
    d_o, d_ox = rnd((B, T, Hq, D), seed + 8), rnd((B, T_out, Hq, D), seed + 9)
    return q, qx, a, b, ax, bx, k, v, d_o, d_ox


@pytest.mark.parametrize("B,T,T_out,Hq,Hkv,D,W", [
    (2, 23, 5, 4, 2, 8, 6),       # SFT-like: a few output rows
    (1, 17, 17, 2, 1, 16, 4),     # PT: every position an output row
    (1, 20, 0, 4, 4, 8, 1),       # base stream only, window of one
    (1, 12, 2, 2, 2, 8, 50),      # window above T
])
def test_backward_equals_autograd(B, T, T_out, Hq, Hkv, D, W):
    args = grad_case(B, T, T_out, Hq, Hkv, D, 700 + T)
    got = oracle.attn_backward(*args, W)
    ref = torch_streams_grad(*args, W)
    for name in ref:
        np.testing.assert_allclose(got[name], ref[name], rtol=1e-10,
                                   atol=1e-11, err_msg=name)


def test_backward_custom_head_map_equals_autograd():
    hm = [1, 0, 1]
    args = list(grad_case(1, 15, 3, 3, 2, 8, 777))
    got = oracle.attn_backward(*args, 5, head_map=hm)
    ref = torch_streams_grad(*args, 5, head_map=hm)
    for name in ref:
        np.testing.assert_allclose(got[name], ref[name], rtol=1e-10,
                                   atol=1e-11, err_msg=name)


def test_backward_finite_differences():
    """Central differences of <o, d_o> + <o', d_ox> through the forward
    oracle for a few coordinates of every input."""
    B, T, T_out, Hq, Hkv, D, W = 1, 9, 2, 2, 1, 4, 3
    q, qx, a, b, ax, bx, k, v, d_o, d_ox = grad_case(B, T, T_out, Hq, Hkv, D,
                                                     901)
    g = oracle.attn_backward(q, qx, a, b, ax, bx, k, v, d_o, d_ox, W)

    def loss(q, qx, a, b, ax, bx, k, v):
        o, _ = oracle.swa(q, a, b, k, v, W)
        ox, _ = oracle.xattn(qx, ax, bx, k, v, T - T_out)
        return float((o * d_o).sum() + (ox * d_ox).sum())

    base = [q, qx, a, b, ax, bx, k, v]
    names = ["dq_pre", "dqx_pre", "d_alpha", "d_beta", "d_alpha_x",
             "d_beta_x", "dk", "dv"]
    rng = np.random.default_rng(5)
    eps = 1e-6
    for i, name in enumerate(names):
        for _ in range(3):
            idx = tuple(int(rng.integers(0, n)) for n in base[i].shape)
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[i][idx] += eps
            minus[i][idx] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(fd - g[name][idx]) < 1e-6, (name, idx, fd, g[name][idx])


def test_backward_sampled_equals_full():
    """The sampled backward (matrix form over the rows that see each key)
    equals the row-by-row one on every sampled entry."""
    B, T, T_out, Hq, Hkv, D, W = 2, 40, 7, 4, 2, 8, 9
    args = grad_case(B, T, T_out, Hq, Hkv, D, 811)
    full = oracle.attn_backward(*args, W)
    rows, out_rows, keys = [0, 5, 8, 9, 39], [0, 3, 6], [0, 4, 30, 33, 39]
    for b in range(B):
        for g in range(Hkv):
            dq, dqx, dk, dv = oracle.attn_backward_sampled(
                *args, W, b, rows, out_rows, keys, g)
            np.testing.assert_allclose(dq, full["dq_pre"][b, rows], atol=1e-12)
            np.testing.assert_allclose(dqx, full["dqx_pre"][b, out_rows], atol=1e-12)
            np.testing.assert_allclose(dk, full["dk"][b, keys, g], atol=1e-12)
            np.testing.assert_allclose(dv, full["dv"][b, keys, g], atol=1e-12)


def test_backward_head_subset_equals_autograd():
    """A subset of query heads (and no dK/dV sums) gives those heads' exact
    entries of every per-head gradient, compared with torch autograd; the
    other heads' entries and dK/dV stay zero."""
    B, T, T_out, Hq, Hkv, D, W = 2, 19, 4, 4, 2, 8, 5
    args = grad_case(B, T, T_out, Hq, Hkv, D, 931)
    heads = [1, 3]
    got = oracle.attn_backward(*args, W, heads=heads, with_kv=False)
    ref = torch_streams_grad(*args, W)
    for name in ("d_alpha", "d_beta", "d_alpha_x", "d_beta_x"):
        g2, r2 = got[name].reshape(Hq, D), ref[name].reshape(Hq, D)
        np.testing.assert_allclose(g2[heads], r2[heads], rtol=1e-10,
                                   atol=1e-11, err_msg=name)
        assert (g2[[0, 2]] == 0).all()
    for name in ("dq_pre", "dqx_pre"):
        np.testing.assert_allclose(got[name][:, :, heads], ref[name][:, :, heads],
                                   rtol=1e-10, atol=1e-11, err_msg=name)
        assert (got[name][:, :, [0, 2]] == 0).all()
    assert (got["dk"] == 0).all() and (got["dv"] == 0).all()
