"""Full-size configurations on the GPU, in the launch configuration the
benchmark times, checked against the fp64 oracle.

Coverage (each test stays well inside a two-minute limit on the GPU host's
cores, so the big cases are split into several tests that share one GPU run
through a module fixture):
  * prefill_32k: every base-stream row of every head (four slices of 8192
    rows), and the output-stream row.
  * sft_dual_8k: every base-stream row and every output-stream row of every
    head, one test per batch entry.
  * prefill_128k: every 64-row tile edge and its two neighbours (t = 64 i - 1,
    64 i, 64 i + 1), the band edges, and 4096 seeded random rows, all heads
    (two tests); the output row; the full causal run and W = 128 on sampled
    rows.
  * decode_pair_b64: all 64 sequences at steps 0, 1, 127 and 255, and four
    sequences at every one of the 256 steps (the latter against the oracle's
    incremental cache, fed the same appended tokens).
  * the backward at the SFT shape: sampled dq rows, dK/dV keys, and the
    scale-offset gradients of four heads over every row.
A base-stream row t is checked over exactly its key slice [max(0, t-W+1), t]
(the pages' range; paper text §3.1), an output row over [0, t].
"""
import numpy as np
import pytest
import torch

import long_context_prefill_swa_amd as lo
import oracle
from gpu_util import TOL, compare, f64, make_cache, say
from workloads import (affine_inputs, decode_all_steps, kv_inputs, normal,
                       prefill_inputs, workload)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


def run_prefill(cfg, cfg_id, W=None):
    """The benchmark's prefill calls (append, window, output stream)."""
    W = cfg.W if W is None else W
    x = prefill_inputs(cfg, cfg_id, DEV)
    B, T, Hq, D = x.q_pre.shape
    kc = torch.empty((B, cfg.Hkv, T, D), dtype=x.k.dtype, device=DEV)
    vc = torch.empty_like(kc)
    cl = torch.zeros(B, dtype=torch.int32, device=DEV)
    lo.orthros_kv_append(kc, vc, cl, x.k, x.v)
    o = torch.empty_like(x.q_pre)
    lo.orthros_swa_prefill(x.q_pre, x.alpha, x.beta, kc, vc, o, W)
    ox = torch.empty_like(x.qx_pre)
    lo.orthros_global_xattn(x.qx_pre, x.alpha_x, x.beta_x, kc, vc, ox,
                            cfg.T_in)
    torch.cuda.synchronize()
    assert cl.tolist() == [T] * B
    return x, kc, vc, o, ox


def check_rows_sliced(o, q, a, b, k_host, v_host, ts, W, what, batch=0):
    """Rows ts of batch entry `batch`, each over its own key slice."""
    got, ref = [], []
    qh = f64(q[batch:batch + 1, ts])          # [1, n, Hq, D]
    for i, t in enumerate(ts):
        lo_t = 0 if W is None else max(0, t - W + 1)
        r, _ = oracle.xattn(qh[:, i:i + 1], a, b,
                            k_host[batch:batch + 1, lo_t:t + 1],
                            v_host[batch:batch + 1, lo_t:t + 1], t - lo_t)
        ref.append(r)
    got = f64(o[batch:batch + 1, ts])
    compare(got, np.concatenate(ref, 1), BF,
            f"{what} ({len(ts)} rows x all heads)")


# ---- prefill_32k: every row -------------------------------------------------

@pytest.fixture(scope="module")
def p32k():
    cfg, cid = workload("prefill_32k")
    say(f"[full size] {cfg.name}: GPU run")
    x, kc, vc, o, ox = run_prefill(cfg, cid)
    host = dict(q=f64(x.q_pre), k=f64(x.k), v=f64(x.v), a=f64(x.alpha),
                b=f64(x.beta), qx=f64(x.qx_pre), ax=f64(x.alpha_x),
                bx=f64(x.beta_x), o=f64(o), ox=f64(ox))
    del x, kc, vc, o, ox
    torch.cuda.empty_cache()
    return cfg, host


@pytest.mark.parametrize("part", range(4))
def test_prefill_32k_every_row(p32k, part):
    cfg, h = p32k
    n = cfg.T // 4
    t0 = part * n
    say(f"[full size] prefill_32k rows {t0}..{t0 + n - 1}, all heads")
    rows = np.array([(0, t) for t in range(t0, t0 + n)], np.int64)
    ref, _ = oracle.swa(h["q"], h["a"], h["b"], h["k"], h["v"], cfg.W,
                        rows=rows)
    compare(h["o"][0, t0:t0 + n], ref, BF, f"base stream rows {t0}+{n}")
    if part == 0:
        rx, _ = oracle.xattn(h["qx"], h["ax"], h["bx"], h["k"], h["v"],
                             cfg.T_in)
        compare(h["ox"], rx, BF, "output row over every key")


# ---- sft_dual_8k: every row of both streams ---------------------------------

@pytest.fixture(scope="module")
def sft():
    cfg, cid = workload("sft_dual_8k")
    say(f"[full size] {cfg.name}: GPU run")
    x, kc, vc, o, ox = run_prefill(cfg, cid)
    host = dict(q=f64(x.q_pre), k=f64(x.k), v=f64(x.v), a=f64(x.alpha),
                b=f64(x.beta), qx=f64(x.qx_pre), ax=f64(x.alpha_x),
                bx=f64(x.beta_x), o=f64(o), ox=f64(ox))
    del x, kc, vc, o, ox
    torch.cuda.empty_cache()
    return cfg, host


@pytest.mark.parametrize("b", range(4))
def test_sft_dual_8k_every_row(sft, b):
    cfg, h = sft
    say(f"[full size] sft_dual_8k batch {b}: {cfg.T} base + {cfg.T_out} "
        "output rows, all heads")
    rows = np.array([(b, t) for t in range(cfg.T)], np.int64)
    ref, _ = oracle.swa(h["q"], h["a"], h["b"], h["k"], h["v"], cfg.W,
                        rows=rows)
    compare(h["o"][b], ref, BF, f"b={b} base stream, every row")
    rows_x = np.array([(b, r) for r in range(cfg.T_out)], np.int64)
    rx, _ = oracle.xattn(h["qx"], h["ax"], h["bx"], h["k"], h["v"], cfg.T_in,
                         rows=rows_x)
    compare(h["ox"][b], rx, BF, f"b={b} output stream, every row")


# ---- prefill_128k: tile edges and random rows ------------------------------

@pytest.fixture(scope="module")
def p128k():
    cfg, cid = workload("prefill_128k")
    say(f"[full size] {cfg.name}: GPU run")
    x, kc, vc, o, ox = run_prefill(cfg, cid)
    del kc, vc
    host = dict(k=f64(x.k), v=f64(x.v), a=f64(x.alpha), b=f64(x.beta))
    return cfg, cid, x, o, ox, host


def rows_128k(cfg, seed):
    T, W = cfg.T, cfg.W
    ts = {0, 1, W - 2, W - 1, W, W + 1, T - 2, T - 1}
    for e in range(0, T + 1, 64):
        ts.update((e - 1, e, e + 1))
    rng = np.random.default_rng(seed)
    extra = set()
    while len(extra) < 4096:
        t = int(rng.integers(0, T))
        if t not in ts:
            extra.add(t)
    return sorted(t for t in ts | extra if 0 <= t < T)


@pytest.mark.parametrize("part", range(2))
def test_prefill_128k_tile_edges_and_random_rows(p128k, part):
    cfg, cid, x, o, ox, h = p128k
    ts = rows_128k(cfg, cid)
    half = ts[part::2]
    say(f"[full size] prefill_128k: {len(half)} of {len(ts)} rows "
        "(every tile edge +-1, band edges, 4096 random), all heads")
    check_rows_sliced(o, x.q_pre, h["a"], h["b"], h["k"], h["v"], half, cfg.W,
                      "base stream")
    if part == 0:
        rx, _ = oracle.xattn(f64(x.qx_pre), f64(x.alpha_x), f64(x.beta_x),
                             h["k"], h["v"], cfg.T_in)
        compare(ox, rx, BF, "output row over 131072 keys")


def test_long_prefill_full_causal_sampled(p128k):
    """The same-T full causal run used for the speedup ratio (W = T)."""
    cfg, cid, x, _, _, h = p128k
    say("[full size] prefill_128k full causal")
    kc, vc, _ = make_cache(x.k, x.v, cfg.T)
    o = torch.empty_like(x.q_pre)
    lo.orthros_swa_prefill(x.q_pre, x.alpha, x.beta, kc, vc, o, cfg.T)
    torch.cuda.synchronize()
    ts = [0, 1, 63, 64, 4095, 4096, 65535, 65536, cfg.T - 65, cfg.T - 64,
          cfg.T - 1]
    check_rows_sliced(o, x.q_pre, h["a"], h["b"], h["k"], h["v"], ts, None,
                      "causal")


def test_long_prefill_trained_window_sampled(p128k):
    """The 128K prefill at the window the paper trains with (W = 128), which
    runs the rolling-window kernel: tile edges of every 16th tile plus
    random rows."""
    cfg, cid, x, _, _, h = p128k
    say("[full size] prefill_128k W=128")
    kc, vc, _ = make_cache(x.k, x.v, cfg.T)
    o = torch.empty_like(x.q_pre)
    lo.orthros_swa_prefill(x.q_pre, x.alpha, x.beta, kc, vc, o, 128)
    torch.cuda.synchronize()
    ts = {0, 1, 126, 127, 128, 129, cfg.T - 1}
    for e in range(0, cfg.T, 1024):
        ts.update((e - 1, e, e + 1))
    ts.update(int(t) for t in np.random.default_rng(cid + 7).integers(0, cfg.T, 1024))
    ts = sorted(t for t in ts if 0 <= t < cfg.T)
    check_rows_sliced(o, x.q_pre, h["a"], h["b"], h["k"], h["v"], ts, 128,
                      "base stream W=128")


# ---- decode_pair_b64 --------------------------------------------------------

KEY_STEPS = (0, 1, 127, 255)
EVERY_STEP_SEQS = (0, 21, 42, 63)


@pytest.fixture(scope="module")
def decode_b64():
    cfg, cid = workload("decode_pair_b64")
    B, Hq, Hkv, D, L0, W = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.T, cfg.W
    steps = cfg.decode_steps
    say(f"[full size] {cfg.name}: {steps} steps on the GPU")
    k0, v0 = kv_inputs(cfg, cid, DEV)          # the 32768 cached tokens
    st = decode_all_steps(cfg, cid, device=DEV)
    cap = L0 + steps
    kc = torch.empty((B, Hkv, cap, D), dtype=BF, device=DEV)
    vc = torch.empty_like(kc)
    cl = torch.zeros(B, dtype=torch.int32, device=DEV)
    lo.orthros_kv_append(kc, vc, cl, k0, v0)
    a, b, ax, bx = affine_inputs(cfg, cid, DEV)
    ws = lo.workspace(lo.orthros_workspace_bytes(lo.ORTHROS_OP_DECODE_PAIR, B,
                                                 Hq, Hkv, D, 1, cap), DEV)
    o_all = torch.empty((steps, B, Hq, D), dtype=BF, device=DEV)
    ox_all = torch.empty_like(o_all)
    for s in range(steps):
        lo.orthros_decode_pair(st.q_pre[s], st.qx_pre[s], a, b, ax, bx,
                               st.k_new[s], st.v_new[s], kc, vc, cl, o_all[s],
                               ox_all[s], max_len_after=L0 + s + 1, W=W, ws=ws)
    torch.cuda.synchronize()
    lo.orthros_check_device_errors()
    assert cl.tolist() == [L0 + steps] * B, "cache lengths"
    # appended rows are the step tokens, bit for bit, for every sequence
    assert torch.equal(kc[:, :, L0:].permute(2, 0, 1, 3).contiguous().view(torch.int16),
                       st.k_new.contiguous().view(torch.int16))
    assert torch.equal(vc[:, :, L0:].permute(2, 0, 1, 3).contiguous().view(torch.int16),
                       st.v_new.contiguous().view(torch.int16))
    host = dict(a=f64(a), b=f64(b), ax=f64(ax), bx=f64(bx))
    return cfg, st, kc, vc, k0, v0, o_all, ox_all, host


@pytest.mark.parametrize("half", range(2))
def test_decode_all_sequences_at_key_steps(decode_b64, half):
    cfg, st, kc, vc, _, _, o_all, ox_all, h = decode_b64
    L0, W = cfg.T, cfg.W
    seqs = range(half * 32, half * 32 + 32)
    say(f"[full size] decode: sequences {seqs[0]}..{seqs[-1]} at steps "
        f"{KEY_STEPS}")
    got_b, ref_b, got_x, ref_x = [], [], [], []
    for bi in seqs:
        kb = f64(kc[bi].permute(1, 0, 2))[None]     # [1, cap, Hkv, D]
        vb = f64(vc[bi].permute(1, 0, 2))[None]
        for s in KEY_STEPS:
            n = L0 + s                               # index of the new key
            lo_t = max(0, n - W + 1)
            rb, _ = oracle.xattn(f64(st.q_pre[s][bi:bi + 1, None]), h["a"],
                                 h["b"], kb[:, lo_t:n + 1], vb[:, lo_t:n + 1],
                                 n - lo_t)
            rx, _ = oracle.xattn(f64(st.qx_pre[s][bi:bi + 1, None]), h["ax"],
                                 h["bx"], kb[:, :n + 1], vb[:, :n + 1], n)
            ref_b.append(rb)
            ref_x.append(rx)
            got_b.append(f64(o_all[s, bi:bi + 1, None]))
            got_x.append(f64(ox_all[s, bi:bi + 1, None]))
    compare(np.concatenate(got_b), np.concatenate(ref_b), BF,
            f"base rows, {len(got_b)} (sequence, step) pairs")
    compare(np.concatenate(got_x), np.concatenate(ref_x), BF,
            f"output rows, {len(got_x)} (sequence, step) pairs")


@pytest.mark.parametrize("bi", EVERY_STEP_SEQS)
def test_decode_one_sequence_every_step(decode_b64, bi):
    """Sequence bi at all 256 steps against the oracle's incremental cache
    (its own decode-pair code path), fed the cached tokens and then each
    step's appended token."""
    cfg, st, _, _, k0, v0, o_all, ox_all, h = decode_b64
    L0, W, steps = cfg.T, cfg.W, cfg.decode_steps
    say(f"[full size] decode: sequence {bi} at every step")
    cache = oracle.Cache(1, cfg.Hkv, cfg.D, L0 + steps)
    cache.append(f64(k0[bi:bi + 1]), f64(v0[bi:bi + 1]))
    q = f64(st.q_pre[:, bi:bi + 1])
    qx = f64(st.qx_pre[:, bi:bi + 1])
    kn = f64(st.k_new[:, bi:bi + 1])
    vn = f64(st.v_new[:, bi:bi + 1])
    ref_b, ref_x = [], []
    for s in range(steps):
        rb, rx = cache.decode_pair(q[s], qx[s], h["a"], h["b"], h["ax"],
                                   h["bx"], kn[s], vn[s], W)
        ref_b.append(rb)
        ref_x.append(rx)
    assert cache.length(0) == L0 + steps
    compare(o_all[:, bi:bi + 1], np.stack(ref_b), BF,
            f"b={bi} base rows, every step")
    compare(ox_all[:, bi:bi + 1], np.stack(ref_x), BF,
            f"b={bi} output rows, every step")


# ---- the largest cache the MFMA paths accept --------------------------------

def test_largest_cache_length():
    """The largest cache the MFMA paths accept: T = 2^24 - 1 keys, whose
    byte offsets within one (sequence, KV head) slab just fit the 32-bit
    buffer offsets. One KV head with four query heads (about 47 GB on the
    GPU). Checked: sampled base-stream rows at W = 4096 (persistent kernel)
    and at W = 128 (rolling kernel), and the output-stream row at the last
    position over all 2^24 - 1 keys. Its reference is the oracle evaluated
    over 16 key slices, each with every key visible, whose results are
    combined by their log-sum-exp weights (exact: o = sum_c
    exp(lse_c - L) o_c with L = log sum_c exp(lse_c))."""
    B, Hq, Hkv, D = 1, 4, 1, 128
    T = (1 << 24) - 1
    dt = BF
    say(f"[full size] largest cache: T={T} Hq={Hq} Hkv={Hkv}")
    q = normal((B, T, Hq, D), 9101, dt, DEV)
    k = normal((B, T, Hkv, D), 9102, dt, DEV)
    v = normal((B, T, Hkv, D), 9103, dt, DEV)
    qx = normal((B, 1, Hq, D), 9104, dt, DEV)
    a = 1 + 0.1 * normal((Hq * D,), 9105, torch.float32, DEV)
    b = 0.1 * normal((Hq * D,), 9106, torch.float32, DEV)
    kc = torch.empty((B, Hkv, T, D), dtype=dt, device=DEV)
    vc = torch.empty_like(kc)
    cl = torch.zeros(B, dtype=torch.int32, device=DEV)
    lo.orthros_kv_append(kc, vc, cl, k, v)
    o = torch.empty_like(q)
    ox = torch.empty_like(qx)
    lo.orthros_global_xattn(qx, a, b, kc, vc, ox, T - 1)
    torch.cuda.synchronize()
    assert cl.tolist() == [T]
    ts = [0, 1, 4095, 4096, (1 << 23) - 1, 1 << 23, T - 65, T - 64, T - 2,
          T - 1]
    for W in (4096, 128):
        lo.orthros_swa_prefill(q, a, b, kc, vc, o, W)
        torch.cuda.synchronize()
        got, ref = [], []
        for t in ts:
            lo_t = max(0, t - W + 1)
            r, _ = oracle.xattn(f64(q[:, t:t + 1]), f64(a), f64(b),
                                f64(k[:, lo_t:t + 1]), f64(v[:, lo_t:t + 1]),
                                t - lo_t)
            ref.append(r)
            got.append(f64(o[:, t:t + 1]))
        compare(np.concatenate(got, 1), np.concatenate(ref, 1), dt,
                f"base stream W={W} ({len(ts)} rows)")
    del o
    torch.cuda.empty_cache()
    # output stream over every key, as 16 slices merged by log-sum-exp
    n_sl = 16
    bounds = [T * i // n_sl for i in range(n_sl + 1)]
    outs, lses = [], []
    for s0, s1 in zip(bounds[:-1], bounds[1:]):
        r, l = oracle.xattn(f64(qx), f64(a), f64(b), f64(k[:, s0:s1]),
                            f64(v[:, s0:s1]), s1 - s0 - 1)
        outs.append(r)     # [B, 1, Hq, D]
        lses.append(l)     # [B, 1, Hq]
    lse = np.stack(lses)                       # [n_sl, B, 1, Hq]
    L = lse.max(0) + np.log(np.exp(lse - lse.max(0)).sum(0))
    wts = np.exp(lse - L)[..., None]           # [n_sl, B, 1, Hq, 1]
    ref = (wts * np.stack(outs)).sum(0)
    compare(ox, ref, dt, f"output row over {T} keys")
