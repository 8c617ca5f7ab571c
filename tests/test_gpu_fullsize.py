"""Full-size configurations on the GPU, in the launch configuration the
benchmark times, checked against the fp64 oracle on sampled rows.

A base-stream row t is checked by evaluating the oracle's softmax formula
over exactly the key slice [max(0, t-W+1), t] (the output-stream routine over
that slice with all of it visible), so the oracle never has to convert the
whole query tensor. Sampled rows: the band edges t in {0, 1, W-2, W-1, W,
T-2, T-1}, tile edges +-1 and seeded random rows, every batch entry, every
head.
"""
import numpy as np
import pytest
import torch

import long_context_prefill_swa_amd as lo
import oracle
from gpu_util import compare, f64, say
from workloads import (affine_inputs, decode_all_steps, kv_inputs,
                       prefill_inputs, workload)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def sample_rows(T, W, n_random, seed):
    base = {0, 1, W - 2, W - 1, W, T - 2, T - 1}
    for e in (64, 128, 4096, T // 2):
        for d in (-1, 0, 1):
            base.add(e + d)
    rng = np.random.default_rng(seed)
    base.update(int(x) for x in rng.integers(0, T, n_random))
    return sorted(t for t in base if 0 <= t < T)


def check_rows(o, q, a, b, k_host, v_host, ts, W, what):
    """o, q on GPU [B,T,Hq,D]; k_host, v_host float64 [B,T,Hkv,D]."""
    got, ref = [], []
    for t in ts:
        lo_t = 0 if W is None else max(0, t - W + 1)
        r, _ = oracle.xattn(f64(q[:, t:t + 1]), f64(a), f64(b),
                            k_host[:, lo_t:t + 1], v_host[:, lo_t:t + 1],
                            t - lo_t)
        ref.append(r)
        got.append(f64(o[:, t:t + 1]))
    compare(np.concatenate(got, 1), np.concatenate(ref, 1), torch.bfloat16,
            f"{what} ({len(ts)} rows x all heads)")


def prefill(cfg, cfg_id, W=None):
    W = cfg.W if W is None else W
    x = prefill_inputs(cfg, cfg_id, DEV)
    B, T, Hq, D = x.q_pre.shape
    Hkv = cfg.Hkv
    kc = torch.empty((B, Hkv, T, D), dtype=x.k.dtype, device=DEV)
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
    return x, o, ox


@pytest.mark.parametrize("name", ["prefill_32k", "sft_dual_8k", "prefill_128k"])
def test_prefill_configuration_sampled(name):
    cfg, cfg_id = workload(name)
    say(f"[full size] {cfg.name}")
    x, o, ox = prefill(cfg, cfg_id)
    k_host, v_host = f64(x.k), f64(x.v)
    ts = sample_rows(cfg.T, cfg.W, 24, cfg_id)
    check_rows(o, x.q_pre, x.alpha, x.beta, k_host, v_host, ts, cfg.W,
               "base stream")
    # output stream: every row if few, else a sample
    T_in = cfg.T_in
    rs = (list(range(cfg.T_out)) if cfg.T_out <= 4 else
          sample_rows(cfg.T_out, 64, 24, cfg_id + 100))
    got, ref = [], []
    for r in rs:
        t = T_in + r
        rr, _ = oracle.xattn(f64(x.qx_pre[:, r:r + 1]), f64(x.alpha_x),
                             f64(x.beta_x), k_host[:, :t + 1], v_host[:, :t + 1], t)
        ref.append(rr)
        got.append(f64(ox[:, r:r + 1]))
    compare(np.concatenate(got, 1), np.concatenate(ref, 1), torch.bfloat16,
            f"output stream ({len(rs)} rows x all heads)")


def test_long_prefill_full_causal_sampled():
    """The same-T full causal run used for the speedup ratio (W = T)."""
    cfg, cfg_id = workload("prefill_128k")
    say("[full size] prefill_128k full causal")
    x, o, _ = prefill(cfg, cfg_id, W=cfg.T)
    k_host, v_host = f64(x.k), f64(x.v)
    ts = [0, 1, 4095, 4096, 65535, cfg.T - 1]
    check_rows(o, x.q_pre, x.alpha, x.beta, k_host, v_host, ts, None,
               "causal")


def test_decode_pair_configuration_sampled():
    cfg, cfg_id = workload("decode_pair_b64")
    B, Hq, Hkv, D, L0, W = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.T, cfg.W
    steps = cfg.decode_steps
    say(f"[full size] {cfg.name}: {steps} steps")
    k0, v0 = kv_inputs(cfg, cfg_id, DEV)          # the 32768 cached tokens
    st = decode_all_steps(cfg, cfg_id, device=DEV)
    cap = L0 + steps
    kc = torch.empty((B, Hkv, cap, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    cl = torch.zeros(B, dtype=torch.int32, device=DEV)
    lo.orthros_kv_append(kc, vc, cl, k0, v0)
    del k0, v0
    a, b, ax, bx = affine_inputs(cfg, cfg_id, DEV)
    keep = {0, 1, 127, 255}
    outs = {}
    ws = lo.workspace(lo.orthros_workspace_bytes(lo.ORTHROS_OP_DECODE_PAIR, B,
                                                 Hq, Hkv, D, 1, cap), DEV)
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    ox = torch.empty_like(o)
    for s in range(steps):
        lo.orthros_decode_pair(st.q_pre[s], st.qx_pre[s], a, b, ax, bx,
                               st.k_new[s], st.v_new[s], kc, vc, cl, o, ox,
                               max_len_after=L0 + s + 1, W=W, ws=ws)
        if s in keep:
            outs[s] = (o.clone(), ox.clone())
    torch.cuda.synchronize()
    assert cl.tolist() == [L0 + steps] * B, "cache lengths"
    lo.orthros_check_device_errors()
    bs = [0, 17, 42, 63]
    for bi in bs:
        kb = f64(kc[bi].permute(1, 0, 2))[None]     # [1, cap, Hkv, D]
        vb = f64(vc[bi].permute(1, 0, 2))[None]
        for s in sorted(keep):
            n = L0 + s                               # index of the new key
            lo_t = max(0, n - W + 1)
            rb, _ = oracle.xattn(f64(st.q_pre[s][bi:bi + 1, None]), f64(a),
                                 f64(b), kb[:, lo_t:n + 1], vb[:, lo_t:n + 1],
                                 n - lo_t)
            rx, _ = oracle.xattn(f64(st.qx_pre[s][bi:bi + 1, None]), f64(ax),
                                 f64(bx), kb[:, :n + 1], vb[:, :n + 1], n)
            compare(outs[s][0][bi:bi + 1, None], rb, torch.bfloat16,
                    f"b={bi} step {s} base")
            compare(outs[s][1][bi:bi + 1, None], rx, torch.bfloat16,
                    f"b={bi} step {s} output")
        # appended rows are the step tokens, bit for bit
        assert torch.equal(kc[bi, :, L0:].permute(1, 0, 2).float(),
                           st.k_new[:, bi].float())


def test_long_prefill_trained_window_sampled():
    """The 128K prefill at the window the paper trains with (W = 128), which
    runs the rolling-window kernel."""
    cfg, cfg_id = workload("prefill_128k")
    say("[full size] prefill_128k W=128")
    x, o, _ = prefill(cfg, cfg_id, W=128)
    k_host, v_host = f64(x.k), f64(x.v)
    ts = sample_rows(cfg.T, 128, 24, cfg_id + 7)
    check_rows(o, x.q_pre, x.alpha, x.beta, k_host, v_host, ts, 128,
               "base stream W=128")


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
    dt = torch.bfloat16
    say(f"[full size] largest cache: T={T} Hq={Hq} Hkv={Hkv}")
    from workloads import normal
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
