"""GPU parity of the training backward (both streams) against the fp64
oracle's attn_backward, through the C ABI.

Inputs are seeded N(0, 1) draws rounded to bf16; the forward outputs o, o'
come from the library's own forward calls (the backward takes them as
inputs, as a training step would), and the oracle gets the exact bf16 bits
of every input. Tolerances: the bf16 gate (max-abs 2e-2, rel-L2 1e-2) is
stated for unit-scale values; gradients are not unit-scale (dK, dV and the
scale-offset gradients are sums over many rows, and a bf16 result of
magnitude 4 is itself only good to 2^-7), so every gradient's max-abs gate
is 2e-2 times max(1, its largest reference magnitude), with rel-L2 1e-2
unchanged."""
import numpy as np
import pytest
import torch

import long_context_prefill_swa_amd as lo
import oracle
from gpu_util import TOL, compare, f64, make_cache, say
from workloads import normal

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


def case(B, T, T_out, Hq, Hkv, W, seed, head_map=None):
    D = 128
    q = normal((B, T, Hq, D), seed, BF, DEV)
    qx = normal((B, T_out, Hq, D), seed + 1, BF, DEV) if T_out else None
    k = normal((B, T, Hkv, D), seed + 2, BF, DEV)
    v = normal((B, T, Hkv, D), seed + 3, BF, DEV)
    a = 1.0 + 0.1 * normal((Hq * D,), seed + 4, torch.float32, DEV)
    b = 0.1 * normal((Hq * D,), seed + 5, torch.float32, DEV)
    ax = 1.0 + 0.1 * normal((Hq * D,), seed + 6, torch.float32, DEV)
    bx = 0.1 * normal((Hq * D,), seed + 7, torch.float32, DEV)
    d_o = normal((B, T, Hq, D), seed + 8, BF, DEV)
    d_ox = normal((B, T_out, Hq, D), seed + 9, BF, DEV) if T_out else None
    kc, vc, _ = make_cache(k, v, T)
    o = torch.empty_like(q)
    lo.orthros_swa_prefill(q, a, b, kc, vc, o, W, head_map=head_map)
    ox = None
    if T_out:
        ox = torch.empty_like(qx)
        lo.orthros_global_xattn(qx, ax, bx, kc, vc, ox, T - T_out,
                                head_map=head_map)
    g = lo.orthros_attn_backward(q, qx, a, b, ax, bx, kc, vc, o, ox, d_o,
                                 d_ox, W, head_map=head_map)
    torch.cuda.synchronize()
    D_ = D
    z = lambda t, shape: f64(t) if t is not None else np.zeros(shape)  # noqa
    ref = oracle.attn_backward(
        f64(q), z(qx, (B, 0, Hq, D_)), f64(a), f64(b), f64(ax), f64(bx),
        f64(k), f64(v), f64(d_o), z(d_ox, (B, 0, Hq, D_)), W,
        head_map=head_map)
    return g, ref, T_out


def check(g, ref, T_out):
    names = ("dq_pre", "dk", "dv", "d_alpha", "d_beta")
    if T_out:
        names += ("dqx_pre", "d_alpha_x", "d_beta_x")
    for name in names:
        scale = max(1.0, float(np.abs(ref[name]).max()))
        compare(g[name], ref[name], BF, f"{name} (largest {scale:.2f})",
                tol=(TOL[BF][0] * scale, TOL[BF][1]))
    if not T_out:
        assert (f64(g["d_alpha_x"]) == 0).all() and (f64(g["d_beta_x"]) == 0).all()


@pytest.mark.parametrize("B,T,T_out,Hq,Hkv,W", [
    (2, 300, 3, 8, 2, 64),      # SFT-like, 4 query heads per KV head
    (1, 257, 257, 4, 4, 100),   # pre-training: every position an output row
    (1, 200, 0, 8, 1, 17),      # base stream only, 8 query heads per KV head
    (1, 130, 5, 4, 2, 1000),    # window above T
    (2, 97, 9, 4, 2, 1),        # window of one
    (1, 700, 40, 8, 4, 129),    # several key tiles per row block
])
def test_backward_parity(B, T, T_out, Hq, Hkv, W):
    say(f"[backward] B={B} T={T} T_out={T_out} Hq={Hq} Hkv={Hkv} W={W}")
    check(*case(B, T, T_out, Hq, Hkv, W, 500 + T))


def test_backward_custom_head_map():
    hm = [2, 0, 1, 1, 0, 2]
    say(f"[backward head map] {hm}")
    check(*case(1, 150, 6, 6, 3, 33, 610, head_map=hm))


def test_backward_xcd_block_order():
    """(batch, KV head) pairs a multiple of 8, so every pair's workgroups
    run on one XCD (the block renumbering the kernels use then): B = 2,
    4 KV heads, every gradient compared in full."""
    say("[backward] B=2 Hq=16 Hkv=4 (8 pairs)")
    check(*case(2, 300, 20, 16, 4, 64, 630))


def _bitwise(t):
    return t.view(torch.int16) if t.dtype == BF else t.view(torch.int32)


@pytest.mark.parametrize("shape", [(1, 333, 7, 8, 2, 50, 620),
                                   (2, 300, 20, 16, 4, 64, 640)])
def test_backward_deterministic(shape):
    a1, _, _ = case(*shape)
    a2, _, _ = case(*shape)
    for name in a1:
        if a1[name] is not None:
            assert torch.equal(_bitwise(a1[name]), _bitwise(a2[name])), name


@pytest.fixture(scope="module")
def sft_backward():
    """The SFT dual-stream shape the benchmark times (B=4, T=8192,
    T_out=2048, W=1024, 32/8 heads): forward outputs from the library,
    seeded upstream gradients, one backward call."""
    from workloads import prefill_inputs, workload
    c, cid = workload("sft_dual_8k")
    say(f"[backward full size] {c.name}: GPU run")
    x = prefill_inputs(c, cid, DEV)
    kc, vc, _ = make_cache(x.k, x.v, c.T)
    o = torch.empty_like(x.q_pre)
    ox = torch.empty_like(x.qx_pre)
    lo.orthros_swa_prefill(x.q_pre, x.alpha, x.beta, kc, vc, o, c.W)
    lo.orthros_global_xattn(x.qx_pre, x.alpha_x, x.beta_x, kc, vc, ox, c.T_in)
    d_o = normal(tuple(o.shape), 9001, BF, DEV)
    d_ox = normal(tuple(ox.shape), 9002, BF, DEV)
    g = lo.orthros_attn_backward(x.q_pre, x.qx_pre, x.alpha, x.beta,
                                 x.alpha_x, x.beta_x, kc, vc, o, ox, d_o,
                                 d_ox, c.W)
    torch.cuda.synchronize()
    args = [f64(t) for t in (x.q_pre, x.qx_pre, x.alpha, x.beta, x.alpha_x,
                             x.beta_x, x.k, x.v, d_o, d_ox)]
    host = {k: (f64(v) if v is not None else None) for k, v in g.items()}
    return c, args, host


def test_backward_sft_shape_sampled(sft_backward):
    """dq_pre on sampled base rows and dqx_pre on sampled output rows (all
    heads), dK and dV on sampled keys of three KV heads, for the first and
    last batch entries."""
    c, args, g = sft_backward
    rng = np.random.default_rng(77)
    rows = sorted({0, 1, c.W - 1, c.W, c.T_in - 1, c.T_in, c.T - 1,
                   *map(int, rng.integers(0, c.T, 6))})
    out_rows = sorted({0, 1, c.T_out - 1, *map(int, rng.integers(0, c.T_out, 3))})
    keys = [0, 1000, c.T_in, c.T - 1]
    for b in (0, c.B - 1):
        for kvh in (0, 3, 7):
            dq, dqx, dk, dv = oracle.attn_backward_sampled(
                *args, c.W, b, rows if kvh == 0 else [],
                out_rows if kvh == 0 else [], keys, kvh)
            checks = [("dk", g["dk"][b, keys, kvh], dk),
                      ("dv", g["dv"][b, keys, kvh], dv)]
            if kvh == 0:
                checks += [("dq_pre", g["dq_pre"][b, rows], dq),
                           ("dqx_pre", g["dqx_pre"][b, out_rows], dqx)]
            for name, got, ref in checks:
                scale = max(1.0, float(np.abs(ref).max()))
                compare(got, ref, BF,
                        f"b={b} kv head {kvh} {name} (largest {scale:.2f})",
                        tol=(TOL[BF][0] * scale, TOL[BF][1]))


@pytest.mark.parametrize("heads", [(0, 13), (22, 31)])
def test_backward_sft_shape_scale_offset_gradients(sft_backward, heads):
    """d_alpha, d_beta, d_alpha_x and d_beta_x of two query heads at the
    SFT shape: each is a sum over all 4 x 8192 base rows (or 4 x 2048
    output rows) of that head, so the oracle evaluates every row of those
    heads (their entries are independent of the other heads)."""
    c, args, g = sft_backward
    Hq, D = c.Hq, c.D
    say(f"[backward full size] scale-offset gradients of heads {heads}")
    ref = oracle.attn_backward(*args, c.W, heads=list(heads), with_kv=False)
    for name in ("d_alpha", "d_beta", "d_alpha_x", "d_beta_x"):
        got = g[name].reshape(Hq, D)[list(heads)]
        want = ref[name].reshape(Hq, D)[list(heads)]
        scale = max(1.0, float(np.abs(want).max()))
        compare(got, want, BF, f"{name} heads {heads} (largest {scale:.2f})",
                tol=(TOL[BF][0] * scale, TOL[BF][1]))
