"""GPU parity of the HIP path against the fp64 oracle (small and medium
sizes that span several tiles and a ragged tail), plus exact probes.

Every call goes through the C ABI (ctypes binding). Inputs are seeded; the
oracle receives the exact bf16/fp32 bits the GPU reads.
"""
import numpy as np
import pytest
import torch

import long_context_prefill_swa_amd as lo
import oracle
from gpu_util import TOL, compare, f64, make_cache, say
from workloads import normal, prefill_inputs, workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def rand(shape, seed, dtype):
    return normal(shape, seed, dtype, DEV)


def affine_pair(n, seed):
    a = 1.0 + 0.1 * normal((n,), seed, torch.float32, DEV)
    b = 0.1 * normal((n,), seed + 1, torch.float32, DEV)
    return a, b


def run_swa(q, a, b, k, v, W, cap=None, head_map=None, fill=0.0):
    B, T, Hq, D = q.shape
    kc, vc, _ = make_cache(k, v, cap or T, fill)
    o = torch.empty_like(q)
    lo.orthros_swa_prefill(q, a, b, kc, vc, o, W, head_map=head_map)
    torch.cuda.synchronize()
    return o


def oracle_swa(q, a, b, k, v, W, head_map=None, rows=None):
    return oracle.swa(f64(q), f64(a), f64(b), f64(k), f64(v), W,
                      head_map=head_map, rows=rows)[0]


# --- tiny fp32 configuration (and its identity run) ------------------------

@pytest.mark.parametrize("W,identity", [(16, False), (64, True)])
def test_tiny_fp32_configuration(W, identity):
    tiny, tiny_id = workload("tiny_f32")
    cfg = tiny.with_(W=W, identity_affine=identity)
    say(f"[tiny fp32] W={W} identity={identity}")
    x = prefill_inputs(cfg, tiny_id, DEV)
    o = run_swa(x.q_pre, x.alpha, x.beta, x.k, x.v, W)
    ref = oracle_swa(x.q_pre, x.alpha, x.beta, x.k, x.v, W)
    compare(o, ref, torch.float32, "swa")
    kc, vc, _ = make_cache(x.k, x.v, cfg.T)
    ox = torch.empty_like(x.qx_pre)
    lo.orthros_global_xattn(x.qx_pre, x.alpha_x, x.beta_x, kc, vc, ox, cfg.T_in)
    torch.cuda.synchronize()
    ref_x = oracle.xattn(f64(x.qx_pre), f64(x.alpha_x), f64(x.beta_x),
                         f64(x.k), f64(x.v), cfg.T_in)[0]
    compare(ox, ref_x, torch.float32, "global")


# --- cache materialisation ---------------------------------------------------

@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 16),
                                     (torch.bfloat16, 6)])
def test_kv_append_is_a_bit_exact_copy(dtype, D):
    B, Hkv, cap = 3, 2, 50
    say(f"[kv_append] {dtype} D={D}")
    k1, v1 = rand((B, 20, Hkv, D), 1, dtype), rand((B, 20, Hkv, D), 2, dtype)
    k2, v2 = rand((B, 7, Hkv, D), 3, dtype), rand((B, 7, Hkv, D), 4, dtype)
    kc, vc, cl = make_cache(k1, v1, cap, fill=float("nan"))
    lo.orthros_kv_append(kc, vc, cl, k2, v2)
    torch.cuda.synchronize()
    assert cl.tolist() == [27] * B
    want_k = torch.cat([k1, k2], 1).permute(0, 2, 1, 3)
    want_v = torch.cat([v1, v2], 1).permute(0, 2, 1, 3)
    assert torch.equal(kc[:, :, :27].float(), want_k.float())
    assert torch.equal(vc[:, :, :27].float(), want_v.float())
    assert torch.isnan(kc[:, :, 27:].float()).all()


def test_kv_append_capacity_fault_sets_flag():
    B, Hkv, D, cap = 2, 2, 128, 10
    k, v = rand((B, 8, Hkv, D), 5, torch.bfloat16), rand((B, 8, Hkv, D), 6, torch.bfloat16)
    kc, vc, cl = make_cache(k, v, cap)
    lo.orthros_check_device_errors()
    k3, v3 = k[:, :3].contiguous(), v[:, :3].contiguous()
    lo.orthros_kv_append(kc, vc, cl, k3, v3)       # 8 + 3 > 10: skipped
    with pytest.raises(lo.OrthrosError) as e:
        lo.orthros_check_device_errors()
    assert e.value.code == -3
    assert cl.tolist() == [8, 8]
    lo.orthros_check_device_errors()               # flag was cleared


# --- base stream: banded MFMA kernel ----------------------------------------

@pytest.mark.parametrize("B,T,Hq,Hkv,W", [
    (2, 300, 8, 2, 1),      # window of one: o_t = v_t
    (2, 300, 8, 2, 17),
    (1, 333, 8, 2, 64),     # window = tile
    (1, 500, 4, 4, 100),    # no GQA (one query head per group)
    (1, 257, 16, 2, 1000),  # 8 query heads per KV head; W > T
    (2, 130, 8, 2, 65),
    (1, 1031, 8, 1, 256),   # all heads on one KV head, two groups
])
def test_swa_bf16_parity(B, T, Hq, Hkv, W):
    D = 128
    say(f"[swa bf16] B={B} T={T} Hq={Hq} Hkv={Hkv} W={W}")
    dt = torch.bfloat16
    q, k, v = rand((B, T, Hq, D), 10, dt), rand((B, T, Hkv, D), 11, dt), rand((B, T, Hkv, D), 12, dt)
    a, b = affine_pair(Hq * D, 13)
    o = run_swa(q, a, b, k, v, W)
    compare(o, oracle_swa(q, a, b, k, v, W), dt, "swa")


# --- base stream: rolling-window kernel (4 query heads per KV head,
# W <= 129) --------------------------------------------------------------------

@pytest.mark.parametrize("B,T,Hq,Hkv,W", [
    (2, 1000, 8, 2, 128),   # the trained window, ragged tail
    (3, 777, 8, 2, 66),     # smallest three-tile window
    (1, 576, 8, 2, 129),    # largest; T a multiple of the tile
    (1, 513, 32, 8, 100),   # eight groups, one row past a tile
    (2, 63, 8, 2, 128),     # a single partial tile
    (1, 333, 8, 2, 2),      # one to five 32-key sub-blocks per row block
    (1, 333, 8, 2, 32),
    (1, 333, 8, 2, 33),
    (1, 333, 8, 2, 64),
    (1, 333, 8, 2, 96),
    (1, 333, 8, 2, 97),
    (1, 333, 8, 2, 98),
])
def test_swa_rolling_parity(B, T, Hq, Hkv, W):
    D = 128
    say(f"[swa rolling] B={B} T={T} Hq={Hq} Hkv={Hkv} W={W}")
    dt = torch.bfloat16
    q, k, v = rand((B, T, Hq, D), 14, dt), rand((B, T, Hkv, D), 15, dt), rand((B, T, Hkv, D), 16, dt)
    a, b = affine_pair(Hq * D, 17)
    o = run_swa(q, a, b, k, v, W)
    compare(o, oracle_swa(q, a, b, k, v, W), dt, "swa")


def test_swa_rolling_long_segments_sampled():
    """One group, so each workgroup walks several query tiles through the
    ring; rows at every segment and tile boundary plus random ones."""
    B, T, Hq, Hkv, D, W = 1, 40000, 4, 1, 128, 128
    say(f"[swa rolling long] T={T} W={W}")
    dt = torch.bfloat16
    q, k, v = rand((B, T, Hq, D), 18, dt), rand((B, T, Hkv, D), 19, dt), rand((B, T, Hkv, D), 20, dt)
    a, b = affine_pair(Hq * D, 21)
    o = run_swa(q, a, b, k, v, W)
    ts = set()
    for e in range(0, T, 64):
        ts.update((e - 1, e, e + 1))
    ts.update(int(x) for x in np.random.default_rng(22).integers(0, T, 500))
    ts = sorted(t for t in ts if 0 <= t < T)
    rows = np.array([(0, t) for t in ts], np.int64)
    ref = oracle_swa(q, a, b, k, v, W, rows=rows)
    compare(o[0, ts], ref, dt, f"swa ({len(ts)} rows)")


def test_swa_rolling_padded_group():
    """A head map whose groups hold 3 and 2 query heads (padded to 4)."""
    hmap = [0, 1, 0, 1, 0]
    B, T, D, Hkv, W = 2, 300, 128, 2, 128
    Hq = len(hmap)
    say(f"[swa rolling head map] {hmap}")
    dt = torch.bfloat16
    q, k, v = rand((B, T, Hq, D), 24, dt), rand((B, T, Hkv, D), 25, dt), rand((B, T, Hkv, D), 26, dt)
    a, b = affine_pair(Hq * D, 27)
    o = run_swa(q, a, b, k, v, W, head_map=hmap)
    compare(o, oracle_swa(q, a, b, k, v, W, head_map=np.array(hmap, np.int32)),
            dt, "swa")


# --- base stream: persistent banded kernel (4 query heads per KV head,
# W > 129) ----------------------------------------------------------------------

@pytest.mark.parametrize("B,T,Hq,Hkv,W", [
    (2, 3000, 8, 2, 300),     # ragged tail, window not a tile multiple
    (1, 5000, 8, 2, 1000),
    (1, 4097, 32, 8, 513),    # eight groups, one row past a tile
    (1, 2048, 8, 2, 512),     # tile multiples
    (3, 700, 8, 2, 130),      # smallest window of this path
    (1, 1000, 8, 2, 1000),    # window = T (full causal)
    (2, 777, 8, 2, 5000),     # window above T
    (1, 2000, 8, 2, 1500),    # window above T / 4
])
def test_swa_persistent_parity(B, T, Hq, Hkv, W):
    D = 128
    say(f"[swa persistent] B={B} T={T} Hq={Hq} Hkv={Hkv} W={W}")
    dt = torch.bfloat16
    q, k, v = rand((B, T, Hq, D), 40, dt), rand((B, T, Hkv, D), 41, dt), rand((B, T, Hkv, D), 42, dt)
    a, b = affine_pair(Hq * D, 43)
    o = run_swa(q, a, b, k, v, W)
    compare(o, oracle_swa(q, a, b, k, v, W), dt, "swa")


def test_swa_persistent_many_heads_sampled():
    """More (batch, KV head) pairs than compute units: each workgroup walks
    every query tile of its pair. Rows at tile boundaries of the first,
    middle and last batch entries, plus random ones."""
    B, T, Hq, Hkv, D, W = 40, 600, 32, 8, 128, 150
    say(f"[swa persistent many heads] B={B} T={T} W={W}")
    dt = torch.bfloat16
    q, k, v = rand((B, T, Hq, D), 48, dt), rand((B, T, Hkv, D), 49, dt), rand((B, T, Hkv, D), 50, dt)
    a, b = affine_pair(Hq * D, 51)
    o = run_swa(q, a, b, k, v, W)
    rows = set()
    for bb in (0, B // 2, B - 1):
        for e in range(0, T, 64):
            rows.update((bb, t) for t in (e - 1, e, e + 63) if 0 <= t < T)
    rng = np.random.default_rng(52)
    rows.update((int(x), int(y)) for x, y in zip(rng.integers(0, B, 100), rng.integers(0, T, 100)))
    rows = np.array(sorted(rows), np.int64)
    ref = oracle_swa(q, a, b, k, v, W, rows=rows)
    got = torch.stack([o[bb, t] for bb, t in rows])
    compare(got, ref, dt, f"swa ({len(rows)} rows)")


def test_swa_persistent_padded_group():
    """A head map whose groups hold 3 and 2 query heads (padded to 4): the
    padded slots' rows are computed on clamped copies and never stored."""
    hmap = [0, 1, 0, 1, 0]
    B, T, D, Hkv, W = 2, 1500, 128, 2, 300
    Hq = len(hmap)
    say(f"[swa persistent head map] {hmap}")
    dt = torch.bfloat16
    q, k, v = rand((B, T, Hq, D), 44, dt), rand((B, T, Hkv, D), 45, dt), rand((B, T, Hkv, D), 46, dt)
    a, b = affine_pair(Hq * D, 47)
    o = run_swa(q, a, b, k, v, W, head_map=hmap)
    compare(o, oracle_swa(q, a, b, k, v, W, head_map=np.array(hmap, np.int32)),
            dt, "swa")


@pytest.mark.parametrize("T", [1, 2, 63, 65])
@pytest.mark.parametrize("Hq,Hkv,W", [
    (8, 2, 1),      # rolling kernel, window of one
    (8, 2, 100),    # rolling kernel
    (8, 2, 300),    # persistent kernel
    (16, 2, 300),   # banded kernel (8 query heads per KV head)
])
def test_swa_short_sequences(T, Hq, Hkv, W):
    """Sequences shorter than, equal to and one past a 64-row tile."""
    B, D = 2, 128
    say(f"[swa short] T={T} Hq={Hq} Hkv={Hkv} W={W}")
    dt = torch.bfloat16
    q, k, v = rand((B, T, Hq, D), 60, dt), rand((B, T, Hkv, D), 61, dt), rand((B, T, Hkv, D), 62, dt)
    a, b = affine_pair(Hq * D, 63)
    o = run_swa(q, a, b, k, v, W)
    compare(o, oracle_swa(q, a, b, k, v, W), dt, "swa")


def test_global_single_row_at_position_zero():
    """T_in = 0, T_out = 1: the one output row sees only key 0."""
    B, Hq, Hkv, D = 2, 8, 2, 128
    dt = torch.bfloat16
    say("[global single row]")
    qx = rand((B, 1, Hq, D), 64, dt)
    k, v = rand((B, 1, Hkv, D), 65, dt), rand((B, 1, Hkv, D), 66, dt)
    a, b = affine_pair(Hq * D, 67)
    kc, vc, _ = make_cache(k, v, 40, fill=float("nan"))
    ox = torch.empty_like(qx)
    lo.orthros_global_xattn(qx, a, b, kc, vc, ox, 0)
    torch.cuda.synchronize()
    ref = oracle.xattn(f64(qx), f64(a), f64(b), f64(k), f64(v), 0)[0]
    compare(ox, ref, dt, "global")


@pytest.mark.parametrize("hmap", [[2, 0, 1, 1, 0, 2], [0, 0, 0, 1, 2, 2]])
def test_swa_custom_head_map(hmap):
    B, T, D, Hkv = 2, 200, 128, 3
    Hq = len(hmap)
    say(f"[swa head map] {hmap}")
    dt = torch.bfloat16
    q, k, v = rand((B, T, Hq, D), 20, dt), rand((B, T, Hkv, D), 21, dt), rand((B, T, Hkv, D), 22, dt)
    a, b = affine_pair(Hq * D, 23)
    o = run_swa(q, a, b, k, v, 40, head_map=hmap)
    compare(o, oracle_swa(q, a, b, k, v, 40, head_map=np.array(hmap, np.int32)),
            dt, "swa")


def test_swa_generic_path_fp32_and_other_head_dims():
    for dt, D, W in [(torch.float32, 64, 33), (torch.bfloat16, 64, 20),
                     (torch.float32, 128, 100)]:
        say(f"[swa generic] {dt} D={D} W={W}")
        q, k, v = rand((2, 150, 4, D), 30, dt), rand((2, 150, 2, D), 31, dt), rand((2, 150, 2, D), 32, dt)
        a, b = affine_pair(4 * D, 33)
        o = run_swa(q, a, b, k, v, W)
        compare(o, oracle_swa(q, a, b, k, v, W), dt, "swa")


# --- output stream -----------------------------------------------------------

@pytest.mark.parametrize("B,T_in,T_out,Hq,Hkv,dt", [
    (2, 999, 1, 8, 2, torch.bfloat16),      # split-KV, prefilling
    (1, 3000, 4, 8, 2, torch.bfloat16),     # split-KV, 16 rows
    (3, 100, 2, 4, 4, torch.bfloat16),
    (2, 400, 100, 8, 2, torch.bfloat16),    # persistent kernel, every key
    (1, 0, 150, 8, 2, torch.bfloat16),      # pre-training setting T_in = 0
    (1, 777, 333, 8, 2, torch.bfloat16),    # ragged T_in and T_out
    (2, 64, 1000, 32, 8, torch.bfloat16),   # eight groups, T_out > T_in
    (1, 200, 64, 16, 2, torch.bfloat16),    # 8 query heads per KV head: banded kernel
    (2, 300, 5, 4, 2, torch.float32),       # generic kernel
])
def test_global_xattn_parity(B, T_in, T_out, Hq, Hkv, dt):
    D = 128
    T = T_in + T_out
    say(f"[global] B={B} T_in={T_in} T_out={T_out} Hq={Hq} Hkv={Hkv} {dt}")
    qx = rand((B, T_out, Hq, D), 40, dt)
    k, v = rand((B, T, Hkv, D), 41, dt), rand((B, T, Hkv, D), 42, dt)
    a, b = affine_pair(Hq * D, 43)
    kc, vc, _ = make_cache(k, v, T + 37, fill=float("nan"))
    ox = torch.empty_like(qx)
    lo.orthros_global_xattn(qx, a, b, kc, vc, ox, T_in)
    torch.cuda.synchronize()
    ref = oracle.xattn(f64(qx), f64(a), f64(b), f64(k), f64(v), T_in)[0]
    compare(ox, ref, dt, "global")


# --- decode pair ---------------------------------------------------------------

def _decode_run(B, Hq, Hkv, D, T0, steps, W, dt, seed=50):
    q = rand((steps, B, Hq, D), seed, dt)
    qx = rand((steps, B, Hq, D), seed + 1, dt)
    kn = rand((steps, B, Hkv, D), seed + 2, dt)
    vn = rand((steps, B, Hkv, D), seed + 3, dt)
    k0, v0 = rand((B, T0, Hkv, D), seed + 4, dt), rand((B, T0, Hkv, D), seed + 5, dt)
    a, b = affine_pair(Hq * D, seed + 6)
    ax, bx = affine_pair(Hq * D, seed + 8)
    cap = T0 + steps + 5
    kc, vc, cl = make_cache(k0, v0, cap, fill=float("nan"))
    outs = []
    for s in range(steps):
        o = torch.empty((B, Hq, D), dtype=dt, device=DEV)
        ox = torch.empty_like(o)
        lo.orthros_decode_pair(q[s], qx[s], a, b, ax, bx, kn[s], vn[s], kc, vc,
                               cl, o, ox, max_len_after=T0 + s + 1, W=W)
        outs.append((o, ox))
    torch.cuda.synchronize()
    return dict(q=q, qx=qx, kn=kn, vn=vn, k0=k0, v0=v0, a=a, b=b, ax=ax,
                bx=bx, kc=kc, vc=vc, cl=cl, outs=outs)


@pytest.mark.parametrize("dt,D,W", [(torch.bfloat16, 128, 64),
                                    (torch.bfloat16, 128, 3000),
                                    (torch.float32, 16, 16)])
def test_decode_pair_matches_incremental_oracle(dt, D, W):
    B, Hq, Hkv, T0, steps = 3, 8, 2, 700, 12
    say(f"[decode] {dt} D={D} W={W}")
    r = _decode_run(B, Hq, Hkv, D, T0, steps, W, dt)
    assert r["cl"].tolist() == [T0 + steps] * B
    cache = oracle.Cache(B, Hkv, D, T0 + steps)
    cache.append(f64(r["k0"]), f64(r["v0"]))
    for s in range(steps):
        o_ref, ox_ref = cache.decode_pair(
            f64(r["q"][s]), f64(r["qx"][s]), f64(r["a"]), f64(r["b"]),
            f64(r["ax"]), f64(r["bx"]), f64(r["kn"][s]), f64(r["vn"][s]), W)
        compare(r["outs"][s][0], o_ref, dt, f"step {s} base")
        compare(r["outs"][s][1], ox_ref, dt, f"step {s} output")
    # appended rows are the new tokens, bit for bit
    appended = r["kc"][:, :, T0:T0 + steps].permute(2, 0, 1, 3)
    assert torch.equal(appended.float(), r["kn"].float())


def test_decode_incremental_equals_batched_fp32():
    """The reproduction note's consistency gate (1e-4) on the GPU: cached
    prefill + decode steps vs one batched prefill over the same tokens."""
    B, Hq, Hkv, D, T0, steps, W = 2, 4, 2, 16, 40, 24, 16
    dt = torch.float32
    r = _decode_run(B, Hq, Hkv, D, T0, steps, W, dt, seed=60)
    T = T0 + steps
    k = torch.cat([r["k0"], r["kn"].permute(1, 0, 2, 3)], 1).contiguous()
    v = torch.cat([r["v0"], r["vn"].permute(1, 0, 2, 3)], 1).contiguous()
    qb = torch.cat([rand((B, T0, Hq, D), 61, dt), r["q"].permute(1, 0, 2, 3)], 1).contiguous()
    o = run_swa(qb, r["a"], r["b"], k, v, W)
    kc, vc, _ = make_cache(k, v, T)
    ox = torch.empty((B, steps, Hq, D), dtype=dt, device=DEV)
    lo.orthros_global_xattn(r["qx"].permute(1, 0, 2, 3).contiguous(), r["ax"],
                            r["bx"], kc, vc, ox, T0)
    torch.cuda.synchronize()
    worst = 0.0
    for s in range(steps):
        worst = max(worst, (r["outs"][s][0] - o[:, T0 + s]).abs().max().item(),
                    (r["outs"][s][1] - ox[:, s]).abs().max().item())
    say(f"  incremental vs batched max-abs {worst:.3e}")
    assert worst <= 1e-4


def test_decode_ragged_lengths_and_capacity():
    dt, B, Hq, Hkv, D, W = torch.bfloat16, 3, 8, 2, 128, 50
    lens = [100, 257, 31]
    cap = 300
    say("[decode ragged]")
    k0 = rand((B, 257, Hkv, D), 70, dt)
    v0 = rand((B, 257, Hkv, D), 71, dt)
    kc, vc, cl = make_cache(k0, v0, cap, fill=float("nan"))
    cl.copy_(torch.tensor(lens, dtype=torch.int32))
    # poison everything past each entry's length
    for bi, n in enumerate(lens):
        kc[bi, :, n:] = float("nan")
        vc[bi, :, n:] = float("nan")
    q, qx = rand((B, Hq, D), 72, dt), rand((B, Hq, D), 73, dt)
    kn, vn = rand((B, Hkv, D), 74, dt), rand((B, Hkv, D), 75, dt)
    a, b = affine_pair(Hq * D, 76)
    o, ox = torch.empty_like(q), torch.empty_like(q)
    lo.orthros_decode_pair(q, qx, a, b, a, b, kn, vn, kc, vc, cl, o, ox,
                           max_len_after=258, W=W)
    torch.cuda.synchronize()
    assert cl.tolist() == [n + 1 for n in lens]
    for bi, n in enumerate(lens):
        c = oracle.Cache(1, Hkv, D, n + 1)
        c.append(f64(k0[bi:bi + 1, :n]), f64(v0[bi:bi + 1, :n]))
        o_r, ox_r = c.decode_pair(f64(q[bi:bi + 1]), f64(qx[bi:bi + 1]), f64(a),
                                  f64(b), f64(a), f64(b), f64(kn[bi:bi + 1]),
                                  f64(vn[bi:bi + 1]), W)
        compare(o[bi:bi + 1], o_r, dt, f"b={bi} base")
        compare(ox[bi:bi + 1], ox_r, dt, f"b={bi} output")
    # an entry already at the bound is skipped and flagged
    lo.orthros_check_device_errors()
    cl.copy_(torch.tensor([258, 10, 10], dtype=torch.int32))
    lo.orthros_decode_pair(q, qx, a, b, a, b, kn, vn, kc, vc, cl, o, ox,
                           max_len_after=258, W=W)
    with pytest.raises(lo.OrthrosError):
        lo.orthros_check_device_errors()
    assert cl.tolist() == [258, 11, 11]
    assert (o[0].float() == 0).all()


# --- exact probes -------------------------------------------------------------

@pytest.mark.parametrize("T,W", [(1000, 16), (700, 64), (333, 100)])
def test_spike_probe_exact_index_ranges(T, W):
    """alpha = 0, beta = s e_0 (every query is s e_0); K = 0 except spike
    keys s' e_0 (score ~20), V = 0 except v_spike = e_c. A spike is in a
    row's range iff o[c] > 0.25; otherwise o[c] is exactly 0. Spikes are more
    than W apart, so a window holds at most one."""
    B, Hq, Hkv, D = 1, 8, 2, 128
    dt = torch.bfloat16
    say(f"[spike] T={T} W={W}")
    for off in (0, 7, W - 1):
        spikes = list(range(off, T, W + 3))[:126]
        k = torch.zeros((B, T, Hkv, D), dtype=dt, device=DEV)
        v = torch.zeros_like(k)
        chan = {}
        for i, j in enumerate(spikes):
            k[0, j, :, 0] = 20.0 * (D ** 0.5) / 4.0
            chan[j] = 1 + i
            v[0, j, :, 1 + i] = 1.0
        q = rand((B, T, Hq, D), 80, dt)
        a = torch.zeros(Hq * D, device=DEV)
        b = torch.zeros(Hq * D, device=DEV)
        b.view(Hq, D)[:, 0] = 4.0
        o = f64(run_swa(q, a, b, k, v, W))
        t = np.arange(T)[:, None]
        js = np.array(spikes)[None, :]
        inside = (js <= t) & (js >= t - W + 1)
        cols = o[0][:, :, [chan[j] for j in spikes]]      # [T, Hq, n_spikes]
        for h in range(Hq):
            got = cols[:, h, :]
            assert np.array_equal(got > 0.25, inside), f"off={off} head {h}"
            assert (got[~inside] == 0).all()
        # the output stream sees every spike up to t with equal weight
        kc, vc, _ = make_cache(k, v, T)
        ox = torch.empty_like(q)
        lo.orthros_global_xattn(q, a, b, kc, vc, ox, 0)
        torch.cuda.synchronize()
        ox = f64(ox)[0][:, :, [chan[j] for j in spikes]]
        seen = js <= t
        cnt = np.maximum(seen.sum(1, keepdims=True), 1)
        for h in range(Hq):
            assert np.array_equal(ox[:, h, :] > 0.5 / cnt, seen)
            assert (ox[:, h, :][~seen] == 0).all()


def test_values_all_one_give_one():
    B, T, Hq, Hkv, D, W = 2, 400, 8, 2, 128, 77
    dt = torch.bfloat16
    q, k = rand((B, T, Hq, D), 90, dt), rand((B, T, Hkv, D), 91, dt)
    v = torch.ones_like(k)
    a, b = affine_pair(Hq * D, 92)
    o = run_swa(q, a, b, k, v, W)
    assert (o.float() == 1.0).all()


def test_deterministic_bitwise():
    B, T, Hq, Hkv, D, W = 1, 600, 8, 2, 128, 200
    dt = torch.bfloat16
    q, k, v = rand((B, T, Hq, D), 93, dt), rand((B, T, Hkv, D), 94, dt), rand((B, T, Hkv, D), 95, dt)
    a, b = affine_pair(Hq * D, 96)
    o1 = run_swa(q, a, b, k, v, W)
    o2 = run_swa(q, a, b, k, v, W)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    kc, vc, _ = make_cache(k, v, T)
    x1, x2 = torch.empty_like(q[:, :2]), torch.empty_like(q[:, :2])
    lo.orthros_global_xattn(q[:, -2:].contiguous(), a, b, kc, vc, x1, T - 2)
    lo.orthros_global_xattn(q[:, -2:].contiguous(), a, b, kc, vc, x2, T - 2)
    torch.cuda.synchronize()
    assert torch.equal(x1.view(torch.int16), x2.view(torch.int16))


def test_tolerances_are_the_stated_ones():
    assert TOL[torch.float32][0] == 1e-4 and TOL[torch.bfloat16][0] == 2e-2
