"""Exact probes of the window kernels and the head grouping on the GPU.

* Reads past the cache length: every row of the cache past T holds NaN. A
  kernel that loaded any of them into a product would return NaN (a masked
  score gives a zero weight, and 0 x NaN is NaN), so a finite, correct output
  shows that no key past T was read. The pages' ranges end at the row's own
  position (paper text §3.1, the o_t and o'_t equations).
* GQA replication: grouped query heads reading Hkv K/V heads give the same
  attention as the same query heads each reading its own copy of its KV head
  (Hkv = Hq, identity map). The two runs take different kernels, so they are
  compared with the bf16 tolerance, and each against the oracle.
* Head and batch permutation: permuting query heads together with their
  scale-offset vectors and map entries, or permuting batch entries, permutes
  the outputs bit for bit (every head and sequence is computed on its own).
"""
import numpy as np
import pytest
import torch

import long_context_prefill_swa_amd as lo
import oracle
from gpu_util import compare, f64, make_cache, say
from workloads import normal

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


def rand(shape, seed, dtype=BF):
    return normal(shape, seed, dtype, DEV)


def affine_pair(n, seed):
    a = 1.0 + 0.1 * normal((n,), seed, torch.float32, DEV)
    b = 0.1 * normal((n,), seed + 1, torch.float32, DEV)
    return a, b


def swa(q, a, b, kc, vc, W, head_map=None):
    o = torch.empty_like(q)
    lo.orthros_swa_prefill(q, a, b, kc, vc, o, W, head_map=head_map)
    torch.cuda.synchronize()
    return o


# --- no key past the cache length is read (NaN-poisoned tail) ---------------

@pytest.mark.parametrize("Hq,Hkv,W,T,dt", [
    (8, 2, 128, 333, BF),     # rolling kernel (4 query heads per KV head)
    (8, 2, 1, 200, BF),       # rolling kernel, window of one
    (8, 2, 129, 64, BF),      # rolling kernel, one tile, W >= T
    (8, 2, 300, 1000, BF),    # persistent kernel
    (8, 2, 5000, 777, BF),    # persistent kernel, W >= T (full causal)
    (8, 2, 1000, 65, BF),     # persistent kernel, W >= T, two tiles
    (16, 2, 300, 1000, BF),   # banded kernel (8 query heads per KV head)
    (16, 2, 4000, 999, BF),   # banded kernel, W >= T
    (4, 4, 64, 257, BF),      # banded kernel, one query head per KV head
    (4, 2, 50, 300, torch.float32),   # generic row kernel
])
def test_window_kernels_never_read_past_the_cache_length(Hq, Hkv, W, T, dt):
    B, D, extra = 2, 128, 200
    say(f"[nan tail] Hq={Hq} Hkv={Hkv} W={W} T={T} {dt}")
    q, k, v = rand((B, T, Hq, D), 100, dt), rand((B, T, Hkv, D), 101, dt), \
        rand((B, T, Hkv, D), 102, dt)
    a, b = affine_pair(Hq * D, 103)
    kc, vc, cl = make_cache(k, v, T + extra, fill=float("nan"))
    assert cl.tolist() == [T] * B
    assert torch.isnan(kc[:, :, T:].float()).all()
    o = swa(q, a, b, kc, vc, W)
    ref, _ = oracle.swa(f64(q), f64(a), f64(b), f64(k), f64(v), W)
    compare(o, ref, dt, "swa with NaN past T")


def test_output_stream_never_reads_past_its_row():
    """The output rows at positions T_in .. T_in + T_out - 1 of a cache whose
    rows from T_in + T_out on are NaN (split-KV and persistent paths)."""
    B, Hq, Hkv, D = 2, 8, 2, 128
    for T_in, T_out in ((500, 1), (300, 4), (200, 300)):
        T = T_in + T_out
        say(f"[nan tail, output stream] T_in={T_in} T_out={T_out}")
        qx = rand((B, T_out, Hq, D), 110)
        k, v = rand((B, T, Hkv, D), 111), rand((B, T, Hkv, D), 112)
        a, b = affine_pair(Hq * D, 113)
        kc, vc, _ = make_cache(k, v, T + 300, fill=float("nan"))
        ox = torch.empty_like(qx)
        lo.orthros_global_xattn(qx, a, b, kc, vc, ox, T_in)
        torch.cuda.synchronize()
        ref, _ = oracle.xattn(f64(qx), f64(a), f64(b), f64(k), f64(v), T_in)
        compare(ox, ref, BF, "output stream with NaN past T")


# --- GQA: grouped heads == each query head with its own copy of its KV head -

@pytest.mark.parametrize("W,T", [(128, 700), (300, 1100), (5000, 600)])
def test_gqa_grouping_equals_replicated_kv_heads(W, T):
    B, Hq, Hkv, D = 1, 32, 8, 128
    G = Hq // Hkv
    say(f"[gqa replication] W={W} T={T}")
    q, k, v = rand((B, T, Hq, D), 120), rand((B, T, Hkv, D), 121), \
        rand((B, T, Hkv, D), 122)
    a, b = affine_pair(Hq * D, 123)
    kc, vc, _ = make_cache(k, v, T)
    o_grouped = swa(q, a, b, kc, vc, W)
    k_rep = k.repeat_interleave(G, dim=2).contiguous()
    v_rep = v.repeat_interleave(G, dim=2).contiguous()
    kr, vr, _ = make_cache(k_rep, v_rep, T)
    o_rep = swa(q, a, b, kr, vr, W)
    ref, _ = oracle.swa(f64(q), f64(a), f64(b), f64(k), f64(v), W)
    compare(o_grouped, ref, BF, "grouped vs oracle")
    compare(o_rep, ref, BF, "replicated vs oracle")
    compare(o_grouped, f64(o_rep), BF, "grouped vs replicated")
    # the output stream and the decode pair, the same way
    qx = rand((B, 2, Hq, D), 124)
    ox_g, ox_r = torch.empty_like(qx), torch.empty_like(qx)
    lo.orthros_global_xattn(qx, a, b, kc, vc, ox_g, T - 2)
    lo.orthros_global_xattn(qx, a, b, kr, vr, ox_r, T - 2)
    torch.cuda.synchronize()
    compare(ox_g, f64(ox_r), BF, "output stream grouped vs replicated")


# --- permutations --------------------------------------------------------------

def _perm_case(Hq, Hkv, W, T, seed, hmap=None):
    B, D = 3, 128
    q, k, v = rand((B, T, Hq, D), seed), rand((B, T, Hkv, D), seed + 1), \
        rand((B, T, Hkv, D), seed + 2)
    a, b = affine_pair(Hq * D, seed + 3)
    kc, vc, _ = make_cache(k, v, T)
    base_map = (list(hmap) if hmap is not None else
                [h // (Hq // Hkv) for h in range(Hq)])
    o = swa(q, a, b, kc, vc, W, head_map=base_map)
    perm = np.random.default_rng(seed).permutation(Hq)
    qp = q[:, :, perm].contiguous()
    ap = a.view(Hq, D)[perm].reshape(-1).contiguous()
    bp = b.view(Hq, D)[perm].reshape(-1).contiguous()
    mp = [base_map[h] for h in perm]
    op = swa(qp, ap, bp, kc, vc, W, head_map=mp)
    assert torch.equal(op.view(torch.int16),
                       o[:, :, perm].contiguous().view(torch.int16)), \
        "head permutation"
    bperm = [2, 0, 1]
    kb, vb, _ = make_cache(k[bperm].contiguous(), v[bperm].contiguous(), T)
    ob = swa(q[bperm].contiguous(), a, b, kb, vb, W, head_map=base_map)
    assert torch.equal(ob.view(torch.int16),
                       o[bperm].contiguous().view(torch.int16)), \
        "batch permutation"


@pytest.mark.parametrize("Hq,Hkv,W,T", [
    (8, 2, 100, 500),      # rolling kernel
    (8, 2, 400, 900),      # persistent kernel
    (16, 2, 200, 400),     # banded kernel
])
def test_head_and_batch_permutation_bitwise(Hq, Hkv, W, T):
    say(f"[permutation] Hq={Hq} Hkv={Hkv} W={W} T={T}")
    _perm_case(Hq, Hkv, W, T, 130 + W)


def test_permutation_with_uneven_map():
    say("[permutation] uneven map")
    _perm_case(6, 3, 150, 400, 140, hmap=[0, 0, 0, 1, 2, 2])


# --- uneven head maps through the split-KV calls (workspace from the map) ----

@pytest.mark.parametrize("hmap,Hkv", [([0, 0, 0, 1, 2, 2], 3),
                                      ([0, 1, 1, 0, 1], 2),
                                      ([1, 1, 1, 1, 1, 1, 1, 0], 2)])
def test_split_kv_calls_with_uneven_head_maps(hmap, Hkv):
    B, D, T0, W = 2, 128, 900, 100
    Hq = len(hmap)
    say(f"[uneven map, split-KV] {hmap}")
    hm = np.array(hmap, np.int32)
    qx = rand((B, 1, Hq, D), 150)
    k, v = rand((B, T0, Hkv, D), 151), rand((B, T0, Hkv, D), 152)
    a, b = affine_pair(Hq * D, 153)
    kc, vc, cl = make_cache(k, v, T0 + 10, fill=float("nan"))
    ox = torch.empty_like(qx)
    lo.orthros_global_xattn(qx, a, b, kc, vc, ox, T0 - 1, head_map=hmap)
    torch.cuda.synchronize()
    ref, _ = oracle.xattn(f64(qx), f64(a), f64(b), f64(k), f64(v), T0 - 1,
                          head_map=hm)
    compare(ox, ref, BF, "global, uneven map")
    q, qd = rand((B, Hq, D), 154), rand((B, Hq, D), 155)
    kn, vn = rand((B, Hkv, D), 156), rand((B, Hkv, D), 157)
    o, od = torch.empty_like(q), torch.empty_like(q)
    lo.orthros_decode_pair(q, qd, a, b, a, b, kn, vn, kc, vc, cl, o, od,
                           max_len_after=T0 + 1, W=W, head_map=hmap)
    torch.cuda.synchronize()
    assert cl.tolist() == [T0 + 1] * B
    c = oracle.Cache(B, Hkv, D, T0 + 1)
    c.append(f64(k), f64(v))
    o_r, od_r = c.decode_pair(f64(q), f64(qd), f64(a), f64(b), f64(a), f64(b),
                              f64(kn), f64(vn), W, head_map=hm)
    compare(o, o_r, BF, "decode base, uneven map")
    compare(od, od_r, BF, "decode output, uneven map")


# --- a caller's stream with the binding's own scratch ---------------------------

def test_side_stream_with_binding_scratch():
    """ws=None on a side stream: the binding's scratch stays reserved for
    that stream's work (record_stream), while the current stream allocates
    and writes new tensors right after the call."""
    B, Hq, Hkv, D, T0, W = 4, 32, 8, 128, 20000, 512
    say("[side stream]")
    q = rand((B, 1, Hq, D), 160)
    k, v = rand((B, T0, Hkv, D), 161), rand((B, T0, Hkv, D), 162)
    a, b = affine_pair(Hq * D, 163)
    kc, vc, cl = make_cache(k, v, T0 + 4)
    q0 = q[:, 0].contiguous()
    k0, v0 = k[:, 0].contiguous(), v[:, 0].contiguous()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ox = torch.empty_like(q)
    outs = []
    with torch.cuda.stream(side):
        for _ in range(3):
            lo.orthros_global_xattn(q, a, b, kc, vc, ox, T0 - 1, stream=side)
            o = torch.empty((B, Hq, D), dtype=BF, device=DEV)
            od = torch.empty_like(o)
            lo.orthros_decode_pair(q0, q0, a, b, a, b, k0, v0, kc, vc, cl,
                                   o, od, max_len_after=T0 + 4, W=W,
                                   stream=side)
            outs.append((ox.clone(), o, od))
    # scribble over freshly allocated memory on the default stream meanwhile
    junk = [torch.full((1 << 22,), float("nan"), device=DEV) for _ in range(8)]
    torch.cuda.synchronize()
    del junk
    assert cl.tolist() == [T0 + 3] * B
    ref, _ = oracle.xattn(f64(q), f64(a), f64(b), f64(k), f64(v), T0 - 1)
    for i, (gx, _o, _od) in enumerate(outs):
        compare(gx, ref, BF, f"global on the side stream, call {i}")
        assert torch.isfinite(_o.float()).all() and torch.isfinite(_od.float()).all()
