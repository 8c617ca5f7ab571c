"""Paged K/V cache on the GPU (variable-length batched decoding).

* orthros_kv_append_paged writes every new row into the page and row the
  block table names, bit for bit, and advances the per-sequence lengths.
* orthros_decode_pair_paged equals the fp64 oracle per sequence (ragged
  lengths, several page sizes, pool rows past each length poisoned with NaN)
  and equals the contiguous orthros_decode_pair bit for bit on the same
  inputs (same chunking, same arithmetic; only the addressing differs).
* An out-of-range block-table entry raises the device flag, is never
  dereferenced, and leaves the other sequences' results intact.
"""
import math

import pytest
import torch

import long_context_prefill_swa_amd as lo
import oracle
from gpu_util import compare, f64, say
from workloads import normal

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def rand(shape, seed, dt):
    return normal(shape, seed, dt, DEV)


def affine_pair(n, seed):
    return (1 + 0.1 * normal((n,), seed, torch.float32, DEV),
            0.1 * normal((n,), seed + 1, torch.float32, DEV))


def block_table(B, max_pages, n_pages, seed):
    """Distinct pages per sequence, drawn as a seeded permutation."""
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n_pages, generator=g)[:B * max_pages]
    return perm.reshape(B, max_pages).to(torch.int32).to(DEV)


def paged_pool(k, v, lens, page_size, bt, n_pages, fill=float("nan")):
    """Pool [n_pages, Hkv, page_size, D] holding rows [0, lens[b]) of k/v
    [B, T, Hkv, D] at the pages of bt; everything else is `fill`."""
    B, T, Hkv, D = k.shape
    kp = torch.full((n_pages, Hkv, page_size, D), fill, dtype=k.dtype, device=DEV)
    vp = torch.full_like(kp, fill)
    for b in range(B):
        for i in range(lens[b]):
            p = int(bt[b, i // page_size])
            kp[p, :, i % page_size] = k[b, i]
            vp[p, :, i % page_size] = v[b, i]
    return kp, vp


def gather_rows(pool, bt, b, i0, i1, page_size):
    """Rows [i0, i1) of sequence b from a pool, as [n, Hkv, D]."""
    return torch.stack([pool[int(bt[b, i // page_size]), :, i % page_size]
                        for i in range(i0, i1)])


@pytest.mark.parametrize("dt,D,page_size", [(torch.bfloat16, 128, 32),
                                            (torch.bfloat16, 64, 64),
                                            (torch.float32, 16, 256)])
def test_kv_append_paged_is_a_bit_exact_scatter(dt, D, page_size):
    B, Hkv, n = 3, 2, 100
    start = [0, 5, 70]
    max_pages = math.ceil((max(start) + n) / page_size)
    n_pages = B * max_pages + 2
    say(f"[paged append] {dt} D={D} page={page_size}")
    bt = block_table(B, max_pages, n_pages, 1)
    kp = torch.full((n_pages, Hkv, page_size, D), float("nan"), dtype=dt, device=DEV)
    vp = torch.full_like(kp, float("nan"))
    cl = torch.tensor(start, dtype=torch.int32, device=DEV)
    kn, vn = rand((B, n, Hkv, D), 2, dt), rand((B, n, Hkv, D), 3, dt)
    lo.orthros_kv_append_paged(kp, vp, bt, cl, kn, vn)
    torch.cuda.synchronize()
    lo.orthros_check_device_errors()
    assert cl.tolist() == [s + n for s in start]
    written = 0
    for b in range(B):
        got_k = gather_rows(kp, bt, b, start[b], start[b] + n, page_size)
        got_v = gather_rows(vp, bt, b, start[b], start[b] + n, page_size)
        assert torch.equal(got_k, kn[b]) and torch.equal(got_v, vn[b])
        written += n
    # nothing else was written: every other pool row is still NaN
    nan_rows = torch.isnan(kp.float()).all(-1).sum().item()
    assert nan_rows == n_pages * Hkv * page_size - written * Hkv


def run_decode_check(B, Hq, Hkv, lens, page_size, W, steps, seed):
    dt, D = torch.bfloat16, 128
    T0 = max(lens)
    max_len = T0 + steps
    max_pages = math.ceil(max_len / page_size)
    n_pages = B * max_pages + 3
    bt = block_table(B, max_pages, n_pages, seed)
    k0, v0 = rand((B, T0, Hkv, D), seed + 1, dt), rand((B, T0, Hkv, D), seed + 2, dt)
    kp, vp = paged_pool(k0, v0, lens, page_size, bt, n_pages)
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    a, b_ = affine_pair(Hq * D, seed + 3)
    ax, bx = affine_pair(Hq * D, seed + 5)
    caches = []
    for b in range(B):
        c = oracle.Cache(1, Hkv, D, max_len)
        c.append(f64(k0[b:b + 1, :lens[b]]), f64(v0[b:b + 1, :lens[b]]))
        caches.append(c)
    o = torch.empty((B, Hq, D), dtype=dt, device=DEV)
    ox = torch.empty_like(o)
    for s in range(steps):
        q, qx = rand((B, Hq, D), seed + 10 + 4 * s, dt), rand((B, Hq, D), seed + 11 + 4 * s, dt)
        kn, vn = rand((B, Hkv, D), seed + 12 + 4 * s, dt), rand((B, Hkv, D), seed + 13 + 4 * s, dt)
        lo.orthros_decode_pair_paged(q, qx, a, b_, ax, bx, kn, vn, kp, vp, bt,
                                     cl, o, ox, max_len_after=max(lens) + s + 1,
                                     W=W)
        torch.cuda.synchronize()
        for b in range(B):
            o_r, ox_r = caches[b].decode_pair(
                f64(q[b:b + 1]), f64(qx[b:b + 1]), f64(a), f64(b_), f64(ax),
                f64(bx), f64(kn[b:b + 1]), f64(vn[b:b + 1]), W)
            compare(o[b:b + 1], o_r, dt, f"step {s} b={b} (len {lens[b] + s}) base")
            compare(ox[b:b + 1], ox_r, dt, f"step {s} b={b} output")
            # the new row landed in its page
            got = gather_rows(kp, bt, b, lens[b] + s, lens[b] + s + 1, page_size)
            assert torch.equal(got[0], kn[b])
    lo.orthros_check_device_errors()
    assert cl.tolist() == [n + steps for n in lens]


@pytest.mark.parametrize("page_size,lens", [(32, [1, 63, 200, 700]),
                                            (64, [64, 65, 129, 1000]),
                                            (256, [3, 255, 256, 2100])])
def test_decode_pair_paged_matches_oracle_ragged(page_size, lens):
    say(f"[paged decode] page={page_size} lens={lens}")
    run_decode_check(B=4, Hq=8, Hkv=2, lens=lens, page_size=page_size, W=48,
                     steps=3, seed=100 + page_size)


def test_decode_pair_paged_custom_head_map():
    """Hq=6 over Hkv=3 with an uneven explicit map."""
    dt, B, Hq, Hkv, D, W, page_size = torch.bfloat16, 2, 6, 3, 128, 40, 64
    lens = [90, 300]
    hmap = [2, 0, 1, 1, 0, 2]
    say("[paged decode] custom head map")
    max_pages = math.ceil((max(lens) + 1) / page_size)
    n_pages = B * max_pages
    bt = block_table(B, max_pages, n_pages, 7)
    k0, v0 = rand((B, max(lens), Hkv, D), 8, dt), rand((B, max(lens), Hkv, D), 9, dt)
    kp, vp = paged_pool(k0, v0, lens, page_size, bt, n_pages)
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q, qx = rand((B, Hq, D), 10, dt), rand((B, Hq, D), 11, dt)
    kn, vn = rand((B, Hkv, D), 12, dt), rand((B, Hkv, D), 13, dt)
    a, b_ = affine_pair(Hq * D, 14)
    o, ox = torch.empty_like(q), torch.empty_like(q)
    lo.orthros_decode_pair_paged(q, qx, a, b_, a, b_, kn, vn, kp, vp, bt, cl,
                                 o, ox, max_len_after=max(lens) + 1, W=W,
                                 head_map=hmap)
    torch.cuda.synchronize()
    for b in range(B):
        c = oracle.Cache(1, Hkv, D, lens[b] + 1)
        c.append(f64(k0[b:b + 1, :lens[b]]), f64(v0[b:b + 1, :lens[b]]))
        o_r, ox_r = c.decode_pair(f64(q[b:b + 1]), f64(qx[b:b + 1]), f64(a),
                                  f64(b_), f64(a), f64(b_), f64(kn[b:b + 1]),
                                  f64(vn[b:b + 1]), W, head_map=hmap)
        compare(o[b:b + 1], o_r, dt, f"b={b} base")
        compare(ox[b:b + 1], ox_r, dt, f"b={b} output")


def test_decode_pair_paged_equals_contiguous_bitwise():
    dt, B, Hq, Hkv, D, W, page_size = torch.bfloat16, 5, 16, 4, 128, 300, 128
    lens = [5000, 17, 4096, 1234, 3333]
    say("[paged decode] bitwise vs contiguous")
    max_len = max(lens) + 1
    cap = max_len
    max_pages = math.ceil(max_len / page_size)
    n_pages = B * max_pages + 1
    bt = block_table(B, max_pages, n_pages, 21)
    k0, v0 = rand((B, max(lens), Hkv, D), 22, dt), rand((B, max(lens), Hkv, D), 23, dt)
    kp, vp = paged_pool(k0, v0, lens, page_size, bt, n_pages, fill=0.0)
    kc = torch.zeros((B, Hkv, cap, D), dtype=dt, device=DEV)
    vc = torch.zeros_like(kc)
    for b in range(B):
        kc[b, :, :lens[b]] = k0[b, :lens[b]].permute(1, 0, 2)
        vc[b, :, :lens[b]] = v0[b, :lens[b]].permute(1, 0, 2)
    cl_p = torch.tensor(lens, dtype=torch.int32, device=DEV)
    cl_c = cl_p.clone()
    q, qx = rand((B, Hq, D), 24, dt), rand((B, Hq, D), 25, dt)
    kn, vn = rand((B, Hkv, D), 26, dt), rand((B, Hkv, D), 27, dt)
    a, b_ = affine_pair(Hq * D, 28)
    o_p, ox_p = torch.empty_like(q), torch.empty_like(q)
    o_c, ox_c = torch.empty_like(q), torch.empty_like(q)
    lo.orthros_decode_pair_paged(q, qx, a, b_, a, b_, kn, vn, kp, vp, bt, cl_p,
                                 o_p, ox_p, max_len_after=max_len, W=W)
    lo.orthros_decode_pair(q, qx, a, b_, a, b_, kn, vn, kc, vc, cl_c, o_c,
                           ox_c, max_len_after=max_len, W=W)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c) and torch.equal(ox_p, ox_c)
    assert torch.equal(cl_p, cl_c)


def test_decode_pair_paged_invalid_entry_is_flagged_not_read():
    dt, B, Hq, Hkv, D, W, page_size = torch.bfloat16, 3, 4, 1, 128, 32, 32
    lens = [100, 100, 100]
    say("[paged decode] out-of-range block-table entry")
    max_pages = 4
    n_pages = B * max_pages
    bt = block_table(B, max_pages, n_pages, 31)
    k0, v0 = rand((B, 100, Hkv, D), 32, dt), rand((B, 100, Hkv, D), 33, dt)
    kp, vp = paged_pool(k0, v0, lens, page_size, bt, n_pages)
    lo.orthros_check_device_errors()
    bt_bad = bt.clone()
    bt_bad[1, 3] = n_pages + 5          # the page that row 100 of b=1 needs
    bt_bad[1, 0] = -7                   # and one it reads
    snapshot = kp.clone()
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q, qx = rand((B, Hq, D), 34, dt), rand((B, Hq, D), 35, dt)
    kn, vn = rand((B, Hkv, D), 36, dt), rand((B, Hkv, D), 37, dt)
    a, b_ = affine_pair(Hq * D, 38)
    o, ox = torch.empty_like(q), torch.empty_like(q)
    lo.orthros_decode_pair_paged(q, qx, a, b_, a, b_, kn, vn, kp, vp, bt_bad,
                                 cl, o, ox, max_len_after=101, W=W)
    with pytest.raises(lo.OrthrosError):
        lo.orthros_check_device_errors()
    for b in (0, 2):     # untouched sequences are still exact
        c = oracle.Cache(1, Hkv, D, 101)
        c.append(f64(k0[b:b + 1]), f64(v0[b:b + 1]))
        o_r, ox_r = c.decode_pair(f64(q[b:b + 1]), f64(qx[b:b + 1]), f64(a),
                                  f64(b_), f64(a), f64(b_), f64(kn[b:b + 1]),
                                  f64(vn[b:b + 1]), W)
        compare(o[b:b + 1], o_r, dt, f"b={b} base")
        compare(ox[b:b + 1], ox_r, dt, f"b={b} output")
    # sequence 1's new row went nowhere: no page other than the two valid
    # new-row pages (b = 0, 2) changed
    changed = (kp.view(torch.int16) != snapshot.view(torch.int16)).flatten(1).any(1)
    changed_pages = set(torch.nonzero(changed).flatten().tolist())
    assert changed_pages <= {int(bt[0, 3]), int(bt[2, 3])}
