"""The split-KV calls' two merge modes and their arrival counters.

A call whose grid the chip holds at once (at most 512 workgroups of one
(chunk, head group, sequence) each) merges in the same launch: the last
workgroup of each head group to finish combines the partials, and in a
decode step the last workgroup of a sequence advances its length. Larger
grids merge in a second launch. These tests run both modes of the output
row and of the decode step against the oracle, and check the counter
contract of the header: the leading counter bytes of a workspace are zero
after every call, so one workspace serves any number of calls.
"""
import pytest
import torch

import long_context_prefill_swa_amd as lo
import oracle
from gpu_util import compare, f64, make_cache, say
from workloads import normal

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


def rand(shape, seed):
    return normal(shape, seed, BF, DEV)


def affine_pair(n, seed):
    a = 1.0 + 0.1 * normal((n,), seed, torch.float32, DEV)
    b = 0.1 * normal((n,), seed + 1, torch.float32, DEV)
    return a, b


def counters_zero(op, B, Hq, Hkv, T_out, max_len, ws):
    cb = lo.orthros_workspace_counter_bytes(op, B, Hq, Hkv, 128, T_out, max_len)
    assert cb > 0
    return bool((ws[:cb] == 0).all().item())


# Output row, 16 query heads on 16 KV heads (16 groups), 1024 keys: B = 8
# takes 512-key chunks, 256 workgroups (one launch); B = 40 takes one
# 4096-key chunk per group, 640 workgroups (two launches).
@pytest.mark.parametrize("B", [8, 40])
def test_output_row_both_merge_modes(B):
    Hq, Hkv, D, T_in, T_out = 16, 16, 128, 1023, 1
    T = T_in + T_out
    say(f"[split-KV modes] output row B={B}")
    qx = rand((B, T_out, Hq, D), 300)
    k, v = rand((B, T, Hkv, D), 301), rand((B, T, Hkv, D), 302)
    a, b = affine_pair(Hq * D, 303)
    kc, vc, _ = make_cache(k, v, T, fill=float("nan"))
    ws = lo.workspace(lo.orthros_workspace_bytes(
        lo.ORTHROS_OP_GLOBAL_XATTN, B, Hq, Hkv, D, T_out, T), DEV)
    outs = []
    for _ in range(2):  # the same workspace twice
        ox = torch.empty_like(qx)
        lo.orthros_global_xattn(qx, a, b, kc, vc, ox, T_in, ws=ws)
        torch.cuda.synchronize()
        assert counters_zero(lo.ORTHROS_OP_GLOBAL_XATTN, B, Hq, Hkv, T_out, T, ws)
        outs.append(ox)
    assert torch.equal(outs[0], outs[1])
    ref = oracle.xattn(f64(qx), f64(a), f64(b), f64(k), f64(v), T_in)[0]
    compare(outs[0], ref, BF, "output row")


# Decode step, 8 query heads on 2 KV heads (2 groups of 4 heads, 8 rows each
# with both streams), up to 600 keys: B = 8 takes 256-key chunks, 48
# workgroups (one launch); B = 300 takes one 2048-key chunk per group, 600
# workgroups (two launches). One sequence sits at the capacity bound and
# must be skipped.
@pytest.mark.parametrize("B", [8, 300])
def test_decode_step_both_merge_modes(B):
    Hq, Hkv, D, W = 8, 2, 128, 300
    L0, cap = 599, 600
    say(f"[split-KV modes] decode B={B}")
    k0, v0 = rand((B, L0, Hkv, D), 310), rand((B, L0, Hkv, D), 311)
    kc, vc, cl = make_cache(k0, v0, cap, fill=float("nan"))
    full = B // 2  # this sequence is already full: skipped, flagged
    kc[full, :, L0:] = 0.0
    vc[full, :, L0:] = 0.0
    cl[full] = cap
    q, qx = rand((B, Hq, D), 312), rand((B, Hq, D), 313)
    kn, vn = rand((B, Hkv, D), 314), rand((B, Hkv, D), 315)
    a, b = affine_pair(Hq * D, 316)
    ax, bx = affine_pair(Hq * D, 318)
    ws = lo.workspace(lo.orthros_workspace_bytes(
        lo.ORTHROS_OP_DECODE_PAIR, B, Hq, Hkv, D, 1, cap), DEV)
    o, ox = torch.empty_like(q), torch.empty_like(q)
    lo.orthros_check_device_errors()
    lo.orthros_decode_pair(q, qx, a, b, ax, bx, kn, vn, kc, vc, cl, o, ox,
                           max_len_after=cap, W=W, ws=ws)
    torch.cuda.synchronize()
    with pytest.raises(lo.OrthrosError):
        lo.orthros_check_device_errors()
    assert counters_zero(lo.ORTHROS_OP_DECODE_PAIR, B, Hq, Hkv, 1, cap, ws)
    want = [L0 + 1] * B
    want[full] = cap
    assert cl.tolist() == want
    assert (o[full].float() == 0).all() and (ox[full].float() == 0).all()
    for bi in sorted({0, 1, B - 1, full - 1}):
        c = oracle.Cache(1, Hkv, D, L0 + 1)
        c.append(f64(k0[bi:bi + 1]), f64(v0[bi:bi + 1]))
        o_r, ox_r = c.decode_pair(f64(q[bi:bi + 1]), f64(qx[bi:bi + 1]), f64(a),
                                  f64(b), f64(ax), f64(bx), f64(kn[bi:bi + 1]),
                                  f64(vn[bi:bi + 1]), W)
        compare(o[bi:bi + 1], o_r, BF, f"b={bi} base")
        compare(ox[bi:bi + 1], ox_r, BF, f"b={bi} output")
