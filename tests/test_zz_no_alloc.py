"""The no-allocation decode pair (orthros_decode_pair_noalloc) against the
decode pair with a caller workspace (orthros_decode_pair), through the C
ABI: two calls in a row on the same device (the second with a smaller
batch, fewer cached keys and another window), each compared bit for bit
with the workspace entry point on an identical copy of the cache: both
outputs, the appended rows and the advanced lengths. Both run the same
kernels, so the results are identical, not merely close."""
import pytest
import torch

import long_context_prefill_swa_amd as lo
from gpu_util import make_cache, say
from workloads import normal

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


def _bits(t):
    return t.view(torch.int16) if t.dtype == BF else t.view(torch.int32)


def _one_call(B, Hq, Hkv, L0, W, seed, dt=BF, D=128):
    q, qx = normal((B, Hq, D), seed, dt, DEV), normal((B, Hq, D), seed + 1, dt, DEV)
    kn, vn = normal((B, Hkv, D), seed + 2, dt, DEV), normal((B, Hkv, D), seed + 3, dt, DEV)
    k0, v0 = normal((B, L0, Hkv, D), seed + 4, dt, DEV), normal((B, L0, Hkv, D), seed + 5, dt, DEV)
    a = 1 + 0.1 * normal((Hq * D,), seed + 6, torch.float32, DEV)
    b = 0.1 * normal((Hq * D,), seed + 7, torch.float32, DEV)
    ax = 1 + 0.1 * normal((Hq * D,), seed + 8, torch.float32, DEV)
    bx = 0.1 * normal((Hq * D,), seed + 9, torch.float32, DEV)
    cap = L0 + 3
    runs = {}
    for name in ("workspace", "noalloc"):
        kc, vc, cl = make_cache(k0, v0, cap, fill=float("nan"))
        o = torch.full((B, Hq, D), float("nan"), dtype=dt, device=DEV)
        ox = torch.full_like(o, float("nan"))
        if name == "workspace":
            lo.orthros_decode_pair(q, qx, a, b, ax, bx, kn, vn, kc, vc, cl, o,
                                   ox, max_len_after=L0 + 1, W=W)
        else:
            lo.orthros_decode_pair_noalloc(q, qx, a, b, ax, bx, kn, vn, kc, vc,
                                           cl, o, ox, max_len_after=L0 + 1,
                                           W=W)
        torch.cuda.synchronize()
        runs[name] = (o, ox, kc, vc, cl)
    lo.orthros_check_device_errors()
    (o1, ox1, kc1, vc1, cl1), (o2, ox2, kc2, vc2, cl2) = runs["workspace"], runs["noalloc"]
    assert cl2.tolist() == [L0 + 1] * B and torch.equal(cl1, cl2)
    assert torch.isfinite(o2.float()).all() and torch.isfinite(ox2.float()).all()
    assert torch.equal(_bits(o1), _bits(o2)), "base outputs differ"
    assert torch.equal(_bits(ox1), _bits(ox2)), "output-stream outputs differ"
    assert torch.equal(_bits(kc1[:, :, :L0 + 1]), _bits(kc2[:, :, :L0 + 1]))
    assert torch.equal(_bits(vc1[:, :, :L0 + 1]), _bits(vc2[:, :, :L0 + 1]))


def test_noalloc_decode_pair_equals_workspace_entry_point():
    say("[no-alloc decode pair] call 1: B=16, 32/8 heads, 5000 keys, W=1024")
    need1 = lo.orthros_workspace_bytes(lo.ORTHROS_OP_DECODE_PAIR, 16, 32, 8,
                                       128, 1, 5001)
    assert 0 < need1 <= lo.ORTHROS_NOALLOC_SCRATCH_BYTES
    _one_call(16, 32, 8, 5000, 1024, 900)
    say("[no-alloc decode pair] call 2: B=3, 8/2 heads, 700 keys, W=64")
    _one_call(3, 8, 2, 700, 64, 920)


def test_noalloc_decode_pair_generic_path():
    """fp32 runs the generic kernels, which use no scratch at all."""
    say("[no-alloc decode pair] fp32, D=16")
    _one_call(2, 4, 2, 90, 16, 940, dt=torch.float32, D=16)
