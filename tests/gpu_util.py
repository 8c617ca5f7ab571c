"""Shared helpers of the GPU parity tests (marshalling and comparison only)."""
import sys

import numpy as np
import torch

import long_context_prefill_swa_amd as lo

# Tolerances: max-abs as fixed for the two precisions (1e-4 fp32, 2e-2 bf16
# inputs with fp32 accumulation); relative L2 added because with N(0,1)
# inputs the outputs are small (about 1/sqrt(number of keys)), where a
# max-abs bound alone says little.
TOL = {torch.float32: (1e-4, 1e-5), torch.bfloat16: (2e-2, 1e-2)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def make_cache(k, v, cap, fill=0.0):
    """Cache [B, Hkv, cap, D] filled with `fill`, then k/v [B, T, Hkv, D]
    appended through the library; returns (k_cache, v_cache, cache_len)."""
    B, T, Hkv, D = k.shape
    kc = torch.full((B, Hkv, cap, D), fill, dtype=k.dtype, device=k.device)
    vc = torch.full((B, Hkv, cap, D), fill, dtype=k.dtype, device=k.device)
    cl = torch.zeros(B, dtype=torch.int32, device=k.device)
    lo.orthros_kv_append(kc, vc, cl, k.contiguous(), v.contiguous())
    return kc, vc, cl


def compare(got, ref, dtype, what, tol=None):
    g = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got)
    ref = np.asarray(ref)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    atol, rl2_tol = tol or TOL[dtype]
    diff = np.abs(g - ref)
    maxabs = float(diff.max()) if diff.size else 0.0
    denom = float(np.linalg.norm(ref)) or 1.0
    rl2 = float(np.linalg.norm(g - ref)) / denom
    say(f"  {what}: max-abs {maxabs:.3e} (<= {atol}), rel-L2 {rl2:.3e} "
        f"(<= {rl2_tol})")
    assert maxabs <= atol, f"{what}: max-abs {maxabs} > {atol}"
    assert rl2 <= rl2_tol, f"{what}: rel-L2 {rl2} > {rl2_tol}"
    return maxabs, rl2
