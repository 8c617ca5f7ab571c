"""GPU parity of the layer forward (projections + attention + W_O) against
the fp64 oracle, through the C ABI. Inputs are the seeded layer recipe of
``workloads.layer_inputs``; the oracle gets the exact bf16 bits."""
import numpy as np
import pytest
import torch

import long_context_prefill_swa_amd as lo
import oracle
from gpu_util import compare, f64, say
from workloads import Config, layer_inputs, workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_layer(cfg, cfg_id, W=None, d_model=None, cap=None, len_before=7):
    W = cfg.W if W is None else W
    x = layer_inputs(cfg, cfg_id, d_model, DEV)
    B, M, dm = x.x.shape
    cap = cfg.T if cap is None else cap
    kc = torch.full((B, cfg.Hkv, cap, cfg.D), float("nan"), dtype=torch.bfloat16,
                    device=DEV)
    vc = torch.full_like(kc, float("nan"))
    cl = torch.full((B,), len_before, dtype=torch.int32, device=DEV)
    y = torch.empty_like(x.x)
    wq, wk, wv, wo = x.stored_weights()
    lo.orthros_layer_forward(x.x, wq, wk, wv, wo, x.alpha, x.beta,
                             x.alpha_x, x.beta_x, kc, vc, cl, y, cfg.T_out, W)
    torch.cuda.synchronize()
    lo.orthros_check_device_errors()
    assert cl.tolist() == [cfg.T] * B
    return x, y, kc, vc


def oracle_layer(x, cfg, W, rows=None):
    return oracle.layer(f64(x.x), f64(x.w_q), f64(x.w_k), f64(x.w_v),
                        f64(x.w_o), f64(x.alpha), f64(x.beta), f64(x.alpha_x),
                        f64(x.beta_x), cfg.T_out, W, cfg.Hkv, cfg.D, rows=rows)


SMALL = [
    # name, B, Hq, Hkv, D, T, W, T_out, d_model
    ("roll", 2, 8, 2, 128, 300, 128, 3, 512),        # rolling-window kernel
    ("band", 1, 8, 2, 128, 1000, 1000, 1, 1024),     # banded kernel, W = T
    ("pt", 1, 4, 4, 128, 257, 64, 257, 384),         # every row also an output
    ("split", 1, 16, 2, 128, 700, 200, 1, 256),      # 8 query heads per KV head
    ("d64", 1, 4, 2, 64, 130, 33, 2, 128),           # D = 64: generic kernels
]


@pytest.mark.parametrize("idx", range(len(SMALL)), ids=[c[0] for c in SMALL])
def test_layer_forward_parity(idx):
    name, B, Hq, Hkv, D, T, W, T_out, dm = SMALL[idx]
    cfg = Config(f"layer_{name}", B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, W=W,
                 T_out=T_out, dtype="bf16")
    say(f"[layer] {name}: B={B} T={T} T_out={T_out} d_model={dm} W={W}")
    x, y, kc, _ = run_layer(cfg, 40 + idx, W=W, d_model=dm)
    compare(y, oracle_layer(x, cfg, W), torch.bfloat16, "layer y")
    # the cache holds x W_K of the base rows (bf16 GEMM result)
    k_ref = (f64(x.x[:, :T]) @ f64(x.w_k)).reshape(B, T, Hkv, D)
    compare(kc[:, :, :T].permute(0, 2, 1, 3), k_ref, torch.bfloat16, "cache K")


@pytest.mark.parametrize("W", [4096, 128])
def test_layer_forward_128k_sampled(W):
    """The 128K prefill layer (d_model 4096, 32/8 heads, one output row) on
    sampled rows: band and tile edges, random rows and the output row."""
    cfg, cfg_id = workload("prefill_128k")
    say(f"[layer full size] prefill_128k W={W}")
    x, y, _, _ = run_layer(cfg, cfg_id, W=W)
    T, M = cfg.T, cfg.T + cfg.T_out
    rng = np.random.default_rng(W)
    rows = {0, 1, 63, 64, W - 1, W, T - 2, T - 1, M - 1}
    rows.update(int(r) for r in rng.integers(0, T, 12))
    rows = sorted(r for r in rows if 0 <= r < M)
    ref = oracle_layer(x, cfg, W, rows=rows)
    compare(y[:, rows], ref, torch.bfloat16, f"layer y ({len(rows)} rows)")
