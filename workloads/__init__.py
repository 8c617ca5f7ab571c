"""Seeded synthetic workloads for Orthros attention.

This module holds only shapes and random draws: none of the method's
arithmetic. Both the fp64 oracle (through the tests) and the HIP path are
fed from it, so the two see the exact same input bits.

Recipe (the same for every configuration):
  * Q (base and output stream), K and V: fp32 draws from N(0, 1) with a
    torch generator seeded per (configuration, tensor), then rounded to
    nearest-even in the configuration's dtype (bf16 or fp32).
  * alpha, alpha': 1 + 0.1 * N(0, 1); beta, beta': 0.1 * N(0, 1); fp32, one
    value per channel of the Hq*D query projection.
  * The 1/sqrt(D) softmax scale is part of the method, not of the inputs.
  * Layer forward: hidden rows x ~ N(0, 1) ([B, T + T_out, d_model], the T
    base rows then the T_out output rows, drawn independently); weights
    N(0, 1) / sqrt(fan_in), then rounded to bf16, so every projection has
    unit variance. d_model = Hq * D unless stated.
The pages' efficiency workloads are length-only (128K input / short
output); these configurations stand in for them with synthetic tensors.
"""
from dataclasses import dataclass, field, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int              # total positions of the prefill (T_in + T_out)
    W: int              # sliding window of the base stream
    T_out: int          # output-stream rows (last T_out positions)
    dtype: str          # "f32" or "bf16"
    decode_steps: int = 0   # > 0: decode-pair workload starting at length T
    identity_affine: bool = False
    notes: str = field(default="", compare=False)

    @property
    def T_in(self) -> int:
        return self.T - self.T_out

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The five workloads (index = configuration id used in seeds).
CONFIGS = [
    Config("tiny_f32", B=1, Hq=2, Hkv=2, D=16, T=64, W=16, T_out=1,
           dtype="f32", notes="tiny prefill, fp32; also W=64 identity run"),
    Config("prefill_32k", B=1, Hq=32, Hkv=8, D=128, T=32768, W=2048,
           T_out=1, dtype="bf16", notes="single-layer prefill, GQA 32/8"),
    Config("sft_dual_8k", B=4, Hq=32, Hkv=8, D=128, T=8192, W=1024,
           T_out=2048, dtype="bf16", notes="SFT-style dual stream"),
    Config("decode_pair_b64", B=64, Hq=32, Hkv=8, D=128, T=32768, W=2048,
           T_out=1, dtype="bf16", decode_steps=256,
           notes="decode pair, 32768 cached tokens, 256 steps"),
    Config("prefill_128k", B=1, Hq=32, Hkv=8, D=128, T=131072, W=4096,
           T_out=1, dtype="bf16", notes="long-context prefill + causal"),
]

def workload(name: str):
    """(config, seed-space id) of the workload called `name`."""
    for i, c in enumerate(CONFIGS):
        if c.name == name:
            return c, i
    raise KeyError(name)


# Tensor ids inside a configuration's seed space.
_TID = {"q_pre": 1, "qx_pre": 2, "k": 3, "v": 4, "alpha": 5, "beta": 6,
        "alpha_x": 7, "beta_x": 8, "x": 9, "w_q": 10, "w_k": 11, "w_v": 12,
        "w_o": 13}


def seed_of(cfg_id: int, tensor: str, step: int = 0) -> int:
    return 1000 * cfg_id + _TID[tensor] + 16 * (step + 1) * (step > 0)


def normal(shape, seed: int, dtype, device="cpu") -> torch.Tensor:
    """fp32 N(0,1) draw with its own generator, rounded to `dtype`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


def affine(n: int, seed_scale: int, seed_shift: int, device="cpu",
           identity: bool = False):
    """Per-channel scale/offset vectors: 1 + 0.1 N(0,1) and 0.1 N(0,1)."""
    if identity:
        return (torch.ones(n, device=device), torch.zeros(n, device=device))
    a = 1.0 + 0.1 * normal((n,), seed_scale, torch.float32, device)
    b = 0.1 * normal((n,), seed_shift, torch.float32, device)
    return a, b


@dataclass
class PrefillInputs:
    q_pre: torch.Tensor    # [B, T, Hq, D]
    qx_pre: torch.Tensor   # [B, T_out, Hq, D]
    k: torch.Tensor        # [B, T, Hkv, D]  (projection layout)
    v: torch.Tensor        # [B, T, Hkv, D]
    alpha: torch.Tensor    # [Hq*D] fp32
    beta: torch.Tensor
    alpha_x: torch.Tensor
    beta_x: torch.Tensor


def affine_inputs(cfg: Config, cfg_id: int, device="cpu"):
    """(alpha, beta, alpha_x, beta_x) of a configuration."""
    s = lambda name: seed_of(cfg_id, name)  # noqa: E731
    n = cfg.Hq * cfg.D
    a, b = affine(n, s("alpha"), s("beta"), device, cfg.identity_affine)
    ax, bx = affine(n, s("alpha_x"), s("beta_x"), device, cfg.identity_affine)
    return a, b, ax, bx


def kv_inputs(cfg: Config, cfg_id: int, device="cpu"):
    """Base-stream K and V [B, T, Hkv, D] of a configuration."""
    dt = cfg.torch_dtype
    shape = (cfg.B, cfg.T, cfg.Hkv, cfg.D)
    return (normal(shape, seed_of(cfg_id, "k"), dt, device),
            normal(shape, seed_of(cfg_id, "v"), dt, device))


def prefill_inputs(cfg: Config, cfg_id: int, device="cpu") -> PrefillInputs:
    dt = cfg.torch_dtype
    B, T, Hq, D = cfg.B, cfg.T, cfg.Hq, cfg.D
    s = lambda name: seed_of(cfg_id, name)  # noqa: E731
    a, b, ax, bx = affine_inputs(cfg, cfg_id, device)
    k, v = kv_inputs(cfg, cfg_id, device)
    return PrefillInputs(
        q_pre=normal((B, T, Hq, D), s("q_pre"), dt, device),
        qx_pre=normal((B, cfg.T_out, Hq, D), s("qx_pre"), dt, device),
        k=k, v=v, alpha=a, beta=b, alpha_x=ax, beta_x=bx)


@dataclass
class DecodeStepInputs:
    q_pre: torch.Tensor    # [B, Hq, D]
    qx_pre: torch.Tensor   # [B, Hq, D]
    k_new: torch.Tensor    # [B, Hkv, D]
    v_new: torch.Tensor    # [B, Hkv, D]


def decode_step_inputs(cfg: Config, cfg_id: int, step: int,
                       device="cpu") -> DecodeStepInputs:
    dt = cfg.torch_dtype
    B, Hq, Hkv, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.D
    s = lambda name: seed_of(cfg_id, name, step + 1)  # noqa: E731
    return DecodeStepInputs(
        q_pre=normal((B, Hq, D), s("q_pre"), dt, device),
        qx_pre=normal((B, Hq, D), s("qx_pre"), dt, device),
        k_new=normal((B, Hkv, D), s("k"), dt, device),
        v_new=normal((B, Hkv, D), s("v"), dt, device))


def decode_all_steps(cfg: Config, cfg_id: int, steps: Optional[int] = None,
                     device="cpu") -> DecodeStepInputs:
    """All decode steps stacked on a leading [steps] axis (one draw each)."""
    n = cfg.decode_steps if steps is None else steps
    dt = cfg.torch_dtype
    B, Hq, Hkv, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.D
    s = lambda name: seed_of(cfg_id, name, 10_000)  # noqa: E731
    return DecodeStepInputs(
        q_pre=normal((n, B, Hq, D), s("q_pre"), dt, device),
        qx_pre=normal((n, B, Hq, D), s("qx_pre"), dt, device),
        k_new=normal((n, B, Hkv, D), s("k"), dt, device),
        v_new=normal((n, B, Hkv, D), s("v"), dt, device))


@dataclass
class LayerInputs:
    x: torch.Tensor        # [B, T + T_out, d_model] bf16
    w_q: torch.Tensor      # [d_model, Hq*D]
    w_k: torch.Tensor      # [d_model, Hkv*D]
    w_v: torch.Tensor      # [d_model, Hkv*D]
    w_o: torch.Tensor      # [Hq*D, d_model]
    alpha: torch.Tensor
    beta: torch.Tensor
    alpha_x: torch.Tensor
    beta_x: torch.Tensor

    def stored_weights(self):
        """The four weights stored out x in (a linear layer's layout, the
        form the layer entry point takes): contiguous transposes."""
        return tuple(w.t().contiguous()
                     for w in (self.w_q, self.w_k, self.w_v, self.w_o))


def scaled_normal(shape, seed: int, fan_in: int, dtype, device="cpu"):
    """N(0, 1) / sqrt(fan_in), drawn in fp32, then rounded to `dtype`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return (w * fan_in ** -0.5).to(dtype)


def layer_inputs(cfg: Config, cfg_id: int, d_model: Optional[int] = None,
                 device="cpu") -> LayerInputs:
    """Inputs of one layer forward: hidden rows, the four weights as the
    matrices of x W (stored_weights() gives them out x in), the affine
    vectors (bf16 tensors, fp32 affine)."""
    dm = cfg.Hq * cfg.D if d_model is None else d_model
    s = lambda name: seed_of(cfg_id, name)  # noqa: E731
    bf = torch.bfloat16
    HqD, HkvD = cfg.Hq * cfg.D, cfg.Hkv * cfg.D
    a, b, ax, bx = affine_inputs(cfg, cfg_id, device)
    return LayerInputs(
        x=normal((cfg.B, cfg.T + cfg.T_out, dm), s("x"), bf, device),
        w_q=scaled_normal((dm, HqD), s("w_q"), dm, bf, device),
        w_k=scaled_normal((dm, HkvD), s("w_k"), dm, bf, device),
        w_v=scaled_normal((dm, HkvD), s("w_v"), dm, bf, device),
        w_o=scaled_normal((HqD, dm), s("w_o"), HqD, bf, device),
        alpha=a, beta=b, alpha_x=ax, beta_x=bx)
