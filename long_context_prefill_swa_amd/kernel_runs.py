"""Single-kernel runs for hardware-counter profiling.

    python -m long_context_prefill_swa_amd.kernel_runs <target> [--reps N]

Targets (synthetic seeded inputs, set up before the measured launches):
  swa_128k      orthros_swa_prefill, B=1 Hq=32 Hkv=8 D=128 T=131072 W=4096
  swa_w128      the same at W=128 (the rolling-window kernel)
  backward_sft  orthros_attn_backward, B=4 Hq=32 Hkv=8 T=8192 T_out=2048
                W=1024 (forward outputs from the library, seeded dO)
  global_128k   orthros_global_xattn, one output row over 131072 keys
  decode_b64    orthros_decode_pair, B=64 with 32768 cached tokens, W=2048
  copy_1g       a plain device-to-device copy of 1 GiB (torch), the
                reference for scaling the memory counters to bytes

Meant to run under `rocprofv3 --pmc ...`: every launch of the target is one
dispatch, and the copy gives FETCH_SIZE / WRITE_SIZE for exactly 1 GiB read
and 1 GiB written, from which the per-launch counters of a kernel are turned
into HBM bytes. Prints one line per target with the launch count.
"""
import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("target", choices=["swa_128k", "swa_w128", "global_128k",
                                       "decode_b64", "backward_sft",
                                       "copy_1g"])
    ap.add_argument("--reps", type=int, default=2)
    args = ap.parse_args()

    import torch

    import long_context_prefill_swa_amd as lo
    from workloads import (affine_inputs, decode_all_steps, kv_inputs,
                           normal, prefill_inputs, workload)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.target == "copy_1g":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy_1g: {args.reps} copies of {1 << 30} bytes", flush=True)
        return

    lo.lib()
    if args.target == "backward_sft":
        c, cid = workload("sft_dual_8k")
        x = prefill_inputs(c, cid, dev)
        kc = torch.empty((c.B, c.Hkv, c.T, c.D), dtype=torch.bfloat16,
                         device=dev)
        vc = torch.empty_like(kc)
        cl = torch.zeros(c.B, dtype=torch.int32, device=dev)
        lo.orthros_kv_append(kc, vc, cl, x.k, x.v)
        o = torch.empty_like(x.q_pre)
        ox = torch.empty_like(x.qx_pre)
        lo.orthros_swa_prefill(x.q_pre, x.alpha, x.beta, kc, vc, o, c.W)
        lo.orthros_global_xattn(x.qx_pre, x.alpha_x, x.beta_x, kc, vc, ox,
                                c.T_in)
        d_o = normal(tuple(o.shape), 9001, torch.bfloat16, dev)
        d_ox = normal(tuple(ox.shape), 9002, torch.bfloat16, dev)
        ws = lo.workspace(lo.orthros_backward_workspace_bytes(
            c.B, c.T, c.T_out, c.Hq, c.Hkv, c.D), dev)
        run = lambda: lo.orthros_attn_backward(  # noqa: E731
            x.q_pre, x.qx_pre, x.alpha, x.beta, x.alpha_x, x.beta_x, kc, vc,
            o, ox, d_o, d_ox, c.W, ws=ws)
    elif args.target in ("swa_128k", "swa_w128", "global_128k"):
        pc, pc_id = workload("prefill_128k")
        px = prefill_inputs(pc, pc_id, dev)
        kc = torch.empty((pc.B, pc.Hkv, pc.T, pc.D), dtype=torch.bfloat16,
                         device=dev)
        vc = torch.empty_like(kc)
        cl = torch.zeros(pc.B, dtype=torch.int32, device=dev)
        lo.orthros_kv_append(kc, vc, cl, px.k, px.v)
        if args.target in ("swa_128k", "swa_w128"):
            o = torch.empty_like(px.q_pre)
            W = pc.W if args.target == "swa_128k" else 128
            run = lambda: lo.orthros_swa_prefill(  # noqa: E731
                px.q_pre, px.alpha, px.beta, kc, vc, o, W)
        else:
            ox = torch.empty_like(px.qx_pre)
            ws = lo.workspace(lo.orthros_workspace_bytes(
                lo.ORTHROS_OP_GLOBAL_XATTN, pc.B, pc.Hq, pc.Hkv, pc.D,
                pc.T_out, pc.T), dev)
            run = lambda: lo.orthros_global_xattn(  # noqa: E731
                px.qx_pre, px.alpha_x, px.beta_x, kc, vc, ox, pc.T_in, ws=ws)
    else:
        dc, dc_id = workload("decode_pair_b64")
        cap = dc.T + args.reps
        kc = torch.empty((dc.B, dc.Hkv, cap, dc.D), dtype=torch.bfloat16,
                         device=dev)
        vc = torch.empty_like(kc)
        cl = torch.zeros(dc.B, dtype=torch.int32, device=dev)
        k0, v0 = kv_inputs(dc, dc_id, dev)
        lo.orthros_kv_append(kc, vc, cl, k0, v0)
        del k0, v0
        a, b, ax, bx = affine_inputs(dc, dc_id, dev)
        st = decode_all_steps(dc, dc_id, steps=args.reps, device=dev)
        o = torch.empty((dc.B, dc.Hq, dc.D), dtype=torch.bfloat16, device=dev)
        ox = torch.empty_like(o)
        ws = lo.workspace(lo.orthros_workspace_bytes(
            lo.ORTHROS_OP_DECODE_PAIR, dc.B, dc.Hq, dc.Hkv, dc.D, 1, cap), dev)
        steps = iter(range(args.reps))

        def run():
            s = next(steps)
            lo.orthros_decode_pair(st.q_pre[s], st.qx_pre[s], a, b, ax, bx,
                                   st.k_new[s], st.v_new[s], kc, vc, cl, o,
                                   ox, dc.T + s + 1, dc.W, ws=ws)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        run()
    torch.cuda.synchronize()
    lo.orthros_check_device_errors()
    print(f"{args.target}: {args.reps} launches", flush=True)


if __name__ == "__main__":
    main()
