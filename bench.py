#!/usr/bin/env python3
"""Throughput of the NF4 + double-quantisation + LoRA linear path on one MI355X.

Step (the timed unit, `value`): forward + backward (Y; dX, dA, dB) of the
seven LoRA linears of a 65B-class decoder layer (hidden 8192, FFN 22016:
q, k, v, o 8192x8192; gate, up 22016x8192; down 8192x22016), weights
0.02 Student-t(5) (heavy tails stress the block absmax), NF4 +
double-quantised, LoRA r=64, alpha=16, 8192 tokens (16 x 512); inputs
resident in HBM. As in a decoder layer, q / k / v share one input and
gate / up another: they run as grouped linears (one pass over the shared
input for the projections and dA, one GEMM for the summed dX).
`--config 7b` makes the LLaMA-7B-shaped layer (hidden 4096, FFN 11008,
N(0, 0.02) weights) the step instead.
`value` = algorithmic TFLOP/s of the step: sum over linears of
4 M N K (base forward + input gradient) + 6 M r (K + N) (LoRA), no dW.

Legs timed in the same run:
  other_layer the step of the other layer shape (LLaMA-7B by default)
  ungrouped the same seven linears run independently, each on its own input
  quantize  NF4 + fp8 DQ of a stack of 65B-class layers (4 x 8192^2 +
            3 x 22016x8192 weights per layer, one batched launch per layer),
            2.51587 B moved per weight
  dequant   round trip of the same stack to bf16, 2.51587 B per weight, the
            outputs rotating over 8 buffers so that nothing stays cached
  gemv      few-token forward (M = 1, 16) of 4096x4096 and 11008x4096 with
            LoRA r=64, rotating over >= 1 GB of distinct weight sets; the
            chain of calls is captured once as a HIP graph and replayed (the
            eager time per call, host launch cost included, is reported too)
  gemm512   forward at M = 512 (small-GEMM regime)
  roofline  the step's dominant kernel alone: the dequant-in-LDS MFMA GEMM
            with the rank term fused in its epilogue, in the step's input-
            gradient and forward orientations over the step's four units
            (qlora_4bit_matmul_lora launches the step's template instance),
            timed with HIP events on the launch stream; the orientation with
            the larger time per step is `roofline`, the other a leg. Its HBM
            traffic per launch comes from the FETCH_SIZE / WRITE_SIZE counter
            runs recorded in profiles/ (null when the GEMM source or the
            kernel has changed since)
  formats   the Int4 / FP4 comparison types and the format without double
            quantisation beside NF4 + DQ: quantise and bf16-dequantise GB/s of
            one 22016x8192 weight (each format's own bytes per weight), the
            relative dequantisation error on N(0, 0.02) weights, bits per
            weight, and the forward GEMM at 8192x4096x4096
  merge     the dense deployment weights bf16(W^ + s B A) of the layer's seven
            linears (2.52 B moved per weight)
  adamw     the adapters' optimizer step for a 32-layer 7B model (160M LoRA
            parameters, 28 B moved per parameter) with the moments in HBM,
            then paged out to pinned host memory (the kernel works on them
            in place over the host link), and the page-out / page-in copies
  copycal   one elementwise pass reading and writing exactly 1 GiB each, the
            calibration point of those counters
            (see bit_nf4_quantized_12_amd/pmc_traffic.py)
cpu_baseline: the float64 oracle (tests only, never on the product path) on
a bounded sample of the step's work, on the host cores.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
# the GEMM template instances the step launches from 1024 tokens on (512 x 128 tiles, rank term fused)
GEMM_KERNEL_DX = "gemm_kernel<512, 128, true, true, true, false>"
GEMM_KERNEL_FWD = "gemm_kernel<512, 128, false, true, true, false>"
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
Q_BYTES_PER_W = 2.0 + 0.5 + 1.0 / 64 + 4.0 / 16384   # read bf16, write codes, c2, c1


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", choices=["7b", "65b"], default="65b",
                    help="layer shapes of the step: 65B-class (default) or LLaMA-7B")
    ap.add_argument("--stack-layers", type=int, default=80, help="65B-class layers in the quantize leg")
    ap.add_argument("--legs", default="other_layer,ungrouped,roofline,quantize,gemv,gemm512,formats,merge,adamw",
                    help="comma list of extra legs, or 'none'")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one MI355X: the path has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_nf4_quantized_12_amd as q
    from bit_nf4_quantized_12_amd import synth

    q.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    def timed(fn, reps):
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record(stream)
        for _ in range(reps):
            fn()
        s1.record(stream)
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / 1e3

    M, r, alpha = 8192, 64, 16.0
    s = alpha / r
    gen_seed = 0

    def build_layer(config):
        """The seven linears of one decoder layer and the step's four units
        (q/k/v and gate/up grouped on their shared inputs), inputs resident."""
        hidden, ffn = (4096, 11008) if config == "7b" else (8192, 22016)
        shapes = synth.llama_linears(hidden, ffn)
        log(f"preparing {config} layer: {[(n, N, K) for n, N, K in shapes]}, M={M}, r={r}")
        lin = []
        ws_bytes = 0
        for i, (name, N, K) in enumerate(shapes):
            base = 1000 * i
            if config == "65b":  # Student-t(5) * 0.02 to stress absmax outliers
                torch.manual_seed(gen_seed + base + 7)
                t = torch.distributions.StudentT(torch.tensor(5.0, device=dev))
                w = (t.sample((N, K)) * 0.02).to(torch.bfloat16)
            else:
                w = synth.device_normal_bf16(N * K, 0.02, gen_seed + base + 1, dev).view(N, K)
            W = q.quantize_weight(w.contiguous())
            del w
            A = synth.device_normal_bf16(r * K, 0.02, gen_seed + base + 2, dev).view(r, K)
            B = synth.device_normal_bf16(N * r, 0.02, gen_seed + base + 3, dev).view(N, r)
            X = synth.device_normal_bf16(M * K, 1.0, gen_seed + base + 4, dev).view(M, K)
            dY = synth.device_normal_bf16(M * N, 1.0, gen_seed + base + 5, dev).view(M, N)
            lin.append(dict(name=name, N=N, K=K, W=W, A=A, B=B, X=X, dY=dY, out=None))
            ws_bytes = max(ws_bytes, q.qlora_linear_workspace_bytes(M, N, K, r))
        # The decoder layer: q / k / v read the same input, and so do gate /
        # up, so they run as grouped linears (stacked weights and adapters;
        # every N K here is a whole number of 16384-weight groups, so the
        # stacked stored weight is the concatenation of the per-linear ones).
        units = []
        for name, idx in (("qkv", [0, 1, 2]), ("o", [3]), ("gate_up", [4, 5]), ("down", [6])):
            Ls = [lin[i] for i in idx]
            K = Ls[0]["K"]
            Nt = sum(L["N"] for L in Ls)
            g = len(Ls)
            out = dict(Y=torch.empty(M, Nt, dtype=torch.bfloat16, device=dev),
                       T=torch.empty(M, g * r, dtype=torch.float32, device=dev),
                       dX=torch.empty(M, K, dtype=torch.bfloat16, device=dev),
                       dA=torch.empty(g * r, K, dtype=torch.bfloat16, device=dev),
                       dB=torch.empty(Nt, r, dtype=torch.bfloat16, device=dev))
            if g == 1:
                L = Ls[0]
                L["out"] = out
                units.append(dict(name=name, g=1, N=Nt, K=K, W=L["W"], A=L["A"], B=L["B"], X=L["X"],
                                  dY=L["dY"], out=out))
                continue
            Wst = q.NF4Weight(torch.cat([L["W"].codes for L in Ls]), torch.cat([L["W"].c2 for L in Ls]),
                              torch.cat([L["W"].c1 for L in Ls]), Nt, K)
            units.append(dict(name=name, g=g, N=Nt, K=K, W=Wst, A=torch.cat([L["A"] for L in Ls]),
                              B=torch.cat([L["B"] for L in Ls]), X=Ls[0]["X"],
                              dY=torch.cat([L["dY"] for L in Ls], dim=1).contiguous(), out=out))
            ws_bytes = max(ws_bytes, q.qlora_linear_grouped_workspace_bytes(M, Nt, K, r, g))
        for L in lin:
            if L["out"] is None:
                L["out"] = dict(Y=torch.empty(M, L["N"], dtype=torch.bfloat16, device=dev),
                                T=torch.empty(M, r, dtype=torch.float32, device=dev),
                                dX=torch.empty(M, L["K"], dtype=torch.bfloat16, device=dev),
                                dA=torch.empty(r, L["K"], dtype=torch.bfloat16, device=dev),
                                dB=torch.empty(L["N"], r, dtype=torch.bfloat16, device=dev))
        ws = q.new_workspace(ws_bytes, dev)
        flops = sum(4.0 * M * L["N"] * L["K"] + 6.0 * M * r * (L["K"] + L["N"]) for L in lin)
        torch.cuda.synchronize()
        return dict(config=config, hidden=hidden, ffn=ffn, lin=lin, units=units, ws=ws, flops=flops)

    def step_of(layer):
        ws = layer["ws"]

        def step():
            for U in layer["units"]:
                o = U["out"]
                if U["g"] == 1:
                    q.qlora_linear_fwd(U["W"], U["X"], U["A"], U["B"], s, Y=o["Y"], T=o["T"], workspace=ws)
                    q.qlora_linear_bwd(U["W"], U["X"], U["A"], U["B"], U["dY"], o["T"], s,
                                       dX=o["dX"], dA=o["dA"], dB=o["dB"], workspace=ws)
                else:
                    q.qlora_linear_fwd_grouped(U["W"], U["g"], U["X"], U["A"], U["B"], s, Y=o["Y"], T=o["T"],
                                               workspace=ws)
                    q.qlora_linear_bwd_grouped(U["W"], U["g"], U["X"], U["A"], U["B"], U["dY"], o["T"], s,
                                               dX=o["dX"], dA=o["dA"], dB=o["dB"], workspace=ws)
        return step

    def ungrouped_of(layer):
        ws = layer["ws"]

        def step_ungrouped():
            for L in layer["lin"]:
                o = L["out"]
                q.qlora_linear_fwd(L["W"], L["X"], L["A"], L["B"], s, Y=o["Y"], T=o["T"], workspace=ws)
                q.qlora_linear_bwd(L["W"], L["X"], L["A"], L["B"], L["dY"], o["T"], s,
                                   dX=o["dX"], dA=o["dA"], dB=o["dB"], workspace=ws)
        return step_ungrouped

    layer = build_layer(args.config)
    hidden, ffn, lin, units = layer["hidden"], layer["ffn"], layer["lin"], layer["units"]
    step = step_of(layer)
    step_flops = layer["flops"]
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t_step = timed(step, args.steps)
    ms_per_step = 1e3 * t_step / args.steps
    tflops = step_flops * args.steps / t_step / 1e12
    log(f"step: {ms_per_step:.3f} ms, {tflops:.1f} TFLOP/s ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")

    legs = {}
    want = set() if args.legs == "none" else set(args.legs.split(","))

    # ---- the same seven linears run independently (no shared inputs) ---------------------
    if "ungrouped" in want:
        step_ungrouped = ungrouped_of(layer)
        for _ in range(2):
            step_ungrouped()
        reps = max(3, args.steps // 2)
        tu = timed(step_ungrouped, reps) / reps
        legs["ungrouped_7_linears"] = {"ms_per_step": round(tu * 1e3, 4),
                                       "tflops": round(step_flops / tu / 1e12, 2)}
        log(f"ungrouped 7 linears: {tu * 1e3:.3f} ms, {step_flops / tu / 1e12:.1f} TFLOP/s")

    # ---- the other layer shape's step (LLaMA-7B when the headline is 65B-class) --------------
    if "other_layer" in want:
        oc = "7b" if args.config == "65b" else "65b"
        other_layer = build_layer(oc)
        ostep = step_of(other_layer)
        for _ in range(max(1, args.warmup)):
            ostep()
        reps = max(3, args.steps // 2)
        to = timed(ostep, reps) / reps
        legs[f"step_{oc}_layer"] = {"ms_per_step": round(to * 1e3, 4),
                                    "step_tflop": round(other_layer["flops"] / 1e12, 4),
                                    "tflops": round(other_layer["flops"] / to / 1e12, 2),
                                    "frac_of_bf16_peak": round(other_layer["flops"] / to / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"{oc} layer step: {to * 1e3:.3f} ms, {other_layer['flops'] / to / 1e12:.1f} TFLOP/s")
        del other_layer, ostep
        torch.cuda.empty_cache()

    # ---- roofline: the step's dominant kernel, timed alone ---------------------------------
    # Both GEMM orientations of the step (forward with (s T) B^T in the
    # epilogue, input gradient with (s U) A) are the same template kernel with
    # the rank term fused; qlora_4bit_matmul_lora launches exactly that
    # instance. Each is timed over the step's four units with the step's rank
    # widths; the one with the larger total time per step is the roofline.
    roofline = None
    if "roofline" in want:
        reps = max(3, args.steps)
        res = {}
        for orient in ("dx", "fwd"):
            runs = []
            for U in units:
                R = U["g"] * r
                if orient == "dx":    # dX = dY W~ + (s U) [A_1; ..; A_g]: rank g r, reduction over N
                    act, nout, rk = U["dY"], U["K"], R
                    Rm = U["A"].t().contiguous()
                else:                 # Y = X W~^T + (s T) B^T: rank r per output column
                    act, nout, rk = U["X"], U["N"], r
                    Rm = U["B"]
                Lm = synth.device_normal_bf16(M * rk, 0.25, 4_000_000 + 7 * rk + nout, dev).view(M, rk)
                o = torch.empty(M, nout, dtype=torch.bfloat16, device=dev)
                runs.append((U["W"], act, Lm, Rm, o, 2.0 * M * U["N"] * U["K"] + 2.0 * M * nout * rk))

            def one_pass(runs=runs, tr=(orient == "dx")):
                for W_, a_, L_, R_, o_, _ in runs:
                    q.qlora_4bit_matmul_lora(W_, a_, L_, R_, transposed=tr, out=o_)

            one_pass()
            t = timed(one_pass, reps)
            launches = reps * len(runs)
            flops = sum(x[5] for x in runs)
            res[orient] = dict(avg_s=t / launches, launches=launches, flops_per_launch=flops / len(runs),
                               pass_s=t / reps)
            del runs
        dom = max(res, key=lambda k: res[k]["pass_s"])
        other = "fwd" if dom == "dx" else "dx"
        kern = {"dx": GEMM_KERNEL_DX, "fwd": GEMM_KERNEL_FWD}
        R0 = res[dom]
        achieved = R0["flops_per_launch"] / R0["avg_s"] / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": measured_traffic(kern[dom], args.config),
                    "kernel": kern[dom] + (" (input gradient dY W~ + (sU) A, as in the step)" if dom == "dx"
                                           else " (forward X W~^T + (sT) B^T, as in the step)"),
                    "avg_launch_us": round(R0["avg_s"] * 1e6, 2), "launches": R0["launches"],
                    "flops_per_launch": R0["flops_per_launch"]}
        log(f"roofline kernel ({dom}): avg {R0['avg_s'] * 1e6:.1f} us/launch, {achieved:.1f} TFLOP/s")
        R1 = res[other]
        legs[f"gemm_{other}_orientation"] = {
            "kernel": kern[other], "tflops": round(R1["flops_per_launch"] / R1["avg_s"] / 1e12, 2),
            "avg_launch_us": round(R1["avg_s"] * 1e6, 2)}
        log(f"other orientation ({other}): avg {R1['avg_s'] * 1e6:.1f} us/launch, "
            f"{R1['flops_per_launch'] / R1['avg_s'] / 1e12:.1f} TFLOP/s")

    if "copycal" in want:
        # one elementwise pass of exactly 1 GiB in and 1 GiB out (bf16 negation)
        src = torch.zeros(1 << 29, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---- few-token forward (GEMV) and M = 512 ----------------------------------------------
    if "gemv" in want or "gemm512" in want:
        for N in (4096, 11008):
            K = 4096
            wbytes = 0.5 * N * K + N * K / 64 + 4 * N * K / 16384
            nsets = max(2, int(-(-1.0e9 // wbytes)))
            sets = []
            for j in range(nsets):
                w = synth.device_normal_bf16(N * K, 0.02, 50_000 + 97 * j + N, dev).view(N, K)
                sets.append(dict(W=q.quantize_weight(w),
                                 A=synth.device_normal_bf16(r * K, 0.02, 60_000 + j, dev).view(r, K),
                                 B=synth.device_normal_bf16(N * r, 0.02, 70_000 + j, dev).view(N, r)))
                del w
            ms = ([1, 16] if "gemv" in want else []) + ([512] if "gemm512" in want else [])
            for Mg in ms:
                X = synth.device_normal_bf16(Mg * K, 1.0, 80_000 + Mg, dev).view(Mg, K)
                Yo = torch.empty(Mg, N, dtype=torch.bfloat16, device=dev)
                wsg = q.new_workspace(q.qlora_linear_workspace_bytes(Mg, N, K, r), dev)

                def run_all():
                    for S in sets:
                        q.qlora_linear_fwd(S["W"], X, S["A"], S["B"], s, save_T=False, Y=Yo, workspace=wsg)

                run_all()
                reps = 5
                t_eager = timed(run_all, reps) / (reps * nsets)
                # the same chain of calls captured once as a HIP graph and replayed:
                # time per call without the host's launch cost
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    run_all()
                graph.replay()
                per = timed(graph.replay, reps) / (reps * nsets)
                del graph
                byts = wbytes + 2.0 * r * (K + N) + 2.0 * Mg * (K + N)
                fl = 2.0 * Mg * N * K + 2.0 * Mg * r * (K + N)
                key = f"{'gemv' if Mg <= 16 else 'gemm'}_M{Mg}_{N}x{K}"
                legs[key] = {"us_per_call": round(per * 1e6, 2), "GB/s": round(byts / per / 1e9, 1),
                             "hbm_frac": round(byts / per / 1e9 / PEAK_HBM_GBS, 4),
                             "TFLOP/s": round(fl / per / 1e12, 2), "weight_sets": nsets,
                             "timing": "hip graph of the chain of calls",
                             "us_per_call_eager": round(t_eager * 1e6, 2)}
                log(f"{key}: {per * 1e6:.2f} us/call ({t_eager * 1e6:.2f} eager), {byts / per / 1e9:.0f} GB/s")
            del sets
            torch.cuda.empty_cache()

    # ---- few-token forward of the grouped decoder-layer units (one launch per call) ------------
    if "gemv" in want:
        for name, g, Ns in (("qkv", 3, 4096), ("gate_up", 2, 11008)):
            K = 4096
            N = g * Ns
            wbytes = 0.5 * N * K + N * K / 64 + 4 * N * K / 16384
            nsets = max(2, int(-(-1.0e9 // wbytes)))
            sets = []
            for j in range(nsets):
                w = synth.device_normal_bf16(N * K, 0.02, 90_000 + 97 * j + N, dev).view(N, K)
                sets.append(dict(W=q.quantize_weight(w),
                                 A=synth.device_normal_bf16(g * r * K, 0.02, 91_000 + j, dev).view(g * r, K),
                                 B=synth.device_normal_bf16(N * r, 0.02, 92_000 + j, dev).view(N, r)))
                del w
            for Mg in (1, 16):
                X = synth.device_normal_bf16(Mg * K, 1.0, 93_000 + Mg, dev).view(Mg, K)
                Yo = torch.empty(Mg, N, dtype=torch.bfloat16, device=dev)
                wsg = q.new_workspace(q.qlora_linear_grouped_workspace_bytes(Mg, N, K, r, g), dev)

                def run_all():
                    for S in sets:
                        q.qlora_linear_fwd_grouped(S["W"], g, X, S["A"], S["B"], s, save_T=False, Y=Yo,
                                                   workspace=wsg)

                run_all()
                reps = 5
                t_eager = timed(run_all, reps) / (reps * nsets)
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    run_all()
                graph.replay()
                per = timed(graph.replay, reps) / (reps * nsets)
                del graph
                byts = wbytes + 2.0 * r * (g * K + N) + 2.0 * Mg * (K + N)
                fl = 2.0 * Mg * N * K + 2.0 * Mg * r * (g * K + N)
                key = f"gemv_grouped_{name}_M{Mg}_{N}x{K}"
                legs[key] = {"us_per_call": round(per * 1e6, 2), "GB/s": round(byts / per / 1e9, 1),
                             "hbm_frac": round(byts / per / 1e9 / PEAK_HBM_GBS, 4),
                             "TFLOP/s": round(fl / per / 1e12, 2), "weight_sets": nsets,
                             "timing": "hip graph of the chain of calls",
                             "us_per_call_eager": round(t_eager * 1e6, 2)}
                log(f"{key}: {per * 1e6:.2f} us/call ({t_eager * 1e6:.2f} eager), {byts / per / 1e9:.0f} GB/s")
            del sets
            torch.cuda.empty_cache()

    # ---- quantise + dequantise a 65B-class stack --------------------------------------------
    if "quantize" in want:
        per_layer = [(8192, 8192)] * 4 + [(22016, 8192)] * 3
        free, _ = torch.cuda.mem_get_info(dev)
        layer_bytes = sum(N * K for N, K in per_layer) * (2 + 0.5 + 1 / 64) + (64 << 20)
        nl = max(1, min(args.stack_layers, int((free - (24 << 30)) // layer_bytes)))
        log(f"quantize leg: {nl} layers of 65B-class weights")
        stack = []
        for li in range(nl):
            for j, (N, K) in enumerate(per_layer):
                w = synth.device_normal_bf16(N * K, 0.02, 1_000_000 + 10 * li + j, dev)
                nc, nb, ng = q.storage_sizes(N * K)
                stack.append((w, (torch.empty(nc, dtype=torch.uint8, device=dev),
                                  torch.empty(nb, dtype=torch.uint8, device=dev),
                                  torch.empty(ng, dtype=torch.float32, device=dev))))
        params = sum(w.numel() for w, _ in stack)

        def quant_all():
            # one launch per layer (its 7 weights)
            for li in range(0, len(stack), len(per_layer)):
                layer = stack[li:li + len(per_layer)]
                q.qlora_quantize_4bit_batch([w for w, _ in layer], "nf4", True, outs=[o for _, o in layer])

        quant_all()
        t = timed(quant_all, 3)
        per = t / 3
        gbs = params * Q_BYTES_PER_W / per / 1e9
        legs["quantize_65b_stack"] = {"layers": nl, "params": params, "ms_per_pass": round(per * 1e3, 3),
                                      "GB/s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"quantize: {nl} layers, {params / 1e9:.2f}e9 params, {per * 1e3:.2f} ms, {gbs:.0f} GB/s")
        maxn = max(w.numel() for w, _ in stack)
        # the bf16 input is no longer needed: free it before the round trip
        stack = [(None, o, w.numel()) for w, o in stack]
        torch.cuda.empty_cache()
        # outputs rotate over 8 buffers (>= 2.8 GB) so that no output stays in
        # the 256 MB Infinity Cache between reuses: cold GB/s
        bufs = [torch.empty(maxn, dtype=torch.bfloat16, device=dev) for _ in range(8)]

        def deq_all():
            for i, (_, (codes, c2, c1), n) in enumerate(stack):
                q.qlora_dequant(codes, c2, c1, n, torch.bfloat16, out=bufs[i % 8][:n])

        deq_all()
        t = timed(deq_all, 3)
        per = t / 3
        gbs = params * Q_BYTES_PER_W / per / 1e9
        legs["dequant_bf16_65b_stack"] = {"layers": nl, "ms_per_pass": round(per * 1e3, 3),
                                          "GB/s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"dequant bf16: {per * 1e3:.2f} ms, {gbs:.0f} GB/s")
        del stack, bufs
        torch.cuda.empty_cache()

    # ---- the other 4-bit data types and the format without double quantisation ---------------
    if "formats" in want:
        Nf, Kf = 22016, 8192
        w = synth.device_normal_bf16(Nf * Kf, 0.02, 2_000_001, dev).view(Nf, Kf)
        wf = w.float()
        ms2 = float((wf * wf).mean())
        Xg = synth.device_normal_bf16(8192 * 4096, 1.0, 2_000_002, dev).view(8192, 4096)
        wg = synth.device_normal_bf16(4096 * 4096, 0.02, 2_000_003, dev).view(4096, 4096)
        og = torch.empty(8192, 4096, dtype=torch.bfloat16, device=dev)
        fmt = {}
        for cb in ("nf4", "int4", "fp4"):
            for dq in (True, False):
                key = f"{cb}_{'dq' if dq else 'fp32_absmax'}"
                byts_w = 2.0 + 0.5 + ((1.0 / 64 + 4.0 / 16384) if dq else 4.0 / 64)
                nw = Nf * Kf
                W = q.quantize_weight(w, codebook=cb, double_quant=dq)
                tq = timed(lambda: q.quantize_weight(w, codebook=cb, double_quant=dq), 3) / 3
                d16 = torch.empty(Nf, Kf, dtype=torch.bfloat16, device=dev)
                td = timed(lambda: q.qlora_dequant_4bit(W.codes, W.c2, W.c1, nw, cb, dq, torch.bfloat16,
                                                        out=d16.view(-1)), 3) / 3
                d32 = q.dequant_weight(W, torch.float32)
                rel_mse = float(((d32 - wf) ** 2).mean()) / ms2
                del d32, d16
                Wg = q.quantize_weight(wg, codebook=cb, double_quant=dq)
                q.qlora_nf4_matmul(Wg, Xg, False, out=og)
                tg = timed(lambda: q.qlora_nf4_matmul(Wg, Xg, False, out=og), 5) / 5
                fmt[key] = {"quantize_GB/s": round(nw * byts_w / tq / 1e9, 1),
                            "dequant_bf16_GB/s": round(nw * byts_w / td / 1e9, 1),
                            "rel_mse_vs_bf16_weights": round(rel_mse, 6),
                            "bits_per_weight": round(4.0 + (8.0 / 64 + 32.0 / 16384 if dq else 32.0 / 64), 4),
                            "gemm_8192x4096x4096_tflops": round(2.0 * 8192 * 4096 * 4096 / tg / 1e12, 1)}
                log(f"format {key}: {fmt[key]}")
                del W, Wg
        legs["formats_22016x8192"] = fmt
        del w, wf, Xg, wg, og
        torch.cuda.empty_cache()

    # ---- merged deployment weights W~ + s B A of the layer's seven linears ----------------
    if "merge" in want:
        outs = [torch.empty(L["N"], L["K"], dtype=torch.bfloat16, device=dev) for L in lin]

        def merge_all():
            for L, o in zip(lin, outs):
                q.qlora_merge_lora(L["W"], L["A"], L["B"], s, out=o)

        merge_all()
        tm = timed(merge_all, 5) / 5
        nw = sum(L["N"] * L["K"] for L in lin)
        mbytes = nw * (0.5 + 1.0 / 64 + 2.0)  # codes + c2 read, bf16 written (c1, A, B: cache)
        mkey = f"merge_{args.config}_layer"
        legs[mkey] = {"weights": nw, "ms": round(tm * 1e3, 3), "GB/s": round(mbytes / tm / 1e9, 1),
                      "hbm_frac": round(mbytes / tm / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"merge: {legs[mkey]}")
        del outs
        torch.cuda.empty_cache()

    # ---- the adapters' optimizer step, state in HBM or paged out to pinned host memory -------
    if "adamw" in want:
        per_layer = sum(r * (K + N) for _, N, K in synth.llama_linears(4096, 11008))
        n_opt = 32 * per_layer  # the LoRA parameters of a 32-layer 7B model
        p32 = torch.zeros(n_opt, dtype=torch.float32, device=dev)
        p16 = torch.empty(n_opt, dtype=torch.bfloat16, device=dev)
        g = synth.device_normal_bf16(n_opt, 1e-3, 3_000_001, dev)
        m_d = torch.zeros(n_opt, dtype=torch.float32, device=dev)
        v_d = torch.zeros(n_opt, dtype=torch.float32, device=dev)
        byts = 28.0 * n_opt  # p32 r/w, m r/w, v r/w, bf16 grad, bf16 copy
        q.qlora_adamw_step(p32, g, m_d, v_d, 1, p16=p16)
        stepno = [1]

        def opt_dev():
            stepno[0] += 1
            q.qlora_adamw_step(p32, g, m_d, v_d, stepno[0], p16=p16)

        td = timed(opt_dev, 5) / 5
        m_h = torch.zeros(n_opt, dtype=torch.float32).pin_memory()
        v_h = torch.zeros(n_opt, dtype=torch.float32).pin_memory()

        def page_out():
            m_h.copy_(m_d, non_blocking=True)
            v_h.copy_(v_d, non_blocking=True)

        def page_in():
            m_d.copy_(m_h, non_blocking=True)
            v_d.copy_(v_h, non_blocking=True)

        tout = timed(page_out, 2) / 2
        tin = timed(page_in, 2) / 2

        def opt_host():
            stepno[0] += 1
            q.qlora_adamw_step(p32, g, m_h, v_h, stepno[0], p16=p16)

        opt_host()
        th = timed(opt_host, 2) / 2
        legs["adamw_7b_adapters"] = {
            "params": n_opt, "bytes_per_param": 28,
            "state_in_hbm_ms": round(td * 1e3, 3), "state_in_hbm_GB/s": round(byts / td / 1e9, 1),
            "state_in_hbm_hbm_frac": round(byts / td / 1e9 / PEAK_HBM_GBS, 4),
            "state_in_pinned_host_ms": round(th * 1e3, 3),
            "state_in_pinned_host_link_GB/s": round(16.0 * n_opt / th / 1e9, 1),
            "page_out_ms": round(tout * 1e3, 3), "page_in_ms": round(tin * 1e3, 3),
            "page_GB/s": round(8.0 * n_opt / ((tout + tin) / 2) / 1e9, 1)}
        log(f"adamw: {legs['adamw_7b_adapters']}")
        del p32, p16, g, m_d, v_d, m_h, v_h
        torch.cuda.empty_cache()

    # ---- CPU oracle on a bounded sample of the step ---------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds, log)

    line = {
        "metric": "NF4-LoRA linear fwd+bwd TFLOP/s (% bf16 peak); quantize/GEMV HBM GB/s (%)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": ("LLaMA-7B-shaped decoder layer (weights N(0, 0.02))" if args.config == "7b"
                                else "65B-class decoder layer (hidden 8192, FFN 22016, weights 0.02 Student-t(5))")
                   + ": 7 NF4+DQ linears (q,k,v,o,gate,up,down), LoRA r=64 alpha=16 on each, "
                   "q/k/v and gate/up on shared inputs (grouped), 8192 tokens, forward + backward (dX, dA, dB)",
                   "hidden": hidden, "ffn": ffn, "tokens": M, "lora_r": r, "lora_alpha": alpha,
                   "step_tflop": round(step_flops / 1e12, 4), "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "legs": legs,
    }
    print(json.dumps(line), flush=True)


def measured_traffic(kernel, config):
    """HBM bytes per launch of the roofline kernel from the counter runs kept in
    profiles/ (pmc_traffic.py), if they were taken on this kernel, this layer
    and the current GEMM source; else None."""
    try:
        from bit_nf4_quantized_12_amd import pmc_traffic
        with open(pmc_traffic.traffic_file(config)) as fh:
            rec = json.load(fh)
        if rec.get("gemm_source_sha256") != pmc_traffic.gemm_source_sha() or rec.get("kernel") != kernel:
            return None
        return round(rec["traffic_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(target_s, log):
    """Time the float64 oracle (dequantise + forward + backward) on a sample of the
    step: one 8192 x 8192 linear of the 65B-class layer (r = 64, Student-t weights)
    for a doubling number of tokens until about target_s / 4 of CPU time."""
    import numpy as np

    import oracle
    from bit_nf4_quantized_12_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:
        blas = None
    ncpu = os.cpu_count() or 1
    N = K = 8192
    r, s = 64, 16.0 / 64
    case = synth.linear_case(1, N, K, r, seed=0, cfg=4, w_dist="student_t")
    w32 = case["W"][1]
    pk, c2, c1 = oracle.quantize_nf4_dq(w32)   # the stored weight (load time, not timed)

    def work(m):
        g = np.random.default_rng(m)
        X = g.standard_normal((m, K)).astype(np.float32)
        dY = g.standard_normal((m, N)).astype(np.float32)
        t0 = time.perf_counter()
        Wt = oracle.bf16_round(oracle.dequant(pk, c2, c1, N * K)).reshape(N, K)
        oracle.linear_fwd(X, Wt, case["A"][1], case["B"][1], s)
        oracle.linear_bwd(X, Wt, case["A"][1], case["B"][1], dY, s)
        return time.perf_counter() - t0

    m = 256
    t = work(m)
    while t < target_s / 4 and m < 65536:
        m *= 2
        t = work(m)
    flops = 4.0 * m * N * K + 6.0 * m * r * (K + N)
    used = blas if blas is not None else ncpu
    log(f"cpu oracle: {m} tokens of one 8192x8192 linear in {t:.2f} s; {ncpu} host CPUs, "
        f"BLAS threads {blas}")
    return {"value": round(flops / t / 1e12, 5), "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "host_cpu_count": ncpu, "blas_threads": blas,
            "sample": f"oracle dequant + fwd + bwd of one 8192x8192 NF4+DQ linear of the 65B-class layer "
                      f"(r=64, Student-t weights) for {m} tokens ({flops / 1e9:.1f} GFLOP in {t:.2f} s); "
                      f"the matrix products run on {blas} BLAS threads, dequantisation on one"}


if __name__ == "__main__":
    main()
