"""Benchmark of the block-scaled MoE hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|verify|prefill]
                    [--no-cpu-baseline] [--no-prefill]

A step is one pass of the whole hot path over one batch of synthetic input:
top-k gate + bucketing (moe_route), the routed-expert FFN with its combine
(moe_expert_ffn) and, for the decode workloads, the dense block-32 FP8
projection (fp8_block_gemm, M = rows, K = N = 4096).  Inputs are resident in
HBM before timing starts.  Weights rotate over R distinct copies so that the
bytes a step touches are never served by the 256 MB MALL or the L2s.

Default workload "decode": one token, hidden 4096, 256 experts, top-8,
intermediate 576 (MXFP4 experts, FP8 block-32 activations), plus the dense
projection at M = 1.  value = algorithmic bytes per step / step time (GB/s).
Unless --no-prefill, the line also carries the 8192-token prefill layer's
expert-GEMM throughput (TFLOP/s) measured in the same run.

Prints ONE JSON line.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_FP8_PEAK_TFLOPS = 5000.0  # dense FP8 matrix rate (the FP8 x FP4 MFMA issues at this rate)
MFMA_FP4_PEAK_TFLOPS = 10100.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix rate (router logits)

EXPERT_BYTES = lambda H, I: 2 * I * (H // 2 + H // 32) + H * (I // 2 + I // 32)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sources_hash():
    """Hash of the library's code: every file under csrc/ with its comments
    removed and its whitespace collapsed, so that a comment-only edit keeps
    the profiles taken on the same code valid."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp8xfp4_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode() + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources_sha") != kernel_sources_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=["decode", "verify", "prefill"], default="decode")
    ap.add_argument("--rotate", type=int, default=0, help="weight copies (0 = enough to exceed 1.5 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-verify", action="store_true", help="decode line without the verification-batch object")
    ap.add_argument("--no-layer-shared", action="store_true",
                    help="decode line without the routed + shared expert layer object")
    ap.add_argument("--graph", action="store_true", help="replay one HIP graph per step instead of eager launches")
    ap.add_argument("--graph-steps", type=int, default=1,
                    help="with --graph: decode steps captured per graph (a multi-layer decode graph)")
    ap.add_argument("--unfused", action="store_true",
                    help="decode step at T=1: moe_route + moe_expert_ffn instead of moe_layer_decode1")
    ap.add_argument("--prefetch", action="store_true",
                    help="decode step: prefetch the dense projection's weights on a side stream from the step's start")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 256 MiB buffer 5 times (reference kernel for the HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "copies": 5}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode "
              "(the layer shards by rows or by the intermediate dimension; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from block_scaled_fp8xfp4_amd import mxmoe, synth
    from block_scaled_fp8xfp4_amd.layer import ExpertFFN, Route, quantize, quantize_experts

    mxmoe.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    result = {}

    def dense_layer(cfg):
        d = synth.dense_inputs()
        w = torch.from_numpy(d.w).to(dev)
        wq, wsc = quantize(w, mxmoe.MX_FMT_E4M3)
        del w
        return d, wq, wsc

    def moe_layer(cfg):
        inp = synth.moe_inputs(cfg)
        t0 = time.time()
        w13q, w13s = quantize_experts(inp.w13())
        w2q, w2s = quantize_experts(inp.w2())
        log(f"{cfg.name}: generated and quantized the expert weights in {time.time() - t0:.1f} s")
        x = torch.from_numpy(inp.x).to(dev).to(torch.bfloat16)
        xq, xsc = quantize(x, mxmoe.MX_FMT_E4M3)
        return inp, xq, xsc, (w13q, w13s, w2q, w2s)

    # ------------------------------------------------------------ decode step
    def run_decode(cfg):
        inp, xq, xsc, W = moe_layer(cfg)
        T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
        dense, gq, gsc = dense_layer(synth.DENSE)
        a = torch.from_numpy(dense.a[:T] if T <= dense.a.shape[0] else np.resize(dense.a, (T, dense.cfg.K)))
        aq, asc = quantize(a.to(dev).to(torch.bfloat16).contiguous(), mxmoe.MX_FMT_E4M3)
        logits = torch.from_numpy(inp.logits).to(dev)
        surv = None if inp.survival is None else torch.from_numpy(inp.survival).to(dev)
        route = Route(T, E, k)
        ffn = ExpertFFN(T, H, E, I, k)
        yg = torch.empty((T, dense.cfg.N), dtype=torch.bfloat16, device=dev)
        # bytes one step streams: touched experts, activations, logits, outputs, dense weights
        route(logits, surv)
        torch.cuda.synchronize()
        offs = route.offsets.cpu().numpy()
        touched = int(np.count_nonzero(np.diff(offs)))
        all_ids = np.unique(route.ids.cpu().numpy())
        moe_bytes = touched * EXPERT_BYTES(H, I) + T * (H + H // 32) + T * E * 4 + T * H * 4
        dense_bytes = dense.cfg.N * (dense.cfg.K + dense.cfg.K // 32) + T * (dense.cfg.K + dense.cfg.K // 32) \
            + T * dense.cfg.N * 2
        step_bytes = moe_bytes + dense_bytes
        per_copy = touched * EXPERT_BYTES(H, I) + dense_bytes
        R = args.rotate or max(2, int(np.ceil(1.5e9 / per_copy)))
        log(f"{cfg.name}: touched experts {touched} (all slots {len(all_ids)}), bytes/step {step_bytes}, "
            f"rotating {R} weight copies")
        copies = [W] + [tuple(t.clone() for t in W) for _ in range(R - 1)]
        gcopies = [(gq, gsc)] + [(gq.clone(), gsc.clone()) for _ in range(R - 1)]
        torch.cuda.synchronize()

        fused = T == 1 and not args.unfused
        side = torch.cuda.Stream() if args.prefetch else None     # default priority
        main = torch.cuda.current_stream()

        def step(i):
            w13q, w13s, w2q, w2s = copies[i % R]
            g, gs = gcopies[i % R]
            if side is not None:
                # the dense weights stream into cache (each 16-row slice into the
                # L2 of the XCD whose workgroup will read it) while route and FFN run
                side.wait_stream(main)
                with torch.cuda.stream(side):
                    mxmoe.prefetch(g, 16 * dense.cfg.K)
                    mxmoe.prefetch(gs, 16 * (dense.cfg.K // 32))
            if fused:
                # one row: the gate runs inside the gate/up kernel (moe_layer_decode1)
                mxmoe.moe_layer_decode1(logits, k, surv, 0.2, xq, xsc, w13q, w13s, w2q, w2s, E, I, route.ids,
                                        route.w, route.offsets, route.perm, route.slot_pos, ffn.y, ffn.ws)
            else:
                route(logits, surv)
                ffn(xq, xsc, route, w13q, w13s, w2q, w2s)
            mxmoe.fp8_block_gemm(aq, asc, g, gs, yg, mxmoe.MX_OUT_BF16)
            if side is not None:
                main.wait_stream(side)

        route(logits, surv)
        ffn(xq, xsc, route, *copies[0])
        ffn_variant = mxmoe.last_variant()
        step(0)
        step_variant = "moe_layer_decode1 + fp8_block_gemm" if fused else "moe_route + moe_expert_ffn + fp8_block_gemm"
        torch.cuda.synchronize()
        if not args.graph:
            run_step = step
        else:
            # HIP graphs of G consecutive steps (each on its own weight copy),
            # as a serving loop replays its decode step (G > 1: several layers
            # in one graph); the library allocates and syncs nothing
            G = max(1, args.graph_steps)
            if args.steps % G or args.warmup % G:
                sys.exit("--steps and --warmup must be multiples of --graph-steps")
            ng = max(1, R // G)
            graphs = []
            for gi in range(ng):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    for u in range(G):
                        step(gi * G + u)
                graphs.append(gr)
            torch.cuda.synchronize()

            def run_step(i):
                if i % G == 0:
                    graphs[(i // G) % ng].replay()
        for i in range(args.warmup):
            run_step(i)
        torch.cuda.synchronize()
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_start.record()
        for i in range(args.steps):
            run_step(i)
        t_end.record()
        torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
        # the FFN call alone: R back-to-back calls over the weight copies (one
        # graph, or eager), bracketed by events on the launch stream
        def ffn_calls():
            for i in range(R):
                if fused:
                    mxmoe.moe_layer_decode1(logits, k, surv, 0.2, xq, xsc, *copies[i % R], E, I, route.ids, route.w,
                                            route.offsets, route.perm, route.slot_pos, ffn.y, ffn.ws)
                else:
                    ffn(xq, xsc, route, *copies[i % R])
        if not args.graph:
            run_ffn = ffn_calls
        else:
            gffn = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gffn):
                ffn_calls()
            run_ffn = gffn.replay
        run_ffn()
        torch.cuda.synchronize()
        reps = max(1, args.steps // R)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        for _ in range(reps):
            run_ffn()
        f1.record()
        torch.cuda.synchronize()
        ffn_ms = f0.elapsed_time(f1) / (reps * R)
        ms = total_ms / args.steps
        ffn_bytes = touched * EXPERT_BYTES(H, I) + T * (H + H // 32) + T * H * 4 + (T * E * 4 if fused else 0)
        achieved = ffn_bytes / (ffn_ms * 1e-3) / 1e9
        if fused:
            ffn_variant = mxmoe.last_variant()          # the last host call was moe_layer_decode1
        if cfg.streams:
            # the same step with router-live verification rows: rows below the
            # confidence threshold take their anchor's experts instead of skipping
            thr = 0.1
            anchor = torch.from_numpy((np.arange(T) // (cfg.drafts + 1) * (cfg.drafts + 1)).astype(np.int32)).to(dev)
            route(logits, surv, thr, anchor=anchor)
            live_variant = mxmoe.last_variant()
            torch.cuda.synchronize()
            touched_l = int(np.count_nonzero(np.diff(route.offsets.cpu().numpy())))
            reusing = int(np.sum((inp.survival < np.float32(thr)) & (np.arange(T) % (cfg.drafts + 1) != 0)))

            def step_live(i):
                w13q, w13s, w2q, w2s = copies[i % R]
                route(logits, surv, thr, anchor=anchor)
                ffn(xq, xsc, route, w13q, w13s, w2q, w2s)
                g, gs = gcopies[i % R]
                mxmoe.fp8_block_gemm(aq, asc, g, gs, yg, mxmoe.MX_OUT_BF16)

            for i in range(args.warmup):
                step_live(i)
            torch.cuda.synchronize()
            l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            l0.record()
            for i in range(args.steps):
                step_live(i)
            l1.record()
            torch.cuda.synchronize()
            live_ms = l0.elapsed_time(l1) / args.steps
            live_bytes = touched_l * EXPERT_BYTES(H, I) + T * (H + H // 32) + T * E * 4 + T * H * 4 + dense_bytes
            live_obj = {"reuse_below": thr, "rows_reusing": reusing, "pairs": T * k,
                                     "touched_experts": touched_l, "ms_per_step": round(live_ms, 5),
                                     "gbs": round(live_bytes / (live_ms * 1e-3) / 1e9, 2),
                                     "variant": live_variant}
            route(logits, surv)                                  # back to the skip-mode routing
        out = {
            "metric": "decode weight-stream GB/s (% HBM peak) + prefill expert TFLOP/s (% MFMA peak)",
            "value": round(step_bytes / (ms * 1e-3) / 1e9, 2),
            "unit": "GB/s",
            "ms_per_step": round(ms, 5),
            "pct_hbm_peak": round(100 * step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "roofline": {"bound": "hbm", "kernel": ("moe_layer_decode1 (" if fused else "moe_expert_ffn (") + ffn_variant + ")",
                         "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(cfg.name),
                         "bytes_per_launch": ffn_bytes, "avg_launch_ms": round(ffn_ms, 5)},
            "config": {"workload": f"{cfg.name} MoE layer step: T={T}, H={H}, E={E}, top-{k}, I={I}, MXFP4 experts, "
                                   f"FP8 block-32 activations, + dense FP8 block-32 projection M={T}, K=N=4096",
                       "rows": T, "hidden": H, "experts": E, "top_k": k, "intermediate": I,
                       "touched_experts": touched, "experts_of_all_rows": len(all_ids),
                       "weight_bytes_skipped": (len(all_ids) - touched) * EXPERT_BYTES(H, I),
                       "bytes_per_step": step_bytes, "weight_copies": R,
                       "launch": (f"hip_graph_{args.graph_steps}_steps" if args.graph else "eager"), "step_calls": step_variant,
                       "prefetch": bool(args.prefetch)},
        }
        if cfg.streams:
            out["router_live"] = live_obj
        if fused and not args.graph and not args.no_layer_shared:
            out["layer_with_shared"] = run_layer_with_shared(cfg, xq, xsc, logits, surv, copies, route, ffn,
                                                             ffn_bytes)
        return inp, touched, out

    def run_layer_with_shared(cfg, xq, xsc, logits, surv, copies, route, ffn, routed_bytes):
        """The row's whole MoE layer, routed + shared experts: moe_layer_decode1_shared
        (two launches) against moe_layer_decode1 + moe_shared_expert (four), each
        over the same rotated routed weight copies and as many shared copies."""
        H, E, k, I = cfg.H, cfg.E, cfg.k, cfg.I
        w13, w2 = synth.shared_expert_weights(cfg)
        S = quantize(torch.from_numpy(w13).to(dev), mxmoe.MX_FMT_E4M3) + \
            quantize(torch.from_numpy(w2).to(dev), mxmoe.MX_FMT_E4M3)
        sbytes = sum(t.numel() for t in S)
        R = len(copies)
        scopies = [S] + [tuple(t.clone() for t in S) for _ in range(R - 1)]
        ys = torch.empty((1, H), dtype=torch.float32, device=dev)
        ws_s = torch.empty(mxmoe.moe_shared_expert_workspace_bytes(1, H, I), dtype=torch.uint8, device=dev)
        ws_f = torch.empty(mxmoe.moe_layer_decode1_shared_workspace_bytes(H, E, I, k, I), dtype=torch.uint8,
                           device=dev)
        r = route

        def separate(i):
            mxmoe.moe_layer_decode1(logits, k, surv, 0.2, xq, xsc, *copies[i % R], E, I, r.ids, r.w, r.offsets,
                                    r.perm, r.slot_pos, ffn.y, ffn.ws)
            mxmoe.moe_shared_expert(xq, xsc, *scopies[i % R], ys, ws_s)

        def fused_call(i):
            mxmoe.moe_layer_decode1_shared(logits, k, surv, 0.2, xq, xsc, *copies[i % R], E, I, *scopies[i % R],
                                           r.ids, r.w, r.offsets, r.perm, r.slot_pos, ffn.y, ys, ws_f)

        def timed(fn):
            for i in range(R):
                fn(i)
            torch.cuda.synchronize()
            reps = max(1, args.steps // R)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                for i in range(R):
                    fn(i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / (reps * R)

        sep_ms = timed(separate)
        fus_ms = timed(fused_call)
        variant = mxmoe.last_variant()
        nbytes = routed_bytes + sbytes + H * 4                 # + the shared weights and y_shared
        return {"shared_I": I, "shared_weight_bytes": sbytes, "bytes": nbytes, "ms": round(fus_ms, 5),
                "gbs": round(nbytes / (fus_ms * 1e-3) / 1e9, 2),
                "pct_hbm_peak": round(100 * nbytes / (fus_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "separate_calls_ms": round(sep_ms, 5), "variant": variant,
                "separate_calls": "moe_layer_decode1 + moe_shared_expert"}

    # ------------------------------------------------------------ dense FP8 GEMM at decode sizes (M = 1, 16)
    def run_dense_decode(steps, warmup):
        """fp8_block_gemm of the dense config alone (M = 1 and 16 drawn rows, K = N = 4096,
        bf16 out), over 64 weight copies (1.1 GB) so that every call streams from HBM; the 64
        calls are replayed from one HIP graph, so host launch cost does not set the rate."""
        d = synth.dense_inputs()
        _, wq, wsc = dense_layer(synth.DENSE)
        out = {}
        R = 64
        copies = [(wq, wsc)] + [(wq.clone(), wsc.clone()) for _ in range(R - 1)]
        for M in d.cfg.M:
            aq, asc = quantize(torch.from_numpy(d.a[:M]).to(dev).to(torch.bfloat16).contiguous(), mxmoe.MX_FMT_E4M3)
            yd = torch.empty((M, d.cfg.N), dtype=torch.bfloat16, device=dev)
            mxmoe.fp8_block_gemm(aq, asc, *copies[0], yd, mxmoe.MX_OUT_BF16)
            variant = mxmoe.last_variant()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for i in range(R):
                    mxmoe.fp8_block_gemm(aq, asc, *copies[i], yd, mxmoe.MX_OUT_BF16)
            for _ in range(max(1, warmup // R)):
                gr.replay()
            torch.cuda.synchronize()
            reps = max(1, steps // R)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                gr.replay()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / (reps * R)
            nbytes = d.cfg.N * (d.cfg.K + d.cfg.K // 32) + M * (d.cfg.K + d.cfg.K // 32) + M * d.cfg.N * 2
            out[f"M{M}"] = dict(ms=round(ms, 5), gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                                pct_hbm_peak=round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                                bytes=nbytes, variant=variant, launch="hip_graph")
            del gr
        del copies
        return out

    # ------------------------------------------------------------ dense FP8 GEMM at prefill size
    def run_dense_prefill(M, steps, warmup):
        """fp8_block_gemm with the chunk's rows (M = T) through the dense 4096 x 4096
        projection: synthetic N(0,1) activations, the dense config's weights, bf16 out."""
        d = synth.dense_inputs()
        _, wq, wsc = dense_layer(synth.DENSE)
        K, N = d.cfg.K, d.cfg.N
        g = torch.Generator(device="cpu").manual_seed(5)
        a = torch.randn((M, K), generator=g).to(dev).to(torch.bfloat16)
        aq, asc = quantize(a, mxmoe.MX_FMT_E4M3)
        del a
        yd = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        copies = [(wq, wsc), (wq.clone(), wsc.clone())]
        for i in range(warmup):
            mxmoe.fp8_block_gemm(aq, asc, *copies[i % 2], yd, mxmoe.MX_OUT_BF16)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            mxmoe.fp8_block_gemm(aq, asc, *copies[i % 2], yd, mxmoe.MX_OUT_BF16)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        flop = 2 * M * N * K
        return dict(M=M, N=N, K=K, ms=round(ms, 4), tflops=round(flop / (ms * 1e-3) / 1e12, 2),
                    pct_fp8_peak=round(100 * flop / (ms * 1e-3) / 1e12 / MFMA_FP8_PEAK_TFLOPS, 2),
                    variant=mxmoe.last_variant())

    # ------------------------------------------------------------ router logits (the gate's input side)
    def run_router_logits(cfg, inp, steps, warmup):
        """moe_router_logits on the workload's bf16 hidden rows and a synthetic
        bf16 gate [E][H]; the gate is rotated over enough copies to leave the
        caches for the row counts of a decode step."""
        from block_scaled_fp8xfp4_amd.layer import RouterLogits
        T, H, E = cfg.T, cfg.H, cfg.E
        hid = torch.from_numpy(inp.x).to(dev).to(torch.bfloat16)
        gate = torch.from_numpy(synth.router_gate(cfg)).to(dev).to(torch.bfloat16)
        R = 2 if T >= 1024 else 256                              # 256 x 2 MB gates > the 256 MB MALL
        gates = [gate] + [gate.clone() for _ in range(R - 1)]
        out = torch.empty((T, E), dtype=torch.float32, device=dev)
        rl = RouterLogits(T, H, E)
        for i in range(warmup):
            rl(hid, gates[i % R], out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            rl(hid, gates[i % R], out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        nbytes, flop = E * H * 2 + T * H * 2 + T * E * 4, 2 * T * H * E
        return dict(T=T, H=H, E=E, ms=round(ms, 5), gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                    pct_hbm_peak=round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                    tflops=round(flop / (ms * 1e-3) / 1e12, 2),
                    pct_bf16_peak=round(100 * flop / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2),
                    bytes=nbytes, flop=flop, variant=mxmoe.last_variant(), gate_copies=R)

    # ------------------------------------------------------------ shared expert
    def run_shared_expert(cfg, inp, steps, warmup):
        """moe_shared_expert (FP8 gate/up [2I][H], SwiGLU + requant, FP8 down [H][I],
        K = I = 576 unpadded) on the layer's own rows, with enough weight copies
        to leave the caches at decode sizes."""
        T, H, I = cfg.T, cfg.H, cfg.I
        x = torch.from_numpy(inp.x).to(dev).to(torch.bfloat16)
        xq, xsc = quantize(x, mxmoe.MX_FMT_E4M3)
        w13, w2 = synth.shared_expert_weights(cfg)
        W = quantize(torch.from_numpy(w13).to(dev), mxmoe.MX_FMT_E4M3) + \
            quantize(torch.from_numpy(w2).to(dev), mxmoe.MX_FMT_E4M3)
        wbytes = sum(t.numel() for t in W)
        R = 2 if T >= 1024 else max(2, int(np.ceil(1.0e9 / wbytes)))
        copies = [W] + [tuple(t.clone() for t in W) for _ in range(R - 1)]
        y = torch.empty((T, H), dtype=torch.float32, device=dev)
        ws = torch.empty(mxmoe.moe_shared_expert_workspace_bytes(T, H, I), dtype=torch.uint8, device=dev)
        for i in range(warmup):
            mxmoe.moe_shared_expert(xq, xsc, *copies[i % R], y, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            mxmoe.moe_shared_expert(xq, xsc, *copies[i % R], y, ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        nbytes = wbytes + T * (H + H // 32) + T * H * 4
        flop = 2 * T * (2 * I) * H + 2 * T * H * I
        return dict(T=T, H=H, I=I, ms=round(ms, 5), gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                    pct_hbm_peak=round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                    tflops=round(flop / (ms * 1e-3) / 1e12, 2),
                    pct_fp8_peak=round(100 * flop / (ms * 1e-3) / 1e12 / MFMA_FP8_PEAK_TFLOPS, 2),
                    bytes=nbytes, flop=flop, weight_copies=R, variant=mxmoe.last_variant())

    # ------------------------------------------------------------ prefill
    def run_prefill(steps, warmup):
        cfg = synth.PREFILL
        inp, xq, xsc, W = moe_layer(cfg)
        T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
        logits = torch.from_numpy(inp.logits).to(dev)
        route = Route(T, E, k)
        ffn = ExpertFFN(T, H, E, I, k)
        copies = [W, tuple(t.clone() for t in W)]
        for i in range(warmup):
            route(logits)
            ffn(xq, xsc, route, *copies[i % 2])
        torch.cuda.synchronize()
        # the library records four events per call on its stream: before the
        # first kernel, after gate/up, after the down projection, after the combine
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for i in range(steps):
            route(logits)
            mxmoe.set_phase_events(ev[i])
            ffn(xq, xsc, route, *copies[i % 2])
        t1.record()
        mxmoe.set_phase_events(None)
        torch.cuda.synchronize()
        ffn_variant = mxmoe.last_variant()
        ph = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in ev])   # ms per phase
        gu_ms, dn_ms, cb_ms = (float(np.mean(ph[:, j])) for j in range(3))
        ffn_ms = float(np.mean(ph.sum(axis=1)))
        P = int(route.offsets[-1].item())
        flop_gu, flop_dn = P * 2 * 2 * I * H, P * 2 * H * I
        flop = flop_gu + flop_dn
        tf = lambda f, ms: f / (ms * 1e-3) / 1e12
        combine_bytes = P * H * 4 + T * H * 4 + T * k * 8
        dense = run_dense_prefill(T, steps, warmup)
        router = run_router_logits(cfg, inp, steps, warmup)
        shared = run_shared_expert(cfg, inp, steps, warmup)
        return dict(router_logits=router, shared_expert=shared, tflops=round(tf(flop, ffn_ms), 2), pct_fp8_peak=round(100 * tf(flop, ffn_ms) / MFMA_FP8_PEAK_TFLOPS, 2),
                    dense_gemm=dense,
                    expert_gemms_tflops=round(tf(flop, gu_ms + dn_ms), 2),
                    expert_gemms_pct_fp8_peak=round(100 * tf(flop, gu_ms + dn_ms) / MFMA_FP8_PEAK_TFLOPS, 2),
                    expert_gemms_pct_fp4_peak=round(100 * tf(flop, gu_ms + dn_ms) / MFMA_FP4_PEAK_TFLOPS, 2),
                    gate_up_ms=round(gu_ms, 4), gate_up_tflops=round(tf(flop_gu, gu_ms), 2),
                    down_ms=round(dn_ms, 4), down_tflops=round(tf(flop_dn, dn_ms), 2),
                    combine_ms=round(cb_ms, 4), combine_gbs=round(combine_bytes / (cb_ms * 1e-3) / 1e9, 1),
                    ffn_ms=round(ffn_ms, 4), step_ms=round(t0.elapsed_time(t1) / steps, 4), flop_per_call=flop,
                    flop_gate_up=flop_gu, variant=ffn_variant, pairs=P), inp

    if args.workload == "prefill":
        pre, inp = run_prefill(args.steps, args.warmup)
        result.update({
            "metric": "decode weight-stream GB/s (% HBM peak) + prefill expert TFLOP/s (% MFMA peak)",
            "value": pre["tflops"], "unit": "TFLOP/s", "ms_per_step": pre["step_ms"],
            "roofline": {"bound": "mfma", "kernel": "gu_prefill (gate/up expert GEMM, the call's dominant kernel)",
                         "achieved": pre["gate_up_tflops"], "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(pre["gate_up_tflops"] / MFMA_FP8_PEAK_TFLOPS, 4),
                         "traffic": recorded_traffic("prefill"),
                         "flop_per_launch": pre["flop_gate_up"], "avg_launch_ms": pre["gate_up_ms"]},
            "phases": {k: pre[k] for k in ("gate_up_ms", "gate_up_tflops", "down_ms", "down_tflops", "combine_ms",
                                           "combine_gbs", "expert_gemms_tflops", "expert_gemms_pct_fp8_peak",
                                           "expert_gemms_pct_fp4_peak", "ffn_ms")},
            "dense_gemm": pre["dense_gemm"],
            "router_logits": pre["router_logits"],
            "shared_expert": pre["shared_expert"],
            "config": {"workload": "prefill MoE chunk: T=8192, H=4096, E=256, top-8, I=576, MXFP4 experts, "
                                   "FP8 block-32 activations", "pairs": pre["pairs"]},
        })
        cpu_cfg = synth.PREFILL
    else:
        cfg = synth.DECODE if args.workload == "decode" else synth.VERIFY
        inp, touched, main_line = run_decode(cfg)
        result.update(main_line)
        if args.workload == "decode" and not args.no_verify:
            # the speculative-verification batch (48 rows = 8 streams x (anchor + 5
            # drafts), Zipf(1.1) expert popularity, rows with survival < 0.2 skip
            # the routed experts): GB/s over the experts the live rows touch
            _, _, v = run_decode(synth.VERIFY)
            c = v["config"]
            result["verify"] = {
                "workload": c["workload"], "gbs": v["value"], "pct_hbm_peak": v["pct_hbm_peak"],
                "ms_per_step": v["ms_per_step"], "bytes_per_step": c["bytes_per_step"],
                "touched_experts": c["touched_experts"], "experts_of_all_rows": c["experts_of_all_rows"],
                "weight_bytes_skipped": c["weight_bytes_skipped"], "roofline": v["roofline"],
                "router_live": v.get("router_live")}
        result["dense_decode"] = run_dense_decode(args.steps, args.warmup)
        result["router_logits"] = run_router_logits(cfg, inp, args.steps, args.warmup)
        result["shared_expert"] = run_shared_expert(cfg, inp, args.steps, args.warmup)
        cpu_cfg = cfg
        if not args.no_prefill:
            torch.cuda.synchronize()
            torch.cuda.empty_cache()                           # the decode weight copies go back to the device
            pre, _ = run_prefill(20, 5)
            result["prefill"] = pre

    result.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                   "scaling": "weak", "vs_baseline": None, "dtype": "fp8xfp4->f32", "data": "synthetic"})

    # ------------------------------------------------------------ CPU baseline: the oracle itself
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cpu_cfg, args.workload)
    print(json.dumps(result), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, workload):
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the same workload (same shapes and distributions)."""
    import oracle
    from block_scaled_fp8xfp4_amd import synth

    # the host's cores, capped by the CPU share this process has on the machine
    # (OMP_NUM_THREADS when set, as on a shared GPU host: 16 cores per GPU)
    hw = oracle.hardware_threads()
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(hw, share) if share > 0 else hw
    inp = synth.moe_inputs(cfg)
    r = oracle.route(inp.logits, cfg.k, inp.survival)
    rows = np.arange(min(cfg.T, 4 if workload == "prefill" else cfg.T), dtype=np.int32)
    need = np.unique(r["ids"][rows][r["live"][rows].astype(bool)])
    H, I, E = cfg.H, cfg.I, cfg.E
    w13 = np.zeros((E, 2 * I, H // 2), np.uint8)
    w13s = np.full((E, 2 * I, H // 32), 127, np.uint8)
    w2 = np.zeros((E, H, I // 2), np.uint8)
    w2s = np.full((E, H, I // 32), 127, np.uint8)
    q, s = oracle.quantize_e2m1(inp.w13(need).reshape(-1, H), threads)
    w13[need], w13s[need] = q.reshape(len(need), 2 * I, H // 2), s.reshape(len(need), 2 * I, H // 32)
    q, s = oracle.quantize_e2m1(inp.w2(need).reshape(-1, I), threads)
    w2[need], w2s[need] = q.reshape(len(need), H, I // 2), s.reshape(len(need), H, I // 32)
    xq, xs = oracle.quantize_e4m3(inp.x, threads)
    d = synth.dense_inputs()
    aq, asc = oracle.quantize_e4m3(d.a[:1], threads)
    wq, wsc = oracle.quantize_e4m3(d.w, threads)
    live_pairs = int(r["live"][rows].sum()) * cfg.k
    t0 = time.time()
    reps = 0
    while True:
        oracle.route(inp.logits[rows], cfg.k, None if inp.survival is None else inp.survival[rows])
        oracle.moe_rows(xq, xs, r["ids"], r["w"], r["live"], w13, w13s, w2, w2s, rows=rows, threads=threads)
        if workload != "prefill":
            oracle.block_gemm(aq, asc, wq, wsc, threads=threads)
        reps += 1
        if time.time() - t0 > 10.0 or reps >= 2000:
            break
    dt = (time.time() - t0) / reps
    if workload == "prefill":
        flop = live_pairs * (2 * 2 * I * H + 2 * H * I)
        return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "host_cores": hw,
                "cpu_model": cpu_model(), "kind": "oracle",
                "sample": f"{len(rows)} of {cfg.T} prefill rows ({live_pairs} routed pairs), {reps} reps, "
                          f"{dt:.2f} s per rep"}
    touched = len(need)
    step_bytes = touched * EXPERT_BYTES(H, I) + len(rows) * (H + H // 32) + len(rows) * E * 4 \
        + len(rows) * H * 4 + d.cfg.N * (d.cfg.K + d.cfg.K // 32) + (d.cfg.K + d.cfg.K // 32) + d.cfg.N * 2
    return {"value": round(step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "host_cores": hw,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"the full {workload} step ({len(rows)} rows, {touched} experts, dense M=1), {reps} reps, "
                      f"{dt:.3f} s per rep"}


if __name__ == "__main__":
    main()
