#!/usr/bin/env python3
"""Decode benchmark of the 30-layer int4 MoE stack with a 16-slot LFU expert
cache per layer, B=1, on one MI355X.

One step = one token through all layers of the stack (per layer: routing,
LFU lookup, host->HBM copies of the missing experts on a side stream
overlapped with the shared-expert gate/up GEMV, routed gate/up GEMVs with
GeGLU, down GEMVs with the weighted combine and the residual). Inputs are
seeded and synthetic (no trained weights); the experts of all layers sit in
pinned host memory, the slot pools, routers and shared experts in HBM.

Prints one JSON line (rank 0). Besides the headline tokens/s it reports the
HBM roofline of the dominant kernel (routed-expert gate/up GEMV; bytes per
launch / mean event-timed duration), the same stack with every expert
resident in HBM (replayed from a HIP graph), and the fp64 oracle timed on
host cores over a bounded sample of (token, layer) units.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE decode tokens/s (B=1, 30 layers) + achieved HBM GB/s on expert bytes"
HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=448, help="timed tokens")
    ap.add_argument("--warmup", type=int, default=64, help="untimed tokens before the timed ones")
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--tokens", type=int, default=512, help="distinct seeded input tokens")
    ap.add_argument("--slots", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget")
    ap.add_argument("--no-resident", action="store_true", help="skip the all-resident variant")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import ctypes as C

    import numpy as np
    import torch

    from bit_quantized_expert_softmax_amd import api
    from synth import gen
    from synth.configs import C2

    sh = C2.shape
    H, E, k, I, Is = sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter
    Lyr, T, S = args.layers, args.tokens, args.slots
    cid = C2.config_id
    devn = "cuda:0"
    torch.cuda.set_device(0)
    lib = api.lib()
    blob = gen.blob_bytes(H, I)
    flags = api.MOE_F_RMSNORM_IN | api.MOE_F_RESIDUAL

    # ---------------------------------------------------------------- inputs
    t_gen = time.perf_counter()
    layers = []
    for l in range(Lyr):
        host = torch.empty((E, blob), dtype=torch.uint8, pin_memory=True)
        gen.expert_blobs(sh, cid, l, out=host.numpy())
        d = {
            "router_np": gen.router(sh, cid, l),
            "bias_np": gen.zipf_bias(E, cid, l),
            "shared_np": gen.shared_blob(sh, cid, l),
            "host": host,
        }
        d["router"] = torch.from_numpy(d["router_np"].view(np.int16)).to(devn)
        d["bias"] = torch.from_numpy(d["bias_np"]).to(devn)
        d["shared"] = torch.from_numpy(d["shared_np"]).to(devn)
        d["pool"] = torch.empty((S, blob), dtype=torch.uint8, device=devn)
        d["ws"] = torch.zeros(api.moe_layer_workspace_bytes(sh, 1, 0), dtype=torch.uint8, device=devn)
        layers.append(d)
    x_np = gen.x_fp32(T, H, cid)
    eps_np = gen.eps_fp16(Lyr, T, H, cid)
    x = torch.from_numpy(x_np).to(devn)
    eps = torch.from_numpy(eps_np.view(np.int16)).to(devn)
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    copy_stream = torch.cuda.Stream()
    main_stream = torch.cuda.current_stream()
    sp = main_stream.cuda_stream
    for d in layers:
        d["h"] = api.moe_layer_create(sh, router=d["router"], shared_blob=d["shared"], workspace=d["ws"],
                                      bias=d["bias"], experts_host=d["host"], slot_pool=d["pool"],
                                      n_slots=S, copy_stream=copy_stream)
    hbuf = [torch.empty((1, H), device=devn) for _ in range(2)]
    hp = [b.data_ptr() for b in hbuf]
    xp0, ep0 = x.data_ptr(), eps.data_ptr()
    stats = [api.moe_decode_stats() for _ in range(Lyr)]
    decode = lib.moe_layer_decode

    def token(t, handles, st=None):
        tt = t % T
        src = xp0 + tt * H * 4
        for l in range(Lyr):
            dst = hp[l & 1]
            rc = decode(handles[l], src, ep0 + (l * T + tt) * H * 2, 1, flags, dst, None, None, None,
                        None, None if st is None else C.byref(st[l]), sp)
            if rc:
                raise api.MoeError(rc, "moe_layer_decode", api.moe_last_error())
            src = dst

    handles = [d["h"] for d in layers]
    for t in range(args.warmup):
        token(t, handles, stats)
    torch.cuda.synchronize()
    warm = [(s.hits, s.misses, s.h2d_bytes) for s in stats]
    for d in layers:
        api.moe_layer_profile(d["h"], True)
    print("[bench] warmup done, timing the cache-mode stack", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.warmup, args.warmup + args.steps):
        token(t, handles, stats)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    for d in layers:
        api.moe_layer_profile(d["h"], False)
    tok_s = args.steps / el
    hits = sum(s.hits - w[0] for s, w in zip(stats, warm))
    misses = sum(s.misses - w[1] for s, w in zip(stats, warm))
    h2d = sum(s.h2d_bytes - w[2] for s, w in zip(stats, warm))
    kinds = {}
    for kind in range(4):
        n = ms = 0
        for d in layers:
            a, b = api.moe_layer_profile_read(d["h"], kind)
            n += a
            ms += b
        kinds[kind] = (n, ms)

    # routed-expert gate/up launch: k experts x (gate + up) rows, nibbles + fp16 scales,
    # plus the fp32 input vector read and the fp32 activations written
    gu_bytes = k * 2 * I * (H // 2 + 2 * (H // 32)) + H * 4 + k * I * 4
    down_bytes = H * (k * (I // 2 + 2 * (I // 32)) + Is // 2 + 2 * (Is // 32)) + (k * I + Is) * 4 + H * 4 * 2
    n_gu, ms_gu = kinds[2]
    us_gu = 1e3 * ms_gu / max(n_gu, 1)
    gbps_gu = gu_bytes / (us_gu * 1e-6) / 1e9
    n_dn, ms_dn = kinds[3]
    us_dn = 1e3 * ms_dn / max(n_dn, 1)
    detail = {
        "hit_rate_timed": hits / max(hits + misses, 1),
        "h2d_MB_per_token": h2d / args.steps / 1e6,
        "h2d_GBps_wall": h2d / el / 1e9,
        "kernel_us": {
            "route": 1e3 * kinds[0][1] / max(kinds[0][0], 1),
            "shared_gateup": 1e3 * kinds[1][1] / max(kinds[1][0], 1),
            "routed_gateup": us_gu,
            "down_combine": us_dn,
        },
        "down_combine_GBps": down_bytes / (us_dn * 1e-6) / 1e9 if us_dn > 0 else None,
    }

    # ---------------------------------------------------------------- all experts resident
    if not args.no_resident:
        res = []
        for d in layers:
            d["experts_dev"] = d["host"].to(devn, non_blocking=False)
            d["ws_r"] = torch.zeros_like(d["ws"])
            res.append(api.moe_layer_create(sh, router=d["router"], shared_blob=d["shared"],
                                            workspace=d["ws_r"], bias=d["bias"],
                                            experts_dev=d["experts_dev"]))
        x_in = torch.empty((1, H), device=devn)
        e_in = torch.empty((Lyr, 1, H), dtype=torch.int16, device=devn)
        cap = torch.cuda.Stream()

        def step_resident():
            s = torch.cuda.current_stream().cuda_stream
            src = x_in.data_ptr()
            for l in range(Lyr):
                dst = hp[l & 1]
                rc = decode(res[l], src, e_in.data_ptr() + l * H * 2, 1, flags, dst, None, None, None,
                            None, None, s)
                if rc:
                    raise api.MoeError(rc, "moe_layer_decode", api.moe_last_error())
                src = dst
        with torch.cuda.stream(cap):
            x_in.copy_(x[0:1])
            e_in.copy_(eps[:, 0:1])
            step_resident()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step_resident()
        torch.cuda.synchronize()
        for t in range(args.warmup):
            x_in.copy_(x[t % T:t % T + 1])
            e_in.copy_(eps[:, t % T:t % T + 1])
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(args.warmup, args.warmup + args.steps):
            x_in.copy_(x[t % T:t % T + 1])
            e_in.copy_(eps[:, t % T:t % T + 1])
            g.replay()
        torch.cuda.synchronize()
        el_r = time.perf_counter() - t0
        detail["resident_tokens_per_s"] = args.steps / el_r
        per_tok = Lyr * (k * blob + gen.blob_bytes(H, Is) + E * H * 2)
        detail["resident_layer_GBps"] = per_tok * args.steps / el_r / 1e9
        # eager pass with per-kernel events for the resident kernels
        for h in res:
            api.moe_layer_profile(h, True)
        for t in range(min(args.steps, 64)):
            x_in.copy_(x[t % T:t % T + 1])
            e_in.copy_(eps[:, t % T:t % T + 1])
            step_resident()
        torch.cuda.synchronize()
        n = ms = 0
        for h in res:
            a, b = api.moe_layer_profile_read(h, 2)
            n += a
            ms += b
        us_r = 1e3 * ms / max(n, 1)
        gu_res = gu_bytes + 2 * Is * (H // 2 + 2 * (H // 32)) + Is * 4
        detail["resident_gateup_us"] = us_r
        detail["resident_gateup_GBps"] = gu_res / (us_r * 1e-6) / 1e9
        for h in res:
            api.moe_layer_destroy(h)

        # batched decode (B tokens per step, grouped by expert) and 2048-token
        # prefill on one layer of the same shape, unbiased routing
        d0 = layers[0]
        for B in (16, 64):
            wsb = torch.zeros(api.moe_layer_workspace_bytes(sh, B, 0), dtype=torch.uint8, device=devn)
            hb = api.moe_layer_create(sh, router=d0["router"], shared_blob=d0["shared"], workspace=wsb,
                                      experts_dev=d0["experts_dev"], max_B=B)
            xb = torch.from_numpy(gen.x_fp32(B * 8, H, 3, sub=B)).to(devn)
            yb = torch.empty((B, H), device=devn)
            idsb = torch.empty((B, k), dtype=torch.int32, device=devn)

            def bstep(i):
                api.moe_layer_decode(hb, xb[(i % 8) * B:(i % 8 + 1) * B], None, B, 0, yb, idsb)
            for i in range(5):
                bstep(i)
            torch.cuda.synchronize()
            n_it = 40
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            touched = 0
            for i in range(n_it):
                bstep(i)
            ev1.record()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / n_it
            for i in range(8):
                bstep(i)
                touched += len(np.unique(idsb.cpu().numpy()))
            step_bytes = touched / 8 * blob + gen.blob_bytes(H, Is) + E * H * 2
            detail[f"batched_B{B}"] = {"tokens_per_s": B / (ms * 1e-3), "ms_per_step": ms,
                                       "distinct_experts": touched / 8,
                                       "GBps": step_bytes / (ms * 1e-3) / 1e9}
            api.moe_layer_destroy(hb)
            del wsb
        Tp = 2048
        wsp = torch.zeros(api.moe_layer_workspace_bytes(sh, 1, Tp), dtype=torch.uint8, device=devn)
        hp_ = api.moe_layer_create(sh, router=d0["router"], shared_blob=d0["shared"], workspace=wsp,
                                   experts_dev=d0["experts_dev"], max_T=Tp)
        xp = torch.from_numpy(gen.x_bf16(Tp, H, 4).view(np.int16)).to(devn)
        lp = torch.from_numpy(gen.logits_uniform(Tp, E, 4)).to(devn)
        yp = torch.empty((Tp, H), device=devn)
        for i in range(3):
            api.moe_layer_prefill(hp_, xp, lp, Tp, yp)
        torch.cuda.synchronize()
        n_it = 10
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(n_it):
            api.moe_layer_prefill(hp_, xp, lp, Tp, yp)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / n_it
        flops = 2.0 * Tp * (k * 3 * H * I + 3 * H * Is)
        detail["prefill_2048"] = {"ms": ms, "TFLOPs": flops / (ms * 1e-3) / 1e12,
                                  "mfma_bf16_frac": flops / (ms * 1e-3) / 2.5e15, "GFLOP": flops / 1e9}
        api.moe_layer_destroy(hp_)
        del wsp
        for d in layers:
            del d["experts_dev"]

    # ---------------------------------------------------------------- oracle on host cores
    cpu = None
    if not args.no_cpu:
        from threadpoolctl import threadpool_info

        from oracle import moe as omoe
        units = 0
        t0 = time.perf_counter()
        rng = np.random.default_rng(0)
        while time.perf_counter() - t0 < args.cpu_seconds:
            t = int(rng.integers(0, T))
            l = int(rng.integers(0, Lyr))
            d = layers[l]
            lay = {"router": d["router_np"], "bias": d["bias_np"], "shared": d["shared_np"],
                   "experts": d["host"].numpy()}
            omoe.stack_layer_step(x_np[t], eps_np[l, t], sh, lay)
            units += 1
        el_c = time.perf_counter() - t0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        cpu = {"value": units / el_c / Lyr, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{units} random (token, layer) units of the 30-layer stack at full shape, "
                         f"fp64 numpy, {el_c:.1f}s; tokens/s = units/s / {Lyr}"}

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * el / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights x 16-bit fixed-point activations -> int32, fp32 scale/accumulate",
        "data": "synthetic (seeded; no trained weights)",
        "config": {"workload": C2.name, "layers": Lyr, "hidden": H, "experts": E, "top_k": k,
                   "inter": I, "shared_inter": Is, "slots_per_layer": S, "batch": 1,
                   "expert_store": "pinned host memory", "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": gbps_gu, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps_gu / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "k_ffn_gateup (routed experts)", "bytes_per_launch": gu_bytes,
                     "mean_us": us_gu, "launches": n_gu},
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(out), flush=True)
    for d in layers:
        api.moe_layer_destroy(d["h"])


if __name__ == "__main__":
    main()
