#!/usr/bin/env python3
"""Decode benchmark of the 30-layer int4 MoE stack with a 16-slot LFU expert
cache per layer, B=1, on one MI355X.

One step = one token through all layers of the stack (per layer: routing,
LFU lookup, host->HBM copies of the missing experts overlapped with the
shared-expert gate/up GEMV -- by hipMemcpyAsync on a side stream, or with
--fill kernel by fill blocks of the shared-expert launch --, routed gate/up
GEMVs with GeGLU, down GEMVs with the weighted combine and the residual). The
fill variant not chosen is timed afterwards and reported in detail. Inputs are
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
    ap.add_argument("--fill", choices=["kernel", "copy-engine"], default="copy-engine",
                    help="how the timed (headline) run fills cache misses; the other way is "
                         "timed afterwards and reported in detail")
    ap.add_argument("--no-variant", action="store_true", help="skip the other fill variant")
    ap.add_argument("--no-file-store", action="store_true",
                    help="skip the variant whose misses are read from an expert file with parallel pread")
    ap.add_argument("--store-threads", type=int, default=8, help="reader threads of the expert file store")
    ap.add_argument("--store-tokens", type=int, default=48, help="tokens timed with the expert file store")
    ap.add_argument("--sweep-slots", default="8,32,64",
                    help="slot counts per layer for the cache-size sweep in the detail ('' to skip)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--attn-ctx", type=int, default=4096,
                    help="context length of the attention step timed next to the MoE layers")
    ap.add_argument("--no-attn", action="store_true", help="skip the attention-step measurements")
    ap.add_argument("--no-device-cache", action="store_true",
                    help="skip the stack with the slot caches stepped on the device")
    ap.add_argument("--probe", choices=["gateup", "copy", "batched", "prefill"], default=None,
                    help="short run for hardware counters: 'gateup' decodes a few cache-mode "
                         "tokens (the measured kernel included), 'copy' copies 1 GiB once")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("GU_FETCH", "GU_WRITE", "CP_FETCH", "CP_WRITE"),
                    help="turn four rocprofv3 --pmc output folders (FETCH_SIZE / WRITE_SIZE of a "
                         "'--probe gateup' and a '--probe copy' run) into the traffic summary (JSON)")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="turn a rocprofv3 --kernel-trace run of this benchmark into the routed gate/up's "
                         "kernel-trace summary (JSON, written to profiles/)")
    ap.add_argument("--summarize-kernels", metavar="TRACE_DIR",
                    help="per-kernel table (markdown) of a rocprofv3 --kernel-trace run: calls, mean and "
                         "median duration and share of the GPU time, by kernel and launch size")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="turn a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE run of "
                         "'--probe prefill' into a per-kernel MFMA-busy table (markdown)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_gateup_routed_gemma_layer.json")
TRACE_FILE = os.path.join(ROOT, "profiles", "trace_k_gateup_routed_gemma_layer.json")
# sources that define the measured kernel: the summary is void once one changes
KERNEL_SOURCES = ["bit_quantized_expert_softmax_amd/csrc/decode.hip",
                  "bit_quantized_expert_softmax_amd/csrc/device_common.h",
                  "bit_quantized_expert_softmax_amd/csrc/launch.h"]
COPY_BYTES = 1 << 30
PROFILE_EVERY = 8


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# lanes per block of the routed gate/up launch (8 waves; launches that carry a
# top-k use 1024)
GU_ROUTED_THREADS = 512


def routed_gateup_grid(sh):
    """Launch size (work-items) of the routed gate/up kernel at B=1."""
    return sh.top_k * (sh.inter // 32) * GU_ROUTED_THREADS


def summarize_pmc(dirs):
    """Per-dispatch HBM bytes of the routed gate/up kernel from FETCH_SIZE and
    WRITE_SIZE, each scaled by the same counter's reading for a plain copy of
    COPY_BYTES (so the counters' unit and coverage cancel out)."""
    import csv
    import glob

    from synth.configs import C2

    def rows(d):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    grid = routed_gateup_grid(C2.shape)

    def kernel_avg(d, counter):
        v = [float(r["Counter_Value"]) for r in rows(d)
             if r["Counter_Name"] == counter and "k_gateup" in r["Kernel_Name"] and int(r["Grid_Size"]) == grid]
        return sum(v) / len(v), len(v)

    def copy_max(d, counter):
        # the 1 GiB copy is the largest dispatch of the probe
        return max(float(r["Counter_Value"]) for r in rows(d) if r["Counter_Name"] == counter)

    f_kib, nf = kernel_avg(dirs[0], "FETCH_SIZE")
    w_kib, nw = kernel_avg(dirs[1], "WRITE_SIZE")
    cf = COPY_BYTES / copy_max(dirs[2], "FETCH_SIZE")
    cw = COPY_BYTES / copy_max(dirs[3], "WRITE_SIZE")
    return {"kernel": "k_gateup (routed experts, cache mode)", "grid": grid,
            "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
            "dispatches": [nf, nw], "copy_bytes_per_fetch_unit": cf, "copy_bytes_per_write_unit": cw,
            "fetch_bytes": f_kib * cf, "write_bytes": w_kib * cw,
            "traffic_bytes": f_kib * cf + w_kib * cw, "source_hash": kernel_source_hash(),
            "commands": [
                "rocprofv3 --pmc FETCH_SIZE --output-format csv -d " + dirs[0] + " -o run -- "
                "python -u bench.py --probe gateup --warmup 8",
                "rocprofv3 --pmc WRITE_SIZE --output-format csv -d " + dirs[1] + " -o run -- "
                "python -u bench.py --probe gateup --warmup 8",
                "rocprofv3 --pmc FETCH_SIZE --output-format csv -d " + dirs[2] + " -o run -- "
                "python -u bench.py --probe copy",
                "rocprofv3 --pmc WRITE_SIZE --output-format csv -d " + dirs[3] + " -o run -- "
                "python -u bench.py --probe copy",
                "python bench.py --summarize-pmc " + " ".join(dirs)],
            "note": "FETCH_SIZE / WRITE_SIZE (KiB units) of the routed gate/up launches (176 x 512), each "
                    "scaled by the bytes per unit the same counter reads for a plain 1 GiB device copy; "
                    "algorithmic bytes per launch 17,875,968"}


# ---------------------------------------------------------------- CPU baseline workers
# The oracle timed on the host: each spawned worker (no GPU use) builds one
# layer of the stack from the seeded generators, then runs random teacher-
# forced (token, layer) units of it for a fixed wall time with one BLAS
# thread; the units are independent, so the workers together use the cores.
_CPU = {}


def _cpu_init(counter, layers, tokens, cid):
    import numpy as np
    from threadpoolctl import threadpool_limits

    from synth import gen
    from synth.configs import C2
    with counter.get_lock():
        idx = counter.value
        counter.value += 1
    sh = C2.shape
    l = idx % layers
    _CPU["lim"] = threadpool_limits(1)
    _CPU["sh"] = sh
    _CPU["lay"] = {"router": gen.router(sh, cid, l), "bias": gen.zipf_bias(sh.n_experts, cid, l),
                   "shared": gen.shared_blob(sh, cid, l), "experts": gen.expert_blobs(sh, cid, l)}
    _CPU["x"] = gen.x_fp32(tokens, sh.hidden, cid)
    _CPU["eps"] = np.ascontiguousarray(gen.eps_fp16(layers, tokens, sh.hidden, cid)[l])
    _CPU["idx"] = idx


def _cpu_run(args):
    import numpy as np

    from oracle import moe as omoe
    seconds, seed = args
    rng = np.random.default_rng(seed)
    t0 = time.time()
    units = 0
    while time.time() - t0 < seconds:
        t = int(rng.integers(0, _CPU["x"].shape[0]))
        omoe.stack_layer_step(_CPU["x"][t], _CPU["eps"][t], _CPU["sh"], _CPU["lay"])
        units += 1
    return t0, time.time(), units


def cpu_baseline(layers, tokens, cid, seconds):
    """fp64 oracle rate in tokens/s on a pool of host cores (at most 16)."""
    import multiprocessing as mp
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    workers = max(1, min(16, avail))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    ctx = mp.get_context("spawn")
    counter = ctx.Value("i", 0)
    with ctx.Pool(workers, initializer=_cpu_init, initargs=(counter, layers, tokens, cid)) as pool:
        # one untimed unit per worker first, so every worker has built its layer
        pool.map(_cpu_run, [(0.0, i) for i in range(workers)], chunksize=1)
        res = pool.map(_cpu_run, [(seconds, 100 + i) for i in range(workers)], chunksize=1)
    units = sum(r[2] for r in res)
    wall = max(r[1] for r in res) - min(r[0] for r in res)
    return {"value": units / wall / layers, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{units} random teacher-forced (token, layer) units of the {layers}-layer stack at full "
                      f"shape, fp64 numpy, on {workers} worker processes with one BLAS thread each "
                      f"({avail} cores available, os.cpu_count() = {os.cpu_count()}, CPU: {model}), "
                      f"{wall:.1f}s wall; tokens/s = units/s / {layers}",
            "cpu_model": model}


def summarize_kernels(d, top=60):
    import csv
    import glob
    from collections import defaultdict
    acc = defaultdict(list)
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"].replace("void ", "").replace("moe::(anonymous namespace)::", "").split("(")[0]
            wg = int(r.get("Workgroup_Size_X", 0) or 0)
            blocks = int(r.get("Grid_Size_X", 0) or 0) // max(wg, 1)
            acc[(name, blocks, wg)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in acc.values())
    lines = ["| kernel | blocks x threads | calls | mean µs | median µs | share |", "|---|---|---|---|---|---|"]
    for (name, blocks, wg), v in sorted(acc.items(), key=lambda kv: -sum(kv[1]))[:top]:
        v = sorted(v)
        lines.append(f"| `{name}` | {blocks} x {wg} | {len(v)} | {sum(v) / len(v):.2f} | {v[len(v) // 2]:.2f} | "
                     f"{100 * sum(v) / total:.1f}% |")
    return "\n".join(lines)


def summarize_mfma(d):
    """MFMA-busy share per prefill kernel: SQ_VALU_MFMA_BUSY_CYCLES summed over
    the SIMDs / (GPU-busy cycles of one XCD x 1024 SIMDs), the MfmaUtil formula
    of rocprofv3's derived counters (GRBM_GUI_ACTIVE is summed over the 8 XCDs,
    so its per-XCD value is the sum / 8)."""
    import csv
    import glob
    from collections import defaultdict
    acc = defaultdict(lambda: defaultdict(list))
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"].replace("void ", "").replace("moe::(anonymous namespace)::", "").split("(")[0]
            key = (name, int(r["Grid_Size"]) // int(r["Workgroup_Size"]), int(r["Workgroup_Size"]),
                   r.get("VGPR_Count", ""), r.get("Accum_VGPR_Count", ""))
            acc[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = ["| kernel | blocks x threads | VGPR (arch + acc) | dispatches | GPU-busy us (one XCD at 2.4 GHz) | MFMA busy |",
             "|---|---|---|---|---|---|"]
    for (name, blocks, wg, vg, ag), c in sorted(acc.items(), key=lambda kv: -sum(kv[1].get("SQ_VALU_MFMA_BUSY_CYCLES", [0]))):
        mf = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        gr = c.get("GRBM_GUI_ACTIVE")
        if not mf or not gr or sum(mf) == 0:
            continue
        n = len(mf)
        per_xcd = sum(gr) / len(gr) / 8
        util = (sum(mf) / n) / (per_xcd * 1024)
        lines.append(f"| `{name}` | {blocks} x {wg} | {vg} + {ag} | {n} | {per_xcd / 2400:.1f} | {util:.3f} |")
    return "\n".join(lines)


def summarize_trace(d):
    """Mean and median duration (kernel trace: dispatch begin to end) of the
    routed gate/up launches that cover all 8 routed experts (176 x 512)."""
    import csv
    import glob

    from synth.configs import C2
    grid = routed_gateup_grid(C2.shape)
    durs = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if "k_gateup" in r["Kernel_Name"] and "false" in r["Kernel_Name"] and \
                    int(r.get("Grid_Size_X", r.get("Grid_Size", 0))) == grid:
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    durs.sort()
    return {"kernel": "k_gateup (routed experts, cache mode)", "grid": grid, "launches": len(durs),
            "mean_us": sum(durs) / len(durs), "median_us": durs[len(durs) // 2],
            "source_hash": kernel_source_hash(),
            "command": "rocprofv3 --kernel-trace --stats --output-format csv -d " + d +
                       " -o run -- python -u bench.py --steps 24 --warmup 8 --no-cpu --no-file-store",
            "note": "kernel-trace durations of the launches of the benchmark's measured kernel"}


def load_trace():
    """The committed kernel-trace summary if it was taken on the current kernel source."""
    try:
        with open(TRACE_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    return t if t.get("source_hash") == kernel_source_hash() else None


def load_traffic():
    """The committed counter summary if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    return t if t.get("source_hash") == kernel_source_hash() else None


def main():
    args = parse()
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(args.summarize_pmc), indent=1))
        return
    if args.summarize_trace:
        t = summarize_trace(args.summarize_trace)
        with open(TRACE_FILE, "w") as fh:
            json.dump(t, fh, indent=1)
        print(json.dumps(t, indent=1))
        return
    if args.summarize_kernels:
        print(summarize_kernels(args.summarize_kernels))
        return
    if args.summarize_mfma:
        print(summarize_mfma(args.summarize_mfma))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import ctypes as C

    import numpy as np
    import torch

    from bit_quantized_expert_softmax_amd import _lib, api
    from synth import gen
    from synth.configs import C2, GEMMA_ATTN

    if args.probe == "copy":
        a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
        b = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
        torch.cuda.synchronize()
        a.copy_(b)
        torch.cuda.synchronize()
        print(f"[bench] copied {COPY_BYTES} bytes", file=sys.stderr, flush=True)
        return
    sh = C2.shape
    H, E, k, I, Is = sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter
    if args.probe == "batched":
        # batched decode at B = 64 over 4 resident layers in turn (1.7 GB of
        # experts, so no step finds its weights in the last-level cache), for
        # counter runs of the matrix-core kernels
        devb, Bp = "cuda:0", 64
        hb, keep = [], []
        wsb = torch.zeros(api.moe_layer_workspace_bytes(sh, Bp, 0), dtype=torch.uint8, device=devb)
        for l in range(4):
            ex = torch.from_numpy(gen.expert_blobs(sh, C2.config_id, l)).to(devb)
            rt = torch.from_numpy(gen.router(sh, C2.config_id, l).view(np.int16)).to(devb)
            shb = torch.from_numpy(gen.shared_blob(sh, C2.config_id, l)).to(devb)
            keep += [ex, rt, shb]
            hb.append(api.moe_layer_create(sh, router=rt, shared_blob=shb, workspace=wsb, experts_dev=ex, max_B=Bp))
        xb = torch.from_numpy(gen.x_fp32(Bp, H, 3, sub=Bp)).to(devb)
        yb = torch.empty((Bp, H), device=devb)
        for i in range(4 * args.warmup):
            api.moe_layer_decode(hb[i % 4], xb, None, Bp, 0, yb)
        torch.cuda.synchronize()
        for h in hb:
            api.moe_layer_destroy(h)
        print(f"[bench] probe: {4 * args.warmup} batched steps at B = {Bp}", file=sys.stderr, flush=True)
        return
    if args.probe == "prefill":
        # 2048-token prefills over 3 resident layers in turn, for counter runs
        # of the matrix-core GEMMs
        devp, Tp = "cuda:0", 2048
        wsp = torch.zeros(api.moe_layer_workspace_bytes(sh, 1, Tp), dtype=torch.uint8, device=devp)
        hp_, keep = [], []
        for l in range(3):
            ex = torch.from_numpy(gen.expert_blobs(sh, C2.config_id, l)).to(devp)
            rt = torch.from_numpy(gen.router(sh, C2.config_id, l).view(np.int16)).to(devp)
            shb = torch.from_numpy(gen.shared_blob(sh, C2.config_id, l)).to(devp)
            keep += [ex, rt, shb]
            hp_.append(api.moe_layer_create(sh, router=rt, shared_blob=shb, workspace=wsp, experts_dev=ex, max_T=Tp))
        xq = torch.from_numpy(gen.x_bf16(Tp, H, 4).view(np.int16)).to(devp)
        lq = torch.from_numpy(gen.logits_uniform(Tp, E, 4)).to(devp)
        yq = torch.empty((Tp, H), device=devp)
        for i in range(args.warmup):
            api.moe_layer_prefill(hp_[i % 3], xq, lq, Tp, yq)
        torch.cuda.synchronize()
        for h in hp_:
            api.moe_layer_destroy(h)
        print(f"[bench] probe: {args.warmup} prefills of {Tp} tokens", file=sys.stderr, flush=True)
        return
    Lyr, T, S = args.layers, args.tokens, args.slots
    cid = C2.config_id
    devn = "cuda:0"
    torch.cuda.set_device(0)
    lib = api.lib()
    blob = gen.blob_bytes(H, I)
    flags_base = api.MOE_F_RMSNORM_IN | api.MOE_F_RESIDUAL
    fill_flag = {"kernel": api.MOE_F_FILL_KERNEL, "copy-engine": 0}
    flags = flags_base | fill_flag[args.fill]

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
    if args.probe == "gateup":
        print(f"[bench] probe: {args.warmup} cache-mode tokens decoded", file=sys.stderr, flush=True)
        for d in layers:
            api.moe_layer_destroy(d["h"])
        return
    warm = [(s.hits, s.misses, s.h2d_bytes) for s in stats]
    # only the measured kernel (routed gate/up, kind 2) is timed during the
    # timed region, on one token in PROFILE_EVERY, with its events created
    # beforehand (timing every launch costs the stack about 10%)
    for d in layers:
        api.moe_layer_profile_kinds(d["h"], 1 << 2, PROFILE_EVERY, 2 * args.steps // PROFILE_EVERY + 16)
    print("[bench] warmup done, timing the cache-mode stack", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.warmup, args.warmup + args.steps):
        token(t, handles, stats)
    torch.cuda.synchronize()
    el_head = time.perf_counter() - t0
    for d in layers:
        api.moe_layer_profile(d["h"], False)
    tok_s = args.steps / el_head
    hits = sum(s.hits - w[0] for s, w in zip(stats, warm))
    misses = sum(s.misses - w[1] for s, w in zip(stats, warm))
    h2d = sum(s.h2d_bytes - w[2] for s, w in zip(stats, warm))
    # per-stage times of all kinds come from a short profiled pass afterwards
    # (out of the timed region: events around every stage slow the stack)
    n_gu, ms_gu = 0, 0.0
    for d in layers:
        a, b = api.moe_layer_profile_read(d["h"], 2)
        n_gu += a
        ms_gu += b
        api.moe_layer_profile(d["h"], True)
    for t in range(args.warmup + args.steps, args.warmup + args.steps + 16):
        token(t, handles, None)
    torch.cuda.synchronize()
    for d in layers:
        api.moe_layer_profile(d["h"], False)
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
    us_gu = 1e3 * ms_gu / max(n_gu, 1)
    gbps_gu = gu_bytes / (us_gu * 1e-6) / 1e9
    n_dn, ms_dn = kinds[3]
    us_dn = 1e3 * ms_dn / max(n_dn, 1)
    detail = {
        "hit_rate_timed": hits / max(hits + misses, 1),
        "h2d_MB_per_token": h2d / args.steps / 1e6,
        "h2d_GBps_wall": h2d / el_head / 1e9,
        "kernel_us": {
            "route": 1e3 * kinds[0][1] / max(kinds[0][0], 1),
            "shared_gateup": 1e3 * kinds[1][1] / max(kinds[1][0], 1),
            "routed_gateup": us_gu,
            "down_combine": us_dn,
        },
        "down_combine_GBps": down_bytes / (us_dn * 1e-6) / 1e9 if us_dn > 0 else None,
    }

    # ---------------------------------------------------------------- stage times
    # A few more tokens with MOE_F_STAGE_TIMES (each call then waits for its
    # own work, so this pass is slower than the headline): per layer call the
    # routing latency until the ids are on the host, the misses' copy time,
    # the compute stream's wait for the copies and the call's GPU time.
    st_t = api.moe_decode_stats()
    acc = {"route": 0.0, "fill": 0.0, "wait": 0.0, "total": 0.0, "calls": 0, "miss_calls": 0, "misses": 0}
    t_base = args.warmup + args.steps + 16
    for t in range(t_base, t_base + 8):
        tt = t % T
        src = xp0 + tt * H * 4
        for l in range(Lyr):
            dst = hp[l & 1]
            m0 = st_t.misses
            rc = decode(handles[l], src, ep0 + (l * T + tt) * H * 2, 1, flags | api.MOE_F_STAGE_TIMES, dst, None,
                        None, None, None, C.byref(st_t), sp)
            if rc:
                raise api.MoeError(rc, "moe_layer_decode", api.moe_last_error())
            src = dst
            nm = st_t.misses - m0
            acc["route"] += st_t.ms_route
            acc["wait"] += st_t.ms_wait_fill
            acc["total"] += st_t.ms_total
            acc["calls"] += 1
            if nm:
                acc["fill"] += st_t.ms_fill
                acc["miss_calls"] += 1
                acc["misses"] += nm
    torch.cuda.synchronize()
    detail["stage_times_ms"] = {
        "route_to_host_per_layer": acc["route"] / acc["calls"],
        "fill_per_layer_with_misses": acc["fill"] / max(acc["miss_calls"], 1),
        "fill_per_missed_expert": acc["fill"] / max(acc["misses"], 1),
        "wait_fill_per_layer": acc["wait"] / acc["calls"],
        "gpu_per_layer": acc["total"] / acc["calls"],
        "layer_calls": acc["calls"], "misses": acc["misses"],
        "note": "MOE_F_STAGE_TIMES pass of 8 tokens after the timed region (each call synchronises)"}

    # ---------------------------------------------------------------- link-bound ceiling
    # The copy engines alone: 8 expert blobs from pinned host memory to HBM,
    # alternating over two streams as the decode does, repeated; the stack
    # cannot beat H2D bytes per token / this rate.
    cp_dst = torch.empty((8, blob), dtype=torch.uint8, device=devn)
    cp_s2 = torch.cuda.Stream()
    hsrc = layers[0]["host"]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_rep = 12
    for r in range(n_rep):
        for j in range(8):
            st_ = copy_stream if j % 2 == 0 else cp_s2
            with torch.cuda.stream(st_):
                cp_dst[j].copy_(hsrc[(8 * r + j) % E], non_blocking=True)
    torch.cuda.synchronize()
    el_cp = time.perf_counter() - t0
    copy_gbps = n_rep * 8 * blob / el_cp / 1e9
    del cp_dst
    h2d_tok = h2d / args.steps
    ceil_tok = copy_gbps * 1e9 / h2d_tok if h2d_tok > 0 else None
    detail["link_bound"] = {"h2d_GBps_copy_engines": copy_gbps, "h2d_MB_per_token": h2d_tok / 1e6,
                            "ceiling_tokens_per_s": ceil_tok,
                            "frac_of_ceiling": tok_s / ceil_tok if ceil_tok else None,
                            "note": "ceiling = H2D bytes per token / rate of 8-blob copies on two streams alone"}

    # ---------------------------------------------------------------- other fill variant
    # Same stack, caches emptied, misses filled the other way (fill blocks of
    # the shared-expert launch vs hipMemcpyAsync on the side stream).
    if not args.no_variant:
        other = "copy-engine" if args.fill == "kernel" else "kernel"
        for d in layers:
            api.moe_cache_reset(api.moe_layer_cache(d["h"]))
        stats_f = [api.moe_decode_stats() for _ in range(Lyr)]
        flags = flags_base | fill_flag[other]
        for t in range(args.warmup):
            token(t, handles, stats_f)
        torch.cuda.synchronize()
        warm_f = [(s.hits, s.misses) for s in stats_f]
        t0 = time.perf_counter()
        for t in range(args.warmup, args.warmup + args.steps):
            token(t, handles, stats_f)
        torch.cuda.synchronize()
        el_f = time.perf_counter() - t0
        flags = flags_base | fill_flag[args.fill]
        hf = sum(s.hits - w[0] for s, w in zip(stats_f, warm_f))
        mf = sum(s.misses - w[1] for s, w in zip(stats_f, warm_f))
        detail["fill_" + other.replace("-", "_")] = {
            "tokens_per_s": args.steps / el_f, "ms_per_step": 1e3 * el_f / args.steps,
            "hit_rate_timed": hf / max(hf + mf, 1)}

    # ---------------------------------------------------------------- slot-count sweep
    # The same stack with other pool sizes (fresh caches, the headline's fill
    # path, half the timed tokens): hit rate, bytes over PCIe and tokens/s per
    # slot count.
    # The last run is the headline's slot count with the LRU policy variant.
    sweep = [int(v) for v in args.sweep_slots.split(",") if v.strip()]
    if sweep:
        detail["slot_sweep"] = {}
        n_sw = max(args.steps // 2, 8)
        for S2, pol in [(v, api.MOE_POLICY_LFU) for v in sweep] + [(S, api.MOE_POLICY_LRU)]:
            if S2 < k or S2 > E:
                continue
            hs = []
            for d in layers:
                d["pool2"] = torch.empty((S2, blob), dtype=torch.uint8, device=devn)
                d["ws2"] = torch.zeros_like(d["ws"])
                hs.append(api.moe_layer_create(sh, router=d["router"], shared_blob=d["shared"],
                                               workspace=d["ws2"], bias=d["bias"], experts_host=d["host"],
                                               slot_pool=d["pool2"], n_slots=S2, copy_stream=copy_stream,
                                               cache_policy=pol))
            st2 = [api.moe_decode_stats() for _ in range(Lyr)]
            for t in range(args.warmup):
                token(t, hs, st2)
            torch.cuda.synchronize()
            w2 = [(s.hits, s.misses, s.h2d_bytes) for s in st2]
            t0 = time.perf_counter()
            for t in range(args.warmup, args.warmup + n_sw):
                token(t, hs, st2)
            torch.cuda.synchronize()
            el2 = time.perf_counter() - t0
            h2 = sum(s.hits - w[0] for s, w in zip(st2, w2))
            m2 = sum(s.misses - w[1] for s, w in zip(st2, w2))
            b2 = sum(s.h2d_bytes - w[2] for s, w in zip(st2, w2))
            key = str(S2) if pol == api.MOE_POLICY_LFU else f"{S2}_lru"
            detail["slot_sweep"][key] = {"tokens_per_s": n_sw / el2, "hit_rate": h2 / max(h2 + m2, 1),
                                         "h2d_MB_per_token": b2 / n_sw / 1e6, "tokens": n_sw}
            for h_ in hs:
                api.moe_layer_destroy(h_)
            for d in layers:
                del d["pool2"], d["ws2"]
            torch.cuda.synchronize()
        print("[bench] slot sweep done", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- device-stepped cache
    # The same stack with each layer's cache stepped on the device by the
    # routing kernel (misses copied by fill blocks): no host wait per layer,
    # run eagerly and as one HIP graph per token (30 layers).
    if not args.no_device_cache:
        hs = []
        for d in layers:
            d["pool3"] = torch.empty((S, blob), dtype=torch.uint8, device=devn)
            d["ws3"] = torch.zeros_like(d["ws"])
            hs.append(api.moe_layer_create(sh, router=d["router"], shared_blob=d["shared"], workspace=d["ws3"],
                                           bias=d["bias"], experts_host=d["host"], slot_pool=d["pool3"], n_slots=S,
                                           copy_stream=copy_stream, cache_on_device=True))

        def dc_counts():
            c = [api.moe_layer_cache_state(h_, S, stream=main_stream) for h_ in hs]
            return sum(v[3] for v in c), sum(v[4] for v in c)

        for t in range(args.warmup):
            token(t, hs)
        torch.cuda.synchronize()
        n_dc = args.steps
        h0, m0 = dc_counts()
        t0 = time.perf_counter()
        for t in range(args.warmup, args.warmup + n_dc):
            token(t, hs)
        torch.cuda.synchronize()
        el_e = time.perf_counter() - t0
        h1, m1 = dc_counts()
        xg = torch.empty((1, H), device=devn)
        eg = torch.empty((Lyr, 1, H), dtype=torch.int16, device=devn)

        def token_graph():
            s_ = torch.cuda.current_stream().cuda_stream
            src = xg.data_ptr()
            for l in range(Lyr):
                dst = hp[l & 1]
                rc = decode(hs[l], src, eg.data_ptr() + l * H * 2, 1, flags, dst, None, None, None, None, None, s_)
                if rc:
                    raise api.MoeError(rc, "moe_layer_decode", api.moe_last_error())
                src = dst
        cap2 = torch.cuda.Stream()
        torch.cuda.synchronize()
        gd = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gd, stream=cap2):
            token_graph()
        torch.cuda.synchronize()
        t_base = args.warmup + n_dc
        for t in range(t_base, t_base + 16):
            xg.copy_(x[t % T:t % T + 1])
            eg.copy_(eps[:, t % T:t % T + 1])
            gd.replay()
        torch.cuda.synchronize()
        h2, m2 = dc_counts()
        t0 = time.perf_counter()
        for t in range(t_base + 16, t_base + 16 + n_dc):
            xg.copy_(x[t % T:t % T + 1])
            eg.copy_(eps[:, t % T:t % T + 1])
            gd.replay()
        torch.cuda.synchronize()
        el_g = time.perf_counter() - t0
        h3, m3 = dc_counts()
        detail["device_cache_step"] = {
            "tokens_per_s_eager": n_dc / el_e, "tokens_per_s_graph": n_dc / el_g, "tokens": n_dc,
            "hit_rate_eager": (h1 - h0) / max(h1 - h0 + m1 - m0, 1),
            "hit_rate_graph": (h3 - h2) / max(h3 - h2 + m3 - m2, 1),
            "h2d_MB_per_token_graph": (m3 - m2) * blob / n_dc / 1e6}
        del gd
        for h_ in hs:
            api.moe_layer_destroy(h_)
        for d in layers:
            del d["pool3"], d["ws3"]
        torch.cuda.synchronize()
        print(f"[bench] device cache step: {detail['device_cache_step']}", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- expert file store
    # The same stack with the misses read from a file of all layers' experts
    # (each blob padded to 16 KiB pages) by parallel pread, unbuffered where
    # the file system allows, then copied like the host-memory misses. The
    # file is written and synced first, so the reads come from the disk.
    if not args.no_file_store:
        import shutil
        tmpdir = os.environ.get("TMPDIR", "/tmp")
        stride = api.moe_store_stride(blob)
        need = Lyr * E * stride
        if shutil.disk_usage(tmpdir).free < need + (8 << 30):
            detail["file_store"] = {"skipped": f"less than {need / 1e9 + 8:.1f} GB free in {tmpdir}"}
        else:
            path = os.path.join(tmpdir, f"moe_experts_{os.getpid()}.bin")
            t_w = time.perf_counter()
            try:
                pad = np.zeros((E, stride), np.uint8)
                with open(path, "wb") as fh:
                    for d in layers:
                        pad[:, :blob] = d["host"].numpy()
                        fh.write(pad.data)
                    fh.flush()
                    os.fsync(fh.fileno())
                t_w = time.perf_counter() - t_w
                store = api.moe_store_open(path, Lyr, E, blob, args.store_threads, True)
                hs = []
                for l, d in enumerate(layers):
                    d["pool3"] = torch.empty((S, blob), dtype=torch.uint8, device=devn)
                    d["ws3"] = torch.zeros_like(d["ws"])
                    hs.append(api.moe_layer_create(sh, router=d["router"], shared_blob=d["shared"],
                                                   workspace=d["ws3"], bias=d["bias"], slot_pool=d["pool3"],
                                                   n_slots=S, copy_stream=copy_stream, store=store,
                                                   store_layer=l))
                st3 = [api.moe_decode_stats() for _ in range(Lyr)]
                n_w3 = min(args.warmup, 16)
                for t in range(n_w3):
                    token(t, hs, st3)
                torch.cuda.synchronize()
                w3 = [(s.hits, s.misses, s.h2d_bytes) for s in st3]
                n3 = args.store_tokens
                t0 = time.perf_counter()
                for t in range(n_w3, n_w3 + n3):
                    token(t, hs, st3)
                torch.cuda.synchronize()
                el3 = time.perf_counter() - t0
                h3 = sum(s.hits - w[0] for s, w in zip(st3, w3))
                m3 = sum(s.misses - w[1] for s, w in zip(st3, w3))
                b3 = sum(s.h2d_bytes - w[2] for s, w in zip(st3, w3))
                detail["file_store"] = {
                    "tokens_per_s": n3 / el3, "ms_per_step": 1e3 * el3 / n3, "tokens": n3,
                    "hit_rate": h3 / max(h3 + m3, 1), "misses_per_token": m3 / n3,
                    "expert_GBps_wall": b3 / el3 / 1e9, "unbuffered": api.moe_store_is_direct(store),
                    "reader_threads": args.store_threads, "file_GB": need / 1e9,
                    "file_write_and_sync_s": t_w}
                for h_ in hs:
                    api.moe_layer_destroy(h_)
                api.moe_store_close(store)
                for d in layers:
                    del d["pool3"], d["ws3"]
            finally:
                if os.path.exists(path):
                    os.remove(path)
        print("[bench] file store done", file=sys.stderr, flush=True)

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
                rc = decode(res[l], src, e_in.data_ptr() + l * H * 2, 1, flags_base, dst, None, None, None,
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
        # attention step next to each MoE layer (RMSNorm, q/k/v, RoPE, fp16 KV
        # cache, grouped-query attention, output projection + residual) at a
        # context of attn_ctx positions: 30 layers with their own weights and
        # caches (1.6 GB together, so nothing stays in the last-level cache);
        # alone, then as full decoder layers with the resident MoE layers
        if not args.no_attn:
            A = GEMMA_ATTN
            pos_a = min(args.attn_ctx, A.max_ctx) - 1
            kc0, vc0 = gen.kv_cache(A, pos_a, 6, 0)
            kc0, vc0 = torch.from_numpy(kc0.view(np.int16)), torch.from_numpy(vc0.view(np.int16))
            at = []
            for l in range(Lyr):
                w_np = gen.attn_weights(A, 6, l)
                at.append({"w": {"norm_w": torch.from_numpy(w_np["norm_w"]).to(devn),
                                 "qkv_q": torch.from_numpy(w_np["qkv_q"]).to(devn),
                                 "qkv_s": torch.from_numpy(w_np["qkv_s"].view(np.int16)).to(devn),
                                 "o_q": torch.from_numpy(w_np["o_q"]).to(devn),
                                 "o_s": torch.from_numpy(w_np["o_s"].view(np.int16)).to(devn)},
                           "kc": kc0.to(devn), "vc": vc0.to(devn),
                           "ws": torch.zeros(api.moe_attn_workspace_bytes(A), dtype=torch.uint8, device=devn)})
            a_mid = torch.empty((1, H), device=devn)
            Wa = A.n_heads * A.head_dim
            attn_bytes = (A.qkv_rows * (H // 2 + 2 * (H // 32)) + H * (Wa // 2 + 2 * (Wa // 32))
                          + 2 * A.n_kv_heads * (pos_a + 1) * A.head_dim * 2)

            def step_attn(with_moe):
                s_ = torch.cuda.current_stream()
                src = x_in.data_ptr()
                for l in range(Lyr):
                    api.moe_attn_decode(A, at[l]["w"], at[l]["kc"], at[l]["vc"], pos_a, src, a_mid, at[l]["ws"],
                                        stream=s_)
                    if with_moe:
                        dst = hp[l & 1]
                        rc = decode(res[l], a_mid.data_ptr(), None, 1, flags_base, dst, None, None, None, None,
                                    None, s_.cuda_stream)
                        if rc:
                            raise api.MoeError(rc, "moe_layer_decode", api.moe_last_error())
                        src = dst
                    else:
                        src = a_mid.data_ptr()

            attn_detail = {"ctx": pos_a + 1, "bytes_per_step": attn_bytes}
            for with_moe in (False, True):
                with torch.cuda.stream(cap):
                    step_attn(with_moe)
                torch.cuda.synchronize()
                ga = torch.cuda.CUDAGraph()
                with torch.cuda.graph(ga, stream=cap):
                    step_attn(with_moe)
                torch.cuda.synchronize()
                for t in range(args.warmup):
                    x_in.copy_(x[t % T:t % T + 1])
                    ga.replay()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for t in range(args.warmup, args.warmup + args.steps):
                    x_in.copy_(x[t % T:t % T + 1])
                    ga.replay()
                torch.cuda.synchronize()
                el_a = time.perf_counter() - t0
                if with_moe:
                    attn_detail["decoder_layers_with_resident_moe_tokens_per_s"] = args.steps / el_a
                else:
                    us_a = 1e6 * el_a / (args.steps * Lyr)
                    attn_detail["us_per_step"] = us_a
                    attn_detail["GBps"] = attn_bytes / (us_a * 1e-6) / 1e9
                    attn_detail["frac_of_8TBps"] = attn_bytes / (us_a * 1e-6) / 8e12
                del ga
            # the cache-mode stack (16-slot LFU per layer, misses over PCIe) with
            # the attention step in place of the seeded perturbation
            a_sh = api.make_attn_shape(A)
            a_w = [_lib.moe_attn_weights(*(a["w"][k].data_ptr() for k in ("norm_w", "qkv_q", "qkv_s", "o_q", "o_s")))
                   for a in at]
            a_ptr = [(a["kc"].data_ptr(), a["vc"].data_ptr(), a["ws"].data_ptr(), a["ws"].numel()) for a in at]
            st_a = [api.moe_decode_stats() for _ in range(Lyr)]
            attn_call = lib.moe_attn_decode

            def token_attn(t):
                src = xp0 + (t % T) * H * 4
                for l in range(Lyr):
                    kcp, vcp, wsp, wsb = a_ptr[l]
                    rc = attn_call(C.byref(a_sh), C.byref(a_w[l]), kcp, vcp, pos_a, src, a_mid.data_ptr(), wsp, wsb,
                                   sp)
                    if rc:
                        raise api.MoeError(rc, "moe_attn_decode", api.moe_last_error())
                    dst = hp[l & 1]
                    rc = decode(handles[l], a_mid.data_ptr(), None, 1, flags, dst, None, None, None, None,
                                C.byref(st_a[l]), sp)
                    if rc:
                        raise api.MoeError(rc, "moe_layer_decode", api.moe_last_error())
                    src = dst
            n_at = max(args.steps // 4, 16)
            for t in range(16):
                token_attn(t)
            torch.cuda.synchronize()
            w_a = [(s_.hits, s_.misses) for s_ in st_a]
            t0 = time.perf_counter()
            for t in range(16, 16 + n_at):
                token_attn(t)
            torch.cuda.synchronize()
            el_a = time.perf_counter() - t0
            h_a = sum(s_.hits - w_[0] for s_, w_ in zip(st_a, w_a))
            m_a = sum(s_.misses - w_[1] for s_, w_ in zip(st_a, w_a))
            attn_detail["decoder_layers_with_lfu16_moe"] = {"tokens_per_s": n_at / el_a, "tokens": n_at,
                                                           "hit_rate": h_a / max(h_a + m_a, 1)}
            detail["attention_step"] = attn_detail
            print(f"[bench] attention step: {attn_detail}", file=sys.stderr, flush=True)

        for h in res:
            api.moe_layer_destroy(h)

        # floor of one launch streaming the routed gate/up's bytes with no
        # arithmetic (same event method), rotating over one layer's 428 MB of
        # experts so that no launch finds its bytes in the last-level cache
        src = layers[0]["experts_dev"]
        fb = gu_bytes // 16 * 16
        stride = (fb + 255) // 256 * 256
        nreg = src.numel() // stride
        fout = torch.zeros(2048 * 16, dtype=torch.int32, device=devn)
        floor = {"bytes": fb, "regions": nreg}
        for blocks in (176, 256, 512, 1024):
            api.moe_debug_read_floor(src, fb, blocks, fout, region_stride=stride, regions=nreg, reps=nreg)
            us_f = api.moe_debug_read_floor(src, fb, blocks, fout, region_stride=stride, regions=nreg,
                                            reps=10 * nreg, timed=True)
            floor[f"grid_{blocks}x1024"] = {"us": us_f, "frac": fb / (us_f * 1e-6) / 8e12}
        one = 176 * 1024 * 16
        us_1 = api.moe_debug_read_floor(src, one, 176, fout, region_stride=stride, regions=nreg,
                                        reps=10 * nreg, timed=True)
        floor["one_load_per_lane_176x1024_us"] = us_1
        # the same read-only stream at 2-16x the bytes per launch (8 loads per
        # lane, as many 1024-thread blocks as that takes), rotating over 1 GiB:
        # how much of the HBM peak one launch reaches as its size grows
        big = torch.empty(1 << 30, dtype=torch.uint8, device=devn)
        bout = torch.zeros(4096 * 16, dtype=torch.int32, device=devn)  # 16 words per block, <= 4096 blocks
        by_size = {}
        for m in (1, 2, 4, 8, 16):
            nb_m = fb * m
            st_m = (nb_m + 255) // 256 * 256
            reg_m = big.numel() // st_m
            blk_m = (nb_m // 16 + 8 * 1024 - 1) // (8 * 1024)
            assert blk_m <= 4096
            api.moe_debug_read_floor(big, nb_m, blk_m, bout, region_stride=st_m, regions=reg_m, reps=reg_m)
            us_m = api.moe_debug_read_floor(big, nb_m, blk_m, bout, region_stride=st_m, regions=reg_m,
                                            reps=max(4 * reg_m, 20), timed=True)
            by_size[f"{nb_m / 1e6:.1f}MB"] = {"blocks": blk_m, "us": us_m, "frac": nb_m / (us_m * 1e-6) / 8e12}
        floor["by_launch_size"] = by_size
        del big, bout
        detail["launch_floor"] = floor
        print(f"[bench] launch floor: {floor}", file=sys.stderr, flush=True)

        # batched decode (B tokens per step, grouped by expert) and 2048-token
        # prefill, unbiased routing. Consecutive steps use consecutive layers
        # (routers, shared and routed experts of all 30 layers resident, one
        # workspace shared by the handles as calls are in stream order), so no
        # step finds its weights in the last-level cache.
        for B in (16, 64):
            wsb = torch.zeros(api.moe_layer_workspace_bytes(sh, B, 0), dtype=torch.uint8, device=devn)
            hbs = [api.moe_layer_create(sh, router=d["router"], shared_blob=d["shared"], workspace=wsb,
                                        experts_dev=d["experts_dev"], max_B=B) for d in layers]
            xb = torch.from_numpy(gen.x_fp32(B * 8, H, 3, sub=B)).to(devn)
            yb = torch.empty((B, H), device=devn)
            idsb = torch.empty((B, k), dtype=torch.int32, device=devn)

            def bstep(i):
                api.moe_layer_decode(hbs[i % Lyr], xb[(i % 8) * B:(i % 8 + 1) * B], None, B, 0, yb, idsb)
            # steady state: 4 untimed rotations over the layers first (the
            # first touches each layer's pages; the clocks settle over about
            # 100 ms of sustained work), then 8 timed rotations
            n_warm, n_it = 4 * Lyr, 8 * Lyr
            for i in range(n_warm):
                bstep(i)
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            touched = 0
            for i in range(n_it):
                bstep(n_warm + i)
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
            for hb in hbs:
                api.moe_layer_destroy(hb)
            del wsb
        Tp = 2048
        wsp = torch.zeros(api.moe_layer_workspace_bytes(sh, 1, Tp), dtype=torch.uint8, device=devn)
        hps = [api.moe_layer_create(sh, router=d["router"], shared_blob=d["shared"], workspace=wsp,
                                    experts_dev=d["experts_dev"], max_T=Tp) for d in layers]
        xp = torch.from_numpy(gen.x_bf16(Tp, H, 4).view(np.int16)).to(devn)
        lp = torch.from_numpy(gen.logits_uniform(Tp, E, 4)).to(devn)
        yp = torch.empty((Tp, H), device=devn)
        # steady state, as for batched decode: 3 untimed rotations over the
        # layers, then 2 timed ones
        n_warm, n_it = 3 * Lyr, 2 * Lyr
        for i in range(n_warm):
            api.moe_layer_prefill(hps[i % Lyr], xp, lp, Tp, yp)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(n_it):
            api.moe_layer_prefill(hps[(n_warm + i) % Lyr], xp, lp, Tp, yp)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / n_it
        flops = 2.0 * Tp * (k * 3 * H * I + 3 * H * Is)
        detail["prefill_2048"] = {"ms": ms, "TFLOPs": flops / (ms * 1e-3) / 1e12,
                                  "mfma_bf16_frac": flops / (ms * 1e-3) / 2.5e15, "GFLOP": flops / 1e9}
        for hp_ in hps:
            api.moe_layer_destroy(hp_)
        del wsp
        for d in layers:
            del d["experts_dev"]

    # ---------------------------------------------------------------- prefill through the slot pool
    # 2048 tokens of one layer in 128-token chunks through a cold 16-slot pool
    # (cache mode, misses from pinned host memory): the time to the first
    # token's layer output when the experts do not fit in HBM.
    Tq = 2048
    wsq = torch.zeros(api.moe_layer_workspace_bytes(sh, 1, Tq), dtype=torch.uint8, device=devn)
    xq = torch.from_numpy(gen.x_bf16(Tq, H, 4).view(np.int16)).to(devn)
    lq = torch.from_numpy(gen.logits_uniform(Tq, E, 4)).to(devn)
    yq = torch.empty((Tq, H), device=devn)
    detail["prefill_2048_slot_pool"] = {}
    for chunk_q in (128, Tq):
        runs = []
        for l in range(3):
            d = layers[l]
            poolq = torch.empty((S, blob), dtype=torch.uint8, device=devn)
            hq = api.moe_layer_create(sh, router=d["router"], shared_blob=d["shared"], workspace=wsq,
                                      bias=d["bias"], experts_host=d["host"], slot_pool=poolq, n_slots=S,
                                      copy_stream=copy_stream, max_T=Tq)
            api.moe_layer_prefill_chunk(hq, chunk_q)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            api.moe_layer_prefill(hq, xq, lq, Tq, yq)
            torch.cuda.synchronize()
            el_q = time.perf_counter() - t0
            hits_q, misses_q, _ = api.moe_cache_counters(api.moe_layer_cache(hq))
            runs.append((el_q, hits_q, misses_q))
            api.moe_layer_destroy(hq)
            del poolq
        ms_q = 1e3 * sum(r[0] for r in runs[1:]) / len(runs[1:])  # the first run also warms the kernels
        miss_q = sum(r[2] for r in runs[1:]) / len(runs[1:])
        hit_q = sum(r[1] for r in runs[1:]) / len(runs[1:])
        detail["prefill_2048_slot_pool"][f"chunk_{chunk_q}"] = {
            "ms": ms_q, "misses": miss_q, "hits": hit_q, "h2d_GB": miss_q * blob / 1e9,
            "h2d_GBps_wall": miss_q * blob / (ms_q * 1e-3) / 1e9, "slots": S}
    del wsq
    print("[bench] slot-pool prefill done", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- oracle on host cores
    cpu = None
    if not args.no_cpu:
        print("[bench] timing the oracle on host cores", file=sys.stderr, flush=True)
        cpu = cpu_baseline(Lyr, T, cid, args.cpu_seconds)

    traffic = load_traffic()
    if traffic:
        detail["traffic_vs_algorithmic"] = traffic["traffic_bytes"] / gu_bytes
    trace = load_trace()
    # all expert weight bytes of a cache-mode layer step (the routed experts'
    # gate/up and down, the shared expert's down) over the routed gate/up and
    # the down kernels' event-timed durations
    exp_bytes = k * 3 * I * (H // 2 + 2 * (H // 32)) + H * (Is // 2 + 2 * (Is // 32))
    detail["expert_GBps_gateup_plus_down"] = exp_bytes / ((us_gu + us_dn) * 1e-6) / 1e9 if us_dn > 0 else None
    fl = detail.get("launch_floor", {}).get("grid_176x1024")
    if fl:
        detail["routed_gateup_frac_of_read_floor"] = fl["us"] / us_gu
    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * el_head / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights x 16-bit fixed-point activations -> int32, fp32 scale/accumulate",
        "data": "synthetic (seeded; no trained weights)",
        "config": {"workload": C2.name, "layers": Lyr, "hidden": H, "experts": E, "top_k": k,
                   "inter": I, "shared_inter": Is, "slots_per_layer": S, "batch": 1,
                   "expert_store": "pinned host memory",
                   "miss_fill": ("fill blocks in the shared-expert gate/up launch" if args.fill == "kernel"
                                 else "hipMemcpyAsync on a side stream"),
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": gbps_gu, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps_gu / HBM_PEAK_GBPS,
                     "traffic": traffic["traffic_bytes"] if traffic else None,
                     "kernel": "k_gateup (routed experts, cache mode)", "bytes_per_launch": gu_bytes,
                     "mean_us": us_gu, "launches": n_gu,
                     "trace_mean_us": trace["mean_us"] if trace else None,
                     "trace_frac": gu_bytes / (trace["mean_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS if trace else None},
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(out), flush=True)
    for d in layers:
        api.moe_layer_destroy(d["h"])


if __name__ == "__main__":
    main()
