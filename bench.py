#!/usr/bin/env python3
"""Speculative-decoding throughput on one MI355X.

Workload (default): the full 28-layer Qwen2.5-7B-shaped random-init model,
vocab 152064; layers 0-10 shared in bf16, layers 11-27 replaced in the draft
by 4-bit group-64 substitutes; chain draft gamma = 16, verify 17 positions,
greedy (T = 0); a 512-token synthetic prompt (prefilled, not timed) and 256
generated tokens.  One step = one generation of 256 tokens from the prompt
state (every speculative cycle it takes: draft, verify, reject, rollback).

Prints one JSON line: tokens/s, the roofline of the dominant kernel (HIP
events around every launch of an extra, instrumented step), and the CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0

# HBM traffic per launch of a draft GEMV site, from two rocprofv3 --pmc runs of
# `bench.py --site NAME` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each
# scaled by what the same counter reads for a 1 GiB device-to-device copy in
# the same run (FETCH_SIZE 524316 KiB -> x2.0, WRITE_SIZE 1048576 KiB -> x1.0).
# Reported only while the kernel sources hash to the value they were taken on.
TRAFFIC = {
    "bf16_gate_up": {"fetch_kib": 132734.0, "write_kib": 148.3, "fetch_scale": 2.0,
                     "write_scale": 1.0, "sources": "8f1af8166c2b2b57"},
    "w4_gate_up": {"fetch_kib": 37409.7, "write_kib": 37.0, "fetch_scale": 2.0,
                   "write_scale": 1.0, "sources": "8f1af8166c2b2b57"},
}
GEMV_SOURCES = ("csrc/gemv.hip", "csrc/gemv_w4t.hip", "csrc/common.h", "csrc/internal.h")


def sources_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "self_speculative_decoding_w4a16_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_bytes(site):
    t = TRAFFIC.get(site)
    if not t or t["sources"] != sources_hash(GEMV_SOURCES):
        return None
    return round(1024 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="full7b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ar", action="store_true")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the tiny and one-7B-layer measurements")
    ap.add_argument("--site", default=None,
                    help="only launch one draft GEMV site (e.g. bf16_gate_up), or one verify GEMM "
                         "(verify_gate_up, verify_down: gamma+1 positions, store epilogue), back to "
                         "back, then copy 1 GiB device to device: the workload for counter runs")
    ap.add_argument("--only", default=None, choices=["tree", "batch_decode", "multilevel", "batch_w4_gemm", "lowbit",
                                                      "adaptive_length"],
                    help="only one widened row's section of the 7B workload, from the same prompt state: "
                         "prints {section: result} (the workload for that row's kernel-trace profile)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the "
              "multi-GPU path (one decode per GPU, or tensor-parallel layers over xGMI) is not built.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from self_speculative_decoding_w4a16_amd import _lib
    from self_speculative_decoding_w4a16_amd.engine import SpecDecoder
    from self_speculative_decoding_w4a16_amd.model import DeviceModel
    from synth import CONFIGS, model_weights, token_ids, uniform_codes

    wl = CONFIGS[args.config]
    shape = wl.shape
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    _lib.lib()
    log(f"building {shape.name}: {shape.n_layers} layers, vocab {shape.vocab}")
    w = model_weights(shape, 0, dev)
    dm = DeviceModel(shape, w)
    torch.cuda.synchronize()
    if args.site and args.site.startswith("verify_"):
        # the verify GEMM of one site on every shared layer's weights, 2 rounds
        name = {"verify_gate_up": "gate_up", "verify_down": "down", "verify_qkv": "qkv",
                "verify_o": "o"}[args.site]
        shared = [l for l in range(shape.n_layers) if l not in dm.substitute_layers]
        mats = [dm.w["layers"][l][name] for l in shared]
        m = wl.gamma + 1
        k = mats[0].shape[1]
        x = (torch.randn(m, k, device=dev, generator=torch.Generator(device=dev).manual_seed(9)) * 0.5).bfloat16()
        y = torch.empty(m, mats[0].shape[0], device=dev, dtype=torch.bfloat16)
        ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
        for _ in range(2):
            for wmat in mats:
                _lib.bf16_gemm(wmat, x, y, ws)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        n, kk = mats[0].shape
        print(json.dumps({"site": args.site, "m": m, "n": n, "k": kk, "launches": 2 * len(mats),
                          "copy_bytes": 1 << 30}), flush=True)
        return
    if args.site:
        iso = isolated_gemvs(dm, shape, dev, reps=1, only=args.site, graph=False)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"site": args.site, **iso[args.site], "copy_bytes": 1 << 30}), flush=True)
        return
    gamma, G = wl.gamma, wl.generate
    cap = ((wl.prompt + G + gamma + 1 + 63) // 64) * 64 + 64
    sparse = None
    if "budget_permille" in wl.extra:
        sparse = dict(n_sink=wl.extra["n_sink"], n_recent=wl.extra["n_recent"],
                      window=wl.extra["window"], budget_permille=wl.extra["budget_permille"])
    dec = SpecDecoder(dm, cap, gamma, wl.temp, wl.draft_temp, sparse=sparse, graphs=True)
    t0 = time.time()
    if sparse:
        # long context: a synthetic KV history (N(0,1) per layer and head)
        # stands in for a prefilled document; there is no 60K-token prefill
        from synth import kv_history
        for l in range(shape.n_layers):
            K, V = kv_history(1, shape.n_kv_heads, wl.prompt, shape.head_dim, wl.prompt, 600 + l, dev)
            dec.k_cache[l, :, :wl.prompt].copy_(K[0])
            dec.v_cache[l, :, :wl.prompt].copy_(V[0])
        kv0, last = wl.prompt, int(token_ids(1, shape.vocab, 5)[0])
        log(f"synthetic KV history of {wl.prompt} positions in {time.time() - t0:.2f}s")
    else:
        prompt = [int(t) for t in token_ids(wl.prompt, shape.vocab, 5)]
        dec.prefill(prompt)
        torch.cuda.synchronize()
        log(f"prefill {len(prompt)} tokens in {time.time() - t0:.2f}s")
        kv0, last = len(prompt) - 1, prompt[-1]

    stochastic = wl.temp > 0 or wl.draft_temp > 0
    if args.only:
        if args.config != "full7b" or stochastic:
            print("--only runs the widened rows of the greedy 7B workload (--config full7b)", file=sys.stderr)
            sys.exit(2)
        n_w4 = len(dm.substitute_layers)
        if args.only == "tree":
            r = tree_rates(dec, dm, shape, wl, kv0, last)
        elif args.only == "batch_decode":
            r = batch_decode_rates(dm, w, shape, wl, dev)
        elif args.only == "multilevel":
            r = multilevel_rates(dec, dm, w, shape, wl, kv0, last)
        elif args.only == "batch_w4_gemm":
            r = batch_rates(dm, shape, dev)
        elif args.only == "lowbit":
            r = lowbit_rates(dec, shape, w, wl, kv0, last, dev)
        else:
            draft_pass, verify_pass = pass_rates(dec, shape, wl, kv0, last, n_w4)
            r = adaptive_rates(dec, dm, wl, kv0, last, draft_pass["avg_us"] / verify_pass["avg_us"])
        print(json.dumps({args.only: r}), flush=True)
        return
    uni = None
    if stochastic:
        C = G + 1
        Ud, _ = uniform_codes(C * gamma, 101)
        R, _ = uniform_codes(C * gamma, 102)
        Uf, _ = uniform_codes(C, 103)
        cvt = lambda a: torch.tensor(a.astype(np.int32), device=dev)
        uni = (cvt(Ud).view(C, gamma), cvt(R).view(C, gamma), cvt(Uf))

    def one_generation():
        dec.reset(kv0, last)
        out, ns = [], []
        c = 0
        while len(out) < G:
            if uni is not None:
                dec.cycle(uni[0][c], uni[1][c], uni[2][c:c + 1])
            else:
                dec.cycle()
            n = int(dec.n_accepted.item())
            out += dec.out_tokens[:n + 1].tolist()
            ns.append(n)
            c += 1
        return out[:G], ns

    for i in range(args.warmup):
        one_generation()
        log(f"warmup {i} done")
    torch.cuda.synchronize()
    all_ns = []
    outs = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        o, ns = one_generation()
        all_ns += ns
        outs.append(o)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tok_s = args.steps * G / elapsed
    tau = float(np.mean([n + 1 for n in all_ns]))
    cycles_per_gen = len(all_ns) / args.steps
    log(f"timed {args.steps} steps: {tok_s:.2f} tok/s, tau {tau:.3f}, {cycles_per_gen:.1f} cycles/gen")
    if not stochastic:
        assert all(o == outs[0] for o in outs), "greedy generations differ between steps"

    # ---------------------------------------------------------------- phases
    ev = lambda: torch.cuda.Event(enable_timing=True)
    dec.reset(kv0, last)
    e = [ev() for _ in range(5)]
    e[0].record()
    dec.draft(uni[0][0] if uni else None)
    e[1].record()
    dec.verify()
    e[2].record()
    dec.reject(uni[1][0] if uni else None, uni[2][0:1] if uni else None)
    e[3].record()
    dec.commit()
    e[4].record()
    torch.cuda.synchronize()
    draft_ms = e[0].elapsed_time(e[1])
    verify_ms = e[1].elapsed_time(e[2])
    reject_ms = e[2].elapsed_time(e[3])
    n_w4 = len(dm.substitute_layers)
    sparse_keys = None
    if sparse:
        sparse_keys = _lib.index_count(kv0, sparse["n_sink"], sparse["n_recent"], sparse["budget_permille"])
        # the index the draft reads: rebuilt from a verify pass at the resident state
        dec.reset(kv0, last)
        dec.verify()
        _lib.kv_select(dm.c, dec.c)
        torch.cuda.synchronize()
    draft_pass, verify_pass = pass_rates(dec, shape, wl, kv0, last, n_w4, sparse_keys)
    log(f"draft step {draft_pass['avg_us']:.1f} us ({draft_pass['frac']:.3f} of peak; "
        f"{draft_pass['avg_us_attn_own_launch']:.1f} us with every attention in its own launch), "
        f"verify pass {verify_pass['avg_us']:.1f} us ({verify_pass['frac']:.3f})")

    # ---------------------------------------------------------------- kernels
    # One more generation with every launch bracketed by HIP events on the
    # launch stream.  Attention's algorithmic bytes depend on the device-side
    # KV length, so they are added here from the host's record of it: a draft
    # step at position p reads K and V of positions [0, p] once per layer, a
    # verify pass reads [0, kv_len + gamma] once per layer.
    dec.use_graphs = False  # recorded replays would bypass the launch profiler
    _lib.profile_start(400000)
    _, ns_prof = one_generation()
    torch.cuda.synchronize()
    _lib.profile_stop()
    dec.use_graphs = True
    kv_row = 2 * shape.n_kv_heads * shape.head_dim * 2 * shape.n_layers  # K+V bytes per position
    attn_bytes = {"attn_draft": 0.0, "attn_verify": 0.0}
    kv = kv0
    for c, n in enumerate(ns_prof):
        if sparse and c > 0:  # the index plus the speculative positions
            n_idx = _lib.index_count(kv, sparse["n_sink"], sparse["n_recent"], sparse["budget_permille"])
            attn_bytes["attn_draft"] += sum((n_idx + i + 1) * kv_row for i in range(gamma))
        else:
            attn_bytes["attn_draft"] += sum((kv + i + 1) * kv_row for i in range(gamma))
        attn_bytes["attn_verify"] += (kv + gamma + 1) * kv_row
        kv += n + 1
    raw = {name: _lib.profile_read(k) for k, name in enumerate(_lib.K_NAMES)}
    # layers whose attention ran inside the QKV launch (low-bit tiled QKV,
    # dense keys) take their share of the KV bytes there
    n_own, n_in = raw["attn_draft"][0], raw["qkv_attn"][0]
    own_frac = n_own / (n_own + n_in) if n_own + n_in else 1.0
    attn_bytes["qkv_attn"] = attn_bytes["attn_draft"] * (1.0 - own_frac)
    attn_bytes["attn_draft"] *= own_frac
    kern = {}
    for name in _lib.K_NAMES:
        n, ms, by = raw[name]
        by += attn_bytes.get(name, 0.0)
        kern[name] = {"launches": n, "ms": ms, "bytes": by}
    for g, members in _lib.K_GROUPS.items():
        kern[g] = {"launches": sum(kern[m]["launches"] for m in members),
                   "ms": sum(kern[m]["ms"] for m in members),
                   "bytes": sum(kern[m]["bytes"] for m in members)}
    for name, k in kern.items():
        n, ms, by = k["launches"], k["ms"], k["bytes"]
        k.update({"ms": round(ms, 4), "avg_us": round(1000 * ms / n, 3) if n else None,
                  "gbs": round(by / (ms * 1e-3) / 1e9, 1) if ms > 0 and by > 0 else None,
                  "bytes_per_launch": round(by / n) if n else None})
        del k["bytes"]
    log("kernels: " + json.dumps(kern))

    def roof(name):
        k = kern[name]
        if not k["launches"] or not k["gbs"]:
            return None
        return {"bound": "hbm", "achieved": k["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k["gbs"] / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": name, "avg_us": k["avg_us"], "bytes_per_launch": k["bytes_per_launch"]}

    # dominant kernel: of the launch sites that are one kernel each (the draft
    # GEMVs and the verify GEMMs; the attention sites are two launches each and
    # have their own entries), the one with the most time in a step; its
    # duration is measured back to back on the model's own weights
    sites = [n for n in _lib.K_NAMES[:14] if kern[n]["launches"] and kern[n]["gbs"]]
    dominant = max(sites, key=lambda n: kern[n]["ms"])
    iso = isolated_gemvs(dm, shape, dev)
    log("isolated: " + json.dumps(iso))

    def roof_iso(names, label):
        if not names:
            return None
        ms = sum(iso[n]["avg_us"] * iso[n]["per_step"] for n in names) / 1000
        by = sum(iso[n]["bytes_per_launch"] * iso[n]["per_step"] for n in names)
        gbs = by / (ms * 1e-3) / 1e9
        out = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": label}
        if len(names) == 1:
            out.update(traffic=traffic_bytes(names[0]), avg_us=iso[names[0]]["avg_us"],
                       bytes_per_launch=iso[names[0]]["bytes_per_launch"], symbol=iso[names[0]]["symbol"])
        return out

    # the draft attention inside the QKV launch: the launch's in-cycle time
    # less the QKV GEMV's own (isolated, back to back) time
    attn_in_qkv = None
    if kern["qkv_attn"]["launches"] and "w4_qkv" in iso:
        fa, q1 = kern["qkv_attn"]["avg_us"], iso["w4_qkv"]["avg_us"]
        attn_in_qkv = {"launch_avg_us": fa, "qkv_gemv_alone_us": q1, "attn_added_us": round(fa - q1, 3),
                       "attn_own_launch_avg_us": kern["attn_draft"]["avg_us"],
                       "layers_per_step": round(kern["qkv_attn"]["launches"] /
                                                max(1, kern["qkv_attn"]["launches"] +
                                                    kern["attn_draft"]["launches"]) * shape.n_layers, 2),
                       "draft_step_us": draft_pass["avg_us"],
                       "draft_step_attn_own_launch_us": draft_pass.get("avg_us_attn_own_launch")}

    ceiling = stream_ceiling(dev)
    log(f"HBM read ceiling: {ceiling['achieved']} GB/s over {ceiling['bytes'] >> 30} GiB")

    # ---------------------------------------------------------------- plain AR
    ar = None
    if not args.no_ar and not stochastic:
        full = DeviceModel(shape, w, substitute_layers=[])
        ar_dec = SpecDecoder(full, cap, 1, 0.0, 0.0)
        ar_dec.k_cache.copy_(dec.k_cache)
        ar_dec.v_cache.copy_(dec.v_cache)
        ar_dec.reset(kv0, last)
        for _ in range(4):
            ar_dec.ar_step()
        torch.cuda.synchronize()
        ar_dec.reset(kv0, last)
        n_ar = 64
        t0 = time.perf_counter()
        for _ in range(n_ar):
            ar_dec.ar_step()
        torch.cuda.synchronize()
        ar = n_ar / (time.perf_counter() - t0)
        del ar_dec, full
        log(f"plain bf16 autoregressive decode: {ar:.2f} tok/s")

    # ---------------------------------------------------------------- small workloads
    tiny = layer = lowbit = None  # noqa: F841
    if args.config == "full7b" and not args.no_small:
        tiny = tiny_rates(dev, oracle=not args.no_cpu_baseline)
        log(f"tiny workload: {json.dumps(tiny)}")
        layer = layer7b_rates(dev)
        log(f"one 7B layer: {json.dumps(layer)}")
        lowbit = lowbit_rates(dec, shape, w, wl, kv0, last, dev)
        log(f"3- and 2-bit substitutes: {json.dumps(lowbit)}")
    batch = None
    if args.config == "full7b" and not args.no_small:
        batch = batch_rates(dm, shape, dev)
        log(f"4-bit skinny GEMM (batch of drafts): {json.dumps(batch)}")
    bdec = None
    if args.config == "full7b" and not args.no_small and not stochastic:
        bdec = batch_decode_rates(dm, w, shape, wl, dev)
    tree = None
    if args.config == "full7b" and not args.no_small and not stochastic:
        tree = tree_rates(dec, dm, shape, wl, kv0, last)
        log(f"static tree k=6 D=48: {json.dumps(tree)}")
    mlev = None
    if args.config == "full7b" and not args.no_small and not stochastic:
        mlev = multilevel_rates(dec, dm, w, shape, wl, kv0, last)
    adapt = None
    if not sparse and not args.no_small and not stochastic:
        adapt = adaptive_rates(dec, dm, wl, kv0, last, draft_pass["avg_us"] / verify_pass["avg_us"])
        log(f"adaptive draft length: {json.dumps(adapt)}")

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        osample = OracleSample(shape, w, wl)
        cpu = cpu_baseline(osample, dm, wl, tau)
        oracle_beside(osample, cpu, wl, layer, lowbit, batch, bdec, tree, mlev, adapt)
        cpu.pop("_cycle_parts")
        del osample

    line = {
        "metric": "spec-decode tokens/s @7B shape \u03b3=16; W4 GEMV & verify HBM GB/s vs peak",
        "value": round(tok_s, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1000 * elapsed / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights, random prompt ids)",
        "config": {"workload": f"{wl.name}: {shape.n_layers}-layer {shape.name} random-init, "
                               f"{shape.n_shared} shared bf16 + {shape.n_layers - shape.n_shared} "
                               f"W4 g64 substitute layers, vocab {shape.vocab}, gamma {gamma}, "
                               f"T {wl.temp}, T_d {wl.draft_temp}, "
                               + (f"synthetic KV history {wl.prompt} positions, draft over a sparse "
                                  f"index (sink {sparse['n_sink']}, recent {sparse['n_recent']}, "
                                  f"budget {sparse['budget_permille'] / 10:g}%, scores of the last "
                                  f"{sparse['window']} verify rows), " if sparse else
                                  f"prompt {wl.prompt}, ")
                               + f"generate {G}",
                   "global_batch": 1, "seq_len": wl.prompt + G, "parallelism": "none (1 GPU)"},
        "roofline": roof_iso([dominant], dominant) if dominant in iso else roof(dominant),
        "roofline_w4_gemv": roof_iso([n for n in ("w4_qkv", "w4_o", "w4_gate_up", "w4_down") if n in iso],
                                     "w4_gemv (byte-weighted over one draft step's W4 GEMVs)"),
        "roofline_w4_gate_up": roof_iso(["w4_gate_up"], "w4_gate_up") if "w4_gate_up" in iso else None,
        "roofline_bf16_gemv": roof_iso([n for n in ("bf16_qkv", "bf16_o", "bf16_gate_up", "bf16_down",
                                                    "lm_head") if n in iso],
                                       "bf16_gemv (byte-weighted over one draft step's bf16 GEMVs)"),
        "roofline_verify_gemm": roof("verify_gemm"),
        "roofline_verify_pass": verify_pass,
        "roofline_draft_step": draft_pass,
        "roofline_attn_draft": roof("attn_draft"),
        "attn_in_qkv_launch": attn_in_qkv,
        "stream_ceiling": ceiling,
        "isolated_gemv": iso,
        "cpu_baseline": cpu,
        "tau": round(tau, 4),
        "cycles_per_step": round(cycles_per_gen, 2),
        "cycle_ms": {"draft": round(draft_ms, 3), "draft_steps": gamma, "verify": round(verify_ms, 3),
                     "reject": round(reject_ms, 3)},
        "plain_ar_tokens_s": round(ar, 3) if ar else None,
        "speculative_over_plain_ar": round(tok_s / ar, 4) if ar else None,
        "tiny": tiny,
        "layer7b": layer,
        "lowbit": lowbit,
        "adaptive_length": adapt,
        "batch_w4_gemm": batch,
        "tree": tree,
        "batch_decode": bdec,
        "multilevel": mlev,
        "kernels": kern,
    }
    # every rate also against the measured read ceiling
    for key, r in list(line.items()) + ([(k, v) for k, v in layer.items() if isinstance(v, dict) and "frac" in v]
                                        if layer else []):
        if (key.startswith("roofline") or key in ("draft_w4_layer", "verify_layer")) and r:
            r["frac_of_stream"] = round(r["achieved"] / ceiling["achieved"], 4)
    # the two bandwidth targets (>= 0.70 of 8 TB/s): the W4 draft GEMV and the verify pass
    w4r = line["roofline_w4_gemv"]
    line["targets"] = {
        "w4_gemv": {"frac": w4r["frac"] if w4r else None, "target": 0.70,
                    "met": bool(w4r and w4r["frac"] >= 0.70)},
        "verify_pass": {"frac": verify_pass["frac"], "target": 0.70, "met": verify_pass["frac"] >= 0.70},
    }
    # and the draft attention's time a layer (<= 3.5 us): its own launch, and
    # what it adds inside the QKV launch where it runs there
    own = kern["attn_draft"]["avg_us"]
    inq = attn_in_qkv["attn_added_us"] if attn_in_qkv else None
    worst = max(v for v in (own, inq) if v is not None) if (own or inq) else None
    line["targets"]["attn_draft_us"] = {"own_launch_us": own, "in_qkv_launch_added_us": inq, "target": 3.5,
                                        "met": bool(worst is not None and worst <= 3.5)}
    print(json.dumps(line), flush=True)


def stream_ceiling(dev, nbytes=4 << 30, reps=10):
    """The HBM read ceiling: one read-only kernel streaming a 4 GiB buffer
    (well past the 256 MB last-level cache), timed with HIP events on its
    launch stream over back-to-back launches."""
    import torch

    from self_speculative_decoding_w4a16_amd import _lib
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev)
    for _ in range(2):
        _lib.hbm_read(buf, sink, st.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        _lib.hbm_read(buf, sink, st.cuda_stream)
    e1.record(st)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000 / reps
    del buf
    torch.cuda.empty_cache()
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"achieved": round(gbs, 1), "unit": "GB/s", "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes": nbytes, "avg_us": round(us, 2), "kernel": "hbm_read_kernel (read-only stream)"}


def isolated_gemvs(dm, shape, dev, reps=3, only=None, graph=True):
    """The draft step's GEMV kernels launched back to back through the fused
    GEMV entry point, timed with one pair of HIP events on the launch stream:
    the average duration of one kernel at one shape.  Each launch reads a
    different weight matrix: the model's layers, plus copies of them until a
    round covers >= 1 GiB, so that no launch finds its weights in the 256 MB
    last-level cache (in the draft step ~130 MB of other weights pass between
    two launches of a site).
    The lm_head runs with a plain store epilogue here (in the draft step it
    also writes per-block max/argmax)."""
    import torch

    from self_speculative_decoding_w4a16_amd import _lib

    H, F = shape.hidden, shape.ffn
    qkv = (shape.n_q_heads + 2 * shape.n_kv_heads) * shape.head_dim
    qd = shape.n_q_heads * shape.head_dim
    gen = torch.Generator(device=dev).manual_seed(7)
    act = lambda n: torch.randn(n, generator=gen, device=dev).to(torch.bfloat16)
    x = {H: act(H), F: act(F), qd: act(qd)}
    resid = act(max(H, F))
    y = torch.empty(max(qkv, F, shape.vocab), dtype=torch.bfloat16, device=dev)
    g = dm.w["final_norm"]
    eps = shape.rms_eps
    sub = dm.substitute_layers
    shared = [l for l in range(shape.n_layers) if l not in sub]
    # site: (struct field, k, rows out, norm prologue, epilogue, per-step count, symbol)
    spec = {
        "qkv": ("qkv", H, qkv, True, 0, "gemv_kernel<{r},{w},1,0>"),
        "o": ("o", qd, H, False, 1, "gemv_kernel<{r},{w},0,1>"),
        "gate_up": ("gate_up", H, F, True, 2, "gemv_kernel<{r},{w},1,2>"),
        "down": ("down", F, H, False, 1, "gemv_kernel<{r},{w},0,1>"),
    }
    # rows per wave as the library picks them (the gate/up GEMVs take one gate and one up row)
    rows_per_wave = lambda n, silu, w4: (2 if silu else 4 if n >= 16384 else (2 if n >= 4096 else 1))

    def timed(lins, k, n_out, norm, epi):
        run = lambda lin: _lib.gemv(lin, x[k], y, norm_w=g if norm else None, eps=eps, epilogue=epi,
                                    resid=resid if epi == 1 else None)
        for lin in lins:
            run(lin)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if not graph:
            e0.record()
            for _ in range(reps):
                for lin in lins:
                    run(lin)
            e1.record()
            torch.cuda.synchronize()
            return 1000.0 * e0.elapsed_time(e1) / (reps * len(lins))
        # captured in a HIP graph, so that the launches reach the GPU faster
        # than the kernels run (host launch cost would otherwise bound the
        # small ones)
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            for _ in range(reps):
                for lin in lins:
                    run(lin)
        cg.replay()
        torch.cuda.synchronize()
        e0.record()
        cg.replay()
        e1.record()
        torch.cuda.synchronize()
        del cg
        return 1000.0 * e0.elapsed_time(e1) / (reps * len(lins))

    out = {}
    for kind, layers in (("w4", sub), ("bf16", shared)):
        if not layers:
            continue
        for site, (name, k, n_out, norm, epi, sym) in spec.items():
            if only and only != f"{kind}_{site}":
                continue
            w4 = kind == "w4"
            mats = [dm.q[l][name] if w4 else (dm.w["layers"][l][name],) for l in layers]
            lay = dm.layout[layers[0]][name] if w4 else 0
            wb = n_out * (2 if epi == 2 else 1) * k * (0.5 + 4 / 64 if w4 else 2.0)
            copies = [tuple(t.clone() for t in m) for _ in range(int((1 << 30) // (wb * len(mats))))
                      for m in mats]
            lins = [_lib.linear(codes=m[0], meta=m[1], layout=lay) if w4 else _lib.linear(w=m[0])
                    for m in mats + copies]
            by = wb + 2 * k + 2 * n_out * (2 if epi == 1 else 1)
            us = timed(lins, k, n_out, norm, epi)
            del copies, lins
            r = rows_per_wave(n_out, epi == 2, w4)
            if lay:  # the tiled GEMV: <width, tiles, chunks in flight, x items per thread, prologue, epilogue>
                nx = next(v for v in (1, 2, 3, 5, 7) if v * 8 * 512 >= k)
                tp = "1,4" if epi == 1 else ("2,3" if epi == 0 else "2,2")
                symbol = f"gemv_w4t_kernel<4,{tp},{nx},{1 if norm else 0},{epi},0>"
            else:
                symbol = sym.format(r=r, w="4" if w4 else "16")
            out[f"{kind}_{site}"] = {"avg_us": round(us, 3), "bytes_per_launch": round(by),
                                     "gbs": round(by / (us * 1e-6) / 1e9, 1), "per_step": len(layers),
                                     "symbol": symbol}
    if only and only != "lm_head":
        return out
    lm = _lib.linear(w=dm.w["lm_head"])
    by = 2.0 * shape.vocab * H + 2 * H + 2 * shape.vocab
    us = timed([lm], H, shape.vocab, True, 0)
    out["lm_head"] = {"avg_us": round(us, 3), "bytes_per_launch": round(by),
                      "gbs": round(by / (us * 1e-6) / 1e9, 1), "per_step": 1,
                      "symbol": "gemv_kernel<4,16,1,0>"}
    return out


def replay_us(fn, reps=20):
    """fn's launches recorded once in a HIP graph, then the graph replayed
    `reps` times between two HIP events on the replay stream: microseconds per
    replay (no host launch cost inside the timed region)."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    del g
    return 1000.0 * e0.elapsed_time(e1) / reps


def hbm(bytes_, us, label, **extra):
    gbs = bytes_ / (us * 1e-6) / 1e9
    out = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": label, "avg_us": round(us, 3),
           "bytes_per_launch": round(bytes_)}
    out.update(extra)
    return out


def model_bytes(shape, draft_w4_layers, kv_positions_draft, kv_positions_verify, bits=4):
    """Algorithmic bytes of one draft step and one verify pass: every weight
    read once (bf16 2 B; a `bits`-bit substitute bits/8 B + 4 B of fp16
    scale/min per 64 weights), the lm_head, and the K/V rows each attention
    reads once."""
    H, F = shape.hidden, shape.ffn
    qkv = (shape.n_q_heads + 2 * shape.n_kv_heads) * shape.head_dim
    qd = shape.n_q_heads * shape.head_dim
    per_layer = qkv * H + H * qd + 2 * F * H + H * F
    kv_row = 2 * shape.n_kv_heads * shape.head_dim * 2  # K + V bytes per position and layer
    lm = 2.0 * shape.vocab * H
    w4 = per_layer * (bits / 8 + 4 / 64)
    draft = (draft_w4_layers * w4 + (shape.n_layers - draft_w4_layers) * 2.0 * per_layer + lm
             + shape.n_layers * kv_positions_draft * kv_row)
    verify = shape.n_layers * 2.0 * per_layer + lm + shape.n_layers * kv_positions_verify * kv_row
    return draft, verify, w4, 2.0 * per_layer, kv_row


def pass_rates(dec, shape, wl, kv0, last, n_w4, sparse_keys=None):
    """tau-independent figures of the workload: one draft step (step 0 at the
    resident prompt state) and one verify pass, each graph-replayed; their
    algorithmic bytes over the replay time."""
    from self_speculative_decoding_w4a16_amd import _lib
    gamma = wl.gamma
    dec.reset(kv0, last)
    if sparse_keys is not None:
        dec.c.use_index = 1
    d_keys = (sparse_keys if sparse_keys is not None else kv0) + 1
    draft_b, verify_b, _, _, _ = model_bytes(shape, n_w4, d_keys, kv0 + gamma + 1)
    u = dec.ud_buf if wl.draft_temp > 0 else None
    t_d = replay_us(lambda: _lib.draft_step(dec.model.c, dec.c, 0, dec.draft_temp, u, dec.ws))
    # the same step with every layer's attention in a launch of its own
    dec.reset(kv0, last)
    dec.c.attn_own_launch = 1
    t_d_own = replay_us(lambda: _lib.draft_step(dec.model.c, dec.c, 0, dec.draft_temp, u, dec.ws))
    dec.c.attn_own_launch = 0
    dec.reset(kv0, last)
    t_v = replay_us(dec.verify)
    dec.reset(kv0, last)
    # matrix-core work of the verify pass: 2 flops per weight and position
    _, _, _, bf, _ = model_bytes(shape, n_w4, 0, 0)
    params = bf / 2 * shape.n_layers + shape.vocab * shape.hidden
    tflops = 2.0 * params * (gamma + 1) / (t_v * 1e-6) / 1e12
    draft = hbm(draft_b, t_d, "draft step (every launch of one draft token, graph-replayed)")
    draft["avg_us_attn_own_launch"] = round(t_d_own, 3)
    return (draft,
            hbm(verify_b, t_v, f"verify pass ({gamma + 1} positions, every launch, graph-replayed)",
                mfma_tflops=round(tflops, 2), mfma_frac=round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)))


def layer7b_rates(dev, gamma=16, ctx=1024):
    """One Qwen2.5-7B-shaped decoder layer with 1024 positions of bf16 KV: the
    4-bit substitute layer of a draft step and the bf16 layer of a 17-position
    verify pass.  Measured as the difference between graph-replayed draft
    steps (and verify passes) of a 5-layer and a 1-layer model of that shape
    (the lm_head, sampling and bookkeeping cancel), divided by 4; the five
    layers' weights are distinct (655 MB of W4, 2.3 GB of bf16), so the 256 MB
    last-level cache holds no layer's weights when it runs again."""
    import torch

    from self_speculative_decoding_w4a16_amd.engine import SpecDecoder
    from self_speculative_decoding_w4a16_amd.model import DeviceModel
    from synth import kv_history, model_weights
    from synth.configs import QWEN7B
    t = {}
    for L in (1, 5):
        shape = QWEN7B.with_(n_layers=L, n_shared=0)
        w = model_weights(shape, 70 + L, dev)
        dm = DeviceModel(shape, w)
        cap = ctx + gamma + 64
        dec = SpecDecoder(dm, cap, gamma, 0.0, 0.0, graphs=False)
        K, V = kv_history(L, shape.n_kv_heads, ctx, shape.head_dim, cap, 80 + L, dev)
        dec.load_kv(K, V, ctx, 7)
        del K, V
        from self_speculative_decoding_w4a16_amd import _lib
        t[L] = (replay_us(lambda: _lib.draft_step(dm.c, dec.c, 0, 0.0, None, dec.ws)),
                replay_us(dec.verify))
        del dec, dm, w
        torch.cuda.empty_cache()
    shape = QWEN7B.with_(n_layers=1, n_shared=0)
    _, _, w4, bf, kv_row = model_bytes(shape, 1, 0, 0)
    d_us, v_us = (t[5][0] - t[1][0]) / 4, (t[5][1] - t[1][1]) / 4
    return {"draft_w4_layer": hbm(w4 + (ctx + 1) * kv_row, d_us,
                                  "one W4 substitute layer of a draft step (GEMVs + attention + norms)"),
            "verify_layer": hbm(bf + (ctx + gamma + 1) * kv_row, v_us,
                                f"one bf16 layer of a {gamma + 1}-position verify pass"),
            "method": "(5-layer - 1-layer graph-replayed step) / 4, KV 1024 positions",
            "raw_us": {"draft_1": round(t[1][0], 2), "draft_5": round(t[5][0], 2),
                       "verify_1": round(t[1][1], 2), "verify_5": round(t[5][1], 2)}}


def lowbit_rates(dec, shape, w, wl, kv0, last, dev):
    """Substitutes at 3 and 2 bits (the paper note's substitute widths) on the
    same model and KV state: one graph-replayed draft step and the isolated
    gate/up and down GEMVs at each width, against their algorithmic bytes."""
    import torch

    from self_speculative_decoding_w4a16_amd import _lib
    from self_speculative_decoding_w4a16_amd.engine import SpecDecoder
    from self_speculative_decoding_w4a16_amd.model import DeviceModel
    out = {}
    H, F = shape.hidden, shape.ffn
    for bits in (3, 2):
        dm = DeviceModel(shape, w, bits=bits)
        d = SpecDecoder(dm, dec.capacity, wl.gamma, 0.0, 0.0, graphs=False)
        d.k_cache.copy_(dec.k_cache)
        d.v_cache.copy_(dec.v_cache)
        d.reset(kv0, last)
        n_sub = len(dm.substitute_layers)
        draft_b, _, layer_b, _, _ = model_bytes(shape, n_sub, kv0 + 1, kv0 + 1, bits=bits)
        us = replay_us(lambda: _lib.draft_step(dm.c, d.c, 0, 0.0, None, d.ws))
        sites = {}
        x = {H: torch.randn(H, device=dev).bfloat16(), F: torch.randn(F, device=dev).bfloat16()}
        y = torch.empty(F, dtype=torch.bfloat16, device=dev)
        g = dm.w["final_norm"]
        resid = torch.zeros(H, dtype=torch.bfloat16, device=dev)
        for site, k, nout, epi in (("gate_up", H, F, 2), ("down", F, H, 1)):
            lins = [dm.linear_d(l, site) for l in dm.substitute_layers]
            reps = max(1, int((1 << 30) // (n_sub * (2 if epi == 2 else 1) * nout * k * (bits / 8 + 4 / 64))))

            def run(lins=lins, k=k, epi=epi):
                for _ in range(reps):
                    for lin in lins:
                        _lib.gemv(lin, x[k], y, norm_w=g if epi == 2 else None, eps=1e-6, epilogue=epi,
                                  resid=resid if epi == 1 else None)
            t = replay_us(run, reps=2) / (reps * len(lins))
            by = (2 if epi == 2 else 1) * nout * k * (bits / 8 + 4 / 64) + 2 * k + 2 * nout * (2 if epi == 1 else 1)
            sites[site] = hbm(by, t, f"{bits}-bit {site} GEMV")
        out[f"w{bits}"] = {"draft_step": hbm(draft_b, us, f"draft step with {bits}-bit substitutes"),
                           "layer_weight_bytes": round(layer_b), **sites}
        del d, dm
        torch.cuda.empty_cache()
    return out


def adaptive_rates(dec, dm, wl, kv0, last, c, steps=2):
    """Greedy speculative decoding of the same workload with the entropy-
    adaptive draft length (gamma as the longest draft; c = measured draft-step
    over verify-pass time): tokens/s, tau and the mean draft length, cycles
    replayed from recorded graphs as in the headline run."""
    import time

    import numpy as np
    import torch

    from self_speculative_decoding_w4a16_amd import _lib
    from self_speculative_decoding_w4a16_amd.engine import SpecDecoder
    G = wl.generate
    d = SpecDecoder(dm, dec.capacity, wl.gamma, wl.temp, wl.draft_temp, graphs=True,
                    adaptive=dict(c=c, beta=0.125))
    d.k_cache.copy_(dec.k_cache)
    d.v_cache.copy_(dec.v_cache)

    def gen():
        d.reset(kv0, last)
        _lib.control_init(d.ctl)
        out, ns, gs = [], [], []
        while len(out) < G:
            d.cycle()
            n = int(d.n_accepted.item())
            out += d.out_tokens[:n + 1].tolist()
            ns.append(n)
            gs.append(d.last_draft_len())
        return out[:G], ns, gs
    gen()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    all_ns, all_gs = [], []
    for _ in range(steps):
        _, ns, gs = gen()
        all_ns += ns
        all_gs += gs
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    del d
    torch.cuda.empty_cache()
    return {"tokens_s": round(steps * G / el, 3), "tau": round(float(np.mean([n + 1 for n in all_ns])), 4),
            "mean_draft_len": round(float(np.mean(all_gs)), 3), "max_draft_len": wl.gamma, "c": round(c, 4),
            "beta": 0.125}


def batch_rates(dm, shape, dev):
    """The 4-bit skinny GEMM (matrix cores) that drafts m sequences at once on
    shared substitutes, at the gate/up and down shapes of the substitute
    layers, m = 1, 4, 8, 16: microseconds per launch (graph-replayed over all
    substitute layers, >= 1 GiB a round) and the weight stream's rate; the
    per-token weight bytes fall as 1/m."""
    import torch

    from self_speculative_decoding_w4a16_amd import _lib
    H, F = shape.hidden, shape.ffn
    out = {}
    sub = dm.substitute_layers
    for site, k, n in (("gate_up", H, 2 * F), ("down", F, H)):
        lins = [dm.linear_d(l, site) for l in sub]
        wb = n * k * (0.5 + 4 / 64)
        reps = max(1, int((1 << 30) // (wb * len(lins))))
        for m in (1, 4, 8, 16):
            x = torch.randn(m, k, device=dev).bfloat16()
            y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
            buf = torch.zeros(_lib.w4_gemm_workspace_bytes(n, k, m), dtype=torch.uint8, device=dev)

            def run():
                for _ in range(reps):
                    for lin in lins:
                        _lib.w4_gemm(lin, x, y, buf)
            us = replay_us(run, reps=2) / (reps * len(lins))
            by = wb + 2 * m * (k + n)
            out[f"{site}_m{m}"] = {"avg_us": round(us, 3), "gbs": round(by / (us * 1e-6) / 1e9, 1),
                                   "frac": round(by / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                   "weight_bytes_per_token": round(wb / m)}
    return out


def tree_rates(dec, dm, shape, wl, kv0, last, k=6, depth=48, G=64, steps=1):
    """Greedy speculative decoding of the same model and prompt state with
    SubSpec's static tree, k = 6 chains of depth 48 ("SubSpec" report,
    sections 6.3 and 3.7): tokens/s and tau over graph-replayed cycles, and
    the tau-independent passes - one draft level (k rows through the draft in
    one weight stream) and the verify pass over all 1 + k D nodes (the GEMMs
    in slices of up to 128 positions), each graph-replayed, against their
    algorithmic bytes and the matrix-core peak."""
    import time

    import numpy as np
    import torch

    from self_speculative_decoding_w4a16_amd import _lib
    from self_speculative_decoding_w4a16_amd.engine import TreeDecoder
    nodes = 1 + k * depth
    cap = kv0 + G + nodes + 64
    t = TreeDecoder(dm, cap, k, depth, 0.0, 0.0, graphs=True)
    t.k_cache[:, :, :kv0].copy_(dec.k_cache[:, :, :kv0])
    t.v_cache[:, :, :kv0].copy_(dec.v_cache[:, :, :kv0])

    def gen():
        t.reset(kv0, last)
        out, ns = [], []
        while len(out) < G:
            t.cycle()
            n = int(t.n_accepted.item())
            out += t.out_tokens[:n + 1].tolist()
            ns.append(n)
        return ns
    gen()
    gen()  # the first cycle runs eagerly, the second records the graph
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    all_ns = []
    for _ in range(steps):
        all_ns += gen()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    n_w4 = len(dm.substitute_layers)
    t.reset(kv0, last)
    t.draft()  # a drafted tree in place for the pass timings
    lvl = replay_us(lambda: _lib.tree_draft(dm.c, t.c, k, depth, 1, 0.0, None, t.ws), reps=10)
    root = replay_us(lambda: _lib.tree_draft(dm.c, t.c, k, depth, 0, 0.0, None, t.ws), reps=10)
    ver = replay_us(t.verify, reps=5)
    draft_b, _, _, bf, kv_row = model_bytes(shape, n_w4, kv0 + 2, 0)
    _, verify_b, _, _, _ = model_bytes(shape, n_w4, 0, kv0 + nodes)
    params = bf / 2 * shape.n_layers + shape.vocab * shape.hidden
    tflops = 2.0 * params * nodes / (ver * 1e-6) / 1e12
    del t
    torch.cuda.empty_cache()
    return {"k": k, "depth": depth, "nodes": nodes, "tokens_s": round(steps * G / el, 3),
            "tau": round(float(np.mean([n + 1 for n in all_ns])), 4), "cycles": len(all_ns),
            "cycle_ms": round(1000 * el / len(all_ns), 3),
            "draft_level": hbm(draft_b, lvl, f"one tree draft level ({k} rows, every launch, graph-replayed)"),
            "draft_root": hbm(draft_b, root, "the tree's root level (1 row, every launch, graph-replayed)"),
            "verify_pass": hbm(verify_b, ver, f"tree verify pass ({nodes} positions, every launch, graph-replayed)",
                               mfma_tflops=round(tflops, 1),
                               mfma_frac=round(tflops / BF16_MFMA_PEAK_TFLOPS, 4))}


def batch_decode_rates(dm, w, shape, wl, dev, G=32, batches=(1, 2, 4, 8, 16)):
    """Batched decoding of B sequences on the same model (the SubSpec
    report's open question of where sharing the substitutes among 2-8 users
    stops paying, section 10.3, item 11): greedy speculative decoding with
    gamma = 16 (graph-replayed cycles) against plain batched bf16
    autoregressive decoding (graph-replayed steps), total tokens/s over all B
    sequences, B random prompts of the workload's prompt length."""
    import time

    import numpy as np
    import torch

    from self_speculative_decoding_w4a16_amd import _lib
    from self_speculative_decoding_w4a16_amd.engine import BatchDecoder
    from self_speculative_decoding_w4a16_amd.model import DeviceModel
    from synth import token_ids
    full = DeviceModel(shape, w, substitute_layers=[])
    P, gamma = wl.prompt, wl.gamma
    cap = P + G + 2 * (gamma + 1) + 64
    out = {}
    for B in batches:
        prompts = [[int(t) for t in token_ids(P, shape.vocab, 900 + b)] for b in range(B)]
        d = BatchDecoder(dm, B, cap, gamma, graphs=True)
        d.generate(prompts, gamma + 1)  # eager cycle, then the recorded graph
        d.generate(prompts, gamma + 1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks, ns = d.generate(prompts, G)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        emitted = sum(sum(n[b] + 1 for n in ns) for b in range(B))
        d.prefill(prompts)
        t_step = replay_us(lambda: _lib.batch_draft_step(dm.c, d.c, 0, 0.0, None, d.ws), reps=10)
        d.prefill(prompts)
        t_ver = replay_us(d.verify, reps=5)
        del d
        a = BatchDecoder(full, B, cap, 1)
        a.prefill(prompts)
        t_ar = replay_us(a.ar_step, reps=G)
        del a
        torch.cuda.empty_cache()
        out[f"B{B}"] = {"spec_tokens_s": round(emitted / el, 2),
                        "tau": round(float(np.mean([n + 1 for c in ns for n in c])), 4),
                        "ar_tokens_s": round(B / (t_ar * 1e-6), 2),
                        "ar_step_us": round(t_ar, 1), "draft_step_us": round(t_step, 1),
                        "verify_pass_us": round(t_ver, 1)}
        log(f"batch B={B}: {json.dumps(out[f'B{B}'])}")
    del full
    torch.cuda.empty_cache()
    return out


def multilevel_rates(dec, dm, w, shape, wl, kv0, last, gamma2s=(4, 8), G=32):
    """Multi-level substitutes ("SubSpec" report, section 10.3, item 9):
    greedy decoding of the same model and prompt state in which a 2-bit
    substitute model drafts gamma2 tokens at a time for the 4-bit draft, whose
    gamma = 16 middle tokens the bf16 target verifies.  Eager host loop (one
    sync per inner round): tokens/s, the outer tau, the inner rounds' mean
    kept fraction n / g and rounds per cycle, and one 2-bit draft step
    (graph-replayed) against the 4-bit one."""
    import time

    import numpy as np
    import torch

    from self_speculative_decoding_w4a16_amd import _lib
    from self_speculative_decoding_w4a16_amd.engine import MultiLevelDecoder
    from self_speculative_decoding_w4a16_amd.model import DeviceModel
    dm2 = DeviceModel(shape, w, bits=2)
    gamma = wl.gamma
    out = {}
    for g2 in gamma2s:
        cap = kv0 + G + gamma + g2 + 64
        d = MultiLevelDecoder(dm, dm2, cap, gamma, g2)
        d.k_cache[:, :, :kv0].copy_(dec.k_cache[:, :, :kv0])
        d.v_cache[:, :, :kv0].copy_(dec.v_cache[:, :, :kv0])

        def gen():
            d.reset(kv0, last)
            n_out, ns, rounds = 0, [], []
            while n_out < G:
                d.cycle()
                n = int(d.n_accepted.item())
                n_out += n + 1
                ns.append(n)
                rounds.append(list(d.rounds))
            return ns, rounds
        gen()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ns, rounds = gen()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        kept = [n / g for rs in rounds for (_, g, n, _) in rs]
        d.reset(kv0, last)
        step2 = replay_us(lambda: _lib.draft_step(dm2.c, d.c2, 0, 0.0, None, d.ws), reps=10)
        step4 = replay_us(lambda: _lib.draft_step(dm.c, d.c, 0, 0.0, None, d.ws), reps=10)
        pass4 = replay_us(lambda: _lib.draft_verify(dm.c, d.c, 0, g2 + 1, d.tokens, d.mid_logits, d.ws), reps=10)
        out[f"gamma2_{g2}"] = {"tokens_s": round(sum(n + 1 for n in ns) / el, 3),
                               "tau": round(float(np.mean([n + 1 for n in ns])), 4),
                               "inner_kept_frac": round(float(np.mean(kept)), 4),
                               "inner_rounds_per_cycle": round(float(np.mean([len(r) for r in rounds])), 2),
                               "cycle_ms": round(1000 * el / len(ns), 3),
                               "draft_step_2bit_us": round(step2, 1), "draft_step_4bit_us": round(step4, 1),
                               "pass_4bit_us": round(pass4, 1)}
        log(f"multi-level gamma2={g2}: {json.dumps(out[f'gamma2_{g2}'])}")
        del d
        torch.cuda.empty_cache()
    del dm2
    torch.cuda.empty_cache()
    return out


def tiny_rates(dev, reps=200, oracle=True):
    """The tiny workload: one 512x512 W4 GEMV at batch 1 and one rejection round
    with V = 1000, gamma = 4.  Both are far too small to stream from HBM (the
    GEMV's 147 KB sit in cache): microseconds per call, back to back in a
    graph, and the GEMV's rate flagged as latency-bound."""
    import numpy as np
    import torch

    from self_speculative_decoding_w4a16_amd import _lib
    from synth import logits_pair, normal_tensor, uniform_codes
    n = k = 512
    w = normal_tensor((n, k), 0.02, 0, dev)
    x = normal_tensor((k,), 1.0, 1, dev)
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    meta = torch.empty((n, k // 64, 2), dtype=torch.float16, device=dev)
    _lib.quantize(w, codes, meta)
    y = torch.empty(n, dtype=torch.bfloat16, device=dev)

    def gemvs():
        for _ in range(reps):
            _lib.w4_gemv(codes, meta, n, k, x, y)
    us_g = replay_us(gemvs, reps=5) / reps
    gamma, V = 4, 1000
    zt, zd = logits_pair(gamma, V, 2, device=dev)
    Ud, _ = uniform_codes(gamma, 4)
    cv = lambda a: torch.tensor(np.asarray(a, np.int64).astype(np.int32), device=dev)
    toks, rr, uf = cv([int(t) for t in torch.argmax(zd.float(), dim=1).tolist()]), cv(Ud), cv([12345])
    n_out = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.zeros(gamma + 1, dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=dev)

    def rejects():
        for _ in range(50):
            _lib.reject(gamma, V, 1.0, 1.0, zt, zd, toks, rr, uf, n_out, out, st, None, ws)
    us_r = replay_us(rejects, reps=5) / 50
    gb = n * k * (0.5 + 4 / 64) + 2 * k + 2 * n
    out = {"w4_gemv_512x512_us": round(us_g, 3),
           "w4_gemv_512x512_gbs": round(gb / (us_g * 1e-6) / 1e9, 1), "latency_bound": True,
           "reject_v1000_gamma4_us": round(us_r, 3),
           "reject_bytes": 2 * (2 * gamma + 1) * V}
    if oracle:
        # the oracle on one host core, the same calls: dequantise + product, one round
        from threadpoolctl import threadpool_limits

        from oracle.model import linear
        from oracle.quant import dequantize, quantize
        from oracle.reject import reject as oreject
        host = lambda t: t.detach().float().cpu().numpy()
        wc, wm = quantize(host(w))
        xh = host(x).astype(np.float64)
        zth, zdh = host(zt), host(zd)
        th = [int(t) for t in toks.tolist()]

        def per_call_us(fn, n_calls):
            t0 = time.perf_counter()
            for _ in range(n_calls):
                fn()
            return 1e6 * (time.perf_counter() - t0) / n_calls
        with threadpool_limits(1):
            o_g = per_call_us(lambda: linear(xh, dequantize(wc, wm)), 5)
            o_r = per_call_us(lambda: oreject(zth, zdh, th, list(Ud), 12345, 1.0, 1.0), 20)
        out["cpu_baseline"] = {"kind": "oracle", "cores": 1, "w4_gemv_512x512_us": round(o_g, 1),
                               "reject_v1000_gamma4_us": round(o_r, 1),
                               "sample": "the same two calls on one host core (5 and 20 calls)"}
    return out


class OracleSample:
    """The oracle, untuned (NumPy float64), on bounded samples at the
    workload's full shapes: host copies of one shared bf16 layer (if the model
    has any), one substitute layer (4, 3 or 2 bits) and the lm_head, over a
    synthetic KV history.  Every timing is the median of `reps` runs; `spent`
    sums the CPU time of all of them."""

    def __init__(self, shape, w, wl):
        import numpy as np

        from oracle.model import OracleModel
        from synth import kv_history, token_ids
        try:
            from threadpoolctl import threadpool_info
            self.cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # noqa: BLE001
            self.cores = os.cpu_count()
        self.host = lambda t: t.detach().float().cpu().numpy()
        log("oracle sample: copying sampled layers to host")
        self.shape, self.wl, self.w = shape, wl, w
        S = shape.n_shared
        self.base = dict(n_layers=0, hidden=shape.hidden, ffn=shape.ffn, n_q_heads=shape.n_q_heads,
                         n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim, vocab=shape.vocab,
                         rope_theta=shape.rope_theta, rms_eps=shape.rms_eps, embed=self.host(w["embed"]),
                         final_norm=self.host(w["final_norm"]), lm_head=self.host(w["lm_head"]), layers=[])
        self.lm = OracleModel(**self.base)
        self.shared = None
        if S > 0:
            self.shared = self._one_layer(0)
        self.sub = {}
        t0 = time.perf_counter()
        self.sub[4] = self._one_layer(S, bits=4)
        self.t_quant = time.perf_counter() - t0
        self.kv_len = max(wl.prompt, 600)
        self.cap = self.kv_len + wl.gamma + 2
        K, V = kv_history(1, shape.n_kv_heads, self.kv_len, shape.head_dim, self.cap, 44, "cpu")
        self.K, self.V = self.host(K).astype(np.float64), self.host(V).astype(np.float64)
        self.K0 = np.zeros((0, shape.n_kv_heads, self.cap, shape.head_dim))
        self.toks = [int(t) for t in token_ids(max(wl.gamma + 1, 64), shape.vocab, 45)]
        self.spent = 0.0

    def _one_layer(self, l, bits=None):
        from oracle.model import OracleModel
        m = OracleModel(**{**self.base, "n_layers": 1,
                           "layers": [{k: self.host(v) for k, v in self.w["layers"][l].items()}]})
        if bits:
            m.make_substitutes([0], bits=bits)
        return m

    def substitute(self, bits):
        if bits not in self.sub:
            self.sub[bits] = self._one_layer(self.shape.n_shared, bits=bits)
        return self.sub[bits]

    def kv(self):
        return (self.K.copy(), self.V.copy())

    def timed(self, fn, reps=3):
        ts = []
        for _ in range(reps):
            t = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t)
        self.spent += sum(ts)
        return sorted(ts)[len(ts) // 2]

    def draft_step_s(self, bits=4, reps=3, sparse=None):
        """One draft token through the whole model: shared layers at the
        shared layer's time, substitute layers at the sampled one's."""
        from oracle.model import forward
        L, S = self.shape.n_layers, self.shape.n_shared
        if not hasattr(self, "_t_lm1"):
            self._t_lm1 = self.timed(lambda: forward(self.lm, (self.K0, self.K0), self.kv_len, self.toks[:1],
                                                     draft=True), reps)
            self._t_sh1 = self.timed(lambda: forward(self.shared, self.kv(), self.kv_len, self.toks[:1],
                                                     draft=True), reps) if self.shared else 0.0
        m = self.substitute(bits)
        t_sub = self.timed(lambda: forward(m, self.kv(), self.kv_len, self.toks[:1], draft=True, sparse=sparse),
                           reps)
        self.sub_layer_s = {**getattr(self, "sub_layer_s", {}), bits: max(t_sub - self._t_lm1, 0)}
        return S * max(self._t_sh1 - self._t_lm1, 0) + (L - S) * max(t_sub - self._t_lm1, 0) + self._t_lm1

    def rows_pass_s(self, rows, draft, bits=4, reps=1, lm_rows=None):
        """`rows` consecutive positions through the whole model (draft or
        target weights); the lm_head timed on lm_rows of them and scaled."""
        from oracle.model import forward
        L, S = self.shape.n_layers, self.shape.n_shared
        lm_rows = lm_rows or rows
        toks = (self.toks * (rows // len(self.toks) + 1))[:rows]
        t_lm = self.timed(lambda: forward(self.lm, (self.K0, self.K0), self.kv_len, toks[:lm_rows], draft=draft),
                          reps)
        t_sh = self.timed(lambda: forward(self.shared, self.kv(), self.kv_len, toks[:lm_rows], draft=draft),
                          reps) if self.shared else t_lm
        layer_sh = max(t_sh - t_lm, 0) * (rows / lm_rows)
        m = self.substitute(bits) if draft else (self.shared or self.substitute(bits))
        layer_sub = layer_sh
        if draft or not self.shared:
            t_sub = self.timed(lambda: forward(m, self.kv(), self.kv_len, toks[:lm_rows], draft=draft), reps)
            layer_sub = max(t_sub - t_lm, 0) * (rows / lm_rows)
        return S * layer_sh + (L - S) * layer_sub + t_lm * rows / lm_rows


def cpu_baseline(o, dm, wl, tau):
    """The headline's oracle line: a cycle is gamma draft steps (one draft
    token through one shared bf16 layer, one W4 substitute layer and the
    lm_head, scaled to the model) + one gamma+1-position verify (one layer and
    the lm_head, scaled) + one reject round, each the median of three runs at
    the workload's shapes and context length (synthetic KV; the long-context
    workload drafts over its sparse index and its verify also computes the
    importance scores); tokens/s = tau (of the GPU run) / cycle."""
    import numpy as np

    from oracle.model import forward
    from oracle.reject import reject
    from oracle.sparse import select_index
    from synth import logits_pair

    shape = o.shape
    gamma = wl.gamma
    L, S = shape.n_layers, shape.n_shared
    sparse, scores = None, None
    ex = wl.extra
    if "budget_permille" in ex:
        rng = np.random.default_rng(46)
        index = [[select_index(rng.random(o.kv_len), o.kv_len, ex["n_sink"], ex["n_recent"],
                               ex["budget_permille"]) for _ in range(shape.n_kv_heads)]]
        sparse, scores = (index, o.kv_len), []
    spent0 = o.spent
    t_draft = o.draft_step_s(4, sparse=sparse)
    toks = o.toks[:gamma + 1]
    t_lm = o.timed(lambda: forward(o.lm, (o.K0, o.K0), o.kv_len, toks, draft=False))
    t_v = o.timed(lambda: forward(o.shared or o.sub[4], o.kv(), o.kv_len, toks, draft=False, scores=scores))
    zt, zd = logits_pair(gamma, shape.vocab, 46)
    zt, zd = o.host(zt), o.host(zd)
    am = [int(np.argmax(zt[i])) for i in range(gamma)]
    t_rej = o.timed(lambda: reject(zt, zd, am, [0] * gamma, 0, wl.temp, wl.draft_temp))
    t_verify = L * max(t_v - t_lm, 0) + t_lm
    o.verify_layer_s = max(t_v - t_lm, 0)
    cycle = gamma * t_draft + t_verify + t_rej
    sample_s = o.spent - spent0
    log(f"cpu baseline: draft step {t_draft:.2f}s, verify {t_verify:.2f}s, reject {t_rej:.2f}s "
        f"(sample {sample_s:.1f}s, quantise {o.t_quant:.1f}s)")
    layers = ("one shared bf16 layer, one W4 layer" if S else "one W4 layer")
    return {"value": round(tau / cycle, 6), "unit": "tokens/s", "cores": int(o.cores), "kind": "oracle",
            "sample": (f"oracle (NumPy float64) timed on {layers}, the lm_head and one reject "
                       f"round at full {shape.name} shapes over {o.kv_len} positions of KV, median "
                       f"of 3 runs each ({sample_s:.1f}s of CPU work in all), scaled to {L} layers and a gamma={gamma} "
                       f"cycle; tokens/s = tau of the GPU run / oracle cycle time"),
            "oracle_draft_step_s": round(t_draft, 3), "oracle_verify_s": round(t_verify, 3),
            "oracle_reject_s": round(t_rej, 3), "_cycle_parts": (t_draft, t_verify, t_rej)}


def oracle_beside(o, cpu, wl, layer, lowbit, batch, bdec, tree, mlev, adapt):
    """The oracle beside every widened row, on bounded samples at the 7B
    shapes (one run each; the headline's draft step, verify and reject
    from cpu_baseline): the static tree's cycle (48 draft levels of 6 rows,
    one 289-node verify with the lm_head timed on 8 rows and scaled, the
    tree's round at the full vocabulary), the 3- and 2-bit draft steps, the
    4-bit skinny GEMM at m = 8 (dequantise + product), batched decoding
    (the oracle decodes the sequences one by one: its tokens/s is the
    headline's), multi-level substitutes (the GPU run's inner rounds per
    cycle of gamma2 2-bit steps and one 4-bit pass of gamma2 + 1 rows) and
    the adaptive length (the GPU run's mean draft length)."""
    import numpy as np

    from oracle.model import linear
    from oracle.quant import dequantize
    from oracle.tree import n_nodes, node, tree_forward, tree_reject
    from synth import logits_pair, normal_tensor, token_ids, uniform_codes
    shape = o.shape
    L, S = shape.n_layers, shape.n_shared
    t_draft, t_verify, t_rej = cpu["_cycle_parts"]
    note = lambda s0: f"{o.spent - s0:.1f}s of CPU work"
    if layer:
        layer["cpu_baseline"] = {"kind": "oracle", "cores": int(o.cores),
                                 "draft_w4_layer_s": round(o.sub_layer_s[4], 4),
                                 "verify_layer_s": round(o.verify_layer_s, 4),
                                 "sample": (f"the headline's oracle samples: one W4 layer of a draft step and one "
                                            f"layer of a {wl.gamma + 1}-position verify at {o.kv_len} KV positions, "
                                            f"median of 3")}
    if lowbit:
        for bits in (3, 2):
            s0 = o.spent
            t = o.draft_step_s(bits, reps=1)
            lowbit[f"w{bits}"]["cpu_baseline"] = {"kind": "oracle", "cores": int(o.cores),
                                                  "draft_step_s": round(t, 3),
                                                  "sample": f"one {bits}-bit layer scaled to the model, {note(s0)}"}
    if batch:
        s0 = o.spent
        H, F = shape.hidden, shape.ffn
        codes, meta, bits = o.sub[4].substitute[0]["gate_up"]
        x = o.host(normal_tensor((8, H), 1.0, 61, "cpu")).astype(np.float64)
        t = o.timed(lambda: linear(x, dequantize(codes, meta, bits=bits)), reps=1)
        batch["cpu_baseline"] = {"kind": "oracle", "cores": int(o.cores), "gate_up_m8_s": round(t, 3),
                                 "sample": f"dequantise + product at {2 * F}x{H}, m = 8, {note(s0)}"}
    if bdec:
        bdec["cpu_baseline"] = {"kind": "oracle", "cores": int(o.cores), "unit": "tokens/s",
                                "value_per_sequence_cycle": cpu["value"],
                                "sample": "the oracle runs each sequence's plain cycle in turn: "
                                          "its tokens/s at every B is the headline's oracle line"}
    if tree:
        s0 = o.spent
        k, D = tree["k"], tree["depth"]
        nn = n_nodes(k, D)
        toks = [int(t) for t in token_ids(nn, shape.vocab, 47)]
        kvt = lambda: (np.concatenate([o.K, np.zeros((1, shape.n_kv_heads, nn, shape.head_dim))], axis=2),
                       np.concatenate([o.V, np.zeros((1, shape.n_kv_heads, nn, shape.head_dim))], axis=2))
        lvl_nodes = [node(c, 1, D) for c in range(k)]
        t_lm = o.timed(lambda: tree_forward(o.lm, (o.K0, o.K0), o.kv_len, lvl_nodes, toks[:k], D, draft=True),
                       reps=1)
        t_sub = o.timed(lambda: tree_forward(o.sub[4], kvt(), o.kv_len, lvl_nodes, toks[:k], D, draft=True),
                        reps=1)
        t_sh = o.timed(lambda: tree_forward(o.shared, kvt(), o.kv_len, lvl_nodes, toks[:k], D, draft=True),
                       reps=1) if o.shared else t_lm
        t_level = S * max(t_sh - t_lm, 0) + (L - S) * max(t_sub - t_lm, 0) + t_lm
        rows8 = list(range(8))
        t_vlm = o.timed(lambda: tree_forward(o.lm, (o.K0, o.K0), o.kv_len, rows8, toks[:8], D), reps=1)
        t_v1 = o.timed(lambda: tree_forward(o.shared or o.sub[4], kvt(), o.kv_len, list(range(nn)), toks, D,
                                            logit_rows=rows8), reps=1)
        t_tverify = L * max(t_v1 - t_vlm, 0) + t_vlm * nn / 8
        zt, zd = logits_pair(nn - 1, shape.vocab, 48)
        zt, zd = o.host(zt), o.host(zd)
        zt = np.concatenate([zt, zt[:1]])[:nn]
        R, _ = uniform_codes(k + D - 1, 49)
        t_trej = o.timed(lambda: tree_reject(zt, zd[:1 + k * (D - 1)], toks, k, D, list(R), 5, 0.0, 0.0), reps=1)
        cycle = D * t_level + t_tverify + t_trej
        tree["cpu_baseline"] = {"kind": "oracle", "cores": int(o.cores), "unit": "tokens/s",
                                "value": round(tree["tau"] / cycle, 6), "draft_level_s": round(t_level, 3),
                                "verify_pass_s": round(t_tverify, 3), "reject_s": round(t_trej, 4),
                                "sample": (f"one draft level ({k} rows) through one shared and one W4 layer "
                                           f"and the lm_head, the {nn}-node verify through one layer (lm_head on "
                                           f"8 rows, scaled), the tree's round at V = {shape.vocab}; scaled to "
                                           f"{L} layers and a {D}-level cycle; tokens/s = tau of the GPU run / "
                                           f"oracle cycle; {note(s0)}")}
    if mlev:
        s0 = o.spent
        t2 = o.draft_step_s(2, reps=1)
        out = {}
        for key, r in mlev.items():
            g2 = int(key.split("_")[1])
            t_pass = o.rows_pass_s(g2 + 1, draft=True, bits=4, reps=1)
            cycle = r["inner_rounds_per_cycle"] * (g2 * t2 + t_pass) + t_verify + t_rej
            out[key] = {"value": round(r["tau"] / cycle, 6), "pass_4bit_s": round(t_pass, 3)}
        mlev["cpu_baseline"] = {"kind": "oracle", "cores": int(o.cores), "unit": "tokens/s",
                                "draft_step_2bit_s": round(t2, 3), **out,
                                "sample": (f"one 2-bit draft step and one 4-bit pass per inner round (one layer "
                                           f"each, scaled), the GPU run's rounds per cycle, the headline's verify "
                                           f"and reject; {note(s0)}")}
    if adapt:
        cycle = adapt["mean_draft_len"] * t_draft + t_verify + t_rej
        adapt["cpu_baseline"] = {"kind": "oracle", "cores": int(o.cores), "unit": "tokens/s",
                                 "value": round(adapt["tau"] / cycle, 6),
                                 "sample": "the headline's oracle step times at the GPU run's mean draft length"}



if __name__ == "__main__":
    main()
