"""Summarise a rocprofv3 ``--kernel-trace --stats`` output directory.

Usage: python -m self_speculative_decoding_w4a16_amd.rocprof_summary DIR [TOP]
       python -m self_speculative_decoding_w4a16_amd.rocprof_summary --counters DIR [REGEX]

Prints one row per kernel (calls, total ms, average / min / max microseconds,
share of GPU time), with the library's template kernels named by the launch
site they serve (for example ``gemv_kernel<2, 16, 1, 2, 256>`` is the bf16
gate/up GEMV with the RMSNorm prologue and the SiLU*up epilogue, 256-thread
blocks; ``gemm_kernel<2, 2, 3>`` the verify GEMM with 2-wave blocks, up to 32
positions, writing split-k partial sums).

With --counters: a ``--pmc`` run's per-dispatch counter values (mean, min,
max over the dispatches of each kernel whose name matches REGEX).
"""
import csv
import glob
import re
import sys

_PRO = {0: "x", 1: "norm", 2: "embed+norm"}
_EPI = {0: "store", 1: "resid", 2: "silu*up", 3: "logits"}
_GEPI = {0: "store", 1: "resid", 2: "silu*up", 3: "split-k partials"}


def describe(name):
    """Short name and launch role of one kernel symbol."""
    m = re.search(r"gemv_kernel<(\d+), (\d+|true|false), (\d+), (\d+)(?:, (\d+))?>", name)
    if m:
        r, wb, pro, epi = int(m[1]), m[2], int(m[3]), int(m[4])
        width = {"16": "bf16", "false": "bf16", "4": "W4", "true": "W4", "3": "W3", "2": "W2"}.get(wb, wb)
        nt = f",{m[5]}" if m[5] else ""
        return (f"gemv_kernel<{r},{wb},{pro},{epi}{nt}>",
                f"{width} GEMV, {r} rows/wave, {_PRO.get(pro, pro)} -> {_EPI.get(epi, epi)}")
    m = re.search(r"gemv_w4t_kernel<(\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)>", name)
    if m:
        wb, t, p, nx, pro, epi, dqr = (int(v) for v in m.groups())
        role = (f"W{wb} GEMV on 16-row tiles (matrix cores), {t} tile(s)/unit, {p} chunks in flight, "
                f"{_PRO.get(pro, pro)} -> {_EPI.get(epi, epi)}")
        if dqr:
            role += f", with the layer's draft attention in the same launch ({dqr} K/V chunk(s) a wave)"
        return f"gemv_w4t_kernel<{wb},{t},{p},{nx},{pro},{epi},{dqr}>", role
    m = re.search(r"gemm_w4_kernel<(true|false), (true|false), (true|false)>", name)
    if m:
        tl, half = m[2] == "true", m[3] == "true"
        return (f"gemm_w4_kernel<{m[1]},{m[2]},{m[3]}>",
                "W4 skinny GEMM (matrix cores, " + ("<= 8" if half else "<= 16") + " positions" +
                (", tiled" if tl else "") + "), " +
                ("SiLU*up epilogue" if m[1] == "true" else "store / split-k partials"))
    m = re.search(r"gemm_kernel<(\d+), (\d+), (\d+)>", name)
    if m:
        nw, tt, epi = int(m[1]), int(m[2]), int(m[3])
        return (f"gemm_kernel<{nw},{tt},{epi}>",
                f"MFMA GEMM, {nw}-wave blocks, <= {16 * tt} positions, {_GEPI.get(epi, epi)}")
    short = name.replace("(anonymous namespace)::", "")
    short = re.sub(r"\(.*$", "", short)
    short = re.sub(r"^void ", "", short)
    base = re.sub(r"<.*$", "", short)
    return short[:60], _ROLES.get(base, "")


_ROLES = {
    "draft_attn_head_kernel": "draft attention: RoPE, KV append, key splits per head, last block merges",
    "draft_attn_kernel": "draft attention: RoPE, KV append, 64-key split partials",
    "draft_merge_kernel": "draft attention: merge of the split partials",
    "rows_attn_kernel": "verify attention: per-row split partials",
    "rows_attn_long_kernel": "verify attention, long context: several key tiles per block",
    "rows_merge_kernel": "verify attention: merge of many split partials (8 groups per block)",
    "rows_merge_seq_kernel": "verify attention: merge of the split partials",
    "hbm_read_kernel": "HBM read ceiling (read-only stream, measurement)",
    "tile_codes_kernel": "low-bit codes + meta into 16-row tiles (model set-up)",
    "rope_append_kernel": "verify RoPE + KV append (sums QKV split-k partials)",
    "rmsnorm_rows_kernel": "verify residual add of split-k partials + RMSNorm",
    "gemm_reduce_kernel": "lm_head split-k reduction",
    "sample_kernel": "draft token sampling (argmax / exact inverse CDF)",
    "pos_guard_kernel": "draft step position check + RoPE table",
    "rope_table_kernel": "verify RoPE table",
    "rej_rowmax_kernel": "rejection: per-row max / argmax",
    "rej_decide_kernel": "rejection: exact accept / resample decision",
    "kv_rollback_kernel": "KV rollback (kv_len += accepted + 1)",
    "embed_rows_kernel": "verify embedding gather",
    "attn_scores_kernel": "sparse draft: importance scores",
    "kv_select_kernel": "sparse draft: index rebuild (radix select)",
    "w4_quantize_kernel": "W4 g64 quantiser",
    "quantize_kernel": "low-bit g64 quantiser",
    "draft_control_kernel": "adaptive draft length: entropy + stop decision",
    "control_update_kernel": "adaptive draft length: EMA centres",
    "rej_rowsum_kernel": "rejection: fixed-point row sums",
    "rows_sample_kernel": "tree / batch: per-row argmax or exact draw (one block per row)",
    "tree_root_kernel": "tree: the root's multi-step rejection + the accepted chain's round",
    "tree_commit_kernel": "tree: accepted chain's K/V moved next to the prefix",
    "silu_rows_kernel": "rows forward: SiLU(gate) * up (split-k gate/up)",
    "batch_rollback_kernel": "batched decoding: per-sequence KV rollback",
    "token_append_kernel": "multi-level: a round's last token appended",
    "zero_kernel": "fill (arrival counters)",
}


def load(path):
    files = glob.glob(path + "/**/*kernel_stats.csv", recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {path}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def main(argv):
    path = argv[1]
    top = int(argv[2]) if len(argv) > 2 else 30
    rows = load(path)
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print(f"{'kernel':34s} {'calls':>8s} {'total ms':>10s} {'avg us':>9s} {'min us':>9s} "
          f"{'max us':>9s} {'share':>7s}  role")
    for r in rows[:top]:
        short, role = describe(r["Name"])
        t = float(r["TotalDurationNs"])
        print(f"{short:34s} {int(r['Calls']):8d} {t / 1e6:10.3f} {float(r['AverageNs']) / 1e3:9.2f} "
              f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
              f"{100 * t / total:6.2f}%  {role}")
    print(f"total GPU kernel time {total / 1e6:.3f} ms over {sum(int(r['Calls']) for r in rows)} launches")


def counters(path, regex=".*"):
    """Per-dispatch counter values of a --pmc run, per kernel and counter."""
    files = glob.glob(path + "/**/*counter_collection.csv", recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {path}")
    vals = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or r.get("KernelName") or ""
            if not re.search(regex, name):
                continue
            key = (describe(name)[0], r.get("Counter_Name") or r.get("Counter-Name") or "")
            vals.setdefault(key, {}).setdefault(r.get("Dispatch_Id") or r.get("Dispatch-Id"), 0.0)
            vals[key][r.get("Dispatch_Id") or r.get("Dispatch-Id")] += float(r.get("Counter_Value") or 0.0)
    print(f"{'kernel':34s} {'counter':14s} {'dispatches':>10s} {'mean':>14s} {'min':>14s} {'max':>14s}")
    for (k, c), d in sorted(vals.items()):
        v = list(d.values())
        print(f"{k:34s} {c:14s} {len(v):10d} {sum(v) / len(v):14.1f} {min(v):14.1f} {max(v):14.1f}")


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--counters":
        counters(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ".*")
    else:
        main(sys.argv)
