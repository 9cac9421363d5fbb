"""Summarise a rocprofv3 ``--kernel-trace --stats`` output directory.

Usage: python -m self_speculative_decoding_w4a16_amd.rocprof_summary DIR [TOP]

Prints one row per kernel (calls, total ms, average / min / max microseconds,
share of GPU time), with the library's template kernels named by the launch
site they serve (for example ``gemv_kernel<4, false, 1, 2>`` is the bf16
gate/up GEMV with the RMSNorm prologue and the SiLU*up epilogue).
"""
import csv
import glob
import re
import sys

_PRO = {0: "x", 1: "norm", 2: "embed+norm", 3: "attn-merge"}
_EPI = {0: "store", 1: "resid", 2: "silu*up", 3: "logits"}
_GEPI = {0: "store", 1: "resid", 2: "silu*up"}


def describe(name):
    """Short name and launch role of one kernel symbol."""
    m = re.search(r"gemv_kernel<(\d+), (true|false), (\d+), (\d+)>", name)
    if m:
        r, w4, pro, epi = int(m[1]), m[2] == "true", int(m[3]), int(m[4])
        return (f"gemv_kernel<{r},{m[2]},{pro},{epi}>",
                f"{'W4' if w4 else 'bf16'} GEMV, {r} rows/wave, {_PRO[pro]} -> {_EPI[epi]}")
    m = re.search(r"gemm_kernel<(\d+), (\d+), (\d+)>", name)
    if m:
        rt, tt, epi = int(m[1]), int(m[2]), int(m[3])
        return (f"gemm_kernel<{rt},{tt},{epi}>",
                f"MFMA GEMM, {16 * rt} rows x <= {16 * tt} positions, {_GEPI[epi]}")
    short = name.replace("(anonymous namespace)::", "")
    short = re.sub(r"\(.*$", "", short)
    short = re.sub(r"^void ", "", short)
    return short[:60], ""


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


if __name__ == "__main__":
    main(sys.argv)
