"""Summaries of rocprofv3 runs of bench.py, written under profiles/.

    python -m top_sparse_attention_attn_amd.profile_summary CONFIG TRACE_DIR FETCH_DIR WRITE_DIR \
        COPY_FETCH_DIR COPY_WRITE_DIR OUT_MD [SQ_DIR TCC_DIR]

TRACE_DIR holds ``rocprofv3 --kernel-trace --stats --output-format csv`` output of
``bench.py --config CONFIG``; FETCH_DIR / WRITE_DIR hold ``--pmc FETCH_SIZE`` /
``--pmc WRITE_SIZE`` runs of the same command; COPY_*_DIR the same counters for
``bench.py --copy-calibration`` (a plain device copy of known size, which fixes the
scale of each counter). SQ_DIR / TCC_DIR, when given, hold ``--pmc MfmaUtil MfmaFlopsBF16
LdsBankConflict LdsUtil`` and ``--pmc TCC_HIT_sum TCC_MISS_sum TCC_REQ_sum`` runs of the same
command (MFMA busy fraction and bf16 MFMA work, LDS bank conflicts and busy fraction, L2 hits).
Writes OUT_MD (kernel times, counters, scaled HBM bytes) and
``profiles/counters_CONFIG.json``, which bench.py reads for ``roofline.traffic`` as long
as the kernel sources still hash to the value recorded there.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

COPY_BYTES = 256 << 20  # bench.py --copy-calibration copies 256 MiB, five times


def kernel_sources_sha256() -> str:
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _one(pattern: str) -> str:
    hits = glob.glob(pattern)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _ours(name: str) -> bool:
    return any(k in name for k in ("sparse_attn", "topk_bitmask", "masked_attn", "candidate_mask"))


def kernel_stats(trace_dir: str):
    rows = []
    for r in csv.DictReader(open(_one(os.path.join(trace_dir, "*kernel_stats.csv")))):
        if _ours(r["Name"]):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3))
    return rows


def timed_means(trace_dir: str, skip: int = 5) -> dict:
    """Mean duration (us) per kernel over its dispatches after the first `skip` (bench warmup)."""
    acc: dict = {}
    for r in csv.DictReader(open(_one(os.path.join(trace_dir, "*kernel_trace.csv")))):
        if _ours(r["Kernel_Name"]):
            acc.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {k: sum(v[skip:]) / max(1, len(v[skip:])) for k, v in acc.items()}


def counter_means(pmc_dir: str, counter: str, select) -> dict:
    acc: dict = {}
    for r in csv.DictReader(open(_one(os.path.join(pmc_dir, "*counter_collection.csv")))):
        if r["Counter_Name"] != counter or not select(r["Kernel_Name"]):
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _short(name: str) -> str:
    name = name.split("(")[0]
    return name.replace("void ", "").strip()


def main(argv):
    config, trace_dir, fetch_dir, write_dir, cfetch_dir, cwrite_dir, out_md = argv[:7]
    sq_dir, tcc_dir = (argv[7], argv[8]) if len(argv) >= 9 else (None, None)
    stats = kernel_stats(trace_dir)
    timed = timed_means(trace_dir)
    fetch = counter_means(fetch_dir, "FETCH_SIZE", _ours)
    write = counter_means(write_dir, "WRITE_SIZE", _ours)
    is_copy = lambda n: "copy" in n.lower() or "elementwise" in n.lower()  # noqa: E731
    cf = max(counter_means(cfetch_dir, "FETCH_SIZE", is_copy).values())
    cw = max(counter_means(cwrite_dir, "WRITE_SIZE", is_copy).values())
    ff, fw = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    dominant = max(stats, key=lambda r: r[2])[0]
    cmds = [
        f"rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace -o p -- python3 bench.py --config {config} --steps 50 --warmup 5 --no-cpu-baseline",
        f"rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d <out>/fetch -o p -- python3 bench.py --config {config} --steps 5 --warmup 2 --no-cpu-baseline",
        f"rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d <out>/write -o p -- python3 bench.py --config {config} --steps 5 --warmup 2 --no-cpu-baseline",
        "rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d <out>/copy_fetch -o p -- python3 bench.py --copy-calibration",
        "rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d <out>/copy_write -o p -- python3 bench.py --copy-calibration",
    ]
    if sq_dir:
        cmds += [
            f"rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 LdsBankConflict LdsUtil --kernel-trace --output-format csv -d <out>/sq "
            f"-o p -- python3 bench.py --config {config} --steps 5 --warmup 2 --no-cpu-baseline",
            f"rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum TCC_REQ_sum --kernel-trace --output-format csv -d <out>/tcc "
            f"-o p -- python3 bench.py --config {config} --steps 5 --warmup 2 --no-cpu-baseline"]
    cmds.append(f"python -m top_sparse_attention_attn_amd.profile_summary {config} <out>/trace <out>/fetch <out>/write "
                f"<out>/copy_fetch <out>/copy_write {os.path.relpath(out_md)}" + (" <out>/sq <out>/tcc" if sq_dir else ""))
    sha = kernel_sources_sha256()
    lines = [f"# rocprofv3 summary: bench.py --config {config}", "",
             "Commands (from the repository root on the GPU host, after `cd /tmp; export TMPDIR=/tmp`; "
             "`bench.py` stands for its absolute path):", "", "```"] + cmds + ["```", "",
             f"Kernel sources sha256: `{sha}`", "", "## Kernel trace", "",
             "| kernel | calls | avg us | avg us after the 5 warmup dispatches | min us | max us |",
             "|---|---|---|---|---|---|"]
    for n, c, a, mn, mx in stats:
        lines.append(f"| `{_short(n)}` | {c} | {a:.2f} | {timed.get(n, a):.2f} | {mn:.2f} | {mx:.2f} |")
    lines += ["", "## HBM bytes per launch (FETCH_SIZE / WRITE_SIZE, KiB per dispatch)", "",
              f"Plain 256 MiB copy: FETCH_SIZE {cf:.1f} KiB (scale {ff:.3f}), WRITE_SIZE {cw:.1f} KiB (scale {fw:.3f}).",
              "", "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB (scaled) |",
              "|---|---|---|---|---|"]
    for n in sorted(set(fetch) | set(write)):
        f, w = fetch.get(n, 0.0), write.get(n, 0.0)
        lines.append(f"| `{_short(n)}` | {f:.1f} | {w:.1f} | {f * 1024 * ff / 1e6:.2f} | {w * 1024 * fw / 1e6:.2f} |")
    units = {}
    if sq_dir:
        mu = counter_means(sq_dir, "MfmaUtil", _ours)
        mf = counter_means(sq_dir, "MfmaFlopsBF16", _ours)
        lb = counter_means(sq_dir, "LdsBankConflict", _ours)
        lu = counter_means(sq_dir, "LdsUtil", _ours)
        hit = counter_means(tcc_dir, "TCC_HIT_sum", _ours)
        miss = counter_means(tcc_dir, "TCC_MISS_sum", _ours)
        req = counter_means(tcc_dir, "TCC_REQ_sum", _ours)
        lines += ["", "## Compute units, LDS and L2 (per dispatch)", "",
                  "MFMA busy: `MfmaUtil` (MFMA busy cycles over all SIMDs / (GPU busy cycles x SIMDs)). "
                  "bf16 MFMA work: `MfmaFlopsBF16` (ops x 512), and that work over the kernel's average "
                  "duration against the 2500 TFLOP/s dense bf16 peak. LDS: `LdsBankConflict` (conflict "
                  "cycles per access) and `LdsUtil` (LDS busy share of CU cycles). L2: hits / (hits + misses).",
                  "", "| kernel | MFMA busy % | bf16 MFMA GFLOP | MFMA TFLOP/s (share of peak) | LDS conflicts/access "
                  "| LDS busy % | L2 requests (M) | L2 hit % |", "|---|---|---|---|---|---|---|---|"]
        for n in sorted(set(mu) | set(hit)):
            us = timed.get(n)
            fl = mf.get(n, 0.0)
            tf = fl / (us * 1e-6) / 1e12 if us else 0.0
            h, m = hit.get(n, 0.0), miss.get(n, 0.0)
            hr = 100.0 * h / (h + m) if h + m > 0 else 0.0
            lines.append(f"| `{_short(n)}` | {mu.get(n, 0.0):.1f} | {fl / 1e9:.2f} | {tf:.0f} ({tf / 2500:.3f}) | "
                         f"{lb.get(n, 0.0):.3f} | {lu.get(n, 0.0):.1f} | {req.get(n, 0.0) / 1e6:.2f} | {hr:.1f} |")
            units[n] = {"mfma_busy_pct": mu.get(n), "mfma_bf16_flop": fl, "mfma_tflops": tf,
                        "lds_conflicts_per_access": lb.get(n), "lds_busy_pct": lu.get(n), "l2_hit_pct": hr,
                        "l2_requests": req.get(n)}
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    rec = {"config": config, "kernel": _short(dominant), "source_sha256": sha,
           "fetch_kib_per_launch": fetch.get(dominant, 0.0), "write_kib_per_launch": write.get(dominant, 0.0),
           "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": COPY_BYTES,
           "avg_us": timed.get(dominant, max(stats, key=lambda r: r[2])[2]), "commands": cmds}
    if dominant in units:
        rec["units"] = units[dominant]
    jpath = os.path.join(os.path.dirname(os.path.abspath(out_md)), f"counters_{config}.json")
    with open(jpath, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"wrote {out_md} and {jpath}")


if __name__ == "__main__":
    main(sys.argv[1:])
