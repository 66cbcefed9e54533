"""rocprofv3 recipes and summaries for the kernels of libpa.

    python -m paged_kv_cache_77_amd.profiling commands [OUTDIR]
        prints the rocprofv3 runs (one MI355X, repository root) whose
        outputs the summary reads: per workload a kernel trace of bench.py
        and one counter run each for FETCH_SIZE and WRITE_SIZE, plus the two
        counters over a plain 1 GiB device copy for calibration.
    python -m paged_kv_cache_77_amd.profiling summarize [OUTDIR] [PROFILES]
        reads OUTDIR/*_results.db (rocpd SQLite) and the bench JSON lines
        captured next to them, writes one short text summary per workload
        into PROFILES and PROFILES/traffic.json (HBM bytes per launch of the
        dominant kernel, tagged with the kernel sources' hash so bench.py
        ignores figures taken on other sources).

Counters: FETCH_SIZE and WRITE_SIZE are KiB per dispatch; the copy
calibration gives the factor that turns each into bytes (a 1 GiB copy reads
and writes 1 GiB).  Dispatches are grouped by kernel name and grid: the
summary of a kernel is the group with the largest total time (the launches
bench.py times; e.g. the prefill-only launches of the mixed batch leave
tiny decode dispatches that are reported separately).
"""
from __future__ import annotations

import json
import os
import sqlite3
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# workload -> bench arguments, kernels whose traffic makes the roofline
# figure(s), and the traffic.json keys bench.py reads
RUNS = {
    "batched_decode": {
        "title": "batched decode: 64 requests, contexts U[512,4096], 32 q / 8 KV heads, "
                 "head_dim 128, bf16; step = pa_decode_append (each request's new K/V row "
                 "written by its decode work-groups, then the single-pass decode), one launch",
        "args": "--config 2",
        "keys": {"config2_append": ["pa::decode_kernel"]},
    },
    "long_context_split": {
        "title": "long-context split-KV decode: 8 requests x 32768 tokens, 32 q / 8 KV heads, "
                 "head_dim 128, bf16, 512-token partitions, then the merge",
        "args": "--config 3",
        "keys": {"config3_split": ["pa::decode_kernel"]},
    },
    "mixed_chunked_prefill": {
        "title": "mixed batch: 128 decode rows (contexts U[1024,8192]) + a 2048-token chunk on "
                 "a 6144-token prefix, 32 q / 8 KV heads, head_dim 128, bf16; step = fused write "
                 "of 2176 tokens, then pa_prefill_varlen (one launch: the chunk's MFMA "
                 "prefill items, then the decode rows)",
        "args": "--config 4",
        "keys": {"config4_varlen": ["pa::varlen_kernel"],
                 "config4_prefill": ["pa::prefill_kernel"]},
        # matrix-core counters (derived metrics of rocprofv3): MfmaUtil = the
        # share of SIMD cycles the MFMA pipe was busy, MfmaFlopsBF16 = bf16
        # MFMA flops executed
        "counters": {"counters": ["MfmaUtil", "MfmaFlopsBF16"],
                     "kernels": ["pa::prefill_kernel", "pa::varlen_kernel"]},
    },
    "shared_prefix_fp8": {
        "title": "shared-prefix fp8 decode: 256 requests sharing 256 blocks (4096 tokens) + "
                 "tails U[64,1024], 28 q / 4 KV heads, head_dim 128, fp8 e4m3 K/V; "
                 "pa_decode_shared_prefix (prefix partials on the matrix cores, tails by "
                 "split-KV, merge)",
        "args": "--config 5",
        "keys": {"config5_shared": ["pa::shared_prefix_kernel", "pa::decode_mfma_kernel",
                                    "pa::merge_few_kernel"]},
        "counters": {"counters": ["MfmaUtil", "MfmaFlopsBF16", "MfmaFlopsF16"],
                     "kernels": ["pa::shared_prefix_kernel", "pa::decode_mfma_kernel"]},
    },
    "shared_prefix_fp8_per_request": {
        "title": "the same workload through the per-request decode (pa_decode, matrix-core "
                 "kernel)",
        "args": "--config 5 --path single",
        "keys": {"config5_single": ["pa::decode_mfma_kernel"]},
    },
    "shared_prefix_fp8_vector_alu": {
        "title": "the same workload on the vector-ALU kernel (the work-balanced decode, which "
                 "always runs there): the A/B for the matrix-core decode of FP8 caches",
        "args": "--config 5 --path balanced",
        "keys": {"config5_balanced": ["pa::decode_balanced_kernel",
                                      "pa::balanced_merge_kernel"]},
        # VALUBusy = % of the time the vector ALUs were busy
        "counters": {"counters": ["VALUBusy"], "kernels": ["pa::decode_balanced_kernel"],
                     "what": "vector-ALU counter per dispatch (median over the group): "
                             "VALUBusy = % of the time the vector ALUs were busy"},
    },
}

BENCH = "python3 bench.py --no-cpu-baseline --no-other-workloads"


def commands(outdir: str = "rocprof_out") -> list:
    """The rocprofv3 command lines (run from the repository root)."""
    cmds = []
    for name, r in RUNS.items():
        cmds.append(f"rocprofv3 --kernel-trace --stats -d {outdir} -o trace_{name} -- "
                    f"{BENCH} {r['args']} --steps 20 --warmup 5 > {outdir}/trace_{name}.json")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            cmds.append(f"rocprofv3 --pmc {c} -d {outdir} -o {c.lower()}_{name} -- "
                        f"{BENCH} {r['args']} --steps 3 --warmup 1")
        if "counters" in r:
            cmds.append(f"rocprofv3 --pmc {' '.join(r['counters']['counters'])} -d {outdir} "
                        f"-o counters_{name} -- {BENCH} {r['args']} --steps 3 --warmup 1")
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cmds.append(f"rocprofv3 --pmc {c} -d {outdir} -o {c.lower()}_copy -- "
                    f"python3 bench.py --copy-calibration")
    return cmds


def _short(name: str) -> str:
    n = name[5:] if name.startswith("void ") else name
    return n.split("(")[0]


def _groups(db: str, counter: str = None) -> dict:
    """(short name, grid) -> list of (duration ns, counter value or None)."""
    con = sqlite3.connect(db)
    cur = con.cursor()
    out = {}
    if counter is None:
        rows = cur.execute("select name, grid_x, grid_y, grid_z, duration from kernels")
        for n, gx, gy, gz, d in rows:
            out.setdefault((_short(n), (gx, gy, gz)), []).append((d, None))
    else:
        grids = {did: (gx, gy, gz) for did, gx, gy, gz in
                 cur.execute("select dispatch_id, grid_x, grid_y, grid_z from kernels")}
        rows = cur.execute("select name, dispatch_id, duration, counter_value from pmc_events "
                           "where counter_name = ?", (counter,))
        for n, did, d, v in rows:
            out.setdefault((_short(n), grids.get(did)), []).append((d, v))
        # without dispatch records, keep each kernel's long dispatches only
        for k in [k for k in out if k[1] is None]:
            dmax = max(d for d, _ in out[k])
            out[k] = [(d, v) for d, v in out[k] if d >= 0.5 * dmax]
    con.close()
    return out


def _per_dispatch(db: str, counter: str) -> dict:
    """(short name, grid) -> list of (duration ns, counter summed over the
    dispatch's instances) -- rocprofv3 stores some derived counters once per
    dispatch and others once per hardware instance."""
    con = sqlite3.connect(db)
    cur = con.cursor()
    grids = {did: (gx, gy, gz) for did, gx, gy, gz in
             cur.execute("select dispatch_id, grid_x, grid_y, grid_z from kernels")}
    out = {}
    rows = cur.execute("select name, dispatch_id, max(duration), sum(counter_value) from "
                       "pmc_events where counter_name = ? group by dispatch_id", (counter,))
    for n, did, d, v in rows:
        out.setdefault((_short(n), grids.get(did)), []).append((d, v))
    con.close()
    return out


def _dominant(groups: dict, prefix: str):
    """The (name, grid) group of kernels starting with prefix with the most total time."""
    cand = [(sum(d for d, _ in v), k) for k, v in groups.items() if k[0].startswith(prefix)]
    return max(cand)[1] if cand else None


def _calibration(outdir: str) -> tuple:
    f = _groups(os.path.join(outdir, "fetch_size_copy_results.db"), "FETCH_SIZE")
    w = _groups(os.path.join(outdir, "write_size_copy_results.db"), "WRITE_SIZE")
    kf = _dominant(f, "__amd_rocclr_copyBuffer")
    kw = _dominant(w, "__amd_rocclr_copyBuffer")
    fk = statistics.median(v for _, v in f[kf])
    wk = statistics.median(v for _, v in w[kw])
    gib = float(1 << 30)
    return gib / (fk * 1024.0), gib / (wk * 1024.0), fk, wk


def summarize(outdir: str = "rocprof_out", profiles: str = "profiles") -> dict:
    sys.path.insert(0, ROOT)
    from bench import kernel_source_sha       # the hash bench.py checks
    sha = kernel_source_sha()
    ff, wf, fk, wk = _calibration(outdir)
    traffic = {}
    for name, r in RUNS.items():
        trace = _groups(os.path.join(outdir, f"trace_{name}_results.db"))
        fetch = _groups(os.path.join(outdir, f"fetch_size_{name}_results.db"), "FETCH_SIZE")
        write = _groups(os.path.join(outdir, f"write_size_{name}_results.db"), "WRITE_SIZE")
        bench_line = None
        jp = os.path.join(outdir, f"trace_{name}.json")
        if os.path.exists(jp):
            for line in open(jp):
                if line.startswith("{"):
                    bench_line = json.loads(line)
        cmds = [c for c in commands(outdir) if f"_{name} " in c or f"_{name} --" in c
                or c.endswith(f"trace_{name}.json")]
        lines = [f"# {name}: {r['title']}",
                 "# commands (repository root, one MI355X, ROCm 7.2 rocprofv3; summary by "
                 "`python -m paged_kv_cache_77_amd.profiling summarize`):"]
        lines += [f"#   {c}" for c in cmds]
        lines += [f"#   calibration: {c}" for c in commands(outdir)[-2:]]
        lines.append(f"# kernel sources sha {sha}")
        lines.append("# kernel trace, dispatches grouped by kernel and grid (microseconds):")
        for k, v in sorted(trace.items(), key=lambda kv: -sum(d for d, _ in kv[1])):
            ds = [d / 1e3 for d, _ in v]
            lines.append(f"{k[0]:55s} grid {str(k[1]):18s} calls {len(ds):4d}  "
                         f"avg {statistics.mean(ds):9.3f}  median {statistics.median(ds):9.3f}")
        lines.append("# HBM counters per dispatch (median over the group), converted to bytes "
                     f"with the copy calibration (FETCH x{ff:.3f}, WRITE x{wf:.3f}):")
        for key, prefixes in r["keys"].items():
            tot = 0.0
            for pfx in prefixes:
                kf, kw = _dominant(fetch, pfx), _dominant(write, pfx)
                fv = statistics.median(v for _, v in fetch[kf])
                wv = statistics.median(v for _, v in write[kw])
                b = fv * 1024 * ff + wv * 1024 * wf
                tot += b
                kt = _dominant(trace, pfx)
                avg_us = statistics.mean(d for d, _ in trace[kt]) / 1e3
                lines.append(f"{kf[0]:55s} grid {str(kf[1]):18s} FETCH {fv:12.1f} KiB  "
                             f"WRITE {wv:10.1f} KiB  -> {b / 1e6:10.2f} MB/launch  "
                             f"trace avg {avg_us:9.3f} us")
            traffic[key] = {"bytes_per_launch": int(round(tot)), "kernel_sha": sha,
                            "kernels": prefixes}
            lines.append(f"# {key}: HBM traffic {tot / 1e6:.2f} MB per launch")
        if "counters" in r:
            db = os.path.join(outdir, f"counters_{name}_results.db")
            lines.append("# " + r["counters"].get(
                "what", "matrix-core counters per dispatch (median over the group): "
                        "MfmaUtil = % of SIMD cycles the MFMA pipe was busy, "
                        "MfmaFlopsBF16 = bf16 MFMA flops executed"))
            vals = {c: _per_dispatch(db, c) for c in r["counters"]["counters"]}
            for pfx in r["counters"]["kernels"]:
                parts = []
                for c, g in vals.items():
                    k = _dominant(g, pfx)
                    if k is not None:
                        parts.append(f"{c} {statistics.median(v for _, v in g[k]):.4g}")
                if parts:
                    lines.append(f"{pfx:55s} " + "  ".join(parts))
        if bench_line is not None:
            rl = bench_line["roofline"]
            lines.append(f"# bench.py (same run, HIP events): kernel {rl['kernel_ms'] * 1e3:.3f} us, "
                         f"algorithmic {rl['algorithmic_bytes_per_launch'] / 1e6:.2f} MB/launch, "
                         f"{rl['achieved']:.1f} GB/s = {rl['frac']:.4f} of {rl['peak']:.0f}")
            if "served_GBps" in rl:
                lines.append(f"# bench.py: served (every request's reads) "
                             f"{rl['served_bytes_per_launch'] / 1e6:.2f} MB/launch, "
                             f"{rl['served_GBps']:.1f} GB/s")
            for extra in ("prefill_roofline", "compute_roofline"):
                if extra in bench_line:
                    e = bench_line[extra]
                    lines.append(f"# bench.py {extra}: {e['achieved']} {e['unit']} = "
                                 f"{e['frac']} of {e['peak']}")
        lines.append(f"# calibration: 1 GiB copy -> FETCH_SIZE {fk:.1f} KiB, WRITE_SIZE "
                     f"{wk:.1f} KiB per dispatch")
        path = os.path.join(profiles, f"{name}.txt")
        with open(path, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(f"wrote {path}")
    with open(os.path.join(profiles, "traffic.json"), "w") as fh:
        json.dump(traffic, fh, indent=1, sort_keys=True)
    print(f"wrote {os.path.join(profiles, 'traffic.json')}")
    return traffic


if __name__ == "__main__":
    mode = sys.argv[1] if len(sys.argv) > 1 else "commands"
    if mode == "commands":
        print("\n".join(commands(*(sys.argv[2:3] or []))))
    elif mode == "summarize":
        summarize(*sys.argv[2:4])
    else:
        raise SystemExit(__doc__)
