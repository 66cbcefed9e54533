"""Measure the decode paths against each other on the current GPU.

    python -m paged_kv_cache_77_amd.tune_dispatch [--hq 32 --hkv 8 --d 128]
    python -m paged_kv_cache_77_amd.tune_dispatch --summarize SWEEP.txt [...]

For a grid of batch sizes R and (equal) context lengths L it times, with HIP
events on the launch stream (median of repeated launches), the single-pass
decode and the split-KV decode + merge at several partition sizes, and
prints one line per (R, L) with the fastest path.  --summarize reads such
output (host only) and prints, per cell, the time of the path the library's
plan (pa_decode_plan_for) picks and of the path the pages' V1/V2 condition
picks ("vLLM 深度解析（二）" §3.3: V1 iff max_seq_len <= 8192 and (one
partition or num_seqs * num_heads > 512), partitions of 512), each against
the fastest measured path.  The selection rule of pa_decode_plan_for
(csrc/pa_api.hip) was set from these tables on MI355X, which are kept
under profiles/.  Inputs are random, timing only (the
values do not affect the kernels' work).
"""
from __future__ import annotations

import argparse
import json
import sys

import torch

import paged_kv_cache_77_amd as pa


def _time(fn, reps: int) -> float:
    s = torch.cuda.current_stream()
    for _ in range(3):
        fn()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn()
        b.record(s)
        ts.append((a, b))
    torch.cuda.synchronize()
    v = sorted(x.elapsed_time(y) * 1e3 for x, y in ts)
    return v[len(v) // 2]


def measure(R: int, L: int, hq: int, hkv: int, d: int, parts=(256, 512, 1024), reps=15):
    nbr = -(-L // 16)
    nb = R * nbr
    lay = pa.make_layout(nb, hkv, d, pa.PA_CACHE_BF16)
    k = torch.randn((nb, hkv, 16, d), dtype=torch.bfloat16, device="cuda")
    v = torch.randn_like(k)
    q = torch.randn((R, hq, d), dtype=torch.bfloat16, device="cuda")
    bt = torch.randperm(nb, device="cuda", dtype=torch.int64).to(torch.int32).view(R, nbr)
    sl = torch.full((R,), L, dtype=torch.int32, device="cuda")
    out = torch.empty((R, hq, d), dtype=torch.bfloat16, device="cuda")
    res = {"R": R, "L": L,
           "single": _time(lambda: pa.pa_decode(lay, out, q, k, v, bt, sl, L, 0.088), reps)}
    for P in parts:
        pm = -(-L // P)
        tmp = torch.empty((R, hq, pm, d), dtype=torch.float32, device="cuda")
        ml = torch.empty((R, hq, pm), dtype=torch.float32, device="cuda")
        es = torch.empty_like(ml)

        def split():
            pa.pa_decode_partitioned(lay, q, k, v, bt, sl, L, 0.088, P, tmp, ml, es)
            pa.pa_merge_partitions(out, tmp, ml, es, sl, P)
        res[f"split{P}"] = _time(split, reps)
    del k, v
    torch.cuda.empty_cache()
    best = min((x for x in res if x not in ("R", "L")), key=lambda x: res[x])
    res["best"] = best
    return res


def pages_rule(R: int, L: int, hq: int) -> str:
    pmax = -(-L // 512)
    return "single" if (L <= 8192 and (pmax == 1 or R * hq > 512)) else "split512"


def summarize(paths) -> None:
    for path in paths:
        lines = open(path).read().splitlines()
        head = lines[0]
        hq = int(head.split("Hq ")[1].split(",")[0])
        hkv = int(head.split("Hkv ")[1].split(",")[0])
        d = int(head.split(" d ")[1].split(",")[0])
        rows = [json.loads(x) for x in lines if x.startswith("{")]
        print(head)
        print(f"{'R':>4} {'L':>6} {'best':>10} {'best_us':>9} {'plan':>10} {'plan_us':>9} "
              f"{'pages':>10} {'pages_us':>9}")
        tot = {"best": 0.0, "plan": 0.0, "pages": 0.0}
        for r in rows:
            lay = pa.make_layout(r["R"] * -(-r["L"] // 16), hkv, d, pa.PA_CACHE_BF16)
            plan = pa.pa_decode_plan_for(lay, r["R"], hq, r["L"])
            mine = f"split{plan.partition_size}" if plan.split else "single"
            theirs = pages_rule(r["R"], r["L"], hq)
            b = r[r["best"]]
            tot["best"] += b
            tot["plan"] += r[mine]
            tot["pages"] += r[theirs]
            print(f"{r['R']:4d} {r['L']:6d} {r['best']:>10} {b:9.2f} {mine:>10} {r[mine]:9.2f} "
                  f"{theirs:>10} {r[theirs]:9.2f}")
        print(f"# sum over cells: fastest {tot['best']:.1f} us, plan {tot['plan']:.1f} us "
              f"(+{100 * (tot['plan'] / tot['best'] - 1):.1f}%), pages' condition "
              f"{tot['pages']:.1f} us (+{100 * (tot['pages'] / tot['best'] - 1):.1f}%)")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--summarize", nargs="+", default=None)
    ap.add_argument("--hq", type=int, default=32)
    ap.add_argument("--hkv", type=int, default=8)
    ap.add_argument("--d", type=int, default=128)
    ap.add_argument("--max-tokens", type=int, default=1 << 21)
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return 0
    pa.lib()
    print(f"# decode paths, Hq {args.hq}, Hkv {args.hkv}, d {args.d}, bf16; median us "
          f"per call (split = partitions + merge)", flush=True)
    for R in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512):
        for L in (256, 512, 1024, 2048, 4096, 8192, 16384, 32768):
            if R * L > args.max_tokens:
                continue
            r = measure(R, L, args.hq, args.hkv, args.d)
            print(json.dumps({k: (round(v, 2) if isinstance(v, float) else v)
                              for k, v in r.items()}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
