"""Summarise rocprofv3 result databases (rocpd SQLite) into the short text tables kept
under profiles/.

  python -m latent_decode_attention_lla_amd.rocprof_summary kernels RUN_results.db
  python -m latent_decode_attention_lla_amd.rocprof_summary traffic \
      --fetch F.db --write W.db --copy-fetch CF.db --copy-write CW.db \
      --copy-bytes N --kernel decode_rotary_fold --out traffic.json

``counters`` prints every counter of a --pmc run averaged per dispatch, for the kernels
whose names contain one of the given fragments:

  python -m latent_decode_attention_lla_amd.rocprof_summary counters RUN_results.db \
      --kernel decode_rotary_fold

``waves`` turns two counter passes of one kernel (between them: SQ_WAVES, SQ_WAVE_CYCLES,
SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_INSTS_VALU, SQ_INSTS_SALU, SQ_INSTS_MFMA, SQ_INSTS_LDS,
SQ_LDS_BANK_CONFLICT, SQ_ACTIVE_INST_LDS, SQ_LDS_IDX_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES,
GRBM_GUI_ACTIVE) into the wave-state evidence bench.py reports for a call bound by neither
roof. SQ_WAVE_CYCLES and the SQ_WAIT_* / SQ_ACTIVE_INST_* counters are in quad-cycles
summed over waves; SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE are cycles summed over CUs,
SQ_VALU_MFMA_BUSY_CYCLES cycles summed over SIMDs, GRBM_GUI_ACTIVE the dispatch's GPU
cycles. The bank-conflict figures follow rocprofv3's own derived metrics (LDSBankConflict:
percent of the dispatch's cycles a CU's LDS is stalled by conflicts; LdsBankConflict:
conflict cycles per conflict-free LDS cycle):

  python -m latent_decode_attention_lla_amd.rocprof_summary waves --p1 A.db --p2 B.db \
      --kernel decode_lla2d --call decode --workload lla2d_long --out counters.json

``traffic`` scales the per-dispatch FETCH_SIZE and WRITE_SIZE (KiB) of the named kernel by
what the same counters read for a plain device copy of N bytes read and N bytes written
(the copy kernel whose counters are largest in the copy runs), and reports HBM bytes per
launch. ``--kernel`` takes comma-separated name fragments; with ``--sum`` the per-dispatch
averages of every kernel matching one of them are added (the kernels one API call
launches once each, e.g. the key and value encodes, or a split decode and its combine).
"""

from __future__ import annotations

import argparse
import json
import sqlite3
import sys


def kernel_table(db: str):
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, count(*), avg(duration), sum(duration), min(duration), max(duration) "
        "from kernels group by name order by sum(duration) desc").fetchall()
    total = sum(r[3] for r in rows) or 1
    return [{"kernel": r[0], "calls": r[1], "avg_us": r[2] / 1e3, "total_ms": r[3] / 1e6,
             "min_us": r[4] / 1e3, "max_us": r[5] / 1e3, "pct": 100.0 * r[3] / total} for r in rows]


def counter_per_kernel(db: str, counter: str):
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, value from counters_collection where counter_name = ?",
                       (counter,)).fetchall()
    agg = {}
    for name, v in rows:
        agg.setdefault(name, []).append(float(v))
    return {k: (len(v), sum(v) / len(v)) for k, v in agg.items()}


def _pick(agg: dict, sub: str, add: bool = False):
    subs = [x for x in sub.split(",") if x]
    hits = [(k, v) for k, v in agg.items() if any(x in k for x in subs)]
    if not hits:
        raise SystemExit(f"no kernel matching {sub!r}")
    if not add:
        return max(hits, key=lambda kv: kv[1][1])
    hits.sort()
    return (" + ".join(k for k, _ in hits),
            (min(v[0] for _, v in hits), sum(v[1] for _, v in hits)))


def derive(c: dict, cus: int, xccs: int) -> dict:
    """Per-wave and per-cycle figures from one dispatch's summed counters. The dispatch's
    GPU cycles are GRBM_GUI_ACTIVE over the XCDs (the database holds its sum over them,
    rocprofv3's derived metrics take the largest)."""
    waves = c.get("SQ_WAVES") or 1.0
    res = {"wave_wait_frac": c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"],
           "wave_issue_wait_frac": c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"],
           "valu_insts_per_wave": (c["SQ_INSTS_VALU"] - c.get("SQ_INSTS_MFMA", 0.0)) / waves,
           "mfma_insts_per_wave": c.get("SQ_INSTS_MFMA", 0.0) / waves,
           "salu_insts_per_wave": c["SQ_INSTS_SALU"] / waves}
    gpu = c.get("GRBM_GUI_ACTIVE", 0.0) / xccs
    if gpu > 0 and "SQ_LDS_BANK_CONFLICT" in c:
        res["lds_bank_conflict_pct"] = 100.0 * c["SQ_LDS_BANK_CONFLICT"] / gpu / cus
    if "SQ_LDS_IDX_ACTIVE" in c and c["SQ_LDS_IDX_ACTIVE"] > c.get("SQ_LDS_BANK_CONFLICT", 0.0):
        res["lds_conflicts_per_access"] = c["SQ_LDS_BANK_CONFLICT"] / (c["SQ_LDS_IDX_ACTIVE"] - c["SQ_LDS_BANK_CONFLICT"])
    if gpu > 0 and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        res["mfma_busy_frac"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gpu * 4 * cus)
    return res


def main(argv=None):
    p = argparse.ArgumentParser()
    sp = p.add_subparsers(dest="cmd", required=True)
    k = sp.add_parser("kernels")
    k.add_argument("db")
    k.add_argument("--top", type=int, default=12)
    cn = sp.add_parser("counters")
    cn.add_argument("db")
    cn.add_argument("--kernel", required=True)
    wv = sp.add_parser("waves")
    wv.add_argument("--p1", required=True)
    wv.add_argument("--p2", required=True)
    wv.add_argument("--kernel", required=True)
    wv.add_argument("--call", required=True)
    wv.add_argument("--workload", required=True)
    wv.add_argument("--path", default="auto", help="decode path the bench run forced")
    wv.add_argument("--cus", type=int, default=256, help="compute units of the device")
    wv.add_argument("--xccs", type=int, default=8, help="XCDs of the device")
    wv.add_argument("--out")
    t = sp.add_parser("traffic")
    for name in ("fetch", "write", "copy-fetch", "copy-write"):
        t.add_argument(f"--{name}", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--sum", action="store_true")
    t.add_argument("--out")
    t.add_argument("--extra", default="{}", help="JSON merged into the output")
    t.add_argument("--call", choices=["decode", "absorbed", "encode", "encode_fused", "teacher",
                                      "reconstruct", "paged"],
                   help="with --workload: record the call's source hash and algorithmic bytes")
    t.add_argument("--workload")
    t.add_argument("--path", default="auto", help="decode path the bench run forced")
    a = p.parse_args(argv)
    if a.cmd == "kernels":
        rows = kernel_table(a.db)
        print("| calls | avg us | min us | max us | total ms | % | kernel |")
        print("|---:|---:|---:|---:|---:|---:|---|")
        for r in rows[:a.top]:
            print(f"| {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | {r['max_us']:.2f} | "
                  f"{r['total_ms']:.3f} | {r['pct']:.2f} | `{r['kernel'][:120]}` |")
        return
    if a.cmd == "counters":
        con = sqlite3.connect(a.db)
        names = [r[0] for r in con.execute("select distinct counter_name from counters_collection")]
        subs = [x for x in a.kernel.split(",") if x]
        print("| counter | per dispatch | dispatches | kernel |")
        print("|---|---:|---:|---|")
        for c in sorted(names):
            for k, (n, v) in sorted(counter_per_kernel(a.db, c).items()):
                if any(x in k for x in subs):
                    print(f"| {c} | {v:.4g} | {n} | `{k[:100]}` |")
        return
    if a.cmd == "waves":
        import os
        sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        import bench
        c = {}
        kname = None
        for n in ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_INSTS_VALU",
                  "SQ_INSTS_SALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
                  "SQ_ACTIVE_INST_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES",
                  "GRBM_GUI_ACTIVE"):
            for db in (a.p1, a.p2):  # each counter is taken from whichever pass holds it
                try:
                    kname, (_, v) = _pick(counter_per_kernel(db, n), a.kernel)
                except SystemExit:
                    continue
                c[n] = v
                break
        res = {"kernel": kname, "counters_per_dispatch": c,
               "call": a.call, "workload": a.workload, "path": a.path,
               "kernel_source_hash": bench.kernel_source_hash(a.call, kname)}
        res.update(derive(c, a.cus, a.xccs))
        txt = json.dumps(res, indent=1)
        if a.out:
            with open(a.out, "w") as f:
                f.write(txt + "\n")
        print(txt)
        return
    fk, (fn, fv) = _pick(counter_per_kernel(a.fetch, "FETCH_SIZE"), a.kernel, a.sum)
    wk, (wn, wv) = _pick(counter_per_kernel(a.write, "WRITE_SIZE"), a.kernel, a.sum)
    ck, (_, cf) = max(counter_per_kernel(a.copy_fetch, "FETCH_SIZE").items(), key=lambda kv: kv[1][1])
    cw_k, (_, cw) = max(counter_per_kernel(a.copy_write, "WRITE_SIZE").items(), key=lambda kv: kv[1][1])
    f_scale = a.copy_bytes / (cf * 1024.0)
    w_scale = a.copy_bytes / (cw * 1024.0)
    res = {
        "kernel": fk,
        "dispatches_fetch": fn, "dispatches_write": wn,
        "fetch_kib_per_dispatch": fv, "write_kib_per_dispatch": wv,
        "copy_kernel": ck, "copy_write_kernel": cw_k, "copy_bytes": a.copy_bytes,
        "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "hbm_read_bytes_per_launch": fv * 1024.0 * f_scale,
        "hbm_write_bytes_per_launch": wv * 1024.0 * w_scale,
    }
    res["hbm_bytes_per_launch"] = res["hbm_read_bytes_per_launch"] + res["hbm_write_bytes_per_launch"]
    if a.call and a.workload:
        import os
        sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        import bench
        from latent_decode_attention_lla_amd.inputs import WORKLOADS
        w = WORKLOADS[a.workload]
        _, n_new, _ = bench.step_shape(w)
        if a.call == "reconstruct":
            alg, _ = bench.algorithmic(w, "reconstruct", L=w.T, n_new=n_new)
        elif a.call == "encode_fused":
            alg, _ = bench.algorithmic(w, "encode_fused", n_new=n_new)
        else:
            alg, _ = bench.algorithmic(w, "encode" if a.call == "encode" else "decode", n_new=n_new)
        res.update({"call": a.call, "workload": a.workload, "path": a.path,
                    "kernel_source_hash": bench.kernel_source_hash(a.call, fk),
                    "algorithmic_bytes_per_launch": alg,
                    "traffic_over_algorithmic": res["hbm_bytes_per_launch"] / alg})
    res.update(json.loads(a.extra))
    txt = json.dumps(res, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(txt + "\n")
    print(txt)


if __name__ == "__main__":
    sys.exit(main())
