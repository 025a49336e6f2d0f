"""rocprofv3 summaries for the kernels of this package.

Turns rocprofv3 output databases (``-d DIR -o run`` writes ``DIR/**/run_results.db``)
into the short text summaries kept with the sources, and provides the plain
device copy used to calibrate the HBM byte counters.

    python -m fp4_quantized_moe_amd.profiling trace DIR --cmd "..." --out FILE
        per-kernel dispatch count and average / min / max duration (kernel trace)
    python -m fp4_quantized_moe_amd.profiling copy --mib 1024 --reps 4
        a plain device-to-device copy of a known size (run under rocprofv3 --pmc)
    python -m fp4_quantized_moe_amd.profiling traffic --kernel REGEX --family F --fetch DIR --write DIR \\
        --copy-fetch DIR --copy-write DIR --copy-mib 1024 --copy-reps 4 --cmd "..." --out FILE
        per-launch FETCH_SIZE / WRITE_SIZE of a kernel, each scaled by what the
        same counter reads for the copy (bytes known), plus the hash of the
        kernel's sources so that a stale figure can be recognised

The traffic summary is read back by ``bench.py`` (``read_traffic``).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import os
import re
import sqlite3
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))

# Sources that determine each kernel's memory traffic.
KERNEL_SOURCES = {
    "k_gemm": ["csrc/gemm.hip", "csrc/fp4_mfma.hpp", "csrc/quads_device.hpp", "csrc/launch.hpp"],
    "k_gemm_small": ["csrc/gemm_small.hip", "csrc/fp4_mfma.hpp", "csrc/quads_device.hpp", "csrc/launch.hpp"],
    "k_rac": ["csrc/rac.hip", "csrc/quads_device.hpp", "csrc/launch.hpp"],
    "k_quantize": ["csrc/quantize.hip", "csrc/quads_device.hpp", "csrc/launch.hpp"],
    "k_combine": ["csrc/route.hip", "csrc/launch.hpp"],
}


def _code_only(text: str) -> str:
    """C++ source without comments and blank space, so that editing a comment
    does not mark a profile as stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def sources_sha256(kernel_family: str) -> str:
    """Hash of the code (comments and spacing removed) of a kernel's sources."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel_family]:
        with open(os.path.join(PKG, rel)) as f:
            h.update(rel.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def _dbs(d):
    out = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not out:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return out


def _short(name: str) -> str:
    name = name.replace("quads::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    name = re.sub(r"^void ", "", name)
    return re.sub(r"\((?:[^()]|\([^()]*\))*\)$", "", name)  # drop the parameter list


def kernel_durations(d):
    """{kernel: [durations ns]} over every dispatch in the databases under d."""
    res = {}
    q = ("select s.display_name, d.end - d.start from rocpd_kernel_dispatch d "
         "join rocpd_info_kernel_symbol s on d.kernel_id = s.id")
    for db in _dbs(d):
        con = sqlite3.connect(db)
        for name, dt in con.execute(q):
            res.setdefault(_short(name), []).append(dt)
        con.close()
    return res


def kernel_counters(d):
    """{kernel: {counter: [value per dispatch]}} from a --pmc run."""
    q = ("select s.display_name, d.id, i.name, e.value from rocpd_pmc_event e "
         "join rocpd_info_pmc i on e.pmc_id = i.id join rocpd_event ev on e.event_id = ev.id "
         "join rocpd_kernel_dispatch d on d.event_id = ev.id "
         "join rocpd_info_kernel_symbol s on d.kernel_id = s.id")
    per = {}
    for db in _dbs(d):
        con = sqlite3.connect(db)
        for name, did, ctr, val in con.execute(q):
            per.setdefault(_short(name), {}).setdefault(ctr, {}).setdefault((db, did), 0.0)
            per[_short(name)][ctr][(db, did)] += val
        con.close()
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in per.items()}


def cmd_trace(a):
    durs = kernel_durations(a.dir)
    rows = sorted(durs.items(), key=lambda kv: -sum(kv[1]))
    lines = [f"# rocprofv3 kernel trace: {a.title}", "", "command (from the repository root):", "",
             f"    {a.cmd}", "",
             f"{'kernel':<72} {'calls':>6} {'avg us':>9} {'min us':>9} {'max us':>9} {'total ms':>9}"]
    for name, v in rows:
        lines.append(f"{name[:72]:<72} {len(v):>6} {statistics.mean(v) / 1e3:>9.2f} {min(v) / 1e3:>9.2f} "
                     f"{max(v) / 1e3:>9.2f} {sum(v) / 1e6:>9.3f}")
    _write(a.out, lines)


def _match(counters, regex):
    hits = {k: v for k, v in counters.items() if re.search(regex, k)}
    if len(hits) != 1:
        raise SystemExit(f"{regex!r} matches {sorted(hits)} (need exactly one kernel)")
    return next(iter(hits.items()))


def _per_dispatch(d, regex, counter):
    name, cs = _match(kernel_counters(d), regex)
    vals = cs.get(counter)
    if not vals:
        raise SystemExit(f"{counter} not recorded for {name} under {d}")
    return name, statistics.mean(vals), len(vals)


def _total(d, regex, counter):
    """Sum of `counter` over every dispatch of the kernels matching regex."""
    tot, n = 0.0, 0
    for name, cs in kernel_counters(d).items():
        if re.search(regex, name) and counter in cs:
            tot += sum(cs[counter])
            n += len(cs[counter])
    if n == 0:
        raise SystemExit(f"{counter} not recorded for {regex!r} under {d}")
    return tot, n


def cmd_traffic(a):
    copy_bytes = a.copy_mib * 2 ** 20 * a.copy_reps
    name, fetch_kib, nf = _per_dispatch(a.fetch, a.kernel, "FETCH_SIZE")
    _, write_kib, nw = _per_dispatch(a.write, a.kernel, "WRITE_SIZE")
    cfetch_kib, ncf = _total(a.copy_fetch, a.copy_kernel, "FETCH_SIZE")
    cwrite_kib, ncw = _total(a.copy_write, a.copy_kernel, "WRITE_SIZE")
    f_fetch = cfetch_kib * 1024 / copy_bytes
    f_write = cwrite_kib * 1024 / copy_bytes
    fetch_b = fetch_kib * 1024 / f_fetch
    write_b = write_kib * 1024 / f_write
    fam = a.family
    lines = [f"# HBM traffic per launch: {name}", "",
             "commands (`cd /tmp && export TMPDIR=/tmp` first; $REPO is the repository root):", ""]
    lines += [f"    {c}" for c in a.cmd]
    lines += ["",
              "Each counter is scaled by what it reads for a plain device copy of known size",
              f"({a.copy_reps} x {a.copy_mib} MiB: that many bytes read and written), i.e.",
              "bytes = counter_KiB * 1024 / (copy_counter_KiB * 1024 / copy_bytes).",
              "",
              f"kernel: {name}",
              f"dispatches: fetch {nf}, write {nw}",
              f"FETCH_SIZE_KiB_per_dispatch: {fetch_kib:.1f}",
              f"WRITE_SIZE_KiB_per_dispatch: {write_kib:.1f}",
              f"copy_bytes: {copy_bytes}",
              f"copy_dispatches: fetch {ncf}, write {ncw}",
              f"copy_FETCH_SIZE_KiB_total: {cfetch_kib:.1f}",
              f"copy_WRITE_SIZE_KiB_total: {cwrite_kib:.1f}",
              f"copy_factor_fetch: {f_fetch:.4f}",
              f"copy_factor_write: {f_write:.4f}",
              f"fetch_bytes_per_launch: {fetch_b:.0f}",
              f"write_bytes_per_launch: {write_b:.0f}",
              f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}"]
    if a.algorithmic_bytes:
        lines.append(f"algorithmic_bytes_per_launch: {a.algorithmic_bytes:.0f}")
        lines.append(f"traffic_over_algorithmic: {(fetch_b + write_b) / a.algorithmic_bytes:.3f}")
    lines += [f"source_family: {fam}",
              f"source_sha256: {sources_sha256(fam)}"]
    _write(a.out, lines)


def read_traffic(path: str):
    """(bytes per launch, fields) from a traffic summary, or (None, reason)
    when it is missing or its kernel sources have changed since."""
    if not os.path.exists(path):
        return None, "no traffic summary"
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^([A-Za-z0-9_]+):\s*(\S+)\s*$", line)
            if m:
                fields[m.group(1)] = m.group(2)
    fam = fields.get("source_family")
    if fam not in KERNEL_SOURCES or fields.get("source_sha256") != sources_sha256(fam):
        return None, "kernel sources changed since the counters were taken"
    return float(fields["traffic_bytes_per_launch"]), fields


def cmd_counters(a):
    """Mean per dispatch of every counter recorded for one kernel in the
    --pmc databases under each directory."""
    lines = [f"# rocprofv3 counters per launch: {a.title}", "",
             "commands (`cd /tmp && export TMPDIR=/tmp` first; $REPO is the repository root):", ""]
    lines += [f"    {c}" for c in a.cmd]
    lines += ["", f"{'counter':<32} {'per launch':>14} {'dispatches':>10}"]
    name = None
    for d in a.dirs:
        n, cs = _match(kernel_counters(d), a.kernel)
        name = name or n
        for c, vals in sorted(cs.items()):
            lines.append(f"{c:<32} {statistics.mean(vals):>14.5g} {len(vals):>10}")
    lines.insert(1, f"kernel: {name}")
    _write(a.out, lines)


def cmd_copy(a):
    import torch
    n = a.mib * 2 ** 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert bool((dst[:: 2 ** 16] == 1).all())
    print(f"copied {a.mib} MiB x {a.reps}", flush=True)


def _write(path, lines):
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--cmd", required=True)
    t.add_argument("--title", default="")
    t.add_argument("--out", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=4)
    r = sub.add_parser("traffic")
    r.add_argument("--kernel", required=True, help="regex selecting one kernel")
    r.add_argument("--family", required=True, choices=sorted(KERNEL_SOURCES))
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--copy-fetch", required=True)
    r.add_argument("--copy-write", required=True)
    r.add_argument("--copy-kernel", default="copyBuffer")
    r.add_argument("--copy-mib", type=int, required=True)
    r.add_argument("--copy-reps", type=int, required=True)
    r.add_argument("--algorithmic-bytes", type=float, default=None)
    r.add_argument("--cmd", action="append", required=True)
    r.add_argument("--out", required=True)
    n = sub.add_parser("counters")
    n.add_argument("dirs", nargs="+")
    n.add_argument("--kernel", required=True, help="regex selecting one kernel")
    n.add_argument("--title", default="")
    n.add_argument("--cmd", action="append", required=True)
    n.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    {"trace": cmd_trace, "copy": cmd_copy, "traffic": cmd_traffic, "counters": cmd_counters}[a.what](a)


if __name__ == "__main__":
    sys.exit(main())
