"""HBM traffic of the fused compressor, measured with rocprofv3 counters.

Two passes of the same program, one counter each (the counters do not fit
one pass):

    rocprofv3 --pmc FETCH_SIZE -f csv -d <fetch_dir> -o p -- \\
        python -m compressed_sparse_kv_overlapping_amd.profiling run
    rocprofv3 --pmc WRITE_SIZE -f csv -d <write_dir> -o p -- \\
        python -m compressed_sparse_kv_overlapping_amd.profiling run
    python -m compressed_sparse_kv_overlapping_amd.profiling summarize \\
        <fetch_dir> <write_dir>

``run`` launches a plain device copy of a known size (the runtime's
copy-buffer kernel, through torch's copy_)
and then the two-scale compressor on the 1M-token layer shapes.  The counters
report KiB per dispatch; each is scaled by what the same counter reads for
the copy (known bytes / counted bytes), so the figure is in true bytes.
``summarize`` writes profiles/traffic.json (per launch of the benchmark's
``compress`` part, keyed by a digest of the kernel sources so that a stale
figure is never reported) and prints the summary kept in profiles/.

``indexer`` runs the selection at the prefill-chunk and decode shapes (the
program profiled for the indexer's SQ counters and kernel trace), and
``sq <pmc_dir> <title> <command>`` prints every counter of a --pmc run per
kernel.

``floor`` times the streaming probe (libcskv_probe.so: the compressor's
reads and writes at 1M tokens with none of its arithmetic, in four mixes)
beside the fused compressor itself, and prints the table kept in
profiles/compress_floor_probe.txt.

``trace <results.db> <command> [phases]`` prints, from a ``rocprofv3
--kernel-trace`` database, each library kernel's dispatch count and average /
min / max duration per grid shape, with the profiled command in the header.
``phases`` (e.g. ``warmup:2,warm:10,cold:10,cold_dirty:10``, the order in
which bench.py runs its steps) splits, for every kernel dispatched exactly
that many times in all, its dispatches in start order into those phases and
prints the average of each.
"""
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 29                 # 512 MiB read + 512 MiB written per copy
T_TOKENS, D = 1 << 20, 512


# the sources the compressor kernels are built from: a traffic figure
# applies to these only
# the sources that define the compressor's device code (kernels.hpp holds
# only host-side launcher declarations)
COMPRESSOR_SOURCES = ("compress.hip", "common.hpp")


def source_digest():
    """Digest of the compressor's kernel sources."""
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for f in COMPRESSOR_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def run():
    import torch
    import compressed_sparse_kv_overlapping_amd as cskv
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn(T_TOKENS, D, device="cuda", generator=g).bfloat16()
    z = torch.randn(T_TOKENS, D, device="cuda", generator=g).bfloat16()
    b4 = 0.1 * torch.randn(8, D, device="cuda", generator=g)
    b128 = 0.1 * torch.randn(256, D, device="cuda", generator=g)
    e4 = torch.empty(T_TOKENS // 4, 576, dtype=torch.bfloat16, device="cuda")
    e128 = torch.empty(T_TOKENS // 128, 576, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(cskv.compress2_workspace_size(T_TOKENS, 128), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    for _ in range(3):
        cskv.compress2(x, z, b4, 4, b128, 128, out_small=e4, out_large=e128, workspace=ws)
    torch.cuda.synchronize()
    print(json.dumps({"source_digest": source_digest(), "copy_bytes": COPY_BYTES}), flush=True)


def indexer():
    """The selection at the prefill chunk (4,096 causal queries over 262,144
    fp8 keys, top-1024) and at the 1M-token decode (32 queries over 262,144
    bf16 keys), three launches each, on random device inputs (the kernels'
    work does not depend on the values beyond the candidate counts, which
    random scores keep near their typical 1.2k per query)."""
    import torch
    import compressed_sparse_kv_overlapping_amd as cskv
    g = torch.Generator(device="cuda").manual_seed(0)
    N, k = 1 << 18, 1024
    for B, dt, causal in ((4096, torch.float8_e4m3fn, True), (32, torch.bfloat16, False)):
        q = torch.randn(B, 64, device="cuda", generator=g).to(dt)
        keys = torch.randn(N, 64, device="cuda", generator=g).to(dt)
        qp = (torch.arange(B, device="cuda", dtype=torch.int64) + (N * 4 - B)) if causal else None
        out = torch.empty(B, k, dtype=torch.int32, device="cuda")
        ws = torch.empty(cskv.index_topk_workspace_size(B, N, k), dtype=torch.uint8, device="cuda")
        for _ in range(3):
            cskv.index_topk(q, keys, k, q_pos=qp, m=4, idx_out=out, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            cskv.index_topk(q, keys, k, q_pos=qp, m=4, idx_out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        print(json.dumps({"queries": B, "entries": N, "k": k, "dtype": str(dt),
                          "ms_per_selection": round(e0.elapsed_time(e1) / 5, 4)}), flush=True)


def floor(reps=7):
    """The compressor against what the memory system delivers for its
    traffic: the streaming probe's four mixes (reads only; reads with the
    entry rows written as they stream; the writes only; reads, then the
    writes) and compress2 on the same 1M-token shapes, each the median of
    reps launches timed by events."""
    import ctypes
    import statistics
    import torch
    import compressed_sparse_kv_overlapping_amd as cskv
    from compressed_sparse_kv_overlapping_amd.build import PROBE_LIB
    lib = ctypes.CDLL(PROBE_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.cskv_probe_stream.argtypes = [ctypes.c_int, vp, vp, i64, vp, vp, vp, vp]
    lib.cskv_probe_stream.restype = ctypes.c_int
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn(T_TOKENS, D, device="cuda", generator=g).bfloat16()
    z = torch.randn(T_TOKENS, D, device="cuda", generator=g).bfloat16()
    o4 = torch.empty(T_TOKENS // 4, D, dtype=torch.bfloat16, device="cuda")
    o128 = torch.empty(T_TOKENS // 128, D, dtype=torch.bfloat16, device="cuda")
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def probe(mode):
        st = lib.cskv_probe_stream(mode, x.data_ptr(), z.data_ptr(), T_TOKENS, o4.data_ptr(),
                                   o128.data_ptr(), sink.data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"probe launch failed ({st})")

    b4 = 0.1 * torch.randn(8, D, device="cuda", generator=g)
    b128 = 0.1 * torch.randn(256, D, device="cuda", generator=g)
    e4 = torch.empty(T_TOKENS // 4, 576, dtype=torch.bfloat16, device="cuda")
    e128 = torch.empty(T_TOKENS // 128, 576, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(cskv.compress2_workspace_size(T_TOKENS, 128), dtype=torch.uint8, device="cuda")

    def compress():
        cskv.compress2(x, z, b4, 4, b128, 128, out_small=e4, out_large=e128, workspace=ws)

    def timed(fn):
        for _ in range(2):
            fn()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3)
        return statistics.median(out)

    rd = 2 * T_TOKENS * D * 2
    wr = (T_TOKENS // 4 + T_TOKENS // 128) * D * 2
    rows = [("reads only", lambda: probe(0), rd),
            ("reads + entry writes as they stream", lambda: probe(1), rd + wr),
            ("entry writes only", lambda: probe(2), wr),
            ("reads, then each wave's writes", lambda: probe(3), rd + wr),
            ("compress2 (fused kernel + table + join)", compress, rd + wr)]
    print(f"# streaming probe vs the fused compressor, {T_TOKENS} tokens x {D} dims bf16 "
          f"(reads {rd / 1e9:.3f} GB, entry writes {wr / 1e9:.3f} GB), median of {reps} launches")
    print("# command: python -m compressed_sparse_kv_overlapping_amd.profiling floor")
    res = {}
    for name, fn, nbytes in rows:
        us = timed(fn)
        res[name] = us
        print(f"{name:42s} {us:9.1f} us  {nbytes / (us * 1e-6) / 1e12:6.2f} TB/s")
    mix = res["reads + entry writes as they stream"]
    print(f"compressor / streaming mix: {res[rows[-1][0]] / mix:.3f}")
    return res


def sq_summary(directory, title, command):
    """Per-kernel averages of every counter in a rocprofv3 --pmc directory."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    acc = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (r["Kernel_Name"], r.get("Grid_Size", ""), r.get("Workgroup_Size", ""))
                acc.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    print(f"# {title}\n# command: {command}\n# per dispatch, averaged over the dispatches of each kernel "
          f"and grid (grid in threads)\n# derived: per wave = counter / SQ_WAVES; busy = SQ_BUSY_CYCLES / 32 "
          f"shader engines; MFMA pipe = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / busy; attention tiles = "
          f"MFMA per wave / 68\n# (36 logit + 32 weighted-sum MFMAs a 32-row tile; a 32x32x16 bf16 MFMA "
          f"occupies its SIMD 32 cycles, so a tile's MFMAs take 2,176 cycles)")
    for key in sorted(acc):
        name, g, w = key
        print(f"\n{name}  (grid {g}, workgroup {w})")
        avg = {c: sum(v) / len(v) for c, v in acc[key].items()}
        for c, v in sorted(avg.items()):
            print(f"  {c:28s} {v:16.1f}")
        _sq_derived(name, avg)


def _sq_derived(name, avg):
    """Per-wave instruction counts, busy cycles (SQ_BUSY_CYCLES over the 32
    shader engines) and MFMA pipe use (SQ_VALU_MFMA_BUSY_CYCLES over the 1,024
    SIMDs and the busy cycles); for the wide attention kernel also per
    32-row tile (36 logit + 32 weighted-sum MFMAs a tile, 32 cycles each)."""
    need = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_BUSY_CYCLES",
            "SQ_VALU_MFMA_BUSY_CYCLES")
    if not all(c in avg for c in need) or avg["SQ_WAVES"] <= 0:
        return
    w = avg["SQ_WAVES"]
    valu, lds, mfma = avg["SQ_INSTS_VALU"] / w, avg["SQ_INSTS_LDS"] / w, avg["SQ_INSTS_MFMA"] / w
    busy = avg["SQ_BUSY_CYCLES"] / 32
    pipe = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / busy if busy > 0 else 0.0
    print(f"  per wave: VALU {valu:.0f}, LDS {lds:.0f}, MFMA {mfma:.0f}")
    line = f"  busy cycles: {busy:.0f}"
    if "attend_wide" in name and mfma > 0:
        tiles = mfma / 68
        per_tile = busy / tiles
        line += (f"; tiles per wave {tiles:.0f}; busy cycles per tile {per_tile:.0f} "
                 f"({per_tile / 2176:.2f}x the MFMA cycles); VALU per wave per tile {valu / tiles:.0f}")
    if mfma > 0:
        line += f"; MFMA pipe {100 * pipe:.0f}%"
    print(line)


def _per_kernel(directory, counter):
    """Average counter value per dispatch, by kernel name."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    acc = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _find(per, needle):
    hits = [k for k in per if needle in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {needle!r}, found {hits}")
    return per[hits[0]]


def summarize(fetch_dir, write_dir, digest=None):
    fetch = _per_kernel(fetch_dir, "FETCH_SIZE")
    write = _per_kernel(write_dir, "WRITE_SIZE")
    # the device-to-device copy runs as the runtime's copy-buffer kernel
    copy_f = _find(fetch, "copyBuffer")
    copy_w = _find(write, "copyBuffer")
    f_scale = COPY_BYTES / (copy_f * 1024.0)
    w_scale = COPY_BYTES / (copy_w * 1024.0)
    parts = {}
    for needle in ("compress_fused_kernel", "compress_join_kernel"):
        fb = _find(fetch, needle) * 1024.0 * f_scale
        wb = _find(write, needle) * 1024.0 * w_scale
        parts[needle] = {"fetch_bytes": round(fb), "write_bytes": round(wb)}
    total = sum(p["fetch_bytes"] + p["write_bytes"] for p in parts.values())
    n4, n128 = T_TOKENS // 4, T_TOKENS // 128
    alg = 2 * T_TOKENS * D * 2 + (n4 + n128) * D * 2
    out = {
        "source_digest": digest or source_digest(),
        "calibration": {"copy_bytes_each_way": COPY_BYTES, "fetch_scale": round(f_scale, 4),
                        "write_scale": round(w_scale, 4)},
        "kernels": {"compress": {"bytes_per_launch": total, "algorithmic_bytes": alg,
                                 "parts": parts}},
    }
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print("# HBM traffic of the two-scale compressor, 1M tokens x 512 dims bf16, m=4 and m'=128")
    print("# commands:")
    fd, wd = os.path.normpath(fetch_dir), os.path.normpath(write_dir)
    print(f"#   rocprofv3 --pmc FETCH_SIZE -f csv -d {fd} -o p -- "
          "python -m compressed_sparse_kv_overlapping_amd.profiling run")
    print(f"#   rocprofv3 --pmc WRITE_SIZE -f csv -d {wd} -o p -- "
          "python -m compressed_sparse_kv_overlapping_amd.profiling run")
    print(f"#   python -m compressed_sparse_kv_overlapping_amd.profiling summarize {fd} {wd}")
    print(f"# calibration: a {COPY_BYTES >> 20} MiB device copy reads FETCH_SIZE {copy_f:.0f} KiB "
          f"and WRITE_SIZE {copy_w:.0f} KiB per dispatch -> scale {f_scale:.4f} (fetch), "
          f"{w_scale:.4f} (write)")
    for k, p in parts.items():
        print(f"{k:24s} fetch {p['fetch_bytes'] / 1e9:8.4f} GB  write {p['write_bytes'] / 1e9:8.4f} GB")
    print(f"{'compress (both)':24s} total {total / 1e9:8.4f} GB per launch; algorithmic "
          f"{alg / 1e9:.4f} GB (ratio {total / alg:.3f})")


def trace(db, command, phases=None):
    import sqlite3
    con = sqlite3.connect(db)
    q = ("select s.kernel_name, d.grid_size_x / d.workgroup_size_x, d.grid_size_y, "
         "d.grid_size_z, d.workgroup_size_x, d.end - d.start from rocpd_kernel_dispatch d "
         "join rocpd_info_kernel_symbol s on d.kernel_id = s.id order by d.start")
    agg = {}
    for name, gx, gy, gz, wx, dur in con.execute(q):
        if "cskv" not in name:
            continue
        key = (name.replace(".kd", ""), f"{gx}x{gy}x{gz}", wx)
        agg.setdefault(key, []).append(dur / 1000.0)
    print(f"# rocprofv3 kernel trace summary\n# command: {command}\n"
          f"# durations in microseconds (per dispatch)")
    print(f"{'kernel':78s} {'grid(blocks)':>14s} {'wg':>4s} {'n':>4s} "
          f"{'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
    for (nm, grid, wx), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        print(f"{nm[:78]:78s} {grid:>14s} {wx:4d} {len(v):4d} {sum(v) / len(v):10.2f} "
              f"{min(v):10.2f} {max(v):10.2f}")
    if not phases:
        return
    spec = [(n, int(c)) for n, c in (p.split(":") for p in phases.split(","))]
    total = sum(c for _, c in spec)
    print(f"# per phase, in dispatch order ({phases}): average microseconds")
    for (nm, grid, wx), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        if len(v) != total:
            continue
        cols, i = [], 0
        for n, c in spec:
            cols.append(f"{n} {sum(v[i:i + c]) / c:.2f}")
            i += c
        print(f"{nm[:78]:78s} {grid:>14s}  " + "  ".join(cols))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) >= 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3], sys.argv[4] if len(sys.argv) > 4 else None)
    elif len(sys.argv) == 2 and sys.argv[1] == "indexer":
        indexer()
    elif len(sys.argv) == 2 and sys.argv[1] == "floor":
        floor()
    elif len(sys.argv) == 5 and sys.argv[1] == "sq":
        sq_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) in (4, 5) and sys.argv[1] == "trace":
        trace(sys.argv[2], sys.argv[3], sys.argv[4] if len(sys.argv) == 5 else None)
    else:
        raise SystemExit(__doc__)
