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

``trace <results.db> <command>`` prints, from a ``rocprofv3 --kernel-trace``
database, each library kernel's dispatch count and average / min / max
duration per grid shape, with the profiled command in the header.
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
    for needle in ("beta_table_kernel", "compress_fused_kernel", "compress_join_kernel"):
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


def trace(db, command):
    import sqlite3
    con = sqlite3.connect(db)
    q = ("select s.kernel_name, d.grid_size_x / d.workgroup_size_x, d.grid_size_y, "
         "d.grid_size_z, d.workgroup_size_x, d.end - d.start from rocpd_kernel_dispatch d "
         "join rocpd_info_kernel_symbol s on d.kernel_id = s.id")
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


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) >= 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3], sys.argv[4] if len(sys.argv) > 4 else None)
    elif len(sys.argv) == 4 and sys.argv[1] == "trace":
        trace(sys.argv[2], sys.argv[3])
    else:
        raise SystemExit(__doc__)
