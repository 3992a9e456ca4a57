"""Build libcskv.so for gfx950 with hipcc, in place next to this file."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libcskv.so")
# the streaming probe (a measurement tool of profiling.py, outside the path)
PROBE_SRC = os.path.join(HERE, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(HERE, "libcskv_probe.so")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         # packed fp32 math is kept off on these GPUs
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) +
                  glob.glob(os.path.join(HERE, "csrc", "*.cpp")))


# per-source additions: the indexer's score kernels keep MFMA results in
# VGPRs (their epilogue reads every result once; no accumulator copies)
EXTRA = {"index_topk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
NOISE = "is not a recognized feature for this target"


def _run(cmds):
    """Run the compile commands in parallel; raise with the output of the
    first that fails."""
    procs = [subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
             for c in cmds]
    msgs = []
    failed = None
    for c, p in zip(cmds, procs):
        out, _ = p.communicate()
        msg = "\n".join(l for l in out.splitlines() if NOISE not in l)
        msgs.append(msg)
        if p.returncode != 0 and failed is None:
            failed = f"{' '.join(c)}\n{msg}"
    if failed:
        raise RuntimeError("hipcc failed:\n" + failed)
    return msgs


def build(verbose=False):
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, cmds = [], []
    for src in sources():
        name = os.path.basename(src)
        obj = os.path.join(objdir, name + ".o")
        flags = [f for f in FLAGS if f != "-shared"]
        cmds.append(["hipcc"] + flags + EXTRA.get(name, []) + ["-c", "-o", obj, src])
        objs.append(obj)
    probe_tmp = PROBE_LIB + ".tmp"
    cmds.append(["hipcc"] + FLAGS + ["-o", probe_tmp, PROBE_SRC])
    msgs = _run(cmds)
    tmp = LIB + ".tmp"
    msgs += _run([["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs])
    if verbose and any(m.strip() for m in msgs):
        print("\n".join(m for m in msgs if m.strip()))
    os.replace(tmp, LIB)
    os.replace(probe_tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
