"""Build libulysses.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Run as `python -m ulysses_sequence_parallelism_rank_amd._build` or through
__graft_entry__.build(). Always recompiles."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libulysses.so")
SOURCES = ["permute.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_f32.hip", "ring.hip", "probe.hip", "abi.cpp"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose=False):
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        # packed fp32 VALU ops are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.rsplit(".", 1)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [hipcc()] + common + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
