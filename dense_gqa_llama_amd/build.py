"""Builds libllama_mi355x.so, the C-ABI library of the gfx950 forward step,
in-tree from csrc/ with hipcc."""
import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(HERE, "libllama_mi355x.so")

FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = [l for l in (r.stderr or "").splitlines()
             if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), flush=True)


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def build(verbose=False, jobs=8):
    os.makedirs(OBJ, exist_ok=True)
    objs = []
    cmds = []
    for src in sources():
        obj = os.path.join(OBJ, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
        cmds.append(["hipcc", *FLAGS, *lang, "-c", src, "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB, *objs], verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
