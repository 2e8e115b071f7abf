"""Builds the synthetic-input generators: libsynth.so (host, gcc) and
libsynth_dev.so (device, hipcc for gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose=False):
    host = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
            "-o", os.path.join(HERE, "libsynth.so"), os.path.join(HERE, "synth.c")]
    dev = ["hipcc", *HIP_FLAGS, "-o", os.path.join(HERE, "libsynth_dev.so"),
           os.path.join(HERE, "synth_dev.hip")]
    for cmd in (host, dev):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = [l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l]
        if r.returncode != 0:
            raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + "\n".join(noise))
        if verbose and noise:
            print("\n".join(noise))


if __name__ == "__main__":
    build(verbose=True)
