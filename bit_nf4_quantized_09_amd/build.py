"""Compile the gfx950 HIP library libqlora_nf4.so in-tree with hipcc."""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libqlora_nf4.so")
PROBE_SOURCE = "hbm_probe.hip"      # the HBM ceiling probes: a library of their own
PROBE_LIB = os.path.join(OUT_DIR, "libnf4_hbm_probe.so")
SOURCES = ["api.hip", "codec.hip", "lora.hip", "fused.hip", "gemv.hip", "adamw.hip", "codebook.hip", "lowrank.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",                                  # no silent multiply-add fusion
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OUT_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, errs))
    if errs.strip() and verbose:
        print(errs, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + [PROBE_SOURCE]))
    probe_obj = objs.pop()
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", probe_obj, "-o", tmp], check=True)
    os.replace(tmp, PROBE_LIB)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
