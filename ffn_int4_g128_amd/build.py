"""Build libqi4.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqi4.so")
BUILD = os.path.join(HERE, "_build")
# per-kernel registers, scratch (spills), occupancy and LDS, from the compiler
RESOURCES = os.path.join(BUILD, "kernel_resources.txt")
SOURCES = ["qi4_api.cpp", "qi4_pack.hip", "qi4_gemm.hip", "qi4_moe.hip", "qi4_prefill.hip",
           "qi4_quant.hip", "qi4_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are kept out of the generated code on purpose.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fno-gpu-rdc", "-ffp-contract=fast"]


_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
           "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}


def _resources(stderr: str) -> list[dict]:
    """The compiler's kernel-resource-usage remarks, one dict per kernel."""
    out, cur = [], None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            out.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*?): (\d+)", line)
        if cur is not None and m and m.group(1) in _FIELDS:
            cur[_FIELDS[m.group(1)]] = int(m.group(2))
    return out


def _compile(src: str, verbose: bool):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage"]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines()
                     if ("packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
                     or "error" in l.lower())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs)
    return obj, _resources(r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        res = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    objs = [o for o, _ in res]
    with open(RESOURCES, "w") as f:
        for src, (_, kernels) in zip(SOURCES, res):
            for k in kernels:
                f.write(f"{src} {k['name']} " + " ".join(f"{v}={k.get(v, -1)}" for v in
                        ("vgprs", "agprs", "scratch", "occupancy", "lds")) + "\n")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
