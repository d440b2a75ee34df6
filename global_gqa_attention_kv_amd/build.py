"""Build libgqa_attn.so in-tree with hipcc for gfx950.

Every .hip/.cpp file under csrc/ is compiled to an object in _build/ (in
parallel) and linked into global_gqa_attention_kv_amd/libgqa_attn.so.
Run ``python -m global_gqa_attention_kv_amd.build`` or call :func:`build`."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgqa_attn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-result"]
# keep the compiler from forming packed fp32 ops on its own
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops"]


# the compiler's per-kernel resource report (remarks on stderr)
RESOURCES = ["-Rpass-analysis=kernel-resource-usage"]
_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|"
                     r"VGPRs Spill|SGPRs Spill): (\S+)")


def kernel_resources(stderr: str) -> dict:
    """{kernel: {"ScratchSize [bytes/lane]": n, "VGPRs Spill": n, ...}} from
    the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for key, val in _REMARK.findall(stderr):
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = int(val)
    return out


def check_resources(res: dict, src: str) -> None:
    """Every kernel must run without private memory: a spill or a stack
    array turns register accesses into memory round trips inside the tile
    loops, and in a direct-to-LDS kernel into flat accesses."""
    bad = {k: v for k, v in res.items() if any(v.values())}
    if bad:
        raise RuntimeError("%s: kernels using private memory: %s" % (src, bad))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE + RESOURCES
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd),
                                                         r.stdout, r.stderr))
    if src.endswith(".hip"):
        res = kernel_resources(r.stderr)
        with open(src) as f:
            has_kernels = "__global__" in f.read()
        if has_kernels and not res:
            raise RuntimeError("%s: no kernel resource report" % src)
        check_resources(res, src)
    return obj


def build(verbose=False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) +
                  glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout,
                                                      r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
