"""Build the gfx950 attention library (libexact_fa.so) in-tree with hipcc.

Usage: ``python -m exact_io_aware_fa_amd.build [--resource-usage]``.

Every HIP source is compiled for gfx950 only, with packed-FP32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``) and
hardware float atomics enabled (``-munsafe-fp-atomics``). The shared library
lands next to this file, where the Python binding loads it from.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libexact_fa.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = [
    os.path.join(CSRC, "fa_api.hip"),
    os.path.join(CSRC, "kernels", "fa_fwd_bf16.hip"),
    os.path.join(CSRC, "kernels", "fa_fwd_bf16_d64.hip"),
    os.path.join(CSRC, "kernels", "fa_bwd_bf16.hip"),
    os.path.join(CSRC, "kernels", "fa_bwd_dkdv_d64.hip"),
    os.path.join(CSRC, "kernels", "fa_bwd_dkdv_d256.hip"),
    os.path.join(CSRC, "kernels", "fa_bwd_dkdv_wide.hip"),
    os.path.join(CSRC, "kernels", "fa_bwd_dq_bf16.hip"),
    os.path.join(CSRC, "kernels", "fa_bwd_dq_d256.hip"),
    os.path.join(CSRC, "kernels", "fa_bwd_aux.hip"),
    os.path.join(CSRC, "kernels", "fa_fp32.hip"),
    os.path.join(CSRC, "kernels", "fa_block_index.hip"),
    os.path.join(CSRC, "kernels", "fa_fp8_quant.hip"),
    os.path.join(CSRC, "kernels", "fa_fwd_fp8.hip"),
]

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src: str, resource_usage: bool) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, "-c", src, "-o", obj]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    log = r.stdout + r.stderr
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{log}")
    return obj, log


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every HIP source and link ``libexact_fa.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(lambda s: _compile(s, resource_usage), SOURCES))
    objs = [o for o, _ in results]
    logs = "".join(l for _, l in results)
    tmp = LIB_PATH + ".tmp"
    # --no-undefined: a kernel whose host stub failed to compile must stop the
    # build, not surface as an unresolved symbol when the library is loaded.
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose or resource_usage:
        sys.stdout.write(logs)
    return LIB_PATH


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel VGPR/AGPR/LDS/spill usage")
    args = ap.parse_args()
    print(build(resource_usage=args.resource_usage))


if __name__ == "__main__":
    main()
