"""Build the HIP library ``liblora_lowp.so`` in-tree for gfx950 with hipcc.

Run as ``python -m precision_gemm_amd.build``; ``__graft_entry__.build()`` calls
:func:`build`.  Every call compiles (no up-to-date check), so a changed source is
always picked up.
"""

from __future__ import annotations

import json
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblora_lowp.so")
SOURCES = ["lora_kernels.hip", "lora_gemm_pf.hip", "lora_backward.hip", "lora_api.cpp"]
ARCH = "gfx950"

# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 in the device code.
# atomic optimizer off: it rewrites a single-lane atomic with return into a wave-level
# scan whose result is consumed at once, which forces a wait for every load in flight.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-result",
    # per-kernel register, scratch and LDS use, kept next to the library (see resources())
    "-Rpass-analysis=kernel-resource-usage",
]
RESOURCES = LIB + ".resources.json"


def parse_resources(stderr: str) -> dict:
    """Per-kernel resource use from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in stderr.splitlines():
        if "[-Rpass-analysis=kernel-resource-usage]" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass", 1)[0].strip()
        key, _, val = body.partition(":")
        key, val = key.strip(), val.strip()
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = int(val) if val.lstrip("-").isdigit() else val
    return out


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
    errs = "\n".join(l for l in lines if "kernel-resource-usage" not in l and not l.lstrip().startswith(("|", "^"))
                     and not l.strip().isdigit())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    with open(RESOURCES, "w") as f:
        json.dump(parse_resources(res.stderr), f, indent=1, sort_keys=True)
    return LIB


def resources() -> dict:
    """Resource use of every kernel of the last build (empty if none was recorded)."""
    try:
        with open(RESOURCES) as f:
            return json.load(f)
    except OSError:
        return {}


if __name__ == "__main__":
    print(build(verbose=True))
