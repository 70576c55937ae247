"""Build the HIP library libgqa_attn.so (gfx950) in-tree.

hipcc compiles each source under csrc/ to an object; the objects are linked
into gqa_attention_ragged_amd/lib/libgqa_attn.so.  The HIP runtime is linked
by the name "libamdhip64.so", so that inside a PyTorch process the runtime
PyTorch already loaded is the one the library uses (same streams, same
allocations); outside PyTorch the loader finds ROCm's own copy.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "lib", "libgqa_attn.so")
SOURCES = ["gqa_attn.cpp", "prefill.hip", "prefill_f16.hip", "prefill_bf16.hip", "prefill_fp8.hip",
           "prefill_kv8_f16.hip", "prefill_kv8_bf16.hip", "prefill_pp.hip",
           "prefill_persist.hip",
           "decode.hip", "kv_cache.hip", "validate.hip", "static_scratch.hip"]
ARCH = os.environ.get("GQA_ATTN_ARCH", "gfx950")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
    # never let the compiler form packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # per-kernel register / scratch / LDS report (parsed into RESOURCES)
    "-Rpass-analysis=kernel-resource-usage",
]
# Per-kernel resources of the last build: VGPRs, AGPRs, scratch bytes per
# lane, occupancy, spills, LDS bytes (one entry per kernel).
RESOURCES = os.path.join(BUILD, "kernel_resources.json")
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]):"
                     r"\s*(\S+)")
_KEYS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
         "Occupancy [waves/SIMD]": "occupancy", "SGPRs Spill": "sgpr_spill",
         "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds"}


def _parse_resources(text: str, src: str) -> list:
    out, cur = [], None
    for m in _REMARK.finditer(text):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = {"kernel": val, "source": src}
            out.append(cur)
        elif cur is not None:
            cur[_KEYS[key]] = int(val) if val.lstrip("-").isdigit() else val
    return out


def _hip_runtime_dir() -> str:
    """Directory holding the libamdhip64.so the library should bind to."""
    try:
        import torch  # noqa: F401  (plumbing only: pick the runtime torch loads)
        d = os.path.join(os.path.dirname(torch.__file__), "lib")
        if os.path.exists(os.path.join(d, "libamdhip64.so")):
            return d
    except Exception:
        pass
    return os.path.join(ROCM, "lib")


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", "-x", "hip", *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj, _parse_resources(r.stderr, src)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    resources = [k for _, ks in done for k in ks]
    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=0)
    rt = _hip_runtime_dir()
    tmp = LIB + ".tmp%d" % os.getpid()
    # plain g++ link: hipcc would add its own -lamdhip64 (soname libamdhip64.so.7)
    cmd = ["g++", "-shared", "-fPIC", *objs, "-o", tmp, "-L", rt, "-l:libamdhip64.so",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
