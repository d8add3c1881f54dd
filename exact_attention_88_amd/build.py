"""Build the HIP libraries in-tree for gfx950.

Each ``csrc/*.hip`` translation unit is compiled to an object in parallel;
the attention sources are linked into ``exact_attention_88_amd/libfa.so``
(``include/fa.h``) and the measurement probes into
``exact_attention_88_amd/libfa_probe.so`` (``include/fa_probe.h``).  Run as
``python -m exact_attention_88_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
PROBE_LIB = os.path.join(PKG, "libfa_probe.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Packed fp32 VALU forms (v_pk_fma_f32 and friends) are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-ffp-contract=fast",
    "-I", os.path.join(ROOT, "include"),
]
# Per-file flags.  The backward files: every MFMA takes the form whose
# accumulator (C and D) is in architectural VGPRs, also in their
# one-wave-per-SIMD kernels, whose 512-register budget would otherwise put
# every product in accumulator registers and read each score and dP element
# back with a v_accvgpr_read; those kernels keep MFMA operands (K, V, dO rows)
# in accumulator registers instead.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA_FLAGS = {"fa_bwd_f16.hip": _VGPR_FORM, "fa_bwd_dkdv.hip": _VGPR_FORM, "fa_bwd_dq.hip": _VGPR_FORM}
SOURCES = ["fa_fwd.hip", "fa_fwd_f16.hip", "fa_bwd_dkdv.hip", "fa_bwd_dq.hip", "fa_bwd_f16.hip",
           "fa_bwd_split.hip", "fa_api.hip"]
PROBE_SOURCES = ["fa_probe.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


# Any kernel that uses scratch (spilled or stack-allocated) memory is a build
# error: spilling tile configurations are pruned from the tile tables, and no
# kernel is exempt.  (Mangled-name fragments of allowed instantiations would
# go here.)
ALLOWED_SCRATCH: tuple = ()


def _scratch_kernels(remarks: str):
    """(kernel, bytes) for every kernel whose resource remark reports scratch."""
    out, name = [], None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in line and name:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split("[")[0].strip())
            if size:
                out.append((name, size))
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj,
           "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    bad = [(k, n) for k, n in _scratch_kernels(res.stderr)
           if not any(frag in k for frag in ALLOWED_SCRATCH)]
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch memory: {bad}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {os.path.basename(PROBE_LIB)}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
