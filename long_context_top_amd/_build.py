"""Build the gfx950 shared libraries in-tree with hipcc.

* ``long_context_top_amd/liblct.so``: the C-ABI library (include/lct.h).
* ``synth/libsynth.so``: the device-side input filler.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
# Packed fp32 VALU forms are switched off for all device code.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# The attention kernels keep their MFMA accumulators in VGPRs: in AGPRs the
# compiler copies the whole output tile out and back on every key tile to
# serve the (rarely taken) softmax rescale branch.
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
SOURCE_FLAGS = {"gsa_prefill.hip": _VGPR_MFMA, "attn.hip": _VGPR_MFMA}

LCT_SOURCES = ["api.hip", "topk.hip", "idx_score.hip", "attn.hip", "gsa.hip", "gsa_prefill.hip", "prefill.hip",
               "misc.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


def _compile(src, obj):
    extra = SOURCE_FLAGS.get(os.path.basename(src), [])
    return _run([HIPCC, *DEVICE_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj])


def build(verbose: bool = False) -> list[str]:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for s in LCT_SOURCES:
        jobs.append((os.path.join(CSRC, s), os.path.join(BUILD, "lct_" + s + ".o")))
    synth_src = os.path.join(ROOT, "synth", "csrc", "synth_fill.hip")
    synth_obj = os.path.join(BUILD, "synth_fill.o")
    jobs.append((synth_src, synth_obj))
    workers = min(len(jobs), max(1, (os.cpu_count() or 2) - 1), 16)
    with cf.ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(lambda j: _compile(*j), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    lct_so = os.path.join(HERE, "liblct.so")
    synth_so = os.path.join(ROOT, "synth", "libsynth.so")
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", lct_so + ".tmp",
          *[o for _, o in jobs[:-1]]])
    os.replace(lct_so + ".tmp", lct_so)
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", synth_so + ".tmp", synth_obj])
    os.replace(synth_so + ".tmp", synth_so)
    return [lct_so, synth_so]


if __name__ == "__main__":
    for p in build(verbose=True):
        print("built", p)
