"""Build liblq.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "liblq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # only the entry points marked LQ_API in lq.h are exported
    "-fvisibility=hidden",
    # bit-exact results: no contraction of a*b+c into fma, no fast math
    "-ffp-contract=off", "-fno-fast-math",
    # never emit packed fp32 ALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(out: str = LIB, defines=(), build_dir: str | None = None, jobs: int = 8) -> str:
    """Compile every HIP source and link the shared library. `defines` are extra
    -D flags (for example LQ_NATIVE_E4M3=0 to use the bit-manipulation encoder)."""
    build_dir = build_dir or os.path.join(ROOT, "_build", os.path.splitext(os.path.basename(out))[0])
    os.makedirs(build_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    units = [("lq_api.hip", "lq_api.o", [])]
    units += [("lq_inst.hip", f"lq_inst_{dt}_{odt}.o", [f"-DLQ_INST_DT={dt}", f"-DLQ_INST_ODT={odt}"])
              for dt in range(3) for odt in range(3)]
    units += [("lq_fast.hip", f"lq_fast_{dt}.o", [f"-DLQ_FAST_DT={dt}"]) for dt in range(2)]
    units += [("lq_lc.hip", "lq_lc.o", [])]
    cmds = []
    for src, obj, extra in units:
        cmds.append([HIPCC, *FLAGS, *dflags, *extra, "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", os.path.join(build_dir, obj)])
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_run, cmds))
    # export the C entry points only (HIP gives kernel symbols default visibility)
    vscript = os.path.join(build_dir, "exports.map")
    with open(vscript, "w") as f:
        f.write("{\n  global: lq_*;\n  local: *;\n};\n")
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", f"-Wl,--version-script={vscript}",
          *[os.path.join(build_dir, o) for _, o, _ in units], "-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
