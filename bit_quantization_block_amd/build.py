"""Build liblq.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "liblq.so")
CEILING_LIB = os.path.join(HERE, "liblq_ceiling.so")

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
    # per-kernel register, scratch and occupancy figures (checked below)
    "-Rpass-analysis=kernel-resource-usage",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def kernel_resources(remarks: str) -> dict:
    """{kernel: {"vgprs", "scratch", "occupancy"}} from the compiler's
    kernel-resource-usage remarks of one unit."""
    out, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        if name is None:
            continue
        for key, pat in (("vgprs", r"remark:\s+VGPRs: (\d+)"), ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"),
                         ("occupancy", r"Occupancy \[waves/SIMD\]: (\d+)")):
            m = re.search(pat, line)
            if m:
                out[name][key] = int(m.group(1))
    return out


def build(out: str = LIB, defines=(), build_dir: str | None = None, jobs: int = 8,
          allow_scratch: bool = False) -> str:
    """Compile every HIP source and link the shared library. `defines` are extra
    -D flags (for example LQ_NATIVE_E4M3=0 to use the bit-manipulation encoder).
    Writes each kernel's VGPRs, scratch and occupancy to kernel_resources.txt in
    the build folder; a kernel that uses scratch (register spills or a local
    array the compiler could not keep in registers) fails the build unless
    `allow_scratch`."""
    build_dir = build_dir or os.path.join(ROOT, "_build", os.path.splitext(os.path.basename(out))[0])
    os.makedirs(build_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    units = [("lq_api.hip", "lq_api.o", [])]
    units += [("lq_inst.hip", f"lq_inst_{dt}_{odt}.o", [f"-DLQ_INST_DT={dt}", f"-DLQ_INST_ODT={odt}"])
              for dt in range(3) for odt in range(3)]
    units += [("lq_fast.hip", f"lq_fast_{dt}.o", [f"-DLQ_FAST_DT={dt}"]) for dt in range(2)]
    units += [("lq_lc.hip", "lq_lc.o", []), ("lq_h16.hip", "lq_h16.o", [])]
    ceiling = ("lq_ceiling.hip", "lq_ceiling.o", [])
    cmds = []
    for src, obj, extra in units + [ceiling]:
        cmds.append([HIPCC, *FLAGS, *dflags, *extra, "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", os.path.join(build_dir, obj)])
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    res = {}
    for (src, obj, _), r in zip(units + [ceiling], results):
        for k, v in kernel_resources(r.stderr).items():
            res[f"{obj}: {k}"] = v
    with open(os.path.join(build_dir, "kernel_resources.txt"), "w") as f:
        for k in sorted(res):
            v = res[k]
            f.write(f"{k} vgprs={v.get('vgprs')} scratch={v.get('scratch')} occupancy={v.get('occupancy')}\n")
    spills = sorted(k for k, v in res.items() if v.get("scratch", 0) > 0)
    if not res:
        raise RuntimeError("no kernel resource remarks in the compiler output")
    if spills and not allow_scratch:
        raise RuntimeError("kernels using scratch:\n  " + "\n  ".join(spills))
    # export the C entry points only (HIP gives kernel symbols default visibility)
    vscript = os.path.join(build_dir, "exports.map")
    with open(vscript, "w") as f:
        f.write("{\n  global: lq_*;\n  local: *;\n};\n")
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", f"-Wl,--version-script={vscript}",
          *[os.path.join(build_dir, o) for _, o, _ in units], "-o", tmp])
    os.replace(tmp, out)
    # the memory-ceiling kernels: a library of their own, beside liblq
    cscript = os.path.join(build_dir, "exports_ceiling.map")
    with open(cscript, "w") as f:
        f.write("{\n  global: lqc_*;\n  local: *;\n};\n")
    cout = os.path.join(os.path.dirname(out), os.path.basename(CEILING_LIB))
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", f"-Wl,--version-script={cscript}",
          os.path.join(build_dir, ceiling[1]), "-o", cout + ".tmp"])
    os.replace(cout + ".tmp", cout)
    return out


if __name__ == "__main__":
    print(build())
