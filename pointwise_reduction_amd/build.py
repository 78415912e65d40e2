"""Build libfr.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, with packed-fp32
instructions disabled (the compiler still vectorizes, but never emits
v_pk_*_f32), without fast-math (NaN propagation and IEEE division matter
here), then linked into pointwise_reduction_amd/libfr.so.
"""
import concurrent.futures
import glob
import re
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "fr")
LIB = os.path.join(HERE, "libfr.so")
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfr")


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def parse_resource_usage(lines):
    """Per-kernel VGPRs, scratch bytes and occupancy from the compiler's
    kernel-resource-usage remarks."""
    usage, cur = {}, None
    for line in lines:
        if "Function Name:" in line:
            cur = line.split("Function Name:", 1)[1].strip()
            usage[cur] = {}
        elif cur and "VGPRs:" in line and "AGPR" not in line:
            usage[cur]["vgpr"] = int(line.rsplit(":", 1)[1].split()[0])
        elif cur and "ScratchSize" in line:
            usage[cur]["scratch"] = int(line.rsplit(":", 1)[1].split()[0])
        elif cur and "Occupancy" in line:
            usage[cur]["occupancy"] = int(line.rsplit(":", 1)[1].split()[0])
    return usage


def check_residency(usage):
    """The single-pass split softmax sizes its grid so that all of its
    workgroups are resident at once, from the occupancy the planner assumes
    for the 256-thread, 8-vector kernel. A kernel compiled to fewer waves per
    SIMD would still be correct (a workgroup that waits too long computes the
    missing partials itself) but part of the grid would start only when
    others end; measured 14% slower. Fail the build instead."""
    with open(os.path.join(CSRC, "fr_plan.cpp")) as f:
        m = re.search(r"constexpr int kOnePassWavesPerSimd = (\d+);", f.read())
    if not m:
        raise RuntimeError("fr_plan.cpp: kOnePassWavesPerSimd not found")
    need = int(m.group(1))
    low = sorted(n for n, u in usage.items()
                 if "fr_split_softmax_oneILi256ELi8E" in n and u.get("occupancy", 0) < need)
    if low:
        raise RuntimeError(f"kernels below the {need} waves per SIMD their grid assumes: " + ", ".join(low))


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


# Host-side sanitizers for the CPU test run: each flag reaches the host pass
# only (-Xarch_host before it); device code is built as usual.
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                       "-Xarch_host", "-g"]


def build(verbose=False, jobs=None, lib=None, build_dir=None, host_extra=None):
    """Compile all sources (in parallel) and link libfr.so. Always rebuilds.
    `lib`, `build_dir` and `host_extra` (e.g. HOST_SANITIZE_FLAGS) serve
    other builds of the same sources."""
    lib = lib or LIB
    build_dir = build_dir or BUILD_DIR
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    flags = common_flags() + list(host_extra or [])

    usage = {}

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        lang = ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
        cmd = [cc] + flags + lang + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        lines = [l for l in (res.stdout + res.stderr).splitlines()
                 if "packed-fp32-ops" not in l]  # host pass does not know the feature
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
        usage.update(parse_resource_usage(lines))
        rest = [l for l in lines if "remark" not in l and "kernel-resource-usage" not in l]
        if rest and verbose:
            print("\n".join(rest))
        return obj

    srcs = sources()
    jobs = jobs or min(8, len(srcs))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    with open(os.path.join(build_dir, "resource_usage.txt"), "w") as f:
        for name, u in sorted(usage.items()):
            f.write(f"{name} vgpr={u.get('vgpr')} scratch={u.get('scratch')} occupancy={u.get('occupancy')}\n")
    spills = sorted(n for n, u in usage.items() if u.get("scratch", 0) > 0)
    if spills:  # Algorithm 9.1 rejects configurations that spill registers
        raise RuntimeError("kernels spill registers to scratch: " + ", ".join(spills))
    check_residency(usage)
    tmp = lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + list(host_extra or []) + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
