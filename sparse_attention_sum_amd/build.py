"""Build libdsa.so (gfx950) in-tree with hipcc.

    python -m sparse_attention_sum_amd.build

Every HIP source under csrc/ is compiled to an object file in parallel, then linked into
``sparse_attention_sum_amd/libdsa.so``.  All HIP code is compiled without packed-fp32 instructions.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
# Per-file flags for the device (gfx950) compilation only.  The sparse-MLA main loop holds a 32x288
# query block and a 32x256 output block in registers at two waves per SIMD, with only a few
# registers to spare; the register-minimising machine scheduler keeps it free of spill reloads (a
# reload there would wait for the tile loads in flight).  LLVM options given to hipcc reach the
# host compilation too, so such files are built in three steps: device code object, offload
# bundle, host object embedding the bundle.
DEVICE_FLAGS = {"sparse_mla.hip": ["-mllvm", "-misched=gcn-iterative-minreg"]}
BUNDLER = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang-offload-bundler")
if not os.path.exists(BUNDLER):
    BUNDLER = "/opt/rocm/llvm/bin/clang-offload-bundler"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{what} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def _compile(src: str, extra) -> str:
    name = os.path.basename(src)
    obj = os.path.join(BUILD, name + ".o")
    dev = DEVICE_FLAGS.get(name)
    if dev is None:
        _run([HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj], f"hipcc {name}")
        return obj
    code = os.path.join(BUILD, name + ".co")
    bundle = os.path.join(BUILD, name + ".hipfb")
    _run([HIPCC, *CFLAGS, *dev, *extra, "--cuda-device-only", "--no-gpu-bundle-output", "-c", src, "-o", code],
         f"hipcc (device) {name}")
    _run([BUNDLER, "-type=o", "-bundle-align=4096",
          f"-targets=host-x86_64-unknown-linux-gnu,hipv4-amdgcn-amd-amdhsa--{ARCH}",
          "-input=/dev/null", f"-input={code}", f"-output={bundle}"], f"bundle {name}")
    _run([HIPCC, *CFLAGS, *extra, "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", bundle,
          "-c", src, "-o", obj], f"hipcc (host) {name}")
    return obj


OBJDUMP = os.path.join(os.path.dirname(BUNDLER), "llvm-objdump")
VMEM_PREFIXES = ("global_", "buffer_", "scratch_", "flat_")


def check_mla_prologue_wait(code_object: str) -> int:
    """The sparse-MLA prologue awaits its index DMA with an explicit `s_waitcnt vmcnt(N)` that is
    correct only if at least N vector-memory instructions are issued between the DMA and the wait
    (loads complete in order, so the DMA is done once at most N of the later ones are outstanding).
    Counted here on the assembly of this build; the build fails if the compiler emitted fewer."""
    r = subprocess.run([OBJDUMP, "-d", "--no-show-raw-insn", code_object], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"llvm-objdump failed on {code_object}:\n{r.stderr}")
    return mla_prologue_loads(r.stdout)


def mla_prologue_loads(disassembly: str) -> int:
    """Vector-memory instructions between sparse_mla_kernel's index DMA and the vmcnt wait for it, in a
    disassembly listing; raises when they are fewer than the wait's count."""
    lines, inside = [], False
    for line in disassembly.splitlines():
        if "<_ZN3dsa12_GLOBAL__N_117sparse_mla_kernel" in line:
            inside = True
            continue
        if inside and line.endswith(">:"):
            break
        if inside:
            lines.append(line.split("//")[0].strip())
    dma = next((i for i, l in enumerate(lines) if l.startswith("global_load_lds_dword ")), None)
    if dma is None:
        raise RuntimeError("sparse_mla_kernel: index DMA (global_load_lds_dword) not found in the assembly")
    for l in lines[dma + 1:]:
        if l.startswith("s_waitcnt") and "vmcnt(" in l:
            wait = l
            break
    else:
        raise RuntimeError("sparse_mla_kernel: no vmcnt wait after the index DMA")
    n = int(wait.split("vmcnt(")[1].split(")")[0])
    end = lines.index(wait, dma + 1)
    issued = sum(1 for l in lines[dma + 1:end] if l.split(" ")[0].startswith(VMEM_PREFIXES))
    if issued < n:
        raise RuntimeError(f"sparse_mla_kernel: {issued} vector-memory instructions between the index DMA and "
                           f"'{wait}'; the wait needs at least {n} (the DMA could still be in flight)")
    return issued


def build(extra_flags=(), verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    check_mla_prologue_wait(os.path.join(BUILD, "sparse_mla.hip.co"))
    if verbose:
        print(f"built {LIB}")
    return LIB


PROBE_SRC = os.path.join(PKG, "probe", "peaks.hip")
PROBE_LIB = os.path.join(PKG, "probe", "libpeaks.so")


def build_probe(verbose: bool = False) -> str:
    """The benchmark's achievable-peak probes (stream read, bf16 MFMA loop): probe/libpeaks.so."""
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, *CFLAGS, "-shared", PROBE_SRC, "-o", tmp], "hipcc peaks.hip")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)
    build_probe(verbose=True)
