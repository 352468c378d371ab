"""Compile the HIP sources into libcsahca.so (gfx950) next to this file, and the same
sources with the host code under AddressSanitizer and UndefinedBehaviorSanitizer into
libcsahca_hostsan.so (device code unchanged in kind; used by the CPU tests of the
library's host-side validation)."""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libcsahca.so")
SAN_LIB = os.path.join(HERE, "libcsahca_hostsan.so")
# sanitizers on the host pass only (each -fsanitize right after -Xarch_host); the device
# code is built lightly, as the sanitized library runs no kernel in its tests
SAN_FLAGS = [
    "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_device", "-g0",
    "-Wno-unused-command-line-argument",
]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # device code only: inputs carry no NaNs (saves the NaN-quieting of every fmaxf), and
    # MFMA results stay in ordinary VGPRs (no copies out of accumulation registers)
    "-Xarch_device", "-fno-honor-nans",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose=False, sanitized=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = SAN_LIB if sanitized else LIB
    tmp = out + ".tmp"
    cmd = [hipcc, *(SAN_FLAGS if sanitized else HIPCC_FLAGS), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, sanitized=True))
