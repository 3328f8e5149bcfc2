"""Builds libpgqa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree, and
libpgqa_probe.so, the benchmark's streaming-read probe (not part of the
attention path)."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# decode / prefill attention, and the QK-norm + RoPE prep
SRCS = [os.path.join(PKG, "csrc", "pgqa.hip"), os.path.join(PKG, "csrc", "prep.hip")]
LIB = os.path.join(PKG, "libpgqa.so")
PROBE_SRCS = [os.path.join(PKG, "csrc", "read_probe.hip")]
PROBE_LIB = os.path.join(PKG, "libpgqa_probe.so")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-command-line-argument",
    # packed-FP32 VALU ops stay off (device side; the host pass ignores it)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: no AGPR<->VGPR copies around the VALU
    # rescaling of the output accumulators
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def build(extra=(), out=LIB, verbose=False, srcs=None):
    """Compile ``srcs`` (default: the attention library's sources) into ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra) + ["-I", INCLUDE] + list(SRCS if srcs is None else srcs) + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err)
    os.replace(tmp, out)
    return out


def build_probe(verbose=False):
    return build(out=PROBE_LIB, verbose=verbose, srcs=PROBE_SRCS)


def build_all(verbose=False):
    return build(verbose=verbose), build_probe(verbose=verbose)


if __name__ == "__main__":
    print(build_all(verbose=True))
