"""Build libsparse_mla.so for gfx950 with hipcc, in place inside this package.

    python -m sparse_mla_decode_03_amd.build [--verbose]
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libsparse_mla.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["smla_api.hip", "smla_decode.hip", "smla_merge.hip", "smla_store.hip", "smla_indexer.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_command(out_path: str = LIB_PATH) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU ops stay off: ordinary float code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out_path,
    ]


def decode_asm_command(out_path: str) -> list:
    """The decode source compiled to gfx950 assembly with the library's own flags."""
    cmd = compile_command("-")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    flags = [a for a in cmd[1:] if a not in srcs and a not in ("-shared", "-fPIC", "-o", "-")]
    return [cmd[0], *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "smla_decode.hip"), "-o", out_path]


def _stderr(res) -> str:
    noise = "is not a recognized feature for this target"
    return "\n".join(l for l in res.stderr.splitlines() if noise not in l)


def check_decode_asm(asm_path: str) -> None:
    """Refuse a build whose VGPR-form MFMA accumulator can be touched in flight."""
    from sparse_mla_decode_03_amd import asm_checks  # noqa: PLC0415 (plain module, no torch)
    text = open(asm_path).read()
    if asm_checks.count_vgpr_mfma_kernels(text) == 0:
        raise RuntimeError("decode assembly holds no VGPR-form MFMA: the O-block-15 check found nothing to check")
    bad = asm_checks.vgpr_mfma_violations(text)
    if bad:
        raise RuntimeError("O block 15 may be read or moved while its MFMA is in flight:\n" + "\n".join(bad[:20]))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB_PATH (always recompiles), and check the decode
    kernels' assembly (compiled beside it with the same flags) before installing it."""
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    with tempfile.TemporaryDirectory() as td:
        asm_path = os.path.join(td, "smla_decode.s")
        asm_cmd = decode_asm_command(asm_path)
        asm_proc = subprocess.Popen(asm_cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        asm_out, asm_err = asm_proc.communicate()
        err = _stderr(res)
        if verbose or res.returncode != 0:
            print(" ".join(cmd))
            if err.strip():
                print(err, file=sys.stderr)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
        if asm_proc.returncode != 0:
            print(" ".join(asm_cmd))
            print(asm_err, file=sys.stderr)
            raise RuntimeError(f"hipcc (assembly of the decode kernels) failed with exit code {asm_proc.returncode}")
        if verbose:
            print(" ".join(asm_cmd))
        check_decode_asm(asm_path)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
