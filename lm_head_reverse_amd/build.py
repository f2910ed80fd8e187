"""Build librkl.so (HIP, gfx950) in-tree with hipcc.

    python -m lm_head_reverse_amd.build          # writes lm_head_reverse_amd/librkl.so

Three checks fail the build:
* register spills: hipcc's per-kernel resource-usage remarks must report no
  VGPR spill and no scratch memory for any kernel (a spill puts per-lane
  scratch traffic into the loops of the MFMA kernels);
* packed fp32: the device code is compiled without the packed-fp32
  instructions (v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32), and the built
  gfx950 code object is disassembled to confirm none is present.  (The host
  pass of hipcc does not know the feature and says it ignores it; the device
  pass honours it.)
* M0: the LDS DMA (global_load_lds_dwordx4) is issued from inline asm that
  sets M0, the LDS base the instruction reads, right before it (the saddr
  form with a 32-bit per-lane offset; the compiler builtin measured 31 %
  slower on the backward).  The disassembly must show M0 written only there,
  each write followed at once by its DMA instruction, and no other
  instruction that reads M0 -- so the clobber of this reserved register
  (which hipcc warns about) cannot disturb compiler-generated code.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librkl.so")
SOURCES = ["rkl_kernels.hip", "rkl_api.hip", "rkl_noalloc.hip"]
ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_NOISE = "'-packed-fp32-ops' is not a recognized feature"
PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def hipcc() -> str:
    for c in (os.path.join(ROCM, "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build librkl.so)")


def kernel_resources(diag: str) -> dict:
    """{kernel symbol: {remark key: value}} from -Rpass-analysis=kernel-resource-usage."""
    out, cur = {}, None
    for line in diag.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([^:]+?): (\S+) \[-Rpass-analysis=kernel-resource-usage\]", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


def check_spills(res: dict) -> list[str]:
    bad = []
    for name, r in res.items():
        spill = int(r.get("VGPRs Spill", "0"))
        scratch = int(r.get("ScratchSize [bytes/lane]", "0"))
        if spill or scratch:
            bad.append(f"{name}: {spill} VGPRs spilled, {scratch} scratch bytes per lane")
    return bad


def disassemble(lib: str) -> list[str]:
    """Instructions of the gfx950 code object of the built library."""
    objdump = os.path.join(ROCM, "llvm", "bin", "llvm-objdump")
    with tempfile.TemporaryDirectory() as d:
        copy = os.path.join(d, "lib.so")
        shutil.copy(lib, copy)
        subprocess.run([objdump, "--offloading", copy], check=True, capture_output=True, text=True, cwd=d)
        objs = [os.path.join(d, f) for f in os.listdir(d) if ARCH in f]
        if not objs:
            raise RuntimeError(f"no {ARCH} code object found in {lib}")
        insts = []
        for o in objs:
            dis = subprocess.run([objdump, "-d", o], check=True, capture_output=True, text=True).stdout
            for line in dis.splitlines():
                text = line.split("//")[0].strip()
                if text and not text.endswith(":") and not text.startswith(("Disassembly", ".", "<")):
                    insts.append(text)
        return insts


# instructions that read M0 without naming it
IMPLICIT_M0 = re.compile(r"^(s_sendmsg|s_sendmsghalt|ds_gws_|ds_append|ds_consume|s_movrel|v_movrel|v_interp_|"
                         r"buffer_load_\w*lds|global_load_lds|scratch_load_lds|ds_bvh)")


def m0_violations(insts: list[str]) -> list[str]:
    bad = []
    for i, ins in enumerate(insts):
        if re.search(r"\bm0\b", ins):
            if not re.match(r"^s_mov_b32 m0, s\d+$", ins):
                bad.append(ins)
            elif i + 1 >= len(insts) or not insts[i + 1].startswith("global_load_lds_dwordx4"):
                bad.append(f"{ins} (not followed by its DMA instruction)")
        elif IMPLICIT_M0.match(ins) and not (ins.startswith("global_load_lds_dwordx4") and i > 0
                                             and re.match(r"^s_mov_b32 m0, s\d+$", insts[i - 1])):
            bad.append(f"{ins} (reads M0 without the DMA's own write before it)")
    return bad


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source for gfx950, link librkl.so and run the checks; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
           # no packed-fp32 instructions in the generated code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Rpass-analysis=kernel-resource-usage",
           "-Wall", "-Wno-unused-function",
           # the M0 clobber of the DMA asm; m0_violations checks the code instead
           "-Wno-inline-asm",
           f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES],
           "-o", tmp]
    if extra:
        cmd[1:1] = extra
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    diag = r.stdout + r.stderr
    if r.returncode != 0:
        sys.stderr.write(diag)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    res = kernel_resources(diag)
    if not res:
        raise RuntimeError("hipcc printed no kernel resource-usage remarks")
    bad = check_spills(res)
    if bad:
        os.remove(tmp)
        raise RuntimeError("register spills:\n  " + "\n  ".join(bad))
    msgs = [l for l in diag.splitlines() if ("warning:" in l or "error:" in l) and HOST_NOISE not in l]
    if msgs and verbose:
        print("\n".join(msgs))
    insts = disassemble(tmp)
    hits = [i for i in insts if PACKED_FP32.search(i)]
    if hits:
        os.remove(tmp)
        raise RuntimeError(f"{len(hits)} packed-fp32 instructions in the device code, e.g. {hits[0]}")
    bad = m0_violations(insts)
    if bad:
        os.remove(tmp)
        raise RuntimeError("M0 used outside the DMA asm:\n  " + "\n  ".join(bad[:10]))
    os.replace(tmp, LIB)
    if verbose:
        print(f"{len(res)} kernels: no VGPR spills, no scratch; no packed-fp32 instructions; M0 written only "
              f"by the DMA asm ({sum(i.startswith('s_mov_b32 m0') for i in insts)} sites)", flush=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
