"""Builds libffpa.so in-tree: hipcc for gfx950, one object per (element type, head dim) kernel,
compiled in parallel, plus the C-ABI object, linked into exact_attention_head_amd/libffpa.so."""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libffpa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          # no packed-fp32 instructions in generated code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-result", "-I", os.path.join(PKG, "..", "include")]


def _dims(macro: str) -> list[int]:
    src = "ffpa_bwd_launch.hpp" if macro.startswith("FFPA_BWD") else "ffpa_launch.hpp"
    with open(os.path.join(CSRC, src)) as f:
        txt = f.read()
    body = txt[txt.index(f"#define {macro}(X)"):]
    one_line = macro != "FFPA_FOR_EACH_D"  # the others are one-line macros
    body = body[:body.index("\n")] if one_line else body[:body.index("\n\n")]
    return [int(x) for x in re.findall(r"X\((\d+)\)", body)]


def head_dims() -> list[int]:
    """Head dims with compiled 16-bit kernels."""
    return _dims("FFPA_FOR_EACH_D")


def fp8_head_dims() -> list[int]:
    """Head dims with compiled fp8 kernels."""
    return _dims("FFPA_FP8_FOR_EACH_D")


def bwd_kernel_dims() -> list[int]:
    """Kernel head dims of the fused backward."""
    return _dims("FFPA_BWD_FOR_EACH_KD")


def bwd_pad_kernel_dims() -> list[int]:
    """Kernel head dims of the fused backward that also serve smaller head dims (columns skipped)."""
    return _dims("FFPA_BWD_PAD_KD")


def _compile(src: str, obj: str, defines: list[str], remarks: bool = False) -> tuple[str, str]:
    """Compiles one object, keeping its gfx950 assembly next to it (obj with .s) for the hazard check."""
    work = obj + ".tmp.d"
    shutil.rmtree(work, ignore_errors=True)
    os.makedirs(work)
    cmd = [HIPCC, *COMMON, *defines, "-save-temps", "-c", os.path.abspath(src), "-o", os.path.abspath(obj)]
    if remarks:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=work)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(obj)}:\n{r.stderr[-4000:]}")
    asm = [f for f in os.listdir(work) if f.endswith(f"-hip-amdgcn-amd-amdhsa-{ARCH}.s")]
    if asm:
        os.replace(os.path.join(work, asm[0]), obj[:-2] + ".s")
    shutil.rmtree(work, ignore_errors=True)
    return obj, r.stderr


def kernel_resources(asm_path: str) -> dict:
    """Per-kernel resources from the code-object metadata in a saved gfx950 assembly file:
    {mangled name: {vgpr, agpr, sgpr, vgpr_spill, sgpr_spill, scratch, lds}}."""
    with open(asm_path) as f:
        txt = f.read()
    i = txt.find("amdhsa.kernels:")
    if i < 0:
        return {}
    j = txt.find("amdhsa.target", i)
    out = {}
    fields = [("vgpr", "vgpr_count"), ("agpr", "agpr_count"), ("sgpr", "sgpr_count"),
              ("vgpr_spill", "vgpr_spill_count"), ("sgpr_spill", "sgpr_spill_count"),
              ("scratch", "private_segment_fixed_size"), ("lds", "group_segment_fixed_size")]
    for blk in re.split(r"\n  - ", txt[i:j if j > 0 else None])[1:]:
        m = re.search(r"\.name:\s+(\S+)", blk)
        if not m:
            continue
        res = {}
        for key, field in fields:
            v = re.search(r"\." + field + r":\s+(\d+)", blk)
            res[key] = int(v.group(1)) if v else 0
        out[m.group(1)] = res
    return out


def spills(resources: dict) -> list[str]:
    """Kernels that spill VGPRs or use scratch memory (SGPR spills go to VGPR lanes, not memory)."""
    return [f"{name}: {r['vgpr_spill']} VGPRs spilled, {r['scratch']} B/lane scratch"
            for name, r in resources.items() if r["vgpr_spill"] > 0 or r["scratch"] > 0]


def build(jobs: int | None = None, verbose: bool = True, report: bool = False) -> str:
    """Compiles every kernel and links libffpa.so; returns its path.  Always rebuilds."""
    t0 = time.time()
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or max(1, min(16, os.cpu_count() or 4))
    tasks = [(os.path.join(CSRC, "ffpa_api.hip"), os.path.join(BUILD, "ffpa_api.o"), []),
             (os.path.join(CSRC, "ffpa_bwd.hip"), os.path.join(BUILD, "ffpa_bwd.o"), []),
             (os.path.join(CSRC, "ffpa_dropout.hip"), os.path.join(BUILD, "ffpa_dropout.o"), [])]
    # per (element type, head dim): part 0 the launcher with the plain variants, 1 the dropout
    # variants, 2 the staged-mask variants (compiled in parallel)
    for tag in ("Bf16", "Fp16"):
        for d in head_dims():
            for part in (0, 1, 2):
                tasks.append((os.path.join(CSRC, "ffpa_inst.hip"),
                              os.path.join(BUILD, f"ffpa_{tag.lower()}_d{d}" + (f"_p{part}" if part else "") + ".o"),
                              [f"-DFFPA_INST_T={tag}", f"-DFFPA_INST_D={d}", f"-DFFPA_INST_PART={part}"]))
    # the fp8 forward: one object per head dim
    for d in fp8_head_dims():
        tasks.append((os.path.join(CSRC, "ffpa_fp8.hip"), os.path.join(BUILD, f"ffpa_fp8_d{d}.o"),
                      [f"-DFFPA_FP8_D={d}"]))
    # the fused backward: one object per kernel head dim (and one for its padded head dims)
    for kd in bwd_kernel_dims():
        tasks.append((os.path.join(CSRC, "ffpa_bwd_inst.hip"), os.path.join(BUILD, f"ffpa_bwdk_d{kd}.o"),
                      [f"-DFFPA_BWD_KD={kd}", "-DFFPA_BWD_PAD=0"]))
    for kd in bwd_pad_kernel_dims():
        tasks.append((os.path.join(CSRC, "ffpa_bwd_inst.hip"), os.path.join(BUILD, f"ffpa_bwdk_d{kd}_p1.o"),
                      [f"-DFFPA_BWD_KD={kd}", "-DFFPA_BWD_PAD=1"]))
    # largest kernels first
    kd = lambda path: re.search(r"_d(\d+)(_p\d)?\.o$", path)  # per-head-dim kernel objects
    tasks.sort(key=lambda t: -int(kd(t[1]).group(1)) if kd(t[1]) else 0)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s, o, d, False) for s, o, d in tasks]
        for f in cf.as_completed(futs):
            f.result()
    objs = [o for _, o, _ in tasks]
    # resource gate: no kernel may spill VGPRs or use scratch memory
    resources = {}
    for o in objs:
        if os.path.exists(o[:-2] + ".s"):
            resources.update(kernel_resources(o[:-2] + ".s"))
    bad = spills(resources)
    if bad:
        raise RuntimeError("kernels spill registers to scratch memory:\n" + "\n".join(bad))
    # the kernels' inline assembly relies on rules the compiler does not check: verify them
    sys.path.insert(0, PKG)
    try:
        from check_mfma_hazards import check as check_hazards
    finally:
        sys.path.remove(PKG)

    hazards = []
    for o in objs:
        if kd(o):
            hazards += check_hazards(o[:-2] + ".s")
    if hazards:
        raise RuntimeError("MFMA / LDS hazards in the generated code:\n" + "\n".join(hazards[:20]))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] {LIB} ({len(objs)} objects, {time.time() - t0:.0f}s, {jobs} jobs)", flush=True)
    if report:
        names = sorted(resources)
        dem = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True).stdout.split("\n")
        for name, pretty in zip(names, dem):
            print(f"[build] {pretty or name}: {resources[name]}", flush=True)
        print(f"[build] {len(resources)} kernels, none spills", flush=True)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    build(report="--report" in sys.argv)
