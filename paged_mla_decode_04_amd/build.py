"""Compile the HIP library libmla_decode.so in-tree for gfx950.

Usage: python -m paged_mla_decode_04_amd.build   (or __graft_entry__.build()).
hipcc cross-compiles the device code without a GPU present.
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libmla_decode.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["mla_api.hip", "mla_kernels.hip", "mla_decode_wide.hip", "mla_cache.hip"]
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep hipcc from forming packed fp32 ops on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# Kernels whose output accumulators live in fixed AGPRs that only inline
# assembly touches: the compiler must not use any AGPR itself there (it would
# spill into them and overwrite the accumulators).
FIXED_AGPR_SOURCES = ["mla_decode_wide.hip"]
_ASM_AGPR = re.compile(r"accvgpr|\ba\[\d|[ ,]a\d+\b")


def check_fixed_agprs(src: str) -> None:
    """Fail if the compiler itself references AGPRs, spills VGPRs or uses scratch memory in the
    kernel's assembly."""
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "k.s")
        cmd = [hipcc(), *HIPCC_FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc -S failed for {src}:\n" + r.stdout.decode(errors="replace"))
        in_asm = False
        bad = []
        with open(out) as f:
            for line in f:
                if ";;#ASMSTART" in line:
                    in_asm = True
                    continue
                if ";;#ASMEND" in line:
                    in_asm = False
                    continue
                code = line.split(";", 1)[0]
                if not in_asm and code.startswith("\t") and _ASM_AGPR.search(code):
                    bad.append(code.strip())
        if bad:
            raise RuntimeError(f"{src}: the compiler uses AGPRs reserved for the accumulators "
                               f"(register pressure too high?): {bad[:4]}")
        with open(out) as f:
            check_no_scratch(f.read(), src)
        if src == "mla_decode_wide.hip":
            check_score_reads_ahead(out, src)
            with open(out) as f:
                check_m0_only_in_copies(f.read(), src)
        check_mfma_operand_hazards(out, src)


_WIDE_KERNEL = re.compile(r"^_ZN\S*decode_wide_kernel\S*:")
_SCORE_MFMA = re.compile(r"^\s*v_mfma_f32_32x32x16_bf16 v\[")
_LGKM = re.compile(r"s_waitcnt\b.*lgkmcnt\((\d+)\)")
SCORE_STEPS = 36  # score MFMAs per chunk (576 / 16)


def check_score_reads_ahead(path: str, src: str) -> None:
    """Fail if the wide kernel's common-step score product waits for all LDS
    reads before more than its last MFMA.  Each score MFMA should wait only
    for the K fragment read a few MFMAs earlier (lgkmcnt(3)); the compiler
    turns that into a full drain (lgkmcnt(0)) when it believes a scalar load,
    which shares the counter and returns out of order, may still be in
    flight -- one change elsewhere in the kernel did exactly that and cost 5%
    of the compute-bound call.  The common step is found by the short wait
    that opens its value product (an s_nop 3 in the assembly) and its 36 score
    MFMAs (the ones writing VGPRs) before it."""
    with open(path) as f:
        lines = f.read().split("\n")
    starts = [i for i, l in enumerate(lines) if _WIDE_KERNEL.match(l)]
    if not starts:
        raise RuntimeError(f"{src}: no decode_wide_kernel in the assembly")
    for start in starts:
        nop = next((i for i in range(start, len(lines)) if lines[i].strip() == "s_nop 3"), None)
        if nop is None:
            raise RuntimeError(f"{src}: common step not found (no s_nop 3 after {lines[start][:60]})")
        waits, k = [], nop
        while len(waits) < SCORE_STEPS and k > start:
            k -= 1
            if _SCORE_MFMA.match(lines[k]):
                w = None
                for j in range(k - 1, max(start, k - 12), -1):
                    m = _LGKM.search(lines[j])
                    if m:
                        w = int(m.group(1))
                        break
                    if _SCORE_MFMA.match(lines[j]):
                        break
                waits.append(w)
        if len(waits) < SCORE_STEPS:
            raise RuntimeError(f"{src}: fewer than {SCORE_STEPS} score MFMAs before the common step's value product")
        drains = sum(1 for w in waits if w == 0)
        if drains > 1:
            raise RuntimeError(f"{src}: {drains} score MFMAs of the common step wait for every LDS read "
                               f"(lgkmcnt(0)): the reads ahead are lost ({lines[start][:60]})")


_M0 = re.compile(r"\bm0\b")
_M0_COPY = re.compile(r"^s_add_u32 m0, s\d+, 0x[0-9a-f]+$|^s_add_u32 m0, s\d+, \d+$")


def check_m0_only_in_copies(text: str, src: str) -> None:
    """Fail if anything but the wide kernel's own chunk copies touches M0.
    Each copy sets M0 (its LDS address) inside the same assembly block as its
    LDS-direct load and lists M0 as clobbered; the compiler treats M0 as
    reserved, and does not promise to keep a value of its own in M0 across
    such a block, so the copies are only safe while the compiler uses M0 for
    nothing else in these kernels."""
    bad = []
    for line in text.split("\n"):
        code = line.split(";", 1)[0].strip()
        if code and not code.startswith(".") and _M0.search(code) and not _M0_COPY.match(code):
            bad.append(code)
    if bad:
        raise RuntimeError(f"{src}: M0 is used outside the chunk copies: {bad[:4]}")


def check_no_scratch(text: str, src: str) -> None:
    """Fail if a kernel in the assembly `text` spills VGPRs or uses scratch memory at all: a
    variable the compiler keeps in memory (an array indexed at run time, or one captured by
    a call it did not inline) is scratch traffic without a spill."""
    spills = [int(m.group(1)) for m in re.finditer(r"\.vgpr_spill_count:\s+(\d+)", text)]
    if any(spills):
        raise RuntimeError(f"{src}: the compiler spills VGPRs to scratch memory ({spills})")
    scratch = [int(m.group(1)) for m in re.finditer(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", text)]
    if any(scratch):
        raise RuntimeError(f"{src}: the kernel uses scratch memory ({scratch} bytes per lane)")


_REG = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)\b")


def _regs(tok: str):
    out = set()
    for m in _REG.finditer(tok):
        if m.group(1):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def check_mfma_operand_hazards(asm_path: str, src: str) -> None:
    """Fail if a VALU write reaches an MFMA operand with fewer than 2 wait states.

    The kernel's MFMAs are inline assembly, so the compiler's hazard recognizer
    does not see them; this walks back from each one over every control-flow
    path (fall-through and every branch into a label on the way), counting
    wait states; a branch instruction itself is not counted as one.
    """
    insts = []    # instruction text, or ("LABEL", name)
    with open(asm_path) as f:
        for line in f:
            code = line.split(";", 1)[0].rstrip()
            if not code.strip():
                continue
            if not code.startswith("\t"):
                if code.endswith(":"):
                    insts.append(("LABEL", code[:-1]))
                continue
            t = code.strip()
            if not t.startswith("."):
                insts.append(t)
    branches = {}  # label name -> indexes of the branches that target it
    for k, t in enumerate(insts):
        if isinstance(t, str) and (t.startswith("s_cbranch") or t.startswith("s_branch")):
            branches.setdefault(t.split()[-1], []).append(k)

    def ends_flow(t) -> bool:
        return isinstance(t, str) and (t.startswith("s_branch") or t.startswith("s_endpgm")
                                       or t.startswith("s_setpc"))

    bad = []

    def walk(j: int, ws: int, src_regs: set, mfma: str, seen: set) -> None:
        while j >= 0 and ws < 2:
            pt = insts[j]
            if isinstance(pt, tuple):
                for b in branches.get(pt[1], []):
                    if (b, ws) not in seen:
                        seen.add((b, ws))
                        walk(b - 1, ws, src_regs, mfma, seen)
                if j == 0 or ends_flow(insts[j - 1]):
                    return
                j -= 1
                continue
            if pt.startswith("s_cbranch") or pt.startswith("s_branch"):
                j -= 1
                continue
            if pt.startswith("s_nop"):
                ws += int(pt.split()[-1], 0) + 1
            else:
                if pt.startswith("v_") and not pt.startswith("v_mfma") and len(pt.split()) > 1:
                    if _regs(pt.split(None, 1)[1].split(",")[0]) & src_regs:
                        bad.append(f"{pt} -> {mfma}")
                ws += 1
            j -= 1

    for k, t in enumerate(insts):
        if isinstance(t, str) and t.startswith("v_mfma"):
            walk(k - 1, 0, _regs(",".join(t.split(None, 1)[1].split(",")[1:4])), t, set())
    if bad:
        raise RuntimeError(f"{src}: VALU result feeds an MFMA too early: {bad[:4]}")


# An LDS-direct load reads M0; after a write of M0 it needs one wait state,
# which the compiler inserts for the loads it emits itself but not for loads
# written as inline assembly.  The kernels' copies carry their own s_nop; this
# check keeps it so.
LDS_DMA_SOURCES = ["mla_decode_wide.hip", "mla_kernels.hip"]
_WRITES_M0 = re.compile(r"^[sv]_\w+\s+m0\b")


def _instructions(asm_path: str):
    insts = []    # instruction text, or ("LABEL", name)
    with open(asm_path) as f:
        for line in f:
            code = line.split(";", 1)[0].rstrip()
            if not code.strip():
                continue
            if not code.startswith("\t"):
                if code.endswith(":"):
                    insts.append(("LABEL", code[:-1]))
                continue
            t = code.strip()
            if not t.startswith("."):
                insts.append(t)
    return insts


def check_lds_dma_m0_hazards(asm_path: str, src: str) -> None:
    """Fail if an LDS-direct load can follow a write of M0 with no wait state between."""
    insts = _instructions(asm_path)
    branches = {}
    for k, t in enumerate(insts):
        if isinstance(t, str) and (t.startswith("s_cbranch") or t.startswith("s_branch")):
            branches.setdefault(t.split()[-1], []).append(k)
    bad = []

    def ends_flow(t) -> bool:
        return isinstance(t, str) and (t.startswith("s_branch") or t.startswith("s_endpgm")
                                       or t.startswith("s_setpc"))

    def walk(j: int, load: str, seen: set) -> None:
        # the instruction right before the load on this path (labels and branches
        # are not wait states)
        while j >= 0:
            pt = insts[j]
            if isinstance(pt, tuple):
                for b in branches.get(pt[1], []):
                    if b not in seen:
                        seen.add(b)
                        walk(b - 1, load, seen)
                if j == 0 or ends_flow(insts[j - 1]):
                    return
                j -= 1
                continue
            if pt.startswith("s_cbranch") or pt.startswith("s_branch"):
                j -= 1
                continue
            if _WRITES_M0.match(pt):
                bad.append(f"{pt} -> {load}")
            return

    for k, t in enumerate(insts):
        if isinstance(t, str) and t.split()[0].startswith(("buffer_load", "global_load")) and t.endswith(" lds"):
            walk(k - 1, t, set())
    if bad:
        raise RuntimeError(f"{src}: an LDS-direct load follows an M0 write without a wait state: {bad[:4]}")


def check_lds_dma(src: str) -> None:
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "k.s")
        cmd = [hipcc(), *HIPCC_FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc -S failed for {src}:\n" + r.stdout.decode(errors="replace"))
        check_lds_dma_m0_hazards(out, src)
        with open(out) as f:
            check_no_scratch(f.read(), src)


def build(verbose: bool = False) -> str:
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(f"{src}:\n{text}")
        elif verbose and text.strip():
            print(text)
    if failed:
        # never leave a library built from older sources next to failed ones
        if os.path.exists(LIB_PATH):
            os.remove(LIB_PATH)
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    try:
        for src in FIXED_AGPR_SOURCES:
            check_fixed_agprs(src)
        for src in LDS_DMA_SOURCES:
            check_lds_dma(src)
    except RuntimeError:
        if os.path.exists(LIB_PATH):
            os.remove(LIB_PATH)
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
        raise
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        if os.path.exists(LIB_PATH):
            os.remove(LIB_PATH)
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB_PATH)
    for o in objs:
        os.remove(o)
    return LIB_PATH


# A copy of the library whose host code runs under AddressSanitizer and
# UndefinedBehaviorSanitizer (the device code is built as usual): the host-side
# argument checks, the host planner and the status strings then run with every
# out-of-bounds access, use after free and undefined operation reported.  Run a
# CPU test against it with the sanitizer runtime preloaded (asan_runtime()).
SANITIZE_FLAGS = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-omit-frame-pointer -Xarch_host -fno-sanitize-recover=undefined".split()
SANITIZED_DIR = os.path.join(os.path.dirname(HERE), "_build", "sanitized")


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    r = subprocess.run([os.path.join(rocm, "llvm", "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    path = r.stdout.decode().strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"no AddressSanitizer runtime found ({path!r})")
    return path


def build_sanitized() -> str:
    """Build the sanitized copy into _build/sanitized (skipped when it is newer than every source)."""
    out = os.path.join(SANITIZED_DIR, LIB_NAME)
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".h"))]
    srcs.append(os.path.join(os.path.dirname(HERE), "include", "mla_decode.h"))
    if os.path.exists(out) and os.path.getmtime(out) > max(os.path.getmtime(f) for f in srcs):
        return out
    os.makedirs(SANITIZED_DIR, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + SANITIZE_FLAGS
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(SANITIZED_DIR, src.replace(".hip", ".o"))
        cmd = [hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        text, _ = p.communicate()
        if p.returncode != 0:
            failed.append(f"{src}:\n{text.decode(errors='replace')}")
    if failed:
        raise RuntimeError("hipcc (sanitized host code) failed:\n" + "\n".join(failed))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE_FLAGS, *objs, "-o", out + ".tmp"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link (sanitized) failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(out + ".tmp", out)
    for o in objs:
        os.remove(o)
    return out


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized())
    else:
        print(build(verbose="-v" in sys.argv))
