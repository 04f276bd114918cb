"""Builds the library's sources for the CPU simulator (test infrastructure).

Every source of ``muon_adamw_amd/csrc`` is compiled as host C++ against
``tests/cpu_sim/include/hip/hip_runtime.h`` and linked with
``tests/cpu_sim/runtime.cpp`` into ``tests/cpu_sim/_build/libmuon_adamw_sim.so``.
The kernels' own code runs on the CPU that way. Only the inline-assembly
statements are replaced, each by the simulator call with that instruction's
effect: a direct load into LDS by ``hipsim::dma16`` and ``s_waitcnt vmcnt(n)``
(with or without the L1 invalidate before it) by ``hipsim::wait_vm(n)``. Any
other inline assembly stops the build. The replacement keeps every line
number, so sites and diagnostics point at the original source.

The product library (``muon_adamw_amd/libmuon_adamw.so``) is a different
build; nothing in the package loads this one.

Usage: python -m tests.cpu_sim.build [--csrc DIR] [--out LIB]
"""
from __future__ import annotations

import argparse
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "muon_adamw_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD, "libmuon_adamw_sim.so")
SOURCES = ["api.hip", "k_momentum.hip", "k_ns_mfma.hip", "k_ns_f32.hip", "k_rowcol.hip",
           "k_apply.hip", "k_adamw.hip", "k_gradnorm.hip", "k_ceiling.hip"]
CXX = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang++")
FLAGS = ["-std=c++17", "-O2", "-g", "-fPIC", "-pthread", "-Wno-unused-function", "-Wno-psabi"]


class AsmError(ValueError):
    pass


def _scan_parens(text: str, start: int) -> int:
    """Index just past the ')' that closes the '(' before ``start``."""
    depth, p, in_str = 1, start, False
    while depth:
        if p >= len(text):
            raise AsmError("unterminated inline assembly statement")
        ch = text[p]
        if in_str:
            if ch == "\\":
                p += 2
                continue
            if ch == '"':
                in_str = False
        elif ch == '"':
            in_str = True
        elif ch == "(":
            depth += 1
        elif ch == ")":
            depth -= 1
        p += 1
    return p


def _split_top(s: str, sep: str) -> list[str]:
    parts, depth, in_str, cur, i = [], 0, False, [], 0
    while i < len(s):
        ch = s[i]
        if in_str:
            cur.append(ch)
            if ch == "\\":
                cur.append(s[i + 1])
                i += 2
                continue
            if ch == '"':
                in_str = False
        elif ch == '"':
            in_str = True
            cur.append(ch)
        elif ch in "([{":
            depth += 1
            cur.append(ch)
        elif ch in ")]}":
            depth -= 1
            cur.append(ch)
        elif ch == sep and depth == 0:
            parts.append("".join(cur))
            cur = []
        else:
            cur.append(ch)
        i += 1
    parts.append("".join(cur))
    return parts


def _template(s: str) -> str:
    """The assembler template: string literals concatenated, a stringised macro
    parameter (#n) kept as {n}."""
    out, i = [], 0
    for m in re.finditer(r'"((?:[^"\\]|\\.)*)"|#\s*([A-Za-z_]\w*)|(\S)', s):
        if m.group(1) is not None:
            out.append(m.group(1).encode().decode("unicode_escape"))
        elif m.group(2) is not None:
            out.append("{" + m.group(2) + "}")
        else:
            raise AsmError(f"unexpected token {m.group(3)!r} in an assembler template")
    return "".join(out)


def _operands(s: str) -> list[tuple[str, str]]:
    ops = []
    for part in _split_top(s, ","):
        part = part.strip()
        if not part:
            continue
        m = re.fullmatch(r'"([^"]*)"\s*\((.*)\)', part, re.S)
        if not m:
            raise AsmError(f"cannot read the operand {part!r}")
        ops.append((m.group(1), m.group(2).strip()))
    return ops


def translate(inner: str) -> str:
    """The simulator call for the inline assembly ``asm volatile(<inner>)``."""
    parts = _split_top(inner, ":")
    tmpl = " ".join(_template(parts[0]).replace("\n", " ").replace("\t", " ").split())
    outs = _operands(parts[1]) if len(parts) > 1 else []
    ins = _operands(parts[2]) if len(parts) > 2 else []
    if tmpl == "":
        # an empty template only hides a value from the optimiser: no effect here
        return "((void)0)"
    if outs:
        raise AsmError(f"inline assembly with outputs is not simulated: {tmpl!r}")
    m = re.fullmatch(r"(?:s_nop \d+ )?global_load_lds_dwordx4 %0, off", tmpl)
    if m:
        cons = dict(ins)
        if set(cons) != {"v", "{m0}"}:
            raise AsmError(f"direct load with operands {sorted(cons)}")
        return f"::hipsim::dma16(({cons['v']}), ({cons['{m0}']}))"
    m = re.fullmatch(r"(?:buffer_inv sc1 )?s_waitcnt vmcnt\((\d+|\{\w+\})\)(?: lgkmcnt\(\d+\))?", tmpl)
    if m:
        n = m.group(1).strip("{}")
        return f"::hipsim::wait_vm({n})"
    raise AsmError(f"inline assembly not simulated: {tmpl!r}")


def rewrite(text: str) -> str:
    out, i = [], 0
    while True:
        j = text.find("asm volatile(", i)
        if j < 0:
            out.append(text[i:])
            return "".join(out)
        out.append(text[i:j])
        end = _scan_parens(text, j + len("asm volatile("))
        call = translate(text[j + len("asm volatile("):end - 1])
        out.append(call + "\n" * text[j:end].count("\n"))
        i = end


def _command(src_path: str, obj: str, gen_dir: str) -> list[str]:
    text = open(src_path).read()
    if "asm volatile(" in text:
        gen = os.path.join(gen_dir, os.path.basename(src_path) + ".cpp")
        with open(gen, "w") as f:
            f.write(f'#line 1 "{os.path.basename(src_path)}"\n')
            f.write(rewrite(text))
        src_path = gen
    return [CXX, "-x", "c++", *FLAGS, "-I", os.path.join(HERE, "include"), "-I", INCLUDE, "-c", src_path,
            "-o", obj]


def build(csrc: str = CSRC, out: str = LIB, verbose: bool = False, extra=()) -> str:
    """``extra``: more compiler flags for every object and the link (a
    sanitizer, say)."""
    os.makedirs(BUILD, exist_ok=True)
    tag = os.path.splitext(os.path.basename(out))[0]
    objdir = os.path.join(BUILD, tag + "_obj")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
        cmd = _command(os.path.join(csrc, s), obj, objdir)
        cmd[cmd.index("-c"):cmd.index("-c")] = ["-I", csrc, *extra]
        jobs.append((s, cmd, obj))
    rt_obj = os.path.join(objdir, "runtime.o")
    jobs.append(("runtime.cpp", [CXX, *FLAGS, *extra, "-I", os.path.join(HERE, "include"), "-c",
                                 os.path.join(HERE, "runtime.cpp"), "-o", rt_obj], rt_obj))

    def run(job):
        name, cmd, _ = job
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"simulator build of {name} failed:\n{r.stdout}{r.stderr}")
        if verbose and (r.stdout + r.stderr).strip():
            print(r.stdout + r.stderr, file=sys.stderr)

    with ThreadPoolExecutor(min(len(jobs), int(os.environ.get("MAX_JOBS", "8")))) as ex:
        list(ex.map(run, jobs))
    tmp = out + ".tmp"
    r = subprocess.run([CXX, "-shared", "-pthread", *extra, "-o", tmp, *[o for _, _, o in jobs]],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("simulator link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


SELFTEST = os.path.join(BUILD, "libhipsim_selftest.so")


def build_selftest(out: str = SELFTEST) -> str:
    """The simulator's own check kernels (selftest.cpp) with the runtime."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = out + ".tmp"
    r = subprocess.run([CXX, *FLAGS, "-shared", "-I", os.path.join(HERE, "include"), "-o", tmp,
                        os.path.join(HERE, "selftest.cpp"), os.path.join(HERE, "runtime.cpp")],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("simulator self-test build failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--csrc", default=CSRC)
    ap.add_argument("--out", default=LIB)
    ap.add_argument("--ubsan", action="store_true",
                    help="with UndefinedBehaviorSanitizer (load with its runtime preloaded)")
    a = ap.parse_args()
    extra = ("-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-shared-libsan") if a.ubsan else ()
    print(build(a.csrc, a.out, verbose=True, extra=extra))
