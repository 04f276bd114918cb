"""Properties of the gfx950 assembly the kernels compile to (host only: the
sources are compiled here with the library's flags and the .s files read).

- No packed fp32 arithmetic (v_pk_fma_f32, v_pk_mul_f32, v_pk_add_f32): the
  build disables the feature, and this checks that nothing brings it back.
- Every direct-to-LDS load (global_load_lds_dwordx4, issued from inline
  assembly) takes a 64-bit VGPR address. With an SGPR base the load reads
  registers that v_readfirstlane writes just before it, and a VMEM read of a
  VALU-written SGPR needs five wait states that the compiler does not insert
  for inline assembly.
- The Newton-Schulz GEMM kernels use no scratch (no register spills): a
  spill reload inside the main loop would also break its explicit
  vmcnt accounting.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from muon_adamw_amd import build as mbuild

CSRC = mbuild.CSRC


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("isa")

    def compile_one(src):
        sub = d / os.path.splitext(src)[0]
        sub.mkdir()
        cmd = [mbuild._hipcc(), *mbuild.FLAGS, "-c", os.path.join(CSRC, src), "-o", str(sub / "k.o"), "-save-temps"]
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=sub)
        assert r.returncode == 0, r.stderr[-2000:]
        stem = os.path.splitext(src)[0]
        with open(sub / f"{stem}-hip-amdgcn-amd-amdhsa-{mbuild.ARCH}.s") as f:
            return src, f.read()

    with ThreadPoolExecutor(min(len(mbuild.SOURCES), 8)) as ex:
        return dict(ex.map(compile_one, mbuild.SOURCES))


def kernels(text):
    """(name, body, private segment bytes) of every kernel in a .s file."""
    res = []
    for m in re.finditer(r"^(_Z\S+):\s*;?.*$", text, flags=re.M):
        name = m.group(1)
        end = text.find("s_endpgm", m.end())
        body = text[m.end():end]
        seg = re.search(rf"\.amdhsa_kernel {re.escape(name)}\n(.*?)\.end_amdhsa_kernel", text, flags=re.S)
        priv = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", seg.group(1)).group(1)) if seg else 0
        res.append((name, body, priv))
    return res


def test_no_packed_fp32_arithmetic(asm):
    for src, text in asm.items():
        assert not re.search(r"\bv_pk_(fma|mul|add)_f32\b", text), src


VGPR_ADDRESS = re.compile(r"global_load_lds_dword\S*\s+v\[\d+:\d+\],\s*off\b")


def test_address_form_check_rejects_an_sgpr_base():
    assert VGPR_ADDRESS.search("global_load_lds_dwordx4 v[12:13], off")
    assert not VGPR_ADDRESS.search("global_load_lds_dwordx4 v8, s[10:11]")


def test_direct_loads_take_vgpr_addresses(asm):
    n = 0
    for src, text in asm.items():
        for line in re.findall(r"global_load_lds_dword\S*[^\n]*", text):
            n += 1
            assert VGPR_ADDRESS.search(line), (src, line)
    assert n > 0   # the Newton-Schulz GEMMs do use them


def test_newton_schulz_kernels_do_not_spill(asm):
    found = 0
    for name, body, priv in kernels(asm["k_ns_mfma.hip"]):
        if "ns_" not in name:
            continue
        found += 1
        assert priv == 0, name
        assert "scratch_" not in body, name
    assert found > 0


# The direct loads read M0 (the LDS destination) as well as their VGPR
# address. The hazard rules of the GCN/CDNA ISA for that operand: an SALU
# write of M0 needs one wait state before a load that writes LDS through it,
# and a VALU write of an SGPR (v_readfirstlane and friends) needs five before
# a VMEM instruction reads it. The check walks back from every direct load
# over the instructions in front of it.
_INSTR = re.compile(r"^\s+([a-z_][a-z0-9_]*)\b(.*)$")


def _instructions(text):
    """(opcode, operands) per instruction; a branch target label becomes
    ("<label>", name), since control can enter there from elsewhere."""
    out = []
    for line in text.splitlines():
        if re.match(r"^\.?L\w*:", line):
            out.append(("<label>", line.split(":")[0]))
            continue
        m = _INSTR.match(line)
        if m and not line.lstrip().startswith((";", ".")):
            out.append((m.group(1), m.group(2).split(";")[0].strip()))
    return out


def _writes_m0(op, args):
    return args.split(",")[0].strip() == "m0" and not op.startswith(("global_", "buffer_", "ds_", "s_waitcnt"))


def _wait_states(op, args):
    if op == "s_nop":
        return int(args, 0) + 1
    return 1


def m0_hazards(text):
    """(index, reason) for every direct load whose M0 write comes too close."""
    ins = _instructions(text)
    bad = []
    for i, (op, args) in enumerate(ins):
        if not op.startswith("global_load_lds_dword"):
            continue
        states, found = 0, False
        for j in range(i - 1, max(-1, i - 64), -1):
            pop, pargs = ins[j]
            if _writes_m0(pop, pargs):
                need = 1 if pop.startswith("s_") else 5
                if states < need:
                    bad.append((i, f"{pop} {pargs} then {states} wait state(s) before {op}"))
                found = True
                break
            if pop == "<label>" or pop.startswith(("s_branch", "s_cbranch", "s_setpc", "s_endpgm")):
                break
            states += _wait_states(pop, pargs)
        if not found:   # M0 set in another basic block: not provable from here
            bad.append((i, f"no M0 write in the straight-line code before {op}"))
    return bad


def test_m0_hazard_check_catches_close_writes():
    ok = "\ts_mov_b32 m0, s4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v[0:1], off\n"
    assert m0_hazards(ok) == []
    salu_close = "\ts_mov_b32 m0, s4\n\tglobal_load_lds_dwordx4 v[0:1], off\n"
    assert len(m0_hazards(salu_close)) == 1
    valu = "\tv_readfirstlane_b32 m0, v4\n\ts_nop 0\n\tv_add_u32 v1, v2, v3\n\tglobal_load_lds_dwordx4 v[0:1], off\n"
    assert len(m0_hazards(valu)) == 1
    valu_far = "\tv_readfirstlane_b32 m0, v4\n\ts_nop 4\n\tglobal_load_lds_dwordx4 v[0:1], off\n"
    assert m0_hazards(valu_far) == []
    across_label = "\ts_mov_b32 m0, s4\n\ts_nop 0\n.LBB0_3:\n\tglobal_load_lds_dwordx4 v[0:1], off\n"
    assert len(m0_hazards(across_label)) == 1


def test_direct_loads_respect_m0_wait_states(asm):
    n = 0
    for src, text in asm.items():
        n += text.count("global_load_lds_dword")
        assert m0_hazards(text) == [], src
    assert n > 0
