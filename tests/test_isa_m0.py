"""The direct-to-LDS loads' use of M0 in the generated gfx950 code.

The kernels move tiles into LDS with global_load_lds_dwordx4 (and the 4-byte
form for the low-bit rows), written as inline asm that first sets M0 (the LDS
destination base) and names M0 as clobbered.  The compiler treats M0 as a reserved register and warns that such
a clobber may not be honoured, so the kernels are only correct while the
compiler itself never keeps a value of its own in M0.  This test compiles
every source that uses the loads and checks, in each kernel, that M0 appears
only as the destination of the helper's s_mov_b32, directly followed by the
load.  CPU only (cross-compiles).
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "head_latent_attention_absorb_amd", "csrc")
SOURCES = ["decode_mfma.hip", "combine_out.hip", "absorb_out.hip", "prefill.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

M0 = re.compile(r"\bm0\b")
# Instructions that read M0 without naming it (indexed moves, messages, GWS,
# the lane-indexed LDS forms, VGPR-index mode, interpolation, buffer loads
# into LDS).
IMPLICIT_M0 = ("s_movrel", "v_movrel", "s_sendmsg", "ds_gws", "s_set_gpr_idx", "ds_read_addtid",
               "ds_write_addtid", "v_interp", "s_ttracedata")


def instructions(asm):
    """(kernel, [instruction lines]) for every kernel body in the assembly."""
    out, name, body = [], None, []
    for raw in asm.splitlines():
        line = raw.split(";")[0].rstrip()
        if not line.strip():
            continue
        if re.match(r"^[A-Za-z_][\w.$]*:", line) and not line.startswith("."):
            if name is not None:
                out.append((name, body))
            name, body = line.split(":")[0], []
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            out.append((name, body))
            name, body = None, []
            continue
        s = line.strip()
        if s.startswith((".", "-")) or s.endswith(":"):
            continue
        body.append(s)
    return out


def m0_problems(body):
    problems = []
    for k, ins in enumerate(body):
        mnem = ins.split()[0]
        if mnem.startswith(IMPLICIT_M0) or (mnem.startswith("buffer_") and " lds" in ins):
            problems.append(f"{ins!r} reads M0")
            continue
        if mnem.startswith("global_load_lds_") and not (k > 0 and M0.search(body[k - 1])):
            problems.append(f"{ins!r} without the helper's M0 set in front")
            continue
        if not M0.search(ins):
            continue
        ok = (re.match(r"^s_mov_b32\s+m0\s*,\s*s\d+$", ins) is not None and k + 1 < len(body)
              and body[k + 1].startswith("global_load_lds_"))
        if not ok:
            problems.append(f"{ins!r} (next: {body[k + 1] if k + 1 < len(body) else None!r})")
    return problems


@pytest.fixture(scope="module")
def compiled():
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from head_latent_attention_absorb_amd.build import FLAGS
    out = {}
    for src in SOURCES:
        r = subprocess.run([HIPCC, *FLAGS, "-I", CSRC, "--cuda-device-only", "-S",
                            os.path.join(CSRC, src), "-o", "-"], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        out[src] = instructions(r.stdout)
    return out


def test_m0_is_only_the_direct_load_base(compiled):
    n_loads = 0
    for src, kernels in compiled.items():
        assert kernels, src
        for name, body in kernels:
            problems = m0_problems(body)
            assert not problems, f"{src} {name}:\n" + "\n".join(problems[:10])
            n_loads += sum(1 for ins in body if ins.startswith("global_load_lds_"))
    assert n_loads > 100  # every source above stages through direct loads


def test_checker_flags_other_uses_of_m0():
    """Compiler uses of M0 (indexed moves, which read it implicitly) and a
    set of M0 that is not followed by the load are reported; the helper's
    pair is not."""
    asm = """
_Z6kernelv:
\ts_mov_b32 m0, s4
\tglobal_load_lds_dwordx4 v[2:3], off
\ts_mov_b32 m0, s5
\tv_add_f32 v1, v2, v3
\ts_movrels_b32 s0, s1
\tv_movrels_b32 v0, v1 ; reads m0 implicitly
\ts_endpgm
.Lfunc_end0:
"""
    (name, body), = instructions(asm)
    assert name == "_Z6kernelv"
    problems = m0_problems(body)
    assert len(problems) == 3, problems
    assert any("s_mov_b32 m0, s5" in p for p in problems)
    assert any("s_movrels_b32" in p and "reads M0" in p for p in problems)
    assert any("v_movrels_b32" in p and "reads M0" in p for p in problems)
    assert not m0_problems(body[:2])  # the helper's pair alone passes
