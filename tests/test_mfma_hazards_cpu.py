"""The two D = 512 attention kernels form S^T with VGPR-form MFMAs written as asm
statements (common.h: mfma_v_first, mfma_v, mfma_v_fence), so the compiler pads no hazard
for them.  This test compiles both files (sparse_attn_wide.hip, sparse_attn_wide_lse.hip)
to gfx950 assembly with the library's own flags and checks, instruction by instruction,
the rules the source relies on:

* each such MFMA and the fence after its chain (one asm statement of two `s_nop 7`, 16 wait
  states; this MFMA shape needs 8 before a vector instruction reads its result) lie in one
  basic block: no label or branch between them, so the compiler has no block join at
  which it would copy the still-changing result registers;
* between an MFMA and that fence no instruction reads or writes its result registers,
  except later MFMAs of the same chain that take exactly them as C;
* no vector instruction writes an MFMA source register in the 2 wait states before it.

A planted slip (a vector read of a result before the fence) is caught.
"""
import os
import re
import subprocess

import pytest

from deepseek_v4_csa_amd import build as B

SOURCES = {   # file: (extra flags as the library builds it, kernel symbol pattern)
    "sparse_attn_wide.hip": ([], r"^(_ZN3csa23sparse_attn_wide_kernelILi\d+EE\S*):"),
    "sparse_attn_wide_lse.hip": (B.VGPR_FORM, r"^(_ZN3csa27sparse_attn_wide_lse_kernel\S*):"),
}


def compile_asm(tmp_path, name="sparse_attn_wide.hip"):
    out = tmp_path / (name + ".s")
    src = os.path.join(B.CSRC, "kernels", name)
    cmd = [B.HIPCC, *B.FLAGS, *SOURCES[name][0], "--cuda-device-only", "-S", "-x", "hip", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr[-2000:])
    return out.read_text()


def kernels(asm, pattern):
    """{name: [(kind, text)]} with kind 'I' (instruction), 'L' (label), 'AS'/'AE' (asm
    statement start / end markers)."""
    res, cur = {}, None
    kre = re.compile(pattern)
    for line in asm.split("\n"):
        m = kre.match(line)
        if m:
            cur = res.setdefault(m.group(1), [])
            continue
        if cur is None:
            continue
        if line.startswith(".Lfunc_end"):
            cur = None
            continue
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            cur.append(("AS", t))
        elif t.startswith(";;#ASMEND"):
            cur.append(("AE", t))
        elif re.match(r"^\.LBB\S*:", t) or re.match(r"^; %bb\.\d+:", t):
            cur.append(("L", t))
        else:
            t = t.split(";")[0].strip()
            if t and not t.startswith("."):
                cur.append(("I", t))
    return res


def vregs(tok):
    tok = tok.strip()
    m = re.match(r"^v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"^v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def parse(t):
    op = t.split()[0]
    rest = t[len(op):].strip()
    return op, [x.strip() for x in rest.split(",")] if rest else []


def wait_states(t):
    op, args = parse(t)
    return int(args[0], 0) + 1 if op == "s_nop" else 1


def is_vgpr_mfma(t):
    op, args = parse(t)
    return op.startswith("v_mfma") and bool(args) and args[0].startswith("v")


def fence_positions(ins):
    """Indices of asm statements that are exactly two s_nop 7."""
    out = []
    for i, (k, _) in enumerate(ins):
        if k != "AS":
            continue
        body = []
        j = i + 1
        while j < len(ins) and ins[j][0] != "AE":
            body.append(ins[j][1])
            j += 1
        if [b.replace("\t", " ") for b in body] == ["s_nop 7", "s_nop 7"]:
            out.append(j)
    return out


def findings(ins):
    bad = []
    fences = fence_positions(ins)
    n_mfma = 0
    for i, (k, t) in enumerate(ins):
        if k != "I" or not is_vgpr_mfma(t):
            continue
        n_mfma += 1
        _, a = parse(t)
        D, A, Bs = vregs(a[0]), vregs(a[1]), vregs(a[2])
        C = vregs(a[3]) if len(a) > 3 else set()
        nxt = [f for f in fences if f > i]
        if not nxt:
            bad.append(("no fence after", t))
            continue
        for kk, tt in ins[i + 1:nxt[0]]:
            if kk == "L":
                bad.append(("block boundary before the fence", t, tt))
                break
            if kk != "I":
                continue
            op2, a2 = parse(tt)
            if op2.startswith("s_cbranch") or op2 in ("s_branch", "s_setpc_b64"):
                bad.append(("branch before the fence", t, tt))
                break
            if is_vgpr_mfma(tt):
                C2 = vregs(a2[3]) if len(a2) > 3 else set()
                if (vregs(a2[1]) | vregs(a2[2])) & D:
                    bad.append(("result used as A/B", t, tt))
                if C2 & D and C2 != D:
                    bad.append(("partial C overlap", t, tt))
                if vregs(a2[0]) & D and C2 != D:
                    bad.append(("result overwritten", t, tt))
            else:
                used = set()
                for x in a2:
                    used |= vregs(x)
                if used & D:
                    bad.append(("result touched before the fence", t, tt))
        ws, j = 0, i - 1
        while j >= 0 and ws < 2:
            kk, tt = ins[j]
            if kk == "L":
                break
            if kk == "I":
                op2, a2 = parse(tt)
                if op2.startswith("v_") and not op2.startswith("v_mfma") and a2 and vregs(a2[0]) & (A | Bs | C):
                    bad.append(("source written by a vector instruction too late", t, tt))
                ws += wait_states(tt)
            j -= 1
    return n_mfma, bad


@pytest.fixture(scope="module")
def wide_kernels(tmp_path_factory):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    ks = {}
    for name, (_, pattern) in SOURCES.items():
        ks.update(kernels(compile_asm(tmp_path_factory.mktemp("asm"), name), pattern))
    # the three- and four-tile instantiations of the second kernel, and the lse kernel
    assert len(ks) >= 3, sorted(ks)
    return ks


def test_vgpr_mfma_hazard_rules(wide_kernels):
    for name, ins in wide_kernels.items():
        n, bad = findings(ins)
        assert n >= 64, (name, n)   # 64 per step
        assert not bad, (name, bad[:5])


def test_planted_read_before_fence_is_caught(wide_kernels):
    ins = list(next(iter(wide_kernels.values())))
    i = next(i for i, (k, t) in enumerate(ins) if k == "I" and is_vgpr_mfma(t))
    d = min(vregs(parse(ins[i][1])[1][0]))
    ins.insert(i + 1, ("I", f"v_add_f32_e32 v{d}, v{d}, v{d}"))
    _, bad = findings(ins)
    assert any(b[0] == "result touched before the fence" for b in bad)


def test_planted_branch_before_fence_is_caught(wide_kernels):
    ins = list(next(iter(wide_kernels.values())))
    i = next(i for i, (k, t) in enumerate(ins) if k == "I" and is_vgpr_mfma(t))
    ins.insert(i + 1, ("L", ".LBB0_999:"))
    _, bad = findings(ins)
    assert any(b[0] == "block boundary before the fence" for b in bad)
