"""Check, on the gfx950 assembly of the fold kernels, that the cache-row loads they issue as
inline assembly (the per-head wide fold's keys; the dense narrow fold's key and value
rows) are safe: on every control-flow path from such a load, its destination registers
are neither read nor written by any instruction before the `; keys` marker that ties them
to the kernel's explicit vmcnt wait.

usage: python -m latent_decode_attention_lla_amd.check_key_loads [asm.s ...]
(without an argument both sources are compiled to assembly with the library's flags)"""
import os
import re
import subprocess
import sys
import tempfile

REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def regs(text):
    out = set()
    for m in REG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


# the kernels whose nontemporal loads are all inline assembly: the per-head wide fold and
# the narrow fold's ring instances (chunks in flight > 0), dense and paged; the narrow
# fold's two-buffer instances load with ordinary, compiler-tracked loads
KERNELS = re.compile(r"^(_Z\S*decode_fold_head_kernel\S*|_Z\S*decode_rotary_fold_kernel\S*ELi[1-9]\d*ELb[01]E\S*):", re.M)
SOURCES = ("decode_fold_wide.hip", "decode_rotary_fold.hip")


def functions(asm):
    for m in KERNELS.finditer(asm):
        end = asm.index(".Lfunc_end", m.end())
        yield m.group(1), asm[m.end():end].splitlines()


def check_function(lines):
    # instructions with their block structure
    insts, labels = [], {}
    for ln in lines:
        t = ln.split(";;")[0].rstrip() if ";;" in ln else ln.rstrip()
        st = ln.strip()
        if re.match(r"^\.LBB\w+:", st):
            labels[st.split(":")[0]] = len(insts)
            insts.append(("label", st))
            continue
        if st.startswith("; keys"):
            insts.append(("hold", st))
            continue
        if not st or st.startswith(";") or st.startswith("."):
            continue
        insts.append(("inst", t.strip()))

    def succ(i):
        kind, text = insts[i]
        op = text.split()[0] if kind == "inst" else ""
        out = []
        if op.startswith("s_branch"):
            out.append(labels[text.split()[1]])
        elif op.startswith("s_cbranch"):
            out.append(labels[text.split()[1]])
            out.append(i + 1)
        elif op.startswith("s_endpgm") or op.startswith("s_setpc"):
            pass
        else:
            out.append(i + 1)
        return [j for j in out if j < len(insts)]

    loads = [i for i, (k, t) in enumerate(insts)
             if k == "inst" and re.match(r"global_load_dwordx[24] .* nt$", t) and "off" not in t.split(",")[1]]
    problems = []
    for i in loads:
        if not insts[i][1].split(",")[2].strip().startswith("s["):
            problems.append((insts[i][1], "(its base is not in scalar registers)"))
        dst = regs(insts[i][1].split(",")[0])
        seen, stack = set(), [i + 1]
        while stack:
            j = stack.pop()
            if j in seen or j >= len(insts):
                continue
            seen.add(j)
            kind, text = insts[j]
            if kind == "hold":
                if regs(text) & dst:
                    continue  # tied to the wait: this path is done
            elif kind == "inst" and regs(text) & dst:
                problems.append((insts[i][1], text))
                continue
            stack.extend(succ(j))
    return len(loads), problems


def main(argv):
    if argv:
        asm = "\n".join(open(p).read() for p in argv)
    else:
        here = os.path.dirname(os.path.abspath(__file__))
        sys.path.insert(0, os.path.dirname(here))
        from latent_decode_attention_lla_amd import build as B
        parts = []
        with tempfile.TemporaryDirectory() as d:
            for fname in SOURCES:
                out = os.path.join(d, fname + ".s")
                cmd = [B._hipcc(), *B.HIP_FLAGS, *B.FILE_FLAGS.get(fname, []), "-I", B.CSRC,
                       "-x", "hip", "--cuda-device-only", "-S", os.path.join(B.CSRC, fname), "-o", out]
                subprocess.run(cmd, check=True, capture_output=True)
                parts.append(open(out).read())
        asm = "\n".join(parts)
    bad = 0
    for name, lines in functions(asm):
        n, problems = check_function(lines)
        print(f"{name[:90]}: {n} key loads, {len(problems)} unsafe uses")
        for ld, use in problems[:5]:
            print(f"   load  {ld}\n   use   {use}")
        bad += len(problems)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
