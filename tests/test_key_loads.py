"""The per-head wide fold kernel issues its key loads, and the narrow fold over a dense cache
its key and value row loads, as inline assembly, which the compiler neither counts nor
waits for; each kernel's own vmcnt wait orders their use. This checks, on the gfx950
assembly of every instance as built, that no instruction reads or writes such a load's
destination registers before the marker that ties them to that wait, and that every such
load takes a scalar base."""
import pytest

from latent_decode_attention_lla_amd import check_key_loads


def test_key_load_registers_untouched_until_their_wait(capsys):
    rc = check_key_loads.main([])
    out = capsys.readouterr().out
    lines = [ln for ln in out.splitlines() if "key loads" in ln]
    wide = [ln for ln in lines if "decode_fold_head_kernel" in ln]
    narrow = [ln for ln in lines if "decode_rotary_fold_kernel" in ln]
    assert len(wide) == 16, out    # 4 shapes x 2 heads-per-workgroup x dense/paged
    assert len(narrow) == 12, out  # 3 shapes with the ring, 4 and 8 heads, dense and paged
    assert all(" 0 unsafe uses" in ln and not ln.split(":")[1].strip().startswith("0 key") for ln in lines), out
    assert rc == 0, out


def test_checker_flags_a_planted_read(tmp_path):
    asm = """_ZN3lla12_GLOBAL__N_123decode_fold_head_kernelILi128ELi96ELi160ELi4ELb0EEEvNS_10DecodeArgsENS_8PageArgsE:
\tglobal_load_dwordx4 v[92:95], v92, s[0:1] offset:0 nt
\tv_mov_b32_e32 v200, v93
\t; keys v[92:95]
\ts_endpgm
.Lfunc_end0:
"""
    p = tmp_path / "k.s"
    p.write_text(asm)
    assert check_key_loads.main([str(p)]) == 1
    ok = asm.replace("\tv_mov_b32_e32 v200, v93\n", "")
    p.write_text(ok)
    assert check_key_loads.main([str(p)]) == 0
