"""Instruction-level checks of the built library (CPU only: disassembles libmxgemm.so).

The global->LDS DMA is inline assembly, and the compiler's hazard pass does not
check inline assembly for the gfx9 rule that a vector-memory instruction may
read an SGPR written by a VALU instruction (v_readfirstlane, v_readlane,
v_cmp, carry-out adds) only 5 or more wait states later.  Missing wait states
make the load use a stale buffer resource at random, so the library is checked
here rather than trusted:

* every LDS DMA is directly preceded by "s_mov_b32 m0, ..." and "s_nop 3" (the
  5 wait states the DMA macro carries, which hold whatever came before);
* no buffer or global memory instruction, compiler-made ones included, reads
  an SGPR that a VALU instruction wrote fewer than 5 wait states before it
  in straight-line code;
* the RoPE kernels and the GEMM with the projection epilogue hold no fused
  multiply-add: the rotation rounds each product and the sum on its own, and
  the compiler forms an FMA from such code unless contraction is off;
* no GEMM kernel instance touches scratch memory inside a loop (a register
  spill there would cost every K step), and the instances with 8-bit operands
  and sf = 32 (the large workloads' kernels) spill nothing at all: the lane
  geometry is held across a tile only where the registers allow it.

The disassembly is of device code built in this repository from its sources.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_scaled_precision_e4m3_amd", "libmxgemm.so")
LLVM = "/opt/rocm/llvm/bin"


def _tool(name):
    path = os.path.join(LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


@pytest.fixture(scope="module")
def code_objects(tmp_path_factory):
    """The library's gfx950 code objects, one per translation unit."""
    if not os.path.exists(LIB):
        pytest.skip("libmxgemm.so is not built")
    objcopy, bundler, objdump = _tool("llvm-objcopy"), _tool("clang-offload-bundler"), _tool("llvm-objdump")
    if not (objcopy and bundler and objdump):
        pytest.skip("LLVM binary tools not found")
    d = tmp_path_factory.mktemp("isa")
    fatbin = str(d / "fatbin.bin")
    subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fatbin}", LIB, str(d / "host.tmp")],
                   check=True, capture_output=True)
    # one offload bundle per translation unit, each starting with the bundle magic
    data = open(fatbin, "rb").read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [i for i in range(0, len(data), 8) if data.startswith(magic, i)]
    assert starts, "no offload bundle in the library"
    codes = []
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
        part, code = str(d / f"bundle{n}.bin"), str(d / f"gfx950_{n}.hsaco")
        with open(part, "wb") as f:
            f.write(data[a:b])
        subprocess.run([bundler, "--unbundle", "--type=o", f"--input={part}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={code}"],
                       check=True, capture_output=True)
        codes.append(code)
    return codes


@pytest.fixture(scope="module")
def disasm_text(code_objects):
    objdump = _tool("llvm-objdump")
    return "".join(subprocess.run([objdump, "-d", "--mcpu=gfx950", "--no-show-raw-insn", code],
                                  check=True, capture_output=True, text=True).stdout for code in code_objects)


@pytest.fixture(scope="module")
def kernel_spills(code_objects):
    """Kernel name -> vector registers spilled, from the code objects' metadata notes."""
    readelf = _tool("llvm-readelf")
    if not readelf:
        pytest.skip("llvm-readelf not found")
    spills = {}
    for code in code_objects:
        notes = subprocess.run([readelf, "--notes", code], check=True, capture_output=True, text=True).stdout
        for kernel in notes.split("  - .")[1:]:
            name = re.search(r"\.name:\s+(\S+)", kernel)
            count = re.search(r"\.vgpr_spill_count:\s+(\d+)", kernel)
            if name and count:
                spills[name.group(1)] = int(count.group(1))
    assert spills, "no kernel metadata found"
    return spills


@pytest.fixture(scope="module")
def disasm(disasm_text):
    out = disasm_text
    insts = []
    for line in out.split("\n"):
        text = line.split("//")[0].strip()
        if not text or text.endswith(":") or text.startswith("Disassembly") or "file format" in text:
            continue
        insts.append(text)
    assert len(insts) > 10000, "unexpectedly small disassembly"
    return insts


def _ops(inst):
    parts = inst.split(None, 1)
    return parts[0], ([o.strip() for o in parts[1].split(",")] if len(parts) > 1 else [])


def _sgprs(tok):
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    if m:
        return {int(m.group(1))}
    if tok in ("vcc", "vcc_lo", "vcc_hi"):
        return {"vcc"}
    return set()


_CARRY_OUT = ("v_add_co_u32", "v_sub_co_u32", "v_subrev_co_u32", "v_addc_co_u32", "v_subb_co_u32",
              "v_subbrev_co_u32", "v_div_scale", "v_mad_u64_u32", "v_mad_i64_i32")


def _valu_sgpr_defs(mn, ops):
    if not mn.startswith("v_") or not ops:
        return set()
    d = set()
    if mn.startswith(("v_readfirstlane", "v_readlane", "v_cmp")):
        d |= _sgprs(ops[0])
    if mn.startswith(_CARRY_OUT) and len(ops) > 1:
        d |= _sgprs(ops[1])
    return d


def _wait_states(mn, ops):
    return int(ops[0], 0) + 1 if mn == "s_nop" else 1


def test_lds_dma_carries_its_wait_states(disasm):
    n = 0
    for i, inst in enumerate(disasm):
        if inst.startswith("buffer_load_dwordx4") and inst.endswith(" lds"):
            n += 1
            assert disasm[i - 1] == "s_nop 3", f"LDS DMA without its s_nop 3: {disasm[i - 2:i + 1]}"
            assert disasm[i - 2].startswith("s_mov_b32 m0,"), f"LDS DMA without its m0 write: {disasm[i - 2:i + 1]}"
    assert n > 1000, f"only {n} LDS DMA instructions found"


def _find_hazards(insts):
    """(VALU def, wait states, VMEM use) for every VMEM read of an SGPR a VALU wrote < 5 wait states before."""
    bad, checked = [], 0
    for i, inst in enumerate(insts):
        mn, ops = _ops(inst)
        if not mn.startswith(("buffer_", "global_", "tbuffer_")):
            continue
        reads = set()
        for t in ops[1:]:
            reads |= _sgprs(t)
        if not reads:
            continue
        checked += 1
        ws, j = 0, i - 1
        while j >= 0 and ws < 5:
            mn2, ops2 = _ops(insts[j])
            if mn2 == "s_endpgm":
                break
            if _valu_sgpr_defs(mn2, ops2) & reads:
                bad.append((insts[j], ws, inst))
            ws += _wait_states(mn2, ops2)
            j -= 1
    return bad, checked


def test_hazard_scan_finds_a_planted_hazard():
    # the pattern of a DMA macro with a single wait state after v_readfirstlane
    planted = ["v_readfirstlane_b32 s66, v7", "s_mov_b32 m0, s3", "s_nop 0",
               "buffer_load_dwordx4 v4, s[64:67], 0 offen lds"]
    bad, checked = _find_hazards(planted)
    assert checked == 1 and len(bad) == 1 and bad[0][1] == 2
    fixed = ["v_readfirstlane_b32 s66, v7", "s_mov_b32 m0, s3", "s_nop 3",
             "buffer_load_dwordx4 v4, s[64:67], 0 offen lds"]
    assert _find_hazards(fixed)[0] == []


def test_no_valu_sgpr_to_vmem_hazard(disasm):
    bad, checked = _find_hazards(disasm)
    assert checked > 1000
    assert not bad, f"{len(bad)} VALU-SGPR -> VMEM hazards, e.g. {bad[:3]}"


def test_rotation_kernels_hold_no_fused_multiply_add(disasm_text):
    # functions by their "<symbol>:" labels; the RoPE kernels and the GEMM
    # instantiations with the projection epilogue (C type 4, 256x256 tiles)
    funcs = re.split(r"\n(?=[0-9a-f]+ <[^>]+>:)", disasm_text)
    checked = 0
    for f in funcs:
        m = re.match(r"[0-9a-f]+ <([^>]+)>:", f)
        if not m:
            continue
        name = m.group(1)
        if "proj_rope_mxfp8_kernel" in name or "ELi4ELi256ELi0E" in name:
            checked += 1
            fused = _FUSED.findall(f)
            assert not fused, f"{name}: {fused[:3]}"
    assert checked >= 3, "expected the RoPE kernels and the projection-epilogue GEMMs"


_FUSED = re.compile(r"\bv_(?:fma|fmac|mad|mac|pk_fma)\w*?_f32")


def test_fused_multiply_add_pattern():
    for inst in ("v_fma_f32 v1, v2, v3, v4", "v_fmac_f32_e32 v1, v2, v3", "v_pk_fma_f32 v[0:1], v[2:3], v[4:5], v[6:7]",
                 "v_mad_f32 v1, v2, v3, v4", "v_fma_mix_f32 v1, v2, v3, v4"):
        assert _FUSED.search(inst), inst
    for inst in ("v_mad_u64_u32 v[0:1], s[0:1], v2, v3, 0", "v_mul_f32_e32 v1, v2, v3", "v_sub_f32_e32 v1, v2, v3"):
        assert not _FUSED.search(inst), inst


def test_sf32_gemm_kernels_with_8bit_operands_do_not_spill(kernel_spills):
    # mxgemm_amax_big_kernel<SF, FA, FB, MODE, CT, BT, MJ, NW>: FA == 2 is packed FP4
    gemm = {k: v for k, v in kernel_spills.items() if "mxgemm_amax_big_kernel" in k}
    assert len(gemm) > 50, "fewer GEMM kernel instances than expected"
    checked = 0
    for name, count in gemm.items():
        args = re.search(r"kernelILi(\d+)ELi(\d+)ELi(\d+)E", name)
        assert args, name
        if args.group(1) != "32" or args.group(2) == "2":
            continue
        checked += 1
        assert count == 0, f"{name} spills {count} vector registers"
    assert checked > 20


def _loops(text, name_part):
    """(function name, instructions of one loop body) for every backward branch in the
    functions whose name holds name_part."""
    for func in re.split(r"\n(?=[0-9a-f]{16} <)", text):
        head = re.match(r"([0-9a-f]{16}) <([^>]*)>", func)
        if not head or name_part not in head.group(2):
            continue
        base, lines, addrs = int(head.group(1), 16), func.split("\n"), []
        for line in lines:
            a = re.search(r"// ([0-9A-F]{12}):", line)
            addrs.append(int(a.group(1), 16) if a else None)
        for i, line in enumerate(lines):
            br = re.search(r"s_cbranch_\w+ \d+.*<[^>]*\+0x([0-9a-f]+)>", line)
            if not br or addrs[i] is None:
                continue
            target = base + int(br.group(1), 16)
            if target >= addrs[i] or target not in addrs:
                continue
            j = addrs.index(target)
            yield head.group(2), [x.split("//")[0].strip() for x in lines[j:i + 1] if "//" in x]


def test_no_scratch_access_inside_gemm_loops(disasm_text):
    loops = list(_loops(disasm_text, "mxgemm_amax_big_kernel"))
    assert len(loops) > 100, "fewer loops than the GEMM instances hold"
    assert any(sum(i.startswith("v_mfma") for i in body) >= 32 for _, body in loops), "no K loop found"
    for name, body in loops:
        bad = [i for i in body if i.startswith("scratch_")]
        assert not bad, f"{name}: scratch access in a loop: {bad[:2]}"


def test_loop_finder_sees_a_planted_scratch_access():
    text = ("0000000000001000 <_Z22mxgemm_amax_big_kernel_test>:\n"
            "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15] // 000000001000: 00000000\n"
            "\tscratch_load_dword v1, off, s0 // 000000001008: 00000000\n"
            "\ts_cbranch_scc1 65533 // 000000001010: 00000000 <_Z22mxgemm_amax_big_kernel_test+0x0>\n")
    loops = list(_loops(text, "mxgemm_amax_big_kernel"))
    assert len(loops) == 1 and any(i.startswith("scratch_") for i in loops[0][1])
