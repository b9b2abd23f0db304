"""Checks on the gfx950 assembly of the library's own kernels (CPU only):
every kernel computes on the matrix cores with the instruction of its dtype,
the large-tile kernels use no scratch memory, fit the 160 KiB LDS, load
operands straight into LDS and stream their outputs."""
from __future__ import annotations

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    from implicit_gemm_convolution_amd import build

    out = tmp_path_factory.mktemp("asm")
    path = build.assembly(str(out))
    text = open(path).read()
    kernels = {}
    for name in sorted(set(re.findall(r"^\s+\.amdhsa_kernel (\S+)", text, re.M))):
        start = re.search(r"^" + re.escape(name) + r":", text, re.M)
        assert start, name
        body = text[start.end():].split(".Lfunc_end", 1)[0]
        meta = text.split(".amdhsa_kernel " + name, 1)[1].split(".end_amdhsa_kernel", 1)[0]
        demangled = subprocess.run(["c++filt", name], capture_output=True, text=True).stdout.strip()
        kernels[demangled] = (body, meta)
    assert kernels
    return kernels


@pytest.fixture(scope="module")
def tiled(asm):
    """The tiled LDS kernels (igc::gemm_kernel<...>)."""
    return {k: v for k, v in asm.items() if "gemm_kernel<" in k}


INT_KINDS = (2, 4)  # u8 x i8 GEMM and convolution


def _params(demangled):
    m = re.search(r"gemm_kernel<(\d+), (\d+), (\d+), (\d+), (\d+), (true|false), (\d+), (\d+)>", demangled)
    assert m, demangled
    kind, bm, bn, wm, wn = (int(m.group(i)) for i in range(1, 6))
    return kind, bm, bn, m.group(6) == "true"


def test_every_kernel_uses_mfma_of_its_dtype(tiled):
    for name, (body, _) in tiled.items():
        kind, bm, bn, fast = _params(name)
        # 16 x 16 output blocks: on MI355X they sustain a higher clock than the
        # 32 x 32 forms within the power limit
        want = "v_mfma_i32_16x16x64_i8" if kind in INT_KINDS else "v_mfma_f32_16x16x32_f16"
        assert want in body, name
        others = {"v_mfma_f32_16x16x32_f16", "v_mfma_i32_16x16x64_i8",
                  "v_mfma_f32_32x32x16_f16", "v_mfma_i32_32x32x32_i8"} - {want}
        for other in others:
            assert other not in body, (name, other)


def test_no_scratch_in_main_loops_and_lds_within_limit(tiled):
    for name, (body, meta) in tiled.items():
        kind, bm, bn, fast = _params(name)
        lds = int(re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", meta).group(1))
        assert lds <= 160 * 1024, name
        scratch = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", meta).group(1))
        # no scratch access between the first and the last MFMA, in any kernel
        lines = body.splitlines()
        mf = [i for i, l in enumerate(lines) if "v_mfma" in l]
        assert not any(l.strip().startswith("scratch_") for l in lines[mf[0]:mf[-1] + 1]), name
        if bn == 256 and kind not in INT_KINDS:
            assert scratch == 0, (name, scratch)
        if bn == 256 and kind in INT_KINDS:
            var = int(re.search(r"gemm_kernel<(?:[^,]+, ){6}(\d+),", name).group(1))
            if var & 4:
                # whole requantize-only tiles: the epilogue has one path; without
                # zero-point sums nothing spills (the 8192^3 requantize GEMM)
                assert scratch <= (0 if var == 4 or bm != 256 else 16), (name, scratch)
            else:
                # the u8 x i8 256x256 epilogue (all 256 accumulator registers
                # live across its two paths) spills a few accumulators once per tile
                assert scratch <= (256 if bm == 256 else 0), (name, scratch)


def test_fast_kernels_load_straight_into_lds_and_stream_outputs(tiled):
    for name, (body, _) in tiled.items():
        kind, bm, bn, fast = _params(name)
        if not fast:
            continue
        assert re.search(r"buffer_load_dwordx4 v\d+, s\[\d+:\d+\], (0|s\d+) offen lds", body), name
        assert re.search(r"global_store_dword(x4)? .* nt", body), name


def test_no_packed_fp32_and_no_fma_in_epilogue_math(tiled):
    for name, (body, _) in tiled.items():
        assert "v_pk_add_f32" not in body and "v_pk_mul_f32" not in body and "v_pk_fma_f32" not in body
        kind, *_ = _params(name)
        if kind in INT_KINDS:  # requantize: two separately rounded operations
            # (the epilogue follows the last MFMA; integer division lowering
            # elsewhere may use fused ops of its own)
            epi = body[body.rfind("v_mfma"):]
            assert "v_fma_f32" not in epi and "v_fmac_f32" not in epi and "v_fmamk_f32" not in epi, name


def test_zero_point_sums_on_matrix_cores_where_accumulators_fit(tiled):
    # u8 x i8 kernels with zero-point sums: one extra MFMA per block and
    # k-step (a fragment of ones), no v_dot4, except at 256x256 where the
    # tile's accumulators fill all 256 accumulator registers.
    seen = 0
    for name, (body, _) in tiled.items():
        m = re.search(r"gemm_kernel<(\d+), (\d+), (\d+), \d+, \d+, (true|false), (\d+), \d+>", name)
        # (the sums are the low two bits of the kernel's VAR argument)
        kind, bm, bn, sums = int(m.group(1)), int(m.group(2)), int(m.group(3)), int(m.group(5)) & 3
        if kind not in INT_KINDS or sums == 0:
            continue
        dot4 = "v_dot4" in body
        if bm == 256 and bn == 256:
            assert dot4, name
        else:
            assert not dot4, name
            seen += 1
    assert seen > 0


def test_bypass_kernel_uses_no_lds(asm):
    # the LDS-bypass fp16 kernel: MFMA operands loaded straight into
    # registers, no LDS, no barrier, no scratch; 16-byte streaming stores
    found = [k for k in asm if "gemm_f16_bypass_kernel" in k]
    assert found
    for name in found:
        body, meta = asm[name]
        assert "v_mfma_f32_16x16x32_f16" in body
        assert int(re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", meta).group(1)) == 0
        assert int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", meta).group(1)) == 0
        assert "ds_read" not in body and "ds_write" not in body and "s_barrier" not in body
        assert re.search(r"global_store_dwordx4 .* nt", body), name


def _sgprs(tok):
    tok = tok.strip().rstrip(",")
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    if m:
        return {int(m.group(1))}
    return {"m0"} if tok == "m0" else set()


def test_direct_to_lds_loads_respect_sgpr_hazards(asm):
    """The direct-to-LDS loads are inline assembly, which the compiler's hazard
    recognizer does not see reading its scalar operands.  A vector memory
    instruction may read an SGPR written by a VALU instruction only five wait
    states later, and M0 one wait state after a scalar write; the main-loop
    loads carry one wait state of their own, the prologue's five.  Check every
    such load of every kernel: no VALU write of its descriptor, offset or M0
    within the five wait states before it, and no M0 write right before it."""
    checked = 0
    for name, (body, _) in asm.items():
        lines = [l.split(";")[0].strip() for l in body.splitlines()]
        ins = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
        for i, l in enumerate(ins):
            if not (l.startswith("buffer_load") and l.endswith(" lds")):
                continue
            checked += 1
            ops = l.split(None, 1)[1].replace(" offen", "").replace(" lds", "").split(",")
            reads = set().union(*[_sgprs(o) for o in ops[1:]]) | {"m0"}
            ws, j = 0, i - 1
            while j >= 0 and ws < 5:
                prev = ins[j]
                op = prev.split()[0]
                dst = _sgprs(prev.split(None, 1)[1].split(",")[0]) if " " in prev else set()
                assert not (op.startswith("v_") and dst & reads), (name, ws, prev, l)
                assert not (op.startswith("s_") and "m0" in dst and ws < 1), (name, prev, l)
                ws += int(prev.split()[1], 0) + 1 if op == "s_nop" else 1
                j -= 1
    assert checked > 1000


# Scalar ALU instructions that set SCC, and those that read it.
_SCC_WRITE = re.compile(r"^s_(add|sub|addk|addc|subb|min|max|and|or|xor|andn2|orn2|nand|nor|xnor|lshl|lshr|ashr|bfe|"
                        r"cmp|cmpk|bitcmp|not|abs|absdiff|bcnt|quadmask|wqm|lshl\d_add)\w*")
_SCC_READ = re.compile(r"^s_(cselect|cbranch_scc|addc|subb|cmov|cmovk)\w*")


def scc_reads_after_asm(body):
    """Instructions that read SCC while its last writer was an inline-asm
    block (an SCC clobber the asm did not declare), in program order."""
    bad, in_asm, asm_writes, scc_from_asm = [], False, False, False
    for line in body.splitlines():
        t = line.split(";")[0].strip()
        if ";;#ASMSTART" in line:
            in_asm, asm_writes = True, False
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            scc_from_asm = scc_from_asm or asm_writes
            continue
        if not t or t.startswith("."):
            if t.startswith(".LBB"):
                scc_from_asm = False  # a join: other paths reach it
            continue
        op = t.split()[0]
        if in_asm:
            asm_writes = asm_writes or bool(_SCC_WRITE.match(op))
            continue
        if _SCC_READ.match(op) and scc_from_asm:
            bad.append(t)
        if _SCC_WRITE.match(op):
            scc_from_asm = False
    return bad


def test_no_scc_read_across_asm(asm):
    """The inline-asm blocks that set SCC declare it clobbered, so no
    compiled comparison is kept in SCC across one."""
    for name, (body, _) in asm.items():
        assert not scc_reads_after_asm(body), (name, scc_reads_after_asm(body)[:4])


def test_no_compiler_vmcnt_wait_in_fast_main_loops(tiled):
    """The K loop's memory waits are the kernel's own (vmcnt with lgkmcnt(0),
    counting the direct-to-LDS loads in flight).  A wait the compiler inserts
    there (for a load it still counts as outstanding, e.g. one carried round
    the stream-K segment loop) would drain the operand loads every K tile."""
    for name, (body, _) in tiled.items():
        kind, bm, bn, fast = _params(name)
        if not fast:
            continue
        lines = [l.split(";")[0].strip() for l in body.splitlines()]
        lines = [l for l in lines if l and not l.startswith(".")]
        mf = [i for i, l in enumerate(lines) if l.startswith("v_mfma")]
        stray = [l for l in lines[mf[0]:mf[-1]] if l.startswith("s_waitcnt") and "vmcnt" in l and "lgkmcnt(0)" not in l]
        assert not stray, (name, stray[:2])


def test_stream_k_count_is_released_and_acquired_at_device_scope(tiled):
    """A split tile's partial sums cross XCDs, each with its own L2: before a
    workgroup counts itself in, its L2 is written back and the write-back has
    completed; after the count, the caches are invalidated before a last
    contributor reads the others' partials."""
    n = 0
    for name, (body, _) in tiled.items():
        lines = [l.split(";")[0].strip() for l in body.splitlines()]
        lines = [l for l in lines if l and not l.startswith(".")]
        at = [i for i, l in enumerate(lines) if l.startswith("global_atomic_add")]
        if not at:
            continue
        n += 1
        i = at[0]
        wb = [k for k in range(max(0, i - 40), i) if lines[k].startswith("buffer_wbl2") and "sc1" in lines[k]]
        assert wb, (name, "no L2 write-back before the count")
        assert any(l.startswith("s_waitcnt") and "vmcnt(0)" in l for l in lines[wb[-1] + 1:i]), \
            (name, "the count does not wait for the write-back")
        inv = [k for k in range(i + 1, min(len(lines), i + 20)) if lines[k].startswith("buffer_inv") and "sc1" in lines[k]]
        assert inv, (name, "no invalidation after the count")
        assert any(l.startswith("s_waitcnt") and "vmcnt(0)" in l for l in lines[i + 1:inv[0]]), name
    assert n > 0  # the stream-K kernels are compiled


def _vregs(tok):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _wide_store_data(ins):
    op, _, rest = ins.partition(" ")
    ops = [o.strip() for o in rest.split(",")]
    if re.match(r"(buffer|scratch)_store_(dwordx[34]|b96|b128)", op):
        return _vregs(ops[0])
    if re.match(r"(global|flat)_store_(dwordx[34]|b96|b128)", op):
        return _vregs(ops[1])
    return set()


def test_no_vector_write_of_a_wide_store_s_data_right_after_it(asm):
    """A store of more than 8 bytes reads its data registers after it issues:
    a vector write to them within the next two wait states can reach the
    store.  (The compiler pads buffer stores only when their scalar offset is
    not a register; the stream-K partial tiles, stored with the slot in the
    scalar offset, had their first value replaced by the next store's offset.)"""
    for name, (body, _) in asm.items():
        lines = [l.split(";")[0].strip() for l in body.splitlines()]
        lines = [l for l in lines if l and not l.startswith(".")]
        for i, ins in enumerate(lines):
            data = _wide_store_data(ins)
            if not data:
                continue
            waits = 0
            for nxt in lines[i + 1:i + 3]:
                if waits >= 2:
                    break
                m = re.match(r"s_nop (\d+)", nxt)
                if m:
                    waits += int(m.group(1)) + 1
                    continue
                if nxt.startswith("v_") and " " in nxt:
                    assert not (_vregs(nxt.split(" ", 1)[1].split(",")[0].strip()) & data), (name, ins, nxt)
                waits += 1
