"""Checks on the gfx950 machine code of the decode kernel (CPU only: hipcc
cross-compiles; nothing runs on a GPU).

* No scratch (spill) access inside the key loop: a spill reload there is a
  vector-memory load, and the wait for it would also wait for every HBM->LDS
  copy in flight, draining the ring once per tile.
* No scalar-memory stores or atomics anywhere.
* Every HBM->LDS copy (global_load_lds) reads its scalar base no sooner than
  five wait states after a VALU instruction wrote it (the CDNA rule for a
  VALU-written SGPR read by a vector-memory instruction; the compiler cannot
  enforce it across the kernel's inline assembly), on every control-flow
  path into the copy.
* The key loop of the default (bf16, one phase) kernel issues the expected
  MFMAs and LDS reads per 16-key tile.

The default plan runs mla_decode_kernel_pairs (32 keys per step); the
checks cover it, every instantiation of the 16-key kernel, the Q-resident
e4m3 rebuild and both two-waves-per-SIMD candidates (their register budgets,
copy runs and wait literals, and the split candidate's exchange order).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_paged_decode_absorbed_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


SOURCES = {
    "library": os.path.join(CSRC, "decode_kernel.hip"),
    # the two-waves-per-SIMD candidate (opt-in, MLA_DECODE_KERNEL=w8)
    "w8": os.path.join(CSRC, "decode_w8_kernel.hip"),
    # the library's e4m3 kernels with Q resident (opt-in, MLA_DECODE_KERNEL=qres)
    "qres": os.path.join(CSRC, "decode_kernel_qres.hip"),
    # pairs of waves sharing 32 rows (opt-in, MLA_DECODE_KERNEL=split)
    "split": os.path.join(CSRC, "decode_split_kernel.hip"),
}
# kernels per source, and copies per wave and round (a branch-free run);
# None: the kernel waits for its copies with vmcnt(0) only, so no count of
# copies per round enters a wait
EXPECTED_KERNELS = {"library": 6, "w8": 2, "qres": 3, "split": 2}
COPIES_PER_ROUND = {"library": {"bf16": (18, 0), "e4m3": (9, 1)},
                    "w8": {"bf16": (9, 0), "e4m3": None},
                    "qres": {"e4m3": (9, 1)}}


@pytest.fixture(scope="module", params=sorted(SOURCES))
def isa(request, tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "decode_kernel.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           SOURCES[request.param], "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return request.param, out.read_text()


def _kernels(text):
    """{kernel symbol: [(block label, [instruction lines])]}"""
    out = {}
    cur = None
    for line in text.splitlines():
        m = re.match(r"^(_ZN3mla\S*mla_decode_kernel\S*):", line)
        if m:
            cur = [("entry", [])]
            out[m.group(1)] = cur
            continue
        if cur is None:
            continue
        s = line.split(";")[0].strip()
        if s.startswith("s_endpgm"):
            cur = None
            continue
        lab = re.match(r"^(\.LBB\S+):", line)
        if lab:
            cur.append((lab.group(1), []))
        elif s and not s.startswith("."):
            cur[-1][1].append(s)
    return out


def _key_loop_blocks(blocks):
    """Blocks of the key loop: the ones that issue MFMAs."""
    return [(lab, ins) for lab, ins in blocks if any("v_mfma" in i for i in ins)]


def test_all_instantiations_present(isa):
    ks = _kernels(isa[1])
    assert len(ks) == EXPECTED_KERNELS[isa[0]], sorted(ks)


# The e4m3 kernel with four phases (opt-in through MLA_PHASES=4, never chosen
# by the planner) runs out of registers in its key loop; every other
# instantiation, including both defaults, must stay spill-free there.
KNOWN_LOOP_SPILLS = {"ILi1ELi4E"}


def test_no_scratch_access_in_key_loop(isa):
    for name, blocks in _kernels(isa[1]).items():
        if any(k in name for k in KNOWN_LOOP_SPILLS):
            continue
        for lab, ins in _key_loop_blocks(blocks):
            bad = [i for i in ins if i.startswith("scratch_") or
                   (i.startswith("buffer_") and "s[0:3]" in i)]
            assert not bad, f"{name} {lab}: {bad[:3]}"


def test_no_scalar_stores(isa):
    for name, blocks in _kernels(isa[1]).items():
        for lab, ins in blocks:
            bad = [i for i in ins if re.match(r"s_(store|buffer_store|atomic|buffer_atomic|dcache_wb|scratch_store)", i)]
            assert not bad, f"{name} {lab}: {bad[:3]}"


def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _predecessors(blocks):
    """Control-flow predecessors of every block: the block before it (unless
    that one ends in an unconditional branch) and every block branching to it."""
    index = {lab: k for k, (lab, _) in enumerate(blocks)}
    preds = {k: [] for k in range(len(blocks))}
    for k, (_, ins) in enumerate(blocks):
        for i in ins:
            m = re.match(r"s_(?:c)?branch\S*\s+(\.LBB\S+)", i)
            if m and m.group(1) in index:
                preds[index[m.group(1)]].append(k)
        last = ins[-1] if ins else ""
        if k + 1 < len(blocks) and not last.startswith("s_branch"):
            preds[k + 1].append(k)
    return preds


def _wait_states(i):
    op = i.split()[0]
    return int(i.split()[1]) + 1 if op == "s_nop" else 1


EXEC = {"exec", "exec_lo", "exec_hi"}


def _valu_sgpr_writes(p):
    """SGPRs a VALU instruction writes (its first operand if scalar), with
    EXEC named "exec" (v_cmpx_* write it, in either encoding)."""
    op = p.split()[0]
    out = set()
    if not op.startswith("v_") or " " not in p:
        return out
    dst = p.split(None, 1)[1].split(",")[0].strip()
    out |= _sgprs(dst)
    if dst in EXEC or op.startswith("v_cmpx"):
        out.add("exec")
    return out


def test_valu_written_sgpr_not_read_by_lds_copy_within_five_wait_states(isa):
    """Walks back from every copy over all control-flow paths (through
    branches and fall-throughs), not only inside the copy's own block.  The
    registers a copy reads are its scalar base and EXEC (the lanes that copy):
    the compiler's hazard recognizer does not see that inline assembly reads
    EXEC, so a VALU write of EXEC (v_cmpx) is held to the same five wait
    states."""
    for name, blocks in _kernels(isa[1]).items():
        preds = _predecessors(blocks)

        def walk(k, end, used, ws, depth):
            lab, ins = blocks[k]
            for j in range(end - 1, -1, -1):
                if ws >= 5:
                    return
                p = ins[j]
                assert not (_valu_sgpr_writes(p) & used), f"{name} {lab}: {p} reaches a copy"
                ws += _wait_states(p)
            if ws < 5 and depth < 8:
                for q in preds[k]:
                    walk(q, len(blocks[q][1]), used, ws, depth + 1)

        copies = 0
        for k, (lab, ins) in enumerate(blocks):
            for j, i in enumerate(ins):
                if not i.startswith("global_load_lds"):
                    continue
                copies += 1
                used = {"exec"}
                for tok in i.split(None, 1)[1].split(","):
                    used |= _sgprs(tok.strip().split()[0])
                walk(k, j, used, 0, 0)
        assert copies > 0, name


def test_valu_exec_write_walk_catches_a_planted_cmpx():
    assert _valu_sgpr_writes("v_cmpx_gt_i32_e32 vcc, s94, v3") == {"exec"}
    assert _valu_sgpr_writes("v_cmpx_lt_u32_e64 s[4:5], v1, v2") == {4, 5, "exec"}
    assert _valu_sgpr_writes("v_readlane_b32 exec_lo, v1, 0") == {"exec"}
    assert _valu_sgpr_writes("v_readfirstlane_b32 s7, v1") == {7}
    assert _valu_sgpr_writes("s_and_saveexec_b64 s[2:3], vcc") == set()


def test_hazard_walk_follows_branches():
    """The walk above sees a VALU write to a copy's base in another block."""
    blocks = [("entry", ["v_readfirstlane_b32 s4, v1", "s_cbranch_scc1 .LBB0_2"]),
              (".LBB0_1", ["s_nop 7"]),
              (".LBB0_2", ["s_mov_b32 m0, s6", "global_load_lds_dwordx4 v2, s[4:5] offset:0"])]
    preds = _predecessors(blocks)
    assert sorted(preds[2]) == [0, 1]
    found = []

    def walk(k, end, ws):
        for j in range(end - 1, -1, -1):
            if ws >= 5:
                return
            p = blocks[k][1][j]
            if p.startswith("v_readfirstlane_b32 s4"):
                found.append(k)
            ws += _wait_states(p)
        if ws < 5:
            for q in preds[k]:
                walk(q, len(blocks[q][1]), ws)

    walk(2, 1, 0)
    assert found == [0]   # through the branch, not through the s_nop 7 path


def test_default_kernel_tile_work(isa):
    which, text = isa
    if which != "library":
        pytest.skip("the library's default kernel")
    ks = _kernels(text)
    name = next(n for n in ks if "mla_decode_kernel_pairsILi0E" in n)
    # per 32 keys: 36 QK (32x32x16) + 32 PV MFMAs, 36 K-fragment and 64
    # transposing V reads
    step_mfma, step_k, step_v = 68, 36, 64
    loop = _key_loop_blocks(ks[name])
    mfma = sum(sum("v_mfma" in i for i in ins) for _, ins in loop)
    k_reads = sum(sum(i.startswith("ds_read_b128") for i in ins) for _, ins in loop)
    v_reads = sum(sum(i.startswith("ds_read_b64_tr_b16") for i in ins) for _, ins in loop)
    copies = sum(i.startswith("global_load_lds_dwordx4") for _, ins in ks[name] for i in ins)
    assert mfma % step_mfma == 0 and mfma >= step_mfma
    steps = mfma // step_mfma
    assert k_reads == step_k * steps and v_reads == step_v * steps
    # one tile's 18 copies in the prologue and in the loop
    assert copies == 36


# ---------------------------------------------------------------- cache append

@pytest.fixture(scope="module")
def append_isa(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "append_kernel.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           os.path.join(CSRC, "append_kernel.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return out.read_text()


def _append_kernels(text):
    out, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"^(_ZN3mla\S*mla_kv_append_kernel\S*):", line)
        if m:
            cur = out.setdefault(m.group(1), [])
            continue
        if cur is None:
            continue
        s = line.split(";")[0].strip()
        if s.startswith("s_endpgm"):
            cur = None
        elif s and not s.startswith(".") and not s.endswith(":"):
            cur.append(s)
    return out


def test_append_kernel_machine_code(append_isa):
    ks = _append_kernels(append_isa)
    assert len(ks) == 2, sorted(ks)
    for name, ins in ks.items():
        assert not [i for i in ins if i.startswith("scratch_")], name
        assert not [i for i in ins if re.match(r"s_(store|buffer_store|atomic|buffer_atomic|dcache_wb|scratch_store)", i)], name
    fp8 = next(ins for n, ins in ks.items() if "ILi1E" in n)
    # x / s and max|x| / 448 are correctly rounded fp32 divisions (the code
    # decision must match the oracle's fp32 quotient): 16 values + 1 scale
    assert sum(i.startswith("v_div_fixup_f32") for i in fp8) >= 17


@pytest.mark.parametrize("src,kernel", [("plan_kernel.hip", "mla_plan_kernel"),
                                        ("tree_kernel.hip", "mla_tree_kernel"),
                                        ("prefill_quant_kernel.hip", "mla_prefill_quant_q_kernel"),
                                        ("prefill_quant_kernel.hip", "mla_prefill_quant_k_kernel"),
                                        ("prefill_quant_kernel.hip", "mla_prefill_quant_v_kernel"),
                                        ("prefill_attn_kernel.hip", "mla_prefill_attn_kernel"),
                                        ("check_kernel.hip", "mla_check_kernel"),
                                        ("combine_kernel.hip", "mla_combine_kernel_bf16")])
def test_small_kernels_machine_code(tmp_path, src, kernel):
    # the device planner, the tree-draft merge, the prefill kernels, the
    # debug check and the merge of bf16 partials: no scratch, no scalar
    # stores, LDS within the 160 KB a workgroup may use
    out = tmp_path / "k.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", os.path.join(CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    text = out.read_text()
    body = text[text.index(kernel):]
    ins = [l.split(";")[0].strip() for l in body.splitlines()]
    assert not [i for i in ins if i.startswith("scratch_")]
    assert not [i for i in ins if re.match(r"s_(store|buffer_store|atomic|buffer_atomic|dcache_wb|scratch_store)", i)]
    lds = int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", text).group(1))
    assert lds <= 160 * 1024


def test_prefill_attention_uses_the_int8_and_fp8_matrix_cores(tmp_path):
    out = tmp_path / "k.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", os.path.join(CSRC, "prefill_attn_kernel.hip"),
           "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    ins = [l.split(";")[0].strip() for l in out.read_text().splitlines()]
    # per key block, wave and 16-query tile: 8 key tiles x 3 dim steps of
    # INT8 products and 8 channel tiles of e4m3 products; the block body
    # exists twice (with and without the causal mask)
    i8 = sum(i.startswith("v_mfma_i32_16x16x64_i8") for i in ins)
    f8 = sum(re.match(r"v_mfma(_scale)?_f32_16x16x128_f8f6f4", i) is not None for i in ins)
    assert i8 > 0 and i8 % (2 * 24) == 0 and f8 * 3 == i8
    assert not [i for i in ins if i.startswith("v_mfma") and "bf16" in i]


# ---------------------------------------------------------------- the copy asm and its neighbours
#
# The HBM -> LDS copies are inline assembly, which the compiler's hazard
# recognizer and wait-count pass do not look into.  The checks below cover,
# in the compiled code, what the compiler therefore cannot: M0 (the copy's
# LDS address) is written and read only inside the copy blocks; the register
# a copy block saves M0 in is never read afterwards before it is rewritten
# (the compiler may pick VCC for it); every copy follows its M0 write by at
# least one wait state; and the vmcnt literals of the e4m3 kernels count
# whole rounds of copies, each round issued as one branch-free run.


def _kernels_asm(text):
    """{kernel: [(label, [(instruction, asm block id or None)])]}"""
    out, cur, asm_id, n_asm = {}, None, None, 0
    for line in text.splitlines():
        m = re.match(r"^(_ZN3mla\S*mla_decode_kernel\S*):", line)
        if m:
            cur = [("entry", [])]
            out[m.group(1)] = cur
            continue
        if cur is None:
            continue
        if ";;#ASMSTART" in line:
            n_asm += 1
            asm_id = n_asm
            continue
        if ";;#ASMEND" in line:
            asm_id = None
            continue
        s = line.split(";")[0].strip()
        if s.startswith("s_endpgm"):
            cur[-1][1].append((s, None))
            cur = None
            continue
        lab = re.match(r"^(\.LBB\S+):", line)
        if lab:
            cur.append((lab.group(1), []))
        elif s and not s.startswith("."):
            cur[-1][1].append((s, asm_id))
    return out


def _regs(tok):
    """Scalar registers a token names: 'sN', 'vcc_lo', 'vcc_hi', 'm0', 'exec_*'."""
    tok = tok.strip()
    if tok == "vcc":
        return {"vcc_lo", "vcc_hi"}
    if tok == "exec":
        return {"exec_lo", "exec_hi"}
    if tok in ("vcc_lo", "vcc_hi", "m0", "exec_lo", "exec_hi"):
        return {tok}
    return {f"s{i}" for i in _sgprs(tok)}


_NO_DST = ("s_cmp", "s_bitcmp", "s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier",
           "s_setprio", "s_endpgm", "s_sleep", "s_setreg", "s_sendmsg", "s_trap")


def _reads_writes(ins):
    """(read, written) scalar registers of one instruction (conservative: an
    operand not known to be a destination counts as read)."""
    parts = ins.split(None, 1)
    op = parts[0]
    ops = [o.strip().split()[0] for o in parts[1].split(",")] if len(parts) > 1 else []
    reads, writes = set(), set()
    dst_pos = set()
    if op.startswith("s_") and not op.startswith(_NO_DST):
        dst_pos = {0}
    elif op.startswith(("v_readfirstlane", "v_readlane")) or (op.startswith("v_cmp") and not op.startswith("v_cmpx")):
        dst_pos = {0}
    elif op.startswith(("v_add_co", "v_sub_co", "v_subrev_co", "v_addc_co", "v_subb_co",
                        "v_subbrev_co", "v_div_scale", "v_mad_u64", "v_mad_i64")):
        dst_pos = {0, 1}
    for k, o in enumerate(ops):
        (writes if k in dst_pos else reads).update(_regs(o))
    if op.startswith(("v_addc_co", "v_subb_co", "v_subbrev_co")) and op.endswith("_e32"):
        reads |= {"vcc_lo", "vcc_hi"}
    if op.startswith(("s_cbranch_vccz", "s_cbranch_vccnz", "v_div_fmas")):
        reads |= {"vcc_lo", "vcc_hi"}
    if op.startswith("v_cmp") and op.endswith("_e32"):
        writes |= {"vcc_lo", "vcc_hi"}
    return reads, writes


def _successors(blocks):
    index = {lab: k for k, (lab, _) in enumerate(blocks)}
    succ = {k: [] for k in range(len(blocks))}
    for k, (_, ins) in enumerate(blocks):
        for i, _a in ins:
            m = re.match(r"s_(?:c)?branch\S*\s+(\.LBB\S+)", i)
            if m and m.group(1) in index:
                succ[k].append(index[m.group(1)])
        last = ins[-1][0] if ins else ""
        if k + 1 < len(blocks) and not last.startswith(("s_branch", "s_endpgm")):
            succ[k].append(k + 1)
    return succ


def _first_access_after(blocks, succ, k, j, regs):
    """Walks every control-flow path forward from instruction j of block k;
    returns the instructions that read any of `regs` before a write to all
    of them on that path."""
    bad, seen = [], set()
    stack = [(k, j + 1, frozenset(regs))]
    while stack:
        b, i, live = stack.pop()
        if (b, i, live) in seen:
            continue
        seen.add((b, i, live))
        ins = blocks[b][1]
        while i < len(ins):
            r, w = _reads_writes(ins[i][0])
            if r & live:
                bad.append((blocks[b][0], ins[i][0]))
                break
            live = live - w
            if not live:
                break
            i += 1
        else:
            for s in succ[b]:
                stack.append((s, 0, live))
    return bad


def _copy_blocks(blocks):
    """[(block index, index of the block's last instruction, [instructions])]
    for every inline-asm block that issues a copy."""
    out = {}
    for k, (_, ins) in enumerate(blocks):
        for j, (i, a) in enumerate(ins):
            if a is not None:
                out.setdefault(a, (k, j, []))
                out[a] = (k, j, out[a][2] + [i])
    return [v for v in out.values() if any(i.startswith("global_load_lds") for i in v[2])]


def test_m0_is_written_and_read_only_inside_the_copy_blocks(isa):
    for name, blocks in _kernels_asm(isa[1]).items():
        for lab, ins in blocks:
            for i, a in ins:
                if a is None:
                    assert not re.search(r"\bm0\b", i), f"{name} {lab}: {i}"


def test_copy_block_shape_and_m0_wait_state(isa):
    for name, blocks in _kernels_asm(isa[1]).items():
        cbs = _copy_blocks(blocks)
        assert cbs, name
        for _k, _j, ins in cbs:
            assert len(ins) == 5, ins
            save = re.match(r"s_mov_b32 (\S+), m0$", ins[0])
            setm0 = re.match(r"s_mov_b32 m0, (\S+)$", ins[1])
            assert save and setm0 and ins[2] == "s_nop 0", ins
            assert ins[3].startswith("global_load_lds_dword"), ins
            assert ins[4] == f"s_mov_b32 m0, {save.group(1)}", ins
            # the saved register is neither the new M0 nor an operand of the copy
            tmp = _regs(save.group(1))
            assert not (tmp & _regs(setm0.group(1))), ins
            copy_regs = set()
            for tok in ins[3].split(None, 1)[1].split(","):
                copy_regs |= _regs(tok.strip().split()[0])
            assert not (tmp & copy_regs), ins
            # SALU write of M0 -> LDS-DMA read of M0: one wait state (s_nop 0)
            assert _wait_states(ins[2]) >= 1


def test_register_holding_saved_m0_is_not_read_after_the_copy(isa):
    for name, blocks in _kernels_asm(isa[1]).items():
        succ = _successors(blocks)
        for k, j, ins in _copy_blocks(blocks):
            tmp = _regs(re.match(r"s_mov_b32 (\S+), m0$", ins[0]).group(1))
            bad = _first_access_after(blocks, succ, k, j, tmp)
            assert not bad, f"{name}: {sorted(tmp)} read after a copy block: {bad[:3]}"


def test_saved_register_walk_catches_a_planted_read():
    blocks = [("entry", [("s_mov_b32 vcc_lo, m0", 1), ("s_mov_b32 m0, vcc_lo", 1),
                         ("s_cbranch_scc1 .LBB0_2", None)]),
              (".LBB0_1", [("v_cmp_gt_f32_e32 vcc, v1, v2", None)]),
              (".LBB0_2", [("s_cbranch_vccnz .LBB0_1", None)])]
    succ = _successors(blocks)
    bad = _first_access_after(blocks, succ, 0, 1, {"vcc_lo"})
    assert bad == [(".LBB0_2", "s_cbranch_vccnz .LBB0_1")]
    # a write on the path first makes it safe
    blocks[0][1].insert(2, ("s_mov_b32 vcc_lo, 0", None))
    assert not _first_access_after(blocks, _successors(blocks), 0, 1, {"vcc_lo"})


def test_literal_vmcnt_waits_count_whole_rounds(isa):
    """bf16 kernels wait for every copy (vmcnt(0)); the e4m3 kernels wait with
    vmcnt(10 * rounds issued after the awaited one), which is sound because
    each round is one branch-free run of exactly 10 copies (9 of 16 bytes per
    lane for the keys, 1 of 4 bytes for the scales) and vector-memory
    operations complete in issue order: any other vector-memory operation only
    adds to the count."""
    if isa[0] == "split":
        pytest.skip("its copy runs are checked below")
    for name, blocks in _kernels_asm(isa[1]).items():
        e4m3 = "ILi1E" in name
        literals = {int(m.group(1)) for _, ins in blocks for i, a in ins if a is not None
                    for m in [re.match(r"s_waitcnt vmcnt\((\d+)\)$", i)] if m}
        assert literals <= ({0, 10, 20} if e4m3 else {0}), (name, literals)
        want = COPIES_PER_ROUND[isa[0]]["e4m3" if e4m3 else "bf16"]
        if want is None:
            assert literals <= {0}, (name, literals)
            continue
        for lab, ins in blocks:
            idx = [j for j, (i, _a) in enumerate(ins) if i.startswith("global_load_lds")]
            if not idx:
                continue
            run = [i for i, _a in ins[idx[0]: idx[-1] + 1]]
            x4 = sum(i.startswith("global_load_lds_dwordx4") for i in run)
            x1 = sum(i.startswith("global_load_lds_dword ") for i in run)
            assert (x4, x1) == want, (name, lab, x4, x1)
            # no branch and no other vector-memory operation inside the run
            assert not [i for i in run if i.startswith(("s_cbranch", "s_branch", "global_load_d",
                                                         "global_store", "buffer_", "scratch_",
                                                         "flat_"))], (name, lab)


def test_two_waves_per_simd_register_budget(isa):
    """The candidate runs eight waves per CU, two per SIMD: each wave must fit
    256 registers (VGPRs and AGPRs together) with nothing spilled, and its key
    loop keeps 2 x 18 QK and 32 PV steps of v_mfma_f32_16x16x32_bf16 per 32
    keys (36 K-fragment and 64 transposing V reads; for e4m3 two more 16-byte
    reads, the keys' scales).  The e4m3 kernel widens each pair once per CU:
    a wave converts at most five 1 KB blocks per pair (one 8-byte read, four
    conversions of two values, one 16-byte write each)."""
    which, text = isa
    if which != "w8":
        pytest.skip("the two-waves-per-SIMD candidate")
    vs = [int(x) for x in re.findall(r"\.vgpr_count:\s+(\d+)", text)]
    as_ = [int(x) for x in re.findall(r"\.agpr_count:\s+(\d+)", text)]
    assert len(vs) == len(as_) == EXPECTED_KERNELS["w8"]
    assert all(v + a <= 256 for v, a in zip(vs, as_)), (vs, as_)
    assert set(re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)) == {"0"}
    assert set(re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)) == {"0"}
    assert "amdhsa_next_free_vgpr" in text
    for name, blocks in _kernels(text).items():
        e4m3 = "ILi1E" in name
        loop = _key_loop_blocks(blocks)

        def count(prefix, where=loop):
            return sum(sum(i.startswith(prefix) for i in ins) for _, ins in where)
        mfma = count("v_mfma_f32_16x16x32_bf16")
        assert mfma % 68 == 0 and mfma >= 68, (name, mfma)
        steps = mfma // 68
        want = (64 * steps, (38 if e4m3 else 36) * steps)
        assert (count("ds_read_b64_tr_b16"), count("ds_read_b128")) == want, (name, steps)
        widen = (count("ds_read_b64 ", blocks), count("ds_write_b128", blocks),
                 count("v_cvt_pk_f32_fp8", blocks))
        if e4m3:
            assert widen[0] % 5 == 0 and widen[0] > 0 and widen == (widen[0], widen[0],
                                                                    4 * widen[0]), widen
        else:
            assert widen == (0, 0, 0), widen


def test_split_copy_runs_and_waits(isa):
    """The split candidate waits for a round with one vmcnt literal while the
    next round is in flight (else vmcnt(0)): 4 for bf16, whose waves issue
    four or five copies per round, 2 for e4m3, whose waves issue two or three
    (and wave 7 the scales).  That is sound when every wave issues at least
    that many copies per round after the awaited ones: each round is one
    branch-free run of four (bf16) or two (e4m3) copies, followed by the
    copies only some waves issue, each in a block of its own, and no other
    vector-memory operation."""
    which, text = isa
    if which != "split":
        pytest.skip("the split candidate")
    for name, blocks in _kernels_asm(text).items():
        e4m3 = "ILi1E" in name
        literals = {int(m.group(1)) for _, ins in blocks for i, a in ins if a is not None
                    for m in [re.match(r"s_waitcnt vmcnt\((\d+)\)$", i)] if m}
        assert literals == ({0, 2} if e4m3 else {0, 4}), (name, literals)
        shapes = []
        for lab, ins in blocks:
            idx = [j for j, (i, _a) in enumerate(ins) if i.startswith("global_load_lds")]
            if not idx:
                continue
            run = [i for i, _a in ins[idx[0]: idx[-1] + 1]]
            assert not [i for i in run if i.startswith(("s_branch", "global_load_d",
                                                         "global_store", "buffer_", "scratch_",
                                                         "flat_"))], lab
            # C: a 16-byte copy, S: a 4-byte copy (the e4m3 scales), B: a
            # conditional branch (around the copies only some waves issue)
            shapes.append("".join(
                ("C" if i.startswith("global_load_lds_dwordx4") else "S")
                if i.startswith("global_load_lds") else "B"
                for i in run if i.startswith(("global_load_lds", "s_cbranch"))))
        # bf16: rounds 0 and 1 in the prologue and round j + 2 in the loop,
        # each four copies, then the branch around the fifth; e4m3: rounds 0,
        # 1, 2 in the prologue and p + 3 in the loop, each two copies, the
        # branch around the third, and the scales' copy in a block of its own
        want = ["CCBC"] * 4 + ["S"] * 4 if e4m3 else ["CCCCBC"] * 3
        assert sorted(shapes) == sorted(want), (name, shapes)


def test_split_register_budget_and_loop_work(isa):
    """The split candidate runs eight waves per CU, two per SIMD: each wave
    fits 256 registers with nothing spilled, and per 32 keys issues 18 QK and
    16 PV steps of v_mfma_f32_32x32x16_bf16 (half the dimensions, half the
    columns), 18 K-fragment reads and 32 transposing V reads, and exchanges
    its partial scores (four 16-byte writes, four reads), waiting for its
    partner's round counter with s_sleep between polls.  For e4m3 it also
    reads its keys' scales (four 16-byte reads) and widens rounds once per CU:
    at most five 1 KB blocks per wave and round (one 8-byte read, four
    conversions of two values, one 16-byte write each), in the prologue and
    in the loop."""
    which, text = isa
    if which != "split":
        pytest.skip("the split candidate")
    vs = [int(x) for x in re.findall(r"\.vgpr_count:\s+(\d+)", text)]
    as_ = [int(x) for x in re.findall(r"\.agpr_count:\s+(\d+)", text)]
    assert len(vs) == len(as_) == 2 and all(v + a <= 256 for v, a in zip(vs, as_)), (vs, as_)
    assert set(re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)) == {"0"}
    assert set(re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)) == {"0"}
    lds = sorted(int(x) for x in re.findall(r"\.group_segment_fixed_size:\s+(\d+)", text))
    exch = 8 * 4096 + 32   # exchange slots and round counters
    assert lds == sorted([3 * 36864 + exch,                            # bf16 ring
                          2 * 36864 + 3 * 18432 + 3 * 256 + 256 + exch]), lds   # e4m3
    for name, blocks in _kernels(text).items():
        e4m3 = "ILi1E" in name
        loop = [(lab, ins) for lab, ins in blocks if any("v_mfma" in i for i in ins)]

        def count(prefix, where=loop):
            return sum(sum(i.startswith(prefix) for i in ins) for _, ins in where)
        # (the kernel's only MFMAs and transposing reads are these)
        assert count("v_mfma_f32_32x32x16_bf16") == count("v_mfma", blocks) == 34, name
        assert count("ds_read_b64_tr_b16") == count("ds_read_b64_tr_b16", blocks) == 32, name
        assert count("ds_read_b128", blocks) == 18 + 4 + (4 if e4m3 else 0), name
        assert count("s_sleep", blocks) >= 1, name
        widen = (count("ds_read_b64 ", blocks), count("ds_write_b128", blocks) - 4,
                 count("v_cvt_pk_f32_fp8", blocks))
        if e4m3:
            assert widen == (10, 10, 40), widen
        else:
            assert widen == (0, 0, 0), widen


def test_split_exchange_order(isa):
    """The exchange in program order: the four 16-byte writes of the partial
    scores, the wait for them (lgkmcnt(0), the kernel's own), the store of
    the round counter, the poll of the partner's counter (a 4-byte read, its
    value made scalar, s_sleep between polls), and only after that the four
    16-byte reads of the partner's slot.  The emulator runs the kernel's
    order; this checks that the compiler kept it."""
    which, text = isa
    if which != "split":
        pytest.skip("the split candidate")
    for name, blocks in _kernels_asm(text).items():
        flat = [(i, a) for _lab, ins in blocks for i, a in ins]
        # the publish: the kernel's lgkmcnt(0) followed by a 4-byte LDS store
        pub = [k for k in range(1, len(flat))
               if flat[k][0].startswith("ds_write_b32") and any(
                   flat[j][1] is not None and flat[j][0] == "s_waitcnt lgkmcnt(0)"
                   for j in range(max(0, k - 4), k))]
        assert len(pub) == 1, (name, pub)
        k = pub[0]
        before = [i for i, _a in flat[:k]]
        assert [i for i in before if i.startswith("ds_write_b128")][-4:] and all(
            i.startswith("ds_write_b128") or not i.startswith("ds_")
            for i in before[len(before) - 12:]), name
        after = [i for i, _a in flat[k + 1:]]
        first_read = next(n for n, i in enumerate(after) if i.startswith("ds_read_b128"))
        poll = after[:first_read]
        assert any(i.startswith("ds_read_b32") for i in poll), name
        assert any(i.startswith("v_readfirstlane_b32") for i in poll), name
        assert any(i.startswith("s_sleep") for i in poll), name
        assert sum(i.startswith("ds_read_b128") for i in after[first_read:first_read + 24]) >= 4


# The library's e4m3 16-key kernels load Q before the key loop without
# forcing it resident there, so the compiler's wait-count pass, which does
# not see the copies, keeps those loads pending into the loop and waits for
# them inside it (vmcnt 35 down to 9 across the QK step): at run time these
# literals also count the copies of the rounds issued ahead, so the step
# waits for most of them.  Fixing it changes their validated machine code.
# The four-phase e4m3 kernel (opt-in MLA_PHASES=4, never chosen by the
# planner) reloads spilled registers inside its key loop, and the compiler
# waits for those reloads there; its Q-resident rebuild keeps that.
KNOWN_LOOP_VMCNT = {"mla_decode_kernelILi1E", "mla_decode_kernel_qresILi1ELi4E"}


def test_every_barrier_follows_the_waves_lds_operations(isa):
    """Each s_barrier of every decode kernel comes after an s_waitcnt that
    includes lgkmcnt(0), with no LDS instruction between the two, on the one
    path into it (a barrier is never a branch target here): a wave's LDS
    stores and reads are complete before other waves pass the barrier.  The
    CPU emulator's race detector takes LDS operations as complete in program
    order at barriers and publishes, which this makes true of the machine
    code (the publish's own wait is checked with the exchange above)."""
    _which, text = isa
    for name, blocks in _kernels_asm(text).items():
        n = 0
        for _lab, ins in blocks:
            for k, (i, _a) in enumerate(ins):
                if not i.startswith("s_barrier"):
                    continue
                n += 1
                # the wait is in the same block (it shares the barrier's asm)
                prior = [x for x, _ in ins[:k]]
                w = next((j for j in range(len(prior) - 1, -1, -1)
                          if prior[j].startswith("s_waitcnt") and "lgkmcnt(0)" in prior[j]), None)
                assert w is not None, (name, _lab, k)
                between = prior[w + 1:]
                assert not any(x.startswith("ds_") for x in between), (name, _lab, between)
        assert n >= 2, (name, n)


def test_no_compiler_vmcnt_wait_in_key_loop(isa):
    """In every block that issues MFMAs, a vmcnt wait comes from the kernel's
    own inline assembly (which counts the copies), never from the compiler."""
    for name, blocks in _kernels_asm(isa[1]).items():
        if any(k in name for k in KNOWN_LOOP_VMCNT):
            continue
        for lab, ins in blocks:
            if not any(i.startswith("v_mfma") for i, _a in ins):
                continue
            bad = [i for i, a in ins if a is None and re.match(r"s_waitcnt .*vmcnt", i)]
            assert not bad, f"{name} {lab}: {bad[:4]}"


def test_known_loop_vmcnt_waits_are_still_there(isa):
    # the exception above is real (and goes once those kernels change)
    if isa[0] != "library":
        pytest.skip("library kernels only")
    found = set()
    for name, blocks in _kernels_asm(isa[1]).items():
        for lab, ins in blocks:
            if any(i.startswith("v_mfma") for i, _a in ins) and any(
                    a is None and re.match(r"s_waitcnt .*vmcnt", i) for i, a in ins):
                found.add(name)
    assert found and all(any(k in n for k in KNOWN_LOOP_VMCNT) for n in found), sorted(found)


@pytest.mark.parametrize("src", ["e4m3_convert_check.hip", "lds_read_probe.hip"])
def test_gpu_check_kernels_machine_code(tmp_path, src):
    # the GPU check and measurement kernels of tests/gpu_checks: no scratch,
    # no scalar stores, LDS within the 160 KB a workgroup may use
    out = tmp_path / "k.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           os.path.join(ROOT, "tests", "gpu_checks", src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    text = out.read_text()
    ins = [l.split(";")[0].strip() for l in text.splitlines()]
    assert not [i for i in ins if i.startswith("scratch_")]
    assert not [i for i in ins if re.match(r"s_(store|buffer_store|atomic|buffer_atomic|dcache_wb|scratch_store)", i)]
    for lds in re.findall(r"\.group_segment_fixed_size:\s+(\d+)", text):
        assert int(lds) <= 160 * 1024
