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
checks cover it and every instantiation of the 16-key kernel.
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
}


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
    assert len(ks) == 6, sorted(ks)


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


def test_valu_written_sgpr_not_read_by_lds_copy_within_five_wait_states(isa):
    """Walks back from every copy over all control-flow paths (through
    branches and fall-throughs), not only inside the copy's own block."""
    for name, blocks in _kernels(isa[1]).items():
        preds = _predecessors(blocks)

        def walk(k, end, used, ws, depth):
            lab, ins = blocks[k]
            for j in range(end - 1, -1, -1):
                if ws >= 5:
                    return
                p = ins[j]
                if p.split()[0].startswith("v_") and " " in p:
                    dst = p.split(None, 1)[1].split(",")[0].strip()
                    assert not (_sgprs(dst) & used), f"{name} {lab}: {p} reaches a copy"
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
                used = set()
                for tok in i.split(None, 1)[1].split(","):
                    used |= _sgprs(tok.strip().split()[0])
                walk(k, j, used, 0, 0)
        assert copies > 0, name


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
                                        ("prefill_attn_kernel.hip", "mla_prefill_attn_kernel")])
def test_small_kernels_machine_code(tmp_path, src, kernel):
    # the device planner, the tree-draft merge and the prefill kernels: no
    # scratch, no scalar stores, LDS within the 160 KB a workgroup may use
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
