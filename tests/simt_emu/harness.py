"""Run a decode or cache-append case through the emulated kernels
(tests/simt_emu/_build/run_case)."""
from __future__ import annotations

import os
import subprocess
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "_build", "run_case")
MAGIC = 0x4D4C4145
TREE_MAGIC = 0x4D4C4154
APPEND_MAGIC = 0x4D4C4141
PREFILL_MAGIC = 0x4D4C5046


def ensure_built() -> str:
    """The emulator binary, built if missing or older than its sources.
    EMU_BINARY names another build to run instead (the UndefinedBehavior-
    Sanitizer one, say), used as it is."""
    other = os.environ.get("EMU_BINARY")
    if other:
        if not os.path.exists(other):
            raise RuntimeError(f"EMU_BINARY {other} does not exist")
        return other
    from tests.simt_emu import build as _b  # noqa: WPS433
    if not os.path.exists(BIN) or _stale():
        _b.build()
    return BIN


def _stale(binary: str = BIN) -> bool:
    from tests.simt_emu import build as _b
    t = os.path.getmtime(binary)
    srcs = [os.path.join(_b.CSRC, f) for f in _b.KERNEL_FILES]
    srcs += [os.path.join(HERE, f) for f in ("gfx950_asm.h", "lds_trace.h", "emu_runtime.cpp",
                                              "run_case.cpp",
                                              os.path.join("hip", "hip_runtime.h"), "build.py")]
    return any(os.path.getmtime(s) > t for s in srcs)


def run(case, num_workgroups: int, phases: int | None = None, timeout: float = 600.0,
        env_extra: dict | None = None, binary: str | None = None, fixed: bool = False,
        tree_mask=None, want_plan: bool = False, plan_kv_lens=None):
    """Returns (out bf16 bits [B, qmax, H, 512] uint16, lse [B, qmax, H] f32, meta).
    ``fixed`` plans with mla_decode_plan_fixed (launch bounds, padded plan);
    ``tree_mask`` [B, qmax] runs the tree-draft path (prefix decode + merge);
    ``want_plan`` adds the plan image the kernels ran (int32 words) to meta;
    ``plan_kv_lens`` plans for these lengths instead of the case's (a stale
    plan: the kernels still get the case's lengths)."""
    B, H, qmax = case.batch, case.num_heads, case.max_q_len
    kv_dtype = {"bf16": 0, "fp8_e4m3": 1}[case.kv_dtype]
    magic = MAGIC if tree_mask is None else TREE_MAGIC
    hdr = np.array([magic, B, H, qmax, case.page_size, case.num_pages, case.max_pages, kv_dtype,
                    int(case.causal), num_workgroups, 1, int(fixed)], dtype=np.int32)
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fin, "wb") as f:
            f.write(hdr.tobytes())
            f.write(np.float32(case.sm_scale).tobytes())
            f.write(np.ascontiguousarray(case.q).tobytes())
            f.write(np.ascontiguousarray(case.kv).tobytes())
            if kv_dtype == 1:
                f.write(np.ascontiguousarray(case.kv_scale, dtype=np.float32).tobytes())
            f.write(np.ascontiguousarray(case.block_table, dtype=np.int32).tobytes())
            f.write(np.ascontiguousarray(case.kv_lens, dtype=np.int32).tobytes())
            f.write(np.ascontiguousarray(case.q_lens, dtype=np.int32).tobytes())
            if tree_mask is not None:
                f.write(np.ascontiguousarray(tree_mask, dtype=np.uint32).tobytes())
        env = dict(os.environ)
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
        if phases is not None:
            env["MLA_PHASES"] = str(phases)
        if env_extra:
            env.update(env_extra)
        if plan_kv_lens is not None:
            env["EMU_PLAN_KV_LENS"] = ",".join(str(int(x)) for x in plan_kv_lens)
        fplan = os.path.join(d, "plan.bin")
        if want_plan:
            env["EMU_PLAN_OUT"] = fplan
        res = subprocess.run([binary or ensure_built(), fin, fout], capture_output=True, text=True,
                             timeout=timeout, env=env)
        if os.environ.get("EMU_SHOW"):
            print(res.stdout[-20000:], res.stderr[-4000:])
        if res.returncode != 0:
            raise RuntimeError(f"emulated run failed (rc {res.returncode}):\n{res.stderr[-6000:]}")
        raw = np.fromfile(fout, dtype=np.uint8)
        plan = np.fromfile(fplan, dtype=np.int32) if want_plan else None
    meta = raw[:16].view(np.int32).copy()
    n_o = B * qmax * H * 512 * 2
    out = raw[16:16 + n_o].view(np.uint16).reshape(B, qmax, H, 512)
    lse = raw[16 + n_o:].view(np.float32).reshape(B, qmax, H)
    info = {"num_items": int(meta[0]), "num_partials": int(meta[1]),
            "num_combine": int(meta[2]), "phases": int(meta[3])}
    if want_plan:
        info["plan"] = plan
    return out, lse, info


def run_many(jobs, workers: int = 6):
    """run(case, num_workgroups, phases, **kw) for each (case, num_workgroups,
    phases, kw) of `jobs`, several emulator processes at a time; the results
    in order (each process is independent: its own files and buffers)."""
    from concurrent.futures import ThreadPoolExecutor
    ensure_built()
    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        futs = [ex.submit(run, c, n, p, **kw) for c, n, p, kw in jobs]
        return [f.result() for f in futs]


def run_append(kv, kv_scale, block_table, kv_lens, new_lens, new_rows_bits, page_size: int,
               kv_dtype: str, with_counter: bool = True, timeout: float = 600.0):
    """mla_kv_append on the emulator.  Returns (kv', kv_scale' or None, skipped
    or None); the inputs are not modified."""
    B, max_new = new_rows_bits.shape[0], new_rows_bits.shape[1]
    kvd = {"bf16": 0, "fp8_e4m3": 1}[kv_dtype]
    hdr = np.array([APPEND_MAGIC, B, max_new, page_size, kv.shape[0], block_table.shape[1], kvd,
                    int(new_lens is not None), int(with_counter), 0, 0, 0], dtype=np.int32)
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fin, "wb") as f:
            f.write(hdr.tobytes())
            f.write(np.ascontiguousarray(new_rows_bits, dtype=np.uint16).tobytes())
            f.write(np.ascontiguousarray(kv).tobytes())
            if kvd == 1:
                f.write(np.ascontiguousarray(kv_scale, dtype=np.float32).tobytes())
            f.write(np.ascontiguousarray(block_table, dtype=np.int32).tobytes())
            f.write(np.ascontiguousarray(kv_lens, dtype=np.int32).tobytes())
            if new_lens is not None:
                f.write(np.ascontiguousarray(new_lens, dtype=np.int32).tobytes())
        env = dict(os.environ)
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
        res = subprocess.run([ensure_built(), fin, fout], capture_output=True, text=True,
                             timeout=timeout, env=env)
        if res.returncode != 0:
            raise RuntimeError(f"emulated append failed (rc {res.returncode}):\n{res.stderr[-6000:]}")
        raw = np.fromfile(fout, dtype=np.uint8)
    skipped = int(raw[:4].view(np.int32)[0])
    n_kv = kv.nbytes
    kv_out = raw[4:4 + n_kv].view(kv.dtype).reshape(kv.shape).copy()
    sc_out = None
    if kvd == 1:
        sc_out = raw[4 + n_kv:].view(np.float32).reshape(kv_scale.shape).copy()
    return kv_out, sc_out, (skipped if with_counter else None)


PLAN_MAGIC = 0x4D4C4150
CHECK_MAGIC = 0x4D4C4143


def run_check(case, num_workgroups: int, plan_kv_lens=None, plan_q_lens=None, kv_lens=None,
              q_lens=None, block_table=None, pokes=(), phases: int | None = None,
              timeout: float = 600.0, want_plan: bool = False):
    """mla_decode_plan from (plan_kv_lens, plan_q_lens) (default: the case's),
    then mla_decode_check against the device lengths and block table (default:
    the case's), with (word, value) pokes applied to the plan image.  Returns
    (call status, check code, index), and the plan image before the pokes
    (int32 words) as a fourth element with ``want_plan``."""
    B = case.batch
    has_ql = case.q_lens is not None
    kvd = {"bf16": 0, "fp8_e4m3": 1}[case.kv_dtype]
    hdr = np.array([CHECK_MAGIC, B, case.num_heads, case.max_q_len, case.page_size,
                    case.num_pages, case.max_pages, kvd, int(case.causal), num_workgroups,
                    int(has_ql), len(pokes)], dtype=np.int32)
    pick = lambda x, d: np.ascontiguousarray(d if x is None else x, dtype=np.int32)  # noqa: E731
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fin, "wb") as f:
            f.write(hdr.tobytes())
            f.write(pick(plan_kv_lens, case.kv_lens).tobytes())
            if has_ql:
                f.write(pick(plan_q_lens, case.q_lens).tobytes())
            f.write(pick(kv_lens, case.kv_lens).tobytes())
            if has_ql:
                f.write(pick(q_lens, case.q_lens).tobytes())
            f.write(pick(block_table, case.block_table).tobytes())
            f.write(np.asarray(pokes, dtype=np.int32).reshape(-1).tobytes())
        env = dict(os.environ)
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
        if phases is not None:
            env["MLA_PHASES"] = str(phases)
        fplan = os.path.join(d, "plan.bin")
        if want_plan:
            env["EMU_PLAN_OUT"] = fplan
        res = subprocess.run([ensure_built(), fin, fout], capture_output=True, text=True,
                             timeout=timeout, env=env)
        if res.returncode != 0:
            raise RuntimeError(f"emulated check failed (rc {res.returncode}):\n{res.stderr[-6000:]}")
        raw = np.fromfile(fout, dtype=np.int32)
        res3 = (int(raw[0]), int(raw[1]), int(raw[2]))
        if want_plan:
            return res3 + (np.fromfile(fplan, dtype=np.int32),)
    return res3


def run_plan_device(batch, num_heads, max_q_len, page_size, num_pages, max_pages, causal,
                    kv_lens, q_lens, num_workgroups, env_extra=None, timeout: float = 600.0):
    """mla_decode_plan_device on the emulator.  Returns (call status, plan
    status, image words of the plan-size bound)."""
    hdr = np.array([PLAN_MAGIC, batch, num_heads, max_q_len, page_size, num_pages, max_pages,
                    int(causal), num_workgroups, int(q_lens is not None), 0, 0], dtype=np.int32)
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fin, "wb") as f:
            f.write(hdr.tobytes())
            f.write(np.ascontiguousarray(kv_lens, dtype=np.int32).tobytes())
            if q_lens is not None:
                f.write(np.ascontiguousarray(q_lens, dtype=np.int32).tobytes())
        env = dict(os.environ)
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
        if env_extra:
            env.update(env_extra)
        res = subprocess.run([ensure_built(), fin, fout], capture_output=True, text=True,
                             timeout=timeout, env=env)
        if res.returncode != 0:
            raise RuntimeError(f"emulated planner failed (rc {res.returncode}):\n{res.stderr[-6000:]}")
        raw = np.fromfile(fout, dtype=np.int32)
    return int(raw[0]), int(raw[1]), raw[3:3 + int(raw[2])].copy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_prefill(case, num_blocks: int, timeout: float = 900.0, env_extra: dict | None = None,
                binary: str | None = None):
    """A packed prefill case (``workloads.prefill.PrefillCase``) through
    mla_prefill_quantize + mla_prefill_attn.  Returns a dict of the outputs:
    qc, qs, kc [T, H, ...], ks [blocks, H], vc [blocks, H, 128, 128], vs [blocks, H, 128],
    o (bf16 bits [T, H, 128]), lse [T, H].  ``env_extra`` and ``binary`` as
    for run."""
    S, T, H = case.num_seqs, case.num_tokens, case.num_heads
    hdr = np.array([PREFILL_MAGIC, S, T, H, num_blocks, 0, 0, 0, 0, 0, 0, 0], dtype=np.int32)
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fin, "wb") as f:
            f.write(hdr.tobytes())
            f.write(np.float32(case.sm_scale).tobytes())
            f.write(np.ascontiguousarray(case.cu_seqlens, dtype=np.int32).tobytes())
            for x in (case.q, case.k, case.v):
                f.write(np.ascontiguousarray(x).tobytes())
        env = dict(os.environ)
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
        env.update(env_extra or {})
        res = subprocess.run([binary or ensure_built(), fin, fout], capture_output=True, text=True,
                             timeout=timeout, env=env)
        if res.returncode != 0:
            raise RuntimeError(f"emulated run failed (rc {res.returncode}):\n{res.stderr[-6000:]}")
        raw = np.fromfile(fout, dtype=np.uint8)
    out, off = {}, 0

    def take(name, n, dtype, shape):
        nonlocal off
        out[name] = raw[off:off + n].view(dtype).reshape(shape)
        off += n

    take("qc", T * H * 192, np.int8, (T, H, 192))
    take("qs", T * H * 4, np.float32, (T, H))
    take("kc", T * H * 192, np.int8, (T, H, 192))
    take("ks", num_blocks * H * 4, np.float32, (num_blocks, H))
    take("vc", num_blocks * H * 128 * 128, np.uint8, (num_blocks, H, 128, 128))
    take("vs", num_blocks * H * 128 * 4, np.float32, (num_blocks, H, 128))
    take("o", T * H * 128 * 2, np.uint16, (T, H, 128))
    take("lse", T * H * 4, np.float32, (T, H))
    assert off == raw.size
    return out
