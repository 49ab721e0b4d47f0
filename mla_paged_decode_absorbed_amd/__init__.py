"""Weight-absorbed MLA decode over a paged latent KV cache on MI355X (gfx950).

Thin ctypes binding over ``libmla_decode.so`` (C ABI in ``include/mla_decode.h``).
It only marshals arguments: every step of the decode runs in the library's HIP
kernels, and torch supplies device memory and the current stream.  There is no
CPU fallback: calls fail loudly when the library is missing.

Typical use::

    import mla_paged_decode_absorbed_amd as mla
    shape = mla.Shape.make(batch=B, num_heads=128, max_q_len=1, page_size=64,
                           num_pages=kv.shape[0], max_pages_per_seq=bt.shape[1])
    plan = mla.plan(shape, kv_lens_host)                 # host planner + upload
    out, lse = mla.decode(shape, plan, q, kv, bt, kv_lens_dev, q_lens_dev, scale)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "Shape", "PlanInfo", "Plan", "MLAError", "MLAInputError", "load_library", "plan",
    "plan_device", "decode_fwd", "combine", "check", "tree_attend", "decode_tree",
    "decode", "kv_append", "status_string", "KV_BF16", "KV_FP8_E4M3", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_decode.so")
KV_BF16 = 0
KV_FP8_E4M3 = 1
ROWS_PER_BLOCK = 128
D_LATENT = 512
D_ROPE = 64

EXPORTED_SYMBOLS = (
    "mla_abi_version", "mla_status_string", "mla_plan_bytes_bound",
    "mla_workspace_bytes_bound", "mla_device_num_cus", "mla_decode_plan",
    "mla_decode_fwd", "mla_combine", "mla_kv_append", "mla_decode_plan_fixed",
    "mla_decode_plan_device", "mla_tree_attend", "mla_prefill_num_blocks",
    "mla_prefill_quantize", "mla_prefill_attn", "mla_decode_check",
)
# codes of mla_decode_check (mla_check_code)
CHECK_NAMES = {0: "ok", 1: "plan image", 2: "device lengths", 3: "block-table entry",
               4: "work item", 5: "combine entry"}
PREFILL_D_QK = 192
PREFILL_D_V = 128
PREFILL_BLOCK = 128


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class MLAInputError(ValueError):
    """A device-resident input failed mla_decode_check (MLA_DEBUG_CHECK=1)."""

    def __init__(self, code: int, index: int):
        self.code, self.index = code, index
        super().__init__(f"mla_decode_check: bad {CHECK_NAMES.get(code, code)} (index {index})")


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("max_q_len", ctypes.c_int32),
        ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
    ]

    @classmethod
    def make(cls, *, batch, num_heads, max_q_len, page_size, num_pages, max_pages_per_seq,
             kv_dtype=KV_BF16, causal=True, d_latent=D_LATENT, d_rope=D_ROPE) -> "Shape":
        return cls(batch, num_heads, max_q_len, d_latent, d_rope, page_size, num_pages,
                   max_pages_per_seq, kv_dtype, int(bool(causal)))


class PrefillShape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
    ]

    @classmethod
    def make(cls, seqlens, num_heads: int) -> "PrefillShape":
        """From host sequence lengths (the block count comes from the library)."""
        lens = np.ascontiguousarray(seqlens, dtype=np.int32)
        nb = load_library().mla_prefill_num_blocks(
            lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(lens.size))
        if nb < 0:
            raise ValueError("bad sequence lengths")
        return cls(int(lens.size), int(lens.sum()), int(num_heads), PREFILL_D_QK, PREFILL_D_V,
                   int(nb))


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("num_workgroups", ctypes.c_int32), ("num_items", ctypes.c_int32),
        ("num_partials", ctypes.c_int32), ("num_combine", ctypes.c_int32),
        ("tile_tokens", ctypes.c_int32), ("rows_per_block", ctypes.c_int32),
        ("phases", ctypes.c_int32),
        ("plan_bytes", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load (once) and type the C ABI.  Raises if the library is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m mla_paged_decode_absorbed_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, U64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float
    sp, ip = ctypes.POINTER(Shape), ctypes.POINTER(PlanInfo)
    lib.mla_abi_version.restype = I32
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [I32]
    lib.mla_plan_bytes_bound.restype = U64
    lib.mla_plan_bytes_bound.argtypes = [sp, I32]
    lib.mla_workspace_bytes_bound.restype = U64
    lib.mla_workspace_bytes_bound.argtypes = [sp, I32]
    lib.mla_device_num_cus.restype = I32
    lib.mla_device_num_cus.argtypes = [I32]
    lib.mla_decode_plan.restype = I32
    lib.mla_decode_plan.argtypes = [sp, P, P, I32, P, U64, ip]
    lib.mla_decode_plan_fixed.restype = I32
    lib.mla_decode_plan_fixed.argtypes = [sp, P, P, I32, P, U64, ip]
    lib.mla_decode_plan_device.restype = I32
    lib.mla_decode_plan_device.argtypes = [sp, I32, P, P, P, U64, P, ip, P]
    lib.mla_tree_attend.restype = I32
    lib.mla_tree_attend.argtypes = [sp, P, P, P, P, P, P, P, F32, P, P, P]
    lib.mla_decode_fwd.restype = I32
    lib.mla_decode_fwd.argtypes = [sp, ip, P, P, P, P, P, P, P, F32, P, P, P, U64, P]
    lib.mla_combine.restype = I32
    lib.mla_combine.argtypes = [sp, ip, P, P, U64, P, P, P, P]
    lib.mla_decode_check.restype = I32
    lib.mla_decode_check.argtypes = [sp, ip, P, P, P, P, P, P]
    lib.mla_kv_append.restype = I32
    lib.mla_kv_append.argtypes = [sp, I32, P, P, P, P, P, P, P, P]
    pp = ctypes.POINTER(PrefillShape)
    lib.mla_prefill_num_blocks.restype = I32
    lib.mla_prefill_num_blocks.argtypes = [ctypes.POINTER(ctypes.c_int32), I32]
    lib.mla_prefill_quantize.restype = I32
    lib.mla_prefill_quantize.argtypes = [pp, P, P, P, P, P, P, P, P, P, P, P]
    lib.mla_prefill_attn.restype = I32
    lib.mla_prefill_attn.argtypes = [pp, P, P, P, P, P, P, P, F32, P, P, P]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mla_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise MLAError(status, where)


def _sized(dev, named):
    """Every (name, tensor, bytes, element size) given a tensor must be
    contiguous, on `dev` and exactly that many bytes of that element size: the
    C ABI takes bare device pointers, so a tensor of another size would make
    the kernels read or write outside it."""
    for name, t, nbytes, esize in named:
        if t is None:
            continue
        if not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be contiguous and on {dev}")
        if t.element_size() != esize or t.numel() * t.element_size() != nbytes:
            raise ValueError(f"{name} must hold {nbytes // esize} elements of {esize} bytes, "
                             f"not {t.numel()} of {t.element_size()}")


def _decode_sizes(shape, q, kv_cache, kv_scale, block_table, kv_lens, q_lens, out=None, lse=None):
    B, qmax, H = shape.batch, shape.max_q_len, shape.num_heads
    NP, P = shape.num_pages, shape.page_size
    fp8 = shape.kv_dtype == KV_FP8_E4M3
    if fp8 and kv_scale is None:
        raise ValueError("an e4m3 cache needs kv_scale")
    rows = B * qmax * H
    _sized(q.device, [
        ("q", q, rows * (D_LATENT + D_ROPE) * 2, 2),
        ("kv_cache", kv_cache, NP * P * (D_LATENT + D_ROPE) * (1 if fp8 else 2), 1 if fp8 else 2),
        ("kv_scale", kv_scale if fp8 else None, NP * P * 4, 4),
        ("block_table", block_table, B * shape.max_pages_per_seq * 4, 4),
        ("kv_lens", kv_lens, B * 4, 4), ("q_lens", q_lens, B * 4, 4),
        ("out", out, rows * D_LATENT * 2, 2), ("lse", lse, rows * 4, 4)])


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


@dataclass
class Plan:
    info: PlanInfo
    host: np.ndarray          # int32 plan image
    device: object            # torch int32 tensor on the GPU (or None before upload)

    @property
    def workspace_bytes(self) -> int:
        return int(self.info.workspace_bytes)

    # Readers of the plan image (layout documented in csrc/plan_layout.h).
    def wg_start(self) -> np.ndarray:
        off, G = int(self.host[8]), int(self.host[2])
        return self.host[off:off + G + 1]

    def items(self) -> np.ndarray:
        """[num_items, 6]: b, row0, k0, k1, slot (-1 = direct output), row offset
        of the item inside its 128-row unit (and partial slot)."""
        off, n = int(self.host[9]), int(self.host[3])
        return self.host[off:off + 8 * n].reshape(n, 8)[:, :6]

    @property
    def phases(self) -> int:
        return int(self.info.phases)

    def combine_entries(self) -> np.ndarray:
        """[num_combine, 4]: b, row0, first_slot, n_splits."""
        off, n = int(self.host[10]), int(self.host[4])
        return self.host[off:off + 4 * n].reshape(n, 4)


def plan(shape: Shape, kv_lens_host, q_lens_host=None, num_workgroups: Optional[int] = None,
         device=None, upload: bool = True, fixed: bool = False) -> Plan:
    """Run the host planner and (optionally) copy the plan image to the GPU.

    ``fixed=True`` uses ``mla_decode_plan_fixed``: the info then holds launch
    bounds shared by every lengths of the shape (for graph capture), and the
    image is padded to ``info.plan_bytes``."""
    lib = load_library()
    kv = np.ascontiguousarray(np.asarray(kv_lens_host, dtype=np.int32))
    ql = None if q_lens_host is None else np.ascontiguousarray(np.asarray(q_lens_host, np.int32))
    if num_workgroups is None:
        dev = 0
        if device is not None:
            import torch
            dev = torch.device(device).index or 0
        num_workgroups = lib.mla_device_num_cus(dev)
        if num_workgroups <= 0:
            raise MLAError(-num_workgroups, "mla_device_num_cus")
    nbytes = lib.mla_plan_bytes_bound(ctypes.byref(shape), int(num_workgroups))
    if nbytes == 0:
        # let the planner report why the shape is rejected
        nbytes = 64
    host = np.zeros((nbytes + 3) // 4, dtype=np.int32)
    info = PlanInfo()
    fn = lib.mla_decode_plan_fixed if fixed else lib.mla_decode_plan
    st = fn(ctypes.byref(shape), kv.ctypes.data if kv.size else None,
            None if ql is None else ql.ctypes.data, int(num_workgroups),
            host.ctypes.data, host.nbytes, ctypes.byref(info))
    _check(st, "mla_decode_plan_fixed" if fixed else "mla_decode_plan")
    host = host[: info.plan_bytes // 4].copy()
    dev_t = None
    if upload:
        import torch
        dev_t = torch.from_numpy(host).to(device or "cuda")
    return Plan(info=info, host=host, device=dev_t)


def plan_device(shape: Shape, kv_lens, q_lens=None, plan_buf=None, status=None,
                num_workgroups: Optional[int] = None, stream=None) -> Plan:
    """Build the fixed-shape plan on the GPU from device length tensors
    (``mla_decode_plan_device``).  ``plan_buf`` (int32, at least
    ``info.plan_bytes``) is reused when given; ``status`` (one int32 on the
    device) receives the plan's status.  The returned Plan has no host image."""
    import torch
    lib = load_library()
    dev = kv_lens.device
    if num_workgroups is None:
        num_workgroups = lib.mla_device_num_cus(dev.index or 0)
        if num_workgroups <= 0:
            raise MLAError(-num_workgroups, "mla_device_num_cus")
    for name, t in (("kv_lens", kv_lens), ("q_lens", q_lens), ("status", status)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or t.device != dev):
            raise ValueError(f"{name} must be a contiguous int32 tensor on {dev}")
    if kv_lens.numel() != shape.batch or (q_lens is not None and q_lens.numel() != shape.batch):
        raise ValueError("kv_lens / q_lens must hold batch elements")
    if status is not None and status.numel() != 1:
        raise ValueError("status must hold one element")
    nbytes = lib.mla_plan_bytes_bound(ctypes.byref(shape), int(num_workgroups))
    if plan_buf is None:
        plan_buf = torch.empty((max(nbytes, 64) + 3) // 4, dtype=torch.int32, device=dev)
    if plan_buf.dtype != torch.int32 or not plan_buf.is_contiguous() or plan_buf.device != dev:
        raise ValueError(f"plan_buf must be a contiguous int32 tensor on {dev}")
    info = PlanInfo()
    st = lib.mla_decode_plan_device(ctypes.byref(shape), int(num_workgroups), _ptr(kv_lens),
                                    _ptr(q_lens), _ptr(plan_buf), plan_buf.numel() * 4,
                                    _ptr(status), ctypes.byref(info), _stream(stream))
    _check(st, "mla_decode_plan_device")
    return Plan(info=info, host=None, device=plan_buf)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def decode_fwd(shape: Shape, pl: Plan, q, kv_cache, block_table, kv_lens, q_lens, sm_scale: float,
               out, lse, workspace, kv_scale=None, stream=None):
    """Launch the main kernel (``mla_decode_fwd``) on torch device tensors.

    The library reads ``MLA_DECODE_KERNEL`` at each call: ``w8`` or ``split``
    run a two-waves-per-SIMD candidate for one-phase plans (bf16 partials,
    merged by ``combine`` under the same setting), ``qres`` the Q-resident
    rebuild of the e4m3 kernels; none of them has run on a GPU yet, and the
    default (unset) runs the validated kernels."""
    lib = load_library()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.mla_decode_fwd(ctypes.byref(shape), ctypes.byref(pl.info), _ptr(pl.device), _ptr(q),
                            _ptr(kv_cache), _ptr(kv_scale), _ptr(block_table), _ptr(kv_lens),
                            _ptr(q_lens), float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                            ws_bytes, _stream(stream))
    _check(st, "mla_decode_fwd")


def combine(shape: Shape, pl: Plan, workspace, q_lens, out, lse, stream=None):
    """Launch the partial merge (``mla_combine``)."""
    lib = load_library()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.mla_combine(ctypes.byref(shape), ctypes.byref(pl.info), _ptr(pl.device),
                         _ptr(workspace), ws_bytes, _ptr(q_lens), _ptr(out), _ptr(lse),
                         _stream(stream))
    _check(st, "mla_combine")


def check(shape: Shape, pl: Plan, block_table, kv_lens, q_lens=None, err=None, stream=None,
          wait: bool = True):
    """Validate the device-resident inputs of a decode (``mla_decode_check``):
    the plan image against the device lengths, the lengths, and the
    block-table entries in use.  Returns (code, index), code 0 when all pass
    (names in CHECK_NAMES).  ``err`` (two int32 on the device) is reused when
    given; with ``wait=False`` nothing is synchronised and the codes stay in
    ``err``."""
    import torch
    dev = kv_lens.device
    if err is None:
        err = torch.empty(2, dtype=torch.int32, device=dev)
    if err.dtype != torch.int32 or err.numel() < 2 or not err.is_contiguous():
        raise ValueError("err must be a contiguous int32 tensor of two elements")
    B = shape.batch
    _sized(dev, [("block_table", block_table, B * shape.max_pages_per_seq * 4, 4),
                 ("kv_lens", kv_lens, B * 4, 4), ("q_lens", q_lens, B * 4, 4)])
    lib = load_library()
    st = lib.mla_decode_check(ctypes.byref(shape), ctypes.byref(pl.info), _ptr(pl.device),
                              _ptr(block_table), _ptr(kv_lens), _ptr(q_lens), _ptr(err),
                              _stream(stream))
    _check(st, "mla_decode_check")
    if not wait:
        return None
    got = err.cpu().tolist()   # waits for the stream
    return int(got[0]), int(got[1])


def debug_check_enabled() -> bool:
    return os.environ.get("MLA_DEBUG_CHECK", "0") not in ("", "0")


def alloc_workspace(pl: Plan, device="cuda"):
    import torch
    n = max(1, (pl.workspace_bytes + 255) // 256 * 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode(shape: Shape, pl: Plan, q, kv_cache, block_table, kv_lens, q_lens, sm_scale: float, *,
           kv_scale=None, out=None, lse=None, workspace=None, stream=None):
    """Full decode step: main kernel, then the combine of split row blocks.

    q [B, q_max, H, 576] bf16; kv_cache [pages, P, 576] bf16 (or uint8 e4m3 with
    kv_scale [pages, P] fp32); block_table [B, max_pages] int32; kv_lens / q_lens
    [B] int32 on the device.  Returns (out [B, q_max, H, 512] bf16, lse fp32).
    With MLA_DEBUG_CHECK=1 the device inputs first pass ``check`` (one small
    kernel and a wait); a failure raises MLAInputError before any decode work."""
    import torch
    B, qmax, H = shape.batch, shape.max_q_len, shape.num_heads
    dev = q.device
    if q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bfloat16 tensor")
    if tuple(q.shape) != (B, qmax, H, D_LATENT + D_ROPE):
        raise ValueError(f"q shape {tuple(q.shape)} does not match the shape struct")
    _decode_sizes(shape, q, kv_cache, kv_scale, block_table, kv_lens, q_lens, out, lse)
    if out is None:
        out = torch.empty((B, qmax, H, D_LATENT), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, qmax, H), dtype=torch.float32, device=dev)
    if workspace is None and pl.info.num_partials > 0:
        workspace = alloc_workspace(pl, dev)
    if debug_check_enabled():
        # checked mode: the device inputs are validated first, and a bad one
        # raises here instead of reaching the kernels
        code, index = check(shape, pl, block_table, kv_lens, q_lens, stream=stream)
        if code:
            raise MLAInputError(code, index)
    decode_fwd(shape, pl, q, kv_cache, block_table, kv_lens, q_lens, sm_scale, out, lse,
               workspace, kv_scale=kv_scale, stream=stream)
    combine(shape, pl, workspace, q_lens, out, lse, stream=stream)
    return out, lse


def kv_append(shape: Shape, new_rows, block_table, kv_lens, kv_cache, *, new_lens=None,
              kv_scale=None, skipped=None, stream=None):
    """Write each sequence's new tokens into the paged cache (``mla_kv_append``).

    new_rows [B, max_new, 576] bf16 (max_new may exceed the decode's q_len
    limit); new_lens [B] int32 device tensor or None (all max_new);
    block_table / kv_lens as for ``decode`` (kv_lens counts the new tokens);
    kv_cache [pages, P, 576] bf16, or uint8 e4m3 with kv_scale [pages, P] fp32;
    skipped: optional int32 device tensor of one element that counts rows whose
    slot falls outside the pool (the caller zeroes it)."""
    import torch
    lib = load_library()
    if new_rows.dtype != torch.bfloat16 or not new_rows.is_contiguous() or new_rows.dim() != 3:
        raise ValueError("new_rows must be a contiguous [B, max_new, 576] bfloat16 tensor")
    if new_rows.shape[0] != shape.batch or new_rows.shape[2] != D_LATENT + D_ROPE:
        raise ValueError(f"new_rows shape {tuple(new_rows.shape)} does not match the shape struct")
    dev = new_rows.device
    for name, t in (("kv_cache", kv_cache), ("block_table", block_table), ("kv_lens", kv_lens),
                    ("new_lens", new_lens), ("kv_scale", kv_scale), ("skipped", skipped)):
        if t is not None and (not t.is_contiguous() or t.device != dev):
            raise ValueError(f"{name} must be contiguous and on {dev}")
    B, P, NP = shape.batch, shape.page_size, shape.num_pages
    fp8 = shape.kv_dtype == KV_FP8_E4M3
    sizes = [("kv_cache", kv_cache, NP * P * (D_LATENT + D_ROPE), 1 if fp8 else 2),
             ("block_table", block_table, B * shape.max_pages_per_seq, 4),
             ("kv_lens", kv_lens, B, 4), ("new_lens", new_lens, B, 4), ("skipped", skipped, 1, 4)]
    if fp8:
        sizes.append(("kv_scale", kv_scale, NP * P, 4))
    for name, t, n, esize in sizes:
        if t is None:
            continue
        if t.numel() != n or t.element_size() != esize:
            raise ValueError(f"{name} must hold {n} elements of {esize} bytes, "
                             f"not {t.numel()} of {t.element_size()}")
    st = lib.mla_kv_append(ctypes.byref(shape), int(new_rows.shape[1]), _ptr(new_rows),
                           _ptr(new_lens), _ptr(block_table), _ptr(kv_lens), _ptr(kv_cache),
                           _ptr(kv_scale), _ptr(skipped), _stream(stream))
    _check(st, "mla_kv_append")


def tree_attend(shape: Shape, q, kv_cache, block_table, kv_lens, q_lens, tree_mask, sm_scale: float,
                out, lse, kv_scale=None, stream=None):
    """Merge the tree-masked draft keys into a prefix decode's (out, lse) in
    place (``mla_tree_attend``).  tree_mask [B, max_q_len] int32/uint32 on the
    device: bit k of word t lets draft token t see draft k."""
    import torch
    B, qmax = shape.batch, shape.max_q_len
    if tuple(tree_mask.shape) != (B, qmax) or tree_mask.element_size() != 4:
        raise ValueError("tree_mask must be a [batch, max_q_len] tensor of 32-bit words")
    if lse is None or lse.dtype != torch.float32:
        raise ValueError("lse (the prefix decode's) is required")
    if not tree_mask.is_contiguous() or tree_mask.device != q.device:
        raise ValueError(f"tree_mask must be contiguous and on {q.device}")
    _decode_sizes(shape, q, kv_cache, kv_scale, block_table, kv_lens, q_lens, out, lse)
    lib = load_library()
    st = lib.mla_tree_attend(ctypes.byref(shape), _ptr(q), _ptr(kv_cache), _ptr(kv_scale),
                             _ptr(block_table), _ptr(kv_lens), _ptr(q_lens), _ptr(tree_mask),
                             float(sm_scale), _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "mla_tree_attend")


def decode_tree(shape: Shape, q, kv_cache, block_table, kv_lens_host, q_lens_host, kv_lens,
                q_lens, tree_mask, sm_scale: float, *, kv_scale=None, num_workgroups=None,
                stream=None):
    """Decode with tree-shaped drafts: a non-causal decode over the cached
    prefix (kv_len - q_len keys), then ``tree_attend``.  Host lengths plan the
    prefix decode; kv_lens / q_lens are their device copies (full kv_lens)."""
    import torch
    kv_h = np.asarray(kv_lens_host, np.int32)
    ql_h = np.asarray(q_lens_host, np.int32)
    prefix_h = (kv_h - ql_h).astype(np.int32)
    pshape = Shape.make(batch=shape.batch, num_heads=shape.num_heads, max_q_len=shape.max_q_len,
                        page_size=shape.page_size, num_pages=shape.num_pages,
                        max_pages_per_seq=shape.max_pages_per_seq, kv_dtype=shape.kv_dtype,
                        causal=False)
    pl = plan(pshape, prefix_h, ql_h, num_workgroups=num_workgroups, device=q.device)
    prefix = torch.from_numpy(prefix_h).to(q.device)
    out, lse = decode(pshape, pl, q, kv_cache, block_table, prefix, q_lens, sm_scale,
                      kv_scale=kv_scale, stream=stream)
    tree_attend(shape, q, kv_cache, block_table, kv_lens, q_lens, tree_mask, sm_scale, out, lse,
                kv_scale=kv_scale, stream=stream)
    return out, lse


# ------------------------------------------------------------- quantized prefill

@dataclass
class PrefillQuant:
    """mla_prefill_quantize's outputs (torch device tensors)."""
    q_codes: object       # [T, H, 192] int8
    q_scale: object       # [T, H] fp32
    k_codes: object       # [T, H, 192] int8
    k_scale: object       # [blocks, H] fp32
    v_codes: object       # [blocks, H, 128, 128] uint8 (e4m3, PV operand key order)
    v_scale: object       # [blocks, H, 128] fp32 powers of two


def prefill_alloc_quant(shape: PrefillShape, device) -> PrefillQuant:
    import torch
    T, H, nb = shape.num_tokens, shape.num_heads, shape.num_blocks
    return PrefillQuant(
        q_codes=torch.empty((T, H, PREFILL_D_QK), dtype=torch.int8, device=device),
        q_scale=torch.empty((T, H), dtype=torch.float32, device=device),
        k_codes=torch.empty((T, H, PREFILL_D_QK), dtype=torch.int8, device=device),
        k_scale=torch.empty((nb, H), dtype=torch.float32, device=device),
        v_codes=torch.empty((nb, H, PREFILL_D_V, PREFILL_BLOCK), dtype=torch.uint8, device=device),
        v_scale=torch.empty((nb, H, PREFILL_D_V), dtype=torch.float32, device=device))


def _prefill_quant_sizes(shape: PrefillShape, dev, quant: PrefillQuant):
    T, H, nb = shape.num_tokens, shape.num_heads, shape.num_blocks
    _sized(dev, [("q_codes", quant.q_codes, T * H * PREFILL_D_QK, 1),
                 ("q_scale", quant.q_scale, T * H * 4, 4),
                 ("k_codes", quant.k_codes, T * H * PREFILL_D_QK, 1),
                 ("k_scale", quant.k_scale, nb * H * 4, 4),
                 ("v_codes", quant.v_codes, nb * H * PREFILL_D_V * PREFILL_BLOCK, 1),
                 ("v_scale", quant.v_scale, nb * H * PREFILL_D_V * 4, 4)])


def prefill_quantize(shape: PrefillShape, cu_seqlens, q, k, v, quant: PrefillQuant = None,
                     stream=None) -> PrefillQuant:
    """``mla_prefill_quantize``: packed bf16 q, k [T, H, 192] and v [T, H, 128]
    to INT8 / e4m3 codes and scales; cu_seqlens [S + 1] int32 on the device."""
    quant = prefill_alloc_quant(shape, q.device) if quant is None else quant
    T, H = shape.num_tokens, shape.num_heads
    _sized(q.device, [("cu_seqlens", cu_seqlens, (shape.num_seqs + 1) * 4, 4),
                      ("q", q, T * H * PREFILL_D_QK * 2, 2), ("k", k, T * H * PREFILL_D_QK * 2, 2),
                      ("v", v, T * H * PREFILL_D_V * 2, 2)])
    _prefill_quant_sizes(shape, q.device, quant)
    lib = load_library()
    st = lib.mla_prefill_quantize(ctypes.byref(shape), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(quant.q_codes), _ptr(quant.q_scale), _ptr(quant.k_codes),
                                  _ptr(quant.k_scale), _ptr(quant.v_codes), _ptr(quant.v_scale),
                                  _stream(stream))
    _check(st, "mla_prefill_quantize")
    return quant


def prefill_attn(shape: PrefillShape, cu_seqlens, quant: PrefillQuant, sm_scale: float, out=None,
                 lse=None, stream=None):
    """``mla_prefill_attn``: causal attention from the quantized inputs.
    Returns (O [T, H, 128] bf16, LSE [T, H] fp32)."""
    import torch
    dev = quant.q_codes.device
    T, H = shape.num_tokens, shape.num_heads
    if out is None:
        out = torch.empty((T, H, PREFILL_D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _sized(dev, [("cu_seqlens", cu_seqlens, (shape.num_seqs + 1) * 4, 4),
                 ("out", out, T * H * PREFILL_D_V * 2, 2), ("lse", lse, T * H * 4, 4)])
    _prefill_quant_sizes(shape, dev, quant)
    lib = load_library()
    st = lib.mla_prefill_attn(ctypes.byref(shape), _ptr(cu_seqlens), _ptr(quant.q_codes),
                              _ptr(quant.q_scale), _ptr(quant.k_codes), _ptr(quant.k_scale),
                              _ptr(quant.v_codes), _ptr(quant.v_scale), float(sm_scale), _ptr(out),
                              _ptr(lse), _stream(stream))
    _check(st, "mla_prefill_attn")
    return out, lse


def prefill(shape: PrefillShape, cu_seqlens, q, k, v, sm_scale: float, stream=None):
    """Quantize, then attend: the whole SageAttention-style prefill."""
    quant = prefill_quantize(shape, cu_seqlens, q, k, v, stream=stream)
    return prefill_attn(shape, cu_seqlens, quant, sm_scale, stream=stream)
