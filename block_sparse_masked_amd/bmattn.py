"""Python binding of libbmattn (ctypes; argument marshalling only).

Every step of the computation runs in the HIP library.  PyTorch provides
device memory and the current stream; this module only fills the C structs
declared in include/bmattn.h, allocates outputs with torch, and raises
``BmattnError`` on a non-zero status.  If the built library is missing (or
lacks a symbol) the first call raises ImportError: there is no other
implementation behind these names.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libbmattn.so")

MASK_FULL, MASK_CAUSAL, MASK_SHARED_PREFIX, MASK_STRIP_THINKING, MASK_COMPOSED = 0, 1, 2, 3, 4
KIND_CODES = {"full": MASK_FULL, "causal": MASK_CAUSAL, "shared_prefix": MASK_SHARED_PREFIX,
              "strip_thinking": MASK_STRIP_THINKING, "composed": MASK_COMPOSED}
TERM_CODES = {"causal": 1, "document": 2, "shared_prefix": 4, "strip_thinking": 8}
MAX_TERM_GROUPS = 4


def term_bits(terms) -> int:
    """The C ABI's terms word of a COMPOSED mask: an int passes through; one
    group (term names) is its OR of TERM_CODES; a sequence of groups puts
    group g in bits 4g .. 4g+3 (an OR of AND-groups)."""
    if isinstance(terms, int):
        return terms
    terms = tuple(terms)
    groups = (terms,) if all(isinstance(t, str) for t in terms) else terms
    _require(0 < len(groups) <= MAX_TERM_GROUPS, "terms",
             f"a composed mask takes 1 to {MAX_TERM_GROUPS} term groups (got {len(groups)})")
    bits = 0
    for g, group in enumerate(groups):
        _require(not isinstance(group, str) and len(group) > 0, "terms", f"malformed term group {group!r}")
        bits |= sum(TERM_CODES[t] for t in set(group)) << (4 * g)
    return bits
F32, BF16 = 0, 1
TILE_EMPTY, TILE_PARTIAL, TILE_FULL = 0, 1, 2
STATUS = {0: "OK", 1: "EINVAL", 2: "EUNSUPPORTED", 3: "EALIGN", 4: "EHIP", 5: "EWORKSPACE"}

EXPORTS = ("bmattn_block_mask_shape", "bmattn_build_block_mask", "bmattn_forward_workspace_size",
           "bmattn_forward", "bmattn_forward_noalloc", "bmattn_paged_gather", "bmattn_debug_dense_mask", "bmattn_validate",
           "bmattn_duplicated_answer_ids", "bmattn_transpose_block_mask",
           "bmattn_backward_workspace_size", "bmattn_backward", "bmattn_status_string",
           "bmattn_last_error", "bmattn_abi_version")

_p = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)


class MaskDescC(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
                ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
                ("total_q", ctypes.c_int64), ("total_k", ctypes.c_int64),
                ("think_role", ctypes.c_int32), ("terms", ctypes.c_int32),
                ("cu_seqlens_q", _p), ("cu_seqlens_k", _p), ("seg_q", _p), ("seg_k", _p),
                ("role_k", _p), ("turn_q", _p), ("turn_k", _p), ("doc_q", _p), ("doc_k", _p)]


class BlockMaskC(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("n_seqs", ctypes.c_int32), ("n_qt", ctypes.c_int32), ("n_kt", ctypes.c_int32),
                ("reserved0", ctypes.c_int32),
                ("tile_class", _p), ("full_cnt", _p), ("part_cnt", _p), ("full_idx", _p),
                ("part_idx", _p), ("row_order", _p)]


class FwdArgsC(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("q", _p), ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
                ("k", _p), ("k_stride_tok", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
                ("v", _p), ("v_stride_tok", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
                ("o", _p), ("o_stride_tok", ctypes.c_int64), ("o_stride_head", ctypes.c_int64),
                ("lse", _p), ("lse_stride_head", ctypes.c_int64),
                ("block_table", _p), ("block_table_stride", ctypes.c_int64),
                ("num_pages", ctypes.c_int64), ("scale", ctypes.c_float),
                ("reserved0", ctypes.c_int32), ("workspace", _p), ("workspace_bytes", ctypes.c_size_t)]


class BlockMaskColsC(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("n_seqs", ctypes.c_int32), ("n_qt", ctypes.c_int32), ("n_kt", ctypes.c_int32),
                ("reserved0", ctypes.c_int32),
                ("full_cnt", _p), ("part_cnt", _p), ("full_idx", _p), ("part_idx", _p),
                ("col_order", _p)]


class BwdArgsC(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("reserved0", ctypes.c_int32)] + [
        f for name in ("q", "k", "v", "o", "do")
        for f in ((name if name != "do" else "dout", _p), (f"{name}_stride_tok", ctypes.c_int64),
                  (f"{name}_stride_head", ctypes.c_int64))] + [
        ("lse", _p), ("lse_stride_head", ctypes.c_int64)] + [
        f for name in ("dq", "dk", "dv")
        for f in ((name, _p), (f"{name}_stride_tok", ctypes.c_int64),
                  (f"{name}_stride_head", ctypes.c_int64))] + [
        ("scale", ctypes.c_float), ("reserved1", ctypes.c_int32), ("workspace", _p),
        ("workspace_bytes", ctypes.c_size_t)]


class BmattnError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}: {msg}")
        self.status = status


_LIB = None


def lib():
    """The loaded library (loaded once; raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libbmattn is not built ({LIB_PATH} missing): run "
                              "python -m block_sparse_masked_amd.build")
        L = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
        L.bmattn_status_string.restype = ctypes.c_char_p
        L.bmattn_last_error.restype = ctypes.c_char_p
        L.bmattn_abi_version.restype = ctypes.c_int
        L.bmattn_block_mask_shape.argtypes = [ctypes.POINTER(MaskDescC), ctypes.c_int32,
                                              ctypes.c_int32, _i32p, _i32p,
                                              ctypes.POINTER(ctypes.c_int64),
                                              ctypes.POINTER(ctypes.c_int64)]
        L.bmattn_build_block_mask.argtypes = [ctypes.POINTER(MaskDescC), ctypes.POINTER(BlockMaskC), _p]
        L.bmattn_forward_workspace_size.argtypes = [ctypes.POINTER(FwdArgsC), ctypes.POINTER(MaskDescC),
                                                    ctypes.POINTER(BlockMaskC),
                                                    ctypes.POINTER(ctypes.c_size_t)]
        L.bmattn_forward.argtypes = [ctypes.POINTER(FwdArgsC), ctypes.POINTER(MaskDescC),
                                     ctypes.POINTER(BlockMaskC), _p]
        L.bmattn_forward_noalloc.argtypes = [ctypes.POINTER(FwdArgsC), ctypes.POINTER(MaskDescC),
                                             ctypes.POINTER(BlockMaskC), _p]
        L.bmattn_paged_gather.argtypes = [_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int64, _p, ctypes.c_int64,
                                          ctypes.POINTER(MaskDescC), _p, _p]
        L.bmattn_debug_dense_mask.argtypes = [ctypes.POINTER(MaskDescC), ctypes.POINTER(BlockMaskC),
                                              ctypes.c_int32, _p, ctypes.c_int64, _p]
        L.bmattn_validate.argtypes = [ctypes.POINTER(MaskDescC), _p, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_int64, _p, _p]
        L.bmattn_duplicated_answer_ids.argtypes = [ctypes.POINTER(MaskDescC), _p, ctypes.c_int32,
                                                   ctypes.c_int32, _p, _p, _p, _p]
        L.bmattn_transpose_block_mask.argtypes = [ctypes.POINTER(BlockMaskC),
                                                  ctypes.POINTER(BlockMaskColsC), _p]
        L.bmattn_backward_workspace_size.argtypes = [ctypes.POINTER(BwdArgsC),
                                                     ctypes.POINTER(MaskDescC),
                                                     ctypes.POINTER(ctypes.c_size_t)]
        L.bmattn_backward.argtypes = [ctypes.POINTER(BwdArgsC), ctypes.POINTER(MaskDescC),
                                      ctypes.POINTER(BlockMaskC), ctypes.POINTER(BlockMaskColsC), _p]
        for name in EXPORTS:
            getattr(L, name).restype = getattr(L, name).restype or ctypes.c_int
        _LIB = L
    return _LIB


def _check(status: int, fn: str):
    if status != 0:
        raise BmattnError(status, fn, lib().bmattn_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _i32(t: Optional[torch.Tensor], device) -> Optional[torch.Tensor]:
    if t is None:
        return None
    t = torch.as_tensor(t)
    return t.to(device=device, dtype=torch.int32).contiguous()


@dataclass
class MaskDesc:
    """A mask description (owns its device id arrays)."""

    kind: int
    n_seqs: int
    max_seqlen_q: int
    max_seqlen_k: int
    total_q: int
    total_k: int
    cu_seqlens_q: torch.Tensor
    cu_seqlens_k: torch.Tensor
    seg_q: Optional[torch.Tensor] = None
    seg_k: Optional[torch.Tensor] = None
    role_k: Optional[torch.Tensor] = None
    turn_q: Optional[torch.Tensor] = None
    turn_k: Optional[torch.Tensor] = None
    think_role: int = 1
    # For a description relabelled from duplicated answers: (the description
    # with the layout's own ids, role_q, loss_role, history_role).
    duplicated_from: Optional[tuple] = None
    terms: int = 0  # COMPOSED: term groups, group g in bits 4g..4g+3 (see term_bits)
    doc_q: Optional[torch.Tensor] = None
    doc_k: Optional[torch.Tensor] = None

    @staticmethod
    def create(kind, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, *,
               device="cuda", seg_q=None, seg_k=None, role_q=None, role_k=None, turn_q=None,
               turn_k=None, think_role: int = 1, loss_role: int = 2,
               history_role: int = 3, doc_q=None, doc_k=None, terms=()) -> "MaskDesc":
        """A description; kind "strip_thinking_duplicated" takes the ids of a
        layout with duplicated answer spans (role_q, role_k with loss_role
        and history_role, turn_q, turn_k) and returns the STRIP_THINKING
        description that bmattn_duplicated_answer_ids relabels them to; kind
        "composed" takes ``terms`` (one group of TERM_CODES names, a sequence
        of such groups -- an OR of ANDs --, or the packed int; see term_bits)
        and the ids those terms read (document: doc_q, doc_k)."""
        if kind == "strip_thinking_duplicated":
            src = MaskDesc.create("strip_thinking", cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                  max_seqlen_k, device=device, role_k=role_k, turn_q=turn_q,
                                  turn_k=turn_k, think_role=think_role)
            return duplicated_answer_ids(src, _i32(role_q, device), loss_role=loss_role,
                                         history_role=history_role)[0]
        kind = KIND_CODES[kind] if isinstance(kind, str) else int(kind)
        cq = _i32(cu_seqlens_q, device)
        ck = _i32(cu_seqlens_k, device)
        n = int(cq.numel()) - 1
        tq = int(cq[-1].item()) if n >= 0 else 0
        tk = int(ck[-1].item()) if n >= 0 else 0
        if kind == MASK_COMPOSED:
            bits = term_bits(terms)
        else:
            bits = 0
        return MaskDesc(kind, n, int(max_seqlen_q), int(max_seqlen_k), tq, tk, cq, ck,
                        _i32(seg_q, device), _i32(seg_k, device), _i32(role_k, device),
                        _i32(turn_q, device), _i32(turn_k, device), int(think_role),
                        terms=int(bits), doc_q=_i32(doc_q, device), doc_k=_i32(doc_k, device))

    def c(self) -> MaskDescC:
        return MaskDescC(self.kind, self.n_seqs, self.max_seqlen_q, self.max_seqlen_k,
                         self.total_q, self.total_k, self.think_role, self.terms,
                         _ptr(self.cu_seqlens_q), _ptr(self.cu_seqlens_k), _ptr(self.seg_q),
                         _ptr(self.seg_k), _ptr(self.role_k), _ptr(self.turn_q), _ptr(self.turn_k),
                         _ptr(self.doc_q), _ptr(self.doc_k))


@dataclass
class BlockMask:
    """Device arrays of a block mask (see bmattn_block_mask in include/bmattn.h)."""

    block_m: int
    block_n: int
    n_seqs: int
    n_qt: int
    n_kt: int
    tile_class: torch.Tensor
    full_cnt: torch.Tensor
    part_cnt: torch.Tensor
    full_idx: torch.Tensor
    part_idx: torch.Tensor
    row_order: torch.Tensor

    def c(self) -> BlockMaskC:
        return BlockMaskC(self.block_m, self.block_n, self.n_seqs, self.n_qt, self.n_kt, 0,
                          _ptr(self.tile_class), _ptr(self.full_cnt), _ptr(self.part_cnt),
                          _ptr(self.full_idx), _ptr(self.part_idx), _ptr(self.row_order))


def block_mask_shape(desc: MaskDesc, block_m: int, block_n: int):
    n_qt, n_kt = ctypes.c_int32(), ctypes.c_int32()
    rows, tiles = ctypes.c_int64(), ctypes.c_int64()
    d = desc.c()
    _check(lib().bmattn_block_mask_shape(ctypes.byref(d), block_m, block_n, ctypes.byref(n_qt),
                                         ctypes.byref(n_kt), ctypes.byref(rows),
                                         ctypes.byref(tiles)), "bmattn_block_mask_shape")
    return n_qt.value, n_kt.value, rows.value, tiles.value


def alloc_block_mask(desc: MaskDesc, block_m: int, block_n: int, device="cuda") -> BlockMask:
    n_qt, n_kt, rows, tiles = block_mask_shape(desc, block_m, block_n)
    i32 = dict(dtype=torch.int32, device=device)
    return BlockMask(block_m, block_n, desc.n_seqs, n_qt, n_kt,
                     torch.empty(tiles, dtype=torch.uint8, device=device),
                     torch.empty(rows, **i32), torch.empty(rows, **i32),
                     torch.empty(tiles, **i32), torch.empty(tiles, **i32), torch.empty(rows, **i32))


def build_block_mask(desc: MaskDesc, block_m: int, block_n: int, out: Optional[BlockMask] = None,
                     stream=None) -> BlockMask:
    """bmattn_build_block_mask: tile classes, kv-tile lists and row schedule."""
    bm = alloc_block_mask(desc, block_m, block_n, desc.cu_seqlens_q.device) if out is None else out
    _check_desc(desc, "build_block_mask", desc.cu_seqlens_q.device)
    _require((bm.block_m, bm.block_n) == (block_m, block_n), "build_block_mask",
             f"out was allocated for {bm.block_m}x{bm.block_n} tiles, not {block_m}x{block_n}")
    _check_tiles(bm, "build_block_mask", desc.cu_seqlens_q.device)
    d, t = desc.c(), bm.c()
    _check(lib().bmattn_build_block_mask(ctypes.byref(d), ctypes.byref(t), _stream(stream)),
           "bmattn_build_block_mask")
    return bm


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise BmattnError(2, "forward", f"dtype {dt} is not supported")


def _require(ok: bool, fn: str, msg: str, status: int = 1):
    if not ok:
        raise BmattnError(status, fn, msg)


def _check_tensor(t, fn: str, name: str, device, dtype=None, shape=None, inner_contig=True):
    """One argument tensor: on ``device``, of ``dtype`` and ``shape`` (None
    entries match any extent), its last dimension contiguous."""
    _require(isinstance(t, torch.Tensor), fn, f"{name} must be a torch tensor")
    _require(t.device == device, fn, f"{name} is on {t.device}, expected {device}")
    if dtype is not None:
        _require(t.dtype == dtype, fn, f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None:
        _require(t.dim() == len(shape) and all(w is None or w == g for w, g in zip(shape, t.shape)),
                 fn, f"{name} has shape {tuple(t.shape)}, expected "
                     f"{tuple('*' if w is None else w for w in shape)}")
    if inner_contig and t.dim() > 0 and t.numel() > 0:
        _require(t.stride(-1) == 1, fn, f"{name} must be contiguous in its last dimension")


def _check_desc(desc: MaskDesc, fn: str, device):
    """The description's device arrays: on ``device``, int32, of the lengths
    its sizes give."""
    n, tq, tk = desc.n_seqs, desc.total_q, desc.total_k
    for name, length in (("cu_seqlens_q", n + 1), ("cu_seqlens_k", n + 1), ("seg_q", tq),
                         ("seg_k", tk), ("role_k", tk), ("turn_q", tq), ("turn_k", tk),
                         ("doc_q", tq), ("doc_k", tk)):
        t = getattr(desc, name)
        if t is not None:
            _check_tensor(t, fn, f"desc.{name}", device, torch.int32, (length,))
            _require(t.is_contiguous(), fn, f"desc.{name} must be contiguous")


def _check_tiles(tiles, fn: str, device, row_major: bool = True):
    """A block mask's arrays (or column lists'): on ``device``, int32 (classes
    uint8), with as many elements as its shape needs."""
    if row_major:
        rows = tiles.n_seqs * tiles.n_qt
        arrays = (("tile_class", torch.uint8, rows * tiles.n_kt), ("full_cnt", torch.int32, rows),
                  ("part_cnt", torch.int32, rows), ("full_idx", torch.int32, rows * tiles.n_kt),
                  ("part_idx", torch.int32, rows * tiles.n_kt), ("row_order", torch.int32, rows))
    else:
        cols = tiles.n_seqs * tiles.n_kt
        arrays = (("full_cnt", torch.int32, cols), ("part_cnt", torch.int32, cols),
                  ("full_idx", torch.int32, cols * tiles.n_qt),
                  ("part_idx", torch.int32, cols * tiles.n_qt), ("col_order", torch.int32, cols))
    for name, dt, numel in arrays:
        t = getattr(tiles, name)
        _check_tensor(t, fn, f"tiles.{name}", device, dt)
        _require(t.is_contiguous() and t.numel() >= numel, fn,
                 f"tiles.{name} must be contiguous with at least {numel} elements")


def _check_fwd(q, k, v, o, lse, desc: MaskDesc, tiles, block_table, workspace, fn="forward"):
    """Everything the C ABI cannot see: devices, dtypes, extents and the
    contiguous head_dim of every tensor argument of bmattn_forward."""
    _check_tensor(q, fn, "q", q.device, None, (desc.total_q, None, None))
    dev, dt = q.device, q.dtype
    H, D = q.shape[1], q.shape[2]
    _check_tensor(o, fn, "out", dev, dt, (desc.total_q, H, D))
    if block_table is None:
        for name, t in (("k", k), ("v", v)):
            _check_tensor(t, fn, name, dev, dt, (desc.total_k, H, D))
    else:
        _check_tensor(k, fn, "k pool", dev, dt, (None, None, H, D))
        _check_tensor(v, fn, "v pool", dev, dt, tuple(k.shape))
        _check_tensor(block_table, fn, "block_table", dev, torch.int32, (None, None))
        _require(block_table.shape[0] >= desc.n_seqs, fn,
                 f"block_table has {block_table.shape[0]} rows for {desc.n_seqs} sequences")
    if lse is not None:
        _check_tensor(lse, fn, "lse", dev, torch.float32, (H, desc.total_q))
    if workspace is not None:
        _check_tensor(workspace, fn, "workspace", dev)
        _require(workspace.is_contiguous(), fn, "workspace must be contiguous")
    _check_desc(desc, fn, dev)
    if tiles is not None:
        _check_tiles(tiles, fn, dev)


def _check_bwd(q, k, v, o, lse, do, dq, dk, dv, desc: MaskDesc, rows, cols, workspace,
               fn="backward"):
    """Devices, dtypes and extents of every tensor argument of bmattn_backward."""
    _check_tensor(q, fn, "q", q.device, None, (desc.total_q, None, None))
    dev, dt = q.device, q.dtype
    H, D = q.shape[1], q.shape[2]
    for name, t in (("o", o), ("do", do), ("dq", dq)):
        _check_tensor(t, fn, name, dev, dt, (desc.total_q, H, D))
    for name, t in (("k", k), ("v", v), ("dk", dk), ("dv", dv)):
        _check_tensor(t, fn, name, dev, dt, (desc.total_k, H, D))
    _check_tensor(lse, fn, "lse", dev, torch.float32, (H, desc.total_q))
    if workspace is not None:
        _check_tensor(workspace, fn, "workspace", dev)
        _require(workspace.is_contiguous(), fn, "workspace must be contiguous")
    _check_desc(desc, fn, dev)
    _check_tiles(rows, fn, dev)
    _check_tiles(cols, fn, dev, row_major=False)


def _fwd_args(q, k, v, o, lse, *, block_table=None, page_size=0, scale=0.0, workspace=None):
    H, D = q.shape[-2], q.shape[-1]
    if block_table is not None:
        # pools [num_pages, page_size, H, D]: token stride is per pool row
        num_pages = k.shape[0]
        page_size = k.shape[1]
        kst, ksh = k.stride(1), k.stride(2)
        vst, vsh = v.stride(1), v.stride(2)
        bt_stride = block_table.stride(0)
    else:
        num_pages = 0
        kst, ksh = k.stride(0), k.stride(1)
        vst, vsh = v.stride(0), v.stride(1)
        bt_stride = 0
    return FwdArgsC(_dtype_code(q.dtype), H, D, int(page_size), _ptr(q), q.stride(0), q.stride(1),
                    _ptr(k), kst, ksh, _ptr(v), vst, vsh, _ptr(o), o.stride(0), o.stride(1),
                    _ptr(lse), 0 if lse is None else lse.stride(0), _ptr(block_table), bt_stride,
                    num_pages, float(scale), 0, _ptr(workspace),
                    0 if workspace is None else workspace.numel() * workspace.element_size())


def forward_workspace_size(q, k, v, desc: MaskDesc, tiles: BlockMask, *, block_table=None) -> int:
    o = q  # only shapes and strides are read
    _check_fwd(q, k, v, o, None, desc, tiles, block_table, None, "forward_workspace_size")
    a = _fwd_args(q, k, v, o, None, block_table=block_table)
    n = ctypes.c_size_t()
    d, t = desc.c(), tiles.c()
    _check(lib().bmattn_forward_workspace_size(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t),
                                               ctypes.byref(n)), "bmattn_forward_workspace_size")
    return n.value


def forward(q, k, v, desc: MaskDesc, tiles: BlockMask, *, block_table=None, scale: float = 0.0,
            out=None, lse=None, workspace=None, with_lse: bool = True, stream=None):
    """bmattn_forward.  q [total_q, H, D]; k, v [total_k, H, D] or page pools
    [num_pages, page_size, H, D] with ``block_table`` [n_seqs, pages] int32.
    Returns (O, LSE) with O like q and LSE fp32 [H, total_q]."""
    _require(isinstance(q, torch.Tensor) and q.is_cuda, "forward", "q must be a device (cuda) tensor")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    _check_fwd(q, k, v, out, lse, desc, tiles, block_table, workspace)
    if workspace is None:
        need = forward_workspace_size(q, k, v, desc, tiles, block_table=block_table)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a = _fwd_args(q, k, v, out, lse, block_table=block_table, scale=scale, workspace=workspace)
    d, t = desc.c(), tiles.c()
    _check(lib().bmattn_forward(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t), _stream(stream)),
           "bmattn_forward")
    return out, lse


NOALLOC_MAX_WORKSPACE = 96 << 20  # BMATTN_NOALLOC_MAX_WORKSPACE


def forward_noalloc(q, k, v, desc: MaskDesc, tiles: BlockMask, *, block_table=None,
                    scale: float = 0.0, out=None, lse=None, stream=None):
    """bmattn_forward_noalloc: the forward with the decode split workspace
    taken from the library's static scratch (the library allocates nothing;
    this binding allocates ``out`` / ``lse`` only when they are not given).
    Calls that overlap in time on one GPU race on that scratch."""
    _require(isinstance(q, torch.Tensor) and q.is_cuda, "forward_noalloc",
             "q must be a device (cuda) tensor")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    _check_fwd(q, k, v, out, lse, desc, tiles, block_table, None, "forward_noalloc")
    a = _fwd_args(q, k, v, out, lse, block_table=block_table, scale=scale, workspace=None)
    d, t = desc.c(), tiles.c()
    _check(lib().bmattn_forward_noalloc(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t),
                                        _stream(stream)), "bmattn_forward_noalloc")
    return out, lse


def paged_gather(pool, block_table, desc: MaskDesc, stream=None):
    """bmattn_paged_gather: pool [num_pages, page_size, H, D] -> [total_k, H, D]."""
    _check_tensor(pool, "paged_gather", "pool", pool.device, None, (None, None, None, None))
    _require(pool.dtype in (torch.bfloat16, torch.float32), "paged_gather",
             f"pool dtype {pool.dtype} is not supported", 2)
    _check_tensor(block_table, "paged_gather", "block_table", pool.device, torch.int32, (None, None))
    _require(block_table.shape[0] >= desc.n_seqs, "paged_gather",
             f"block_table has {block_table.shape[0]} rows for {desc.n_seqs} sequences")
    _check_desc(desc, "paged_gather", pool.device)
    n_pages, ps, H, D = pool.shape
    out = torch.empty((desc.total_k, H, D), dtype=pool.dtype, device=pool.device)
    d = desc.c()
    _check(lib().bmattn_paged_gather(_ptr(pool), pool.stride(1), pool.stride(2), pool.element_size(),
                                     H, D, ps, n_pages, _ptr(block_table), block_table.stride(0),
                                     ctypes.byref(d), _ptr(out), _stream(stream)),
           "bmattn_paged_gather")
    return out


def debug_dense_mask(desc: MaskDesc, tiles: BlockMask, seq: int, stream=None):
    """bmattn_debug_dense_mask: uint8 [n_qt*block_m, n_kt*block_n] of one sequence."""
    dev = tiles.tile_class.device
    _check_desc(desc, "debug_dense_mask", dev)
    _check_tiles(tiles, "debug_dense_mask", dev)
    rows, cols = tiles.n_qt * tiles.block_m, tiles.n_kt * tiles.block_n
    out = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    d, t = desc.c(), tiles.c()
    _check(lib().bmattn_debug_dense_mask(ctypes.byref(d), ctypes.byref(t), int(seq), _ptr(out), cols,
                                         _stream(stream)), "bmattn_debug_dense_mask")
    return out


def validate(desc: MaskDesc, block_table=None, page_size: int = 0, num_pages: int = 0,
             stream=None) -> int:
    """bmattn_validate: returns the flag word (0 = valid); synchronises."""
    dev = desc.cu_seqlens_q.device
    _check_desc(desc, "validate", dev)
    if block_table is not None:
        _check_tensor(block_table, "validate", "block_table", dev, torch.int32, (None, None))
        _require(block_table.shape[0] >= desc.n_seqs, "validate",
                 f"block_table has {block_table.shape[0]} rows for {desc.n_seqs} sequences")
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    d = desc.c()
    _check(lib().bmattn_validate(ctypes.byref(d), _ptr(block_table),
                                 0 if block_table is None else block_table.stride(0),
                                 int(page_size), int(num_pages), _ptr(flags), _stream(stream)),
           "bmattn_validate")
    return int(flags.item())


@dataclass
class BlockMaskCols:
    """Column lists of a block mask (see bmattn_block_mask_cols)."""

    block_m: int
    block_n: int
    n_seqs: int
    n_qt: int
    n_kt: int
    full_cnt: torch.Tensor
    part_cnt: torch.Tensor
    full_idx: torch.Tensor
    part_idx: torch.Tensor
    col_order: torch.Tensor

    def c(self) -> BlockMaskColsC:
        return BlockMaskColsC(self.block_m, self.block_n, self.n_seqs, self.n_qt, self.n_kt, 0,
                              _ptr(self.full_cnt), _ptr(self.part_cnt), _ptr(self.full_idx),
                              _ptr(self.part_idx), _ptr(self.col_order))


def transpose_block_mask(tiles: BlockMask, out: Optional[BlockMaskCols] = None,
                         stream=None) -> BlockMaskCols:
    """bmattn_transpose_block_mask: the column (kv-tile major) lists."""
    if out is None:
        cols = tiles.n_seqs * tiles.n_kt
        i32 = dict(dtype=torch.int32, device=tiles.tile_class.device)
        out = BlockMaskCols(tiles.block_m, tiles.block_n, tiles.n_seqs, tiles.n_qt, tiles.n_kt,
                            torch.empty(cols, **i32), torch.empty(cols, **i32),
                            torch.empty(cols * tiles.n_qt, **i32), torch.empty(cols * tiles.n_qt, **i32),
                            torch.empty(cols, **i32))
    _check_tiles(tiles, "transpose_block_mask", tiles.tile_class.device)
    _check_tiles(out, "transpose_block_mask", tiles.tile_class.device, row_major=False)
    t, c = tiles.c(), out.c()
    _check(lib().bmattn_transpose_block_mask(ctypes.byref(t), ctypes.byref(c), _stream(stream)),
           "bmattn_transpose_block_mask")
    return out


BWD_ROWS = (128, 64)   # block mask of the dQ pass (the forward's)
BWD_COLS = (64, 128)   # block mask whose column lists drive the dK / dV pass


def build_backward_cols(desc: MaskDesc, tiles: Optional[BlockMask] = None,
                        out: Optional[BlockMaskCols] = None, stream=None):
    """The 64 x 128 block mask of ``desc`` and its column lists; returns
    (tiles, cols).  Pass both back to rebuild into the same arrays."""
    tiles = build_block_mask(desc, *BWD_COLS, out=tiles, stream=stream)
    return tiles, transpose_block_mask(tiles, out=out, stream=stream)


def _bwd_args(q, k, v, o, do, lse, dq, dk, dv, scale=0.0, workspace=None):
    H, D = q.shape[-2], q.shape[-1]
    return BwdArgsC(_dtype_code(q.dtype), H, D, 0,
                    _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1),
                    _ptr(v), v.stride(0), v.stride(1), _ptr(o), o.stride(0), o.stride(1),
                    _ptr(do), do.stride(0), do.stride(1), _ptr(lse), lse.stride(0) if lse is not None else 0,
                    _ptr(dq), dq.stride(0), dq.stride(1), _ptr(dk), dk.stride(0), dk.stride(1),
                    _ptr(dv), dv.stride(0), dv.stride(1), float(scale), 0, _ptr(workspace),
                    0 if workspace is None else workspace.numel() * workspace.element_size())


def backward_workspace_size(q, desc: MaskDesc) -> int:
    a = _bwd_args(q, q, q, q, q, None, q, q, q)
    n = ctypes.c_size_t()
    d = desc.c()
    _check(lib().bmattn_backward_workspace_size(ctypes.byref(a), ctypes.byref(d), ctypes.byref(n)),
           "bmattn_backward_workspace_size")
    return n.value


def backward(q, k, v, o, lse, do, desc: MaskDesc, rows: BlockMask, cols: BlockMaskCols, *,
             scale: float = 0.0, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """bmattn_backward: (dQ, dK, dV) like q, k, v.  ``rows`` is the forward's
    128 x 64 block mask, ``cols`` the column lists of the 64 x 128 one
    (build_backward_cols)."""
    _require(isinstance(q, torch.Tensor) and q.is_cuda, "backward", "q must be a device (cuda) tensor")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_bwd(q, k, v, o, lse, do, dq, dk, dv, desc, rows, cols, workspace)
    if workspace is None:
        need = backward_workspace_size(q, desc)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    a = _bwd_args(q, k, v, o, do, lse, dq, dk, dv, scale, workspace)
    d, t, c = desc.c(), rows.c(), cols.c()
    _check(lib().bmattn_backward(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t), ctypes.byref(c),
                                 _stream(stream)), "bmattn_backward")
    return dq, dk, dv


def duplicated_answer_ids(desc: MaskDesc, role_q: torch.Tensor, *, loss_role: int = 2,
                          history_role: int = 3, out: Optional[MaskDesc] = None,
                          check: bool = False, stream=None):
    """bmattn_duplicated_answer_ids.  ``desc`` is a STRIP_THINKING description
    holding the ids of a layout with duplicated answer spans; returns
    (relabelled description, flags) where flags is a device int32 [1] tensor
    (0 = the layout meets the conditions) when ``check``, else None.  With
    ``out`` (a description from an earlier call on the same layout) the ids
    are rewritten into its arrays."""
    if out is None:
        out = MaskDesc(desc.kind, desc.n_seqs, desc.max_seqlen_q, desc.max_seqlen_k, desc.total_q,
                       desc.total_k, desc.cu_seqlens_q, desc.cu_seqlens_k, None, None,
                       torch.empty_like(desc.role_k), torch.empty_like(desc.turn_q), desc.turn_k,
                       desc.think_role, (desc, role_q, int(loss_role), int(history_role)))
    dev = desc.cu_seqlens_q.device
    _check_desc(desc, "duplicated_answer_ids", dev)
    _check_tensor(role_q, "duplicated_answer_ids", "role_q", dev, torch.int32, (desc.total_q,))
    _check_desc(out, "duplicated_answer_ids", dev)
    flags = torch.empty(1, dtype=torch.int32, device=role_q.device) if check else None
    d = desc.c()
    _check(lib().bmattn_duplicated_answer_ids(ctypes.byref(d), _ptr(role_q), int(loss_role),
                                              int(history_role), _ptr(out.role_k), _ptr(out.turn_q),
                                              _ptr(flags), _stream(stream)),
           "bmattn_duplicated_answer_ids")
    return out, flags


def relabel(desc: MaskDesc, check: bool = False, stream=None):
    """Reruns the relabelling of a description made from duplicated answers
    (into its own arrays); returns the flags tensor when ``check``."""
    src, role_q, loss_role, history_role = desc.duplicated_from
    return duplicated_answer_ids(src, role_q, loss_role=loss_role, history_role=history_role,
                                 out=desc, check=check, stream=stream)[1]

