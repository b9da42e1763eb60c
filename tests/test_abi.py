"""C-ABI checks that need no GPU: the library loads, exports every function
include/bmattn.h declares, and rejects invalid calls on the host before any
launch.  Every call here fails validation, so nothing reaches a device (the
fake pointers are never dereferenced)."""

import ctypes
import os
import re

import pytest

from block_sparse_masked_amd import bmattn as bm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a non-NULL, 16-byte aligned value that is never dereferenced


def _header_functions():
    src = open(os.path.join(ROOT, "include", "bmattn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bmattn_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _header_functions()
    assert len(names) >= 10
    L = bm.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(bm.EXPORTS)


def test_version_and_status_strings():
    L = bm.lib()
    assert L.bmattn_abi_version() == 2
    assert L.bmattn_status_string(0) == b"ok"
    assert L.bmattn_status_string(2) == b"unsupported configuration"
    assert L.bmattn_status_string(99) == b"unknown status"


def _desc(kind=bm.MASK_CAUSAL, n=2, mq=100, mk=100, tq=150, tk=150, ids=True, terms=0, docs=True):
    i = FAKE if ids else None
    dd = FAKE if docs else None
    d = bm.MaskDescC(kind, n, mq, mk, tq, tk, 1, terms, FAKE, FAKE, i, i, i, i, i, dd, dd)
    return d


def _call_shape(d, bm_, bn_):
    n_qt, n_kt = ctypes.c_int32(), ctypes.c_int32()
    rows, tiles = ctypes.c_int64(), ctypes.c_int64()
    rc = bm.lib().bmattn_block_mask_shape(ctypes.byref(d), bm_, bn_, ctypes.byref(n_qt),
                                          ctypes.byref(n_kt), ctypes.byref(rows), ctypes.byref(tiles))
    return rc, n_qt.value, n_kt.value, rows.value, tiles.value


def test_block_mask_shape_host_only():
    rc, n_qt, n_kt, rows, tiles = _call_shape(_desc(), 128, 64)
    assert rc == 0 and (n_qt, n_kt, rows, tiles) == (1, 2, 2, 4)
    rc, n_qt, n_kt, rows, tiles = _call_shape(_desc(mq=257, mk=20480), 128, 64)
    assert rc == 0 and (n_qt, n_kt) == (3, 320) and rows == 6 and tiles == 6 * 320


@pytest.mark.parametrize("bad", [
    dict(kind=7), dict(n=0), dict(mq=0), dict(mk=0), dict(tq=-1),
])
def test_desc_rejected(bad):
    rc, *_ = _call_shape(_desc(**bad), 128, 64)
    assert rc == 1
    assert bm.lib().bmattn_last_error()


@pytest.mark.parametrize("kind", [bm.MASK_SHARED_PREFIX, bm.MASK_STRIP_THINKING])
def test_missing_ids_rejected(kind):
    rc, *_ = _call_shape(_desc(kind=kind, ids=False), 128, 64)
    assert rc == 1
    assert b"needs" in bm.lib().bmattn_last_error()


@pytest.mark.parametrize("bmn", [(0, 64), (128, 0), (2048, 64), (128, 1025)])
def test_tile_shape_out_of_range(bmn):
    rc, *_ = _call_shape(_desc(), *bmn)
    assert rc == 2


def _tiles(d, block_m=128, block_n=64, **over):
    rc, n_qt, n_kt, rows, tiles = _call_shape(d, block_m, block_n)
    assert rc == 0
    t = bm.BlockMaskC(block_m, block_n, d.n_seqs, n_qt, n_kt, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for k, v in over.items():
        setattr(t, k, v)
    return t


def test_build_rejects_shape_mismatch_and_nulls():
    L = bm.lib()
    d = _desc()
    t = _tiles(d, n_kt=99)
    assert L.bmattn_build_block_mask(ctypes.byref(d), ctypes.byref(t), None) == 1
    t = _tiles(d, full_idx=None)
    assert L.bmattn_build_block_mask(ctypes.byref(d), ctypes.byref(t), None) == 1
    assert L.bmattn_build_block_mask(None, ctypes.byref(_tiles(d)), None) == 1


def _args(**over):
    a = bm.FwdArgsC(bm.BF16, 4, 128, 16, FAKE, 512, 128, FAKE, 512, 128, FAKE, 512, 128,
                    FAKE, 512, 128, None, 0, None, 0, 0, 0.0, 0, None, 0)
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=96), 2),
    (dict(dtype=5), 2),
    (dict(num_heads=0), 1),
    (dict(q=None), 1),
    (dict(k=FAKE + 8), 3),
    (dict(q_stride_tok=513), 3),
    (dict(scale=float("nan")), 1),
    (dict(lse=FAKE, lse_stride_head=3), 1),
    (dict(block_table=FAKE, page_size=0, num_pages=10, block_table_stride=100), 1),
    (dict(block_table=FAKE, page_size=16, num_pages=10, block_table_stride=2), 1),
])
def test_forward_rejected_before_launch(over, code):
    L = bm.lib()
    d = _desc()
    t = _tiles(d)
    a = _args(**over)
    assert L.bmattn_forward(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t), None) == code
    assert L.bmattn_last_error()


def test_forward_rejects_uncompiled_tile_shape():
    L = bm.lib()
    d = _desc()
    t = _tiles(d, block_m=64, block_n=64)
    assert L.bmattn_forward(ctypes.byref(_args()), ctypes.byref(d), ctypes.byref(t), None) == 2
    assert b"tile shape" in L.bmattn_last_error()


def test_decode_requires_workspace():
    L = bm.lib()
    d = _desc(mq=1, tq=2)
    t = _tiles(d, block_m=1, block_n=64)
    a = _args()
    n = ctypes.c_size_t()
    assert L.bmattn_forward_workspace_size(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t),
                                           ctypes.byref(n)) == 0
    # rows 2 x splits ceil(2/8)=1 x H 4 x (D 128 + 2) floats
    assert n.value == 2 * 1 * 4 * 130 * 4
    assert L.bmattn_forward(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t), None) == 5
    a = _args(workspace=FAKE, workspace_bytes=n.value - 4)
    assert L.bmattn_forward(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t), None) == 5


def test_prefill_needs_no_workspace():
    L = bm.lib()
    d = _desc()
    t = _tiles(d)
    n = ctypes.c_size_t(123)
    assert L.bmattn_forward_workspace_size(ctypes.byref(_args()), ctypes.byref(d), ctypes.byref(t),
                                           ctypes.byref(n)) == 0
    assert n.value == 0


def test_gather_and_debug_and_validate_rejections():
    L = bm.lib()
    d = _desc()
    assert L.bmattn_paged_gather(FAKE, 512, 128, 3, 4, 128, 16, 10, FAKE, 100, ctypes.byref(d),
                                 FAKE, None) == 1
    assert L.bmattn_paged_gather(FAKE, 512, 128, 2, 4, 128, 16, 10, FAKE, 2, ctypes.byref(d),
                                 FAKE, None) == 1
    assert L.bmattn_paged_gather(FAKE, 513, 128, 2, 4, 128, 16, 10, FAKE, 100, ctypes.byref(d),
                                 FAKE, None) == 3
    t = _tiles(d)
    assert L.bmattn_debug_dense_mask(ctypes.byref(d), ctypes.byref(t), 5, FAKE, 1 << 20, None) == 1
    assert L.bmattn_debug_dense_mask(ctypes.byref(d), ctypes.byref(t), 0, FAKE, 3, None) == 1
    assert L.bmattn_validate(ctypes.byref(d), None, 0, 0, 0, None, None) == 1
    assert L.bmattn_validate(ctypes.byref(d), FAKE, 0, 16, 10, FAKE, None) == 1


@pytest.mark.parametrize("terms,docs,ids,ok", [
    (1, True, True, True), (15, True, True, True), (2, True, False, True),
    (0, True, True, False),    # COMPOSED needs at least one term
    (16, True, True, True),    # group 1 alone ({causal})
    (0x8421, True, True, True),  # four groups
    (0x10000, True, True, False),  # beyond four groups
    (-1, True, True, False),
    (0x21, False, True, False),    # DOCUMENT in group 1 without doc arrays
    (0x4001, True, False, False),  # SHARED_PREFIX in group 3 without segments
    (2, False, True, False),   # DOCUMENT without doc arrays
    (4, True, False, False),   # SHARED_PREFIX without segments
    (8, True, False, False),   # STRIP_THINKING without roles / turns
])
def test_composed_description_validation(terms, docs, ids, ok):
    rc, *_ = _call_shape(_desc(kind=bm.MASK_COMPOSED, terms=terms, docs=docs, ids=ids), 128, 64)
    assert (rc == 0) == ok, bm.lib().bmattn_last_error()


def test_term_bits_packs_groups():
    assert bm.term_bits(("causal", "document")) == 3
    assert bm.term_bits((("causal",), ("document",))) == 0x21
    assert bm.term_bits((("strip_thinking",), ("document", "causal"), ("shared_prefix",),
                         ("causal",))) == 0x1438
    assert bm.term_bits(0x21) == 0x21
    for bad in ((), ((),), ((("causal",),) * 5)):
        with pytest.raises(bm.BmattnError):
            bm.term_bits(bad)


def test_terms_rejected_on_plain_kinds():
    rc, *_ = _call_shape(_desc(kind=bm.MASK_CAUSAL, terms=1), 128, 64)
    assert rc == 1 and b"terms must be 0" in bm.lib().bmattn_last_error()


def test_duplicated_answer_ids_rejected_before_launch():
    L = bm.lib()
    f = ctypes.c_void_p(FAKE)

    def call(d, role_q=f, loss=2, hist=3, rk=f, tq=f):
        return L.bmattn_duplicated_answer_ids(ctypes.byref(d), role_q, loss, hist, rk, tq, None, None)

    assert call(_desc(kind=bm.MASK_CAUSAL)) == 1          # not a STRIP_THINKING description
    assert call(_desc(kind=bm.MASK_STRIP_THINKING, ids=False)) == 1  # its ids missing
    st = _desc(kind=bm.MASK_STRIP_THINKING)
    assert call(st, role_q=None) == 1
    assert call(st, rk=None) == 1 and call(st, tq=None) == 1
    assert call(st, loss=3, hist=3) == 1                  # roles must differ
    assert call(st, loss=1) == 1 and call(st, hist=1) == 1  # think_role is 1
    assert b"roles must differ" in L.bmattn_last_error()


def test_missing_library_fails_loudly_on_first_call(tmp_path, monkeypatch):
    # No fallback: with the library path pointing nowhere, a call raises.
    from block_sparse_masked_amd import bmattn
    monkeypatch.setattr(bmattn, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(bmattn, "_LIB", None)
    with pytest.raises(ImportError):
        bmattn.lib()


def test_struct_layouts_match_the_header(tmp_path):
    # The binding's ctypes structs have the header's sizes and offsets
    # (compiled with the host C compiler; no device code involved).
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    checks = {
        "bmattn_mask_desc": (bm.MaskDescC, ["kind", "think_role", "terms", "cu_seqlens_q", "turn_k",
                                            "doc_q", "doc_k"]),
        "bmattn_block_mask": (bm.BlockMaskC, ["block_m", "tile_class", "row_order"]),
        "bmattn_block_mask_cols": (bm.BlockMaskColsC, ["block_m", "full_cnt", "col_order"]),
        "bmattn_fwd_args": (bm.FwdArgsC, ["q", "lse", "block_table", "scale", "workspace_bytes"]),
        "bmattn_bwd_args": (bm.BwdArgsC, ["q", "dout", "do_stride_head", "lse", "dq", "dv_stride_head",
                                          "scale", "workspace", "workspace_bytes"]),
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "bmattn.h"', 'int main(void) {']
    for cname, (_, fields) in checks.items():
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for f in fields:
            lines.append(f'  printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(l.split() for l in subprocess.run([str(exe)], check=True, capture_output=True,
                                                 text=True).stdout.splitlines())
    for cname, (cls, fields) in checks.items():
        assert int(out[cname]) == ctypes.sizeof(cls), cname
        for f in fields:
            assert int(out[f"{cname}.{f}"]) == getattr(cls, f).offset, (cname, f)


def test_forward_grid_beyond_int32_rejected():
    # 2 sequences x ceil(2^30 / 128) query tiles x 256 heads is more than
    # 2^31 - 1 workgroups: refused on the host, never launched short.
    L = bm.lib()
    d = _desc(mq=1 << 30, mk=100)
    t = _tiles(d)
    a = _args(num_heads=256)
    assert L.bmattn_forward(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t), None) == 2
    assert b"grid" in L.bmattn_last_error()
    a = _args(num_heads=1)
    assert L.bmattn_forward_workspace_size(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t),
                                           ctypes.byref(ctypes.c_size_t())) == 0


# ---- the binding's tensor checks (CPU tensors; no library call is reached) --

def _cpu_case(paged=False, T=40, H=2, D=64):
    import torch
    import synth
    lay = synth.Layout("t", "causal", "bf16", H, D, [T], [T])
    desc = bm.MaskDesc.create("causal", lay.cu_q, lay.cu_k, T, T, device="cpu")
    q = torch.zeros(T, H, D, dtype=torch.bfloat16)
    if paged:
        k = torch.zeros(4, 16, H, D, dtype=torch.bfloat16)
        bt = torch.zeros(1, 3, dtype=torch.int32)
    else:
        k, bt = torch.zeros(T, H, D, dtype=torch.bfloat16), None
    lse = torch.zeros(H, T, dtype=torch.float32)
    return desc, q, k, k.clone(), q.clone(), lse, bt


@pytest.mark.parametrize("bad", ["kshape", "vdtype", "oshape", "lse_dtype", "lse_shape",
                                 "q_inner_stride", "ktokens"])
def test_binding_rejects_bad_tensors(bad):
    import torch
    desc, q, k, v, o, lse, bt = _cpu_case()
    if bad == "kshape":
        k = torch.zeros(40, 1, 64, dtype=torch.bfloat16)  # fewer heads than q (GQA shape)
    elif bad == "vdtype":
        v = v.float()
    elif bad == "oshape":
        o = o[:20]
    elif bad == "lse_dtype":
        lse = lse.double()
    elif bad == "lse_shape":
        lse = lse[:, :10]
    elif bad == "q_inner_stride":
        q = torch.zeros(40, 2, 128, dtype=torch.bfloat16)[:, :, ::2]
    elif bad == "ktokens":
        k = k[:30]
    with pytest.raises(bm.BmattnError) as e:
        bm._check_fwd(q, k, v, o, lse, desc, None, None, None)
    assert e.value.status == 1


@pytest.mark.parametrize("bad", ["int64_table", "short_table", "pool_rank", "vpool_shape"])
def test_binding_rejects_bad_paged_tensors(bad):
    import torch
    desc, q, k, v, o, lse, bt = _cpu_case(paged=True)
    if bad == "int64_table":
        bt = bt.long()  # torch.tensor's default integer type; the kernels read int32
    elif bad == "short_table":
        bt = torch.zeros(0, 3, dtype=torch.int32)
    elif bad == "pool_rank":
        k = k.reshape(64, 2, 64)
    elif bad == "vpool_shape":
        v = torch.zeros(3, 16, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(bm.BmattnError) as e:
        bm._check_fwd(q, k, v, o, lse, desc, None, bt, None)
    assert e.value.status == 1


def test_binding_accepts_consistent_tensors():
    for paged in (False, True):
        desc, q, k, v, o, lse, bt = _cpu_case(paged=paged)
        bm._check_fwd(q, k, v, o, lse, desc, None, bt, None)


@pytest.mark.parametrize("bad", ["dk_shape", "do_dtype", "lse_shape"])
def test_binding_rejects_bad_backward_tensors(bad):
    import torch
    desc, q, k, v, o, lse, _ = _cpu_case()
    do, dq, dk, dv = q.clone(), q.clone(), k.clone(), v.clone()
    if bad == "dk_shape":
        dk = dk[:10]
    elif bad == "do_dtype":
        do = do.float()
    elif bad == "lse_shape":
        lse = lse[:1]
    with pytest.raises(bm.BmattnError) as e:
        bm._check_bwd(q, k, v, o, lse, do, dq, dk, dv, desc, None, None, None)
    assert e.value.status == 1


def test_binding_rejects_wrong_id_lengths():
    import torch
    lay_cu = [0, 40]
    d = bm.MaskDesc.create("shared_prefix", lay_cu, lay_cu, 40, 40, device="cpu",
                           seg_q=[0] * 40, seg_k=[0] * 39)
    with pytest.raises(bm.BmattnError):
        bm._check_desc(d, "forward", torch.device("cpu"))


def test_noalloc_forward_rejected_before_any_device_call():
    # The entry point without allocation refuses a workspace argument and a
    # decode whose split workspace exceeds its static scratch; neither check
    # touches a device.
    L = bm.lib()
    d = _desc(mq=1, tq=2)
    t = _tiles(d, block_m=1, block_n=64)
    a = _args(workspace=FAKE, workspace_bytes=1 << 20)
    assert L.bmattn_forward_noalloc(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t), None) == 1
    assert b"workspace = NULL" in L.bmattn_last_error()
    # 2000 rows x 64 splits x 32 heads x (128 + 2) floats = 2.1 GB > 96 MiB
    d = _desc(n=2000, mq=1, mk=32768, tq=2000, tk=2000 * 32768)
    t = _tiles(d, block_m=1, block_n=64)
    a = _args(num_heads=32)
    assert L.bmattn_forward_noalloc(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t), None) == 5
    assert b"static scratch" in L.bmattn_last_error()
    n = ctypes.c_size_t()
    assert L.bmattn_forward_workspace_size(ctypes.byref(a), ctypes.byref(d), ctypes.byref(t),
                                           ctypes.byref(n)) == 0
    assert n.value > bm.NOALLOC_MAX_WORKSPACE


def test_noalloc_limit_matches_the_header():
    src = open(os.path.join(ROOT, "include", "bmattn.h")).read()
    m = re.search(r"#define BMATTN_NOALLOC_MAX_WORKSPACE \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == bm.NOALLOC_MAX_WORKSPACE
