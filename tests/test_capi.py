"""CPU checks of the C ABI: the built library loads and exports every
function include/*.h declares, and host-side argument validation rejects
bad calls before anything reaches the GPU (no kernel is launched here)."""
import ctypes
import glob
import os
import re

import pytest

from mla_tree_verify_parents_amd import build, ddt

HEADERS = sorted(glob.glob(os.path.join(build.ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(ddt_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.LIB):
        build.build()
    return ddt.lib()


def test_header_declares_the_path():
    names = declared_functions()
    for f in ("ddt_build_mask", "ddt_verify_attn", "ddt_verify_workspace", "ddt_argmax",
              "ddt_argmax_workspace", "ddt_greedy_accept", "ddt_compact_kv"):
        assert f in names


def test_headers_found():
    assert {os.path.basename(h) for h in HEADERS} >= {"ddt.h", "ddt_probe.h"}
    assert "ddt_probe_mfma_bf16" in declared_functions()


def test_every_declared_symbol_is_exported(lib):
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing, missing


def test_version_and_status_strings(lib):
    assert lib.ddt_version() >= 100
    assert b"EINVAL" in lib.ddt_status_string(-1)
    assert b"OK" in lib.ddt_status_string(0)


def test_host_side_validation(lib):
    null = None
    # N out of range / negative B: rejected before any launch
    assert lib.ddt_build_mask(null, 1, 0, null, null, null, null) == -1
    assert lib.ddt_build_mask(null, 1, 1025, null, null, null, null) == -1
    assert lib.ddt_build_mask(null, -1, 4, null, null, null, null) == -1
    assert lib.ddt_build_mask(null, 0, 4, null, null, null, null) == 0      # nothing to do
    assert lib.ddt_greedy_accept(null, null, null, 2, 0, null, null, null, null) == -1
    assert lib.ddt_argmax(null, 0, 4, 10, 5, null, null, 0, null) == -1     # ld < V
    assert lib.ddt_argmax(null, 7, 4, 10, 10, null, null, 0, null) == -2    # dtype
    assert lib.ddt_compact_kv(null, 576, null, 576, 1, 512, 64, null, null, null, null, 1, 0, null, null) == -1
    assert lib.ddt_accept_compact(null, null, null, 1, 0, null, null, null, null, 576, null, 576, 1, 512, 64,
                                  null, null, null, null, null) == -1              # N < 1
    assert lib.ddt_accept_compact(null, null, null, 1, 8, null, null, null, null, 576, null, 576, 1, 512, 64,
                                  null, null, null, null, null) == -1              # null pointers
    assert lib.ddt_accept_compact(null, null, null, 0, 8, null, null, null, null, 576, null, 576, 1, 512, 64,
                                  null, null, null, null, null) == 0               # nothing to do
    d = ddt.AttnDesc(1, 8, 64, 512, 64, ddt.DDT_BF16, 0.04, 0, 576, 576, 576, 576)
    pl = (ctypes.c_int32 * 1)(100)
    n = ctypes.c_size_t(0)
    bad = ddt.AttnDesc(1, 8, 64, 256, 64, ddt.DDT_BF16, 0.04, 0, 576, 576, 576, 576)
    assert lib.ddt_verify_workspace(ctypes.byref(bad), pl, ctypes.byref(n)) == -2   # not built
    bad = ddt.AttnDesc(1, 8, 64, 512, 64, ddt.DDT_BF16, 0.04, 0, 577, 576, 576, 576)
    assert lib.ddt_verify_workspace(ctypes.byref(bad), pl, ctypes.byref(n)) == -1   # stride alignment
    bad = ddt.AttnDesc(1, 8, 64, 512, 64, ddt.DDT_BF16, 0.04, 0, 576, 576, 1 << 30, 576)
    assert lib.ddt_verify_workspace(ctypes.byref(bad), pl, ctypes.byref(n)) == -1   # 2 GiB cache rows
    bad = ddt.AttnDesc(129, 8, 64, 512, 64, ddt.DDT_BF16, 0.04, 0, 576, 576, 576, 576)
    assert lib.ddt_verify_workspace(ctypes.byref(bad), pl, ctypes.byref(n)) == -1   # batch limit
    for scale in (0.0, -0.04, float("inf"), float("nan")):                         # scale must be > 0
        bad = ddt.AttnDesc(1, 8, 64, 512, 64, ddt.DDT_BF16, scale, 0, 576, 576, 576, 576)
        assert lib.ddt_verify_workspace(ctypes.byref(bad), pl, ctypes.byref(n)) == -1, scale
    assert lib.ddt_verify_workspace(ctypes.byref(d), pl, ctypes.byref(n)) == 0
    assert lib.ddt_verify_attn(ctypes.byref(d), null, null, null, null, null, pl, null, null, null,
                               null, 0, null) == -1
    # every other pointer set (never dereferenced): no kv_base and no block table is rejected
    f = ctypes.c_void_p(1 << 20)
    assert lib.ddt_verify_attn(ctypes.byref(d), f, f, f, f, null, pl, f, f, f, f, 1 << 30, null) == -1


def test_noalloc_validation(lib):
    """ddt_verify_attn_noalloc: its scratch size, and the host-side refusals
    that come before any device call (placeholder pointers, never
    dereferenced)."""
    assert lib.ddt_verify_noalloc_scratch_bytes() == 64 << 20
    null = None
    pl = (ctypes.c_int32 * 1)(100)
    assert lib.ddt_verify_attn_noalloc(null, null, null, null, null, null, pl, null, null, null, null) == -1
    bad = ddt.AttnDesc(1, 8, 64, 256, 64, ddt.DDT_BF16, 0.04, 0, 576, 576, 576, 576)
    f = ctypes.c_void_p(1 << 20)
    assert lib.ddt_verify_attn_noalloc(ctypes.byref(bad), f, f, f, f, f, pl, f, f, f, null) == -2   # not built
    # 32 requests x 5 splits x 8 row tiles of fp32 partials (160 MiB): beyond the scratch
    P = (ctypes.c_int32 * 32)(*([1024] * 32))
    d = ddt.AttnDesc(32, 8, 64, 512, 64, ddt.DDT_BF16, 0.04, 256, 576, 576, 576, 576)
    n = ctypes.c_size_t(0)
    assert lib.ddt_verify_workspace(ctypes.byref(d), P, ctypes.byref(n)) == 0 and n.value > 64 << 20
    assert lib.ddt_verify_attn_noalloc(ctypes.byref(d), f, f, f, f, f, P, f, f, f, null) == -3


def test_verify_step_validation(lib):
    """ddt_verify_step rejects a missing or mismatched argmax task and a
    missing acceptance output before launching.  The device pointers are
    placeholders that are never dereferenced: every call fails validation."""
    fake = ctypes.c_void_p(1 << 16)
    d = ddt.AttnDesc(1, 8, 64, 512, 64, ddt.DDT_BF16, 0.04, 0, 576, 576, 576, 576)
    pl = (ctypes.c_int32 * 1)(100)
    args = (ctypes.byref(d), fake, fake, fake, fake, fake, pl, fake, fake, fake, fake, 1 << 30)
    good_am = ddt.ArgmaxTask(fake, ddt.DDT_F32, 64, 1000, 1000, fake, fake, 1 << 30)
    good_acc = ddt.AcceptTask(fake, fake, fake, fake, fake, fake, fake, None)
    assert lib.ddt_verify_step(*args, None, ctypes.byref(good_acc), None) == -1            # no argmax task
    assert lib.ddt_verify_step(*args, ctypes.byref(good_am), None, None) == -1             # no acceptance task
    rows63 = ddt.ArgmaxTask(fake, ddt.DDT_F32, 63, 1000, 1000, fake, fake, 1 << 30)
    assert lib.ddt_verify_step(*args, ctypes.byref(rows63), ctypes.byref(good_acc), None) == -1  # rows != B*N
    for k in range(7):                                                                    # each output needed
        f = [fake] * 7
        f[k] = None
        acc = ddt.AcceptTask(*f, None)
        assert lib.ddt_verify_step(*args, ctypes.byref(good_am), ctypes.byref(acc), None) == -1, k



def test_draft_validation(lib):
    n = ctypes.c_size_t(0)
    assert lib.ddt_draft_topk_workspace(256, 163840, 8, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.ddt_draft_topk_workspace(4, 100, 0, ctypes.byref(n)) == -1          # K < 1
    assert lib.ddt_draft_topk_workspace(4, 100, 17, ctypes.byref(n)) == -1         # K > 16
    assert lib.ddt_draft_topk_workspace(4, 5, 8, ctypes.byref(n)) == -1            # K > V
    assert lib.ddt_draft_topk_workspace(4, (1 << 20) + 1, 8, ctypes.byref(n)) == -1  # V > 2^20
    assert lib.ddt_draft_topk(None, 4, 100, 99, 4, None, None, None, 0, None) == -1  # ld < V
    assert lib.ddt_draft_topk(None, 0, 100, 100, 4, None, None, None, 0, None) == 0  # nothing to do
    # tree: the candidates must suffice, sizes in range
    assert lib.ddt_best_first_tree(None, None, 1, 2, 2, 7, None, None, None, None, None) == -1  # 6 candidates
    assert lib.ddt_best_first_tree(None, None, 0, 2, 2, 6, None, None, None, None, None) == 0   # B = 0
    assert lib.ddt_best_first_tree(None, None, 1, 0, 2, 1, None, None, None, None, None) == -1  # D < 1
    assert lib.ddt_best_first_tree(None, None, 1, 8, 8, 1024, None, None, None, None, None) == -1  # budget + 1 > 1024
    assert lib.ddt_best_first_tree(None, None, 1, 64, 65, 10, None, None, None, None, None) == -1  # D*K > 4096
    assert lib.ddt_best_first_tree(None, None, 1, 8, 8, 63, None, None, None, None, None) == -1   # null pointers


def test_paged_desc_validation(lib):
    """Block-table fields of ddt_attn_desc, checked on the host (no launch)."""
    from mla_tree_verify_parents_amd import ddt
    P = (ctypes.c_int * 2)(100, 3000)
    n = ctypes.c_size_t(0)

    def desc(page_size, bt_ld, table=1 << 20):
        d = ddt.AttnDesc(2, 8, 32, 512, 64, 1, 1 / 24, 0, 576, 576, 576, 576)
        d.block_table, d.bt_ld, d.page_size = table, bt_ld, page_size
        return ctypes.byref(d)
    assert lib.ddt_verify_workspace(desc(64, 48), P, ctypes.byref(n)) == 0      # ceil(3032/64) = 48 pages
    assert lib.ddt_verify_workspace(desc(64, 47), P, ctypes.byref(n)) == -1     # table row too short
    assert lib.ddt_verify_workspace(desc(48, 100), P, ctypes.byref(n)) == -1    # not a power of two
    assert lib.ddt_verify_workspace(desc(16, 400), P, ctypes.byref(n)) == -1    # smaller than a key tile
    assert lib.ddt_verify_workspace(desc(1 << 17, 1), P, ctypes.byref(n)) == -1  # larger than 65536
    assert lib.ddt_verify_workspace(desc(0, 0, table=None), P, ctypes.byref(n)) == 0  # contiguous
    big = ddt.AttnDesc(2, 8, 32, 512, 64, 1, 1 / 24, 0, 576, 576, 1 << 15, 576)  # 64 KiB rows
    big.block_table, big.bt_ld, big.page_size = 1 << 20, 100, 1 << 16          # 4 GiB pages
    assert lib.ddt_verify_workspace(ctypes.byref(big), P, ctypes.byref(n)) == -1
    big.page_size, big.bt_ld = 1 << 15, 100                                     # 2 GiB pages
    assert lib.ddt_verify_workspace(ctypes.byref(big), P, ctypes.byref(n)) == 0
    d = ddt.AttnDesc(2, 2, 8, 64, 16, 0, 0.1, 0, 80, 80, 80, 80)                 # fp32 (64, 16) instance
    d.block_table, d.bt_ld, d.page_size = 1 << 20, 100, 32
    assert lib.ddt_verify_workspace(ctypes.byref(d), P, ctypes.byref(n)) == -2  # paged: bf16 instance only


def test_compact_paged_validation(lib):
    f = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails validation or has B = 0
    null = None
    args = lambda ps, bt_ld, B=1, table=f: (f, 576, f, 576, 1, 512, 64, table, bt_ld, ps, f, f, f, B, 8, null, null)
    assert lib.ddt_compact_kv_paged(*args(48, 10)) == -1          # page size not a power of two
    assert lib.ddt_compact_kv_paged(*args(1 << 17, 10)) == -1     # page size too large
    assert lib.ddt_compact_kv_paged(*args(64, 0)) == -1           # bt_ld < 1
    assert lib.ddt_compact_kv_paged(*args(64, 10, table=null)) == -1
    assert lib.ddt_compact_kv_paged(*args(64, 10, B=0)) == 0       # nothing to do
    # acceptance + compaction on a paged cache: the same table checks
    acp = lambda ps, bt_ld, B=1, table=f, N=8: (f, f, f, B, N, f, f, f, f, 576, f, 576, 1, 512, 64, table, bt_ld, ps,
                                                 f, f, null, null)
    assert lib.ddt_accept_compact_paged(*acp(48, 10)) == -1
    assert lib.ddt_accept_compact_paged(*acp(64, 0)) == -1
    assert lib.ddt_accept_compact_paged(*acp(64, 10, table=null)) == -1
    assert lib.ddt_accept_compact_paged(*acp(64, 10, N=0)) == -1
    assert lib.ddt_accept_compact_paged(*acp(64, 10, B=0)) == 0


def test_proj_validation(lib):
    a, b, c = ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20), ctypes.c_void_p(3 << 20)  # never dereferenced
    null = None
    # pack: shapes, dtype, aliasing
    assert lib.ddt_proj_pack_weight(a, 8, 96, 512, 1, b, null) == -1        # K not built in
    assert lib.ddt_proj_pack_weight(a, 8, 128, 500, 1, b, null) == -1       # n_out % 32
    assert lib.ddt_proj_pack_weight(a, 0, 128, 512, 1, b, null) == -1       # H < 1
    assert lib.ddt_proj_pack_weight(a, 8, 128, 512, 0, b, null) == -2       # fp32 not built in
    assert lib.ddt_proj_pack_weight(a, 8, 128, 512, 1, a, null) == -1       # in place
    assert lib.ddt_proj_pack_weight(null, 8, 128, 512, 1, b, null) == -1
    # projection: strides, alignment, overlap; M = 0 is a no-op
    assert lib.ddt_head_proj(a, 128, b, 0, 8, 128, 512, 1, c, 576, null) == 0
    assert lib.ddt_head_proj(a, 127, b, 0, 8, 128, 512, 1, c, 576, null) == -1   # ld_x < K
    assert lib.ddt_head_proj(a, 130, b, 0, 8, 128, 512, 1, c, 576, null) == -1   # ld_x % 8
    assert lib.ddt_head_proj(a, 128, b, 0, 8, 128, 512, 1, c, 500, null) == -1   # ld_y < n_out
    assert lib.ddt_head_proj(ctypes.c_void_p((1 << 20) + 8), 128, b, 4, 8, 128, 512, 1, c, 576, null) == -1
    assert lib.ddt_head_proj(a, 128, b, 4, 8, 128, 512, 1, ctypes.c_void_p((1 << 20) + 4096), 576, null) == -1
    assert lib.ddt_head_proj(a, 128, b, 4, 8, 128, 512, 0, c, 576, null) == -2   # fp32 not built in
    assert lib.ddt_head_proj(a, 128, b, -1, 8, 128, 512, 1, c, 576, null) == -1
    assert lib.ddt_head_proj(null, 128, b, 0, 8, 128, 512, 1, null, 576, null) == 0   # M = 0: untouched
    assert lib.ddt_head_proj(null, 128, b, 1, 8, 128, 512, 1, c, 576, null) == -1


def test_probe_validation(lib):
    null = None
    one = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
    assert lib.ddt_probe_mfma_bf16(null, one, null, 1, 1, null) == -1     # null operands
    assert lib.ddt_probe_mfma_bf16(one, one, null, 0, 1, null) == -1      # no workgroups
    assert lib.ddt_probe_mfma_bf16(one, one, null, 1, 0, null) == -1      # no iterations
    assert lib.ddt_probe_read(one, 24, one, 1, null) == -1                # not a multiple of 16
    assert lib.ddt_probe_read(one, 0, one, 1, null) == -1
    assert lib.ddt_probe_copy(one, ctypes.c_void_p(32), 64, 1, null) == -1  # overlapping ranges
    assert lib.ddt_probe_copy(one, null, 64, 1, null) == -1
