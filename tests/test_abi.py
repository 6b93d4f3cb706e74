"""The C-ABI library: it loads, exports every entry point of include/dsa.h, and
its host-side validation answers with the documented status codes without
touching a device (no GPU is needed for any test here)."""
import ctypes as C
import os
import re

import pytest

import sparse_attention_dsa_amd as dsa
from sparse_attention_dsa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return dsa.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, text in [(0, b"ok"), (-1, b"invalid argument"), (-3, b"workspace too small"),
                       (-4, b"current device is not gfx950"), (7, b"unknown status")]:
        assert L.dsa_status_string(code) == text


def _batch(B_=2, T=2, maxq=1, maxctx=1000, bs=64, maxblocks=16):
    # device pointers are never dereferenced by the host checks: any non-null value works
    return B.DsaBatch(B_, T, maxq, maxctx, 0x1000, 0x2000, 0x3000, maxblocks, bs)


def test_workspace_size_host_only(L):
    b = _batch()
    assert L.dsa_workspace_size(B.OP_TOPK, C.byref(b), 2048, 0) == 0     # rows too short to need slots
    long_ = _batch(maxctx=100000, maxblocks=1600)
    ws_topk = L.dsa_workspace_size(B.OP_TOPK, C.byref(long_), 2048, 0)
    assert ws_topk >= 2 * 13 * 4096 * 8                # 13 chunks of candidate slots per row
    assert L.dsa_workspace_size(B.OP_TOPK, C.byref(long_), 0, 0) == 0
    assert L.dsa_workspace_size(B.OP_TOPK, C.byref(long_), 5000, 0) == 0
    assert L.dsa_workspace_size(99, C.byref(b), 16, 0) == 0
    step = L.dsa_workspace_size(B.OP_DECODE_STEP, C.byref(long_), 2048, 128)
    assert step >= 2 * 100000 * 4 + 2 * 2048 * 4 + ws_topk     # scores + indices + candidate slots
    bad = _batch(maxctx=5000)                   # 16 blocks * 64 < 5000
    assert L.dsa_workspace_size(B.OP_TOPK, C.byref(bad), 16, 0) == 0


def test_invalid_arguments_rejected_before_device(L):
    b = _batch()
    ic = B.DsaIndexCache(0x10, None, B.E4M3, 128)
    assert L.dsa_indexer_scores(None, C.byref(ic), 0x1, 0x1, 64, 0x1, 1024, None) == -1
    assert L.dsa_indexer_scores(C.byref(b), C.byref(ic), None, 0x1, 64, 0x1, 1024, None) == -1
    assert L.dsa_indexer_scores(C.byref(b), C.byref(ic), 0x1, 0x1, 64, 0x1, 10, None) == -1  # ld < ctx
    bad_dt = B.DsaIndexCache(0x10, None, B.BF16, 128)
    assert L.dsa_indexer_scores(C.byref(b), C.byref(bad_dt), 0x1, 0x1, 64, 0x1, 1024, None) == -2
    bad_f4 = B.DsaIndexCache(0x10, None, B.DSA_MXFP4, 48)   # MXFP4 blocks of 32 need dim % 32 == 0
    assert L.dsa_indexer_scores(C.byref(b), C.byref(bad_f4), 0x1, 0x1, 64, 0x1, 1024, None) == -2
    assert L.dsa_topk(C.byref(b), 0x1, 1024, 0, 0x1, 0x1, 1 << 30, None) == -1
    assert L.dsa_topk(C.byref(b), 0x1, 1024, 5000, 0x1, 0x1, 1 << 30, None) == -2
    assert L.dsa_topk(C.byref(long_b := _batch(maxctx=100000, maxblocks=1600)), 0x1, 100000, 16, 0x1, 0x1, 8,
                      None) == -3                   # workspace too small
    lc = B.DsaLatentCache(0x10, None, B.E4M3, 512, 64)      # fp8 latent needs scales
    assert L.dsa_sparse_mla_decode(C.byref(b), C.byref(lc), 0x1, 128, 0x1, 2048, 0.1, 0x1, None,
                                   0x1, 1 << 30, None) == -2
    lc_ok = B.DsaLatentCache(0x10, None, B.BF16, 512, 64)
    assert L.dsa_sparse_mla_decode(C.byref(b), C.byref(lc_ok), 0x1, 128, None, 2048, 0.1, 0x1, None,
                                   0x1, 1 << 30, None) == -1
    assert L.dsa_sparse_mla_decode(C.byref(b), C.byref(lc_ok), 0x1, 128, 0x1, 2048, 0.1, 0x1, None,
                                   0x1, 16, None) == -3
    # the measurement variant of the decode step: too few or null event handles
    ev = (C.c_void_p * 5)(*[C.c_void_p(0x100 + i) for i in range(5)])
    args = (C.byref(b), C.byref(ic), 0x1, 0x1, 64, C.byref(lc_ok), 0x1, 128, 2048, 0.1, 0x1, None, None, 0x1,
            1 << 30, None)
    assert L.dsa_decode_step_timed(*args, ev, 4) == -1
    assert L.dsa_decode_step_timed(*args, None, 5) == -1
    ev_null = (C.c_void_p * 5)(0x100, 0x101, None, 0x103, 0x104)
    assert L.dsa_decode_step_timed(*args, ev_null, 5) == -1
    # the read-bandwidth probe: null or misaligned buffer, size not a multiple of 16, null sink
    assert L.dsa_read_probe(None, 1024, 0x100, 1 << 20, None) == -1
    assert L.dsa_read_probe(0x108, 1024, 0x100, 1 << 20, None) == -1
    assert L.dsa_read_probe(0x100, 1000, 0x100, 1 << 20, None) == -1
    assert L.dsa_read_probe(0x100, 1024, None, 1 << 20, None) == -1
    # the random-page probe: null pointers, page size not a multiple of 1 KB or
    # above 8 KB, scale size above 256 or not a multiple of 4, scales missing,
    # misaligned pools, negative count
    pp = L.dsa_page_probe
    assert pp(None, 8192, 0x100, 256, 0x200, 10, 0x300, 1 << 20, None) == -1
    assert pp(0x100, 8192, 0x100, 256, None, 10, 0x300, 1 << 20, None) == -1
    assert pp(0x100, 8192, 0x100, 256, 0x200, 10, None, 1 << 20, None) == -1
    assert pp(0x100, 8000, 0x100, 256, 0x200, 10, 0x300, 1 << 20, None) == -1
    assert pp(0x100, 9216, 0x100, 256, 0x200, 10, 0x300, 1 << 20, None) == -1
    assert pp(0x100, 8192, 0x100, 260, 0x200, 10, 0x300, 1 << 20, None) == -1
    assert pp(0x100, 8192, 0x100, 6, 0x200, 10, 0x300, 1 << 20, None) == -1
    # the row-gather probe: null pointers, misaligned pool, row size not a
    # multiple of 128 or above 1152, rows per workgroup not a multiple of 32
    # or not dividing the count
    rp = L.dsa_row_probe
    assert rp(None, 1152, 0x200, 512, 256, 0x300, 1 << 20, None) == -1
    assert rp(0x100, 1152, None, 512, 256, 0x300, 1 << 20, None) == -1
    assert rp(0x100, 1152, 0x200, 512, 256, None, 1 << 20, None) == -1
    assert rp(0x108, 1152, 0x200, 512, 256, 0x300, 1 << 20, None) == -1
    assert rp(0x100, 1000, 0x200, 512, 256, 0x300, 1 << 20, None) == -1
    assert rp(0x100, 1280, 0x200, 512, 256, 0x300, 1 << 20, None) == -1
    assert rp(0x100, 1152, 0x200, 512, 48, 0x300, 1 << 20, None) == -1
    assert rp(0x100, 1152, 0x200, 500, 256, 0x300, 1 << 20, None) == -1
    assert L.dsa_row_probe_sink_size(512, 256) == 8
    assert pp(0x100, 8192, None, 256, 0x200, 10, 0x300, 1 << 20, None) == -1
    assert pp(0x108, 8192, 0x100, 256, 0x200, 10, 0x300, 1 << 20, None) == -1
    assert pp(0x100, 8192, 0x102, 256, 0x200, 10, 0x300, 1 << 20, None) == -1
    assert pp(0x100, 8192, 0x100, 256, 0x200, -1, 0x300, 1 << 20, None) == -1


def test_hot_cache_arguments_rejected_before_device(L):
    b = _batch(T=2)
    assert L.dsa_hot_cache_workspace_size(None, 16, 64) == 0
    assert L.dsa_hot_cache_workspace_size(C.byref(b), 0, 64) == 0
    assert L.dsa_hot_cache_workspace_size(C.byref(b), 16, 0) == 0
    small = L.dsa_hot_cache_workspace_size(C.byref(b), 16, 64)
    assert 0 < small < L.dsa_hot_cache_workspace_size(C.byref(b), 16, 1 << 20)   # grows with the hot set
    hot = B.DsaHotCache(0x100, None, 64, 0x200, 0x300, 0x400, 0x500)
    bf = B.DsaLatentCache(0x10, None, B.BF16, 512, 64)
    ws = 1 << 30
    assert L.dsa_hot_cache_reset(C.byref(b), None, None) == -1
    no_clock = B.DsaHotCache(0x100, None, 64, 0x200, 0x300, 0x400, None)
    assert L.dsa_hot_cache_reset(C.byref(b), C.byref(no_clock), None) == -1
    assert L.dsa_hot_cache_fetch(C.byref(b), C.byref(bf), None, 16, C.byref(hot), None, 0x1, ws, None) == -1
    assert L.dsa_hot_cache_fetch(C.byref(b), C.byref(bf), 0x1, 33, C.byref(hot), None, 0x1, ws, None) == -1  # 2 x 33 > 64 slots
    odd = B.DsaLatentCache(0x10, None, B.BF16, 7, 0)                           # 14-byte rows
    assert L.dsa_hot_cache_fetch(C.byref(b), C.byref(odd), 0x1, 16, C.byref(hot), None, 0x1, ws, None) == -2
    wide = B.DsaLatentCache(0x10, None, B.F32, 512, 64)                        # 2304-byte rows
    assert L.dsa_hot_cache_fetch(C.byref(b), C.byref(wide), 0x1, 16, C.byref(hot), None, 0x1, ws, None) == -2
    fp8 = B.DsaLatentCache(0x10, 0x20, B.E4M3, 512, 64)                        # hot set without scales
    assert L.dsa_hot_cache_fetch(C.byref(b), C.byref(fp8), 0x1, 16, C.byref(hot), None, 0x1, ws, None) == -2
    assert L.dsa_hot_cache_fetch(C.byref(b), C.byref(bf), 0x1, 16, C.byref(hot), None, 0x1, small - 1, None) == -3


def test_valid_call_without_gpu_reports_device(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    b = _batch()
    ic = B.DsaIndexCache(0x10, None, B.E4M3, 128)
    assert L.dsa_indexer_scores(C.byref(b), C.byref(ic), 0x1, 0x1, 64, 0x1, 1024, None) == -4
    assert L.dsa_check_device() == -4
    hot = B.DsaHotCache(0x100, None, 64, 0x200, 0x300, 0x400, 0x500)
    bf = B.DsaLatentCache(0x10, None, B.BF16, 512, 64)
    assert L.dsa_hot_cache_reset(C.byref(b), C.byref(hot), None) == -4
    assert L.dsa_hot_cache_fetch(C.byref(b), C.byref(bf), 0x1, 16, C.byref(hot), None, 0x1, 1 << 30, None) == -4
    assert L.dsa_read_probe(0x100, 1024, 0x100, 1 << 20, None) == -4
    assert L.dsa_page_probe(0x100, 8192, None, 0, 0x200, 10, 0x300, 1 << 20, None) == -4
    assert L.dsa_row_probe(0x100, 1152, 0x200, 512, 256, 0x300, 1 << 20, None) == -4


def test_noalloc_rejects_batches_beyond_its_scratch(L):
    """The no-allocation entry point refuses a batch whose workspace would not
    fit its built-in scratch, before touching a device."""
    ic = B.DsaIndexCache(0x10, 0x20, B.E4M3, 128)
    lc = B.DsaLatentCache(0x10, None, B.BF16, 512, 64)
    huge = _batch(B_=64, T=64, maxctx=1 << 20, maxblocks=(1 << 20) // 64)
    st = L.dsa_decode_step_noalloc(C.byref(huge), C.byref(ic), 0x1, 0x1, 64, C.byref(lc), 0x1, 128, 2048,
                                   0.04, 0x1, None, None, None)
    assert st == -6
    assert L.dsa_status_string(-6).startswith(b"batch needs more than")
    assert L.dsa_workspace_size(B.OP_DECODE_STEP, C.byref(huge), 2048, 128) > (128 << 20)


def test_check_batch_host_arguments(L):
    b = _batch()
    failed = C.c_uint32(99)
    assert L.dsa_check_batch(None, 0, None, 0, C.byref(failed), None) == -1
    assert failed.value == 0
    assert L.dsa_check_batch(C.byref(b), 0, 0x1, 0, None, None) == -1      # indices without k
    assert L.dsa_check_batch(C.byref(_batch(maxctx=5000)), 0, None, 0, None, None) == -1   # pages cannot hold it
    assert L.dsa_status_string(-7) == b"a device-side size, page id or index is out of range"


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes structures have the sizes and field offsets that a C
    compiler gives the header's structs."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    structs = {"dsa_batch": B.DsaBatch, "dsa_index_cache": B.DsaIndexCache,
               "dsa_latent_cache": B.DsaLatentCache, "dsa_hot_cache": B.DsaHotCache}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "dsa.h"', "int main(void) {"]
    for name, cls in structs.items():
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (name, name))
        for f, _ in cls._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (name, f, name, f))
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = str(tmp_path / "layout")
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", exe], check=True)
    got = dict(l.split() for l in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
               if l)
    for name, cls in structs.items():
        assert int(got[name]) == C.sizeof(cls), name
        for f, _ in cls._fields_:
            assert int(got["%s.%s" % (name, f)]) == getattr(cls, f).offset, (name, f)


def test_hot_cache_plan_and_copy_host_checks(L):
    b = _batch()
    bf = B.DsaLatentCache(0x10, None, B.BF16, 512, 64)
    hot = B.DsaHotCache(0x100, None, 64, 0x200, 0x300, 0x400, 0x500)
    assert L.dsa_hot_cache_plan(C.byref(b), C.byref(bf), None, 16, C.byref(hot), 0x1, 1 << 30, None) == -1
    assert L.dsa_hot_cache_copy(C.byref(b), C.byref(bf), 0x1, 33, C.byref(hot), None, 0x1, 1 << 30, None) == -1
    assert L.dsa_hot_cache_plan(C.byref(b), C.byref(bf), 0x1, 16, C.byref(hot), 0x1, 8, None) == -3


def test_mla_decode_layers_host_checks(L):
    b = _batch()
    caches = (B.DsaLatentCache * 2)(B.DsaLatentCache(0x10, None, B.BF16, 512, 64),
                                   B.DsaLatentCache(0x20, None, B.BF16, 512, 64))
    ptrs = (C.c_void_p * 2)(0x100, 0x200)
    args = lambda n, c=caches, q=ptrs, o=ptrs: (C.byref(b), c, n, q, 128, 0x1, 2048, 0.1, o, None, 0x1, 1 << 30, None)
    assert L.dsa_sparse_mla_decode_layers(*args(0)) == -1
    assert L.dsa_sparse_mla_decode_layers(*args(5)) == -1
    assert L.dsa_sparse_mla_decode_layers(*args(2, q=None)) == -1
    mixed = (B.DsaLatentCache * 2)(B.DsaLatentCache(0x10, None, B.BF16, 512, 64),
                                  B.DsaLatentCache(0x20, None, B.F32, 512, 64))
    assert L.dsa_sparse_mla_decode_layers(*args(2, c=mixed)) == -2
    small = (C.byref(b), caches, 2, ptrs, 128, 0x1, 2048, 0.1, ptrs, None, 0x1, 16, None)
    assert L.dsa_sparse_mla_decode_layers(*small) == -3
