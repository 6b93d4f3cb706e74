"""The measurement probes read exactly what they are given: the XOR of the
random-page probe's sink equals the XOR of every word of the listed pages and
their scales (a list with repeats and a count that leaves waves empty), and
each word of the row-gather probe's sink the XOR of its workgroup's rows."""
import numpy as np
import pytest
import torch

from sparse_attention_dsa_amd import binding as B

pytestmark = pytest.mark.gpu


def _xor(a):
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(a).view(np.uint32).ravel(), initial=np.uint32(0)))


@pytest.mark.parametrize("page_bytes,scale_bytes,n", [(8192, 256, 700), (4096, 0, 37), (1024, 4, 5000)])
def test_page_probe_reads_the_listed_pages(page_bytes, scale_bytes, n):
    rng = np.random.default_rng(page_bytes + n)
    pool = 900
    pages = rng.integers(0, 256, size=(pool, page_bytes), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(pool, max(scale_bytes, 4)), dtype=np.uint8)
    ids = rng.integers(0, pool, size=n).astype(np.int32)
    print("page probe", page_bytes, scale_bytes, n, flush=True)
    sink = B.page_probe(torch.from_numpy(pages).cuda(), page_bytes,
                        torch.from_numpy(scales).cuda() if scale_bytes else None, scale_bytes,
                        torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    want = _xor(pages[ids])
    if scale_bytes:
        want ^= _xor(scales[ids, :scale_bytes])
    assert _xor(sink.cpu().numpy()) == want


@pytest.mark.parametrize("row_bytes,rows_per_wg,n", [(1152, 512, 4096), (1152, 32, 96), (128, 64, 640), (640, 96, 288)])
def test_row_probe_reads_the_listed_rows(row_bytes, rows_per_wg, n):
    rng = np.random.default_rng(row_bytes + n)
    pool = 3000
    rows = rng.integers(0, 256, size=(pool, row_bytes), dtype=np.uint8)
    ids = rng.integers(0, pool, size=n).astype(np.int32)
    print("row probe", row_bytes, rows_per_wg, n, flush=True)
    sink = B.row_probe(torch.from_numpy(rows).cuda(), row_bytes, torch.from_numpy(ids).cuda(), rows_per_wg)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    for w in range(n // rows_per_wg):
        assert int(got[w]) == _xor(rows[ids[w * rows_per_wg:(w + 1) * rows_per_wg]]), "workgroup %d" % w


def test_read_probe_reads_the_buffer():
    rng = np.random.default_rng(5)
    buf = rng.integers(0, 256, size=(1 << 20) + 48, dtype=np.uint8)
    sink = B.read_probe(torch.from_numpy(buf).cuda())
    torch.cuda.synchronize()
    words = int(B.lib().dsa_read_probe_sink_size()) // 4
    assert _xor(sink.cpu().numpy()[: 4 * words]) == _xor(buf)
