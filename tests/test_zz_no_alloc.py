"""The allocation-free decode entry point (fp8bq_grouped_gemm_decode_noalloc,
the library's static device scratch as the workspace) through the C ABI,
against the workspace form fp8bq_grouped_gemm_decode_ws with a torch-allocated
workspace: bit-identical outputs on two calls in a row, the second smaller, and
a refused launch when the scratch is too small."""

import numpy as np
import pytest

import fp8_fine_grained_fp8bq_amd as fb
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _operands(seed, counts, n, k):
    import torch
    g = torch.Generator().manual_seed(seed)
    G, m = len(counts), int(sum(counts))
    codes = torch.from_numpy(_CODES)
    a = codes[torch.randint(0, _CODES.size, (m, k), generator=g)].cuda()
    b = codes[torch.randint(0, _CODES.size, (G, n, k), generator=g)].cuda()
    sa = (torch.rand((k // 128, m), generator=g) * 1e-2 + 1e-3).cuda()
    sb = (torch.rand((G, n // 128, k // 128), generator=g) * 1e-2 + 1e-3).cuda()
    return a, sa, b, sb


def _both(seed, counts, n, k):
    import torch
    row_off = [0] + list(np.cumsum(counts))
    G, m = len(counts), int(row_off[-1])
    a, sa, b, sb = _operands(seed, counts, n, k)
    sp = torch.cuda.current_stream().cuda_stream
    need = fb.fp8bq_grouped_gemm_decode_workspace_size(G, row_off, n, k)
    log(f"[noalloc] counts={counts} n={n} k={k} workspace {need} bytes")
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    ref = torch.full((m, n), -1, dtype=torch.int16, device="cuda")
    out = torch.full((m, n), -2, dtype=torch.int16, device="cuda")
    fb.fp8bq_grouped_gemm_decode_ws(G, row_off, n, k, a.data_ptr(), k, sa.data_ptr(), m, b.data_ptr(), k,
                                    sb.data_ptr(), k // 128, ref.data_ptr(), n, ws.data_ptr(), ws.numel(), 0, sp)
    fb.fp8bq_grouped_gemm_decode_noalloc(G, row_off, n, k, a.data_ptr(), k, sa.data_ptr(), m, b.data_ptr(), k,
                                         sb.data_ptr(), k // 128, out.data_ptr(), n, 0, sp)
    torch.cuda.synchronize()
    assert need > 0
    assert torch.equal(out, ref), f"counts {counts}: outputs differ"
    assert not torch.equal(ref, torch.full_like(ref, -1))


def test_noalloc_matches_workspace_form_two_calls():
    # the 256-token decode step's expert sizes, then a smaller call through the same scratch
    _both(201, [217, 179, 120, 93, 75, 57, 69, 43], 2048, 7168)
    _both(202, [100, 40, 33], 256, 1152)


def test_noalloc_without_split_and_oversize():
    import torch
    # experts of at most 32 rows need no scratch
    a, sa, b, sb = _operands(203, [20, 7], 256, 640)
    sp = torch.cuda.current_stream().cuda_stream
    out = torch.empty((27, 256), dtype=torch.int16, device="cuda")
    ref = torch.empty((27, 256), dtype=torch.int16, device="cuda")
    fb.fp8bq_grouped_gemm_decode(2, [0, 20, 27], 256, 640, a.data_ptr(), 640, sa.data_ptr(), 27, b.data_ptr(), 640,
                                 sb.data_ptr(), 5, ref.data_ptr(), 256, 0, sp)
    fb.fp8bq_grouped_gemm_decode_noalloc(2, [0, 20, 27], 256, 640, a.data_ptr(), 640, sa.data_ptr(), 27,
                                         b.data_ptr(), 640, sb.data_ptr(), 5, out.data_ptr(), 256, 0, sp)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    # 8 experts of 256 rows at n = 4096 need 64 MiB of partial sums: refused before any launch
    with pytest.raises(fb.Fp8bqError, match="scratch"):
        fb.fp8bq_grouped_gemm_decode_noalloc(8, [256 * e for e in range(9)], 4096, 7168, a.data_ptr(), 7168,
                                             sa.data_ptr(), 2048, b.data_ptr(), 7168, sb.data_ptr(), 56,
                                             out.data_ptr(), 4096, 0, sp)


def test_noalloc_replays_in_a_captured_graph():
    # the use it is for: captured once in a HIP graph (the first call, which
    # takes the scratch's address, runs eagerly before the capture), replayed
    # with eager work and synchronisations between replays; every replay must
    # equal the eager result (the counters reset themselves, nothing is cleared
    # by a memset node)
    import torch
    counts = [120, 75, 43, 10]
    row_off = [0] + list(np.cumsum(counts))
    G, m, n, k = len(counts), int(row_off[-1]), 512, 1536
    a, sa, b, sb = _operands(204, counts, n, k)
    out = torch.empty((m, n), dtype=torch.int16, device="cuda")
    ref = torch.empty_like(out)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fb.fp8bq_grouped_gemm_decode_noalloc(G, row_off, n, k, a.data_ptr(), k, sa.data_ptr(), m, b.data_ptr(), k,
                                             sb.data_ptr(), k // 128, ref.data_ptr(), n, 0, s.cuda_stream)
    s.synchronize()
    log(f"[noalloc] graph capture, counts={counts}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fb.fp8bq_grouped_gemm_decode_noalloc(G, row_off, n, k, a.data_ptr(), k, sa.data_ptr(), m, b.data_ptr(), k,
                                             sb.data_ptr(), k // 128, out.data_ptr(), n, 0,
                                             torch.cuda.current_stream().cuda_stream)
    for i in range(4):
        out.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager result"
        # eager work on the same scratch between replays
        fb.fp8bq_grouped_gemm_decode_noalloc(G, row_off, n, k, a.data_ptr(), k, sa.data_ptr(), m, b.data_ptr(), k,
                                             sb.data_ptr(), k // 128, out.data_ptr(), n, 0,
                                             torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"eager call after replay {i} differs"
