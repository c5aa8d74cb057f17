"""svdq_quantize_act_noalloc (the activation pass with the library's fixed
device scratch instead of a caller workspace) against svdq_quantize_act
given a workspace, through the C-ABI: two calls in a row on the scratch, the
second on a smaller input, each byte-identical to the workspace path (same
kernels, same split of K) and its codes and scales equal to the oracle's."""

import numpy as np
import pytest

from bit_quantized_linear_amd import binding as b
from oracle import svdquant as sq
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert b.svdq_check_device(torch.cuda.current_device()) == b.SVDQ_OK


def _noalloc(Xbits, abi, rank, qfmt):
    t = H.torch()
    M, K = Xbits.shape
    qx = t.empty((M, b.svdq_qrow_bytes(K, qfmt)), dtype=t.uint8, device="cuda")
    sx = t.empty((K // 64, M), dtype=t.float32, device="cuda")
    T = t.empty((M, max(rank, 1)), dtype=t.int16, device="cuda") if rank else None
    b.svdq_quantize_act_noalloc(H.dev(Xbits), H.dev(abi["s"]), H.dev(abi["l1t"]) if rank else None, qx, sx, T,
                                rank, qfmt=qfmt)
    t.cuda.synchronize()
    return qx, sx, T


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
def test_noalloc_matches_the_workspace_path_twice(qfmt):
    # a K-split shape first (the scratch holds 3 x 4608 x 32 partials), then a
    # smaller one (fewer parts and rows: stale partials of the first call must
    # not leak into the second)
    for M, K, N, r, seed in ((4608, 3072, 64, 32, 1), (1000, 1024, 64, 16, 2)):
        print("noalloc", M, K, r, qfmt, "parts", b.svdq_act_workspace_bytes(M, K, r) // max(1, 4 * M * r),
              flush=True)
        assert b.svdq_act_workspace_bytes(M, K, r) > 0, "shape does not split K"
        p = H.make_problem(M, K, N, r, seed=seed, outliers=(3, K - 5))
        ws = H.run_quantize_act(p["X"]["bits"], p["abi"], r, qfmt, split=True)
        na = _noalloc(p["X"]["bits"], p["abi"], r, qfmt)
        for a, c in zip(ws, na):
            assert np.array_equal(H.host(a), H.host(c))
        cx, csx = sq.quantize_activations(p["X"]["values"], p["prep"]["s"])
        assert np.array_equal(H.host(na[0]), H.pack_codes(cx, qfmt))
        assert np.array_equal(H.host(na[1]), csx)


def test_noalloc_rank_zero_and_empty():
    t = H.torch()
    p = H.make_problem(300, 512, 64, 16, seed=4)
    qx, sx, _ = _noalloc(p["X"]["bits"], {"s": p["abi"]["s"]}, 0, b.QFMT_FP6)
    cx, csx = sq.quantize_activations(p["X"]["values"], p["prep"]["s"])
    assert np.array_equal(H.host(qx), H.pack_codes(cx, b.QFMT_FP6))
    assert np.array_equal(H.host(sx), csx)
    e16 = t.empty((0, 512), dtype=t.int16, device="cuda")
    b.svdq_quantize_act_noalloc(e16, H.dev(p["abi"]["s"]), H.dev(p["abi"]["l1t"]),
                                t.empty((0, 256), dtype=t.uint8, device="cuda"),
                                t.empty((8, 0), dtype=t.float32, device="cuda"),
                                t.empty((0, 16), dtype=t.int16, device="cuda"), 16)
    t.cuda.synchronize()
