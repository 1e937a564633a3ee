"""The allocation-free AWQ search (woq_awq_search_noalloc, static scratch)
against the workspace entry point woq_awq_search, through the C ABI: two
calls in a row, the second on a smaller layer, each equal to the workspace
call's losses, index and scale."""
import numpy as np
import pytest
import torch

from weight_only_quantization_quantize_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(T, N, K, seed):
    ch = synth.outlier_channels(K, seed)
    X = torch.from_numpy(synth.to_f16(synth.activations_f32(T, K, seed, ch))).to(DEV)
    W = torch.from_numpy(synth.weights(N, K, seed + 1)).to(DEV)
    return X, W


def _outs(n_grid, K):
    return (torch.full((n_grid,), -1.0, dtype=torch.float64, device=DEV),
            torch.full((K,), -1.0, dtype=torch.float32, device=DEV),
            torch.full((1,), -1, dtype=torch.int32, device=DEV))


def _with_workspace(lib, X, W, bits, G, asym, n_grid):
    T, K = X.shape
    N = W.shape[0]
    nbytes = lib.woq_awq_search_workspace_bytes(T, N, K, bits, G, int(asym))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    losses, scale, idx = _outs(n_grid, K)
    st = lib.woq_awq_search(X.data_ptr(), W.data_ptr(), T, N, K, bits, G, int(asym), n_grid, losses.data_ptr(),
                            scale.data_ptr(), idx.data_ptr(), ws.data_ptr(), nbytes,
                            torch.cuda.current_stream().cuda_stream)
    _lib.check(st, "woq_awq_search")
    torch.cuda.synchronize()
    return losses.cpu().numpy(), scale.cpu().numpy(), int(idx.cpu().numpy()[0])


def _noalloc(lib, X, W, bits, G, asym, n_grid):
    T, K = X.shape
    N = W.shape[0]
    losses, scale, idx = _outs(n_grid, K)
    st = lib.woq_awq_search_noalloc(X.data_ptr(), W.data_ptr(), T, N, K, bits, G, int(asym), n_grid,
                                    losses.data_ptr(), scale.data_ptr(), idx.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    _lib.check(st, "woq_awq_search_noalloc")
    torch.cuda.synchronize()
    return losses.cpu().numpy(), scale.cpu().numpy(), int(idx.cpu().numpy()[0])


def test_noalloc_search_equals_the_workspace_search_on_two_calls():
    lib = _lib.load()
    assert lib.woq_awq_search_noalloc_max_bytes() == 32 << 20
    # the larger call first (a q_proj-sized layer, register-B GEMM, several
    # exponents per batched launch in the workspace call), then a smaller one
    # on another quantizer: the second must not see the first's leftovers
    for (T, N, K, bits, G, asym, n_grid, seed) in [(512, 4096, 4096, 4, 128, True, 20, 3200),
                                                  (64, 384, 1024, 3, 64, False, 10, 77)]:
        print(f"awq noalloc T={T} N={N} K={K} bits={bits} G={G} asym={asym} n_grid={n_grid}", flush=True)
        X, W = _inputs(T, N, K, seed)
        ref = _with_workspace(lib, X, W, bits, G, asym, n_grid)
        got = _noalloc(lib, X, W, bits, G, asym, n_grid)
        # every output of the search is computed by the same kernels in the
        # same order: losses, scale and index are bit-equal
        assert np.array_equal(got[0], ref[0]), (got[0], ref[0])
        assert np.array_equal(got[1].view(np.uint32), ref[1].view(np.uint32))
        assert got[2] == ref[2]
        assert np.all(np.isfinite(got[0])) and 0 <= got[2] < n_grid
