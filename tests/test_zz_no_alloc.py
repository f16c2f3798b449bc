"""serq_linear_noalloc (the allocation-free entry point, its quantized
activations in the library's own device array) through the C ABI against
serq_linear with a caller workspace: the same Y bit for bit, on two calls in
a row, the second with fewer tokens and a narrower input, so that the second
call reads the array as the first left it beyond its own bytes."""
import numpy as np
import pytest

from rank_error_compensated_amd import binding as B
from rank_error_compensated_amd import workloads as WL

pytestmark = pytest.mark.gpu


def _run(torch, layer, X, M, noalloc):
    Y = torch.full((M, layer.L.d_out), float("nan"), dtype=torch.float32, device="cuda")
    d = layer.dev
    if noalloc:
        B.serq_linear_noalloc(layer.L, X, d["wq"], d["wscale"], d["rq"], d["rscale"], Y)
    else:
        ws = torch.empty(B.serq_linear_workspace_bytes(layer.L, M), dtype=torch.uint8, device="cuda")
        B.serq_linear(layer.L, X, d["wq"], d["wscale"], d["rq"], d["rscale"], Y, ws)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


@pytest.mark.parametrize("fmt", ["int4", "w4a8", "mxfp4", "mxw4a8"])
def test_noalloc_matches_workspace_entry_point(fmt):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    B.lib()
    # a prefill call, then a smaller one (fewer tokens, narrower input)
    for seed, (M, d_in, d_out, r) in ((1, (520, 1024, 400, 128)), (2, (9, 512, 272, 64))):
        c = WL.random_case(seed * 31 + len(fmt), M, d_in, d_out, r, fmt, n_out=4, factor=50.0, n_cal=32)
        layer = B.PreparedLayer.prepare(c.W, c.X_cal, r, fmt, "cuda")
        X = torch.from_numpy(B.serq_flatten_act(c.X, layer.host["perm"], layer.host["s"])).to("cuda")
        want = _run(torch, layer, X, M, noalloc=False)
        got = _run(torch, layer, X, M, noalloc=True)
        assert np.all(np.isfinite(got))
        np.testing.assert_array_equal(got, want)


def test_noalloc_rejects_inputs_beyond_its_array():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    L = B.serq_query_layout(4096, 256, 128, "w4a8")
    M = B.NOALLOC_SCRATCH_BYTES // 4096 + 1
    X = torch.zeros((M, 4096), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((1, 256), dtype=torch.float32, device="cuda")
    w = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.SerqError) as e:
        B.serq_linear_noalloc(L, X, w, w, w, w, Y)
    assert e.value.status == B.SERQ_ERR_BUFFER
