"""GPU check of the no-allocation decode entry point, through the C ABI.

moe_decode_layer_noalloc runs the decode kernels on the library's static
device scratch instead of a caller workspace. Two calls in a row (four
tokens, then one: the second call reuses the scratch the first one left
behind) must give exactly what moe_decode_layer gives on a fresh workspace
(outputs, logits and routing metadata, bit for bit) and pass the oracle bar.
"""
import numpy as np
import pytest

from int4_grouped_gemm_router_amd import binding as B
from int4_grouped_gemm_router_amd import synth

from parity import check_layer

pytestmark = pytest.mark.gpu


def _run(torch, fn, dw, x):
    d = dw.dims
    T = x.shape[0]
    y = torch.empty((T, d.H), dtype=torch.int16, device="cuda")
    logits = torch.empty((T, d.E), dtype=torch.float32, device="cuda")
    ro = B.RouteBuffers(d, T)
    fn(d, dw, torch.from_numpy(x).cuda(), y, T, logits, ro)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16), logits.cpu().numpy(), ro.to_numpy()


def test_noalloc_decode_matches_workspace_decode():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _, w, _ = synth.generate("prefill_t512", with_x=False)
    dw = B.DeviceWeights.from_logical(w)
    rng = np.random.default_rng(2024)

    def with_ws(d, dw_, x, y, T, logits, ro):
        B.moe_decode_layer(d, dw_, x, y, T, logits, ro, B.workspace(d, T, B.MODE_DECODE))

    def noalloc(d, dw_, x, y, T, logits, ro):
        B.moe_decode_layer_noalloc(d, dw_, x, y, T, logits, ro)

    for T in (4, 1):  # the second call is smaller than the first
        x = synth.make_x(rng, T, w.H)
        print(f"noalloc decode T={T}", flush=True)
        ref = _run(torch, with_ws, dw, x)
        got = _run(torch, noalloc, dw, x)
        assert np.array_equal(got[0], ref[0]), f"T={T}: y differs from moe_decode_layer"
        assert np.array_equal(got[1], ref[1]), f"T={T}: logits differ"
        for f in ("topk_idx", "topk_w", "hist", "offsets", "perm", "inv_perm", "block_map", "num_blocks"):
            assert np.array_equal(np.asarray(got[2][f]), np.asarray(ref[2][f])), (T, f)
        idx = got[2]["topk_idx"].reshape(T, 8)
        wsel = got[2]["topk_w"].reshape(T, 8)
        s = check_layer(x, w, got[0], got[1], idx, wsel)
        print(f"noalloc decode T={T}: {s}", flush=True)
