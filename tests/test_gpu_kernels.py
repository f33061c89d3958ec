"""GPU unit parity: packed-weight expansion and GPU-resident routing.

- moe_test_dequant expands a packed expert with the GEMM kernels' own loads
  and code expansion; the result must equal the oracle's q*scale + bias
  exactly (both round q*s + b once to fp32).
- moe_route on identical fp32 logits (seeded, including forced ties) must
  reproduce the oracle's top-k indices, histogram, offsets, permutation,
  inverse permutation, block map and block count bit for bit; weights agree
  to 1e-6 relative.
"""
import numpy as np
import pytest

import oracle
from int4_grouped_gemm_router_amd import binding as B
from int4_grouped_gemm_router_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


@pytest.mark.parametrize("paired,N,K", [(True, 128, 512), (False, 512, 128), (True, 512, 2048),
                                        (False, 2048, 512)])
def test_dequant_matches_oracle(torch_cuda, paired, N, K):
    torch = torch_cuda
    rng = np.random.default_rng(N * 7 + K)
    count = 3
    mats = []
    for _ in range(2 if paired else 1):
        q = rng.integers(0, 16, size=(count, N, K), dtype=np.uint8)
        s = synth.f32_to_bf16_bits(rng.uniform(-0.05, 0.05, size=(count, N, K // 64)).astype(np.float32))
        b = synth.f32_to_bf16_bits(rng.uniform(-0.5, 0.5, size=(count, N, K // 64)).astype(np.float32))
        mats.append((q, s, b))
    blob = B.pack_int4_g64(*mats[0], *(mats[1] if paired else (None, None, None)))
    dblob = torch.from_numpy(blob).cuda()
    for e in (0, count - 1):
        out = torch.full(((2 if paired else 1), N, K), float("nan"), dtype=torch.float32, device="cuda")
        B.moe_test_dequant(dblob, count, N, K, paired, e, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for m, (q, s, b) in enumerate(mats):
            want = oracle.dequant(q[e], s[e], b[e]).astype(np.float32)
            assert np.array_equal(got[m], want), f"matrix {m} expert {e}"


def _route(torch, logits, E=256, BM=32):
    T = logits.shape[0]
    d = B.dims(2048, 512, E=E)
    out = B.RouteBuffers(d, T)
    ws = B.workspace(d, T, B.MODE_ROUTE)
    B.moe_route(d, torch.from_numpy(logits).cuda(), T, out, ws)
    torch.cuda.synchronize()
    return out.to_numpy()


@pytest.mark.parametrize("T,ties", [(1, 0), (3, 2), (32, 0), (129, 3), (512, 0), (1000, 4),
                                    (2048, 0), (4096, 3)])
def test_route_bit_exact(torch_cuda, T, ties):
    rng = np.random.default_rng(1000 + T)
    logits = synth.random_logits(rng, T, 256, ties=ties)
    got = _route(torch_cuda, logits)
    idx, w = oracle.topk(logits, 8)
    ref = oracle.route_meta(idx, 256, 32)
    assert np.array_equal(got["topk_idx"], idx)
    np.testing.assert_allclose(got["topk_w"], w, rtol=1e-6, atol=1e-7)
    for f in ("hist", "offsets", "perm", "inv_perm"):
        assert np.array_equal(got[f], ref[f]), f
    assert got["num_blocks"] == ref["num_blocks"]
    assert np.array_equal(got["block_map"], ref["block_map"])


def test_route_skewed_groups(torch_cuda):
    # a few experts get almost every token: heavy groups, many empty experts,
    # partial 32-row blocks, and ties inside the top 8
    rng = np.random.default_rng(5)
    T = 777
    logits = synth.random_logits(rng, T, 256, ties=1)
    logits[:, 10:20] += 8.0
    logits[::3, 200] = 100.0
    got = _route(torch_cuda, logits)
    idx, w = oracle.topk(logits, 8)
    ref = oracle.route_meta(idx, 256, 32)
    assert np.array_equal(got["topk_idx"], idx)
    for f in ("hist", "offsets", "perm", "inv_perm", "block_map"):
        assert np.array_equal(got[f], ref[f]), f
    assert (ref["hist"] == 0).sum() > 200


def test_route_all_equal_logits(torch_cuda):
    got = _route(torch_cuda, np.zeros((70, 256), np.float32))
    assert (got["topk_idx"] == np.arange(8)).all()
    assert (got["topk_w"] == np.float32(0.125)).all()
    assert got["num_blocks"] == 8 * 3
