"""GPU layer parity against the CPU oracle, through the C ABI.

Covers every workload shape: the tiny layer (all tokens, ragged token counts),
the 512-token prefill (all tokens), the Zipf-skewed 2048-token prefill (all
tokens, routing metadata), the 16384-token prompt in 4096-token chunks (all
tokens; chunked equals unchunked bit for bit), decode at 1 and 4 tokens, a
seeded sweep of token counts, chunk sizes and GEMM choices (all tokens), plus
edge cases (forced heavy routing with empty experts, determinism, T = 0).
"""
import numpy as np
import pytest

import oracle
from int4_grouped_gemm_router_amd import binding as B
from int4_grouped_gemm_router_amd import synth

from parity import assert_y_close, check_layer, check_route_meta

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


_cache = {}


def _layer(name, seed=0):
    key = (name, seed)
    if key not in _cache:
        wl, w, _ = synth.generate(name, seed=seed, with_x=False)
        _cache.clear()
        _cache[key] = (wl, w, B.DeviceWeights.from_logical(w))
    return _cache[key]


def _prefill(torch, dw, x, chunk=0, route=True, d=None):
    d = dw.dims if d is None else d
    T = x.shape[0]
    xd = torch.from_numpy(x).cuda()
    y = torch.empty((T, d.H), dtype=torch.int16, device="cuda")
    logits = torch.empty((T, d.E), dtype=torch.float32, device="cuda")
    Tc = chunk if chunk else T
    last = T - ((T - 1) // Tc) * Tc
    ro = B.RouteBuffers(d, last) if route else None
    ws = B.workspace(d, Tc, B.MODE_PREFILL)
    B.moe_prefill_layer(d, dw, xd, y, T, chunk, logits, ro, ws)
    torch.cuda.synchronize()
    return (y.cpu().numpy().view(np.uint16), logits.cpu().numpy(),
            ro.to_numpy() if ro is not None else None)


def _route_of(meta_gpu, T):
    return meta_gpu["topk_idx"].reshape(T, 8), meta_gpu["topk_w"].reshape(T, 8)


@pytest.mark.parametrize("T", [1, 5, 17, 32, 64, 100])
def test_prefill_tiny_all_tokens(torch_cuda, T):
    wl, w, dw = _layer("tiny_t32")
    x = synth.make_x(np.random.default_rng(T), T, w.H)
    y, logits, meta = _prefill(torch_cuda, dw, x)
    idx, wsel = _route_of(meta, T)
    s = check_layer(x, w, y, logits, idx, wsel)
    check_route_meta(meta, idx, 256, 8, 32)
    print(f"tiny T={T}: {s}")


def test_prefill_t512_all_tokens(torch_cuda):
    wl, w, dw = _layer("prefill_t512")
    _, _, x = synth.generate("prefill_t512", with_x=True)
    y, logits, meta = _prefill(torch_cuda, dw, x)
    idx, wsel = _route_of(meta, 512)
    s = check_layer(x, w, y, logits, idx, wsel)
    check_route_meta(meta, idx, 256, 8, 32)
    # with no near-tie the oracle's own metadata must match bit for bit
    ref_l = oracle.router_logits(x, w.router_w, w.router_bias)
    ridx, _ = oracle.topk(ref_l, 8)
    if np.array_equal(ridx, idx):
        ref = oracle.route_meta(ridx, 256, 32)
        for f in ("hist", "offsets", "perm", "inv_perm", "block_map"):
            assert np.array_equal(meta[f], ref[f]), f
    print(f"T=512: {s}")


def test_prefill_t512_block16(torch_cuda):
    # 16-row routing blocks, which are also the GEMMs' work items: the block
    # map follows the oracle's for BM = 16, and y equals the 32-row run bit
    # for bit (every output row is computed alone, in the same order)
    torch = torch_cuda
    wl, w, dw = _layer("prefill_t512")
    _, _, x = synth.generate("prefill_t512", with_x=True)
    T = x.shape[0]
    y32, logits32, _ = _prefill(torch, dw, x)
    d16 = B.dims(w.H, w.I, block_m=16)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty((T, w.H), dtype=torch.int16, device="cuda")
    logits = torch.empty((T, w.E), dtype=torch.float32, device="cuda")
    ro = B.RouteBuffers(d16, T)
    B.moe_prefill_layer(d16, dw, xd, y, T, 0, logits, ro, B.workspace(d16, T, B.MODE_PREFILL))
    torch.cuda.synchronize()
    y = y.cpu().numpy().view(np.uint16)
    meta = ro.to_numpy()
    idx, wsel = _route_of(meta, T)
    check_route_meta(meta, idx, 256, 8, 16)
    ref = oracle.route_meta(idx, 256, 16)
    assert np.array_equal(meta["block_map"], ref["block_map"])
    assert np.array_equal(logits.cpu().numpy(), logits32)
    assert np.array_equal(y, y32), "16-row and 32-row work items differ"
    s = check_layer(x, w, y, logits.cpu().numpy(), idx, wsel, tokens=np.arange(0, T, 7))
    print(f"T=512 block_m 16: {s}")


def test_prefill_host_routed_matches(torch_cuda):
    # the host-synchronised routing variant launches exact grids; every unit
    # is computed the same way, so y equals the GPU-routed call bit for bit,
    # and on its own inputs it meets the oracle bar (every token)
    torch = torch_cuda
    for name, T in (("prefill_t512", 512), ("skew_t2048", 2048), ("tiny_t32", 37)):
        wl, w, dw = _layer(name)
        x = synth.make_x(np.random.default_rng(T), T, w.H)
        y_ref, logits, meta = _prefill(torch, dw, x)
        d = dw.dims
        y = torch.empty((T, d.H), dtype=torch.int16, device="cuda")
        B.moe_prefill_layer_host_routed(d, dw, torch.from_numpy(x).cuda(), y, T, 0,
                                        B.workspace(d, T, B.MODE_PREFILL))
        torch.cuda.synchronize()
        y = y.cpu().numpy().view(np.uint16)
        assert np.array_equal(y, y_ref), name
        s = check_layer(x, w, y, logits, *_route_of(meta, T))
        print(f"host-routed {name} T={T}: {s}", flush=True)


def test_prefill_unfused_matches_oracle(torch_cuda):
    # weights expanded to bf16 in memory, then the GEMMs on bf16 weights:
    # the layer bar against the oracle still holds
    torch = torch_cuda
    for name, T in (("tiny_t32", 33), ("prefill_t512", 512)):
        wl, w, dw = _layer(name)
        x = synth.make_x(np.random.default_rng(T + 1), T, w.H)
        d = dw.dims
        y = torch.empty((T, d.H), dtype=torch.int16, device="cuda")
        B.moe_prefill_layer_unfused(d, dw, torch.from_numpy(x).cuda(), y, T, B.unfused_weights(d),
                                    ws=B.workspace(d, T, B.MODE_PREFILL))
        y_ref, logits, meta = _prefill(torch, dw, x)
        torch.cuda.synchronize()
        y = y.cpu().numpy().view(np.uint16)
        idx, wsel = _route_of(meta, T)
        s = check_layer(x, w, y, logits, idx, wsel, tokens=np.arange(0, T, 3))
        print(f"unfused {name} T={T}: {s}")


def test_prefill_skew_t2048_all_tokens(torch_cuda):
    # the Zipf-skewed workload (automatic choice: the wide 144-row GEMMs),
    # every token against the oracle
    wl, w, dw = _layer("skew_t2048")
    _, _, x = synth.generate("skew_t2048", with_x=True)
    T = x.shape[0]
    y, logits, meta = _prefill(torch_cuda, dw, x)
    idx, wsel = _route_of(meta, T)
    check_route_meta(meta, idx, 256, 8, 32)
    hist = meta["hist"]
    assert (hist == 0).sum() > 50 and hist.max() > 500, "skewed routing expected"
    s = check_layer(x, w, y, logits, idx, wsel)
    print(f"skew T=2048 (all {T} tokens): {s}", flush=True)
    # the same prompt in 512-token chunks (64-token router tiles instead of
    # 128-token ones, exact 32-row GEMMs instead of wide ones): identical
    # logits, and outputs within the bar of the oracle
    y2, logits2, _ = _prefill(torch_cuda, dw, x, chunk=512, route=False)
    assert np.array_equal(logits, logits2)
    s2 = check_layer(x, w, y2, logits2, idx, wsel)
    print(f"skew T=2048 in 512-token chunks: {s2}", flush=True)


# Seeded sweep: token counts from 1 to 2600, chunked or not (chunk sizes that
# leave ragged last chunks), each GEMM choice, on the near-uniform and the
# Zipf-skewed layer. Every token against the oracle, with the selections
# re-derived for all tokens from the GPU's logits (the route output holds the
# last chunk only).
@pytest.mark.parametrize("case", range(8))
def test_prefill_random_shapes_all_tokens(torch_cuda, case):
    rng = np.random.default_rng(7000 + case)
    name = ("prefill_t512", "skew_t2048")[case % 2]
    gemm = (B.GEMM_AUTO, B.GEMM_EXACT, B.GEMM_WIDE, B.GEMM_AUTO)[case % 4]
    wl, w, dw = _layer(name)
    T = int(rng.integers(1, 2601))
    chunk = int(rng.choice([0, 0, 96, 517, 1024]))
    x = synth.make_x(rng, T, w.H)
    d = B.dims(w.H, w.I, w.E, gemm=gemm)
    print(f"case {case}: {name} T={T} chunk={chunk} gemm={gemm}", flush=True)
    y, logits, _ = _prefill(torch_cuda, dw, x, chunk=chunk, route=False, d=d)
    ro = B.RouteBuffers(d, T)
    B.moe_route(d, torch_cuda.from_numpy(logits).cuda(), T, ro, B.workspace(d, T, B.MODE_ROUTE))
    torch_cuda.cuda.synchronize()
    idx, wsel = _route_of(ro.to_numpy(), T)
    s = check_layer(x, w, y, logits, idx, wsel)
    print(f"case {case}: {s}", flush=True)


def test_prefill_long_chunked_all_tokens(torch_cuda):
    wl, w, dw = _layer("prefill_t512")   # same layer shape as the long prompt
    x = synth.make_x(np.random.default_rng(16384), 16384, w.H)
    y, logits, meta = _prefill(torch_cuda, dw, x, chunk=4096)
    T = x.shape[0]
    # the route output holds the last chunk's metadata
    idx_last, _ = _route_of(meta, 4096)
    check_route_meta(meta, idx_last, 256, 8, 32)
    y1, logits1, _ = _prefill(torch_cuda, dw, x, chunk=0, route=False)
    assert np.array_equal(y, y1), "chunked and unchunked outputs differ"
    assert np.array_equal(logits, logits1)
    # the GPU's selections for every token, from its own logits via moe_route
    torch = torch_cuda
    d = dw.dims
    ro = B.RouteBuffers(d, T)
    B.moe_route(d, torch.from_numpy(logits).cuda(), T, ro, B.workspace(d, T, B.MODE_ROUTE))
    torch.cuda.synchronize()
    idx_all, w_all = _route_of(ro.to_numpy(), T)
    assert np.array_equal(idx_all[-4096:], idx_last)
    s = check_layer(x, w, y, logits, idx_all, w_all)
    print(f"long T=16384 chunk 4096 (all {T} tokens): {s}", flush=True)


@pytest.mark.parametrize("T", [1, 5, 100, 300])
def test_prefill_wide_tiny_all_tokens(torch_cuda, T):
    # the wide GEMMs (items of up to 144 rows, bf16 weights expanded once per
    # item) forced on the tiny layer: one gate/up and two down column tiles,
    # 8 and 2 groups, ragged items and shared items
    wl, w, dw = _layer("tiny_t32")
    d = B.dims(w.H, w.I, gemm=B.GEMM_WIDE)
    x = synth.make_x(np.random.default_rng(500 + T), T, w.H)
    y, logits, meta = _prefill(torch_cuda, dw, x, d=d)
    idx, wsel = _route_of(meta, T)
    check_route_meta(meta, idx, 256, 8, 32)
    s = check_layer(x, w, y, logits, idx, wsel)
    print(f"wide tiny T={T}: {s}", flush=True)


def test_prefill_wide_forced_heavy_routing(torch_cuda):
    # twelve experts take nearly every pair: items of 144 rows plus ragged
    # tails, 244 empty experts; wide and exact GEMMs both against the oracle
    import copy
    _, w, _ = _layer("tiny_t32")
    w2 = copy.deepcopy(w)
    rb = np.zeros(256, np.float32)
    rb[:8] = 6.0
    rb[100:104] = 5.9
    w2.router_bias = rb
    dw2 = B.DeviceWeights.from_logical(w2)
    x = synth.make_x(np.random.default_rng(4), 700, w.H)
    for gemm in (B.GEMM_WIDE, B.GEMM_EXACT):
        y, logits, meta = _prefill(torch_cuda, dw2, x, d=B.dims(w.H, w.I, gemm=gemm))
        idx, wsel = _route_of(meta, 700)
        check_route_meta(meta, idx, 256, 8, 32)
        assert (meta["hist"] == 0).sum() >= 200 and meta["hist"].max() > 300
        s = check_layer(x, w2, y, logits, idx, wsel)
        print(f"forced heavy routing, gemm {gemm}: {s}", flush=True)


def test_prefill_wide_t512_all_tokens(torch_cuda):
    # the 512-token layer with the wide GEMMs forced (about 16 rows per
    # expert): every token against the oracle
    wl, w, dw = _layer("prefill_t512")
    _, _, x = synth.generate("prefill_t512", with_x=True)
    y, logits, meta = _prefill(torch_cuda, dw, x, d=B.dims(w.H, w.I, gemm=B.GEMM_WIDE))
    idx, wsel = _route_of(meta, 512)
    s = check_layer(x, w, y, logits, idx, wsel)
    print(f"wide T=512: {s}", flush=True)


def test_prefill_ragged_chunks(torch_cuda):
    # 100 tokens in chunks of 32 (32, 32, 32, 4): every token against the
    # oracle, bit-identical to the unchunked call, and the route output holds
    # the last (4-token) chunk's metadata
    _, w, dw = _layer("tiny_t32")
    x = synth.make_x(np.random.default_rng(21), 100, w.H)
    y, logits, meta = _prefill(torch_cuda, dw, x, chunk=32)
    y1, logits1, _ = _prefill(torch_cuda, dw, x, chunk=0, route=False)
    assert np.array_equal(y, y1) and np.array_equal(logits, logits1)
    idx_last, _ = _route_of(meta, 4)
    check_route_meta(meta, idx_last, 256, 8, 32)
    d = dw.dims
    ro = B.RouteBuffers(d, 100)
    B.moe_route(d, torch_cuda.from_numpy(logits).cuda(), 100, ro, B.workspace(d, 100, B.MODE_ROUTE))
    torch_cuda.cuda.synchronize()
    idx_all, w_all = _route_of(ro.to_numpy(), 100)
    assert np.array_equal(idx_all[-4:], idx_last)
    check_layer(x, w, y, logits, idx_all, w_all)


def test_zero_input_exact(torch_cuda):
    # x = 0: every logit is 0, so the selection is experts 0..7 (ties to the
    # lower index) with weights exactly 1/8, every product is 0 and y is +0
    # bit for bit, through prefill and decode alike
    _, w, dw = _layer("tiny_t32")
    for T in (1, 4, 37):
        x = np.zeros((T, w.H), np.uint16)
        outs = [_prefill(torch_cuda, dw, x)]
        if T <= 4:
            outs.append(_decode(torch_cuda, dw, x))
        for y, logits, meta in outs:
            assert not y.any(), "y must be +0 everywhere"
            assert not logits.any()
            idx, wsel = _route_of(meta, T)
            assert np.array_equal(idx, np.tile(np.arange(8), (T, 1)))
            assert np.all(wsel == np.float32(0.125))


def test_prefill_forced_heavy_routing(torch_cuda):
    # a router bias that sends nearly every token to experts 0..7 and 100..103:
    # groups of hundreds of rows, 244 empty experts, ragged 64-row items
    import copy
    _, w, _ = _layer("tiny_t32")
    w2 = copy.deepcopy(w)
    rb = np.zeros(256, np.float32)
    rb[:8] = 6.0
    rb[100:104] = 5.9
    w2.router_bias = rb
    dw2 = B.DeviceWeights.from_logical(w2)
    x = synth.make_x(np.random.default_rng(3), 300, w.H)
    y, logits, meta = _prefill(torch_cuda, dw2, x)
    idx, wsel = _route_of(meta, 300)
    check_route_meta(meta, idx, 256, 8, 32)
    assert (meta["hist"] == 0).sum() >= 200
    check_layer(x, w2, y, logits, idx, wsel)


def test_prefill_deterministic_and_empty(torch_cuda):
    _, w, dw = _layer("tiny_t32")
    x = synth.make_x(np.random.default_rng(9), 77, w.H)
    y1, l1, m1 = _prefill(torch_cuda, dw, x)
    y2, l2, m2 = _prefill(torch_cuda, dw, x)
    assert np.array_equal(y1, y2) and np.array_equal(l1, l2)
    for f in m1:
        assert np.array_equal(np.asarray(m1[f]), np.asarray(m2[f])), f
    # T = 0 enqueues nothing and succeeds
    B.moe_prefill_layer(dw.dims, dw, None, None, 0)


def _decode(torch, dw, x):
    d = dw.dims
    T = x.shape[0]
    y = torch.empty((T, d.H), dtype=torch.int16, device="cuda")
    logits = torch.empty((T, d.E), dtype=torch.float32, device="cuda")
    ro = B.RouteBuffers(d, T)
    ws = B.workspace(d, T, B.MODE_DECODE)
    B.moe_decode_layer(d, dw, torch.from_numpy(x).cuda(), y, T, logits, ro, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16), logits.cpu().numpy(), ro.to_numpy()


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_decode_matches_oracle(torch_cuda, T):
    wl, w, dw = _layer("prefill_t512")
    rng = np.random.default_rng(40 + T)
    for step in range(3):
        x = synth.make_x(rng, T, w.H)
        y, logits, meta = _decode(torch_cuda, dw, x)
        idx, wsel = _route_of(meta, T)
        s = check_layer(x, w, y, logits, idx, wsel)
        check_route_meta(meta, idx, 256, 8, 32)
        uniq = np.unique(idx)
        assert meta["num_blocks"] == len(uniq)
        assert np.array_equal(meta["block_map"][:, 0], uniq)
        print(f"decode T={T} step {step}: {s}")


@pytest.mark.parametrize("T", [1, 4])
def test_decode_skewed_router_bias(torch_cuda, T):
    # the skewed layer's per-expert logit bias goes through the decode router
    # kernel; with it most tokens pick from a few heavy experts, so at T = 4
    # the tokens share experts (fewer unique experts than pairs)
    wl, w, dw = _layer("skew_t2048")
    assert w.router_bias is not None
    rng = np.random.default_rng(70 + T)
    uniq_counts = []
    for step in range(3):
        x = synth.make_x(rng, T, w.H)
        y, logits, meta = _decode(torch_cuda, dw, x)
        idx, wsel = _route_of(meta, T)
        s = check_layer(x, w, y, logits, idx, wsel)
        check_route_meta(meta, idx, 256, 8, 32)
        uniq = np.unique(idx)
        assert meta["num_blocks"] == len(uniq)
        uniq_counts.append(len(uniq))
        print(f"skewed decode T={T} step {step}: {s}")
    if T == 4:
        assert min(uniq_counts) < 8 * T, "skewed routing should make tokens share experts"


@pytest.mark.parametrize("T", [3, 4])
def test_decode_all_distinct_experts(torch_cuda, T):
    # router rows 8t..8t+7 read input dimension t strongly and token t alone
    # carries that dimension, so the k*T pairs select k*T distinct experts:
    # at T = 4 every routed slot is taken and the shared expert's gate/up
    # tiles run after the last slot's own (at T = 3 it has a slot of its own)
    import copy
    _, w, _ = _layer("prefill_t512")
    w2 = copy.deepcopy(w)
    for t in range(T):
        w2.router_w[8 * t:8 * t + 8, t] = 2.0
    dw2 = B.DeviceWeights.from_logical(w2)
    rng = np.random.default_rng(90 + T)
    for step in range(2):
        xf = synth.bf16_bits_to_f32(synth.make_x(rng, T, w.H))
        xf[:, :T] = 0.0
        for t in range(T):
            xf[t, t] = 8.0
        x = synth.f32_to_bf16_bits(xf)
        y, logits, meta = _decode(torch_cuda, dw2, x)
        idx, wsel = _route_of(meta, T)
        assert np.array_equal(np.sort(idx, axis=1), np.arange(8 * T).reshape(T, 8))
        assert meta["num_blocks"] == 8 * T
        s = check_layer(x, w2, y, logits, idx, wsel)
        print(f"all-distinct decode T={T} step {step}: {s}")


def test_decode_tiny_and_vs_prefill(torch_cuda):
    _, w, dw = _layer("tiny_t32")
    x = synth.make_x(np.random.default_rng(11), 4, w.H)
    yd, ld, md = _decode(torch_cuda, dw, x)
    yp, lp, mp = _prefill(torch_cuda, dw, x)
    check_layer(x, w, yd, ld, *_route_of(md, 4))
    if np.array_equal(md["topk_idx"], mp["topk_idx"]):
        assert_y_close(synth.bf16_bits_to_f32(yd), synth.bf16_bits_to_f32(yp), "decode vs prefill")


# Other sizes of the same layer family, chosen to reach the paths the main
# shapes do not: (1024, 384, E=128): gate/up over 16 groups, down over K = 384
# (6 groups: not a multiple of four); (4096, 256, E=64): gate/up over 64 groups
# (the most the GEMMs and the decode kernels take), down over 4 groups;
# (768, 640, E=192): 12 and 10 groups; (256, 4096, E=64): the largest
# intermediate size, down over 64 groups (eight rounds in the decode down
# kernel) and 128 gate/up wave tiles. Prefill on a ragged 40-token batch,
# then decode at T = 1 and 4.
@pytest.mark.parametrize("H,I,E", [(1024, 384, 128), (4096, 256, 64), (768, 640, 192), (256, 4096, 64)])
def test_other_family_sizes(torch_cuda, H, I, E):
    rng = np.random.default_rng(H + I + E)
    w = synth.make_weights(rng, H, I, E)
    dw = B.DeviceWeights.from_logical(w)
    x = synth.make_x(rng, 40, H)
    y, logits, meta = _prefill(torch_cuda, dw, x)
    idx, wsel = _route_of(meta, 40)
    s = check_layer(x, w, y, logits, idx, wsel)
    check_route_meta(meta, idx, E, 8, 32)
    print(f"prefill H={H} I={I} E={E}: {s}")
    for T in (1, 4):
        xt = synth.make_x(rng, T, H)
        yd, ld, md = _decode(torch_cuda, dw, xt)
        idx, wsel = _route_of(md, T)
        s = check_layer(xt, w, yd, ld, idx, wsel)
        check_route_meta(md, idx, E, 8, 32)
        print(f"decode T={T} H={H} I={I} E={E}: {s}")


# The wide GEMMs at the same family sizes (their automatic choice needs
# thousands of tokens): 300 tokens forced wide, every token against the
# oracle, reaching gate/up over 64 groups (H = 4096), 128 gate/up wave tiles
# and a down K of 4096 (I = 4096, 64 groups per item), and the partial last
# 512-column tile (I = 384 and 640: 12 and 20 wave tiles; H = 768).
@pytest.mark.parametrize("H,I,E", [(1024, 384, 128), (4096, 256, 64), (768, 640, 192), (256, 4096, 64)])
def test_other_family_sizes_wide(torch_cuda, H, I, E):
    rng = np.random.default_rng(H + I + E + 1)
    w = synth.make_weights(rng, H, I, E)
    dw = B.DeviceWeights.from_logical(w)
    d = B.dims(H, I, E, gemm=B.GEMM_WIDE)
    x = synth.make_x(rng, 300, H)
    y, logits, meta = _prefill(torch_cuda, dw, x, d=d)
    idx, wsel = _route_of(meta, 300)
    s = check_layer(x, w, y, logits, idx, wsel)
    print(f"wide prefill H={H} I={I} E={E}: {s}")


def test_gemm_auto_threshold(torch_cuda):
    # the automatic choice takes the wide GEMMs from 36 pairs per expert on
    # (8 T >= 36 E: T >= 1152 at E = 256): bit for bit the forced choice on
    # each side of the threshold, and the two choices differ
    _, w, dw = _layer("prefill_t512")
    x = synth.make_x(np.random.default_rng(33), 1152, w.H)
    auto = B.dims(w.H, w.I)
    exact = B.dims(w.H, w.I, gemm=B.GEMM_EXACT)
    wide = B.dims(w.H, w.I, gemm=B.GEMM_WIDE)
    for T, same in ((1151, exact), (1152, wide)):
        ya, _, _ = _prefill(torch_cuda, dw, x[:T], route=False, d=auto)
        yf, _, _ = _prefill(torch_cuda, dw, x[:T], route=False, d=same)
        other = wide if same is exact else exact
        yo, _, _ = _prefill(torch_cuda, dw, x[:T], route=False, d=other)
        assert np.array_equal(ya, yf), T
        assert not np.array_equal(ya, yo), T
        assert_y_close(synth.bf16_bits_to_f32(ya), synth.bf16_bits_to_f32(yo), f"T={T} exact vs wide")


def test_prefill_graph_replay_matches_eager(torch_cuda):
    """The layer captured in a HIP graph and replayed (with eager work and
    synchronisations in between) gives exactly the eager output every time."""
    torch = torch_cuda
    wl, w, dw = _layer("prefill_t512")
    _, _, x = synth.generate("prefill_t512", with_x=True)
    d = dw.dims
    T = x.shape[0]
    xd = torch.from_numpy(x).cuda()
    ws = B.workspace(d, T, B.MODE_PREFILL)
    y_eager = torch.empty((T, d.H), dtype=torch.int16, device="cuda")
    B.moe_prefill_layer(d, dw, xd, y_eager, T, 0, None, None, ws)
    torch.cuda.synchronize()
    y = torch.zeros_like(y_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.moe_prefill_layer(d, dw, xd, y, T, 0, None, None, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.moe_prefill_layer(d, dw, xd, y, T, 0, None, None, ws)
    for rep in range(3):
        y.zero_()
        ws.fill_(0xA5)                      # the workspace holds no state between calls
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {rep} differs from the eager output"
        B.moe_prefill_layer(d, dw, xd, y, T, 0, None, None, ws)   # eager work in between
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager)


@pytest.mark.parametrize("T", [1, 4])
def test_decode_graph_replay_matches_eager(torch_cuda, T):
    """Three decode steps (different tokens) captured in one HIP graph and
    replayed with eager work and synchronisations in between: outputs,
    logits and routing metadata equal the eager ones every time."""
    torch = torch_cuda
    wl, w, dw = _layer("prefill_t512")
    d = dw.dims
    rng = np.random.default_rng(90 + T)
    xs = [torch.from_numpy(synth.make_x(rng, T, w.H)).cuda() for _ in range(3)]
    ws = B.workspace(d, T, B.MODE_DECODE)
    ys = [torch.empty((T, d.H), dtype=torch.int16, device="cuda") for _ in range(3)]
    lg = [torch.empty((T, d.E), dtype=torch.float32, device="cuda") for _ in range(3)]
    ro = [B.RouteBuffers(d, T) for _ in range(3)]

    def steps():
        for i in range(3):
            B.moe_decode_layer(d, dw, xs[i], ys[i], T, lg[i], ro[i], ws)

    steps()
    torch.cuda.synchronize()
    ref = [(y.clone(), l.clone(), r.to_numpy()) for y, l, r in zip(ys, lg, ro)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        steps()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps()
    # the eager steps against the oracle on their own inputs
    for i in range(3):
        xi = xs[i].cpu().numpy()
        got = ref[i][2]
        s = check_layer(xi, w, ref[i][0].cpu().numpy().view(np.uint16), ref[i][1].cpu().numpy(),
                        got["topk_idx"].reshape(T, 8), got["topk_w"].reshape(T, 8))
        print(f"graph decode T={T} step {i}: {s}", flush=True)
    for rep in range(3):
        for y, l, r in zip(ys, lg, ro):
            y.zero_()
            l.zero_()
            for f, _ in B.MoeRouteOut._fields_:
                getattr(r, f).zero_()
        ws.fill_(0xA5)                      # the workspace holds no state between calls
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(ys[i], ref[i][0]), f"replay {rep} step {i}: y differs"
            assert torch.equal(lg[i], ref[i][1]), f"replay {rep} step {i}: logits differ"
            got = ro[i].to_numpy()
            for f in ("topk_idx", "topk_w", "hist", "offsets", "perm", "inv_perm", "block_map",
                      "num_blocks"):
                assert np.array_equal(np.asarray(got[f]), np.asarray(ref[i][2][f])), (rep, i, f)
        steps()                               # eager work in between
        torch.cuda.synchronize()


def test_concurrent_streams_match_sequential(torch_cuda):
    """A prefill and two decodes enqueued on three streams at once, each with
    its own workspace, give exactly what the same calls give one after
    another: the library keeps no state shared between calls."""
    torch = torch_cuda
    _, w, dw = _layer("prefill_t512")
    d = dw.dims
    rng = np.random.default_rng(123)
    xp = torch.from_numpy(synth.make_x(rng, 300, w.H)).cuda()
    xd = [torch.from_numpy(synth.make_x(rng, T, w.H)).cuda() for T in (1, 4)]
    wsp = B.workspace(d, 300, B.MODE_PREFILL)
    wsd = [B.workspace(d, T, B.MODE_DECODE) for T in (1, 4)]

    def run(streams):
        yp = torch.empty((300, d.H), dtype=torch.int16, device="cuda")
        yd = [torch.empty((T, d.H), dtype=torch.int16, device="cuda") for T in (1, 4)]
        with torch.cuda.stream(streams[0]):
            B.moe_prefill_layer(d, dw, xp, yp, 300, 0, None, None, wsp)
        for i, T in enumerate((1, 4)):
            with torch.cuda.stream(streams[i + 1]):
                B.moe_decode_layer(d, dw, xd[i], yd[i], T, None, None, wsd[i])
        torch.cuda.synchronize()
        return [yp] + yd

    cur = torch.cuda.current_stream()
    seq = run([cur, cur, cur])
    streams = [torch.cuda.Stream() for _ in range(3)]
    for s_ in streams:
        s_.wait_stream(cur)
    for rep in range(3):
        par = run(streams)
        for a, b in zip(seq, par):
            assert torch.equal(a, b), f"repeat {rep}: concurrent result differs"


@pytest.mark.gpu
def test_ceiling_helpers_run():
    """The measurement kernels launch through the C ABI, finish, and leave the
    sink untouched (their conditional store never fires on these inputs)."""
    import torch
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * B.CEILING_MFMA_BLOCKS, dtype=torch.int64, device="cuda")
    B.moe_ceiling_read(buf, sink)
    for random in (True, False):
        flops = B.moe_ceiling_mfma(8, sink, random=random, clocks=clocks)
        torch.cuda.synchronize()
        assert flops == 1024 * 4 * 8 * 4 * 8 * (16 * 16 * 32 * 2)
        mhz = B.ceiling_clock_mhz(clocks)
        print(f"matrix-core loop, random operands {random}: shader clock {mhz:.0f} MHz", flush=True)
        assert 100.0 < mhz < 4000.0
    assert torch.count_nonzero(sink).item() == 0
    with pytest.raises(B.MoeError):
        B.moe_ceiling_read(buf[:15], sink)  # not a multiple of 16 bytes


# The exact 32-row GEMMs at family sizes whose down projection has a group
# count that is not a multiple of four (I / 64 = 6 and 10), on 8192 tokens:
# about 20 work units per persistent block, so the ring's hand-off of loads
# to the next unit and the rollover past a block's 16-unit batch both run.
# Every token against the oracle; the wide kernels on the same inputs too
# (their half-filled last column tile at I = 384 and 640).
@pytest.mark.parametrize("H,I,E", [(1024, 384, 128), (768, 640, 192)])
def test_exact_gemm_long_run_odd_group_pairs(torch_cuda, H, I, E):
    rng = np.random.default_rng(H * 7 + I)
    w = synth.make_weights(rng, H, I, E)
    dw = B.DeviceWeights.from_logical(w)
    T = 8192
    x = synth.make_x(rng, T, H)
    for gemm in (B.GEMM_EXACT, B.GEMM_WIDE):
        y, logits, meta = _prefill(torch_cuda, dw, x, d=B.dims(H, I, E, gemm=gemm))
        idx, wsel = _route_of(meta, T)
        s = check_layer(x, w, y, logits, idx, wsel)
        print(f"H={H} I={I} E={E} T={T} gemm {gemm}: {s}", flush=True)
