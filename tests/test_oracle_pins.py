"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks one oracle function against a closed form, an invariant, a
brute-force enumeration, a library routine on a special case, or a hand-derived
fixture under tests/golden/. Together they are chosen so that a plausible slip
(a dropped bias, the group index taken along the wrong axis, gate and up
swapped, a transposed down projection, a wrong tie-break, weights not
renormalised, an unstable scatter) fails at least one of them.

  oracle_dequant        golden fixture; group axis probe; (q-8)*s exact in fp32
  oracle_router_logits  integer-valued inputs vs numpy int64 matmul (exact)
  oracle_topk           golden fixture; brute-force sort; scipy softmax
  oracle_route_meta     numpy bincount / cumsum / stable argsort; block tiling
  oracle_expert_ffn     closed form with one-hot input (gate/up asymmetric);
                        x = 0; transposed-down probe
  oracle_layer          dense masked brute force; identical experts; zero
                        routed experts; independent numpy reformulation
"""
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from int4_grouped_gemm_router_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(v):
    return synth.f32_to_bf16_bits(np.asarray(v, np.float32))


def _read_rows(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line)
    return rows


# ---------------------------------------------------------------- dequant

def test_dequant_golden_fixture():
    for row in _read_rows("dequant_affine_int4.txt"):
        q, s, b, want = row.split()
        qq = np.full((1, 64), int(q), np.uint8)
        ss = _bf16([[float(s)]])
        bb = _bf16([[float(b)]])
        assert synth.bf16_bits_to_f32(ss)[0, 0] == float(s)
        assert synth.bf16_bits_to_f32(bb)[0, 0] == float(b)
        w = oracle.dequant(qq, ss, bb)
        assert np.all(w == float(want)), row


def test_dequant_group_axis_is_input_dim():
    # scale[n][g] = 2**g (+ n/8 to tell rows apart), bias 0, q = 1:
    # w[n][c] must follow the group of column c, not of row n.
    rows, cols = 3, 256
    q = np.ones((rows, cols), np.uint8)
    s = np.array([[2.0 ** g + n / 8.0 for g in range(cols // 64)] for n in range(rows)],
                 np.float32)
    w = oracle.dequant(q, _bf16(s), _bf16(np.zeros_like(s)))
    for n in range(rows):
        for c in range(cols):
            assert w[n, c] == 2.0 ** (c // 64) + n / 8.0


def test_dequant_symmetric_form_exact_in_fp32():
    # With bias = -8*scale the affine form is (q-8)*scale, exactly representable in fp32.
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, size=(64, 128), dtype=np.uint8)
    s = _bf16(rng.uniform(0.005, 0.02, size=(64, 2)).astype(np.float32))
    b = _bf16(-8.0 * synth.bf16_bits_to_f32(s))
    w = oracle.dequant(q, s, b)
    sf = np.repeat(synth.bf16_bits_to_f32(s).astype(np.float64), 64, axis=1)
    assert np.array_equal(w, (q.astype(np.float64) - 8.0) * sf)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)


def test_dequant_rejects_out_of_range_nibble():
    q = np.full((1, 64), 16, np.uint8)
    with pytest.raises(RuntimeError):
        oracle.dequant(q, _bf16([[1.0]]), _bf16([[0.0]]))


# ---------------------------------------------------------------- router logits

def test_router_logits_integer_inputs_match_int_matmul():
    rng = np.random.default_rng(2)
    T, H, E = 5, 128, 16
    xi = rng.integers(-8, 9, size=(T, H))
    wi = rng.integers(-100, 101, size=(E, H))
    x = _bf16(xi.astype(np.float32))
    wr = (wi / 64.0).astype(np.float32)          # dyadic: exact in fp32
    rb = (rng.integers(-50, 51, size=E) / 8.0).astype(np.float32)
    got = oracle.router_logits(x, wr, rb)
    want = (xi.astype(np.int64) @ wi.T.astype(np.int64)) / 64.0 + rb.astype(np.float64)
    assert np.array_equal(got.astype(np.float64), want)
    got0 = oracle.router_logits(x, wr, None)
    assert np.array_equal(got0.astype(np.float64), (xi @ wi.T) / 64.0)


# ---------------------------------------------------------------- top-k

def test_topk_golden_fixture():
    for row in _read_rows("topk_cases.txt"):
        k, l, idx, w = [part.strip() for part in row.split("|")]
        logits = np.array([[float(v) for v in l.split()]], np.float32)
        gi, gw = oracle.topk(logits, int(k))
        assert gi[0].tolist() == [int(v) for v in idx.split()], row
        np.testing.assert_allclose(gw[0], [float(v) for v in w.split()], rtol=1e-6)


@pytest.mark.parametrize("ties", [0, 2, 4])
def test_topk_matches_brute_force_sort(ties):
    rng = np.random.default_rng(3 + ties)
    T, E, k = 64, 256, 8
    logits = synth.random_logits(rng, T, E, ties=ties)
    idx, w = oracle.topk(logits, k)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        assert idx[t].tolist() == order[:k]
        p = scipy.special.softmax(logits[t].astype(np.float64))
        ref = p[order[:k]] / p[order[:k]].sum()
        np.testing.assert_allclose(w[t], ref, rtol=2e-7, atol=0)
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) < 1e-6


def test_topk_all_equal_logits():
    idx, w = oracle.topk(np.zeros((3, 256), np.float32), 8)
    assert (idx == np.arange(8)).all()
    assert (w == np.float32(0.125)).all()


def test_topk_alt_swap_takes_ninth():
    logits = np.arange(16, dtype=np.float32)[None, ::-1].copy()  # expert e has logit 15-e
    i0, _ = oracle.topk(logits, 8)
    i1, w1 = oracle.topk(logits, 8, alt_swap=True)
    assert i0[0].tolist() == list(range(8))
    assert i1[0].tolist() == list(range(7)) + [8]
    p = scipy.special.softmax(logits[0].astype(np.float64))[i1[0]]
    np.testing.assert_allclose(w1[0], p / p.sum(), rtol=2e-7)


# ---------------------------------------------------------------- routing metadata

def _check_meta(idx, E, BM, meta):
    T, k = idx.shape
    flat = idx.ravel()
    assert np.array_equal(meta["hist"], np.bincount(flat, minlength=E))
    assert int(meta["hist"].sum()) == k * T
    assert np.array_equal(meta["offsets"], np.concatenate([[0], np.cumsum(meta["hist"])]))
    assert np.array_equal(meta["perm"], np.argsort(flat, kind="stable"))
    assert np.array_equal(meta["inv_perm"][meta["perm"]], np.arange(k * T))
    bm = meta["block_map"]
    assert meta["num_blocks"] == sum(-(-int(c) // BM) for c in meta["hist"])
    covered = np.zeros(k * T, np.int64)
    prev_e = -1
    for e, start, rows in bm:
        assert 1 <= rows <= BM and e >= prev_e
        assert meta["offsets"][e] <= start and start + rows <= meta["offsets"][e + 1]
        assert (start - meta["offsets"][e]) % BM == 0
        covered[start:start + rows] += 1
        prev_e = e
    assert (covered == 1).all()


@pytest.mark.parametrize("T,ties", [(1, 0), (32, 0), (100, 3), (512, 0)])
def test_route_meta_against_numpy(T, ties):
    rng = np.random.default_rng(T)
    logits = synth.random_logits(rng, T, 256, ties=ties)
    idx, _ = oracle.topk(logits, 8)
    meta = oracle.route_meta(idx, 256, 32)
    _check_meta(idx, 256, 32, meta)


def test_route_meta_skewed_and_empty_experts():
    # all tokens on experts 0..7 (248 empty experts, 37-row segments: partial blocks)
    idx = np.tile(np.arange(8, dtype=np.int32), (37, 1))
    meta = oracle.route_meta(idx, 256, 32)
    _check_meta(idx, 256, 32, meta)
    assert meta["num_blocks"] == 16
    assert (meta["hist"][8:] == 0).all()


# ---------------------------------------------------------------- one expert

def _const_mat(rows, cols, qval, scale=1.0, bias=0.0):
    q = np.full((rows, cols), qval, np.uint8)
    s = _bf16(np.full((rows, cols // 64), scale, np.float32))
    b = _bf16(np.full((rows, cols // 64), bias, np.float32))
    return q, s, b


def test_expert_ffn_closed_form_gate_up_asymmetric():
    H, I = 128, 64
    x = np.zeros(H, np.uint16)
    x[5] = _bf16([1.0])[0]                       # one-hot input
    gate = _const_mat(I, H, 1)                   # g_n = 1
    up = _const_mat(I, H, 2)                     # u_n = 2
    qd = np.zeros((H, I), np.uint8)
    for r in range(H):
        qd[r, r % I] = 1                         # d_r = h_{r mod I}
    down = (qd, _bf16(np.ones((H, 1), np.float32)), _bf16(np.zeros((H, 1), np.float32)))
    out = oracle.expert_ffn(x, gate, up, down)
    want = 2.0 / (1.0 + math.exp(-1.0))          # silu(1) * 2 (swapped would be silu(2))
    np.testing.assert_allclose(out, want, rtol=1e-15)
    assert abs(want - 2.0 / (1.0 + math.exp(-2.0))) > 0.1


def test_expert_ffn_down_not_transposed():
    H, I = 128, 64
    x = np.zeros(H, np.uint16)
    x[0] = _bf16([1.0])[0]
    gate = _const_mat(I, H, 1, scale=4.0)        # g = 4 for every n
    qu = np.zeros((I, H), np.uint8)
    qu[:, 0] = np.arange(I) % 16                 # u_n = n mod 16
    up = (qu, _bf16(np.ones((I, H // 64), np.float32)), _bf16(np.zeros((I, H // 64), np.float32)))
    qd = np.zeros((H, I), np.uint8)
    qd[7, 3] = 1                                 # only d_7 = h_3
    down = (qd, _bf16(np.ones((H, 1), np.float32)), _bf16(np.zeros((H, 1), np.float32)))
    out = oracle.expert_ffn(x, gate, up, down)
    want = np.zeros(H)
    want[7] = 4.0 / (1.0 + math.exp(-4.0)) * 3.0
    np.testing.assert_allclose(out, want, rtol=1e-15, atol=0)


def test_expert_ffn_zero_input_is_zero():
    _, w, _ = synth.generate("tiny_t32", with_x=False)
    out = oracle.expert_ffn(np.zeros(w.H, np.uint16), w.expert(3, "gate"),
                            w.expert(3, "up"), w.expert(3, "down"))
    assert (out == 0.0).all()


# ---------------------------------------------------------------- whole layer

@pytest.fixture(scope="module")
def tiny():
    return synth.generate("tiny_t32", T=6)


def test_layer_dense_masked_equals_sparse(tiny):
    _, w, x = tiny
    sparse = oracle.layer(x, w)["y"]
    dense = oracle.layer_dense_masked(x, w)
    scale = np.abs(dense).max()
    assert np.abs(sparse - dense).max() <= 1e-12 * scale


def test_layer_zero_input_is_zero(tiny):
    _, w, _ = tiny
    r = oracle.layer(np.zeros((2, w.H), np.uint16), w)
    assert (r["y"] == 0.0).all()
    assert (r["idx"] == np.arange(8)).all() and (r["w"] == np.float32(0.125)).all()


def test_layer_identical_experts_is_one_mlp_plus_shared(tiny):
    _, w, x = tiny
    import copy
    w2 = copy.deepcopy(w)
    for m in synth.MATS:
        for arr in (w2.q, w2.scale, w2.bias):
            arr[m][:w.E] = arr[m][0]
    y = oracle.layer(x, w2)["y"]
    for t in range(x.shape[0]):
        want = (oracle.expert_ffn(x[t], *[w2.expert(0, m) for m in synth.MATS])
                + oracle.expert_ffn(x[t], *[w2.expert(w.E, m) for m in synth.MATS]))
        # the k weights are fp32, so they sum to one within k * 2**-24
        np.testing.assert_allclose(y[t], want, rtol=0, atol=8 * 2.0 ** -24 * np.abs(want).max() * 2)


def test_layer_routed_zero_leaves_shared_only(tiny):
    _, w, x = tiny
    import copy
    w2 = copy.deepcopy(w)
    w2.q["down"][:w.E] = 8                       # (8 - 8) * s = 0 for every routed expert
    y = oracle.layer(x, w2)["y"]
    for t in range(x.shape[0]):
        want = oracle.expert_ffn(x[t], *[w2.expert(w.E, m) for m in synth.MATS])
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=0)


def test_layer_token_subset_matches_full(tiny):
    _, w, x = tiny
    full = oracle.layer(x, w)
    sub = oracle.layer(x, w, tokens=[4, 1])
    assert np.array_equal(sub["y"], full["y"][[4, 1]])
    assert np.array_equal(sub["idx"], full["idx"][[4, 1]])


def _np_dequant(q, s, b):
    sf = synth.bf16_bits_to_f32(s).astype(np.float64)
    bf = synth.bf16_bits_to_f32(b).astype(np.float64)
    return q.astype(np.float64) * np.repeat(sf, 64, axis=1) + np.repeat(bf, 64, axis=1)


def test_layer_against_numpy_reformulation(tiny):
    # An independent vectorised formulation (numpy dense matrices, scipy expit)
    # of the same definition; it catches indexing slips in the C loops.
    _, w, x = tiny
    r = oracle.layer(x, w)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    logits = (xf @ w.router_w.astype(np.float64).T).astype(np.float32)
    assert np.array_equal(logits, r["logits"])

    def ffn(e, xv):
        Wg, Wu, Wd = (_np_dequant(*w.expert(e, m)) for m in synth.MATS)
        g, u = Wg @ xv, Wu @ xv
        return Wd @ (g * scipy.special.expit(g) * u)

    for t in range(x.shape[0]):
        want = ffn(w.E, xf[t])
        for j in range(8):
            want = want + float(r["w"][t, j]) * ffn(int(r["idx"][t, j]), xf[t])
        np.testing.assert_allclose(r["y"][t], want, rtol=1e-9, atol=1e-12)


def test_skew_bias_follows_zipf_ranks():
    _, w, _ = synth.generate("skew_t2048", with_x=False)
    ranks = np.rint(np.exp(-w.router_bias.astype(np.float64) / 1.1)).astype(int)
    assert sorted(ranks.tolist()) == list(range(1, 257))
