"""Shared helpers for the GPU parity tests (imported by tests, not collected).

The HIP path is compared with the CPU oracle on the same seeded inputs.

Layer outputs: relative L2 error <= 5e-3 and max abs error <= 3e-2 * max|ref|
over the compared tokens (y is bf16; the oracle is double).

Routing: the GPU computes fp32 router logits on the matrix cores, the oracle
sums in double and rounds once, so logits agree within a small bound but not
bit for bit. Where a token's k-th and (k+1)-th oracle logits are closer than
twice that bound, both selections are correct results; for such a token the
GPU's selection is accepted if it equals the oracle's or the oracle's with the
k-th and (k+1)-th experts swapped, and y is compared with the oracle's output
for that same selection (computed by the oracle from its own logits).
"""
from __future__ import annotations

import numpy as np

import oracle
from int4_grouped_gemm_router_amd import synth

REL_L2 = 5e-3
MAX_ABS_FRAC = 3e-2
LOGIT_TOL_FRAC = 2.0 ** -18   # |gpu - oracle| <= this * sum_h |x_h * Wr_eh|


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def assert_y_close(gpu_y, ref_y, what=""):
    gpu_y = np.asarray(gpu_y, np.float64)
    ref_y = np.asarray(ref_y, np.float64)
    assert np.isfinite(gpu_y).all(), f"{what}: non-finite outputs"
    r = rel_l2(gpu_y, ref_y)
    m = float(np.abs(gpu_y - ref_y).max()) if gpu_y.size else 0.0
    lim = MAX_ABS_FRAC * float(np.abs(ref_y).max()) if ref_y.size else 0.0
    assert r <= REL_L2, f"{what}: relative L2 error {r:.3e} > {REL_L2}"
    assert m <= lim, f"{what}: max abs error {m:.3e} > {lim:.3e}"
    return r, m


def logit_bound(x_bits, wr, rows=None):
    """Per (token, expert) tolerance for fp32 router logits."""
    xf = np.abs(synth.bf16_bits_to_f32(x_bits if rows is None else x_bits[rows]).astype(np.float64))
    return LOGIT_TOL_FRAC * (xf @ np.abs(wr.astype(np.float64)).T) + 1e-30


def check_layer(x, w, gpu_y, gpu_logits, gpu_idx, gpu_w, tokens=None, k=8, nthreads=0):
    """Compare GPU layer results on `tokens` (all when None) with the oracle.

    gpu_* arrays are indexed by token over the whole batch. Returns a summary dict.
    """
    T = x.shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    ref = oracle.layer(x, w, k=k, tokens=toks, nthreads=nthreads)
    tol = logit_bound(x, w.router_w, toks)
    dl = np.abs(gpu_logits[toks].astype(np.float64) - ref["logits"].astype(np.float64))
    assert (dl <= tol).all(), f"router logits: max |d|/bound = {(dl / tol).max():.3f}"
    # gap between rank k-1 and rank k of the oracle logits
    srt = -np.sort(-ref["logits"].astype(np.float64), axis=1)
    gap = srt[:, k - 1] - srt[:, k]
    ambiguous = gap <= 2.0 * tol.max(axis=1)
    y_ref = ref["y"].copy()
    w_ref = ref["w"].copy()
    idx_ref = ref["idx"].copy()
    n_alt = 0
    alt_rows = np.nonzero(ambiguous)[0]
    alt = oracle.layer(x, w, k=k, tokens=toks[alt_rows], alt_swap=True) if alt_rows.size else None
    for i, t in enumerate(toks):
        g = set(int(e) for e in gpu_idx[t])
        if g == set(int(e) for e in idx_ref[i]):
            continue
        assert ambiguous[i], f"token {t}: GPU experts {sorted(g)} != oracle {sorted(idx_ref[i])}"
        j = int(np.nonzero(alt_rows == i)[0][0])
        assert g == set(int(e) for e in alt["idx"][j]), f"token {t}: selection is neither valid choice"
        y_ref[i], w_ref[i], idx_ref[i] = alt["y"][j], alt["w"][j], alt["idx"][j]
        n_alt += 1
    # weights per selected expert (slot order may differ on near-ties inside the top k)
    for i, t in enumerate(toks):
        gw = dict(zip(gpu_idx[t].tolist(), gpu_w[t].tolist()))
        rw = dict(zip(idx_ref[i].tolist(), w_ref[i].tolist()))
        for e, v in rw.items():
            assert abs(gw[e] - v) <= 1e-5 * max(abs(v), 1e-3), f"token {t} expert {e}: weight {gw[e]} vs {v}"
    r, m = assert_y_close(synth.bf16_bits_to_f32(gpu_y[toks]), y_ref, "layer output")
    return dict(rel_l2=r, max_abs=m, ambiguous=int(ambiguous.sum()), alt_used=n_alt,
                logit_err=float((dl / tol).max()) * LOGIT_TOL_FRAC)


def check_route_meta(meta, idx, E, k, BM):
    """Structural invariants of routing metadata for the selections `idx`."""
    T = idx.shape[0]
    flat = idx.reshape(-1)
    assert np.array_equal(meta["hist"], np.bincount(flat, minlength=E)[:E])
    assert int(meta["hist"].sum()) == k * T
    assert np.array_equal(meta["offsets"], np.concatenate([[0], np.cumsum(meta["hist"])]))
    assert np.array_equal(meta["perm"], np.argsort(flat, kind="stable"))
    assert np.array_equal(meta["inv_perm"][meta["perm"]], np.arange(k * T))
    assert meta["num_blocks"] == sum(-(-int(c) // BM) for c in meta["hist"])
