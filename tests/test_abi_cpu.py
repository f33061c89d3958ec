"""Host-side checks of the C-ABI library (no GPU needed).

- the library loads and exports every function include/moe_int4.h declares;
- the host packers round-trip: a reader written here from the documented
  layout (not the packer's code) recovers q, scale and bias exactly, and the
  three router planes add up to the fp32 router matrix exactly;
- every entry point rejects bad arguments with the documented code before
  anything would be launched (fake device addresses are never dereferenced).
"""
import ctypes

import numpy as np
import pytest

from int4_grouped_gemm_router_amd import binding as B
from int4_grouped_gemm_router_amd import synth


def test_library_exports_every_header_symbol():
    L = B.lib()
    names = B.header_functions()
    assert {"moe_route", "moe_prefill_layer", "moe_decode_layer", "pack_int4_g64"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libmoe_int4.so does not export {n}"


# ---------------------------------------------------------------- packed layout reader

def _read_packed(blob, count, N, K, paired):
    """Recover (q, scale, bias) per matrix from a blob, following the layout
    documented in csrc/layout.h: per expert nib [wt][g][half][lane][4 words],
    then sb [wt][g][c16][8 bf16] (four scales of columns 16*ct + c16, then
    their four biases); codes o at nibble (o&1)*4 + o>>1."""
    hdr = np.frombuffer(blob[:32].tobytes(), dtype=np.int32)
    assert hdr[0] == 0x4734494D and hdr[1] == 3
    assert tuple(hdr[2:6]) == (count, N, K, int(paired))
    n_eff = 2 * N if paired else N
    n_wt, G = n_eff // 64, K // 64
    nib_bytes = n_wt * G * 2048
    sb_bytes = n_wt * G * 256
    end = nib_bytes + sb_bytes
    ebytes = -(-end // 256) * 256
    nmat = 2 if paired else 1
    q = np.zeros((nmat, count, N, K), np.uint8)
    s = np.zeros((nmat, count, N, G), np.uint16)
    b = np.zeros((nmat, count, N, G), np.uint16)
    pos = np.array([(o & 1) * 4 + (o >> 1) for o in range(8)])
    for e in range(count):
        base = 256 + e * ebytes
        words = np.frombuffer(blob[base:base + nib_bytes].tobytes(), np.uint32).reshape(n_wt, G, 2, 64, 4)
        words = words.transpose(0, 1, 3, 2, 4).reshape(n_wt, G, 64, 8)
        sb = np.frombuffer(blob[base + nib_bytes:base + end].tobytes(), np.uint16).reshape(n_wt, G, 16, 8)
        for wt in range(n_wt):
            for j in range(64):
                mat, row = (((j // 16) % 2, 32 * wt + 16 * (j // 32) + j % 16) if paired
                            else (0, 64 * wt + j))
                ct, c16 = j // 16, j % 16
                s[mat, e, row] = sb[wt, :, c16, ct]
                b[mat, e, row] = sb[wt, :, c16, 4 + ct]
                for ks in range(2):
                    for kb in range(4):
                        w = words[wt, :, kb * 16 + c16, 2 * ct + ks]          # [G]
                        codes = (w[:, None] >> (4 * pos[None, :])) & 0xF      # [G, 8]
                        for g in range(G):
                            k0 = 64 * g + 32 * ks + 8 * kb
                            q[mat, e, row, k0:k0 + 8] = codes[g]
    return q, s, b


@pytest.mark.parametrize("paired,N,K,count", [(False, 64, 128, 2), (True, 32, 64, 3),
                                              (True, 128, 512, 1), (False, 256, 128, 1)])
def test_pack_int4_round_trip(paired, N, K, count):
    rng = np.random.default_rng(N + K + count)
    mats = []
    for _ in range(2 if paired else 1):
        q = rng.integers(0, 16, size=(count, N, K), dtype=np.uint8)
        s = rng.integers(0, 65536, size=(count, N, K // 64), dtype=np.uint16)
        b = rng.integers(0, 65536, size=(count, N, K // 64), dtype=np.uint16)
        mats.append((q, s, b))
    blob = B.pack_int4_g64(*mats[0], *(mats[1] if paired else (None, None, None)))
    assert blob.size == B.moe_packed_bytes(count, N, K, paired)
    q, s, b = _read_packed(blob, count, N, K, paired)
    for m, (qq, ss, bb) in enumerate(mats):
        assert np.array_equal(q[m], qq)
        assert np.array_equal(s[m], ss)
        assert np.array_equal(b[m], bb)


def test_pack_rejects_bad_codes_and_small_buffers():
    q = np.full((1, 64, 64), 16, np.uint8)
    s = np.zeros((1, 64, 1), np.uint16)
    with pytest.raises(B.MoeError) as e:
        B.pack_int4_g64(q, s, s)
    assert e.value.code == B.MOE_EFORMAT
    L = B.lib()
    out = np.zeros(16, np.uint8)
    q[:] = 1
    rc = L.pack_int4_g64(q.ctypes.data, s.ctypes.data, s.ctypes.data, None, None, None,
                         1, 64, 64, out.ctypes.data, 16)
    assert rc == B.MOE_EBUFFER
    assert B.moe_packed_bytes(1, 48, 64, 0) == 0      # N % 64 != 0 unpaired
    assert B.moe_packed_bytes(1, 64, 100, 0) == 0     # K % 64 != 0


def test_router_planes_sum_exactly():
    rng = np.random.default_rng(7)
    E, H = 128, 256
    wr = rng.normal(0, 0.02, size=(E, H)).astype(np.float32)
    wr[0, :4] = [0.0, -0.0, 1.0, -3.1415927]
    blob = B.pack_router_bf16x3(wr)
    planes = np.frombuffer(blob[256:].tobytes(), np.uint16)
    n_et, G = E // 64, H // 64
    vals = synth.bf16_bits_to_f32(planes).astype(np.float64).reshape(3, n_et, G, 4, 2, 4, 16, 8)
    # index [plane][et][g][ct][ks][kb][c16][o] -> expert 64et+16ct+c16, k 64g+32ks+8kb+o
    total = vals.sum(axis=0)                                    # [et][g][ct][ks][kb][c16][o]
    total = total.transpose(0, 2, 5, 1, 3, 4, 6).reshape(E, H)
    assert np.array_equal(total, wr.astype(np.float64))


# ---------------------------------------------------------------- argument checks

FAKE = 0x10000  # never dereferenced: every call below returns before any launch


def _route_out(d):
    return B.MoeRouteOut(*([FAKE] * 8))


def test_entry_points_reject_bad_arguments():
    L = B.lib()
    d = B.dims(2048, 512)
    bad = B.dims(2048, 512, top_k=4)
    ro = _route_out(d)
    w = B.MoeLayerWeights(*([FAKE] * 7))
    ws_need = B.moe_workspace_bytes(d, 64, B.MODE_PREFILL)
    by = ctypes.byref
    assert L.moe_route(by(d), FAKE, -1, by(ro), FAKE, 1 << 30, None) == B.MOE_EINVAL
    assert L.moe_route(by(bad), FAKE, 4, by(ro), FAKE, 1 << 30, None) == B.MOE_EUNSUPPORTED
    assert L.moe_route(by(d), FAKE, 0, by(ro), FAKE, 0, None) == B.MOE_OK
    assert L.moe_route(by(d), None, 4, by(ro), FAKE, 1 << 30, None) == B.MOE_EINVAL
    assert L.moe_route(by(d), FAKE, 4, by(ro), FAKE, 0, None) == B.MOE_EWORKSPACE
    assert L.moe_prefill_layer(by(d), by(w), FAKE, FAKE, 64, 0, None, None, FAKE, ws_need - 1,
                               None) == B.MOE_EWORKSPACE
    assert L.moe_prefill_layer(by(d), by(w), None, FAKE, 64, 0, None, None, FAKE, ws_need,
                               None) == B.MOE_EINVAL
    assert L.moe_prefill_layer(by(d), by(w), FAKE, FAKE, 0, 0, None, None, None, 0,
                               None) == B.MOE_OK
    assert L.moe_prefill_layer(by(bad), by(w), FAKE, FAKE, 64, 0, None, None, FAKE, ws_need,
                               None) == B.MOE_EUNSUPPORTED
    assert L.moe_decode_layer(by(d), by(w), FAKE, FAKE, 5, None, None, FAKE, 1 << 30,
                              None) == B.MOE_EUNSUPPORTED
    dws = B.moe_workspace_bytes(d, 1, B.MODE_DECODE)
    assert L.moe_decode_layer(by(d), by(w), FAKE, FAKE, 1, None, None, FAKE, dws - 1,
                              None) == B.MOE_EWORKSPACE
    assert L.moe_test_dequant(FAKE, 2, 64, 64, 0, 2, FAKE, None) == B.MOE_EINVAL
    for dd in (B.dims(2048, 512, E=320), B.dims(2000, 512), B.dims(2048, 100),
               B.dims(2048, 512, block_m=24), B.dims(2048, 512, block_m=64),
               B.dims(2048, 512, gemm=3), B.dims(2048, 512, gemm=-1)):
        n = ctypes.c_size_t(0)
        assert L.moe_workspace_bytes(by(dd), 64, 0, by(n)) == B.MOE_EUNSUPPORTED
    assert B.strerror(B.MOE_EWORKSPACE) == "workspace too small"
    # pair indices are 32-bit: T * top_k must stay below 2^30
    big = 1 << 27
    assert L.moe_prefill_layer(by(d), by(w), FAKE, FAKE, big, 4096, None, None, FAKE, 1 << 40,
                               None) == B.MOE_EUNSUPPORTED
    assert L.moe_route(by(d), FAKE, big, by(ro), FAKE, 1 << 40, None) == B.MOE_EUNSUPPORTED
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_bytes(by(d), big, 0, by(n)) == B.MOE_EUNSUPPORTED


def test_entry_points_reject_misaligned_pointers():
    # 16-byte vectors for activations, outputs, workspace and packed weights,
    # 4-byte words for logits and routing metadata: misaligned pointers are
    # rejected before any launch
    L = B.lib()
    d = B.dims(2048, 512)
    by = ctypes.byref
    w = B.MoeLayerWeights(*([FAKE] * 7))
    ws = B.moe_workspace_bytes(d, 64, B.MODE_PREFILL)
    dws = B.moe_workspace_bytes(d, 1, B.MODE_DECODE)
    ro = _route_out(d)

    def prefill(x=FAKE, y=FAKE, logits=None, wts=w, wsp=FAKE):
        return L.moe_prefill_layer(by(d), by(wts), x, y, 64, 0, logits, None, wsp, ws, None)

    for kw in ({"x": FAKE + 2}, {"y": FAKE + 8}, {"wsp": FAKE + 4}, {"logits": FAKE + 2}):
        assert prefill(**kw) == B.MOE_EINVAL, kw
    for i in (0, 3, 4, 5, 6):  # router_w3 and the four blobs
        fields = [FAKE] * 7
        fields[i] = FAKE + 8
        assert prefill(wts=B.MoeLayerWeights(*fields)) == B.MOE_EINVAL, i
    fields = [FAKE] * 7
    fields[2] = FAKE + 2  # router_bias
    assert prefill(wts=B.MoeLayerWeights(*fields)) == B.MOE_EINVAL
    assert L.moe_decode_layer(by(d), by(w), FAKE + 4, FAKE, 1, None, None, FAKE, dws,
                              None) == B.MOE_EINVAL
    fields = [FAKE] * 7
    fields[1] = FAKE + 4  # router_w (decode)
    assert L.moe_decode_layer(by(d), by(B.MoeLayerWeights(*fields)), FAKE, FAKE, 1, None, None,
                              FAKE, dws, None) == B.MOE_EINVAL
    rws = B.moe_workspace_bytes(d, 4, B.MODE_ROUTE)
    assert L.moe_route(by(d), FAKE + 2, 4, by(ro), FAKE, rws, None) == B.MOE_EINVAL
    bad_ro = B.MoeRouteOut(*([FAKE] * 7 + [FAKE + 1]))
    assert L.moe_route(by(d), FAKE, 4, by(bad_ro), FAKE, rws, None) == B.MOE_EINVAL
    assert L.moe_test_dequant(FAKE + 8, 2, 64, 64, 0, 0, FAKE, None) == B.MOE_EINVAL


def test_workspace_and_block_bounds():
    d = B.dims(2048, 512)
    assert B.moe_max_blocks(d, 2048) == 2048 * 8 // 32 + 256
    a = B.moe_workspace_bytes(d, 512, B.MODE_PREFILL)
    b = B.moe_workspace_bytes(d, 4096, B.MODE_PREFILL)
    assert 0 < a < b
    # the down outputs dominate: k*T*H bf16 routed rows + T*H fp32 shared rows
    assert b >= 8 * 4096 * 2048 * 2 + 4096 * 2048 * 4
    assert B.moe_workspace_bytes(d, 4, B.MODE_DECODE) > 0


def test_noalloc_decode_rejects_bad_arguments():
    # the no-allocation decode entry point checks its arguments before it
    # touches the device (its scratch address is resolved only for valid calls)
    L = B.lib()
    d = B.dims(2048, 512)
    by = ctypes.byref
    w = B.MoeLayerWeights(*([FAKE] * 7))
    f = L.moe_decode_layer_noalloc
    assert f(by(d), by(w), FAKE, FAKE, 0, None, None, None) == B.MOE_OK
    assert f(by(d), by(w), FAKE, FAKE, -1, None, None, None) == B.MOE_EINVAL
    assert f(by(d), by(w), FAKE, FAKE, 5, None, None, None) == B.MOE_EUNSUPPORTED
    assert f(by(B.dims(2048, 512, top_k=4)), by(w), FAKE, FAKE, 1, None, None, None) == B.MOE_EUNSUPPORTED
    assert f(by(d), by(w), None, FAKE, 1, None, None, None) == B.MOE_EINVAL
    assert f(by(d), by(w), FAKE + 4, FAKE, 1, None, None, None) == B.MOE_EINVAL
    assert f(by(d), None, FAKE, FAKE, 1, None, None, None) == B.MOE_EINVAL
    assert B.strerror(B.MOE_ESCRATCH).startswith("request exceeds the static scratch")


def test_noalloc_scratch_covers_every_supported_decode():
    # the static scratch is stated in the header; every supported decode call
    # (T <= 4, E <= 256, I <= 4096) fits in it, the largest needing 299,520 bytes
    hdr = open(B.HEADER).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES (320 * 1024)" in hdr
    need = max(B.moe_workspace_bytes(B.dims(H, I, E), T, B.MODE_DECODE)
               for H in (256, 4096) for I in (128, 4096) for E in (64, 256) for T in (1, 4))
    assert need == 299520 <= B.NOALLOC_SCRATCH_BYTES
