"""Thin ctypes binding of libmoe_int4.so (include/moe_int4.h).

Argument marshalling only: every step of the layer runs in the HIP library.
torch supplies device memory and the current stream; it is imported before
the library is loaded so that the library binds to the HIP runtime torch
already loaded (both carry the same soname).
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_INT4_LIB", os.path.join(HERE, "libmoe_int4.so"))
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe_int4.h")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_EBUFFER, MOE_EFORMAT = (
    0, -1, -2, -3, -4, -5, -6)
MOE_ESCRATCH = -7
NOALLOC_SCRATCH_BYTES = 320 * 1024
MODE_PREFILL, MODE_DECODE, MODE_ROUTE = 0, 1, 2
GEMM_AUTO, GEMM_EXACT, GEMM_WIDE = 0, 1, 2
HEADER_BYTES = 256

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


class MoeDims(ctypes.Structure):
    _fields_ = [("H", _i32), ("I", _i32), ("E", _i32), ("top_k", _i32), ("block_m", _i32),
                ("gemm", _i32)]


class MoeLayerWeights(ctypes.Structure):
    _fields_ = [("router_w3", _vp), ("router_w", _vp), ("router_bias", _vp),
                ("experts_gate_up", _vp), ("experts_down", _vp),
                ("shared_gate_up", _vp), ("shared_down", _vp)]


class MoeRouteOut(ctypes.Structure):
    _fields_ = [("topk_idx", _vp), ("topk_w", _vp), ("hist", _vp), ("offsets", _vp),
                ("perm", _vp), ("inv_perm", _vp), ("block_map", _vp), ("num_blocks", _vp)]


class MoeError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


_lib = None


def header_functions():
    """Names of the functions declared in include/moe_int4.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s*([a-z_][\w]*)\s*\(", text, flags=re.M)


def lib():
    """Load libmoe_int4.so (raises if it has not been built: there is no fallback)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (binds the library to torch's HIP runtime)
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.moe_max_blocks.argtypes = [P(MoeDims), _i32]
        L.moe_max_blocks.restype = _i64
        L.moe_packed_bytes.argtypes = [_i32, _i32, _i32, _i32]
        L.moe_packed_bytes.restype = _sz
        L.pack_int4_g64.argtypes = [_vp] * 6 + [_i32, _i32, _i32, _vp, _sz]
        L.moe_router_packed_bytes.argtypes = [_i32, _i32]
        L.moe_router_packed_bytes.restype = _sz
        L.pack_router_bf16x3.argtypes = [_vp, _i32, _i32, _vp, _sz]
        L.moe_workspace_bytes.argtypes = [P(MoeDims), _i32, _i32, P(_sz)]
        L.moe_route.argtypes = [P(MoeDims), _vp, _i32, P(MoeRouteOut), _vp, _sz, _vp]
        L.moe_prefill_layer.argtypes = [P(MoeDims), P(MoeLayerWeights), _vp, _vp, _i32, _i32,
                                        _vp, P(MoeRouteOut), _vp, _sz, _vp]
        L.moe_decode_layer.argtypes = [P(MoeDims), P(MoeLayerWeights), _vp, _vp, _i32, _vp,
                                       P(MoeRouteOut), _vp, _sz, _vp]
        L.moe_prefill_layer_profiled.argtypes = L.moe_prefill_layer.argtypes + [_vp, _i32]
        L.moe_prefill_layer_host_routed.argtypes = [P(MoeDims), P(MoeLayerWeights), _vp, _vp, _i32,
                                                    _i32, _vp, _sz, _vp]
        L.moe_unfused_weight_bytes.argtypes = [P(MoeDims), P(_sz)]
        L.moe_prefill_layer_unfused.argtypes = [P(MoeDims), P(MoeLayerWeights), _vp, _vp, _i32, _i32,
                                                _vp, _sz, _vp, _sz, _vp]
        L.moe_decode_layer_profiled.argtypes = L.moe_decode_layer.argtypes + [_vp, _i32]
        L.moe_decode_layer_noalloc.argtypes = [P(MoeDims), P(MoeLayerWeights), _vp, _vp, _i32, _vp,
                                               P(MoeRouteOut), _vp]
        L.moe_ceiling_read.argtypes = [_vp, _sz, _vp, _vp]
        L.moe_ceiling_mfma.argtypes = [_i32, _i32, _vp, _vp, P(ctypes.c_double), _vp]
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_test_dequant.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp]
        for name in ("pack_int4_g64", "pack_router_bf16x3", "moe_workspace_bytes", "moe_route",
                     "moe_prefill_layer", "moe_decode_layer", "moe_test_dequant",
                     "moe_prefill_layer_profiled", "moe_decode_layer_profiled",
                     "moe_prefill_layer_host_routed", "moe_unfused_weight_bytes",
                     "moe_prefill_layer_unfused", "moe_ceiling_read", "moe_ceiling_mfma",
                     "moe_decode_layer_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def _check(code, what):
    if code != MOE_OK:
        raise MoeError(code, what)


def dims(H, I, E=256, top_k=8, block_m=32, gemm=GEMM_AUTO) -> MoeDims:
    return MoeDims(H, I, E, top_k, block_m, gemm)


def _ptr(t):
    """Device or host address of a torch tensor / numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        assert t.flags["C_CONTIGUOUS"]
        return t.ctypes.data
    assert t.is_contiguous(), "tensors passed to the library must be contiguous"
    return t.data_ptr()


def _stream(stream, device=None):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream(device).cuda_stream


# ------------------------------------------------------------------ packing (host)

def moe_max_blocks(d: MoeDims, T: int) -> int:
    v = lib().moe_max_blocks(ctypes.byref(d), T)
    if v < 0:
        raise MoeError(int(v), "moe_max_blocks")
    return int(v)


def moe_packed_bytes(count, N, K, paired) -> int:
    return int(lib().moe_packed_bytes(count, N, K, int(paired)))


def pack_int4_g64(q0, s0, b0, q1=None, s1=None, b1=None) -> np.ndarray:
    """Pack [count][N][K] codes with [count][N][K/64] bf16 scales/biases (host)."""
    q0 = np.ascontiguousarray(q0, np.uint8)
    count, N, K = q0.shape
    arrs = [q0, np.ascontiguousarray(s0, np.uint16), np.ascontiguousarray(b0, np.uint16)]
    paired = q1 is not None
    if paired:
        arrs += [np.ascontiguousarray(q1, np.uint8), np.ascontiguousarray(s1, np.uint16),
                 np.ascontiguousarray(b1, np.uint16)]
    else:
        arrs += [None, None, None]
    nbytes = moe_packed_bytes(count, N, K, paired)
    if nbytes == 0:
        raise MoeError(MOE_EUNSUPPORTED, "moe_packed_bytes")
    out = np.empty(nbytes, np.uint8)
    _check(lib().pack_int4_g64(*[_ptr(a) for a in arrs], count, N, K, _ptr(out), nbytes),
           "pack_int4_g64")
    return out


def pack_router_bf16x3(wr) -> np.ndarray:
    wr = np.ascontiguousarray(wr, np.float32)
    E, H = wr.shape
    nbytes = int(lib().moe_router_packed_bytes(E, H))
    if nbytes == 0:
        raise MoeError(MOE_EUNSUPPORTED, "moe_router_packed_bytes")
    out = np.empty(nbytes, np.uint8)
    _check(lib().pack_router_bf16x3(_ptr(wr), E, H, _ptr(out), nbytes), "pack_router_bf16x3")
    return out


def moe_workspace_bytes(d: MoeDims, T_chunk: int, mode: int) -> int:
    n = _sz(0)
    _check(lib().moe_workspace_bytes(ctypes.byref(d), T_chunk, mode, ctypes.byref(n)),
           "moe_workspace_bytes")
    return int(n.value)


# ------------------------------------------------------------------ device buffers

class DeviceWeights:
    """Packed layer weights resident on the GPU (torch uint8 tensors)."""

    def __init__(self, d: MoeDims, tensors: dict):
        self.dims = d
        self.t = tensors
        self.struct = MoeLayerWeights(
            _ptr(tensors["router_w3"]), _ptr(tensors["router_w"]), _ptr(tensors.get("router_bias")),
            _ptr(tensors["experts_gate_up"]), _ptr(tensors["experts_down"]),
            _ptr(tensors["shared_gate_up"]), _ptr(tensors["shared_down"]))

    @staticmethod
    def pack_host(w):
        """Host blobs of a logical layer (anything with the synth.LayerWeights fields)."""
        E = w.E
        blobs = {
            "router_w3": pack_router_bf16x3(w.router_w),
            "router_w": np.ascontiguousarray(w.router_w, np.float32),
            "experts_gate_up": pack_int4_g64(w.q["gate"][:E], w.scale["gate"][:E], w.bias["gate"][:E],
                                             w.q["up"][:E], w.scale["up"][:E], w.bias["up"][:E]),
            "experts_down": pack_int4_g64(w.q["down"][:E], w.scale["down"][:E], w.bias["down"][:E]),
            "shared_gate_up": pack_int4_g64(w.q["gate"][E:], w.scale["gate"][E:], w.bias["gate"][E:],
                                            w.q["up"][E:], w.scale["up"][E:], w.bias["up"][E:]),
            "shared_down": pack_int4_g64(w.q["down"][E:], w.scale["down"][E:], w.bias["down"][E:]),
        }
        if w.router_bias is not None:
            blobs["router_bias"] = np.ascontiguousarray(w.router_bias, np.float32)
        return blobs

    @classmethod
    def upload(cls, d: MoeDims, host_blobs: dict, device="cuda"):
        import torch
        t = {k: torch.from_numpy(v).to(device) for k, v in host_blobs.items()}
        return cls(d, t)

    @classmethod
    def from_logical(cls, w, device="cuda"):
        d = dims(w.H, w.I, w.E)
        return cls.upload(d, cls.pack_host(w), device)

    def clone(self):
        """A second copy at new device addresses (same contents)."""
        return DeviceWeights(self.dims, {k: v.clone() for k, v in self.t.items()})

    @property
    def expert_bytes_read(self):
        return sum(v.numel() * v.element_size() for v in self.t.values())


class RouteBuffers:
    """Device buffers for moe_route_out sized for T tokens."""

    def __init__(self, d: MoeDims, T: int, device="cuda"):
        import torch
        k = d.top_k
        mb = moe_max_blocks(d, T)
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.full((T, k), -1, **i32)
        self.topk_w = torch.zeros((T, k), dtype=torch.float32, device=device)
        self.hist = torch.full((d.E,), -1, **i32)
        self.offsets = torch.full((d.E + 1,), -1, **i32)
        self.perm = torch.full((T * k,), -1, **i32)
        self.inv_perm = torch.full((T * k,), -1, **i32)
        self.block_map = torch.full((mb, 3), -1, **i32)
        self.num_blocks = torch.full((1,), -1, **i32)
        self.struct = MoeRouteOut(*[_ptr(getattr(self, f)) for f, _ in MoeRouteOut._fields_])

    def to_numpy(self):
        out = {f: getattr(self, f).cpu().numpy() for f, _ in MoeRouteOut._fields_}
        nb = int(out["num_blocks"][0])
        out["num_blocks"] = nb
        out["block_map"] = out["block_map"][:nb]
        return out


def workspace(d: MoeDims, T_chunk: int, mode: int, device="cuda"):
    import torch
    return torch.zeros(moe_workspace_bytes(d, T_chunk, mode), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points

def moe_route(d: MoeDims, logits, T: int, out: RouteBuffers, ws, stream=None):
    _check(lib().moe_route(ctypes.byref(d), _ptr(logits), T, ctypes.byref(out.struct), _ptr(ws),
                           ws.numel(), _stream(stream)), "moe_route")


def moe_prefill_layer(d: MoeDims, w: DeviceWeights, x, y, T: int, chunk_T: int = 0,
                      logits_out=None, route_out: RouteBuffers | None = None, ws=None,
                      stream=None):
    ro = ctypes.byref(route_out.struct) if route_out is not None else None
    _check(lib().moe_prefill_layer(ctypes.byref(d), ctypes.byref(w.struct), _ptr(x), _ptr(y), T,
                                   chunk_T, _ptr(logits_out), ro, _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(stream)),
           "moe_prefill_layer")


def moe_prefill_layer_host_routed(d: MoeDims, w: DeviceWeights, x, y, T: int, chunk_T: int = 0,
                                  ws=None, stream=None):
    _check(lib().moe_prefill_layer_host_routed(ctypes.byref(d), ctypes.byref(w.struct), _ptr(x),
                                               _ptr(y), T, chunk_T, _ptr(ws),
                                               0 if ws is None else ws.numel(), _stream(stream)),
           "moe_prefill_layer_host_routed")


def unfused_weights(d: MoeDims, device="cuda"):
    """Device buffer for moe_prefill_layer_unfused's bf16 weights."""
    import torch
    n = _sz(0)
    _check(lib().moe_unfused_weight_bytes(ctypes.byref(d), ctypes.byref(n)), "moe_unfused_weight_bytes")
    return torch.empty(n.value, dtype=torch.uint8, device=device)


def moe_prefill_layer_unfused(d: MoeDims, w: DeviceWeights, x, y, T: int, wbuf, chunk_T: int = 0,
                              ws=None, stream=None):
    _check(lib().moe_prefill_layer_unfused(ctypes.byref(d), ctypes.byref(w.struct), _ptr(x), _ptr(y), T,
                                           chunk_T, _ptr(wbuf), wbuf.numel(), _ptr(ws),
                                           0 if ws is None else ws.numel(), _stream(stream)),
           "moe_prefill_layer_unfused")


def moe_decode_layer(d: MoeDims, w: DeviceWeights, x, y, T: int, logits_out=None,
                     route_out: RouteBuffers | None = None, ws=None, stream=None):
    ro = ctypes.byref(route_out.struct) if route_out is not None else None
    _check(lib().moe_decode_layer(ctypes.byref(d), ctypes.byref(w.struct), _ptr(x), _ptr(y), T,
                                  _ptr(logits_out), ro, _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(stream)),
           "moe_decode_layer")


def moe_decode_layer_noalloc(d: MoeDims, w: DeviceWeights, x, y, T: int, logits_out=None,
                             route_out: RouteBuffers | None = None, stream=None):
    """moe_decode_layer on the library's static scratch (no workspace argument)."""
    ro = ctypes.byref(route_out.struct) if route_out is not None else None
    _check(lib().moe_decode_layer_noalloc(ctypes.byref(d), ctypes.byref(w.struct), _ptr(x), _ptr(y), T,
                                          _ptr(logits_out), ro, _stream(stream)),
           "moe_decode_layer_noalloc")


def _event_array(events):
    """ctypes array of raw hipEvent_t handles from torch.cuda.Event objects."""
    handles = []
    for e in events:
        if not e.cuda_event:
            e.record()          # torch creates the underlying event lazily
        handles.append(e.cuda_event)
    return (ctypes.c_void_p * len(handles))(*handles)


def moe_prefill_layer_profiled(d: MoeDims, w: DeviceWeights, x, y, T: int, chunk_T: int, events,
                               logits_out=None, route_out: RouteBuffers | None = None, ws=None,
                               stream=None):
    ro = ctypes.byref(route_out.struct) if route_out is not None else None
    arr = events if isinstance(events, ctypes.Array) else _event_array(events)
    _check(lib().moe_prefill_layer_profiled(ctypes.byref(d), ctypes.byref(w.struct), _ptr(x),
                                            _ptr(y), T, chunk_T, _ptr(logits_out), ro, _ptr(ws),
                                            0 if ws is None else ws.numel(), _stream(stream),
                                            ctypes.cast(arr, _vp), len(arr)),
           "moe_prefill_layer_profiled")


def moe_decode_layer_profiled(d: MoeDims, w: DeviceWeights, x, y, T: int, events,
                              logits_out=None, route_out: RouteBuffers | None = None, ws=None,
                              stream=None):
    ro = ctypes.byref(route_out.struct) if route_out is not None else None
    arr = events if isinstance(events, ctypes.Array) else _event_array(events)
    _check(lib().moe_decode_layer_profiled(ctypes.byref(d), ctypes.byref(w.struct), _ptr(x),
                                           _ptr(y), T, _ptr(logits_out), ro, _ptr(ws),
                                           0 if ws is None else ws.numel(), _stream(stream),
                                           ctypes.cast(arr, _vp), len(arr)),
           "moe_decode_layer_profiled")


def moe_ceiling_read(buf, sink, stream=None):
    """Enqueue one streaming read of the device buffer `buf` (measurement helper)."""
    _check(lib().moe_ceiling_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                  _stream(stream)), "moe_ceiling_read")


CEILING_MFMA_BLOCKS = 1024  # blocks of the matrix-core loop (two clock values each)


def moe_ceiling_mfma(iters: int, sink, random: bool = True, clocks=None, stream=None) -> float:
    """Enqueue the bf16 matrix-core loop (random or nearly constant operands);
    `clocks`, if given, is an int64 device tensor of 2 * CEILING_MFMA_BLOCKS
    values that receives each block's real-time and shader-clock ticks.
    Returns the launch's flop count."""
    if clocks is not None and clocks.numel() * clocks.element_size() < 16 * CEILING_MFMA_BLOCKS:
        raise ValueError("moe_ceiling_mfma: clocks needs 2 * CEILING_MFMA_BLOCKS int64 values")
    flops = ctypes.c_double(0.0)
    _check(lib().moe_ceiling_mfma(iters, int(random), _ptr(sink), _ptr(clocks), ctypes.byref(flops),
                                  _stream(stream)), "moe_ceiling_mfma")
    return flops.value


def ceiling_clock_mhz(clocks) -> float:
    """Mean shader clock of the last moe_ceiling_mfma launch that wrote `clocks`
    (shader-clock ticks over 100 MHz real-time ticks, summed over the blocks)."""
    c = clocks.view(-1, 2).cpu().double()
    return float(c[:, 1].sum() / c[:, 0].sum() * 100.0)


def moe_test_dequant(blob, count, N, K, paired, expert, out, stream=None):
    _check(lib().moe_test_dequant(_ptr(blob), count, N, K, int(paired), expert, _ptr(out),
                                  _stream(stream)), "moe_test_dequant")
