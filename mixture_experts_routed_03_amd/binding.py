"""Thin ctypes binding of libmoe.so (the C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and the stream; it is imported before
the library is loaded so that libmoe binds to the HIP runtime torch already
loaded (one runtime per process).

The functions carry the C names (``moe_plan_create``, ``moe_route``,
``moe_expert_fwd``, ``moe_combine``, ``moe_expert_bwd``, ...) and take torch
tensors / ints; ``MoeLayer`` bundles a plan with caller-owned buffers
allocated through torch.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime first)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

PREC = {"f32": 0, "bf16": 1, "mxfp8": 2, "mxfp4": 3}
DTYPE = {"f32": 0, "bf16": 1}
STATUS_BAD_ID = 0x1
STATUS_PAD_SCORE = 0x2
STATUS_ARENA = 0x4
STATUS_NULL_INPUT = 0x8
STATUS_SYNC_TIMEOUT = 0x10
BWD_ACCUMULATE_DX = 0x1
BWD_ACCUMULATE_DW = 0x2
BWD_MEGA = 0x4
_ERRORS = {1: "MOE_ERR_ARG", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_UNSUPPORTED",
           4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_ERRORS.get(code, code)}")
        self.code = code


class moe_desc(ctypes.Structure):
    _fields_ = [("t_max", ctypes.c_int64), ("d", ctypes.c_int32), ("f", ctypes.c_int32),
                ("e", ctypes.c_int32), ("k", ctypes.c_int32), ("prec", ctypes.c_int32),
                ("dw_dtype", ctypes.c_int32), ("training", ctypes.c_int32),
                ("max_layers", ctypes.c_int32), ("arena_budget", ctypes.c_int64),
                ("swiglu_limit", ctypes.c_float), ("mx_w1x32", ctypes.c_int32),
                ("hot_tiles", ctypes.c_int32)]


class moe_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("route_ws", "scratch", "h3_slots", "arena", "layer_state_max",
                 "q13", "s13", "q2", "s2")]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w13", "w2", "q13", "s13", "q2", "s2")]


class moe_grads(ctypes.Structure):
    _fields_ = [("dx", ctypes.c_void_p), ("dw13", ctypes.c_void_p), ("dw2", ctypes.c_void_p),
                ("dscores", ctypes.c_void_p)]


_P = ctypes.c_void_p
_SIGS = {
    "moe_plan_create": [ctypes.POINTER(moe_desc), ctypes.POINTER(_P)],
    "moe_plan_sizes": [_P, ctypes.POINTER(moe_sizes)],
    "moe_plan_explain": [_P, ctypes.c_char_p, ctypes.c_size_t],
    "moe_plan_destroy": [_P],
    "moe_prepare_weights": [_P, _P, _P, _P, _P, _P, _P, _P],
    "moe_route": [_P, ctypes.c_int64, _P, _P, _P],
    "moe_expert_fwd": [_P, ctypes.c_int32, _P, _P, ctypes.POINTER(moe_weights), _P, _P, _P, _P],
    "moe_expert_fwd_mega": [_P, ctypes.c_int32, _P, _P, ctypes.POINTER(moe_weights), _P, _P, _P,
                            _P],
    "moe_combine": [_P, _P, _P, _P, _P, _P, _P],
    "moe_expert_fwd_fused": [_P, _P, _P, _P, ctypes.POINTER(moe_weights), _P, _P, _P, _P, _P],
    "moe_expert_fwd_fused_noalloc": [_P, _P, _P, _P, ctypes.POINTER(moe_weights), _P, _P, _P],
    "moe_expert_bwd": [_P, ctypes.c_int32, _P, _P, _P, _P, ctypes.POINTER(moe_weights), _P, _P,
                       _P, ctypes.POINTER(moe_grads), ctypes.c_uint32, _P],
    "moe_read_status": [_P, ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_int32), _P],
    "moe_arena_reset": [_P, _P, _P],
    "moe_route_readback": [_P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(ctypes.c_int32), _P],
    "moe_saved_ptrs": [_P, _P, ctypes.POINTER(_P), ctypes.POINTER(_P), _P],
    "moe_mx_quantize": [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P],
    "moe_timing_enable": [_P, ctypes.c_int32],
    "moe_timing_flush": [_P, _P, ctypes.c_size_t],
    "moe_timing_read": [_P, ctypes.c_int32, ctypes.c_char_p, ctypes.c_size_t,
                        ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)],
}
EXPORTED = tuple(_SIGS)

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_routed_03_amd.build` (there is no "
                               "CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = None if name == "moe_plan_destroy" else ctypes.c_int
        _lib = L
    return _lib


def _check(code: int, what: str):
    if code != 0:
        raise MoeError(code, what)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------------ C entry points

HOT_TILES = {"auto": 0, "always": 1, "never": 2}


def moe_plan_create(t_max, d, f, e, k, prec="bf16", dw_dtype=None, training=False,
                    max_layers=1, arena_budget=0, swiglu_limit=0.0, mx_w1x32=False,
                    hot_tiles="auto"):
    if dw_dtype is None:
        dw_dtype = "f32" if prec == "f32" else "bf16"
    ht = HOT_TILES[hot_tiles] if isinstance(hot_tiles, str) else int(hot_tiles)
    desc = moe_desc(int(t_max), int(d), int(f), int(e), int(k), PREC[prec], DTYPE[dw_dtype],
                    int(bool(training)), int(max_layers), int(arena_budget),
                    float(swiglu_limit), int(bool(mx_w1x32)), ht)
    h = _P()
    _check(lib().moe_plan_create(ctypes.byref(desc), ctypes.byref(h)), "moe_plan_create")
    return h


def moe_plan_sizes(plan) -> dict:
    s = moe_sizes()
    _check(lib().moe_plan_sizes(plan, ctypes.byref(s)), "moe_plan_sizes")
    return {n: getattr(s, n) for n, _ in moe_sizes._fields_}


def moe_plan_explain(plan) -> str:
    buf = ctypes.create_string_buffer(4096)
    _check(lib().moe_plan_explain(plan, buf, 4096), "moe_plan_explain")
    return buf.value.decode()


def moe_plan_destroy(plan):
    lib().moe_plan_destroy(plan)


def moe_route(plan, T, ids, route_ws, stream=None):
    _check(lib().moe_route(plan, int(T), _ptr(ids), _ptr(route_ws), _stream(stream)), "moe_route")


def _weights(w13, w2, q13=None, s13=None, q2=None, s2=None):
    return moe_weights(_ptr(w13), _ptr(w2), _ptr(q13), _ptr(s13), _ptr(q2), _ptr(s2))


def moe_expert_fwd(plan, layer, route_ws, x, weights, h3_slots, arena, scratch, stream=None):
    w = weights if isinstance(weights, moe_weights) else _weights(*weights)
    _check(lib().moe_expert_fwd(plan, int(layer), _ptr(route_ws), _ptr(x), ctypes.byref(w),
                                _ptr(h3_slots), _ptr(arena), _ptr(scratch), _stream(stream)),
           "moe_expert_fwd")


def moe_expert_fwd_mega(plan, layer, route_ws, x, weights, h3_slots, arena, scratch,
                        stream=None):
    w = weights if isinstance(weights, moe_weights) else _weights(*weights)
    _check(lib().moe_expert_fwd_mega(plan, int(layer), _ptr(route_ws), _ptr(x), ctypes.byref(w),
                                     _ptr(h3_slots), _ptr(arena), _ptr(scratch),
                                     _stream(stream)), "moe_expert_fwd_mega")


def moe_combine(plan, route_ws, scores, h3_slots, y_addend, y, stream=None):
    _check(lib().moe_combine(plan, _ptr(route_ws), _ptr(scores), _ptr(h3_slots), _ptr(y_addend),
                             _ptr(y), _stream(stream)), "moe_combine")


def moe_expert_fwd_fused(plan, route_ws, x, scores, weights, y32, y_addend, y, scratch,
                         stream=None):
    w = _weights(*weights)
    _check(lib().moe_expert_fwd_fused(plan, _ptr(route_ws), _ptr(x), _ptr(scores),
                                      ctypes.byref(w), _ptr(y32), _ptr(y_addend), _ptr(y),
                                      _ptr(scratch), _stream(stream)), "moe_expert_fwd_fused")


def moe_expert_fwd_fused_noalloc(plan, route_ws, x, scores, weights, y_addend, y, stream=None):
    w = _weights(*weights)
    _check(lib().moe_expert_fwd_fused_noalloc(plan, _ptr(route_ws), _ptr(x), _ptr(scores),
                                              ctypes.byref(w), _ptr(y_addend), _ptr(y),
                                              _stream(stream)), "moe_expert_fwd_fused_noalloc")


def moe_expert_bwd(plan, layer, route_ws, x, scores, dy, weights, h3_slots, arena, scratch,
                   dx, dw13, dw2, dscores=None, flags=0, stream=None):
    w = weights if isinstance(weights, moe_weights) else _weights(*weights)
    g = moe_grads(_ptr(dx), _ptr(dw13), _ptr(dw2), _ptr(dscores))
    _check(lib().moe_expert_bwd(plan, int(layer), _ptr(route_ws), _ptr(x), _ptr(scores), _ptr(dy),
                                ctypes.byref(w), _ptr(h3_slots), _ptr(arena), _ptr(scratch),
                                ctypes.byref(g), int(flags), _stream(stream)), "moe_expert_bwd")


def moe_read_status(route_ws, stream=None):
    st = ctypes.c_uint32()
    rp = ctypes.c_int32()
    _check(lib().moe_read_status(_ptr(route_ws), ctypes.byref(st), ctypes.byref(rp),
                                 _stream(stream)), "moe_read_status")
    return st.value, rp.value


def moe_arena_reset(plan, arena, stream=None):
    _check(lib().moe_arena_reset(plan, _ptr(arena), _stream(stream)), "moe_arena_reset")


def moe_route_readback(plan, route_ws, T, E, K, stream=None) -> dict:
    import numpy as np
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    poffsets = np.zeros(E + 1, np.int32)
    sorted_route = np.zeros(max(1, T * K), np.int32)
    route_to_row = np.zeros(max(1, T * K), np.int32)
    R = ctypes.c_int32()
    c_i32 = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    _check(lib().moe_route_readback(plan, _ptr(route_ws), c_i32(counts), c_i32(offsets),
                                    c_i32(poffsets), c_i32(sorted_route), c_i32(route_to_row),
                                    ctypes.byref(R), _stream(stream)), "moe_route_readback")
    return dict(counts=counts, offsets=offsets, poffsets=poffsets,
                sorted_route=sorted_route[:R.value], route_to_row=route_to_row[:T * K], R=R.value)


def moe_saved_ptrs(plan, route_ws, stream=None):
    xr, h1 = _P(), _P()
    _check(lib().moe_saved_ptrs(plan, _ptr(route_ws), ctypes.byref(xr), ctypes.byref(h1),
                                _stream(stream)), "moe_saved_ptrs")
    return xr.value, h1.value


def moe_prepare_weights(plan, w13, w2, q13, s13, q2, s2, stream=None):
    _check(lib().moe_prepare_weights(plan, _ptr(w13), _ptr(w2), _ptr(q13), _ptr(s13), _ptr(q2),
                                     _ptr(s2), _stream(stream)), "moe_prepare_weights")


def moe_mx_quantize(plan, route_ws, src, n, kind, q, sc, stream=None):
    _check(lib().moe_mx_quantize(plan, _ptr(route_ws), _ptr(src), int(n), int(kind), _ptr(q),
                                 _ptr(sc), _stream(stream)), "moe_mx_quantize")


def moe_timing_enable(plan, enable=True):
    _check(lib().moe_timing_enable(plan, int(bool(enable))), "moe_timing_enable")


def moe_timing_flush(plan, buf, nbytes=None):
    """Benchmark only: write ``buf`` (a device tensor; None = off) before each
    timed kernel, outside its events (see moe.h)."""
    n = 0 if buf is None else (int(nbytes) if nbytes is not None
                               else buf.numel() * buf.element_size())
    _check(lib().moe_timing_flush(plan, _ptr(buf), n), "moe_timing_flush")


def moe_timing_read(plan) -> dict:
    """{kernel name: (total ms, launches)} accumulated since timing was enabled."""
    out = {}
    i = 0
    name = ctypes.create_string_buffer(64)
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    while lib().moe_timing_read(plan, i, name, 64, ctypes.byref(ms), ctypes.byref(n)) == 0:
        out[name.value.decode()] = (ms.value, n.value)
        i += 1
    return out


# ------------------------------------------------------------------ convenience

def _bytes(n, device):
    return torch.empty(max(int(n), 256), dtype=torch.uint8, device=device)


class MoeLayer:
    """A plan plus its caller-owned buffers (allocated through torch).

    One instance per layer shape; ``route_ws`` and ``h3_slots`` can be
    allocated per layer with ``new_layer_buffers`` for multi-layer stacks.
    """

    def __init__(self, T_max, D, F, E, K, prec="bf16", dw_dtype=None, training=False,
                 max_layers=1, arena_budget=0, device="cuda", swiglu_limit=0.0,
                 mx_w1x32=False, hot_tiles="auto"):
        self.T_max, self.D, self.F, self.E, self.K = T_max, D, F, E, K
        self.swiglu_limit, self.mx_w1x32 = swiglu_limit, bool(mx_w1x32)
        self.prec, self.training, self.max_layers = prec, training, max_layers
        self.device = torch.device(device)
        self.act_dtype = torch.float32 if prec == "f32" else torch.bfloat16
        self.dw_dtype = (torch.float32 if (dw_dtype or ("f32" if prec == "f32" else "bf16")) == "f32"
                         else torch.bfloat16)
        self.plan = moe_plan_create(T_max, D, F, E, K, prec, dw_dtype, training, max_layers,
                                    arena_budget, swiglu_limit, mx_w1x32, hot_tiles)
        self.sizes = moe_plan_sizes(self.plan)
        self.scratch = _bytes(self.sizes["scratch"], self.device)
        self.arena = _bytes(self.sizes["arena"], self.device) if training else None
        self.route_ws, self.h3 = self.new_layer_buffers()
        self.prepared = None

    def prepare(self, w13, w2):
        """MXFP8: quantize bf16 weights once into E4M3 + E8M0 scales, in 32x32
        blocks, or (mx_w1x32 plans) 1x32 blocks along each weight row with
        the exponents grouped by 128-value stage: s13 [D/128, E*2F, 4],
        s2 [F/128, E*D, 4].  MXFP4: packed E2M1 codes q13 [E, 2F, D/2],
        q2 [E, D, F/2], 1x32 exponents grouped by 256-value stage:
        s13 [D/256, E*2F, 8], s2 [F/256, E*D, 8]."""
        E, D, F = self.E, self.D, self.F
        u8 = dict(dtype=torch.uint8, device=self.device)
        if self.prec == "mxfp4":
            q13 = torch.empty((E, 2 * F, D // 2), **u8)
            q2 = torch.empty((E, D, F // 2), **u8)
            s13 = torch.empty((D // 256, E * 2 * F, 8), **u8)
            s2 = torch.empty((F // 256, E * D, 8), **u8)
            moe_prepare_weights(self.plan, w13, w2, q13, s13, q2, s2)
            self.prepared = (q13, s13, q2, s2)
            return self.prepared
        q13 = torch.empty((E, 2 * F, D), **u8)
        q2 = torch.empty((E, D, F), **u8)
        if self.mx_w1x32:
            s13 = torch.empty((D // 128, E * 2 * F, 4), **u8)
            s2 = torch.empty((F // 128, E * D, 4), **u8)
        else:
            s13 = torch.empty((E, 2 * F // 32, D // 32), **u8)
            s2 = torch.empty((E, D // 32, F // 32), **u8)
        moe_prepare_weights(self.plan, w13, w2, q13, s13, q2, s2)
        self.prepared = (q13, s13, q2, s2)
        return self.prepared

    def _w(self, w13, w2, prepared=None):
        prep = prepared if prepared is not None else self.prepared
        if self.prec in ("mxfp8", "mxfp4"):
            if prep is None:
                raise RuntimeError("block-scaled layer: call prepare(w13, w2) first")
            return (w13, w2) + tuple(prep)
        return (w13, w2)

    def new_layer_buffers(self):
        route_ws = _bytes(self.sizes["route_ws"], self.device)
        h3 = torch.empty((self.T_max * self.K, self.D), dtype=self.act_dtype, device=self.device)
        return route_ws, h3

    def explain(self) -> str:
        return moe_plan_explain(self.plan)

    def route(self, ids, route_ws=None):
        T = ids.shape[0]
        moe_route(self.plan, T, ids, self.route_ws if route_ws is None else route_ws)

    def forward(self, x, w13, w2, layer=0, route_ws=None, h3=None, prepared=None):
        moe_expert_fwd(self.plan, layer, self.route_ws if route_ws is None else route_ws, x,
                       self._w(w13, w2, prepared), self.h3 if h3 is None else h3, self.arena,
                       self.scratch)

    def forward_mega(self, x, w13, w2, layer=0, route_ws=None, h3=None, prepared=None):
        """The expert forward as one fused (Mega) launch; same outputs as forward."""
        moe_expert_fwd_mega(self.plan, layer, self.route_ws if route_ws is None else route_ws, x,
                            self._w(w13, w2, prepared), self.h3 if h3 is None else h3, self.arena,
                            self.scratch)

    def combine(self, scores, y, y_addend=None, route_ws=None, h3=None):
        moe_combine(self.plan, self.route_ws if route_ws is None else route_ws, scores,
                    self.h3 if h3 is None else h3, y_addend, y)

    def forward_fused(self, x, w13, w2, scores, y, y_addend=None, y32=None, route_ws=None,
                      prepared=None):
        """Inference forward with the combine fused into the W2 epilogue
        (fp32 atomics into y32, then y); returns y32."""
        if y32 is None:
            y32 = torch.empty((x.shape[0], self.D), dtype=torch.float32, device=self.device)
        moe_expert_fwd_fused(self.plan, self.route_ws if route_ws is None else route_ws, x, scores,
                             self._w(w13, w2, prepared), y32, y_addend, y, self.scratch)
        return y32

    def backward(self, x, scores, dy, w13, w2, dx, dw13, dw2, dscores=None, layer=0, flags=0,
                 route_ws=None, h3=None, prepared=None):
        moe_expert_bwd(self.plan, layer, self.route_ws if route_ws is None else route_ws, x,
                       scores, dy, self._w(w13, w2, prepared), self.h3 if h3 is None else h3,
                       self.arena, self.scratch, dx, dw13, dw2, dscores, flags)

    def quantize(self, src, kind, route_ws=None):
        """Block-scaled codes of bf16 rows src [R, n]: kind 0 = MXFP8 1x32
        row blocks, 1 = MXFP8 per-expert column bundles, 2 = MXFP4 1x32 row
        blocks (packed E2M1) (see moe_mx_quantize)."""
        n = src.shape[1]
        rb = self.readback(self.T_max, route_ws)
        if kind in (0, 2):
            R = src.shape[0]
            q = torch.zeros((R, n // 2 if kind == 2 else n), dtype=torch.uint8, device=self.device)
            sc = torch.zeros((R, n // 32), dtype=torch.uint8, device=self.device)
        else:
            Rp = int(rb["poffsets"][-1])
            q = torch.zeros((max(1, n * Rp),), dtype=torch.uint8, device=self.device)
            sc = torch.zeros((max(1, n * Rp // 32),), dtype=torch.uint8, device=self.device)
        moe_mx_quantize(self.plan, self.route_ws if route_ws is None else route_ws, src, n, kind,
                        q, sc)
        return q, sc, rb

    def status(self, route_ws=None):
        return moe_read_status(self.route_ws if route_ws is None else route_ws)

    def readback(self, T, route_ws=None):
        return moe_route_readback(self.plan, self.route_ws if route_ws is None else route_ws, T,
                                  self.E, self.K)

    def saved_ptrs(self, route_ws=None):
        return moe_saved_ptrs(self.plan, self.route_ws if route_ws is None else route_ws)

    def view(self, ptr, shape, dtype):
        """A tensor view of device memory at ``ptr`` inside this layer's
        scratch or arena buffer (for inspecting saved state)."""
        n = 1
        for d in shape:
            n *= int(d)
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        for buf in (self.scratch, self.arena):
            if buf is None:
                continue
            off = ptr - buf.data_ptr()
            if 0 <= off and off + nbytes <= buf.numel():
                return buf[off:off + nbytes].view(dtype).view(*shape)
        raise ValueError("pointer is not inside scratch or arena")

    def __del__(self):
        try:
            if getattr(self, "plan", None) is not None and _lib is not None:
                moe_plan_destroy(self.plan)
                self.plan = None
        except Exception:
            pass


class MoeStack:
    """L routed-expert layers of one shape sharing one plan, one arena and
    one scratch buffer: forwards in layer order, then backwards in reverse
    order (each backward rewinds the arena to its layer's start)."""

    def __init__(self, L, T_max, D, F, E, K, prec="mxfp8", dw_dtype=None, arena_budget=0,
                 device="cuda"):
        self.L = L
        self.layer = MoeLayer(T_max, D, F, E, K, prec, dw_dtype, training=True, max_layers=L,
                              arena_budget=arena_budget, device=device)
        self.bufs = [self.layer.new_layer_buffers() for _ in range(L)]

    def route(self, l, ids):
        self.layer.route(ids, route_ws=self.bufs[l][0])

    def forward(self, l, x, w13, w2, scores, y, prepared=None, y_addend=None, mega=False):
        rw, h3 = self.bufs[l]
        fwd = self.layer.forward_mega if mega else self.layer.forward
        fwd(x, w13, w2, layer=l, route_ws=rw, h3=h3, prepared=prepared)
        self.layer.combine(scores, y, y_addend=y_addend, route_ws=rw, h3=h3)

    def backward(self, l, x, scores, dy, w13, w2, dx, dw13, dw2, dscores=None, prepared=None,
                 flags=0):
        rw, h3 = self.bufs[l]
        self.layer.backward(x, scores, dy, w13, w2, dx, dw13, dw2, dscores, layer=l, flags=flags,
                            route_ws=rw, h3=h3, prepared=prepared)

    def status(self, l):
        return self.layer.status(route_ws=self.bufs[l][0])

    def readback(self, l, T):
        return self.layer.readback(T, route_ws=self.bufs[l][0])
