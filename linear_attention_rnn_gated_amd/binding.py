"""ctypes binding of libgdn.so (include/gdn.h).

Argument marshalling only: torch provides device memory and the current HIP
stream; every step of the layer runs in the library's kernels.  If the library
is not built, lib() raises -- there is no fallback implementation.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_OK = 0
GDN_ERR_INVALID_ARG = -1
GDN_ERR_UNSUPPORTED = -2
GDN_ERR_WORKSPACE = -3
GDN_ERR_HIP = -4
GDN_F32 = 0
GDN_BF16 = 1
OP_PREFILL, OP_DECODE, OP_FWD_BWD, OP_PREFILL_CHUNKED, OP_PREFILL_CONTINUE = 0, 1, 2, 3, 4

EXPORTS = ["gdn_workspace_bytes", "gdn_cache_init", "gdn_prefill", "gdn_decode_step",
           "gdn_fwd_bwd", "gdn_profile_enable", "gdn_profile_read", "gdn_contract_id",
           "gdn_contract_check", "gdn_error_string", "gdn_prefill_chunked",
           "gdn_prefill_continue", "gdn_fwd_bwd_ex", "gdn_decode_step_noalloc",
           "gdn_fwd_bwd_chunked", "gdn_decode_step_native", "gdn_profile_filter"]


class Shape(ctypes.Structure):
    _fields_ = [("H_qk", ctypes.c_int32), ("H_v", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("C", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("qk_l2norm", ctypes.c_int32), ("scale", ctypes.c_float)]


class CacheStruct(ctypes.Structure):
    _fields_ = [("S_run", ctypes.c_void_p), ("S_chunk", ctypes.c_void_p),
                ("kbuf", ctypes.c_void_p), ("vbuf", ctypes.c_void_p),
                ("bbuf", ctypes.c_void_p), ("gbuf", ctypes.c_void_p),
                ("pos", ctypes.c_void_p)]


_lib = None


def lib():
    """Loads libgdn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run linear_attention_rnn_gated_amd/build.py "
                               "(the GPU path has no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sp = ctypes.POINTER(Shape)
        cp = ctypes.POINTER(CacheStruct)
        L.gdn_workspace_bytes.argtypes = [sp, i32, i64, i32]
        L.gdn_workspace_bytes.restype = sz
        L.gdn_cache_init.argtypes = [sp, i32, vp, cp, vp]
        L.gdn_cache_init.restype = ctypes.c_int
        L.gdn_prefill.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, cp, vp, sz, vp]
        L.gdn_prefill_chunked.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                          vp]
        L.gdn_prefill_chunked.restype = ctypes.c_int
        L.gdn_prefill_continue.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp, cp, vp, vp,
                                           vp, sz, vp]
        L.gdn_prefill_continue.restype = ctypes.c_int
        L.gdn_prefill.restype = ctypes.c_int
        L.gdn_decode_step.argtypes = [sp, i32, vp, vp, vp, vp, vp, cp, vp, vp, vp, sz, vp]
        L.gdn_decode_step.restype = ctypes.c_int
        L.gdn_decode_step_noalloc.argtypes = [sp, i32, vp, vp, vp, vp, vp, cp, vp, vp, vp]
        L.gdn_decode_step_noalloc.restype = ctypes.c_int
        L.gdn_fwd_bwd.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_fwd_bwd.restype = ctypes.c_int
        L.gdn_fwd_bwd_ex.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                     vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_fwd_bwd_ex.restype = ctypes.c_int
        L.gdn_fwd_bwd_chunked.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_fwd_bwd_chunked.restype = ctypes.c_int
        L.gdn_decode_step_native.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gdn_decode_step_native.restype = ctypes.c_int
        L.gdn_profile_enable.argtypes = [ctypes.c_int]
        L.gdn_profile_enable.restype = ctypes.c_int
        L.gdn_profile_filter.argtypes = [ctypes.c_char_p]
        L.gdn_profile_filter.restype = ctypes.c_int
        L.gdn_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64)]
        L.gdn_profile_read.restype = ctypes.c_int
        L.gdn_contract_id.argtypes = []
        L.gdn_contract_id.restype = ctypes.c_char_p
        L.gdn_contract_check.argtypes = [ctypes.c_char_p]
        L.gdn_contract_check.restype = ctypes.c_int
        L.gdn_error_string.argtypes = [ctypes.c_int]
        L.gdn_error_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


class GdnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().gdn_error_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def _check(status, where):
    if status != GDN_OK:
        raise GdnError(status, where)


def make_shape(H_qk, H_v, d, C, in_dtype, qk_l2norm=True, scale=1.0, d_v=None):
    dt = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}[in_dtype] \
        if isinstance(in_dtype, torch.dtype) else int(in_dtype)
    return Shape(H_qk, H_v, d, d if d_v is None else d_v, C, dt, int(bool(qk_l2norm)),
                 float(scale))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_bytes(shape, n_seqs, total_tokens, op):
    return int(lib().gdn_workspace_bytes(ctypes.byref(shape), n_seqs, total_tokens, op))


def profile_enable(on=True):
    _check(lib().gdn_profile_enable(int(bool(on))), "gdn_profile_enable")


def profile_filter(kernel=""):
    """Only launches whose kernel name contains `kernel` are timed ("" = all)."""
    _check(lib().gdn_profile_filter(kernel.encode() if kernel else None), "gdn_profile_filter")


def profile_read(kernel=""):
    """(total ms, launches) of the timed launches whose name contains `kernel`;
    waits for them and forgets them."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().gdn_profile_read(kernel.encode() if kernel else None, ctypes.byref(ms),
                                  ctypes.byref(n)), "gdn_profile_read")
    return ms.value, n.value


def contract_id():
    return lib().gdn_contract_id().decode()


def contract_check(other_id):
    """GDN_OK (0) if another library's contract id equals this library's."""
    return lib().gdn_contract_check(other_id.encode())


def _workspace(shape, n, T, op, device, ws=None):
    need = workspace_bytes(shape, n, T, op)
    if need == 0:
        raise GdnError(GDN_ERR_UNSUPPORTED, "gdn_workspace_bytes")
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws


def _req(t, dtype, shape, name):
    if t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")


class Cache:
    """Decode cache (gdn_cache_t) of n sequences, owned by torch tensors."""

    def __init__(self, shape, n, device, in_dtype):
        d, C, Hq, Hv = shape.d_k, shape.C, shape.H_qk, shape.H_v
        f32 = dict(dtype=torch.float32, device=device)
        self.S_run = torch.empty(n, Hv, d, d, **f32)
        self.S_chunk = torch.empty(n, Hv, d, d, **f32)
        self.kbuf = torch.empty(n, C, Hq, d, **f32)
        self.vbuf = torch.empty(n, C, Hv, d, dtype=in_dtype, device=device)
        self.bbuf = torch.empty(n, C, Hv, **f32)
        self.gbuf = torch.empty(n, C, Hv, **f32)
        self.pos = torch.zeros(n, Hv, dtype=torch.int32, device=device)
        self.n = n

    def struct(self):
        return CacheStruct(*[t.data_ptr() for t in self.tensors()])

    def tensors(self):
        return [self.S_run, self.S_chunk, self.kbuf, self.vbuf, self.bbuf, self.gbuf, self.pos]

    def clone(self):
        c = object.__new__(Cache)
        for name in ["S_run", "S_chunk", "kbuf", "vbuf", "bbuf", "gbuf", "pos"]:
            setattr(c, name, getattr(self, name).clone())
        c.n = self.n
        return c


def gdn_cache_init(shape, n, device, in_dtype, h0=None):
    c = Cache(shape, n, device, in_dtype)
    cs = c.struct()
    _check(lib().gdn_cache_init(ctypes.byref(shape), n, _ptr(h0), ctypes.byref(cs),
                                _stream(device)), "gdn_cache_init")
    return c


def _cu_pair(cu_seqlens, dev, cu_seqlens_host):
    """Device and host int32 copies of cu_seqlens.  A caller that keeps a host
    copy (cu_seqlens_host, CPU int32 [N+1], same values) saves the
    device-to-host copy, which waits for the stream, on every call.  With
    cu_seqlens_host=False the library gets NULL and makes that copy itself."""
    cu_dev = cu_seqlens.to(dev, torch.int32).contiguous()
    if cu_seqlens_host is False:
        return cu_dev, None
    if cu_seqlens_host is None:
        return cu_dev, cu_seqlens.to("cpu", torch.int32).contiguous()
    if (cu_seqlens_host.device.type != "cpu" or cu_seqlens_host.dtype != torch.int32
            or cu_seqlens_host.numel() != cu_seqlens.numel()):
        raise ValueError("cu_seqlens_host: expected a CPU int32 tensor shaped like cu_seqlens")
    return cu_dev, cu_seqlens_host.contiguous()


def gdn_prefill(shape, q, k, v, beta, g, cu_seqlens, h0=None, cache=None, want_hT=True,
                ws=None, out=None, cu_seqlens_host=None, hT_out=None):
    """Packed prefill.  cu_seqlens: int32 device tensor [N+1]; its host copy is
    taken here unless cu_seqlens_host is given.  out / hT_out: optional
    caller-owned o [T, H_v, d] and hT [N, H_v, d, d] fp32.  Returns (o, hT)."""
    dev = q.device
    T = q.shape[0]
    n = cu_seqlens.numel() - 1
    d, Hq, Hv = shape.d_k, shape.H_qk, shape.H_v
    idt = q.dtype
    _req(q, idt, (T, Hq, d), "q")
    _req(k, idt, (T, Hq, d), "k")
    _req(v, idt, (T, Hv, d), "v")
    _req(beta, torch.float32, (T, Hv), "beta")
    _req(g, torch.float32, (T, Hv), "g")
    if h0 is not None:
        _req(h0, torch.float32, (n, Hv, d, d), "h0")
    cu_dev, cu_host = _cu_pair(cu_seqlens, dev, cu_seqlens_host)
    o = torch.empty(T, Hv, d, dtype=torch.float32, device=dev) if out is None else out
    _req(o, torch.float32, (T, Hv, d), "out")
    if hT_out is not None:
        _req(hT_out, torch.float32, (n, Hv, d, d), "hT_out")
        hT = hT_out
    else:
        hT = torch.empty(n, Hv, d, d, dtype=torch.float32, device=dev) if want_hT else None
    ws = _workspace(shape, n, T, OP_PREFILL, dev, ws)
    cs = cache.struct() if cache is not None else None
    st = lib().gdn_prefill(ctypes.byref(shape), n, _ptr(cu_dev),
                           _ptr(cu_host), _ptr(q), _ptr(k), _ptr(v),
                           _ptr(beta), _ptr(g), _ptr(h0), _ptr(o), _ptr(hT),
                           ctypes.byref(cs) if cs is not None else None, _ptr(ws),
                           ws.numel(), _stream(dev))
    _check(st, "gdn_prefill")
    return o, hT


def gdn_prefill_continue(shape, q, k, v, beta, g, cu_seqlens, cache, pos_host, want_hT=True,
                         ws=None, out=None, cu_seqlens_host=None):
    """Next tokens of sequences whose cache stands anywhere inside a chunk.
    pos_host: each sequence's position in its current chunk (host int32 [N],
    the value of cache.pos).  Returns (o, hT) of the new tokens."""
    dev = q.device
    T = q.shape[0]
    n = cu_seqlens.numel() - 1
    d, Hq, Hv = shape.d_k, shape.H_qk, shape.H_v
    idt = q.dtype
    _req(q, idt, (T, Hq, d), "q")
    _req(k, idt, (T, Hq, d), "k")
    _req(v, idt, (T, Hv, d), "v")
    _req(beta, torch.float32, (T, Hv), "beta")
    _req(g, torch.float32, (T, Hv), "g")
    cu_dev, cu_host = _cu_pair(cu_seqlens, dev, cu_seqlens_host)
    pos = torch.as_tensor(pos_host, dtype=torch.int32).to("cpu").contiguous()
    if pos.numel() != n:
        raise ValueError(f"pos_host: expected {n} values, got {pos.numel()}")
    o = torch.empty(T, Hv, d, dtype=torch.float32, device=dev) if out is None else out
    hT = torch.empty(n, Hv, d, d, dtype=torch.float32, device=dev) if want_hT else None
    ws = _workspace(shape, n, T, OP_PREFILL_CONTINUE, dev, ws)
    cs = cache.struct()
    st = lib().gdn_prefill_continue(ctypes.byref(shape), n, _ptr(cu_dev),
                                    _ptr(cu_host),
                                    ctypes.c_void_p(pos.data_ptr()), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(beta), _ptr(g), ctypes.byref(cs), _ptr(o), _ptr(hT),
                                    _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "gdn_prefill_continue")
    return o, hT


def gdn_prefill_chunked(shape, q, k, v, beta, g, cu_seqlens, h0=None, want_hT=True, ws=None,
                        out=None, cu_seqlens_host=None):
    """Native-mixed baseline prefill (chunk-form outputs; not bit-identical to
    gdn_prefill / decode).  Returns (o, hT)."""
    dev = q.device
    T = q.shape[0]
    n = cu_seqlens.numel() - 1
    d, Hq, Hv = shape.d_k, shape.H_qk, shape.H_v
    idt = q.dtype
    _req(q, idt, (T, Hq, d), "q")
    _req(k, idt, (T, Hq, d), "k")
    _req(v, idt, (T, Hv, d), "v")
    _req(beta, torch.float32, (T, Hv), "beta")
    _req(g, torch.float32, (T, Hv), "g")
    if h0 is not None:
        _req(h0, torch.float32, (n, Hv, d, d), "h0")
    cu_dev, cu_host = _cu_pair(cu_seqlens, dev, cu_seqlens_host)
    o = torch.empty(T, Hv, d, dtype=torch.float32, device=dev) if out is None else out
    hT = torch.empty(n, Hv, d, d, dtype=torch.float32, device=dev) if want_hT else None
    ws = _workspace(shape, n, T, OP_PREFILL_CHUNKED, dev, ws)
    st = lib().gdn_prefill_chunked(ctypes.byref(shape), n, _ptr(cu_dev),
                                   _ptr(cu_host), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(beta), _ptr(g), _ptr(h0), _ptr(o), _ptr(hT), _ptr(ws),
                                   ws.numel(), _stream(dev))
    _check(st, "gdn_prefill_chunked")
    return o, hT


def gdn_decode_step(shape, q, k, v, beta, g, cache, pos_host=None, ws=None, out=None):
    """One token per sequence: q, k [N, H_qk, d], v [N, H_v, d], beta, g [N, H_v].
    pos_host: optional int32 CPU tensor [N, H_v] mirroring cache.pos.  Returns o."""
    dev = q.device
    n = q.shape[0]
    d, Hq, Hv = shape.d_k, shape.H_qk, shape.H_v
    idt = q.dtype
    _req(q, idt, (n, Hq, d), "q")
    _req(k, idt, (n, Hq, d), "k")
    _req(v, idt, (n, Hv, d), "v")
    _req(beta, torch.float32, (n, Hv), "beta")
    _req(g, torch.float32, (n, Hv), "g")
    o = torch.empty(n, Hv, d, dtype=torch.float32, device=dev) if out is None else out
    ws = _workspace(shape, n, 0, OP_DECODE, dev, ws)
    cs = cache.struct()
    ph = None
    if pos_host is not None:
        ph = ctypes.c_void_p(pos_host.data_ptr())
    st = lib().gdn_decode_step(ctypes.byref(shape), n, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                               _ptr(g), ctypes.byref(cs), ph, _ptr(o), _ptr(ws), ws.numel(),
                               _stream(dev))
    _check(st, "gdn_decode_step")
    return o


def gdn_decode_step_noalloc(shape, q, k, v, beta, g, cache, pos_host=None, out=None):
    """gdn_decode_step without a workspace: the library's fixed device scratch
    holds the resync's chunk factors (for callers that cannot allocate).  Pass
    `out` (fp32 [N, H_v, d]) to keep this call free of allocations too."""
    dev = q.device
    n = q.shape[0]
    d, Hq, Hv = shape.d_k, shape.H_qk, shape.H_v
    idt = q.dtype
    _req(q, idt, (n, Hq, d), "q")
    _req(k, idt, (n, Hq, d), "k")
    _req(v, idt, (n, Hv, d), "v")
    _req(beta, torch.float32, (n, Hv), "beta")
    _req(g, torch.float32, (n, Hv), "g")
    o = torch.empty(n, Hv, d, dtype=torch.float32, device=dev) if out is None else out
    _req(o, torch.float32, (n, Hv, d), "out")
    cs = cache.struct()
    ph = None if pos_host is None else ctypes.c_void_p(pos_host.data_ptr())
    st = lib().gdn_decode_step_noalloc(ctypes.byref(shape), n, _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(beta), _ptr(g), ctypes.byref(cs), ph, _ptr(o),
                                       _stream(dev))
    _check(st, "gdn_decode_step_noalloc")
    return o


def gdn_decode_step_native(shape, q, k, v, beta, g, S, out=None):
    """Native-mixed baseline decode: the plain token step on the state S
    (fp32 [N, H_v, d, d], updated in place); no chunk buffers, no resync.
    Returns o."""
    dev = q.device
    n = q.shape[0]
    d, Hq, Hv = shape.d_k, shape.H_qk, shape.H_v
    idt = q.dtype
    _req(q, idt, (n, Hq, d), "q")
    _req(k, idt, (n, Hq, d), "k")
    _req(v, idt, (n, Hv, d), "v")
    _req(beta, torch.float32, (n, Hv), "beta")
    _req(g, torch.float32, (n, Hv), "g")
    _req(S, torch.float32, (n, Hv, d, d), "S")
    o = torch.empty(n, Hv, d, dtype=torch.float32, device=dev) if out is None else out
    _req(o, torch.float32, (n, Hv, d), "out")
    st = lib().gdn_decode_step_native(ctypes.byref(shape), n, _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(beta), _ptr(g), _ptr(S), _ptr(o), _stream(dev))
    _check(st, "gdn_decode_step_native")
    return o


def gdn_fwd_bwd_chunked(shape, q, k, v, beta, g, cu_seqlens, dO, h0=None, dhT=None, ws=None,
                        cu_seqlens_host=None):
    """Native-mixed baseline trainer step: chunk-form forward outputs, the same
    backward (fp32 gradients).  Returns dict(o, hT, dq, dk, dv, dbeta, dg, dh0)."""
    return gdn_fwd_bwd(shape, q, k, v, beta, g, cu_seqlens, dO, h0=h0, dhT=dhT, ws=ws,
                       cu_seqlens_host=cu_seqlens_host, _native=True)


def gdn_fwd_bwd(shape, q, k, v, beta, g, cu_seqlens, dO, h0=None, dhT=None, ws=None,
                grad_dtype=torch.float32, cu_seqlens_host=None, out=None, _native=False):
    """Trainer forward + backward.  Returns dict(o, hT, dq, dk, dv, dbeta, dg, dh0);
    dq, dk, dv in grad_dtype (float32 or bfloat16), the rest float32.  out:
    optional dict of caller-owned tensors for some or all of those outputs."""
    dev = q.device
    T = q.shape[0]
    n = cu_seqlens.numel() - 1
    d, Hq, Hv = shape.d_k, shape.H_qk, shape.H_v
    idt = q.dtype
    _req(q, idt, (T, Hq, d), "q")
    _req(k, idt, (T, Hq, d), "k")
    _req(v, idt, (T, Hv, d), "v")
    _req(beta, torch.float32, (T, Hv), "beta")
    _req(g, torch.float32, (T, Hv), "g")
    _req(dO, torch.float32, (T, Hv, d), "dO")
    if h0 is not None:
        _req(h0, torch.float32, (n, Hv, d, d), "h0")
    if dhT is not None:
        _req(dhT, torch.float32, (n, Hv, d, d), "dhT")
    cu_dev, cu_host = _cu_pair(cu_seqlens, dev, cu_seqlens_host)
    f32 = dict(dtype=torch.float32, device=dev)
    gd = dict(dtype=grad_dtype, device=dev)
    code = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}[grad_dtype]
    r = dict(o=torch.empty(T, Hv, d, **f32), hT=torch.empty(n, Hv, d, d, **f32),
             dq=torch.empty(T, Hq, d, **gd), dk=torch.empty(T, Hq, d, **gd),
             dv=torch.empty(T, Hv, d, **gd), dbeta=torch.empty(T, Hv, **f32),
             dg=torch.empty(T, Hv, **f32), dh0=torch.empty(n, Hv, d, d, **f32))
    for key, t in (out or {}).items():
        _req(t, r[key].dtype, tuple(r[key].shape), f"out[{key!r}]")
        r[key] = t
    ws = _workspace(shape, n, T, OP_FWD_BWD, dev, ws)
    if _native:
        if grad_dtype != torch.float32:
            raise ValueError("gdn_fwd_bwd_chunked writes fp32 gradients")
        st = lib().gdn_fwd_bwd_chunked(
            ctypes.byref(shape), n, _ptr(cu_dev), _ptr(cu_host), _ptr(q), _ptr(k), _ptr(v),
            _ptr(beta), _ptr(g), _ptr(h0), _ptr(dO), _ptr(dhT), _ptr(r["o"]), _ptr(r["hT"]),
            _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]), _ptr(r["dbeta"]), _ptr(r["dg"]),
            _ptr(r["dh0"]), _ptr(ws), ws.numel(), _stream(dev))
        _check(st, "gdn_fwd_bwd_chunked")
        return r
    st = lib().gdn_fwd_bwd_ex(ctypes.byref(shape), n, _ptr(cu_dev),
                              _ptr(cu_host), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(beta), _ptr(g), _ptr(h0), _ptr(dO), _ptr(dhT), _ptr(r["o"]),
                              _ptr(r["hT"]), code, _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]),
                              _ptr(r["dbeta"]), _ptr(r["dg"]), _ptr(r["dh0"]), _ptr(ws),
                              ws.numel(), _stream(dev))
    _check(st, "gdn_fwd_bwd_ex")
    return r
