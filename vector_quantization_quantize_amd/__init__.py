"""Python binding of libtq (TurboQuant quantize / score path on gfx950).

Argument marshalling only: every function below forwards to the C entry
point of the same name in ``libtq.so`` (declared in ``include/tq.h``); all
arithmetic runs in the library's HIP kernels.  torch provides device memory
and the current stream.  Importing this package loads the shared library and
fails loudly if it has not been built (run ``__graft_entry__.build()`` or
``python vector_quantization_quantize_amd/_build.py``); there is no CPU or
PyTorch fallback.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_LIBRARY names another build of the same library (the host-sanitizer
# build the CPU tests use); by default the in-tree libtq.so
LIB_PATH = os.environ.get("TQ_LIBRARY") or os.path.join(HERE, "libtq.so")

TQ_OK = 0
TQ_EINVAL = -1
TQ_EUNSUPPORTED = -2
TQ_EHIP = -3
TQ_ENOMEM = -4
TQ_ESCRATCH = -5
TQ_F32 = 0
TQ_BF16 = 1
TQ_FORMAT_VERSION = 1

# every symbol include/tq.h declares
EXPORTS = ("tq_init", "tq_init_explicit", "tq_init_hadamard", "tq_init_split", "tq_init_polar", "tq_polar_codebook",
           "tq_hadamard_rotation", "tq_destroy", "tq_get_layout", "tq_host_params",
           "tq_params_hash", "tq_quantize", "tq_logits_workspace_size", "tq_logits",
           "tq_logits_topk_workspace_size", "tq_logits_topk", "tq_dequant_mse", "tq_dequant_prod", "tq_dense_logits", "tq_pack_values",
           "tq_attention_workspace_size", "tq_attention", "tq_logits_noalloc", "tq_noalloc_scratch_bytes",
           "tq_strerror")


class TqError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {code} ({_lib().tq_strerror(code).decode()})")
        self.code = code


class Layout(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits", ctypes.c_int32), ("code_bits", ctypes.c_int32),
                ("levels", ctypes.c_int32), ("words", ctypes.c_int32),
                ("format_version", ctypes.c_int32), ("code_bytes", ctypes.c_int64),
                ("sign_bytes", ctypes.c_int64), ("key_bytes", ctypes.c_int64),
                ("hi", ctypes.c_int32), ("hi_words", ctypes.c_int32), ("polar", ctypes.c_int32)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libtq.so is not built ({LIB_PATH}); build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    fp = ctypes.POINTER(ctypes.c_float)
    sig = {
        "tq_init": (ctypes.c_int, [i32, i32, u64, ctypes.POINTER(vp)]),
        "tq_init_explicit": (ctypes.c_int, [i32, i32, fp, fp, ctypes.POINTER(vp)]),
        "tq_init_hadamard": (ctypes.c_int, [i32, i32, u64, ctypes.POINTER(vp)]),
        "tq_init_split": (ctypes.c_int, [i32, i32, i32, u64, ctypes.POINTER(vp)]),
        "tq_init_polar": (ctypes.c_int, [i32, i32, u64, ctypes.POINTER(vp)]),
        "tq_polar_codebook": (ctypes.c_int, [i32, i32, i32, vp, vp]),
        "tq_hadamard_rotation": (ctypes.c_int, [i32, u64, vp]),
        "tq_destroy": (ctypes.c_int, [vp]),
        "tq_get_layout": (ctypes.c_int, [vp, ctypes.POINTER(Layout)]),
        "tq_host_params": (ctypes.c_int, [i32, i32, u64, vp, vp, vp, vp]),
        "tq_params_hash": (u64, [vp]),
        "tq_quantize": (ctypes.c_int, [vp, vp, i32, i64, i64, vp, vp, vp, vp, vp]),
        "tq_logits_workspace_size": (sz, [vp, i64, i64]),
        "tq_logits": (ctypes.c_int, [vp, vp, i64, i64, vp, vp, vp, vp, i64, vp, vp, sz, vp]),
        "tq_dequant_mse": (ctypes.c_int, [vp, vp, vp, i64, vp, vp]),
        "tq_logits_topk_workspace_size": (sz, [vp, i64, i64, i64, i32]),
        "tq_logits_topk": (ctypes.c_int, [vp, vp, i64, i64, vp, vp, vp, vp, i64, i32, vp, vp, vp, sz, vp]),
        "tq_dequant_prod": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, vp, vp]),
        "tq_dense_logits": (ctypes.c_int, [vp, i64, i64, vp, i32, i64, i32, i64, vp, vp]),
        "tq_pack_values": (ctypes.c_int, [vp, vp, i64, i64, vp, vp]),
        "tq_attention_workspace_size": (sz, [vp, vp, i64, i64, i64]),
        "tq_attention": (ctypes.c_int, [vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, i64, ctypes.c_float, vp, vp,
                                        vp, sz, vp]),
        "tq_logits_noalloc": (ctypes.c_int, [vp, vp, i64, i64, vp, vp, vp, vp, i64, vp, vp]),
        "tq_noalloc_scratch_bytes": (sz, []),
        "tq_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _LIB = lib
    return lib


def _check(fn, rc):
    if rc != TQ_OK:
        raise TqError(fn, rc)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


class Handle:
    """Owns one ``tq_handle``; destroyed with the object."""

    def __init__(self, ptr):
        self._ptr = ptr
        lay = Layout()
        _check("tq_get_layout", _lib().tq_get_layout(ptr, ctypes.byref(lay)))
        self.layout = lay
        self.d = lay.d
        self.bits = lay.bits
        self.code_bits = lay.code_bits
        self.words = lay.words
        self.hi = lay.hi
        self.hi_words = lay.hi_words
        self.polar = lay.polar
        # per-key shape of the codes: (B, W) planes, or flat B W + hi_words
        # words with fractional widths
        self.code_shape = ((lay.code_bits * lay.words + lay.hi_words,) if lay.hi
                           else (lay.code_bits, lay.words))

    @property
    def ptr(self):
        return self._ptr

    def close(self):
        if self._ptr is not None and _LIB is not None:
            _LIB.tq_destroy(self._ptr)
        self._ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tq_init(d, bits, seed):
    out = ctypes.c_void_p()
    _check("tq_init", _lib().tq_init(int(d), int(bits), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)),
                                     ctypes.byref(out)))
    return Handle(out)


def tq_init_split(d, bits, hi, seed):
    """Handle with fractional widths: rotated coordinates 0 .. hi-1 get one
    more index bit (bits + hi / d bits per coordinate)."""
    out = ctypes.c_void_p()
    _check("tq_init_split", _lib().tq_init_split(int(d), int(bits), int(hi), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)),
                                                 ctypes.byref(out)))
    return Handle(out)


def tq_init_hadamard(d, bits, seed):
    """Handle with the randomized Hadamard rotation (d a power of two)."""
    out = ctypes.c_void_p()
    _check("tq_init_hadamard", _lib().tq_init_hadamard(int(d), int(bits), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)),
                                                       ctypes.byref(out)))
    return Handle(out)


def tq_init_polar(d, bits, seed):
    """Handle with the recursive polar-angle stage 1 (d a power of two)."""
    out = ctypes.c_void_p()
    _check("tq_init_polar", _lib().tq_init_polar(int(d), int(bits), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)),
                                                 ctypes.byref(out)))
    return Handle(out)


def tq_polar_codebook(d, bits, level):
    """Host-only: (levels, thresholds) float32 of recursion level `level`."""
    import numpy as np
    L = 1 << (int(bits) - 1)
    lv = np.empty(L, dtype=np.float32)
    th = np.empty(max(L - 1, 1), dtype=np.float32)
    _check("tq_polar_codebook", _lib().tq_polar_codebook(int(d), int(bits), int(level), lv.ctypes.data_as(ctypes.c_void_p),
                                                         th.ctypes.data_as(ctypes.c_void_p)))
    return lv, th[:L - 1]


def tq_hadamard_rotation(d, seed):
    """Host-only: the rotation tq_init_hadamard uses (numpy float32 (d, d))."""
    import numpy as np
    pi = np.empty((d, d), dtype=np.float32)
    _check("tq_hadamard_rotation", _lib().tq_hadamard_rotation(int(d), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)),
                                                               pi.ctypes.data))
    return pi


def tq_init_explicit(d, bits, pi, g):
    """``pi``, ``g``: host float32 arrays (d, d), row-major."""
    import numpy as np
    pi = np.ascontiguousarray(pi, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    assert pi.shape == (d, d) and g.shape == (d, d)
    fp = ctypes.POINTER(ctypes.c_float)
    out = ctypes.c_void_p()
    _check("tq_init_explicit", _lib().tq_init_explicit(int(d), int(bits), pi.ctypes.data_as(fp),
                                                       g.ctypes.data_as(fp), ctypes.byref(out)))
    return Handle(out)


def tq_destroy(h):
    h.close()


def tq_get_layout(h):
    return h.layout


def tq_params_hash(h):
    return int(_lib().tq_params_hash(h.ptr))


def tq_host_params(d, bits, seed):
    """Host-only parameters (numpy float32): pi, g (d, d), centroids, thresholds."""
    import numpy as np
    levels = 1 << (bits - 1)
    pi = np.empty((d, d), dtype=np.float32)
    g = np.empty((d, d), dtype=np.float32)
    c = np.empty(levels, dtype=np.float32)
    t = np.empty(max(levels - 1, 1), dtype=np.float32)
    _check("tq_host_params", _lib().tq_host_params(int(d), int(bits), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)),
                                                   pi.ctypes.data, g.ctypes.data, c.ctypes.data, t.ctypes.data))
    return pi, g, c, t[:levels - 1]


def empty_packed(h, n, device="cuda"):
    """Allocate (codes, signs, norms, rnorms) device tensors for n keys."""
    import torch
    codes = torch.empty((n,) + h.code_shape, dtype=torch.int32, device=device)
    signs = torch.empty((n, h.words), dtype=torch.int32, device=device)
    norms = torch.empty((n,), dtype=torch.float32, device=device)
    rnorms = torch.empty((n,), dtype=torch.float32, device=device)
    return codes, signs, norms, rnorms


def tq_quantize(h, keys, out=None, stream=None):
    """keys: cuda tensor (n, d) float32 or bfloat16 with unit column stride.

    Returns (codes int32 (n,) + h.code_shape, signs int32 (n, W), norms, rnorms); the
    int32 tensors hold the uint32 words bit for bit."""
    import torch
    if keys.dim() != 2 or keys.shape[1] != h.d or keys.stride(1) != 1:
        raise ValueError("keys must be (n, d) with unit column stride")
    if keys.dtype == torch.float32:
        kdt = TQ_F32
    elif keys.dtype == torch.bfloat16:
        kdt = TQ_BF16
    else:
        raise ValueError("keys must be float32 or bfloat16")
    n = keys.shape[0]
    if out is None:
        out = empty_packed(h, n, keys.device)
    codes, signs, norms, rnorms = out
    _check("tq_quantize", _lib().tq_quantize(h.ptr, _ptr(keys), kdt, n, keys.stride(0) if n else h.d,
                                             _ptr(codes), _ptr(signs), _ptr(norms), _ptr(rnorms),
                                             _stream(stream)))
    return codes, signs, norms, rnorms


def tq_logits_workspace_size(h, groups, nq):
    return int(_lib().tq_logits_workspace_size(h.ptr, int(groups), int(nq)))


def tq_logits(h, queries, codes, signs, norms, rnorms, n=None, scores=None, workspace=None, stream=None):
    """queries: cuda float32 (groups, nq, d); packed arrays hold groups*n keys.

    Returns scores float32 (groups, nq, n)."""
    import torch
    if queries.dim() == 2:
        queries = queries.unsqueeze(0)
    groups, nq, d = queries.shape
    if d != h.d or not queries.is_contiguous() or queries.dtype != torch.float32:
        raise ValueError("queries must be contiguous float32 (groups, nq, d)")
    total = norms.shape[0]
    if n is None:
        n = total // groups
    if groups * n > total:
        raise ValueError("packed arrays hold fewer than groups * n keys")
    if scores is None:
        scores = torch.empty((groups, nq, n), dtype=torch.float32, device=queries.device)
    ws_bytes = tq_logits_workspace_size(h, groups, nq)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 256) + 255) // 4, dtype=torch.float32, device=queries.device)
    _check("tq_logits", _lib().tq_logits(h.ptr, _ptr(queries), groups, nq, _ptr(codes), _ptr(signs),
                                         _ptr(norms), _ptr(rnorms), n, _ptr(scores), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))
    return scores


def tq_noalloc_scratch_bytes():
    return int(_lib().tq_noalloc_scratch_bytes())


def tq_logits_noalloc(h, queries, codes, signs, norms, rnorms, n=None, scores=None, stream=None):
    """tq_logits with the library's static scratch as workspace (the C entry
    point allocates nothing; pass `scores` to allocate nothing here either).

    queries: cuda float32 (groups, nq, d); packed arrays hold groups*n keys.
    Returns scores float32 (groups, nq, n)."""
    import torch
    if queries.dim() == 2:
        queries = queries.unsqueeze(0)
    groups, nq, d = queries.shape
    if d != h.d or not queries.is_contiguous() or queries.dtype != torch.float32:
        raise ValueError("queries must be contiguous float32 (groups, nq, d)")
    total = norms.shape[0]
    if n is None:
        n = total // groups
    if groups * n > total:
        raise ValueError("packed arrays hold fewer than groups * n keys")
    if scores is None:
        scores = torch.empty((groups, nq, n), dtype=torch.float32, device=queries.device)
    _check("tq_logits_noalloc", _lib().tq_logits_noalloc(h.ptr, _ptr(queries), groups, nq, _ptr(codes), _ptr(signs),
                                                         _ptr(norms), _ptr(rnorms), n, _ptr(scores),
                                                         _stream(stream)))
    return scores


def tq_logits_topk_workspace_size(h, groups, nq, n, k):
    return int(_lib().tq_logits_topk_workspace_size(h.ptr, int(groups), int(nq), int(n), int(k)))


def tq_logits_topk(h, queries, codes, signs, norms, rnorms, k, n=None, out=None, workspace=None, stream=None):
    """The k best keys per query by the score tq_logits computes.

    queries: cuda float32 (groups, nq, d); packed arrays hold groups*n keys.
    Returns (indices int64 (groups, nq, k), scores float32 (groups, nq, k)),
    best first; index -1 / score -inf past n keys."""
    import torch
    if queries.dim() == 2:
        queries = queries.unsqueeze(0)
    groups, nq, d = queries.shape
    if d != h.d or not queries.is_contiguous() or queries.dtype != torch.float32:
        raise ValueError("queries must be contiguous float32 (groups, nq, d)")
    total = norms.shape[0]
    if n is None:
        n = total // groups
    if groups * n > total:
        raise ValueError("packed arrays hold fewer than groups * n keys")
    if out is None:
        out = (torch.empty((groups, nq, k), dtype=torch.int64, device=queries.device),
               torch.empty((groups, nq, k), dtype=torch.float32, device=queries.device))
    idx, sc = out
    ws_bytes = tq_logits_topk_workspace_size(h, groups, nq, n, k)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 256) + 255) // 4, dtype=torch.float32, device=queries.device)
    _check("tq_logits_topk", _lib().tq_logits_topk(h.ptr, _ptr(queries), groups, nq, _ptr(codes), _ptr(signs),
                                                   _ptr(norms), _ptr(rnorms), n, int(k), _ptr(idx), _ptr(sc),
                                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                   _stream(stream)))
    return idx, sc


def tq_dequant_mse(h, codes, norms, khat=None, stream=None):
    """Stage-1 reconstruction (n, d) float32 of n packed keys."""
    import torch
    n = norms.shape[0]
    if khat is None:
        khat = torch.empty((n, h.d), dtype=torch.float32, device=norms.device)
    _check("tq_dequant_mse", _lib().tq_dequant_mse(h.ptr, _ptr(codes), _ptr(norms), n, _ptr(khat),
                                                   _stream(stream)))
    return khat


def tq_dequant_prod(h, codes, signs, norms, rnorms, ktilde=None, stream=None):
    """Reconstruction with the QJL correction (n, d) float32: inner products
    with it equal tq_logits' scores."""
    import torch
    n = norms.shape[0]
    if ktilde is None:
        ktilde = torch.empty((n, h.d), dtype=torch.float32, device=norms.device)
    _check("tq_dequant_prod", _lib().tq_dequant_prod(h.ptr, _ptr(codes), _ptr(signs), _ptr(norms), _ptr(rnorms),
                                                     n, _ptr(ktilde), _stream(stream)))
    return ktilde


def tq_dense_logits(queries, keys, n=None, scores=None, stream=None):
    """Raw inner products with unquantized keys (the uncompressed
    comparison).  queries: cuda float32 (groups, nq, d); keys: cuda float32
    or bfloat16 (groups * n, d), rows may be strided.  Returns float32
    (groups, nq, n)."""
    import torch
    if queries.dim() == 2:
        queries = queries.unsqueeze(0)
    groups, nq, d = queries.shape
    if not queries.is_contiguous() or queries.dtype != torch.float32:
        raise ValueError("queries must be contiguous float32 (groups, nq, d)")
    if keys.dim() != 2 or keys.shape[1] != d or keys.stride(1) != 1:
        raise ValueError("keys must be (rows, d) with unit column stride")
    kdt = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}.get(keys.dtype)
    if kdt is None:
        raise ValueError("keys must be float32 or bfloat16")
    if n is None:
        n = keys.shape[0] // groups
    if groups * n > keys.shape[0]:
        raise ValueError("keys hold fewer than groups * n rows")
    if scores is None:
        scores = torch.empty((groups, nq, n), dtype=torch.float32, device=queries.device)
    _check("tq_dense_logits", _lib().tq_dense_logits(_ptr(queries), groups, nq, _ptr(keys), kdt, int(n), d,
                                                     keys.stride(0), _ptr(scores), _stream(stream)))
    return scores


def tq_pack_values(h, codes, groups=1, n=None, vcodes=None, stream=None):
    """Token blocks (groups, ceil(n/32), B, 32 W) uint32 of value codes
    (groups * n, B, W) from tq_quantize."""
    import torch
    if n is None:
        n = codes.shape[0] // groups
    if groups * n > codes.shape[0]:
        raise ValueError("codes hold fewer than groups * n values")
    nb = (n + 31) // 32
    if vcodes is None:
        vcodes = torch.empty((groups, nb, h.code_bits, 32 * h.words), dtype=torch.int32, device=codes.device)
    _check("tq_pack_values", _lib().tq_pack_values(h.ptr, _ptr(codes), int(groups), int(n), _ptr(vcodes),
                                                   _stream(stream)))
    return vcodes


def tq_attention_workspace_size(hk, hv, groups, nq, n):
    return int(_lib().tq_attention_workspace_size(hk.ptr, hv.ptr, int(groups), int(nq), int(n)))


def tq_attention(hk, hv, queries, kcodes, ksigns, knorms, krnorms, vcodes, vnorms, scale=None, n=None, out=None,
                 lse=None, workspace=None, stream=None):
    """Decode attention over a compressed cache.

    queries: cuda float32 (groups, nq, d); keys packed by tq_quantize(hk)
    (groups * n of them); values: token blocks from tq_pack_values(hv) and
    their norms (groups * n).  scale defaults to 1/sqrt(d).  Returns
    (out float32 (groups, nq, d), lse float32 (groups, nq))."""
    import torch
    if queries.dim() == 2:
        queries = queries.unsqueeze(0)
    groups, nq, d = queries.shape
    if d != hk.d or d != hv.d or not queries.is_contiguous() or queries.dtype != torch.float32:
        raise ValueError("queries must be contiguous float32 (groups, nq, d)")
    if n is None:
        n = knorms.shape[0] // groups
    if groups * n > knorms.shape[0] or groups * n > vnorms.shape[0]:
        raise ValueError("packed arrays hold fewer than groups * n tokens")
    if scale is None:
        scale = 1.0 / d ** 0.5
    if out is None:
        out = torch.empty((groups, nq, d), dtype=torch.float32, device=queries.device)
    if lse is None:
        lse = torch.empty((groups, nq), dtype=torch.float32, device=queries.device)
    ws_bytes = tq_attention_workspace_size(hk, hv, groups, nq, n)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 256) + 255) // 4, dtype=torch.float32, device=queries.device)
    _check("tq_attention", _lib().tq_attention(hk.ptr, hv.ptr, _ptr(queries), groups, nq, _ptr(kcodes),
                                               _ptr(ksigns), _ptr(knorms), _ptr(krnorms), _ptr(vcodes),
                                               _ptr(vnorms), int(n), float(scale), _ptr(out), _ptr(lse),
                                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                                               _stream(stream)))
    return out, lse


_lib()
