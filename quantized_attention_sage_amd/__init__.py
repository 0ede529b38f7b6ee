"""Python binding of the MI355X quantized-attention library (libsage_attn.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/sage_attn.h. PyTorch provides device
memory and the current stream. If the shared library has not been built the
import still works but every call raises; there is no other implementation.

    from quantized_attention_sage_amd import sageattn
    o = sageattn(q, k, v, tensor_layout="HND", is_causal=False)

mirrors the ``sageattn`` call of the README usage section (gittoolsai.com
translation): q, k, v fp16/bf16 on the GPU in (B, H, S, D) ("HND") or
(B, S, H, D) ("NHD"), grouped-query heads allowed, Lq may differ from Lk.
``sageattn_qk_int8_pv_fp8`` and ``sageattn_qk_int8_pv_fp16`` pick the P.V
format explicitly (the README's kernel list; ``sageattn`` uses FP8).
``is_causal`` takes False / True (top-left, as torch's SDPA) or
"bottom_right" (the last query sees every key); ``return_lse=True`` also
returns the natural-log sum of the softmax weights per query. Short-query,
long-key shapes run their keys in several ranges merged exactly (the split
count is picked from the shape unless ``nsplit`` is given). ``block_mask``
(uint8/bool [B, Hq, ceil(Lq/128), ceil(Lk/128)]) skips whole 128 x 128
blocks (``block_sparse_sageattn``).
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsage_attn.so")

SAGE_OK, SAGE_E_INVALID, SAGE_E_UNSUPPORTED, SAGE_E_WORKSPACE, SAGE_E_HIP = range(5)
SAGE_FP16, SAGE_BF16 = 0, 1
SAGE_HND, SAGE_NHD = 0, 1
SAGE_PV_FP8, SAGE_PV_FP16 = 0, 1
_PV_CODES = {"fp8": SAGE_PV_FP8, "fp16": SAGE_PV_FP16}

EXPORTED = (
    "sage_status_str", "sage_last_error", "sage_problem_init", "sage_problem_check",
    "sage_workspace_bytes", "sage_workspace_layout", "sage_softmax_block_keys", "sage_softmax_spec",
    "sage_quantize", "sage_attn_quantized", "sage_attn", "sage_debug_qk_int32",
    "sage_varlen_problem_init", "sage_varlen_problem_check", "sage_varlen_workspace_bytes",
    "sage_varlen_workspace_layout", "sage_varlen_attn",
    "sage_split_count", "sage_split_bytes", "sage_attn_quantized_ex",
    "sage_varlen_split_count", "sage_varlen_split_bytes", "sage_varlen_attn_ex", "sage_attn_ex",
    "sage_quantize_kv", "sage_attn_q_ex", "sage_noalloc_bytes", "sage_attn_noalloc",
)
MAX_SPLIT = 16


class SageError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (status %d): %s" % (_status_name(status), status, message))
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Lq", ctypes.c_int32), ("Lk", ctypes.c_int32), ("D", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("pv", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
    ]


class VarlenProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("pv", ctypes.c_int32),
        ("total_q", ctypes.c_int32), ("total_k", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 2), ("k_stride", ctypes.c_int64 * 2),
        ("v_stride", ctypes.c_int64 * 2), ("o_stride", ctypes.c_int64 * 2),
    ]


class WsLayout(ctypes.Structure):
    _fields_ = [
        ("Dp", ctypes.c_int32), ("Lq_pad", ctypes.c_int32), ("Lk_pad", ctypes.c_int32),
        ("nkb", ctypes.c_int32), ("nchunk", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("qhat", ctypes.c_int64), ("sq", ctypes.c_int64), ("khat", ctypes.c_int64),
        ("sk", ctypes.c_int64), ("kbar", ctypes.c_int64), ("vhat", ctypes.c_int64),
        ("vmax", ctypes.c_int64), ("kpart", ctypes.c_int64), ("vpart", ctypes.c_int64),
        ("total_bytes", ctypes.c_int64),
    ]


class AttnOpts(ctypes.Structure):
    _fields_ = [
        ("is_causal", ctypes.c_int32), ("nsplit", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("reserved", ctypes.c_int32), ("lse", ctypes.c_void_p), ("part", ctypes.c_void_p),
        ("part_bytes", ctypes.c_size_t), ("block_mask", ctypes.c_void_p),
    ]


MASK_BLOCK_Q = 128     # queries per block-mask flag
MASK_BLOCK_K = 128     # keys per block-mask flag


_lib = None


def lib():
    """The loaded shared library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libsage_attn.so is not built (%s); run "
                           "`python -m quantized_attention_sage_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    PP = ctypes.POINTER(Problem)
    L.sage_status_str.argtypes = [I]
    L.sage_status_str.restype = ctypes.c_char_p
    L.sage_last_error.argtypes = []
    L.sage_last_error.restype = ctypes.c_char_p
    L.sage_problem_init.argtypes = [PP, I, I, I, I, I, I, I, I]
    L.sage_problem_check.argtypes = [PP]
    L.sage_workspace_bytes.argtypes = [PP]
    L.sage_workspace_bytes.restype = ctypes.c_size_t
    L.sage_workspace_layout.argtypes = [PP, ctypes.POINTER(WsLayout)]
    L.sage_softmax_block_keys.argtypes = []
    L.sage_softmax_spec.argtypes = [I, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    L.sage_quantize.argtypes = [PP, P, P, P, I, P, ctypes.c_size_t, P]
    L.sage_attn_quantized.argtypes = [PP, P, ctypes.c_size_t, P, I, F, P]
    L.sage_attn.argtypes = [PP, P, P, P, P, I, F, I, P, ctypes.c_size_t, P]
    L.sage_debug_qk_int32.argtypes = [PP, P, ctypes.c_size_t, I, I, P, P]
    VP = ctypes.POINTER(VarlenProblem)
    L.sage_varlen_problem_init.argtypes = [VP, I, I, I, I, I, I, I, I, I, I]
    L.sage_varlen_problem_check.argtypes = [VP]
    L.sage_varlen_workspace_bytes.argtypes = [VP]
    L.sage_varlen_workspace_bytes.restype = ctypes.c_size_t
    L.sage_varlen_workspace_layout.argtypes = [VP, ctypes.POINTER(WsLayout)]
    L.sage_varlen_attn.argtypes = [VP, P, P, P, P, P, P, I, F, I, P, ctypes.c_size_t, P]
    OP = ctypes.POINTER(AttnOpts)
    L.sage_split_count.argtypes = [PP]
    L.sage_split_bytes.argtypes = [PP, I]
    L.sage_split_bytes.restype = ctypes.c_size_t
    L.sage_attn_quantized_ex.argtypes = [PP, P, ctypes.c_size_t, P, OP, P]
    L.sage_attn_ex.argtypes = [PP, P, P, P, P, I, P, ctypes.c_size_t, OP, P]
    L.sage_quantize_kv.argtypes = [PP, P, P, I, P, ctypes.c_size_t, P]
    L.sage_attn_q_ex.argtypes = [PP, P, P, ctypes.c_size_t, P, OP, P]
    L.sage_noalloc_bytes.argtypes = [PP, I]
    L.sage_noalloc_bytes.restype = ctypes.c_size_t
    L.sage_attn_noalloc.argtypes = [PP, P, P, P, P, I, OP, P]
    L.sage_varlen_split_count.argtypes = [VP]
    L.sage_varlen_split_bytes.argtypes = [VP, I]
    L.sage_varlen_split_bytes.restype = ctypes.c_size_t
    L.sage_varlen_attn_ex.argtypes = [VP, P, P, P, P, P, P, I, P, ctypes.c_size_t, OP, P]
    for name in ("sage_problem_init", "sage_problem_check", "sage_workspace_layout",
                 "sage_softmax_block_keys", "sage_softmax_spec", "sage_quantize", "sage_attn_quantized",
                 "sage_attn", "sage_debug_qk_int32", "sage_varlen_problem_init",
                 "sage_varlen_problem_check", "sage_varlen_workspace_layout", "sage_varlen_attn",
                 "sage_split_count", "sage_attn_quantized_ex", "sage_varlen_split_count",
                 "sage_varlen_attn_ex", "sage_attn_ex", "sage_quantize_kv", "sage_attn_q_ex",
                 "sage_attn_noalloc"):
        getattr(L, name).restype = I
    _lib = L
    return L


def _status_name(status):
    try:
        return lib().sage_status_str(status).decode()
    except Exception:  # library missing: still produce a message
        return "status"


def _check(status):
    if status != SAGE_OK:
        raise SageError(status, lib().sage_last_error().decode())


_CAUSAL_CODES = {"none": 0, "top_left": 1, "bottom_right": 2}


def causal_code(is_causal):
    """0 (no mask), 1 (top-left) or 2 (bottom-right) from a bool, an int or a name."""
    if isinstance(is_causal, str):
        if is_causal not in _CAUSAL_CODES:
            raise SageError(SAGE_E_INVALID, "is_causal %r is none of %s" % (is_causal, sorted(_CAUSAL_CODES)))
        return _CAUSAL_CODES[is_causal]
    c = int(is_causal)
    if c not in (0, 1, 2):
        raise SageError(SAGE_E_INVALID, "is_causal must be False, True, 2 or a name (got %r)" % (is_causal,))
    return c


def _dtype_code(t):
    if t == torch.float16:
        return SAGE_FP16
    if t == torch.bfloat16:
        return SAGE_BF16
    raise SageError(SAGE_E_INVALID, "dtype %s is not float16/bfloat16" % t)


def _bht_strides(x, layout):
    s = x.stride()
    if x.dim() != 4:
        raise SageError(SAGE_E_INVALID, "expected a 4-d tensor, got shape %s" % (tuple(x.shape),))
    if x.shape[3] > 1 and s[3] != 1:
        raise SageError(SAGE_E_INVALID, "the head-dim stride must be 1")
    return (s[0], s[1], s[2]) if layout == "HND" else (s[0], s[2], s[1])


def _bhld(x, layout):
    B, a, b, D = x.shape
    return (B, a, b, D) if layout == "HND" else (B, b, a, D)


def _pv_code(pv):
    if pv not in _PV_CODES:
        raise SageError(SAGE_E_INVALID, "pv must be 'fp8' or 'fp16', got %r" % (pv,))
    return _PV_CODES[pv]


def make_problem(q, k, v, o=None, tensor_layout="HND", pv="fp8"):
    """Problem for the given tensors (shapes, dtype and element strides).

    pv: "fp8" (FP8 P and V) or "fp16" (P and V in the inputs' 16-bit format)."""
    if tensor_layout not in ("HND", "NHD"):
        raise SageError(SAGE_E_INVALID, "tensor_layout must be 'HND' or 'NHD'")
    B, Hq, Lq, D = _bhld(q, tensor_layout)
    Bk, Hkv, Lk, Dk = _bhld(k, tensor_layout)
    if _bhld(v, tensor_layout) != (Bk, Hkv, Lk, Dk) or Bk != B or Dk != D:
        raise SageError(SAGE_E_INVALID, "q %s, k %s, v %s shapes are inconsistent"
                        % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if not (q.dtype == k.dtype == v.dtype):
        raise SageError(SAGE_E_INVALID, "q, k, v must share one dtype")
    p = Problem()
    p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.D = B, Hq, Hkv, Lq, Lk, D
    p.dtype = _dtype_code(q.dtype)
    p.pv = _pv_code(pv)
    p.q_stride[:] = _bht_strides(q, tensor_layout)
    p.k_stride[:] = _bht_strides(k, tensor_layout)
    p.v_stride[:] = _bht_strides(v, tensor_layout)
    if o is not None:
        if _bhld(o, tensor_layout) != (B, Hq, Lq, D) or o.dtype != q.dtype:
            raise SageError(SAGE_E_INVALID, "o must match q's shape and dtype")
        p.o_stride[:] = _bht_strides(o, tensor_layout)
    else:
        p.o_stride[:] = _bht_strides(q, tensor_layout) if q.is_contiguous() else (0, 0, 0)
    return p


def contiguous_problem(layout, B, Hq, Hkv, Lq, Lk, D, dtype, pv="fp8"):
    p = Problem()
    code = SAGE_HND if layout == "HND" else SAGE_NHD
    _check(lib().sage_problem_init(ctypes.byref(p), code, B, Hq, Hkv, Lq, Lk, D, _dtype_code(dtype)))
    p.pv = _pv_code(pv)
    check_problem(p)
    return p


def check_problem(p):
    _check(lib().sage_problem_check(ctypes.byref(p)))


def workspace_layout(p):
    L = WsLayout()
    _check(lib().sage_workspace_layout(ctypes.byref(p), ctypes.byref(L)))
    return L


def workspace_bytes(p):
    n = lib().sage_workspace_bytes(ctypes.byref(p))
    if n == 0:
        _check(lib().sage_problem_check(ctypes.byref(p)))
    return n


SAGE_REF_MAX = 0
SAGE_REF_LAZY = 2


def softmax_spec(pv="fp8"):
    """(keys per online-softmax step, reference rule) of a P.V format: the rule
    is "lazy" (SAGE_REF_LAZY, FP8 P.V) or "max" (SAGE_REF_MAX, 16-bit P.V)."""
    bk, ref = ctypes.c_int(), ctypes.c_int()
    _check(lib().sage_softmax_spec(_pv_code(pv), ctypes.byref(bk), ctypes.byref(ref)))
    return bk.value, {SAGE_REF_MAX: "max", SAGE_REF_LAZY: "lazy"}[ref.value]


def softmax_block_keys():
    return lib().sage_softmax_block_keys()


def new_workspace(p, device="cuda"):
    # torch's caching allocator returns 256-byte (or larger) aligned blocks
    return torch.empty(workspace_bytes(p), dtype=torch.uint8, device=device)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def quantize(p, q, k, v, ws, smooth_k=True):
    """Run the quantization prologue into workspace tensor ws (uint8, device)."""
    _check(lib().sage_quantize(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), int(bool(smooth_k)),
                               _ptr(ws), ws.numel(), _stream()))


def attn_quantized(p, ws, o, is_causal=False, sm_scale=None):
    """Attention on a quantized workspace; writes o."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(p.D)
    _check(lib().sage_attn_quantized(ctypes.byref(p), _ptr(ws), ws.numel(), _ptr(o),
                                     causal_code(is_causal), float(sm_scale), _stream()))


def attn(p, q, k, v, o, ws, is_causal=False, sm_scale=None, smooth_k=True):
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(p.D)
    _check(lib().sage_attn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                           causal_code(is_causal), float(sm_scale), int(bool(smooth_k)),
                           _ptr(ws), ws.numel(), _stream()))


def split_count(p):
    """Key ranges the library picks for problem p."""
    n = lib().sage_split_count(ctypes.byref(p))
    if n == 0:
        _check(lib().sage_problem_check(ctypes.byref(p)))
    return n


def split_bytes(p, nsplit=0):
    """Scratch bytes a run of p with nsplit key ranges needs (0 = the library's choice)."""
    _check(lib().sage_problem_check(ctypes.byref(p)))
    return lib().sage_split_bytes(ctypes.byref(p), int(nsplit))


def block_mask_shape(p):
    """Shape of the block mask of dense problem p: (B, Hq, ceil(Lq/128), ceil(Lk/128))."""
    return (p.B, p.Hq, -(-p.Lq // MASK_BLOCK_Q), -(-p.Lk // MASK_BLOCK_K))


def _mask_tensor(p, block_mask):
    if block_mask is None:
        return None
    if not block_mask.is_cuda:
        raise SageError(SAGE_E_INVALID, "block_mask must be a device tensor")
    if tuple(block_mask.shape) != block_mask_shape(p):
        raise SageError(SAGE_E_INVALID, "block_mask has shape %s, the problem needs %s"
                        % (tuple(block_mask.shape), block_mask_shape(p)))
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.view(torch.uint8)
    if block_mask.dtype != torch.uint8:
        raise SageError(SAGE_E_INVALID, "block_mask must be uint8 or bool")
    return block_mask.contiguous()


def _opts(is_causal, sm_scale, nsplit, lse, part, block_mask=None):
    op = AttnOpts()
    op.is_causal = causal_code(is_causal)
    op.nsplit = int(nsplit)
    op.sm_scale = float(sm_scale)
    op.reserved = 0
    op.lse = lse.data_ptr() if lse is not None else None
    op.part = part.data_ptr() if part is not None else None
    op.part_bytes = part.numel() * part.element_size() if part is not None else 0
    op.block_mask = block_mask.data_ptr() if block_mask is not None else None
    return op


def attn_quantized_ex(p, ws, o, is_causal=False, sm_scale=None, nsplit=0, lse=None, part=None,
                      block_mask=None):
    """Attention on a quantized workspace with key ranges, an optional LSE and block mask.

    nsplit: key ranges per query tile (0 = the library's choice); lse: None or
    a float32 device tensor of B * Hq * Lq elements; part: split scratch
    (allocated here when needed and not given); block_mask: None or a uint8 /
    bool device tensor of block_mask_shape(p), nonzero = block computed."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(p.D)
    if part is None:
        n = split_bytes(p, nsplit)
        if n:
            part = torch.empty(n, dtype=torch.uint8, device=ws.device)
    block_mask = _mask_tensor(p, block_mask)
    op = _opts(is_causal, sm_scale, nsplit, lse, part, block_mask)
    _check(lib().sage_attn_quantized_ex(ctypes.byref(p), _ptr(ws), ws.numel(), _ptr(o), ctypes.byref(op),
                                        _stream()))


def attn_ex(p, q, k, v, o, ws, smooth_k=True, is_causal=False, sm_scale=None, nsplit=0, lse=None,
            part=None, block_mask=None):
    """The whole path in one call (sage_attn_ex): the K/V prologue, then the
    attention kernel, which quantizes Q itself; the same result as quantize()
    followed by attn_quantized_ex(), bit for bit. Options as in attn_quantized_ex."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(p.D)
    if part is None:
        n = split_bytes(p, nsplit)
        if n:
            part = torch.empty(n, dtype=torch.uint8, device=ws.device)
    block_mask = _mask_tensor(p, block_mask)
    op = _opts(is_causal, sm_scale, nsplit, lse, part, block_mask)
    _check(lib().sage_attn_ex(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), int(bool(smooth_k)), _ptr(ws),
                              ws.numel(), ctypes.byref(op), _stream()))


NOALLOC_SCRATCH_BYTES = 96 << 20


def noalloc_bytes(p, nsplit=0):
    """Scratch bytes sage_attn_noalloc needs for problem p (0 if p is invalid)."""
    return int(lib().sage_noalloc_bytes(ctypes.byref(p), int(nsplit)))


def attn_noalloc(p, q, k, v, o, smooth_k=True, is_causal=False, sm_scale=None, nsplit=0, lse=None,
                 block_mask=None):
    """attn_ex() with the workspace and split partials in the library's static
    per-GPU scratch (sage_attn_noalloc): neither the caller nor the library
    allocates device memory. Calls that overlap in time on one GPU race."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(p.D)
    block_mask = _mask_tensor(p, block_mask)
    op = _opts(is_causal, sm_scale, nsplit, lse, None, block_mask)
    _check(lib().sage_attn_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), int(bool(smooth_k)),
                                   ctypes.byref(op), _stream()))


def quantize_kv(p, k, v, ws, smooth_k=True):
    """The K/V part of the prologue (sage_quantize_kv); the Q sections are left unwritten."""
    _check(lib().sage_quantize_kv(ctypes.byref(p), _ptr(k), _ptr(v), int(bool(smooth_k)), _ptr(ws), ws.numel(),
                                  _stream()))


def attn_q_ex(p, q, ws, o, is_causal=False, sm_scale=None, nsplit=0, lse=None, part=None, block_mask=None):
    """Attention on a workspace with K/V written, quantizing Q from q in the kernel
    (sage_attn_q_ex). quantize_kv() then attn_q_ex() is the one-call path attn_ex()."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(p.D)
    if part is None:
        n = split_bytes(p, nsplit)
        if n:
            part = torch.empty(n, dtype=torch.uint8, device=ws.device)
    block_mask = _mask_tensor(p, block_mask)
    op = _opts(is_causal, sm_scale, nsplit, lse, part, block_mask)
    _check(lib().sage_attn_q_ex(ctypes.byref(p), _ptr(q), _ptr(ws), ws.numel(), _ptr(o), ctypes.byref(op),
                                _stream()))


def debug_qk_int32(p, ws, b, hq):
    """int32 logits of head (b, hq) from the attention kernel's tile routine."""
    L = workspace_layout(p)
    out = torch.empty((L.Lq_pad, L.Lk_pad), dtype=torch.int32, device=ws.device)
    _check(lib().sage_debug_qk_int32(ctypes.byref(p), _ptr(ws), ws.numel(), int(b), int(hq),
                                     _ptr(out), _stream()))
    return out


def workspace_views(p, ws):
    """Tensor views of the quantized workspace (for inspection and tests)."""
    L = workspace_layout(p)
    B, Hq, Hkv, Dp = p.B, p.Hq, p.Hkv, L.Dp

    def view(off, n, dtype, shape):
        return ws[off:off + n * torch.tensor([], dtype=dtype).element_size()].view(dtype).view(shape)

    return dict(
        layout=L,
        qhat=view(L.qhat, B * Hq * L.Lq_pad * Dp, torch.int8, (B, Hq, L.Lq_pad, Dp)),
        sq=view(L.sq, B * Hq * L.Lq_pad, torch.float32, (B, Hq, L.Lq_pad)),
        khat=view(L.khat, B * Hkv * L.Lk_pad * Dp, torch.int8, (B, Hkv, L.Lk_pad, Dp)),
        sk=view(L.sk, B * Hkv * L.nkb, torch.float32, (B, Hkv, L.nkb)),
        kbar=view(L.kbar, B * Hkv * Dp, torch.float32, (B, Hkv, Dp)),
        vhat=(view(L.vhat, B * Hkv * L.nkb * Dp * 64, torch.uint8, (B, Hkv, L.nkb, Dp, 64))
              if p.pv == SAGE_PV_FP8 else
              view(L.vhat, B * Hkv * L.nkb * Dp * 64, torch.int16, (B, Hkv, L.nkb, Dp, 64))),
        vmax=view(L.vmax, B * Hkv * Dp, torch.float32, (B, Hkv, Dp)),
    )


def vhat_position(j, pv="fp8"):
    """Position of token j (0..63) inside a permuted 64-token V^T block of the workspace."""
    if _pv_code(pv) == SAGE_PV_FP16:
        return (j & ~12) | ((j >> 1) & 4) | ((j << 1) & 8)
    return 32 * ((j >> 2) & 1) + 16 * (j >> 5) + 4 * ((j >> 3) & 3) + (j & 3)


def sageattn(q, k, v, tensor_layout="HND", is_causal=False, sm_scale=None, smooth_k=True,
             workspace=None, pv="fp8", return_lse=False, nsplit=0, block_mask=None):
    """Quantized attention (INT8 QK^T with smoothed K, FP8 or 16-bit P.V) on the GPU.

    sm_scale defaults to 1/sqrt(D) of the given head dim. The output has q's
    shape, layout and dtype. ``workspace`` may pass a preallocated uint8
    device tensor of at least ``workspace_bytes`` bytes. ``pv`` selects the
    P.V format: "fp8" (default) or "fp16" (the inputs' 16-bit format).
    ``is_causal``: False, True (top-left) or "bottom_right". With
    ``return_lse`` the result is (o, lse), lse float32 [B, Hq, Lq].
    ``nsplit``: key ranges per query tile, 0 = picked from the shape.
    ``block_mask``: None, or uint8 / bool [B, Hq, ceil(Lq/128), ceil(Lk/128)]
    on the device; a zero flag skips that block of 128 queries x 128 keys.
    """
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise SageError(SAGE_E_INVALID, "q, k and v must be device tensors")
    o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    p = make_problem(q, k, v, o, tensor_layout, pv=pv)
    ws = workspace if workspace is not None else new_workspace(p, q.device)
    lse = torch.empty((p.B, p.Hq, p.Lq), dtype=torch.float32, device=q.device) if return_lse else None
    attn_ex(p, q, k, v, o, ws, smooth_k=smooth_k, is_causal=is_causal, sm_scale=sm_scale, nsplit=nsplit,
            lse=lse, block_mask=block_mask)
    return (o, lse) if return_lse else o


def block_sparse_sageattn(q, k, v, block_mask, tensor_layout="HND", is_causal=False, sm_scale=None,
                          smooth_k=True, pv="fp8", return_lse=False, nsplit=0, workspace=None):
    """Quantized attention under a block-sparse pattern (the pages' Sparse SageAttention API):
    block_mask uint8 / bool [B, Hq, ceil(Lq/128), ceil(Lk/128)] on the device, nonzero =
    the block of 128 queries x 128 keys is computed, zero = skipped (-inf logits)."""
    return sageattn(q, k, v, tensor_layout, is_causal, sm_scale, smooth_k, workspace, pv=pv,
                    return_lse=return_lse, nsplit=nsplit, block_mask=block_mask)


def sageattn_qk_int8_pv_fp8(q, k, v, tensor_layout="HND", is_causal=False, sm_scale=None,
                            smooth_k=True, workspace=None, return_lse=False):
    """INT8 QK^T, FP8 P.V ("8+8")."""
    return sageattn(q, k, v, tensor_layout, is_causal, sm_scale, smooth_k, workspace, pv="fp8",
                    return_lse=return_lse)


def sageattn_qk_int8_pv_fp16(q, k, v, tensor_layout="HND", is_causal=False, sm_scale=None,
                             smooth_k=True, workspace=None, return_lse=False):
    """INT8 QK^T, 16-bit P.V ("8+16"; bf16 inputs use bfloat16 P and V)."""
    return sageattn(q, k, v, tensor_layout, is_causal, sm_scale, smooth_k, workspace, pv="fp16",
                    return_lse=return_lse)


# --------------------------------------------------------------------------
# Packed variable-length sequences
# --------------------------------------------------------------------------
def make_varlen_problem(q, k, v, o, B, max_seqlen_q, max_seqlen_k, pv="fp16"):
    """Problem for B packed sequences: q [total_q, Hq, D], k/v [total_k, Hkv, D] (strided views allowed)."""
    for name, x in (("q", q), ("k", k), ("v", v), ("o", o)):
        if x.dim() != 3:
            raise SageError(SAGE_E_INVALID, "%s must be [total, H, D], got %s" % (name, tuple(x.shape)))
        if x.shape[2] > 1 and x.stride(2) != 1:
            raise SageError(SAGE_E_INVALID, "the head-dim stride of %s must be 1" % name)
    if not (q.dtype == k.dtype == v.dtype == o.dtype):
        raise SageError(SAGE_E_INVALID, "q, k, v, o must share one dtype")
    if k.shape != v.shape or q.shape[2] != k.shape[2] or o.shape != q.shape:
        raise SageError(SAGE_E_INVALID, "q %s, k %s, v %s, o %s shapes are inconsistent"
                        % (tuple(q.shape), tuple(k.shape), tuple(v.shape), tuple(o.shape)))
    p = VarlenProblem()
    p.B = B
    p.Hq, p.Hkv, p.D = q.shape[1], k.shape[1], q.shape[2]
    p.dtype = _dtype_code(q.dtype)
    p.pv = _pv_code(pv)
    p.total_q, p.total_k = q.shape[0], k.shape[0]
    p.max_seqlen_q, p.max_seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    p.q_stride[:] = (q.stride(0), q.stride(1))
    p.k_stride[:] = (k.stride(0), k.stride(1))
    p.v_stride[:] = (v.stride(0), v.stride(1))
    p.o_stride[:] = (o.stride(0), o.stride(1))
    _check(lib().sage_varlen_problem_check(ctypes.byref(p)))
    return p


def varlen_workspace_layout(p):
    L = WsLayout()
    _check(lib().sage_varlen_workspace_layout(ctypes.byref(p), ctypes.byref(L)))
    return L


def varlen_workspace_bytes(p):
    n = lib().sage_varlen_workspace_bytes(ctypes.byref(p))
    if n == 0:
        _check(lib().sage_varlen_problem_check(ctypes.byref(p)))
    return n


def varlen_attn(p, q, k, v, o, cu_seqlens_q, cu_seqlens_k, ws, is_causal=False, sm_scale=None,
                smooth_k=True):
    """Packed prologue + attention into o with a caller-owned workspace ws."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(p.D)
    _check(lib().sage_varlen_attn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                  _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), causal_code(is_causal),
                                  float(sm_scale), int(bool(smooth_k)), _ptr(ws), ws.numel(), _stream()))


def varlen_split_count(p):
    n = lib().sage_varlen_split_count(ctypes.byref(p))
    if n == 0:
        _check(lib().sage_varlen_problem_check(ctypes.byref(p)))
    return n


def varlen_split_bytes(p, nsplit=0):
    _check(lib().sage_varlen_problem_check(ctypes.byref(p)))
    return lib().sage_varlen_split_bytes(ctypes.byref(p), int(nsplit))


def varlen_attn_ex(p, q, k, v, o, cu_seqlens_q, cu_seqlens_k, ws, is_causal=False, sm_scale=None,
                   smooth_k=True, nsplit=0, lse=None, part=None):
    """Packed prologue + attention with key ranges and an optional LSE ([Hq, total_q] float32)."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(p.D)
    if part is None:
        n = varlen_split_bytes(p, nsplit)
        if n:
            part = torch.empty(n, dtype=torch.uint8, device=ws.device)
    op = _opts(is_causal, sm_scale, nsplit, lse, part)
    _check(lib().sage_varlen_attn_ex(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                     _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), int(bool(smooth_k)),
                                     _ptr(ws), ws.numel(), ctypes.byref(op), _stream()))


def sageattn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    is_causal=False, sm_scale=None, smooth_k=True, pv="fp16", workspace=None,
                    return_lse=False, nsplit=0):
    """Quantized attention over packed variable-length sequences.

    q: [total_q, Hq, D], k, v: [total_k, Hkv, D] fp16/bf16 on the GPU;
    cu_seqlens_q / cu_seqlens_k: int32 device tensors of B + 1 offsets;
    max_seqlen_q / max_seqlen_k: the longest sequence lengths (ints).
    Each sequence is attended on its own (its own smoothing, scales and causal
    mask). pv defaults to "fp16", the reference's sageattn_varlen format.
    With ``return_lse`` the result is (o, lse), lse float32 [Hq, total_q].
    """
    for name, x in (("q", q), ("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_k", cu_seqlens_k)):
        if not x.is_cuda:
            raise SageError(SAGE_E_INVALID, "%s must be a device tensor" % name)
    for name, c in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous():
            raise SageError(SAGE_E_INVALID, "%s must be a contiguous 1-d int32 tensor" % name)
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise SageError(SAGE_E_INVALID, "cu_seqlens_q and cu_seqlens_k must both hold B + 1 >= 2 offsets")
    B = cu_seqlens_q.numel() - 1
    o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    p = make_varlen_problem(q, k, v, o, B, max_seqlen_q, max_seqlen_k, pv=pv)
    n = varlen_workspace_bytes(p)
    ws = workspace if workspace is not None else torch.empty(n, dtype=torch.uint8, device=q.device)
    lse = torch.empty((p.Hq, p.total_q), dtype=torch.float32, device=q.device) if return_lse else None
    varlen_attn_ex(p, q, k, v, o, cu_seqlens_q, cu_seqlens_k, ws, is_causal=is_causal, sm_scale=sm_scale,
                   smooth_k=smooth_k, nsplit=nsplit, lse=lse)
    return (o, lse) if return_lse else o
