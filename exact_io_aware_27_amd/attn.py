"""Thin ctypes binding of libattn.so (include/attn.h).

Argument marshalling only: tensors become device pointers, the stream
becomes a hipStream_t handle, and a nonzero status becomes an exception.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  If the library is missing, loading raises.

torch is imported before the library is opened so that libattn.so binds to
the HIP runtime torch already loaded (both carry the soname
libamdhip64.so.7): one runtime per process, so torch's streams and device
pointers are valid in the library.
"""

import ctypes
import os

import torch  # noqa: F401  (must be loaded first: see the module docstring)

# ATTN_LIB_PATH: another build of the same sources (the host-sanitizer build
# of tests/sanitize_cpu.py); by default the in-tree library.
LIB_PATH = os.environ.get("ATTN_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK = 0
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_NULL_PTR", 2: "ATTN_BAD_SHAPE", 3: "ATTN_UNSUPPORTED_D",
                4: "ATTN_BAD_SCALE", 5: "ATTN_MISALIGNED", 6: "ATTN_ALIAS", 7: "ATTN_HIP",
                8: "ATTN_BAD_WORKSPACE", 9: "ATTN_BAD_ARGUMENT", 10: "ATTN_SCRATCH_TOO_SMALL"}
EXPORTS = ("attn_fwd", "attn_fwd_splitkv", "attn_fwd_splitkv_noalloc", "attn_noalloc_scratch_bytes",
           "attn_fwd_splitkv_workspace_bytes", "attn_bwd",
           "attn_bwd_workspace_bytes", "attn_fp8_padded_rows", "attn_fp8_quantize", "attn_fp8_quantize_q", "attn_fwd_fp8",
           "attn_status_string", "attn_last_hip_error")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, hip_error=0):
        self.status = status
        self.hip_error = hip_error
        msg = STATUS_NAMES.get(status, str(status))
        if hip_error:
            msg += " (hipError %d)" % hip_error
        super().__init__(msg)


def load():
    """Open libattn.so and declare its signatures; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            "libattn.so is not built (%s); run __graft_entry__.build() or "
            "python exact_io_aware_27_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [p, p, p, p, p, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float, p]
    lib.attn_fwd_splitkv.restype = ctypes.c_int
    lib.attn_fwd_splitkv.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                     i64, p, i64, p]
    lib.attn_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.attn_fwd_splitkv_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, ctypes.c_int,
                                             ctypes.c_float, i64, p]
    lib.attn_noalloc_scratch_bytes.restype = i64
    lib.attn_noalloc_scratch_bytes.argtypes = []
    lib.attn_fwd_splitkv_workspace_bytes.restype = i64
    lib.attn_fwd_splitkv_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                             p, i64, p]
    lib.attn_bwd_workspace_bytes.restype = i64
    lib.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.attn_fp8_padded_rows.restype = i64
    lib.attn_fp8_padded_rows.argtypes = [i64]
    lib.attn_fp8_quantize.restype = ctypes.c_int
    lib.attn_fp8_quantize.argtypes = [p, i64, i64, i64, i64, ctypes.c_int, p, p, p, p]
    lib.attn_fwd_fp8.restype = ctypes.c_int
    lib.attn_fp8_quantize_q.restype = ctypes.c_int
    lib.attn_fp8_quantize_q.argtypes = [p, i64, i64, i64, i64, p, ctypes.c_float, p, p, p]
    lib.attn_fwd_fp8.restype = ctypes.c_int
    lib.attn_fwd_fp8.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, ctypes.c_int, p]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_last_hip_error.restype = ctypes.c_int
    lib.attn_last_hip_error.argtypes = []
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # torch.cuda.Stream


def _check(x, name, shape, dtype):
    """Tensors handed to the kernel must be exactly what its grid assumes."""
    if x is None or isinstance(x, int):
        return
    if x.dtype != dtype or tuple(x.shape) != shape or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("%s must be a contiguous %s CUDA tensor of shape %s, got %s %s %s"
                         % (name, dtype, shape, x.dtype, tuple(x.shape), x.device))


def attn_fwd_status(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None):
    """Call attn_fwd and return its status code (0 = ATTN_OK).

    q, k, v, o: device tensors (or raw pointers) bf16 [B, H, N, d];
    lse: fp32 [B, H, N] device tensor, pointer, or None;
    stream: torch.cuda.Stream, a raw hipStream_t, or None (null stream).
    Tensors are checked against (B, H, N, d); raw pointers are the caller's
    responsibility.
    """
    shape = (int(B), int(H), int(N), int(d))
    for x, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check(x, name, shape, torch.bfloat16)
    _check(lse, "lse", shape[:3], torch.float32)
    lib = load()
    return lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(N),
                        int(d), 1 if causal else 0, float(scale), _stream(stream))


def attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None):
    """attn_fwd of include/attn.h; raises AttnError on a nonzero status."""
    st = attn_fwd_status(q, k, v, o, lse, B, H, N, d, causal, scale, stream)
    if st != ATTN_OK:
        raise AttnError(st, load().attn_last_hip_error() if st == 7 else 0)


def attention(q, k, v, causal=False, scale=None, with_lse=True, stream=None):
    """Allocate O (and LSE) like q and run attn_fwd on torch's current stream.

    q, k, v: contiguous bf16 CUDA tensors [B, H, N, d].  Returns (o, lse).
    """
    B, H, N, d = q.shape
    if scale is None:
        scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if with_lse else None
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream)
    return o, lse


def splitkv_workspace_bytes(B, H, Nq, d, num_splits):
    """attn_fwd_splitkv_workspace_bytes of include/attn.h (-1: invalid arguments)."""
    return load().attn_fwd_splitkv_workspace_bytes(int(B), int(H), int(Nq), int(d), int(num_splits))


def attn_fwd_splitkv_status(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits,
                            workspace, workspace_bytes, stream=None):
    """Call attn_fwd_splitkv and return its status code (0 = ATTN_OK).

    q, o: bf16 [B, H, Nq, d]; k, v: bf16 [B, H, Nk, d]; lse: fp32 [B, H, Nq]
    or None; workspace: a device tensor (its data pointer is passed), a raw
    pointer, or None.  Tensors are checked against the shapes; raw pointers
    are the caller's responsibility.
    """
    qs, ks = (int(B), int(H), int(Nq), int(d)), (int(B), int(H), int(Nk), int(d))
    _check(q, "q", qs, torch.bfloat16)
    _check(o, "o", qs, torch.bfloat16)
    _check(k, "k", ks, torch.bfloat16)
    _check(v, "v", ks, torch.bfloat16)
    _check(lse, "lse", qs[:3], torch.float32)
    lib = load()
    return lib.attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq),
                                int(Nk), int(d), 1 if causal else 0, float(scale), int(num_splits),
                                _ptr(workspace), int(workspace_bytes), _stream(stream))


def attn_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, workspace,
                     workspace_bytes, stream=None):
    """attn_fwd_splitkv of include/attn.h; raises AttnError on a nonzero status."""
    st = attn_fwd_splitkv_status(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits,
                                 workspace, workspace_bytes, stream)
    if st != ATTN_OK:
        raise AttnError(st, load().attn_last_hip_error() if st == 7 else 0)


def noalloc_scratch_bytes():
    """attn_noalloc_scratch_bytes of include/attn.h: the per-GPU scratch size."""
    return load().attn_noalloc_scratch_bytes()


def attn_fwd_splitkv_noalloc_status(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, stream=None):
    """Call attn_fwd_splitkv_noalloc and return its status code (0 = ATTN_OK).
    Arguments as attn_fwd_splitkv_status, without the workspace."""
    qs, ks = (int(B), int(H), int(Nq), int(d)), (int(B), int(H), int(Nk), int(d))
    _check(q, "q", qs, torch.bfloat16)
    _check(o, "o", qs, torch.bfloat16)
    _check(k, "k", ks, torch.bfloat16)
    _check(v, "v", ks, torch.bfloat16)
    _check(lse, "lse", qs[:3], torch.float32)
    lib = load()
    return lib.attn_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq),
                                        int(Nk), int(d), 1 if causal else 0, float(scale), int(num_splits),
                                        _stream(stream))


def attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, stream=None):
    """attn_fwd_splitkv_noalloc of include/attn.h; raises AttnError on a nonzero status."""
    st = attn_fwd_splitkv_noalloc_status(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, stream)
    if st != ATTN_OK:
        raise AttnError(st, load().attn_last_hip_error() if st == 7 else 0)


def attention_splitkv(q, k, v, num_splits, causal=False, scale=None, with_lse=True, stream=None,
                      workspace=None):
    """Allocate O (and LSE, and the workspace unless given) and run
    attn_fwd_splitkv on torch's current stream.

    q: contiguous bf16 CUDA tensor [B, H, Nq, d]; k, v: [B, H, Nk, d].
    Returns (o, lse).
    """
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if with_lse else None
    nbytes = splitkv_workspace_bytes(B, H, Nq, d, num_splits)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    attn_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, workspace,
                     max(nbytes, 0) if workspace is not None else 0, stream)
    return o, lse


def bwd_workspace_bytes(B, H, N, d):
    """attn_bwd_workspace_bytes of include/attn.h (-1: invalid arguments)."""
    return load().attn_bwd_workspace_bytes(int(B), int(H), int(N), int(d))


def attn_bwd_status(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, causal, scale, workspace,
                    workspace_bytes, stream=None):
    """Call attn_bwd and return its status code (0 = ATTN_OK).

    q, k, v, o, dout, dq, dk, dv: bf16 [B, H, N, d]; lse: fp32 [B, H, N] (the
    forward pass's); workspace: a device tensor, a raw pointer, or None.
    Tensors are checked against the shapes; raw pointers are the caller's
    responsibility.
    """
    shape = (int(B), int(H), int(N), int(d))
    for x, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
                    (dv, "dv")):
        _check(x, name, shape, torch.bfloat16)
    _check(lse, "lse", shape[:3], torch.float32)
    lib = load()
    return lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                        _ptr(dv), int(B), int(H), int(N), int(d), 1 if causal else 0, float(scale),
                        _ptr(workspace), int(workspace_bytes), _stream(stream))


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, causal, scale, workspace, workspace_bytes,
             stream=None):
    """attn_bwd of include/attn.h; raises AttnError on a nonzero status."""
    st = attn_bwd_status(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, causal, scale, workspace,
                         workspace_bytes, stream)
    if st != ATTN_OK:
        raise AttnError(st, load().attn_last_hip_error() if st == 7 else 0)


def attention_bwd(q, k, v, o, lse, dout, causal=False, scale=None, stream=None, workspace=None):
    """Allocate dQ, dK, dV (and the workspace unless given) and run attn_bwd
    on torch's current stream.

    q, k, v, o, dout: contiguous bf16 CUDA tensors [B, H, N, d]; lse: the
    forward pass's fp32 [B, H, N].  Returns (dq, dk, dv).
    """
    B, H, N, d = q.shape
    if scale is None:
        scale = d ** -0.5
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, causal, scale, workspace,
             workspace.numel() * workspace.element_size(), stream)
    return dq, dk, dv


def fp8_padded_rows(N):
    """attn_fp8_padded_rows of include/attn.h: N rounded up to 64."""
    return load().attn_fp8_padded_rows(int(N))


def sign_bits(signs):
    """+-1 signs [128] -> the 4-word host bit array attn_fp8_quantize takes
    (bit c set: sign of column c is -1)."""
    neg = [float(x) < 0 for x in (signs.tolist() if hasattr(signs, "tolist") else signs)]
    if len(neg) != 128:
        raise ValueError("signs must hold 128 values")
    words = (ctypes.c_uint32 * 4)()
    for c, is_neg in enumerate(neg):
        if is_neg:
            words[c // 32] |= 1 << (c % 32)
    return words


def fp8_quantize_status(x, B, H, N, d, transpose, signs, out, exps, stream=None, scale=None):
    """Call attn_fp8_quantize (scale None: K or V) or attn_fp8_quantize_q
    (scale given: Q, with transpose False) and return its status.  signs:
    None or +-1 [128]."""
    lib = load()
    bits = None if signs is None else sign_bits(signs)
    bits_p = None if bits is None else ctypes.cast(bits, ctypes.c_void_p)
    if scale is not None:
        if transpose:
            raise ValueError("Q is quantized without the transposed layout")
        return lib.attn_fp8_quantize_q(_ptr(x), int(B), int(H), int(N), int(d), bits_p, float(scale),
                                       _ptr(out), _ptr(exps), _stream(stream))
    return lib.attn_fp8_quantize(_ptr(x), int(B), int(H), int(N), int(d), 1 if transpose else 0, bits_p,
                                 _ptr(out), _ptr(exps), _stream(stream))


def fp8_quantize(x, transpose=False, signs=None, stream=None, scale=None):
    """Quantize a contiguous bf16 CUDA tensor [B, H, N, 128] to FP8 (with
    `scale`, the softmax scale: as Q, by attn_fp8_quantize_q).

    Returns (codes, exps): uint8 tensors [B, H, Np, 128] (or [B, H, 128, Np]
    with transpose, in the kernel's key order) and [B, H, Np // 64].
    """
    B, H, N, d = x.shape
    _check(x, "x", (B, H, N, d), torch.bfloat16)
    Np = fp8_padded_rows(N)
    shape = (B, H, d, Np) if transpose else (B, H, Np, d)
    out = torch.empty(shape, dtype=torch.uint8, device=x.device)
    exps = torch.empty((B, H, Np // 64), dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    st = fp8_quantize_status(x, B, H, N, d, transpose, signs, out, exps, stream, scale)
    if st != ATTN_OK:
        raise AttnError(st, load().attn_last_hip_error() if st == 7 else 0)
    return out, exps


def attn_fwd_fp8_status(q8, k8, vt8, qe, ke, ve, o, lse, B, H, N, d, causal, stream=None):
    """Call attn_fwd_fp8 and return its status (0 = ATTN_OK)."""
    _check(o, "o", (int(B), int(H), int(N), int(d)), torch.bfloat16)
    _check(lse, "lse", (int(B), int(H), int(N)), torch.float32)
    lib = load()
    return lib.attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), _ptr(qe), _ptr(ke), _ptr(ve), _ptr(o), _ptr(lse),
                            int(B), int(H), int(N), int(d), 1 if causal else 0, _stream(stream))


def attn_fwd_fp8(q8, k8, vt8, qe, ke, ve, o, lse, B, H, N, d, causal, stream=None):
    """attn_fwd_fp8 of include/attn.h; raises AttnError on a nonzero status."""
    st = attn_fwd_fp8_status(q8, k8, vt8, qe, ke, ve, o, lse, B, H, N, d, causal, stream)
    if st != ATTN_OK:
        raise AttnError(st, load().attn_last_hip_error() if st == 7 else 0)


def attention_fp8(q, k, v, causal=False, scale=None, signs=None, stream=None):
    """Quantize q, k (rotated with `signs` when given) and v, then run
    attn_fwd_fp8 on torch's current stream.  q, k, v: contiguous bf16 CUDA
    tensors [B, H, N, 128].  Returns (o, lse)."""
    B, H, N, d = q.shape
    if scale is None:
        scale = d ** -0.5
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    q8, qe = fp8_quantize(q, signs=signs, stream=stream, scale=scale)
    k8, ke = fp8_quantize(k, signs=signs, stream=stream)
    vt8, ve = fp8_quantize(v, transpose=True, stream=stream)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    attn_fwd_fp8(q8, k8, vt8, qe, ke, ve, o, lse, B, H, N, d, causal, stream)
    return o, lse
