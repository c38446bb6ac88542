"""ggml_q2_dequant_amd — the Q2_K weight path on MI355X (gfx950).

A thin ctypes binding over ``libq2k.so`` (C ABI in ``include/q2k.h``). Every
step of the path runs in the library's HIP kernels; this module only turns
torch device tensors into pointers and sizes and raises on a non-zero status.
PyTorch supplies device memory and the current stream, nothing else.

Functions carry the C names:

* ``q2k_dequantize(blocks, out)`` — decode whole 84-byte blocks to f32.
* ``q2k_matmul(x, w, y, M, N, K)`` — y[M, N] = x[M, K] * W[N, K]^T, W in Q2_K.
* ``q2k_matmul_path(x, w, y, M, N, K, path)`` — same with a forced kernel;
  ``q2k_matmul_pooled`` takes caller-held scratch of ``q2k_matmul_scratch_bytes``
  bytes instead of the library's per-stream workspace.
* ``q2k_matmul_batched(x, w, y, batches, M, N, K)`` — independent products, one
  per matrix of a batch-major stack (1 <= M <= 8).
* ``q2k_embedding_gather(table, ids, out, vocab, embed_dim, n_tokens)`` — rows
  of a Q2_K table; raises ``Q2KIdOutOfRange`` for an id >= vocab.
* ``q2k_embedding_gather_async(table, ids, out, vocab, embed_dim, n_tokens,
  status)`` — the same without waiting; a bad id sets the device int ``status``.
* ``q2k_argmax_candidates(logits, n_slots, vocab, cap, top1_idx, top1_val,
  cand_count, overflow, cand_ids)`` — first-max argmax and the logits within
  0.5 of it, per slot; ``q2k_argmax_candidates_pooled`` with caller-held scratch.
* ``q2k_matmul_id(x, w, ids, y, params, status=None)`` — the expert-routed
  product (route token*top_k+slot uses expert ids[route]); ``q2k_matmul_id_path``
  forces a schedule; ``q2k_matmul_id_pooled``, ``..._pooled_pair`` and
  ``..._pooled_slotted`` take caller-held scratch of
  ``q2k_matmul_id_scratch_bytes(params)`` bytes. ``params`` is a
  ``MatmulIdParams`` (or a dict with its fields).
* ``GGUFFile(path)`` — the GGUF tensor directory (``q2k_gguf_*``): names,
  ``tensor_info(name)`` and ``tensor_bytes(name)`` (host side, no GPU work).

The library is built in-tree by ``ggml_q2_dequant_amd.build``; importing this
package never builds or falls back to anything, and a call fails loudly when
``libq2k.so`` is missing.
"""
from __future__ import annotations

import ctypes
import os

QK_K = 256
BLOCK_BYTES = 84

Q2K_OK = 0
Q2K_ERR_INVALID_ARGUMENT = 1
Q2K_ERR_ID_OUT_OF_RANGE = 2
Q2K_ERR_DEVICE = 3

GGML_TYPE_Q2_K = 10
GGUF_MAX_DIMS = 4

PATH_AUTO = 0
PATH_GEMV = 1
PATH_MFMA = 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq2k.so")

# Every symbol include/q2k.h declares.
EXPORTS = (
    "q2k_dequantize",
    "q2k_matmul",
    "q2k_matmul_path",
    "q2k_matmul_scratch_bytes",
    "q2k_matmul_pooled",
    "q2k_matmul_noalloc",
    "q2k_matmul_batched",
    "q2k_embedding_gather",
    "q2k_embedding_gather_async",
    "q2k_argmax_candidates",
    "q2k_argmax_candidates_scratch_bytes",
    "q2k_argmax_candidates_pooled",
    "q2k_matmul_id",
    "q2k_matmul_id_path",
    "q2k_matmul_id_scratch_bytes",
    "q2k_matmul_id_pooled",
    "q2k_matmul_id_pooled_pair",
    "q2k_matmul_id_pooled_slotted",
    "q2k_gguf_open",
    "q2k_gguf_close",
    "q2k_gguf_tensor_count",
    "q2k_gguf_tensor_name",
    "q2k_gguf_tensor_info",
    "q2k_gguf_tensor_data",
    "q2k_status_string",
    "q2k_last_error_message",
)


class Q2KError(RuntimeError):
    """A libq2k call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_status_name(status), message))
        self.status = status


class Q2KInvalidArgument(Q2KError, ValueError):
    pass


class Q2KIdOutOfRange(Q2KError, IndexError):
    pass


class Q2KDeviceError(Q2KError):
    pass


class GGUFInfo(ctypes.Structure):
    """q2k_gguf_info: one tensor record of a GGUF file."""
    _fields_ = [("ggml_type", ctypes.c_uint32), ("n_dims", ctypes.c_uint32),
                ("dims", ctypes.c_uint64 * GGUF_MAX_DIMS), ("file_offset", ctypes.c_uint64),
                ("byte_len", ctypes.c_uint64)]


class MatmulIdParams(ctypes.Structure):
    """q2k_matmul_id_params: the expert-routed product's sizes."""
    _fields_ = [("n_tokens", ctypes.c_uint32), ("top_k", ctypes.c_uint32), ("n", ctypes.c_uint32),
                ("k", ctypes.c_uint32), ("n_experts", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("expert_stride", ctypes.c_uint64)]


def _params(p) -> MatmulIdParams:
    if isinstance(p, MatmulIdParams):
        return p
    return MatmulIdParams(**p)


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libq2k.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libq2k.so is not built (expected %s); run "
                           "`python -m ggml_q2_dequant_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, U32, SZ = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_size_t
    lib.q2k_dequantize.argtypes = [P, SZ, P, SZ, P]
    lib.q2k_matmul.argtypes = [P, P, P, U32, U32, U32, P]
    lib.q2k_matmul_path.argtypes = [P, P, P, U32, U32, U32, ctypes.c_int, P]
    lib.q2k_matmul_batched.argtypes = [P, P, P, U32, U32, U32, U32, P]
    lib.q2k_embedding_gather.argtypes = [P, P, P, U32, U32, U32, P]
    lib.q2k_embedding_gather_async.argtypes = [P, P, P, U32, U32, U32, P, P]
    for name in ("q2k_dequantize", "q2k_matmul", "q2k_matmul_path", "q2k_matmul_batched", "q2k_embedding_gather",
                 "q2k_embedding_gather_async"):
        getattr(lib, name).restype = ctypes.c_int
    lib.q2k_argmax_candidates.argtypes = [P, U32, U32, U32, P, P, P, P, P, P]
    lib.q2k_argmax_candidates.restype = ctypes.c_int
    U64, PU64 = ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)
    lib.q2k_matmul_scratch_bytes.argtypes = [U32, U32, U32, ctypes.c_int, PU64]
    lib.q2k_matmul_pooled.argtypes = [P, P, P, U32, U32, U32, ctypes.c_int, P, U64, P]
    lib.q2k_matmul_noalloc.argtypes = [P, P, P, U32, U32, U32, P]
    lib.q2k_argmax_candidates_scratch_bytes.argtypes = [U32, U32, PU64]
    lib.q2k_argmax_candidates_pooled.argtypes = [P, U32, U32, U32, P, P, P, P, P, P, U64, P]
    for name in ("q2k_matmul_scratch_bytes", "q2k_matmul_pooled", "q2k_matmul_noalloc",
                 "q2k_argmax_candidates_scratch_bytes",
                 "q2k_argmax_candidates_pooled"):
        getattr(lib, name).restype = ctypes.c_int
    PP = ctypes.POINTER(MatmulIdParams)
    lib.q2k_matmul_id.argtypes = [P, P, P, P, PP, P, P]
    lib.q2k_matmul_id_path.argtypes = [P, P, P, P, PP, P, ctypes.c_int, P]
    lib.q2k_matmul_id_scratch_bytes.argtypes = [PP]
    lib.q2k_matmul_id_scratch_bytes.restype = ctypes.c_uint64
    lib.q2k_matmul_id_pooled.argtypes = [P, P, P, P, PP, P, ctypes.c_uint64, P, P]
    lib.q2k_matmul_id_pooled_pair.argtypes = [P, P, P, P, P, P, PP, P, ctypes.c_uint64, P, P]
    lib.q2k_matmul_id_pooled_slotted.argtypes = [P, P, P, P, PP, P, ctypes.c_uint64, P, P]
    for name in ("q2k_matmul_id", "q2k_matmul_id_path", "q2k_matmul_id_pooled", "q2k_matmul_id_pooled_pair",
                 "q2k_matmul_id_pooled_slotted"):
        getattr(lib, name).restype = ctypes.c_int
    lib.q2k_gguf_open.argtypes = [ctypes.c_char_p, ctypes.POINTER(P)]
    lib.q2k_gguf_open.restype = ctypes.c_int
    lib.q2k_gguf_close.argtypes = [P]
    lib.q2k_gguf_close.restype = None
    lib.q2k_gguf_tensor_count.argtypes = [P]
    lib.q2k_gguf_tensor_count.restype = ctypes.c_uint64
    lib.q2k_gguf_tensor_name.argtypes = [P, ctypes.c_uint64]
    lib.q2k_gguf_tensor_name.restype = ctypes.c_char_p
    lib.q2k_gguf_tensor_info.argtypes = [P, ctypes.c_char_p, ctypes.POINTER(GGUFInfo)]
    lib.q2k_gguf_tensor_info.restype = ctypes.c_int
    lib.q2k_gguf_tensor_data.argtypes = [P, ctypes.c_char_p, ctypes.POINTER(P), ctypes.POINTER(ctypes.c_uint64)]
    lib.q2k_gguf_tensor_data.restype = ctypes.c_int
    lib.q2k_status_string.argtypes = [ctypes.c_int]
    lib.q2k_status_string.restype = ctypes.c_char_p
    lib.q2k_last_error_message.argtypes = []
    lib.q2k_last_error_message.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    try:
        return load_library().q2k_status_string(status).decode()
    except Exception:  # the name is only for messages
        return "status %d" % status


def _check(status: int) -> None:
    if status == Q2K_OK:
        return
    msg = load_library().q2k_last_error_message().decode(errors="replace")
    cls = {Q2K_ERR_INVALID_ARGUMENT: Q2KInvalidArgument, Q2K_ERR_ID_OUT_OF_RANGE: Q2KIdOutOfRange,
           Q2K_ERR_DEVICE: Q2KDeviceError}.get(status, Q2KError)
    raise cls(status, msg)


def _ptr(t) -> int | None:
    """Device pointer of a torch tensor (or a raw integer address)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def q2k_dequantize(blocks, out, stream=None, blocks_bytes: int | None = None, out_elems: int | None = None) -> None:
    """Decode ``blocks`` (uint8 device tensor of whole 84-byte blocks) into ``out`` (f32)."""
    nb = _nbytes(blocks) if blocks_bytes is None else int(blocks_bytes)
    ne = out.numel() if out_elems is None else int(out_elems)
    _check(load_library().q2k_dequantize(_ptr(blocks), nb, _ptr(out), ne, _stream(stream)))


def q2k_matmul(x, w, y, M: int, N: int, K: int, stream=None) -> None:
    """y[M, N] = x[M, K] * W[N, K]^T; x, y f32 device tensors, w uint8 Q2_K bytes."""
    _check(load_library().q2k_matmul(_ptr(x), _ptr(w), _ptr(y), M, N, K, _stream(stream)))


def q2k_matmul_path(x, w, y, M: int, N: int, K: int, path: int, stream=None) -> None:
    """q2k_matmul with a forced kernel: PATH_AUTO, PATH_GEMV (M <= 8) or PATH_MFMA."""
    _check(load_library().q2k_matmul_path(_ptr(x), _ptr(w), _ptr(y), M, N, K, int(path), _stream(stream)))


def q2k_matmul_scratch_bytes(M: int, N: int, K: int, path: int = PATH_AUTO) -> int:
    """Device scratch bytes q2k_matmul_pooled needs (0 for the GEMV path)."""
    n = ctypes.c_uint64()
    _check(load_library().q2k_matmul_scratch_bytes(M, N, K, int(path), ctypes.byref(n)))
    return int(n.value)


def q2k_matmul_pooled(x, w, y, M: int, N: int, K: int, scratch, path: int = PATH_AUTO, stream=None,
                      scratch_bytes: int | None = None) -> None:
    """q2k_matmul_path with caller-held scratch (a device tensor, or None when the path needs none)."""
    nb = (0 if scratch is None else _nbytes(scratch)) if scratch_bytes is None else int(scratch_bytes)
    _check(load_library().q2k_matmul_pooled(_ptr(x), _ptr(w), _ptr(y), M, N, K, int(path), _ptr(scratch), nb,
                                            _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20


def q2k_matmul_noalloc(x, w, y, M: int, N: int, K: int, stream=None) -> None:
    """q2k_matmul that allocates nothing (M > 8 needs 2*M*K <= 16 MiB); calls on one GPU must not overlap."""
    _check(load_library().q2k_matmul_noalloc(_ptr(x), _ptr(w), _ptr(y), M, N, K, _stream(stream)))


def q2k_matmul_batched(x, w, y, batches: int, M: int, N: int, K: int, stream=None) -> None:
    """y[b] = x[b] * W[b]^T for each of ``batches`` stacked problems (1 <= M <= 8)."""
    _check(load_library().q2k_matmul_batched(_ptr(x), _ptr(w), _ptr(y), batches, M, N, K, _stream(stream)))


def q2k_embedding_gather(table, ids, out, vocab: int, embed_dim: int, n_tokens: int, stream=None) -> None:
    """out[t, :] = decoded row ids[t] of ``table``; raises Q2KIdOutOfRange for any id >= vocab."""
    _check(load_library().q2k_embedding_gather(_ptr(table), _ptr(ids), _ptr(out), vocab, embed_dim, n_tokens,
                                               _stream(stream)))


def q2k_embedding_gather_async(table, ids, out, vocab: int, embed_dim: int, n_tokens: int, status,
                               stream=None) -> None:
    """q2k_embedding_gather without the wait: an id >= vocab sets ``status`` (a device int32 tensor) to 1."""
    _check(load_library().q2k_embedding_gather_async(_ptr(table), _ptr(ids), _ptr(out), vocab, embed_dim, n_tokens,
                                                     _ptr(status), _stream(stream)))


def q2k_argmax_candidates(logits, n_slots: int, vocab: int, cap: int, top1_idx, top1_val, cand_count, overflow,
                          cand_ids, stream=None) -> None:
    """Per slot: first-max index/value, candidate count (may exceed cap), overflow flag, candidate ids."""
    _check(load_library().q2k_argmax_candidates(_ptr(logits), n_slots, vocab, cap, _ptr(top1_idx), _ptr(top1_val),
                                                _ptr(cand_count), _ptr(overflow), _ptr(cand_ids), _stream(stream)))


def q2k_argmax_candidates_scratch_bytes(n_slots: int, vocab: int) -> int:
    """Device scratch bytes q2k_argmax_candidates_pooled needs."""
    n = ctypes.c_uint64()
    _check(load_library().q2k_argmax_candidates_scratch_bytes(n_slots, vocab, ctypes.byref(n)))
    return int(n.value)


def q2k_argmax_candidates_pooled(logits, n_slots: int, vocab: int, cap: int, top1_idx, top1_val, cand_count,
                                 overflow, cand_ids, scratch, stream=None, scratch_bytes: int | None = None) -> None:
    """q2k_argmax_candidates with caller-held scratch (a device tensor)."""
    nb = _nbytes(scratch) if scratch_bytes is None else int(scratch_bytes)
    _check(load_library().q2k_argmax_candidates_pooled(_ptr(logits), n_slots, vocab, cap, _ptr(top1_idx),
                                                       _ptr(top1_val), _ptr(cand_count), _ptr(overflow),
                                                       _ptr(cand_ids), _ptr(scratch), nb, _stream(stream)))


def q2k_matmul_id(x, w, ids, y, params, status=None, stream=None) -> None:
    """Expert-routed product; the schedule follows the page's rule (matrix cores for > 32 tokens, top_k 1/6/8)."""
    p = _params(params)
    _check(load_library().q2k_matmul_id(_ptr(x), _ptr(w), _ptr(ids), _ptr(y), ctypes.byref(p), _ptr(status),
                                        _stream(stream)))


def q2k_matmul_id_path(x, w, ids, y, params, path: int, status=None, stream=None) -> None:
    """q2k_matmul_id with a forced schedule: PATH_AUTO, PATH_GEMV (fp32 per route) or PATH_MFMA."""
    p = _params(params)
    _check(load_library().q2k_matmul_id_path(_ptr(x), _ptr(w), _ptr(ids), _ptr(y), ctypes.byref(p), _ptr(status),
                                             int(path), _stream(stream)))


def q2k_matmul_id_scratch_bytes(params) -> int:
    """Scratch bytes the pooled calls need (0 for invalid parameters)."""
    p = _params(params)
    return int(load_library().q2k_matmul_id_scratch_bytes(ctypes.byref(p)))


def q2k_matmul_id_pooled(x, w, ids, y, params, scratch, status=None, stream=None, scratch_bytes: int | None = None):
    """Matrix-core expert-routed product with caller-held scratch (a device tensor)."""
    p = _params(params)
    nb = _nbytes(scratch) if scratch_bytes is None else int(scratch_bytes)
    _check(load_library().q2k_matmul_id_pooled(_ptr(x), _ptr(w), _ptr(ids), _ptr(y), ctypes.byref(p),
                                               _ptr(scratch), nb, _ptr(status), _stream(stream)))


def q2k_matmul_id_pooled_pair(x, w0, w1, ids, y0, y1, params, scratch, status=None, stream=None,
                              scratch_bytes: int | None = None):
    """Two weight sets (gate/up) with one routing: y0 from w0, y1 from w1."""
    p = _params(params)
    nb = _nbytes(scratch) if scratch_bytes is None else int(scratch_bytes)
    _check(load_library().q2k_matmul_id_pooled_pair(_ptr(x), _ptr(w0), _ptr(w1), _ptr(ids), _ptr(y0), _ptr(y1),
                                                    ctypes.byref(p), _ptr(scratch), nb, _ptr(status),
                                                    _stream(stream)))


def q2k_matmul_id_pooled_slotted(x, w, ids, y, params, scratch, status=None, stream=None,
                                 scratch_bytes: int | None = None):
    """One activation row per route: x [n_tokens, top_k, k], y [n_tokens, top_k, n]."""
    p = _params(params)
    nb = _nbytes(scratch) if scratch_bytes is None else int(scratch_bytes)
    _check(load_library().q2k_matmul_id_pooled_slotted(_ptr(x), _ptr(w), _ptr(ids), _ptr(y), ctypes.byref(p),
                                                       _ptr(scratch), nb, _ptr(status), _stream(stream)))


class GGUFFile:
    """A GGUF file's tensor directory, read by libq2k (q2k_gguf_*). Use as a context manager or call close()."""

    def __init__(self, path: str):
        lib = load_library()
        h = ctypes.c_void_p()
        _check(lib.q2k_gguf_open(os.fsencode(path), ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        if self._h:
            load_library().q2k_gguf_close(self._h)
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def tensor_names(self) -> list:
        lib = load_library()
        return [lib.q2k_gguf_tensor_name(self._h, i).decode(errors="replace")
                for i in range(lib.q2k_gguf_tensor_count(self._h))]

    def tensor_info(self, name: str) -> dict:
        info = GGUFInfo()
        _check(load_library().q2k_gguf_tensor_info(self._h, name.encode(), ctypes.byref(info)))
        return {"ggml_type": info.ggml_type, "n_dims": info.n_dims, "dims": list(info.dims)[:info.n_dims],
                "file_offset": info.file_offset, "byte_len": info.byte_len}

    def tensor_bytes(self, name: str):
        """A numpy uint8 copy of the tensor's data."""
        import numpy as np
        ptr, n = ctypes.c_void_p(), ctypes.c_uint64()
        _check(load_library().q2k_gguf_tensor_data(self._h, name.encode(), ctypes.byref(ptr), ctypes.byref(n)))
        return np.frombuffer(ctypes.string_at(ptr.value, n.value), dtype=np.uint8).copy()
