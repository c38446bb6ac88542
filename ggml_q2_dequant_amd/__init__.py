"""ggml_q2_dequant_amd — the Q2_K weight path on MI355X (gfx950).

A thin ctypes binding over ``libq2k.so`` (C ABI in ``include/q2k.h``). Every
step of the path runs in the library's HIP kernels; this module only turns
torch device tensors into pointers and sizes and raises on a non-zero status.
PyTorch supplies device memory and the current stream, nothing else.

Functions carry the C names:

* ``q2k_dequantize(blocks, out)`` — decode whole 84-byte blocks to f32.
* ``q2k_matmul(x, w, y, M, N, K)`` — y[M, N] = x[M, K] * W[N, K]^T, W in Q2_K.
* ``q2k_matmul_path(x, w, y, M, N, K, path)`` — same with a forced kernel.
* ``q2k_matmul_batched(x, w, y, batches, M, N, K)`` — independent products, one
  per matrix of a batch-major stack (1 <= M <= 8).
* ``q2k_embedding_gather(table, ids, out, vocab, embed_dim, n_tokens)`` — rows
  of a Q2_K table; raises ``Q2KIdOutOfRange`` for an id >= vocab.

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

PATH_AUTO = 0
PATH_GEMV = 1
PATH_MFMA = 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq2k.so")

# Every symbol include/q2k.h declares.
EXPORTS = (
    "q2k_dequantize",
    "q2k_matmul",
    "q2k_matmul_path",
    "q2k_matmul_batched",
    "q2k_embedding_gather",
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
    for name in ("q2k_dequantize", "q2k_matmul", "q2k_matmul_path", "q2k_matmul_batched", "q2k_embedding_gather"):
        getattr(lib, name).restype = ctypes.c_int
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
    msg = load_library().q2k_last_error_message().decode()
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


def q2k_matmul_batched(x, w, y, batches: int, M: int, N: int, K: int, stream=None) -> None:
    """y[b] = x[b] * W[b]^T for each of ``batches`` stacked problems (1 <= M <= 8)."""
    _check(load_library().q2k_matmul_batched(_ptr(x), _ptr(w), _ptr(y), batches, M, N, K, _stream(stream)))


def q2k_embedding_gather(table, ids, out, vocab: int, embed_dim: int, n_tokens: int, stream=None) -> None:
    """out[t, :] = decoded row ids[t] of ``table``; raises Q2KIdOutOfRange for any id >= vocab."""
    _check(load_library().q2k_embedding_gather(_ptr(table), _ptr(ids), _ptr(out), vocab, embed_dim, n_tokens,
                                               _stream(stream)))
