"""Q2_K CPU oracle (test infrastructure only).

Python access to ``q2k_oracle.c``, the slow reference definition that the HIP
path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product library
never uses it and shares no code with it.

Every function restates an item of the docs.rs source page of mlx-native
0.10.8, tests/deepseek_q2_k.rs: the 84-byte super-block layout (constants and
fn block), the decode (fn reference_dequant), the dense product (fn run_dense,
fn cpu_dot), the batched mat-vec test and the embedding gather test; and, from
the docs.rs source page of mlx-native 0.9.5, src/mlx_native/ops/gpu_sample.rs,
the first-max argmax with threshold candidates; and the expert-routed product
(fn run_expert and the slotted down-projection test). The C file documents each one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

QK_K = 256
BLOCK_BYTES = 84

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q2k_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


class OracleError(ValueError):
    """The oracle rejected its arguments (bad length or shape, id out of range)."""


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, no FP contraction, no fast-math, OpenMP."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        # Q2K_ORACLE_LIB names another build of q2k_oracle.c to load instead
        # (the sanitizer build of tests/test_sanitizers.py).
        path = os.environ.get("Q2K_ORACLE_LIB")
        if not path:
            path = build(force=False)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        L = ctypes.c_long
        lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f32.restype = ctypes.c_float
        lib.oracle_dequant_block.argtypes = [P, P]
        lib.oracle_dequant_block.restype = None
        lib.oracle_dequant_element.argtypes = [P, ctypes.c_int]
        lib.oracle_dequant_element.restype = ctypes.c_float
        lib.oracle_dequantize.argtypes = [P, ctypes.c_size_t, P, ctypes.c_size_t]
        lib.oracle_dequantize.restype = ctypes.c_int
        lib.oracle_bf16_round.argtypes = [ctypes.c_float]
        lib.oracle_bf16_round.restype = ctypes.c_float
        lib.oracle_matmul.argtypes = [P, P, P, P, L, L, L, ctypes.c_int, ctypes.c_int]
        lib.oracle_matmul.restype = ctypes.c_int
        lib.oracle_matmul_f32seq.argtypes = [P, P, P, L, L, L]
        lib.oracle_matmul_f32seq.restype = ctypes.c_int
        lib.oracle_gather.argtypes = [P, P, P, L, L, L, ctypes.c_int]
        lib.oracle_gather.restype = ctypes.c_int
        lib.oracle_argmax_candidates.argtypes = [P, L, L, L, P, P, P, P, P]
        lib.oracle_argmax_candidates.restype = ctypes.c_int
        lib.oracle_matmul_id.argtypes = [P, P, P, P, P, L, L, L, L, L, L, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.POINTER(L)]
        lib.oracle_matmul_id.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _u8(a) -> np.ndarray:
    return np.ascontiguousarray(np.frombuffer(bytes(a), dtype=np.uint8) if isinstance(a, (bytes, bytearray)) else a, dtype=np.uint8)


def host_threads() -> int:
    """Host cores this process may run on (its CPU affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def f16_to_f32(bits) -> np.ndarray:
    """Decode f16 bit patterns (uint16) to f32 with the oracle's own decoder."""
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.empty(b.shape, dtype=np.float32)
    for i, v in enumerate(b.tolist()):
        out[i] = lib.oracle_f16_to_f32(v)
    return out


def dequant_block(block) -> np.ndarray:
    """Decode one 84-byte block to 256 f32, in the page's loop order."""
    blk = _u8(block)
    if blk.size != BLOCK_BYTES:
        raise OracleError("a block is %d bytes, got %d" % (BLOCK_BYTES, blk.size))
    out = np.empty(QK_K, dtype=np.float32)
    _load().oracle_dequant_block(_ptr(blk), _ptr(out))
    return out


def dequant_element(block, e: int) -> np.float32:
    """Decode element e of one block through the closed-form index map."""
    blk = _u8(block)
    if blk.size != BLOCK_BYTES or not 0 <= e < QK_K:
        raise OracleError("bad block or element index")
    return np.float32(_load().oracle_dequant_element(_ptr(blk), int(e)))


def dequantize(data, out_elems: int | None = None) -> np.ndarray:
    """Decode a byte buffer of whole blocks; reject ragged lengths.

    ``out_elems`` is the caller's output length (default: 256 per block); any
    mismatch is rejected, as the page's malformed-buffer test requires.
    """
    buf = _u8(data)
    nblk = buf.size // BLOCK_BYTES
    n_out = nblk * QK_K if out_elems is None else int(out_elems)
    out = np.empty(max(n_out, 0), dtype=np.float32)
    rc = _load().oracle_dequantize(_ptr(buf), buf.size, _ptr(out), n_out)
    if rc != 0:
        raise OracleError("rejected: %d bytes into %d outputs" % (buf.size, n_out))
    return out


def bf16_round(values) -> np.ndarray:
    """Round f32 values to bf16 (ties to even), returned as f32."""
    lib = _load()
    v = np.asarray(values, dtype=np.float32).ravel()
    return np.array([lib.oracle_bf16_round(float(f)) for f in v.tolist()], dtype=np.float32)


def matmul(x, w, M: int, N: int, K: int, bf16_operands: bool = False, nthreads: int = 1):
    """y[m, n] = sum_k x[m, k] * w[n, k] in f64; returns (y, a) with a = sum |x*w|.

    x: f32 [M, K] row-major; w: N*K/256 blocks of 84 bytes, rows contiguous.
    """
    xa = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    wa = _u8(w)
    if K % QK_K or xa.size != M * K or wa.size != N * (K // QK_K) * BLOCK_BYTES:
        raise OracleError("matmul shape mismatch")
    y = np.empty((M, N), dtype=np.float64)
    a = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_matmul(_ptr(xa), _ptr(wa), _ptr(y), _ptr(a), M, N, K,
                               1 if bf16_operands else 0, int(nthreads))
    if rc != 0:
        raise OracleError("matmul rejected shape")
    return y, a


def matmul_batched(x, w, batches: int, M: int, N: int, K: int, nthreads: int = 1):
    """The page's batched mat-vec (test q2_k_batched_mv_is_byte_identical_to_independent_dispatches):
    problem b multiplies x[b] (M x K) by the b-th weight matrix of a batch-major stack (N rows of K/256
    blocks each). Defined there as separate single-matrix products; returns (y, a) stacked [batches, M, N].
    """
    xa = np.ascontiguousarray(x, dtype=np.float32).reshape(batches, M, K)
    wa = _u8(w)
    per = N * (K // QK_K) * BLOCK_BYTES
    if K % QK_K or wa.size != batches * per:
        raise OracleError("batched matmul shape mismatch")
    ys, as_ = [], []
    for b in range(batches):
        y, a = matmul(xa[b], wa[b * per:(b + 1) * per], M, N, K, nthreads=nthreads)
        ys.append(y)
        as_.append(a)
    return np.stack(ys), np.stack(as_)


def matmul_id(x, w, ids, n_tokens: int, top_k: int, n: int, K: int, n_experts: int, expert_stride: int,
              slotted: bool = False, bf16_operands: bool = False, nthreads: int = 1):
    """The page's expert-routed product (fn run_expert; slotted: the down-projection test).

    Route r = token * top_k + slot uses expert ids[r] (u32 [n_tokens, top_k]) and activation row r // top_k
    of x [n_tokens, K], or row r of x [n_tokens, top_k, K] when ``slotted``. Expert e's n weight rows start
    e * expert_stride bytes into w. Returns (y, a, bad): y and a are f64 [n_tokens * top_k, n] (a = sum |x*w|),
    rows of routes whose id is >= n_experts are NaN, and bad counts those routes.
    """
    routes = n_tokens * top_k
    xa = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    wa = _u8(w)
    ia = np.ascontiguousarray(ids, dtype=np.uint32).reshape(-1)
    rows_x = routes if slotted else n_tokens
    row_bytes = (K // QK_K) * BLOCK_BYTES
    if (K % QK_K or xa.size != rows_x * K or ia.size != routes or expert_stride < n * row_bytes
            or wa.size < (n_experts - 1) * expert_stride + n * row_bytes):
        raise OracleError("matmul_id shape mismatch")
    y = np.empty((routes, n), dtype=np.float64)
    a = np.empty((routes, n), dtype=np.float64)
    bad = ctypes.c_long(0)
    rc = _load().oracle_matmul_id(_ptr(xa), _ptr(wa), _ptr(ia), _ptr(y), _ptr(a), n_tokens, top_k, n, K,
                                  n_experts, expert_stride, 1 if slotted else 0, 1 if bf16_operands else 0,
                                  int(nthreads), ctypes.byref(bad))
    if rc != 0:
        raise OracleError("matmul_id rejected shape")
    return y, a, bad.value


def matmul_f32seq(x, w, M: int, N: int, K: int) -> np.ndarray:
    """The page's cpu_dot: f32 products summed left to right in f32."""
    xa = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    wa = _u8(w)
    if K % QK_K or xa.size != M * K or wa.size != N * (K // QK_K) * BLOCK_BYTES:
        raise OracleError("matmul shape mismatch")
    y = np.empty((M, N), dtype=np.float32)
    if _load().oracle_matmul_f32seq(_ptr(xa), _ptr(wa), _ptr(y), M, N, K) != 0:
        raise OracleError("matmul rejected shape")
    return y


def gather(table, ids, vocab: int, embed_dim: int, n_tokens: int, nthreads: int = 1) -> np.ndarray:
    """out[t, :] = decoded table row ids[t]; raises OracleError for any id >= vocab."""
    tb = _u8(table)
    ia = np.ascontiguousarray(ids, dtype=np.uint32).reshape(-1)
    if ia.size != n_tokens or embed_dim % QK_K or tb.size != vocab * (embed_dim // QK_K) * BLOCK_BYTES:
        raise OracleError("gather shape mismatch")
    out = np.empty((n_tokens, embed_dim), dtype=np.float32)
    rc = _load().oracle_gather(_ptr(tb), _ptr(ia), _ptr(out), vocab, embed_dim, n_tokens, int(nthreads))
    if rc == -2:
        raise OracleError("token id out of range")
    if rc != 0:
        raise OracleError("gather rejected shape")
    return out


def argmax_candidates(logits, n_slots: int, vocab: int, cap: int):
    """gpu_sample.rs: per slot (top1_idx, top1_val, cand_count, overflow, cand_ids[:min(count, cap)])."""
    lg = np.ascontiguousarray(logits, dtype=np.float32).reshape(-1)
    if lg.size != n_slots * vocab:
        raise OracleError("logits shape mismatch")
    idx = np.empty(n_slots, np.uint32)
    val = np.empty(n_slots, np.float32)
    cnt = np.empty(n_slots, np.uint32)
    ovf = np.empty(n_slots, np.uint32)
    ids = np.full((n_slots, cap), 0xFFFFFFFF, np.uint32)
    if _load().oracle_argmax_candidates(_ptr(lg), n_slots, vocab, cap, _ptr(idx), _ptr(val), _ptr(cnt), _ptr(ovf),
                                        _ptr(ids)) != 0:
        raise OracleError("argmax_candidates rejected a zero size")
    return idx, val, cnt, ovf, [ids[s, :min(int(cnt[s]), cap)] for s in range(n_slots)]
