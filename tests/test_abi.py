"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device.

The rejection rules restate the docs.rs source page of mlx-native 0.10.8,
tests/deepseek_q2_k.rs (malformed-buffer test: an 83-byte block and a
255-value output are errors) plus the header's shape, alignment and overlap
rules. Every call below fails validation, so no HIP work is ever enqueued.
"""
import ctypes
import os
import re

import pytest

import ggml_q2_dequant_amd as q2k

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q2k.h")

# Fake, well-aligned, non-overlapping "device" addresses: validation never
# dereferences them.
A = 1 << 32
B = 2 << 32
C = 3 << 32


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q2k_[a-z_]+)\s*\(", text)))


# Q2K_ABI_TEST_LIB names another build of the same C ABI layer to test instead
# of libq2k.so (the sanitizer build of tests/test_sanitizers.py).
LIB_UNDER_TEST = os.environ.get("Q2K_ABI_TEST_LIB") or q2k.LIB_PATH


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_UNDER_TEST):
        pytest.skip("%s not built" % LIB_UNDER_TEST)
    return q2k.load_library(LIB_UNDER_TEST)


def test_header_declares_the_expected_entry_points():
    assert _header_functions() == sorted(q2k.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _header_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    names = [lib.q2k_status_string(i).decode() for i in range(4)]
    assert names == ["Q2K_OK", "Q2K_ERR_INVALID_ARGUMENT", "Q2K_ERR_ID_OUT_OF_RANGE", "Q2K_ERR_DEVICE"]
    assert lib.q2k_status_string(99).decode() == "Q2K_UNKNOWN_STATUS"


def _err(lib, rc, fragment):
    assert rc == q2k.Q2K_ERR_INVALID_ARGUMENT
    assert fragment in lib.q2k_last_error_message().decode()


@pytest.mark.parametrize("nbytes,nout,frag", [
    (83, 256, "multiple of 84"),          # the page's short block
    (84, 255, "need 256 outputs"),        # the page's short output
    (0, 0, "multiple of 84"),             # empty input
    (168, 256, "need 512 outputs"),
])
def test_dequantize_rejects_malformed_lengths(lib, nbytes, nout, frag):
    _err(lib, lib.q2k_dequantize(A, nbytes, B, nout, None), frag)


def test_dequantize_rejects_null_misaligned_and_overlap(lib):
    _err(lib, lib.q2k_dequantize(None, 84, B, 256, None), "null")
    _err(lib, lib.q2k_dequantize(A + 2, 84, B, 256, None), "aligned")
    _err(lib, lib.q2k_dequantize(A, 84, B + 4, 256, None), "aligned")
    _err(lib, lib.q2k_dequantize(A, 84, A + 16, 256, None), "overlaps")


@pytest.mark.parametrize("M,N,K,frag", [
    (0, 8, 256, ">= 1"), (1, 0, 256, ">= 1"), (1, 8, 0, ">= 1"),
    (1, 8, 100, "multiple of 256"), (4, 8, 255, "multiple of 256"), (1, 1, (1 << 21) + 256, "exceeds the limit"),
])
def test_matmul_rejects_bad_shapes(lib, M, N, K, frag):
    _err(lib, lib.q2k_matmul(A, B, C, M, N, K, None), frag)


def test_matmul_rejects_null_misaligned_overlap_and_bad_path(lib):
    _err(lib, lib.q2k_matmul(None, B, C, 1, 8, 256, None), "null")
    _err(lib, lib.q2k_matmul(A + 4, B, C, 1, 8, 256, None), "aligned")
    _err(lib, lib.q2k_matmul(A, B + 2, C, 1, 8, 256, None), "aligned")
    _err(lib, lib.q2k_matmul(A, B, A + 16, 1, 8, 256, None), "overlaps")
    _err(lib, lib.q2k_matmul(A, B, B + 16, 1, 8, 256, None), "overlaps")
    _err(lib, lib.q2k_matmul_path(A, B, C, 9, 8, 256, q2k.PATH_GEMV, None), "M <= 8")
    _err(lib, lib.q2k_matmul_path(A, B, C, 1, 8, 256, 7, None), "unknown path")


def test_matmul_rejects_size_overflow(lib):
    _err(lib, lib.q2k_matmul(A, B, C, 0xFFFFFFFF, 0xFFFFFFFF, 1 << 21, None), "overflow")


@pytest.mark.parametrize("bt,M,N,K,frag", [
    (0, 1, 8, 256, ">= 1"), (2, 0, 8, 256, ">= 1"), (2, 1, 0, 256, ">= 1"), (2, 1, 8, 0, ">= 1"),
    (2, 9, 8, 256, "1 <= M <= 8"), (2, 1, 8, 300, "multiple of 256"), (2, 1, 8, (1 << 21) + 256, "exceeds"),
    (0xFFFFFFFF, 8, 0xFFFFFFFF, 1 << 21, "overflow"),
])
def test_matmul_batched_rejects_bad_shapes(lib, bt, M, N, K, frag):
    _err(lib, lib.q2k_matmul_batched(A, B, C, bt, M, N, K, None), frag)


def test_matmul_batched_rejects_null_misaligned_and_overlap(lib):
    _err(lib, lib.q2k_matmul_batched(None, B, C, 3, 1, 8, 256, None), "null")
    _err(lib, lib.q2k_matmul_batched(A + 4, B, C, 3, 1, 8, 256, None), "aligned")
    _err(lib, lib.q2k_matmul_batched(A, B + 1, C, 3, 1, 8, 256, None), "aligned")
    # y of 3 batches x 8 floats ends 96 bytes after C: it overlaps an x that starts inside it
    _err(lib, lib.q2k_matmul_batched(C + 64, B, C, 3, 1, 8, 256, None), "overlaps")
    _err(lib, lib.q2k_matmul_batched(A, C + 80, C, 3, 1, 8, 256, None), "overlaps")


@pytest.mark.parametrize("vocab,dim,nt,frag", [
    (0, 256, 2, ">= 1"), (3, 0, 2, ">= 1"), (3, 256, 0, ">= 1"), (3, 100, 2, "multiple of 256"),
])
def test_gather_rejects_bad_shapes(lib, vocab, dim, nt, frag):
    _err(lib, lib.q2k_embedding_gather(A, B, C, vocab, dim, nt, None), frag)


def test_gather_rejects_null_misaligned_and_overlap(lib):
    _err(lib, lib.q2k_embedding_gather(None, B, C, 3, 256, 2, None), "null")
    _err(lib, lib.q2k_embedding_gather(A + 1, B, C, 3, 256, 2, None), "aligned")
    _err(lib, lib.q2k_embedding_gather(A, B + 2, C, 3, 256, 2, None), "aligned")
    _err(lib, lib.q2k_embedding_gather(A, B, C + 8, 3, 256, 2, None), "aligned")
    _err(lib, lib.q2k_embedding_gather(A, B, A, 3, 256, 2, None), "overlaps")
    _err(lib, lib.q2k_embedding_gather(A, C + 4, C, 3, 256, 2, None), "overlaps")


D = 4 << 32


def test_gather_async_rejects_like_the_gather_and_checks_status(lib):
    f = lib.q2k_embedding_gather_async
    _err(lib, f(None, B, C, 3, 256, 2, D, None), "null")
    _err(lib, f(A, B, C, 3, 255, 2, D, None), "multiple of 256")
    _err(lib, f(A, B, C + 8, 3, 256, 2, D, None), "aligned")
    _err(lib, f(A, B, A, 3, 256, 2, D, None), "overlaps")
    _err(lib, f(A, B, C, 3, 256, 2, None, None), "status is required")
    _err(lib, f(A, B, C, 3, 256, 2, D + 2, None), "aligned")
    _err(lib, f(A, B, C, 3, 256, 2, C + 1024, None), "status overlaps")    # inside out (2 rows x 1 KiB)
    _err(lib, f(A, B, C, 3, 256, 2, B + 4, None), "status overlaps")       # the second id
    _err(lib, f(A, B, C, 3, 256, 2, A + 84, None), "status overlaps")      # inside the table


D, E, F, G = 4 << 32, 5 << 32, 6 << 32, 7 << 32


@pytest.mark.parametrize("ns,vocab,cap,frag", [
    (0, 8, 4, "> 0"), (2, 0, 4, "> 0"), (2, 8, 0, "> 0"), (2, (1 << 29) + 1, 4, "exceeds the limit"),
    (0xFFFFFFFF, 1 << 29, 0xFFFFFFFF, "overflow"),
])
def test_argmax_candidates_rejects_bad_sizes(lib, ns, vocab, cap, frag):
    _err(lib, lib.q2k_argmax_candidates(A, ns, vocab, cap, B, C, D, E, F, None), frag)


def test_argmax_candidates_rejects_null_misaligned_and_overlap(lib):
    _err(lib, lib.q2k_argmax_candidates(A, 2, 8, 4, B, C, D, E, None, None), "null")
    _err(lib, lib.q2k_argmax_candidates(A + 2, 2, 8, 4, B, C, D, E, F, None), "aligned")
    _err(lib, lib.q2k_argmax_candidates(A, 2, 8, 4, B, C + 1, D, E, F, None), "aligned")
    _err(lib, lib.q2k_argmax_candidates(A, 2, 8, 4, A + 60, C, D, E, F, None), "overlaps the logits")
    _err(lib, lib.q2k_argmax_candidates(A, 2, 8, 4, B, B + 4, D, E, F, None), "overlap each other")
    _err(lib, lib.q2k_argmax_candidates(A, 2, 8, 4, B, C, D, E, E + 4, None), "overlap each other")


# ---------------------------------------------------------------- expert-routed product

def _idp(**kw):
    d = dict(n_tokens=2, top_k=2, n=8, k=256, n_experts=3, reserved=0, expert_stride=8 * 84)
    d.update(kw)
    return q2k.MatmulIdParams(**d)


def _id(lib, p, x=A, w=B, ids=C, y=D, status=None, path=0):
    return lib.q2k_matmul_id_path(x, w, ids, y, ctypes.byref(p), status, path, None)


@pytest.mark.parametrize("kw,frag", [
    (dict(n_tokens=0), ">= 1"), (dict(top_k=0), ">= 1"), (dict(n=0), ">= 1"), (dict(n_experts=0), ">= 1"),
    (dict(k=0), ">= 1"), (dict(k=300), "multiple of 256"), (dict(k=(1 << 21) + 256), "exceeds the limit"),
    (dict(n_experts=513), "exceeds the limit"), (dict(n_tokens=1 << 13, top_k=(1 << 11) + 1), "exceeds the limit"),
    (dict(expert_stride=8 * 84 - 4), "expert_stride"), (dict(expert_stride=8 * 84 + 2), "expert_stride"),
    (dict(reserved=1), "reserved"),
])
def test_matmul_id_rejects_bad_params(lib, kw, frag):
    _err(lib, _id(lib, _idp(**kw)), frag)
    assert lib.q2k_matmul_id_scratch_bytes(ctypes.byref(_idp(**kw))) == 0


def test_matmul_id_rejects_null_misaligned_overlap_and_bad_path(lib):
    p = _idp()
    _err(lib, _id(lib, p, x=None), "null")
    _err(lib, lib.q2k_matmul_id_path(A, B, C, D, None, None, 0, None), "null")
    _err(lib, _id(lib, p, x=A + 4), "aligned")
    _err(lib, _id(lib, p, w=B + 2), "aligned")
    _err(lib, _id(lib, p, ids=C + 1), "aligned")
    _err(lib, _id(lib, p, y=A + 2 * 256 * 4 - 16), "overlaps an input")     # end of x
    _err(lib, _id(lib, p, y=B + 3 * 8 * 84 - 16), "overlaps an input")      # last expert of w
    _err(lib, _id(lib, p, y=C), "overlaps an input")
    _err(lib, _id(lib, p, status=E + 2), "status")
    _err(lib, _id(lib, p, status=D + 4 * 8 * 4 - 4), "status overlaps")
    _err(lib, _id(lib, p, path=7), "unknown path")


def test_matmul_id_scratch_bytes_cover_the_bf16_rows(lib):
    for tokens, top_k, k, experts in ((2, 2, 256, 3), (33, 6, 256, 8), (512, 6, 4096, 8), (1, 1, 256, 1)):
        p = _idp(n_tokens=tokens, top_k=top_k, k=k, n_experts=experts, expert_stride=8 * k // 256 * 84)
        b = lib.q2k_matmul_id_scratch_bytes(ctypes.byref(p))
        assert b >= 2 * tokens * top_k * k + 4 * tokens * top_k
    assert lib.q2k_matmul_id_scratch_bytes(None) == 0


def test_matmul_id_pooled_rejects_bad_scratch(lib):
    p = _idp()
    need = lib.q2k_matmul_id_scratch_bytes(ctypes.byref(p))
    pooled = lib.q2k_matmul_id_pooled
    _err(lib, pooled(A, B, C, D, ctypes.byref(p), None, need, None, None), "null scratch")
    _err(lib, pooled(A, B, C, D, ctypes.byref(p), F + 128, need, None, None), "256-byte aligned")
    _err(lib, pooled(A, B, C, D, ctypes.byref(p), F, need - 1, None, None), "needed")
    _err(lib, pooled(A, B, C, D, ctypes.byref(p), A - 256, need, None, None), "scratch overlaps")
    _err(lib, pooled(A, B, C, D, ctypes.byref(p), F, need, F + 64, None), "status overlaps")
    slotted = lib.q2k_matmul_id_pooled_slotted
    # Slotted: x holds one row per route (4 rows), so y right after 2 rows overlaps it.
    _err(lib, slotted(A, B, C, A + 2 * 256 * 4, ctypes.byref(p), F, need, None, None), "overlaps an input")


def test_matmul_id_pair_rejects_overlapping_outputs(lib):
    p = _idp()
    need = lib.q2k_matmul_id_scratch_bytes(ctypes.byref(p))
    pair = lib.q2k_matmul_id_pooled_pair
    _err(lib, pair(A, B, B, C, D, D + 64, ctypes.byref(p), F, need, None, None), "overlaps the other")
    _err(lib, pair(A, B, G, C, D, G, ctypes.byref(p), F, need, None, None), "overlaps an input")
    _err(lib, pair(A, B, G, C, G, E, ctypes.byref(p), F, need, None, None), "overlaps the other")
    _err(lib, pair(A, B, B, C, D, None, ctypes.byref(p), F, need, None, None), "null")


# ---------------------------------------------------------------- caller-held scratch

def _u64():
    return ctypes.c_uint64(0xDEAD)


def test_matmul_scratch_bytes_per_path(lib):
    n = _u64()
    assert lib.q2k_matmul_scratch_bytes(8, 10, 512, 0, ctypes.byref(n)) == 0 and n.value == 0      # GEMV
    assert lib.q2k_matmul_scratch_bytes(9, 10, 512, 0, ctypes.byref(n)) == 0 and n.value == 2 * 9 * 512
    assert lib.q2k_matmul_scratch_bytes(1, 10, 512, 2, ctypes.byref(n)) == 0 and n.value == 2 * 512
    assert lib.q2k_matmul_scratch_bytes(8, 10, 512, 1, ctypes.byref(n)) == 0 and n.value == 0
    n = _u64()
    _err(lib, lib.q2k_matmul_scratch_bytes(9, 10, 512, 1, ctypes.byref(n)), "M <= 8")
    _err(lib, lib.q2k_matmul_scratch_bytes(0, 10, 512, 0, ctypes.byref(n)), ">= 1")
    _err(lib, lib.q2k_matmul_scratch_bytes(9, 10, 500, 0, ctypes.byref(n)), "multiple of 256")
    _err(lib, lib.q2k_matmul_scratch_bytes(9, 10, 512, 5, ctypes.byref(n)), "unknown path")
    _err(lib, lib.q2k_matmul_scratch_bytes(9, 10, 512, 0, None), "null")
    assert n.value == 0xDEAD  # untouched on failure


def test_matmul_pooled_rejects_bad_scratch(lib):
    M, N, K = 16, 8, 512
    need = 2 * M * K
    pooled = lib.q2k_matmul_pooled
    _err(lib, pooled(A, B, C, M, N, K, 0, None, need, None), "null scratch")
    _err(lib, pooled(A, B, C, M, N, K, 0, F + 16, need, None), "256-byte aligned")
    _err(lib, pooled(A, B, C, M, N, K, 0, F, need - 1, None), "needed")
    _err(lib, pooled(A, B, C, M, N, K, 0, A + 256, need, None), "scratch overlaps")      # inside x
    _err(lib, pooled(A, B, C, M, N, K, 0, C - 256, need, None), "scratch overlaps")      # runs into y
    _err(lib, pooled(A, B, C, M, N, K, 1, F, need, None), "M <= 8")
    _err(lib, pooled(A, B, C + 4, M, N, K, 0, F, need, None), "aligned")                 # matmul rules first
    _err(lib, pooled(A, B, C, 0, N, K, 0, F, need, None), ">= 1")


def test_argmax_pooled_rejects_bad_scratch(lib):
    n = _u64()
    assert lib.q2k_argmax_candidates_scratch_bytes(2, 8, ctypes.byref(n)) == 0 and n.value > 0
    need = n.value
    _err(lib, lib.q2k_argmax_candidates_scratch_bytes(0, 8, ctypes.byref(n)), "n_slots >= 1")
    _err(lib, lib.q2k_argmax_candidates_scratch_bytes(2, (1 << 29) + 1, ctypes.byref(n)), "vocab")
    pooled = lib.q2k_argmax_candidates_pooled
    _err(lib, pooled(A, 2, 8, 4, B, C, D, E, F, None, need, None), "null scratch")
    _err(lib, pooled(A, 2, 8, 4, B, C, D, E, F, G + 4, need, None), "256-byte aligned")
    _err(lib, pooled(A, 2, 8, 4, B, C, D, E, F, G, need - 1, None), "needed")
    _err(lib, pooled(A, 2, 8, 4, B, C, D, E, F, F, need, None), "scratch overlaps")
    _err(lib, pooled(A, 0, 8, 4, B, C, D, E, F, G, need, None), "> 0")


def test_argmax_scratch_covers_one_launch_of_slots(lib):
    # More than 65535 slots run in several launches that reuse the same scratch.
    a, b = ctypes.c_uint64(), ctypes.c_uint64()
    assert lib.q2k_argmax_candidates_scratch_bytes(65535, 262144, ctypes.byref(a)) == 0
    assert lib.q2k_argmax_candidates_scratch_bytes(200000, 262144, ctypes.byref(b)) == 0
    assert a.value == b.value > 0


def test_python_binding_raises_typed_errors(lib):
    with pytest.raises(q2k.Q2KInvalidArgument, match="multiple of 256"):
        q2k.q2k_matmul(A, B, C, 1, 8, 100, stream=0)
    with pytest.raises(ValueError):
        q2k.q2k_matmul(A, B, C, 0, 8, 256, stream=0)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        _load_fresh(str(tmp_path / "nope.so"))


def _load_fresh(path):
    saved = q2k._lib
    q2k._lib = None
    try:
        return q2k.load_library(path)
    finally:
        q2k._lib = saved
