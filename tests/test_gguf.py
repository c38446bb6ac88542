"""GGUF tensor directory (host side of libq2k, no GPU needed except the last test).

The page is the docs.rs source page of mlx-native 0.10.8, tests/deepseek_q2_k.rs,
test q2_k_gguf_type_10_parses_with_exact_block_size: it writes a GGUF v3 file
("GGUF", version 3, one tensor, no metadata, tensor "q2.weight" with one
dimension of 256 and type 10 at offset 0, zero padding to 32 bytes, then the
84 bytes of fn block(3)) and expects the tensor's type to be Q2_K and its
length 84. The writer below restates that layout independently of the reader
under test; the other files extend it with metadata of every value type,
alignment overrides, several tensors and every kind of damage.
"""
import os
import struct

import numpy as np
import pytest

import ggml_q2_dequant_amd as q2k
import synth

QK_K, BB = 256, 84


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(q2k.LIB_PATH):
        pytest.skip("libq2k.so not built")
    return q2k.load_library()


def gstr(s):
    b = s.encode() if isinstance(s, str) else s
    return struct.pack("<Q", len(b)) + b


def kv(key, vtype, payload):
    return gstr(key) + struct.pack("<I", vtype) + payload


def write_gguf(path, tensors, kvs=(), version=3, align=32, data=b""):
    """tensors: (name, dims, type, offset); data is appended after padding to `align`."""
    out = bytearray(b"GGUF")
    out += struct.pack("<IQQ", version, len(tensors), len(kvs))
    for item in kvs:
        out += item
    for name, dims, ttype, off in tensors:
        out += gstr(name) + struct.pack("<I", len(dims)) + b"".join(struct.pack("<Q", d) for d in dims)
        out += struct.pack("<IQ", ttype, off)
    while len(out) % align:
        out.append(0)
    out += data
    with open(path, "wb") as f:
        f.write(out)
    return bytes(out)


def page_file(path):
    return write_gguf(path, [("q2.weight", [QK_K], 10, 0)], data=synth.page_block(3).tobytes())


def test_page_q2k_tensor_has_type_10_and_84_bytes(tmp_path):
    p = str(tmp_path / "q2.gguf")
    raw = page_file(p)
    with q2k.GGUFFile(p) as f:
        assert f.tensor_names() == ["q2.weight"]
        info = f.tensor_info("q2.weight")
        assert info["ggml_type"] == q2k.GGML_TYPE_Q2_K == 10
        assert info["byte_len"] == BB
        assert info["dims"] == [QK_K] and info["n_dims"] == 1
        assert info["file_offset"] % 32 == 0 and info["file_offset"] + BB == len(raw)
        assert np.array_equal(f.tensor_bytes("q2.weight"), synth.page_block(3))


def _all_value_kinds():
    return [
        kv("general.architecture", 8, gstr("deepseek")),
        kv("u8", 0, b"\x07"), kv("i8", 1, b"\xff"), kv("u16", 2, struct.pack("<H", 9)),
        kv("i16", 3, struct.pack("<h", -9)), kv("u32", 4, struct.pack("<I", 5)), kv("i32", 5, struct.pack("<i", -5)),
        kv("f32", 6, struct.pack("<f", 1.5)), kv("bool", 7, b"\x01"), kv("u64", 10, struct.pack("<Q", 1 << 40)),
        kv("i64", 11, struct.pack("<q", -(1 << 40))), kv("f64", 12, struct.pack("<d", 2.5)),
        kv("arr_u32", 9, struct.pack("<IQ", 4, 3) + struct.pack("<3I", 1, 2, 3)),
        kv("arr_str", 9, struct.pack("<IQ", 8, 2) + gstr("a") + gstr("bcd")),
        kv("arr_arr", 9, struct.pack("<IQ", 9, 2) + struct.pack("<IQ", 0, 2) + b"\x01\x02"
           + struct.pack("<IQ", 8, 1) + gstr("z")),
    ]


def test_metadata_of_every_kind_is_skipped_and_alignment_is_honoured(tmp_path):
    rng = np.random.Generator(np.random.PCG64(51))
    q2a = synth.random_blocks(rng, 2 * 3)              # Q2_K [512, 3]: 6 blocks
    f32 = np.arange(7, dtype="<f4").tobytes()           # F32 [7]
    kvs = _all_value_kinds() + [kv("general.alignment", 4, struct.pack("<I", 64))]
    data = q2a.tobytes() + b"\0" * 8 + f32 + b"\0" * 4 + b"\x11" * 40
    tensors = [("blk.0.w", [512, 3], 10, 0), ("norm", [7], 0, len(q2a) + 8),
               ("other", [32, 2], 12, len(q2a) + 8 + 28 + 4)]
    p = str(tmp_path / "many.gguf")
    raw = write_gguf(p, tensors, kvs=kvs, align=64, data=data)
    with q2k.GGUFFile(p) as f:
        assert f.tensor_names() == ["blk.0.w", "norm", "other"]
        a = f.tensor_info("blk.0.w")
        assert a["file_offset"] % 64 == 0 and a["byte_len"] == 6 * BB and a["dims"] == [512, 3]
        assert np.array_equal(f.tensor_bytes("blk.0.w"), q2a)
        n = f.tensor_info("norm")
        assert n["byte_len"] == 28 and n["ggml_type"] == 0
        assert np.array_equal(f.tensor_bytes("norm").view("<f4"), np.arange(7, dtype=np.float32))
        o = f.tensor_info("other")
        assert o["ggml_type"] == 12 and o["byte_len"] == 0  # size of that type unknown here
        with pytest.raises(q2k.Q2KInvalidArgument, match="unknown"):
            f.tensor_bytes("other")
        with pytest.raises(q2k.Q2KInvalidArgument, match="no tensor"):
            f.tensor_info("missing")
    assert len(raw) > 0


def test_version_2_is_read_like_version_3(tmp_path):
    p = str(tmp_path / "v2.gguf")
    write_gguf(p, [("q2.weight", [QK_K], 10, 0)], version=2, data=synth.page_block(3).tobytes())
    with q2k.GGUFFile(p) as f:
        assert f.tensor_info("q2.weight")["byte_len"] == BB


@pytest.mark.parametrize("mutate,frag", [
    (lambda b: b"GGUG" + b[4:], "magic"),
    (lambda b: b[:4] + struct.pack("<I", 1) + b[8:], "version"),
    (lambda b: b[:8] + struct.pack("<Q", 1 << 60) + b[16:], "implausible"),
])
def test_damaged_headers_are_rejected(tmp_path, mutate, frag):
    p = str(tmp_path / "bad.gguf")
    raw = page_file(p)
    with open(p, "wb") as f:
        f.write(mutate(raw))
    with pytest.raises(q2k.Q2KInvalidArgument, match=frag):
        q2k.GGUFFile(p)


def test_every_truncation_fails_cleanly(tmp_path):
    p = str(tmp_path / "t.gguf")
    raw = write_gguf(p, [("blk.0.w", [512, 3], 10, 0)], kvs=_all_value_kinds(),
                     data=synth.random_blocks(np.random.Generator(np.random.PCG64(52)), 6).tobytes())
    header_end = raw.index(b"blk.0.w") + len("blk.0.w") + 4 + 16 + 12
    for cut in range(len(raw)):
        with open(p, "wb") as f:
            f.write(raw[:cut])
        if cut < header_end:
            with pytest.raises(q2k.Q2KInvalidArgument):
                q2k.GGUFFile(p)
        else:  # the directory is whole; the data itself is short
            with q2k.GGUFFile(p) as f:
                if cut < len(raw):
                    with pytest.raises(q2k.Q2KInvalidArgument, match="outside the file"):
                        f.tensor_info("blk.0.w")


def test_random_byte_damage_never_crashes(tmp_path):
    p = str(tmp_path / "fuzz.gguf")
    raw = bytearray(write_gguf(p, [("a", [QK_K], 10, 0), ("b", [QK_K, 2], 10, BB)], kvs=_all_value_kinds(),
                               data=synth.random_blocks(np.random.Generator(np.random.PCG64(53)), 3).tobytes()))
    rng = np.random.Generator(np.random.PCG64(54))
    for _ in range(400):
        bad = bytearray(raw)
        for pos in rng.integers(0, len(bad), int(rng.integers(1, 6))):
            bad[pos] = int(rng.integers(0, 256))
        with open(p, "wb") as f:
            f.write(bad)
        try:
            with q2k.GGUFFile(p) as f:
                for name in f.tensor_names():
                    try:
                        info = f.tensor_info(name)
                        if info["byte_len"]:
                            assert info["file_offset"] + info["byte_len"] <= len(bad)
                            f.tensor_bytes(name)
                    except q2k.Q2KInvalidArgument:
                        pass
        except q2k.Q2KInvalidArgument:
            pass


@pytest.mark.parametrize("tensors,frag", [
    ([("w", [300], 10, 0)], "multiple of 256"),
    ([("w", [QK_K], 10, 1 << 20)], "outside the file"),
])
def test_bad_tensor_records_are_rejected_on_lookup(tmp_path, tensors, frag):
    p = str(tmp_path / "r.gguf")
    write_gguf(p, tensors, data=synth.page_block(3).tobytes())
    with q2k.GGUFFile(p) as f:
        with pytest.raises(q2k.Q2KInvalidArgument, match=frag):
            f.tensor_info("w")


@pytest.mark.parametrize("tensors,frag", [
    ([("w", [], 10, 0)], "dimensions"),
    ([("w", [1, 1, 1, 1, 256], 10, 0)], "dimensions"),
    ([("w", [QK_K], 10, 0), ("w", [QK_K], 10, 0)], "duplicate"),
])
def test_bad_directories_are_rejected_on_open(tmp_path, tensors, frag):
    p = str(tmp_path / "d.gguf")
    write_gguf(p, tensors, data=synth.page_block(3).tobytes())
    with pytest.raises(q2k.Q2KInvalidArgument, match=frag):
        q2k.GGUFFile(p)


def test_missing_file_and_null_arguments(tmp_path, lib):
    with pytest.raises(q2k.Q2KInvalidArgument, match="cannot open"):
        q2k.GGUFFile(str(tmp_path / "nope.gguf"))
    assert lib.q2k_gguf_open(None, None) == q2k.Q2K_ERR_INVALID_ARGUMENT
    assert lib.q2k_gguf_tensor_count(None) == 0
    assert lib.q2k_gguf_tensor_name(None, 0) is None
    lib.q2k_gguf_close(None)


@pytest.mark.gpu
def test_page_tensor_decodes_on_the_gpu_like_the_oracle(tmp_path):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    p = str(tmp_path / "q2.gguf")
    page_file(p)
    with q2k.GGUFFile(p) as f:
        data = f.tensor_bytes("q2.weight")
    out = torch.empty(QK_K, dtype=torch.float32, device="cuda:0")
    q2k.q2k_dequantize(torch.from_numpy(data).to("cuda:0"), out)
    torch.cuda.synchronize()
    want = oracle.dequant_block(synth.page_block(3))
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))

