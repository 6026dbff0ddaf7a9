"""CPU tests of the C ABI: the library loads, exports every function the header
declares, and rejects bad arguments on the host before anything is launched.
No call here reaches a kernel."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gva.h")

gva = pytest.importorskip("compact_kv_cache_amd", reason="libgva.so not built")
from compact_kv_cache_amd import _lib  # noqa: E402

FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gva_[a-z_0-9]+)\s*\(", text)))


def test_header_functions_exported():
    funcs = _header_functions()
    assert set(funcs) == set(_lib.SIGNATURES), "binding and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for f in funcs:
        assert f in exported, f"{f} declared in gva.h but not exported"
        assert hasattr(gva.lib, f)


def test_no_cxx_symbols_leak_into_abi():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    gva_syms = [ln.split()[-1] for ln in out.splitlines() if " T gva_" in ln]
    assert sorted(gva_syms) == _header_functions()


def test_struct_layout_matches_header():
    assert ctypes.sizeof(_lib.GvaShape) == 13 * 4


def test_status_strings_and_version():
    assert gva.gva_status_string(0) == "GVA_OK"
    assert gva.gva_status_string(3) == "GVA_ERR_WORKSPACE"
    assert gva.gva_abi_version() == 1


def test_cache_bytes_per_token():
    # G value rows plus one shared positional key
    assert gva.gva_cache_bytes_per_token(4, 64, 16, "bf16") == 544
    assert gva.gva_cache_bytes_per_token(4, 64, 24, "bf16") == 560
    assert gva.gva_cache_bytes_per_token(4, 64, 16, "f32") == 1088
    assert gva.gva_cache_bytes_per_token(4, 64, 0, "bf16") * 2 == 2 * 4 * 64 * 2  # half of GQA


def _shape(**kw):
    base = dict(B=4, H=16, G=4, d_n=64, d_v=64, d_r=16, capacity=131072, max_seq_len=131072,
                split_tokens=4096, dtype="bf16")
    base.update(kw)
    return gva.make_shape(**base)


def test_workspace_size_long_split():
    s = _shape()
    assert gva.gva_decode_split_tokens(s) == 4096
    # arrival counters (B * G + B of them, one per 128-byte line), then
    # B * H * 32 partitions * (64 + 2) floats of partials
    assert gva.gva_decode_workspace_bytes(s) == (16 + 4) * 128 + 4 * 16 * 32 * 66 * 4 == 2560 + 540672
    assert gva.gva_decode_workspace_bytes(_shape(max_seq_len=4096)) == 0


def test_auto_split_is_multiple_of_64():
    for n in [1, 63, 64, 4096, 4197, 32768, 131072]:
        s = _shape(split_tokens=0, max_seq_len=n, capacity=131072)
        sp = gva.gva_decode_split_tokens(s)
        assert sp > 0 and sp % 64 == 0


@pytest.mark.parametrize("B,n", [(16, 4096), (16, 4196), (16, 2100), (32, 8192), (4, 131072),
                                 (64, 32868), (64, 16960), (64, 30720), (1, 256), (3, 1100)])
def test_auto_split_partitions(B, n):
    """Auto partitions: whole 64-token tiles, at least 8 per partition, and no
    more (sequence, group, partition) workgroups than the 256 compute units
    when the sequences are long enough to need more than one partition --
    except a batch that fills the units by itself (B*G >= 256) with sequences
    of at least 3 x 160 tiles, which is split into thirds of >= 160 tiles."""
    s = _shape(B=B, split_tokens=0, max_seq_len=n, capacity=max(n, 64))
    tiles_per = gva.gva_decode_split_tokens(s) // 64
    tiles = -(-n // 64)
    parts = -(-tiles // tiles_per)
    assert tiles_per >= 8
    want = -(-256 // (B * 4))
    if want == 1 and tiles >= 3 * 160:
        want = 3
        assert parts == 3 and tiles_per >= 160
    elif parts > 1:
        assert parts * B * 4 <= 256
    assert tiles_per == max(8, -(-tiles // want))


def test_auto_split_mid():
    # 16 sequences of up to 4196 tokens (66 tiles): 4 partitions of 17 tiles
    assert gva.gva_decode_split_tokens(_shape(B=16, split_tokens=0, max_seq_len=4196)) == 17 * 64
    assert gva.gva_decode_split_tokens(_shape(B=16, split_tokens=0, max_seq_len=4096)) == 16 * 64


def _decode_status(shape, ws=None, ws_bytes=0, **ptrs):
    p = dict(q_nope=FAKE, q_rope=FAKE, M=FAKE, v=FAKE, kr=FAKE, seq=FAKE, table=None, out=FAKE)
    p.update(ptrs)
    return gva.lib.gva_decode(shape, p["q_nope"], p["q_rope"], p["M"], p["v"], p["kr"], p["seq"],
                              p["table"], 0.125, p["out"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=15), _lib.GVA_ERR_INVALID_ARGUMENT),          # H % G
    (dict(H=64), _lib.GVA_ERR_UNSUPPORTED),               # 16 heads per group
    (dict(d_v=128), _lib.GVA_ERR_UNSUPPORTED),
    (dict(d_r=15), _lib.GVA_ERR_INVALID_ARGUMENT),
    (dict(d_r=40), _lib.GVA_ERR_UNSUPPORTED),
    (dict(dtype="bf16", split_tokens=100), _lib.GVA_ERR_INVALID_ARGUMENT),
    (dict(max_seq_len=200000), _lib.GVA_ERR_INVALID_ARGUMENT),   # beyond capacity
    (dict(block_size=32), _lib.GVA_ERR_UNSUPPORTED),
    (dict(B=0), _lib.GVA_ERR_INVALID_ARGUMENT),
])
def test_decode_rejects_bad_shapes(kw, status):
    assert _decode_status(_shape(**kw), FAKE, 1 << 30) == status
    assert gva.lib.gva_last_error()


def test_decode_rejects_missing_pointers_and_workspace():
    s = _shape()
    assert _decode_status(s, FAKE, 1 << 30, q_nope=None) == _lib.GVA_ERR_INVALID_ARGUMENT
    assert _decode_status(s, FAKE, 1 << 30, kr=None) == _lib.GVA_ERR_INVALID_ARGUMENT
    assert _decode_status(s, None, 0) == _lib.GVA_ERR_WORKSPACE
    assert _decode_status(s, FAKE, 256 + 540671) == _lib.GVA_ERR_WORKSPACE
    assert _decode_status(s, FAKE + 8, 1 << 30) == _lib.GVA_ERR_WORKSPACE   # (m, l) pairs: 8-byte words
    paged = _shape(block_size=64, num_blocks=100, max_blocks_per_seq=2048, capacity=0)
    assert _decode_status(paged, FAKE, 1 << 30, table=None) == _lib.GVA_ERR_INVALID_ARGUMENT
    assert gva.lib.gva_decode(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1.0, FAKE, None, 0,
                              None) == _lib.GVA_ERR_INVALID_ARGUMENT


def test_decode_rejects_bad_scale():
    s = _shape()
    for bad in (0.0, -0.5, float("inf"), float("nan")):
        st = gva.lib.gva_decode(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, bad, FAKE, FAKE, 1 << 30,
                                None)
        assert st == _lib.GVA_ERR_INVALID_ARGUMENT


def test_append_and_rope_query_reject_bad_arguments():
    s = _shape()
    L = gva.lib
    assert L.gva_append(s, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, 10000.0, None) == 1   # n_new
    assert L.gva_append(s, None, FAKE, 1, FAKE, FAKE, FAKE, None, 10000.0, None) == 1
    assert L.gva_append(s, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, -1.0, None) == 1     # base
    paged = _shape(block_size=64, num_blocks=10, max_blocks_per_seq=8, capacity=0, max_seq_len=512)
    assert L.gva_append(paged, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, 10000.0, None) == 1
    assert L.gva_rope_query(s, None, FAKE, FAKE, 10000.0, None) == 1
    assert L.gva_rope_query(_shape(H=15), FAKE, FAKE, FAKE, 10000.0, None) == 1


def test_gqa_reference_rejects_positional_width():
    s = _shape(d_r=16)
    st = gva.lib.gva_gqa_ref_decode(s, FAKE, FAKE, FAKE, FAKE, None, 0.125, FAKE, FAKE, 1 << 30,
                                    None)
    assert st == _lib.GVA_ERR_INVALID_ARGUMENT


def test_binding_refuses_host_tensors():
    import torch
    s = _shape(split_tokens=0, max_seq_len=64, capacity=64, B=1)
    x = torch.zeros(16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gva.gva_decode(s, x, x, x, x, x, torch.zeros(1, dtype=torch.int32), None, 0.1, x)


def _short_size_error(fn, *args):
    """The wrapper must refuse before the C call: a size error, not the
    device check that a host tensor of the right size would reach."""
    with pytest.raises(ValueError, match="elements"):
        fn(*args)


def test_binding_rejects_short_tensors():
    import torch
    bf = torch.bfloat16
    B, H, G, cap = 2, 16, 4, 128
    s = _shape(B=B, split_tokens=0, max_seq_len=cap, capacity=cap)
    z = lambda *shape, dt=bf: torch.zeros(*shape, dtype=dt)  # noqa: E731
    q, qr, M = z(B, H, 64), z(B, H, 16), z(H, 64, 64)
    vc, kc = z(B, G, cap, 64), z(B, cap, 16)
    lens, out = z(B, dt=torch.int32), z(B, H, 64)
    # every tensor of the decode one element short (the tensors before it are
    # passed as None, so that the short one is the first the binding checks)
    tensor_slots = [0, 1, 2, 3, 4, 5, 8]
    for slot in tensor_slots:
        args = [q, qr, M, vc, kc, lens, None, 0.1, out]
        for j in tensor_slots:
            if j < slot:
                args[j] = None
        args[slot] = args[slot].reshape(-1)[:-1].clone()
        _short_size_error(gva.gva_decode, s, *args)
    # the fused step's new-token tensors and the append's
    _short_size_error(gva.gva_decode_step, s, z(B, G, 63), z(B, 16), q, qr, M, vc, kc, lens, None,
                      0.1, 10000.0, out, None)
    _short_size_error(gva.gva_decode_step, s, None, z(B * 16 - 1), q, qr, M, vc, kc, lens,
                      None, 0.1, 10000.0, out, None)
    _short_size_error(gva.gva_append, s, z(B, G, 3, 64), z(B, 4, 16), 4, lens, vc, kc)
    # a paged cache: the table and the pool size come from the shape
    sp = gva.make_shape(B, H, G, 64, 64, 16, max_seq_len=128, block_size=64, num_blocks=8,
                        max_blocks_per_seq=2)
    _short_size_error(gva.gva_decode, sp, None, None, None, None, None, None,
                      z(3, dt=torch.int32), 0.1, out)
    _short_size_error(gva.gva_decode, sp, None, None, None, z(7, G, 64, 64), z(8, 64, 16), lens,
                      z(4, dt=torch.int32), 0.1, out)
    _short_size_error(gva.gva_rollback, sp, None, z(B - 1, dt=torch.int32))
    _short_size_error(gva.gva_rope_query, s, None, z(B * H * 16 - 1), lens)


def test_binding_right_sizes_reach_the_device_check():
    import torch
    B, cap = 2, 128
    s = _shape(B=B, split_tokens=0, max_seq_len=cap, capacity=cap)
    z = lambda *shape, dt=torch.bfloat16: torch.zeros(*shape, dtype=dt)  # noqa: E731
    with pytest.raises(ValueError, match="device tensor"):
        gva.gva_decode(s, z(B, 16, 64), z(B, 16, 16), z(16, 64, 64), z(B, 4, cap, 64), z(B, cap, 16),
                       z(B, dt=torch.int32), None, 0.1, z(B, 16, 64))
