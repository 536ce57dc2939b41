"""C-ABI checks that need no GPU: exported symbols, host-side validation, layout sizes."""
import ctypes
import re
import os

import pytest

import bit_asymmetric_kv_amd as kvq
from bit_asymmetric_kv_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvq.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = kvq.load()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in kvq.h but not exported"
    assert set(names) == set(_lib.EXPORTED)


def test_group_bytes():
    assert kvq.group_bytes(2) == 3072
    assert kvq.group_bytes(4) == 5120
    assert kvq.group_bytes(3) == 4096
    assert kvq.group_bytes(5) == 0


def _status(cfg):
    lib = kvq.load()
    h = ctypes.c_void_p(0)
    s = lib.kvq_create(ctypes.byref(cfg), None, 0, None, ctypes.byref(h))
    return s, lib.kvq_last_error().decode()


@pytest.mark.parametrize("field,value", [
    ("batch", 0), ("num_kv_heads", 0), ("num_q_heads", 12), ("head_dim", 64), ("bits", 1), ("bits", 5), ("bits", 8),
    ("group", 64), ("residual", 48), ("residual", -32), ("rotate", 2), ("max_tokens", 0),
    ("max_tokens", 1 << 31), ("softmax_scale", -1.0), ("softmax_scale", float("inf")), ("sink", 2),
    ("sink", -1), ("rope", 2), ("rope_base", 0.5), ("rope_base", float("inf")), ("rope_base", -3.0),
    ("page_groups", 3), ("page_groups", -1), ("page_groups", 1 << 17),
])
def test_invalid_configs_rejected_before_any_device_call(field, value):
    cfg = kvq.make_config(2, 32, 8, residual=128, max_tokens=1000)
    setattr(cfg, field, value)
    s, msg = _status(cfg)
    assert s == _lib.KVQ_ERR_INVALID_ARG, (field, value, s, msg)
    assert msg


@pytest.mark.parametrize("batch,hq,hkv,max_tokens", [
    (65536, 8, 8, 1000),            # sequences in grid.z / grid.y of the append and combine launches
    (1, 65536, 65536, 1000),        # kv-heads in grid.y of the append launches
    (65535, 32, 32, 1 << 20),       # 2.1e6 (sequence, kv-head) pairs x 2049 decode workgroups overflow the 1-D grid
    (40000, 8 * 60000, 60000, 64),  # within the per-axis limits, but 2.4e9 (sequence, kv-head) pairs
])
def test_launch_grid_limits_rejected_before_any_device_call(batch, hq, hkv, max_tokens):
    cfg = kvq.make_config(batch, hq, hkv, residual=32, max_tokens=max_tokens)
    s, msg = _status(cfg)
    assert s == _lib.KVQ_ERR_INVALID_ARG, (batch, hkv, s, msg)
    assert "grid" in msg or "workgroups" in msg


def test_largest_grid_shapes_pass_validation():
    # at the limits the configuration is valid (only its size is asked for: no device call)
    assert kvq.cache_bytes(kvq.make_config(65535, 8, 8, residual=0, max_tokens=32)) > 0
    assert kvq.cache_bytes(kvq.make_config(1, 65535, 65535, residual=0, max_tokens=32)) > 0


def test_paged_cache_needs_a_pool():
    cfg = kvq.make_config(1, 8, 8, residual=32, max_tokens=100, page_groups=4, pool_pages=0)
    assert _status(cfg)[0] == _lib.KVQ_ERR_INVALID_ARG


def test_paged_cache_bytes_follow_the_pool():
    small = kvq.cache_bytes(kvq.make_config(2, 32, 8, residual=128, max_tokens=131072, page_groups=16,
                                            pool_pages=10))
    big = kvq.cache_bytes(kvq.make_config(2, 32, 8, residual=128, max_tokens=131072, page_groups=16,
                                          pool_pages=110))
    assert big - small == 100 * 8 * 16 * 3072


def test_rope_with_hadamard_rotation_rejected():
    cfg = kvq.make_config(1, 8, 8, residual=32, max_tokens=100, rotate=True, rope=True)
    assert _status(cfg)[0] == _lib.KVQ_ERR_INVALID_ARG


def test_rope_cache_holds_its_rotary_tables():
    plain = kvq.cache_bytes(kvq.make_config(1, 32, 8, residual=128, max_tokens=131072))
    rope = kvq.cache_bytes(kvq.make_config(1, 32, 8, residual=128, max_tokens=131072, rope=True))
    # one 512-byte row per group start (4096 groups) plus the 16 KB in-group table
    assert rope - plain >= 4096 * 512 + 32 * 128 * 4


def test_gqa_ratio_16_rejected():
    cfg = kvq.make_config(1, 32, 2)
    assert _status(cfg)[0] == _lib.KVQ_ERR_INVALID_ARG


def test_valid_config_reports_no_device_here_or_succeeds():
    import torch
    cfg = kvq.make_config(1, 8, 8, residual=32, max_tokens=100)
    s, _ = _status(cfg)
    if torch.cuda.is_available():
        assert s == _lib.KVQ_OK
    else:
        assert s == _lib.KVQ_ERR_NO_DEVICE


def test_null_arguments():
    lib = kvq.load()
    assert lib.kvq_append(None, None, None, None, 0, None) == _lib.KVQ_ERR_INVALID_ARG
    assert lib.kvq_decode_attention(None, None, None, None) == _lib.KVQ_ERR_INVALID_ARG
    assert lib.kvq_seq_len(None, 0, None, None) == _lib.KVQ_ERR_INVALID_ARG
    assert lib.kvq_set_decode_split(None, 0) == _lib.KVQ_ERR_INVALID_ARG
    assert lib.kvq_read_state(None, 0, 0, 0, 0, None, 0, None) == _lib.KVQ_ERR_INVALID_ARG
    lib.kvq_destroy(None)
    n = ctypes.c_size_t(0)
    assert lib.kvq_cache_bytes(None, ctypes.byref(n)) == _lib.KVQ_ERR_INVALID_ARG


def test_cache_bytes_grows_with_capacity_and_holds_the_blocks():
    small = kvq.cache_bytes(kvq.make_config(1, 32, 8, residual=128, max_tokens=131072))
    big = kvq.cache_bytes(kvq.make_config(1, 32, 8, residual=128, max_tokens=1 << 20))
    assert big > small
    # the packed store alone: 8 heads x 32768 groups x 3072 B = 768 MiB at 1M tokens
    assert big >= 8 * 32768 * 3072
    four = kvq.cache_bytes(kvq.make_config(1, 32, 8, bits=4, residual=128, max_tokens=131072))
    assert four - small >= 8 * 4096 * (5120 - 3072)
    # an attention sink adds one FP16 key and value row per (sequence, kv-head)
    sink = kvq.cache_bytes(kvq.make_config(1, 32, 8, residual=128, max_tokens=131072, sink=True))
    assert sink - small >= 8 * 2 * 128 * 2


def test_comparison_entry_points_validate_on_the_host():
    lib = kvq.load()
    cfg = _lib.KVQFp16Config(1, 32, 8, 128, 4096, 0.0)
    n = ctypes.c_size_t(0)
    assert lib.kvq_fp16_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)) == _lib.KVQ_OK
    assert n.value == 1 * 32 * 1024 * 130 * 4
    bad = _lib.KVQFp16Config(1, 12, 8, 128, 4096, 0.0)   # Hq not a multiple of Hkv
    assert lib.kvq_fp16_workspace_bytes(ctypes.byref(bad), ctypes.byref(n)) == _lib.KVQ_ERR_INVALID_ARG
    fake = ctypes.c_void_p(256)   # never dereferenced: every check below fails first
    # head_dim other than 128
    c2 = _lib.KVQFp16Config(1, 32, 8, 64, 4096, 0.0)
    assert lib.kvq_fp16_decode_attention(ctypes.byref(c2), fake, fake, fake, 10, fake, fake, fake, 1 << 30,
                                         None) == _lib.KVQ_ERR_INVALID_ARG
    # max_len above t_cap
    assert lib.kvq_fp16_decode_attention(ctypes.byref(cfg), fake, fake, fake, 4097, fake, fake, fake, 1 << 30,
                                         None) == _lib.KVQ_ERR_INVALID_ARG
    # workspace too small
    assert lib.kvq_fp16_decode_attention(ctypes.byref(cfg), fake, fake, fake, 100, fake, fake, fake, 16,
                                         None) == _lib.KVQ_ERR_OOM
    # null pointers
    assert lib.kvq_fp16_decode_attention(ctypes.byref(cfg), None, fake, fake, 100, fake, fake, fake, 1 << 30,
                                         None) == _lib.KVQ_ERR_INVALID_ARG
    # stream read: size not a multiple of 16, misaligned buffer, null fold array, fold words out of range
    assert lib.kvq_stream_read(fake, 100, fake, 64, None) == _lib.KVQ_ERR_INVALID_ARG
    assert lib.kvq_stream_read(ctypes.c_void_p(264), 1024, fake, 64, None) == _lib.KVQ_ERR_INVALID_ARG
    assert lib.kvq_stream_read(fake, 1024, None, 64, None) == _lib.KVQ_ERR_INVALID_ARG
    assert lib.kvq_stream_read(fake, 1024, fake, 0, None) == _lib.KVQ_ERR_INVALID_ARG
    assert lib.kvq_stream_read(fake, 1024, fake, (1 << 16) + 1, None) == _lib.KVQ_ERR_INVALID_ARG
