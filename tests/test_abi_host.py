"""C-ABI checks that need no GPU: the library loads, exports every function
include/fs.h declares, and rejects invalid requests on the host before any
device work (status codes as documented in the header)."""
import ctypes
import os
import re

import pytest

import lm_head_gumbel_amd as fs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fs.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fs.LIB_PATH),
                                reason="libfs.so not built (python -m lm_head_gumbel_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fs_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fs_sample", "fs_sample_grouped", "fs_sample_topk", "fs_sample_topk_topp",
              "fs_merge_online",
              "fs_logits", "fs_multinomial", "fs_workspace_bytes", "fs_status_string",
              "fs_debug_noise", "fs_num_tiles", "fs_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    raw = ctypes.CDLL(fs.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(raw, n)]
    assert not missing, missing
    # and the binding wraps every one of them under the same name
    for n in declared_functions():
        assert callable(getattr(fs, n)), n


def test_status_strings_and_version():
    assert fs.fs_status_string(fs.FS_OK) == "FS_OK"
    assert fs.fs_status_string(fs.FS_ERR_WORKSPACE) == "FS_ERR_WORKSPACE"
    assert fs.fs_status_string(99) == "FS_ERR_UNKNOWN"
    assert "gfx950" in fs.fs_version()


def test_struct_layout_matches_header():
    assert ctypes.sizeof(fs.fs_params) == 56
    assert fs.fs_params.seed.offset == 24
    assert fs.fs_params.seeds.offset == 40 and fs.fs_params.step_ptr.offset == 48


def test_num_tiles():
    assert fs.fs_num_tiles(fs.params(4, 256, 4096, tile_v=512)) == 8
    assert fs.fs_num_tiles(fs.params(1, 4096, 151936, tile_v=128)) == 1187
    assert fs.fs_num_tiles(fs.params(1, 4096, 151936, tile_v=256)) == 594
    assert fs.fs_num_tiles(fs.params(1, 4096, 151936)) == 1187       # default 128
    assert fs.fs_num_tiles(fs.params(1, 64, 0)) == 0
    assert fs.fs_num_tiles(fs.params(1, 64, 100, tile_v=24)) == -1   # not a multiple of 16


def test_null_and_negative_arguments_are_rejected():
    p = fs.params(2, 64, 128)
    assert fs.lib().fs_sample(None, None, None, None, None, None, None, None, 0, None) == \
        fs.FS_ERR_INVALID_ARG
    assert fs.fs_sample(p, None, None, None, None, None) == fs.FS_ERR_INVALID_ARG
    assert fs.fs_sample(p, None, None, None, None, 0x1000) == fs.FS_ERR_INVALID_ARG  # null H/W
    assert fs.fs_sample(fs.params(-1, 64, 128), 16, 16, None, None, 16) == fs.FS_ERR_INVALID_ARG
    assert fs.fs_sample(fs.params(2, 64, -5), 16, 16, None, None, 16) == fs.FS_ERR_INVALID_ARG
    assert fs.fs_sample(fs.params(2, 64, 128, flags=8), 16, 16, None, None, 16) == \
        fs.FS_ERR_INVALID_ARG
    assert fs.fs_sample_topk(p, 16, 16, None, None, 0, 16) == fs.FS_ERR_INVALID_ARG
    for bad in (0.0, -0.5, 1.5, float("nan")):
        assert fs.fs_sample_topk_topp(p, 16, 16, None, None, 5, bad, 16) == fs.FS_ERR_INVALID_ARG
    assert fs.fs_sample_grouped(p, 16, 16, None, None, None, None, None) == fs.FS_ERR_INVALID_ARG
    assert fs.fs_merge_online(-1, 4, None, None, None, 0, 0, 0, None) == fs.FS_ERR_INVALID_ARG
    assert fs.fs_merge_online(2, 4, None, None, None, 0, 0, 0, 0x1000) == fs.FS_ERR_INVALID_ARG
    assert fs.fs_logits(p, 16, 16, None, 16, 1 << 20) == fs.FS_ERR_INVALID_ARG
    assert fs.fs_multinomial(p, None, None, None, 0x1000) == fs.FS_ERR_INVALID_ARG
    assert fs.fs_debug_noise(0, 0, 0, 0, 1, -1, 4, 0x1000) == fs.FS_ERR_INVALID_ARG
    # the shared-read probe wants whole 32 KiB steps and at least one pass
    assert fs.fs_debug_shared_read_probe(0x1000, 1000, 1, 0x1000, 8) == fs.FS_ERR_INVALID_ARG
    assert fs.fs_debug_shared_read_probe(0x1000, 32768, 0, 0x1000, 8) == fs.FS_ERR_INVALID_ARG
    # both read probes want whole 16-byte words, a sink and a grid
    for probe in (fs.fs_debug_read_probe, fs.fs_debug_read_probe_nt):
        assert probe(0x1000, 1000, 0x1000, 8) == fs.FS_ERR_INVALID_ARG
        assert probe(0x1000, 1024, None, 8) == fs.FS_ERR_INVALID_ARG
        assert probe(0x1000, 1024, 0x1000, 0) == fs.FS_ERR_INVALID_ARG


def test_unsupported_requests_are_reported():
    assert fs.fs_sample(fs.params(2, 60, 128), 16, 16, None, None, 16) == fs.FS_ERR_UNSUPPORTED
    assert fs.fs_sample(fs.params(2, 64, 128, v_offset=8), 16, 16, None, None, 16) == \
        fs.FS_ERR_UNSUPPORTED
    assert fs.fs_sample_grouped(fs.params(2, 64, 128, tile_v=100), 16, 16, None, None,
                                16, 16, 16) == fs.FS_ERR_UNSUPPORTED
    assert fs.fs_sample_topk(fs.params(2, 64, 128), 16, 16, None, None, 1025, 16) == \
        fs.FS_ERR_UNSUPPORTED
    assert fs.fs_sample_topk_topp(fs.params(2, 64, 128), 16, 16, None, None, 1025, 0.5, 16) == \
        fs.FS_ERR_UNSUPPORTED
    # misaligned operands (16-byte loads)
    assert fs.fs_sample(fs.params(2, 64, 128), 18, 16, None, None, 16) == fs.FS_ERR_UNSUPPORTED


def test_empty_batch_is_a_no_op():
    p = fs.params(0, 64, 128)
    assert fs.fs_sample(p, None, None, None, None, None) == fs.FS_OK
    assert fs.fs_sample_topk(p, None, None, None, None, 5, None) == fs.FS_OK
    assert fs.fs_sample_topk_topp(p, None, None, None, None, 5, 0.9, None) == fs.FS_OK
    assert fs.fs_logits(p, None, None, None, None) == fs.FS_OK
    assert fs.fs_merge_online(0, 3, None, None, None, 0, 0, 0, None) == fs.FS_OK


def test_workspace_query_rejects_bad_requests():
    assert fs.fs_workspace_bytes(fs.params(2, 60, 128), fs.FS_VARIANT_FLAT) == 0
    assert fs.fs_workspace_bytes(fs.params(2, 64, 128), 7) == 0
    assert fs.fs_workspace_bytes(fs.params(2, 64, 128), -1) == 0
    assert fs.fs_workspace_bytes(fs.params(2, 64, 128), fs.FS_VARIANT_TOPK, 0) == 0
