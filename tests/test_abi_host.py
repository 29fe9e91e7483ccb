"""Host-side checks of libpw.so that need no GPU: every function declared in
include/pw.h is exported, the host bit-plane packer matches an independent
numpy unpacker written from the header's format description, and argument
validation returns PW_ERR_INVALID."""
import ctypes
import os
import re

import numpy as np
import pytest

import any_precision_expert_amd as pw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "pw.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pw_[a-z_]+)\s*\(", src)))


def test_header_declares_what_the_binding_lists():
    assert _declared() == sorted(pw.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(pw.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name


def _unpack_top(planes, R, K, q):
    """Child codes from the top q planes, following the layout stated in pw.h:
    word w of row r at [(w // 4) * R + r] * 4 + w % 4 of each plane; column
    32w + 8P + 2i + h at bit 8i + 4h + P; plane p = bit (7 - p)."""
    codes = np.zeros((R, K), dtype=np.int64)
    j = np.arange(32)
    bitpos = 8 * ((j >> 1) & 3) + 4 * (j & 1) + (j >> 3)
    for w in range(K // 32):
        at = ((w // 4) * R + np.arange(R)) * 4 + (w % 4)
        for p in range(q):
            words = planes[p][at].astype(np.int64)
            bits = (words[:, None] >> bitpos[None, :]) & 1
            codes[:, 32 * w:32 * w + 32] |= bits << (q - 1 - p)
    return codes


@pytest.mark.parametrize("R,K", [(1, 32), (3, 96), (64, 128), (70, 416), (5, 256)])
def test_packer_truncation_identity(R, K):
    rng = np.random.default_rng(R * 1000 + K)
    code8 = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    planes = pw.pack_bitplanes(code8)
    nchunks = -(-K // 128)
    assert planes.shape == (8, nchunks * R * 4)
    for q in range(1, 9):
        assert np.array_equal(_unpack_top(planes, R, K, q), code8.astype(np.int64) >> (8 - q)), q


def test_packer_pads_partial_chunk_with_zero_words():
    code8 = np.full((4, 160), 255, dtype=np.uint8)  # 5 words: one full chunk + 1 word
    planes = pw.pack_bitplanes(code8)
    second = planes[:, 4 * 4:].reshape(8, 4, 4)  # chunk 1: [R][4]
    assert np.all(second[:, :, 0] == 0xFFFFFFFF)
    assert np.all(second[:, :, 1:] == 0)


def test_packer_every_code_every_position():
    # each code value at every column position of a word, across rows
    R, K = 256, 32
    code8 = ((np.arange(R)[:, None] + np.arange(K)[None, :]) % 256).astype(np.uint8)
    planes = pw.pack_bitplanes(code8)
    assert np.array_equal(_unpack_top(planes, R, K, 8), code8.astype(np.int64))


def test_packer_rejects_bad_shapes():
    L = pw.lib()
    buf = np.zeros(1024, dtype=np.uint32)
    codes = np.zeros(64, dtype=np.uint8)
    assert L.pw_pack_bitplanes(codes.ctypes.data, 2, 30, buf.ctypes.data) == pw.PW_ERR_INVALID
    assert "multiple of 32" in pw.last_error()
    assert L.pw_pack_bitplanes(None, 2, 32, buf.ctypes.data) == pw.PW_ERR_INVALID
    assert L.pw_pack_bitplanes(codes.ctypes.data, 0, 32, buf.ctypes.data) == pw.PW_ERR_INVALID


def test_plane_words():
    assert pw.plane_words(10, 128) == 40
    assert pw.plane_words(10, 160) == 80
    assert pw.plane_words(0, 128) == 0


def test_create_rejects_bad_descriptions():
    L = pw.lib()
    h = ctypes.c_void_p()
    bad = [pw.ModelDesc(1, 4, 250, 512, 0, 2, 1),   # H not a multiple of 32
           pw.ModelDesc(1, 4, 256, 500, 0, 2, 1),   # I not a multiple of 32
           pw.ModelDesc(1, 4, 256, 512, 0, 9, 1),   # top_k > 8
           pw.ModelDesc(1, 2, 256, 512, 0, 3, 1),   # top_k > E
           pw.ModelDesc(0, 4, 256, 512, 0, 2, 1),   # no layers
           pw.ModelDesc(1, 300, 256, 512, 0, 2, 1)]  # E > 256
    for d in bad:
        assert L.pw_create(ctypes.byref(h), 0, ctypes.byref(d)) == pw.PW_ERR_INVALID
    assert L.pw_create(None, 0, None) == pw.PW_ERR_INVALID


def test_null_context_calls_are_invalid():
    L = pw.lib()
    assert L.pw_route_topk(None, None, 1, None, None, None) == pw.PW_ERR_INVALID
    assert L.pw_permute_by_expert(None, None, 1, None, None, None) == pw.PW_ERR_INVALID
    assert L.pw_route_permute(None, None, 1, None, None, None, None, None) == pw.PW_ERR_INVALID
    assert L.pw_moe_ffn_bitplane(None, 0, None, 1, None, None, None, None, None, None, 0, None) == pw.PW_ERR_INVALID
    assert L.pw_moe_layer(None, 0, None, None, 1, None, None, None, None, None, None, 0, None) == pw.PW_ERR_INVALID
    assert L.pw_request_widths(None, 0, None, None, None) == pw.PW_ERR_INVALID
    assert L.pw_commit_ready(None, None, None) == pw.PW_ERR_INVALID
    assert L.pw_block_state(None, 0, None, None, None) == pw.PW_ERR_INVALID
    assert L.pw_routing_mass_enable(None, 1) == pw.PW_ERR_INVALID
    assert L.pw_routing_mass_reset(None, None) == pw.PW_ERR_INVALID
    assert L.pw_routing_mass_read(None, None, None) == pw.PW_ERR_INVALID
    assert L.pw_plan_widths(1, 1, 32, 32, None, None, None, None, 0, None, None) == pw.PW_ERR_INVALID
    assert L.pw_set_committed_bits(None, 1, None, None, None, None) == pw.PW_ERR_INVALID
    assert L.pw_set_tokens_per_pass(None, 8) == pw.PW_ERR_INVALID
    assert L.pw_destroy(None) == pw.PW_OK
    assert L.pw_workspace_size(None, 4) == 0
    assert L.pw_block_id(None, 0, 0, 0) == -1


# (T, top_k, E, I_shared) -> tokens per decode pass, each worked by hand from
# the rule the header states: the largest expected unit m is T for a shared
# expert, else a + 2 sqrt(a) with a = T top_k / E; the width is the smallest of
# 8, 16, 32 with m <= width; 0 outside the decode path.
@pytest.mark.parametrize("T,k,E,Is,want", [
    (1, 2, 8, 0, 8),        # a = 0.25, m = 1.25
    (16, 2, 8, 0, 8),       # a = 4, m = 4 + 4 = 8 (boundary: covered)
    (24, 2, 8, 0, 16),      # a = 6, m = 6 + 4.90 = 10.90
    (32, 2, 8, 0, 16),      # a = 8, m = 8 + 5.66 = 13.66
    (40, 2, 8, 0, 32),      # a = 10, m = 10 + 6.32 = 16.32
    (255, 2, 8, 0, 32),     # a = 63.75: several 32-token passes
    (4, 4, 60, 5632, 8),    # shared expert: m = T = 4
    (9, 4, 60, 5632, 16),   # m = 9
    (16, 4, 60, 5632, 16),  # m = 16 (boundary: covered)
    (17, 4, 60, 5632, 32),  # m = 17
    (64, 4, 60, 0, 16),     # no shared expert: a = 4.27, m = 4.27 + 4.13 = 8.40
    (0, 2, 8, 0, 0),
    (256, 2, 8, 0, 0),      # prefill path
    (5, 0, 8, 0, 0),        # invalid top_k
])
def test_decode_tokens_per_pass(T, k, E, Is, want):
    assert pw.decode_tokens_per_pass(T, k, E, Is) == want
