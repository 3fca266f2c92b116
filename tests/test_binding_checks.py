"""The Python binding checks what the C ABI cannot see (dtype, element count, device, contiguity)
and raises before anything reaches the library, so a wrong tensor never becomes an out-of-bounds
device access.  CPU only: every case here is rejected before the library is called."""

import pytest
import torch

import kv_cache_compression_pass_amd as kvc


def _desc():
    return kvc.make_desc(4, 2, 64, 128, 64, True)


def _good():
    # correct dtypes and sizes, but host tensors: the device check is the last one made
    return dict(q=torch.zeros(4, 64, 64, dtype=torch.bfloat16), k=torch.zeros(2, 128, 64, dtype=torch.bfloat16),
                lse=torch.zeros(4, 64, dtype=torch.float32))


def test_wrong_dtype_is_rejected():
    a = _good()
    with pytest.raises(ValueError, match="q: dtype torch.float32"):
        kvc.kvc_row_lse(_desc(), a["q"].float(), a["k"], a["lse"])


def test_wrong_size_is_rejected():
    a = _good()
    with pytest.raises(ValueError, match="k: 8000 elements, expected 16384"):
        kvc.kvc_row_lse(_desc(), a["q"], a["k"].flatten()[:8000], a["lse"])
    with pytest.raises(ValueError, match="scores: 100 elements, expected 256"):
        kvc.kvc_score_tokens(_desc(), kvc.SCORE_SUM, a["q"], a["k"], a["lse"], torch.zeros(100), None)


def test_host_tensor_is_rejected():
    a = _good()
    with pytest.raises(ValueError, match="expected a GPU tensor"):
        kvc.kvc_row_lse(_desc(), a["q"], a["k"], a["lse"])


def test_non_contiguous_is_rejected():
    a = _good()
    qt = torch.zeros(4, 64, 64, dtype=torch.bfloat16).transpose(1, 2)
    with pytest.raises(ValueError, match="contiguous"):
        kvc.kvc_row_lse(_desc(), qt, a["k"], a["lse"])


def test_not_a_tensor_is_rejected():
    a = _good()
    with pytest.raises(TypeError):
        kvc.kvc_row_lse(_desc(), 12345, a["k"], a["lse"])


def test_allocation_shapes_follow_the_stage():
    d = _desc()
    w_tok = torch.zeros(2, 128)
    w_ch = torch.zeros(2, 64)
    # the K stage needs the channel weights [H_kv][d] and bits_v [H_kv][N]
    with pytest.raises(ValueError, match="weight: 256 elements, expected 128"):
        kvc.kvc_allocate_bits(d, kvc.ALLOC_K_CHANNELS, w_tok, torch.zeros(2, 64, dtype=torch.uint8), None)
    with pytest.raises(ValueError, match="bits_v: a tensor is required"):
        kvc.kvc_allocate_bits(d, kvc.ALLOC_K_CHANNELS, w_ch, torch.zeros(2, 64, dtype=torch.uint8), None)
    with pytest.raises(ValueError, match="bits_out: dtype torch.float32"):
        kvc.kvc_allocate_bits(d, kvc.ALLOC_V_TOKENS, w_tok, torch.zeros(2, 128), None)


def test_append_buffers_must_match():
    d = _desc()
    kn = torch.zeros(2, 10, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="give both or neither"):
        kvc.kvc_compressed_attend_append(d, None, None, kn, None, None, None, None)
    with pytest.raises(ValueError, match="expected \\[2\\]\\[n_new\\]\\[64\\] both"):
        kvc.kvc_compressed_attend_append(d, None, None, kn, torch.zeros(2, 9, 64, dtype=torch.bfloat16), None, None,
                                         None)


def test_ridge_sizes_follow_the_split():
    # n_keys = n_c + m: with n_c = 100 of 128 keys, v_r holds the other 28 tokens
    d = kvc.make_desc(4, 2, 64, 128, 64, False)
    q = torch.zeros(4, 64, 64, dtype=torch.bfloat16)
    k = torch.zeros(2, 128, 64, dtype=torch.bfloat16)
    y = torch.zeros(4, 64, 64)
    with pytest.raises(ValueError, match="v_r: a tensor is required"):
        kvc.kvc_ridge_value_fit(d, 100, q, k, None, y, 0.1, torch.zeros(2, 100, 64), None)
    with pytest.raises(ValueError, match="v_r: 3456 elements, expected 3584"):
        kvc.kvc_ridge_value_fit(d, 100, q, k, torch.zeros(2, 27, 64, dtype=torch.bfloat16), y, 0.1,
                                torch.zeros(2, 100, 64), None)
