"""The seeded input generator: deterministic, and drawing the stated distributions."""
import hashlib

import numpy as np
import torch

from bit_quantized_decode_amd import inputs as I


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_same_seed_same_bytes_different_seed_different_bytes():
    a = I.nvfp4_matrix(0, 0, 64, 128)
    b = I.nvfp4_matrix(0, 0, 64, 128)
    c = I.nvfp4_matrix(0, 1, 64, 128)
    assert sha(a[0]) == sha(b[0]) and sha(a[1]) == sha(b[1])
    assert sha(a[0]) != sha(c[0])
    assert sha(I.activations(1, 2, 3, 32)) == sha(I.activations(1, 2, 3, 32))
    assert sha(I.router_logits(3, 32, 512)) == sha(I.router_logits(3, 32, 512))


def test_code_distribution_is_uniform_over_16_codes():
    codes, _ = I.nvfp4_matrix(0, 0, 1024, 1024)
    nib = np.concatenate([(codes & 15).ravel(), (codes >> 4).ravel()])
    counts = np.bincount(nib, minlength=16)
    expect = nib.size / 16
    assert counts.min() > 0.98 * expect and counts.max() < 1.02 * expect


def test_scales_are_rounded_powers_in_range():
    _, scales = I.nvfp4_matrix(0, 0, 1024, 1024)
    v = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert v.min() >= 2.0 ** -6 and v.max() <= 4.0
    lg = np.log2(v)
    assert -6.05 < lg.mean() + 2.0 < 0.05   # u is uniform on [-6, 2]: mean -2


def test_activations_are_bf16_of_standard_normal():
    x = I.activations(1, 0, 4, 4096)
    v = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert abs(v.mean()) < 0.03 and abs(v.std() - 1.0) < 0.03


def test_router_bias_is_zipf_like():
    logits = I.router_logits(3, 32, 512)
    r = I.generator(3, 0, 4).permutation(512) + 1
    hottest = int(np.argmin(r))
    assert np.argmax(logits.mean(axis=0)) == hottest
