"""Host generator properties (CPU only): determinism, independence from the
partition, the distributions the workloads ask for, truncation and
injection."""
import numpy as np
import pytest

from sharded_mixed_precision_zs_amd import synth


def test_index_addressable_and_deterministic():
    wl = synth.WORKLOADS["gpt2s-w8"]
    full = synth.host_grad(wl, 3, 2, 0, 1000, 5000)
    win = synth.host_grad(wl, 3, 2, 0, 3000, 100)
    np.testing.assert_array_equal(full[2000:2100], win)
    np.testing.assert_array_equal(full, synth.host_grad(wl, 3, 2, 0, 1000, 5000))
    # different worker / step / micro-batch give different streams
    assert not np.array_equal(full, synth.host_grad(wl, 4, 2, 0, 1000, 5000))
    assert not np.array_equal(full, synth.host_grad(wl, 3, 3, 0, 1000, 5000))
    assert not np.array_equal(full, synth.host_grad(wl, 3, 2, 1, 1000, 5000))


@pytest.mark.parametrize("sigma", [1e-3, 0.02, 1e-4])
def test_normal_moments(sigma):
    k = synth.key(5, synth.STREAM_MASTER)
    x = synth.normal_f32(k, 0, 1 << 20, synth.ks_normal(sigma)).astype(np.float64)
    assert abs(x.mean()) < 5 * sigma / 1024
    assert abs(x.std() / sigma - 1) < 0.01
    # four-term Irwin-Hall: bounded at sqrt(12) sigma, light tails
    assert np.abs(x).max() <= np.sqrt(12.0) * sigma * 1.0001


def test_uniform_range():
    x = synth.uniform_f32(synth.key(1, synth.STREAM_V), 0, 1 << 18, synth.ku_uniform(1e-6))
    assert x.min() >= 0 and x.max() < 1e-6
    assert abs(x.mean() / 5e-7 - 1) < 0.01


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP16])
def test_sixteen_bit_values_truncate_toward_zero(dtype):
    ks = synth.ks_normal(1e-3, 1024.0)
    k = synth.key(0, synth.STREAM_GRAD, 1, 1, 0)
    bits = synth.grad16(k, 0, 0, 0, 1 << 16, ks, dtype)
    x32 = synth.normal_f32(k, 0, 1 << 16, ks)
    x16 = (bits.view(np.float16).astype(np.float32) if dtype == synth.FP16 else
           (bits.astype(np.uint32) << 16).view(np.float32))
    assert np.all(np.abs(x16) <= np.abs(x32))
    assert np.all(np.sign(x16) * np.sign(x32) >= 0)
    # within one 16-bit step below |x|
    step = np.spacing(np.abs(x16).astype(np.float16)).astype(np.float32) if dtype == synth.FP16 \
        else np.abs(x16) * 2.0 ** -7
    assert np.all(np.abs(x32) - np.abs(x16) <= np.maximum(step, 2.0 ** -24))


def test_injection_rate_and_kinds():
    wl = synth.WORKLOADS["1p3b-w4-acc4-fp16"]
    n = 1 << 22
    clean = synth.host_grad(wl, 0, 2, 1, 0, n, scale=2.0 ** 16)
    assert np.all(np.isfinite(clean.view(np.float16)))
    hit = synth.host_grad(wl, 0, 3, 1, 0, n, scale=2.0 ** 16)
    bad = ~np.isfinite(hit.view(np.float16))
    assert abs(bad.mean() / 1e-3 - 1) < 0.05
    kinds = hit[bad]
    assert set(np.unique(kinds)) <= {0x7C00, 0xFC00, 0x7E00}
    assert len(set(np.unique(kinds))) == 3
    # outside the injected positions the values equal the clean stream's
    # generator at that step (injection only replaces)
    assert np.all(np.isfinite(hit[~bad].view(np.float16)))


def test_workload_shapes():
    W = synth.WORKLOADS
    assert W["mlp9-w3"].n == 349_526 and sum(W["mlp9-w3"].tensors) == 2 ** 20
    assert W["gpt2s-w8"].n == 15_554_976
    assert W["7p5b-shard-w64"].n == 117_187_500
    assert W["7b-full-w1"].n == 7_000_000_000
    assert W["1p3b-w4-acc4-fp16"].n == 325_000_000
    assert W["7b-full-w1"].bytes_per_param() == (14, 14)
    assert W["7p5b-shard-w64"].bytes_per_param() == (140, 14)
    assert W["1p3b-w4-acc4-fp16"].bytes_per_param() == (56, 26)
