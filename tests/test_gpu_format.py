"""GPU format kernels against the oracle, bit for bit: quantize+pack, the
repack / unrepack bijection, and dequantization."""
import numpy as np
import pytest

from gpuhelp import orc, say, to_dev, torch
from weight_only_int4_03_amd import synth, w4a16

pytestmark = pytest.mark.gpu

SMALL = [(128, 8), (256, 40), (4096, 4096), (11008, 264), (384, 4104), (1024, 4160)]


@pytest.mark.parametrize("K,N", SMALL)
def test_pack_device_bit_exact(K, N):
    say("pack K=%d N=%d" % (K, N))
    W = synth.weights(K, N, seed=K * 3 + N)
    packed, scales = w4a16.pack(to_dev(W))
    po, so = orc().quantize_pack(W)
    assert np.array_equal(packed.cpu().numpy(), po)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), so)


def test_pack_device_ties_zero_groups_and_grid():
    W = synth.grid_weights(512, 48, p=5, seed=2)
    W[:, 7] = 0.0
    col = np.zeros(128, np.float32)
    col[0] = 7.0
    col[1:9] = [2.5, -2.5, 0.5, -0.5, 1.5, 3.5, 6.5, -6.5]
    W[128:256, 9] = col
    packed, scales = w4a16.pack(to_dev(W))
    po, so = orc().quantize_pack(W)
    assert np.array_equal(packed.cpu().numpy(), po)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), so)


@pytest.mark.parametrize("K,N", SMALL)
def test_repack_roundtrip_bit_exact(K, N):
    say("repack K=%d N=%d" % (K, N))
    packed, scales = synth.random_words(K, N, seed=K + N)   # every nibble value 0..15
    w = w4a16.repack(to_dev(packed), to_dev(scales.view(np.int16)))
    p2, s2 = w4a16.unrepack(w)
    assert np.array_equal(p2.cpu().numpy(), packed)
    assert np.array_equal(s2.cpu().numpy().view(np.uint16), scales)


@pytest.mark.parametrize("K,N", SMALL)
def test_dequant_bit_exact(K, N):
    say("dequant K=%d N=%d" % (K, N))
    packed, scales = synth.random_words(K, N, seed=7 * K + N)
    w = w4a16.repack(to_dev(packed), to_dev(scales.view(np.int16)))
    W16 = w4a16.dequant(w).cpu().numpy().view(np.uint16)
    assert np.array_equal(W16, orc().dequant(packed, scales))


@pytest.mark.parametrize("K,N", SMALL)
def test_dequant_bf16_bit_exact(K, N):
    """bf16 dequantization (the bf16 reading of the data contract's
    dequantize) is bit-exact with the oracle, every nibble value and random
    fp16 scales included."""
    say("dequant bf16 K=%d N=%d" % (K, N))
    packed, scales = synth.random_words(K, N, seed=5 * K + N)
    w = w4a16.repack(to_dev(packed), to_dev(scales.view(np.int16)))
    Wb = w4a16.dequant(w, bf16=True).view(torch().int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(Wb, orc().dequant_bf16(packed, scales))


@pytest.mark.parametrize("K,N", [(8192, 57344), (28672, 8192)])
def test_pack_and_dequant_full_size_sampled_columns(K, N):
    """Largest config weights: device pack, repack and dequant at full size,
    checked bit for bit on 256 sampled columns (the quantizer is per column)."""
    say("full-size pack K=%d N=%d" % (K, N))
    W = synth.weights(K, N, seed=0)
    Wd = to_dev(W)
    packed, scales = w4a16.pack(Wd)
    del Wd
    w = w4a16.repack(packed, scales)
    rng = np.random.default_rng(1)
    cols = np.sort(np.concatenate([[0, N - 1], rng.choice(np.arange(1, N - 1), 254, replace=False)]))
    po, so = orc().quantize_pack(np.ascontiguousarray(W[:, cols]))
    idx = torch().from_numpy(cols).cuda()
    assert np.array_equal(packed.index_select(1, idx).cpu().numpy(), po)
    assert np.array_equal(scales.index_select(1, idx).cpu().numpy().view(np.uint16), so)
    W16 = w4a16.dequant(w).index_select(1, idx).cpu().numpy().view(np.uint16)
    assert np.array_equal(W16, orc().dequant(po, so))
    Wb = w4a16.dequant(w, bf16=True).index_select(1, idx).view(torch().int16).cpu().numpy()
    assert np.array_equal(Wb.view(np.uint16), orc().dequant_bf16(po, so))
    p2, s2 = w4a16.unrepack(w)
    assert torch().equal(p2, packed) and torch().equal(s2, scales)


GROUPS = [(32, 1024, 264), (64, 2048, 1088), (256, 4096, 512), (1152, 1152, 328), (2048, 2048, 96)]


@pytest.mark.parametrize("G,K,N", GROUPS)
def test_other_group_sizes_format_bit_exact(G, K, N):
    """G = 32, 64, 256 and channelwise (G = K, also not a power of two):
    device pack, repack / unrepack and fp16 / bf16 dequantization, bit for bit."""
    say("group G=%d K=%d N=%d" % (G, K, N))
    W = synth.weights(K, N, seed=G + K + N)
    packed, scales = w4a16.pack(to_dev(W), G)
    po, so = orc().quantize_pack(W, G)
    assert np.array_equal(packed.cpu().numpy(), po)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), so)
    w = w4a16.repack(packed, scales, G)
    p2, s2 = w4a16.unrepack(w)
    assert torch().equal(p2, packed) and torch().equal(s2, scales)
    W16 = w4a16.dequant(w).cpu().numpy().view(np.uint16)
    assert np.array_equal(W16, orc().dequant(po, so, G))
    Wb = w4a16.dequant(w, bf16=True).view(torch().int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(Wb, orc().dequant_bf16(po, so, G))
