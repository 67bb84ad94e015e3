"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.mark.parametrize("check", pins.FAST_CHECKS, ids=lambda f: f.__name__)
def test_pin(o, check):
    check(o)


def test_page_byte_counts(o):
    """The page's worked example: 4096 x 11008 at G=128 packs into 512 x 11008
    int32 (about 22.5 MB) plus 32 x 11008 fp16 scales (about 0.7 MB), against
    90 MB in fp16 -- about 23 MB in all, a ratio close to 4x; at 2 TB/s about
    45 us against 11.5 us."""
    g = pins._golden("page_byte_counts.json")
    K, N, MB = g["K"], g["N"], g["MB"]
    W = np.zeros((K, N), np.float32)
    packed, s16 = o.quantize_pack(W, g["G"])
    assert list(packed.shape) == g["packed_shape"]
    assert list(s16.shape) == g["scales_shape"]
    assert packed.nbytes == 22_544_384 and s16.nbytes == 704_512
    assert abs(packed.nbytes / MB - g["packed_MB_printed"]) < 0.05
    assert abs(s16.nbytes / MB - g["scales_MB_printed"]) < 0.05
    fp16 = K * N * 2
    assert abs(fp16 / MB - g["fp16_MB_printed"]) < 0.5
    int4 = packed.nbytes + s16.nbytes
    assert abs(int4 / MB - g["int4_plus_scales_MB_printed"]) < 0.5
    assert 3.8 < fp16 / int4 < 4.0
    assert abs(fp16 / 2e12 * 1e6 - g["fp16_us_at_2TBps_printed"]) < 0.5
    assert abs(int4 / 2e12 * 1e6 - g["int4_us_at_2TBps_printed"]) < 0.2


def test_quantize_rejects_nonfinite(o):
    W = np.zeros((128, 4), np.float32)
    W[3, 1] = np.nan
    with pytest.raises(ValueError):
        o.quantize(W)
    W[3, 1] = np.inf
    with pytest.raises(ValueError):
        o.quantize(W)


def test_quantize_rejects_bad_shapes(o):
    with pytest.raises(ValueError):
        o.quantize(np.zeros((100, 4), np.float32))       # K % G != 0


def test_rtn_ties_occur_on_config_weights(o):
    """Exact .5 ties happen on the seeded config weights, so the rounding mode
    is observable: half-away-from-zero would change some nibbles."""
    W = pins.synth.weights(4096, 1024, seed=0)
    u, s16 = o.quantize(W)
    s = np.repeat(np.maximum(np.abs(W.reshape(32, 128, 1024)).max(axis=1)
                             / np.float32(7.0), np.float32(1e-8)), 128, axis=0)
    r = W / s
    ties = np.abs(r - np.trunc(r)) == 0.5
    away = np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -8, 7) + 8
    # every tie is decided to even, never away from zero where they differ
    assert ties.sum() > 0
    assert np.all(((u[ties].astype(np.int64) - 8) % 2) == 0)
    assert np.any(u[ties] != away[ties].astype(np.uint8))
    assert np.array_equal(u[~ties], away[~ties].astype(np.uint8))
