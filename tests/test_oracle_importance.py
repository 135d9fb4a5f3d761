"""Pins for the oracle's Sobel magnitude and patch pooling (fp32, fixed order)."""
import numpy as np
import pytest
import scipy.ndimage

from oracle import importance, patch_mean, sobel_magnitude


def _brute_sobel(img):
    """Explicit 3x3 correlation with zero padding, one pixel at a time."""
    kx = [[-1, 0, 1], [-2, 0, 2], [-1, 0, 1]]
    ky = [[-1, -2, -1], [0, 0, 0], [1, 2, 1]]
    H, W = img.shape
    out = np.zeros((H, W), np.float32)
    for y in range(H):
        for x in range(W):
            gx = 0.0
            gy = 0.0
            for dy in range(3):
                for dx in range(3):
                    yy, xx = y + dy - 1, x + dx - 1
                    p = float(img[yy, xx]) if (0 <= yy < H and 0 <= xx < W) else 0.0
                    gx += kx[dy][dx] * p
                    gy += ky[dy][dx] * p
            out[y, x] = np.sqrt(np.float32(gx * gx + gy * gy))
    return out


@pytest.mark.parametrize("seed", range(5))
def test_sobel_matches_brute_force_bitwise_on_integer_images(seed):
    # Integer pixels keep every intermediate exact, so any order gives the same bits.
    rng = np.random.default_rng(seed)
    img = rng.integers(0, 256, size=(8, 8)).astype(np.float32)
    got = sobel_magnitude(img)
    want = _brute_sobel(img)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("seed", range(3))
def test_sobel_matches_scipy_on_float_images(seed):
    rng = np.random.default_rng(100 + seed)
    img = rng.normal(0.5, 0.3, size=(37, 53)).astype(np.float32)
    gx = scipy.ndimage.sobel(img.astype(np.float64), axis=1, mode="constant")
    gy = scipy.ndimage.sobel(img.astype(np.float64), axis=0, mode="constant")
    want = np.hypot(gx, gy)
    got = sobel_magnitude(img).astype(np.float64)
    # fp32 rounding of at most ~10 operations on values below 16
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-5)


def test_sobel_on_8x8_brute_force_random_floats_close():
    rng = np.random.default_rng(7)
    img = rng.uniform(-1, 1, size=(8, 8)).astype(np.float32)
    np.testing.assert_allclose(sobel_magnitude(img), _brute_sobel(img), rtol=0, atol=5e-6)


@pytest.mark.parametrize("k", [0, 1, 3, 6])
def test_sobel_ramp_closed_form(k):
    a = np.float32(2.0 ** -k)
    img = (np.arange(32, dtype=np.float32)[None, :] * a).repeat(20, axis=0)
    m = sobel_magnitude(img)
    assert np.all(m[1:-1, 1:-1] == np.float32(8) * a)
    # vertical ramp: same magnitude, the other axis
    m2 = sobel_magnitude(img.T.copy())
    assert np.all(m2[1:-1, 1:-1] == np.float32(8) * a)


def test_sobel_constant_image_interior_zero_border_nonzero():
    img = np.full((10, 12), 0.75, np.float32)
    m = sobel_magnitude(img)
    assert np.all(m[1:-1, 1:-1] == 0)
    # zero padding outside the image gives an edge at the border: corner has gx = gy = 3c
    assert m[0, 0] == np.float32(np.sqrt(np.float32(2 * (3 * 0.75) ** 2)))
    assert m[0, 5] == np.float32(4 * 0.75)  # top edge: gy = 4c, gx = 0


def test_sobel_sign_and_axis_invariance():
    # integer pixels: every intermediate is exact, so mirrored evaluation orders agree bitwise
    rng = np.random.default_rng(3)
    img = rng.integers(-500, 500, size=(16, 16)).astype(np.float32)
    m = sobel_magnitude(img)
    assert np.array_equal(sobel_magnitude(img[:, ::-1].copy()), m[:, ::-1])
    assert np.array_equal(sobel_magnitude(img[::-1, :].copy()), m[::-1, :])
    assert np.array_equal(sobel_magnitude(img.T.copy()), m.T)
    assert np.array_equal(sobel_magnitude(-img), m)


def test_patch_mean_constant_exact():
    mag = np.full((64, 48), 0.3125, np.float32)
    assert np.all(patch_mean(mag, 16) == np.float32(0.3125))


def test_patch_mean_hand_sums():
    mag = np.zeros((32, 32), np.float32)
    mag[0:16, 16:32] = np.arange(256, dtype=np.float32).reshape(16, 16)  # token (0, 1)
    mag[16, 16] = 256.0                                                 # token (1, 1)
    out = patch_mean(mag, 16)
    assert out.shape == (4,)
    assert out[0] == 0
    assert out[1] == np.float32(255 * 256 / 2 / 256)  # sum 0..255 = 32640, / 256
    assert out[2] == 0
    assert out[3] == 1.0


def test_patch_mean_order_and_error_bound():
    rng = np.random.default_rng(11)
    mag = rng.uniform(0, 4, size=(48, 64)).astype(np.float32)
    got = patch_mean(mag, 16).astype(np.float64)
    want = mag.astype(np.float64).reshape(3, 16, 4, 16).mean(axis=(1, 3)).reshape(-1)
    # sequential fp32 sum of 256 terms <= 4: error below 256 * 2^-24 * 1024 / 256
    np.testing.assert_allclose(got, want, rtol=0, atol=256 * 2.0 ** -24 * 4)
    # the fixed order: rows left to right, then row sums top to bottom
    t = mag[0:16, 0:16]
    acc = np.float32(0)
    for r in range(16):
        row = np.float32(0)
        for c in range(16):
            row = np.float32(row + t[r, c])
        acc = np.float32(acc + row)
    assert patch_mean(mag, 16)[0] == np.float32(acc / np.float32(256))


def test_importance_shape_and_token_order():
    img = np.zeros((64, 32), np.float32)
    img[40:44, 20:24] = 1.0  # a small square inside token (2, 1) of a 4 x 2 grid
    imp = importance(img, 16)
    assert imp.shape == (8,)
    assert np.argmax(imp) == 2 * 2 + 1
    assert np.count_nonzero(imp[[0, 1, 2, 3, 4, 6]]) == 0
