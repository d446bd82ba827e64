"""Plain reference for a Hilbert-curve token order before 64-token blocking.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this module.  It shares no code with the library.

Source: the HilbertA blog page (blogs.edgentiq.com, "optimizing image
generation: HilbertA's efficient sparse attention for diffusion models").
Section "Introducing HilbertA": image tokens are reordered along a Hilbert
curve so that tokens that are close on the grid stay close in the 1-D
sequence.  Section "Future Directions": a three-dimensional curve for video.

Reading taken here (the page gives no construction):
* the curve is the standard n-dimensional Hilbert curve on a 2^k cube, with
  its index computed by Skilling's transform (J. Skilling, "Programming the
  Hilbert curve", AIP Conf. Proc. 707, 2004): coordinates are turned into the
  "transposed" index by undoing the curve's rotations and reflections level by
  level, Gray-decoded, and their bits interleaved, most significant level first;
* a grid that is not a 2^k cube is ordered by the indices its points have on
  the smallest enclosing 2^k cube;
* coordinates enter in the grid's axis order, slowest axis first ((y, x) for
  an image, (t, y, x) for a video), and text tokens stay first, in order.
"""
import numpy as np


def hilbert_index(coords, bits):
    """Position along the Hilbert curve of the 2^bits cube of the point
    `coords` (a sequence of n non-negative integers < 2^bits)."""
    x = [int(c) for c in coords]
    n = len(x)
    if bits == 0:
        return 0
    # Undo the per-level rotations/reflections, highest level first.
    q = 1 << (bits - 1)
    while q > 1:
        low = q - 1
        for i in range(n):
            if x[i] & q:
                x[0] ^= low                      # reflect the lower bits of axis 0
            else:
                t = (x[0] ^ x[i]) & low          # swap the lower bits of axes 0 and i
                x[0] ^= t
                x[i] ^= t
        q >>= 1
    # Gray code to binary, across the axes and then across the levels.
    for i in range(1, n):
        x[i] ^= x[i - 1]
    flip = 0
    q = 1 << (bits - 1)
    while q > 1:
        if x[n - 1] & q:
            flip ^= q - 1
        q >>= 1
    for i in range(n):
        x[i] ^= flip
    # Interleave: level by level from the top, axis 0 most significant.
    h = 0
    for b in range(bits - 1, -1, -1):
        for i in range(n):
            h = (h << 1) | ((x[i] >> b) & 1)
    return h


def bits_for(dims):
    """Smallest k with every extent <= 2^k."""
    k = 0
    while any(s > (1 << k) for s in dims):
        k += 1
    return k


def token_order(dims, n_text=0):
    """Permutation of n_text + prod(dims) tokens: text first (unchanged), then
    the grid tokens (raster order, slowest axis first) sorted by Hilbert index.
    perm[i] is the original position of the token placed at position i, so a
    reordered tensor is x[..., perm, :]."""
    dims = tuple(int(s) for s in dims)
    k = bits_for(dims)
    pts = np.array(np.unravel_index(np.arange(int(np.prod(dims))), dims)).T
    keys = np.array([hilbert_index(p, k) for p in pts], dtype=np.int64)
    order = np.argsort(keys, kind="stable")
    return np.concatenate([np.arange(n_text), n_text + order]).astype(np.int32)


def permute_rows(x, perm, inverse=False):
    """Gather x[..., perm[i], :] into row i, or (inverse) scatter row i to
    position perm[i]."""
    x = np.asarray(x)
    if not inverse:
        return x[..., perm, :]
    out = np.empty_like(x)
    out[..., perm, :] = x
    return out
