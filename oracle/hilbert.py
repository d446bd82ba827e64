"""Plain reference for a Hilbert-curve token order before 64-token blocking.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this module.  It shares no code with the library.

Source: the HilbertA blog page (blogs.edgentiq.com, "optimizing image
generation: HilbertA's efficient sparse attention for diffusion models").
Section "Introducing HilbertA": image tokens are reordered along a Hilbert
curve so that tokens that are close on the grid stay close in the 1-D
sequence.  Section "Future Directions": a three-dimensional curve for video.

Reading taken here (the page gives no construction).  The curve on a cube of
side 2^k in n dimensions (n = 1, 2, 3) is defined by recursion on k:

* Level 1.  The 2^n half-size sub-cubes, labelled by their corner c in
  {0,1}^n, are visited in reflected binary Gray-code order with coordinate
  axis 0 as the most significant digit: c_j = bits of j XOR (j >> 1).
  In 2-D: (0,0) (0,1) (1,1) (1,0); in 3-D: (0,0,0) (0,0,1) (0,1,1) (0,1,0)
  (1,1,0) (1,1,1) (1,0,1) (1,0,0).
* Inside sub-cube j the curve is the whole curve one level smaller, carried
  into the sub-cube by a fixed signed permutation of the axes T_j (table
  CHILD below).  T_j is what makes the pieces join: the curve starts at the
  origin and ends at the corner (side-1, 0, ..., 0); T_j places that start
  next to where piece j-1 ended and that end next to where piece j+1 starts.
* The position of a point is j * (side/2)^n plus the position, on the
  smaller curve, of its offset inside sub-cube j mapped back through T_j.

In 2-D the table is the textbook one (Hilbert 1891): the first quarter is
the curve mirrored in the diagonal, the middle two are unchanged, the last is
mirrored in the anti-diagonal.  In 3-D several curves meet these rules; the
table is the one of the curve that J. Skilling's transform ("Programming the
Hilbert curve", AIP Conf. Proc. 707, 2004) indexes, so that the library's
reorder and this one are two constructions of one curve.  The tests pin the
table by the curve's defining properties (a bijection, unit steps, aligned
sub-cubes, the end points, the textbook 2-D drawings).

A grid that is not a 2^k cube is ordered by the positions its points have on
the smallest enclosing 2^k cube.  Coordinates enter in the grid's axis order,
slowest axis first ((y, x) for an image, (t, y, x) for a video), and text
tokens stay first, in order.
"""
import numpy as np

# CHILD[n][j] = (perm, flip): a point y inside sub-cube j (offsets in
# [0, s) per axis, s = side/2) lies on the smaller curve at the point x with
#   x[a] = y[perm[a]]          if flip[a] == 0
#   x[a] = s - 1 - y[perm[a]]  if flip[a] == 1.
# The comments give where each piece enters and leaves, in units of the
# sub-cube side, on the order-2 curve.
CHILD = {
    1: [((0,), (0,)), ((0,), (0,))],
    2: [
        ((1, 0), (0, 0)),  # (0,0): enters (0,0), leaves (0,1)   mirrored in the diagonal
        ((0, 1), (0, 0)),  # (0,1): enters (0,2), leaves (1,2)   unchanged
        ((0, 1), (0, 0)),  # (1,1): enters (2,2), leaves (3,2)   unchanged
        ((1, 0), (1, 1)),  # (1,0): enters (3,1), leaves (3,0)   mirrored in the anti-diagonal
    ],
    3: [
        ((2, 0, 1), (0, 0, 0)),  # (0,0,0): enters (0,0,0), leaves (0,0,1)
        ((1, 0, 2), (0, 0, 0)),  # (0,0,1): enters (0,0,2), leaves (0,1,2)
        ((0, 1, 2), (0, 0, 0)),  # (0,1,1): enters (0,2,2), leaves (1,2,2)
        ((2, 1, 0), (1, 0, 1)),  # (0,1,0): enters (1,2,1), leaves (1,2,0)
        ((2, 1, 0), (0, 0, 0)),  # (1,1,0): enters (2,2,0), leaves (2,2,1)
        ((0, 1, 2), (0, 0, 0)),  # (1,1,1): enters (2,2,2), leaves (3,2,2)
        ((1, 0, 2), (1, 1, 0)),  # (1,0,1): enters (3,1,2), leaves (3,0,2)
        ((2, 0, 1), (1, 1, 0)),  # (1,0,0): enters (3,0,1), leaves (3,0,0)
    ],
}


def level1_corners(n):
    """Corners of the 2^n sub-cubes in the order the curve visits them."""
    out = []
    for j in range(1 << n):
        g = j ^ (j >> 1)
        out.append(tuple((g >> (n - 1 - a)) & 1 for a in range(n)))
    return out


def hilbert_index(coords, bits):
    """Position along the curve of the 2^bits cube of the point `coords` (a
    sequence of n non-negative integers < 2^bits, n = 1, 2 or 3)."""
    x = tuple(int(c) for c in coords)
    n = len(x)
    if bits == 0:
        return 0
    s = 1 << (bits - 1)                             # side of a sub-cube
    corner = tuple(c // s for c in x)
    j = level1_corners(n).index(corner)             # which piece of the curve
    y = tuple(c - s * h for c, h in zip(x, corner))  # offset inside the sub-cube
    perm, flip = CHILD[n][j]
    back = tuple(s - 1 - y[perm[a]] if flip[a] else y[perm[a]] for a in range(n))
    return j * s ** n + hilbert_index(back, bits - 1)


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
