"""Pins of the Hilbert token-order oracle against facts outside it.

Each pin takes the oracle module and returns None when it holds, or a short
message.  Facts used:
* the order-1 and order-2 two-dimensional Hilbert curves as drawn in every
  textbook (Hilbert 1891): four points in a U, then four U's joined end to end;
* continuity: consecutive positions are grid neighbours (one unit step);
* self-similarity: every aligned run of 2^(n j) positions fills one aligned
  cube of side 2^j;
* the curve starts at the origin and ends at a corner one axis away from it;
* a reorder followed by its inverse is the identity.
"""
import itertools

import numpy as np

ORDER2_2D = [(0, 0), (1, 0), (1, 1), (0, 1), (0, 2), (0, 3), (1, 3), (1, 2),
             (2, 2), (2, 3), (3, 3), (3, 2), (3, 1), (2, 1), (2, 0), (3, 0)]


def _curve(h, n, k):
    pts = list(itertools.product(range(1 << k), repeat=n))
    by_index = {}
    for p in pts:
        i = h.hilbert_index(p, k)
        if i in by_index or not 0 <= i < len(pts):
            return None
        by_index[i] = p
    return [by_index[i] for i in range(len(pts))]


def pin_textbook_2d(h):
    c1, c2 = _curve(h, 2, 1), _curve(h, 2, 2)
    if c1 != [(0, 0), (0, 1), (1, 1), (1, 0)]:
        return f"order-1 curve {c1}"
    if c2 != ORDER2_2D:
        return f"order-2 curve {c2}"
    return None


def pin_bijective_and_continuous(h):
    for n, k in ((2, 1), (2, 3), (2, 5), (3, 1), (3, 2), (3, 3), (1, 4)):
        c = _curve(h, n, k)
        if c is None:
            return f"n={n} k={k}: not a bijection onto [0, 2^(nk))"
        for a, b in zip(c, c[1:]):
            if sum(abs(x - y) for x, y in zip(a, b)) != 1:
                return f"n={n} k={k}: step {a} -> {b} is not a unit step"
    return None


def pin_nested_cubes(h):
    for n, k in ((2, 4), (3, 3)):
        c = np.array(_curve(h, n, k))
        for j in range(1, k):
            run = 1 << (n * j)
            for s in range(0, len(c), run):
                blk = c[s: s + run]
                lo = blk.min(axis=0)
                if (blk.max(axis=0) - lo + 1 != (1 << j)).any() or (lo % (1 << j)).any():
                    return f"n={n} k={k}: run at {s} of length {run} is not an aligned cube"
    return None


def pin_endpoints(h):
    for n, k in ((2, 3), (3, 3), (3, 2)):
        c = _curve(h, n, k)
        last = np.array(c[-1])
        if c[0] != (0,) * n or sorted(last.tolist()) != [0] * (n - 1) + [(1 << k) - 1]:
            return f"n={n} k={k}: ends {c[0]} .. {c[-1]}"
    return None


def pin_token_order(h):
    # square image grid: every aligned 64-token block is an 8x8 square
    perm = h.token_order((16, 16), 0)
    if sorted(perm.tolist()) != list(range(256)):
        return "16x16 order is not a permutation"
    ys, xs = np.divmod(perm, 16)
    for s in range(0, 256, 64):
        y, x = ys[s: s + 64], xs[s: s + 64]
        if y.max() - y.min() != 7 or x.max() - x.min() != 7:
            return f"block at {s} is not an 8x8 square"
    # video grid with text first: text unchanged, grid part sorted by index
    dims, n_text = (3, 5, 6), 7
    perm = h.token_order(dims, n_text)
    if sorted(perm.tolist()) != list(range(n_text + 90)) or perm[:n_text].tolist() != list(range(n_text)):
        return "video order: not a permutation with the text first"
    pts = np.array(np.unravel_index(perm[n_text:] - n_text, dims)).T
    keys = [h.hilbert_index(p, 3) for p in pts]
    if any(b <= a for a, b in zip(keys, keys[1:])):
        return "video order: indices not increasing"
    return None


def pin_permute_round_trip(h):
    rng = np.random.default_rng(3)
    x = rng.normal(size=(2, 3, 97, 5))
    perm = h.token_order((4, 5, 4), 17)
    y = h.permute_rows(x, perm)
    if not np.array_equal(y[..., 20, :], x[..., perm[20], :]):
        return "gather does not place row perm[i] at i"
    if not np.array_equal(h.permute_rows(y, perm, inverse=True), x):
        return "inverse of the reorder is not the identity"
    return None


ALL = [pin_textbook_2d, pin_bijective_and_continuous, pin_nested_cubes, pin_endpoints, pin_token_order,
       pin_permute_round_trip]


def failing(h):
    out = []
    for p in ALL:
        try:
            msg = p(h)
        except Exception as e:  # a crash counts as a failure
            msg = f"raised {type(e).__name__}: {e}"
        if msg:
            out.append((p.__name__, msg))
    return out
