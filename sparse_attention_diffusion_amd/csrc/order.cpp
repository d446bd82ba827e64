// Locality-preserving token order: positions of grid tokens along a Hilbert
// curve, computed on the host once per grid shape.
//
// Method: the HilbertA blog page (blogs.edgentiq.com, "optimizing image
// generation: HilbertA's efficient sparse attention for diffusion models"),
// section "Introducing HilbertA" (tokens reordered along a Hilbert curve so
// that grid neighbours stay close in the sequence) and section "Future
// Directions" (a three-dimensional curve for video).  The page gives no
// construction.  This library uses the standard n-dimensional Hilbert curve on
// the smallest 2^k cube enclosing the grid, with the index computed by
// Skilling's transform (J. Skilling, "Programming the Hilbert curve", AIP
// Conf. Proc. 707, 2004), and orders the grid's points by that index.
#include <stdint.h>

#include <algorithm>
#include <utility>
#include <vector>

namespace rettn {

namespace {

// Index of point p (n axes, each < 2^bits) along the Hilbert curve of the
// 2^bits cube.  Axis 0 is the most significant within every level.
uint64_t hilbert_key(uint32_t* p, int n, int bits) {
  if (bits == 0) return 0;
  // Levels from the top: where axis i's bit is set, reflect axis 0's lower
  // bits; where it is clear, exchange the lower bits of axes 0 and i.
  for (uint32_t top = 1u << (bits - 1); top > 1; top >>= 1) {
    const uint32_t below = top - 1;
    for (int i = 0; i < n; ++i) {
      if (p[i] & top) {
        p[0] ^= below;
      } else {
        const uint32_t diff = (p[0] ^ p[i]) & below;
        p[0] ^= diff;
        p[i] ^= diff;
      }
    }
  }
  // Gray decode across the axes, then across the levels.
  for (int i = 1; i < n; ++i) p[i] ^= p[i - 1];
  uint32_t mask = 0;
  for (uint32_t top = 1u << (bits - 1); top > 1; top >>= 1)
    if (p[n - 1] & top) mask ^= top - 1;
  for (int i = 0; i < n; ++i) p[i] ^= mask;
  uint64_t key = 0;
  for (int b = bits - 1; b >= 0; --b)
    for (int i = 0; i < n; ++i) key = (key << 1) | ((p[i] >> b) & 1u);
  return key;
}

}  // namespace

// perm[0..n_text) = identity; perm[n_text + r] = n_text + (raster index of the
// grid point with the r-th smallest Hilbert key).  dims: slowest axis first.
void hilbert_order(const int32_t* dims, int ndims, int n_text, int32_t* perm) {
  int bits = 0;
  for (int a = 0; a < ndims; ++a)
    while ((int64_t)dims[a] > ((int64_t)1 << bits)) ++bits;
  int64_t count = 1;
  for (int a = 0; a < ndims; ++a) count *= dims[a];
  std::vector<std::pair<uint64_t, int32_t>> keyed((size_t)count);
  for (int64_t r = 0; r < count; ++r) {
    uint32_t p[3];
    int64_t rest = r;
    for (int a = ndims - 1; a >= 0; --a) {  // raster: the last axis varies fastest
      p[a] = (uint32_t)(rest % dims[a]);
      rest /= dims[a];
    }
    keyed[(size_t)r] = {hilbert_key(p, ndims, bits), (int32_t)r};
  }
  std::sort(keyed.begin(), keyed.end());  // keys are distinct
  for (int i = 0; i < n_text; ++i) perm[i] = i;
  for (int64_t r = 0; r < count; ++r) perm[n_text + r] = n_text + keyed[(size_t)r].second;
}

}  // namespace rettn
