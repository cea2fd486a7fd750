// Strided element layouts and whether two of them can share an element.
// Host-only C++ (no HIP), used by the C ABI to reject overlapping outputs.
#pragma once

#include <stdint.h>

#include <algorithm>

namespace rgg {

// Elements at base + sum_k i_k * st_k + c (0 <= i_k < n_k, 0 <= c < width),
// every element `esize` bytes.  Dimensions of size 1 are dropped on entry.
struct Layout {
    uintptr_t base = 0;
    int64_t esize = 2;
    int nd = 0;
    int64_t n[3] = {1, 1, 1};
    int64_t st[3] = {0, 0, 0};
    int64_t width = 0;
    bool empty = false;
};

inline Layout make_layout(const void *base, int64_t esize, int nd, const int64_t *n, const int64_t *st,
                   int64_t width)
{
    Layout L;
    L.base = reinterpret_cast<uintptr_t>(base);
    L.esize = esize;
    L.width = width;
    L.empty = width <= 0;
    for (int k = 0; k < nd; ++k) {
        if (n[k] <= 0)
            L.empty = true;
        if (n[k] > 1) {
            L.n[L.nd] = n[k];
            L.st[L.nd] = st[k];
            ++L.nd;
        }
    }
    // innermost (smallest stride) first
    for (int a = 0; a < L.nd; ++a)
        for (int b = a + 1; b < L.nd; ++b)
            if (L.st[b] < L.st[a]) {
                std::swap(L.st[a], L.st[b]);
                std::swap(L.n[a], L.n[b]);
            }
    return L;
}

// Byte range [lo, hi) covered by a non-empty layout (strides are >= 0).
inline void byte_span(const Layout &L, uintptr_t &lo, uintptr_t &hi)
{
    int64_t last = L.width;
    for (int k = 0; k < L.nd; ++k)
        last += (L.n[k] - 1) * L.st[k];
    lo = L.base;
    hi = L.base + (uintptr_t)(last * L.esize);
}

// No two index tuples of L address the same element: with dimensions sorted
// by stride, each stride exceeds everything the dimensions below can reach.
inline bool rows_disjoint(const Layout &L)
{
    if (L.empty)
        return true;
    int64_t reach = L.width;
    for (int k = 0; k < L.nd; ++k) {
        if (L.st[k] < reach)
            return false;
        reach += (L.n[k] - 1) * L.st[k];
    }
    return true;
}

// Is there d_k in [-(nb_k - 1), na_k - 1] for k < level and dc in
// [-(wb - 1), wa - 1] with sum d_k st_k + dc == r?  Exact search over at most
// a few candidates per level; gives up (answers yes) if a level admits more.
inline bool reachable(const Layout &a, const Layout &b, int level, int64_t r)
{
    if (level == 0)
        return r >= -(b.width - 1) && r <= a.width - 1;
    int k = level - 1;
    int64_t lo = -(b.width - 1), hi = a.width - 1;  // what levels below k can add
    for (int m = 0; m < k; ++m) {
        lo -= (b.n[m] - 1) * a.st[m];
        hi += (a.n[m] - 1) * a.st[m];
    }
    int64_t s = a.st[k];
    if (s <= 0)
        return true;
    // d with lo <= r - d*s <= hi  <=>  (r - hi)/s <= d <= (r - lo)/s
    auto floordiv = [](int64_t x, int64_t y) { return x >= 0 ? x / y : -((-x + y - 1) / y); };
    int64_t dmin = -floordiv(-(r - hi), s);  // ceil((r - hi) / s)
    int64_t dmax = floordiv(r - lo, s);
    dmin = std::max(dmin, -(b.n[k] - 1));
    dmax = std::min(dmax, a.n[k] - 1);
    if (dmax - dmin > 4)
        return true;
    for (int64_t d = dmin; d <= dmax; ++d)
        if (reachable(a, b, k, r - d * s))
            return true;
    return false;
}

// May the element sets of a and b intersect?  Exact when both have the same
// element size, dimensions and strides; otherwise by byte range.
inline bool may_overlap(const Layout &a, const Layout &b)
{
    if (a.empty || b.empty)
        return false;
    uintptr_t alo, ahi, blo, bhi;
    byte_span(a, alo, ahi);
    byte_span(b, blo, bhi);
    if (ahi <= blo || bhi <= alo)
        return false;
    bool same = a.esize == b.esize && a.nd == b.nd;
    for (int k = 0; same && k < a.nd; ++k)
        same = a.st[k] == b.st[k];
    if (!same || !rows_disjoint(a) || !rows_disjoint(b))
        return true;
    intptr_t delta = (intptr_t)(b.base - a.base);
    if (delta % a.esize != 0)
        return true;
    return reachable(a, b, a.nd, delta / a.esize);
}

}  // namespace rgg
