// Brute-force check of the C ABI's overlap analysis (csrc/layout.h).
//
// Random small strided layouts are expanded into their element sets; then
//   - rows_disjoint(L) may only be true if L addresses no element twice
//     (it is a sufficient test: nested strides),
//   - may_overlap(a, b) must be true whenever the sets intersect, and must be
//     exactly the intersection test when a and b have equal strides and
//     neither addresses an element twice (the exact path of the analysis).
// Exits nonzero on the first disagreement.  Built with g++ and sanitizers by
// tests/test_capi_host.py.
#include <stdint.h>
#include <stdio.h>

#include <random>
#include <set>
#include <vector>

#include "layout.h"

using namespace rgg;

struct Spec {
    int nd;
    int64_t n[3], st[3], width, base;  // base in elements
};

static std::vector<int64_t> elements(const Spec &s)
{
    std::vector<int64_t> out;
    int64_t n0 = s.nd > 0 ? s.n[0] : 1, n1 = s.nd > 1 ? s.n[1] : 1, n2 = s.nd > 2 ? s.n[2] : 1;
    for (int64_t i = 0; i < n0; ++i)
        for (int64_t j = 0; j < n1; ++j)
            for (int64_t k = 0; k < n2; ++k)
                for (int64_t c = 0; c < s.width; ++c)
                    out.push_back(s.base + i * (s.nd > 0 ? s.st[0] : 0) +
                                  j * (s.nd > 1 ? s.st[1] : 0) + k * (s.nd > 2 ? s.st[2] : 0) + c);
    return out;
}

static Layout to_layout(const Spec &s)
{
    return make_layout(reinterpret_cast<const void *>((uintptr_t)(4096 + 2 * s.base)), 2, s.nd,
                       s.n, s.st, s.width);
}

int main()
{
    std::mt19937_64 rng(12345);
    auto U = [&](int64_t lo, int64_t hi) {
        return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
    };
    long exact_cases = 0, overlap_cases = 0;
    for (int iter = 0; iter < 200000; ++iter) {
        Spec a;
        a.nd = (int)U(1, 3);
        a.width = U(1, 6);
        bool nested = U(0, 1);
        int64_t reach = a.width;
        for (int k = 0; k < a.nd; ++k) {
            a.n[k] = U(1, 4);
            a.st[k] = nested ? reach + U(0, 5) : U(0, 24);
            reach = a.st[k] * (a.n[k] - 1) + reach;
        }
        for (int k = a.nd; k < 3; ++k) {
            a.n[k] = 1;
            a.st[k] = 0;
        }
        a.base = U(0, 40);
        Spec b = a;
        b.base = U(0, 60);
        if (U(0, 3) == 0) {
            b.width = U(1, 6);
            for (int k = 0; k < a.nd; ++k)
                b.n[k] = U(1, 4);
        }
        if (U(0, 4) == 0)
            for (int k = 0; k < b.nd; ++k)
                b.st[k] = U(0, 24);

        std::vector<int64_t> ea = elements(a), eb = elements(b);
        std::set<int64_t> sa(ea.begin(), ea.end()), sb(eb.begin(), eb.end());
        bool dup_a = sa.size() != ea.size();
        bool inter = false;
        for (int64_t e : sb)
            if (sa.count(e)) {
                inter = true;
                break;
            }
        Layout la = to_layout(a), lb = to_layout(b);
        if (rows_disjoint(la) && dup_a) {
            printf("rows_disjoint wrong at iter %d\n", iter);
            return 1;
        }
        bool mo = may_overlap(la, lb);
        if (inter && !mo) {
            printf("missed overlap at iter %d\n", iter);
            return 1;
        }
        bool same = true;
        for (int k = 0; k < 3; ++k)
            same &= la.st[k] == lb.st[k] || (la.n[k] == 1 && lb.n[k] == 1);
        same &= la.nd == lb.nd;
        if (same && rows_disjoint(la) && rows_disjoint(lb)) {
            ++exact_cases;
            if (mo != inter) {
                printf("inexact answer at iter %d (said %d, truth %d)\n", iter, mo, inter);
                return 1;
            }
        }
        overlap_cases += inter;
    }
    printf("ok: %ld exact-path cases, %ld overlapping pairs\n", exact_cases, overlap_cases);
    return 0;
}
