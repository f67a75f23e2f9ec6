// Host check that dg::xcd_remap (the workgroup placement every kernel applies) is a bijection
// of [0, n) for grid sizes up to 4096 and XCD counts 1 to 16, and that it keeps the order of
// grids that do not divide evenly; likewise for dg::full_first (the rel-pos windows' dispatch
// order).  Built and run by tests/test_plan.py; prints "ok".
#include <cstdio>
#include <vector>

#include "../gqa_flash_attention_dg_amd/csrc/dg_common.hpp"

int main() {
    for (int nx = 1; nx <= 16; ++nx) {
        for (int n = 1; n <= 4096; ++n) {
            std::vector<int> seen(n, 0);
            for (int b = 0; b < n; ++b) {
                const int l = dg::xcd_remap(b, n, nx);
                if (l < 0 || l >= n || seen[l]++) {
                    std::printf("not a bijection: n %d nxcd %d bid %d -> %d\n", n, nx, b, l);
                    return 1;
                }
                if (n % nx != 0 && l != b) {
                    std::printf("uneven grid reordered: n %d nxcd %d\n", n, nx);
                    return 1;
                }
                // workgroup b runs on XCD b % nx; logical ids of one XCD are contiguous
                if (n % nx == 0 && l / (n / nx) != b % nx) {
                    std::printf("wrong XCD block: n %d nxcd %d bid %d -> %d\n", n, nx, b, l);
                    return 1;
                }
            }
        }
    }
    // dg::full_first: a bijection that keeps every id on its XCD and, within an XCD's
    // dispatch order, gives every even (full) id before any odd one
    for (int nx = 1; nx <= 16; ++nx) {
        for (int n = 1; n <= 4096; ++n) {
            std::vector<int> seen(n, 0);
            const int m = n % nx == 0 ? n / nx : 0;
            for (int l = 0; l < n; ++l) {
                const int p = dg::full_first(l, n, nx);
                if (p < 0 || p >= n || seen[p]++) {
                    std::printf("full_first not a bijection: n %d nxcd %d id %d -> %d\n", n, nx, l, p);
                    return 1;
                }
                if (m == 0) {
                    if (p != l) { std::printf("full_first moved an uneven grid\n"); return 1; }
                    continue;
                }
                if (p / m != l / m) { std::printf("full_first left the XCD: n %d nxcd %d\n", n, nx); return 1; }
                if (l % m > 0) {
                    const int prev = dg::full_first(l - 1, n, nx);
                    if ((prev & 1) > (p & 1)) {
                        std::printf("full_first order: n %d nxcd %d id %d\n", n, nx, l);
                        return 1;
                    }
                }
            }
        }
    }
    std::printf("ok\n");
    return 0;
}
