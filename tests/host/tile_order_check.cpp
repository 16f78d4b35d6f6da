// Host check of the work-group -> tile mapping: for every shape given on the
// command line, each tile must be produced by exactly one work-group id.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tile_order.h"

int main(int argc, char **argv) {
    int bad = 0;
    for (int a = 1; a + 2 < argc; a += 3) {
        const int tm_count = atoi(argv[a]), tn_count = atoi(argv[a + 1]), group = atoi(argv[a + 2]);
        std::vector<int> seen((size_t)tm_count * tn_count, 0);
        for (int pid = 0; pid < tm_count * tn_count; ++pid) {
            int tm = -1, tn = -1;
            sgemm::tile_order(pid, tm_count, tn_count, group, &tm, &tn);
            if (tm < 0 || tm >= tm_count || tn < 0 || tn >= tn_count) {
                printf("out of range: shape %dx%d group %d pid %d -> (%d,%d)\n", tm_count,
                       tn_count, group, pid, tm, tn);
                ++bad;
                continue;
            }
            seen[(size_t)tm * tn_count + tn]++;
        }
        for (size_t t = 0; t < seen.size(); ++t)
            if (seen[t] != 1) {
                printf("tile %zu of %dx%d group %d seen %d times\n", t, tm_count, tn_count, group,
                       seen[t]);
                ++bad;
            }
    }
    printf("%s\n", bad ? "FAIL" : "OK");
    return bad ? 1 : 0;
}
