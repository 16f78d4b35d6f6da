// Host check of the element index of the one-element-per-work-item rungs.
//   element_index_check at BLOCK TILES_N TILE_M TILE_N TX TY
//       prints the row and column that work-item (TX, TY) of work-group BLOCK owns.
//   element_index_check cover M N TILE_M TILE_N
//       checks that a grid of ceil(M/TILE_M) * ceil(N/TILE_N) work-groups of
//       TILE_N x TILE_M work-items owns every element of an M x N matrix once
//       (work-items past the edge own elements outside it); prints OK or FAIL.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "tile_order.h"

int main(int argc, char **argv) {
    if (argc == 8 && strcmp(argv[1], "at") == 0) {
        int row = -1, col = -1;
        sgemm::element_of(atoi(argv[2]), atoi(argv[3]), atoi(argv[4]), atoi(argv[5]),
                          atoi(argv[6]), atoi(argv[7]), &row, &col);
        printf("%d %d\n", row, col);
        return 0;
    }
    if (argc == 6 && strcmp(argv[1], "cover") == 0) {
        const int M = atoi(argv[2]), N = atoi(argv[3]), tm = atoi(argv[4]), tn = atoi(argv[5]);
        const int tiles_m = (M + tm - 1) / tm, tiles_n = (N + tn - 1) / tn;
        std::vector<int> seen((size_t)M * N, 0);
        int bad = 0;
        for (int b = 0; b < tiles_m * tiles_n; ++b)
            for (int ty = 0; ty < tm; ++ty)
                for (int tx = 0; tx < tn; ++tx) {
                    int row, col;
                    sgemm::element_of(b, tiles_n, tm, tn, tx, ty, &row, &col);
                    if (row < 0 || col < 0) ++bad;
                    else if (row < M && col < N) seen[(size_t)row * N + col]++;
                }
        for (size_t e = 0; e < seen.size(); ++e)
            if (seen[e] != 1) ++bad;
        printf("%s\n", bad ? "FAIL" : "OK");
        return bad ? 1 : 0;
    }
    fprintf(stderr, "usage: at BLOCK TILES_N TILE_M TILE_N TX TY | cover M N TILE_M TILE_N\n");
    return 2;
}
