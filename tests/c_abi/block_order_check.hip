// Host-side check of the kernels' work decomposition (built and run by tests/test_block_order_cpu.py):
// for each launch shape, the XCD dealing `attn::xcd_remap` must be a permutation of the workgroup
// ids, and `attn::block_work` must then hand every (split, b*H + h, Q tile) to exactly one
// workgroup.  Prints "ok <cases>" and exits 0, or names the first failing shape and exits 1.
#include <stdio.h>
#include <vector>

#include "attn_common.h"

static int check(int B, int H, int n_qtiles, int n_splits, int inter) {
    attn::Params p{};
    p.B = B;
    p.H = H;
    p.n_qtiles = n_qtiles;
    p.n_splits = n_splits;
    const int group = n_qtiles * n_splits;
    const int n = group * B * H;
    std::vector<int> seen_id(n, 0), seen_work(n, 0);
    for (int bid = 0; bid < n; ++bid) {
        const int blk = attn::xcd_remap(bid, n, group, inter);
        if (blk < 0 || blk >= n || seen_id[blk]++) return 1;
        const attn::BlockWork w = attn::block_work(p, blk);
        if (w.split < 0 || w.split >= n_splits || w.bh < 0 || w.bh >= B * H || w.qt < 0 || w.qt >= n_qtiles)
            return 1;
        // a group's items stay on one XCD (workgroup id mod 8) whenever the groups are dealt
        if (((n / group) & 7) == 0 && (bid & 7) != (w.bh & 7)) return 1;
        if (seen_work[(w.bh * n_qtiles + w.qt) * n_splits + w.split]++) return 1;
    }
    return 0;
}

int main() {
    const int Bs[] = {1, 2, 3, 4, 16, 32}, Hs[] = {1, 2, 8, 12, 32}, Qs[] = {1, 2, 3, 4, 32, 128},
              Ss[] = {1, 2, 5, 64}, Ps[] = {1, 2, 3, 4};
    int cases = 0;
    for (int B : Bs)
        for (int H : Hs)
            for (int Q : Qs)
                for (int S : Ss)
                    for (int P : Ps) {
                        ++cases;
                        if (check(B, H, Q, S, P)) {
                            printf("FAIL B=%d H=%d n_qtiles=%d n_splits=%d interleave=%d\n", B, H, Q, S, P);
                            return 1;
                        }
                    }
    printf("ok %d\n", cases);
    return 0;
}
