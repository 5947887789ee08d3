/* A plain C client of libmedusa, built with the system C compiler against include/medusa.h
 * alone: the boundary needs no C++ or HIP headers on the caller's side.  It exercises the
 * host-only calls (tree plans, the expected accepted length, status strings, argument
 * checks) and prints one line per check; the exit status is the number of failures. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "medusa.h"

static int failures = 0;

static void check(int ok, const char* what) {
    printf("%s %s\n", ok ? "ok  " : "FAIL", what);
    if (!ok) ++failures;
}

int main(void) {
    /* the page's example: top-2 of head 1 by top-3 of head 2 gives a 9-node tree */
    const int32_t s23[2] = {2, 3};
    medusa_tree_plan* full = NULL;
    check(medusa_tree_plan_full(s23, 2, &full) == MEDUSA_OK && full, "plan_full (2,3)");
    int n = 0, d = 0, w = 0;
    check(medusa_tree_plan_info(full, &n, &d, &w) == MEDUSA_OK && n == 9 && d == 2 && w == 1,
          "9 nodes, depth 2, one mask word");
    int32_t parent[9], depth[9], rank[9];
    uint64_t mask[9];
    check(medusa_tree_plan_arrays(full, parent, depth, rank, mask) == MEDUSA_OK, "plan arrays");
    int leaves = 0;
    for (int i = 0; i < n; ++i) {
        int has_child = 0;
        for (int j = 0; j < n; ++j) has_child |= parent[j] == i;
        leaves += !has_child;
    }
    check(leaves == 6, "six leaves");
    check(mask[8] == ((1ull << 0) | (1ull << 2) | (1ull << 8)), "node 8 sees the root, node 2, itself");

    /* expected accepted length: with every accuracy 1/2 at rank 0 and 1/4 at rank 1..2,
     * E[a] = sum over the 8 non-root nodes of the product along the path */
    const double acc[2 * 3] = {0.5, 0.25, 0.0, 0.5, 0.25, 0.25};
    double ea = -1.0;
    check(medusa_tree_plan_expected_accept(full, acc, 3, 2, &ea) == MEDUSA_OK, "expected_accept");
    /* depth 1: 0.5 + 0.25; depth 2: (0.5 + 0.25) * (0.5 + 0.25 + 0.25) */
    check(fabs(ea - (0.75 + 0.75 * 1.0)) < 1e-15, "expected_accept closed form");

    /* a sparse plan of the 4 most accurate combinations is a prefix-closed subset */
    medusa_tree_plan* sparse = NULL;
    check(medusa_tree_plan_from_accuracy(acc, 3, s23, 2, 5, &sparse) == MEDUSA_OK, "plan_from_accuracy");
    check(medusa_tree_plan_info(sparse, &n, &d, &w) == MEDUSA_OK && n == 5, "5 nodes");

    /* malformed input is rejected before anything runs */
    const int32_t one[2] = {1, -1};      /* the path (1,): its prefix is the root */
    const int32_t neg[2] = {-2, -1};
    medusa_tree_plan* p = NULL;
    check(medusa_tree_plan_create(one, 1, 2, &p) == MEDUSA_OK, "single path (1,)");
    medusa_tree_plan_destroy(p);
    p = NULL;
    check(medusa_tree_plan_create(neg, 1, 2, &p) == MEDUSA_ERR_TREE && p == NULL, "negative rank");
    check(medusa_tree_plan_full(NULL, 2, &p) == MEDUSA_ERR_NULL, "null sizes");
    check(medusa_rope(MEDUSA_BF16, 4, 2, 1, 60, (const int32_t*)16, 1e4f, (void*)16, (void*)16,
                      NULL) == MEDUSA_ERR_SHAPE, "rope head dim 60");
    check(strlen(medusa_status_string(MEDUSA_ERR_SHAPE)) > 0, "status string");

    medusa_tree_plan_destroy(sparse);
    medusa_tree_plan_destroy(full);
    printf("%d failures\n", failures);
    return failures;
}
