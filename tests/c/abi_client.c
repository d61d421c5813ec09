/* A plain C client of the library: it includes the public header as C99 and
 * calls only what needs no GPU (status strings, argument validation and the
 * host-side planner), printing one line per check. Built and run by
 * tests/test_abi.py. */
#include <stdio.h>
#include <stdint.h>

#include "agq.h"

int main(void) {
    int failures = 0;
    agq_plan plan;
    agq_status st;

    printf("version %d\n", agq_version());
    printf("status %s %s\n", agq_status_str(AGQ_OK), agq_status_str(AGQ_ENOTSUP));

    /* Malformed arguments are rejected before any HIP call. */
    st = agq_qmv(NULL, NULL, NULL, NULL, NULL, 16, 64, 4, 64, NULL);
    printf("null pointers -> %s (%s)\n", agq_status_str(st), agq_last_error());
    failures += st != AGQ_EINVAL;

    st = agq_plan_product(1, 128256, 4096, 4, 64, 256, 8, 0, &plan);
    printf("plan 128256x4096: status %s cpt %d rows/iter %d stages %d groups %lld blocks %lld threads %d\n",
           agq_status_str(st), plan.cpt, plan.rows_per_iter, plan.stages, (long long)plan.row_groups,
           (long long)plan.blocks, plan.threads_per_block);
    failures += st != AGQ_OK;
    failures += plan.row_groups * plan.rows_per_group < 128256;

    st = agq_plan_product(9, 64, 64, 4, 64, 256, 8, 0, &plan);
    printf("plan M=9 -> %s\n", agq_status_str(st));
    failures += st != AGQ_ENOTSUP;

    printf("failures %d\n", failures);
    return failures;
}
