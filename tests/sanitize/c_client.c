/*
 * A plain C client of the library (C99, no C++): it includes include/hyena.h and
 * calls the entry points whose argument checks run on the host before any HIP
 * call, so it runs without a GPU (tests/test_abi.py builds and runs it). Exit
 * status 0 when every call returned the documented status.
 */
#include <stdio.h>
#include <string.h>

#include "hyena.h"

static int fails = 0;
static void expect(int cond, const char* what) {
    if (!cond) {
        fprintf(stderr, "unexpected: %s\n", what);
        ++fails;
    }
}

int main(void) {
    hyena_plan_t plan = NULL;
    expect(hyena_plan_create(NULL, 1024, 4, 2, HYENA_F32) == HYENA_ERR_INVALID_ARG, "NULL out");
    expect(hyena_plan_create(&plan, 1000, 4, 2, HYENA_F32) == HYENA_ERR_UNSUPPORTED, "L not a power of two");
    expect(hyena_plan_create(&plan, 1024, 4, 1, HYENA_F32) == HYENA_ERR_INVALID_ARG, "order 1");
    expect(hyena_plan_create(&plan, 1024, 0, 2, HYENA_F32) == HYENA_ERR_INVALID_ARG, "D = 0");
    expect(plan == NULL, "no plan after a failed create");
    expect(hyena_plan_destroy(NULL) == HYENA_OK, "destroy(NULL)");
    expect(hyena_spectrum_bytes(NULL) == 0 && hyena_workspace_bytes(NULL, 1) == 0, "sizes of a NULL plan");
    expect(hyena_forward(NULL, 1, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == HYENA_ERR_INVALID_ARG,
           "forward on a NULL plan");
    expect(hyena_backward(NULL, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
               HYENA_ERR_INVALID_ARG,
           "backward on a NULL plan");
    const hyena_status_t all[] = {HYENA_OK, HYENA_ERR_INVALID_ARG, HYENA_ERR_UNSUPPORTED, HYENA_ERR_WORKSPACE,
                                  HYENA_ERR_DEVICE};
    for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) {
        const char* s = hyena_status_string(all[i]);
        expect(s != NULL && strlen(s) > 0, "status string");
    }
    printf("c client: %d unexpected\n", fails);
    return fails ? 1 : 0;
}
