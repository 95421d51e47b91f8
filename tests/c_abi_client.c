/* A plain C client of libspecverify: the header compiles as C (C99 and C11,
 * -pedantic -Werror), the library links from C, and every call below returns
 * from the host without touching a device (no GPU is needed to run it).
 * It prints one "name value..." line per check; tests/test_c_client.py
 * compares them with the binding and the oracle. */
#include <math.h>
#include <stdio.h>

#include "libspecverify.h"

static void* const FAKE = (void*)0x1000; /* never dereferenced: every call fails validation */

int main(void) {
    int s;
    int32_t i;
    float raw[9] = {1.0f, 3.0f, 2.0f, 5.0f, 4.0f, 4.5f, 7.0f, 6.0f, 8.0f};
    float out[7];
    float bad[3] = {1.0f, 0.0f, 2.0f};
    sv_status st;

    for (s = 0; s <= 8; ++s) printf("status %d %s\n", s, sv_status_str((sv_status)s));
    printf("budget_ws %lu\n", (unsigned long)sv_budget_workspace_bytes(256, 7));
    printf("verify_ws %lu\n", (unsigned long)sv_verify_workspace_bytes(256, 7));
    printf("verify_ws_refused %lu\n", (unsigned long)sv_verify_workspace_bytes(1, 65));

    /* the host-only cost shaping: running max, then a staircase of granule 2 */
    st = sv_cost_table_prepare(raw, 9, 2, out, 7);
    printf("cost_status %d\n", (int)st);
    printf("cost");
    for (i = 0; i < 7; ++i) printf(" %.9g", (double)out[i]);
    printf("\n");
    printf("cost_bad_value %d\n", (int)sv_cost_table_prepare(bad, 3, 1, out, 3));
    printf("cost_null %d\n", (int)sv_cost_table_prepare(NULL, 9, 2, out, 7));

    /* refusals before any launch */
    printf("budget_null %d\n",
           (int)sv_budget_select(NULL, FAKE, 4, 3, FAKE, 13, 4, 4, FAKE, FAKE, NULL, NULL, FAKE,
                                 sv_budget_workspace_bytes(4, 3), NULL));
    printf("pack_shape %d\n",
           (int)sv_pack_varlen(FAKE, FAKE, FAKE, -1, 3, FAKE, FAKE, FAKE, FAKE, NULL, NULL));
    printf("verify_dtype %d\n",
           (int)sv_verify(FAKE, 32, 16, FAKE, 32, (sv_dtype)7, 32, FAKE, FAKE, 4, 3,
                          SV_STOCHASTIC, 1.0f, 0, 0, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL,
                          NULL, FAKE, sv_verify_workspace_bytes(4, 3), NULL));
    printf("verify_temperature %d\n",
           (int)sv_verify(FAKE, 32, 16, FAKE, 32, SV_BF16, 32, FAKE, FAKE, 4, 3, SV_STOCHASTIC,
                          (float)NAN, 0, 0, FAKE, FAKE, NULL, NULL, NULL, NULL, NULL, NULL, FAKE,
                          sv_verify_workspace_bytes(4, 3), NULL));
    printf("verify_nothing %d\n",
           (int)sv_verify(NULL, 32, 0, NULL, 32, SV_F32, 32, NULL, NULL, 0, 3, SV_GREEDY, 1.0f,
                          0, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL));
    printf("noalloc_capacity %d\n",
           (int)sv_verify_noalloc(FAKE, 32, 16, FAKE, 32, SV_BF16, 32, FAKE, FAKE, 4000, 7,
                                  SV_STOCHASTIC, 1.0f, 0, 0, FAKE, FAKE, NULL, NULL, NULL, NULL,
                                  NULL, NULL, NULL));
    return 0;
}
