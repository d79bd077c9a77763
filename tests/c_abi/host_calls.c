/* A C99 client of the library: includes adam.h as a C translation unit and
 * makes the calls that need no GPU (plan, two-buffer plan, a handle over an
 * empty list, the host step counter of that handle, the handle-free step
 * on an empty list, status strings).  Exit status 0 when
 * every call behaves as the header states, else the number of the first
 * failed check. */
#include <stdio.h>
#include <string.h>

#include "adam.h"

int main(void)
{
    adam_tensor t[2], a[2];
    adam_tl_desc d;
    adam_tl_stats st;
    adam_tl *tl = NULL;
    adam_hparams hp = {0.9f, 0.999f, 1e-8f, 0.01f, 1, 1};
    int32_t step = 0;

    memset(t, 0, sizeof t);
    memset(&d, 0, sizeof d);
    d.p = ADAM_DT_F32;
    d.g = ADAM_DT_BF16;
    d.p_out = ADAM_DT_NONE;
    /* planning reads only the pointer values, never the memory */
    t[0].p = (void *)0x100000;
    t[0].m = (void *)0x200000;
    t[0].v = (void *)0x300000;
    t[0].g = (const void *)0x400000;
    t[0].numel = 4096;

    if (adam_abi_version() != ADAM_ABI_VERSION) return 1;
    if (adam_tl_plan(t, 2, &d, &st) != ADAM_OK) return 2;
    if (st.elements != 4096 || st.nonempty != 1 || st.tensors != 2 || st.bytes_per_elem != 26) return 3;
    if (adam_tl_plan(t, 1, NULL, &st) != ADAM_EINVAL) return 4;
    d.g = ADAM_DT_NONE;
    if (adam_tl_plan(t, 1, &d, &st) != ADAM_EDTYPE) return 5;
    d.g = ADAM_DT_BF16;
    if (adam_tl_build(t, 0, &d, 0, &tl) != ADAM_OK || tl == NULL) return 6;
    if (adam_step(tl, &hp, 1e-3f, &step, 1.0f, NULL, 0) != ADAM_OK || step != 1) return 7;
    if (adam_step(tl, &hp, 1e-3f, &step, 1.0f, NULL, 0) != ADAM_OK || step != 2) return 8;
    hp.mode = 2;
    if (adam_step(tl, &hp, 1e-3f, &step, 1.0f, NULL, 0) != ADAM_EINVAL || step != 2) return 9;
    if (adam_step_remainders(tl, &hp, 1e-3f, &step, 1.0f, NULL, 0) != ADAM_EINVAL) return 10;
    adam_tl_destroy(tl);
    adam_tl_destroy(NULL);
    if (strcmp(adam_status_string(ADAM_EDTYPE), adam_status_string(ADAM_OK)) == 0) return 11;

    /* two-buffer state: a second set of p, m, v, 128-byte multiples away */
    memset(a, 0, sizeof a);
    a[0].p = (void *)0x500000;
    a[0].m = (void *)0x600000;
    a[0].v = (void *)0x700000;
    a[0].numel = 4096;
    if (adam_tl_plan_two_buffer(t, a, 2, &d, &st) != ADAM_OK || st.two_buffer != 1 || st.chunks == 0) return 12;
    if (adam_tl_plan(t, 2, &d, &st) != ADAM_OK || st.two_buffer != 0) return 13;
    a[0].m = (void *)0x600040; /* 64 bytes off: the sets would not share alignment */
    if (adam_tl_plan_two_buffer(t, a, 2, &d, &st) != ADAM_EINVAL) return 14;
    a[0].m = (void *)0x600000;
    a[0].g = (const void *)0x800000; /* the gradient has one buffer */
    if (adam_tl_plan_two_buffer(t, a, 2, &d, &st) != ADAM_EINVAL) return 15;
    a[0].g = NULL;
    if (adam_tl_plan_two_buffer(t, NULL, 2, &d, &st) != ADAM_EINVAL) return 16;
    if (adam_tl_build_two_buffer(t, a, 0, &d, 0, &tl) != ADAM_OK || tl == NULL) return 17;
    step = 0;
    if (adam_step(tl, &hp, 1e-3f, &step, 1.0f, NULL, 0) != ADAM_EINVAL) return 18; /* hp.mode is still 2 */
    hp.mode = 1;
    if (adam_step(tl, &hp, 1e-3f, &step, 1.0f, NULL, 0) != ADAM_OK || step != 1) return 19;
    adam_tl_destroy(tl);

    /* the step without a handle: an empty list advances the counter without
     * touching a device; a refused list leaves it */
    step = 0;
    if (adam_step_noalloc(t, 0, &d, &hp, 1e-3f, &step, 1.0f, NULL, 0) != ADAM_OK || step != 1) return 20;
    d.with_remainders = 1;
    if (adam_step_noalloc(t, 1, &d, &hp, 1e-3f, &step, 1.0f, NULL, 0) != ADAM_EINVAL || step != 1) return 21;
    d.with_remainders = 0;
    if (adam_status_string(ADAM_ETOOBIG) == adam_status_string(-99)) return 22;
    puts("ok");
    return 0;
}
