/* A plain C99 client of include/ga.h, built and run on the host by
 * tests/test_c_client.py.  It calls only what runs without a GPU: the
 * planners, the z helper, the status strings, and entry points whose
 * arguments are rejected on the host before any HIP call.  Prints "ok" and
 * exits 0 when every check holds. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "ga.h"

static int failures = 0;

static void check(int cond, const char *what) {
    if (!cond) {
        printf("FAILED: %s (last error: %s)\n", what, ga_last_error());
        ++failures;
    }
}

int main(void) {
    ga_plan p;
    double z;
    const void *fake_in = (const void *)(unsigned long)0x7F0000000000UL;
    void *fake_out = (void *)(unsigned long)0x7F1000000000UL;

    check(ga_version() > 0, "version");
    check(strcmp(ga_status_str(GA_OK), "GA_OK") == 0, "status string");

    /* The headline shape: one workgroup of 8 waves per row, 4 vectors per lane, up late. */
    memset(&p, 0, sizeof p);
    check(ga_plan_gelu_and_mul_sparse(2048, 16384, GA_BF16, 1, 256, 1, &p) == GA_OK, "plan headline");
    check(p.path == 0 && p.waves_per_row == 8 && p.per_lane == 4 && p.up_late == 1 && p.splits == 1 &&
              p.block == 512 && p.grid == 2048,
          "headline geometry");
    /* Few long rows with a workspace: split rows. */
    check(ga_plan_gelu_and_mul_sparse(1, 32768, GA_BF16, 1, 256, 1, &p) == GA_OK && p.splits > 1, "split plan");
    /* Short rows: packed, 256-lane workgroups. */
    check(ga_plan_gelu_and_mul_sparse(4096, 128, GA_BF16, 1, 256, 1, &p) == GA_OK && p.path == 3 &&
              p.block == 256,
          "packed plan");
    check(ga_gelu_and_mul_sparse_workspace_bytes(0) == 0 && ga_gelu_and_mul_sparse_workspace_bytes(64) > 0,
          "workspace size");
    check(ga_plan_silu_and_mul_bounded(16384, 768, GA_BF16, 1, 256, &p) == GA_OK && p.grid >= 1, "silu plan");

    z = ga_z_from_sparsity(0.95);
    check(fabs(z - 1.6448536269514722) < 1e-12, "z(0.95)");
    check(ga_z_from_sparsity(0.5) == 0.0, "z(0.5)");

    /* Rejected on the host: nothing is launched. */
    check(ga_gelu_and_mul_sparse(NULL, fake_out, 4, 64, GA_BF16, 1.6448536f, NULL, NULL) == GA_EINVAL,
          "null input");
    check(strlen(ga_last_error()) > 0, "error message");
    check(ga_gelu_and_mul_sparse(fake_in, fake_out, 4, 65537, GA_BF16, 1.6448536f, NULL, NULL) ==
              GA_EUNSUPPORTED,
          "d above GA_MAX_D");
    check(ga_silu_and_mul_bounded(fake_in, fake_out, 16, 768, GA_BF16, NULL, NULL) == GA_EINVAL,
          "silu without a live count");
    check(ga_gelu_and_mul(fake_in, fake_out, 4, 64, GA_BF16, 7, NULL, NULL) == GA_EINVAL, "bad GELU form");
    check(ga_gelu_and_mul_sparse(fake_in, fake_out, 0, 64, GA_BF16, 1.6448536f, NULL, NULL) == GA_OK,
          "zero rows");

    if (failures == 0) printf("ok\n");
    return failures == 0 ? 0 : 1;
}
