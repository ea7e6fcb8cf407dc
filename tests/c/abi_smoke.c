/* A plain C caller of the library's boundary: includes the public header,
 * links libssd_mi355x.so and exercises the calls that need no GPU (version,
 * status strings, workspace sizes, argument checks that fail before any
 * launch).  Built and run by tests/test_abi_host.py. */
#include <stdio.h>
#include <string.h>

#include "ssd_mi355x.h"

static int fails = 0;
#define CHECK(cond) do { if (!(cond)) { printf("FAIL line %d: %s\n", __LINE__, #cond); ++fails; } } while (0)

int main(void) {
    CHECK(ssd_abi_version() == SSD_ABI_VERSION);
    CHECK(strlen(ssd_status_str(SSD_OK)) > 0);
    CHECK(strlen(ssd_status_str(12345)) > 0);
    /* the bench workload's workspace: cs, dtc, S, Hin regions */
    CHECK(ssd_forward_workspace_bytes(4, 8192, 80, 64, 128, 1, 256, SSD_DTYPE_BF16) > 0);
    CHECK(ssd_forward_workspace_bytes(4, 8192, 80, 64, 128, 3, 256, SSD_DTYPE_BF16) == 0);
    CHECK(ssd_state_passing_seg_workspace_bytes(1, 32, 64, 128, 64) > 0);
    /* argument errors are reported before anything touches a device */
    float *f = (float *)0x10000;
    void *v = (void *)0x20000;
    CHECK(ssd_forward(0, 64, 2, 16, 16, 1, 64, SSD_DTYPE_F32, v, f, f, v, v, NULL, NULL, v, NULL,
                      v, 1 << 20, NULL) == SSD_ERR_SHAPE);
    CHECK(ssd_forward(1, 64, 2, 16, 16, 1, 64, SSD_DTYPE_F32, NULL, f, f, v, v, NULL, NULL, v,
                      NULL, v, 1 << 20, NULL) == SSD_ERR_NULL);
    CHECK(ssm_step(1, 2, 16, 16, 1, 7, (float *)0x100000, v, f, f, v, v, NULL, v, NULL) ==
          SSD_ERR_UNSUPPORTED);
    CHECK(ssd_layer_out(0, SSD_DTYPE_BF16, v, v, v, NULL) == SSD_ERR_SHAPE);
    printf(fails ? "abi_smoke: %d failures\n" : "abi_smoke: ok\n", fails);
    return fails != 0;
}
