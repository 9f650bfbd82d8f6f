/* Plain C99 use of the C ABI: the header compiles as C, the library links
 * from C, and the argument checks answer before any launch (no GPU needed). */
#include <stdint.h>
#include <stdio.h>

#include "specverify.h"
#include "sv_measure.h"

int main(void) {
    int fails = 0;
    int32_t dummy[4] = {0, 0, 0, 0};
    /* a NULL target with B > 0 is refused before any launch */
    if (sv_verify_greedy(NULL, dummy, 2, 1, 3, 100, 100, SV_DTYPE_BF16, dummy, dummy, NULL,
                         NULL, 0, NULL) != SV_ERR_NULL)
        ++fails;
    /* an empty batch is a no-op */
    if (sv_verify_stochastic(NULL, NULL, NULL, NULL, NULL, 0, 3, 100, 100, SV_DTYPE_F32, 1.0f,
                             NULL, NULL, NULL, NULL, 0, NULL) != SV_OK)
        ++fails;
    if (sv_verify_stochastic(NULL, NULL, NULL, NULL, NULL, 1, SV_MAX_K + 1, 100, 100,
                             SV_DTYPE_F32, 1.0f, dummy, dummy, NULL, NULL, 0, NULL) != SV_ERR_SHAPE)
        ++fails;
    if (sv_sample(dummy, NULL, 1, 10, 10, SV_DTYPE_F32, 0.0f, 0, dummy, NULL, 0, NULL) !=
        SV_ERR_TEMPERATURE)
        ++fails;
    if (sv_commit(NULL, NULL, 0, 1, NULL, NULL, 0, 0, NULL, 1, NULL) != SV_OK) ++fails;
    if (sv_stream_read(NULL, 0, 1, NULL, NULL) != SV_OK) ++fails;
    if (sv_stream_read(dummy, 15, 1, (uint32_t*)dummy, NULL) != SV_ERR_SHAPE) ++fails;
    if (sv_workspace_bytes(64, 1, 4, 128256) == 0) ++fails;
    if (sv_status_string(SV_ERR_WORKSPACE)[0] == '\0') ++fails;
    printf("%s\n", fails ? "FAIL" : "ok");
    return fails;
}
