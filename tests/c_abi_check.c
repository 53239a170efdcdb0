/* A plain C11 consumer of include/moe.h, linked against libmoe.so: the ABI is
 * usable from C with nothing but device pointers, sizes and a stream. Only
 * host-side paths run here (status strings, workspace sizes, argument
 * validation), so no GPU is needed; every call given non-null fake pointers is
 * one that validation rejects before anything is launched. Exit status 0 when
 * every check holds. */
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;
#define CHECK(cond)                                                     \
    do {                                                                \
        if (!(cond)) {                                                  \
            fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #cond); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

int main(void) {
    void *fake = (void *)0x1000; /* never dereferenced */
    moe_layer_desc d;

    CHECK(strcmp(moe_status_string(MOE_OK), "MOE_OK") == 0);
    CHECK(moe_status_string(MOE_ERR_HIP) != NULL);

    /* router: k > E, fp8 tokens, an fp8 gate beside bf16 tokens, T = 0 */
    CHECK(moe_route(fake, MOE_BF16, fake, MOE_BF16, NULL, 4, 64, 8, 9, fake, fake, fake, NULL, 0, NULL) ==
          MOE_ERR_INVALID_ARG);
    CHECK(moe_route(fake, MOE_FP8_E4M3, fake, MOE_FP8_E4M3, NULL, 4, 64, 8, 2, fake, fake, fake, NULL, 0, NULL) ==
          MOE_ERR_UNSUPPORTED);
    CHECK(moe_route(fake, MOE_BF16, fake, MOE_FP8_E4M3, NULL, 4, 64, 8, 2, fake, fake, fake, NULL, 0, NULL) ==
          MOE_ERR_UNSUPPORTED);
    CHECK(moe_route(NULL, MOE_BF16, NULL, MOE_BF16, NULL, 0, 64, 8, 2, NULL, NULL, NULL, NULL, 0, NULL) == MOE_OK);

    /* whole layer: a zero-initialised bf16 descriptor keeps the gate in bf16 */
    memset(&d, 0, sizeof d);
    d.H = 512;
    d.F = 1024;
    d.E = 8;
    d.k = 2;
    d.act_dt = MOE_BF16;
    d.w_dt = MOE_BF16;
    d.path = MOE_PATH_AUTO;
    d.Wg = d.W1 = d.W3 = d.W2 = fake;
    CHECK(moe_forward_workspace_bytes(&d, 16) > 0);
    CHECK(moe_forward_workspace_bytes(&d, 4096) > moe_forward_workspace_bytes(&d, 16));
    CHECK(moe_forward(&d, fake, 16, fake, fake, 16, NULL, NULL, NULL, NULL, NULL, NULL) ==
          MOE_ERR_WORKSPACE_TOO_SMALL);
    CHECK(moe_forward(&d, NULL, 0, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL) == MOE_OK);
    CHECK(moe_forward(NULL, fake, 16, fake, fake, 1 << 30, NULL, NULL, NULL, NULL, NULL, NULL) ==
          MOE_ERR_INVALID_ARG);

    /* a shared expert needs its dtype: zero (F32) beside bf16 experts is refused */
    d.Fs = 512;
    d.Ws1 = d.Ws3 = d.Ws2 = fake;
    CHECK(moe_forward(&d, fake, 16, fake, fake, 1 << 30, NULL, NULL, NULL, NULL, NULL, NULL) ==
          MOE_ERR_UNSUPPORTED);
    d.ws_dt = MOE_BF16;
    CHECK(moe_forward_workspace_bytes(&d, 16) > 0);
    d.gate_f32 = 2; /* a 0/1 flag */
    CHECK(moe_forward_workspace_bytes(&d, 16) == 0);

    /* extreme sizes: products such as T*k or M*H pass 2^31; each call must
     * answer with a status or a size, without overflowing an int */
    CHECK(moe_permute_workspace_bytes(1 << 20, 4096, 8) == 0 || moe_permute_workspace_bytes(1 << 20, 4096, 8) > 0);
    CHECK(moe_permute(fake, 1 << 20, 4096, 8192, fake, fake, fake, fake, NULL, MOE_BF16, 0, NULL, NULL, 0, NULL) !=
          MOE_OK);
    CHECK(moe_permute(fake, 0x7fffffff, 2, 8, fake, fake, fake, fake, NULL, MOE_BF16, 0, NULL, NULL, 0, NULL) ==
          MOE_ERR_UNSUPPORTED);
    (void)moe_route_workspace_bytes(0x7fffffff, 1 << 20, 1024);
    CHECK(moe_route(fake, MOE_BF16, fake, MOE_BF16, NULL, 0x7fffffff, 1 << 20, 1024, 8, fake, fake, fake, NULL, 0,
                    NULL) == MOE_ERR_UNSUPPORTED); /* T*E logits past 2^31 */
    CHECK(moe_route(fake, MOE_BF16, fake, MOE_BF16, NULL, 600, 1 << 20, 1024, 8, fake, fake, fake, NULL, 0,
                    NULL) == MOE_ERR_WORKSPACE_TOO_SMALL);
    CHECK(moe_route(fake, MOE_BF16, fake, MOE_BF16, NULL, 16, 1 << 21, 8, 2, fake, fake, fake, NULL, 0, NULL) ==
          MOE_ERR_UNSUPPORTED); /* H beyond 2^20 */
    (void)moe_grouped_ffn_workspace_bytes(0x7fffffff, 1024, 1 << 20, 1 << 20, MOE_BF16, MOE_BF16, MOE_PATH_AUTO);
    (void)moe_grouped_ffn_workspace_bytes(0x7fffffff, 1, 1 << 20, 1 << 20, MOE_BF16, MOE_FP8_E4M3, MOE_PATH_GEMV);
    CHECK(moe_grouped_ffn(fake, NULL, 1, 0x7fffffff, fake, 1024, 1 << 20, 1 << 20, fake, fake, fake, MOE_BF16, NULL,
                          NULL, NULL, MOE_BF16, fake, MOE_PATH_AUTO, fake, 16, NULL) != MOE_OK);
    CHECK(moe_quantize_e4m3_rows(fake, MOE_BF16, 64, NULL, 1, 4, 128, fake, fake, NULL) == MOE_ERR_INVALID_ARG);
    memset(&d, 0, sizeof d);
    d.H = 1 << 20;
    d.F = 1 << 20;
    d.E = 1024;
    d.k = 64;
    d.act_dt = MOE_BF16;
    d.w_dt = MOE_BF16;
    d.Wg = d.W1 = d.W3 = d.W2 = fake;
    (void)moe_forward_workspace_bytes(&d, 65535);
    CHECK(moe_forward(&d, fake, 65536, fake, fake, 16, NULL, NULL, NULL, NULL, NULL, NULL) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_forward(&d, fake, 65535, fake, fake, 16, NULL, NULL, NULL, NULL, NULL, NULL) ==
          MOE_ERR_WORKSPACE_TOO_SMALL);
    d.H = -32;
    CHECK(moe_forward_workspace_bytes(&d, 16) == 0);
    CHECK(moe_combine(fake, fake, fake, 70000, 2, 64, NULL, MOE_BF16, fake, NULL) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_combine(fake, fake, fake, -1, 2, 64, NULL, MOE_BF16, fake, NULL) == MOE_ERR_INVALID_ARG);

    if (failures) return 1;
    printf("c abi: all checks passed\n");
    return 0;
}
