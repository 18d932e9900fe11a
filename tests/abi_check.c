/* Compiled as C99 against include/ck.h and linked against the library by
 * tests/test_abi.py: the header is valid C, every entry point links, and the
 * host-side argument checks answer from plain C (no call reaches a launch). */
#include <stdint.h>
#include <stdio.h>

#include "ck.h"

#define FAKE ((void *)(uintptr_t)(1u << 20))

static int fails = 0;

static void expect(const char *what, ck_status got, ck_status want)
{
    if (got != want) {
        printf("FAIL %s: got %d (%s), want %d\n", what, (int)got, ck_status_str(got), (int)want);
        ++fails;
    }
}

int main(void)
{
    printf("%s\n", ck_version());
    expect("weight_prep n=0", ck_weight_prep(FAKE, 0, 256, 128, FAKE, FAKE, NULL), CK_OK);
    expect("weight_prep k%group", ck_weight_prep(FAKE, 4, 192, 128, FAKE, FAKE, NULL), CK_ESHAPE);
    expect("act_quant null", ck_act_quant(NULL, 256, 4, 256, CK_ACT_NONE, 128, CK_LAYOUT_ROWS, FAKE, FAKE, NULL),
           CK_EINVAL);
    expect("act_quant swiglu ld", ck_act_quant(FAKE, 256, 4, 256, CK_ACT_SWIGLU, 128, CK_LAYOUT_ROWS, FAKE, FAKE,
                                               NULL),
           CK_ESHAPE);
    size_t ws = ck_int8_linear_workspace_size(4, 256, 32);
    expect("int8_linear workspace", ck_int8_linear(FAKE, 256, CK_ACT_NONE, FAKE, FAKE, NULL, NULL,
                                                   CK_LAYOUT_BLOCKED, 4, 32, 256, 128, FAKE, FAKE, ws - 1, NULL),
           CK_EWORKSPACE);
    expect("int8_linear decode m>64", ck_int8_linear(FAKE, 256, CK_ACT_NONE, FAKE, NULL, NULL, NULL,
                                                     CK_LAYOUT_DECODE, 65, 32, 256, 128, FAKE, FAKE,
                                                     ck_int8_linear_workspace_size(65, 256, 32), NULL),
           CK_EUNSUPPORTED);
    expect("swiglu_mlp shape", ck_swiglu_mlp(FAKE, FAKE, FAKE, FAKE, FAKE, CK_LAYOUT_BLOCKED, 8, 256, 500, 128,
                                             FAKE, FAKE, ck_swiglu_mlp_workspace_size(8, 256, 512), NULL),
           CK_ESHAPE);
    expect("gemm_bf16 n%16", ck_int8_gemm_bf16(FAKE, FAKE, FAKE, FAKE, NULL, NULL, CK_LAYOUT_ROWS, 4, 20, 256, FAKE,
                                               NULL),
           CK_ESHAPE);
    expect("pack n=0", ck_weight_pack(FAKE, 0, 128, FAKE, NULL), CK_OK);
    expect("pack_decode n%16", ck_weight_pack_decode(FAKE, FAKE, 20, 256, FAKE, NULL), CK_ESHAPE);
    expect("w8a16 gemm k%64", ck_w8a16_gemm_bf16(FAKE, FAKE, FAKE, NULL, NULL, 4, 32, 100, FAKE, NULL), CK_ESHAPE);
    expect("w8a16 linear ws", ck_int8_linear_w8a16(FAKE, 256, CK_ACT_NONE, FAKE, FAKE, NULL, NULL, 8, 32, 256, 128,
                                                   FAKE, FAKE, ck_int8_linear_w8a16_workspace_size(8, 256) - 1, NULL),
           CK_EWORKSPACE);
    expect("w8a16 mlp ws", ck_swiglu_mlp_w8a16(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 256, 512, 128, FAKE, FAKE, 0, NULL),
           CK_EWORKSPACE);
    expect("rotate_bf16 layout", ck_act_rotate_bf16(FAKE, 256, 4, 256, CK_ACT_NONE, 128, CK_LAYOUT_DECODE, FAKE,
                                                    NULL),
           CK_EINVAL);
    if (ck_blocked_rows(300) != 512 || ck_blocked_size(300, 128) != 512 * 128 || ck_decode_size(32, 256) != 2 * (64 + 16 * 256)) {
        printf("FAIL size helpers\n");
        ++fails;
    }
    printf(fails ? "%d failures\n" : "all checks passed\n", fails);
    return fails != 0;
}
