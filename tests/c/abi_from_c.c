/*
 * A C99 program against include/attn_decode.h: the header compiles as strict
 * C, the library links from C, and its host-side answers come back as the
 * header documents them -- workspace sizes, status text, and the argument
 * checks every entry point makes before any GPU call.  Only calls that must
 * fail those checks are made, so nothing reaches the GPU.  Built and run by
 * tests/test_abi.py.
 */
#include <stdio.h>
#include <string.h>

#include "attn_decode.h"

static int fails = 0;

#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            printf("FAIL line %d: %s\n", __LINE__, #cond);            \
            ++fails;                                                  \
        }                                                             \
    } while (0)

int main(void) {
    static uint16_t h[64];   /* stands in for tensors the checks never reach */
    static float f[64];
    const uint16_t *odd = (const uint16_t *)(const void *)((const char *)h + 1);
    size_t ws;
    attn_status_t st;
    int s;

    ws = attn_decode_workspace_bytes(1, 32, 128, 4096);
    CHECK(ws > 0 && ws % 256 == 0);
    CHECK(attn_decode_workspace_bytes(64, 32, 128, 8192) >= ws);
    CHECK(attn_decode_workspace_bytes(0, 32, 128, 4096) == 0);
    CHECK(attn_decode_workspace_bytes(1, 32, ATTN_MAX_HEAD_DIM + 1, 4096) == 0);
    CHECK(attn_softmax_workspace_bytes(64, 1000) > 0);
    CHECK(attn_softmax_workspace_bytes(0, 1000) == 0);
    for (s = ATTN_OK; s <= ATTN_ERR_HIP; ++s) {
        const char *t = attn_status_string((attn_status_t)s);
        CHECK(t != NULL && t[0] != '\0');
    }

    st = attn_decode_f16(NULL, h, h, h, 32, 128, 4096, 4095, NULL, NULL, 0, NULL);
    CHECK(st == ATTN_ERR_NULL);
    CHECK(attn_last_error() != NULL && attn_last_error()[0] != '\0');
    st = attn_decode_f16(h, h, h, h, 32, ATTN_MAX_HEAD_DIM + 2, 4096, 4095, NULL, NULL, 0, NULL);
    CHECK(st == ATTN_ERR_DIM);
    st = attn_decode_f16(odd, h, h, h, 32, 128, 4096, 4095, NULL, NULL, 0, NULL);
    CHECK(st == ATTN_ERR_ALIGN);
    st = attn_decode_f16(h, h, h, h, 32, 128, 4096, 4095, NULL, NULL, 0, NULL);
    CHECK(st == ATTN_ERR_WORKSPACE);
    st = attn_decode_f16_batched(h, h, h, h, NULL, 2, 32, 128, 4096, NULL, NULL, 0, NULL);
    CHECK(st == ATTN_ERR_NULL);
    st = attn_qk_f16(h, h, NULL, 32, 128, 4096, 4095, NULL);
    CHECK(st == ATTN_ERR_NULL);
    st = attn_softmax_f32(f, f, 0, 10, NULL, 0, NULL);
    CHECK(st == ATTN_ERR_DIM);
    st = attn_rope_f16(h, h, NULL, 1, 4, 64, 64, 10000.0, 0, NULL);
    CHECK(st == ATTN_ERR_NULL);

    {   /* the plan query: host only, C struct layout as declared */
        attn_plan_info pi;
        CHECK(attn_decode_plan(1, 4, 64, 128, 100, 0, &pi) == ATTN_OK);
        CHECK(pi.launches == 1 && pi.chunks == 1 && pi.partial_slots == 0);
        CHECK(attn_decode_plan(64, 32, 128, 8192, 0, ATTN_PLAN_DEVICE_POS, &pi) == ATTN_OK);
        CHECK(pi.balanced == 1 && pi.launches == 2 && pi.partial_slots <= pi.workspace_slots);
        CHECK(attn_decode_plan(1, 4, 64, 128, 0, 0, NULL) == ATTN_ERR_NULL);
        CHECK(attn_decode_plan(1, 4, 64, 128, 0, 16u, &pi) == ATTN_ERR_DIM);
    }

    printf("%s\n", fails ? "FAILED" : "ok");
    return fails != 0;
}
