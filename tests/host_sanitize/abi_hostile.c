/*
 * Drives every entry point of include/llama_mi355x.h with hostile arguments on the host: the
 * library must return the documented status without touching memory it does not own.  Built
 * with AddressSanitizer and UndefinedBehaviorSanitizer against a library whose host code is
 * built the same way (tests/test_host_sanitizers.py); needs no GPU -- every call here fails
 * host-side validation, or fails at its first HIP call when no device is present.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/llama_mi355x.h"

static int fails = 0;
#define EXPECT(cond)                                                       \
    do {                                                                   \
        if (!(cond)) {                                                     \
            printf("FAIL line %d: %s\n", __LINE__, #cond);                 \
            fails++;                                                       \
        }                                                                  \
    } while (0)

static llama_args tiny(void) {
    llama_args a = {256, 4, 8, 2, 512, 768, 1e-5f, 1e4f, 2, 128, LLAMA_FP32};
    return a;
}

int main(void) {
    llama_args a = tiny(), b;
    EXPECT(llama_check_args(&a) == LLAMA_OK);
    EXPECT(llama_check_args(NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_workspace_bytes(NULL) == 0);
    EXPECT(llama_workspace_bytes(&a) > 0);

    /* hostile configurations: every one is refused, and its workspace size is 0 */
    const int32_t bad_ints[] = {0, -1, -64, INT32_MIN, 63, 65, INT32_MAX};
    for (size_t i = 0; i < sizeof bad_ints / sizeof bad_ints[0]; ++i) {
        int32_t v = bad_ints[i];
        b = a; b.dim = v;            EXPECT(llama_check_args(&b) != LLAMA_OK && llama_workspace_bytes(&b) == 0);
        b = a; b.n_layers = v;       EXPECT(v > 0 || llama_check_args(&b) != LLAMA_OK);
        b = a; b.n_heads = v;        EXPECT(llama_check_args(&b) != LLAMA_OK);
        b = a; b.n_kv_heads = v;     EXPECT(llama_check_args(&b) != LLAMA_OK);
        b = a; b.hidden_dim = v;     EXPECT(llama_check_args(&b) != LLAMA_OK);
        b = a; b.vocab_size = v;     EXPECT(v > 0 && v % 2 == 0 ? 1 : llama_check_args(&b) != LLAMA_OK);
        b = a; b.max_batch_size = v; EXPECT(v > 0 || llama_check_args(&b) != LLAMA_OK);
        b = a; b.max_seq_len = v;    EXPECT((v > 0 && v <= 65536) || llama_check_args(&b) != LLAMA_OK);
        b = a; b.dtype = v;          EXPECT((v >= 0 && v <= 2) || llama_check_args(&b) == LLAMA_ERR_INVALID_ARG);
    }
    b = a; b.norm_eps = NAN;    EXPECT(llama_check_args(&b) == LLAMA_ERR_INVALID_ARG);
    b = a; b.norm_eps = -1.f;   EXPECT(llama_check_args(&b) == LLAMA_ERR_INVALID_ARG);
    b = a; b.rope_theta = 0.f;  EXPECT(llama_check_args(&b) == LLAMA_ERR_INVALID_ARG);
    b = a; b.rope_theta = NAN;  EXPECT(llama_check_args(&b) == LLAMA_ERR_INVALID_ARG);
    /* the largest accepted shape: the size arithmetic must not overflow or wrap */
    b = a; b.max_batch_size = INT32_MAX; b.max_seq_len = 65536; b.dim = 8192; b.n_heads = 64;
    b.n_kv_heads = 8; b.hidden_dim = 28672; b.n_layers = 80; b.dtype = LLAMA_BF16;
    EXPECT(llama_check_args(&b) == LLAMA_OK);
    EXPECT(llama_workspace_bytes(&b) > (size_t)1 << 50);

    /* llama_init: missing pieces, misaligned pointers; *out is cleared on every error */
    static unsigned char host_buf[4096] __attribute__((aligned(256)));
    void *fake = host_buf;                               /* never dereferenced by the host code */
    llama_layer_weights lw[4];
    for (int l = 0; l < 4; ++l) {
        const void *p[9] = {fake, fake, fake, fake, fake, fake, fake, fake, fake};
        memcpy(&lw[l], p, sizeof lw[l]);
    }
    llama_weights w = {fake, fake, fake, lw};
    llama_ctx *c = (llama_ctx *)(uintptr_t)1;
    EXPECT(llama_init(&a, NULL, fake, 1 << 20, NULL, &c) == LLAMA_ERR_INVALID_ARG && c == NULL);
    EXPECT(llama_init(&a, &w, fake, 1 << 20, NULL, NULL) == LLAMA_ERR_INVALID_ARG);
    c = (llama_ctx *)(uintptr_t)1;
    EXPECT(llama_init(NULL, &w, fake, 1 << 20, NULL, &c) == LLAMA_ERR_INVALID_ARG && c == NULL);
    llama_weights w2 = w; w2.layers = NULL;
    EXPECT(llama_init(&a, &w2, fake, 1 << 20, NULL, &c) == LLAMA_ERR_INVALID_ARG && c == NULL);
    w2 = w; w2.output = (const char *)fake + 4;
    EXPECT(llama_init(&a, &w2, fake, 1 << 20, NULL, &c) == LLAMA_ERR_INVALID_ARG && c == NULL);
    llama_layer_weights lw2[4];
    memcpy(lw2, lw, sizeof lw);
    lw2[3].w2 = (const char *)fake + 2;
    w2 = w; w2.layers = lw2;
    EXPECT(llama_init(&a, &w2, fake, 1 << 20, NULL, &c) == LLAMA_ERR_INVALID_ARG && c == NULL);
    lw2[3].w2 = NULL;
    EXPECT(llama_init(&a, &w2, fake, 1 << 20, NULL, &c) == LLAMA_ERR_INVALID_ARG && c == NULL);
    /* workspace: too small, misaligned, missing */
    const size_t need = llama_workspace_bytes(&a);
    EXPECT(llama_init(&a, &w, fake, need - 1, NULL, &c) == LLAMA_ERR_WORKSPACE && c == NULL);
    EXPECT(llama_init(&a, &w, (char *)fake + 16, need, NULL, &c) == LLAMA_ERR_WORKSPACE && c == NULL);
    EXPECT(llama_init(&a, &w, NULL, need, NULL, &c) == LLAMA_ERR_WORKSPACE && c == NULL);
    /* valid host arguments with no device present (the test sets ABI_HOSTILE_NO_DEVICE only
     * then, since the workspace here is host memory): the ctx is built (RoPE table, layer
     * copy) and released again when the first device call fails */
    if (getenv("ABI_HOSTILE_NO_DEVICE")) {
        b = a; b.max_seq_len = 65536; b.n_heads = 2; b.n_kv_heads = 2;   /* head_dim 128 */
        c = (llama_ctx *)(uintptr_t)1;
        EXPECT(llama_init(&b, &w, fake, llama_workspace_bytes(&b), NULL, &c) == LLAMA_ERR_HIP && c == NULL);
    }

    /* calls without a ctx or with bad sizes: refused before any device work */
    int32_t tok[8] = {0};
    float logits[8];
    EXPECT(llama_prefill(NULL, tok, 8, 1, 1, 0, logits, 0, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_decode_step(NULL, tok, 1, 1, 0, logits, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_decode_step_noalloc(NULL, tok, 1, 1, 0, logits, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_argmax(NULL, 1, 8, 8, tok, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_argmax(logits, 0, 8, 8, tok, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_argmax(logits, 1, 8, 7, tok, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_argmax(logits, 1, 0, 8, tok, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_argmax(logits, 1, 8, 8, NULL, NULL) == LLAMA_ERR_INVALID_ARG);
    float u[1] = {0.5f};
    EXPECT(llama_sample_top_p(logits, 1, 8, 8, 0.f, 0.9f, u, tok, NULL, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_sample_top_p(logits, 1, 8, 8, NAN, 0.9f, u, tok, NULL, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_sample_top_p(logits, 1, 8, 8, INFINITY, 0.9f, u, tok, NULL, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_sample_top_p(logits, 1, 8, 8, 1.f, NAN, u, tok, NULL, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_sample_top_p(logits, 1, 8, 8, 1.f, -0.5f, u, tok, NULL, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_sample_top_p(logits, 1, 8, 8, 1.f, 0.9f, NULL, tok, NULL, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_sample_top_p(logits, 1, 40000, 40000, 1.f, 0.9f, u, tok, NULL, NULL) == LLAMA_ERR_UNSUPPORTED);
    EXPECT(llama_select_next(NULL, tok, 8, 0, tok, 1, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_select_next(tok, tok, 8, 8, tok, 1, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_select_next(tok, tok, 8, -1, tok, 1, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_select_next(tok, tok, 8, 0, tok, 0, NULL) == LLAMA_ERR_INVALID_ARG);
    EXPECT(llama_profile_select(NULL, 1) == LLAMA_ERR_INVALID_ARG);
    int64_t n;
    double ms;
    EXPECT(llama_profile_read(NULL, &n, &ms) == LLAMA_ERR_INVALID_ARG);
    llama_destroy(NULL);

    const llama_status codes[] = {LLAMA_OK, LLAMA_ERR_INVALID_ARG, LLAMA_ERR_UNSUPPORTED, LLAMA_ERR_WORKSPACE,
                                  LLAMA_ERR_HIP, (llama_status)-99, (llama_status)42};
    for (size_t i = 0; i < sizeof codes / sizeof codes[0]; ++i) EXPECT(strlen(llama_status_str(codes[i])) > 0);

    printf("abi_hostile: %d failures\n", fails);
    return fails != 0;
}
