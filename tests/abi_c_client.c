/* A plain C11 client of the library's host-only entry points (no device
 * work): the header compiles as C, and the ABI is usable without Python.
 * Built and run by tests/test_abi_c_client.py; prints "ok" on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "q4adamw.h"

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            printf("FAIL line %d: %s (%s)\n", __LINE__, #c, q4adamw_last_error()); \
            return 1;                                                     \
        }                                                                 \
    } while (0)

/* Addresses for the validation calls, which check alignment and presence
 * but never dereference. */
static void* fake(uintptr_t k) { return (void*)(uintptr_t)(0x100000u + 0x1000u * k); }

static void packed_tensor(q4_tensor* t, uint32_t id, int ndim, const int64_t* shape) {
    memset(t, 0, sizeof *t);
    t->tensor_id = id;
    t->ndim = ndim;
    t->numel = 1;
    for (int d = 0; d < ndim; ++d) {
        t->shape[d] = shape[d];
        t->numel *= shape[d];
    }
    t->param = (float*)fake(8 * id + 1);
    t->grad = (const uint16_t*)fake(8 * id + 2);
    t->m_codes = (uint8_t*)fake(8 * id + 3);
    t->m_scales = (float*)fake(8 * id + 4);
    t->v_codes = (uint8_t*)fake(8 * id + 5);
    t->v_scales = (float*)fake(8 * id + 6);
}

int main(void) {
    CHECK(q4adamw_abi_version() == Q4ADAMW_ABI_VERSION);
    CHECK(q4adamw_status_string(Q4_ERR_CONFLICT) != NULL);

    q4_config cfg;
    CHECK(q4adamw_default_config(Q4_RECIPE_ZIP_SR, &cfg) == Q4_OK);
    CHECK(cfg.block == Q4ADAMW_BLOCK && cfg.m_codebook == Q4_CB_NF4 && cfg.v_codebook == Q4_CB_DYN4);
    CHECK(cfg.v_rule == Q4_RULE_UPDATE_SR && cfg.eden == 0);

    /* a vector of 1000 elements and a 64 x 520 matrix */
    const int64_t s0[1] = {1000}, s1[2] = {64, 520};
    q4_tensor t[2];
    packed_tensor(&t[0], 0, 1, s0);
    packed_tensor(&t[1], 1, 2, s1);

    q4_hparams hp;
    memset(&hp, 0, sizeof hp);
    hp.lr = 1e-3f;
    hp.beta1 = 0.9f;
    hp.beta2 = 0.999f;
    hp.eps = 1e-8f;
    hp.weight_decay = 0.1f;
    hp.step = 1;
    CHECK(q4adamw_validate(&cfg, &hp, t, 2) == Q4_OK);
    hp.step = 0;
    CHECK(q4adamw_validate(&cfg, &hp, t, 2) == Q4_ERR_INVALID_ARG);
    CHECK(strlen(q4adamw_last_error()) > 0);
    hp.step = 1;
    q4_config bad = cfg;
    bad.block = 64;
    CHECK(q4adamw_validate(&bad, &hp, t, 2) == Q4_ERR_INVALID_ARG);

    /* codes ceil(n/2) bytes per moment, one FP32 scale per 128 elements per moment */
    q4_state_bytes sb;
    CHECK(q4adamw_state_bytes(&cfg, t, 2, &sb) == Q4_OK);
    CHECK(sb.adam4_quantized_state_bytes == 2u * (500u + 16640u));
    CHECK(sb.adam4_scale_metadata_bytes == 2u * 4u * (8u + 260u));
    CHECK(sb.adam4_total_bytes == sb.adam4_quantized_state_bytes + sb.adam4_scale_metadata_bytes);

    size_t ws = 0;
    CHECK(q4adamw_workspace_bytes(&cfg, t, 2, &ws) == Q4_OK && ws >= 256);

    /* the flat microbatch layout: each tensor at 512 x (chunks before it) */
    int64_t off[2], total = 0;
    CHECK(q4adamw_flat_offsets(t, 2, off, &total) == Q4_OK);
    CHECK(off[0] == 0 && off[1] == 1024 && total == 1024 + 33280);

    q4_state_header h;
    CHECK(q4adamw_make_header(&cfg, &h) == Q4_OK && h.magic == Q4ADAMW_STATE_MAGIC);
    CHECK(q4adamw_check_header(&cfg, &h) == Q4_OK);
    q4_config other;
    CHECK(q4adamw_default_config(Q4_RECIPE_ZE_EDEN, &other) == Q4_OK);
    CHECK(q4adamw_check_header(&other, &h) == Q4_ERR_STATE_FORMAT);

    float lv[256];
    CHECK(q4adamw_codebook(Q4_CB_NF4, lv) == Q4_OK);
    CHECK(lv[0] == -1.0f && lv[7] == 0.0f && lv[15] == 1.0f);
    float sc[5];
    CHECK(q4adamw_host_scalars(&hp, sc) == Q4_OK);
    CHECK(sc[3] == 1.0f - 0.9f && sc[4] == 1.0f - 0.999f);

    printf("ok\n");
    return 0;
}
