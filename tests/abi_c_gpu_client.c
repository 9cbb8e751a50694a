/* A plain C11 program that drives the fused step through the C ABI on the
 * GPU, with its own hipMalloc buffers and the null stream: init_state, three
 * ZIP-SR steps, then the state and weights copied back and written to the
 * file named by argv[1] (param, m codes, m scales, v codes, v scales, raw).
 * The inputs come from integer hashes so that tests/test_abi_c_client.py
 * can rebuild the same bytes and step the oracle on them. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "q4adamw.h"

#define N 1000
#define NB ((N + 127) / 128)
#define NC ((N + 1) / 2)

#define CHECK(c)                                                                    \
    do {                                                                            \
        if (!(c)) {                                                                 \
            printf("FAIL line %d: %s (%s)\n", __LINE__, #c, q4adamw_last_error());   \
            return 1;                                                               \
        }                                                                           \
    } while (0)

static uint32_t hash32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7FEB352Du;
    x ^= x >> 15;
    x *= 0x846CA68Bu;
    x ^= x >> 16;
    return x;
}
/* a float in [-0.5, 0.5) from 24 hash bits, times `scale` */
static float unit(uint32_t h, float scale) { return ((float)(h >> 8) * (1.0f / 16777216.0f) - 0.5f) * scale; }
static uint16_t bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int main(int argc, char** argv) {
    if (argc < 2) return 2;
    static float param[N];
    static uint16_t grad[3][N];
    for (uint32_t i = 0; i < N; ++i) {
        param[i] = unit(hash32(i), 0.04f);
        for (uint32_t s = 0; s < 3; ++s) grad[s][i] = bf16_bits(unit(hash32(i + 7919u * (s + 1)), 2e-3f));
    }
    q4_config cfg;
    CHECK(q4adamw_default_config(Q4_RECIPE_ZIP_SR, &cfg) == Q4_OK);

    q4_tensor t;
    memset(&t, 0, sizeof t);
    t.tensor_id = 3;
    t.ndim = 1;
    t.shape[0] = N;
    t.numel = N;
    void *dp, *dg, *dmc, *dms, *dvc, *dvs, *dws;
    CHECK(hipMalloc(&dp, 4 * N) == hipSuccess && hipMalloc(&dg, 2 * N) == hipSuccess);
    CHECK(hipMalloc(&dmc, NC) == hipSuccess && hipMalloc(&dms, 4 * NB) == hipSuccess);
    CHECK(hipMalloc(&dvc, NC) == hipSuccess && hipMalloc(&dvs, 4 * NB) == hipSuccess);
    t.param = (float*)dp;
    t.grad = (const uint16_t*)dg;
    t.m_codes = (uint8_t*)dmc;
    t.m_scales = (float*)dms;
    t.v_codes = (uint8_t*)dvc;
    t.v_scales = (float*)dvs;
    size_t ws = 0;
    CHECK(q4adamw_workspace_bytes(&cfg, &t, 1, &ws) == Q4_OK);
    CHECK(hipMalloc(&dws, ws) == hipSuccess);
    CHECK(hipMemcpy(dp, param, 4 * N, hipMemcpyHostToDevice) == hipSuccess);
    CHECK(q4adamw_init_state(&cfg, &t, 1, NULL) == Q4_OK);

    q4_hparams hp;
    memset(&hp, 0, sizeof hp);
    hp.lr = 1e-3f;
    hp.beta1 = 0.9f;
    hp.beta2 = 0.999f;
    hp.eps = 1e-8f;
    hp.weight_decay = 0.1f;
    hp.seed = 5;
    for (int s = 0; s < 3; ++s) {
        CHECK(hipMemcpy(dg, grad[s], 2 * N, hipMemcpyHostToDevice) == hipSuccess);
        hp.step = (uint64_t)(s + 1);
        hp.flags = s > 0 ? Q4_HP_REUSE_TABLE : 0u;
        CHECK(q4adamw_step(&cfg, &hp, &t, 1, dws, ws, NULL) == Q4_OK);
    }
    CHECK(hipDeviceSynchronize() == hipSuccess);

    static uint8_t mc[NC], vc[NC];
    static float ms[NB], vs[NB];
    CHECK(hipMemcpy(param, dp, 4 * N, hipMemcpyDeviceToHost) == hipSuccess);
    CHECK(hipMemcpy(mc, dmc, NC, hipMemcpyDeviceToHost) == hipSuccess);
    CHECK(hipMemcpy(ms, dms, 4 * NB, hipMemcpyDeviceToHost) == hipSuccess);
    CHECK(hipMemcpy(vc, dvc, NC, hipMemcpyDeviceToHost) == hipSuccess);
    CHECK(hipMemcpy(vs, dvs, 4 * NB, hipMemcpyDeviceToHost) == hipSuccess);
    FILE* f = fopen(argv[1], "wb");
    CHECK(f != NULL);
    CHECK(fwrite(param, 4, N, f) == N && fwrite(mc, 1, NC, f) == NC && fwrite(ms, 4, NB, f) == NB);
    CHECK(fwrite(vc, 1, NC, f) == NC && fwrite(vs, 4, NB, f) == NB);
    fclose(f);
    (void)hipFree(dp);
    (void)hipFree(dg);
    (void)hipFree(dmc);
    (void)hipFree(dms);
    (void)hipFree(dvc);
    (void)hipFree(dvs);
    (void)hipFree(dws);
    printf("ok\n");
    return 0;
}
