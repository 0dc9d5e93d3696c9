/* A real decode step driven from plain C99 through include/kvdec.h: device
 * buffers from the HIP runtime, a self cache and a static encoder cache,
 * kvdec_append_attend_cross for one token (outputs against the f64 oracle,
 * libkvdec_oracle.so, test infrastructure; appended rows and lengths bit for
 * bit), then a second token that one sequence has no room for, refused
 * before anything is enqueued.  Needs an MI355X.  Prints "0 failed" when
 * every check passes. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvdec.h"

/* the oracle's entry points (oracle/kvdec_oracle.c) */
int kvdec_oracle_attend(const float* q, const void* K, const void* V, int dtype, int64_t B,
                        int64_t Hq, int64_t Hkv, int64_t D, int64_t cap, const int32_t* lens,
                        double scale, double* out);
int kvdec_oracle_append(void* cacheK, void* cacheV, const void* k_new, const void* v_new,
                        int64_t esz, int64_t B, int64_t Hkv, int64_t D, int64_t cap,
                        int32_t* lens);
int kvdec_oracle_seed(void* dst, const void* src, int64_t esz, int64_t B, int64_t rows,
                      int64_t Hkv, int64_t D, int64_t cap);

static int fails = 0;

#define CHECK(cond)                                                                \
    do {                                                                           \
        if (!(cond)) {                                                             \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);     \
            ++fails;                                                               \
        }                                                                          \
    } while (0)

#define HIP(call) CHECK((call) == hipSuccess)

enum { B = 3, HKV = 2, HQ = 4, D = 64, CAP = 100, ENC = 150 };

/* deterministic values in [-1, 1) */
static float val(unsigned i)
{
    i = i * 2654435761u + 12345u;
    i ^= i >> 13;
    return (float)(i % 2000u) / 1000.0f - 1.0f;
}

/* row-relative error of the GPU rows against the oracle's */
static double worst(const float* got, const double* ref, int rows)
{
    double w = 0.0;
    for (int r = 0; r < rows; ++r) {
        double num = 0.0, den = 1e-30;
        for (int d = 0; d < D; ++d) {
            const double e = fabs((double)got[r * D + d] - ref[r * D + d]);
            if (e > num) num = e;
            if (fabs(ref[r * D + d]) > den) den = fabs(ref[r * D + d]);
        }
        if (num / den > w) w = num / den;
    }
    return w;
}

int main(void)
{
    const int cap_pad = kvdec_padded_capacity(CAP);
    const int enc_pad = kvdec_padded_capacity(ENC);
    const size_t cache_elems = (size_t)B * HKV * cap_pad * D;
    const size_t enc_elems = (size_t)B * HKV * enc_pad * D;
    float* hk = calloc(cache_elems, sizeof(float));
    float* hv = calloc(cache_elems, sizeof(float));
    float* tok_k = malloc((size_t)B * ENC * HKV * D * sizeof(float));
    float* tok_v = malloc((size_t)B * ENC * HKV * D * sizeof(float));
    float* ek = calloc(enc_elems, sizeof(float));
    float* ev = calloc(enc_elems, sizeof(float));
    int32_t lens[B] = {0, 37, 99};           /* empty, ragged, one row short of the capacity */
    for (size_t i = 0; i < cache_elems; ++i) {
        hk[i] = val((unsigned)i);
        hv[i] = val((unsigned)i + 7777777u);
    }
    for (size_t i = 0; i < (size_t)B * ENC * HKV * D; ++i) {
        tok_k[i] = val((unsigned)i + 333u);
        tok_v[i] = val((unsigned)i + 999999u);
    }
    CHECK(kvdec_oracle_seed(ek, tok_k, 4, B, ENC, HKV, D, enc_pad) == 0);
    CHECK(kvdec_oracle_seed(ev, tok_v, 4, B, ENC, HKV, D, enc_pad) == 0);

    void *dk, *dv, *dek, *dev, *dtk, *dtv, *dkn, *dvn, *dq, *dqx, *dout, *doutx, *dws;
    int32_t *dlens, *delens;
    int n_dev = 0;
    if (hipGetDeviceCount(&n_dev) != hipSuccess || n_dev < 1) {
        printf("no GPU\n");
        return 2;
    }
    HIP(hipMalloc(&dk, cache_elems * 4));
    HIP(hipMalloc(&dv, cache_elems * 4));
    HIP(hipMalloc(&dek, enc_elems * 4));
    HIP(hipMalloc(&dev, enc_elems * 4));
    HIP(hipMalloc(&dtk, (size_t)B * ENC * HKV * D * 4));
    HIP(hipMalloc(&dtv, (size_t)B * ENC * HKV * D * 4));
    HIP(hipMalloc(&dkn, (size_t)B * HKV * D * 4));
    HIP(hipMalloc(&dvn, (size_t)B * HKV * D * 4));
    HIP(hipMalloc(&dq, (size_t)B * HQ * D * 4));
    HIP(hipMalloc(&dqx, (size_t)B * HQ * D * 4));
    HIP(hipMalloc(&dout, (size_t)B * HQ * D * 4));
    HIP(hipMalloc(&doutx, (size_t)B * HQ * D * 4));
    HIP(hipMalloc((void**)&dlens, B * 4));
    HIP(hipMalloc((void**)&delens, B * 4));
    HIP(hipMemcpy(dk, hk, cache_elems * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(dv, hv, cache_elems * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(dtk, tok_k, (size_t)B * ENC * HKV * D * 4, hipMemcpyHostToDevice));
    HIP(hipMemcpy(dtv, tok_v, (size_t)B * ENC * HKV * D * 4, hipMemcpyHostToDevice));

    kvdec_cache_desc sd = {B, HKV, D, CAP, KVDEC_F32, 0, 0, 0, dk, dv, dlens};
    kvdec_cache_desc xd = {B, HKV, D, ENC, KVDEC_F32, 1, 0, 0, dek, dev, delens};
    int32_t zeros[B] = {0, 0, 0};
    kvdec_cache *self = NULL, *cross = NULL;
    CHECK(kvdec_cache_create(&sd, lens, NULL, &self) == KVDEC_OK);
    CHECK(kvdec_cache_create(&xd, zeros, NULL, &cross) == KVDEC_OK);
    CHECK(kvdec_seed(cross, dtk, dtv, ENC, NULL) == KVDEC_OK);
    const size_t ws_bytes = kvdec_workspace_bytes(self, HQ) + kvdec_workspace_bytes(cross, HQ);
    HIP(hipMalloc(&dws, ws_bytes));

    float kn[B * HKV * D], vn[B * HKV * D], q[B * HQ * D], qx[B * HQ * D];
    float out[B * HQ * D], outx[B * HQ * D];
    double ref[B * HQ * D], refx[B * HQ * D];
    int32_t enc_lens[B] = {ENC, ENC, ENC};
    for (int step = 0; step < 2; ++step) {
        for (int i = 0; i < B * HKV * D; ++i) {
            kn[i] = val(5000000u + 1000u * step + i);
            vn[i] = val(6000000u + 1000u * step + i);
        }
        for (int i = 0; i < B * HQ * D; ++i) {
            q[i] = val(7000000u + 1000u * step + i);
            qx[i] = val(8000000u + 1000u * step + i);
        }
        HIP(hipMemcpy(dkn, kn, sizeof kn, hipMemcpyHostToDevice));
        HIP(hipMemcpy(dvn, vn, sizeof vn, hipMemcpyHostToDevice));
        HIP(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice));
        HIP(hipMemcpy(dqx, qx, sizeof qx, hipMemcpyHostToDevice));
        /* the second token would overflow sequence 2: only the first runs the layer step */
        if (step == 1) {
            CHECK(kvdec_append_attend_cross(self, cross, NULL, dkn, dvn, dq, dqx, HQ, 0.125f, 0, 0,
                                            dout, doutx, dws, ws_bytes, NULL) == KVDEC_E_OVERFLOW);
            CHECK(strlen(kvdec_last_error()) > 0);
            break;
        }
        CHECK(kvdec_append_attend_cross(self, cross, NULL, dkn, dvn, dq, dqx, HQ, 0.125f, 0, 0,
                                        dout, doutx, dws, ws_bytes, NULL) == KVDEC_OK);
        HIP(hipDeviceSynchronize());
        HIP(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(outx, doutx, sizeof outx, hipMemcpyDeviceToHost));
        CHECK(kvdec_oracle_append(hk, hv, kn, vn, 4, B, HKV, D, cap_pad, lens) == 0);
        CHECK(kvdec_oracle_attend(q, hk, hv, 0, B, HQ, HKV, D, cap_pad, lens, 0.125, ref) == 0);
        CHECK(kvdec_oracle_attend(qx, ek, ev, 0, B, HQ, HKV, D, enc_pad, enc_lens, 0.125, refx) == 0);
        CHECK(worst(out, ref, B * HQ) <= 1e-4);
        CHECK(worst(outx, refx, B * HQ) <= 1e-4);
    }
    int32_t got[B];
    CHECK(kvdec_get_lens(self, got) == KVDEC_OK);
    HIP(hipMemcpy(got, dlens, sizeof got, hipMemcpyDeviceToHost));
    for (int b = 0; b < B; ++b) CHECK(got[b] == lens[b]);
    float* back = malloc(cache_elems * 4);
    HIP(hipMemcpy(back, dk, cache_elems * 4, hipMemcpyDeviceToHost));
    CHECK(memcmp(back, hk, cache_elems * 4) == 0);            /* the appended rows, bit for bit */
    free(back);

    kvdec_cache_destroy(self);
    kvdec_cache_destroy(cross);
    hipFree(dk); hipFree(dv); hipFree(dek); hipFree(dev); hipFree(dtk); hipFree(dtv);
    hipFree(dkn); hipFree(dvn); hipFree(dq); hipFree(dqx); hipFree(dout); hipFree(doutx);
    hipFree(dws); hipFree(dlens); hipFree(delens);
    free(hk); free(hv); free(tok_k); free(tok_v); free(ek); free(ev);
    printf("%d failed\n", fails);
    return fails != 0;
}
