/* A C host program that drives libsparseloco.so through include/sparseloco.h
 * alone (no Python, no torch), for a GPU test that checks its outputs against
 * the oracle.
 *
 * usage: sl_c_roundtrip <input> <output>
 * input:  int64 n, float beta, float delta[n], float theta[n]
 * output: uint8 payload1[n/4096][112], float scales1[n/4096],
 *         uint8 payload2[n/4096][112], float scales2[n/4096],
 *         float ef[n], float out[n], float theta[n]
 * Steps, on the current HIP device and the null stream: ef = 0; two rounds of
 * sl_compress(delta, ef) (records 1 and 2); sl_aggregate of the two records
 * into out; sl_apply_mean(theta, out, 2).  Exit status 0 on success, 1 on a
 * usage, file or HIP error, 2 on a library status other than SL_OK. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sparseloco.h"

#define HIP_OK(x)                                                              \
    do {                                                                       \
        if ((x) != hipSuccess) {                                               \
            fprintf(stderr, "HIP error at %s:%d\n", __FILE__, __LINE__);      \
            return 1;                                                          \
        }                                                                      \
    } while (0)

#define SL_OK_OR_EXIT(x)                                                       \
    do {                                                                       \
        sl_status st_ = (x);                                                   \
        if (st_ != SL_OK) {                                                    \
            fprintf(stderr, "%s: %s\n", #x, sl_status_string((int)st_));     \
            return 2;                                                          \
        }                                                                      \
    } while (0)

static int read_all(FILE* f, void* p, size_t bytes) { return fread(p, 1, bytes, f) == bytes ? 0 : 1; }
static int write_all(FILE* f, const void* p, size_t bytes) { return fwrite(p, 1, bytes, f) == bytes ? 0 : 1; }

int main(int argc, char** argv) {
    FILE* in;
    FILE* out;
    int64_t n, chunks;
    float beta;
    size_t dense, pbytes, sbytes;
    float *h_delta, *h_theta, *h_ef, *h_out, *h_s1, *h_s2;
    uint8_t *h_p1, *h_p2;
    float *d_delta, *d_theta, *d_ef, *d_out, *d_s1, *d_s2;
    uint8_t *d_p1, *d_p2;
    const uint8_t* payloads[2];
    const float* scales[2];
    int bad;

    if (argc != 3) {
        fprintf(stderr, "usage: %s <input> <output>\n", argv[0]);
        return 1;
    }
    in = fopen(argv[1], "rb");
    if (!in) return 1;
    if (read_all(in, &n, sizeof n) || read_all(in, &beta, sizeof beta) || n <= 0 || n % SL_CHUNK != 0) {
        fclose(in);
        return 1;
    }
    chunks = n / SL_CHUNK;
    dense = (size_t)n * sizeof(float);
    pbytes = (size_t)chunks * SL_PAYLOAD_BYTES;
    sbytes = (size_t)chunks * sizeof(float);
    h_delta = (float*)malloc(dense);
    h_theta = (float*)malloc(dense);
    h_ef = (float*)malloc(dense);
    h_out = (float*)malloc(dense);
    h_p1 = (uint8_t*)malloc(pbytes);
    h_p2 = (uint8_t*)malloc(pbytes);
    h_s1 = (float*)malloc(sbytes);
    h_s2 = (float*)malloc(sbytes);
    if (!h_delta || !h_theta || !h_ef || !h_out || !h_p1 || !h_p2 || !h_s1 || !h_s2) return 1;
    bad = read_all(in, h_delta, dense) || read_all(in, h_theta, dense);
    fclose(in);
    if (bad) return 1;

    HIP_OK(hipMalloc((void**)&d_delta, dense));
    HIP_OK(hipMalloc((void**)&d_theta, dense));
    HIP_OK(hipMalloc((void**)&d_ef, dense));
    HIP_OK(hipMalloc((void**)&d_out, dense));
    HIP_OK(hipMalloc((void**)&d_p1, pbytes));
    HIP_OK(hipMalloc((void**)&d_p2, pbytes));
    HIP_OK(hipMalloc((void**)&d_s1, sbytes));
    HIP_OK(hipMalloc((void**)&d_s2, sbytes));
    HIP_OK(hipMemcpy(d_delta, h_delta, dense, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_theta, h_theta, dense, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(d_ef, 0, dense));

    SL_OK_OR_EXIT(sl_compress(d_delta, d_ef, beta, d_p1, d_s1, n, NULL));
    SL_OK_OR_EXIT(sl_compress(d_delta, d_ef, beta, d_p2, d_s2, n, NULL));
    payloads[0] = d_p1;
    payloads[1] = d_p2;
    scales[0] = d_s1;
    scales[1] = d_s2;
    SL_OK_OR_EXIT(sl_aggregate(payloads, scales, 2, d_out, n, NULL));
    SL_OK_OR_EXIT(sl_apply_mean(d_theta, d_out, 2, n, NULL));
    HIP_OK(hipDeviceSynchronize());

    HIP_OK(hipMemcpy(h_p1, d_p1, pbytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_s1, d_s1, sbytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_p2, d_p2, pbytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_s2, d_s2, sbytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_ef, d_ef, dense, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_out, d_out, dense, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_theta, d_theta, dense, hipMemcpyDeviceToHost));

    out = fopen(argv[2], "wb");
    if (!out) return 1;
    bad = write_all(out, h_p1, pbytes) || write_all(out, h_s1, sbytes) || write_all(out, h_p2, pbytes) ||
          write_all(out, h_s2, sbytes) || write_all(out, h_ef, dense) || write_all(out, h_out, dense) ||
          write_all(out, h_theta, dense);
    if (fclose(out) != 0) bad = 1;

    (void)hipFree(d_delta);
    (void)hipFree(d_theta);
    (void)hipFree(d_ef);
    (void)hipFree(d_out);
    (void)hipFree(d_p1);
    (void)hipFree(d_p2);
    (void)hipFree(d_s1);
    (void)hipFree(d_s2);
    free(h_delta);
    free(h_theta);
    free(h_ef);
    free(h_out);
    free(h_p1);
    free(h_p2);
    free(h_s1);
    free(h_s2);
    if (bad) return 1;
    printf("OK %lld\n", (long long)n);
    return 0;
}
