/*
 * A plain C client of libpdq: device memory from hipMalloc, the library's C
 * entry points, no Python and no PyTorch.  Reads one case from a binary file,
 * runs the offline weight quantization, the static calibration, the prefill
 * linear and the decode linear on the default stream, and writes every output
 * to a binary file, for the GPU test that checks them against the oracle.
 *
 *   pdq_c_client <in> <out>
 *
 * in  (little-endian): int64 M, N, K, C; then float32 x[M*K], w[N*K],
 *     cal[C*K] (all row-major, K contiguous)
 * out: wq (pdq_weight_bytes(N, K) bytes), w_scale f32[N], colsum i32[N];
 *      prefill xq (pdq_act_bytes(M, K) bytes), x_scale f32[M], y u16[M*N],
 *      acc i32[M*N]; calibration minmax f32[2], S f32, Z i32; decode xq
 *      (pdq_act_bytes(M, K) bytes), y u16[M*N], acc i32[M*N], saturated u32.
 * Exit status 0 on success; 1 with a message on any failure.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "pdq.h"

static void die(const char* what) {
    fprintf(stderr, "pdq_c_client: %s\n", what);
    exit(1);
}

#define HIP_OK(call)                                   \
    do {                                               \
        if ((call) != hipSuccess) die(#call " failed"); \
    } while (0)

#define PDQ_OK_OR_DIE(call)                                                   \
    do {                                                                      \
        pdq_status s_ = (call);                                               \
        if (s_ != PDQ_OK) {                                                   \
            fprintf(stderr, "pdq_c_client: %s: %s\n", #call, pdq_status_string(s_)); \
            exit(1);                                                          \
        }                                                                     \
    } while (0)

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    HIP_OK(hipMalloc(&p, bytes ? bytes : 16));
    return p;
}

static void* read_exact(FILE* f, size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p || fread(p, 1, bytes, f) != bytes) die("short input file");
    return p;
}

/* device -> host -> file */
static void dump(FILE* f, const void* d, size_t bytes) {
    void* h = malloc(bytes ? bytes : 1);
    if (!h) die("out of host memory");
    HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    if (fwrite(h, 1, bytes, f) != bytes) die("write failed");
    free(h);
}

int main(int argc, char** argv) {
    if (argc != 3) die("usage: pdq_c_client <in> <out>");
    FILE* in = fopen(argv[1], "rb");
    if (!in) die("cannot open the input file");
    int64_t dims[4];
    if (fread(dims, sizeof(int64_t), 4, in) != 4) die("short input file");
    const int64_t M = dims[0], N = dims[1], K = dims[2], C = dims[3];
    if (M < 1 || N < 1 || K < 16 || C < 1) die("bad dimensions");
    float* hx = read_exact(in, (size_t)(M * K) * sizeof(float));
    float* hw = read_exact(in, (size_t)(N * K) * sizeof(float));
    float* hc = read_exact(in, (size_t)(C * K) * sizeof(float));
    fclose(in);

    const size_t wbytes = pdq_weight_bytes(N, K), abytes = pdq_act_bytes(M, K);
    float* x = dev_alloc((size_t)(M * K) * sizeof(float));
    float* w = dev_alloc((size_t)(N * K) * sizeof(float));
    float* cal = dev_alloc((size_t)(C * K) * sizeof(float));
    HIP_OK(hipMemcpy(x, hx, (size_t)(M * K) * sizeof(float), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(w, hw, (size_t)(N * K) * sizeof(float), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(cal, hc, (size_t)(C * K) * sizeof(float), hipMemcpyHostToDevice));

    int8_t* wq = dev_alloc(wbytes);
    float* w_scale = dev_alloc((size_t)N * sizeof(float));
    int32_t* colsum = dev_alloc((size_t)N * sizeof(int32_t));
    int8_t* xq = dev_alloc(abytes);
    float* x_scale = dev_alloc((size_t)M * sizeof(float));
    uint16_t* y = dev_alloc((size_t)(M * N) * sizeof(uint16_t));
    int32_t* acc = dev_alloc((size_t)(M * N) * sizeof(int32_t));
    float* minmax = dev_alloc(2 * sizeof(float));
    float* s_dev = dev_alloc(sizeof(float));
    int32_t* z_dev = dev_alloc(sizeof(int32_t));
    int8_t* xq_dec = dev_alloc(abytes);
    uint16_t* y_dec = dev_alloc((size_t)(M * N) * sizeof(uint16_t));
    int32_t* acc_dec = dev_alloc((size_t)(M * N) * sizeof(int32_t));
    uint32_t* sat = dev_alloc(sizeof(uint32_t));

    /* offline: the weight, once */
    PDQ_OK_OR_DIE(pdq_quantize_weight(w, PDQ_F32, N, K, K, wq, w_scale, colsum, NULL));
    /* prefill: per-token dynamic symmetric */
    PDQ_OK_OR_DIE(pdq_linear_prefill(x, PDQ_F32, M, K, K, wq, w_scale, NULL, N, xq, x_scale, y, N, acc, NULL));
    /* calibration: one batch, finalised */
    const float init[2] = {__builtin_inff(), -__builtin_inff()};
    HIP_OK(hipMemcpy(minmax, init, sizeof(init), hipMemcpyHostToDevice));
    PDQ_OK_OR_DIE(pdq_calibrate_static(cal, PDQ_F32, C, K, K, minmax, s_dev, z_dev, NULL));
    HIP_OK(hipDeviceSynchronize());
    float s = 0.0f;
    int32_t z = 0;
    HIP_OK(hipMemcpy(&s, s_dev, sizeof(s), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&z, z_dev, sizeof(z), hipMemcpyDeviceToHost));
    /* decode: per-tensor static asymmetric with that S and Z */
    const uint32_t zero = 0;
    HIP_OK(hipMemcpy(sat, &zero, sizeof(zero), hipMemcpyHostToDevice));
    PDQ_OK_OR_DIE(pdq_linear_decode(x, PDQ_F32, M, K, K, s, z, wq, w_scale, colsum, NULL, N, xq_dec, y_dec, N,
                                    acc_dec, sat, NULL));
    HIP_OK(hipDeviceSynchronize());

    FILE* out = fopen(argv[2], "wb");
    if (!out) die("cannot open the output file");
    dump(out, wq, wbytes);
    dump(out, w_scale, (size_t)N * sizeof(float));
    dump(out, colsum, (size_t)N * sizeof(int32_t));
    dump(out, xq, abytes);
    dump(out, x_scale, (size_t)M * sizeof(float));
    dump(out, y, (size_t)(M * N) * sizeof(uint16_t));
    dump(out, acc, (size_t)(M * N) * sizeof(int32_t));
    dump(out, minmax, 2 * sizeof(float));
    dump(out, s_dev, sizeof(float));
    dump(out, z_dev, sizeof(int32_t));
    dump(out, xq_dec, abytes);
    dump(out, y_dec, (size_t)(M * N) * sizeof(uint16_t));
    dump(out, acc_dec, (size_t)(M * N) * sizeof(int32_t));
    dump(out, sat, sizeof(uint32_t));
    if (fclose(out) != 0) die("write failed");
    printf("pdq_c_client: M=%lld N=%lld K=%lld S=%.9g Z=%d\n", (long long)M, (long long)N, (long long)K, (double)s,
           (int)z);
    return 0;
}
