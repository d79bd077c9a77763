/* A C99 client that runs the update on the GPU through the C ABI with only
 * the HIP runtime: reads one fp32 tensor and hyperparameters from a file,
 * copies them to the device, runs `steps` calls of adam_step on a stream of
 * its own, and writes the updated p, m, v and the host step counter back.
 *
 *   gpu_step IN OUT [two-buffer]
 *   IN : int64 n; float lr, beta1, beta2, eps, wd, grad_scale;
 *        int32 mode, bias_correction, steps; float32 p[n], m[n], v[n], g[n]
 *   OUT: float32 p[n], m[n], v[n]; int32 step
 * With "two-buffer" the handle is built by adam_tl_build_two_buffer with a
 * second set of p, m, v, and the state is read back from set (step & 1).
 * Exit status 0 on success; a failing call prints its status and exits 1. */
#include <stdio.h>
#include <stdlib.h>

#include "adam.h"

#define CHECK_HIP(x)                                                           \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
            return 1;                                                          \
        }                                                                      \
    } while (0)

#define CHECK_ADAM(x)                                                          \
    do {                                                                       \
        int s_ = (x);                                                          \
        if (s_ != ADAM_OK) {                                                   \
            fprintf(stderr, "%s: %s\n", #x, adam_status_string(s_));           \
            return 1;                                                          \
        }                                                                      \
    } while (0)

static int read_all(FILE *f, void *dst, size_t bytes) { return fread(dst, 1, bytes, f) == bytes; }

int main(int argc, char **argv)
{
    FILE *in, *out;
    int64_t n;
    float hf[6];
    int32_t hi[3];
    float *h[4];
    float *d[4];
    float *d2[3] = {NULL, NULL, NULL};
    int two = 0;
    int i, k;
    int32_t step = 0;
    adam_tensor t, t2;
    adam_tl_desc desc = {ADAM_DT_F32, ADAM_DT_F32, ADAM_DT_NONE, 0, 0, 0, 0, 0, 0};
    adam_hparams hp;
    adam_tl *tl = NULL;
    hipStream_t stream;

    if (argc == 4 && argv[3][0] == 't') two = 1;
    else if (argc != 3) return 2;
    in = fopen(argv[1], "rb");
    if (in == NULL || !read_all(in, &n, sizeof n) || !read_all(in, hf, sizeof hf) || !read_all(in, hi, sizeof hi))
        return 2;
    if (n <= 0 || n > ((int64_t)1 << 28)) return 2;
    for (i = 0; i < 4; ++i) {
        h[i] = (float *)malloc((size_t)n * sizeof(float));
        if (h[i] == NULL || !read_all(in, h[i], (size_t)n * sizeof(float))) return 2;
    }
    fclose(in);

    CHECK_HIP(hipStreamCreate(&stream));
    for (i = 0; i < 4; ++i) {
        CHECK_HIP(hipMalloc((void **)&d[i], (size_t)n * sizeof(float)));
        CHECK_HIP(hipMemcpy(d[i], h[i], (size_t)n * sizeof(float), hipMemcpyHostToDevice));
    }
    t.p = d[0];
    t.rem = NULL;
    t.m = d[1];
    t.v = d[2];
    t.g = d[3];
    t.p_out = NULL;
    t.scales = NULL;
    t.numel = n;
    hp.beta1 = hf[1];
    hp.beta2 = hf[2];
    hp.eps = hf[3];
    hp.weight_decay = hf[4];
    hp.mode = hi[0];
    hp.bias_correction = hi[1];
    if (two) {
        for (i = 0; i < 3; ++i) CHECK_HIP(hipMalloc((void **)&d2[i], (size_t)n * sizeof(float)));
        t2 = t;
        t2.p = d2[0];
        t2.m = d2[1];
        t2.v = d2[2];
        t2.g = NULL;
        CHECK_ADAM(adam_tl_build_two_buffer(&t, &t2, 1, &desc, stream, &tl));
    } else {
        CHECK_ADAM(adam_tl_build(&t, 1, &desc, stream, &tl));
    }
    for (k = 0; k < hi[2]; ++k) CHECK_ADAM(adam_step(tl, &hp, hf[0], &step, hf[5], NULL, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    adam_tl_destroy(tl);

    out = fopen(argv[2], "wb");
    if (out == NULL) return 2;
    for (i = 0; i < 3; ++i) {
        const float *src = two && (step & 1) ? d2[i] : d[i];
        CHECK_HIP(hipMemcpy(h[i], src, (size_t)n * sizeof(float), hipMemcpyDeviceToHost));
        if (fwrite(h[i], sizeof(float), (size_t)n, out) != (size_t)n) return 2;
    }
    if (fwrite(&step, sizeof step, 1, out) != 1) return 2;
    fclose(out);
    for (i = 0; i < 4; ++i) {
        CHECK_HIP(hipFree(d[i]));
        free(h[i]);
    }
    for (i = 0; i < 3; ++i)
        if (d2[i] != NULL) CHECK_HIP(hipFree(d2[i]));
    CHECK_HIP(hipStreamDestroy(stream));
    return 0;
}
