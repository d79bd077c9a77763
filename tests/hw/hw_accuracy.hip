// Test-only library: accuracy of gfx950's fp32 square root and reciprocal
// instructions over every float input, against double-precision results.
// The scaled-state maxima pass bounds its approximate params by assuming
// both are within 2^-22 (relative) of the exact value for normal inputs,
// that a subnormal input to the reciprocal gives +inf or an accurate value,
// and that sqrt(0) = 0 and rcp(+inf) = 0.  The tests call hw_accuracy() and
// check those assumptions on the device they run on.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <vector>

namespace {

constexpr int kBlocksPerExp = 64;
constexpr int kThreads = 256;
constexpr uint32_t kPerBlock = (1u << 23) / kBlocksPerExp;

// Block (e, part) covers the positive floats with biased exponent e and
// significand bits in [part * kPerBlock, (part + 1) * kPerBlock): writes the
// largest relative errors of sqrt and rcp (finite, normal results only) and
// a count of rcp results, for inputs below 2^126, that are finite but off
// by more than 2^-23 (a subnormal input must give +inf or an accurate value).
__global__ __launch_bounds__(kThreads) void probe(double *err, uint32_t *loose)
{
    const uint32_t e = blockIdx.x / kBlocksPerExp;
    const uint32_t part = blockIdx.x % kBlocksPerExp;
    double es = 0.0, er = 0.0;
    uint32_t nl = 0;
    for (uint32_t i = threadIdx.x; i < kPerBlock; i += kThreads) {
        const float x = __uint_as_float((e << 23) | (part * kPerBlock + i));
        const double xs = sqrt(double(x)), xr = 1.0 / double(x);
        const double s = double(__builtin_amdgcn_sqrtf(x)), r = double(__builtin_amdgcn_rcpf(x));
        if (e != 0) es = fmax(es, fabs(s - xs) / xs);
        if (xr < 0x1p126) er = fmax(er, fabs(r - xr) / xr);  // normal reciprocal
        if (x < 0x1p126f && std::isfinite(r) && !(fabs(r - xr) <= 0x1p-23 * xr)) ++nl;
    }
    __shared__ double ss[kThreads], sr[kThreads];
    __shared__ uint32_t sl[kThreads];
    ss[threadIdx.x] = es;
    sr[threadIdx.x] = er;
    sl[threadIdx.x] = nl;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) {
            ss[threadIdx.x] = fmax(ss[threadIdx.x], ss[threadIdx.x + o]);
            sr[threadIdx.x] = fmax(sr[threadIdx.x], sr[threadIdx.x + o]);
            sl[threadIdx.x] += sl[threadIdx.x + o];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        err[2 * blockIdx.x] = ss[0];
        err[2 * blockIdx.x + 1] = sr[0];
        loose[blockIdx.x] = sl[0];
    }
}

__global__ void specials(float *o)
{
    if (threadIdx.x == 0) {
        o[0] = __builtin_amdgcn_sqrtf(0.0f);
        o[1] = __builtin_amdgcn_rcpf(__uint_as_float(0x7f800000u));
        o[2] = __builtin_amdgcn_rcpf(0.0f);
        o[3] = __builtin_amdgcn_sqrtf(__uint_as_float(0x7f800000u));
    }
}

}  // namespace

// per_exp_sqrt[e], per_exp_rcp[e] (e = biased exponent 0..254): largest
// relative error over that binade (sqrt: inputs of that binade; rcp: inputs
// of that binade whose reciprocal is a normal float).  *loose_rcp: finite
// reciprocals off by more than 2^-23, over all inputs below 2^126.  special[4]: sqrt(0),
// rcp(+inf), rcp(0), sqrt(+inf).  Returns 0, or -1 on a HIP error.
extern "C" int hw_accuracy(double *per_exp_sqrt, double *per_exp_rcp, uint32_t *loose_rcp, float *special)
{
    const int blocks = 255 * kBlocksPerExp;
    double *d_err = nullptr;
    uint32_t *d_loose = nullptr;
    float *d_sp = nullptr;
    int rc = -1;
    if (hipMalloc(&d_err, sizeof(double) * 2 * blocks) == hipSuccess &&
        hipMalloc(&d_loose, sizeof(uint32_t) * blocks) == hipSuccess && hipMalloc(&d_sp, 4 * sizeof(float)) == hipSuccess) {
        hipLaunchKernelGGL(probe, dim3(blocks), dim3(kThreads), 0, 0, d_err, d_loose);
        hipLaunchKernelGGL(specials, dim3(1), dim3(64), 0, 0, d_sp);
        std::vector<double> err(2 * blocks);
        std::vector<uint32_t> loose(blocks);
        if (hipGetLastError() == hipSuccess && hipDeviceSynchronize() == hipSuccess &&
            hipMemcpy(err.data(), d_err, sizeof(double) * 2 * blocks, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(loose.data(), d_loose, sizeof(uint32_t) * blocks, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(special, d_sp, 4 * sizeof(float), hipMemcpyDeviceToHost) == hipSuccess) {
            *loose_rcp = 0;
            for (int e = 0; e < 255; ++e) {
                per_exp_sqrt[e] = per_exp_rcp[e] = 0.0;
                for (int k = 0; k < kBlocksPerExp; ++k) {
                    per_exp_sqrt[e] = fmax(per_exp_sqrt[e], err[2 * (e * kBlocksPerExp + k)]);
                    per_exp_rcp[e] = fmax(per_exp_rcp[e], err[2 * (e * kBlocksPerExp + k) + 1]);
                    *loose_rcp += loose[e * kBlocksPerExp + k];
                }
            }
            rc = 0;
        }
    }
    (void)hipFree(d_err);
    (void)hipFree(d_loose);
    (void)hipFree(d_sp);
    return rc;
}
