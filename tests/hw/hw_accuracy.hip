// Test-only library: accuracy of gfx950's fp32 square root and reciprocal
// instructions over every float input, against double-precision results.
// The scaled-state maxima pass bounds its approximate params by assuming
// both are within 2^-22 (relative) of the exact value for normal inputs,
// that a subnormal input to the reciprocal gives +inf or an accurate value,
// and that sqrt(0) = 0 and rcp(+inf) = 0.  The tests call hw_accuracy() and
// check those assumptions on the device they run on.  bf16_conversion()
// checks the other fact the kernels rely on: the float -> bf16 conversion
// instruction, which the one-pass scaled kernel stores with, gives the bits
// of round to nearest even for every float (NaN: sign and top payload kept,
// made quiet).
#include <hip/hip_runtime.h>
#include <algorithm>
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

constexpr uint32_t kBf16Blocks = 16384;
constexpr uint32_t kPerBf16Block = uint32_t((uint64_t(1) << 32) / kBf16Blocks);

// Block b covers the bit patterns [b * kPerBf16Block, (b + 1) * kPerBf16Block):
// counts those whose conversion by the instruction differs from round to
// nearest even (written out on the bits: add 0x7FFF plus the lowest kept
// bit, keep the high half; a NaN keeps sign and top payload, quiet bit set),
// and the smallest such pattern.
__global__ __launch_bounds__(kThreads) void bf16_probe(uint32_t *count, uint32_t *first)
{
    uint32_t n = 0, lo = 0xFFFFFFFFu;
    for (uint32_t i = threadIdx.x; i < kPerBf16Block; i += kThreads) {
        const uint32_t u = blockIdx.x * kPerBf16Block + i;
        float x = __uint_as_float(u);
        asm("" : "+v"(x));
        const uint32_t hw = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
        const uint32_t rne = (u & 0x7FFFFFFFu) > 0x7F800000u ? (u >> 16) | 0x40u : (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
        if (hw != rne) {
            ++n;
            lo = min(lo, u);
        }
    }
    __shared__ uint32_t sn[kThreads], sl[kThreads];
    sn[threadIdx.x] = n;
    sl[threadIdx.x] = lo;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) {
            sn[threadIdx.x] += sn[threadIdx.x + o];
            sl[threadIdx.x] = min(sl[threadIdx.x], sl[threadIdx.x + o]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        count[blockIdx.x] = sn[0];
        first[blockIdx.x] = sl[0];
    }
}

}  // namespace

// *mismatches: floats whose bf16 conversion by the instruction differs from
// round to nearest even, over all 2^32 bit patterns; *first: the smallest
// such pattern (0xFFFFFFFF when there is none).  Returns 0, or -1 on a HIP
// error.
extern "C" int bf16_conversion(uint64_t *mismatches, uint32_t *first)
{
    uint32_t *d_count = nullptr, *d_first = nullptr;
    int rc = -1;
    if (hipMalloc(&d_count, sizeof(uint32_t) * kBf16Blocks) == hipSuccess &&
        hipMalloc(&d_first, sizeof(uint32_t) * kBf16Blocks) == hipSuccess) {
        hipLaunchKernelGGL(bf16_probe, dim3(kBf16Blocks), dim3(kThreads), 0, 0, d_count, d_first);
        std::vector<uint32_t> count(kBf16Blocks), lo(kBf16Blocks);
        if (hipGetLastError() == hipSuccess && hipDeviceSynchronize() == hipSuccess &&
            hipMemcpy(count.data(), d_count, sizeof(uint32_t) * kBf16Blocks, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(lo.data(), d_first, sizeof(uint32_t) * kBf16Blocks, hipMemcpyDeviceToHost) == hipSuccess) {
            *mismatches = 0;
            *first = 0xFFFFFFFFu;
            for (uint32_t b = 0; b < kBf16Blocks; ++b) {
                *mismatches += count[b];
                *first = std::min(*first, lo[b]);
            }
            rc = 0;
        }
    }
    (void)hipFree(d_count);
    (void)hipFree(d_first);
    return rc;
}

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
