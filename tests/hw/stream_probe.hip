// Measurement-only library: what the HBM delivers to plain streams with the
// fused Adam update's access shape and none of its arithmetic.  R fp32 input
// streams are each read once and W fp32 output streams each written once:
// 128-thread workgroups, one 512-element tile per workgroup, 16 bytes per
// lane and stream, non-temporal loads and stores, tiles taken in runs of
// 64 (32768 elements) per XCD, and optionally the same resident-workgroup
// limit the update uses (unused local data share reserved at launch).  The
// only arithmetic is a sum of the inputs, written (plus the stream's index)
// to every output; with no outputs it is kept live by an empty asm
// statement and stored only when the caller's `sink` flag is set.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

constexpr int kThreads = 128;
constexpr int kTile = 512;
constexpr uint32_t kXcds = 8;
constexpr uint32_t kRunTiles = 64;
constexpr int kMaxStreams = 4;

typedef float f32x4 __attribute__((ext_vector_type(4)));
#define PROBE_GLOBAL __attribute__((address_space(1)))

struct Streams {
    const float *in[kMaxStreams];
    float *out[kMaxStreams];
};

// Workgroups are handed to the XCDs round-robin; within each group of
// kXcds * kRunTiles workgroups, XCD x takes kRunTiles consecutive tiles.
__device__ __forceinline__ uint32_t probe_tile(uint32_t b, uint32_t grid)
{
    constexpr uint32_t group = kXcds * kRunTiles;
    if (b >= grid - grid % group) return b;
    const uint32_t r = b % group;
    return b - r + (r % kXcds) * kRunTiles + r / kXcds;
}

template <int R, int W>
__global__ __launch_bounds__(kThreads) void stream_probe(Streams s, int sink)
{
    const uint32_t t = probe_tile(blockIdx.x, gridDim.x);
    const size_t q = size_t(t) * (kTile / 4) + threadIdx.x;  // f32x4 index
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < R; ++k)
        acc += __builtin_nontemporal_load((const PROBE_GLOBAL f32x4 *)(s.in[k]) + q);
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const f32x4 v = acc + float(k);
        __builtin_nontemporal_store(v, (PROBE_GLOBAL f32x4 *)(s.out[k]) + q);
    }
    if constexpr (W == 0) {
        // the sum is an operand of an empty asm statement, so the loads
        // cannot be dropped or moved under the flag
        asm volatile("" ::"v"(acc.x), "v"(acc.y), "v"(acc.z), "v"(acc.w));
        if (sink) ((PROBE_GLOBAL f32x4 *)(s.out[0]))[q] = acc;
    }
}

typedef void (*ProbeFn)(Streams, int);

template <int R, int W>
constexpr ProbeFn fn_of() { return stream_probe<R, W>; }

// [R][W], R, W in 0..4; (0, 0) is not a probe.
constexpr ProbeFn kProbes[kMaxStreams + 1][kMaxStreams + 1] = {
    {nullptr, fn_of<0, 1>(), fn_of<0, 2>(), fn_of<0, 3>(), fn_of<0, 4>()},
    {fn_of<1, 0>(), fn_of<1, 1>(), fn_of<1, 2>(), fn_of<1, 3>(), fn_of<1, 4>()},
    {fn_of<2, 0>(), fn_of<2, 1>(), fn_of<2, 2>(), fn_of<2, 3>(), fn_of<2, 4>()},
    {fn_of<3, 0>(), fn_of<3, 1>(), fn_of<3, 2>(), fn_of<3, 3>(), fn_of<3, 4>()},
    {fn_of<4, 0>(), fn_of<4, 1>(), fn_of<4, 2>(), fn_of<4, 3>(), fn_of<4, 4>()},
};

// ---------------------------------------------------------------------------
// In-place mixes: the update's own streams, read and written where the update
// reads and writes them.  Per 4-element lane group: load m, v, g, p (and the
// remainders), store m, v, p (and the remainders) back unchanged, and write
// the param-out stream; PB, MB, GB, OB are the bytes per element of p, of m
// and v, of g and of p_out (0: none), REM adds a 2-byte remainder stream
// read and written like p.  Empty asm statements after the loads make every
// loaded value opaque, so a store of what was loaded is not dropped.
// ---------------------------------------------------------------------------
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int B>
struct Group;  // one lane group of a B-byte stream: 4 elements
template <>
struct Group<4> {
    u32x4 x;
};
template <>
struct Group<2> {
    u32x2 x;
};

template <int B>
__device__ __forceinline__ Group<B> load_group(const void *base, int64_t q)
{
    Group<B> g;
    g.x = __builtin_nontemporal_load((const PROBE_GLOBAL decltype(g.x) *)(base) + q);
    return g;
}

// After every load of the lane group is issued: the values become opaque
// (the first use waits for all loads at once).
template <int B>
__device__ __forceinline__ void opaque(Group<B> &g)
{
#pragma unroll
    for (int k = 0; k < int(sizeof(g.x) / 4); ++k) asm volatile("" : "+v"(g.x[k]));
}

template <int B>
__device__ __forceinline__ void store_group(void *base, int64_t q, Group<B> g)
{
    __builtin_nontemporal_store(g.x, (PROBE_GLOBAL decltype(g.x) *)(base) + q);
}

struct MixStreams {
    void *p, *rem, *m, *v;
    const void *g;
    void *p_out;
};

template <int PB, int MB, int GB, int OB, bool REM>
__global__ __launch_bounds__(kThreads) void stream_probe_mix(MixStreams s, int64_t groups)
{
    const uint32_t t = probe_tile(blockIdx.x, gridDim.x);
    const int64_t q = int64_t(t) * kThreads + threadIdx.x;
    if (q >= groups) return;
    Group<MB> m = load_group<MB>(s.m, q);
    Group<MB> v = load_group<MB>(s.v, q);
    Group<GB> g = load_group<GB>(s.g, q);
    Group<PB> p = load_group<PB>(s.p, q);
    Group<2> r;
    if constexpr (REM) r = load_group<2>(s.rem, q);
    opaque(m);
    opaque(v);
    opaque(g);
    opaque(p);
    if constexpr (REM) opaque(r);
    store_group<MB>(s.m, q, m);
    store_group<MB>(s.v, q, v);
    store_group<PB>(s.p, q, p);
    if constexpr (REM) store_group<2>(s.rem, q, r);
    if constexpr (OB != 0) {
        // the param-out stream gets a value built from p and g
        Group<OB> o;
#pragma unroll
        for (int k = 0; k < int(sizeof(o.x) / 4); ++k) o.x[k] = p.x[k % (sizeof(p.x) / 4)] ^ g.x[k % (sizeof(g.x) / 4)];
        store_group<OB>(s.p_out, q, o);
    } else {
        asm volatile("" ::"v"(g.x[0]));
    }
}

typedef void (*MixFn)(MixStreams, int64_t);

// The mixes of the workloads: (p, m/v, g, p_out bytes, remainders)
struct MixKind {
    int pb, mb, gb, ob;
    bool rem;
    MixFn fn;
};
constexpr MixKind kMixes[] = {
    {4, 4, 4, 0, false, stream_probe_mix<4, 4, 4, 0, false>},  // fp32 p, m, v, g
    {4, 4, 2, 0, false, stream_probe_mix<4, 4, 2, 0, false>},  // 16-bit g
    {4, 4, 2, 2, false, stream_probe_mix<4, 4, 2, 2, false>},  // 16-bit g and param-out
    {4, 4, 4, 4, false, stream_probe_mix<4, 4, 4, 4, false>},  // fp32 g and param-out
    {2, 4, 2, 0, true, stream_probe_mix<2, 4, 2, 0, true>},    // bf16 p + remainders, 16-bit g
    {2, 4, 2, 2, true, stream_probe_mix<2, 4, 2, 2, true>},    // ... and param-out
    {2, 2, 2, 2, false, stream_probe_mix<2, 2, 2, 2, false>},  // 16-bit p, m, v, g, param-out
    {2, 2, 2, 0, false, stream_probe_mix<2, 2, 2, 0, false>},  // 16-bit p, m, v, g
};

}  // namespace

extern "C" {

// Runs `launches` in-place probes over n elements of the streams p, rem, m,
// v, g, p_out (bytes per element pb, 2, mb, mb, gb, ob; rem and p_out
// nullable as `rem` and `ob` say), in the update's tile map, at most
// `wg_per_cu` workgroups per compute unit (0: no limit), on `stream`, and
// writes the mean launch time in milliseconds (HIP events on that stream) to
// *ms.  p, m, v and rem keep their values.  n must be a multiple of 4 and
// every pointer aligned for its 4-element group.  Returns 0, -1 for an
// invalid argument or a mix with no kernel, -4 for a HIP error.
int stream_probe_mix_run(int pb, int mb, int gb, int ob, int rem, void *p, void *remp, void *m, void *v,
                         const void *g, void *p_out, int64_t n, int wg_per_cu, int launches, hipStream_t stream,
                         float *ms)
{
    MixFn fn = nullptr;
    for (const MixKind &k : kMixes)
        if (k.pb == pb && k.mb == mb && k.gb == gb && k.ob == ob && k.rem == (rem != 0)) fn = k.fn;
    if (fn == nullptr || n <= 0 || n % 4 != 0 || launches <= 0 || wg_per_cu < 0 || ms == nullptr || p == nullptr ||
        m == nullptr || v == nullptr || g == nullptr || (rem && remp == nullptr) || (ob && p_out == nullptr))
        return -1;
    auto aligned = [](const void *x, int b) { return reinterpret_cast<uintptr_t>(x) % uintptr_t(4 * b) == 0; };
    if (!aligned(p, pb) || !aligned(m, mb) || !aligned(v, mb) || !aligned(g, gb) || (rem && !aligned(remp, 2)) ||
        (ob && !aligned(p_out, ob)))
        return -1;
    const int64_t groups = n / 4;
    const int64_t tiles = (groups + kThreads - 1) / kThreads;
    if (tiles * kThreads > int64_t(UINT32_MAX)) return -1;  // one dispatch
    MixStreams s = {p, remp, m, v, g, p_out};
    int device = 0, lds = 0;
    if (hipGetDevice(&device) != hipSuccess ||
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, device) != hipSuccess)
        return -4;
    const size_t reserve = wg_per_cu > 0 ? size_t(lds / wg_per_cu) / 512 * 512 : 0;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return -4;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return -4;
    }
    int rc = 0;
    if (hipEventRecord(e0, stream) != hipSuccess) rc = -4;
    for (int i = 0; i < launches && rc == 0; ++i) {
        hipLaunchKernelGGL(fn, dim3(uint32_t(tiles)), dim3(kThreads), reserve, stream, s, groups);
        if (hipGetLastError() != hipSuccess) rc = -4;
    }
    if (rc == 0 && (hipEventRecord(e1, stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                    hipEventElapsedTime(ms, e0, e1) != hipSuccess))
        rc = -4;
    if (rc == 0) *ms /= float(launches);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return rc;
}


// Runs `launches` probes of r input and w output streams of n floats each
// (n a positive multiple of 512, every pointer 16-byte aligned; with w = 0,
// out[0] must still hold n floats, written only if `sink`), at most
// `wg_per_cu` workgroups resident per compute unit (0: no limit), on
// `stream`, and writes the mean launch time in milliseconds (HIP events on
// that stream) to *ms.  Returns 0, -1 for an invalid argument, -4 for a HIP
// error.
int stream_probe_run(int r, int w, const float *const *in, float *const *out, int64_t n, int wg_per_cu,
                     int launches, int sink, hipStream_t stream, float *ms)
{
    if (r < 0 || r > kMaxStreams || w < 0 || w > kMaxStreams || r + w == 0 || n <= 0 || n % kTile != 0 ||
        n / kTile > INT32_MAX || launches <= 0 || wg_per_cu < 0 || ms == nullptr || out == nullptr ||
        out[0] == nullptr || (r > 0 && in == nullptr))
        return -1;
    Streams s = {};
    for (int k = 0; k < r; ++k) {
        if (in[k] == nullptr || reinterpret_cast<uintptr_t>(in[k]) % 16) return -1;
        s.in[k] = in[k];
    }
    for (int k = 0; k < (w > 0 ? w : 1); ++k) {
        if (out[k] == nullptr || reinterpret_cast<uintptr_t>(out[k]) % 16) return -1;
        s.out[k] = out[k];
    }
    int device = 0, lds = 0;
    if (hipGetDevice(&device) != hipSuccess ||
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, device) != hipSuccess)
        return -4;
    const size_t reserve = wg_per_cu > 0 ? size_t(lds / wg_per_cu) / 512 * 512 : 0;
    const dim3 grid(uint32_t(n / kTile));
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return -4;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return -4;
    }
    int rc = 0;
    if (hipEventRecord(e0, stream) != hipSuccess) rc = -4;
    for (int i = 0; i < launches && rc == 0; ++i) {
        hipLaunchKernelGGL(kProbes[r][w], grid, dim3(kThreads), reserve, stream, s, sink);
        if (hipGetLastError() != hipSuccess) rc = -4;
    }
    if (rc == 0 && (hipEventRecord(e1, stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                    hipEventElapsedTime(ms, e0, e1) != hipSuccess))
        rc = -4;
    if (rc == 0) *ms /= float(launches);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return rc;
}

}  // extern "C"
