// adam.hip - fused multi-tensor Adam / AdamW step for AMD Instinct MI355X
// (gfx950), behind the C ABI declared in include/adam.h.
//
// What is computed is defined by the apex patch "Enhance Distributed Fused
// Adam (#1794)" (DistAdamCapturableFunctor::local_step and operator()) and by
// apex distributed_fused_adam.py (step(), _bf16_rem_to_fp32); the header
// states it in full.  How it runs is this file's own design:
//
//  * The host turns a tensor list into a flat table of 64-byte work items.
//    Each item is a run of at most `chunk_elems` elements of one tensor with
//    every stream pointer already advanced to the run's start, so a
//    workgroup fetches one item with a single scalar load and needs no other
//    indirection.
//  * One persistent grid (a few workgroups per compute unit, sized from the
//    occupancy query) walks the table with a grid stride.  Items are
//    independent and no item is shared, so there is no synchronisation.
//  * Lanes move 4 consecutive elements per access: 16-byte loads and stores
//    for fp32 streams, 8-byte ones for bf16 / int16 streams, so a wave's
//    access covers 1 KiB (fp32) or 512 B (16-bit) of contiguous memory.
//    ADAM_UNROLL accesses per stream are issued before any arithmetic.
//    Loads and stores carry the non-temporal hint: every byte is touched
//    exactly once.
//  * Tensors whose buffers are not all aligned to 4 elements take a
//    per-element path (still coalesced, just narrower accesses); ragged
//    tails of aligned tensors are finished element by element.
//  * Per-step scalars are kernel arguments (non-capturable) or device loads
//    that every workgroup performs once (capturable): lr, the step counter,
//    the grad scale and the noop flag.  The capturable counter is advanced
//    by a one-lane kernel enqueued after the update, so every workgroup of
//    the update has read the old value before it changes.
//  * Arithmetic follows the header's expressions operation for operation in
//    binary32 (the library is built with -ffp-contract=off; division and
//    square root are the compiler's correctly rounded sequences; fp32
//    denormals are kept), so results match a scalar C evaluation bit for
//    bit and do not depend on chunking, grid size or alignment.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "adam.h"

#ifndef ADAM_UNROLL
#define ADAM_UNROLL 2
#endif
#ifndef ADAM_NONTEMPORAL
#define ADAM_NONTEMPORAL 1
#endif
#ifndef ADAM_BLOCK
#define ADAM_BLOCK 256
#endif

namespace {

constexpr int kBlock = ADAM_BLOCK;         // threads per workgroup (256: 4 wave64)
constexpr int kLaneElems = 4;              // elements per lane per access
constexpr int64_t kChunkQuantum = 4096;
constexpr int64_t kDefaultChunk = 16384;
constexpr int64_t kMaxChunk = int64_t(1) << 30;
constexpr int64_t kMaxNumel = int64_t(1) << 56;

enum : uint32_t { kItemVector = 1u };

// One run of consecutive elements of one tensor.  Pointers address the run's
// first element; absent streams are null.
struct alignas(64) WorkItem {
    void *p;
    int16_t *rem;
    float *m;
    float *v;
    const void *g;
    void *p_out;
    int32_t n;       // elements in the run, 1 .. chunk_elems
    uint32_t flags;  // kItemVector: every stream allows 4-element accesses
};
static_assert(sizeof(WorkItem) == 64, "work item must be one 64-byte record");

struct StepArgs {
    float lr, beta1, beta2, eps, weight_decay, bc1, bc2, grad_scale;
    const float *d_grad_scale;  // nullable: read on the device instead of grad_scale
    const float *d_lr;          // capturable only
    const int32_t *d_step;      // capturable only: the counter before this step
    const int32_t *d_noop;      // capturable only, nullable
    int32_t bias_correction;
};

// Per-workgroup constants of the update.
struct Coeffs {
    float lr, beta1, keep1, beta2, keep2, eps, wd, bc1, bc2, scale;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Bias correction.  beta^t by square-and-multiply over the bits of t, least
// significant bit first, in double; t <= 0 gives 1.  The same sequence of
// double multiplications runs on the host (non-capturable) and on the device
// (capturable), so both give the same bits.
// ---------------------------------------------------------------------------
__host__ __device__ inline double beta_power(double beta, int32_t t)
{
    double acc = 1.0;
    double sq = beta;
    for (uint32_t e = t > 0 ? uint32_t(t) : 0u; e != 0u; e >>= 1) {
        if (e & 1u) acc = acc * sq;
        sq = sq * sq;
    }
    return acc;
}

__host__ __device__ inline void corrections(float beta1, float beta2, int32_t t, int32_t on,
                                            float &bc1, float &bc2)
{
    if (on == 1) {
        bc1 = float(1.0 - beta_power(double(beta1), t));
        bc2 = float(1.0 - beta_power(double(beta2), t));
    } else {
        bc1 = 1.0f;
        bc2 = 1.0f;
    }
}

// ---------------------------------------------------------------------------
// Element arithmetic
// ---------------------------------------------------------------------------

// One element of the update.  MODE 0: decay joins the gradient (L2);
// MODE 1: decay joins the update (AdamW) using the param before the step.
template <int MODE>
__device__ __forceinline__ float update_element(float p, float g, float &m, float &v,
                                                const Coeffs &c)
{
    float x = g * c.scale;
    if constexpr (MODE == 0) x = x + c.wd * p;
    const float m1 = c.beta1 * m + c.keep1 * x;
    const float v1 = c.beta2 * v + c.keep2 * (x * x);
    const float m_hat = m1 / c.bc1;
    const float v_hat = v1 / c.bc2;
    float u = m_hat / (sqrtf(v_hat) + c.eps);
    if constexpr (MODE == 1) u = u + c.wd * p;
    m = m1;
    v = v1;
    return p - c.lr * u;
}

// bf16 bits (round to nearest, ties to even) of a float: adding 0x7FFF plus
// the lowest kept bit carries into the kept half exactly when the dropped
// half is above one half, or equal to it with an odd kept half.  NaN keeps
// sign and top payload and is made quiet.
__device__ __forceinline__ uint32_t bf16_bits_rne(float x)
{
    const uint32_t b = __float_as_uint(x);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (b >> 16) | 0x40u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Remainder encoding.  The fp32 master word is the bf16 half shifted up plus
// the sign-extended int16 remainder (mod 2^32): a negative remainder borrows
// one from the bf16 half, which is how the stored bf16 was rounded up.
__device__ __forceinline__ float master_from(uint32_t bf16, uint32_t rem16)
{
    const int32_t rem = int32_t(rem16 << 16) >> 16;
    return __uint_as_float((bf16 << 16) + uint32_t(rem));
}

__device__ __forceinline__ void master_to(float x, uint32_t &bf16, uint32_t &rem16)
{
    const uint32_t b = __float_as_uint(x);
    const int32_t low = int32_t(b << 16) >> 16;
    rem16 = b & 0xFFFFu;
    bf16 = (b - uint32_t(low)) >> 16;
}

// ---------------------------------------------------------------------------
// Memory access helpers.  Table pointers are generic; casting them to the
// global address space lets the compiler emit global (not flat) accesses.
// ---------------------------------------------------------------------------
#define ADAM_GLOBAL __attribute__((address_space(1)))

template <class T>
__device__ __forceinline__ T load_stream(const void *base, int idx)
{
    const ADAM_GLOBAL T *ptr = (const ADAM_GLOBAL T *)(base) + idx;
#if ADAM_NONTEMPORAL
    return __builtin_nontemporal_load(ptr);
#else
    return *ptr;
#endif
}

template <class T>
__device__ __forceinline__ void store_stream(void *base, int idx, T val)
{
    ADAM_GLOBAL T *ptr = (ADAM_GLOBAL T *)(base) + idx;
#if ADAM_NONTEMPORAL
    __builtin_nontemporal_store(val, ptr);
#else
    *ptr = val;
#endif
}

template <class T>
__device__ __forceinline__ T load_one(const void *base, int idx)
{
    return ((const ADAM_GLOBAL T *)(base))[idx];
}

template <class T>
__device__ __forceinline__ void store_one(void *base, int idx, T val)
{
    ((ADAM_GLOBAL T *)(base))[idx] = val;
}

// Kernel configuration (compile-time).
template <bool G_BF16, bool P_REM, bool OUT, int MODE, bool CAPT>
struct Config {
    static constexpr bool g_bf16 = G_BF16;
    static constexpr bool p_rem = P_REM;
    static constexpr bool out = OUT;
    static constexpr int mode = MODE;
    static constexpr bool capturable = CAPT;
};

// Four consecutive elements of one lane.
struct Quad {
    float p[4], m[4], v[4], g[4];
};

template <class C>
__device__ __forceinline__ void load_quad(Quad &q, const WorkItem &w, int vi)
{
    const f32x4 m = load_stream<f32x4>(w.m, vi);
    const f32x4 v = load_stream<f32x4>(w.v, vi);
    q.m[0] = m.x; q.m[1] = m.y; q.m[2] = m.z; q.m[3] = m.w;
    q.v[0] = v.x; q.v[1] = v.y; q.v[2] = v.z; q.v[3] = v.w;
    if constexpr (C::g_bf16) {
        const u32x2 g = load_stream<u32x2>(w.g, vi);
        q.g[0] = __uint_as_float(g.x << 16);
        q.g[1] = __uint_as_float(g.x & 0xFFFF0000u);
        q.g[2] = __uint_as_float(g.y << 16);
        q.g[3] = __uint_as_float(g.y & 0xFFFF0000u);
    } else {
        const f32x4 g = load_stream<f32x4>(w.g, vi);
        q.g[0] = g.x; q.g[1] = g.y; q.g[2] = g.z; q.g[3] = g.w;
    }
    if constexpr (C::p_rem) {
        const u32x2 h = load_stream<u32x2>(w.p, vi);
        const u32x2 r = load_stream<u32x2>(w.rem, vi);
        q.p[0] = master_from(h.x & 0xFFFFu, r.x & 0xFFFFu);
        q.p[1] = master_from(h.x >> 16, r.x >> 16);
        q.p[2] = master_from(h.y & 0xFFFFu, r.y & 0xFFFFu);
        q.p[3] = master_from(h.y >> 16, r.y >> 16);
    } else {
        const f32x4 p = load_stream<f32x4>(w.p, vi);
        q.p[0] = p.x; q.p[1] = p.y; q.p[2] = p.z; q.p[3] = p.w;
    }
}

template <class C>
__device__ __forceinline__ void compute_quad(Quad &q, const Coeffs &c)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) q.p[k] = update_element<C::mode>(q.p[k], q.g[k], q.m[k], q.v[k], c);
}

template <class C>
__device__ __forceinline__ void store_quad(const Quad &q, const WorkItem &w, int vi)
{
    store_stream<f32x4>(w.m, vi, f32x4{q.m[0], q.m[1], q.m[2], q.m[3]});
    store_stream<f32x4>(w.v, vi, f32x4{q.v[0], q.v[1], q.v[2], q.v[3]});
    if constexpr (C::p_rem) {
        uint32_t h[4], r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) master_to(q.p[k], h[k], r[k]);
        const u32x2 hv = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        store_stream<u32x2>(w.p, vi, hv);
        store_stream<u32x2>(w.rem, vi,
                            u32x2{r[0] | (r[1] << 16), r[2] | (r[3] << 16)});
        if constexpr (C::out) store_stream<u32x2>(w.p_out, vi, hv);
    } else {
        store_stream<f32x4>(w.p, vi, f32x4{q.p[0], q.p[1], q.p[2], q.p[3]});
        if constexpr (C::out) {
            const u32x2 o = u32x2{bf16_bits_rne(q.p[0]) | (bf16_bits_rne(q.p[1]) << 16),
                                  bf16_bits_rne(q.p[2]) | (bf16_bits_rne(q.p[3]) << 16)};
            store_stream<u32x2>(w.p_out, vi, o);
        }
    }
}

// One element at index i of a run, with plain (narrow) accesses.
template <class C>
__device__ __forceinline__ void single_element(const WorkItem &w, int i, const Coeffs &c)
{
    float g;
    if constexpr (C::g_bf16)
        g = __uint_as_float(uint32_t(load_one<uint16_t>(w.g, i)) << 16);
    else
        g = load_one<float>(w.g, i);
    float m = load_one<float>(w.m, i);
    float v = load_one<float>(w.v, i);
    if constexpr (C::p_rem) {
        const float p = master_from(load_one<uint16_t>(w.p, i), load_one<uint16_t>(w.rem, i));
        const float pn = update_element<C::mode>(p, g, m, v, c);
        uint32_t h, r;
        master_to(pn, h, r);
        store_one<uint16_t>(w.p, i, uint16_t(h));
        store_one<uint16_t>(w.rem, i, uint16_t(r));
        if constexpr (C::out) store_one<uint16_t>(w.p_out, i, uint16_t(h));
    } else {
        const float pn = update_element<C::mode>(load_one<float>(w.p, i), g, m, v, c);
        store_one<float>(w.p, i, pn);
        if constexpr (C::out) store_one<uint16_t>(w.p_out, i, uint16_t(bf16_bits_rne(pn)));
    }
    store_one<float>(w.m, i, m);
    store_one<float>(w.v, i, v);
}

template <class C>
__device__ __forceinline__ void run_vector(const WorkItem &w, const Coeffs &c)
{
    constexpr int U = ADAM_UNROLL;
    const int tid = threadIdx.x;
    const int nvec = w.n / kLaneElems;
    int base = 0;
    for (; base + kBlock * U <= nvec; base += kBlock * U) {
        Quad q[U];
#pragma unroll
        for (int u = 0; u < U; ++u) load_quad<C>(q[u], w, base + u * kBlock + tid);
#pragma unroll
        for (int u = 0; u < U; ++u) compute_quad<C>(q[u], c);
#pragma unroll
        for (int u = 0; u < U; ++u) store_quad<C>(q[u], w, base + u * kBlock + tid);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int vi = base + u * kBlock + tid;
        if (vi < nvec) {
            Quad q;
            load_quad<C>(q, w, vi);
            compute_quad<C>(q, c);
            store_quad<C>(q, w, vi);
        }
    }
    const int tail = w.n - nvec * kLaneElems;
    if (tid < tail) single_element<C>(w, nvec * kLaneElems + tid, c);
}

template <class C>
__device__ __forceinline__ void run_scalar(const WorkItem &w, const Coeffs &c)
{
    for (int i = threadIdx.x; i < w.n; i += kBlock) single_element<C>(w, i, c);
}

template <class C>
__global__ __launch_bounds__(kBlock) void adam_update(const WorkItem *__restrict__ items,
                                                       int64_t n_items, StepArgs a)
{
    Coeffs c;
    float lr = a.lr, bc1 = a.bc1, bc2 = a.bc2;
    if constexpr (C::capturable) {
        if (a.d_noop != nullptr && *a.d_noop == 1) return;
        const int32_t t = int32_t(uint32_t(*a.d_step) + 1u);
        corrections(a.beta1, a.beta2, t, a.bias_correction, bc1, bc2);
        lr = *a.d_lr;
    }
    c.lr = lr;
    c.beta1 = a.beta1;
    c.keep1 = 1.0f - a.beta1;
    c.beta2 = a.beta2;
    c.keep2 = 1.0f - a.beta2;
    c.eps = a.eps;
    c.wd = a.weight_decay;
    c.bc1 = bc1;
    c.bc2 = bc2;
    c.scale = a.d_grad_scale != nullptr ? *a.d_grad_scale : a.grad_scale;

    for (int64_t e = blockIdx.x; e < n_items; e += gridDim.x) {
        const WorkItem w = items[e];
        if (w.flags & kItemVector)
            run_vector<C>(w, c);
        else
            run_scalar<C>(w, c);
    }
}

// Advances the device step counter after the update unless the step was
// skipped.  One lane does the read-modify-write.
__global__ void adam_advance_counter(int32_t *d_step, const int32_t *d_noop)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        if (d_noop == nullptr || *d_noop != 1) d_step[0] = int32_t(uint32_t(d_step[0]) + 1u);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

typedef void (*KernelFn)(const WorkItem *, int64_t, StepArgs);

// Kernel table index: g_bf16 | p_rem << 1 | out << 2 | mode << 3 | capturable << 4.
template <int I>
constexpr KernelFn kernel_at()
{
    return adam_update<Config<(I & 1) != 0, (I & 2) != 0, (I & 4) != 0, (I >> 3) & 1, (I & 16) != 0>>;
}

template <int... I>
struct KernelTable {
    static constexpr KernelFn fns[sizeof...(I)] = {kernel_at<I>()...};
};
using AllKernels = KernelTable<0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19,
                               20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31>;

inline int kernel_index(bool g_bf16, bool p_rem, bool out, int mode, bool capturable)
{
    return int(g_bf16) | int(p_rem) << 1 | int(out) << 2 | (mode & 1) << 3 | int(capturable) << 4;
}

struct Plan {
    adam_tl_stats stats;
    std::vector<WorkItem> items;
};

bool valid_dtype_set(const adam_tl_desc &d)
{
    const bool g_ok = d.g == ADAM_DT_F32 || d.g == ADAM_DT_BF16;
    const bool out_ok = d.p_out == ADAM_DT_NONE || d.p_out == ADAM_DT_BF16;
    if (!g_ok || !out_ok) return false;
    if (d.with_remainders == 1) return d.p == ADAM_DT_BF16;
    if (d.with_remainders == 0) return d.p == ADAM_DT_F32;
    return false;
}

struct Span {
    uintptr_t lo, hi;
    bool read_only;
};

// Returns true when two spans overlap, other than two read-only ones.
bool spans_conflict(std::vector<Span> &spans)
{
    std::sort(spans.begin(), spans.end(), [](const Span &a, const Span &b) { return a.lo < b.lo; });
    uintptr_t end_any = 0, end_written = 0;
    for (const Span &s : spans) {
        if (s.lo < end_written) return true;
        if (!s.read_only && s.lo < end_any) return true;
        end_any = std::max(end_any, s.hi);
        if (!s.read_only) end_written = std::max(end_written, s.hi);
    }
    return false;
}

int make_plan(const adam_tensor *tensors, int64_t count, const adam_tl_desc *desc, Plan &plan,
              bool keep_items)
{
    if (desc == nullptr || count < 0 || (count > 0 && tensors == nullptr)) return ADAM_EINVAL;
    if (desc->reserved != 0 || desc->grid_blocks < 0) return ADAM_EINVAL;
    if (desc->with_remainders != 0 && desc->with_remainders != 1) return ADAM_EINVAL;
    if (!valid_dtype_set(*desc)) return ADAM_EDTYPE;
    const int64_t chunk = desc->chunk_elems == 0 ? kDefaultChunk : desc->chunk_elems;
    if (chunk <= 0 || chunk % kChunkQuantum != 0 || chunk > kMaxChunk) return ADAM_EINVAL;

    const bool rem = desc->with_remainders == 1;
    const bool out = desc->p_out == ADAM_DT_BF16;
    const size_t p_size = rem ? 2 : 4;
    const size_t g_size = desc->g == ADAM_DT_BF16 ? 2 : 4;

    adam_tl_stats st = {};
    st.tensors = count;
    st.chunk_elems = chunk;
    st.bytes_per_elem = int32_t(2 * (p_size + (rem ? 2 : 0) + 4 + 4) + g_size + (out ? 2 : 0));
    st.block_threads = kBlock;
    st.device = -1;

    std::vector<Span> spans;
    spans.reserve(size_t(count) * 6);
    for (int64_t k = 0; k < count; ++k) {
        const adam_tensor &t = tensors[k];
        if (t.numel < 0 || t.numel > kMaxNumel) return ADAM_EINVAL;
        if (t.numel == 0) continue;
        if (t.p == nullptr || t.m == nullptr || t.v == nullptr || t.g == nullptr) return ADAM_EINVAL;
        if ((t.rem != nullptr) != rem || (t.p_out != nullptr) != out) return ADAM_EINVAL;
        const uintptr_t n = uintptr_t(t.numel);
        spans.push_back({uintptr_t(t.p), uintptr_t(t.p) + n * p_size, false});
        spans.push_back({uintptr_t(t.m), uintptr_t(t.m) + n * 4, false});
        spans.push_back({uintptr_t(t.v), uintptr_t(t.v) + n * 4, false});
        spans.push_back({uintptr_t(t.g), uintptr_t(t.g) + n * g_size, true});
        if (rem) spans.push_back({uintptr_t(t.rem), uintptr_t(t.rem) + n * 2, false});
        if (out) spans.push_back({uintptr_t(t.p_out), uintptr_t(t.p_out) + n * 2, false});
        // every stream must be naturally aligned for its element type
        if (uintptr_t(t.p) % p_size || uintptr_t(t.m) % 4 || uintptr_t(t.v) % 4 ||
            uintptr_t(t.g) % g_size || (rem && uintptr_t(t.rem) % 2) ||
            (out && uintptr_t(t.p_out) % 2))
            return ADAM_EINVAL;
        const bool vec = uintptr_t(t.p) % (4 * p_size) == 0 && uintptr_t(t.m) % 16 == 0 &&
                         uintptr_t(t.v) % 16 == 0 && uintptr_t(t.g) % (4 * g_size) == 0 &&
                         (!rem || uintptr_t(t.rem) % 8 == 0) && (!out || uintptr_t(t.p_out) % 8 == 0);
        st.nonempty += 1;
        st.elements += t.numel;
        st.vector_tensors += vec ? 1 : 0;
        const int64_t n_chunks = (t.numel + chunk - 1) / chunk;
        st.chunks += n_chunks;
        if (!keep_items) continue;
        for (int64_t c = 0; c < n_chunks; ++c) {
            const int64_t off = c * chunk;
            WorkItem w = {};
            w.p = static_cast<char *>(t.p) + off * int64_t(p_size);
            w.rem = rem ? t.rem + off : nullptr;
            w.m = t.m + off;
            w.v = t.v + off;
            w.g = static_cast<const char *>(t.g) + off * int64_t(g_size);
            w.p_out = out ? static_cast<char *>(t.p_out) + off * 2 : nullptr;
            w.n = int32_t(std::min(chunk, t.numel - off));
            w.flags = vec ? kItemVector : 0u;
            plan.items.push_back(w);
        }
    }
    if (spans_conflict(spans)) return ADAM_EINVAL;
    plan.stats = st;
    return ADAM_OK;
}

// Makes `device` current for the life of the guard, restoring the caller's.
struct DeviceGuard {
    int previous = -1;
    bool switched = false;
    hipError_t status = hipSuccess;
    explicit DeviceGuard(int device)
    {
        status = hipGetDevice(&previous);
        if (status == hipSuccess && previous != device) {
            status = hipSetDevice(device);
            switched = status == hipSuccess;
        }
    }
    ~DeviceGuard()
    {
        if (switched) (void)hipSetDevice(previous);
    }
};

bool valid_hparams(const adam_hparams *hp)
{
    return hp != nullptr && (hp->mode == 0 || hp->mode == 1) &&
           (hp->bias_correction == 0 || hp->bias_correction == 1);
}

}  // namespace

struct adam_tl {
    adam_tl_stats stats;
    bool remainders;
    bool g_bf16;
    bool out;
    WorkItem *d_items;                 // device table, null when there is no work
    int32_t grid[4];                   // per (mode, capturable) kernel variant
};

namespace {

int launch_update(const adam_tl *tl, int mode, bool capturable, const StepArgs &args, hipStream_t stream)
{
    const int idx = kernel_index(tl->g_bf16, tl->remainders, tl->out, mode, capturable);
    const int grid = tl->grid[(mode & 1) | int(capturable) << 1];
    hipLaunchKernelGGL(AllKernels::fns[idx], dim3(grid), dim3(kBlock), 0, stream, tl->d_items,
                       tl->stats.chunks, args);
    return hipGetLastError() == hipSuccess ? ADAM_OK : ADAM_EHIP;
}

int host_step(const adam_tl *tl, const adam_hparams *hp, float lr, int32_t *step_io, float grad_scale,
              const float *d_grad_scale, hipStream_t stream, bool want_remainders)
{
    if (tl == nullptr || step_io == nullptr || !valid_hparams(hp)) return ADAM_EINVAL;
    if (tl->remainders != want_remainders) return ADAM_EINVAL;
    const int32_t before = *step_io;
    if (before < 0 || before == INT32_MAX) return ADAM_EINVAL;
    const int32_t t = before + 1;
    *step_io = t;  // the counter advances even for a list with no elements
    if (tl->stats.chunks == 0) return ADAM_OK;
    StepArgs a = {};
    a.lr = lr;
    a.beta1 = hp->beta1;
    a.beta2 = hp->beta2;
    a.eps = hp->eps;
    a.weight_decay = hp->weight_decay;
    a.grad_scale = grad_scale;
    a.d_grad_scale = d_grad_scale;
    a.bias_correction = hp->bias_correction;
    corrections(hp->beta1, hp->beta2, t, hp->bias_correction, a.bc1, a.bc2);
    DeviceGuard guard(tl->stats.device);
    int rc = guard.status == hipSuccess ? launch_update(tl, hp->mode, false, a, stream) : ADAM_EHIP;
    if (rc != ADAM_OK) *step_io = before;
    return rc;
}

}  // namespace

extern "C" {

int adam_abi_version(void) { return ADAM_ABI_VERSION; }

const char *adam_status_string(int status)
{
    switch (status) {
    case ADAM_OK: return "ok";
    case ADAM_EINVAL: return "invalid argument";
    case ADAM_EDTYPE: return "unsupported dtype combination";
    case ADAM_ENOMEM: return "out of memory";
    case ADAM_EHIP: return "HIP runtime or launch failure";
    default: return "unknown status";
    }
}

int adam_tl_plan(const adam_tensor *tensors, int64_t count, const adam_tl_desc *desc,
                 adam_tl_stats *stats)
{
    if (stats == nullptr) return ADAM_EINVAL;
    Plan plan;
    int rc;
    try {
        rc = make_plan(tensors, count, desc, plan, false);
    } catch (const std::bad_alloc &) {
        return ADAM_ENOMEM;
    }
    if (rc == ADAM_OK) *stats = plan.stats;
    return rc;
}

int adam_tl_build(const adam_tensor *tensors, int64_t count, const adam_tl_desc *desc,
                  hipStream_t stream, adam_tl **out)
{
    if (out == nullptr) return ADAM_EINVAL;
    *out = nullptr;
    Plan plan;
    int rc;
    try {
        rc = make_plan(tensors, count, desc, plan, true);
    } catch (const std::bad_alloc &) {
        return ADAM_ENOMEM;
    }
    if (rc != ADAM_OK) return rc;

    adam_tl *tl = new (std::nothrow) adam_tl();
    if (tl == nullptr) return ADAM_ENOMEM;
    tl->stats = plan.stats;
    tl->remainders = desc->with_remainders == 1;
    tl->g_bf16 = desc->g == ADAM_DT_BF16;
    tl->out = desc->p_out == ADAM_DT_BF16;
    tl->d_items = nullptr;
    for (int i = 0; i < 4; ++i) tl->grid[i] = 0;
    if (plan.items.empty()) {  // nothing to launch: no device state at all
        *out = tl;
        return ADAM_OK;
    }

    int device = 0, cus = 0;
    if (hipGetDevice(&device) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
        delete tl;
        return ADAM_EHIP;
    }
    tl->stats.device = device;
    for (int variant = 0; variant < 4; ++variant) {
        const int idx = kernel_index(tl->g_bf16, tl->remainders, tl->out, variant & 1, (variant & 2) != 0);
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, AllKernels::fns[idx], kBlock, 0) !=
            hipSuccess) {
            delete tl;
            return ADAM_EHIP;
        }
        int64_t grid = int64_t(std::max(per_cu, 1)) * std::max(cus, 1);
        if (desc->grid_blocks > 0) grid = desc->grid_blocks;
        grid = std::min<int64_t>(grid, plan.stats.chunks);
        tl->grid[variant] = int32_t(std::max<int64_t>(grid, 1));
    }
    tl->stats.grid_blocks = tl->grid[1];

    const size_t bytes = plan.items.size() * sizeof(WorkItem);
    if (hipMalloc(reinterpret_cast<void **>(&tl->d_items), bytes) != hipSuccess) {
        (void)hipGetLastError();
        delete tl;
        return ADAM_ENOMEM;
    }
    if (hipMemcpyAsync(tl->d_items, plan.items.data(), bytes, hipMemcpyHostToDevice, stream) !=
            hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipFree(tl->d_items);
        delete tl;
        return ADAM_EHIP;
    }
    *out = tl;
    return ADAM_OK;
}

void adam_tl_destroy(adam_tl *tl)
{
    if (tl == nullptr) return;
    if (tl->d_items != nullptr) {
        DeviceGuard guard(tl->stats.device);
        (void)hipFree(tl->d_items);
    }
    delete tl;
}

int adam_tl_info(const adam_tl *tl, adam_tl_stats *stats)
{
    if (tl == nullptr || stats == nullptr) return ADAM_EINVAL;
    *stats = tl->stats;
    return ADAM_OK;
}

int adam_step(const adam_tl *tl, const adam_hparams *hp, float lr, int32_t *step_io, float grad_scale,
              const float *d_grad_scale, hipStream_t stream)
{
    return host_step(tl, hp, lr, step_io, grad_scale, d_grad_scale, stream, false);
}

int adam_step_remainders(const adam_tl *tl, const adam_hparams *hp, float lr, int32_t *step_io,
                         float grad_scale, const float *d_grad_scale, hipStream_t stream)
{
    return host_step(tl, hp, lr, step_io, grad_scale, d_grad_scale, stream, true);
}

int adam_step_capturable(const adam_tl *tl, const adam_hparams *hp, const float *d_lr, int32_t *d_step,
                         const float *d_grad_scale, const int32_t *d_noop, hipStream_t stream)
{
    if (tl == nullptr || d_lr == nullptr || d_step == nullptr || !valid_hparams(hp)) return ADAM_EINVAL;
    if (tl->remainders) return ADAM_EINVAL;
    int device = tl->stats.device;
    if (device < 0 && hipGetDevice(&device) != hipSuccess) return ADAM_EHIP;
    DeviceGuard guard(device);
    if (guard.status != hipSuccess) return ADAM_EHIP;
    if (tl->stats.chunks > 0) {
        StepArgs a = {};
        a.beta1 = hp->beta1;
        a.beta2 = hp->beta2;
        a.eps = hp->eps;
        a.weight_decay = hp->weight_decay;
        a.grad_scale = 1.0f;
        a.d_grad_scale = d_grad_scale;
        a.d_lr = d_lr;
        a.d_step = d_step;
        a.d_noop = d_noop;
        a.bias_correction = hp->bias_correction;
        const int rc = launch_update(tl, hp->mode, true, a, stream);
        if (rc != ADAM_OK) return rc;
    }
    hipLaunchKernelGGL(adam_advance_counter, dim3(1), dim3(64), 0, stream, d_step, d_noop);
    return hipGetLastError() == hipSuccess ? ADAM_OK : ADAM_EHIP;
}

}  // extern "C"
