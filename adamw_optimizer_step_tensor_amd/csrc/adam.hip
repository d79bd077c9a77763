// adam.hip - fused multi-tensor Adam / AdamW step for AMD Instinct MI355X
// (gfx950), behind the C ABI declared in include/adam.h.
//
// What is computed is defined by the apex patch "Enhance Distributed Fused
// Adam (#1794)" (DistAdamCapturableFunctor::local_step and operator()) and by
// apex distributed_fused_adam.py (step(), _bf16_rem_to_fp32, grad_norm,
// clip_grad_norm, _local_step_with_scaled_states, _apply_state_scale); the
// header states it in full.  How it runs is this file's own design:
//
//  * The host turns a tensor list into a table of 128-byte work items.  Each
//    item is a run of at most `chunk` elements (a power of two) of one tensor
//    with every stream pointer already advanced to the run's start.
//  * One launch covers the whole list with one 128-thread workgroup (two
//    waves) per 512-element tile.  Each lane moves exactly one 4-element
//    group per stream (16-byte fp32, 8-byte bf16 / fp16 / int16 accesses), so
//    a wave's access is 1 KiB (or 512 B) of contiguous memory.  Measured on
//    MI355X: 8-element lanes (16-byte accesses of the 16-bit streams, two
//    adjacent 16-byte accesses of the fp32 ones) run 10-25% slower on every
//    list with a 16-bit stream.  Workgroup b reads item t >> shift of tile
//    t = tile_of_block(b) (one 128-byte scalar load, shared through L2 by the
//    item's tiles) and updates tile t & (2^shift - 1) of it.
//  * XCD-aware order: the hardware hands workgroups to the 8 XCDs
//    round-robin; tile_of_block permutes each group of 8 x run workgroups so
//    that every XCD streams `run` consecutive tiles (32768 elements, 128 KiB
//    of each fp32 stream) while the 8 XCDs sit side by side.  Measured over
//    the 201-tensor, 30B-shard, ZeRO-bucket and remainder workloads: small
//    short-lived workgroups beat persistent or large-chunk ones on this
//    7-stream read/write pattern, and per-XCD runs of this length beat the
//    plain round-robin order (6.1-6.3 vs 5.7 TB/s on the 201-tensor step).
//  * Loads and stores carry the non-temporal hint: every byte is touched
//    exactly once (measured: 10-15% faster than without).
//  * Records start on a 128-byte boundary in every stream when one element
//    index gets there for all of them (true for views at equal offsets into
//    flat buffers, the usual layout), else where every stream is aligned for
//    its 4-element access: a tensor's first record carries `head`, the 0..63
//    leading elements before that point, which tile 0 of the record updates
//    element by element at negative indices.  Line-aligned tiles keep two
//    workgroups from writing parts of one cache line (measured on ragged
//    lists: 4% extra HBM traffic without it).  Tensors whose streams cannot
//    all be aligned at one element take a per-element path (still
//    coalesced, narrower accesses); the ragged tail of a tile is finished
//    element by element.
//  * Per-step scalars are kernel arguments (non-capturable).  The capturable
//    steps first run a one-lane prologue that reads the device lr, step,
//    grad scale and noop flag, advances the step (unless noop == 1), and
//    writes the resolved scalars, bias corrections included, to a 64-byte
//    block beside the work table; every tile then reads that one block.
//  * Two-buffer state: an item may also carry the byte offsets of a second
//    set of p, m, v (and remainder) buffers; a step then reads one set and
//    writes the other, chosen by the parity of the step counter (the host
//    counter, or the device counter through the capturable prologue's
//    block).  Measured on MI355X: writing the lines a tile has just read
//    costs ~5% of the HBM rate (the update, and a plain 4-read / 3-write
//    stream probe, both run ~5% faster with separate output buffers).
//  * Scaled 16-bit state needs each buffer's largest magnitude after the
//    update before any of it can be stored, so it takes two passes over the
//    same tiles: the first (one wave per tile) computes the update in
//    registers and writes each tile's three magnitude maxima, taking the
//    param through the hardware square root and reciprocal with an error
//    bound and recomputing exactly only the elements that can hold the
//    maximum; one workgroup per tensor folds its tiles' maxima and derives
//    the reciprocal scales; the second pass recomputes the exact update and
//    stores it with those; a one-lane-per-tensor kernel then writes the
//    scales.  (Folding with one atomic maximum per workgroup instead was
//    measured 8x slower: a tensor's ~1000 workgroups contend for one word.)
//    A large list's step runs in up to 16 pieces of consecutive tensors,
//    alternating between the caller's stream and a second stream of the
//    handle, each piece's maxima pass (VALU-bound) beside the previous
//    piece's store pass (HBM-bound); events fork and join the streams.
//  * Arithmetic follows the header's expressions operation for operation in
//    binary32 (the library is built with -ffp-contract=off; division and
//    square root are correctly rounded -- the compiler's sequences, or for
//    the two divisions by the step's bias corrections a double reciprocal
//    product proven to give the same bits; fp32 denormals are kept), so
//    results match a scalar C evaluation bit for bit and do not depend on
//    chunking or alignment.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <new>
#include <utility>
#include <vector>

#include "adam.h"

#ifndef ADAM_NONTEMPORAL
#define ADAM_NONTEMPORAL 1
#endif
#ifndef ADAM_BLOCK
#define ADAM_BLOCK 128
#endif
#ifndef ADAM_RUN_ELEMS
#define ADAM_RUN_ELEMS 32768
#endif
#ifndef ADAM_NORM_RUN_ELEMS
#define ADAM_NORM_RUN_ELEMS 65536
#endif

namespace {

constexpr int kBlock = ADAM_BLOCK;          // threads per workgroup
constexpr int kLane = 4;                    // elements per lane and stream
constexpr int kTile = kBlock * kLane;       // elements per workgroup
constexpr int64_t kMinChunk = 1024;
constexpr int64_t kMaxChunk = int64_t(1) << 30;
constexpr int64_t kAutoChunkMax = 65536;
constexpr int64_t kMaxNumel = int64_t(1) << 56;
constexpr int64_t kMaxGrid = int64_t(1) << 31;  // tiles of one list (32-bit tile indices)
// Tiles of one dispatch.  A dispatch packet counts its grid in work-items
// with 32 bits, so a dispatch of 128-thread workgroups holds fewer than 2^25
// of them (64-thread ones fewer than 2^26); larger lists are launched as
// several dispatches, each over consecutive tiles.  A multiple of the XCD
// group (8 XCDs x kRun tiles) keeps every dispatch but the last in the
// XCD-ordered tile map.
constexpr int64_t kDispatchTiles = (int64_t(1) << 25) - 512;
constexpr int64_t kMaxHead = 63;            // a 2-byte stream reaches a 128-byte boundary within 63 elements
constexpr int kRunElems = ADAM_RUN_ELEMS;   // elements each XCD updates before the next XCD's run
constexpr uint32_t kRun = uint32_t(kRunElems / kTile);
constexpr uint32_t kNormRun = ADAM_NORM_RUN_ELEMS / kTile;  // tiles per reduction workgroup
// Scaled state: a list of at least kPipelineMinTiles tiles (4M elements) in
// two or more tensors runs its step in up to kMaxPieces pieces of
// consecutive tensors, each piece at least kMinPieceTiles tiles (512K
// elements), pipelined so that one piece's store pass (bound by HBM) runs
// beside the next piece's maxima pass (bound by the VALU).  Measured on
// MI355X on the 1e9-element fp16-state shard: 4.29 ms in one piece, 4.12 ms
// in two, 4.02-4.06 ms in four; in one later process at most 2, 4, 6 and 8
// pieces gave 4.40, 4.32, 4.29 and 4.25 ms; in a third, 8, 16, 24 and 32
// pieces gave 4.12-4.15, 4.08-4.10, 4.13-4.17 and 4.23-4.24 ms.
constexpr int kMaxPieces = 16;
constexpr uint32_t kPipelineMinTiles = (1u << 22) / kTile;
constexpr uint32_t kMinPieceTiles = (1u << 19) / kTile;

// Pieces of a scaled step over `tensors` nonempty tensors and `tiles` tiles.
int piece_count(int64_t tensors, int64_t tiles)
{
    if (tensors < 2 || tiles < int64_t(kPipelineMinTiles)) return 1;
    return int(std::min<int64_t>(std::min<int64_t>(kMaxPieces, tensors), tiles / kMinPieceTiles));
}
static_assert(kBlock > kMaxHead, "tile 0 updates the head with one element per lane");
static_assert(kBlock % 64 == 0, "whole waves");
static_assert(kDispatchTiles % (8 * kRun) == 0 && kDispatchTiles * kBlock <= int64_t(UINT32_MAX),
              "a dispatch keeps whole XCD groups and a 32-bit work-item count");
static_assert(kMinChunk % kTile == 0 && kRunElems % kTile == 0 && ADAM_NORM_RUN_ELEMS % kTile == 0,
              "records and runs hold whole tiles");

// Element types: the adam_dtype values.
constexpr int kNone = ADAM_DT_NONE;
constexpr int kF32 = ADAM_DT_F32;
constexpr int kBF16 = ADAM_DT_BF16;
constexpr int kF16 = ADAM_DT_F16;

// How params and moments are stored (non-scaled update kernels).
constexpr int kParamF32 = 0;   // fp32 p, m, v
constexpr int kParamRem = 1;   // bf16 params + int16 remainders, fp32 m, v
constexpr int kParamBF16 = 2;  // bf16 p, m, v (16-bit state)
constexpr int kParamF16 = 3;   // fp16 p, m, v (16-bit state)

enum : uint32_t { kItemVector = 1u, kItemTwoBuffer = 2u };

// One run of consecutive elements of one tensor.  Pointers address the run's
// first element in the first buffer set; absent streams are null.
struct alignas(64) WorkItem {
    void *p;
    void *aux;       // int16 remainders (remainder mode), or the tensor's float[3] scales (scaled state)
    void *m;
    void *v;
    const void *g;
    void *p_out;
    int32_t n;       // elements in the run, 1 .. chunk
    uint32_t flags;  // kItemVector: every stream allows 4-element accesses; kItemTwoBuffer: alt is set
    int32_t head;    // elements just before the run, updated by its tile 0 (0..63)
    int32_t tensor;  // ordinal of the tensor among the non-empty ones
    // two-buffer state: byte offsets from p, aux (remainders), m, v to the
    // same elements of the second buffer set (multiples of 128), else 0
    int64_t alt[4];
    int64_t unused[4];
};
static_assert(sizeof(WorkItem) == 128, "work item must be one 128-byte record");

// Scalars of one capturable step, resolved on the device by the prologue.
struct alignas(64) StepBlock {
    double rbc1, rbc2;  // 1/bc1, 1/bc2 rounded to double
    float lr, scale, bc1, bc2;
    int32_t skip;       // the noop flag was 1: the update does nothing
    int32_t t;          // step used by this update
    int32_t side;       // two-buffer state: the buffer set read ((t - 1) & 1)
};

struct StepArgs {
    double rbc1, rbc2;  // 1/bc1, 1/bc2 rounded to double
    float lr, beta1, beta2, eps, weight_decay, bc1, bc2, grad_scale;
    const float *d_grad_scale;  // nullable: read on the device instead of grad_scale
    const StepBlock *block;     // capturable only
    int32_t side;               // two-buffer state, non-capturable: the buffer set read
};

// Per-workgroup constants of the update.
struct Coeffs {
    double rbc1, rbc2;
    float lr, beta1, keep1, beta2, keep2, eps, wd, bc1, bc2, scale;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Bias correction.  beta^t by square-and-multiply over the bits of t, least
// significant bit first, in double; t <= 0 gives 1.  The same sequence of
// double multiplications runs on the host (non-capturable) and on the device
// (capturable prologue), so both give the same bits.
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

// The corrections and their double reciprocals (see quotient_by below).
__host__ __device__ inline void step_corrections(float beta1, float beta2, int32_t t, int32_t on,
                                                 float &bc1, float &bc2, double &rbc1, double &rbc2)
{
    corrections(beta1, beta2, t, on, bc1, bc2);
    rbc1 = 1.0 / double(bc1);
    rbc2 = 1.0 / double(bc2);
}

// ---------------------------------------------------------------------------
// Element arithmetic
// ---------------------------------------------------------------------------

// The float quotient x / y for a y shared by every element, given r, the
// double nearest 1/y: float(double(x) * r).  This is x / y rounded to float,
// bit for bit, for every float x.  The double product is within 2^-52
// (relative) of x / y, while a quotient of two floats is never within 2^-49
// of a float rounding midpoint: a midpoint m has a 25-bit odd significand, so
// x - m*y is a non-zero multiple of 2^k with |m*y| < 2^(k+49) (and x / y is
// never exactly a midpoint); so both round to the same float.  Zeros,
// infinities, NaN, subnormal quotients and overflow follow from IEEE double
// arithmetic and the double -> float conversion.  Checked against float
// division for all 2^32 x and 36 divisors (bias corrections at several
// steps and betas, 1, values next to 0.5 and 1, a subnormal).  A convert, a
// double multiply and a convert replace the ~12-cycle division expansion:
// the ALU-bound scaled-state passes use it (10% faster); the HBM-bound
// update keeps the float division (the product form measured 1% slower
// there, both give the same bits).
__device__ __forceinline__ float quotient_by(float x, double r)
{
    return float(double(x) * r);
}

// One element of the update, in two halves.  MODE 0: decay joins the
// gradient (L2); MODE 1: decay joins the update (AdamW) using the param
// before the step.  RECIP: divide by the bias corrections through their
// double reciprocals (same bits, fewer instructions).
//
// moments: the new m and v (in place) and the bias-corrected m_hat, v_hat.
template <int MODE, bool RECIP = false>
__device__ __forceinline__ void moments(float p, float g, float &m, float &v, const Coeffs &c,
                                        float &m_hat, float &v_hat)
{
    float x = g * c.scale;
    if constexpr (MODE == 0) x = x + c.wd * p;
    const float m1 = c.beta1 * m + c.keep1 * x;
    const float v1 = c.beta2 * v + c.keep2 * (x * x);
    m_hat = RECIP ? quotient_by(m1, c.rbc1) : m1 / c.bc1;
    v_hat = RECIP ? quotient_by(v1, c.rbc2) : v1 / c.bc2;
    m = m1;
    v = v1;
}

// param_from: the new param from the param before the step and m_hat, v_hat.
template <int MODE>
__device__ __forceinline__ float param_from(float p, float m_hat, float v_hat, const Coeffs &c)
{
    float u = m_hat / (sqrtf(v_hat) + c.eps);
    if constexpr (MODE == 1) u = u + c.wd * p;
    return p - c.lr * u;
}

template <int MODE, bool RECIP = false>
__device__ __forceinline__ float update_element(float p, float g, float &m, float &v,
                                                const Coeffs &c)
{
    float m_hat, v_hat;
    moments<MODE, RECIP>(p, g, m, v, c, m_hat, v_hat);
    return param_from<MODE>(p, m_hat, v_hat, c);
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

// binary16 bits of a float and back, with the hardware conversions: the
// kernels run in round-to-nearest-even with fp16 and fp32 subnormals kept
// (the code object's default float mode), so float -> fp16 is the IEEE
// nearest-even cast (overflow to infinity, subnormal results kept, NaN stays
// NaN) and fp16 -> float is exact.  One instruction each, where an integer
// implementation costs 10-15: the scaled-state passes are ALU-bound (the
// hardware casts made the scaled step 7% faster than the integer form).
// The empty register constraint keeps the compiler from folding the float
// operation that produced x into the conversion: gfx950's mixed-precision
// multiply-add would round the exact product once, straight to fp16, where
// the method rounds it to float first (measured: 1 element in ~10^6 differs).
__device__ __forceinline__ uint32_t f16_bits_rne(float x)
{
    asm("" : "+v"(x));
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

__device__ __forceinline__ float f16_to_f32(uint32_t h)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// 16-bit storage types: bits -> float, float -> bits.
template <int T>
__device__ __forceinline__ float widen16(uint32_t h)
{
    static_assert(T == kBF16 || T == kF16, "16-bit type");
    if constexpr (T == kBF16)
        return __uint_as_float(h << 16);
    else
        return f16_to_f32(h);
}

template <int T>
__device__ __forceinline__ uint32_t narrow16(float x)
{
    static_assert(T == kBF16 || T == kF16, "16-bit type");
    if constexpr (T == kBF16)
        return bf16_bits_rne(x);
    else
        return f16_bits_rne(x);
}

// bf16 bits of a float through gfx950's float -> bf16 conversion
// instruction: the same bits as bf16_bits_rne for every float, NaN payloads
// included (compared over all 2^32 inputs on the GPU), in one instruction
// where the integer form takes five.  The one-pass scaled kernel stores
// with it (1% faster there); the two-pass store pass measured 3% slower
// with it and keeps the integer form.  The empty register constraint keeps
// the compiler from folding the producing operation into the conversion.
__device__ __forceinline__ uint32_t bf16_bits_hw(float x)
{
    asm("" : "+v"(x));
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// narrow16 with the bf16 conversion instruction (same bits).
template <int T>
__device__ __forceinline__ uint32_t narrow16_hw(float x)
{
    static_assert(T == kBF16 || T == kF16, "16-bit type");
    if constexpr (T == kBF16)
        return bf16_bits_hw(x);
    else
        return f16_bits_rne(x);
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

// A scaled tensor's three scales (p, m, v), the same for every lane and
// never written while a kernel that reads them runs: scalar loads through
// the constant address space, for the one-pass kernel.  They count apart
// from the vector loads, so waiting for them never waits for a vector load
// in flight (as a flat load, counted by both counters, or a vector load
// issued after others would).  The two passes, one short-lived tile per
// workgroup, measured faster reading them with a vector load (3.95 against
// 4.01 ms on the 1e9 shard).
#define ADAM_CONSTANT __attribute__((address_space(4)))
__device__ __forceinline__ void load_scales(const void *aux, float *sc)
{
    const ADAM_CONSTANT float *s = (const ADAM_CONSTANT float *)aux;
    sc[0] = s[0];
    sc[1] = s[1];
    sc[2] = s[2];
}

template <class T>
__device__ __forceinline__ void store_one(void *base, int idx, T val)
{
    ((ADAM_GLOBAL T *)(base))[idx] = val;
}

// Four consecutive 16-bit values of lane group gi (one 8-byte access), each
// widened to the low half of a uint32, and back.
__device__ __forceinline__ void load_u16x4(const void *base, int gi, uint32_t *x)
{
    const u32x2 q = load_stream<u32x2>(base, gi);
    x[0] = q.x & 0xFFFFu;
    x[1] = q.x >> 16;
    x[2] = q.y & 0xFFFFu;
    x[3] = q.y >> 16;
}

__device__ __forceinline__ void store_u16x4(void *base, int gi, const uint32_t *x)
{
    store_stream<u32x2>(base, gi, u32x2{x[0] | (x[1] << 16), x[2] | (x[3] << 16)});
}

__device__ __forceinline__ void load_f32x4(const void *base, int gi, float *x)
{
    const f32x4 q = load_stream<f32x4>(base, gi);
    x[0] = q.x;
    x[1] = q.y;
    x[2] = q.z;
    x[3] = q.w;
}

__device__ __forceinline__ void store_f32x4(void *base, int gi, const float *x)
{
    store_stream<f32x4>(base, gi, f32x4{x[0], x[1], x[2], x[3]});
}

// Gradients of type GT (fp32, bf16 or fp16) as float: a lane group, or one.
template <int GT>
__device__ __forceinline__ void load_grad4(const void *g, int gi, float *x)
{
    if constexpr (GT == kF32) {
        load_f32x4(g, gi, x);
    } else {
        uint32_t h[kLane];
        load_u16x4(g, gi, h);
#pragma unroll
        for (int k = 0; k < kLane; ++k) x[k] = widen16<GT>(h[k]);
    }
}

template <int GT>
__device__ __forceinline__ float load_grad1(const void *g, int i)
{
    if constexpr (GT == kF32)
        return load_one<float>(g, i);
    else
        return widen16<GT>(load_one<uint16_t>(g, i));
}

// ---------------------------------------------------------------------------
// The update kernel (fp32 params or bf16 params + remainders)
// ---------------------------------------------------------------------------

// Kernel configuration (compile-time).
template <int GT, int PK, int OT, int MODE, bool CAPT>
struct Config {
    static constexpr int gt = GT;     // gradient type
    static constexpr int pk = PK;     // kParamF32, kParamRem, kParamBF16 or kParamF16
    static constexpr int ot = OT;     // param-out type, kNone if absent
    static constexpr int mode = MODE;
    static constexpr bool capturable = CAPT;
    // the 16-bit type of p, m, v (16-bit state), else kNone
    static constexpr int st = PK == kParamBF16 ? kBF16 : PK == kParamF16 ? kF16 : kNone;
    static_assert(PK != kParamRem || OT == kNone || OT == kBF16, "remainder param-out is the new bf16 param");
};

// The param-out of a new param x (float), or for 16-bit state of the new
// stored bits h of type ST: the cast of that value to OT.
template <int OT, int ST>
__device__ __forceinline__ uint32_t out16(float x, uint32_t h)
{
    if constexpr (ST == kNone)
        return narrow16<OT>(x);
    else if constexpr (OT == ST)
        return h;
    else
        return narrow16<OT>(widen16<ST>(h));
}

// The four consecutive elements of lane group gi, updated in registers:
// every load is issued before any arithmetic.  p, aux, m and v are read
// through `in` and written through `out` (the same record unless the state
// has two buffer sets); g and p_out are the same in both.
template <class C>
__device__ __forceinline__ void update_group(const WorkItem &in, const WorkItem &out, int gi, const Coeffs &c)
{
    float p[kLane], m[kLane], v[kLane], g[kLane];
    uint32_t hp[kLane], hm[kLane], hv[kLane];
    if constexpr (C::st != kNone) {
        load_u16x4(in.m, gi, hm);
        load_u16x4(in.v, gi, hv);
    } else {
        load_f32x4(in.m, gi, m);
        load_f32x4(in.v, gi, v);
    }
    load_grad4<C::gt>(in.g, gi, g);
    if constexpr (C::pk == kParamRem) {
        uint32_t r[kLane];
        load_u16x4(in.p, gi, hp);
        load_u16x4(in.aux, gi, r);
#pragma unroll
        for (int k = 0; k < kLane; ++k) p[k] = master_from(hp[k], r[k]);
    } else if constexpr (C::st != kNone) {
        load_u16x4(in.p, gi, hp);
#pragma unroll
        for (int k = 0; k < kLane; ++k) {
            p[k] = widen16<C::st>(hp[k]);
            m[k] = widen16<C::st>(hm[k]);
            v[k] = widen16<C::st>(hv[k]);
        }
    } else {
        load_f32x4(in.p, gi, p);
    }
#pragma unroll
    for (int k = 0; k < kLane; ++k) p[k] = update_element<C::mode>(p[k], g[k], m[k], v[k], c);

    if constexpr (C::st != kNone) {
#pragma unroll
        for (int k = 0; k < kLane; ++k) {
            hm[k] = narrow16<C::st>(m[k]);
            hv[k] = narrow16<C::st>(v[k]);
            hp[k] = narrow16<C::st>(p[k]);
        }
        store_u16x4(out.m, gi, hm);
        store_u16x4(out.v, gi, hv);
        store_u16x4(out.p, gi, hp);
    } else {
        store_f32x4(out.m, gi, m);
        store_f32x4(out.v, gi, v);
    }
    if constexpr (C::pk == kParamRem) {
        uint32_t r[kLane];
#pragma unroll
        for (int k = 0; k < kLane; ++k) master_to(p[k], hp[k], r[k]);
        store_u16x4(out.p, gi, hp);
        store_u16x4(out.aux, gi, r);
        if constexpr (C::ot != kNone) store_u16x4(out.p_out, gi, hp);
    } else {
        if constexpr (C::pk == kParamF32) store_f32x4(out.p, gi, p);
        if constexpr (C::ot == kF32) {
            float o[kLane];
#pragma unroll
            for (int k = 0; k < kLane; ++k) {
                if constexpr (C::st == kNone)
                    o[k] = p[k];
                else
                    o[k] = widen16<C::st>(hp[k]);
            }
            store_f32x4(out.p_out, gi, o);
        } else if constexpr (C::ot != kNone) {
            uint32_t o[kLane];
#pragma unroll
            for (int k = 0; k < kLane; ++k) o[k] = out16<C::ot, C::st>(p[k], hp[k]);
            store_u16x4(out.p_out, gi, o);
        }
    }
}

// One element at index i of an item, with plain (narrow) accesses; `in`
// and `out` as for update_group.
template <class C>
__device__ __forceinline__ void update_single(const WorkItem &in, const WorkItem &out, int i, const Coeffs &c)
{
    const float g = load_grad1<C::gt>(in.g, i);
    if constexpr (C::pk == kParamRem) {
        float m = load_one<float>(in.m, i);
        float v = load_one<float>(in.v, i);
        const float p = master_from(load_one<uint16_t>(in.p, i), load_one<uint16_t>(in.aux, i));
        const float pn = update_element<C::mode>(p, g, m, v, c);
        uint32_t h, r;
        master_to(pn, h, r);
        store_one<uint16_t>(out.p, i, uint16_t(h));
        store_one<uint16_t>(out.aux, i, uint16_t(r));
        if constexpr (C::ot != kNone) store_one<uint16_t>(out.p_out, i, uint16_t(h));
        store_one<float>(out.m, i, m);
        store_one<float>(out.v, i, v);
    } else if constexpr (C::st != kNone) {
        float m = widen16<C::st>(load_one<uint16_t>(in.m, i));
        float v = widen16<C::st>(load_one<uint16_t>(in.v, i));
        const float pn = update_element<C::mode>(widen16<C::st>(load_one<uint16_t>(in.p, i)), g, m, v, c);
        const uint32_t h = narrow16<C::st>(pn);
        store_one<uint16_t>(out.m, i, uint16_t(narrow16<C::st>(m)));
        store_one<uint16_t>(out.v, i, uint16_t(narrow16<C::st>(v)));
        store_one<uint16_t>(out.p, i, uint16_t(h));
        if constexpr (C::ot == kF32)
            store_one<float>(out.p_out, i, widen16<C::st>(h));
        else if constexpr (C::ot != kNone)
            store_one<uint16_t>(out.p_out, i, uint16_t(out16<C::ot, C::st>(pn, h)));
    } else {
        float m = load_one<float>(in.m, i);
        float v = load_one<float>(in.v, i);
        const float pn = update_element<C::mode>(load_one<float>(in.p, i), g, m, v, c);
        store_one<float>(out.p, i, pn);
        if constexpr (C::ot == kF32)
            store_one<float>(out.p_out, i, pn);
        else if constexpr (C::ot != kNone)
            store_one<uint16_t>(out.p_out, i, uint16_t(narrow16<C::ot>(pn)));
        store_one<float>(out.m, i, m);
        store_one<float>(out.v, i, v);
    }
}

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on
// XCD b % 8).  Each group of 8 * RUN workgroups is permuted so that every XCD
// updates RUN consecutive tiles; a grid's last partial group keeps the
// identity.  The map is a bijection on [0, grid).
constexpr uint32_t kXcds = 8;

template <uint32_t RUN>
__device__ __forceinline__ uint32_t tile_of_block(uint32_t b, uint32_t grid)
{
    if constexpr (RUN > 1) {
        constexpr uint32_t group = kXcds * RUN;
        if (b < grid - grid % group) {
            const uint32_t r = b % group;
            return (b - r) + (r % kXcds) * RUN + r / kXcds;
        }
    }
    return b;
}

// The per-workgroup constants of a non-capturable step.
__device__ __forceinline__ Coeffs host_coeffs(const StepArgs &a)
{
    Coeffs c;
    c.lr = a.lr;
    c.scale = a.d_grad_scale != nullptr ? *a.d_grad_scale : a.grad_scale;
    c.rbc1 = a.rbc1;
    c.rbc2 = a.rbc2;
    c.bc1 = a.bc1;
    c.bc2 = a.bc2;
    c.beta1 = a.beta1;
    c.keep1 = 1.0f - a.beta1;
    c.beta2 = a.beta2;
    c.keep2 = 1.0f - a.beta2;
    c.eps = a.eps;
    c.wd = a.weight_decay;
    return c;
}

// The constants of a step of the scaled-state kernels: from the host
// arguments, or, when the step is capturable (a.block set), from the block
// the prologue resolved.  False when that block says the step is a noop.
__device__ __forceinline__ bool step_coeffs(const StepArgs &a, Coeffs &c)
{
    c = host_coeffs(a);
    if (a.block != nullptr) {
        const StepBlock s = *a.block;
        if (s.skip) return false;
        c.lr = s.lr;
        c.scale = s.scale;
        c.rbc1 = s.rbc1;
        c.rbc2 = s.rbc2;
        c.bc1 = s.bc1;
        c.bc2 = s.bc2;
    }
    return true;
}

// The update: workgroup b of a dispatch that starts at tile `tile0` handles
// tile t = tile0 + tile_of_block(b): tile (t & mask) of work item (t >> shift).
template <class C>
__global__ __launch_bounds__(kBlock) void adam_update(const WorkItem *__restrict__ items,
                                                       uint32_t shift, uint32_t tile0, StepArgs a)
{
    const uint32_t b = tile0 + tile_of_block<kRun>(blockIdx.x, gridDim.x);
    const WorkItem w = items[b >> shift];
    const int start = int(b & ((1u << shift) - 1u)) * kTile;
    if (start >= w.n) return;  // past the end of a tensor's last item

    Coeffs c = host_coeffs(a);
    int32_t side = a.side;
    if constexpr (C::capturable) {
        const StepBlock s = *a.block;
        if (s.skip) return;
        c.lr = s.lr;
        c.scale = s.scale;
        c.rbc1 = s.rbc1;
        c.rbc2 = s.rbc2;
        c.bc1 = s.bc1;
        c.bc2 = s.bc2;
        side = s.side;
    }
    // two-buffer state: read the set `side`, write the other one
    WorkItem in = w, out = w;
    if (w.flags & kItemTwoBuffer) {
        void *p1 = static_cast<char *>(w.p) + w.alt[0];
        void *aux1 = w.aux != nullptr ? static_cast<char *>(w.aux) + w.alt[1] : nullptr;
        void *m1 = static_cast<char *>(w.m) + w.alt[2];
        void *v1 = static_cast<char *>(w.v) + w.alt[3];
        if (side) {
            in.p = p1;
            in.aux = aux1;
            in.m = m1;
            in.v = v1;
        } else {
            out.p = p1;
            out.aux = aux1;
            out.m = m1;
            out.v = v1;
        }
    }

    const int n = min(kTile, w.n - start);
    const int tid = threadIdx.x;
    if (w.flags & kItemVector) {
        if (start == 0 && tid < w.head) update_single<C>(in, out, tid - w.head, c);
        const int groups = n / kLane;
        if (tid < groups) update_group<C>(in, out, start / kLane + tid, c);
        // the 0..3 elements after the last whole group of a ragged tile
        if (tid < n - groups * kLane) update_single<C>(in, out, start + groups * kLane + tid, c);
    } else {
        for (int i = tid; i < n; i += kBlock) update_single<C>(in, out, start + i, c);
    }
}

// Capturable prologue (one lane): resolves the step's scalars on the device.
// The counter advances here unless the noop flag is 1; the update reads the
// resolved block, never the counter.
__global__ void adam_capture_prologue(StepBlock *block, const float *d_lr, int32_t *d_step,
                                      const float *d_grad_scale, const int32_t *d_noop, float beta1,
                                      float beta2, int32_t bias_correction)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    const bool skip = d_noop != nullptr && *d_noop == 1;
    const int32_t t = int32_t(uint32_t(*d_step) + (skip ? 0u : 1u));
    if (!skip) *d_step = t;
    if (block == nullptr) return;  // a list with no elements: only the counter
    StepBlock s;
    s.skip = skip ? 1 : 0;
    s.t = t;
    s.side = int32_t((uint32_t(t) - 1u) & 1u);
    s.lr = *d_lr;
    s.scale = d_grad_scale != nullptr ? *d_grad_scale : 1.0f;
    step_corrections(beta1, beta2, t, bias_correction, s.bc1, s.bc2, s.rbc1, s.rbc2);
    *block = s;
}

// ---------------------------------------------------------------------------
// Scaled 16-bit state (apex distributed_fused_adam.py,
// _local_step_with_scaled_states and _apply_state_scale).  p, m, v of type ST
// times the tensor's three float scales are the fp32 values; the step
// updates those and stores them again with new scales.
// ---------------------------------------------------------------------------

// Half the largest finite value of the state type, as a float.
template <int ST>
__host__ __device__ constexpr float scaled_limit()
{
    // bfloat16: (2 - 2^-7) * 2^127 / 2 (bits 0x7EFF0000);  binary16: 65504 / 2
    return ST == kBF16 ? 1.69476569462576773e38f : 32752.0f;
}

template <int ST, int GT, int OT, int MODE, int PASS>
struct ScaledConfig {
    static constexpr int st = ST;      // state type of p, m, v
    static constexpr int gt = GT;
    static constexpr int ot = OT;
    static constexpr int mode = MODE;
    static constexpr int pass = PASS;  // 0: fold maxima; 1: store
};

// Magnitude bits of a float: ordering them as unsigned integers orders the
// magnitudes, with every NaN above infinity.
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// The reciprocal scale that maps a buffer with largest magnitude `amax` to
// the state type: 1 / (amax / limit), or 0 when that scale is not positive
// (also NaN).
template <int ST>
__device__ __forceinline__ float rscale_of(uint32_t amax)
{
    const float scale = __uint_as_float(amax) / scaled_limit<ST>();
    return scale > 0.0f ? 1.0f / scale : 0.0f;
}

// One lane group of the store pass: unscale, update, store with the new
// reciprocal scales r.
template <class S>
__device__ __forceinline__ void scaled_group(const WorkItem &w, int gi, const Coeffs &c,
                                             const float *sc, const float *r)
{
    uint32_t hp[kLane], hm[kLane], hv[kLane];
    float p[kLane], m[kLane], v[kLane], g[kLane];
    load_u16x4(w.p, gi, hp);
    load_u16x4(w.m, gi, hm);
    load_u16x4(w.v, gi, hv);
    load_grad4<S::gt>(w.g, gi, g);
#pragma unroll
    for (int k = 0; k < kLane; ++k) {
        p[k] = widen16<S::st>(hp[k]) * sc[0];
        m[k] = widen16<S::st>(hm[k]) * sc[1];
        v[k] = widen16<S::st>(hv[k]) * sc[2];
        p[k] = update_element<S::mode, true>(p[k], g[k], m[k], v[k], c);
    }
    if constexpr (S::ot != kNone) {
        uint32_t o[kLane];
#pragma unroll
        for (int k = 0; k < kLane; ++k) o[k] = narrow16<S::ot>(p[k]);
        store_u16x4(w.p_out, gi, o);
    }
#pragma unroll
    for (int k = 0; k < kLane; ++k) {
        hp[k] = narrow16<S::st>(p[k] * r[0]);
        hm[k] = narrow16<S::st>(m[k] * r[1]);
        hv[k] = narrow16<S::st>(v[k] * r[2]);
    }
    store_u16x4(w.p, gi, hp);
    store_u16x4(w.m, gi, hm);
    store_u16x4(w.v, gi, hv);
}

// One element, exact: fold its magnitudes into mx (maxima pass) or store it
// (store pass).
template <class S>
__device__ __forceinline__ void scaled_single(const WorkItem &w, int i, const Coeffs &c,
                                              const float *sc, const float *r, uint32_t *mx)
{
    const float g = load_grad1<S::gt>(w.g, i);
    float p = widen16<S::st>(load_one<uint16_t>(w.p, i)) * sc[0];
    float m = widen16<S::st>(load_one<uint16_t>(w.m, i)) * sc[1];
    float v = widen16<S::st>(load_one<uint16_t>(w.v, i)) * sc[2];
    p = update_element<S::mode, true>(p, g, m, v, c);
    if constexpr (S::pass == 0) {
        mx[0] = max(mx[0], abs_bits(p));
        mx[1] = max(mx[1], abs_bits(m));
        mx[2] = max(mx[2], abs_bits(v));
    } else {
        if constexpr (S::ot != kNone) store_one<uint16_t>(w.p_out, i, uint16_t(narrow16<S::ot>(p)));
        store_one<uint16_t>(w.p, i, uint16_t(narrow16<S::st>(p * r[0])));
        store_one<uint16_t>(w.m, i, uint16_t(narrow16<S::st>(m * r[1])));
        store_one<uint16_t>(w.v, i, uint16_t(narrow16<S::st>(v * r[2])));
    }
}

// Largest of x over the 64 lanes of the wave, returned to every lane; every
// lane must be active.  Data-parallel-primitive moves: shifts right by 1, 2,
// 4 and 8 lanes within each row of 16 leave the row's maximum in its lane 15;
// broadcasting lane 15 into the next row (rows 1 and 3) and lane 31 into
// rows 2 and 3 leaves the wave's maximum in lane 63, the lane read at the
// end.  A lane with no source reads 0, the identity of unsigned max; lanes
// of the rows a broadcast skips hold values that lane 63 never reads.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_max(uint32_t x)
{
    return max(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), CTRL, ROWS, 0xf, true)));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x)
{
    x = dpp_max<0x111, 0xf>(x);  // row_shr:1
    x = dpp_max<0x112, 0xf>(x);  // row_shr:2
    x = dpp_max<0x114, 0xf>(x);  // row_shr:4
    x = dpp_max<0x118, 0xf>(x);  // row_shr:8
    x = dpp_max<0x142, 0xa>(x);  // row_bcast:15
    x = dpp_max<0x143, 0xc>(x);  // row_bcast:31
    return uint32_t(__builtin_amdgcn_readlane(int(x), 63));
}

// The maxima pass over a tile's lane groups: lane l takes groups gi0 + l +
// 64 j (j < G) that are below `groups`; every lane of the wave calls it.
// m, v and their maxima are exact.  The param is first computed with the
// hardware square root and reciprocal, which are within 0.78 ulp of the exact
// values for every normal input (checked over all floats; subnormal inputs
// flush).  With rho = 2^-24, mu = 2^-150 and 2^-22 taken as their relative
// error, the exact chain
//   q = RN(m_hat / RN(RN(sqrt v_hat) + eps)),  u = q (+ RN(wd p)),
//   t = RN(lr u),  p' = RN(p - t)
// and the approximate one (q~ = RN(m_hat * rcp(RN(sqrt~ v_hat + eps))), then
// the same roundings) differ by
//   |q~ - q|   <= 0.84 * 2^-20 |q~| + 3 mu   (eps >= 0 keeps the root's
//                                             relative error in the sum)
//   |p~ - p'|  <= 1.01 (|lr| |q~ - q| + 4.2 rho |t~|) + 2.01 rho |p~|
//                 + 10 mu (|lr| + 1)
// so E = 2^-19 |lr| max|q~| + 2^-21 max|t~| + 2^-22 max|p~| + 2^-140 (|lr|+1),
// over the wave, bounds every element's error with a factor 2 to spare (which
// also covers rounding in E and in the cut).  The element with the largest
// exact magnitude has |p~| >= max|p~| - 2E, and any element below
// max|p~| - 2.5 E has an exact magnitude below that one's; so the exact
// maximum is the maximum over the elements at or above the cut, each
// recomputed exactly.  The bound assumes finite values clear of overflow and
// a normal (or zero) v_hat: a wave with a subnormal v_hat of either sign (the
// hardware root flushes it to a signed zero, where the exact root of a
// negative one is NaN), or |q~|, |u~|, |t~| or |p~| not below 2^126 (NaN
// included; a negative normal v_hat gives NaN in both chains), recomputes
// all its elements, as does every wave when `approx` is off (eps < 0 or
// >= 2^125, |lr| >= 2^126).
template <class S, int G>
__device__ __forceinline__ void scaled_group_max(const WorkItem &w, int gi0, int groups, const Coeffs &c,
                                                 const float *sc, bool approx, uint32_t *mx)
{
    const int lane = threadIdx.x % 64;
    float p[G][kLane], m_hat[G][kLane], v_hat[G][kLane], pa[G][kLane];
    uint32_t pbits = 0u;
    float qmax = 0.0f, umax = 0.0f, tmax = 0.0f;
    bool ok = true;
#pragma unroll
    for (int j = 0; j < G; ++j) {
        if (lane + 64 * j >= groups) continue;
        const int gi = gi0 + lane + 64 * j;
        uint32_t hp[kLane], hm[kLane], hv[kLane];
        float g[kLane];
        load_u16x4(w.p, gi, hp);
        load_u16x4(w.m, gi, hm);
        load_u16x4(w.v, gi, hv);
        load_grad4<S::gt>(w.g, gi, g);
#pragma unroll
        for (int k = 0; k < kLane; ++k) {
            p[j][k] = widen16<S::st>(hp[k]) * sc[0];
            float m = widen16<S::st>(hm[k]) * sc[1];
            float v = widen16<S::st>(hv[k]) * sc[2];
            moments<S::mode, true>(p[j][k], g[k], m, v, c, m_hat[j][k], v_hat[j][k]);
            mx[1] = max(mx[1], abs_bits(m));
            mx[2] = max(mx[2], abs_bits(v));
            ok = ok && !__builtin_isfpclass(v_hat[j][k], __FPCLASS_POSSUBNORMAL | __FPCLASS_NEGSUBNORMAL);
            const float q = m_hat[j][k] * __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(v_hat[j][k]) + c.eps);
            float u = q;
            if constexpr (S::mode == 1) u = q + c.wd * p[j][k];
            const float t = c.lr * u;
            pa[j][k] = p[j][k] - t;
            qmax = fmaxf(qmax, fabsf(q));
            umax = fmaxf(umax, fabsf(u));
            tmax = fmaxf(tmax, fabsf(t));
            pbits = max(pbits, abs_bits(pa[j][k]));
        }
    }
    ok = ok && pbits < 0x7E800000u && qmax < 0x1p126f && umax < 0x1p126f && tmax < 0x1p126f;
    const float alr = fabsf(c.lr);
    const float e = 0x1p-19f * alr * qmax + 0x1p-21f * tmax + 0x1p-22f * __uint_as_float(pbits) +
                    0x1p-140f * (alr + 1.0f);
    const float top = __uint_as_float(wave_max(pbits));
    const float we = __uint_as_float(wave_max(__float_as_uint(e)));
    const bool all = !(approx && __all(ok) && we < 0x1p126f);
    const float cut = top - 2.5f * we;
#pragma unroll
    for (int j = 0; j < G; ++j) {
        if (lane + 64 * j >= groups) continue;
#pragma unroll
        for (int k = 0; k < kLane; ++k)
            if (all || fabsf(pa[j][k]) >= cut)
                mx[0] = max(mx[0], abs_bits(param_from<S::mode>(p[j][k], m_hat[j][k], v_hat[j][k], c)));
    }
}

// The maxima pass: one wave per tile (same tile map as the update), two lane
// groups per lane.  Writes the three magnitude maxima (p, m, v) of tile t to
// maxima[3t .. 3t+2], zeros for a tile past its record's end.
constexpr int kMaxBlock = 64;

template <class S>
__global__ __launch_bounds__(kMaxBlock) void adam_scaled_maxima(const WorkItem *__restrict__ items,
                                                                 uint32_t shift, uint32_t tile0, StepArgs a,
                                                                 uint32_t *__restrict__ maxima)
{
    static_assert(kTile == 2 * kLane * kMaxBlock, "two lane groups per lane");
    Coeffs c;
    if (!step_coeffs(a, c)) return;  // a noop step changes nothing (the fold skips too)
    const uint32_t b = tile0 + tile_of_block<kRun>(blockIdx.x, gridDim.x);
    const WorkItem w = items[b >> shift];
    const int start = int(b & ((1u << shift) - 1u)) * kTile;
    const int tid = threadIdx.x;
    uint32_t mx[3] = {0u, 0u, 0u};
    if (start < w.n) {  // uniform across the wave
        const float *scales = static_cast<const float *>(w.aux);
        const float sc[3] = {scales[0], scales[1], scales[2]};
        const int n = min(kTile, w.n - start);
        if (w.flags & kItemVector) {
            if (start == 0 && tid < w.head) scaled_single<S>(w, tid - w.head, c, sc, nullptr, mx);
            const int groups = n / kLane;
            const bool approx = c.eps >= 0.0f && c.eps < 0x1p125f && fabsf(c.lr) < 0x1p126f;
            scaled_group_max<S, 2>(w, start / kLane, groups, c, sc, approx, mx);
            if (tid < n - groups * kLane) scaled_single<S>(w, start + groups * kLane + tid, c, sc, nullptr, mx);
        } else {
            for (int i = tid; i < n; i += kMaxBlock) scaled_single<S>(w, start + i, c, sc, nullptr, mx);
        }
    }
    const uint32_t x0 = wave_max(mx[0]), x1 = wave_max(mx[1]), x2 = wave_max(mx[2]);
    if (tid < 3) maxima[3 * size_t(b) + tid] = tid == 0 ? x0 : tid == 1 ? x1 : x2;
}

// The store pass over the tiles of a scaled-state list (same tile map as the
// update): reads the reciprocal scales of its tensor from folded[6k + 3 ..].
template <class S>
__global__ __launch_bounds__(kBlock) void adam_scaled_pass(const WorkItem *__restrict__ items,
                                                            uint32_t shift, uint32_t tile0, StepArgs a,
                                                            uint32_t *__restrict__ folded)
{
    const uint32_t b = tile0 + tile_of_block<kRun>(blockIdx.x, gridDim.x);
    const WorkItem w = items[b >> shift];
    const int start = int(b & ((1u << shift) - 1u)) * kTile;
    const int tid = threadIdx.x;
    if (start >= w.n) return;  // uniform across the workgroup
    Coeffs c;
    if (!step_coeffs(a, c)) return;

    const float *scales = static_cast<const float *>(w.aux);
    const float sc[3] = {scales[0], scales[1], scales[2]};
    const uint32_t *f = folded + 6 * size_t(w.tensor) + 3;
    const float r[3] = {__uint_as_float(f[0]), __uint_as_float(f[1]), __uint_as_float(f[2])};

    const int n = min(kTile, w.n - start);
    if (w.flags & kItemVector) {
        if (start == 0 && tid < w.head) scaled_single<S>(w, tid - w.head, c, sc, r, nullptr);
        const int groups = n / kLane;
        if (tid < groups) scaled_group<S>(w, start / kLane + tid, c, sc, r);
        if (tid < n - groups * kLane) scaled_single<S>(w, start + groups * kLane + tid, c, sc, r, nullptr);
    } else {
        for (int i = tid; i < n; i += kBlock) scaled_single<S>(w, start + i, c, sc, r, nullptr);
    }
}

constexpr int kFoldMaxBlock = 256;

// One workgroup per tensor: the maxima of its tiles [tiles[2k], tiles[2k+1])
// folded into folded[6k .. 6k+2], and the reciprocal scales the store pass
// applies into folded[6k+3 .. 6k+5] (float bits).  `block` (capturable
// steps, else null): nothing to do when it marks the step a noop.
template <int ST>
__global__ __launch_bounds__(kFoldMaxBlock) void adam_scaled_fold(const uint32_t *__restrict__ tile_maxima,
                                                                  const uint32_t *__restrict__ tiles,
                                                                  uint32_t *__restrict__ folded, uint32_t k0,
                                                                  const StepBlock *__restrict__ block)
{
    if (block != nullptr && block->skip) return;
    const uint32_t k = k0 + blockIdx.x;
    const uint32_t lo = tiles[2 * k], hi = tiles[2 * k + 1];
    uint32_t x[3] = {0u, 0u, 0u};
    for (uint32_t t = lo + threadIdx.x; t < hi; t += kFoldMaxBlock)
#pragma unroll
        for (int j = 0; j < 3; ++j) x[j] = max(x[j], tile_maxima[3 * size_t(t) + j]);
    __shared__ uint32_t wave_maxima[3][kFoldMaxBlock / 64];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const uint32_t m = wave_max(x[j]);
        if (threadIdx.x % 64 == 0) wave_maxima[j][threadIdx.x / 64] = m;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        uint32_t m = 0u;
        for (int i = 0; i < kFoldMaxBlock / 64; ++i) m = max(m, wave_maxima[threadIdx.x][i]);
        folded[6 * size_t(k) + threadIdx.x] = m;
        folded[6 * size_t(k) + 3 + threadIdx.x] = __float_as_uint(rscale_of<ST>(m));
    }
}

// One lane per tensor: the new scales, amax / limit (none for a noop step).
template <int ST>
__global__ void adam_scaled_finish(float *const *__restrict__ scale_ptrs,
                                   const uint32_t *__restrict__ folded, uint32_t k0, uint32_t k1,
                                   const StepBlock *__restrict__ block)
{
    if (block != nullptr && block->skip) return;
    const uint32_t k = k0 + blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= k1) return;
    float *s = scale_ptrs[k];
#pragma unroll
    for (int j = 0; j < 3; ++j) s[j] = __uint_as_float(folded[6 * size_t(k) + j]) / scaled_limit<ST>();
}

// ---------------------------------------------------------------------------
// Scaled state in one pass.  A workgroup (four waves) updates a 4096-element
// tile exactly into registers, publishes the tile's three magnitude maxima
// and counts itself in as arrived for the tile's tensor; the workgroup that
// arrives last for a tensor folds that tensor's tile maxima, derives the
// reciprocal scales and publishes them; the tile (state and param-sync
// copy) is stored once its tensor's scales are out.  The inputs are read
// once and the update is computed once (the two-pass step reads them twice
// and computes the update twice).  A tile whose bounded wait runs out is
// left to a follow-up pass, which recomputes it from its untouched inputs; a
// kernel of one lane per tensor then writes the new scales and clears the
// counts and the published scales.
//
// Everything shared between workgroups (tile maxima, counts, reciprocal
// scales, the follow-up list) is read and written with relaxed device-scope
// atomic operations, which go to the device-coherent level of the memory
// hierarchy; a wait for the completion of a workgroup's stores orders them
// before its count.  A reciprocal scale is published as one 64-bit word, a
// tag bit above the float's bits, so a waiter that sees the tag has the
// value from the same store: no separate flag, and one round trip reads all
// three.  No release or acquire fence of device scope (which would write
// back or invalidate whole L2 caches) is needed.
//
// Measured on MI355X (1e9 elements in 2048 tensors): 3.65 ms per step
// against 3.97 for the two pipelined passes in the same process (a copy
// without the exchange, inexact, takes 3.29).  What it took: the tiles of
// one round of the grid cover a few tensors, and device-scope atomic
// operations on one address are performed one at a time, so each tensor's
// count is spread over kOneSpread addresses; each tile's exchange costs
// two round trips to device-coherent memory (the wait for the maxima's
// stores, with the previous tile's scales riding along, and the count),
// the second completing under the previous tile's stores; barriers order
// the local data share only; and the waits the compiler places on the
// vector memory counter, which drains in issue order, let the next tile's
// loads and the previous tile's stores stay in flight while a tile is
// computed (a first version waited for everything once per tile, with one
// counter per tensor, and took 4.66 ms).
// ---------------------------------------------------------------------------
constexpr int kOneBlock = 256;                            // four waves
constexpr int kOneGroups = 4;                             // lane groups per lane
constexpr int kOneSlots = kOneGroups * kLane;             // elements per lane (16)
constexpr int kOneTile = kOneBlock * kOneSlots;           // 4096 elements
constexpr uint32_t kOneSub = uint32_t(kOneTile / kTile);  // update tiles per one-pass tile (8)
constexpr uint32_t kOneSubLog = kOneSub == 8 ? 3 : kOneSub == 4 ? 2 : kOneSub == 2 ? 1 : 0;
constexpr uint32_t kOneRun = uint32_t(kRunElems / kOneTile);
static_assert(kOneBlock > kMaxHead && kRunElems % kOneTile == 0 && (1u << kOneSubLog) == kOneSub,
              "one-pass tile shape");

struct OneArgs {
    const uint32_t *tiles;     // per tensor: [first, end) update tiles
    const uint32_t *arrivals;  // per tensor: its non-empty spread counters, then kOneSpread rows (one per
                               // spread s) of its non-empty tiles at positions = s mod kOneSpread
    uint32_t *count;           // the same layout: arrivals in this step (0 between steps)
    uint64_t *ready;           // per tensor: its three reciprocal scales, kPublished | bits once published
                               // (0 between steps)
    uint32_t *tile_max;        // per one-pass tile: three magnitude maxima
    uint32_t *folded;          // per tensor: three magnitude maxima, three reciprocal scales (float bits)
    uint32_t *redo;            // [0]: tiles left to the follow-up pass, then their indices
    uint32_t *started;         // workgroups of the kernel that have started (0 between steps)
    uint64_t wait_ticks;       // a workgroup's wait, in ticks of the device's real-time clock; 0: none
    uint64_t grace_ticks;      // after this long, a wait ends if not every workgroup has started
    uint32_t wait_polls;       // and at most this many polls of the scales (each takes longer than 0.25 us)
    uint32_t tensors;          // non-empty tensors (the row length of arrivals and count)
};

// A tensor's arrivals are counted in kOneSpread counters, by the tile's
// position modulo kOneSpread; the last arrival at each of those counts
// itself in at the tensor's own counter, whose last arrival folds.  The
// tiles of one round of the grid cover a few tensors, and device-scope
// atomic operations on one address are performed one at a time: spread
// over several addresses they wait on each other far less.
constexpr uint32_t kOneSpread = 8;

constexpr uint64_t kPublished = uint64_t(1) << 32;  // the tag of a published reciprocal scale

__device__ __forceinline__ uint32_t shared_load(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void shared_store(uint32_t *p, uint32_t x)
{
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t shared_load64(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void shared_store64(uint64_t *p, uint64_t x)
{
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One element at index i of a record: the exact update of its unscaled
// value; P, M, V the new fp32 values.
template <class S>
__device__ __forceinline__ void one_element(const WorkItem &w, int i, const Coeffs &c, const float *sc, float &P,
                                            float &M, float &V)
{
    const float g = load_grad1<S::gt>(w.g, i);
    P = widen16<S::st>(load_one<uint16_t>(w.p, i)) * sc[0];
    M = widen16<S::st>(load_one<uint16_t>(w.m, i)) * sc[1];
    V = widen16<S::st>(load_one<uint16_t>(w.v, i)) * sc[2];
    P = update_element<S::mode, true>(P, g, M, V, c);
}

// Stores it: the scaled state with the reciprocal scales r, the param-sync
// copy of P.
template <class S>
__device__ __forceinline__ void one_store_element(const WorkItem &w, int i, const float *r, float P, float M, float V)
{
    store_one<uint16_t>(w.p, i, uint16_t(narrow16_hw<S::st>(P * r[0])));
    store_one<uint16_t>(w.m, i, uint16_t(narrow16_hw<S::st>(M * r[1])));
    store_one<uint16_t>(w.v, i, uint16_t(narrow16_hw<S::st>(V * r[2])));
    if constexpr (S::ot != kNone) store_one<uint16_t>(w.p_out, i, uint16_t(narrow16_hw<S::ot>(P)));
}

// The lane's elements of a one-pass tile (start, n elements of record w).
// A 4-element tensor: slot 4 j + e is element e of lane group j * kOneBlock +
// lane, slot kOneSlots the 0..3 elements after the tile's last whole group,
// slot kOneSlots + 1 the record's head (tile 0).  An element-path tensor:
// slot j is element lane + j * kOneBlock.
struct OneSlots {
    float P[kOneSlots + 2], M[kOneSlots + 2], V[kOneSlots + 2];
};

// Computes the lane's elements; folds their magnitudes into mx when it is
// not null.
template <class S>
__device__ __forceinline__ void one_compute(const WorkItem &w, int start, int n, const Coeffs &c, const float *sc,
                                            OneSlots &x, uint32_t *mx)
{
    const int tid = threadIdx.x;
    auto fold = [&](float P, float M, float V) {
        if (mx != nullptr) {
            mx[0] = max(mx[0], abs_bits(P));
            mx[1] = max(mx[1], abs_bits(M));
            mx[2] = max(mx[2], abs_bits(V));
        }
    };
    if (w.flags & kItemVector) {
        const int groups = n / kLane;
        uint32_t hp[kOneGroups][kLane], hm[kOneGroups][kLane], hv[kOneGroups][kLane];
        float g[kOneGroups][kLane];
#pragma unroll
        for (int j = 0; j < kOneGroups; ++j) {
            const int lg = j * kOneBlock + tid;
            if (lg < groups) {
                const int gi = start / kLane + lg;
                load_u16x4(w.p, gi, hp[j]);
                load_u16x4(w.m, gi, hm[j]);
                load_u16x4(w.v, gi, hv[j]);
                load_grad4<S::gt>(w.g, gi, g[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < kOneGroups; ++j) {
            const int lg = j * kOneBlock + tid;
            if (lg < groups) {
#pragma unroll
                for (int e = 0; e < kLane; ++e) {
                    float &P = x.P[j * kLane + e], &M = x.M[j * kLane + e], &V = x.V[j * kLane + e];
                    P = widen16<S::st>(hp[j][e]) * sc[0];
                    M = widen16<S::st>(hm[j][e]) * sc[1];
                    V = widen16<S::st>(hv[j][e]) * sc[2];
                    P = update_element<S::mode, true>(P, g[j][e], M, V, c);
                    fold(P, M, V);
                }
            }
        }
        if (tid < n - groups * kLane) {
            one_element<S>(w, start + groups * kLane + tid, c, sc, x.P[kOneSlots], x.M[kOneSlots], x.V[kOneSlots]);
            fold(x.P[kOneSlots], x.M[kOneSlots], x.V[kOneSlots]);
        }
        if (start == 0 && tid < w.head) {
            one_element<S>(w, tid - w.head, c, sc, x.P[kOneSlots + 1], x.M[kOneSlots + 1], x.V[kOneSlots + 1]);
            fold(x.P[kOneSlots + 1], x.M[kOneSlots + 1], x.V[kOneSlots + 1]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kOneSlots; ++j) {
            if (tid + j * kOneBlock < n) {
                one_element<S>(w, start + tid + j * kOneBlock, c, sc, x.P[j], x.M[j], x.V[j]);
                fold(x.P[j], x.M[j], x.V[j]);
            }
        }
    }
}

// Stores the lane's elements with the reciprocal scales r, and their
// param-sync copy.
template <class S>
__device__ __forceinline__ void one_store(const WorkItem &w, int start, int n, const float *r, const OneSlots &x)
{
    const int tid = threadIdx.x;
    if (w.flags & kItemVector) {
        const int groups = n / kLane;
#pragma unroll
        for (int j = 0; j < kOneGroups; ++j) {
            const int lg = j * kOneBlock + tid;
            if (lg < groups) {
                uint32_t hp[kLane], hm[kLane], hv[kLane];
#pragma unroll
                for (int e = 0; e < kLane; ++e) {
                    hp[e] = narrow16_hw<S::st>(x.P[j * kLane + e] * r[0]);
                    hm[e] = narrow16_hw<S::st>(x.M[j * kLane + e] * r[1]);
                    hv[e] = narrow16_hw<S::st>(x.V[j * kLane + e] * r[2]);
                }
                const int gi = start / kLane + lg;
                store_u16x4(w.p, gi, hp);
                store_u16x4(w.m, gi, hm);
                store_u16x4(w.v, gi, hv);
                if constexpr (S::ot != kNone) {
                    uint32_t o[kLane];
#pragma unroll
                    for (int e = 0; e < kLane; ++e) o[e] = narrow16_hw<S::ot>(x.P[j * kLane + e]);
                    store_u16x4(w.p_out, gi, o);
                }
            }
        }
        if (tid < n - groups * kLane)
            one_store_element<S>(w, start + groups * kLane + tid, r, x.P[kOneSlots], x.M[kOneSlots], x.V[kOneSlots]);
        if (start == 0 && tid < w.head)
            one_store_element<S>(w, tid - w.head, r, x.P[kOneSlots + 1], x.M[kOneSlots + 1], x.V[kOneSlots + 1]);
    } else {
#pragma unroll
        for (int j = 0; j < kOneSlots; ++j)
            if (tid + j * kOneBlock < n) one_store_element<S>(w, start + tid + j * kOneBlock, r, x.P[j], x.M[j], x.V[j]);
    }
}

// Waits until at most N vector memory operations of the wave are in flight
// (they complete in issue order): expcnt and lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vector_memory()
{
    static_assert(N >= 0 && N < 64, "vmcnt has six bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// A workgroup barrier that orders the local data share only.  The one-pass
// kernel shares nothing else between the waves of a workgroup (its global
// accesses are ordered by explicit waits), and a barrier with a fence over
// all memory would wait for every load and store in flight, such as the
// next tile's loads and the count's round trip.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The largest of three values per lane over the workgroup, in lane 0 of
// wave 0 (every lane must call it).
__device__ __forceinline__ void one_block_max(uint32_t *mx)
{
    __shared__ uint32_t wave_maxima[3][kOneBlock / 64];
    const uint32_t x0 = wave_max(mx[0]), x1 = wave_max(mx[1]), x2 = wave_max(mx[2]);
    if (threadIdx.x % 64 == 0) {
        wave_maxima[0][threadIdx.x / 64] = x0;
        wave_maxima[1][threadIdx.x / 64] = x1;
        wave_maxima[2][threadIdx.x / 64] = x2;
    }
    lds_barrier();
    if (threadIdx.x == 0)
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            uint32_t m = wave_maxima[j][0];
            for (int i = 1; i < kOneBlock / 64; ++i) m = max(m, wave_maxima[j][i]);
            mx[j] = m;
        }
}

// The prefetched lane groups of a 4-element tile: p, m, v (16-bit) and g.
template <int GT>
struct OneRaw {
    u32x2 p[kOneGroups], m[kOneGroups], v[kOneGroups];
    typename std::conditional<GT == kF32, f32x4, u32x2>::type g[kOneGroups];
};

// Whether a one-pass tile is whole: 4096 elements in lane groups, no head.
__device__ __forceinline__ bool one_whole(const WorkItem &w, int start, int n)
{
    return n == kOneTile && (start != 0 || w.head == 0);
}

// Issues the loads of `groups` lane groups of a tile (0 for no tile): always
// 16 per lane, lanes past the tile's groups reading `spare` (any 16 readable
// bytes), so that every path leaves the same loads in flight.
template <int GT>
__device__ __forceinline__ void one_load_raw(const WorkItem &w, int start, int groups, const void *spare,
                                             OneRaw<GT> &raw)
{
    using G = std::remove_reference_t<decltype(raw.g[0])>;
    const int tid = threadIdx.x;
    const int g0 = start / kLane;
    if (groups == kOneGroups * kOneBlock) {
#pragma unroll
        for (int j = 0; j < kOneGroups; ++j) {
            const int gi = g0 + j * kOneBlock + tid;
            raw.p[j] = load_stream<u32x2>(w.p, gi);
            raw.m[j] = load_stream<u32x2>(w.m, gi);
            raw.v[j] = load_stream<u32x2>(w.v, gi);
            raw.g[j] = load_stream<G>(w.g, gi);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kOneGroups; ++j) {
            const int lg = j * kOneBlock + tid;
            const bool in = lg < groups;
            const int gi = in ? g0 + lg : 0;
            raw.p[j] = load_stream<u32x2>(in ? w.p : spare, gi);
            raw.m[j] = load_stream<u32x2>(in ? w.m : spare, gi);
            raw.v[j] = load_stream<u32x2>(in ? w.v : spare, gi);
            raw.g[j] = load_stream<G>(in ? w.g : spare, gi);
        }
    }
}

// one_compute for a 4-element tile whose lane groups are already loaded;
// WHOLE: a whole tile (no condition, no element path, no memory access).
template <class S, bool WHOLE>
__device__ __forceinline__ void one_compute_raw(const WorkItem &w, int start, int n, const Coeffs &c, const float *sc,
                                                const OneRaw<S::gt> &raw, OneSlots &x, uint32_t *mx)
{
    const int tid = threadIdx.x;
    const int groups = n / kLane;
    auto fold = [&](float P, float M, float V) {
        mx[0] = max(mx[0], abs_bits(P));
        mx[1] = max(mx[1], abs_bits(M));
        mx[2] = max(mx[2], abs_bits(V));
    };
#pragma unroll
    for (int j = 0; j < kOneGroups; ++j) {
        if (WHOLE || j * kOneBlock + tid < groups) {
            const uint32_t hp[kLane] = {raw.p[j].x & 0xFFFFu, raw.p[j].x >> 16, raw.p[j].y & 0xFFFFu, raw.p[j].y >> 16};
            const uint32_t hm[kLane] = {raw.m[j].x & 0xFFFFu, raw.m[j].x >> 16, raw.m[j].y & 0xFFFFu, raw.m[j].y >> 16};
            const uint32_t hv[kLane] = {raw.v[j].x & 0xFFFFu, raw.v[j].x >> 16, raw.v[j].y & 0xFFFFu, raw.v[j].y >> 16};
            float g[kLane];
            if constexpr (S::gt == kF32) {
                g[0] = raw.g[j].x;
                g[1] = raw.g[j].y;
                g[2] = raw.g[j].z;
                g[3] = raw.g[j].w;
            } else {
                g[0] = widen16<S::gt>(raw.g[j].x & 0xFFFFu);
                g[1] = widen16<S::gt>(raw.g[j].x >> 16);
                g[2] = widen16<S::gt>(raw.g[j].y & 0xFFFFu);
                g[3] = widen16<S::gt>(raw.g[j].y >> 16);
            }
#pragma unroll
            for (int e = 0; e < kLane; ++e) {
                float &P = x.P[j * kLane + e], &M = x.M[j * kLane + e], &V = x.V[j * kLane + e];
                P = widen16<S::st>(hp[e]) * sc[0];
                M = widen16<S::st>(hm[e]) * sc[1];
                V = widen16<S::st>(hv[e]) * sc[2];
                P = update_element<S::mode, true>(P, g[e], M, V, c);
                fold(P, M, V);
            }
        }
    }
    if constexpr (!WHOLE) {
        if (tid < n - groups * kLane) {
            one_element<S>(w, start + groups * kLane + tid, c, sc, x.P[kOneSlots], x.M[kOneSlots], x.V[kOneSlots]);
            fold(x.P[kOneSlots], x.M[kOneSlots], x.V[kOneSlots]);
        }
        if (start == 0 && tid < w.head) {
            one_element<S>(w, tid - w.head, c, sc, x.P[kOneSlots + 1], x.M[kOneSlots + 1], x.V[kOneSlots + 1]);
            fold(x.P[kOneSlots + 1], x.M[kOneSlots + 1], x.V[kOneSlots + 1]);
        }
    }
}

// The one-pass step, persistent: workgroup j takes the tiles at positions
// j, j + G, j + 2G, ... (G = the grid; position -> tile in the update's XCD
// order), in that order.  For each tile it issues the next tile's loads,
// computes the tile into registers, arrives for the tile's tensor (folding
// and publishing the tensor's scales if it is the last), then stores the
// previous tile from local memory once its tensor's scales are out, and
// puts this tile there.  The wait for a tensor thus has the next tile's
// loads and arithmetic to cover it, and its scales are read in the same
// round trip as the arrival.  Publishing never waits for anything but
// stores already issued, and a workgroup waits for the tensor of its
// previous tile only after arriving for its current one, so no wait depends
// on a tile of the same workgroup unless a tensor spans more than 2G
// positions; the handle keeps tensors below that, and the bounded wait
// covers the rest.  Every tensor of a one-pass list takes 4-element
// accesses: a list with a tensor on the element path (buffers that cannot
// all be aligned at one element) takes two passes, which keeps this kernel
// at three waves per SIMD.
template <class S>
__global__ __launch_bounds__(kOneBlock) void adam_scaled_one(const WorkItem *__restrict__ items, uint32_t shift,
                                                              uint32_t total, StepArgs a, OneArgs f)
{
    Coeffs c;
    if (!step_coeffs(a, c)) return;  // a noop step changes nothing
    __shared__ float keep[3][kOneSlots][kOneBlock];  // the previous tile's new p, m, v (4-element slots)
    __shared__ uint32_t last, ready;
    __shared__ uint64_t qs[3];  // what lane 0 of wave 0 read of the previous tile's tensor's scales
    __shared__ float rs[3];
    const int tid = threadIdx.x;
    const uint32_t mask = (1u << shift) - 1u;
    auto tile_at = [&](uint32_t pos) { return tile_of_block<kOneRun>(pos, total); };
    auto published = [](const uint64_t *q) { return (q[0] & q[1] & q[2] & kPublished) != 0u; };

    uint32_t pos = blockIdx.x;
    // counted in, so that a wait can tell whether the tiles it waits for
    // belong to workgroups that are not running yet (other kernels holding
    // the compute units they need)
    if (tid == 0) __hip_atomic_fetch_add(f.started, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    OneRaw<S::gt> raw[2];  // the current and the next tile's lane groups, alternating
    {
        const uint32_t t = tile_at(pos);
        const WorkItem w = items[t >> shift];
        const int start = int(t & mask) * kOneTile;
        one_load_raw<S::gt>(w, start, start < w.n ? min(kOneTile, w.n - start) / kLane : 0, items, raw[0]);
        __builtin_amdgcn_s_waitcnt(0);  // enter the loop with nothing in flight
    }
    bool have_prev = false, whole_prev = false;
    uint32_t t_prev = 0;
    float sp[2] = {0.0f, 0.0f}, sm[2] = {0.0f, 0.0f}, sv[2] = {0.0f, 0.0f};  // the previous tile's tail and head

    // lane 0 of wave 0: the previous tile's tensor's published words
    auto look = [&](uint64_t *q) {
        const uint64_t *rk = f.ready + 3 * size_t(items[t_prev >> shift].tensor);
#pragma unroll
        for (int j = 0; j < 3; ++j) q[j] = shared_load64(rk + j);
    };

    // waits (lane 0 of wave 0) until the previous tile's tensor's scales are
    // out, qs being what it last read of them, else leaves the tile to the
    // follow-up pass; whether they are out, for every lane
    auto wait_prev = [&]() {
        if (tid == 0) {
            uint64_t q[3] = {qs[0], qs[1], qs[2]};
            bool seen = f.wait_ticks != 0 && published(q);
            if (f.wait_ticks != 0 && !seen) {
                const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                for (uint32_t polls = 0; !seen && polls < f.wait_polls &&
                                         __builtin_amdgcn_s_memrealtime() - t0 < f.wait_ticks;
                     ++polls) {
                    __builtin_amdgcn_s_sleep(16);
                    look(q);
                    seen = published(q);
                    // not every workgroup running: leave the tile to the
                    // follow-up pass rather than wait for one that is not
                    if (!seen && __builtin_amdgcn_s_memrealtime() - t0 >= f.grace_ticks &&
                        shared_load(f.started) < gridDim.x)
                        break;
                }
            }
            if (seen) {
#pragma unroll
                for (int j = 0; j < 3; ++j) rs[j] = __uint_as_float(uint32_t(q[j]));
            } else {
                // leave the tile to the follow-up pass (its inputs are untouched)
                const uint32_t slot = __hip_atomic_fetch_add(f.redo, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                shared_store(f.redo + 1 + slot, t_prev);
            }
            ready = seen ? 1u : 0u;
        }
        lds_barrier();
        return ready != 0u;
    };

    // Stores the previous tile from local memory once its scales are out:
    // its lane groups (all of them for a whole tile) ...
    auto store_prev = [&](auto whole_tag, const float *r) {
        constexpr bool whole = decltype(whole_tag)::value;
        const WorkItem w = items[t_prev >> shift];
        const int start = int(t_prev & mask) * kOneTile;
        const int n = min(kOneTile, w.n - start);
        const int groups = n / kLane;
#pragma unroll
        for (int j = 0; j < kOneGroups; ++j) {
            const int lg = j * kOneBlock + tid;
            if (whole || lg < groups) {
                uint32_t hp[kLane], hm[kLane], hv[kLane];
                float P[kLane];
#pragma unroll
                for (int e = 0; e < kLane; ++e) {
                    P[e] = keep[0][j * kLane + e][tid];
                    hp[e] = narrow16_hw<S::st>(P[e] * r[0]);
                    hm[e] = narrow16_hw<S::st>(keep[1][j * kLane + e][tid] * r[1]);
                    hv[e] = narrow16_hw<S::st>(keep[2][j * kLane + e][tid] * r[2]);
                }
                const int gi = start / kLane + lg;
                store_u16x4(w.p, gi, hp);
                store_u16x4(w.m, gi, hm);
                store_u16x4(w.v, gi, hv);
                if constexpr (S::ot != kNone) {
                    uint32_t o[kLane];
#pragma unroll
                    for (int e = 0; e < kLane; ++e) o[e] = narrow16_hw<S::ot>(P[e]);
                    store_u16x4(w.p_out, gi, o);
                }
            }
        }
        // ... and, for a tile that is not whole, its element path
        if (!whole) {
            if (tid < n - groups * kLane) one_store_element<S>(w, start + groups * kLane + tid, r, sp[0], sm[0], sv[0]);
            if (start == 0 && tid < w.head) one_store_element<S>(w, tid - w.head, r, sp[1], sm[1], sv[1]);
        }
    };

    // the last workgroup of tensor k: fold the maxima of its non-empty
    // one-pass tiles, publish the reciprocal scales (all lanes)
    auto fold = [&](uint32_t k) {
        const uint32_t lo = f.tiles[2 * k] / kOneSub, hi = f.tiles[2 * k + 1] / kOneSub;
        uint32_t m[3] = {0u, 0u, 0u};
        for (uint32_t u = lo + tid; u < hi; u += kOneBlock) {
            const bool live_u = int(u & mask) * kOneTile < items[u >> shift].n;
            uint32_t x[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) x[j] = shared_load(f.tile_max + 3 * size_t(u) + j);
            if (live_u) {
#pragma unroll
                for (int j = 0; j < 3; ++j) m[j] = max(m[j], x[j]);
            }
        }
        one_block_max(m);
        if (tid == 0) {
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const uint32_t rbits = __float_as_uint(rscale_of<S::st>(m[j]));
                shared_store(f.folded + 6 * size_t(k) + j, m[j]);
                shared_store(f.folded + 6 * size_t(k) + 3 + j, rbits);
                shared_store64(f.ready + 3 * size_t(k) + j, kPublished | rbits);
            }
        }
        lds_barrier();  // the block maxima are read before any wave writes them again
    };

    // one tile: the next one's loads into nxt, this one computed from cur
    auto body = [&](const OneRaw<S::gt> &cur, OneRaw<S::gt> &nxt) {
        const uint32_t t = tile_at(pos);
        const WorkItem w = items[t >> shift];
        const int start = int(t & mask) * kOneTile;
        const bool live = start < w.n;
        const int n = live ? min(kOneTile, w.n - start) : 0;
        {
            // the next tile's lane groups, in flight while this one is computed
            const bool more = pos + gridDim.x < total;
            const uint32_t t2 = more ? tile_at(pos + gridDim.x) : t;
            const WorkItem w2 = items[t2 >> shift];
            const int start2 = int(t2 & mask) * kOneTile;
            const int groups2 = more && start2 < w2.n ? min(kOneTile, w2.n - start2) / kLane : 0;
            one_load_raw<S::gt>(w2, start2, groups2, items, nxt);
        }
        const uint32_t k = uint32_t(w.tensor);
        const bool whole = live && one_whole(w, start, n);
        OneSlots x;
        uint32_t mx[3] = {0u, 0u, 0u};
        if (whole) {
            float sc[3];
            load_scales(w.aux, sc);  // every tensor of a one-pass list takes 4-element accesses
            one_compute_raw<S, true>(w, start, n, c, sc, cur, x, mx);
        } else if (live) {
            float sc[3];
            load_scales(w.aux, sc);
            one_compute_raw<S, false>(w, start, n, c, sc, cur, x, mx);
        }
        if (live) one_block_max(mx);
        // Waits for vector memory count in issue order, and the compiler
        // places them from what any path may leave in flight.  A drain here,
        // after the tile's arithmetic (the scheduling barrier keeps it
        // there), costs little: the next tile's loads and the previous
        // tile's stores have had that long.  It leaves the next tile's
        // arithmetic with no wait on its loads, complete by then.
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0);
        // lane 0 of wave 0: read the previous tile's scales, publish this
        // tile's maxima, wait until both are done, then count this tile in
        // (the count's round trip runs while the previous tile is stored)
        const size_t sub = size_t(1 + pos % kOneSpread) * f.tensors + k;
        uint32_t before = 0u;
        if (tid == 0) {
            // (both unconditional: a branch here lets the compiler split the
            // block and leave the reads unwaited on some path; without a
            // previous tile the words read are ignored, and an empty tile's
            // maxima, all 0, are never folded)
            uint64_t q[3];
            look(q);
#pragma unroll
            for (int j = 0; j < 3; ++j) shared_store(f.tile_max + 3 * size_t(t) + j, mx[j]);
            __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
            for (int j = 0; j < 3; ++j) qs[j] = q[j];
            if (live) before = __hip_atomic_fetch_add(f.count + sub, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        lds_barrier();
        // the previous tile, if its scales are out already
        const uint64_t q[3] = {qs[0], qs[1], qs[2]};
        const bool early = have_prev && f.wait_ticks != 0 && published(q);
        // The count's round trip (lane 0 of wave 0) then completes under the
        // previous tile's stores: issued after it, a whole tile's kPrevStores
        // stores may stay in flight while the wait retires the count.
        constexpr int kPrevStores = kOneGroups * (S::ot != kNone ? 4 : 3);
        if (early) {
            const float r[3] = {__uint_as_float(uint32_t(q[0])), __uint_as_float(uint32_t(q[1])),
                                __uint_as_float(uint32_t(q[2]))};
            if (whole_prev) {
                store_prev(std::true_type(), r);
                wait_vector_memory<kPrevStores>();
            } else {
                store_prev(std::false_type(), r);
                wait_vector_memory<0>();
            }
        } else {
            wait_vector_memory<0>();
        }
        // this tile's count (its tensor's last tile folds: publishing never
        // waits for anything but the stores and counts already issued)
        if (tid == 0 && live) {
            // the count's value is first used here, after the stores above
            // (the compiler would otherwise use it, and wait for it, at once)
            asm volatile("" : "+v"(before)::"memory");
            const ADAM_CONSTANT uint32_t *arrivals = (const ADAM_CONSTANT uint32_t *)f.arrivals;
            uint32_t is_last = 0u;
            if (before + 1u == arrivals[sub]) {
                const uint32_t before_k =
                    __hip_atomic_fetch_add(f.count + k, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                is_last = before_k + 1u == arrivals[k] ? 1u : 0u;
            }
            last = is_last;
        }
        lds_barrier();
        if (live && last) fold(k);
        // the previous tile, if its scales were not out: wait for them
        if (have_prev && !early && wait_prev()) {
            if (whole_prev)
                store_prev(std::true_type(), rs);
            else
                store_prev(std::false_type(), rs);
        }
        // each lane's own columns of keep: no lane reads another's
        if (live) {
#pragma unroll
            for (int j = 0; j < kOneSlots; ++j) {
                keep[0][j][tid] = x.P[j];
                keep[1][j][tid] = x.M[j];
                keep[2][j][tid] = x.V[j];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                sp[j] = x.P[kOneSlots + j];
                sm[j] = x.M[kOneSlots + j];
                sv[j] = x.V[kOneSlots + j];
            }
            t_prev = t;
        }
        have_prev = live;
        whole_prev = whole;
        pos += gridDim.x;
    };

    // two tiles per turn, so that the two buffers swap roles without copies
    while (pos < total) {
        body(raw[0], raw[1]);
        if (pos >= total) break;
        body(raw[1], raw[0]);
    }
    if (have_prev) {
        if (tid == 0) {
            uint64_t q[3];
            look(q);
#pragma unroll
            for (int j = 0; j < 3; ++j) qs[j] = q[j];
        }
        lds_barrier();
        if (wait_prev()) {
            if (whole_prev)
                store_prev(std::true_type(), rs);
            else
                store_prev(std::false_type(), rs);
        }
    }
}

// The follow-up pass: recomputes and stores the one-pass tiles whose wait
// ran out (their tensors' scales are all published by then).
template <class S>
__global__ __launch_bounds__(kOneBlock) void adam_scaled_one_redo(const WorkItem *__restrict__ items, uint32_t shift,
                                                                   StepArgs a, OneArgs f)
{
    Coeffs c;
    if (!step_coeffs(a, c)) return;
    const uint32_t total = shared_load(f.redo);
    for (uint32_t i = blockIdx.x; i < total; i += gridDim.x) {
        const uint32_t b = shared_load(f.redo + 1 + i);
        const WorkItem w = items[b >> shift];
        const int start = int(b & ((1u << shift) - 1u)) * kOneTile;
        const int n = min(kOneTile, w.n - start);
        float sc[3];
        load_scales(w.aux, sc);
        const uint32_t *rk = f.folded + 6 * size_t(w.tensor) + 3;
        const float r[3] = {__uint_as_float(shared_load(rk)), __uint_as_float(shared_load(rk + 1)),
                            __uint_as_float(shared_load(rk + 2))};
        OneSlots x;
        one_compute<S>(w, start, n, c, sc, x, nullptr);
        one_store<S>(w, start, n, r, x);
    }
}

// One lane per tensor: the new scales (amax / limit), and the counts and
// published scales cleared for the next step; lane 0 clears the follow-up
// list.
template <int ST>
__global__ void adam_scaled_one_finish(float *const *__restrict__ scale_ptrs, OneArgs f, uint32_t tensors,
                                       const StepBlock *__restrict__ block)
{
    if (block != nullptr && block->skip) return;
    const uint32_t k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k == 0) {
        shared_store(f.redo, 0u);
        shared_store(f.started, 0u);
    }
    if (k >= tensors) return;
    float *s = scale_ptrs[k];
#pragma unroll
    for (int j = 0; j < 3; ++j) s[j] = __uint_as_float(shared_load(f.folded + 6 * size_t(k) + j)) / scaled_limit<ST>();
#pragma unroll
    for (uint32_t row = 0; row <= kOneSpread; ++row) shared_store(f.count + size_t(row) * tensors + k, 0u);
#pragma unroll
    for (int j = 0; j < 3; ++j) shared_store64(f.ready + 3 * size_t(k) + j, 0u);
}

// ---------------------------------------------------------------------------
// Gradient sum of squares and the clip / found-inf step (apex
// distributed_fused_adam.py: grad_norm, clip_grad_norm, the found-inf check
// of step()).  Squares of float, bf16 or fp16 gradients are exact in double;
// every workgroup adds its squares in a fixed order, partial sums are folded
// in a fixed order, so the result does not depend on scheduling.
// ---------------------------------------------------------------------------
constexpr int kFoldBlock = 256;
constexpr int kNormUnroll = 4;  // 16-byte loads in flight per lane

// Sum over a workgroup of one double per lane, in a fixed tree order.
template <int BLOCK>
__device__ __forceinline__ double block_sum(double x)
{
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    __shared__ double wave_sums[BLOCK / 64];
    if (threadIdx.x % 64 == 0) wave_sums[threadIdx.x / 64] = x;
    __syncthreads();
    double total = 0.0;
    if (threadIdx.x == 0)
        for (int i = 0; i < BLOCK / 64; ++i) total += wave_sums[i];
    return total;  // meaningful in thread 0
}

// The squares of the gradients in one 16-byte word (8 bf16 / fp16 or 4 fp32),
// added to acc in element order.
template <int GT>
__device__ __forceinline__ double add_squares16(double acc, u32x4 q)
{
    const uint32_t x[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if constexpr (GT == kF32) {
            const double f = __uint_as_float(x[k]);
            acc += f * f;
        } else {
            const double lo = widen16<GT>(x[k] & 0xFFFFu);
            const double hi = widen16<GT>(x[k] >> 16);
            acc += lo * lo;
            acc += hi * hi;
        }
    }
    return acc;
}

// Workgroup b adds the squares of the gradients of tiles [b*run, (b+1)*run)
// and writes one partial sum.  The tiles of a run are consecutive, so it
// walks them record by record: one scalar load of the record, then a strided
// loop over its contiguous gradient elements with 16-byte loads, kNormUnroll
// of them in flight per lane (one stream, so unlike the update it needs wide
// loads to keep enough bytes in flight: measured 1.5x faster than 8-byte
// loads on bf16 gradients).  The 0..7 elements before the first 16-byte
// boundary and after the last whole word go element by element; the update's
// alignment of the other streams does not matter here.
template <int GT>
__global__ __launch_bounds__(kBlock) void grad_sumsq_partial(const WorkItem *__restrict__ items,
                                                              uint32_t shift, uint32_t tiles,
                                                              uint32_t run,
                                                              double *__restrict__ partials)
{
    constexpr int GS = GT == kF32 ? 4 : 2;  // bytes per gradient element
    constexpr int W = 16 / GS;              // gradient elements per 16-byte word
    const uint32_t first = blockIdx.x * run;
    const uint32_t last = min(first + run, tiles);
    const int tid = threadIdx.x;
    double acc = 0.0;
    for (uint32_t t = first; t < last;) {
        const uint32_t r = t >> shift;
        const WorkItem w = items[r];
        const uint32_t rec_first = r << shift;
        const uint32_t t_end = min(last, rec_first + (1u << shift));
        const int e0 = int((t - rec_first) * kTile);
        const int e1 = min(w.n, int((t_end - rec_first) * kTile));
        t = t_end;
        if (e0 >= e1) continue;  // tiles past the end of a tensor's last record
        if ((w.flags & kItemVector) && e0 == 0 && tid < w.head) {
            const double x = load_grad1<GT>(w.g, tid - w.head);
            acc += x * x;
        }
        // e0 is a whole number of tiles, so element e0 has the record's
        // alignment modulo 16 bytes
        const int lead = min(e1 - e0, int(((16u - (uintptr_t(w.g) & 15u)) & 15u) / GS));
        if (tid < lead) {
            const double x = load_grad1<GT>(w.g, e0 + tid);
            acc += x * x;
        }
        const int words = (e1 - e0 - lead) / W;
        const void *base = static_cast<const char *>(w.g) + size_t(e0 + lead) * GS;
        for (int vb = 0; vb < words; vb += kBlock * kNormUnroll) {
            u32x4 q[kNormUnroll];
#pragma unroll
            for (int u = 0; u < kNormUnroll; ++u) {
                const int vi = vb + u * kBlock + tid;
                q[u] = vi < words ? load_stream<u32x4>(base, vi) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kNormUnroll; ++u) acc = add_squares16<GT>(acc, q[u]);
        }
        for (int i = e0 + lead + words * W + tid; i < e1; i += kBlock) {
            const double x = load_grad1<GT>(w.g, i);
            acc += x * x;
        }
    }
    const double total = block_sum<kBlock>(acc);
    if (tid == 0) partials[blockIdx.x] = total;
}

// One workgroup: *d_sumsq = (accumulate ? *d_sumsq : 0) + the partial sums.
__global__ __launch_bounds__(kFoldBlock) void grad_sumsq_fold(const double *__restrict__ partials,
                                                              uint32_t count, double *d_sumsq,
                                                              int32_t accumulate)
{
    double acc = 0.0;
    for (uint32_t i = threadIdx.x; i < count; i += kFoldBlock) acc += partials[i];
    const double total = block_sum<kFoldBlock>(acc);
    if (threadIdx.x == 0) *d_sumsq = (accumulate ? *d_sumsq : 0.0) + total;
}

// One lane: the norm, the found-inf flag and the clipped grad scale, in
// float as the pages' tensors are.
__global__ void clip_grad_scale_kernel(const double *d_sumsq, float *d_grad_scale, float max_norm,
                                       float *d_norm, int32_t *d_noop)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    const float raw = float(sqrt(*d_sumsq));
    const float scale = d_grad_scale != nullptr ? *d_grad_scale : 1.0f;
    const float norm = raw * scale;
    const bool found_inf = !isfinite(norm);
    if (d_norm != nullptr) *d_norm = norm;
    if (d_noop != nullptr) *d_noop = found_inf ? 1 : 0;
    if (!found_inf && max_norm > 0.0f && d_grad_scale != nullptr) {
        float coef = max_norm / (norm + 1e-6f);
        if (coef > 1.0f) coef = 1.0f;
        *d_grad_scale = scale * coef;
    }
}

// ---------------------------------------------------------------------------
// Host side: kernel tables
// ---------------------------------------------------------------------------

typedef void (*UpdateFn)(const WorkItem *, uint32_t, uint32_t, StepArgs);
typedef void (*ScaledFn)(const WorkItem *, uint32_t, uint32_t, StepArgs, uint32_t *);
typedef void (*OneFn)(const WorkItem *, uint32_t, uint32_t, StepArgs, OneArgs);
typedef void (*OneRedoFn)(const WorkItem *, uint32_t, StepArgs, OneArgs);

constexpr int kGradTypes[3] = {kF32, kBF16, kF16};
constexpr int kOutTypes[3] = {kNone, kBF16, kF16};              // scaled state
constexpr int kUpdateOutTypes[4] = {kNone, kBF16, kF16, kF32};  // update kernels
constexpr int kStateTypes[2] = {kBF16, kF16};

// Update table index: g + 3 * (param kind + 4 * (out + 4 * (mode + 2 * capturable))),
// with g and out positions in kGradTypes / kUpdateOutTypes.
template <int I>
constexpr UpdateFn update_at()
{
    constexpr int g = kGradTypes[I % 3];
    constexpr int pk = (I / 3) % 4;
    constexpr int ot = kUpdateOutTypes[(I / 12) % 4];
    constexpr int mode = (I / 48) % 2;
    constexpr bool capt = (I / 96) != 0;
    if constexpr (pk == kParamRem && ot != kNone && ot != kBF16)
        return nullptr;  // refused by the planner
    else
        return adam_update<Config<g, pk, ot, mode, capt>>;
}

// Scaled table index: g + 3 * (out + 3 * (state + 2 * (mode + 2 * pass))).
template <int I>
constexpr ScaledFn scaled_at()
{
    constexpr int g = kGradTypes[I % 3];
    constexpr int ot = kOutTypes[(I / 3) % 3];
    constexpr int st = kStateTypes[(I / 9) % 2];
    constexpr int mode = (I / 18) % 2;
    constexpr int pass = I / 36;
    if constexpr (pass == 0)
        return adam_scaled_maxima<ScaledConfig<st, g, ot, mode, 0>>;
    else
        return adam_scaled_pass<ScaledConfig<st, g, ot, mode, 1>>;
}

template <int... I>
struct UpdateTable {
    static constexpr UpdateFn fns[sizeof...(I)] = {update_at<I>()...};
};
template <int... I>
struct ScaledTable {
    static constexpr ScaledFn fns[sizeof...(I)] = {scaled_at<I>()...};
};

template <int... I>
UpdateTable<I...> update_table(std::integer_sequence<int, I...>);
template <int... I>
ScaledTable<I...> scaled_table(std::integer_sequence<int, I...>);

using UpdateKernels = decltype(update_table(std::make_integer_sequence<int, 192>()));
using ScaledKernels = decltype(scaled_table(std::make_integer_sequence<int, 72>()));

// One-pass scaled-state table index: g + 3 * (out + 3 * (state + 2 * mode)),
// as the scaled passes.
template <int I>
using OneConfig = ScaledConfig<kStateTypes[(I / 9) % 2], kGradTypes[I % 3], kOutTypes[(I / 3) % 3], I / 18, 1>;
template <int... I>
struct OneTable {
    static constexpr OneFn fns[sizeof...(I)] = {adam_scaled_one<OneConfig<I>>...};
    static constexpr OneRedoFn redo[sizeof...(I)] = {adam_scaled_one_redo<OneConfig<I>>...};
};
template <int... I>
OneTable<I...> one_table(std::integer_sequence<int, I...>);
using OneKernels = decltype(one_table(std::make_integer_sequence<int, 36>()));

int type_pos(const int *types, int n, int t)
{
    for (int i = 0; i < n; ++i)
        if (types[i] == t) return i;
    return -1;
}

// ---------------------------------------------------------------------------
// Host side: planning
// ---------------------------------------------------------------------------

struct Plan {
    adam_tl_stats stats;
    uint32_t shift;
    std::vector<WorkItem> items;
    std::vector<float *> scale_ptrs;    // scaled state: per non-empty tensor
    std::vector<uint32_t> tile_ranges;  // [first, end) tiles per non-empty tensor
    std::vector<uint32_t> arrivals;     // one-pass scaled state: non-empty one-pass tiles per tensor
    uint32_t piece_tile[kMaxPieces + 1];    // scaled state: first tile of each piece, then the grid
    uint32_t piece_tensor[kMaxPieces + 1];  // scaled state: first tensor of each piece, then the tensors
};

// Dispatches that cover `tiles` tiles at most `per` at a time.
int32_t dispatch_count(uint32_t tiles, int32_t per)
{
    return int32_t((int64_t(tiles) + per - 1) / per);
}

// The position of one-pass tile u in the persistent kernel's order (the
// inverse of tile_of_block<kOneRun> over `total` tiles).
uint32_t one_position(uint32_t u, uint32_t total)
{
    constexpr uint32_t group = kXcds * kOneRun;
    if (u >= total - total % group) return u;
    const uint32_t q = u % group;
    return u - q + (q % kOneRun) * kXcds + q / kOneRun;
}

// A one-pass list's largest tensor, in one-pass tiles (2M elements): 512
// tiles, two thirds of one round of MI355X's resident grid (768 workgroups,
// 3 per compute unit), so that a workgroup's wait for a tensor is covered by
// the next tile it computes; the handle also checks the device's own grid
// (every tensor within 2 * grid - 1 positions).
constexpr int64_t kOneMaxTensorTiles = (int64_t(1) << 21) / kOneTile;  // tensors of at most 2M elements
constexpr uint32_t kOneRedoBlocks = 1024;  // workgroups of the follow-up pass
constexpr int kOneWaitUs = 200;            // default wait of a one-pass workgroup
constexpr int kOneGraceUs = 20;            // its wait while not every workgroup has started

// Splits a scaled-state list into pieces of consecutive tensors (see
// kMaxPieces): about equal tiles each, cut only at tensor boundaries, every
// piece at least kMinPieceTiles.  `ranges` holds each non-empty tensor's
// [first, end) tiles; fills tile[0..n] and tensor[0..n] (piece i is tiles
// [tile[i], tile[i+1]) and tensors [tensor[i], tensor[i+1])) and n.
void plan_pieces(const std::vector<uint32_t> &ranges, uint32_t tiles, uint32_t *tile, uint32_t *tensor, int32_t &n)
{
    const uint32_t count = uint32_t(ranges.size() / 2);
    const int want = piece_count(count, tiles);
    n = 0;
    tile[0] = 0;
    tensor[0] = 0;
    if (want >= 2) {
        // greedy: close a piece once it reaches its share of the tiles
        // still to cut, if what is left after it is a piece too
        uint32_t k = 0;
        while (n < want - 1) {
            const uint32_t first = tile[n];
            const uint64_t share = (uint64_t(tiles) - first) / uint64_t(want - n);
            while (k < count && ranges[2 * k + 1] - first < share) ++k;
            if (k >= count) break;
            const uint32_t end = ranges[2 * k + 1];  // the piece ends with tensor k
            if (end - first < kMinPieceTiles || tiles - end < kMinPieceTiles) break;
            ++k;
            ++n;
            tile[n] = end;
            tensor[n] = k;
        }
    }
    ++n;  // the last piece takes the rest
    tile[n] = tiles;
    tensor[n] = count;
}

bool valid_dtype_set(const adam_tl_desc &d)
{
    const bool g_ok = d.g == ADAM_DT_F32 || d.g == ADAM_DT_BF16 || d.g == ADAM_DT_F16;
    const bool p16 = d.p == ADAM_DT_BF16 || d.p == ADAM_DT_F16;
    const bool out16 = d.p_out == ADAM_DT_BF16 || d.p_out == ADAM_DT_F16;
    if (!g_ok || !(d.p_out == ADAM_DT_NONE || out16 || d.p_out == ADAM_DT_F32)) return false;
    if (d.with_remainders == 1) return d.p == ADAM_DT_BF16 && (d.p_out == ADAM_DT_NONE || d.p_out == ADAM_DT_BF16);
    if (d.scaled_state == 1) return p16 && d.p_out != ADAM_DT_F32;
    return d.p == ADAM_DT_F32 || p16;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

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

// The default chunk: the largest power of two up to 65536 elements whose
// workgroups past the end of tensors (the last item of each tensor rounds up
// to whole items) stay within 1% of the tiles that do work.
int64_t auto_chunk(const std::vector<int64_t> &sizes, int64_t tile)
{
    int64_t need = 0;
    for (int64_t n : sizes) need += (n + tile - 1) / tile;
    for (int64_t chunk = kAutoChunkMax; chunk > tile; chunk /= 2) {
        int64_t launched = 0;
        for (int64_t n : sizes) launched += (n + chunk - 1) / chunk * (chunk / tile);
        if ((launched - need) * 100 <= need) return chunk;
    }
    return tile;
}

// `alts` (nullable): the second buffer set of a two-buffer state, one entry
// per tensor with only p, m, v (and rem) set.
int make_plan(const adam_tensor *tensors, const adam_tensor *alts, int64_t count, const adam_tl_desc *desc,
              Plan &plan, bool keep_items)
{
    if (desc == nullptr || count < 0 || (count > 0 && tensors == nullptr)) return ADAM_EINVAL;
    if (desc->dispatch_tiles < 0) return ADAM_EINVAL;
    if (desc->scaled_passes < 0 || desc->scaled_passes > 2 || desc->scaled_wait_us < -1) return ADAM_EINVAL;
    if (desc->scaled_state != 1 && (desc->scaled_passes != 0 || desc->scaled_wait_us != 0)) return ADAM_EINVAL;
    if (desc->with_remainders != 0 && desc->with_remainders != 1) return ADAM_EINVAL;
    if (desc->scaled_state != 0 && desc->scaled_state != 1) return ADAM_EINVAL;
    if (desc->with_remainders == 1 && desc->scaled_state == 1) return ADAM_EINVAL;
    if (alts != nullptr && desc->scaled_state == 1) return ADAM_EINVAL;  // scaled state stays in place
    if (!valid_dtype_set(*desc)) return ADAM_EDTYPE;
    if (desc->chunk_elems != 0 &&
        (!is_pow2(desc->chunk_elems) || desc->chunk_elems < kMinChunk || desc->chunk_elems > kMaxChunk))
        return ADAM_EINVAL;

    const bool rem = desc->with_remainders == 1;
    const bool scaled = desc->scaled_state == 1;
    const bool out = desc->p_out != ADAM_DT_NONE;
    const uintptr_t p_size = desc->p == ADAM_DT_F32 ? 4 : 2;
    const uintptr_t mv_size = desc->p != ADAM_DT_F32 && !rem ? 2 : 4;  // 16-bit or scaled state
    const uintptr_t g_size = desc->g == ADAM_DT_F32 ? 4 : 2;
    const uintptr_t out_size = desc->p_out == ADAM_DT_F32 ? 4 : 2;
    const int64_t tile = kTile;

    adam_tl_stats st = {};
    st.tensors = count;
    st.bytes_per_elem =
        int32_t(2 * (p_size + (rem ? 2 : 0) + 2 * mv_size) + g_size + (out ? out_size : 0));
    st.block_threads = kBlock;
    st.tile_elems = int32_t(tile);
    st.device = -1;
    st.two_buffer = alts != nullptr ? 1 : 0;
    st.pieces = 1;

    std::vector<Span> spans;
    std::vector<int64_t> sizes;  // elements covered by records (a vector body excludes its head)
    std::vector<int32_t> heads;  // head elements of a vector tensor, -1 for the element path
    spans.reserve(size_t(count) * (alts != nullptr ? 11 : 7));
    for (int64_t k = 0; k < count; ++k) {
        const adam_tensor &t = tensors[k];
        if (t.numel < 0 || t.numel > kMaxNumel) return ADAM_EINVAL;
        if (alts != nullptr && alts[k].numel != t.numel) return ADAM_EINVAL;
        if (t.numel == 0) continue;
        if (t.p == nullptr || t.m == nullptr || t.v == nullptr || t.g == nullptr) return ADAM_EINVAL;
        if ((t.rem != nullptr) != rem || (t.p_out != nullptr) != out || (t.scales != nullptr) != scaled)
            return ADAM_EINVAL;
        const uintptr_t n = uintptr_t(t.numel);
        spans.push_back({uintptr_t(t.p), uintptr_t(t.p) + n * p_size, false});
        spans.push_back({uintptr_t(t.m), uintptr_t(t.m) + n * mv_size, false});
        spans.push_back({uintptr_t(t.v), uintptr_t(t.v) + n * mv_size, false});
        spans.push_back({uintptr_t(t.g), uintptr_t(t.g) + n * g_size, true});
        if (rem) spans.push_back({uintptr_t(t.rem), uintptr_t(t.rem) + n * 2, false});
        if (out) spans.push_back({uintptr_t(t.p_out), uintptr_t(t.p_out) + n * out_size, false});
        if (scaled) spans.push_back({uintptr_t(t.scales), uintptr_t(t.scales) + 3 * sizeof(float), false});
        if (alts != nullptr) {
            // the second set: p, m, v (and rem), each a multiple of 128 bytes
            // away from the first, so both sets share every alignment
            const adam_tensor &a = alts[k];
            if (a.p == nullptr || a.m == nullptr || a.v == nullptr || (a.rem != nullptr) != rem ||
                a.g != nullptr || a.p_out != nullptr || a.scales != nullptr)
                return ADAM_EINVAL;
            auto apart = [](const void *x, const void *y) {
                return (intptr_t(x) - intptr_t(y)) % 128 == 0;
            };
            if (!apart(a.p, t.p) || !apart(a.m, t.m) || !apart(a.v, t.v) || (rem && !apart(a.rem, t.rem)))
                return ADAM_EINVAL;
            spans.push_back({uintptr_t(a.p), uintptr_t(a.p) + n * p_size, false});
            spans.push_back({uintptr_t(a.m), uintptr_t(a.m) + n * mv_size, false});
            spans.push_back({uintptr_t(a.v), uintptr_t(a.v) + n * mv_size, false});
            if (rem) spans.push_back({uintptr_t(a.rem), uintptr_t(a.rem) + n * 2, false});
        }
        // every stream must be naturally aligned for its element type
        if (uintptr_t(t.p) % p_size || uintptr_t(t.m) % mv_size || uintptr_t(t.v) % mv_size ||
            uintptr_t(t.g) % g_size || (rem && uintptr_t(t.rem) % 2) ||
            (out && uintptr_t(t.p_out) % out_size) || (scaled && uintptr_t(t.scales) % 4))
            return ADAM_EINVAL;
        // The head: the fewest leading elements after which every stream sits
        // on a 128-byte boundary, else on the boundary of its 4-element access
        // (16 bytes for fp32, 8 for 16-bit streams), else none.
        auto all_aligned = [&](int64_t e, bool line) {
            auto ok = [&](const void *ptr, uintptr_t size) {
                const uintptr_t need = line ? 128u : uintptr_t(kLane) * size;
                return (uintptr_t(ptr) + uintptr_t(e) * size) % need == 0;
            };
            return ok(t.p, p_size) && ok(t.m, mv_size) && ok(t.v, mv_size) && ok(t.g, g_size) &&
                   (!rem || ok(t.rem, 2)) && (!out || ok(t.p_out, out_size));
        };
        int64_t head = -1;
        for (int64_t e = 0; e <= kMaxHead && e < t.numel && head < 0; ++e)
            if (all_aligned(e, true)) head = e;
        for (int64_t e = 0; e < kLane && e < t.numel && head < 0; ++e)
            if (all_aligned(e, false)) head = e;
        const bool vec = head >= 0;
        st.nonempty += 1;
        st.elements += t.numel;
        st.vector_tensors += vec ? 1 : 0;
        sizes.push_back(vec ? t.numel - head : t.numel);
        heads.push_back(vec ? int32_t(head) : -1);
    }
    if (spans_conflict(spans)) return ADAM_EINVAL;
    if (st.nonempty >= (int64_t(1) << 31) / 3) return ADAM_EINVAL;

    int64_t chunk = desc->chunk_elems != 0 ? desc->chunk_elems : auto_chunk(sizes, tile);
    // one-pass scaled state (only when asked: two passes, which depend on
    // nothing being resident, are the default) takes records of whole
    // one-pass tiles
    const bool want_one = scaled && desc->scaled_passes == 1;
    if (want_one && desc->chunk_elems == 0) chunk = std::max<int64_t>(chunk, kOneTile);
    uint32_t shift = 0;
    while ((tile << shift) < chunk) ++shift;
    for (int64_t n : sizes) st.chunks += (n + chunk - 1) / chunk;
    if ((st.chunks << shift) >= kMaxGrid) return ADAM_EINVAL;
    st.chunk_elems = chunk;
    st.grid_blocks = st.chunks << shift;
    st.dispatch_tiles = int32_t(desc->dispatch_tiles == 0 ? kDispatchTiles
                                                          : std::min<int64_t>(desc->dispatch_tiles, kDispatchTiles));
    plan.shift = shift;
    // each non-empty tensor's tiles [first, end): records are per tensor
    std::vector<uint32_t> &ranges = plan.tile_ranges;
    ranges.reserve(2 * sizes.size());
    int64_t records = 0;
    for (int64_t n : sizes) {
        ranges.push_back(uint32_t(records << shift));
        records += (n + chunk - 1) / chunk;
        ranges.push_back(uint32_t(records << shift));
    }
    st.pieces = 1;
    // one pass: every tensor's non-empty one-pass tiles, at most kOneMaxTensorTiles
    bool one = want_one && chunk % kOneTile == 0 && st.vector_tensors == st.nonempty;
    if (one) {
        plan.arrivals.reserve(sizes.size());
        for (int64_t n : sizes) {
            int64_t a = 0;
            for (int64_t off = 0; off < n; off += chunk) a += (std::min(chunk, n - off) + kOneTile - 1) / kOneTile;
            one = one && a <= kOneMaxTensorTiles;
            plan.arrivals.push_back(uint32_t(a));
        }
    }
    if (desc->scaled_passes == 1 && !one) return ADAM_EINVAL;
    if (scaled) st.scaled_passes = one ? 1 : 2;
    if (one) {
        plan.piece_tile[0] = 0;
        plan.piece_tile[1] = uint32_t(st.grid_blocks);
        plan.piece_tensor[0] = 0;
        plan.piece_tensor[1] = uint32_t(sizes.size());
        st.dispatches = 1;  // one persistent dispatch
    } else if (scaled) {
        plan.arrivals.clear();
        plan_pieces(ranges, uint32_t(st.grid_blocks), plan.piece_tile, plan.piece_tensor, st.pieces);
        for (int i = 0; i < st.pieces; ++i)
            st.dispatches += dispatch_count(plan.piece_tile[i + 1] - plan.piece_tile[i], st.dispatch_tiles);
    } else {
        plan.piece_tile[0] = 0;
        plan.piece_tile[1] = uint32_t(st.grid_blocks);
        plan.piece_tensor[0] = 0;
        plan.piece_tensor[1] = uint32_t(sizes.size());
        st.dispatches = dispatch_count(uint32_t(st.grid_blocks), st.dispatch_tiles);
    }
    plan.stats = st;
    if (!keep_items) return ADAM_OK;

    plan.items.reserve(size_t(st.chunks));
    size_t j = 0;
    for (int64_t k = 0; k < count; ++k) {
        const adam_tensor &t = tensors[k];
        if (t.numel == 0) continue;
        const int32_t ordinal = int32_t(j);
        const int32_t head = heads[j];
        const int64_t body = sizes[j++];
        const int64_t first = head > 0 ? head : 0;  // element index where records start
        if (scaled) plan.scale_ptrs.push_back(t.scales);
        for (int64_t off = 0; off < body; off += chunk) {
            const int64_t e = first + off;
            WorkItem w = {};
            w.p = static_cast<char *>(t.p) + e * int64_t(p_size);
            w.aux = rem ? static_cast<void *>(t.rem + e) : scaled ? static_cast<void *>(t.scales) : nullptr;
            w.m = static_cast<char *>(t.m) + e * int64_t(mv_size);
            w.v = static_cast<char *>(t.v) + e * int64_t(mv_size);
            w.g = static_cast<const char *>(t.g) + e * int64_t(g_size);
            w.p_out = out ? static_cast<char *>(t.p_out) + e * int64_t(out_size) : nullptr;
            w.n = int32_t(std::min(chunk, body - off));
            w.flags = head >= 0 ? kItemVector : 0u;
            w.head = off == 0 && head > 0 ? head : 0;
            w.tensor = ordinal;
            if (alts != nullptr) {
                const adam_tensor &a = alts[k];
                w.flags |= kItemTwoBuffer;
                w.alt[0] = intptr_t(a.p) - intptr_t(t.p);
                w.alt[1] = rem ? intptr_t(a.rem) - intptr_t(t.rem) : 0;
                w.alt[2] = intptr_t(a.m) - intptr_t(t.m);
                w.alt[3] = intptr_t(a.v) - intptr_t(t.v);
            }
            plan.items.push_back(w);
        }
    }
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


// What kind of storage a handle updates; each step entry point takes one.
enum class Kind { Plain, Remainders, Scaled };

}  // namespace

struct adam_tl {
    adam_tl_stats stats;
    uint32_t shift;
    Kind kind;
    int g;                 // adam_dtype of the gradients
    int p;                 // adam_dtype of the params (the state type when scaled)
    int out;               // adam_dtype of p_out, ADAM_DT_NONE if absent
    WorkItem *d_items;     // device table, null when there is no work
    StepBlock *d_block;    // device scalar block of the capturable steps (after the table)
    double *d_partials;    // reduction partial sums (after the block), one per kNormRun tiles
    uint32_t n_partials;
    float **d_scale_ptrs;  // scaled state: each non-empty tensor's scales (after the partials)
    uint32_t *d_tiles;     // scaled state: [first, end) tile range per non-empty tensor
    uint32_t *d_tile_max;  // scaled state: three magnitude maxima per tile
    uint32_t *d_folded;    // scaled state: three magnitude maxima, then three reciprocal scales, per non-empty tensor
    // one-pass scaled state (one_pass): per tensor its published reciprocal
    // scales, arrival count and non-empty one-pass tiles; the follow-up list
    bool one_pass;
    uint64_t *d_ready;
    uint32_t *d_count, *d_redo, *d_arrivals;
    uint32_t *d_started;
    uint64_t wait_ticks, grace_ticks;
    uint32_t wait_polls;
    uint32_t one_grid;     // workgroups of the persistent one-pass kernel
    uint32_t n_tensors;    // non-empty tensors
    int lds_per_cu;        // local data share bytes per compute unit of the device (0: unknown)
    // scaled state: the step's pieces (consecutive tensors), pipelined over
    // the caller's stream and `aux` when there are two or more
    int n_pieces;
    uint32_t piece_tile[kMaxPieces + 1];    // first tile of each piece, then the grid
    uint32_t piece_tensor[kMaxPieces + 1];  // first tensor of each piece, then n_tensors
    hipStream_t aux;                        // null unless n_pieces >= 2
    hipEvent_t ev[kMaxPieces + 2];          // fork, after each piece's maxima and fold, join
};

namespace {

// Workgroups of the update kept resident per compute unit, by storage:
// with fp32 moments each lane has 48-64 bytes of loads in flight, and the
// HBM delivers most for this read / write mix with about 50 KB of loads in
// flight per CU (~13 MB over the chip, what ~6.5 TB/s needs at ~2 us of
// loaded latency); more waves only queue and contend in the DRAM.
// Measured on MI355X (workgroups per CU 5..14 against no limit): 7 gave
// +6.0% on the 201 x 20.97M fp32 list, +3-4% on the bf16- and fp16-gradient
// ZeRO shards and on bf16 params with remainders.  16-bit state moves half
// the bytes per lane and needs every wave it can get (any limit was slower).
// The limit is imposed by reserving local data share the kernel never
// touches: the per-CU share divided by the limit, in 512-byte units.
constexpr int kResidentFp32Moments = 7;

size_t update_lds_reserve(const adam_tl *tl)
{
    const bool fp32_moments = tl->kind == Kind::Remainders || tl->p == kF32;
    if (!fp32_moments || tl->lds_per_cu <= 0) return 0;
    return size_t(tl->lds_per_cu / kResidentFp32Moments) / 512 * 512;
}

// Counts the launches a step has enqueued, so that a failure can tell
// whether anything of the step reached the stream.
struct Launches {
    int enqueued = 0;
    bool ok(hipError_t e)
    {
        if (e != hipSuccess) return false;
        ++enqueued;
        return true;
    }
};

// Enqueues kernel `fn` over tiles [t0, t1) as dispatches of at most
// `per` tiles, each told its first tile.
template <class Fn, class... Args>
bool launch_tiles(Launches &log, Fn fn, uint32_t t0, uint32_t t1, int32_t per, int threads, size_t lds,
                  hipStream_t stream, const WorkItem *items, uint32_t shift, Args... args)
{
    for (uint32_t first = t0; first < t1;) {
        const uint32_t n = uint32_t(std::min<int64_t>(per, int64_t(t1) - first));
        hipLaunchKernelGGL(fn, dim3(n), dim3(threads), lds, stream, items, shift, first, args...);
        if (!log.ok(hipGetLastError())) return false;
        first += n;
    }
    return true;
}

int launch_update(const adam_tl *tl, int mode, bool capturable, const StepArgs &args, hipStream_t stream,
                  Launches &log)
{
    const int pk = tl->kind == Kind::Remainders ? kParamRem
                   : tl->p == kBF16             ? kParamBF16
                   : tl->p == kF16              ? kParamF16
                                                : kParamF32;
    const int idx = type_pos(kGradTypes, 3, tl->g) +
                    3 * (pk + 4 * (type_pos(kUpdateOutTypes, 4, tl->out) + 4 * (mode + 2 * int(capturable))));
    const UpdateFn fn = UpdateKernels::fns[idx];
    if (fn == nullptr) return ADAM_EDTYPE;
    return launch_tiles(log, fn, 0u, uint32_t(tl->stats.grid_blocks), tl->stats.dispatch_tiles, kBlock,
                        update_lds_reserve(tl), stream, tl->d_items, tl->shift, args)
               ? ADAM_OK
               : ADAM_EHIP;
}

int launch_scaled(const adam_tl *tl, int mode, const StepArgs &args, hipStream_t stream, Launches &log)
{
    const int base = type_pos(kGradTypes, 3, tl->g) +
                     3 * (type_pos(kOutTypes, 3, tl->out) + 3 * (type_pos(kStateTypes, 2, tl->p) + 2 * mode));
    auto fold = tl->p == kBF16 ? adam_scaled_fold<kBF16> : adam_scaled_fold<kF16>;
    auto finish = tl->p == kBF16 ? adam_scaled_finish<kBF16> : adam_scaled_finish<kF16>;
    const int32_t per = tl->stats.dispatch_tiles;
    if (tl->one_pass) {
        // the one-pass kernel, its follow-up pass, the new scales
        const int idx = base;  // the one-pass tables use the scaled passes' order
        const OneArgs f = {tl->d_tiles,   tl->d_arrivals, tl->d_count,      tl->d_ready,     tl->d_tile_max,
                           tl->d_folded,  tl->d_redo,     tl->d_started,    tl->wait_ticks,  tl->grace_ticks,
                           tl->wait_polls, tl->n_tensors};
        const uint32_t shift = tl->shift - kOneSubLog;  // one-pass tiles per record: 2^shift
        const uint32_t tiles = uint32_t(tl->stats.grid_blocks) / kOneSub;
        hipLaunchKernelGGL(OneKernels::fns[idx], dim3(tl->one_grid), dim3(kOneBlock), 0, stream, tl->d_items, shift,
                           tiles, args, f);
        if (!log.ok(hipGetLastError())) return ADAM_EHIP;
        hipLaunchKernelGGL(OneKernels::redo[idx], dim3(std::min<uint32_t>(tiles, kOneRedoBlocks)), dim3(kOneBlock), 0,
                           stream, tl->d_items, shift, args, f);
        if (!log.ok(hipGetLastError())) return ADAM_EHIP;
        auto finish1 = tl->p == kBF16 ? adam_scaled_one_finish<kBF16> : adam_scaled_one_finish<kF16>;
        hipLaunchKernelGGL(finish1, dim3((tl->n_tensors + 255) / 256), dim3(256), 0, stream, tl->d_scale_ptrs, f,
                           tl->n_tensors, args.block);
        return log.ok(hipGetLastError()) ? ADAM_OK : ADAM_EHIP;
    }
    // piece i: its tiles' maxima, then its tensors' fold ...
    auto maxima = [&](int i, hipStream_t s) {
        const uint32_t k0 = tl->piece_tensor[i];
        if (!launch_tiles(log, ScaledKernels::fns[base], tl->piece_tile[i], tl->piece_tile[i + 1], per, kMaxBlock,
                          0, s, tl->d_items, tl->shift, args, tl->d_tile_max))
            return false;
        hipLaunchKernelGGL(fold, dim3(tl->piece_tensor[i + 1] - k0), dim3(kFoldMaxBlock), 0, s,
                           tl->d_tile_max, tl->d_tiles, tl->d_folded, k0, args.block);
        return log.ok(hipGetLastError());
    };
    // ... and its store pass, then its tensors' new scales
    auto store = [&](int i, hipStream_t s) {
        const uint32_t k0 = tl->piece_tensor[i], k1 = tl->piece_tensor[i + 1];
        if (!launch_tiles(log, ScaledKernels::fns[base + 36], tl->piece_tile[i], tl->piece_tile[i + 1], per, kBlock,
                          0, s, tl->d_items, tl->shift, args, tl->d_folded))
            return false;
        hipLaunchKernelGGL(finish, dim3((k1 - k0 + 255) / 256), dim3(256), 0, s, tl->d_scale_ptrs, tl->d_folded,
                           k0, k1, args.block);
        return log.ok(hipGetLastError());
    };
    if (tl->n_pieces <= 1) return maxima(0, stream) && store(0, stream) ? ADAM_OK : ADAM_EHIP;
    // Pieces alternate between the caller's stream and aux; piece i starts
    // once piece i-1's maxima and fold are done, so its maxima pass runs
    // beside piece i-1's store pass.  Events fork aux from the caller's
    // stream and join it back (the same pattern holds under graph capture).
    if (hipEventRecord(tl->ev[0], stream) != hipSuccess || hipStreamWaitEvent(tl->aux, tl->ev[0], 0) != hipSuccess)
        return ADAM_EHIP;
    for (int i = 0; i < tl->n_pieces; ++i) {
        hipStream_t s = i % 2 == 0 ? stream : tl->aux;
        if (i > 0 && hipStreamWaitEvent(s, tl->ev[i], 0) != hipSuccess) return ADAM_EHIP;
        if (!maxima(i, s) || hipEventRecord(tl->ev[i + 1], s) != hipSuccess || !store(i, s)) return ADAM_EHIP;
    }
    const int j = tl->n_pieces + 1;
    if (hipEventRecord(tl->ev[j], tl->aux) != hipSuccess || hipStreamWaitEvent(stream, tl->ev[j], 0) != hipSuccess)
        return ADAM_EHIP;
    return ADAM_OK;
}

// The arguments of a non-capturable step whose counter was `before`.
StepArgs host_args(const adam_hparams *hp, float lr, int32_t before, float grad_scale, const float *d_grad_scale)
{
    const int32_t t = before + 1;
    StepArgs a = {};
    a.lr = lr;
    a.beta1 = hp->beta1;
    a.beta2 = hp->beta2;
    a.eps = hp->eps;
    a.weight_decay = hp->weight_decay;
    a.grad_scale = grad_scale;
    a.d_grad_scale = d_grad_scale;
    a.side = int32_t(uint32_t(before) & 1u);  // two-buffer state: the set the step reads
    step_corrections(hp->beta1, hp->beta2, t, hp->bias_correction, a.bc1, a.bc2, a.rbc1, a.rbc2);
    return a;
}

int host_step(const adam_tl *tl, const adam_hparams *hp, float lr, int32_t *step_io, float grad_scale,
              const float *d_grad_scale, hipStream_t stream, Kind want)
{
    if (tl == nullptr || step_io == nullptr || !valid_hparams(hp)) return ADAM_EINVAL;
    if (tl->kind != want) return ADAM_EINVAL;
    const int32_t before = *step_io;
    if (before < 0 || before == INT32_MAX) return ADAM_EINVAL;
    *step_io = before + 1;  // the counter advances even for a list with no elements
    if (tl->stats.chunks == 0) return ADAM_OK;
    const StepArgs a = host_args(hp, lr, before, grad_scale, d_grad_scale);
    DeviceGuard guard(tl->stats.device);
    int rc = ADAM_EHIP;
    Launches log;
    if (guard.status == hipSuccess)
        rc = want == Kind::Scaled ? launch_scaled(tl, hp->mode, a, stream, log)
                                  : launch_update(tl, hp->mode, false, a, stream, log);
    // a failure before anything was enqueued leaves the counter; once part
    // of the step is on the stream the counter stays with the step
    if (rc != ADAM_OK && log.enqueued == 0) *step_io = before;
    return rc;
}

int capturable_step(const adam_tl *tl, const adam_hparams *hp, const float *d_lr, int32_t *d_step,
                    const float *d_grad_scale, const int32_t *d_noop, hipStream_t stream, Kind want)
{
    if (tl == nullptr || d_lr == nullptr || d_step == nullptr || !valid_hparams(hp)) return ADAM_EINVAL;
    if (tl->kind != want) return ADAM_EINVAL;
    int device = tl->stats.device;
    if (device < 0 && hipGetDevice(&device) != hipSuccess) return ADAM_EHIP;
    DeviceGuard guard(device);
    if (guard.status != hipSuccess) return ADAM_EHIP;
    hipLaunchKernelGGL(adam_capture_prologue, dim3(1), dim3(64), 0, stream, tl->d_block, d_lr, d_step,
                       d_grad_scale, d_noop, hp->beta1, hp->beta2, hp->bias_correction);
    if (hipGetLastError() != hipSuccess) return ADAM_EHIP;
    if (tl->stats.chunks == 0) return ADAM_OK;
    StepArgs a = {};
    a.beta1 = hp->beta1;
    a.beta2 = hp->beta2;
    a.eps = hp->eps;
    a.weight_decay = hp->weight_decay;
    a.block = tl->d_block;
    Launches log;
    return want == Kind::Scaled ? launch_scaled(tl, hp->mode, a, stream, log)
                                : launch_update(tl, hp->mode, true, a, stream, log);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

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
    case ADAM_ETOOBIG: return "list needs more work-table records than the static scratch holds (65536)";
    default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// Destroys the pipelining stream and events of a handle (if any).
void release_pieces(adam_tl *tl)
{
    for (hipEvent_t &e : tl->ev) {
        if (e != nullptr) (void)hipEventDestroy(e);
        e = nullptr;
    }
    if (tl->aux != nullptr) (void)hipStreamDestroy(tl->aux);
    tl->aux = nullptr;
    tl->n_pieces = 1;
}

// Creates the second stream and the events that pipeline a scaled-state
// list planned in two or more pieces.  Anything that cannot be created
// leaves one piece (the same results, one sequence of launches).
void start_pieces(adam_tl *tl)
{
    if (tl->n_pieces < 2) return;
    bool ok = hipStreamCreateWithFlags(&tl->aux, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; ok && i < tl->n_pieces + 2; ++i)
        ok = hipEventCreateWithFlags(&tl->ev[i], hipEventDisableTiming) == hipSuccess;
    if (ok) return;
    (void)hipGetLastError();
    release_pieces(tl);
    const uint32_t tiles = uint32_t(tl->stats.grid_blocks);
    tl->stats.pieces = 1;
    tl->stats.dispatches = dispatch_count(tiles, tl->stats.dispatch_tiles);
    tl->piece_tile[1] = tiles;
    tl->piece_tensor[1] = tl->n_tensors;
}

int plan_tl(const adam_tensor *tensors, const adam_tensor *alts, int64_t count, const adam_tl_desc *desc,
            adam_tl_stats *stats)
{
    if (stats == nullptr) return ADAM_EINVAL;
    Plan plan;
    int rc;
    try {
        rc = make_plan(tensors, alts, count, desc, plan, false);
    } catch (const std::bad_alloc &) {
        return ADAM_ENOMEM;
    }
    if (rc == ADAM_OK) *stats = plan.stats;
    return rc;
}

// Whether the device keeps at least twice the largest tensor's one-pass
// workgroups resident (else tl->one_pass is cleared, or, when the caller
// asked for one pass, ADAM_EINVAL); sets the wait in real-time clock ticks.
int one_pass_fits(adam_tl *tl, int device, Plan &plan, const adam_tl_desc *desc)
{
    int cus = 0, khz = 0, per_cu = INT32_MAX;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) != hipSuccess)
        return ADAM_EHIP;
    for (int mode = 0; mode < 2; ++mode) {
        const int idx = type_pos(kGradTypes, 3, tl->g) +
                        3 * (type_pos(kOutTypes, 3, tl->out) + 3 * (type_pos(kStateTypes, 2, tl->p) + 2 * mode));
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void *>(OneKernels::fns[idx]),
                                                         kOneBlock, 0) != hipSuccess)
            return ADAM_EHIP;
        per_cu = std::min(per_cu, nb);
    }
    // the persistent grid: every workgroup the device keeps resident (or
    // the caller's smaller figure), at most one per tile
    const uint32_t total = uint32_t(tl->stats.grid_blocks / kOneSub);
    int64_t grid = std::min<int64_t>(int64_t(per_cu) * cus, total);
    if (desc->dispatch_tiles != 0) grid = std::min<int64_t>(grid, std::max(1, desc->dispatch_tiles / int32_t(kOneSub)));
    // no workgroup may hold three tiles of one tensor: every tensor's tiles
    // must lie within 2 * grid - 1 consecutive positions
    // (and each tensor's arrivals counted per spread counter)
    bool fits = grid > 0;
    const uint32_t shift = tl->shift - kOneSubLog;
    const size_t n = plan.arrivals.size();
    std::vector<uint32_t> spread((1 + kOneSpread) * n, 0u);
    for (size_t k = 0; fits && k < n; ++k) {
        const uint32_t lo = plan.tile_ranges[2 * k] / kOneSub, hi = plan.tile_ranges[2 * k + 1] / kOneSub;
        uint32_t first = UINT32_MAX, end = 0;
        for (uint32_t u = lo; u < hi; ++u) {
            if (int64_t(u & ((1u << shift) - 1u)) * kOneTile >= plan.items[u >> shift].n) continue;
            const uint32_t p = one_position(u, total);
            first = std::min(first, p);
            end = std::max(end, p + 1);
            ++spread[(1 + p % kOneSpread) * n + k];
        }
        fits = end <= first || int64_t(end - first) < 2 * grid;
        for (uint32_t s = 0; s < kOneSpread; ++s) spread[k] += spread[(1 + s) * n + k] != 0u ? 1u : 0u;
    }
    if (!fits) {
        if (desc->scaled_passes == 1) return ADAM_EINVAL;
        tl->one_pass = false;
        return ADAM_OK;
    }
    plan.arrivals.swap(spread);
    tl->one_grid = uint32_t(grid);
    const int64_t us = desc->scaled_wait_us == 0 ? kOneWaitUs : std::max(0, desc->scaled_wait_us);
    tl->wait_ticks = uint64_t(us) * uint64_t(std::max(khz, 1)) / 1000u;
    if (us > 0 && tl->wait_ticks == 0) tl->wait_ticks = 1;
    tl->grace_ticks = std::min<uint64_t>(tl->wait_ticks, uint64_t(kOneGraceUs) * uint64_t(std::max(khz, 1)) / 1000u);
    // a poll (a device-coherent load and a sleep of 1024 cycles) takes well
    // over 0.25 us, so this many polls outlast the wait: the loop ends even
    // if the clock did not advance
    tl->wait_polls = us > 0 ? uint32_t(4 * us + 16) : 0u;
    return ADAM_OK;
}

int build_tl(const adam_tensor *tensors, const adam_tensor *alts, int64_t count, const adam_tl_desc *desc,
             hipStream_t stream, adam_tl **out)
{
    if (out == nullptr) return ADAM_EINVAL;
    *out = nullptr;
    Plan plan;
    int rc;
    try {
        rc = make_plan(tensors, alts, count, desc, plan, true);
    } catch (const std::bad_alloc &) {
        return ADAM_ENOMEM;
    }
    if (rc != ADAM_OK) return rc;

    adam_tl *tl = new (std::nothrow) adam_tl();
    if (tl == nullptr) return ADAM_ENOMEM;
    tl->stats = plan.stats;
    tl->shift = plan.shift;
    tl->kind = desc->with_remainders == 1 ? Kind::Remainders
               : desc->scaled_state == 1  ? Kind::Scaled
                                          : Kind::Plain;
    tl->g = desc->g;
    tl->p = desc->p;
    tl->out = desc->p_out;
    tl->d_items = nullptr;
    tl->d_block = nullptr;
    tl->d_partials = nullptr;
    tl->n_partials = 0;
    tl->d_scale_ptrs = nullptr;
    tl->d_tiles = nullptr;
    tl->d_tile_max = nullptr;
    tl->d_folded = nullptr;
    tl->one_pass = plan.stats.scaled_passes == 1;
    tl->d_ready = nullptr;
    tl->d_arrivals = tl->d_count = tl->d_redo = nullptr;
    tl->d_started = nullptr;
    tl->wait_ticks = tl->grace_ticks = 0;
    tl->wait_polls = 0;
    tl->one_grid = 0;
    tl->n_tensors = uint32_t(plan.stats.nonempty);
    tl->lds_per_cu = 0;
    tl->n_pieces = plan.stats.pieces;
    std::copy(plan.piece_tile, plan.piece_tile + tl->n_pieces + 1, tl->piece_tile);
    std::copy(plan.piece_tensor, plan.piece_tensor + tl->n_pieces + 1, tl->piece_tensor);
    tl->aux = nullptr;
    for (hipEvent_t &e : tl->ev) e = nullptr;
    if (plan.items.empty()) {  // nothing to launch: no device state at all
        *out = tl;
        return ADAM_OK;
    }

    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) {
        delete tl;
        return ADAM_EHIP;
    }
    tl->stats.device = device;
    if (hipDeviceGetAttribute(&tl->lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, device) !=
        hipSuccess) {
        (void)hipGetLastError();
        tl->lds_per_cu = 0;  // no limit
    }
    tl->n_partials = uint32_t((tl->stats.grid_blocks + kNormRun - 1) / kNormRun);
    if (tl->one_pass) {
        // one pass needs each tensor's workgroups resident together: its
        // largest tensor must fit in half of what the device keeps resident
        int rc1 = one_pass_fits(tl, device, plan, desc);
        if (rc1 != ADAM_OK) {
            delete tl;
            return rc1;
        }
        if (!tl->one_pass) {  // two passes after all
            plan.arrivals.clear();
            plan_pieces(plan.tile_ranges, uint32_t(tl->stats.grid_blocks), plan.piece_tile, plan.piece_tensor,
                        tl->stats.pieces);
            tl->stats.scaled_passes = 2;
            tl->stats.dispatches = 0;
            for (int i = 0; i < tl->stats.pieces; ++i)
                tl->stats.dispatches +=
                    dispatch_count(plan.piece_tile[i + 1] - plan.piece_tile[i], tl->stats.dispatch_tiles);
            tl->n_pieces = tl->stats.pieces;
            std::copy(plan.piece_tile, plan.piece_tile + tl->n_pieces + 1, tl->piece_tile);
            std::copy(plan.piece_tensor, plan.piece_tensor + tl->n_pieces + 1, tl->piece_tensor);
        }
    }
    // layout: [work table][scalar block][partial sums][scale pointers]
    //         [tile ranges][per-tile maxima][per-tensor maxima]
    //         [one pass: published reciprocal scales (three 64-bit words)
    //          and counts per tensor; follow-up list; started count;
    //          arrivals per tensor]
    const bool scaled = tl->kind == Kind::Scaled;
    const size_t table_bytes = plan.items.size() * sizeof(WorkItem);
    const size_t block_off = table_bytes;
    const size_t partials_off = block_off + sizeof(StepBlock);
    const size_t ptrs_off = align_up(partials_off + tl->n_partials * sizeof(double), 8);
    const size_t tiles_off = ptrs_off + plan.scale_ptrs.size() * sizeof(float *);
    const size_t tile_max_off = tiles_off + (scaled ? plan.tile_ranges.size() * sizeof(uint32_t) : 0);
    const size_t folded_off =
        tile_max_off + (scaled ? 3 * sizeof(uint32_t) * size_t(tl->stats.grid_blocks) : 0);
    const size_t one_off = align_up(folded_off + (scaled ? 6 * sizeof(uint32_t) * tl->n_tensors : 0), 8);
    const size_t one_tiles = size_t(tl->stats.grid_blocks / kOneSub);
    // the part that starts at zero: published scales, counts, follow-up list
    const size_t counters = (1 + kOneSpread) * size_t(tl->n_tensors);
    const size_t one_zero = 3 * sizeof(uint64_t) * tl->n_tensors + sizeof(uint32_t) * (counters + 2 + one_tiles);
    const size_t total = one_off + (tl->one_pass ? one_zero + sizeof(uint32_t) * counters : 0);
    void *mem = nullptr;
    if (hipMalloc(&mem, total) != hipSuccess) {
        (void)hipGetLastError();
        delete tl;
        return ADAM_ENOMEM;
    }
    char *base = static_cast<char *>(mem);
    tl->d_items = reinterpret_cast<WorkItem *>(base);
    tl->d_block = reinterpret_cast<StepBlock *>(base + block_off);
    tl->d_partials = reinterpret_cast<double *>(base + partials_off);
    if (scaled) {
        tl->d_scale_ptrs = reinterpret_cast<float **>(base + ptrs_off);
        tl->d_tiles = reinterpret_cast<uint32_t *>(base + tiles_off);
        tl->d_tile_max = reinterpret_cast<uint32_t *>(base + tile_max_off);
        tl->d_folded = reinterpret_cast<uint32_t *>(base + folded_off);
    }
    if (tl->one_pass) {
        tl->d_ready = reinterpret_cast<uint64_t *>(base + one_off);
        tl->d_count = reinterpret_cast<uint32_t *>(tl->d_ready + 3 * size_t(tl->n_tensors));
        tl->d_redo = tl->d_count + counters;
        tl->d_started = tl->d_redo + 1 + one_tiles;
        tl->d_arrivals = tl->d_started + 1;
    }
    bool ok = hipMemcpyAsync(tl->d_items, plan.items.data(), table_bytes, hipMemcpyHostToDevice,
                             stream) == hipSuccess;
    if (ok && scaled)
        ok = hipMemcpyAsync(tl->d_scale_ptrs, plan.scale_ptrs.data(),
                            plan.scale_ptrs.size() * sizeof(float *), hipMemcpyHostToDevice,
                            stream) == hipSuccess &&
             hipMemcpyAsync(tl->d_tiles, plan.tile_ranges.data(),
                            plan.tile_ranges.size() * sizeof(uint32_t), hipMemcpyHostToDevice,
                            stream) == hipSuccess;
    if (ok && tl->one_pass)
        ok = hipMemcpyAsync(tl->d_arrivals, plan.arrivals.data(), plan.arrivals.size() * sizeof(uint32_t),
                            hipMemcpyHostToDevice, stream) == hipSuccess &&
             hipMemsetAsync(tl->d_ready, 0, one_zero, stream) == hipSuccess;
    if (!ok || hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipFree(mem);
        delete tl;
        return ADAM_EHIP;
    }
    if (scaled) start_pieces(tl);
    *out = tl;
    return ADAM_OK;
}

}  // namespace

extern "C" {

int adam_tl_plan(const adam_tensor *tensors, int64_t count, const adam_tl_desc *desc,
                 adam_tl_stats *stats)
{
    return plan_tl(tensors, nullptr, count, desc, stats);
}

int adam_tl_plan_two_buffer(const adam_tensor *tensors, const adam_tensor *alternates, int64_t count,
                            const adam_tl_desc *desc, adam_tl_stats *stats)
{
    if (count > 0 && alternates == nullptr) return ADAM_EINVAL;
    static const adam_tensor kNone[1] = {};  // an empty list: nothing to read
    return plan_tl(tensors, alternates != nullptr ? alternates : kNone, count, desc, stats);
}

int adam_tl_build(const adam_tensor *tensors, int64_t count, const adam_tl_desc *desc,
                  hipStream_t stream, adam_tl **out)
{
    return build_tl(tensors, nullptr, count, desc, stream, out);
}

int adam_tl_build_two_buffer(const adam_tensor *tensors, const adam_tensor *alternates, int64_t count,
                             const adam_tl_desc *desc, hipStream_t stream, adam_tl **out)
{
    if (count > 0 && alternates == nullptr) {
        if (out != nullptr) *out = nullptr;
        return ADAM_EINVAL;
    }
    static const adam_tensor kNone[1] = {};  // an empty list: nothing to read
    return build_tl(tensors, alternates != nullptr ? alternates : kNone, count, desc, stream, out);
}

void adam_tl_destroy(adam_tl *tl)
{
    if (tl == nullptr) return;
    if (tl->d_items != nullptr) {
        DeviceGuard guard(tl->stats.device);
        release_pieces(tl);
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
    return host_step(tl, hp, lr, step_io, grad_scale, d_grad_scale, stream, Kind::Plain);
}

int adam_step_remainders(const adam_tl *tl, const adam_hparams *hp, float lr, int32_t *step_io,
                         float grad_scale, const float *d_grad_scale, hipStream_t stream)
{
    return host_step(tl, hp, lr, step_io, grad_scale, d_grad_scale, stream, Kind::Remainders);
}

int adam_step_scaled(const adam_tl *tl, const adam_hparams *hp, float lr, int32_t *step_io,
                     float grad_scale, const float *d_grad_scale, hipStream_t stream)
{
    return host_step(tl, hp, lr, step_io, grad_scale, d_grad_scale, stream, Kind::Scaled);
}

int adam_step_capturable(const adam_tl *tl, const adam_hparams *hp, const float *d_lr, int32_t *d_step,
                         const float *d_grad_scale, const int32_t *d_noop, hipStream_t stream)
{
    return capturable_step(tl, hp, d_lr, d_step, d_grad_scale, d_noop, stream, Kind::Plain);
}

int adam_step_remainders_capturable(const adam_tl *tl, const adam_hparams *hp, const float *d_lr,
                                    int32_t *d_step, const float *d_grad_scale,
                                    const int32_t *d_noop, hipStream_t stream)
{
    return capturable_step(tl, hp, d_lr, d_step, d_grad_scale, d_noop, stream, Kind::Remainders);
}

int adam_step_scaled_capturable(const adam_tl *tl, const adam_hparams *hp, const float *d_lr, int32_t *d_step,
                                const float *d_grad_scale, const int32_t *d_noop, hipStream_t stream)
{
    return capturable_step(tl, hp, d_lr, d_step, d_grad_scale, d_noop, stream, Kind::Scaled);
}

int adam_grad_sumsq(const adam_tl *tl, double *d_sumsq, int32_t accumulate, hipStream_t stream)
{
    if (tl == nullptr || d_sumsq == nullptr || (accumulate != 0 && accumulate != 1)) return ADAM_EINVAL;
    int device = tl->stats.device;
    if (device < 0 && hipGetDevice(&device) != hipSuccess) return ADAM_EHIP;
    DeviceGuard guard(device);
    if (guard.status != hipSuccess) return ADAM_EHIP;
    if (tl->n_partials > 0) {
        auto fn = tl->g == kF32    ? grad_sumsq_partial<kF32>
                  : tl->g == kBF16 ? grad_sumsq_partial<kBF16>
                                   : grad_sumsq_partial<kF16>;
        hipLaunchKernelGGL(fn, dim3(tl->n_partials), dim3(kBlock), 0, stream, tl->d_items, tl->shift,
                           uint32_t(tl->stats.grid_blocks), kNormRun, tl->d_partials);
        if (hipGetLastError() != hipSuccess) return ADAM_EHIP;
    }
    hipLaunchKernelGGL(grad_sumsq_fold, dim3(1), dim3(kFoldBlock), 0, stream, tl->d_partials,
                       tl->n_partials, d_sumsq, accumulate);
    return hipGetLastError() == hipSuccess ? ADAM_OK : ADAM_EHIP;
}

int adam_clip_grad_scale(const double *d_sumsq, float *d_grad_scale, float max_norm, float *d_norm,
                         int32_t *d_noop, hipStream_t stream)
{
    if (d_sumsq == nullptr || max_norm != max_norm) return ADAM_EINVAL;
    if (max_norm > 0.0f && d_grad_scale == nullptr) return ADAM_EINVAL;
    hipLaunchKernelGGL(clip_grad_scale_kernel, dim3(1), dim3(64), 0, stream, d_sumsq, d_grad_scale,
                       max_norm, d_norm, d_noop);
    return hipGetLastError() == hipSuccess ? ADAM_OK : ADAM_EHIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The step without a handle, for callers that cannot allocate device memory:
// its work table goes to a static device array instead of a handle's
// allocation.  Every call on a device shares that device's copy of the
// array, so calls that overlap on one device race.
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kScratchItems = 65536;  // work-table records: 8 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) WorkItem scratch[kScratchItems];

struct ScratchOfDevice {
    WorkItem *table = nullptr;  // the device's copy of `scratch`
    int lds_per_cu = 0;
};
std::mutex scratch_mutex;
ScratchOfDevice scratch_of_device[kMaxDevices];

// The device address of `scratch` on `device` (current), looked up once per
// device; the array's host-side name is not a device address.
int scratch_table(int device, ScratchOfDevice &out)
{
    if (device < 0 || device >= kMaxDevices) return ADAM_EHIP;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    ScratchOfDevice &d = scratch_of_device[device];
    if (d.table == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return ADAM_EHIP;
        }
        if (hipDeviceGetAttribute(&d.lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, device) !=
            hipSuccess) {
            (void)hipGetLastError();
            d.lds_per_cu = 0;
        }
        d.table = static_cast<WorkItem *>(ptr);
    }
    out = d;
    return ADAM_OK;
}

// Plans a list for the static table: with an automatic chunk, the chunk is
// doubled until the table fits, while that still merges records (a tensor
// takes at least one record; coarser records also round tensor ends up to
// more tiles).
int plan_for_scratch(const adam_tensor *tensors, int64_t count, const adam_tl_desc *desc, Plan &plan)
{
    int rc = make_plan(tensors, nullptr, count, desc, plan, true);
    adam_tl_desc d = *desc;
    while (rc == ADAM_OK && int64_t(plan.items.size()) > kScratchItems) {
        if (desc->chunk_elems != 0 || plan.stats.chunks == plan.stats.nonempty ||
            plan.stats.chunk_elems >= kMaxChunk)
            return ADAM_ETOOBIG;
        d.chunk_elems = std::max(kMinChunk, plan.stats.chunk_elems * 2);
        plan = Plan();
        rc = make_plan(tensors, nullptr, count, &d, plan, true);
        if (rc != ADAM_OK) return ADAM_ETOOBIG;  // the list planned, but not at a coarser chunk
    }
    return rc;
}

}  // namespace

extern "C" {

int adam_step_noalloc(const adam_tensor *tensors, int64_t count, const adam_tl_desc *desc,
                      const adam_hparams *hp, float lr, int32_t *step_io, float grad_scale,
                      const float *d_grad_scale, hipStream_t stream)
{
    if (desc == nullptr || step_io == nullptr || !valid_hparams(hp)) return ADAM_EINVAL;
    if (desc->with_remainders != 0 || desc->scaled_state != 0) return ADAM_EINVAL;  // adam_step's storage
    const int32_t before = *step_io;
    if (before < 0 || before == INT32_MAX) return ADAM_EINVAL;
    Plan plan;
    int rc;
    try {
        rc = plan_for_scratch(tensors, count, desc, plan);
    } catch (const std::bad_alloc &) {
        return ADAM_ENOMEM;
    }
    if (rc != ADAM_OK) return rc;
    if (plan.items.empty()) {
        *step_io = before + 1;  // the counter advances even for a list with no elements
        return ADAM_OK;
    }
    int device = 0;
    ScratchOfDevice sd;
    if (hipGetDevice(&device) != hipSuccess) return ADAM_EHIP;
    rc = scratch_table(device, sd);
    if (rc != ADAM_OK) return rc;
    // the table is enqueued behind earlier work on `stream` (which may still
    // read the previous table) and the host waits for the copy, so the
    // planned records can be released on return
    if (hipMemcpyAsync(sd.table, plan.items.data(), plan.items.size() * sizeof(WorkItem), hipMemcpyHostToDevice,
                       stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipGetLastError();
        return ADAM_EHIP;
    }
    adam_tl tl{};
    tl.stats = plan.stats;
    tl.stats.device = device;
    tl.shift = plan.shift;
    tl.kind = Kind::Plain;
    tl.g = desc->g;
    tl.p = desc->p;
    tl.out = desc->p_out;
    tl.d_items = sd.table;
    tl.lds_per_cu = sd.lds_per_cu;
    tl.n_pieces = 1;
    *step_io = before + 1;
    Launches log;
    rc = launch_update(&tl, hp->mode, false, host_args(hp, lr, before, grad_scale, d_grad_scale), stream, log);
    if (rc != ADAM_OK && log.enqueued == 0) *step_io = before;
    return rc;
}
}  // extern "C"
