// common.hpp -- storage-type traits, 16-byte vector loads and wavefront/block reductions shared by
// the gfx950 kernels of the contextual-sparsity FFN library.
//
// Every weight row is streamed in 16-byte chunks (one global_load_dwordx4 per lane, 1 KiB per
// 64-lane wavefront instruction).  A chunk holds E elements of the storage type: 4 float32 or 8
// binary16 / bfloat16 values.  Dot products accumulate in float32: binary16 and bfloat16 pairs go
// through the packed dot2 instructions (products of 16-bit values are exact in float32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csf {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Buckets of the score histogram that top-k selection starts from.
constexpr int kScoreBuckets = 2048;

// Counters that workgroups of one kernel add to and poll each sit in a 128-byte line of their own
// (a line that is polled while it takes many atomic adds serialises both).
constexpr int kLineWords = 32;

// Monotone, non-decreasing map of a score to a bucket in [0, NB): uniform buckets over [0, 1]
// (the range of a sigmoid); values below 0 (and NaN, the lowest in the selection's order) land in
// bucket 0, values >= 1 in NB - 1.
// Scaling by NB is exact (a power of two) and truncation of a non-negative float is its floor.
template <int NB>
__device__ __forceinline__ int score_bucket(float s)
{
    const float v = fminf(fmaxf(s * (float)NB, 0.0f), (float)(NB - 1));
    return (int)v;
}

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Streaming load of a weight chunk that is read once per call: non-temporal so that it does not
// evict the small, reused operands (x, a, h, index lists) from the caches.
__device__ __forceinline__ u32x4 ld_stream(const u32x4 *p) { return __builtin_nontemporal_load(p); }

struct F32T {
    static constexpr int E = 4;
    __device__ static __forceinline__ float dot(u32x4 w, u32x4 x, float acc)
    {
        acc = fmaf(u2f(w.x), u2f(x.x), acc);
        acc = fmaf(u2f(w.y), u2f(x.y), acc);
        acc = fmaf(u2f(w.z), u2f(x.z), acc);
        acc = fmaf(u2f(w.w), u2f(x.w), acc);
        return acc;
    }
    __device__ static __forceinline__ void unpack(u32x4 w, float *o)
    {
        o[0] = u2f(w.x); o[1] = u2f(w.y); o[2] = u2f(w.z); o[3] = u2f(w.w);
    }
};

struct F16T {
    static constexpr int E = 8;
    __device__ static __forceinline__ float dot(u32x4 w, u32x4 x, float acc)
    {
        acc = __builtin_amdgcn_fdot2(as_f16x2(w.x), as_f16x2(x.x), acc, false);
        acc = __builtin_amdgcn_fdot2(as_f16x2(w.y), as_f16x2(x.y), acc, false);
        acc = __builtin_amdgcn_fdot2(as_f16x2(w.z), as_f16x2(x.z), acc, false);
        acc = __builtin_amdgcn_fdot2(as_f16x2(w.w), as_f16x2(x.w), acc, false);
        return acc;
    }
    __device__ static __forceinline__ void unpack(u32x4 w, float *o)
    {
        f16x2 p;
        p = as_f16x2(w.x); o[0] = (float)p.x; o[1] = (float)p.y;
        p = as_f16x2(w.y); o[2] = (float)p.x; o[3] = (float)p.y;
        p = as_f16x2(w.z); o[4] = (float)p.x; o[5] = (float)p.y;
        p = as_f16x2(w.w); o[6] = (float)p.x; o[7] = (float)p.y;
    }
    // D += A B on one 16x16x32 matrix-core tile; A and B hold 8 binary16 values per lane
    __device__ static __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    // largest power of two a value split into 16-bit terms may reach unscaled: binary16 holds
    // magnitudes up to 65504, so |v| >= 2^15 is scaled down first (split_shift below)
    static constexpr int kSplitExp = 15;
    // round to nearest even (the conversion instruction's default mode)
    __device__ static __forceinline__ uint16_t round_bits(float v)
    {
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    }
    __device__ static __forceinline__ float widen_bits(uint16_t b)
    {
        return (float)__builtin_bit_cast(_Float16, b);
    }
};

struct BF16T {
    static constexpr int E = 8;
    __device__ static __forceinline__ float dot(u32x4 w, u32x4 x, float acc)
    {
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.x), as_bf16x2(x.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.y), as_bf16x2(x.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.z), as_bf16x2(x.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.w), as_bf16x2(x.w), acc, false);
        return acc;
    }
    // a bfloat16 value is the upper half of the binary32 pattern with the same value
    __device__ static __forceinline__ void unpack(u32x4 w, float *o)
    {
        o[0] = u2f(w.x << 16); o[1] = u2f(w.x & 0xffff0000u);
        o[2] = u2f(w.y << 16); o[3] = u2f(w.y & 0xffff0000u);
        o[4] = u2f(w.z << 16); o[5] = u2f(w.z & 0xffff0000u);
        o[6] = u2f(w.w << 16); o[7] = u2f(w.w & 0xffff0000u);
    }
    __device__ static __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // bfloat16 has binary32's exponent range: only |v| >= 2^127 (next to overflow) is scaled
    static constexpr int kSplitExp = 127;
    // round to nearest even on the bit pattern (finite inputs)
    __device__ static __forceinline__ uint16_t round_bits(float v)
    {
        const uint32_t u = __float_as_uint(v);
        return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    }
    __device__ static __forceinline__ float widen_bits(uint16_t b) { return u2f((uint32_t)b << 16); }
};

// ---- scaled split of float32 values into 16-bit terms ------------------------------------------
// A float32 vector v that feeds a 16-bit matrix-core product is written as v = t0 + t1 (+ t2),
// t0 = round(v), t1 = round(v - t0), ...  For binary16 that overflows once |v| reaches 65520, so
// the split is taken of v 2^k instead, with k <= 0 chosen from the largest |v| of the vector (its
// float32 bits with the sign cleared, `maxbits`) so that the largest scaled value lies in
// [2^(E-1), 2^E), E = T::kSplitExp; the product is multiplied by 2^-k afterwards.  Powers of
// two scale exactly, so k = 0 (every |v| < 2^E, the common case) leaves the bits unchanged, and
// a non-finite maximum gets k = 0 (nothing to rescale: the outputs are non-finite).
template <class T>
__device__ __forceinline__ bool split_needs_scale(uint32_t absbits)
{
    return absbits >= (uint32_t)(127 + T::kSplitExp) << 23;
}
template <class T>
__device__ __forceinline__ int split_shift(uint32_t maxbits)
{
    if (!split_needs_scale<T>(maxbits) || maxbits >= 0x7f800000u)
        return 0;
    return T::kSplitExp - 1 - ((int)(maxbits >> 23) - 127);   // in [kSplitExp - 128, -1]
}
// 2^k for k in [-126, 127]
__device__ __forceinline__ float pow2_exact(int k) { return u2f((uint32_t)(127 + k) << 23); }

// ---- hand-over between workgroups of one kernel -------------------------------------------------
// Each XCD has its own L2, and the L2s are not coherent with one another.  Values that one
// workgroup hands to another inside the same kernel therefore travel with the device-coherent
// policy (agent-scope relaxed atomics: the store is written through to, and the load is served
// from, the level all XCDs share), and a counter says when they are complete.  The producer
// waits until its own coherent stores are acknowledged before it adds to the counter, so a
// consumer that sees the count and then issues coherent loads reads the new values.  This costs
// no L2 write-back or invalidate (which a release/acquire fence at agent scope would add).
__device__ __forceinline__ void st_coherent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coherent_u32(const uint32_t *p)
{
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this thread issued has completed (stores acknowledged).
__device__ __forceinline__ void wait_own_memory()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ void count_add(uint32_t *p, uint32_t v)
{
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Polls of a hand-over counter before a waiting workgroup gives up (about 2^15 round trips of a
// microsecond or less).  A consumer only ever waits for workgroups with lower indices, which the
// hardware dispatches first, so the count always arrives; the bound only guarantees that a
// kernel ends even if that did not hold: the waiter then records the failure in *err (read by
// the tests) and goes on.
constexpr uint32_t kSpinLimit = 1u << 15;
// A value that marks "not written yet" in a buffer of float32 results handed over inside a kernel:
// a NaN bit pattern (all ones) that float32 arithmetic on finite inputs never produces; a producer
// whose inputs may carry NaN payloads stores every NaN as the default quiet NaN 0x7fc00000.
constexpr uint32_t kHSentinel = 0xffffffffu;
__device__ __forceinline__ void wait_count(const uint32_t *p, uint32_t target, uint32_t *err)
{
    for (uint32_t it = 0; it < kSpinLimit; ++it) {
        if (ld_coherent_u32(p) >= target)
            return;
        __builtin_amdgcn_s_sleep(4);
    }
    count_add(err, 1u);
}

// Activation codes (the csf_act values): 0 ReLU, 1 ReGLU, 2 SiLU, 3 SwiGLU.  The gated forms
// multiply the gate activation by the up projection W_up x.
__host__ __device__ constexpr bool act_gated(int act) { return act == 1 || act == 3; }
__host__ __device__ constexpr int act_silu(int act) { return act == 2 || act == 3 ? 1 : 0; }

// The gate nonlinearity of the FFN: ReLU (the ReLU and ReLU-fied gated forms) or SiLU,
// silu(p) = p / (1 + exp(-p)) (the LLaMA-style forms, never exactly zero).
__device__ __forceinline__ float gate_act(float p, int silu)
{
    return silu ? p / (1.0f + expf(-p)) : (p > 0.0f ? p : 0.0f);
}

// Order of the top-k selection: a monotone 32-bit key of a float32 score (-0.0 ranks as +0.0; a
// NaN ranks below every number, -inf included), and a (score, index) pair as one integer, larger
// first: score descending, index ascending.
__device__ __forceinline__ uint32_t order_key(float s)
{
    uint32_t u = __float_as_uint(s);
    if ((u & 0x7fffffffu) == 0u)
        u = 0u;
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int j)
{
    return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - (uint32_t)j);
}

// Sum over the 64 lanes of a wavefront; every lane receives the total.  The butterfly order is
// fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, kWave);
    return v;
}

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane of a group receives its
// group's total.
template <int G>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, kWave);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wavefront, with DPP cross-lane moves (no LDS
// round trips): inside each 16-lane row, adds of the value 1, 2, 4 and 8 lanes lower (lanes with
// no such source add 0); then the row totals are carried across rows -- lane 15 of row 0 into row
// 1 and of row 2 into row 3 (row_bcast:15 with rows 1 and 3 enabled), then lane 31 into rows 2
// and 3 (row_bcast:31).  Disabled rows take the `old` operand, 0.  Every lane must be active.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v)
{
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);    // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);    // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);    // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);    // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return (uint32_t)x;
}

// Exclusive prefix sum over a workgroup of NW wavefronts (blockDim.x == 64 * NW).  `scratch` is
// LDS of at least NW words; the call contains two barriers and must be reached by every thread.
template <int NW>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *scratch,
                                                         uint32_t *total)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const uint32_t incl = wave_inclusive_scan(v);
    if (lane == kWave - 1)
        scratch[w] = incl;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        uint32_t s = scratch[i];
        before += (i < w) ? s : 0u;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

// Ascending list of the set bits of an LDS bitmap: out[wpos[w] + rank of bit b in word w] =
// 32 w + b, where wpos (LDS) holds the exclusive prefix of the words' popcounts and `total` the
// number of set bits.  A sparse bitmap (at most 12 bits per word on average) is emitted by the
// words' owners, thread t walking the bits of words t wpt .. t wpt + wpt - 1; a denser one by half
// wavefronts, one word each with lane b taking bit b, so that a wavefront's stores go to
// consecutive addresses.  Both give the same list.  Positions >= cap are dropped.  Every thread of
// the NT-thread block calls.
template <int NT>
__device__ __forceinline__ void emit_bit_list(const uint32_t *words, const uint32_t *wpos, int nwords,
                                              uint32_t total, int32_t *out, int cap)
{
    if (total <= 12u * (uint32_t)nwords) {
        const int wpt = (nwords + NT - 1) / NT;
        for (int q = 0; q < wpt; ++q) {
            const int w = threadIdx.x * wpt + q;
            if (w >= nwords)
                break;
            uint32_t bits = words[w];
            uint32_t p = wpos[w];
            while (bits) {
                const int b = __ffs(bits) - 1;
                bits &= bits - 1;
                if (p < (uint32_t)cap)
                    out[p] = 32 * w + b;
                ++p;
            }
        }
        return;
    }
    const int half = threadIdx.x >> 5, bit = threadIdx.x & 31;
#pragma unroll 4
    for (int w = half; w < nwords; w += NT / 32) {
        const uint32_t v = words[w];
        if ((v >> bit) & 1u) {
            const uint32_t p = wpos[w] + __popc(v & ((1u << bit) - 1u));
            if (p < (uint32_t)cap)
                out[p] = 32 * w + bit;
        }
    }
}

}  // namespace csf
