// select.hip -- active-set selection on gfx950: exact top-k and threshold compaction.
//
// Top-k: "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm", section
// "The Prediction Problem" -- the k largest predictor scores are the active set.  Among equal
// scores the lower neuron index wins; -0.0 equals +0.0; the list is written in ascending order.
// Threshold: "Activation sparsity", section "Implementation sketch" -- active = scores >= threshold.
//
// One 1024-thread workgroup per token.  Thread t owns the contiguous index range
// [t*J, t*J + J) (J = ceil(f/1024)) and keeps those scores in registers, so every pass after the
// first load runs out of registers and LDS:
//   1. scores -> order-preserving 32-bit keys (binary32 sign/magnitude mapped onto unsigned order,
//      -0.0 folded onto +0.0);
//   2. radix select, 8 bits per pass, LDS histogram: finds T, the k-th largest key, and `need`,
//      how many keys equal to T belong in the set (the lowest-indexed ones);
//   3. one block-wide exclusive scan of the per-thread count of keys equal to T gives each
//      thread its tie rank; a second scan of the per-thread selection count gives each thread
//      its output position, so the list comes out in ascending index order with no sort.
#include "common.hpp"
#include "launch.hpp"

namespace csf {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxWords = 2048;            // bitmap words held in LDS: f <= 65536

__device__ __forceinline__ uint32_t order_key(float s)
{
    uint32_t u = __float_as_uint(s);
    if ((u & 0x7fffffffu) == 0u)
        u = 0u;                                   // -0.0 ranks as +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void clear_words(uint32_t *bm, int words)
{
    for (int w = threadIdx.x; w < words; w += kSelThreads)
        bm[w] = 0u;
}

__device__ __forceinline__ void store_words(const uint32_t *bm, int words, uint32_t *out)
{
    for (int w = threadIdx.x; w < words; w += kSelThreads)
        out[w] = bm[w];
}

template <int J>
__global__ __launch_bounds__(kSelThreads) void k_select_topk(const float *__restrict__ scores,
                                                             int f, int Jr, int k,
                                                             int32_t *__restrict__ idx,
                                                             int idx_stride,
                                                             int32_t *__restrict__ count,
                                                             uint32_t *__restrict__ bitmap)
{
    __shared__ uint32_t hist[256];
    __shared__ uint32_t scan_tmp[kSelWaves];
    __shared__ uint32_t pick[2];
    __shared__ uint32_t bm[kMaxWords];

    const int t = threadIdx.x;
    const int token = blockIdx.x;
    const float *s = scores + (size_t)token * f;
    const int words = (f + 31) / 32;
    const int base = t * Jr;
    int nvalid = f - base;
    nvalid = nvalid < 0 ? 0 : (nvalid > Jr ? Jr : nvalid);

    if (bitmap)
        clear_words(bm, words);
    if (t == 0 && count)
        count[token] = k;

    uint32_t key[J];
#pragma unroll
    for (int q = 0; q < J; ++q)
        key[q] = q < nvalid ? order_key(s[base + q]) : 0u;

    uint32_t T = 0u, need = 0u;
    if (k > 0) {
        uint32_t prefix = 0u, pmask = 0u, krem = (uint32_t)k;
#pragma unroll 1
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (t < 256)
                hist[t] = 0u;
            __syncthreads();
#pragma unroll
            for (int q = 0; q < J; ++q)
                if (q < nvalid && (key[q] & pmask) == prefix)
                    atomicAdd(&hist[(key[q] >> shift) & 0xffu], 1u);
            __syncthreads();
            if (t < kWave) {
                // lane l holds digits 4l..4l+3; find the digit where the count of keys with a
                // larger digit is < krem and including this digit's keys reaches krem
                const uint32_t c0 = hist[4 * t], c1 = hist[4 * t + 1];
                const uint32_t c2 = hist[4 * t + 2], c3 = hist[4 * t + 3];
                const uint32_t local = c0 + c1 + c2 + c3;
                uint32_t suffix = local;               // sum over lanes >= t
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    uint32_t n = __shfl_down(suffix, o, kWave);
                    if (t + o < kWave)
                        suffix += n;
                }
                uint32_t above = suffix - local;       // keys in digits > 4t+3
                const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
                for (int b = 3; b >= 0; --b) {
                    if (above < krem && above + cs[b] >= krem) {
                        pick[0] = (uint32_t)(4 * t + b);
                        pick[1] = krem - above;
                    }
                    above += cs[b];
                }
            }
            __syncthreads();
            const uint32_t digit = pick[0];
            krem = pick[1];
            prefix |= digit << shift;
            pmask |= 0xffu << shift;
            __syncthreads();
        }
        T = prefix;
        need = krem;
    }

    // per-thread counts of keys above T and equal to T
    uint32_t cgt = 0u, ceq = 0u;
    if (k > 0) {
#pragma unroll
        for (int q = 0; q < J; ++q) {
            if (q < nvalid) {
                cgt += key[q] > T ? 1u : 0u;
                ceq += key[q] == T ? 1u : 0u;
            }
        }
    }
    uint32_t total;
    const uint32_t eq_before = block_exclusive_scan<kSelWaves>(ceq, scan_tmp, &total);
    uint32_t take_eq = 0u;
    if (need > eq_before)
        take_eq = (need - eq_before) < ceq ? (need - eq_before) : ceq;
    const uint32_t nsel = cgt + take_eq;
    uint32_t pos = block_exclusive_scan<kSelWaves>(nsel, scan_tmp, &total);

    if (nsel) {
        int32_t *out = idx + (size_t)token * idx_stride;
        uint32_t er = eq_before;
#pragma unroll
        for (int q = 0; q < J; ++q) {
            if (q < nvalid) {
                bool sel = key[q] > T;
                if (key[q] == T) {
                    sel = er < need;
                    ++er;
                }
                if (sel) {
                    const int j = base + q;
                    if (pos < (uint32_t)idx_stride)
                        out[pos] = j;
                    ++pos;
                    if (bitmap)
                        atomicOr(&bm[j >> 5], 1u << (j & 31));
                }
            }
        }
    }
    if (bitmap) {
        __syncthreads();
        store_words(bm, words, bitmap + (size_t)token * words);
    }
}

template <int J>
__global__ __launch_bounds__(kSelThreads) void k_select_threshold(
    const float *__restrict__ scores, int f, int Jr, float tau, int32_t *__restrict__ idx,
    int idx_stride, int32_t *__restrict__ count, uint32_t *__restrict__ bitmap)
{
    __shared__ uint32_t scan_tmp[kSelWaves];
    __shared__ uint32_t bm[kMaxWords];

    const int t = threadIdx.x;
    const int token = blockIdx.x;
    const float *s = scores + (size_t)token * f;
    const int words = (f + 31) / 32;
    const int base = t * Jr;
    int nvalid = f - base;
    nvalid = nvalid < 0 ? 0 : (nvalid > Jr ? Jr : nvalid);

    if (bitmap)
        clear_words(bm, words);

    float v[J];
#pragma unroll
    for (int q = 0; q < J; ++q)
        v[q] = q < nvalid ? s[base + q] : 0.0f;
    uint32_t nsel = 0u;
#pragma unroll
    for (int q = 0; q < J; ++q)
        nsel += (q < nvalid && v[q] >= tau) ? 1u : 0u;
    uint32_t total;
    uint32_t pos = block_exclusive_scan<kSelWaves>(nsel, scan_tmp, &total);
    if (t == 0)
        count[token] = (int32_t)total;
    if (nsel) {
        int32_t *out = idx + (size_t)token * idx_stride;
#pragma unroll
        for (int q = 0; q < J; ++q) {
            if (q < nvalid && v[q] >= tau) {
                const int j = base + q;
                if (pos < (uint32_t)idx_stride)
                    out[pos] = j;
                ++pos;
                if (bitmap)
                    atomicOr(&bm[j >> 5], 1u << (j & 31));
            }
        }
    }
    if (bitmap) {
        __syncthreads();
        store_words(bm, words, bitmap + (size_t)token * words);
    }
}

int per_thread(int f) { return (f + kSelThreads - 1) / kSelThreads; }

}  // namespace

int select_max_f() { return 64 * kSelThreads; }

hipError_t launch_select_topk(const float *scores, int B, int f, int k, int32_t *idx,
                              int idx_stride, int32_t *count, uint32_t *bitmap, hipStream_t st)
{
    const int Jr = per_thread(f);
    dim3 grid(B), block(kSelThreads);
#define CSF_TOPK(JJ) \
    k_select_topk<JJ><<<grid, block, 0, st>>>(scores, f, Jr, k, idx, idx_stride, count, bitmap)
    if (Jr <= 1) CSF_TOPK(1);
    else if (Jr <= 2) CSF_TOPK(2);
    else if (Jr <= 4) CSF_TOPK(4);
    else if (Jr <= 8) CSF_TOPK(8);
    else if (Jr <= 16) CSF_TOPK(16);
    else if (Jr <= 32) CSF_TOPK(32);
    else if (Jr <= 64) CSF_TOPK(64);
    else return hipErrorInvalidValue;
#undef CSF_TOPK
    return hipGetLastError();
}

hipError_t launch_select_threshold(const float *scores, int B, int f, float tau, int32_t *idx,
                                   int idx_stride, int32_t *count, uint32_t *bitmap,
                                   hipStream_t st)
{
    const int Jr = per_thread(f);
    dim3 grid(B), block(kSelThreads);
#define CSF_THR(JJ) \
    k_select_threshold<JJ><<<grid, block, 0, st>>>(scores, f, Jr, tau, idx, idx_stride, count, \
                                                   bitmap)
    if (Jr <= 1) CSF_THR(1);
    else if (Jr <= 2) CSF_THR(2);
    else if (Jr <= 4) CSF_THR(4);
    else if (Jr <= 8) CSF_THR(8);
    else if (Jr <= 16) CSF_THR(16);
    else if (Jr <= 32) CSF_THR(32);
    else if (Jr <= 64) CSF_THR(64);
    else return hipErrorInvalidValue;
#undef CSF_THR
    return hipGetLastError();
}

}  // namespace csf
