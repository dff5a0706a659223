// stack.hip -- the residual-stream step between layers of a stack, on gfx950.
//
// [CP] "Contextual Sparsity and Activation Predictors", section "The predictor and its budget":
// the residual stream changes slowly from block to block, which is what lets layer l+1's active
// set be predicted from layer l's input.  Each block here reads the normalised stream
// xhat = x / sqrt(mean(x^2) + eps) (or x itself in literal mode), rounded once to the weight type;
// the block's output is added back to the float32 stream by the FFN's partial-sum reduction.
//
//   k_rms_norm  one 1024-thread workgroup per token, the row held in registers: fixed-order sum of
//               squares (so the result is deterministic), the scale, the rounding to the storage
//               type; optional copies of the stream and of xhat for inspection.  It also prepares
//               the hand-over state of the block's one-kernel FFN (counters cleared, h slots
//               marked unwritten): it runs after the previous block's FFN and before this one's,
//               on the same stream.
#include "common.hpp"
#include "launch.hpp"

namespace csf {

namespace {

constexpr int kNormThreads = 1024;

template <int DT>
__device__ __forceinline__ void store_elem(void *p, size_t i, float v)
{
    if constexpr (DT == 0)
        static_cast<float *>(p)[i] = v;
    else if constexpr (DT == 1)
        static_cast<uint16_t *>(p)[i] = F16T::round_bits(v);
    else
        static_cast<uint16_t *>(p)[i] = BF16T::round_bits(v);
}

// One 1024-thread workgroup per token.  Thread t holds float4 chunks t, t + 1024, ... (NPT of
// them) in registers, all loaded before the first use; the sum of squares is reduced in a fixed
// order (lanes, then waves), so the scale is deterministic.
template <int DT, int NPT>
__global__ __launch_bounds__(kNormThreads) void k_rms_norm(const float *__restrict__ x, int d,
                                                           float eps, int norm,
                                                           void *__restrict__ xhat,
                                                           float *__restrict__ x_log,
                                                           void *__restrict__ xhat_log,
                                                           uint32_t *__restrict__ zero, int nzero,
                                                           uint32_t *__restrict__ fill, int nfill)
{
    __shared__ float red[kNormThreads / kWave];
    for (int i = blockIdx.x * kNormThreads + threadIdx.x; i < nzero; i += gridDim.x * kNormThreads)
        zero[i] = 0u;
    for (int i = blockIdx.x * kNormThreads + threadIdx.x; i < nfill; i += gridDim.x * kNormThreads)
        fill[i] = kHSentinel;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const size_t base = (size_t)blockIdx.x * d;
    const float4 *xt = reinterpret_cast<const float4 *>(x + base);
    const int n4 = d / 4;
    float4 v[NPT];
#pragma unroll
    for (int q = 0; q < NPT; ++q) {
        const int c = t + kNormThreads * q;
        v[q] = c < n4 ? xt[c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    float scale = 1.0f;
    if (norm) {
        float ss = 0.0f;
#pragma unroll
        for (int q = 0; q < NPT; ++q) {
            ss = fmaf(v[q].x, v[q].x, ss);
            ss = fmaf(v[q].y, v[q].y, ss);
            ss = fmaf(v[q].z, v[q].z, ss);
            ss = fmaf(v[q].w, v[q].w, ss);
        }
        ss = wave_sum(ss);
        if (lane == 0)
            red[w] = ss;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int i = 0; i < kNormThreads / kWave; ++i)
            tot += red[i];
        scale = 1.0f / sqrtf(tot / (float)d + eps);
    }
#pragma unroll
    for (int q = 0; q < NPT; ++q) {
        const int c = t + kNormThreads * q;
        if (c >= n4)
            break;
        const float e[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            store_elem<DT>(xhat, base + 4 * c + i, e[i] * scale);
            if (xhat_log)
                store_elem<DT>(xhat_log, base + 4 * c + i, e[i] * scale);
        }
        if (x_log)
            reinterpret_cast<float4 *>(x_log + base)[c] = v[q];
    }
}

template <int DT>
hipError_t norm_dt(const float *x, int B, int d, float eps, int norm, void *xhat, float *x_log,
                   void *xhat_log, uint32_t *zero, int nzero, uint32_t *fill, int nfill,
                   hipStream_t st)
{
    const int npt = (d / 4 + kNormThreads - 1) / kNormThreads;
    if (npt <= 1)
        return launch(k_rms_norm<DT, 1>, dim3(B), dim3(kNormThreads), st, nullptr, x, d, eps, norm,
                      xhat, x_log, xhat_log, zero, nzero, fill, nfill);
    if (npt <= 2)
        return launch(k_rms_norm<DT, 2>, dim3(B), dim3(kNormThreads), st, nullptr, x, d, eps, norm,
                      xhat, x_log, xhat_log, zero, nzero, fill, nfill);
    if (npt <= 4)
        return launch(k_rms_norm<DT, 4>, dim3(B), dim3(kNormThreads), st, nullptr, x, d, eps, norm,
                      xhat, x_log, xhat_log, zero, nzero, fill, nfill);
    if (npt <= 8)
        return launch(k_rms_norm<DT, 8>, dim3(B), dim3(kNormThreads), st, nullptr, x, d, eps, norm,
                      xhat, x_log, xhat_log, zero, nzero, fill, nfill);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rms_norm(int dtype, const float *x, int B, int d, float eps, int norm, void *xhat,
                           float *x_log, void *xhat_log, hipStream_t st, uint32_t *zero,
                           int nzero, uint32_t *fill, int nfill)
{
    if (!zero)
        nzero = 0;
    if (!fill)
        nfill = 0;
    if (B <= 0)
        return hipSuccess;
    if (d % 4 != 0)
        return hipErrorInvalidValue;
    if (dtype == 0)
        return norm_dt<0>(x, B, d, eps, norm, xhat, x_log, xhat_log, zero, nzero, fill, nfill, st);
    if (dtype == 1)
        return norm_dt<1>(x, B, d, eps, norm, xhat, x_log, xhat_log, zero, nzero, fill, nfill, st);
    return norm_dt<2>(x, B, d, eps, norm, xhat, x_log, xhat_log, zero, nzero, fill, nfill, st);
}

}  // namespace csf
