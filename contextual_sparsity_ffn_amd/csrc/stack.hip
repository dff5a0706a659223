// stack.hip -- the residual-stream step between layers of a stack, on gfx950.
//
// [CP] "Contextual Sparsity and Activation Predictors", section "The predictor and its budget":
// the residual stream changes slowly from block to block, which is what lets layer l+1's active
// set be predicted from layer l's input.  Each block here reads the normalised stream
// xhat = x / sqrt(mean(x^2) + eps) (or x itself in literal mode), rounded once to the weight type;
// the block's output is added back to the float32 stream by the FFN's partial-sum reduction.
//
//   k_rms_norm  one 256-thread workgroup per token: fixed-order sum of squares (so the result is
//               deterministic), the scale, the rounding to the storage type; optional copies of
//               the stream and of xhat for inspection.
#include "common.hpp"
#include "launch.hpp"

namespace csf {

namespace {

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

template <int DT>
__global__ __launch_bounds__(256) void k_rms_norm(const float *__restrict__ x, int d, float eps,
                                                  int norm, void *__restrict__ xhat,
                                                  float *__restrict__ x_log,
                                                  void *__restrict__ xhat_log)
{
    __shared__ float red[4];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const size_t base = (size_t)blockIdx.x * d;
    const float *xt = x + base;
    float scale = 1.0f;
    if (norm) {
        float ss = 0.0f;
        for (int c = t; c < d; c += 256)
            ss = fmaf(xt[c], xt[c], ss);
        ss = wave_sum(ss);
        if (lane == 0)
            red[w] = ss;
        __syncthreads();
        const float tot = (red[0] + red[1]) + (red[2] + red[3]);
        scale = 1.0f / sqrtf(tot / (float)d + eps);
    }
    for (int c = t; c < d; c += 256) {
        const float v = xt[c];
        store_elem<DT>(xhat, base + c, v * scale);
        if (x_log)
            x_log[base + c] = v;
        if (xhat_log)
            store_elem<DT>(xhat_log, base + c, v * scale);
    }
}

}  // namespace

hipError_t launch_rms_norm(int dtype, const float *x, int B, int d, float eps, int norm, void *xhat,
                           float *x_log, void *xhat_log, hipStream_t st)
{
    if (B <= 0)
        return hipSuccess;
    if (dtype == 0)
        return launch(k_rms_norm<0>, dim3(B), dim3(256), st, nullptr, x, d, eps, norm, xhat, x_log,
                      xhat_log);
    if (dtype == 1)
        return launch(k_rms_norm<1>, dim3(B), dim3(256), st, nullptr, x, d, eps, norm, xhat, x_log,
                      xhat_log);
    return launch(k_rms_norm<2>, dim3(B), dim3(256), st, nullptr, x, d, eps, norm, xhat, x_log,
                  xhat_log);
}

}  // namespace csf
