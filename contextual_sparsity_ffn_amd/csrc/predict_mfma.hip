// predict_mfma.hip -- the activation predictor for a batch of tokens on the matrix cores (gfx950).
//
// "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm", section "The
// Prediction Problem": scores = sigmoid(U relu(V x)) for every token, V: d -> r, U: r -> f.
//
// With B tokens the two projections are skinny GEMMs, [B x d] x [d x r] and [B x r] x [r x f].  The
// vector-ALU kernels of predict.hip walk the tokens one after another, so each token's hidden
// vector costs a round trip to L2; here the tokens are the M side of 16x16x32 MFMA tiles (padded to
// 16 or 32), so every weight row is read once for the whole batch:
//   k_pred_down_mfma  tile of 16 rows of V x (a range of the d steps); the 4 waves of a workgroup
//                     split that range and are summed in order; float32 partial sums out;
//   k_pred_hidden     one workgroup per token: a = relu(sum of the partials, in order), written
//                     as NA 16-bit terms of a 2^k, a 2^k = t0 + t1 (+ t2) (t0 = round(a 2^k),
//                     t1 = round(a 2^k - t0), ...): about 22 bits of a for binary16 (NA = 2) and
//                     24 for bfloat16 (NA = 3), so the products with U (exact in float32) lose
//                     nothing the float32 scores would keep.  k = 0 unless the token's largest a
//                     reaches the 16-bit split limit (2^15 for binary16); the up projection
//                     multiplies the token's sums by 2^-k before the sigmoid;
//   k_pred_up_mfma    tile of 16 rows of U, the 4 waves split r; sigmoid epilogue
//                     (k_pred_up_mfma_res when r <= 512: the hidden terms held in registers
//                     across the tiles of a 512-workgroup grid).
// MFMA lane layout: lane l holds A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16], e < 8,
// and receives D[4 (l / 16) + i][l % 16], i < 4 (A = tokens x K, B = K x rows).
#include "common.hpp"
#include "launch.hpp"

namespace csf {

namespace {

constexpr int kRing = 4;           // K steps of loads in flight per wave

// 4 waves' 16x16 (x MT) accumulators summed in wave order; thread e of the workgroup receives
// element e = (m, i, lane): token 16 m + 4 (lane / 16) + i, row lane % 16.
template <int MT>
__device__ __forceinline__ void sum_waves(float (*red)[MT * 4][kWave], const f32x4 *acc, int w,
                                          int lane)
{
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[w][m * 4 + i][lane] = acc[m][i];
}

template <class T, int MT>
__global__ __launch_bounds__(256) void k_pred_down_mfma(const u32x4 *__restrict__ V,
                                                        const u32x4 *__restrict__ X, int B, int C,
                                                        int r, int ks_n, float *__restrict__ part)
{
    __shared__ float red[4][MT * 4][kWave];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int ln = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16, ks = blockIdx.y;
    const int steps = C / 4;
    const int sa = ks * steps / ks_n, sz = (ks + 1) * steps / ks_n;
    const int s0 = sa + w * (sz - sa) / 4, s1 = sa + (w + 1) * (sz - sa) / 4;
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
    const u32x4 *wr = V + (size_t)(n0 + ln) * C;
    const u32x4 *xr[MT];
    bool xok[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int tok = 16 * m + ln;
        xok[m] = tok < B;
        xr[m] = X + (size_t)(xok[m] ? tok : 0) * C;
    }
    f32x4 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (s1 > s0) {
        u32x4 rw[kRing], rx[kRing][MT];
        auto fill = [&](int p, int st) {
            const int c = 4 * (st < s1 ? st : s1 - 1) + g;
            rw[p] = ld_stream(wr + c);
#pragma unroll
            for (int m = 0; m < MT; ++m)
                rx[p][m] = xr[m][c];
        };
#pragma unroll
        for (int p = 0; p < kRing; ++p)
            fill(p, s0 + p);
        const int groups = (s1 - s0 + kRing - 1) / kRing;
        for (int gi = 0; gi < groups; ++gi) {
#pragma unroll
            for (int p = 0; p < kRing; ++p) {
                const bool ok = s0 + gi * kRing + p < s1;
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    acc[m] = T::mfma((ok && xok[m]) ? rx[p][m] : zero, rw[p], acc[m]);
                fill(p, s0 + (gi + 1) * kRing + p);
            }
        }
    }
    sum_waves<MT>(red, acc, w, lane);
    __syncthreads();
    for (int e = t; e < MT * 4 * kWave; e += 256) {
        const int mi = e / kWave, l = e % kWave;
        const int tok = 16 * (mi / 4) + 4 * (l >> 4) + (mi % 4);
        if (tok < B)
            part[((size_t)ks * B + tok) * r + n0 + (l & 15)] =
                (red[0][mi][l] + red[1][mi][l]) + (red[2][mi][l] + red[3][mi][l]);
    }
}

constexpr int kHiddenThreads = 1024;
constexpr int kHiddenKeep = 4;     // hidden values per thread kept in registers between the passes

template <class T, int NA>
__global__ __launch_bounds__(kHiddenThreads) void k_pred_hidden(const float *__restrict__ part,
                                                                int ks_n, int B, int r,
                                                                uint16_t *__restrict__ ahid,
                                                                float *__restrict__ hinv)
{
    __shared__ uint32_t wmax[kHiddenThreads / kWave];
    const int tok = blockIdx.x, t = threadIdx.x;
    const float *pt = part + (size_t)tok * r;
    const size_t kstride = (size_t)B * r;
    auto hidden = [&](int j) {
        float a = 0.0f;
#pragma unroll 8
        for (int ks = 0; ks < ks_n; ++ks)
            a += pt[ks * kstride + j];
        return a > 0.0f ? a : 0.0f;
    };
    // pass 1: the token's largest a (a >= 0, so its float32 bits order like its value)
    float keep[kHiddenKeep];
    uint32_t mx = 0u;
#pragma unroll
    for (int q = 0; q < kHiddenKeep; ++q) {
        const int j = t + kHiddenThreads * q;
        keep[q] = j < r ? hidden(j) : 0.0f;
        mx = max(mx, __float_as_uint(keep[q]));
    }
    for (int j = t + kHiddenThreads * kHiddenKeep; j < r; j += kHiddenThreads)
        mx = max(mx, __float_as_uint(hidden(j)));
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    if ((t & (kWave - 1)) == 0)
        wmax[t / kWave] = mx;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kHiddenThreads / kWave; ++i)
        mx = max(mx, wmax[i]);
    // pass 2: the terms of a 2^k (values past the kept ones are recomputed in the same order)
    const int k = split_shift<T>(mx);
    const float sc = pow2_exact(k);
    if (t == 0)
        hinv[tok] = pow2_exact(-k);
    auto put = [&](int j, float a) {
        a *= sc;
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            const uint16_t b = T::round_bits(a);
            ahid[((size_t)e * B + tok) * r + j] = b;
            a -= T::widen_bits(b);
        }
    };
#pragma unroll
    for (int q = 0; q < kHiddenKeep; ++q) {
        const int j = t + kHiddenThreads * q;
        if (j < r)
            put(j, keep[q]);
    }
    for (int j = t + kHiddenThreads * kHiddenKeep; j < r; j += kHiddenThreads)
        put(j, hidden(j));
}

template <class T, int MT, int NA>
__global__ __launch_bounds__(256) void k_pred_up_mfma(const u32x4 *__restrict__ U,
                                                      const uint16_t *__restrict__ ahid,
                                                      const float *__restrict__ hinv, int B,
                                                      int r, int f, float *__restrict__ s)
{
    __shared__ float red[4][MT * 4][kWave];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int ln = lane & 15, g = lane >> 4;
    const int C = r / 8;
    const int steps = C / 4;
    const int s0 = w * steps / 4, s1 = (w + 1) * steps / 4;
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
    const u32x4 *ar[NA][MT];
    bool aok[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int tok = 16 * m + ln;
        aok[m] = tok < B;
#pragma unroll
        for (int e = 0; e < NA; ++e)
            ar[e][m] = reinterpret_cast<const u32x4 *>(ahid + ((size_t)e * B + (aok[m] ? tok : 0)) * r);
    }
    // the token scales of the epilogue elements this thread writes (the same in every tile;
    // MT * 4 * kWave = 256 MT elements, element t + 256 q for thread t)
    float tinv[MT];
#pragma unroll
    for (int q = 0; q < MT; ++q) {
        const int e = t + 256 * q, mi = e / kWave, l = e % kWave;
        const int tok = 16 * (mi / 4) + 4 * (l >> 4) + (mi % 4);
        tinv[q] = tok < B ? hinv[tok] : 1.0f;
    }
    for (int n0 = blockIdx.x * 16; n0 < f; n0 += gridDim.x * 16) {
        const int n = n0 + ln;
        const u32x4 *wr = U + (size_t)(n < f ? n : f - 1) * C;   // a row past f is discarded
        f32x4 acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (s1 > s0) {
            u32x4 rw[kRing], rx[kRing][NA][MT];
            auto fill = [&](int p, int st) {
                const int c = 4 * (st < s1 ? st : s1 - 1) + g;
                rw[p] = ld_stream(wr + c);
#pragma unroll
                for (int e = 0; e < NA; ++e)
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        rx[p][e][m] = ar[e][m][c];
            };
#pragma unroll
            for (int p = 0; p < kRing; ++p)
                fill(p, s0 + p);
            const int groups = (s1 - s0 + kRing - 1) / kRing;
            for (int gi = 0; gi < groups; ++gi) {
#pragma unroll
                for (int p = 0; p < kRing; ++p) {
                    const bool ok = s0 + gi * kRing + p < s1;
#pragma unroll
                    for (int e = 0; e < NA; ++e)
#pragma unroll
                        for (int m = 0; m < MT; ++m)
                            acc[m] = T::mfma((ok && aok[m]) ? rx[p][e][m] : zero, rw[p], acc[m]);
                    fill(p, s0 + (gi + 1) * kRing + p);
                }
            }
        }
        sum_waves<MT>(red, acc, w, lane);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < MT; ++q) {
            const int e = t + 256 * q, mi = e / kWave, l = e % kWave;
            const int tok = 16 * (mi / 4) + 4 * (l >> 4) + (mi % 4);
            const int nn = n0 + (l & 15);
            if (tok < B && nn < f) {
                const float z = ((red[0][mi][l] + red[1][mi][l]) + (red[2][mi][l] + red[3][mi][l])) *
                                tinv[q];
                s[(size_t)tok * f + nn] = 1.0f / (1.0f + expf(-z));
            }
        }
        __syncthreads();
    }
}

// The same product when each wave's share of r is at most KW K steps (r <= 512 for KW = 4): the
// wave's 16-bit hidden terms are loaded once into registers and serve every tile the workgroup
// takes (tiles b, b + grid, ...), so only U streams; the next tile's U chunks are loaded before the
// current tile is multiplied.  k_pred_up_mfma instead re-reads the terms from L2 for every tile,
// which at 32 tokens is about four times U's own bytes.  Same products and sums in the same order,
// so the same scores.
template <class T, int MT, int NA, int KW>
__global__ __launch_bounds__(256) void k_pred_up_mfma_res(const u32x4 *__restrict__ U,
                                                          const uint16_t *__restrict__ ahid,
                                                          const float *__restrict__ hinv, int B,
                                                          int r, int f, float *__restrict__ s)
{
    __shared__ float red[4][MT * 4][kWave];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int ln = lane & 15, g = lane >> 4;
    const int C = r / 8;
    const int steps = C / 4;
    const int s0 = w * steps / 4, s1 = (w + 1) * steps / 4;
    const int ns = s1 - s0;                      // <= KW (checked by the launcher)
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
    u32x4 ra[KW][NA][MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int tok = 16 * m + ln;
        const bool ok = tok < B;
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            const u32x4 *ar = reinterpret_cast<const u32x4 *>(ahid + ((size_t)e * B + (ok ? tok : 0)) * r);
#pragma unroll
            for (int q = 0; q < KW; ++q)
                ra[q][e][m] = (ok && q < ns) ? ar[4 * (s0 + q) + g] : zero;
        }
    }
    auto load_tile = [&](int n0, u32x4 (&dst)[KW]) {
        const int n = n0 + ln;
        const u32x4 *wr = U + (size_t)(n < f ? n : f - 1) * C;   // a row past f is discarded
#pragma unroll
        for (int q = 0; q < KW; ++q)
            dst[q] = (n0 < f && q < ns) ? ld_stream(wr + 4 * (s0 + q) + g) : zero;
    };
    // the token scales of the epilogue elements this thread writes (the same in every tile;
    // MT * 4 * kWave = 256 MT elements, element t + 256 q for thread t)
    float tinv[MT];
#pragma unroll
    for (int q = 0; q < MT; ++q) {
        const int e = t + 256 * q, mi = e / kWave, l = e % kWave;
        const int tok = 16 * (mi / 4) + 4 * (l >> 4) + (mi % 4);
        tinv[q] = tok < B ? hinv[tok] : 1.0f;
    }
    u32x4 rw[KW];
    load_tile(blockIdx.x * 16, rw);
    for (int n0 = blockIdx.x * 16; n0 < f; n0 += gridDim.x * 16) {
        u32x4 rn[KW];
        load_tile(n0 + gridDim.x * 16, rn);
        f32x4 acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < KW; ++q) {
            if (q < ns) {
#pragma unroll
                for (int e = 0; e < NA; ++e)
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        acc[m] = T::mfma(ra[q][e][m], rw[q], acc[m]);
            }
        }
        sum_waves<MT>(red, acc, w, lane);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < MT; ++q) {
            const int e = t + 256 * q, mi = e / kWave, l = e % kWave;
            const int tok = 16 * (mi / 4) + 4 * (l >> 4) + (mi % 4);
            const int nn = n0 + (l & 15);
            if (tok < B && nn < f) {
                const float z = ((red[0][mi][l] + red[1][mi][l]) + (red[2][mi][l] + red[3][mi][l])) *
                                tinv[q];
                s[(size_t)tok * f + nn] = 1.0f / (1.0f + expf(-z));
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < KW; ++q)
            rw[q] = rn[q];
    }
}

template <class T, int MT, int NA>
hipError_t predict_group(const u32x4 *x, int B, int d, const u32x4 *V, int r, const u32x4 *U,
                         int f, float *s, float *part, uint16_t *ahid, float *hinv, hipStream_t st,
                         Trace *tr, int res_grid)
{
    const int C = d / 8;
    const int ks_n = pred_mfma_split(r, d);
    hipError_t e = launch(k_pred_down_mfma<T, MT>, dim3(r / 16, ks_n), dim3(256), st, tr, V, x, B,
                          C, r, ks_n, part);
    if (e != hipSuccess)
        return e;
    e = launch(k_pred_hidden<T, NA>, dim3(B), dim3(kHiddenThreads), st, tr, part, ks_n, B, r, ahid,
               hinv);
    if (e != hipSuccess)
        return e;
    const int tiles = (f + 15) / 16;
    if ((r / 32 + 3) / 4 <= 4) {
        // two workgroups per CU (512 on MI355X, 3.5 tiles each at the OPT-30B shape): 8.9 / 9.3 /
        // 12.9 us at 8 / 16 / 32 tokens, against 9.7 / 12.4 / 20.9 for k_pred_up_mfma; one or four
        // per CU and one workgroup per tile measured slower
        return launch(k_pred_up_mfma_res<T, MT, NA, 4>, dim3(tiles < res_grid ? tiles : res_grid),
                      dim3(256), st, tr, U, ahid, hinv, B, r, f, s);
    }
    return launch(k_pred_up_mfma<T, MT, NA>, dim3(tiles < 4096 ? tiles : 4096), dim3(256), st, tr,
                  U, ahid, hinv, B, r, f, s);
}

template <class T, int NA>
hipError_t predict_t(const void *x, int B, int d, const void *V, int r, const void *U, int f,
                     float *s, float *part, uint16_t *ahid, float *hinv, hipStream_t st, Trace *tr,
                     int res_grid)
{
    for (int b0 = 0; b0 < B; b0 += kMaxPredMfmaTokens) {
        const int nb = B - b0 < kMaxPredMfmaTokens ? B - b0 : kMaxPredMfmaTokens;
        const u32x4 *xb = static_cast<const u32x4 *>(x) + (size_t)b0 * (d / 8);
        float *sb = s + (size_t)b0 * f;
        hipError_t e = nb <= 16
            ? predict_group<T, 1, NA>(xb, nb, d, static_cast<const u32x4 *>(V), r,
                                      static_cast<const u32x4 *>(U), f, sb, part, ahid, hinv, st, tr,
                                      res_grid)
            : predict_group<T, 2, NA>(xb, nb, d, static_cast<const u32x4 *>(V), r,
                                      static_cast<const u32x4 *>(U), f, sb, part, ahid, hinv, st, tr,
                                      res_grid);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace

int pred_mfma_split(int r, int d)
{
    // about 512 workgroups over the rows of V, each wave at least 2 K steps
    const int tiles = r / 16;
    const int steps = d / 32;
    int ks = (512 + tiles - 1) / tiles;
    while (ks > 1 && steps / ks < 8)
        --ks;
    if (ks > kMaxPredMfmaSplit)
        ks = kMaxPredMfmaSplit;
    return ks < 1 ? 1 : ks;
}

bool pred_mfma_supported(int dtype, int B, int d, int r)
{
    return dtype != 0 && B >= kPredMfmaMinBatch && d % 128 == 0 && r % 128 == 0;
}

size_t pred_mfma_ws_floats(int B, int r)
{
    const int nb = B < kMaxPredMfmaTokens ? B : kMaxPredMfmaTokens;
    // partial sums [split][nb][r] float32, then NA <= 3 16-bit terms [3][nb][r] (as floats: / 2),
    // then the per-token scales [nb] float32 (plus alignment)
    return (size_t)kMaxPredMfmaSplit * nb * r + ((size_t)3 * nb * r + 1) / 2 + kMaxPredMfmaTokens + 64;
}

hipError_t launch_predict_mfma(int dtype, const void *x, int B, int d, const void *V, int r,
                               const void *U, int f, float *s, float *ws, hipStream_t st,
                               Trace *tr, int res_grid)
{
    if (res_grid < 1)
        return hipErrorInvalidValue;
    const int nb = B < kMaxPredMfmaTokens ? B : kMaxPredMfmaTokens;
    float *part = ws;
    // 16-byte aligned start for the 16-bit terms
    size_t off = ((size_t)kMaxPredMfmaSplit * nb * r + 3) / 4 * 4;
    uint16_t *ahid = reinterpret_cast<uint16_t *>(ws + off);
    float *hinv = ws + off + ((size_t)3 * nb * r + 1) / 2;
    if (dtype == 1)
        return predict_t<F16T, 2>(x, B, d, V, r, U, f, s, part, ahid, hinv, st, tr, res_grid);
    return predict_t<BF16T, 3>(x, B, d, V, r, U, f, s, part, ahid, hinv, st, tr, res_grid);
}

}  // namespace csf
