// predict.hip -- the low-rank activation predictor on gfx950.
//
// "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm", section "The
// Prediction Problem": a bias-free two-layer network per layer scores every FFN neuron,
// scores = sigmoid(up(relu(down(x)))), with down: d -> r and up: r -> f.
//
// Both halves are skinny GEMVs bound by HBM bandwidth (2 flops per weight element read), so they
// are written as streaming dot-product kernels, not as MFMA tiles:
//   k_pred_down  S 256-thread workgroups per R rows of V (split-K); each thread keeps its 16-byte
//                chunks in registers and reuses them for every token; partial sums out.
//   k_pred_up    (batches; k_pred_up_loop is its persistent form for one token)
//                groups of LPR lanes per row of U (LPR = 16/32/64 so short rows still use whole
//                128-byte lines); the weight loads are issued first, then the workgroup adds
//                the split-K partials, applies ReLU and stages the hidden activation a (float32)
//                in LDS once, and each lane takes its chunk positions from there (one read of a
//                from L2 per workgroup rather than per wavefront); sigmoid in the epilogue.
#include "common.hpp"
#include "launch.hpp"

namespace csf {

namespace {

// Split-K down projection: S workgroups per R rows of V, each over a contiguous 1/S of the rows'
// 16-byte chunks (more, shorter workgroups keep more of HBM busy than one workgroup per row); the
// x chunks a thread loads serve all R rows.  The partial sums go to part[S][B][r]; the
// up-projection kernel adds them in order and applies ReLU.
template <class T, int MX, int TG, int R>
__global__ __launch_bounds__(256) void k_pred_down(const u32x4 *__restrict__ V,
                                                   const u32x4 *__restrict__ x, int C, int r,
                                                   int B, int S, float *__restrict__ part,
                                                   uint32_t *__restrict__ zero, int nzero,
                                                   uint32_t *__restrict__ fill, int nfill)
{
    __shared__ float red[4][R * TG];
    // the workgroups also prepare blocks of a caller's workspace for a later kernel of the same
    // call: counters cleared, hand-over slots marked unwritten
    for (int i = blockIdx.x * 256 + threadIdx.x; i < nzero; i += gridDim.x * 256)
        zero[i] = 0u;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < nfill; i += gridDim.x * 256)
        fill[i] = kHSentinel;
    const int i0 = (blockIdx.x / S) * R, sp = blockIdx.x % S;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int cper = (C + S - 1) / S;
    const int c0 = sp * cper;
    const int c1 = c0 + cper < C ? c0 + cper : C;
    u32x4 wv[R][MX];
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const u32x4 *row = V + (size_t)(i0 + q) * C;
#pragma unroll
        for (int m = 0; m < MX; ++m) {
            const int c = c0 + t + 256 * m;
            wv[q][m] = (c < c1 && i0 + q < r) ? ld_stream(row + c) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    // tokens in groups of TG (TG = 1 for a single token: one accumulator per row, one reduction)
    for (int t0 = 0; t0 < B; t0 += TG) {
        float acc[R][TG];
#pragma unroll
        for (int p = 0; p < TG; ++p) {
            const int tok = t0 + p;
            u32x4 xv[MX];
#pragma unroll
            for (int m = 0; m < MX; ++m) {
                const int c = c0 + t + 256 * m;
                xv[m] = (tok < B && c < c1) ? x[(size_t)tok * C + c] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int q = 0; q < R; ++q) {
                acc[q][p] = 0.0f;
#pragma unroll
                for (int m = 0; m < MX; ++m) {
                    const int c = c0 + t + 256 * m;
                    if (tok < B && c < c1)
                        acc[q][p] = T::dot(wv[q][m], xv[m], acc[q][p]);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < R; ++q)
#pragma unroll
            for (int p = 0; p < TG; ++p)
                acc[q][p] = wave_sum(acc[q][p]);
        if (lane == 0) {
#pragma unroll
            for (int q = 0; q < R; ++q)
#pragma unroll
                for (int p = 0; p < TG; ++p)
                    red[w][q * TG + p] = acc[q][p];
        }
        __syncthreads();
        if (t < R * TG) {
            const int q = t / TG, p = t % TG;
            if (t0 + p < B && i0 + q < r)
                part[((size_t)sp * B + t0 + p) * r + i0 + q] =
                    (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
        }
        __syncthreads();
    }
}

template <class T, int LPR, int MM, int RW, int NT = 256>
__global__ __launch_bounds__(NT) void k_pred_up(const u32x4 *__restrict__ U,
                                                 const float *__restrict__ a, int C, int r, int f,
                                                 int B, int S, float *__restrict__ s)
{
    constexpr int G = kWave / LPR;   // rows handled side by side by one wavefront
    constexpr int E = T::E;
    __shared__ float4 sa[kWave * MM * E / 4];   // the token's hidden activation (C * E <= its size)
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int g = lane / LPR, li = lane % LPR;
    const int wave = blockIdx.x * (NT / kWave) + t / kWave;
    const int row0 = wave * (RW * G);
    u32x4 wv[RW][MM];
#pragma unroll
    for (int st = 0; st < RW; ++st) {
        const int j = row0 + st * G + g;
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const int c = li + LPR * m;
            wv[st][m] = (j < f && c < C) ? ld_stream(U + (size_t)j * C + c)
                                         : u32x4{0u, 0u, 0u, 0u};
        }
    }
    const int n4 = C * E / 4;
    for (int tok = 0; tok < B; ++tok) {
        // hidden activation a = relu(sum of the S split-K partial sums, in order), staged once per
        // workgroup in LDS
        if (tok > 0)
            __syncthreads();
        for (int i = t; i < n4; i += NT) {
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int sp = 0; sp < S; ++sp) {
                const float4 v = reinterpret_cast<const float4 *>(a + ((size_t)sp * B + tok) * r)[i];
                acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
            }
            acc.x = acc.x > 0.0f ? acc.x : 0.0f;
            acc.y = acc.y > 0.0f ? acc.y : 0.0f;
            acc.z = acc.z > 0.0f ? acc.z : 0.0f;
            acc.w = acc.w > 0.0f ? acc.w : 0.0f;
            sa[i] = acc;
        }
        __syncthreads();
        float av[MM][E];
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const int c = li + LPR * m;
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                const float4 v = c < C ? sa[(c * E + e) / 4] : make_float4(0.f, 0.f, 0.f, 0.f);
                av[m][e] = v.x; av[m][e + 1] = v.y; av[m][e + 2] = v.z; av[m][e + 3] = v.w;
            }
        }
#pragma unroll
        for (int st = 0; st < RW; ++st) {
            float acc = 0.0f;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                float wf[E];
                T::unpack(wv[st][m], wf);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    acc = fmaf(wf[e], av[m][e], acc);
            }
            acc = group_sum<LPR>(acc);
            const int j = row0 + st * G + g;
            if (li == 0 && j < f)
                s[(size_t)tok * f + j] = 1.0f / (1.0f + expf(-acc));
        }
    }
}

// One token, persistent form of k_pred_up: a grid of about as many workgroups as the GPU holds at
// once walks the row groups of U (workgroup b takes groups b, b + grid, ...).  The hidden
// activation is staged once per workgroup and each lane keeps its chunk positions of it in
// registers; the next group's weight loads are issued before the current group is reduced, so
// every lane always has a group of loads in flight.  Same lane mapping, sums and rounding as
// k_pred_up, so the scores are bit-identical.
template <class T, int LPR, int MM, int RW>
__global__ __launch_bounds__(256) void k_pred_up_loop(const u32x4 *__restrict__ U,
                                                      const float *__restrict__ a, int C, int r,
                                                      int f, int S, float *__restrict__ s)
{
    constexpr int G = kWave / LPR;
    constexpr int E = T::E;
    constexpr int NW = 4;
    constexpr int RPG = NW * RW * G;             // rows per workgroup step
    __shared__ float4 sa[kWave * MM * E / 4];
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1), w = t / kWave;
    const int g = lane / LPR, li = lane % LPR;
    const int ngroups = (f + RPG - 1) / RPG;
    int grp = blockIdx.x;
    u32x4 wv[RW][MM];
#pragma unroll
    for (int st = 0; st < RW; ++st) {
        const int j = (grp * NW + w) * (RW * G) + st * G + g;
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const int c = li + LPR * m;
            wv[st][m] = (j < f && c < C) ? ld_stream(U + (size_t)j * C + c)
                                         : u32x4{0u, 0u, 0u, 0u};
        }
    }
    const int n4 = C * E / 4;
    for (int i = t; i < n4; i += 256) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sp = 0; sp < S; ++sp) {
            const float4 v = reinterpret_cast<const float4 *>(a + (size_t)sp * r)[i];
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        acc.x = acc.x > 0.0f ? acc.x : 0.0f;
        acc.y = acc.y > 0.0f ? acc.y : 0.0f;
        acc.z = acc.z > 0.0f ? acc.z : 0.0f;
        acc.w = acc.w > 0.0f ? acc.w : 0.0f;
        sa[i] = acc;
    }
    __syncthreads();
    float av[MM][E];
#pragma unroll
    for (int m = 0; m < MM; ++m) {
        const int c = li + LPR * m;
#pragma unroll
        for (int e = 0; e < E; e += 4) {
            const float4 v = c < C ? sa[(c * E + e) / 4] : make_float4(0.f, 0.f, 0.f, 0.f);
            av[m][e] = v.x; av[m][e + 1] = v.y; av[m][e + 2] = v.z; av[m][e + 3] = v.w;
        }
    }
    while (grp < ngroups) {
        const int nxt = grp + (int)gridDim.x;
        u32x4 wn[RW][MM];
#pragma unroll
        for (int st = 0; st < RW; ++st) {
            const int j = (nxt * NW + w) * (RW * G) + st * G + g;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                const int c = li + LPR * m;
                wn[st][m] = (nxt < ngroups && j < f && c < C) ? ld_stream(U + (size_t)j * C + c)
                                                              : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int st = 0; st < RW; ++st) {
            float acc = 0.0f;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                float wf[E];
                T::unpack(wv[st][m], wf);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    acc = fmaf(wf[e], av[m][e], acc);
            }
            acc = group_sum<LPR>(acc);
            const int j = (grp * NW + w) * (RW * G) + st * G + g;
            if (li == 0 && j < f)
                s[j] = 1.0f / (1.0f + expf(-acc));
        }
#pragma unroll
        for (int st = 0; st < RW; ++st)
#pragma unroll
            for (int m = 0; m < MM; ++m)
                wv[st][m] = wn[st][m];
        grp = nxt;
    }
}

// Scores and selection of one token with few scores (f <= kSmallF), in one 1024-thread
// workgroup: the up projection as in k_pred_up (LPR lanes per row of U, rows in passes of 16
// waves), each score kept in LDS as well as written out; then the selection on the LDS copy --
// top-k: a score's rank is the number of (score, index) pairs ordered before it (the order of the
// one-workgroup bucket select, so the lists are the same), threshold: s >= tau -- and a block
// scan of the selected flags writes the ascending list.  Saves the launch of a separate selection
// kernel, which dominates when f is a few hundred (attention heads).
template <class T, int LPR, int MM>
__global__ __launch_bounds__(1024) void k_pred_up_select(const u32x4 *__restrict__ U,
                                                         const float *__restrict__ a, int C, int r,
                                                         int f, int S, float *__restrict__ s,
                                                         int k, float tau,
                                                         int32_t *__restrict__ idx,
                                                         int32_t *__restrict__ count)
{
    constexpr int G = kWave / LPR;
    constexpr int E = T::E;
    __shared__ float ss[kSmallF];
    __shared__ uint64_t key[kSmallF];
    __shared__ uint32_t scan_tmp[16];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int g = lane / LPR, li = lane % LPR;
    // hidden activation a = relu(sum of the S split-K partial sums, in order)
    float av[MM][E];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int e = 0; e < E; ++e)
            av[m][e] = 0.0f;
    for (int sp = 0; sp < S; ++sp) {
        const float *at = a + (size_t)sp * r;
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const int c = li + LPR * m;
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                float4 v = c < C ? *reinterpret_cast<const float4 *>(at + c * E + e)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
                av[m][e] += v.x; av[m][e + 1] += v.y; av[m][e + 2] += v.z; av[m][e + 3] += v.w;
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int e = 0; e < E; ++e)
            av[m][e] = av[m][e] > 0.0f ? av[m][e] : 0.0f;
    // rows in groups of four passes of the 16 waves, every load of a group issued first
    constexpr int NP = 4;
    for (int row0 = 0; row0 < f; row0 += NP * 16 * G) {
        u32x4 wv[NP][MM];
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int j = row0 + q * 16 * G + w * G + g;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                const int c = li + LPR * m;
                wv[q][m] = (j < f && c < C) ? ld_stream(U + (size_t)j * C + c)
                                            : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int j = row0 + q * 16 * G + w * G + g;
            float acc = 0.0f;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                float wf[E];
                T::unpack(wv[q][m], wf);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    acc = fmaf(wf[e], av[m][e], acc);
            }
            acc = group_sum<LPR>(acc);
            if (li == 0 && j < f) {
                const float sc = 1.0f / (1.0f + expf(-acc));
                s[j] = sc;
                ss[j] = sc;
            }
        }
    }
    __syncthreads();
    bool sel = false;
    if (k >= 0) {
        if (t < f)
            key[t] = composite(order_key(ss[t]), t);
        __syncthreads();
        if (t < f) {
            const uint64_t me = key[t];
            int rank = 0;
            for (int i = 0; i < f; ++i)
                rank += key[i] > me ? 1 : 0;
            sel = rank < k;
        }
    } else {
        sel = t < f && ss[t] >= tau;
    }
    uint32_t total;
    const uint32_t pos = block_exclusive_scan<16>(sel ? 1u : 0u, scan_tmp, &total);
    if (sel)
        idx[pos] = t;
    if (t == 0 && count)
        *count = k >= 0 ? k : (int32_t)total;
}

struct DownArgs {
    const void *x;
    int B, C;
    const void *V;
    int r, S;
    float *a;
    uint32_t *zero;
    int nzero;
    uint32_t *fill;
    int nfill;
};

template <class T, int MX, int R>
hipError_t down_r(const DownArgs &g, hipStream_t st, Trace *tr)
{
    const u32x4 *V = static_cast<const u32x4 *>(g.V), *x = static_cast<const u32x4 *>(g.x);
    const dim3 grid((g.r + R - 1) / R * g.S);
    if (g.B == 1)
        return launch(k_pred_down<T, MX, 1, R>, grid, dim3(256), st, tr, V, x, g.C, g.r, g.B, g.S,
                      g.a, g.zero, g.nzero, g.fill, g.nfill);
    return launch(k_pred_down<T, MX, 8, R>, grid, dim3(256), st, tr, V, x, g.C, g.r, g.B, g.S,
                  g.a, g.zero, g.nzero, g.fill, g.nfill);
}

// Two rows per workgroup halve the re-reads of x when that still leaves >= 512 workgroups.
template <class T, int MX>
hipError_t down_mx(const DownArgs &g, hipStream_t st, Trace *tr)
{
    if (MX <= 8 && (long)g.r * g.S >= 1024)
        return down_r<T, MX, 2>(g, st, tr);
    return down_r<T, MX, 1>(g, st, tr);
}

template <class T>
hipError_t down_t(const DownArgs &g, hipStream_t st, Trace *tr)
{
    const int mx = ((g.C + g.S - 1) / g.S + 255) / 256;
    if (mx <= 1) return down_mx<T, 1>(g, st, tr);
    if (mx <= 2) return down_mx<T, 2>(g, st, tr);
    if (mx <= 4) return down_mx<T, 4>(g, st, tr);
    if (mx <= 6) return down_mx<T, 6>(g, st, tr);
    if (mx <= 8) return down_mx<T, 8>(g, st, tr);
    if (mx <= 12) return down_mx<T, 12>(g, st, tr);
    if (mx <= 16) return down_mx<T, 16>(g, st, tr);
    return hipErrorInvalidValue;
}

template <class T, int LPR, int MM, int RW>
hipError_t up_loop_launch(const float *a, int S, int r, int C, const void *U, int f, float *s,
                          hipStream_t st, Trace *tr, int grid)
{
    constexpr int RPG = 4 * RW * (kWave / LPR);
    const int ngroups = (f + RPG - 1) / RPG;
    const int blocks = grid < ngroups ? grid : ngroups;
    return launch(k_pred_up_loop<T, LPR, MM, RW>, dim3(blocks), dim3(256), st, tr,
                  static_cast<const u32x4 *>(U), a, C, r, f, S, s);
}

template <class T, int LPR, int MM, int RW>
hipError_t up_launch(const float *a, int B, int S, int r, int C, const void *U, int f, float *s,
                     hipStream_t st, Trace *tr, int grid)
{
    constexpr int rows_per_wave = RW * (kWave / LPR);
    constexpr int NT = 256;   // measured: 512-thread workgroups are slower (19.5 against 18.2 us)
    // one token: the persistent form on the caller's grid (measured at the OPT-175B / OPT-30B /
    // LLaMA-class predictor shapes with 8 workgroups per CU: 17.4 / 8.1 / 4.2 us against 18.1 / 9.5
    // / 4.35 us for one short workgroup per 8 rows; 4 or 2 per CU, or 2 and 4 rows per lane
    // group, are slower)
    if (B == 1)
        return grid > 0 ? up_loop_launch<T, LPR, MM, 1>(a, S, r, C, U, f, s, st, tr, grid)
                        : hipErrorInvalidValue;
    const int waves = (f + rows_per_wave - 1) / rows_per_wave;
    const int blocks = (waves + NT / kWave - 1) / (NT / kWave);
    return launch(k_pred_up<T, LPR, MM, RW, NT>, dim3(blocks), dim3(NT), st, tr,
                  static_cast<const u32x4 *>(U), a, C, r, f, B, S, s);
}

// Rows per lane group: up to 4, so that each wavefront's read of the hidden activation (S partial
// vectors, from L2) is amortized over several rows; fewer when the matrix is too short to give
// every CU several workgroups.
template <class T, int LPR, int MM>
hipError_t up_rw(const float *a, int B, int S, int r, int C, const void *U, int f, float *s,
                 hipStream_t st, Trace *tr, int grid)
{
    constexpr int G = kWave / LPR;
    int rw = MM >= 2 ? 2 : 4;   // rows of two 16-byte chunks per lane: 2 rows (measured fastest)
    while (rw > 1 && (long)f / (rw * G) < 4096)   // keep >= 1024 workgroups when f allows
        rw /= 2;
    if (rw >= 4) return up_launch<T, LPR, MM, 4>(a, B, S, r, C, U, f, s, st, tr, grid);
    if (rw >= 2) return up_launch<T, LPR, MM, 2>(a, B, S, r, C, U, f, s, st, tr, grid);
    return up_launch<T, LPR, MM, 1>(a, B, S, r, C, U, f, s, st, tr, grid);
}

template <class T>
hipError_t up_t(const float *a, int B, int S, int r, int C, const void *U, int f, float *s,
                hipStream_t st, Trace *tr, int grid)
{
    if (C <= 16) return up_rw<T, 16, 1>(a, B, S, r, C, U, f, s, st, tr, grid);
    if (C <= 32) return up_rw<T, 32, 1>(a, B, S, r, C, U, f, s, st, tr, grid);
    if (C <= 64) return up_rw<T, 64, 1>(a, B, S, r, C, U, f, s, st, tr, grid);
    if (C <= 128) return up_rw<T, 64, 2>(a, B, S, r, C, U, f, s, st, tr, grid);
    if (C <= 256) return up_rw<T, 64, 4>(a, B, S, r, C, U, f, s, st, tr, grid);
    if (C <= 512) return up_rw<T, 64, 8>(a, B, S, r, C, U, f, s, st, tr, grid);
    return hipErrorInvalidValue;
}

template <class T>
hipError_t up_select_t(const float *a, int S, int r, int C, const void *U, int f, float *s, int k,
                       float tau, int32_t *idx, int32_t *count, hipStream_t st, Trace *tr)
{
    const u32x4 *u = static_cast<const u32x4 *>(U);
    if (C <= 16)
        return launch(k_pred_up_select<T, 16, 1>, dim3(1), dim3(1024), st, tr, u, a, C, r, f, S, s,
                      k, tau, idx, count);
    if (C <= 32)
        return launch(k_pred_up_select<T, 32, 1>, dim3(1), dim3(1024), st, tr, u, a, C, r, f, S, s,
                      k, tau, idx, count);
    if (C <= 64)
        return launch(k_pred_up_select<T, 64, 1>, dim3(1), dim3(1024), st, tr, u, a, C, r, f, S, s,
                      k, tau, idx, count);
    if (C <= 128)
        return launch(k_pred_up_select<T, 64, 2>, dim3(1), dim3(1024), st, tr, u, a, C, r, f, S, s,
                      k, tau, idx, count);
    if (C <= 256)
        return launch(k_pred_up_select<T, 64, 4>, dim3(1), dim3(1024), st, tr, u, a, C, r, f, S, s,
                      k, tau, idx, count);
    if (C <= 512)
        return launch(k_pred_up_select<T, 64, 8>, dim3(1), dim3(1024), st, tr, u, a, C, r, f, S, s,
                      k, tau, idx, count);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_pred_up_select(int dtype, const float *a, int d, int r, const void *U, int f,
                                 float *s, int k, float tau, int32_t *idx, int32_t *count,
                                 hipStream_t st, Trace *tr)
{
    if (f < 1 || f > kSmallF)
        return hipErrorInvalidValue;
    const int S = pred_split(r, d, dtype);
    if (dtype == 0) return up_select_t<F32T>(a, S, r, r / 4, U, f, s, k, tau, idx, count, st, tr);
    if (dtype == 1) return up_select_t<F16T>(a, S, r, r / 8, U, f, s, k, tau, idx, count, st, tr);
    return up_select_t<BF16T>(a, S, r, r / 8, U, f, s, k, tau, idx, count, st, tr);
}

int pred_split(int r, int d, int dtype)
{
    // Split only short predictors (r < 1024): every wavefront of the up projection re-reads all S
    // partial vectors, which costs more than the split gains once r is large.  Each workgroup
    // keeps at least 256 16-byte chunks of its row.
    const int C = d / (dtype == 0 ? 4 : 8);
    int S = 1024 / r;
    if (S > kMaxPredSplit)
        S = kMaxPredSplit;
    while (S > 1 && C / S < 256)
        --S;
    return S < 1 ? 1 : S;
}

hipError_t launch_pred_down(int dtype, const void *x, int B, int d, const void *V, int r,
                            float *a, hipStream_t st, Trace *tr, uint32_t *zero, int nzero,
                            uint32_t *fill, int nfill)
{
    DownArgs g{x, B, d / (dtype == 0 ? 4 : 8), V, r, pred_split(r, d, dtype), a,
               zero, zero ? nzero : 0, fill, fill ? nfill : 0};
    if (dtype == 0) return down_t<F32T>(g, st, tr);
    if (dtype == 1) return down_t<F16T>(g, st, tr);
    return down_t<BF16T>(g, st, tr);
}

hipError_t launch_pred_up(int dtype, const float *a, int B, int d, int r, const void *U, int f,
                          float *s, hipStream_t st, Trace *tr, int grid)
{
    const int S = pred_split(r, d, dtype);
    if (dtype == 0) return up_t<F32T>(a, B, S, r, r / 4, U, f, s, st, tr, grid);
    if (dtype == 1) return up_t<F16T>(a, B, S, r, r / 8, U, f, s, st, tr, grid);
    return up_t<BF16T>(a, B, S, r, r / 8, U, f, s, st, tr, grid);
}

}  // namespace csf
