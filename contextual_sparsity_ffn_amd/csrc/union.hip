// union.hip -- the batched sparse FFN over the union of the tokens' active sets, on gfx950.
//
// [CP] "Contextual Sparsity and Activation Predictors", section "When it breaks": the tokens of a
// batch have different active sets, so a batched layer has to read the union of them.
// [DV] "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm", section
// "Kernel-Level Implementation": each token keeps its own index list; section "Implications for
// System Design": sparse batching has a crossover batch size.
//
// Semantics.  Every row of the union is read from HBM once per call and applied to all B tokens.
// Per token (the default), token t keeps only its own neurons: h[t][n] is forced to 0 for a union
// row that t did not select, so y_t is the sparse FFN of x_t over its own set.  Union semantics
// apply every union row to every token.
//
// Kernels (all loops over the union are grid-stride loops that read the union size from device
// memory, so nothing is sized from data the host does not have):
//   k_union_list     one workgroup: OR of the B bitmaps, ascending union list and its size;
//   gather path (vector ALU, for few tokens):
//     k_union_up_valu    rows of the union in registers, one dot product per token; h in float32;
//     k_union_down_valu  d-slices x union chunks x token groups, B accumulators per column;
//   matrix-core path (MFMA 16x16x32, tokens padded to 16 or 32 as M):
//     k_union_up_lds     32 union rows x all tokens per workgroup: row and token segments staged
//                        through LDS (whole 128-byte lines per load), M = tokens, N = rows;
//                        h stored in float32, and each token's largest |h| past the 16-bit
//                        split limit recorded (an atomic max, taken only on that rare path);
//     k_union_down_mfma  tile of 256 output columns x a chunk of the union: the rows of W2T are
//                        staged through LDS and read back column-wise, because W2T is contiguous
//                        along the output columns while the product contracts over rows; h
//                        enters the matrix cores as a hi/lo pair of 16-bit values of h 2^k
//                        (hi = round(h 2^k), lo = round(h 2^k - hi); k = 0 unless the token's
//                        |h| reaches the split limit), which keeps about 22 bits of h for
//                        binary16 and 16 for bfloat16, and the token's outputs are scaled by
//                        2^-k;
//   both paths end in the ordered partial-row reduction of the single-token FFN.
#include "common.hpp"
#include "launch.hpp"

namespace csf {

namespace {

constexpr int kUnionThreads = 1024;
constexpr int kKStep = 32;           // K of one MFMA: 32 elements = 4 16-byte chunks
constexpr int kDownCols = 256;       // output columns per MFMA down workgroup (512 bytes of a row)
constexpr int kDownLdsStride = 260;  // 16-bit elements per staged row: 520 bytes (8-byte aligned,
                                     // rows 8 apart fall 16 banks apart)
constexpr int kValuTokens = 8;       // tokens per vector-ALU down-projection workgroup
constexpr int kMaxDownSteps = 64;    // K steps (of 32 union rows) per matrix-core down chunk

// Union rows per gather-path workgroup: about 12 chunk loads in flight per thread, at most 4 rows.
template <int MX, bool GATED>
struct UpRows {
    static constexpr int loads = MX * (GATED ? 2 : 1);
    static constexpr int value = loads >= 12 ? 1 : (loads >= 6 ? 2 : 4);
};

__device__ __forceinline__ int union_size(const int32_t *ucount, int f)
{
    const int u = *ucount;
    return u < 0 ? 0 : (u > f ? f : u);
}

__device__ __forceinline__ bool token_has(const uint32_t *bitmaps, int words, int t, int j)
{
    return (bitmaps[(size_t)t * words + (j >> 5)] >> (j & 31)) & 1u;
}

// ---- union list --------------------------------------------------------------------------------
__global__ __launch_bounds__(kUnionThreads) void k_union_list(const uint32_t *__restrict__ bitmaps,
                                                              int B, int f,
                                                              int32_t *__restrict__ ulist,
                                                              int32_t *__restrict__ ucount,
                                                              int32_t *__restrict__ ucount_out,
                                                              uint32_t *__restrict__ hmax)
{
    __shared__ uint32_t scan_tmp[kUnionThreads / kWave];
    __shared__ uint32_t ow[2 * kUnionThreads], opos[2 * kUnionThreads];   // OR words, prefixes
    const int t = threadIdx.x;
    const int words = (f + 31) / 32;
    const int wpt = (words + kUnionThreads - 1) / kUnionThreads;   // 1 or 2 (f <= 65536)
    uint32_t orw[2] = {0u, 0u};
    uint32_t n = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int w = t * wpt + q;
        if (q < wpt && w < words) {
            // every token's word is loaded before the first OR (one round of load latency)
            uint32_t v[kMaxUnionBatch];
#pragma unroll
            for (int b = 0; b < kMaxUnionBatch; ++b)
                v[b] = bitmaps[(size_t)(b < B ? b : 0) * words + w];
            uint32_t o = 0u;
#pragma unroll
            for (int b = 0; b < kMaxUnionBatch; ++b)
                o |= b < B ? v[b] : 0u;
            if (w == words - 1 && (f & 31))
                o &= (1u << (f & 31)) - 1u;          // bits past f are not neurons
            orw[q] = o;
            n += __popc(o);
        }
    }
    uint32_t total;
    uint32_t pos = block_exclusive_scan<kUnionThreads / kWave>(n, scan_tmp, &total);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int w = t * wpt + q;
        if (q < wpt && w < words) {
            ow[w] = orw[q];
            opos[w] = pos;
            pos += __popc(orw[q]);
        }
    }
    __syncthreads();
    emit_bit_list<kUnionThreads>(ow, opos, words, total, ulist, f);
    if (hmax && t < kMaxUnionBatch)
        hmax[t] = 0u;                                  // per-token |h| maxima of this call
    if (t == 0) {
        *ucount = (int32_t)total;
        if (ucount_out)
            *ucount_out = (int32_t)total;
    }
}

// ---- gather path -------------------------------------------------------------------------------
// Workgroup of 256 threads per RPW union rows (grid-stride): the rows' chunks stay in registers
// and each token's x is streamed past them (x is small and cache-resident).  Wave partial sums go
// to LDS; after one barrier threads (token, row) finish h in a fixed order.
template <class T, int MX, bool GATED, int RPW>
__global__ __launch_bounds__(256) void k_union_up_valu(const u32x4 *__restrict__ X,
                                                       const u32x4 *__restrict__ W1,
                                                       const u32x4 *__restrict__ Wup,
                                                       const float *__restrict__ b1,
                                                       const int32_t *__restrict__ ulist,
                                                       const int32_t *__restrict__ ucount,
                                                       const uint32_t *__restrict__ bitmaps,
                                                       int per_token, int B, int f, int C,
                                                       float *__restrict__ h, int hs, int silu)
{
    constexpr int NV = GATED ? 2 : 1;
    __shared__ float red[4][kMaxUnionBatch][RPW][NV];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int u = union_size(ucount, f);
    const int words = (f + 31) / 32;

    for (int n0 = blockIdx.x * RPW; n0 < u; n0 += gridDim.x * RPW) {
        int jr[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i)
            jr[i] = n0 + i < u ? ulist[n0 + i] : -1;
        u32x4 wv[RPW][MX];
        u32x4 uv[GATED ? RPW : 1][GATED ? MX : 1];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const size_t rb = (size_t)(jr[i] < 0 ? 0 : jr[i]) * C;
#pragma unroll
            for (int m = 0; m < MX; ++m) {
                const int c = t + 256 * m;
                const bool ok = jr[i] >= 0 && c < C;
                wv[i][m] = ok ? ld_stream(W1 + rb + c) : u32x4{0u, 0u, 0u, 0u};
                if constexpr (GATED)
                    uv[i][m] = ok ? ld_stream(Wup + rb + c) : u32x4{0u, 0u, 0u, 0u};
            }
        }
        for (int tok = 0; tok < B; ++tok) {
            u32x4 xv[MX];
#pragma unroll
            for (int m = 0; m < MX; ++m) {
                const int c = t + 256 * m;
                xv[m] = c < C ? X[(size_t)tok * C + c] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                float acc = 0.0f;
#pragma unroll
                for (int m = 0; m < MX; ++m)
                    acc = T::dot(wv[i][m], xv[m], acc);
                acc = wave_sum(acc);
                if (lane == 0)
                    red[w][tok][i][0] = acc;
                if constexpr (GATED) {
                    float au = 0.0f;
#pragma unroll
                    for (int m = 0; m < MX; ++m)
                        au = T::dot(uv[i][m], xv[m], au);
                    au = wave_sum(au);
                    if (lane == 0)
                        red[w][tok][i][NV - 1] = au;
                }
            }
        }
        __syncthreads();
        for (int e = t; e < B * RPW; e += 256) {
            const int tok = e / RPW, i = e % RPW;
            const int j = jr[i];
            if (j < 0)
                continue;
            float p = (red[0][tok][i][0] + red[1][tok][i][0]) + (red[2][tok][i][0] + red[3][tok][i][0]);
            if (b1)
                p += b1[j];
            float hv = gate_act(p, silu);
            if constexpr (GATED)
                hv *= (red[0][tok][i][NV - 1] + red[1][tok][i][NV - 1]) +
                      (red[2][tok][i][NV - 1] + red[3][tok][i][NV - 1]);
            if (per_token && !token_has(bitmaps, words, tok, j))
                hv = 0.0f;
            h[(size_t)tok * hs + n0 + i] = hv;
        }
        __syncthreads();
    }
}

// Grid (d-slice of 64 chunks, union chunk, token group of TB).  Each lane owns one 16-byte column
// chunk of the slice and keeps TB x E float32 accumulators; the rows' h values are per token.
template <class T, int TB, int UNR>
__global__ __launch_bounds__(256) void k_union_down_valu(const u32x4 *__restrict__ W2T,
                                                         const float *__restrict__ h, int hs,
                                                         const int32_t *__restrict__ ulist,
                                                         const int32_t *__restrict__ ucount,
                                                         int B, int f, int C, int nchunk,
                                                         float *__restrict__ part)
{
    constexpr int E = T::E;
    __shared__ float red[3][TB][kWave * E];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int slice = blockIdx.x, chunk = blockIdx.y, tg = blockIdx.z * TB;
    const int D = C * E;
    const int c = slice * kWave + lane;
    const int u = union_size(ucount, f);
    const int per = (u + nchunk - 1) / nchunk;
    const int nb = chunk * per;
    const int ne = nb + per < u ? nb + per : u;

    float acc[TB][E];
#pragma unroll
    for (int q = 0; q < TB; ++q)
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[q][e] = 0.0f;

    for (int n = nb + w; n < ne; n += 4 * UNR) {
        u32x4 wv[UNR];
        float hv[UNR][TB];
#pragma unroll
        for (int r = 0; r < UNR; ++r) {
            const int nn = n + 4 * r;
            const bool ok = nn < ne;
            const int j = ok ? ulist[nn] : 0;
            wv[r] = (ok && c < C) ? ld_stream(W2T + (size_t)j * C + c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int q = 0; q < TB; ++q)
                hv[r][q] = (ok && tg + q < B) ? h[(size_t)(tg + q) * hs + nn] : 0.0f;
        }
#pragma unroll
        for (int r = 0; r < UNR; ++r) {
            float wf[E];
            T::unpack(wv[r], wf);
#pragma unroll
            for (int q = 0; q < TB; ++q)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    acc[q][e] = fmaf(hv[r][q], wf[e], acc[q][e]);
        }
    }
    if (w > 0) {
#pragma unroll
        for (int q = 0; q < TB; ++q)
#pragma unroll
            for (int e = 0; e < E; ++e)
                red[w - 1][q][lane * E + e] = acc[q][e];
    }
    __syncthreads();
    if (w == 0 && c < C) {
#pragma unroll
        for (int q = 0; q < TB; ++q) {
            if (tg + q >= B)
                break;
            float *out = part + ((size_t)(tg + q) * nchunk + chunk) * (size_t)D + (size_t)c * E;
#pragma unroll
            for (int e = 0; e < E; ++e)
                out[e] = ((acc[q][e] + red[0][q][lane * E + e]) + red[1][q][lane * E + e]) +
                         red[2][q][lane * E + e];
        }
    }
}

// ---- matrix-core path --------------------------------------------------------------------------
// One 16x16x32 MFMA: lane l holds A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16],
// e < 8, and receives D[4 (l / 16) + i][l % 16], i < 4.  A = tokens x K, B = K x union rows.
//
// Up projection through LDS.  A workgroup takes ROWS union rows (one or two 16-row tiles) and all B
// tokens over the whole of d, in segments of ST elements: per segment the 256 threads stage the
// segment of every weight row (and, gated, of every up row) and of every token row in LDS -- each
// wavefront load reads whole row segments, whole 128-byte lines -- with the loads of the
// next PD - 1 segments in flight in a register ring.  The waves then take (gate or up, row tile,
// token tile) pairs: four or more pairs give each wave its own (no reduction); two pairs split
// each segment's K steps over two waves each, summed in a fixed order in the epilogue.
template <class T, int MT, int NV, int PD, int ST, int ROWS>
__global__ __launch_bounds__(256) void k_union_up_lds(const u32x4 *__restrict__ X,
                                                      const u32x4 *__restrict__ W1,
                                                      const u32x4 *__restrict__ Wup,
                                                      const float *__restrict__ b1,
                                                      const int32_t *__restrict__ ulist,
                                                      const int32_t *__restrict__ ucount,
                                                      const uint32_t *__restrict__ bitmaps,
                                                      int per_token, int B, int f, int C,
                                                      float *__restrict__ h32,
                                                      uint32_t *__restrict__ hmax, int hs,
                                                      int silu)
{
    constexpr int RT = ROWS / 16;                // 16-row tiles of union rows
    constexpr int WR = NV * ROWS;                // staged weight rows
    constexpr int SR = WR + 16 * MT;             // staged rows: weight rows, then token rows
    constexpr int SEGC = ST / 8;                 // 16-byte chunks of a row segment
    constexpr int RPP = 256 / SEGC;              // rows staged per pass of the workgroup
    constexpr int LPT = SR / RPP;                // staged chunks per thread
    constexpr int WPT = WR / RPP;                // ... of which weight rows
    constexpr int TPR = ROWS / RPP;              // chunks per thread per weight matrix
    constexpr int STRIDE = ST + 8;               // staged row stride (16-bit elements)
    constexpr int PAIRS = NV * RT * MT;          // (gate/up, row tile, token tile) products
    constexpr int KSPLIT = PAIRS >= 4 ? 1 : 4 / PAIRS;
    constexpr int PPW = PAIRS >= 4 ? PAIRS / 4 : 1;
    constexpr int SPW = ST / kKStep / KSPLIT;    // K steps per wave per segment
    static_assert(SR % RPP == 0 && ROWS % RPP == 0 && 256 % SEGC == 0 && SPW >= 1 && RT >= 1,
                  "staging covers whole rows");
    __shared__ __align__(16) uint16_t seg[2][SR][STRIDE];
    __shared__ float red[KSPLIT][PAIRS][4][kWave];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int ln = lane & 15, g = lane >> 4;
    const int u = union_size(ucount, f);
    const int upad = (u + kKStep - 1) / kKStep * kKStep;   // h is written (zeros) up to here
    const int words = (f + 31) / 32;
    const int nseg = C / SEGC;
    const int srow = t / SEGC, scol = t % SEGC;   // thread t stages rows srow + 8 i, chunk scol
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};

    // this wave's products: pair pi = (v, q, m) with v = pi / (RT MT), q = (pi / MT) % RT, m = pi % MT
    const int kp = PAIRS >= 4 ? 0 : w / PAIRS;
    int pv[PPW], pq[PPW], pm[PPW], pidx[PPW];
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
        const int pi = PAIRS >= 4 ? w + 4 * j : w % PAIRS;
        pidx[j] = pi;
        pv[j] = pi / (RT * MT);
        pq[j] = (pi / MT) % RT;
        pm[j] = pi % MT;
    }
    // token rows staged by this thread (chunks WPT .. LPT - 1); tokens past B stage zeros
    const u32x4 *src[LPT];
    bool tok_ok[LPT];
#pragma unroll
    for (int i = WPT; i < LPT; ++i) {
        const int tok = srow + RPP * (i - WPT);
        tok_ok[i] = tok < B;
        src[i] = X + (size_t)(tok < B ? tok : 0) * C + scol;
    }

    for (int n0 = blockIdx.x * ROWS; n0 < upad; n0 += gridDim.x * ROWS) {
        // weight rows staged by this thread: matrix i / TPR, tile row srow + RPP (i % TPR); a
        // row past the union re-reads the union's last row (its D columns are discarded)
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int n = n0 + srow + RPP * (i % TPR);
            const size_t rb = (size_t)ulist[n < u ? n : u - 1] * C + scol;
            src[i] = (i / TPR == 0 ? W1 : Wup) + rb;
            tok_ok[i] = true;
        }
        f32x4 acc[PPW];
#pragma unroll
        for (int j = 0; j < PPW; ++j)
            acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

        u32x4 ring[PD][LPT];
        auto fill = [&](int p, int sg) {         // a segment past the end re-reads the last one
            const int c = (sg < nseg ? sg : nseg - 1) * SEGC;
#pragma unroll
            for (int i = 0; i < LPT; ++i)
                ring[p][i] = i < WPT ? ld_stream(src[i] + c) : src[i][c];
        };
        auto stage = [&](int p, int buf) {
#pragma unroll
            for (int i = 0; i < LPT; ++i)
                *reinterpret_cast<u32x4 *>(&seg[buf][srow + RPP * i][8 * scol]) =
                    tok_ok[i] ? ring[p][i] : zero;
        };
        auto compute = [&](int buf) {
#pragma unroll
            for (int s = 0; s < SPW; ++s) {
                const int k0 = kKStep * (kp * SPW + s) + 8 * g;
#pragma unroll
                for (int j = 0; j < PPW; ++j) {
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(&seg[buf][WR + 16 * pm[j] + ln][k0]);
                    const u32x4 b = *reinterpret_cast<const u32x4 *>(
                        &seg[buf][ROWS * pv[j] + 16 * pq[j] + ln][k0]);
                    acc[j] = T::mfma(a, b, acc[j]);
                }
            }
        };

#pragma unroll
        for (int p = 0; p < PD; ++p)
            fill(p, p);
        stage(0, 0);
        __syncthreads();
        const int groups = (nseg + PD - 1) / PD;
        for (int gi = 0; gi < groups; ++gi) {
#pragma unroll
            for (int p = 0; p < PD; ++p) {
                const int i = gi * PD + p;
                if (i < nseg) {                      // uniform across the workgroup
                    // slot p (segment i) is already in LDS: refill it with segment i + PD
                    fill(p, i + PD);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(i & 1);
                    if (i + 1 < nseg)
                        stage((p + 1) % PD, (i + 1) & 1);
                    __syncthreads();
                }
            }
        }

#pragma unroll
        for (int j = 0; j < PPW; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[kp][pidx[j]][i][lane] = acc[j][i];
        __syncthreads();
        // element e: tile q, token tile m, D index i, lane l -> token 16 m + 4 (l / 16) + i,
        // row n0 + 16 q + l % 16
        for (int e = t; e < RT * MT * 4 * kWave; e += 256) {
            const int q = e / (MT * 4 * kWave);
            const int m = (e / (4 * kWave)) % MT;
            const int i = (e / kWave) % 4, l = e % kWave;
            const int tok = 16 * m + 4 * (l >> 4) + i;
            const int nn = n0 + 16 * q + (l & 15);
            if (tok >= B || nn >= upad)
                continue;
            float hv = 0.0f;
            if (nn < u) {
                const int jj = ulist[nn];
                const int p0 = q * MT + m;
                float p = red[0][p0][i][l];
#pragma unroll
                for (int k = 1; k < KSPLIT; ++k)
                    p += red[k][p0][i][l];
                if (b1)
                    p += b1[jj];
                hv = gate_act(p, silu);
                if constexpr (NV == 2) {
                    const int p1 = RT * MT + q * MT + m;
                    float uv = red[0][p1][i][l];
#pragma unroll
                    for (int k = 1; k < KSPLIT; ++k)
                        uv += red[k][p1][i][l];
                    hv *= uv;
                }
                if (per_token && !token_has(bitmaps, words, tok, jj))
                    hv = 0.0f;
            }
            h32[(size_t)tok * hs + nn] = hv;
            const uint32_t hb = __float_as_uint(hv) & 0x7fffffffu;
            if (split_needs_scale<T>(hb))
                atomicMax(hmax + tok, hb);
        }
        __syncthreads();
    }
}

// Down projection.  Grid (256-column tile, union chunk).  The chunk's union indices are staged in
// LDS first.  Per K step of 32 union rows the workgroup stages the rows' 512-byte column segments
// and the 32 rows' h values of every token (split into hi and lo while they are staged) in LDS,
// double-buffered, with the global loads of the next PD steps in flight in a register ring; wave
// w then multiplies columns 64 w .. 64 w + 63 as 4 tiles of 16: A = h (tokens x 32 rows, hi then
// lo), B = the staged rows read column-wise (W2T is contiguous along the output columns, the
// product contracts over rows).
template <class T, int MT, int PD>
__global__ __launch_bounds__(256) void k_union_down_mfma(const u32x4 *__restrict__ W2T,
                                                         const float *__restrict__ h32,
                                                         const uint32_t *__restrict__ hmax,
                                                         int hs,
                                                         const int32_t *__restrict__ ulist,
                                                         const int32_t *__restrict__ ucount,
                                                         int B, int f, int C, int nchunk,
                                                         float *__restrict__ part)
{
    constexpr int SEG = kDownCols / 8;            // 16-byte chunks per staged row segment: 32
    __shared__ __align__(16) uint16_t tile[2][kKStep][kDownLdsStride];
    __shared__ __align__(16) uint16_t hst[2][2][kMaxUnionBatch][kKStep];   // [buf][hi/lo][tok][row]
    __shared__ int32_t rows[kMaxDownSteps * kKStep];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int ln = lane & 15, g = lane >> 4;
    const int D = C * 8;
    const int col0 = blockIdx.x * kDownCols;
    const int chunk = blockIdx.y;
    const int u = union_size(ucount, f);
    const int steps = (u + kKStep - 1) / kKStep;
    const int per = (steps + nchunk - 1) / nchunk;
    const int sb = chunk * per;
    const int se = sb + per < steps ? sb + per : steps;
    const int ns = se > sb ? se - sb : 0;         // <= kMaxDownSteps (the host sizes nchunk)

    // union indices of this chunk (positions past the union read the last entry; their h is 0)
    for (int i = t; i < ns * kKStep; i += 256) {
        const int nn = sb * kKStep + i;
        rows[i] = ulist[nn < u ? nn : u - 1];
    }
    __syncthreads();

    // staging: thread t moves rows srow + 8 q (q < 4) of column chunk scol, and 4 h values:
    // token ht, rows 4 hq .. 4 hq + 3, scaled by the token's 2^k and split into hi and lo
    const int srow = t / SEG, scol = t % SEG;
    const int ht = t >> 3, hq = t & 7;
    const bool hok = ht < B;
    const float *hsrc = h32 + (size_t)(hok ? ht : 0) * hs + 4 * hq;
    const float hsc = pow2_exact(hok ? split_shift<T>(hmax[ht]) : 0);
    // The ring holds raw loads (a step past the chunk re-reads its last step); they are only
    // read when staged, PD - 1 steps later, where a step past the chunk stages h = 0 (so the
    // re-read rows add nothing) and a token past B stages h = 0.
    u32x4 rw[PD][kKStep / 8], rh[PD];
    auto fill = [&](int p, int i) {            // i: step index within the chunk
        const int ic = i < ns ? i : ns - 1;
#pragma unroll
        for (int q = 0; q < kKStep / 8; ++q) {
            const int r = ic * kKStep + srow + 8 * q;
            rw[p][q] = ld_stream(W2T + (size_t)rows[r] * C + (col0 / 8) + scol);
        }
        rh[p] = *reinterpret_cast<const u32x4 *>(hsrc + (size_t)(sb + ic) * kKStep);
    };
    auto split2 = [&](uint32_t a, uint32_t b, uint32_t &hi, uint32_t &lo) {
        const float va = u2f(a) * hsc, vb = u2f(b) * hsc;
        const uint16_t ha = T::round_bits(va), hb = T::round_bits(vb);
        const uint16_t la = T::round_bits(va - T::widen_bits(ha));
        const uint16_t lb = T::round_bits(vb - T::widen_bits(hb));
        hi = (uint32_t)ha | ((uint32_t)hb << 16);
        lo = (uint32_t)la | ((uint32_t)lb << 16);
    };
    auto stage = [&](int p, int buf, int i) {
#pragma unroll
        for (int q = 0; q < kKStep / 8; ++q) {
            uint32_t *dst = reinterpret_cast<uint32_t *>(&tile[buf][srow + 8 * q][scol * 8]);
            // two 8-byte stores: the staged row stride is 8-byte aligned only
            *reinterpret_cast<uint2 *>(dst) = uint2{rw[p][q].x, rw[p][q].y};
            *reinterpret_cast<uint2 *>(dst + 2) = uint2{rw[p][q].z, rw[p][q].w};
        }
        uint2 hi = uint2{0u, 0u}, lo = uint2{0u, 0u};
        if (i < ns && hok) {
            split2(rh[p].x, rh[p].y, hi.x, lo.x);
            split2(rh[p].z, rh[p].w, hi.y, lo.y);
        }
        *reinterpret_cast<uint2 *>(&hst[buf][0][ht][4 * hq]) = hi;
        *reinterpret_cast<uint2 *>(&hst[buf][1][ht][4 * hq]) = lo;
    };

    f32x4 acc[4][MT];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[q][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    if (ns > 0) {
#pragma unroll
        for (int p = 0; p < PD; ++p)
            fill(p, p);
        stage(0, 0, 0);
        __syncthreads();
        const int groups = (ns + PD - 1) / PD;
        for (int gi = 0; gi < groups; ++gi) {
#pragma unroll
            for (int p = 0; p < PD; ++p) {
                const int i = gi * PD + p;
                const int buf = i & 1;
                // slot p (step i) is already in LDS: refill it with step i + PD (the barrier keeps
                // the scheduler from sinking these loads toward the staging)
                fill(p, i + PD);
                __builtin_amdgcn_sched_barrier(0);
                u32x4 ahi[MT], alo[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    ahi[m] = *reinterpret_cast<const u32x4 *>(&hst[buf][0][16 * m + ln][8 * g]);
                    alo[m] = *reinterpret_cast<const u32x4 *>(&hst[buf][1][16 * m + ln][8 * g]);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int cc = 64 * w + 16 * q + ln;
                    uint32_t bv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        bv[e] = (uint32_t)tile[buf][8 * g + 2 * e][cc] |
                                ((uint32_t)tile[buf][8 * g + 2 * e + 1][cc] << 16);
                    const u32x4 b = u32x4{bv[0], bv[1], bv[2], bv[3]};
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        acc[q][m] = T::mfma(ahi[m], b, acc[q][m]);
                        acc[q][m] = T::mfma(alo[m], b, acc[q][m]);
                    }
                }
                stage((p + 1) % PD, buf ^ 1, i + 1);   // step i + 1
                __syncthreads();
            }
        }
    }

    // D[4 g + i][ln] of tile (q, m): token 16 m + 4 g + i, column col0 + 64 w + 16 q + ln; the
    // token's 2^-k undoes the scale of its h (exactly: a power of two)
    float unsc[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 16 * m + 4 * g + i;
            unsc[m][i] = pow2_exact(tok < B ? -split_shift<T>(hmax[tok]) : 0);
        }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int col = col0 + 64 * w + 16 * q + ln;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * m + 4 * g + i;
                if (tok < B && col < D)
                    part[((size_t)tok * nchunk + chunk) * (size_t)D + col] = acc[q][m][i] * unsc[m][i];
            }
    }
}

// ---- dispatch ----------------------------------------------------------------------------------
template <class T, int MX, bool GATED>
hipError_t up_valu(const UnionArgs &a, int C, hipStream_t st, Trace *tr)
{
    constexpr int RPW = UpRows<MX, GATED>::value;
    const int blocks = (a.f + RPW - 1) / RPW < 4096 ? (a.f + RPW - 1) / RPW : 4096;
    return launch(k_union_up_valu<T, MX, GATED, RPW>, dim3(blocks), dim3(256), st, tr,
                  static_cast<const u32x4 *>(a.X), static_cast<const u32x4 *>(a.W1),
                  static_cast<const u32x4 *>(a.Wup), a.b1, a.ulist, a.ucount, a.bitmaps,
                  a.per_token, a.B, a.f, C, a.h32, a.hs, act_silu(a.act));
}

template <class T, bool GATED>
hipError_t up_valu_mx(const UnionArgs &a, int C, hipStream_t st, Trace *tr)
{
    const int mx = (C + 255) / 256;
    if (mx <= 1) return up_valu<T, 1, GATED>(a, C, st, tr);
    if (mx <= 2) return up_valu<T, 2, GATED>(a, C, st, tr);
    if (mx <= 4) return up_valu<T, 4, GATED>(a, C, st, tr);
    if (mx <= 6) return up_valu<T, 6, GATED>(a, C, st, tr);
    if (mx <= 8) return up_valu<T, 8, GATED>(a, C, st, tr);
    if (mx <= 12) return up_valu<T, 12, GATED>(a, C, st, tr);
    if (mx <= 16) return up_valu<T, 16, GATED>(a, C, st, tr);
    return hipErrorInvalidValue;
}

template <class T>
hipError_t union_valu(const UnionArgs &a, hipStream_t st, Trace *tr)
{
    const int C = a.d / T::E;
    hipError_t e = act_gated(a.act) ? up_valu_mx<T, true>(a, C, st, tr) : up_valu_mx<T, false>(a, C, st, tr);
    if (e != hipSuccess)
        return e;
    const int nchunk = union_num_chunks(0, a.d, a.dtype, a.f, a.cus);
    const dim3 grid(ffn_num_slices(a.d, a.dtype), nchunk, (a.B + kValuTokens - 1) / kValuTokens);
    if (a.B <= 1)
        e = launch(k_union_down_valu<T, 1, 4>, grid, dim3(256), st, tr,
                   static_cast<const u32x4 *>(a.W2T), a.h32, a.hs, a.ulist, a.ucount, a.B, a.f, C,
                   nchunk, a.partials);
    else if (a.B <= 4)
        e = launch(k_union_down_valu<T, 4, 2>, grid, dim3(256), st, tr,
                   static_cast<const u32x4 *>(a.W2T), a.h32, a.hs, a.ulist, a.ucount, a.B, a.f, C,
                   nchunk, a.partials);
    else
        e = launch(k_union_down_valu<T, kValuTokens, 2>, grid, dim3(256), st, tr,
                   static_cast<const u32x4 *>(a.W2T), a.h32, a.hs, a.ulist, a.ucount, a.B, a.f, C,
                   nchunk, a.partials);
    if (e != hipSuccess)
        return e;
    return launch_reduce_partials(a.partials, nchunk, a.d, a.B, a.Y, st, tr);
}

template <class T, int MT, int ST, int ROWS>
hipError_t union_mfma_mt(const UnionArgs &a, hipStream_t st, Trace *tr)
{
    const int C = a.d / 8;
    const int tiles = (a.f + ROWS - 1) / ROWS;
    const int blocks = tiles < 4096 ? tiles : 4096;
    hipError_t e;
    if (act_gated(a.act))
        e = launch(k_union_up_lds<T, MT, 2, 3, ST, ROWS>, dim3(blocks), dim3(256), st, tr,
                   static_cast<const u32x4 *>(a.X), static_cast<const u32x4 *>(a.W1),
                   static_cast<const u32x4 *>(a.Wup), a.b1, a.ulist, a.ucount, a.bitmaps,
                   a.per_token, a.B, a.f, C, a.h32, a.hmax, a.hs, act_silu(a.act));
    else
        e = launch(k_union_up_lds<T, MT, 1, 3, ST, ROWS>, dim3(blocks), dim3(256), st, tr,
                   static_cast<const u32x4 *>(a.X), static_cast<const u32x4 *>(a.W1),
                   static_cast<const u32x4 *>(a.Wup), a.b1, a.ulist, a.ucount, a.bitmaps,
                   a.per_token, a.B, a.f, C, a.h32, a.hmax, a.hs, act_silu(a.act));
    if (e != hipSuccess)
        return e;
    const int nchunk = union_num_chunks(1, a.d, a.dtype, a.f, a.cus);
    // two K steps of loads in flight ahead (measured at 8 / 16 / 32 tokens: 47.8 / 57.1 / 73.9 us
    // against 49.2 / 59.7 / 75.2 with three and 51.4 / 61.6 / 79.6 with four)
    e = launch(k_union_down_mfma<T, MT, 2>, dim3(a.d / kDownCols, nchunk), dim3(256), st, tr,
               static_cast<const u32x4 *>(a.W2T), a.h32, a.hmax, a.hs, a.ulist, a.ucount, a.B, a.f,
               C, nchunk, a.partials);
    if (e != hipSuccess)
        return e;
    return launch_reduce_partials(a.partials, nchunk, a.d, a.B, a.Y, st, tr);
}

template <class T>
hipError_t union_mfma(const UnionArgs &a, hipStream_t st, Trace *tr)
{
    // staged segment length (measured): 512-byte segments for one token tile of few tokens,
    // 256-byte ones (less LDS and fewer registers per workgroup, so two workgroups per CU)
    // from 8 tokens on.  Up-projection rows per workgroup (measured on clustered OPT-30B-shape
    // batches): 16 at two tokens (26.8 against 29.9 us: the small union gives twice as many
    // workgroups); 32 from four on, where 16 measured 1-1.5 us slower at 4 and 16 tokens and
    // 31 us slower at 32 (the token rows re-read from L2 per tile double)
    if (a.B <= 2)
        return union_mfma_mt<T, 1, 256, 16>(a, st, tr);
    if (a.B <= 7)
        return union_mfma_mt<T, 1, 256, 32>(a, st, tr);
    if (a.B <= 16)
        return union_mfma_mt<T, 1, 128, 32>(a, st, tr);
    return union_mfma_mt<T, 2, 128, 32>(a, st, tr);
}

}  // namespace

bool union_mfma_supported(int dtype, int d, int B)
{
    return dtype != 0 && d % kDownCols == 0 && B >= 1 && B <= kMaxUnionBatch;
}

int union_num_chunks(int mfma, int d, int dtype, int f, int cus)
{
    if (!mfma)
        return ffn_num_chunks(d, dtype, f);
    // as many chunks as keep the grid at two workgroups of 256 columns per CU or fewer (a chunk
    // holds at most kMaxDownSteps K steps, which can force more); the partial rows (B x chunks x
    // d float32) stay a few percent of the weight bytes.  Measured per batch of 32 tokens at the
    // OPT-30B shape (28 column tiles): 18 chunks (504 workgroups) 179.2 us, 14 / 16 chunks 185.0 /
    // 181.5 (CUs with one workgroup beside CUs with two), 19 chunks 192.3 (three workgroups on
    // some CUs, two on the rest), three on every CU 192.5; the same order at 8 and 16 tokens and
    // for the dense batched step
    const int tiles = d / kDownCols > 0 ? d / kDownCols : 1;
    const int steps = (f + kKStep - 1) / kKStep;
    int n = (int)(2L * cus / tiles);
    const int least = (steps + kMaxDownSteps - 1) / kMaxDownSteps;
    if (n > steps)
        n = steps;
    if (n > 64)
        n = 64;
    if (n < least)
        n = least;
    return n < 1 ? 1 : n;
}

size_t union_h_stride(int f) { return (size_t)(f + kKStep - 1) / kKStep * kKStep; }

hipError_t launch_union_ffn(const UnionArgs &a, hipStream_t st, Trace *tr)
{
    hipError_t e = launch(k_union_list, dim3(1), dim3(kUnionThreads), st, tr, a.bitmaps, a.B, a.f,
                          a.ulist, a.ucount, a.ucount_out, a.hmax);
    if (e != hipSuccess)
        return e;
    if (a.mfma) {
        if (a.dtype == 1) return union_mfma<F16T>(a, st, tr);
        return union_mfma<BF16T>(a, st, tr);
    }
    if (a.B == 1) {
        // one token: the union is its own list, so the single-token gathered FFN applies as it
        // is (rows whole per workgroup, the list staged in LDS for the down projection)
        FfnArgs fa;
        fa.dtype = a.dtype;
        fa.act = a.act;
        fa.x = a.X;
        fa.B = 1;
        fa.d = a.d;
        fa.f = a.f;
        fa.W1 = a.W1;
        fa.Wup = a.Wup;
        fa.W2T = a.W2T;
        fa.b1 = a.b1;
        fa.idx = a.ulist;
        fa.idx_stride = a.f;
        fa.count = a.ucount;
        fa.max_count = a.f;
        fa.h = a.h32;
        fa.h_stride = a.hs;
        fa.y = a.Y;
        fa.partials = a.partials;
        return launch_ffn(fa, st, tr);
    }
    if (a.dtype == 0) return union_valu<F32T>(a, st, tr);
    if (a.dtype == 1) return union_valu<F16T>(a, st, tr);
    return union_valu<BF16T>(a, st, tr);
}

}  // namespace csf
