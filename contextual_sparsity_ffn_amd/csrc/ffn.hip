// ffn.hip -- the gathered FFN on gfx950: active gate/up rows, activation, and the neuron-major
// down projection with a deterministic two-phase float32 reduction.
//
// "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm":
//   "The Prediction Problem" (sparse_mlp_forward) -- gather the active gate rows and the matching
//   down weights and compute only those;
//   "Kernel-Level Implementation" -- one dot product per selected neuron with float32 accumulation,
//   then max(acc, 0); plain indexing must not break coalescing;
//   "The SiLU/GELU Challenge: TurboSparse" -- the ReLU-fied gated form relu(gate x) * (up x).
//
// The page's sketch gives one thread per neuron, so a wavefront's lanes walk 64 different rows and
// no load is coalesced.  Here every row is read whole by a full workgroup in 16-byte chunks (1 KiB
// per wavefront instruction, contiguous), and the down projection is stored neuron-major so that
// the weights of an active neuron are one contiguous row as well:
//   k_gather_up    workgroup of 256 threads per RPW active rows: h_n = act(W1[j_n].x + b1, Wup[j_n].x)
//   k_gather_down  grid (d-slice of 1 KiB per row) x (chunk of the active list) x token; a partial
//                  row per chunk;
//   k_reduce_partials  sums the partial rows in chunk order (fixed order, so deterministic).
#include "common.hpp"
#include "launch.hpp"

namespace csf {

namespace {

constexpr int kDownUnroll = 12;   // list entries whose 16-byte chunks are in flight per lane
constexpr int kMaxChunkRows = 1024; // list entries per down-projection chunk (staged in LDS)
constexpr int kSliceChunks = 64;  // one 16-byte chunk per lane: a d-slice is 1 KiB of a row
constexpr int kMaxChunks = 64;    // most neuron chunks (partial rows) per slice

__device__ __forceinline__ int token_count(const int32_t *count, int token, int max_count)
{
    if (!count)
        return max_count;
    int c = count[token];
    return c < 0 ? 0 : (c > max_count ? max_count : c);
}

template <int MX, bool GATED>
struct UpShape {
    // rows per workgroup: about 12 chunk loads in flight per thread, at most 4 rows (measured:
    // deeper queues per thread with fewer workgroups gather more slowly)
    static constexpr int loads = MX * (GATED ? 2 : 1);
    static constexpr int RPW = loads >= 12 ? 1 : (loads >= 6 ? 2 : 4);
};

// SKIP (post-gate skip): a neuron whose gate activation a = act(W1[j].x + b1_j) has
// |a| <= gate_tau gets h = 0 (for the ReLU forms with gate_tau = 0: exactly the neurons whose h is
// zero anyway).  In the gated forms the gate dot products are finished first and the workgroup
// then loads only the up rows that are still needed.
template <class T, int MX, bool GATED, bool SKIP = false, int RPW = UpShape<MX, GATED>::RPW>
__global__ __launch_bounds__(256) void k_gather_up(const u32x4 *__restrict__ x,
                                                   const u32x4 *__restrict__ W1,
                                                   const u32x4 *__restrict__ Wup,
                                                   const float *__restrict__ b1,
                                                   const int32_t *__restrict__ idx,
                                                   int idx_stride,
                                                   const int32_t *__restrict__ count,
                                                   int max_count, int f, int C,
                                                   float *__restrict__ h, int h_stride, int silu,
                                                   float gate_tau)
{
    __shared__ float red[4][RPW][GATED ? 2 : 1];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int token = blockIdx.y;
    const int n0 = blockIdx.x * RPW;
    const int cnt = token_count(count, token, max_count);
    if (n0 >= cnt)
        return;                                   // uniform across the workgroup

    const u32x4 *xt = x + (size_t)token * C;
    u32x4 xv[MX];
#pragma unroll
    for (int m = 0; m < MX; ++m) {
        const int c = t + 256 * m;
        xv[m] = c < C ? xt[c] : u32x4{0u, 0u, 0u, 0u};
    }

    // jr = neuron of list entry n0+i; -1 past the list end; -2 for an index outside [0, f), which
    // contributes nothing (its h is written as 0 and the down projection skips it)
    int jr[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int n = n0 + i;
        int j = n < cnt ? (idx ? idx[(size_t)token * idx_stride + n] : n) : -1;
        if (n < cnt && (j < 0 || j >= f))
            j = -2;
        jr[i] = j;
    }

    u32x4 wv[RPW][MX];
    u32x4 uv[GATED ? RPW : 1][GATED ? MX : 1];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const u32x4 *row = W1 + (size_t)(jr[i] < 0 ? 0 : jr[i]) * C;
#pragma unroll
        for (int m = 0; m < MX; ++m) {
            const int c = t + 256 * m;
            wv[i][m] = (jr[i] >= 0 && c < C) ? ld_stream(row + c) : u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (GATED && !SKIP) {
            const u32x4 *urow = Wup + (size_t)(jr[i] < 0 ? 0 : jr[i]) * C;
#pragma unroll
            for (int m = 0; m < MX; ++m) {
                const int c = t + 256 * m;
                uv[i][m] = (jr[i] >= 0 && c < C) ? ld_stream(urow + c) : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }

    if constexpr (GATED && SKIP) {
        // gates first; then the up rows of the rows whose gate (with bias) is positive
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            float acc = 0.0f;
#pragma unroll
            for (int m = 0; m < MX; ++m)
                acc = T::dot(wv[i][m], xv[m], acc);
            acc = wave_sum(acc);
            if (lane == 0)
                red[w][i][0] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            float p = (red[0][i][0] + red[1][i][0]) + (red[2][i][0] + red[3][i][0]);
            if (b1 && jr[i] >= 0)
                p += b1[jr[i]];
            // uniform across the workgroup
            const bool live = jr[i] >= 0 && fabsf(gate_act(p, silu)) > gate_tau;
            const u32x4 *urow = Wup + (size_t)(live ? jr[i] : 0) * C;
#pragma unroll
            for (int m = 0; m < MX; ++m) {
                const int c = t + 256 * m;
                uv[i][m] = (live && c < C) ? ld_stream(urow + c) : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }

#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int m = 0; m < MX; ++m)
            acc = T::dot(wv[i][m], xv[m], acc);
        acc = wave_sum(acc);
        if (lane == 0 && !(GATED && SKIP))
            red[w][i][0] = acc;
        if constexpr (GATED) {
            float au = 0.0f;
#pragma unroll
            for (int m = 0; m < MX; ++m)
                au = T::dot(uv[i][m], xv[m], au);
            au = wave_sum(au);
            if (lane == 0)
                red[w][i][GATED ? 1 : 0] = au;
        }
    }
    __syncthreads();
    if (t < RPW && jr[t] == -2)
        h[(size_t)token * h_stride + n0 + t] = 0.0f;
    if (t < RPW && jr[t] >= 0) {
        const int i = t;
        float p = (red[0][i][0] + red[1][i][0]) + (red[2][i][0] + red[3][i][0]);
        if (b1)
            p += b1[jr[i]];
        float hv = gate_act(p, silu);
        const bool drop = SKIP && !(fabsf(hv) > gate_tau);
        if constexpr (GATED) {
            const int g = GATED ? 1 : 0;
            const float u = (red[0][i][g] + red[1][i][g]) + (red[2][i][g] + red[3][i][g]);
            hv *= u;
        }
        h[(size_t)token * h_stride + n0 + i] = drop ? 0.0f : hv;
    }
}

// Down projection.  Grid: (d-slice of 64 chunks, neuron chunk, token).  Each lane owns one
// 16-byte chunk column of the slice, so a wavefront instruction reads 1 KiB of one row, contiguous.
// The chunk's list entries and their h values are staged in LDS first (so no row load waits on an
// index load), then the 4 wavefronts take every 4th entry with kDownUnroll rows in flight each.
// The wavefronts are summed in a fixed order and the chunk's partial row is stored;
// k_reduce_partials then sums the partial rows in chunk order.  Handing the partials to another
// workgroup inside this kernel would need a device-coherent write-back of each XCD's L2 per
// workgroup, which costs more than the kernel boundary.  No float atomics anywhere, so y is
// deterministic.
template <class T>
__global__ __launch_bounds__(256) void k_gather_down(const u32x4 *__restrict__ W2T,
                                                     const float *__restrict__ h, int h_stride,
                                                     const int32_t *__restrict__ idx,
                                                     int idx_stride,
                                                     const int32_t *__restrict__ count,
                                                     int max_count, int f, int C, int nchunk,
                                                     int skip_zero, float *__restrict__ part)
{
    constexpr int E = T::E;
    __shared__ float red[3][kSliceChunks * E];
    __shared__ int32_t sj[kMaxChunkRows];
    __shared__ float sh[kMaxChunkRows];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int slice = blockIdx.x, chunk = blockIdx.y, token = blockIdx.z;
    const int D = C * E;
    const int c = slice * kSliceChunks + lane;
    const int cnt = token_count(count, token, max_count);
    const int per = (cnt + nchunk - 1) / nchunk;
    const int nb = chunk * per;
    const int ne = nb + per < cnt ? nb + per : cnt;
    const int ns = ne > nb ? ne - nb : 0;          // <= kMaxChunkRows (the host sizes nchunk)
    const int32_t *it = idx ? idx + (size_t)token * idx_stride : nullptr;
    const float *ht = h + (size_t)token * h_stride;

    // an entry outside [0, f) contributes nothing: row 0 with h = 0.  skip_zero: entries with
    // h = 0 are dropped (order kept), so their rows are not read at all.
    int nk = ns;
    if (!skip_zero) {
        for (int i = t; i < ns; i += 256) {
            const int j = it ? it[nb + i] : nb + i;
            const bool ok = j >= 0 && j < f;
            sj[i] = ok ? j : 0;
            sh[i] = ok ? ht[nb + i] : 0.0f;
        }
    } else {
        __shared__ uint32_t scan_tmp[4];
        int base = 0;
        for (int r0 = 0; r0 < ns; r0 += 256) {
            const int i = r0 + t;
            int j = 0;
            float hv = 0.0f;
            if (i < ns) {
                j = it ? it[nb + i] : nb + i;
                hv = (j >= 0 && j < f) ? ht[nb + i] : 0.0f;
            }
            const bool keep = hv != 0.0f;
            uint32_t tot;
            const uint32_t pos = block_exclusive_scan<4>(keep ? 1u : 0u, scan_tmp, &tot);
            if (keep) {
                sj[base + pos] = j;
                sh[base + pos] = hv;
            }
            base += (int)tot;
        }
        nk = base;
    }
    __syncthreads();

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        acc[e] = 0.0f;
    for (int i0 = w; i0 < nk; i0 += 4 * kDownUnroll) {
        u32x4 wv[kDownUnroll];
        float hv[kDownUnroll];
#pragma unroll
        for (int u = 0; u < kDownUnroll; ++u) {
            const int i = i0 + 4 * u;
            const bool ok = i < nk && c < C;
            hv[u] = i < nk ? sh[i] : 0.0f;
            wv[u] = ok ? ld_stream(W2T + (size_t)sj[i] * C + c) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kDownUnroll; ++u) {
            float wf[E];
            T::unpack(wv[u], wf);
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[e] = fmaf(hv[u], wf[e], acc[e]);
        }
    }

    // fixed-order sum of the 4 wavefronts: ((wave 0 + wave 1) + wave 2) + wave 3
    if (w > 0) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            red[w - 1][lane * E + e] = acc[e];
    }
    __syncthreads();
    if (w == 0 && c < C) {
        float *out = part + ((size_t)token * nchunk + chunk) * (size_t)D + (size_t)c * E;
#pragma unroll
        for (int e = 0; e < E; ++e)
            out[e] = ((acc[e] + red[0][lane * E + e]) + red[1][lane * E + e]) + red[2][lane * E + e];
    }
}

// y[token][col] = sum over chunks q of part[token][q][col] in a fixed order; accumulate: y += that
// sum (the residual add of a stack of blocks).  A workgroup covers 64 columns: wave w sums chunks
// w, w + 4, ... for the lane's column (every load issued before the first add) and the 4 waves'
// sums are added in wave order.
__global__ __launch_bounds__(256) void k_reduce_partials(const float *__restrict__ part, int nchunk,
                                                         int D, float *__restrict__ y,
                                                         int accumulate)
{
    __shared__ float red[4][kWave];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int col = blockIdx.x * kWave + lane;
    const int token = blockIdx.y;
    const float *p = part + (size_t)token * nchunk * (size_t)D + (col < D ? col : 0);
    float pv[kMaxChunks / 4];
#pragma unroll
    for (int q = 0; q < kMaxChunks / 4; ++q) {
        const int ch = w + 4 * q;
        pv[q] = (ch < nchunk && col < D) ? p[(size_t)ch * D] : 0.0f;
    }
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < kMaxChunks / 4; ++q)
        sum += pv[q];
    red[w][lane] = sum;
    __syncthreads();
    if (w == 0 && col < D) {
        const float tot = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
        float *out = y + (size_t)token * D + col;
        *out = accumulate ? *out + tot : tot;
    }
}

// ---- one token in one kernel: up rows, down rows and the reduction ----------------------------
// The three stages above as roles of one launch, in this order of workgroup index:
//   nup     "up" workgroups, RPW list entries each with every row load issued at once, as
//           k_gather_up computes them (the up rows are the critical path, so they are all
//           requested first).  Each h is stored coherently over a sentinel the call's first
//           kernel wrote there (kHSentinel, a NaN pattern; a NaN h, which a float32 input's NaN
//           payload could carry through, is stored as the default quiet NaN instead), so no
//           counter and no wait for the store is needed;
//   nitems  "down" workgroups, one (chunk, d-slice) item of k_gather_down each, chunk-major: each
//           wavefront's first kDownUnroll rows of the item are requested first, then the
//           workgroup polls the chunk's h values until none is the sentinel and finishes; the
//           partial row is stored coherently (whole 128-byte lines) and counted in done[slice];
//   nred    "reduce" workgroups of 64 output columns: each waits for done[slice] == nchunk and
//           sums the partial rows as k_reduce_partials does.
// Down workgroups take the slots the up workgroups free and stream their rows while the last up
// rows arrive, and no kernel boundary separates the stages.  Every sum has the order of the
// three-kernel form, so y is bit-identical to it.  A workgroup only waits for workgroups of lower
// index (dispatched first), and every wait is bounded (common.hpp).  h[0, max_count) must hold
// kHSentinel and the counters (done[kMaxChunks], err, one 128-byte line each) zero when the
// kernel starts: the call's first kernel writes them.
struct FusedFfnArgs {
    const u32x4 *x, *W1, *Wup, *W2T;
    const float *b1;
    const int32_t *idx;
    const int32_t *count;
    int max_count, f, C, silu, nup, nslice, nchunk, accumulate;
    float *h, *part, *y;
    uint32_t *sync;    // done[kMaxChunks], err: one 128-byte line each
};

__device__ __forceinline__ uint32_t *done_ctr(const FusedFfnArgs &a, int s) { return a.sync + s * kLineWords; }
__device__ __forceinline__ uint32_t *err_ctr(const FusedFfnArgs &a) { return a.sync + kMaxChunks * kLineWords; }

template <class T, int MX, bool GATED, int RPW = UpShape<MX, GATED>::RPW>
__device__ __forceinline__ void fused_up(const FusedFfnArgs &a, int blk)
{
    __shared__ float red[4][RPW][GATED ? 2 : 1];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int n0 = blk * RPW;
    const int cnt = token_count(a.count, 0, a.max_count);
    if (n0 >= cnt)
        return;
    const int C = a.C;
    int jr[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int n = n0 + i;
        int j = n < cnt ? (a.idx ? a.idx[n] : n) : -1;
        if (n < cnt && (j < 0 || j >= a.f))
            j = -2;
        jr[i] = j;
    }
    u32x4 wv[RPW][MX];
    u32x4 uv[GATED ? RPW : 1][GATED ? MX : 1];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const u32x4 *row = a.W1 + (size_t)(jr[i] < 0 ? 0 : jr[i]) * C;
#pragma unroll
        for (int m = 0; m < MX; ++m) {
            const int c = t + 256 * m;
            wv[i][m] = (jr[i] >= 0 && c < C) ? ld_stream(row + c) : u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (GATED) {
            const u32x4 *urow = a.Wup + (size_t)(jr[i] < 0 ? 0 : jr[i]) * C;
#pragma unroll
            for (int m = 0; m < MX; ++m) {
                const int c = t + 256 * m;
                uv[i][m] = (jr[i] >= 0 && c < C) ? ld_stream(urow + c) : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    u32x4 xv[MX];
#pragma unroll
    for (int m = 0; m < MX; ++m) {
        const int c = t + 256 * m;
        xv[m] = c < C ? a.x[c] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int m = 0; m < MX; ++m)
            acc = T::dot(wv[i][m], xv[m], acc);
        acc = wave_sum(acc);
        if (lane == 0)
            red[w][i][0] = acc;
        if constexpr (GATED) {
            float au = 0.0f;
#pragma unroll
            for (int m = 0; m < MX; ++m)
                au = T::dot(uv[i][m], xv[m], au);
            au = wave_sum(au);
            if (lane == 0)
                red[w][i][GATED ? 1 : 0] = au;
        }
    }
    __syncthreads();
    if (t < RPW && jr[t] != -1) {
        const int i = t;
        float hv = 0.0f;
        if (jr[i] >= 0) {
            float p = (red[0][i][0] + red[1][i][0]) + (red[2][i][0] + red[3][i][0]);
            if (a.b1)
                p += a.b1[jr[i]];
            hv = gate_act(p, a.silu);
            if constexpr (GATED) {
                const int g = GATED ? 1 : 0;
                const float u = (red[0][i][g] + red[1][i][g]) + (red[2][i][g] + red[3][i][g]);
                hv *= u;
            }
        }
        if ((__float_as_uint(hv) & 0x7fffffffu) > 0x7f800000u)
            hv = __uint_as_float(0x7fc00000u);
        st_coherent(a.h + n0 + i, hv);
    }
}

template <class T>
__device__ __forceinline__ void fused_down(const FusedFfnArgs &a, int item)
{
    constexpr int E = T::E;
    constexpr int COLS = kSliceChunks * E;
    __shared__ float red[3][COLS];
    __shared__ float outp[COLS];
    __shared__ int32_t sj[kMaxChunkRows];
    __shared__ float sh[kMaxChunkRows];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int C = a.C, D = C * E;
    const int cnt = token_count(a.count, 0, a.max_count);
    const int per = (cnt + a.nchunk - 1) / a.nchunk;
    const int chunk = item / a.nslice, slice = item % a.nslice;
    const int c = slice * kSliceChunks + lane;
    const int nb = chunk * per;
    const int ne = nb + per < cnt ? nb + per : cnt;
    const int ns = ne > nb ? ne - nb : 0;
    for (int i = t; i < ns; i += 256) {
        const int j = a.idx ? a.idx[nb + i] : nb + i;
        sj[i] = (j >= 0 && j < a.f) ? j : -1;
    }
    __syncthreads();
    // the first rows of every wavefront are requested before h is known
    u32x4 wv[kDownUnroll];
#pragma unroll
    for (int u = 0; u < kDownUnroll; ++u) {
        const int i = w + 4 * u;
        const int j = i < ns ? sj[i] : -1;
        wv[u] = (i < ns && c < C) ? ld_stream(a.W2T + (size_t)(j < 0 ? 0 : j) * C + c)
                                  : u32x4{0u, 0u, 0u, 0u};
    }
    // the chunk's h values: poll each until the up workgroup has replaced the sentinel (bounded)
    bool late = false;
    for (int i = t; i < ns; i += 256) {
        uint32_t v = __float_as_uint(ld_coherent(a.h + nb + i));
        for (uint32_t it = 0; v == kHSentinel && it < kSpinLimit; ++it) {
            __builtin_amdgcn_s_sleep(2);
            v = __float_as_uint(ld_coherent(a.h + nb + i));
        }
        if (v == kHSentinel) {
            late = true;
            v = 0u;
        }
        sh[i] = sj[i] >= 0 ? __uint_as_float(v) : 0.0f;
    }
    if (late)
        count_add(err_ctr(a), 1u);
    __syncthreads();

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        acc[e] = 0.0f;
    for (int i0 = w; i0 < ns; i0 += 4 * kDownUnroll) {
        float hv[kDownUnroll];
        if (i0 != w) {
#pragma unroll
            for (int u = 0; u < kDownUnroll; ++u) {
                const int i = i0 + 4 * u;
                const int j = i < ns ? sj[i] : -1;
                wv[u] = (i < ns && c < C) ? ld_stream(a.W2T + (size_t)(j < 0 ? 0 : j) * C + c)
                                          : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < kDownUnroll; ++u) {
            const int i = i0 + 4 * u;
            hv[u] = i < ns ? sh[i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kDownUnroll; ++u) {
            float wf[E];
            T::unpack(wv[u], wf);
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[e] = fmaf(hv[u], wf[e], acc[e]);
        }
    }
    if (w > 0) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            red[w - 1][lane * E + e] = acc[e];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            outp[lane * E + e] = ((acc[e] + red[0][lane * E + e]) + red[1][lane * E + e]) +
                                 red[2][lane * E + e];
    }
    __syncthreads();
    // the slice's partial row, two columns per thread: each store instruction writes whole lines
    float *out = a.part + (size_t)chunk * D + (size_t)slice * COLS;
    for (int qq = 2 * t; qq < COLS; qq += 512) {
        if (slice * COLS + qq < D) {
            const uint64_t v = (uint64_t)__float_as_uint(outp[qq]) |
                               ((uint64_t)__float_as_uint(outp[qq + 1]) << 32);
            __hip_atomic_store(reinterpret_cast<uint64_t *>(out + qq), v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // no load is in flight any more: this waits for the partial row's stores only
    wait_own_memory();
    __syncthreads();
    if (t == 0)
        count_add(done_ctr(a, slice), 1u);
}

// 64 output columns, as k_reduce_partials: wave w sums chunks w, w + 4, ... for the lane's column
// (every load issued before the first add) and the four sums are added in wave order
template <class T>
__device__ __forceinline__ void fused_reduce(const FusedFfnArgs &a, int blk)
{
    constexpr int COLS = kSliceChunks * T::E;
    __shared__ float red[4][kWave];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int D = a.C * T::E;
    const int col = blk * kWave + lane;
    if (t == 0)
        wait_count(done_ctr(a, blk * kWave / COLS), (uint32_t)a.nchunk, err_ctr(a));
    __syncthreads();
    const float *p = a.part + (col < D ? col : 0);
    float pv[kMaxChunks / 4];
#pragma unroll
    for (int q = 0; q < kMaxChunks / 4; ++q) {
        const int ch = w + 4 * q;
        pv[q] = (ch < a.nchunk && col < D) ? ld_coherent(p + (size_t)ch * D) : 0.0f;
    }
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < kMaxChunks / 4; ++q)
        sum += pv[q];
    red[w][lane] = sum;
    __syncthreads();
    if (w == 0 && col < D) {
        const float tot = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
        a.y[col] = a.accumulate ? a.y[col] + tot : tot;
    }
}

template <class T, int MX, bool GATED>
__global__ __launch_bounds__(256) void k_ffn_fused(FusedFfnArgs a)
{
    const int b = blockIdx.x;
    const int items = a.nslice * a.nchunk;
    if (b < a.nup)
        fused_up<T, MX, GATED>(a, b);
    else if (b < a.nup + items)
        fused_down<T>(a, b - a.nup);
    else
        fused_reduce<T>(a, b - a.nup - items);
}

template <class T, int MX, bool GATED>
hipError_t fused_launch(const FfnArgs &a, uint32_t *sync, hipStream_t st, Trace *tr)
{
    constexpr int RPW = UpShape<MX, GATED>::RPW;
    FusedFfnArgs g;
    g.x = static_cast<const u32x4 *>(a.x);
    g.W1 = static_cast<const u32x4 *>(a.W1);
    g.Wup = static_cast<const u32x4 *>(a.Wup);
    g.W2T = static_cast<const u32x4 *>(a.W2T);
    g.b1 = a.b1;
    g.idx = a.idx;
    g.count = a.count;
    g.max_count = a.max_count;
    g.f = a.f;
    g.C = a.d / T::E;
    g.silu = act_silu(a.act);
    g.nslice = ffn_num_slices(a.d, a.dtype);
    g.nchunk = ffn_num_chunks(a.d, a.dtype, a.max_count);
    g.accumulate = a.accumulate;
    g.h = a.h;
    g.part = a.partials;
    g.y = a.y;
    g.sync = sync;
    g.nup = (a.max_count + RPW - 1) / RPW;
    const int nred = (a.d + kWave - 1) / kWave;
    const int blocks = g.nup + g.nslice * g.nchunk + nred;
    return launch(k_ffn_fused<T, MX, GATED>, dim3(blocks), dim3(256), st, tr, g);
}

template <class T, bool GATED>
hipError_t fused_gated(const FfnArgs &a, uint32_t *sync, hipStream_t st, Trace *tr)
{
    const int mx = (a.d / T::E + 255) / 256;
    if (mx <= 1) return fused_launch<T, 1, GATED>(a, sync, st, tr);
    if (mx <= 2) return fused_launch<T, 2, GATED>(a, sync, st, tr);
    if (mx <= 4) return fused_launch<T, 4, GATED>(a, sync, st, tr);
    if (mx <= 6) return fused_launch<T, 6, GATED>(a, sync, st, tr);
    if (mx <= 8) return fused_launch<T, 8, GATED>(a, sync, st, tr);
    if (mx <= 12) return fused_launch<T, 12, GATED>(a, sync, st, tr);
    if (mx <= 16) return fused_launch<T, 16, GATED>(a, sync, st, tr);
    return hipErrorInvalidValue;
}

template <class T>
hipError_t fused_t(const FfnArgs &a, uint32_t *sync, hipStream_t st, Trace *tr)
{
    return act_gated(a.act) ? fused_gated<T, true>(a, sync, st, tr)
                            : fused_gated<T, false>(a, sync, st, tr);
}

template <class T, int MX, bool GATED>
hipError_t up_launch(const FfnArgs &a, int C, hipStream_t st, Trace *tr)
{
    constexpr int RPW = UpShape<MX, GATED>::RPW;
    const int blocks = (a.max_count + RPW - 1) / RPW;
    if (blocks == 0)
        return hipSuccess;
    const int silu = act_silu(a.act);
    if (a.skip_zero)
        return launch(k_gather_up<T, MX, GATED, true>, dim3(blocks, a.B), dim3(256), st, tr,
                      static_cast<const u32x4 *>(a.x), static_cast<const u32x4 *>(a.W1),
                      static_cast<const u32x4 *>(a.Wup), a.b1, a.idx, a.idx_stride, a.count,
                      a.max_count, a.f, C, a.h, a.h_stride, silu, a.gate_tau);
    return launch(k_gather_up<T, MX, GATED>, dim3(blocks, a.B), dim3(256), st, tr,
                  static_cast<const u32x4 *>(a.x), static_cast<const u32x4 *>(a.W1),
                  static_cast<const u32x4 *>(a.Wup), a.b1, a.idx, a.idx_stride, a.count,
                  a.max_count, a.f, C, a.h, a.h_stride, silu, 0.0f);
}

template <class T, bool GATED>
hipError_t up_gated(const FfnArgs &a, int C, hipStream_t st, Trace *tr)
{
    const int mx = (C + 255) / 256;
    if (mx <= 1) return up_launch<T, 1, GATED>(a, C, st, tr);
    if (mx <= 2) return up_launch<T, 2, GATED>(a, C, st, tr);
    if (mx <= 4) return up_launch<T, 4, GATED>(a, C, st, tr);
    if (mx <= 6) return up_launch<T, 6, GATED>(a, C, st, tr);
    if (mx <= 8) return up_launch<T, 8, GATED>(a, C, st, tr);
    if (mx <= 12) return up_launch<T, 12, GATED>(a, C, st, tr);
    if (mx <= 16) return up_launch<T, 16, GATED>(a, C, st, tr);
    return hipErrorInvalidValue;
}

template <class T>
hipError_t down_t(const FfnArgs &a, hipStream_t st, Trace *tr)
{
    const int C = a.d / T::E;
    const int nchunk = ffn_num_chunks(a.d, a.dtype, a.max_count);
    hipError_t e = launch(k_gather_down<T>, dim3(ffn_num_slices(a.d, a.dtype), nchunk, a.B),
                          dim3(256), st, tr, static_cast<const u32x4 *>(a.W2T), a.h, a.h_stride,
                          a.idx, a.idx_stride, a.count, a.max_count, a.f, C, nchunk, a.skip_zero,
                          a.partials);
    if (e != hipSuccess)
        return e;
    return launch_reduce_partials(a.partials, nchunk, a.d, a.B, a.y, st, tr, a.accumulate);
}

template <class T>
hipError_t ffn_t(const FfnArgs &a, hipStream_t st, Trace *tr)
{
    const int C = a.d / T::E;
    hipError_t e = act_gated(a.act) ? up_gated<T, true>(a, C, st, tr) : up_gated<T, false>(a, C, st, tr);
    if (e != hipSuccess)
        return e;
    const int nchunk = ffn_num_chunks(a.d, a.dtype, a.max_count);
    e = launch(k_gather_down<T>, dim3(ffn_num_slices(a.d, a.dtype), nchunk, a.B), dim3(256), st,
               tr, static_cast<const u32x4 *>(a.W2T), a.h, a.h_stride, a.idx, a.idx_stride, a.count,
               a.max_count, a.f, C, nchunk, a.skip_zero, a.partials);
    if (e != hipSuccess)
        return e;
    return launch_reduce_partials(a.partials, nchunk, a.d, a.B, a.y, st, tr, a.accumulate);
}

}  // namespace

int ffn_max_count() { return kMaxChunks * kMaxChunkRows; }

int ffn_num_slices(int d, int dtype)
{
    const int C = d / (dtype == 0 ? 4 : 8);
    return (C + kSliceChunks - 1) / kSliceChunks;
}

int ffn_num_chunks(int d, int dtype, int max_count)
{
    // about 768 workgroups per token in the down projection, at least 16 list entries per chunk
    // (measured at the OPT-175B shape: 768 is 0.5 us faster per layer than 1536, whose partial
    // rows the reduction then reads twice over; 576 and 384 are slower again).  The split depends
    // on neither the batch size nor the data, so a token's summation order (and its bits) are the
    // same in every batch.
    const int slices = ffn_num_slices(d, dtype);
    int want = (768 + slices - 1) / slices;
    const int cap = max_count / 16;
    if (want > cap)
        want = cap;
    if (want > kMaxChunks)
        want = kMaxChunks;
    // a chunk holds at most kMaxChunkRows list entries
    const int least = (max_count + kMaxChunkRows - 1) / kMaxChunkRows;
    if (want < least)
        want = least;
    if (want < 1)
        want = 1;
    return want;
}

hipError_t launch_reduce_partials(const float *part, int nchunk, int D, int B, float *y,
                                  hipStream_t st, Trace *tr, int accumulate)
{
    if (nchunk < 1 || nchunk > kMaxChunks)
        return hipErrorInvalidValue;
    return launch(k_reduce_partials, dim3((D + kWave - 1) / kWave, B), dim3(256), st, tr, part, nchunk,
                  D, y, accumulate);
}

hipError_t launch_ffn_down(const FfnArgs &a, hipStream_t st, Trace *tr)
{
    if (a.dtype == 0) return down_t<F32T>(a, st, tr);
    if (a.dtype == 1) return down_t<F16T>(a, st, tr);
    return down_t<BF16T>(a, st, tr);
}

int ffn_fused_sync_words() { return (kMaxChunks + 1) * kLineWords; }

hipError_t launch_ffn_fused(const FfnArgs &a, uint32_t *sync, hipStream_t st, Trace *tr)
{
    if (a.B != 1 || a.skip_zero)
        return hipErrorInvalidValue;
    if (a.max_count == 0)   // an empty list still writes y = 0 (or leaves y for accumulate)
        return launch_ffn(a, st, tr);
    if (a.dtype == 0) return fused_t<F32T>(a, sync, st, tr);
    if (a.dtype == 1) return fused_t<F16T>(a, sync, st, tr);
    return fused_t<BF16T>(a, sync, st, tr);
}

hipError_t launch_ffn(const FfnArgs &a, hipStream_t st, Trace *tr)
{
    if (a.dtype == 0) return ffn_t<F32T>(a, st, tr);
    if (a.dtype == 1) return ffn_t<F16T>(a, st, tr);
    return ffn_t<BF16T>(a, st, tr);
}

}  // namespace csf
