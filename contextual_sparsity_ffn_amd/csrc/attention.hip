// attention.hip -- attention-head sparsity on gfx950: one decode step of multi-head attention
// computed for a set of heads only.
//
// "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm": the opening
// section (for a given input a small set of attention heads, with the MLP neurons, approximates
// the dense layer), "The Empirical Foundation" (a fifth to a third of the heads matter per token),
// "Implications for System Design" (choosing heads per token saves attention work and, above
// all, key/value cache traffic and memory).
//
// For each listed head h and the new token x:
//   q = Wq_h x + bq_h,  k = Wk_h x + bk_h,  v = Wv_h x + bv_h   (rows h*dh .. h*dh+dh-1)
//   k, v rounded to the cache's storage type and written at the head's next position len[h];
//   a_t = q . K_h[t] / sqrt(dh) over t = 0 .. len[h] (the new token included), p = softmax(a),
//   o_h = sum_t p_t V_h[t];   y = sum over the listed heads of WoT[h*dh + i] * o_h[i].
//
// Kernels (each bound by HBM reads of weight rows or cached keys and values):
//   k_head_proj     whole projection rows in 16-byte chunks, RPW rows per 256-thread workgroup,
//                   x held in registers (the gathered-row pattern of the FFN's up projection);
//   k_head_attn     one workgroup per (listed head, block of 128 cached positions): a group of
//                   dh*es/16 lanes reads one cached row per 16-byte load, so a wavefront reads
//                   whole 128-byte lines; the block's softmax numerator and partial o are kept
//                   with the block maximum (the flash-decoding split);
//   k_head_combine  one workgroup per listed head merges the blocks in a fixed order
//                   (deterministic), turns o_h into the list of output-projection rows and their
//                   weights, and advances the cache lengths;
//   then the FFN's neuron-major down projection (k_gather_down + k_reduce_partials) reads the
//   rows of WoT of the listed heads.
#include "common.hpp"
#include "launch.hpp"

namespace csf {

namespace {

constexpr int kAttnChunk = 128;   // cached positions per attention workgroup
constexpr int kMaxAttnSplits = 1024;   // blocks per head: caches of up to 131072 positions

template <class T>
__device__ __forceinline__ void store_cache(void *base, size_t i, float v)
{
    if constexpr (T::E == 4)
        static_cast<float *>(base)[i] = v;
    else
        static_cast<uint16_t *>(base)[i] = T::round_bits(v);
}

// Head of list entry n, or -1 when the entry is past the count, outside [0, H) or its cache is
// full (such a head is skipped everywhere).
__device__ __forceinline__ int list_head(const int32_t *heads, const int32_t *count, int max_heads,
                                         int n, int H, const int32_t *len, int Tmax)
{
    int cnt = count ? *count : max_heads;
    cnt = cnt < 0 ? 0 : (cnt > max_heads ? max_heads : cnt);
    if (n >= cnt)
        return -1;
    const int h = heads ? heads[n] : n;
    if (h < 0 || h >= H)
        return -1;
    const int L = len[h];
    return (L >= 0 && L < Tmax) ? h : -1;
}

// Projection rows.  Row r of the launch: list entry n = r / (np*dh), projection number p, head
// dimension i; proj says which projections the launch computes (1 = q only, 6 = k and v,
// 7 = q, k and v) and np how many.  q rows go to qbuf[n][i] (float32), k and v rows to the
// cache position len[h] of their head.
template <class T, int MX, int RPW>
__global__ __launch_bounds__(256) void k_head_proj(const u32x4 *__restrict__ x,
                                                   const u32x4 *__restrict__ Wq,
                                                   const u32x4 *__restrict__ Wk,
                                                   const u32x4 *__restrict__ Wv,
                                                   const float *__restrict__ bq,
                                                   const float *__restrict__ bk,
                                                   const float *__restrict__ bv,
                                                   const int32_t *__restrict__ heads,
                                                   const int32_t *__restrict__ count,
                                                   int max_heads, int H, int dh, int C, int proj,
                                                   int np, float *__restrict__ qbuf,
                                                   void *__restrict__ Kc, void *__restrict__ Vc,
                                                   int Tmax, const int32_t *__restrict__ len)
{
    __shared__ float red[4][RPW];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int per_entry = np * dh;
    const int r0 = blockIdx.x * RPW;
    if (r0 >= max_heads * per_entry)
        return;

    // matrix (0 q, 1 k, 2 v), head, dimension and list entry of each row; mat = -1: skipped
    int mat[RPW], hh[RPW], dim[RPW], ent[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = r0 + i;
        const int n = r / per_entry, rem = r % per_entry;
        const int p = rem / dh;
        ent[i] = n;
        dim[i] = rem % dh;
        hh[i] = r < max_heads * per_entry ? list_head(heads, count, max_heads, n, H, len, Tmax) : -1;
        mat[i] = hh[i] < 0 ? -1 : (proj == 6 ? p + 1 : p);
    }
    bool any = false;
#pragma unroll
    for (int i = 0; i < RPW; ++i)
        any |= mat[i] >= 0;
    if (!any)
        return;                                     // uniform across the workgroup

    u32x4 xv[MX];
#pragma unroll
    for (int m = 0; m < MX; ++m) {
        const int c = t + 256 * m;
        xv[m] = c < C ? x[c] : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 wv[RPW][MX];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const u32x4 *W = mat[i] == 2 ? Wv : (mat[i] == 1 ? Wk : Wq);
        const u32x4 *row = W + (size_t)(mat[i] < 0 ? 0 : hh[i] * dh + dim[i]) * C;
#pragma unroll
        for (int m = 0; m < MX; ++m) {
            const int c = t + 256 * m;
            wv[i][m] = (mat[i] >= 0 && c < C) ? ld_stream(row + c) : u32x4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int m = 0; m < MX; ++m)
            acc = T::dot(wv[i][m], xv[m], acc);
        acc = wave_sum(acc);
        if (lane == 0)
            red[w][i] = acc;
    }
    __syncthreads();
    if (t < RPW && mat[t] >= 0) {
        const int i = t;
        float v = (red[0][i] + red[1][i]) + (red[2][i] + red[3][i]);
        const size_t row = (size_t)hh[i] * dh + dim[i];
        const float *b = mat[i] == 2 ? bv : (mat[i] == 1 ? bk : bq);
        if (b)
            v += b[row];
        if (mat[i] == 0) {
            qbuf[(size_t)ent[i] * dh + dim[i]] = v;
        } else {
            const size_t pos = ((size_t)hh[i] * Tmax + len[hh[i]]) * dh + dim[i];
            store_cache<T>(mat[i] == 1 ? Kc : Vc, pos, v);
        }
    }
}

// One block of kAttnChunk cached positions of one listed head: part = {m, l, o[dh]} with
// m = max of the block's logits, l = sum of exp(a_t - m), o = sum of exp(a_t - m) V[t].
// LPP = lanes per cached row (dh * element size / 16), PPW = rows per wavefront load.
template <class T, int LPP>
__global__ __launch_bounds__(256) void k_head_attn(const float *__restrict__ qbuf,
                                                   const u32x4 *__restrict__ Kc,
                                                   const u32x4 *__restrict__ Vc,
                                                   const int32_t *__restrict__ heads,
                                                   const int32_t *__restrict__ count,
                                                   int max_heads, int H, int dh, int Tmax,
                                                   const int32_t *__restrict__ len, int nsplit,
                                                   float scale, float *__restrict__ part,
                                                   int32_t *__restrict__ lnew)
{
    constexpr int E = T::E;
    constexpr int PPW = kWave / LPP;            // cached rows per wavefront load
    constexpr int PPI = 4 * PPW;                // rows per workgroup step
    constexpr int IT = kAttnChunk / PPI;        // steps per block
    static_assert(IT >= 1 && IT * PPI == kAttnChunk, "block of positions must be whole steps");
    __shared__ float sc[kAttnChunk];
    __shared__ float ored[PPI][LPP * E];
    __shared__ float wred[4];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int g = lane / LPP, li = lane % LPP;
    const int n = blockIdx.x, s = blockIdx.y;
    const int h = list_head(heads, count, max_heads, n, H, len, Tmax);
    if (s == 0 && t == 0)
        lnew[n] = h < 0 ? -1 : len[h] + 1;      // for the combine kernel, which advances len
    if (h < 0)
        return;
    const int L = len[h] + 1;                   // the new token was appended at len[h]
    const int p0 = s * kAttnChunk;
    if (p0 >= L)
        return;
    const int p1 = p0 + kAttnChunk < L ? p0 + kAttnChunk : L;
    const size_t hrow = (size_t)h * Tmax;

    float qv[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        qv[e] = qbuf[(size_t)n * dh + li * E + e];

    // every key and value load of the block is issued before the first use
    u32x4 kv[IT], vv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int pos = p0 + it * PPI + w * PPW + g;
        kv[it] = pos < p1 ? Kc[(hrow + pos) * LPP + li] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int pos = p0 + it * PPI + w * PPW + g;
        vv[it] = pos < p1 ? Vc[(hrow + pos) * LPP + li] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        float kf[E];
        T::unpack(kv[it], kf);
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e)
            a = fmaf(qv[e], kf[e], a);
        a = group_sum<LPP>(a);
        const int loc = it * PPI + w * PPW + g;
        if (li == 0)
            sc[loc] = p0 + loc < p1 ? a * scale : -INFINITY;
    }
    __syncthreads();

    // block maximum and softmax numerators (fixed-order reductions)
    float mv = t < kAttnChunk ? sc[t] : -INFINITY;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        mv = fmaxf(mv, __shfl_xor(mv, o, kWave));
    if (lane == 0)
        wred[w] = mv;
    __syncthreads();
    const float m = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
    __syncthreads();
    float ev = 0.0f;
    if (t < kAttnChunk) {
        ev = p0 + t < p1 ? expf(sc[t] - m) : 0.0f;
        sc[t] = ev;
    }
    ev = wave_sum(ev);
    if (lane == 0)
        wred[w] = ev;
    __syncthreads();
    const float l = (wred[0] + wred[1]) + (wred[2] + wred[3]);

    // o = sum_t e_t V[t]: each lane group accumulates its rows, then the groups are summed
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        acc[e] = 0.0f;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const float pe = sc[it * PPI + w * PPW + g];
        float vf[E];
        T::unpack(vv[it], vf);
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[e] = fmaf(pe, vf[e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        ored[w * PPW + g][li * E + e] = acc[e];
    __syncthreads();
    float *out = part + ((size_t)n * nsplit + s) * (dh + 2);
    for (int i = t; i < dh; i += 256) {
        float sum = 0.0f;
        for (int q = 0; q < PPI; ++q)
            sum += ored[q][i];
        out[2 + i] = sum;
    }
    if (t == 0) {
        out[0] = m;
        out[1] = l;
    }
}

// One workgroup per list entry: merge the blocks of the head into o_h (block weights
// w_s = exp(m_s - M), M the largest block maximum; o_h = sum_s w_s o_s / sum_s w_s l_s, every sum
// in a fixed order), write the output projection's row list (rows h*dh + i with weights o_h[i];
// -1 for a skipped entry) and the optional copy of o.  Workgroup 0 also writes the row count and
// advances the cache lengths; no workgroup of this kernel reads len, so the update cannot race
// (the attention lengths come from lnew).  The G = 256 / dh thread groups take every G-th block.
__global__ __launch_bounds__(256) void k_head_combine(const float *__restrict__ part,
                                                      const int32_t *__restrict__ heads,
                                                      const int32_t *__restrict__ count,
                                                      int max_heads, int H, int dh, int Tmax,
                                                      const int32_t *__restrict__ lnew,
                                                      int32_t *__restrict__ len, int kv_all,
                                                      int nsplit, int32_t *__restrict__ rows,
                                                      float *__restrict__ hv,
                                                      int32_t *__restrict__ rows_count,
                                                      float *__restrict__ o_out)
{
    __shared__ float sw[kMaxAttnSplits];
    __shared__ float red[4];
    __shared__ float osum[256];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int n = blockIdx.x;
    int cnt = count ? *count : max_heads;
    cnt = cnt < 0 ? 0 : (cnt > max_heads ? max_heads : cnt);
    const int L = n < cnt ? lnew[n] : -1;
    const int h = L > 0 ? (heads ? heads[n] : n) : -1;
    if (h < 0) {
        for (int i = t; i < dh; i += 256) {
            rows[(size_t)n * dh + i] = -1;
            hv[(size_t)n * dh + i] = 0.0f;
            if (o_out)
                o_out[(size_t)n * dh + i] = 0.0f;
        }
    } else {
        const int ns = (L + kAttnChunk - 1) / kAttnChunk;
        const int stride = dh + 2;
        const float *pp = part + (size_t)n * nsplit * stride;
        // M: every block maximum loaded at once (thread t owns blocks t, t + 256, ...)
        float mv = -INFINITY;
        for (int s = t; s < ns; s += 256)
            mv = fmaxf(mv, pp[(size_t)s * stride]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            mv = fmaxf(mv, __shfl_xor(mv, o, kWave));
        if (lane == 0)
            red[w] = mv;
        __syncthreads();
        const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        float lv = 0.0f;
        for (int s = t; s < ns; s += 256) {
            const float ws = expf(pp[(size_t)s * stride] - M);
            sw[s] = ws;
            lv += ws * pp[(size_t)s * stride + 1];
        }
        lv = wave_sum(lv);
        if (lane == 0)
            red[w] = lv;
        __syncthreads();
        const float inv = 1.0f / ((red[0] + red[1]) + (red[2] + red[3]));
        // o: thread t takes dimension t % dh over blocks t / dh, t / dh + G, ... (four loads in
        // flight per step)
        const int G = 256 / dh;
        const int i = t % dh, g = t / dh;
        float acc = 0.0f;
        if (g < G) {
            int s = g;
            for (; s + 3 * G < ns; s += 4 * G) {
                const float a0 = pp[(size_t)s * stride + 2 + i];
                const float a1 = pp[(size_t)(s + G) * stride + 2 + i];
                const float a2 = pp[(size_t)(s + 2 * G) * stride + 2 + i];
                const float a3 = pp[(size_t)(s + 3 * G) * stride + 2 + i];
                acc = fmaf(sw[s], a0, acc);
                acc = fmaf(sw[s + G], a1, acc);
                acc = fmaf(sw[s + 2 * G], a2, acc);
                acc = fmaf(sw[s + 3 * G], a3, acc);
            }
            for (; s < ns; s += G)
                acc = fmaf(sw[s], pp[(size_t)s * stride + 2 + i], acc);
        }
        osum[t] = acc;
        __syncthreads();
        if (t < dh) {
            float o = 0.0f;
            for (int q = 0; q < G; ++q)
                o += osum[q * dh + t];
            o *= inv;
            rows[(size_t)n * dh + t] = h * dh + t;
            hv[(size_t)n * dh + t] = o;
            if (o_out)
                o_out[(size_t)n * dh + t] = o;
        }
    }
    if (n == 0) {
        if (t == 0)
            *rows_count = cnt * dh;
        if (kv_all) {
            for (int q = t; q < H; q += 256)
                if (len[q] >= 0 && len[q] < Tmax)
                    len[q] += 1;
        } else {
            for (int q = t; q < cnt; q += 256)
                if (lnew[q] > 0)
                    len[heads ? heads[q] : q] = lnew[q];
        }
    }
}

template <class T, int MX>
hipError_t proj_launch(const AttnArgs &a, const int32_t *heads, const int32_t *count, int nlist,
                       int proj, hipStream_t st, Trace *tr)
{
    constexpr int loads = MX;
    constexpr int RPW = loads >= 12 ? 1 : (loads >= 6 ? 2 : 4);
    const int np = proj == 7 ? 3 : (proj == 6 ? 2 : 1);
    const int rows = nlist * np * a.dh;
    const int blocks = (rows + RPW - 1) / RPW;
    if (blocks == 0)
        return hipSuccess;
    return launch(k_head_proj<T, MX, RPW>, dim3(blocks), dim3(256), st, tr,
                  static_cast<const u32x4 *>(a.x), static_cast<const u32x4 *>(a.Wq),
                  static_cast<const u32x4 *>(a.Wk), static_cast<const u32x4 *>(a.Wv), a.bq, a.bk,
                  a.bv, heads, count, nlist, a.H, a.dh, a.d / T::E, proj, np, a.qbuf, a.Kc, a.Vc,
                  a.Tmax, a.len);
}

template <class T>
hipError_t proj_t(const AttnArgs &a, const int32_t *heads, const int32_t *count, int nlist,
                  int proj, hipStream_t st, Trace *tr)
{
    const int mx = (a.d / T::E + 255) / 256;
    if (mx <= 1) return proj_launch<T, 1>(a, heads, count, nlist, proj, st, tr);
    if (mx <= 2) return proj_launch<T, 2>(a, heads, count, nlist, proj, st, tr);
    if (mx <= 4) return proj_launch<T, 4>(a, heads, count, nlist, proj, st, tr);
    if (mx <= 6) return proj_launch<T, 6>(a, heads, count, nlist, proj, st, tr);
    if (mx <= 8) return proj_launch<T, 8>(a, heads, count, nlist, proj, st, tr);
    if (mx <= 12) return proj_launch<T, 12>(a, heads, count, nlist, proj, st, tr);
    if (mx <= 16) return proj_launch<T, 16>(a, heads, count, nlist, proj, st, tr);
    return hipErrorInvalidValue;
}

template <class T, int LPP>
hipError_t attn_launch(const AttnArgs &a, hipStream_t st, Trace *tr)
{
    const int nsplit = attn_num_splits(a.Tmax);
    return launch(k_head_attn<T, LPP>, dim3(a.max_heads, nsplit), dim3(256), st, tr, a.qbuf,
                  static_cast<const u32x4 *>(a.Kc), static_cast<const u32x4 *>(a.Vc), a.heads,
                  a.count, a.max_heads, a.H, a.dh, a.Tmax, a.len, nsplit,
                  1.0f / sqrtf((float)a.dh), a.part, a.lnew);
}

template <class T>
hipError_t attn_t(const AttnArgs &a, hipStream_t st, Trace *tr)
{
    const int lpp = a.dh * (16 / T::E) / 16;
    switch (lpp) {
    case 2: return attn_launch<T, 2>(a, st, tr);
    case 4: return attn_launch<T, 4>(a, st, tr);
    case 8: return attn_launch<T, 8>(a, st, tr);
    case 16: return attn_launch<T, 16>(a, st, tr);
    case 32: return attn_launch<T, 32>(a, st, tr);
    default: return hipErrorInvalidValue;
    }
}

template <class T>
hipError_t decode_t(const AttnArgs &a, hipStream_t st, Trace *tr)
{
    hipError_t e;
    if (a.kv_all) {
        e = proj_t<T>(a, a.heads, a.count, a.max_heads, 1, st, tr);              // q of the list
        if (e == hipSuccess)
            e = proj_t<T>(a, nullptr, nullptr, a.H, 6, st, tr);               // k, v of every head
    } else {
        e = proj_t<T>(a, a.heads, a.count, a.max_heads, 7, st, tr);
    }
    if (e != hipSuccess)
        return e;
    if (a.max_heads > 0) {
        e = attn_t<T>(a, st, tr);
        if (e != hipSuccess)
            return e;
    }
    e = launch(k_head_combine, dim3(a.max_heads > 0 ? a.max_heads : 1), dim3(256), st, tr,
               a.part, a.heads, a.count, a.max_heads, a.H, a.dh, a.Tmax, a.lnew, a.len, a.kv_all,
               attn_num_splits(a.Tmax), a.rows, a.hv, a.rows_count, a.o);
    if (e != hipSuccess)
        return e;
    FfnArgs f;
    f.dtype = a.dtype;
    f.act = 0;
    f.x = nullptr;
    f.B = 1;
    f.d = a.d;
    f.f = a.H * a.dh;
    f.W1 = nullptr;
    f.Wup = nullptr;
    f.W2T = a.WoT;
    f.b1 = nullptr;
    f.idx = a.rows;
    f.idx_stride = a.max_heads * a.dh;
    f.count = a.rows_count;
    f.max_count = a.max_heads * a.dh;
    f.h = a.hv;
    f.h_stride = a.max_heads * a.dh;
    f.y = a.y;
    f.partials = a.ffn_partials;
    return launch_ffn_down(f, st, tr);
}

}  // namespace

int attn_num_splits(int Tmax) { return (Tmax + kAttnChunk - 1) / kAttnChunk; }

int attn_max_cache() { return kMaxAttnSplits * kAttnChunk; }

bool attn_head_dim_supported(int dtype, int dh)
{
    const int es = dtype == 0 ? 4 : 2;
    if (dh <= 0 || (dh * es) % 16 != 0)
        return false;
    const int lpp = dh * es / 16;
    return lpp == 2 || lpp == 4 || lpp == 8 || lpp == 16 || lpp == 32;
}

hipError_t launch_attention_decode(const AttnArgs &a, hipStream_t st, Trace *tr)
{
    if (a.dtype == 0) return decode_t<F32T>(a, st, tr);
    if (a.dtype == 1) return decode_t<F16T>(a, st, tr);
    return decode_t<BF16T>(a, st, tr);
}

}  // namespace csf
