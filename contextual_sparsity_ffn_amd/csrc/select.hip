// select.hip -- active-set selection on gfx950: exact top-k and threshold compaction.
//
// Top-k: "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm", section
// "The Prediction Problem" -- the k largest predictor scores are the active set.  Among equal
// scores the lower neuron index wins; -0.0 equals +0.0; the list is written in ascending order.
// Threshold: "Activation sparsity", section "Implementation sketch" -- active = scores >= threshold.
//
// Top-k runs as a bucket select.  Every score falls in one of kScoreBuckets buckets by a monotone
// map of its value (uniform over [0, 1], the range of a sigmoid score; values outside clamp), so
// all neurons in buckets above the bucket B* that holds the k-th score are selected, all below are
// not, and only the candidates inside B* need ranking.  One 1024-thread workgroup per token holds
// the scores in registers -- thread t takes scores 4t..4t+3 of every sweep of 4096, one coalesced
// 16-byte load each, all issued before any is used -- and:
//   1. builds the bucket histogram in LDS and finds B* and `need` (how many of B*'s candidates to
//      take) with one block scan of the histogram, top bucket first;
//   2. classifies its scores into 4-bit nibbles, ORs the nibbles of 8 neighbouring lanes into a
//      bitmap word (lane shuffles, then one LDS store; no ballots or branches, so the CU's single
//      scalar unit, shared by all 16 wavefronts, stays out of the loop); candidates go to an LDS
//      list;
//   3. ranks the candidates by (score desc, index asc) -- a direct count when there are at most
//      kMaxDirect of them, else a radix select over the bucket's 32-bit order keys with an
//      index-ordered pass for exact ties -- and sets their bits;
//   4. compacts the bitmap into the ascending index list (popcounts + one block scan).
#include "common.hpp"
#include "launch.hpp"

namespace csf {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kQuad = 4 * kSelThreads;     // scores per sweep: four consecutive per thread
constexpr int kMaxWords = 2048;            // bitmap words held in LDS: f <= 65536
constexpr int kMaxDirect = 512;            // candidates ranked by direct counting


// Four consecutive scores j0..j0+3 of one row; positions past f read as NaN (callers test the
// position, since a score may itself be NaN).  VEC: the row is 16-byte aligned (f % 4 == 0), so a
// full quad is one 16-byte load.
template <bool VEC>
__device__ __forceinline__ float4 load_quad(const float *s, int j0, int f)
{
    const float nan = __builtin_nanf("");
    if (VEC && j0 + 3 < f)
        return *reinterpret_cast<const float4 *>(s + j0);
    float4 q;
    q.x = j0 < f ? s[j0] : nan;
    q.y = j0 + 1 < f ? s[j0 + 1] : nan;
    q.z = j0 + 2 < f ? s[j0 + 2] : nan;
    q.w = j0 + 3 < f ? s[j0 + 3] : nan;
    return q;
}

// Lane l holds a 4-bit nibble for scores 4l..4l+3 of a 256-score block; OR it across each group of
// 8 lanes into the block's 32-bit words and store word l/8 from the group's first lane.  Other
// lanes store into a per-lane trash slot, so no branch (and no scalar work) is needed.
__device__ __forceinline__ void store_nibbles(uint32_t nib, uint32_t *bm, int word0, int words,
                                              uint32_t *trash)
{
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t x = nib << (4 * (lane & 7));
    x |= __shfl_xor(x, 1, kWave);
    x |= __shfl_xor(x, 2, kWave);
    x |= __shfl_xor(x, 4, kWave);
    const int widx = word0 + (lane >> 3);
    uint32_t *dst = ((lane & 7) == 0 && widx < words) ? &bm[widx] : &trash[threadIdx.x];
    *dst = x;
}

// Add one to rhist[dig] for every lane with `hit`.  When all the wavefront's hitting lanes share
// a digit (equal scores, the case this serves), one lane adds their count: the lanes would
// otherwise serialize on one LDS word.
__device__ __forceinline__ void add_digit(uint32_t *rhist, bool hit, uint32_t dig)
{
    if (hit) {
        const uint64_t act = __ballot(1);                       // the hitting lanes
        const uint32_t d0 = __builtin_amdgcn_readfirstlane(dig);
        if (__ballot(dig == d0) == act) {
            const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                (uint32_t)(act >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)act, 0u));
            if (below == 0)
                atomicAdd(&rhist[d0], (uint32_t)__popcll(act));
        } else {
            atomicAdd(&rhist[dig], 1u);
        }
    }
}

// Compaction of an LDS bitmap into the ascending index list (index + base); also copies the bitmap
// out.
__device__ void bitmap_to_list(const uint32_t *bm, int words, int32_t *out, int out_cap, int base,
                               uint32_t *bitmap_out, uint32_t *scan_tmp, uint32_t *total_out)
{
    const int t = threadIdx.x;
    const int wpt = (words + kSelThreads - 1) / kSelThreads;   // <= 2 for f <= 65536
    const int w0 = t * wpt;
    uint32_t n = 0;
    for (int q = 0; q < wpt; ++q)
        if (w0 + q < words)
            n += __popc(bm[w0 + q]);
    uint32_t total;
    uint32_t pos = block_exclusive_scan<kSelWaves>(n, scan_tmp, &total);
    if (total_out)
        *total_out = total;
    for (int q = 0; q < wpt; ++q) {
        const int w = w0 + q;
        if (w >= words)
            break;
        uint32_t bits = bm[w];
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            if (pos < (uint32_t)out_cap)
                out[pos] = base + w * 32 + b;
            ++pos;
        }
    }
    if (bitmap_out)
        for (int w = t; w < words; w += kSelThreads)
            bitmap_out[w] = bm[w];
}

// The whole selection of one token by one 1024-thread workgroup (steps 1-4 above).  ghist
// (optional): the token's finished bucket histogram, which step 1 then reads instead of counting.
template <int NB, int J, bool VEC>
__device__ __forceinline__ void topk_one_workgroup(const float *__restrict__ scores, int token,
                                                   int f, int k, int32_t *__restrict__ idx,
                                                   int idx_stride, int32_t *__restrict__ count,
                                                   uint32_t *__restrict__ bitmap, int prefix,
                                                   const uint32_t *__restrict__ ghist = nullptr)
{
    __shared__ uint32_t hist[NB];
    __shared__ uint32_t bm[kMaxWords];
    __shared__ uint32_t trash[kSelThreads];
    __shared__ uint64_t cand[kMaxDirect];
    __shared__ uint32_t scan_tmp[kSelWaves];
    __shared__ uint32_t rhist[256];
    __shared__ uint32_t misc[8];   // 0: B*, 1: need, 2: candidate count, 3: digit, 4: krem

    const int t = threadIdx.x;
    if (t == 0) {
        misc[0] = 0u;
        misc[1] = 0u;
    }
    const float *s = scores + (size_t)token * f;
    const int words = (f + 31) / 32;
    int32_t *out = idx + (size_t)token * idx_stride;
    uint32_t *bm_out = bitmap ? bitmap + (size_t)token * words : nullptr;

    // a leading block of `prefix` neurons always belongs to the list (they are not scored)
    for (int i = t; i < prefix; i += kSelThreads)
        out[i] = i;
    if (t == 0) {
        misc[2] = 0u;
        if (count)
            count[token] = prefix + k;
    }
    if (k == 0) {                                     // uniform: nothing is selected
        if (bm_out)
            for (int q = t; q < words; q += kSelThreads)
                bm_out[q] = 0u;
        return;
    }

    // scores 4t..4t+3 of each sweep of 4096, held in registers; every load is issued first
    float4 v[J];
#pragma unroll
    for (int i = 0; i < J; ++i)
        v[i] = load_quad<VEC>(s, i * kQuad + 4 * t, f);

    // ---- 1. the bucket histogram and the boundary bucket B* ------------------------------------
    if (ghist) {
        for (int b = t; b < NB; b += kSelThreads)
            hist[b] = ghist[b];
    } else {
        for (int b = t; b < NB; b += kSelThreads)
            hist[b] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < J; ++i) {
            const float e[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (i * kQuad + 4 * t + q < f)
                    atomicAdd(&hist[score_bucket<NB>(e[q])], 1u);
        }
    }
    __syncthreads();

    // thread t owns buckets NB-1-BPT*t-q, q < BPT (thread 0 holds the top buckets)
    constexpr int BPT = NB / kSelThreads;
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q)
        mine += hist[NB - 1 - (BPT * t + q)];
    uint32_t total;
    uint32_t above = block_exclusive_scan<kSelWaves>(mine, scan_tmp, &total);
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        const int b = NB - 1 - (BPT * t + q);
        const uint32_t c = hist[b];
        if (above < (uint32_t)k && above + c >= (uint32_t)k) {
            misc[0] = (uint32_t)b;
            misc[1] = (uint32_t)k - above;
        }
        above += c;
    }
    __syncthreads();
    const int bstar = (int)misc[0];
    const uint32_t need = misc[1];
    const bool direct = hist[bstar] <= (uint32_t)kMaxDirect;

    // ---- 2. certain members into the bitmap, candidates into LDS --------------------------------
#pragma unroll
    for (int i = 0; i < J; ++i) {
        const float e[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t nib = 0u, cmask = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int b = i * kQuad + 4 * t + q < f ? score_bucket<NB>(e[q]) : -1;
            nib |= (b > bstar ? 1u : 0u) << q;
            cmask |= (b == bstar ? 1u : 0u) << q;
        }
        const int j0 = i * kQuad + 4 * t;
        store_nibbles(nib, bm, j0 >> 5 & ~7, words, trash);
        if (direct && cmask) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (cmask & (1u << q)) {
                    const uint32_t p = atomicAdd(&misc[2], 1u);
                    if (p < (uint32_t)kMaxDirect)
                        cand[p] = composite(order_key(e[q]), j0 + q);
                }
            }
        }
    }
    __syncthreads();

    // ---- 3. rank the candidates of bucket B* -------------------------------------------------------
    if (direct) {
        const uint32_t nc = misc[2] < (uint32_t)kMaxDirect ? misc[2] : (uint32_t)kMaxDirect;
        for (uint32_t i = t; i < nc; i += kSelThreads) {
            const uint64_t me = cand[i];
            uint32_t rank = 0;
#pragma unroll 8
            for (uint32_t q = 0; q < nc; ++q)
                rank += cand[q] > me ? 1u : 0u;
            if (rank < need) {
                const int j = (int)(0xffffffffu - (uint32_t)me);
                atomicOr(&bm[j >> 5], 1u << (j & 31));
            }
        }
    } else {
        // many candidates (heavy ties or a concentrated distribution): radix select over the
        // 32-bit order keys of bucket B*, 8 bits per pass.  This rare path re-reads the scores
        // from memory so that the common path keeps its registers.  Shortcut first: when the
        // candidates holding the bucket's largest key are at least `need` (equal scores at the top
        // of the bucket, the usual cause of this path), that key is the k-th and no radix pass is
        // needed.
        uint32_t kmax = 0u, kcnt = 0u;
        for (int j = t; j < f; j += kSelThreads) {
            const float x = s[j];
            if (score_bucket<NB>(x) == bstar) {
                const uint32_t key = order_key(x);
                kcnt = key > kmax ? 1u : kcnt + (key == kmax ? 1u : 0u);
                kmax = key > kmax ? key : kmax;
            }
        }
        uint32_t wmax = kmax;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t other = (uint32_t)__shfl_xor((int)wmax, o, kWave);
            wmax = other > wmax ? other : wmax;
        }
        if ((t & (kWave - 1)) == 0)
            rhist[t / kWave] = wmax;
        __syncthreads();
        uint32_t gmax = 0u;
#pragma unroll
        for (int w2 = 0; w2 < kSelWaves; ++w2)
            gmax = rhist[w2] > gmax ? rhist[w2] : gmax;
        uint32_t at_max;
        // (its barriers also keep the reads of rhist above before a radix pass clears it)
        (void)block_exclusive_scan<kSelWaves>(kmax == gmax ? kcnt : 0u, scan_tmp, &at_max);
        uint32_t kpre = gmax, pmask = 0u, krem = need;
        if (at_max < need) {
            kpre = 0u;
#pragma unroll 1
            for (int shift = 24; shift >= 0; shift -= 8) {
                if (t < 256)
                    rhist[t] = 0u;
                __syncthreads();
                for (int j = t; j < f; j += kSelThreads) {
                    const float x = s[j];
                    const uint32_t key = order_key(x);
                    add_digit(rhist, score_bucket<NB>(x) == bstar && (key & pmask) == kpre,
                              (key >> shift) & 0xffu);
                }
                __syncthreads();
                if (t < kWave) {
                    const uint32_t c0 = rhist[4 * t], c1 = rhist[4 * t + 1];
                    const uint32_t c2 = rhist[4 * t + 2], c3 = rhist[4 * t + 3];
                    const uint32_t local = c0 + c1 + c2 + c3;
                    uint32_t suffix = local;
#pragma unroll
                    for (int o = 1; o < kWave; o <<= 1) {
                        const uint32_t n = __shfl_down(suffix, o, kWave);
                        if (t + o < kWave)
                            suffix += n;
                    }
                    uint32_t ab = suffix - local;
                    const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
                    for (int b = 3; b >= 0; --b) {
                        if (ab < krem && ab + cs[b] >= krem) {
                            misc[3] = (uint32_t)(4 * t + b);
                            misc[4] = krem - ab;
                        }
                        ab += cs[b];
                    }
                }
                __syncthreads();
                kpre |= misc[3] << shift;
                pmask |= 0xffu << shift;
                krem = misc[4];
                __syncthreads();
            }
        }
        // keys above T are in; of the keys equal to T the krem lowest-indexed are in (blocks of
        // 4096 indices in ascending order, four consecutive per thread; a block scan of the
        // threads' equal-key counts ranks them inside each block)
        const uint32_t T = kpre;
        uint32_t taken = 0;
#pragma unroll 1
        for (int base = 0; base < f; base += kQuad) {
            const int j0 = base + 4 * t;
            const float4 xq = load_quad<VEC>(s, j0, f);
            const float e[4] = {xq.x, xq.y, xq.z, xq.w};
            uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (j0 + q < f && score_bucket<NB>(e[q]) == bstar) {
                    const uint32_t key = order_key(e[q]);
                    gtm |= (key > T ? 1u : 0u) << q;
                    eqm |= (key == T ? 1u : 0u) << q;
                }
            }
            uint32_t eq_total;
            uint32_t rank = taken + block_exclusive_scan<kSelWaves>(
                                        (uint32_t)__builtin_popcount(eqm), scan_tmp, &eq_total);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = j0 + q;
                bool in = (gtm >> q) & 1u;
                if ((eqm >> q) & 1u)
                    in = rank++ < krem;
                if (in)
                    atomicOr(&bm[j >> 5], 1u << (j & 31));
            }
            taken += eq_total;
        }
    }
    __syncthreads();

    // ---- 4. ascending list ------------------------------------------------------------------------
    bitmap_to_list(bm, words, out + prefix, idx_stride - prefix, prefix, bm_out, scan_tmp, nullptr);
}

template <int NB, int J, bool VEC>
__global__ __launch_bounds__(kSelThreads) void k_select_topk(const float *__restrict__ scores,
                                                             int f, int k,
                                                             int32_t *__restrict__ idx,
                                                             int idx_stride,
                                                             int32_t *__restrict__ count,
                                                             uint32_t *__restrict__ bitmap,
                                                             int prefix)
{
    topk_one_workgroup<NB, J, VEC>(scores, blockIdx.x, f, k, idx, idx_stride, count, bitmap,
                                   prefix);
}

// ---- top-k over many workgroups (one token, large f) -----------------------------------------
// The same bucket select as topk_one_workgroup, spread over slices of kWideSlice scores so that
// the work of one token runs on many compute units (a single workgroup retires about 64 lane
// operations per cycle, so its passes over 49152 scores cost microseconds each):
//   k_wide_hist      one workgroup per slice: LDS histogram of the slice, added into the token's
//                    histogram with one global atomic per non-empty bucket (zeroed by the launch
//                    before; integer adds, so the order does not matter); the slice is also
//                    counting-sorted by bucket, top bucket first: above[b] (members in buckets
//                    above b) and the members' (order key, index) composites in that order;
//   k_wide_finish    one 1024-thread workgroup per slice, thread t owning score t of the slice:
//                    every workgroup scans the finished histogram and finds the same boundary
//                    bucket B* and `need`; two words of each slice's above[] give the slice's
//                    certain members (bucket above B*) and the place of its B* members, which
//                    are gathered from the sorted composites into LDS and ranked by (score desc,
//                    index asc); the first `need` are kept.  The slice's output offset is the
//                    certain members of the earlier slices plus the kept candidates below the
//                    slice; a block scan places the slice's indices (ascending).  With more than
//                    kWideMaxCand candidates (heavy ties) workgroup 0 runs topk_one_workgroup
//                    instead and the others exit.
// Everything is integer arithmetic on the same bucket map and order keys (a NaN score sits in
// bucket 0 with the lowest key), so the list equals the one-workgroup result bit for bit.
constexpr int kWideSlice = 1024;
constexpr int kWideMaxCand = 512;
// Workspace of one token (32-bit words): the histogram [NB], then per slice above[NB + 1]
// (above[b + 1] for b = -1 .. NB-1), one pad word and the sorted composites [kWideSlice] (64-bit).
constexpr int kWideAbove = kScoreBuckets + 2;
constexpr int kWideSliceWords = kWideAbove + 2 * kWideSlice;

__device__ __forceinline__ uint32_t *wide_slice(uint32_t *W, int slice)
{
    return W + kScoreBuckets + (size_t)slice * kWideSliceWords;
}

template <int NB, bool VEC>
__global__ __launch_bounds__(256) void k_wide_hist(const float *__restrict__ scores, int f,
                                                   uint32_t *__restrict__ ws, int ws_stride)
{
    static_assert(NB == kScoreBuckets && NB % 256 == 0, "workspace layout");
    constexpr int BPT = NB / 256;
    __shared__ uint32_t hist[NB];
    __shared__ uint32_t start[NB];
    __shared__ uint32_t scan_tmp[4];
    const int t = threadIdx.x;
    const int token = blockIdx.y, slice = blockIdx.x;
    const float *s = scores + (size_t)token * f;
    uint32_t *W = ws + (size_t)token * ws_stride;
    uint32_t *above = wide_slice(W, slice);
    uint64_t *keys = reinterpret_cast<uint64_t *>(above + kWideAbove);
    const int j0 = slice * kWideSlice + 4 * t;
    const float4 q = load_quad<VEC>(s, j0, f);
    for (int b = t; b < NB; b += 256)
        hist[b] = 0u;
    __syncthreads();
    const float e[4] = {q.x, q.y, q.z, q.w};
    int bk[4];
    uint32_t rk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bk[i] = j0 + i < f ? score_bucket<NB>(e[i]) : -1;        // -1: past f
        rk[i] = bk[i] >= 0 ? atomicAdd(&hist[bk[i]], 1u) : 0u;  // place inside the bucket
    }
    __syncthreads();
    // thread t owns buckets NB-1-(BPT*t+i), top first; the scan gives the members above each
    uint32_t c[BPT];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        c[i] = hist[NB - 1 - (BPT * t + i)];
        sum += c[i];
    }
    uint32_t valid;
    uint32_t run = block_exclusive_scan<4>(sum, scan_tmp, &valid);
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        start[NB - 1 - (BPT * t + i)] = run;            // members above the bucket
        run += c[i];
    }
    __syncthreads();
    // global traffic with consecutive lanes on consecutive words
    for (int b = t; b < NB; b += 256) {
        above[b + 1] = start[b];
        const uint32_t n = hist[b];
        if (n)
            atomicAdd(&W[b], n);
    }
    if (t == 0)
        above[0] = valid;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (bk[i] >= 0)
            keys[start[bk[i]] + rk[i]] = composite(order_key(e[i]), j0 + i);
}

template <int NB, int J, bool VEC>
__global__ __launch_bounds__(kSelThreads) void k_wide_finish(const float *__restrict__ scores,
                                                             int f, int k,
                                                             const uint32_t *__restrict__ ws,
                                                             int ws_stride,
                                                             int32_t *__restrict__ idx,
                                                             int idx_stride,
                                                             int32_t *__restrict__ count,
                                                             uint32_t *__restrict__ bitmap,
                                                             int prefix)
{
    static_assert(NB % kSelThreads == 0, "whole buckets per thread");
    constexpr int BPT = NB / kSelThreads;
    __shared__ uint64_t cand[kWideMaxCand];
    __shared__ uint32_t keep_bits[kWideSlice / 32];
    __shared__ uint32_t scan_tmp[kSelWaves];
    __shared__ uint32_t soff[kSelThreads];    // first candidate of each slice
    __shared__ uint32_t sbeg[kSelThreads];    // its place among the slice's sorted composites
    __shared__ uint32_t misc[4];              // B*, need, members of B*, candidates
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int token = blockIdx.y, slice = blockIdx.x;
    const int nslices = (f + kWideSlice - 1) / kWideSlice;
    const float *s = scores + (size_t)token * f;
    const uint32_t *W = ws + (size_t)token * ws_stride;
    const int lim = slice * kWideSlice;
    const int j = lim + t;
    const float mine = j < f ? s[j] : 0.0f;
    uint32_t c[BPT];
    uint32_t csum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        c[i] = W[NB - 1 - (BPT * t + i)];
        csum += c[i];
    }
    if (t == 0) {
        misc[0] = 0u;
        misc[1] = 0u;
        misc[2] = 0u;
    }
    if (t < kWideSlice / 32)
        keep_bits[t] = 0u;
    uint32_t total;
    uint32_t above = block_exclusive_scan<kSelWaves>(csum, scan_tmp, &total);
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        if (above < (uint32_t)k && above + c[i] >= (uint32_t)k) {
            misc[0] = (uint32_t)(NB - 1 - (BPT * t + i));
            misc[1] = (uint32_t)k - above;
            misc[2] = c[i];
        }
        above += c[i];
    }
    __syncthreads();
    const int bstar = (int)misc[0];
    const uint32_t need = misc[1];
    if (misc[2] > (uint32_t)kWideMaxCand) {
        // heavy ties in the boundary bucket: the one-workgroup selection (uniform branch)
        if (slice == 0)
            topk_one_workgroup<NB, J, VEC>(scores, token, f, k, idx, idx_stride, count, bitmap,
                                           prefix, W);
        return;
    }
    // slice t: members above B* (certain) and B*'s members, from its above[] words
    uint32_t sab = 0, scnt = 0;
    if (t < nslices) {
        const uint32_t *ab = wide_slice(const_cast<uint32_t *>(W), t);
        sab = ab[bstar + 1];
        scnt = ab[bstar] - sab;
    }
    // at most 64 slices (f <= 65536): wavefront 0 places each slice's first candidate
    if (w == 0) {
        const uint32_t incl = wave_inclusive_scan(scnt);
        soff[t] = incl - scnt;
        sbeg[t] = sab;
        if (lane == kWave - 1)
            misc[3] = incl;
    }
    uint32_t before = t < slice ? sab : 0u;
    __syncthreads();
    const uint32_t nc = misc[3];
    if (nc > (uint32_t)kWideMaxCand) {
        // only without a boundary bucket (fewer than k non-NaN scores), when B* = 0 stands in;
        // the one-workgroup selection decides as above
        if (slice == 0)
            topk_one_workgroup<NB, J, VEC>(scores, token, f, k, idx, idx_stride, count, bitmap,
                                           prefix, W);
        return;
    }
    if ((uint32_t)t < nc) {
        // candidate t lives in the last slice whose first candidate is at or before t
        int lo = 0, hi = nslices - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (soff[mid] <= (uint32_t)t)
                lo = mid;
            else
                hi = mid - 1;
        }
        const uint64_t *keys =
            reinterpret_cast<const uint64_t *>(wide_slice(const_cast<uint32_t *>(W), lo) + kWideAbove);
        cand[t] = keys[sbeg[lo] + (uint32_t)t - soff[lo]];
    }
    __syncthreads();
    // rank the candidates by (score desc, index asc): L lanes per candidate (a power of two, at
    // most 64, with nc * L <= 1024) each count the candidates ordered before it in every L-th
    // place, and the group adds its counts.  Count the kept ones below this slice and mark those
    // inside it.
    uint32_t L = kWave;
    while (L > 1 && nc * L > (uint32_t)kSelThreads)
        L >>= 1;
    const uint32_t ci = (uint32_t)t / L, sub = (uint32_t)t % L;
    uint64_t me = 0;
    uint32_t rank = 0;
    if (ci < nc) {
        me = cand[ci];
        for (uint32_t r = sub; r < nc; r += L)
            rank += cand[r] > me ? 1u : 0u;
    }
    for (uint32_t o = 1; o < L; o <<= 1)
        rank += __shfl_xor(rank, (int)o, kWave);
    if (ci < nc && sub == 0 && rank < need) {
        const int jc = (int)(0xffffffffu - (uint32_t)me);
        if (jc < lim)
            ++before;
        else if (jc < lim + kWideSlice)
            atomicOr(&keep_bits[(jc - lim) >> 5], 1u << (jc & 31));
    }
    __syncthreads();
    const bool sel = (j < f && score_bucket<NB>(mine) > bstar) ||
                     ((keep_bits[t >> 5] >> (t & 31)) & 1u);
    // one scan for both counts, packed as (before << 11) | sel: the low field's exclusive prefix
    // (< 1024) is this thread's place among the slice's selected, the high field's block total
    // the selected neurons of the earlier slices (<= 65536, so the word does not overflow)
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<kSelWaves>((before << 11) | (sel ? 1u : 0u), scan_tmp,
                                                        &tot);
    const uint32_t pos = (tot >> 11) + (ex & 0x7ffu);
    int32_t *out = idx + (size_t)token * idx_stride;
    if (sel && prefix + pos < (uint32_t)idx_stride)
        out[prefix + pos] = prefix + j;
    if (bitmap) {
        // words lim/32 + 2w and + 2w+1 from the wavefront's 64 bits (positions past f are clear)
        const int words = (f + 31) / 32;
        const uint64_t m = __ballot(sel);
        const int wd = lim / 32 + 2 * w + (lane >> 5);
        if ((lane & 31) == 0 && wd < words)
            bitmap[(size_t)token * words + wd] = (uint32_t)(m >> (lane & 32));
    }
    if (slice == 0) {
        for (int i = t; i < prefix; i += kSelThreads)
            out[i] = i;
        if (t == 0 && count)
            count[token] = prefix + k;
    }
}

template <int J, bool VEC>
__global__ __launch_bounds__(kSelThreads) void k_select_threshold(
    const float *__restrict__ scores, int f, float tau, int32_t *__restrict__ idx, int idx_stride,
    int32_t *__restrict__ count, uint32_t *__restrict__ bitmap, int prefix)
{
    __shared__ uint32_t bm[kMaxWords];
    __shared__ uint32_t trash[kSelThreads];
    __shared__ uint32_t scan_tmp[kSelWaves];
    const int t = threadIdx.x;
    const int token = blockIdx.x;
    const float *s = scores + (size_t)token * f;
    const int words = (f + 31) / 32;
    float4 v[J];
#pragma unroll
    for (int i = 0; i < J; ++i)
        v[i] = load_quad<VEC>(s, i * kQuad + 4 * t, f);
#pragma unroll
    for (int i = 0; i < J; ++i) {
        // NaN (positions past f) never compares >= tau
        const uint32_t nib = (v[i].x >= tau ? 1u : 0u) | (v[i].y >= tau ? 2u : 0u) |
                             (v[i].z >= tau ? 4u : 0u) | (v[i].w >= tau ? 8u : 0u);
        store_nibbles(nib, bm, (i * kQuad + 4 * t) >> 5 & ~7, words, trash);
    }
    __syncthreads();
    uint32_t total;
    int32_t *out = idx + (size_t)token * idx_stride;
    for (int i = t; i < prefix; i += kSelThreads)
        out[i] = i;
    bitmap_to_list(bm, words, out + prefix, idx_stride - prefix, prefix,
                   bitmap ? bitmap + (size_t)token * words : nullptr, scan_tmp, &total);
    if (t == 0)
        count[token] = prefix + (int32_t)total;
}


template <int J>
hipError_t topk_j(const float *scores, int B, int f, int k, int32_t *idx, int idx_stride,
                  int32_t *count, uint32_t *bitmap, hipStream_t st, Trace *tr, int prefix)
{
    if (f % 4 == 0)
        return launch(k_select_topk<kScoreBuckets, J, true>, dim3(B), dim3(kSelThreads), st, tr,
                      scores, f, k, idx, idx_stride, count, bitmap, prefix);
    return launch(k_select_topk<kScoreBuckets, J, false>, dim3(B), dim3(kSelThreads), st, tr,
                  scores, f, k, idx, idx_stride, count, bitmap, prefix);
}

template <int J>
hipError_t threshold_j(const float *scores, int B, int f, float tau, int32_t *idx, int idx_stride,
                       int32_t *count, uint32_t *bitmap, hipStream_t st, Trace *tr, int prefix)
{
    if (f % 4 == 0)
        return launch(k_select_threshold<J, true>, dim3(B), dim3(kSelThreads), st, tr, scores, f,
                      tau, idx, idx_stride, count, bitmap, prefix);
    return launch(k_select_threshold<J, false>, dim3(B), dim3(kSelThreads), st, tr, scores, f,
                  tau, idx, idx_stride, count, bitmap, prefix);
}

template <int J>
hipError_t wide_j(const float *scores, int B, int f, int k, int32_t *idx, int idx_stride,
                  int32_t *count, uint32_t *bitmap, uint32_t *ws, int ws_stride, hipStream_t st,
                  Trace *tr, int prefix)
{
    const dim3 grid((f + kWideSlice - 1) / kWideSlice, B);
    const bool vec = f % 4 == 0;
    hipError_t e = vec ? launch(k_wide_hist<kScoreBuckets, true>, grid, dim3(256), st, tr, scores,
                                f, ws, ws_stride)
                       : launch(k_wide_hist<kScoreBuckets, false>, grid, dim3(256), st, tr,
                                scores, f, ws, ws_stride);
    if (e != hipSuccess)
        return e;
    if (vec)
        return launch(k_wide_finish<kScoreBuckets, J, true>, grid, dim3(kSelThreads), st, tr,
                      scores, f, k, static_cast<const uint32_t *>(ws), ws_stride, idx, idx_stride,
                      count, bitmap, prefix);
    return launch(k_wide_finish<kScoreBuckets, J, false>, grid, dim3(kSelThreads), st, tr, scores,
                  f, k, static_cast<const uint32_t *>(ws), ws_stride, idx, idx_stride, count,
                  bitmap, prefix);
}

__global__ __launch_bounds__(256) void k_wide_zero(uint32_t *__restrict__ ws, int ws_stride, int n)
{
    uint32_t *W = ws + (size_t)blockIdx.x * ws_stride;
    for (int i = threadIdx.x; i < n; i += 256)
        W[i] = 0u;
}

}  // namespace

int select_max_f() { return 32 * kMaxWords; }

// measured: the three-kernel form pays off from about 20000 scores (at 14336 both take the same
// time, at 49152 the layer is 3 us faster)
bool select_wide_used(int B, int f, int k) { return B >= 1 && B <= 4 && f >= 20000 && k > 0; }

int select_wide_ws_words(int f)
{
    const int slices = (f + kWideSlice - 1) / kWideSlice;
    return (kScoreBuckets + slices * kWideSliceWords + 63) / 64 * 64;
}

int select_wide_zero_words() { return kScoreBuckets; }

hipError_t launch_select_topk_wide(const float *scores, int B, int f, int k, int32_t *idx,
                                   int idx_stride, int32_t *count, uint32_t *bitmap, uint32_t *ws,
                                   bool zeroed, hipStream_t st, Trace *tr, int prefix)
{
    const int stride = select_wide_ws_words(f);
    if (!zeroed) {
        hipError_t e = launch(k_wide_zero, dim3(B), dim3(256), st, nullptr, ws, stride,
                              select_wide_zero_words());
        if (e != hipSuccess)
            return e;
    }
    const int J = (f + kQuad - 1) / kQuad;
    if (J <= 1) return wide_j<1>(scores, B, f, k, idx, idx_stride, count, bitmap, ws, stride, st, tr, prefix);
    if (J <= 2) return wide_j<2>(scores, B, f, k, idx, idx_stride, count, bitmap, ws, stride, st, tr, prefix);
    if (J <= 4) return wide_j<4>(scores, B, f, k, idx, idx_stride, count, bitmap, ws, stride, st, tr, prefix);
    if (J <= 8) return wide_j<8>(scores, B, f, k, idx, idx_stride, count, bitmap, ws, stride, st, tr, prefix);
    if (J <= 12) return wide_j<12>(scores, B, f, k, idx, idx_stride, count, bitmap, ws, stride, st, tr, prefix);
    if (J <= 16) return wide_j<16>(scores, B, f, k, idx, idx_stride, count, bitmap, ws, stride, st, tr, prefix);
    return hipErrorInvalidValue;
}

hipError_t launch_select_topk(const float *scores, int B, int f, int k, int32_t *idx,
                              int idx_stride, int32_t *count, uint32_t *bitmap, hipStream_t st,
                              Trace *tr, int prefix)
{
    const int J = (f + kQuad - 1) / kQuad;     // sweeps of 4096 scores
    if (J <= 1) return topk_j<1>(scores, B, f, k, idx, idx_stride, count, bitmap, st, tr, prefix);
    if (J <= 2) return topk_j<2>(scores, B, f, k, idx, idx_stride, count, bitmap, st, tr, prefix);
    if (J <= 4) return topk_j<4>(scores, B, f, k, idx, idx_stride, count, bitmap, st, tr, prefix);
    if (J <= 8) return topk_j<8>(scores, B, f, k, idx, idx_stride, count, bitmap, st, tr, prefix);
    if (J <= 12) return topk_j<12>(scores, B, f, k, idx, idx_stride, count, bitmap, st, tr, prefix);
    if (J <= 16) return topk_j<16>(scores, B, f, k, idx, idx_stride, count, bitmap, st, tr, prefix);
    return hipErrorInvalidValue;
}

hipError_t launch_select_threshold(const float *scores, int B, int f, float tau, int32_t *idx,
                                   int idx_stride, int32_t *count, uint32_t *bitmap,
                                   hipStream_t st, Trace *tr, int prefix)
{
    const int J = (f + kQuad - 1) / kQuad;
    if (J <= 1) return threshold_j<1>(scores, B, f, tau, idx, idx_stride, count, bitmap, st, tr, prefix);
    if (J <= 2) return threshold_j<2>(scores, B, f, tau, idx, idx_stride, count, bitmap, st, tr, prefix);
    if (J <= 4) return threshold_j<4>(scores, B, f, tau, idx, idx_stride, count, bitmap, st, tr, prefix);
    if (J <= 8) return threshold_j<8>(scores, B, f, tau, idx, idx_stride, count, bitmap, st, tr, prefix);
    if (J <= 12) return threshold_j<12>(scores, B, f, tau, idx, idx_stride, count, bitmap, st, tr, prefix);
    if (J <= 16) return threshold_j<16>(scores, B, f, tau, idx, idx_stride, count, bitmap, st, tr, prefix);
    return hipErrorInvalidValue;
}

}  // namespace csf
