// launch.hpp -- internal launchers of the gfx950 kernels (not part of the C ABI).
//
// Each launcher takes validated arguments (the C-ABI layer in api.cpp checks every size, pointer
// and alignment first), picks the template instance and grid, enqueues on `stream` and returns the
// launch status.  Sizes are in elements unless named *_chunks (16-byte units).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csf {

// Optional per-kernel timing: while set, each launch takes the next two caller-owned events and
// has the runtime record them at the kernel's start and end (hipExtLaunchKernel), so their
// difference is the kernel's own duration.
struct Trace {
    hipEvent_t *ev = nullptr;
    int n = 0;
    int pos = 0;
    bool next(hipEvent_t *start, hipEvent_t *stop)
    {
        if (!ev || pos + 1 >= n)
            return false;
        *start = ev[pos];
        *stop = ev[pos + 1];
        pos += 2;
        return true;
    }
};

template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                         Trace *tr, Args... args)
{
    hipEvent_t start, stop;
    if (tr && tr->next(&start, &stop))
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, start, stop, 0, static_cast<KArgs>(args)...);
    else
        kernel<<<grid, block, 0, st>>>(static_cast<KArgs>(args)...);
    return hipGetLastError();
}

// ---- predictor (predict.hip) ----------------------------------------------------------------
// Split-K factor of the predictor's down projection (rows of V split over S workgroups).
constexpr int kMaxPredSplit = 4;
int pred_split(int r, int d, int dtype);
// part[S][B][r] = split-K partial sums of V x_t (float32), S = pred_split(r, d, dtype).  zero
// (optional): nzero words that the launch also clears, and fill: nfill words it sets to
// kHSentinel, for a later kernel of the same call.
hipError_t launch_pred_down(int dtype, const void *x, int B, int d, const void *V, int r,
                            float *part, hipStream_t stream, Trace *trace = nullptr,
                            uint32_t *zero = nullptr, int nzero = 0, uint32_t *fill = nullptr,
                            int nfill = 0);
// One token with at most kSmallF scores: s[f] = sigmoid(U relu(sum of the partials)) and, in the
// same kernel, the selection: top-k (k >= 0) or s >= tau (k == -1) into the ascending list idx
// and count (k, or the threshold count).  The lists equal those of the selection kernels.
constexpr int kSmallF = 1024;
hipError_t launch_pred_up_select(int dtype, const float *part, int d, int r, const void *U, int f,
                                 float *s, int k, float tau, int32_t *idx, int32_t *count,
                                 hipStream_t stream, Trace *trace = nullptr);
// s[B][f] = sigmoid(U relu(sum of the partials)) in float32.  grid: workgroups of the persistent
// one-token form (the caller's choice from the device's compute units: the most resident at once,
// or fewer for a predictor that runs beside other work on a second stream); unused for batches.
hipError_t launch_pred_up(int dtype, const float *part, int B, int d, int r, const void *U, int f,
                          float *s, hipStream_t stream, Trace *trace, int grid);

// ---- predictor for a batch on the matrix cores (predict_mfma.hip) --------------------------
constexpr int kPredMfmaMinBatch = 4;      // tokens from which the batched predictor is used
constexpr int kMaxPredMfmaTokens = 32;    // tokens per pass (two 16-token MFMA tiles)
constexpr int kMaxPredMfmaSplit = 32;     // split of d over workgroups in the down projection
bool pred_mfma_supported(int dtype, int B, int d, int r);
int pred_mfma_split(int r, int d);
size_t pred_mfma_ws_floats(int B, int r);   // workspace (floats) of launch_predict_mfma
// s[B][f] = sigmoid(U relu(V x)) for 16-bit weights; ws: pred_mfma_ws_floats(B, r) floats.
// res_grid: workgroups of the register-resident up projection (two per compute unit).
hipError_t launch_predict_mfma(int dtype, const void *x, int B, int d, const void *V, int r,
                               const void *U, int f, float *s, float *ws, hipStream_t stream,
                               Trace *trace, int res_grid);

// ---- selection (select.hip) -----------------------------------------------------------------
// prefix: the list of each token starts with the neurons 0 .. prefix-1 (a block that is always
// computed) and the selected neurons follow as prefix + their index among the scores; counts
// include the prefix, idx_stride must hold it.
hipError_t launch_select_topk(const float *scores, int B, int f, int k, int32_t *idx,
                              int idx_stride, int32_t *count, uint32_t *bitmap,
                              hipStream_t stream, Trace *trace = nullptr, int prefix = 0);
hipError_t launch_select_threshold(const float *scores, int B, int f, float tau, int32_t *idx,
                                   int idx_stride, int32_t *count, uint32_t *bitmap,
                                   hipStream_t stream, Trace *trace = nullptr, int prefix = 0);
int select_max_f();   // largest f the selection kernels accept
// Top-k of a few tokens with many scores, spread over many workgroups (two kernels).  ws holds
// select_wide_ws_words(f) 32-bit words per token; its first select_wide_zero_words() words of each
// token must be zero at the start: pass zeroed = false to have this launch clear them.
bool select_wide_used(int B, int f, int k);
int select_wide_ws_words(int f);
int select_wide_zero_words();
hipError_t launch_select_topk_wide(const float *scores, int B, int f, int k, int32_t *idx,
                                   int idx_stride, int32_t *count, uint32_t *bitmap, uint32_t *ws,
                                   bool zeroed, hipStream_t stream, Trace *trace = nullptr,
                                   int prefix = 0);

// ---- FFN (ffn.hip) --------------------------------------------------------------------------
struct FfnArgs {
    int dtype, act;
    const void *x;          // [B][d]
    int B, d, f;
    const void *W1, *Wup, *W2T;
    const float *b1;        // may be null
    const int32_t *idx;     // [B][idx_stride]; null = identity list (dense)
    int idx_stride;
    const int32_t *count;   // [B] device; null = max_count for every token
    int max_count;
    float *h;               // [B][h_stride]
    int h_stride;
    float *y;               // [B][d]
    float *partials;        // [B][ffn_num_chunks][d] workspace
    int accumulate = 0;     // 1: y += the FFN output (residual add)
    int skip_zero = 0;      // 1: post-gate skip: a neuron whose |gate activation| <= gate_tau
                            // gets h = 0, and rows with h = 0 are not read (down rows; up rows
                            // of the gated forms)
    float gate_tau = 0.0f;
};
// Shape of the down projection's two-phase reduction (sizes its workspace).
int ffn_num_slices(int d, int dtype);
int ffn_max_count();   // longest active list (and widest dense layer) the FFN kernels take
int ffn_num_chunks(int d, int dtype, int max_count);
hipError_t launch_ffn(const FfnArgs &a, hipStream_t stream, Trace *trace = nullptr);
// One token (B == 1, no skip) in one kernel: the up rows, the down rows and the reduction as
// roles of one launch, handing h and the partial rows over inside it (bit-identical y).  When
// the kernel starts, a.h[0, max_count) must hold kHSentinel and sync (ffn_fused_sync_words()
// words) must be zero: an earlier kernel of the same call writes them.  The last counter line
// counts waits that gave up (0 in a correct run).
int ffn_fused_sync_words();
hipError_t launch_ffn_fused(const FfnArgs &a, uint32_t *sync, hipStream_t stream,
                            Trace *trace = nullptr);
// The down projection and reduction alone, over a list whose h values are already in a.h.
hipError_t launch_ffn_down(const FfnArgs &a, hipStream_t stream, Trace *trace = nullptr);
// y[t][col] = sum over chunks q, in order, of part[t][q][col] (part is [B][nchunk][D] float32).
hipError_t launch_reduce_partials(const float *part, int nchunk, int D, int B, float *y,
                                  hipStream_t stream, Trace *trace = nullptr, int accumulate = 0);

// ---- attention-head sparsity (attention.hip) --------------------------------------------------
struct AttnArgs {
    int dtype;
    const void *x;                  // [d]
    int d, H, dh;
    const void *Wq, *Wk, *Wv, *WoT; // [H*dh][d]
    const float *bq, *bk, *bv;      // [H*dh] or null
    void *Kc, *Vc;                  // [H][Tmax][dh]
    int Tmax;
    int32_t *len;                   // [H] device, advanced for the heads that store the token
    const int32_t *heads;           // [max_heads] device, or null = every head (max_heads == H)
    const int32_t *count;           // device, or null = max_heads
    int max_heads, kv_all;
    float *o;                       // [max_heads][dh] or null
    float *y;                       // [d]
    // workspace
    int32_t *lnew;                  // [max_heads] attention length of each list entry (-1: skip)
    float *qbuf;                    // [max_heads][dh]
    float *part;                    // [max_heads][attn_num_splits(Tmax)][dh + 2]
    int32_t *rows;                  // [max_heads * dh]
    float *hv;                      // [max_heads * dh]
    int32_t *rows_count;            // [1]
    float *ffn_partials;            // [ffn_num_chunks(d, dtype, max_heads * dh)][d]
};
int attn_num_splits(int Tmax);
int attn_max_cache();   // largest Tmax the attention kernels take
bool attn_head_dim_supported(int dtype, int dh);
hipError_t launch_attention_decode(const AttnArgs &a, hipStream_t stream, Trace *trace = nullptr);

// ---- static scratch (scratch.hip) -------------------------------------------------------------
// Bytes of the library's static device scratch; scratch_init reads its device address on
// `device` (which must be current; once per device, later calls return at once) and scratch_ptr
// returns that address (NULL before scratch_init succeeded).
size_t scratch_bytes();
hipError_t scratch_init(int device);
void *scratch_ptr(int device);

// ---- stack of blocks (stack.hip) -------------------------------------------------------------
// xhat[t] = storage-type rounding of x[t] / sqrt(mean(x[t]^2) + eps) (norm = 1) or of x[t]
// (norm = 0); x_log / xhat_log (optional) receive copies of x and xhat.  zero (optional): nzero
// words the launch also clears, and fill: nfill words it sets to kHSentinel (the hand-over state
// of a one-kernel FFN that follows on the same stream).
hipError_t launch_rms_norm(int dtype, const float *x, int B, int d, float eps, int norm, void *xhat,
                           float *x_log, void *xhat_log, hipStream_t stream,
                           uint32_t *zero = nullptr, int nzero = 0, uint32_t *fill = nullptr,
                           int nfill = 0);

// ---- batched FFN over the union of the tokens' sets (union.hip) -------------------------------
constexpr int kMaxUnionBatch = 32;   // tokens per call (two 16-token matrix-core tiles)
struct UnionArgs {
    int cus = 0;            // compute units of the device
    int dtype, act;
    int per_token;          // 1: token t keeps only its own rows; 0: every union row for all
    int mfma;               // 1: matrix-core path (16-bit types, d % 256 == 0); 0: vector ALU
    const void *X;          // [B][d]
    int B, d, f;
    const void *W1, *Wup, *W2T;
    const float *b1;        // may be null
    const uint32_t *bitmaps;  // [B][ceil(f / 32)]
    float *Y;               // [B][d]
    int32_t *ucount_out;    // optional device copy of the union size
    // workspace
    int32_t *ulist;         // [f]
    int32_t *ucount;        // [1]
    float *h32;             // [B][hs]
    uint32_t *hmax;         // [kMaxUnionBatch] per-token largest |h| past the 16-bit split limit
    int hs;                 // union_h_stride(f)
    float *partials;        // [B][union_num_chunks][d]
};
bool union_mfma_supported(int dtype, int d, int B);
// chunks of the union's down projection (sizes its workspace); cus: the device's compute units
int union_num_chunks(int mfma, int d, int dtype, int f, int cus);
size_t union_h_stride(int f);
hipError_t launch_union_ffn(const UnionArgs &a, hipStream_t stream, Trace *trace = nullptr);

}  // namespace csf
