// api.cpp -- the C ABI of the contextual-sparsity FFN library (declared in include/csf.h):
// host-side argument validation, workspace carving and kernel dispatch.
//
// Every entry point checks all of its arguments before it enqueues anything, so a rejected call
// leaves the stream untouched.  Nothing here allocates device memory or synchronises the device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>
#include <string>

#include "../../include/csf.h"
#include "common.hpp"
#include "launch.hpp"

// The state a handle owns: facts of its device (queried once), the gathered FFN's options, the
// per-kernel timing hook, and what the stack keeps between calls (events, a capture stream, the
// captured graph).  No tensor and no device memory.
struct csf_context {
    int device = 0;
    int cus = 0;                  // compute units
    int pred_up_grid = 0;         // persistent one-token up projection: 8 workgroups per CU
    int pred_up_side_grid = 0;    // the look-ahead stack's side-stream copy: 4 per CU
    int ffn_flags = 0;
    float gate_tau = 0.0f;
    hipEvent_t trace[16] = {};
    int trace_n = 0;
    hipEvent_t stack_ev[4] = {};  // look-ahead stack: input ready x2, selection ready x2
    hipStream_t capture = nullptr;
    uint64_t graph_key = 0;
    hipGraphExec_t graph = nullptr;
};

namespace {

thread_local std::string g_last_error;

// Live handles: a destroyed handle (or any other pointer) is recognised as not a handle.
std::mutex g_handles_mu;
std::unordered_set<const csf_context *> g_handles;

bool is_live(const csf_context *h)
{
    if (!h)
        return false;
    std::lock_guard<std::mutex> lock(g_handles_mu);
    return g_handles.count(h) != 0;
}

int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok()
{
    g_last_error.clear();
    return CSF_OK;
}

int hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return ok();
    return fail(CSF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes(int dtype) { return dtype == CSF_F32 ? 4 : 2; }
bool valid_dtype(int dtype) { return dtype == CSF_F32 || dtype == CSF_F16 || dtype == CSF_BF16; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Limits of the library's kernels (rows held in registers per thread).
constexpr long kMaxRowChunks = 16 * 256;   // d: 16-byte chunks per row for the gathered kernels
constexpr long kMaxPredChunks = 512;       // r: 16-byte chunks per row of U

#define REQUIRE(cond, status, ...)                 \
    do {                                           \
        if (!(cond))                               \
            return fail(status, __VA_ARGS__);      \
    } while (0)

// Test hook: the environment variable CSF_FAULT_INJECT names entry points (comma-separated, or
// "all") whose dispatch fails with CSF_ERR_HIP once their arguments have passed every check and
// before anything is enqueued, so a caller can exercise its handling of a HIP failure without a
// failing device (and without a device at all).  Read on every call; unset or empty: off.
bool fault_injected(const char *op)
{
    const char *v = getenv("CSF_FAULT_INJECT");
    if (!v || !*v)
        return false;
    if (!strcmp(v, "all"))
        return true;
    const size_t n = strlen(op);
    for (const char *p = v;;) {
        const char *c = strchr(p, ',');
        const size_t len = c ? (size_t)(c - p) : strlen(p);
        if (len == n && !strncmp(p, op, n))
            return true;
        if (!c)
            return false;
        p = c + 1;
    }
}

// A handle is checked after every other argument (so host-side argument checks need none) and
// before anything is enqueued: it must be live and belong to the current device.  The fault
// injection hook comes first, so it also answers for a call without a live handle.
int check_handle(csf_handle h, const char *op)
{
    if (fault_injected(op))
        return fail(CSF_ERR_HIP, "%s: failure injected by CSF_FAULT_INJECT (nothing enqueued)", op);
    if (!is_live(h))
        return fail(CSF_ERR_INVALID_ARG, "handle is NULL or not a live handle (csf_create)");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(CSF_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev != h->device)
        return fail(CSF_ERR_INVALID_ARG, "the handle belongs to device %d but device %d is current",
                    h->device, dev);
    return CSF_OK;
}

#define CHECK_HANDLE(h)                                    \
    do {                                                   \
        int _s = check_handle(h, __func__);                \
        if (_s != CSF_OK)                                  \
            return _s;                                     \
    } while (0)

// the timing hook of a handle (empty when off)
csf::Trace make_trace(csf_handle h)
{
    csf::Trace tr;
    if (h && h->trace_n > 0) {
        tr.ev = h->trace;
        tr.n = h->trace_n;
    }
    return tr;
}

// compute units a workspace is sized for: a live handle's device, or (no handle) any device
int sizing_cus(csf_handle h) { return is_live(h) ? h->cus : 1 << 20; }

int check_ptr(const void *p, const char *name, bool required)
{
    if (!p) {
        if (required)
            return fail(CSF_ERR_INVALID_ARG, "%s must not be NULL", name);
        return CSF_OK;
    }
    if (!aligned16(p))
        return fail(CSF_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
    return CSF_OK;
}

#define CHECK_PTR(p, req)                                  \
    do {                                                   \
        int _s = check_ptr((p), #p, (req));                \
        if (_s != CSF_OK)                                  \
            return _s;                                     \
    } while (0)

int check_row(int n, int dtype, const char *name, long max_chunks)
{
    if (n <= 0)
        return fail(CSF_ERR_INVALID_ARG, "%s must be positive (got %d)", name, n);
    long bytes = (long)n * elem_bytes(dtype);
    if (bytes % 16 != 0)
        return fail(CSF_ERR_UNSUPPORTED,
                    "%s = %d: a row must be a multiple of 16 bytes (%s of 8 for 16-bit types, 4 for float32)",
                    name, n, name);
    if (bytes / 16 > max_chunks)
        return fail(CSF_ERR_UNSUPPORTED, "%s = %d exceeds the library's limit of %ld elements", name,
                    n, max_chunks * 16 / elem_bytes(dtype));
    return CSF_OK;
}

#define CHECK_ROW(n, dtype, maxc)                          \
    do {                                                   \
        int _s = check_row((n), (dtype), #n, (maxc));      \
        if (_s != CSF_OK)                                  \
            return _s;                                     \
    } while (0)

// ---- workspace layouts -------------------------------------------------------------------------
// predictor scratch: split-K partial vectors (vector-ALU path) or partial sums and the 16-bit
// terms of the hidden activation (matrix-core path for batches), whichever is larger
size_t pred_ws_bytes(int B, int r)
{
    const size_t Bn = B > 0 ? (size_t)B : 1;
    const size_t v = (size_t)csf::kMaxPredSplit * Bn * r;
    const size_t m = csf::pred_mfma_ws_floats((int)Bn, r);
    return round_up((v > m ? v : m) * sizeof(float));
}

struct PredictWs {
    size_t a, total;
};
PredictWs predict_ws(int B, int r)
{
    PredictWs w;
    w.a = 0;
    w.total = pred_ws_bytes(B, r);
    return w;
}

// the predictor for B tokens: matrix cores for batches of 16-bit weights, else vector ALU.
// zero (optional): nzero words the vector-ALU path clears on the way (*zeroed tells whether it
// did), for a later kernel of the same call.
// side: the look-ahead stack's second-stream copy (a smaller persistent grid).
hipError_t enqueue_predict(int dtype, const void *x, int B, int d, const void *V, int r,
                           const void *U, int f, float *scores, float *ws, hipStream_t st,
                           csf::Trace *tr, const csf_context *h, bool side = false,
                           uint32_t *zero = nullptr, int nzero = 0, bool *zeroed = nullptr)
{
    if (zeroed)
        *zeroed = false;
    if (csf::pred_mfma_supported(dtype, B, d, r))
        return csf::launch_predict_mfma(dtype, x, B, d, V, r, U, f, scores, ws, st, tr,
                                        2 * h->cus);
    const int pu_grid = side ? h->pred_up_side_grid : h->pred_up_grid;
    if (zeroed)
        *zeroed = zero != nullptr;
    hipError_t e = csf::launch_pred_down(dtype, x, B, d, V, r, ws, st, tr, zero, nzero);
    if (e != hipSuccess)
        return e;
    return csf::launch_pred_up(dtype, ws, B, d, r, U, f, scores, st, tr, pu_grid);
}

struct FfnWs {
    size_t h, partials, total;
};
FfnWs ffn_ws(int B, int d, int dtype, int max_count)
{
    FfnWs w;
    w.h = 0;
    w.partials = round_up((size_t)B * (max_count > 0 ? max_count : 1) * sizeof(float));
    const size_t nchunk = (size_t)csf::ffn_num_chunks(d, dtype, max_count);
    w.total = w.partials + round_up((size_t)B * nchunk * d * sizeof(float));
    return w;
}

// counters of the one-kernel gathered FFN, rounded so that the selection's counter block that
// follows them starts 256-byte aligned: one clear covers both
int fused_sync_words() { return (csf::ffn_fused_sync_words() + 63) / 64 * 64; }

struct LayerWs {
    size_t a, scores, idx, count, sync, sel, ffn, total;
};
LayerWs layer_ws(int d, int f, int r, int max_count, int dtype)
{
    LayerWs w;
    w.a = 0;
    w.scores = w.a + round_up((size_t)csf::kMaxPredSplit * r * sizeof(float));
    w.idx = w.scores + round_up((size_t)f * sizeof(float));
    w.count = w.idx + round_up((size_t)f * sizeof(int32_t));
    w.sync = w.count + round_up(sizeof(int32_t));
    w.sel = w.sync + (size_t)fused_sync_words() * sizeof(uint32_t);
    w.ffn = w.sel + round_up((size_t)csf::select_wide_ws_words(f) * sizeof(uint32_t));
    w.total = w.ffn + ffn_ws(1, d, dtype, max_count).total;
    return w;
}

// Batches of at least this many tokens take the matrix-core path when it applies (the gather
// path's vector ALU work grows with B per weight byte; the matrix cores' does not bind).
constexpr int kMfmaMinBatch = 2;   // measured: from two tokens on the matrix-core path is faster

struct UnionWs {
    size_t ulist, ucount, hmax, h, partials, total;
};
UnionWs union_ws(int B, int d, int f, int dtype, int cus)
{
    UnionWs w;
    const size_t hs = csf::union_h_stride(f);
    const size_t Bn = B > 0 ? (size_t)B : 1;
    w.ulist = 0;
    w.ucount = round_up((size_t)f * sizeof(int32_t));
    w.hmax = w.ucount + kAlign / 2;   // the union size, then the per-token |h| maxima
    static_assert(csf::kMaxUnionBatch * sizeof(uint32_t) <= kAlign / 2, "maxima fit the line");
    w.h = w.ucount + kAlign;
    w.partials = w.h + round_up(Bn * hs * sizeof(float));
    int nch = csf::union_num_chunks(0, d, dtype, f, cus);
    const int nm = csf::union_num_chunks(1, d, dtype, f, cus);
    if (nm > nch)
        nch = nm;
    w.total = w.partials + round_up(Bn * (size_t)nch * d * sizeof(float));
    return w;
}

struct BatchedLayerWs {
    size_t a, scores, idx, count, bitmap, uni, total;
};
BatchedLayerWs batched_layer_ws(int B, int d, int f, int r, int max_count, int dtype, int cus)
{
    BatchedLayerWs w;
    const size_t Bn = B > 0 ? (size_t)B : 1;
    w.a = 0;
    w.scores = w.a + pred_ws_bytes(B, r);
    w.idx = w.scores + round_up(Bn * f * sizeof(float));
    w.count = w.idx + round_up(Bn * (max_count > 0 ? max_count : 1) * sizeof(int32_t));
    w.bitmap = w.count + round_up(Bn * sizeof(int32_t));
    w.uni = w.bitmap + round_up(Bn * ((f + 31) / 32) * sizeof(uint32_t));
    w.total = w.uni + union_ws(B, d, f, dtype, cus).total;
    if (B == 1) {
        // a batch of one on the gather path runs the single-token layer in this workspace
        const size_t one = layer_ws(d, f, r, max_count, dtype).total;
        if (one > w.total)
            w.total = one;
    }
    return w;
}

struct StackWs {
    size_t xhat[2], a_main, s_main, a_side, s_side, sel_main, sel_side, idx[2], count[2], sync, ffn,
        total;
};
StackWs stack_ws(int B, int d, int f, int r, int max_count, int dtype)
{
    StackWs w;
    const size_t Bn = B > 0 ? (size_t)B : 1;
    const size_t mc = max_count > 0 ? (size_t)max_count : 1;
    size_t o = 0;
    for (int i = 0; i < 2; ++i) {
        w.xhat[i] = o;
        o += round_up(Bn * d * elem_bytes(dtype));
    }
    const size_t pa = pred_ws_bytes(B, r);
    const size_t ps = round_up(Bn * f * sizeof(float));
    w.a_main = o;
    o += pa;
    w.s_main = o;
    o += ps;
    w.a_side = o;
    o += pa;
    w.s_side = o;
    o += ps;
    const size_t psel = round_up(Bn * csf::select_wide_ws_words(f) * sizeof(uint32_t));
    w.sel_main = o;
    o += psel;
    w.sel_side = o;
    o += psel;
    for (int i = 0; i < 2; ++i) {
        w.idx[i] = o;
        o += round_up(Bn * mc * sizeof(int32_t));
        w.count[i] = o;
        o += round_up(Bn * sizeof(int32_t));
    }
    w.sync = o;   // counters of the one-kernel FFN (single token)
    o += round_up((size_t)fused_sync_words() * sizeof(uint32_t));
    w.ffn = o;
    w.total = o + ffn_ws(B > 0 ? B : 1, d, dtype, max_count).total;
    return w;
}

char *at(void *ws, size_t off) { return static_cast<char *>(ws) + off; }

// top-k of a few tokens with many scores runs over many workgroups and needs a counter block
size_t select_ws_bytes(int B, int f, int k)
{
    if (!csf::select_wide_used(B, f, k))
        return 0;
    return round_up((size_t)B * csf::select_wide_ws_words(f) * sizeof(uint32_t));
}

int check_ws(void *ws, size_t ws_bytes, size_t need)
{
    if (need == 0)
        return CSF_OK;
    if (ws_bytes < need)
        return fail(CSF_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes,
                    need);
    return check_ptr(ws, "ws", true);
}

#define CHECK_WS(ws, bytes, need)                          \
    do {                                                   \
        int _s = check_ws((ws), (bytes), (need));          \
        if (_s != CSF_OK)                                  \
            return _s;                                     \
    } while (0)

int validate_ffn(const void *x, int B, int d, int f, int act, int dtype, const void *W1,
                 const float *b1, const void *Wup, const void *W2T)
{
    REQUIRE(B >= 0, CSF_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    REQUIRE(f > 0, CSF_ERR_INVALID_ARG, "f must be positive (got %d)", f);
    REQUIRE(valid_dtype(dtype), CSF_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    REQUIRE(act >= CSF_ACT_RELU && act <= CSF_ACT_SWIGLU, CSF_ERR_INVALID_ARG,
            "unknown activation %d", act);
    CHECK_ROW(d, dtype, kMaxRowChunks);
    CHECK_PTR(x, B > 0);
    CHECK_PTR(W1, true);
    CHECK_PTR(W2T, true);
    CHECK_PTR(b1, false);
    if (act == CSF_ACT_REGLU || act == CSF_ACT_SWIGLU) {
        CHECK_PTR(Wup, true);
    } else {
        REQUIRE(Wup == nullptr, CSF_ERR_INVALID_ARG, "Wup must be NULL for the ungated forms");
    }
    return CSF_OK;
}

int validate_union(const void *X, int B, int d, int f, int act, int dtype, const void *W1,
                   const float *b1, const void *Wup, const void *W2T, int semantics, int path,
                   const float *Y, const int32_t *union_count)
{
    int s = validate_ffn(X, B, d, f, act, dtype, W1, b1, Wup, W2T);
    if (s != CSF_OK)
        return s;
    REQUIRE(B <= csf::kMaxUnionBatch, CSF_ERR_UNSUPPORTED,
            "B = %d exceeds the library's limit of %d tokens per batched call", B,
            csf::kMaxUnionBatch);
    REQUIRE(f <= csf::select_max_f(), CSF_ERR_UNSUPPORTED, "f = %d exceeds the library's limit %d",
            f, csf::select_max_f());
    REQUIRE(semantics == CSF_SEM_PER_TOKEN || semantics == CSF_SEM_UNION, CSF_ERR_INVALID_ARG,
            "unknown semantics %d", semantics);
    REQUIRE(path == CSF_PATH_AUTO || path == CSF_PATH_GATHER || path == CSF_PATH_MFMA,
            CSF_ERR_INVALID_ARG, "unknown path %d", path);
    CHECK_PTR(Y, B > 0);
    CHECK_PTR(union_count, false);
    REQUIRE(path != CSF_PATH_MFMA || csf::union_mfma_supported(dtype, d, B > 0 ? B : 1),
            CSF_ERR_UNSUPPORTED,
            "the matrix-core path needs a 16-bit dtype and d %% 256 == 0 (dtype %d, d = %d)", dtype,
            d);
    return CSF_OK;
}

bool choose_union_path(int path, int dtype, int d, int B)
{
    if (path == CSF_PATH_MFMA)
        return true;
    return path == CSF_PATH_AUTO && csf::union_mfma_supported(dtype, d, B > 0 ? B : 1) &&
           B >= kMfmaMinBatch;
}

int enqueue_union(const void *X, int B, int d, int f, int act, int dtype, const void *W1,
                  const float *b1, const void *Wup, const void *W2T, const uint32_t *bitmaps,
                  int semantics, bool mfma, float *Y, int32_t *union_count, void *ws,
                  const UnionWs &w, int cus, hipStream_t st, csf::Trace *tr)
{
    csf::UnionArgs a;
    a.cus = cus;
    a.dtype = dtype;
    a.act = act;
    a.per_token = semantics == CSF_SEM_PER_TOKEN;
    a.mfma = mfma;
    a.X = X;
    a.B = B;
    a.d = d;
    a.f = f;
    a.W1 = W1;
    a.Wup = Wup;
    a.W2T = W2T;
    a.b1 = b1;
    a.bitmaps = bitmaps;
    a.Y = Y;
    a.ucount_out = union_count;
    a.ulist = reinterpret_cast<int32_t *>(at(ws, w.ulist));
    a.ucount = reinterpret_cast<int32_t *>(at(ws, w.ucount));
    a.h32 = reinterpret_cast<float *>(at(ws, w.h));
    a.hmax = reinterpret_cast<uint32_t *>(at(ws, w.hmax));
    a.hs = (int)csf::union_h_stride(f);
    a.partials = reinterpret_cast<float *>(at(ws, w.partials));
    return hip_status(csf::launch_union_ffn(a, st, tr), "batched union FFN launch");
}

// The look-ahead stack's four events ("layer input ready" and "selection ready", each
// double-buffered across consecutive layers), created on the handle's first use of them.
int stack_events(csf_handle h, hipEvent_t ev_x[2], hipEvent_t ev_s[2])
{
    for (int i = 0; i < 4; ++i) {
        if (!h->stack_ev[i]) {
            hipError_t e = hipEventCreateWithFlags(&h->stack_ev[i], hipEventDisableTiming);
            if (e != hipSuccess) {
                h->stack_ev[i] = nullptr;
                return hip_status(e, "hipEventCreateWithFlags");
            }
        }
    }
    ev_x[0] = h->stack_ev[0];
    ev_x[1] = h->stack_ev[1];
    ev_s[0] = h->stack_ev[2];
    ev_s[1] = h->stack_ev[3];
    return CSF_OK;
}

// The stack's graph form is captured on a stream of the handle's own (the caller's stream may be
// the legacy default stream, which cannot be captured) and launched on the caller's stream.
int capture_stream(csf_handle h, hipStream_t *out)
{
    if (!h->capture) {
        hipError_t e = hipStreamCreateWithFlags(&h->capture, hipStreamNonBlocking);
        if (e != hipSuccess) {
            h->capture = nullptr;
            return hip_status(e, "hipStreamCreateWithFlags");
        }
    }
    *out = h->capture;
    return CSF_OK;
}

int enqueue_stack(csf_handle h, const csf_layer_weights *layers, int L, int d, int f, int r,
                  int act, int dtype, float *x, int B, int sched, int k, float tau, int norm,
                  float eps, float *x_log, void *xhat_log, int32_t *idx_log, int32_t *count_log,
                  void *ws, hipStream_t st, hipStream_t side, bool captured)
{
    const int max_count = k >= 0 ? k : f;
    const int stride = max_count > 0 ? max_count : 1;
    StackWs w = stack_ws(B, d, f, r, max_count, dtype);
    const bool ahead = sched == CSF_STACK_LOOKAHEAD;
    hipEvent_t ev_x[2] = {nullptr, nullptr}, ev_s[2] = {nullptr, nullptr};
    if (ahead) {
        int s = stack_events(h, ev_x, ev_s);
        if (s != CSF_OK)
            return s;
    }
    const size_t es = elem_bytes(dtype);
    FfnWs fw = ffn_ws(B, d, dtype, max_count);
    // one token without the post-gate skip: each block's FFN is the one-kernel form, whose
    // hand-over state the block's normalisation kernel prepares -- except in a captured look-ahead
    // schedule, where the next block's predictor runs beside the FFN: there the one-kernel form's
    // waiting workgroups share the CUs with the predictor and it gains nothing (measured at the
    // OPT-30B shape, 48 blocks: 2.34-2.49 ms per token against 2.32-2.37 with the three-kernel
    // FFN), while the synchronous schedule gains about 0.1 ms (2.73 against 2.83) and the eager
    // look-ahead schedule, bound by the host's enqueue, saves two launches per block
    const bool fused = B == 1 && !(h->ffn_flags & CSF_FFN_SKIP_ZERO_H) && !(ahead && captured);
    uint32_t *sync = reinterpret_cast<uint32_t *>(at(ws, w.sync));
    float *hbuf = reinterpret_cast<float *>(at(ws, w.ffn + fw.h));

    auto sel_idx = [&](int l) {
        return idx_log ? idx_log + (size_t)l * B * stride
                       : reinterpret_cast<int32_t *>(at(ws, w.idx[l & 1]));
    };
    auto sel_count = [&](int l) {
        return count_log ? count_log + (size_t)l * B
                         : reinterpret_cast<int32_t *>(at(ws, w.count[l & 1]));
    };
    // predictor of layer `l` applied to `xh`, then the selection, on stream `q`
    auto predict_select = [&](int l, const void *xh, hipStream_t q, bool on_side) -> int {
        float *a = reinterpret_cast<float *>(at(ws, on_side ? w.a_side : w.a_main));
        float *sc = reinterpret_cast<float *>(at(ws, on_side ? w.s_side : w.s_main));
        const bool wide = k >= 0 && csf::select_wide_used(B, f, k);
        uint32_t *selws = reinterpret_cast<uint32_t *>(at(ws, on_side ? w.sel_side : w.sel_main));
        bool zeroed = false;
        // the clear covers token 0's counter block: only a single token can skip the clear kernel
        hipError_t e = enqueue_predict(dtype, xh, B, d, layers[l].V, r, layers[l].U, f, sc, a, q,
                                       nullptr, h, on_side, wide && B == 1 ? selws : nullptr,
                                       wide && B == 1 ? csf::select_wide_zero_words() : 0, &zeroed);
        if (e == hipSuccess) {
            if (wide)
                e = csf::launch_select_topk_wide(sc, B, f, k, sel_idx(l), stride, sel_count(l),
                                                 nullptr, selws, zeroed, q);
            else if (k >= 0)
                e = csf::launch_select_topk(sc, B, f, k, sel_idx(l), stride, sel_count(l), nullptr, q);
            else
                e = csf::launch_select_threshold(sc, B, f, tau, sel_idx(l), stride, sel_count(l),
                                                 nullptr, q);
        }
        return hip_status(e, "stack predictor/selection launch");
    };

    for (int l = 0; l < L; ++l) {
        void *xh = at(ws, w.xhat[l & 1]);
        hipError_t e = csf::launch_rms_norm(
            dtype, x, B, d, eps, norm, xh, x_log ? x_log + (size_t)l * B * d : nullptr,
            xhat_log ? static_cast<char *>(xhat_log) + (size_t)l * B * d * es : nullptr, st,
            fused ? sync : nullptr, fused_sync_words(),
            fused ? reinterpret_cast<uint32_t *>(hbuf) : nullptr, max_count);
        if (e != hipSuccess)
            return hip_status(e, "stack normalisation launch");
        int s = CSF_OK;
        if (!ahead || l == 0)
            s = predict_select(l, xh, st, false);
        if (s != CSF_OK)
            return s;
        if (ahead && l + 1 < L) {
            // layer l+1's set from this layer's input, on the side stream, while this layer runs
            e = hipEventRecord(ev_x[l & 1], st);
            if (e == hipSuccess)
                e = hipStreamWaitEvent(side, ev_x[l & 1], 0);
            if (e != hipSuccess)
                return hip_status(e, "stack event");
            s = predict_select(l + 1, xh, side, true);
            if (s != CSF_OK)
                return s;
            e = hipEventRecord(ev_s[(l + 1) & 1], side);
            if (e != hipSuccess)
                return hip_status(e, "stack event");
        }
        if (ahead && l > 0) {
            e = hipStreamWaitEvent(st, ev_s[l & 1], 0);
            if (e != hipSuccess)
                return hip_status(e, "stack event");
        }
        csf::FfnArgs fa;
        fa.dtype = dtype;
        fa.act = act;
        fa.x = xh;
        fa.B = B;
        fa.d = d;
        fa.f = f;
        fa.W1 = layers[l].W1;
        fa.Wup = layers[l].Wup;
        fa.W2T = layers[l].W2T;
        fa.b1 = layers[l].b1;
        fa.idx = sel_idx(l);
        fa.idx_stride = stride;
        fa.count = k >= 0 ? nullptr : sel_count(l);
        fa.max_count = max_count;
        fa.h = hbuf;
        fa.h_stride = stride;
        fa.y = x;
        fa.partials = reinterpret_cast<float *>(at(ws, w.ffn + fw.partials));
        fa.accumulate = 1;
        fa.skip_zero = (h->ffn_flags & CSF_FFN_SKIP_ZERO_H) ? 1 : 0;
        fa.gate_tau = h->gate_tau;
        e = fused ? csf::launch_ffn_fused(fa, sync, st) : csf::launch_ffn(fa, st);
        if (e != hipSuccess)
            return hip_status(e, "stack FFN launch");
    }
    return ok();
}



// ---- attention-head sparsity ---------------------------------------------------------------------
struct AttnWs {
    size_t lnew, q, part, rows, hv, rcount, ffn, a, scores, heads, count, total;
};
AttnWs attn_ws(int d, int H, int dh, int r, int Tmax, int max_heads, int dtype, bool layer)
{
    AttnWs w{};
    const size_t mh = max_heads > 0 ? (size_t)max_heads : 1;
    const int max_rows = max_heads * dh;
    size_t o = 0;
    w.lnew = o;
    o += round_up(mh * sizeof(int32_t));
    w.q = o;
    o += round_up(mh * dh * sizeof(float));
    w.part = o;
    o += round_up(mh * csf::attn_num_splits(Tmax) * (size_t)(dh + 2) * sizeof(float));
    w.rows = o;
    o += round_up(mh * dh * sizeof(int32_t));
    w.hv = o;
    o += round_up(mh * dh * sizeof(float));
    w.rcount = o;
    o += kAlign;
    w.ffn = o;
    o += round_up((size_t)csf::ffn_num_chunks(d, dtype, max_rows) * d * sizeof(float));
    if (layer) {
        w.a = o;
        o += pred_ws_bytes(1, r);
        w.scores = o;
        o += round_up((size_t)H * sizeof(float));
        w.heads = o;
        o += round_up((size_t)H * sizeof(int32_t));
        w.count = o;
        o += kAlign;
    }
    w.total = o;
    return w;
}

int validate_attention(const void *x, int d, int H, int dh, int dtype, const void *Wq,
                       const void *Wk, const void *Wv, const float *bq, const float *bk,
                       const float *bv, const void *WoT, const void *Kc, const void *Vc, int Tmax,
                       const int32_t *len, int kv_all, const float *o, const float *y)
{
    REQUIRE(valid_dtype(dtype), CSF_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    CHECK_ROW(d, dtype, kMaxRowChunks);
    REQUIRE(H > 0, CSF_ERR_INVALID_ARG, "H must be positive (got %d)", H);
    REQUIRE(dh > 0, CSF_ERR_INVALID_ARG, "dh must be positive (got %d)", dh);
    REQUIRE(csf::attn_head_dim_supported(dtype, dh), CSF_ERR_UNSUPPORTED,
            "dh = %d: a cached row must be 32, 64, 128, 256 or 512 bytes", dh);
    REQUIRE((long)H * dh <= csf::ffn_max_count(), CSF_ERR_UNSUPPORTED,
            "H * dh = %ld exceeds the library's limit %d", (long)H * dh, csf::ffn_max_count());
    REQUIRE(Tmax > 0, CSF_ERR_INVALID_ARG, "Tmax must be positive (got %d)", Tmax);
    REQUIRE(Tmax <= csf::attn_max_cache(), CSF_ERR_UNSUPPORTED,
            "Tmax = %d exceeds the library's limit %d", Tmax, csf::attn_max_cache());
    REQUIRE(kv_all == 0 || kv_all == 1, CSF_ERR_INVALID_ARG, "kv_all must be 0 or 1");
    CHECK_PTR(x, true);
    CHECK_PTR(Wq, true);
    CHECK_PTR(Wk, true);
    CHECK_PTR(Wv, true);
    CHECK_PTR(WoT, true);
    CHECK_PTR(bq, false);
    CHECK_PTR(bk, false);
    CHECK_PTR(bv, false);
    CHECK_PTR(Kc, true);
    CHECK_PTR(Vc, true);
    CHECK_PTR(len, true);
    CHECK_PTR(o, false);
    CHECK_PTR(y, true);
    return CSF_OK;
}

int enqueue_attention(const void *x, int d, int H, int dh, int dtype, const void *Wq,
                      const void *Wk, const void *Wv, const float *bq, const float *bk,
                      const float *bv, const void *WoT, void *Kc, void *Vc, int Tmax,
                      int32_t *len, const int32_t *heads, const int32_t *count, int max_heads,
                      int kv_all, float *o, float *y, void *ws, const AttnWs &w, hipStream_t st,
                      csf::Trace *tr)
{
    csf::AttnArgs a;
    a.dtype = dtype;
    a.x = x;
    a.d = d;
    a.H = H;
    a.dh = dh;
    a.Wq = Wq;
    a.Wk = Wk;
    a.Wv = Wv;
    a.WoT = WoT;
    a.bq = bq;
    a.bk = bk;
    a.bv = bv;
    a.Kc = Kc;
    a.Vc = Vc;
    a.Tmax = Tmax;
    a.len = len;
    a.heads = heads;
    a.count = count;
    a.max_heads = max_heads;
    a.kv_all = kv_all;
    a.o = o;
    a.y = y;
    a.lnew = reinterpret_cast<int32_t *>(at(ws, w.lnew));
    a.qbuf = reinterpret_cast<float *>(at(ws, w.q));
    a.part = reinterpret_cast<float *>(at(ws, w.part));
    a.rows = reinterpret_cast<int32_t *>(at(ws, w.rows));
    a.hv = reinterpret_cast<float *>(at(ws, w.hv));
    a.rows_count = reinterpret_cast<int32_t *>(at(ws, w.rcount));
    a.ffn_partials = reinterpret_cast<float *>(at(ws, w.ffn));
    return hip_status(csf::launch_attention_decode(a, st, tr), "attention decode launch");
}

// One token's layer (predict, select, gathered FFN) on validated arguments, in the LayerWs
// layout of `ws`.  Optional outputs: scores, list, count, bitmap (NULL: kept in the workspace or
// not written).
int enqueue_layer1(csf_handle h, const void *x, int d, int f, int r, int act, int dtype, const void *V,
                   const void *U, const void *W1, const float *b1, const void *Wup,
                   const void *W2T, int k, float tau, float *y, float *scores_out,
                   int32_t *idx_out, int32_t *count_out, uint32_t *bitmap, void *ws,
                   const LayerWs &w, int skip_zero, float gate_tau, hipStream_t st,
                   csf::Trace *trp)
{
    const int max_count = k >= 0 ? k : f;
    float *a = reinterpret_cast<float *>(at(ws, w.a));
    float *sc = scores_out ? scores_out : reinterpret_cast<float *>(at(ws, w.scores));
    int32_t *ix = idx_out ? idx_out : reinterpret_cast<int32_t *>(at(ws, w.idx));
    int32_t *cn = count_out ? count_out : reinterpret_cast<int32_t *>(at(ws, w.count));

    const bool wide = k >= 0 && csf::select_wide_used(1, f, k);
    uint32_t *selws = reinterpret_cast<uint32_t *>(at(ws, w.sel));
    // the first kernel clears the gathered FFN's counters and, for the many-workgroup selection,
    // its histogram (the two blocks are adjacent), and marks the FFN's h slots unwritten
    uint32_t *sync = reinterpret_cast<uint32_t *>(at(ws, w.sync));
    FfnWs fw = ffn_ws(1, d, dtype, max_count);
    const bool fused = !skip_zero;
    hipError_t e = csf::launch_pred_down(
        dtype, x, 1, d, V, r, a, st, trp, sync,
        fused_sync_words() + (wide ? csf::select_wide_zero_words() : 0),
        fused ? reinterpret_cast<uint32_t *>(at(ws, w.ffn + fw.h)) : nullptr, max_count);
    if (e != hipSuccess)
        return hip_status(e, "predictor down-projection launch");
    if (f <= csf::kSmallF && !bitmap) {
        // few neurons: the scores and their selection in one kernel
        e = csf::launch_pred_up_select(dtype, a, d, r, U, f, sc, k, tau, ix, cn, st, trp);
    } else {
        e = csf::launch_pred_up(dtype, a, 1, d, r, U, f, sc, st, trp, h->pred_up_grid);
        if (e == hipSuccess && wide)
            e = csf::launch_select_topk_wide(sc, 1, f, k, ix, max_count > 0 ? max_count : 1, cn,
                                             bitmap, selws, true, st, trp);
        else if (e == hipSuccess && k >= 0)
            e = csf::launch_select_topk(sc, 1, f, k, ix, max_count > 0 ? max_count : 1, cn, bitmap,
                                        st, trp);
        else if (e == hipSuccess)
            e = csf::launch_select_threshold(sc, 1, f, tau, ix, f, cn, bitmap, st, trp);
    }
    if (e != hipSuccess)
        return hip_status(e, "predictor / selection launch");

    csf::FfnArgs fa;
    fa.dtype = dtype;
    fa.act = act;
    fa.x = x;
    fa.B = 1;
    fa.d = d;
    fa.f = f;
    fa.W1 = W1;
    fa.Wup = Wup;
    fa.W2T = W2T;
    fa.b1 = b1;
    fa.idx = ix;
    fa.idx_stride = max_count > 0 ? max_count : 1;
    fa.count = k >= 0 ? nullptr : cn;
    fa.max_count = max_count;
    fa.h = reinterpret_cast<float *>(at(ws, w.ffn + fw.h));
    fa.h_stride = max_count > 0 ? max_count : 1;
    fa.y = y;
    fa.partials = reinterpret_cast<float *>(at(ws, w.ffn + fw.partials));
    fa.skip_zero = skip_zero;
    fa.gate_tau = gate_tau;
    if (fused)
        return hip_status(csf::launch_ffn_fused(fa, sync, st, trp), "sparse FFN launch");
    return hip_status(csf::launch_ffn(fa, st, trp), "sparse FFN launch");
}

}  // namespace

extern "C" {

int csf_abi_version(void) { return CSF_ABI_VERSION; }

const char *csf_status_string(int status)
{
    switch (status) {
    case CSF_OK: return "CSF_OK";
    case CSF_ERR_INVALID_ARG: return "CSF_ERR_INVALID_ARG";
    case CSF_ERR_UNSUPPORTED: return "CSF_ERR_UNSUPPORTED";
    case CSF_ERR_MISALIGNED: return "CSF_ERR_MISALIGNED";
    case CSF_ERR_WORKSPACE_TOO_SMALL: return "CSF_ERR_WORKSPACE_TOO_SMALL";
    case CSF_ERR_HIP: return "CSF_ERR_HIP";
    default: return "CSF_ERR_UNKNOWN";
    }
}

const char *csf_last_error(void) { return g_last_error.c_str(); }

int csf_create(csf_handle *out, int device)
{
    REQUIRE(out, CSF_ERR_INVALID_ARG, "out must not be NULL");
    *out = nullptr;
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess)
        return hip_status(e, "hipGetDeviceCount");
    REQUIRE(device >= 0 && device < n, CSF_ERR_INVALID_ARG, "device %d is not in [0, %d)", device,
            n);
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess)
        return hip_status(e, "hipDeviceGetAttribute");
    REQUIRE(cus > 0, CSF_ERR_UNSUPPORTED, "device %d reports %d compute units", device, cus);
    // the static scratch's address on this device, read with the device current
    int prev = -1;
    e = hipGetDevice(&prev);
    if (e != hipSuccess)
        return hip_status(e, "hipGetDevice");
    if (prev != device && (e = hipSetDevice(device)) != hipSuccess)
        return hip_status(e, "hipSetDevice");
    const hipError_t es = csf::scratch_init(device);
    if (prev != device && (e = hipSetDevice(prev)) != hipSuccess)
        return hip_status(e, "hipSetDevice");
    if (es != hipSuccess)
        return hip_status(es, "static scratch address (hipGetSymbolAddress)");
    csf_context *h = new (std::nothrow) csf_context;
    REQUIRE(h, CSF_ERR_INVALID_ARG, "out of host memory");
    h->device = device;
    h->cus = cus;
    // measured on MI355X (256 CUs): the persistent one-token up projection is fastest with the
    // most workgroups resident at once, 8 of 256 threads per CU (2048; 1024 / 512 slower).  On the
    // look-ahead stack's second stream, beside the FFN, 4 per CU: 2.35 ms/token for the 48-layer
    // OPT-30B-shape stack (graph replay) against 2.52 with 8 per CU (it then crowds out the FFN)
    // and 2.42 / 2.37 / 2.48 with 3 / 5 / 6 per CU
    h->pred_up_grid = 8 * cus;
    h->pred_up_side_grid = 4 * cus;
    {
        std::lock_guard<std::mutex> lock(g_handles_mu);
        g_handles.insert(h);
    }
    *out = h;
    return ok();
}

int csf_destroy(csf_handle h)
{
    if (!h)
        return ok();
    {
        std::lock_guard<std::mutex> lock(g_handles_mu);
        REQUIRE(g_handles.erase(h) == 1, CSF_ERR_INVALID_ARG, "not a live handle");
    }
    int prev = -1;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(h->device);
    if (h->graph)
        (void)hipGraphExecDestroy(h->graph);
    for (hipEvent_t ev : h->stack_ev)
        if (ev)
            (void)hipEventDestroy(ev);
    if (h->capture)
        (void)hipStreamDestroy(h->capture);
    if (prev >= 0)
        (void)hipSetDevice(prev);
    delete h;
    return ok();
}

int csf_get_device_info(csf_handle h, int *device, int *compute_units)
{
    REQUIRE(is_live(h), CSF_ERR_INVALID_ARG, "handle is NULL or not a live handle");
    if (device)
        *device = h->device;
    if (compute_units)
        *compute_units = h->cus;
    return ok();
}

int csf_set_ffn_flags(csf_handle h, int flags)
{
    REQUIRE(is_live(h), CSF_ERR_INVALID_ARG, "handle is NULL or not a live handle");
    REQUIRE((flags & ~CSF_FFN_SKIP_ZERO_H) == 0, CSF_ERR_INVALID_ARG, "unknown FFN flags 0x%x",
            flags);
    h->ffn_flags = flags;
    return ok();
}

int csf_set_ffn_gate_threshold(csf_handle h, float tau)
{
    REQUIRE(is_live(h), CSF_ERR_INVALID_ARG, "handle is NULL or not a live handle");
    REQUIRE(tau >= 0.0f && tau <= 3.4e38f, CSF_ERR_INVALID_ARG,
            "gate threshold %g must be finite and >= 0", (double)tau);
    h->gate_tau = tau;
    return ok();
}

int csf_set_trace_events(csf_handle h, void *const *events, int n)
{
    REQUIRE(is_live(h), CSF_ERR_INVALID_ARG, "handle is NULL or not a live handle");
    REQUIRE(n >= 0 && n <= 16, CSF_ERR_INVALID_ARG, "n = %d must be in [0, 16]", n);
    REQUIRE(n == 0 || events, CSF_ERR_INVALID_ARG, "events must not be NULL when n > 0");
    for (int i = 0; i < n; ++i)
        REQUIRE(events[i], CSF_ERR_INVALID_ARG, "events[%d] is NULL", i);
    for (int i = 0; i < n; ++i)
        h->trace[i] = static_cast<hipEvent_t>(events[i]);
    h->trace_n = n;
    return ok();
}

size_t csf_attention_workspace_size(int op, int d, int H, int dh, int r, int Tmax, int max_heads,
                                    int dtype)
{
    if (d <= 0 || H <= 0 || dh <= 0 || Tmax <= 0 || max_heads < 0 || max_heads > H ||
        !valid_dtype(dtype))
        return 0;
    if (op == CSF_OP_ATTN_DECODE)
        return attn_ws(d, H, dh, 0, Tmax, max_heads, dtype, false).total;
    if (op == CSF_OP_ATTN_LAYER)
        return r > 0 ? attn_ws(d, H, dh, r, Tmax, max_heads, dtype, true).total : 0;
    return 0;
}

size_t csf_workspace_size(csf_handle h, int op, int B, int d, int f, int r, int max_count,
                          int dtype)
{
    const int cus = sizing_cus(h);
    if (B < 0 || d <= 0 || f <= 0 || !valid_dtype(dtype) || max_count < 0)
        return 0;
    switch (op) {
    case CSF_OP_PREDICT:
        return r > 0 ? predict_ws(B, r).total : 0;
    case CSF_OP_SELECT_TOPK:
        return select_ws_bytes(B, f, max_count);
    case CSF_OP_SELECT_THRESHOLD:
        return 0;
    case CSF_OP_SPARSE_FFN:
        return ffn_ws(B, d, dtype, max_count).total;
    case CSF_OP_DENSE_FFN:
        return ffn_ws(B, d, dtype, f).total;
    case CSF_OP_LAYER:
        return r > 0 ? layer_ws(d, f, r, max_count, dtype).total : 0;
    case CSF_OP_BATCHED_UNION:
        return union_ws(B, d, f, dtype, cus).total;
    case CSF_OP_BATCHED_LAYER:
        return r > 0 ? batched_layer_ws(B, d, f, r, max_count, dtype, cus).total : 0;
    case CSF_OP_STACK:
        return r > 0 ? stack_ws(B, d, f, r, max_count, dtype).total : 0;
    default:
        return 0;
    }
}

int csf_predict_active(csf_handle h, const void *x, int B, int d, const void *V, int r,
                       const void *U, int f, int dtype, float *scores, void *ws, size_t ws_bytes,
                       void *stream)
{
    REQUIRE(B >= 0, CSF_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    REQUIRE(f > 0, CSF_ERR_INVALID_ARG, "f must be positive (got %d)", f);
    REQUIRE(valid_dtype(dtype), CSF_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    CHECK_ROW(d, dtype, kMaxRowChunks);
    CHECK_ROW(r, dtype, kMaxPredChunks);
    CHECK_PTR(x, B > 0);
    CHECK_PTR(V, true);
    CHECK_PTR(U, true);
    CHECK_PTR(scores, B > 0);
    if (B == 0)
        return ok();
    PredictWs w = predict_ws(B, r);
    CHECK_WS(ws, ws_bytes, w.total);
    CHECK_HANDLE(h);
    hipStream_t st = static_cast<hipStream_t>(stream);
    float *a = reinterpret_cast<float *>(at(ws, w.a));
    return hip_status(enqueue_predict(dtype, x, B, d, V, r, U, f, scores, a, st, nullptr, h),
                      "predictor launch");
}

int csf_select_topk(csf_handle h, const float *scores, int B, int f, int k, int32_t *idx,
                    int32_t *count, uint32_t *bitmap, void *ws, size_t ws_bytes, void *stream)
{
    REQUIRE(B >= 0, CSF_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    REQUIRE(f > 0, CSF_ERR_INVALID_ARG, "f must be positive (got %d)", f);
    REQUIRE(k >= 0 && k <= f, CSF_ERR_INVALID_ARG, "k = %d is outside [0, f = %d]", k, f);
    REQUIRE(f <= csf::select_max_f(), CSF_ERR_UNSUPPORTED, "f = %d exceeds the library's limit %d",
            f, csf::select_max_f());
    CHECK_PTR(scores, B > 0);
    CHECK_PTR(idx, B > 0 && k > 0);
    CHECK_PTR(count, false);
    CHECK_PTR(bitmap, false);
    if (B == 0)
        return ok();
    if (csf::select_wide_used(B, f, k)) {
        CHECK_WS(ws, ws_bytes, select_ws_bytes(B, f, k));
        CHECK_HANDLE(h);
        return hip_status(csf::launch_select_topk_wide(scores, B, f, k, idx, k, count, bitmap,
                                                       static_cast<uint32_t *>(ws), false,
                                                       static_cast<hipStream_t>(stream)),
                          "top-k selection launch");
    }
    CHECK_HANDLE(h);
    return hip_status(csf::launch_select_topk(scores, B, f, k, idx, k > 0 ? k : 1, count, bitmap,
                                              static_cast<hipStream_t>(stream)),
                      "top-k selection launch");
}

int csf_select_threshold(csf_handle h, const float *scores, int B, int f, float tau,
                         int32_t *idx, int32_t *count, uint32_t *bitmap, void *ws, size_t ws_bytes,
                         void *stream)
{
    (void)ws;
    (void)ws_bytes;
    REQUIRE(B >= 0, CSF_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    REQUIRE(f > 0, CSF_ERR_INVALID_ARG, "f must be positive (got %d)", f);
    REQUIRE(f <= csf::select_max_f(), CSF_ERR_UNSUPPORTED, "f = %d exceeds the library's limit %d",
            f, csf::select_max_f());
    REQUIRE(tau == tau, CSF_ERR_INVALID_ARG, "tau must not be NaN");
    CHECK_PTR(scores, B > 0);
    CHECK_PTR(idx, B > 0);
    CHECK_PTR(count, B > 0);
    CHECK_PTR(bitmap, false);
    if (B == 0)
        return ok();
    CHECK_HANDLE(h);
    return hip_status(csf::launch_select_threshold(scores, B, f, tau, idx, f, count, bitmap,
                                                   static_cast<hipStream_t>(stream)),
                      "threshold selection launch");
}

int csf_sparse_ffn(csf_handle hd, const void *x, int B, int d, int f, int act, int dtype,
                   const void *W1, const float *b1, const void *Wup, const void *W2T,
                   const int32_t *idx, int idx_stride, const int32_t *count, int max_count,
                   float *h, float *y, void *ws, size_t ws_bytes, void *stream)
{
    int s = validate_ffn(x, B, d, f, act, dtype, W1, b1, Wup, W2T);
    if (s != CSF_OK)
        return s;
    REQUIRE(max_count >= 0 && max_count <= idx_stride, CSF_ERR_INVALID_ARG,
            "max_count = %d must be in [0, idx_stride = %d]", max_count, idx_stride);
    REQUIRE(max_count <= csf::ffn_max_count(), CSF_ERR_UNSUPPORTED,
            "max_count = %d exceeds the library's limit %d", max_count, csf::ffn_max_count());
    CHECK_PTR(idx, B > 0 && max_count > 0);
    CHECK_PTR(count, false);
    CHECK_PTR(h, false);
    CHECK_PTR(y, B > 0);
    if (B == 0)
        return ok();
    FfnWs w = ffn_ws(B, d, dtype, max_count);
    CHECK_WS(ws, ws_bytes, w.total);
    CHECK_HANDLE(hd);
    csf::FfnArgs a;
    a.dtype = dtype;
    a.act = act;
    a.x = x;
    a.B = B;
    a.d = d;
    a.f = f;
    a.W1 = W1;
    a.Wup = Wup;
    a.W2T = W2T;
    a.b1 = b1;
    a.idx = idx;
    a.idx_stride = idx_stride;
    a.count = count;
    a.max_count = max_count;
    a.h = h ? h : reinterpret_cast<float *>(at(ws, w.h));
    a.h_stride = h ? idx_stride : (max_count > 0 ? max_count : 1);
    a.y = y;
    a.partials = reinterpret_cast<float *>(at(ws, w.partials));
    a.skip_zero = (hd->ffn_flags & CSF_FFN_SKIP_ZERO_H) ? 1 : 0;
    a.gate_tau = hd->gate_tau;
    return hip_status(csf::launch_ffn(a, static_cast<hipStream_t>(stream)), "sparse FFN launch");
}

int csf_dense_ffn(csf_handle h, const void *X, int B, int d, int f, int act, int dtype,
                  const void *W1, const float *b1, const void *Wup, const void *W2T, float *H,
                  float *Y, void *ws, size_t ws_bytes, void *stream)
{
    int s = validate_ffn(X, B, d, f, act, dtype, W1, b1, Wup, W2T);
    if (s != CSF_OK)
        return s;
    REQUIRE(f <= csf::ffn_max_count(), CSF_ERR_UNSUPPORTED, "f = %d exceeds the library's limit %d",
            f, csf::ffn_max_count());
    CHECK_PTR(H, false);
    CHECK_PTR(Y, B > 0);
    if (B == 0)
        return ok();
    FfnWs w = ffn_ws(B, d, dtype, f);
    CHECK_WS(ws, ws_bytes, w.total);
    CHECK_HANDLE(h);
    csf::FfnArgs a;
    a.dtype = dtype;
    a.act = act;
    a.x = X;
    a.B = B;
    a.d = d;
    a.f = f;
    a.W1 = W1;
    a.Wup = Wup;
    a.W2T = W2T;
    a.b1 = b1;
    a.idx = nullptr;
    a.idx_stride = f;
    a.count = nullptr;
    a.max_count = f;
    a.h = H ? H : reinterpret_cast<float *>(at(ws, w.h));
    a.h_stride = f;
    a.y = Y;
    a.partials = reinterpret_cast<float *>(at(ws, w.partials));
    a.skip_zero = (h->ffn_flags & CSF_FFN_SKIP_ZERO_H) ? 1 : 0;
    a.gate_tau = h->gate_tau;
    return hip_status(csf::launch_ffn(a, static_cast<hipStream_t>(stream)), "dense FFN launch");
}

int csf_sparse_ffn_batched_union(csf_handle h, const void *X, int B, int d, int f, int act, int dtype,
                                 const void *W1, const float *b1, const void *Wup,
                                 const void *W2T, const uint32_t *bitmaps, int semantics,
                                 int path, float *Y, int32_t *union_count, int *path_taken,
                                 void *ws, size_t ws_bytes, void *stream)
{
    int s = validate_union(X, B, d, f, act, dtype, W1, b1, Wup, W2T, semantics, path, Y,
                           union_count);
    if (s != CSF_OK)
        return s;
    CHECK_PTR(bitmaps, B > 0);
    const bool mfma = choose_union_path(path, dtype, d, B);
    if (B == 0) {
        if (path_taken)
            *path_taken = mfma ? CSF_PATH_MFMA : CSF_PATH_GATHER;
        return ok();
    }
    UnionWs w = union_ws(B, d, f, dtype, sizing_cus(h));
    CHECK_WS(ws, ws_bytes, w.total);
    CHECK_HANDLE(h);
    csf::Trace tr = make_trace(h);
    s = enqueue_union(X, B, d, f, act, dtype, W1, b1, Wup, W2T, bitmaps, semantics, mfma, Y,
                      union_count, ws, w, h->cus, static_cast<hipStream_t>(stream),
                      tr.ev ? &tr : nullptr);
    if (s == CSF_OK && path_taken)
        *path_taken = mfma ? CSF_PATH_MFMA : CSF_PATH_GATHER;
    return s;
}

int csf_sparse_ffn_batched_layer(csf_handle h, const void *X, int B, int d, int f, int r, int act,
                                 int dtype,
                                 const void *V, const void *U, const void *W1, const float *b1,
                                 const void *Wup, const void *W2T, int k, float tau,
                                 int semantics, int path, float *Y, uint32_t *bitmaps_out,
                                 int32_t *union_count, int *path_taken, void *ws,
                                 size_t ws_bytes, void *stream)
{
    int s = validate_union(X, B, d, f, act, dtype, W1, b1, Wup, W2T, semantics, path, Y,
                           union_count);
    if (s != CSF_OK)
        return s;
    CHECK_ROW(r, dtype, kMaxPredChunks);
    CHECK_PTR(V, true);
    CHECK_PTR(U, true);
    CHECK_PTR(bitmaps_out, false);
    REQUIRE(k >= -1 && k <= f, CSF_ERR_INVALID_ARG, "k = %d must be -1 (threshold) or in [0, f = %d]",
            k, f);
    REQUIRE(k >= 0 || tau == tau, CSF_ERR_INVALID_ARG, "tau must not be NaN");
    const bool mfma = choose_union_path(path, dtype, d, B);
    if (B == 0) {
        if (path_taken)
            *path_taken = mfma ? CSF_PATH_MFMA : CSF_PATH_GATHER;
        return ok();
    }
    const int max_count = k >= 0 ? k : f;
    BatchedLayerWs w = batched_layer_ws(B, d, f, r, max_count, dtype, sizing_cus(h));
    CHECK_WS(ws, ws_bytes, w.total);
    CHECK_HANDLE(h);
    hipStream_t st = static_cast<hipStream_t>(stream);
    csf::Trace tr = make_trace(h);
    csf::Trace *trp = tr.ev ? &tr : nullptr;
    if (B == 1 && !mfma) {
        // One token on the gather path: its union is its own set, so the single-token layer
        // (selection over many workgroups for large f, the gathered FFN over the token's list)
        // computes the same thing without the union list.  No post-gate skip, as on the union
        // path; the count is the union size.
        s = enqueue_layer1(h, X, d, f, r, act, dtype, V, U, W1, b1, Wup, W2T, k, tau, Y, nullptr,
                           nullptr, union_count, bitmaps_out, ws, layer_ws(d, f, r, max_count, dtype),
                           0, 0.0f, st, trp);
        if (s == CSF_OK && path_taken)
            *path_taken = CSF_PATH_GATHER;
        return s;
    }
    float *a = reinterpret_cast<float *>(at(ws, w.a));
    float *sc = reinterpret_cast<float *>(at(ws, w.scores));
    int32_t *ix = reinterpret_cast<int32_t *>(at(ws, w.idx));
    int32_t *cn = reinterpret_cast<int32_t *>(at(ws, w.count));
    uint32_t *bm = bitmaps_out ? bitmaps_out : reinterpret_cast<uint32_t *>(at(ws, w.bitmap));
    hipError_t e = enqueue_predict(dtype, X, B, d, V, r, U, f, sc, a, st, trp, h);
    if (e != hipSuccess)
        return hip_status(e, "predictor launch");
    const int stride = max_count > 0 ? max_count : 1;
    if (k >= 0)
        e = csf::launch_select_topk(sc, B, f, k, ix, stride, cn, bm, st, trp);
    else
        e = csf::launch_select_threshold(sc, B, f, tau, ix, f, cn, bm, st, trp);
    if (e != hipSuccess)
        return hip_status(e, "selection launch");
    UnionWs uw = union_ws(B, d, f, dtype, h->cus);
    s = enqueue_union(X, B, d, f, act, dtype, W1, b1, Wup, W2T, bm, semantics, mfma, Y,
                      union_count, at(ws, w.uni), uw, h->cus, st, trp);
    if (s == CSF_OK && path_taken)
        *path_taken = mfma ? CSF_PATH_MFMA : CSF_PATH_GATHER;
    return s;
}

int csf_sparse_ffn_layer_hot(csf_handle h, const void *x, int d, int f, int r, int act, int dtype,
                             const void *V, const void *U_cold, const void *W1, const float *b1,
                             const void *Wup, const void *W2T, int hot, int k_cold, float tau,
                             float *y, float *scores_out, int32_t *idx_out, int32_t *count_out,
                             void *ws, size_t ws_bytes, void *stream)
{
    int s = validate_ffn(x, 1, d, f, act, dtype, W1, b1, Wup, W2T);
    if (s != CSF_OK)
        return s;
    REQUIRE(hot >= 0 && hot < f, CSF_ERR_INVALID_ARG,
            "hot = %d must be in [0, f = %d) (a fully hot layer is csf_dense_ffn)", hot, f);
    const int fc = f - hot;
    CHECK_ROW(r, dtype, kMaxPredChunks);
    CHECK_PTR(V, true);
    CHECK_PTR(U_cold, true);
    CHECK_PTR(y, true);
    CHECK_PTR(scores_out, false);
    CHECK_PTR(idx_out, false);
    CHECK_PTR(count_out, false);
    REQUIRE(k_cold >= -1 && k_cold <= fc, CSF_ERR_INVALID_ARG,
            "k_cold = %d must be -1 (threshold) or in [0, f - hot = %d]", k_cold, fc);
    REQUIRE(f <= csf::select_max_f(), CSF_ERR_UNSUPPORTED, "f = %d exceeds the library's limit %d",
            f, csf::select_max_f());
    REQUIRE(k_cold >= 0 || tau == tau, CSF_ERR_INVALID_ARG, "tau must not be NaN");
    const int max_count = hot + (k_cold >= 0 ? k_cold : fc);
    LayerWs w = layer_ws(d, f, r, max_count, dtype);
    CHECK_WS(ws, ws_bytes, w.total);
    CHECK_HANDLE(h);
    hipStream_t st = static_cast<hipStream_t>(stream);
    csf::Trace tr = make_trace(h);
    csf::Trace *trp = tr.ev ? &tr : nullptr;
    float *a = reinterpret_cast<float *>(at(ws, w.a));
    float *sc = scores_out ? scores_out : reinterpret_cast<float *>(at(ws, w.scores));
    int32_t *ix = idx_out ? idx_out : reinterpret_cast<int32_t *>(at(ws, w.idx));
    int32_t *cn = count_out ? count_out : reinterpret_cast<int32_t *>(at(ws, w.count));
    const int stride = max_count > 0 ? max_count : 1;

    // the predictor scores the cold rows only; the list is the hot block, then the selection
    const bool wide = k_cold >= 0 && csf::select_wide_used(1, fc, k_cold);
    uint32_t *selws = reinterpret_cast<uint32_t *>(at(ws, w.sel));
    hipError_t e = csf::launch_pred_down(dtype, x, 1, d, V, r, a, st, trp, wide ? selws : nullptr,
                                         wide ? csf::select_wide_zero_words() : 0);
    if (e == hipSuccess)
        e = csf::launch_pred_up(dtype, a, 1, d, r, U_cold, fc, sc, st, trp, h->pred_up_grid);
    if (e != hipSuccess)
        return hip_status(e, "predictor launch");
    if (wide)
        e = csf::launch_select_topk_wide(sc, 1, fc, k_cold, ix, stride, cn, nullptr, selws, true, st,
                                         trp, hot);
    else if (k_cold >= 0)
        e = csf::launch_select_topk(sc, 1, fc, k_cold, ix, stride, cn, nullptr, st, trp, hot);
    else
        e = csf::launch_select_threshold(sc, 1, fc, tau, ix, stride, cn, nullptr, st, trp, hot);
    if (e != hipSuccess)
        return hip_status(e, "selection launch");

    FfnWs fw = ffn_ws(1, d, dtype, max_count);
    csf::FfnArgs fa;
    fa.dtype = dtype;
    fa.act = act;
    fa.x = x;
    fa.B = 1;
    fa.d = d;
    fa.f = f;
    fa.W1 = W1;
    fa.Wup = Wup;
    fa.W2T = W2T;
    fa.b1 = b1;
    fa.idx = ix;
    fa.idx_stride = stride;
    fa.count = k_cold >= 0 ? nullptr : cn;
    fa.max_count = max_count;
    fa.h = reinterpret_cast<float *>(at(ws, w.ffn + fw.h));
    fa.h_stride = stride;
    fa.y = y;
    fa.partials = reinterpret_cast<float *>(at(ws, w.ffn + fw.partials));
    fa.skip_zero = (h->ffn_flags & CSF_FFN_SKIP_ZERO_H) ? 1 : 0;
    fa.gate_tau = h->gate_tau;
    return hip_status(csf::launch_ffn(fa, st, trp), "sparse FFN launch");
}

int csf_sparse_ffn_layer(csf_handle h, const void *x, int d, int f, int r, int act, int dtype,
                         const void *V, const void *U, const void *W1, const float *b1,
                         const void *Wup, const void *W2T, int k, float tau, float *y,
                         float *scores_out, int32_t *idx_out, int32_t *count_out, void *ws,
                         size_t ws_bytes, void *stream)
{
    int s = validate_ffn(x, 1, d, f, act, dtype, W1, b1, Wup, W2T);
    if (s != CSF_OK)
        return s;
    CHECK_ROW(r, dtype, kMaxPredChunks);
    CHECK_PTR(V, true);
    CHECK_PTR(U, true);
    CHECK_PTR(y, true);
    CHECK_PTR(scores_out, false);
    CHECK_PTR(idx_out, false);
    CHECK_PTR(count_out, false);
    REQUIRE(k >= -1 && k <= f, CSF_ERR_INVALID_ARG, "k = %d must be -1 (threshold) or in [0, f = %d]",
            k, f);
    REQUIRE(f <= csf::select_max_f(), CSF_ERR_UNSUPPORTED, "f = %d exceeds the library's limit %d",
            f, csf::select_max_f());
    REQUIRE(k >= 0 || tau == tau, CSF_ERR_INVALID_ARG, "tau must not be NaN");
    const int max_count = k >= 0 ? k : f;
    LayerWs w = layer_ws(d, f, r, max_count, dtype);
    CHECK_WS(ws, ws_bytes, w.total);
    CHECK_HANDLE(h);
    csf::Trace tr = make_trace(h);
    return enqueue_layer1(h, x, d, f, r, act, dtype, V, U, W1, b1, Wup, W2T, k, tau, y,
                          scores_out, idx_out, count_out, nullptr, ws, w,
                          (h->ffn_flags & CSF_FFN_SKIP_ZERO_H) ? 1 : 0, h->gate_tau,
                          static_cast<hipStream_t>(stream), tr.ev ? &tr : nullptr);
}

int csf_sparse_ffn_layer_noalloc(csf_handle h, const void *x, int d, int f, int r, int act,
                                 int dtype, const void *V, const void *U, const void *W1,
                                 const float *b1, const void *Wup, const void *W2T, int k,
                                 float tau, float *y, float *scores_out, int32_t *idx_out,
                                 int32_t *count_out, void *stream)
{
    int s = validate_ffn(x, 1, d, f, act, dtype, W1, b1, Wup, W2T);
    if (s != CSF_OK)
        return s;
    CHECK_ROW(r, dtype, kMaxPredChunks);
    CHECK_PTR(V, true);
    CHECK_PTR(U, true);
    CHECK_PTR(y, true);
    CHECK_PTR(scores_out, false);
    CHECK_PTR(idx_out, false);
    CHECK_PTR(count_out, false);
    REQUIRE(k >= -1 && k <= f, CSF_ERR_INVALID_ARG, "k = %d must be -1 (threshold) or in [0, f = %d]",
            k, f);
    REQUIRE(f <= csf::select_max_f(), CSF_ERR_UNSUPPORTED, "f = %d exceeds the library's limit %d",
            f, csf::select_max_f());
    REQUIRE(k >= 0 || tau == tau, CSF_ERR_INVALID_ARG, "tau must not be NaN");
    const int max_count = k >= 0 ? k : f;
    LayerWs w = layer_ws(d, f, r, max_count, dtype);
    REQUIRE(w.total <= csf::scratch_bytes(), CSF_ERR_UNSUPPORTED,
            "this layer needs %zu bytes of scratch; the library's static scratch holds %zu "
            "(csf_sparse_ffn_layer takes a caller workspace of any size)",
            w.total, csf::scratch_bytes());
    CHECK_HANDLE(h);
    void *ws = csf::scratch_ptr(h->device);
    REQUIRE(ws, CSF_ERR_INVALID_ARG, "the static scratch of device %d has no address", h->device);
    csf::Trace tr = make_trace(h);
    return enqueue_layer1(h, x, d, f, r, act, dtype, V, U, W1, b1, Wup, W2T, k, tau, y,
                          scores_out, idx_out, count_out, nullptr, ws, w,
                          (h->ffn_flags & CSF_FFN_SKIP_ZERO_H) ? 1 : 0, h->gate_tau,
                          static_cast<hipStream_t>(stream), tr.ev ? &tr : nullptr);
}

int csf_stack_forward(csf_handle h, const csf_layer_weights *layers, int L, int d, int f, int r,
                      int act,
                      int dtype, float *x, int B, int mode, int k, float tau, int norm, float eps,
                      float *x_log, void *xhat_log, int32_t *idx_log, int32_t *count_log,
                      void *ws, size_t ws_bytes, void *stream, void *side_stream)
{
    REQUIRE(L >= 0, CSF_ERR_INVALID_ARG, "L must be >= 0 (got %d)", L);
    REQUIRE(L == 0 || layers, CSF_ERR_INVALID_ARG, "layers must not be NULL when L > 0");
    const int sched = mode & ~CSF_STACK_GRAPH;
    REQUIRE(sched == CSF_STACK_SYNC || sched == CSF_STACK_LOOKAHEAD, CSF_ERR_INVALID_ARG,
            "unknown stack mode %d", mode);
    REQUIRE(norm == 0 || norm == 1, CSF_ERR_INVALID_ARG, "norm must be 0 or 1 (got %d)", norm);
    REQUIRE(eps >= 0.0f && eps < 1e30f, CSF_ERR_INVALID_ARG, "eps must be finite and >= 0");
    REQUIRE(sched == CSF_STACK_SYNC || (side_stream && side_stream != stream), CSF_ERR_INVALID_ARG,
            "look-ahead needs a side stream distinct from the main stream");
    for (int l = 0; l < L; ++l) {
        int s = validate_ffn(x, B, d, f, act, dtype, layers[l].W1, layers[l].b1, layers[l].Wup,
                             layers[l].W2T);
        if (s != CSF_OK)
            return fail(s, "layer %d: %s", l, g_last_error.c_str());
        s = check_ptr(layers[l].V, "V", true);
        if (s == CSF_OK)
            s = check_ptr(layers[l].U, "U", true);
        if (s != CSF_OK)
            return fail(s, "layer %d: %s", l, g_last_error.c_str());
    }
    CHECK_ROW(r, dtype, kMaxPredChunks);
    REQUIRE(B >= 0, CSF_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    REQUIRE(k >= -1 && k <= f, CSF_ERR_INVALID_ARG, "k = %d must be -1 (threshold) or in [0, f = %d]",
            k, f);
    REQUIRE(k >= 0 || tau == tau, CSF_ERR_INVALID_ARG, "tau must not be NaN");
    REQUIRE(f > 0 && f <= csf::select_max_f(), CSF_ERR_UNSUPPORTED,
            "f = %d is outside the library's range [1, %d]", f, csf::select_max_f());
    CHECK_PTR(x, B > 0 && L > 0);
    CHECK_PTR(x_log, false);
    CHECK_PTR(xhat_log, false);
    CHECK_PTR(idx_log, false);
    CHECK_PTR(count_log, false);
    if (L == 0 || B == 0)
        return ok();
    const int max_count = k >= 0 ? k : f;
    CHECK_WS(ws, ws_bytes, stack_ws(B, d, f, r, max_count, dtype).total);
    CHECK_HANDLE(h);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!(mode & CSF_STACK_GRAPH))
        return enqueue_stack(h, layers, L, d, f, r, act, dtype, x, B, sched, k, tau, norm, eps,
                             x_log, xhat_log, idx_log, count_log, ws, st,
                             static_cast<hipStream_t>(side_stream), false);

    // graph replay: the whole stack as one launch, captured on first use for these arguments
    hipError_t e = hipSuccess;
    uint64_t key = 1469598103934665603ull;
    auto mix = [&](const void *p, size_t n) {
        const unsigned char *c = static_cast<const unsigned char *>(p);
        for (size_t i = 0; i < n; ++i)
            key = (key ^ c[i]) * 1099511628211ull;
    };
    mix(layers, sizeof(csf_layer_weights) * (size_t)L);
    const void *ptrs[] = {x, x_log, xhat_log, idx_log, count_log, ws, stream, side_stream};
    mix(ptrs, sizeof ptrs);
    const int ints[] = {L, d, f, r, act, dtype, B, mode, k, norm, h->ffn_flags};
    mix(ints, sizeof ints);
    mix(&tau, sizeof tau);
    mix(&eps, sizeof eps);
    mix(&h->gate_tau, sizeof h->gate_tau);
    mix(&ws_bytes, sizeof ws_bytes);
    if (!(h->graph && h->graph_key == key)) {
        if (h->graph) {
            (void)hipGraphExecDestroy(h->graph);
            h->graph = nullptr;
        }
        hipStream_t cap = nullptr;
        int s1 = capture_stream(h, &cap);
        if (s1 != CSF_OK)
            return s1;
        e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess)
            return hip_status(e, "hipStreamBeginCapture");
        const int s2 = enqueue_stack(h, layers, L, d, f, r, act, dtype, x, B, sched, k, tau, norm,
                                     eps, x_log, xhat_log, idx_log, count_log, ws, cap,
                                     static_cast<hipStream_t>(side_stream), true);
        const std::string msg = g_last_error;
        hipGraph_t graph = nullptr;
        e = hipStreamEndCapture(cap, &graph);
        if (s2 != CSF_OK) {
            if (graph)
                (void)hipGraphDestroy(graph);
            return fail(s2, "%s", msg.c_str());
        }
        if (e != hipSuccess)
            return hip_status(e, "hipStreamEndCapture");
        e = hipGraphInstantiateWithFlags(&h->graph, graph, 0);
        (void)hipGraphDestroy(graph);
        if (e != hipSuccess) {
            h->graph = nullptr;
            return hip_status(e, "hipGraphInstantiateWithFlags");
        }
        h->graph_key = key;
    }
    return hip_status(hipGraphLaunch(h->graph, st), "hipGraphLaunch");
}

int csf_sparse_attention_decode(csf_handle h, const void *x, int d, int H, int dh, int dtype,
                                const void *Wq,
                                const void *Wk, const void *Wv, const float *bq, const float *bk,
                                const float *bv, const void *WoT, void *Kc, void *Vc, int Tmax,
                                int32_t *len, const int32_t *heads, const int32_t *count,
                                int max_heads, int kv_all, float *o, float *y, void *ws,
                                size_t ws_bytes, void *stream)
{
    int s = validate_attention(x, d, H, dh, dtype, Wq, Wk, Wv, bq, bk, bv, WoT, Kc, Vc, Tmax, len,
                               kv_all, o, y);
    if (s != CSF_OK)
        return s;
    CHECK_PTR(heads, false);
    CHECK_PTR(count, false);
    if (heads)
        REQUIRE(max_heads >= 0 && max_heads <= H, CSF_ERR_INVALID_ARG,
                "max_heads = %d must be in [0, H = %d]", max_heads, H);
    else
        REQUIRE(max_heads == H && !count, CSF_ERR_INVALID_ARG,
                "without a head list every head is computed: max_heads must be H and count NULL");
    AttnWs w = attn_ws(d, H, dh, 0, Tmax, max_heads, dtype, false);
    CHECK_WS(ws, ws_bytes, w.total);
    CHECK_HANDLE(h);
    csf::Trace tr = make_trace(h);
    return enqueue_attention(x, d, H, dh, dtype, Wq, Wk, Wv, bq, bk, bv, WoT, Kc, Vc, Tmax, len,
                             heads, count, max_heads, kv_all, o, y, ws, w,
                             static_cast<hipStream_t>(stream), tr.ev ? &tr : nullptr);
}

int csf_sparse_attention_layer(csf_handle h, const void *x, int d, int H, int dh, int r,
                               int dtype,
                               const void *Vp, const void *Up, const void *Wq, const void *Wk,
                               const void *Wv, const float *bq, const float *bk, const float *bv,
                               const void *WoT, void *Kc, void *Vc, int Tmax, int32_t *len, int k,
                               float tau, int kv_all, float *scores_out, int32_t *heads_out,
                               int32_t *count_out, float *o, float *y, void *ws, size_t ws_bytes,
                               void *stream)
{
    int s = validate_attention(x, d, H, dh, dtype, Wq, Wk, Wv, bq, bk, bv, WoT, Kc, Vc, Tmax, len,
                               kv_all, o, y);
    if (s != CSF_OK)
        return s;
    CHECK_ROW(r, dtype, kMaxPredChunks);
    CHECK_PTR(Vp, true);
    CHECK_PTR(Up, true);
    CHECK_PTR(scores_out, false);
    CHECK_PTR(heads_out, false);
    CHECK_PTR(count_out, false);
    REQUIRE(k >= -1 && k <= H, CSF_ERR_INVALID_ARG, "k = %d must be -1 (threshold) or in [0, H = %d]",
            k, H);
    REQUIRE(H <= csf::select_max_f(), CSF_ERR_UNSUPPORTED, "H = %d exceeds the library's limit %d",
            H, csf::select_max_f());
    REQUIRE(k >= 0 || tau == tau, CSF_ERR_INVALID_ARG, "tau must not be NaN");
    const int max_heads = k >= 0 ? k : H;
    AttnWs w = attn_ws(d, H, dh, r, Tmax, max_heads, dtype, true);
    CHECK_WS(ws, ws_bytes, w.total);
    CHECK_HANDLE(h);
    hipStream_t st = static_cast<hipStream_t>(stream);
    csf::Trace tr = make_trace(h);
    csf::Trace *trp = tr.ev ? &tr : nullptr;
    float *a = reinterpret_cast<float *>(at(ws, w.a));
    float *sc = scores_out ? scores_out : reinterpret_cast<float *>(at(ws, w.scores));
    int32_t *hd = heads_out ? heads_out : reinterpret_cast<int32_t *>(at(ws, w.heads));
    int32_t *cn = count_out ? count_out : reinterpret_cast<int32_t *>(at(ws, w.count));
    hipError_t e;
    if (H <= csf::kSmallF) {
        // the usual case: the head scores and their selection in one kernel
        e = csf::launch_pred_down(dtype, x, 1, d, Vp, r, a, st, trp);
        if (e == hipSuccess)
            e = csf::launch_pred_up_select(dtype, a, d, r, Up, H, sc, k, tau, hd, cn, st, trp);
        if (e != hipSuccess)
            return hip_status(e, "head predictor launch");
    } else {
        e = enqueue_predict(dtype, x, 1, d, Vp, r, Up, H, sc, a, st, trp, h);
        if (e != hipSuccess)
            return hip_status(e, "head predictor launch");
        if (k >= 0)
            e = csf::launch_select_topk(sc, 1, H, k, hd, max_heads > 0 ? max_heads : 1, cn, nullptr,
                                        st, trp);
        else
            e = csf::launch_select_threshold(sc, 1, H, tau, hd, H, cn, nullptr, st, trp);
        if (e != hipSuccess)
            return hip_status(e, "head selection launch");
    }
    return enqueue_attention(x, d, H, dh, dtype, Wq, Wk, Wv, bq, bk, bv, WoT, Kc, Vc, Tmax, len, hd,
                             cn, max_heads, kv_all, o, y, ws, w, st, trp);
}

}  // extern "C"
