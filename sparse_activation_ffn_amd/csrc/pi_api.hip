// pi_api.hip -- host side of the C ABI declared in include/pi.h: argument
// validation (before anything is enqueued), workspace layout, launch shapes,
// template dispatch and the kernel timing hooks.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <algorithm>
#include <chrono>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "pi.h"
#include "pi_ffn.h"
#include "pi_host.h"
#include "pi_kernels.h"
#include "pi_mfma.h"

using namespace pi;

// Scratch of pi_sparse_ffn_split_noalloc (h and the partials of y), in device
// memory the library owns: one copy per GPU.  In host code this name is only a
// stand-in; the device address comes from hipGetSymbolAddress (scratch_ptr).
static __device__ __align__(256) uint8_t scratch[PI_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

pi_status fail(pi_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

#define CHECK(cond, status, ...)                          \
    do {                                                  \
        if (!(cond)) return fail(status, __VA_ARGS__);    \
    } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---- workspace layout -------------------------------------------------------
// [0, 256)     reserved header
// [256, ...)   per-call scratch: u [B][r] for the predictor; h [B][n] then
//              chunk partials [nch][B][d] for the FFN.  Nothing persists
//              between calls.
constexpr size_t WS_CTR_BYTES = 256;
constexpr int MAX_SLICES = 1024;
constexpr int NCH_MAX = 64;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int down_cols(int wt) { return wt == F32 ? Down<F32>::COLS : wt == F16 ? Down<F16>::COLS : Down<Q4>::COLS; }

int pick_nch(int d, int wt, int B) {
    const int slices = (d + down_cols(wt) - 1) / down_cols(wt);
    int nch = 512 / slices;
    if (B > 8) nch = nch * 8 / B;
    return nch < 2 ? 2 : nch > NCH_MAX ? NCH_MAX : nch;
}

// Fused kernel (k_ffn): one workgroup per compute unit of the MI355X.
#ifndef PI_FFN_WORKGROUPS
#define PI_FFN_WORKGROUPS 256
#endif
constexpr int NWG_FUSED = PI_FFN_WORKGROUPS;
constexpr int FUSED_MAX_BATCH = 4;

// token tile of the batch-templated kernels
int batch_tile(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8; }

// 16-byte chunks per thread of k_ffn for rows of d elements (1, 2 or 4; 0 = too wide)
int fused_nc(int d, int wt) {
    const int epc = wt == F32 ? 4 : wt == F16 ? 8 : 32;
    const int nc = (d / epc + FT - 1) / FT;
    return nc <= 1 ? 1 : nc <= 2 ? 2 : nc <= 4 ? 4 : 0;
}

// The fused path takes batch 1, and batches up to 4 that the matrix-core path
// does not take (f32 weights), with the natural x dtype of the weights, where
// its double-buffered rows and accumulators fit in registers (Q4_0: batch 1 and
// d <= 16384; four chunks per thread: batch 1); other shapes take the gathered
// two-kernel path.
bool use_fused(int d, int wt, int xt, int B) {
    const bool pair = (wt == F32 && xt == F32) || (wt != F32 && xt == F16);
    const int nc = fused_nc(d, wt);
    if (!pair || B > FUSED_MAX_BATCH || nc == 0) return false;
    // x of the token tile and the mask words, or the partial at the end, and
    // the static LDS
    const size_t bt = (size_t)batch_tile(B);
    const size_t lds = std::max(bt * d * (xt == F32 ? 4 : 2) + 8 * (size_t)FUSED_MASK_WORDS, bt * d * 4) + 4096;
    if (lds > 160 * 1024) return false;
    if (wt == Q4 && (B > 1 || nc == 4)) return false;
    if (nc == 4 && B > 1) return false;
    return true;
}

// Matrix-core path: batches of 2..64 tokens with f16 x and f16 / Q4_0 weights
// (measured faster than the fused kernel from batch 2 on: at batch 4 of the
// ReGLU 70B layer 130 vs 163 us per layer step; at batch 1 the fused kernel
// wins, 48 vs 77 us on the OPT-30B layer).
constexpr int MFMA_MIN_BATCH = 2;
bool use_mfma(int d, int wt, int xt, int B, int64_t max_rows = 0) {
    // (the Q4_0 down kernel addresses a partition with 32-bit offsets)
    return B >= MFMA_MIN_BATCH && B <= MM && xt == F16 && (wt == F16 || wt == Q4) && d % DC == 0 &&
           (wt != Q4 || max_rows * row_bytes(Q4, d) < ((int64_t)1 << 31));
}
// split-K chunks of the matrix-core down kernel: about two workgroups per
// compute unit, a multiple of the 8 XCDs (each XCD takes whole chunks)
int mfma_chunks(int d) {
    const int tiles = d / DC;
    const int k = (512 / (tiles > 0 ? tiles : 1) + NXCD - 1) / NXCD * NXCD;
    return k < NXCD ? NXCD : k > NCH_MAX ? NCH_MAX : k;
}

// u [B][r], then (matrix-core predictor, B >= 2) the per-token u scales [B]
// and the K-slice partials of x P1
size_t ws_pred_bytes(int r, int B) {
    size_t v = WS_CTR_BYTES + align256((size_t)B * r * 4);
    if (B >= MFMA_MIN_BATCH) v += align256((size_t)B * 4) + align256((size_t)P1_KS * B * r * 4);
    return v;
}

// h: f32 [B][n] (gathered path) or f16 [B][mfma_h_ld(n)] (matrix-core path)
int mfma_h_ld(int n) { return (n + 7) / 8 * 8 + 8; }
size_t ws_h_bytes(int n, int B) {
    const size_t f32 = (size_t)B * n * 4, f16 = (size_t)B * mfma_h_ld(n) * 2;
    return align256(f32 > f16 ? f32 : f16);
}

// Split of the matrix-core up kernel over K, for Q4_0 weights at batches of up
// to 16 (one 16-token tile): there the active tiles alone leave the compute
// units short of work (OPT-175B-shaped layer, batch 8: about 235 tiles of 64
// items for 256 CUs that hold 4 such workgroups each); four slices took the
// step from 141 to 133 us.  Measured no gain at batch 64 (the tiles already
// fill the chip; 315 -> 323 us with two slices) nor for f16 weights at batch 4
// (ReGLU-70B-shaped layer 132 -> 139 us), so those run unsplit.
constexpr int UP_SPLIT_SMALL_B = 4;
constexpr int UP_SPLIT_MAX_B = 32;
static_assert(UP_SPLIT_SMALL_B <= UP_FINISH_MAX_S, "k_up_finish holds at most UP_FINISH_MAX_S slices");
// K slices of the Q4_0 up kernel (measured on the OPT-175B Q4_0 layer: two
// slices beat four from 4 to 14 tokens, e.g. up 44 -> 40 us at batch 8 and
// 52 -> 42 us at batch 12; four beat two at 16 tokens, 62.5 against 69.4 us;
// with 17..32 tokens two slices beat none, step 191.5 -> 179.7 us at batch 24
// and 204.7 -> 193.3 us at batch 32; with 64 tokens none is best, 282 against
// 296.6 us)
int up_split_want(int B, int wt) {
    if (wt != Q4 || B > UP_SPLIT_MAX_B) return 1;
    return B == 15 || B == 16 ? UP_SPLIT_SMALL_B : 2;
}
int64_t up_part_ld(int n) { return (int64_t)(n + 63) / 64 * 64; }

// the partials of y (down kernels), which the split up kernel's partials share
size_t ws_part_bytes(int d, int n, int B, int nparts) {
    size_t v = (size_t)nparts * B * d * 4;
    if (B >= MFMA_MIN_BATCH && B <= UP_SPLIT_MAX_B) {
        const size_t u = (size_t)UP_SPLIT_SMALL_B * B * up_part_ld(n) * 4;
        if (u > v) v = u;
    }
    return align256(v);
}

// h and the partials
size_t ws_ffn_bytes(int d, int n, int B, int nparts) {
    return WS_CTR_BYTES + ws_h_bytes(n, B) + ws_part_bytes(d, n, B, nparts);
}

// ---- timing hooks --------------------------------------------------------------
struct Timer {
    bool armed = false;
    int max = 0, used = 0;
    std::vector<hipEvent_t> ev;   // 2 per launch
};
thread_local Timer g_timers[PI_K_COUNT];

template <typename K, typename... Args>
pi_status launch(int kid, K kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                 Args... args) {
    Timer& t = g_timers[kid];
    if (t.armed && t.used < t.max) {
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, s, t.ev[2 * t.used],
                              t.ev[2 * t.used + 1], 0, args...);
        ++t.used;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(PI_ERR_HIP, "%s launch: %s", pi_kernel_name(kid), hipGetErrorString(e));
    return PI_OK;
}

// ---- static scratch of the no-allocation entry point ------------------------------
// `scratch` (file scope, below the includes): one copy per GPU, held until the
// process ends.  Host code never uses the array's name as an address: the device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per device
// with that device current.
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

pi_status scratch_ptr(hipStream_t s, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PI_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (s) {
        int sdev = -1;
        e = hipStreamGetDevice(s, &sdev);
        if (e != hipSuccess) return fail(PI_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sdev != dev) return fail(PI_ERR_ARG, "the stream belongs to device %d, the current device is %d", sdev, dev);
    }
    if (dev < 0 || dev >= MAX_DEVICES) return fail(PI_ERR_HIP, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PI_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PI_OK;
}

// ---- host side of the hybrid step --------------------------------------------------
// An event marks the arrival of mask and x in the host workspace; the host spins
// on it, then computes.  One per host thread and device (created on first use,
// kept until the process ends): calls from different threads, on different
// streams, each wait for their own record.
thread_local hipEvent_t g_arrive[MAX_DEVICES] = {};

pi_status arrival_event(hipStream_t s, hipEvent_t* out) {
    int dev = -1;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PI_ERR_HIP, "stream device: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES) return fail(PI_ERR_HIP, "device %d out of range", dev);
    if (!g_arrive[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&g_arrive[dev], hipEventDisableTiming);
        if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess) {
            g_arrive[dev] = nullptr;
            return fail(PI_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
        }
    }
    *out = g_arrive[dev];
    return PI_OK;
}

// Where a pointer lives, as the runtime reports it; Unregistered for memory it
// does not know (ordinary pageable host memory).  Clears the error an unknown
// pointer may leave.
hipMemoryType memory_type(const void* p) {
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return hipMemoryTypeUnregistered;
    }
    return a.type;
}

size_t align64(size_t v) { return (v + 63) & ~size_t(63); }

// host workspace of the hybrid step: mask words, x, the host's partial of y, the cold ids
size_t hybrid_host_layout(int d, int n, int B, size_t off[4]) {
    size_t o = 0;
    off[0] = o;
    o = align64(o + (size_t)((n + 63) / 64) * 8);
    off[1] = o;
    o = align64(o + (size_t)B * d * 4);
    off[2] = o;
    o = align64(o + (size_t)B * d * 4);
    off[3] = o;
    o = align64(o + (size_t)n * 4);
    return o;
}

double us_since(const std::chrono::steady_clock::time_point& t0) {
    return std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
}

// ---- argument checks ----------------------------------------------------------------
pi_status check_dtype_x(int xdtype) {
    CHECK(xdtype == PI_F32 || xdtype == PI_F16, PI_ERR_DTYPE, "x dtype must be PI_F32 or PI_F16");
    return PI_OK;
}

pi_status check_part(const pi_ffn_part* p, const char* name, bool allow_empty) {
    CHECK(p, PI_ERR_ARG, "%s: NULL partition", name);
    CHECK(p->wdtype == PI_F32 || p->wdtype == PI_F16 || p->wdtype == PI_Q4_0, PI_ERR_DTYPE,
          "%s: wdtype must be PI_F32, PI_F16 or PI_Q4_0", name);
    CHECK(p->act == PI_RELU || p->act == PI_REGLU || p->act == PI_SQRELU, PI_ERR_ARG,
          "%s: act must be PI_RELU, PI_REGLU or PI_SQRELU", name);
    CHECK(p->d > 0 && p->d % 64 == 0, PI_ERR_SHAPE, "%s: d must be a positive multiple of 64", name);
    CHECK(p->wdtype != PI_Q4_0 || p->d % 256 == 0, PI_ERR_SHAPE, "%s: Q4_0 rows need d %% 256 == 0", name);
    CHECK(p->d <= down_cols(p->wdtype) * MAX_SLICES, PI_ERR_SHAPE, "%s: d too large", name);
    CHECK(p->rows >= 0 && (allow_empty || p->rows > 0), PI_ERR_SHAPE, "%s: bad row count", name);
    if (p->rows == 0) return PI_OK;
    CHECK(p->W_up && p->W_downT, PI_ERR_ARG, "%s: W_up and W_downT are required", name);
    CHECK(p->act != PI_REGLU || p->W_gate, PI_ERR_ARG, "%s: ReGLU needs W_gate", name);
    CHECK(aligned(p->W_up, 16) && aligned(p->W_downT, 16) &&
              (p->act != PI_REGLU || aligned(p->W_gate, 16)),
          PI_ERR_ALIGN, "%s: weights must be 16-byte aligned", name);
    CHECK(aligned(p->b_up, 4) && aligned(p->b_gate, 4), PI_ERR_ALIGN, "%s: biases must be 4-byte aligned", name);
    return PI_OK;
}

pi_status check_ws(void* ws, size_t have, size_t need) {
    CHECK(ws, PI_ERR_WORKSPACE, "workspace is NULL");
    CHECK(aligned(ws, 256), PI_ERR_ALIGN, "workspace must be 256-byte aligned");
    CHECK(have >= need, PI_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
    return PI_OK;
}

#define TRY(expr)                         \
    do {                                  \
        pi_status _s = (expr);            \
        if (_s != PI_OK) return _s;       \
    } while (0)

// ---- template dispatch ---------------------------------------------------------
// kernels with more than 64 KiB of dynamic LDS must opt in
template <typename K>
pi_status allow_lds(K kernel, size_t bytes) {
    if (bytes <= 65536) return PI_OK;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return fail(PI_ERR_HIP, "LDS attribute: %s", hipGetErrorString(e));
    return PI_OK;
}

template <int WT, int XT, int BT>
pi_status launch_pred_l1(const pi_predictor* p, const void* x, int B, float* u, hipStream_t s) {
    return launch(PI_K_PRED_L1, k_pred_l1<WT, XT, BT>, dim3(p->r), dim3(THREADS), 0, s,
                  (const uint8_t*)p->P1t, (const uint8_t*)x, p->d, p->r, B, u);
}

template <int WT, int XT>
pi_status pred_l1_bt(const pi_predictor* p, const void* x, int B, float* u, hipStream_t s) {
    switch (batch_tile(B)) {
    case 1: return launch_pred_l1<WT, XT, 1>(p, x, B, u, s);
    case 2: return launch_pred_l1<WT, XT, 2>(p, x, B, u, s);
    case 4: return launch_pred_l1<WT, XT, 4>(p, x, B, u, s);
    default: return launch_pred_l1<WT, XT, 8>(p, x, B, u, s);
    }
}

template <int WT, int BT>
pi_status launch_pred_l2(const pi_predictor* p, const float* u, int B, uint64_t* mask, float* logits,
                         hipStream_t s) {
    // one workgroup per 16-bit quarter of every mask word (tail quarters included)
    const int grid = (p->n + 63) / 64 * (64 / L2_ROWS);
    const size_t sh = (size_t)BT * p->r * sizeof(float);
    auto kern = k_pred_l2<WT, BT>;
    TRY(allow_lds(kern, sh));
    return launch(PI_K_PRED_L2, kern, dim3(grid), dim3(THREADS), sh, s, (const uint8_t*)p->P2t,
                  p->b2, p->threshold, u, p->n, p->r, B, reinterpret_cast<uint16_t*>(mask), logits);
}

template <int WT>
pi_status pred_l2_bt(const pi_predictor* p, const float* u, int B, uint64_t* mask, float* logits,
                     hipStream_t s) {
    switch (batch_tile(B)) {
    case 1: return launch_pred_l2<WT, 1>(p, u, B, mask, logits, s);
    case 2: return launch_pred_l2<WT, 2>(p, u, B, mask, logits, s);
    case 4: return launch_pred_l2<WT, 4>(p, u, B, mask, logits, s);
    default: return launch_pred_l2<WT, 8>(p, u, B, mask, logits, s);
    }
}

// x is staged in LDS by k_up when a token group of it fits in 64 KiB
constexpr size_t XLDS_MAX = 65536;

template <int WT, int XT, int BT, int ACT>
pi_status launch_up(const FfnArgs& a, int rows_cap, hipStream_t s) {
    int grid = (rows_cap + NWAVES - 1) / NWAVES;
    if (grid > 2048) grid = 2048;
    if (grid < 1) grid = 1;
    const size_t xbytes = (size_t)BT * a.d * (XT == F32 ? 4 : 2);
    const size_t words = a.mask ? (size_t)(a.n + 63) / 64 : 0;
    const size_t mbytes = words ? words * 8 + (words + 1) * 4 : 0;   // mask words + their scan
    if (xbytes <= XLDS_MAX) {
        auto kern = k_up<WT, XT, BT, ACT, true>;
        TRY(allow_lds(kern, xbytes + mbytes));
        return launch(PI_K_UP, kern, dim3(grid), dim3(THREADS), xbytes + mbytes, s, a);
    }
    auto kern = k_up<WT, XT, BT, ACT, false>;
    TRY(allow_lds(kern, mbytes));
    return launch(PI_K_UP, kern, dim3(grid), dim3(THREADS), mbytes, s, a);
}

// chunk partials -> y_hot, y_cold, y (one thread per 4 consecutive outputs)
pi_status launch_reduce(const FfnArgs& a, const DownOut& o, hipStream_t s) {
    const int64_t len4 = (int64_t)a.B * a.d / 4;
    int grid = (int)((len4 + THREADS - 1) / THREADS);
    if (grid > 4096) grid = 4096;
    return launch(PI_K_REDUCE, k_reduce, dim3(grid), dim3(THREADS), 0, s, a, o);
}

template <int WT, int BT>
pi_status launch_down(const FfnArgs& a, const DownOut& o, hipStream_t s) {
    const int slices = (a.d + Down<WT>::COLS - 1) / Down<WT>::COLS;
    TRY(launch(PI_K_DOWN, k_down<WT, BT>, dim3(slices, o.nch), dim3(THREADS), 0, s, a, o));
    return launch_reduce(a, o, s);
}

template <int WT, int XT, int BT>
pi_status ffn_act(const FfnArgs& a, const DownOut& o, int act, int rows_cap, hipStream_t s) {
    pi_status st = act == PI_REGLU    ? launch_up<WT, XT, BT, REGLU>(a, rows_cap, s)
                   : act == PI_SQRELU ? launch_up<WT, XT, BT, SQRELU>(a, rows_cap, s)
                                      : launch_up<WT, XT, BT, RELU>(a, rows_cap, s);
    if (st != PI_OK) return st;
    return launch_down<WT, BT>(a, o, s);
}

template <int WT, int XT>
pi_status ffn_bt(const FfnArgs& a, const DownOut& o, int act, int rows_cap, hipStream_t s) {
    switch (batch_tile(a.B)) {
    case 1: return ffn_act<WT, XT, 1>(a, o, act, rows_cap, s);
    case 2: return ffn_act<WT, XT, 2>(a, o, act, rows_cap, s);
    case 4: return ffn_act<WT, XT, 4>(a, o, act, rows_cap, s);
    default: return ffn_act<WT, XT, 8>(a, o, act, rows_cap, s);
    }
}

// ---- fused path -------------------------------------------------------------

template <int WT, int XT, int BT, int ACT, int NC>
pi_status launch_fused(const FfnArgs& a, const DownOut& o, hipStream_t s) {
    const size_t xbytes = (size_t)BT * a.d * (XT == F32 ? 4 : 2);
    const size_t words = a.mask ? (size_t)(a.n + 63) / 64 : 0;
    const size_t pbytes = (size_t)BT * a.d * 4;       // the partial, staged at the end
    const size_t sh = std::max(xbytes + words * 8, pbytes);   // x, then the mask words
    auto kern = k_ffn<WT, XT, BT, ACT, NC>;
    TRY(allow_lds(kern, sh));
    TRY(launch(PI_K_FFN, kern, dim3(o.nch), dim3(FT), sh, s, a, o));
    const int64_t len = (int64_t)a.B * a.d;
    return launch(PI_K_REDUCE, k_reduce_parts, dim3((unsigned)((len + RE - 1) / RE)),
                  dim3(RE * RS), 0, s, a, o);
}

// Only the (chunks per thread, batch tile) pairs use_fused admits are
// instantiated: four chunks per thread at batch 1 with f32 / f16 weights.
template <int WT, int XT, int BT, int ACT>
pi_status fused_nc_dispatch(const FfnArgs& a, const DownOut& o, hipStream_t s) {
    switch (fused_nc(a.d, WT)) {
    case 1: return launch_fused<WT, XT, BT, ACT, 1>(a, o, s);
    case 2: return launch_fused<WT, XT, BT, ACT, 2>(a, o, s);
    default:
        if constexpr (BT == 1 && WT != Q4) return launch_fused<WT, XT, BT, ACT, 4>(a, o, s);
        return fail(PI_ERR_SHAPE, "fused kernel: row too wide for this batch");
    }
}

template <int WT, int XT, int BT>
pi_status fused_act(const FfnArgs& a, const DownOut& o, int act, hipStream_t s) {
    return act == PI_REGLU    ? fused_nc_dispatch<WT, XT, BT, REGLU>(a, o, s)
           : act == PI_SQRELU ? fused_nc_dispatch<WT, XT, BT, SQRELU>(a, o, s)
                              : fused_nc_dispatch<WT, XT, BT, RELU>(a, o, s);
}

template <int WT, int XT>
pi_status fused_bt(const FfnArgs& a, const DownOut& o, int act, hipStream_t s) {
    switch (batch_tile(a.B)) {
    case 1: return fused_act<WT, XT, 1>(a, o, act, s);
    case 2: return fused_act<WT, XT, 2>(a, o, act, s);
    default: return fused_act<WT, XT, 4>(a, o, act, s);
    }
}

pi_status run_fused(const FfnArgs& a, const DownOut& o, int wt, int act, hipStream_t s) {
    if (wt == F32) return fused_bt<F32, F32>(a, o, act, s);
    if (wt == F16) return fused_bt<F16, F16>(a, o, act, s);
    return fused_act<Q4, F16, 1>(a, o, act, s);          // Q4_0: batch 1 only (use_fused)
}

// ---- matrix-core path -------------------------------------------------------
// token tiles of 16 covering the batch (1, 2 or 4)
int mfma_mt(int B) { return B <= 16 ? 1 : B <= 32 ? 2 : 4; }

template <typename K>
pi_status launch_up_kernel(K kern, const FfnArgs& a, int rows_cap, hipStream_t s) {
    constexpr int UR = 64;                             // items per workgroup
    const int grid = rows_cap > 0 ? (rows_cap + UR - 1) / UR : 1;
    // mask words and the rank of each word's first set bit
    const size_t sh = a.mask ? (size_t)(a.n + 63) / 64 * 12 + 4 : 0;
    TRY(allow_lds(kern, sh));
    return launch(PI_K_UP, kern, dim3(grid, a.ksplit > 1 ? a.ksplit : 1), dim3(MFMA_WG), sh, s, a,
                  reinterpret_cast<_Float16*>(a.h));
}

template <int WT, int ACT, int MT>
pi_status launch_mfma_up(const FfnArgs& a, int rows_cap, hipStream_t s) {
    TRY(launch_up_kernel(k_mfma_up<WT, ACT, MT, 1>, a, rows_cap, s));
    if (a.ksplit <= 1) return PI_OK;
    // the slices' sum and the activation (item count from the device)
    constexpr int NM = ACT == REGLU ? 2 : 1;
    const int gx = std::max(1, (rows_cap + THREADS - 1) / THREADS);   // one item per thread
    return launch(PI_K_UP_FINISH, k_up_finish<ACT, NM>, dim3(gx, a.B), dim3(THREADS), 0, s,
                  (const float*)a.upart, a.ksplit, a.upart_ld, a.B, (const int*)a.up_ht,
                  reinterpret_cast<_Float16*>(a.h), a.h_ld);
}

template <int WT, int ACT>
pi_status mfma_up_mt(const FfnArgs& a, int rows_cap, hipStream_t s) {
    switch (mfma_mt(a.B)) {
    case 1: return launch_mfma_up<WT, ACT, 1>(a, rows_cap, s);
    case 2: return launch_mfma_up<WT, ACT, 2>(a, rows_cap, s);
    default: return launch_mfma_up<WT, ACT, 4>(a, rows_cap, s);
    }
}

template <int WT, bool LISTS, int MT>
pi_status mfma_down(const FfnArgs& a, const DownOut& o, hipStream_t s) {
    // one linear grid: chunk = (id % 8) + 8 m, column tile = (id / 8) % tiles (see the kernel)
    return launch(PI_K_DOWN, k_mfma_down<WT, LISTS, MT>, dim3((a.d / DC) * o.nch), dim3(DOWN_WG), 0, s, a,
                  o, (const _Float16*)a.h);
}

template <int WT>
pi_status run_mfma_wt(const FfnArgs& a, const DownOut& o, int act, int rows_cap, hipStream_t s) {
    if (act == PI_REGLU) TRY((mfma_up_mt<WT, REGLU>(a, rows_cap, s)));
    else if (act == PI_SQRELU) TRY((mfma_up_mt<WT, SQRELU>(a, rows_cap, s)));
    else TRY((mfma_up_mt<WT, RELU>(a, rows_cap, s)));
    const bool lists = a.idx[0] || a.idx[1];          // else dense rows
    switch (mfma_mt(a.B) * 2 + (lists ? 1 : 0)) {
    case 2: TRY((mfma_down<WT, false, 1>(a, o, s))); break;
    case 3: TRY((mfma_down<WT, true, 1>(a, o, s))); break;
    case 4: TRY((mfma_down<WT, false, 2>(a, o, s))); break;
    case 5: TRY((mfma_down<WT, true, 2>(a, o, s))); break;
    case 8: TRY((mfma_down<WT, false, 4>(a, o, s))); break;
    default: TRY((mfma_down<WT, true, 4>(a, o, s))); break;
    }
    return launch_reduce(a, o, s);
}

pi_status run_ffn(const FfnArgs& a, const DownOut& o, int wt, int xt, int act, int rows_cap,
                  hipStream_t s) {
    if (wt == F32) return xt == F32 ? ffn_bt<F32, F32>(a, o, act, rows_cap, s) : ffn_bt<F32, F16>(a, o, act, rows_cap, s);
    if (wt == F16) return xt == F32 ? ffn_bt<F16, F32>(a, o, act, rows_cap, s) : ffn_bt<F16, F16>(a, o, act, rows_cap, s);
    return xt == F32 ? ffn_bt<Q4, F32>(a, o, act, rows_cap, s) : ffn_bt<Q4, F16>(a, o, act, rows_cap, s);
}

// Shared body of pi_sparse_ffn / pi_sparse_ffn_split / pi_dense_ffn.
// mask != NULL: the active set is read from mask words and the lists (idx0,
// idx1, counts) are outputs, written by k_up; otherwise they are inputs.
pi_status ffn_common(const pi_ffn_part* hot, const pi_ffn_part* cold, const void* x, int B,
                     int xdtype, const uint64_t* mask, const int32_t* idx0, const int32_t* idx1,
                     const int32_t* counts, bool dense, float* y0, float* y1, float* y, void* ws,
                     size_t ws_bytes, hipStream_t s, bool static_ws = false, int dense_from = 0,
                     bool check_only = false) {
    TRY(check_part(hot, "hot", !dense));
    const bool has_cold = cold && cold->rows > 0;
    if (cold) TRY(check_part(cold, "cold", true));
    if (has_cold) {
        CHECK(cold->d == hot->d && cold->wdtype == hot->wdtype && cold->act == hot->act,
              PI_ERR_SHAPE, "hot and cold partitions differ in d, wdtype or act");
    }
    TRY(check_dtype_x(xdtype));
    CHECK(B >= 1 && B <= PI_MAX_BATCH, PI_ERR_SHAPE, "B must be in 1..%d", PI_MAX_BATCH);
    CHECK(x && aligned(x, 16), x ? PI_ERR_ALIGN : PI_ERR_ARG, "x must be non-NULL and 16-byte aligned");
    CHECK(y0 || y1 || y, PI_ERR_ARG, "no output given");
    CHECK(aligned(y0, 16) && aligned(y1, 16) && aligned(y, 16), PI_ERR_ALIGN, "outputs must be 16-byte aligned");
    if (!dense) {
        CHECK(counts && aligned(counts, 4), counts ? PI_ERR_ALIGN : PI_ERR_ARG, "counts must be non-NULL, 4-byte aligned");
        CHECK(hot->rows == 0 || (idx0 && aligned(idx0, 4)), PI_ERR_ARG, "hot index list missing");
        CHECK(!has_cold || (idx1 && aligned(idx1, 4)), PI_ERR_ARG, "cold index list missing");
    }
    const int d = hot->d, wt = hot->wdtype;
    const int n = hot->rows + (has_cold ? cold->rows : 0);
    const bool mfma = use_mfma(d, wt, xdtype, B, std::max<int64_t>(hot->rows, has_cold ? cold->rows : 0));
    // the dense crossover is decided on the device by the two-kernel paths; the
    // fused batch-1 kernel does not take it
    const bool fused = !mfma && dense_from <= 0 && use_fused(d, wt, xdtype, B);
    const int nch = fused ? NWG_FUSED : mfma ? mfma_chunks(d) : pick_nch(d, wt, B);
    if (static_ws) {
        // the no-allocation entry point: the library's own scratch, checked first
        const size_t need = ws_ffn_bytes(d, n, B, nch);
        CHECK(need <= (size_t)PI_SCRATCH_BYTES, PI_ERR_WORKSPACE,
              "these shapes need %zu bytes of scratch; the static scratch holds %zu (PI_SCRATCH_BYTES)",
              need, (size_t)PI_SCRATCH_BYTES);
        TRY(scratch_ptr(s, &ws));
        ws_bytes = PI_SCRATCH_BYTES;
    }
    TRY(check_ws(ws, ws_bytes, ws_ffn_bytes(d, n, B, nch)));
    if (mask) CHECK(aligned(mask, 8), PI_ERR_ALIGN, "mask must be 8-byte aligned");
    if (check_only) return PI_OK;

    uint8_t* base = static_cast<uint8_t*>(ws);
    FfnArgs a{};
    a.up[0] = (const uint8_t*)hot->W_up;
    a.gate[0] = (const uint8_t*)hot->W_gate;
    a.bup[0] = hot->b_up;
    a.bgate[0] = hot->b_gate;
    a.down[0] = (const uint8_t*)hot->W_downT;
    a.idx[0] = dense ? nullptr : idx0;
    if (has_cold) {
        a.up[1] = (const uint8_t*)cold->W_up;
        a.gate[1] = (const uint8_t*)cold->W_gate;
        a.bup[1] = cold->b_up;
        a.bgate[1] = cold->b_gate;
        a.down[1] = (const uint8_t*)cold->W_downT;
        a.idx[1] = idx1;
    }
    a.counts = dense ? nullptr : counts;
    a.nparts = has_cold ? 2 : 1;
    a.rows[0] = hot->rows;
    a.rows[1] = has_cold ? cold->rows : 0;
    if (mask) {
        Lists L{hot->rows, const_cast<int32_t*>(idx0), const_cast<int32_t*>(idx1),
                const_cast<int32_t*>(counts)};
        if ((n + 63) / 64 <= (fused ? FUSED_MASK_WORDS : MASK_WORDS_MAX)) {
            a.mask = mask;                   // compaction fused into k_ffn / k_up
            a.n = n;
            a.out_idx[0] = L.hot;
            a.out_idx[1] = L.cold;
            a.out_counts = L.counts;
        } else {
            TRY(launch(PI_K_COMPACT, k_compact, dim3(1), dim3(THREADS), 0, s, mask, n, L));
        }
    }
    a.dense_rows = dense ? hot->rows : 0;
    a.dense_from = dense ? 0 : dense_from;
    a.d = d;
    a.B = B;
    a.rb = row_bytes(wt, d);
    a.x = (const uint8_t*)x;
    a.h = reinterpret_cast<float*>(base + WS_CTR_BYTES);
    // f32 h [B][n] (gathered path) or f16 h [B][h_ld] (matrix-core path: hot
    // items, then cold items from the next multiple of 8)
    a.h_ld = mfma ? mfma_h_ld(n) : (n > 0 ? n : 1);
    DownOut o{};
    o.partials = reinterpret_cast<float*>(base + WS_CTR_BYTES + ws_h_bytes(n, B));
    a.ksplit = 1;
    if (mfma) {
        // slices of the up kernel: as many as wanted that the partial region holds
        const int nm = hot->act == PI_REGLU ? 2 : 1;
        const int64_t per = (int64_t)nm * B * up_part_ld(n) * 4;
        const int64_t fit = (int64_t)ws_part_bytes(d, n, B, nch) / per;
        a.ksplit = (int)std::max<int64_t>(1, std::min<int64_t>(up_split_want(B, wt), fit));
        a.upart = o.partials;
        a.upart_ld = (int)up_part_ld(n);
        a.up_ht = reinterpret_cast<int*>(base);
    }
    o.y_part[0] = y0;
    o.y_part[1] = y1;
    o.y = y;
    o.nch = nch;
    if (fused) return run_fused(a, o, wt, hot->act, s);
    if (mfma)
        return wt == F16 ? run_mfma_wt<F16>(a, o, hot->act, n, s) : run_mfma_wt<Q4>(a, o, hot->act, n, s);
    return run_ffn(a, o, wt, xdtype, hot->act, n, s);
}

// The predictor's kernels for B tokens (validated arguments; `base` is a
// workspace of at least ws_pred_bytes(r, B) bytes).
pi_status predict_launch(const pi_predictor* p, const void* x, int B, int xdtype, uint64_t* mask,
                         float* logits, uint8_t* base, hipStream_t s) {
    float* u = reinterpret_cast<float*>(base + WS_CTR_BYTES);
    const int wt = p->wdtype;
    if (B >= MFMA_MIN_BATCH && wt == F16 && xdtype == F16 && p->r % KS == 0 && p->d % KS == 0) {
        // matrix-core predictor: K-split first layer, slice sum + ReLU, second layer
        float* uscale = reinterpret_cast<float*>(base + WS_CTR_BYTES + align256((size_t)B * p->r * 4));
        float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(uscale) + align256((size_t)B * 4));
        const dim3 g1((p->r + P1_ROWS - 1) / P1_ROWS, P1_KS);
        const int mt = mfma_mt(B);
        auto pred1 = mt == 1 ? k_mfma_pred1<1> : mt == 2 ? k_mfma_pred1<2> : k_mfma_pred1<4>;
        TRY(launch(PI_K_PRED_L1, pred1, g1, dim3(MFMA_WG), 0, s, (const uint8_t*)p->P1t,
                   (const uint8_t*)x, p->d, p->r, B, part));
        // the u region holds the second layer's f16 operand: uh [B][r] then ul [B][r]
        _Float16* uhl = reinterpret_cast<_Float16*>(u);
        TRY(launch(PI_K_PRED_L1, k_u_relu, dim3(B), dim3(THREADS), 0, s, (const float*)part, B, p->r,
                   uhl, uscale));
        auto pred2 = mt == 1 ? k_mfma_pred2<1> : mt == 2 ? k_mfma_pred2<2> : k_mfma_pred2<4>;
        TRY(launch(PI_K_PRED_L2, pred2, dim3((p->n + P2_ROWS - 1) / P2_ROWS), dim3(MFMA_WG), 0, s,
                   (const uint8_t*)p->P2t, p->b2, p->threshold, (const _Float16*)uhl, (const float*)uscale,
                   p->n, p->r, B, mask, logits));
    } else {
        pi_status st;
        if (wt == F32)
            st = xdtype == F32 ? pred_l1_bt<F32, F32>(p, x, B, u, s) : pred_l1_bt<F32, F16>(p, x, B, u, s);
        else
            st = xdtype == F32 ? pred_l1_bt<F16, F32>(p, x, B, u, s) : pred_l1_bt<F16, F16>(p, x, B, u, s);
        TRY(st);
        TRY(wt == F32 ? pred_l2_bt<F32>(p, u, B, mask, logits, s) : pred_l2_bt<F16>(p, u, B, mask, logits, s));
    }
    return PI_OK;
}

}  // namespace

// =================================================================================
// C ABI
// =================================================================================
extern "C" {

const char* pi_status_string(pi_status s) {
    switch (s) {
    case PI_OK: return "ok";
    case PI_ERR_ARG: return "invalid argument";
    case PI_ERR_SHAPE: return "invalid shape";
    case PI_ERR_ALIGN: return "misaligned pointer";
    case PI_ERR_DTYPE: return "unsupported dtype";
    case PI_ERR_WORKSPACE: return "workspace too small";
    case PI_ERR_BUDGET: return "invalid budget";
    case PI_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* pi_last_error(void) { return g_err; }

const char* pi_kernel_name(int32_t kid) {
    static const char* names[PI_K_COUNT] = {"k_pred_l1", "k_pred_l2", "k_compact", "k_up", "k_down",
                                            "k_merge", "k_profile", "k_index", "k_copy", "k_reduce",
                                            "k_ffn", "k_accumulate_mask", "k_stream_read",
                                            "k_up_finish"};
    return (kid >= 0 && kid < PI_K_COUNT) ? names[kid] : "?";
}

size_t pi_workspace_bytes(int32_t d, int32_t n, int32_t r, int32_t B) {
    if (d <= 0 || n <= 0 || r <= 0 || B <= 0 || B > PI_MAX_BATCH) return 0;
    size_t need = ws_pred_bytes(r, B);
    for (int wt = F32; wt <= Q4; ++wt) {
        size_t f = ws_ffn_bytes(d, n, B, pick_nch(d, wt, B));
        if (f > need) need = f;
        if (B <= FUSED_MAX_BATCH) {
            f = ws_ffn_bytes(d, n, B, NWG_FUSED);
            if (f > need) need = f;
        }
        if (B >= MFMA_MIN_BATCH) {
            f = ws_ffn_bytes(d, n, B, mfma_chunks(d));
            if (f > need) need = f;
        }
    }
    return need;
}

pi_status pi_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    CHECK(ws && aligned(ws, 256), PI_ERR_ALIGN, "workspace must be non-NULL and 256-byte aligned");
    CHECK(ws_bytes >= WS_CTR_BYTES && ws_bytes % 16 == 0, PI_ERR_WORKSPACE, "workspace too small");
    const int64_t n16 = (int64_t)(ws_bytes / 16);
    int grid = (int)((n16 + THREADS - 1) / THREADS);
    if (grid > 4096) grid = 4096;
    return launch(PI_K_COPY, k_zero, dim3(grid), dim3(THREADS), 0, (hipStream_t)stream,
                  reinterpret_cast<u4*>(ws), n16);
}

pi_status pi_predict(const pi_predictor* p, const void* x, int32_t B, int32_t xdtype,
                     uint64_t* mask, float* logits, const pi_active_lists* lists, void* ws,
                     size_t ws_bytes, void* stream) {
    CHECK(p, PI_ERR_ARG, "NULL predictor");
    CHECK(p->wdtype == PI_F32 || p->wdtype == PI_F16, PI_ERR_DTYPE, "predictor wdtype must be PI_F32 or PI_F16");
    TRY(check_dtype_x(xdtype));
    CHECK(p->d > 0 && p->d % 64 == 0, PI_ERR_SHAPE, "d must be a positive multiple of 64");
    CHECK(p->r > 0 && p->r % 16 == 0 && p->r <= 4096, PI_ERR_SHAPE, "r must be a multiple of 16 in 16..4096");
    CHECK(p->n > 0 && p->n <= (1 << 24), PI_ERR_SHAPE, "n must be in 1..2^24");
    CHECK(B >= 1 && B <= PI_MAX_BATCH, PI_ERR_SHAPE, "B must be in 1..%d", PI_MAX_BATCH);
    CHECK(p->P1t && p->P2t && x && mask, PI_ERR_ARG, "P1t, P2t, x and mask are required");
    CHECK(aligned(p->P1t, 16) && aligned(p->P2t, 16) && aligned(x, 16), PI_ERR_ALIGN,
          "P1t, P2t and x must be 16-byte aligned");
    CHECK(aligned(mask, 8) && aligned(logits, 4) && aligned(p->b2, 4), PI_ERR_ALIGN, "mask/logits/b2 misaligned");
    Lists L{};
    if (lists) {
        CHECK(lists->n_hot >= 0 && lists->n_hot <= p->n, PI_ERR_SHAPE, "lists->n_hot out of range");
        CHECK(lists->counts && aligned(lists->counts, 8), PI_ERR_ARG, "lists->counts required (8-byte aligned)");
        CHECK(lists->n_hot == 0 || lists->hot_idx, PI_ERR_ARG, "lists->hot_idx required");
        CHECK(lists->n_hot == p->n || lists->cold_idx, PI_ERR_ARG, "lists->cold_idx required");
        L = Lists{lists->n_hot, lists->hot_idx, lists->cold_idx, lists->counts};
    }
    TRY(check_ws(ws, ws_bytes, ws_pred_bytes(p->r, B)));
    hipStream_t s = (hipStream_t)stream;
    TRY(predict_launch(p, x, B, xdtype, mask, logits, static_cast<uint8_t*>(ws), s));
    if (!lists) return PI_OK;
    return launch(PI_K_COMPACT, k_compact, dim3(1), dim3(THREADS), 0, s, (const uint64_t*)mask, p->n, L);
}

// ---- adaptive predictor threshold (offline) -----------------------------------
// workspace: logits [S][n] f32, keys [n][S] u32, the selection histogram and
// state, a mask word per 64 neurons, then the predictor's own scratch
static size_t calib_layout(int32_t d, int32_t n, int32_t r, int32_t S, size_t off[5]) {
    off[0] = WS_CTR_BYTES;                                          // logits
    off[1] = off[0] + align256((size_t)S * n * 4);                  // keys
    off[2] = off[1] + align256((size_t)S * n * 4);                  // hist [SEL_BINS] + state [8]
    off[3] = off[2] + align256((SEL_BINS + 8) * 4);                 // mask words
    off[4] = off[3] + align256((size_t)(n + 63) / 64 * 8);          // predictor scratch
    (void)d;
    return off[4] + ws_pred_bytes(r, PI_MAX_BATCH);
}

pi_status pi_compact_active(const uint64_t* mask, int32_t n, const pi_active_lists* lists,
                            void* stream) {
    CHECK(mask && aligned(mask, 8), PI_ERR_ARG, "mask required (8-byte aligned)");
    CHECK(n > 0 && n <= (1 << 24), PI_ERR_SHAPE, "n must be in 1..2^24");
    CHECK(lists, PI_ERR_ARG, "lists required");
    CHECK(lists->n_hot >= 0 && lists->n_hot <= n, PI_ERR_SHAPE, "lists->n_hot out of range");
    CHECK(lists->counts && aligned(lists->counts, 8), PI_ERR_ARG, "lists->counts required (8-byte aligned)");
    CHECK(lists->n_hot == 0 || lists->hot_idx, PI_ERR_ARG, "lists->hot_idx required");
    CHECK(lists->n_hot == n || lists->cold_idx, PI_ERR_ARG, "lists->cold_idx required");
    Lists L{lists->n_hot, lists->hot_idx, lists->cold_idx, lists->counts};
    return launch(PI_K_COMPACT, k_compact, dim3(1), dim3(THREADS), 0, (hipStream_t)stream, mask, n, L);
}

pi_status pi_sparse_ffn(const pi_ffn_part* part, const void* x, int32_t B, int32_t xdtype,
                        const int32_t* idx, const int32_t* count, float* y, void* ws,
                        size_t ws_bytes, void* stream) {
    CHECK(y, PI_ERR_ARG, "y required");
    CHECK(count && aligned(count, 4), PI_ERR_ARG, "count required (4-byte aligned)");
    // a single partition runs as the hot half of a split with no cold part:
    // items are idx[0 .. *count) and only count[0] is read
    return ffn_common(part, nullptr, x, B, xdtype, nullptr, idx, nullptr, count, false, nullptr, nullptr,
                      y, ws, ws_bytes, (hipStream_t)stream);
}

pi_status pi_sparse_ffn_split(const pi_ffn_part* hot, const pi_ffn_part* cold, const void* x,
                              int32_t B, int32_t xdtype, const uint64_t* mask,
                              const pi_active_lists* lists, float* y_hot, float* y_cold, float* y,
                              void* ws, size_t ws_bytes, void* stream) {
    CHECK(lists, PI_ERR_ARG, "lists required");
    CHECK(hot && lists->n_hot == hot->rows, PI_ERR_SHAPE, "lists->n_hot must equal hot->rows");
    return ffn_common(hot, cold, x, B, xdtype, mask, lists->hot_idx, lists->cold_idx,
                      lists->counts, false, y_hot, y_cold, y, ws, ws_bytes, (hipStream_t)stream);
}

pi_status pi_sparse_ffn_split_noalloc(const pi_ffn_part* hot, const pi_ffn_part* cold, const void* x,
                                      int32_t B, int32_t xdtype, const uint64_t* mask,
                                      const pi_active_lists* lists, float* y_hot, float* y_cold,
                                      float* y, void* stream) {
    CHECK(lists, PI_ERR_ARG, "lists required");
    CHECK(hot && lists->n_hot == hot->rows, PI_ERR_SHAPE, "lists->n_hot must equal hot->rows");
    return ffn_common(hot, cold, x, B, xdtype, mask, lists->hot_idx, lists->cold_idx, lists->counts,
                      false, y_hot, y_cold, y, nullptr, 0, (hipStream_t)stream, true);
}

pi_status pi_sparse_ffn_crossover(const pi_ffn_part* hot, const pi_ffn_part* cold, const void* x,
                                  int32_t B, int32_t xdtype, const uint64_t* mask,
                                  const pi_active_lists* lists, int32_t dense_from, float* y_hot,
                                  float* y_cold, float* y, void* ws, size_t ws_bytes, void* stream) {
    CHECK(lists, PI_ERR_ARG, "lists required");
    CHECK(hot && lists->n_hot == hot->rows, PI_ERR_SHAPE, "lists->n_hot must equal hot->rows");
    CHECK(dense_from >= 1, PI_ERR_ARG, "dense_from must be >= 1");
    return ffn_common(hot, cold, x, B, xdtype, mask, lists->hot_idx, lists->cold_idx, lists->counts,
                      false, y_hot, y_cold, y, ws, ws_bytes, (hipStream_t)stream, false, dense_from);
}

pi_status pi_dense_ffn(const pi_ffn_part* part, const void* x, int32_t B, int32_t xdtype, float* y,
                       void* ws, size_t ws_bytes, void* stream) {
    CHECK(y, PI_ERR_ARG, "y required");
    return ffn_common(part, nullptr, x, B, xdtype, nullptr, nullptr, nullptr, nullptr, true, nullptr,
                      nullptr, y, ws, ws_bytes, (hipStream_t)stream);
}

pi_status pi_merge(const float* y_hot, const float* y_cold, int32_t B, int32_t d, float* y,
                   void* stream) {
    CHECK(y_hot && y, PI_ERR_ARG, "y_hot and y are required");
    CHECK(B >= 1 && d >= 1, PI_ERR_SHAPE, "B and d must be positive");
    CHECK(aligned(y_hot, 4) && aligned(y_cold, 4) && aligned(y, 4), PI_ERR_ALIGN, "misaligned output");
    const int64_t len = (int64_t)B * d;
    int grid = (int)((len + THREADS - 1) / THREADS);
    if (grid > 1024) grid = 1024;
    return launch(PI_K_MERGE, k_merge, dim3(grid), dim3(THREADS), 0, (hipStream_t)stream, y_hot,
                  y_cold, len, y);
}

pi_status pi_profile_counts(const pi_ffn_part* part, const void* X, int32_t S, int32_t xdtype,
                            uint32_t* counts, void* stream) {
    TRY(check_part(part, "part", false));
    TRY(check_dtype_x(xdtype));
    CHECK(S >= 0, PI_ERR_SHAPE, "S must be >= 0");
    CHECK(counts && aligned(counts, 4), PI_ERR_ARG, "counts required");
    CHECK(S == 0 || (X && aligned(X, 16)), PI_ERR_ARG, "X required (16-byte aligned)");
    const bool reglu = part->act == PI_REGLU;
    const uint8_t* W = (const uint8_t*)(reglu ? part->W_gate : part->W_up);
    const float* bias = reglu ? part->b_gate : part->b_up;
    const int grid = (part->rows + NWAVES - 1) / NWAVES;
    hipStream_t s = (hipStream_t)stream;
    const int wt = part->wdtype;
#define PROF(WT_, XT_) launch(PI_K_PROFILE, k_profile<WT_, XT_, 8>, dim3(grid), dim3(THREADS), 0, s, \
                              W, bias, (const uint8_t*)X, part->d, part->rows, S, counts)
    if (wt == F32) return xdtype == F32 ? PROF(F32, F32) : PROF(F32, F16);
    if (wt == F16) return xdtype == F32 ? PROF(F16, F32) : PROF(F16, F16);
    return xdtype == F32 ? PROF(Q4, F32) : PROF(Q4, F16);
#undef PROF
}

pi_status pi_build_neuron_index(const uint32_t* counts, int32_t n, int64_t budget_bytes,
                                int64_t bytes_per_neuron, int32_t* perm, int32_t* n_hot,
                                void* stream) {
    CHECK(n >= 0 && n <= (1 << 24), PI_ERR_SHAPE, "n must be in 0..2^24");
    CHECK(budget_bytes >= 0 && bytes_per_neuron > 0, PI_ERR_BUDGET,
          "budget must be >= 0 and bytes_per_neuron > 0");
    CHECK(n_hot, PI_ERR_ARG, "n_hot required");
    CHECK(n == 0 || (counts && perm && aligned(counts, 4) && aligned(perm, 4)), PI_ERR_ARG,
          "counts and perm required");
    const int64_t k = budget_bytes / bytes_per_neuron;
    *n_hot = (int32_t)(k < n ? k : n);
    if (n == 0) return PI_OK;
    return launch(PI_K_INDEX, k_index, dim3((n + THREADS - 1) / THREADS), dim3(THREADS), 0,
                  (hipStream_t)stream, counts, n, perm);
}

pi_status pi_plan_hot_split(const uint32_t* counts_slot, int32_t n, int64_t budget_bytes,
                            int64_t bytes_per_neuron, double hbm_gbps, double link_gbps,
                            int32_t* n_hot) {
    CHECK(n >= 0 && n <= (1 << 24), PI_ERR_SHAPE, "n must be in 0..2^24");
    CHECK(budget_bytes >= 0 && bytes_per_neuron > 0, PI_ERR_BUDGET,
          "budget must be >= 0 and bytes_per_neuron > 0");
    CHECK(hbm_gbps > 0.0 && link_gbps > 0.0 && hbm_gbps < 1e300 && link_gbps < 1e300, PI_ERR_ARG,
          "read rates must be positive and finite");
    CHECK(n_hot && (n == 0 || counts_slot), PI_ERR_ARG, "counts and n_hot required");
    // expected activations read from each tier per step for every split point K:
    // hot = counts of slots [0, K), cold = the rest; each tier's read time is its
    // activations over its rate, and the tiers overlap, so a step costs the larger
    std::vector<uint64_t> prefix((size_t)n + 1, 0);
    for (int32_t s = 0; s < n; ++s) prefix[s + 1] = prefix[s] + counts_slot[s];
    const uint64_t total = prefix[n];
    int32_t best = 0;
    double best_t = 0.0;
    for (int32_t K = 0; K <= n; ++K) {
        const double t_hot = (double)prefix[K] / hbm_gbps;
        const double t_cold = (double)(total - prefix[K]) / link_gbps;
        const double t = std::max(t_hot, t_cold);
        if (K == 0 || t < best_t) {                  // ties keep the smaller split
            best_t = t;
            best = K;
        }
    }
    const int64_t cap = budget_bytes / bytes_per_neuron;
    *n_hot = (int32_t)std::min<int64_t>(std::min<int64_t>(best, cap), n);
    return PI_OK;
}

size_t pi_calibrate_workspace_bytes(int32_t d, int32_t n, int32_t r, int32_t S) {
    if (d <= 0 || n <= 0 || r <= 0 || S <= 0 || (int64_t)S * n > (int64_t)1 << 31) return 0;
    size_t off[5];
    return calib_layout(d, n, r, S, off);
}

pi_status pi_calibrate_threshold(const pi_predictor* p, const pi_ffn_part* part, const void* X,
                                 int32_t S, int32_t xdtype, double target_recall, float* tau,
                                 uint32_t* stats, void* ws, size_t ws_bytes, void* stream) {
    CHECK(p && part, PI_ERR_ARG, "predictor and partition required");
    CHECK(p->wdtype == PI_F32 || p->wdtype == PI_F16, PI_ERR_DTYPE, "predictor wdtype must be PI_F32 or PI_F16");
    TRY(check_dtype_x(xdtype));
    TRY(check_part(part, "part", false));
    CHECK(p->d > 0 && p->d % 64 == 0 && p->r > 0 && p->r % 16 == 0 && p->r <= 4096, PI_ERR_SHAPE,
          "predictor d or r out of range");
    CHECK(part->rows == p->n && part->d == p->d, PI_ERR_SHAPE,
          "the partition must be the whole layer (rows == n, same d) in the predictor's neuron order");
    CHECK(S >= 1 && (int64_t)S * p->n <= (int64_t)1 << 31, PI_ERR_SHAPE, "S * n must be in 1..2^31");
    CHECK(target_recall > 0.0 && target_recall <= 1.0, PI_ERR_ARG, "target_recall must be in (0, 1]");
    CHECK(p->P1t && p->P2t && X && tau && stats, PI_ERR_ARG, "P1t, P2t, X, tau and stats required");
    CHECK(aligned(p->P1t, 16) && aligned(p->P2t, 16) && aligned(X, 16) && aligned(tau, 4) && aligned(stats, 4) &&
          aligned(p->b2, 4), PI_ERR_ALIGN, "misaligned pointer");
    size_t off[5];
    TRY(check_ws(ws, ws_bytes, calib_layout(p->d, p->n, p->r, S, off)));
    uint8_t* base = static_cast<uint8_t*>(ws);
    float* logits = reinterpret_cast<float*>(base + off[0]);
    uint32_t* keys = reinterpret_cast<uint32_t*>(base + off[1]);
    uint32_t* hist = reinterpret_cast<uint32_t*>(base + off[2]);
    uint32_t* state = hist + SEL_BINS;
    uint64_t* mask = reinterpret_cast<uint64_t*>(base + off[3]);
    hipStream_t s = (hipStream_t)stream;
    // 1. the predictor's logits for every sample, in batches the library computes at decode
    const int64_t xrow = (int64_t)p->d * (xdtype == PI_F32 ? 4 : 2);
    for (int s0 = 0; s0 < S; s0 += PI_MAX_BATCH) {
        const int nb = std::min(PI_MAX_BATCH, S - s0);
        TRY(predict_launch(p, static_cast<const uint8_t*>(X) + s0 * xrow, nb, xdtype, mask,
                           logits + (int64_t)s0 * p->n, base + off[4], s));
    }
    // 2. keys of the firing pairs
    const bool reglu = part->act == PI_REGLU;
    const uint8_t* W = (const uint8_t*)(reglu ? part->W_gate : part->W_up);
    const float* bias = reglu ? part->b_gate : part->b_up;
    const int grid = (part->rows + NWAVES - 1) / NWAVES;
    const int wt = part->wdtype;
#define FIRE(WT_, XT_) launch(PI_K_PROFILE, k_fire_keys<WT_, XT_, 8>, dim3(grid), dim3(THREADS), 0, s, \
                              W, bias, (const uint8_t*)X, part->d, part->rows, S, (const float*)logits, keys)
    if (wt == F32) TRY(xdtype == F32 ? FIRE(F32, F32) : FIRE(F32, F16));
    else if (wt == F16) TRY(xdtype == F32 ? FIRE(F16, F32) : FIRE(F16, F16));
    else TRY(xdtype == F32 ? FIRE(Q4, F32) : FIRE(Q4, F16));
#undef FIRE
    // 3. exact selection of the m-th largest key: digits of 11, 11 and 10 bits
    const int64_t len = (int64_t)S * p->n;
    const int64_t n16 = (SEL_BINS + 8) * 4 / 16;
    TRY(launch(PI_K_INDEX, k_zero, dim3(1), dim3(THREADS), 0, s, reinterpret_cast<u4*>(hist), n16));
    int hgrid = (int)std::min<int64_t>(1024, (len + THREADS - 1) / THREADS);
    const int shifts[3] = {21, 10, 0}, bits[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        TRY(launch(PI_K_INDEX, k_key_hist, dim3(hgrid), dim3(THREADS), 0, s, (const uint32_t*)keys, len,
                   (const uint32_t*)state, shifts[pass], bits[pass], hist));
        TRY(launch(PI_K_INDEX, k_key_select, dim3(1), dim3(THREADS), 0, s, hist, shifts[pass], bits[pass],
                   pass == 0 ? 1 : 0, target_recall, state));
    }
    TRY(launch(PI_K_INDEX, k_key_finish, dim3(1), dim3(64), 0, s, (const uint32_t*)state, tau, stats));
    return launch(PI_K_INDEX, k_key_count, dim3(hgrid), dim3(THREADS), 0, s, (const uint32_t*)keys, len,
                  (const float*)tau, stats);
}

pi_status pi_true_mask(const pi_ffn_part* part, const void* x, int32_t B, int32_t xdtype,
                       uint64_t* mask, void* stream) {
    TRY(check_part(part, "part", false));
    TRY(check_dtype_x(xdtype));
    CHECK(B >= 1 && B <= PI_MAX_BATCH, PI_ERR_SHAPE, "B must be in 1..%d", PI_MAX_BATCH);
    CHECK(x && mask && aligned(x, 16) && aligned(mask, 8), PI_ERR_ARG, "x (16-byte) and mask (8-byte) required");
    const bool reglu = part->act == PI_REGLU;
    const uint8_t* W = (const uint8_t*)(reglu ? part->W_gate : part->W_up);
    const float* bias = reglu ? part->b_gate : part->b_up;
    const int grid = (part->rows + 63) / 64;
    hipStream_t s = (hipStream_t)stream;
    const int wt = part->wdtype;
#define TM(WT_, XT_) launch(PI_K_PROFILE, k_true_mask<WT_, XT_>, dim3(grid), dim3(THREADS), 0, s, \
                            W, bias, (const uint8_t*)x, part->d, part->rows, B, mask)
    if (wt == F32) return xdtype == F32 ? TM(F32, F32) : TM(F32, F16);
    if (wt == F16) return xdtype == F32 ? TM(F16, F32) : TM(F16, F16);
    return xdtype == F32 ? TM(Q4, F32) : TM(Q4, F16);
#undef TM
}

pi_status pi_host_sparse_ffn(const pi_ffn_part* part, const void* x, int32_t B, int32_t xdtype,
                             const int32_t* idx, int32_t count, float* y, int32_t threads) {
    TRY(check_part(part, "part", true));
    TRY(check_dtype_x(xdtype));
    CHECK(B >= 1 && B <= PI_MAX_BATCH, PI_ERR_SHAPE, "B must be in 1..%d", PI_MAX_BATCH);
    CHECK(x && y, PI_ERR_ARG, "x and y required");
    CHECK(count >= 0, PI_ERR_SHAPE, "count must be >= 0");
    CHECK(count == 0 || idx, PI_ERR_ARG, "idx required for count > 0");
    CHECK(threads >= 0, PI_ERR_ARG, "threads must be >= 0");
    host::sparse_ffn(*part, x, B, xdtype, idx, part->rows > 0 ? count : 0, y, threads);
    return PI_OK;
}

size_t pi_hybrid_host_bytes(int32_t d, int32_t n, int32_t B) {
    if (d <= 0 || n <= 0 || n > (1 << 24) || B <= 0 || B > PI_MAX_BATCH) return 0;
    size_t off[4];
    return hybrid_host_layout(d, n, B, off);
}

pi_status pi_sparse_ffn_hybrid(const pi_ffn_part* hot, const pi_ffn_part* cold, const void* x,
                               int32_t B, int32_t xdtype, const uint64_t* mask,
                               const pi_active_lists* lists, float* y_cold, float* y, void* ws,
                               size_t ws_bytes, void* host_ws, size_t host_ws_bytes,
                               int32_t threads, pi_hybrid_info* info, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    TRY(check_part(hot, "hot", true));
    CHECK(cold, PI_ERR_ARG, "cold partition required (it may have 0 rows)");
    TRY(check_part(cold, "cold", true));
    CHECK(cold->d == hot->d && cold->wdtype == hot->wdtype && cold->act == hot->act, PI_ERR_SHAPE,
          "hot and cold partitions differ in d, wdtype or act");
    TRY(check_dtype_x(xdtype));
    CHECK(B >= 1 && B <= PI_MAX_BATCH, PI_ERR_SHAPE, "B must be in 1..%d", PI_MAX_BATCH);
    CHECK(x && aligned(x, 16), x ? PI_ERR_ALIGN : PI_ERR_ARG, "x must be non-NULL and 16-byte aligned");
    CHECK(mask && aligned(mask, 8), mask ? PI_ERR_ALIGN : PI_ERR_ARG, "mask must be non-NULL and 8-byte aligned");
    CHECK(lists && lists->n_hot == hot->rows, PI_ERR_SHAPE, "lists required with n_hot == hot->rows");
    CHECK(y_cold && y && aligned(y_cold, 16) && aligned(y, 16), PI_ERR_ARG,
          "y_cold and y required (16-byte aligned)");
    CHECK(threads >= 0, PI_ERR_ARG, "threads must be >= 0");
    const int d = hot->d;
    const int64_t n64 = (int64_t)hot->rows + cold->rows;
    CHECK(n64 >= 1 && n64 <= (1 << 24), PI_ERR_SHAPE, "hot rows + cold rows must be in 1..2^24");
    const int n = (int)n64;
    size_t off[4];
    const size_t hneed = hybrid_host_layout(d, n, B, off);
    CHECK(host_ws && aligned(host_ws, 64), PI_ERR_ARG, "host_ws required (64-byte aligned)");
    CHECK(host_ws_bytes >= hneed, PI_ERR_WORKSPACE, "host_ws has %zu bytes, needs %zu", host_ws_bytes, hneed);
    CHECK(memory_type(host_ws) == hipMemoryTypeHost, PI_ERR_ARG, "host_ws must be pinned host memory (hipHostMalloc)");
    if (cold->rows > 0) {
        const void* w[3] = {cold->W_up, cold->W_downT, cold->act == PI_REGLU ? cold->W_gate : nullptr};
        for (const void* p : w)
            CHECK(!p || memory_type(p) != hipMemoryTypeDevice, PI_ERR_ARG,
                  "cold weights must be in host memory (the host cores read them)");
        const float* b[2] = {cold->b_up, cold->b_gate};
        for (const float* p : b)
            CHECK(!p || memory_type(p) != hipMemoryTypeDevice, PI_ERR_ARG, "cold biases must be in host memory");
    }
    if (hot->rows > 0)
        TRY(ffn_common(hot, nullptr, x, B, xdtype, mask, lists->hot_idx, nullptr, lists->counts, false, nullptr,
                       nullptr, y, ws, ws_bytes, s, false, 0, /*check_only=*/true));
    hipEvent_t arrive;
    TRY(arrival_event(s, &arrive));

    // the device's address of the host workspace (pinned memory is mapped for the GPU)
    void* hdev = nullptr;
    hipError_t e = hipHostGetDevicePointer(&hdev, host_ws, 0);
    if (e != hipSuccess || !hdev) {
        (void)hipGetLastError();
        return fail(PI_ERR_ARG, "host_ws is not mapped for the device (allocate it with hipHostMalloc)");
    }
    uint8_t* hd = static_cast<uint8_t*>(hdev);

    // 1. mask and x to host memory, then the hot partition behind them on the GPU
    uint8_t* hb = static_cast<uint8_t*>(host_ws);
    const int words = (n + 63) / 64;
    const int x16 = (int)((size_t)B * d * (xdtype == PI_F32 ? 4 : 2) / 16);
    TRY(launch(PI_K_MERGE, k_export, dim3((std::max(words, x16) + THREADS - 1) / THREADS), dim3(THREADS), 0, s,
               mask, words, (const uint4*)x, x16, (uint64_t*)(hd + off[0]), (uint4*)(hd + off[1])));
    e = hipEventRecord(arrive, s);
    if (e != hipSuccess) return fail(PI_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
    if (hot->rows > 0)
        TRY(ffn_common(hot, nullptr, x, B, xdtype, mask, lists->hot_idx, nullptr, lists->counts, false, nullptr,
                       nullptr, y, ws, ws_bytes, s));

    // 2. the cold partition on the host cores while the GPU runs the hot one
    const auto t0 = std::chrono::steady_clock::now();
    e = hipEventSynchronize(arrive);
    if (e != hipSuccess) return fail(PI_ERR_HIP, "waiting for mask and x: %s", hipGetErrorString(e));
    const double wait_us = us_since(t0);
    const auto t1 = std::chrono::steady_clock::now();
    int32_t* ids = reinterpret_cast<int32_t*>(hb + off[3]);
    float* yc = reinterpret_cast<float*>(hb + off[2]);
    const int count = cold->rows > 0 ? host::cold_list(reinterpret_cast<const uint64_t*>(hb + off[0]), hot->rows, n, ids) : 0;
    host::sparse_ffn(*cold, hb + off[1], B, xdtype, ids, count, yc, threads);
    const double host_us = us_since(t1);
    if (info) {
        info->cold_count = count;
        info->threads = std::max(1, std::min({threads > 0 ? threads : host::threads_available(),
                                               host::threads_available(), std::max(count, 1)}));
        info->wait_us = wait_us;
        info->host_us = host_us;
    }

    // 3. y_cold = the host's partial (read from host memory), y = hot partial + y_cold
    const int64_t len4 = (int64_t)B * d / 4;
    const int grid = (int)std::min<int64_t>((len4 + THREADS - 1) / THREADS, 1024);
    return launch(PI_K_MERGE, k_merge_host, dim3(grid), dim3(THREADS), 0, s, (const float4*)(hd + off[2]), len4,
                  hot->rows > 0, (float4*)y_cold, (float4*)y);
}

pi_status pi_accumulate_mask(const uint64_t* mask, int32_t n, uint32_t* counts, void* stream) {
    CHECK(n >= 1 && n <= (1 << 24), PI_ERR_SHAPE, "n must be in 1..2^24");
    CHECK(mask && counts, PI_ERR_ARG, "mask and counts required");
    CHECK(aligned(mask, 8) && aligned(counts, 4), PI_ERR_ALIGN, "misaligned mask or counts");
    return launch(PI_K_ACCUMULATE, k_accumulate_mask, dim3((n + THREADS - 1) / THREADS), dim3(THREADS),
                  0, (hipStream_t)stream, mask, n, counts);
}

pi_status pi_permute_rows(const void* src, void* dst, const int32_t* perm, int32_t rows,
                          int64_t row_bytes_, void* stream) {
    CHECK(rows >= 0 && row_bytes_ > 0 && row_bytes_ % 4 == 0, PI_ERR_SHAPE,
          "rows >= 0 and row_bytes a positive multiple of 4");
    if (rows == 0) return PI_OK;
    CHECK(src && dst && perm, PI_ERR_ARG, "src, dst and perm required");
    CHECK(aligned(src, 4) && aligned(dst, 4) && aligned(perm, 4), PI_ERR_ALIGN, "misaligned");
    const uint8_t* s0 = (const uint8_t*)src;
    const uint8_t* d0 = (const uint8_t*)dst;
    const int64_t total = (int64_t)rows * row_bytes_;
    CHECK(d0 + total <= s0 || s0 + total <= d0, PI_ERR_ARG, "src and dst overlap");
    return launch(PI_K_COPY, k_permute_rows, dim3(rows), dim3(THREADS), 0, (hipStream_t)stream,
                  (const uint32_t*)src, (uint32_t*)dst, perm, row_bytes_ / 4);
}

pi_status pi_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    CHECK(bytes >= 0 && bytes % 16 == 0, PI_ERR_SHAPE, "bytes must be a multiple of 16");
    if (bytes == 0) return PI_OK;
    CHECK(src && dst && aligned(src, 16) && aligned(dst, 16), PI_ERR_ALIGN, "src/dst 16-byte aligned");
    const int64_t n16 = bytes / 16;
    int64_t grid = (n16 + THREADS - 1) / THREADS;
    if (grid > 8192) grid = 8192;
    return launch(PI_K_COPY, k_copy, dim3((unsigned)grid), dim3(THREADS), 0, (hipStream_t)stream,
                  (const u4*)src, (u4*)dst, n16);
}

pi_status pi_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    CHECK(bytes >= 0 && bytes % 16 == 0, PI_ERR_SHAPE, "bytes must be a multiple of 16");
    CHECK(sink && aligned(sink, 4), PI_ERR_ARG, "sink required (4-byte aligned)");
    CHECK(bytes == 0 || (src && aligned(src, 16)), PI_ERR_ALIGN, "src must be 16-byte aligned");
    const int64_t n16 = bytes / 16;
    return launch(PI_K_STREAM, k_stream_read, dim3(STREAM_WG), dim3(THREADS), 0, (hipStream_t)stream,
                  (const u4*)src, n16, sink);
}

pi_status pi_kernel_timer_start(int32_t kid, int32_t max_launches) {
    CHECK(kid >= 0 && kid < PI_K_COUNT, PI_ERR_ARG, "bad kernel id");
    CHECK(max_launches >= 1 && max_launches <= 100000, PI_ERR_ARG, "max_launches in 1..100000");
    Timer& t = g_timers[kid];
    while ((int)t.ev.size() < 2 * max_launches) {
        hipEvent_t e;
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return fail(PI_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(err));
        t.ev.push_back(e);
    }
    t.armed = true;
    t.max = max_launches;
    t.used = 0;
    return PI_OK;
}

pi_status pi_kernel_timer_stop(int32_t kid, float* total_ms, int32_t* launches) {
    CHECK(kid >= 0 && kid < PI_K_COUNT, PI_ERR_ARG, "bad kernel id");
    CHECK(total_ms && launches, PI_ERR_ARG, "outputs required");
    Timer& t = g_timers[kid];
    float sum = 0.0f;
    for (int i = 0; i < t.used; ++i) {
        hipError_t err = hipEventSynchronize(t.ev[2 * i + 1]);
        if (err != hipSuccess) return fail(PI_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(err));
        float ms = 0.0f;
        err = hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]);
        if (err != hipSuccess) return fail(PI_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(err));
        sum += ms;
    }
    *total_ms = sum;
    *launches = t.used;
    t.armed = false;
    t.used = 0;
    return PI_OK;
}

}  // extern "C"
