// la_api.cpp -- the C ABI of liblinattn: host-side validation, work planning
// (chunks, segments, windows, workspace) and kernel dispatch.
//
// Every argument is checked on the host before anything is enqueued; no call
// allocates, frees or synchronises.  See include/la.h for the contract.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "la_internal.h"

using namespace la;

namespace {

thread_local std::string g_last_error;

la_status fail(la_status s, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

la_status ok()
{
    return LA_OK;
}

la_status hip_fail(hipError_t e, const char* what)
{
    return fail(LA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- per-launch timing for la_profile_begin / la_profile_end
struct Profiler {
    bool on = false;
    int max = 0;
    int used = 0;
    std::vector<hipEvent_t> ev;  // 2 per launch
    std::vector<int> ids;
};
thread_local Profiler g_prof;
thread_local LaunchEvents g_launch_ev = {nullptr, nullptr, false};

void prof_before(int id)
{
    if (!g_prof.on || g_prof.used >= g_prof.max) return;
    g_launch_ev = {g_prof.ev[2 * g_prof.used], g_prof.ev[2 * g_prof.used + 1], false};
    g_prof.ids[g_prof.used] = id;
}

void prof_after()
{
    // a call that launched nothing (empty copy, say) leaves no record
    if (g_launch_ev.fired) ++g_prof.used;
    g_launch_ev = {nullptr, nullptr, false};
}

// Launch through `fn`; while recording is on, the kernel it launches stores
// its own start and end timestamps in the next pair of events.
template <class Fn>
hipError_t launch(int id, Fn&& fn)
{
    prof_before(id);
    const hipError_t e = fn();
    prof_after();
    return e;
}

}  // namespace

int la::device_slots(const void* kernel, int threads)
{
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, int> cache;  // (kernel, device) -> slots
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(kernel, dev);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
        return 0;
    const int slots = cus * (per_cu > 0 ? per_cu : 1);
    cache[key] = slots;
    return slots;
}

LaunchEvents& la::launch_events()
{
    return g_launch_ev;
}

namespace {

bool is_rf(int kind)
{
    return kind == LA_PHI_TRIG_RF || kind == LA_PHI_TRIG_RF_PLAIN || kind == LA_PHI_TRIG_RF_SOFTMAX;
}

// The kernel family of a feature-map kind: the three random-feature kinds
// share one kernel and differ only in the prefactor's sign.
int kernel_phi(int kind)
{
    return is_rf(kind) ? LA_PHI_TRIG_RF : kind;
}

// s in the random-feature prefactor exp(s |x'|^2 / 2) / sqrt(m)
float rf_sign(int kind)
{
    return kind == LA_PHI_TRIG_RF ? -1.f : (kind == LA_PHI_TRIG_RF_SOFTMAX ? 1.f : 0.f);
}

const KernelEntry* find_entry(int in_dtype, int phi, int dk, int F, int dv)
{
    const KernelEntry* tables[] = {kEntriesBf16Elu, kEntriesBf16Rf, kEntriesBf16Relu, kEntriesF32, kEntriesF32Relu,
                                   kEntriesIdentBf16, kEntriesIdentF32};
    const int counts[] = {kNumEntriesBf16Elu, kNumEntriesBf16Rf, kNumEntriesBf16Relu, kNumEntriesF32,
                          kNumEntriesF32Relu, kNumEntriesIdentBf16, kNumEntriesIdentF32};
    for (int t = 0; t < 7; ++t)
        for (int i = 0; i < counts[t]; ++i) {
            const KernelEntry& e = tables[t][i];
            if (e.in_dtype == in_dtype && e.phi == phi && e.dk == dk && e.F == F && e.dv == dv) return &e;
        }
    return nullptr;
}

bool aligned16(const void* p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

size_t elem_size(int dtype)
{
    return dtype == LA_BF16 ? 2 : 4;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// Shape and feature-map checks shared by every entry point.  On success sets
// F and the kernel table entry.  split_ok: the caller runs a map of F = 512
// (m = 256 random features, bf16, d_k = 64) as two halves of 256 features;
// the entry is then that of one half.
la_status check_shape(const la_shape* s, const la_phi* phi, int64_t min_n, int64_t max_n,
                      int* F_out, const KernelEntry** entry_out, bool split_ok = false)
{
    if (!s) return fail(LA_ERR_INVALID_ARGUMENT, "shape is NULL");
    if (!phi) return fail(LA_ERR_INVALID_ARGUMENT, "phi is NULL");
    if (s->B < 1 || s->H < 1) return fail(LA_ERR_INVALID_ARGUMENT, "B and H must be >= 1 (got B=%lld H=%lld)",
                                          (long long)s->B, (long long)s->H);
    if (s->N < min_n || s->N > max_n)
        return fail(LA_ERR_INVALID_ARGUMENT, "N=%lld outside [%lld, %lld]", (long long)s->N, (long long)min_n,
                    (long long)max_n);
    if (s->H > LA_MAX_HEADS) return fail(LA_ERR_UNSUPPORTED, "H=%lld exceeds LA_MAX_HEADS=%d", (long long)s->H, LA_MAX_HEADS);
    if (s->d_k < 1 || s->d_v < 1) return fail(LA_ERR_INVALID_ARGUMENT, "d_k and d_v must be >= 1");
    if (s->in_dtype != LA_F32 && s->in_dtype != LA_BF16) return fail(LA_ERR_INVALID_ARGUMENT, "unknown in_dtype %d", s->in_dtype);
    if (s->out_dtype != LA_F32 && s->out_dtype != LA_BF16) return fail(LA_ERR_INVALID_ARGUMENT, "unknown out_dtype %d", s->out_dtype);
    if (s->out_dtype != s->in_dtype && s->out_dtype != LA_F32)
        return fail(LA_ERR_UNSUPPORTED, "out_dtype must equal in_dtype or be LA_F32");
    if ((s->d_k != 64 && s->d_k != 128) || (s->d_v != 64 && s->d_v != 128))
        return fail(LA_ERR_UNSUPPORTED, "d_k=%d d_v=%d: supported head sizes are 64 and 128", s->d_k, s->d_v);
    int F = 0;
    if (phi->kind == LA_PHI_ELU1 || phi->kind == LA_PHI_RELU) {
        if (phi->m != 0 || phi->omega != nullptr)
            return fail(LA_ERR_INVALID_ARGUMENT, "elementwise feature maps take m = 0 and omega = NULL");
        if (phi->qk_scale != 1.0f) return fail(LA_ERR_INVALID_ARGUMENT, "elementwise feature maps take qk_scale = 1");
        F = s->d_k;
    } else if (is_rf(phi->kind)) {
        if (phi->m < 1) return fail(LA_ERR_INVALID_ARGUMENT, "random features need m >= 1 (got %d)", phi->m);
        if (!phi->omega) return fail(LA_ERR_INVALID_ARGUMENT, "random features need omega");
        if (!aligned16(phi->omega)) return fail(LA_ERR_INVALID_ARGUMENT, "omega must be 16-byte aligned");
        if (!std::isfinite(phi->qk_scale) || phi->qk_scale <= 0.f)
            return fail(LA_ERR_INVALID_ARGUMENT, "qk_scale must be finite and > 0");
        if (phi->m == 256) {
            if (!split_ok || s->in_dtype != LA_BF16 || s->d_k != 64 || s->d_v != 64)
                return fail(LA_ERR_UNSUPPORTED,
                            "m=256 random features are supported by the causal forward with bf16 inputs and "
                            "d_k = d_v = 64");
            const KernelEntry* e = find_entry(s->in_dtype, LA_PHI_TRIG_RF, s->d_k, 256, s->d_v);
            if (!e) return fail(LA_ERR_UNSUPPORTED, "no kernel for m=256 halves with d_v=%d", s->d_v);
            *F_out = 512;
            *entry_out = e;
            return LA_OK;
        }
        if (phi->m != 32 && phi->m != 64 && phi->m != 128)
            return fail(LA_ERR_UNSUPPORTED, "m=%d: supported random-feature counts are 32, 64, 128, 256", phi->m);
        if ((int64_t)s->d_k * phi->m > 8192) return fail(LA_ERR_UNSUPPORTED, "d_k * m must be <= 8192");
        F = 2 * phi->m;
    } else {
        return fail(LA_ERR_INVALID_ARGUMENT, "unknown feature map kind %d", phi->kind);
    }
    const KernelEntry* e = find_entry(s->in_dtype, kernel_phi(phi->kind), s->d_k, F, s->d_v);
    if (!e) return fail(LA_ERR_UNSUPPORTED, "no kernel for dtype=%d phi=%d d_k=%d F=%d d_v=%d", s->in_dtype, phi->kind,
                        s->d_k, F, s->d_v);
    *F_out = F;
    *entry_out = e;
    return LA_OK;
}

la_status make_lam(const float* lambda_h, int64_t H, LamTable* t)
{
    std::memset(t, 0, sizeof(*t));
    for (int64_t h = 0; h < H; ++h) {
        const float l = lambda_h ? lambda_h[h] : 1.0f;
        if (!std::isfinite(l) || l < 0.f || l > 1.f)
            return fail(LA_ERR_INVALID_ARGUMENT, "lambda_h[%lld]=%g outside [0, 1]", (long long)h, (double)l);
        t->lam[h] = l;
        t->log2lam[h] = (l == 0.f) ? -INFINITY : (float)std::log2((double)l);
    }
    return LA_OK;
}

int env_int(const char* name, int dflt)
{
    const char* v = std::getenv(name);
    if (!v || !*v) return dflt;
    return std::atoi(v);
}

// Work plan of one forward call.
struct Plan {
    int C;          // chunk length
    int Pmax;       // upper bound of segments per window (sizes the workspace)
    int W;          // windows
    int64_t SZ;     // floats per state slot: F*d_v + F
    size_t ws_bytes;
};

// Number of workgroups per pass the planner aims for: two per compute unit of
// an MI355X (256 CUs).
constexpr int kTargetWorkgroups = 512;

// Workgroups a causal forward over fixed rows aims for: one per compute unit
// where the segment-state pass streams elementwise bf16 features of width 128
// or more (it is bound by its stream of loads, and fewer, longer segments
// write and scan fewer states; the causal output kernel of that width holds
// one workgroup per unit anyway), two elsewhere (the random-feature state
// pass is bound by its arithmetic and gains from the second workgroup).
int64_t causal_target_workgroups(const KernelEntry* e, int F)
{
    return (e->in_dtype == LA_BF16 && e->phi != LA_PHI_TRIG_RF && F >= 128) ? kTargetWorkgroups / 2
                                                                            : kTargetWorkgroups;
}

// Segments wanted for a row of NC chunks (before rounding to whole chunks).
// max_P: an upper bound on the segments (the static-scratch forward caps them
// so that their states fit its scratch).
int64_t target_segments(int64_t NC, int64_t BH, int64_t max_P = INT64_MAX, int64_t target = kTargetWorkgroups)
{
    int64_t P = (target + BH - 1) / BH;
    const int forced = env_int("LA_SEGMENTS", 0);
    if (forced > 0) P = forced;
    if (P > max_P) P = max_P;
    if (P > NC) P = NC;
    if (P < 1) P = 1;
    return P;
}

// Cut NC chunks into segments of cps chunks: every segment but the last is full.
void cut_segments(int64_t NC, int64_t BH, int* P, int64_t* cps, int64_t max_P = INT64_MAX,
                  int64_t target = kTargetWorkgroups)
{
    const int64_t Pt = target_segments(NC, BH, max_P, target);
    *cps = (NC + Pt - 1) / Pt;
    *P = (int)((NC + *cps - 1) / *cps);
}

// Segments of packed variable-length rows: one length of cps chunks for every
// sequence, sized so that the head-sequences' segments number about
// kTargetWorkgroups in all (total chunks per head row <= T/C + B), and P grid
// segments to cover the longest sequence (the last one takes any remainder,
// so an understated max_len costs speed, not correctness).
void varlen_segments(int64_t T, int64_t B, int64_t H, int64_t max_len, int C, int* P, int64_t* cps)
{
    const int64_t chunks = ((T + C - 1) / C + B) * H;
    int64_t c = (chunks + kTargetWorkgroups - 1) / kTargetWorkgroups;
    if (c < 1) c = 1;
    int64_t p = ((max_len + C - 1) / C + c - 1) / c;
    if (p < 1) p = 1;
    if (p > 65535) {  // grid limit: longer segments instead
        c = ((max_len + C - 1) / C + 65534) / 65535;
        p = ((max_len + C - 1) / C + c - 1) / c;
    }
    *cps = c;
    *P = (int)p;
}

// Work items per head of packed sequences: sum_b max(1, min(ceil(chunks_b /
// cps), P)) <= ceil((ceil(T / C) + B) / cps) + B, and <= B * P.
int64_t varlen_items_bound(int64_t T, int64_t B, int C, int64_t cps, int P)
{
    int64_t G = ((T + C - 1) / C + B + cps - 1) / cps + B;
    return G < B * (int64_t)P ? G : B * (int64_t)P;
}

size_t bytes256(size_t n) { return (n + 255) & ~size_t(255); }

// Plan of a forward over rows of N tokens (causal: may be cut into windows).
// varlen_P > 0: packed variable-length rows cut into varlen_P segments, one window.
Plan make_plan(const la_shape* s, int F, const KernelEntry* e, bool causal, int varlen_P = 0,
               int64_t max_P = INT64_MAX)
{
    Plan p;
    p.C = e->C;
    p.SZ = (int64_t)F * s->d_v + F;
    const int64_t BH = s->B * s->H;
    const int64_t NC = (s->N + p.C - 1) / p.C;
    int W = (causal && varlen_P == 0) ? env_int("LA_WINDOWS", 1) : 1;
    if (W < 1) W = 1;
    if (W > NC) W = (int)(NC > 0 ? NC : 1);
    p.W = W;
    // every window has at most NC chunks, so it is cut into at most this many segments
    p.Pmax = varlen_P > 0 ? varlen_P
                          : (int)target_segments(NC > 0 ? NC : 1, BH, max_P,
                                                 causal ? causal_target_workgroups(e, F) : kTargetWorkgroups);
    size_t floats = 0;
    if (causal) {
        if (p.Pmax > 1) floats += (size_t)p.Pmax * BH * p.SZ;
        if (p.W > 1) floats += (size_t)BH * p.SZ;
    } else {
        floats += (size_t)p.Pmax * BH * p.SZ;
    }
    p.ws_bytes = floats ? ((floats * sizeof(float) + 255) & ~size_t(255)) : 0;
    return p;
}

la_status check_ws(const Plan& p, void* ws, size_t ws_bytes)
{
    if (p.ws_bytes == 0) return LA_OK;
    if (!ws) return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", p.ws_bytes);
    if (ws_bytes < p.ws_bytes) return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", p.ws_bytes, ws_bytes);
    if (!aligned16(ws)) return fail(LA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    return LA_OK;
}

// Pointer checks for q, y with rows_q rows and k, v with rows_k rows.
la_status check_io_rows(const void* q, const void* k, const void* v, const void* y, const la_shape* s,
                        size_t rows_q, size_t rows_k)
{
    if (!q || !k || !v || !y) return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v and y must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y))
        return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v, y must be 16-byte aligned");
    const size_t es = elem_size(s->in_dtype);
    const size_t nq = rows_q * s->d_k * es, nk = rows_k * s->d_k * es, nv = rows_k * s->d_v * es;
    const size_t ny = rows_q * s->d_v * elem_size(s->out_dtype);
    if (overlaps(y, ny, q, nq) || overlaps(y, ny, k, nk) || overlaps(y, ny, v, nv))
        return fail(LA_ERR_INVALID_ARGUMENT, "y must not alias q, k or v");
    return LA_OK;
}

la_status check_io(const void* q, const void* k, const void* v, const void* y, const la_shape* s)
{
    const size_t rows = (size_t)s->B * s->H * s->N;
    return check_io_rows(q, k, v, y, s, rows, rows);
}

la_status check_eps(float eps)
{
    if (!std::isfinite(eps) || eps < 0.f) return fail(LA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0 (got %g)", (double)eps);
    return LA_OK;
}

}  // namespace

extern "C" {

const char* la_status_string(la_status s)
{
    switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARGUMENT: return "LA_ERR_INVALID_ARGUMENT";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE";
    case LA_ERR_HIP: return "LA_ERR_HIP";
    }
    return "LA_ERR_UNKNOWN";
}

const char* la_last_error(void)
{
    return g_last_error.c_str();
}

la_status la_profile_begin(int32_t max_launches)
{
    if (g_prof.on) return fail(LA_ERR_INVALID_ARGUMENT, "profiling already on");
    if (max_launches < 1) return fail(LA_ERR_INVALID_ARGUMENT, "max_launches must be >= 1");
    g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
    g_prof.ids.assign((size_t)max_launches, -1);
    for (size_t i = 0; i < g_prof.ev.size(); ++i) {
        const hipError_t e = hipEventCreate(&g_prof.ev[i]);
        if (e != hipSuccess) {
            for (size_t j = 0; j < i; ++j) hipEventDestroy(g_prof.ev[j]);
            g_prof.ev.clear();
            return hip_fail(e, "hipEventCreate");
        }
    }
    g_prof.max = max_launches;
    g_prof.used = 0;
    g_prof.on = true;
    return ok();
}

la_status la_profile_end(int32_t* kernel_ids, float* ms, int32_t capacity, int32_t* count)
{
    if (!g_prof.on) return fail(LA_ERR_INVALID_ARGUMENT, "profiling is not on");
    la_status st = LA_OK;
    int n = 0;
    if (g_prof.used > 0) {
        const hipError_t e = hipEventSynchronize(g_prof.ev[2 * g_prof.used - 1]);
        if (e != hipSuccess) st = hip_fail(e, "hipEventSynchronize");
    }
    for (int i = 0; st == LA_OK && i < g_prof.used && i < capacity; ++i) {
        float t = 0.f;
        const hipError_t e = hipEventElapsedTime(&t, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
        if (e != hipSuccess) {
            st = hip_fail(e, "hipEventElapsedTime");
            break;
        }
        if (kernel_ids) kernel_ids[i] = g_prof.ids[i];
        if (ms) ms[i] = t;
        n = i + 1;
    }
    if (count) *count = n;
    for (hipEvent_t ev : g_prof.ev) hipEventDestroy(ev);
    g_prof.ev.clear();
    g_prof.ids.clear();
    g_prof.on = false;
    g_prof.used = 0;
    return st;
}

const char* la_kernel_name(int32_t id)
{
    switch (id) {
    case LA_KERNEL_FWD_LOCAL: return "segment state pass";
    case LA_KERNEL_FWD_CAUSAL: return "causal output pass";
    case LA_KERNEL_FWD_QUERY: return "non-causal output pass";
    case LA_KERNEL_SCAN: return "la_scan_kernel";
    case LA_KERNEL_DECODE: return "la_decode_kernel";
    case LA_KERNEL_FILL: return "la_fill_zero_kernel";
    case LA_KERNEL_COPY: return "la_copy_kernel";
    case LA_KERNEL_BWD_Q: return "la_bwd_q_kernel";
    case LA_KERNEL_BWD_RLOCAL: return "la_bwd_kv_kernel (adjoint segment)";
    case LA_KERNEL_BWD_KV: return "la_bwd_kv_kernel (dk dv)";
    case LA_KERNEL_BWD_DLAM: return "la_dlam_rows_kernel";
    case LA_KERNEL_VARLEN_ITEMS: return "la_varlen_items_kernel";
    case LA_KERNEL_BWD_NCQ: return "la_bwd_q_kernel (non-causal)";
    case LA_KERNEL_BWD_NCKV: return "la_bwd_kv_kernel (non-causal dk dv)";
    case LA_KERNEL_RF_FEATURES: return "la_rf_features_kernel";
    case LA_KERNEL_RF_VJP: return "la_rf_vjp_kernel";
    }
    return "unknown";
}

la_status la_init_state(float* S, float* z, int64_t B, int64_t H, int32_t F, int32_t d_v, la_stream_t stream)
{
    if (B < 1 || H < 1 || F < 1 || d_v < 1) return fail(LA_ERR_INVALID_ARGUMENT, "B, H, F, d_v must be >= 1");
    if ((S && !aligned16(S)) || (z && !aligned16(z))) return fail(LA_ERR_INVALID_ARGUMENT, "S and z must be 16-byte aligned");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (S) e = launch(LA_KERNEL_FILL, [&] { return launch_fill_zero(S, B * H * (int64_t)F * d_v, st); });
    if (e == hipSuccess && z) e = launch(LA_KERNEL_FILL, [&] { return launch_fill_zero(z, B * H * (int64_t)F, st); });
    if (e != hipSuccess) return hip_fail(e, "la_init_state launch");
    return ok();
}

la_status la_init_state_identity(float* S, float* z, int64_t B, int64_t H, int32_t F, int32_t d_v, float alpha,
                                 la_stream_t stream)
{
    if (B < 1 || H < 1 || F < 1 || d_v < 1) return fail(LA_ERR_INVALID_ARGUMENT, "B, H, F, d_v must be >= 1");
    if ((S && !aligned16(S)) || (z && !aligned16(z))) return fail(LA_ERR_INVALID_ARGUMENT, "S and z must be 16-byte aligned");
    if (!std::isfinite(alpha)) return fail(LA_ERR_INVALID_ARGUMENT, "alpha must be finite");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = launch(LA_KERNEL_FILL, [&] { return launch_fill_identity(S, z, B * H, F, d_v, alpha, st); });
    if (e != hipSuccess) return hip_fail(e, "la_init_state_identity launch");
    return ok();
}

// Features per launch: a map of F > 256 runs as two halves.
int half_features(int F) { return F > 256 ? F / 2 : F; }

// Bytes of the numerators and denominators one half of a split map leaves
// for the other: `rows` rows of d_v + 1 floats.
size_t split_bytes(const la_shape* s, int F, int64_t rows)
{
    return F > 256 ? bytes256((size_t)rows * (s->d_v + 1) * sizeof(float)) : 0;
}

size_t la_workspace_size(const la_shape* shape, const la_phi* phi, int32_t causal)
{
    int F = 0;
    const KernelEntry* e = nullptr;
    const std::string saved = g_last_error;
    const la_status st = check_shape(shape, phi, causal ? 0 : 1, INT64_MAX / 4, &F, &e, causal != 0);
    g_last_error = saved;
    if (st != LA_OK || shape->N == 0) return 0;
    return make_plan(shape, half_features(F), e, causal != 0).ws_bytes +
           split_bytes(shape, F, shape->B * shape->H * shape->N);
}

namespace {

// Causal forward shared by the fixed-length, masked, packed and static-scratch
// entry points.  kpm: key padding mask [B][N] bytes or null.  cu: packed
// sequences (device [B+1] offsets into head rows of N tokens) or null; max_len
// then plans the segments (the longest sequence).  use_scratch: the workspace
// is the library's static device scratch (workspace arguments ignored); the
// segments are capped so that their states fit it.
la_status forward_causal(const void* q, const void* k, const void* v, void* y, const la_shape* shape,
                         const la_phi* phi, const float* lambda_h, float eps, const uint8_t* kpm,
                         const int32_t* cu, int64_t max_len, const float* S_in, const float* z_in, float* S_out,
                         float* z_out, void* workspace, size_t workspace_bytes, la_stream_t stream,
                         bool use_scratch = false)
{
    int F = 0;
    const KernelEntry* ent = nullptr;
    la_status st = check_shape(shape, phi, 0, INT64_MAX / 4, &F, &ent, true);
    if (st != LA_OK) return st;
    // a map of F = 512 runs as two halves of Fh features; the first leaves its
    // numerators and denominators, the second adds them in
    const int Fh = half_features(F), nhalf = F / Fh;
    if ((S_in == nullptr) != (z_in == nullptr)) return fail(LA_ERR_INVALID_ARGUMENT, "S_in and z_in must be given together");
    if ((S_out == nullptr) != (z_out == nullptr)) return fail(LA_ERR_INVALID_ARGUMENT, "S_out and z_out must be given together");
    if ((S_in && (!aligned16(S_in) || !aligned16(z_in))) || (S_out && (!aligned16(S_out) || !aligned16(z_out))))
        return fail(LA_ERR_INVALID_ARGUMENT, "state buffers must be 16-byte aligned");
    if ((st = check_eps(eps)) != LA_OK) return st;
    LamTable lam;
    if ((st = make_lam(lambda_h, shape->H, &lam)) != LA_OK) return st;
    const int64_t BH = shape->B * shape->H;
    if (BH > 65535) return fail(LA_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)BH);
    hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
    const int64_t nS = BH * F * (int64_t)shape->d_v, nz = BH * F;

    if (shape->N == 0) {
        hipError_t e = hipSuccess;
        if (S_out) {
            if (S_in) {
                e = launch(LA_KERNEL_COPY, [&] { return launch_copy(S_out, S_in, nS, strm); });
                if (e == hipSuccess) e = launch(LA_KERNEL_COPY, [&] { return launch_copy(z_out, z_in, nz, strm); });
            } else {
                e = launch(LA_KERNEL_FILL, [&] { return launch_fill_zero(S_out, nS, strm); });
                if (e == hipSuccess) e = launch(LA_KERNEL_FILL, [&] { return launch_fill_zero(z_out, nz, strm); });
            }
        }
        if (e != hipSuccess) return hip_fail(e, "la_forward_causal (N=0)");
        return ok();
    }
    int vP = 0;
    int64_t vcps = 1, vG = 0;
    if (cu) {
        // packed rows: q, k, v, y hold H rows of N tokens
        const size_t rows = (size_t)shape->H * shape->N;
        if ((st = check_io_rows(q, k, v, y, shape, rows, rows)) != LA_OK) return st;
        varlen_segments(shape->N, shape->B, shape->H, max_len, ent->C, &vP, &vcps);
        vG = varlen_items_bound(shape->N, shape->B, ent->C, vcps, vP);
        if (vG > 65535) return fail(LA_ERR_UNSUPPORTED, "%lld work items per head exceed 65535", (long long)vG);
    } else {
        if ((st = check_io(q, k, v, y, shape)) != LA_OK) return st;
    }
    int64_t max_P = INT64_MAX;
    if (use_scratch) {
        // segment states of P segments: P slots of BH states; a window carry
        // (LA_WINDOWS > 1) one more slot that must fit on its own
        const size_t slot = (size_t)BH * ((size_t)Fh * shape->d_v + Fh) * sizeof(float);
        const Plan p1 = make_plan(shape, F, ent, true, 0, 1);
        const size_t carry = p1.W > 1 ? slot : 0;
        if (carry > kScratchBytes)
            return fail(LA_ERR_WORKSPACE, "the window carry needs %zu bytes; the static scratch holds %zu", carry,
                        kScratchBytes);
        max_P = (int64_t)((kScratchBytes - carry) / slot);
        if (max_P < 1) max_P = 1;
    }
    Plan plan = make_plan(shape, Fh, ent, true, vP, max_P);
    const size_t seg_bytes = plan.ws_bytes;
    const size_t item_bytes = cu ? bytes256((size_t)vG * sizeof(int32_t)) : 0;
    const int64_t rows = cu ? shape->H * shape->N : BH * shape->N;  // rows of y
    plan.ws_bytes = seg_bytes + item_bytes + split_bytes(shape, F, rows);
    if (use_scratch) {
        if (plan.ws_bytes > kScratchBytes)
            return fail(LA_ERR_WORKSPACE, "the plan needs %zu bytes; the static scratch holds %zu", plan.ws_bytes,
                        kScratchBytes);
        workspace = nullptr;
        workspace_bytes = kScratchBytes;
        if (plan.ws_bytes > 0) {
            const hipError_t se = scratch_ptr(&workspace);
            if (se != hipSuccess) return hip_fail(se, "static scratch address");
        }
    }
    if ((st = check_ws(plan, workspace, workspace_bytes)) != LA_OK) return st;
    int32_t* items = cu ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + seg_bytes) : nullptr;
    float* part_num = nhalf > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + seg_bytes + item_bytes)
                                : nullptr;

    float* ws = static_cast<float*>(workspace);
    float* segs = ws;                                                     // [P][BH][SZ]
    float* carry = ws ? ws + (plan.Pmax > 1 ? (size_t)plan.Pmax * BH * plan.SZ : 0) : nullptr;  // [BH][SZ]
    const int64_t NC = (shape->N + plan.C - 1) / plan.C;

    FwdArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.y = y;
    a.N = shape->N;
    a.BH = (int32_t)BH;
    a.H = (int32_t)shape->H;
    a.out_f32 = shape->out_dtype == LA_F32 && shape->in_dtype != LA_F32;
    a.eps = eps;
    a.qk_scale = is_rf(phi->kind) ? phi->qk_scale : 1.0f;
    a.rf_sign = rf_sign(phi->kind);
    a.rf_scale = is_rf(phi->kind) ? 1.f / std::sqrt((float)phi->m) : 0.f;
    a.part_num = part_num;
    a.part_den = part_num ? part_num + rows * shape->d_v : nullptr;
    a.kpm = kpm;
    a.kpm_stride = shape->N;
    a.cu_seqlens = cu;
    a.lam = lam;

    for (int half = 0; half < nhalf; ++half) {
    // this half's rows of omega and of the caller's states
    a.omega = phi->omega ? phi->omega + (size_t)half * (Fh / 2) * shape->d_k : nullptr;
    a.part_mode = nhalf > 1 ? 1 + half : 0;
    // the caller's rows of a half: its cos rows at (Fh/2) half, its sin rows
    // F/2 further (a gap of Fh/2 rows after the half's first Fh/2)
    const size_t sh = (size_t)half * (Fh / 2) * shape->d_v, zh = (size_t)half * (Fh / 2);
    const int32_t gap = nhalf > 1 ? Fh / 2 : 0;
    const float* S_in_h = S_in ? S_in + sh : nullptr;
    const float* z_in_h = z_in ? z_in + zh : nullptr;
    float* S_out_h = S_out ? S_out + sh : nullptr;
    float* z_out_h = z_out ? z_out + zh : nullptr;
    for (int w = 0; w < plan.W; ++w) {
        const int64_t c0 = (int64_t)w * NC / plan.W, c1 = (int64_t)(w + 1) * NC / plan.W;
        const int64_t n0 = c0 * plan.C, n_len = std::min(c1 * plan.C, shape->N) - n0;
        int P = 1;
        int64_t cps = 1;
        if (cu) {
            // one segment length for every packed sequence (n0, n_len unused)
            P = vP;
            cps = vcps;
            a.G = (int32_t)vG;
            a.items = items;
            hipError_t ie = launch(LA_KERNEL_VARLEN_ITEMS, [&] {
                return launch_varlen_items(cu, (int)shape->B, shape->N, plan.C, cps, P, (int)vG, items, strm);
            });
            if (ie != hipSuccess) return hip_fail(ie, "packed sequence items launch");
        } else {
            cut_segments(c1 - c0, BH, &P, &cps, max_P, causal_target_workgroups(ent, Fh));
        }
        // state entering and leaving this window
        const float* Si = nullptr;
        const float* zi = nullptr;
        int64_t si_stride = 0, zi_stride = 0;
        int32_t si_gap = 0, so_gap = 0;
        if (w == 0) {
            Si = S_in_h; zi = z_in_h; si_stride = (int64_t)F * shape->d_v; zi_stride = F; si_gap = gap;
        } else {
            Si = carry; zi = carry + (int64_t)Fh * shape->d_v; si_stride = plan.SZ; zi_stride = plan.SZ;
        }
        float* So = nullptr;
        float* zo = nullptr;
        int64_t so_stride = 0, zo_stride = 0;
        if (w == plan.W - 1) {
            So = S_out_h; zo = z_out_h; so_stride = (int64_t)F * shape->d_v; zo_stride = F; so_gap = gap;
        } else {
            So = carry; zo = carry + (int64_t)Fh * shape->d_v; so_stride = plan.SZ; zo_stride = plan.SZ;
        }
        a.n0 = n0;
        a.n_len = n_len;
        a.P = P;
        a.cps = cps;
        a.chunk = plan.C;
        hipError_t e;
        if (P > 1) {
            // pass 1: segment-local states
            FwdArgs l = a;
            l.S_dst = segs;
            l.z_dst = segs + (int64_t)Fh * shape->d_v;
            l.dst_stride = plan.SZ;
            l.dst_zstride = plan.SZ;
            // with no state leaving this window, no segment reads the local
            // state of a row's last segment
            l.skip_last = So == nullptr;
            if ((e = launch(LA_KERNEL_FWD_LOCAL, [&] { return ent->fwd(l, MODE_LOCAL, strm); })) != hipSuccess)
                return hip_fail(e, "segment state launch");
            // pass 2: decayed exclusive scan over segments
            ScanArgs sa;
            std::memset(&sa, 0, sizeof(sa));
            sa.ws = segs;
            sa.P = P;
            sa.BH = (int32_t)BH;
            sa.H = (int32_t)shape->H;
            sa.F = Fh;
            sa.DV = shape->d_v;
            sa.n_len = n_len;
            sa.seg_len = cps * plan.C;
            sa.causal = 1;
            sa.cu_seqlens = cu;
            sa.N = shape->N;
            sa.S_init = Si; sa.z_init = zi; sa.init_stride = si_stride; sa.init_zstride = zi_stride;
            sa.S_fin = So; sa.z_fin = zo; sa.fin_stride = so_stride; sa.fin_zstride = zo_stride;
            sa.init_gap = si_gap;
            sa.fin_gap = so_gap;
            sa.skip_last = l.skip_last;
            sa.lam = lam;
            if ((e = launch(LA_KERNEL_SCAN, [&] { return launch_scan(sa, strm); })) != hipSuccess)
                return hip_fail(e, "segment scan launch");
            // pass 3: outputs from the carried-in state of each segment
            FwdArgs c = a;
            c.S_src = segs;
            c.z_src = segs + (int64_t)Fh * shape->d_v;
            c.src_stride = plan.SZ;
            c.src_zstride = plan.SZ;
            c.src_seg_stride = BH * plan.SZ;
            if ((e = launch(LA_KERNEL_FWD_CAUSAL, [&] { return ent->fwd(c, MODE_CAUSAL, strm); })) != hipSuccess)
                return hip_fail(e, "causal output launch");
        } else {
            FwdArgs c = a;
            c.S_src = Si; c.z_src = zi; c.src_stride = si_stride; c.src_zstride = zi_stride;
            c.src_seg_stride = 0;
            c.src_gap = si_gap;
            c.S_dst = So; c.z_dst = zo; c.dst_stride = so_stride; c.dst_zstride = zo_stride;
            c.dst_gap = so_gap;
            if ((e = launch(LA_KERNEL_FWD_CAUSAL, [&] { return ent->fwd(c, MODE_CAUSAL, strm); })) != hipSuccess)
                return hip_fail(e, "causal launch");
        }
    }
    }
    return ok();
}

}  // namespace

la_status la_forward_causal(const void* q, const void* k, const void* v, void* y, const la_shape* shape,
                            const la_phi* phi, const float* lambda_h, float eps, const float* S_in,
                            const float* z_in, float* S_out, float* z_out, void* workspace, size_t workspace_bytes,
                            la_stream_t stream)
{
    return forward_causal(q, k, v, y, shape, phi, lambda_h, eps, nullptr, nullptr, 0, S_in, z_in, S_out, z_out,
                          workspace, workspace_bytes, stream);
}

la_status la_forward_causal_noalloc(const void* q, const void* k, const void* v, void* y, const la_shape* shape,
                                    const la_phi* phi, const float* lambda_h, float eps, const float* S_in,
                                    const float* z_in, float* S_out, float* z_out, la_stream_t stream)
{
    return forward_causal(q, k, v, y, shape, phi, lambda_h, eps, nullptr, nullptr, 0, S_in, z_in, S_out, z_out,
                          nullptr, 0, stream, true);
}

la_status la_forward_causal_masked(const void* q, const void* k, const void* v, void* y, const la_shape* shape,
                                   const la_phi* phi, const float* lambda_h, float eps,
                                   const uint8_t* key_padding_mask, const float* S_in, const float* z_in,
                                   float* S_out, float* z_out, void* workspace, size_t workspace_bytes,
                                   la_stream_t stream)
{
    if (!key_padding_mask) return fail(LA_ERR_INVALID_ARGUMENT, "key_padding_mask is NULL");
    return forward_causal(q, k, v, y, shape, phi, lambda_h, eps, key_padding_mask, nullptr, 0, S_in, z_in, S_out,
                          z_out, workspace, workspace_bytes, stream);
}

size_t la_workspace_size_varlen(const la_shape* shape, int64_t max_seqlen, const la_phi* phi)
{
    int F = 0;
    const KernelEntry* e = nullptr;
    const std::string saved = g_last_error;
    const la_status st = check_shape(shape, phi, 0, INT64_MAX / 4, &F, &e, true);
    g_last_error = saved;
    if (st != LA_OK || shape->N == 0 || max_seqlen < 0 || max_seqlen > shape->N) return 0;
    int P = 1;
    int64_t cps = 1;
    varlen_segments(shape->N, shape->B, shape->H, max_seqlen, e->C, &P, &cps);
    const int64_t G = varlen_items_bound(shape->N, shape->B, e->C, cps, P);
    return make_plan(shape, half_features(F), e, true, P).ws_bytes + bytes256((size_t)G * sizeof(int32_t)) +
           split_bytes(shape, F, shape->H * shape->N);
}

la_status la_forward_causal_varlen(const void* q, const void* k, const void* v, void* y,
                                   const int32_t* cu_seqlens, int64_t max_seqlen, const la_shape* shape,
                                   const la_phi* phi, const float* lambda_h, float eps, const float* S_in,
                                   const float* z_in, float* S_out, float* z_out, void* workspace,
                                   size_t workspace_bytes, la_stream_t stream)
{
    if (!cu_seqlens) return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
    if ((uintptr_t)cu_seqlens % 4) return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
    if (shape && (max_seqlen < 0 || max_seqlen > shape->N))
        return fail(LA_ERR_INVALID_ARGUMENT, "max_seqlen=%lld outside [0, N=%lld]", (long long)max_seqlen,
                    (long long)shape->N);
    return forward_causal(q, k, v, y, shape, phi, lambda_h, eps, nullptr, cu_seqlens, max_seqlen, S_in, z_in, S_out,
                          z_out, workspace, workspace_bytes, stream);
}

la_status la_forward_noncausal(const void* q, const void* k, const void* v, void* y, const la_shape* shape,
                               const la_phi* phi, float eps, void* workspace, size_t workspace_bytes, la_stream_t stream)
{
    int F = 0;
    const KernelEntry* ent = nullptr;
    la_status st = check_shape(shape, phi, 1, INT64_MAX / 4, &F, &ent);
    if (st != LA_OK) return st;
    if ((st = check_eps(eps)) != LA_OK) return st;
    const int64_t BH = shape->B * shape->H;
    if (BH > 65535) return fail(LA_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)BH);
    if ((st = check_io(q, k, v, y, shape)) != LA_OK) return st;
    const Plan plan = make_plan(shape, F, ent, false);
    if ((st = check_ws(plan, workspace, workspace_bytes)) != LA_OK) return st;
    hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
    float* ws = static_cast<float*>(workspace);

    FwdArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.y = y;
    a.N = shape->N;
    a.n0 = 0;
    a.n_len = shape->N;
    a.BH = (int32_t)BH;
    a.H = (int32_t)shape->H;
    // the state sums cut as the causal segment-state pass is (one round of
    // its workgroups: at d_k = d_v = 128, 8 segments per row measured 0.118
    // ms against 0.119-0.124 at 16); the query pass reads only the summed
    // state, so it is cut on its own (there 16 segments: 0.118 ms against
    // 0.137 at 8)
    const int64_t NC = (shape->N + plan.C - 1) / plan.C;
    int P = 1;
    int64_t cps = 1;
    cut_segments(NC, BH, &P, &cps, INT64_MAX, causal_target_workgroups(ent, F));
    int Pq = 1;
    int64_t cpsq = 1;
    cut_segments(NC, BH, &Pq, &cpsq);
    a.P = P;
    a.cps = cps;
    a.chunk = plan.C;
    a.out_f32 = shape->out_dtype == LA_F32 && shape->in_dtype != LA_F32;
    a.eps = eps;
    a.qk_scale = is_rf(phi->kind) ? phi->qk_scale : 1.0f;
    a.rf_sign = rf_sign(phi->kind);
    a.rf_scale = is_rf(phi->kind) ? 1.f / std::sqrt((float)phi->m) : 0.f;
    a.omega = phi->omega;
    make_lam(nullptr, shape->H, &a.lam);  // no decay in the non-causal form

    hipError_t e;
    FwdArgs l = a;
    l.S_dst = ws;
    l.z_dst = ws + (int64_t)F * shape->d_v;
    l.dst_stride = plan.SZ;
    l.dst_zstride = plan.SZ;
    if ((e = launch(LA_KERNEL_FWD_LOCAL, [&] { return ent->fwd(l, MODE_LOCAL, strm); })) != hipSuccess)
        return hip_fail(e, "state sum launch");
    if (P > 1) {
        ScanArgs sa;
        std::memset(&sa, 0, sizeof(sa));
        sa.ws = ws;
        sa.P = P;
        sa.BH = (int32_t)BH;
        sa.H = (int32_t)shape->H;
        sa.F = F;
        sa.DV = shape->d_v;
        sa.n_len = shape->N;
        sa.seg_len = cps * plan.C;
        sa.causal = 0;
        if ((e = launch(LA_KERNEL_SCAN, [&] { return launch_scan(sa, strm); })) != hipSuccess)
            return hip_fail(e, "state reduction launch");
    }
    FwdArgs qa = a;
    qa.P = Pq;
    qa.cps = cpsq;
    qa.S_src = ws;
    qa.z_src = ws + (int64_t)F * shape->d_v;
    qa.src_stride = plan.SZ;
    qa.src_zstride = plan.SZ;
    qa.src_seg_stride = 0;
    if ((e = launch(LA_KERNEL_FWD_QUERY, [&] { return ent->fwd(qa, MODE_QUERY, strm); })) != hipSuccess)
        return hip_fail(e, "query launch");
    return ok();
}

size_t la_workspace_size_cross(const la_shape* shape, int64_t n_kv, const la_phi* phi)
{
    int F = 0;
    const KernelEntry* e = nullptr;
    const std::string saved = g_last_error;
    const la_status st = check_shape(shape, phi, 1, INT64_MAX / 4, &F, &e);
    g_last_error = saved;
    if (st != LA_OK || n_kv < 1 || n_kv > INT64_MAX / 4) return 0;
    la_shape ks = *shape;
    ks.N = n_kv;
    return make_plan(&ks, F, e, false).ws_bytes;
}

la_status la_forward_cross(const void* q, const void* k, const void* v, void* y, const la_shape* shape,
                           int64_t n_kv, const uint8_t* key_padding_mask, const la_phi* phi, float eps,
                           void* workspace, size_t workspace_bytes, la_stream_t stream)
{
    int F = 0;
    const KernelEntry* ent = nullptr;
    la_status st = check_shape(shape, phi, 1, INT64_MAX / 4, &F, &ent);
    if (st != LA_OK) return st;
    if (n_kv < 1 || n_kv > INT64_MAX / 4) return fail(LA_ERR_INVALID_ARGUMENT, "n_kv=%lld must be >= 1", (long long)n_kv);
    if ((st = check_eps(eps)) != LA_OK) return st;
    const int64_t BH = shape->B * shape->H;
    if (BH > 65535) return fail(LA_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)BH);
    if ((st = check_io_rows(q, k, v, y, shape, (size_t)BH * shape->N, (size_t)BH * n_kv)) != LA_OK) return st;
    la_shape ks = *shape;
    ks.N = n_kv;
    const Plan plan = make_plan(&ks, F, ent, false);
    if ((st = check_ws(plan, workspace, workspace_bytes)) != LA_OK) return st;
    hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
    float* ws = static_cast<float*>(workspace);

    FwdArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.y = y;
    a.BH = (int32_t)BH;
    a.H = (int32_t)shape->H;
    a.out_f32 = shape->out_dtype == LA_F32 && shape->in_dtype != LA_F32;
    a.eps = eps;
    a.qk_scale = is_rf(phi->kind) ? phi->qk_scale : 1.0f;
    a.rf_sign = rf_sign(phi->kind);
    a.rf_scale = is_rf(phi->kind) ? 1.f / std::sqrt((float)phi->m) : 0.f;
    a.omega = phi->omega;
    make_lam(nullptr, shape->H, &a.lam);  // no decay in the non-causal form
    a.chunk = plan.C;

    // pass 1 over the n_kv keys: segment sums of phi(k) [v, 1]^T
    int Pk = 1;
    int64_t cpsk = 1;
    cut_segments((n_kv + plan.C - 1) / plan.C, BH, &Pk, &cpsk);
    FwdArgs l = a;
    l.N = n_kv;
    l.n_len = n_kv;
    l.P = Pk;
    l.cps = cpsk;
    l.kpm = key_padding_mask;
    l.kpm_stride = n_kv;
    l.S_dst = ws;
    l.z_dst = ws + (int64_t)F * shape->d_v;
    l.dst_stride = plan.SZ;
    l.dst_zstride = plan.SZ;
    hipError_t e;
    if ((e = launch(LA_KERNEL_FWD_LOCAL, [&] { return ent->fwd(l, MODE_LOCAL, strm); })) != hipSuccess)
        return hip_fail(e, "cross state sum launch");
    if (Pk > 1) {
        ScanArgs sa;
        std::memset(&sa, 0, sizeof(sa));
        sa.ws = ws;
        sa.P = Pk;
        sa.BH = (int32_t)BH;
        sa.H = (int32_t)shape->H;
        sa.F = F;
        sa.DV = shape->d_v;
        sa.n_len = n_kv;
        sa.seg_len = cpsk * plan.C;
        sa.causal = 0;
        if ((e = launch(LA_KERNEL_SCAN, [&] { return launch_scan(sa, strm); })) != hipSuccess)
            return hip_fail(e, "cross state reduction launch");
    }
    // pass 2 over the N queries
    int Pq = 1;
    int64_t cpsq = 1;
    cut_segments((shape->N + plan.C - 1) / plan.C, BH, &Pq, &cpsq);
    FwdArgs qa = a;
    qa.N = shape->N;
    qa.n_len = shape->N;
    qa.P = Pq;
    qa.cps = cpsq;
    qa.S_src = ws;
    qa.z_src = ws + (int64_t)F * shape->d_v;
    qa.src_stride = plan.SZ;
    qa.src_zstride = plan.SZ;
    qa.src_seg_stride = 0;
    if ((e = launch(LA_KERNEL_FWD_QUERY, [&] { return ent->fwd(qa, MODE_QUERY, strm); })) != hipSuccess)
        return hip_fail(e, "cross query launch");
    return ok();
}

namespace {

const BwdEntry* find_bwd(int in_dtype, int phi, int dk, int F, int dv)
{
    const BwdEntry* tabs[] = {kBwdEntriesBf16, kBwdEntriesF32, kBwdEntriesIdentBf16, kBwdEntriesIdentF32};
    const int counts[] = {kNumBwdEntriesBf16, kNumBwdEntriesF32, kNumBwdEntriesIdentBf16, kNumBwdEntriesIdentF32};
    for (int t = 0; t < 4; ++t)
        for (int i = 0; i < counts[t]; ++i) {
            const BwdEntry& e = tabs[t][i];
            if (e.in_dtype == in_dtype && e.phi == phi && e.dk == dk && e.F == F && e.dv == dv) return &e;
        }
    return nullptr;
}

// Shape checks of the backward beyond the forward's; sets F, the forward entry
// that runs the segment-state pass and the entry of the backward sweeps.
// Random features: both entries are those of the identity map at d_k = F,
// run on phi(q), phi(k) computed beforehand.
la_status check_backward(const la_shape* shape, const la_phi* phi, int* F, const KernelEntry** ent,
                         const BwdEntry** bent)
{
    la_status st = check_shape(shape, phi, 0, INT64_MAX / 4, F, ent);
    if (st != LA_OK) return st;
    const bool rf = is_rf(phi->kind);
    if (shape->out_dtype != shape->in_dtype)
        return fail(LA_ERR_UNSUPPORTED, "the backward takes y and dy in the input type (out_dtype == in_dtype)");
    if (rf) {
        *ent = find_entry(shape->in_dtype, kPhiIdentity, *F, *F, shape->d_v);
        *bent = find_bwd(shape->in_dtype, kPhiIdentity, *F, *F, shape->d_v);
        if (!*ent || !*bent)
            return fail(LA_ERR_UNSUPPORTED, "no random-feature backward for dtype=%d F=%d d_v=%d", shape->in_dtype, *F,
                        shape->d_v);
        return LA_OK;
    }
    *bent = find_bwd(shape->in_dtype, phi->kind, shape->d_k, *F, shape->d_v);
    if (!*bent) return fail(LA_ERR_UNSUPPORTED, "no backward kernel for this shape");
    return LA_OK;
}

// q, k, v, y, dy and dq, dk, dv: non-NULL and 16-byte aligned; the outputs
// overlap no input and no other output.  q, y, dy, dq have rows_q rows,
// k, v, dk, dv rows_k.
la_status check_bwd_io(const void* q, const void* k, const void* v, const void* y, const void* dy, void* dq,
                       void* dk, void* dv, const la_shape* s, size_t rows_q, size_t rows_k)
{
    const void* ins[] = {q, k, v, y, dy};
    void* outs[] = {dq, dk, dv};
    for (const void* p : ins)
        if (!p || !aligned16(p)) return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v, y, dy must be non-NULL and 16-byte aligned");
    for (const void* p : outs)
        if (!p || !aligned16(p)) return fail(LA_ERR_INVALID_ARGUMENT, "dq, dk, dv must be non-NULL and 16-byte aligned");
    const size_t es = elem_size(s->in_dtype);
    const size_t nq = rows_q * s->d_k * es, nyq = rows_q * s->d_v * es;
    const size_t nk = rows_k * s->d_k * es, nv = rows_k * s->d_v * es;
    const size_t in_sz[] = {nq, nk, nv, nyq, nyq};
    const size_t out_sz[] = {nq, nk, nv};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 5; ++i)
            if (overlaps(outs[o], out_sz[o], ins[i], in_sz[i]))
                return fail(LA_ERR_INVALID_ARGUMENT, "dq, dk, dv must not alias q, k, v, y or dy");
        for (int o2 = 0; o2 < o; ++o2)
            if (overlaps(outs[o], out_sz[o], outs[o2], out_sz[o2]))
                return fail(LA_ERR_INVALID_ARGUMENT, "dq, dk, dv must not overlap");
    }
    return LA_OK;
}

struct BwdPlan {
    int P;
    int64_t cps;
    int64_t SZ;
    size_t tok_floats, seg_floats, dlam_floats, bytes;
};

size_t round256(size_t floats) { return ((floats * sizeof(float) + 255) & ~size_t(255)) / sizeof(float); }
size_t round256b(size_t bytes) { return (bytes + 255) & ~size_t(255); }

// Random-feature backward buffers after the plan's: phi(q) [rows_q, F] and
// phi(k) [rows_k, F] in the input type, d phi(q) and d phi(k) in fp32.
struct RfBufs {
    size_t fq, fk, dfq, dfk, bytes;
};
RfBufs rf_bufs(const la_shape* s, int F, size_t rows_q, size_t rows_k)
{
    RfBufs b;
    const size_t es = elem_size(s->in_dtype);
    b.fq = round256b(rows_q * F * es);
    b.fk = round256b(rows_k * F * es);
    b.dfq = round256b(rows_q * F * es);
    b.dfk = round256b(rows_k * F * es);
    b.bytes = b.fq + b.fk + b.dfq + b.dfk;
    return b;
}

// The feature-map end of the random-feature backward: phi(q), phi(k) into
// the buffers at `base` (laid out as rf_bufs), the kernels' pointers then
// redirected to them; rf_finish maps d phi back to dq, dk through omega.
struct RfRoute {
    RfGradArgs g;
    void* fq;
    void* fk;
    void* dfq;
    void* dfk;
};
hipError_t rf_begin(const la_phi* phi, const la_shape* s, int64_t rows_q, int64_t rows_k, const RfBufs& rb,
                    char* base, const void* q, const void* k, RfRoute* r, hipStream_t strm)
{
    std::memset(&r->g, 0, sizeof(r->g));
    r->fq = base;
    r->fk = base + rb.fq;
    r->dfq = base + rb.fq + rb.fk;
    r->dfk = base + rb.fq + rb.fk + rb.dfq;
    r->g.omega = phi->omega;
    r->g.dk = s->d_k;
    r->g.m = phi->m;
    r->g.scale = phi->qk_scale;
    r->g.sign = rf_sign(phi->kind);
    r->g.in_f32 = s->in_dtype == LA_F32;
    r->g.H = (int32_t)s->H;
    RfGradArgs a = r->g;
    a.x = q;
    a.out = r->fq;
    a.rows = rows_q;
    hipError_t e = launch(LA_KERNEL_RF_FEATURES, [&] { return launch_rf_grad(a, false, strm); });
    if (e != hipSuccess) return e;
    a.x = k;
    a.out = r->fk;
    a.rows = rows_k;
    return launch(LA_KERNEL_RF_FEATURES, [&] { return launch_rf_grad(a, false, strm); });
}
hipError_t rf_finish(const RfRoute& r, int64_t rows_q, int64_t rows_k, int64_t n_k, const uint8_t* kpm,
                     const void* q, const void* k, void* dq, void* dk, hipStream_t strm)
{
    RfGradArgs a = r.g;
    a.x = q;
    a.dphi = r.dfq;
    a.out = dq;
    a.rows = rows_q;
    hipError_t e = launch(LA_KERNEL_RF_VJP, [&] { return launch_rf_grad(a, true, strm); });
    if (e != hipSuccess) return e;
    // keys: rows (b*H + h)*n_k + n, padded keys get dk = 0
    a.x = k;
    a.dphi = r.dfk;
    a.out = dk;
    a.rows = rows_k;
    a.kpm = kpm;
    a.N = n_k;
    a.kpm_stride = n_k;
    return launch(LA_KERNEL_RF_VJP, [&] { return launch_rf_grad(a, true, strm); });
}

BwdPlan bwd_plan(const la_shape* s, int F, int C)
{
    BwdPlan p;
    const int64_t BH = s->B * s->H;
    const int64_t NC = (s->N + C - 1) / C;
    p.P = 1;
    p.cps = 1;
    if (NC > 0) cut_segments(NC, BH, &p.P, &p.cps);
    p.SZ = (int64_t)F * s->d_v + F;
    p.tok_floats = (size_t)BH * s->N * 2;
    p.seg_floats = p.P > 1 ? (size_t)p.P * BH * p.SZ : 0;
    // lambda gradient: the segments' dT, their partials, one sum per row
    p.dlam_floats = round256((size_t)p.P * BH * p.SZ) + round256((size_t)p.P * BH) +
                    round256((size_t)BH * dlam_blocks(F, s->d_v));
    p.bytes = s->N > 0 ? (round256(p.tok_floats) + round256(p.seg_floats) + p.dlam_floats) * sizeof(float) : 0;
    return p;
}

}  // namespace

size_t la_workspace_size_backward(const la_shape* shape, const la_phi* phi)
{
    int F = 0;
    const KernelEntry* e = nullptr;
    const BwdEntry* be = nullptr;
    const std::string saved = g_last_error;
    const la_status st = check_backward(shape, phi, &F, &e, &be);
    g_last_error = saved;
    if (st != LA_OK) return 0;
    const size_t base = bwd_plan(shape, F, be->C).bytes;
    const size_t rows = (size_t)(shape->B * shape->H * shape->N);
    return is_rf(phi->kind) && shape->N > 0 ? base + rf_bufs(shape, F, rows, rows).bytes : base;
}

la_status la_backward_causal(const void* q, const void* k, const void* v, const void* y, const void* dy,
                             void* dq, void* dk, void* dv, const la_shape* shape, const la_phi* phi,
                             const float* lambda_h, float eps, const uint8_t* key_padding_mask,
                             const float* S_in, const float* z_in, const float* dS_out, const float* dz_out,
                             float* dS_in, float* dz_in, float* dlambda, void* workspace, size_t workspace_bytes,
                             la_stream_t stream)
{
    int F = 0;
    const KernelEntry* ent = nullptr;
    const BwdEntry* bent = nullptr;
    la_status st = check_backward(shape, phi, &F, &ent, &bent);
    if (st != LA_OK) return st;
    const bool rf = is_rf(phi->kind);
    if ((S_in == nullptr) != (z_in == nullptr)) return fail(LA_ERR_INVALID_ARGUMENT, "S_in and z_in must be given together");
    if ((dS_out == nullptr) != (dz_out == nullptr))
        return fail(LA_ERR_INVALID_ARGUMENT, "dS_out and dz_out must be given together");
    if ((dS_in == nullptr) != (dz_in == nullptr))
        return fail(LA_ERR_INVALID_ARGUMENT, "dS_in and dz_in must be given together");
    const float* st_ptrs[] = {S_in, z_in, dS_out, dz_out, dS_in, dz_in};
    for (const float* p : st_ptrs)
        if (p && !aligned16(p)) return fail(LA_ERR_INVALID_ARGUMENT, "state buffers must be 16-byte aligned");
    if (dlambda && !bent->dlam)
        return fail(LA_ERR_UNSUPPORTED, "the lambda gradient is not available for this type and head size");
    if (dlambda && ((uintptr_t)dlambda % 4)) return fail(LA_ERR_INVALID_ARGUMENT, "dlambda must be 4-byte aligned");
    if ((st = check_eps(eps)) != LA_OK) return st;
    LamTable lam;
    if ((st = make_lam(lambda_h, shape->H, &lam)) != LA_OK) return st;
    const int64_t BH = shape->B * shape->H;
    if (BH > 65535) return fail(LA_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)BH);
    hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
    const int64_t nS = BH * F * (int64_t)shape->d_v, nz = BH * F;

    if (shape->N == 0) {
        // no tokens: the initial state's gradient is the final state's, and
        // nothing depends on lambda
        hipError_t e = hipSuccess;
        if (dlambda) e = launch(LA_KERNEL_FILL, [&] { return launch_fill_zero(dlambda, shape->H, strm); });
        if (dS_in && e == hipSuccess) {
            if (dS_out) {
                e = launch(LA_KERNEL_COPY, [&] { return launch_copy(dS_in, dS_out, nS, strm); });
                if (e == hipSuccess) e = launch(LA_KERNEL_COPY, [&] { return launch_copy(dz_in, dz_out, nz, strm); });
            } else {
                e = launch(LA_KERNEL_FILL, [&] { return launch_fill_zero(dS_in, nS, strm); });
                if (e == hipSuccess) e = launch(LA_KERNEL_FILL, [&] { return launch_fill_zero(dz_in, nz, strm); });
            }
        }
        if (e != hipSuccess) return hip_fail(e, "la_backward_causal (N=0)");
        return ok();
    }
    const size_t rows = (size_t)BH * shape->N;
    if ((st = check_bwd_io(q, k, v, y, dy, dq, dk, dv, shape, rows, rows)) != LA_OK) return st;
    const BwdPlan plan = bwd_plan(shape, F, bent->C);
    const RfBufs rb = rf_bufs(shape, F, rows, rows);
    const size_t need = plan.bytes + (rf ? rb.bytes : 0);
    if (!workspace) return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (workspace_bytes < need)
        return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, workspace_bytes);
    if (!aligned16(workspace)) return fail(LA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    float* tok = static_cast<float*>(workspace);
    float* segs = tok + round256(plan.tok_floats);
    float* tseg = segs + round256(plan.seg_floats);
    float* dlp = tseg + round256((size_t)plan.P * BH * plan.SZ);
    float* drows = dlp + round256((size_t)plan.P * BH);
    // random features: the sweeps run on phi(q), phi(k) (identity map) and
    // write d phi in fp32; dq and dk follow from it through omega at the end
    const void* q_in = q;
    const void* k_in = k;
    void* dq_out = dq;
    void* dk_out = dk;
    RfRoute rr;
    if (rf) {
        hipError_t e = rf_begin(phi, shape, (int64_t)rows, (int64_t)rows, rb, static_cast<char*>(workspace) + plan.bytes,
                                q, k, &rr, strm);
        if (e != hipSuccess) return hip_fail(e, "backward: random-feature launch");
        q_in = rr.fq;
        k_in = rr.fk;
        dq_out = rr.dfq;
        dk_out = rr.dfk;
    }
    DlamArgs da;
    std::memset(&da, 0, sizeof(da));
    da.tseg = tseg;
    da.dlp = dlp;
    da.dS_out = dS_out;
    da.dz_out = dz_out;
    da.rows = drows;
    da.dlam = dlambda;
    da.P = plan.P;
    da.BH = (int32_t)BH;
    da.H = (int32_t)shape->H;
    da.F = F;
    da.DV = shape->d_v;
    da.n_len = shape->N;
    da.seg_len = plan.cps * bent->C;

    BwdArgs b;
    std::memset(&b, 0, sizeof(b));
    b.q = q_in;
    b.k = k_in;
    b.v = v;
    b.y = y;
    b.gy = dy;
    b.dq = dq_out;
    b.dk = dk_out;
    b.dv = dv;
    b.tok = tok;
    b.N = shape->N;
    b.BH = (int32_t)BH;
    b.H = (int32_t)shape->H;
    b.P = plan.P;
    b.cps = plan.cps;
    b.eps = eps;
    b.kpm = key_padding_mask;
    b.lam = lam;
    da.lam = lam;
    const int64_t FD = (int64_t)F * shape->d_v;
    hipError_t e;
    if (plan.P > 1) {
        // forward state at each segment's start: segment sums, then the scan
        FwdArgs a;
        std::memset(&a, 0, sizeof(a));
        a.q = q_in;
        a.k = k_in;
        a.v = v;
        a.N = shape->N;
        a.n_len = shape->N;
        a.BH = (int32_t)BH;
        a.H = (int32_t)shape->H;
        a.P = plan.P;
        a.cps = plan.cps;
        a.chunk = bent->C;
        a.eps = eps;
        a.qk_scale = 1.0f;
        a.kpm = key_padding_mask;
        a.kpm_stride = shape->N;
        a.lam = lam;
        a.S_dst = segs;
        a.z_dst = segs + FD;
        a.dst_stride = plan.SZ;
        a.dst_zstride = plan.SZ;
        if ((e = launch(LA_KERNEL_FWD_LOCAL, [&] { return ent->fwd(a, MODE_LOCAL, strm); })) != hipSuccess)
            return hip_fail(e, "backward: segment state launch");
        ScanArgs sa;
        std::memset(&sa, 0, sizeof(sa));
        sa.ws = segs;
        sa.P = plan.P;
        sa.BH = (int32_t)BH;
        sa.H = (int32_t)shape->H;
        sa.F = F;
        sa.DV = shape->d_v;
        sa.n_len = shape->N;
        sa.seg_len = plan.cps * bent->C;
        sa.causal = 1;
        sa.S_init = S_in; sa.z_init = z_in; sa.init_stride = FD; sa.init_zstride = F;
        sa.lam = lam;
        if ((e = launch(LA_KERNEL_SCAN, [&] { return launch_scan(sa, strm); })) != hipSuccess)
            return hip_fail(e, "backward: segment scan launch");
        BwdArgs bq = b;
        bq.S_src = segs; bq.z_src = segs + FD;
        bq.src_stride = plan.SZ; bq.src_zstride = plan.SZ; bq.src_seg_stride = BH * plan.SZ;
        if (dlambda) { bq.tseg = tseg; bq.dlp = dlp; }
        if ((e = launch(LA_KERNEL_BWD_Q, [&] { return bent->bwd(bq, BMODE_Q, strm); })) != hipSuccess)
            return hip_fail(e, "backward: dq launch");
        // adjoint at each segment's end: reverse segment sums, then the reverse scan
        BwdArgs br = b;
        br.S_dst = segs; br.z_dst = segs + FD;
        br.dst_stride = plan.SZ; br.dst_zstride = plan.SZ;
        if ((e = launch(LA_KERNEL_BWD_RLOCAL, [&] { return bent->bwd(br, BMODE_RLOCAL, strm); })) != hipSuccess)
            return hip_fail(e, "backward: adjoint segment launch");
        if (dlambda) {
            // before the reverse scan turns the adjoint segment sums into carries
            da.wloc = segs;
            if ((e = launch(LA_KERNEL_BWD_DLAM, [&] { return launch_dlam(da, strm); })) != hipSuccess)
                return hip_fail(e, "backward: lambda gradient launch");
        }
        ScanArgs ra = sa;
        ra.reverse = 1;
        ra.S_init = dS_out; ra.z_init = dz_out;
        ra.S_fin = dS_in; ra.z_fin = dz_in; ra.fin_stride = FD; ra.fin_zstride = F;
        if ((e = launch(LA_KERNEL_SCAN, [&] { return launch_scan(ra, strm); })) != hipSuccess)
            return hip_fail(e, "backward: adjoint scan launch");
        BwdArgs bk = b;
        bk.S_src = segs; bk.z_src = segs + FD;
        bk.src_stride = plan.SZ; bk.src_zstride = plan.SZ; bk.src_seg_stride = BH * plan.SZ;
        if ((e = launch(LA_KERNEL_BWD_KV, [&] { return bent->bwd(bk, BMODE_KV, strm); })) != hipSuccess)
            return hip_fail(e, "backward: dk dv launch");
    } else {
        BwdArgs bq = b;
        bq.S_src = S_in; bq.z_src = z_in; bq.src_stride = FD; bq.src_zstride = F;
        if (dlambda) { bq.tseg = tseg; bq.dlp = dlp; }
        if ((e = launch(LA_KERNEL_BWD_Q, [&] { return bent->bwd(bq, BMODE_Q, strm); })) != hipSuccess)
            return hip_fail(e, "backward: dq launch");
        if (dlambda && (e = launch(LA_KERNEL_BWD_DLAM, [&] { return launch_dlam(da, strm); })) != hipSuccess)
            return hip_fail(e, "backward: lambda gradient launch");
        BwdArgs bk = b;
        bk.S_src = dS_out; bk.z_src = dz_out; bk.src_stride = FD; bk.src_zstride = F;
        bk.S_dst = dS_in; bk.z_dst = dz_in; bk.dst_stride = FD; bk.dst_zstride = F;
        if ((e = launch(LA_KERNEL_BWD_KV, [&] { return bent->bwd(bk, BMODE_KV, strm); })) != hipSuccess)
            return hip_fail(e, "backward: dk dv launch");
    }
    if (rf) {
        // dq, dk = J_phi^T d phi (padded keys: 0)
        e = rf_finish(rr, (int64_t)rows, (int64_t)rows, shape->N, key_padding_mask, q, k, dq, dk, strm);
        if (e != hipSuccess) return hip_fail(e, "backward: random-feature gradient launch");
    }
    return ok();
}

namespace {

// Segments of the non-causal backward: the keys' state sums (forward chunk
// Cf), the query sweep and the key sweep (backward chunk Cb); the workspace
// holds the state slots [Pk][BH][SZ] and the adjoint slots [Pq][BH][SZ]
// (slot 0 of each ends as the total).
struct CrossBwdPlan {
    int Pk, Pq, Pv;
    int64_t cpsk, cpsq, cpsv, SZ;
    size_t state_floats, adj_floats, bytes;
};

CrossBwdPlan cross_bwd_plan(const la_shape* s, int64_t n_kv, int F, int Cf, int Cb)
{
    CrossBwdPlan p;
    const int64_t BH = s->B * s->H;
    cut_segments((n_kv + Cf - 1) / Cf, BH, &p.Pk, &p.cpsk);
    cut_segments((s->N + Cb - 1) / Cb, BH, &p.Pq, &p.cpsq);
    cut_segments((n_kv + Cb - 1) / Cb, BH, &p.Pv, &p.cpsv);
    p.SZ = (int64_t)F * s->d_v + F;
    p.state_floats = round256((size_t)p.Pk * BH * p.SZ);
    p.adj_floats = round256((size_t)p.Pq * BH * p.SZ);
    p.bytes = (p.state_floats + p.adj_floats) * sizeof(float);
    return p;
}

}  // namespace

size_t la_workspace_size_backward_cross(const la_shape* shape, int64_t n_kv, const la_phi* phi)
{
    int F = 0;
    const KernelEntry* e = nullptr;
    const BwdEntry* be = nullptr;
    const std::string saved = g_last_error;
    const la_status st = check_backward(shape, phi, &F, &e, &be);
    g_last_error = saved;
    if (st != LA_OK || shape->N < 1 || n_kv < 1 || n_kv > INT64_MAX / 4) return 0;
    const size_t base = cross_bwd_plan(shape, n_kv, F, e->C, be->C).bytes;
    const size_t BH = (size_t)(shape->B * shape->H);
    return is_rf(phi->kind) ? base + rf_bufs(shape, F, BH * shape->N, BH * n_kv).bytes : base;
}

la_status la_backward_cross(const void* q, const void* k, const void* v, const void* y, const void* dy,
                            void* dq, void* dk, void* dv, const la_shape* shape, int64_t n_kv,
                            const uint8_t* key_padding_mask, const la_phi* phi, float eps,
                            void* workspace, size_t workspace_bytes, la_stream_t stream)
{
    int F = 0;
    const KernelEntry* ent = nullptr;
    const BwdEntry* bent = nullptr;
    la_status st = check_backward(shape, phi, &F, &ent, &bent);
    if (st != LA_OK) return st;
    const bool rf = is_rf(phi->kind);
    if (shape->N < 1) return fail(LA_ERR_INVALID_ARGUMENT, "N must be >= 1");
    if (n_kv < 1 || n_kv > INT64_MAX / 4) return fail(LA_ERR_INVALID_ARGUMENT, "n_kv=%lld must be >= 1", (long long)n_kv);
    if ((st = check_eps(eps)) != LA_OK) return st;
    const int64_t BH = shape->B * shape->H;
    if (BH > 65535) return fail(LA_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)BH);
    if ((st = check_bwd_io(q, k, v, y, dy, dq, dk, dv, shape, (size_t)BH * shape->N, (size_t)BH * n_kv)) != LA_OK)
        return st;
    const CrossBwdPlan plan = cross_bwd_plan(shape, n_kv, F, ent->C, bent->C);
    const int64_t rows_q = BH * shape->N, rows_k = BH * n_kv;
    const RfBufs rb = rf_bufs(shape, F, (size_t)rows_q, (size_t)rows_k);
    const size_t need = plan.bytes + (rf ? rb.bytes : 0);
    if (!workspace) return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (workspace_bytes < need)
        return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, workspace_bytes);
    if (!aligned16(workspace)) return fail(LA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
    // random features: as the causal backward, the sweeps run on phi(q),
    // phi(k) with the identity map and d phi returns through omega
    const void* q_in = q;
    const void* k_in = k;
    void* dq_out = dq;
    void* dk_out = dk;
    RfRoute rr;
    if (rf) {
        hipError_t e0 = rf_begin(phi, shape, rows_q, rows_k, rb, static_cast<char*>(workspace) + plan.bytes, q, k, &rr,
                                 strm);
        if (e0 != hipSuccess) return hip_fail(e0, "cross backward: random-feature launch");
        q_in = rr.fq;
        k_in = rr.fk;
        dq_out = rr.dfq;
        dk_out = rr.dfk;
    }
    float* sws = static_cast<float*>(workspace);
    float* aws = sws + plan.state_floats;
    const int64_t FD = (int64_t)F * shape->d_v;
    LamTable ones;
    make_lam(nullptr, shape->H, &ones);  // no decay in the non-causal form
    hipError_t e;

    // total state over the kept keys: segment sums, then their sum into slot 0
    FwdArgs l;
    std::memset(&l, 0, sizeof(l));
    l.q = q_in;
    l.k = k_in;
    l.v = v;
    l.N = n_kv;
    l.n_len = n_kv;
    l.BH = (int32_t)BH;
    l.H = (int32_t)shape->H;
    l.P = plan.Pk;
    l.cps = plan.cpsk;
    l.chunk = ent->C;
    l.eps = eps;
    l.qk_scale = 1.0f;
    l.kpm = key_padding_mask;
    l.kpm_stride = n_kv;
    l.lam = ones;
    l.S_dst = sws;
    l.z_dst = sws + FD;
    l.dst_stride = plan.SZ;
    l.dst_zstride = plan.SZ;
    if ((e = launch(LA_KERNEL_FWD_LOCAL, [&] { return ent->fwd(l, MODE_LOCAL, strm); })) != hipSuccess)
        return hip_fail(e, "cross backward: state sum launch");
    ScanArgs sa;
    std::memset(&sa, 0, sizeof(sa));
    sa.BH = (int32_t)BH;
    sa.H = (int32_t)shape->H;
    sa.F = F;
    sa.DV = shape->d_v;
    sa.causal = 0;
    sa.lam = ones;
    if (plan.Pk > 1) {
        sa.ws = sws;
        sa.P = plan.Pk;
        if ((e = launch(LA_KERNEL_SCAN, [&] { return launch_scan(sa, strm); })) != hipSuccess)
            return hip_fail(e, "cross backward: state reduction launch");
    }
    // query sweep: dq, and the segments' adjoint sums
    BwdArgs b;
    std::memset(&b, 0, sizeof(b));
    b.q = q_in;
    b.k = k_in;
    b.v = v;
    b.y = y;
    b.gy = dy;
    b.dq = dq_out;
    b.dk = dk_out;
    b.dv = dv;
    b.BH = (int32_t)BH;
    b.H = (int32_t)shape->H;
    b.eps = eps;
    b.lam = ones;
    BwdArgs bq = b;
    bq.N = shape->N;
    bq.P = plan.Pq;
    bq.cps = plan.cpsq;
    bq.S_src = sws; bq.z_src = sws + FD;
    bq.src_stride = plan.SZ; bq.src_zstride = plan.SZ; bq.src_seg_stride = 0;
    bq.S_dst = aws; bq.z_dst = aws + FD;
    bq.dst_stride = plan.SZ; bq.dst_zstride = plan.SZ;
    if ((e = launch(LA_KERNEL_BWD_NCQ, [&] { return bent->bwd(bq, BMODE_NCQ, strm); })) != hipSuccess)
        return hip_fail(e, "cross backward: dq launch");
    if (plan.Pq > 1) {
        sa.ws = aws;
        sa.P = plan.Pq;
        if ((e = launch(LA_KERNEL_SCAN, [&] { return launch_scan(sa, strm); })) != hipSuccess)
            return hip_fail(e, "cross backward: adjoint reduction launch");
    }
    // key sweep: dk, dv from the total adjoint
    BwdArgs bk = b;
    bk.N = n_kv;
    bk.P = plan.Pv;
    bk.cps = plan.cpsv;
    bk.kpm = key_padding_mask;
    bk.S_src = aws; bk.z_src = aws + FD;
    bk.src_stride = plan.SZ; bk.src_zstride = plan.SZ; bk.src_seg_stride = 0;
    if ((e = launch(LA_KERNEL_BWD_NCKV, [&] { return bent->bwd(bk, BMODE_NCKV, strm); })) != hipSuccess)
        return hip_fail(e, "cross backward: dk dv launch");
    if (rf) {
        e = rf_finish(rr, rows_q, rows_k, n_kv, key_padding_mask, q, k, dq, dk, strm);
        if (e != hipSuccess) return hip_fail(e, "cross backward: random-feature gradient launch");
    }
    return ok();
}

la_status la_decode_step(const void* q, const void* k, const void* v, void* y, float* S, float* z,
                         const la_shape* shape, const la_phi* phi, const float* lambda_h, float eps, la_stream_t stream)
{
    int F = 0;
    const KernelEntry* ent = nullptr;
    la_status st = check_shape(shape, phi, 1, LA_DECODE_MAX_TOKENS, &F, &ent);
    if (st != LA_OK) return st;
    if (!S || !z) return fail(LA_ERR_INVALID_ARGUMENT, "S and z must be non-NULL");
    if (!aligned16(S) || !aligned16(z)) return fail(LA_ERR_INVALID_ARGUMENT, "S and z must be 16-byte aligned");
    if ((st = check_eps(eps)) != LA_OK) return st;
    if ((st = check_io(q, k, v, y, shape)) != LA_OK) return st;
    const int64_t BH = shape->B * shape->H;
    if (BH > 0x7fffffff) return fail(LA_ERR_UNSUPPORTED, "B*H too large");
    // Several tokens per call with an elementwise map on bf16 inputs: the
    // causal forward over the call's tokens, from S back into S, is faster
    // from about ten tokens on (its output kernel does the per-token products
    // on the matrix cores, while the decode kernel's fp32 arithmetic grows
    // with the tokens; measured at B = 256, H = 32: d = 128 ties at 10 tokens
    // and wins from 12, d = 64 wins from 10).  At most 64 tokens are one
    // chunk, one segment per row, so it needs no workspace; its grid takes at
    // most 65535 head-states (more stay on the decode kernel).
    if (shape->in_dtype == LA_BF16 && (phi->kind == LA_PHI_ELU1 || phi->kind == LA_PHI_RELU) &&
        shape->N >= ((int64_t)F * shape->d_v >= 128 * 128 ? 11 : 10) && shape->N <= 64 && BH <= 65535)
        return forward_causal(q, k, v, y, shape, phi, lambda_h, eps, nullptr, nullptr, 0, S, z, S, z, nullptr, 0,
                              stream);
    DecArgs a;
    std::memset(&a, 0, sizeof(a));
    if ((st = make_lam(lambda_h, shape->H, &a.lam)) != LA_OK) return st;
    a.q = q;
    a.k = k;
    a.v = v;
    a.y = y;
    a.S = S;
    a.z = z;
    a.BH = (int32_t)BH;
    a.H = (int32_t)shape->H;
    a.ntok = (int32_t)shape->N;
    a.out_f32 = shape->out_dtype == LA_F32 && shape->in_dtype != LA_F32;
    a.eps = eps;
    a.qk_scale = is_rf(phi->kind) ? phi->qk_scale : 1.0f;
    a.rf_sign = rf_sign(phi->kind);
    a.omega = phi->omega;
    hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = launch(LA_KERNEL_DECODE, [&] { return ent->dec(a, strm); });
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
}

}  // extern "C"
