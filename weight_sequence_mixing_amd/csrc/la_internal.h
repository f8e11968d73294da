// la_internal.h -- host/device interface between the C ABI (la_api.cpp) and
// the HIP kernels.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/la.h"

namespace la {

// Internal feature-map kind: the inputs are already features (F = d_k).  The
// random-feature backward runs the elementwise sweeps on phi(q), phi(k) with
// it and maps their d phi back through omega itself.
constexpr int kPhiIdentity = 100;

// Per-head decay, passed by value in the kernel arguments so that a launch
// never needs a host-to-device copy (and can be recorded into a graph).
struct LamTable {
    float lam[LA_MAX_HEADS];
    float log2lam[LA_MAX_HEADS];  // log2(lambda); -inf for lambda == 0
};

enum FwdMode : int {
    MODE_LOCAL = 0,   // segment-local state  sum_j lambda^(L-1-j) phi(k_j) [v_j, 1]^T
    MODE_CAUSAL = 1,  // chunked causal output with a carried state
    MODE_QUERY = 2,   // non-causal output phi(Q) S / (phi(Q) z + eps) for a fixed state
};

// One launch of the forward kernel covers tokens [n0, n0 + n_len) of every
// (batch, head) row, cut into P segments of cps whole chunks each (the last
// may be shorter; blockIdx.x = segment, blockIdx.y = batch*head).
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* y;
    int64_t N;        // full sequence length (token stride of q, k, v, y)
    int64_t n0;       // first token of this launch
    int64_t n_len;    // tokens in this launch
    int32_t BH;       // batch * heads
    int32_t H;
    int32_t P;        // segments
    int64_t cps;      // units of `chunk` tokens per segment
    int32_t chunk;    // tokens per unit of cps: the planning chunk, a multiple of every kernel's own
    int32_t out_f32;  // 1: y is fp32, 0: y has the input type
    float eps;
    float qk_scale;
    // random features: sign s of the prefactor exp(s |x'|^2 / 2) / sqrt(m),
    // and its scale 1 / sqrt(m) (m of the whole map: a launch may cover half
    // of the features)
    float rf_sign;
    float rf_scale;
    // causal output over one half of the features (random features with
    // m = 256): 1 stores each row's numerator and denominator (fp32, at
    // part_num + row * d_v and part_den + row, rows indexed as y), 2 adds the
    // stored ones to its own before the division; 0 = a whole map
    int32_t part_mode;
    float* part_num;
    float* part_den;
    const float* omega;  // [m, d_k] fp32 (random features) or null
    // key padding mask: byte kpm[b * kpm_stride + n0 + t] nonzero drops key t
    // of batch b from every sum; null = no mask
    const uint8_t* kpm;
    int64_t kpm_stride;
    // packed variable-length rows: sequence b holds tokens
    // [cu_seqlens[b], cu_seqlens[b+1]) of each head row h (N tokens per head
    // row; offsets are clamped to [0, N]).  Every sequence is cut into
    // segments of cps chunks, at most P (the last takes the remainder); the
    // grid is (G work items, H heads), item w of a head being the w-th
    // (sequence, segment) pair in order; items past the last exit.  The
    // kernels address states as row bh = b*H + h, segment s.  null = fixed rows.
    const int32_t* cu_seqlens;
    const int32_t* items;  // [G]: b * P + s of each work item in order, -1 past the last
    int32_t G;             // work items per head (an upper bound of the segments' count)
    // initial state (MODE_CAUSAL, MODE_QUERY): S at
    // S_src + seg*src_seg_stride + bh*src_stride as [F][d_v], z at
    // z_src + seg*src_seg_stride + bh*src_zstride as [F]; null S_src = zero state.
    const float* S_src;
    const float* z_src;
    int64_t src_stride;
    int64_t src_zstride;
    int64_t src_seg_stride;
    // rows f >= F/2 of S_src, z_src (S_dst, z_dst) sit src_gap (dst_gap) rows
    // further: one half of a split random-feature map in the caller's layout
    // (its cos and its sin rows); 0 elsewhere
    int32_t src_gap, dst_gap;
    // final state (MODE_CAUSAL, optional) or segment-local state (MODE_LOCAL):
    // written at S_dst + (seg*BH + bh)*dst_stride (MODE_LOCAL) or
    // S_dst + bh*dst_stride (MODE_CAUSAL), z likewise.
    float* S_dst;
    float* z_dst;
    int64_t dst_stride;
    int64_t dst_zstride;
    // MODE_LOCAL: 1 when no final state is wanted, so that the segment that
    // reaches the end of its row is not computed (no later segment reads it)
    int32_t skip_last;
    LamTable lam;
};

struct ScanArgs {
    float* ws;               // slots [P][BH][F*d_v + F]
    int32_t P, BH, H, F, DV;
    int64_t n_len;           // tokens covered by the P segments
    int64_t seg_len;         // tokens per segment (cps * C); the last may be shorter
    int32_t causal;          // 1: exclusive decayed scan; 0: plain sum into slot 0
    // packed variable-length rows (as FwdArgs): per-sequence length from
    // cu_seqlens (clamped to [0, N]); a sequence covers its first
    // ceil(n / seg_len) segments (at most P), the others are empty and skipped
    const int32_t* cu_seqlens;
    int64_t N;
    const float* S_init;     // initial state (causal), user layout or carry slot
    const float* z_init;
    int64_t init_stride, init_zstride;
    float* S_fin;            // final state (causal) or null
    float* z_fin;
    int64_t fin_stride, fin_zstride;
    // rows f >= F/2 of S_init, z_init (S_fin, z_fin) sit init_gap (fin_gap)
    // rows further (as FwdArgs src_gap)
    int32_t init_gap, fin_gap;
    // 1: visit the segments last to first (the adjoint state of the backward
    // pass, carried from the end of the sequence towards its start)
    int32_t reverse;
    // causal, forward order, no final state: the local state of the last
    // segment holding tokens is neither read nor needed (FwdArgs skip_last)
    int32_t skip_last;
    LamTable lam;
};

// Backward passes of the causal forward.  One launch covers P segments of cps
// chunks of every (batch, head) row of N tokens (grid: P x BH), like FwdArgs.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* y;    // forward output (dq pass)
    const void* gy;   // gradient of y
    void* dq;
    void* dk;
    void* dv;
    float* tok;       // [BH][N][2]: 1/den and dden per token (written by the dq pass)
    int64_t N;
    int32_t BH, H, P;
    int64_t cps;
    float eps;
    const uint8_t* kpm;  // key padding mask [B][N] or null
    // carried-in state of each segment: forward state [S|z] (dq pass) or
    // adjoint [U|u] at the segment's end (kv pass), at
    // src + seg*src_seg_stride + bh*src_stride; null = zero
    const float* S_src;
    const float* z_src;
    int64_t src_stride, src_zstride, src_seg_stride;
    // reverse-local pass: segment sums at dst + (seg*BH + bh)*dst_stride;
    // kv pass with one segment: the initial state's gradient at
    // dst + bh*dst_stride, if set
    float* S_dst;
    float* z_dst;
    int64_t dst_stride, dst_zstride;
    // gradient of lambda (dq pass, optional): each workgroup writes its
    // segment's dT = d[S|z]/dlambda with the segment's start state held fixed
    // at tseg + (seg*BH + bh)*SZ, and its partial dlambda at dlp[seg*BH + bh]
    float* tseg;
    float* dlp;
    LamTable lam;
};

// Reduction of the lambda gradient: per (batch, head) row, the dq sweep's
// partials, plus <T_in(s), W_loc(s)> over the segments (T_in: the scan of the
// segments' dT; W_loc: the adjoint segment sums, or null with one segment),
// plus <[dS_out|dz_out], T_final>; then the sum over the batch per head.
struct DlamArgs {
    const float* wloc;    // [P][BH][SZ] or null
    const float* tseg;    // [P][BH][SZ]
    const float* dlp;     // [P][BH]
    const float* dS_out;  // [BH][F][DV] or null
    const float* dz_out;  // [BH][F]
    float* rows;          // [BH][dlam_blocks(F, DV)] partial sums
    float* dlam;          // [H] output
    int32_t P, BH, H, F, DV;
    int64_t n_len, seg_len;
    LamTable lam;
};
hipError_t launch_dlam(const DlamArgs& a, hipStream_t stream);
int dlam_blocks(int F, int DV);  // workgroups per row of the reduction

enum BwdMode : int {
    BMODE_Q = 0,       // dq, and 1/den, dden per token
    BMODE_RLOCAL = 1,  // segment sums of lambda^(i-s0) phi(q_i) [dnum_i, dden_i]^T
    BMODE_KV = 2,      // dk, dv from the carried adjoint
    BMODE_NCQ = 3,     // non-causal: dq from the total state, segment sums of phi(q_i) [dnum_i, dden_i]^T
    BMODE_NCKV = 4,    // non-causal: dk, dv from the total adjoint
};

struct DecArgs {
    const void* q;
    const void* k;
    const void* v;
    void* y;
    float* S;
    float* z;
    int32_t BH, H;
    int32_t out_f32;
    float eps;
    float qk_scale;
    float rf_sign;  // random features: sign of the prefactor's exponent
    const float* omega;
    int32_t ntok;      // tokens per head-state, processed in order ([B,H,ntok,d] inputs)
    LamTable lam;
};

typedef hipError_t (*fwd_launch_fn)(const FwdArgs&, int mode, hipStream_t);
typedef hipError_t (*dec_launch_fn)(const DecArgs&, hipStream_t);
typedef hipError_t (*bwd_launch_fn)(const BwdArgs&, int mode, hipStream_t);  // BMODE_Q with a.tseg: the dlambda variant

struct KernelEntry {
    int in_dtype;   // LA_F32 / LA_BF16
    int phi;        // LA_PHI_*
    int dk, F, dv;
    int C;          // chunk length used by the forward kernels
    fwd_launch_fn fwd;
    dec_launch_fn dec;
};

struct BwdEntry {
    int in_dtype, phi, dk, F, dv;
    int C;
    bwd_launch_fn bwd;
    bool dlam;  // the lambda-gradient variant of the dq sweep fits in LDS
};
extern BwdEntry kBwdEntriesBf16[];
extern int kNumBwdEntriesBf16;
extern BwdEntry kBwdEntriesF32[];
extern int kNumBwdEntriesF32;

// Tables defined by the instantiation units.
extern KernelEntry kEntriesBf16Elu[];
extern int kNumEntriesBf16Elu;
extern KernelEntry kEntriesBf16Rf[];
extern int kNumEntriesBf16Rf;
extern KernelEntry kEntriesF32[];
extern int kNumEntriesF32;
// identity-map entries of the random-feature backward (F = d_k = 2m)
extern KernelEntry kEntriesIdentBf16[];
extern int kNumEntriesIdentBf16;
extern KernelEntry kEntriesIdentF32[];
extern int kNumEntriesIdentF32;
extern BwdEntry kBwdEntriesIdentBf16[];
extern int kNumBwdEntriesIdentBf16;
extern BwdEntry kBwdEntriesIdentF32[];
extern int kNumBwdEntriesIdentF32;
extern KernelEntry kEntriesBf16Relu[];
extern int kNumEntriesBf16Relu;
extern KernelEntry kEntriesF32Relu[];
extern int kNumEntriesF32Relu;

// Per-launch timing: while `start` is set, the next kernel launched through
// launch_kernel records the dispatch's own begin and end timestamps into
// start/stop (the interval a kernel trace reports, without the queueing gap
// that a separate event record before the launch would add) and sets `fired`.
struct LaunchEvents {
    hipEvent_t start;
    hipEvent_t stop;
    bool fired;
};
LaunchEvents& launch_events();

template <class K, class... Args>
hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t stream, Args... args)
{
    LaunchEvents& ev = launch_events();
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev.start, ev.stop, 0, args...);
    if (ev.start) ev.fired = true;
    return hipGetLastError();
}

// Workgroups of `threads` threads of `kernel` resident at once on the current
// device (compute units x workgroups per unit); 0 if the runtime cannot say.
// Cached per kernel and device.
int device_slots(const void* kernel, int threads);
template <class K>
int device_slots(K kernel, int threads)
{
    return device_slots(reinterpret_cast<const void*>(kernel), threads);
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream);
// Work items of packed sequences: items[w] = b * P + s for the w-th
// (sequence, segment) pair in order, -1 for w past the last (G entries).
// Sequence b has max(1, min(ceil(chunks_b / cps), P)) segments.
hipError_t launch_varlen_items(const int32_t* cu, int B, int64_t N, int C, int64_t cps, int P, int G,
                               int32_t* items, hipStream_t stream);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);

// Random-feature backward, feature-map end (la_rf_grad.hip): phi(x) of `rows`
// rows ([rows, d_k] in, [rows, 2m] out, input type), or the vector-Jacobian
// product dx = J_phi(x)^T dphi (dphi [rows, 2m] input type, dx [rows, d_k] input
// type; rows of padded keys get 0 when kpm is set).
struct RfGradArgs {
    const void* x;
    const float* omega;  // [m, d_k] fp32
    const void* dphi;    // vjp only
    void* out;
    const uint8_t* kpm;  // vjp of keys: byte kpm[b * kpm_stride + n] of row (b*H + h)*N + n
    int64_t kpm_stride;
    int64_t N;
    int32_t H;
    int64_t rows;
    int32_t dk, m;
    float scale, sign;
    int32_t in_f32;
};
hipError_t launch_rf_grad(const RfGradArgs& a, bool vjp, hipStream_t stream);
// S[BH][F][DV] = alpha * I (f == d), z[BH][F] = alpha for f < min(F, DV)
hipError_t launch_fill_identity(float* S, float* z, int64_t BH, int F, int DV, float alpha, hipStream_t stream);
hipError_t launch_copy(float* dst, const float* src, int64_t n, hipStream_t stream);

// Static device scratch of la_forward_causal_noalloc (la_scratch.hip): one
// array of kScratchBytes per device, held until the process ends.  Its
// address on the current device, looked up once per device.
constexpr size_t kScratchBytes = (size_t)LA_NOALLOC_SCRATCH_BYTES;
hipError_t scratch_ptr(void** out);

}  // namespace la
