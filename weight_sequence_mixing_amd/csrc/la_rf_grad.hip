// la_rf_grad.hip -- the feature-map end of the random-feature backward.
//
// The trigonometric random features ("From standard attention to linear
// attention", sec. 4.2, with the prefactor variants of la.h):
//   x' = s x,  u_r = omega_r . x'  (r < m),  c = exp(sigma |x'|^2 / 2) / sqrt(m),
//   phi(x) = c [cos u_1 .. cos u_m, sin u_1 .. sin u_m]        (F = 2m)
// with sigma = -1, 0 or +1 for the three kinds.  The backward computes phi(q),
// phi(k) once (the features kernels), runs the elementwise backward sweeps on
// them as if they were the inputs (identity map), and maps the resulting
// d phi back to the inputs with the vector-Jacobian product of the map (the
// vjp kernels):
//   g_r   = c (-sin u_r dphi_r + cos u_r dphi_{m+r}),
//   P     = sum_r c (cos u_r dphi_r + sin u_r dphi_{m+r})       (= phi . dphi),
//   dx    = s (omega^T g + sigma x' P).
//
// bf16 inputs: both products run on the matrix cores, one wave per 16 rows.
// U^T = omega' X^T with omega' = omega s / (2 pi) as bf16 high and low parts
// (the angles come out in revolutions, the unit of the hardware sine and
// cosine, and x is exact in bf16), then dX^T = omega^T G^T with omega and G
// each split into high and low parts (three products: hi.hi, lo.hi, hi.lo).
// In the accumulator of U^T a lane holds four features of token l%16 per
// 16-row block; a pair of blocks gives the lane eight features, which are
// its B operand of the second product once omega^T's fragments list the same
// features in the same order, so g never leaves registers.  The lane's x
// fragment holds the x' entries of the dx^T tile it ends with.  omega's
// operand fragments of both products are built once per workgroup in LDS.
//
// fp32 inputs: fp32 vector arithmetic, one workgroup per kRfRows rows with
// the rows' x' in LDS.  Phase A (u, sine, cosine): thread j owns feature
// r = j % m and keeps omega's row r in registers; the threads of one r step
// through the rows, reading each x' row as 16-byte broadcasts.  Phase B (dx):
// thread j owns input column d = j % d_k and keeps omega's column d in
// registers, reading g rows the same way.
#include <type_traits>

#include "la_device.h"
#include "la_internal.h"

namespace la {

constexpr int kRfThreads = 256;
constexpr int kRfRows = 64;        // rows (tokens) per workgroup
constexpr int kRfMaxM = 128;       // largest m


// Shared set-up: the scaled rows x' of this workgroup in LDS ([TB][DK],
// zero past the end) and each row's prefactor c.
template <class T, int DK>
__device__ __forceinline__ void rf_stage(const RfGradArgs& a, int64_t r0, int nt, float* sX, float* sC)
{
    const int tid = threadIdx.x;
    const T* x = (const T*)a.x;
    for (int i = tid; i < kRfRows * DK; i += kRfThreads) {
        const int t = i / DK, d = i % DK;
        sX[i] = t < nt ? a.scale * to_f32(x[(r0 + t) * DK + d]) : 0.f;
    }
    __syncthreads();
    if (tid < kRfRows) {
        float s2 = 0.f;
        for (int d = 0; d < DK; ++d) s2 += sX[tid * DK + d] * sX[tid * DK + d];
        sC[tid] = expf(0.5f * a.sign * s2) * rsqrtf((float)a.m);
    }
    __syncthreads();
}

// u = omega_r . x'_t with omega_r in registers and x'_t read as broadcasts
template <int DK>
__device__ __forceinline__ float rf_dot(const float (&w)[DK], const float* xrow)
{
    float u0 = 0.f, u1 = 0.f;
#pragma unroll
    for (int d = 0; d < DK; d += 8) {
        const f32x4 a = *(const f32x4*)(xrow + d), b = *(const f32x4*)(xrow + d + 4);
        u0 += w[d] * a[0] + w[d + 1] * a[1] + w[d + 2] * a[2] + w[d + 3] * a[3];
        u1 += w[d + 4] * b[0] + w[d + 5] * b[1] + w[d + 6] * b[2] + w[d + 7] * b[3];
    }
    return u0 + u1;
}

// phi(x) for a.rows rows, written in the input type ([rows, 2m]).
template <class T, int DK>
__global__ void __launch_bounds__(kRfThreads) la_rf_features_kernel(const RfGradArgs a)
{
    __shared__ __attribute__((aligned(16))) float sX[kRfRows * DK];
    __shared__ float sC[kRfRows];
    const int64_t r0 = (int64_t)blockIdx.x * kRfRows;
    const int nt = (int)min((int64_t)kRfRows, a.rows - r0);
    const int m = a.m, F = 2 * m, tid = threadIdx.x;
    // thread j: feature r = j % m of rows j / m, j / m + G, ... (G = 256 / m)
    const int r = tid % m, G = kRfThreads / m;
    float w[DK];
#pragma unroll
    for (int d = 0; d < DK; ++d) w[d] = a.omega[r * DK + d];
    rf_stage<T, DK>(a, r0, nt, sX, sC);
    T* out = (T*)a.out;
    for (int t = tid / m; t < nt; t += G) {
        const float u = rf_dot<DK>(w, sX + t * DK);
        float sn, cs;
        sincosf(u, &sn, &cs);
        out[(r0 + t) * F + r] = from_f32<T>(sC[t] * cs);
        out[(r0 + t) * F + m + r] = from_f32<T>(sC[t] * sn);
    }
}

// dx = s (omega^T g + sigma x' P) from d phi ([rows, 2m], input type); rows whose
// key is padded (a.kpm) get dx = 0.
template <class T, int DK, int M>
__global__ void __launch_bounds__(kRfThreads) la_rf_vjp_kernel(const RfGradArgs a)
{
    __shared__ __attribute__((aligned(16))) float sX[kRfRows * DK];
    // a row's m features span NH = max(1, M / 64) waves (or share one)
    constexpr int NH = M > 64 ? M / 64 : 1;
    __shared__ __attribute__((aligned(16))) float sG[kRfRows * M];
    __shared__ float sPw[kRfRows * NH];
    __shared__ float sC[kRfRows];
    __shared__ float sP[kRfRows];
    const int64_t r0 = (int64_t)blockIdx.x * kRfRows;
    const int nt = (int)min((int64_t)kRfRows, a.rows - r0);
    constexpr int m = M, F = 2 * M;
    const int tid = threadIdx.x;
    {
        // phase A: g_r and the terms of P for feature r = tid % m, rows
        // tid / m + j G; the rows' d phi values are all requested first
        constexpr int G = kRfThreads / M, NTH = kRfRows / G;
        const int r = tid % m, t0 = tid / m;
        float dc[NTH], ds[NTH];
#pragma unroll
        for (int j = 0; j < NTH; ++j) {
            const int t = t0 + j * G;
            const int64_t row = r0 + min(t, nt - 1);  // in bounds; rows past the end unused
            dc[j] = to_f32(((const T*)a.dphi)[row * F + r]);
            ds[j] = to_f32(((const T*)a.dphi)[row * F + m + r]);
        }
        float w[DK];
#pragma unroll
        for (int d = 0; d < DK; ++d) w[d] = a.omega[r * DK + d];
        rf_stage<T, DK>(a, r0, nt, sX, sC);
#pragma unroll
        for (int j = 0; j < NTH; ++j) {
            const int t = t0 + j * G;
            float g = 0.f, p = 0.f;
            if (t < nt) {
                const float u = rf_dot<DK>(w, sX + t * DK);
                float sn, cs;
                sincosf(u, &sn, &cs);
                g = sC[t] * (cs * ds[j] - sn * dc[j]);
                p = sC[t] * (cs * dc[j] + sn * ds[j]);
            }
            sG[t * m + r] = g;
            // P's terms summed over the lanes of this row (all 64 lanes of
            // the wave for m >= 64, each half for m = 32)
            p = wave_sum_xor(p, 1, (M < 64 ? M : 64) / 2);
            if (r % 64 == 0) sPw[t * NH + r / 64] = p;
        }
    }
    __syncthreads();
    if (tid < kRfRows) {
        float s = 0.f;
#pragma unroll
        for (int h = 0; h < NH; ++h) s += sPw[tid * NH + h];
        sP[tid] = s;
    }
    __syncthreads();
    // phase B: column d = tid % DK of omega in registers, rows tid / DK, +G, ...
    const int d = tid % DK, G = kRfThreads / DK;
    float wc[M];
#pragma unroll
    for (int r = 0; r < M; ++r) wc[r] = a.omega[r * DK + d];
    T* out = (T*)a.out;
    for (int t = tid / DK; t < nt; t += G) {
        const int64_t row = r0 + t;
        const float* grow = sG + t * m;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int r = 0; r < M; r += 8) {
            const f32x4 ga = *(const f32x4*)(grow + r), gb = *(const f32x4*)(grow + r + 4);
            acc0 += wc[r] * ga[0] + wc[r + 1] * ga[1] + wc[r + 2] * ga[2] + wc[r + 3] * ga[3];
            acc1 += wc[r + 4] * gb[0] + wc[r + 5] * gb[1] + wc[r + 6] * gb[2] + wc[r + 7] * gb[3];
        }
        float dx = a.scale * (acc0 + acc1 + a.sign * sX[t * DK + d] * sP[t]);
        if (a.kpm) {
            const int64_t bh = row / a.N, n = row % a.N;
            if (a.kpm[(bh / a.H) * a.kpm_stride + n]) dx = 0.f;
        }
        out[row * DK + d] = from_f32<T>(dx);
    }
}

// ---- bf16 inputs: matrix-core kernels -----------------------------------

constexpr int kMfWaves = 4;  // waves per workgroup; each wave takes 16-row tiles

template <int DK, int M> struct RfMf {
    static constexpr int KX = DK / 32;  // k blocks of the first product (over d)
    static constexpr int RB = M / 16;   // 16-feature row blocks of U^T
    static constexpr int DB = DK / 16;  // 16-row blocks of dX^T (input columns)
    static constexpr int KF = M / 32;   // k blocks of the second product (over r)
    // omega' fragments of U^T = omega' X^T: (rb, kb, part)
    static constexpr int NA = RB * KX * 2;
    // omega^T fragments of dX^T = omega^T G^T: (db, kf, part)
    static constexpr int NB = DB * KF * 2;
    // Feature held in accumulator row j (= 4 (l/16) + r) of U^T block rb:
    // the blocks pair up, and lane group g of pair p holds features
    // 32 p + 8 g + 0..7, so a lane's eight values of a pair are adjacent in
    // phi's row and the four groups cover 64 contiguous bytes of it.
    __device__ static __forceinline__ int feat(int rb, int j) { return 32 * (rb / 2) + 8 * (j / 4) + 4 * (rb % 2) + j % 4; }
    __device__ static __forceinline__ int fa(int rb, int kb, int part) { return (rb * KX + kb) * 2 + part; }
    __device__ static __forceinline__ int fb(int db, int kf, int part) { return NA + (db * KF + kf) * 2 + part; }
};

// High and low bf16 parts of 8 fp32 values (hi + lo = w to about 16 bits).
__device__ __forceinline__ void rf_split(const float (&w)[8], Frag<bf16>& hi, Frag<bf16>& lo)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        hi.v[e] = (bf16)w[e];
        lo.v[e] = (bf16)(w[e] - (float)hi.v[e]);
    }
}

// Builds omega's operand fragments of the workgroup in LDS.  For U^T, lane L
// of fragment (rb, kb) holds feature feat(rb, L%16) of omega (scaled into
// revolutions) at the input columns K(L/16) of k block kb.  For dX^T, lane L
// of fragment (db, kf) holds input column 16 db + L%16 of omega at the eight
// features 32 kf + 8 (L/16) + 0..7 -- the features its lane holds of the
// U^T block pair kf, in the same order, which is what makes the two
// operands of the second product agree on the contraction index.
template <int DK, int M, bool NEED_B>
__device__ __forceinline__ void rf_build_frags(const RfGradArgs& a, Frag<bf16>* sOm)
{
    using P = RfMf<DK, M>;
    const float om_scale = a.scale * 0.159154943091895336f;  // s / (2 pi)
    constexpr int NPAIR = (P::NA + (NEED_B ? P::NB : 0)) / 2;
    for (int i = threadIdx.x; i < NPAIR * 64; i += kMfWaves * 64) {
        const int pr = i / 64, L = i % 64, r16 = L % 16, g = L / 16;
        float w[8];
        int idx;
        if (pr < P::NA / 2) {
            const int rb = pr / P::KX, kb = pr % P::KX;
            const float* p = a.omega + P::feat(rb, r16) * DK + 32 * kb + 4 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                w[e] = p[e] * om_scale;
                w[4 + e] = p[16 + e] * om_scale;
            }
            idx = P::fa(rb, kb, 0);
        } else {
            const int q = pr - P::NA / 2, db = q / P::KF, kf = q % P::KF;
            const float* p = a.omega + (32 * kf + 8 * g) * DK + 16 * db + r16;
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = p[e * DK];
            idx = P::fb(db, kf, 0);
        }
        Frag<bf16> hi, lo;
        rf_split(w, hi, lo);
        sOm[idx * 64 + L] = hi;
        sOm[(idx + 1) * 64 + L] = lo;
    }
    __syncthreads();
}

// Per-tile values shared by both kernels: this lane's x fragments (its token
// row, clamped into range for the loads) and the row's prefactor c.
template <int DK, int M>
struct RfTile {
    Frag<bf16> xf[DK / 32];
    float c;
};

template <int DK, int M>
__device__ __forceinline__ void rf_load_x(const RfGradArgs& a, int64_t tr, int g, RfTile<DK, M>& t)
{
    const bf16* x = (const bf16*)a.x + tr * DK;
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) t.xf[kb] = frag_rm(x, 0, 0, 32 * kb, g);
}

template <int DK, int M>
__device__ __forceinline__ void rf_prefactor(const RfGradArgs& a, RfTile<DK, M>& t)
{
    float s2 = 0.f;
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = (float)t.xf[kb].v[e];
            s2 += v * v;
        }
    s2 += __shfl_xor(s2, 16, 64);
    s2 += __shfl_xor(s2, 32, 64);
    t.c = __expf(0.5f * a.sign * a.scale * a.scale * s2) * rsqrtf((float)M);
}

// U^T block rb against this lane's token (features feat(rb, 4 g + r)), in
// revolutions.
template <int DK, int M>
__device__ __forceinline__ f32x4 rf_angles(const Frag<bf16>* sOm, const RfTile<DK, M>& t, int rb, int lane)
{
    using P = RfMf<DK, M>;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < P::KX; ++kb) {
        mma(acc, sOm[P::fa(rb, kb, 0) * 64 + lane], t.xf[kb]);
        mma(acc, sOm[P::fa(rb, kb, 1) * 64 + lane], t.xf[kb]);
    }
    return acc;
}

// Zero that the compiler cannot see through, taken once per tile: offsetting
// the fragment base by it keeps the fragment reads inside the tile loop
// instead of hoisted out of it into registers (all of omega's fragments at
// once would not fit).
__device__ __forceinline__ int rf_opaque_zero()
{
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    return z;
}

// Persistent grid: as many workgroups as fit on the device at once; wave w
// of workgroup b takes tiles 8 b + w, + 8 * gridDim.x, ...
template <class K>
hipError_t rf_mf_launch(K kernel, const RfGradArgs& a, hipStream_t stream)
{
    const int slots = device_slots(kernel, kMfWaves * 64);
    if (slots <= 0) return hipErrorInvalidDevice;
    const int64_t tiles = (a.rows + 15) / 16;
    const int64_t want = (tiles + kMfWaves - 1) / kMfWaves;
    const int64_t cap = slots;
    const dim3 grid((unsigned)(want < cap ? want : cap)), block(kMfWaves * 64);
    return launch_kernel(kernel, grid, block, stream, a);
}

// phi(x) for a.rows rows ([rows, 2m] bf16).
template <int DK, int M>
__global__ void __launch_bounds__(kMfWaves * 64) la_rf_features_mfma_kernel(const RfGradArgs a)
{
    using P = RfMf<DK, M>;
    __shared__ Frag<bf16> sOm[P::NA * 64];
    rf_build_frags<DK, M, false>(a, sOm);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const int64_t tiles = (a.rows + 15) / 16;
    bf16* out = (bf16*)a.out;
    for (int64_t tile = (int64_t)blockIdx.x * kMfWaves + wave; tile < tiles; tile += (int64_t)gridDim.x * kMfWaves) {
        const int64_t row = tile * 16 + l16, tr = row < a.rows ? row : a.rows - 1;
        const Frag<bf16>* om = sOm + rf_opaque_zero();
        RfTile<DK, M> t;
        rf_load_x(a, tr, g, t);
        rf_prefactor(a, t);
        bf16* o = out + tr * (2 * M) + 8 * g;
#pragma unroll
        for (int pr = 0; pr < P::RB / 2; ++pr) {
            bf16x8 cs, sn;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 u = rf_angles(om, t, 2 * pr + h, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    cs[4 * h + r] = (bf16)(t.c * __builtin_amdgcn_cosf(u[r]));
                    sn[4 * h + r] = (bf16)(t.c * __builtin_amdgcn_sinf(u[r]));
                }
            }
            if (row < a.rows) {
                *(bf16x8*)(o + 32 * pr) = cs;
                *(bf16x8*)(o + M + 32 * pr) = sn;
            }
        }
    }
}

// dx = s (omega^T g + sigma x' P) from bf16 d phi ([rows, 2m]), bf16 out;
// rows whose key is padded (a.kpm) get dx = 0.
template <int DK, int M>
__global__ void __launch_bounds__(kMfWaves * 64) la_rf_vjp_mfma_kernel(const RfGradArgs a)
{
    using P = RfMf<DK, M>;
    __shared__ Frag<bf16> sOm[(P::NA + P::NB) * 64];
    rf_build_frags<DK, M, true>(a, sOm);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const int64_t tiles = (a.rows + 15) / 16;
    bf16* out = (bf16*)a.out;
    const float s = a.scale, ssig = a.sign * a.scale * a.scale;
    for (int64_t tile = (int64_t)blockIdx.x * kMfWaves + wave; tile < tiles; tile += (int64_t)gridDim.x * kMfWaves) {
        const int64_t row = tile * 16 + l16, tr = row < a.rows ? row : a.rows - 1;
        // every load of the tile first: d phi of this lane's features, x
        const bf16* dp = (const bf16*)a.dphi + tr * (2 * M) + 8 * g;
        bf16x8 dc[P::RB / 2], ds[P::RB / 2];
#pragma unroll
        for (int pr = 0; pr < P::RB / 2; ++pr) {
            dc[pr] = *(const bf16x8*)(dp + 32 * pr);
            ds[pr] = *(const bf16x8*)(dp + M + 32 * pr);
        }
        const Frag<bf16>* om = sOm + rf_opaque_zero();
        RfTile<DK, M> t;
        rf_load_x(a, tr, g, t);
        rf_prefactor(a, t);
        // g (the B operand of the second product, in accumulator layout) and
        // this lane's terms of P
        f32x4 gt[P::RB];
        float p = 0.f;
#pragma unroll
        for (int rb = 0; rb < P::RB; ++rb) {
            const f32x4 u = rf_angles(om, t, rb, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float cs = __builtin_amdgcn_cosf(u[r]), sn = __builtin_amdgcn_sinf(u[r]);
                const float c1 = (float)dc[rb / 2][4 * (rb % 2) + r], s1 = (float)ds[rb / 2][4 * (rb % 2) + r];
                gt[rb][r] = t.c * (cs * s1 - sn * c1);
                p += cs * c1 + sn * s1;
            }
        }
        p += __shfl_xor(p, 16, 64);
        p += __shfl_xor(p, 32, 64);
        p *= t.c;
        // dX^T: lane holds input columns 16 db + 4 g + 0..3 of its token
        f32x4 dx[P::DB];
#pragma unroll
        for (int db = 0; db < P::DB; ++db) dx[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kf = 0; kf < P::KF; ++kf) {
            float w[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                w[e] = gt[2 * kf][e];
                w[4 + e] = gt[2 * kf + 1][e];
            }
            Frag<bf16> ghi, glo;
            rf_split(w, ghi, glo);
#pragma unroll
            for (int db = 0; db < P::DB; ++db) {
                const Frag<bf16> whi = om[P::fb(db, kf, 0) * 64 + lane];
                mma(dx[db], whi, ghi);
                mma(dx[db], om[P::fb(db, kf, 1) * 64 + lane], ghi);
                mma(dx[db], whi, glo);
            }
        }
        bool zero = false;
        if (a.kpm) {
            const int64_t bh = tr / a.N, n = tr % a.N;
            zero = a.kpm[(bh / a.H) * a.kpm_stride + n] != 0;
        }
        if (row < a.rows) {
            bf16* o = out + row * DK + 4 * g;
#pragma unroll
            for (int db = 0; db < P::DB; ++db) {
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float xd = (float)t.xf[db / 2].v[4 * (db % 2) + r];
                    v[r] = zero ? 0.f : s * dx[db][r] + ssig * xd * p;
                }
                st4(o + 16 * db, v[0], v[1], v[2], v[3]);
            }
        }
    }
}

template <int DK>
hipError_t rf_mf_dispatch(const RfGradArgs& a, bool vjp, hipStream_t stream)
{
    auto go = [&](auto mc) {
        constexpr int M = decltype(mc)::value;
        // random features need d_k * m <= 8192 (the forward's bound)
        if constexpr (DK * M > 8192) {
            return hipErrorInvalidValue;
        } else {
            return vjp ? rf_mf_launch(la_rf_vjp_mfma_kernel<DK, M>, a, stream)
                       : rf_mf_launch(la_rf_features_mfma_kernel<DK, M>, a, stream);
        }
    };
    switch (a.m) {
    case 32: return go(std::integral_constant<int, 32>());
    case 64: return go(std::integral_constant<int, 64>());
    case 128: return go(std::integral_constant<int, 128>());
    default: return hipErrorInvalidValue;
    }
}

template <class T, int DK>
hipError_t rf_launch(const RfGradArgs& a, bool vjp, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.rows + kRfRows - 1) / kRfRows)), block(kRfThreads);
    if (!vjp) return launch_kernel(la_rf_features_kernel<T, DK>, grid, block, stream, a);
    switch (a.m) {
    case 32: return launch_kernel(la_rf_vjp_kernel<T, DK, 32>, grid, block, stream, a);
    case 64: return launch_kernel(la_rf_vjp_kernel<T, DK, 64>, grid, block, stream, a);
    case 128: return launch_kernel(la_rf_vjp_kernel<T, DK, 128>, grid, block, stream, a);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rf_grad(const RfGradArgs& a, bool vjp, hipStream_t stream)
{
    if (a.rows <= 0) return hipSuccess;
    if (a.m < 1 || a.m > kRfMaxM || (a.dk != 64 && a.dk != 128)) return hipErrorInvalidValue;
    if (a.in_f32) return a.dk == 64 ? rf_launch<float, 64>(a, vjp, stream) : rf_launch<float, 128>(a, vjp, stream);
    return a.dk == 64 ? rf_mf_dispatch<64>(a, vjp, stream) : rf_mf_dispatch<128>(a, vjp, stream);
}

}  // namespace la
