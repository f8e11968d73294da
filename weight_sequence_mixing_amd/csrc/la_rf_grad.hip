// la_rf_grad.hip -- the feature-map end of the random-feature backward.
//
// The trigonometric random features ("From standard attention to linear
// attention", sec. 4.2, with the prefactor variants of la.h):
//   x' = s x,  u_r = omega_r . x'  (r < m),  c = exp(sigma |x'|^2 / 2) / sqrt(m),
//   phi(x) = c [cos u_1 .. cos u_m, sin u_1 .. sin u_m]        (F = 2m)
// with sigma = -1, 0 or +1 for the three kinds.  The backward computes phi(q),
// phi(k) once (la_rf_features_kernel), runs the elementwise backward sweeps
// on them as if they were the inputs (identity map), and maps the resulting
// d phi back to the inputs with the vector-Jacobian product of the map
// (la_rf_vjp_kernel):
//   g_r   = c (-sin u_r dphi_r + cos u_r dphi_{m+r}),
//   P     = sum_r c (cos u_r dphi_r + sin u_r dphi_{m+r})       (= phi . dphi),
//   dx    = s (omega^T g + sigma x' P).
// Both kernels recompute u in fp32 from the stored x and fp32 omega, one
// workgroup per TB rows, the rows' scaled x' in LDS.  Phase A (u, sine,
// cosine): thread j owns feature r = j % m and keeps omega's row r in
// registers; the threads of one r step through the rows, reading each x'
// row as 16-byte broadcasts.  Phase B (dx): thread j owns input column
// d = j % d_k and keeps omega's column d in registers, reading g rows the
// same way.
#include "la_device.h"
#include "la_internal.h"

namespace la {

constexpr int kRfThreads = 256;
constexpr int kRfRows = 64;        // rows (tokens) per workgroup
constexpr int kRfMaxM = 128;       // largest m

template <class T> __device__ __forceinline__ void rf_sincos(float u, float* s, float* c);
template <> __device__ __forceinline__ void rf_sincos<bf16>(float u, float* s, float* c) {
    *s = __sinf(u);
    *c = __cosf(u);
}
template <> __device__ __forceinline__ void rf_sincos<float>(float u, float* s, float* c) { sincosf(u, s, c); }

template <class T> __device__ __forceinline__ float rf_exp(float x);
template <> __device__ __forceinline__ float rf_exp<bf16>(float x) { return __expf(x); }
template <> __device__ __forceinline__ float rf_exp<float>(float x) { return expf(x); }

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
        sC[tid] = rf_exp<T>(0.5f * a.sign * s2) * rsqrtf((float)a.m);
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
        rf_sincos<T>(u, &sn, &cs);
        out[(r0 + t) * F + r] = from_f32<T>(sC[t] * cs);
        out[(r0 + t) * F + m + r] = from_f32<T>(sC[t] * sn);
    }
}

// dx = s (omega^T g + sigma x' P) from fp32 d phi ([rows, 2m]); rows whose
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
            dc[j] = a.dphi[row * F + r];
            ds[j] = a.dphi[row * F + m + r];
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
                rf_sincos<T>(u, &sn, &cs);
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
    return a.dk == 64 ? rf_launch<bf16, 64>(a, vjp, stream) : rf_launch<bf16, 128>(a, vjp, stream);
}

}  // namespace la
