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
// workgroup per TB rows: omega sits transposed in LDS with a padded row
// (omega^T[d][r] at d*(MP) + r, MP = 129), so that a sweep over r (phase A)
// and one over d (phase B) both touch distinct banks.
#include "la_device.h"
#include "la_internal.h"

namespace la {

constexpr int kRfThreads = 256;
constexpr int kRfRows = 32;        // rows (tokens) per workgroup
constexpr int kRfMaxM = 128;       // largest m
constexpr int kRfMP = kRfMaxM + 1; // padded row of omega^T and of the per-row arrays

template <class T> __device__ __forceinline__ void rf_sincos(float u, float* s, float* c);
template <> __device__ __forceinline__ void rf_sincos<bf16>(float u, float* s, float* c) {
    *s = __sinf(u);
    *c = __cosf(u);
}
template <> __device__ __forceinline__ void rf_sincos<float>(float u, float* s, float* c) { sincosf(u, s, c); }

template <class T> __device__ __forceinline__ float rf_exp(float x);
template <> __device__ __forceinline__ float rf_exp<bf16>(float x) { return __expf(x); }
template <> __device__ __forceinline__ float rf_exp<float>(float x) { return expf(x); }

// Shared set-up of both kernels: omega^T and the scaled rows x' of this
// workgroup in LDS, and each row's prefactor c.  Rows past the end are zero.
template <class T, int DK>
__device__ __forceinline__ void rf_stage(const RfGradArgs& a, int64_t r0, int nt, float* sOmT, float* sX, float* sC)
{
    const int tid = threadIdx.x, m = a.m;
    for (int i = tid; i < m * DK; i += kRfThreads) {
        const int r = i / DK, d = i % DK;
        sOmT[d * kRfMP + r] = a.omega[i];
    }
    const T* x = (const T*)a.x;
    for (int i = tid; i < kRfRows * DK; i += kRfThreads) {
        const int t = i / DK, d = i % DK;
        sX[t * (DK + 1) + d] = t < nt ? a.scale * to_f32(x[(r0 + t) * DK + d]) : 0.f;
    }
    __syncthreads();
    if (tid < kRfRows) {
        float s2 = 0.f;
        for (int d = 0; d < DK; ++d) s2 += sX[tid * (DK + 1) + d] * sX[tid * (DK + 1) + d];
        sC[tid] = rf_exp<T>(0.5f * a.sign * s2) * rsqrtf((float)m);
    }
    __syncthreads();
}

// phi(x) for a.rows rows, written in the input type ([rows, 2m]).
template <class T, int DK>
__global__ void __launch_bounds__(kRfThreads) la_rf_features_kernel(const RfGradArgs a)
{
    __shared__ float sOmT[DK * kRfMP];
    __shared__ float sX[kRfRows * (DK + 1)];
    __shared__ float sC[kRfRows];
    const int64_t r0 = (int64_t)blockIdx.x * kRfRows;
    const int nt = (int)min((int64_t)kRfRows, a.rows - r0);
    rf_stage<T, DK>(a, r0, nt, sOmT, sX, sC);
    const int m = a.m, F = 2 * m;
    T* out = (T*)a.out;
    // r fastest: omega^T reads are consecutive, the row of x' is shared
    for (int i = threadIdx.x; i < kRfRows * m; i += kRfThreads) {
        const int t = i / m, r = i % m;
        if (t >= nt) continue;
        float u = 0.f;
#pragma unroll 8
        for (int d = 0; d < DK; ++d) u += sOmT[d * kRfMP + r] * sX[t * (DK + 1) + d];
        float sn, cs;
        rf_sincos<T>(u, &sn, &cs);
        out[(r0 + t) * F + r] = from_f32<T>(sC[t] * cs);
        out[(r0 + t) * F + m + r] = from_f32<T>(sC[t] * sn);
    }
}

// dx = s (omega^T g + sigma x' P) from fp32 d phi ([rows, 2m]); rows whose
// key is padded (a.kpm) get dx = 0.
template <class T, int DK>
__global__ void __launch_bounds__(kRfThreads) la_rf_vjp_kernel(const RfGradArgs a)
{
    __shared__ float sOmT[DK * kRfMP];
    __shared__ float sX[kRfRows * (DK + 1)];
    __shared__ float sC[kRfRows];
    __shared__ float sG[kRfRows * kRfMP];
    __shared__ float sPp[kRfRows * kRfMP];
    __shared__ float sP[kRfRows];
    const int64_t r0 = (int64_t)blockIdx.x * kRfRows;
    const int nt = (int)min((int64_t)kRfRows, a.rows - r0);
    rf_stage<T, DK>(a, r0, nt, sOmT, sX, sC);
    const int m = a.m, F = 2 * m, tid = threadIdx.x;
    // phase A (r fastest): g_r and the terms of P
    for (int i = tid; i < kRfRows * m; i += kRfThreads) {
        const int t = i / m, r = i % m;
        float g = 0.f, p = 0.f;
        if (t < nt) {
            float u = 0.f;
#pragma unroll 8
            for (int d = 0; d < DK; ++d) u += sOmT[d * kRfMP + r] * sX[t * (DK + 1) + d];
            float sn, cs;
            rf_sincos<T>(u, &sn, &cs);
            const float dc = a.dphi[(r0 + t) * F + r], ds = a.dphi[(r0 + t) * F + m + r];
            g = sC[t] * (cs * ds - sn * dc);
            p = sC[t] * (cs * dc + sn * ds);
        }
        sG[t * kRfMP + r] = g;
        sPp[t * kRfMP + r] = p;
    }
    __syncthreads();
    if (tid < kRfRows) {
        float s = 0.f;
        for (int r = 0; r < m; ++r) s += sPp[tid * kRfMP + r];
        sP[tid] = s;
    }
    __syncthreads();
    // phase B (d fastest): dx_d = s (sum_r omega_rd g_r + sigma x'_d P)
    T* out = (T*)a.out;
    for (int i = tid; i < kRfRows * DK; i += kRfThreads) {
        const int t = i / DK, d = i % DK;
        if (t >= nt) continue;
        const int64_t row = r0 + t;
        float acc = 0.f;
#pragma unroll 8
        for (int r = 0; r < m; ++r) acc += sOmT[d * kRfMP + r] * sG[t * kRfMP + r];
        float dx = a.scale * (acc + a.sign * sX[t * (DK + 1) + d] * sP[t]);
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
    return vjp ? launch_kernel(la_rf_vjp_kernel<T, DK>, grid, block, stream, a)
               : launch_kernel(la_rf_features_kernel<T, DK>, grid, block, stream, a);
}

hipError_t launch_rf_grad(const RfGradArgs& a, bool vjp, hipStream_t stream)
{
    if (a.rows <= 0) return hipSuccess;
    if (a.m < 1 || a.m > kRfMaxM || (a.dk != 64 && a.dk != 128)) return hipErrorInvalidValue;
    if (a.in_f32) return a.dk == 64 ? rf_launch<float, 64>(a, vjp, stream) : rf_launch<float, 128>(a, vjp, stream);
    return a.dk == 64 ? rf_launch<bf16, 64>(a, vjp, stream) : rf_launch<bf16, 128>(a, vjp, stream);
}

}  // namespace la
