// la_scan.hip -- combination of per-segment states, and small fill/copy
// kernels.
//
// A sequence cut into P segments of lengths L_0..L_{P-1} has segment-local
// states S_loc(s) = sum over the segment of lambda^(L_s-1-j) phi(k_j)[v_j,1]^T.
// The state entering segment s is the decayed prefix
//   S_in(0) = S_init,  S_in(s) = lambda^(L_{s-1}) S_in(s-1) + S_loc(s-1),
// the same carry the chunked method applies between chunks ("Attention is
// also an FFN", kwkr.cn/news/587576, sec. 5.2: parallel inside a block,
// carried between blocks), applied once more between segments.  Each thread
// owns four elements of the [F x (d_v + 1)] state of one (batch, head) row and
// walks the P segments in order, in place.
#include "la_device.h"
#include "la_internal.h"

namespace la {

// Threads per workgroup of the scan, and segments whose loads are in flight
// together (one memory round trip per batch, not one per segment).
constexpr int kScanThreads = 64;
constexpr int kScanBatch = 16;

__global__ void __launch_bounds__(kScanThreads) la_scan_kernel(const ScanArgs a)
{
    // each thread owns 4 consecutive elements (F*d_v and F are multiples of 4,
    // so a group never straddles S and z; every base is 16-byte aligned)
    const int SZ = a.F * a.DV + a.F;
    const int e = 4 * (blockIdx.x * kScanThreads + threadIdx.x);
    const int bh = blockIdx.y;
    if (e >= SZ) return;
    const bool isz = e >= a.F * a.DV;
    const int ez = e - a.F * a.DV;
    f32x4* base = (f32x4*)(a.ws + (int64_t)bh * SZ + e);
    const int64_t slot = (int64_t)a.BH * SZ / 4;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 loc[kScanBatch];
    if (!a.causal) {
        f32x4 acc = zero;
        for (int s0 = 0; s0 < a.P; s0 += kScanBatch) {
#pragma unroll
            for (int b = 0; b < kScanBatch; ++b) loc[b] = (s0 + b < a.P) ? base[(s0 + b) * slot] : zero;
#pragma unroll
            for (int b = 0; b < kScanBatch; ++b) acc += loc[b];
        }
        base[0] = acc;
        return;
    }
    const float l2l = a.lam.log2lam[bh % a.H];
    int64_t n_len = a.n_len;
    if (a.cu_seqlens) {
        int64_t s0, s1;
        varlen_range(a.cu_seqlens, bh / a.H, a.N, &s0, &s1);
        n_len = s1 - s0;
    }
    // segments holding tokens (the last of the P takes the remainder)
    const int nseg = (int)min((n_len + a.seg_len - 1) / a.seg_len, (int64_t)a.P);
    f32x4 carry = zero;
    // the caller's layout may hold the upper half of the rows further on
    const int half_rows = a.F / 2;
    const int ei = isz ? ez + (ez >= half_rows ? a.init_gap : 0)
                       : e + (e >= half_rows * a.DV ? a.init_gap * a.DV : 0);
    const int ef = isz ? ez + (ez >= half_rows ? a.fin_gap : 0)
                       : e + (e >= half_rows * a.DV ? a.fin_gap * a.DV : 0);
    if (a.S_init)
        carry = isz ? *(const f32x4*)(a.z_init + bh * a.init_zstride + ei)
                    : *(const f32x4*)(a.S_init + bh * a.init_stride + ei);
    // reverse: the segments are visited last to first (the carry enters a
    // segment at its end)
    for (int s0 = 0; s0 < nseg; s0 += kScanBatch) {
#pragma unroll
        for (int b = 0; b < kScanBatch; ++b) {
            const int s = a.reverse ? nseg - 1 - (s0 + b) : s0 + b;
            const bool skipped = a.skip_last && s == nseg - 1;  // never computed
            loc[b] = (s0 + b < nseg && !skipped) ? base[s * slot] : zero;
        }
#pragma unroll
        for (int b = 0; b < kScanBatch; ++b) {
            if (s0 + b < nseg) {
                const int s = a.reverse ? nseg - 1 - (s0 + b) : s0 + b;
                const int64_t L = (s == a.P - 1 ? n_len : min((int64_t)(s + 1) * a.seg_len, n_len)) -
                                  (int64_t)s * a.seg_len;
                base[s * slot] = carry;
                carry = lam_pow(l2l, (int)L) * carry + loc[b];
            }
        }
    }
    if (a.S_fin) {
        if (isz) *(f32x4*)(a.z_fin + bh * a.fin_zstride + ef) = carry;
        else *(f32x4*)(a.S_fin + bh * a.fin_stride + ef) = carry;
    }
}

// Work items of packed sequences (one workgroup): each thread counts the
// segments of its sequences, a workgroup-wide exclusive scan gives their
// first item, and the items are written in order; the rest of the table is -1.
constexpr int kItemThreads = 1024;

__global__ void __launch_bounds__(kItemThreads) la_varlen_items_kernel(const int32_t* cu, int B, int64_t N, int C,
                                                                      int64_t cps, int P, int G, int32_t* items)
{
    __shared__ int part[kItemThreads];
    __shared__ int carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    for (int w = tid; w < G; w += kItemThreads) items[w] = -1;
    __syncthreads();
    for (int b0 = 0; b0 < B; b0 += kItemThreads) {
        const int b = b0 + tid;
        int cnt = 0;
        if (b < B) {
            int64_t s0, s1;
            varlen_range(cu, b, N, &s0, &s1);
            const int64_t k = ((s1 - s0 + C - 1) / C + cps - 1) / cps;
            cnt = (int)max((int64_t)1, min(k, (int64_t)P));
        }
        // inclusive scan over the workgroup (Hillis-Steele in LDS)
        part[tid] = cnt;
        __syncthreads();
        for (int o = 1; o < kItemThreads; o <<= 1) {
            const int t = tid >= o ? part[tid - o] : 0;
            __syncthreads();
            part[tid] += t;
            __syncthreads();
        }
        const int first = carry + part[tid] - cnt;
        for (int s = 0; s < cnt; ++s)
            if (first + s < G) items[first + s] = b * P + s;
        __syncthreads();
        if (tid == kItemThreads - 1) carry += part[tid];
        __syncthreads();
    }
}

hipError_t launch_varlen_items(const int32_t* cu, int B, int64_t N, int C, int64_t cps, int P, int G,
                               int32_t* items, hipStream_t stream)
{
    return launch_kernel(la_varlen_items_kernel, dim3(1), dim3(kItemThreads), stream, cu, B, N, C, cps, P, G, items);
}

// Lambda gradient, per (batch, head) row: the dq sweep's partials, plus
// sum_s <T_in(s), W_loc(s)> with T_in(0) = 0 and T_in(s+1) = lambda^(L_s)
// T_in(s) + dT(s) (the segments' own dT, their start state held fixed), plus
// <[dS_out | dz_out], T_in(P)> -- the terms through which each segment's start
// state and the final state depend on lambda.  Like the scan, each thread owns
// four elements of a row's [F x (d_v + 1)] state and walks the segments with
// kScanBatch loads in flight; each workgroup writes one partial sum
// (deterministic: no atomics), and the per-head kernel adds them up.
__global__ void __launch_bounds__(kScanThreads) la_dlam_rows_kernel(const DlamArgs a)
{
    const int FD = a.F * a.DV, SZ = FD + a.F;
    const int e = 4 * (blockIdx.x * kScanThreads + threadIdx.x);
    const int bh = blockIdx.y;
    const float l2l = a.lam.log2lam[bh % a.H];
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc = zero;
    if (e < SZ) {
        f32x4 t = zero;
        f32x4 w[kScanBatch], d[kScanBatch];
        for (int s0 = 0; s0 < a.P; s0 += kScanBatch) {
#pragma unroll
            for (int b = 0; b < kScanBatch; ++b) {
                const int64_t slot = (int64_t)(s0 + b) * a.BH + bh;
                const bool in = s0 + b < a.P;
                d[b] = in ? *(const f32x4*)(a.tseg + slot * SZ + e) : zero;
                w[b] = (in && a.wloc) ? *(const f32x4*)(a.wloc + slot * SZ + e) : zero;
            }
#pragma unroll
            for (int b = 0; b < kScanBatch; ++b) {
                const int s = s0 + b;
                if (s < a.P) {
                    acc += t * w[b];  // T_in(0) = 0, so segment 0 adds nothing
                    const int64_t L = (s == a.P - 1 ? a.n_len : min((int64_t)(s + 1) * a.seg_len, a.n_len)) -
                                      (int64_t)s * a.seg_len;
                    t = lam_pow(l2l, (int)L) * t + d[b];
                }
            }
        }
        if (a.dS_out) {
            const bool isz = e >= FD;
            const f32x4 g = isz ? *(const f32x4*)(a.dz_out + (int64_t)bh * a.F + (e - FD))
                                : *(const f32x4*)(a.dS_out + (int64_t)bh * FD + e);
            acc += t * g;
        }
    }
    float part = acc[0] + acc[1] + acc[2] + acc[3];
    __shared__ float red[kScanThreads / 64];
    part = wave_sum_xor(part, 1, 32);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
    __syncthreads();
    if (threadIdx.x == 0) {
        float sum = 0.f;
        for (int w2 = 0; w2 < kScanThreads / 64; ++w2) sum += red[w2];
        if (blockIdx.x == 0)
            for (int s = 0; s < a.P; ++s) sum += a.dlp[(int64_t)s * a.BH + bh];
        a.rows[(int64_t)bh * gridDim.x + blockIdx.x] = sum;
    }
}

// dlambda[h] = sum over the batch of the rows' partial sums
__global__ void __launch_bounds__(256) la_dlam_heads_kernel(const DlamArgs a, int nblk)
{
    const int h = blockIdx.x * 256 + threadIdx.x;
    if (h >= a.H) return;
    float sum = 0.f;
    for (int b = 0; b < a.BH / a.H; ++b)
        for (int k = 0; k < nblk; ++k) sum += a.rows[(int64_t)(b * a.H + h) * nblk + k];
    a.dlam[h] = sum;
}

int dlam_blocks(int F, int DV)
{
    const int SZ4 = (F * DV + F) / 4;
    return (SZ4 + kScanThreads - 1) / kScanThreads;
}

hipError_t launch_dlam(const DlamArgs& a, hipStream_t stream)
{
    const int nblk = dlam_blocks(a.F, a.DV);
    hipError_t e = launch_kernel(la_dlam_rows_kernel, dim3(nblk, a.BH), dim3(kScanThreads), stream, a);
    if (e != hipSuccess) return e;
    return launch_kernel(la_dlam_heads_kernel, dim3((a.H + 255) / 256), dim3(256), stream, a, nblk);
}

__global__ void __launch_bounds__(256) la_fill_zero_kernel(float* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// dst[0..n) = src[0..n): 16-byte accesses, eight in flight per thread
// (pointers are 16-byte aligned; a scalar loop finishes a ragged tail).
__global__ void __launch_bounds__(256) la_copy_kernel(float* dst, const float* src, int64_t n)
{
    constexpr int U = 8;
    const int64_t n4 = n / 4;
    const f32x4* s4 = (const f32x4*)src;
    f32x4* d4 = (f32x4*)dst;
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + (U - 1) * stride < n4; i += U * stride) {
        f32x4 t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) t[u] = s4[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) d4[i + u * stride] = t[u];
    }
    for (; i < n4; i += stride) d4[i] = s4[i];
    for (int64_t t = 4 * n4 + (int64_t)blockIdx.x * 256 + threadIdx.x; t < n; t += stride) dst[t] = src[t];
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream)
{
    const int SZ4 = (a.F * a.DV + a.F) / 4;
    return launch_kernel(la_scan_kernel, dim3((SZ4 + kScanThreads - 1) / kScanThreads, a.BH), dim3(kScanThreads),
                         stream, a);
}

static unsigned grid_for(int64_t n)
{
    int64_t b = (n + 255) / 256;
    if (b > 4096) b = 4096;
    if (b < 1) b = 1;
    return (unsigned)b;
}

// S = alpha * I per head-state (rectangular identity) and z = alpha on the
// first min(F, DV) features; grid-stride over both buffers.
__global__ void __launch_bounds__(256) la_fill_identity_kernel(float* S, float* z, int64_t BH, int F, int DV,
                                                              float alpha)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t nS = S ? BH * F * (int64_t)DV : 0, nz = z ? BH * F : 0;
    const int fz = F < DV ? F : DV;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nS; i += stride) {
        const int64_t e = i % ((int64_t)F * DV);
        S[i] = (e / DV == e % DV) ? alpha : 0.f;
    }
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nz; i += stride)
        z[i] = (i % F < fz) ? alpha : 0.f;
}

hipError_t launch_fill_identity(float* S, float* z, int64_t BH, int F, int DV, float alpha, hipStream_t stream)
{
    const int64_t nS = S ? BH * F * (int64_t)DV : 0, nz = z ? BH * F : 0;
    const int64_t n = nS > nz ? nS : nz;
    if (n <= 0) return hipSuccess;
    return launch_kernel(la_fill_identity_kernel, dim3(grid_for(n)), dim3(256), stream, S, z, BH, F, DV, alpha);
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    return launch_kernel(la_fill_zero_kernel, dim3(grid_for(n)), dim3(256), stream, p, n);
}

hipError_t launch_copy(float* dst, const float* src, int64_t n, hipStream_t stream)
{
    if (n <= 0 || dst == src) return hipSuccess;
    int64_t b = (n / 4 + 2047) / 2048;  // about eight 16-byte vectors per thread
    if (b > 16384) b = 16384;
    if (b < 1) b = 1;
    return launch_kernel(la_copy_kernel, dim3((unsigned)b), dim3(256), stream, dst, src, n);
}

}  // namespace la
