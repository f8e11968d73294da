// la_decode.h -- recurrent decode steps (gfx950): ntok tokens per (batch,
// head) in order, the fp32 state read once, kept in registers across the
// tokens, and written once.
//
// Per head-state ("From standard attention to linear attention",
// tqpw.cn/news/561043, sec. 6 autoregressive step; decay from "Attention is
// also an FFN", kwkr.cn/news/587576, sec. 3.2; normaliser sec. 4.2):
//   S <- lambda S + phi(k) v^T,  z <- lambda z + phi(k),
//   y  = phi(q)^T S / (phi(q)^T z + eps)          (update, then query)
//
// A step is bound by HBM: 8 bytes of state traffic per state element against
// 4 flops, so a call takes ntok tokens per head-state and reads and writes
// the state once for all of them (the fused multi-token decode).  The value
// columns of a head-state may be split over DS workgroups of 256 threads (see
// decode_split).  Each thread owns a 4-column quad of F/RG rows, issues all of
// its 16-byte loads before the first use so that many bytes are in flight,
// and keeps them in registers across the tokens.  Per token it updates them
// and accumulates phi(q)^T S for its columns; partial sums over rows are
// reduced across lanes and then across waves through LDS.  Every workgroup
// recomputes the new z for its denominator; the first column slice writes it
// back.

#pragma once

#include "la_device.h"
#include "la_internal.h"

namespace la {

// Column slices per head-state.  Two 32 KB slices per d_v = 128 head-state
// measured slower than one 64 KB workgroup (the per-workgroup feature map and
// reductions are paid twice), so every head-state is one workgroup.
template <int DV>
constexpr int decode_split() { return 1; }

template <class T, int PHI, int DK, int F, int DV, bool SCALED>
__global__ void __launch_bounds__(256)
la_decode_kernel(const DecArgs a)
{
    constexpr int NT = 256;
    constexpr bool RF = PHI == LA_PHI_TRIG_RF;
    constexpr int M = RF ? F / 2 : 0;
    constexpr int DS = decode_split<DV>();
    constexpr int DW = DV / DS;     // value columns of this workgroup
    constexpr int CQ = DW / 4;      // column quads
    constexpr int RG = NT / CQ;     // row groups
    constexpr int RPT = F / RG;     // rows per thread
    static_assert(F <= NT && DV <= NT && F % RG == 0 && NT % CQ == 0, "decode thread mapping");

    __shared__ float sPq[F], sPk[F], sV[DW];
    __shared__ float sX[RF ? 2 * DK : 1];
    __shared__ f32x4 sRed[NT / 64][CQ];
    __shared__ float sDen[NT / 64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int blk = (int)blockIdx.x;
    const int bh = blk / DS, part = blk % DS, h = bh % a.H;
    const int d0 = part * DW;
    const float lam = a.lam.lam[h];
    float* Sb = a.S + (int64_t)bh * F * DV + d0;
    float* zb = a.z + (int64_t)bh * F;

    const int cq = tid % CQ, rg = tid / CQ;
    // issue the state loads first: they are the whole cost of a step
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = *(const f32x4*)(Sb + (rg + RG * i) * DV + 4 * cq);
    float zf = (tid < F) ? zb[tid] : 0.f;

    // SCALED (several tokens per call, every lambda >= 2^-12): within blocks
    // of at most kDecBlock tokens the registers hold s' = lambda^-e S (e
    // tokens into the block), so that a token costs one fused multiply-add
    // per state element for the update (s' += lambda^-e phi(k) v^T) and one
    // for the query (phi(q)^T S = lambda^e phi(q)^T s'); s' returns to S at
    // the block's end.  lambda^-e stays below 2^96.  Otherwise the plain
    // update S <- lambda S + phi(k) v^T.
    constexpr int kDecBlock = 8;
    const float ilam = SCALED ? 1.0f / lam : 1.f;
    float g = 1.f, pe = 1.f;  // lambda^-e and lambda^e of the current token
    int e_blk = 0;

    for (int t = 0; t < a.ntok; ++t) {
        const int64_t row = (int64_t)bh * a.ntok + t;
        const T* q = (const T*)a.q + row * DK;
        const T* k = (const T*)a.k + row * DK;
        const T* v = (const T*)a.v + row * DV;
        // the previous token's reductions are done before its LDS is reused
        if (t > 0) __syncthreads();

        // feature maps of this token
        if constexpr (RF) {
            if (tid < DK) {
                sX[tid] = to_f32(q[tid]);
                sX[DK + tid] = to_f32(k[tid]);
            }
            if (tid < DW) sV[tid] = to_f32(v[d0 + tid]);
            __syncthreads();
            if (tid < 2 * M) {
                const int which = tid / M, r = tid % M;
                const float* x = sX + which * DK;
                const float* om = a.omega + (int64_t)r * DK;
                float u = 0.f, n2 = 0.f;
                for (int d = 0; d < DK; ++d) {
                    u += om[d] * x[d];
                    n2 += x[d] * x[d];
                }
                const float qs = a.qk_scale;
                const float c = exp_rf<T>(a.rf_sign * 0.5f * qs * qs * n2) * rsqrtf((float)M);
                float sn, cs;
                sincos_rf<T>(qs * u, &sn, &cs);
                float* dst = which ? sPk : sPq;
                dst[r] = c * cs;
                dst[M + r] = c * sn;
            }
        } else {
            if (tid < DK) {
                sPq[tid] = phi_elem<T, PHI>(to_f32(q[tid]));
                sPk[tid] = phi_elem<T, PHI>(to_f32(k[tid]));
            }
            if (tid < DW) sV[tid] = to_f32(v[d0 + tid]);
        }
        __syncthreads();

        // S <- lambda S + phi(k) v^T ; partial phi(q)^T S
        const f32x4 v4 = {sV[4 * cq], sV[4 * cq + 1], sV[4 * cq + 2], sV[4 * cq + 3]};
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float dz = 0.f;
        if constexpr (SCALED) {
            ++e_blk;
            g *= ilam;
            pe *= lam;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int f = rg + RG * i;
                s[i] += (g * sPk[f]) * v4;
                acc += sPq[f] * s[i];
            }
            // z the same way ; partial phi(q)^T z
            if (tid < F) {
                zf += g * sPk[tid];
                dz = sPq[tid] * zf;
            }
        } else {
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int f = rg + RG * i;
                s[i] = lam * s[i] + sPk[f] * v4;
                acc += sPq[f] * s[i];
            }
            // z <- lambda z + phi(k) ; partial phi(q)^T z
            if (tid < F) {
                zf = lam * zf + sPk[tid];
                dz = sPq[tid] * zf;
            }
        }
        // reduce over row groups: lanes of one wave first, then waves
#pragma unroll
        for (int m = CQ; m < 64; m <<= 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], m, 64);
        }
        dz = wave_sum_xor(dz, 1, 32);
        if (lane < CQ) sRed[wave][lane] = acc;
        if (lane == 0) sDen[wave] = dz;
        __syncthreads();
        if (tid < CQ) {
            f32x4 num = {0.f, 0.f, 0.f, 0.f};
            float den = 0.f;
#pragma unroll
            for (int w = 0; w < NT / 64; ++w) {
                num += sRed[w][tid];
                den += sDen[w];
            }
            num *= pe;  // 1 unless SCALED
            den *= pe;
            const float inv = 1.0f / (den + a.eps);
            const int64_t yo = row * DV + d0 + 4 * tid;
            if (a.out_f32) {
                *(f32x4*)((float*)a.y + yo) = num * inv;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) ((T*)a.y)[yo + e] = from_f32<T>(num[e] * inv);
            }
        }
        // end of a scaled block: s' back to S
        if (SCALED && (e_blk == kDecBlock || t == a.ntok - 1)) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) s[i] *= pe;
            zf *= pe;
            e_blk = 0;
            g = pe = 1.f;
        }
    }

    // the state after the last token, written once
#pragma unroll
    for (int i = 0; i < RPT; ++i) *(f32x4*)(Sb + (rg + RG * i) * DV + 4 * cq) = s[i];
    if (tid < F && part == 0) zb[tid] = zf;
}

template <class T, int PHI, int DK, int F, int DV>
hipError_t dec_launch(const DecArgs& a, hipStream_t stream)
{
    const unsigned blocks = (unsigned)a.BH * (unsigned)decode_split<DV>();
    bool scaled = a.ntok > 1;
    for (int h = 0; h < a.H && scaled; ++h) scaled = a.lam.lam[h] >= 0x1p-12f;
    if (scaled) return launch_kernel(la_decode_kernel<T, PHI, DK, F, DV, true>, dim3(blocks), dim3(256), stream, a);
    return launch_kernel(la_decode_kernel<T, PHI, DK, F, DV, false>, dim3(blocks), dim3(256), stream, a);
}

}  // namespace la
