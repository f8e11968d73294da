// la_backward.h -- backward passes (gfx950) of the chunked causal forward for
// the elementwise feature maps (elu+1, ReLU), templated on element type and
// head sizes.  Instantiated by la_inst_bwd.hip.
//
// Gradients of y_i = phi(q_i)^T S_i / (phi(q_i)^T z_i + eps) with the decayed
// state of "Attention is also an FFN" (kwkr.cn/news/587576) sec. 3.2 and 4.2,
// whose chunked evaluation (sec. 4.1 notes and 5.2) the forward kernel uses.
// With dnum_i = g_i / den_i and dden_i = -(g_i . y_i) / den_i (g = dL/dy):
//
//   d phi(q_i) = S_i dnum_i + z_i dden_i
//              = lambda^(i+1) [S, z]_prev [dnum_i; dden_i]
//              + sum_{j<=i} lambda^(i-j) (dnum_i . v_j + dden_i) phi(k_j)
//   with the adjoint U_j = sum_{i>=j} lambda^(i-j) phi(q_i) dnum_i^T (u: dden)
//   d phi(k_j) = U_j v_j + u_j,   dv_j = U_j^T phi(k_j).
//
// The adjoint is carried between chunks as W = lambda U at the next chunk's
// first token (at the end of the sequence W is the final state's gradient,
// which enters the last token with weight 1).  For a chunk of n tokens,
//   U_j   = lambda^(n-1-j) W + sum_{i>=j in chunk} lambda^(i-j) phi(q_i) dnum_i^T
//   W    <- lambda^n W + sum_i lambda^(i+1) phi(q_i) dnum_i^T,
// and after the first chunk W is the initial state's gradient lambda U_0.
//
// so the backward is two more chunked linear-attention sweeps over the same
// tiles: one in token order carrying the forward state (dq), one in reverse
// order carrying the adjoint (dk, dv).  The score tiles
//   A_ij = phi(q_i) . phi(k_j)   and   B_ij = dnum_i . v_j + dden_i
// (decayed, i >= j) are formed per chunk on the matrix cores, as in the
// forward.  Segments of a long row run in parallel as in the forward: the dq
// sweep reads the forward state at its segment's start (forward segment pass
// + scan), the kv sweep the adjoint at its segment's end (reverse-local pass
// + reverse scan).
//
// Work split (4 waves): the carried state [F x d_v] is split over the waves by
// value columns (as in the forward); each chunk it is also published to LDS
// in the element type, so that products contracting over d_v (d phi(q) from
// S, d phi(k) from U) can read its rows.  Every wave computes the chunk's
// score tiles itself; outputs are split over the waves by feature blocks
// (dq, dk) or value blocks (dv).  The state is multiplied by lambda^n once a
// chunk (no deferred scale: lambda <= 1, so nothing overflows).
//
// The non-causal form (cross attention: N queries against M keys, "From
// standard attention to linear attention" sec. 2, 3 and 6) holds one state
// S = sum_j phi(k_j) v_j^T, z = sum_j phi(k_j) for every query, so both sweeps
// lose their score tiles and their carries: the query sweep reads the total
// state (d phi(q_i) = S dnum_i + z dden_i) and sums the adjoint
// U = sum_i phi(q_i) dnum_i^T, u = sum_i phi(q_i) dden_i over its segment;
// the key sweep reads the total adjoint (d phi(k_j) = U v_j + u,
// dv_j = U^T phi(k_j)).
//
// The feature maps' derivatives come from the staged features themselves:
// elu+1: phi'(x) = 1 for x > 0 and e^x = phi(x) otherwise, i.e. min(phi(x), 1);
// ReLU: phi'(x) = [phi(x) > 0].
#pragma once

#include <type_traits>

#include "la_device.h"
#include "la_internal.h"

namespace la {

#define LA_BINLINE __attribute__((always_inline))

// Fragment with slot e scaled by lo[e] (slots 0..3) and hi[e-4] (slots 4..7):
// a per-k weight on an operand (the k positions of the slots are K(g)).
template <class T> __device__ __forceinline__ Frag<T> frag_scale(const Frag<T>& f, const f32x4& lo, const f32x4& hi);
template <> __device__ __forceinline__ Frag<bf16> frag_scale<bf16>(const Frag<bf16>& f, const f32x4& lo, const f32x4& hi) {
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = (float)f.v[e] * lo[e];
        b[e] = (float)f.v[4 + e] * hi[e];
    }
    return frag_acc<bf16>(a, b);
}
template <> __device__ __forceinline__ Frag<float> frag_scale<float>(const Frag<float>& f, const f32x4& lo, const f32x4& hi) {
    Frag<float> r;
    r.lo = f.lo * lo;
    r.hi = f.hi * hi;
    return r;
}

// Four consecutive elements (one 8- or 16-byte LDS read) as floats.
__device__ __forceinline__ f32x4 ld4f(const bf16* p) {
    const bf16x4 v = ld4(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 ld4f(const float* p) { return ld4(p); }

template <class T, int PHI> __device__ __forceinline__ float phi_deriv_from_phi(float p) {
    if constexpr (PHI == LA_PHI_RELU) return p > 0.f ? 1.f : 0.f;
    else if constexpr (PHI == kPhiIdentity) return 1.f;
    else return p < 1.f ? p : 1.f;
}

// This wave's FBW blocks of a per-feature-block register array (blocks
// wave * FBW + u), read with compile-time indices: a compare over the waves
// replaces the run-time index, which for 16 blocks (F = 256) moved the whole
// array to scratch memory.  Smaller arrays keep the run-time index (the
// copies would cost registers, and occupancy, there).
template <int NW, int FBW, int N>
__device__ __forceinline__ void wave_blocks(const f32x4 (&src)[N], int wave, f32x4 (&dst)[FBW]) {
#pragma unroll
    for (int u = 0; u < FBW; ++u) {
        dst[u] = src[u];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            if (w * FBW + u < N && wave == w) dst[u] = src[(w * FBW + u) % N];
    }
}

// dq / dk rows in the input type (for the identity map these are d phi,
// which the random-feature backward maps through omega afterwards)
template <class T, int PHI>
__device__ __forceinline__ void store_grad(void* base, int64_t off, const float* o) {
    st4((T*)base + off, o[0], o[1], o[2], o[3]);
}

template <class T, int DK, int F, int DV, int C, int NW, int MODE, bool DL = false>
struct BwdCfg {
    static constexpr int NT = NW * 64;
    static constexpr int VEC = 16 / (int)sizeof(T);
    static constexpr int QB = C / 16;
    static constexpr int CB = C / 32;
    static constexpr int FB = F / 16;
    static constexpr int DB = DV / 16;
    static constexpr int DBW = DB / NW;  // value blocks per wave (state columns, dv)
    static constexpr int FBW = FB / NW;  // feature blocks per wave (dq, dk)
    static constexpr int TQ = C * TileL<T, F>::STRIDE;
    static constexpr int TV = C * TileL<T, DV>::STRIDE;
    static constexpr int TS = F * TileL<T, DV>::STRIDE;  // published state
    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    // dq: Q, K (feature tiles), V, G, Y (value tiles), S
    // kv: Q, Qw, K (feature tiles), V, DN (value tiles), U; dden [C]
    static constexpr bool KV = MODE != BMODE_Q;
    static constexpr bool RL = MODE == BMODE_RLOCAL;
    static constexpr size_t OFF_F0 = 0;                                   // phi(Q)
    static constexpr size_t OFF_F1 = al(OFF_F0 + size_t(TQ) * sizeof(T)); // phi(K) (dq) / lambda-weighted phi(Q) (kv)
    static constexpr size_t OFF_F2 = al(OFF_F1 + size_t(TQ) * sizeof(T)); // phi(K) (kv only)
    static constexpr size_t OFF_V0 = al(OFF_F2 + (KV ? size_t(TQ) * sizeof(T) : 0)); // V
    static constexpr size_t OFF_V1 = al(OFF_V0 + size_t(TV) * sizeof(T)); // G (dq) / dnum (kv)
    static constexpr size_t OFF_V2 = al(OFF_V1 + size_t(TV) * sizeof(T)); // Y (dq only)
    static constexpr size_t OFF_S = al(OFF_V2 + (KV ? 0 : size_t(TV) * sizeof(T)));  // published state
    static constexpr size_t OFF_T = al(OFF_S + size_t(TS) * sizeof(T));   // published dS/dlambda (DL)
    static constexpr size_t OFF_R = al(OFF_T + (DL ? size_t(TS) * sizeof(T) : 0));  // per-token scalars
    static constexpr size_t TOTAL = al(OFF_R + size_t(C) * sizeof(float));

    static_assert(C == 32, "one 32-token block per chunk");
    static_assert((C * (DK / VEC)) % NT == 0 && (C * (DV / VEC)) % NT == 0, "tile rows split evenly over the threads");
    static_assert(DK == F, "elementwise feature maps");
    static_assert(DBW >= 1 && FBW >= 1 && DB % NW == 0 && FB % NW == 0, "blocks must split over the waves");
    static_assert(DL || TOTAL <= 160 * 1024, "LDS budget");
};

// Whether the lambda-gradient variant of the dq sweep fits in LDS.
template <class T, int DK, int F, int DV>
constexpr bool bwd_dlam_fits() { return BwdCfg<T, DK, F, DV, 32, 4, BMODE_Q, true>::TOTAL <= 160 * 1024; }

// ---------------------------------------------------------------------------
// dq sweep (token order).
// DL: also the lambda gradient.  T = d[S|z]/dlambda is carried beside the
// state (zero at the segment's start, whose state is held fixed; the
// segments are joined by the reduction kernel).  Per chunk of n tokens:
//   dlambda += sum_i [ lambda^(i+1) phi(q_i).(T dnum_i + t dden_i)
//                    + (i+1) lambda^i phi(q_i).(S dnum_i + z dden_i) ]
//            + sum_{j<=i} (i-j) lambda^(i-j-1) A_ij B_ij
//   T <- lambda^n T + n lambda^(n-1) S + sum_j (n-1-j) lambda^(n-2-j) phi(k_j) [v_j, 1]^T
// (the product rule on the chunk's recurrence, with S, T before the chunk).
// NC: the non-causal form -- the state read at S_src is the total for every
// query (no score tiles, no carry), and the adjoint sums
// sum_i phi(q_i) [dnum_i, dden_i]^T over the segment go to S_dst / z_dst at
// (seg*BH + bh)*dst_stride.
template <class T, int PHI, int DK, int F, int DV, int C, int NW, bool DL, bool NC = false>
__global__ void __launch_bounds__(NW * 64, 1) la_bwd_q_kernel(const BwdArgs a)
{
    static_assert(!(DL && NC), "no decay in the non-causal form");
    using Cfg = BwdCfg<T, DK, F, DV, C, NW, BMODE_Q, DL>;
    using TF = TileL<T, F>;
    using TVL = TileL<T, DV>;
    constexpr int NT = Cfg::NT, VEC = Cfg::VEC, QB = Cfg::QB, CB = Cfg::CB, FB = Cfg::FB;
    constexpr int DBW = Cfg::DBW, FBW = Cfg::FBW;
    constexpr int KB = F / 32, VB = DV / 32;
    constexpr int VPRQ = DK / VEC, VPRV = DV / VEC;
    constexpr int RQ = (C * VPRQ + NT - 1) / NT, RV = (C * VPRV + NT - 1) / NT;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    T* const sQ = (T*)(smem + Cfg::OFF_F0);
    T* const sK = (T*)(smem + Cfg::OFF_F1);
    T* const sV = (T*)(smem + Cfg::OFF_V0);
    T* const sG = (T*)(smem + Cfg::OFF_V1);
    T* const sY = (T*)(smem + Cfg::OFF_V2);
    T* const sS = (T*)(smem + Cfg::OFF_S);
    T* const sT = (T*)(smem + Cfg::OFF_T);
    T* const sDN = sV;  // NC: dnum rows (no values are staged)
    float* const sDD = (float*)(smem + Cfg::OFF_R);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int seg = blockIdx.x, bh = blockIdx.y, h = bh % a.H;
    const float l2l = NC ? 0.f : a.lam.log2lam[h];
    const int64_t nch = (a.N + C - 1) / C;
    const int64_t c_beg = (int64_t)seg * a.cps, c_end = (seg == a.P - 1) ? nch : min(nch, c_beg + a.cps);
    const int64_t row0 = (int64_t)bh * a.N;
    const T* qg = (const T*)a.q + row0 * DK;
    const T* kg = (const T*)a.k + row0 * DK;
    const T* vg = (const T*)a.v + row0 * DV;
    const T* yg = (const T*)a.y + row0 * DV;
    const T* gg = (const T*)a.gy + row0 * DV;
    const uint8_t* kp = a.kpm ? a.kpm + (int64_t)(bh / a.H) * a.N : nullptr;
    const Frag<T> ones = frag_ones<T>();

    // decay of score element (j = 16 jb + 4 g + r, i = 16 ib + l16), i >= j
    float m0[4], m1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = l16 - 4 * g - r;
        m0[r] = e < 0 ? 0.f : lam_pow(l2l, e);
        m1[r] = lam_pow(l2l, 16 + e);
    }

    // carried forward state: S tiles (all f, this wave's value columns), z (all f)
    f32x4 accS[FB][DBW], accZ[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
        accZ[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < DBW; ++t) accS[fb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (a.S_src) {
        const float* Sb = a.S_src + (int64_t)seg * a.src_seg_stride + (int64_t)bh * a.src_stride;
        const float* zb = a.z_src + (int64_t)seg * a.src_seg_stride + (int64_t)bh * a.src_zstride;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
            for (int t = 0; t < DBW; ++t) {
                const int d = 16 * (wave * DBW + t) + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) accS[fb][t][r] = Sb[(16 * fb + 4 * g + r) * DV + d];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) accZ[fb][r] = zb[16 * fb + 4 * g + r];
        }
    }
    // dS/dlambda and dz/dlambda (DL), from zero at the segment's start
    constexpr int TF1 = DL ? FB : 1, TD1 = DL ? DBW : 1;
    f32x4 accT[TF1][TD1], accTz[TF1];
#pragma unroll
    for (int fb = 0; fb < TF1; ++fb) {
        accTz[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < TD1; ++t) accT[fb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float dl = 0.f;  // this lane's share of the segment's lambda gradient
    // publish S (element type, row-major [F][DV]) for reads that contract over d
    auto publish = [&]() LA_BINLINE {
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int t = 0; t < DBW; ++t) {
                const int d = 16 * (wave * DBW + t) + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int f = 16 * fb + 4 * g + r;
                    sS[TVL::off(f, d & ~3) + (d & 3)] = from_f32<T>(accS[fb][t][r]);
                    if constexpr (DL) sT[TVL::off(f, d & ~3) + (d & 3)] = from_f32<T>(accT[fb][t][r]);
                }
            }
    };

    // NC: the total state is published once; its registers then sum the adjoint
    f32x4 accu[NC ? FB : 1];
#pragma unroll
    for (int fb = 0; fb < (NC ? FB : 1); ++fb) accu[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (NC) {
        publish();
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int t = 0; t < DBW; ++t) accS[fb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    uint4 rq[RQ], rk[RQ], rv[RV], rg[RV], ry[RV];
    int mk[RQ];
    for (int64_t c = c_beg; c < c_end; ++c) {
        const int64_t t0 = c * C;
        const int n = (int)min((int64_t)C, a.N - t0);
        // ---- loads (rows past the end re-read the last row; zeroed below)
#pragma unroll
        for (int r = 0; r < RQ; ++r) {
            const int idx = tid + r * NT, j = min(idx / VPRQ, n - 1), c4 = idx % VPRQ;
            rq[r] = *(const uint4*)(qg + (t0 + j) * DK + c4 * VEC);
            if constexpr (!NC) {
                rk[r] = *(const uint4*)(kg + (t0 + j) * DK + c4 * VEC);
                mk[r] = kp ? (int)kp[t0 + j] : 0;
            }
        }
#pragma unroll
        for (int r = 0; r < RV; ++r) {
            const int idx = tid + r * NT, j = min(idx / VPRV, n - 1), c4 = idx % VPRV;
            if constexpr (!NC) rv[r] = *(const uint4*)(vg + (t0 + j) * DV + c4 * VEC);
            rg[r] = *(const uint4*)(gg + (t0 + j) * DV + c4 * VEC);
            ry[r] = *(const uint4*)(yg + (t0 + j) * DV + c4 * VEC);
        }
        // ---- publish the state and stage the chunk (the previous chunk's
        // reads of both ended at its closing barrier)
        if constexpr (!NC) publish();
#pragma unroll
        for (int r = 0; r < RQ; ++r) {
            const int idx = tid + r * NT, j = idx / VPRQ, cg = idx % VPRQ;
            float xq[VEC], pq[VEC];
            unpack16(rq[r], xq, (const T*)nullptr);
#pragma unroll
            for (int e = 0; e < VEC; ++e) pq[e] = j < n ? phi_elem<T, PHI>(xq[e]) : 0.f;
#pragma unroll
            for (int e = 0; e < VEC; e += 4) st4(sQ + TF::off(j, cg * VEC + e), pq[e], pq[e + 1], pq[e + 2], pq[e + 3]);
            if constexpr (!NC) {
                float xk[VEC], pk[VEC];
                unpack16(rk[r], xk, (const T*)nullptr);
                const bool dead = j >= n || mk[r];
#pragma unroll
                for (int e = 0; e < VEC; ++e) pk[e] = dead ? 0.f : phi_elem<T, PHI>(xk[e]);
#pragma unroll
                for (int e = 0; e < VEC; e += 4) st4(sK + TF::off(j, cg * VEC + e), pk[e], pk[e + 1], pk[e + 2], pk[e + 3]);
            }
        }
#pragma unroll
        for (int r = 0; r < RV; ++r) {
            const int idx = tid + r * NT, j = idx / VPRV, cg = idx % VPRV;
            float xv[VEC], xg[VEC], xy[VEC];
            if constexpr (!NC) unpack16(rv[r], xv, (const T*)nullptr);
            unpack16(rg[r], xg, (const T*)nullptr);
            unpack16(ry[r], xy, (const T*)nullptr);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                if (j >= n) {
                    xv[e] = 0.f;
                    xg[e] = 0.f;
                    xy[e] = 0.f;
                }
            }
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                if constexpr (!NC) st4(sV + TVL::off(j, cg * VEC + e), xv[e], xv[e + 1], xv[e + 2], xv[e + 3]);
                st4(sG + TVL::off(j, cg * VEC + e), xg[e], xg[e + 1], xg[e + 2], xg[e + 3]);
                st4(sY + TVL::off(j, cg * VEC + e), xy[e], xy[e + 1], xy[e + 2], xy[e + 3]);
            }
        }
        __syncthreads();

        // ---- per 16-token query block: den, dnum, dden, B scores, d phi(q)
        Frag<T> zf[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) zf[kb] = frag_acc<T>(accZ[2 * kb], accZ[2 * kb + 1]);
        // this wave's z (and dz/dlambda) tiles for d phi(q)
        constexpr bool WCOPY = FB >= 16;
        f32x4 zw[WCOPY ? FBW : 1], tzw[(WCOPY && DL) ? FBW : 1];
        if constexpr (WCOPY) {
            wave_blocks<NW, FBW>(accZ, wave, zw);
            if constexpr (DL) wave_blocks<NW, FBW>(accTz, wave, tzw);
        }
#pragma unroll
        for (int ib = 0; ib < QB; ++ib) {
            const int i = 16 * ib + l16;
            const float lqi = lam_pow(l2l, i + 1);
            Frag<T> qf[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) qf[kb] = lds_frag_row<T, F>(sQ, i, kb, g);
            f32x4 dz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) mma(dz, zf[kb], qf[kb]);
            // A^T tiles (rows j, column i) for the normaliser
            f32x4 pt[2 * CB], praw[DL ? 2 * CB : 1];
#pragma unroll
            for (int jb = 0; jb < 2 * CB; ++jb) {
                pt[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (!NC && jb <= ib) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) mma(pt[jb], lds_frag_row<T, F>(sK, 16 * jb + l16, kb, g), qf[kb]);
                    if constexpr (DL) praw[jb] = pt[jb];
#pragma unroll
                    for (int r = 0; r < 4; ++r) pt[jb][r] *= (jb == ib) ? m0[r] : m1[r] * lam_pow(l2l, 16 * (ib - jb - 1));
                }
            }
            f32x4 rs = {0.f, 0.f, 0.f, 0.f};
            if constexpr (!NC) {
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) mma(rs, ones, frag_acc<T>(pt[2 * kb], pt[2 * kb + 1]));
            }
            const float den = rs[0] + lqi * dz[0] + a.eps;
            const float rden = fast_rcp(den);
            // dnum_i as B operand fragments (k = value column, n = token i),
            // and dden_i = -dnum_i . y_i from the same rounded dnum, so that
            // dnum_i . v_j + dden_i = dnum_i . (v_j - y_i) keeps the exact
            // cancellation of the weighted mean (the first token's dq is 0)
            Frag<T> dn[VB];
            float gy = 0.f;
#pragma unroll
            for (int kb = 0; kb < VB; ++kb) {
                const f32x4 g0 = ld4f(sG + TVL::off(i, 32 * kb + 4 * g));
                const f32x4 g1 = ld4f(sG + TVL::off(i, 32 * kb + 16 + 4 * g));
                const f32x4 y0 = ld4f(sY + TVL::off(i, 32 * kb + 4 * g));
                const f32x4 y1 = ld4f(sY + TVL::off(i, 32 * kb + 16 + 4 * g));
                f32x4 lo, hi;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo[e] = to_f32(from_f32<T>(g0[e] * rden));
                    hi[e] = to_f32(from_f32<T>(g1[e] * rden));
                    gy += lo[e] * y0[e] + hi[e] * y1[e];
                }
                dn[kb] = frag_acc<T>(lo, hi);
                if (NC && wave == 0) {
                    st4(sDN + TVL::off(i, 32 * kb + 4 * g), lo[0], lo[1], lo[2], lo[3]);
                    st4(sDN + TVL::off(i, 32 * kb + 16 + 4 * g), hi[0], hi[1], hi[2], hi[3]);
                }
            }
            gy += __shfl_xor(gy, 16, 64);
            gy += __shfl_xor(gy, 32, 64);
            const float dden = -gy;
            if (NC && wave == 0 && g == 0) sDD[i] = dden;
            // B^T tiles (rows j, column i): v_j . dnum_i + dden_i, decayed
            f32x4 bt[2 * CB];
#pragma unroll
            for (int jb = 0; jb < 2 * CB; ++jb) {
                bt[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (!NC && jb <= ib) {
#pragma unroll
                    for (int kb = 0; kb < VB; ++kb) mma(bt[jb], lds_frag_row<T, DV>(sV, 16 * jb + l16, kb, g), dn[kb]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float braw = bt[jb][r] + dden;
                        if constexpr (DL) {
                            // pairs inside the chunk: (i-j) lambda^(i-j-1) A_ij B_ij (one wave)
                            const int e = 16 * (ib - jb) + l16 - 4 * g - r;
                            if (wave == 0 && e >= 1) dl += (float)e * lam_pow(l2l, e - 1) * praw[jb][r] * braw;
                        }
                        bt[jb][r] = braw * ((jb == ib) ? m0[r] : m1[r] * lam_pow(l2l, 16 * (ib - jb - 1)));
                    }
                }
            }
            Frag<T> bf[CB];
#pragma unroll
            for (int kb = 0; kb < CB; ++kb) bf[kb] = frag_acc<T>(bt[2 * kb], bt[2 * kb + 1]);
            // d phi(q) for this wave's feature blocks (rows f, column i)
#pragma unroll
            for (int u = 0; u < FBW; ++u) {
                const int fb = wave * FBW + u;
                f32x4 inter = {0.f, 0.f, 0.f, 0.f}, intra = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < VB; ++kb) mma(inter, lds_frag_row<T, DV>(sS, 16 * fb + l16, kb, g), dn[kb]);
                if constexpr (!NC) {
#pragma unroll
                    for (int kb = 0; kb < CB; ++kb) mma(intra, ColRead<T, F>::get(sK, 32 * kb, 16 * fb, lane), bf[kb]);
                }
                if constexpr (DL) {
                    // phi(q_i).(S dnum_i + z dden_i) and phi(q_i).(T dnum_i + t dden_i) over
                    // this wave's feature rows (phi(q) = 0 past the chunk's end)
                    f32x4 tint = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < VB; ++kb) mma(tint, lds_frag_row<T, DV>(sT, 16 * fb + l16, kb, g), dn[kb]);
                    float rs_ = 0.f, rt_ = 0.f;
                    const f32x4 pq4 = ld4f(sQ + TF::off(i, 16 * fb + 4 * g));
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float p = pq4[r];
                        const float zr = WCOPY ? zw[WCOPY ? u : 0][r] : accZ[fb][r];
                        const float tr = WCOPY ? tzw[WCOPY ? u : 0][r] : accTz[fb][r];
                        rs_ += p * (inter[r] + zr * dden);
                        rt_ += p * (tint[r] + tr * dden);
                    }
                    dl += (float)(i + 1) * lam_pow(l2l, i) * rs_ + lqi * rt_;
                }
                if (i < n) {
                    const f32x4 ph = ld4f(sQ + TF::off(i, 16 * fb + 4 * g));
                    float o[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float zr = WCOPY ? zw[WCOPY ? u : 0][r] : accZ[fb][r];
                        const float dp = lqi * (inter[r] + zr * dden) + intra[r];
                        o[r] = dp * phi_deriv_from_phi<T, PHI>(ph[r]);
                    }
                    store_grad<T, PHI>(a.dq, (row0 + t0 + i) * DK + 16 * fb + 4 * g, o);
                }
            }
            if (!NC && wave == 0 && g == 0 && i < n) {
                float* tp = a.tok + (row0 + t0 + i) * 2;
                tp[0] = rden;
                tp[1] = dden;
            }
        }

        // ---- dS/dlambda carry (before S changes): T <- lambda^n T + n lambda^(n-1) S
        // + phi(K)^T (w' V), w'_j = (n-1-j) lambda^(n-2-j)
        if constexpr (DL) {
            const float ln_ = lam_pow(l2l, n), dn1 = (float)n * lam_pow(l2l, n - 1);
#pragma unroll
            for (int kb = 0; kb < CB; ++kb) {
                f32x4 wlo, whi;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j0 = 32 * kb + 4 * g + e, j1 = j0 + 16;
                    wlo[e] = j0 < n - 1 ? (float)(n - 1 - j0) * lam_pow(l2l, n - 2 - j0) : 0.f;
                    whi[e] = j1 < n - 1 ? (float)(n - 1 - j1) * lam_pow(l2l, n - 2 - j1) : 0.f;
                }
                const Frag<T> dwf = frag_acc<T>(wlo, whi);
                Frag<T> dwv[DBW];
#pragma unroll
                for (int t = 0; t < DBW; ++t)
                    dwv[t] = frag_scale<T>(ColRead<T, DV>::get(sV, 32 * kb, 16 * (wave * DBW + t), lane), wlo, whi);
#pragma unroll
                for (int fb = 0; fb < FB; ++fb) {
                    if (kb == 0) {
                        accTz[fb] = accTz[fb] * ln_ + accZ[fb] * dn1;
#pragma unroll
                        for (int t = 0; t < DBW; ++t) accT[fb][t] = accT[fb][t] * ln_ + accS[fb][t] * dn1;
                    }
                    const Frag<T> kf = ColRead<T, F>::get(sK, 32 * kb, 16 * fb, lane);
#pragma unroll
                    for (int t = 0; t < DBW; ++t) mma(accT[fb][t], kf, dwv[t]);
                    mma(accTz[fb], kf, dwf);
                }
            }
        }
        if constexpr (NC) {
            // ---- adjoint sums: U += phi(Q)^T dnum, u += phi(Q)^T dden (rows of wave 0)
            __syncthreads();
            Frag<T> ddf[CB];
#pragma unroll
            for (int kb = 0; kb < CB; ++kb)
                ddf[kb] = frag_acc<T>(*(const f32x4*)(sDD + 32 * kb + 4 * g), *(const f32x4*)(sDD + 32 * kb + 16 + 4 * g));
#pragma unroll
            for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) {
                    const Frag<T> qf = ColRead<T, F>::get(sQ, 32 * kb, 16 * fb, lane);
#pragma unroll
                    for (int t = 0; t < DBW; ++t)
                        mma(accS[fb][t], qf, ColRead<T, DV>::get(sDN, 32 * kb, 16 * (wave * DBW + t), lane));
                    mma(accu[fb], qf, ddf[kb]);
                }
            }
            __syncthreads();  // every wave has read the chunk's tiles
            continue;
        }
        // ---- state carry: S <- lambda^n S + phi(K)^T (w V), z <- lambda^n z + phi(K)^T w,
        // w_j = lambda^(n-1-j), applied to the V fragments in registers
        const float ln = lam_pow(l2l, n);
        Frag<T> wv[CB][DBW], wf[CB];
#pragma unroll
        for (int kb = 0; kb < CB; ++kb) {
            f32x4 wlo, whi;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j0 = 32 * kb + 4 * g + e, j1 = j0 + 16;
                wlo[e] = j0 < n ? lam_pow(l2l, n - 1 - j0) : 0.f;
                whi[e] = j1 < n ? lam_pow(l2l, n - 1 - j1) : 0.f;
            }
            wf[kb] = frag_acc<T>(wlo, whi);
#pragma unroll
            for (int t = 0; t < DBW; ++t)
                wv[kb][t] = frag_scale<T>(ColRead<T, DV>::get(sV, 32 * kb, 16 * (wave * DBW + t), lane), wlo, whi);
        }
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
            accZ[fb] *= ln;
#pragma unroll
            for (int t = 0; t < DBW; ++t) accS[fb][t] *= ln;
#pragma unroll
            for (int kb = 0; kb < CB; ++kb) {
                const Frag<T> kf = ColRead<T, F>::get(sK, 32 * kb, 16 * fb, lane);
#pragma unroll
                for (int t = 0; t < DBW; ++t) mma(accS[fb][t], kf, wv[kb][t]);
                mma(accZ[fb], kf, wf[kb]);
            }
        }
        __syncthreads();  // every wave has read sS before it is republished
    }

    if constexpr (NC) {
        float* Sd = a.S_dst + ((int64_t)seg * a.BH + bh) * a.dst_stride;
        float* zd = a.z_dst + ((int64_t)seg * a.BH + bh) * a.dst_zstride;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
            for (int t = 0; t < DBW; ++t) {
                const int d = 16 * (wave * DBW + t) + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) Sd[(16 * fb + 4 * g + r) * DV + d] = accS[fb][t][r];
            }
            if (wave == 0 && l16 == 0) *(f32x4*)(zd + 16 * fb + 4 * g) = accu[fb];
        }
    }
    if constexpr (DL) {
        // the segment's dT (start state held fixed) and its partial dlambda
        const int64_t slot = (int64_t)seg * a.BH + bh;
        constexpr int SZ = F * DV + F;
        float* Td = a.tseg + slot * SZ;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
            for (int t = 0; t < DBW; ++t) {
                const int d = 16 * (wave * DBW + t) + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) Td[(16 * fb + 4 * g + r) * DV + d] = accT[fb][t][r];
            }
            if (wave == 0 && l16 == 0) *(f32x4*)(Td + F * DV + 16 * fb + 4 * g) = accTz[fb];
        }
        dl = wave_sum_xor(dl, 1, 32);
        float* red = (float*)(smem + Cfg::OFF_R);
        if (lane == 0) red[wave] = dl;
        __syncthreads();
        if (tid == 0) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) sum += red[w];
            a.dlp[slot] = sum;
        }
    }
}

// ---------------------------------------------------------------------------
// Adjoint sweep (reverse chunk order): dk, dv (BMODE_KV) or the segment sums
// of the adjoint (BMODE_RLOCAL); BMODE_NCKV: dk, dv of the non-causal form
// from the total adjoint at S_src (keys only: no score tiles, no carry).
template <class T, int PHI, int DK, int F, int DV, int C, int NW, int MODE>
__global__ void __launch_bounds__(NW * 64, 1) la_bwd_kv_kernel(const BwdArgs a)
{
    using Cfg = BwdCfg<T, DK, F, DV, C, NW, MODE>;
    using TF = TileL<T, F>;
    using TVL = TileL<T, DV>;
    constexpr bool RL = MODE == BMODE_RLOCAL;
    constexpr bool NCK = MODE == BMODE_NCKV;
    constexpr int NT = Cfg::NT, VEC = Cfg::VEC, QB = Cfg::QB, CB = Cfg::CB, FB = Cfg::FB;
    constexpr int DBW = Cfg::DBW, FBW = Cfg::FBW;
    constexpr int KB = F / 32, VB = DV / 32;
    constexpr int VPRQ = DK / VEC, VPRV = DV / VEC;
    constexpr int RQ = (C * VPRQ + NT - 1) / NT, RV = (C * VPRV + NT - 1) / NT;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    T* const sQ = (T*)(smem + Cfg::OFF_F0);
    T* const sQw = (T*)(smem + Cfg::OFF_F1);
    T* const sK = (T*)(smem + Cfg::OFF_F2);
    T* const sV = (T*)(smem + Cfg::OFF_V0);
    T* const sDN = (T*)(smem + Cfg::OFF_V1);
    T* const sU = (T*)(smem + Cfg::OFF_S);
    float* const sDD = (float*)(smem + Cfg::OFF_R);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int seg = blockIdx.x, bh = blockIdx.y, h = bh % a.H;
    const float l2l = NCK ? 0.f : a.lam.log2lam[h];
    const int64_t NC = (a.N + C - 1) / C;
    const int64_t c_beg = (int64_t)seg * a.cps, c_end = (seg == a.P - 1) ? NC : min(NC, c_beg + a.cps);
    const int64_t row0 = (int64_t)bh * a.N;
    const T* qg = (const T*)a.q + row0 * DK;
    const T* kg = (const T*)a.k + row0 * DK;
    const T* vg = (const T*)a.v + row0 * DV;
    const T* gg = (const T*)a.gy + row0 * DV;
    const float* tk = NCK ? nullptr : a.tok + row0 * 2;
    const uint8_t* kp = a.kpm ? a.kpm + (int64_t)(bh / a.H) * a.N : nullptr;

    // decay of score element (i = 16 ib + 4 g + r, j = 16 jb + l16), i >= j
    float n0[4], n1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = 4 * g + r - l16;
        n0[r] = e < 0 ? 0.f : lam_pow(l2l, e);
        n1[r] = lam_pow(l2l, 16 + e);
    }

    // carried adjoint: U tiles (all f, this wave's value columns), u (all f)
    f32x4 accU[FB][DBW], accu[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
        accu[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < DBW; ++t) accU[fb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (!RL && a.S_src) {
        const float* Sb = a.S_src + (int64_t)seg * a.src_seg_stride + (int64_t)bh * a.src_stride;
        const float* zb = a.z_src + (int64_t)seg * a.src_seg_stride + (int64_t)bh * a.src_zstride;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
            for (int t = 0; t < DBW; ++t) {
                const int d = 16 * (wave * DBW + t) + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) accU[fb][t][r] = Sb[(16 * fb + 4 * g + r) * DV + d];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) accu[fb][r] = zb[16 * fb + 4 * g + r];
        }
    }
    auto publish = [&]() LA_BINLINE {
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int t = 0; t < DBW; ++t) {
                const int d = 16 * (wave * DBW + t) + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int f = 16 * fb + 4 * g + r;
                    sU[TVL::off(f, d & ~3) + (d & 3)] = from_f32<T>(accU[fb][t][r]);
                }
            }
    };

    if constexpr (NCK) publish();  // the total adjoint, read by every chunk

    uint4 rq[RQ], rk[RQ], rv[RV], rg[RV];
    int mk[RQ];
    for (int64_t c = c_end - 1; c >= c_beg; --c) {
        const int64_t t0 = c * C;
        const int n = (int)min((int64_t)C, a.N - t0);
#pragma unroll
        for (int r = 0; r < RQ; ++r) {
            const int idx = tid + r * NT, j = min(idx / VPRQ, n - 1), c4 = idx % VPRQ;
            if constexpr (!NCK) rq[r] = *(const uint4*)(qg + (t0 + j) * DK + c4 * VEC);
            if constexpr (!RL) {
                rk[r] = *(const uint4*)(kg + (t0 + j) * DK + c4 * VEC);
                mk[r] = kp ? (int)kp[t0 + j] : 0;
            }
        }
        float rden_r[RV], dd_r[RV];
#pragma unroll
        for (int r = 0; r < RV; ++r) {
            const int idx = tid + r * NT, j = min(idx / VPRV, n - 1), c4 = idx % VPRV;
            if constexpr (!RL) rv[r] = *(const uint4*)(vg + (t0 + j) * DV + c4 * VEC);
            if constexpr (!NCK) {
                rg[r] = *(const uint4*)(gg + (t0 + j) * DV + c4 * VEC);
                rden_r[r] = tk[(t0 + j) * 2];
                dd_r[r] = tk[(t0 + j) * 2 + 1];
            }
        }
        if constexpr (!RL && !NCK) publish();
#pragma unroll
        for (int r = 0; r < RQ; ++r) {
            const int idx = tid + r * NT, j = idx / VPRQ, cg = idx % VPRQ;
            if constexpr (!NCK) {
                float xq[VEC], pq[VEC], pw[VEC];
                unpack16(rq[r], xq, (const T*)nullptr);
                const float w = j < n ? lam_pow(l2l, j + 1) : 0.f;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    pq[e] = j < n ? phi_elem<T, PHI>(xq[e]) : 0.f;
                    pw[e] = pq[e] * w;
                }
#pragma unroll
                for (int e = 0; e < VEC; e += 4) {
                    if constexpr (!RL) st4(sQ + TF::off(j, cg * VEC + e), pq[e], pq[e + 1], pq[e + 2], pq[e + 3]);
                    st4(sQw + TF::off(j, cg * VEC + e), pw[e], pw[e + 1], pw[e + 2], pw[e + 3]);
                }
            }
            if constexpr (!RL) {
                float xk[VEC], pk[VEC];
                unpack16(rk[r], xk, (const T*)nullptr);
                const bool dead = j >= n || mk[r];
#pragma unroll
                for (int e = 0; e < VEC; ++e) pk[e] = dead ? 0.f : phi_elem<T, PHI>(xk[e]);
#pragma unroll
                for (int e = 0; e < VEC; e += 4) st4(sK + TF::off(j, cg * VEC + e), pk[e], pk[e + 1], pk[e + 2], pk[e + 3]);
            }
        }
#pragma unroll
        for (int r = 0; r < RV; ++r) {
            const int idx = tid + r * NT, j = idx / VPRV, cg = idx % VPRV;
            if constexpr (!NCK) {
                float xg[VEC];
                unpack16(rg[r], xg, (const T*)nullptr);
#pragma unroll
                for (int e = 0; e < VEC; ++e) xg[e] = j < n ? xg[e] * rden_r[r] : 0.f;
#pragma unroll
                for (int e = 0; e < VEC; e += 4) st4(sDN + TVL::off(j, cg * VEC + e), xg[e], xg[e + 1], xg[e + 2], xg[e + 3]);
            }
            if constexpr (!RL) {
                float xv[VEC];
                unpack16(rv[r], xv, (const T*)nullptr);
#pragma unroll
                for (int e = 0; e < VEC; ++e) xv[e] = j < n ? xv[e] : 0.f;
#pragma unroll
                for (int e = 0; e < VEC; e += 4) st4(sV + TVL::off(j, cg * VEC + e), xv[e], xv[e + 1], xv[e + 2], xv[e + 3]);
            }
            if (!NCK && cg == 0) sDD[j] = j < n ? dd_r[r] : 0.f;
        }
        __syncthreads();

        if constexpr (!RL) {
            // this wave's carried u tiles for d phi(k)
            constexpr bool WCOPY = FB >= 16;
            f32x4 uw[WCOPY ? FBW : 1];
            if constexpr (WCOPY) wave_blocks<NW, FBW>(accu, wave, uw);
            // per 16-key block: A and B score tiles (rows i, column j), dv, d phi(k)
#pragma unroll
            for (int jb = 0; jb < QB; ++jb) {
                const int j = 16 * jb + l16;
                const float lj = NCK ? 1.f : lam_pow(l2l, max(n - 1 - j, 0));  // the carried adjoint's decay for key j
                Frag<T> kf[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) kf[kb] = lds_frag_row<T, F>(sK, j, kb, g);
                Frag<T> vfr[VB];
#pragma unroll
                for (int kb = 0; kb < VB; ++kb) vfr[kb] = lds_frag_row<T, DV>(sV, j, kb, g);
                f32x4 at[2 * CB], bt[2 * CB];
#pragma unroll
                for (int ib = 0; ib < 2 * CB; ++ib) {
                    at[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
                    bt[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (!NCK && ib >= jb) {
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) mma(at[ib], lds_frag_row<T, F>(sQ, 16 * ib + l16, kb, g), kf[kb]);
#pragma unroll
                        for (int kb = 0; kb < VB; ++kb) mma(bt[ib], lds_frag_row<T, DV>(sDN, 16 * ib + l16, kb, g), vfr[kb]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float m = (ib == jb) ? n0[r] : n1[r] * lam_pow(l2l, 16 * (ib - jb - 1));
                            at[ib][r] *= m;
                            bt[ib][r] = (bt[ib][r] + sDD[16 * ib + 4 * g + r]) * m;
                        }
                    }
                }
                Frag<T> af[CB], bf[CB];
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) {
                    af[kb] = frag_acc<T>(at[2 * kb], at[2 * kb + 1]);
                    bf[kb] = frag_acc<T>(bt[2 * kb], bt[2 * kb + 1]);
                }
                // dv^T (rows d, column j) for this wave's value blocks
#pragma unroll
                for (int t = 0; t < DBW; ++t) {
                    const int d0 = 16 * (wave * DBW + t);
                    f32x4 intra = {0.f, 0.f, 0.f, 0.f}, inter = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (!NCK) {
#pragma unroll
                        for (int kb = 0; kb < CB; ++kb) mma(intra, ColRead<T, DV>::get(sDN, 32 * kb, d0, lane), af[kb]);
                    }
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) mma(inter, frag_acc<T>(accU[2 * kb][t], accU[2 * kb + 1][t]), kf[kb]);
                    if (j < n) {
                        const f32x4 o = intra + inter * lj;
                        st4((T*)a.dv + (row0 + t0 + j) * DV + d0 + 4 * g, o[0], o[1], o[2], o[3]);
                    }
                }
                // d phi(k)^T (rows f, column j) for this wave's feature blocks
#pragma unroll
                for (int u = 0; u < FBW; ++u) {
                    const int fb = wave * FBW + u;
                    f32x4 intra = {0.f, 0.f, 0.f, 0.f}, inter = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (!NCK) {
#pragma unroll
                        for (int kb = 0; kb < CB; ++kb) mma(intra, ColRead<T, F>::get(sQ, 32 * kb, 16 * fb, lane), bf[kb]);
                    }
#pragma unroll
                    for (int kb = 0; kb < VB; ++kb) mma(inter, lds_frag_row<T, DV>(sU, 16 * fb + l16, kb, g), vfr[kb]);
                    if (j < n) {
                        float o[4];
                        const f32x4 ph = ld4f(sK + TF::off(j, 16 * fb + 4 * g));
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float ur = WCOPY ? uw[WCOPY ? u : 0][r] : accu[fb][r];
                            const float dp = intra[r] + lj * (inter[r] + ur);
                            o[r] = dp * phi_deriv_from_phi<T, PHI>(ph[r]);
                        }
                        store_grad<T, PHI>(a.dk, (row0 + t0 + j) * DK + 16 * fb + 4 * g, o);
                    }
                }
            }
        }

        if constexpr (NCK) {
            __syncthreads();  // every wave has read the chunk's tiles
            continue;
        }
        // ---- adjoint carry: W <- lambda^n W + (w phi(Q))^T dnum, w_i = lambda^(i+1); u likewise with dden
        const float ln = lam_pow(l2l, n);
        Frag<T> ddf[CB];
#pragma unroll
        for (int kb = 0; kb < CB; ++kb)
            ddf[kb] = frag_acc<T>(*(const f32x4*)(sDD + 32 * kb + 4 * g), *(const f32x4*)(sDD + 32 * kb + 16 + 4 * g));
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
            accu[fb] *= ln;
#pragma unroll
            for (int t = 0; t < DBW; ++t) accU[fb][t] *= ln;
#pragma unroll
            for (int kb = 0; kb < CB; ++kb) {
                const Frag<T> qw = ColRead<T, F>::get(sQw, 32 * kb, 16 * fb, lane);
#pragma unroll
                for (int t = 0; t < DBW; ++t)
                    mma(accU[fb][t], qw, ColRead<T, DV>::get(sDN, 32 * kb, 16 * (wave * DBW + t), lane));
                mma(accu[fb], qw, ddf[kb]);
            }
        }
        __syncthreads();
    }

    // ---- segment sums (RLOCAL) or the initial state's gradient (KV, one segment)
    float* Sd = nullptr;
    float* zd = nullptr;
    if constexpr (RL) {
        Sd = a.S_dst + ((int64_t)seg * a.BH + bh) * a.dst_stride;
        zd = a.z_dst + ((int64_t)seg * a.BH + bh) * a.dst_zstride;
    } else if (!NCK && a.S_dst) {
        Sd = a.S_dst + (int64_t)bh * a.dst_stride;
        zd = a.z_dst + (int64_t)bh * a.dst_zstride;
    }
    if (Sd) {
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
            for (int t = 0; t < DBW; ++t) {
                const int d = 16 * (wave * DBW + t) + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) Sd[(16 * fb + 4 * g + r) * DV + d] = accU[fb][t][r];
            }
            if (wave == 0 && l16 == 0) *(f32x4*)(zd + 16 * fb + 4 * g) = accu[fb];
        }
    }
}

template <class T, int PHI, int DK, int F, int DV>
hipError_t bwd_launch(const BwdArgs& a, int mode, hipStream_t stream)
{
    constexpr int C = 32, NW = 4;
    const dim3 grid((unsigned)a.P, (unsigned)a.BH), block(NW * 64);
    switch (mode) {
    case BMODE_Q:
        if (a.tseg) {
            if constexpr (BwdCfg<T, DK, F, DV, C, NW, BMODE_Q, true>::TOTAL <= 160 * 1024)
                return launch_kernel(la_bwd_q_kernel<T, PHI, DK, F, DV, C, NW, true>, grid, block, stream, a);
            else
                return hipErrorInvalidConfiguration;
        }
        return launch_kernel(la_bwd_q_kernel<T, PHI, DK, F, DV, C, NW, false>, grid, block, stream, a);
    case BMODE_RLOCAL:
        return launch_kernel(la_bwd_kv_kernel<T, PHI, DK, F, DV, C, NW, BMODE_RLOCAL>, grid, block, stream, a);
    case BMODE_NCQ:
        return launch_kernel(la_bwd_q_kernel<T, PHI, DK, F, DV, C, NW, false, true>, grid, block, stream, a);
    case BMODE_NCKV:
        return launch_kernel(la_bwd_kv_kernel<T, PHI, DK, F, DV, C, NW, BMODE_NCKV>, grid, block, stream, a);
    default:
        return launch_kernel(la_bwd_kv_kernel<T, PHI, DK, F, DV, C, NW, BMODE_KV>, grid, block, stream, a);
    }
}

}  // namespace la
