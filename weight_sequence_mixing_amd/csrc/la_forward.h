// la_forward.h -- chunked forward kernel (gfx950) for causal and non-causal
// kernelized linear attention, templated on element type, feature map and
// head sizes.  Instantiated by the la_inst_*.hip units.
//
// Method ("Attention is also an FFN", kwkr.cn/news/587576, sec. 4.1 and
// sec. 5.2: cut the sequence into chunks, compute in parallel inside a chunk
// and carry a state across chunks; decay from sec. 3.2, normaliser from
// sec. 4.2).  For a chunk of n tokens starting after state (S, z), with local
// positions i, j in [0, n):
//
//   num_i, den_i = lambda^(i+1) phi(q_i)^T [S, z]
//                + sum_{j<=i} lambda^(i-j) (phi(q_i).phi(k_j)) [v_j, 1]
//   y_i          = num_i / (den_i + eps)
//   S            <- lambda^n S + sum_j lambda^(n-1-j) phi(k_j) v_j^T   (z likewise)
//
// which equals the token-by-token recurrence exactly up to rounding order.
//
// One workgroup of 4 waves owns one segment (a run of whole chunks) of one
// (batch, head) row.  The fp32 state lives in the waves' accumulator
// registers, split by value column: wave w owns d_v columns
// [16*DBW*w, 16*DBW*(w+1)) of S for all F feature rows, so the product
// phi(Q) S reads its B operand straight from the accumulators (see the
// fragment note in la_device.h) and the state never goes through LDS.
// The chunk's scores phi(K) phi(Q)^T are computed once, cooperatively, and
// shared through LDS as the masked, decayed matrix P (row-major, bf16).
//
// Modes: MODE_LOCAL   segment-local state from a zero start (pass 1),
//        MODE_CAUSAL  outputs of a segment from its carried-in state (pass 3),
//        MODE_QUERY   non-causal outputs for a fixed state.
#pragma once

#include "la_device.h"
#include "la_internal.h"

namespace la {

// Transposed [rows][C] buffers are XOR-swizzled in groups of 4 columns so that
// the scattered 2-byte staging writes spread over the LDS banks while every
// 4-element group stays contiguous (and 8-byte aligned) for fragment reads.
__device__ __forceinline__ int tsw(int r, int j) { return j ^ (((r >> 3) & 7) << 2); }

template <class T, int PHI>
constexpr int chunk_len(int F) {
    return (sizeof(T) == 4) ? 32 : (F > 128 ? 32 : 64);
}

template <class T, int PHI, int DK, int F, int DV, int C, int NW, int MODE>
struct FwdCfg {
    static constexpr int NT = NW * 64;
    static constexpr int VEC = 16 / (int)sizeof(T);
    static constexpr bool RF = PHI == LA_PHI_TRIG_RF;
    static constexpr int M = RF ? F / 2 : 0;
    static constexpr int QB = C / 16;
    static constexpr int FB = F / 16;
    static constexpr int DB = DV / 16;
    static constexpr int DBW = DB / NW;
    static constexpr int PAD = 4;
    static constexpr int QLD = F + PAD;
    static constexpr int PLD = C + PAD;
    static constexpr int XLD = DK + PAD;
    static constexpr bool NEED_Q = MODE != MODE_LOCAL;
    static constexpr bool NEED_K = MODE != MODE_QUERY;
    static constexpr bool NEED_KROW = MODE == MODE_CAUSAL;
    static constexpr bool NEED_P = MODE == MODE_CAUSAL;
    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t SZ_Q = NEED_Q ? size_t(C) * QLD * sizeof(T) : 0;
    static constexpr size_t OFF_K = al(OFF_Q + SZ_Q);
    static constexpr size_t SZ_K = NEED_KROW ? size_t(C) * QLD * sizeof(T) : 0;
    static constexpr size_t OFF_KT = al(OFF_K + SZ_K);
    static constexpr size_t SZ_KT = NEED_K ? size_t(F) * C * sizeof(T) : 0;
    static constexpr size_t OFF_VT = al(OFF_KT + SZ_KT);
    static constexpr size_t SZ_VT = NEED_K ? size_t(DV) * C * sizeof(T) : 0;
    static constexpr size_t OFF_P = al(OFF_VT + SZ_VT);
    static constexpr size_t SZ_P = NEED_P ? size_t(C) * PLD * sizeof(T) : 0;
    static constexpr size_t OFF_Z = al(OFF_P + SZ_P);
    static constexpr size_t SZ_Z = size_t(F) * sizeof(float);
    static constexpr size_t OFF_DEN = al(OFF_Z + SZ_Z);
    static constexpr size_t SZ_DEN = size_t(C) * sizeof(float);
    static constexpr size_t OFF_ROW = al(OFF_DEN + SZ_DEN);
    static constexpr size_t SZ_ROW = NEED_P ? size_t(QB) * C * sizeof(float) : 0;
    static constexpr size_t OFF_XQ = al(OFF_ROW + SZ_ROW);
    static constexpr size_t SZ_XQ = (RF && NEED_Q) ? size_t(C) * XLD * sizeof(T) : 0;
    static constexpr size_t OFF_XK = al(OFF_XQ + SZ_XQ);
    static constexpr size_t SZ_XK = (RF && NEED_K) ? size_t(C) * XLD * sizeof(T) : 0;
    static constexpr size_t OFF_XN = al(OFF_XK + SZ_XK);
    static constexpr size_t SZ_XN = RF ? size_t(2) * C * sizeof(float) : 0;
    // partial sums over token groups of the weighted key features (for z)
    static constexpr int ZR = NW > QB ? NW : QB;
    static constexpr size_t OFF_ZP = al(OFF_XN + SZ_XN);
    static constexpr size_t SZ_ZP = NEED_K ? size_t(ZR) * F * sizeof(float) : 0;
    static constexpr size_t OFF_OM = al(OFF_ZP + SZ_ZP);
    // omega in LDS: bf16 high and low parts (bf16 inputs) or fp32 (fp32 inputs)
    static constexpr size_t SZ_OM = RF ? (sizeof(T) == 2 ? size_t(2) * M * XLD * 2 : size_t(M) * XLD * 4) : 0;
    static constexpr size_t TOTAL = al(OFF_OM + SZ_OM);

    static_assert(C % 32 == 0 && C >= 32, "chunk must be a multiple of 32");
    static_assert(F % 32 == 0 && DV % 16 == 0 && DK % 32 == 0, "head sizes");
    static_assert(DBW >= 1 && DB % NW == 0, "value columns must split over the waves");
    static_assert(F <= NT && C <= NT && NT % C == 0, "thread mapping");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

template <class T, int PHI, int DK, int F, int DV, int C, int NW, int MODE>
__global__ void __launch_bounds__(NW * 64)
la_fwd_kernel(const FwdArgs a)
{
    using Cfg = FwdCfg<T, PHI, DK, F, DV, C, NW, MODE>;
    constexpr int NT = Cfg::NT, VEC = Cfg::VEC, M = Cfg::M, QB = Cfg::QB, FB = Cfg::FB;
    constexpr int DBW = Cfg::DBW, QLD = Cfg::QLD, PLD = Cfg::PLD, XLD = Cfg::XLD;
    constexpr bool RF = Cfg::RF;
    constexpr int VPRQ = DK / VEC;              // 16-byte vectors per q/k row
    constexpr int VPRV = DV / VEC;              // 16-byte vectors per v row
    constexpr int VQ = C * VPRQ, VV = C * VPRV; // vectors per tile
    constexpr int RQ = (VQ + NT - 1) / NT, RV = (VV + NT - 1) / NT;
    static_assert(VQ % NT == 0 && VV % NT == 0, "tiles must split evenly over threads");

    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    T* sQ = (T*)(smem + Cfg::OFF_Q);
    T* sK = (T*)(smem + Cfg::OFF_K);
    T* sKT = (T*)(smem + Cfg::OFF_KT);
    T* sVT = (T*)(smem + Cfg::OFF_VT);
    T* sP = (T*)(smem + Cfg::OFF_P);
    float* sZ = (float*)(smem + Cfg::OFF_Z);
    float* sDen = (float*)(smem + Cfg::OFF_DEN);
    float* sRow = (float*)(smem + Cfg::OFF_ROW);
    T* sXq = (T*)(smem + Cfg::OFF_XQ);
    T* sXk = (T*)(smem + Cfg::OFF_XK);
    float* sXn = (float*)(smem + Cfg::OFF_XN);
    float* sZp = (float*)(smem + Cfg::OFF_ZP);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int seg = blockIdx.x, bh = blockIdx.y, h = bh % a.H;
    const float l2l = (MODE == MODE_QUERY) ? 0.f : a.lam.log2lam[h];
    const int64_t NC = (a.n_len + C - 1) / C;
    const int64_t c_beg = (int64_t)seg * NC / a.P, c_end = (int64_t)(seg + 1) * NC / a.P;
    const T* qg = (const T*)a.q + ((int64_t)bh * a.N + a.n0) * DK;
    const T* kg = (const T*)a.k + ((int64_t)bh * a.N + a.n0) * DK;
    const T* vg = (const T*)a.v + ((int64_t)bh * a.N + a.n0) * DV;
    const float qs = a.qk_scale;

    // ---- random-feature directions into LDS (once per workgroup)
    if constexpr (RF) {
        for (int idx = tid; idx < M * DK; idx += NT) {
            const int r = idx / DK, d = idx % DK;
            const float w = a.omega[idx];
            if constexpr (sizeof(T) == 2) {
                bf16* hi = (bf16*)(smem + Cfg::OFF_OM);
                bf16* lo = hi + M * XLD;
                const bf16 wh = (bf16)w;
                hi[r * XLD + d] = wh;
                lo[r * XLD + d] = (bf16)(w - (float)wh);
            } else {
                ((float*)(smem + Cfg::OFF_OM))[r * XLD + d] = w;
            }
        }
    }

    // ---- carried state: accumulator tiles (fb, this wave's d-blocks)
    f32x4 accS[FB][DBW];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int t = 0; t < DBW; ++t) accS[fb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float zreg = 0.f;  // z[tid] (tid < F)
    if constexpr (MODE != MODE_LOCAL) {
        if (a.S_src) {
            const float* Sb = a.S_src + (int64_t)seg * a.src_seg_stride + (int64_t)bh * a.src_stride;
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                for (int t = 0; t < DBW; ++t) {
                    const int d = 16 * (wave * DBW + t) + l16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) accS[fb][t][r] = Sb[(16 * fb + 4 * g + r) * DV + d];
                }
            if (tid < F) zreg = a.z_src[(int64_t)seg * a.src_seg_stride + (int64_t)bh * a.src_zstride + tid];
        }
        if (tid < F) sZ[tid] = zreg;
    }
    if constexpr (Cfg::NEED_P) {
        for (int idx = tid; idx < C * PLD; idx += NT) sP[idx] = from_f32<T>(0.f);
    }

    // ---- global -> register prefetch of one chunk.  Rows past the end of the
    // sequence re-read the last valid row (always in bounds) and are replaced
    // by zeros in registers, so the loads stay unconditional global loads.
    uint4 rq[Cfg::NEED_Q ? RQ : 1], rk[Cfg::NEED_K ? RQ : 1], rv[Cfg::NEED_K ? RV : 1];
    auto load_chunk = [&](int64_t c) {
        const int64_t t0 = c * C;
        const int n = (int)min((int64_t)C, a.n_len - t0);
        const uint4 zero = {0u, 0u, 0u, 0u};
        if constexpr (Cfg::NEED_Q) {
#pragma unroll
            for (int r = 0; r < RQ; ++r) {
                const int idx = tid + r * NT, j = idx / VPRQ, cg = idx % VPRQ;
                const uint4 val = *(const uint4*)(qg + (t0 + min(j, n - 1)) * DK + cg * VEC);
                rq[r] = (j < n) ? val : zero;
            }
        }
        if constexpr (Cfg::NEED_K) {
#pragma unroll
            for (int r = 0; r < RQ; ++r) {
                const int idx = tid + r * NT, j = idx / VPRQ, cg = idx % VPRQ;
                const uint4 val = *(const uint4*)(kg + (t0 + min(j, n - 1)) * DK + cg * VEC);
                rk[r] = (j < n) ? val : zero;
            }
#pragma unroll
            for (int r = 0; r < RV; ++r) {
                const int idx = tid + r * NT, j = idx / VPRV, cg = idx % VPRV;
                const uint4 val = *(const uint4*)(vg + (t0 + min(j, n - 1)) * DV + cg * VEC);
                rv[r] = (j < n) ? val : zero;
            }
        }
    };

    // ---- register -> LDS staging (feature map for elu+1; raw tiles for RF)
    auto stage = [&](int n) {
        if constexpr (Cfg::NEED_Q) {
#pragma unroll
            for (int r = 0; r < RQ; ++r) {
                const int idx = tid + r * NT, j = idx / VPRQ, cg = idx % VPRQ;
                float x[VEC];
                unpack16(rq[r], x, (const T*)nullptr);
                if constexpr (RF) {
                    float s2 = 0.f;
#pragma unroll
                    for (int e = 0; e < VEC; e += 4) {
                        st4(sXq + j * XLD + cg * VEC + e, x[e], x[e + 1], x[e + 2], x[e + 3]);
                        s2 += x[e] * x[e] + x[e + 1] * x[e + 1] + x[e + 2] * x[e + 2] + x[e + 3] * x[e + 3];
                    }
                    s2 = wave_sum_xor(s2, 1, VPRQ / 2);
                    if (cg == 0) sXn[j] = s2;
                } else {
                    float p[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) p[e] = (j < n) ? phi_elu1<T>(x[e]) : 0.f;
#pragma unroll
                    for (int e = 0; e < VEC; e += 4) st4(sQ + j * QLD + cg * VEC + e, p[e], p[e + 1], p[e + 2], p[e + 3]);
                }
            }
        }
        if constexpr (Cfg::NEED_K) {
            // every r visits the same feature group cg = tid % VPRQ
            float zacc[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) zacc[e] = 0.f;
#pragma unroll
            for (int r = 0; r < RQ; ++r) {
                const int idx = tid + r * NT, j = idx / VPRQ, cg = idx % VPRQ;
                float x[VEC];
                unpack16(rk[r], x, (const T*)nullptr);
                if constexpr (RF) {
                    float s2 = 0.f;
#pragma unroll
                    for (int e = 0; e < VEC; e += 4) {
                        st4(sXk + j * XLD + cg * VEC + e, x[e], x[e + 1], x[e + 2], x[e + 3]);
                        s2 += x[e] * x[e] + x[e + 1] * x[e + 1] + x[e + 2] * x[e + 2] + x[e + 3] * x[e + 3];
                    }
                    s2 = wave_sum_xor(s2, 1, VPRQ / 2);
                    if (cg == 0) sXn[C + j] = s2;
                } else {
                    const float w = (j < n) ? lam_pow(l2l, n - 1 - j) : 0.f;
                    float p[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) p[e] = (j < n) ? phi_elu1<T>(x[e]) : 0.f;
                    if constexpr (Cfg::NEED_KROW) {
#pragma unroll
                        for (int e = 0; e < VEC; e += 4) st4(sK + j * QLD + cg * VEC + e, p[e], p[e + 1], p[e + 2], p[e + 3]);
                    }
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const int f = cg * VEC + e;
                        const T wp = from_f32<T>(w * p[e]);
                        sKT[f * C + tsw(f, j)] = wp;
                        zacc[e] += to_f32(wp);
                    }
                }
            }
            if constexpr (!RF) {
                // sum over the lanes of this wave that hold the same feature group
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    for (int m = VPRQ; m < 64; m <<= 1) zacc[e] += __shfl_xor(zacc[e], m, 64);
                if (lane < VPRQ) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) sZp[wave * F + lane * VEC + e] = zacc[e];
                }
            }
#pragma unroll
            for (int r = 0; r < RV; ++r) {
                const int idx = tid + r * NT, j = idx / VPRV, cg = idx % VPRV;
                float x[VEC];
                unpack16(rv[r], x, (const T*)nullptr);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int d = cg * VEC + e;
                    sVT[d * C + tsw(d, j)] = from_f32<T>(x[e]);
                }
            }
        }
    };

    // ---- random features on the matrix cores: U^T = omega x^T, then cos/sin
    auto rf_features = [&](const T* sX, const float* xn, T* dst_row, T* dst_t, int n) {
        if constexpr (RF) {
            constexpr int TILES = (M / 16) * QB;
            const float cnorm = rsqrtf((float)M);
            for (int t = wave; t < TILES; t += NW) {
                const int rb = t / QB, ib = t % QB;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    const Frag<T> b = frag_rm(sX, XLD, 16 * ib + l16, 32 * kb, g);
                    if constexpr (sizeof(T) == 2) {
                        const bf16* hi = (const bf16*)(smem + Cfg::OFF_OM);
                        const bf16* lo = hi + M * XLD;
                        mma(acc, frag_rm(hi, XLD, 16 * rb + l16, 32 * kb, g), b);
                        mma(acc, frag_rm(lo, XLD, 16 * rb + l16, 32 * kb, g), b);
                    } else {
                        const float* om = (const float*)(smem + Cfg::OFF_OM);
                        mma(acc, frag_rm(om, XLD, 16 * rb + l16, 32 * kb, g), b);
                    }
                }
                const int i = 16 * ib + l16;
                const float cfac = (i < n) ? exp_rf<T>(-0.5f * qs * qs * xn[i]) * cnorm : 0.f;
                float cs[4], sn[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sincos_rf<T>(qs * acc[r], &sn[r], &cs[r]);
                    cs[r] *= cfac;
                    sn[r] *= cfac;
                }
                const int f0 = 16 * rb + 4 * g;
                if (dst_row) {
                    st4(dst_row + i * QLD + f0, cs[0], cs[1], cs[2], cs[3]);
                    st4(dst_row + i * QLD + M + f0, sn[0], sn[1], sn[2], sn[3]);
                }
                if (dst_t) {
                    const float w = (i < n) ? lam_pow(l2l, n - 1 - i) : 0.f;
                    float zc[4], zs[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const T wc = from_f32<T>(w * cs[r]), ws = from_f32<T>(w * sn[r]);
                        dst_t[(f0 + r) * C + tsw(f0 + r, i)] = wc;
                        dst_t[(M + f0 + r) * C + tsw(M + f0 + r, i)] = ws;
                        zc[r] = wave_sum_xor(to_f32(wc), 1, 8);
                        zs[r] = wave_sum_xor(to_f32(ws), 1, 8);
                    }
                    if (l16 == 0) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            sZp[ib * F + f0 + r] = zc[r];
                            sZp[ib * F + M + f0 + r] = zs[r];
                        }
                    }
                }
            }
        }
    };

    // ---- main loop over the segment's chunks
    if (c_beg < c_end) load_chunk(c_beg);
    __syncthreads();  // LDS initialisation complete
    for (int64_t c = c_beg; c < c_end; ++c) {
        const int64_t t0 = c * C;
        const int n = (int)min((int64_t)C, a.n_len - t0);
        stage(n);
        __syncthreads();
        if (c + 1 < c_end) load_chunk(c + 1);
        if constexpr (RF) {
            if constexpr (Cfg::NEED_Q) rf_features(sXq, sXn, sQ, (T*)nullptr, n);
            if constexpr (Cfg::NEED_K) rf_features(sXk, sXn + C, Cfg::NEED_KROW ? sK : (T*)nullptr, sKT, n);
            __syncthreads();
        }

        // -- scores P = mask(lambda^(i-j) phi(q_i).phi(k_j)), row sums
        if constexpr (MODE == MODE_CAUSAL) {
            constexpr int NSC = QB * (QB + 1) / 2;
            for (int t = wave; t < NSC; t += NW) {
                int ib = 0, jb = t;
                while (jb > ib) { jb -= ib + 1; ++ib; }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < F / 32; ++kb)
                    mma(acc, frag_rm(sK, QLD, 16 * jb + l16, 32 * kb, g), frag_rm(sQ, QLD, 16 * ib + l16, 32 * kb, g));
                const int i = 16 * ib + l16;
                float pv[4], rs = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * jb + 4 * g + r;
                    const float x = (j <= i) ? acc[r] * lam_pow(l2l, i - j) : 0.f;
                    pv[r] = to_f32(from_f32<T>(x));
                    rs += pv[r];
                }
                st4(sP + i * PLD + 16 * jb + 4 * g, pv[0], pv[1], pv[2], pv[3]);
                rs += __shfl_xor(rs, 16, 64);
                rs += __shfl_xor(rs, 32, 64);
                if (g == 0) sRow[jb * C + i] = rs;
            }
        }

        // -- phi(q_i).z for the denominator, and the next z
        constexpr int TPR = NT / C;
        const int row = tid / TPR, sub = tid % TPR;
        float dqz = 0.f;
        if constexpr (Cfg::NEED_Q) {
            for (int f = sub; f < F; f += TPR) dqz += to_f32(sQ[row * QLD + f]) * sZ[f];
            dqz = wave_sum_xor(dqz, 1, TPR / 2);
        }
        float znew = zreg;
        if constexpr (Cfg::NEED_K) {
            if (tid < F) {
                constexpr int NZP = RF ? QB : NW;  // row groups that wrote partial sums
                float zs = 0.f;
#pragma unroll
                for (int w = 0; w < NZP; ++w) zs += sZp[w * F + tid];
                znew = lam_pow(l2l, n) * zreg + zs;
            }
        }

        if constexpr (Cfg::NEED_Q) {
            if constexpr (MODE == MODE_CAUSAL) __syncthreads();  // sRow complete
            if (sub == 0) {
                float den = dqz;
                if constexpr (MODE == MODE_CAUSAL) {
                    float rsum = 0.f;
                    for (int jb = 0; jb <= row / 16; ++jb) rsum += sRow[jb * C + row];
                    den = rsum + lam_pow(l2l, row + 1) * dqz;
                }
                sDen[row] = den;
            }
            __syncthreads();  // sDen complete

            // -- outputs: O = lambda^(i+1) phi(Q) S  (+ P V), normalised
            Frag<T> sfr[F / 32][DBW];
#pragma unroll
            for (int kb = 0; kb < F / 32; ++kb)
#pragma unroll
                for (int t = 0; t < DBW; ++t) sfr[kb][t] = frag_acc<T>(accS[2 * kb][t], accS[2 * kb + 1][t]);
            const float eps = a.eps;
#pragma unroll
            for (int ib = 0; ib < QB; ++ib) {
                f32x4 o[DBW];
#pragma unroll
                for (int t = 0; t < DBW; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < F / 32; ++kb) {
                    const Frag<T> fa = frag_rm(sQ, QLD, 16 * ib + l16, 32 * kb, g);
#pragma unroll
                    for (int t = 0; t < DBW; ++t) mma(o[t], fa, sfr[kb][t]);
                }
                if constexpr (MODE == MODE_CAUSAL) {
#pragma unroll
                    for (int t = 0; t < DBW; ++t)
#pragma unroll
                        for (int r = 0; r < 4; ++r) o[t][r] *= lam_pow(l2l, 16 * ib + 4 * g + r + 1);
#pragma unroll
                    for (int kb2 = 0; kb2 <= ib / 2; ++kb2) {
                        const Frag<T> fp = frag_rm(sP, PLD, 16 * ib + l16, 32 * kb2, g);
#pragma unroll
                        for (int t = 0; t < DBW; ++t) {
                            const int rr = 16 * (wave * DBW + t) + l16;
                            const T* vrow = sVT + rr * C;
                            mma(o[t], fp, frag2(vrow + tsw(rr, 32 * kb2 + 4 * g), vrow + tsw(rr, 32 * kb2 + 16 + 4 * g)));
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * ib + 4 * g + r;
                    if (i < n) {
                        const float inv = 1.0f / (sDen[i] + eps);
                        const int64_t yo = ((int64_t)bh * a.N + a.n0 + t0 + i) * DV;
#pragma unroll
                        for (int t = 0; t < DBW; ++t) {
                            const int d = 16 * (wave * DBW + t) + l16;
                            if (a.out_f32) ((float*)a.y)[yo + d] = o[t][r] * inv;
                            else ((T*)a.y)[yo + d] = from_f32<T>(o[t][r] * inv);
                        }
                    }
                }
            }
        }

        // -- state carry: S <- lambda^n S + (w phi(K))^T V
        if constexpr (Cfg::NEED_K) {
            const float dec = lam_pow(l2l, n);
            Frag<T> vfr[C / 32][DBW];
#pragma unroll
            for (int kb = 0; kb < C / 32; ++kb)
#pragma unroll
                for (int t = 0; t < DBW; ++t) {
                    const int rr = 16 * (wave * DBW + t) + l16;
                    const T* vrow = sVT + rr * C;
                    vfr[kb][t] = frag2(vrow + tsw(rr, 32 * kb + 4 * g), vrow + tsw(rr, 32 * kb + 16 + 4 * g));
                }
#pragma unroll
            for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
                for (int t = 0; t < DBW; ++t) accS[fb][t] *= dec;
                const int rr = 16 * fb + l16;
                const T* krow = sKT + rr * C;
#pragma unroll
                for (int kb = 0; kb < C / 32; ++kb) {
                    const Frag<T> fk = frag2(krow + tsw(rr, 32 * kb + 4 * g), krow + tsw(rr, 32 * kb + 16 + 4 * g));
#pragma unroll
                    for (int t = 0; t < DBW; ++t) mma(accS[fb][t], fk, vfr[kb][t]);
                }
            }
        }
        __syncthreads();  // every read of this chunk's LDS tiles is done
        if constexpr (Cfg::NEED_K) {
            zreg = znew;
            if constexpr (MODE == MODE_CAUSAL) {
                if (tid < F) sZ[tid] = znew;
            }
        }
    }

    // ---- state out
    if constexpr (MODE != MODE_QUERY) {
        float* Sd = nullptr;
        float* zd = nullptr;
        if constexpr (MODE == MODE_LOCAL) {
            Sd = a.S_dst + ((int64_t)seg * a.BH + bh) * a.dst_stride;
            zd = a.z_dst + ((int64_t)seg * a.BH + bh) * a.dst_zstride;
        } else if (a.S_dst) {
            Sd = a.S_dst + (int64_t)bh * a.dst_stride;
            zd = a.z_dst + (int64_t)bh * a.dst_zstride;
        }
        if (Sd) {
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                for (int t = 0; t < DBW; ++t) {
                    const int d = 16 * (wave * DBW + t) + l16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) Sd[(16 * fb + 4 * g + r) * DV + d] = accS[fb][t][r];
                }
            if (tid < F) zd[tid] = zreg;
        }
    }
}

template <class T, int PHI, int DK, int F, int DV>
hipError_t fwd_launch(const FwdArgs& a, int mode, hipStream_t stream)
{
    constexpr int C = chunk_len<T, PHI>(F);
    constexpr int NW = 4;
    const dim3 grid((unsigned)a.P, (unsigned)a.BH), block(NW * 64);
    switch (mode) {
    case MODE_LOCAL:
        hipLaunchKernelGGL((la_fwd_kernel<T, PHI, DK, F, DV, C, NW, MODE_LOCAL>), grid, block, 0, stream, a);
        break;
    case MODE_CAUSAL:
        hipLaunchKernelGGL((la_fwd_kernel<T, PHI, DK, F, DV, C, NW, MODE_CAUSAL>), grid, block, 0, stream, a);
        break;
    default:
        hipLaunchKernelGGL((la_fwd_kernel<T, PHI, DK, F, DV, C, NW, MODE_QUERY>), grid, block, 0, stream, a);
        break;
    }
    return hipGetLastError();
}

}  // namespace la
