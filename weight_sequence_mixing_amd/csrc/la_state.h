// la_state.h -- the segment-state pass for bf16 inputs (elu+1, ReLU and the
// trigonometric random features): the state a segment of L tokens leaves
// when it starts from zero,
//
//   S = sum_t lambda^(L-1-t) phi(k_t) v_t^T,   z = sum_t lambda^(L-1-t) phi(k_t)
//
// (the recurrence of "Attention is also an FFN", kwkr.cn/news/587576,
// sec. 4.1 and the chunked form of sec. 5.2, decay sec. 3.2; keys and values
// only).  The scan of la_scan.hip turns these into each segment's carried-in
// state.
//
// Work split.  A workgroup takes one segment in 64-token chunks; the next
// chunk's loads are issued as soon as the current one is staged, and the
// LDS buffers are doubled, so a chunk needs one barrier.
//
// Elementwise maps: the weighted key features w_j phi(k_j) (w_j the decay
// weight, zero for a dropped key) and the values are staged in TileX, whose
// staging writes and transposing reads are both conflict-free.  The state's
// 16 x 16 tiles are split over a 4 x 2 grid of eight waves, or 4 x 4 of
// sixteen where d_k = d_v = 128 (feature blocks x value columns); each wave
// reads the (w phi(K))^T and V fragments of its tiles and adds their product.
//
// Random features ("From standard attention to linear attention", sec. 4.2:
// phi(x) = c(x) [cos(omega x'), sin(omega x')] / sqrt(m), x' = qk_scale x):
// only the raw key rows, the weights w_j c(k_j) and the values are staged.
// Each wave owns the cos and the sin rows of one 16-row block of omega and
// forms them in registers: U = X omega^T on the matrix cores (omega scaled
// to revolutions and split into bf16 high and low parts, as in the output
// pass), whose two accumulator tiles over 32 tokens are already the A operand
// of the state update (la_device.h: an accumulator pair is a fragment over
// the k positions K(g)), so the features never pass through LDS and each is
// computed once.  Where omega has fewer row blocks than there are waves, the
// two waves of a row block split the chunk's tokens and their states are
// added at the end.
#pragma once

#include <type_traits>

#include "la_device.h"
#include "la_internal.h"

namespace la {

template <int PHI, int DK, int F, int DV>
struct StateCfg {
    static constexpr bool RF = PHI == LA_PHI_TRIG_RF;
    static constexpr int M = RF ? F / 2 : 0;
    static constexpr int C = 64, CB = C / 32;
    static constexpr int FB = F / 16, DB = DV / 16;
    // random features: row blocks of omega, one per wave (two waves each
    // where there are fewer than eight: TS token splits)
    static constexpr int RBN = RF ? M / 16 : 1;
    // elementwise maps: a 4 x (NWE / 4) grid of waves; 16 waves where both
    // widths are 128 (the plan then gives one workgroup per compute unit)
    static constexpr int NWE = (DK >= 128 && DV >= 128) ? 16 : 8;
    static constexpr int NW = RF ? (2 * RBN < 8 ? 2 * RBN : 8) : NWE;
    static constexpr int NT = NW * 64;
    static constexpr int TS = RF ? NW / RBN : 1;
    // state tiles of a wave: FBW feature blocks x DBW value-column tiles
    static constexpr int WD = RF ? 1 : NW / 4;
    static constexpr int FBW = RF ? 2 : FB / 4;
    static constexpr int DBW = RF ? DB : DB / WD;
    // register sets of loads in flight (one chunk ahead)
    static constexpr int PF = 1;
    static constexpr int VEC = 8, VPRK = DK / VEC, VPRV = DV / VEC;
    static constexpr int RK = C * VPRK / NT, RV = C * VPRV / NT;
    // raw key rows padded by 16 bytes: a row-fragment read of 16 rows is then
    // conflict-free as single 8-byte reads
    static constexpr int KX = DK / 32, XLD = DK + 8;
    // one LDS buffer: the keys (weighted features, or raw rows), the values,
    // the key weights (random features)
    static constexpr size_t KBYTES = RF ? size_t(C) * XLD * 2 : size_t(C) * F * 2;
    static constexpr size_t VBYTES = size_t(C) * DV * 2;
    static constexpr size_t WBYTES = RF ? size_t(C) * 4 : 0;
    static constexpr size_t BUF = KBYTES + VBYTES + WBYTES;
    // the second token split's tiles, handed to the first at the end
    static constexpr int TPW = FBW * DBW + FBW;
    static constexpr size_t RED = TS > 1 ? size_t(RBN) * TPW * 64 * 16 : 0;
    static constexpr size_t TOTAL = 2 * BUF > RED ? 2 * BUF : RED;
    // waves per SIMD asked of the register allocator: four (128 registers:
    // two workgroups of eight waves, or one of sixteen, per compute unit);
    // for the random features beyond d_k = d_v = 64, whose omega fragments
    // and value tiles need more, one workgroup per compute unit
    static constexpr int WPE = RF ? ((DK > 64 || DV > 64) ? NW / 4 : 2 * NW / 4) : 4;
    static_assert(F % 64 == 0 && DV % 64 == 0 && DK % 64 == 0, "head sizes");
    static_assert(RF || DK == F, "elementwise maps keep the width");
    static_assert(!RF || (RBN >= 2 && TS <= 2 && RBN * TS == NW), "omega row blocks over the waves");
    static_assert(RF || (FB % 4 == 0 && DB % WD == 0), "wave grid");
    static_assert(RK >= 1 && RV >= 1 && (C * VPRK) % NT == 0 && (C * VPRV) % NT == 0, "loads per thread");
    static_assert(BUF % 16 == 0 && KBYTES % 16 == 0, "alignment");
    static_assert(TOTAL <= 80 * 1024, "two workgroups per compute unit");
};

// w phi(x) for an elementwise map, w = 2^lw: for elu+1 the weight goes into
// the exponent of its exponential branch (2^(x log2(e) + lw)), which saves a
// multiplication; a dropped key has x = 0, w = 0, lw = -inf.
template <int PHI>
__device__ __forceinline__ float phi_weighted(float x, float w, float lw)
{
    if constexpr (PHI == LA_PHI_ELU1)
        return x > 0.f ? fmaf(x, w, w) : __builtin_amdgcn_exp2f(fmaf(x, 1.44269504088896341f, lw));
    else
        return phi_elem<bf16, PHI>(x) * w;
}

template <int PHI, int DK, int F, int DV>
__global__ void __launch_bounds__((StateCfg<PHI, DK, F, DV>::NT), (StateCfg<PHI, DK, F, DV>::WPE))
la_state_kernel(const FwdArgs a)
{
    using Cfg = StateCfg<PHI, DK, F, DV>;
    using T = bf16;
    constexpr int C = Cfg::C, CB = Cfg::CB, NT = Cfg::NT, VEC = Cfg::VEC;
    constexpr int FBW = Cfg::FBW, DBW = Cfg::DBW, RK = Cfg::RK, RV = Cfg::RV;
    constexpr int VPRK = Cfg::VPRK, VPRV = Cfg::VPRV, KX = Cfg::KX, XLD = Cfg::XLD;
    constexpr int RBN = Cfg::RBN, TS = Cfg::TS, PF = Cfg::PF;
    constexpr bool RF = Cfg::RF;
    using TK = TileX<T, F>;
    using TVL = TileX<T, DV>;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    // buffer b: keys, values, key weights
    auto sKb = [&](int b) LA_INLINE { return (T*)(smem + b * Cfg::BUF); };
    auto sVb = [&](int b) LA_INLINE { return (T*)(smem + b * Cfg::BUF + Cfg::KBYTES); };
    auto sWb = [&](int b) LA_INLINE { return (float*)(smem + b * Cfg::BUF + Cfg::KBYTES + Cfg::VBYTES); };

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    // wave roles.  Elementwise maps: feature blocks FBW wf .. and value
    // tiles DBW wd ..; random features: omega row block wf (state feature
    // blocks wf for its cos rows and RBN + wf for its sin rows), all value
    // tiles, 32-token half ts of each chunk where TS = 2
    const int wf = RF ? wave % RBN : wave % 4;
    const int wd = RF ? 0 : wave / 4;  // 0 .. WD - 1
    const int ts = RF ? wave / RBN : 0;
    auto fblock = [&](int u) LA_INLINE { return RF ? (u == 0 ? wf : RBN + wf) : FBW * wf + u; };

    // fixed rows: blockIdx = (segment, batch*head); packed sequences:
    // blockIdx = (work item of head blockIdx.y), mapped to (sequence, segment)
    int seg = blockIdx.x, bh = blockIdx.y;
    bool spare = false;
    if (a.cu_seqlens) {
        const int it = a.items[blockIdx.x];
        spare = it < 0;
        seg = spare ? 0 : it % a.P;
        bh = (spare ? 0 : it / a.P) * a.H + (int)blockIdx.y;
    }
    const int h = bh % a.H;
    const float l2l = a.lam.log2lam[h];
    const bool decay = l2l != 0.f;
    int64_t row0 = (int64_t)bh * a.N + a.n0, n_len = a.n_len;
    if (a.cu_seqlens) {
        int64_t s0, s1;
        varlen_range(a.cu_seqlens, bh / a.H, a.N, &s0, &s1);
        row0 = (int64_t)h * a.N + s0;
        n_len = s1 - s0;
    }
    // segments of cps units of a.chunk tokens (a multiple of C); the last one
    // takes whatever remains.  An empty segment stores nothing (the scan
    // reads only the segments a row has), nor, with skip_last, the one that
    // reaches the row's end (only a final state would read it).
    const int64_t cps = a.cps * (a.chunk / C);
    const int64_t NC = spare ? 0 : (n_len + C - 1) / C;
    const int64_t c_beg = (int64_t)seg * cps, c_end = (seg == a.P - 1) ? NC : min(NC, c_beg + cps);
    if (c_beg >= c_end || (a.skip_last && c_end == NC)) return;
    const T* kg = (const T*)a.k + row0 * DK;
    const T* vg = (const T*)a.v + row0 * DV;
    const uint8_t* kp = a.kpm ? a.kpm + (int64_t)(bh / a.H) * a.kpm_stride + a.n0 : nullptr;
    const Frag<T> ones = frag_ones<T>();
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // ---- random features: rows 16 wf + l16 of omega as B-operand fragments,
    // scaled by qk_scale / (2 pi) (angles in revolutions for the hardware
    // sine and cosine) and split into bf16 high and low parts
    Frag<T> om_hi[RF ? KX : 1], om_lo[RF ? KX : 1];
    if constexpr (RF) {
        const float om_scale = a.qk_scale * 0.159154943091895336f;
#pragma unroll
        for (int kx = 0; kx < KX; ++kx) {
            // k positions in natural order (8 g .. 8 g + 7), as the raw rows
            // are read below
            const float* p = a.omega + (int64_t)(16 * wf + l16) * DK + 32 * kx + 8 * g;
            const f32x4 w0 = *(const f32x4*)p * om_scale, w1 = *(const f32x4*)(p + 4) * om_scale;
            f32x4 r0, r1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r0[e] = w0[e] - (float)(bf16)w0[e];
                r1[e] = w1[e] - (float)(bf16)w1[e];
            }
            om_hi[kx] = frag_acc<T>(w0, w1);
            om_lo[kx] = frag_acc<T>(r0, r1);
        }
    }

    // ---- loads of one chunk into registers: a ragged last chunk re-reads
    // its last row for the rows past its end and zeroes them
    const bool ragged = c_end * C > n_len;
    const int64_t c_full = ragged ? c_end - 1 : c_end;
    const int n_tail = ragged ? (int)(n_len - c_full * C) : C;
    // PF register sets: chunk c is loaded into set (c - c_beg) % PF
    uint4 rk[PF][RK], rv[PF][RV];
    int mk[PF][RK];
    auto load_rows = [&](uint4* dst, const T* base, int vpr, int ld, int nreg, int n, auto tail_c) LA_INLINE {
        constexpr bool TAIL = decltype(tail_c)::value;
#pragma unroll
        for (int r = 0; r < nreg; ++r) {
            const int idx = tid + r * NT, j = idx / vpr, c4 = idx % vpr;
            if constexpr (!TAIL) {
                dst[r] = load16(base, (uint32_t)((j * ld + c4 * VEC) * sizeof(T)));
            } else {
                const uint4 val = *(const uint4*)(base + min(j, n - 1) * ld + c4 * VEC);
                const bool in = j < n;  // per component: a select of the whole vector goes through memory
                dst[r] = uint4{in ? val.x : 0u, in ? val.y : 0u, in ? val.z : 0u, in ? val.w : 0u};
            }
        }
    };
    auto load_chunk = [&](auto set_c, int64_t c, auto tail_c) LA_INLINE {
        constexpr int st = decltype(set_c)::value;
        const int64_t t0 = c * C;
        const int n = decltype(tail_c)::value ? n_tail : C;
        load_rows(rk[st], kg + t0 * DK, VPRK, DK, RK, n, tail_c);
        load_rows(rv[st], vg + t0 * DV, VPRV, DV, RV, n, tail_c);
#pragma unroll
        for (int r = 0; r < RK; ++r) {
            const int j = (tid + r * NT) / VPRK;
            mk[st][r] = kp ? (int)kp[t0 + (decltype(tail_c)::value ? min(j, n - 1) : j)] : 0;
        }
    };
    // ---- decay weights.  The chunks are visited from the segment's end to
    // its start, so that the last ones read (the segment's first chunks)
    // are the first the causal output pass reads.  Key t of the segment
    // enters with lambda^(t_last - t) (lambda^0 = 1 also for lambda = 0),
    // t_last its last token: weights only shrink along the visit, so the
    // accumulators hold the true state and the smallest weights underflow
    // to zero harmlessly.  dbase: t_last - t for the chunk's first key.
    const int64_t t_last = min(c_end * C, n_len) - 1;
    auto key_lw = [&](int64_t dist) LA_INLINE { return dist == 0 ? 0.f : (float)dist * l2l; };

    // ---- staging of one chunk into buffer b.  A key past the end of the
    // sequence or masked is dropped: its row enters as zeros (so that no
    // non-finite value of it survives) with a zero weight.
    const float rf_cexp = 0.5f * a.rf_sign * a.qk_scale * a.qk_scale;
    const float rf_cnorm = a.rf_scale;
    auto stage = [&](auto set_c, int b, int n, int64_t dbase, auto tail_c) LA_INLINE {
        constexpr bool TAIL = decltype(tail_c)::value;
        constexpr int st = decltype(set_c)::value;
        const int cg = tid % VPRK;
#pragma unroll
        for (int r = 0; r < RK; ++r) {
            const int j = (tid + r * NT) / VPRK;
            const bool drop = (TAIL && j >= n) || mk[st][r];
            const float lw = drop ? -INFINITY : (decay ? key_lw(dbase - j) : 0.f);
            const float w = __builtin_amdgcn_exp2f(lw);
            // a dropped key's row is replaced by zeros: its features are then
            // finite whatever it held, and its weight zeroes them
            const uint4 u = drop ? uint4{0u, 0u, 0u, 0u} : rk[st][r];
            if constexpr (!RF) {
                float x[VEC], p[VEC];
                unpack16(u, x, (const T*)nullptr);
#pragma unroll
                for (int e = 0; e < VEC; ++e) p[e] = phi_weighted<PHI>(x[e], w, lw);
                T* const sK = sKb(b);
                st4(sK + TK::off(j, cg * VEC), p[0], p[1], p[2], p[3]);
                st4(sK + TK::off(j, cg * VEC + 4), p[4], p[5], p[6], p[7]);
            } else {
                *(uint4*)(sKb(b) + j * XLD + cg * VEC) = u;
                float x[VEC];
                unpack16(u, x, (const T*)nullptr);
                float s2 = 0.f;
#pragma unroll
                for (int e = 0; e < VEC; ++e) s2 += x[e] * x[e];
                s2 = group_sum<VPRK>(s2);
                if (cg == 0) sWb(b)[j] = drop ? 0.f : exp_rf<T>(rf_cexp * s2) * rf_cnorm * w;
            }
        }
        T* const sV = sVb(b);
#pragma unroll
        for (int r = 0; r < RV; ++r) {
            const int idx = tid + r * NT, j = idx / VPRV, c4 = idx % VPRV;
            const uint4 u = rv[st][r];
            *(uint2*)(sV + TVL::off(j, c4 * VEC)) = uint2{u.x, u.y};
            *(uint2*)(sV + TVL::off(j, c4 * VEC + 4)) = uint2{u.z, u.w};
        }
    };

    // ---- this wave's state tiles: accS[u][c] holds S[16 fblock(u) + 4 g + r]
    // [16 (DBW wd + c) + l16]; accZ[u] holds z[16 fblock(u) + 4 g + r] in
    // every column (kept by the waves of the first value-column group)
    f32x4 accS[FBW][DBW], accZ[FBW];
#pragma unroll
    for (int u = 0; u < FBW; ++u) {
        accZ[u] = zero4;
#pragma unroll
        for (int c = 0; c < DBW; ++c) accS[u][c] = zero4;
    }

    // ---- the chunk in buffer b into this wave's tiles
    auto update = [&](int b) LA_INLINE {
        const T* const sV = sVb(b);
        if constexpr (!RF) {
            const T* const sK = sKb(b);
            Frag<T> kf[FBW][CB];
#pragma unroll
            for (int u = 0; u < FBW; ++u)
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) kf[u][kb] = ColRead<T, F, TK>::get(sK, 32 * kb, 16 * fblock(u), lane);
#pragma unroll
            for (int c = 0; c < DBW; ++c) {
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) {
                    const Frag<T> vf = ColRead<T, DV, TVL>::get(sV, 32 * kb, 16 * (DBW * wd + c), lane);
#pragma unroll
                    for (int u = 0; u < FBW; ++u) mma(accS[u][c], kf[u][kb], vf);
                }
            }
            if (wd == 0) {
#pragma unroll
                for (int u = 0; u < FBW; ++u)
#pragma unroll
                    for (int kb = 0; kb < CB; ++kb) mma(accZ[u], kf[u][kb], ones);
            }
        } else {
            const T* const sX = sKb(b);
            const float* const sW = sWb(b);
#pragma unroll
            for (int kk = 0; kk < CB / TS; ++kk) {
                const int kb = TS == 1 ? kk : ts;  // 32-token block
                // angles of omega rows 16 wf + l16 for tokens 32 kb + 16 h + 4 g + r
                f32x4 ang[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int j = 32 * kb + 16 * hh + l16;
                    ang[hh] = zero4;
#pragma unroll
                    for (int kx = 0; kx < KX; ++kx) {
                        const Frag<T> xf = frag_row16(sX, XLD, j, 32 * kx, g);
                        mma(ang[hh], xf, om_hi[kx]);
                        mma(ang[hh], xf, om_lo[kx]);
                    }
                }
                const f32x4 w0 = *(const f32x4*)(sW + 32 * kb + 4 * g);
                const f32x4 w1 = *(const f32x4*)(sW + 32 * kb + 16 + 4 * g);
                f32x4 c0, c1, s0, s1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    c0[r] = __builtin_amdgcn_cosf(ang[0][r]) * w0[r];
                    s0[r] = __builtin_amdgcn_sinf(ang[0][r]) * w0[r];
                    c1[r] = __builtin_amdgcn_cosf(ang[1][r]) * w1[r];
                    s1[r] = __builtin_amdgcn_sinf(ang[1][r]) * w1[r];
                }
                // (w phi(K))^T fragments of the cos and sin rows over this
                // 32-token block
                const Frag<T> kc = frag_acc<T>(c0, c1), ks = frag_acc<T>(s0, s1);
#pragma unroll
                for (int c = 0; c < DBW; ++c) {
                    const Frag<T> vf = ColRead<T, DV, TVL>::get(sV, 32 * kb, 16 * c, lane);
                    mma(accS[0][c], kc, vf);
                    mma(accS[1][c], ks, vf);
                }
                mma(accZ[0], kc, ones);
                mma(accZ[1], ks, ones);
            }
        }
    };

    // ---- the segment, last chunk first, one barrier per chunk: staging a
    // chunk into buffer b follows the barrier after which every wave has
    // finished reading b for the chunk before the previous one.  The next
    // chunk's loads go out as soon as the current one is staged; inside the
    // loop they are always full-chunk loads (at the segment's first chunk
    // they re-read it, in bounds and unused), so that the compiler cannot
    // merge them with the ragged chunk's zeroing, which would wait for them
    // on the spot.  A ragged chunk (the row's last) comes first.
    const std::integral_constant<int, 0> s0;
    int buf = 0;
    if (ragged) {
        load_chunk(s0, c_full, std::true_type{});
        stage(s0, buf, n_tail, t_last - c_full * C, std::true_type{});
        if (c_full > c_beg) load_chunk(s0, c_full - 1, std::false_type{});
        __syncthreads();
        update(buf);
        buf ^= 1;
    } else {
        load_chunk(s0, c_full - 1, std::false_type{});
    }
    for (int64_t c = c_full - 1; c >= c_beg; --c) {
        stage(s0, buf, C, t_last - c * C, std::false_type{});
        load_chunk(s0, max(c - 1, c_beg), std::false_type{});
        __syncthreads();
        update(buf);
        buf ^= 1;
    }

    // ---- two token splits: the second hands its tiles to the first
    if constexpr (TS > 1) {
        f32x4* const red = (f32x4*)smem;
        __syncthreads();  // every wave is done with the chunk buffers
        if (ts == 1) {
#pragma unroll
            for (int u = 0; u < FBW; ++u) {
#pragma unroll
                for (int c = 0; c < DBW; ++c) red[(wf * Cfg::TPW + u * DBW + c) * 64 + lane] = accS[u][c];
                red[(wf * Cfg::TPW + FBW * DBW + u) * 64 + lane] = accZ[u];
            }
        }
        __syncthreads();
        if (ts == 1) return;
#pragma unroll
        for (int u = 0; u < FBW; ++u) {
#pragma unroll
            for (int c = 0; c < DBW; ++c) accS[u][c] += red[(wf * Cfg::TPW + u * DBW + c) * 64 + lane];
            accZ[u] += red[(wf * Cfg::TPW + FBW * DBW + u) * 64 + lane];
        }
    }

    // ---- the segment's state (true scale)
    float* const Sd = a.S_dst + ((int64_t)seg * a.BH + bh) * a.dst_stride;
    float* const zd = a.z_dst + ((int64_t)seg * a.BH + bh) * a.dst_zstride;
#pragma unroll
    for (int u = 0; u < FBW; ++u) {
        const int f0 = 16 * fblock(u) + 4 * g;
#pragma unroll
        for (int c = 0; c < DBW; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) Sd[(int64_t)(f0 + r) * DV + 16 * (DBW * wd + c) + l16] = accS[u][c][r];
        if (wd == 0 && l16 == 0) *(f32x4*)(zd + f0) = accZ[u];
    }
}

template <int PHI, int DK, int F, int DV>
hipError_t state_launch(const FwdArgs& a, hipStream_t stream)
{
    using Cfg = StateCfg<PHI, DK, F, DV>;
    if (a.chunk % Cfg::C != 0) return hipErrorInvalidValue;  // segments must be whole chunks
    const dim3 grid(a.cu_seqlens ? (unsigned)a.G : (unsigned)a.P, a.cu_seqlens ? (unsigned)a.H : (unsigned)a.BH),
        block(Cfg::NT);
    return launch_kernel(la_state_kernel<PHI, DK, F, DV>, grid, block, stream, a);
}

}  // namespace la
