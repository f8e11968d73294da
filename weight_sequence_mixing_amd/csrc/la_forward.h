// la_forward.h -- chunked forward kernel (gfx950) for causal and non-causal
// kernelized linear attention, templated on element type, feature map and
// head sizes.  Instantiated by the la_inst_*.hip units.
//
// Method ("Attention is also an FFN", kwkr.cn/news/587576, sec. 4.1 notes and
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
// Work split.  One workgroup of NW waves owns one segment (a run of whole
// chunks) of one (batch, head) row.  The fp32 state S lives in accumulator
// registers, split by value column: wave w owns columns
// [16*DBW*w, 16*DBW*(w+1)) for all F feature rows.  Outputs are computed
// transposed, O^T = S^T phi(Q)^T + V^T P^T, so that
//   - S^T is an A operand read straight from the accumulators,
//   - the transposed score tile phi(K) phi(Q)^T that a wave holds is already
//     the B operand P^T (no LDS round trip for P), and
//   - each lane ends up with 4 consecutive output columns of one token, which
//     it stores with one 8-byte (bf16) or 16-byte (fp32) write.
// Every wave computes the (small) score tiles it needs itself.
//
// The normaliser runs on the matrix cores too: z is an accumulator tile set
// updated with an all-ones B operand (every column holds z), phi(Q) z is a
// product with z broadcast as the A operand, and the row sums of P are a
// product with an all-ones A operand -- so numerator and denominator see the
// same bf16-rounded operands.
//
// Decay without a per-chunk multiply of the state: the true state is D * S^
// with a scalar D that is the same in every thread.  A chunk multiplies D by
// lambda^n and adds its keys with weights lambda^(n-1-j) / D; S^ (and z^) are
// rescaled only when D would fall below 2^-60, which for lambda = 0 is every
// chunk (then the weights are lambda^(n-1-j) themselves and 0^0 = 1).
//
// Per chunk, the tiles phi(Q), phi(K), lambda-weighted phi(K) and V are staged
// row-major in LDS (see TileL in la_device.h); products that contract over
// the token axis read them with transposing LDS reads.  The tiles are double
// buffered so that a chunk needs one barrier; the next chunk's q, k, v are
// loaded into registers while the current one is computed.
//
// Modes: MODE_LOCAL   segment-local state from a zero start (pass 1),
//        MODE_CAUSAL  outputs of a segment from its carried-in state (pass 3),
//        MODE_QUERY   non-causal outputs for a fixed state.
#pragma once

#include <type_traits>

#include "la_device.h"
#include "la_internal.h"

namespace la {

// The kernel body is written as lambdas over the workgroup's registers; each
// must be inlined (a call would move the captured arrays to scratch memory).
#define LA_INLINE __attribute__((always_inline))

// Tokens per chunk.  32 for every shape: against 64 it halves the LDS tiles
// and the registers of the staged chunk (the d = 64 output kernel fits three
// waves per SIMD), and the outputs of a chunk depend on fewer score tiles;
// measured faster for d = 64 and d = 128.
template <class T, int PHI>
constexpr int chunk_len(int F) {
    return 32;
}

// The causal output pass runs la_out_kernel (64-token chunks) for bf16 inputs
// with elu+1, ReLU or random features.
template <class T, int PHI>
constexpr bool query_split_output() {
    return sizeof(T) == 2 && (PHI == LA_PHI_ELU1 || PHI == LA_PHI_RELU || PHI == LA_PHI_TRIG_RF);
}

// Tokens per planning chunk (the unit in which a call cuts segments): 64 where
// the causal output pass is la_out_kernel; the kernel's own chunk length
// elsewhere.
template <class T, int PHI>
constexpr int plan_chunk(int F) {
    return query_split_output<T, PHI>() ? 64 : chunk_len<T, PHI>(F);
}

// log2 of the smallest pending decay factor before the state is rescaled
constexpr float kLog2MinScale = -60.f;

// Chunks whose loads are in flight while one chunk is computed.  The d = 128
// output pass needs more than 256 registers per lane, so one workgroup holds a
// compute unit alone and its own prefetch is all that covers HBM latency:
// one 24 KB chunk ahead leaves the pass latency-bound.  Deeper prefetch there
// costs registers but no occupancy.
#ifndef LA_PREFETCH_DEPTH_WIDE
#define LA_PREFETCH_DEPTH_WIDE 1
#endif
template <int PHI, int F, int DV, int MODE>
constexpr int prefetch_depth()
{
    return (MODE == MODE_CAUSAL && PHI != LA_PHI_TRIG_RF && F >= 128 && DV >= 128) ? LA_PREFETCH_DEPTH_WIDE : 1;
}

// Calls f(integral_constant<int, I>) for I = B .. E-1 in order until one returns true.
template <int I, int E, class Fn>
__device__ __forceinline__ bool static_until(Fn&& f)
{
    if constexpr (I >= E) {
        return false;
    } else {
        if (f(std::integral_constant<int, I>{})) return true;
        return static_until<I + 1, E>(f);
    }
}

template <class T, int PHI, int DK, int F, int DV, int C, int NW, int MODE>
struct FwdCfg {
    static constexpr int NT = NW * 64;
    static constexpr int PF = prefetch_depth<PHI, F, DV, MODE>();
    static constexpr int VEC = 16 / (int)sizeof(T);
    static constexpr bool RF = PHI == LA_PHI_TRIG_RF;
    static constexpr int M = RF ? F / 2 : 0;
    static constexpr int QB = C / 16;
    static constexpr int FB = F / 16;
    static constexpr int DB = DV / 16;
    static constexpr int DBW = DB / NW;
    static constexpr int ZB = FB / NW;  // z tiles per wave
    static constexpr int XLD = DK + 4;  // raw q/k rows of the random-feature prologue
    static constexpr bool NEED_Q = MODE != MODE_LOCAL;
    static constexpr bool NEED_K = MODE != MODE_QUERY;
    static constexpr bool NEED_KROW = MODE == MODE_CAUSAL;
    // feature tiles are double buffered for elu+1; the random-feature prologue
    // has a barrier of its own before it writes them, so one buffer suffices
    static constexpr int NBF = RF ? 1 : 2;
    static constexpr int TQ = C * TileL<T, F>::STRIDE;   // elements of a feature tile
    static constexpr int TV = C * TileL<T, DV>::STRIDE;  // elements of a value tile
    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t SZ_Q = NEED_Q ? size_t(NBF) * TQ * sizeof(T) : 0;
    static constexpr size_t OFF_K = al(OFF_Q + SZ_Q);
    static constexpr size_t SZ_K = NEED_KROW ? size_t(NBF) * TQ * sizeof(T) : 0;
    static constexpr size_t OFF_KW = al(OFF_K + SZ_K);
    static constexpr size_t SZ_KW = NEED_K ? size_t(NBF) * TQ * sizeof(T) : 0;
    static constexpr size_t OFF_V = al(OFF_KW + SZ_KW);
    static constexpr size_t SZ_V = NEED_K ? size_t(2) * TV * sizeof(T) : 0;
    static constexpr size_t OFF_XQ = al(OFF_V + SZ_V);
    static constexpr size_t SZ_XQ = (RF && NEED_Q) ? size_t(C) * XLD * sizeof(T) : 0;
    static constexpr size_t OFF_XK = al(OFF_XQ + SZ_XQ);
    static constexpr size_t SZ_XK = (RF && NEED_K) ? size_t(C) * XLD * sizeof(T) : 0;
    static constexpr size_t OFF_XN = al(OFF_XK + SZ_XK);
    static constexpr size_t SZ_XN = RF ? size_t(2) * C * sizeof(float) : 0;
    // Random features with bf16 inputs: omega enters the matrix cores as bf16
    // high and low parts (SPLIT).  z is published after each chunk as bf16
    // operand values and read where it is used (ZB16), and for F <= 128
    // omega's operand fragments live in LDS instead of registers (OMLDS),
    // which lets two workgroups share a compute unit.  At F = 256 the LDS
    // tiles alone allow one workgroup per compute unit; there the fragments
    // stay in registers (measured faster than LDS reads).
    static constexpr bool SPLIT = RF && sizeof(T) == 2;
    static constexpr bool OMLDS = SPLIT && F <= 128;
    static constexpr bool ZB16 = SPLIT && NEED_Q && NEED_K;
    // the normaliser z after each chunk, double buffered (MODE_CAUSAL; fp32,
    // or bf16 with ZB16)
    static constexpr size_t OFF_Z = al(OFF_XN + SZ_XN);
    static constexpr size_t SZ_Z = (NEED_Q && NEED_K) ? size_t(2) * F * (ZB16 ? 2 : sizeof(float)) : 0;
    // omega fragments: [row block][k block][high, low][lane], 16 bytes each
    static constexpr size_t OFF_OM = al(OFF_Z + SZ_Z);
    static constexpr size_t SZ_OM = OMLDS ? size_t(M / 16) * (DK / 32) * 2 * 64 * 16 : 0;
    static constexpr size_t TOTAL = al(OFF_OM + SZ_OM);
    // random features: each wave computes the feature blocks of one 16-token
    // block (ib = wave % QB) for TPW 16-row blocks of omega, whose operand
    // fragments it keeps in registers
    static constexpr int KX = DK / 32;
    static constexpr int TPW = RF ? (M / 16) * QB / NW : 1;
    // waves per SIMD the register allocation must allow: two where the state
    // is small (d_k, d_v <= 64 and F <= 64), so that two workgroups share a CU
    static constexpr int MIN_WAVES = (F <= 64 && DV <= 64) ? 2 : 1;

    static_assert(C % 32 == 0 && C >= 32, "chunk must be a multiple of 32");
    static_assert(F % 64 == 0 && DV % 64 == 0 && DK % 32 == 0, "head sizes");
    static_assert(DBW >= 1 && DB % NW == 0, "value columns must split over the waves");
    static_assert(ZB >= 1 && FB % NW == 0, "z tiles must split over the waves");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    static_assert(!RF || ((M / 16) * QB % NW == 0 && NW % QB == 0), "random-feature tiles must split over the waves");
};

// OUTF32: y is fp32 (bf16 inputs with fp32 outputs).  A template argument, not
// a runtime branch: branches around the output stores make the compiler wait
// for every earlier store before the next chunk's loaded data is used.
template <class T, int PHI, int DK, int F, int DV, int C, int NW, int MODE, bool OUTF32>
__global__ void __launch_bounds__(NW * 64, (FwdCfg<T, PHI, DK, F, DV, C, NW, MODE>::MIN_WAVES))
la_fwd_kernel(const FwdArgs a)
{
    using Cfg = FwdCfg<T, PHI, DK, F, DV, C, NW, MODE>;
    constexpr int NT = Cfg::NT, VEC = Cfg::VEC, M = Cfg::M, QB = Cfg::QB, FB = Cfg::FB;
    constexpr int DBW = Cfg::DBW, XLD = Cfg::XLD, TQ = Cfg::TQ, TV = Cfg::TV, ZB = Cfg::ZB;
    constexpr bool RF = Cfg::RF;
    constexpr int KB = F / 32;                  // 32-wide feature blocks
    constexpr int CB = C / 32;                  // 32-wide token blocks
    constexpr int VPRQ = DK / VEC;              // 16-byte vectors per q/k row
    constexpr int VPRV = DV / VEC;              // 16-byte vectors per v row
    constexpr int VQ = C * VPRQ, VV = C * VPRV; // vectors per tile
    constexpr int RQ = (VQ + NT - 1) / NT, RV = (VV + NT - 1) / NT;
    static_assert(VQ % NT == 0 && VV % NT == 0, "tiles must split evenly over threads");
    using TF = TileL<T, F>;
    using TVL = TileL<T, DV>;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    T* const sQ0 = (T*)(smem + Cfg::OFF_Q);
    T* const sK0 = (T*)(smem + Cfg::OFF_K);
    T* const sKw0 = (T*)(smem + Cfg::OFF_KW);
    T* const sV0 = (T*)(smem + Cfg::OFF_V);
    T* const sXq = (T*)(smem + Cfg::OFF_XQ);
    T* const sXk = (T*)(smem + Cfg::OFF_XK);
    float* const sXn = (float*)(smem + Cfg::OFF_XN);
    float* const sZ = (float*)(smem + Cfg::OFF_Z);
    bf16* const sZb = (bf16*)(smem + Cfg::OFF_Z);
    Frag<T>* const sOm = (Frag<T>*)(smem + Cfg::OFF_OM);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    // fixed rows: blockIdx = (segment, batch*head); packed sequences:
    // blockIdx = (work item of head blockIdx.y), mapped to (sequence, segment)
    int seg = blockIdx.x, bh = blockIdx.y;
    bool spare = false;  // a packed-sequence item past the last: no work, no stores
    if (a.cu_seqlens) {
        const int it = a.items[blockIdx.x];  // b * P + s, or -1
        spare = it < 0;
        seg = spare ? 0 : it % a.P;
        bh = (spare ? 0 : it / a.P) * a.H + (int)blockIdx.y;
    }
    const int h = bh % a.H;
    const float l2l = (MODE == MODE_QUERY) ? 0.f : a.lam.log2lam[h];
    const bool decay = l2l != 0.f;  // uniform over the workgroup
    // token range of this row: [n0, n0 + n_len) of row bh, or the packed
    // sequence bh / H of head row h
    int64_t row0 = (int64_t)bh * a.N + a.n0, n_len = a.n_len;
    if (a.cu_seqlens) {
        int64_t s0, s1;
        varlen_range(a.cu_seqlens, bh / a.H, a.N, &s0, &s1);
        row0 = (int64_t)h * a.N + s0;
        n_len = s1 - s0;
    }
    // segments of cps units of a.chunk tokens (a multiple of C); the last one
    // takes whatever remains
    const int64_t cps = a.chunk > C ? a.cps * (a.chunk / C) : a.cps;
    const int64_t NC = spare ? 0 : (n_len + C - 1) / C;
    const int64_t c_beg = (int64_t)seg * cps, c_end = (seg == a.P - 1) ? NC : min(NC, c_beg + cps);
    // an empty segment (an empty packed sequence) has nothing to compute and
    // nothing to store, unless it carries a state through
    if (c_beg >= c_end) {
        if constexpr (MODE != MODE_CAUSAL) return;
        else if (!a.S_dst || spare) return;
    }
    // with skip_last, the segment that reaches the row's end (whose local
    // state only a final state would read)
    if constexpr (MODE == MODE_LOCAL)
        if (a.skip_last && c_end == NC) return;
    const T* qg = (const T*)a.q + row0 * DK;
    const T* kg = (const T*)a.k + row0 * DK;
    const T* vg = (const T*)a.v + row0 * DV;
    // key padding mask of this row (keys only)
    const uint8_t* kp = (Cfg::NEED_K && a.kpm) ? a.kpm + (int64_t)(bh / a.H) * a.kpm_stride + a.n0 : nullptr;
    const float qs = a.qk_scale;
    const Frag<T> ones = frag_ones<T>();

    // ---- decay tables of this lane (lambda is fixed per workgroup).  Score
    // element (i = 16 ib + l16, j = 16 jb + 4 g + r) is weighted by lambda^(i-j):
    //   jb == ib: m0[r] = lambda^(l16-4g-r), or 0 above the diagonal;
    //   jb <  ib: m1[r] * lambda^(16 (ib-jb-1)), m1[r] = lambda^(16+l16-4g-r)
    // (every exponent is >= 0, so nothing overflows for small lambda).
    // Query row i reads the carried state with lambda^(i+1) = lq1 * lambda^(16 ib).
    float m0[4], m1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = l16 - 4 * g - r;
        m0[r] = e < 0 ? 0.f : (decay ? lam_pow(l2l, e) : 1.f);
        m1[r] = decay ? lam_pow(l2l, 16 + e) : 1.f;
    }
    const float lq1 = decay ? lam_pow(l2l, l16 + 1) : 1.f;

    // ---- random-feature directions as operand fragments, in registers for
    // the whole workgroup: rows 16 rb.. of omega (rb = wave / QB + (NW / QB) u),
    // as bf16 high and low parts for bf16 inputs (omega = hi + lo to 16 bits)
    constexpr int TPW = Cfg::TPW, KX = Cfg::KX;
    // bf16 inputs: omega is scaled by qk_scale / (2 pi) before the split, so
    // that the products are the angles in revolutions, the unit of the
    // hardware sine and cosine; fp32 inputs keep radians for sincosf
    constexpr bool REV = sizeof(T) == 2;
    const float om_scale = REV ? qs * 0.159154943091895336f : 1.f;
    Frag<T> om_hi[Cfg::OMLDS ? 1 : TPW][KX], om_lo[(Cfg::SPLIT && !Cfg::OMLDS) ? TPW : 1][KX];
    if constexpr (RF) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int rb = wave / QB + (NW / QB) * u;
#pragma unroll
            for (int kb = 0; kb < KX; ++kb) {
                const float* p = a.omega + (int64_t)(16 * rb + l16) * DK + 32 * kb + 4 * g;
                const f32x4 w0 = *(const f32x4*)p * om_scale, w1 = *(const f32x4*)(p + 16) * om_scale;
                const Frag<T> hi = frag_acc<T>(w0, w1);
                if constexpr (Cfg::SPLIT) {
                    f32x4 r0, r1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        r0[e] = w0[e] - (float)(bf16)w0[e];
                        r1[e] = w1[e] - (float)(bf16)w1[e];
                    }
                    const Frag<T> lo = frag_acc<T>(r0, r1);
                    if constexpr (Cfg::OMLDS) {
                        // waves of the same row blocks hold the same
                        // fragments; one of them stores (read after the
                        // first barrier)
                        if (wave % QB == 0) {
                            sOm[((rb * KX + kb) * 2 + 0) * 64 + lane] = hi;
                            sOm[((rb * KX + kb) * 2 + 1) * 64 + lane] = lo;
                        }
                    } else {
                        om_hi[u][kb] = hi;
                        om_lo[u][kb] = lo;
                    }
                } else {
                    om_hi[u][kb] = hi;
                }
            }
        }
    }
    // operand fragment of omega rows 16 rb.. (high or low part)
    auto omega_frag = [&](int u, int kb, int part) LA_INLINE {
        if constexpr (Cfg::OMLDS) {
            const int rb = wave / QB + (NW / QB) * u;
            return sOm[((rb * KX + kb) * 2 + part) * 64 + lane];
        } else {
            return part ? om_lo[(Cfg::SPLIT && !Cfg::OMLDS) ? u : 0][kb] : om_hi[u][kb];
        }
    };

    // ---- global -> register prefetch of one chunk.  A full chunk is read at
    // fixed per-thread offsets from a uniform base.  In a ragged last chunk,
    // rows past the end re-read the last valid row (always in bounds) and are
    // replaced by zeros in registers, so the loads stay unconditional.
    const bool ragged = c_end > c_beg && c_end * C > n_len;
    const int64_t c_full = ragged ? c_end - 1 : c_end;
    const int n_tail = ragged ? (int)(n_len - c_full * C) : C;
    // PF register sets, each holding one chunk's loads (set s, chunk c: any
    // chunk with c - c_beg = s mod PF)
    constexpr int PF = Cfg::PF;
    uint4 rq[PF][Cfg::NEED_Q ? RQ : 1], rk[PF][Cfg::NEED_K ? RQ : 1], rv[PF][Cfg::NEED_K ? RV : 1];
    int mk[PF][Cfg::NEED_K ? RQ : 1];  // mask bytes of this thread's key rows
    auto load_rows = [&](uint4* dst, const T* base, int vpr, int ld, int nreg, int n, auto tail_c) LA_INLINE {
        constexpr bool TAIL = decltype(tail_c)::value;
#pragma unroll
        for (int r = 0; r < nreg; ++r) {
            const int idx = tid + r * NT, j = idx / vpr, c4 = idx % vpr;
            if constexpr (!TAIL) {
                dst[r] = *(const uint4*)(base + j * ld + c4 * VEC);
            } else {
                const uint4 val = *(const uint4*)(base + min(j, n - 1) * ld + c4 * VEC);
                const bool in = j < n;  // per component: a select of the whole vector goes through memory
                dst[r] = uint4{in ? val.x : 0u, in ? val.y : 0u, in ? val.z : 0u, in ? val.w : 0u};
            }
        }
    };
    // chunk c into register set `set_c`: a full one (c < c_full) or, with
    // TAIL, the ragged last one
    auto load_chunk = [&](auto set_c, int64_t c, auto tail_c) LA_INLINE {
        constexpr int st = decltype(set_c)::value;
        const int64_t t0 = c * C;
        const int n = decltype(tail_c)::value ? n_tail : C;
        if constexpr (Cfg::NEED_Q) load_rows(rq[st], qg + t0 * DK, VPRQ, DK, RQ, n, tail_c);
        if constexpr (Cfg::NEED_K) {
            load_rows(rk[st], kg + t0 * DK, VPRQ, DK, RQ, n, tail_c);
            load_rows(rv[st], vg + t0 * DV, VPRV, DV, RV, n, tail_c);
#pragma unroll
            for (int r = 0; r < RQ; ++r) {
                const int j = (tid + r * NT) / VPRQ;
                mk[st][r] = kp ? (int)kp[t0 + (decltype(tail_c)::value ? min(j, n - 1) : j)] : 0;
            }
        }
    };

    // the first chunks' loads go out before the carried state is read, so
    // that the memory latencies overlap.  With PF > 1 the sets are filled
    // with chunks c_beg .. c_beg + PF - 1; a chunk past the last full one is
    // replaced by the last full one (loads that hit in the cache and are
    // never used), so that every load of the chunk loop is unconditional.
    if (c_beg < c_full) {
        static_until<0, PF>([&](auto s_c) LA_INLINE {
            load_chunk(s_c, min(c_beg + (int64_t)decltype(s_c)::value, c_full - 1), std::false_type{});
            return false;
        });
    } else if (c_beg < c_end) {
        load_chunk(std::integral_constant<int, 0>{}, c_beg, std::true_type{});
    }

    // ---- carried state: S tiles (fb, this wave's d-blocks) and this wave's z
    // tiles fb = ZB * wave + u; lane (g, l16) of a z tile holds
    // z[16 fb + 4 g + r] in every column
    f32x4 accS[FB][DBW], accZ[ZB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int t = 0; t < DBW; ++t) accS[fb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < ZB; ++u) accZ[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    // z as an operand fragment (A operand of z phi(Q)^T, z in every row)
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    Frag<T> zf[Cfg::ZB16 ? 1 : KB];
#pragma unroll
    for (int kb = 0; kb < (Cfg::ZB16 ? 1 : KB); ++kb) zf[kb] = frag_acc<T>(zero4, zero4);
    if constexpr (MODE != MODE_LOCAL) {
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
            }
#pragma unroll
            for (int u = 0; u < ZB; ++u) accZ[u] = *(const f32x4*)(zb + 16 * (ZB * wave + u) + 4 * g);
            if constexpr (Cfg::NEED_Q && !Cfg::ZB16) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    zf[kb] = frag_acc<T>(*(const f32x4*)(zb + 32 * kb + 4 * g), *(const f32x4*)(zb + 32 * kb + 16 + 4 * g));
            }
        }
    }
    // ZB16: the carried-in z goes to the slot the first chunk reads (1)
    auto publish_z = [&](int par) LA_INLINE {
        if (l16 == 0) {
#pragma unroll
            for (int u = 0; u < ZB; ++u) {
                if constexpr (Cfg::ZB16) {
                    st4(sZb + par * F + 16 * (ZB * wave + u) + 4 * g, accZ[u][0], accZ[u][1], accZ[u][2], accZ[u][3]);
                } else {
                    *(f32x4*)(sZ + par * F + 16 * (ZB * wave + u) + 4 * g) = accZ[u];
                }
            }
        }
    };
    if constexpr (Cfg::ZB16) publish_z(1);
    // S as operand fragments (A operands of S^T phi(Q)^T)
    Frag<T> sf[KB][DBW];
    auto convert_state = [&]() LA_INLINE {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < DBW; ++t) sf[kb][t] = frag_acc<T>(accS[2 * kb][t], accS[2 * kb + 1][t]);
    };
    // z after the previous chunk, published in LDS by the waves that own it
    auto read_z = [&](int par) LA_INLINE {
        if constexpr (!Cfg::ZB16) {
            const float* zs = sZ + par * F;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                zf[kb] = frag_acc<T>(*(const f32x4*)(zs + 32 * kb + 4 * g), *(const f32x4*)(zs + 32 * kb + 16 + 4 * g));
        }
    };
    if constexpr (Cfg::NEED_Q) convert_state();
    float log2D = 0.f;  // the true state is 2^log2D times the accumulators

    // raw 16-byte vector -> row-major value tile (no conversion)
    auto put_raw = [&](T* tile, int row, int col, const uint4& u) LA_INLINE {
        if constexpr (sizeof(T) == 2) {
            *(uint2*)(tile + TVL::off(row, col)) = uint2{u.x, u.y};
            *(uint2*)(tile + TVL::off(row, col + 4)) = uint2{u.z, u.w};
        } else {
            *(uint4*)(tile + TVL::off(row, col)) = u;
        }
    };
    // VEC floats -> row-major feature tile (rounded to T)
    auto put_feat = [&](T* tile, int row, int col, const float* p) LA_INLINE {
#pragma unroll
        for (int e = 0; e < VEC; e += 4) st4(tile + TF::off(row, col + e), p[e], p[e + 1], p[e + 2], p[e + 3]);
    };

    // lambda^k / 2^kw_l2 with lambda^0 = 1 also for lambda = 0
    auto key_weight = [&](int k, float kw_l2) LA_INLINE {
        return k == 0 ? __builtin_amdgcn_exp2f(-kw_l2) : __builtin_amdgcn_exp2f((float)k * l2l - kw_l2);
    };

    // ---- staging of one chunk from registers.  elu+1: the feature map and
    // the weighted keys; random features: raw rows and their squared norms.
    // kw_l2: log2 of the key weight of token 0 relative to lambda^(n-1-j),
    // i.e. weight_j = 2^((n-1-j) log2 lambda - kw_l2) (kw_l2 = 0 after a rescale).
    // TAIL (a std::bool_constant): the chunk is a ragged last chunk.  Query
    // rows past its end need no masking: each feeds only its own output row,
    // which is never stored.  Key rows past the end must not reach the state.
    auto stage = [&](auto set_c, int buf, int n, float kw_l2, auto tail_c) LA_INLINE {
        constexpr int st = decltype(set_c)::value;
        constexpr bool TAIL = decltype(tail_c)::value;
        T* const sQ = sQ0 + (RF ? 0 : buf * TQ);
        T* const sK = sK0 + (RF ? 0 : buf * TQ);
        T* const sKw = sKw0 + (RF ? 0 : buf * TQ);
        T* const sV = sV0 + buf * TV;
        const int cg = tid % VPRQ;
        if constexpr (Cfg::NEED_Q) {
#pragma unroll
            for (int r = 0; r < RQ; ++r) {
                const int idx = tid + r * NT, j = idx / VPRQ;
                float x[VEC];
                unpack16(rq[st][r], x, (const T*)nullptr);
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
                    for (int e = 0; e < VEC; ++e) p[e] = phi_elem<T, PHI>(x[e]);
                    put_feat(sQ, j, cg * VEC, p);
                }
            }
        }
        if constexpr (Cfg::NEED_K) {
#pragma unroll
            for (int r = 0; r < RQ; ++r) {
                const int idx = tid + r * NT, j = idx / VPRQ;
                float x[VEC];
                unpack16(rk[st][r], x, (const T*)nullptr);
                if constexpr (RF) {
                    float s2 = 0.f;
#pragma unroll
                    for (int e = 0; e < VEC; e += 4) {
                        st4(sXk + j * XLD + cg * VEC + e, x[e], x[e + 1], x[e + 2], x[e + 3]);
                        s2 += x[e] * x[e] + x[e + 1] * x[e + 1] + x[e + 2] * x[e + 2] + x[e + 3] * x[e + 3];
                    }
                    s2 = wave_sum_xor(s2, 1, VPRQ / 2);
                    // a padded key is marked by a negative norm
                    if (cg == 0) sXn[C + j] = mk[st][r] ? -1.f : s2;
                } else {
                    float p[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) p[e] = phi_elem<T, PHI>(x[e]);
                    if ((TAIL && j >= n) || mk[st][r]) {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) p[e] = 0.f;
                    }
                    if (!decay) {
                        // unweighted keys serve the scores and the state update
                        put_feat(Cfg::NEED_KROW ? sK : sKw, j, cg * VEC, p);
                    } else {
                        if constexpr (Cfg::NEED_KROW) put_feat(sK, j, cg * VEC, p);
                        const float w = (TAIL && j >= n) ? 0.f : key_weight(n - 1 - j, kw_l2);
                        float pw[VEC];
#pragma unroll
                        for (int e = 0; e < VEC; ++e) pw[e] = p[e] * w;
                        put_feat(sKw, j, cg * VEC, pw);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < RV; ++r) {
                const int idx = tid + r * NT, j = idx / VPRV, c4 = idx % VPRV;
                put_raw(sV, j, c4 * VEC, rv[st][r]);
            }
        }
    };

    // ---- random features on the matrix cores: U^T = omega x^T, then cos/sin,
    // written row-major into the feature tiles
    auto rf_features = [&](int n, float kw_l2) LA_INLINE {
        if constexpr (RF) {
            const float cnorm = a.rf_scale;
            constexpr int NPASS = (Cfg::NEED_Q ? 1 : 0) + (Cfg::NEED_K ? 1 : 0);
            const int i = 16 * (wave % QB) + l16;  // this lane's token
#pragma unroll
            for (int pass = 0; pass < NPASS; ++pass) {
                const bool isq = Cfg::NEED_Q && pass == 0;
                const T* sX = isq ? sXq : sXk;
                const float* xn = sXn + (isq ? 0 : C);
                Frag<T> xf[KX];
#pragma unroll
                for (int kb = 0; kb < KX; ++kb) xf[kb] = frag_rm(sX, XLD, i, 32 * kb, g);
                const bool use = i < n && (isq || !(xn[i] < 0.f));  // not past the end, not padded
                const float cfac = use ? exp_rf<T>(a.rf_sign * 0.5f * qs * qs * xn[i]) * cnorm : 0.f;
                // prefactor of the weighted keys (the key weight folded in)
                const float cw = decay ? key_weight(n - 1 - i, kw_l2) * cfac : cfac;
#pragma unroll
                for (int u = 0; u < TPW; ++u) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < KX; ++kb) {
                        mma(acc, omega_frag(u, kb, 0), xf[kb]);
                        if constexpr (Cfg::SPLIT) mma(acc, omega_frag(u, kb, 1), xf[kb]);
                    }
                    // acc[r] = (omega x_i)_{f0+r} with f0 = 16 rb + 4 g
                    const int f0 = 16 * (wave / QB + (NW / QB) * u) + 4 * g;
                    float cs[4], sn[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if constexpr (REV) {
                            sn[r] = __builtin_amdgcn_sinf(acc[r]);
                            cs[r] = __builtin_amdgcn_cosf(acc[r]);
                        } else {
                            sincos_rf<T>(qs * acc[r], &sn[r], &cs[r]);
                        }
                    }
                    auto put = [&](T* tile, float f) LA_INLINE {
                        st4(tile + TF::off(i, f0), f * cs[0], f * cs[1], f * cs[2], f * cs[3]);
                        st4(tile + TF::off(i, M + f0), f * sn[0], f * sn[1], f * sn[2], f * sn[3]);
                    };
                    if (isq) {
                        put(sQ0, cfac);
                    } else {
                        // without decay the unweighted key tile serves both
                        // the scores and the state update
                        if constexpr (Cfg::NEED_KROW) put(sK0, cfac);
                        if (!Cfg::NEED_KROW || decay) put(sKw0, cw);
                    }
                }
            }
        }
    };

    // ---- outputs and state update of one staged chunk.  dscale: 2^log2D of
    // the state the chunk reads; rescale: factor applied to the accumulators
    // before this chunk's keys are added (1 when none).
    auto compute = [&](int buf, int n, int64_t t0, float dscale, bool do_rescale, float rescale, int zpar, auto tail_c) LA_INLINE {
        constexpr bool TAIL = decltype(tail_c)::value;
        const T* const sQ = sQ0 + (RF ? 0 : buf * TQ);
        const T* const sK = sK0 + (RF ? 0 : buf * TQ);
        const T* const sKw = (Cfg::NEED_KROW && !decay) ? sK : sKw0 + (RF ? 0 : buf * TQ);
        const T* const sV = sV0 + buf * TV;
        // V column fragments: A operand of V^T P^T and B operand of the state update
        Frag<T> vf[Cfg::NEED_K ? CB : 1][DBW];
        if constexpr (Cfg::NEED_K) {
#pragma unroll
            for (int kb = 0; kb < CB; ++kb)
#pragma unroll
                for (int t = 0; t < DBW; ++t) vf[kb][t] = ColRead<T, DV>::get(sV, 32 * kb, 16 * (wave * DBW + t), lane);
        }
        if constexpr (Cfg::NEED_Q) {
            const float eps = a.eps;
#pragma unroll
            for (int ib = 0; ib < QB; ++ib) {
                const int i = 16 * ib + l16;
                const float lqi = decay ? lq1 * lam_pow(l2l, 16 * ib) : 1.f;
                Frag<T> qf[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) qf[kb] = lds_frag_row<T, F>(sQ, i, kb, g);
                // phi(q_i).z (every row of the tile holds it)
                f32x4 dq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    if constexpr (Cfg::ZB16) {
                        const bf16* zs = sZb + (zpar ^ 1) * F + 32 * kb + 4 * g;
                        mma(dq, frag2(zs, zs + 16), qf[kb]);
                    } else {
                        mma(dq, zf[kb], qf[kb]);
                    }
                }
                float den = dq[0];
                Frag<T> pf[CB];
                if constexpr (MODE == MODE_CAUSAL) {
                    // scores of query block ib against key blocks jb <= ib, as P^T fragments
                    f32x4 pt[2 * CB];
#pragma unroll
                    for (int jb = 0; jb < 2 * CB; ++jb) {
                        pt[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (jb <= ib) {
#pragma unroll
                            for (int kb = 0; kb < KB; ++kb)
                                mma(pt[jb], lds_frag_row<T, F>(sK, 16 * jb + l16, kb, g), qf[kb]);
                            if (jb == ib) {
#pragma unroll
                                for (int r = 0; r < 4; ++r) pt[jb][r] *= m0[r];
                            } else if (decay) {
                                const float dj = lam_pow(l2l, 16 * (ib - jb - 1));
#pragma unroll
                                for (int r = 0; r < 4; ++r) pt[jb][r] *= m1[r] * dj;
                            }
                        }
                    }
                    f32x4 rs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < CB; ++kb) {
                        pf[kb] = frag_acc<T>(pt[2 * kb], pt[2 * kb + 1]);
                        if (2 * kb <= ib) mma(rs, ones, pf[kb]);
                    }
                    den = rs[0] + lqi * dscale * den;
                }
                const float inv = fast_rcp(den + eps);
                const float sc = (MODE == MODE_CAUSAL) ? lqi * dscale * inv : inv;
                const int64_t yrow = row0 + t0 + i;
#pragma unroll
                for (int t = 0; t < DBW; ++t) {
                    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) mma(o, sf[kb][t], qf[kb]);
                    if constexpr (MODE == MODE_CAUSAL) {
                        // o = (lambda^(i+1) D S^T phi(q) + V^T P^T) / den
                        o *= sc;
                        f32x4 oi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kb = 0; kb < CB; ++kb)
                            if (2 * kb <= ib) mma(oi, vf[kb][t], pf[kb]);
                        o += oi * inv;
                    } else {
                        o *= sc;
                    }
                    if (!TAIL || i < n) {
                        const int64_t yo = yrow * DV + 16 * (wave * DBW + t) + 4 * g;
                        if constexpr (OUTF32) st4((float*)a.y + yo, o[0], o[1], o[2], o[3]);
                        else st4((T*)a.y + yo, o[0], o[1], o[2], o[3]);
                    }
                }
            }
        }
        // state carry: S^ <- S^ + (w phi(K))^T V, z^ <- z^ + (w phi(K))^T 1
        if constexpr (Cfg::NEED_K) {
            if (do_rescale) {
#pragma unroll
                for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                    for (int t = 0; t < DBW; ++t) accS[fb][t] *= rescale;
#pragma unroll
                for (int u = 0; u < ZB; ++u) accZ[u] *= rescale;
            }
#pragma unroll
            for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) {
                    const Frag<T> kf = ColRead<T, F>::get(sKw, 32 * kb, 16 * fb, lane);
#pragma unroll
                    for (int t = 0; t < DBW; ++t) mma(accS[fb][t], kf, vf[kb][t]);
                }
            }
            // z: this wave's feature blocks only (a column offset, no branch)
#pragma unroll
            for (int u = 0; u < ZB; ++u)
#pragma unroll
                for (int kb = 0; kb < CB; ++kb)
                    mma(accZ[u], ColRead<T, F>::get(sKw, 32 * kb, 16 * (ZB * wave + u), lane), ones);
            if constexpr (Cfg::NEED_Q) {
                convert_state();
                // publish z for the next chunk (read after its barrier)
                publish_z(zpar);
            }
        }
    };

    // ---- main loop over the segment's chunks.  The loop is rotated: an
    // iteration issues the next chunk's loads, computes the staged chunk and
    // then stages the next one, so that every load is consumed in the
    // iteration that issued it.  (A load consumed across the back edge, after
    // the output stores, is waited for with vmcnt(0), i.e. after the stores.)
    // The ragged last chunk of the sequence, if any, is loaded unprefetched and
    // computed after the loop, so that the loop's stores are unconditional.

    // decay bookkeeping of the next chunk, in chunk order (uniform): the
    // pending factor 2^log2D * lambda^n and the key-weight offset
    struct Dec { float dscale, rescale, kw_l2; bool do_rescale; };
    auto book = [&](int n) LA_INLINE {
        Dec d = {decay ? exp2f(log2D) : 1.f, 1.f, 0.f, false};
        if (decay) {
            const float cand = log2D + (float)n * l2l;
            if (cand >= kLog2MinScale) {
                d.kw_l2 = cand;
                log2D = cand;
            } else {
                d.do_rescale = true;
                d.rescale = exp2f(cand);  // 0 for lambda = 0
                log2D = 0.f;
            }
        }
        return d;
    };
    // barrier, features (random features), carried z, outputs and state
    auto finish = [&](int64_t c, int n, const Dec& d, auto tail_c) LA_INLINE {
        const int buf = (int)((c - c_beg) & 1);
        __syncthreads();
        if constexpr (RF) {
            rf_features(n, d.kw_l2);
            __syncthreads();
        }
        if constexpr (Cfg::NEED_Q && Cfg::NEED_K) {
            if (c > c_beg) read_z(buf ^ 1);
        }
        compute(buf, n, c * C, d.dscale, d.do_rescale, d.rescale, buf, tail_c);
    };

    using S0 = std::integral_constant<int, 0>;
    if (c_beg < c_end) {
        Dec d;
        if (c_beg < c_full) {
            d = book(C);
            stage(S0{}, 0, C, d.kw_l2, std::false_type{});
        } else {
            d = book(n_tail);
            stage(S0{}, 0, n_tail, d.kw_l2, std::true_type{});
        }
        if constexpr (PF == 1) {
            for (int64_t c = c_beg; c < c_full; ++c) {
                const int buf = (int)((c - c_beg) & 1);
                const bool next_full = c + 1 < c_full;
                if (next_full) load_chunk(S0{}, c + 1, std::false_type{});
                finish(c, C, d, std::false_type{});
                if (next_full) {
                    d = book(C);
                    stage(S0{}, buf ^ 1, C, d.kw_l2, std::false_type{});
                }
            }
        } else if (c_beg < c_full) {
            // unrolled PF times so that every register set has a fixed
            // name: sub-step s computes the chunk held by set s, refills
            // the set with the chunk PF ahead, and stages the next chunk
            // from set s + 1
            int64_t c = c_beg;
            auto sub = [&](auto s_c) LA_INLINE {
                constexpr int st = decltype(s_c)::value;
                const int buf = (int)((c - c_beg) & 1);
                load_chunk(s_c, min(c + PF, c_full - 1), std::false_type{});
                finish(c, C, d, std::false_type{});
                if (c + 1 >= c_full) return true;
                d = book(C);
                stage(std::integral_constant<int, (st + 1) % PF>{}, buf ^ 1, C, d.kw_l2, std::false_type{});
                ++c;
                return false;
            };
            while (!static_until<0, PF>(sub)) {
            }
        }
        if (ragged) {
            if (c_full > c_beg) {
                load_chunk(S0{}, c_full, std::true_type{});
                d = book(n_tail);
                stage(S0{}, (int)((c_full - c_beg) & 1), n_tail, d.kw_l2, std::true_type{});
            }
            finish(c_full, n_tail, d, std::true_type{});
        }
    }

    // ---- state out (true scale)
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
            // every wave has consumed its carried-in state (z is read by all
            // waves) before any writes the final one: S_dst may alias S_src
            if constexpr (MODE == MODE_CAUSAL) __syncthreads();
            const float ds = decay ? exp2f(log2D) : 1.f;
#pragma unroll
            for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
                for (int t = 0; t < DBW; ++t) {
                    const int d = 16 * (wave * DBW + t) + l16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) Sd[(16 * fb + 4 * g + r) * DV + d] = ds * accS[fb][t][r];
                }
            }
            if (l16 == 0) {
#pragma unroll
                for (int u = 0; u < ZB; ++u) *(f32x4*)(zd + 16 * (ZB * wave + u) + 4 * g) = accZ[u] * ds;
            }
        }
    }
}

}  // namespace la

#include "la_output.h"
#include "la_state.h"

namespace la {

template <class T, int PHI, int DK, int F, int DV>
hipError_t fwd_launch(const FwdArgs& a, int mode, hipStream_t stream)
{
    constexpr int C = chunk_len<T, PHI>(F);
    constexpr int NW = 4;
    const dim3 grid(a.cu_seqlens ? (unsigned)a.G : (unsigned)a.P, a.cu_seqlens ? (unsigned)a.H : (unsigned)a.BH),
        block(NW * 64);
    // fp32 inputs always write fp32 outputs, so only bf16 needs both variants
    const bool o32 = sizeof(T) == 2 && a.out_f32;
    switch (mode) {
    case MODE_LOCAL:
        // la_state_kernel for the maps of the query-split output pass, where
        // the segments are whole 64-token chunks (the backward cuts its
        // segments in its own chunks)
        if constexpr (query_split_output<T, PHI>())
            if (a.chunk % StateCfg<PHI, DK, F, DV>::C == 0) return state_launch<PHI, DK, F, DV>(a, stream);
        return launch_kernel(la_fwd_kernel<T, PHI, DK, F, DV, C, NW, MODE_LOCAL, false>, grid, block, stream, a);
    case MODE_CAUSAL:
        if constexpr (query_split_output<T, PHI>() && OutCfg<PHI, DK, F, DV>::FITS)
            return out_launch<PHI, DK, F, DV>(a, stream);
        return o32 ? launch_kernel(la_fwd_kernel<T, PHI, DK, F, DV, C, NW, MODE_CAUSAL, true>, grid, block, stream, a)
                   : launch_kernel(la_fwd_kernel<T, PHI, DK, F, DV, C, NW, MODE_CAUSAL, false>, grid, block, stream, a);
    default:
        return o32 ? launch_kernel(la_fwd_kernel<T, PHI, DK, F, DV, C, NW, MODE_QUERY, true>, grid, block, stream, a)
                   : launch_kernel(la_fwd_kernel<T, PHI, DK, F, DV, C, NW, MODE_QUERY, false>, grid, block, stream, a);
    }
}

// The segment-state pass alone: the random-feature backward runs it on
// features it has already computed (identity map), and needs no other mode.
template <class T, int PHI, int DK, int F, int DV>
hipError_t fwd_local_launch(const FwdArgs& a, int mode, hipStream_t stream)
{
    constexpr int C = chunk_len<T, PHI>(F);
    constexpr int NW = 4;
    if (mode != MODE_LOCAL || a.cu_seqlens) return hipErrorInvalidValue;
    return launch_kernel(la_fwd_kernel<T, PHI, DK, F, DV, C, NW, MODE_LOCAL, false>, dim3((unsigned)a.P, (unsigned)a.BH),
                         dim3(NW * 64), stream, a);
}

}  // namespace la
