// la_output.h -- the causal output pass for bf16 inputs (elu+1, ReLU and the
// trigonometric random features), with the work of a chunk split by query
// rows.
//
// What is computed is the chunked form of la_forward.h ("Attention is also an
// FFN", kwkr.cn/news/587576, sec. 4.1 notes and sec. 5.2: parallel inside a
// chunk, carried between chunks; decay sec. 3.2; normaliser sec. 4.2).  For
// a chunk of n tokens after the state (S, z), local positions i, j:
//
//   num_i, den_i = lambda^(i+1) phi(q_i)^T [S, z]
//                + sum_{j<=i} lambda^(i-j) (phi(q_i).phi(k_j)) [v_j, 1]
//   y_i          = num_i / (den_i + eps)
//   S            <- lambda^n S + sum_j lambda^(n-1-j) phi(k_j) v_j^T   (z likewise)
//
// Work split.  A chunk is C = 64 tokens, four 16-row query blocks.  Each wave
// owns one query block (with 8 waves, half of its output columns): it forms
// that block's decayed score tiles, its row sums, the inter-chunk product
// S^T phi(Q)^T and the intra-chunk product V^T P^T, and stores its outputs.
// The fp32 state is split over the waves in blocks of FBW feature blocks by
// the wave's own output columns, so that the value fragments of a column tile
// serve both the intra-chunk product and the state update; each wave adds the
// chunk's keys to its part with the matrix cores and writes it, rounded to
// bf16, into a shared LDS copy of S^T, which every wave reads as the A
// operand of the next chunk's inter-chunk product.
//
// Random features ("From standard attention to linear attention", sec. 4.2:
// phi(x) = c(x) [cos(omega x'), sin(omega x')] / sqrt(m), x' = qk_scale x).
// The raw q and k rows of a chunk are staged in LDS with the prefactor of
// each token; then every wave computes a share of the feature tiles on the
// matrix cores (omega x^T from omega's row blocks, kept in LDS as bf16 high
// and low parts, angles in revolutions for the hardware sine and cosine)
// and writes cos and sin into the same tiles the elementwise maps use.  Half
// of the waves take the queries, half the keys; a wave takes one pair of
// omega's 16-row blocks, whose features are the two halves of the tiles'
// 16-byte units, so that a lane writes its cosines (and its sines) of a token
// as one 16-byte unit (8-byte halves from 16 rows at once would meet in the
// banks two by two).  The prefactors stay out of the tiles: a key's enters the score
// weights and the value weights of the state update, a query's the
// normaliser, since num_i and den_i are both linear in phi(q_i).
//
// Decay weights of the state update.  The elementwise maps stage the key
// features a second time with the weight lambda^(n-1-j) (rescaled, see book);
// the random features, whose feature rows are wider than the value rows, put
// the weight (times the key's prefactor) on the values instead (and the
// weights themselves form the B operand of the z update), which halves the
// LDS tiles of the keys.  With WV the values are staged already weighted, so
// that one value fragment serves both the state update and V^T P^T: for a
// query i of the chunk, lambda^(i-j) c_j = r_i w_j with w_j the key's weight
// in the update and r_i = lambda^(i-n+1) times the pending scale, a factor of
// the query alone, so the score tiles need only the causal selection, the row
// sums take the weights as their A operand, and r_i multiplies the query's
// intra-chunk numerator and denominator.  w_j spans lambda^(C-1) inside a
// chunk, which the host allows only for lambda = 1 or lambda >= 2^-1/2 (the
// smallest weight then stays above 2^-32 of the largest); other heads run
// without WV.
//
// Layouts.  phi(Q), phi(K) and the weighted phi(K) are staged in LDS as in
// la_forward.h (TileL, swizzled 8-byte units); V in TileX, whose swizzle is
// conflict-free for transposing reads and staging (la_device.h has the bank
// model); the raw q, k rows padded by 16 bytes.  S^T is [DV][F] bf16 with the
// feature order inside each 32-wide block permuted so that the 8 k positions
// K(g) a lane needs (la_device.h) are contiguous: one 16-byte read per
// fragment; the 16-byte units are XOR-swizzled by row (st_off).  z is kept
// the same way ([F] bf16, permuted), so its fragment is one 16-byte read too.
//
// Per chunk there are two barriers: one after the chunk is staged (tiles,
// S^T and z of the previous chunk visible), one after every wave has read the
// tiles and S^T; the state's new S^T and z and the next chunk's tiles are
// written after the second (for random features, the next chunk's raw rows
// before it, as no wave reads them while computing).  The next chunk's q, k,
// v are loaded into registers while the current one is computed (for the
// elementwise maps issued right after the previous staging, so that they
// have the first barrier's wait too).
#pragma once

#include <type_traits>

#include "la_device.h"
#include "la_internal.h"

namespace la {

template <int PHI, int DK, int F, int DV>
struct OutCfg {
    static constexpr bool RF = PHI == LA_PHI_TRIG_RF;
    static constexpr bool VW = RF;       // decay weights on the values (else on the key features)
    static constexpr int M = RF ? F / 2 : 0;
    static constexpr int C = 64;
    static constexpr int QB = C / 16;
    static constexpr int FB = F / 16, DB = DV / 16, KB = F / 32, CB = C / 32;
    // eight waves (two per SIMD) where the state has at least eight feature
    // blocks; otherwise four
    static constexpr int NW = FB >= 8 ? 8 : 4;
    static constexpr int NT = NW * 64;
    static constexpr int QW = NW / QB;   // waves per query block
    static constexpr int DBQ = DB / QW;  // output column tiles per wave
    // state tiles per wave: FBW feature blocks of the wave's own DBQ output
    // column tiles (the QB waves of one column half split the feature rows)
    static constexpr int FBW = FB / QB;
    static constexpr int VEC = 8;        // bf16 per 16-byte vector
    static constexpr int VPRQ = DK / VEC, VPRV = DV / VEC;
    static constexpr int RQ = C * VPRQ / NT, RV = C * VPRV / NT;
    // random features: raw q, k rows of XLD elements (16 bytes of padding:
    // a row-fragment read of 16 rows is then conflict-free as a single 8-byte
    // read); omega row blocks per wave, each wave covering one of the two
    // token matrices
    static constexpr int KX = DK / 32, XLD = DK + 8;
    // random features: a wave of feature work takes one pair of omega's
    // 16-row blocks (2 p, 2 p + 1: the two halves of each 16-byte TileP unit)
    // and FTB of the four token blocks of its token matrix
    static constexpr int RBP = RF ? M / 32 : 0;
    static constexpr int FTB = RF ? RBP * (C / 16) / (NW / 2) : 0;
    static constexpr int TQ = C * F, TV = C * DV;  // elements of a tile
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t OFF_K = OFF_Q + size_t(TQ) * 2;
    static constexpr size_t OFF_KW = OFF_K + size_t(TQ) * 2;
    static constexpr size_t OFF_V = OFF_KW + (VW ? 0 : size_t(TQ) * 2);
    static constexpr size_t OFF_ST = OFF_V + size_t(TV) * 2;
    static constexpr size_t OFF_Z = OFF_ST + size_t(DV) * F * 2;
    static constexpr size_t OFF_X = OFF_Z + size_t(F) * 2;
    static constexpr size_t OFF_CF = OFF_X + (RF ? size_t(2) * C * XLD * 2 : 0);
    // omega's operand fragments: [row block][k block][high, low][lane], 16 bytes
    static constexpr size_t OFF_OM = OFF_CF + (RF ? size_t(4) * C * 4 : 0);
    static constexpr size_t OFF_W = OFF_OM + (RF ? size_t(M / 16) * KX * 2 * 64 * 16 : 0);
    static constexpr size_t TOTAL = OFF_W + (VW ? size_t(C) * 4 : 0);
    static_assert(F % 64 == 0 && DV % 64 == 0 && DK % 64 == 0, "head sizes");
    static_assert(RF || DK == F, "elementwise maps keep the width");
    static_assert(FBW >= 1 && FB % QB == 0 && NW % QB == 0 && DB % QW == 0, "wave split");
    static_assert(RQ >= 1 && RV >= 1 && (C * VPRQ) % NT == 0 && (C * VPRV) % NT == 0, "loads per thread");
    static_assert(!RF || (FTB >= 1 && FTB <= C / 16 && (C / 16) % FTB == 0 && FTB * (NW / 2) == RBP * (C / 16)),
                  "feature tiles must split over the waves");
    static_assert(OFF_X % 16 == 0 && OFF_CF % 16 == 0 && OFF_OM % 16 == 0 && OFF_W % 16 == 0, "alignment");
    // the LDS of one workgroup (not met by m = 128 random features with
    // d_v = 128, whose S^T alone is 64 KiB: the causal pass of la_forward.h
    // serves that shape)
    static constexpr bool FITS = TOTAL <= 160 * 1024;
};

// Element offset in S^T ([DV][F] bf16) of 16-byte unit u of row r: the units
// are XOR-swizzled by row, so that the 16 rows of a fragment read fall in
// distinct 16-byte slots of the 64 banks (rows of F = 64 share a 256-byte
// window two by two).
template <int F>
__device__ __forceinline__ int st_off(int r, int u)
{
    if constexpr (F >= 128) return r * F + ((u ^ (r & 15)) << 3);
    else return r * F + ((u ^ ((r >> 1) & 7)) << 3);
}

// PART: 0 for a whole map; 1, 2 for the first and second half of a split
// random-feature map (FwdArgs part_mode).  WV (random features): the values
// are staged with their key weights.
template <int PHI, int DK, int F, int DV, bool OUTF32, int PART, bool WV>
__global__ void __launch_bounds__((OutCfg<PHI, DK, F, DV>::NT), 2)
la_out_kernel(const FwdArgs a)
{
    using Cfg = OutCfg<PHI, DK, F, DV>;
    using T = bf16;
    constexpr int C = Cfg::C, NT = Cfg::NT, NW = Cfg::NW, QW = Cfg::QW, DBQ = Cfg::DBQ, FBW = Cfg::FBW;
    constexpr int KB = Cfg::KB, CB = Cfg::CB, DB = Cfg::DB, VEC = Cfg::VEC;
    constexpr int VPRQ = Cfg::VPRQ, VPRV = Cfg::VPRV, RQ = Cfg::RQ, RV = Cfg::RV;
    constexpr bool RF = Cfg::RF, VW = Cfg::VW;
    static_assert(!WV || VW, "weighted values only where the weights are on the values");
    constexpr int M = Cfg::M, KX = Cfg::KX, FTB = Cfg::FTB, XLD = Cfg::XLD;
    // phi(Q), phi(K) and the weighted phi(K) in TileP (a row fragment is one
    // 16-byte read); V in TileX
    using TF = TileP<T, F>;
    using TVL = TileX<T, DV>;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
    T* const sQ = (T*)(smem + Cfg::OFF_Q);
    T* const sK = (T*)(smem + Cfg::OFF_K);
    T* const sKw0 = (T*)(smem + Cfg::OFF_KW);
    T* const sV = (T*)(smem + Cfg::OFF_V);
    T* const sST = (T*)(smem + Cfg::OFF_ST);
    T* const sZ = (T*)(smem + Cfg::OFF_Z);
    T* const sX = (T*)(smem + Cfg::OFF_X);        // raw q rows, then raw k rows ([C][XLD] each)
    // prefactors of those rows, two buffers by chunk parity: the next
    // chunk's are written while the current chunk's are still read
    float* const sCF0 = (float*)(smem + Cfg::OFF_CF);
    int cb = 0;  // buffer of the chunk being staged and computed
    Frag<T>* const sOm = (Frag<T>*)(smem + Cfg::OFF_OM);
    float* const sWt = (float*)(smem + Cfg::OFF_W);  // key weights of the chunk (decay, weights on V)

    // the wave index as a scalar: every branch on the query block below is
    // uniform over the wave
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    // query block of this wave; the two waves of a SIMD (w, w + 4) take
    // blocks b and 3 - b, so that every SIMD forms the same number of score
    // tiles; with two waves per block, w < 4 takes the first half of the
    // output columns
    const int ib = (wave < 4) ? wave : 3 - (wave - 4);
    const int dq0 = (QW == 2 && wave >= 4) ? DBQ : 0;

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
    // segments of cps units of a.chunk tokens (a multiple of C)
    const int64_t cps = a.cps * (a.chunk / C);
    const int64_t NC = spare ? 0 : (n_len + C - 1) / C;
    const int64_t c_beg = (int64_t)seg * cps, c_end = (seg == a.P - 1) ? NC : min(NC, c_beg + cps);
    if (c_beg >= c_end && (!a.S_dst || spare)) return;
    const T* qg = (const T*)a.q + row0 * DK;
    const T* kg = (const T*)a.k + row0 * DK;
    const T* vg = (const T*)a.v + row0 * DV;
    const uint8_t* kp = a.kpm ? a.kpm + (int64_t)(bh / a.H) * a.kpm_stride + a.n0 : nullptr;
    const Frag<T> ones = frag_ones<T>();

    // decay tables of this lane: score element (i = 16 ib + l16, j = 16 jb +
    // 4 g + r) is weighted by lambda^(i-j): m0 on the diagonal block (zero
    // above the diagonal, by selection so that a non-finite key cannot reach
    // an earlier query through a zero weight), m1 * lambda^(16 (ib-jb-1))
    // below it
    float m0[4], m1[4];
    bool above[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = l16 - 4 * g - r;
        above[r] = e < 0;
        m0[r] = e < 0 ? 0.f : (decay ? lam_pow(l2l, e) : 1.f);
        m1[r] = decay ? lam_pow(l2l, 16 + e) : 1.f;
    }
    const float lq = decay ? lam_pow(l2l, 16 * ib + l16 + 1) : 1.f;  // lambda^(i+1)

    // ---- random features: rows 16 rb + l16 of omega as A-operand fragments,
    // scaled by qk_scale / (2 pi) so that the products are angles in
    // revolutions, and split into bf16 high and low parts (omega = hi + lo to
    // 16 bits), into LDS (read after the first barrier).  Wave rbg of token
    // matrix xpass takes items rbg FTB .. rbg FTB + FTB - 1 of that matrix's
    // (row-block pair, token block) items, all of one pair.
    const int rbg = wave % (NW / 2), xpass = wave / (NW / 2);
    if constexpr (RF) {
        const float om_scale = a.qk_scale * 0.159154943091895336f;
        for (int fi = wave; fi < (M / 16) * KX; fi += NW) {
            const int rb = fi / KX, kb = fi % KX;
            // k positions in natural order (8 g .. 8 g + 7), as the raw rows
            // are read in features()
            const float* p = a.omega + (int64_t)(16 * rb + l16) * DK + 32 * kb + 8 * g;
            const f32x4 w0 = *(const f32x4*)p * om_scale, w1 = *(const f32x4*)(p + 4) * om_scale;
            f32x4 r0, r1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r0[e] = w0[e] - (float)(bf16)w0[e];
                r1[e] = w1[e] - (float)(bf16)w1[e];
            }
            sOm[(fi * 2 + 0) * 64 + lane] = frag_acc<T>(w0, w1);
            sOm[(fi * 2 + 1) * 64 + lane] = frag_acc<T>(r0, r1);
        }
    }

    // ---- loads of one chunk into registers (as la_forward.h: a ragged last
    // chunk re-reads its last row and zeroes the rows past its end)
    const bool ragged = c_end > c_beg && c_end * C > n_len;
    const int64_t c_full = ragged ? c_end - 1 : c_end;
    const int n_tail = ragged ? (int)(n_len - c_full * C) : C;
    uint4 rq[RQ], rk[RQ], rv[RV];
    int mk[RQ];
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
    auto load_chunk = [&](int64_t c, auto tail_c) LA_INLINE {
        const int64_t t0 = c * C;
        const int n = decltype(tail_c)::value ? n_tail : C;
        load_rows(rq, qg + t0 * DK, VPRQ, DK, RQ, n, tail_c);
        load_rows(rk, kg + t0 * DK, VPRQ, DK, RQ, n, tail_c);
        load_rows(rv, vg + t0 * DV, VPRV, DV, RV, n, tail_c);
#pragma unroll
        for (int r = 0; r < RQ; ++r) {
            const int j = (tid + r * NT) / VPRQ;
            mk[r] = kp ? (int)kp[t0 + (decltype(tail_c)::value ? min(j, n - 1) : j)] : 0;
        }
    };
    // one tensor of a full chunk (0: v, 1: q, 2: k and its mask bytes), so
    // that each tensor's next loads go out as soon as its registers are staged
    auto load_part = [&](int part, int64_t c) LA_INLINE {
        const int64_t t0 = c * C;
        if (part == 0) {
            load_rows(rv, vg + t0 * DV, VPRV, DV, RV, C, std::false_type{});
        } else if (part == 1) {
            load_rows(rq, qg + t0 * DK, VPRQ, DK, RQ, C, std::false_type{});
        } else {
            load_rows(rk, kg + t0 * DK, VPRQ, DK, RQ, C, std::false_type{});
#pragma unroll
            for (int r = 0; r < RQ; ++r) mk[r] = kp ? (int)kp[t0 + (tid + r * NT) / VPRQ] : 0;
        }
    };
    if (c_beg < c_full) load_chunk(c_beg, std::false_type{});
    else if (c_beg < c_end) load_chunk(c_beg, std::true_type{});

    // ---- this wave's part of the state: accS[u][c] holds S[16 fb + 4 g + r]
    // [16 (dq0 + c) + l16] with fb = FBW * qw + u (qw: the wave's index among
    // the QB waves of its column half); accZ[u] holds z[16 fb + 4 g + r] in
    // every column (the first column half publishes and stores z)
    const int qw = wave % Cfg::QB;
    const bool zowner = dq0 == 0;
    f32x4 accS[FBW][DBQ], accZ[FBW];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < FBW; ++u) {
        accZ[u] = zero4;
#pragma unroll
        for (int c = 0; c < DBQ; ++c) accS[u][c] = zero4;
    }
    if (a.S_src) {
        const float* Sb = a.S_src + (int64_t)seg * a.src_seg_stride + (int64_t)bh * a.src_stride;
        const float* zb = a.z_src + (int64_t)seg * a.src_seg_stride + (int64_t)bh * a.src_zstride;
#pragma unroll
        for (int u = 0; u < FBW; ++u) {
            const int f0 = 16 * (FBW * qw + u) + 4 * g;
            const int fr = f0 + (f0 >= F / 2 ? a.src_gap : 0);  // row in the source's layout
#pragma unroll
            for (int c = 0; c < DBQ; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) accS[u][c][r] = Sb[(int64_t)(fr + r) * DV + 16 * (dq0 + c) + l16];
            accZ[u] = *(const f32x4*)(zb + fr);
        }
    }
    // this wave's rows into the shared S^T and z (bf16, permuted features)
    auto publish = [&]() LA_INLINE {
        if constexpr (FBW % 2 == 0) {
            // feature blocks fb (even) and fb + 1 fill the two halves of one
            // 16-byte unit: one store each
#pragma unroll
            for (int u = 0; u < FBW; u += 2) {
                const int unit = 4 * ((FBW * qw + u) >> 1) + g;
#pragma unroll
                for (int c = 0; c < DBQ; ++c) {
                    const int r = 16 * (dq0 + c) + l16;
                    const f32x4 a0 = accS[u][c], a1 = accS[u + 1][c];
                    *(bf16x8*)(sST + st_off<F>(r, unit)) = bf16x8{(T)a0[0], (T)a0[1], (T)a0[2], (T)a0[3],
                                                                   (T)a1[0], (T)a1[1], (T)a1[2], (T)a1[3]};
                }
                if (zowner && l16 == 0) {
                    const f32x4 z0 = accZ[u], z1 = accZ[u + 1];
                    *(bf16x8*)(sZ + unit * 8) = bf16x8{(T)z0[0], (T)z0[1], (T)z0[2], (T)z0[3],
                                                       (T)z1[0], (T)z1[1], (T)z1[2], (T)z1[3]};
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < FBW; ++u) {
                const int fb = FBW * qw + u;
                const int unit = 4 * (fb >> 1) + g, half = (fb & 1) * 4;
#pragma unroll
                for (int c = 0; c < DBQ; ++c) {
                    const int r = 16 * (dq0 + c) + l16;
                    st4(sST + st_off<F>(r, unit) + half, accS[u][c][0], accS[u][c][1], accS[u][c][2], accS[u][c][3]);
                }
                if (zowner && l16 == 0) st4(sZ + unit * 8 + half, accZ[u][0], accZ[u][1], accZ[u][2], accZ[u][3]);
            }
        }
    };
    publish();
    float log2D = 0.f;  // the true state is 2^log2D times the accumulators

    // ---- staging of one chunk from the registers.  Elementwise maps: phi(q),
    // phi(k), the lambda-weighted phi(k) (decay only) and v.  Random features:
    // v and the key weights; their q, k rows go in raw by stage_x and become
    // features in features().  kw_l2 as in
    // la_forward.h.
    auto key_weight = [&](int k, float kw_l2) LA_INLINE {
        return k == 0 ? __builtin_amdgcn_exp2f(-kw_l2) : __builtin_amdgcn_exp2f((float)k * l2l - kw_l2);
    };
    auto put_feat = [&](T* tile, int row, int col, const float* p) LA_INLINE {
        st4(tile + TF::off(row, col), p[0], p[1], p[2], p[3]);
        st4(tile + TF::off(row, col + 4), p[4], p[5], p[6], p[7]);
    };
    // after_part(p) runs once tensor p (0: v, 1: q, 2: k) is staged
    auto stage = [&](int n, float kw_l2, auto tail_c, auto&& after_part) LA_INLINE {
        constexpr bool TAIL = decltype(tail_c)::value;
        const int cg = tid % VPRQ;
#pragma unroll
        for (int r = 0; r < RV; ++r) {
            const int idx = tid + r * NT, j = idx / VPRV, c4 = idx % VPRV;
            const uint4 u = rv[r];
            if constexpr (WV) {
                // v_j times its key weight; a dropped key's row is zeroed by
                // selection, whatever its values
                const float w = (TAIL && j >= n) ? 0.f
                                                 : (decay ? key_weight(n - 1 - j, kw_l2) : 1.f) * sCF0[cb * 2 * C + C + j];
                float x[VEC];
                unpack16(u, x, (const T*)nullptr);
#pragma unroll
                for (int e = 0; e < VEC; ++e) x[e] = w == 0.f ? 0.f : x[e] * w;
                st4(sV + TVL::off(j, c4 * VEC), x[0], x[1], x[2], x[3]);
                st4(sV + TVL::off(j, c4 * VEC + 4), x[4], x[5], x[6], x[7]);
            } else {
                *(uint2*)(sV + TVL::off(j, c4 * VEC)) = uint2{u.x, u.y};
                *(uint2*)(sV + TVL::off(j, c4 * VEC + 4)) = uint2{u.z, u.w};
            }
        }
        after_part(0);
        if constexpr (!RF) {
#pragma unroll
            for (int r = 0; r < RQ; ++r) {
                const int j = (tid + r * NT) / VPRQ;
                float x[VEC], p[VEC];
                unpack16(rq[r], x, (const T*)nullptr);
#pragma unroll
                for (int e = 0; e < VEC; ++e) p[e] = phi_elem<T, PHI>(x[e]);
                put_feat(sQ, j, cg * VEC, p);
            }
            after_part(1);
#pragma unroll
            for (int r = 0; r < RQ; ++r) {
                const int j = (tid + r * NT) / VPRQ;
                float x[VEC], p[VEC];
                unpack16(rk[r], x, (const T*)nullptr);
#pragma unroll
                for (int e = 0; e < VEC; ++e) p[e] = phi_elem<T, PHI>(x[e]);
                if ((TAIL && j >= n) || mk[r]) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) p[e] = 0.f;
                }
                put_feat(sK, j, cg * VEC, p);
                if (decay) {
                    const float w = (TAIL && j >= n) ? 0.f : key_weight(n - 1 - j, kw_l2);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) p[e] *= w;
                    put_feat(sKw0, j, cg * VEC, p);
                }
            }
            after_part(2);
        }
        if constexpr (VW) {
            // weight of key tid in the state update: its decay weight times
            // its prefactor (zero for a dropped key)
            if (tid < C)
                sWt[tid] = (TAIL && tid >= n) ? 0.f : (decay ? key_weight(n - 1 - tid, kw_l2) : 1.f) * sCF0[cb * 2 * C + C + tid];
        }
    };
    const auto no_loads = [](int) {};

    // ---- random features, part 1: the raw q and k rows and the prefactor
    // c(x) = exp(s |x'|^2 / 2) / sqrt(m) of each.  A key that is past the end
    // of the sequence or masked is dropped: its row is staged as zeros (finite
    // features whatever its values) and its prefactor is zero.
    const float rf_cexp = 0.5f * a.rf_sign * a.qk_scale * a.qk_scale;
    const float rf_cnorm = a.rf_scale;
    auto stage_x = [&](int n, int buf, auto tail_c) LA_INLINE {
        if constexpr (RF) {
            constexpr bool TAIL = decltype(tail_c)::value;
            const int cg = tid % VPRQ;
#pragma unroll
            for (int pass = 0; pass < 2; ++pass)
#pragma unroll
                for (int r = 0; r < RQ; ++r) {
                    const int j = (tid + r * NT) / VPRQ;
                    const bool drop = pass == 1 && ((TAIL && j >= n) || mk[r]);
                    const uint4 u = drop ? uint4{0u, 0u, 0u, 0u} : (pass ? rk[r] : rq[r]);
                    *(uint4*)(sX + (pass * C + j) * XLD + cg * VEC) = u;
                    float x[VEC];
                    unpack16(u, x, (const T*)nullptr);
                    float s2 = 0.f;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) s2 += x[e] * x[e];
                    s2 = group_sum<VPRQ>(s2);
                    if (cg == 0) sCF0[buf * 2 * C + pass * C + j] = drop ? 0.f : exp_rf<T>(rf_cexp * s2) * rf_cnorm;
                }
        }
    };

    // ---- random features, part 2: U^T = omega x^T on the matrix cores for
    // this wave's row blocks of omega and token matrix (queries or keys), all
    // four token blocks; cos and sin (without the prefactor) written
    // row-major into phi(Q) or phi(K) (columns f and m + f)
    auto features = [&]() LA_INLINE {
        if constexpr (RF) {
            const T* const xs = sX + xpass * C * XLD;
            T* const tile = xpass ? sK : sQ;
            const int it0 = rbg * FTB, pr = it0 / Cfg::QB;  // first item, row-block pair
            Frag<T> om_hi[2][KX], om_lo[2][KX];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int kb = 0; kb < KX; ++kb) {
                    const int fi = (2 * pr + u) * KX + kb;
                    om_hi[u][kb] = sOm[(fi * 2 + 0) * 64 + lane];
                    om_lo[u][kb] = sOm[(fi * 2 + 1) * 64 + lane];
                }
#pragma unroll
            for (int t = 0; t < FTB; ++t) {
                const int j = 16 * ((it0 + t) % Cfg::QB) + l16;
                Frag<T> xf[KX];
#pragma unroll
                for (int kb = 0; kb < KX; ++kb) xf[kb] = frag_row16(xs, XLD, j, 32 * kb, g);
                // acc[u][r]: angle of feature 16 (2 pr + u) + 4 g + r for token j
                f32x4 acc[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    acc[u] = zero4;
#pragma unroll
                    for (int kb = 0; kb < KX; ++kb) {
                        mma(acc[u], om_hi[u][kb], xf[kb]);
                        mma(acc[u], om_lo[u][kb], xf[kb]);
                    }
                }
                float cs[2][4], sn[2][4];
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        cs[u][r] = __builtin_amdgcn_cosf(acc[u][r]);
                        sn[u][r] = __builtin_amdgcn_sinf(acc[u][r]);
                    }
                // the pair's features 32 pr + 4 g .. + 3 and 32 pr + 16 + 4 g
                // .. + 3 fill TileP unit 4 pr + g: one 16-byte write for the
                // cosines, one for the sines (columns m + f)
                *(bf16x8*)(tile + TF::unit_off(j, 4 * pr + g)) =
                    bf16x8{(T)cs[0][0], (T)cs[0][1], (T)cs[0][2], (T)cs[0][3], (T)cs[1][0], (T)cs[1][1], (T)cs[1][2], (T)cs[1][3]};
                *(bf16x8*)(tile + TF::unit_off(j, 4 * (M / 32 + pr) + g)) =
                    bf16x8{(T)sn[0][0], (T)sn[0][1], (T)sn[0][2], (T)sn[0][3], (T)sn[1][0], (T)sn[1][1], (T)sn[1][2], (T)sn[1][3]};
            }
        }
    };

    // ---- outputs of this wave's query block and the update of its state
    // rows, for one staged chunk.  dscale: 2^log2D of the state in S^T;
    // rescale: factor on the accumulators before the chunk's keys are added.
    auto compute = [&](int n, int64_t t0, float dscale, bool do_rescale, float rescale, float kw_l2, auto tail_c) LA_INLINE {
        constexpr bool TAIL = decltype(tail_c)::value;
        const int i = 16 * ib + l16;
        // products with phi(Q): phi(q_i).z (every row holds it), the scores
        // of this query block against all four key blocks as P^T, and the
        // inter-chunk part S^T phi(Q)^T of this wave's column tiles t = dq0 ..
        // dq0 + DBQ - 1.  Where the feature row has no more k blocks than the
        // wave has column tiles, the fragments of phi(q_i) are read first and
        // the inter-chunk part follows per column tile; otherwise the
        // products run one k block at a time into DBQ accumulators.
        constexpr bool QF_ALL = KB <= DBQ;
        f32x4 dq = zero4, pt[QF_ALL ? 1 : 4], o[QF_ALL ? 1 : DBQ];
        Frag<T> qf[QF_ALL ? KB : 1];
        if constexpr (!QF_ALL) {
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) pt[jb] = zero4;
        }
        auto sfrag = [&](int t, int kb) LA_INLINE {
            Frag<T> sf;
            sf.v = *(const bf16x8*)(sST + st_off<F>(16 * t + l16, 4 * kb + g));
            return sf;
        };
        auto zfrag = [&](int kb) LA_INLINE {
            Frag<T> zf;
            zf.v = *(const bf16x8*)(sZ + (4 * kb + g) * 8);
            return zf;
        };
        // B operands of the z update (with WV also the A operands of the row
        // sums): the chunk's key weights where they are not in the key
        // features, else ones
        Frag<T> wf[CB];
        f32x4 wlo[VW ? CB : 1], whi[VW ? CB : 1];  // the weights of this lane's k positions
        auto load_weights = [&]() LA_INLINE {
#pragma unroll
            for (int kb = 0; kb < CB; ++kb) {
                if constexpr (VW) {
                    wlo[kb] = *(const f32x4*)(sWt + 32 * kb + 4 * g);
                    whi[kb] = *(const f32x4*)(sWt + 32 * kb + 16 + 4 * g);
                    wf[kb] = frag_acc<T>(wlo[kb], whi[kb]);
                } else {
                    wf[kb] = ones;
                }
            }
        };
        if constexpr (WV) load_weights();
        Frag<T> pf[CB];
        f32x4 rs = zero4;
        if constexpr (QF_ALL) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) qf[kb] = lds_frag_row<T, F, TF>(sQ, i, kb, g);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) mma(dq, zfrag(kb), qf[kb]);
            // one version per query block (ib is the same in every lane of
            // the wave): the score tiles of key blocks 0 .. ib are formed and
            // given their decay weights (random features: times the key's
            // prefactor), those after it are zero; only the diagonal block
            // needs a selection, which zeroes its keys above the diagonal
            // (by selection, so that a non-finite key cannot reach an
            // earlier query through a zero weight)
            auto scores = [&](auto ib_c) LA_INLINE {
                constexpr int IB = decltype(ib_c)::value;
                f32x4 p4[4];
                static_until<0, 4>([&](auto jb_c) LA_INLINE {
                    constexpr int JB = decltype(jb_c)::value;
                    if constexpr (JB <= IB) {
                        f32x4 acc = zero4;
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
                            mma(acc, lds_frag_row<T, F, TF>(sK, 16 * JB + l16, kb, g), qf[kb]);
                        f32x4 ck = {1.f, 1.f, 1.f, 1.f};
                        if constexpr (RF && !WV) ck = *(const f32x4*)(sCF0 + cb * 2 * C + C + 16 * JB + 4 * g);
                        if constexpr (JB == IB) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) p4[JB][r] = above[r] ? 0.f : (WV ? acc[r] : acc[r] * (m0[r] * ck[r]));
                        } else if constexpr (WV) {
                            p4[JB] = acc;
                        } else {
                            // lambda^(16 (ib-jb-1)) for blocks before the query block
                            const float dj = lam_pow(l2l, 16 * (IB - JB - 1));
#pragma unroll
                            for (int r = 0; r < 4; ++r) p4[JB][r] = acc[r] * (m1[r] * dj * ck[r]);
                        }
                    } else {
                        p4[JB] = zero4;
                    }
                    return false;
                });
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) {
                    pf[kb] = frag_acc<T>(p4[2 * kb], p4[2 * kb + 1]);
                    if (2 * kb <= IB) mma(rs, WV ? wf[kb] : ones, pf[kb]);
                }
            };
            switch (ib) {
            case 0: scores(std::integral_constant<int, 0>{}); break;
            case 1: scores(std::integral_constant<int, 1>{}); break;
            case 2: scores(std::integral_constant<int, 2>{}); break;
            default: scores(std::integral_constant<int, 3>{}); break;
            }
        } else {
            // the products one k block at a time: where the feature row has
            // at most 128 features, in one version per query block that
            // forms key blocks 0 .. ib only (kloop below); wider rows form all
            // four blocks in one version of the loop (four versions spill
            // there)
            constexpr bool KLOOP_IB = F <= 128;
            auto kloop = [&](auto ib_c) LA_INLINE {
                constexpr int IB = decltype(ib_c)::value;
#pragma unroll
                for (int tq = 0; tq < DBQ; ++tq) o[tq] = zero4;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const Frag<T> q1 = lds_frag_row<T, F, TF>(sQ, i, kb, g);
                    mma(dq, zfrag(kb), q1);
#pragma unroll
                    for (int jb = 0; jb <= IB; ++jb) mma(pt[jb], lds_frag_row<T, F, TF>(sK, 16 * jb + l16, kb, g), q1);
#pragma unroll
                    for (int tq = 0; tq < DBQ; ++tq) mma(o[tq], sfrag(dq0 + tq, kb), q1);
                }
            };
            if constexpr (!KLOOP_IB) {
#pragma unroll
                for (int tq = 0; tq < DBQ; ++tq) o[tq] = zero4;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const Frag<T> q1 = lds_frag_row<T, F, TF>(sQ, i, kb, g);
                    mma(dq, zfrag(kb), q1);
#pragma unroll
                    for (int jb = 0; jb < 4; ++jb) mma(pt[jb], lds_frag_row<T, F, TF>(sK, 16 * jb + l16, kb, g), q1);
#pragma unroll
                    for (int tq = 0; tq < DBQ; ++tq) mma(o[tq], sfrag(dq0 + tq, kb), q1);
                }
            }
            // decay weights of the scores (random features: times the key's
            // prefactor), in one version per query block as above: blocks
            // after the query block are zero, keys above the diagonal are
            // zeroed by selection
            auto weigh = [&](auto ib_c) LA_INLINE {
                constexpr int IB = decltype(ib_c)::value;
                f32x4 p4[4];
                static_until<0, 4>([&](auto jb_c) LA_INLINE {
                    constexpr int JB = decltype(jb_c)::value;
                    if constexpr (JB <= IB) {
                        f32x4 ck = {1.f, 1.f, 1.f, 1.f};
                        if constexpr (RF && !WV) ck = *(const f32x4*)(sCF0 + cb * 2 * C + C + 16 * JB + 4 * g);
                        if constexpr (JB == IB) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) p4[JB][r] = above[r] ? 0.f : (WV ? pt[JB][r] : pt[JB][r] * (m0[r] * ck[r]));
                        } else if constexpr (WV) {
                            p4[JB] = pt[JB];
                        } else {
                            const float dj = lam_pow(l2l, 16 * (IB - JB - 1));
#pragma unroll
                            for (int r = 0; r < 4; ++r) p4[JB][r] = pt[JB][r] * (m1[r] * dj * ck[r]);
                        }
                    } else {
                        p4[JB] = zero4;
                    }
                    return false;
                });
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) {
                    pf[kb] = frag_acc<T>(p4[2 * kb], p4[2 * kb + 1]);
                    if (2 * kb <= IB) mma(rs, WV ? wf[kb] : ones, pf[kb]);
                }
            };
            auto both = [&](auto ib_c) LA_INLINE {
                if constexpr (KLOOP_IB) kloop(ib_c);
                weigh(ib_c);
            };
            switch (ib) {
            case 0: both(std::integral_constant<int, 0>{}); break;
            case 1: both(std::integral_constant<int, 1>{}); break;
            case 2: both(std::integral_constant<int, 2>{}); break;
            default: both(std::integral_constant<int, 3>{}); break;
            }
        }
        // y_i = c_i (o + o_i) / (c_i den + eps) with c_i the query's
        // prefactor (random features), else y_i = (o + o_i) / (den + eps).
        // Over half of the features (part_mode 1, 2) the numerator and the
        // denominator of the other half are stored, or added in.
        const float lqd = lq * dscale;
        const float cq = RF ? sCF0[cb * 2 * C + i] : 1.f;
        const int64_t yrow = row0 + t0 + i;
        const bool live = !TAIL || i < n;  // rows past the end are neither read nor stored
        constexpr int pmode = PART;
        // WV: the query's factor on its intra-chunk parts, lambda^(i-n+1)
        // times the pending scale
        const float ri = (WV && decay) ? __builtin_amdgcn_exp2f((float)(i - (n - 1)) * l2l + kw_l2) : 1.f;
        const float den = cq * (rs[0] * ri + lqd * dq[0]);
        const float den1 = (pmode == 2 && live) ? a.part_den[yrow] : 0.f;
        const float inv0 = pmode == 1 ? 1.f : fast_rcp(den + den1 + a.eps);
        const float inv = RF ? cq * inv0 : inv0;
        const float sc = lqd * inv, si = inv * ri;
        if (pmode == 1 && live && dq0 == 0 && g == 0) a.part_den[yrow] = den;
        if constexpr (!WV) load_weights();
        if (do_rescale) {
#pragma unroll
            for (int u = 0; u < FBW; ++u) {
                accZ[u] *= rescale;
#pragma unroll
                for (int c = 0; c < DBQ; ++c) accS[u][c] *= rescale;
            }
        }
        // A operands of the state update: the weighted key features, or (the
        // weights on the values, or no decay) the key features themselves.
        // Where a wave has no more feature blocks than column tiles, their
        // fragments are read first and each column tile's update follows its
        // outputs; otherwise the (weighted) value fragments of every column
        // tile are kept and the update runs one feature block at a time.
        const T* const sKu = (VW || !decay) ? sK : sKw0;
        constexpr bool KEYS_FIRST = FBW <= DBQ;
        Frag<T> kwf[KEYS_FIRST ? FBW : 1][CB];
        if constexpr (KEYS_FIRST) {
#pragma unroll
            for (int u = 0; u < FBW; ++u)
#pragma unroll
                for (int kb = 0; kb < CB; ++kb)
                    kwf[u][kb] = ColRead<T, F, TF>::get(sKu, 32 * kb, 16 * (FBW * qw + u), lane);
        }
        // outputs of this wave's column tiles: O^T = S^T phi(Q)^T (scaled) +
        // V^T P^T; the value fragments of a column tile are the A operands of
        // V^T P^T and (weighted where the weights are on the values) the B
        // operands of the state update
        Frag<T> vwf[KEYS_FIRST ? 1 : DBQ][CB];
#pragma unroll
        for (int tq = 0; tq < DBQ; ++tq) {
            const int t = dq0 + tq;
            Frag<T> vf[CB];
#pragma unroll
            for (int kb = 0; kb < CB; ++kb) vf[kb] = ColRead<T, DV, TVL>::get(sV, 32 * kb, 16 * t, lane);
            f32x4 ot, oi = zero4;
            if constexpr (QF_ALL) {
                ot = zero4;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) mma(ot, sfrag(t, kb), qf[kb]);
            } else {
                ot = o[tq];
            }
#pragma unroll
            for (int kb = 0; kb < CB; ++kb) mma(oi, vf[kb], pf[kb]);
            f32x4 y = ot * sc + oi * si;
            if (live) {
                const int64_t yo = yrow * DV + 16 * t + 4 * g;
                if (pmode == 1) {
                    st4(a.part_num + yo, y[0], y[1], y[2], y[3]);
                } else {
                    if (pmode == 2) y += *(const f32x4*)(a.part_num + yo) * inv0;
                    if constexpr (OUTF32) st4((float*)a.y + yo, y[0], y[1], y[2], y[3]);
                    else st4((T*)a.y + yo, y[0], y[1], y[2], y[3]);
                }
            }
            const int vs = KEYS_FIRST ? 0 : tq;
#pragma unroll
            for (int kb = 0; kb < CB; ++kb) vwf[vs][kb] = vf[kb];
            if constexpr (VW && !WV) {
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) {
                    f32x4 lo, hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        lo[e] = (float)vf[kb].v[e] * wlo[kb][e];
                        hi[e] = (float)vf[kb].v[4 + e] * whi[kb][e];
                    }
                    vwf[vs][kb] = frag_acc<T>(lo, hi);
                }
            }
            // state update of this column tile: S^ += (w phi(K))^T V, or
            // phi(K)^T (w V)
            if constexpr (KEYS_FIRST) {
#pragma unroll
                for (int u = 0; u < FBW; ++u)
#pragma unroll
                    for (int kb = 0; kb < CB; ++kb) mma(accS[u][tq], kwf[u][kb], vwf[0][kb]);
            }
        }
        if constexpr (KEYS_FIRST) {
#pragma unroll
            for (int u = 0; u < FBW; ++u)
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) mma(accZ[u], kwf[u][kb], wf[kb]);
        } else {
            // state update one feature block at a time, z likewise
#pragma unroll
            for (int u = 0; u < FBW; ++u) {
                Frag<T> kf[CB];
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) kf[kb] = ColRead<T, F, TF>::get(sKu, 32 * kb, 16 * (FBW * qw + u), lane);
#pragma unroll
                for (int tq = 0; tq < DBQ; ++tq)
#pragma unroll
                    for (int kb = 0; kb < CB; ++kb) mma(accS[u][tq], kf[kb], vwf[tq][kb]);
#pragma unroll
                for (int kb = 0; kb < CB; ++kb) mma(accZ[u], kf[kb], wf[kb]);
            }
        }
    };

    // decay bookkeeping, in chunk order (as la_forward.h)
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
                d.rescale = exp2f(cand);
                log2D = 0.f;
            }
        }
        return d;
    };

    if (c_beg < c_end) {
        Dec d;
        // (random features: the key weights of stage() need the prefactors
        // of stage_x(), and features() the raw rows, so a barrier follows
        // stage_x() where no other one does)
        // elementwise maps: the next chunk's loads go out as soon as this
        // one's tensors are staged, before the barrier (random features keep
        // them after it: their staging registers are live until the raw rows
        // are staged)
        constexpr bool EARLY = !RF;
        if (c_beg < c_full) {
            d = book(C);
            stage_x(C, cb, std::false_type{});
            if constexpr (RF) __syncthreads();
            const bool load1 = EARLY && c_beg + 1 < c_full;
            stage(C, d.kw_l2, std::false_type{}, [&](int part) LA_INLINE {
                if (load1) load_part(part, c_beg + 1);
            });
        } else {
            d = book(n_tail);
            stage_x(n_tail, cb, std::true_type{});
            if constexpr (RF) __syncthreads();
            stage(n_tail, d.kw_l2, std::true_type{}, no_loads);
        }
        features();
        for (int64_t c = c_beg; c < c_full; ++c) {
            const bool next_full = c + 1 < c_full;
            __syncthreads();
            if (!EARLY && next_full) load_chunk(c + 1, std::false_type{});
            compute(C, c * C, d.dscale, d.do_rescale, d.rescale, d.kw_l2, std::false_type{});
            // raw rows of the next chunk: features() of this chunk read them
            // before the barrier above
            if (next_full) stage_x(C, cb ^ 1, std::false_type{});
            __syncthreads();
            publish();
            if (next_full) {
                cb ^= 1;
                d = book(C);
                // elementwise maps: each tensor's loads for chunk c + 2 go
                // out right after the tensor is staged
                const bool load2 = EARLY && c + 2 < c_full;
                stage(C, d.kw_l2, std::false_type{}, [&](int part) LA_INLINE {
                    if (load2) load_part(part, c + 2);
                });
                features();
            }
        }
        if (ragged) {
            if (c_full > c_beg) {
                load_chunk(c_full, std::true_type{});
                cb ^= 1;
                d = book(n_tail);
                stage_x(n_tail, cb, std::true_type{});
                if constexpr (RF) __syncthreads();
                stage(n_tail, d.kw_l2, std::true_type{}, no_loads);
                features();
            }
            __syncthreads();
            compute(n_tail, c_full * C, d.dscale, d.do_rescale, d.rescale, d.kw_l2, std::true_type{});
        }
    }

    // ---- final state (true scale), this wave's rows
    if (a.S_dst) {
        float* Sd = a.S_dst + (int64_t)bh * a.dst_stride;
        float* zd = a.z_dst + (int64_t)bh * a.dst_zstride;
        const float ds = decay ? exp2f(log2D) : 1.f;
#pragma unroll
        for (int u = 0; u < FBW; ++u) {
            const int f0 = 16 * (FBW * qw + u) + 4 * g;
            const int fr = f0 + (f0 >= F / 2 ? a.dst_gap : 0);  // row in the destination's layout
#pragma unroll
            for (int c = 0; c < DBQ; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) Sd[(int64_t)(fr + r) * DV + 16 * (dq0 + c) + l16] = ds * accS[u][c][r];
            if (zowner && l16 == 0) *(f32x4*)(zd + fr) = accZ[u] * ds;
        }
    }
}

template <int PHI, int DK, int F, int DV>
hipError_t out_launch(const FwdArgs& a, hipStream_t stream)
{
    using Cfg = OutCfg<PHI, DK, F, DV>;
    static_assert(Cfg::FITS, "LDS budget");
    if (a.chunk % Cfg::C != 0) return hipErrorInvalidValue;  // segments must be whole chunks
    // the halves of a split map: only the instance that can be one (m = 128
    // directions per half, d_k = d_v = 64) has them
    constexpr bool SPLIT = PHI == LA_PHI_TRIG_RF && F == 256 && DK == 64 && DV == 64;
    if (a.part_mode != 0 && !SPLIT) return hipErrorInvalidValue;
    // random features: the values are staged with their key weights where
    // every head has lambda = 1 or lambda >= 2^-1/2 (the range of the weights
    // inside a chunk, lambda^(C-1), stays within 2^-32)
    bool wv = false;
    if constexpr (Cfg::VW) {
        wv = true;
        for (int h = 0; h < a.H; ++h) {
            const float l2 = a.lam.log2lam[h];
            if (!(l2 == 0.f || l2 >= -0.5f)) wv = false;
        }
    }
    auto pick = [&](auto wv_c) {
        constexpr bool W = decltype(wv_c)::value;
        auto k = a.out_f32 ? la_out_kernel<PHI, DK, F, DV, true, 0, W> : la_out_kernel<PHI, DK, F, DV, false, 0, W>;
        if constexpr (SPLIT) {
            if (a.part_mode == 1) k = la_out_kernel<PHI, DK, F, DV, false, 1, W>;
            else if (a.part_mode == 2)
                k = a.out_f32 ? la_out_kernel<PHI, DK, F, DV, true, 2, W> : la_out_kernel<PHI, DK, F, DV, false, 2, W>;
        }
        return k;
    };
    auto kernel = pick(std::false_type{});
    if constexpr (Cfg::VW)
        if (wv) kernel = pick(std::true_type{});
    // More segments than workgroups resident at once: each workgroup takes k
    // consecutive segments (their carried-in state is the first one's), so
    // that the pass runs in one round of workgroups.
    FwdArgs b = a;
    if (!a.cu_seqlens && a.P > 1) {
        const int slots = device_slots(kernel, Cfg::NT);
        const int64_t wgs = (int64_t)a.P * a.BH;
        const int k = slots > 0 ? (int)((wgs + slots - 1) / slots) : 1;
        if (k > 1) {
            b.P = (a.P + k - 1) / k;
            b.cps = a.cps * k;
            b.src_seg_stride = a.src_seg_stride * k;
        }
    }
    const dim3 grid(b.cu_seqlens ? (unsigned)b.G : (unsigned)b.P, b.cu_seqlens ? (unsigned)b.H : (unsigned)b.BH),
        block(Cfg::NT);
    return launch_kernel(kernel, grid, block, stream, b);
}

}  // namespace la
