// la_device.h -- device helpers for the gfx950 kernels: element types, MFMA
// fragments, feature maps and decay powers.
//
// Matrix-core fragments.  Every product in this library is built from the
// 16x16 output tile of v_mfma_f32_16x16x32_bf16 (bf16 operands) or of eight
// chained v_mfma_f32_16x16x4_f32 (fp32 operands).  In the 16x16 fp32
// accumulator, lane l holds rows 4*(l/16)+r (r = 0..3) of column l%16.
//
// A contraction over a 32-wide block of the k index is fed as one "fragment"
// per lane: 8 values for the lane's row (A operand) or column (B operand), at
// the k positions
//     K(g) = { 4g, 4g+1, 4g+2, 4g+3, 16+4g, 16+4g+1, 16+4g+2, 16+4g+3 },
// g = l/16.  Both operands use the same K(g), so the product is the full
// contraction whatever order the hardware assigns to the 8 slots.  K(g) is
// exactly the set of rows a lane holds in two vertically adjacent accumulator
// tiles, so an accumulator pair converts into the next product's operand with
// no data movement between lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/la.h"
#include "la_internal.h"

namespace la {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <class T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Four consecutive elements at p (p must be 4-element aligned).
__device__ __forceinline__ bf16x4 ld4(const bf16* p) { return *(const bf16x4*)p; }
__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const f32x4*)p; }

__device__ __forceinline__ void st4(bf16* p, float a, float b, float c, float d) {
    bf16x4 t = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *(bf16x4*)p = t;
}
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
    f32x4 t = {a, b, c, d};
    *(f32x4*)p = t;
}

// Fragment from two 4-element groups (k = 4g.. and k = 16+4g..).
__device__ __forceinline__ Frag<bf16> frag2(const bf16* lo, const bf16* hi) {
    Frag<bf16> f;
    f.v = __builtin_shufflevector(ld4(lo), ld4(hi), 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
}
__device__ __forceinline__ Frag<float> frag2(const float* lo, const float* hi) {
    Frag<float> f;
    f.lo = ld4(lo);
    f.hi = ld4(hi);
    return f;
}

// Fragment of a row-major [rows][ld] buffer: row `row`, k block starting at k0.
template <class T>
__device__ __forceinline__ Frag<T> frag_rm(const T* base, int ld, int row, int k0, int g) {
    const T* p = base + row * ld + k0 + 4 * g;
    return frag2(p, p + 16);
}

// Fragment of a row-major bf16 [rows][ld] buffer holding the 8 consecutive
// elements k0 + 8 g .. + 7 of row `row`, one 16-byte read (k positions in
// natural order: pair it only with operands built in the same order).  With
// ld = 72 (144-byte rows) the 16 rows of a read fall in distinct 16-byte
// slots of the banks, where the two 8-byte halves of frag_rm meet two by two
// once the compiler pairs them into one two-address read.
__device__ __forceinline__ Frag<bf16> frag_row16(const bf16* base, int ld, int row, int k0, int g) {
    Frag<bf16> f;
    f.v = *(const bf16x8*)(base + row * ld + k0 + 8 * g);
    return f;
}

// Fragment from two accumulator tiles (rows 0..15 then 16..31 of the k block).
template <class T> __device__ __forceinline__ Frag<T> frag_acc(const f32x4& a, const f32x4& b);
template <> __device__ __forceinline__ Frag<bf16> frag_acc<bf16>(const f32x4& a, const f32x4& b) {
    Frag<bf16> f;
    f.v = bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                 (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
    return f;
}
template <> __device__ __forceinline__ Frag<float> frag_acc<float>(const f32x4& a, const f32x4& b) {
    Frag<float> f;
    f.lo = a;
    f.hi = b;
    return f;
}

// A fragment whose every slot is 1: as the A operand it turns a product into
// column sums of B over the k block (rows of the result all equal), as the B
// operand into row sums of A.
template <class T> __device__ __forceinline__ Frag<T> frag_ones();
template <> __device__ __forceinline__ Frag<bf16> frag_ones<bf16>() {
    Frag<bf16> f;
    const bf16 one = (bf16)1.0f;
    f.v = bf16x8{one, one, one, one, one, one, one, one};
    return f;
}
template <> __device__ __forceinline__ Frag<float> frag_ones<float>() {
    Frag<float> f;
    f.lo = f32x4{1.f, 1.f, 1.f, 1.f};
    f.hi = f.lo;
    return f;
}

// acc += A(16 x 32) * B(32 x 16) for one 32-wide k block.
__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[e], b.lo[e], acc, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[e], b.hi[e], acc, 0, 0, 0);
}

// ---- LDS tiles ----------------------------------------------------------
// Bank model of the gfx950 LDS (64 banks of 4 bytes), as measured with the
// bank-conflict counter: a single 8-byte read is served 32 lanes at a time,
// without conflict when their 8-byte slots differ modulo 256 bytes; an
// 8-byte write, and each half of a two-address 8-byte read (ds_read2*), 16
// lanes at a time, slots modulo 128 bytes; a 16-byte read 16 lanes at a time,
// 16-byte slots modulo 256 bytes.
//
// A per-chunk operand tile holds `rows` tokens of W elements each, row-major.
// bf16 tiles have no padding; their 8-byte units (4 elements) are XOR-swizzled
// by the row.  Two layouts:
//   TileL: u ^ (4 (r & 3) + bits2..3(r)), inside aligned groups of 16 units.
//          A row-fragment read (16 consecutive rows, one unit each) is
//          conflict-free in the two-address form the compiler makes of the
//          reads of row blocks 16 rows apart, and so is an 8-byte write of
//          one unit of 16 consecutive rows; single 8-byte reads (two units per
//          32 lanes) and transposing reads pay one extra cycle per 32 lanes.
//          Its address pattern repeats every 16 units, which keeps the
//          number of address registers small.
//   TileX: W >= 128: u ^ (4 (r & 7) + 2 bit3(r) + bit2(r)) ^ bit4(u);
//          W == 64:  u ^ (4 bits1..2(r) + 2 bit3(r) + bit0(r)).
//          Conflict-free for all of the above and for the two 8-byte halves
//          of a staged 16-byte vector (consecutive threads along a row).
//   TileP: the features of each 32-wide block permuted so that the 8 k
//          positions K(g) of a row fragment are one 16-byte unit (unit
//          4 kb + g holds features 32 kb + 4 g .. + 3, then 32 kb + 16 + 4 g
//          .. + 3), units XOR-swizzled by row & 15 (W >= 128) or
//          bits 1..3 of the row (W == 64, two rows per 256 B): a row fragment
//          is one conflict-free 16-byte read straight into the operand's
//          registers.  A 4-feature group is one 8-byte half of a unit, so
//          transposing reads and 4-element writes work as on the others.
// fp32 tiles are padded by 4 elements per row instead.
template <class T, int W> struct TileL;
template <int W> struct TileL<bf16, W> {
    static_assert(W % 64 == 0, "bf16 tiles need at least 16 units per row");
    static constexpr int STRIDE = W;
    // element offset of the 4-element unit holding column col (col % 4 == 0)
    __device__ static __forceinline__ int off(int row, int col) {
        return row * W + ((((col >> 2) ^ (((row & 3) << 2) | ((row >> 2) & 3)))) << 2);
    }
};
template <class T, int W> struct TileP;
template <int W> struct TileP<bf16, W> {
    static_assert(W == 64 || W % 128 == 0, "rows of 64 or a multiple of 128 elements");
    static constexpr int STRIDE = W;
    static constexpr bool kRowUnits = true;  // a row fragment is one unit
    // element offset of 16-byte unit u (u = 4 kb + g) of row `row`
    __device__ static __forceinline__ int unit_off(int row, int u) {
        if constexpr (W >= 128) return row * W + ((u ^ (row & 15)) << 3);
        else return row * W + ((u ^ ((row >> 1) & 7)) << 3);
    }
    // element offset of the 4-element group holding feature col (col % 4 == 0)
    __device__ static __forceinline__ int off(int row, int col) {
        const int w = col & 31;
        return unit_off(row, 4 * (col >> 5) + ((w & 15) >> 2)) + ((w >> 4) << 2);
    }
};
template <class T, int W> struct TileX;
template <int W> struct TileX<bf16, W> {
    static_assert(W == 64 || W % 128 == 0, "rows of 64 or a multiple of 128 elements");
    static constexpr int STRIDE = W;
    __device__ static __forceinline__ int off(int row, int col) {
        const int u = col >> 2;
        if constexpr (W >= 128)
            return row * W + ((u ^ (((row & 7) << 2) | ((row >> 2) & 2) | ((row >> 2) & 1)) ^ ((u >> 4) & 1)) << 2);
        else
            return row * W + ((u ^ ((((row >> 1) & 3) << 2) | ((row >> 2) & 2) | (row & 1))) << 2);
    }
};
template <int W> struct TileL<float, W> {
    static constexpr int STRIDE = W + 4;
    __device__ static __forceinline__ int off(int row, int col) { return row * (W + 4) + col; }
};

// Row fragment: lane (row, g) holds columns {32kb+4g..+3, 32kb+16+4g..+3}.
template <class L, class = void> struct RowUnits { static constexpr bool value = false; };
template <class L> struct RowUnits<L, decltype(void(L::kRowUnits))> { static constexpr bool value = L::kRowUnits; };

template <class T, int W, class L = TileL<T, W>>
__device__ __forceinline__ Frag<T> lds_frag_row(const T* t, int row, int kb, int g) {
    if constexpr (RowUnits<L>::value) {
        Frag<T> f;
        f.v = *(const bf16x8*)(t + L::unit_off(row, 4 * kb + g));
        return f;
    } else {
        return frag2(t + L::off(row, 32 * kb + 4 * g), t + L::off(row, 32 * kb + 16 + 4 * g));
    }
}

// Column fragment of rows j0..j0+31 and columns m0..m0+15 (j0 % 32 == 0,
// m0 % 16 == 0): lane l holds X[j0+4g+e][m0+l%16] in slot e and
// X[j0+16+4g+e][m0+l%16] in slot 4+e, g = l/16 -- the same k positions as a
// row fragment, so it pairs with row fragments and accumulator fragments.
// bf16: two ds_read_b64_tr_b16.  Within each group of 16 lanes that
// instruction returns to lane i, slot e, element i%4 of the 8 bytes addressed
// by lane 4e+i/4; lane 16g+l' therefore addresses row j0+4g+l'/4 at column
// m0+4(l'%4).  fp32: eight scalar reads.
template <class T, int W, class L = TileL<T, W>> struct ColRead;
template <int W, class L> struct ColRead<bf16, W, L> {
    __device__ static __forceinline__ Frag<bf16> get(const bf16* t, int j0, int m0, int lane) {
        typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
        const int g = lane >> 4, lp = lane & 15;
        const int row = j0 + 4 * g + (lp >> 2), col = m0 + 4 * (lp & 3);
        const bf16* p = t + L::off(row, col);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 16 * W));
        Frag<bf16> f;
        f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return f;
    }
};
template <int W, class L> struct ColRead<float, W, L> {
    __device__ static __forceinline__ Frag<float> get(const float* t, int j0, int m0, int lane) {
        const int g = lane >> 4, m = m0 + (lane & 15);
        constexpr int S = TileL<float, W>::STRIDE;
        Frag<float> f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f.lo[e] = t[(j0 + 4 * g + e) * S + m];
            f.hi[e] = t[(j0 + 16 + 4 * g + e) * S + m];
        }
        return f;
    }
};

// 1/x on the transcendental unit (1 ulp).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// lambda^k from log2(lambda), with lambda^0 = 1 also for lambda = 0.
// Token range [s0, s1) of packed sequence b in a head row of N tokens, the
// offsets clamped so that any values stay inside the row.
__device__ __forceinline__ void varlen_range(const int32_t* cu, int b, int64_t N, int64_t* s0, int64_t* s1) {
    const int64_t a = min(max((int64_t)cu[b], (int64_t)0), N);
    *s0 = a;
    *s1 = min(max((int64_t)cu[b + 1], a), N);
}

__device__ __forceinline__ float lam_pow(float log2lam, int k) {
    return k == 0 ? 1.0f : __builtin_amdgcn_exp2f((float)k * log2lam);
}

// elu(x) + 1 ("From standard attention to linear attention" sec. 4.1).
template <class T> __device__ __forceinline__ float phi_elu1(float x);
template <> __device__ __forceinline__ float phi_elu1<bf16>(float x) { return x > 0.f ? x + 1.f : __expf(x); }
template <> __device__ __forceinline__ float phi_elu1<float>(float x) { return x > 0.f ? x + 1.f : expf(x); }

// max(x, 0) ("Attention is also an FFN" sec. 5.1 names ReLU beside elu+1).
__device__ __forceinline__ float phi_relu(float x) { return x > 0.f ? x : 0.f; }

// The elementwise feature maps (F = d_k) by kind.
template <class T, int PHI> __device__ __forceinline__ float phi_elem(float x) {
    if constexpr (PHI == LA_PHI_RELU) return phi_relu(x);
    else if constexpr (PHI == kPhiIdentity) return x;
    else return phi_elu1<T>(x);
}

template <class T> __device__ __forceinline__ void sincos_rf(float u, float* s, float* c);
template <> __device__ __forceinline__ void sincos_rf<bf16>(float u, float* s, float* c) {
    *s = __sinf(u);
    *c = __cosf(u);
}
template <> __device__ __forceinline__ void sincos_rf<float>(float u, float* s, float* c) {
    sincosf(u, s, c);
}
template <class T> __device__ __forceinline__ float exp_rf(float x);
template <> __device__ __forceinline__ float exp_rf<bf16>(float x) { return __expf(x); }
template <> __device__ __forceinline__ float exp_rf<float>(float x) { return expf(x); }

// Unpack a 16-byte vector of VEC elements into floats (bit operations only,
// so the vector never leaves registers).
__device__ __forceinline__ void unpack16(const uint4& u, float* out, const bf16*) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        out[2 * e] = __uint_as_float(w[e] << 16);
        out[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack16(const uint4& u, float* out, const float*) {
    out[0] = __uint_as_float(u.x);
    out[1] = __uint_as_float(u.y);
    out[2] = __uint_as_float(u.z);
    out[3] = __uint_as_float(u.w);
}

// 16 bytes at byte offset voff (per lane) from a base address that is the
// same in every lane, through a raw buffer resource: the lane's offset is a
// 32-bit register that stays fixed from chunk to chunk, so the loads of a
// chunk need no 64-bit address arithmetic per load.  voff must stay below
// 2^31 (the resource's range).
__device__ __forceinline__ uint4 load16(const void* base, uint32_t voff) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                                                        0x00020000);
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
}

__device__ __forceinline__ float wave_sum_xor(float v, int mask_lo, int mask_hi) {
    for (int m = mask_lo; m <= mask_hi; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Sum over aligned groups of N lanes (N = 2, 4, 8 or 16), the result in
// every lane of the group, with DPP lane moves in the vector unit instead of
// LDS permutes: quad_perm swaps for lanes 1 and 2 apart, then the mirror of
// the half row (lane i of 8 takes lane 7 - i, which lies in the other quad)
// and of the row (i of 16 takes 15 - i, in the other half row); each step
// adds a lane that holds the sum of a disjoint group of the same size.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group of 2 to 16 lanes");
    auto dpp = [](float x, auto ctrl_c) {
        constexpr int CTRL = decltype(ctrl_c)::value;
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
    };
    v += dpp(v, std::integral_constant<int, 0xB1>{});  // quad_perm(1, 0, 3, 2)
    if constexpr (N >= 4) v += dpp(v, std::integral_constant<int, 0x4E>{});  // quad_perm(2, 3, 0, 1)
    if constexpr (N >= 8) v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
    if constexpr (N >= 16) v += dpp(v, std::integral_constant<int, 0x140>{});  // row_mirror
    return v;
}

}  // namespace la
