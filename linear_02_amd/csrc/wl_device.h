// Device-side helpers of the reconstruct-and-project linear kernels.
// gfx950 (CDNA4) only: wave64, v_dot2c_f32_bf16, v_cvt_pk_bf16_f32, DPP row
// broadcasts and the bf16 matrix-core instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wl {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Load through the global address space. A pointer the compiler cannot trace to
// a kernel argument (chosen by a select, rebuilt from registers) is otherwise
// loaded with a flat instruction, which also counts on the scalar-load counter,
// so the next wait for a scalar load would wait for this load as well.
template <class T>
__device__ __forceinline__ T ldg(const T *p) {
    return *(const __attribute__((address_space(1))) T *)p;
}

// bf16 bit pattern -> fp32. Exact: a bf16 is the upper half of a binary32.
__device__ __forceinline__ float bf16_f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f_bf16(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// acc + dot of two 16-byte pieces (8 bf16 each); products are exact in fp32
// and are added into the fp32 accumulator. The components are named one by
// one: bit-casting a subscripted vector element inside an unrolled loop
// (bit_cast(bf16x2, w[j])) reads element 0 for every j with this compiler.
__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, x), acc,
                                           false);
}
__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float acc) {
    acc = dot2(w.x, x.x, acc);
    acc = dot2(w.y, x.y, acc);
    acc = dot2(w.z, x.z, acc);
    return dot2(w.w, x.w, acc);
}

template <int ctrl, int row_mask = 0xF, bool bound_ctrl = true>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, row_mask, 0xF,
                                                      bound_ctrl));
}

// Sum over the 64 lanes of a wave. The full sum lands in lane 63; the other
// lanes hold partial sums. Butterflies inside each 16-lane row (quad swaps,
// half-row and row mirrors), then the row-15 and lane-31 broadcasts fold rows
// 0..3 into row 3.
__device__ __forceinline__ float wave_sum_last(float v) {
    v += dpp<0xB1>(v);             // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);             // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);            // row_half_mirror
    v += dpp<0x140>(v);            // row_mirror: every lane holds its row's sum
    v += dpp<0x142, 0xA, false>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp<0x143, 0xC, false>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Sum over the 64 lanes, returned in every lane.
__device__ __forceinline__ float wave_sum(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sum_last(v)), 63));
}

// Swizzled position of piece kc of LDS row `row` (rows of KP pieces). The XOR
// pattern varies over 16 consecutive rows, so the 16 lanes that one LDS pass
// serves (32 rows x one piece per fragment read) land on distinct 4-bank
// groups of the 64 banks.
template <int KP>
__device__ __forceinline__ int swz_key(int row) {
    constexpr int sh = KP == 8 ? 0 : KP == 4 ? 1 : 2;
    return ((row >> sh) ^ (row >> 3)) & (KP - 1);
}
template <int KP>
__device__ __forceinline__ int swz(int row, int kc) {
    return row * KP + (kc ^ swz_key<KP>(row));
}

// One direct-to-LDS load: the wave's 64 lanes each fetch 16 bytes from their
// own global address into 64 consecutive 16-byte LDS slots starting at dst.
__device__ __forceinline__ void lds_dma16(const u32x4 *src, u32x4 *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// tanh-approximated GELU (Hendrycks & Gimpel, 2016), fp32, device tanhf.
__device__ __forceinline__ float gelu_tanh(float z) {
    const float c0 = 0.7978845608028654f;   // sqrt(2 / pi)
    const float c1 = 0.044715f;
    return 0.5f * z * (1.0f + tanhf(c0 * (z + c1 * z * z * z)));
}
// The same function for results rounded to bf16 (2^-9 relative): since
// 1 + tanh(u) = 2 / (1 + e^(-2u)), 0.5 z (1 + tanh(u)) = z / (1 + e^(-2u)).
// With u = c0 (z + c1 z^3), -2u log2(e) = z (k1 + k2 z^2), k1 = -2 c0 log2(e),
// k2 = k1 c1; the power of two comes from v_exp_f32 and the quotient from the
// hardware reciprocal (v_rcp_f32, 1 ulp) times z: a few ulp of fp32 in all, no
// cancellation for any sign of u, and eight instructions fewer per element
// than an IEEE division. Large u give exactly z (the power underflows to 0 and
// 1/1 = 1), large negative u a zero of z's sign.
__device__ __forceinline__ float gelu_tanh_bf16out(float z) {
    constexpr float k1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;   // sqrt(2 / pi), log2(e)
    constexpr float k2 = k1 * 0.044715f;
    const float a = z * __builtin_fmaf(z * z, k2, k1);
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a));
}

}  // namespace wl
