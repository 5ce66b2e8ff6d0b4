// Device-side bf16 primitives for gfx950.
//
// The det_gemm contract (RL-Kernel operator page "Batch-Invariant Deterministic
// GEMM (det_gemm)", section "Ascend NPU backend", bullet "Reduction tree") needs
// two scalar operations besides the leaf product-sum:
//   * rounding an fp32 value to bf16 with round-to-nearest-even, and
//   * the bf16 add: the fp32 sum of two bf16 values, rounded to bf16.
// On gfx950 both map to single VALU instructions that work on pairs:
//   v_cvt_pk_bf16_f32  rounds two fp32 values to bf16 (RNE) and packs them;
//   v_dot2_f32_bf16    with the constant pair (1.0, 1.0) adds the two bf16
//                      halves of a register in fp32 (the products are exact,
//                      so the only rounding is that of the fp32 sum).
// A tree node therefore lives in a register as its unrounded fp32 value; it is
// rounded exactly once, together with its sibling, by the v_cvt_pk that forms
// the pair its parent adds.  The addend -0.0 keeps the sign of an exact zero sum
// as IEEE addition gives it (x + (-0) == x for every x, including -0 and +0).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace detgemm {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Round two fp32 values to bf16 (RNE) and pack them: a in bits 0..15, b in 16..31.
__device__ __forceinline__ bf16x2 round_pair(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_convertvector(v, bf16x2);
}

// fp32 sum of the two bf16 halves of a packed pair.  The library is built
// without the two-address v_dot2c_f32_bf16 form (target feature dot13-insts
// off), so this is the three-address v_dot2_f32_bf16 with the -0.0 addend in a
// register that stays live across the loop, instead of a v_dot2c plus a move
// per add to initialise its accumulator.  Being a builtin, the compiler also
// inserts the wait states a VALU read of a dot result needs.
__device__ __forceinline__ float sum_pair(bf16x2 p) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(p, one, -0.0f, false);
}

// One tree add on unrounded node values: round both children, add them in fp32.
// The result is the parent's unrounded value.
__device__ __forceinline__ float merge(float left, float right) {
    return sum_pair(round_pair(left, right));
}

__device__ __forceinline__ f32x4 merge4(f32x4 l, f32x4 r) {
    f32x4 o;
    o[0] = merge(l[0], r[0]);
    o[1] = merge(l[1], r[1]);
    o[2] = merge(l[2], r[2]);
    o[3] = merge(l[3], r[3]);
    return o;
}

__device__ __forceinline__ uint32_t pair_bits(bf16x2 p) {
    return __builtin_bit_cast(uint32_t, p);
}

}  // namespace detgemm
