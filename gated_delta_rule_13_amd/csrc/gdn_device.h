// gdn_device.h -- gfx950 building blocks for the chunkwise gated delta rule:
// MFMA fragment helpers, bf16 hi/lo splitting, wave-level scans.
//
// MFMA shapes used (CDNA4, wave64):
//   v_mfma_f32_16x16x32_bf16  A 16x32, B 32x16, D 16x16 fp32
//   v_mfma_f32_16x16x4_f32    A 16x4,  B 4x16,  D 16x16 fp32
// Lane layout, with lane = 16*h + n (n in 0..15, h in 0..3):
//   A operand: row m = n, k-slots h*KPL .. h*KPL+KPL-1  (KPL = 8 bf16 / 1 f32)
//   B operand: col  = n, same k-slots
//   D (4 floats): col = n, rows 4*h + j, j = 0..3
// The contraction index may be permuted freely as long as A and B agree; the
// kernels use that to feed an accumulator (rows 4h+j of consecutive tiles)
// straight back as the next product's operand, and load the other operand
// from LDS with the same permutation ("perm-k").
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Raw buffer resource over [base, base + bytes), bytes < 2^31.  The hardware
// range check of raw buffers makes loads at byte offsets >= bytes return zero
// and drops stores there; offsets are per lane, 32-bit.
typedef __amdgpu_buffer_rsrc_t buf_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
__device__ __forceinline__ buf_t buffer_over(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// one bf16 as its raw bits in the low half of a 32-bit register (kept
// unpacked so that nothing waits for the load until the value is used)
__device__ __forceinline__ uint32_t buf_load_bf16_bits(buf_t r, uint32_t off) {
    return (uint32_t)(unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __builtin_bit_cast(float, b << 16); }
__device__ __forceinline__ uint2 buf_load_8B(buf_t r, uint32_t off) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint4 buf_load_16B(buf_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
// Streaming output stores (written once, never read back by the kernel).
// Cache-policy bits of the gfx950 buffer store: 1 = sc0, 2 = nt, 16 = sc1.
// buf_store: non-temporal only.  buf_store_wt: 16-byte pieces written
// through at system scope as well, which leaves no partly written lines for
// a later write-back (measured: the written bytes equal the output size,
// against 16 % more with non-temporal only; the same speed up to d_v = 192,
// 6 % slower at d_v = 256).  8-byte pieces written through would reach
// memory as partial sectors, so bf16 output stays non-temporal only.
constexpr int kStoreNtSys = 1 | 2 | 16;
constexpr int kStoreNt = 2;
__device__ __forceinline__ void buf_store(buf_t r, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kStoreNt);
}
__device__ __forceinline__ void buf_store_wt(buf_t r, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kStoreNtSys);
}
__device__ __forceinline__ void buf_store(buf_t r, uint32_t off, bf16x4 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0, kStoreNt);
}

// Round to bf16 (nearest-even) and the exact fp32 residual rounded again:
// x ~= hi + lo with |x - hi - lo| <= 2^-17 |x| (about 16 significant bits).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

// Eight accumulator values (two consecutive 16-row tiles, rows 4h+j) as the
// hi / lo halves of a perm-k bf16 operand.
__device__ __forceinline__ void split8(const f32x4& a0, const f32x4& a1, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        __bf16 h0, l0, h1, l1;
        split_bf16(a0[e], h0, l0);
        split_bf16(a1[e], h1, l1);
        hi[e] = h0; lo[e] = l0;
        hi[e + 4] = h1; lo[e + 4] = l1;
    }
}

// perm-k bf16 operand from an LDS row: elements [32s + 4h, +4) and
// [32s + 16 + 4h, +4) -- matches split8 of accumulator tiles 2s, 2s+1.
__device__ __forceinline__ bf16x8 ld_perm8(const __bf16* row, int s, int h) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(row + 32 * s + 4 * h);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(row + 32 * s + 16 + 4 * h);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// natural bf16 operand from an LDS row: elements [32s + 8h, +8).
__device__ __forceinline__ bf16x8 ld_nat8(const __bf16* row, int s, int h) {
    return *reinterpret_cast<const bf16x8*>(row + 32 * s + 8 * h);
}

// Value of lane (l - N) within the same row of 16 lanes, 0 where that lane
// lies before the row (DPP row_shr:N).
template <int N>
__device__ __forceinline__ float row_shr_zero(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N,
                                                                  0xf, 0xf, false));
}
__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele steps
// 1, 2, 4, 8 within each row of 16 lanes (register-to-register, no LDS
// round trip), then each row adds the totals of the rows before it.
__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
    x += row_shr_zero<1>(x);
    x += row_shr_zero<2>(x);
    x += row_shr_zero<4>(x);
    x += row_shr_zero<8>(x);
    const float t0 = lane_value(x, 15), t1 = lane_value(x, 31), t2 = lane_value(x, 47);
    const int row = lane >> 4;
    return x + ((row >= 1 ? t0 : 0.f) + (row >= 2 ? t1 : 0.f) + (row >= 3 ? t2 : 0.f));
}

}  // namespace gdn
