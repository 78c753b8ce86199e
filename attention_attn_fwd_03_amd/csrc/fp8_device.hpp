// 8-bit float helpers shared by the FP8 decode and prefill kernels (gfx950 / CDNA4).
#pragma once
#include "attn_device.hpp"

namespace attnfwd {

// Element formats: bf16, or an 8-bit float code (OCP E4M3 / E5M2) with one scale per tensor.
enum KvFormat : int { kKvBf16 = 0, kKvE4M3 = 1, kKvE5M2 = 2 };

// Eight 8-bit float codes (bytes 0..7 of w) as eight bf16 values; exact for both formats.
template <int KV>
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w) {
  bf16x2 p0, p1, p2, p3;
  if constexpr (KV == kKvE4M3) {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  } else {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w[0], 1.0f, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w[0], 1.0f, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w[1], 1.0f, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w[1], 1.0f, true);
  }
  const u32x4 r = {__builtin_bit_cast(unsigned, p0), __builtin_bit_cast(unsigned, p1), __builtin_bit_cast(unsigned, p2),
                   __builtin_bit_cast(unsigned, p3)};
  return __builtin_bit_cast(bf16x8, r);
}

typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// ds_read_b64_tr_b8: inside each 16-lane group, lane i receives byte i%8 of the 8-byte pieces
// addressed by lanes i/8 + 2c, c = 0..7 (checked on the hardware with a lane-layout probe).  If
// lane j of the group addresses row r0 + j/2, bytes c0 + 8*(j%2) .. +7 of a row-major byte
// matrix, lane i receives rows r0 .. r0+7 of column c0 + i.
__device__ __forceinline__ u32x2 lds_read_tr8(const void* lds_generic_ptr) {
  const lds_i32x2* p = (const lds_i32x2*)(__attribute__((address_space(3))) unsigned char*)lds_generic_ptr;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(const_cast<lds_i32x2*>(p)));
}

// Row order of an FP8 V stage: LDS row r holds tile row r with bits 2 and 3 exchanged, so that
// the 8 rows one ds_read_b64_tr_b8 gives a lane (rows 16j + 8h .. +7 of the stage) are tile rows
// 16j + 8*(e/4) + 4h + e%4 for byte e -- the rows whose probabilities the lane holds at
// k = 8h + e of the P operand (the S^T accumulator rounded to bf16, see exp_block).
__host__ __device__ constexpr int fp8_v_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

typedef __attribute__((ext_vector_type(8))) int i32x8;

// v_mfma_f32_32x32x64_f8f6f4 without block scales, both operands in format FMT.  Lane l supplies
// 32 codes of row l%32 of A and 32 codes of column l%32 of B; byte j of A in lane l meets byte j of
// B in lanes with the same l/32, so any assignment of the 64 contraction indices to (l/32, byte)
// serves if A and B use the same one (checked on the hardware with random codes).  C has the
// 32x32 accumulator layout of the bf16 MFMA.
template <int FMT>
__device__ __forceinline__ f32x16 mfma_32x32x64_f8(i32x8 a, i32x8 b, f32x16 c) {
  constexpr int code = FMT == kKvE4M3 ? 0 : 1;  // 0: E4M3, 1: E5M2
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, code, code, 0, 0, 0, 0);
}

}  // namespace attnfwd
