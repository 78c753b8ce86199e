// Device-side building blocks shared by the prefill and decode kernels (gfx950 / CDNA4).
//
// Layout facts used throughout (checked on the hardware with a lane-layout probe):
//  * v_mfma_f32_32x32x16_bf16: lane l supplies A[m = l%32][k = 8*(l/32) + e] and
//    B[k = 8*(l/32) + e][n = l%32] for e = 0..7; it receives C[m][n = l%32] for
//    m = 8*(i/4) + 4*(l/32) + i%4, i = 0..15.
//  * v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][l/32] and B[l/32][l%32]; same C layout.
//  * ds_read_b64_tr_b16: inside each 16-lane group, lane i receives element i%4 of the 8-byte
//    piece addressed by lane 4c + i/4, for c = 0..3.  If lane j of the group addresses row
//    r0 + j/4, columns c0 + 4*(j%4) .. +3 of a row-major 16-bit matrix, lane i receives
//    rows r0..r0+3 of column c0 + i: a column read, which is how V reaches the MFMA A operand.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnfwd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) unsigned short lds_u16;

// log2(e): scores are kept in base 2 so that exp becomes one v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The reference maximum of a row is only raised when a new tile's maximum exceeds it by more
// than this many binary orders; until then probabilities are computed against the stale
// reference (they stay below 2^kRescaleSlack) and the accumulator is not rescaled.  The
// final O = acc / l is unchanged because acc and l share the reference.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Reductions over the lane pair (l, l ^ 32).  v_permlane32_swap with both operands = x hands
// back {x[l], x[l - 32]} in lanes >= 32 and {x[l], x[l + 32]} in lanes < 32 (as the pair of
// results in some order), so a symmetric reduction of the two results is the pair's value.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ float bf16_bits_to_float(unsigned short b) {
  return __builtin_bit_cast(float, ((unsigned)b) << 16);
}

// Transposed 4 x 16-bit read from LDS (see the header comment).
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_generic_ptr) {
  const lds_i16x4* p = (const lds_i16x4*)(lds_u16*)lds_generic_ptr;
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p));
  return __builtin_bit_cast(u32x2, r);
}

// s_waitcnt immediate that waits until at most n vector-memory instructions are outstanding and
// leaves the LDS/scalar and export counters unconstrained (vmcnt split over bits 3:0 and 15:14).
constexpr unsigned vmcnt_at_most(unsigned n) { return 0x0F70u | (n & 0xFu) | ((n >> 4) << 14); }

typedef __attribute__((address_space(3))) void lds_void_t;

// N wave-wide global->LDS loads of one tile: load i writes LDS bytes [j*1024, +1024) of `stage`,
// j = wave + waves*i (loads with j >= total are skipped; j is uniform), from byte offset voff[i]
// of the buffer `rs`.  The buffer covers exactly the tile's valid rows, so rows past the end of
// the sequence read as zeros; lanes that land on pad slots carry an offset past any buffer and
// write zeros there, which nothing reads.  No lane needs its own branch.  (The scalar offset
// is kept 0: only the per-lane offset is range-checked.)
template <int N>
__device__ __forceinline__ void issue_loads(__amdgpu_buffer_rsrc_t rs, unsigned char* stage, int wave, int waves,
                                            int total, const unsigned (&voff)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int j = wave + waves * i;
    if (j < total) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(stage + j * 1024), 16, voff[i], 0, 0, 0);
  }
}

// Buffer descriptor over rows [row0, nrows) of a row-major [nrows, D] bf16 matrix at `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const unsigned short* base, int row0, int nrows,
                                                            int row_bytes) {
  const int left = nrows - row0 > 0 ? nrows - row0 : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)base + (size_t)row0 * row_bytes), 0,
                                           left * row_bytes, 0x00020000);
}

// Online-softmax state of one query row as held by one lane.  Lanes l and l ^ 32 hold the
// same row and keep identical m; each keeps the partial sum over the keys it holds.
struct RowState {
  float m;   // reference maximum, base-2 scaled units (score * |scale| * log2 e); -inf at start
  float l;   // this lane's partial sum of probabilities, relative to m
  float mb;  // what the exponentials subtract: m, or 0 while m is -inf (a row that has seen no key)
};

// The online softmax of one tile ("003-注意力机制详解…", §二: new row max, running sum and
// accumulator rescaled by exp(old max - new max), exponentials of the tile, row sums), split so
// that the rarely taken rescale branch comes first and the exponentials form straight-line code
// that the scheduler can interleave with MFMA work of the next tile.
//
// A tile is NB 32-key blocks in the S^T accumulator layout: lane value i of block kb is key
// kbase + 32*kb + 8*(i/4) + (i%4), where kbase = tile start + 4*(lane/32).  Scores are scaled
// here, in fp32, by c = |scale| * log2(e).

// Edge tiles: keys outside [kbase + lo, kbase + hi] become -inf.
template <int NB>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[NB], int lo, int hi) {
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ci = kb * 32 + (i >> 2) * 8 + (i & 3);
      const bool vis = (ci >= lo) & (ci <= hi);
      s[kb][i] = vis ? s[kb][i] : -INFINITY;
    }
}

// Row maximum of the tile; raises the reference maximum (rescaling the running sum and the
// accumulator) only when the tile's maximum exceeds it by more than kRescaleSlack.  Returns
// the reference to subtract, with the -inf guard of a row that has seen no key yet.
// A lane holds half of its row's keys; the row's maximum exceeds the reference by more than the
// slack exactly when one of the two halves' maxima does (scaling by c > 0 keeps the order, also
// after rounding), so the lanes test their own halves and the maximum over the lane pair is
// formed only in the rarely taken branch that raises the reference.
template <int NB, int ND>
__device__ __forceinline__ float update_max(const f32x16 (&s)[NB], RowState& st, f32x16 (&o)[ND], float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
  // c > 0 and finite, so a half that saw only masked keys stays at -inf
  if (wave_any(mx * c > st.m + kRescaleSlack)) {
    const float tmax = pair_max(mx) * c;
    const bool need = tmax > st.m + kRescaleSlack;
    const float m_new = need ? tmax : st.m;
    const float alpha = need ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[dt] *= alpha;
    st.m = m_new;
    st.mb = (m_new == -INFINITY) ? 0.f : m_new;
  }
  return st.mb;
}

// Probabilities p = exp2(s * c - mb) of a 32-key block, added to the running sum in fp32 and
// returned packed as bf16 pairs (round to nearest even) in the order of the P.V B operand.
// Masked keys hold s = -inf and c > 0, so they give exp2(-inf) = 0 without a select (a zero
// scale is run as Q = 0 with c = 1, which yields the same all-zero scores).
__device__ __forceinline__ void exp_block(const f32x16& s, float c, float mb, RowState& st, unsigned (&pk)[8]) {
  float l0 = __builtin_amdgcn_exp2f(fmaf(s[0], c, -mb));
  float l1 = __builtin_amdgcn_exp2f(fmaf(s[1], c, -mb));
  pk[0] = pack_bf16x2(l0, l1);
#pragma unroll
  for (int i = 2; i < 16; i += 2) {
    const float e0 = __builtin_amdgcn_exp2f(fmaf(s[i], c, -mb));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c, -mb));
    l0 += e0;
    l1 += e1;
    pk[i >> 1] = pack_bf16x2(e0, e1);
  }
  st.l += l0 + l1;
}

// fp32 variant for the fp32 path (P stays fp32).
__device__ __forceinline__ void exp_block_f32(const f32x16& s, float c, float mb, RowState& st, float (&p)[16]) {
  p[0] = __builtin_amdgcn_exp2f(fmaf(s[0], c, -mb));
  p[1] = __builtin_amdgcn_exp2f(fmaf(s[1], c, -mb));
  float l0 = p[0], l1 = p[1];
#pragma unroll
  for (int i = 2; i < 16; i += 2) {
    const float e0 = __builtin_amdgcn_exp2f(fmaf(s[i], c, -mb));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c, -mb));
    l0 += e0;
    l1 += e1;
    p[i] = e0;
    p[i + 1] = e1;
  }
  st.l += l0 + l1;
}

// How Q enters the kernels: as given, with its sign flipped (negative scale, run as |scale|), or
// as zeros (scale = 0, run with c = 1).  All three are exact.  The mode is applied branch-free as
// (w & keep) ^ flip, so the loads that feed it are not split up by control flow.
enum QMode : int { kQAsIs = 0, kQNegate = 1, kQZero = 2 };

struct QTransform {
  unsigned keep, flip;
};
__device__ __forceinline__ QTransform q_transform(int qmode) {
  QTransform t;
  t.keep = qmode == kQZero ? 0u : 0xFFFFFFFFu;
  t.flip = qmode == kQNegate ? 0x80008000u : 0u;
  return t;
}

// Q fragment word with the mode applied; `valid` false gives zeros (a row or head past the end).
__device__ __forceinline__ u32x4 q_word(u32x4 w, QTransform t, bool valid) {
  const unsigned keep = valid ? t.keep : 0u;
  return (w & keep) ^ (valid ? t.flip : 0u);
}

// Read-only view of a buffer that stays constant for the whole kernel: a load through it at a
// wave-uniform address becomes a scalar load, which is not counted with the vector loads in
// flight and so never makes the wave wait for them.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* kernel_constant(const T* p) {
  return (const __attribute__((address_space(4))) T*)p;
}

}  // namespace attnfwd
