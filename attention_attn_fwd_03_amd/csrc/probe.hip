// Measurement probe: the matrix-core ceiling of the prefill kernel's inner loop on this part.
//
// Same launch shape as fwd_bf16_kernel<128, 32, false, *> (256 threads, three workgroups per CU,
// two 19 KB LDS stages), and per 32-key step the same matrix work and LDS operand reads: eight
// v_mfma_f32_32x32x16_bf16 of S^T = K Q^T with K read from LDS, then eight of O^T = V^T P^T with
// V^T read by ds_read_b64_tr_b16.  No softmax, no global loads, no barrier: how many FLOP/s the
// matrix cores and LDS alone sustain under the part's power limit, the ceiling against which the
// prefill kernel's own fraction of the nominal peak is read.
#include <hip/hip_runtime.h>

#include "attn_device.hpp"
#include "kernels.hpp"

namespace attnfwd {

namespace {
constexpr int kProbeD = 128, kProbeKpb = kProbeD * 2 + 16, kProbeVpb = kProbeD * 2 + 64;
constexpr int kProbeKTile = 9216, kProbeVTile = 10240;  // the prefill kernel's stage sizes at d = 128
}  // namespace

__global__ __launch_bounds__(256, 3) void probe_mfma_lds_kernel(int steps, float* sink) {
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds[2][kProbeKTile];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds[2][kProbeVTile];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  // Small bf16 values (1/64 .. 1/4 in magnitude) so that nothing overflows over long runs.
  for (int i = tid; i < kProbeKTile / 2; i += 256) {
    const __bf16 x = (__bf16)((float)((i * 37) % 17 - 8) * (1.f / 64.f));
    ((__bf16*)k_lds[0])[i] = x;
    ((__bf16*)k_lds[1])[i] = -x;
  }
  for (int i = tid; i < kProbeVTile / 2; i += 256) {
    const __bf16 x = (__bf16)((float)((i * 29) % 13 - 6) * (1.f / 64.f));
    ((__bf16*)v_lds[0])[i] = x;
    ((__bf16*)v_lds[1])[i] = -x;
  }
  __syncthreads();
  bf16x8 qf[kProbeD / 16];
  for (int ks = 0; ks < kProbeD / 16; ++ks)
    for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)((float)((lane + 3 * ks + e) % 7 - 3) * (1.f / 32.f));
  f32x16 o[kProbeD / 32];
  for (int dt = 0; dt < kProbeD / 32; ++dt)
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  const int k_lane = col * kProbeKpb + h * 16;
  const int v_lane = (4 * h + ((lane & 15) >> 2)) * kProbeVpb + ((lane >> 4) & 1) * 32 + (lane & 3) * 8;
  for (int step = 0; step < steps; ++step) {
    const int st = step & 1;
    f32x16 s = {};
    const unsigned char* Ks = k_lds[st] + k_lane;
#pragma unroll
    for (int ks = 0; ks < kProbeD / 16; ++ks) s = mfma_32x32x16(*(const bf16x8*)(Ks + ks * 32), qf[ks], s);
    // P as bf16, from the scores (one conversion per pair, as the real kernel's packing)
    unsigned pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pk[i] = pack_bf16x2(s[2 * i] * (1.f / 256.f), s[2 * i + 1] * (1.f / 256.f));
    const unsigned char* Vs = v_lds[st] + v_lane;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[4 * half], pk[4 * half + 1], pk[4 * half + 2],
                                                         pk[4 * half + 3]});
#pragma unroll
      for (int dt = 0; dt < kProbeD / 32; ++dt) {
        const u32x2 r0 = lds_read_tr16(Vs + 16 * half * kProbeVpb + dt * 64);
        const u32x2 r1 = lds_read_tr16(Vs + (16 * half + 8) * kProbeVpb + dt * 64);
        o[dt] = mfma_32x32x16(__builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3)), pb, o[dt]);
      }
    }
  }
  float acc = 0.f;
  for (int dt = 0; dt < kProbeD / 32; ++dt)
    for (int i = 0; i < 16; ++i) acc += o[dt][i];
  sink[(size_t)blockIdx.x * 256 + tid] = acc;
}

hipError_t launch_probe_mfma(int workgroups, int steps, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_lds_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, steps, sink);
  return hipGetLastError();
}

}  // namespace attnfwd
