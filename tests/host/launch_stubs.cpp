// Host-only stand-ins for the GPU side of libattnfwd, for the sanitizer build of the C ABI
// (tests/test_host_sanitizers.py).  api.cpp is compiled by the host compiler under AddressSanitizer
// and UndefinedBehaviorSanitizer and linked with these: every launch "succeeds" without touching
// the device or any tensor memory, so argument validation, launch planning and workspace layout
// run on the CPU with any argument values, including fake pointers.  The launch-shape queries
// return the values the GPU build's prefill.hip returns.  Nothing here is part of the library.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace attnfwd {

int prefill_block_q(bool) { return 128; }
int prefill_block_k(bool f32, int d) { return f32 ? 32 : (d == 128 ? 32 : 64); }
int prefill_threads(bool) { return 256; }
int prefill_lds_bytes(bool, int) { return 0; }
hipError_t launch_prefill(const FwdArgs&, bool, int, hipStream_t) { return hipSuccess; }
hipError_t launch_prefill_varlen(const FwdArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_prefill_fp8(const FwdArgs&, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_decode(const DecArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_backward(const BwdArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_probe_mfma(int, int, int, float*, hipStream_t) { return hipSuccess; }
int decode_workers(int, bool, bool packed) { return packed ? 768 : 512; }
void* decode_scratch() {
  alignas(256) static unsigned char fake[256];
  return fake;  // never dereferenced: the stubbed launches read nothing
}

}  // namespace attnfwd

// Present only in the host-stub library: lets a test refuse to make valid-argument calls (which, in the real
// library, would launch kernels on fake pointers) against anything else.
extern "C" int attn_host_stub_build(void) { return 1; }
