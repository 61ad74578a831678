// hip_stub.cpp - host-only stand-ins for the kernel launchers and the few
// HIP runtime calls that the C ABI (fa_api.cpp) makes, so that the ABI's host
// code can be built with g++ under AddressSanitizer/UndefinedBehaviorSanitizer
// and run on a machine without a GPU. Test infrastructure only.
//
// * The launchers record the parameter block of the last launch and count
//   launches; they touch no memory behind the pointers.
// * hipMemcpyAsync copies host memory (the tests pass host arrays where the
//   library expects device index arrays); hipStreamSynchronize does nothing.
#include <string.h>

#include "stub_state.h"

StubState g_stub;

namespace fa {

hipError_t launch_fwd(const FwdParams& p, Dt, int, bool, int grid_blocks, hipStream_t) {
  g_stub.launches++;
  g_stub.last_kind = StubState::FWD;
  g_stub.fwd = p;
  g_stub.grid = grid_blocks;
  return hipSuccess;
}

int fwd_block_rows(Dt dt) { return dt == Dt::F32 ? 32 : 256; }

hipError_t launch_fwd_paged(const FwdParams& p, Dt, int, bool, int grid_blocks, hipStream_t) {
  g_stub.launches++;
  g_stub.last_kind = StubState::FWD_PAGED;
  g_stub.fwd = p;
  g_stub.grid = grid_blocks;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, Dt, int, hipStream_t) {
  g_stub.launches++;
  g_stub.last_kind = StubState::DECODE;
  g_stub.dec = p;
  return hipSuccess;
}

hipError_t launch_decode_cascade(const DecodeParams& p, Dt, int, hipStream_t) {
  g_stub.launches++;
  g_stub.last_kind = StubState::CASCADE;
  g_stub.dec = p;
  return hipSuccess;
}

hipError_t launch_append(const AppendParams& p, int T_new, hipStream_t) {
  g_stub.launches++;
  g_stub.last_kind = StubState::APPEND;
  g_stub.app = p;
  g_stub.grid = T_new;
  return hipSuccess;
}

hipError_t launch_bwd(const BwdParams& p, Dt, int, bool, hipStream_t) {
  g_stub.launches++;
  g_stub.last_kind = StubState::BWD;
  g_stub.bwd = p;
  return hipSuccess;
}

int64_t bwd_grid_blocks(int B, int Nq, int Nk, int Hq, int Hkv) {
  const int64_t a = (int64_t)B * Hq * ((Nq + 127) / 128);
  const int64_t c = (int64_t)B * Hkv * ((Nk + 127) / 128);
  return a > c ? a : c;
}

// a fixed host buffer stands in for the library's device scratch array
hipError_t decode_scratch(void** ptr) {
  alignas(256) static char buf[256];
  g_stub.scratch_lookups++;
  *ptr = buf;
  return hipSuccess;
}

}  // namespace fa

extern "C" {

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  g_stub.copies++;
  if (g_stub.fail_copies) return hipErrorInvalidValue;
  memcpy(dst, src, bytes);
  return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

}  // extern "C"
