// fa_cache.hip - appending new tokens' K/V rows to the paged cache, gfx950.
//
// The paged KV layout of the page "I/O-Aware Kernels" (datasystem.school,
// Module 5), section "FlashInfer: I/O-aware attention for serving": a pool of
// 16-token pages and a page table per sequence. Appending n tokens to a
// sequence that holds L writes token i to position L + i: page
// page_table[s][(L+i) / 16], slot (L+i) % 16. The kernel moves bits only.
//
// One wavefront per new token and tensor: workgroups of four wavefronts
// take four consecutive tokens (grid x), grid y picks the tensor (0 = K,
// 1 = V). A wavefront finds the token's sequence, then copies the token row
// (Hkv * d values, a multiple of 16 bytes) in 16-byte pieces. This is a pure
// HBM copy: 2 x row bytes read and written per token and tensor.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kAppendWaves = 4;

__global__ __launch_bounds__(64 * kAppendWaves) void append_kernel(AppendParams p, int T_new) {
  const int t = blockIdx.x * kAppendWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T_new) return;
  const int lane = threadIdx.x & 63;
  const bool is_v = blockIdx.y != 0;
  // its sequence: cu_new[s] <= t < cu_new[s+1] (cu_new non-decreasing, cu_new[0] = 0,
  // cu_new[B] = T_new > t)
  int lo = 0, hi = p.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.cu_new[mid] <= t) lo = mid;
    else hi = mid;
  }
  const int s = lo;
  const int64_t pos = (int64_t)p.seq_lens_before[s] + (t - p.cu_new[s]);
  // a position outside the sequence's page-table row, or a page outside the
  // pool, is not written
  if (pos < 0 || pos >= (int64_t)p.max_pages * kPageRows) return;
  const int page = p.page_table[(int64_t)s * p.max_pages + (pos / kPageRows)];
  if (page < 0 || page >= p.num_pages) return;
  const int64_t row = (int64_t)page * kPageRows + (pos % kPageRows);
  const char* src = (const char*)(is_v ? p.v_new : p.k_new) + (int64_t)t * p.row_bytes;
  char* dst = (char*)(is_v ? p.v_pool : p.k_pool) + row * p.row_bytes;
  const int chunks = (int)(p.row_bytes / 16);
  for (int c = lane; c < chunks; c += 64) ((uint4*)dst)[c] = ((const uint4*)src)[c];
}

}  // namespace

hipError_t launch_append(const AppendParams& p, int T_new, hipStream_t st) {
  hipLaunchKernelGGL(append_kernel, dim3((T_new + kAppendWaves - 1) / kAppendWaves, 2),
                     dim3(64 * kAppendWaves), 0, st, p, T_new);
  return hipGetLastError();
}

}  // namespace fa
