// abi_host_check.cpp - host-side checks of the C ABI (include/fa.h), built
// with g++ together with fa_api.cpp and the launcher stubs of hip_stub.cpp,
// under AddressSanitizer and UndefinedBehaviorSanitizer. No GPU: the stubs
// record launches instead of running kernels, and the device index arrays
// are host arrays that the stubbed hipMemcpyAsync copies.
//
// Covers: argument rejection before any launch, the parameter blocks the
// valid calls hand to the launchers (grid sizes, split layout, workspace
// carve-up), NULL pointers of empty tensors, and the opt-in
// FA_DEBUG_VALIDATE check of cu_seqlens / page tables / lengths.
// Prints "abi_host_check: N checks passed" and exits 0, or names the first
// failed check and exits 1. Test infrastructure only.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "fa.h"
#include "stub_state.h"

static int g_checks = 0;

#define CHECK(cond)                                                          \
  do {                                                                       \
    ++g_checks;                                                              \
    if (!(cond)) {                                                           \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      exit(1);                                                               \
    }                                                                        \
  } while (0)

// A 16-byte aligned stand-in for device buffers that are never dereferenced.
alignas(16) static char g_buf[64];
static void* const P = g_buf;

static fa_status fwd(int B, int Nq, int Nk, int Hq, int Hkv, int d, fa_dtype dt, float scale) {
  return fa_fwd(P, P, P, P, (float*)P, B, Nq, Nk, Hq, Hkv, d, dt, scale, 1, nullptr);
}

static void check_fwd() {
  const int before = g_stub.launches;
  CHECK(fa_fwd(nullptr, P, P, P, (float*)P, 1, 8, 8, 2, 1, 64, FA_BF16, 0.125f, 0, nullptr) ==
        FA_ERR_INVALID_ARG);
  CHECK(fwd(0, 8, 8, 2, 1, 64, FA_BF16, 0.125f) == FA_ERR_INVALID_ARG);
  CHECK(fwd(1, 8, 8, 3, 2, 64, FA_BF16, 0.125f) == FA_ERR_INVALID_ARG);
  CHECK(fwd(1, 8, 8, 2, 1, 96, FA_BF16, 0.125f) == FA_ERR_UNSUPPORTED);
  CHECK(fwd(1, 8, 8, 2, 1, 64, FA_BF16, -1.f) == FA_ERR_INVALID_ARG);
  CHECK(fwd(1, 8, 8, 2, 1, 64, (fa_dtype)9, 0.1f) == FA_ERR_INVALID_ARG);
  // B * N beyond int32 rows
  CHECK(fwd(65536, 65536, 8, 2, 1, 64, FA_BF16, 0.125f) == FA_ERR_UNSUPPORTED);
  CHECK(g_stub.launches == before);
  // cfg2-shaped call: 64 query tiles x 32 heads
  CHECK(fwd(1, 16384, 16384, 32, 32, 128, FA_BF16, 0.0883883f) == FA_OK);
  CHECK(g_stub.last_kind == StubState::FWD && g_stub.grid == 64 * 32);
  CHECK(g_stub.fwd.n_qtiles == 64 && g_stub.fwd.q_row == 32 * 128 && g_stub.fwd.group == 1);
  // fp32 takes 32-row tiles
  CHECK(fwd(2, 100, 100, 4, 2, 64, FA_F32, 0.125f) == FA_OK);
  CHECK(g_stub.grid == 4 * 4 * 2 && g_stub.fwd.group == 2 && g_stub.fwd.kv_row == 2 * 64);
}

static void check_varlen() {
  int32_t cu[3] = {0, 5, 9};
  const int before = g_stub.launches;
  // no query rows: q, o, lse may be NULL, nothing is launched
  CHECK(fa_fwd_varlen(nullptr, P, P, nullptr, nullptr, cu, cu, 2, 0, 4, 0, 9, 2, 2, 64, FA_BF16,
                      0.1f, 1, nullptr) == FA_OK);
  CHECK(g_stub.launches == before);
  // no key rows: k, v may be NULL, the kernel still writes O = 0, LSE = -inf
  int32_t ck[3] = {0, 0, 0};
  CHECK(fa_fwd_varlen(P, nullptr, nullptr, P, (float*)P, cu, ck, 2, 5, 0, 9, 0, 2, 2, 64, FA_BF16,
                      0.1f, 1, nullptr) == FA_OK);
  CHECK(g_stub.launches == before + 1 && g_stub.last_kind == StubState::FWD);
  // but not when there are keys
  CHECK(fa_fwd_varlen(P, nullptr, P, P, (float*)P, cu, cu, 2, 5, 5, 9, 9, 2, 2, 64, FA_BF16, 0.1f,
                      1, nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_fwd_varlen(nullptr, P, P, P, (float*)P, cu, cu, 2, 5, 5, 9, 9, 2, 2, 64, FA_BF16, 0.1f,
                      1, nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_fwd_varlen(P, P, P, P, (float*)P, cu, cu, 2, 10, 5, 9, 9, 2, 2, 64, FA_BF16, 0.1f, 1,
                      nullptr) == FA_ERR_INVALID_ARG);  // max_seqlen_q > Tq
}

static void check_decode() {
  const int before = g_stub.launches;
  const size_t need = fa_decode_paged_workspace_size(64, 32, 128, 2017, 16, 0);
  CHECK(need == (size_t)64 * 32 * 43 * 129 * 4);
  CHECK(fa_decode_paged_workspace_size(0, 32, 128, 2017, 16, 0) == 0);
  CHECK(fa_decode_paged_workspace_size(64, 32, 128, 2017, 16, 2018) == 0);
  CHECK(fa_decode_paged(P, P, P, P, (float*)P, (int32_t*)P, (int32_t*)P, 64, 2017, 75219, 16, 32, 8,
                        128, FA_BF16, 0.1f, 0, P, need - 1, nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_decode_paged(P, P, P, P, (float*)P, (int32_t*)P, (int32_t*)P, 64, 2017, 75219, 8, 32, 8,
                        128, FA_BF16, 0.1f, 0, P, need, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_decode_paged(P, P, P, P, (float*)P, (int32_t*)P, (int32_t*)P, 64, 2017, 75219, 16, 32, 8,
                        128, FA_F32, 0.1f, 0, P, need, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(g_stub.launches == before);
  CHECK(fa_decode_paged(P, P, P, P, (float*)P, (int32_t*)P, (int32_t*)P, 64, 2017, 75219, 16, 32, 8,
                        128, FA_BF16, 0.1f, 0, P, need, nullptr) == FA_OK);
  CHECK(g_stub.last_kind == StubState::DECODE && g_stub.dec.pages_per_split == 48 &&
        g_stub.dec.max_splits == 43 && g_stub.dec.group == 4);
  // the workspace holds O partials [B, Hq, S, d], then LSE partials [B, Hq, S]
  CHECK((char*)g_stub.dec.lse_part - (char*)g_stub.dec.o_part == (ptrdiff_t)64 * 32 * 43 * 128 * 4);
  // explicit split count: ceil(2017 / 7) = 289 pages would exceed 64, so 64
  const size_t need7 = fa_decode_paged_workspace_size(64, 32, 128, 2017, 16, 7);
  CHECK(fa_decode_paged(P, P, P, P, (float*)P, (int32_t*)P, (int32_t*)P, 64, 2017, 75219, 16, 32, 8,
                        128, FA_BF16, 0.1f, 7, P, need7, nullptr) == FA_OK);
  CHECK(g_stub.dec.pages_per_split == 64 && g_stub.dec.max_splits == 32);

  // the allocation-free variant: the same launch, partials in the library's buffer
  const int lookups = g_stub.scratch_lookups;
  CHECK(fa_decode_paged_noalloc(P, P, P, P, (float*)P, (int32_t*)P, (int32_t*)P, 64, 2017, 75219,
                                16, 32, 8, 128, FA_BF16, 0.1f, 0, nullptr) == FA_OK);
  CHECK(g_stub.last_kind == StubState::DECODE && g_stub.dec.pages_per_split == 48 &&
        g_stub.dec.max_splits == 43 && g_stub.scratch_lookups == lookups + 1);
  CHECK((char*)g_stub.dec.lse_part - (char*)g_stub.dec.o_part == (ptrdiff_t)64 * 32 * 43 * 128 * 4);
  // a request beyond the fixed buffer: FA_ERR_NO_SPACE, nothing launched or looked up
  const size_t big = fa_decode_paged_workspace_size(128, 64, 128, 2017, 16, 0);
  CHECK(big > FA_DECODE_NOALLOC_MAX_WORKSPACE);
  const int n = g_stub.launches;
  CHECK(fa_decode_paged_noalloc(P, P, P, P, (float*)P, (int32_t*)P, (int32_t*)P, 128, 2017, 75219,
                                16, 64, 8, 128, FA_BF16, 0.1f, 0, nullptr) == FA_ERR_NO_SPACE);
  CHECK(fa_decode_paged_noalloc(P, P, P, P, (float*)P, (int32_t*)P, (int32_t*)P, 64, 2017, 75219,
                                8, 32, 8, 128, FA_BF16, 0.1f, 0, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(g_stub.launches == n && g_stub.scratch_lookups == lookups + 1);
}

static void check_append() {
  int32_t cu[3] = {0, 0, 0};
  const int before = g_stub.launches;
  // no new rows: k_new / v_new may be NULL
  CHECK(fa_kv_append(nullptr, nullptr, P, P, cu, (int32_t*)P, (int32_t*)P, 2, 0, 4, 8, 16, 2, 128,
                     FA_BF16, nullptr) == FA_OK);
  CHECK(fa_kv_append(nullptr, P, P, P, cu, (int32_t*)P, (int32_t*)P, 2, 3, 4, 8, 16, 2, 128,
                     FA_BF16, nullptr) == FA_ERR_INVALID_ARG);
  CHECK(g_stub.launches == before);
  CHECK(fa_kv_append(P, P, P, P, cu, (int32_t*)P, (int32_t*)P, 2, 3, 4, 8, 16, 2, 128, FA_F32,
                     nullptr) == FA_OK);
  CHECK(g_stub.last_kind == StubState::APPEND && g_stub.app.row_bytes == 2 * 128 * 4 &&
        g_stub.grid == 3);
}

static void check_bwd() {
  const size_t ws = fa_bwd_workspace_size(1, 16384, 32);
  CHECK(ws == (size_t)2 * 16384 * 32 * 4);  // D and the LSE offsets, rows padded to 64
  CHECK(fa_bwd_workspace_size(2, 100, 3) == (size_t)2 * 2 * 3 * 128 * 4);
  auto call = [&](void* dq, size_t bytes, fa_dtype dt) {
    return fa_bwd(P, P, P, P, (float*)P, P, dq, P, P, 1, 16384, 16384, 32, 8, 128, dt, 0.088f, 1,
                  P, bytes, nullptr);
  };
  const int before = g_stub.launches;
  CHECK(call(nullptr, ws, FA_BF16) == FA_ERR_INVALID_ARG);
  CHECK(call(P, ws - 4, FA_BF16) == FA_ERR_INVALID_ARG);
  CHECK(call(P, ws, FA_F32) == FA_ERR_UNSUPPORTED);
  CHECK(g_stub.launches == before);
  CHECK(call(P, ws, FA_BF16) == FA_OK);
  CHECK(g_stub.last_kind == StubState::BWD && g_stub.bwd.group == 4 &&
        g_stub.bwd.q_row == 32 * 128 && g_stub.bwd.kv_row == 8 * 128 && g_stub.bwd.dsum == P);
  CHECK(g_stub.bwd.n_pad == 16384 && g_stub.bwd.lse2 == (float*)P + (size_t)32 * 16384);
}

// ---- FA_DEBUG_VALIDATE: the stubbed copy reads these host arrays --------
static void check_validate() {
  setenv("FA_DEBUG_VALIDATE", "1", 1);
  const int before = g_stub.launches;
  auto varlen = [](const int32_t* cq, const int32_t* ck, int B, int mq, int Tq, int Tk) {
    return fa_fwd_varlen(P, P, P, P, (float*)P, cq, ck, B, mq, 0, Tq, Tk, 4, 2, 128, FA_BF16, 0.1f,
                         1, nullptr);
  };
  const int32_t good[4] = {0, 3, 3, 10};
  CHECK(varlen(good, good, 3, 7, 10, 10) == FA_OK);
  CHECK(g_stub.launches == before + 1);
  const int32_t not_zero[4] = {1, 3, 3, 10};
  const int32_t decreasing[4] = {0, 5, 4, 10};
  const int32_t wrong_total[4] = {0, 3, 3, 9};
  CHECK(varlen(not_zero, good, 3, 7, 10, 10) == FA_ERR_INVALID_ARG);
  CHECK(varlen(decreasing, good, 3, 7, 10, 10) == FA_ERR_INVALID_ARG);
  CHECK(varlen(good, decreasing, 3, 7, 10, 10) == FA_ERR_INVALID_ARG);
  CHECK(varlen(wrong_total, good, 3, 7, 10, 10) == FA_ERR_INVALID_ARG);
  CHECK(varlen(good, good, 3, 6, 10, 10) == FA_ERR_INVALID_ARG);  // a run of 7 > max_seqlen_q
  CHECK(g_stub.launches == before + 1);

  // paged decode: B = 2, max_pages = 3, num_pages = 5
  auto decode = [](const int32_t* pt, const int32_t* sl) {
    static alignas(16) char ws[1 << 16];
    return fa_decode_paged(P, P, P, P, (float*)P, pt, sl, 2, 3, 5, 16, 4, 1, 64, FA_F16, 0.1f, 0,
                           ws, sizeof(ws), nullptr);
  };
  const int32_t pt[6] = {4, 0, -1, 2, -1, -1};
  const int32_t sl_ok[2] = {17, 16};        // pages 0,1 of row 0; page 0 of row 1
  const int32_t sl_long[2] = {49, 0};       // beyond 3 pages
  const int32_t sl_neg[2] = {1, -1};
  const int32_t sl_unmapped[2] = {33, 0};   // needs entry 2 of row 0 (-1)
  const int32_t pt_oob[6] = {5, 0, -1, 2, -1, -1};
  CHECK(decode(pt, sl_ok) == FA_OK);
  CHECK(decode(pt, sl_long) == FA_ERR_INVALID_ARG);
  CHECK(decode(pt, sl_neg) == FA_ERR_INVALID_ARG);
  CHECK(decode(pt, sl_unmapped) == FA_ERR_INVALID_ARG);
  CHECK(decode(pt_oob, sl_ok) == FA_ERR_INVALID_ARG);
  CHECK(g_stub.launches == before + 2);

  // chunked prefill: a chunk longer than its sequence is rejected
  auto chunks = [&](const int32_t* cq, const int32_t* sl, int Tq, int mq) {
    return fa_fwd_paged(P, P, P, P, (float*)P, cq, pt, sl, 2, mq, Tq, 3, 5, 16, 4, 2, 128, FA_BF16,
                        0.1f, 1, nullptr);
  };
  const int32_t cq_ok[3] = {0, 17, 20};
  const int32_t cq_long[3] = {0, 18, 20};
  CHECK(chunks(cq_ok, sl_ok, 20, 17) == FA_OK);
  CHECK(chunks(cq_long, sl_ok, 20, 18) == FA_ERR_INVALID_ARG);
  CHECK(chunks(cq_ok, sl_unmapped, 20, 17) == FA_ERR_INVALID_ARG);

  // cascade: prefix pages in the pool
  auto cascade = [&](const int32_t* pp, int plen) {
    static alignas(16) char ws[1 << 16];
    return fa_decode_cascade(P, P, P, P, (float*)P, pp, plen, pt, sl_ok, 2, 3, 5, 16, 4, 1, 64,
                             FA_BF16, 0.1f, ws, sizeof(ws), nullptr);
  };
  const int32_t pre_ok[2] = {1, 3};
  const int32_t pre_bad[2] = {1, 7};
  CHECK(cascade(pre_ok, 20) == FA_OK);
  CHECK(cascade(pre_bad, 20) == FA_ERR_INVALID_ARG);
  CHECK(cascade(pre_bad, 16) == FA_OK);  // only the first page is used

  // append: cu_new must describe T_new rows
  const int32_t cn_ok[3] = {0, 2, 3};
  const int32_t cn_bad[3] = {0, 4, 3};
  CHECK(fa_kv_append(P, P, P, P, cn_ok, pt, sl_ok, 2, 3, 3, 5, 16, 1, 64, FA_BF16, nullptr) == FA_OK);
  CHECK(fa_kv_append(P, P, P, P, cn_bad, pt, sl_ok, 2, 3, 3, 5, 16, 1, 64, FA_BF16, nullptr) ==
        FA_ERR_INVALID_ARG);

  // a failing copy is a HIP error, and nothing is launched
  const int launched = g_stub.launches;
  g_stub.fail_copies = true;
  CHECK(varlen(good, good, 3, 7, 10, 10) == FA_ERR_HIP);
  g_stub.fail_copies = false;
  CHECK(g_stub.launches == launched);

  // "0" turns the check off: bad contents pass through to the launch
  setenv("FA_DEBUG_VALIDATE", "0", 1);
  const int copies = g_stub.copies;
  CHECK(varlen(decreasing, good, 3, 7, 10, 10) == FA_OK);
  CHECK(g_stub.copies == copies && g_stub.launches == launched + 1);
  unsetenv("FA_DEBUG_VALIDATE");
}

int main() {
  CHECK(fa_version() >= 100);
  CHECK(fa_status_string((fa_status)42) != nullptr);
  CHECK(fa_status_string(FA_ERR_NO_SPACE)[0] == 'F');
  check_fwd();
  check_varlen();
  check_decode();
  check_append();
  check_bwd();
  check_validate();
  printf("abi_host_check: %d checks passed\n", g_checks);
  return 0;
}
