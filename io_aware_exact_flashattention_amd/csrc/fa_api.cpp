// fa_api.cpp - the C ABI: host-side argument validation, grid sizing and
// dispatch to the gfx950 kernels. Validation happens before any HIP call,
// so an invalid request launches nothing and touches no output.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

constexpr int kPageSize = 16;
// Pages per split of a plain decode without a split count. 43-50 pages gave
// the highest K/V read rate on MI355X for 64 sequences of U[512, 32768]
// tokens (about 3% above 32 pages): fewer partial results and item
// start-ups, while the ~2.8 rounds of work items still let the dispatcher
// balance the ragged lengths.
constexpr int kDecodePagesPerSplit = 48;
// Pages per split of the shared-prefix pass of a cascade decode.
constexpr int kPrefixPagesPerSplit = 32;
constexpr int kMaxPagesPerSplit = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }

// Shared checks of the attention calls. A tensor pointer may be null only
// when that tensor holds no element: q/o/lse when there is no query row
// (q_rows == false), k/v when there is no key (kv_rows == false). A null
// pointer of an empty tensor is never dereferenced.
fa_status check_common(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, int Hq, int Hkv, int d, fa_dtype dt, float scale,
                       bool q_rows = true, bool kv_rows = true) {
  if (q_rows && (!q || !o || !lse)) return FA_ERR_INVALID_ARG;
  if (kv_rows && (!k || !v)) return FA_ERR_INVALID_ARG;
  if (dt != FA_F32 && dt != FA_F16 && dt != FA_BF16) return FA_ERR_INVALID_ARG;
  if (Hq <= 0 || Hkv <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_INVALID_ARG;
  if (!head_dim_ok(d)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

fa::Dt to_dt(fa_dtype t) {
  return t == FA_F32 ? fa::Dt::F32 : t == FA_F16 ? fa::Dt::F16 : fa::Dt::Bf16;
}

constexpr float kLog2e = 1.4426950408889634f;

fa_status run_fwd(fa::FwdParams& p, fa_dtype dt, int d, int causal, int max_q, void* stream) {
  const int bm = fa::fwd_block_rows(to_dt(dt));
  p.n_qtiles = (max_q + bm - 1) / bm;
  const int64_t blocks = (int64_t)p.n_qtiles * p.Hq * p.B;
  if (blocks == 0) return FA_OK;  // nothing to compute
  if (blocks > INT32_MAX) return FA_ERR_UNSUPPORTED;
  hipError_t e = fa::launch_fwd(p, to_dt(dt), d, causal != 0, (int)blocks, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---- opt-in check of the device index arrays --------------------------
// With FA_DEBUG_VALIDATE set to anything but "" or "0" in the environment,
// each call first copies its device index arrays (cu_seqlens, page table,
// lengths) to the host, ordered after the work already queued on its stream,
// waits for the copy, and rejects contents that break the documented
// preconditions with FA_ERR_INVALID_ARG before anything is launched. The
// variable is read at every call. Off by default: the check synchronises the
// stream and costs a device-to-host copy per call.
bool debug_validate() {
  const char* e = getenv("FA_DEBUG_VALIDATE");
  return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
}

// n int32 values of a device array -> host; false when HIP reports an error.
bool fetch(const int32_t* dev, int64_t n, std::vector<int32_t>& host, void* stream) {
  host.assign((size_t)(n > 0 ? n : 0), 0);
  if (n <= 0) return true;
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(host.data(), dev, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
      hipSuccess)
    return false;
  return hipStreamSynchronize(st) == hipSuccess;
}

// cu[0] = 0, non-decreasing, cu[B] = total, and no run longer than max_len
// (max_len < 0: no bound).
bool cu_ok(const std::vector<int32_t>& cu, int B, int64_t total, int64_t max_len) {
  if ((int)cu.size() != B + 1 || cu[0] != 0 || cu[B] != total) return false;
  for (int s = 0; s < B; ++s) {
    const int64_t len = (int64_t)cu[s + 1] - cu[s];
    if (len < 0 || (max_len >= 0 && len > max_len)) return false;
  }
  return true;
}

// 0 <= len[b] <= max_pages * 16 and the entries of the first ceil(len / 16)
// pages of row b of the table lie in [0, num_pages).
bool pages_ok(const std::vector<int32_t>& table, const std::vector<int32_t>& lens, int B,
              int max_pages, int num_pages) {
  for (int b = 0; b < B; ++b) {
    const int64_t len = lens[b];
    if (len < 0 || len > (int64_t)max_pages * kPageSize) return false;
    const int64_t used = (len + kPageSize - 1) / kPageSize;
    for (int64_t i = 0; i < used; ++i) {
      const int32_t pg = table[(size_t)b * max_pages + i];
      if (pg < 0 || pg >= num_pages) return false;
    }
  }
  return true;
}

// Result of a validation: FA_OK, FA_ERR_INVALID_ARG (bad contents) or
// FA_ERR_HIP (the copy failed).
fa_status validate_varlen(const int32_t* cu_q, const int32_t* cu_k, int B, int max_q, int Tq,
                          int Tk, void* stream) {
  std::vector<int32_t> hq, hk;
  if (!fetch(cu_q, B + 1, hq, stream) || !fetch(cu_k, B + 1, hk, stream)) return FA_ERR_HIP;
  return cu_ok(hq, B, Tq, max_q) && cu_ok(hk, B, Tk, -1) ? FA_OK : FA_ERR_INVALID_ARG;
}

fa_status validate_paged(const int32_t* table, const int32_t* lens, int B, int max_pages,
                         int num_pages, void* stream, std::vector<int32_t>* lens_out = nullptr) {
  std::vector<int32_t> ht, hl;
  if (!fetch(table, (int64_t)B * max_pages, ht, stream) || !fetch(lens, B, hl, stream))
    return FA_ERR_HIP;
  if (!pages_ok(ht, hl, B, max_pages, num_pages)) return FA_ERR_INVALID_ARG;
  if (lens_out) *lens_out = hl;
  return FA_OK;
}

fa_status validate_chunks(const int32_t* cu_q, const int32_t* table, const int32_t* lens, int B,
                          int max_q, int Tq, int max_pages, int num_pages, void* stream) {
  std::vector<int32_t> hq, hl;
  if (!fetch(cu_q, B + 1, hq, stream)) return FA_ERR_HIP;
  if (!cu_ok(hq, B, Tq, max_q)) return FA_ERR_INVALID_ARG;
  const fa_status st = validate_paged(table, lens, B, max_pages, num_pages, stream, &hl);
  if (st != FA_OK) return st;
  for (int s = 0; s < B; ++s)  // a chunk's queries are the last tokens of its sequence
    if (hq[s + 1] - hq[s] > hl[s]) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

fa_status validate_prefix(const int32_t* prefix_pages, int prefix_len, int num_pages,
                          void* stream) {
  std::vector<int32_t> hp;
  if (!fetch(prefix_pages, (prefix_len + kPageSize - 1) / kPageSize, hp, stream)) return FA_ERR_HIP;
  for (int32_t pg : hp)
    if (pg < 0 || pg >= num_pages) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

fa_status validate_append(const int32_t* cu_new, int B, int T_new, void* stream) {
  std::vector<int32_t> hc;
  if (!fetch(cu_new, B + 1, hc, stream)) return FA_ERR_HIP;
  return cu_ok(hc, B, T_new, -1) ? FA_OK : FA_ERR_INVALID_ARG;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported configuration";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error at launch";
    case FA_ERR_NO_SPACE:
      return "FA_ERR_NO_SPACE: the request needs more than the fixed scratch buffer";
  }
  return "unknown fa_status";
}

int fa_version(void) { return 100; }

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Nq,
                 int Nk, int Hq, int Hkv, int d, fa_dtype dtype, float scale, int causal,
                 void* stream) {
  fa_status st = check_common(q, k, v, o, lse, Hq, Hkv, d, dtype, scale);
  if (st != FA_OK) return st;
  if (B <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_INVALID_ARG;
  if ((int64_t)B * Nq > INT32_MAX || (int64_t)B * Nk > INT32_MAX) return FA_ERR_UNSUPPORTED;
  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.cu_q = nullptr; p.cu_k = nullptr;
  p.B = B; p.Nq = Nq; p.Nk = Nk;
  p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.scale_log2 = scale * kLog2e;
  p.q_row = (int64_t)Hq * d;
  p.kv_row = (int64_t)Hkv * d;
  return run_fwd(p, dtype, d, causal, Nq, stream);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                        int max_seqlen_q, int max_seqlen_k, int Tq, int Tk, int Hq, int Hkv,
                        int d, fa_dtype dtype, float scale, int causal, void* stream) {
  fa_status st = check_common(q, k, v, o, lse, Hq, Hkv, d, dtype, scale, Tq > 0, Tk > 0);
  if (st != FA_OK) return st;
  if (!cu_seqlens_q || !cu_seqlens_k) return FA_ERR_INVALID_ARG;
  if (B <= 0 || Tq < 0 || Tk < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return FA_ERR_INVALID_ARG;
  if (max_seqlen_q > Tq) return FA_ERR_INVALID_ARG;
  if (Tq == 0 || max_seqlen_q == 0) return FA_OK;  // no query rows
  if (debug_validate()) {
    st = validate_varlen(cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, Tq, Tk, stream);
    if (st != FA_OK) return st;
  }
  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
  p.B = B; p.Nq = 0; p.Nk = 0;
  p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.scale_log2 = scale * kLog2e;
  p.q_row = (int64_t)Hq * d;
  p.kv_row = (int64_t)Hkv * d;
  return run_fwd(p, dtype, d, causal, max_seqlen_q, stream);
}

fa_status fa_fwd_paged(const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                       const int32_t* cu_seqlens_q, const int32_t* page_table,
                       const int32_t* seq_lens, int B, int max_seqlen_q, int Tq, int max_pages,
                       int num_pages, int page_size, int Hq, int Hkv, int d, fa_dtype dtype,
                       float scale, int causal, void* stream) {
  fa_status st = check_common(q, k_pool, v_pool, o, lse, Hq, Hkv, d, dtype, scale, Tq > 0);
  if (st != FA_OK) return st;
  if (!cu_seqlens_q || !page_table || !seq_lens) return FA_ERR_INVALID_ARG;
  if (B <= 0 || Tq < 0 || max_seqlen_q < 0 || max_seqlen_q > Tq) return FA_ERR_INVALID_ARG;
  if (max_pages <= 0 || num_pages <= 0 || page_size <= 0) return FA_ERR_INVALID_ARG;
  if (page_size != kPageSize) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (max_pages > fa::kFwdPagedMaxPages) return FA_ERR_UNSUPPORTED;
  if ((int64_t)num_pages * kPageSize > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (Tq == 0 || max_seqlen_q == 0) return FA_OK;  // no query rows
  if (debug_validate()) {
    st = validate_chunks(cu_seqlens_q, page_table, seq_lens, B, max_seqlen_q, Tq, max_pages,
                         num_pages, stream);
    if (st != FA_OK) return st;
  }
  fa::FwdParams p{};
  p.q = q; p.k = k_pool; p.v = v_pool; p.o = o; p.lse = lse;
  p.cu_q = cu_seqlens_q; p.cu_k = nullptr;
  p.page_table = page_table; p.seq_lens = seq_lens; p.max_pages = max_pages;
  p.B = B; p.Nq = 0; p.Nk = 0;
  p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.scale_log2 = scale * kLog2e;
  p.q_row = (int64_t)Hq * d;
  p.kv_row = (int64_t)Hkv * d;
  const int bm = fa::fwd_block_rows(to_dt(dtype));
  p.n_qtiles = (max_seqlen_q + bm - 1) / bm;
  const int64_t blocks = (int64_t)p.n_qtiles * p.Hq * p.B;
  if (blocks > INT32_MAX) return FA_ERR_UNSUPPORTED;
  hipError_t e = fa::launch_fwd_paged(p, to_dt(dtype), d, causal != 0, (int)blocks,
                                      (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Pages per split: kDecodePagesPerSplit when automatic; otherwise the
// longest sequence is cut into num_splits ranges, but a range never exceeds
// kMaxPagesPerSplit pages (the decode kernel holds one split's page indices
// in the lanes of a wave).
static int pages_per_split(int max_pages, int num_splits) {
  if (num_splits <= 0) return kDecodePagesPerSplit;
  const int pps = (max_pages + num_splits - 1) / num_splits;
  return pps < kMaxPagesPerSplit ? pps : kMaxPagesPerSplit;
}

size_t fa_decode_paged_workspace_size(int B, int Hq, int d, int max_pages, int page_size,
                                      int num_splits) {
  if (B <= 0 || Hq <= 0 || d <= 0 || max_pages <= 0 || page_size <= 0 || num_splits < 0)
    return 0;
  if (num_splits > max_pages) return 0;
  const int pps = pages_per_split(max_pages, num_splits);
  const int64_t splits = (max_pages + pps - 1) / pps;
  return (size_t)B * Hq * splits * ((size_t)d + 1) * sizeof(float);
}

// Checks shared by fa_decode_paged and fa_decode_paged_noalloc (everything
// but the workspace); on success `need` is the workspace size in bytes.
static fa_status check_decode(const void* q, const void* k_pool, const void* v_pool, const void* o,
                              const float* lse, const int32_t* page_table,
                              const int32_t* seq_lens, int B, int max_pages, int num_pages,
                              int page_size, int Hq, int Hkv, int d, fa_dtype dtype, float scale,
                              int num_splits, size_t& need) {
  fa_status st = check_common(q, k_pool, v_pool, o, lse, Hq, Hkv, d, dtype, scale);
  if (st != FA_OK) return st;
  if (!page_table || !seq_lens) return FA_ERR_INVALID_ARG;
  if (B <= 0 || max_pages <= 0 || num_pages <= 0 || page_size <= 0) return FA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > max_pages) return FA_ERR_INVALID_ARG;
  if (page_size != kPageSize) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  need = fa_decode_paged_workspace_size(B, Hq, d, max_pages, page_size, num_splits);
  if (need == 0) return FA_ERR_INVALID_ARG;
  const int pps = pages_per_split(max_pages, num_splits);
  const int splits = (max_pages + pps - 1) / pps;
  if (B > 65535) return FA_ERR_UNSUPPORTED;  // grid y of the split merge
  if ((int64_t)B * splits * Hq > INT32_MAX) return FA_ERR_UNSUPPORTED;  // work items
  return FA_OK;
}

// Launches a checked decode with its partials in `workspace`.
static fa_status run_decode(const void* q, const void* k_pool, const void* v_pool, void* o,
                            float* lse, const int32_t* page_table, const int32_t* seq_lens, int B,
                            int max_pages, int num_pages, int Hq, int Hkv, int d, fa_dtype dtype,
                            float scale, int num_splits, void* workspace, void* stream) {
  if (debug_validate()) {
    const fa_status st = validate_paged(page_table, seq_lens, B, max_pages, num_pages, stream);
    if (st != FA_OK) return st;
  }
  const int pps = pages_per_split(max_pages, num_splits);
  const int splits = (max_pages + pps - 1) / pps;
  fa::DecodeParams p{};
  p.q = q; p.k_pool = k_pool; p.v_pool = v_pool; p.o = o; p.lse = lse;
  p.page_table = page_table; p.seq_lens = seq_lens;
  p.B = B; p.max_pages = max_pages; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.pages_per_split = pps;
  p.max_splits = splits;
  p.scale_log2 = scale * kLog2e;
  float* ws = static_cast<float*>(workspace);
  p.o_part = ws;
  p.lse_part = ws + (size_t)B * Hq * splits * d;
  hipError_t e = fa::launch_decode(p, to_dt(dtype), d, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_decode_paged(const void* q, const void* k_pool, const void* v_pool, void* o,
                          float* lse, const int32_t* page_table, const int32_t* seq_lens, int B,
                          int max_pages, int num_pages, int page_size, int Hq, int Hkv, int d,
                          fa_dtype dtype, float scale, int num_splits, void* workspace,
                          size_t workspace_bytes, void* stream) {
  size_t need = 0;
  fa_status st = check_decode(q, k_pool, v_pool, o, lse, page_table, seq_lens, B, max_pages,
                              num_pages, page_size, Hq, Hkv, d, dtype, scale, num_splits, need);
  if (st != FA_OK) return st;
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return FA_ERR_INVALID_ARG;
  return run_decode(q, k_pool, v_pool, o, lse, page_table, seq_lens, B, max_pages, num_pages, Hq,
                    Hkv, d, dtype, scale, num_splits, workspace, stream);
}

fa_status fa_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool, void* o,
                                  float* lse, const int32_t* page_table, const int32_t* seq_lens,
                                  int B, int max_pages, int num_pages, int page_size, int Hq,
                                  int Hkv, int d, fa_dtype dtype, float scale, int num_splits,
                                  void* stream) {
  size_t need = 0;
  fa_status st = check_decode(q, k_pool, v_pool, o, lse, page_table, seq_lens, B, max_pages,
                              num_pages, page_size, Hq, Hkv, d, dtype, scale, num_splits, need);
  if (st != FA_OK) return st;
  static_assert(fa::kDecodeScratchBytes == FA_DECODE_NOALLOC_MAX_WORKSPACE, "scratch size");
  if (need > fa::kDecodeScratchBytes) return FA_ERR_NO_SPACE;
  void* scratch = nullptr;
  if (fa::decode_scratch(&scratch) != hipSuccess) return FA_ERR_HIP;
  return run_decode(q, k_pool, v_pool, o, lse, page_table, seq_lens, B, max_pages, num_pages, Hq,
                    Hkv, d, dtype, scale, num_splits, scratch, stream);
}

// Splits of a cascade decode: prefix splits (32 pages each) lead, then the
// suffix splits of the longest suffix (8 pages each: suffixes are short, so
// shorter splits give the suffix pass enough independent work items).
constexpr int kCascadeSuffixPagesPerSplit = 8;
static void cascade_splits(int prefix_len, int max_pages, int& s_pre, int& s_suf) {
  const int pre_pages = (prefix_len + kPageSize - 1) / kPageSize;
  s_pre = (pre_pages + kPrefixPagesPerSplit - 1) / kPrefixPagesPerSplit;
  s_suf = (max_pages + kCascadeSuffixPagesPerSplit - 1) / kCascadeSuffixPagesPerSplit;
}

size_t fa_decode_cascade_workspace_size(int B, int Hq, int d, int prefix_len, int max_pages,
                                        int page_size) {
  if (B <= 0 || Hq <= 0 || d <= 0 || prefix_len < 0 || max_pages <= 0 || page_size <= 0) return 0;
  int s_pre, s_suf;
  cascade_splits(prefix_len, max_pages, s_pre, s_suf);
  return (size_t)B * Hq * (size_t)(s_pre + s_suf) * ((size_t)d + 1) * sizeof(float);
}

fa_status fa_decode_cascade(const void* q, const void* k_pool, const void* v_pool, void* o,
                            float* lse, const int32_t* prefix_pages, int prefix_len,
                            const int32_t* page_table, const int32_t* seq_lens, int B,
                            int max_pages, int num_pages, int page_size, int Hq, int Hkv, int d,
                            fa_dtype dtype, float scale, void* workspace, size_t workspace_bytes,
                            void* stream) {
  fa_status st = check_common(q, k_pool, v_pool, o, lse, Hq, Hkv, d, dtype, scale);
  if (st != FA_OK) return st;
  if (!page_table || !seq_lens || !workspace) return FA_ERR_INVALID_ARG;
  if (prefix_len < 0 || (prefix_len > 0 && !prefix_pages)) return FA_ERR_INVALID_ARG;
  if (B <= 0 || max_pages <= 0 || num_pages <= 0 || page_size <= 0) return FA_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return FA_ERR_INVALID_ARG;
  if (page_size != kPageSize) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  const size_t need = fa_decode_cascade_workspace_size(B, Hq, d, prefix_len, max_pages, page_size);
  if (need == 0 || workspace_bytes < need) return FA_ERR_INVALID_ARG;
  int s_pre, s_suf;
  cascade_splits(prefix_len, max_pages, s_pre, s_suf);
  if (B > 65535) return FA_ERR_UNSUPPORTED;  // grid y of the split merge
  if ((int64_t)B * (s_pre + s_suf) * Hq > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (debug_validate()) {
    st = validate_prefix(prefix_pages, prefix_len, num_pages, stream);
    if (st == FA_OK) st = validate_paged(page_table, seq_lens, B, max_pages, num_pages, stream);
    if (st != FA_OK) return st;
  }

  fa::DecodeParams p{};
  p.q = q; p.k_pool = k_pool; p.v_pool = v_pool; p.o = o; p.lse = lse;
  p.page_table = page_table; p.seq_lens = seq_lens;
  p.B = B; p.max_pages = max_pages; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.pages_per_split = kCascadeSuffixPagesPerSplit;
  p.prefix_pages_per_split = kPrefixPagesPerSplit;
  p.max_splits = s_pre + s_suf;
  p.scale_log2 = scale * kLog2e;
  p.prefix_pages = prefix_pages;
  p.prefix_len = prefix_len;
  p.prefix_splits = s_pre;
  p.split_offset = s_pre;
  float* ws = static_cast<float*>(workspace);
  p.o_part = ws;
  p.lse_part = ws + (size_t)B * Hq * p.max_splits * d;
  hipError_t e = fa::launch_decode_cascade(p, to_dt(dtype), d, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int Nq, int Hq) {
  if (B <= 0 || Nq <= 0 || Hq <= 0) return 0;
  const size_t n_pad = ((size_t)Nq + 63) / 64 * 64;
  return 2 * (size_t)B * Hq * n_pad * sizeof(float);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq,
                 int Hkv, int d, fa_dtype dtype, float scale, int causal, void* workspace,
                 size_t workspace_bytes, void* stream) {
  fa_status st = check_common(q, k, v, o, lse, Hq, Hkv, d, dtype, scale);
  if (st != FA_OK) return st;
  if (!dout || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID_ARG;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(workspace))
    return FA_ERR_INVALID_ARG;
  if (B <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_INVALID_ARG;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if ((int64_t)B * Nq > INT32_MAX || (int64_t)B * Nk > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa_bwd_workspace_size(B, Nq, Hq)) return FA_ERR_INVALID_ARG;
  if (fa::bwd_grid_blocks(B, Nq, Nk, Hq, Hkv) > INT32_MAX) return FA_ERR_UNSUPPORTED;
  fa::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.n_pad = (Nq + 63) / 64 * 64;
  p.dsum = static_cast<float*>(workspace);
  p.lse2 = p.dsum + (size_t)B * Hq * p.n_pad;
  p.B = B; p.Nq = Nq; p.Nk = Nk; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
  p.q_row = (int64_t)Hq * d;
  p.kv_row = (int64_t)Hkv * d;
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  hipError_t e = fa::launch_bwd(p, to_dt(dtype), d, causal != 0, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                       const int32_t* cu_new, const int32_t* page_table,
                       const int32_t* seq_lens_before, int B, int T_new, int max_pages,
                       int num_pages, int page_size, int Hkv, int d, fa_dtype dtype, void* stream) {
  // k_new / v_new hold T_new rows and may be null when T_new == 0
  if ((T_new > 0 && (!k_new || !v_new)) || !k_pool || !v_pool || !cu_new || !page_table ||
      !seq_lens_before)
    return FA_ERR_INVALID_ARG;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (B <= 0 || T_new < 0 || max_pages <= 0 || num_pages <= 0 || page_size <= 0 || Hkv <= 0 ||
      d <= 0)
    return FA_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return FA_ERR_INVALID_ARG;
  if (page_size != kPageSize) return FA_ERR_UNSUPPORTED;
  if (!head_dim_ok(d)) return FA_ERR_UNSUPPORTED;
  if (T_new == 0) return FA_OK;
  if (debug_validate()) {
    const fa_status st = validate_append(cu_new, B, T_new, stream);
    if (st != FA_OK) return st;
  }
  fa::AppendParams p{};
  p.k_new = k_new; p.v_new = v_new; p.k_pool = k_pool; p.v_pool = v_pool;
  p.cu_new = cu_new; p.page_table = page_table; p.seq_lens_before = seq_lens_before;
  p.B = B; p.max_pages = max_pages; p.num_pages = num_pages;
  p.row_bytes = (int64_t)Hkv * d * (dtype == FA_F32 ? 4 : 2);
  hipError_t e = fa::launch_append(p, T_new, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
