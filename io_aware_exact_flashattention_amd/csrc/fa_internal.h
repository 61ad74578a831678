// fa_internal.h - parameter blocks and launchers shared between the C ABI
// (fa_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

// Prefill (dense or ragged). Tokens of every tensor are rows of a packed
// [T, H, d] view; a dense [B, N, H, d] tensor is the ragged case with
// sequence s starting at row s * N. cu_q / cu_k are null for dense calls.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int B;
  int Nq, Nk;        // dense lengths (unused when cu_q != null)
  int Hq, Hkv, group;
  int n_qtiles;      // query tiles of the longest sequence
  float scale_log2;  // scale * log2(e)
  int64_t q_row;     // elements between consecutive tokens of q and o (Hq * d)
  int64_t kv_row;    // elements between consecutive tokens of k and v (Hkv * d)
  // Paged K/V (fa_fwd_paged): k and v are pools of 16-token pages, token t
  // of sequence s lives in row page_table[s][t / 16] * 16 + t % 16; the key
  // length of sequence s is seq_lens[s]. Null for contiguous K/V.
  const int32_t* page_table;
  const int32_t* seq_lens;
  int max_pages;
};

// Most page-table entries one paged prefill sequence may use (staged in LDS).
constexpr int kFwdPagedMaxPages = 8192;

// Split-KV decode over a paged cache.
struct DecodeParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  void* o;
  float* lse;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* o_part;      // [B, Hq, max_splits, d]
  float* lse_part;    // [B, Hq, max_splits]
  int B, max_pages, Hq, Hkv, group;
  int pages_per_split;
  int max_splits;
  float scale_log2;
  // Shared-prefix (cascade) decode: every sequence's keys are the prefix_len
  // tokens on prefix_pages followed by its own seq_lens[b] tokens. The prefix
  // is reduced once for all queries into splits [0, prefix_splits); the
  // split kernel writes its splits from split_offset on. All zero/null for
  // a plain decode.
  const int32_t* prefix_pages;
  int prefix_len;
  int prefix_splits;
  int prefix_pages_per_split;  // pages per prefix split (pages_per_split: suffix splits)
  int split_offset;
};

// Appending new tokens to the paged cache.
constexpr int kPageRows = 16;  // token slots per page
struct AppendParams {
  const void* k_new;             // [T_new, Hkv, d]
  const void* v_new;
  void* k_pool;                  // [num_pages, 16, Hkv, d]
  void* v_pool;
  const int32_t* cu_new;         // [B+1]
  const int32_t* page_table;     // [B, max_pages]
  const int32_t* seq_lens_before;  // [B]
  int B, max_pages, num_pages;
  int64_t row_bytes;             // Hkv * d * element size (a multiple of 16)
};

// Gradients of dense attention (fa_bwd). q, o, dout, dq: [B, Nq, Hq, d];
// k, v, dk, dv: [B, Nk, Hkv, d]; lse, dsum: [B, Nq, Hq] fp32.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  // workspace, both [B, Hq, n_pad] float32 (rows padded to a multiple of 64
  // so that a 64-row tile of one head is one contiguous run):
  float* dsum;       // D = rowsum(dO o O) of every query row
  float* lse2;       // log2-domain lse offset lse * log2(e) (+inf where lse = -inf)
  int n_pad;         // Nq rounded up to a multiple of 64
  int B, Nq, Nk, Hq, Hkv, group;
  int64_t q_row;     // Hq * d
  int64_t kv_row;    // Hkv * d
  float scale;       // scale of the logits
  float scale_log2;  // scale * log2(e)
};

enum class Dt { F32, F16, Bf16 };

// Each launcher enqueues its kernel(s) on `stream` and returns hipGetLastError().
hipError_t launch_fwd(const FwdParams& p, Dt dt, int d, bool causal, int grid_blocks,
                      hipStream_t stream);
int fwd_block_rows(Dt dt);  // query rows per workgroup for this dtype
// Prefill over a paged K/V cache (16-bit types only).
hipError_t launch_fwd_paged(const FwdParams& p, Dt dt, int d, bool causal, int grid_blocks,
                            hipStream_t stream);

hipError_t launch_decode(const DecodeParams& p, Dt dt, int d, hipStream_t stream);
// Cascade decode: prefix pass (when p.prefix_len > 0), suffix pass, merge.
hipError_t launch_decode_cascade(const DecodeParams& p, Dt dt, int d, hipStream_t stream);

hipError_t launch_append(const AppendParams& p, int T_new, hipStream_t stream);

// Backward pass: the dQ kernel (which also writes dsum), then the dK/dV kernel.
hipError_t launch_bwd(const BwdParams& p, Dt dt, int d, bool causal, hipStream_t stream);
// Workgroups of the larger of the two backward launches.
int64_t bwd_grid_blocks(int B, int Nq, int Nk, int Hq, int Hkv);

// Bytes of the fixed device workspace behind fa_decode_paged_noalloc.
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
// Device address of that workspace on the current device (looked up once
// per device, then cached); the memory itself lives until the process ends.
hipError_t decode_scratch(void** ptr);

}  // namespace fa
