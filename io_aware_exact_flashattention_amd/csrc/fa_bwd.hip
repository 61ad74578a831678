// fa_bwd.hip - gradients of exact attention (the backward pass), gfx950.
//
// The forward definition of the page "I/O-Aware Kernels" (datasystem.school,
// Module 5), section "Naive attention: materializing the k x k score
// matrix" is S = scale Q K^T, P = row softmax of S, O = P V. Its gradients
// for an output gradient dO follow by the chain rule:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D) with D_i = sum_j P_ij dP_ij,
//   dQ = scale dS K,  dK = scale dS^T Q.
// As in the fused forward pass of section "FlashAttention: tiling + online
// softmax", nothing of size Nq x Nk touches device memory: P is recomputed
// tile by tile from the log-sum-exp the forward pass saved,
// P_ij = exp(scale q_i.k_j - lse_i), and D_i is taken as rowsum(dO_i o O_i),
// which equals sum_j P_ij dP_ij because O_i = sum_j P_ij v_j.
//
// Two kernels, both deterministic (no atomics, fixed summation order):
//  * bwd_dq_kernel: a workgroup owns 128 query rows of one head (4 waves x
//    32 rows) and streams the K/V tiles of the rows' key range through LDS.
//    Per 32-key block it forms S^T = K Q^T and dP^T = V dO^T with the query
//    vectors as MFMA B operands held in registers (a lane owns one query
//    row), then dS^T, then dQ^T += K^T dS^T with K^T read transposed from the
//    K tile. It also writes D of its rows to the workspace.
//  * bwd_dkdv_kernel: a workgroup owns 128 keys of one key/value head (4
//    waves x 32 keys), K and V of those keys held in registers, and streams
//    the Q/dO tiles (with their lse and D) of every query head of the group
//    through LDS. Per 32-row block it forms S = Q K^T and dP = dO V^T (a
//    lane owns one key), P and dS, then dV^T += dO^T P and dK^T += Q^T dS
//    with dO^T and Q^T read transposed from the tiles. At d = 128 a wave
//    runs its blocks as a two-stage pipeline: the score MFMAs of the next
//    block are interleaved with the softmax of the current one.
// Tiles reach LDS by direct-to-LDS copies; S and dP live in VGPRs and the
// gradient accumulators in AGPRs (inline-asm MFMAs with explicit waits).
// The score and probability fragments of one product are the B operands of
// the next: in a 32x32 MFMA result lane l holds column l % 32 and rows
// 8(r/4) + 4(l/32) + r%4 of its 16 registers r, so registers 8u .. 8u+7
// feed a 16-deep MFMA step whose A operand (read with ds_read_b64_tr_b16)
// lists its rows in that same order.
// Causal masks are aligned bottom-right (key j visible to query i iff
// j <= i + Nk - Nq); tiles that no pair of the workgroup can see are
// skipped. A row whose saved LSE is -inf (it sees no key) has P = 0.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBwdThreads = 256;  // four wavefronts
constexpr int kDqRows = 128;      // query rows per workgroup of the dQ kernel
constexpr int kDqKeys = 64;       // keys per K/V tile of the dQ kernel
constexpr int kKvKeys = 128;      // keys per workgroup of the dK/dV kernel
constexpr int kKvRows = 64;       // query rows per Q/dO tile of the dK/dV kernel
constexpr int kRing = 3;          // LDS buffers of the dK/dV kernel's Q/dO tile ring (d = 128)

// Calls f(std::integral_constant<int, i>) for i = I .. N-1: the index is a
// constant expression in the body.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
// Keep a value's computation ahead of this point (an empty volatile asm
// uses it; the compiler does not move volatile asm across the scheduling
// fences that lay out the MFMA/softmax interleave).
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

typedef short b_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) b_s16x4 b_lds_s16x4;
typedef __attribute__((address_space(3))) const char b_lds_cchar;
typedef unsigned int b_u32x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane j receives
// element j%4 of the 8 bytes addressed by lane 4e + j/4, as its element e.
__device__ __forceinline__ uint2 lds_tr8(b_lds_cchar* p) {
  const b_s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((b_lds_s16x4*)p);
  return __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ uint4 lds_row16(b_lds_cchar* p) {
  return __builtin_bit_cast(uint4, *(const __attribute__((address_space(3))) b_u32x4*)p);
}

// An LDS tile of ROWS rows of D 16-bit values, row-major, its 16-byte
// chunks XOR-permuted inside each row by the row index (the rows that one
// MFMA operand reads then spread over the banks). Both read patterns below
// address whole chunks through the same permutation.
template <int D>
struct Tile {
  static constexpr int ROWB = 2 * D;  // bytes per row
  static constexpr int CH = D / 8;    // 16-byte chunks per row
  // The permutation serves both read patterns below. Row reads take one
  // chunk of 16 consecutive rows: swz is one-to-one on those rows. A
  // transposed read takes two (or, per 32 lanes, four) consecutive chunks of
  // four consecutive rows: swz / 4 (d = 128) differs between those rows, so
  // each row's chunks land in a block of four chunk positions of its own.
  // At d = 64 two rows share 256 bytes; the same holds for the rows of one
  // parity, with the bits of row / 2 permuted instead.
  __device__ static __forceinline__ int swz(int row) {
    if constexpr (CH == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    const int r = (row >> 1) & 7;
    return ((r & 1) << 2) | (r >> 1);
  }
  __device__ static __forceinline__ int chunk(int row, int c) {
    return row * ROWB + 16 * (c ^ swz(row));
  }
  // Row-major A operand of a 32x32x16 MFMA: lane l reads values
  // 16 s + 8 (l/32) .. +7 of row r0 + l % 32.
  __device__ static __forceinline__ uint4 row_frag(b_lds_cchar* t, int r0, int s, int lane) {
    return lds_row16(t + chunk(r0 + (lane & 31), 2 * s + (lane >> 5)));
  }
  // Transposed A operand (A = X^T, 32 columns db of X x 16 rows): lane l
  // gets X[row][32 db + l % 32] for rows r0 + 4 (l/32) + e (elements 0..3)
  // and r0 + 8 + 4 (l/32) + e (elements 4..7), the row order of registers
  // 8u .. 8u+7 of a 32x32 MFMA result (r0 = 16 u of a 32-row block).
  __device__ static __forceinline__ uint4 tr_frag(b_lds_cchar* t, int r0, int db, int lane) {
    const int i = lane & 15;
    const int row = r0 + 4 * (lane >> 5) + (i >> 2);
    const int gran = 8 * db + 4 * ((lane >> 4) & 1) + (i & 3);  // 8-byte granule of the row
    const int off = 16 * ((gran >> 1) ^ swz(row)) + 8 * (gran & 1);
    const int off8 = 16 * ((gran >> 1) ^ swz(row + 8)) + 8 * (gran & 1);
    const uint2 lo = lds_tr8(t + row * ROWB + off);
    const uint2 hi = lds_tr8(t + (row + 8) * ROWB + off8);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
};

// Direct-to-LDS copy of a ROWS x D tile (global_load_lds_dwordx4, no
// registers held while in flight). Load n of thread tid fills LDS chunk
// n * 256 + tid of the tile, so each wavefront instruction writes 1 KB
// contiguously; the lane fetches the logical chunk that Tile<D>'s
// permutation puts there. Rows at or past `valid` repeat row valid - 1:
// the callers give their products a zero weight (masked keys; query rows
// with P = 0).
template <int D, int ROWS>
struct TileCopy {
  static constexpr int CH = D / 8;
  static constexpr int N = ROWS * CH / kBwdThreads;  // loads per thread
  static_assert(N * kBwdThreads == ROWS * CH, "tile pieces");
  __device__ static __forceinline__ void issue(const uint16_t* base, int64_t stride, int row0,
                                               int valid, uint32_t lds_tile, int wave, int lane) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int idx = n * kBwdThreads + wave * 64 + lane, row = idx / CH;
      const int c = (idx % CH) ^ Tile<D>::swz(row);
      const int r = min(row0 + row, valid - 1);
      load_to_lds(base + (int64_t)r * stride + 8 * c, lds_tile + 16 * (n * kBwdThreads + wave * 64));
    }
  }
};
__device__ __forceinline__ void wait_tile_copies() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The MFMAs are written out so that each accumulator keeps one register
// class: the score blocks S and dP, which the vector ALUs read, in VGPRs;
// the gradient accumulators, read once at the end, in AGPRs. (Left to
// itself the compiler placed the scores in AGPRs and moved accumulators
// between the classes on every tile.) It does not know the latency of an
// inline-asm MFMA, so the waits for its results are explicit below.
template <typename T>
__device__ __forceinline__ void mma_v0(f32x16& d, uint4 a, uint4 b) {  // d = a b
  const b_u32x4 x = __builtin_bit_cast(b_u32x4, a), y = __builtin_bit_cast(b_u32x4, b);
  if constexpr (std::is_same<T, Bf16>::value)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(x), "v"(y));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(x), "v"(y));
}
template <typename T>
__device__ __forceinline__ void mma_v(f32x16& d, uint4 a, uint4 b) {  // d += a b
  const b_u32x4 x = __builtin_bit_cast(b_u32x4, a), y = __builtin_bit_cast(b_u32x4, b);
  if constexpr (std::is_same<T, Bf16>::value)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(x), "v"(y));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(x), "v"(y));
}
template <typename T>
__device__ __forceinline__ void mma_a(f32x16& d, uint4 a, uint4 b) {  // d += a b, d in AGPRs
  const b_u32x4 x = __builtin_bit_cast(b_u32x4, a), y = __builtin_bit_cast(b_u32x4, b);
  if constexpr (std::is_same<T, Bf16>::value)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(x), "v"(y));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(d) : "v"(x), "v"(y));
}
// 19 wait states after the MFMAs that wrote S and dP, before anything else
// touches them (an 8-pass MFMA's result may be read 18 states after issue).
// S and dP are operands, so no read of them is scheduled ahead of the wait.
__device__ __forceinline__ void wait_scores(f32x16& a, f32x16& b) {
  asm volatile("s_nop 15\n\ts_nop 2" : "+v"(a), "+v"(b));
}
// 4 wait states between the vector-ALU writes of MFMA B operands and the
// MFMAs that read them
__device__ __forceinline__ void wait_operands(uint4 (&a)[2], uint4 (&b)[2]) {
  b_u32x4 x0 = __builtin_bit_cast(b_u32x4, a[0]), x1 = __builtin_bit_cast(b_u32x4, a[1]);
  b_u32x4 y0 = __builtin_bit_cast(b_u32x4, b[0]), y1 = __builtin_bit_cast(b_u32x4, b[1]);
  asm volatile("s_nop 3" : "+v"(x0), "+v"(x1), "+v"(y0), "+v"(y1));
  a[0] = __builtin_bit_cast(uint4, x0);
  a[1] = __builtin_bit_cast(uint4, x1);
  b[0] = __builtin_bit_cast(uint4, y0);
  b[1] = __builtin_bit_cast(uint4, y1);
}
// the same for two accumulator sets
template <int DB>
__device__ __forceinline__ void wait_acc2(f32x16 (&a)[DB], f32x16 (&b)[DB]) {
  if constexpr (DB == 4)
    asm volatile("s_nop 15\n\ts_nop 2"
                 : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]), "+a"(b[0]), "+a"(b[1]),
                   "+a"(b[2]), "+a"(b[3]));
  else
    asm volatile("s_nop 15\n\ts_nop 2" : "+a"(a[0]), "+a"(a[1]), "+a"(b[0]), "+a"(b[1]));
}
// 19 wait states after the last accumulation, before the epilogue reads the
// accumulators
template <int DB>
__device__ __forceinline__ void wait_acc(f32x16 (&a)[DB]) {
  if constexpr (DB == 4)
    asm volatile("s_nop 15\n\ts_nop 2" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]));
  else
    asm volatile("s_nop 15\n\ts_nop 2" : "+a"(a[0]), "+a"(a[1]));
}

// sum of the products of the eight 16-bit values of a and b, in fp32
template <typename T>
__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
  using E = Elem<T>;
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s = fmaf(E::lo(wa[i]), E::lo(wb[i]), fmaf(E::hi(wa[i]), E::hi(wb[i]), s));
  return s;
}

// lse (natural log) -> the log2-domain offset of P = exp2(s * scale_log2 -
// offset); a row that sees no key (lse = -inf) gets +inf, so its P is 0.
__device__ __forceinline__ float lse_offset(float lse) {
  return lse == neg_inf() ? __builtin_inff() : lse * kLog2e;
}

// 32 x D gradient block, transposed in MFMA layout (lane: one column, rows
// 32 db + 8 gq + 4 (l/32) + 0..3 in registers 4 gq .. 4 gq + 3 of block
// db), times `mul`, stored as one row of D 16-bit values.
template <typename T, int DB>
__device__ __forceinline__ void store_row(uint16_t* dst, const f32x16 (&acc)[DB], float mul,
                                          int hh) {
  using E = Elem<T>;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      uint2 val;
      val.x = E::pack2(acc[db][4 * gq + 0] * mul, acc[db][4 * gq + 1] * mul);
      val.y = E::pack2(acc[db][4 * gq + 2] * mul, acc[db][4 * gq + 3] * mul);
      *(uint2*)(dst + 32 * db + 8 * gq + 4 * hh) = val;
    }
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(BwdParams p) {
  using E = Elem<T>;
  using G = Tile<D>;
  constexpr int KS = D / 16;        // MFMA k-steps over d
  constexpr int DB = D / 32;        // 32-row blocks of dQ^T
  constexpr int NB = kDqKeys / 32;  // 32-key blocks per tile
  constexpr int TB = kDqKeys * G::ROWB;
  __shared__ __attribute__((aligned(16))) char lds[2][2][TB];  // [buffer][K, V]

  // work item (sequence b, query head h, query tile t), longest causal tiles first
  const int nt = (p.Nq + kDqRows - 1) / kDqRows;
  int idx = blockIdx.x;
  const int t = nt - 1 - idx % nt;
  idx /= nt;
  const int h = idx % p.Hq, b = idx / p.Hq;
  const int g = h / p.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int Lq = p.Nq, Lk = p.Nk, delta = Lk - Lq;
  const int row0 = t * kDqRows;
  const int my_row = row0 + wave * 32 + l32;
  const bool row_ok = my_row < Lq;
  const int64_t tok = (int64_t)b * Lq + my_row;  // token index of the row
  const int64_t qoff = tok * p.q_row + (int64_t)h * D;

  // query and output-gradient fragments (B operands, lane = query row) and
  // D = rowsum(dO o O) of the row
  uint4 qf[KS], df[KS];
  float dpart = 0.f;
  if (row_ok) {
    const uint16_t* qs = (const uint16_t*)p.q + qoff + 8 * hh;
    const uint16_t* ds = (const uint16_t*)p.dout + qoff + 8 * hh;
    const uint16_t* os = (const uint16_t*)p.o + qoff + 8 * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = *(const uint4*)(qs + 16 * s);
      df[s] = *(const uint4*)(ds + 16 * s);
      dpart += dot8<T>(df[s], *(const uint4*)(os + 16 * s));
    }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = df[s] = make_uint4(0, 0, 0, 0);
  }
  const float Dq = sum_halves(dpart);
  const float off = row_ok ? lse_offset(p.lse[tok * p.Hq + h]) : __builtin_inff();
  if (row_ok && hh == 0) p.dsum[tok * p.Hq + h] = Dq;

  int kv_end = Lk;
  if (CAUSAL) kv_end = min(Lk, row0 + kDqRows + delta);
  const int n_kv = kv_end > 0 ? (kv_end + kDqKeys - 1) / kDqKeys : 0;
  // last key this row may see
  const int lim = CAUSAL ? min(Lk - 1, my_row + delta) : Lk - 1;
  const float c2 = p.scale_log2;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  const uint16_t* kbase = (const uint16_t*)p.k + (int64_t)b * Lk * p.kv_row + (int64_t)g * D;
  const uint16_t* vbase = (const uint16_t*)p.v + (int64_t)b * Lk * p.kv_row + (int64_t)g * D;
  const uint32_t lds0 = lds_address(lds);
  using Copy = TileCopy<D, kDqKeys>;
  auto issue = [&](int j) {
    const uint32_t t0 = lds0 + (j & 1) * 2 * TB;
    Copy::issue(kbase, p.kv_row, j * kDqKeys, Lk, t0, wave, lane);
    Copy::issue(vbase, p.kv_row, j * kDqKeys, Lk, t0 + TB, wave, lane);
  };
  if (n_kv > 0) issue(0);
  for (int j = 0; j < n_kv; ++j) {
    char* kt = lds[j & 1][0];
    char* vt = lds[j & 1][1];
    // tile j complete everywhere; tile j + 1 goes to the other buffer, last
    // read in iteration j - 1, before every thread passed this barrier
    wait_tile_copies();
    __syncthreads();
    if (j + 1 < n_kv) issue(j + 1);
    b_lds_cchar* K = (b_lds_cchar*)kt;
    b_lds_cchar* V = (b_lds_cchar*)vt;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      f32x16 st, dp;
      mma_v0<T>(st, G::row_frag(K, 32 * kb, 0, lane), qf[0]);
      mma_v0<T>(dp, G::row_frag(V, 32 * kb, 0, lane), df[0]);
#pragma unroll
      for (int s = 1; s < KS; ++s) {
        mma_v<T>(st, G::row_frag(K, 32 * kb, s, lane), qf[s]);
        mma_v<T>(dp, G::row_frag(V, 32 * kb, s, lane), df[s]);
      }
      wait_scores(st, dp);
      // register r holds key j*64 + 32 kb + 4 hh + 8 (r/4) + r%4 of this row
      const int thr = lim - (j * kDqKeys + 32 * kb + 4 * hh);
      uint4 dsf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * u + i;
          const float pv = (8 * (r >> 2) + (r & 3) > thr) ? 0.f : fast_exp2(fmaf(st[r], c2, -off));
          e[i] = pv * (dp[r] - Dq);
        }
        dsf[u] = make_uint4(E::pack2(e[0], e[1]), E::pack2(e[2], e[3]), E::pack2(e[4], e[5]),
                            E::pack2(e[6], e[7]));
      }
      wait_operands(dsf, dsf);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int u = 0; u < 2; ++u) mma_a<T>(acc[db], G::tr_frag(K, 32 * kb + 16 * u, db, lane), dsf[u]);
    }
  }
  wait_acc<DB>(acc);
  if (row_ok) store_row<T, DB>((uint16_t*)p.dq + qoff, acc, p.scale, hh);
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkdv_kernel(BwdParams p) {
  using E = Elem<T>;
  using G = Tile<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int QB = kKvRows / 32;  // 32-row blocks per Q/dO tile
  constexpr int TB = kKvRows * G::ROWB;
  constexpr int RING = D == 128 ? kRing : 2;
  __shared__ __attribute__((aligned(16))) char lds[RING][2][TB];  // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float lds_r[RING][2][kKvRows];  // [buffer][offset, D]

  // work item (sequence b, key/value head g, key tile t); under a causal
  // mask the first key tiles see the most queries and come first
  const int nt = (p.Nk + kKvKeys - 1) / kKvKeys;
  int idx = blockIdx.x;
  const int t = idx % nt;
  idx /= nt;
  const int g = idx % p.Hkv, b = idx / p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int Lq = p.Nq, Lk = p.Nk, delta = Lk - Lq;
  const int my_key = t * kKvKeys + wave * 32 + l32;
  const bool key_ok = my_key < Lk;
  const int64_t ktok = (int64_t)b * Lk + my_key;
  const int64_t koff = ktok * p.kv_row + (int64_t)g * D;

  // K and V of this lane's key (B operands of S = Q K^T and dP = dO V^T)
  uint4 kf[KS], vf[KS];
  if (key_ok) {
    const uint16_t* ks = (const uint16_t*)p.k + koff + 8 * hh;
    const uint16_t* vs = (const uint16_t*)p.v + koff + 8 * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = *(const uint4*)(ks + 16 * s);
      vf[s] = *(const uint4*)(vs + 16 * s);
    }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = vf[s] = make_uint4(0, 0, 0, 0);
  }

  // query rows that may see a key of this tile
  const int q_first = CAUSAL ? max(0, t * kKvKeys - delta) : 0;
  const int qt0 = q_first / kKvRows;
  const int n_qt = Lq > qt0 * kKvRows ? (Lq + kKvRows - 1) / kKvRows - qt0 : 0;
  const int n_it = n_qt * p.group;  // (query head of the group, query tile), head-major
  const float c2 = p.scale_log2;

  f32x16 acc_k[DB], acc_v[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_k[db][r] = acc_v[db][r] = 0.f;

  // Q/dO tiles go through a ring of RING LDS buffers: the barrier opening
  // tile it issues the copies of tile it + 1 into the buffer of tile
  // it + 1 - RING, whose last reads every wave has finished by then (with
  // the pipeline below, the gradients of tile it - 1 still read their
  // buffer after that barrier, hence three buffers at d = 128).
  const uint32_t lds0 = lds_address(lds);
  using Copy = TileCopy<D, kKvRows>;
  float sr = 0.f;  // thread tid < 2*kKvRows stages one lse offset or D value
  auto load = [&](int it) {
    const int h = g * p.group + it / n_qt;
    const int q0 = (qt0 + it % n_qt) * kKvRows;
    const int64_t base = (int64_t)b * Lq * p.q_row + (int64_t)h * D;
    const uint32_t t0 = lds0 + (it % RING) * 2 * TB;
    Copy::issue((const uint16_t*)p.q + base, p.q_row, q0, Lq, t0, wave, lane);
    Copy::issue((const uint16_t*)p.dout + base, p.q_row, q0, Lq, t0 + TB, wave, lane);
    if (tid < 2 * kKvRows) {
      const int row = q0 + (tid % kKvRows);
      const int64_t li = ((int64_t)b * Lq + row) * p.Hq + h;
      if (tid < kKvRows) sr = row < Lq ? lse_offset(p.lse[li]) : __builtin_inff();
      else sr = row < Lq ? p.dsum[li] : 0.f;
    }
  };
  auto open_tile = [&](int it) {
    if (tid < 2 * kKvRows) lds_r[it % RING][tid / kKvRows][tid % kKvRows] = sr;
    wait_tile_copies();
    __syncthreads();
    if (it + 1 < n_it) load(it + 1);
  };
  auto qtile = [&](int it) { return (b_lds_cchar*)lds[it % RING][0]; };
  auto dotile = [&](int it) { return (b_lds_cchar*)lds[it % RING][1]; };

  // The 32-row blocks m = QB it + qb run as a pipeline in one wave: slot m
  // issues the 16 score MFMAs of block m + 1 (S = Q K^T, dP = dO V^T; lane
  // = key), each followed by one element of block m's softmax (P and
  // dS = P o (dP - D) for one query row), then the 16 gradient MFMAs of
  // block m (dV^T += dO^T P, dK^T += Q^T dS). The matrix core then has the
  // next block's MFMAs to run while the vector ALUs work on the current
  // block. Scores alternate between two register sets by block parity.
  f32x16 sA, dA, sB, dB;
  // scores of block (it, qb) into (sn, dn), each MFMA followed by element
  // j of the softmax of the block (itc, qbc) in (sc, dc) when soft is set
  auto slot = [&](int it, int qb, f32x16& sc, f32x16& dc, f32x16& sn, f32x16& dn, int itn,
                  int qbn, auto next_c, auto soft_c) {
    constexpr bool has_next = decltype(next_c)::value;
    constexpr bool soft = decltype(soft_c)::value;
    b_lds_cchar* Qn = qtile(itn);
    b_lds_cchar* dOn = dotile(itn);
    const int buf = it % RING;
    const int q0 = (qt0 + it % n_qt) * kKvRows;
    // register r holds query row q0 + 32 qb + 4 hh + 8 (r/4) + r%4 of this
    // key; under the causal mask it is visible iff 8 (r/4) + r%4 >= thr
    const int thr = my_key - delta - (q0 + 32 * qb + 4 * hh);
    float pe0 = 0.f, de0 = 0.f;
    uint32_t pw[8], dw[8];  // P and dS of the block, packed to 16 bits
    // the block's lse offsets and D values, read before its 16 steps so that
    // their LDS latency is not waited out inside them
    float ov[16], dv[16];
    if constexpr (soft) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int rb = 32 * qb + 8 * gq + 4 * hh;  // first of four rows
        const float4 o4 = *(const float4*)&lds_r[buf][0][rb];
        const float4 d4 = *(const float4*)&lds_r[buf][1][rb];
        ov[4 * gq] = o4.x; ov[4 * gq + 1] = o4.y; ov[4 * gq + 2] = o4.z; ov[4 * gq + 3] = o4.w;
        dv[4 * gq] = d4.x; dv[4 * gq + 1] = d4.y; dv[4 * gq + 2] = d4.z; dv[4 * gq + 3] = d4.w;
      }
    }
    // score fragments read AHEAD MFMAs ahead of their use, in a ring of
    // AHEAD + 1 register sets (one MFMA plus one softmax element covers
    // only a fraction of an LDS read's latency)
    constexpr int AHEAD = 3;
    uint4 fr[AHEAD + 1];
    // 16 steps, one softmax element each; the 2 KS score MFMAs go to every
    // STEP-th step (MFMA mi: k-step mi / 2, S for even mi, dP for odd)
    constexpr int STEP = 16 / (2 * KS);
    static_assert(STEP * 2 * KS == 16, "score MFMAs per block");
    if constexpr (has_next)
      static_for<0, AHEAD>([&](auto m_c) {
        constexpr int m = decltype(m_c)::value;
        if constexpr (m < 2 * KS) fr[m] = G::row_frag((m & 1) ? dOn : Qn, 32 * qbn, m / 2, lane);
      });
    static_for<0, 16>([&](auto j_c) {
      constexpr int j = decltype(j_c)::value;
      if constexpr (has_next && j % STEP == 0) {
        constexpr int mi = j / STEP, s = mi / 2, nx = mi + AHEAD;
        if constexpr (nx < 2 * KS)
          fr[nx % (AHEAD + 1)] = G::row_frag((nx & 1) ? dOn : Qn, 32 * qbn, nx / 2, lane);
        constexpr int fi = mi % (AHEAD + 1);
        if constexpr (mi & 1) {
          if constexpr (s == 0) mma_v0<T>(dn, fr[fi], vf[0]);
          else mma_v<T>(dn, fr[fi], vf[s]);
        } else {
          if constexpr (s == 0) mma_v0<T>(sn, fr[fi], kf[0]);
          else mma_v<T>(sn, fr[fi], kf[s]);
        }
      }
      if constexpr (soft) {
        constexpr int r = j, gq = r / 4, i = r % 4;
        const bool vis = !CAUSAL || (8 * gq + i >= thr);
        float e = fast_exp2(fmaf(sc[r], c2, -ov[r]));
        pin(e);  // computed for every lane, then selected: no branch
        const float pv = vis ? e : 0.f;
        const float dsv = pv * (dc[r] - dv[r]);
        if constexpr (r % 2 == 0) {
          pe0 = pv;
          de0 = dsv;
        } else {  // registers r - 1, r: one 32-bit word of each operand
          pw[r / 2] = E::pack2(pe0, pv);
          dw[r / 2] = E::pack2(de0, dsv);
          pin(pw[r / 2]);
          pin(dw[r / 2]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (has_next) wait_scores(sn, dn);
    if constexpr (soft) {
      uint4 pf[2] = {make_uint4(pw[0], pw[1], pw[2], pw[3]), make_uint4(pw[4], pw[5], pw[6], pw[7])};
      uint4 dsf[2] = {make_uint4(dw[0], dw[1], dw[2], dw[3]), make_uint4(dw[4], dw[5], dw[6], dw[7])};
      wait_operands(pf, dsf);
      b_lds_cchar* Q = qtile(it);
      b_lds_cchar* dO = dotile(it);
      // transposed fragments two MFMA pairs ahead, in a ring of three
      uint4 ta[3], tb[3];
      static_for<0, 2>([&](auto m_c) {
        constexpr int m = decltype(m_c)::value;
        ta[m] = G::tr_frag(dO, 32 * qb + 16 * (m % 2), m / 2, lane);
        tb[m] = G::tr_frag(Q, 32 * qb + 16 * (m % 2), m / 2, lane);
      });
      static_for<0, 2 * DB>([&](auto k_c) {
        constexpr int k = decltype(k_c)::value, db = k / 2, u = k % 2, nx = k + 2;
        if constexpr (nx < 2 * DB) {
          ta[nx % 3] = G::tr_frag(dO, 32 * qb + 16 * (nx % 2), nx / 2, lane);
          tb[nx % 3] = G::tr_frag(Q, 32 * qb + 16 * (nx % 2), nx / 2, lane);
        }
        mma_a<T>(acc_v[db], ta[k % 3], pf[u]);
        mma_a<T>(acc_k[db], tb[k % 3], dsf[u]);
        __builtin_amdgcn_sched_barrier(0);
      });
      // every accumulation complete before the compiler may move an
      // accumulator for its own register allocation
      wait_acc2<DB>(acc_v, acc_k);
    }
  };

  std::integral_constant<bool, true> yes;
  std::integral_constant<bool, false> no;
  static_assert(QB == 2, "two blocks per tile");
  if constexpr (D == 128) {
    if (n_it > 0) {
      load(0);
      open_tile(0);
      slot(0, 0, sA, dA, sA, dA, 0, 0, yes, no);  // scores of block 0 only
      for (int it = 0; it + 1 < n_it; ++it) {
        // block (it, 0): the scores of (it, 1) come from the same tile
        slot(it, 0, sA, dA, sB, dB, it, 1, yes, yes);
        // block (it, 1): the scores of (it + 1, 0) need tile it + 1 opened
        open_tile(it + 1);
        slot(it, 1, sB, dB, sA, dA, it + 1, 0, yes, yes);
      }
      const int il = n_it - 1;
      slot(il, 0, sA, dA, sB, dB, il, 1, yes, yes);
      slot(il, 1, sB, dB, sA, dA, il, 0, no, yes);
    }
  } else {
    // d = 64: the blocks one after the other (the pipeline's second score set
    // would cost the second workgroup per CU that this variant otherwise has)
    if (n_it > 0) load(0);
    for (int it = 0; it < n_it; ++it) {
      const int buf = it % RING;
      // Q/dO tile it complete everywhere; tile it + 1 goes to the other
      // buffer, last read in iteration it - 1, before every thread passed
      // this barrier
      if (tid < 2 * kKvRows) lds_r[buf][tid / kKvRows][tid % kKvRows] = sr;
      wait_tile_copies();
      __syncthreads();
      const int q0 = (qt0 + it % n_qt) * kKvRows;
      if (it + 1 < n_it) load(it + 1);
      b_lds_cchar* Q = (b_lds_cchar*)lds[buf][0];
      b_lds_cchar* dO = (b_lds_cchar*)lds[buf][1];
  #pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x16 st, dp;
        mma_v0<T>(st, G::row_frag(Q, 32 * qb, 0, lane), kf[0]);
        mma_v0<T>(dp, G::row_frag(dO, 32 * qb, 0, lane), vf[0]);
  #pragma unroll
        for (int s = 1; s < KS; ++s) {
          mma_v<T>(st, G::row_frag(Q, 32 * qb, s, lane), kf[s]);
          mma_v<T>(dp, G::row_frag(dO, 32 * qb, s, lane), vf[s]);
        }
        wait_scores(st, dp);
        // register r holds query row q0 + 32 qb + 4 hh + 8 (r/4) + r%4 of this key;
        // under the causal mask it is visible iff 8 (r/4) + r%4 >= thr
        const int thr = my_key - delta - (q0 + 32 * qb + 4 * hh);
        uint4 pf[2], dsf[2];
  #pragma unroll
        for (int u = 0; u < 2; ++u) {
          float pe[8], de[8];
  #pragma unroll
          for (int gq = 0; gq < 2; ++gq) {
            const int rb = 32 * qb + 8 * (2 * u + gq) + 4 * hh;  // first of four rows
            const float4 o4 = *(const float4*)&lds_r[buf][0][rb];
            const float4 d4 = *(const float4*)&lds_r[buf][1][rb];
            const float ov[4] = {o4.x, o4.y, o4.z, o4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 8 * u + 4 * gq + i;
              const bool vis = !CAUSAL || (8 * (r >> 2) + (r & 3) >= thr);
              const float pv = vis ? fast_exp2(fmaf(st[r], c2, -ov[i])) : 0.f;
              pe[4 * gq + i] = pv;
              de[4 * gq + i] = pv * (dp[r] - dv[i]);
            }
          }
          pf[u] = make_uint4(E::pack2(pe[0], pe[1]), E::pack2(pe[2], pe[3]), E::pack2(pe[4], pe[5]),
                             E::pack2(pe[6], pe[7]));
          dsf[u] = make_uint4(E::pack2(de[0], de[1]), E::pack2(de[2], de[3]),
                              E::pack2(de[4], de[5]), E::pack2(de[6], de[7]));
        }
        wait_operands(pf, dsf);
  #pragma unroll
        for (int db = 0; db < DB; ++db)
  #pragma unroll
          for (int u = 0; u < 2; ++u) {
            mma_a<T>(acc_v[db], G::tr_frag(dO, 32 * qb + 16 * u, db, lane), pf[u]);
            mma_a<T>(acc_k[db], G::tr_frag(Q, 32 * qb + 16 * u, db, lane), dsf[u]);
          }
      }
    }
  }
  wait_acc<DB>(acc_v);
  wait_acc<DB>(acc_k);
  if (key_ok) {
    store_row<T, DB>((uint16_t*)p.dk + koff, acc_k, p.scale, hh);
    store_row<T, DB>((uint16_t*)p.dv + koff, acc_v, 1.f, hh);
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t st) {
  const int64_t dq_blocks = (int64_t)p.B * p.Hq * ((p.Nq + kDqRows - 1) / kDqRows);
  const int64_t kv_blocks = (int64_t)p.B * p.Hkv * ((p.Nk + kKvKeys - 1) / kKvKeys);
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL>), dim3((int)dq_blocks), dim3(kBwdThreads), 0, st,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>), dim3((int)kv_blocks), dim3(kBwdThreads), 0,
                     st, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_d(const BwdParams& p, bool causal, hipStream_t st) {
  return causal ? launch_bwd_t<T, D, true>(p, st) : launch_bwd_t<T, D, false>(p, st);
}

}  // namespace

int64_t bwd_grid_blocks(int B, int Nq, int Nk, int Hq, int Hkv) {
  const int64_t a = (int64_t)B * Hq * ((Nq + kDqRows - 1) / kDqRows);
  const int64_t c = (int64_t)B * Hkv * ((Nk + kKvKeys - 1) / kKvKeys);
  return a > c ? a : c;
}

hipError_t launch_bwd(const BwdParams& p, Dt dt, int d, bool causal, hipStream_t st) {
  switch (dt) {
    case Dt::Bf16:
      return d == 64 ? launch_bwd_d<Bf16, 64>(p, causal, st)
                     : launch_bwd_d<Bf16, 128>(p, causal, st);
    case Dt::F16:
      return d == 64 ? launch_bwd_d<F16, 64>(p, causal, st) : launch_bwd_d<F16, 128>(p, causal, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fa
