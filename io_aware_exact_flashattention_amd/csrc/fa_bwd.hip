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
//  * dK/dV: a workgroup owns 128 keys of one key/value head, K and V of
//    those keys held in registers, and streams the Q/dO tiles (with their
//    lse and D) of every query head of the group through LDS. Per 32-row
//    block it forms S = Q K^T and dP = dO V^T (a lane owns one key), P and
//    dS, then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read
//    transposed from the tiles. At d = 128 (bwd_dkdv_pair_kernel) two waves
//    of a SIMD share each 32-key group: one forms S, P and dV, the other dP,
//    dS and dK, with P passed through LDS, in counter-phase like the
//    forward kernel's wave pairs. At d = 64 (bwd_dkdv_kernel) one wave does
//    all of it for its 32 keys, so that two workgroups fit on a CU.
// Work items are numbered so that each XCD runs a contiguous stretch of the
// work list, longest tiles of its heads first: the items running on one XCD
// at a time read the same Q/dO (or K/V) tiles, which then stay in its L2.
// Tiles reach LDS by direct-to-LDS copies; S and dP live in VGPRs, the
// gradient accumulators in AGPRs or VGPRs (inline-asm MFMAs with fixed
// register classes and explicit waits).
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

// Calls f(std::integral_constant<int, i>) for i = I .. N-1: the index is a
// constant expression in the body.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

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
template <int D, int ROWS, int THREADS = kBwdThreads>
struct TileCopy {
  static constexpr int CH = D / 8;
  static constexpr int N = ROWS * CH / THREADS;  // loads per thread
  static_assert(N * THREADS == ROWS * CH, "tile pieces");
  __device__ static __forceinline__ void issue(const uint16_t* base, int64_t stride, int row0,
                                               int valid, uint32_t lds_tile, int wave, int lane) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int idx = n * THREADS + wave * 64 + lane, row = idx / CH;
      const int c = (idx % CH) ^ Tile<D>::swz(row);
      const int r = min(row0 + row, valid - 1);
      load_to_lds(base + (int64_t)r * stride + 8 * c, lds_tile + 16 * (n * THREADS + wave * 64));
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
// 19 wait states after the last accumulation, before the epilogue reads the
// accumulators
template <int DB>
__device__ __forceinline__ void wait_acc(f32x16 (&a)[DB]) {
  if constexpr (DB == 4)
    asm volatile("s_nop 15\n\ts_nop 2" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]));
  else
    asm volatile("s_nop 15\n\ts_nop 2" : "+a"(a[0]), "+a"(a[1]));
}

// the same for accumulators held in VGPRs
template <int DB>
__device__ __forceinline__ void wait_acc_v(f32x16 (&a)[DB]) {
  if constexpr (DB == 4)
    asm volatile("s_nop 15\n\ts_nop 2" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
  else
    asm volatile("s_nop 15\n\ts_nop 2" : "+v"(a[0]), "+v"(a[1]));
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

// Work order. Workgroups are dealt round-robin over the 8 XCDs (workgroup L
// runs on XCD L % 8), so the ids are renumbered: XCD x takes the contiguous
// stretch [x*per + min(x, rem), ...) of the work list of (sequence, head)
// units of n_tiles items each, and the items running on one XCD at a time
// share the units' tiles in its L2. When the stretch is made of whole units
// it is taken tile-major - the first tile of each of its units, then the
// second, and so on - so that its longest items (under a causal mask) start
// first on every unit. Returns the unit and the tile rank.
__device__ __forceinline__ void xcd_unit_tile(int n_tiles, int& unit, int& rank) {
  const int L = blockIdx.x, total = gridDim.x;
  const int xcd = L & 7, idx = L >> 3, per = total >> 3, rem = total & 7;
  if (rem == 0 && per % n_tiles == 0) {
    const int upx = per / n_tiles;
    unit = xcd * upx + idx % upx;
    rank = idx / upx;
  } else {
    const int item = xcd * per + min(xcd, rem) + idx;
    unit = item / n_tiles;
    rank = item % n_tiles;
  }
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
  int idx, rank;
  xcd_unit_tile(nt, idx, rank);
  const int t = nt - 1 - rank;
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
  // D and the lse offset of the row, head by head for the dK/dV kernels
  // (their 64-row tiles then read one contiguous run)
  if (row_ok && hh == 0) {
    const int64_t ti = ((int64_t)b * p.Hq + h) * p.n_pad + my_row;
    p.dsum[ti] = Dq;
    p.lse2[ti] = off;
  }

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
  static_assert(D == 64, "d = 128 always runs bwd_dkdv_pair_kernel");
  using E = Elem<T>;
  using G = Tile<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int QB = kKvRows / 32;  // 32-row blocks per Q/dO tile
  constexpr int TB = kKvRows * G::ROWB;
  constexpr int RING = 2;
  __shared__ __attribute__((aligned(16))) char lds[RING][2][TB];  // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float lds_r[RING][2][kKvRows];  // [buffer][offset, D]

  // work item (sequence b, key/value head g, key tile t); under a causal
  // mask the first key tiles see the most queries and come first
  const int nt = (p.Nk + kKvKeys - 1) / kKvKeys;
  int idx, t;
  xcd_unit_tile(nt, idx, t);
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

  // Q/dO tiles alternate between two LDS buffers: the barrier opening tile
  // it issues the copies of tile it + 1 into the other buffer, whose last
  // reads (tile it - 1) every wave has finished by then.
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
      const int64_t ti = ((int64_t)b * p.Hq + h) * p.n_pad + row;
      if (tid < kKvRows) sr = row < Lq ? p.lse2[ti] : __builtin_inff();
      else sr = row < Lq ? p.dsum[ti] : 0.f;
    }
  };
  // one 32-row block after the other
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
  wait_acc<DB>(acc_v);
  wait_acc<DB>(acc_k);
  if (key_ok) {
    store_row<T, DB>((uint16_t*)p.dk + koff, acc_k, p.scale, hh);
    store_row<T, DB>((uint16_t*)p.dv + koff, acc_v, 1.f, hh);
  }
}

// dK/dV with the work of a 32-key group split over two waves that share a
// SIMD. The "P wave" holds K, forms S = Q K^T and P and accumulates
// dV^T += dO^T P; the "dS wave" holds V, forms dP = dO V^T and
// dS = P o (dP - D) and accumulates dK^T += Q^T dS. P goes from the one to
// the other through LDS in fp32, so every value is the one that one wave
// doing all of it would compute (as bwd_dkdv_kernel does at d = 64). Each wave alternates a matrix phase (MFMAs and LDS
// fragment reads) with a vector phase (P, or dS), the two waves of a SIMD in
// counter-phase, every phase boundary a workgroup barrier, as in the forward
// kernel:
//   first half of slot i:  P wave  S(i+1), dV(i)   |  dS wave  dS(i)
//   second half of slot i: P wave  P(i+1)          |  dS wave  dP(i+1), dK(i)
// where i is a 64-row Q/dO tile. Tile i is read in slots i-1 and i; the
// barrier that ends slot i-2 completes it, the one that ends slot i-3 issues
// its copies into a ring of three buffers.
constexpr int kPairThreads = 512;  // 4 key groups x 2 roles
constexpr int kCUs = 256;          // compute units of an MI355X

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kPairThreads) void bwd_dkdv_pair_kernel(BwdParams p) {
  using E = Elem<T>;
  using G = Tile<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TB = kKvRows * G::ROWB;
  constexpr int RING = 3;
  constexpr int STEPS = 2 * KS;  // MFMAs of each kind per matrix phase (two 32-row blocks)
  static_assert(2 * 2 * DB == STEPS, "score and gradient MFMAs pair up");
  constexpr int LD = kKvRows * G::CH / kPairThreads;  // copies per thread per tensor and tile
  static_assert(LD * kPairThreads == kKvRows * G::CH, "tile pieces");
  __shared__ __attribute__((aligned(16))) char lds[RING][2][TB];          // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float lds_r[RING][2][kKvRows];  // [buffer][offset, D]
  // P of the current tile, per key group: float4 w of lane l at [w][l]
  __shared__ __attribute__((aligned(16))) float4 xch[4][8][64];

  const int nt = (p.Nk + kKvKeys - 1) / kKvKeys;
  int idx, t;
  xcd_unit_tile(nt, idx, t);
  const int g = idx % p.Hkv, b = idx / p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3;     // key group; waves kg and kg + 4 share a SIMD
  const int role = wave >> 2;  // 0: S, P, dV; 1: dP, dS, dK
  const int l32 = lane & 31, hh = lane >> 5;
  const int Lq = p.Nq, Lk = p.Nk, delta = Lk - Lq;
  const int my_key = t * kKvKeys + kg * 32 + l32;
  const bool key_ok = my_key < Lk;
  const int64_t ktok = (int64_t)b * Lk + my_key;
  const int64_t koff = ktok * p.kv_row + (int64_t)g * D;

  // K (P wave) or V (dS wave) of this lane's key: the B operand of the
  // wave's score product
  uint4 bf[KS];
  if (key_ok) {
    const uint16_t* src = (const uint16_t*)(role == 0 ? p.k : p.v) + koff + 8 * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) bf[s] = *(const uint4*)(src + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) bf[s] = make_uint4(0, 0, 0, 0);
  }

  const int q_first = CAUSAL ? max(0, t * kKvKeys - delta) : 0;
  const int qt0 = q_first / kKvRows;
  const int n_qt = Lq > qt0 * kKvRows ? (Lq + kKvRows - 1) / kKvRows - qt0 : 0;
  const int n_it = n_qt * p.group;  // (query head of the group, query tile), head-major
  const float c2 = p.scale_log2;

  f32x16 acc[DB];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  f32x16 sc[2];    // S or dP of the two 32-row blocks of a tile
  uint4 op[2][2];  // P or dS of a tile, packed: B operands of the gradient MFMAs

  // ---- tile copies: a wave-uniform base plus 32-bit lane offsets ----
  // Copy n of thread tid fills LDS chunk n * 512 + tid of the tile with the
  // logical chunk that the tile permutation puts there; rows past the
  // sequence end repeat its last row (their P is 0).
  int cp_row[LD], cp_col[LD];  // row inside the tile, byte offset inside the row
#pragma unroll
  for (int n = 0; n < LD; ++n) {
    const int i = n * kPairThreads + tid, row = i / G::CH;
    cp_row[n] = row;
    cp_col[n] = 16 * ((i % G::CH) ^ G::swz(row));
  }
  const uint32_t lds0 = lds_address(lds);
  float sr = 0.f;  // thread tid < 2*kKvRows stages one lse offset or D value
  auto load = [&](int it) {
    const int h = g * p.group + it / n_qt;
    const int q0 = (qt0 + it % n_qt) * kKvRows;
    const int64_t e0 = ((int64_t)b * Lq + q0) * p.q_row + (int64_t)h * D;
    const uint16_t* qb = (const uint16_t*)p.q + e0;
    const uint16_t* db = (const uint16_t*)p.dout + e0;
    const int last = Lq - 1 - q0;  // last row of the tile inside the sequence
    const uint32_t t0 = lds0 + __builtin_amdgcn_readfirstlane((it % RING) * 2 * TB) + wave * 1024;
#pragma unroll
    for (int n = 0; n < LD; ++n) {
      const uint32_t vo = (uint32_t)(min(cp_row[n], last) * (int)p.q_row * 2 + cp_col[n]);
      load_to_lds_sv(qb, vo, t0 + n * kPairThreads * 16);
      load_to_lds_sv(db, vo, t0 + TB + n * kPairThreads * 16);
    }
    if (tid < 2 * kKvRows) {
      const int row = q0 + (tid % kKvRows);
      const int64_t ti = ((int64_t)b * p.Hq + h) * p.n_pad + row;
      if (tid < kKvRows) sr = row < Lq ? p.lse2[ti] : __builtin_inff();
      else sr = row < Lq ? p.dsum[ti] : 0.f;
    }
  };
  // barrier that ends slot it: tile it + 2 (issued one slot earlier) is
  // complete and its lse/D values staged; tile it + 3 goes to the buffer of
  // tile it, last read in slot it
  auto end_slot = [&](int it) {
    if (it + 2 < n_it && tid < 2 * kKvRows)
      lds_r[(it + 2) % RING][tid / kKvRows][tid % kKvRows] = sr;
    wait_tile_copies();
    __syncthreads();
    if (it + 3 < n_it) load(it + 3);
  };

  // ---- per-lane LDS read offsets inside a tile (bytes) ----
  // Score A operand, row-major: row 32 qb + l32, logical chunk 2 s + hh (the
  // 32-row step leaves the permutation unchanged: an immediate offset).
  int s_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) s_off[s] = G::chunk(l32, 2 * s + hh);
  // Gradient A operand, transposed: for d-block db the rows 4 hh + (l%16)/4
  // and 8 more, at granule 8 db + 4 ((l/16)%2) + l%4 (the 16-row steps of
  // qb and u leave the permutation unchanged).
  int g_off[DB][2];
  {
    const int i = lane & 15, row = 4 * hh + (i >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int gran = 8 * db + 4 * ((lane >> 4) & 1) + (i & 3);
      g_off[db][0] = row * G::ROWB + 16 * ((gran >> 1) ^ G::swz(row)) + 8 * (gran & 1);
      g_off[db][1] = (row + 8) * G::ROWB + 16 * ((gran >> 1) ^ G::swz(row + 8)) + 8 * (gran & 1);
    }
  }
  // byte offset of a tile's Q (tensor 0) or dO (tensor 1) inside lds, as a
  // wave-uniform value (so that the fragment addresses stay lane offset +
  // uniform base instead of one induction variable each)
  auto tile_base = [&](int it, int tensor) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((it % RING) * 2 * TB + tensor * TB);
  };
  b_lds_cchar* const L = (b_lds_cchar*)lds;

  // Matrix phase: the score product of tile it + 1 (NEXT) and the gradient
  // product of tile it (GRAD), one MFMA of each per step; A fragments are
  // read two steps ahead. Score MFMA i: block i / KS, k-step i % KS.
  // Gradient MFMA i: block i / (2 DB), d-block (i % (2 DB)) / 2, rows
  // 16 (i % 2) of the block (the order in which bwd_dkdv_kernel accumulates).
  // score A operand rows: Q (P wave) or dO (dS wave) of tile it + 1;
  // gradient A operand: dO (P wave) or Q (dS wave) of tile it, transposed
  auto sfrag = [&](int it, int i) {
    return lds_row16(L + tile_base(it + 1, role) + s_off[i % KS] + 32 * (i / KS) * G::ROWB);
  };
  auto gfrag = [&](int it, int i) {
    const uint32_t yb = tile_base(it, 1 - role);
    const int r0 = 32 * (i / (2 * DB)) + 16 * (i % 2), db = (i % (2 * DB)) / 2;
    const uint2 lo = lds_tr8(L + yb + g_off[db][0] + r0 * G::ROWB);
    const uint2 hi = lds_tr8(L + yb + g_off[db][1] + r0 * G::ROWB);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };
  // fragment rings of the matrix phase; the first two of each are read
  // ahead of the phase (pre_s, pre_g), while the vector phase runs when the
  // tile is already complete
  uint4 fs[3], fg[3];
  auto pre_s = [&](int it) { fs[0] = sfrag(it, 0); fs[1] = sfrag(it, 1); };
  auto pre_g = [&](int it) { fg[0] = gfrag(it, 0); fg[1] = gfrag(it, 1); };
  auto matrix = [&](int it, auto next_c, auto grad_c) {
    constexpr bool NEXT = decltype(next_c)::value;
    constexpr bool GRAD = decltype(grad_c)::value;
    __builtin_amdgcn_s_setprio(1);
    static_for<0, STEPS>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      if constexpr (i + 2 < STEPS) {
        if constexpr (NEXT) fs[(i + 2) % 3] = sfrag(it, i + 2);
        if constexpr (GRAD) fg[(i + 2) % 3] = gfrag(it, i + 2);
      }
      if constexpr (NEXT) {
        constexpr int qb = i / KS, s = i % KS;
        if constexpr (s == 0) mma_v0<T>(sc[qb], fs[i % 3], bf[0]);
        else mma_v<T>(sc[qb], fs[i % 3], bf[s]);
      }
      if constexpr (GRAD) {
        constexpr int qb = i / (2 * DB), db = (i % (2 * DB)) / 2, u = i % 2;
        mma_v<T>(acc[db], fg[i % 3], op[qb][u]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    __builtin_amdgcn_s_setprio(0);
    if constexpr (NEXT) wait_scores(sc[0], sc[1]);
    if constexpr (GRAD) wait_acc_v<DB>(acc);
  };

  const int q_lane = 4 * hh;  // first query row of this lane in each group of 8
  // P wave, vector phase: P of tile it from its scores, to the exchange
  // buffer (fp32) and to op (packed)
  auto probs = [&](int it) {
    const int buf = it % RING, q0 = (qt0 + it % n_qt) * kKvRows;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // register r holds query row q0 + 32 qb + 4 hh + 8 (r/4) + r%4 of this
      // key; under the causal mask it is visible iff 8 (r/4) + r%4 >= thr
      const int thr = my_key - delta - (q0 + 32 * qb + q_lane);
      float pv[16];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float4 o4 = *(const float4*)&lds_r[buf][0][32 * qb + 8 * gq + q_lane];
        const float ov[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * gq + i;
          const bool vis = !CAUSAL || (8 * gq + i >= thr);
          const float e = fast_exp2(fmaf(sc[qb][r], c2, -ov[i]));
          pv[r] = vis ? e : 0.f;
        }
        xch[kg][4 * qb + gq][lane] =
            make_float4(pv[4 * gq], pv[4 * gq + 1], pv[4 * gq + 2], pv[4 * gq + 3]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        op[qb][u] = make_uint4(E::pack2(pv[8 * u], pv[8 * u + 1]), E::pack2(pv[8 * u + 2], pv[8 * u + 3]),
                               E::pack2(pv[8 * u + 4], pv[8 * u + 5]),
                               E::pack2(pv[8 * u + 6], pv[8 * u + 7]));
    }
    wait_operands(op[0], op[1]);
  };
  // dS wave, vector phase: dS of tile it from P (exchange buffer) and dP
  auto grads = [&](int it) {
    const int buf = it % RING;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float dsv[16];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float4 d4 = *(const float4*)&lds_r[buf][1][32 * qb + 8 * gq + q_lane];
        const float4 p4 = xch[kg][4 * qb + gq][lane];
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w}, pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) dsv[4 * gq + i] = pv[i] * (sc[qb][4 * gq + i] - dv[i]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        op[qb][u] = make_uint4(E::pack2(dsv[8 * u], dsv[8 * u + 1]), E::pack2(dsv[8 * u + 2], dsv[8 * u + 3]),
                               E::pack2(dsv[8 * u + 4], dsv[8 * u + 5]),
                               E::pack2(dsv[8 * u + 6], dsv[8 * u + 7]));
    }
    wait_operands(op[0], op[1]);
  };

  std::integral_constant<bool, true> yes;
  std::integral_constant<bool, false> no;
  if (n_it > 0) {
    load(0);
    if (tid < 2 * kKvRows) lds_r[0][tid / kKvRows][tid % kKvRows] = sr;
    wait_tile_copies();
    __syncthreads();
    if (n_it > 1) load(1);
    if (role == 0) {
      pre_s(-1);
      matrix(-1, yes, no);  // S(0)
      __syncthreads();
      probs(0);
      pre_g(0);
      end_slot(-1);
      for (int it = 0; it + 1 < n_it; ++it) {
        pre_s(it);  // tile it + 1, complete since the last barrier
        matrix(it, yes, yes);  // S(it+1), dV(it)
        __syncthreads();
        probs(it + 1);
        pre_g(it + 1);
        end_slot(it);
      }
      matrix(n_it - 1, no, yes);  // dV(last)
      __syncthreads();
    } else {
      __syncthreads();
      pre_s(-1);
      matrix(-1, yes, no);  // dP(0)
      end_slot(-1);
      for (int it = 0; it + 1 < n_it; ++it) {
        grads(it);
        pre_s(it);
        pre_g(it);
        __syncthreads();
        matrix(it, yes, yes);  // dP(it+1), dK(it)
        end_slot(it);
      }
      grads(n_it - 1);
      pre_g(n_it - 1);
      __syncthreads();
      matrix(n_it - 1, no, yes);  // dK(last)
    }
  }
  if (key_ok) store_row<T, DB>((uint16_t*)(role == 0 ? p.dv : p.dk) + koff, acc,
                               role == 0 ? 1.f : p.scale, hh);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t st) {
  const int64_t dq_blocks = (int64_t)p.B * p.Hq * ((p.Nq + kDqRows - 1) / kDqRows);
  const int64_t kv_blocks = (int64_t)p.B * p.Hkv * ((p.Nk + kKvKeys - 1) / kKvKeys);
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL>), dim3((int)dq_blocks), dim3(kBwdThreads), 0, st,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // d = 128: always the wave-pair kernel. d = 64: the one-wave kernel, whose
  // two workgroups per CU fill the chip when there are enough of them; with
  // fewer key workgroups than CUs the wave-pair kernel's eight waves per
  // workgroup do more. Both give the same bits.
  if constexpr (D == 128) {
    hipLaunchKernelGGL((bwd_dkdv_pair_kernel<T, D, CAUSAL>), dim3((int)kv_blocks),
                       dim3(kPairThreads), 0, st, p);
  } else {
    if (kv_blocks < kCUs)
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<T, D, CAUSAL>), dim3((int)kv_blocks),
                         dim3(kPairThreads), 0, st, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>), dim3((int)kv_blocks), dim3(kBwdThreads),
                         0, st, p);
  }
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
