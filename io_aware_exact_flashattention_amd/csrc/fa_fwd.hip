// fa_fwd.hip - fused attention forward (prefill) kernels for gfx950.
//
// The method is the fused forward pass of the page "I/O-Aware Kernels"
// (datasystem.school, Module 5), section "FlashAttention: tiling + online
// softmax": a workgroup holds one tile of query rows on chip, streams the
// key/value tiles of its sequence through LDS, computes the partial scores
// of each tile, keeps a running row max m and row sum l, and rescales its
// output accumulator whenever m grows. The score matrix lives only in
// registers; device memory sees Q, K, V read and O, LSE written.
//
// gfx950 mapping of the 16-bit path (fwd_mfma_kernel):
//  * 4 wavefronts x 32 query rows = 128-row Q tile; K/V tiles of 64 keys.
//  * Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_{bf16,f16}: the Q fragment is the B operand held in
//    VGPRs for the whole loop, K rows come from LDS as the A operand. In the
//    32x32 result a lane owns one query (lane % 32) and 16 of the 32 keys, so
//    a row max / row sum is a per-lane reduction plus one exchange with
//    lane ^ 32 - no LDS and no atomics.
//  * The same lane layout is exactly the B operand of O^T += V^T P^T, so the
//    probabilities go from the score accumulator to the second MFMA after a
//    round-to-nearest conversion to 16 bits, without leaving the lane.
//  * V is stored transposed in LDS (V^T, keys permuted to match the lane
//    layout of P), written from two key rows at a time as packed pairs.
//  * K and V^T tiles are double-buffered in LDS: the global loads of tile
//    j+1 are in flight while tile j is multiplied; one barrier per tile.
//  * LDS rows are XOR-swizzled in 16-byte chunks so that the 32 rows read
//    by one MFMA operand fall in distinct banks.
//  * Workgroup ids are remapped so that each XCD (workgroups are dealt out
//    round-robin over the 8 XCDs) gets a contiguous run of (sequence, head)
//    units, keeping a head's K/V in that XCD's L2; inside a head the query
//    tiles run longest (last, under a causal mask) first.
//  * Causal: K/V tiles that no row of the Q tile may see are never loaded;
//    only tiles that cross the diagonal or the sequence end are masked.
//
// fp32 inputs take fwd_f32_kernel: the same tiling and online softmax on
// the vector ALUs (4 lanes per query row), for exact fp32 arithmetic.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBM = 256;      // query rows per workgroup, 16-bit path (8 waves x 32)
constexpr int kBN = 64;       // keys per K/V tile, 16-bit path
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kStages = 4;    // LDS ring of K/V tiles
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maximum.
constexpr int kWaitVmcnt0 = 0x0F70;
// s_waitcnt immediate: vmcnt(n) for n < 16, expcnt and lgkmcnt at their maximum.
constexpr int wait_vmcnt(int n) { return 0x0F70 | n; }
// Rescale threshold of the running max (log2 units): weights stay <= 2^8.
constexpr float kRescale = 8.f;

struct Work {
  int b, h, tile;
};

// Workgroup -> (sequence, query head, query tile). Consecutive workgroups
// land on different XCDs, so the linear id is first regrouped so that XCD x
// owns the contiguous logical range [x*per, (x+1)*per) of the work list.
__device__ __forceinline__ Work map_block(int n_qtiles, int Hq) {
  const int L = blockIdx.x;
  const int total = gridDim.x;
  const int xcd = L & 7, idx = L >> 3;
  const int per = total >> 3, rem = total & 7;
  const int logical = xcd * per + min(xcd, rem) + idx;
  const int t = logical % n_qtiles;
  const int hb = logical / n_qtiles;
  Work w;
  w.tile = n_qtiles - 1 - t;
  w.h = hb % Hq;
  w.b = hb / Hq;
  return w;
}

__device__ __forceinline__ void seq_bounds(const FwdParams& p, int b, int& q0, int& Lq, int& k0,
                                           int& Lk) {
  if (p.cu_q) {
    q0 = p.cu_q[b];
    Lq = p.cu_q[b + 1] - q0;
    k0 = p.cu_k[b];
    Lk = p.cu_k[b + 1] - k0;
  } else {
    q0 = b * p.Nq;
    Lq = p.Nq;
    k0 = b * p.Nk;
    Lk = p.Nk;
  }
}

// LDS geometry of one K or V tile: kBN rows of D 16-bit values, row-major,
// in 16-byte chunks whose order inside a row is XOR-swizzled by the row.
template <int D>
struct TileGeom {
  static constexpr int ROWB = 2 * D;                    // bytes per row
  static constexpr int CH = D / 8;                      // chunks per row
  static constexpr int BYTES = kBN * ROWB;              // bytes per tile
  static constexpr int LOADS = BYTES / (kThreads * 16); // 16-byte loads per lane per tile
  // K is read as the A operand of S^T = K Q^T: 32 consecutive rows, one
  // chunk each; the swizzle spreads any 16 consecutive rows over all banks.
  __device__ static __forceinline__ int k_swz(int row) {
    if constexpr (CH == 16) return row & 15;
    else return (row >> 1) & 7;
  }
  // V is read with ds_read_b64_tr_b16: per instruction 8 rows (4 per half
  // wave) x 64 contiguous bytes; the swizzle moves the 4 rows of a half
  // wave to disjoint bank groups.
  __device__ static __forceinline__ int v_swz(int row) {
    if constexpr (CH == 16) return 4 * (row & 3);
    else return 4 * ((row >> 1) & 1);
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16. Inside each group of 16 lanes, lane j receives element
// j%4 of the 8 bytes addressed by lane 4e + j/4, as its element e.
__device__ __forceinline__ uint2 lds_read_tr(const char* lds_byte_ptr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lds_byte_ptr);
  return __builtin_bit_cast(uint2, v);
}

// Keep a value's computation ahead of this point: the empty volatile asm
// "uses" it, and the compiler does not move volatile asm across the
// scheduling fences that lay out the MFMA/softmax overlap.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint4& x) {
  asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
}


template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_mfma_kernel(FwdParams p) {
  using E = Elem<T>;
  using G = TileGeom<D>;
  constexpr int KS = D / 16;    // MFMA k-steps of Q K^T
  constexpr int DB = D / 32;    // 32-row blocks of O^T
  constexpr int NB = kBN / 32;  // 32-key blocks per tile
  constexpr int LD = G::LOADS;
  constexpr int TILE_LOADS = 2 * LD;             // K and V loads per lane per tile
  constexpr int STAGE = 2 * G::BYTES;            // one K tile then one V tile

  // Ring of kStages (K, V) tile pairs. Tile j lives in stage j % kStages; it
  // is loaded two steps before its keys are first used.
  __shared__ __attribute__((aligned(16))) char lds[kStages * STAGE];

  const Work w = map_block(p.n_qtiles, p.Hq);
  int q0, Lq, k0, Lk;
  seq_bounds(p, w.b, q0, Lq, k0, Lk);
  const int row0 = w.tile * kBM;
  if (row0 >= Lq) return;  // ragged batch: this sequence has fewer tiles

  const int g = w.h / p.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int delta = Lk - Lq;  // bottom-right causal offset

  int kv_end = Lk;
  if (CAUSAL) kv_end = min(Lk, row0 + kBM + delta);
  const int n_kv = kv_end > 0 ? (kv_end + kBN - 1) / kBN : 0;

  const int wrow0 = row0 + wave * 32;
  const int my_row = wrow0 + l32;

  // Q fragment: B operand of S^T = K Q^T. Lane (l32, hh) holds
  // Q[my_row][16s + 8hh .. +7] for every k-step s.
  uint4 qf[KS];
  if (my_row < Lq) {
    const uint16_t* src = (const uint16_t*)p.q + (int64_t)(q0 + my_row) * p.q_row +
                          (int64_t)w.h * D + hh * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *(const uint4*)(src + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = make_uint4(0, 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // ---- direct-to-LDS tile loads: this lane's rows and source chunks ----
  // Load n of thread tid fills LDS bytes (n*kThreads + tid)*16 of a tile;
  // the swizzle is applied on the source side.
  int ld_row[LD], k_col[LD], v_col[LD];
#pragma unroll
  for (int n = 0; n < LD; ++n) {
    const int pos = (n * kThreads + tid) * 16;
    const int r = pos / G::ROWB, pc = (pos % G::ROWB) / 16;
    ld_row[n] = r;
    k_col[n] = 8 * (pc ^ G::k_swz(r));
    v_col[n] = 8 * (pc ^ G::v_swz(r));
  }
  const uint16_t* kbase = (const uint16_t*)p.k + (int64_t)k0 * p.kv_row + (int64_t)g * D;
  const uint16_t* vbase = (const uint16_t*)p.v + (int64_t)k0 * p.kv_row + (int64_t)g * D;
  const int last_key = Lk - 1;
  const uint32_t lds0 = lds_address(lds);
  const uint32_t lds_wave = lds0 + wave * 64 * 16;

  auto issue_tile = [&](int j) {
    const uint32_t st = lds_wave + (j % kStages) * STAGE;
#pragma unroll
    for (int n = 0; n < LD; ++n) {
      // rows past the sequence end repeat its last row (finite values that
      // the mask gives weight zero)
      const int64_t key = min(j * kBN + ld_row[n], last_key);
      load_to_lds(kbase + key * p.kv_row + k_col[n], st + n * kThreads * 16);
      load_to_lds(vbase + key * p.kv_row + v_col[n], st + G::BYTES + n * kThreads * 16);
    }
  };

  // ---- per-lane LDS read offsets (bytes, inside a tile) ----
  // K, A operand of S^T: row 32kb + l32, logical chunk 2s + hh. The kb term
  // (32 rows) leaves the swizzle unchanged and is an immediate offset.
  int k_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) k_off[s] = l32 * G::ROWB + 16 * ((2 * s + hh) ^ G::k_swz(l32));
  // V, A operand of O^T += V^T P^T via transpose reads. For (kb, u, t) the
  // 16-lane group reads rows 32kb + 16u + 8t + 4hh + i/4 (i = lane % 16) at
  // columns d = 32db + 16*((lane/16)%2) + 4*(i%4): lane j of the group then
  // holds V[those 4 rows][32db + lane%32], which are the keys of its P
  // fragment (registers 8u + 4t .. +3 of score block kb). Multiples of 8
  // rows leave the swizzle unchanged and are immediate offsets.
  const int vi = lane & 15;
  const int v_row = 4 * hh + (vi >> 2);
  int v_off[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int gran = 8 * db + 4 * ((lane >> 4) & 1) + (vi & 3);  // 8-byte granule of the row
    v_off[db] = G::BYTES + v_row * G::ROWB + 16 * ((gran >> 1) ^ G::v_swz(v_row)) + 8 * (gran & 1);
  }

  f32x16 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
  // Reference max of the scaled logits (log2 domain). It is raised only
  // when a tile brings a logit more than kRescale above it, so the weights
  // exp2(s - m_ref) stay below 2^kRescale and most tiles skip the O rescale;
  // numerator and denominator share the reference, so the result is the
  // same as with the exact running max.
  float m_run = neg_inf();
  float l_run = 0.f;        // this lane's share of the running row sum
  const float c2 = p.scale_log2;

  // scores of tile j (s_cur) and of tile j+1 (s_nxt)
  f32x16 s_cur[NB], s_nxt[NB];
  auto scores = [&](const char* stage, f32x16* acc) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[kb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const char* kp = stage + k_off[s];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        const uint4 a = *(const uint4*)(kp + kb * 32 * G::ROWB);
        acc[kb] = E::mma32(a, qf[s], acc[kb]);
      }
      // bound the K fragments held in registers (two k-steps in flight)
      if (s % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue: tiles 0..2 in flight, scores of tile 0 ----
  for (int j = 0; j < min(n_kv, kStages - 1); ++j) issue_tile(j);
  if (n_kv > 2) __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * TILE_LOADS));
  else if (n_kv > 1) __builtin_amdgcn_s_waitcnt(wait_vmcnt(TILE_LOADS));
  else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (n_kv > 0) scores(lds, s_cur);

  // One pipeline step: the softmax and P.V of tile j, plus the scores of
  // tile j+1. The score MFMAs of tile j+1 and the softmax of tile j are
  // independent; they are laid out as KS chunks, each "read the next K
  // fragments, two MFMAs, a slice of the softmax", fenced so the compiler
  // keeps that order: the matrix core works on the MFMAs while the vector
  // ALUs work on the softmax slice.
  auto step = [&](int j, f32x16* s_cur, f32x16* s_nxt) {
    const char* st_cur = lds + (j % kStages) * STAGE;
    const char* st_nxt = lds + ((j + 1) % kStages) * STAGE;
    // tile j+1 has landed for every wave, and every wave is done with the
    // stage that tile j+3 goes to (it held tile j-1)
    if (j + 2 < n_kv) __builtin_amdgcn_s_waitcnt(wait_vmcnt(TILE_LOADS));
    else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (j + 3 < n_kv) issue_tile(j + 3);

    // ---- mask keys past the sequence end / above the diagonal ----
    const bool need_mask = (j * kBN + kBN > Lk) || (CAUSAL && (j * kBN + kBN - 1 > wrow0 + delta));
    if (need_mask) {
      const int lim = CAUSAL ? min(Lk - 1, my_row + delta) : Lk - 1;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * kBN + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key > lim) s_cur[kb][r] = neg_inf();
        }
    }

    // ---- S_{j+1} = K_{j+1} Q^T  ||  online softmax of tile j ----
    // (past the last tile the next stage holds stale data; those scores are
    // never used)
    constexpr int MAXC = KS / 2;       // chunks that reduce the row max
    constexpr int EXPC = KS - MAXC;    // chunks that exponentiate
    constexpr int GROUPS = 2 * NB;     // groups of 8 probabilities
    constexpr int PER_MAX = 16 * NB / MAXC;
    constexpr int PER_EXP = GROUPS / EXPC;
    static_assert(PER_EXP >= 1 && GROUPS % EXPC == 0 && (16 * NB) % MAXC == 0, "chunking");
    uint4 kfr[2][NB];
    uint4 pf[NB][2];
    float mx = neg_inf(), rs = 0.f, alpha = 1.f, base = 0.f;
    bool raise = false;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s_nxt[kb][r] = 0.f;
      kfr[0][kb] = *(const uint4*)(st_nxt + k_off[0] + kb * 32 * G::ROWB);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 1 < KS) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
          kfr[(s + 1) & 1][kb] = *(const uint4*)(st_nxt + k_off[s + 1] + kb * 32 * G::ROWB);
      }
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) s_nxt[kb] = E::mma32(kfr[s & 1][kb], qf[s], s_nxt[kb]);
      if (s < MAXC) {
#pragma unroll
        for (int i = s * PER_MAX; i < (s + 1) * PER_MAX; ++i) mx = fmaxf(mx, s_cur[i / 16][i % 16]);
        if (s == MAXC - 1) mx = fmaxf(mx, xor_lane(mx, 32));
        pin(mx);
      } else {
        if (s == MAXC) {
          const float mx2 = mx * c2;  // -inf when the row sees no key of this tile
          raise = mx2 > m_run + kRescale;
          alpha = fast_exp2(raise ? m_run - mx2 : 0.f);  // exp2(0) = 1
          m_run = raise ? mx2 : m_run;
          base = (m_run == neg_inf()) ? 0.f : m_run;
        }
#pragma unroll
        for (int gi = (s - MAXC) * PER_EXP; gi < (s - MAXC + 1) * PER_EXP; ++gi) {
          const int kb = gi / 2, u = gi % 2;
          float e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            e[i] = fast_exp2(fmaf(s_cur[kb][8 * u + i], c2, -base));
            rs += e[i];
          }
          pf[kb][u] = make_uint4(E::pack2(e[0], e[1]), E::pack2(e[2], e[3]),
                                 E::pack2(e[4], e[5]), E::pack2(e[6], e[7]));
          pin(pf[kb][u]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run = l_run * alpha + rs;
    if (__ballot(raise)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
    }

    // ---- O^T += V_j^T P_j^T ----
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const char* vp = st_cur + v_off[db];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const char* vq = vp + (32 * kb + 16 * u) * G::ROWB;
          const uint2 lo = lds_read_tr(vq);
          const uint2 hi = lds_read_tr(vq + 8 * G::ROWB);
          acc_o[db] = E::mma32(make_uint4(lo.x, lo.y, hi.x, hi.y), pf[kb][u], acc_o[db]);
        }
    }
  };

  for (int j = 0; j < n_kv; ++j) {
    step(j, s_cur, s_nxt);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) s_cur[kb] = s_nxt[kb];
  }

  // ---- epilogue: O = O / l, LSE = ln(sum exp) ----
  const float l_tot = l_run + xor_lane(l_run, 32);
  if (my_row < Lq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* dst = (uint16_t*)p.o + (int64_t)(q0 + my_row) * p.q_row + (int64_t)w.h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * db + 8 * gq + 4 * hh;
        uint2 val;
        val.x = E::pack2(acc_o[db][4 * gq + 0] * inv, acc_o[db][4 * gq + 1] * inv);
        val.y = E::pack2(acc_o[db][4 * gq + 2] * inv, acc_o[db][4 * gq + 3] * inv);
        *(uint2*)(dst + d0) = val;
      }
    if (hh == 0)
      p.lse[(int64_t)(q0 + my_row) * p.Hq + w.h] =
          l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : neg_inf();
  }
}

// ------------------------------------------------------------------ fp32 --
constexpr int kBM32 = 32;  // query rows per workgroup
constexpr int kBN32 = 32;  // keys per tile
constexpr int kThreads32 = 128;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads32) void fwd_f32_kernel(FwdParams p) {
  constexpr int DQ = D / 4;  // d values per lane (4 lanes per query row)
  __shared__ float4 k_lds[kBN32 * D / 4];
  __shared__ float4 v_lds[kBN32 * D / 4];

  const Work w = map_block(p.n_qtiles, p.Hq);
  int q0, Lq, k0, Lk;
  seq_bounds(p, w.b, q0, Lq, k0, Lk);
  const int row0 = w.tile * kBM32;
  if (row0 >= Lq) return;
  const int g = w.h / p.group;
  const int tid = threadIdx.x;
  const int quad = tid & 3;
  const int my_row = row0 + (tid >> 2);
  const int delta = Lk - Lq;

  int kv_end = Lk;
  if (CAUSAL) kv_end = min(Lk, row0 + kBM32 + delta);
  const int n_kv = kv_end > 0 ? (kv_end + kBN32 - 1) / kBN32 : 0;

  float q[DQ], o[DQ];
  if (my_row < Lq) {
    const float* src = (const float*)p.q + (int64_t)(q0 + my_row) * p.q_row + (int64_t)w.h * D + quad * DQ;
#pragma unroll
    for (int i = 0; i < DQ; i += 4) {
      const float4 t = *(const float4*)(src + i);
      q[i] = t.x; q[i + 1] = t.y; q[i + 2] = t.z; q[i + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < DQ; ++i) q[i] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < DQ; ++i) o[i] = 0.f;
  float m_run = neg_inf(), l_run = 0.f;
  const float c2 = p.scale_log2;
  const float* kbase = (const float*)p.k + (int64_t)k0 * p.kv_row + (int64_t)g * D;
  const float* vbase = (const float*)p.v + (int64_t)k0 * p.kv_row + (int64_t)g * D;

  for (int j = 0; j < n_kv; ++j) {
    __syncthreads();
    for (int u = tid; u < kBN32 * D / 4; u += kThreads32) {
      const int r = u / (D / 4), c = u % (D / 4);
      const int key = j * kBN32 + r;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (key < Lk) {
        kv = *(const float4*)(kbase + (int64_t)key * p.kv_row + 4 * c);
        vv = *(const float4*)(vbase + (int64_t)key * p.kv_row + 4 * c);
      }
      k_lds[u] = kv;
      v_lds[u] = vv;
    }
    __syncthreads();

    float s[kBN32];
#pragma unroll
    for (int jj = 0; jj < kBN32; ++jj) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; i += 4) {
        const float4 kk = k_lds[jj * (D / 4) + quad * (DQ / 4) + i / 4];
        part = fmaf(q[i], kk.x, part);
        part = fmaf(q[i + 1], kk.y, part);
        part = fmaf(q[i + 2], kk.z, part);
        part = fmaf(q[i + 3], kk.w, part);
      }
      part += xor_lane(part, 1);
      part += xor_lane(part, 2);
      const int key = j * kBN32 + jj;
      bool vis = key < Lk;
      if (CAUSAL) vis = vis && key <= my_row + delta;
      s[jj] = vis ? part : neg_inf();
    }
    float mx = neg_inf();
#pragma unroll
    for (int jj = 0; jj < kBN32; ++jj) mx = fmaxf(mx, s[jj]);
    const float m_new = fmaxf(m_run, mx * c2);
    const float base = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - base);
    float rs = 0.f;
#pragma unroll
    for (int jj = 0; jj < kBN32; ++jj) {
      s[jj] = fast_exp2(fmaf(s[jj], c2, -base));
      rs += s[jj];
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DQ; ++i) o[i] *= alpha;
#pragma unroll
    for (int jj = 0; jj < kBN32; ++jj) {
#pragma unroll
      for (int i = 0; i < DQ; i += 4) {
        const float4 vv = v_lds[jj * (D / 4) + quad * (DQ / 4) + i / 4];
        o[i] = fmaf(s[jj], vv.x, o[i]);
        o[i + 1] = fmaf(s[jj], vv.y, o[i + 1]);
        o[i + 2] = fmaf(s[jj], vv.z, o[i + 2]);
        o[i + 3] = fmaf(s[jj], vv.w, o[i + 3]);
      }
    }
  }

  if (my_row < Lq) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* dst = (float*)p.o + (int64_t)(q0 + my_row) * p.q_row + (int64_t)w.h * D + quad * DQ;
#pragma unroll
    for (int i = 0; i < DQ; i += 4)
      *(float4*)(dst + i) = make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
    if (quad == 0)
      p.lse[(int64_t)(q0 + my_row) * p.Hq + w.h] =
          l_run > 0.f ? (m_run + __builtin_log2f(l_run)) * kLn2 : neg_inf();
  }
}

template <typename T, int D>
hipError_t launch_mfma(const FwdParams& p, bool causal, int blocks, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, true>), dim3(blocks), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, false>), dim3(blocks), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const FwdParams& p, bool causal, int blocks, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL((fwd_f32_kernel<D, true>), dim3(blocks), dim3(kThreads32), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, false>), dim3(blocks), dim3(kThreads32), 0, st, p);
  return hipGetLastError();
}

}  // namespace

int fwd_block_rows(Dt dt) { return dt == Dt::F32 ? kBM32 : kBM; }

hipError_t launch_fwd(const FwdParams& p, Dt dt, int d, bool causal, int blocks, hipStream_t st) {
  switch (dt) {
    case Dt::Bf16:
      return d == 64 ? launch_mfma<Bf16, 64>(p, causal, blocks, st)
                     : launch_mfma<Bf16, 128>(p, causal, blocks, st);
    case Dt::F16:
      return d == 64 ? launch_mfma<F16, 64>(p, causal, blocks, st)
                     : launch_mfma<F16, 128>(p, causal, blocks, st);
    case Dt::F32:
      return d == 64 ? launch_f32<64>(p, causal, blocks, st) : launch_f32<128>(p, causal, blocks, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
