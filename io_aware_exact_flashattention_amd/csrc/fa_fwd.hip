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
//  * A workgroup owns a 256-row Q tile: 8 wavefronts x 32 query rows, two
//    per SIMD; K/V tiles of 128 keys.
//  * Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_{bf16,f16}: the Q fragment is the B operand held in
//    VGPRs for the whole loop, K rows come from LDS as the A operand. In the
//    32x32 result a lane owns one query (lane % 32) and 16 of the 32 keys, so
//    a row max / row sum is a per-lane reduction plus one exchange with
//    lane ^ 32 (v_permlane32_swap) - no LDS traffic for the softmax, no
//    atomics.
//  * The same lane layout is exactly the B operand of O^T += V^T P^T, so the
//    probabilities go from the score registers to the second MFMA after a
//    round-to-nearest conversion to 16 bits, without leaving the lane. The
//    V^T operand is read from the row-major V tile with ds_read_b64_tr_b16.
//  * K and V tiles reach LDS by direct-to-LDS global loads (no register
//    round trip) into two 2-slot rings, issued at least two phases before
//    they are first read.
//    A tile whose rows all lie inside the sequence is addressed from a
//    wave-uniform base plus a 32-bit lane offset. LDS rows are XOR-swizzled
//    in 16-byte chunks so that the rows read by one MFMA operand fall in
//    distinct banks.
//  * The two waves of a SIMD run in counter-phase: while one multiplies
//    (P.V of tile j and the scores of tile j+1: MFMAs and LDS reads only),
//    the other computes the softmax of its tile (vector ALUs only), and a
//    workgroup barrier separates the phases. The matrix core and the vector
//    ALUs of the SIMD are then busy at the same time.
//  * The running max is a reference raised only when a tile exceeds it by
//    more than 2^8 (weights stay below 2^8 in fp32), so most tiles skip the
//    rescale of the output accumulator; numerator and denominator share the
//    reference, so the result equals the exact running-max recurrence.
//  * Workgroup ids are remapped (workgroups are dealt out round-robin over
//    the 8 XCDs): the groups of query heads that share a K/V head go
//    round-robin over the XCDs, keeping that K/V in one XCD's L2, and each
//    XCD runs its query tiles longest (last, under a causal mask) first.
//  * Causal: K/V tiles that no row of the Q tile may see are never loaded;
//    only tiles that cross the diagonal or the sequence end are masked. A
//    wave skips the computation of the tiles that none of its own rows may
//    see (and a wave whose rows all lie past the sequence end computes
//    nothing), passing only their barriers.
//
// fp32 inputs take fwd_f32_kernel: the same fused pass on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32), fp32 throughout, with the key range of a
// 32-row tile shared by four wavefronts and merged.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBM = 256;      // query rows per workgroup, 16-bit path (8 waves x 32)
constexpr int kBN = 128;      // keys per K/V tile, 16-bit path
constexpr int kThreads = 512;
constexpr int kKStages = 2;   // LDS ring of K tiles
constexpr int kVStages = 2;   // LDS ring of V tiles
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maximum.
constexpr int kWaitVmcnt0 = 0x0F70;
// Rescale threshold of the running max (log2 units): weights stay <= 2^8.
constexpr float kRescale = 8.f;

struct Work {
  int b, h, tile;
};

// Workgroup -> (sequence, query head, query tile). Consecutive workgroups
// land on different XCDs, so the linear id is first regrouped so that XCD x
// owns the contiguous logical range [x*per, (x+1)*per) of the work list.
// When that range is made of whole (sequence, head) units:
//  * the groups of query heads that share a K/V head are dealt round-robin
//    over the XCDs (a group stays on one XCD and in its L2; every XCD gets
//    a share of every sequence of a ragged batch);
//  * each XCD takes its units tile-major: the last query tile of each
//    head first (the longest under a causal mask), then the one before,
//    and so on, which is longest-first list scheduling over its CUs.
__device__ __forceinline__ Work map_block(int n_qtiles, int Hq, int group) {
  const int L = blockIdx.x;
  const int total = gridDim.x;
  const int xcd = L & 7, idx = L >> 3;
  const int per = total >> 3, rem = total & 7;
  if (rem == 0 && per % n_qtiles == 0) {
    const int hpx = per / n_qtiles;  // (sequence, head) units per XCD
    const int j = idx % hpx;         // unit slot of this XCD
    const int hb = (hpx % group == 0) ? ((j / group) * 8 + xcd) * group + j % group
                                      : xcd * hpx + j;
    Work w;
    w.tile = n_qtiles - 1 - idx / hpx;
    w.h = hb % Hq;
    w.b = hb / Hq;
    return w;
  }
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
  if (p.seq_lens) {  // paged K/V: keys are addressed through the page table
    q0 = p.cu_q[b];
    Lq = p.cu_q[b + 1] - q0;
    k0 = 0;
    Lk = p.seq_lens[b];
  } else if (p.cu_q) {
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
typedef __attribute__((address_space(3))) const char lds_cchar;
__device__ __forceinline__ uint2 lds_read_tr(lds_cchar* lds_byte_ptr) {
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
__device__ __forceinline__ void pin16(f32x16& x) { asm volatile("" : "+v"(x)); }


template <typename T, int D, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(kThreads) void fwd_mfma_kernel(FwdParams p) {
  using E = Elem<T>;
  using G = TileGeom<D>;
  constexpr int KS = D / 16;        // MFMA k-steps of Q K^T (= chunks of a step)
  constexpr int DB = D / 32;        // 32-row blocks of O^T
  constexpr int NB = kBN / 32;      // 32-key blocks per tile
  constexpr int LD = G::LOADS;      // 16-byte loads per lane per K (or V) tile
  constexpr int PV_N = DB * NB * 2; // P.V MFMAs per tile
  static_assert(PV_N == KS * NB && PV_N % 2 == 0, "as many P.V as score MFMAs per tile");

  // K ring (kKStages tiles), then V ring (kVStages tiles); the load
  // schedule is laid out with the barriers of the main loop.
  __shared__ __attribute__((aligned(16))) char lds[(kKStages + kVStages) * G::BYTES];
  // paged K/V: the sequence's page-table row
  __shared__ int32_t pt_lds[PAGED ? kFwdPagedMaxPages : 1];

  const Work w = map_block(p.n_qtiles, p.Hq, p.group);
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
  // Key tiles that some row of this wave can see: none when every row lies
  // past the sequence end, and under the causal mask none past the wave's
  // last row. The later tiles of the workgroup add exactly nothing to this
  // wave's rows (weights 0, running max unchanged), so the wave skips their
  // softmax and products and only passes their barriers (with its share of
  // the tile loads).
  int kv_end_w = wrow0 < Lq ? Lk : 0;
  if (CAUSAL) kv_end_w = min(kv_end_w, wrow0 + 32 + delta);
  const int n_kv_w =
      __builtin_amdgcn_readfirstlane(kv_end_w > 0 ? (kv_end_w + kBN - 1) / kBN : 0);

  if (n_kv == 0) {  // no row of the tile sees a key: O = 0, LSE = -inf
    if (my_row < Lq) {
      uint16_t* dst = (uint16_t*)p.o + (int64_t)(q0 + my_row) * p.q_row + (int64_t)w.h * D;
#pragma unroll
      for (int c = hh; c < D / 8; c += 2) *(uint4*)(dst + 8 * c) = make_uint4(0, 0, 0, 0);
      if (hh == 0) p.lse[(int64_t)(q0 + my_row) * p.Hq + w.h] = neg_inf();
    }
    return;
  }

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
  // the swizzle is applied on the source side: tile row ld_row(n), source
  // element column ld_col(n).
  auto ld_row = [&](int n) { return (n * kThreads + tid) * 16 / G::ROWB; };
  auto ld_col = [&](int n, bool k_side) {
    const int pos = (n * kThreads + tid) * 16;
    const int r = pos / G::ROWB, pc = (pos % G::ROWB) / 16;
    return 8 * (pc ^ (k_side ? G::k_swz(r) : G::v_swz(r)));
  };
  // The same loads as byte offsets from the tile's first row, for tiles
  // whose rows all lie inside the sequence (every tile but a ragged last
  // one): the tile base is then wave-uniform and the per-lane address
  // needs no 64-bit arithmetic. Needs kv_row * kBN * 2 bytes < 2^31.
  const bool uniform_rows = !PAGED && p.kv_row < (1 << 30) / kBN;
  uint32_t k_voff[LD], v_voff[LD];
#pragma unroll
  for (int n = 0; n < LD; ++n) {
    k_voff[n] = 2u * (uint32_t)(ld_row(n) * p.kv_row + ld_col(n, true));
    v_voff[n] = 2u * (uint32_t)(ld_row(n) * p.kv_row + ld_col(n, false));
  }
  const uint16_t* kbase = (const uint16_t*)p.k + (int64_t)k0 * p.kv_row + (int64_t)g * D;
  const uint16_t* vbase = (const uint16_t*)p.v + (int64_t)k0 * p.kv_row + (int64_t)g * D;
  const int last_key = Lk - 1;
  const uint32_t lds0 = lds_address(lds);
  const uint32_t lds_wave = lds0 + wave * 64 * 16;
  if (PAGED) {
    // Stage the page indices of every key this tile may see (plain loads,
    // completed here, before any direct-to-LDS load is counted).
    const int32_t* pt = p.page_table + (int64_t)w.b * p.max_pages;
    const int n_pg = (kv_end + 15) >> 4;
    for (int i = tid; i < n_pg; i += kThreads) pt_lds[i] = pt[i];
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }
  // Pool row of key `key`, clamped to the last key the tile may see (rows
  // past it repeat that row: finite values that the mask gives weight
  // zero). With paged K/V only the pages of keys below kv_end are staged.
  auto key_row = [&](int key) -> int64_t {
    if (PAGED) {
      key = min(key, kv_end - 1);
      return (int64_t)pt_lds[key >> 4] * 16 + (key & 15);
    }
    return min(key, last_key);
  };

  // Both paths issue LD loads per lane, so the wait counts below do not
  // depend on which one a tile takes.
  auto issue_k = [&](int j) {
    const uint32_t st = lds_wave + (j % kKStages) * G::BYTES;
    if (uniform_rows && (j + 1) * kBN <= Lk) {
      const uint16_t* tb = kbase + (int64_t)j * kBN * p.kv_row;
#pragma unroll
      for (int n = 0; n < LD; ++n) load_to_lds_sv(tb, k_voff[n], st + n * kThreads * 16);
    } else {
#pragma unroll
      for (int n = 0; n < LD; ++n)
        load_to_lds(kbase + key_row(j * kBN + ld_row(n)) * p.kv_row + ld_col(n, true),
                    st + n * kThreads * 16);
    }
  };
  auto issue_v = [&](int j) {
    const uint32_t st = lds_wave + (kKStages + j % kVStages) * G::BYTES;
    if (uniform_rows && (j + 1) * kBN <= Lk) {
      const uint16_t* tb = vbase + (int64_t)j * kBN * p.kv_row;
#pragma unroll
      for (int n = 0; n < LD; ++n) load_to_lds_sv(tb, v_voff[n], st + n * kThreads * 16);
    } else {
#pragma unroll
      for (int n = 0; n < LD; ++n)
        load_to_lds(vbase + key_row(j * kBN + ld_row(n)) * p.kv_row + ld_col(n, false),
                    st + n * kThreads * 16);
    }
  };
  // Slot byte offsets inside the LDS array (K ring, then V ring). Passed
  // through readfirstlane so that loop strength reduction does not turn
  // every fragment address into an induction variable of its own.
  auto k_stage = [&](int j) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((j % kKStages) * G::BYTES);
  };
  auto v_stage = [&](int j) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((kKStages + j % kVStages) * G::BYTES);
  };
  lds_cchar* const L = (lds_cchar*)lds;

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
    v_off[db] = v_row * G::ROWB + 16 * ((gran >> 1) ^ G::v_swz(v_row)) + 8 * (gran & 1);
  }
  // P.V MFMA m of a tile (m = 0 .. PV_N-1): probabilities block (kb, u) =
  // m / DB (outer, so each P fragment dies after its DB MFMAs), d-block m % DB.
  auto v_frag = [&](uint32_t vst, int m) {
    const int pidx = m / DB, db = m % DB;
    lds_cchar* vq = L + (vst + v_off[db]) + (32 * (pidx / 2) + 16 * (pidx % 2)) * G::ROWB;
    const uint2 lo = lds_read_tr(vq);
    const uint2 hi = lds_read_tr(vq + 8 * G::ROWB);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };
  auto k_frag = [&](uint32_t kst, int st, int kb) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(L + (kst + k_off[st]) + kb * 32 * G::ROWB);
    return __builtin_bit_cast(uint4, v);
  };

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

  // ---- two groups of waves in counter-phase ----
  // Waves 0-3 (group 0) and 4-7 (group 1) sit one per SIMD, so every SIMD
  // holds one wave of each group. A wave alternates a softmax phase (vector
  // ALUs only: probabilities of tile j) and a matrix phase (P.V of tile j
  // and the scores of tile j+1: MFMAs and LDS reads only). Group 1 runs one
  // phase behind group 0, and every phase boundary is a workgroup barrier,
  // so on each SIMD one wave keeps the matrix core busy while the other
  // computes its softmax.
  //   slot 2j:   group 0 softmax(j),  group 1 matrix(j-1) (scores of tile 0 for j = 0)
  //   slot 2j+1: group 0 matrix(j),   group 1 softmax(j)
  // Loads: the barrier opening slot 2j issues V tile j+1; the one opening
  // slot 2j+1 waits for K tile j+1 and V tile j and issues K tile j+2, so
  // each slot carries half of the load issue.
  const int grp = wave >> 2;
  f32x16 sc[NB];   // scores of the tile being worked on
  uint4 pf[NB][2]; // its probabilities, B operand of O^T += V^T P^T

  // Matrix phase: P.V of tile j and the scores of tile j+1, as KS groups
  // of "two P.V MFMAs + one k-step (NB MFMAs) of the scores". The LDS
  // fragments of group g+1 are read while group g multiplies (two register
  // buffers); fences keep the compiler from hoisting more reads than that.
  // (After the last tile the "next scores" come from a stale slot and are
  // never used.)
  auto matrix = [&](int j) {
    const uint32_t vst = v_stage(j);
    const uint32_t kst = k_stage(j + 1);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
    // group g: P.V MFMAs m = 2g, 2g+1 and score MFMAs s = 2g, 2g+1 (k-step
    // s / NB of 32-key block s % NB)
    uint4 vf[2][2], kf[2][2];
    auto load_group = [&](int g, int buf) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        vf[buf][h] = v_frag(vst, 2 * g + h);
        kf[buf][h] = k_frag(kst, (2 * g + h) / NB, (2 * g + h) % NB);
      }
    };
    __builtin_amdgcn_s_setprio(1);
    load_group(0, 0);
#pragma unroll
    for (int g = 0; g < PV_N / 2; ++g) {
      if (g + 1 < PV_N / 2) load_group(g + 1, (g + 1) & 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = 2 * g + h, pidx = m / DB;
        acc_o[m % DB] = E::mma32(vf[g & 1][h], pf[pidx / 2][pidx % 2], acc_o[m % DB]);
        sc[m % NB] = E::mma32(kf[g & 1][h], qf[m / NB], sc[m % NB]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // results complete before the barrier that ends the phase
#pragma unroll
    for (int db = 0; db < DB; ++db) pin16(acc_o[db]);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) pin16(sc[kb]);
  };

  auto softmax = [&](int j) {
    const bool need_mask = (j * kBN + kBN > Lk) || (CAUSAL && (j * kBN + kBN - 1 > wrow0 + delta));
    if (need_mask) {
      // key of register r of block kb: j*kBN + 4hh + (32kb + 8(r/4) + r%4);
      // compare the constant part against one per-lane threshold
      const int lim = CAUSAL ? min(Lk - 1, my_row + delta) : Lk - 1;
      const int t = lim - j * kBN - 4 * hh;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + (r & 3) > t) sc[kb][r] = neg_inf();
    }
    // row max: one chain per score block, then across the lane halves
    float mk[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      mk[kb] = sc[kb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mk[kb] = fmaxf(mk[kb], sc[kb][r]);
    }
    float mx = mk[0];
#pragma unroll
    for (int kb = 1; kb < NB; ++kb) mx = fmaxf(mx, mk[kb]);
    mx = max_halves(mx);
    const float mx2 = mx * c2;  // -inf when the row sees no key of this tile
    const bool raise = mx2 > m_run + kRescale;
    const float alpha = fast_exp2(raise ? m_run - mx2 : 0.f);  // exp2(0) = 1
    m_run = raise ? mx2 : m_run;
    const float base = (m_run == neg_inf()) ? 0.f : m_run;
    if (__ballot(raise)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
    }
    // row sum (fp32, before rounding): four independent partial sums
    float rs4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e[i] = fast_exp2(fmaf(sc[kb][8 * u + i], c2, -base));
          rs4[i & 3] += e[i];
        }
        pf[kb][u] = make_uint4(E::pack2(e[0], e[1]), E::pack2(e[2], e[3]),
                               E::pack2(e[4], e[5]), E::pack2(e[6], e[7]));
      }
    l_run = l_run * alpha + ((rs4[0] + rs4[1]) + (rs4[2] + rs4[3]));
    // probabilities complete before the barrier that ends the phase (the
    // compiler may not sink this arithmetic into the matrix phase)
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      pin(pf[kb][0]);
      pin(pf[kb][1]);
    }
    pin(l_run);
  };

  auto scores0 = [&]() {
    if (n_kv_w == 0) return;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) sc[kb] = E::mma32(k_frag(k_stage(0), st, kb), qf[st], sc[kb]);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) pin16(sc[kb]);
  };

  // ---- prologue: K tiles 0, 1 and V tile 0 ----
  issue_k(0);
  if (n_kv > 1) issue_k(1);
  issue_v(0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (grp == 0) scores0();

  // Barrier k opens slot k. The prologue issued K tiles 0, 1 and V tile 0;
  // barrier 2m+1 issues K tile m+2 and V tile m+1. Slot 2m+1 (group 0's
  // matrix phase of tile m) and slot 2m+2 (group 1's) read V tile m and K
  // tile m+1, which barrier 2m+1 awaits; even barriers issue nothing.
  auto barrier = [&](int k) {
    const int m = k >> 1;
    // Barrier 2m+1 waits for everything in flight (K tile m+1 and V tile m,
    // issued at barrier 2m-1) and issues K tile m+2 and V tile m+1 into the
    // slots of K tile m and V tile m-1, both last read in slot 2m.
    if ((k & 1) == 0) {
      __syncthreads();
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      if (m + 2 < n_kv) issue_k(m + 2);
      if (m + 1 < n_kv) issue_v(m + 1);
    }
  };
  // Each group runs its own loop; both pass barriers 0 .. 2 n_kv in order.
  // A wave works on tiles 0 .. n_kv_w - 1 and only passes the barriers of
  // the rest.
  if (grp == 0) {
    barrier(0);
    for (int j = 0; j < n_kv_w; ++j) {
      softmax(j);     // slot 2j
      barrier(2 * j + 1);
      matrix(j);      // slot 2j+1
      barrier(2 * j + 2);
    }
  } else {
    barrier(0);
    scores0();        // slot 0
    for (int j = 0; j < n_kv_w; ++j) {
      barrier(2 * j + 1);
      softmax(j);     // slot 2j+1
      barrier(2 * j + 2);
      matrix(j);      // slot 2j+2
    }
  }
  for (int j = n_kv_w; j < n_kv; ++j) {
    barrier(2 * j + 1);
    barrier(2 * j + 2);
  }

  // ---- epilogue: O = O / l, LSE = ln(sum exp) ----
  const float l_tot = sum_halves(l_run);
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
// key splits of a workgroup, one wavefront each: eight at d = 64 (128 KB
// of tiles), four at d = 128 (the same LDS)
template <int D> constexpr int waves32() { return D == 64 ? 8 : 4; }

// fp32 path: both products on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32: A and B one float per lane, 32x32 fp32 result).
// A workgroup owns 32 query rows; wavefront w of its W takes K/V tiles w,
// w+W, ... of the rows' key range, runs the online softmax over them with
// the exact running max, and the W (m, l, O) states are merged at the end
// in a fixed order (the log-sum-exp algebra of the split merge of the
// decode).
//  * S^T = K Q^T as in the 16-bit kernel, a lane owning query l % 32. The
//    contraction over d is taken in a permuted order so that one
//    ds_read_b128 of a K row gives the A operands of four MFMA steps: step
//    4u + i, lane half h reads d = 8u + 4h + i. The Q fragment (B) follows
//    the same order and stays in registers.
//  * O^T += V^T P^T: step s covers keys 8(s/4) + 4h + s%4 for lane half h,
//    the keys of result register s of the score block, so the B operand of
//    step s is the lane's own probability register s (no exchange, no
//    rounding). V^T comes from the row-major V tile one float per lane.
//  * LDS tiles (per wavefront): K rows with their 16-byte chunks XOR-permuted
//    by the row (the 16 rows read at one chunk position hit distinct banks);
//    V rows with their 32-float blocks swapped on every other group of four
//    rows, so the two lane halves of a V^T read (rows four apart) use
//    disjoint bank halves.
__device__ __forceinline__ f32x16 mma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * waves32<D>()) void fwd_f32_kernel(FwdParams p) {
  constexpr int W = waves32<D>();
  constexpr int CH = D / 4;     // 16-byte chunks per row
  constexpr int KU = D / 8;     // K reads per tile (four MFMA steps each)
  constexpr int DB = D / 32;    // 32-row blocks of O^T
  constexpr int TILE4 = kBN32 * CH;  // float4 per tile
  constexpr int RED = 16 * DB + 2;   // floats per lane in the merge: m, l, O
  static_assert(64 * W * RED <= W * 2 * TILE4 * 4, "merge fits in the tile buffers");
  __shared__ float4 tiles[W][2][TILE4];  // per wavefront: K tile, V tile

  const Work w = map_block(p.n_qtiles, p.Hq, p.group);
  int q0, Lq, k0, Lk;
  seq_bounds(p, w.b, q0, Lq, k0, Lk);
  const int row0 = w.tile * kBM32;
  if (row0 >= Lq) return;
  const int g = w.h / p.group;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int my_row = row0 + l32;
  const int delta = Lk - Lq;

  int kv_end = Lk;
  if (CAUSAL) kv_end = min(Lk, row0 + kBM32 + delta);
  const int n_kv = kv_end > 0 ? (kv_end + kBN32 - 1) / kBN32 : 0;

  // Q fragment: qf[u] = Q[my_row][8u + 4hh .. +3]
  float4 qf[KU];
  if (my_row < Lq) {
    const float* src = (const float*)p.q + (int64_t)(q0 + my_row) * p.q_row + (int64_t)w.h * D + 4 * hh;
#pragma unroll
    for (int u = 0; u < KU; ++u) qf[u] = *(const float4*)(src + 8 * u);
  } else {
#pragma unroll
    for (int u = 0; u < KU; ++u) qf[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  f32x16 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
  float m_run = neg_inf(), l_run = 0.f;  // log2 domain; l_run: this lane's keys
  const float c2 = p.scale_log2;
  const float* kbase = (const float*)p.k + (int64_t)k0 * p.kv_row + (int64_t)g * D;
  const float* vbase = (const float*)p.v + (int64_t)k0 * p.kv_row + (int64_t)g * D;
  float4* kt = tiles[wave][0];
  float4* vt = tiles[wave][1];
  const float* vtf = (const float*)vt;

  const int n_iter = (n_kv + W - 1) / W;
  for (int it = 0; it < n_iter; ++it) {
    const int j = it * W + wave;  // this wavefront's tile
    const bool have = j < n_kv;          // uniform over the wavefront
    __syncthreads();
    if (have) {
      // rows past the sequence end load as zeros (their V must stay finite)
#pragma unroll
      for (int n = 0; n < TILE4 / 64; ++n) {
        const int u = n * 64 + lane;
        const int r = u / CH, c = u % CH;
        const int key = j * kBN32 + r;
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        if (key < Lk) {
          kv = *(const float4*)(kbase + (int64_t)key * p.kv_row + 4 * c);
          vv = *(const float4*)(vbase + (int64_t)key * p.kv_row + 4 * c);
        }
        kt[r * CH + (c ^ (r & 15))] = kv;
        vt[r * CH + (c ^ (8 * ((r >> 2) & 1)))] = vv;
      }
    }
    __syncthreads();
    if (!have) continue;

    // ---- S^T = K Q^T ----
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const float4 kf = kt[l32 * CH + ((2 * u + hh) ^ (l32 & 15))];
      sc = mma_f32(kf.x, qf[u].x, sc);
      sc = mma_f32(kf.y, qf[u].y, sc);
      sc = mma_f32(kf.z, qf[u].z, sc);
      sc = mma_f32(kf.w, qf[u].w, sc);
    }
    // ---- mask, online softmax (exact running max) ----
    // register r holds key j*32 + 8(r/4) + 4hh + r%4
    const int lim = CAUSAL ? min(Lk - 1, my_row + delta) : Lk - 1;
    const int thr = lim - j * kBN32 - 4 * hh;
    float mx = neg_inf();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (8 * (r >> 2) + (r & 3) > thr) sc[r] = neg_inf();
      mx = fmaxf(mx, sc[r]);
    }
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx * c2);
    const float base = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - base);
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[r] = fast_exp2(fmaf(sc[r], c2, -base));
      rs += sc[r];
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int key = 8 * (st >> 2) + 4 * hh + (st & 3);  // (key >> 2) & 1 == hh
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc_o[db] = mma_f32(vtf[key * D + 32 * (db ^ hh) + l32], sc[st], acc_o[db]);
    }
  }

  // ---- merge the wavefronts (fixed order), then O = O / l, LSE ----
  l_run = sum_halves(l_run);
  float* red = (float*)&tiles[0][0][0];
  __syncthreads();  // every wavefront is done with its tiles
  {
    float* mine = red + (int64_t)tid * RED;
    mine[0] = m_run;
    mine[1] = l_run;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) mine[2 + 16 * db + r] = acc_o[db][r];
  }
  __syncthreads();
  if (wave != 0) return;
  float M = neg_inf();
#pragma unroll
  for (int wv = 0; wv < W; ++wv) M = fmaxf(M, red[(wv * 64 + lane) * RED]);
  float l_tot = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
  if (M != neg_inf()) {
#pragma unroll
    for (int wv = 0; wv < W; ++wv) {
      const float* st = red + (wv * 64 + lane) * RED;
      const float ws = st[0] == neg_inf() ? 0.f : fast_exp2(st[0] - M);
      l_tot = fmaf(st[1], ws, l_tot);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] = fmaf(st[2 + 16 * db + r], ws, acc_o[db][r]);
    }
  }
  if (my_row < Lq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* dst = (float*)p.o + (int64_t)(q0 + my_row) * p.q_row + (int64_t)w.h * D;
    // register r of block db holds d = 32 db + 8(r/4) + 4hh + r%4
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        *(float4*)(dst + 32 * db + 8 * gq + 4 * hh) =
            make_float4(acc_o[db][4 * gq] * inv, acc_o[db][4 * gq + 1] * inv,
                        acc_o[db][4 * gq + 2] * inv, acc_o[db][4 * gq + 3] * inv);
    if (hh == 0)
      p.lse[(int64_t)(q0 + my_row) * p.Hq + w.h] =
          l_tot > 0.f ? (M + __builtin_log2f(l_tot)) * kLn2 : neg_inf();
  }
}

template <typename T, int D, bool PAGED = false>
hipError_t launch_mfma(const FwdParams& p, bool causal, int blocks, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, true, PAGED>), dim3(blocks), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, false, PAGED>), dim3(blocks), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const FwdParams& p, bool causal, int blocks, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL((fwd_f32_kernel<D, true>), dim3(blocks), dim3(64 * waves32<D>()), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, false>), dim3(blocks), dim3(64 * waves32<D>()), 0, st, p);
  return hipGetLastError();
}

}  // namespace

int fwd_block_rows(Dt dt) { return dt == Dt::F32 ? kBM32 : kBM; }

hipError_t launch_fwd_paged(const FwdParams& p, Dt dt, int d, bool causal, int blocks,
                            hipStream_t st) {
  switch (dt) {
    case Dt::Bf16:
      return d == 64 ? launch_mfma<Bf16, 64, true>(p, causal, blocks, st)
                     : launch_mfma<Bf16, 128, true>(p, causal, blocks, st);
    case Dt::F16:
      return d == 64 ? launch_mfma<F16, 64, true>(p, causal, blocks, st)
                     : launch_mfma<F16, 128, true>(p, causal, blocks, st);
    default:
      return hipErrorInvalidValue;
  }
}

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
