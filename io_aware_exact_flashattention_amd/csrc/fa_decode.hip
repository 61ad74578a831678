// fa_decode.hip - split-KV decode over a paged K/V cache, gfx950.
//
// The serving variant of the page "I/O-Aware Kernels" (datasystem.school,
// Module 5), section "FlashInfer: I/O-aware attention for serving": the
// fused kernel with keys and values gathered from a paged cache through a
// page table, for a batch of sequences of different lengths and
// grouped-query heads. One query token per sequence.
//
// Decode reads every K/V byte once and does ~4 flops per byte, so it is
// bound by HBM bandwidth; the design goal is many independent 16-byte loads
// in flight and little arithmetic per byte:
//  * Work item = (sequence, KV head, split). A split is a run of
//    `pages_per_split` pages; the GB query heads that share the KV head are
//    handled together, so each K/V byte is read once for all of them.
//  * One wavefront per item; the next page's K/V loads are issued before the
//    current page is consumed.
//  * Scores of a page on the matrix cores (v_mfma_f32_16x16x32, K rows as
//    the A operand, the GB query vectors as columns of B).
//  * The online softmax of section "FlashAttention: tiling + online
//    softmax": a running max per head (wave-uniform), a running sum and a
//    rescaled output accumulator. The accumulator is rescaled only when a
//    page max exceeds the running max by more than 2^8; between rescales the
//    weights stay <= 2^8 in fp32 and the same reference enters numerator and
//    denominator, so the result is unchanged.
//  * P.V on the vector ALUs: each lane owns a 16-byte slice of the head
//    dimension for a few tokens of the page, so V is read in its natural
//    row layout with coalesced 16-byte loads. The shared-prefix pass of a
//    cascade decode (32 query columns) does P.V on the matrix cores.
//  * A second kernel merges the splits of each (sequence, query head):
//    lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s, in fixed
//    split order (deterministic).
// Slots of a last page beyond the sequence end never enter the result:
// their scores are -inf and their V values are replaced by zero before use,
// so NaN garbage there cannot leak.
#include <mutex>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kPage = 16;
constexpr float kRescaleThreshold = 8.f;  // log2 units

// Chunk permutation of K row t in a staging slot (VCH 16-byte chunks per
// row), XOR-ed onto the chunk index: 16 consecutive rows read at one logical
// chunk land on 16 distinct 16-byte bank groups. The score operand read
// (ds_read_b128: lane l reads row l%16 at logical chunk c0 + (l/16) *
// (VCH/4)) is free of bank conflicts on gfx950 only when the chunk bit that
// the lane group l/16 steps through is XOR-ed with a low row bit (row bit 0
// or 1 at 256-byte rows; bit 1 at 128-byte rows, where bit 0 picks the bank
// half): the plain t & 15 (or (t >> 1) & 7) costs four conflict cycles per
// read, measured with SQ_LDS_BANK_CONFLICT. Hence row bits 1 and 2 trade
// places (d = 128), and bits 1 and 2 of t >> 1 do (d = 64).
template <int VCH> __device__ __forceinline__ int kswz(int t) {
  return VCH == 16 ? ((t & 9) | ((t & 2) << 1) | ((t & 4) >> 1))
                   : ((((t >> 3) & 1) << 2) | (t & 2) | ((t >> 2) & 1));
}

template <typename T> struct Mma16;
template <> struct Mma16<Bf16> {
  // D(16x16, f32) += A(16x32) * B(32x16); 8 bf16 per lane per operand.
  __device__ static __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma16<F16> {
  __device__ static __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// O^T(16 d x 16 queries) += V^T(16 d x 16 tokens) * P^T(16 tokens x 16
// queries); 4 16-bit values per lane per operand.
template <typename T> struct Mma16k16;
template <> struct Mma16k16<Bf16> {
  __device__ static __forceinline__ f32x4 mma(uint2 a, uint2 b, f32x4 c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
};
template <> struct Mma16k16<F16> {
  __device__ static __forceinline__ f32x4 mma(uint2 a, uint2 b, f32x4 c) {
    typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h16x4, a),
                                                 __builtin_bit_cast(h16x4, b), c, 0, 0, 0);
  }
};

typedef short dec_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dec_s16x4 dec_lds_s16x4;
// ds_read_b64_tr_b16: inside each group of 16 lanes, lane j receives
// element j%4 of the 8 bytes addressed by lane 4e + j/4, as its element e.
__device__ __forceinline__ uint2 lds_read_tr8(const char* lds_byte_ptr) {
  const dec_s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (dec_lds_s16x4*)(const __attribute__((address_space(3))) char*)lds_byte_ptr);
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

constexpr int kWavesPerBlock = 4;
constexpr int kWaveLds = 8192;  // LDS bytes per wave: the staging ring of its pages

// Waits written as inline assembly with a memory clobber, so that the LDS
// reads of a page stay after the wait for its direct-to-LDS loads, and the
// next loads into a slot stay after the reads that empty it.
template <int N> __device__ __forceinline__ void wait_loads() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds_reads() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
// Make the compiler consider a loaded value complete here (its own wait
// count for the load is then settled before the direct-to-LDS loads start).
__device__ __forceinline__ void settle(uint4& x) {
  asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
}
__device__ __forceinline__ void settle(int& x) { asm volatile("" : "+v"(x)); }

// One wavefront per work item (sequence b, KV head g, block of GB query
// heads, split s); four independent wavefronts per workgroup.
//
// Each page of a split is copied by direct-to-LDS loads (no registers held
// while in flight) into the wave's 8 KB staging ring: one page slot for
// d = 128, two for d = 64. The next page's loads are issued as soon as the
// current page has been read out of its slot, so a page is in flight during
// the whole computation of the previous one.
//
// Scores of a 16-token page for the GB query heads of the block come from
// v_mfma_f32_16x16x32: A = the page's K rows (lane l: token l%16, an 8-value
// slice of d chosen by l/16), B = Q^T (lane l: query head l%16, zero past
// GB). In the 16x16 result lane l holds tokens 4(l/16)+i of head l%16.
// The running max of each head is wave-uniform: a page max is reduced over
// the token lanes and read back with readlane.
// P.V on the vector ALUs: lane c owns d values c*VPL .. c*VPL+VPL-1 (VPL =
// d/64) of every head of the block for all 16 tokens, so each probability
// is a wave-wide scalar (readlane) and no lane exchange is needed at the end.
// The shared-prefix pass (blocks of 16 query columns) does P.V on the matrix cores
// instead: the probabilities of lane l (tokens 4(l/16)+i of query l%16) are
// exactly its B operand of O^T += V^T P^T (v_mfma_f32_16x16x16), and V^T
// comes from the row-major V slot with ds_read_b64_tr_b16. O^T then sits
// in MFMA layout (lane l: query l%16, d = 16 db + 4(l/16) + i), so the
// running max and the rescale are per lane.
// Five waves per SIMD (five workgroups per CU) is what the LDS rings allow;
// the widest head block needs more registers and runs four, the 32-column
// prefix pass at d = 128 three.
template <int D, int GB, bool PREFIX>
constexpr int decode_waves_per_simd() {
  return PREFIX ? (D == 128 ? 3 : 4) : (D * GB > 512 ? 4 : 5);
}

// PREFIX: the shared-prefix pass of a cascade decode. A work item is then
// (block of 32 query columns, prefix split, KV head); column c of block qb is
// query r = 32 qb + c of the r-th (sequence, head-in-group) pair of the KV
// head, so the prefix pages are read once for every 32 queries of the group.
// The 32 columns are two 16-column MFMA operands that share each page's K
// and V fragments.
template <typename T, int D, int GB, bool PREFIX = false>
__global__ __launch_bounds__(64 * kWavesPerBlock)
__attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<D, GB, PREFIX>()))) void decode_split_kernel(
    DecodeParams p) {
  using E = Elem<T>;
  constexpr int KSTEP = D / 32;       // MFMA k-steps per page (K loads per page)
  constexpr int DL = D / 4;           // d values per lane group in the score MFMA
  constexpr int VCH = D / 8;          // 16-byte chunks per token row
  constexpr int TPI = 64 / VCH;       // tokens per V load instruction
  constexpr int VI = kPage / TPI;     // V loads per page
  constexpr int NLOAD = KSTEP + VI;   // direct-to-LDS loads per page
  constexpr int KBYTES = kPage * D * 2;
  constexpr int SLOT = 2 * KBYTES;
  constexpr int NSLOT = kWaveLds / SLOT;
  constexpr int VPL = D / 64;         // d values per lane in P.V
  constexpr int NCB = PREFIX ? 2 : 1; // 16-column blocks of an item (prefix pass: 32 queries)
  static_assert(GB <= 16 && VI >= 1 && (NSLOT == 1 || NSLOT == 2), "bad decode tile");
  static_assert(KSTEP * 1024 == KBYTES && VI * 1024 == KBYTES, "page layout");
  __shared__ uint4 lds[kWavesPerBlock][kWaveLds / 16];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  int item = blockIdx.x * kWavesPerBlock + wave;
  int b, g, h0, s, L, qb = 0;
  const int32_t* pt;
  if (PREFIX) {
    // work item: (query block, prefix split, KV head), KV head fastest
    g = item % p.Hkv;
    item /= p.Hkv;
    s = item % p.prefix_splits;
    qb = item / p.prefix_splits;
    if (qb * GB * NCB >= p.B * p.group) return;
    b = 0;
    h0 = 0;
    L = p.prefix_len;
    pt = p.prefix_pages;
  } else {
    // work item: (sequence, split, KV head, head block), head block fastest
    const int nhb = p.group / GB;
    const int nh = p.Hkv * nhb;
    const int nsplit = p.max_splits - p.split_offset;  // splits of this pass
    const int hb = item % nh;
    item /= nh;
    s = item % nsplit;
    b = item / nsplit;
    if (b >= p.B) return;
    g = hb / nhb;
    h0 = g * p.group + (hb % nhb) * GB;
    L = p.seq_lens[b];
    pt = p.page_table + (int64_t)b * p.max_pages;
  }
  // query row (sequence * Hq + head) of column c
  auto q_row_of = [&](int c) -> int64_t {
    if (PREFIX) {
      const int r = qb * GB * NCB + c;
      return (int64_t)(r / p.group) * p.Hq + g * p.group + r % p.group;
    }
    return (int64_t)b * p.Hq + h0 + c;
  };
  auto column_valid = [&](int c) { return !PREFIX || qb * GB * NCB + c < p.B * p.group; };
  const int npages = (L + kPage - 1) / kPage;
  const int pps = PREFIX ? p.prefix_pages_per_split : p.pages_per_split;
  const int pg0 = s * pps;
  if (pg0 >= npages) return;
  const int pg1 = min(npages, pg0 + pps);

  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, j = lane >> 4;  // score layout
  const float c2 = p.scale_log2;

  // B operands: Q^T, columns 16 cb + 0 .. 16 cb + GB-1 of column block cb
  // (zero for absent queries)
  uint4 qf[NCB][KSTEP];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int st = 0; st < KSTEP; ++st) qf[cb][st] = make_uint4(0, 0, 0, 0);
    if (l16 < GB && column_valid(16 * cb + l16)) {
      const uint16_t* src = (const uint16_t*)p.q + q_row_of(16 * cb + l16) * D + j * DL;
#pragma unroll
      for (int st = 0; st < KSTEP; ++st) qf[cb][st] = *(const uint4*)(src + 8 * st);
    }
  }
  // Page indices of the split (at most 64 pages): lane i holds entry
  // pg0 + i; each page's index is read from its lane.
  int pg_idx = pg0 + lane < pg1 ? pt[pg0 + lane] : 0;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int st = 0; st < KSTEP; ++st) settle(qf[cb][st]);
  settle(pg_idx);

  // Direct-to-LDS copies of whole token rows (each load instruction reads
  // TPI complete rows, so every cache line is requested once). In the
  // slot, K and V are row-major [token][d]; the 16-byte chunks of K row t
  // are stored XOR-permuted by kswz(t) so that the score operand reads
  // (16 tokens, one chunk each) hit distinct LDS banks.
  const int64_t tok = (int64_t)p.Hkv * D;  // elements between tokens of a page
  const int dma_t = lane / VCH, dma_c = lane % VCH;  // row and stored chunk of this lane
  const uint16_t* kdma = (const uint16_t*)p.k_pool + (int64_t)g * D + dma_t * tok;
  const uint16_t* vdma = (const uint16_t*)p.v_pool + (int64_t)g * D + dma_c * 8 + dma_t * tok;
  int kcol[KSTEP];  // K chunk fetched by this lane for load st (un-permuted)
#pragma unroll
  for (int st = 0; st < KSTEP; ++st) kcol[st] = 8 * (dma_c ^ kswz<VCH>(st * TPI + dma_t));
  const uint32_t ring = lds_address(&lds[wave][0]);
  const char* ring_ptr = (const char*)&lds[wave][0];
  auto issue_page = [&](int pg, int slot) {
    const int64_t base = (int64_t)__builtin_amdgcn_readlane(pg_idx, pg - pg0) * kPage * tok;
    const uint32_t dst = ring + slot * SLOT;
#pragma unroll
    for (int st = 0; st < KSTEP; ++st)
      stream_to_lds(kdma + base + st * TPI * tok + kcol[st], dst + st * 1024);
#pragma unroll
    for (int r = 0; r < VI; ++r) stream_to_lds(vdma + base + r * TPI * tok, dst + KBYTES + r * 1024);
  };
  // score operand: lane l reads token l16, chunk j*(DL/8) + st
  int kread[KSTEP];
#pragma unroll
  for (int st = 0; st < KSTEP; ++st)
    kread[st] = l16 * 2 * D + 16 * ((j * (DL / 8) + st) ^ kswz<VCH>(l16));

  constexpr bool MFMA_PV = PREFIX;  // P.V on the matrix cores (16 columns per block)
  static_assert(!MFMA_PV || GB == 16, "MFMA P.V takes 16 query columns");
  constexpr int DB16 = D / 16;      // 16-row blocks of O^T
  float m[MFMA_PV ? 1 : GB];        // running max per head, log2 domain (wave-uniform)
  float o[MFMA_PV ? 1 : GB][VPL];   // this lane's d values of O for each head
  f32x4 oacc[NCB][MFMA_PV ? DB16 : 1];  // O^T blocks in MFMA layout (MFMA_PV)
  float m_lane[NCB];                // running max of query 16 cb + l16 (MFMA_PV)
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) m_lane[cb] = neg_inf();
  if constexpr (MFMA_PV) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int db = 0; db < DB16; ++db) oacc[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      m[h] = neg_inf();
#pragma unroll
      for (int e = 0; e < VPL; ++e) o[h][e] = 0.f;
    }
  }
  float l_lane[NCB];    // share of the row sum of column 16 cb + l16 (tokens of this lane)
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) l_lane[cb] = 0.f;
  // V^T operand address of d-block db: lane a of 16-lane group g reads the
  // 8 bytes of row 4g + a/4 at column 16 db + 4 (a % 4)
  const int vt_off = KBYTES + (4 * j + l16 / 4) * 2 * D + 8 * (l16 & 3);

  issue_page(pg0, 0);
  if (NSLOT == 2 && pg0 + 1 < pg1) issue_page(pg0 + 1, 1);

  for (int pg = pg0; pg < pg1; ++pg) {
    const int slot = NSLOT == 2 ? ((pg - pg0) & 1) : 0;
    if (NSLOT == 2 && pg + 1 < pg1) wait_loads<NLOAD>();
    else wait_loads<0>();
    const char* sp = ring_ptr + slot * SLOT;
    uint4 kf[KSTEP];
#pragma unroll
    for (int st = 0; st < KSTEP; ++st) kf[st] = *(const uint4*)(sp + kread[st]);
    uint32_t vr[MFMA_PV ? 1 : kPage];
    uint2 vt[MFMA_PV ? DB16 : 1];
    if constexpr (MFMA_PV) {
#pragma unroll
      for (int db = 0; db < DB16; ++db) vt[db] = lds_read_tr8(sp + vt_off + 32 * db);
    } else {
#pragma unroll
      for (int t = 0; t < kPage; ++t) {
        if constexpr (VPL == 2) vr[t] = *(const uint32_t*)(sp + KBYTES + t * 2 * D + 4 * lane);
        else vr[t] = *(const uint16_t*)(sp + KBYTES + t * 2 * D + 2 * lane);
      }
    }
    wait_lds_reads();
    if (pg + NSLOT < pg1) issue_page(pg + NSLOT, slot);

    const int tok0 = pg * kPage;
    // slots past the sequence end may hold anything (NaN): zero their V
    if (tok0 + kPage > L) {
      if constexpr (MFMA_PV) {
        // element e of vt[db] is token 4j + e
#pragma unroll
        for (int db = 0; db < DB16; ++db) {
          if (tok0 + 4 * j + 0 >= L) vt[db].x &= 0xffff0000u;
          if (tok0 + 4 * j + 1 >= L) vt[db].x &= 0x0000ffffu;
          if (tok0 + 4 * j + 2 >= L) vt[db].y &= 0xffff0000u;
          if (tok0 + 4 * j + 3 >= L) vt[db].y &= 0x0000ffffu;
        }
      } else {
#pragma unroll
        for (int t = 0; t < kPage; ++t)
          if (tok0 + t >= L) vr[t] = 0u;
      }
    }

    // ---- scores S[token][column] on the matrix cores, per column block ----
    float sc[NCB][4];
    float mx[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KSTEP; ++st) acc = Mma16<T>::mma(kf[st], qf[cb][st], acc);
      mx[cb] = neg_inf();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = (l16 < GB) && (tok0 + 4 * j + i < L);
        sc[cb][i] = ok ? acc[i] * c2 : neg_inf();
        mx[cb] = fmaxf(mx[cb], sc[cb][i]);
      }
      // across the four token groups (lanes l16 + 16 j), inside the vector ALU
      {
        float a, b;
        row_pair(mx[cb], a, b);
        mx[cb] = max_halves(fmaxf(a, b));
      }
    }

    if constexpr (MFMA_PV) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        // ---- running max of query 16 cb + l16 (same in its four token lanes) ----
        const bool raise = mx[cb] > m_lane[cb] + kRescaleThreshold;
        const float alpha = fast_exp2(raise ? m_lane[cb] - mx[cb] : 0.f);  // exp2(0) = 1
        m_lane[cb] = raise ? mx[cb] : m_lane[cb];
        if (__ballot(raise)) {
#pragma unroll
          for (int db = 0; db < DB16; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) oacc[cb][db][i] *= alpha;
        }
        l_lane[cb] *= alpha;
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[i] = (sc[cb][i] == neg_inf()) ? 0.f : fast_exp2(sc[cb][i] - m_lane[cb]);
          l_lane[cb] += pr[i];
        }
        // ---- O^T += V^T P^T on the matrix cores ----
        const uint2 pb = make_uint2(E::pack2(pr[0], pr[1]), E::pack2(pr[2], pr[3]));
#pragma unroll
        for (int db = 0; db < DB16; ++db)
          oacc[cb][db] = Mma16k16<T>::mma(vt[db], pb, oacc[cb][db]);
      }
      continue;
    }

    // ---- running max per head; rescale only when it grows by > 2^8 ----
    float m_sel = m[0], a_sel = 1.f;
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      const float pm = lane_value(mx[0], h);
      if (pm > m[h] + kRescaleThreshold) {
        const float alpha = fast_exp2(m[h] - pm);
        m[h] = pm;
#pragma unroll
        for (int e = 0; e < VPL; ++e) o[h][e] *= alpha;
        if (l16 == h) a_sel = alpha;
      }
      if (l16 == h) m_sel = m[h];
    }
    l_lane[0] *= a_sel;

    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = (sc[0][i] == neg_inf()) ? 0.f : fast_exp2(sc[0][i] - m_sel);
      l_lane[0] += pr[i];
    }

    // ---- O += P V: P[t][h] sits in register t%4 of lane 16(t/4) + h ----
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      float v[VPL];
      v[0] = E::lo(vr[t]);
      if constexpr (VPL == 2) v[1] = E::hi(vr[t]);
#pragma unroll
      for (int h = 0; h < GB; ++h) {
        const float w = lane_value(pr[t & 3], 16 * (t >> 2) + h);
#pragma unroll
        for (int e = 0; e < VPL; ++e) o[h][e] = fmaf(w, v[e], o[h][e]);
      }
    }
  }

#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    float a, b;
    row_pair(l_lane[cb], a, b);
    l_lane[cb] = sum_halves(a + b);
  }
  if constexpr (MFMA_PV) {
    // lane l: query 16 cb + l16, d = 16 db + 4 j + i
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      if (!column_valid(16 * cb + l16)) continue;
      const int64_t row = q_row_of(16 * cb + l16) * p.max_splits + s;
      const float inv = l_lane[cb] > 0.f ? 1.f / l_lane[cb] : 0.f;
      float* dst = p.o_part + row * D + 4 * j;
#pragma unroll
      for (int db = 0; db < DB16; ++db)
        *(float4*)(dst + 16 * db) =
            make_float4(oacc[cb][db][0] * inv, oacc[cb][db][1] * inv, oacc[cb][db][2] * inv,
                        oacc[cb][db][3] * inv);
      if (j == 0)
        p.lse_part[row] =
            l_lane[cb] > 0.f ? (m_lane[cb] + __builtin_log2f(l_lane[cb])) * kLn2 : neg_inf();
    }
    return;
  }
#pragma unroll
  for (int h = 0; h < GB; ++h) {
    const float lt = lane_value(l_lane[0], h);
    if (!column_valid(h)) continue;
    const int64_t row = q_row_of(h) * p.max_splits + (PREFIX ? 0 : p.split_offset) + s;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float* dst = p.o_part + row * D + lane * VPL;
    if constexpr (VPL == 2) *(float2*)dst = make_float2(o[h][0] * inv, o[h][1] * inv);
    else *dst = o[h][0] * inv;
    if (lane == 0) p.lse_part[row] = lt > 0.f ? (m[h] + __builtin_log2f(lt)) * kLn2 : neg_inf();
  }
}

// Split merge for one (sequence, query head), 256 threads: thread (sg, q)
// with sg = tid / 32 in 0..7 and q = tid % 32 accumulates the d values
// q*D/32 .. of splits sg, sg+8, ...; the eight partial sums are then added
// through LDS. The max and the sum of exp over the split log-sum-exps are
// taken by every wave in parallel over lanes (64 splits per pass).
constexpr int kCombineThreads = 256;
constexpr int kCombineGroups = kCombineThreads / 32;

template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeParams p) {
  using E = Elem<T>;
  constexpr int PER = D / 32;  // d values per thread (one 8- or 16-byte load per split)
  static_assert(PER == 2 || PER == 4, "combine layout");
  __shared__ float part[kCombineGroups][D];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int sg = tid >> 5, q = tid & 31;
  const int L = p.seq_lens[b];
  const int npages = (L + kPage - 1) / kPage;
  const int ns = p.prefix_splits + (npages + p.pages_per_split - 1) / p.pages_per_split;
  const int64_t row = ((int64_t)b * p.Hq + h) * p.max_splits;
  const float* lp = p.lse_part + row;
  const float* op = p.o_part + row * D + q * PER;

  float mx = neg_inf();
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) mx = fmaxf(mx, lp[s0 + lane]);
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) mx = fmaxf(mx, xor_lane(mx, x));
  float sum = 0.f;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  if (mx != neg_inf()) {
    for (int s0 = 0; s0 < ns; s0 += 64)
      if (s0 + lane < ns) sum += fast_exp2((lp[s0 + lane] - mx) * kLog2e);
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) sum += xor_lane(sum, x);
#pragma unroll 4
    for (int s = sg; s < ns; s += kCombineGroups) {
      const float w = fast_exp2((lp[s] - mx) * kLog2e);
      if constexpr (PER == 4) {
        const float4 v = *(const float4*)(op + (int64_t)s * D);
        acc[0] = fmaf(w, v.x, acc[0]);
        acc[1] = fmaf(w, v.y, acc[1]);
        acc[2] = fmaf(w, v.z, acc[2]);
        acc[3] = fmaf(w, v.w, acc[3]);
      } else {
        const float2 v = *(const float2*)(op + (int64_t)s * D);
        acc[0] = fmaf(w, v.x, acc[0]);
        acc[1] = fmaf(w, v.y, acc[1]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) part[sg][q * PER + i] = acc[i];
  __syncthreads();
  if (tid < D / 2) {
    // thread tid finishes d values 2 tid, 2 tid + 1 in fixed group order
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int g = 0; g < kCombineGroups; ++g) {
      r0 += part[g][2 * tid];
      r1 += part[g][2 * tid + 1];
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    uint32_t* dst = (uint32_t*)((uint16_t*)p.o + ((int64_t)b * p.Hq + h) * D);
    dst[tid] = E::pack2(r0 * inv, r1 * inv);
  }
  if (tid == 0)
    p.lse[(int64_t)b * p.Hq + h] = sum > 0.f ? mx + __builtin_logf(sum) : neg_inf();
}

template <typename T, int D, int GB>
hipError_t launch_t(const DecodeParams& p, hipStream_t st) {
  if (p.prefix_len > 0) {
    constexpr int QB = 16;  // columns per MFMA block; an item takes two blocks
    const int64_t items =
        (int64_t)((p.B * p.group + 2 * QB - 1) / (2 * QB)) * p.prefix_splits * p.Hkv;
    const int blocks = (int)((items + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL((decode_split_kernel<T, D, QB, true>), dim3(blocks),
                       dim3(64 * kWavesPerBlock), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t items = (int64_t)p.B * (p.max_splits - p.split_offset) * p.Hkv * (p.group / GB);
  const int blocks = (int)((items + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL((decode_split_kernel<T, D, GB>), dim3(blocks), dim3(64 * kWavesPerBlock), 0,
                     st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(p.Hq, p.B), dim3(kCombineThreads), 0, st,
                     p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t st) {
  if (p.group % 8 == 0) return launch_t<T, D, 8>(p, st);
  if (p.group % 4 == 0) return launch_t<T, D, 4>(p, st);
  if (p.group % 2 == 0) return launch_t<T, D, 2>(p, st);
  return launch_t<T, D, 1>(p, st);
}

}  // namespace

// Fixed device workspace of the allocation-free decode entry point: each GPU
// the library runs on holds its own copy until the process ends. In host
// code `scratch` names a host-side stand-in, never the device memory: its
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// launch_t runs the prefix pass whenever p.prefix_len > 0.
hipError_t launch_decode_cascade(const DecodeParams& p, Dt dt, int d, hipStream_t st) {
  return launch_decode(p, dt, d, st);
}

hipError_t launch_decode(const DecodeParams& p, Dt dt, int d, hipStream_t st) {
  switch (dt) {
    case Dt::Bf16:
      return d == 64 ? launch_d<Bf16, 64>(p, st) : launch_d<Bf16, 128>(p, st);
    case Dt::F16:
      return d == 64 ? launch_d<F16, 64>(p, st) : launch_d<F16, 128>(p, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fa
