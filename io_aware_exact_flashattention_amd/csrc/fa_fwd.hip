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

constexpr int kBM = 128;  // query rows per workgroup, 16-bit path
constexpr int kBN = 64;   // keys per K/V tile, 16-bit path
constexpr int kThreads = 256;

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

// 16-byte chunk swizzle of an LDS row holding `chunks` chunks: rows that one
// MFMA operand read touches together map to distinct banks.
template <int chunks>
__device__ __forceinline__ int swz(int row) {
  if constexpr (chunks == 16) return row & 15;
  else return (row >> 1) & 7;
}

// Position of key `key` (0..63 inside a tile) in a V^T row. The score
// accumulator gives lane-half h, register r of 32-key block kb the key
// 32kb + 8(r/4) + 4h + r%4; the PV B operand of (kb, u) is registers
// 8u..8u+7, i.e. keys 16u + {4h..4h+3, 8+4h..8+4h+3}. Those 8 keys sit
// contiguously at 32kb + 16u + 8h, so one 16-byte LDS read is the matching A
// operand.
__device__ __forceinline__ int vt_pos(int key) {
  const int o = key & 15;
  return (key & ~15) + 8 * ((o >> 2) & 1) + (o & 3) + 4 * (o >> 3);
}

__device__ __forceinline__ uint32_t comp(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_mfma_kernel(FwdParams p) {
  using E = Elem<T>;
  constexpr int KCH = D / 8;    // 16-byte chunks per K row
  constexpr int VCH = kBN / 8;  // 16-byte chunks per V^T row
  constexpr int KS = D / 16;    // MFMA k-steps of Q K^T
  constexpr int DB = D / 32;    // 32-row blocks of O^T
  constexpr int NB = kBN / 32;  // 32-key blocks per tile
  constexpr int K_UNITS = kBN * KCH / kThreads;
  constexpr int V_UNITS = (kBN / 2) * (D / 8) / kThreads;
  static_assert(K_UNITS >= 1 && V_UNITS >= 1, "tile too small for the workgroup");

  __shared__ uint4 k_lds[2][kBN * KCH];
  __shared__ uint4 v_lds[2][D * VCH];

  const Work w = map_block(p.n_qtiles, p.Hq);
  int q0, Lq, k0, Lk;
  seq_bounds(p, w.b, q0, Lq, k0, Lk);
  const int row0 = w.tile * kBM;
  if (row0 >= Lq) return;  // ragged batch: this sequence has fewer tiles

  const int g = w.h / p.group;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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

  const uint16_t* kbase = (const uint16_t*)p.k + (int64_t)k0 * p.kv_row + (int64_t)g * D;
  const uint16_t* vbase = (const uint16_t*)p.v + (int64_t)k0 * p.kv_row + (int64_t)g * D;

  uint4 kreg[K_UNITS];
  uint4 vreg[V_UNITS][2];

  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < K_UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int r = u / KCH, c = u % KCH;
      const int key = j * kBN + r;
      kreg[i] = make_uint4(0, 0, 0, 0);
      if (key < Lk) kreg[i] = *(const uint4*)(kbase + (int64_t)key * p.kv_row + c * 8);
    }
#pragma unroll
    for (int i = 0; i < V_UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int c = u % (D / 8), m = u / (D / 8);
      const int key = j * kBN + 2 * m;
      vreg[i][0] = make_uint4(0, 0, 0, 0);
      vreg[i][1] = make_uint4(0, 0, 0, 0);
      if (key < Lk) vreg[i][0] = *(const uint4*)(vbase + (int64_t)key * p.kv_row + c * 8);
      if (key + 1 < Lk) vreg[i][1] = *(const uint4*)(vbase + (int64_t)(key + 1) * p.kv_row + c * 8);
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int r = u / KCH, c = u % KCH;
      k_lds[buf][r * KCH + (c ^ swz<KCH>(r))] = kreg[i];
    }
    uint32_t* vt = (uint32_t*)v_lds[buf];
#pragma unroll
    for (int i = 0; i < V_UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int c = u % (D / 8), m = u / (D / 8);
      const int pos = vt_pos(2 * m);  // even; key 2m+1 sits at pos+1
      const int chunk = pos >> 3, wi = (pos & 7) >> 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t a = comp(vreg[i][0], e >> 1), b = comp(vreg[i][1], e >> 1);
        const uint32_t packed = (e & 1) ? byte_perm(b, a, 0x07060302u) : byte_perm(b, a, 0x05040100u);
        const int d = 8 * c + e;
        vt[(d * VCH + (chunk ^ swz<VCH>(d))) * 4 + wi] = packed;
      }
    }
  };

  f32x16 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
  float m_run = neg_inf();  // running max of scaled logits, log2 domain
  float l_run = 0.f;        // this lane's share of the running row sum
  const float c2 = p.scale_log2;

  if (n_kv > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_kv; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_kv) load_tile(j + 1);

    bool active = wrow0 < Lq;
    if (CAUSAL) active = active && (j * kBN <= wrow0 + 31 + delta);
    if (active) {
      // ---- partial scores S^T = K_j Q^T (two 32x32 blocks) ----
      f32x16 acc_s[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_s[kb][r] = 0.f;
        const int krow = 32 * kb + l32;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const uint4 a = k_lds[buf][krow * KCH + ((2 * s + hh) ^ swz<KCH>(krow))];
          acc_s[kb] = E::mma32(a, qf[s], acc_s[kb]);
        }
      }
      // ---- mask keys past the sequence end / above the diagonal ----
      const bool need_mask =
          (j * kBN + kBN > Lk) || (CAUSAL && (j * kBN + kBN - 1 > wrow0 + delta));
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j * kBN + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            bool vis = key < Lk;
            if (CAUSAL) vis = vis && (key <= my_row + delta);
            if (!vis) acc_s[kb][r] = neg_inf();
          }
      }
      // ---- online softmax: running max m, running sum l ----
      float mx = neg_inf();
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc_s[kb][r]);
      mx = fmaxf(mx, xor_lane(mx, 32));
      const float m_new = fmaxf(m_run, mx * c2);
      const float base = (m_new == neg_inf()) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - base);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(fmaf(acc_s[kb][r], c2, -base));
          acc_s[kb][r] = e;
          rs += e;
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
      }
      // ---- O^T += V_j^T P^T ----
      uint4 pf[NB][2];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 8 * u;
          pf[kb][u] = make_uint4(E::pack2(acc_s[kb][r + 0], acc_s[kb][r + 1]),
                                 E::pack2(acc_s[kb][r + 2], acc_s[kb][r + 3]),
                                 E::pack2(acc_s[kb][r + 4], acc_s[kb][r + 5]),
                                 E::pack2(acc_s[kb][r + 6], acc_s[kb][r + 7]));
        }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 32 * db + l32;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int chunk = 4 * kb + 2 * u + hh;
            const uint4 a = v_lds[buf][d * VCH + (chunk ^ swz<VCH>(d))];
            acc_o[db] = E::mma32(a, pf[kb][u], acc_o[db]);
          }
      }
    }

    if (j + 1 < n_kv) store_tile(buf ^ 1);
    __syncthreads();
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
