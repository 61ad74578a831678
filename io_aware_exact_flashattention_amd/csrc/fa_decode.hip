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
//    row layout with coalesced 16-byte loads.
//  * A second kernel merges the splits of each (sequence, query head):
//    lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s, in fixed
//    split order (deterministic).
// Slots of a last page beyond the sequence end never enter the result:
// their scores are -inf and their V values are replaced by zero before use,
// so NaN garbage there cannot leak.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kPage = 16;
constexpr float kRescaleThreshold = 8.f;  // log2 units

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

__device__ __forceinline__ uint32_t comp(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// One wavefront per (sequence b, KV head g, head block, split s).
//
// Scores of a 16-token page for the GB query heads of the block come from
// v_mfma_f32_16x16x32: A = the page's K rows (lane l: token l%16, an 8-value
// slice of d chosen by l/16), B = Q^T (lane l: query head l%16, zero past
// GB). In the 16x16 result lane l holds tokens 4(l/16)+i of head l%16.
// The running max of each head is wave-uniform (kept in scalar registers):
// a page max is reduced over the token lanes and read back with readlane.
// The probabilities go through a small LDS array to the P.V lanes, where
// lane (tg, c) owns the 16-byte slice c of d for tokens tg, tg+TPI, ... and
// accumulates O on the vector ALUs (V is read in its natural row layout).
template <typename T, int D, int GB>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  using E = Elem<T>;
  constexpr int KSTEP = D / 32;  // MFMA k-steps per page
  constexpr int DL = D / 4;      // d values per lane group in the score MFMA
  constexpr int VCH = D / 8;     // 16-byte chunks per V row
  constexpr int TPI = 64 / VCH;  // tokens covered by one V load instruction
  constexpr int VI = kPage / TPI;
  static_assert(GB <= 16 && VI >= 1, "bad decode tile");
  __shared__ float p_lds[2][kPage * GB];

  const int s = blockIdx.x, b = blockIdx.z;
  const int nhb = p.group / GB;
  const int g = blockIdx.y / nhb;
  const int h0 = g * p.group + (blockIdx.y % nhb) * GB;
  const int L = p.seq_lens[b];
  const int npages = (L + kPage - 1) / kPage;
  const int pg0 = s * p.pages_per_split;
  if (pg0 >= npages) return;
  const int pg1 = min(npages, pg0 + p.pages_per_split);

  const int lane = threadIdx.x;
  const int l16 = lane & 15, j = lane >> 4;   // score layout
  const int c = lane % VCH, tg = lane / VCH;  // P.V layout
  const float c2 = p.scale_log2;

  // B operand: Q^T, heads h0 .. h0+GB-1 in columns 0..GB-1
  uint4 qf[KSTEP];
#pragma unroll
  for (int st = 0; st < KSTEP; ++st) qf[st] = make_uint4(0, 0, 0, 0);
  if (l16 < GB) {
    const uint16_t* src = (const uint16_t*)p.q + ((int64_t)b * p.Hq + h0 + l16) * D + j * DL;
#pragma unroll
    for (int st = 0; st < KSTEP; ++st) qf[st] = *(const uint4*)(src + 8 * st);
  }

  float m[GB];          // running max per head, log2 domain (wave-uniform)
  float o[GB][8];       // this lane's slice of O for each head
#pragma unroll
  for (int h = 0; h < GB; ++h) {
    m[h] = neg_inf();
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  float l_lane = 0.f;   // share of the row sum of head l16 (tokens of this lane)

  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
  const int64_t tok = (int64_t)p.Hkv * D;  // elements between tokens of a page
  const uint16_t* kpool = (const uint16_t*)p.k_pool + (int64_t)g * D + j * DL + l16 * tok;
  const uint16_t* vpool = (const uint16_t*)p.v_pool + (int64_t)g * D + c * 8 + tg * tok;

  uint4 kc[KSTEP], vc[VI], kn[KSTEP], vn[VI];
  auto load_page = [&](int pg, uint4* kk, uint4* vv) {
    const int64_t base = (int64_t)pt[pg] * kPage * tok;
#pragma unroll
    for (int st = 0; st < KSTEP; ++st) kk[st] = *(const uint4*)(kpool + base + 8 * st);
#pragma unroll
    for (int r = 0; r < VI; ++r) vv[r] = *(const uint4*)(vpool + base + r * TPI * tok);
  };
  load_page(pg0, kc, vc);

  for (int pg = pg0; pg < pg1; ++pg) {
    if (pg + 1 < pg1) load_page(pg + 1, kn, vn);
    const int tok0 = pg * kPage;

    // ---- scores S[token][head] on the matrix cores ----
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KSTEP; ++st) acc = Mma16<T>::mma(kc[st], qf[st], acc);
    float sc[4];
    float mx = neg_inf();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (l16 < GB) && (tok0 + 4 * j + i < L);
      sc[i] = ok ? acc[i] * c2 : neg_inf();
      mx = fmaxf(mx, sc[i]);
    }
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));

    // ---- running max per head; rescale only when it grows by > 2^8 ----
    float m_sel = m[0], a_sel = 1.f;
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      const float pm = lane_value(mx, h);
      if (pm > m[h] + kRescaleThreshold) {
        const float alpha = fast_exp2(m[h] - pm);
        m[h] = pm;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
        if (l16 == h) a_sel = alpha;
      }
      if (l16 == h) m_sel = m[h];
    }
    l_lane *= a_sel;

    // ---- probabilities -> LDS ----
    float* pl = p_lds[pg & 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pr = (sc[i] == neg_inf()) ? 0.f : fast_exp2(sc[i] - m_sel);
      l_lane += pr;
      if (l16 < GB) pl[(4 * j + i) * GB + l16] = pr;
    }
    __syncthreads();

    // ---- O += P V on the vector ALUs ----
#pragma unroll
    for (int r = 0; r < VI; ++r) {
      const int t = tg + r * TPI;
      const bool ok = tok0 + t < L;
      float pv[GB];
#pragma unroll
      for (int h = 0; h < GB; ++h) pv[h] = pl[t * GB + h];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = ok ? comp(vc[r], w) : 0u;
        const float v0 = E::lo(x), v1 = E::hi(x);
#pragma unroll
        for (int h = 0; h < GB; ++h) {
          o[h][2 * w] = fmaf(pv[h], v0, o[h][2 * w]);
          o[h][2 * w + 1] = fmaf(pv[h], v1, o[h][2 * w + 1]);
        }
      }
    }

#pragma unroll
    for (int st = 0; st < KSTEP; ++st) kc[st] = kn[st];
#pragma unroll
    for (int r = 0; r < VI; ++r) vc[r] = vn[r];
  }

  // ---- merge token groups (same running max everywhere: plain sums) ----
#pragma unroll
  for (int x = VCH; x < 64; x <<= 1)
#pragma unroll
    for (int h = 0; h < GB; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] += xor_lane(o[h][e], x);
  l_lane += xor_lane(l_lane, 16);
  l_lane += xor_lane(l_lane, 32);

#pragma unroll
  for (int h = 0; h < GB; ++h) {
    const float lt = lane_value(l_lane, h);
    const int64_t row = ((int64_t)b * p.Hq + h0 + h) * p.max_splits + s;
    if (tg == 0) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      float* dst = p.o_part + row * D + c * 8;
      *(float4*)dst = make_float4(o[h][0] * inv, o[h][1] * inv, o[h][2] * inv, o[h][3] * inv);
      *(float4*)(dst + 4) = make_float4(o[h][4] * inv, o[h][5] * inv, o[h][6] * inv, o[h][7] * inv);
    }
    if (lane == 0) p.lse_part[row] = lt > 0.f ? (m[h] + __builtin_log2f(lt)) * kLn2 : neg_inf();
  }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeParams p) {
  using E = Elem<T>;
  constexpr int PER = D / 64;  // head-dim values per lane
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = p.seq_lens[b];
  const int npages = (L + kPage - 1) / kPage;
  const int ns = (npages + p.pages_per_split - 1) / p.pages_per_split;
  const int64_t row = ((int64_t)b * p.Hq + h) * p.max_splits;
  const float* lp = p.lse_part + row;
  const float* op = p.o_part + row * D;

  float mx = neg_inf();
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, lp[s]);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float sum = 0.f;
  if (mx != neg_inf()) {
    for (int s = 0; s < ns; ++s) {
      const float w = fast_exp2((lp[s] - mx) * kLog2e);
      sum += w;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, op[(int64_t)s * D + lane + 64 * i], acc[i]);
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  uint16_t* dst = (uint16_t*)p.o + ((int64_t)b * p.Hq + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t w = E::pack2(acc[i] * inv, 0.f);
    dst[lane + 64 * i] = (uint16_t)(w & 0xffffu);
  }
  if (lane == 0)
    p.lse[(int64_t)b * p.Hq + h] = sum > 0.f ? mx + __builtin_logf(sum) : neg_inf();
}

template <typename T, int D, int GB>
hipError_t launch_t(const DecodeParams& p, hipStream_t st) {
  const dim3 grid_split(p.max_splits, p.Hkv * (p.group / GB), p.B);
  hipLaunchKernelGGL((decode_split_kernel<T, D, GB>), grid_split, dim3(64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(p.Hq, p.B), dim3(64), 0, st, p);
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
