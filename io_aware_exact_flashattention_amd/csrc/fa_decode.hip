// fa_decode.hip - split-KV decode over a paged K/V cache, gfx950.
//
// The serving variant of the page "I/O-Aware Kernels" (datasystem.school,
// Module 5), section "FlashInfer: I/O-aware attention for serving": the
// fused kernel with keys and values gathered from a paged cache through a
// page table, for a batch of sequences of different lengths and
// grouped-query heads. One query token per sequence.
//
// Decode reads every K/V byte once and does ~4 flops per byte, so it is
// bound by HBM bandwidth, not by matrix throughput; the work runs on the
// vector ALUs and the design goal is many independent 16-byte loads in
// flight:
//  * Work item = (sequence, KV head, split). A split is a run of
//    `pages_per_split` pages; the GB query heads that share the KV head are
//    handled together, so each K/V byte is read once for all of them.
//  * One wavefront per item. Lane = (token slot t = lane/4, quarter
//    c = lane%4): per 16-token page each lane loads 64 contiguous bytes of
//    one token's K row and of its V row (head dimension 128), and the next
//    page's loads are issued before the current page is consumed.
//  * Scores: packed 16-bit dot products (v_dot2_f32_{bf16,f16}) over the
//    lane's quarter of the head dimension, summed over the 4 lanes of a
//    token with two lane exchanges.
//  * Each lane keeps its own running max / sum / output accumulator for its
//    token slot (the online softmax of section "FlashAttention: tiling +
//    online softmax"), so no cross-lane reduction happens per page. The
//    accumulator is rescaled only when a logit exceeds the lane's reference
//    max by more than 2^8 (kept exact: the same reference enters the
//    numerator and the denominator; weights stay <= 2^8 in fp32).
//  * At the end of the split the 16 token slots are merged with lane
//    exchanges (log-sum-exp merge), and the normalised partial output and
//    its log-sum-exp go to the workspace.
//  * A second kernel merges the splits of each (sequence, query head):
//    lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s, in fixed
//    split order (deterministic).
// Slots of a last page beyond the sequence end are never allowed into the
// result: their scores are -inf and their V values are replaced by zero
// before use, so NaN garbage there cannot leak.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kPage = 16;
constexpr float kRescaleThreshold = 8.f;  // log2 units

template <typename T> struct Dot2;
template <> struct Dot2<Bf16> {
  __device__ static __forceinline__ float dot(uint32_t a, uint32_t b, float c) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  }
};
template <> struct Dot2<F16> {
  __device__ static __forceinline__ float dot(uint32_t a, uint32_t b, float c) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
  }
};

__device__ __forceinline__ uint32_t comp(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <typename T, int D, int GB>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  using E = Elem<T>;
  constexpr int DQ = D / 4;     // head-dim values per lane
  constexpr int NCH = DQ / 8;   // 16-byte chunks per lane per row
  constexpr int NW = DQ / 2;    // packed 32-bit words per lane per row

  const int s = blockIdx.x, b = blockIdx.z;
  const int nhb = p.group / GB;
  const int g = blockIdx.y / nhb;
  const int h0 = g * p.group + (blockIdx.y % nhb) * GB;
  const int L = p.seq_lens[b];
  const int npages = (L + kPage - 1) / kPage;
  const int pg0 = s * p.pages_per_split;
  if (pg0 >= npages) return;
  const int pg1 = min(npages, pg0 + p.pages_per_split);

  const int lane = threadIdx.x, t = lane >> 2, c = lane & 3;
  const float c2 = p.scale_log2;

  // query heads h0 .. h0+GB-1, this lane's quarter, packed 16-bit pairs
  uint32_t qw[GB][NW];
#pragma unroll
  for (int h = 0; h < GB; ++h) {
    const uint16_t* src = (const uint16_t*)p.q + ((int64_t)b * p.Hq + h0 + h) * D + c * DQ;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const uint4 v = *(const uint4*)(src + 8 * i);
      qw[h][4 * i + 0] = v.x;
      qw[h][4 * i + 1] = v.y;
      qw[h][4 * i + 2] = v.z;
      qw[h][4 * i + 3] = v.w;
    }
  }

  float m[GB], l[GB], o[GB][DQ];
#pragma unroll
  for (int h = 0; h < GB; ++h) {
    m[h] = neg_inf();
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < DQ; ++i) o[h][i] = 0.f;
  }

  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
  const int64_t tok_stride = (int64_t)p.Hkv * D;  // elements between tokens of a page
  const uint16_t* kpool = (const uint16_t*)p.k_pool + (int64_t)g * D + c * DQ;
  const uint16_t* vpool = (const uint16_t*)p.v_pool + (int64_t)g * D + c * DQ;

  uint4 kc[NCH], vc[NCH], kn[NCH], vn[NCH];
  {
    const int64_t off = ((int64_t)pt[pg0] * kPage + t) * tok_stride;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      kc[i] = *(const uint4*)(kpool + off + 8 * i);
      vc[i] = *(const uint4*)(vpool + off + 8 * i);
    }
  }

  for (int pg = pg0; pg < pg1; ++pg) {
    if (pg + 1 < pg1) {
      const int64_t off = ((int64_t)pt[pg + 1] * kPage + t) * tok_stride;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        kn[i] = *(const uint4*)(kpool + off + 8 * i);
        vn[i] = *(const uint4*)(vpool + off + 8 * i);
      }
    }
    const bool valid = pg * kPage + t < L;

    // scores of this lane's token for every head (log2 domain)
    float sc[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) part = Dot2<T>::dot(comp(kc[i], w), qw[h][4 * i + w], part);
      part += xor_lane(part, 1);
      part += xor_lane(part, 2);
      sc[h] = valid ? part * c2 : neg_inf();
    }

    // lazy rescale: only when some lane's logit passes its reference by 2^8
    bool need = false;
#pragma unroll
    for (int h = 0; h < GB; ++h) need |= sc[h] > m[h] + kRescaleThreshold;
    if (__ballot(need)) {
#pragma unroll
      for (int h = 0; h < GB; ++h) {
        const bool up = sc[h] > m[h] + kRescaleThreshold;
        const float alpha = up ? fast_exp2(m[h] - sc[h]) : 1.f;
        m[h] = up ? sc[h] : m[h];
        l[h] *= alpha;
#pragma unroll
        for (int i = 0; i < DQ; ++i) o[h][i] *= alpha;
      }
    }

    // V row of this token (zero for slots past the sequence end)
    float vf[DQ];
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = valid ? comp(vc[i], w) : 0u;
        vf[8 * i + 2 * w] = E::lo(x);
        vf[8 * i + 2 * w + 1] = E::hi(x);
      }
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      const float pr = valid ? fast_exp2(sc[h] - m[h]) : 0.f;
      l[h] += pr;
#pragma unroll
      for (int i = 0; i < DQ; ++i) o[h][i] = fmaf(pr, vf[i], o[h][i]);
    }

#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      kc[i] = kn[i];
      vc[i] = vn[i];
    }
  }

  // merge the 16 token slots that share a quarter c (lanes c, c+4, ...)
#pragma unroll
  for (int x = 4; x < 64; x <<= 1) {
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      const float mo = xor_lane(m[h], x);
      const float lo = xor_lane(l[h], x);
      const float mn = fmaxf(m[h], mo);
      const float base = (mn == neg_inf()) ? 0.f : mn;
      const float a = fast_exp2(m[h] - base), bo = fast_exp2(mo - base);
      l[h] = l[h] * a + lo * bo;
      m[h] = mn;
#pragma unroll
      for (int i = 0; i < DQ; ++i) {
        const float oo = xor_lane(o[h][i], x);
        o[h][i] = o[h][i] * a + oo * bo;
      }
    }
  }

  if (t == 0) {
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      const int64_t row = ((int64_t)b * p.Hq + h0 + h) * p.max_splits + s;
      const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
      float* dst = p.o_part + row * D + c * DQ;
#pragma unroll
      for (int i = 0; i < DQ; i += 4)
        *(float4*)(dst + i) = make_float4(o[h][i] * inv, o[h][i + 1] * inv, o[h][i + 2] * inv,
                                          o[h][i + 3] * inv);
      if (c == 0) p.lse_part[row] = l[h] > 0.f ? (m[h] + __builtin_log2f(l[h])) * kLn2 : neg_inf();
    }
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
