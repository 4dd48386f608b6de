// Split-KV decoding (Flash-Decoding) for gfx950: one query row per (batch, head).
//
// Method (page "Bellek Duvarının Fiziği: Standart Attention'dan FlashAttention'a", section
// "Decode Aşaması: Flash-Decoding"): the keys of each (b, h) are cut into C chunks handled by
// separate workgroups; each chunk produces its own triple (max, sum, unnormalised output); one
// reduction then merges the chunks with the same rescaling identity the forward pass uses
// between key tiles (section "Online Softmax").
//
// CDNA4 mapping. The step reads every K and V element exactly once and does ~1 FLOP per byte, so
// it is bound by HBM bandwidth and does not use the matrix cores. A key row (d bf16) is read by
// d/8 consecutive lanes with 16-byte non-temporal loads, so one wave instruction moves whole rows
// (1 KiB at d = 128) and each lane keeps U rows of K and of V in flight. Scores are bf16 dot
// products (v_dot2_f32_bf16) reduced across the row's lanes with DPP row rotations. Every group of
// lanes that shares a key row keeps its own running (max, sum, output) for its rows; the groups
// of a workgroup are merged once through LDS at the end, so the hot loop has no barriers and no
// cross-group traffic. Partial outputs are stored normalised with their natural-log log-sum-exp,
// and a small second kernel combines them.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecUnroll = 8;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8(u32x4 a, u32x4 b) {
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // Copy the words out first: hipcc (clang 22) folds __builtin_bit_cast of a vector element
    // indexed by the unrolled loop variable to element 0.
    const uint32_t aw = a[w], bw = b[w];
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw),
                                        __builtin_bit_cast(bf16x2, bw), s, false);
  }
  return s;
}

template <int D>
__global__ __launch_bounds__(kDecWaves * 64) void decode_split_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    float* __restrict__ part_o, float* __restrict__ part_lse, int C, int Nk, int chunk, float c) {
  constexpr int G = D / 8;            // lanes per key row
  constexpr int KPI = 64 / G;         // key rows per wave instruction
  constexpr int KPW = KPI * kDecUnroll;
  constexpr int NGRP = kDecWaves * KPI;  // lane groups per workgroup
  __shared__ float sm_m[NGRP], sm_l[NGRP];
  __shared__ float sm_acc[NGRP][D];

  const int bid = blockIdx.x;
  const int bh = bid / C, split = bid % C;
  const int k0 = split * chunk;
  const int k1 = min(Nk, k0 + chunk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane / G, gl = lane % G;

  const bf16* Kh = K + (size_t)bh * Nk * D + gl * 8;
  const bf16* Vh = V + (size_t)bh * Nk * D + gl * 8;
  const u32x4 qv = ld16(Q + (size_t)bh * D + gl * 8);

  float m = kNegInf, l = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;

  for (int base = k0 + wave * KPW; base < k1; base += kDecWaves * KPW) {
    u32x4 kr[kDecUnroll], vr[kDecUnroll];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int key = base + u * KPI + g;
      const u32x4 z = {0u, 0u, 0u, 0u};
      kr[u] = z;
      vr[u] = z;
      if (key < k1) {
        kr[u] = ld16_nt(Kh + (size_t)key * D);
        vr[u] = ld16_nt(Vh + (size_t)key * D);
      }
    }
    float s[kDecUnroll];
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const float dot = group_sum<G>(dot8(kr[u], qv));
      s[u] = (base + u * KPI + g < k1) ? dot * c : kNegInf;
      mx = fmaxf(mx, s[u]);
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const float p = exp2_fast(s[u] - m_use);
      l += p;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] = __builtin_fmaf(p, bf16_lo(vr[u][w]), acc[2 * w]);
        acc[2 * w + 1] = __builtin_fmaf(p, bf16_hi(vr[u][w]), acc[2 * w + 1]);
      }
    }
  }

  // ---- merge the lane groups of the workgroup
  const int grp = wave * KPI + g;
  if (gl == 0) {
    sm_m[grp] = m;
    sm_l[grp] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm_acc[grp][gl * 8 + e] = acc[e];
  __syncthreads();
  float M = kNegInf;
#pragma unroll 4
  for (int i = 0; i < NGRP; ++i) M = fmaxf(M, sm_m[i]);
  const size_t pidx = (size_t)bh * C + split;
  for (int d = tid; d < D; d += kDecWaves * 64) {
    if (M == kNegInf) {  // empty chunk: weight zero in the combine
      part_o[pidx * D + d] = 0.f;
      if (d == 0) part_lse[pidx] = kNegInf;
      continue;
    }
    float L = 0.f, o = 0.f;
    for (int i = 0; i < NGRP; ++i) {
      const float w = exp2_fast(sm_m[i] - M);
      L += sm_l[i] * w;
      o += sm_acc[i][d] * w;
    }
    part_o[pidx * D + d] = o / L;
    if (d == 0) part_lse[pidx] = (M + log2_fast(L)) * kLn2;
  }
}

// Merge the C partial results of each (b, h): L = ln sum_c e^{L_c}, O = sum_c e^{L_c - L} O_c.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_lse,
                                                            bf16* __restrict__ O,
                                                            float* __restrict__ LSE, int C) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float* pl = part_lse + (size_t)bh * C;
  const float* po = part_o + (size_t)bh * C * D;
  float M = kNegInf;
  for (int i = 0; i < C; ++i) M = fmaxf(M, pl[i]);
  if (M == kNegInf) {  // no position at all (an empty paged sequence): o = 0, lse = -inf
#pragma unroll
    for (int j = 0; j < D / 64; ++j) O[(size_t)bh * D + tid + 64 * j] = (__bf16)0.f;
    if (tid == 0) LSE[bh] = kNegInf;
    return;
  }
  float S = 0.f;
  float o[D / 64];
#pragma unroll
  for (int j = 0; j < D / 64; ++j) o[j] = 0.f;
  for (int i = 0; i < C; ++i) {
    const float w = exp2_fast((pl[i] - M) * kLog2e);
    S += w;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) o[j] += w * po[(size_t)i * D + tid + 64 * j];
  }
  const float inv = 1.f / S;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) O[(size_t)bh * D + tid + 64 * j] = (__bf16)(o[j] * inv);
  if (tid == 0) LSE[bh] = M + log2_fast(S) * kLn2;
}

template <int D>
hipError_t launch(const DecodeArgs& a) {
  const int BH = a.B * a.H;
  const int C = a.splits;
  const int chunk = (a.Nk + C - 1) / C;
  const long long grid = (long long)BH * C;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c = a.scale * kLog2e;
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3((unsigned)grid), dim3(kDecWaves * 64), 0,
                     a.stream, a.q, a.k, a.v, a.part_o, a.part_lse, C, a.Nk, chunk, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(BH), dim3(64), 0, a.stream, a.part_o,
                     a.part_lse, a.o, a.lse, C);
  return hipGetLastError();
}


// Split-KV decode over a paged cache with grouped query heads. One workgroup per (b, group of HG
// query heads that share one K/V head, split): every K/V row of the split is read once and
// scored against the HG query rows, so the K/V bytes are shared by the group. Rows are found
// through the block table (power-of-two block size: shift and mask); everything else is the
// contiguous kernel above, with HG running (max, sum, output) triples per lane group.
template <int D, int HG>
__global__ __launch_bounds__(kDecWaves * 64) void decode_paged_split_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ Kc, const bf16* __restrict__ Vc,
    const int* __restrict__ table, const int* __restrict__ lens, float* __restrict__ part_o,
    float* __restrict__ part_lse, int H, int Hkv, int C, int chunk, int bs_log2, int num_blocks,
    int max_blocks, float c) {
  constexpr int G = D / 8;     // lanes per key row
  constexpr int KPI = 64 / G;  // key rows per wave instruction
  constexpr int U = HG >= 8 ? 4 : 8;
  constexpr int KPW = KPI * U;
  constexpr int NGRP = kDecWaves * KPI;
  __shared__ float sm_m[NGRP], sm_l[NGRP];
  __shared__ float sm_acc[NGRP][D];

  const int bid = blockIdx.x;
  const int split = bid % C, bhg = bid / C;
  const int ngroups = H / HG;
  const int b = bhg / ngroups, h0 = (bhg % ngroups) * HG;
  const int kvh = h0 / (H / Hkv);
  const int len = min(max(lens[b], 0), max_blocks << bs_log2);
  const int k0 = split * chunk;
  const int k1 = min(len, k0 + chunk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane / G, gl = lane % G;
  const int bmask = (1 << bs_log2) - 1;
  const size_t head_off = ((size_t)kvh << bs_log2) * D + gl * 8;  // this head inside a block
  const size_t block_stride = ((size_t)Hkv << bs_log2) * D;
  const int* trow = table + (size_t)b * max_blocks;

  u32x4 qv[HG];
#pragma unroll
  for (int j = 0; j < HG; ++j) qv[j] = ld16(Q + ((size_t)b * H + h0 + j) * D + gl * 8);
  float m[HG], l[HG], acc[HG][8];
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    m[j] = kNegInf;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }

  // block ids of the next iteration's rows are loaded one iteration ahead, so the table lookup
  // latency overlaps the current rows' K/V loads instead of preceding them
  auto block_of = [&](int key) -> unsigned {
    return key < k1 ? (unsigned)trow[key >> bs_log2] : 0xffffffffu;
  };
  unsigned blk[U];
#pragma unroll
  for (int u = 0; u < U; ++u) blk[u] = block_of(k0 + wave * KPW + u * KPI + g);
  for (int base = k0 + wave * KPW; base < k1; base += kDecWaves * KPW) {
    u32x4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * KPI + g;
      const u32x4 z = {0u, 0u, 0u, 0u};
      kr[u] = z;
      vr[u] = z;
      if (blk[u] < (unsigned)num_blocks) {  // past the chunk, or an id out of range: zero rows
        const size_t off = blk[u] * block_stride + head_off + (size_t)(key & bmask) * D;
        kr[u] = ld16_nt(Kc + off);
        vr[u] = ld16_nt(Vc + off);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) blk[u] = block_of(base + kDecWaves * KPW + u * KPI + g);
#pragma unroll
    for (int j = 0; j < HG; ++j) {
      float s[U];
      float mx = kNegInf;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float dot = group_sum<G>(dot8(kr[u], qv[j]));
        s[u] = (base + u * KPI + g < k1) ? dot * c : kNegInf;
        mx = fmaxf(mx, s[u]);
      }
      const float m_new = fmaxf(m[j], mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2_fast(m[j] - m_use);
      m[j] = m_new;
      l[j] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = exp2_fast(s[u] - m_use);
        l[j] += p;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t vw = vr[u][w];
          acc[j][2 * w] = __builtin_fmaf(p, bf16_lo(vw), acc[j][2 * w]);
          acc[j][2 * w + 1] = __builtin_fmaf(p, bf16_hi(vw), acc[j][2 * w + 1]);
        }
      }
    }
  }

  // ---- merge the lane groups of the workgroup, one query head at a time
  const int grp = wave * KPI + g;
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    __syncthreads();  // the previous head's reads of the LDS slots are done
    if (gl == 0) {
      sm_m[grp] = m[j];
      sm_l[grp] = l[j];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_acc[grp][gl * 8 + e] = acc[j][e];
    __syncthreads();
    float M = kNegInf;
#pragma unroll 4
    for (int i = 0; i < NGRP; ++i) M = fmaxf(M, sm_m[i]);
    const size_t pidx = ((size_t)b * H + h0 + j) * C + split;
    for (int d = tid; d < D; d += kDecWaves * 64) {
      if (M == kNegInf) {  // empty chunk: weight zero in the combine
        part_o[pidx * D + d] = 0.f;
        if (d == 0) part_lse[pidx] = kNegInf;
        continue;
      }
      float L = 0.f, o = 0.f;
      for (int i = 0; i < NGRP; ++i) {
        const float w = exp2_fast(sm_m[i] - M);
        L += sm_l[i] * w;
        o += sm_acc[i][d] * w;
      }
      part_o[pidx * D + d] = o / L;
      if (d == 0) part_lse[pidx] = (M + log2_fast(L)) * kLn2;
    }
  }
}

template <int D, int HG>
hipError_t launch_paged(const DecodePagedArgs& a) {
  const int C = a.splits;
  const int max_len = a.max_blocks * a.block_size;
  const int chunk = (max_len + C - 1) / C;
  const long long grid = (long long)a.B * (a.H / HG) * C;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c = a.scale * kLog2e;
  const int bs_log2 = __builtin_ctz((unsigned)a.block_size);
  hipLaunchKernelGGL((decode_paged_split_kernel<D, HG>), dim3((unsigned)grid),
                     dim3(kDecWaves * 64), 0, a.stream, a.q, a.k_cache, a.v_cache, a.block_table,
                     a.seq_lens, a.part_o, a.part_lse, a.H, a.Hkv, C, chunk, bs_log2,
                     a.num_blocks, a.max_blocks, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.B * a.H), dim3(64), 0, a.stream,
                     a.part_o, a.part_lse, a.o, a.lse, C);
  return hipGetLastError();
}

template <int D>
hipError_t launch_paged_d(const DecodePagedArgs& a) {
  switch (decode_paged_heads_per_group(a.H, a.Hkv)) {
    case 8: return launch_paged<D, 8>(a);
    case 4: return launch_paged<D, 4>(a);
    case 2: return launch_paged<D, 2>(a);
    default: return launch_paged<D, 1>(a);
  }
}
}  // namespace

int decode_auto_splits(int B, int H, int Nk, int d) {
  (void)d;
  const long long bh = (long long)B * H;
  const long long target = 4096;  // workgroups: 16 per CU on 256 CUs
  long long c = (target + bh - 1) / bh;
  const long long by_len = ((long long)Nk + 511) / 512;  // at least ~512 keys per split
  if (c > by_len) c = by_len;
  if (c > 1024) c = 1024;
  if (c < 1) c = 1;
  return (int)c;
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.d == 128 ? launch<128>(a) : launch<64>(a);
}

int decode_paged_heads_per_group(int H, int Hkv) {
  const int g = H / Hkv;
  for (int hg = 8; hg > 1; hg >>= 1)
    if (g % hg == 0) return hg;
  return 1;
}

int decode_paged_auto_splits(int B, int H, int Hkv, int max_len, int d) {
  (void)d;
  const long long wgs = (long long)B * (H / decode_paged_heads_per_group(H, Hkv));
  // workgroups: 4 per CU on 256 CUs. Measured at B8 H32 H_kv8, 65536 positions: 16 splits
  // (1024 workgroups) 0.36 ms, 64 splits 0.38 ms, 256 splits 0.50 ms; the per-workgroup merge of
  // several heads makes short chunks cost more than in the contiguous kernel.
  const long long target = 1024;
  long long c = (target + wgs - 1) / wgs;
  const long long by_len = ((long long)max_len + 1023) / 1024;  // at least ~1024 positions
  if (c > by_len) c = by_len;
  if (c > 1024) c = 1024;
  if (c < 1) c = 1;
  return (int)c;
}

hipError_t launch_decode_paged(const DecodePagedArgs& a) {
  return a.d == 128 ? launch_paged_d<128>(a) : launch_paged_d<64>(a);
}

}  // namespace fa
