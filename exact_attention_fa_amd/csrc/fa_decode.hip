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


// Split-KV decode over a paged cache with grouped query heads, on the matrix cores: with several
// query heads per K/V head the vector-ALU scheme above would spend a dot product, a lane
// reduction and d/8 multiply-adds per row and per query head, while the matrix cores take a whole
// group per instruction (measured at B8, 65536 positions, d128, against a vector-ALU kernel of
// that scheme: as fast with one query head per K/V head, 1.06x with 4, 1.6x with 8, 2.1x with
// 16, 2.9x with 32). One wave per (b, K/V head, block of up to 32 query
// heads of its group, split): the block's query heads play the 32 query rows of the forward
// kernel's transposed products, so S^T = K Q^T and O^T = V^T P^T run on
// v_mfma_f32_32x32x16_bf16 with lane = query head. A tile is 32 positions: the wave reads its K
// and V rows with whole-row 16-byte loads (d/8 consecutive lanes per row, as the vector kernel
// does), keeps them in registers while the previous tile is computed, then writes them to two
// private LDS tiles, from which the K rows come back in the A-operand order of the first product
// and the V rows transposed (ds_read_b64_tr_b16) for the second, as in the forward kernel. The
// block ids of a tile's rows are loaded one tile ahead, one row per lane, and handed to the lanes
// that load each row by a lane shuffle. The online softmax is the forward's; each wave writes its
// split's normalised output and log-sum-exp per query head, and the combine kernel merges the
// splits. Heads past the group in the last block have zero queries and are never stored.
// PAGED = false: the same kernel over a contiguous cache K, V [B, H_kv, Nk, d] (no block table,
// every sequence Nk positions long; table, lens, bs_log2, num_blocks and max_blocks unused).
template <int D, bool PAGED>
__global__ __attribute__((amdgpu_waves_per_eu(2, 2))) __launch_bounds__(64) void
decode_paged_mfma_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ Kc,
                         const bf16* __restrict__ Vc, const int* __restrict__ table,
                         const int* __restrict__ lens, float* __restrict__ part_o,
                         float* __restrict__ part_lse, int H, int Hkv, int C, int chunk,
                         int bs_log2, int num_blocks, int max_blocks, float c, int Nk) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KS = D / 16;          // 16-dim steps of the first product = row pieces per lane
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;       // rows per wave-wide load
  constexpr int KST = 2 * D + 16;     // K row stride in LDS (bytes), as in the forward kernel
  constexpr int VST = 2 * D + (D == 128 ? 32 : 16);  // V row stride, as in the forward kernel
  __shared__ __attribute__((aligned(16))) unsigned char kt[32 * KST];
  __shared__ __attribute__((aligned(16))) unsigned char vt[32 * VST];

  const int G = H / Hkv, nhb = (G + 31) / 32;
  int bid = blockIdx.x;
  const int split = bid % C;
  bid /= C;
  const int hb = bid % nhb;
  bid /= nhb;
  const int kvh = bid % Hkv, b = bid / Hkv;
  const int lane = threadIdx.x, l32 = lane & 31, hi = lane >> 5;
  const int nheads = min(32, G - 32 * hb);  // query heads of this block
  const int h0 = kvh * G + 32 * hb;          // first query head of the block
  const int len = PAGED ? min(max(lens[b], 0), max_blocks << bs_log2) : Nk;
  const int k0 = split * chunk;
  const int k1 = min(len, k0 + chunk);
  const int ntiles = k1 > k0 ? (k1 - k0 + 31) / 32 : 0;
  const int bmask = (1 << bs_log2) - 1;
  const size_t head_off = ((size_t)kvh << bs_log2) * D;  // this K/V head inside a block
  const size_t block_stride = ((size_t)Hkv << bs_log2) * D;
  const int* trow = PAGED ? table + (size_t)b * max_blocks : nullptr;
  const size_t seq_off = ((size_t)b * Hkv + kvh) * (size_t)Nk * D;  // contiguous: row 0

  // B operand of S^T = K Q^T: query head h0 + l32, dims 16 ks + 8 hi (zero past the block)
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (l32 < nheads) x = ld16(Q + ((size_t)b * H + h0 + l32) * D + ks * 16 + hi * 8);
    qf[ks] = as_bf16x8(x);
  }

  // loads: piece j of this lane is chunk (lane % CPR) of tile row RPI j + lane / CPR
  const int lrow = lane / CPR, lch = lane % CPR;
  auto block_of = [&](int t) -> unsigned {  // block id of tile row l32 of tile t (k1: none)
    if constexpr (!PAGED) return 0u;
    const int key = k0 + 32 * t + l32;
    return key < k1 ? (unsigned)trow[key >> bs_log2] : 0xffffffffu;
  };
  auto load_tile = [&](int t, unsigned blk_row, u32x4 (&kr)[KS], u32x4 (&vr)[KS]) {
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int r = RPI * j + lrow;
      const u32x4 z = {0u, 0u, 0u, 0u};
      if constexpr (PAGED) {
        const unsigned blk = (unsigned)__shfl((int)blk_row, r);
        // past the split, or an id out of range: zero rows
        const bool ok = blk < (unsigned)num_blocks;
        const size_t off = blk * block_stride + head_off +
                           (size_t)((k0 + 32 * t + r) & bmask) * D + lch * 8;
        kr[j] = ok ? ld16_nt(Kc + off) : z;
        vr[j] = ok ? ld16_nt(Vc + off) : z;
      } else {
        const int key = k0 + 32 * t + r;  // past the split: zero rows
        const size_t off = seq_off + (size_t)key * D + lch * 8;
        kr[j] = key < k1 ? ld16_nt(Kc + off) : z;
        vr[j] = key < k1 ? ld16_nt(Vc + off) : z;
      }
    }
  };
  // rows into the LDS tiles (the reads of the previous tile came earlier in this wave's program
  // order, and one wave's LDS operations complete in order)
  auto put_tile = [&](const u32x4 (&kr)[KS], const u32x4 (&vr)[KS]) {
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int r = RPI * j + lrow;
      st16(kt + r * KST + lch * 16, kr[j]);
      st16(vt + r * VST + lch * 16, vr[j]);
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  // m in log2 units of the scaled scores; l: fp32 sum (log-sum-exp); lq: sum of the bf16 P that
  // feed the second product (the normaliser of the output)
  float m_run = kNegInf, l_run = 0.f, lq_run = 0.f;

  // A operand of S^T: K row key_of_row(l32), dims 16 ks + 8 hi; A operand of O^T (V^T rows =
  // dims) by ds_read_b64_tr_b16, as in the forward kernel
  const int kr0 = key_of_row(l32) * KST + hi * 16;
  const int vj = lane & 15, vg = lane >> 4;
  const int vr0 = (8 * (vg >> 1) + (vj >> 2)) * VST + (16 * (vg & 1) + 4 * (vj & 3)) * 2;

  auto step = [&](int t) {
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma32(as_bf16x8(ld16(kt + kr0 + ks * 32)), qf[ks], sc);
    // register r holds key k0 + 32 t + key_of_reg(r, hi); keys at or past k1 are masked
    const int kb = k0 + 32 * t;
    if (kb + 32 > k1) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb + key_of_reg(r, hi) >= k1) sc[r] = kNegInf;
    }
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    // finite: every tile that is visited holds at least one key below k1
    const float m_new = fmaxf(m_run, halves_max(mx) * c);
    const float alpha = exp2_fast(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    lq_run *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[r] = exp2_fast(__builtin_fmaf(sc[r], c, -m_new));
      l_run += sc[r];
    }
    bf16x8 pf[2];
    pf[0] = pack_bf16x8(sc[0], sc[1], sc[2], sc[3], sc[4], sc[5], sc[6], sc[7]);
    pf[1] = pack_bf16x8(sc[8], sc[9], sc[10], sc[11], sc[12], sc[13], sc[14], sc[15]);
    lq_run = sum_bf16x8(pf[1], sum_bf16x8(pf[0], lq_run));
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        acc[db] = mfma32(lds_read_tr_pair(vt + vr0 + st * 16 * VST + db * 64, 4 * VST), pf[st],
                         acc[db]);
  };

  // tile t is computed from the LDS tiles while tile t + 1 loads into (kr, vr) (written to LDS
  // after the products of tile t) and the block ids of tile t + 2 are fetched
  u32x4 kr[KS], vr[KS];
  unsigned blk_next = 0xffffffffu;
  if (ntiles > 0) {
    load_tile(0, block_of(0), kr, vr);
    put_tile(kr, vr);
    if (ntiles > 1) blk_next = block_of(1);
  }
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1, blk_next, kr, vr);
    blk_next = t + 2 < ntiles ? block_of(t + 2) : 0xffffffffu;
    step(t);
    if (more) put_tile(kr, vr);
  }

  // ---- this split's partial for every query head of the block (rows of acc = dims)
  const float l_tot = halves_sum(l_run);
  const float lq_tot = halves_sum(lq_run);
  if (l32 < nheads) {
    const size_t pidx = ((size_t)b * H + h0 + l32) * C + split;
    const bool empty = ntiles == 0;
    const float inv = empty ? 0.f : 1.f / lq_tot;
    float* orow = part_o + pidx * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = acc[db][4 * q4 + e] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * q4 + 4 * hi) = w;
      }
    if (hi == 0) part_lse[pidx] = empty ? kNegInf : (m_run + log2_fast(l_tot)) * kLn2;
  }
#endif
}

template <int D>
hipError_t launch_paged(const DecodePagedArgs& a) {
  const int C = a.splits;
  const int max_len = a.max_blocks * a.block_size;
  const int chunk = (max_len + C - 1) / C;
  const int nhb = (a.H / a.Hkv + 31) / 32;
  const long long grid = (long long)a.B * a.Hkv * nhb * C;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c = a.scale * kLog2e;
  const int bs_log2 = __builtin_ctz((unsigned)a.block_size);
  hipLaunchKernelGGL((decode_paged_mfma_kernel<D, true>), dim3((unsigned)grid), dim3(64), 0,
                     a.stream, a.q, a.k_cache, a.v_cache, a.block_table, a.seq_lens, a.part_o,
                     a.part_lse, a.H, a.Hkv, C, chunk, bs_log2, a.num_blocks, a.max_blocks, c, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.B * a.H), dim3(64), 0, a.stream,
                     a.part_o, a.part_lse, a.o, a.lse, C);
  return hipGetLastError();
}

// grouped query heads over a contiguous cache: K, V [B, Hkv, Nk, d]
template <int D>
hipError_t launch_gqa(const DecodeArgs& a) {
  const int C = a.splits;
  const int chunk = (a.Nk + C - 1) / C;
  const int nhb = (a.H / a.Hkv + 31) / 32;
  const long long grid = (long long)a.B * a.Hkv * nhb * C;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c = a.scale * kLog2e;
  hipLaunchKernelGGL((decode_paged_mfma_kernel<D, false>), dim3((unsigned)grid), dim3(64), 0,
                     a.stream, a.q, a.k, a.v, nullptr, nullptr, a.part_o, a.part_lse, a.H, a.Hkv,
                     C, chunk, 0, 0, 0, c, a.Nk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.B * a.H), dim3(64), 0, a.stream,
                     a.part_o, a.part_lse, a.o, a.lse, C);
  return hipGetLastError();
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
  if (a.Hkv > 0 && a.Hkv != a.H) return a.d == 128 ? launch_gqa<128>(a) : launch_gqa<64>(a);
  return a.d == 128 ? launch<128>(a) : launch<64>(a);
}

int decode_paged_auto_splits(int B, int H, int Hkv, int max_len, int d) {
  (void)d;
  // one wave per split of each (b, K/V head, block of 32 query heads): about 8 waves per CU,
  // with at least ~512 positions per split. Measured at B8, 65536 positions, d128: 4 query heads
  // per K/V head (64 waves per split) 16 splits 0.353 ms, 32 splits 0.333 ms, 64 splits 0.354 ms;
  // 32 heads on one K/V head (8 waves per split) 32 splits 0.145 ms, 64 0.097 ms, 128 0.092 ms,
  // 256 0.129 ms (each split also writes and the combine reads one partial row per query head).
  const long long waves = (long long)B * Hkv * ((H / Hkv + 31) / 32);
  long long c = (2048 + waves - 1) / waves;
  const long long by_len = ((long long)max_len + 511) / 512;
  if (c > by_len) c = by_len;
  if (c > 1024) c = 1024;
  if (c < 1) c = 1;
  return (int)c;
}

hipError_t launch_decode_paged(const DecodePagedArgs& a) {
  return a.d == 128 ? launch_paged<128>(a) : launch_paged<64>(a);
}

}  // namespace fa
