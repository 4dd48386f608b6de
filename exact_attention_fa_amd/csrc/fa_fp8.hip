// FP8 attention forward with incoherent processing for gfx950 (CDNA4).
//
// Method (page "FlashAttention-3 (TR)", section on lowering precision to FP8 while reducing the
// quantization error; and the FlashAttention-3 paragraph of "Bellek Duvarının Fiziği"):
//   1. Q and K are multiplied by a random orthogonal matrix M = diag(sigma) H_d / sqrt(d) (random
//      signs times a Hadamard matrix): outlier coordinates are spread over all coordinates, and
//      (Q M)(K M)^T = Q K^T because M is orthogonal.
//   2. Q, K and V are quantized to FP8 with block-wise scales (Q per 32 rows, K per 64 rows, V one
//      scale per head): scale = amax / 448, code = E4M3(x / scale) after clamping to +-448,
//      with x / scale evaluated as x times the fp32 reciprocal of the scale.
//   3. Attention runs on the FP8 codes: S^T = K8 Q8^T on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3
//      operands, unit block exponents) with the two block scales folded into the softmax
//      multiply; the probabilities are quantized to E4M3 for O^T = V8^T P8^T on the same
//      instruction; O is normalised and scaled by the V scale at the end.
//
// Kernels.
//   * fp8_prep_kernel: one workgroup per 64 rows of Q, of K, or of V of one head. For Q and K it
//     applies the signs and the fast Walsh-Hadamard butterfly in fp32 (spans 1, 2, 4 inside a
//     lane's 8 values, then lane distances 1 .. d/16 by DPP moves inside the row's 16 or 8
//     lanes), multiplies by 1/sqrt(d),
//     reduces the block maxima, writes the scales and the E4M3 codes. For V it only writes the
//     block's max |x| (the head scale needs all of them).
//   * fp8_prep_v_kernel: one workgroup per 64 keys of one head: the head scale from the partial
//     maxima, then the E4M3 codes written transposed, V8^T [d][N_k padded to 64], so that the
//     second product's A operand (rows = head dimensions, k = keys) is a plain row read; padding
//     keys are zero.
//   * fwd_fp8_kernel: the bf16 forward's structure (waves of 32 queries, 64-key tiles copied
//     HBM -> LDS by buffer_load ... lds and double buffered, causal longest-first and XCD-aware
//     grid; here 4 waves per workgroup and one score buffer, see the kernel) with FP8 operands:
//       - operand layout of the 32x32x64 instruction (measured on the MI355X): lane (i, h)
//         holds row/column i and k = 32 h + 0..31 in its 32 bytes, for A and B alike; output
//         register r of lane (i, h) is row 8 (r / 4) + 4 h + (r % 4), column i;
//       - the K rows of a tile are handed to the first product in an order such that output
//         register r of block b in lane half h is key 32 h + 16 b + r, which is exactly byte
//         16 b + r of that lane's B operand of the second product (k = 32 h + byte): the
//         probabilities are packed in place, and V^T tile rows are read as 32 contiguous bytes;
//       - P is quantized as 2^8 P relative to the running maximum, with the running maximum
//         moved whenever a row would exceed it by more than 0.5 (log2 units), so 2^8 P stays
//         below 2^8.5 < 448.
#include "fa_device.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

constexpr float kFp8Max = 448.f;
constexpr int kBC8 = 64;             // keys per tile
constexpr float kSlack8 = 0.5f;      // lazy-rescale slack (log2 units)
constexpr float kPShift = 8.f;       // the second product uses E4M3(2^8 P)

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // E4M3 A and B (format 0), unit block exponents (127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Round a, b (|a|, |b| <= 448) to E4M3 (nearest even) into bytes 0-1 (HI = false) or 2-3 of w.
template <bool HI>
__device__ __forceinline__ int cvt2_fp8(float a, float b, int w) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, HI);
}

__device__ __forceinline__ float clamp_fp8(float x) { return fminf(fmaxf(x, -kFp8Max), kFp8Max); }

// y = clamp(x * r) with r = 1 / s rounded to fp32; when r overflows (s below 2^-128, a block of
// subnormal values) the quotient x / s itself. r and s are the same for all lanes of a block.
__device__ __forceinline__ void scale_by_reciprocal(const float (&x)[8], float s, float r,
                                                    float (&y)[8]) {
  if (__builtin_isinf(r)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = clamp_fp8(x[e] / s);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = clamp_fp8(x[e] * r);
  }
}

// max over the 256 threads of a workgroup (all threads must call it)
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int tid = threadIdx.x;
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ---------------------------------------------------------------------------------------------
// Q / K rotation and quantization, V partial maxima
template <int D>
__global__ __launch_bounds__(256) void fp8_prep_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    unsigned char* __restrict__ q8, unsigned char* __restrict__ k8, float* __restrict__ sq,
    float* __restrict__ sk, float* __restrict__ vpart, int Nq, int Nk, int nqb64, int nkb64,
    int nqb32, int incoherent, uint32_t key0, uint32_t key1, float inv_sqrt_d) {
  constexpr int TPR = D / 8;          // lanes per row (8 values each)
  constexpr int RPP = 256 / TPR;      // rows per pass
  constexpr int PASSES = 64 / RPP;
  __shared__ float red[2][4];
  const int tid = threadIdx.x, chunk = tid % TPR, rsub = tid / TPR;
  const int J = nqb64 + 2 * nkb64;
  const int bh = blockIdx.x / J, r = blockIdx.x % J;
  const int kind = r < nqb64 ? 0 : (r < nqb64 + nkb64 ? 1 : 2);  // Q, K, V
  const int blk = kind == 0 ? r : (kind == 1 ? r - nqb64 : r - nqb64 - nkb64);
  const int N = kind == 0 ? Nq : Nk;
  const bf16* src = (kind == 0 ? Q : (kind == 1 ? K : V)) + (size_t)bh * N * D;

  float x[PASSES][8];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = blk * 64 + p * RPP + rsub;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (row < N) w = ld16(src + (size_t)row * D + chunk * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[p][2 * i] = bf16_lo(w[i]);
      x[p][2 * i + 1] = bf16_hi(w[i]);
    }
  }
  if (kind < 2 && incoherent) {
    const u32x4 sw = philox4x32_10(0u, 0u, 0u, 0u, key0, key1);
    const uint32_t word = (chunk >> 2) == 0 ? sw[0] : (chunk >> 2) == 1 ? sw[1]
                          : (chunk >> 2) == 2 ? sw[2] : sw[3];
    const uint32_t bits = (word >> (8 * (chunk & 3))) & 0xFFu;  // signs of dims 8 chunk + 0..7
    uint32_t smask[8];  // sign bit to flip per value
#pragma unroll
    for (int e = 0; e < 8; ++e) smask[e] = ((bits >> e) & 1u) << 31;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[p][e] = __uint_as_float(__float_as_uint(x[p][e]) ^ smask[e]);
      // butterfly stages of span 1, 2, 4 inside the lane
#pragma unroll
      for (int h = 1; h < 8; h *= 2)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & h) == 0) {
            const float a = x[p][e], b = x[p][e + h];
            x[p][e] = a + b;
            x[p][e + h] = a - b;
          }
      // spans 8 .. D/2: lane distance 1 .. TPR/2 inside the row's lane group; the upper lane
      // of a pair takes o - x, the lower x + o, both as one exactly rounded fma(x, +-1, o)
      auto lane_stage = [&](auto DIST) {
        constexpr int dist = decltype(DIST)::value;
        const float sg = (chunk & dist) ? -1.f : 1.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[p][e] = fmaf(x[p][e], sg, lane_xor<dist>(x[p][e]));
      };
      static_assert(TPR == 8 || TPR == 16, "rows of 8 or 16 lanes");
      lane_stage(std::integral_constant<int, 1>());
      lane_stage(std::integral_constant<int, 2>());
      lane_stage(std::integral_constant<int, 4>());
      if constexpr (TPR == 16) lane_stage(std::integral_constant<int, 8>());
#pragma unroll
      for (int e = 0; e < 8; ++e) x[p][e] *= inv_sqrt_d;
    }
  }
  // block maxima: Q has two 32-row blocks per workgroup, K and V one 64-row block
  float am[2] = {0.f, 0.f};
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int b = kind == 0 ? (p * RPP) / 32 : 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) am[b] = fmaxf(am[b], fabsf(x[p][e]));
  }
  const float m0 = block_max(am[0], red[0]);
  const float m1 = block_max(am[1], red[1]);
  if (kind == 2) {
    if (tid == 0) vpart[(size_t)bh * nkb64 + blk] = m0;
    return;
  }
  float s[2];
  s[0] = m0 > 0.f ? m0 / kFp8Max : 1.f;
  s[1] = m1 > 0.f ? m1 / kFp8Max : 1.f;
  if (tid == 0) {
    if (kind == 0) {
      if (2 * blk < nqb32) sq[(size_t)bh * nqb32 + 2 * blk] = s[0];
      if (2 * blk + 1 < nqb32) sq[(size_t)bh * nqb32 + 2 * blk + 1] = s[1];
    } else {
      sk[(size_t)bh * nkb64 + blk] = s[0];
    }
  }
  unsigned char* dst = (kind == 0 ? q8 : k8) + (size_t)bh * N * D;
  const float rs[2] = {1.f / s[0], 1.f / s[1]};
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = blk * 64 + p * RPP + rsub;
    if (row >= N) continue;
    const int b = kind == 0 ? (p * RPP) / 32 : 0;
    float y[8];
    scale_by_reciprocal(x[p], s[b], rs[b], y);
    u32x2 w;
    w[0] = (uint32_t)cvt2_fp8<true>(y[2], y[3], cvt2_fp8<false>(y[0], y[1], 0));
    w[1] = (uint32_t)cvt2_fp8<true>(y[6], y[7], cvt2_fp8<false>(y[4], y[5], 0));
    *reinterpret_cast<u32x2*>(dst + (size_t)row * D + chunk * 8) = w;
  }
}

// ---------------------------------------------------------------------------------------------
// V: head scale, E4M3 codes written transposed to [d][N_k padded to a multiple of 64]
template <int D>
__global__ __launch_bounds__(256) void fp8_prep_v_kernel(
    const bf16* __restrict__ V, const float* __restrict__ vpart, unsigned char* __restrict__ v8t,
    float* __restrict__ sv, int Nk, int nkb64) {
  constexpr int TPR = D / 8, RPP = 256 / TPR, PASSES = 64 / RPP;  // PASSES: keys per thread
  static_assert(PASSES == 2 || PASSES == 4, "one 16- or 32-bit LDS word per dimension");
  constexpr int TST = 80;  // tile row stride (bytes): 64 keys + 16, keeps 16-byte row reads aligned
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) unsigned char tile[D * TST];
  const int tid = threadIdx.x, chunk = tid % TPR, rsub = tid / TPR;
  const int bh = blockIdx.x / nkb64, blk = blockIdx.x % nkb64;
  // this thread's keys are PASSES * rsub + p: its bytes of one dimension form one LDS word.
  // The row loads are issued before the head-scale reduction so that the two latencies overlap.
  const bf16* src = V + (size_t)bh * Nk * D;
  u32x4 w[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int key = blk * 64 + PASSES * rsub + p;
    w[p] = u32x4{0u, 0u, 0u, 0u};
    if (key < Nk) w[p] = ld16(src + (size_t)key * D + chunk * 8);
  }
  float am = 0.f;
  for (int i = tid; i < nkb64; i += 256) am = fmaxf(am, vpart[(size_t)bh * nkb64 + i]);
  am = block_max(am, red);
  const float s = am > 0.f ? am / kFp8Max : 1.f;
  const float r = 1.f / s;
  if (blk == 0 && tid == 0) sv[bh] = s;
  uint32_t c[PASSES][2];  // E4M3 codes of dimensions 8 chunk + 0..3 and + 4..7 of key p
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    float x[8], y[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[p][i]);
      x[2 * i + 1] = bf16_hi(w[p][i]);
    }
    scale_by_reciprocal(x, s, r, y);
    c[p][0] = (uint32_t)cvt2_fp8<true>(y[2], y[3], cvt2_fp8<false>(y[0], y[1], 0));
    c[p][1] = (uint32_t)cvt2_fp8<true>(y[6], y[7], cvt2_fp8<false>(y[4], y[5], 0));
  }
  unsigned char* trow = tile + (chunk * 8) * TST + PASSES * rsub;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // byte transpose: lo = [k0.b0, k1.b0, k0.b1, k1.b1], hi = [k0.b2, k1.b2, k0.b3, k1.b3]
    const uint32_t lo01 = __builtin_amdgcn_perm(c[1][h], c[0][h], 0x05010400u);
    const uint32_t hi01 = __builtin_amdgcn_perm(c[1][h], c[0][h], 0x07030602u);
    if constexpr (PASSES == 4) {
      const uint32_t lo23 = __builtin_amdgcn_perm(c[3][h], c[2][h], 0x05010400u);
      const uint32_t hi23 = __builtin_amdgcn_perm(c[3][h], c[2][h], 0x07030602u);
      const uint32_t d[4] = {__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                             __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                             __builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
                             __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
#pragma unroll
      for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t*>(trow + (4 * h + e) * TST) = d[e];
    } else {
      const uint32_t d[2] = {lo01, hi01};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<uint16_t*>(trow + (4 * h + e) * TST) = (uint16_t)(d[e >> 1] >> (16 * (e & 1)));
    }
  }
  __syncthreads();
  const size_t Nkp = (size_t)nkb64 * 64;
  for (int c4 = tid; c4 < D * 4; c4 += 256) {
    const int dim = c4 >> 2, part = c4 & 3;
    const u32x4 val = *reinterpret_cast<const u32x4*>(tile + dim * TST + 16 * part);
    st16(v8t + ((size_t)bh * D + dim) * Nkp + (size_t)blk * 64 + 16 * part, val);
  }
}

// ---------------------------------------------------------------------------------------------
// Forward on the FP8 codes
template <int D>
struct Fp8Lds {
  static constexpr int KST = D + 16;                  // K tile row stride (bytes), rows = keys
  static constexpr int VST = kBC8 + 16;               // V^T tile row stride, rows = dims
  static constexpr int KCPR = KST / 16, VCPR = VST / 16;
  static constexpr int KT = kBC8 * KST, VT = D * VST;
  static constexpr int KC = kBC8 * KCPR, VC = D * VCPR;  // 16-byte chunks per tile
};

// key (0..63) of the tile given to A-operand row i of block b: output register r of lane half h
// is then key 32 h + 16 b + r (see the header).
__device__ __forceinline__ int fp8_key_of_row(int i, int b) {
  return 32 * ((i >> 2) & 1) + 16 * b + 4 * (i >> 3) + (i & 3);
}

// One buffer of scores: the next tile's S^T is formed after this tile's P is packed, over its
// scores. That keeps the kernel within 168 VGPRs, so three 4-wave workgroups share a CU (three
// waves per SIMD) and the softmax of one wave hides under the products of the others; with the
// matrix-core time halved against bf16 the softmax dominates, and this beats two waves per SIMD
// that each overlap the next tile's products with their own softmax (measured, causal B2 H16
// N8192 d128: 0.402 against 0.424 ms for the whole call; 12-wave workgroups 0.431 ms).
template <int D, int NW, bool CAUSAL>
__global__ __attribute__((amdgpu_waves_per_eu(3, 3))) __launch_bounds__(NW * 64) void fwd_fp8_kernel(
    const unsigned char* __restrict__ q8, const unsigned char* __restrict__ k8,
    const unsigned char* __restrict__ v8t, const float* __restrict__ sq,
    const float* __restrict__ sk, const float* __restrict__ sv, bf16* __restrict__ O,
    float* __restrict__ LSE, int BH, int Nq, int Nk, int nqb32, int nkb64, float c) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = Fp8Lds<D>;
  constexpr int BR = NW * 32;
  constexpr int KIW = (L::KC / 64 + NW - 1) / NW, VIW = (L::VC / 64 + NW - 1) / NW;
  static_assert(L::KC % 64 == 0 && L::VC % 64 == 0, "tiles are whole wave copies");
  __shared__ __attribute__((aligned(16))) unsigned char kb0[L::KT];
  __shared__ __attribute__((aligned(16))) unsigned char kb1[L::KT];
  __shared__ __attribute__((aligned(16))) unsigned char vb0[L::VT];
  __shared__ __attribute__((aligned(16))) unsigned char vb1[L::VT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  const int nqt = (Nq + BR - 1) / BR;
  int bh, rank;
  xcd_map(blockIdx.x, BH, 1, (Nq + BR - 1) / BR, 1 << 30, bh, rank);
  const int qt = CAUSAL ? nqt - 1 - rank : rank;
  const int q0 = qt * BR;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;
  const int shift = Nk - Nq;
  const size_t Nkp = (size_t)nkb64 * 64;

  const unsigned char* Kh = k8 + (size_t)bh * Nk * D;
  const unsigned char* Vh = v8t + (size_t)bh * D * Nkp;

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(q0 + BR, Nq) + shift);
  const int ntiles = max(0, (kend + kBC8 - 1) / kBC8);
  const int horizon = CAUSAL ? min(qw + 31, Nq - 1) + shift : Nk - 1;
  const int last_tile = min(ntiles - 1, horizon / kBC8);

  // ---- LDS fill offsets: chunk p of a tile lands at byte 16 p; pad chunks re-read chunk 0
  int koff[KIW], voff[VIW];
#pragma unroll
  for (int i = 0; i < KIW; ++i) {
    const int p = (wave + i * NW) * 64 + lane, row = p / L::KCPR, ch = p % L::KCPR;
    koff[i] = row * D + (ch < D / 16 ? ch : 0) * 16;
  }
#pragma unroll
  for (int i = 0; i < VIW; ++i) {
    const int p = (wave + i * NW) * 64 + lane, row = p / L::VCPR, ch = p % L::VCPR;
    voff[i] = row * (int)Nkp + (ch < kBC8 / 16 ? ch : 0) * 16;
  }
  auto copy_k = [&](int t, unsigned char* dst) {
    const int rows = max(0, Nk - t * kBC8);  // rows past N_k read as zero
    const auto r = make_rsrc(Kh + (size_t)t * kBC8 * D, rows * D);
#pragma unroll
    for (int i = 0; i < KIW; ++i)
      if (wave + i * NW < L::KC / 64) buffer_to_lds(r, dst + (wave + i * NW) * 1024, koff[i]);
  };
  auto copy_v = [&](int t, unsigned char* dst) {
    // the whole head's V^T (padding keys are zero codes); the tile starts at column 64 t
    const auto r = make_rsrc(Vh + (size_t)t * kBC8, (int)(D * Nkp - (size_t)t * kBC8));
#pragma unroll
    for (int i = 0; i < VIW; ++i)
      if (wave + i * NW < L::VC / 64) buffer_to_lds(r, dst + (wave + i * NW) * 1024, voff[i]);
  };

  // ---- Q codes: B operand of S^T, lane (query qi, h) holds dims 64 m + 32 h + 0..31
  i32x8 qf[D / 64];
#pragma unroll
  for (int m = 0; m < D / 64; ++m) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (qi < Nq) {
      const unsigned char* p = q8 + ((size_t)bh * Nq + qi) * D + 64 * m + 32 * hi;
      a = ld16(p);
      b = ld16(p + 16);
    }
    qf[m] = __builtin_bit_cast(i32x8, u32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
  }
  // c s_q: the scale of this wave's 32-row block of Q (uniform per wave)
  const float cq = c * (qw < Nq ? sq[(size_t)bh * nqb32 + (qw >> 5)] : 1.f);
  const float* skh = sk + (size_t)bh * nkb64;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  // A operand row of S^T block b: key fp8_key_of_row(l32, b) of the tile, dims 64 m + 32 h
  const int kr[2] = {fp8_key_of_row(l32, 0) * L::KST + 32 * hi,
                     fp8_key_of_row(l32, 1) * L::KST + 32 * hi};
  auto ld32 = [&](const unsigned char* p) {
    const u32x4 a = ld16(p), b = ld16(p + 16);
    return __builtin_bit_cast(i32x8, u32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
  };
  auto qk = [&](f32x16& s0, f32x16& s1, const unsigned char* kt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
#pragma unroll
    for (int m = 0; m < D / 64; ++m) {
      s0 = mfma_fp8(ld32(kt + kr[0] + 64 * m), qf[m], s0);
      s1 = mfma_fp8(ld32(kt + kr[1] + 64 * m), qf[m], s1);
    }
  };
  const int vr = l32 * L::VST + 32 * hi;  // V^T row (dim 32 db + l32), keys 32 h + 0..31

  auto step = [&](auto PAR, f32x16& sc0, f32x16& sc1, int t) {
    constexpr int P = decltype(PAR)::value;
    wait_vmem();
    __syncthreads();
    if (t + 2 < ntiles) copy_k(t + 2, P ? kb1 : kb0);
    if (t + 1 < ntiles) copy_v(t + 1, P ? vb0 : vb1);
    if (t > last_tile) return;
    const int kbase = t * kBC8;
    const float ct = cq * skh[t];  // scale * log2(e) * s_q * s_k of this tile
    // register r of block b in lane half h holds key kbase + 32 h + 16 b + r
    const bool need_mask = (kbase + kBC8 > Nk) || (CAUSAL && kbase + kBC8 - 1 > qw + shift);
    if (need_mask) {
      const int lim = (CAUSAL ? min(Nk - 1, qi + shift) : Nk - 1) - kbase - 32 * hi;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r > lim) sc0[r] = kNegInf;
        if (16 + r > lim) sc1[r] = kNegInf;
      }
    }
    float ma = fmaxf(fmaxf(sc0[0], sc0[1]), sc0[2]), mb = fmaxf(fmaxf(sc1[0], sc1[1]), sc1[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      ma = fmaxf(fmaxf(ma, sc0[r]), sc0[r + 1]);
      mb = fmaxf(fmaxf(mb, sc1[r]), sc1[r + 1]);
    }
    const float mx = halves_max(fmaxf(fmaxf(ma, sc0[15]), fmaxf(mb, sc1[15]))) * ct;
    if (__any(mx > m_run + kSlack8)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    // 2^8 P: below 2^8.5 because no score exceeds m_run by more than the slack
    const float mo = m_run - kPShift;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc0[r] = exp2_fast(__builtin_fmaf(sc0[r], ct, -mo));
      sc1[r] = exp2_fast(__builtin_fmaf(sc1[r], ct, -mo));
    }
    float ps[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ps[j] = sc0[j] + sc1[j];
#pragma unroll
    for (int r = 4; r < 16; ++r) ps[r & 3] += sc0[r] + sc1[r];
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // B operand of O^T: byte 16 b + r = key 32 h + 16 b + r
    u32x8 pw;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      pw[w] = (uint32_t)cvt2_fp8<true>(sc0[4 * w + 2], sc0[4 * w + 3],
                                       cvt2_fp8<false>(sc0[4 * w], sc0[4 * w + 1], 0));
      pw[4 + w] = (uint32_t)cvt2_fp8<true>(sc1[4 * w + 2], sc1[4 * w + 3],
                                           cvt2_fp8<false>(sc1[4 * w], sc1[4 * w + 1], 0));
    }
    const i32x8 pf = __builtin_bit_cast(i32x8, pw);
    qk(sc0, sc1, P ? kb0 : kb1);  // the next tile's scores, over this one's
    const unsigned char* vt = P ? vb1 : vb0;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      oacc[db] = mfma_fp8(ld32(vt + vr + 32 * db * L::VST), pf, oacc[db]);
  };

  f32x16 sa0, sa1;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  copy_k(0, kb0);
  copy_v(0, vb0);
  if (ntiles > 1) copy_k(1, kb1);
  wait_vmem();
  __syncthreads();
  qk(sa0, sa1, kb0);
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    step(I0(), sa0, sa1, t);
    step(I1(), sa0, sa1, t + 1);
  }
  if (t < ntiles) step(I0(), sa0, sa1, t);

  // ---- epilogue: O = s_v acc / l, L = ln 2 (m - 8 + log2 l)
  const float l_tot = halves_sum(l_run);
  if (qi < Nq) {
    const float inv = sv[bh] / l_tot;
    bf16* orow = O + ((size_t)bh * Nq + qi) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * j + 4 * hi) = w;
      }
    if (hi == 0) LSE[(size_t)bh * Nq + qi] = (m_run - kPShift + log2_fast(l_tot)) * kLn2;
  }
#endif
}

template <int D>
hipError_t launch_d(const Fp8Args& a) {
  const int BH = a.B * a.H;
  const int nqb64 = (a.Nq + 63) / 64, nkb64 = (a.Nk + 63) / 64, nqb32 = (a.Nq + 31) / 32;
  const long long gp = (long long)BH * (nqb64 + 2 * nkb64);
  if (gp > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fp8_prep_kernel<D>), dim3((unsigned)gp), dim3(256), 0, a.stream, a.q, a.k,
                     a.v, a.ws.q8, a.ws.k8, a.ws.sq, a.ws.sk, a.ws.vpart, a.Nq, a.Nk, nqb64, nkb64,
                     nqb32, a.incoherent ? 1 : 0, a.key0, a.key1, (float)(1.0 / __builtin_sqrt((double)D)));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fp8_prep_v_kernel<D>), dim3((unsigned)(BH * nkb64)), dim3(256), 0, a.stream,
                     a.v, a.ws.vpart, a.ws.v8t, a.ws.sv, a.Nk, nkb64);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int NW = 4, BR = NW * 32;  // three workgroups per CU
  const int nqt = (a.Nq + BR - 1) / BR;
  const long long grid = (long long)BH * nqt;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c = a.scale * kLog2e;
  if (a.causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, NW, true>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       a.stream, a.ws.q8, a.ws.k8, a.ws.v8t, a.ws.sq, a.ws.sk, a.ws.sv, a.o,
                       a.lse, BH, a.Nq, a.Nk, nqb32, nkb64, c);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, NW, false>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       a.stream, a.ws.q8, a.ws.k8, a.ws.v8t, a.ws.sq, a.ws.sk, a.ws.sv, a.o,
                       a.lse, BH, a.Nq, a.Nk, nqb32, nkb64, c);
  return hipGetLastError();
}

}  // namespace

Fp8Workspace fp8_workspace_layout(void* base, int B, int H, int Nq, int Nk, int d, size_t* bytes) {
  const size_t BH = (size_t)B * H;
  const size_t nqb32 = (Nq + 31) / 32, nkb64 = (Nk + 63) / 64;
  auto al = [](size_t n) { return (n + 255) & ~size_t(255); };
  size_t off = 0;
  Fp8Workspace w;
  unsigned char* b = static_cast<unsigned char*>(base);
  auto take = [&](size_t n) {
    unsigned char* p = b ? b + off : nullptr;
    off += al(n);
    return p;
  };
  w.q8 = take(BH * Nq * d);
  w.k8 = take(BH * Nk * d);
  w.v8t = take(BH * d * nkb64 * 64);
  w.sq = reinterpret_cast<float*>(take(BH * nqb32 * 4));
  w.sk = reinterpret_cast<float*>(take(BH * nkb64 * 4));
  w.vpart = reinterpret_cast<float*>(take(BH * nkb64 * 4));
  w.sv = reinterpret_cast<float*>(take(BH * 4));
  if (bytes) *bytes = off;
  return w;
}

hipError_t launch_fwd_fp8(const Fp8Args& a) {
  return a.d == 128 ? launch_d<128>(a) : launch_d<64>(a);
}

}  // namespace fa
