// Attention backward for gfx950 (CDNA4): recomputation from the stored log-sum-exp.
//
// Method (page "Bellek Duvarının Fiziği: Standart Attention'dan FlashAttention'a", section
// "Geri Yayılım"): nothing of size N_q x N_k is stored by the forward pass; the backward rebuilds
// each probability tile on chip as P = exp(S - L) from the per-row log-sum-exp L, takes
// D = rowsum(dO * O) from the forward output, and applies the softmax gradient identity
// dS = P * (dP - D) with dP = dO V^T. Then dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K.
//
// Three kernels on one stream:
//   1. bwd_delta:  -D_i = -sum_k dO_ik O_ik, and -L_i / scale (the log-sum-exp in the units of the
//                  unscaled scores q.k), both negated; one pass over O and dO, HBM-bound;
//   2. bwd_dkdv:   one workgroup per (b, h, 128-key tile); each wave keeps 32 keys' K and V
//                  fragments and fp32 dK, dV accumulators in registers and streams the query
//                  tiles (Q, dO, nLs, nD) through LDS;
//   3. bwd_dq:     one workgroup per (b, h, 128-query tile); each wave keeps 32 queries' Q and dO
//                  fragments and an fp32 dQ accumulator in registers and streams K/V tiles.
// Splitting dQ into its own pass recomputes S and dP a second time (7 products where a fused
// kernel would run 5) but needs no atomics, so every gradient is bitwise reproducible.
//
// CDNA4 mapping. All products are v_mfma_f32_32x32x16_bf16. In the dK/dV kernel the score tile
// is S = Q K^T (lane = key, registers = queries) so that P and dS are directly the B operands of
// dV^T = dO^T P and dK^T = Q^T dS, whose A operands (the transposes of the dO and Q tiles) come
// from ds_read_b64_tr_b16. The dQ kernel mirrors the forward: S^T = K Q^T (lane = query), and
// dQ^T = K^T dS^T takes K^T the same way. Tiles are copied HBM/L2 -> LDS by
// buffer_load_dwordx4 ... lds (rows past the end read as zero) into padded rows whose stride makes
// both the 16-byte row reads and the 4-row transposing reads free of bank conflicts, so every LDS
// address is a per-lane base plus a compile-time offset. Tiles are double-buffered, one ahead.
#include "fa_device.h"
#include "fa_launch.h"

#include <algorithm>
#include <type_traits>

namespace fa {
namespace {

constexpr int kNW = 4;  // waves per workgroup
constexpr int kNT = kNW * 64;

// Row stride (bytes) of a [rows][D] bf16 tile read both by 16-byte row reads from 16 rows and by
// 4-row x 32-byte transposing reads: the stride in 4-byte words is 4 mod 8 (16 row reads hit 16
// distinct 16-byte bank groups) and 4 consecutive rows start in disjoint 32-byte windows.
template <int D>
constexpr int dual_stride() { return D == 128 ? 2 * D + 48 : 2 * D + 16; }
// Row stride for tiles read only by 16-byte row reads.
template <int D>
constexpr int row_stride() { return 2 * D + 16; }

// Wave-wide copies that fill a [64][D] bf16 tile with row stride ST: copy p covers 16-byte chunk
// positions 64 p .. 64 p + 63; pad positions re-read chunk 0 of their row.
template <int D, int ST>
struct PaddedTile {
  static constexpr int kCpr = ST / 16;          // chunks per row including pad
  static constexpr int kCopies = 64 * kCpr / 64;
  static constexpr int kPerWave = (kCopies + kNW - 1) / kNW;
  static constexpr int kBytes = 64 * ST;
  int off[kPerWave];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int p = (wave + i * kNW) * 64 + lane, row = p / kCpr, ch = p % kCpr;
      off[i] = row * D * 2 + (ch < D / 8 ? ch : 0) * 16;
    }
  }
  // rows [row0, row0 + 64) of a [nrows][D] tensor starting at base (rows past nrows read as
  // zero; one head spans fewer than 2^31 bytes, which the host checks)
  __device__ __forceinline__ void copy(const bf16* base, int row0, int nrows, unsigned char* dst,
                                      int wave) const {
    const auto r = make_rsrc(base + (size_t)row0 * D, max(0, nrows - row0) * D * 2);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      if (wave + i * kNW < kCopies) buffer_to_lds(r, dst + (wave + i * kNW) * 1024, off[i]);
  }
};

// 64 floats (rows [row0, row0 + 64) of a [nrows] fp32 vector) -> LDS by the 16 first lanes.
__device__ __forceinline__ void copy_row_vec(const float* base, int row0, int nrows,
                                             unsigned char* dst, int lane) {
  if (lane < 16) {
    const auto r = make_rsrc(base + row0, max(0, nrows - row0) * 4);
    buffer_to_lds(r, dst, lane * 16);
  }
}

// Store an fp32 accumulator tile held as X^T (lane = sequence row, registers = dims
// 32 db + 8 j + 4 h + i) to one bf16 row of a [.][D] tensor, multiplied by `mul`.
template <int D>
__device__ __forceinline__ void store_row(bf16* dst_row, const f32x16 (&acc)[D / 32], float mul,
                                          int hi) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[db][4 * j] * mul, acc[db][4 * j + 1] * mul);
      w[1] = pack_bf16x2(acc[db][4 * j + 2] * mul, acc[db][4 * j + 3] * mul);
      *reinterpret_cast<u32x2*>(dst_row + db * 32 + 8 * j + 4 * hi) = w;
    }
}

template <int D>
__device__ __forceinline__ void store_zero_row(bf16* dst_row, int hi) {
  const u32x2 z = {0u, 0u};
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(dst_row + db * 32 + 8 * j + 4 * hi) = z;
}

// The same rows in fp32 (partial sums that a later kernel adds up); live = false stores zeros.
template <int D>
__device__ __forceinline__ void store_row_f32(float* dst_row, const f32x16 (&acc)[D / 32],
                                              float mul, bool live, int hi) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = live ? acc[db][4 * j + e] * mul : 0.f;
      *reinterpret_cast<f32x4*>(dst_row + db * 32 + 8 * j + 4 * hi) = w;
    }
}

// Per-lane base offset of the ds_read_b64_tr_b16 pair that assembles a transposed 16-row x
// 32-column block of a tile with row stride ST: within each group of 16 lanes, input lane j reads
// row 8 h + (j >> 2), columns 16 (group & 1) + 4 (j & 3).
template <int ST>
__device__ __forceinline__ int tr_base(int lane) {
  const int j = lane & 15, grp = lane >> 4;
  return (8 * (grp >> 1) + (j >> 2)) * ST + (16 * (grp & 1) + 4 * (j & 3)) * 2;
}

// ---------------------------------------------------------------------------------------------
// 1. nD = -rowsum(dO * O) and nLs = -L / scale.
// Both are stored negated and in the units of the unscaled scores so that the dK/dV kernel can
// start its score and dP accumulators at them: S - L/scale and dP - D then leave the matrix cores
// directly, and P = exp2(c (S - L/scale)), dS = P (dP - D) take one multiply each.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const bf16* __restrict__ O,
                                                        const bf16* __restrict__ dO,
                                                        const float* __restrict__ LSE,
                                                        float* __restrict__ ndelta,
                                                        float* __restrict__ nls, int rows,
                                                        float inv_scale) {
  constexpr int G = D / 8;      // lanes per row
  constexpr int RPB = 256 / G;  // rows per block pass
  const int g = threadIdx.x / G, gl = threadIdx.x % G;
  for (int row = blockIdx.x * RPB + g; row < rows; row += gridDim.x * RPB) {
    const u32x4 a = ld16_nt(O + (size_t)row * D + gl * 8);
    const u32x4 b = ld16_nt(dO + (size_t)row * D + gl * 8);
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t aw = a[w], bw = b[w];
      s = __builtin_fmaf(bf16_lo(aw), bf16_lo(bw), s);
      s = __builtin_fmaf(bf16_hi(aw), bf16_hi(bw), s);
    }
    s = group_sum<G>(s);
    if (gl == 0) {
      ndelta[row] = -s;
      // a row that saw no key (LSE = -inf) gets nLs = -inf, so that every probability the
      // backward rebuilds for it is exp2(c (S - inf)) = 0
      const float l = LSE[row];
      nls[row] = l == kNegInf ? kNegInf : -l * inv_scale;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// 2. dK, dV
constexpr int kBKV = 128;  // keys per workgroup (32 per wave)
constexpr int kBQ = 64;    // queries per streamed tile

template <int D, int DV>
struct DkdvLds {
  static constexpr int ST = dual_stride<D>(), STO = dual_stride<DV>();
  using Tile = PaddedTile<D, ST>;     // Q
  using TileO = PaddedTile<DV, STO>;  // dO
  // one buffer: Q tile, dO tile, nLs and nD of its 64 rows
  static constexpr int kQ = 0, kDO = Tile::kBytes, kL = kDO + TileO::kBytes, kDl = kL + kBQ * 4;
  static constexpr int kBuf = kDl + kBQ * 4;
};

// VL: per-sequence lengths lens_q[b] <= Nq, lens_k[b] <= Nk inside the padded tensors; the
// gradients of padding rows are zero.
// DROP: dropout on P, regenerated from the forward's seed and offset: dV = (P Z)^T dO / (1 - p),
// dS = P (Z dP / (1 - p) - D).
// MODE: kDkDv computes both; kDvOnly / kDkOnly one of them (two launches then cover the
// gradients with fewer live registers: the dropout's generator work does not fit beside both
// sets of accumulators at d = 128).
// BIAS: the forward's additive bias is added again when P is rebuilt (no gradient is formed for
// the bias itself).
// DV: head dimension of V, dO and dV (the notation's d_v; the same as D unless asked otherwise).
constexpr int kDkDv = 0, kDvOnly = 1, kDkOnly = 2;
template <int D, bool CAUSAL, bool VL, bool DROP, int MODE, bool BIAS, int DV = D>
__global__ __attribute__((amdgpu_waves_per_eu(2, 2))) __launch_bounds__(kNT) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ NLs, const float* __restrict__ ND,
    bf16* __restrict__ dK, bf16* __restrict__ dV, const int* __restrict__ lens_q,
    const int* __restrict__ lens_k, int BH, int H, int G, int GL, float* __restrict__ pK,
    float* __restrict__ pV, int Nq, int Nk, float c, float scale, DropoutParams drop,
    BiasParams bias, int hg) {
#if defined(__HIP_DEVICE_COMPILE__)
  using SM = DkdvLds<D, DV>;
  constexpr int ST = SM::ST, STO = SM::STO;
  // one array per buffer, so that the LDS copies into one buffer provably do not alias the reads
  // of the other and need no wait before those reads
  __shared__ __attribute__((aligned(16))) unsigned char buf0[SM::kBuf];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[SM::kBuf];
  // DROP: per-wave staging (64 bytes) that hands the keep bits from lane = query row to
  // lane = key
  __shared__ __attribute__((aligned(16))) unsigned char xbuf[DROP ? 4 * 64 : 16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // The workgroup's unit u and key tile: query heads u GL .. u GL + GL - 1, which read K/V head
  // kvbh = u GL / G (G query heads per K/V head; G = 1 without grouped query heads). With
  // GL = G the unit is the whole group and the K/V gradients sum over its heads here; with
  // GL = 1 (pK != nullptr) each query head's contribution goes to fp32 partial rows pK, pV
  // (row bh of [B H, N_k]) that bwd_gqa_reduce_kernel adds up.
  int u, rank;
  xcd_map(blockIdx.x, BH / GL, G / GL, (Nk + kBKV - 1) / kBKV, hg, u, rank);
  const int kvbh = u * GL / G;
  const int bseq = u * GL / H;  // batch index
  const int k0 = rank * kBKV;  // causal: low key tiles see the most queries and go first
  const int kw = k0 + wave * 32;
  const int key = kw + l32;
  const int nq = VL ? min(max(lens_q[bseq], 0), Nq) : Nq;  // valid lengths of this sequence
  const int nk = VL ? min(max(lens_k[bseq], 0), Nk) : Nk;
  const int shift = nk - nq;  // causal: key j visible to query i iff j <= i + shift

  // the query head being streamed, and its rows (set per head below)
  int bh = u * GL;
  const bf16* Qh = Q;
  const bf16* dOh = dO;
  const float* Lh = NLs;
  const float* Dh = ND;

  // resident B operands: K^T and V^T columns (lane = key, 8 dims per k-step)
  bf16x8 kf[D / 16], vf[DV / 16];
  if constexpr (D == DV) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key < nk) {
        a = ld16(K + ((size_t)kvbh * Nk + key) * D + ks * 16 + hi * 8);
        b = ld16(V + ((size_t)kvbh * Nk + key) * D + ks * 16 + hi * 8);
      }
      kf[ks] = as_bf16x8(a);
      vf[ks] = as_bf16x8(b);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u};
      if (key < nk) a = ld16(K + ((size_t)kvbh * Nk + key) * D + ks * 16 + hi * 8);
      kf[ks] = as_bf16x8(a);
    }
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks) {
      u32x4 b = {0u, 0u, 0u, 0u};
      if (key < nk) b = ld16(V + ((size_t)kvbh * Nk + key) * DV + ks * 16 + hi * 8);
      vf[ks] = as_bf16x8(b);
    }
  }
  f32x16 dk[D / 32], dv[DV / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[db][r] = 0.f;
#pragma unroll
  for (int db = 0; db < DV / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[db][r] = 0.f;

  // query tiles that can see any key of this workgroup; the first ones (causal) cross the
  // diagonal of some wave and are masked, from tm on every query sees every key of the workgroup
  const int t0 = CAUSAL ? max(0, k0 - shift) / kBQ : 0;
  const int t1 = (VL && k0 >= nk) ? t0 : (nq + kBQ - 1) / kBQ;  // no valid key: nothing to do
  int tm = t0;
  if (CAUSAL) tm = min(t1, max(t0, (k0 + kBKV - 1 - shift + kBQ - 1) / kBQ));

  typename SM::Tile tile;
  typename SM::TileO tileo;
  tile.init(wave, lane);
  if constexpr (D != DV) tileo.init(wave, lane);
  auto copy = [&](int t, unsigned char* b) {
    // the wave index passes through an empty asm so that the copies' LDS addresses and wave
    // conditions are formed here, per tile, from one register: hoisted out of the loop they
    // would hold a score of scalar registers for the whole kernel and push live values into
    // scratch memory
    int w = wave;
    asm volatile("" : "+s"(w));
    const int q0 = t * kBQ;
    tile.copy(Qh, q0, nq, b + SM::kQ, w);
    if constexpr (D == DV)
      tile.copy(dOh, q0, nq, b + SM::kDO, w);
    else
      tileo.copy(dOh, q0, nq, b + SM::kDO, w);
    if (w == 0) copy_row_vec(Lh, q0, nq, b + SM::kL, lane);
    if (w == 1) copy_row_vec(Dh, q0, nq, b + SM::kDl, lane);
  };
  // rows past N_q read as zero: their Q and dO rows are zero and nLs = nD = 0, so P = 1, dP = 0
  // and dS = 0: they add nothing to dK or dV.

  const int qrow = key_of_row(l32) * ST + hi * 16;  // A operand of S and dP: row reads
  const int trb = tr_base<ST>(lane);                 // A operand of dV^T and dK^T: transposed
  const int orow = key_of_row(l32) * STO + hi * 16;  // the same for the dO tile (DV != D)
  const int trbo = tr_base<STO>(lane);

  // One query tile t from buffer P; the copies of tile t+1 go to the other buffer. MASKED: tiles
  // that cross the causal diagonal of some wave (a wave whose keys all lie past the tile skips it).
  // BIAS: the bias of key `key` for the 16 queries of a 32-query block. Read row-wise: lane
  // (x = l32 & 7, group g = l32 >> 3, hi) loads 16 bytes, the 8 keys of its group, of query rows
  // 8 hi + x and 16 + 8 hi + x of the block; an 8 x 8 transpose of 16-bit values inside each
  // group of 8 lanes then hands lane x its key's values of those 8 + 8 rows, as bf16 pairs.
  auto brs = bias_rsrc(bias.ptr, Nq, Nk, bias.sq);  // set per query head below
  auto load_bias = [&](int t, int qb, u32x4 (&raw)[2]) {
    const int kg = kw + 8 * (l32 >> 3);  // first key of the lane's group
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = t * kBQ + qb * 32 + 16 * j + 8 * hi + (l32 & 7);
      u32x4 w = {0u, 0u, 0u, 0u};
      const int off = (int)(((long long)row * bias.sq + kg) * 2);
      if (row < nq && kg + 8 <= nk) {
        w = bias_ld16(brs, off);
      } else if (row < nq && kg < nk) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kg + e < nk) w[e >> 1] |= bias_ld2(brs, off + 2 * e, 0) << (16 * (e & 1));
      }
      raw[j] = w;
    }
  };
  // 8 x 8 transpose of 16-bit values across the 8 lanes x of a group: in, lane x holds row x
  // (word m = columns 2m, 2m + 1); out, lane x holds column x (word m = rows 2m, 2m + 1).
  const int tx = l32 & 7;
  auto transpose8 = [&](u32x4 w) {
    // stage 1: column bit 2 <-> row bit 2 (lane distance 4), 2-word halves
    {
      const bool b = tx & 4;
      const uint32_t s0 = b ? w[0] : w[2], s1 = b ? w[1] : w[3];
      const uint32_t r0 = lane_xor<4>(s0), r1 = lane_xor<4>(s1);
      if (b) { w[0] = r0; w[1] = r1; } else { w[2] = r0; w[3] = r1; }
    }
    // now word 2 a + m holds rows (lane's row with bit 2 = a), columns 4 (tx >> 2) + 2 m, + 1
    // stage 2: column bit 1 <-> row bit 1 (lane distance 2), single words
    {
      const bool b = tx & 2;
      const uint32_t s0 = b ? w[0] : w[1], s1 = b ? w[2] : w[3];
      const uint32_t r0 = lane_xor<2>(s0), r1 = lane_xor<2>(s1);
      if (b) { w[0] = r0; w[2] = r1; } else { w[1] = r0; w[3] = r1; }
    }
    // now word 2 a + c holds rows (bit 2 = a, bit 1 = c, bit 0 = tx & 1), columns
    // 4 (tx >> 2) + 2 ((tx >> 1) & 1), + 1
    // stage 3: column bit 0 <-> row bit 0 (lane distance 1), 16-bit halves
    const bool b = tx & 1;
    // send the halves the partner needs: column (tx ^ 1), i.e. half (1 - b) of each word
    const uint32_t s0 = b ? __builtin_amdgcn_perm(w[1], w[0], 0x05040100u)   // lo halves
                          : __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);  // hi halves
    const uint32_t s1 = b ? __builtin_amdgcn_perm(w[3], w[2], 0x05040100u)
                          : __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
    const uint32_t r0 = lane_xor<1>(s0), r1 = lane_xor<1>(s1);
    // r0 = (partner's half for word 0, for word 1), r1 likewise for words 2, 3: rows with bit 0
    // = 1 - b. Word m of the result: rows 2 m (low half) and 2 m + 1 (high half).
    u32x4 o;
    const uint32_t keep0 = b ? __builtin_amdgcn_perm(w[1], w[0], 0x07060302u)
                             : __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
    const uint32_t keep1 = b ? __builtin_amdgcn_perm(w[3], w[2], 0x07060302u)
                             : __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
    // keepK / rK hold (value for word 2K, value for word 2K + 1) in (lo, hi)
    const uint32_t ev0 = b ? r0 : keep0, od0 = b ? keep0 : r0;  // rows with bit 0 = 0 / = 1
    const uint32_t ev1 = b ? r1 : keep1, od1 = b ? keep1 : r1;
    o[0] = __builtin_amdgcn_perm(od0, ev0, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(od0, ev0, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(od1, ev1, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(od1, ev1, 0x07060302u);
    return o;
  };
  u32x4 bwn[2];

  auto step = [&](auto PAR, auto MASKED, int t) {
    constexpr int P = decltype(PAR)::value;
    constexpr bool MK = decltype(MASKED)::value;
    const unsigned char* b = P ? buf1 : buf0;
    const unsigned char* qt = b + SM::kQ;
    const unsigned char* ot = b + SM::kDO;
    const float* ls = reinterpret_cast<const float*>(b + SM::kL);
    const float* dls = reinterpret_cast<const float*>(b + SM::kDl);
    wait_vmem();
    __syncthreads();
    if (t + 1 < t1) copy(t + 1, P ? buf0 : buf1);
    const int q0 = t * kBQ;
    // every query of the tile is before this wave's first visible position: nothing to do
    if (MK && min(q0 + kBQ, nq) - 1 + shift < kw) return;
#pragma unroll
    for (int qb = 0; qb < kBQ / 32; ++qb) {
      // keep the two 32-query blocks apart: overlapping them would double the live scores and
      // push the register allocator into copying through AGPRs
      __builtin_amdgcn_sched_barrier(0);
      // DROP: keep bits of the 8 x 8 (query, key) blocks of this lane's key group: half h covers
      // queries q0 + 32 qb + 16 h + 8 hi + 0..7 (byte e = query e, bit x = key 8 (l32 >> 3) + x).
      u32x2 mbits[2];
      if constexpr (DROP) {
        // Lane (x = l32 & 7, group l32 >> 3, hi) draws the call of query row 16 h + 8 hi + x and
        // key group (kw >> 3) + (l32 >> 3), turns its eight numbers into eight keep bits and
        // stores them as byte x of the group's 8-byte block in LDS; every lane of the group then
        // reads the whole block (its key's bits are bit x of each byte).
        const int x = l32 & 7;
        typedef __attribute__((address_space(3))) unsigned char lds_u8;
        lds_u8* xb = (lds_u8*)xbuf + wave * 64 + ((l32 >> 3) * 2 + hi) * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w = philox4x32_10((uint32_t)(kw >> 3) + (uint32_t)(l32 >> 3),
                                        (uint32_t)(q0 + qb * 32 + 16 * h + 8 * hi + x),
                                        (uint32_t)bh, drop.offset, drop.key0, drop.key1);
          uint32_t bits = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t u = (k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFFu);
            bits |= (u < drop.thresh ? 1u : 0u) << k;
          }
          xb[x] = (unsigned char)bits;
          mbits[h] = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(xb);
        }
      }
      // BIAS: the bias of this lane's key for the 16 queries of its registers, as bf16 pairs.
      // In the unmasked loop it is prefetched one 32-query block ahead (an HBM latency is longer
      // than one block's products); the few diagonal tiles load their own.
      uint32_t bw[8];
      if constexpr (BIAS) {
        u32x4 raw[2];
        if (MK || (qb == 0 && t == tm)) {
          load_bias(t, qb, raw);
        } else {
          raw[0] = bwn[0];
          raw[1] = bwn[1];
        }
        if (!MK) {
          if (qb == 0) load_bias(t, 1, bwn);
          else if (t + 1 < t1) load_bias(t + 1, 0, bwn);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4 c = transpose8(raw[j]);  // rows 16 j + 8 hi + 0..7 of the lane's key
#pragma unroll
          for (int m = 0; m < 4; ++m) bw[4 * j + m] = c[m];
        }
      }
      // the accumulators start at -L/scale and (without dropout) -D of their query rows, so the
      // products leave S - L/scale and dP - D; register r holds query
      // qb*32 + key_of_reg(r, hi) = qb*32 + 16 (r >> 3) + 8 hi + (r & 7)
      f32x16 s, dp;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qi0 = qb * 32 + 16 * half + 8 * hi;
        const f32x4 la = *reinterpret_cast<const f32x4*>(ls + qi0);
        const f32x4 lb = *reinterpret_cast<const f32x4*>(ls + qi0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[8 * half + e] = la[e];
          s[8 * half + 4 + e] = lb[e];
        }
        if constexpr (DROP) {
#pragma unroll
          for (int e = 0; e < 8; ++e) dp[8 * half + e] = 0.f;
        } else {
          const f32x4 da = *reinterpret_cast<const f32x4*>(dls + qi0);
          const f32x4 db4 = *reinterpret_cast<const f32x4*>(dls + qi0 + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dp[8 * half + e] = da[e];
            dp[8 * half + 4 + e] = db4[e];
          }
        }
      }
      if constexpr (D == DV) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const int off = qrow + qb * 32 * ST + ks * 32;
          s = mfma32(as_bf16x8(ld16(qt + off)), kf[ks], s);
          dp = mfma32(as_bf16x8(ld16(ot + off)), vf[ks], dp);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
          s = mfma32(as_bf16x8(ld16(qt + qrow + qb * 32 * ST + ks * 32)), kf[ks], s);
#pragma unroll
        for (int ks = 0; ks < DV / 16; ++ks)
          dp = mfma32(as_bf16x8(ld16(ot + orow + qb * 32 * STO + ks * 32)), vf[ks], dp);
      }
      // queries of register r: qb*32 + key_of_reg(r, hi) = qb*32 + 16 (r >> 3) + 8 hi + (r & 7)
      if (MK) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key > q0 + qb * 32 + key_of_reg(r, hi) + shift) s[r] = kNegInf;
      }
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x4 da, db4;  // DROP: -D of the rows, applied after the mask
        if constexpr (DROP) {
          const int qi0 = qb * 32 + 16 * half + 8 * hi;
          da = *reinterpret_cast<const f32x4*>(dls + qi0);
          db4 = *reinterpret_cast<const f32x4*>(dls + qi0 + 4);
        }
        float p[8], ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * half + e;
          float x = s[r] * c;  // log2 units: c (S - L/scale)
          if constexpr (BIAS) {
            const uint32_t w = bw[r >> 1];
            x = __builtin_fmaf((r & 1) ? bf16_hi(w) : bf16_lo(w), kLog2e, x);
          }
          const float pv = exp2_fast(x);
          if constexpr (DROP) {
            // bit x of byte e: 0 or all ones after the sign-extending extract
            const uint32_t km = (uint32_t)__builtin_amdgcn_sbfe(
                (int)mbits[half][e >> 2], 8 * (e & 3) + (l32 & 7), 1);
            p[e] = __uint_as_float(__float_as_uint(pv) & km);
            ds[e] = pv * __builtin_fmaf(__uint_as_float(__float_as_uint(drop.inv_keep) & km),
                                         dp[r], e < 4 ? da[e] : db4[e - 4]);
          } else {
            p[e] = pv;
            ds[e] = pv * dp[r];
          }
        }
        pf[half] = pack_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        dsf[half] = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS (A operands: transposed 32-dim x 16-query blocks)
      if constexpr (D == DV) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const int off = trb + (qb * 32 + 16 * st) * ST + db * 64;
            dv[db] = mfma32(lds_read_tr_pair(ot + off, 4 * ST), pf[st], dv[db]);
            dk[db] = mfma32(lds_read_tr_pair(qt + off, 4 * ST), dsf[st], dk[db]);
          }
      } else {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int db = 0; db < DV / 32; ++db)
            dv[db] = mfma32(lds_read_tr_pair(ot + trbo + (qb * 32 + 16 * st) * STO + db * 64,
                                             4 * STO), pf[st], dv[db]);
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
            dk[db] = mfma32(lds_read_tr_pair(qt + trb + (qb * 32 + 16 * st) * ST + db * 64,
                                             4 * ST), dsf[st], dk[db]);
        }
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using BT = std::integral_constant<bool, true>;
  using BF = std::integral_constant<bool, false>;

  for (int g = 0; g < GL; ++g) {
    bh = u * GL + g;
    Qh = Q + (size_t)bh * Nq * D;
    dOh = dO + (size_t)bh * Nq * DV;
    Lh = NLs + (size_t)bh * Nq;
    Dh = ND + (size_t)bh * Nq;
    if constexpr (BIAS)
      brs = bias_rsrc(bias.ptr + (long long)(bh / H) * bias.sb + (long long)(bh % H) * bias.sh,
                      Nq, Nk, bias.sq);
    if (g > 0) __syncthreads();  // every wave is done with the previous head's last tile
    if (t0 < t1) copy(t0, buf0);
    // buffer of tile t: (t - t0) & 1
    int t = t0;
    for (; t + 1 < tm; t += 2) {
      step(I0(), BT(), t);
      step(I1(), BT(), t + 1);
    }
    if (t < tm) {
      step(I0(), BT(), t);
      ++t;
      if (t < t1) step(I1(), BF(), t++);
    }
    for (; t + 1 < t1; t += 2) {
      step(I0(), BF(), t);
      step(I1(), BF(), t + 1);
    }
    if (t < t1) step(I0(), BF(), t);
  }

  // (in a one-gradient mode the other gradient's products are dead code and compile away)
  // one query head's partial rows, zero past the sequence's keys (the launcher passes
  // pK = nullptr to the variants with a bias or a V head dimension of its own)
  constexpr bool kPartialOk = !BIAS && D == DV;
  if (kPartialOk && pK != nullptr) {
    if (key < Nk) {
      const bool live = key < nk;
      if (MODE != kDvOnly) store_row_f32<D>(pK + ((size_t)bh * Nk + key) * D, dk, scale, live, hi);
      if (MODE != kDkOnly)
        store_row_f32<DV>(pV + ((size_t)bh * Nk + key) * DV, dv, DROP ? drop.inv_keep : 1.f,
                          live, hi);
    }
  } else if (key < nk) {
    if (MODE != kDvOnly) store_row<D>(dK + ((size_t)kvbh * Nk + key) * D, dk, scale, hi);
    if (MODE != kDkOnly)
      store_row<DV>(dV + ((size_t)kvbh * Nk + key) * DV, dv, DROP ? drop.inv_keep : 1.f, hi);
  } else if (VL && key < Nk) {  // padding keys
    store_zero_row<D>(dK + ((size_t)kvbh * Nk + key) * D, hi);
    store_zero_row<DV>(dV + ((size_t)kvbh * Nk + key) * DV, hi);
  }
#endif
}

// ---------------------------------------------------------------------------------------------
// 2b. Grouped query heads with partial rows: dK, dV of K/V head kvbh = the sums of the fp32
// partial rows of its G query heads kvbh G .. kvbh G + G - 1, in that order, rounded to bf16.
// HBM-bound: each thread reads 8 elements of G rows of pK and pV and writes 16 bytes of each.
template <int D>
__global__ __launch_bounds__(256) void bwd_gqa_reduce_kernel(const float* __restrict__ pK,
                                                             const float* __restrict__ pV,
                                                             bf16* __restrict__ dK,
                                                             bf16* __restrict__ dV, int G, int Nk,
                                                             long long rows) {
  constexpr int LPR = D / 8;  // threads per row
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < rows * LPR;
       idx += (long long)gridDim.x * 256) {
    const long long row = idx / LPR;
    const int c8 = (int)(idx % LPR) * 8;
    const long long kvbh = row / Nk, j = row % Nk;
    float sk[8], sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.f;
    for (int g = 0; g < G; ++g) {
      const size_t off = ((size_t)(kvbh * G + g) * Nk + j) * D + c8;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(pK + off);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(pK + off + 4);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(pV + off);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(pV + off + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sk[e] += a0[e];
        sk[4 + e] += a1[e];
        sv[e] += b0[e];
        sv[4 + e] += b1[e];
      }
    }
    u32x4 wk, wv;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wk[w] = pack_bf16x2(sk[2 * w], sk[2 * w + 1]);
      wv[w] = pack_bf16x2(sv[2 * w], sv[2 * w + 1]);
    }
    st16(dK + row * D + c8, wk);
    st16(dV + row * D + c8, wv);
  }
}

// ---------------------------------------------------------------------------------------------
// 3. dQ
constexpr int kBR = 128;  // queries per workgroup (32 per wave)
constexpr int kBC = 64;   // keys per streamed tile

template <int D, int DV>
struct DqLds {
  static constexpr int KST = dual_stride<D>(), VST = row_stride<DV>();
  using KTile = PaddedTile<D, KST>;
  using VTile = PaddedTile<DV, VST>;
};

template <int D, bool CAUSAL, bool VL, bool DROP, bool BIAS, int DV = D>
__global__ __attribute__((amdgpu_waves_per_eu(2, 2))) __launch_bounds__(kNT) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ NLs, const float* __restrict__ ND,
    bf16* __restrict__ dQ, const int* __restrict__ lens_q, const int* __restrict__ lens_k,
    int BH, int H, int G, int Nq, int Nk, float c, float scale, DropoutParams drop,
    BiasParams bias, int hg) {
#if defined(__HIP_DEVICE_COMPILE__)
  using SM = DqLds<D, DV>;
  // one array per buffer: the LDS copies into one buffer then provably do not alias the reads of
  // the other, so no wait for the copies in flight is needed before those reads
  __shared__ __attribute__((aligned(16))) unsigned char kb0[SM::KTile::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char kb1[SM::KTile::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char vb0[SM::VTile::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char vb1[SM::VTile::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  const int nqt = (Nq + kBR - 1) / kBR;
  int bh, rank;
  xcd_map(blockIdx.x, BH, G, (Nq + kBR - 1) / kBR, hg, bh, rank);
  const int qt = CAUSAL ? nqt - 1 - rank : rank;
  const int q0 = qt * kBR;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;
  const int nq = VL ? min(max(lens_q[bh / H], 0), Nq) : Nq;  // valid lengths of this sequence
  const int nk = VL ? min(max(lens_k[bh / H], 0), Nk) : Nk;
  const int shift = nk - nq;

  const bf16* Kh = K + (size_t)(bh / G) * Nk * D;  // K/V head of this query head
  const bf16* Vh = V + (size_t)(bh / G) * Nk * DV;

  // resident B operands: Q^T and dO^T columns (lane = query)
  bf16x8 qf[D / 16], dof[DV / 16];
  if constexpr (D == DV) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (qi < nq) {
        a = ld16(Q + ((size_t)bh * Nq + qi) * D + ks * 16 + hi * 8);
        b = ld16(dO + ((size_t)bh * Nq + qi) * D + ks * 16 + hi * 8);
      }
      qf[ks] = as_bf16x8(a);
      dof[ks] = as_bf16x8(b);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u};
      if (qi < nq) a = ld16(Q + ((size_t)bh * Nq + qi) * D + ks * 16 + hi * 8);
      qf[ks] = as_bf16x8(a);
    }
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks) {
      u32x4 b = {0u, 0u, 0u, 0u};
      if (qi < nq) b = ld16(dO + ((size_t)bh * Nq + qi) * DV + ks * 16 + hi * 8);
      dof[ks] = as_bf16x8(b);
    }
  }
  // this lane's row: L in log2 units (+inf for a row that saw no key) and -D
  const float lq = qi < nq ? -c * NLs[(size_t)bh * Nq + qi] : 0.f;
  const float nd = qi < nq ? ND[(size_t)bh * Nq + qi] : 0.f;

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  int kend = nk;
  if (CAUSAL) kend = min(nk, min(q0 + kBR, nq) + shift);
  if (VL && q0 >= nq) kend = 0;  // every row of the workgroup is padding
  const int ntiles = max(0, (kend + kBC - 1) / kBC);
  const int horizon = CAUSAL ? min(qw + 31, nq - 1) + shift : nk - 1;
  // leading tiles that need no mask for any row of the workgroup: below the key length, and
  // (causal) every key at or before the first row's diagonal
  int nfull = nk / kBC;
  if (CAUSAL) nfull = min(nfull, max(0, q0 + shift + 1) / kBC);
  nfull = min(nfull, ntiles);

  typename SM::KTile ktile;
  typename SM::VTile vtile;
  ktile.init(wave, lane);
  vtile.init(wave, lane);
  const int krow = key_of_row(l32);
  const int kro = krow * SM::KST + hi * 16, vro = krow * SM::VST + hi * 16;
  const int trb = tr_base<SM::KST>(lane);
  const int lim = CAUSAL ? min(nk - 1, qi + shift) : nk - 1;

  // One key tile t from buffer P (K tile kt, V tile vt); the copies of tile t+1 go to the other
  // buffer. MASKED: tiles on the causal diagonal or past N_k; waves whose rows see no key of the
  // tile skip it.
  auto step = [&](auto PAR, auto MASKED, int t) {
    constexpr int P = decltype(PAR)::value;
    constexpr bool MK = decltype(MASKED)::value;
    const unsigned char* kt = P ? kb1 : kb0;
    const unsigned char* vt = P ? vb1 : vb0;
    wait_vmem();
    __syncthreads();
    if (t + 1 < ntiles) {
      int w = wave;  // formed per tile, as in the dK/dV kernel
      asm volatile("" : "+s"(w));
      ktile.copy(Kh, (t + 1) * kBC, nk, P ? kb0 : kb1, w);
      vtile.copy(Vh, (t + 1) * kBC, nk, P ? vb0 : vb1, w);
    }
    const int kbase = t * kBC;
    if (MK && kbase > horizon) return;
    // BIAS: keys kbase + 32 kb + 16 tt + 8 hi + 0..7 of this lane's query row, issued before the
    // products
    u32x4 bv[4];
    if constexpr (BIAS) {
      const auto brs = bias_rsrc(
          bias.ptr + (long long)(bh / H) * bias.sb + (long long)(bh % H) * bias.sh, Nq, Nk,
          bias.sq);
      const int boff = (int)((long long)min(qi, Nq - 1) * bias.sq * 2);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = kbase + 16 * g + 8 * hi;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qi < nq && j0 + 8 <= nk) {
          w = bias_ld16(brs, boff + 2 * j0);
        } else if (qi < nq && j0 < nk) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (j0 + e < nk) w[e >> 1] |= bias_ld2(brs, boff + 2 * (j0 + e), 0) << (16 * (e & 1));
        }
        bv[g] = w;
      }
    }
    // dP^T starts at -D, so the products leave dP - D (not with dropout, where D is subtracted
    // after the mask, nor with a bias or d_v != d, where the early live range would not fit the
    // registers)
    constexpr bool fold_d = !DROP && !BIAS && D == DV;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb][r] = 0.f;
        dp[kb][r] = fold_d ? nd : 0.f;
      }
    if constexpr (D == DV) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = mfma32(as_bf16x8(ld16(kt + kro + kb * 32 * SM::KST + ks * 32)), qf[ks], s[kb]);
          dp[kb] = mfma32(as_bf16x8(ld16(vt + vro + kb * 32 * SM::VST + ks * 32)), dof[ks], dp[kb]);
        }
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[kb] = mfma32(as_bf16x8(ld16(kt + kro + kb * 32 * SM::KST + ks * 32)), qf[ks], s[kb]);
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          dp[kb] = mfma32(as_bf16x8(ld16(vt + vro + kb * 32 * SM::VST + ks * 32)), dof[ks], dp[kb]);
    }
    if (MK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + kb * 32 + key_of_reg(r, hi) > lim) s[kb][r] = kNegInf;
    }
    bf16x8 dsf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float ds[16];
      // DROP: registers 8 tt .. 8 tt + 7 hold keys kbase + 32 kb + 16 tt + 8 hi + 0..7, the
      // eight keys of one generator call
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 mw;
        if constexpr (DROP)
          mw = philox4x32_10((uint32_t)(kbase >> 3) + (uint32_t)(4 * kb + 2 * tt + hi),
                             (uint32_t)qi, (uint32_t)bh, drop.offset, drop.key0, drop.key1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * tt + e;
          float lr = -lq;
          if constexpr (BIAS) {
            const uint32_t w = bv[2 * kb + tt][e >> 1];
            lr = __builtin_fmaf((e & 1) ? bf16_hi(w) : bf16_lo(w), kLog2e, lr);
          }
          const float pv = exp2_fast(__builtin_fmaf(s[kb][r], c, lr));
          if constexpr (DROP) {
            const float z = keep_factor(mw[e >> 1], e & 1, drop.thresh, drop.inv_keep);
            ds[r] = pv * __builtin_fmaf(z, dp[kb][r], nd);
          } else {
            ds[r] = pv * (fold_d ? dp[kb][r] : dp[kb][r] + nd);
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        dsf[kb * 2 + tt] = pack_bf16x8(ds[8 * tt], ds[8 * tt + 1], ds[8 * tt + 2], ds[8 * tt + 3],
                                       ds[8 * tt + 4], ds[8 * tt + 5], ds[8 * tt + 6],
                                       ds[8 * tt + 7]);
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int st = 0; st < kBC / 16; ++st)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int off = trb + 16 * st * SM::KST + db * 64;
        acc[db] = mfma32(lds_read_tr_pair(kt + off, 4 * SM::KST), dsf[st], acc[db]);
      }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using BT = std::integral_constant<bool, true>;
  using BF = std::integral_constant<bool, false>;

  if (ntiles > 0) {
    ktile.copy(Kh, 0, nk, kb0, wave);
    vtile.copy(Vh, 0, nk, vb0, wave);
  }
  int t = 0;
  for (; t + 1 < nfull; t += 2) {
    step(I0(), BF(), t);
    step(I1(), BF(), t + 1);
  }
  if (t < nfull) {
    step(I0(), BF(), t);
    ++t;
    if (t < ntiles) step(I1(), BT(), t++);
  }
  for (; t + 1 < ntiles; t += 2) {
    step(I0(), BT(), t);
    step(I1(), BT(), t + 1);
  }
  if (t < ntiles) step(I0(), BT(), t);

  if (qi < nq) store_row<D>(dQ + ((size_t)bh * Nq + qi) * D, acc, scale, hi);
  else if (VL && qi < Nq) store_zero_row<D>(dQ + ((size_t)bh * Nq + qi) * D, hi);  // padding
#endif
}

// ---------------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VL, bool DROP, bool BIAS, int DV = D>
hipError_t launch(const BwdArgs& a, unsigned phases) {
  const int BH = a.B * a.H;
  const float c = a.scale * kLog2e;
  const int rows = BH * a.Nq;
  float* nls = a.delta + bwd_lse2_offset(a.B, a.H, a.Nq);
  if (phases & 1u) {
    constexpr int RPB = 256 / (DV / 8);
    const int grid = (rows + RPB * 4 - 1) / (RPB * 4);
    hipLaunchKernelGGL((bwd_delta_kernel<DV>), dim3(grid), dim3(256), 0, a.stream, a.o, a.dout,
                       a.lse, a.delta, nls, rows, 1.f / a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int G = a.Hkv ? a.H / a.Hkv : 1;  // query heads per K/V head
  // grouped query heads with too few K/V workgroups to fill the chip, or with per-sequence
  // lengths (which make the workgroups that visit a whole group of heads very unequal, so that
  // the longest ones set the time): one workgroup per query head and fp32 partial rows in the
  // workspace, summed by a second kernel
  constexpr bool split = (DROP || BIAS) && D == 128;
  const bool partial = G > 1 && !BIAS && D == DV &&
                       (VL || bwd_gqa_uses_partials(a.B, a.H, a.H / G, a.Nk));
  const int GL = partial ? 1 : G;
  // dK/dV workgroups stream the Q and dO rows of the query heads of their unit (GL of them)
  const int hg_kv = xcd_head_group((size_t)GL * a.Nq * (D + DV) * 2, (long long)BH / GL);
  float* pK = partial ? a.delta + bwd_part_offset(a.B, a.H, a.Nq) : nullptr;
  float* pV = partial ? pK + (size_t)BH * a.Nk * D : nullptr;
  if (phases & 2u) {
    const long long grid = (long long)(BH / GL) * ((a.Nk + kBKV - 1) / kBKV);
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VL, DROP, split ? kDvOnly : kDkDv, BIAS, DV>),
                       dim3((unsigned)grid), dim3(kNT), 0, a.stream, a.q, a.k, a.v, a.dout, nls,
                       a.delta, a.dk, a.dv, a.lens_q, a.lens_k, BH, a.H, G, GL, pK, pV, a.Nq, a.Nk, c, a.scale,
                       a.drop, a.bias, hg_kv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (split) {
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VL, DROP, kDkOnly, BIAS, DV>),
                         dim3((unsigned)grid), dim3(kNT), 0, a.stream, a.q, a.k, a.v, a.dout, nls,
                         a.delta, a.dk, a.dv, a.lens_q, a.lens_k, BH, a.H, G, GL, pK, pV, a.Nq, a.Nk, c, a.scale,
                         a.drop, a.bias, hg_kv);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (partial) {
      const long long rows = (long long)(BH / G) * a.Nk;
      const long long threads = rows * (D / 8);
      const int rgrid = (int)std::min<long long>((threads + 255) / 256, 8192);
      hipLaunchKernelGGL((bwd_gqa_reduce_kernel<D>), dim3(rgrid), dim3(256), 0, a.stream, pK, pV,
                         a.dk, a.dv, G, a.Nk, rows);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (phases & 4u) {
    const long long grid = (long long)BH * ((a.Nq + kBR - 1) / kBR);
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, VL, DROP, BIAS, DV>), dim3((unsigned)grid),
                       dim3(kNT), 0, a.stream, a.q, a.k, a.v, a.dout, nls, a.delta, a.dq, a.lens_q,
                       a.lens_k, BH, a.H, G, a.Nq, a.Nk, c, a.scale, a.drop, a.bias,
                       xcd_head_group((size_t)a.Nk * (D + DV) * 2, (long long)BH / G));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool bwd_gqa_uses_partials(int B, int H, int Hkv, int Nk) {
  // fewer than 8 workgroups per CU (256 CUs) with one workgroup per K/V head and key tile:
  // one per query head instead, and the group sums formed by a second pass
  if (Hkv <= 0 || Hkv >= H) return false;
  const long long wgs = (long long)B * Hkv * ((Nk + kBKV - 1) / kBKV);
  return wgs < 2048;
}

size_t bwd_part_offset(int B, int H, int Nq) { return 2 * bwd_lse2_offset(B, H, Nq); }

size_t bwd_lse2_offset(int B, int H, int Nq) {
  // nD first, then nLs, each padded to a multiple of 16 bytes (counted in floats)
  return (((size_t)B * H * Nq + 3) / 4) * 4;
}

template <int D, bool VL, bool DROP, bool BIAS, int DV = D>
hipError_t launch_d(const BwdArgs& a, unsigned phases) {
  return a.causal ? launch<D, true, VL, DROP, BIAS, DV>(a, phases)
                  : launch<D, false, VL, DROP, BIAS, DV>(a, phases);
}

template <int D>
hipError_t launch_variant(const BwdArgs& a, unsigned phases) {
  // per-sequence lengths and dropout combine (with any grouping of the K/V heads); a bias runs
  // on its own
  if (a.bias.ptr != nullptr) return launch_d<D, false, false, true>(a, phases);
  const bool vl = a.lens_q != nullptr, drop = a.drop.thresh < 65536u;
  if (drop)
    return vl ? launch_d<D, true, true, false>(a, phases) : launch_d<D, false, true, false>(a, phases);
  return vl ? launch_d<D, true, false, false>(a, phases) : launch_d<D, false, false, false>(a, phases);
}

hipError_t launch_bwd(const BwdArgs& a, unsigned phases) {
  const int dv = a.d_v ? a.d_v : a.d;
  if (dv != a.d)  // a V head dimension of its own: the plain variant only
    return a.d == 128 ? launch_d<128, false, false, false, 64>(a, phases)
                      : launch_d<64, false, false, false, 128>(a, phases);
  return a.d == 128 ? launch_variant<128>(a, phases) : launch_variant<64>(a, phases);
}

}  // namespace fa
