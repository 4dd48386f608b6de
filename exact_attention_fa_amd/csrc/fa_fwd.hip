// Fused attention forward for gfx950 (CDNA4): one workgroup per (batch, head, query tile).
//
// Method (page "Bellek Duvarının Fiziği: Standart Attention'dan FlashAttention'a"):
//   * "Forward geçişin iskeleti": Q is split into row tiles that stay on chip for the whole pass,
//     K/V are streamed tile by tile, and the running row maximum m, running sum l and unscaled
//     output accumulator are updated per tile; O = diag(l)^-1 * acc once at the end (the
//     deferred normalisation of "FlashAttention-2, -3 ve -4", item 2). The score and
//     probability tiles exist only in registers.
//   * "Online Softmax": the exponentials are taken base 2 with the scale and log2(e) folded into
//     one multiply-add per score, and the row statistics are kept in base-2 units.
//   * "Maskeleme ve Dropout": tiles entirely above the causal diagonal are never visited; only
//     tiles that cross it (or the ragged end of the keys) are masked, with -inf written before
//     the row maximum is taken.
//   * "FlashAttention-2, -3 ve -4", items 1 and 3: the loop over query tiles is the parallel
//     (grid) dimension, and inside a workgroup each wave owns 32 query rows while all waves
//     share the K/V tiles in LDS.
//
// CDNA4 mapping. The products are computed transposed, S^T = K Q^T and O^T = V^T P^T, on
// v_mfma_f32_32x32x16_bf16, so that one lane owns one query: the row maximum is an in-lane max
// plus one exchange with the other half-wave, the row sum needs no exchange until the end, and
// the rescale of the accumulator by alpha is in-lane. The keys of each 32-key block are given
// to the MFMA rows in an order (key_of_row) that leaves every lane's eight probabilities of a
// 16-key step in consecutive registers, so they feed the second product directly as its B
// operand. V is stored transposed in LDS (row = head dimension, keys along the row, 16-byte
// chunks XOR-swizzled against bank conflicts); K is stored row-major with one 16-byte pad per
// row. K/V tiles are double-buffered in LDS and the next tile's global loads are issued before
// the current tile's math.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBC = 64;  // keys per tile
constexpr float kRescaleSlack = 8.f;  // log2 units

// Byte offset of the 16-byte chunk `c` (keys 8c..8c+7) of transposed-V row `d` in LDS.
// Rows are kBC * 2 = 128 bytes; the chunk index is XOR-swizzled with the row so that both the
// MFMA operand reads (16 consecutive rows, one chunk) and the transposing writes are free of
// bank conflicts.
__device__ __forceinline__ int vt_offset(int d, int c) {
  const int swz = ((d >> 1) & 7) ^ (((d >> 4) & 1) << 1);
  return d * (kBC * 2) + 16 * (c ^ swz);
}

template <int D>
struct FwdSmem {
  static constexpr int kStride = D + 8;                 // K row stride in bf16 (16-byte pad)
  static constexpr int kKBytes = kBC * kStride * 2;     // one K tile
  static constexpr int kVBytes = D * kBC * 2;           // one transposed V tile
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static constexpr int kBytes = 2 * kBufBytes;          // double buffered
};

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(const bf16* __restrict__ Q,
                                                      const bf16* __restrict__ K,
                                                      const bf16* __restrict__ V,
                                                      bf16* __restrict__ O,
                                                      float* __restrict__ LSE, int BH, int Nq,
                                                      int Nk, float c) {
  constexpr int NT = NW * 64;         // threads
  constexpr int BR = NW * 32;         // query rows per workgroup
  constexpr int DCH = D / 8;          // 16-byte chunks per row
  constexpr int KCH = kBC * DCH / NT; // K chunks per thread
  constexpr int VTOT = (kBC / 2) * DCH;       // V (key pair, chunk) items per tile
  constexpr int VIT = (VTOT + NT - 1) / NT;   // per thread (the last pass may be partial)
  static_assert(KCH >= 1 && KCH * NT == kBC * DCH, "K tile must split evenly over the threads");
  using SM = FwdSmem<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // ---- workgroup -> (b*h, query tile): longest causal tiles first; with BH a multiple of 8,
  // all query tiles of one head go to one XCD (workgroups are dealt to the 8 XCDs round robin),
  // so that head's K/V stays in that XCD's L2.
  const int nqt = (Nq + BR - 1) / BR;
  int bh, rank;
  const int bid = blockIdx.x;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, local = bid >> 3, per = BH >> 3;
    bh = (local % per) * 8 + xcd;
    rank = local / per;
  } else {
    bh = bid % BH;
    rank = bid / BH;
  }
  const int qt = CAUSAL ? nqt - 1 - rank : rank;
  const int q0 = qt * BR;
  const int qw = q0 + wave * 32;  // first query row of this wave
  const int shift = Nk - Nq;      // causal: key j visible to query i iff j <= i + shift

  const bf16* Qh = Q + (size_t)bh * Nq * D;
  const bf16* Kh = K + (size_t)bh * Nk * D;
  const bf16* Vh = V + (size_t)bh * Nk * D;

  // ---- key range of the workgroup
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(q0 + BR, Nq) - 1 + shift + 1);
  const int ntiles = (kend + kBC - 1) / kBC;

  // ---- Q fragments (B operand of S^T = K Q^T): query qw + l32, dims 16 ks + 8 hi + 0..7
  bf16x8 qf[D / 16];
  {
    const int qi = qw + l32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qi < Nq) x = ld16(Qh + (size_t)qi * D + ks * 16 + hi * 8);
      qf[ks] = as_bf16x8(x);
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = kNegInf, l_run = 0.f, lq_run = 0.f;  // lq: sum of the bf16-rounded P

  // ---- global -> register staging of one K/V tile
  u32x4 kreg[KCH], vreg[VIT][2];
  auto load_tile = [&](int t) {
    const int kb0 = t * kBC;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int it = tid + i * NT;
      const int key = kb0 + it / DCH, dc = it % DCH;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < Nk) x = ld16(Kh + (size_t)key * D + dc * 8);
      kreg[i] = x;
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int it = tid + i * NT;
      if (VTOT % NT != 0 && it >= VTOT) break;
      const int dc = (it & 3) + 4 * ((it >> 6) % (DCH / 4));
      const int kp = ((it >> 2) & 15) + 16 * ((it >> 6) / (DCH / 4));
      const int key = kb0 + 2 * kp;
      u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
      if (key < Nk) x0 = ld16(Vh + (size_t)key * D + dc * 8);
      if (key + 1 < Nk) x1 = ld16(Vh + (size_t)(key + 1) * D + dc * 8);
      vreg[i][0] = x0;
      vreg[i][1] = x1;
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* kbuf = smem + buf * SM::kBufBytes;
    unsigned char* vbuf = kbuf + SM::kKBytes;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int it = tid + i * NT;
      const int key = it / DCH, dc = it % DCH;
      st16(kbuf + (key * SM::kStride + dc * 8) * 2, kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int it = tid + i * NT;
      if (VTOT % NT != 0 && it >= VTOT) break;
      const int dc = (it & 3) + 4 * ((it >> 6) % (DCH / 4));
      const int kp = ((it >> 2) & 15) + 16 * ((it >> 6) / (DCH / 4));
      const u32x4 a = vreg[i][0], b = vreg[i][1];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // dims 8 dc + 2w (low halves) and 8 dc + 2w + 1 (high halves) of keys 2kp, 2kp + 1
        const uint32_t lo = __builtin_amdgcn_perm(b[w], a[w], 0x05040100u);
        const uint32_t hw = __builtin_amdgcn_perm(b[w], a[w], 0x07060302u);
        const int d0 = dc * 8 + 2 * w;
        *reinterpret_cast<uint32_t*>(vbuf + vt_offset(d0, kp >> 2) + 4 * (kp & 3)) = lo;
        *reinterpret_cast<uint32_t*>(vbuf + vt_offset(d0 + 1, kp >> 2) + 4 * (kp & 3)) = hw;
      }
    }
  };

  // horizon of this wave: last key any of its rows can see
  const int wave_last_q = min(qw + 31, Nq - 1);
  const int wave_horizon = CAUSAL ? wave_last_q + shift : Nk - 1;
  const int qi = qw + l32;

  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    store_tile(buf);
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);

    const int kbase = t * kBC;
    if (kbase > wave_horizon) continue;  // every row of this wave is masked for this tile
    const unsigned char* kbuf = smem + buf * SM::kBufBytes;
    const unsigned char* vbuf = kbuf + SM::kKBytes;

    // ---- S^T = K Q^T for the 64 keys of the tile (two 32-key blocks)
    f32x16 s[kBC / 32];
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const int krow = kb * 32 + key_of_row(l32);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = as_bf16x8(ld16(kbuf + (krow * SM::kStride + ks * 16 + hi * 8) * 2));
        s[kb] = mfma32(a, qf[ks], s[kb]);
      }
    }

    // ---- mask the ragged end of the keys and the causal diagonal
    const bool need_mask = (kbase + kBC > Nk) || (CAUSAL && kbase + kBC - 1 > qw + shift);
    if (need_mask) {
      const int lim = CAUSAL ? min(Nk - 1, qi + shift) : Nk - 1;
#pragma unroll
      for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + kb * 32 + key_of_reg(r, hi) > lim) s[kb][r] = kNegInf;
    }

    // ---- online softmax (base 2, scale folded into c = scale * log2 e)
    // The running maximum is only moved when some row of the wave would exceed it by more than
    // kRescaleSlack (in log2 units); otherwise the stale maximum is kept. Softmax is invariant
    // to the reference value, so the result is the same up to rounding: probabilities are then
    // bounded by 2^kRescaleSlack instead of 1, far inside fp32 and bf16 range, and the rescale
    // of the accumulator (D/2 multiplies per lane) is skipped on most tiles.
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = halves_max(mx) * c;
    if (__any(mx > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast(m_run - m_new);  // m_new is finite: key 0 of tile 0 is visible
      m_run = m_new;
      l_run *= alpha;
      lq_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float m_use = m_run;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb][r] = exp2_fast(__builtin_fmaf(s[kb][r], c, -m_use));
        psum += s[kb][r];
      }
    l_run += psum;

    // P goes to the second product in bf16. The normaliser of O is the row sum of those same
    // bf16 values (one v_dot2_f32_bf16 against (1, 1) per pair), so O is an exact convex
    // combination of V rows under the rounded weights: its error becomes
    // sum_j w_j e_j (v_j - O) instead of sum_j w_j e_j v_j, much smaller when a few keys dominate
    // a row. The log-sum-exp keeps the fp32 sum.
    bf16x8 pf[kBC / 16];
    float qsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int r0 = 8 * tt;
        pf[kb * 2 + tt] = pack_bf16x8(s[kb][r0], s[kb][r0 + 1], s[kb][r0 + 2], s[kb][r0 + 3],
                                      s[kb][r0 + 4], s[kb][r0 + 5], s[kb][r0 + 6], s[kb][r0 + 7]);
        qsum = sum_bf16x8(pf[kb * 2 + tt], qsum);
      }
    lq_run += qsum;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + l32;
#pragma unroll
      for (int st = 0; st < kBC / 16; ++st) {
        const bf16x8 a = as_bf16x8(ld16(vbuf + vt_offset(d, 2 * st + hi)));
        oacc[db] = mfma32(a, pf[st], oacc[db]);
      }
    }
  }

  // ---- epilogue: O = acc / l, L = ln 2 * (m + log2 l)
  const float l_tot = halves_sum(l_run);
  const float lq_tot = halves_sum(lq_run);
  if (qi < Nq) {
    const float inv = 1.f / lq_tot;
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
    if (hi == 0) LSE[(size_t)bh * Nq + qi] = (m_run + log2_fast(l_tot)) * kLn2;
  }
}

template <int D, int NW, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  constexpr int BR = NW * 32;
  const int nqt = (a.Nq + BR - 1) / BR;
  const long long grid = (long long)a.B * a.H * nqt;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_kernel<D, NW, CAUSAL>), dim3((unsigned)grid), dim3(NW * 64), 0,
                     a.stream, a.q, a.k, a.v, a.o, a.lse, a.B * a.H, a.Nq, a.Nk, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch<128, 8, true>(a) : launch<128, 8, false>(a);
  return a.causal ? launch<64, 8, true>(a) : launch<64, 8, false>(a);
}

}  // namespace fa
