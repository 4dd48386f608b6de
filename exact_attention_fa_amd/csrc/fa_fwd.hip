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
// CDNA4 mapping.
//   * The products are computed transposed, S^T = K Q^T and O^T = V^T P^T, on
//     v_mfma_f32_32x32x16_bf16, so that one lane owns one query: the row maximum is an in-lane
//     max plus one v_permlane32_swap, the row sum needs no exchange until the end, and the rescale
//     of the accumulator is in-lane. The keys of each 32-key block are given to the MFMA rows in
//     an order (key_of_row) that leaves every lane's eight probabilities of a 16-key step in
//     consecutive registers, so they feed the second product directly as its B operand.
//   * K and V tiles (64 keys) are copied HBM/L2 -> LDS by buffer_load_dwordx4 ... lds, with no
//     register staging; rows past N_k read as zero through the buffer range check. Tiles are
//     padded (K rows by 16 bytes, V rows by 32 bytes at d = 128) so that the 16-byte K reads of
//     the first product and the ds_read_b64_tr_b16 reads that assemble V^T for the second product
//     are free of bank conflicts. K is copied two tiles ahead and V one tile ahead.
//   * Software pipeline: the QK^T product of tile t+1 is issued while the softmax of tile t runs,
//     so the matrix cores and the vector ALUs overlap inside a wave; two waves share each SIMD.
//   * The reference m of the exponentials is a running maximum that only moves when needed, so
//     the accumulator rescale is skipped on most tiles; softmax is invariant to the reference
//     value, and every probability stays at most 2^kRescaleSlack. In most forms no row maximum is
//     taken on the common path: the exponentials are taken against m as it stands, and only when
//     some lane's sum of the tile exceeds 2^kRescaleSlack (or on the first tile) is the maximum
//     taken, m moved and the tile redone. The bias form takes the maximum first and moves m when
//     a row would exceed it by more than kRescaleSlack (log2 units).
//   * O is normalised by the sum of the same bf16 probabilities that feed the PV product, so it is
//     an exact convex combination of V rows under the rounded weights; the log-sum-exp keeps the
//     fp32 sum.
#include "fa_device.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kBC = 64;               // keys per tile
constexpr float kRescaleSlack = 8.f;  // log2 units
constexpr float kTileSumMax = 256.f;  // 2^kRescaleSlack

template <int D, int DV>
struct FwdLds {
  static constexpr int KST = 2 * D + 16;                        // K row stride (bytes)
  static constexpr int VST = 2 * DV + (DV == 128 ? 32 : 16);    // V row stride (bytes)
  static constexpr int KCPR = KST / 16, VCPR = VST / 16;        // 16-byte chunks per row
  static constexpr int KT = kBC * KST, VT = kBC * VST;          // tile bytes
  static constexpr int KI = kBC * KCPR / 64, VI = kBC * VCPR / 64;  // wave-wide copies per tile
  static_assert(KI * 64 == kBC * KCPR && VI * 64 == kBC * VCPR, "tiles are whole wave copies");
};

// VL: per-sequence lengths lens_q[b] <= Nq, lens_k[b] <= Nk inside the padded [B, H, N, d]
// tensors; query rows past a sequence's length, and rows that see no key, get O = 0 and
// LSE = -inf.
// DROP: dropout on P ("Maskeleme ve Dropout"): the row sums (and so the normaliser and L) use
// every probability; the PV product sees the kept ones, and O is scaled by 1 / (1 - p).
// BIAS: an additive bias on the scores (S = scale Q K^T + B of the notation of "FlashAttention'ı
// Anlamak Bölüm 1", 0.2), read from HBM one tile ahead; -inf entries mask, and a row whose scores
// are all -inf gets O = 0 and LSE = -inf.
// DV: head dimension of V and O (the notation's d_v; the same as D unless asked otherwise).
// G: query heads per K/V head (grouped-query attention; 1 unless asked otherwise): query head bh
// reads K/V head bh / G, K and V holding BH / G heads.
// d = d_v = 64 without dropout or a bias: one buffer of scores (the next tile's S^T is formed after
// this tile's P is packed, over its scores) fits the kernel in 168 VGPRs, so three waves share each
// SIMD (three 4-wave workgroups per CU) and the softmax of one wave hides under the products of
// the others. At d = 64 the softmax's share of the work is twice that of d = 128, and such waves
// beat two that each overlap the next tile's products with their own softmax (measured causal
// B1 H64 N32768 d64: 9.36 against 9.95 ms with four waves of 128 VGPRs, which take the row
// maximum first; three waves that take it late, 9.02 against 9.19 ms for those four). At d = 128
// the same form with three waves per SIMD (12-wave workgroups, 162 VGPRs) is slower than two
// double-buffered waves (0.560 against 0.514 ms, causal B2 H16 N8192).
template <int D, int DV, bool DROP, bool BIAS>
constexpr bool kOneScoreBuffer = D == 64 && DV == 64 && !DROP && !BIAS;

template <int D, int DV, int NW, bool CAUSAL, bool VL, bool DROP, bool BIAS>
__global__ __attribute__((amdgpu_waves_per_eu(kOneScoreBuffer<D, DV, DROP, BIAS> ? 3 : 2,
                                               kOneScoreBuffer<D, DV, DROP, BIAS> ? 3 : 2)))
__launch_bounds__(NW * 64) void fwd_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, const int* __restrict__ lens_q,
    const int* __restrict__ lens_k, int BH, int H, int G, int Nq, int Nk, float c,
    DropoutParams drop, BiasParams bias, int hg) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = FwdLds<D, DV>;
  constexpr int BR = NW * 32;  // query rows per workgroup
  constexpr bool kSB = kOneScoreBuffer<D, DV, DROP, BIAS>;
  // the row maximum only when the tile's sums call for it: the scores then stay live beside the
  // probabilities, which would push the bias form into scratch memory
  constexpr bool kLateMax = !BIAS;
  constexpr int KIW = (L::KI + NW - 1) / NW, VIW = (L::VI + NW - 1) / NW;
  // one array per buffer: the LDS copies into one buffer then provably do not alias the reads of
  // the other, so the reads wait for nothing but their own data
  __shared__ __attribute__((aligned(16))) unsigned char kb0[L::KT];
  __shared__ __attribute__((aligned(16))) unsigned char kb1[L::KT];
  __shared__ __attribute__((aligned(16))) unsigned char vb0[L::VT];
  __shared__ __attribute__((aligned(16))) unsigned char vb1[L::VT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // ---- workgroup -> (b*h, query tile): longest causal tiles first, all tiles that read one K/V
  // head on one XCD, K/V heads taken hg at a time (xcd_map).
  const int nqt = (Nq + BR - 1) / BR;
  int bh, rank;
  xcd_map(blockIdx.x, BH, G, nqt, hg, bh, rank);
  const int qt = CAUSAL ? nqt - 1 - rank : rank;
  const int q0 = qt * BR;
  const int qw = q0 + wave * 32;  // first query row of this wave
  const int qi = qw + l32;        // this lane's query row
  // valid lengths of this sequence (the whole padded extent without per-sequence lengths)
  const int nq = VL ? min(max(lens_q[bh / H], 0), Nq) : Nq;
  const int nk = VL ? min(max(lens_k[bh / H], 0), Nk) : Nk;
  const int shift = nk - nq;      // causal: key j visible to query i iff j <= i + shift

  const bf16* Qh = Q + (size_t)bh * Nq * D;
  const bf16* Kh = K + (size_t)(bh / G) * Nk * D;  // K/V head of this query head
  const bf16* Vh = V + (size_t)(bh / G) * Nk * DV;

  int kend = nk;
  if (CAUSAL) kend = min(nk, min(q0 + BR, nq) + shift);
  if (VL && q0 >= nq) kend = 0;  // every row of the workgroup is padding
  const int ntiles = max(0, (kend + kBC - 1) / kBC);
  // last tile any row of this wave can see
  const int horizon = CAUSAL ? min(qw + 31, nq - 1) + shift : nk - 1;
  const int last_tile = min(ntiles - 1, horizon / kBC);

  // ---- LDS fill: copy p of a tile (wave-wide, 64 consecutive 16-byte chunks) lands at chunk
  // positions p*64 .. p*64+63 of the padded tile; pad positions re-read chunk 0 of their row.
  int koff[KIW], voff[VIW];
#pragma unroll
  for (int i = 0; i < KIW; ++i) {
    const int p = (wave + i * NW) * 64 + lane, row = p / L::KCPR, ch = p % L::KCPR;
    koff[i] = row * D * 2 + (ch < D / 8 ? ch : 0) * 16;
  }
#pragma unroll
  for (int i = 0; i < VIW; ++i) {
    const int p = (wave + i * NW) * 64 + lane, row = p / L::VCPR, ch = p % L::VCPR;
    voff[i] = row * DV * 2 + (ch < DV / 8 ? ch : 0) * 16;
  }
  auto tile_rsrc = [&](const bf16* base, int t, int w) {  // w: row width (elements)
    // reads at or past the key length return zero (one head spans fewer than 2^31 bytes, which
    // the host checks, so the range fits its 32 bits)
    const int rows = max(0, nk - t * kBC);
    return make_rsrc(base + (size_t)t * kBC * w, rows * w * 2);
  };
  auto copy_k = [&](int t, unsigned char* dst) {
    const auto r = tile_rsrc(Kh, t, D);
#pragma unroll
    for (int i = 0; i < KIW; ++i)
      if (wave + i * NW < L::KI) buffer_to_lds(r, dst + (wave + i * NW) * 1024, koff[i]);
  };
  auto copy_v = [&](int t, unsigned char* dst) {
    const auto r = tile_rsrc(Vh, t, DV);
#pragma unroll
    for (int i = 0; i < VIW; ++i)
      if (wave + i * NW < L::VI) buffer_to_lds(r, dst + (wave + i * NW) * 1024, voff[i]);
  };

  // ---- Q fragments (B operand of S^T = K Q^T): query qi, dims 16 ks + 8 hi + 0..7
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < nq) x = ld16(Qh + (size_t)qi * D + ks * 16 + hi * 8);
    qf[ks] = as_bf16x8(x);
  }
  // rows that may end up with no finite score: padding (VL) or a bias that masks a whole row
  constexpr bool GUARD = VL || BIAS;
  // BIAS: this lane's bias row; lane half h needs keys kbase + 8 h + 16 g + 0..7, g = 0..3
  // (registers 8 (g & 1) .. + 7 of sc0 for g < 2, of sc1 for g >= 2)
  // (built in every variant; without a bias nothing reads it and it compiles away)
  const __amdgpu_buffer_rsrc_t brs = bias_rsrc(
      bias.ptr + (long long)(bh / H) * bias.sb + (long long)(bh % H) * bias.sh, Nq, Nk, bias.sq);
  const int boff = (int)((long long)min(qi, Nq - 1) * bias.sq * 2);
  auto load_bias = [&](int t, u32x4 (&bv)[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j0 = t * kBC + 8 * hi + 16 * g;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qi < nq && j0 + 8 <= nk) {
        w = bias_ld16(brs, boff + 2 * j0);
      } else if (qi < nq && j0 < nk) {  // ragged end of the keys: element by element
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (j0 + e < nk) w[e >> 1] |= bias_ld2(brs, boff + 2 * (j0 + e), 0) << (16 * (e & 1));
      }
      bv[g] = w;
    }
  };
  u32x4 bnext[4];
  const float cs = BIAS ? 1.f : c;  // with a bias the scores are turned into log2 units first
  f32x16 oacc[DV / 32];
#pragma unroll
  for (int db = 0; db < DV / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  // m in log2 units of the scaled scores; l: fp32 row sum; lq: sum of the bf16-rounded P
  float m_run = kNegInf, l_run = 0.f, lq_run = 0.f;

  // A operand of S^T: K row key_of_row(l32) (and +32), dims 16 ks + 8 hi
  const int kr0 = key_of_row(l32) * L::KST + hi * 16;
  // A operand of O^T (V^T rows = dims) via ds_read_b64_tr_b16: within each group of 16 lanes,
  // input lane j reads row 8 h + (j >> 2), columns 16 (group & 1) + 4 (j & 3) of the 16 x 32
  // block; the instruction hands output lane i element e of input lane 4 e + (i >> 2).
  const int vj = lane & 15, vg = lane >> 4;
  const int vr0 = (8 * (vg >> 1) + (vj >> 2)) * L::VST + (16 * (vg & 1) + 4 * (vj & 3)) * 2;

  auto qk = [&](f32x16& s0, f32x16& s1, const unsigned char* kt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 a0 = as_bf16x8(ld16(kt + kr0 + ks * 32));
      const bf16x8 a1 = as_bf16x8(ld16(kt + kr0 + 32 * L::KST + ks * 32));
      s0 = mfma32(a0, qf[ks], s0);
      s1 = mfma32(a1, qf[ks], s1);
    }
  };
  auto vt_frag = [&](const unsigned char* vt, int st, int db) {
    const unsigned char* p = vt + vr0 + st * 16 * L::VST + db * 64;
    return lds_read_tr_pair(p, 4 * L::VST);
  };

  // One pipeline step: mask, softmax and PV of tile t (scores in sc0/sc1), and the QK^T of
  // tile t+1 into sn0/sn1, issued between them so that it overlaps the softmax.
  // Tile t uses buffer t & 1 == P for V[t] and K[t+2], the other buffer for K[t+1] and V[t+1].
  auto step = [&](auto PAR, f32x16& sc0, f32x16& sc1, f32x16& sn0, f32x16& sn1, int t) {
    constexpr int P = decltype(PAR)::value;
    wait_vmem();      // this thread's copies of K[t+1] and V[t] have landed
    __syncthreads();  // ... everyone's have, and everyone is done with K[t], V[t-1]
    if (t + 2 < ntiles) copy_k(t + 2, P ? kb1 : kb0);
    if (t + 1 < ntiles) copy_v(t + 1, P ? vb0 : vb1);
    u32x4 bcur[4];
    if constexpr (BIAS) {
#pragma unroll
      for (int g = 0; g < 4; ++g) bcur[g] = bnext[g];
      if (t + 1 < ntiles) load_bias(t + 1, bnext);
    }
    if (t > last_tile) return;  // every row of this wave is masked from here on
    const int kbase = t * kBC;
    if constexpr (BIAS) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t w0 = bcur[r >> 3][(r & 7) >> 1], w1 = bcur[2 + (r >> 3)][(r & 7) >> 1];
        const float b0 = (r & 1) ? bf16_hi(w0) : bf16_lo(w0);
        const float b1 = (r & 1) ? bf16_hi(w1) : bf16_lo(w1);
        sc0[r] = __builtin_fmaf(b0, kLog2e, sc0[r] * c);
        sc1[r] = __builtin_fmaf(b1, kLog2e, sc1[r] * c);
      }
    }
    const bool need_mask = (kbase + kBC > nk) || (CAUSAL && kbase + kBC - 1 > qw + shift);
    if (need_mask) {
      const int lim = CAUSAL ? min(nk - 1, qi + shift) : nk - 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (kbase + key_of_reg(r, hi) > lim) sc0[r] = kNegInf;
        if (kbase + 32 + key_of_reg(r, hi) > lim) sc1[r] = kNegInf;
      }
    }
    // Softmax of the tile against the running reference m_run (log2 units of the scaled scores).
    // row_max: two independent v_max3 chains over the 32 scores of the lane
    auto row_max = [&]() {
      float ma = fmaxf(fmaxf(sc0[0], sc0[1]), sc0[2]), mb = fmaxf(fmaxf(sc1[0], sc1[1]), sc1[2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) {
        ma = fmaxf(fmaxf(ma, sc0[r]), sc0[r + 1]);
        mb = fmaxf(fmaxf(mb, sc1[r]), sc1[r + 1]);
      }
      return halves_max(fmaxf(fmaxf(ma, sc0[15]), fmaxf(mb, sc1[15]))) * cs;
    };
    // move the reference up to mx (a no-op for rows already at or above it)
    auto rescale_to = [&](float mx) {
      // finite for every row that sees a key: key 0 of tile 0 is visible to all of them
      const float m_new = fmaxf(m_run, mx);
      // a row that has seen no key yet has nothing to rescale; with per-sequence lengths it may
      // still have no key here (m_new = -inf), and exp2(-inf - -inf) would be NaN
      const float alpha = (GUARD && m_new == kNegInf) ? 1.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      lq_run *= alpha;
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    };
    // probabilities p = exp2(cs s - m) into p0/p1 (may alias sc0/sc1); returns the lane's sum
    auto probs = [&](f32x16& p0, f32x16& p1) {
      // a row that sees no key at all (possible only with per-sequence lengths or a bias) keeps
      // m = -inf; reference it to 0 so that its probabilities are exp2(-inf) = 0, not NaN
      const float m_use = (GUARD && m_run == kNegInf) ? 0.f : m_run;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p0[r] = exp2_fast(__builtin_fmaf(sc0[r], cs, -m_use));
        p1[r] = exp2_fast(__builtin_fmaf(sc1[r], cs, -m_use));
      }
      float ps[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ps[j] = p0[j] + p1[j];
#pragma unroll
      for (int r = 4; r < 16; ++r) ps[r & 3] += p0[r] + p1[r];
      return (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };
    f32x16 pa, pb;  // kLateMax: the probabilities (the scores stay for a second pass)
    f32x16& p0 = kLateMax ? pa : sc0;
    f32x16& p1 = kLateMax ? pb : sc1;
    float ts;  // sum of the lane's probabilities of this tile
    if constexpr (kLateMax) {
      if constexpr (!kSB) qk(sn0, sn1, P ? kb0 : kb1);
      // No row maximum on the common path: the exponentials are taken against m_run as it is,
      // and the tile is redone after a rescale only when some lane's sum leaves [0, 2^slack]
      // (so no probability exceeds 2^slack) or is not finite (m_run = -inf before the first
      // visit), or when a row without a reference meets its first finite score. On the first
      // tile the maximum is taken up front.
      bool again = t == 0;
      if (!again) {
        ts = probs(pa, pb);
        again = __any(!(ts <= kTileSumMax) || (GUARD && m_run == kNegInf && ts > 0.f));
      }
      if (again) {
        rescale_to(row_max());
        ts = probs(pa, pb);
      }
    } else {
      const float mx = row_max();
      if (__any(mx > m_run + kRescaleSlack)) rescale_to(mx);
      // Issued unconditionally so that it shares a basic block with the softmax below; past the
      // last tile it reads stale (in-bounds) LDS and its result is never used.
      if constexpr (!kSB) qk(sn0, sn1, P ? kb0 : kb1);
      ts = probs(sc0, sc1);
    }
    l_run += ts;
    bf16x8 pf[4];
    pf[0] = pack_bf16x8(p0[0], p0[1], p0[2], p0[3], p0[4], p0[5], p0[6], p0[7]);
    pf[1] = pack_bf16x8(p0[8], p0[9], p0[10], p0[11], p0[12], p0[13], p0[14], p0[15]);
    pf[2] = pack_bf16x8(p1[0], p1[1], p1[2], p1[3], p1[4], p1[5], p1[6], p1[7]);
    pf[3] = pack_bf16x8(p1[8], p1[9], p1[10], p1[11], p1[12], p1[13], p1[14], p1[15]);
    lq_run = sum_bf16x8(pf[3], sum_bf16x8(pf[2], sum_bf16x8(pf[1], sum_bf16x8(pf[0], lq_run))));
    if constexpr (DROP) {
      // pf[st] holds keys kbase + 16 st + 8 hi + 0..7: one generator call each
      const uint32_t g0 = (uint32_t)(kbase >> 3) + (uint32_t)hi;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4 w = philox4x32_10(g0 + 2u * st, (uint32_t)qi, (uint32_t)bh, drop.offset,
                                      drop.key0, drop.key1);
        u32x4 x = as_u32x4(pf[st]);
#pragma unroll
        for (int m = 0; m < 4; ++m) x[m] &= keep_halves(w[m], drop.thresh);
        pf[st] = as_bf16x8(x);
      }
    }
    // one score buffer: the next tile's S^T over this tile's scores, now packed into pf
    if constexpr (kSB) qk(sn0, sn1, P ? kb0 : kb1);
    const unsigned char* vt = P ? vb1 : vb0;
#pragma unroll
    for (int st = 0; st < kBC / 16; ++st)
#pragma unroll
      for (int db = 0; db < DV / 32; ++db) oacc[db] = mfma32(vt_frag(vt, st, db), pf[st], oacc[db]);
  };

  f32x16 sa0, sa1, sb0, sb1;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // (ntiles is the same for every wave; a workgroup with no tile to visit, e.g. padding rows of a
  // short sequence, goes straight to writing its empty rows)
  if (ntiles > 0) {
    if constexpr (BIAS) load_bias(0, bnext);
    copy_k(0, kb0);
    copy_v(0, vb0);
    if (ntiles > 1) copy_k(1, kb1);
    wait_vmem();
    __syncthreads();
    qk(sa0, sa1, kb0);
  }
  int t = 0;
  if constexpr (kSB) {
    for (; t + 1 < ntiles; t += 2) {
      step(I0(), sa0, sa1, sa0, sa1, t);
      step(I1(), sa0, sa1, sa0, sa1, t + 1);
    }
    if (t < ntiles) step(I0(), sa0, sa1, sa0, sa1, t);
  } else {
    for (; t + 1 < ntiles; t += 2) {
      step(I0(), sa0, sa1, sb0, sb1, t);
      step(I1(), sb0, sb1, sa0, sa1, t + 1);
    }
    if (t < ntiles) step(I0(), sa0, sa1, sb0, sb1, t);
  }

  // ---- epilogue: O = acc / lq, L = ln 2 * (m + log2 l)
  const float l_tot = halves_sum(l_run);
  const float lq_tot = halves_sum(lq_run);
  if (qi < Nq) {
    // padding, or a row that sees no key / whose scores are all -inf
    const bool empty = GUARD && (qi >= nq || lq_tot == 0.f);
    const float inv = empty ? 0.f : (DROP ? drop.inv_keep : 1.f) / lq_tot;
    bf16* orow = O + ((size_t)bh * Nq + qi) * DV;
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * j + 4 * hi) = w;
      }
    if (hi == 0) LSE[(size_t)bh * Nq + qi] = empty ? kNegInf : (m_run + log2_fast(l_tot)) * kLn2;
  }
#endif
}

template <int D, int DV, int NW, bool CAUSAL, bool VL, bool DROP, bool BIAS>
hipError_t launch(const FwdArgs& a) {
  constexpr int BR = NW * 32;
  const int nqt = (a.Nq + BR - 1) / BR;
  const long long grid = (long long)a.B * a.H * nqt;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float c = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_kernel<D, DV, NW, CAUSAL, VL, DROP, BIAS>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, a.stream, a.q, a.k, a.v, a.o, a.lse, a.lens_q, a.lens_k,
                     a.B * a.H, a.H, a.Hkv ? a.H / a.Hkv : 1, a.Nq, a.Nk, c, a.drop, a.bias,
                     xcd_head_group((size_t)a.Nk * (D + DV) * 2,
                                    (long long)a.B * (a.Hkv ? a.Hkv : a.H)));
  return hipGetLastError();
}

}  // namespace

// Workgroups of 8 waves (256 queries) share each K/V tile among the most waves; when that gives
// fewer than two workgroups per CU, 4-wave workgroups (128 queries) fill the chip instead
// (measured: causal B2 H8 N2048 d128, 128 workgroups of 8 waves, 0.055 ms; 256 of 4 waves,
// 0.041 ms; with two or more per CU the 8-wave form is as fast or faster).
template <int D, bool VL, bool DROP, bool BIAS, int DV = D>
hipError_t launch_d(const FwdArgs& a) {
  const long long tiles = (long long)a.B * a.H * ((a.Nq + 255) / 256);
  if constexpr (kOneScoreBuffer<D, DV, DROP, BIAS>) {  // three 4-wave workgroups per CU
    return a.causal ? launch<D, DV, 4, true, VL, DROP, BIAS>(a)
                    : launch<D, DV, 4, false, VL, DROP, BIAS>(a);
  } else {
    if (tiles < 512)
      return a.causal ? launch<D, DV, 4, true, VL, DROP, BIAS>(a)
                      : launch<D, DV, 4, false, VL, DROP, BIAS>(a);
    return a.causal ? launch<D, DV, 8, true, VL, DROP, BIAS>(a)
                    : launch<D, DV, 8, false, VL, DROP, BIAS>(a);
  }
}

template <int D>
hipError_t launch_variant(const FwdArgs& a) {
  // per-sequence lengths and dropout combine (with any grouping of the K/V heads); a bias runs
  // on its own
  if (a.bias.ptr != nullptr) return launch_d<D, false, false, true>(a);
  const bool vl = a.lens_q != nullptr, drop = a.drop.thresh < 65536u;
  if (drop) return vl ? launch_d<D, true, true, false>(a) : launch_d<D, false, true, false>(a);
  return vl ? launch_d<D, true, false, false>(a) : launch_d<D, false, false, false>(a);
}

hipError_t launch_fwd(const FwdArgs& a) {
  const int dv = a.d_v ? a.d_v : a.d;
  if (dv != a.d)  // a V head dimension of its own: the plain variant only
    return a.d == 128 ? launch_d<128, false, false, false, 64>(a)
                      : launch_d<64, false, false, false, 128>(a);
  return a.d == 128 ? launch_variant<128>(a) : launch_variant<64>(a);
}

}  // namespace fa
