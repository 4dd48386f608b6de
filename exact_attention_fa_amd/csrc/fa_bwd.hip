// Attention backward for gfx950 (CDNA4): recomputation from the stored log-sum-exp.
//
// Method (page "Bellek Duvarının Fiziği: Standart Attention'dan FlashAttention'a", section
// "Geri Yayılım"): nothing of size N_q x N_k is stored by the forward pass; the backward rebuilds
// each probability tile on chip as P = exp(S - L) from the per-row log-sum-exp L, takes
// D = rowsum(dO * O) from the forward output, and applies the softmax gradient identity
// dS = P * (dP - D) with dP = dO V^T. Then dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K.
//
// Three kernels on one stream:
//   1. bwd_delta:  D_i = sum_k dO_ik O_ik (HBM-bound, one pass over O and dO);
//   2. bwd_dkdv:   one workgroup per (b, h, 128-key tile); each wave keeps 32 keys' K and V
//                  fragments and fp32 dK, dV accumulators in registers and streams the query
//                  tiles (Q, dO, L, D) through LDS;
//   3. bwd_dq:     one workgroup per (b, h, 128-query tile); each wave keeps 32 queries' Q and dO
//                  fragments and an fp32 dQ accumulator in registers and streams K/V tiles.
// Splitting dQ into its own pass recomputes S and dP a second time (7 products where a fused
// kernel would run 5) but needs no atomics, so every gradient is bitwise reproducible.
//
// CDNA4 mapping. All products are v_mfma_f32_32x32x16_bf16. In the dK/dV kernel the score tile
// is S = Q K^T (lane = key, registers = queries) so that P and dS are directly the B operands of
// dV^T = dO^T P and dK^T = Q^T dS, whose A operands (the transposes of the dO and Q tiles) come
// from ds_read_b64_tr_b16. The dQ kernel mirrors the forward: S^T = K Q^T (lane = query), and
// dQ^T = K^T dS^T takes K^T the same way. LDS tiles are row-major with XOR-swizzled 16-byte
// chunks and double-buffered; the next tile's global loads are issued before the current math.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kNW = 4;     // waves per workgroup
constexpr int kNT = kNW * 64;

// ---------------------------------------------------------------------------------------------
// 1. D = rowsum(dO * O)
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const bf16* __restrict__ O,
                                                        const bf16* __restrict__ dO,
                                                        float* __restrict__ delta, int rows) {
  constexpr int G = D / 8;           // lanes per row
  constexpr int RPB = 256 / G;       // rows per block pass
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
    if (gl == 0) delta[row] = s;
  }
}

// ---------------------------------------------------------------------------------------------
// Global -> register -> LDS staging of a [ROWS][D] row-major bf16 tile (rows past `nrows` zero).
template <int D, int ROWS>
struct TileStage {
  static constexpr int kChunks = ROWS * D / 8 / kNT;
  static_assert(kChunks >= 1, "tile smaller than the workgroup");
  u32x4 r[kChunks];
  __device__ __forceinline__ void load(const bf16* src, int row0, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int it = tid + i * kNT;
      const int row = it / (D / 8), ch = it % (D / 8);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row0 + row < nrows) x = ld16(src + (size_t)(row0 + row) * D + ch * 8);
      r[i] = x;
    }
  }
  __device__ __forceinline__ void store(unsigned char* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int it = tid + i * kNT;
      const int row = it / (D / 8), ch = it % (D / 8);
      st16(dst + tile_off<D>(row, ch * 8), r[i]);
    }
  }
};

// Store an fp32 accumulator tile held as D^T (lane = sequence row `row`, registers = dims
// 32 db + 8 j + 4 h + i) to a bf16 [.][D] tensor, multiplied by `mul`.
template <int D>
__device__ __forceinline__ void store_rows(bf16* dst_row, const f32x16 (&acc)[D / 32], float mul,
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

__device__ __forceinline__ void xcd_map(int bid, int BH, int& bh, int& rank) {
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, local = bid >> 3, per = BH >> 3;
    bh = (local % per) * 8 + xcd;
    rank = local / per;
  } else {
    bh = bid % BH;
    rank = bid / BH;
  }
}

// ---------------------------------------------------------------------------------------------
// 2. dK, dV
constexpr int kBKV = 128;  // keys per workgroup (32 per wave)
constexpr int kBQ = 64;    // queries per streamed tile

template <int D>
struct DkdvSmem {
  static constexpr int kTile = kBQ * D * 2;
  static constexpr int kQ = 0, kDO = kTile, kL = 2 * kTile, kDl = 2 * kTile + kBQ * 4;
  static constexpr int kBuf = 2 * kTile + 2 * kBQ * 4;
  static constexpr int kBytes = 2 * kBuf;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kNT) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int BH, int Nq, int Nk, float c, float scale) {
  using SM = DkdvSmem<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  int bh, rank;
  xcd_map(blockIdx.x, BH, bh, rank);
  const int kt = rank;  // causal: low key tiles see the most queries and are launched first
  const int k0 = kt * kBKV;
  const int kw = k0 + wave * 32;
  const int key = kw + l32;
  const int shift = Nk - Nq;

  const bf16* Qh = Q + (size_t)bh * Nq * D;
  const bf16* dOh = dO + (size_t)bh * Nq * D;
  const float* Lh = LSE + (size_t)bh * Nq;
  const float* Dh = Dl + (size_t)bh * Nq;

  // resident B operands: K^T and V^T columns (lane = key, 8 dims per k-step)
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (key < Nk) {
      a = ld16(K + ((size_t)bh * Nk + key) * D + ks * 16 + hi * 8);
      b = ld16(V + ((size_t)bh * Nk + key) * D + ks * 16 + hi * 8);
    }
    kf[ks] = as_bf16x8(a);
    vf[ks] = as_bf16x8(b);
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }

  // query tiles that can see any key of this workgroup
  int qbeg = 0;
  if (CAUSAL) qbeg = max(0, k0 - shift);
  const int t0 = qbeg / kBQ;
  const int t1 = (Nq + kBQ - 1) / kBQ;

  TileStage<D, kBQ> sq, sdo;
  float lreg = 0.f, dreg = 0.f;
  auto load = [&](int t) {
    const int q0 = t * kBQ;
    sq.load(Qh, q0, Nq, tid);
    sdo.load(dOh, q0, Nq, tid);
    if (tid < kBQ) {
      const int q = q0 + tid;
      // rows past N_q get L = +inf, so their probabilities are exactly zero
      lreg = q < Nq ? Lh[q] * kLog2e : __builtin_huge_valf();
      dreg = q < Nq ? Dh[q] : 0.f;
    }
  };
  auto store = [&](int buf) {
    unsigned char* b = smem + buf * SM::kBuf;
    sq.store(b + SM::kQ, tid);
    sdo.store(b + SM::kDO, tid);
    if (tid < kBQ) {
      reinterpret_cast<float*>(b + SM::kL)[tid] = lreg;
      reinterpret_cast<float*>(b + SM::kDl)[tid] = dreg;
    }
  };

  if (t0 < t1) load(t0);
  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    store(buf);
    __syncthreads();
    if (t + 1 < t1) load(t + 1);
    const int q0 = t * kBQ;
    // every query of the tile is before this wave's first visible position: nothing to do
    if (CAUSAL && min(q0 + kBQ, Nq) - 1 + shift < kw) continue;
    const unsigned char* b = smem + buf * SM::kBuf;
    const float* ls = reinterpret_cast<const float*>(b + SM::kL);
    const float* dls = reinterpret_cast<const float*>(b + SM::kDl);
    const bool need_mask = CAUSAL && (q0 + shift < kw + 31);
#pragma unroll
    for (int qb = 0; qb < kBQ / 32; ++qb) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
      const int qrow = qb * 32 + key_of_row(l32);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = as_bf16x8(ld16(b + SM::kQ + tile_off<D>(qrow, ks * 16 + hi * 8)));
        s = mfma32(a, kf[ks], s);
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = as_bf16x8(ld16(b + SM::kDO + tile_off<D>(qrow, ks * 16 + hi * 8)));
        dp = mfma32(a, vf[ks], dp);
      }
      // P = exp2(c S - L log2 e), dS = P (dP - D); queries of register r: qb*32 + key_of_reg(r, hi)
      float p[16], ds[16];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qi0 = qb * 32 + 16 * half + 8 * hi;
        const f32x4 la = *reinterpret_cast<const f32x4*>(ls + qi0);
        const f32x4 lb = *reinterpret_cast<const f32x4*>(ls + qi0 + 4);
        const f32x4 da = *reinterpret_cast<const f32x4*>(dls + qi0);
        const f32x4 db4 = *reinterpret_cast<const f32x4*>(dls + qi0 + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * half + e;
          const float lv = e < 4 ? la[e] : lb[e - 4];
          const float dv4 = e < 4 ? da[e] : db4[e - 4];
          float pv = exp2_fast(__builtin_fmaf(s[r], c, -lv));
          if (need_mask && key > q0 + qi0 + e + shift) pv = 0.f;
          p[r] = pv;
          ds[r] = pv * (dp[r] - dv4);
        }
      }
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        pf[st] = pack_bf16x8(p[8 * st], p[8 * st + 1], p[8 * st + 2], p[8 * st + 3], p[8 * st + 4],
                             p[8 * st + 5], p[8 * st + 6], p[8 * st + 7]);
        dsf[st] = pack_bf16x8(ds[8 * st], ds[8 * st + 1], ds[8 * st + 2], ds[8 * st + 3],
                              ds[8 * st + 4], ds[8 * st + 5], ds[8 * st + 6], ds[8 * st + 7]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS (A operands: transposed 32-dim x 16-query blocks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 ao = lds_read_transposed<D>(b + SM::kDO, qb * 32 + 16 * st, db * 32, lane);
          dv[db] = mfma32(ao, pf[st], dv[db]);
          const bf16x8 aq = lds_read_transposed<D>(b + SM::kQ, qb * 32 + 16 * st, db * 32, lane);
          dk[db] = mfma32(aq, dsf[st], dk[db]);
        }
    }
  }

  if (key < Nk) {
    store_rows<D>(dK + ((size_t)bh * Nk + key) * D, dk, scale, hi);
    store_rows<D>(dV + ((size_t)bh * Nk + key) * D, dv, 1.f, hi);
  }
}

// ---------------------------------------------------------------------------------------------
// 3. dQ
constexpr int kBR = 128;  // queries per workgroup (32 per wave)
constexpr int kBC = 64;   // keys per streamed tile

template <int D>
struct DqSmem {
  static constexpr int kTile = kBC * D * 2;
  static constexpr int kK = 0, kV = kTile;
  static constexpr int kBuf = 2 * kTile;
  static constexpr int kBytes = 2 * kBuf;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kNT) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    bf16* __restrict__ dQ, int BH, int Nq, int Nk, float c, float scale) {
  using SM = DqSmem<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  int bh, rank;
  xcd_map(blockIdx.x, BH, bh, rank);
  const int nqt = (Nq + kBR - 1) / kBR;
  const int qt = CAUSAL ? nqt - 1 - rank : rank;
  const int q0 = qt * kBR;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;
  const int shift = Nk - Nq;

  const bf16* Kh = K + (size_t)bh * Nk * D;
  const bf16* Vh = V + (size_t)bh * Nk * D;

  // resident B operands: Q^T and dO^T columns (lane = query)
  bf16x8 qf[D / 16], dof[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (qi < Nq) {
      a = ld16(Q + ((size_t)bh * Nq + qi) * D + ks * 16 + hi * 8);
      b = ld16(dO + ((size_t)bh * Nq + qi) * D + ks * 16 + hi * 8);
    }
    qf[ks] = as_bf16x8(a);
    dof[ks] = as_bf16x8(b);
  }
  const float lq = qi < Nq ? LSE[(size_t)bh * Nq + qi] * kLog2e : 0.f;
  const float dq_d = qi < Nq ? Dl[(size_t)bh * Nq + qi] : 0.f;

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(q0 + kBR, Nq) - 1 + shift + 1);
  const int ntiles = (kend + kBC - 1) / kBC;
  const int wave_horizon = CAUSAL ? min(qw + 31, Nq - 1) + shift : Nk - 1;

  TileStage<D, kBC> sk, sv;
  if (ntiles > 0) {
    sk.load(Kh, 0, Nk, tid);
    sv.load(Vh, 0, Nk, tid);
  }
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    unsigned char* b = smem + buf * SM::kBuf;
    sk.store(b + SM::kK, tid);
    sv.store(b + SM::kV, tid);
    __syncthreads();
    if (t + 1 < ntiles) {
      sk.load(Kh, (t + 1) * kBC, Nk, tid);
      sv.load(Vh, (t + 1) * kBC, Nk, tid);
    }
    const int kbase = t * kBC;
    if (kbase > wave_horizon) continue;
    const bool need_mask = (kbase + kBC > Nk) || (CAUSAL && kbase + kBC - 1 > qw + shift);
    const int lim = CAUSAL ? min(Nk - 1, qi + shift) : Nk - 1;
    bf16x8 dsf[kBC / 16];
#pragma unroll
    for (int kb = 0; kb < kBC / 32; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
      const int krow = kb * 32 + key_of_row(l32);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = as_bf16x8(ld16(b + SM::kK + tile_off<D>(krow, ks * 16 + hi * 8)));
        s = mfma32(a, qf[ks], s);
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = as_bf16x8(ld16(b + SM::kV + tile_off<D>(krow, ks * 16 + hi * 8)));
        dp = mfma32(a, dof[ks], dp);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = exp2_fast(__builtin_fmaf(s[r], c, -lq));
        if (need_mask && kbase + kb * 32 + key_of_reg(r, hi) > lim) pv = 0.f;
        ds[r] = pv * (dp[r] - dq_d);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        dsf[kb * 2 + tt] = pack_bf16x8(ds[8 * tt], ds[8 * tt + 1], ds[8 * tt + 2], ds[8 * tt + 3],
                                       ds[8 * tt + 4], ds[8 * tt + 5], ds[8 * tt + 6],
                                       ds[8 * tt + 7]);
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int st = 0; st < kBC / 16; ++st) {
        const bf16x8 a = lds_read_transposed<D>(b + SM::kK, 16 * st, db * 32, lane);
        acc[db] = mfma32(a, dsf[st], acc[db]);
      }
  }

  if (qi < Nq) store_rows<D>(dQ + ((size_t)bh * Nq + qi) * D, acc, scale, hi);
}

// ---------------------------------------------------------------------------------------------
template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a, unsigned phases) {
  const int BH = a.B * a.H;
  const float c = a.scale * kLog2e;
  const int rows = BH * a.Nq;
  if (phases & 1u) {
    constexpr int RPB = 256 / (D / 8);
    int grid = (rows + RPB * 4 - 1) / (RPB * 4);
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3(grid), dim3(256), 0, a.stream, a.o, a.dout,
                       a.delta, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 2u) {
    const long long grid = (long long)BH * ((a.Nk + kBKV - 1) / kBKV);
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kNT), 0, a.stream,
                       a.q, a.k, a.v, a.dout, a.lse, a.delta, a.dk, a.dv, BH, a.Nq, a.Nk, c,
                       a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 4u) {
    const long long grid = (long long)BH * ((a.Nq + kBR - 1) / kBR);
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kNT), 0, a.stream,
                       a.q, a.k, a.v, a.dout, a.lse, a.delta, a.dq, BH, a.Nq, a.Nk, c, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, unsigned phases) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, phases) : launch<128, false>(a, phases);
  return a.causal ? launch<64, true>(a, phases) : launch<64, false>(a, phases);
}

}  // namespace fa
