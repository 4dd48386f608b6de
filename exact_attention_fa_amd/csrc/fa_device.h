// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---- 16-byte memory moves -----------------------------------------------------------------

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// ---- bf16 conversion (round to nearest even: v_cvt_pk_bf16_f32) ----------------------------

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                              float a5, float a6, float a7) {
  u32x4 u;
  u[0] = pack_bf16x2(a0, a1);
  u[1] = pack_bf16x2(a2, a3);
  u[2] = pack_bf16x2(a4, a5);
  u[3] = pack_bf16x2(a6, a7);
  return as_bf16x8(u);
}

// acc + the sum of the eight bf16 values of v (exact products with 1 in v_dot2_f32_bf16).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const u32x4 u = as_u32x4(v);
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t uw = u[w];  // copy first: bit_cast of an indexed vector element miscompiles
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, uw), one, acc, false);
  }
  return acc;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---- matrix cores --------------------------------------------------------------------------
// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] B[16x32].
// Operand lanes: lane l holds A row (l % 32), k = 8 * (l / 32) + 0..7, and B column (l % 32),
// the same k. Result: lane l holds column (l % 32), rows 8 * (r / 4) + 4 * (l / 32) + r % 4 for
// r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- transcendental ops --------------------------------------------------------------------
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// ---- cross-lane ----------------------------------------------------------------------------
// v_permlane32_swap(x, x) returns, in every lane, the pair {x[l], x[l ^ 32]} (in some order), so
// a max or a sum over the two half-waves needs no lane select.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- DPP reductions within rows of 16 lanes ---------------------------------------------------
template <int ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl,
                                                               0xF, 0xF, true));
}

// Sum over the G consecutive lanes that share one key row (G = 16 or 8); every lane of the
// group receives the total.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G == 16) {
    x += dpp<0x128>(x);  // row_ror:8
    x += dpp<0x124>(x);  // row_ror:4
    x += dpp<0x122>(x);  // row_ror:2
    x += dpp<0x121>(x);  // row_ror:1
  } else {
    static_assert(G == 8, "group of 8 or 16 lanes");
    x += dpp<0x141>(x);  // row_half_mirror: lane i of 8 gets lane 7 - i
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  }
  return x;
}

// ---- MFMA row order for the score tiles ------------------------------------------------------
// In a 32 x 32 score tile computed as D = A B with A holding 32 sequence rows, MFMA row m is given
// the sequence row key_of_row(m) = 16 (j >> 1) + 8 h + 4 (j & 1) + i (m = 8 j + 4 h + i). Result
// register r of a lane in half-wave h then holds sequence row key_of_reg(r, h) =
// 16 (r >> 3) + 8 h + (r & 7), so registers 8t..8t+7 cover 8 consecutive rows of the 16-row step t
// and feed a following MFMA that contracts over those rows without any data movement.
__device__ __forceinline__ int key_of_row(int m) {
  const int j = m >> 3, h = (m >> 2) & 1, i = m & 3;
  return 16 * (j >> 1) + 8 * h + 4 * (j & 1) + i;
}
__device__ __forceinline__ int key_of_reg(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

// ---- row-major [rows][D] bf16 tiles in LDS ---------------------------------------------------
// Each row is D/8 chunks of 16 bytes; the chunk index is XOR-swizzled with bits of the row so
// that 16-byte reads of one chunk from 16 different rows, and the 8-byte transposing reads of a
// 4-row x 16-column block, spread over distinct banks.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  constexpr int NCH = D / 8;
  const int swz = (((row & 3) << 1) | ((row >> 2) & 1) | (row & 8)) & (NCH - 1);
  return row * (D * 2) + ((((col >> 3) ^ swz)) << 4) + ((col & 7) << 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 concat_s16x4(s16x4 lo, s16x4 hi) {
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  u32x4 u;
  u[0] = a[0];
  u[1] = a[1];
  u[2] = b[0];
  u[3] = b[1];
  return as_bf16x8(u);
}

// Two ds_read_b64_tr_b16 at p and p + second: within each group of 16 lanes the instruction
// hands output lane i, element e, the element (i & 3) of the 4-element piece that input lane
// 4 e + (i >> 2) addressed; the two reads give elements 0..3 and 4..7 of an MFMA operand.
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const unsigned char* p, int second) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + second));
  return concat_s16x4(lo, hi);
}

// MFMA A-operand fragment of the transpose of a row-major LDS tile T ([rows][D], tile_off
// layout): lane (l32 = lane % 32, h = lane / 32) receives T[r0 + 8 h + e][c0 + l32] for e = 0..7,
// i.e. the 32 x 16 block (columns c0.., rows r0..r0+15) transposed. Input lane j of each group of
// 16 loads row r0 + 8 h + (j >> 2) (plus 4 for the second half), columns
// c0 + 16 (group & 1) + 4 (j & 3) .. + 3.
template <int D>
__device__ __forceinline__ bf16x8 lds_read_transposed(const unsigned char* tile, int r0, int c0,
                                                      int lane) {
  const int j = lane & 15, grp = lane >> 4;
  const int row = r0 + 8 * (grp >> 1) + (j >> 2);
  const int col = c0 + 16 * (grp & 1) + 4 * (j & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + tile_off<D>(row, col)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + tile_off<D>(row + 4, col)));
  return concat_s16x4(lo, hi);
}

// ---- workgroup -> (head, tile rank) -------------------------------------------------------
// For a grid of BH * nt workgroups over BH query heads of nt tiles each, the query heads coming
// in groups of G consecutive heads that share one K/V head (G = 1: every head has its own).
// Workgroups are dealt to the 8 XCDs round robin (XCD = blockIdx & 7), each XCD with its own L2.
// With the number of K/V heads BH / G a multiple of 8, XCD x serves the query heads of K/V heads
// x, x + 8, ... only, so all tiles that read one K/V head meet in one L2. Inside an XCD its K/V
// heads are taken hg at a time (hg >= 1), and the workgroups of such a head group go rank by rank
// (rank 0 first: the longest tiles of the causal kernels), so that the workgroups running at
// once stream the K/V (or Q/dO) tiles of few heads and find them in the L2.
__device__ __forceinline__ void xcd_map(int bid, int BH, int G, int nt, int hg, int& bh,
                                        int& rank) {
  const int BHkv = BH / G;
  if ((BHkv & 7) == 0) {
    const int xcd = bid & 7, local = bid >> 3, nkv = BHkv >> 3;  // K/V heads on this XCD
    const int hgc = min(max(hg, 1), nkv);
    const int grp = local / (hgc * G * nt);
    const int in = local - grp * (hgc * G * nt);
    const int kv0 = grp * hgc;
    const int per = min(hgc, nkv - kv0) * G;  // query heads in this group (the last may be short)
    rank = in / per;
    const int rem = in - rank * per;
    bh = ((kv0 + rem / G) * 8 + xcd) * G + rem % G;
  } else {
    bh = bid % BH;
    rank = bid / BH;
  }
}

// ---- HBM/L2 -> LDS copies without register staging ------------------------------------------
// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes return zero.
// Word 3 is the gfx9-family raw-buffer configuration (32-bit data format, no swizzle).
// `bytes` must be the same in every lane: it is read from the first active lane, so that the
// resource stays in scalar registers (a range the compiler would compute on the vector ALU, e.g.
// a clamp, would otherwise turn every load through it into a loop over distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
#else
  (void)base;
  (void)bytes;
  __builtin_unreachable();  // device code: never executed by the host pass
#endif
}
// buffer_load_dwordx4 ... lds: lane l of the wave writes its 16 bytes (from voffset) to
// dst + 16 l. dst must be the same for the whole wave.
__device__ __forceinline__ void buffer_to_lds(__amdgpu_buffer_rsrc_t r, unsigned char* dst,
                                              int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  // the LDS address is the low half of the flat address of an LDS location; going through the
  // integer avoids the null check a pointer cast from the generic space would carry
  typedef __attribute__((address_space(3))) void lds_void;
  lds_void* lds = (lds_void*)(uintptr_t)(uint32_t)(uintptr_t)dst;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voffset, 0, 0, 0);
#else
  (void)r;
  (void)dst;
  (void)voffset;
#endif
}
// Raw buffer resource over one head's additive bias (bf16, row stride sq elements) and the
// loads the kernels take from it: 32-bit offsets, and no fault for any offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bias_rsrc(const __bf16* base, int Nq, int Nk,
                                                            long long sq) {
  return make_rsrc(base, (int)(((long long)(Nq - 1) * sq + Nk) * 2));
}
__device__ __forceinline__ u32x4 bias_ld16(__amdgpu_buffer_rsrc_t r, int byte_off) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
#else
  (void)r;
  (void)byte_off;
  return u32x4{0u, 0u, 0u, 0u};
#endif
}
__device__ __forceinline__ uint32_t bias_ld2(__amdgpu_buffer_rsrc_t r, int byte_off, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, soff, 0);
#else
  (void)r;
  (void)byte_off;
  (void)soff;
  return 0u;
#endif
}

// Wait until this thread's outstanding vector-memory operations (including the LDS copies
// above) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The value of the lane whose index differs from this lane's in bit DIST (1, 2, 4 or 8), inside
// each row of 16 lanes, by DPP moves (no LDS traffic): quad permutations for 1 and 2; for 4 the
// mirror inside each 8 lanes (index ^ 7) and then the quad permutation index ^ 3; for 8 the
// rotation of the row by 8.
template <int DIST>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  const int v = (int)x;
  int r;
  if constexpr (DIST == 1) {
    r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (DIST == 2) {
    r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);  // quad_perm [2, 3, 0, 1]
  } else if constexpr (DIST == 4) {
    const int m = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);  // row_half_mirror
    r = __builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, true);             // quad_perm [3, 2, 1, 0]
  } else {
    static_assert(DIST == 8, "lane distances 1, 2, 4, 8");
    r = __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);  // row_ror:8
  }
  return (uint32_t)r;
}
template <int DIST>
__device__ __forceinline__ float lane_xor(float x) {
  return __uint_as_float(lane_xor<DIST>(__float_as_uint(x)));
}

// ---- dropout on the probabilities ------------------------------------------------------------
// The mask is never stored: every kernel that needs it regenerates it from a counter-based
// generator (the seed-and-offset scheme of "Maskeleme ve Dropout"). Generator: Philox-4x32-10
// (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds over a 4-word counter; each round forms the two
// 64-bit products of words 0 and 2 with fixed odd multipliers and outputs
// (hi(product of word 2) ^ word 1 ^ key 0, lo(product of word 2),
//  hi(product of word 0) ^ word 3 ^ key 1, lo(product of word 0)); the key grows by the Weyl
// constants (golden ratio and sqrt(3) fractions) between rounds.
// Call layout: the call with counter (j / 8, i, b*H + h, offset) decides scores (i, 8 (j/8) .. +7);
// key j uses 16-bit half (j & 1) (low half first) of output word (j & 7) / 2; it is kept iff that
// number is below the threshold t = floor((1 - p) 65536) < 65536.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-input exclusive or in one v_bitop3_b32 (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c0 = n0;
    c1 = (uint32_t)p1;
    c2 = n2;
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// 0xFFFF in each 16-bit half of w whose number is below t (t < 65536), 0 elsewhere: ANDed with a
// word of two packed bf16 probabilities, it zeroes the dropped ones.
__device__ __forceinline__ uint32_t keep_halves(uint32_t w, uint32_t t) {
  const uint32_t lo = (w & 0xFFFFu) < t ? 0x0000FFFFu : 0u;
  const uint32_t hi = (w >> 16) < t ? 0xFFFF0000u : 0u;
  return lo | hi;
}

// Per-element factor of the dropout: inv_keep where the number in half `h` of w is below t,
// else 0.
__device__ __forceinline__ float keep_factor(uint32_t w, int h, uint32_t t, float inv_keep) {
  const uint32_t u = h ? (w >> 16) : (w & 0xFFFFu);
  return u < t ? inv_keep : 0.f;
}

}  // namespace fa
