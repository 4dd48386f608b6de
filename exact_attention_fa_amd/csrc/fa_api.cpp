// C ABI of the attention library: argument validation, workspace sizing and dispatch.
// Every check runs before anything is enqueued, so an error leaves the outputs untouched.
#include "fa.h"

#include <math.h>

#include "fa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// One head's rows of width w (bf16) span fewer than 2^31 bytes: the kernels address inside a
// head with 32-bit byte offsets.
bool head_extent_ok(int n, int w) { return (long long)n * w * 2 < (1LL << 31); }

fa_status check_common(int B, int H, int Nq, int Nk, int d, float scale, int causal) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  const long long bh = (long long)B * H;
  if (bh * Nq >= (1LL << 31) || bh * Nk >= (1LL << 31)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!head_extent_ok(Nq, d) || !head_extent_ok(Nk, d)) return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (causal && Nq > Nk) return FA_ERR_CAUSAL;
  return FA_OK;
}

fa_status from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

const __bf16* bf(const fa_bf16* p) { return reinterpret_cast<const __bf16*>(p); }
__bf16* bf(fa_bf16* p) { return reinterpret_cast<__bf16*>(p); }

size_t round_up16(size_t n) { return (n + 15) & ~size_t(15); }

}  // namespace

namespace fa {

int xcd_head_group(size_t bytes_per_head, long long heads) {
  // Measured on causal workloads (rows per head streamed by each workgroup, heads per XCD):
  //   B8 H16 d128, eight sequences of 1363..8174 positions (4 MiB, 16): forward 1.075 / 0.986 /
  //     0.972 / 1.201 ms and backward 3.33 / 2.95 / 2.89 / 3.48 ms with all of an XCD's heads /
  //     1 / 2 / 4 at a time;
  //   B1 H64 N32768 d64 (8 MiB, 8): forward 11.02 ms with all, 10.13 ms with 2;
  //   B2 H16 N8192 d128 (4 MiB, 4): 0.525 ms with all, 0.532 ms with 2;
  //   B4 H16 N2048 d128 (1 MiB, 8): 0.090 ms with all, 0.107 ms with 2.
  // Grouping pays once an XCD's heads stream more than its share of the 256 MiB last-level
  // cache (32 MiB); then two heads at a time, or as many as fit in about 2 MiB.
  const long long per_xcd = (heads + 7) / 8;
  if ((double)per_xcd * (double)bytes_per_head <= (double)(32u << 20)) return 1 << 20;
  const size_t n = bytes_per_head ? ((size_t)2 << 20) / bytes_per_head : 2;
  return (int)(n < 2 ? 2 : (n > (1u << 20) ? (1u << 20) : n));
}

fa_status decode_validate(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                          const float* lse, int B, int H, int N_q, int N_k, int d, float scale,
                          int causal, int num_splits, int* splits) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status s = check_common(B, H, N_q, N_k, d, scale, causal);
  if (s != FA_OK) return s;
  if (N_q != 1) return FA_ERR_ARG;
  if (num_splits < 0 || num_splits > 1024 || num_splits > N_k) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  *splits = num_splits == 0 ? decode_auto_splits(B, H, N_k, d) : num_splits;
  return FA_OK;
}

fa_status decode_run(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                     void* workspace, int B, int H, int N_k, int d, float scale, int splits,
                     hipStream_t stream) {
  const size_t rows = (size_t)B * H * splits;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             round_up16(rows * d * sizeof(float)));
  DecodeArgs a{bf(q), bf(k), bf(v), bf(o), lse, part_o, part_lse, B, H, N_k, d, splits, scale,
               stream};
  return from_hip(launch_decode(a));
}

}  // namespace fa

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: a size is < 1 or an index range is too large";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: head dimension must be 64 or 128";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: pointers must be 16-byte aligned";
    case FA_ERR_CAUSAL: return "FA_ERR_CAUSAL: causal attention needs N_q <= N_k";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0";
    case FA_ERR_ARG: return "FA_ERR_ARG: argument out of range";
    case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch failed";
  }
  return "FA_ERR_UNKNOWN";
}

fa_status fa_fwd(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                 int B, int H, int N_q, int N_k, int d, float scale, int causal,
                 hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status s = check_common(B, H, N_q, N_k, d, scale, causal);
  if (s != FA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{bf(q), bf(k), bf(v), bf(o), lse, B, H, N_q, N_k, d, scale, causal != 0, stream};
  return from_hip(fa::launch_fwd(a));
}

size_t fa_bwd_workspace_bytes(int B, int H, int N_q, int N_k, int d) {
  (void)N_k;
  (void)d;
  if (B < 1 || H < 1 || N_q < 1) return 0;
  // -D then -LSE / scale, each [B, H, N_q] fp32 padded to 16 bytes
  return 2 * round_up16((size_t)B * H * N_q * sizeof(float));
}

namespace {

// Shared validation of fa_bwd and its phases; `need` says which pointers the phase uses
// (bit 0: o and lse, 1: q/k/v, 2: dk/dv, 3: dq; dout and the workspace are always used).
fa_status bwd_checked(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                      const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk,
                      fa_bf16* dv, void* workspace, size_t workspace_bytes, int B, int H,
                      int N_q, int N_k, int d, float scale, int causal, hipStream_t stream,
                      unsigned need, unsigned phases, const int32_t* lens_q = nullptr,
                      const int32_t* lens_k = nullptr, const fa::DropoutParams* drop = nullptr,
                      const fa::BiasParams* bias = nullptr, int d_v = 0, int H_kv = 0) {
  const bool varlen = lens_q != nullptr;
  const bool use_o = need & 1u, use_qkv = need & 2u, use_kv_out = need & 4u, use_q_out = need & 8u;
  if (!dout || (use_o && (!o || !lse)) || (use_qkv && (!q || !k || !v)) ||
      (use_kv_out && (!dk || !dv)) || (use_q_out && !dq))
    return FA_ERR_NULL;
  // per-sequence lengths define their own causal alignment; the padded extents need not
  // satisfy N_q <= N_k
  fa_status s = check_common(B, H, N_q, N_k, d, scale, varlen ? 0 : causal);
  if (s != FA_OK) return s;
  if (!aligned16(dout) || (use_o && (!aligned16(o) || !aligned16(lse))) ||
      (use_qkv && (!aligned16(q) || !aligned16(k) || !aligned16(v))) ||
      (use_kv_out && (!aligned16(dk) || !aligned16(dv))) || (use_q_out && !aligned16(dq)))
    return FA_ERR_ALIGN;
  if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, H, N_q, N_k, d))
    return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  fa::BwdArgs a{bf(q), bf(k), bf(v), bf(o), lse, bf(dout), bf(dq), bf(dk), bf(dv),
                static_cast<float*>(workspace), B, H, N_q, N_k, d, scale, causal != 0, stream,
                lens_q, lens_k};
  if (drop) a.drop = *drop;
  if (bias) a.bias = *bias;
  a.d_v = d_v;
  a.Hkv = H_kv;
  return from_hip(fa::launch_bwd(a, phases));
}

}  // namespace

fa_status fa_bwd(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                 const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
                 void* workspace, size_t workspace_bytes, int B, int H, int N_q, int N_k, int d,
                 float scale, int causal, hipStream_t stream) {
  return bwd_checked(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N_q,
                     N_k, d, scale, causal, stream, 15u, 7u);
}

fa_status fa_bwd_preprocess(const fa_bf16* o, const float* lse, const fa_bf16* dout,
                            void* workspace, size_t workspace_bytes, int B, int H, int N_q,
                            int N_k, int d, hipStream_t stream) {
  // scale and causal play no part in D; pass valid values to the shared checks
  return bwd_checked(nullptr, nullptr, nullptr, o, lse, dout, nullptr, nullptr, nullptr,
                     workspace, workspace_bytes, B, H, N_q, N_k, d, 1.f, 0, stream, 1u, 1u);
}

fa_status fa_bwd_dkdv(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v,
                      const fa_bf16* dout, fa_bf16* dk, fa_bf16* dv, void* workspace,
                      size_t workspace_bytes, int B, int H, int N_q, int N_k, int d, float scale,
                      int causal, hipStream_t stream) {
  return bwd_checked(q, k, v, nullptr, nullptr, dout, nullptr, dk, dv, workspace,
                     workspace_bytes, B, H, N_q, N_k, d, scale, causal, stream, 6u, 2u);
}

fa_status fa_bwd_dq(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* dout,
                    fa_bf16* dq, void* workspace, size_t workspace_bytes, int B, int H, int N_q,
                    int N_k, int d, float scale, int causal, hipStream_t stream) {
  return bwd_checked(q, k, v, nullptr, nullptr, dout, dq, nullptr, nullptr, workspace,
                     workspace_bytes, B, H, N_q, N_k, d, scale, causal, stream, 10u, 4u);
}

int fa_decode_num_splits(int B, int H, int N_k, int d) {
  if (B < 1 || H < 1 || N_k < 1) return 1;
  return fa::decode_auto_splits(B, H, N_k, d);
}

size_t fa_decode_workspace_bytes(int B, int H, int N_k, int d, int num_splits) {
  if (B < 1 || H < 1 || N_k < 1 || (d != 64 && d != 128) || num_splits < 0) return 0;
  const int c = num_splits == 0 ? fa_decode_num_splits(B, H, N_k, d) : num_splits;
  const size_t rows = (size_t)B * H * c;
  return round_up16(rows * d * sizeof(float)) + round_up16(rows * sizeof(float));
}

fa_status fa_decode(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                    void* workspace, size_t workspace_bytes, int B, int H, int N_q, int N_k,
                    int d, float scale, int causal, int num_splits, hipStream_t stream) {
  int c = 0;
  const fa_status s =
      fa::decode_validate(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, num_splits, &c);
  if (s != FA_OK) return s;
  if (!workspace || workspace_bytes < fa_decode_workspace_bytes(B, H, N_k, d, c))
    return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  return fa::decode_run(q, k, v, o, lse, workspace, B, H, N_k, d, scale, c, stream);
}

int fa_decode_gqa_num_splits(int B, int H, int H_kv, int N_k, int d) {
  if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0 || N_k < 1) return 1;
  return H_kv == H ? fa::decode_auto_splits(B, H, N_k, d)
                   : fa::decode_paged_auto_splits(B, H, H_kv, N_k, d);
}

size_t fa_decode_gqa_workspace_bytes(int B, int H, int H_kv, int N_k, int d, int num_splits) {
  if (B < 1 || H < 1 || H_kv < 1 || N_k < 1 || (d != 64 && d != 128) || num_splits < 0) return 0;
  const int c = num_splits == 0 ? fa_decode_gqa_num_splits(B, H, H_kv, N_k, d) : num_splits;
  const size_t rows = (size_t)B * H * c;
  return round_up16(rows * d * sizeof(float)) + round_up16(rows * sizeof(float));
}

fa_status fa_decode_gqa(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                        float* lse, void* workspace, size_t workspace_bytes, int B, int H,
                        int H_kv, int N_k, int d, float scale, int num_splits,
                        hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status s = check_common(B, H, 1, N_k, d, scale, 0);
  if (s != FA_OK) return s;
  if (H_kv < 1 || H % H_kv != 0) return FA_ERR_ARG;
  if (num_splits < 0 || num_splits > 1024 || num_splits > N_k) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const int c = num_splits == 0 ? fa_decode_gqa_num_splits(B, H, H_kv, N_k, d) : num_splits;
  if (!workspace || workspace_bytes < fa_decode_gqa_workspace_bytes(B, H, H_kv, N_k, d, c))
    return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  const size_t rows = (size_t)B * H * c;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             round_up16(rows * d * sizeof(float)));
  fa::DecodeArgs a{bf(q), bf(k), bf(v), bf(o), lse, part_o, part_lse, B, H, N_k, d, c, scale,
                   stream};
  a.Hkv = H_kv;
  return from_hip(fa::launch_decode(a));
}

int fa_decode_paged_num_splits(int B, int H, int H_kv, int max_blocks_per_seq, int block_size,
                               int d) {
  if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0 || max_blocks_per_seq < 1 || block_size < 1)
    return 1;
  const long long max_len = (long long)max_blocks_per_seq * block_size;
  if (max_len >= (1LL << 31)) return 1;
  return fa::decode_paged_auto_splits(B, H, H_kv, (int)max_len, d);
}

size_t fa_decode_paged_workspace_bytes(int B, int H, int H_kv, int max_blocks_per_seq,
                                       int block_size, int d, int num_splits) {
  if (B < 1 || H < 1 || H_kv < 1 || max_blocks_per_seq < 1 || block_size < 1 ||
      (d != 64 && d != 128) || num_splits < 0)
    return 0;
  const int c = num_splits == 0
                    ? fa_decode_paged_num_splits(B, H, H_kv, max_blocks_per_seq, block_size, d)
                    : num_splits;
  const size_t rows = (size_t)B * H * c;
  return round_up16(rows * d * sizeof(float)) + round_up16(rows * sizeof(float));
}

fa_status fa_decode_paged(const fa_bf16* q, const fa_bf16* k_cache, const fa_bf16* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, fa_bf16* o,
                          float* lse, void* workspace, size_t workspace_bytes, int B, int H,
                          int H_kv, int d, int block_size, int num_blocks, int max_blocks_per_seq,
                          float scale, int num_splits, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || H_kv < 1 || num_blocks < 1 || max_blocks_per_seq < 1 || block_size < 1)
    return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (H % H_kv != 0) return FA_ERR_ARG;
  if (block_size > 4096 || (block_size & (block_size - 1)) != 0) return FA_ERR_ARG;
  const long long max_len = (long long)max_blocks_per_seq * block_size;
  if (max_len >= (1LL << 31) || (long long)B * max_blocks_per_seq >= (1LL << 31) ||
      (long long)B * H >= (1LL << 31))
    return FA_ERR_SHAPE;
  // the cache holds num_blocks * H_kv * block_size rows of d elements
  if ((long long)num_blocks * H_kv * block_size >= (1LL << 40)) return FA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > 1024 || num_splits > max_len) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return FA_ERR_ALIGN;
  const int c = num_splits == 0
                    ? fa_decode_paged_num_splits(B, H, H_kv, max_blocks_per_seq, block_size, d)
                    : num_splits;
  if (!workspace || workspace_bytes < fa_decode_paged_workspace_bytes(
                                          B, H, H_kv, max_blocks_per_seq, block_size, d, c))
    return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  const size_t rows = (size_t)B * H * c;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             round_up16(rows * d * sizeof(float)));
  fa::DecodePagedArgs a{bf(q), bf(k_cache), bf(v_cache), block_table, seq_lens, bf(o), lse,
                        part_o, part_lse, B, H, H_kv, d, block_size, num_blocks,
                        max_blocks_per_seq, c, scale, stream};
  return from_hip(fa::launch_decode_paged(a));
}

namespace {
bool lens_ok(const int32_t* p) { return p && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
}  // namespace

namespace {
// Dropout parameters from the drop probability: threshold t = floor((1 - p) 65536) in double
// precision (a 16-bit draw keeps iff below t), scale 1 / (1 - p); p = 0 gives t = 65536 (no
// dropout, the plain kernels).
fa_status dropout_params(float p_drop, uint64_t seed, uint32_t offset, fa::DropoutParams* out) {
  if (!(p_drop >= 0.f) || !(p_drop < 1.f)) return FA_ERR_ARG;
  const double keep = 1.0 - (double)p_drop;
  out->key0 = (unsigned)(seed & 0xFFFFFFFFull);
  out->key1 = (unsigned)(seed >> 32);
  out->offset = offset;
  out->thresh = (unsigned)floor(keep * 65536.0);
  out->inv_keep = (float)(1.0 / keep);
  return FA_OK;
}
}  // namespace

fa_status fa_fwd_dropout(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                         float* lse, int B, int H, int N_q, int N_k, int d, float scale,
                         int causal, float p_drop, uint64_t seed, uint32_t offset,
                         hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status s = check_common(B, H, N_q, N_k, d, scale, causal);
  if (s != FA_OK) return s;
  fa::DropoutParams dp;
  s = dropout_params(p_drop, seed, offset, &dp);
  if (s != FA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{bf(q), bf(k), bf(v), bf(o), lse, B, H, N_q, N_k, d, scale, causal != 0, stream};
  a.drop = dp;
  return from_hip(fa::launch_fwd(a));
}

fa_status fa_bwd_dropout(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                         const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk,
                         fa_bf16* dv, void* workspace, size_t workspace_bytes, int B, int H,
                         int N_q, int N_k, int d, float scale, int causal, float p_drop,
                         uint64_t seed, uint32_t offset, hipStream_t stream) {
  fa::DropoutParams dp;
  const fa_status s = dropout_params(p_drop, seed, offset, &dp);
  if (s != FA_OK) return s;
  return bwd_checked(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N_q,
                     N_k, d, scale, causal, stream, 15u, 7u, nullptr, nullptr, &dp);
}

size_t fa_fwd_fp8_workspace_bytes(int B, int H, int N_q, int N_k, int d) {
  if (B < 1 || H < 1 || N_q < 1 || N_k < 1 || (d != 64 && d != 128)) return 0;
  size_t bytes = 0;
  fa::fp8_workspace_layout(nullptr, B, H, N_q, N_k, d, &bytes);
  return bytes;
}

fa_status fa_fwd_fp8(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                     float* lse, int B, int H, int N_q, int N_k, int d, float scale, int causal,
                     int incoherent, uint64_t seed, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status s = check_common(B, H, N_q, N_k, d, scale, causal);
  if (s != FA_OK) return s;
  // the transposed V codes are [B, H, d, N_k padded to 64]: keep their byte count in range
  if ((long long)B * H * d * ((N_k + 63) / 64 * 64) >= (1LL << 31)) return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  if (!workspace || workspace_bytes < fa_fwd_fp8_workspace_bytes(B, H, N_q, N_k, d))
    return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  fa::Fp8Args a{};
  a.q = bf(q);
  a.k = bf(k);
  a.v = bf(v);
  a.o = bf(o);
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Nq = N_q;
  a.Nk = N_k;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  a.incoherent = incoherent != 0;
  a.key0 = (unsigned)(seed & 0xFFFFFFFFull);
  a.key1 = (unsigned)(seed >> 32);
  a.ws = fa::fp8_workspace_layout(workspace, B, H, N_q, N_k, d, nullptr);
  a.stream = stream;
  return from_hip(fa::launch_fwd_fp8(a));
}

namespace {
// Bias strides: non-negative multiples of 8 elements (16-byte rows), pointer 16-byte aligned, and
// one head's extent ((N_q - 1) sq + N_k elements) within 2^30 so byte offsets stay 32-bit.
fa_status bias_params(const fa_bf16* bias, int64_t sb, int64_t sh, int64_t sq, int N_q, int N_k,
                      fa::BiasParams* out) {
  if (!bias) return FA_ERR_NULL;
  if (!aligned16(bias)) return FA_ERR_ALIGN;
  if (sb < 0 || sh < 0 || sq < 0 || (sb % 8) || (sh % 8) || (sq % 8)) return FA_ERR_ARG;
  if ((long double)(N_q - 1) * sq + N_k >= (long double)(1LL << 30)) return FA_ERR_SHAPE;
  out->ptr = reinterpret_cast<const __bf16*>(bias);
  out->sb = sb;
  out->sh = sh;
  out->sq = sq;
  return FA_OK;
}
}  // namespace

fa_status fa_fwd_bias(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                      float* lse, const fa_bf16* bias, int64_t bias_stride_b,
                      int64_t bias_stride_h, int64_t bias_stride_q, int B, int H, int N_q, int N_k,
                      int d, float scale, int causal, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status s = check_common(B, H, N_q, N_k, d, scale, causal);
  if (s != FA_OK) return s;
  fa::BiasParams bp;
  s = bias_params(bias, bias_stride_b, bias_stride_h, bias_stride_q, N_q, N_k, &bp);
  if (s != FA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{bf(q), bf(k), bf(v), bf(o), lse, B, H, N_q, N_k, d, scale, causal != 0, stream};
  a.bias = bp;
  return from_hip(fa::launch_fwd(a));
}

fa_status fa_bwd_bias(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                      const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk,
                      fa_bf16* dv, const fa_bf16* bias, int64_t bias_stride_b,
                      int64_t bias_stride_h, int64_t bias_stride_q, void* workspace,
                      size_t workspace_bytes, int B, int H, int N_q, int N_k, int d, float scale,
                      int causal, hipStream_t stream) {
  fa::BiasParams bp;
  const fa_status s = bias_params(bias, bias_stride_b, bias_stride_h, bias_stride_q, N_q, N_k, &bp);
  if (s != FA_OK) return s;
  return bwd_checked(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N_q,
                     N_k, d, scale, causal, stream, 15u, 7u, nullptr, nullptr, nullptr, &bp);
}

fa_status fa_fwd_dv(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                    int B, int H, int N_q, int N_k, int d, int d_v, float scale, int causal,
                    hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status s = check_common(B, H, N_q, N_k, d, scale, causal);
  if (s != FA_OK) return s;
  if (d_v != 64 && d_v != 128) return FA_ERR_HEADDIM;
  if (!head_extent_ok(N_q, d_v) || !head_extent_ok(N_k, d_v)) return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{bf(q), bf(k), bf(v), bf(o), lse, B, H, N_q, N_k, d, scale, causal != 0, stream};
  a.d_v = d_v;
  return from_hip(fa::launch_fwd(a));
}

fa_status fa_bwd_dv(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                    const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
                    void* workspace, size_t workspace_bytes, int B, int H, int N_q, int N_k, int d,
                    int d_v, float scale, int causal, hipStream_t stream) {
  if (d_v != 64 && d_v != 128) return FA_ERR_HEADDIM;
  if (N_q >= 1 && N_k >= 1 && (!head_extent_ok(N_q, d_v) || !head_extent_ok(N_k, d_v)))
    return FA_ERR_SHAPE;
  return bwd_checked(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N_q,
                     N_k, d, scale, causal, stream, 15u, 7u, nullptr, nullptr, nullptr, nullptr,
                     d_v);
}

fa_status fa_fwd_varlen(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                        float* lse, const int32_t* seq_lens_q, const int32_t* seq_lens_k, int B,
                        int H, int N_q, int N_k, int d, float scale, int causal,
                        hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !seq_lens_q || !seq_lens_k) return FA_ERR_NULL;
  fa_status s = check_common(B, H, N_q, N_k, d, scale, 0);
  if (s != FA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !lens_ok(seq_lens_q) || !lens_ok(seq_lens_k))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{bf(q), bf(k), bf(v), bf(o), lse, B, H, N_q, N_k, d, scale, causal != 0, stream,
                seq_lens_q, seq_lens_k};
  return from_hip(fa::launch_fwd(a));
}

fa_status fa_bwd_varlen(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                        const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk,
                        fa_bf16* dv, const int32_t* seq_lens_q, const int32_t* seq_lens_k,
                        void* workspace, size_t workspace_bytes, int B, int H, int N_q, int N_k,
                        int d, float scale, int causal, hipStream_t stream) {
  if (!seq_lens_q || !seq_lens_k) return FA_ERR_NULL;
  if (!lens_ok(seq_lens_q) || !lens_ok(seq_lens_k)) return FA_ERR_ALIGN;
  return bwd_checked(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N_q,
                     N_k, d, scale, causal, stream, 15u, 7u, seq_lens_q, seq_lens_k);
}

fa_status fa_fwd_gqa(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                     int B, int H, int H_kv, int N_q, int N_k, int d, float scale, int causal,
                     hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status s = check_common(B, H, N_q, N_k, d, scale, causal);
  if (s != FA_OK) return s;
  if (H_kv < 1 || H % H_kv != 0) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{bf(q), bf(k), bf(v), bf(o), lse, B, H, N_q, N_k, d, scale, causal != 0, stream};
  a.Hkv = H_kv;
  return from_hip(fa::launch_fwd(a));
}

size_t fa_bwd_gqa_workspace_bytes(int B, int H, int H_kv, int N_q, int N_k, int d) {
  const size_t base = fa_bwd_workspace_bytes(B, H, N_q, N_k, d);
  if (base == 0 || H_kv < 1 || H % H_kv != 0 || N_k < 1 || (d != 64 && d != 128)) return 0;
  if (!fa::bwd_gqa_uses_partials(B, H, H_kv, N_k)) return base;
  // fp32 partial rows of dK and dV per query head
  return base + 2 * round_up16((size_t)B * H * N_k * d * sizeof(float));
}

fa_status fa_bwd_gqa(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                     const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
                     void* workspace, size_t workspace_bytes, int B, int H, int H_kv, int N_q,
                     int N_k, int d, float scale, int causal, hipStream_t stream) {
  if (H_kv < 1 || (H >= 1 && H % H_kv != 0)) return FA_ERR_ARG;
  const size_t need = fa_bwd_gqa_workspace_bytes(B, H, H_kv, N_q, N_k, d);
  if (need != 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  return bwd_checked(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N_q,
                     N_k, d, scale, causal, stream, 15u, 7u, nullptr, nullptr, nullptr, nullptr,
                     0, H_kv);
}

fa_status fa_fwd_ext(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                     const int32_t* seq_lens_q, const int32_t* seq_lens_k, int B, int H, int H_kv,
                     int N_q, int N_k, int d, float scale, int causal, float p_drop,
                     uint64_t seed, uint32_t offset, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  const bool varlen = seq_lens_q != nullptr || seq_lens_k != nullptr;
  if (varlen && (!seq_lens_q || !seq_lens_k)) return FA_ERR_ARG;
  fa_status s = check_common(B, H, N_q, N_k, d, scale, varlen ? 0 : causal);
  if (s != FA_OK) return s;
  if (H_kv < 1 || H % H_kv != 0) return FA_ERR_ARG;
  fa::DropoutParams dp;
  s = dropout_params(p_drop, seed, offset, &dp);
  if (s != FA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  if (varlen && (!lens_ok(seq_lens_q) || !lens_ok(seq_lens_k))) return FA_ERR_ALIGN;
  fa::FwdArgs a{bf(q), bf(k), bf(v), bf(o), lse, B, H, N_q, N_k, d, scale, causal != 0, stream,
                seq_lens_q, seq_lens_k};
  a.drop = dp;
  a.Hkv = H_kv;
  return from_hip(fa::launch_fwd(a));
}

size_t fa_bwd_ext_workspace_bytes(int B, int H, int H_kv, int N_q, int N_k, int d) {
  const size_t base = fa_bwd_workspace_bytes(B, H, N_q, N_k, d);
  if (base == 0 || H_kv < 1 || H % H_kv != 0 || N_k < 1 || (d != 64 && d != 128)) return 0;
  if (H_kv == H) return base;
  // grouped K/V heads: room for the fp32 partial rows of dK and dV per query head, which the
  // dK/dV pass uses with per-sequence lengths (unknown here) and on small grids
  return base + 2 * round_up16((size_t)B * H * N_k * d * sizeof(float));
}

fa_status fa_bwd_ext(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                     const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
                     const int32_t* seq_lens_q, const int32_t* seq_lens_k, void* workspace,
                     size_t workspace_bytes, int B, int H, int H_kv, int N_q, int N_k, int d,
                     float scale, int causal, float p_drop, uint64_t seed, uint32_t offset,
                     hipStream_t stream) {
  const bool varlen = seq_lens_q != nullptr || seq_lens_k != nullptr;
  if (varlen && (!seq_lens_q || !seq_lens_k)) return FA_ERR_ARG;
  if (varlen && (!lens_ok(seq_lens_q) || !lens_ok(seq_lens_k))) return FA_ERR_ALIGN;
  if (H_kv < 1 || (H >= 1 && H % H_kv != 0)) return FA_ERR_ARG;
  fa::DropoutParams dp;
  const fa_status s = dropout_params(p_drop, seed, offset, &dp);
  if (s != FA_OK) return s;
  const size_t need = fa_bwd_ext_workspace_bytes(B, H, H_kv, N_q, N_k, d);
  if (need != 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  return bwd_checked(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N_q,
                     N_k, d, scale, causal, stream, 15u, 7u, varlen ? seq_lens_q : nullptr,
                     varlen ? seq_lens_k : nullptr, &dp, nullptr, 0, H_kv);
}

}  // extern "C"
