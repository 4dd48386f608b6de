// Host-side launch entry points of the attention kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "fa.h"

namespace fa {

// Dropout on the attention probabilities (Philox-4x32-10 keyed by the 64-bit seed; the call
// layout and the keep rule are stated beside the generator in fa_device.h). thresh = 65536
// means no dropout.
struct DropoutParams {
  unsigned key0 = 0, key1 = 0, offset = 0, thresh = 65536;
  float inv_keep = 1.f;
};

// Additive bias on the scores: element (b, h, i, j) at ptr[b sb + h sh + i sq + j] (bf16; strides
// in elements, multiples of 8; -inf masks). ptr = nullptr: no bias.
struct BiasParams {
  const __bf16* ptr = nullptr;
  long long sb = 0, sh = 0, sq = 0;
};

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int B, H, Nq, Nk, d;
  float scale;
  bool causal;
  hipStream_t stream;
  const int* lens_q = nullptr;  // per-sequence lengths (both or neither), device int32 [B]
  const int* lens_k = nullptr;
  DropoutParams drop{};
  BiasParams bias{};
  int d_v = 0;  // head dimension of V and O; 0: the same as d
  int Hkv = 0;  // key/value heads (H a multiple of Hkv); 0: the same as H
};

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const float* lse;
  const __bf16* dout;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* delta;  // workspace: -D = -rowsum(dO * O) [B, H, Nq], then -LSE / scale [B, H, Nq]
  int B, H, Nq, Nk, d;
  float scale;
  bool causal;
  hipStream_t stream;
  const int* lens_q = nullptr;  // per-sequence lengths (both or neither), device int32 [B]
  const int* lens_k = nullptr;
  DropoutParams drop{};
  BiasParams bias{};
  int d_v = 0;  // head dimension of V, O, dO and dV; 0: the same as d
  int Hkv = 0;  // key/value heads of K, V, dK and dV (H a multiple of Hkv); 0: the same as H
};

struct DecodeArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  float* part_o;    // workspace: [B, H, splits, d]
  float* part_lse;  // workspace: [B, H, splits]
  int B, H, Nk, d, splits;
  float scale;
  hipStream_t stream;
  int Hkv = 0;  // K/V heads [B, Hkv, Nk, d] (0 or H: one per query head)
};

struct DecodePagedArgs {
  const __bf16* q;        // [B, H, d]
  const __bf16* k_cache;  // [num_blocks, H_kv, block_size, d]
  const __bf16* v_cache;
  const int* block_table;  // [B, max_blocks]
  const int* seq_lens;     // [B]
  __bf16* o;               // [B, H, d]
  float* lse;              // [B, H]
  float* part_o;           // workspace: [B, H, splits, d]
  float* part_lse;         // workspace: [B, H, splits]
  int B, H, Hkv, d, block_size, num_blocks, max_blocks, splits;
  float scale;
  hipStream_t stream;
};

// FP8 forward: device buffers inside the caller's workspace (see fp8_workspace_layout)
struct Fp8Workspace {
  unsigned char* q8 = nullptr;   // [B, H, Nq, d] E4M3 codes of (rotated) Q
  unsigned char* k8 = nullptr;   // [B, H, Nk, d] E4M3 codes of (rotated) K
  unsigned char* v8t = nullptr;  // [B, H, d, Nk padded to 64] E4M3 codes of V, transposed
  float* sq = nullptr;           // [B, H, ceil(Nq / 32)] Q block scales
  float* sk = nullptr;           // [B, H, ceil(Nk / 64)] K block scales
  float* vpart = nullptr;        // [B, H, ceil(Nk / 64)] max |V| per 64 keys
  float* sv = nullptr;           // [B, H] V scale per head
};

struct Fp8Args {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int B, H, Nq, Nk, d;
  float scale;
  bool causal;
  bool incoherent;
  unsigned key0, key1;  // seed of the random signs
  Fp8Workspace ws;
  hipStream_t stream;
};

// Carves the FP8 buffers out of `base` (nullptr: only computes the size); *bytes = total size.
Fp8Workspace fp8_workspace_layout(void* base, int B, int H, int Nq, int Nk, int d, size_t* bytes);
hipError_t launch_fwd_fp8(const Fp8Args& a);

hipError_t launch_fwd(const FwdArgs& a);
// Offset (in floats) of L2 after D in the backward workspace.
size_t bwd_lse2_offset(int B, int H, int Nq);
// Grouped query heads: whether the dK/dV pass runs one workgroup per query head and sums fp32
// partial rows in a second kernel (too few K/V workgroups otherwise), and where those rows start
// in the workspace (floats; [B H, N_k, d] for dK, then the same for dV).
bool bwd_gqa_uses_partials(int B, int H, int Hkv, int Nk);
size_t bwd_part_offset(int B, int H, int Nq);
// Backward phases; `phase_mask` bit 0 = D preprocess, bit 1 = dK/dV, bit 2 = dQ.
hipError_t launch_bwd(const BwdArgs& a, unsigned phase_mask = 7u);
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_decode_paged(const DecodePagedArgs& a);

// fa_decode's argument checks (everything but the workspace); *splits receives the split count
// the call uses (num_splits, or the automatic count for 0).
fa_status decode_validate(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                          const float* lse, int B, int H, int N_q, int N_k, int d, float scale,
                          int causal, int num_splits, int* splits);
// Launches the split and combine kernels of a validated decode with its partials in `workspace`
// (at least fa_decode_workspace_bytes(B, H, N_k, d, splits) bytes, 16-byte aligned).
fa_status decode_run(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                     void* workspace, int B, int H, int N_k, int d, float scale, int splits,
                     hipStream_t stream);

// K/V heads an XCD works on at a time (xcd_map), for `heads` heads whose workgroups each stream
// bytes_per_head from their head: all of them while an XCD's heads stream at most its share of
// the last-level cache, else 2 (more when that many heads' rows fit in about 2 MiB).
int xcd_head_group(size_t bytes_per_head, long long heads);

// Split count used by the decode when the caller passes 0.
int decode_auto_splits(int B, int H, int Nk, int d);
// Split count used by the paged decode when the caller passes 0.
int decode_paged_auto_splits(int B, int H, int Hkv, int max_len, int d);

}  // namespace fa
