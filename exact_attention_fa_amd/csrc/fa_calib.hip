// Measurement only (not part of the attention library): the matrix-core rate this card sustains on
// random bf16 operands, and on random E4M3 operands, and its shader clock meanwhile. The
// attention kernels' fractions of the published dense peaks are read against them, since the
// card lowers its clock under such loads.
//
// Every wave keeps 8 independent accumulators of v_mfma_f32_32x32x16_bf16 (or of the E4M3
// v_mfma_scale_f32_32x32x64_f8f6f4) busy with operands read once from a buffer of random values
// (so the datapath switches as it does on attention data), and times itself with s_memtime
// (shader clock cycles) and s_memrealtime (constant 100 MHz), from which the host derives the
// clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;

// operands: [gridDim.x * 256 threads][2 * kChains] 16-byte chunks of random bf16 values;
// clocks: [gridDim.x * 4 waves][4] = start/end shader clock, start/end real time;
// sink: [gridDim.x * 256] one float per thread, keeps the products alive.
__global__ __attribute__((amdgpu_waves_per_eu(2, 2))) __launch_bounds__(256) void mfma_loop_kernel(
    const u32x4* __restrict__ operands, int iters, unsigned long long* __restrict__ clocks,
    float* __restrict__ sink) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int tid = blockIdx.x * 256 + threadIdx.x;
  bf16x8 a[kChains], b[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    a[c] = __builtin_bit_cast(bf16x8, operands[(size_t)tid * 2 * kChains + 2 * c]);
    b[c] = __builtin_bit_cast(bf16x8, operands[(size_t)tid * 2 * kChains + 2 * c + 1]);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[tid] = s;
  if ((threadIdx.x & 63) == 0) {
    unsigned long long* w = clocks + ((size_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4;
    w[0] = t0;
    w[1] = t1;
    w[2] = r0;
    w[3] = r1;
  }
#endif
}

// The same loop on E4M3 operands: v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales (the
// FP8 attention kernel's instruction), each operand 32 bytes of random codes per lane.
typedef int i32x8 __attribute__((ext_vector_type(8)));

__global__ __attribute__((amdgpu_waves_per_eu(2, 2))) __launch_bounds__(256) void mfma_fp8_loop_kernel(
    const u32x4* __restrict__ operands, int iters, unsigned long long* __restrict__ clocks,
    float* __restrict__ sink) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int tid = blockIdx.x * 256 + threadIdx.x;
  i32x8 a[kChains], b[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    const u32x4 a0 = operands[(size_t)tid * 4 * kChains + 4 * c];
    const u32x4 a1 = operands[(size_t)tid * 4 * kChains + 4 * c + 1];
    const u32x4 b0 = operands[(size_t)tid * 4 * kChains + 4 * c + 2];
    const u32x4 b1 = operands[(size_t)tid * 4 * kChains + 4 * c + 3];
    a[c] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                 (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    b[c] = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                 (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[c], b[c], acc[c], 0, 0, 0, 127, 0,
                                                                127);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[tid] = s;
  if ((threadIdx.x & 63) == 0) {
    unsigned long long* w = clocks + ((size_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4;
    w[0] = t0;
    w[1] = t1;
    w[2] = r0;
    w[3] = r1;
  }
#endif
}

}  // namespace

// Launches the loop on `blocks` workgroups of 4 waves; every wave issues iters * 8 MFMAs of
// 2 * 32 * 32 * 16 FLOPs. Buffers as described above; returns the launch status.
extern "C" int fa_calib_mfma_bf16(const void* operands, int blocks, int iters, void* clocks,
                                  void* sink, hipStream_t stream) {
  if (!operands || !clocks || !sink || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(operands), iters,
                     static_cast<unsigned long long*>(clocks), static_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The E4M3 loop: every wave issues iters * 8 MFMAs of 2 * 32 * 32 * 64 FLOPs; operands hold
// [blocks * 256 threads][4 * 8] 16-byte chunks of random E4M3 codes; other buffers as above.
extern "C" int fa_calib_mfma_fp8(const void* operands, int blocks, int iters, void* clocks,
                                 void* sink, hipStream_t stream) {
  if (!operands || !clocks || !sink || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_fp8_loop_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(operands), iters,
                     static_cast<unsigned long long*>(clocks), static_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
