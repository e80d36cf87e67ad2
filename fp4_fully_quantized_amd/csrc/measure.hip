// measure.hip -- ceilings of the chip measured on the box, beside the data-sheet
// peaks the benchmark scores against (libfp4_measure.so; measurement only, not
// part of the FP4 library's interface).
//
//   fp4m_mfma_f16   back-to-back v_mfma_f32_32x32x16_f16, the instruction the
//                   NVFP4 GEMM runs (operands decoded from FP4 to f16);
//   fp4m_mfma_fp4   back-to-back v_mfma_scale_f32_32x32x64_f8f6f4 with FP4
//                   operands and E8M0 scales, the instruction of the MXFP4 GEMM;
//   fp4m_stream_*   grid-strided streaming passes over device buffers: read
//                   only, copy, and a quantize-like pass that reads 16 bytes and
//                   writes 4 per lane (coalesced both ways).
//
// The MFMA loops rotate through four operand sets so the matrix pipe sees
// changing data (power draw, and so the clock, depends on it), and keep eight
// independent accumulators per wave so no instruction waits for another's
// result. Every kernel ends with a data-dependent store so its work is kept.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kSets = 4;   // operand sets per wave
constexpr int kAcc = 8;    // independent accumulators per wave

// ops: kSets x 2 (A, B) x 64 lanes x 16 bytes.
__global__ __launch_bounds__(256) void k_mfma_f16(const v4u* __restrict__ ops, float* __restrict__ sink,
                                                   int iters) {
  const int lane = threadIdx.x & 63;
  v8h a[kSets], b[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s) {
    a[s] = __builtin_bit_cast(v8h, ops[(2 * s) * 64 + lane]);
    b[s] = __builtin_bit_cast(v8h, ops[(2 * s + 1) * 64 + lane]);
  }
  v16f acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = (v16f){};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j % kSets], b[(j + 1) % kSets], acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_mfma_fp4(const v4u* __restrict__ ops, float* __restrict__ sink,
                                                   int iters) {
  const int lane = threadIdx.x & 63;
  v8i a[kSets], b[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s) {
    const v4u x = ops[(2 * s) * 64 + lane], y = ops[(2 * s + 1) * 64 + lane];
    a[s] = (v8i){(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
    b[s] = (v8i){(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
  }
  const int scale = 0x7F7F7F7F;   // E8M0 1.0 in every byte
  v16f acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = (v16f){};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j % kSets], b[(j + 1) % kSets], acc[j], 4, 4,
                                                               0, scale, 0, scale);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Read n 16-byte words, four loads in flight per lane.
__global__ __launch_bounds__(256) void k_stream_read(const v4u* __restrict__ src, uint64_t n,
                                                     uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  v4u acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n; i += 4 * stride) {
    const v4u x0 = __builtin_nontemporal_load(src + i);
    const v4u x1 = __builtin_nontemporal_load(src + i + stride);
    const v4u x2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4u x3 = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= x0 ^ x1 ^ x2 ^ x3;
  }
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t h = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (h == 0x9E3779B9u) sink[0] = h;
}

// Copy n 16-byte words.
__global__ __launch_bounds__(256) void k_stream_copy(const v4u* __restrict__ src, v4u* __restrict__ dst,
                                                     uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const v4u x0 = __builtin_nontemporal_load(src + i);
    const v4u x1 = __builtin_nontemporal_load(src + i + stride);
    const v4u x2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4u x3 = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(x0, dst + i);
    __builtin_nontemporal_store(x1, dst + i + stride);
    __builtin_nontemporal_store(x2, dst + i + 2 * stride);
    __builtin_nontemporal_store(x3, dst + i + 3 * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Read n 16-byte words and write one 4-byte word for each (the ratio of a
// bf16 -> FP4 quantize pass: 16 bytes of input per 4 bytes of codes).
__global__ __launch_bounds__(256) void k_stream_read4_write1(const v4u* __restrict__ src,
                                                             uint32_t* __restrict__ dst, uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const v4u x0 = __builtin_nontemporal_load(src + i);
    const v4u x1 = __builtin_nontemporal_load(src + i + stride);
    const v4u x2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4u x3 = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(x0.x ^ x0.y ^ x0.z ^ x0.w, dst + i);
    __builtin_nontemporal_store(x1.x ^ x1.y ^ x1.z ^ x1.w, dst + i + stride);
    __builtin_nontemporal_store(x2.x ^ x2.y ^ x2.z ^ x2.w, dst + i + 2 * stride);
    __builtin_nontemporal_store(x3.x ^ x3.y ^ x3.z ^ x3.w, dst + i + 3 * stride);
  }
  for (; i < n; i += stride) {
    const v4u x = __builtin_nontemporal_load(src + i);
    __builtin_nontemporal_store(x.x ^ x.y ^ x.z ^ x.w, dst + i);
  }
}

int status() { return hipGetLastError() == hipSuccess ? 0 : 1; }

}  // namespace

extern "C" {

// ops: device, 8 KiB (4 sets x A, B x 64 lanes x 16 bytes); sink: device,
// grid * 256 floats. Each of the grid's 256-thread workgroups runs 4 waves,
// each issuing iters * 8 MFMAs. Returns 0, or 1 on a launch error.
int fp4m_mfma_f16(const void* ops, float* sink, int grid, int iters, hipStream_t s) {
  if (!ops || !sink || grid <= 0 || iters <= 0) return 2;
  hipLaunchKernelGGL(k_mfma_f16, dim3(grid), dim3(256), 0, s, static_cast<const v4u*>(ops), sink, iters);
  return status();
}

int fp4m_mfma_fp4(const void* ops, float* sink, int grid, int iters, hipStream_t s) {
  if (!ops || !sink || grid <= 0 || iters <= 0) return 2;
  hipLaunchKernelGGL(k_mfma_fp4, dim3(grid), dim3(256), 0, s, static_cast<const v4u*>(ops), sink, iters);
  return status();
}

// bytes: a multiple of 16; src/dst 16-byte aligned device buffers of that
// size (read4_write1: dst holds bytes / 4). sink: one device word.
int fp4m_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int grid, hipStream_t s) {
  if (!src || !sink || bytes % 16 != 0 || grid <= 0) return 2;
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, s, static_cast<const v4u*>(src), bytes / 16,
                     sink);
  return status();
}

int fp4m_stream_copy(const void* src, void* dst, uint64_t bytes, int grid, hipStream_t s) {
  if (!src || !dst || bytes % 16 != 0 || grid <= 0) return 2;
  hipLaunchKernelGGL(k_stream_copy, dim3(grid), dim3(256), 0, s, static_cast<const v4u*>(src),
                     static_cast<v4u*>(dst), bytes / 16);
  return status();
}

int fp4m_stream_read4_write1(const void* src, void* dst, uint64_t bytes, int grid, hipStream_t s) {
  if (!src || !dst || bytes % 16 != 0 || grid <= 0) return 2;
  hipLaunchKernelGGL(k_stream_read4_write1, dim3(grid), dim3(256), 0, s, static_cast<const v4u*>(src),
                     static_cast<uint32_t*>(dst), bytes / 16);
  return status();
}

}  // extern "C"
