// Chip-ceiling microbenchmarks (include/moe_peaks.h): the matrix-core rate on
// random operands and the HBM read-stream rate.  Not used by the MoE layer.
#include <hip/hip_runtime.h>

#include "../../include/moe_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;        // independent accumulators per wavefront
constexpr int kFrags = 4;         // distinct operand fragments per wavefront
constexpr int kThreads = 256;
constexpr int kWavesOfData = 1024;  // operand buffer: fragments of 1024 wavefronts
// bytes of one wavefront's operands: kFrags A and kFrags B fragments of 32 bytes per lane
constexpr size_t kWaveBytes = (size_t)2 * kFrags * 64 * 32;

// One wavefront's operand fragments: lane l reads 32 bytes per fragment.  Both
// kinds read the same bytes; bf16 uses the first 16 of each.
__device__ __forceinline__ const int32_t* wave_data(const void* base) {
  const int wave = (blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) % kWavesOfData;
  return reinterpret_cast<const int32_t*>(static_cast<const char*>(base) + wave * kWaveBytes) +
         (threadIdx.x & 63) * 8;
}

__global__ __launch_bounds__(kThreads) void mfma_bf16_kernel(const void* src, int iters,
                                                             float* out) {
  const int32_t* p = wave_data(src);
  bf16x8 a[kFrags], b[kFrags];
#pragma unroll
  for (int f = 0; f < kFrags; ++f) {
    const int32_t* pa = p + f * 64 * 8;
    const int32_t* pb = p + (kFrags + f) * 64 * 8;
    a[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const int4*>(pa));
    b[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const int4*>(pb));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  // kFrags rounds per trip, so that every fragment index is a constant
  for (int it = 0; it < iters; it += kFrags) {
#pragma unroll
    for (int r = 0; r < kFrags; ++r)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c % kFrags], b[(c + r) % kFrags],
                                                         acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void mfma_fp8_kernel(const void* src, int iters,
                                                            float* out) {
  const int32_t* p = wave_data(src);
  i32x8 a[kFrags], b[kFrags];
#pragma unroll
  for (int f = 0; f < kFrags; ++f) {
    const int32_t* pa = p + f * 64 * 8;
    const int32_t* pb = p + (kFrags + f) * 64 * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[f][i] = pa[i];
      b[f][i] = pb[i];
    }
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; it += kFrags) {
#pragma unroll
    for (int r = 0; r < kFrags; ++r)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        // E4M3 x E4M3 (cbsz = blgp = 0), unit scales (E8M0 127 = 2^0)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a[c % kFrags], b[(c + r) % kFrags], acc[c], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void read_kernel(const uint4* src, size_t chunk16,
                                                        uint32_t* out) {
  // block b streams the contiguous elements [b * chunk16, (b + 1) * chunk16)
  // (chunk16 a multiple of kThreads, under 2 GiB) with 16-byte buffer loads
  // marked non-temporal, U of them in flight per lane
  constexpr int U = 8;
  constexpr int kNonTemporal = 2;  // buffer cache-policy bit NT
  const char* base = reinterpret_cast<const char*>(src + (size_t)blockIdx.x * chunk16);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(base), 0, (int)(chunk16 * 16), 0x00020000);
  uint32_t x = 0;
  size_t j = threadIdx.x;
  for (; j + (U - 1) * kThreads < chunk16; j += U * kThreads) {
    uint32_t w[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((j + u * kThreads) * 16), 0,
                                                           kNonTemporal);
      w[u][0] = v[0]; w[u][1] = v[1]; w[u][2] = v[2]; w[u][3] = v[3];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= w[u][0] ^ w[u][1] ^ w[u][2] ^ w[u][3];
  }
  for (; j < chunk16; j += kThreads) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(j * 16), 0, kNonTemporal);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // block XOR through LDS
  __shared__ uint32_t part[kThreads];
  part[threadIdx.x] = x;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] ^= part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = part[0];
}

}  // namespace

extern "C" {

size_t moe_peaks_operand_bytes(void) { return kWaveBytes * kWavesOfData; }

double moe_peaks_mfma_flops(int kind, int blocks, int iters) {
  const double per_mfma = kind == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  return per_mfma * kChains * (double)iters * (double)blocks * (kThreads / 64);
}

int moe_peaks_mfma(int kind, const void* operands, int blocks, int iters, float* out,
                   void* stream) {
  if ((kind != 0 && kind != 1) || !operands || !out || blocks < 1 || iters < 1 ||
      iters % kFrags)
    return MOE_PEAKS_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(mfma_bf16_kernel, dim3(blocks), dim3(kThreads), 0, s, operands, iters, out);
  else
    hipLaunchKernelGGL(mfma_fp8_kernel, dim3(blocks), dim3(kThreads), 0, s, operands, iters, out);
  return hipGetLastError() == hipSuccess ? MOE_PEAKS_OK : MOE_PEAKS_EHIP;
}

int moe_peaks_read(const void* src, size_t bytes, int blocks, uint32_t* out, void* stream) {
  if (!src || !out || blocks < 1 || bytes == 0 || bytes % 4096) return MOE_PEAKS_EINVAL;
  const size_t chunk = bytes / (size_t)blocks;  // bytes per block
  if (bytes % ((size_t)blocks * 4096) || chunk >= ((size_t)1 << 31)) return MOE_PEAKS_EINVAL;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                     chunk / 16, out);
  return hipGetLastError() == hipSuccess ? MOE_PEAKS_OK : MOE_PEAKS_EHIP;
}

}  // extern "C"
