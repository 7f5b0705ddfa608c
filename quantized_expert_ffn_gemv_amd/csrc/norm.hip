// Elementwise kernels between stacked layers and the workspace fill.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// z = h / sqrt(mean(h^2) + eps), one workgroup per row, fp32 math.
__global__ __launch_bounds__(256) void k_rmsnorm(const uint16_t* __restrict__ h, uint16_t* __restrict__ z, int H,
                                                  float eps) {
  const int t = blockIdx.x;
  const uint16_t* row = h + (size_t)t * H;
  float ss = 0.0f;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + c);
    const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float a = bf16_lo(vv[i]), b = bf16_hi(vv[i]);
      ss = __builtin_fmaf(a, a, ss);
      ss = __builtin_fmaf(b, b, ss);
    }
  }
  __shared__ float red[4];
  ss = group_sum_f32(ss, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + c);
    uint4 o;
    o.x = pack_bf16x2(bf16_lo(v.x) * inv, bf16_hi(v.x) * inv);
    o.y = pack_bf16x2(bf16_lo(v.y) * inv, bf16_hi(v.y) * inv);
    o.z = pack_bf16x2(bf16_lo(v.z) * inv, bf16_hi(v.z) * inv);
    o.w = pack_bf16x2(bf16_lo(v.w) * inv, bf16_hi(v.w) * inv);
    *reinterpret_cast<uint4*>(z + (size_t)t * H + c) = o;
  }
}

// h = bf16(h + y), 8 elements per thread.
__global__ __launch_bounds__(256) void k_residual(uint16_t* __restrict__ h, const uint16_t* __restrict__ y, size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  uint4 a = reinterpret_cast<uint4*>(h)[i];
  const uint4 b = reinterpret_cast<const uint4*>(y)[i];
  a.x = pack_bf16x2(bf16_lo(a.x) + bf16_lo(b.x), bf16_hi(a.x) + bf16_hi(b.x));
  a.y = pack_bf16x2(bf16_lo(a.y) + bf16_lo(b.y), bf16_hi(a.y) + bf16_hi(b.y));
  a.z = pack_bf16x2(bf16_lo(a.z) + bf16_lo(b.z), bf16_hi(a.z) + bf16_hi(b.z));
  a.w = pack_bf16x2(bf16_lo(a.w) + bf16_lo(b.w), bf16_hi(a.w) + bf16_hi(b.w));
  reinterpret_cast<uint4*>(h)[i] = a;
}

// Zero fill with plain stores (no memset node in captured graphs).
__global__ __launch_bounds__(256) void k_fill(uint32_t* __restrict__ p, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_rmsnorm(const uint16_t* h, uint16_t* z, int T, int H, float eps, hipStream_t st) {
  (void)launch_k(KC_NORM, k_rmsnorm, dim3(T), dim3(256), 0, st, h, z, H, eps);
  return hipGetLastError();
}

hipError_t launch_residual(uint16_t* h, const uint16_t* y, int T, int H, hipStream_t st) {
  const size_t n8 = (size_t)T * H / 8;
  (void)launch_k(KC_RESIDUAL, k_residual, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, h, y, n8);
  return hipGetLastError();
}

hipError_t launch_fill(void* p, size_t bytes, hipStream_t st) {
  const size_t n4 = bytes / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) return hipSuccess;
  (void)launch_k(KC_FILL, k_fill, dim3((unsigned)blocks), dim3(256), 0, st, reinterpret_cast<uint32_t*>(p), n4);
  return hipGetLastError();
}

}  // namespace moe
