// LastKV previous-chunk blending (gfx950): the pre-step that builds the blended K~, V~ of
// the most recent completed chunk, and its backward.
//
// Source: zefan-cai.github.io/en/blog/lastkv-rl ("In RL, Does the Trainer Evaluate the
// Policy That Generated the Rollout?"), section "LastKV: making recurrence boundaries part
// of the policy", the chunk attention and previous-chunk blending equations: the
// chunk just completed keeps its per-layer K/V and mixes it with the last-layer K/V
// through one gate per layer and KV head,
//   x~ = (1 - alpha_g) x_layer + alpha_g x_last   (x = K or V),
// and only older chunks are read as last-layer K/V alone.  The chunk's attention then
// runs over [last-layer K/V of older chunks; x~ of the previous chunk; the current chunk's
// own per-layer K/V, causal], which is the resident-history-plus-causal-part shape of the
// replay attention kernels.
//
// blend_fwd: one thread per 8 elements, fp32 arithmetic, stored in the input dtype.
// blend_bwd: one workgroup per KV head; every thread walks a fixed strided share of the
// head's elements, writing d_layer = (1 - alpha) d_out and d_last = alpha d_out and
// summing (x_last - x_layer) d_out, then the workgroup adds the partial sums in a fixed
// tree: d_alpha is deterministic.
#include "k_common.h"
#include "kernels.h"

namespace rr {

namespace {

template <bool BF16>
__device__ __forceinline__ void load8(const void* x, int64_t i, float (&v)[8]) {
  if (BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + i);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void blend_fwd(int64_t n8, int Hkv, int d, const float* __restrict__ alpha,
                                                 const void* __restrict__ x_layer, const void* __restrict__ x_last,
                                                 void* __restrict__ x_out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n8) return;
  const int64_t i = t * 8;
  const int g = (int)((i / d) % Hkv);
  const float a = alpha[g], b = 1.0f - a;
  float x[8], y[8];
  load8<BF16>(x_layer, i, x);
  load8<BF16>(x_last, i, y);
  float z[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = fmaf(a, y[j], b * x[j]);
  if (BF16) {
    uint4 u;
    u.x = pack_bf16x2(z[0], z[1]);
    u.y = pack_bf16x2(z[2], z[3]);
    u.z = pack_bf16x2(z[4], z[5]);
    u.w = pack_bf16x2(z[6], z[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(x_out) + i) = u;
  } else {
    float* o = static_cast<float*>(x_out) + i;
    *reinterpret_cast<float4*>(o) = make_float4(z[0], z[1], z[2], z[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(z[4], z[5], z[6], z[7]);
  }
}

constexpr int kBlendBwdThreads = 1024;

template <bool BF16>
__global__ __launch_bounds__(kBlendBwdThreads) void blend_bwd(int64_t rows, int Hkv, int d,
                                                              const float* __restrict__ alpha,
                                                              const void* __restrict__ x_layer,
                                                              const void* __restrict__ x_last,
                                                              const float* __restrict__ d_out,
                                                              float* __restrict__ d_layer,
                                                              float* __restrict__ d_last,
                                                              float* __restrict__ d_alpha, int accumulate) {
  __shared__ float part[kBlendBwdThreads / 64];
  const int g = blockIdx.x;
  const float a = alpha[g], b = 1.0f - a;
  const int per_row = d / 8;   // 8-element groups per (row, head)
  const int64_t n = rows * per_row;
  float acc = 0.0f;
  for (int64_t t = threadIdx.x; t < n; t += kBlendBwdThreads) {
    const int64_t r = t / per_row;
    const int64_t i = (r * Hkv + g) * d + (t % per_row) * 8;
    float x[8], y[8];
    load8<BF16>(x_layer, i, x);
    load8<BF16>(x_last, i, y);
    const float4 g0 = *reinterpret_cast<const float4*>(d_out + i);
    const float4 g1 = *reinterpret_cast<const float4*>(d_out + i + 4);
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(y[j] - x[j], gv[j], acc);
    if (d_layer) {
      float4 u0 = make_float4(b * gv[0], b * gv[1], b * gv[2], b * gv[3]);
      float4 u1 = make_float4(b * gv[4], b * gv[5], b * gv[6], b * gv[7]);
      if (accumulate) {
        const float4 p0 = *reinterpret_cast<const float4*>(d_layer + i);
        const float4 p1 = *reinterpret_cast<const float4*>(d_layer + i + 4);
        u0.x += p0.x; u0.y += p0.y; u0.z += p0.z; u0.w += p0.w;
        u1.x += p1.x; u1.y += p1.y; u1.z += p1.z; u1.w += p1.w;
      }
      *reinterpret_cast<float4*>(d_layer + i) = u0;
      *reinterpret_cast<float4*>(d_layer + i + 4) = u1;
    }
    if (d_last) {
      float4 u0 = make_float4(a * gv[0], a * gv[1], a * gv[2], a * gv[3]);
      float4 u1 = make_float4(a * gv[4], a * gv[5], a * gv[6], a * gv[7]);
      if (accumulate) {
        const float4 p0 = *reinterpret_cast<const float4*>(d_last + i);
        const float4 p1 = *reinterpret_cast<const float4*>(d_last + i + 4);
        u0.x += p0.x; u0.y += p0.y; u0.z += p0.z; u0.w += p0.w;
        u1.x += p1.x; u1.y += p1.y; u1.z += p1.z; u1.w += p1.w;
      }
      *reinterpret_cast<float4*>(d_last + i) = u0;
      *reinterpret_cast<float4*>(d_last + i + 4) = u1;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.0f;
    for (int w = 0; w < kBlendBwdThreads / 64; ++w) s += part[w];
    d_alpha[g] = accumulate ? d_alpha[g] + s : s;
  }
}

}  // namespace

hipError_t launch_lastkv_blend(int64_t rows, int Hkv, int d, int dtype, const float* alpha, const void* x_layer,
                               const void* x_last, void* x_out, hipStream_t s) {
  const int64_t n8 = rows * Hkv * d / 8;
  if (n8 == 0) return hipSuccess;
  const dim3 grid((unsigned)((n8 + 255) / 256)), block(256);
  if (dtype == RR_BF16)
    hipLaunchKernelGGL(blend_fwd<true>, grid, block, 0, s, n8, Hkv, d, alpha, x_layer, x_last, x_out);
  else
    hipLaunchKernelGGL(blend_fwd<false>, grid, block, 0, s, n8, Hkv, d, alpha, x_layer, x_last, x_out);
  return hipGetLastError();
}

hipError_t launch_lastkv_blend_bwd(int64_t rows, int Hkv, int d, int dtype, const float* alpha,
                                   const void* x_layer, const void* x_last, const float* d_out, float* d_layer,
                                   float* d_last, float* d_alpha, int accumulate, hipStream_t s) {
  if (Hkv == 0) return hipSuccess;
  if (dtype == RR_BF16)
    hipLaunchKernelGGL(blend_bwd<true>, dim3(Hkv), dim3(kBlendBwdThreads), 0, s, rows, Hkv, d, alpha, x_layer,
                       x_last, d_out, d_layer, d_last, d_alpha, accumulate);
  else
    hipLaunchKernelGGL(blend_bwd<false>, dim3(Hkv), dim3(kBlendBwdThreads), 0, s, rows, Hkv, d, alpha, x_layer,
                       x_last, d_out, d_layer, d_last, d_alpha, accumulate);
  return hipGetLastError();
}

}  // namespace rr
