// Inner RMSNorm of the Mamba layer (optional): delta, B and C, each normalised over its
// own feature axis right after x_proj, v <- v / sqrt(mean(v^2) + eps) * gain (the Jamba
// paper, §2 on the Mamba layer's implementation and §6.4 / Fig. 9, applies RMSNorm to the
// layer's internal activations without placing it; this library places it here).
//
// One wave per token row, in place: delta (R values, the activation dtype) is read with
// the 64 lanes striding along the row; B and C (16 fp32 values each) take lanes 0-15 and
// 16-31. Sums of squares are fp32 and reduced with lane shuffles; the root and division
// are IEEE. HBM-bound and small: (2 * R * sizeof(act) + 4 * 16 * 4) bytes per token.
#include "jm_internal.h"

namespace jm {
namespace {

constexpr int NS = 16;

template <typename T>
__global__ __launch_bounds__(256)
void inner_rmsnorm_kernel(T* __restrict__ delta, float* __restrict__ Bm, float* __restrict__ Cm,
                          const float* __restrict__ g_delta, const float* __restrict__ g_B,
                          const float* __restrict__ g_C, float eps, int64_t M, int R) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;                 // wave-uniform
  T* dr = delta + row * R;
  float ss = 0.0f;
  for (int j = lane; j < R; j += 64) {
    const float v = to_f32(dr[j]);
    ss = fmaf(v, v, ss);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float sd = 1.0f / sqrtf(ss / (float)R + eps);
  for (int j = lane; j < R; j += 64) dr[j] = from_f32<T>(to_f32(dr[j]) * sd * g_delta[j]);

  const int q = lane & 15;
  const bool isB = lane < 16;
  float* p = (isB ? Bm : Cm) + row * NS;
  const float* g = isB ? g_B : g_C;
  const float v = lane < 32 ? p[q] : 0.0f;
  float s2 = v * v;                     // sums within each group of 16 lanes
  s2 += __shfl_xor(s2, 8);
  s2 += __shfl_xor(s2, 4);
  s2 += __shfl_xor(s2, 2);
  s2 += __shfl_xor(s2, 1);
  if (lane < 32) p[q] = v / sqrtf(s2 / (float)NS + eps) * g[q];
}

}  // namespace

template <typename T>
hipError_t launch_inner_rmsnorm(T* delta, float* Bm, float* Cm, const float* g_delta,
                                const float* g_B, const float* g_C, float eps, int64_t M, int R,
                                hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int64_t blocks = (M + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(inner_rmsnorm_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, s, delta, Bm,
                     Cm, g_delta, g_B, g_C, eps, M, R);
  return hipGetLastError();
}

template hipError_t launch_inner_rmsnorm<float>(float*, float*, float*, const float*,
                                                const float*, const float*, float, int64_t, int,
                                                hipStream_t);
template hipError_t launch_inner_rmsnorm<bf16>(bf16*, float*, float*, const float*, const float*,
                                               const float*, float, int64_t, int, hipStream_t);

}  // namespace jm
