// Inner RMSNorm of the Mamba layer (optional): delta, B and C, each normalised over its
// own feature axis right after x_proj, v <- v / sqrt(mean(v^2) + eps) * gain (the Jamba
// paper, §2 on the Mamba layer's implementation and §6.4 / Fig. 9, applies RMSNorm to the
// layer's internal activations without placing it; this library places it here).
//
// Delta rows (R values of the activation dtype, R a multiple of 8) are read as 16-byte
// vectors: a row takes P lanes (R / vector length, rounded up to a power of two, at most 64),
// so one wave holds 64 / P rows at once; each lane keeps its vector in registers, so the row
// is read once and written once. Rows longer than 64 vectors loop, and re-read their tail for
// the write. B and C (16 fp32 values per token each) of the wave's rows follow as float4s,
// four lanes per row. Sums of squares are fp32 and reduced with lane shuffles; the root and
// division are IEEE. All pointers are 16-byte aligned (the entry points check tensors and
// gains). HBM-bound and small: (2 * R * sizeof(act) + 4 * 16 * 4) bytes per token.
#include "jm_internal.h"

namespace jm {
namespace {

constexpr int NS = 16;

template <typename T> struct Vec16;
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int n = 4; };
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int n = 8; };

template <typename T>
__global__ __launch_bounds__(256)
void inner_rmsnorm_kernel(T* __restrict__ delta, float* __restrict__ Bm, float* __restrict__ Cm,
                          const float* __restrict__ g_delta, const float* __restrict__ g_B,
                          const float* __restrict__ g_C, float eps, int64_t M, int R, int plog) {
  typedef typename Vec16<T>::type VT;
  constexpr int V = Vec16<T>::n;
  const int lane = threadIdx.x & 63;
  const int P = 1 << plog;
  const int rpw = 64 >> plog;                       // rows per wave
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * rpw;
  if (row0 >= M) return;                            // wave-uniform
  const int nv = R / V;                             // vectors per row
  const int64_t row = row0 + (lane >> plog);
  const int c0 = lane & (P - 1);
  const bool mine = row < M && c0 < nv;
  VT* dr = reinterpret_cast<VT*>(delta + row * R);

  // delta: sum of squares over the row's P lanes
  VT v0 = {};
  if (mine) v0 = dr[c0];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < V; ++i) ss = fmaf(to_f32(v0[i]), to_f32(v0[i]), ss);
  if (row < M)
    for (int c = c0 + 64; c < nv; c += 64) {        // only when P = 64 and nv > 64
      const VT v = dr[c];
#pragma unroll
      for (int i = 0; i < V; ++i) ss = fmaf(to_f32(v[i]), to_f32(v[i]), ss);
    }
  for (int o = P >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float sd = 1.0f / sqrtf(ss / (float)R + eps);
  auto scale = [&](const VT& v, int c) {
    const f32x4* g = reinterpret_cast<const f32x4*>(g_delta + c * V);
    VT o;
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
      const f32x4 gg = g[h];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[4 * h + i] = from_f32<T>(to_f32(v[4 * h + i]) * sd * gg[i]);
    }
    dr[c] = o;
  };
  if (mine) scale(v0, c0);
  if (row < M)
    for (int c = c0 + 64; c < nv; c += 64) scale(dr[c], c);

  // B and C of the wave's rows: task t covers float4 (t & 3) of B (bit 2 clear) or C (set)
  // of row row0 + t / 8; the groups of 4 lanes of one row reduce together.
  for (int t = lane; t < 8 * rpw; t += 64) {
    const int64_t r = row0 + (t >> 3);
    const bool isC = (t >> 2) & 1;
    const int q = t & 3;
    f32x4* p = reinterpret_cast<f32x4*>((isC ? Cm : Bm) + r * NS) + q;
    f32x4 b = {};
    if (r < M) b = *p;
    float s2 = b[0] * b[0] + b[1] * b[1] + b[2] * b[2] + b[3] * b[3];
    s2 += __shfl_xor(s2, 2);
    s2 += __shfl_xor(s2, 1);
    const float den = sqrtf(s2 / (float)NS + eps);
    const f32x4 g = reinterpret_cast<const f32x4*>(isC ? g_C : g_B)[q];
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = b[i] / den * g[i];
    if (r < M) *p = o;
  }
}

}  // namespace

template <typename T>
hipError_t launch_inner_rmsnorm(T* delta, float* Bm, float* Cm, const float* g_delta,
                                const float* g_B, const float* g_C, float eps, int64_t M, int R,
                                hipStream_t s) {
  if (M <= 0) return hipSuccess;
  constexpr int V = Vec16<T>::n;
  if (R <= 0 || R % V) return hipErrorInvalidValue;
  int plog = 0;
  while ((1 << plog) < R / V && plog < 6) ++plog;
  const int64_t rows_per_block = 4 * (64 >> plog);
  const int64_t blocks = (M + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(inner_rmsnorm_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, s, delta, Bm,
                     Cm, g_delta, g_B, g_C, eps, M, R, plog);
  return hipGetLastError();
}

template hipError_t launch_inner_rmsnorm<float>(float*, float*, float*, const float*,
                                                const float*, const float*, float, int64_t, int,
                                                hipStream_t);
template hipError_t launch_inner_rmsnorm<bf16>(bf16*, float*, float*, const float*, const float*,
                                               const float*, float, int64_t, int, hipStream_t);

}  // namespace jm
