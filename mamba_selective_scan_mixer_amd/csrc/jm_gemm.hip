// Projections of the Mamba mixer layer (in_proj, x_proj, dt_proj, out_proj).
//
// All four are Y[m, n] = sum_k X[m, k] * W[n, k] with both operands K-contiguous
// (activations (tokens, K), nn.Linear-style weights (features, K)); they differ
// only in the epilogue. The bf16 path runs on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation); the fp32 path (small fp32
// layers) is a plain LDS-tiled FMA kernel.
//
// bf16 kernel structure:
//   * macro tile BM x BN (tokens x features), K step 64, 256 threads = 4 waves;
//   * operand tiles staged global -> registers -> LDS, double-buffered, with the
//     next tile's global loads issued before the current tile's MFMAs;
//   * LDS rows are 64 bf16 = 8 chunks of 16 bytes; chunk c of row r is stored at
//     chunk position c ^ (r & 7), so the 16-byte fragment reads of 8 consecutive
//     rows hit 8 different bank groups;
//   * the MFMA "A" operand is the weight tile and "B" the activation tile, so each
//     lane ends up owning 4 consecutive output features of one token (8-byte
//     bf16 stores);
//   * workgroup -> tile order: consecutive workgroups walk down M inside a group
//     of GROUP_M row blocks (sharing one weight block), and the 8 XCDs each get a
//     contiguous range of that order (workgroups are dealt round-robin to XCDs).
#include "jm_internal.h"

namespace jm {
namespace {

// ---- epilogue -------------------------------------------------------------------
// v[0..3] are the results for features n..n+3 of token m (n % 4 == 0).
template <typename T>
__device__ __forceinline__ void store4(T* p, const float v[4], int valid) {
  if (valid >= 4) {
    if constexpr (sizeof(T) == 2) {
      bf16 b[4] = {from_f32<bf16>(v[0]), from_f32<bf16>(v[1]), from_f32<bf16>(v[2]),
                   from_f32<bf16>(v[3])};
      *reinterpret_cast<uint2*>(p) = *reinterpret_cast<uint2*>(b);
    } else {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else {
    for (int j = 0; j < valid; ++j) p[j] = from_f32<T>(v[j]);
  }
}

template <typename T>
__device__ __forceinline__ void epilogue(const EpiArgs& e, int64_t m, int n, int N,
                                         float v[4]) {
  int valid = N - n;
  if (valid <= 0) return;
  if (valid > 4) valid = 4;
  switch (e.kind) {
    case EPI_STORE:
      store4<T>(static_cast<T*>(e.out0) + m * e.ldo + n, v, valid);
      break;
    case EPI_SPLIT2:
      if (n < e.split)
        store4<T>(static_cast<T*>(e.out0) + m * e.split + n, v, valid);
      else
        store4<T>(static_cast<T*>(e.out1) + m * e.split + (n - e.split), v, valid);
      break;
    case EPI_XPROJ: {
      if (n < e.split) {
        store4<T>(static_cast<T*>(e.out0) + m * e.split + n, v, valid);
      } else {
        int j = n - e.split;
        if (j < e.n_state)
          store4<float>(e.outf0 + m * e.n_state + j, v, valid);
        else
          store4<float>(e.outf1 + m * e.n_state + (j - e.n_state), v, valid);
      }
      break;
    }
    case EPI_SOFTPLUS: {
      float w[4];
      for (int j = 0; j < 4; ++j) w[j] = j < valid ? softplus(v[j] + e.bias[n + j]) : 0.0f;
      store4<float>(e.outf0 + m * N + n, w, valid);
      break;
    }
    case EPI_F32:
      store4<float>(e.outf0 + m * N + n, v, valid);
      break;
  }
}

// Tile order: GROUP_M row blocks share a weight block; XCD-contiguous ranges.
__device__ __forceinline__ void tile_coords(int bid, int n_wg, int tiles_m, int tiles_n,
                                            int group_m, int& tm, int& tn) {
  // Undo the round-robin XCD dealing: XCD x gets logical ids [x*per, (x+1)*per).
  int logical = bid;
  if ((n_wg & 7) == 0) {
    int per = n_wg >> 3;
    logical = (bid & 7) * per + (bid >> 3);
  }
  int per_group = group_m * tiles_n;
  int g = logical / per_group;
  int first_m = g * group_m;
  int gm = tiles_m - first_m;
  if (gm > group_m) gm = group_m;
  int r = logical - g * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

constexpr int BK = 64;

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N)
void gemm_bf16_kernel(const bf16* __restrict__ X, int64_t ldx,
                      const bf16* __restrict__ W, int64_t ldw,
                      int64_t M, int N, int K, int tiles_m, int tiles_n, EpiArgs epi) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int TM = BM / WAVES_M;   // wave tile (tokens)
  constexpr int TN = BN / WAVES_N;   // wave tile (features)
  constexpr int FM = TM / 32;
  constexpr int FN = TN / 32;
  constexpr int XCH = BM * 8 / NT;   // 16-byte chunks per thread per tile
  constexpr int WCH = BN * 8 / NT;
  static_assert(XCH >= 1 && WCH >= 1, "tile too small for the thread count");

  __shared__ __attribute__((aligned(16))) bf16 sX[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16 sW[2][BN * BK];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, 16, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave / WAVES_N) * TM;
  const int wn0 = (wave % WAVES_N) * TN;

  uint4 rx[XCH], rw[WCH];

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      int id = tid + i * NT;
      int r = id >> 3, c = id & 7;
      int64_t row = m0 + r;
      int k = k0 + c * 8;
      rx[i] = (row < M && k < K) ? *reinterpret_cast<const uint4*>(X + row * ldx + k)
                                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      int id = tid + i * NT;
      int r = id >> 3, c = id & 7;
      int row = n0 + r;
      int k = k0 + c * 8;
      rw[i] = (row < N && k < K) ? *reinterpret_cast<const uint4*>(W + (int64_t)row * ldw + k)
                                 : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      int id = tid + i * NT;
      int r = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(&sX[buf][r * BK + ((c ^ (r & 7)) << 3)]) = rx[i];
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      int id = tid + i * NT;
      int r = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(&sW[buf][r * BK + ((c ^ (r & 7)) << 3)]) = rw[i];
    }
  };

  f32x16 acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();

  const int lrow = lane & 31;
  const int khalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int c = 2 * s + khalf;
      bf16x8 pw[FN], px[FM];
#pragma unroll
      for (int a = 0; a < FN; ++a) {
        int r = wn0 + a * 32 + lrow;
        pw[a] = *reinterpret_cast<const bf16x8*>(&sW[buf][r * BK + ((c ^ (r & 7)) << 3)]);
      }
#pragma unroll
      for (int b = 0; b < FM; ++b) {
        int r = wm0 + b * 32 + lrow;
        px[b] = *reinterpret_cast<const bf16x8*>(&sX[buf][r * BK + ((c ^ (r & 7)) << 3)]);
      }
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pw[a], px[b], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // Lane owns features n = base + 8q + 4*(lane/32) + 0..3 of token m = base + lane%32.
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b) {
      int64_t m = m0 + wm0 + b * 32 + lrow;
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int n = n0 + wn0 + a * 32 + 8 * q + 4 * khalf;
        float v[4] = {acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2],
                      acc[a][b][4 * q + 3]};
        epilogue<bf16>(epi, m, n, N, v);
      }
    }
}

// ---- fp32 path ----------------------------------------------------------------------
// 64x64 tile, 256 threads, each thread 4 tokens x 4 consecutive features.
template <int BM, int BN, int BKF>
__global__ __launch_bounds__(256)
void gemm_f32_kernel(const float* __restrict__ X, int64_t ldx,
                     const float* __restrict__ W, int64_t ldw,
                     int64_t M, int N, int K, EpiArgs epi) {
  __shared__ float sX[BKF][BM + 4];
  __shared__ float sW[BKF][BN + 4];
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int tid = threadIdx.x;
  const int tx = tid % (BN / 4);   // feature group
  const int ty = tid / (BN / 4);   // token group
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BKF) {
    for (int i = tid; i < BM * BKF; i += 256) {
      int r = i / BKF, k = i % BKF;
      int64_t row = m0 + r;
      sX[k][r] = (row < M && k0 + k < K) ? X[row * ldx + k0 + k] : 0.0f;
    }
    for (int i = tid; i < BN * BKF; i += 256) {
      int r = i / BKF, k = i % BKF;
      int row = n0 + r;
      sW[k][r] = (row < N && k0 + k < K) ? W[(int64_t)row * ldw + k0 + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < BKF; ++k) {
      float xv[4], wv[4];
      for (int i = 0; i < 4; ++i) xv[i] = sX[k][ty * 4 + i];
      for (int j = 0; j < 4; ++j) wv[j] = sW[k][tx * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    int64_t m = m0 + ty * 4 + i;
    if (m < M) epilogue<float>(epi, m, n0 + tx * 4, N, acc[i]);
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const bf16* X, int64_t ldx, const bf16* W, int64_t ldw,
                            int64_t M, int N, int K, const EpiArgs& epi, hipStream_t s) {
  constexpr int BM = 128, BN = 128;
  if (M <= 0 || N <= 0) return hipSuccess;
  int64_t tiles_m = (M + BM - 1) / BM;
  int tiles_n = (N + BN - 1) / BN;
  int64_t n_wg = tiles_m * tiles_n;
  if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 2, 2>), dim3((unsigned)n_wg), dim3(256), 0, s,
                     X, ldx, W, ldw, M, N, K, (int)tiles_m, tiles_n, epi);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const float* X, int64_t ldx, const float* W, int64_t ldw,
                           int64_t M, int N, int K, const EpiArgs& epi, hipStream_t s) {
  constexpr int BM = 64, BN = 64, BKF = 16;
  if (M <= 0 || N <= 0) return hipSuccess;
  int64_t gy = (M + BM - 1) / BM;
  if (gy > 65535 * 16) return hipErrorInvalidValue;
  dim3 grid((N + BN - 1) / BN, (unsigned)gy);
  hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, BKF>), grid, dim3(256), 0, s, X, ldx, W, ldw, M, N,
                     K, epi);
  return hipGetLastError();
}

}  // namespace jm
