// Projections of the Mamba mixer layer (in_proj, x_proj, dt_proj, out_proj).
//
// All four are Y[m, n] = sum_k X[m, k] * W[n, k] with both operands K-contiguous
// (activations (tokens, K), nn.Linear-style weights (features, K)); they differ
// only in the epilogue, which is a compile-time parameter (one kernel symbol per
// projection). The bf16 path runs on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation); the fp32 path runs on the fp32
// matrix cores (v_mfma_f32_32x32x2f32, 64 x 64 tiles).
//
// Main bf16 kernel (K % 64 == 0):
//   * 256 x 256 macro tile, 256 threads = 4 waves (one per SIMD), wave tile 128 x 128:
//     16 accumulator blocks of 32 x 32 in AGPRs, a third less LDS fragment traffic per
//     MFMA than 8 waves of 64 x 128 (the board runs at its power limit under these
//     kernels, and the lower traffic buys clock);
//   * operands go global -> LDS directly (buffer_load_dwordx4 ... lds, no VGPR
//     staging) in 64-deep K slices (128-byte row segments) through two 64 KB
//     buffers, and the waits are explicit vmcnt counts;
//   * LDS rows are 64 bf16 = 8 chunks of 16 bytes; chunk c of row r sits at
//     c ^ ((r & 7) ^ ((r >> 3) & 1)), which keeps the 16-byte fragment reads of 16
//     consecutive rows on distinct banks (measured: no conflicts);
//   * with one wave per SIMD every stall of the wave idles its matrix core, so each k16
//     step is issued in a fixed order (sched_barrier fences around each MFMA): MFMA q,
//     then fragment read q of the next step, and after every second MFMA one of the 16
//     DMA instructions of a later slice, spread so the address unit never backs up into
//     the wave's instruction stream; the barrier of each slice opens its last k16 step
//     (measured against the middle of it and a quarter in: 0.4-0.6% faster);
//   * the MFMA "A" operand is the weight tile and "B" the activation tile, so a
//     lane owns 4 consecutive output features of one token; tiles inside one output
//     leave through a per-wave LDS area as whole 128-byte lines;
//   * tile order: groups of 4 row blocks share a weight block, and each of the 8
//     XCDs (workgroups are dealt to them round-robin) gets a contiguous range;
//   * persistent: one workgroup per CU walks its tiles, issuing the next tile's first
//     loads before storing the current tile's results.
// x_proj with 288 outputs has its own 256 x 288 kernel (16x16x32 MFMA blocks), and
// dt_proj + softplus its own store-bound kernel.
// Fallback (K % 64 != 0): 128 x 128 tiles staged through registers with zero-
// filled K tails.
#include "jm_internal.h"

#include <atomic>

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

template <typename T, int KIND>
__device__ __forceinline__ void epilogue(const EpiArgs& e, int64_t m, int n, int N,
                                         float v[4]) {
  int valid = N - n;
  if (valid <= 0) return;
  if (valid > 4) valid = 4;
  switch (KIND) {
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

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N)
void gemm_bf16_regstage_kernel(const bf16* __restrict__ X, int64_t ldx,
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
        epilogue<bf16, EPI>(epi, m, n, N, v);
      }
    }
}

// ---- main bf16 kernel: multi-stage direct-to-LDS ring ----------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// Fourth word of a raw buffer descriptor on gfx9-family GPUs (32-bit data format; no swizzle,
// no index stride).
constexpr int kBufferRsrcWord3 = 0x00020000;

// Chunk position of 16-byte chunk 0 of row r in a 64-column (128-byte) LDS row: the 16 lanes
// an LDS read serves together (rows r0..r0+15, one chunk column) then hit 16 distinct 16-byte
// bank groups (even rows take chunk positions 0..7 in the first 64 bytes of the bank window,
// odd rows in the second).
__device__ __forceinline__ int swz64(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int CNT>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CNT) : "memory");
}

// 256 x 256 tiles, 4 waves, K slices of 64 (128-byte row segments: one L2 request per row per
// slice, half the requests of 64-byte segments), two LDS buffers of 64 KB, and 4 KB per wave
// behind them where the epilogue turns result rows into whole 128-byte lines.
constexpr int MS_BM = 256, MS_BN = 256, MS_WM = 2, MS_WN = 2, MS_BK = 64;
constexpr int MS_DMA_SPACING = 2;   // MFMAs between two DMA instructions of a wave
constexpr int MS_BARRIER_AT = 0;    // MFMAs of a slice's last k16 step before its barrier
constexpr int MS_EPI_WAVE_BYTES = 32 * 128;   // 32 token rows x 64 bf16 features
constexpr int MS_LDS_BYTES =
    2 * (MS_BM + MS_BN) * MS_BK * 2 + MS_WM * MS_WN * MS_EPI_WAVE_BYTES;

template <int BM, int BN, int WAVES_M, int WAVES_N, int BKC, int EPI>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N)
__attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const bf16* __restrict__ X, int64_t ldx, const bf16* __restrict__ W,
                      int64_t ldw, int64_t M, int N, int K, int tiles_m, int tiles_n,
                      EpiArgs epi) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int CPR = BKC / 8;               // 16-byte chunks per LDS row
  constexpr int RPI = 64 / CPR;              // rows written by one 1 KB DMA instruction
  constexpr int XI = BM / RPI / NW;          // DMA instructions per wave per stage (X)
  constexpr int WI = BN / RPI / NW;          // (W)
  constexpr int SPS = BKC / 16;              // k16 steps per stage
  constexpr int STAGE = (BM + BN) * BKC;     // bf16 elements per stage
  constexpr int NM = FN * FM;                // MFMAs per k16 step
  constexpr int NR = FN + FM;                // fragment reads per k16 step
  static_assert(BKC == 64 && SPS == 4 && XI == 8 && WI == 8 && NM == 16 && NR == 8,
                "the issue order below is laid out for 4 waves of 128 x 128");
  static_assert(FN % 2 == 0, "the staged epilogue writes 64-feature row segments");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  bf16* lds = reinterpret_cast<bf16*>(smem);

  const int n_tiles = tiles_m * tiles_n;
  const int lane = threadIdx.x & 63;
  // The wave index in scalar registers: each DMA's LDS address (M0) is then scalar
  // arithmetic; as a vector value every DMA needed a readfirstlane -> M0 chain that stalled
  // the single wave of its SIMD (in_proj 14.7 -> 13.7 ms at 128K tokens).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm0 = (wave / WAVES_N) * TM;
  const int wn0 = (wave % WAVES_N) * TN;
  // this wave's epilogue staging area, behind the two stage buffers
  char* const stg = smem + 2 * STAGE * 2 + wave * MS_EPI_WAVE_BYTES;

  // Persistent: workgroup b takes tiles b, b + G, b + 2G, ... (G = gridDim.x, a multiple of
  // 8, so a workgroup stays on one XCD and the tile order per XCD is the one tile_coords
  // gives). The next tile's first loads are issued before this tile's results are stored, so
  // their latency hides behind the epilogue.
  int64_t m0;
  int n0;
  // Each DMA instruction fills 1 KB of LDS: lane l writes slot l, i.e. row l / CPR,
  // chunk position l % CPR, so it loads the global chunk that belongs there.
  // Rows past M / N are clamped to the last row (their results are never stored).
  // The loads are buffer loads: one descriptor per operand whose base is the tile's first
  // row, a fixed 32-bit byte offset per lane and instruction, and the k advance in the
  // scalar offset (the host checks that 256 rows + K fit 2^31 bytes).
  uint32_t xoff[XI], woff[WI];
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t xr, wr;
#endif
  auto setup = [&](int tile) {
    int tm, tn;
    tile_coords(tile, n_tiles, tiles_m, tiles_n, 4, tm, tn);
    m0 = (int64_t)tm * BM;
    n0 = tn * BN;
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int row = (wave * XI + i) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swz64(row);
      int64_t r = row;
      if (m0 + r >= M) r = M - 1 - m0;
      xoff[i] = (uint32_t)((r * ldx + c * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      const int row = (wave * WI + i) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swz64(row);
      int64_t r = row;
      if (n0 + r >= N) r = N - 1 - n0;
      woff[i] = (uint32_t)((r * ldw + c * 8) * 2);
    }
#if defined(__HIP_DEVICE_COMPILE__)
    xr = __builtin_amdgcn_make_buffer_rsrc((void*)(X + m0 * ldx), (short)0, 0x7fffffff,
                                           kBufferRsrcWord3);
    wr = __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)n0 * ldw), (short)0, 0x7fffffff,
                                           kBufferRsrcWord3);
#endif
  };
  // the X half and the W half of a stage's DMA, issued at different points of the loop
  auto issue_x = [&](int kt, int buf) {
#if defined(__HIP_DEVICE_COMPILE__)
    char* base = reinterpret_cast<char*>(lds + buf * STAGE);
#pragma unroll
    for (int i = 0; i < XI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(base + (wave * XI + i) * 1024), 16,
                                               xoff[i], kt * BKC * 2, 0, 0);
#endif
  };
  auto issue_w = [&](int kt, int buf) {
#if defined(__HIP_DEVICE_COMPILE__)
    char* base = reinterpret_cast<char*>(lds + buf * STAGE) + BM * BKC * 2;
#pragma unroll
    for (int i = 0; i < WI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)(base + (wave * WI + i) * 1024), 16,
                                               woff[i], kt * BKC * 2, 0, 0);
#endif
  };
  const int lrow = lane & 31;
  const int khalf = lane >> 5;
  const int sw = swz64(lrow);   // equal for all fragment rows of a lane (they differ by 32s)
  int offW[FN], offX[FM];
#pragma unroll
  for (int a = 0; a < FN; ++a) offW[a] = BM * BKC + (wn0 + a * 32 + lrow) * BKC;
#pragma unroll
  for (int b = 0; b < FM; ++b) offX[b] = (wm0 + b * 32 + lrow) * BKC;
  auto load_frags = [&](int buf, int s, bf16x8* pw, bf16x8* px) {
    const int c = ((2 * s + khalf) ^ sw) << 3;
    const bf16* st = lds + buf * STAGE;
#pragma unroll
    for (int a = 0; a < FN; ++a) pw[a] = *reinterpret_cast<const bf16x8*>(&st[offW[a] + c]);
#pragma unroll
    for (int b = 0; b < FM; ++b) px[b] = *reinterpret_cast<const bf16x8*>(&st[offX[b] + c]);
  };

  f32x16 acc[FN][FM];
  bf16x8 fw[2][FN], fx[2][FM];
  auto mfma_range = [&](int cur, int lo, int hi) {
#pragma unroll
    for (int i = lo; i < hi; ++i) {
      const int a = i / FM, b = i % FM;
      acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[cur][a], fx[cur][b], acc[a][b], 0, 0, 0);
    }
  };

  // Single-instruction pieces of the issue order. DMA j of a stage (j < XI: X rows, else W
  // rows) fills 1 KB; fragment idx of a step (idx < FN: W, else X) is one 16-byte read.
  auto dma1 = [&](int kt, int buf, int j) {
#if defined(__HIP_DEVICE_COMPILE__)
    char* base = reinterpret_cast<char*>(lds + buf * STAGE);
    if (j < XI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(base + (wave * XI + j) * 1024), 16,
                                               xoff[j], kt * BKC * 2, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (lds_void*)(base + BM * BKC * 2 + (wave * WI + (j - XI)) * 1024), 16, woff[j - XI],
          kt * BKC * 2, 0, 0);
#endif
  };
  auto frag1 = [&](int buf, int s, int idx, int set) {
    const int c = ((2 * s + khalf) ^ sw) << 3;
    const bf16* st = lds + buf * STAGE;
    if (idx < FN) fw[set][idx] = *reinterpret_cast<const bf16x8*>(&st[offW[idx] + c]);
    else fx[set][idx - FN] = *reinterpret_cast<const bf16x8*>(&st[offX[idx - FN] + c]);
  };
  auto mf1 = [&](int cur, int i) {
    const int a = i / FM, b = i % FM;
    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[cur][a], fx[cur][b], acc[a][b], 0, 0, 0);
  };
  // a step's fragment reads in the order its MFMAs first use them: W0, X0..X3, W1..W3
  constexpr int kReadOrder[8] = {0, 4, 5, 6, 7, 1, 2, 3};
  constexpr int DSP = MS_DMA_SPACING;
  constexpr int BAR = MS_BARRIER_AT;
  static_assert(NM - BAR >= NR, "the next stage's first fragment reads follow the barrier");
  // DMA j of stage kt+2 goes out at MFMA position DSP * j counted from the barrier in stage
  // kt's last step; the first J0 of them fall in the rest of that step, the others into the
  // first steps of stage kt+1.
  constexpr int J0 = (NM - BAR + DSP - 1) / DSP;

  // Two buffers: stage kt lives in buffer kt & 1. The barrier in stage kt's last k16 step
  // (every fragment of stage kt is in registers by then) frees its buffer for stage kt+2,
  // whose 2 XI DMA instructions are spread over the following MFMAs as above; all are waited
  // for (vmcnt 0) before the barrier in stage kt+1's last step.
  const int nk = K / BKC;
  // store instructions this wave issues for a whole tile: the staged epilogue (1 KB of whole
  // lines each) and the per-element one (one per 4 results)
  constexpr int NST_LINES = FM * (FN / 2) * 4;
  constexpr int NST = FN * FM * 4;
  int tile = blockIdx.x;
  setup(tile);
  issue_x(0, 0);
  issue_w(0, 0);
  if (nk > 1) {
#pragma unroll
    for (int j = 0; j < J0; ++j) dma1(1, 1, j);
  }
  int stores_pending = 0;   // store instructions of the previous tile issued after these loads
  for (;;) {
    if (nk > 1) {
      // stage 0 complete; stage 1's first J0 DMAs (and the previous tile's stores) may be in
      // flight (vmcnt counts to 63: beyond that the wait takes some of the stores too)
      if (stores_pending == NST) wait_vmcnt<(J0 + NST > 63 ? 63 : J0 + NST)>();
      else if (stores_pending == NST_LINES) wait_vmcnt<J0 + NST_LINES>();
      else wait_vmcnt<J0>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int b = 0; b < FM; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
    load_frags(0, 0, fw[0], fx[0]);
    int kt = 0;
    // Steady state (stages kt+1 and kt+2 exist): no conditionals, so the compiler counts
    // outstanding LDS reads exactly.
    for (; kt + 2 < nk; ++kt) {
      const int rb = kt & 1;
#pragma unroll
      for (int s = 0; s < SPS; ++s) {
        const int cur = s & 1;
        __builtin_amdgcn_sched_barrier(0);
        if (s + 1 < SPS) {
          // MFMA q, the next step's fragment read q, and stage kt+1's remaining DMAs
#pragma unroll
          for (int q = 0; q < NM; ++q) {
            __builtin_amdgcn_sched_barrier(0);
            mf1(cur, q);
            if (q < NR) frag1(rb, s + 1, kReadOrder[q], cur ^ 1);
            const int pos = NM - BAR + NM * s + q;
            if (pos % DSP == 0 && pos / DSP >= J0 && pos / DSP < XI + WI)
              dma1(kt + 1, rb ^ 1, pos / DSP);
          }
        } else {
          // BAR MFMAs, the stage barrier, then the rest with the next stage's first fragments
          // and stage kt+2's first DMAs. The wait before the barrier also covers this wave's
          // fragment reads from the buffer those DMAs refill, so no wave's read can race
          // another wave's DMA write.
#pragma unroll
          for (int q = 0; q < BAR; ++q) {
            __builtin_amdgcn_sched_barrier(0);
            mf1(cur, q);
          }
          __builtin_amdgcn_sched_barrier(0);
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_s_barrier();
#pragma unroll
          for (int q = BAR; q < NM; ++q) {
            __builtin_amdgcn_sched_barrier(0);
            mf1(cur, q);
            if (q - BAR < NR) frag1(rb ^ 1, 0, kReadOrder[q - BAR], cur ^ 1);
            const int pos = q - BAR;
            if (pos % DSP == 0) dma1(kt + 2, rb, pos / DSP);
          }
        }
      }
    }
    // Last two stages: stage kt+1's DMAs not issued yet go out at once.
    for (; kt < nk; ++kt) {
      const int rb = kt & 1;
#pragma unroll
      for (int s = 0; s < SPS; ++s) {
        const int cur = s & 1;
        if (s == 0 && kt + 1 < nk) {
#pragma unroll
          for (int j = J0; j < XI + WI; ++j) dma1(kt + 1, rb ^ 1, j);
        }
        if (s + 1 < SPS) {
          load_frags(rb, s + 1, fw[cur ^ 1], fx[cur ^ 1]);
        } else if (kt + 1 < nk) {
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_s_barrier();
          load_frags(rb ^ 1, 0, fw[cur ^ 1], fx[cur ^ 1]);
        }
        mfma_range(cur, 0, NM);
      }
    }

    // The tile's LDS is no longer read once every wave is here: the next tile's first
    // loads go out now and land while this tile's results are stored.
    const int64_t em0 = m0;
    const int en0 = n0;
    const int next = tile + (int)gridDim.x;
    if (next < n_tiles) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's fragment reads done
      __builtin_amdgcn_s_barrier();
      setup(next);
      issue_x(0, 0);
      issue_w(0, 0);
      if (nk > 1) {
#pragma unroll
        for (int j = 0; j < J0; ++j) dma1(1, 1, j);
      }
    }
    // Lane owns features n = base + 8q + 4*(lane/32) + 0..3 of token m = base + lane%32.
    // A tile whose 256 features lie inside one output (every tile of STORE; of SPLIT2 when the
    // split is a multiple of 256), with 16-byte aligned rows, gets its base and row stride once
    // per tile and goes out as whole lines: per 32 tokens x 64 features, each wave writes its
    // results into its own 4 KB of LDS (row r, 16-byte chunk c at position c ^ (r & 7), so a
    // write or a read of 8 rows touches every bank once) and reads them back a row segment per
    // 8 lanes, so each store instruction writes 8 whole 128-byte lines. Stored straight from the
    // MFMA layout, each instruction wrote 16 bytes into each of 32 rows, and the L2 write
    // requests (16 per line) took ~10% of in_proj's time.
    bf16* tile_out = nullptr;
    int64_t tile_ld = 0;
    if constexpr (EPI == EPI_STORE) {
      if (en0 + BN <= N && epi.ldo % 8 == 0) {
        tile_out = static_cast<bf16*>(epi.out0) + en0;
        tile_ld = epi.ldo;
      }
    } else if constexpr (EPI == EPI_SPLIT2) {
      if (en0 + BN <= N && epi.split % BN == 0) {
        tile_out = en0 < epi.split ? static_cast<bf16*>(epi.out0) + en0
                                   : static_cast<bf16*>(epi.out1) + (en0 - epi.split);
        tile_ld = epi.split;
      }
    }
    if (tile_out && (reinterpret_cast<uintptr_t>(tile_out) & 15) != 0) tile_out = nullptr;
    // The accumulators leave the AGPRs four at a time, right where they are used, through
    // inline-asm reads: read by plain code, all 256 were copied to VGPRs at once and half of
    // them spilled. The hazard recognizer does not look inside inline asm, so 24 wait states
    // separate the tile's last MFMA from the first read (32x32x16 results need 18).
    __builtin_amdgcn_sched_barrier(0);   // no MFMA is scheduled past the guard
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    auto acc4 = [&](int a, int b, int q, float v[4]) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[u]) : "a"(acc[a][b][4 * q + u]));
    };
    if ((EPI == EPI_STORE || EPI == EPI_SPLIT2) && tile_out) {
#pragma unroll
      for (int b = 0; b < FM; ++b)
#pragma unroll
        for (int ap = 0; ap < FN / 2; ++ap) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float c[4];
              acc4(2 * ap + j, b, q, c);
              const bf16 h[4] = {from_f32<bf16>(c[0]), from_f32<bf16>(c[1]),
                                 from_f32<bf16>(c[2]), from_f32<bf16>(c[3])};
              const int chunk = 4 * j + q;   // features 8 chunk .. 8 chunk + 7 of the 64
              *reinterpret_cast<uint2*>(stg + lrow * 128 + ((chunk ^ (lrow & 7)) << 4) +
                                        khalf * 8) = *reinterpret_cast<const uint2*>(h);
            }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = 8 * i + (lane >> 3), cc = lane & 7;
            const uint4 v =
                *reinterpret_cast<const uint4*>(stg + rr * 128 + ((cc ^ (rr & 7)) << 4));
            const int64_t m = em0 + wm0 + b * 32 + rr;
            if (m < M)
              *reinterpret_cast<uint4*>(tile_out + m * tile_ld + wn0 + ap * 64 + cc * 8) = v;
          }
        }
    } else {
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) {
          const int64_t m = em0 + wm0 + b * 32 + lrow;
          if (m >= M) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = en0 + wn0 + a * 32 + 8 * q + 4 * khalf;
            float v[4];
            acc4(a, b, q, v);
            epilogue<bf16, EPI>(epi, m, n, N, v);
          }
        }
    }
    if (next >= n_tiles) break;
    // A whole tile issued exactly NST_LINES (staged) or at least NST (per element: a wave whose
    // lanes straddle two outputs issues both stores) store instructions, all after the loads
    // above; a partial tile may skip some, so the next wait takes them all.
    stores_pending = em0 + BM <= M && en0 + BN <= N
                         ? ((EPI == EPI_STORE || EPI == EPI_SPLIT2) && tile_out ? NST_LINES : NST)
                         : 0;
    tile = next;
  }
}

// ---- fp32 path ----------------------------------------------------------------------
// fp32 layers on the fp32 matrix cores (v_mfma_f32_32x32x2f32: fp32 products and sums). 64 x 64
// tile, 4 waves, wave w owns the 32 x 32 block of tokens 32 (w >> 1) and features 32 (w & 1);
// as in the bf16 kernel the weight block is the "A" operand, so a lane ends up with 4 consecutive
// features of one token. K goes through LDS in 16-deep slices (rows padded to 20 floats, so the
// 16-byte row reads of 32 lanes spread over the banks); the next slice's global loads are in
// flight while the current one is multiplied. One MFMA takes 2 values of K, one per half-wave;
// each lane reads 4 consecutive K values of its row at once and feeds them to 4 MFMAs, the
// values of a half-wave being K = 4h .. 4h+3 of each group of 8: the weight and token operands
// use the same assignment, so every product W[n, k] X[m, k] is formed exactly once.
constexpr int F32_BM = 64, F32_BN = 64, F32_BK = 16, F32_PITCH = 20;

__device__ __forceinline__ float4 load_row4(const float* __restrict__ base, int64_t ld, int64_t row,
                                            int64_t rows, int k, int K, bool vec_ok) {
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (row >= rows) return v;
  const float* p = base + row * ld + k;
  if (vec_ok && k + 4 <= K) return *reinterpret_cast<const float4*>(p);
  if (k < K) v.x = p[0];
  if (k + 1 < K) v.y = p[1];
  if (k + 2 < K) v.z = p[2];
  if (k + 3 < K) v.w = p[3];
  return v;
}

template <int EPI>
__global__ __launch_bounds__(256)
void gemm_f32_mfma_kernel(const float* __restrict__ X, int64_t ldx,
                          const float* __restrict__ W, int64_t ldw,
                          int64_t M, int N, int K, EpiArgs epi) {
  __shared__ __attribute__((aligned(16))) float sX[F32_BM * F32_PITCH];
  __shared__ __attribute__((aligned(16))) float sW[F32_BN * F32_PITCH];
  const int64_t m0 = (int64_t)blockIdx.y * F32_BM;
  const int n0 = blockIdx.x * F32_BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = 32 * (wave >> 1), wn = 32 * (wave & 1);
  const int half = lane >> 5, r32 = lane & 31;
  // loader: thread t moves 4 consecutive K values of row t / 4 of each operand
  const int lrow = tid >> 2, lcol = (tid & 3) * 4;
  const bool xvec = (ldx & 3) == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0;
  const bool wvec = (ldw & 3) == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0;
  float4 xv = load_row4(X, ldx, m0 + lrow, M, lcol, K, xvec);
  float4 wv = load_row4(W, ldw, n0 + lrow, N, lcol, K, wvec);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += F32_BK) {
    __syncthreads();   // every wave is done reading the previous slice
    *reinterpret_cast<float4*>(&sX[lrow * F32_PITCH + lcol]) = xv;
    *reinterpret_cast<float4*>(&sW[lrow * F32_PITCH + lcol]) = wv;
    __syncthreads();
    if (k0 + F32_BK < K) {
      xv = load_row4(X, ldx, m0 + lrow, M, k0 + F32_BK + lcol, K, xvec);
      wv = load_row4(W, ldw, n0 + lrow, N, k0 + F32_BK + lcol, K, wvec);
    }
#pragma unroll
    for (int g = 0; g < F32_BK / 8; ++g) {
      const float4 a = *reinterpret_cast<const float4*>(&sW[(wn + r32) * F32_PITCH + 8 * g + 4 * half]);
      const float4 b = *reinterpret_cast<const float4*>(&sX[(wm + r32) * F32_PITCH + 8 * g + 4 * half]);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, acc, 0, 0, 0);
    }
  }
  // lane: token m0 + wm + lane % 32; registers 4q .. 4q+3: features n0 + wn + 8q + 4 half + 0..3
  const int64_t m = m0 + wm + r32;
  if (m < M) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4] = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
      epilogue<float, EPI>(epi, m, n0 + wn + 8 * q + 4 * half, N, v);
    }
  }
}

// ---- dt_proj + bias + softplus (bf16 in, fp32 out) -----------------------------------
// Delta[t, d] = softplus(sum_k delta[t, k] * W[d, k] + b[d]) for dt_rank K = 128 or 256.
// The fp32 output (8x the bytes of the input row) makes this a store- and VALU-bound
// kernel, so it is shaped for the stores rather than for the MFMAs:
//   * a workgroup = 16 waves = 512 channels; wave w keeps the weight rows of channels
//     32w..32w+31 in registers for its whole life (MFMA B operand: lane -> channel
//     lane % 32, k half lane / 32). Every workgroup reads every token row once, so wide
//     workgroups cut the L2 traffic of the shared token rows (16 channel groups at
//     d_inner 8192 instead of 64);
//   * it walks 32-token blocks blockIdx.y, += gridDim.y; each block of token rows is
//     copied once into LDS (direct-to-LDS loads, double-buffered, issued a block ahead)
//     and read from there by all four waves as the MFMA A operand. LDS row r holds its
//     16-byte chunk c at c ^ (r % 16), so the fragment reads of 16 rows hit distinct banks;
//   * a lane's results are channel lane % 32 of tokens 8(r/4) + 4(lane/32) + r%4, so each
//     store instruction writes two full 128-byte row segments;
//   * 4 waves per SIMD, whose stores overlap each other's loads and math.
constexpr int DT_NW = 16;
constexpr int DT_CH = 32 * DT_NW;
template <int KS>   // K / 16
__global__ __launch_bounds__(64 * DT_NW)
void dt_proj_softplus_kernel(const bf16* __restrict__ X, int64_t ldx, const bf16* __restrict__ W,
                             int64_t ldw, int64_t M, int N, const float* __restrict__ bias,
                             float* __restrict__ out) {
  constexpr int K = KS * 16;
  constexpr int ROWB = K * 2;                 // bytes per token row
  constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  constexpr int BLKB = 32 * ROWB;             // bytes per 32-token block
  constexpr int NDMA = BLKB / 1024;           // 1 KB DMA instructions per block
  constexpr int DPW = (NDMA + DT_NW - 1) / DT_NW;   // per wave (some idle when NDMA < DT_NW)
  __shared__ __attribute__((aligned(1024))) char sx[2][BLKB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // in scalar registers
  const int kh = lane >> 5;
  const int ch = blockIdx.x * DT_CH + wave * 32 + (lane & 31);
  bf16x8 w[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    w[s] = *reinterpret_cast<const bf16x8*>(W + (int64_t)ch * ldw + 16 * s + 8 * kh);
  const float b = bias[ch];
  // Settle the weight loads here, with a wait the compiler sees (vmcnt(0) = 0x0F70 on gfx9),
  // so it does not re-wait for them inside the loop, where vmcnt also counts the block
  // prefetch and the previous block's stores.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  const int64_t nblk = (M + 31) >> 5;
  // DMA slot of this lane: instruction j of wave w fills LDS bytes [1 KB * s, +1 KB) with
  // s = DT_NW j + w, i.e. rows (1024 / ROWB) s + lane / CPR, physical chunk lane % CPR.
  auto issue = [&](int64_t blk, int buf) {
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int slot = DT_NW * j + wave;
      if (slot >= NDMA) break;
      const int r = slot * (1024 / ROWB) + lane / CPR;
      const int c = (lane % CPR) ^ (r & 15);
      int64_t t = (blk << 5) + r;
      if (t >= M) t = M - 1;            // past the end: a copy of the last row, never stored
      __builtin_amdgcn_global_load_lds((const void*)(X + t * ldx + c * 8),
                                       (lds_void*)(&sx[buf][slot * 1024]), 16, 0, 0);
    }
  };
  int64_t blk = blockIdx.y;
  if (blk < nblk) issue(blk, 0);
  for (int it = 0; blk < nblk; ++it, blk += gridDim.y) {
    const int buf = it & 1;
    // this block's rows have landed (the previous block's 16 stores may still be in flight)
    if (it == 0) wait_vmcnt<0>(); else wait_vmcnt<16>();
    __builtin_amdgcn_s_barrier();     // ... for every wave; and the other buffer is free
    if (blk + gridDim.y < nblk) issue(blk + gridDim.y, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    const int t0r = lane & 31;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int c = (2 * s + kh) ^ (t0r & 15);
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sx[buf][t0r * ROWB + c * 16]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w[s], acc, 0, 0, 0);
    }
    // Delta is written once and first read back by the scan after all of it is written (4 GiB
    // at 128K tokens, far more than the caches): streaming (non-temporal) stores.
    const int64_t t0 = blk << 5;
    float* op = out + (t0 + 4 * kh) * N + ch;
    if (t0 + 32 <= M) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __builtin_nontemporal_store(softplus(acc[r] + b), &op[(int64_t)(8 * (r >> 2) + (r & 3)) * N]);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (t0 + 4 * kh + 8 * (r >> 2) + (r & 3) < M)
          __builtin_nontemporal_store(softplus(acc[r] + b),
                                      &op[(int64_t)(8 * (r >> 2) + (r & 3)) * N]);
    }
  }
}

// ---- x_proj: 256 tokens x 288 outputs (dt_rank 256, then B and C) -------------------------
// 288 output features are 18 blocks of 16. On the 256 x 256 kernel they would take two column
// tiles, the second one 7/8 padding; here one workgroup covers all of them. 8 waves as 4
// (tokens) x 2 (features): wave tile 64 tokens x 144 features in 16x16x32 MFMA blocks (A = a
// weight block, so a lane's 4 D registers are 4 consecutive features of one token, the shape
// the epilogue takes). K is staged in 64-deep slices (128-byte rows, swizzled as in the main
// kernel) through two LDS buffers filled by direct-to-LDS buffer loads.
constexpr int XP_BM = 256, XP_N = 288, XP_BK = 64;
constexpr int XP_STAGE = (XP_BM + XP_N) * XP_BK;   // bf16 elements per stage
constexpr int XP_LDS_BYTES = 2 * XP_STAGE * 2;      // 139,264

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void xproj_kernel(const bf16* __restrict__ X, int64_t ldx, const bf16* __restrict__ W,
                  int64_t ldw, int64_t M, int K, EpiArgs epi) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  bf16* lds = reinterpret_cast<bf16*>(smem);
  const int64_t m0 = (int64_t)blockIdx.x * XP_BM;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // in scalar registers
  // DMA instructions (1 KB = 8 rows each): X 32 (4 per wave), W 36 (5 for waves 0-3, 4 after)
  constexpr int XI = 4, WI = 5;
  const int wi = wave < 4 ? 5 : 4;
  const int wfirst = wave < 4 ? 5 * wave : 20 + 4 * (wave - 4);
  uint32_t xoff[XI], woff[WI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int row = (wave * XI + i) * 8 + lane / 8;
    const int c = (lane % 8) ^ swz64(row);
    int64_t r = row;
    if (m0 + r >= M) r = M - 1 - m0;      // past the end: a copy of the last row, never stored
    xoff[i] = (uint32_t)((r * ldx + c * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int row = (wfirst + i) * 8 + lane / 8;   // < 288 for every instruction issued
    const int c = (lane % 8) ^ swz64(row);
    woff[i] = (uint32_t)(((int64_t)row * ldw + c * 8) * 2);
  }
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + m0 * ldx), (short)0, 0x7fffffff, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)W, (short)0, 0x7fffffff, kBufferRsrcWord3);
#endif
  auto issue = [&](int kt, int buf) {
#if defined(__HIP_DEVICE_COMPILE__)
    char* base = reinterpret_cast<char*>(lds + buf * XP_STAGE);
#pragma unroll
    for (int i = 0; i < XI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(base + (wave * XI + i) * 1024), 16,
                                               xoff[i], kt * XP_BK * 2, 0, 0);
    char* wb = base + XP_BM * XP_BK * 2;
#pragma unroll
    for (int i = 0; i < WI; ++i)
      if (i < wi)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)(wb + (wfirst + i) * 1024), 16,
                                                 woff[i], kt * XP_BK * 2, 0, 0);
#endif
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, kg = lane >> 4;
  const int sw = swz64(lr);            // every fragment row of this lane is lr mod 16
  const int offW = XP_BM * XP_BK + (wn * 144 + lr) * XP_BK;
  const int offX = (wm * 64 + lr) * XP_BK;
  f32x4 acc[9][4];
#pragma unroll
  for (int a = 0; a < 9; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = K / XP_BK;
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    // the other buffer was released by the barrier that ended the previous slice
    if (kt + 1 < nk) {
      issue(kt + 1, buf ^ 1);
      if (wave < 4) wait_vmcnt<XI + 5>(); else wait_vmcnt<XI + 4>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();      // this slice has landed for every wave
    const bf16* st = lds + buf * XP_STAGE;
#pragma unroll
    for (int s = 0; s < XP_BK / 32; ++s) {
      const int c = ((4 * s + kg) ^ sw) << 3;
      bf16x8 fw[9], fx[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        fx[b] = *reinterpret_cast<const bf16x8*>(&st[offX + b * 16 * XP_BK + c]);
#pragma unroll
      for (int a = 0; a < 9; ++a)
        fw[a] = *reinterpret_cast<const bf16x8*>(&st[offW + a * 16 * XP_BK + c]);
#pragma unroll
      for (int a = 0; a < 9; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[a], fx[b], acc[a][b], 0, 0, 0);
    }
    // Every wave is done with this buffer: its own reads have returned (the compiler may
    // otherwise leave the last ones in flight and wait for them after the barrier, where
    // another wave may already be refilling the buffer), then the barrier.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  }

  // D block (16 features x 16 tokens): lane holds token lr, features 4 kg .. 4 kg + 3.
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t m = m0 + wm * 64 + b * 16 + lr;
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < 9; ++a) {
      const int n = wn * 144 + a * 16 + 4 * kg;
      float v[4] = {acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]};
      epilogue<bf16, EPI_XPROJ>(epi, m, n, XP_N, v);
    }
  }
}

// Per-device launch set-up, done once per device and thread-safe: each GPU a process uses
// gets its own flag (the LDS attribute is set for the current device) and its own CU count.
constexpr int kMaxDevices = 64;
hipError_t current_device(int& dev) {
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  return dev >= 0 && dev < kMaxDevices ? hipSuccess : hipErrorInvalidDevice;
}
hipError_t allow_big_lds_once(std::atomic<bool> (&done)[kMaxDevices], int dev, const void* fn,
                              int bytes) {
  if (done[dev].load(std::memory_order_acquire)) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done[dev].store(true, std::memory_order_release);
  return e;
}

template <int EPI>
hipError_t launch_bf16_epi(const bf16* X, int64_t ldx, const bf16* W, int64_t ldw, int64_t M,
                           int N, int K, const EpiArgs& epi, hipStream_t s) {
  if (EPI == EPI_SOFTPLUS && (K == 256 || K == 128) && N % DT_CH == 0) {
    const int64_t nblk = (M + 31) / 32;
    const dim3 grid(N / DT_CH, (unsigned)(nblk < 32 ? nblk : 32));
    if (K == 256)
      hipLaunchKernelGGL(dt_proj_softplus_kernel<16>, grid, dim3(64 * DT_NW), 0, s, X, ldx, W, ldw, M, N,
                         epi.bias, epi.outf0);
    else
      hipLaunchKernelGGL(dt_proj_softplus_kernel<8>, grid, dim3(64 * DT_NW), 0, s, X, ldx, W, ldw, M, N,
                         epi.bias, epi.outf0);
    return hipGetLastError();
  }
  if (EPI == EPI_XPROJ && N == XP_N && K % XP_BK == 0 &&
      ((int64_t)XP_BM * ldx + K) * 2 < ((int64_t)1 << 31) &&
      ((int64_t)XP_N * ldw + K) * 2 < ((int64_t)1 << 31)) {
    const int64_t n_wg = (M + XP_BM - 1) / XP_BM;
    if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
    // dynamic LDS above 64 KB must be enabled once per device
    static std::atomic<bool> xp_attr_set[kMaxDevices];
    int dev = 0;
    hipError_t e = current_device(dev);
    if (e == hipSuccess)
      e = allow_big_lds_once(xp_attr_set, dev, (const void*)xproj_kernel, XP_LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(xproj_kernel, dim3((unsigned)n_wg), dim3(512), XP_LDS_BYTES, s, X, ldx, W,
                       ldw, M, K, epi);
    return hipGetLastError();
  }
  // buffer-load offsets (256 rows + K, in bytes) must fit 31 bits
  const bool offsets_fit = ((int64_t)MS_BM * ldx + K) * 2 < ((int64_t)1 << 31) &&
                           ((int64_t)MS_BN * ldw + K) * 2 < ((int64_t)1 << 31);
  if (K % MS_BK == 0 && offsets_fit) {
    const int64_t tiles_m = (M + MS_BM - 1) / MS_BM;
    const int tiles_n = (N + MS_BN - 1) / MS_BN;
    const int64_t n_wg = tiles_m * tiles_n;
    if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
    auto kern = gemm_bf16_kernel<MS_BM, MS_BN, MS_WM, MS_WN, MS_BK, EPI>;
    static std::atomic<bool> attr_set[kMaxDevices];   // per device, as for x_proj
    int dev = 0;
    hipError_t e = current_device(dev);
    if (e == hipSuccess) e = allow_big_lds_once(attr_set, dev, (const void*)kern, MS_LDS_BYTES);
    if (e != hipSuccess) return e;
    // One persistent workgroup per CU (128 KB of LDS each; a multiple of 8 for the XCD
    // dealing): each tile's first loads are issued before the previous tile's stores, so their
    // latency hides behind the epilogue (in_proj at 128K tokens: 128 tiles per CU, 2-3% faster
    // than one workgroup per tile; out_proj, 32 tiles per CU, unchanged).
    static std::atomic<int> cu_count[kMaxDevices];
    int n_cu = cu_count[dev].load(std::memory_order_relaxed);
    if (n_cu == 0) {
      if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          n_cu < 8)
        n_cu = 8;
      cu_count[dev].store(n_cu, std::memory_order_relaxed);
    }
    int64_t grid = n_cu & ~7;
    if (grid > n_wg) grid = n_wg;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * MS_WM * MS_WN), MS_LDS_BYTES, s, X,
                       ldx, W, ldw, M, N, K, (int)tiles_m, tiles_n, epi);
    return hipGetLastError();
  }
  constexpr int BM = 128, BN = 128;
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int64_t n_wg = tiles_m * tiles_n;
  if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_regstage_kernel<BM, BN, 2, 2, EPI>), dim3((unsigned)n_wg),
                     dim3(256), 0, s, X, ldx, W, ldw, M, N, K, (int)tiles_m, tiles_n, epi);
  return hipGetLastError();
}


template <int EPI>
hipError_t launch_f32_epi(const float* X, int64_t ldx, const float* W, int64_t ldw, int64_t M,
                          int N, int K, const EpiArgs& epi, hipStream_t s) {
  const int64_t gy = (M + F32_BM - 1) / F32_BM;
  if (gy > 65535) return hipErrorInvalidValue;
  dim3 grid((N + F32_BN - 1) / F32_BN, (unsigned)gy);
  hipLaunchKernelGGL((gemm_f32_mfma_kernel<EPI>), grid, dim3(256), 0, s, X, ldx, W, ldw, M, N, K,
                     epi);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const bf16* X, int64_t ldx, const bf16* W, int64_t ldw,
                            int64_t M, int N, int K, const EpiArgs& epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  switch (epi.kind) {
    case EPI_STORE: return launch_bf16_epi<EPI_STORE>(X, ldx, W, ldw, M, N, K, epi, s);
    case EPI_SPLIT2: return launch_bf16_epi<EPI_SPLIT2>(X, ldx, W, ldw, M, N, K, epi, s);
    case EPI_XPROJ: return launch_bf16_epi<EPI_XPROJ>(X, ldx, W, ldw, M, N, K, epi, s);
    case EPI_SOFTPLUS: return launch_bf16_epi<EPI_SOFTPLUS>(X, ldx, W, ldw, M, N, K, epi, s);
    case EPI_F32: return launch_bf16_epi<EPI_F32>(X, ldx, W, ldw, M, N, K, epi, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_f32(const float* X, int64_t ldx, const float* W, int64_t ldw,
                           int64_t M, int N, int K, const EpiArgs& epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  switch (epi.kind) {
    case EPI_STORE: return launch_f32_epi<EPI_STORE>(X, ldx, W, ldw, M, N, K, epi, s);
    case EPI_SPLIT2: return launch_f32_epi<EPI_SPLIT2>(X, ldx, W, ldw, M, N, K, epi, s);
    case EPI_XPROJ: return launch_f32_epi<EPI_XPROJ>(X, ldx, W, ldw, M, N, K, epi, s);
    case EPI_SOFTPLUS: return launch_f32_epi<EPI_SOFTPLUS>(X, ldx, W, ldw, M, N, K, epi, s);
    case EPI_F32: return launch_f32_epi<EPI_F32>(X, ldx, W, ldw, M, N, K, epi, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace jm
