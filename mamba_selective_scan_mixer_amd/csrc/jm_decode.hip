// Single-token decode of the Mamba mixer layer (bf16 weights/activations, fp32
// state), for up to 64 sequences per launch.
//
// At one token per sequence every projection is a skinny (M <= 64) product whose
// cost is streaming the weights (210 MB per step at the Jamba-7B-class sizes), so
// the kernels here are built for bandwidth:
//   dec_gemm_lds  64 output features x 64 tokens per workgroup, optional split-K over a
//                 second grid dimension (fp32 partials). Weight and token rows reach LDS
//                 through direct-to-LDS loads of whole 128-byte row segments (or contiguous
//                 runs from 64 x 64-tiled weights), 3 stages of 64 K columns in flight
//                 (7 for x_proj); each wave owns a 32 x 32 output tile.
//   in_proj epilogue: the conv-state shift, the causal conv (kernel 4) and SiLU are
//                 applied right there for the x half; the z half is stored.
//   out_proj epilogue: the workgroup that completes a 64-feature block last adds the four
//                 split-K partial sums in split order and writes the bf16 output.
//   xproj_reduce: x_proj's split-K partial sums, added in a fixed order.
//   update        per 32 channels x 16 sequences: dt_proj on MFMA (W_dt and delta rows
//                 staged in LDS), softplus, the 16-state update in place, the D skip and
//                 the SiLU(z) gate.
#include "jm_internal.h"

#include <atomic>

namespace jm {
namespace {

constexpr int NS = 16;

enum DecEpi : int { DEC_STORE = 0, DEC_INPROJ_CONV = 1, DEC_PARTIAL = 2, DEC_PARTIAL_SUM = 3 };

constexpr int OUTPROJ_SPLITS = 4;   // out_proj split-K (256 workgroups at d_model 4096)

struct DecEpiArgs {
  bf16* out;             // STORE: (M, N) bf16
  bf16* xh;              // INPROJ: (M, d_inner) conv+SiLU output
  bf16* z;               // INPROJ: (M, d_inner)
  bf16* conv_state;      // INPROJ: (rows, d_inner, 3) in/out
  const int32_t* rows;   // INPROJ: state row of token row m (NULL: m)
  const bf16* conv_w;    // INPROJ: (d_inner, 4)
  const bf16* conv_b;    // INPROJ: (d_inner) or null
  int d_inner;           // INPROJ split point
  float* partial;        // PARTIAL: (splits, M, N) fp32; PARTIAL_SUM: per split, block, thread
  int* counters;         // INPROJ: zeroed (n_counters); PARTIAL_SUM: arrivals per 64-feature block
  int n_counters;
  int w_tiled;           // INPROJ, PARTIAL_SUM: W in 64 x 64 tiles (see tile_weights_kernel)
};

// ---- write-out of one item: token m, features n .. n+7 (n % 8 == 0) ------------------------
// STORE: bf16 outputs; PARTIAL: fp32 split-K partial sums of split `split`.
template <int EPI>
__device__ __forceinline__ void dec_store_item(const DecEpiArgs& e, int m, int n, int N, int M,
                                               int split, const float v[8]) {
  const bool whole = n + 8 <= N;
  if constexpr (EPI == DEC_STORE) {
    if (whole) {
      bf16x8 o;
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] = from_f32<bf16>(v[c]);
      *reinterpret_cast<bf16x8*>(e.out + (int64_t)m * N + n) = o;
    } else {
      for (int c = 0; c < 8 && n + c < N; ++c) e.out[(int64_t)m * N + n + c] = from_f32<bf16>(v[c]);
    }
  } else {
    float* dst = e.partial + ((int64_t)split * M + m) * N + n;
    if (whole) {
      *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      for (int c = 0; c < 8 && n + c < N; ++c) dst[c] = v[c];
    }
  }
}

// in_proj items of the x half (n < d_inner) read the token's conv-state row (48 bytes), the taps
// (64 bytes) and the bias (16 bytes) of their 8 features; z items read nothing.
__device__ __forceinline__ void dec_inproj_load(const DecEpiArgs& e, int m, int n, bf16x8 s3[3],
                                                bf16x8 w4[4], bf16x8& b8) {
  const int di = e.d_inner;
  if (n >= di) return;
  const int64_t row = e.rows ? (int64_t)e.rows[m] : (int64_t)m;
  const bf16x8* st = reinterpret_cast<const bf16x8*>(e.conv_state + (row * di + n) * 3);
  const bf16x8* cw = reinterpret_cast<const bf16x8*>(e.conv_w + (int64_t)n * 4);
#pragma unroll
  for (int k = 0; k < 3; ++k) s3[k] = st[k];
#pragma unroll
  for (int k = 0; k < 4; ++k) w4[k] = cw[k];
  if (e.conv_b) b8 = *reinterpret_cast<const bf16x8*>(e.conv_b + n);
}

// in_proj: features < d_inner are x (conv-state shift, conv, SiLU), the rest z. d_inner % 64 == 0,
// so an item is entirely x or entirely z.
__device__ __forceinline__ void dec_inproj_item(const DecEpiArgs& e, int m, int n, const float v[8],
                                                const bf16x8 s3[3], const bf16x8 w4[4],
                                                const bf16x8 b8) {
  const int di = e.d_inner;
  if (n < di) {
    const int64_t row = e.rows ? (int64_t)e.rows[m] : (int64_t)m;
    bf16x8* st = reinterpret_cast<bf16x8*>(e.conv_state + (row * di + n) * 3);   // 48 bytes
    bf16x8 xo, so[3];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // state of feature n + c: elements 3c .. 3c+2 of the 24 (oldest first);
      // taps of feature n + c: elements 4c .. 4c+3 of the 32
      const float h0 = to_f32(s3[(3 * c) >> 3][(3 * c) & 7]);
      const float h1 = to_f32(s3[(3 * c + 1) >> 3][(3 * c + 1) & 7]);
      const float h2 = to_f32(s3[(3 * c + 2) >> 3][(3 * c + 2) & 7]);
      const bf16 xb = from_f32<bf16>(v[c]);
      float acc = e.conv_b ? to_f32(b8[c]) : 0.0f;
      acc = fmaf(to_f32(w4[c >> 1][4 * (c & 1)]), h0, acc);
      acc = fmaf(to_f32(w4[c >> 1][4 * (c & 1) + 1]), h1, acc);
      acc = fmaf(to_f32(w4[c >> 1][4 * (c & 1) + 2]), h2, acc);
      acc = fmaf(to_f32(w4[c >> 1][4 * (c & 1) + 3]), to_f32(xb), acc);
      xo[c] = from_f32<bf16>(silu(acc));
      so[(3 * c) >> 3][(3 * c) & 7] = s3[(3 * c + 1) >> 3][(3 * c + 1) & 7];
      so[(3 * c + 1) >> 3][(3 * c + 1) & 7] = s3[(3 * c + 2) >> 3][(3 * c + 2) & 7];
      so[(3 * c + 2) >> 3][(3 * c + 2) & 7] = xb;
    }
    *reinterpret_cast<bf16x8*>(e.xh + (int64_t)m * di + n) = xo;
#pragma unroll
    for (int k = 0; k < 3; ++k) st[k] = so[k];
  } else {
    bf16x8 o;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = from_f32<bf16>(v[c]);
    *reinterpret_cast<bf16x8*>(e.z + (int64_t)m * di + (n - di)) = o;
  }
}

// ---- LDS-staged decode GEMM ------------------------------------------------------------------
// Y[m, n] = sum_k U[m, k] W[n, k] for M <= 64 token rows: 64 output features per workgroup, K
// split over grid.y. Both operands reach LDS through direct-to-LDS buffer loads, each
// instruction fetching 8 whole 128-byte row segments: loads straight into the MFMA operand
// layout touch 32 lines per instruction and 32 bytes of each, and counters showed the address
// unit stalled on the L1 for most of such a kernel. Stages of 64 K columns (16 KB: 64 weight
// rows and 64 token rows) rotate through DL_NBUF LDS buffers (4 for the decode projections),
// all but the one being read in flight; each wave issues a quarter of every stage's loads.
// Wave w owns the 32 x 32 output tile of features
// 32 (w & 1) and tokens 32 (w >> 1) over the whole K range, so no partial sums cross waves.
constexpr int DL_BK = 64;                       // K columns per stage
constexpr int DL_TILE = 64 * DL_BK * 2;         // bytes of one operand's stage tile (8 KB)
constexpr int DL_STAGE = 2 * DL_TILE;           // weight tile, then token tile
constexpr int DL_OUT_PITCH = 68;                // floats per token row of the output tile in LDS
constexpr int kBufWord3 = 0x00020000;           // raw buffer descriptor word 3 (32-bit data)
typedef __attribute__((address_space(3))) void lds_void_t;

// Position of 16-byte chunk c of row r inside a 128-byte LDS row: the 16 rows one LDS read
// serves together then fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int dl_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int CNT>
__device__ __forceinline__ void dl_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CNT) : "memory");
}

// out_proj's split-K epilogue. Each workgroup stores its 64 x 64 partial sums (16 per thread, as
// 8-byte halves at [split][block][c][thread], so a wave's store covers 512 contiguous bytes) and
// then counts itself in for its block of 64 features; the workgroup that arrives last reads all
// four partial sets back and writes bf16(0 + p0 + p1 + p2 + p3), the sum of a separate reduction
// launch in the same order. The workgroups of a block may run on different XCDs, whose L2 caches
// are not coherent with each other: the partial sums go through agent-scope atomic stores and loads,
// which reach the device-coherent level, and only the ordering is fenced (every store has
// completed, vmcnt(0), before the count moves; the reads start after the count is seen), so no
// L2 write-back or invalidation is needed.
__device__ __forceinline__ void dec_partial_sum_epilogue(const DecEpiArgs& e, const float* ot,
                                                         const int it_m[2], const int it_n[2],
                                                         int n0, int M, int N, int split,
                                                         int* last_flag) {
  float own[16];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const float4* src = reinterpret_cast<const float4*>(ot + it_m[it] * DL_OUT_PITCH + (it_n[it] - n0));
    const float4 lo = src[0], hi = src[1];
    own[8 * it + 0] = lo.x; own[8 * it + 1] = lo.y; own[8 * it + 2] = lo.z; own[8 * it + 3] = lo.w;
    own[8 * it + 4] = hi.x; own[8 * it + 5] = hi.y; own[8 * it + 6] = hi.z; own[8 * it + 7] = hi.w;
  }
  uint64_t* P = reinterpret_cast<uint64_t*>(e.partial);
  const int64_t blocks = gridDim.x;
  auto slot = [&](int s, int c) {
    return P + ((((int64_t)s * blocks + blockIdx.x) * 8 + c) * 256 + threadIdx.x);
  };
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint64_t w = (uint64_t)__float_as_uint(own[2 * c]) |
                       ((uint64_t)__float_as_uint(own[2 * c + 1]) << 32);
    __hip_atomic_store(slot(split, c), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's partial sums have landed
  __syncthreads();
  if (threadIdx.x == 0)
    *last_flag = __hip_atomic_fetch_add(e.counters + blockIdx.x, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == OUTPROJ_SPLITS - 1;
  __syncthreads();
  if (!*last_flag) return;
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // every split's values, this workgroup's own included (they round-trip bit-exactly)
  uint64_t q[OUTPROJ_SPLITS][8];
#pragma unroll
  for (int s = 0; s < OUTPROJ_SPLITS; ++s)
#pragma unroll
    for (int c = 0; c < 8; ++c)
      q[s][c] = __hip_atomic_load(slot(s, c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float sum[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) sum[j] = 0.0f;
#pragma unroll
  for (int s = 0; s < OUTPROJ_SPLITS; ++s)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      sum[2 * c] += __uint_as_float((uint32_t)q[s][c]);
      sum[2 * c + 1] += __uint_as_float((uint32_t)(q[s][c] >> 32));
    }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int m = it_m[it], n = it_n[it];
    if (m >= M || n >= N) continue;
    bf16x8 o;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = from_f32<bf16>(sum[8 * it + c]);
    *reinterpret_cast<bf16x8*>(e.out + (int64_t)m * N + n) = o;
  }
}

template <int EPI, int DL_NBUF>   // DL_NBUF LDS stage buffers of DL_STAGE bytes
__global__ __launch_bounds__(256)
void dec_gemm_lds_kernel(const bf16* __restrict__ U, const bf16* __restrict__ W, int M, int N,
                         int K, int k_per_split, DecEpiArgs e) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // in scalar registers
  const int n0 = blockIdx.x * 64;
  const int split = blockIdx.y;
  const int kbeg = split * k_per_split;
  const int nst = k_per_split / DL_BK;

  // Write-out items (token m, features n .. n+7): 512 per workgroup, two per thread. The in_proj
  // epilogue's operands are requested first, so they arrive under the K loop.
  constexpr int IPT = 2;
  int it_m[IPT], it_n[IPT];
  bf16x8 s3[IPT][3], w4[IPT][4], b8[IPT];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int item = threadIdx.x + 256 * it;
    it_m[it] = item >> 3;
    it_n[it] = n0 + 8 * (item & 7);
    if constexpr (EPI == DEC_INPROJ_CONV) {
      if (it_m[it] < M && it_n[it] < N) dec_inproj_load(e, it_m[it], it_n[it], s3[it], w4[it], b8[it]);
    }
  }
  // in_proj clears the arrival counters of the out_proj launched after it in the same step
  if constexpr (EPI == DEC_INPROJ_CONV) {
    if (blockIdx.x == 0 && blockIdx.y == 0)
      for (int i = threadIdx.x; i < e.n_counters; i += 256) e.counters[i] = 0;
  }

  // Loads: wave w fills rows 16w .. 16w+15 of both stage tiles, 8 rows per instruction; lane l
  // writes LDS slot l of its instruction (row +l/8, chunk position l%8) and so loads the global
  // chunk that the swizzle puts there. Rows past N (weights) or M (tokens) repeat the last row;
  // their results are never stored. Buffer loads: a descriptor per operand, 32-bit lane offsets,
  // the K advance in the scalar offset.
  // Tiled weights (N a multiple of 64): the block's tiles follow each other along K, 8 KB
  // apiece, so a load instruction reads one contiguous KB and a stage one contiguous 8 KB
  // instead of 64 rows x 128 bytes at the row stride; lanes land in the same LDS positions.
  const bool tiled = EPI != DEC_PARTIAL && e.w_tiled;
  const int wstage = tiled ? DL_TILE : DL_BK * 2;   // weight bytes between stages
  uint32_t woff[2], uoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ dl_swz(r);
    const int wr = n0 + r < N ? r : N - 1 - n0;
    const int ur = r < M ? r : M - 1;
    woff[i] = tiled ? (uint32_t)((kbeg / DL_BK) * DL_TILE + r * (DL_BK * 2) + c * 16)
                    : (uint32_t)(((int64_t)wr * K + kbeg + c * 8) * 2);
    uoff[i] = (uint32_t)(((int64_t)ur * K + kbeg + c * 8) * 2);
  }
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * K), (short)0, 0x7fffffff, kBufWord3);
  const __amdgpu_buffer_rsrc_t urs =
      __builtin_amdgcn_make_buffer_rsrc((void*)U, (short)0, 0x7fffffff, kBufWord3);
#endif
  auto issue = [&](int t, int b) {
#if defined(__HIP_DEVICE_COMPILE__)
    char* base = smem + b * DL_STAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_void_t*)(base + (2 * wave + i) * 1024), 16,
                                               woff[i], t * wstage, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(urs,
                                               (lds_void_t*)(base + DL_TILE + (2 * wave + i) * 1024),
                                               16, uoff[i], t * DL_BK * 2, 0, 0);
    }
#endif
  };

  // Fragments: the A operand is the wave's 32 weight rows, B its 32 token rows; k step j of a
  // stage takes chunk 2j + (lane / 32) of each row. Both row sets start at multiples of 32, so
  // one swizzle serves both.
  const int sw = dl_swz(lane & 31);
  const int offA = (32 * (wave & 1) + (lane & 31)) * 128;
  const int offB = DL_TILE + (32 * (wave >> 1) + (lane & 31)) * 128;
  const int half = lane >> 5;
  f32x16 acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) { acc0[r] = 0.0f; acc1[r] = 0.0f; }
  auto compute = [&](int b) {   // all of a stage's fragment reads, then its four MFMAs
    const char* base = smem + b * DL_STAGE;
    bf16x8 a[4], bb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = ((2 * j + half) ^ sw) << 4;
      a[j] = *reinterpret_cast<const bf16x8*>(base + offA + pos);
      bb[j] = *reinterpret_cast<const bf16x8*>(base + offB + pos);
    }
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], bb[j], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j + 1], bb[j + 1], acc1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // the 8 LDS reads first
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // then the 4 MFMAs
  };

  const int pre = nst < DL_NBUF - 1 ? nst : DL_NBUF - 1;
  for (int t = 0; t < pre; ++t) issue(t, t);
  int t = 0;
  // Steady state: stages t .. t+DL_NBUF-2 in flight (4 loads each per wave); once stage t has
  // landed for every wave (wait, barrier), buffer t-1 is free and stage t+DL_NBUF-1 goes there.
  for (; t + DL_NBUF - 1 < nst; ++t) {
    dl_wait_vmcnt<4 * (DL_NBUF - 2)>();
    __builtin_amdgcn_s_barrier();
    issue(t + DL_NBUF - 1, (t + DL_NBUF - 1) % DL_NBUF);
    compute(t % DL_NBUF);
  }
  dl_wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  for (; t < nst; ++t) compute(t % DL_NBUF);

  // Output tile through LDS (token-major, fp32), then written out by items.
  __syncthreads();
  float* ot = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int f = 32 * (wave & 1) + 8 * (r >> 2) + 4 * half + (r & 3);
    const int m = 32 * (wave >> 1) + (lane & 31);
    ot[m * DL_OUT_PITCH + f] = acc0[r] + acc1[r];
  }
  __syncthreads();
  if constexpr (EPI == DEC_PARTIAL_SUM) {
    dec_partial_sum_epilogue(e, ot, it_m, it_n, n0, M, N, split,
                             reinterpret_cast<int*>(smem + 64 * DL_OUT_PITCH * 4));
    return;
  }
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int m = it_m[it], n = it_n[it];
    if (m >= M || n >= N) continue;
    const float4* src = reinterpret_cast<const float4*>(ot + m * DL_OUT_PITCH + (n - n0));
    const float4 lo = src[0], hi = src[1];
    const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    if constexpr (EPI == DEC_INPROJ_CONV)
      dec_inproj_item(e, m, n, v, s3[it], w4[it], b8[it]);
    else
      dec_store_item<EPI>(e, m, n, N, M, split, v);
  }
}

// Decode copy of a projection's weights in 64 x 64 tiles: tile (b, s) = rows 64b .. 64b+63,
// columns 64s .. 64s+63 of W (N x K, row-major), stored as 64 rows of 64 values, tiles in order
// of b, then s. A workgroup copies one tile: 512 chunks of 16 bytes, two per thread, read as
// 128-byte row segments and written contiguously.
__global__ __launch_bounds__(256)
void tile_weights_kernel(const bf16* __restrict__ W, bf16* __restrict__ tiles, int K) {
  const int kt = K / 64;
  const int64_t tile = blockIdx.x;
  const int64_t b = tile / kt, st = tile % kt;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = threadIdx.x + 256 * h;        // chunk q: row q / 8, columns 8 (q % 8) ..
    const int r = q >> 3, c = (q & 7) * 8;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(W + (64 * b + r) * (int64_t)K + 64 * st + c);
    *reinterpret_cast<bf16x8*>(tiles + tile * 4096 + r * 64 + c) = v;
  }
}

// Split-K partial sums of 4 consecutive outputs, added in split order (deterministic). With
// SPLITS known at compile time every split's load is issued before the first add, so the
// reduction costs about one memory latency instead of one per split.
template <int SPLITS>
__device__ __forceinline__ float4 sum_splits(const float* __restrict__ p, int splits,
                                             int64_t stride) {
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if constexpr (SPLITS > 0) {
    float4 q[SPLITS];
#pragma unroll
    for (int s = 0; s < SPLITS; ++s) q[s] = *reinterpret_cast<const float4*>(p + s * stride);
#pragma unroll
    for (int s = 0; s < SPLITS; ++s) {
      v.x += q[s].x; v.y += q[s].y; v.z += q[s].z; v.w += q[s].w;
    }
  } else {
    for (int s = 0; s < splits; ++s) {
      const float4 q = *reinterpret_cast<const float4*>(p + s * stride);
      v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
    }
  }
  return v;
}

// Sum split-K partials of x_proj: delta (bf16), B and C (fp32); 4 outputs per thread (R and
// the state width are multiples of 4, so a group never straddles two of them).
template <int SPLITS>
__global__ __launch_bounds__(256)
void dec_xproj_reduce_kernel(const float* __restrict__ partial, int splits, int M, int R,
                             bf16* __restrict__ delta, float* __restrict__ Bm,
                             float* __restrict__ Cm) {
  const int N = R + 2 * NS;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * (N / 4)) return;
  const int m = idx / (N / 4), n = (idx % (N / 4)) * 4;
  const float4 v = sum_splits<SPLITS>(partial + (int64_t)m * N + n, splits, (int64_t)M * N);
  if (n < R) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 o = {from_f32<bf16>(v.x), from_f32<bf16>(v.y), from_f32<bf16>(v.z),
                      from_f32<bf16>(v.w)};
    *reinterpret_cast<bf16x4*>(delta + (int64_t)m * R + n) = o;
  } else if (n < R + NS) {
    *reinterpret_cast<float4*>(Bm + m * NS + (n - R)) = v;
  } else {
    *reinterpret_cast<float4*>(Cm + m * NS + (n - R - NS)) = v;
  }
}

constexpr int UPD_CH = 32;   // channels per update workgroup
constexpr int UPD_MT = 16;   // tokens per update workgroup

// Decode update, LDS-staged (dt_rank R = 128 or 256): the same 32 channels x 16 tokens per
// workgroup and the same arithmetic as dec_update_kernel, laid out for whole-line memory access.
// The W_dt rows of the block's channels and the delta rows of its tokens come in through
// direct-to-LDS loads (1 KB of whole rows per instruction; 16-byte chunk c of row r kept at
// position c ^ (r & 15), so the 16 rows an MFMA fragment read serves together hit distinct
// bank groups); wave w sums the w-th quarter of dt_rank on MFMA from there. In the update a
// lane owns four states of one channel (lane = channel (l / 4) of the wave's 16, quad l % 4)
// for 8 tokens, so each state load or store instruction of a wave covers 1 KB of contiguous
// state (16 channels x 64 bytes); y is summed over a channel's 4 lanes with lane exchanges.
template <int R>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(4, 4)))   // 4 workgroups per CU: all 1024 of a 64-row step at once
void dec_update_lds_kernel(const bf16* __restrict__ xh, const bf16* __restrict__ z,
                           const bf16* __restrict__ delta, const float* __restrict__ Bm,
                           const float* __restrict__ Cm, const bf16* __restrict__ W_dt,
                           const float* __restrict__ b_dt, const float* __restrict__ A_log,
                           const float* __restrict__ Dv, float* __restrict__ state,
                           const int32_t* __restrict__ rows, bf16* __restrict__ g, int M,
                           int d_inner) {
  static_assert(R == 128 || R == 256, "dt_rank tile");
  constexpr int CPR = R / 8;                  // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;               // rows per 1 KB load instruction
  constexpr int WI = UPD_CH / RPI;            // load instructions for the W_dt tile
  constexpr int DI = UPD_MT / RPI;            // and for the delta tile
  __shared__ __attribute__((aligned(1024))) bf16 sW[UPD_CH * R];
  __shared__ __attribute__((aligned(1024))) bf16 sD[UPD_MT * R];
  __shared__ float sdt[4][UPD_MT][UPD_CH + 1];
  __shared__ float4 sbc[UPD_MT][8];           // B_t (4 float4) | C_t (4 float4)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // provably uniform
  const int d0 = blockIdx.x * UPD_CH;
  const int m0 = blockIdx.y * UPD_MT;
  const int mend = min(M - m0, UPD_MT);

  // Small operands first: B|C of the tile's tokens, this lane's four A values, D and the bias of
  // its channel, and the state rows of its 8 tokens (slot map); all L2 hits, waited for at once.
  const int t_bc = threadIdx.x >> 3, part = threadIdx.x & 7;
  float4 bcv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (t_bc < mend)
    bcv = *reinterpret_cast<const float4*>((part < 4 ? Bm : Cm) + (int64_t)(m0 + t_bc) * NS +
                                           4 * (part & 3));
  const int cl = 16 * (wave & 1) + (lane >> 2);   // channel within the block
  const int d = d0 + cl;
  const int sq = lane & 3;                        // states 4 sq .. 4 sq + 3
  const float4 al = *reinterpret_cast<const float4*>(A_log + (int64_t)d * NS + 4 * sq);
  const float Dd = Dv[d];
  const float bias = b_dt[d];
  constexpr int TPT = UPD_MT / 2;                 // tokens per lane: (wave >> 1) + 2j
  int32_t srow[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int ml = (wave >> 1) + 2 * j;
    const int m = m0 + (ml < mend ? ml : 0);
    srow[j] = rows ? rows[m] : m;
  }
  dl_wait_vmcnt<0>();
  // Then the W_dt and delta tiles (rows past the batch repeat the tile's first token; unused),
  // and right behind them the state, x and z of this lane's 8 tokens (a token past the batch
  // reads the tile's first token; its results are dropped): 24 loads, so waiting until at most
  // 24 loads are outstanding waits for the tiles alone and leaves the state in flight under the
  // dt_proj MFMAs. Compiler memory barriers keep the two groups in this order.
  constexpr int NDMA = (UPD_CH + UPD_MT) / RPI / 4;   // tile load instructions per wave
  static_assert((WI + DI) % 4 == 0, "tile loads split evenly over the waves");
#if defined(__HIP_DEVICE_COMPILE__)
  {
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W_dt + (int64_t)d0 * R), (short)0, 0x7fffffff, kBufWord3);
    const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(delta + (int64_t)m0 * R), (short)0, 0x7fffffff, kBufWord3);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int q = wave + 4 * i;
      const bool isw = q < WI;
      const int qq = isw ? q : q - WI;
      const int r = RPI * qq + lane / CPR;
      const int c = (lane % CPR) ^ (r & 15);
      const int rr = isw ? r : (r < mend ? r : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          isw ? wrs : drs, (lds_void_t*)((isw ? (char*)sW : (char*)sD) + qq * 1024), 16,
          (uint32_t)((rr * R + c * 8) * 2), 0, 0, 0);
    }
  }
#endif
  asm volatile("" ::: "memory");
  float h[TPT][4], xv[TPT], zv[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int ml = (wave >> 1) + 2 * j;
    const int m = m0 + (ml < mend ? ml : 0);
    const int64_t o = (int64_t)m * d_inner + d;
    xv[j] = to_f32(xh[o]);
    zv[j] = to_f32(z[o]);
    const float4 f = *reinterpret_cast<const float4*>(state + ((int64_t)srow[j] * d_inner + d) * NS +
                                                      4 * sq);
    h[j][0] = f.x; h[j][1] = f.y; h[j][2] = f.z; h[j][3] = f.w;
  }
  dl_wait_vmcnt<3 * TPT>();
  __builtin_amdgcn_s_barrier();                   // every wave's tile loads have landed
  if (t_bc < mend) sbc[t_bc][part] = bcv;
  // dt_proj: wave w sums k in [w R/4, (w+1) R/4) over the block's 32 channels (MFMA A rows)
  // and its tokens (B columns; 16 valid, columns 16..31 repeat them and are dropped)
  {
    const int lr = lane & 31, hf = lane >> 5;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < R / 64; ++s) {
      const int c = (R / 32) * wave + 2 * s + hf;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sW + lr * R + ((c ^ (lr & 15)) << 3));
      const int tr = lr & 15;
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(sD + tr * R + ((c ^ tr) << 3));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    if (lr < UPD_MT) {   // acc row = channel, column = token
#pragma unroll
      for (int r = 0; r < 16; ++r) sdt[wave][lr][8 * (r >> 2) + 4 * hf + (r & 3)] = acc[r];
    }
  }
  // sdt and sbc written by every wave (LDS writes done; the state loads stay in flight)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  float a2[4] = {-fast_exp(al.x) * kLog2e, -fast_exp(al.y) * kLog2e, -fast_exp(al.z) * kLog2e,
                 -fast_exp(al.w) * kLog2e};
  // All of the lane's tokens are updated first, then y is summed over each channel's 4 lanes
  // (DPP quad exchanges: partners 1 apart, then 2 apart; every lane of the quad ends with the
  // same sum, in a fixed order), then one lane per channel writes g.
  float yp[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int ml = (wave >> 1) + 2 * j;
    const int mc = ml < mend ? ml : 0;           // tokens past the batch: computed, not stored
    const float dtv = softplus(((sdt[0][mc][cl] + sdt[1][mc][cl]) +
                                (sdt[2][mc][cl] + sdt[3][mc][cl])) + bias);
    const float dx = dtv * xv[j];
    const float4 b4 = sbc[mc][sq], c4 = sbc[mc][4 + sq];
    const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, cc[4] = {c4.x, c4.y, c4.z, c4.w};
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h[j][k] = fmaf(__builtin_amdgcn_exp2f(dtv * a2[k]), h[j][k], dx * bb[k]);
      acc = fmaf(cc[k], h[j][k], acc);
    }
    yp[j] = acc;
    if (ml < mend)
      *reinterpret_cast<float4*>(state + ((int64_t)srow[j] * d_inner + d) * NS + 4 * sq) =
          make_float4(h[j][0], h[j][1], h[j][2], h[j][3]);
  }
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const float y01 = yp[j] + __int_as_float(__builtin_amdgcn_update_dpp(
                                  0, __float_as_int(yp[j]), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
    yp[j] = y01 + __int_as_float(__builtin_amdgcn_update_dpp(
                      0, __float_as_int(y01), 0x4E, 0xF, 0xF, false));                  // quad [2,3,0,1]
  }
  if (sq == 0) {
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int ml = (wave >> 1) + 2 * j;
      if (ml < mend)
        g[(int64_t)(m0 + ml) * d_inner + d] = from_f32<bf16>(fmaf(Dd, xv[j], yp[j]) * silu(zv[j]));
    }
  }
}

// Dynamic LDS above 64 KB is enabled once per device (per-device flags, thread-safe).
constexpr int kDlMaxDevices = 64;
template <int EPI, int NBUF = 8>
hipError_t launch_dec_gemm_lds(const bf16* U, const bf16* W, int M, int N, int K, int splits,
                               const DecEpiArgs& e, hipStream_t s) {
  constexpr int DL_LDS = NBUF * DL_STAGE;
  static std::atomic<bool> lds_set[kDlMaxDevices];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kDlMaxDevices) return hipErrorInvalidDevice;
  if (!lds_set[dev].load(std::memory_order_acquire)) {
    err = hipFuncSetAttribute((const void*)dec_gemm_lds_kernel<EPI, NBUF>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, DL_LDS);
    if (err != hipSuccess) return err;
    lds_set[dev].store(true, std::memory_order_release);
  }
  dim3 grid((N + 63) / 64, splits);
  hipLaunchKernelGGL((dec_gemm_lds_kernel<EPI, NBUF>), grid, dim3(256), DL_LDS, s, U, W, M, N, K,
                     K / splits, e);
  return hipGetLastError();
}

constexpr int XPROJ_SPLIT_K = 512;   // K per workgroup for x_proj (16 splits at d_inner 8192)
// LDS stage buffers of the in_proj and out_proj launches (measured per step at batch 64 on one
// box, alternating builds: 4 buffers 60.8-60.9 us, 6 buffers 61.1-61.4, 8 buffers 61.4-61.5;
// from the tiled weights 60.2 / 60.7 / 61.0-61.1)
constexpr int DL_NBUF_DECODE = 4;

}  // namespace

bool decode_fast_path_ok(int d_model, int d_inner, int dt_rank) {
  return d_model % 256 == 0 && d_inner % 1024 == 0 && (dt_rank == 128 || dt_rank == 256);
}

int decode_fast_counters(int d_model) { return d_model / 64; }

size_t decode_fast_partial_floats(int d_model, int d_inner, int dt_rank, int batch_tile) {
  const size_t xp = (size_t)(d_inner / XPROJ_SPLIT_K) * batch_tile * (dt_rank + 2 * NS);
  const size_t op = (size_t)OUTPROJ_SPLITS * batch_tile * d_model;
  return xp > op ? xp : op;
}

hipError_t launch_tile_weights(const bf16* W, bf16* tiles, int N, int K, hipStream_t s) {
  if (N <= 0 || K <= 0 || N % 64 || K % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tile_weights_kernel, dim3((unsigned)((int64_t)(N / 64) * (K / 64))),
                     dim3(256), 0, s, W, tiles, K);
  return hipGetLastError();
}

hipError_t launch_dec_in_proj(const bf16* u, const bf16* W_in, bool w_tiled, const bf16* conv_w,
                              const bf16* conv_b, bf16* conv_state, const int32_t* rows,
                              bf16* xh, bf16* z, int* counters, int M, int d_model, int d_inner,
                              hipStream_t s) {
  DecEpiArgs e = {};
  e.w_tiled = w_tiled;
  e.xh = xh; e.z = z; e.conv_state = conv_state; e.rows = rows; e.conv_w = conv_w;
  e.conv_b = conv_b;
  e.counters = counters;
  e.n_counters = decode_fast_counters(d_model);
  e.d_inner = d_inner;
  return launch_dec_gemm_lds<DEC_INPROJ_CONV, DL_NBUF_DECODE>(u, W_in, M, 2 * d_inner, d_model, 1,
                                                              e, s);
}

hipError_t launch_dec_x_proj(const bf16* xh, const bf16* W_x, float* partial, bf16* delta,
                             float* Bm, float* Cm, int M, int d_inner, int dt_rank,
                             hipStream_t s) {
  const int N = dt_rank + 2 * NS;
  const int splits = d_inner / XPROJ_SPLIT_K;   // 128-deep K slice per wave
  DecEpiArgs e = {};
  e.partial = partial;
  hipError_t err = launch_dec_gemm_lds<DEC_PARTIAL>(xh, W_x, M, N, d_inner, splits, e, s);
  if (err != hipSuccess) return err;
  const dim3 rgrid((M * (N / 4) + 255) / 256);
  if (splits == 16)   // d_inner 8192
    hipLaunchKernelGGL(dec_xproj_reduce_kernel<16>, rgrid, dim3(256), 0, s, partial, splits, M,
                       dt_rank, delta, Bm, Cm);
  else
    hipLaunchKernelGGL(dec_xproj_reduce_kernel<0>, rgrid, dim3(256), 0, s, partial, splits, M,
                       dt_rank, delta, Bm, Cm);
  return hipGetLastError();
}

hipError_t launch_dec_update(const bf16* xh, const bf16* z, const bf16* delta, const float* Bm,
                             const float* Cm, const bf16* W_dt, const float* b_dt,
                             const float* A_log, const float* D, float* ssm_state,
                             const int32_t* rows, bf16* g, int M, int d_inner, int dt_rank,
                             hipStream_t s) {
  const dim3 grid(d_inner / UPD_CH, (M + UPD_MT - 1) / UPD_MT);
  if (dt_rank == 256)
    hipLaunchKernelGGL(dec_update_lds_kernel<256>, grid, dim3(256), 0, s, xh, z, delta, Bm, Cm,
                       W_dt, b_dt, A_log, D, ssm_state, rows, g, M, d_inner);
  else   // dt_rank 128 (decode_fast_path_ok)
    hipLaunchKernelGGL(dec_update_lds_kernel<128>, grid, dim3(256), 0, s, xh, z, delta, Bm, Cm,
                       W_dt, b_dt, A_log, D, ssm_state, rows, g, M, d_inner);
  return hipGetLastError();
}

hipError_t launch_dec_out_proj(const bf16* g, const bf16* W_out, bool w_tiled, float* partial,
                               int* counters, bf16* out, int M, int d_model, int d_inner,
                               hipStream_t s) {
  DecEpiArgs e = {};
  e.w_tiled = w_tiled;
  e.partial = partial;
  e.counters = counters;
  e.out = out;
  return launch_dec_gemm_lds<DEC_PARTIAL_SUM, DL_NBUF_DECODE>(g, W_out, M, d_model, d_inner,
                                                              OUTPROJ_SPLITS, e, s);
}

}  // namespace jm
