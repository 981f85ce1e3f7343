// Single-token decode of the Mamba mixer layer (bf16 weights/activations, fp32
// state), for up to 64 sequences per launch.
//
// At one token per sequence every projection is a skinny (M <= 64) product whose
// cost is streaming the weights (210 MB per step at the Jamba-7B-class sizes), so
// the kernels here are built for bandwidth:
//   dec_gemm      32 output features per workgroup; each wave takes a K slice and
//                 loads weight rows and token rows straight into MFMA operand
//                 registers (no LDS staging): a lane reads 64 contiguous bytes of a
//                 row, and A and B use the same permutation of k, so the products
//                 pair up correctly. Partial sums of the waves are combined in LDS
//                 in a fixed order (deterministic). Optional split-K over a second
//                 grid dimension writes fp32 partials.
//   in_proj epilogue: the conv-state shift, the causal conv (kernel 4) and SiLU are
//                 applied right there for the x half; the z half is stored.
//   xproj_reduce  sums the split-K partials of x_proj in a fixed order.
//   update        per 32 channels x 16 sequences: dt_proj on MFMA, softplus, the
//                 16-state update in place, the D skip and the SiLU(z) gate.
#include "jm_internal.h"

namespace jm {
namespace {

constexpr int NS = 16;
constexpr int DEC_NB = 32;   // output features per workgroup
constexpr int DEC_MT = 64;   // token rows per launch

enum DecEpi : int { DEC_STORE = 0, DEC_INPROJ_CONV = 1, DEC_PARTIAL = 2 };

struct DecEpiArgs {
  bf16* out;             // STORE: (M, N) bf16
  bf16* xh;              // INPROJ: (M, d_inner) conv+SiLU output
  bf16* z;               // INPROJ: (M, d_inner)
  bf16* conv_state;      // INPROJ: (rows, d_inner, 3) in/out
  const int32_t* rows;   // INPROJ: state row of token row m (NULL: m)
  const bf16* conv_w;    // INPROJ: (d_inner, 4)
  const bf16* conv_b;    // INPROJ: (d_inner) or null
  int d_inner;           // INPROJ split point
  float* partial;        // PARTIAL: (splits, M, N) fp32
};

__device__ __forceinline__ void load64B(const bf16* p, bf16x8 v[4]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint4 r = q[j];
    v[j] = *reinterpret_cast<bf16x8*>(&r);
  }
}

template <int WAVES, int FB, int EPI>
__global__ __launch_bounds__(64 * WAVES)
void dec_gemm_kernel(const bf16* __restrict__ U, const bf16* __restrict__ W, int M, int N, int K,
                     int k_per_split, DecEpiArgs e) {
  constexpr int NB = 32 * FB;                   // output features per workgroup
  __shared__ float red[WAVES][FB * 2][16][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * NB;
  const int split = blockIdx.y;
  const int kbeg = split * k_per_split;
  const int kw = k_per_split / WAVES;          // multiple of 64
  const int ka = kbeg + wave * kw;
  const int lrow = lane & 31;
  const int half = lane >> 5;

  const bf16* wp[FB];
#pragma unroll
  for (int f = 0; f < FB; ++f) {
    int wrow = n0 + f * 32 + lrow;
    if (wrow >= N) wrow = N - 1;               // clamped rows are never stored
    wp[f] = W + (int64_t)wrow * K + ka + half * 32;
  }
  // Token rows past M read row 0 instead: an MFMA output column depends only on
  // its own token's operand, and columns >= M are never stored.
  const int t0 = lrow, t1 = lrow + 32;
  const bf16* up0 = U + (int64_t)(t0 < M ? t0 : 0) * K + ka + half * 32;
  const bf16* up1 = U + (int64_t)(t1 < M ? t1 : 0) * K + ka + half * 32;

  f32x16 acc[FB][2];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc[f][0][r] = 0.0f; acc[f][1][r] = 0.0f; }
  // Register double buffer: the loads of block i+1 are in flight while block i's
  // MFMAs run. The steady-state loop has no branches, so the compiler can wait for
  // exactly the older buffer.
  struct Buf { bf16x8 w[FB][4], a[4], b[4]; };
  // Workgroups walk their K slice starting at different 64-wide blocks, so the
  // token rows (shared by every workgroup, served from L2) are not all requested
  // from the same few cache lines at the same moment.
  const int nblk = kw >> 6;
  const int rot = blockIdx.x % nblk;
  auto load = [&](Buf& B, int kk) {
    int blk = (kk >> 6) + rot;
    if (blk >= nblk) blk -= nblk;
    const int ko = blk << 6;
#pragma unroll
    for (int f = 0; f < FB; ++f) load64B(wp[f] + ko, B.w[f]);
    load64B(up0 + ko, B.a);
    load64B(up1 + ko, B.b);
  };
  auto compute = [&](const Buf& B) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        acc[f][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B.w[f][j], B.a[j], acc[f][0], 0, 0, 0);
        acc[f][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B.w[f][j], B.b[j], acc[f][1], 0, 0, 0);
      }
  };
  constexpr int NLOAD = FB * 4 + 8;   // 16-byte loads per block
  constexpr int NMFMA = FB * 8;       // MFMAs per block
  auto order = [&]() {                // next blocks' loads first, then this block's MFMAs
    __builtin_amdgcn_sched_group_barrier(0x020, NLOAD, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NMFMA, 0);
  };
  const int nb = kw >> 6;
  if (nb % 4 == 0) {
    // Four register buffers: blocks i+1..i+3 are in flight while block i computes.
    Buf b0, b1, b2, b3;
    load(b0, 0); load(b1, 64); load(b2, 128);
    int i = 0;
    for (; i + 4 < nb; i += 4) {
      const int k0 = i << 6;
      load(b3, k0 + 192); compute(b0); order();
      load(b0, k0 + 256); compute(b1); order();
      load(b1, k0 + 320); compute(b2); order();
      load(b2, k0 + 384); compute(b3); order();
    }
    load(b3, (i << 6) + 192);
    compute(b0); compute(b1); compute(b2); compute(b3);
  } else {
    // Two register buffers. The loop leaves one block (nb odd) or two (nb even) in flight;
    // a load past the last block would wrap to block `rot` and count it twice.
    Buf b0, b1;
    load(b0, 0);
    int kk = 0;
    for (; kk + 128 < kw; kk += 128) {
      load(b1, kk + 64); compute(b0); order();
      load(b0, kk + 128); compute(b1); order();
    }
    if (kk + 64 < kw) {
      load(b1, kk + 64);
      compute(b0);
      compute(b1);
    } else {
      compute(b0);
    }
  }
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      red[wave][2 * f][r][lane] = acc[f][0][r];
      red[wave][2 * f + 1][r][lane] = acc[f][1][r];
    }
  __syncthreads();
  // FB x 2 x 16 x 64 outputs; block (f, tb), register r, lane l:
  // feature n0 + 32 f + 8(r/4) + 4(l/32) + r%4, token l%32 + 32 tb.
  // Write-out by items of one token and 8 consecutive features (16-byte loads and stores):
  // item (m, g) covers features n0 + 8g .. +7, i.e. f = g/4, r = 4(g%4) + c%4 and
  // l = m%32 + 32(c/4) for feature c of the item. All of an item's global loads are issued
  // before any is used, and a thread's items are independent, so the write-out costs about
  // one memory latency rather than one per output.
  constexpr int ITEMS = 64 * NB / 8;
  constexpr int IPT = (ITEMS + 64 * WAVES - 1) / (64 * WAVES);
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int item = threadIdx.x + it * 64 * WAVES;
    if (item >= ITEMS) break;
    const int m = item / (NB / 8), g = item % (NB / 8);
    const int f = g >> 2, q = g & 3, tb = m >> 5;
    const int n = n0 + 8 * g;
    if (m >= M || n >= N) continue;
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int r = 4 * q + (c & 3), l = (m & 31) + 32 * (c >> 2);
      float a = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) a += red[w][2 * f + tb][r][l];
      v[c] = a;
    }
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
    } else if constexpr (EPI == DEC_PARTIAL) {
      float* dst = e.partial + ((int64_t)split * M + m) * N + n;
      if (whole) {
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
      } else {
        for (int c = 0; c < 8 && n + c < N; ++c) dst[c] = v[c];
      }
    } else {
      // in_proj: features < d_inner are x (conv-state shift, conv, SiLU), the rest z.
      // d_inner % 64 == 0, so an item is entirely x or entirely z.
      const int di = e.d_inner;
      if (n < di) {
        const int64_t row = e.rows ? (int64_t)e.rows[m] : (int64_t)m;
        bf16x8* st = reinterpret_cast<bf16x8*>(e.conv_state + (row * di + n) * 3);   // 48 bytes
        const bf16x8* cw = reinterpret_cast<const bf16x8*>(e.conv_w + (int64_t)n * 4);  // 64 bytes
        bf16x8 s3[3], w4[4], b8;
#pragma unroll
        for (int k = 0; k < 3; ++k) s3[k] = st[k];
#pragma unroll
        for (int k = 0; k < 4; ++k) w4[k] = cw[k];
        if (e.conv_b) b8 = *reinterpret_cast<const bf16x8*>(e.conv_b + n);
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

// out = bf16(sum of split-K partials); 4 outputs per thread (count % 4 == 0).
template <int SPLITS>
__global__ __launch_bounds__(256)
void dec_sum_partials_kernel(const float* __restrict__ partial, int splits, int64_t count,
                             bf16* __restrict__ out) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= count) return;
  const float4 v = sum_splits<SPLITS>(partial + i4, splits, count);
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 o = {from_f32<bf16>(v.x), from_f32<bf16>(v.y), from_f32<bf16>(v.z),
                    from_f32<bf16>(v.w)};
  *reinterpret_cast<bf16x4*>(out + i4) = o;
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

// dt_proj (MFMA) + softplus + state update + D skip + gate for 32 channels x 16 tokens
// (grid.y takes the token quarters of a 64-row tile, so a 64-row step runs 4 d_inner/32
// workgroups: twice as many as with 32-token tiles, 22.6 -> 21.0 us at batch 64, as the
// state reads of some workgroups overlap the state writes of others). Wave w computes a
// 32x32 dt tile over the w-th quarter of dt_rank (columns past the tile's 16 tokens are
// dropped); the four partial tiles are added in LDS. In the update, lane l takes channel
// l % 32 and its tokens one at a time, with their 16 states in registers (every state row
// of the thread's tokens requested before the dt_proj MFMAs).
constexpr int UPD_CH = 32;
constexpr int UPD_MT = 16;
// KQ: each wave's share of dt_rank when known at compile time (0: dt_rank / 4 at run time)
template <int KQ>
__global__ __launch_bounds__(256)
void dec_update_kernel(const bf16* __restrict__ xh, const bf16* __restrict__ z,
                       const bf16* __restrict__ delta, const float* __restrict__ Bm,
                       const float* __restrict__ Cm, const bf16* __restrict__ W_dt,
                       const float* __restrict__ b_dt, const float* __restrict__ A_log,
                       const float* __restrict__ Dv, float* __restrict__ state,
                       const int32_t* __restrict__ rows, bf16* __restrict__ g, int M,
                       int d_inner, int R) {
  __shared__ float sdt[4][UPD_MT][UPD_CH + 1];
  __shared__ float4 sbc[UPD_MT][8];         // B_t (4 float4) | C_t (4 float4) of the tile's tokens
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int d0 = blockIdx.x * UPD_CH;
  const int m0 = blockIdx.y * UPD_MT;
  const int mend = min(M - m0, UPD_MT);
  const int c = lane & (UPD_CH - 1);
  const int d = d0 + c;
  // Everything that does not depend on dt_proj is requested first, so its latency overlaps
  // the dt_proj MFMAs and the barrier: B|C of the tile's tokens (staged into LDS after the
  // MFMAs), A, D, the bias, the state rows and then every state row, x and z of this thread's
  // tokens (ml0, ml0 + 8, ...). A token past the batch reads token m0's rows instead and its
  // results are dropped. State rows of a batch are distinct: the host rejects a slot that
  // appears twice, and without a slot map row m is token m.
  const int t_bc = threadIdx.x >> 3, part = threadIdx.x & 7;
  float4 bcv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (t_bc < mend)
    bcv = *reinterpret_cast<const float4*>((part < 4 ? Bm : Cm) + (int64_t)(m0 + t_bc) * NS +
                                           4 * (part & 3));
  float a2[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) a2[n] = A_log[(int64_t)d * NS + n];
  const float Dd = Dv[d];
  const float bias = b_dt[d];
  constexpr int TPT = UPD_MT / 8;           // tokens per thread
  const int ml0 = (wave << 1) | (lane >> 5);
  int64_t srow[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int m = ml0 + 8 * j < mend ? m0 + ml0 + 8 * j : m0;
    srow[j] = rows ? (int64_t)rows[m] : (int64_t)m;
  }
  {
    // dt_proj on MFMA: this wave sums a quarter of dt_rank; all its fragments are fetched
    // before the first MFMA (dt_rank <= 256 here: at most 4 k-steps per wave)
    const int lrow = lane & 31, half = lane >> 5;
    const int tok = m0 + lrow;              // rows >= M read row 0; their results are unused
    const int kq = KQ ? KQ : R / 4;          // this wave's share of dt_rank (multiple of 32)
    const bf16* dp = delta + (int64_t)(tok < M ? tok : 0) * R + wave * kq + 8 * half;
    const bf16* wp = W_dt + (int64_t)(d0 + lrow) * R + wave * kq + 8 * half;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    for (int kk = 0; kk < kq; kk += 64) {
      bf16x8 a[4], w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = kk + 16 * u < kq ? kk + 16 * u : kk;   // past kq: a repeat, not used
        a[u] = *reinterpret_cast<const bf16x8*>(dp + k);
        w[u] = *reinterpret_cast<const bf16x8*>(wp + k);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (kk + 16 * u < kq) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[u], a[u], acc, 0, 0, 0);
    }
    // acc row = channel, column = token
    if (lrow < UPD_MT) {   // the MFMA's 32 token columns cover this tile's UPD_MT tokens
#pragma unroll
      for (int r = 0; r < 16; ++r) sdt[wave][lrow][8 * (r >> 2) + 4 * half + (r & 3)] = acc[r];
    }
  }
  float h[TPT][NS], xv[TPT], zv[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int m = ml0 + 8 * j < mend ? m0 + ml0 + 8 * j : m0;
    const int64_t o = (int64_t)m * d_inner + d;
    xv[j] = to_f32(xh[o]);
    zv[j] = to_f32(z[o]);
    const float4* st = reinterpret_cast<const float4*>(state + (srow[j] * d_inner + d) * NS);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = st[q];
      h[j][4 * q] = f.x; h[j][4 * q + 1] = f.y; h[j][4 * q + 2] = f.z; h[j][4 * q + 3] = f.w;
    }
  }
  if (t_bc < mend) sbc[t_bc][part] = bcv;
  __syncthreads();
#pragma unroll
  for (int n = 0; n < NS; ++n) a2[n] = -fast_exp(a2[n]) * kLog2e;
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int ml = ml0 + 8 * j;
    if (ml < mend) {
      const int m = m0 + ml;
      const int64_t o = (int64_t)m * d_inner + d;
      const float dtv =
          softplus(((sdt[0][ml][c] + sdt[1][ml][c]) + (sdt[2][ml][c] + sdt[3][ml][c])) + bias);
      const float dx = dtv * xv[j];
      float bb[NS], cc[NS];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 b4 = sbc[ml][q], c4 = sbc[ml][4 + q];
        bb[4 * q] = b4.x; bb[4 * q + 1] = b4.y; bb[4 * q + 2] = b4.z; bb[4 * q + 3] = b4.w;
        cc[4 * q] = c4.x; cc[4 * q + 1] = c4.y; cc[4 * q + 2] = c4.z; cc[4 * q + 3] = c4.w;
      }
      float y = 0.0f;
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        h[j][n] = fmaf(__builtin_amdgcn_exp2f(dtv * a2[n]), h[j][n], dx * bb[n]);
        y = fmaf(cc[n], h[j][n], y);
      }
      float4* st = reinterpret_cast<float4*>(state + (srow[j] * d_inner + d) * NS);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        st[q] = make_float4(h[j][4 * q], h[j][4 * q + 1], h[j][4 * q + 2], h[j][4 * q + 3]);
      y = fmaf(Dd, xv[j], y);
      g[o] = from_f32<bf16>(y * silu(zv[j]));
    }
  }
}

template <int WAVES, int FB, int EPI>
hipError_t launch_dec_gemm(const bf16* U, const bf16* W, int M, int N, int K, int splits,
                           const DecEpiArgs& e, hipStream_t s) {
  dim3 grid((N + 32 * FB - 1) / (32 * FB), splits);
  hipLaunchKernelGGL((dec_gemm_kernel<WAVES, FB, EPI>), grid, dim3(64 * WAVES), 0, s, U, W, M, N,
                     K, K / splits, e);
  return hipGetLastError();
}

constexpr int XPROJ_SPLIT_K = 512;   // K per workgroup for x_proj
constexpr int OUTPROJ_SPLITS = 4;

}  // namespace

bool decode_fast_path_ok(int d_model, int d_inner, int dt_rank) {
  return d_model % 256 == 0 && d_inner % 1024 == 0 && dt_rank % 128 == 0;
}

size_t decode_fast_partial_floats(int d_model, int d_inner, int dt_rank, int batch_tile) {
  const size_t xp = (size_t)(d_inner / XPROJ_SPLIT_K) * batch_tile * (dt_rank + 2 * NS);
  const size_t op = (size_t)OUTPROJ_SPLITS * batch_tile * d_model;
  return xp > op ? xp : op;
}

hipError_t launch_dec_in_proj(const bf16* u, const bf16* W_in, const bf16* conv_w,
                              const bf16* conv_b, bf16* conv_state, const int32_t* rows,
                              bf16* xh, bf16* z, int M, int d_model, int d_inner, hipStream_t s) {
  DecEpiArgs e = {};
  e.xh = xh; e.z = z; e.conv_state = conv_state; e.rows = rows; e.conv_w = conv_w;
  e.conv_b = conv_b;
  e.d_inner = d_inner;
  return launch_dec_gemm<4, 2, DEC_INPROJ_CONV>(u, W_in, M, 2 * d_inner, d_model, 1, e, s);
}

hipError_t launch_dec_x_proj(const bf16* xh, const bf16* W_x, float* partial, bf16* delta,
                             float* Bm, float* Cm, int M, int d_inner, int dt_rank,
                             hipStream_t s) {
  const int N = dt_rank + 2 * NS;
  const int splits = d_inner / XPROJ_SPLIT_K;   // 128-deep K slice per wave
  DecEpiArgs e = {};
  e.partial = partial;
  hipError_t err = launch_dec_gemm<4, 1, DEC_PARTIAL>(xh, W_x, M, N, d_inner, splits, e, s);
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
    hipLaunchKernelGGL(dec_update_kernel<64>, grid, dim3(256), 0, s, xh, z, delta, Bm, Cm, W_dt,
                       b_dt, A_log, D, ssm_state, rows, g, M, d_inner, dt_rank);
  else if (dt_rank == 128)
    hipLaunchKernelGGL(dec_update_kernel<32>, grid, dim3(256), 0, s, xh, z, delta, Bm, Cm, W_dt,
                       b_dt, A_log, D, ssm_state, rows, g, M, d_inner, dt_rank);
  else
    hipLaunchKernelGGL(dec_update_kernel<0>, grid, dim3(256), 0, s, xh, z, delta, Bm, Cm, W_dt,
                       b_dt, A_log, D, ssm_state, rows, g, M, d_inner, dt_rank);
  return hipGetLastError();
}

hipError_t launch_dec_out_proj(const bf16* g, const bf16* W_out, float* partial, bf16* out, int M,
                               int d_model, int d_inner, hipStream_t s) {
  DecEpiArgs e = {};
  e.partial = partial;
  hipError_t err = launch_dec_gemm<4, 2, DEC_PARTIAL>(g, W_out, M, d_model, d_inner,
                                                      OUTPROJ_SPLITS, e, s);
  if (err != hipSuccess) return err;
  const int64_t count = (int64_t)M * d_model;
  hipLaunchKernelGGL(dec_sum_partials_kernel<OUTPROJ_SPLITS>,
                     dim3((unsigned)((count / 4 + 255) / 256)), dim3(256), 0, s, partial,
                     OUTPROJ_SPLITS, count, out);
  return hipGetLastError();
}

}  // namespace jm
