// Causal depthwise conv1d (kernel 4) + bias + SiLU over packed sequences.
//
// Each thread owns 8 consecutive channels (one 16-byte bf16 load per token) and a
// run of consecutive tokens; it keeps the last three pre-conv values in registers
// as a sliding window, so every x value is read from HBM once. Where a new
// sequence begins (row == cu_seqlens[i]) the window restarts from that
// sequence's initial conv state (oldest first) or from zeros, so no value ever
// crosses a sequence boundary.
#include "jm_internal.h"

namespace jm {
namespace {

constexpr int VEC = 8;    // channels per thread
constexpr int KC = 4;     // conv taps (d_conv)

template <typename T>
__device__ __forceinline__ void load8(const T* p, float v[VEC]) {
  if constexpr (sizeof(T) == 2) {
    uint4 raw = *reinterpret_cast<const uint4*>(p);
    const bf16* b = reinterpret_cast<const bf16*>(&raw);
#pragma unroll
    for (int j = 0; j < VEC; ++j) v[j] = (float)b[j];
  } else {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float v[VEC]) {
  if constexpr (sizeof(T) == 2) {
    bf16 b[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) b[j] = from_f32<bf16>(v[j]);
    *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(b);
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// 8 channels of one token as loaded (bit patterns), converted only where they are used, so a
// load in flight is not waited for when it is moved between registers.
template <typename T> struct RawRow;
template <> struct RawRow<bf16> { uint4 a; };
template <> struct RawRow<float> { uint4 a, b; };
__device__ __forceinline__ RawRow<bf16> load_raw(const bf16* p) {
  return RawRow<bf16>{*reinterpret_cast<const uint4*>(p)};
}
__device__ __forceinline__ RawRow<float> load_raw(const float* p) {
  return RawRow<float>{reinterpret_cast<const uint4*>(p)[0], reinterpret_cast<const uint4*>(p)[1]};
}
__device__ __forceinline__ void unpack_raw(const RawRow<bf16>& r, float v[VEC]) {
  const uint32_t u[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(u[j] << 16);
    v[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack_raw(const RawRow<float>& r, float v[VEC]) {
  const uint32_t u[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(u[j]);
}

// Largest i in [0, n_seqs) with cu[i] <= t.
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int n_seqs, int64_t t) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// State row of sequence (or batch row) i: rows[i] when a slot map is given (-1 = no
// state: zeros / nothing written), else i.
__device__ __forceinline__ int64_t state_row(const int32_t* rows, int i) {
  return rows ? (int64_t)rows[i] : (int64_t)i;
}

// History value of channel d, `back` (1..3) positions before sequence i's start.
template <typename T>
__device__ __forceinline__ float hist(const T* __restrict__ init, const int32_t* rows, int i,
                                      int d_inner, int d, int back) {
  const int64_t r = state_row(rows, i);
  if (init == nullptr || r < 0) return 0.0f;
  return to_f32(init[(r * d_inner + d) * (KC - 1) + (KC - 1 - back)]);
}

template <typename T>
__global__ __launch_bounds__(256)
void conv_silu_kernel(const T* __restrict__ x, T* __restrict__ xh,
                      const T* __restrict__ conv_w, const T* __restrict__ conv_b,
                      const T* __restrict__ init, const int32_t* __restrict__ init_rows,
                      const int32_t* __restrict__ cu, int n_seqs, int64_t n_tok, int d_inner,
                      int run_len) {
  const int d0 = (blockIdx.x * blockDim.x + threadIdx.x) * VEC;
  if (d0 >= d_inner) return;
  const int64_t t0 = (int64_t)blockIdx.y * run_len;
  if (t0 >= n_tok) return;
  const int64_t t1 = t0 + run_len < n_tok ? t0 + run_len : n_tok;

  float w[VEC][KC], b[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
#pragma unroll
    for (int k = 0; k < KC; ++k) w[j][k] = to_f32(conv_w[(int64_t)(d0 + j) * KC + k]);
    b[j] = conv_b ? to_f32(conv_b[d0 + j]) : 0.0f;
  }

  int i = find_seq(cu, n_seqs, t0);
  int64_t s_begin = cu[i], s_end = cu[i + 1];
  // win[0] oldest (t-3) .. win[2] newest (t-1)
  float win[KC - 1][VEC];
#pragma unroll
  for (int q = 0; q < KC - 1; ++q) {
    int64_t p = t0 - (KC - 1) + q;
    if (p >= s_begin) {
      load8(x + p * d_inner + d0, win[q]);
    } else {
      int back = (int)(s_begin - p);
#pragma unroll
      for (int j = 0; j < VEC; ++j) win[q][j] = hist(init, init_rows, i, d_inner, d0 + j, back);
    }
  }
  // Tokens in groups of PF: the next group's rows are loaded (kept raw) while the current
  // group is computed; the loads past the run's end re-read its last row.
  constexpr int PF = 4;
  RawRow<T> cur[PF], nxt[PF];
  const int64_t tl = t1 - 1;
#pragma unroll
  for (int q = 0; q < PF; ++q) cur[q] = load_raw(x + (t0 + q < tl ? t0 + q : tl) * d_inner + d0);
  for (int64_t t = t0; t < t1; t += PF) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int64_t p = t + PF + q;
      nxt[q] = load_raw(x + (p < tl ? p : tl) * d_inner + d0);
    }
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int64_t tq = t + q;
      if (tq >= t1) break;
      if (tq == s_end) {   // next sequence starts here: restart the window from its history
        ++i;
        s_begin = tq;
        s_end = cu[i + 1];
#pragma unroll
        for (int w2 = 0; w2 < KC - 1; ++w2)
#pragma unroll
          for (int j = 0; j < VEC; ++j)
            win[w2][j] = hist(init, init_rows, i, d_inner, d0 + j, KC - 1 - w2);
      }
      float xc[VEC], out[VEC];
      unpack_raw(cur[q], xc);
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        float c = b[j];
        c = fmaf(w[j][0], win[0][j], c);
        c = fmaf(w[j][1], win[1][j], c);
        c = fmaf(w[j][2], win[2][j], c);
        c = fmaf(w[j][3], xc[j], c);
        out[j] = silu(c);
        win[0][j] = win[1][j];
        win[1][j] = win[2][j];
        win[2][j] = xc[j];
      }
      store8(xh + tq * d_inner + d0, out);
    }
#pragma unroll
    for (int q = 0; q < PF; ++q) cur[q] = nxt[q];
  }
}

// Final conv state of each sequence: its last three pre-conv values, oldest first
// (reaching into the initial state for sequences shorter than three tokens). All
// three values are read before any is written, so final may alias init (the same row,
// or with slot maps the same slot).
template <typename T>
__global__ __launch_bounds__(256)
void conv_final_kernel(const T* __restrict__ x, const T* init, const int32_t* init_rows,
                       T* final_state, const int32_t* final_rows,
                       const int32_t* __restrict__ cu, int d_inner) {
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = blockIdx.y;
  if (d >= d_inner) return;
  const int64_t rf = state_row(final_rows, i);
  if (rf < 0) return;
  const int64_t ri = state_row(init_rows, i);
  const int64_t s = cu[i], e = cu[i + 1];
  T v[KC - 1];
#pragma unroll
  for (int q = 0; q < KC - 1; ++q) {
    int64_t p = e - (KC - 1) + q;
    if (p >= s) {
      v[q] = x[p * d_inner + d];
    } else {
      int back = (int)(s - p);
      v[q] = (init && ri >= 0) ? init[(ri * d_inner + d) * (KC - 1) + (KC - 1 - back)]
                               : from_f32<T>(0.0f);
    }
  }
#pragma unroll
  for (int q = 0; q < KC - 1; ++q) final_state[(rf * d_inner + d) * (KC - 1) + q] = v[q];
}

// Decode: one token per sequence; shift the window in place.
template <typename T>
__global__ __launch_bounds__(256)
void decode_conv_kernel(const T* __restrict__ x, T* __restrict__ xh, T* __restrict__ state,
                        const int32_t* __restrict__ rows, const T* __restrict__ conv_w,
                        const T* __restrict__ conv_b, int d_inner) {
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  const int bidx = blockIdx.y;
  if (d >= d_inner) return;
  T* st = state + (state_row(rows, bidx) * d_inner + d) * (KC - 1);
  float s0 = to_f32(st[0]), s1 = to_f32(st[1]), s2 = to_f32(st[2]);
  T xr = x[(int64_t)bidx * d_inner + d];
  float xv = to_f32(xr);
  const T* w = conv_w + (int64_t)d * KC;
  float c = conv_b ? to_f32(conv_b[d]) : 0.0f;
  c = fmaf(to_f32(w[0]), s0, c);
  c = fmaf(to_f32(w[1]), s1, c);
  c = fmaf(to_f32(w[2]), s2, c);
  c = fmaf(to_f32(w[3]), xv, c);
  xh[(int64_t)bidx * d_inner + d] = from_f32<T>(silu(c));
  st[0] = st[1];
  st[1] = st[2];
  st[2] = xr;
}

}  // namespace

template <typename T>
hipError_t launch_conv_silu(const T* x, T* xh, const T* conv_w, const T* conv_b,
                            const T* init_conv, const int32_t* init_rows, const int32_t* cu,
                            int n_seqs, int64_t n_tok, int d_inner, hipStream_t s) {
  if (n_tok <= 0) return hipSuccess;
  const int groups = d_inner / VEC;
  const int block = groups >= 256 ? 256 : ((groups + 63) / 64) * 64;
  int64_t run = 32;
  while ((n_tok + run - 1) / run > 65535) run *= 2;
  dim3 grid((groups + block - 1) / block, (unsigned)((n_tok + run - 1) / run));
  hipLaunchKernelGGL(conv_silu_kernel<T>, grid, dim3(block), 0, s, x, xh, conv_w, conv_b,
                     init_conv, init_rows, cu, n_seqs, n_tok, d_inner, (int)run);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_conv_final(const T* x, const T* init_conv, const int32_t* init_rows,
                             T* final_conv, const int32_t* final_rows, const int32_t* cu,
                             int n_seqs, int d_inner, hipStream_t s) {
  if (n_seqs <= 0) return hipSuccess;
  dim3 grid((d_inner + 255) / 256, n_seqs);
  hipLaunchKernelGGL(conv_final_kernel<T>, grid, dim3(256), 0, s, x, init_conv, init_rows,
                     final_conv, final_rows, cu, d_inner);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_decode_conv(const T* x, T* xh, T* conv_state, const int32_t* rows,
                              const T* conv_w, const T* conv_b, int batch, int d_inner,
                              hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  dim3 grid((d_inner + 255) / 256, batch);
  hipLaunchKernelGGL(decode_conv_kernel<T>, grid, dim3(256), 0, s, x, xh, conv_state, rows,
                     conv_w, conv_b, d_inner);
  return hipGetLastError();
}

#define JM_CONV_INST(T)                                                                        \
  template hipError_t launch_conv_silu<T>(const T*, T*, const T*, const T*, const T*,           \
                                          const int32_t*, const int32_t*, int, int64_t, int,     \
                                          hipStream_t);                                          \
  template hipError_t launch_conv_final<T>(const T*, const T*, const int32_t*, T*,               \
                                           const int32_t*, const int32_t*, int, int,             \
                                           hipStream_t);                                         \
  template hipError_t launch_decode_conv<T>(const T*, T*, T*, const int32_t*, const T*, const T*,\
                                            int, int, hipStream_t);
JM_CONV_INST(float)
JM_CONV_INST(bf16)

}  // namespace jm
