// Selective scan of the Mamba mixer layer, chunked along the packed token axis.
//
// Recurrence per channel d and state n (A = -exp(A_log), fp32 state):
//   h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x^_t ;  y_t = C_t . h_t + D x^_t
// followed by the gate g_t = y_t * SiLU(z_t).
//
// One lane owns one channel and keeps all 16 states in registers; B_t and C_t are
// the same for every channel, so they are read as wave-uniform values. The token
// axis is cut into chunks so that even one 128K-token sequence fills the GPU:
//   A  chunk_state : each chunk runs its tokens from a zero state and records the
//                    end state h_loc and P = exp(A * sum(Delta)) (P = 0 when a
//                    sequence starts inside the chunk: nothing carries across it);
//   B  chunk_carry : carry_k = P_{k-1} carry_{k-1} + h_loc_{k-1}, per (d, n);
//   C  chunk_output: each chunk reruns its tokens from carry_k, emits g and writes
//                    the final state of every sequence that ends in it.
// Sequence starts inside a chunk reset the state to the sequence's initial state
// (or zero); exp is evaluated as exp2 with A pre-scaled by log2(e).
//
// Phases A and C are bound by VALU issue (per state and token: two multiplies, one FMA,
// one exp2; phase C adds the C_t.h FMA). Both run at 8 waves per SIMD (at most 64 VGPRs),
// which the in-place update h = dx*B + h*exp2(dt*A) allows (the form fma(e, h, dx*B) makes
// the compiler alternate registers and copy them back every token). Per-token rows are
// reached through buffer instructions from a wave-uniform row base with 32-bit lane offsets,
// so all per-token address arithmetic is scalar, and each token's lane inputs are loaded
// while the previous token is computed.
#include "jm_internal.h"

namespace jm {
namespace {

constexpr int NS = 16;   // d_state

// Buffer-resource loads and stores: a wave-uniform base (scalar registers) plus a 32-bit
// per-lane byte offset, so per-token addressing stays in scalar arithmetic.
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}
#endif
__device__ __forceinline__ float ld_f32(const void* base, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_of(base), (int)off, 0, 0));
#else
  return 0.0f;
#endif
}
// An activation's bits, kept as a 32-bit value until it is used (two 16-bit loads in flight
// would otherwise be packed into one register, which waits for both).
template <typename T> __device__ __forceinline__ uint32_t ld_bits(const void* base, uint32_t off);
template <> __device__ __forceinline__ uint32_t ld_bits<float>(const void* base, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b32(rsrc_of(base), (int)off, 0, 0);
#else
  return 0u;
#endif
}
template <> __device__ __forceinline__ uint32_t ld_bits<bf16>(const void* base, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rsrc_of(base), (int)off, 0, 0);
#else
  return 0u;
#endif
}
template <typename T> __device__ __forceinline__ float bits_f32(uint32_t v);
template <> __device__ __forceinline__ float bits_f32<float>(uint32_t v) { return __uint_as_float(v); }
template <> __device__ __forceinline__ float bits_f32<bf16>(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ void st_act(void* base, uint32_t off, float v) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc_of(base), (int)off, 0, 0);
#endif
}
__device__ __forceinline__ void st_act(void* base, uint32_t off, bf16 v) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), rsrc_of(base),
                                        (int)off, 0, 0);
#endif
}

__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int n_seqs, int64_t t) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ void load_a2(const float* __restrict__ A_log, int d, float a2[NS]) {
#pragma unroll
  for (int n = 0; n < NS; ++n) a2[n] = -fast_exp(A_log[(int64_t)d * NS + n]) * kLog2e;
}

__device__ __forceinline__ void load16(const float* __restrict__ p, float v[NS]) {
#pragma unroll
  for (int q = 0; q < NS / 4; ++q) {
    float4 f = reinterpret_cast<const float4*>(p)[q];
    v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
  }
}

__device__ __forceinline__ void store16(float* __restrict__ p, const float v[NS]) {
#pragma unroll
  for (int q = 0; q < NS / 4; ++q)
    reinterpret_cast<float4*>(p)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}

// ROWS: whether initial states go through a slot map (init_rows); a compile-time choice so
// the plain path keeps its register allocation and schedule.
template <typename T, bool ROWS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8, 8)))
void scan_chunk_state_kernel(const T* __restrict__ x, const float* __restrict__ dt,
                             const float* __restrict__ A_log, const float* __restrict__ Bm,
                             const float* __restrict__ init,
                             const int32_t* __restrict__ init_rows,
                             const int32_t* __restrict__ cu, float* __restrict__ agg_P,
                             float* __restrict__ agg_h, int n_seqs, int64_t n_tok, int d_inner,
                             int chunk_len) {
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  const int k = blockIdx.y;
  const int64_t t0 = (int64_t)k * chunk_len;
  const int64_t t1 = t0 + chunk_len < n_tok ? t0 + chunk_len : n_tok;
  float a2[NS], h[NS];
  load_a2(A_log, d, a2);
#pragma unroll
  for (int n = 0; n < NS; ++n) h[n] = 0.0f;
  float dsum = 0.0f;
  bool reset = false;
  // Per-token rows are addressed as a wave-uniform row pointer (advanced with scalar
  // arithmetic) plus this lane's 32-bit byte offset; the next token's dt and x are in
  // flight while the current one is computed (the last token re-reads itself).
  const uint32_t of = (uint32_t)d * 4u, oa = (uint32_t)d * (uint32_t)sizeof(T);
  const float* dtp = dt + t0 * d_inner;
  const T* xp = x + t0 * d_inner;
  const float* bp = Bm + t0 * NS;
  float pdt = ld_f32(dtp, of);
  uint32_t px = ld_bits<T>(xp, oa);
  int i = find_seq(cu, n_seqs, t0);
  int64_t t = t0;
  while (t < t1) {
    const int64_t s_begin = cu[i], s_end = cu[i + 1];
    if (s_begin == t) {
      reset = true;
      dsum = 0.0f;
      const int64_t r = ROWS ? (int64_t)init_rows[i] : (int64_t)i;   // -1: zeros
      if (init && r >= 0) load16(init + (r * d_inner + d) * NS, h);
      else
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = 0.0f;
    }
    const int64_t e = s_end < t1 ? s_end : t1;
    const int cnt = (int)(e - t);
    const int last = (int)(t1 - 1 - t);     // tokens left in the chunk after this one
    for (int j = 0; j < cnt; ++j) {
      const float dtv = pdt;
      const float xv = bits_f32<T>(px);
      const int64_t step = j < last ? d_inner : 0;
      dtp += step;
      xp += step;
      pdt = ld_f32(dtp, of);
      px = ld_bits<T>(xp, oa);
      const float dx = dtv * xv;
#pragma unroll
      for (int n = 0; n < NS; ++n)
        h[n] = fmaf(dx, bp[n], h[n] * __builtin_amdgcn_exp2f(dtv * a2[n]));
      bp += NS;
      dsum += dtv;
    }
    t = e;
    ++i;
  }
  float P[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) P[n] = reset ? 0.0f : __builtin_amdgcn_exp2f(a2[n] * dsum);
  const int64_t o = ((int64_t)k * d_inner + d) * NS;
  store16(agg_P + o, P);
  store16(agg_h + o, h);
}

// One thread per (d, n): sequential over chunks (loads coalesced across threads).
__global__ __launch_bounds__(256)
void scan_chunk_carry_kernel(const float* __restrict__ agg_P, const float* __restrict__ agg_h,
                             float* __restrict__ carry, int64_t dn_count, int n_chunks) {
  const int64_t dn = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (dn >= dn_count) return;
  // Chunk 0 always begins a sequence, so its carry is never used; the last
  // chunk's aggregate is never produced.
  float c = 0.0f;
  carry[dn] = c;
  // eight chunks per step: their aggregates are loaded before the chain uses them, so the
  // loads of a step are in flight together (the chain itself is one FMA per chunk)
  constexpr int U = 8;
  for (int k0 = 1; k0 < n_chunks; k0 += U) {
    float P[U], h[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t prev = (int64_t)(k0 + u - 1) * dn_count + dn;
      P[u] = k0 + u < n_chunks ? agg_P[prev] : 0.0f;
      h[u] = k0 + u < n_chunks ? agg_h[prev] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u < n_chunks) {
        c = fmaf(P[u], c, h[u]);
        carry[(int64_t)(k0 + u) * dn_count + dn] = c;
      }
    }
  }
}

template <typename T, bool ROWS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8, 8)))
void scan_chunk_output_kernel(const T* __restrict__ x, const float* __restrict__ dt,
                              const float* __restrict__ A_log, const float* __restrict__ Bm,
                              const float* __restrict__ Cm, const float* __restrict__ Dv,
                              const T* __restrict__ z, T* __restrict__ g,
                              const float* __restrict__ init,
                              const int32_t* __restrict__ init_rows,
                              float* __restrict__ final_state, const float* __restrict__ carry,
                              const int32_t* __restrict__ cu, int n_seqs, int64_t n_tok,
                              int d_inner, int chunk_len) {
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  const int k = blockIdx.y;
  const int64_t t0 = (int64_t)k * chunk_len;
  const int64_t t1 = t0 + chunk_len < n_tok ? t0 + chunk_len : n_tok;
  float a2[NS], h[NS];
  load_a2(A_log, d, a2);
  const float Dd = Dv[d];
  if (carry) load16(carry + ((int64_t)k * d_inner + d) * NS, h);
  else
#pragma unroll
    for (int n = 0; n < NS; ++n) h[n] = 0.0f;
  // Per-token rows are addressed as a wave-uniform row pointer (advanced with scalar
  // arithmetic) plus this lane's 32-bit byte offset; the next token's inputs are in
  // flight while the current one is computed (the last token re-reads itself).
  const uint32_t of = (uint32_t)d * 4u, oa = (uint32_t)d * (uint32_t)sizeof(T);
  const char* dtp = (const char*)(dt + t0 * d_inner);
  const char* xp = (const char*)(x + t0 * d_inner);
  const char* zp = (const char*)(z + t0 * d_inner);
  char* gp = (char*)(g + t0 * d_inner);
  const float* bp = Bm + t0 * NS;
  const float* cp = Cm + t0 * NS;
  float pdt = ld_f32(dtp, of);
  uint32_t px = ld_bits<T>(xp, oa), pz = ld_bits<T>(zp, oa);
  int i = find_seq(cu, n_seqs, t0);
  int64_t t = t0;
  while (t < t1) {
    const int64_t s_begin = cu[i], s_end = cu[i + 1];
    if (s_begin == t) {
      const int64_t r = ROWS ? (int64_t)init_rows[i] : (int64_t)i;   // -1: zeros
      if (init && r >= 0) load16(init + (r * d_inner + d) * NS, h);
      else
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = 0.0f;
    }
    const int64_t e = s_end < t1 ? s_end : t1;
    const int cnt = (int)(e - t);
    const int last = (int)(t1 - 1 - t);
    for (int j = 0; j < cnt; ++j) {
      const float dtv = pdt;
      const float xv = bits_f32<T>(px);
      const float zv = bits_f32<T>(pz);
      const int64_t step = j < last ? (int64_t)d_inner : 0;
      dtp += step * 4;
      xp += step * (int64_t)sizeof(T);
      zp += step * (int64_t)sizeof(T);
      pdt = ld_f32(dtp, of);
      px = ld_bits<T>(xp, oa);
      pz = ld_bits<T>(zp, oa);
      const float dx = dtv * xv;
      float y = Dd * xv;
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        // decay the state in place, then add the input term (no register copies)
        h[n] = fmaf(dx, bp[n], h[n] * __builtin_amdgcn_exp2f(dtv * a2[n]));
        y = fmaf(cp[n], h[n], y);
      }
      st_act(gp, oa, from_f32<T>(y * silu(zv)));
      gp += (int64_t)d_inner * (int64_t)sizeof(T);
      bp += NS;
      cp += NS;
    }
    t = e;
    if (e == s_end && final_state) store16(final_state + ((int64_t)i * d_inner + d) * NS, h);
    ++i;
  }
}

// Decode: one token per sequence (block row = sequence), fused dt_proj + softplus +
// state update + D skip + gate. The state is read and written in place.
template <typename T>
__global__ __launch_bounds__(256)
void decode_update_kernel(const T* __restrict__ xh, const T* __restrict__ z,
                          const T* __restrict__ delta, const float* __restrict__ Bm,
                          const float* __restrict__ Cm, const T* __restrict__ W_dt,
                          const float* __restrict__ b_dt, const float* __restrict__ A_log,
                          const float* __restrict__ Dv, float* __restrict__ state,
                          const int32_t* __restrict__ rows, T* __restrict__ g, int d_inner,
                          int dt_rank) {
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  const int bi = blockIdx.y;
  if (d >= d_inner) return;
  const T* wrow = W_dt + (int64_t)d * dt_rank;
  const T* drow = delta + (int64_t)bi * dt_rank;
  float acc = 0.0f;
  for (int r = 0; r < dt_rank; ++r) acc = fmaf(to_f32(wrow[r]), to_f32(drow[r]), acc);
  const float dtv = softplus(acc + b_dt[d]);
  const int64_t o = (int64_t)bi * d_inner + d;
  const float xv = to_f32(xh[o]);
  const float zv = to_f32(z[o]);
  const float dx = dtv * xv;
  float a2[NS], h[NS];
  load_a2(A_log, d, a2);
  float* st = state + ((rows ? (int64_t)rows[bi] : (int64_t)bi) * d_inner + d) * NS;
  load16(st, h);
  const float* b = Bm + (int64_t)bi * NS;
  const float* c = Cm + (int64_t)bi * NS;
  float y = 0.0f;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    h[n] = fmaf(__builtin_amdgcn_exp2f(dtv * a2[n]), h[n], dx * b[n]);
    y = fmaf(c[n], h[n], y);
  }
  store16(st, h);
  y = fmaf(Dv[d], xv, y);
  g[o] = from_f32<T>(y * silu(zv));
}

// Copy row i of src (row_floats values) to row rows[i] of dst, for rows[i] >= 0.
__global__ __launch_bounds__(256)
void scatter_rows_kernel(const float* __restrict__ src, float* __restrict__ dst,
                         const int32_t* __restrict__ rows, int64_t row_floats) {
  const int i = blockIdx.y;
  const int64_t r = rows[i];
  if (r < 0) return;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < row_floats;
       j += (int64_t)gridDim.x * 256)
    dst[r * row_floats + j] = src[(int64_t)i * row_floats + j];
}

inline int scan_block(int d_inner) { return d_inner % 256 == 0 ? 256 : (d_inner % 128 == 0 ? 128 : 64); }

}  // namespace

template <typename T>
hipError_t launch_scan_chunk_state(const T* x, const float* dt, const float* A_log,
                                   const float* Bm, const float* init, const int32_t* init_rows,
                                   const int32_t* cu,
                                   float* agg_P, float* agg_h, int n_seqs, int64_t n_tok,
                                   int d_inner, int chunk_len, int n_chunks, hipStream_t s) {
  if (n_chunks <= 0) return hipSuccess;
  const int block = scan_block(d_inner);
  dim3 grid(d_inner / block, n_chunks);
  if (init_rows)
    hipLaunchKernelGGL((scan_chunk_state_kernel<T, true>), grid, dim3(block), 0, s, x, dt, A_log,
                       Bm, init, init_rows, cu, agg_P, agg_h, n_seqs, n_tok, d_inner, chunk_len);
  else
    hipLaunchKernelGGL((scan_chunk_state_kernel<T, false>), grid, dim3(block), 0, s, x, dt, A_log,
                       Bm, init, init_rows, cu, agg_P, agg_h, n_seqs, n_tok, d_inner, chunk_len);
  return hipGetLastError();
}

hipError_t launch_scan_chunk_carry(const float* agg_P, const float* agg_h, float* carry,
                                   int d_inner, int n_chunks, hipStream_t s) {
  const int64_t dn = (int64_t)d_inner * NS;
  hipLaunchKernelGGL(scan_chunk_carry_kernel, dim3((unsigned)((dn + 255) / 256)), dim3(256), 0, s,
                     agg_P, agg_h, carry, dn, n_chunks);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_scan_chunk_output(const T* x, const float* dt, const float* A_log,
                                    const float* Bm, const float* Cm, const float* D, const T* z,
                                    T* g, const float* init, const int32_t* init_rows,
                                    float* final_state, const float* carry, const int32_t* cu,
                                    int n_seqs,
                                    int64_t n_tok, int d_inner, int chunk_len, int n_chunks,
                                    hipStream_t s) {
  const int block = scan_block(d_inner);
  dim3 grid(d_inner / block, n_chunks);
  if (init_rows)
    hipLaunchKernelGGL((scan_chunk_output_kernel<T, true>), grid, dim3(block), 0, s, x, dt, A_log,
                       Bm, Cm, D, z, g, init, init_rows, final_state, carry, cu, n_seqs, n_tok,
                       d_inner, chunk_len);
  else
    hipLaunchKernelGGL((scan_chunk_output_kernel<T, false>), grid, dim3(block), 0, s, x, dt, A_log,
                       Bm, Cm, D, z, g, init, init_rows, final_state, carry, cu, n_seqs, n_tok,
                       d_inner, chunk_len);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_decode_update(const T* xh, const T* z, const T* delta, const float* Bm,
                                const float* Cm, const T* W_dt, const float* b_dt,
                                const float* A_log, const float* D, float* ssm_state,
                                const int32_t* rows, T* g, int batch, int d_inner, int dt_rank,
                                hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  dim3 grid((d_inner + 255) / 256, batch);
  hipLaunchKernelGGL(decode_update_kernel<T>, grid, dim3(256), 0, s, xh, z, delta, Bm, Cm, W_dt,
                     b_dt, A_log, D, ssm_state, rows, g, d_inner, dt_rank);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const float* src, float* dst, const int32_t* rows, int n_rows,
                               int64_t row_floats, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  const int64_t bx = (row_floats + 255) / 256 < 64 ? (row_floats + 255) / 256 : 64;
  hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)bx, n_rows), dim3(256), 0, s, src, dst,
                     rows, row_floats);
  return hipGetLastError();
}

#define JM_INST_SCAN(T)                                                                          \
  template hipError_t launch_scan_chunk_state<T>(const T*, const float*, const float*,          \
                                                 const float*, const float*, const int32_t*,    \
                                                 const int32_t*, float*, float*, int, int64_t,  \
                                                 int, int, int, hipStream_t);                   \
  template hipError_t launch_scan_chunk_output<T>(const T*, const float*, const float*,         \
                                                  const float*, const float*, const float*,     \
                                                  const T*, T*, const float*, const int32_t*,   \
                                                  float*, const float*, const int32_t*, int,    \
                                                  int64_t, int, int, int, hipStream_t);         \
  template hipError_t launch_decode_update<T>(const T*, const T*, const T*, const float*,        \
                                              const float*, const T*, const float*,             \
                                              const float*, const float*, float*,               \
                                              const int32_t*, T*, int, int, int, hipStream_t);
JM_INST_SCAN(float)
JM_INST_SCAN(bf16)
#undef JM_INST_SCAN

}  // namespace jm
