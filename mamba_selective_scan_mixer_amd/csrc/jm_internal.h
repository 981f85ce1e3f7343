// Internal declarations shared by the library's HIP translation units.
// Device helpers (bf16 conversion, activations) and the host-side launchers
// each kernel file provides. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace jm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

// ---- scalar conversions ------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// gfx950 converts float->bf16 with round-to-nearest-even in hardware.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// ---- activations (fp32) --------------------------------------------------------
// exp(v) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float v) { return __builtin_amdgcn_exp2f(v * kLog2e); }
// SiLU(v) = v * sigmoid(v), with the hardware reciprocal (about 1 ulp) in place of an
// IEEE division.
__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + fast_exp(-v));
}
// log1p(x) for x in [0, 1] with hardware log2. u = fl(1 + x) carries a rounding error
// e = x - (u - 1), computed exactly (Sterbenz), and ln(1 + x) = ln(u) + e / u + O(e^2).
// With e / u taken as e the dropped part is e (1/u - 1), at most 2^-24 x for small x and
// 2^-25 near x = 1: a relative error of order 2^-24 everywhere, so tiny x keeps full
// relative precision (u == 1 gives exactly x) without a division or reciprocal.
__device__ __forceinline__ float log1p_unit(float x) {
  const float u = 1.0f + x;
  return fmaf(__builtin_amdgcn_logf(u), 0.69314718055994531f, x - (u - 1.0f));
}
// softplus(v) = ln(1 + e^v) = max(v, 0) + log1p(e^-|v|): no overflow, and full
// relative precision for the small step sizes the layer uses (v << 0).
__device__ __forceinline__ float softplus(float v) {
  return fmaxf(v, 0.0f) + log1p_unit(fast_exp(-fabsf(v)));
}

// ---- launchers (host) ------------------------------------------------------------
enum EpiKind : int {
  EPI_STORE = 0,     // out0[m*ldo + n] = v                      (act dtype)
  EPI_SPLIT2 = 1,    // n < split: out0[m*split+n], else out1[m*split + n-split]
  EPI_XPROJ = 2,     // n < split: delta (act) ; then B, C (fp32, width n_state each)
  EPI_SOFTPLUS = 3,  // outf[m*N + n] = softplus(v + bias[n])   (fp32)
  EPI_F32 = 4        // outf[m*N + n] = v                          (fp32)
};

struct EpiArgs {
  int kind;
  void* out0;        // act-dtype output (STORE, SPLIT2 first half, XPROJ delta)
  void* out1;        // act-dtype output (SPLIT2 second half)
  float* outf0;      // fp32 output (SOFTPLUS, F32, XPROJ B)
  float* outf1;      // fp32 output (XPROJ C)
  const float* bias; // SOFTPLUS bias
  int split;         // SPLIT2 / XPROJ boundary
  int n_state;       // XPROJ width of B and C
  int ldo;           // STORE row stride
};

// Y[m, n] = sum_k X[m, k] * W[n, k]; X (M, K) row stride ldx, W (N, K) row stride ldw.
hipError_t launch_gemm_bf16(const bf16* X, int64_t ldx, const bf16* W, int64_t ldw,
                            int64_t M, int N, int K, const EpiArgs& epi, hipStream_t s);
hipError_t launch_gemm_f32(const float* X, int64_t ldx, const float* W, int64_t ldw,
                           int64_t M, int N, int K, const EpiArgs& epi, hipStream_t s);

template <typename T>
hipError_t launch_conv_silu(const T* x, T* xh, const T* conv_w, const T* conv_b,
                            const T* init_conv, const int32_t* init_rows, const int32_t* cu,
                            int n_seqs, int64_t n_tok, int d_inner, hipStream_t s);
template <typename T>
hipError_t launch_conv_final(const T* x, const T* init_conv, const int32_t* init_rows,
                             T* final_conv, const int32_t* final_rows, const int32_t* cu,
                             int n_seqs, int d_inner, hipStream_t s);

// Chunked selective scan: phase A (per-chunk end state and decay product),
// phase B (carry across chunks), phase C (outputs g and final states).
template <typename T>
hipError_t launch_scan_chunk_state(const T* x, const float* dt, const float* A_log,
                                   const float* Bm, const float* init, const int32_t* init_rows,
                                   const int32_t* cu, float* agg_P, float* agg_h, int n_seqs,
                                   int64_t n_tok, int d_inner, int chunk_len, int n_chunks,
                                   hipStream_t s);
hipError_t launch_scan_chunk_carry(const float* agg_P, const float* agg_h, float* carry,
                                   int d_inner, int n_chunks, hipStream_t s);
template <typename T>
hipError_t launch_scan_chunk_output(const T* x, const float* dt, const float* A_log,
                                    const float* Bm, const float* Cm, const float* D, const T* z,
                                    T* g, const float* init, const int32_t* init_rows,
                                    float* final_state, const float* carry, const int32_t* cu,
                                    int n_seqs, int64_t n_tok, int d_inner, int chunk_len,
                                    int n_chunks, hipStream_t s);
// Copy row i of src to row rows[i] of dst (rows[i] >= 0), row_floats floats per row.
hipError_t launch_scatter_rows(const float* src, float* dst, const int32_t* rows, int n_rows,
                               int64_t row_floats, hipStream_t s);

// Decode (one token per sequence).
template <typename T>
hipError_t launch_decode_conv(const T* x, T* xh, T* conv_state, const int32_t* rows,
                              const T* conv_w, const T* conv_b, int batch, int d_inner,
                              hipStream_t s);
template <typename T>
hipError_t launch_decode_update(const T* xh, const T* z, const T* delta, const float* Bm,
                                const float* Cm, const T* W_dt, const float* b_dt,
                                const float* A_log, const float* D, float* ssm_state,
                                const int32_t* rows, T* g, int batch, int d_inner, int dt_rank,
                                hipStream_t s);

// Backward of the scan step (scan + D skip + gate) over packed sequences; all gradients
// fp32; d_inner % 64 == 0. Workspace: scan_backward_workspace_floats floats, carved by
// scan_backward_layout. Order: forward chunk states (launch_scan_chunk_state / _carry at
// chunk length layout.chunk), adjoint, carry, main, reduce.
struct ScanBwdLayout {
  int K, chunk;
  float *aggP, *aggh, *carry, *L, *Iin, *dA_part, *dD_part, *bc_part;
};
size_t scan_backward_workspace_floats(int64_t n_tok, int d_inner);
ScanBwdLayout scan_backward_layout(float* ws, int64_t n_tok, int d_inner);
template <typename T>
hipError_t launch_scan_bwd_adjoint(const T* dg, const T* z, const float* dt, const float* A_log,
                                   const float* Cm, const float* dh_last, const int32_t* cu,
                                   const ScanBwdLayout& w, int n_seqs, int64_t n_tok, int d_inner,
                                   hipStream_t s);
hipError_t launch_scan_bwd_carry(const ScanBwdLayout& w, int d_inner, hipStream_t s);
template <typename T>
hipError_t launch_scan_bwd_main(const T* x, const float* dt, const float* A_log, const float* Bm,
                                const float* Cm, const float* D, const T* z, const T* dg,
                                const float* h0, const float* dh_last, const int32_t* cu,
                                const ScanBwdLayout& w, int n_seqs, int64_t n_tok, int d_inner,
                                float* dx, float* ddt, float* dz, float* dh0, hipStream_t s);
hipError_t launch_scan_bwd_reduce(const ScanBwdLayout& w, const float* A_log, int64_t n_tok,
                                  int d_inner, float* dB, float* dC, float* dA_log, float* dD,
                                  hipStream_t s);

// Inner RMSNorm (optional), in place, row by row: delta (M, R) act dtype, B and C (M, 16)
// fp32, each v <- v / sqrt(mean(v^2) + eps) * gain.
template <typename T>
hipError_t launch_inner_rmsnorm(T* delta, float* Bm, float* Cm, const float* g_delta,
                                const float* g_B, const float* g_C, float eps, int64_t M, int R,
                                hipStream_t s);

// Decode fast path (bf16; d_model % 256, d_inner % 1024, dt_rank 128 or 256; <= 64 rows per launch).
bool decode_fast_path_ok(int d_model, int d_inner, int dt_rank);
size_t decode_fast_partial_floats(int d_model, int d_inner, int dt_rank, int batch_tile);
// Arrival counters out_proj needs (one per 64 output features); in_proj zeroes them.
int decode_fast_counters(int d_model);
// rows: state row (slot) of each token row, or NULL for row m = token row m. counters:
// decode_fast_counters(d_model) ints that in_proj sets to zero for the out_proj that follows.
// Decode copy of W (N x K, N and K multiples of 64) in 64 x 64 tiles, tile (b, s) = rows
// 64b.., columns 64s.., tiles ordered by b then s, each 64 rows of 64 values.
hipError_t launch_tile_weights(const bf16* W, bf16* tiles, int N, int K, hipStream_t s);
// W_in / W_out: row-major, or in the tiles above when w_tiled.
hipError_t launch_dec_in_proj(const bf16* u, const bf16* W_in, bool w_tiled, const bf16* conv_w,
                              const bf16* conv_b, bf16* conv_state, const int32_t* rows,
                              bf16* xh, bf16* z, int* counters, int M, int d_model, int d_inner,
                              hipStream_t s);
hipError_t launch_dec_x_proj(const bf16* xh, const bf16* W_x, float* partial, bf16* delta,
                             float* Bm, float* Cm, int M, int d_inner, int dt_rank, hipStream_t s);
hipError_t launch_dec_update(const bf16* xh, const bf16* z, const bf16* delta, const float* Bm,
                             const float* Cm, const bf16* W_dt, const float* b_dt,
                             const float* A_log, const float* D, float* ssm_state,
                             const int32_t* rows, bf16* g, int M, int d_inner, int dt_rank,
                             hipStream_t s);
// counters: zeroed by the launch_dec_in_proj of the same step (stream order).
hipError_t launch_dec_out_proj(const bf16* g, const bf16* W_out, bool w_tiled, float* partial,
                               int* counters, bf16* out, int M, int d_model, int d_inner,
                               hipStream_t s);

}  // namespace jm
