// Backward pass of the scan step (selective scan + D skip + SiLU(z) gate), for training.
//
// Forward, per channel d and state n (A = -exp(A_log), a_t = exp(Delta_t A)):
//   h_t = a_t h_{t-1} + Delta_t B_t x_t,  y_t = C_t . h_t + D x_t,  g_t = y_t SiLU(z_t).
// Given dg (and optionally dL/dh of each sequence's last state), reverse mode runs the
// adjoint lam_t = dL/dh_t backwards, lam_t = a_{t+1} lam_{t+1} + dy_t C_t (dy = dg SiLU(z)),
// and reads every gradient off lam_t, h_{t-1} and h_t:
//   dz = dg y SiLU'(z), dD = sum dy x, dC_t = sum_d dy_t h_t, dh0 = a_first lam_first,
//   dx_t = dy_t D + sum_n lam_t Delta_t B_t, dDelta_t = sum_n lam_t (h_{t-1} a_t A + B_t x_t),
//   dB_t = sum_d lam_t Delta_t x_t, dA_log = A sum_t lam_t h_{t-1} a_t Delta_t.
// Sequences (cu_seqlens) are independent: the state restarts at each sequence start and the
// adjoint at each sequence end (from dL/dh_last or zero).
//
// Chunked like the forward, in reverse: tokens are cut into chunks of BW_CHUNK = 64.
//   1. forward chunk-entry states: the forward's phases A and B (jm_scan.hip) at this
//      chunk length give P_k (decay product, 0 when a sequence starts in chunk k) and the
//      state entering every chunk;
//   2. adjoint out of each chunk (bwd_adjoint_kernel): the adjoint chunk k sends to chunk
//      k-1, computed from zero incoming: L_k = a_s lam_s over the chunk's first sequence
//      segment (0 if a sequence starts at the chunk's first token);
//   3. adjoint into each chunk (bwd_carry_kernel), sequential over chunks in reverse:
//      I_{K-1} = 0, I_{k-1} = L_k + P_k I_k;
//   4. main (bwd_main_kernel), per chunk: a forward pass from the entry state keeps the
//      state before every 8-token sub-block in LDS; then, sub-block by sub-block from the
//      end, the 8 states are recomputed into registers (with their decays) and the adjoint
//      runs backwards from I_k, emitting per-token gradients;
//   5. fixed-order reductions: dB and dC over channel blocks, dA_log and dD over chunks.
// Lanes: thread = (channel d, quad q), q owning states 4q..4q+3; a workgroup of 256
// threads covers 64 channels. Reductions over n run over the 4 lanes of a channel (lane
// shuffles); dB and dC reduce over the wave's 16 channels by shuffles and over the
// workgroup's 4 waves through LDS, then across workgroups in the fixed-order reduction.
// All gradients are fp32. Deterministic: no atomics.
#include "jm_internal.h"

namespace jm {
namespace {

constexpr int NS = 16;
constexpr int BW_CHUNK = 64;         // tokens per chunk
constexpr int BW_CH = 64;            // channels per workgroup
constexpr int SUB = 8;               // tokens per sub-block
constexpr int NSUB = BW_CHUNK / SUB; // sub-blocks per chunk

__device__ __forceinline__ int find_seq_b(const int32_t* __restrict__ cu, int n_seqs, int64_t t) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float sigm(float v) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp(-v));
}

// Lane layout helpers.
struct Lane {
  int d;      // channel
  int q;      // quad: states 4q..4q+3
  int lane;   // lane in the wave
  int wave;
};

__device__ __forceinline__ Lane lane_of(int cblock) {
  Lane L;
  L.lane = threadIdx.x & 63;
  L.wave = threadIdx.x >> 6;
  L.q = threadIdx.x & 3;
  L.d = cblock * BW_CH + (threadIdx.x >> 2);
  return L;
}

__device__ __forceinline__ void load4(const float* p, float v[4]) {
  const float4 f = *reinterpret_cast<const float4*>(p);
  v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
}
__device__ __forceinline__ void store4(float* p, const float v[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// Sum over the 4 lanes of a channel.
__device__ __forceinline__ float quad_sum(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  return v;
}
// Sum over the 16 channels of a wave for one quad position (lanes q, q+4, ..., q+60).
__device__ __forceinline__ float wave_channel_sum(float v) {
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

template <typename T>
__device__ __forceinline__ float dy_of(const T* dg, const T* z, int64_t o) {
  const float zv = to_f32(z[o]);
  return to_f32(dg[o]) * zv * sigm(zv);
}

// ---- 2. adjoint sent by chunk k (k >= 1) to chunk k-1 ------------------------------------
template <typename T>
__global__ __launch_bounds__(256)
void bwd_adjoint_kernel(const T* __restrict__ dg, const T* __restrict__ z,
                        const float* __restrict__ dt, const float* __restrict__ A_log,
                        const float* __restrict__ Cm, const float* __restrict__ dh_last,
                        const int32_t* __restrict__ cu, float* __restrict__ Lout, int n_seqs,
                        int64_t n_tok, int d_inner) {
  const Lane L = lane_of(blockIdx.x);
  const int k = blockIdx.y + 1;
  const int64_t s = (int64_t)k * BW_CHUNK;
  const int64_t e = s + BW_CHUNK < n_tok ? s + BW_CHUNK : n_tok;
  float lam[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int i = find_seq_b(cu, n_seqs, s);
  float* out = Lout + ((int64_t)k * d_inner + L.d) * NS + 4 * L.q;
  if (cu[i] == s) {                      // nothing flows into another sequence
    store4(out, lam);
    return;
  }
  const int64_t e1 = cu[i + 1] < e ? cu[i + 1] : e;
  if (e1 == cu[i + 1] && dh_last) load4(dh_last + ((int64_t)i * d_inner + L.d) * NS + 4 * L.q, lam);
  float a2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a2[j] = -fast_exp(A_log[(int64_t)L.d * NS + 4 * L.q + j]) * kLog2e;
  for (int64_t t = e1 - 1; t >= s; --t) {
    const int64_t o = t * d_inner + L.d;
    const float dy = dy_of(dg, z, o);
    const float dtv = dt[o];
    float c[4];
    load4(Cm + t * NS + 4 * L.q, c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lam[j] = fmaf(dy, c[j], lam[j]);
      lam[j] *= __builtin_amdgcn_exp2f(dtv * a2[j]);     // flows to t-1
    }
  }
  store4(out, lam);
}

// ---- 3. adjoint entering every chunk from the next one ------------------------------------
__global__ __launch_bounds__(256)
void bwd_carry_kernel(const float* __restrict__ Lin, const float* __restrict__ P,
                      float* __restrict__ Iin, int64_t dn, int n_chunks) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= dn) return;
  float I = 0.0f;
  Iin[(int64_t)(n_chunks - 1) * dn + idx] = 0.0f;
  for (int k = n_chunks - 1; k >= 1; --k) {
    // I = adjoint entering chunk k at its end; chunk k passes P_k I + L_k to chunk k-1
    // (P_{K-1} is never needed: I is 0 there)
    const float p = k < n_chunks - 1 ? P[(int64_t)k * dn + idx] : 0.0f;
    I = fmaf(p, I, Lin[(int64_t)k * dn + idx]);
    Iin[(int64_t)(k - 1) * dn + idx] = I;
  }
}

// ---- 4. main: per chunk, states recomputed from LDS checkpoints, adjoint backwards ----------
template <typename T>
__global__ __launch_bounds__(256)
void bwd_main_kernel(const T* __restrict__ x, const float* __restrict__ dt,
                     const float* __restrict__ A_log, const float* __restrict__ Bm,
                     const float* __restrict__ Cm, const float* __restrict__ Dv,
                     const T* __restrict__ z, const T* __restrict__ dg,
                     const float* __restrict__ h0, const float* __restrict__ dh_last,
                     const float* __restrict__ carry, const float* __restrict__ Iin,
                     const int32_t* __restrict__ cu, float* __restrict__ dx,
                     float* __restrict__ ddt, float* __restrict__ dz,
                     float* __restrict__ dBC_part, float* __restrict__ dA_part,
                     float* __restrict__ dD_part, float* __restrict__ dh0, int n_seqs,
                     int64_t n_tok, int d_inner) {
  __shared__ float4 ck[NSUB][256];                 // state before each sub-block, per lane
  __shared__ float stage[SUB][4][2 * NS];          // per-wave dB | dC of each sub-block token
  const Lane L = lane_of(blockIdx.x);
  const int k = blockIdx.y;
  const int64_t s = (int64_t)k * BW_CHUNK;
  const int64_t e = s + BW_CHUNK < n_tok ? s + BW_CHUNK : n_tok;
  const int64_t dn4 = (int64_t)L.d * NS + 4 * L.q;   // this lane's 4 states in a (d, n) row
  float A4[4], a2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    A4[j] = -fast_exp(A_log[dn4 + j]);
    a2[j] = A4[j] * kLog2e;
  }
  const float Dd = Dv[L.d];

  // pass 1: forward from the entry state, keeping the state before each sub-block
  int i = find_seq_b(cu, n_seqs, s);
  float h[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (cu[i] != s) {
    load4(carry + (int64_t)k * d_inner * NS + dn4, h);   // k >= 1 here
  }
  for (int64_t t = s; t < e; ++t) {
    if (t == cu[i + 1]) ++i;
    if (t == cu[i]) {                                     // sequence start: initial state
      if (h0) load4(h0 + (int64_t)i * d_inner * NS + dn4, h);
      else h[0] = h[1] = h[2] = h[3] = 0.0f;
    }
    if (((t - s) & (SUB - 1)) == 0) ck[(t - s) / SUB][threadIdx.x] = make_float4(h[0], h[1], h[2], h[3]);
    const int64_t o = t * d_inner + L.d;
    const float dtv = dt[o];
    const float dxv = dtv * to_f32(x[o]);
    float b[4];
    load4(Bm + t * NS + 4 * L.q, b);
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = fmaf(__builtin_amdgcn_exp2f(dtv * a2[j]), h[j], dxv * b[j]);
  }

  // pass 2: backwards. lam = adjoint arriving at the current token from later ones.
  int ie = find_seq_b(cu, n_seqs, e - 1);
  float lam[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (cu[ie + 1] == e) {
    if (dh_last) load4(dh_last + (int64_t)ie * d_inner * NS + dn4, lam);
  } else {
    load4(Iin + (int64_t)k * d_inner * NS + dn4, lam);
  }
  float dA[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float dDacc = 0.0f;
  const int nsub = (int)((e - s + SUB - 1) / SUB);
  int iseq = ie;                                          // sequence of the current token
  for (int sb = nsub - 1; sb >= 0; --sb) {
    const int64_t t0 = s + (int64_t)sb * SUB;
    const int len = (int)(e - t0 < SUB ? e - t0 : SUB);
    // recompute the sub-block's states before each token, and its decays
    float hp[SUB][4], av[SUB][4];
    {
      const float4 c4 = ck[sb][threadIdx.x];
      float hh[4] = {c4.x, c4.y, c4.z, c4.w};
      int ii = find_seq_b(cu, n_seqs, t0);
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        if (u < len) {
          const int64_t t = t0 + u;
          if (u > 0 && t == cu[ii + 1]) {                 // a sequence starts inside
            ++ii;
            if (h0) load4(h0 + (int64_t)ii * d_inner * NS + dn4, hh);
            else hh[0] = hh[1] = hh[2] = hh[3] = 0.0f;
          }
          const int64_t o = t * d_inner + L.d;
          const float dtv = dt[o];
          const float dxv = dtv * to_f32(x[o]);
          float b[4];
          load4(Bm + t * NS + 4 * L.q, b);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            hp[u][j] = hh[j];
            av[u][j] = __builtin_amdgcn_exp2f(dtv * a2[j]);
            hh[j] = fmaf(av[u][j], hh[j], dxv * b[j]);
          }
        }
      }
    }
#pragma unroll
    for (int u = SUB - 1; u >= 0; --u) {
      if (u < len) {
        const int64_t t = t0 + u;
        while (cu[iseq] > t) --iseq;                      // sequence of token t
        // t ends its sequence inside the chunk: nothing arrives from the next sequence
        // (the chunk's last token got its incoming adjoint before the loop)
        if (t + 1 == cu[iseq + 1] && t + 1 < e) {
          if (dh_last) load4(dh_last + (int64_t)iseq * d_inner * NS + dn4, lam);
          else lam[0] = lam[1] = lam[2] = lam[3] = 0.0f;
        }
        const int64_t o = t * d_inner + L.d;
        const float dtv = dt[o];
        const float xv = to_f32(x[o]);
        const float zv = to_f32(z[o]);
        const float gv = to_f32(dg[o]);
        const float sg = sigm(zv);
        const float dy = gv * zv * sg;
        float b[4], c[4];
        load4(Bm + t * NS + 4 * L.q, b);
        load4(Cm + t * NS + 4 * L.q, c);
        float ypart = 0.0f, ddt_part = 0.0f, dx_part = 0.0f;
        float dBv[4], dCv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float ht = fmaf(av[u][j], hp[u][j], dtv * xv * b[j]);
          ypart = fmaf(c[j], ht, ypart);
          dCv[j] = dy * ht;
          const float lt = fmaf(dy, c[j], lam[j]);                 // lam_t
          const float da = lt * hp[u][j];
          const float dda = da * av[u][j];
          ddt_part = fmaf(dda, A4[j], fmaf(lt * b[j], xv, ddt_part));
          dA[j] = fmaf(dda, dtv, dA[j]);
          dBv[j] = lt * dtv * xv;
          dx_part = fmaf(lt, b[j], dx_part);
          lam[j] = av[u][j] * lt;                                  // flows to t-1
        }
        ypart = quad_sum(ypart);
        ddt_part = quad_sum(ddt_part);
        dx_part = quad_sum(dx_part);
        if (L.q == 0) {
          const float y = fmaf(Dd, xv, ypart);
          dx[o] = fmaf(dx_part, dtv, dy * Dd);
          ddt[o] = ddt_part;
          dz[o] = gv * y * sg * (1.0f + zv * (1.0f - sg));
          dDacc = fmaf(dy, xv, dDacc);
        }
        if (t == cu[iseq] && dh0) store4(dh0 + (int64_t)iseq * d_inner * NS + dn4, lam);
        // dB, dC: sum over the wave's 16 channels, then stage per wave
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dBv[j] = wave_channel_sum(dBv[j]);
          dCv[j] = wave_channel_sum(dCv[j]);
        }
        if (L.lane < 4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            stage[u][L.wave][4 * L.q + j] = dBv[j];
            stage[u][L.wave][NS + 4 * L.q + j] = dCv[j];
          }
        }
      }
    }
    __syncthreads();
    // workgroup partial of dB | dC for the sub-block's tokens: thread = (token, value)
    {
      const int u = threadIdx.x >> 5, v = threadIdx.x & 31;
      if (u < len) {
        const float sum = (stage[u][0][v] + stage[u][1][v]) + (stage[u][2][v] + stage[u][3][v]);
        dBC_part[((int64_t)blockIdx.x * n_tok + t0 + u) * (2 * NS) + v] = sum;
      }
    }
    __syncthreads();
  }
  store4(dA_part + (int64_t)k * d_inner * NS + dn4, dA);
  if (L.q == 0) dD_part[(int64_t)k * d_inner + L.d] = dDacc;
}

// ---- 5. fixed-order reductions ---------------------------------------------------------
__global__ __launch_bounds__(256)
void bwd_reduce_bc_kernel(const float* __restrict__ part, float* __restrict__ dB,
                          float* __restrict__ dC, int n_cblocks, int64_t n_tok) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // token * 32 + value
  if (idx >= n_tok * 2 * NS) return;
  float sum = 0.0f;
  for (int cb = 0; cb < n_cblocks; ++cb) sum += part[(int64_t)cb * n_tok * 2 * NS + idx];
  const int64_t t = idx / (2 * NS);
  const int v = (int)(idx % (2 * NS));
  if (v < NS) dB[t * NS + v] = sum;
  else dC[t * NS + (v - NS)] = sum;
}

__global__ __launch_bounds__(256)
void bwd_reduce_param_kernel(const float* __restrict__ dA_part, const float* __restrict__ dD_part,
                             const float* __restrict__ A_log, float* __restrict__ dA_log,
                             float* __restrict__ dD, int n_chunks, int d_inner) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t dn = (int64_t)d_inner * NS;
  if (idx < dn) {
    float sum = 0.0f;
    for (int k = 0; k < n_chunks; ++k) sum += dA_part[(int64_t)k * dn + idx];
    dA_log[idx] = -fast_exp(A_log[idx]) * sum;     // dA/dA_log = A
  }
  if (idx < d_inner) {
    float sum = 0.0f;
    for (int k = 0; k < n_chunks; ++k) sum += dD_part[(int64_t)k * d_inner + idx];
    dD[idx] = sum;
  }
}

}  // namespace

size_t scan_backward_workspace_floats(int64_t n_tok, int d_inner) {
  const int64_t K = (n_tok + BW_CHUNK - 1) / BW_CHUNK;
  const int64_t dn = (int64_t)d_inner * NS;
  const int64_t ncb = d_inner / BW_CH;
  // forward aggP, aggh, carry; L, Iin; dA partials (K x dn each); dD partials; dB|dC partials
  return (size_t)(6 * K * dn + K * d_inner + ncb * n_tok * 2 * NS);
}

ScanBwdLayout scan_backward_layout(float* ws, int64_t n_tok, int d_inner) {
  ScanBwdLayout w;
  w.K = (int)((n_tok + BW_CHUNK - 1) / BW_CHUNK);
  w.chunk = BW_CHUNK;
  const int64_t dn = (int64_t)d_inner * NS;
  w.aggP = ws;
  w.aggh = w.aggP + (int64_t)w.K * dn;
  w.carry = w.aggh + (int64_t)w.K * dn;
  w.L = w.carry + (int64_t)w.K * dn;
  w.Iin = w.L + (int64_t)w.K * dn;
  w.dA_part = w.Iin + (int64_t)w.K * dn;
  w.dD_part = w.dA_part + (int64_t)w.K * dn;
  w.bc_part = w.dD_part + (int64_t)w.K * d_inner;
  return w;
}

template <typename T>
hipError_t launch_scan_bwd_adjoint(const T* dg, const T* z, const float* dt, const float* A_log,
                                   const float* Cm, const float* dh_last, const int32_t* cu,
                                   const ScanBwdLayout& w, int n_seqs, int64_t n_tok, int d_inner,
                                   hipStream_t s) {
  if (w.K <= 1) return hipSuccess;
  hipLaunchKernelGGL(bwd_adjoint_kernel<T>, dim3(d_inner / BW_CH, w.K - 1), dim3(256), 0, s, dg,
                     z, dt, A_log, Cm, dh_last, cu, w.L, n_seqs, n_tok, d_inner);
  return hipGetLastError();
}

hipError_t launch_scan_bwd_carry(const ScanBwdLayout& w, int d_inner, hipStream_t s) {
  if (w.K <= 1) return hipSuccess;
  const int64_t dn = (int64_t)d_inner * NS;
  hipLaunchKernelGGL(bwd_carry_kernel, dim3((unsigned)((dn + 255) / 256)), dim3(256), 0, s, w.L,
                     w.aggP, w.Iin, dn, w.K);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_scan_bwd_main(const T* x, const float* dt, const float* A_log, const float* Bm,
                                const float* Cm, const float* D, const T* z, const T* dg,
                                const float* h0, const float* dh_last, const int32_t* cu,
                                const ScanBwdLayout& w, int n_seqs, int64_t n_tok, int d_inner,
                                float* dx, float* ddt, float* dz, float* dh0, hipStream_t s) {
  hipLaunchKernelGGL(bwd_main_kernel<T>, dim3(d_inner / BW_CH, w.K), dim3(256), 0, s, x, dt, A_log,
                     Bm, Cm, D, z, dg, h0, dh_last, w.carry, w.Iin, cu, dx, ddt, dz, w.bc_part,
                     w.dA_part, w.dD_part, dh0, n_seqs, n_tok, d_inner);
  return hipGetLastError();
}

hipError_t launch_scan_bwd_reduce(const ScanBwdLayout& w, const float* A_log, int64_t n_tok,
                                  int d_inner, float* dB, float* dC, float* dA_log, float* dD,
                                  hipStream_t s) {
  const int64_t nbc = n_tok * 2 * NS;
  hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3((unsigned)((nbc + 255) / 256)), dim3(256), 0, s,
                     w.bc_part, dB, dC, d_inner / BW_CH, n_tok);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t dn = (int64_t)d_inner * NS;
  hipLaunchKernelGGL(bwd_reduce_param_kernel, dim3((unsigned)((dn + 255) / 256)), dim3(256), 0, s,
                     w.dA_part, w.dD_part, A_log, dA_log, dD, w.K, d_inner);
  return hipGetLastError();
}

#define JM_BWD_INST(T)                                                                          \
  template hipError_t launch_scan_bwd_adjoint<T>(const T*, const T*, const float*, const float*, \
                                                 const float*, const float*, const int32_t*,    \
                                                 const ScanBwdLayout&, int, int64_t, int,        \
                                                 hipStream_t);                                   \
  template hipError_t launch_scan_bwd_main<T>(const T*, const float*, const float*, const float*,\
                                              const float*, const float*, const T*, const T*,    \
                                              const float*, const float*, const int32_t*,        \
                                              const ScanBwdLayout&, int, int64_t, int, float*,   \
                                              float*, float*, float*, hipStream_t);
JM_BWD_INST(float)
JM_BWD_INST(bf16)

}  // namespace jm
