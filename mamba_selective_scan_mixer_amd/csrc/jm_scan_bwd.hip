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
//      state before every 8-token sub-block (in registers); then, sub-block by
//      sub-block from the end, the 8 states after each token are recomputed into registers
//      (with their decays) and the adjoint runs backwards from I_k, emitting per-token
//      gradients;
//   5. fixed-order reductions: dB and dC over channel blocks, dA_log and dD over chunks.
// Lanes: thread = (channel d, quad q), q owning states 4q..4q+3; a workgroup of 256
// threads covers 64 channels. The chunk's Delta and x (and B, C) are copied once into LDS
// with coalesced loads; dy and dz's factor dg SiLU'(z) are formed once per element when a
// sub-block's z and dg are copied in, so the per-token work reads LDS only. Reductions over n
// run over the 4 lanes of a channel (DPP quad permutes); dB and dC reduce over the 4 channels
// of a 16-lane row by DPP row rotations, then over the workgroup's 16 rows in LDS, then
// across workgroups in the fixed-order reduction. Per-token outputs go through LDS and leave
// as whole rows. All gradients are fp32. Deterministic: no atomics.
#include "jm_internal.h"

namespace jm {
namespace {

constexpr int NS = 16;
constexpr int BW_CHUNK = 64;         // tokens per chunk
constexpr int BW_CH = 64;            // channels per workgroup
constexpr int SUB = 8;               // tokens per sub-block
constexpr int NSUB = BW_CHUNK / SUB; // sub-blocks per chunk
static_assert(NSUB * 4 == 32, "a lane's sub-block entry states fill one 32-element vector");

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

__device__ __forceinline__ void load4(const float* p, float v[4]) {
  const float4 f = *reinterpret_cast<const float4*>(p);
  v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
}
__device__ __forceinline__ void store4(float* p, const float v[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void zero4(float v[4]) { v[0] = v[1] = v[2] = v[3] = 0.0f; }

// Buffer-resource accesses: a wave-uniform base (scalar registers) plus a 32-bit per-lane
// byte offset. The main loop's addresses then never become 64-bit per-lane pointers, which the
// compiler would otherwise hoist out of the loop and keep live (or spill) for every array.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// the per-sub-block entry states of a lane (4 states x 8 sub-blocks), kept in registers
typedef float f32x32 __attribute__((ext_vector_type(32)));
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}
#endif
__device__ __forceinline__ uint32_t ld_b32(const void* base, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b32(rsrc_at(base), (int)off, 0, 0);
#else
  return 0u;
#endif
}
__device__ __forceinline__ uint2 ld_b64(const void* base, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rsrc_at(base), (int)off, 0, 0);
  return make_uint2(v[0], v[1]);
#else
  return make_uint2(0u, 0u);
#endif
}
// A lane's 4 states of a (d_inner, 16) state row (`lo` = its byte offset in the row).
__device__ __forceinline__ void ld4_at(const float* row, uint32_t lo, float v[4]) {
#if defined(__HIP_DEVICE_COMPILE__)
  const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(rsrc_at(row), (int)lo, 0, 0);
  v[0] = __uint_as_float(r[0]); v[1] = __uint_as_float(r[1]);
  v[2] = __uint_as_float(r[2]); v[3] = __uint_as_float(r[3]);
#endif
}
__device__ __forceinline__ void st4_at(float* row, uint32_t lo, const float v[4]) {
#if defined(__HIP_DEVICE_COMPILE__)
  const u32x4 r = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                   __float_as_uint(v[3])};
  __builtin_amdgcn_raw_buffer_store_b128(r, rsrc_at(row), (int)lo, 0, 0);
#endif
}
// Streaming (non-temporal, cache-policy bit nt) store for the per-token gradient rows: 12 bytes
// per token and channel that nothing in the backward reads again.
__device__ __forceinline__ void st2_at(float* row, uint32_t lo, float a, float b) {
#if defined(__HIP_DEVICE_COMPILE__)
  const u32x2 r = {__float_as_uint(a), __float_as_uint(b)};
  __builtin_amdgcn_raw_buffer_store_b64(r, rsrc_at(row), (int)lo, 0, 2);
#endif
}
__device__ __forceinline__ void st1_at(float* row, uint32_t lo, float a) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), rsrc_at(row), (int)lo, 0, 0);
#endif
}

// 4 consecutive activations as fp32 (bf16: the bit pattern shifted into the high half).
__device__ __forceinline__ void load4f(const float* p, float v[4]) { load4(p, v); }
__device__ __forceinline__ void load4f(const bf16* p, float v[4]) {
  const uint2 r = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(r.x << 16); v[1] = __uint_as_float(r.x & 0xffff0000u);
  v[2] = __uint_as_float(r.y << 16); v[3] = __uint_as_float(r.y & 0xffff0000u);
}

// Lane exchange through DPP (the add folds into v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                            0xF, true));
}
// Sum over the 4 lanes of a channel (quad permutes [1,0,3,2] then [2,3,0,1]).
__device__ __forceinline__ float quad_sum(float v) {
#pragma clang fp contract(off)   // keep the adds separate so they fold into v_add_f32_dpp
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  return v;
}
// Sum over the 4 channels of a 16-lane row, per quad position (row rotations by 4 and 8).
__device__ __forceinline__ float row_channel_sum(float v) {
#pragma clang fp contract(off)
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  return v;
}

// dy = dg SiLU(z) and gz = dg SiLU'(z), SiLU'(z) = s (1 + z (1 - s)), s = sigmoid(z).
__device__ __forceinline__ float2 dy_gz(float zv, float gv) {
  const float sg = sigm(zv);
  return make_float2(gv * zv * sg, gv * sg * fmaf(zv, 1.0f - sg, 1.0f));
}

// Copies rows [0, nrows) of a chunk's (Delta, x) into LDS as {Delta, x} pairs: thread =
// (row tid/16 + 16 j, channels 4 (tid % 16) .. +3); rows past nrows are zero.
template <typename T>
__device__ __forceinline__ void stage_dtx(float2 (*sxd)[BW_CH], const float* __restrict__ dt,
                                          const T* __restrict__ x, int64_t s, int nrows,
                                          int c0, int d_inner) {
  const int cc = 4 * (threadIdx.x & 15);
#pragma unroll
  for (int j = 0; j < BW_CHUNK / 16; ++j) {
    const int r = (threadIdx.x >> 4) + 16 * j;
    float dv[4] = {0.0f, 0.0f, 0.0f, 0.0f}, xv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (r < nrows) {
      const int64_t o = (s + r) * d_inner + c0 + cc;
      load4(dt + o, dv);
      load4f(x + o, xv);
    }
    float4* dst = reinterpret_cast<float4*>(&sxd[r][cc]);
    dst[0] = make_float4(dv[0], xv[0], dv[1], xv[1]);
    dst[1] = make_float4(dv[2], xv[2], dv[3], xv[3]);
  }
}

// ---- 2. adjoint sent by chunk k (k >= 1) to chunk k-1 ------------------------------------
template <typename T>
__global__ __launch_bounds__(256)
void bwd_adjoint_kernel(const T* __restrict__ dg, const T* __restrict__ z,
                        const float* __restrict__ dt, const float* __restrict__ A_log,
                        const float* __restrict__ Cm, const float* __restrict__ dh_last,
                        const int32_t* __restrict__ cu, float* __restrict__ Lout, int n_seqs,
                        int64_t n_tok, int d_inner) {
  __shared__ float2 sdy[BW_CHUNK][BW_CH];         // {Delta, dy}
  __shared__ float4 sc[BW_CHUNK][4];              // C_t[4q..4q+3]
  const int q = threadIdx.x & 3;
  const int c0 = blockIdx.x * BW_CH;
  const int d = c0 + (threadIdx.x >> 2);
  const int k = blockIdx.y + 1;
  const int64_t s = (int64_t)k * BW_CHUNK;
  const int64_t e = s + BW_CHUNK < n_tok ? s + BW_CHUNK : n_tok;
  const int64_t dn4 = (int64_t)d * NS + 4 * q;
  float lam[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int i = find_seq_b(cu, n_seqs, s);
  float* out = Lout + (int64_t)k * d_inner * NS + dn4;
  if (cu[i] == s) {                      // nothing flows into another sequence
    store4(out, lam);
    return;
  }
  const int64_t e1 = cu[i + 1] < e ? cu[i + 1] : e;
  const int n1 = (int)(e1 - s);          // tokens of the chunk's first sequence segment
  {
    const int cc = 4 * (threadIdx.x & 15);
#pragma unroll
    for (int j = 0; j < BW_CHUNK / 16; ++j) {
      const int r = (threadIdx.x >> 4) + 16 * j;
      if (r < n1) {
        const int64_t o = (s + r) * d_inner + c0 + cc;
        float dv[4], zv[4], gv[4];
        load4(dt + o, dv);
        load4f(z + o, zv);
        load4f(dg + o, gv);
        float4* dst = reinterpret_cast<float4*>(&sdy[r][cc]);
        dst[0] = make_float4(dv[0], dy_gz(zv[0], gv[0]).x, dv[1], dy_gz(zv[1], gv[1]).x);
        dst[1] = make_float4(dv[2], dy_gz(zv[2], gv[2]).x, dv[3], dy_gz(zv[3], gv[3]).x);
      }
    }
    const int r = threadIdx.x >> 2;
    if (r < n1) sc[r][q] = *reinterpret_cast<const float4*>(Cm + (s + r) * NS + 4 * q);
  }
  if (e1 == cu[i + 1] && dh_last) load4(dh_last + (int64_t)i * d_inner * NS + dn4, lam);
  float a2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a2[j] = -fast_exp(A_log[dn4 + j]) * kLog2e;
  __syncthreads();
  const int dl = threadIdx.x >> 2;
  for (int r = n1 - 1; r >= 0; --r) {
    const float2 v = sdy[r][dl];
    const float4 c = sc[r][q];
    lam[0] = fmaf(v.y, c.x, lam[0]) * __builtin_amdgcn_exp2f(v.x * a2[0]);   // flows to t-1
    lam[1] = fmaf(v.y, c.y, lam[1]) * __builtin_amdgcn_exp2f(v.x * a2[1]);
    lam[2] = fmaf(v.y, c.z, lam[2]) * __builtin_amdgcn_exp2f(v.x * a2[2]);
    lam[3] = fmaf(v.y, c.w, lam[3]) * __builtin_amdgcn_exp2f(v.x * a2[3]);
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
  // I = adjoint entering chunk k at its end; chunk k passes P_k I + L_k to chunk k-1
  // (P_{K-1} is never needed: I is 0 there). Eight chunks per step, loads first.
  constexpr int U = 8;
  for (int k0 = n_chunks - 1; k0 >= 1; k0 -= U) {
    float p[U], l[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 - u;
      p[u] = k >= 1 && k < n_chunks - 1 ? P[(int64_t)k * dn + idx] : 0.0f;
      l[u] = k >= 1 ? Lin[(int64_t)k * dn + idx] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 - u;
      if (k >= 1) {
        I = fmaf(p[u], I, l[u]);
        Iin[(int64_t)(k - 1) * dn + idx] = I;
      }
    }
  }
}

// ---- 4. main: per chunk, states recomputed from checkpoints, adjoint backwards --------------
// z and dg of one sub-block for the {dy, gz} copy, kept as raw bits until they are used
// (so the loads stay in flight across the sub-block's work): thread = (token tid/32,
// channels 2 (tid % 32), +1).
struct RawZg {
  uint2 z, g;
};
__device__ __forceinline__ void load_raw2(const float* row, uint32_t lo, uint2& r) {
  r = ld_b64(row, lo);
}
__device__ __forceinline__ void load_raw2(const bf16* row, uint32_t lo, uint2& r) {
  r.x = ld_b32(row, lo);
  r.y = 0u;
}
template <typename T> __device__ __forceinline__ void unpack2(uint2 r, float v[2]);
template <> __device__ __forceinline__ void unpack2<float>(uint2 r, float v[2]) {
  v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y);
}
template <> __device__ __forceinline__ void unpack2<bf16>(uint2 r, float v[2]) {
  v[0] = __uint_as_float(r.x << 16); v[1] = __uint_as_float(r.x & 0xffff0000u);
}

// Rows t0 .. t0 + SUB - 1 of z and dg: `lo` = this thread's byte offset from row t0 (token
// tid/32, channels 2 (tid % 32), +1), `valid` = its token is before the chunk's end.
template <typename T>
__device__ __forceinline__ void fetch_zg(const T* __restrict__ z, const T* __restrict__ dg,
                                         int64_t t0, int d_inner, uint32_t lo, bool valid,
                                         RawZg& r) {
  if (valid) {
    load_raw2(z + t0 * d_inner, lo, r.z);
    load_raw2(dg + t0 * d_inner, lo, r.g);
  } else {
    r.z = r.g = make_uint2(0u, 0u);
  }
}

template <typename T>
__device__ __forceinline__ void put_gy(float2 (*sgyb)[BW_CH], int su, int scp, const RawZg& r) {
  float zv[2], gv[2];
  unpack2<T>(r.z, zv);
  unpack2<T>(r.g, gv);
  const float2 a = dy_gz(zv[0], gv[0]), b = dy_gz(zv[1], gv[1]);
  *reinterpret_cast<float4*>(&sgyb[su][scp]) = make_float4(a.x, a.y, b.x, b.y);
}

// Forward over one sub-block (pass 1). CHECK: the sub-block may be short or hold a sequence
// start after its first token (then the state restarts there); without it, neither happens.
template <bool CHECK>
__device__ __forceinline__ void forward_sub(const float2 (*sxd)[BW_CH], const float4 (*sbc)[8],
                                            int r0, int len, int64_t t0, int dl, int q,
                                            const float (&a2)[4], float (&h)[4], int& i,
                                            int& nstart, const int32_t* __restrict__ cu,
                                            const float* __restrict__ h0, int64_t dn,
                                            uint32_t lo4) {
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    if (!CHECK || u < len) {
      if (CHECK && u > 0 && t0 + u == nstart) {
        ++i;
        nstart = cu[i + 1];
        if (h0) ld4_at(h0 + (int64_t)i * dn, lo4, h); else zero4(h);
      }
      const float2 v = sxd[r0 + u][dl];
      const float4 b = sbc[r0 + u][q];
      const float dtx = v.x * v.y;
      h[0] = fmaf(__builtin_amdgcn_exp2f(v.x * a2[0]), h[0], dtx * b.x);
      h[1] = fmaf(__builtin_amdgcn_exp2f(v.x * a2[1]), h[1], dtx * b.y);
      h[2] = fmaf(__builtin_amdgcn_exp2f(v.x * a2[2]), h[2], dtx * b.z);
      h[3] = fmaf(__builtin_amdgcn_exp2f(v.x * a2[3]), h[3], dtx * b.w);
    }
  }
}

// The sub-block's states after each token (hq[u + 1]; hq[0] = state entering it) and decays.
// ii = sequence of the sub-block's first token.
template <bool CHECK>
__device__ __forceinline__ void recompute_sub(const float2 (*sxd)[BW_CH],
                                              const float4 (*sbc)[8], int r0, int len,
                                              int64_t t0, int dl, int q, const float (&a2)[4],
                                              float (&hq)[SUB + 1][4], float (&av)[SUB][4],
                                              int ii, const int32_t* __restrict__ cu,
                                              const float* __restrict__ h0, int64_t dn,
                                              uint32_t lo4) {
  int ns = CHECK ? cu[ii + 1] : 0;
  float hh[4] = {hq[0][0], hq[0][1], hq[0][2], hq[0][3]};
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    if (!CHECK || u < len) {
      if (CHECK && u > 0 && t0 + u == ns) {             // a sequence starts inside
        ++ii;
        ns = cu[ii + 1];
        if (h0) ld4_at(h0 + (int64_t)ii * dn, lo4, hh); else zero4(hh);
      }
      const float2 v = sxd[r0 + u][dl];
      const float4 b = sbc[r0 + u][q];
      const float dtx = v.x * v.y;
      const float bb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        av[u][j] = __builtin_amdgcn_exp2f(v.x * a2[j]);
        hh[j] = fmaf(av[u][j], hh[j], dtx * bb[j]);
        hq[u + 1][j] = hh[j];
      }
    }
  }
}

// The adjoint backwards over one sub-block, with every per-token gradient. CHECK: the
// sub-block may be short or hold sequence boundaries (the adjoint restarts where a sequence
// ends, the state before a sequence's first token is its initial state, dL/dh0 is written
// at a sequence's first token); without it the caller handles the sub-block's edges.
template <bool CHECK>
__device__ __forceinline__ void reverse_sub(float2 (*sxd)[BW_CH], float2 (*sgyb)[BW_CH],
                                            const float4 (*sbc)[8], float (*red)[16][2 * NS],
                                            int r0, int len, int64_t t0, int64_t e, int dl,
                                            int q, int lane, int tid,
                                            const float (&hq)[SUB + 1][4],
                                            const float (&av)[SUB][4], const float (&A4)[4],
                                            float Dd, float (&lam)[4], float (&dA)[4],
                                            float& dDacc, int& iseq,
                                            const int32_t* __restrict__ cu,
                                            const float* __restrict__ h0,
                                            const float* __restrict__ dh_last,
                                            float* __restrict__ dh0, int64_t dn, uint32_t lo4) {
#pragma unroll
  for (int u = SUB - 1; u >= 0; --u) {
    if (!CHECK || u < len) {
      const int64_t t = t0 + u;
      bool start = false;
      if (CHECK) {
        while (cu[iseq] > t) --iseq;                      // sequence of token t
        // t ends its sequence inside the chunk: nothing arrives from the next sequence
        // (the chunk's last token got its incoming adjoint before the loop)
        if (t + 1 == cu[iseq + 1] && t + 1 < e) {
          if (dh_last) ld4_at(dh_last + (int64_t)iseq * dn, lo4, lam); else zero4(lam);
        }
        start = t == cu[iseq];
      }
      float hp[4];
      if (CHECK && start && u > 0) {                      // state before t: the initial one
        if (h0) ld4_at(h0 + (int64_t)iseq * dn, lo4, hp); else zero4(hp);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) hp[j] = hq[u][j];
      }
      const float2 v = sxd[r0 + u][dl];
      const float2 gy = sgyb[u][dl];
      const float4 b4 = sbc[r0 + u][q];
      const float4 c4 = sbc[r0 + u][4 + q];
      const float dtv = v.x, xv = v.y, dy = gy.x, gz = gy.y;
      const float dtx = dtv * xv;
      const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, cc[4] = {c4.x, c4.y, c4.z, c4.w};
      float yp = 0.0f, ddtA = 0.0f, dxp = 0.0f;
      float dBv[4], dCv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float ht = hq[u + 1][j];
        yp = fmaf(cc[j], ht, yp);
        dCv[j] = dy * ht;
        const float lt = fmaf(dy, cc[j], lam[j]);              // lam_t
        const float dda = lt * hp[j] * av[u][j];               // dL/d(a_t) a_t
        ddtA = fmaf(dda, A4[j], ddtA);
        dA[j] = fmaf(dda, dtv, dA[j]);
        dxp = fmaf(lt, bb[j], dxp);
        dBv[j] = lt * dtx;
        lam[j] = av[u][j] * lt;                                // flows to t-1
      }
      yp = quad_sum(yp);
      ddtA = quad_sum(ddtA);
      dxp = quad_sum(dxp);
      // materialise the sums here, outside the lane-masked stores below, so the last DPP
      // step of each stays fused into its add
      asm volatile("" : "+v"(yp), "+v"(ddtA), "+v"(dxp));
      const float y = fmaf(Dd, xv, yp);
      const float2 o1 = make_float2(fmaf(xv, dxp, ddtA), gz * y);     // dDelta, dz
      const float o2 = fmaf(dxp, dtv, dy * Dd);                        // dx
      if (q == 0) {
        sxd[r0 + u][dl] = o1;
        sgyb[u][dl].x = o2;
        dDacc = fmaf(dy, xv, dDacc);
      }
      if (CHECK && start && dh0) st4_at(dh0 + (int64_t)iseq * dn, lo4, lam);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dBv[j] = row_channel_sum(dBv[j]);
        dCv[j] = row_channel_sum(dCv[j]);
      }
      asm volatile("" : "+v"(dBv[0]), "+v"(dBv[1]), "+v"(dBv[2]), "+v"(dBv[3]));
      asm volatile("" : "+v"(dCv[0]), "+v"(dCv[1]), "+v"(dCv[2]), "+v"(dCv[3]));
      if ((lane & 12) == 0) {                        // channel 0 of each row: the row's sums
        const int pr = tid >> 4;                     // row within the workgroup
        *reinterpret_cast<float4*>(&red[u][pr][4 * q]) = make_float4(dBv[0], dBv[1], dBv[2], dBv[3]);
        *reinterpret_cast<float4*>(&red[u][pr][NS + 4 * q]) =
            make_float4(dCv[0], dCv[1], dCv[2], dCv[3]);
      }
    }
    // one token at a time: hoisting later tokens' LDS reads would exceed the register budget
    //__builtin_amdgcn_sched_barrier(0);
  }
}

template <typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
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
  __shared__ float2 sxd[BW_CHUNK][BW_CH];   // {Delta, x}; {dDelta, dz} once a token is done
  __shared__ float2 sgy[2][SUB][BW_CH];     // {dy, gz} of a sub-block (two buffers); dx once done
  __shared__ float4 sbc[BW_CHUNK][8];       // [t][q] = B_t[4q..4q+3], [t][4 + q] = C_t[4q..4q+3]
  __shared__ float red[SUB][16][2 * NS];    // per-row partials of dB | dC, per token

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = tid & 3;
  const int dl = tid >> 2;                  // channel within the workgroup
  const int c0 = blockIdx.x * BW_CH;
  const int d = c0 + dl;
  const int k = blockIdx.y;
  const int64_t s = (int64_t)k * BW_CHUNK;
  const int64_t e = s + BW_CHUNK < n_tok ? s + BW_CHUNK : n_tok;
  const int nt = (int)(e - s);
  const int nsub = (nt + SUB - 1) / SUB;
  const int64_t dn = (int64_t)d_inner * NS;
  const int64_t dn4 = (int64_t)d * NS + 4 * q;   // this lane's 4 states in a (d, n) row
  const uint32_t lo4 = (uint32_t)dn4 * 4u;       //   as a byte offset (d_inner * 64 < 2^32)
  const int su = tid >> 5;                       // copy / write-out map: token of a sub-block
  const int scp = 2 * (tid & 31);                //   and channel pair
  const uint32_t lo_el = (uint32_t)(su * d_inner + c0 + scp);   // its element offset from the
                                                                 // sub-block's first row

  // the chunk's {Delta, x}, B and C; {dy, gz} of the last sub-block
  stage_dtx<T>(sxd, dt, x, s, nt, c0, d_inner);
  if (dl < nt) {
    sbc[dl][q] = *reinterpret_cast<const float4*>(Bm + (s + dl) * NS + 4 * q);
    sbc[dl][4 + q] = *reinterpret_cast<const float4*>(Cm + (s + dl) * NS + 4 * q);
  }
  RawZg nxt;
  fetch_zg(z, dg, s + (int64_t)(nsub - 1) * SUB, d_inner, lo_el * (uint32_t)sizeof(T),
           (nsub - 1) * SUB + su < nt, nxt);
  put_gy<T>(sgy[(nsub - 1) & 1], su, scp, nxt);
  float A4[4], a2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    A4[j] = -fast_exp(A_log[dn4 + j]);
    a2[j] = A4[j] * kLog2e;
  }
  const float Dd = Dv[d];
  __syncthreads();

  // pass 1: forward from the entry state; the state entering sub-block sb is kept in
  // ck[4 sb .. 4 sb + 3]. ck is one register vector indexed by the (wave-uniform) sub-block:
  // the compiler reaches its elements through GPR indexing, where a shifted stack of
  // separate registers cost a copy of every entry per sub-block in both passes.
  f32x32 ck;
  {
    int i = find_seq_b(cu, n_seqs, s);
    float h[4];
    if (cu[i] == s) {
      if (h0) ld4_at(h0 + (int64_t)i * dn, lo4, h); else zero4(h);
    } else {
      ld4_at(carry + (int64_t)k * dn, lo4, h);     // k >= 1 here
    }
    int nstart = cu[i + 1];                        // next sequence start (n_tok if none)
    for (int sb = 0; sb < nsub; ++sb) {
      const int r0 = sb * SUB;
      const int64_t t0 = s + r0;
      const int len = nt - r0 < SUB ? nt - r0 : SUB;
      if (t0 == nstart) {                          // a sequence starts at the sub-block
        ++i;
        nstart = cu[i + 1];
        if (h0) ld4_at(h0 + (int64_t)i * dn, lo4, h); else zero4(h);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) ck[4 * sb + j] = h[j];
      if (len == SUB && nstart >= t0 + SUB)
        forward_sub<false>(sxd, sbc, r0, len, t0, dl, q, a2, h, i, nstart, cu, h0, dn, lo4);
      else
        forward_sub<true>(sxd, sbc, r0, len, t0, dl, q, a2, h, i, nstart, cu, h0, dn, lo4);
    }
  }

  // pass 2: backwards. lam = adjoint arriving at the current token from later ones.
  int iseq = find_seq_b(cu, n_seqs, e - 1);               // sequence of the current token
  float lam[4];
  if (cu[iseq + 1] == e) {
    if (dh_last) ld4_at(dh_last + (int64_t)iseq * dn, lo4, lam); else zero4(lam);
  } else {
    ld4_at(Iin + (int64_t)k * dn, lo4, lam);
  }
  float dA[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float dDacc = 0.0f;
  for (int sb = nsub - 1; sb >= 0; --sb) {
    const int p = sb & 1;
    const int r0 = sb * SUB;
    const int64_t t0 = s + r0;
    const int len = nt - r0 < SUB ? nt - r0 : SUB;
    if (sb > 0) fetch_zg(z, dg, t0 - SUB, d_inner, lo_el * (uint32_t)sizeof(T), true, nxt);
    float hq[SUB + 1][4], av[SUB][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) hq[0][j] = ck[4 * sb + j];
    // sequence of the sub-block's last token; a full sub-block inside one sequence takes the
    // path without per-token boundary checks
    int il = iseq;
    while (cu[il] > t0 + len - 1) --il;
    if (len == SUB && cu[il] <= t0) {
      iseq = il;
      if (t0 + SUB < e && cu[il + 1] == t0 + SUB) {       // its last token ends the sequence
        if (dh_last) ld4_at(dh_last + (int64_t)il * dn, lo4, lam); else zero4(lam);
      }
      recompute_sub<false>(sxd, sbc, r0, len, t0, dl, q, a2, hq, av, il, cu, h0, dn, lo4);
      reverse_sub<false>(sxd, sgy[p], sbc, red, r0, len, t0, e, dl, q, lane, tid, hq, av, A4,
                         Dd, lam, dA, dDacc, iseq, cu, h0, dh_last, dh0, dn, lo4);
      if (cu[il] == t0 && dh0) st4_at(dh0 + (int64_t)il * dn, lo4, lam);
    } else {
      int ii = iseq;
      while (cu[ii] > t0) --ii;
      recompute_sub<true>(sxd, sbc, r0, len, t0, dl, q, a2, hq, av, ii, cu, h0, dn, lo4);
      reverse_sub<true>(sxd, sgy[p], sbc, red, r0, len, t0, e, dl, q, lane, tid, hq, av, A4,
                        Dd, lam, dA, dDacc, iseq, cu, h0, dh_last, dh0, dn, lo4);
    }
    __syncthreads();
    // write-out: dB | dC partial of the workgroup (thread = token su, value tid % 32) and the
    // sub-block's dx, dDelta, dz rows (thread = token su, channels scp, scp + 1)
    if (su < len) {
      float sum = 0.0f;
#pragma unroll
      for (int pr = 0; pr < 16; ++pr) sum += red[su][pr][tid & 31];
      // thread tid writes value tid % 32 of token su: offset tid from the sub-block's first row
      st1_at(dBC_part + ((int64_t)blockIdx.x * n_tok + t0) * (2 * NS), (uint32_t)tid * 4u, sum);
      const float4 o1 = *reinterpret_cast<const float4*>(&sxd[r0 + su][scp]);
      const float4 o2 = *reinterpret_cast<const float4*>(&sgy[p][su][scp]);
      const int64_t row = t0 * d_inner;
      const uint32_t lo = lo_el * 4u;
      st2_at(ddt + row, lo, o1.x, o1.z);
      st2_at(dz + row, lo, o1.y, o1.w);
      st2_at(dx + row, lo, o2.x, o2.z);
    }
    if (sb > 0) put_gy<T>(sgy[p ^ 1], su, scp, nxt);   // {dy, gz} of the next sub-block
    __syncthreads();
  }
  st4_at(dA_part + (int64_t)k * dn, lo4, dA);
  if (q == 0) dD_part[(int64_t)k * d_inner + d] = dDacc;
}

// ---- 5. fixed-order reductions ---------------------------------------------------------
__global__ __launch_bounds__(256)
void bwd_reduce_bc_kernel(const float* __restrict__ part, float* __restrict__ dB,
                          float* __restrict__ dC, int n_cblocks, int64_t n_tok) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // token * 32 + value
  if (idx >= n_tok * 2 * NS) return;
  // eight running sums (channel blocks cb = u mod 8), combined pairwise: fixed order
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = 0; c0 < n_cblocks; c0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 + u < n_cblocks) acc[u] += part[(int64_t)(c0 + u) * n_tok * 2 * NS + idx];
  }
  const float sum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  const int64_t t = idx / (2 * NS);
  const int v = (int)(idx % (2 * NS));
  if (v < NS) dB[t * NS + v] = sum;
  else dC[t * NS + (v - NS)] = sum;
}

// dA_log and dD: sums over the chunks' partials. Workgroup = 64 consecutive entries; wave w
// sums chunks w, w + 4, w + 8, ... with eight running sums (eight loads in flight), and the
// four waves' sums are added in LDS in a fixed order.
__global__ __launch_bounds__(256)
void bwd_reduce_param_kernel(const float* __restrict__ dA_part, const float* __restrict__ dD_part,
                             const float* __restrict__ A_log, float* __restrict__ dA_log,
                             float* __restrict__ dD, int n_chunks, int d_inner) {
  __shared__ float part[4][64];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t dn = (int64_t)d_inner * NS;
  const int64_t nA = dn / 64;                           // workgroups for dA_log
  const bool isA = blockIdx.x < nA;
  const int64_t idx = (isA ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - nA) * 64 + l;
  const float* src = isA ? dA_part : dD_part;
  const int64_t stride = isA ? dn : d_inner;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = w; k0 < n_chunks; k0 += 32) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + 4 * u;
      if (k < n_chunks) acc[u] += src[(int64_t)k * stride + idx];
    }
  }
  part[w][l] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  if (w == 0) {
    const float sum = (part[0][l] + part[1][l]) + (part[2][l] + part[3][l]);
    if (isA) dA_log[idx] = -fast_exp(A_log[idx]) * sum;   // dA/dA_log = A
    else dD[idx] = sum;
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
  const int64_t dn = (int64_t)d_inner * NS;   // d_inner % 64 == 0: whole workgroups
  hipLaunchKernelGGL(bwd_reduce_param_kernel, dim3((unsigned)((dn + d_inner) / 64)), dim3(256), 0,
                     s, w.dA_part, w.dD_part, A_log, dA_log, dD, w.K, d_inner);
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
