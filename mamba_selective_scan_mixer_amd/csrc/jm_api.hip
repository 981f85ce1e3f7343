// C ABI of the Mamba mixer layer library: argument validation, the packed-sequence
// chunk plan, workspace carving and the launch sequences of prefill and decode.
// Validation runs entirely on the host before any HIP call, so a rejected call
// enqueues nothing.
#include "jamba_mamba.h"
#include "jm_internal.h"

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

using namespace jm;

// Fixed scratch of jamba_mamba_decode_step_noalloc: the decode step's temporaries (no
// kernel reads any of it before writing it, so it needs no clearing between calls).
static __device__ __align__(256) unsigned char scratch[JM_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;
// Scan chunk-length override (jm_set_scan_chunk_len); read by every prefill, size query and
// plan, so it is atomic (relaxed: it orders nothing else).
std::atomic<int32_t> g_chunk_override{0};

jm_status fail(jm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

jm_status ok() {
  g_last_error.clear();
  return JM_OK;
}

// ---- kernel timing -----------------------------------------------------------------
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
std::atomic<bool> g_prof{false};   // read by every launch, set by jm_profile_enable
std::mutex g_prof_mu;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t pool_get() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

int prof_begin(const char* name, hipStream_t s) {
  if (!g_prof) return -1;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfRec r{name, pool_get(), pool_get()};
  if (!r.a || !r.b) return -1;
  (void)hipEventRecord(r.a, s);
  g_recs.push_back(r);
  return (int)g_recs.size() - 1;
}

void prof_end(int idx, hipStream_t s) {
  if (idx < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  (void)hipEventRecord(g_recs[idx].b, s);
}

#define JM_LAUNCH(name, call)                                                        \
  do {                                                                               \
    int prof_idx_ = prof_begin(name, stream);                                        \
    hipError_t err_ = (call);                                                        \
    prof_end(prof_idx_, stream);                                                     \
    if (err_ != hipSuccess)                                                          \
      return fail(JM_ERR_HIP, "%s launch failed: %s", name, hipGetErrorString(err_)); \
  } while (0)

// ---- validation ----------------------------------------------------------------------
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t act_size(const jm_layer_dims& d) { return d.act_dtype == JM_BF16 ? 2 : 4; }

jm_status check_dims(const jm_layer_dims* d) {
  if (!d) return fail(JM_ERR_INVALID_ARG, "dims is NULL");
  if ((d->act_dtype != JM_F32 && d->act_dtype != JM_BF16) ||
      (d->weight_dtype != JM_F32 && d->weight_dtype != JM_BF16))
    return fail(JM_ERR_INVALID_ARG, "unknown dtype (act %d, weight %d)", d->act_dtype,
                d->weight_dtype);
  if (d->act_dtype != d->weight_dtype)
    return fail(JM_ERR_UNSUPPORTED, "act and weight dtypes must match (both fp32 or both bf16)");
  if (d->d_model <= 0 || d->d_inner <= 0 || d->d_state <= 0 || d->d_conv <= 0 || d->dt_rank <= 0)
    return fail(JM_ERR_INVALID_ARG, "layer sizes must be positive");
  if (d->d_state != 16) return fail(JM_ERR_UNSUPPORTED, "d_state must be 16 (got %d)", d->d_state);
  if (d->d_conv != 4) return fail(JM_ERR_UNSUPPORTED, "d_conv must be 4 (got %d)", d->d_conv);
  if (d->d_model % 64 || d->d_inner % 64)
    return fail(JM_ERR_UNSUPPORTED, "d_model and d_inner must be multiples of 64 (got %d, %d)",
                d->d_model, d->d_inner);
  if (d->dt_rank % 8)
    return fail(JM_ERR_UNSUPPORTED, "dt_rank must be a multiple of 8 (got %d)", d->dt_rank);
  if ((int64_t)d->d_inner * 2 > 0x7fffffff) return fail(JM_ERR_UNSUPPORTED, "d_inner too large");
  return JM_OK;
}

jm_status check_weights(const jm_layer_weights* w) {
  if (!w) return fail(JM_ERR_INVALID_ARG, "weights is NULL");
  const void* req[] = {w->in_proj_w, w->conv_w, w->x_proj_w, w->dt_proj_w, w->dt_proj_b,
                       w->A_log, w->D, w->out_proj_w};
  const char* names[] = {"in_proj_w", "conv_w", "x_proj_w", "dt_proj_w", "dt_proj_b",
                         "A_log", "D", "out_proj_w"};
  for (int i = 0; i < 8; ++i) {
    if (!req[i]) return fail(JM_ERR_INVALID_ARG, "weights->%s is NULL", names[i]);
    if (!aligned16(req[i])) return fail(JM_ERR_ALIGNMENT, "weights->%s not 16-byte aligned", names[i]);
  }
  if (w->conv_b && !aligned16(w->conv_b))
    return fail(JM_ERR_ALIGNMENT, "weights->conv_b not 16-byte aligned");
  const int n_gains = (w->dt_norm_w != nullptr) + (w->B_norm_w != nullptr) + (w->C_norm_w != nullptr);
  if (n_gains != 0 && n_gains != 3)
    return fail(JM_ERR_INVALID_ARG, "inner norm: dt_norm_w, B_norm_w and C_norm_w must be all "
                "set or all NULL");
  if (n_gains == 3) {
    if (!(w->norm_eps > 0.0f) || !(w->norm_eps < 3.0e38f))
      return fail(JM_ERR_INVALID_ARG, "inner norm: norm_eps must be finite and > 0");
    if (!aligned16(w->dt_norm_w) || !aligned16(w->B_norm_w) || !aligned16(w->C_norm_w))
      return fail(JM_ERR_ALIGNMENT, "inner norm gains must be 16-byte aligned");
  }
  if ((w->in_proj_w_tiles != nullptr) != (w->out_proj_w_tiles != nullptr))
    return fail(JM_ERR_INVALID_ARG, "decode tiles: in_proj_w_tiles and out_proj_w_tiles must be "
                "both set or both NULL");
  if (w->in_proj_w_tiles && (!aligned16(w->in_proj_w_tiles) || !aligned16(w->out_proj_w_tiles)))
    return fail(JM_ERR_ALIGNMENT, "decode tiles must be 16-byte aligned");
  return JM_OK;
}

bool decode_tiles_apply(const jm_layer_dims& d) {
  return d.act_dtype == JM_BF16 && decode_fast_path_ok(d.d_model, d.d_inner, d.dt_rank);
}

// Decode entry points: tiled weights only where the bf16 decode kernels run.
jm_status check_decode_tiles(const jm_layer_dims* d, const jm_layer_weights* w) {
  if (w->in_proj_w_tiles && !decode_tiles_apply(*d))
    return fail(JM_ERR_UNSUPPORTED, "decode tiles are read by the bf16 decode kernels only "
                "(d_model %% 256 == 0, d_inner %% 1024 == 0, dt_rank 128 or 256)");
  return JM_OK;
}

jm_status check_cu(const int32_t* cu, int32_t n_seqs, int64_t total) {
  if (!cu) return fail(JM_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
  if (cu[0] != 0) return fail(JM_ERR_SHAPE, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
  for (int32_t i = 0; i < n_seqs; ++i)
    if (cu[i + 1] <= cu[i])
      return fail(JM_ERR_SHAPE, "sequence %d is empty or cu_seqlens decreases (%d -> %d)", i,
                  cu[i], cu[i + 1]);
  if ((int64_t)cu[n_seqs] != total)
    return fail(JM_ERR_SHAPE, "cu_seqlens[n_seqs] = %d but total_tokens = %lld", cu[n_seqs],
                (long long)total);
  return JM_OK;
}

// ---- plan ----------------------------------------------------------------------------
int scan_block(int d_inner) { return d_inner % 256 == 0 ? 256 : (d_inner % 128 == 0 ? 128 : 64); }

void plan_chunks(const jm_layer_dims& d, int64_t T, int32_t* chunk_len, int32_t* n_chunks) {
  int64_t cl;
  const int32_t forced = g_chunk_override.load(std::memory_order_relaxed);
  if (forced > 0) {
    cl = forced;
  } else {
    // Aim for ~16384 workgroups across channel groups x chunks: 8 are resident per CU at a
    // time, and many short chunks (256 tokens for one 128K sequence at d_inner 8192) keep
    // every CU busy to the end; fewer, longer chunks leave the last round partly idle.
    const int64_t groups = d.d_inner / scan_block(d.d_inner);
    const int64_t want = (16384 + groups - 1) / groups;
    cl = (T + want - 1) / want;
    if (cl < 64) cl = 64;
    cl = (cl + 15) / 16 * 16;
  }
  if (cl > 0x7fffffff) cl = 0x7fffffff;
  *chunk_len = (int32_t)cl;
  *n_chunks = (int32_t)((T + cl - 1) / cl);
}

// ---- workspace layouts -------------------------------------------------------------------
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct PrefillLayout {
  size_t x, z, xh, delta, Bm, Cm, dt, agg, total;
};
size_t scan_agg_bytes(const jm_layer_dims& d, int32_t n_chunks);

PrefillLayout prefill_layout(const jm_layer_dims& d, int64_t T, int32_t n_chunks) {
  PrefillLayout L;
  const size_t a = act_size(d);
  const size_t di = (size_t)d.d_inner;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  L.x = take(T * di * a);
  L.z = take(T * di * a);
  L.xh = take(T * di * a);
  L.delta = take(T * (size_t)d.dt_rank * a);
  L.Bm = take(T * 16 * sizeof(float));
  L.Cm = take(T * 16 * sizeof(float));
  L.dt = take(T * di * sizeof(float));
  L.agg = take(3 * scan_agg_bytes(d, n_chunks));   // decay products | end states | carries
  L.total = off;
  return L;
}

struct DecodeLayout {
  size_t x, z, xh, delta, Bm, Cm, g, partial, counters, total;
};

DecodeLayout decode_layout(const jm_layer_dims& d, int64_t b) {
  DecodeLayout L;
  const size_t a = act_size(d);
  const size_t di = (size_t)d.d_inner;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  L.x = take(b * di * a);
  L.z = take(b * di * a);
  L.xh = take(b * di * a);
  L.delta = take(b * (size_t)d.dt_rank * a);
  L.Bm = take(b * 16 * sizeof(float));
  L.Cm = take(b * 16 * sizeof(float));
  L.g = take(b * di * a);
  const bool fast = d.act_dtype == JM_BF16 && decode_fast_path_ok(d.d_model, d.d_inner, d.dt_rank);
  L.partial = take(fast ? decode_fast_partial_floats(d.d_model, d.d_inner, d.dt_rank, 64) * sizeof(float)
                        : 0);
  L.counters = take(fast ? decode_fast_counters(d.d_model) * sizeof(int) : 0);
  L.total = off;
  return L;
}

template <typename T>
hipError_t gemm(const T* X, int64_t ldx, const T* W, int64_t ldw, int64_t M, int N, int K,
                const EpiArgs& e, hipStream_t s) {
  if constexpr (sizeof(T) == 2)
    return launch_gemm_bf16(X, ldx, W, ldw, M, N, K, e, s);
  else
    return launch_gemm_f32(X, ldx, W, ldw, M, N, K, e, s);
}

EpiArgs epi_none() {
  EpiArgs e;
  std::memset(&e, 0, sizeof(e));
  return e;
}

// ---- prefill steps (each also exported on its own as a jm_stage_* entry point) -------------
template <typename T>
jm_status step_in_proj(const jm_layer_dims& d, const jm_layer_weights& w, const T* u,
                       int64_t n_tok, T* x, T* z, hipStream_t stream) {
  EpiArgs e = epi_none();
  e.kind = EPI_SPLIT2; e.out0 = x; e.out1 = z; e.split = d.d_inner;
  JM_LAUNCH("in_proj", gemm<T>(u, d.d_model, static_cast<const T*>(w.in_proj_w), d.d_model,
                               n_tok, 2 * d.d_inner, d.d_model, e, stream));
  return JM_OK;
}

// init_rows / final_rows: state row (slot) of each sequence, -1 = none; NULL = row i.
template <typename T>
jm_status step_conv(const jm_layer_dims& d, const jm_layer_weights& w, const T* x,
                    const int32_t* cu, int32_t n_seqs, int64_t n_tok, const T* init_conv,
                    T* xh, T* final_conv, hipStream_t stream,
                    const int32_t* init_rows = nullptr, const int32_t* final_rows = nullptr) {
  JM_LAUNCH("conv1d_silu",
            launch_conv_silu<T>(x, xh, static_cast<const T*>(w.conv_w),
                                static_cast<const T*>(w.conv_b), init_conv, init_rows, cu, n_seqs,
                                n_tok, d.d_inner, stream));
  if (final_conv)
    JM_LAUNCH("conv_final", launch_conv_final<T>(x, init_conv, init_rows, final_conv, final_rows,
                                                 cu, n_seqs, d.d_inner, stream));
  return JM_OK;
}

template <typename T>
jm_status step_x_proj(const jm_layer_dims& d, const jm_layer_weights& w, const T* xh,
                      int64_t n_tok, T* delta, float* Bm, float* Cm, hipStream_t stream) {
  EpiArgs e = epi_none();
  e.kind = EPI_XPROJ; e.out0 = delta; e.outf0 = Bm; e.outf1 = Cm; e.split = d.dt_rank;
  e.n_state = 16;
  JM_LAUNCH("x_proj", gemm<T>(xh, d.d_inner, static_cast<const T*>(w.x_proj_w), d.d_inner, n_tok,
                              d.dt_rank + 32, d.d_inner, e, stream));
  if (w.dt_norm_w)
    JM_LAUNCH("inner_norm", launch_inner_rmsnorm<T>(delta, Bm, Cm, w.dt_norm_w, w.B_norm_w,
                                                    w.C_norm_w, w.norm_eps, n_tok, d.dt_rank,
                                                    stream));
  return JM_OK;
}

template <typename T>
jm_status step_dt_proj(const jm_layer_dims& d, const jm_layer_weights& w, const T* delta,
                       int64_t n_tok, float* dt, hipStream_t stream) {
  EpiArgs e = epi_none();
  e.kind = EPI_SOFTPLUS; e.outf0 = dt; e.bias = w.dt_proj_b;
  JM_LAUNCH("dt_proj", gemm<T>(delta, d.dt_rank, static_cast<const T*>(w.dt_proj_w), d.dt_rank,
                               n_tok, d.d_inner, d.dt_rank, e, stream));
  return JM_OK;
}

// Scan aggregates (chunk decay products, chunk end states, carries) after the given offset.
size_t scan_agg_bytes(const jm_layer_dims& d, int32_t n_chunks) {
  return n_chunks > 1 ? align256((size_t)n_chunks * d.d_inner * 16 * sizeof(float)) : 0;
}

template <typename T>
jm_status step_scan(const jm_layer_dims& d, const jm_layer_weights& w, const T* xh,
                    const float* dt, const float* Bm, const float* Cm, const T* z,
                    const int32_t* cu, int32_t n_seqs, int64_t n_tok, const float* init_ssm,
                    T* g, float* final_ssm, char* agg, int32_t chunk_len, int32_t n_chunks,
                    hipStream_t stream, const int32_t* init_rows = nullptr) {
  const size_t ab = scan_agg_bytes(d, n_chunks);
  float* aggP = reinterpret_cast<float*>(agg);
  float* aggh = reinterpret_cast<float*>(agg + ab);
  float* carry = reinterpret_cast<float*>(agg + 2 * ab);
  const int di = d.d_inner;
  if (n_chunks > 1) {
    JM_LAUNCH("scan_chunk_state",
              launch_scan_chunk_state<T>(xh, dt, w.A_log, Bm, init_ssm, init_rows, cu, aggP, aggh,
                                         n_seqs, n_tok, di, chunk_len, n_chunks - 1, stream));
    JM_LAUNCH("scan_chunk_carry", launch_scan_chunk_carry(aggP, aggh, carry, di, n_chunks, stream));
  }
  JM_LAUNCH("scan_chunk_output",
            launch_scan_chunk_output<T>(xh, dt, w.A_log, Bm, Cm, w.D, z, g, init_ssm, init_rows,
                                        final_ssm, n_chunks > 1 ? carry : nullptr, cu, n_seqs,
                                        n_tok, di, chunk_len, n_chunks, stream));
  return JM_OK;
}

template <typename T>
jm_status step_out_proj(const jm_layer_dims& d, const jm_layer_weights& w, const T* g,
                        int64_t n_tok, T* out, hipStream_t stream) {
  EpiArgs e = epi_none();
  e.kind = EPI_STORE; e.out0 = out; e.ldo = d.d_model;
  JM_LAUNCH("out_proj", gemm<T>(g, d.d_inner, static_cast<const T*>(w.out_proj_w), d.d_inner,
                                n_tok, d.d_model, d.d_inner, e, stream));
  return JM_OK;
}

// With slot maps (init_rows / final_rows, device arrays): the states live in caches of
// n_slots rows; init_conv / init_ssm and final_conv are the caches, and final_ssm_tmp is a
// per-sequence workspace buffer that is scattered into the SSM cache (final_ssm_cache)
// after the scan, so no sequence's state is overwritten while another chunk still reads it.
template <typename T>
jm_status run_prefill(const jm_layer_dims& d, const jm_layer_weights& w, const T* u,
                      const int32_t* cu, int32_t n_seqs, int64_t n_tok, const T* init_conv,
                      const float* init_ssm, T* out, T* final_conv, float* final_ssm,
                      char* ws, int32_t chunk_len, int32_t n_chunks, hipStream_t stream,
                      const int32_t* init_rows = nullptr, const int32_t* final_rows = nullptr,
                      float* final_ssm_cache = nullptr) {
  const PrefillLayout L = prefill_layout(d, n_tok, n_chunks);
  T* x = reinterpret_cast<T*>(ws + L.x);
  T* z = reinterpret_cast<T*>(ws + L.z);
  T* xh = reinterpret_cast<T*>(ws + L.xh);
  T* delta = reinterpret_cast<T*>(ws + L.delta);
  float* Bm = reinterpret_cast<float*>(ws + L.Bm);
  float* Cm = reinterpret_cast<float*>(ws + L.Cm);
  float* dt = reinterpret_cast<float*>(ws + L.dt);
  T* g = x;  // x is dead once the conv and its final state are done
  jm_status st;
  if ((st = step_in_proj<T>(d, w, u, n_tok, x, z, stream)) != JM_OK) return st;
  if ((st = step_conv<T>(d, w, x, cu, n_seqs, n_tok, init_conv, xh, final_conv, stream,
                         init_rows, final_rows)) != JM_OK)
    return st;
  if ((st = step_x_proj<T>(d, w, xh, n_tok, delta, Bm, Cm, stream)) != JM_OK) return st;
  if ((st = step_dt_proj<T>(d, w, delta, n_tok, dt, stream)) != JM_OK) return st;
  if ((st = step_scan<T>(d, w, xh, dt, Bm, Cm, z, cu, n_seqs, n_tok, init_ssm, g, final_ssm,
                         ws + L.agg, chunk_len, n_chunks, stream, init_rows)) != JM_OK)
    return st;
  if (final_ssm_cache && final_rows)
    JM_LAUNCH("state_scatter", launch_scatter_rows(final_ssm, final_ssm_cache, final_rows, n_seqs,
                                                   (int64_t)d.d_inner * 16, stream));
  if ((st = step_out_proj<T>(d, w, g, n_tok, out, stream)) != JM_OK) return st;
  return ok();
}

// Decode update for `b` rows: dt_proj + softplus + state update + D skip + gate (the fused
// decode kernel; also exported on its own as jm_stage_decode_update). rows: state row (slot) of
// each batch row, NULL = row i. The bf16 kernel takes at most 64 rows per launch.
template <typename T>
jm_status step_decode_update(const jm_layer_dims& d, const jm_layer_weights& w, const T* xh,
                             const T* z, const T* delta, const float* Bm, const float* Cm,
                             int32_t b, float* ssm_state, const int32_t* rows, T* g,
                             hipStream_t stream) {
  const int di = d.d_inner, R = d.dt_rank;
  if constexpr (sizeof(T) == 2) {
    if (decode_fast_path_ok(d.d_model, di, R)) {
      for (int32_t b0 = 0; b0 < b; b0 += 64) {
        const int M = b - b0 < 64 ? b - b0 : 64;
        float* st = rows ? ssm_state : ssm_state + (int64_t)b0 * di * 16;
        JM_LAUNCH("dec_update",
                  launch_dec_update(xh + (int64_t)b0 * di, z + (int64_t)b0 * di,
                                    delta + (int64_t)b0 * R, Bm + (int64_t)b0 * 16,
                                    Cm + (int64_t)b0 * 16, static_cast<const bf16*>(w.dt_proj_w),
                                    w.dt_proj_b, w.A_log, w.D, st, rows ? rows + b0 : nullptr,
                                    g + (int64_t)b0 * di, M, di, R, stream));
      }
      return JM_OK;
    }
  }
  JM_LAUNCH("dec_update",
            launch_decode_update<T>(xh, z, delta, Bm, Cm, static_cast<const T*>(w.dt_proj_w),
                                    w.dt_proj_b, w.A_log, w.D, ssm_state, rows, g, b, di, R,
                                    stream));
  return JM_OK;
}

// rows (device, batch entries) maps batch row -> state row (slot) of conv_state / ssm_state;
// NULL: batch row b uses state row b.
template <typename T>
jm_status run_decode(const jm_layer_dims& d, const jm_layer_weights& w, const T* u, int32_t b,
                     T* conv_state, float* ssm_state, T* out, char* ws, hipStream_t stream,
                     const int32_t* rows = nullptr) {
  const DecodeLayout L = decode_layout(d, b);
  T* x = reinterpret_cast<T*>(ws + L.x);
  T* z = reinterpret_cast<T*>(ws + L.z);
  T* xh = reinterpret_cast<T*>(ws + L.xh);
  T* delta = reinterpret_cast<T*>(ws + L.delta);
  float* Bm = reinterpret_cast<float*>(ws + L.Bm);
  float* Cm = reinterpret_cast<float*>(ws + L.Cm);
  T* g = reinterpret_cast<T*>(ws + L.g);
  const int di = d.d_inner, dm = d.d_model, R = d.dt_rank;

  if constexpr (sizeof(T) == 2) {
    if (decode_fast_path_ok(dm, di, R)) {
      float* partial = reinterpret_cast<float*>(ws + L.partial);
      int* counters = reinterpret_cast<int*>(ws + L.counters);
      const bool tiled = w.in_proj_w_tiles != nullptr;
      const bf16* Win = static_cast<const bf16*>(tiled ? w.in_proj_w_tiles : w.in_proj_w);
      const bf16* Wout = static_cast<const bf16*>(tiled ? w.out_proj_w_tiles : w.out_proj_w);
      for (int32_t b0 = 0; b0 < b; b0 += 64) {
        const int M = b - b0 < 64 ? b - b0 : 64;
        const bf16* ut = u + (int64_t)b0 * dm;
        // without a slot map, the tile's states are the next M rows; with one, the tile's
        // entries of the map index the whole caches
        bf16* ct = rows ? conv_state : conv_state + (int64_t)b0 * di * 3;
        float* st = rows ? ssm_state : ssm_state + (int64_t)b0 * di * 16;
        const int32_t* rt = rows ? rows + b0 : nullptr;
        bf16* ot = out + (int64_t)b0 * dm;
        JM_LAUNCH("dec_in_proj", launch_dec_in_proj(ut, Win, tiled, static_cast<const bf16*>(w.conv_w),
                                                    static_cast<const bf16*>(w.conv_b), ct, rt, xh,
                                                    z, counters, M, dm, di, stream));
        JM_LAUNCH("dec_x_proj", launch_dec_x_proj(xh, static_cast<const bf16*>(w.x_proj_w),
                                                  partial, delta, Bm, Cm, M, di, R, stream));
        if (w.dt_norm_w)
          JM_LAUNCH("dec_inner_norm",
                    launch_inner_rmsnorm<bf16>(delta, Bm, Cm, w.dt_norm_w, w.B_norm_w, w.C_norm_w,
                                               w.norm_eps, M, R, stream));
        jm_status su = step_decode_update<bf16>(d, w, xh, z, delta, Bm, Cm, M, st, rt, g, stream);
        if (su != JM_OK) return su;
        JM_LAUNCH("dec_out_proj", launch_dec_out_proj(g, Wout, tiled, partial, counters, ot, M,
                                                      dm, di, stream));
      }
      return ok();
    }
  }

  jm_status st;
  EpiArgs e = epi_none();
  e.kind = EPI_SPLIT2; e.out0 = x; e.out1 = z; e.split = di;
  JM_LAUNCH("dec_in_proj", gemm<T>(u, dm, static_cast<const T*>(w.in_proj_w), dm, b, 2 * di, dm,
                                   e, stream));
  JM_LAUNCH("dec_conv", launch_decode_conv<T>(x, xh, conv_state, rows,
                                              static_cast<const T*>(w.conv_w),
                                              static_cast<const T*>(w.conv_b), b, di, stream));
  e = epi_none();
  e.kind = EPI_XPROJ; e.out0 = delta; e.outf0 = Bm; e.outf1 = Cm; e.split = R; e.n_state = 16;
  JM_LAUNCH("dec_x_proj", gemm<T>(xh, di, static_cast<const T*>(w.x_proj_w), di, b, R + 32, di, e,
                                  stream));
  if (w.dt_norm_w)
    JM_LAUNCH("dec_inner_norm", launch_inner_rmsnorm<T>(delta, Bm, Cm, w.dt_norm_w, w.B_norm_w,
                                                        w.C_norm_w, w.norm_eps, b, R, stream));
  if ((st = step_decode_update<T>(d, w, xh, z, delta, Bm, Cm, b, ssm_state, rows, g, stream)) !=
      JM_OK)
    return st;
  e = epi_none();
  e.kind = EPI_STORE; e.out0 = out; e.ldo = dm;
  JM_LAUNCH("dec_out_proj", gemm<T>(g, di, static_cast<const T*>(w.out_proj_w), di, b, dm, di, e,
                                    stream));
  return ok();
}


// ---- stage entry points: shared validation ----------------------------------------------
jm_status check_stage(const jm_layer_dims* dims, const jm_layer_weights* w, int64_t n_tok) {
  jm_status st = check_dims(dims);
  if (st != JM_OK) return st;
  if ((st = check_weights(w)) != JM_OK) return st;
  if (n_tok < 1 || n_tok >= ((int64_t)1 << 31))
    return fail(JM_ERR_SHAPE, "total_tokens must be in [1, 2^31) (got %lld)", (long long)n_tok);
  return JM_OK;
}

// Required pointers: non-NULL and 16-byte aligned; optional ones: aligned when given.
jm_status check_ptrs(std::initializer_list<const void*> required,
                     std::initializer_list<const void*> optional = {}) {
  for (const void* p : required) {
    if (!p) return fail(JM_ERR_INVALID_ARG, "a required tensor argument is NULL");
    if (!aligned16(p)) return fail(JM_ERR_ALIGNMENT, "a tensor argument is not 16-byte aligned");
  }
  for (const void* p : optional)
    if (p && !aligned16(p)) return fail(JM_ERR_ALIGNMENT, "a tensor argument is not 16-byte aligned");
  return JM_OK;
}

bool is_bf16(const jm_layer_dims* d) { return d->act_dtype == JM_BF16; }


// ---- state-cache (slot) entry points: validation of the slot arrays ------------------------
// Prefill: init slots in [-1, n_slots); final slots in [-1, n_slots), distinct where >= 0, and
// never another sequence's init slot (a sequence may write back to its own init slot).
jm_status check_prefill_slots(const int32_t* init_dev, const int32_t* init_host,
                              const int32_t* final_dev, const int32_t* final_host, int32_t n_seqs,
                              int32_t n_slots) {
  if ((init_dev == nullptr) != (init_host == nullptr) ||
      (final_dev == nullptr) != (final_host == nullptr))
    return fail(JM_ERR_INVALID_ARG, "slot arrays need both the device and the host copy (or neither)");
  std::vector<int32_t> owner((size_t)n_slots, -1);
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t a = init_host ? init_host[i] : -1;
    const int32_t b = final_host ? final_host[i] : -1;
    if (a < -1 || a >= n_slots || b < -1 || b >= n_slots)
      return fail(JM_ERR_SHAPE, "sequence %d: slot out of range (init %d, final %d, n_slots %d)",
                  i, a, b, n_slots);
    if (b >= 0) {
      if (owner[b] >= 0)
        return fail(JM_ERR_INVALID_ARG, "final slot %d is written by sequences %d and %d", b,
                    owner[b], i);
      owner[b] = i;
    }
  }
  if (init_host && final_host)
    for (int32_t j = 0; j < n_seqs; ++j) {
      const int32_t a = init_host[j];
      if (a >= 0 && owner[a] >= 0 && owner[a] != j)
        return fail(JM_ERR_INVALID_ARG, "slot %d is sequence %d's initial state and sequence "
                    "%d's final state", a, j, owner[a]);
    }
  return JM_OK;
}

jm_status check_decode_slots(const int32_t* dev, const int32_t* host, int32_t batch,
                             int32_t n_slots) {
  if (!dev || !host) return fail(JM_ERR_INVALID_ARG, "slots and slots_host must not be NULL");
  std::vector<char> used((size_t)n_slots, 0);
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t v = host[b];
    if (v < 0 || v >= n_slots)
      return fail(JM_ERR_SHAPE, "batch row %d: slot %d out of range [0, %d)", b, v, n_slots);
    if (used[v]) return fail(JM_ERR_INVALID_ARG, "slot %d appears twice in the batch", v);
    used[v] = 1;
  }
  return JM_OK;
}

size_t slots_tmp_bytes(const jm_layer_dims& d, int32_t n_seqs) {
  return align256((size_t)n_seqs * d.d_inner * 16 * sizeof(float));
}


// ---- backward of the scan step: launch sequence ---------------------------------------------
template <typename T>
jm_status run_scan_backward(const jm_layer_dims& d, const jm_layer_weights& wt, const T* x,
                            const float* dt, const float* B, const float* C, const T* z,
                            const T* dg, const int32_t* cu, int32_t n_seqs, int64_t n_tok,
                            const float* h0, const float* dh_last, float* dx, float* ddt,
                            float* dB, float* dC, float* dz, float* dA_log, float* dD, float* dh0,
                            const ScanBwdLayout& w, hipStream_t stream) {
  const int di = d.d_inner;
  if (w.K > 1) {
    JM_LAUNCH("bwd_fwd_state", launch_scan_chunk_state<T>(x, dt, wt.A_log, B, h0, nullptr, cu,
                                                          w.aggP, w.aggh, n_seqs, n_tok, di,
                                                          w.chunk, w.K - 1, stream));
    JM_LAUNCH("bwd_fwd_carry", launch_scan_chunk_carry(w.aggP, w.aggh, w.carry, di, w.K, stream));
    JM_LAUNCH("bwd_adjoint", launch_scan_bwd_adjoint<T>(dg, z, dt, wt.A_log, C, dh_last, cu, w,
                                                        n_seqs, n_tok, di, stream));
    JM_LAUNCH("bwd_carry", launch_scan_bwd_carry(w, di, stream));
  }
  JM_LAUNCH("bwd_main", launch_scan_bwd_main<T>(x, dt, wt.A_log, B, C, wt.D, z, dg, h0, dh_last,
                                                cu, w, n_seqs, n_tok, di, dx, ddt, dz, dh0,
                                                stream));
  JM_LAUNCH("bwd_reduce", launch_scan_bwd_reduce(w, wt.A_log, n_tok, di, dB, dC, dA_log, dD,
                                                 stream));
  return JM_OK;
}

// ---- decode: shared validation and dispatch ------------------------------------------------
jm_status check_decode_args(const jm_layer_dims* dims, const jm_layer_weights* weights,
                            const void* u, int32_t batch, const void* conv_state,
                            const float* ssm_state, const void* out) {
  jm_status st = check_dims(dims);
  if (st != JM_OK) return st;
  if ((st = check_weights(weights)) != JM_OK) return st;
  if ((st = check_decode_tiles(dims, weights)) != JM_OK) return st;
  if (batch < 0) return fail(JM_ERR_INVALID_ARG, "negative batch");
  if (batch == 0) return JM_OK;
  if (!u || !conv_state || !ssm_state || !out)
    return fail(JM_ERR_INVALID_ARG, "u, conv_state, ssm_state and out must not be NULL");
  const void* ptrs[] = {u, conv_state, ssm_state, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(JM_ERR_ALIGNMENT, "a tensor argument is not 16-byte aligned");
  return JM_OK;
}

jm_status dispatch_decode(const jm_layer_dims& d, const jm_layer_weights& w, const void* u,
                          int32_t batch, void* conv_state, float* ssm_state, void* out, char* ws,
                          hipStream_t s) {
  if (d.act_dtype == JM_BF16)
    return run_decode<bf16>(d, w, static_cast<const bf16*>(u), batch,
                            static_cast<bf16*>(conv_state), ssm_state, static_cast<bf16*>(out),
                            ws, s);
  return run_decode<float>(d, w, static_cast<const float*>(u), batch,
                           static_cast<float*>(conv_state), ssm_state, static_cast<float*>(out),
                           ws, s);
}

// ---- fixed device-side scratch (decode without a caller workspace) -------------------------
// Each GPU holds its own copy of `scratch` at its own address. Host code never passes the
// array's name to a kernel or a copy (on the host that name is only a stand-in): the address
// is looked up once per device, with that device current, and kept.
constexpr size_t kScratchBytes = JM_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int kScratchDevices = 64;
std::atomic<char*> g_scratch_ptr[kScratchDevices];

jm_status scratch_for_current_device(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(JM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchDevices)
    return fail(JM_ERR_UNSUPPORTED, "device %d: the fixed scratch serves devices 0..%d", dev,
                kScratchDevices - 1);
  char* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !addr)
      return fail(JM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    p = static_cast<char*>(addr);
    g_scratch_ptr[dev].store(p, std::memory_order_release);   // same value from any thread
  }
  *out = p;
  return JM_OK;
}

}  // namespace

extern "C" {

const char* jm_status_string(jm_status status) {
  // A C caller may pass any int; read the argument's bits as an int (a value outside the
  // enumerators is not a valid jm_status in C++).
  static_assert(sizeof(jm_status) == sizeof(int), "jm_status is an int");
  int s;
  std::memcpy(&s, &status, sizeof s);
  switch (s) {
    case JM_OK: return "JM_OK";
    case JM_ERR_INVALID_ARG: return "JM_ERR_INVALID_ARG";
    case JM_ERR_SHAPE: return "JM_ERR_SHAPE";
    case JM_ERR_UNSUPPORTED: return "JM_ERR_UNSUPPORTED";
    case JM_ERR_ALIGNMENT: return "JM_ERR_ALIGNMENT";
    case JM_ERR_WORKSPACE: return "JM_ERR_WORKSPACE";
    case JM_ERR_HIP: return "JM_ERR_HIP";
  }
  return "JM_ERR_UNKNOWN";
}

const char* jm_last_error(void) { return g_last_error.c_str(); }

jm_status jm_set_scan_chunk_len(int32_t chunk_len) {
  if (chunk_len < 0) return fail(JM_ERR_INVALID_ARG, "chunk_len must be >= 0");
  g_chunk_override.store(chunk_len, std::memory_order_relaxed);
  return ok();
}

jm_status jm_prefill_workspace_size(const jm_layer_dims* dims, int32_t n_seqs,
                                    int64_t total_tokens, size_t* bytes) {
  jm_status st = check_dims(dims);
  if (st != JM_OK) return st;
  if (!bytes) return fail(JM_ERR_INVALID_ARG, "bytes is NULL");
  if (n_seqs < 0 || total_tokens < 0) return fail(JM_ERR_INVALID_ARG, "negative size");
  if (total_tokens >= ((int64_t)1 << 31)) return fail(JM_ERR_SHAPE, "total_tokens must be < 2^31");
  if (total_tokens == 0) { *bytes = 0; return ok(); }
  int32_t cl, nc;
  plan_chunks(*dims, total_tokens, &cl, &nc);
  *bytes = prefill_layout(*dims, total_tokens, nc).total;
  return ok();
}

jm_status jm_decode_workspace_size(const jm_layer_dims* dims, int32_t batch, size_t* bytes) {
  jm_status st = check_dims(dims);
  if (st != JM_OK) return st;
  if (!bytes) return fail(JM_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 0) return fail(JM_ERR_INVALID_ARG, "negative batch");
  *bytes = batch == 0 ? 0 : decode_layout(*dims, batch).total;
  return ok();
}

jm_status jm_prefill_plan(const jm_layer_dims* dims, const int32_t* cu_host, int32_t n_seqs,
                          int64_t total_tokens, int32_t* chunk_len, int32_t* n_chunks,
                          jm_chunk_segment* segments, int64_t max_segments,
                          int64_t* n_segments) {
  jm_status st = check_dims(dims);
  if (st != JM_OK) return st;
  if (!chunk_len || !n_chunks || !n_segments)
    return fail(JM_ERR_INVALID_ARG, "chunk_len, n_chunks and n_segments must not be NULL");
  if (max_segments > 0 && !segments) return fail(JM_ERR_INVALID_ARG, "segments is NULL");
  if (n_seqs < 1 || total_tokens < 1) return fail(JM_ERR_SHAPE, "need at least one token");
  if (total_tokens >= ((int64_t)1 << 31)) return fail(JM_ERR_SHAPE, "total_tokens must be < 2^31");
  st = check_cu(cu_host, n_seqs, total_tokens);
  if (st != JM_OK) return st;
  plan_chunks(*dims, total_tokens, chunk_len, n_chunks);
  int64_t count = 0;
  int32_t i = 0;
  for (int32_t c = 0; c < *n_chunks; ++c) {
    const int64_t t0 = (int64_t)c * *chunk_len;
    const int64_t t1 = t0 + *chunk_len < total_tokens ? t0 + *chunk_len : total_tokens;
    while (cu_host[i + 1] <= t0) ++i;
    int64_t t = t0;
    int32_t j = i;
    while (t < t1) {
      const int64_t e = cu_host[j + 1] < t1 ? cu_host[j + 1] : t1;
      if (count < max_segments) {
        jm_chunk_segment& s = segments[count];
        s.chunk = c;
        s.seq = j;
        s.begin = (int32_t)t;
        s.end = (int32_t)e;
        s.starts_seq = cu_host[j] == t ? 1 : 0;
        s.ends_seq = cu_host[j + 1] == e ? 1 : 0;
      }
      ++count;
      t = e;
      ++j;
    }
  }
  *n_segments = count;
  return ok();
}

jm_status jamba_mamba_prefill(const jm_layer_dims* dims, const jm_layer_weights* weights,
                              const void* u, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_host, int32_t n_seqs,
                              int64_t total_tokens, const void* init_conv_state,
                              const float* init_ssm_state, void* out, void* final_conv_state,
                              float* final_ssm_state, void* workspace, size_t workspace_bytes,
                              void* stream_ptr) {
  jm_status st = check_dims(dims);
  if (st != JM_OK) return st;
  st = check_weights(weights);
  if (st != JM_OK) return st;
  if (n_seqs < 0 || total_tokens < 0) return fail(JM_ERR_INVALID_ARG, "negative size");
  if (total_tokens >= ((int64_t)1 << 31)) return fail(JM_ERR_SHAPE, "total_tokens must be < 2^31");
  if (n_seqs == 0 || total_tokens == 0) {
    if (n_seqs != 0 || total_tokens != 0)
      return fail(JM_ERR_SHAPE, "n_seqs = %d with total_tokens = %lld", n_seqs,
                  (long long)total_tokens);
    return ok();   // nothing to do
  }
  if (!u || !out || !cu_seqlens)
    return fail(JM_ERR_INVALID_ARG, "u, out and cu_seqlens must not be NULL");
  st = check_cu(cu_seqlens_host, n_seqs, total_tokens);
  if (st != JM_OK) return st;
  const void* ptrs[] = {u, out, init_conv_state, init_ssm_state, final_conv_state,
                        final_ssm_state, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(JM_ERR_ALIGNMENT, "a tensor argument is not 16-byte aligned");
  if (init_ssm_state && final_ssm_state) {
    const char* a = reinterpret_cast<const char*>(init_ssm_state);
    const char* b = reinterpret_cast<const char*>(final_ssm_state);
    const size_t bytes = (size_t)n_seqs * dims->d_inner * 16 * sizeof(float);
    if (a < b + bytes && b < a + bytes)
      return fail(JM_ERR_INVALID_ARG, "init_ssm_state and final_ssm_state must not overlap");
  }
  int32_t cl, nc;
  plan_chunks(*dims, total_tokens, &cl, &nc);
  const size_t need = prefill_layout(*dims, total_tokens, nc).total;
  if (!workspace || workspace_bytes < need)
    return fail(JM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  hipStream_t s = static_cast<hipStream_t>(stream_ptr);
  char* ws = static_cast<char*>(workspace);
  if (dims->act_dtype == JM_BF16)
    return run_prefill<bf16>(*dims, *weights, static_cast<const bf16*>(u), cu_seqlens, n_seqs,
                             total_tokens, static_cast<const bf16*>(init_conv_state),
                             init_ssm_state, static_cast<bf16*>(out),
                             static_cast<bf16*>(final_conv_state), final_ssm_state, ws, cl, nc, s);
  return run_prefill<float>(*dims, *weights, static_cast<const float*>(u), cu_seqlens, n_seqs,
                            total_tokens, static_cast<const float*>(init_conv_state),
                            init_ssm_state, static_cast<float*>(out),
                            static_cast<float*>(final_conv_state), final_ssm_state, ws, cl, nc, s);
}

jm_status jamba_mamba_decode_step(const jm_layer_dims* dims, const jm_layer_weights* weights,
                                  const void* u, int32_t batch, void* conv_state,
                                  float* ssm_state, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream_ptr) {
  jm_status st = check_decode_args(dims, weights, u, batch, conv_state, ssm_state, out);
  if (st != JM_OK || batch == 0) return st == JM_OK ? ok() : st;
  if (workspace && !aligned16(workspace))
    return fail(JM_ERR_ALIGNMENT, "a tensor argument is not 16-byte aligned");
  const size_t need = decode_layout(*dims, batch).total;
  if (!workspace || workspace_bytes < need)
    return fail(JM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  return dispatch_decode(*dims, *weights, u, batch, conv_state, ssm_state, out,
                         static_cast<char*>(workspace), static_cast<hipStream_t>(stream_ptr));
}

jm_status jamba_mamba_decode_step_noalloc(const jm_layer_dims* dims,
                                          const jm_layer_weights* weights, const void* u,
                                          int32_t batch, void* conv_state, float* ssm_state,
                                          void* out, void* stream_ptr) {
  jm_status st = check_decode_args(dims, weights, u, batch, conv_state, ssm_state, out);
  if (st != JM_OK || batch == 0) return st == JM_OK ? ok() : st;
  const size_t need = decode_layout(*dims, batch).total;
  if (need > kScratchBytes)
    return fail(JM_ERR_WORKSPACE, "batch %d needs %zu bytes of scratch; the fixed scratch holds "
                "%zu", batch, need, kScratchBytes);
  char* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != JM_OK) return st;
  return dispatch_decode(*dims, *weights, u, batch, conv_state, ssm_state, out, ws,
                         static_cast<hipStream_t>(stream_ptr));
}

jm_status jm_tile_decode_weights(const jm_layer_dims* dims, const void* in_proj_w,
                                 const void* out_proj_w, void* in_proj_w_tiles,
                                 void* out_proj_w_tiles, void* stream_ptr) {
  jm_status st = check_dims(dims);
  if (st != JM_OK) return st;
  if (!decode_tiles_apply(*dims))
    return fail(JM_ERR_UNSUPPORTED, "decode tiles are read by the bf16 decode kernels only "
                "(d_model %% 256 == 0, d_inner %% 1024 == 0, dt_rank 128 or 256)");
  if (!in_proj_w || !out_proj_w || !in_proj_w_tiles || !out_proj_w_tiles)
    return fail(JM_ERR_INVALID_ARG, "weights and tiles must not be NULL");
  const void* ptrs[] = {in_proj_w, out_proj_w, in_proj_w_tiles, out_proj_w_tiles};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(JM_ERR_ALIGNMENT, "a tensor argument is not 16-byte aligned");
  const int dm = dims->d_model, di = dims->d_inner;
  const size_t in_bytes = (size_t)2 * di * dm * 2, out_bytes = (size_t)dm * di * 2;
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const char *pa = static_cast<const char*>(a), *pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
  };
  if (overlap(in_proj_w_tiles, in_bytes, in_proj_w, in_bytes) ||
      overlap(in_proj_w_tiles, in_bytes, out_proj_w, out_bytes) ||
      overlap(out_proj_w_tiles, out_bytes, in_proj_w, in_bytes) ||
      overlap(out_proj_w_tiles, out_bytes, out_proj_w, out_bytes) ||
      overlap(in_proj_w_tiles, in_bytes, out_proj_w_tiles, out_bytes))
    return fail(JM_ERR_INVALID_ARG, "tiles overlap each other or the weights");
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  JM_LAUNCH("tile_in_proj", launch_tile_weights(static_cast<const bf16*>(in_proj_w),
                                                static_cast<bf16*>(in_proj_w_tiles), 2 * di, dm,
                                                stream));
  JM_LAUNCH("tile_out_proj", launch_tile_weights(static_cast<const bf16*>(out_proj_w),
                                                 static_cast<bf16*>(out_proj_w_tiles), dm, di,
                                                 stream));
  return ok();
}

// ---- state-cache (slot) entry points -----------------------------------------------------
jm_status jm_prefill_slots_workspace_size(const jm_layer_dims* dims, int32_t n_seqs,
                                          int64_t total_tokens, size_t* bytes) {
  jm_status st = jm_prefill_workspace_size(dims, n_seqs, total_tokens, bytes);
  if (st != JM_OK) return st;
  if (total_tokens > 0) *bytes += slots_tmp_bytes(*dims, n_seqs);
  return ok();
}

jm_status jamba_mamba_prefill_slots(const jm_layer_dims* dims, const jm_layer_weights* weights,
                                    const void* u, const int32_t* cu_seqlens,
                                    const int32_t* cu_seqlens_host, int32_t n_seqs,
                                    int64_t total_tokens, const int32_t* init_slots,
                                    const int32_t* init_slots_host, const int32_t* final_slots,
                                    const int32_t* final_slots_host, void* conv_cache,
                                    float* ssm_cache, int32_t n_slots, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream_ptr) {
  jm_status st = check_dims(dims);
  if (st != JM_OK || (st = check_weights(weights)) != JM_OK) return st;
  if (n_seqs < 0 || total_tokens < 0 || n_slots < 1)
    return fail(JM_ERR_INVALID_ARG, "negative size or n_slots < 1");
  if (total_tokens >= ((int64_t)1 << 31)) return fail(JM_ERR_SHAPE, "total_tokens must be < 2^31");
  if (n_seqs == 0 || total_tokens == 0) {
    if (n_seqs != 0 || total_tokens != 0)
      return fail(JM_ERR_SHAPE, "n_seqs = %d with total_tokens = %lld", n_seqs,
                  (long long)total_tokens);
    return ok();
  }
  if (!cu_seqlens) return fail(JM_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if ((st = check_cu(cu_seqlens_host, n_seqs, total_tokens)) != JM_OK) return st;
  if ((st = check_ptrs({u, out, conv_cache, ssm_cache}, {workspace})) != JM_OK) return st;
  if ((st = check_prefill_slots(init_slots, init_slots_host, final_slots, final_slots_host,
                                n_seqs, n_slots)) != JM_OK)
    return st;
  int32_t cl, nc;
  plan_chunks(*dims, total_tokens, &cl, &nc);
  const size_t base = prefill_layout(*dims, total_tokens, nc).total;
  const size_t need = base + slots_tmp_bytes(*dims, n_seqs);
  if (!workspace || workspace_bytes < need)
    return fail(JM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  hipStream_t s = static_cast<hipStream_t>(stream_ptr);
  char* ws = static_cast<char*>(workspace);
  float* tmp = final_slots ? reinterpret_cast<float*>(ws + base) : nullptr;
  const float* init_ssm = init_slots ? ssm_cache : nullptr;
  if (dims->act_dtype == JM_BF16) {
    bf16* cc = static_cast<bf16*>(conv_cache);
    return run_prefill<bf16>(*dims, *weights, static_cast<const bf16*>(u), cu_seqlens, n_seqs,
                             total_tokens, init_slots ? cc : nullptr, init_ssm,
                             static_cast<bf16*>(out), final_slots ? cc : nullptr, tmp, ws, cl, nc,
                             s, init_slots, final_slots, ssm_cache);
  }
  float* cc = static_cast<float*>(conv_cache);
  return run_prefill<float>(*dims, *weights, static_cast<const float*>(u), cu_seqlens, n_seqs,
                            total_tokens, init_slots ? cc : nullptr, init_ssm,
                            static_cast<float*>(out), final_slots ? cc : nullptr, tmp, ws, cl, nc,
                            s, init_slots, final_slots, ssm_cache);
}

jm_status jamba_mamba_decode_step_slots(const jm_layer_dims* dims,
                                        const jm_layer_weights* weights, const void* u,
                                        int32_t batch, const int32_t* slots,
                                        const int32_t* slots_host, void* conv_cache,
                                        float* ssm_cache, int32_t n_slots, void* out,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream_ptr) {
  jm_status st = check_dims(dims);
  if (st != JM_OK || (st = check_weights(weights)) != JM_OK) return st;
  if ((st = check_decode_tiles(dims, weights)) != JM_OK) return st;
  if (batch < 0 || n_slots < 1) return fail(JM_ERR_INVALID_ARG, "negative batch or n_slots < 1");
  if (batch == 0) return ok();
  if ((st = check_ptrs({u, conv_cache, ssm_cache, out}, {workspace})) != JM_OK) return st;
  if ((st = check_decode_slots(slots, slots_host, batch, n_slots)) != JM_OK) return st;
  const size_t need = decode_layout(*dims, batch).total;
  if (!workspace || workspace_bytes < need)
    return fail(JM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  hipStream_t s = static_cast<hipStream_t>(stream_ptr);
  char* ws = static_cast<char*>(workspace);
  if (dims->act_dtype == JM_BF16)
    return run_decode<bf16>(*dims, *weights, static_cast<const bf16*>(u), batch,
                            static_cast<bf16*>(conv_cache), ssm_cache, static_cast<bf16*>(out),
                            ws, s, slots);
  return run_decode<float>(*dims, *weights, static_cast<const float*>(u), batch,
                           static_cast<float*>(conv_cache), ssm_cache, static_cast<float*>(out),
                           ws, s, slots);
}

// ---- stage entry points ------------------------------------------------------------------
jm_status jm_stage_in_proj(const jm_layer_dims* dims, const jm_layer_weights* weights,
                           const void* u, int64_t total_tokens, void* x, void* z, void* stream) {
  jm_status st = check_stage(dims, weights, total_tokens);
  if (st != JM_OK || (st = check_ptrs({u, x, z})) != JM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = is_bf16(dims) ? step_in_proj<bf16>(*dims, *weights, static_cast<const bf16*>(u),
                                         total_tokens, static_cast<bf16*>(x),
                                         static_cast<bf16*>(z), s)
                     : step_in_proj<float>(*dims, *weights, static_cast<const float*>(u),
                                           total_tokens, static_cast<float*>(x),
                                           static_cast<float*>(z), s);
  return st == JM_OK ? ok() : st;
}

jm_status jm_stage_conv(const jm_layer_dims* dims, const jm_layer_weights* weights,
                        const void* x, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                        int32_t n_seqs, int64_t total_tokens, const void* init_conv_state,
                        void* x_hat, void* final_conv_state, void* stream) {
  jm_status st = check_stage(dims, weights, total_tokens);
  if (st != JM_OK) return st;
  if (n_seqs < 1) return fail(JM_ERR_SHAPE, "n_seqs must be >= 1");
  if (!cu_seqlens) return fail(JM_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if ((st = check_cu(cu_seqlens_host, n_seqs, total_tokens)) != JM_OK) return st;
  if ((st = check_ptrs({x, x_hat}, {init_conv_state, final_conv_state})) != JM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = is_bf16(dims)
           ? step_conv<bf16>(*dims, *weights, static_cast<const bf16*>(x), cu_seqlens, n_seqs,
                             total_tokens, static_cast<const bf16*>(init_conv_state),
                             static_cast<bf16*>(x_hat), static_cast<bf16*>(final_conv_state), s)
           : step_conv<float>(*dims, *weights, static_cast<const float*>(x), cu_seqlens, n_seqs,
                              total_tokens, static_cast<const float*>(init_conv_state),
                              static_cast<float*>(x_hat), static_cast<float*>(final_conv_state),
                              s);
  return st == JM_OK ? ok() : st;
}

jm_status jm_stage_x_proj(const jm_layer_dims* dims, const jm_layer_weights* weights,
                          const void* x_hat, int64_t total_tokens, void* delta, float* B,
                          float* C, void* stream) {
  jm_status st = check_stage(dims, weights, total_tokens);
  if (st != JM_OK || (st = check_ptrs({x_hat, delta, B, C})) != JM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = is_bf16(dims) ? step_x_proj<bf16>(*dims, *weights, static_cast<const bf16*>(x_hat),
                                        total_tokens, static_cast<bf16*>(delta), B, C, s)
                     : step_x_proj<float>(*dims, *weights, static_cast<const float*>(x_hat),
                                          total_tokens, static_cast<float*>(delta), B, C, s);
  return st == JM_OK ? ok() : st;
}

jm_status jm_stage_dt_proj(const jm_layer_dims* dims, const jm_layer_weights* weights,
                           const void* delta, int64_t total_tokens, float* dt, void* stream) {
  jm_status st = check_stage(dims, weights, total_tokens);
  if (st != JM_OK || (st = check_ptrs({delta, dt})) != JM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = is_bf16(dims) ? step_dt_proj<bf16>(*dims, *weights, static_cast<const bf16*>(delta),
                                         total_tokens, dt, s)
                     : step_dt_proj<float>(*dims, *weights, static_cast<const float*>(delta),
                                           total_tokens, dt, s);
  return st == JM_OK ? ok() : st;
}

jm_status jm_stage_scan_workspace_size(const jm_layer_dims* dims, int64_t total_tokens,
                                       size_t* bytes) {
  jm_status st = check_dims(dims);
  if (st != JM_OK) return st;
  if (!bytes) return fail(JM_ERR_INVALID_ARG, "bytes is NULL");
  if (total_tokens < 1 || total_tokens >= ((int64_t)1 << 31))
    return fail(JM_ERR_SHAPE, "total_tokens must be in [1, 2^31)");
  int32_t cl, nc;
  plan_chunks(*dims, total_tokens, &cl, &nc);
  *bytes = 3 * scan_agg_bytes(*dims, nc);
  return ok();
}

jm_status jm_stage_scan(const jm_layer_dims* dims, const jm_layer_weights* weights,
                        const void* x_hat, const float* dt, const float* B, const float* C,
                        const void* z, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                        int32_t n_seqs, int64_t total_tokens, const float* init_ssm_state,
                        void* g, float* final_ssm_state, void* workspace,
                        size_t workspace_bytes, void* stream) {
  jm_status st = check_stage(dims, weights, total_tokens);
  if (st != JM_OK) return st;
  if (n_seqs < 1) return fail(JM_ERR_SHAPE, "n_seqs must be >= 1");
  if (!cu_seqlens) return fail(JM_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if ((st = check_cu(cu_seqlens_host, n_seqs, total_tokens)) != JM_OK) return st;
  if ((st = check_ptrs({x_hat, dt, B, C, z, g}, {init_ssm_state, final_ssm_state, workspace})) !=
      JM_OK)
    return st;
  if (init_ssm_state && final_ssm_state) {
    const char* a = reinterpret_cast<const char*>(init_ssm_state);
    const char* b = reinterpret_cast<const char*>(final_ssm_state);
    const size_t n = (size_t)n_seqs * dims->d_inner * 16 * sizeof(float);
    if (a < b + n && b < a + n)
      return fail(JM_ERR_INVALID_ARG, "init_ssm_state and final_ssm_state must not overlap");
  }
  int32_t cl, nc;
  plan_chunks(*dims, total_tokens, &cl, &nc);
  const size_t need = 3 * scan_agg_bytes(*dims, nc);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(JM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  st = is_bf16(dims)
           ? step_scan<bf16>(*dims, *weights, static_cast<const bf16*>(x_hat), dt, B, C,
                             static_cast<const bf16*>(z), cu_seqlens, n_seqs, total_tokens,
                             init_ssm_state, static_cast<bf16*>(g), final_ssm_state, ws, cl, nc, s)
           : step_scan<float>(*dims, *weights, static_cast<const float*>(x_hat), dt, B, C,
                              static_cast<const float*>(z), cu_seqlens, n_seqs, total_tokens,
                              init_ssm_state, static_cast<float*>(g), final_ssm_state, ws, cl, nc,
                              s);
  return st == JM_OK ? ok() : st;
}

jm_status jm_stage_out_proj(const jm_layer_dims* dims, const jm_layer_weights* weights,
                            const void* g, int64_t total_tokens, void* out, void* stream) {
  jm_status st = check_stage(dims, weights, total_tokens);
  if (st != JM_OK || (st = check_ptrs({g, out})) != JM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = is_bf16(dims) ? step_out_proj<bf16>(*dims, *weights, static_cast<const bf16*>(g),
                                          total_tokens, static_cast<bf16*>(out), s)
                     : step_out_proj<float>(*dims, *weights, static_cast<const float*>(g),
                                            total_tokens, static_cast<float*>(out), s);
  return st == JM_OK ? ok() : st;
}

jm_status jm_stage_decode_update(const jm_layer_dims* dims, const jm_layer_weights* weights,
                                 const void* x_hat, const void* z, const void* delta,
                                 const float* B, const float* C, int32_t batch,
                                 const int32_t* slots, const int32_t* slots_host, int32_t n_slots,
                                 float* ssm_state, void* g, void* stream) {
  jm_status st = check_dims(dims);
  if (st != JM_OK || (st = check_weights(weights)) != JM_OK) return st;
  if (batch < 0) return fail(JM_ERR_INVALID_ARG, "negative batch");
  if (batch == 0) return ok();
  if ((st = check_ptrs({x_hat, z, delta, B, C, ssm_state, g})) != JM_OK) return st;
  if (slots || slots_host) {
    if (n_slots < 1) return fail(JM_ERR_INVALID_ARG, "n_slots < 1");
    if ((st = check_decode_slots(slots, slots_host, batch, n_slots)) != JM_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = is_bf16(dims)
           ? step_decode_update<bf16>(*dims, *weights, static_cast<const bf16*>(x_hat),
                                      static_cast<const bf16*>(z), static_cast<const bf16*>(delta),
                                      B, C, batch, ssm_state, slots, static_cast<bf16*>(g), s)
           : step_decode_update<float>(*dims, *weights, static_cast<const float*>(x_hat),
                                       static_cast<const float*>(z),
                                       static_cast<const float*>(delta), B, C, batch, ssm_state,
                                       slots, static_cast<float*>(g), s);
  return st == JM_OK ? ok() : st;
}

// ---- backward of the scan step (training) -------------------------------------------------
jm_status jm_scan_backward_workspace_size(const jm_layer_dims* dims, int64_t total_tokens,
                                          size_t* bytes) {
  jm_status st = check_dims(dims);
  if (st != JM_OK) return st;
  if (!bytes) return fail(JM_ERR_INVALID_ARG, "bytes is NULL");
  if (total_tokens < 0 || total_tokens >= ((int64_t)1 << 31))
    return fail(JM_ERR_SHAPE, "total_tokens must be in [0, 2^31)");
  *bytes = total_tokens == 0 ? 0
                             : scan_backward_workspace_floats(total_tokens, dims->d_inner) * 4;
  return ok();
}

jm_status jamba_mamba_scan_backward(const jm_layer_dims* dims, const jm_layer_weights* weights,
                                    const void* x_hat, const float* dt, const float* B,
                                    const float* C, const void* z, const void* dg,
                                    const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                    int32_t n_seqs, int64_t total_tokens,
                                    const float* init_ssm_state, const float* d_final_ssm_state,
                                    float* dx_hat, float* ddt, float* dB, float* dC, float* dz,
                                    float* dA_log, float* dD, float* d_init_ssm_state,
                                    void* workspace, size_t workspace_bytes, void* stream_ptr) {
  jm_status st = check_stage(dims, weights, total_tokens);
  if (st != JM_OK) return st;
  if (n_seqs < 1) return fail(JM_ERR_SHAPE, "n_seqs must be >= 1");
  if (!cu_seqlens) return fail(JM_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if ((st = check_cu(cu_seqlens_host, n_seqs, total_tokens)) != JM_OK) return st;
  if ((st = check_ptrs({x_hat, dt, B, C, z, dg, dx_hat, ddt, dB, dC, dz, dA_log, dD, workspace},
                       {init_ssm_state, d_final_ssm_state, d_init_ssm_state})) != JM_OK)
    return st;
  const size_t need = scan_backward_workspace_floats(total_tokens, dims->d_inner) * 4;
  if (workspace_bytes < need)
    return fail(JM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const ScanBwdLayout w = scan_backward_layout(static_cast<float*>(workspace), total_tokens,
                                               dims->d_inner);
  if (dims->act_dtype == JM_BF16)
    st = run_scan_backward<bf16>(*dims, *weights, static_cast<const bf16*>(x_hat), dt, B, C,
                                 static_cast<const bf16*>(z), static_cast<const bf16*>(dg),
                                 cu_seqlens, n_seqs, total_tokens, init_ssm_state,
                                 d_final_ssm_state, dx_hat, ddt, dB, dC, dz, dA_log, dD,
                                 d_init_ssm_state, w, stream);
  else
    st = run_scan_backward<float>(*dims, *weights, static_cast<const float*>(x_hat), dt, B, C,
                                  static_cast<const float*>(z), static_cast<const float*>(dg),
                                  cu_seqlens, n_seqs, total_tokens, init_ssm_state,
                                  d_final_ssm_state, dx_hat, ddt, dB, dC, dz, dA_log, dD,
                                  d_init_ssm_state, w, stream);
  return st == JM_OK ? ok() : st;
}

jm_status jm_profile_enable(int32_t enable) {
  g_prof = enable != 0;
  return ok();
}

jm_status jm_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_recs) {
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return ok();
}

jm_status jm_profile_read(jm_kernel_time* out, int32_t max_entries, int32_t* n_entries) {
  if (!n_entries || (max_entries > 0 && !out))
    return fail(JM_ERR_INVALID_ARG, "out and n_entries must not be NULL");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::vector<jm_kernel_time> agg;
  for (auto& r : g_recs) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return fail(JM_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return fail(JM_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
    jm_kernel_time* slot = nullptr;
    for (auto& a : agg)
      if (std::strncmp(a.name, r.name, sizeof(a.name)) == 0) slot = &a;
    if (!slot) {
      jm_kernel_time t;
      std::memset(&t, 0, sizeof(t));
      std::strncpy(t.name, r.name, sizeof(t.name) - 1);
      agg.push_back(t);
      slot = &agg.back();
    }
    slot->launches += 1;
    slot->total_ms += ms;
  }
  *n_entries = (int32_t)agg.size();
  for (int32_t i = 0; i < (int32_t)agg.size() && i < max_entries; ++i) out[i] = agg[i];
  return ok();
}

}  // extern "C"
