// C ABI of the decoder-block library: host-side validation, workspace sizing
// and kernel launches on the caller's stream.  Every check runs before the
// first launch, so an error return leaves every buffer untouched.
#include "../../include/llama_block.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "attention.hpp"
#include "gemm.hpp"
#include "misc.hpp"
#include "sample.hpp"

using llama::bf16;

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline size_t elem_size(llama_dtype dt) { return dt == LLAMA_BF16 ? 2 : 4; }
inline bool dtype_ok(int dt) { return dt == LLAMA_F32 || dt == LLAMA_BF16; }
inline int hip_status(hipError_t e) { return e == hipSuccess ? LLAMA_OK : LLAMA_ERR_HIP; }

// Alignment the kernels rely on: tensors are read and written with 16-byte
// vectors and global -> LDS DMA of 16-byte chunks; int32 id/position arrays and
// per-row floats are read element-wise.  A null pointer counts as aligned (the
// null checks are separate).
inline bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }
inline bool al4(const void* p) { return ((uintptr_t)p & 3) == 0; }
template <typename... P>
inline bool all_al16(const P*... p) {
  return (al16(p) && ...);
}

struct Dims {
  int D, H, Hkv, d, F, n_rep;
};

// Validates the model arguments that every call needs; fills `o`.
int model_dims(const llama_model_args* a, llama_dtype dt, Dims* o) {
  if (!a || !dtype_ok(dt)) return LLAMA_ERR_INVALID_ARG;
  if (a->dim <= 0 || a->n_heads <= 0 || a->multiple_of <= 0) return LLAMA_ERR_INVALID_ARG;
  if (a->max_batch_size <= 0 || a->max_seq_len <= 0) return LLAMA_ERR_INVALID_ARG;
  if (!(a->norm_eps >= 0.f) || !(a->rope_theta > 0.f)) return LLAMA_ERR_INVALID_ARG;
  const int H = a->n_heads;
  const int Hkv = a->n_kv_heads <= 0 ? H : a->n_kv_heads;
  if (a->dim % H != 0 || H % Hkv != 0) return LLAMA_ERR_INVALID_ARG;
  const int d = a->dim / H;
  if (d % 2 != 0) return LLAMA_ERR_INVALID_ARG;
  // one sequence's cache rows are addressed with 32-bit element offsets
  if ((int64_t)a->max_seq_len * Hkv * d > INT32_MAX) return LLAMA_ERR_UNSUPPORTED;
  int32_t F = 0;
  int rc = llama_ffn_hidden_dim(a, &F);
  if (rc != LLAMA_OK) return rc;
  if (dt == LLAMA_BF16) {
    if (d != 64 && d != 128) return LLAMA_ERR_UNSUPPORTED;
    if (a->dim % 8 != 0 || F % 8 != 0) return LLAMA_ERR_INVALID_ARG;
  } else {
    if (d != 32 && d != 64 && d != 128) return LLAMA_ERR_UNSUPPORTED;
    if (a->dim % 4 != 0 || F % 4 != 0) return LLAMA_ERR_INVALID_ARG;
  }
  *o = Dims{a->dim, H, Hkv, d, F, H / Hkv};
  return LLAMA_OK;
}

int call_shape(const llama_model_args* a, int32_t bsz, int32_t seqlen, int32_t start_pos) {
  if (bsz < 1 || bsz > a->max_batch_size) return LLAMA_ERR_INVALID_ARG;
  if (seqlen < 1 || start_pos < 0) return LLAMA_ERR_INVALID_ARG;
  if ((int64_t)start_pos + seqlen > a->max_seq_len) return LLAMA_ERR_INVALID_ARG;
  return LLAMA_OK;
}

// split-K partial buffer (floats) for one GEMM
size_t gemm_partial_floats(int M, int N, int K, bool dual, llama_dtype dt) {
  const int s = llama::gemm_pick_splits(M, N, K, dual, dt == LLAMA_BF16);
  return s > 1 ? (size_t)s * M * N * (dual ? 2 : 1) : 0;
}

size_t decode_partial_floats(const Dims& g, int bsz, int T, llama_dtype dt) {
  if (dt != LLAMA_BF16) return 0;
  const int ns = llama::attn_decode_splits(bsz, g.H, g.Hkv, T);
  return ns > 1 ? (size_t)bsz * g.H * ns * (g.d + 2) : 0;
}

struct BlockWs {
  size_t xn, q, o, h, hn, g, r1, r2, partial, total;
};

BlockWs block_ws_layout(const Dims& g, int bsz, int seqlen, int start_pos, llama_dtype dt) {
  const size_t es = elem_size(dt);
  const int64_t N = (int64_t)bsz * seqlen;
  BlockWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align_up(bytes);
    return at;
  };
  w.xn = take(N * g.D * es);
  w.q = take(N * g.H * g.d * es);
  w.o = take(N * g.H * g.d * es);
  w.h = take(N * g.D * es);
  w.hn = take(N * g.D * es);
  w.g = take(N * g.F * es);
  w.r1 = take(N * sizeof(float));
  w.r2 = take(N * sizeof(float));
  size_t pf = 0;
  const int M = (int)N;
  pf = std::max(pf, gemm_partial_floats(M, (g.H + 2 * g.Hkv) * g.d, g.D, false, dt));
  pf = std::max(pf, gemm_partial_floats(M, g.D, g.H * g.d, false, dt));
  pf = std::max(pf, gemm_partial_floats(M, g.F, g.D, true, dt));
  pf = std::max(pf, gemm_partial_floats(M, g.D, g.F, false, dt));
  if (seqlen == 1) pf = std::max(pf, decode_partial_floats(g, bsz, start_pos + 1, dt));
  w.partial = take(pf * sizeof(float));
  w.total = off;
  return w;
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + bn && pb < pa + an;
}

template <typename T>
int block_forward_t(const Dims& g, const llama_model_args* a, const llama_block_weights* w, T* ck, T* cv,
                    const float* freqs, const T* x, T* out, int bsz, int seqlen, int start_pos, char* ws,
                    const BlockWs& L, hipStream_t st, hipEvent_t* ev, const int32_t* pos_dev) {
  // pos_dev (optional, one-token bf16 calls): the position is read on the device,
  // start_pos is then its upper bound
  // ev (optional): ev[0] before the first stage, ev[i] after stage i (i = 1..7)
  auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], st) : hipSuccess; };
  if (mark(0) != hipSuccess) return LLAMA_ERR_HIP;
  const int M = bsz * seqlen;
  T* xn = (T*)(ws + L.xn);
  T* q = (T*)(ws + L.q);
  T* o = (T*)(ws + L.o);
  T* h = (T*)(ws + L.h);
  T* hn = (T*)(ws + L.hn);
  T* gt = (T*)(ws + L.g);
  float* r1 = (float*)(ws + L.r1);
  float* r2 = (float*)(ws + L.r2);
  float* part = (float*)(ws + L.partial);
  const bool bf = sizeof(T) == 2;
  const llama_dtype dt = bf ? LLAMA_BF16 : LLAMA_F32;
  const int nq = g.H * g.d, nkv = g.Hkv * g.d;
  hipError_t e = hipSuccess;
  // h = x + wo(attention(RMSNorm(x))).  RMSNorm(x) W^T is computed as
  // rsqrt(mean(x^2) + eps) * ((x * g) W^T): the row factor is applied to the fp32
  // accumulators, so the normalised activation is never rounded to bf16.
  // Up to four tokens: the weight-streaming kernels take the un-normalised
  // rows and apply the same factor themselves, so no normalisation pass runs.
  const bool fused_norm = llama::gemv_fits<T>(M, nq + 2 * nkv, g.D, g.D) && llama::gemv_fits<T>(M, g.F, g.D, g.D);
  if (!fused_norm) e = llama::rmsnorm<T>(x, g.D, (const T*)w->attention_norm, xn, M, g.D, a->norm_eps, st, r1);
  if (e != hipSuccess || mark(1) != hipSuccess) return LLAMA_ERR_HIP;
  {
    llama::WeightRows<T> wr{(const T*)w->wq, (const T*)w->wk, (const T*)w->wv, nq, nq + nkv};
    const int N = nq + 2 * nkv;
    if (fused_norm) {
      llama::EpiQKV<T> epi{q, ck, cv, freqs, seqlen, start_pos, a->max_seq_len, nq, nkv, g.d, nullptr, pos_dev};
      e = llama::gemv_launch<T>(x, g.D, wr, M, N, g.D, (const T*)w->attention_norm, a->norm_eps, epi, st);
    }
    if (!fused_norm) {
      llama::EpiQKV<T> epi{q, ck, cv, freqs, seqlen, start_pos, a->max_seq_len, nq, nkv, g.d, r1, pos_dev};
      e = llama::gemm_launch<T>(xn, g.D, wr, M, N, g.D, epi, llama::gemm_pick_splits(M, N, g.D, false, bf), part, st);
    }
    if (e != hipSuccess || mark(2) != hipSuccess) return LLAMA_ERR_HIP;
  }
  llama::AttnShape sh{bsz, seqlen, start_pos, g.H, g.Hkv, g.d, a->max_seq_len};
  if (seqlen == 1)
    e = llama::attn_decode<T>(q, ck, cv, o, sh, part, st, pos_dev);
  else
    e = llama::attn_prefill<T>(q, ck, cv, o, sh, st);
  if (e != hipSuccess || mark(3) != hipSuccess) return LLAMA_ERR_HIP;
  // 5..64 tokens in bf16 with wo split over K: the split reduction also applies
  // the residual and computes ffn_norm's x * g and row factor (one pass over h)
  const bool wo_norm = bf && !fused_norm && llama::gemm_residual_norm_fits(M, g.D, nq, nq);
  {
    llama::WeightRows<T> wr{(const T*)w->wo, nullptr, nullptr, g.D, g.D};
    llama::EpiResidual<T> epi{h, x, g.D};
    if constexpr (sizeof(T) == 2) {
      if (wo_norm)
        e = llama::gemm_residual_norm_launch(o, nq, (const T*)w->wo, M, g.D, nq, h, x, (const T*)w->ffn_norm, hn, r2,
                                             a->norm_eps, part, st);
    }
    if (!wo_norm)
      e = llama::gemm_launch<T>(o, nq, wr, M, g.D, nq, epi, llama::gemm_pick_splits(M, g.D, nq, false, bf), part, st);
    if (e != hipSuccess || mark(4) != hipSuccess) return LLAMA_ERR_HIP;
  }
  // out = h + w2(silu(w1 hn) * w3 hn), hn = RMSNorm(h)
  if (!fused_norm && !wo_norm) e = llama::rmsnorm<T>(h, g.D, (const T*)w->ffn_norm, hn, M, g.D, a->norm_eps, st, r2);
  if (e != hipSuccess || mark(5) != hipSuccess) return LLAMA_ERR_HIP;
  {
    if (fused_norm) {
      llama::EpiSwiGLU<T> epi{gt, g.F, nullptr};
      e = llama::gemv_dual_launch<T>(h, g.D, (const T*)w->w1, (const T*)w->w3, M, g.F, g.D, (const T*)w->ffn_norm,
                                     a->norm_eps, epi, st);
    }
    if (!fused_norm) {
      llama::EpiSwiGLU<T> epi{gt, g.F, r2};
      e = llama::gemm_dual_launch<T>(hn, g.D, (const T*)w->w1, (const T*)w->w3, M, g.F, g.D, epi,
                                     llama::gemm_pick_splits(M, g.F, g.D, true, bf), part, st);
    }
    if (e != hipSuccess || mark(6) != hipSuccess) return LLAMA_ERR_HIP;
  }
  {
    llama::WeightRows<T> wr{(const T*)w->w2, nullptr, nullptr, g.D, g.D};
    llama::EpiResidual<T> epi{out, h, g.D};
    e = llama::gemm_launch<T>(gt, g.F, wr, M, g.D, g.F, epi, llama::gemm_pick_splits(M, g.D, g.F, false, bf), part,
                              st);
    if (e != hipSuccess || mark(7) != hipSuccess) return LLAMA_ERR_HIP;
  }
  (void)dt;
  return LLAMA_OK;
}

}  // namespace

extern "C" {

const char* llama_status_str(int s) {
  switch (s) {
    case LLAMA_OK: return "ok";
    case LLAMA_ERR_INVALID_ARG: return "invalid argument";
    case LLAMA_ERR_UNSUPPORTED: return "unsupported dtype/head_dim combination";
    case LLAMA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case LLAMA_ERR_HIP: return "HIP launch error";
    case LLAMA_ERR_SCRATCH_TOO_SMALL: return "the call needs more than the library's static scratch holds";
    default: return "unknown status";
  }
}

int llama_ffn_hidden_dim(const llama_model_args* a, int32_t* hidden) {
  if (!a || !hidden || a->dim <= 0 || a->multiple_of <= 0) return LLAMA_ERR_INVALID_ARG;
  // int(2 * (4*dim) / 3), then int(multiplier * hidden), then round up to multiple_of
  int64_t hd = (int64_t)(2.0 * (4.0 * (double)a->dim) / 3.0);
  if (a->ffn_dim_multiplier > 0.f) hd = (int64_t)((double)a->ffn_dim_multiplier * (double)hd);
  const int64_t m = a->multiple_of;
  hd = m * ((hd + m - 1) / m);
  if (hd <= 0 || hd > INT32_MAX) return LLAMA_ERR_INVALID_ARG;
  *hidden = (int32_t)hd;
  return LLAMA_OK;
}

int llama_block_workspace_size(const llama_model_args* a, int32_t bsz, int32_t seqlen, int32_t start_pos,
                               llama_dtype dt, size_t* bytes) {
  Dims g;
  int rc = model_dims(a, dt, &g);
  if (rc != LLAMA_OK) return rc;
  if (!bytes) return LLAMA_ERR_INVALID_ARG;
  rc = call_shape(a, bsz, seqlen, start_pos);
  if (rc != LLAMA_OK) return rc;
  *bytes = block_ws_layout(g, bsz, seqlen, start_pos, dt).total;
  return LLAMA_OK;
}

int llama_attn_decode_workspace_size(const llama_model_args* a, int32_t bsz, int32_t start_pos, size_t* bytes) {
  if (!a || !bytes) return LLAMA_ERR_INVALID_ARG;
  const int H = a->n_heads, Hkv = a->n_kv_heads <= 0 ? a->n_heads : a->n_kv_heads;
  if (a->dim <= 0 || H <= 0 || Hkv <= 0 || H % Hkv || a->dim % H || bsz < 1 || start_pos < 0)
    return LLAMA_ERR_INVALID_ARG;
  Dims g{a->dim, H, Hkv, a->dim / H, 0, H / Hkv};
  *bytes = decode_partial_floats(g, bsz, start_pos + 1, LLAMA_BF16) * sizeof(float);
  return LLAMA_OK;
}

int llama_ffn_workspace_size(int64_t rows, int32_t dim, int32_t hidden, llama_dtype dt, size_t* bytes) {
  if (!bytes || rows < 0 || dim <= 0 || hidden <= 0 || !dtype_ok(dt) || rows > INT32_MAX) return LLAMA_ERR_INVALID_ARG;
  // the gated activation plus the larger of the two GEMMs' split-K partials
  const int M = (int)rows;
  size_t g = align_up((size_t)rows * hidden * elem_size(dt));
  size_t pf = std::max(gemm_partial_floats(M, hidden, dim, true, dt), gemm_partial_floats(M, dim, hidden, false, dt));
  *bytes = g + align_up(pf * sizeof(float));
  return LLAMA_OK;
}

int llama_lm_head_workspace_size(int32_t bsz, int32_t dim, int32_t vocab, llama_dtype dt, size_t* bytes) {
  if (!bytes || bsz < 1 || dim <= 0 || vocab <= 0 || !dtype_ok(dt)) return LLAMA_ERR_INVALID_ARG;
  size_t xn = align_up((size_t)bsz * dim * elem_size(dt));
  size_t pf = gemm_partial_floats(bsz, vocab, dim, false, dt);
  *bytes = xn + align_up(pf * sizeof(float));
  return LLAMA_OK;
}

int llama_rope_freqs(float* freqs, int32_t head_dim, int32_t end, float theta, llama_stream_t stream) {
  if (!freqs || head_dim <= 0 || head_dim % 2 || end < 1 || !(theta > 0.f)) return LLAMA_ERR_INVALID_ARG;
  if (((uintptr_t)freqs) % 16) return LLAMA_ERR_INVALID_ARG;
  return hip_status(llama::rope_table(freqs, head_dim, end, (double)theta, (hipStream_t)stream));
}

int llama_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int32_t dim, float eps, llama_dtype dt,
                  llama_stream_t stream) {
  if (!dtype_ok(dt) || rows < 0 || dim < 1 || !(eps >= 0.f)) return LLAMA_ERR_INVALID_ARG;
  if (rows == 0) return LLAMA_OK;
  if (!x || !w || !y) return LLAMA_ERR_INVALID_ARG;
  if (!all_al16(x, w, y)) return LLAMA_ERR_INVALID_ARG;
  if (dim % (dt == LLAMA_BF16 ? 8 : 4)) return LLAMA_ERR_INVALID_ARG;
  if (rows > INT32_MAX) return LLAMA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (dt == LLAMA_BF16)
    return hip_status(llama::rmsnorm<bf16>((const bf16*)x, dim, (const bf16*)w, (bf16*)y, rows, dim, eps, st));
  return hip_status(llama::rmsnorm<float>((const float*)x, dim, (const float*)w, (float*)y, rows, dim, eps, st));
}

int llama_rope(void* xq, void* xk, const float* freqs, int32_t freqs_end, int32_t bsz, int32_t seqlen,
               int32_t start_pos, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, llama_dtype dt,
               llama_stream_t stream) {
  if (!dtype_ok(dt) || !xq || !freqs) return LLAMA_ERR_INVALID_ARG;
  if (bsz < 1 || seqlen < 1 || start_pos < 0 || n_heads < 1 || head_dim < 4 || head_dim % 4)
    return LLAMA_ERR_INVALID_ARG;
  if (xk && n_kv_heads < 1) return LLAMA_ERR_INVALID_ARG;
  if ((int64_t)start_pos + seqlen > freqs_end) return LLAMA_ERR_INVALID_ARG;
  if (!all_al16(xq, xk, freqs)) return LLAMA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (dt == LLAMA_BF16) {
    e = llama::rope_apply<bf16>((bf16*)xq, freqs, bsz, seqlen, start_pos, n_heads, head_dim, st);
    if (e == hipSuccess && xk)
      e = llama::rope_apply<bf16>((bf16*)xk, freqs, bsz, seqlen, start_pos, n_kv_heads, head_dim, st);
  } else {
    e = llama::rope_apply<float>((float*)xq, freqs, bsz, seqlen, start_pos, n_heads, head_dim, st);
    if (e == hipSuccess && xk)
      e = llama::rope_apply<float>((float*)xk, freqs, bsz, seqlen, start_pos, n_kv_heads, head_dim, st);
  }
  return hip_status(e);
}

int llama_gqa_attn_prefill(const void* xq, const void* xk, const void* xv, void* cache_k, void* cache_v, void* out,
                           const llama_model_args* a, int32_t bsz, int32_t seqlen, int32_t start_pos, llama_dtype dt,
                           llama_stream_t stream) {
  Dims g;
  int rc = model_dims(a, dt, &g);
  if (rc != LLAMA_OK) return rc;
  rc = call_shape(a, bsz, seqlen, start_pos);
  if (rc != LLAMA_OK) return rc;
  if (!xq || !xk || !xv || !cache_k || !cache_v || !out) return LLAMA_ERR_INVALID_ARG;
  if (!all_al16(xq, xk, xv, cache_k, cache_v, out)) return LLAMA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  llama::AttnShape sh{bsz, seqlen, start_pos, g.H, g.Hkv, g.d, a->max_seq_len};
  hipError_t e;
  if (dt == LLAMA_BF16) {
    e = llama::kv_append<bf16>((const bf16*)xk, (const bf16*)xv, (bf16*)cache_k, (bf16*)cache_v, sh, st);
    if (e == hipSuccess)
      e = llama::attn_prefill<bf16>((const bf16*)xq, (const bf16*)cache_k, (const bf16*)cache_v, (bf16*)out, sh, st);
  } else {
    e = llama::kv_append<float>((const float*)xk, (const float*)xv, (float*)cache_k, (float*)cache_v, sh, st);
    if (e == hipSuccess)
      e = llama::attn_prefill<float>((const float*)xq, (const float*)cache_k, (const float*)cache_v, (float*)out, sh,
                                     st);
  }
  return hip_status(e);
}

// Validation and launch shared by llama_gqa_attn_decode and its allocation-free
// variant; `partial` is the split-K buffer (at least `need` bytes, reported
// through need_out before any launch so the caller can bound it).
static int attn_decode_impl(const void* xq, const void* xk, const void* xv, void* cache_k, void* cache_v, void* out,
                            const llama_model_args* a, int32_t bsz, int32_t start_pos, void* ws, size_t ws_bytes,
                            llama_dtype dt, llama_stream_t stream, bool static_ws) {
  Dims g;
  int rc = model_dims(a, dt, &g);
  if (rc != LLAMA_OK) return rc;
  rc = call_shape(a, bsz, 1, start_pos);
  if (rc != LLAMA_OK) return rc;
  if (!xq || !xk || !xv || !cache_k || !cache_v || !out) return LLAMA_ERR_INVALID_ARG;
  const size_t need = decode_partial_floats(g, bsz, start_pos + 1, dt) * sizeof(float);
  if (need && !ws) return static_ws ? LLAMA_ERR_HIP : LLAMA_ERR_INVALID_ARG;
  if (!all_al16(xq, xk, xv, cache_k, cache_v, out, need ? ws : nullptr)) return LLAMA_ERR_INVALID_ARG;
  if (ws_bytes < need) return static_ws ? LLAMA_ERR_SCRATCH_TOO_SMALL : LLAMA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;
  llama::AttnShape sh{bsz, 1, start_pos, g.H, g.Hkv, g.d, a->max_seq_len};
  hipError_t e;
  if (dt == LLAMA_BF16) {
    e = llama::kv_append<bf16>((const bf16*)xk, (const bf16*)xv, (bf16*)cache_k, (bf16*)cache_v, sh, st);
    if (e == hipSuccess)
      e = llama::attn_decode<bf16>((const bf16*)xq, (const bf16*)cache_k, (const bf16*)cache_v, (bf16*)out, sh,
                                   (float*)ws, st);
  } else {
    e = llama::kv_append<float>((const float*)xk, (const float*)xv, (float*)cache_k, (float*)cache_v, sh, st);
    if (e == hipSuccess)
      e = llama::attn_decode<float>((const float*)xq, (const float*)cache_k, (const float*)cache_v, (float*)out, sh,
                                    (float*)ws, st);
  }
  return hip_status(e);
}

int llama_gqa_attn_decode(const void* xq, const void* xk, const void* xv, void* cache_k, void* cache_v, void* out,
                          const llama_model_args* a, int32_t bsz, int32_t start_pos, void* ws, size_t ws_bytes,
                          llama_dtype dt, llama_stream_t stream) {
  return attn_decode_impl(xq, xk, xv, cache_k, cache_v, out, a, bsz, start_pos, ws, ws_bytes, dt, stream, false);
}

// Allocation-free decode attention: the split-K partials live in `scratch`, one
// copy per GPU (a file-scope device array, so the library never calls hipMalloc).
// On the first call on a device its address is fetched with hipGetSymbolAddress
// (the array's name is only a host-side stand-in, not a device address) and kept
// per device; kernels receive that address.  Nothing in the partials has to start
// at zero: every split writes all of its (max, sum, o) entries before the merge
// kernel reads them.
}  // extern "C"

namespace {
// 8 MiB: the split rule gives at most about 4 MiB of partials below four million
// attended keys (at most 512 splits x 16 query heads per kv head), 8.1 MiB beyond
constexpr size_t kScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's scratch array, or nullptr on a HIP error.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

size_t llama_static_scratch_bytes(void) { return kScratchBytes; }

int llama_gqa_attn_decode_static(const void* xq, const void* xk, const void* xv, void* cache_k, void* cache_v,
                                 void* out, const llama_model_args* a, int32_t bsz, int32_t start_pos, llama_dtype dt,
                                 llama_stream_t stream) {
  // the size check comes first, on the host, so an oversized call never touches the device
  Dims g;
  int rc = model_dims(a, dt, &g);
  if (rc != LLAMA_OK) return rc;
  rc = call_shape(a, bsz, 1, start_pos);
  if (rc != LLAMA_OK) return rc;
  const size_t need = decode_partial_floats(g, bsz, start_pos + 1, dt) * sizeof(float);
  if (need > kScratchBytes) return LLAMA_ERR_SCRATCH_TOO_SMALL;
  void* ws = need ? scratch_on_current_device() : nullptr;
  if (need && !ws) return LLAMA_ERR_HIP;
  return attn_decode_impl(xq, xk, xv, cache_k, cache_v, out, a, bsz, start_pos, ws, kScratchBytes, dt, stream, true);
}

int llama_linear(const void* x, const void* w, void* y, int64_t rows, int32_t in, int32_t outf, llama_dtype dt,
                 llama_stream_t stream) {
  if (!dtype_ok(dt) || rows < 0 || in < 1 || outf < 1) return LLAMA_ERR_INVALID_ARG;
  if (rows == 0) return LLAMA_OK;
  if (!x || !w || !y || rows > INT32_MAX) return LLAMA_ERR_INVALID_ARG;
  if (in % (dt == LLAMA_BF16 ? 8 : 4) || outf % 4) return LLAMA_ERR_INVALID_ARG;
  if (!all_al16(x, w, y)) return LLAMA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (dt == LLAMA_BF16) {
    llama::WeightRows<bf16> wr{(const bf16*)w, nullptr, nullptr, outf, outf};
    e = llama::gemm_launch<bf16>((const bf16*)x, in, wr, (int)rows, outf, in, llama::EpiStore<bf16>{(bf16*)y, outf},
                                 1, nullptr, st);
  } else {
    llama::WeightRows<float> wr{(const float*)w, nullptr, nullptr, outf, outf};
    e = llama::gemm_launch<float>((const float*)x, in, wr, (int)rows, outf, in,
                                  llama::EpiStore<float>{(float*)y, outf}, 1, nullptr, st);
  }
  return hip_status(e);
}

int llama_swiglu_ffn(const void* x, const void* w1, const void* w3, const void* w2, void* y, int64_t rows,
                     int32_t dim, int32_t hidden, void* ws, size_t ws_bytes, llama_dtype dt, llama_stream_t stream) {
  if (!dtype_ok(dt) || rows < 0 || dim < 1 || hidden < 1) return LLAMA_ERR_INVALID_ARG;
  const int al = dt == LLAMA_BF16 ? 8 : 4;
  if (dim % al || hidden % al || rows > INT32_MAX) return LLAMA_ERR_INVALID_ARG;
  size_t need = 0;
  llama_ffn_workspace_size(rows, dim, hidden, dt, &need);
  if (rows == 0) return LLAMA_OK;
  if (!x || !w1 || !w3 || !w2 || !y || !ws) return LLAMA_ERR_INVALID_ARG;
  if (!all_al16(x, w1, w3, w2, y, ws)) return LLAMA_ERR_INVALID_ARG;
  if (ws_bytes < need) return LLAMA_ERR_WORKSPACE_TOO_SMALL;
  const int M = (int)rows;
  const bool bf = dt == LLAMA_BF16;
  char* wsb = (char*)ws;
  float* part = (float*)(wsb + align_up((size_t)rows * hidden * elem_size(dt)));
  const int s1 = llama::gemm_pick_splits(M, hidden, dim, true, bf);
  const int s2 = llama::gemm_pick_splits(M, dim, hidden, false, bf);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (bf) {
    bf16* g = (bf16*)wsb;
    e = llama::gemm_dual_launch<bf16>((const bf16*)x, dim, (const bf16*)w1, (const bf16*)w3, M, hidden, dim,
                                      llama::EpiSwiGLU<bf16>{g, hidden, nullptr}, s1, part, st);
    if (e == hipSuccess) {
      llama::WeightRows<bf16> wr{(const bf16*)w2, nullptr, nullptr, dim, dim};
      e = llama::gemm_launch<bf16>(g, hidden, wr, M, dim, hidden, llama::EpiStore<bf16>{(bf16*)y, dim}, s2, part, st);
    }
  } else {
    float* g = (float*)wsb;
    e = llama::gemm_dual_launch<float>((const float*)x, dim, (const float*)w1, (const float*)w3, M, hidden, dim,
                                       llama::EpiSwiGLU<float>{g, hidden, nullptr}, s1, part, st);
    if (e == hipSuccess) {
      llama::WeightRows<float> wr{(const float*)w2, nullptr, nullptr, dim, dim};
      e = llama::gemm_launch<float>(g, hidden, wr, M, dim, hidden, llama::EpiStore<float>{(float*)y, dim}, s2, part,
                                    st);
    }
  }
  return hip_status(e);
}

static int block_forward_impl(const llama_model_args* a, const llama_block_weights* w, void* cache_k, void* cache_v,
                              const float* freqs, int32_t freqs_end, const void* x, void* out, int32_t bsz,
                              int32_t seqlen, int32_t start_pos, void* ws, size_t ws_bytes, llama_dtype dt,
                              llama_stream_t stream, hipEvent_t* ev, const int32_t* pos_dev = nullptr) {
  Dims g;
  int rc = model_dims(a, dt, &g);
  if (rc != LLAMA_OK) return rc;
  rc = call_shape(a, bsz, seqlen, start_pos);
  if (rc != LLAMA_OK) return rc;
  if (!w || !cache_k || !cache_v || !freqs || !x || !out || !ws) return LLAMA_ERR_INVALID_ARG;
  if (!w->attention_norm || !w->wq || !w->wk || !w->wv || !w->wo || !w->ffn_norm || !w->w1 || !w->w2 || !w->w3)
    return LLAMA_ERR_INVALID_ARG;
  if ((int64_t)start_pos + seqlen > freqs_end) return LLAMA_ERR_INVALID_ARG;
  if (!all_al16(freqs, x, out, ws, cache_k, cache_v, w->attention_norm, w->wq, w->wk, w->wv, w->wo, w->ffn_norm,
                w->w1, w->w2, w->w3))
    return LLAMA_ERR_INVALID_ARG;
  const size_t act = (size_t)bsz * seqlen * g.D * elem_size(dt);
  if (overlaps(x, act, out, act)) return LLAMA_ERR_INVALID_ARG;
  if ((int64_t)bsz * seqlen > INT32_MAX / 2) return LLAMA_ERR_INVALID_ARG;
  const BlockWs L = block_ws_layout(g, bsz, seqlen, start_pos, dt);
  if (ws_bytes < L.total) return LLAMA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;
  if (dt == LLAMA_BF16)
    return block_forward_t<bf16>(g, a, w, (bf16*)cache_k, (bf16*)cache_v, freqs, (const bf16*)x, (bf16*)out, bsz,
                                 seqlen, start_pos, (char*)ws, L, st, ev, pos_dev);
  return block_forward_t<float>(g, a, w, (float*)cache_k, (float*)cache_v, freqs, (const float*)x, (float*)out, bsz,
                                seqlen, start_pos, (char*)ws, L, st, ev, nullptr);
}

int llama_block_forward(const llama_model_args* a, const llama_block_weights* w, void* cache_k, void* cache_v,
                        const float* freqs, int32_t freqs_end, const void* x, void* out, int32_t bsz, int32_t seqlen,
                        int32_t start_pos, void* ws, size_t ws_bytes, llama_dtype dt, llama_stream_t stream) {
  return block_forward_impl(a, w, cache_k, cache_v, freqs, freqs_end, x, out, bsz, seqlen, start_pos, ws, ws_bytes,
                            dt, stream, nullptr);
}

int llama_block_forward_events(const llama_model_args* a, const llama_block_weights* w, void* cache_k,
                               void* cache_v, const float* freqs, int32_t freqs_end, const void* x, void* out,
                               int32_t bsz, int32_t seqlen, int32_t start_pos, void* ws, size_t ws_bytes,
                               llama_dtype dt, llama_stream_t stream, void* const* events) {
  if (!events) return LLAMA_ERR_INVALID_ARG;
  for (int i = 0; i < 8; ++i)
    if (!events[i]) return LLAMA_ERR_INVALID_ARG;
  return block_forward_impl(a, w, cache_k, cache_v, freqs, freqs_end, x, out, bsz, seqlen, start_pos, ws, ws_bytes,
                            dt, stream, (hipEvent_t*)events);
}

int llama_block_decode_at(const llama_model_args* a, const llama_block_weights* w, void* cache_k, void* cache_v,
                          const float* freqs, int32_t freqs_end, const void* x, void* out, int32_t bsz,
                          const int32_t* start_pos_dev, int32_t max_start_pos, void* ws, size_t ws_bytes,
                          llama_dtype dt, llama_stream_t stream) {
  if (!start_pos_dev || ((uintptr_t)start_pos_dev) % 4) return LLAMA_ERR_INVALID_ARG;
  if (dt != LLAMA_BF16) return LLAMA_ERR_UNSUPPORTED;
  return block_forward_impl(a, w, cache_k, cache_v, freqs, freqs_end, x, out, bsz, 1, max_start_pos, ws, ws_bytes,
                            dt, stream, nullptr, start_pos_dev);
}

int llama_embedding(const int32_t* tokens, const void* table, void* out, int64_t n, int32_t dim, int32_t vocab,
                    llama_dtype dt, llama_stream_t stream) {
  if (!dtype_ok(dt) || n < 0 || dim < 1 || vocab < 1) return LLAMA_ERR_INVALID_ARG;
  if (n == 0) return LLAMA_OK;
  if (!tokens || !table || !out) return LLAMA_ERR_INVALID_ARG;
  if (dim % (dt == LLAMA_BF16 ? 8 : 4)) return LLAMA_ERR_INVALID_ARG;
  if (!al4(tokens) || !all_al16(table, out)) return LLAMA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (dt == LLAMA_BF16)
    return hip_status(llama::embedding<bf16>(tokens, (const bf16*)table, (bf16*)out, n, dim, vocab, st));
  return hip_status(llama::embedding<float>(tokens, (const float*)table, (float*)out, n, dim, vocab, st));
}

int llama_lm_head_argmax(const void* h, int64_t h_row_stride, const void* norm_w, const void* w_out, float* logits,
                         int32_t* next, int32_t bsz, int32_t dim, int32_t vocab, float eps, void* ws,
                         size_t ws_bytes, llama_dtype dt, llama_stream_t stream) {
  if (!dtype_ok(dt) || bsz < 1 || dim < 1 || vocab < 1 || h_row_stride < dim || !(eps >= 0.f))
    return LLAMA_ERR_INVALID_ARG;
  if (!h || !norm_w || !w_out || !logits || !next || !ws) return LLAMA_ERR_INVALID_ARG;
  if (dim % (dt == LLAMA_BF16 ? 8 : 4) || vocab % 4 || h_row_stride % (dt == LLAMA_BF16 ? 8 : 4))
    return LLAMA_ERR_INVALID_ARG;
  if (!all_al16(h, norm_w, w_out, logits, ws) || !al4(next)) return LLAMA_ERR_INVALID_ARG;
  size_t need = 0;
  llama_lm_head_workspace_size(bsz, dim, vocab, dt, &need);
  if (ws_bytes < need) return LLAMA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;
  const bool bf = dt == LLAMA_BF16;
  char* wsb = (char*)ws;
  float* part = (float*)(wsb + align_up((size_t)bsz * dim * elem_size(dt)));
  const int splits = llama::gemm_pick_splits(bsz, vocab, dim, false, bf);
  hipError_t e;
  if (bf) {
    bf16* xn = (bf16*)wsb;
    e = llama::rmsnorm<bf16>((const bf16*)h, h_row_stride, (const bf16*)norm_w, xn, bsz, dim, eps, st);
    if (e == hipSuccess) {
      llama::WeightRows<bf16> wr{(const bf16*)w_out, nullptr, nullptr, vocab, vocab};
      e = llama::gemm_launch<bf16>(xn, dim, wr, bsz, vocab, dim, llama::EpiF32{logits, vocab}, splits, part, st);
    }
  } else {
    float* xn = (float*)wsb;
    e = llama::rmsnorm<float>((const float*)h, h_row_stride, (const float*)norm_w, xn, bsz, dim, eps, st);
    if (e == hipSuccess) {
      llama::WeightRows<float> wr{(const float*)w_out, nullptr, nullptr, vocab, vocab};
      e = llama::gemm_launch<float>(xn, dim, wr, bsz, vocab, dim, llama::EpiF32{logits, vocab}, splits, part, st);
    }
  }
  if (e == hipSuccess) e = llama::argmax_rows(logits, next, bsz, vocab, st);
  return hip_status(e);
}

int llama_sample_top_p(const float* logits, int32_t* next, int32_t bsz, int32_t vocab, float temperature,
                       float top_p, const float* uniforms, llama_stream_t stream) {
  if (!logits || !next || bsz < 1 || vocab < 1) return LLAMA_ERR_INVALID_ARG;
  if (temperature != temperature || top_p != top_p) return LLAMA_ERR_INVALID_ARG;
  if (!al16(logits) || !al4(next) || !al4(uniforms)) return LLAMA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (!(temperature > 0.f)) return hip_status(llama::argmax_rows(logits, next, bsz, vocab, st));
  if (!uniforms) return LLAMA_ERR_INVALID_ARG;
  return hip_status(llama::sample_top_p(logits, next, bsz, vocab, temperature, top_p, uniforms, st));
}

}  // extern "C"
