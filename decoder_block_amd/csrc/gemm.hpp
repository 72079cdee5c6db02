// Projection GEMMs of the decoder block: C[m][n] = sum_k A[m][k] * W[n][k]
// (nn.Linear, y = x W^T) with fused epilogues.  Declarations shared by the
// launch layer; the kernels live in gemm.hip.
#pragma once

#include "common.hpp"

namespace llama {

// Where weight row n of the virtual [N][K] operand lives.  Plain GEMMs use w0
// only (n1 = n2 = N).  The QKV projection concatenates wq | wk | wv: rows
// [0, n1) from w0, [n1, n2) from w1, [n2, N) from w2.
template <typename T>
struct WeightRows {
  const T* w0;
  const T* w1;
  const T* w2;
  int n1, n2;
};

// Epilogues receive 4 consecutive output columns n..n+3 of row m in fp32.
template <typename T>
struct EpiStore {
  T* y;
  int64_t ldy;
  __device__ __forceinline__ void operator()(int m, int n, f32x4 v) const {
    store4(y + (int64_t)m * ldy + n, v);
  }
};

// y = r + acc (the residual add of TransformerBlock.forward); y may equal r.
template <typename T>
struct EpiResidual {
  T* y;
  const T* r;
  int64_t ld;
  __device__ __forceinline__ void operator()(int m, int n, f32x4 v) const {
    int64_t o = (int64_t)m * ld + n;
    f32x4 rv = load4(r + o);
    store4(y + o, rv + v);
  }
};

// fp32 output (LM-head logits).
struct EpiF32 {
  float* y;
  int64_t ldy;
  __device__ __forceinline__ void operator()(int m, int n, f32x4 v) const {
    store4(y + (int64_t)m * ldy + n, v);
  }
};

// QKV epilogue: columns [0, nq) are q, [nq, nq+nkv) are k, the rest v.  q and k
// get the interleaved-pair rotation of their position (start_pos + m % seqlen)
// from the fp32 (cos, sin) table; q goes to q_out [M][nq]; k and v are written
// straight into the caches at [b][start_pos + s] (cache append).  head_dim is a
// power of two.  With pos_dev set, the base position is *pos_dev, read when the
// kernel runs and clamped to [0, start_pos] (start_pos then holds the largest
// position the caller allows).
template <typename T>
struct EpiQKV {
  T* q_out;
  T* cache_k;
  T* cache_v;
  const float* freqs;  // [freqs_end][head_dim/2][2]
  int seqlen, start_pos, max_seq, nq, nkv, head_dim;
  const float* rscale; // optional per-row RMSNorm factor applied to the accumulators
  const int32_t* pos_dev = nullptr;  // optional device-resident base position
  __device__ __forceinline__ int base() const { return pos_dev ? min(max(*pos_dev, 0), start_pos) : start_pos; }
  // (cos_i, sin_i, cos_i+1, sin_i+1) of columns n..n+3 (zero for v columns)
  __device__ __forceinline__ f32x4 cos_sin(int m, int n) const {
    if (n >= nq + nkv) return f32x4{};
    const int pos = base() + (m - (m / seqlen) * seqlen);
    const int e = (n < nq ? n : n - nq) & (head_dim - 1);
    return *(const f32x4*)(freqs + ((int64_t)pos * (head_dim >> 1) + (e >> 1)) * 2);
  }
  __device__ __forceinline__ static f32x4 rotate(f32x4 v, f32x4 cs) {
    return f32x4{v[0] * cs[0] - v[1] * cs[1], v[0] * cs[1] + v[1] * cs[0],
                 v[2] * cs[2] - v[3] * cs[3], v[2] * cs[3] + v[3] * cs[2]};
  }
  __device__ __forceinline__ void apply(int m, int n, f32x4 v, f32x4 cs) const {
    if (rscale) v *= rscale[m];
    int b = m / seqlen, s = m - b * seqlen;
    int pos = base() + s;
    if (n < nq) {
      store4(q_out + (int64_t)m * nq + n, rotate(v, cs));
    } else if (n < nq + nkv) {
      int c = n - nq;
      store4(cache_k + ((int64_t)b * max_seq + pos) * nkv + c, rotate(v, cs));
    } else {
      int c = n - nq - nkv;
      store4(cache_v + ((int64_t)b * max_seq + pos) * nkv + c, v);
    }
  }
  __device__ __forceinline__ void operator()(int m, int n, f32x4 v) const { apply(m, n, v, cos_sin(m, n)); }
};

// Row-hoisted, two-phase form of an epilogue for the GEMM kernels.  epi_row(m)
// computes what depends on the row only (once per row fragment); epi_pre(row,
// n) loads what the group of columns n..n+3 needs (the QKV epilogue's (cos,
// sin)), fetched for a whole fragment before its stores, which the compiler
// could not otherwise move the loads past (the pointers may alias); epi_apply
// finishes the group.  Plain epilogues take the row index and load nothing.
struct NoPre {};
template <class Epi>
__device__ __forceinline__ int epi_row(const Epi&, int m) {
  return m;
}
template <class Epi>
__device__ __forceinline__ NoPre epi_pre(const Epi&, int, int) {
  return {};
}
template <class Epi>
__device__ __forceinline__ void epi_apply(const Epi& e, int m, int n, f32x4 v, NoPre) {
  e(m, n, v);
}

// The residual epilogue's pre-load is the residual group itself (8 bytes in
// bf16), small enough that the GEMM kernel fetches a wave's whole tile of them
// before its first store.
__device__ __forceinline__ bf16x4 epi_pre(const EpiResidual<bf16>& e, int m, int n) {
  return *(const bf16x4*)(e.r + (int64_t)m * e.ld + n);
}
__device__ __forceinline__ void epi_apply(const EpiResidual<bf16>& e, int m, int n, f32x4 v, bf16x4 r) {
  const f32x4 rv = {(float)r[0], (float)r[1], (float)r[2], (float)r[3]};
  store4(e.y + (int64_t)m * e.ld + n, rv + v);
}

template <typename T>
struct QkvRow {
  T* q;              // q_out row
  T* k;              // cache_k row at the token's position
  T* v;              // cache_v row
  const float* cs;   // (cos, sin) table row of the position
  float scale;       // RMSNorm factor (1 without)
};
template <typename T>
__device__ __forceinline__ QkvRow<T> epi_row(const EpiQKV<T>& e, int m) {
  const int b = m / e.seqlen, s = m - b * e.seqlen;
  const int pos = e.base() + s;
  const int64_t crow = ((int64_t)b * e.max_seq + pos) * e.nkv;
  return QkvRow<T>{e.q_out + (int64_t)m * e.nq, e.cache_k + crow, e.cache_v + crow,
                   e.freqs + (int64_t)pos * e.head_dim, e.rscale ? e.rscale[m] : 1.0f};
}
template <typename T>
__device__ __forceinline__ f32x4 epi_pre(const EpiQKV<T>& e, const QkvRow<T>& r, int n) {
  const int c = n < e.nq ? n : n - e.nq;   // v columns load a harmless table entry
  return *(const f32x4*)(r.cs + (c & (e.head_dim - 1)));
}
template <typename T>
__device__ __forceinline__ void epi_apply(const EpiQKV<T>& e, const QkvRow<T>& r, int n, f32x4 v, f32x4 cs) {
  v *= r.scale;
  const bool is_q = n < e.nq, is_v = n >= e.nq + e.nkv;
  const f32x4 o = is_v ? v : EpiQKV<T>::rotate(v, cs);
  T* dst = is_q ? r.q + n : (is_v ? r.v + (n - e.nq - e.nkv) : r.k + (n - e.nq));
  store4(dst, o);
}

// SwiGLU epilogue: g = silu(a1) * a3 with a1 = (x w1^T), a3 = (x w3^T).
template <typename T>
struct EpiSwiGLU {
  T* g;
  int64_t ldg;
  const float* rscale; // optional per-row RMSNorm factor applied to both accumulators
  __device__ __forceinline__ float row_scale(int m) const { return rscale ? rscale[m] : 1.0f; }
  // with the row factor r fetched beforehand (the GEMM kernel loads a wave's
  // factors before its first store, which they could otherwise not pass)
  __device__ __forceinline__ void apply(int m, int n, f32x4 a1, f32x4 a3, float r) const {
    a1 *= r;
    a3 *= r;
    // silu(a) = a / (1 + e^-a) as a * rcp(1 + 2^(-a log2 e)): v_exp_f32 and
    // v_rcp_f32 (about 1 ulp each) instead of a correctly rounded division, a
    // quarter of the epilogue's instructions; large |a| give the limits a and 0
    constexpr float kLog2e = 1.4426950408889634f;
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = a1[i] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a1[i] * kLog2e)) * a3[i];
    store4(g + (int64_t)m * ldg + n, o);
  }
  __device__ __forceinline__ void operator()(int m, int n, f32x4 a1, f32x4 a3) const {
    apply(m, n, a1, a3, row_scale(m));
  }
  __device__ __forceinline__ static f32x4 silu_mul(f32x4 a1, f32x4 a3) {
    constexpr float kLog2e = 1.4426950408889634f;
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = a1[i] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a1[i] * kLog2e)) * a3[i];
    return o;
  }
  // columns n..n+7 (lo, hi of both products) as one 16-byte store
  __device__ __forceinline__ void apply8(int m, int n, f32x4 a1lo, f32x4 a1hi, f32x4 a3lo, f32x4 a3hi,
                                         float r) const {
    store8(g + (int64_t)m * ldg + n, silu_mul(a1lo * r, a3lo * r), silu_mul(a1hi * r, a3hi * r));
  }
};

// 8-column forms, used by the large-tile kernel on interior tiles when every
// row it writes (and reads) is 16-byte aligned: columns n..n+7 (n a multiple
// of 8) arrive as lo = n..n+3 and hi = n+4..n+7 and are stored as 16 bytes.
// epi_vec8_ok says whether an epilogue's pointers and row strides allow it.
template <class Epi>
__device__ __forceinline__ bool epi_vec8_ok(const Epi&) {
  return false;
}
template <class Epi, class Row>
__device__ __forceinline__ NoPre epi_pre8(const Epi&, const Row&, int) {
  return {};
}

__device__ __forceinline__ bool epi_vec8_ok(const EpiStore<bf16>& e) { return e.ldy % 8 == 0 && aligned16(e.y); }
__device__ __forceinline__ void epi_apply8(const EpiStore<bf16>& e, int m, int n, f32x4 lo, f32x4 hi, NoPre) {
  store8(e.y + (int64_t)m * e.ldy + n, lo, hi);
}

__device__ __forceinline__ bool epi_vec8_ok(const EpiF32& e) { return e.ldy % 4 == 0 && aligned16(e.y); }
__device__ __forceinline__ void epi_apply8(const EpiF32& e, int m, int n, f32x4 lo, f32x4 hi, NoPre) {
  float* p = e.y + (int64_t)m * e.ldy + n;
  store4(p, lo);
  store4(p + 4, hi);
}

__device__ __forceinline__ bool epi_vec8_ok(const EpiResidual<bf16>& e) {
  return e.ld % 8 == 0 && aligned16(e.y) && aligned16(e.r);
}
__device__ __forceinline__ bf16x8 epi_pre8(const EpiResidual<bf16>& e, int m, int n) {
  return *(const bf16x8*)(e.r + (int64_t)m * e.ld + n);
}
__device__ __forceinline__ void epi_apply8(const EpiResidual<bf16>& e, int m, int n, f32x4 lo, f32x4 hi, bf16x8 r) {
  const f32x4 rlo = {(float)r[0], (float)r[1], (float)r[2], (float)r[3]};
  const f32x4 rhi = {(float)r[4], (float)r[5], (float)r[6], (float)r[7]};
  store8(e.y + (int64_t)m * e.ld + n, rlo + lo, rhi + hi);
}

// (cos, sin) of the four column pairs of columns n..n+7
struct CosSin8 {
  f32x4 lo, hi;
};
template <typename T>
__device__ __forceinline__ bool epi_vec8_ok(const EpiQKV<T>& e) {
  return sizeof(T) == 2 && e.nq % 8 == 0 && e.nkv % 8 == 0 && e.head_dim % 8 == 0 && aligned16(e.q_out) &&
         aligned16(e.cache_k) && aligned16(e.cache_v) && aligned16(e.freqs);
}
template <typename T>
__device__ __forceinline__ CosSin8 epi_pre8(const EpiQKV<T>& e, const QkvRow<T>& r, int n) {
  const int c = n < e.nq ? n : n - e.nq;   // v columns load a harmless table entry
  const float* t = r.cs + (c & (e.head_dim - 1));
  return CosSin8{*(const f32x4*)t, *(const f32x4*)(t + 4)};
}
template <typename T>
__device__ __forceinline__ void epi_apply8(const EpiQKV<T>& e, const QkvRow<T>& r, int n, f32x4 lo, f32x4 hi,
                                           CosSin8 cs) {
  lo *= r.scale;
  hi *= r.scale;
  const bool is_q = n < e.nq, is_v = n >= e.nq + e.nkv;
  const f32x4 olo = is_v ? lo : EpiQKV<T>::rotate(lo, cs.lo);
  const f32x4 ohi = is_v ? hi : EpiQKV<T>::rotate(hi, cs.hi);
  T* dst = is_q ? r.q + n : (is_v ? r.v + (n - e.nq - e.nkv) : r.k + (n - e.nq));
  store8(dst, olo, ohi);
}

// the dual epilogue over 8 columns, with the row factor fetched beforehand
template <typename T>
__device__ __forceinline__ bool epi_vec8_ok(const EpiSwiGLU<T>& e) {
  return sizeof(T) == 2 && e.ldg % 8 == 0 && aligned16(e.g);
}

// Host-side launch helpers (gemm.hip).  `splits` > 1 runs split-K: partial
// sums go to `partial` (fp32, splits * M * N_out * (dual ? 2 : 1) floats) and a
// second kernel reduces them and applies the epilogue.
template <typename T, class Epi>
hipError_t gemm_launch(const T* A, int64_t lda, WeightRows<T> w, int M, int N, int K, Epi epi,
                       int splits, float* partial, hipStream_t st);
template <typename T, class Epi>
hipError_t gemm_dual_launch(const T* A, int64_t lda, const T* w1, const T* w3, int M, int N,
                            int K, Epi epi, int splits, float* partial, hipStream_t st);

// Split count the launch layer uses for an M x N x K problem (1 for large M).
int gemm_pick_splits(int M, int N, int K, bool dual, bool bf16);

// The residual projection of a decode-sized call (bf16, 5..64 token rows, split K)
// with its reduction fused with the next RMSNorm: y = r + A W^T, then yn = y * g
// and rscale[m] = rsqrt(mean(y^2) + eps) for the GEMM that consumes yn.  `partial`
// is sized as for gemm_launch.  Only valid where gemm_residual_norm_fits.
bool gemm_residual_norm_fits(int M, int N, int K, int64_t lda);
hipError_t gemm_residual_norm_launch(const bf16* A, int64_t lda, const bf16* w, int M, int N, int K, bf16* y,
                                     const bf16* r, const bf16* g, bf16* yn, float* rscale, float eps,
                                     float* partial, hipStream_t st);

// Weight-streaming kernels for M <= kGemvMaxM token rows in bf16 or fp32
// (gemv.hip); gemm_launch routes such problems there by itself.  They need
// N % 4 == 0 and K, lda multiples of one 16-byte vector (8 bf16, 4 floats)
// (gemv_fits); for the QKV map, n1 and n2 must be multiples of 4 as well.  With
// norm_w set, A's rows are RMS-normalised on the fly (A * norm_w in the
// products, rsqrt(mean(A^2) + eps) on the accumulators); the epilogue's own
// rscale must then be null.
constexpr int kGemvMaxM = 4;
template <typename T>
bool gemv_fits(int M, int N, int K, int64_t lda);
template <typename T, class Epi>
hipError_t gemv_launch(const T* A, int64_t lda, WeightRows<T> w, int M, int N, int K, const T* norm_w, float eps,
                       Epi epi, hipStream_t st);
template <typename T, class Epi>
hipError_t gemv_dual_launch(const T* A, int64_t lda, const T* w1, const T* w3, int M, int N, int K,
                            const T* norm_w, float eps, Epi epi, hipStream_t st);

}  // namespace llama
