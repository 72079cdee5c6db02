// Row and elementwise kernels (gfx950): all HBM-bound, 16-byte vector
// accesses, fp32 arithmetic, one rounding per stored value.
#include "misc.hpp"

#include <math.h>

namespace llama {

namespace {

constexpr int kThreads = 256;

// 16-byte vectors: 8 bf16 or 4 f32
template <typename T> struct Vec;
template <> struct Vec<bf16> {
  static constexpr int N = 8;
  typedef bf16x8 type;
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  typedef f32x4 type;
};

// RMSNorm (LLaMA notes, section 3, class RMSNorm): one workgroup per row; the
// sum of squares is reduced in fp32 across the wavefront and then the four
// waves; y = x * rsqrt(mean + eps) * w with a single rounding at the store.
// With `rscale` set, the kernel stores y = x * w (one rounding; exact when w is
// all ones) and the row factor rsqrt(mean + eps) in rscale[row], for a
// projection that applies the factor to its fp32 accumulators.
template <typename T>
__global__ void __launch_bounds__(kThreads)
rmsnorm_kernel(const T* __restrict__ x, int64_t x_stride, const T* __restrict__ w, T* y, int dim,
               float eps, float* __restrict__ rscale) {
  constexpr int V = Vec<T>::N;
  constexpr int CACHE = 4;
  typedef typename Vec<T>::type vec;
  __shared__ float red[kThreads / 64];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * x_stride;
  T* yr = y + row * (int64_t)dim;
  const int nvec = dim / V;
  // the row's first CACHE * kThreads vectors and their gains are loaded up front
  // (the gain loads would otherwise wait behind the reduction)
  vec cached[CACHE], wcached[CACHE];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CACHE; ++c) {
    int i = threadIdx.x + c * kThreads;
    if (i < nvec) {
      cached[c] = *(const vec*)(xr + i * V);
      wcached[c] = *(const vec*)(w + i * V);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        float f = (float)cached[c][e];
        ss += f * f;
      }
    }
  }
  for (int i = threadIdx.x + CACHE * kThreads; i < nvec; i += kThreads) {
    vec v = *(const vec*)(xr + i * V);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float f = (float)v[e];
      ss += f * f;
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) tot += red[i];
  const float rr = 1.0f / sqrtf(tot / (float)dim + eps);
  const float r = rscale ? 1.0f : rr;
  if (rscale && threadIdx.x == 0) rscale[row] = rr;
  auto emit = [&](int i, const vec& v, const vec& wv) {
    vec o;
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = from_f<T>((float)v[e] * r * (float)wv[e]);
    *(vec*)(yr + i * V) = o;
  };
#pragma unroll
  for (int c = 0; c < CACHE; ++c) {
    int i = threadIdx.x + c * kThreads;
    if (i < nvec) emit(i, cached[c], wcached[c]);
  }
  for (int i = threadIdx.x + CACHE * kThreads; i < nvec; i += kThreads)
    emit(i, *(const vec*)(xr + i * V), *(const vec*)(w + i * V));
}

// RoPE table: angle p * theta^(-2i/d) and its cos/sin in fp64, stored as fp32
// pairs (LLaMA notes, section 3, precompute_freqs_cis).
__global__ void rope_table_kernel(float* __restrict__ freqs, int head_dim, int end, double theta) {
  const int half = head_dim / 2;
  const int64_t total = (int64_t)end * half;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total;
       k += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(k / half), i = (int)(k % half);
    const double inv = pow(theta, -2.0 * (double)i / (double)head_dim);
    const double ang = (double)p * inv;
    freqs[2 * k] = (float)cos(ang);
    freqs[2 * k + 1] = (float)sin(ang);
  }
}

// Standalone rotation of [bsz][seqlen][heads][head_dim] in place: each thread
// rotates two interleaved pairs (4 consecutive elements).
template <typename T>
__global__ void rope_apply_kernel(T* __restrict__ x, const float* __restrict__ freqs, int seqlen,
                                  int start_pos, int heads, int head_dim, int64_t total4) {
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total4;
       k += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = k * 4;
    const int c = (int)(e % head_dim);
    const int64_t bs = e / ((int64_t)heads * head_dim);
    const int s = (int)(bs % seqlen);
    const int pos = start_pos + s;
    const f32x4 cs = *(const f32x4*)(freqs + ((int64_t)pos * (head_dim / 2) + c / 2) * 2);
    const f32x4 v = load4(x + e);
    store4(x + e, f32x4{v[0] * cs[0] - v[1] * cs[1], v[0] * cs[1] + v[1] * cs[0],
                        v[2] * cs[2] - v[3] * cs[3], v[2] * cs[3] + v[3] * cs[2]});
  }
}

template <typename T>
__global__ void embedding_kernel(const int32_t* __restrict__ tok, const T* __restrict__ table,
                                 T* __restrict__ out, int64_t n, int dim, int vocab) {
  constexpr int V = Vec<T>::N;
  typedef typename Vec<T>::type vec;
  const int nvec = dim / V;
  const int64_t total = n * nvec;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total;
       k += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = k / nvec;
    const int c = (int)(k % nvec);
    const int id = tok[r];
    vec v = (id >= 0 && id < vocab) ? *(const vec*)(table + (int64_t)id * dim + c * V) : vec{};
    *(vec*)(out + r * dim + c * V) = v;
  }
}

// Greedy token: argmax of a fp32 row, the lowest index among equal maxima.
// 1024 threads per row; VEC: 16-byte loads (vocab % 4 == 0, aligned rows).
constexpr int kArgmaxThreads = 1024;
template <bool VEC>
__global__ void __launch_bounds__(kArgmaxThreads) argmax_kernel(const float* __restrict__ logits,
                                                                int32_t* __restrict__ next, int cols) {
  __shared__ float bv[kArgmaxThreads / 64];
  __shared__ int bi[kArgmaxThreads / 64];
  const float* r = logits + (int64_t)blockIdx.x * cols;
  float best = -INFINITY;
  int idx = 0x7fffffff;
  // each thread visits its columns in increasing order and keeps the first maximum
  if constexpr (VEC) {
    const f32x4* rv = (const f32x4*)r;
    for (int v = threadIdx.x; v < cols / 4; v += kArgmaxThreads) {
      const f32x4 x = rv[v];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (x[e] > best) {
          best = x[e];
          idx = 4 * v + e;
        }
    }
  } else {
    for (int c = threadIdx.x; c < cols; c += kArgmaxThreads) {
      const float v = r[c];
      if (v > best) {
        best = v;
        idx = c;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(best, off, 64);
    int oi = __shfl_xor(idx, off, 64);
    if (ov > best || (ov == best && oi < idx)) {
      best = ov;
      idx = oi;
    }
  }
  if ((threadIdx.x & 63) == 0) {
    bv[threadIdx.x >> 6] = best;
    bi[threadIdx.x >> 6] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kArgmaxThreads / 64; ++i)
      if (bv[i] > best || (bv[i] == best && bi[i] < idx)) {
        best = bv[i];
        idx = bi[i];
      }
    next[blockIdx.x] = idx == 0x7fffffff ? 0 : idx;
  }
}

inline int grid_for(int64_t work, int per_block = kThreads) {
  int64_t b = (work + per_block - 1) / per_block;
  return (int)(b < 1 ? 1 : (b > 16384 ? 16384 : b));
}

}  // namespace

template <typename T>
hipError_t rmsnorm(const T* x, int64_t x_stride, const T* w, T* y, int64_t rows, int dim, float eps,
                   hipStream_t st, float* rscale) {
  if (rows == 0) return hipSuccess;
  rmsnorm_kernel<T><<<(unsigned)rows, kThreads, 0, st>>>(x, x_stride, w, y, dim, eps, rscale);
  return hipGetLastError();
}

hipError_t rope_table(float* freqs, int head_dim, int end, double theta, hipStream_t st) {
  rope_table_kernel<<<grid_for((int64_t)end * head_dim / 2), kThreads, 0, st>>>(freqs, head_dim, end, theta);
  return hipGetLastError();
}

template <typename T>
hipError_t rope_apply(T* x, const float* freqs, int bsz, int seqlen, int start_pos, int heads, int head_dim,
                      hipStream_t st) {
  const int64_t total4 = (int64_t)bsz * seqlen * heads * head_dim / 4;
  if (total4 == 0) return hipSuccess;
  rope_apply_kernel<T><<<grid_for(total4), kThreads, 0, st>>>(x, freqs, seqlen, start_pos, heads, head_dim,
                                                               total4);
  return hipGetLastError();
}

template <typename T>
hipError_t embedding(const int32_t* tok, const T* table, T* out, int64_t n, int dim, int vocab,
                     hipStream_t st) {
  if (n == 0) return hipSuccess;
  embedding_kernel<T><<<grid_for(n * dim / Vec<T>::N), kThreads, 0, st>>>(tok, table, out, n, dim, vocab);
  return hipGetLastError();
}

hipError_t argmax_rows(const float* logits, int32_t* next, int rows, int cols, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (cols % 4 == 0 && (uintptr_t)logits % 16 == 0)
    argmax_kernel<true><<<rows, kArgmaxThreads, 0, st>>>(logits, next, cols);
  else
    argmax_kernel<false><<<rows, kArgmaxThreads, 0, st>>>(logits, next, cols);
  return hipGetLastError();
}

template hipError_t rmsnorm<bf16>(const bf16*, int64_t, const bf16*, bf16*, int64_t, int, float, hipStream_t,
                                  float*);
template hipError_t rmsnorm<float>(const float*, int64_t, const float*, float*, int64_t, int, float, hipStream_t,
                                   float*);
template hipError_t rope_apply<bf16>(bf16*, const float*, int, int, int, int, int, hipStream_t);
template hipError_t rope_apply<float>(float*, const float*, int, int, int, int, int, hipStream_t);
template hipError_t embedding<bf16>(const int32_t*, const bf16*, bf16*, int64_t, int, int, hipStream_t);
template hipError_t embedding<float>(const int32_t*, const float*, float*, int64_t, int, int, hipStream_t);

}  // namespace llama
