// Projections at small token counts (M <= 4 rows, bf16 or fp32): y[m][n] = epi(sum_k A[m][k] W[n][k]).
//
// With one to four tokens every weight element is used at most four times, so
// the projection is a stream of the weight matrix from HBM and nothing else
// matters: no MFMA tiles, no LDS staging, no split-K partials.  A workgroup owns
// four consecutive output columns (four weight rows, eight for the w1/w3 pair)
// and its waves split K: of NW waves, wave w reads the chunks w, w+NW, ...
// (512 elements in bf16, 256 in fp32), each lane loading 16 bytes of every row,
// so one load instruction covers 1 KiB of a row contiguously.  Lane partial
// sums are folded over the wave with shuffles and over the waves through LDS;
// one thread per token row then applies the fused epilogue to its four columns
// (the same epilogues the MFMA kernels use: RoPE + cache append, SwiGLU,
// residual add).
//
// With norm_w set, A is the un-normalised block input and the kernel applies
// RMSNorm on the fly (LLaMA notes, section 3, class RMSNorm): the products use
// A * norm_w and the row factor rsqrt(mean(A^2) + eps) scales the fp32
// accumulators, with the sum of squares taken from the same A loads.  The
// decode step then needs no separate normalisation pass.
#include "gemm.hpp"

namespace llama {

namespace {

constexpr int kGvCols = 4;            // output columns per workgroup

// 16-byte vectors of the element type
template <typename T> struct GvVec;
template <> struct GvVec<bf16> {
  typedef bf16x8 type;
  static constexpr int N = 8;
  static __device__ __forceinline__ type stream(const bf16* p) { return load_stream8(p); }
};
template <> struct GvVec<float> {
  typedef f32x4 type;
  static constexpr int N = 4;
  static __device__ __forceinline__ type stream(const float* p) {
    return __builtin_nontemporal_load((const f32x4*)p);
  }
};
template <typename T>
constexpr int gv_chunk() { return kWave * GvVec<T>::N; }   // k elements of one 16-byte load per lane

template <int M, int NR, bool NORM>
struct GvAcc {
  float acc[M][NR];
  float ss[M];
};

// Accumulates U chunks (c, c + NW, ...), all inside [0, nch).  Lanes past
// the end of K (the last chunk of a ragged K) read a valid address and
// contribute zeros.
template <typename T, int M, int NR, bool NORM, int U, int NW>
__device__ __forceinline__ void gv_chunks(GvAcc<M, NR, NORM>& a, const T* const (&wr)[NR],
                                          const T* __restrict__ A, int64_t lda,
                                          const T* __restrict__ norm_w, int K, int c, int lane) {
  typedef typename GvVec<T>::type vec;
  constexpr int EL = GvVec<T>::N;
  vec wv[U][NR];
  vec xv[U][M];
  vec gv[U];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int k = (c + u * NW) * gv_chunk<T>() + lane * EL;
    ok[u] = k < K;
    k = ok[u] ? k : 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) wv[u][r] = GvVec<T>::stream(wr[r] + k);
#pragma unroll
    for (int m = 0; m < M; ++m) xv[u][m] = *(const vec*)(A + m * lda + k);
    if constexpr (NORM) gv[u] = *(const vec*)(norm_w + k);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float xf[EL];
#pragma unroll
      for (int i = 0; i < EL; ++i) xf[i] = ok[u] ? (float)xv[u][m][i] : 0.0f;
      if constexpr (NORM) {
#pragma unroll
        for (int i = 0; i < EL; ++i) {
          a.ss[m] += xf[i] * xf[i];
          xf[i] *= (float)gv[u][i];
        }
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int i = 0; i < EL; ++i) a.acc[m][r] += xf[i] * (float)wv[u][r][i];
      }
    }
  }
}

template <typename T, int M, int NW, bool DUAL, bool NORM, class Epi>
__global__ void __launch_bounds__(NW * kWave)
gemv_kernel(const T* __restrict__ A, int64_t lda, WeightRows<T> w, int K, const T* __restrict__ norm_w,
            float eps, Epi epi) {
  constexpr int NR = DUAL ? 2 * kGvCols : kGvCols;   // weight rows streamed
  constexpr int U = DUAL ? 1 : 2;                     // chunks in flight: 8 row loads per lane
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int n0 = blockIdx.x * kGvCols;
  const T* wr[NR];
  if constexpr (DUAL) {
#pragma unroll
    for (int r = 0; r < kGvCols; ++r) {
      wr[r] = w.w0 + (int64_t)(n0 + r) * K;
      wr[kGvCols + r] = w.w1 + (int64_t)(n0 + r) * K;
    }
  } else {
    // n1 and n2 are multiples of four: the four rows lie in one matrix
    const T* base = n0 < w.n1 ? w.w0 + (int64_t)n0 * K
                                 : (n0 < w.n2 ? w.w1 + (int64_t)(n0 - w.n1) * K : w.w2 + (int64_t)(n0 - w.n2) * K);
#pragma unroll
    for (int r = 0; r < NR; ++r) wr[r] = base + (int64_t)r * K;
  }

  GvAcc<M, NR, NORM> a;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    a.ss[m] = 0.0f;
#pragma unroll
    for (int r = 0; r < NR; ++r) a.acc[m][r] = 0.0f;
  }
  const int nch = (K + gv_chunk<T>() - 1) / gv_chunk<T>();
  int c = wave;
  for (; c + (U - 1) * NW < nch; c += U * NW) gv_chunks<T, M, NR, NORM, U, NW>(a, wr, A, lda, norm_w, K, c, lane);
  if constexpr (U > 1) {
    for (; c < nch; c += NW) gv_chunks<T, M, NR, NORM, 1, NW>(a, wr, A, lda, norm_w, K, c, lane);
  }

  __shared__ float red[NW][M][NR + 1];
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float v = wave_sum(a.acc[m][r]);
      if (lane == 0) red[wave][m][r] = v;
    }
    if constexpr (NORM) {
      const float v = wave_sum(a.ss[m]);
      if (lane == 0) red[wave][m][NR] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x < M) {
    const int m = threadIdx.x;
    float s[NR + 1];
#pragma unroll
    for (int j = 0; j <= NR; ++j) {
      s[j] = red[0][m][j];
#pragma unroll
      for (int v = 1; v < NW; ++v) s[j] += red[v][m][j];
    }
    const float rr = NORM ? 1.0f / sqrtf(s[NR] / (float)K + eps) : 1.0f;
    const f32x4 a1 = f32x4{s[0], s[1], s[2], s[3]} * rr;
    if constexpr (DUAL)
      epi(m, n0, a1, f32x4{s[4], s[5], s[6], s[7]} * rr);
    else
      epi(m, n0, a1);
  }
}

template <typename T, int NW, bool DUAL, bool NORM, class Epi>
hipError_t gv_launch_nw(const T* A, int64_t lda, WeightRows<T> w, int M, int N, int K, const T* norm_w,
                        float eps, Epi epi, hipStream_t st) {
  const dim3 grid(N / kGvCols), block(NW * kWave);
  switch (M) {
    case 1: gemv_kernel<T, 1, NW, DUAL, NORM, Epi><<<grid, block, 0, st>>>(A, lda, w, K, norm_w, eps, epi); break;
    case 2: gemv_kernel<T, 2, NW, DUAL, NORM, Epi><<<grid, block, 0, st>>>(A, lda, w, K, norm_w, eps, epi); break;
    case 3: gemv_kernel<T, 3, NW, DUAL, NORM, Epi><<<grid, block, 0, st>>>(A, lda, w, K, norm_w, eps, epi); break;
    case 4: gemv_kernel<T, 4, NW, DUAL, NORM, Epi><<<grid, block, 0, st>>>(A, lda, w, K, norm_w, eps, epi); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Four waves per workgroup, or eight when the grid is small (under 2048
// workgroups, e.g. 4096 output columns): the extra waves keep more weight
// loads in flight per CU.
template <typename T, bool DUAL, bool NORM, class Epi>
hipError_t gv_launch(const T* A, int64_t lda, WeightRows<T> w, int M, int N, int K, const T* norm_w,
                     float eps, Epi epi, hipStream_t st) {
  if (N / kGvCols < 2048 && K > 4 * gv_chunk<T>())
    return gv_launch_nw<T, 8, DUAL, NORM>(A, lda, w, M, N, K, norm_w, eps, epi, st);
  return gv_launch_nw<T, 4, DUAL, NORM>(A, lda, w, M, N, K, norm_w, eps, epi, st);
}

}  // namespace

template <typename T>
bool gemv_fits(int M, int N, int K, int64_t lda) {
  constexpr int EL = 16 / sizeof(T);
  return M >= 1 && M <= kGemvMaxM && N > 0 && N % kGvCols == 0 && K > 0 && K % EL == 0 && lda % EL == 0;
}

template <typename T, class Epi>
hipError_t gemv_launch(const T* A, int64_t lda, WeightRows<T> w, int M, int N, int K, const T* norm_w, float eps,
                       Epi epi, hipStream_t st) {
  if (!gemv_fits<T>(M, N, K, lda) || w.n1 % kGvCols || w.n2 % kGvCols) return hipErrorInvalidValue;
  if (norm_w) return gv_launch<T, false, true>(A, lda, w, M, N, K, norm_w, eps, epi, st);
  return gv_launch<T, false, false>(A, lda, w, M, N, K, norm_w, eps, epi, st);
}

template <typename T, class Epi>
hipError_t gemv_dual_launch(const T* A, int64_t lda, const T* w1, const T* w3, int M, int N, int K,
                            const T* norm_w, float eps, Epi epi, hipStream_t st) {
  if (!gemv_fits<T>(M, N, K, lda)) return hipErrorInvalidValue;
  WeightRows<T> w{w1, w3, nullptr, N, N};
  if (norm_w) return gv_launch<T, true, true>(A, lda, w, M, N, K, norm_w, eps, epi, st);
  return gv_launch<T, true, false>(A, lda, w, M, N, K, norm_w, eps, epi, st);
}

#define LLAMA_GEMV_INST(T)                                                                                        \
  template bool gemv_fits<T>(int, int, int, int64_t);                                                            \
  template hipError_t gemv_launch<T, EpiStore<T>>(const T*, int64_t, WeightRows<T>, int, int, int, const T*, float, \
                                                  EpiStore<T>, hipStream_t);                                     \
  template hipError_t gemv_launch<T, EpiResidual<T>>(const T*, int64_t, WeightRows<T>, int, int, int, const T*,   \
                                                     float, EpiResidual<T>, hipStream_t);                        \
  template hipError_t gemv_launch<T, EpiQKV<T>>(const T*, int64_t, WeightRows<T>, int, int, int, const T*, float, \
                                                EpiQKV<T>, hipStream_t);                                         \
  template hipError_t gemv_dual_launch<T, EpiSwiGLU<T>>(const T*, int64_t, const T*, const T*, int, int, int,     \
                                                        const T*, float, EpiSwiGLU<T>, hipStream_t);

LLAMA_GEMV_INST(bf16)
LLAMA_GEMV_INST(float)
template hipError_t gemv_launch<bf16, EpiF32>(const bf16*, int64_t, WeightRows<bf16>, int, int, int, const bf16*,
                                              float, EpiF32, hipStream_t);
template hipError_t gemv_launch<float, EpiF32>(const float*, int64_t, WeightRows<float>, int, int, int, const float*,
                                               float, EpiF32, hipStream_t);

}  // namespace llama
