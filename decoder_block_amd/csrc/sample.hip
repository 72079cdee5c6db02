// Next-token selection on the device: temperature softmax + nucleus (top-p)
// cut + draw (linkmax.top LLaMA walkthrough, section 3.3, generate and
// sample_top_p), without sorting the vocabulary.
//
// Order: tokens sorted by descending probability, equal probabilities by
// ascending id.  Each token gets a 64-bit key whose order is that order:
//   key = (float bits of w) << 32 | (0xffffffff - id),  w = exp((l - max l) / T)
// (w is positive, so its float bits order like its value).  With Z = sum w:
//   * a token is kept when the weight strictly before it, F(key) = sum of w
//     over larger keys, is <= top_p * Z;  F falls as the key grows, so the
//     kept set is {key >= k*} with k* the smallest key value where F <= top_p*Z;
//   * the draw takes the kept token whose inclusive prefix I(key) = sum of kept
//     w over keys >= key first exceeds u * (kept sum): the largest key value
//     k_s with I(k_s) > u * S.
// Both boundaries are found digit by digit (16 digits of 4 bits, most
// significant first): one pass over the row per digit sums w into the 16
// sub-ranges of the current range.  Sums are per-thread fp32 in a fixed
// element order and fp64 across the workgroup in a fixed tree, so the result
// is deterministic.
#include "sample.hpp"

#include <math.h>

namespace llama {

namespace {

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / 64;

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sums NB per-thread values over the workgroup (fixed order); every thread
// receives the totals.  `red` holds kSampleWaves * NB doubles.
template <int NB>
__device__ __forceinline__ void block_sums(const double (&v)[NB], double (&out)[NB], double* red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const double s = wave_sum_d(v[b]);
    if (lane == 0) red[wave * NB + b] = s;
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kSampleWaves; ++w) s += red[w * NB + b];
    out[b] = s;
  }
  __syncthreads();
}

__device__ __forceinline__ float block_max(float v, float* redf) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) redf[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < kSampleWaves; ++w) m = fmaxf(m, redf[w]);
  __syncthreads();
  return m;
}

// Visits every element of the row once, in a fixed order per thread: 16-byte
// loads, four in flight per thread (VEC: vocab % 4 == 0 and an aligned row),
// else single floats.
template <bool VEC, class F>
__device__ __forceinline__ void for_each(const float* __restrict__ l, int vocab, F&& f) {
  const int tid = threadIdx.x;
  if constexpr (VEC) {
    const int nv = vocab >> 2;
    const f32x4* lv = (const f32x4*)l;
    constexpr int U = 4;
    for (int b = tid; b < nv; b += U * kSampleThreads) {
      f32x4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = b + u * kSampleThreads;
        x[u] = v < nv ? lv[v] : f32x4{};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = b + u * kSampleThreads;
        if (v < nv) {
#pragma unroll
          for (int e = 0; e < 4; ++e) f(4 * v + e, x[u][e]);
        }
      }
    }
  } else {
    for (int i = tid; i < vocab; i += kSampleThreads) f(i, l[i]);
  }
}

// Smallest id, and count, of the elements whose weight bits equal wb among
// those accepted by `ok` (one pass).
template <bool VEC, class W, class OK>
__device__ __forceinline__ void ties_at(const float* l, int vocab, W&& weight, uint32_t wb, OK&& ok, int* redi,
                                        int& min_id, int& count) {
  int mn = 0x7fffffff, cnt = 0;
  for_each<VEC>(l, vocab, [&](int i, float x) {
    if (__float_as_uint(weight(x)) == wb && ok(i)) {
      mn = min(mn, i);
      ++cnt;
    }
  });
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = min(mn, __shfl_xor(mn, off, 64));
    cnt += __shfl_xor(cnt, off, 64);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    redi[wave] = mn;
    redi[kSampleWaves + wave] = cnt;
  }
  __syncthreads();
  min_id = 0x7fffffff;
  count = 0;
#pragma unroll
  for (int w = 0; w < kSampleWaves; ++w) {
    min_id = min(min_id, redi[w]);
    count += redi[kSampleWaves + w];
  }
  __syncthreads();
}

// The j-th smallest id (j >= 0) among the elements with weight bits wb that `ok`
// accepts, given the smallest (`first`).  Short runs of ties take successive
// minima (one pass each); longer ones a binary search over the id with one
// counting pass per step, so a row of many equal logits costs ~17 passes.
template <bool VEC, class W, class OK>
__device__ __forceinline__ int nth_tie(const float* l, int vocab, W&& weight, uint32_t wb, OK&& ok, int* redi,
                                       int first, int j) {
  if (j <= 2) {
    int id = first;
    for (int r = 0; r < j; ++r) {
      int mn, cnt;
      const int prev = id;
      ties_at<VEC>(l, vocab, weight, wb, [&](int i) { return i > prev && ok(i); }, redi, mn, cnt);
      id = mn;
    }
    return id;
  }
  // smallest x in [first, vocab) with #{ties with id <= x} >= j + 1
  int lo = first, hi = vocab - 1;
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    int mn, cnt;
    ties_at<VEC>(l, vocab, weight, wb, [&](int i) { return i <= mid && ok(i); }, redi, mn, cnt);
    if (cnt >= j + 1)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

template <bool VEC>
__global__ void __launch_bounds__(kSampleThreads)
sample_top_p_kernel(const float* __restrict__ logits, int32_t* __restrict__ next, int vocab, float scale_log2,
                    float top_p, const float* __restrict__ uniforms) {
  __shared__ double red[kSampleWaves * 17];
  __shared__ float redf[kSampleWaves];
  __shared__ int redi[2 * kSampleWaves];
  const int row = blockIdx.x;
  const float* l = logits + (int64_t)row * vocab;

  // max and normaliser in one pass: a running maximum whose sum is rescaled when it grows
  float mloc = -INFINITY, zl = 0.f;
  for_each<VEC>(l, vocab, [&](int, float x) {
    if (x > mloc) {
      zl = zl * exp2f((mloc - x) * scale_log2) + 1.f;
      mloc = x;
    } else {
      zl += exp2f((x - mloc) * scale_log2);
    }
  });
  const float m = block_max(mloc, redf);
  double z;
  {
    double in[1] = {mloc == -INFINITY ? 0.0 : (double)zl * (double)exp2f((mloc - m) * scale_log2)}, out[1];
    block_sums<1>(in, out, red);
    z = out[0];
  }
  // top_p >= 1 keeps every token (no rounding of the two sums may cut the tail)
  const double limit = top_p >= 1.f ? (double)INFINITY : (double)top_p * z;
  auto weight = [&](float x) { return exp2f((x - m) * scale_log2); };

  // ---- the nucleus cut.  First the weight bits wc of the cut's block: the
  // smallest bits b with G(b) = sum of w over larger bits <= limit.
  uint32_t wc = 0;
  double g_c = 0.0;
  for (int shift = 28; shift >= 0; shift -= 4) {
    const uint32_t base = wc >> shift;             // low 4 bits zero
    float above = 0.f, s[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) s[d] = 0.f;
    for_each<VEC>(l, vocab, [&](int, float x) {
      const float w = weight(x);
      const uint32_t hi = __float_as_uint(w) >> shift;
      if (hi >= base + 16) {
        above += w;
      } else if (hi >= base) {
        const int dg = (int)(hi - base);
#pragma unroll
        for (int d = 0; d < 16; ++d) s[d] += d < dg ? w : 0.f;
      }
    });
    double in[16], f[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) in[d] = (double)s[d] + (double)above;
    block_sums<16>(in, f, red);
    // f[d] = G(top of sub-range d); it falls with d and f[15] <= limit holds
    int sel = 15;
#pragma unroll
    for (int d = 14; d >= 0; --d)
      if (f[d] <= limit) sel = d;
    wc |= (uint32_t)sel << shift;
    g_c = f[sel];
  }
  // Within the block, tokens of equal weight follow in ascending id: the j-th
  // has G + j*w before it, so the last kept is j = floor((limit - G) / w),
  // capped by the tie count (w = 0: all of them).
  const double w_c = (double)__uint_as_float(wc);
  int cut_id, n_c;
  {
    int mn;
    ties_at<VEC>(l, vocab, weight, wc, [](int) { return true; }, redi, mn, n_c);
    const double room = limit - g_c;
    if (w_c == 0.0 || room >= (double)(n_c - 1) * w_c) {
      cut_id = 0x7fffffff;                         // the whole block is kept
    } else {
      const int j = max(0, (int)floor(room / w_c));
      cut_id = nth_tie<VEC>(l, vocab, weight, wc, [](int) { return true; }, redi, mn, j);
      n_c = j + 1;                                 // kept tokens of the cut block
    }
  }
  // kept: weight bits > wc, or == wc with id <= cut_id
  auto kept_tok = [&](int i, uint32_t b) { return b > wc || (b == wc && i <= cut_id); };
  const double kept = g_c + (double)n_c * w_c;
  const double target = (double)uniforms[row] * kept;

  // ---- the draw.  The weight bits ws of the drawn token's block: the largest
  // bits b with H(b) = kept weight at bits >= b exceeding the target.
  uint32_t wsel = 0;
  double h_above = 0.0;                            // kept weight at bits > wsel
  for (int shift = 28; shift >= 0; shift -= 4) {
    const uint32_t base = wsel >> shift;
    float above = 0.f, s[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) s[d] = 0.f;
    for_each<VEC>(l, vocab, [&](int i, float x) {
      const float w = weight(x);
      const uint32_t b = __float_as_uint(w);
      if (!kept_tok(i, b)) return;
      const uint32_t hi = b >> shift;
      if (hi >= base + 16) {
        above += w;
      } else if (hi >= base) {
        const int dg = (int)(hi - base);
#pragma unroll
        for (int d = 0; d < 16; ++d) s[d] += d <= dg ? w : 0.f;
      }
    });
    double in[17], inc[17];
#pragma unroll
    for (int d = 0; d < 16; ++d) in[d] = (double)s[d] + (double)above;
    in[16] = (double)above;
    block_sums<17>(in, inc, red);
    // inc[d] = H(bottom of sub-range d) falls with d, inc[0] > target holds,
    // and inc[16] = H(top of the range + 1)
    int sel = 0;
#pragma unroll
    for (int d = 1; d < 16; ++d)
      if (inc[d] > target) sel = d;
    wsel |= (uint32_t)sel << shift;
    h_above = inc[sel + 1];
  }
  // Within the block the j-th kept token of equal weight (ascending id) ends its
  // cumulative interval at H_above + (j + 1) * w: the first to pass the target.
  const double w_s = (double)__uint_as_float(wsel);
  int mn, n_s;
  ties_at<VEC>(l, vocab, weight, wsel, [&](int i) { return kept_tok(i, wsel); }, redi, mn, n_s);
  int j = 0;
  if (w_s > 0.0) j = min(max(n_s - 1, 0), max(0, (int)floor((target - h_above) / w_s)));
  const int tok = nth_tie<VEC>(l, vocab, weight, wsel, [&](int i) { return kept_tok(i, wsel); }, redi, mn, j);
  if (threadIdx.x == 0) next[row] = tok;
}

}  // namespace

hipError_t sample_top_p(const float* logits, int32_t* next, int rows, int vocab, float temperature, float top_p,
                        const float* uniforms, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const float scale_log2 = 1.4426950408889634f / temperature;
  if (vocab % 4 == 0 && (uintptr_t)logits % 16 == 0)
    sample_top_p_kernel<true><<<rows, kSampleThreads, 0, st>>>(logits, next, vocab, scale_log2, top_p, uniforms);
  else
    sample_top_p_kernel<false><<<rows, kSampleThreads, 0, st>>>(logits, next, vocab, scale_log2, top_p, uniforms);
  return hipGetLastError();
}

}  // namespace llama
