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
// Both boundaries are found digit by digit (8 digits of 4 bits, most
// significant first): one pass per digit sums w into the 16 sub-ranges of the
// current range.  After three digits the elements left in the range are copied
// into LDS and the remaining digits read that list instead of the row.  Sums
// are per-thread fp32 in a fixed element order (each thread owns its LDS
// slots) and fp64 across the workgroup in a fixed order, so the result is
// deterministic.
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

// Per-thread partial sums of one digit pass, in LDS: slot b of thread t at
// slot[b * kSampleThreads + t], b < 16 the sub-ranges of the digit, b = 16 the
// weight above the range, b = 17 a discard slot for elements outside (never
// summed).  Each slot has one owner, which updates it with plain LDS reads and
// writes, so its sum is taken in element order.
constexpr int kBins = 17;                             // summed slots
constexpr uint32_t kDiscard = 17;
constexpr int kSlots = 18;
static_assert(kSampleWaves == 16, "one wave per sub-range in bin_totals");

// Slot of an element whose shifted weight bits are hi, in the range starting at
// base.  The difference and its clamp are taken unconditionally (wrapping when
// hi < base) and the range test selects afterwards: written as a guarded
// min(hi - base, 16), the optimiser marks the guarded subtraction no-wrap,
// hoists it out of the guard with the flag kept, and then folds the range test
// away from that flag.
__device__ __forceinline__ uint32_t slot_of(bool in, uint32_t hi, uint32_t base) {
  const uint32_t d = hi - base;
  const uint32_t c = d < 16u ? d : 16u;
  const bool keep = in & (hi >= base);
  return keep ? c : kDiscard;
}

// Adds w[e] to this thread's slot b[e], e = 0..3 in order.  The four slots are
// read at once and equal slots chained in registers, so one LDS round trip
// serves four elements; of repeated writes to one slot the last, which holds
// every earlier addition, lands last (LDS keeps a wave's order).
__device__ __forceinline__ void slot_add4(float* slot, const uint32_t (&b)[4], const float (&w)[4]) {
  float* my = slot + threadIdx.x;
  float r[4], v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = my[b[e] * kSampleThreads];
  v[0] = r[0] + w[0];
  v[1] = (b[1] == b[0] ? v[0] : r[1]) + w[1];
  v[2] = (b[2] == b[1] ? v[1] : b[2] == b[0] ? v[0] : r[2]) + w[2];
  v[3] = (b[3] == b[2] ? v[2] : b[3] == b[1] ? v[1] : b[3] == b[0] ? v[0] : r[3]) + w[3];
#pragma unroll
  for (int e = 0; e < 4; ++e) my[b[e] * kSampleThreads] = v[e];
}

// Workgroup totals of the slots (fp64, fixed order: wave w sums sub-range w),
// returned to every thread as suffix sums S[d] = slots d..16 (S[16] = the weight
// above the range).  Clears the slots for the next pass.  `part` holds 2 *
// kSampleWaves doubles.
__device__ __forceinline__ void bin_totals(float* slot, double* part, double (&S)[kBins]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int k = 0; k < kSampleWaves; ++k) {
    float* p = slot + wave * kSampleThreads + k * 64 + lane;
    t += (double)*p;
    *p = 0.f;
  }
  float* q = slot + 16 * kSampleThreads + threadIdx.x;
  double a = (double)*q;
  *q = 0.f;
  t = wave_sum_d(t);
  a = wave_sum_d(a);
  if (lane == 0) {
    part[wave] = t;
    part[kSampleWaves + wave] = a;
  }
  __syncthreads();
  double run = 0.0;
#pragma unroll
  for (int w = 0; w < kSampleWaves; ++w) run += part[kSampleWaves + w];
  S[16] = run;
#pragma unroll
  for (int d = 15; d >= 0; --d) {
    run += part[d];
    S[d] = run;
  }
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

// Visits every element of the row once, in a fixed order per thread, four at a
// time: f(id[4], x[4], valid[4]).  VEC (vocab % 4 == 0 and an aligned row):
// 16-byte loads, four in flight per thread; else single floats.
template <bool VEC, class F>
__device__ __forceinline__ void for_each4(const float* __restrict__ l, int vocab, F&& f) {
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
          const int id[4] = {4 * v, 4 * v + 1, 4 * v + 2, 4 * v + 3};
          const float xs[4] = {x[u][0], x[u][1], x[u][2], x[u][3]};
          const bool ok[4] = {true, true, true, true};
          f(id, xs, ok);
        }
      }
    }
  } else {
    for (int i = tid; i < vocab; i += 4 * kSampleThreads) {
      int id[4];
      float xs[4];
      bool ok[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        id[e] = i + e * kSampleThreads;
        ok[e] = id[e] < vocab;
        xs[e] = ok[e] ? l[id[e]] : 0.f;
      }
      f(id, xs, ok);
    }
  }
}

template <bool VEC, class F>
__device__ __forceinline__ void for_each(const float* __restrict__ l, int vocab, F&& f) {
  for_each4<VEC>(l, vocab, [&](const int(&id)[4], const float(&x)[4], const bool(&ok)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (ok[e]) f(id[e], x[e]);
  });
}

// Candidate list in LDS: after the first digits, the elements still inside the
// search range are copied here (per wave, in a fixed order), and the remaining
// digits and the tie resolution read the list instead of the row.
constexpr int kCandSeg = 512;                         // entries per wave
constexpr int kCandCap = kCandSeg * kSampleWaves;     // 8192 entries, 64 KiB
constexpr int kCompactShift = 20;                     // compaction after the digits at 28, 24, 20

struct Cand {
  float* w;
  int* id;
  int* count;                                         // per wave
};

// Smallest id and count of the elements with weight bits wb that `ok` accepts
// (one visit).
template <class V, class OK>
__device__ __forceinline__ void ties_at(V&& visit, uint32_t wb, OK&& ok, int* redi, int& min_id, int& count) {
  int mn = 0x7fffffff, cnt = 0;
  visit([&](int i, float w) {
    if (__float_as_uint(w) == wb && ok(i)) {
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
// minima (one visit each); longer ones a binary search over the id with one
// counting visit per step, so a row of many equal logits costs ~17 visits.
template <class V, class OK>
__device__ __forceinline__ int nth_tie(V&& visit, int vocab, uint32_t wb, OK&& ok, int* redi, int first, int j) {
  if (j <= 2) {
    int id = first;
    for (int r = 0; r < j; ++r) {
      int mn, cnt;
      const int prev = id;
      ties_at(visit, wb, [&](int i) { return i > prev && ok(i); }, redi, mn, cnt);
      id = mn;
    }
    return id;
  }
  // smallest x in [first, vocab) with #{ties with id <= x} >= j + 1
  int lo = first, hi = vocab - 1;
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    int mn, cnt;
    ties_at(visit, wb, [&](int i) { return i <= mid && ok(i); }, redi, mn, cnt);
    if (cnt >= j + 1)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// Copies the row's elements with pred(i, w) into the candidate list (each wave
// appends in element order, lanes in order: a fixed order).  Returns false when
// a wave's segment overflows (the caller then keeps reading the row).
template <bool VEC, class W, class P>
__device__ __forceinline__ bool compact(const float* __restrict__ l, int vocab, W&& weight, P&& pred, Cand c,
                                        int* redi) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int cnt = 0;
  auto take = [&](int i, bool valid, float x) {
    const bool t = valid && pred(i, weight(x));
    const uint64_t mask = __ballot(t);
    const int pos = cnt + __popcll(mask & lt);
    if (t && pos < kCandSeg) {
      c.w[wave * kCandSeg + pos] = weight(x);
      c.id[wave * kCandSeg + pos] = i;
    }
    cnt += __popcll(mask);
  };
  if constexpr (VEC) {
    const int nv = vocab >> 2;
    const f32x4* lv = (const f32x4*)l;
    const int iters = (nv + kSampleThreads - 1) / kSampleThreads;
    for (int k = 0; k < iters; ++k) {
      const int v = tid + k * kSampleThreads;
      const bool valid = v < nv;
      const f32x4 x = valid ? lv[v] : f32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) take(4 * v + e, valid, x[e]);
    }
  } else {
    const int iters = (vocab + kSampleThreads - 1) / kSampleThreads;
    for (int k = 0; k < iters; ++k) {
      const int i = tid + k * kSampleThreads;
      const bool valid = i < vocab;
      take(i, valid, valid ? l[i] : 0.f);
    }
  }
  if (lane == 0) {
    c.count[wave] = min(cnt, kCandSeg);
    redi[wave] = cnt > kCandSeg;
  }
  __syncthreads();                                   // (also publishes the list)
  bool ok = true;
#pragma unroll
  for (int w = 0; w < kSampleWaves; ++w) ok = ok && !redi[w];
  __syncthreads();
  return ok;
}

template <bool VEC>
__global__ void __launch_bounds__(kSampleThreads)
sample_top_p_kernel(const float* __restrict__ logits, int32_t* __restrict__ next, int vocab, float scale_log2,
                    float top_p, const float* __restrict__ uniforms) {
  __shared__ double red[kSampleWaves];
  __shared__ double part[2 * kSampleWaves];
  __shared__ float slot[kSlots * kSampleThreads];
  __shared__ float redf[kSampleWaves];
  __shared__ int redi[2 * kSampleWaves];
  __shared__ float cand_w[kCandCap];
  __shared__ int cand_id[kCandCap];
  __shared__ int cand_n[kSampleWaves];
  const Cand cand{cand_w, cand_id, cand_n};
  for (int b = 0; b < kSlots; ++b) slot[b * kSampleThreads + threadIdx.x] = 0.f;
  const int row = blockIdx.x;
  const float* l = logits + (int64_t)row * vocab;

  // max and normaliser in one pass: a running maximum whose sum is rescaled when it grows
  float mloc = -INFINITY, zl = 0.f;
  for_each<VEC>(l, vocab, [&](int, float x) {
    if (x > mloc) {
      zl = zl * __builtin_amdgcn_exp2f((mloc - x) * scale_log2) + 1.f;
      mloc = x;
    } else {
      zl += __builtin_amdgcn_exp2f((x - mloc) * scale_log2);
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
  // hardware exp2 (v_exp_f32): the argument is <= 0, weights far below 2^-126 read as 0
  auto weight = [&](float x) { return __builtin_amdgcn_exp2f((x - m) * scale_log2); };
  // the two element sources, four elements at a time: the whole row, or the
  // candidate list of this wave
  auto row_visit4 = [&](auto&& f) {
    for_each4<VEC>(l, vocab, [&](const int(&id)[4], const float(&x)[4], const bool(&ok)[4]) {
      const float w[4] = {weight(x[0]), weight(x[1]), weight(x[2]), weight(x[3])};
      f(id, w, ok);
    });
  };
  auto list_visit4 = [&](auto&& f) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = cand_n[wave];
    const int* ids = cand_id + wave * kCandSeg;
    const float* ws = cand_w + wave * kCandSeg;
    for (int e0 = lane; e0 < n; e0 += 256) {
      int id[4];
      float w[4];
      bool ok[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = e0 + 64 * e;
        ok[e] = k < n;
        id[e] = ok[e] ? ids[k] : 0;
        w[e] = ok[e] ? ws[k] : 0.f;
      }
      f(id, w, ok);
    }
  };
  auto one_by_one = [](auto&& visit4) {
    return [&visit4](auto&& f) {
      visit4([&](const int(&id)[4], const float(&w)[4], const bool(&ok)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (ok[e]) f(id[e], w[e]);
      });
    };
  };
  auto row_visit = one_by_one(row_visit4);
  auto list_visit = one_by_one(list_visit4);

  // ---- the nucleus cut.  First the weight bits wc of the cut's block: the
  // smallest bits b with G(b) = sum of w over larger bits <= limit.  `extra` is
  // the weight above the visited elements' range (0 for the whole row).
  uint32_t wc = 0;
  double g_c = 0.0;
  auto cut_digits = [&](auto&& visit4, double extra, int from, int to) {
    for (int shift = from; shift >= to; shift -= 4) {
      const uint32_t base = wc >> shift;           // low 4 bits zero
      visit4([&](const int(&)[4], const float(&w)[4], const bool(&ok)[4]) {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          b[e] = slot_of(ok[e], __float_as_uint(w[e]) >> shift, base);
        }
        slot_add4(slot, b, w);
      });
      double S[kBins];
      bin_totals(slot, part, S);
      // G(top of sub-range d) = S[d + 1] + extra falls with d; G(top of 15) <= limit holds
      int sel = 15;
      double g = S[16] + extra;
#pragma unroll
      for (int d = 14; d >= 0; --d)
        if (S[d + 1] + extra <= limit) {
          sel = d;
          g = S[d + 1] + extra;
        }
      wc |= (uint32_t)sel << shift;
      g_c = g;
    }
  };
  cut_digits(row_visit4, 0.0, 28, kCompactShift);
  // the weight above the listed range is g_c, the weight above the selected sub-range
  const uint32_t pc = wc >> kCompactShift;
  const bool listed = compact<VEC>(
      l, vocab, weight, [&](int, float w) { return (__float_as_uint(w) >> kCompactShift) == pc; }, cand, redi);
  // Within the block, tokens of equal weight follow in ascending id: the j-th
  // has G + j*w before it, so the last kept is j = floor((limit - G) / w),
  // capped by the tie count (w = 0: all of them).
  int cut_id, n_c;
  auto finish_cut = [&](auto&& visit) {
    int mn;
    ties_at(visit, wc, [](int) { return true; }, redi, mn, n_c);
    const double w_c = (double)__uint_as_float(wc);
    const double room = limit - g_c;
    if (w_c == 0.0 || room >= (double)(n_c - 1) * w_c) {
      cut_id = 0x7fffffff;                         // the whole block is kept
    } else {
      const int j = max(0, (int)floor(room / w_c));
      cut_id = nth_tie(visit, vocab, wc, [](int) { return true; }, redi, mn, j);
      n_c = j + 1;                                 // kept tokens of the cut block
    }
  };
  if (listed) {
    cut_digits(list_visit4, g_c, kCompactShift - 4, 0);
    finish_cut(list_visit);
  } else {
    cut_digits(row_visit4, 0.0, kCompactShift - 4, 0);
    finish_cut(row_visit);
  }
  // kept: weight bits > wc, or == wc with id <= cut_id
  auto kept_tok = [&](int i, uint32_t b) { return b > wc || (b == wc && i <= cut_id); };
  const double kept = g_c + (double)n_c * (double)__uint_as_float(wc);
  const double target = (double)uniforms[row] * kept;

  // ---- the draw.  The weight bits ws of the drawn token's block: the largest
  // bits b with H(b) = kept weight at bits >= b exceeding the target.
  uint32_t wsel = 0;
  double h_above = 0.0;                            // kept weight at bits > wsel
  auto draw_digits = [&](auto&& visit4, double extra, int from, int to) {
    for (int shift = from; shift >= to; shift -= 4) {
      const uint32_t base = wsel >> shift;
      visit4([&](const int(&id)[4], const float(&w)[4], const bool(&ok)[4]) {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t bits = __float_as_uint(w[e]);
          b[e] = slot_of(ok[e] && kept_tok(id[e], bits), bits >> shift, base);
        }
        slot_add4(slot, b, w);
      });
      double S[kBins];
      bin_totals(slot, part, S);
      // H(bottom of sub-range d) = S[d] + extra falls with d; H(bottom of 0) > target holds
      int sel = 0;
      double h = S[1] + extra;
#pragma unroll
      for (int d = 1; d < 16; ++d)
        if (S[d] + extra > target) {
          sel = d;
          h = S[d + 1] + extra;
        }
      wsel |= (uint32_t)sel << shift;
      h_above = h;
    }
  };
  draw_digits(row_visit4, 0.0, 28, kCompactShift);
  const uint32_t pd = wsel >> kCompactShift;
  const bool listed2 = compact<VEC>(
      l, vocab, weight,
      [&](int i, float w) { return kept_tok(i, __float_as_uint(w)) && (__float_as_uint(w) >> kCompactShift) == pd; },
      cand, redi);
  // Within the block the j-th kept token of equal weight (ascending id) ends its
  // cumulative interval at H_above + (j + 1) * w: the first to pass the target.
  auto finish_draw = [&](auto&& visit) {
    const double w_s = (double)__uint_as_float(wsel);
    int mn, n_s;
    ties_at(visit, wsel, [&](int i) { return kept_tok(i, wsel); }, redi, mn, n_s);
    int j = 0;
    if (w_s > 0.0) j = min(max(n_s - 1, 0), max(0, (int)floor((target - h_above) / w_s)));
    return nth_tie(visit, vocab, wsel, [&](int i) { return kept_tok(i, wsel); }, redi, mn, j);
  };
  int tok;
  if (listed2) {
    draw_digits(list_visit4, h_above, kCompactShift - 4, 0);
    tok = finish_draw(list_visit);
  } else {
    draw_digits(row_visit4, 0.0, kCompactShift - 4, 0);
    tok = finish_draw(row_visit);
  }
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
