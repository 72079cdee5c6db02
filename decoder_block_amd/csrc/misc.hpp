// Elementwise and row kernels of the decoder block (misc.hip): RMSNorm, the
// RoPE table and standalone rotation, embedding gather and greedy argmax.
#pragma once

#include "common.hpp"

namespace llama {

// y = RMSNorm(x) * w.  With rscale != nullptr: y = x * w and rscale[row] =
// rsqrt(mean(x^2) + eps), for a projection that scales its accumulators.
template <typename T>
hipError_t rmsnorm(const T* x, int64_t x_stride, const T* w, T* y, int64_t rows, int dim, float eps,
                   hipStream_t st, float* rscale = nullptr);

hipError_t rope_table(float* freqs, int head_dim, int end, double theta, hipStream_t st);

template <typename T>
hipError_t rope_apply(T* x, const float* freqs, int bsz, int seqlen, int start_pos, int heads,
                      int head_dim, hipStream_t st);

template <typename T>
hipError_t embedding(const int32_t* tok, const T* table, T* out, int64_t n, int dim, int vocab,
                     hipStream_t st);

hipError_t argmax_rows(const float* logits, int32_t* next, int rows, int cols, hipStream_t st);

}  // namespace llama
