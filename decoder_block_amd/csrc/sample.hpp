// Next-token selection from fp32 logits: temperature softmax, nucleus (top-p)
// cut and a draw driven by one caller-supplied uniform number per row
// (sample.hip).
#pragma once

#include "common.hpp"

namespace llama {

// next[r] for rows r < rows of logits [rows][vocab]; temperature > 0.
hipError_t sample_top_p(const float* logits, int32_t* next, int rows, int vocab, float temperature, float top_p,
                        const float* uniforms, hipStream_t st);

}  // namespace llama
