// Causal grouped-query attention over the KV cache (prefill and single-token
// decode).  Kernels live in attention.hip.
#pragma once

#include "common.hpp"

namespace llama {

struct AttnShape {
  int bsz, seqlen, start_pos;   // T = start_pos + seqlen keys are attended
  int n_heads, n_kv_heads, head_dim;
  int max_seq;                  // cache row count per batch entry
};

// Append xk/xv ([bsz][seqlen][n_kv_heads][head_dim]) into the caches at
// [b][start_pos + s].
template <typename T>
hipError_t kv_append(const T* xk, const T* xv, T* cache_k, T* cache_v, const AttnShape& sh,
                     hipStream_t st);

// Prefill: out[b][s][h*d..] for q [bsz][seqlen][n_heads][d], keys/values read
// from the caches (already appended).
template <typename T>
hipError_t attn_prefill(const T* q, const T* cache_k, const T* cache_v, T* out,
                        const AttnShape& sh, hipStream_t st);

// Decode (seqlen == 1): split-K over the T keys; `partial` holds
// bsz * n_heads * splits * (head_dim + 2) floats.  With pos_dev set (bf16
// only), the position is *pos_dev, read when the kernel runs and clamped to
// [0, sh.start_pos]; the splits are laid out for T = sh.start_pos + 1 and those
// past the actual length stay empty.
int attn_decode_splits(int bsz, int n_heads, int n_kv_heads, int T);
template <typename T>
hipError_t attn_decode(const T* q, const T* cache_k, const T* cache_v, T* out,
                       const AttnShape& sh, float* partial, hipStream_t st, const int32_t* pos_dev = nullptr);

}  // namespace llama
