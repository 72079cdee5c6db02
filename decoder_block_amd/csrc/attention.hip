// Causal grouped-query attention for gfx950.
//
// Definition (LLaMA notes, section 3, Attention.forward; causal mask with cache
// offset from "灵哥讲llama3(中)", Transformer forward): for query head h at
// sequence index s, kv head j = h / n_rep, keys t <= start_pos + s:
//     o = sum_t softmax_t(q . k_t / sqrt(d)) v_t.
// The kernels compute it as an exact rearrangement: scores in fp32, a running
// (max, sum) online softmax in the log2 domain, probabilities rounded to bf16
// only as the operand of the P.V contraction.
//
// Prefill (bf16): one workgroup owns 128 query rows = G heads of one kv group
// x 128/G positions, so each K/V tile is staged in LDS once and used by all G
// heads (GQA sharing).  Key tiles entirely above the causal diagonal of the
// block are never loaded, and the mask is evaluated only on tiles that meet
// the diagonal.  S^T = K.Q^T and O^T = V^T.P^T on v_mfma_f32_32x32x16_bf16 put
// one query row per lane column, so the row max/sum need one cross-half
// exchange only, and the probabilities feed the second MFMA straight from
// registers (the V^T operand is read with transposing LDS loads whose key
// order matches the accumulator layout).
//
// Decode (bf16): split-K over keys.  Each wave streams chunks of 32 keys from
// HBM (K straight into MFMA operand registers, V through a wave-private
// transposed LDS tile), keeps its own online-softmax state for all n_rep heads
// of the kv group (padded to 16 on v_mfma_f32_16x16x32_bf16), the four waves
// merge in LDS and each split writes (max, sum, o) partials that a second
// kernel combines with log-sum-exp weights.
//
// f32: one wavefront per (b, s, h) with scalar online softmax (small shapes).
#include "attention.hpp"

#include <algorithm>
#include <type_traits>

#include <math.h>

namespace llama {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// K/V bytes per group of sequences in prefill attention: three quarters of the
// 256 MB Infinity Cache (measured on the 32-layer batch-64 prefill, 537 MB of
// K/V per layer: 1678 -> 1647 ms against one group; 96 MB groups: 1643 ms, but
// they split the 134 MB batch of the 7B shape and slowed it by 10 %)
constexpr int64_t kPrefillKvGroupBytes = (int64_t)192 << 20;
// decode workgroups resident at once: 4 waves each, 2 waves per SIMD (the
// kernel's register budget), 4 SIMDs per CU, 256 CUs
constexpr int kResidentDecodeWgs = 2 * 256;

// ------------------------------------------------------------------ KV append
template <typename T>
__global__ void kv_append_kernel(const T* __restrict__ xk, const T* __restrict__ xv, T* __restrict__ ck,
                                 T* __restrict__ cv, AttnShape sh) {
  const int row = sh.n_kv_heads * sh.head_dim;  // elements per (b, position)
  const int64_t total4 = (int64_t)sh.bsz * sh.seqlen * row / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total4;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t e = i * 4;
    int64_t bs = e / row;
    int c = (int)(e - bs * row);
    int b = (int)(bs / sh.seqlen), s = (int)(bs - (int64_t)b * sh.seqlen);
    int64_t dst = ((int64_t)b * sh.max_seq + sh.start_pos + s) * row + c;
    store4(ck + dst, load4(xk + e));
    store4(cv + dst, load4(xv + e));
  }
}

// ------------------------------------------------------------------ simple (f32)
template <typename T>
__global__ void __launch_bounds__(256) attn_simple(const T* __restrict__ q, const T* __restrict__ ck,
                                                   const T* __restrict__ cv, T* __restrict__ out,
                                                   AttnShape sh, float scale) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H = sh.n_heads, HD = sh.head_dim, S = sh.seqlen;
  if (wid >= (int64_t)sh.bsz * S * H) return;
  const int h = (int)(wid % H);
  const int64_t bs = wid / H;
  const int b = (int)(bs / S), s = (int)(bs % S);
  const int n_rep = H / sh.n_kv_heads;
  const int j = h / n_rep;
  const T* qr = q + bs * (int64_t)H * HD + (int64_t)h * HD;
  const bool has0 = lane < HD, has1 = lane + 64 < HD;
  const float q0 = has0 ? to_f(qr[lane]) : 0.f;
  const float q1 = has1 ? to_f(qr[lane + 64]) : 0.f;
  const int64_t stride = (int64_t)sh.n_kv_heads * HD;
  const T* kb = ck + ((int64_t)b * sh.max_seq * sh.n_kv_heads + j) * HD;
  const T* vb = cv + ((int64_t)b * sh.max_seq * sh.n_kv_heads + j) * HD;
  const int kend = sh.start_pos + s + 1;
  // Keys in blocks of U: the block's K and V rows are all loaded before any is
  // used (a key at a time would wait out one memory latency per key), the U
  // scores are reduced over the wave independently, and the running (max, sum,
  // o) moves once per block.  Keys past the end are clamped for the loads and
  // weigh 0.
  constexpr int U = 8;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int t0 = 0; t0 < kend; t0 += U) {
    float k0[U], k1[U], v0[U], v1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = (int64_t)min(t0 + u, kend - 1) * stride;
      k0[u] = has0 ? to_f(kb[off + lane]) : 0.f;
      k1[u] = has1 ? to_f(kb[off + lane + 64]) : 0.f;
      v0[u] = has0 ? to_f(vb[off + lane]) : 0.f;
      v1[u] = has1 ? to_f(vb[off + lane + 64]) : 0.f;
    }
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) sc[u] = wave_sum(q0 * k0[u] + q1 * k1[u]) * scale;
    float mb = m;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t0 + u < kend) mb = fmaxf(mb, sc[u]);
    const float a = expf(m - mb);             // 0 on the first block (m = -inf)
    l *= a;
    o0 *= a;
    o1 *= a;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = t0 + u < kend ? expf(sc[u] - mb) : 0.f;
      l += p;
      o0 += p * v0[u];
      o1 += p * v1[u];
    }
    m = mb;
  }
  T* orow = out + bs * (int64_t)H * HD + (int64_t)h * HD;
  if (has0) orow[lane] = from_f<T>(o0 / l);
  if (has1) orow[lane + 64] = from_f<T>(o1 / l);
}

// ------------------------------------------------------------------ prefill (bf16 MFMA)
#define LLAMA_LDS __attribute__((address_space(3)))
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

template <int N>
__device__ __forceinline__ void attn_wait_vmcnt() {
  // s_waitcnt simm16 on gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// K and V tiles of 64 keys are copied global -> LDS by global_load_lds_dwordx4
// in their natural [key][d] layout (2-slot ring), 16-byte chunks XOR-swizzled
// per key.  Q.K^T reads K fragments with ds_read_b128; the P.V product needs
// V^T fragments (8 keys of one d per lane), which ds_read_b64_tr_b16 delivers
// from the natural layout: within each 16-lane group, lane i receives element i
// of the 16-element rows read by lanes 4r..4r+3, r = 0..3 (four keys).
template <int HD>
__global__ void __launch_bounds__(256, 2)
attn_prefill_mfma(const bf16* __restrict__ q, const bf16* __restrict__ ck, const bf16* __restrict__ cv,
                  bf16* __restrict__ out, AttnShape sh, int G, float scale_log2, int bgrp) {
  constexpr int BKV = 64;
  constexpr int CHK = HD / 8;                 // 16-byte chunks per key row
  constexpr int KPB = 1024 / (HD * 2);        // key rows per 1 KiB DMA block
  constexpr int DMA = BKV / KPB / 4;          // DMA instructions per wave per tensor per tile
  static_assert(HD == 64 || HD == 128, "head_dim");
  // one array per ring slot: the waitcnt pass then sees that reads of one slot
  // cannot alias the DMA into the other, and does not drain the prefetch first
  __shared__ bf16x8 Ks0[BKV * CHK], Ks1[BKV * CHK];
  __shared__ bf16x8 Vs0[BKV * CHK], Vs1[BKV * CHK];
  // bank-group swizzles: K rows are read 16 keys at a time (one chunk), V rows 4 keys x 32 bytes
  auto kswz = [](int key) { return CHK == 16 ? (key & 15) : ((key >> 1) & 7); };
  auto vswz = [](int key) { return CHK == 16 ? ((key & 3) << 2) : (((key >> 1) & 1) << 2); };

  const int H = sh.n_heads, Hkv = sh.n_kv_heads, S = sh.seqlen, p0 = sh.start_pos;
  const int n_rep = H / Hkv;
  const int BQ = 128 / G;
  const int hgroups = H / G;
  const int qblocks = (S + BQ - 1) / BQ;
  // Sequences are taken bgrp at a time (their K/V fits in the Infinity Cache);
  // within a group the heavy (late) query blocks go first.
  const int per_grp = bgrp * hgroups * qblocks;
  const int grp = (int)(blockIdx.x / per_grp);
  const int local = (int)(blockIdx.x % per_grp);
  const int b0 = grp * bgrp;
  const int per = min(bgrp, sh.bsz - b0) * hgroups;
  const int qb = qblocks - 1 - local / per;
  const int rest = local % per;
  const int hg = rest % hgroups, b = b0 + rest / hgroups;
  const int h0 = hg * G;
  const int j = h0 / n_rep;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar LDS bases and branches
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int R = wave * 32 + lrow;
  const int s = qb * BQ + R % BQ;
  const int h = h0 + R / BQ;
  const bool row_valid = s < S;
  const int s_c = row_valid ? s : S - 1;
  const int qpos = p0 + s;
  const int wave_qmin = p0 + qb * BQ + (wave * 32) % BQ;   // smallest query position of this wave
  const int wave_qmax = wave_qmin + min(32, BQ) - 1;        // and its largest

  bf16x8 qf[HD / 16];
  {
    const bf16* qr = q + (((int64_t)b * S + s_c) * H + h) * HD;
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk) qf[kk] = *(const bf16x8*)(qr + (kk * 2 + lhalf) * 8);
  }

  const int s_hi = min(S - 1, qb * BQ + BQ - 1);
  const int kend = p0 + s_hi + 1;
  const int ntiles = (kend + BKV - 1) / BKV;
  const int64_t stride = (int64_t)Hkv * HD;
  const bf16* kbase = ck + ((int64_t)b * sh.max_seq * Hkv + j) * HD;
  const bf16* vbase = cv + ((int64_t)b * sh.max_seq * Hkv + j) * HD;

  // DMA of key tile t0 into ring slot ST: block (wave*DMA + i) holds keys
  // KPB*(wave*DMA + i) .. +KPB; lane l fetches key + l/CHK, chunk (l%CHK) ^ swz(key).
  // Per-lane parts are computed once: 32-bit byte offsets from the sequence's
  // cache base (one sequence's rows stay below 2^31 elements, checked on the
  // host) and the chunk swizzles; a tile adds its first key.
  const char* kb8 = (const char*)kbase;
  const char* vb8 = (const char*)vbase;
  const uint32_t stride_b = (uint32_t)stride * 2;
  int dkey[DMA];
  uint32_t dk_off[DMA], dv_off[DMA];
#pragma unroll
  for (int i = 0; i < DMA; ++i) {
    const int key = (wave * DMA + i) * KPB + lane / CHK;
    dkey[i] = key;
    // byte offset of the lane's chunk in the tile's first row block (a tile adds t0 rows)
    dk_off[i] = (uint32_t)key * stride_b + (uint32_t)(((lane % CHK) ^ kswz(key)) * 16);
    dv_off[i] = (uint32_t)key * stride_b + (uint32_t)(((lane % CHK) ^ vswz(key)) * 16);
  }
  auto issue = [&](int t0, auto st_c) {
    constexpr int ST = decltype(st_c)::value;
    auto copy = [&](int i, uint32_t ko, uint32_t vo) {
      __builtin_amdgcn_global_load_lds((const void*)(kb8 + ko), (LLAMA_LDS void*)&(ST ? Ks1 : Ks0)[(wave * DMA + i) * 64],
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vb8 + vo), (LLAMA_LDS void*)&(ST ? Vs1 : Vs0)[(wave * DMA + i) * 64],
                                       16, 0, 0);
    };
    if (t0 + BKV <= kend) {                      // no key of the tile past the end: no clamp
      const uint32_t tb = (uint32_t)t0 * stride_b;
#pragma unroll
      for (int i = 0; i < DMA; ++i) copy(i, dk_off[i] + tb, dv_off[i] + tb);
    } else {
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        const uint32_t tb = (uint32_t)(min(t0 + dkey[i], kend - 1) - dkey[i]) * stride_b;
        copy(i, dk_off[i] + tb, dv_off[i] + tb);
      }
    }
  };

  f32x16 oacc[HD / 32];
#pragma unroll
  for (int i = 0; i < HD / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  // Fragment addresses, per lane, for slot 0 and key sub-tile 0; the slot, the
  // sub-tile and the second 8 keys of a V^T read are immediate offsets.  The
  // swizzles depend only on the key's low bits, which the sub-tile offsets
  // (multiples of 8 keys) leave unchanged.
  int kfo[HD / 16];
#pragma unroll
  for (int kk = 0; kk < HD / 16; ++kk) {
    const int c = kk * 2 + lhalf;
    kfo[kk] = lrow * CHK + (c ^ kswz(lrow));
  }
  // V^T read: lane group g = lane/16 covers d0 = (g&1)*16 (+32*dt), keys base + hf*4 (+8)
  const int li = lane & 15;
  const int vkey_off = lhalf * 4 + (li >> 2);
  const int vd_off = ((lane >> 4) & 1) * 16 + (li & 3) * 4;
  int vto[HD / 32];                           // element offsets into a V slot
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) {
    const int d = dt * 32 + vd_off;
    vto[dt] = (vkey_off * CHK + ((d >> 3) ^ vswz(vkey_off))) * 8 + (d & 7);
  }

  auto tile = [&](int it, auto st_c) {
    constexpr int ST = decltype(st_c)::value;
    const int t0 = it * BKV;
    attn_wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (it + 1 < ntiles) issue(t0 + BKV, std::integral_constant<int, ST ^ 1>{});
    // a tile above all of this wave's rows is fully masked for it: nothing to add
    if (t0 > wave_qmax) return;

    // S^T = K.Q^T: the K fragment reads run AHEAD reads in front of the MFMAs
    // that consume them (left to itself the compiler kept one or two reads in
    // flight, so each MFMA waited out a whole LDS latency)
    constexpr int NKF = 2 * (HD / 16);        // K fragments per tile
    constexpr int AHEAD = HD / 16;
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    bf16x8 kf[2][HD / 16];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kk = 0; kk < HD / 16; ++kk) kf[kt][kk] = (ST ? Ks1 : Ks0)[kfo[kk] + kt * 32 * CHK];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kk = 0; kk < HD / 16; ++kk)
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kt][kk], qf[kk], sacc[kt], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int i = 0; i < NKF - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
    __builtin_amdgcn_sched_barrier(0);
    // causal mask only where this wave's rows meet the diagonal
    if (t0 + BKV - 1 > wave_qmin) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int t = t0 + kt * 32 + (v >> 2) * 8 + lhalf * 4 + (v & 3);
          if (t > qpos) sacc[kt][v] = -INFINITY;
        }
    }
    // Probabilities against the running max (log2 domain, scale > 0) and their
    // row sum exactly as P.V uses them (bf16, two per dot2).
    bf16x8 pf[2][2];
    float psum;
    auto probs = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          pf[kt][v >> 3][v & 7] = (bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][v], scale_log2, -m_run));
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
      const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x2 pp = {pf[kt][h2][2 * j], pf[kt][h2][2 * j + 1]};
            ps[j] = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, ps[j], false);
          }
      psum = pair_sum32((ps[0] + ps[1]) + (ps[2] + ps[3]));
    };
    probs();
    // Lazy rescale: the running max moves only when some row's max grows by more
    // than 8 (probabilities then stay below 2^8).  A row sum of at most 2^8 bounds
    // every probability of the row, so the tile max is only taken when some row's
    // sum exceeds it (or is not finite: the first tile, against a max of -inf).
    if (__any(!(psum <= 256.0f))) {
      float mraw = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mraw = fmaxf(mraw, sacc[kt][v]);
      mraw = pair_max32(mraw);
      const float mt = mraw * scale_log2;
      if (__any(mt > m_run + 8.0f)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
        probs();
      }
    }
    l_run += psum;

#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt) {
          const bf16* v1 = (const bf16*)(ST ? Vs1 : Vs0) + vto[dt] + (kt * 32 + h2 * 16) * CHK * 8;
          const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LLAMA_LDS bf16x4_t*)v1);
          const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LLAMA_LDS bf16x4_t*)(v1 + 8 * CHK * 8));
          const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kt][h2], oacc[dt], 0, 0, 0);
        }
      }
    asm volatile("" ::: "memory");
  };

  issue(0, std::integral_constant<int, 0>{});
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    tile(it, std::integral_constant<int, 0>{});
    tile(it + 1, std::integral_constant<int, 1>{});
  }
  if (it < ntiles) tile(it, std::integral_constant<int, 0>{});

  if (!row_valid) return;
  const float inv = 1.0f / l_run;
  bf16* orow = out + (((int64_t)b * S + s) * H + h) * HD;
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v = {oacc[dt][g * 4], oacc[dt][g * 4 + 1], oacc[dt][g * 4 + 2], oacc[dt][g * 4 + 3]};
      store4(orow + dt * 32 + g * 8 + lhalf * 4, v * inv);
    }
}

// ------------------------------------------------------------------ decode (bf16 MFMA, split-K)
template <int HD, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_decode_mfma(const bf16* __restrict__ q, const bf16* __restrict__ ck, const bf16* __restrict__ cv,
                 bf16* __restrict__ out, float* __restrict__ partial, AttnShape sh, int nsplit, int L,
                 float scale_log2, const int32_t* __restrict__ pos_dev) {
  constexpr int CH = HD / 8;
  static_assert(HD == 64 || HD == 128, "head_dim");
  constexpr int RPI = 64 / CH;                // K rows per load instruction (whole rows)
  constexpr int KL = 32 / RPI;                // K loads per lane per 32-key chunk
  constexpr int CSTR = NW * 32;              // key stride between a wave's chunks
  __shared__ bf16x8 Vt[NW][HD * 4];         // per wave: [d][4 chunks of 8 permuted keys]
  __shared__ bf16x8 Kt[NW][32 * CH];        // per wave: [key][chunk ^ ksw(key)]
  __shared__ float mrg_m[NW][16], mrg_l[NW][16];

  const int H = sh.n_heads, Hkv = sh.n_kv_heads;
  const int n_rep = H / Hkv;
  const int hgs = (n_rep + 15) / 16;
  // grid x walks the kv heads fastest, and the flattened workgroup id is
  // remapped so that consecutive ids share an XCD: the workgroups that read the
  // pieces of the same cache rows (2*head_dim bytes per kv head) run together
  // on one XCD instead of being dealt round-robin over all eight
  const int nbx = gridDim.x, nby = gridDim.y;
  const int lid = xcd_remap(blockIdx.x + nbx * (blockIdx.y + nby * blockIdx.z), nbx * nby * gridDim.z);
  const int bx = lid % nbx, by = (lid / nbx) % nby;
  const int j = bx / hgs, hg = bx % hgs;
  const int z = by;
  const int b = lid / (nbx * nby);
  // (a device-resident position may leave the last splits without keys: they
  // write an empty partial, max -inf and sum 0, which the combine weighs 0)
  const int T = (pos_dev ? min(max(*pos_dev, 0), sh.start_pos) : sh.start_pos) + 1;
  const int t_begin = z * L, t_end = min(T, t_begin + L);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int hl = hg * 16 + l16;               // head within the kv group
  const bool hvalid = hl < n_rep;
  const int h = j * n_rep + (hvalid ? hl : 0);

  bf16x8 qf[HD / 32];
  {
    const bf16* qr = q + ((int64_t)b * H + h) * HD;
#pragma unroll
    for (int kk = 0; kk < HD / 32; ++kk)
      qf[kk] = hvalid ? *(const bf16x8*)(qr + (kk * 4 + g) * 8) : bf16x8{};
  }
  const int64_t stride = (int64_t)Hkv * HD;
  const bf16* kbase = ck + ((int64_t)b * sh.max_seq * Hkv + j) * HD;
  const bf16* vbase = cv + ((int64_t)b * sh.max_seq * Hkv + j) * HD;

  f32x4 oacc[HD / 16];
#pragma unroll
  for (int i = 0; i < HD / 16; ++i) oacc[i] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const bool vtask = lane < 4 * CH;
  const int vg = lane / CH, vdc = lane % CH;

  // Each wave walks 32-key chunks c0, c0 + 128, ... of [t_begin, t_end).  The
  // next chunk's K and V loads are issued before the current chunk is used, so
  // the wave always has one chunk in flight.  Key indices are clamped to
  // t_end - 1 (a row of this split that is always written): the loads need no
  // guard and the softmax masks those keys out, so their V rows get weight 0.
  // Offsets within one sequence's cache rows fit 32 bits (the host rejects
  // max_seq * n_kv_heads * head_dim >= 2^31).
  // K is loaded whole rows per instruction (CH lanes per key: a head's row is
  // one contiguous piece), which streams measurably faster from HBM than the
  // MFMA operand layout (16 keys x 64 bytes per instruction); the rows go
  // through a per-wave LDS tile into that layout.  The swizzle ksw keeps both
  // the row writes and the 16-key operand reads free of bank conflicts.
  auto ksw = [](int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); };
  // V tile slot of (dim d, key group kg): the four slots of each dim, XOR-ed
  // within their 16-slot block by d / 4, so that the operand reads (16 dims of
  // one key group) hit 16 different bank groups and the transposed writes (16
  // dims 8 apart) at most two lanes per bank group.
  auto vsw = [](int d, int kg) { return (d * 4 + kg) ^ ((d >> 2) & 15); };
  const int rstride = (int)stride;
  auto load = [&](int c0, bf16x8 (&kr)[KL], bf16x8 (&vk)[8]) {
#pragma unroll
    for (int e = 0; e < KL; ++e) {
      const int key = min(c0 + e * RPI + lane / CH, t_end - 1);
      kr[e] = load_stream8(kbase + (uint32_t)(key * rstride + (lane % CH) * 8));
    }
    if (vtask) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = min(c0 + (e < 4 ? vg * 4 + e : 16 + vg * 4 + (e - 4)), t_end - 1);
        vk[e] = load_stream8(vbase + (uint32_t)(key * rstride + vdc * 8));
      }
    }
  };
  auto compute = [&](int c0, const bf16x8 (&kr)[KL], const bf16x8 (&vk)[8]) {
#pragma unroll
    for (int e = 0; e < KL; ++e) {
      const int r = e * RPI + lane / CH;
      Kt[wave][r * CH + ((lane % CH) ^ ksw(r))] = kr[e];
    }
    if (vtask) {
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int d = vdc * 8 + dd;
        bf16x8 w = {vk[0][dd], vk[1][dd], vk[2][dd], vk[3][dd], vk[4][dd], vk[5][dd], vk[6][dd], vk[7][dd]};
        Vt[wave][vsw(d, vg)] = w;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kk = 0; kk < HD / 32; ++kk) {
        const int r = kt * 16 + l16, c = kk * 4 + g;
        const bf16x8 kf = Kt[wave][r * CH + (c ^ ksw(r))];
        sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], sacc[kt], 0, 0, 0);
      }
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = c0 + kt * 16 + g * 4 + v;
        float x = key < t_end ? sacc[kt][v] * scale_log2 : -INFINITY;
        sacc[kt][v] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = pair_max32(pair_max16(mloc));
    // lazy rescale: the running max moves only when some head's max grows by
    // more than 8 (probabilities then stay below 2^8); the result is unchanged
    if (__any(mloc > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
    bf16x8 pf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float p = __builtin_amdgcn_exp2f(sacc[kt][v] - m_run);
        psum += p;
        pf[kt * 4 + v] = (bf16)p;
      }
    psum = pair_sum32(pair_sum16(psum));
    l_run += psum;
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) {
      const int d = dt * 16 + l16;
      bf16x8 vf = Vt[wave][vsw(d, g)];
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  const int c_first = t_begin + wave * 32;
  const int nit = c_first < t_end ? (t_end - c_first + CSTR - 1) / CSTR : 0;
  bf16x8 kA[KL], vA[8], kB[KL], vB[8];
  if (nit > 0) load(c_first, kA, vA);
  int it = 0;
  // (the scheduling barriers keep each prefetch ahead of the compute that
  // would otherwise be hoisted above it and wait for every load in flight)
  for (; it + 1 < nit; it += 2) {
    load(c_first + (it + 1) * CSTR, kB, vB);
    __builtin_amdgcn_sched_barrier(0);
    compute(c_first + it * CSTR, kA, vA);
    __builtin_amdgcn_sched_barrier(0);
    load(c_first + (it + 2) * CSTR, kA, vA);   // past the end: clamped rows, never used
    __builtin_amdgcn_sched_barrier(0);
    compute(c_first + (it + 1) * CSTR, kB, vB);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (it < nit) compute(c_first + it * CSTR, kA, vA);

  // merge the NW waves' (max, sum, o) in LDS
  __syncthreads();
  float* obuf = (float*)&Vt[0][0];            // [NW waves][16 heads][HD] floats
  if (g == 0) {
    mrg_m[wave][l16] = m_run;
    mrg_l[wave][l16] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt)
#pragma unroll
    for (int v = 0; v < 4; ++v) obuf[(wave * 16 + l16) * HD + dt * 16 + g * 4 + v] = oacc[dt][v];
  __syncthreads();

  const int hh = tid >> 4;                    // head slot 0..15 (the first 256 threads)
  const int d0 = (tid & 15) * (HD / 16);
  const int hl2 = hg * 16 + hh;
  if (tid >= 256 || hl2 >= n_rep) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, mrg_m[w][hh]);
  float wt[NW], Ls = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wt[w] = mrg_m[w][hh] == -INFINITY ? 0.f : exp2f(mrg_m[w][hh] - M);
    Ls += wt[w] * mrg_l[w][hh];
  }
  float o[HD / 16];
#pragma unroll
  for (int k = 0; k < HD / 16; ++k) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) acc += wt[w] * obuf[(w * 16 + hh) * HD + d0 + k];
    o[k] = acc;
  }
  const int hq = j * n_rep + hl2;
  if (nsplit == 1) {
    bf16* orow = out + ((int64_t)b * H + hq) * HD + d0;
    const float inv = 1.0f / Ls;
#pragma unroll
    for (int k = 0; k < HD / 16; k += 4) store4(orow + k, f32x4{o[k], o[k + 1], o[k + 2], o[k + 3]} * inv);
  } else {
    float* p = partial + (((int64_t)b * H + hq) * nsplit + z) * (HD + 2);
#pragma unroll
    for (int k = 0; k < HD / 16; ++k) p[d0 + k] = o[k];
    if ((tid & 15) == 0) {
      p[HD] = M;
      p[HD + 1] = Ls;
    }
  }
}

// The same merge for at most NB splits: one wave per (b, head), four rows per
// workgroup, every split loaded before any is used, no LDS.
template <typename T, int HD, int NB>
__global__ void __launch_bounds__(256)
attn_decode_combine_wave(const float* __restrict__ partial, T* __restrict__ out, int nsplit, int rows) {
  constexpr int PD = HD / 64;
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= rows) return;
  const float* base = partial + bh * nsplit * (HD + 2);
  float mz[NB], lz[NB], oz[NB][PD];
#pragma unroll
  for (int z = 0; z < NB; ++z) {
    const float* p = base + (int64_t)min(z, nsplit - 1) * (HD + 2);
    mz[z] = z < nsplit ? p[HD] : -INFINITY;
    lz[z] = p[HD + 1];
#pragma unroll
    for (int k = 0; k < PD; ++k) oz[z][k] = p[lane * PD + k];
  }
  float M = mz[0];
#pragma unroll
  for (int z = 1; z < NB; ++z) M = fmaxf(M, mz[z]);
  float Ls = 0.f, o[PD];
#pragma unroll
  for (int k = 0; k < PD; ++k) o[k] = 0.f;
#pragma unroll
  for (int z = 0; z < NB; ++z) {
    const float w = exp2f(mz[z] - M);
    Ls += w * lz[z];
#pragma unroll
    for (int k = 0; k < PD; ++k) o[k] += w * oz[z][k];
  }
  const float inv = 1.0f / Ls;
#pragma unroll
  for (int k = 0; k < PD; ++k) out[bh * HD + lane * PD + k] = from_f<T>(o[k] * inv);
}

// Log-sum-exp merge of the split partials of one (b, head).  Wave w takes the
// splits w, w + 4, ...; each lane owns HD / 64 output dimensions.  A wave loads
// up to 16 splits (maximum, sum and its dimensions of o) before using any of
// them, keeps a running (max, sum, o) that it rescales as the maximum grows,
// and the four waves merge in LDS: one memory round trip for up to 64 splits.
// Maxima are in the log2 domain of the decode kernel; an empty split (max -inf)
// weighs 0, and split 0 always holds keys, so the total sum is positive.
template <typename T, int HD>
__global__ void __launch_bounds__(256)
attn_decode_combine(const float* __restrict__ partial, T* __restrict__ out, int nsplit) {
  constexpr int PD = HD / 64;
  constexpr int NB = 16;
  __shared__ float sm[4], sl[4], so[4][HD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t bh = blockIdx.x;
  const float* base = partial + bh * nsplit * (HD + 2);
  float M = -INFINITY, Ls = 0.f, o[PD];
#pragma unroll
  for (int k = 0; k < PD; ++k) o[k] = 0.f;
  for (int z0 = wave; z0 < nsplit; z0 += 4 * NB) {
    float mz[NB], lz[NB], oz[NB][PD];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int z = z0 + 4 * i;
      const float* p = base + (int64_t)min(z, nsplit - 1) * (HD + 2);
      mz[i] = z < nsplit ? p[HD] : -INFINITY;
      lz[i] = p[HD + 1];
#pragma unroll
      for (int k = 0; k < PD; ++k) oz[i][k] = p[lane * PD + k];
    }
    float mb = M;
#pragma unroll
    for (int i = 0; i < NB; ++i) mb = fmaxf(mb, mz[i]);
    if (mb == -INFINITY) continue;
    const float a = exp2f(M - mb);
    Ls *= a;
#pragma unroll
    for (int k = 0; k < PD; ++k) o[k] *= a;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float w = exp2f(mz[i] - mb);
      Ls += w * lz[i];
#pragma unroll
      for (int k = 0; k < PD; ++k) o[k] += w * oz[i][k];
    }
    M = mb;
  }
  if (lane == 0) {
    sm[wave] = M;
    sl[wave] = Ls;
  }
#pragma unroll
  for (int k = 0; k < PD; ++k) so[wave][lane * PD + k] = o[k];
  __syncthreads();
  if (wave != 0) return;
  const float Mx = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  float wt[4], tot = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wt[w] = sm[w] == -INFINITY ? 0.f : exp2f(sm[w] - Mx);
    tot += wt[w] * sl[w];
  }
  const float inv = 1.0f / tot;
#pragma unroll
  for (int k = 0; k < PD; ++k) {
    const int d = lane * PD + k;
    const float acc = wt[0] * so[0][d] + wt[1] * so[1][d] + wt[2] * so[2][d] + wt[3] * so[3][d];
    out[bh * HD + d] = from_f<T>(acc * inv);
  }
}

}  // namespace

// ------------------------------------------------------------------ host launchers
template <typename T>
hipError_t kv_append(const T* xk, const T* xv, T* cache_k, T* cache_v, const AttnShape& sh,
                     hipStream_t st) {
  int64_t total4 = (int64_t)sh.bsz * sh.seqlen * sh.n_kv_heads * sh.head_dim / 4;
  if (total4 == 0) return hipSuccess;
  int64_t nb = (total4 + 255) / 256;
  int blocks = (int)(nb < 8192 ? nb : 8192);
  kv_append_kernel<T><<<blocks, 256, 0, st>>>(xk, xv, cache_k, cache_v, sh);
  return hipGetLastError();
}

static int prefill_group(int n_rep) {
  int g = 1;
  while (g < 8 && n_rep % (g * 2) == 0) g *= 2;
  return g;
}

template <typename T>
hipError_t attn_prefill(const T* q, const T* cache_k, const T* cache_v, T* out, const AttnShape& sh,
                        hipStream_t st) {
  const float scale = 1.0f / sqrtf((float)sh.head_dim);
  if constexpr (sizeof(T) == 2) {
    const int G = prefill_group(sh.n_heads / sh.n_kv_heads);
    const int BQ = 128 / G;
    const int64_t blocks = (int64_t)((sh.seqlen + BQ - 1) / BQ) * (sh.n_heads / G) * sh.bsz;
    // sequences per dispatch group: as many as keep their attended K/V within
    // kPrefillKvGroupBytes, so that a group's re-reads of K/V tiles hit the
    // Infinity Cache (a whole batch when it fits: 7B-shaped batch 4, 134 MB)
    const int64_t kv_seq = (int64_t)(sh.start_pos + sh.seqlen) * sh.n_kv_heads * sh.head_dim * 2 * sizeof(T);
    const int bgrp = (int)std::max<int64_t>(1, std::min<int64_t>(sh.bsz, kPrefillKvGroupBytes / kv_seq));
    if (sh.head_dim == 128)
      attn_prefill_mfma<128><<<(unsigned)blocks, 256, 0, st>>>(q, cache_k, cache_v, out, sh, G, scale * kLog2e, bgrp);
    else
      attn_prefill_mfma<64><<<(unsigned)blocks, 256, 0, st>>>(q, cache_k, cache_v, out, sh, G, scale * kLog2e, bgrp);
  } else {
    const int64_t waves = (int64_t)sh.bsz * sh.seqlen * sh.n_heads;
    attn_simple<T><<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(q, cache_k, cache_v, out, sh, scale);
  }
  return hipGetLastError();
}

static int attn_decode_waves(int bsz, int n_heads, int n_kv_heads) {
  // one 8-wave workgroup per (sequence, kv group) when those units alone fill
  // between half and all of the CUs (one resident round at one workgroup per CU):
  // no split, no merge kernel
  const int units = bsz * n_kv_heads * ((n_heads / n_kv_heads + 15) / 16);
  return units >= kResidentDecodeWgs / 4 && units <= kResidentDecodeWgs / 2 ? 8 : 4;
}

int attn_decode_splits(int bsz, int n_heads, int n_kv_heads, int T) {
  if (attn_decode_waves(bsz, n_heads, n_kv_heads) == 8) return 1;
  const int n_rep = n_heads / n_kv_heads;
  const int units = bsz * n_kv_heads * ((n_rep + 15) / 16);
  // two rounds of the 512 workgroups that are resident at once (two per CU);
  // when that leaves under 4096 keys per split, the whole grid is one round
  // instead: a short split is a single latency-bound pass that a second round
  // would double, and one round of longer splits also measured faster (70B
  // shape, batch 32 at 4097 keys: 2 splits of 2049 keys against 4 of 1025)
  int ns = (1024 + units - 1) / units;
  if ((T + ns - 1) / ns < 4096) ns = max(1, kResidentDecodeWgs / units);
  ns = max(1, min(ns, (T + 127) / 128));
  int L = (T + ns - 1) / ns;
  L = (L + 31) / 32 * 32;
  return (T + L - 1) / L;
}

template <typename T>
hipError_t attn_decode(const T* q, const T* cache_k, const T* cache_v, T* out, const AttnShape& sh,
                       float* partial, hipStream_t st, const int32_t* pos_dev) {
  const float scale = 1.0f / sqrtf((float)sh.head_dim);
  if constexpr (sizeof(T) == 2) {
    const int T_ = sh.start_pos + 1;
    const int ns = attn_decode_splits(sh.bsz, sh.n_heads, sh.n_kv_heads, T_);
    int L = (T_ + ns - 1) / ns;
    L = (L + 31) / 32 * 32;
    const int n_rep = sh.n_heads / sh.n_kv_heads;
    dim3 grid(sh.n_kv_heads * ((n_rep + 15) / 16), ns, sh.bsz);
    const bool w8 = attn_decode_waves(sh.bsz, sh.n_heads, sh.n_kv_heads) == 8;
    if (sh.head_dim == 128 && w8)
      attn_decode_mfma<128, 8><<<grid, 512, 0, st>>>(q, cache_k, cache_v, out, partial, sh, ns, L, scale * kLog2e,
                                                     pos_dev);
    else if (sh.head_dim == 128)
      attn_decode_mfma<128, 4><<<grid, 256, 0, st>>>(q, cache_k, cache_v, out, partial, sh, ns, L, scale * kLog2e,
                                                     pos_dev);
    else if (w8)
      attn_decode_mfma<64, 8><<<grid, 512, 0, st>>>(q, cache_k, cache_v, out, partial, sh, ns, L, scale * kLog2e,
                                                    pos_dev);
    else
      attn_decode_mfma<64, 4><<<grid, 256, 0, st>>>(q, cache_k, cache_v, out, partial, sh, ns, L, scale * kLog2e,
                                                    pos_dev);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;
    const int rows = sh.bsz * sh.n_heads;
    const int wgs = (rows + 3) / 4;
    if (ns <= 4) {
      if (sh.head_dim == 128)
        attn_decode_combine_wave<T, 128, 4><<<wgs, 256, 0, st>>>(partial, out, ns, rows);
      else
        attn_decode_combine_wave<T, 64, 4><<<wgs, 256, 0, st>>>(partial, out, ns, rows);
    } else if (ns <= 16) {
      if (sh.head_dim == 128)
        attn_decode_combine_wave<T, 128, 16><<<wgs, 256, 0, st>>>(partial, out, ns, rows);
      else
        attn_decode_combine_wave<T, 64, 16><<<wgs, 256, 0, st>>>(partial, out, ns, rows);
    } else if (sh.head_dim == 128) {
      attn_decode_combine<T, 128><<<rows, 256, 0, st>>>(partial, out, ns);
    } else {
      attn_decode_combine<T, 64><<<rows, 256, 0, st>>>(partial, out, ns);
    }
  } else {
    if (pos_dev) return hipErrorNotSupported;
    const int64_t waves = (int64_t)sh.bsz * sh.n_heads;
    attn_simple<T><<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(q, cache_k, cache_v, out, sh, scale);
  }
  return hipGetLastError();
}

template hipError_t kv_append<bf16>(const bf16*, const bf16*, bf16*, bf16*, const AttnShape&, hipStream_t);
template hipError_t kv_append<float>(const float*, const float*, float*, float*, const AttnShape&, hipStream_t);
template hipError_t attn_prefill<bf16>(const bf16*, const bf16*, const bf16*, bf16*, const AttnShape&, hipStream_t);
template hipError_t attn_prefill<float>(const float*, const float*, const float*, float*, const AttnShape&,
                                        hipStream_t);
template hipError_t attn_decode<bf16>(const bf16*, const bf16*, const bf16*, bf16*, const AttnShape&, float*,
                                      hipStream_t, const int32_t*);
template hipError_t attn_decode<float>(const float*, const float*, const float*, float*, const AttnShape&,
                                       float*, hipStream_t, const int32_t*);

}  // namespace llama
