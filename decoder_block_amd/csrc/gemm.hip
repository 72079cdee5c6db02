// Projection GEMMs C[m][n] = sum_k A[m][k] W[n][k] for gfx950.
//
// bf16: LDS-staged, double-buffered tiles feeding v_mfma_f32_16x16x32_bf16
// (large tiles) or v_mfma_f32_32x32x16_bf16 (decode-sized tiles).
// The weight tile is the MFMA "A" operand (rows i = n) and the activation tile
// the "B" operand (columns j = m), so each lane's accumulators hold four
// consecutive output columns n of one token row m: the epilogue can rotate
// RoPE pairs and pair w1/w3 results in registers and store 8-byte vectors.
// Both operands are K-contiguous (nn.Linear layout), which is the layout the
// MFMA wants per lane (8 consecutive k values); tiles sit in LDS as 16-byte
// chunks with an XOR swizzle on the chunk index so that the 16 lanes of one
// ds_read_b128 phase (16 consecutive rows) cover all 64 banks.
//
// f32: a plain LDS-tiled FMA kernel (the fp32 workload is tiny and launch
// bound), same epilogues.
#include "gemm.hpp"

#include <type_traits>

namespace llama {

namespace {

constexpr int kThreads = 256;
// large M: 256 x 256 tiles, 64-deep k-tiles in a 2-stage LDS ring (2 x 64 KiB), eight
// waves (two per SIMD: one wave's MFMAs cover the other's waits)
constexpr int kBigBK = 64;
constexpr int kBigStages = 2;
constexpr int kBigWaves = 8;
// MFMA shape of the large tiles: 16x16x32.  Per flop it reads and writes half
// the accumulator registers of 32x32x16 for the same LDS fragment bytes (a
// 128 x 64 wave tile reads 192 rows of k either way); measured on the
// Llama-3-8B-shaped block (M = 8192) it ran the dual w1/w3 GEMM at 1.32-1.34
// instead of 1.24-1.25 PF/s, w2 1.34-1.35 instead of 1.24-1.25, QKV and wo 8-9 %
// faster, at the same LDS traffic and the same number of waves.
constexpr int kBigMI = 16;
constexpr int kCUs = 256;         // MI355X compute units
// Unsplit 256 x 256 tiles run on a resident grid that walks the tiles (measured
// at M = 131072: 1-2 % faster for K = 2048-8192, 0.3-0.5 % at K = 14336 or
// N = 14336; the same at M = 8192)
constexpr bool kResidentLargeTiles = true;
// small M (<= 64 tokens: the weights stream from HBM once): 64-deep k-tiles
// (128-byte row pieces).  Tiles: M <= 32: 32 rows x 128 columns, 32 x 256 for
// the dual w1/w3 kernel; 33..64 rows: 64 x 128.  Narrow tiles need fewer
// K-splits to cover the CUs (measured: LLaMA-3-8B-shaped w1/w3 at M = 64 went
// from 70 to 48 us).  Ring depths: more stages buy no weight bandwidth here
// (the DMA queue is already deep), while a smaller LDS footprint lets the next
// kernel's workgroups start on a CU before the last ones of this kernel end --
// measured over whole decode steps, 3 stages for the plain 64-row tile and 4
// for the others ran 1-2% faster than 6.
constexpr int kSkinnyBK = 64;
constexpr int kSkinnyStages = 4;         // 32 x 128, dual 32 x 256, dual 64 x 128
constexpr int kSkinnyStages64 = 3;       // 64 x 128
// cache-policy operand of the LDS-DMA load: the non-temporal bit (gfx940 family)
constexpr int kCpolNT = 2;

template <typename T>
__device__ __forceinline__ const T* weight_row(const WeightRows<T>& w, int n, int K) {
  if (n < w.n1) return w.w0 + (int64_t)n * K;
  if (n < w.n2) return w.w1 + (int64_t)(n - w.n1) * K;
  return w.w2 + (int64_t)(n - w.n2) * K;
}

// Tile coordinates of a logical workgroup id: XCD-aware remap, then grouped
// ordering (GROUP_M tile rows share their weight tiles in L2).
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn, int bid) {
  constexpr int GROUP_M = 4;
  int nb = tiles_m * tiles_n;
  int pid = xcd_remap(bid, nb);
  int in_group = GROUP_M * tiles_n;
  int gid = pid / in_group;
  int first_m = gid * GROUP_M;
  int gsz = min(tiles_m - first_m, GROUP_M);
  int r = pid - gid * in_group;
  tm = first_m + r % gsz;
  tn = r / gsz;
}

// ------------------------------------------------------------------ bf16 MFMA kernel
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool DUAL, bool SPLIT, class Epi>
__global__ void __launch_bounds__(kThreads)
gemm_bf16_mfma(const bf16* __restrict__ A, int64_t lda, WeightRows<bf16> w, int M, int N, int K,
               int k_per_split, Epi epi, float* __restrict__ partial) {
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int CH = BK / 8;                 // 16-byte chunks per tile row
  constexpr int ROWS = BM + BN;
  constexpr int LOADS = ROWS * CH / kThreads;
  constexpr int BN_OUT = DUAL ? BN / 2 : BN;
  static_assert(WAVES_M * WAVES_N == 4, "four waves");
  static_assert(TM >= 1 && TN >= 1 && (!DUAL || TN % 2 == 0), "wave tile");
  static_assert((ROWS * CH) % kThreads == 0 && (BM * CH) % kThreads == 0, "load split");
  static_assert(CH == 8, "swizzle assumes 8 chunks per row");

  __shared__ bf16x8 smem[2][ROWS * CH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;

  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN_OUT - 1) / BN_OUT;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn, (int)blockIdx.x);
  const int m0 = tm * BM, n0 = tn * BN_OUT;
  const int kb = blockIdx.z * k_per_split;
  const int ke = min(K, kb + k_per_split);
  const int nk = (ke - kb + BK - 1) / BK;

  // global -> register staging: chunk q = tid + i*256 of the (A rows | W rows) tile
  const bf16* src[LOADS];
  int row_of[LOADS], chunk_of[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    int q = tid + i * kThreads;
    int r = q / CH, c = q % CH;
    row_of[i] = r;
    chunk_of[i] = c;
    const bf16* p = nullptr;
    if (r < BM) {
      int m = m0 + r;
      if (m < M) p = A + (int64_t)m * lda;
    } else {
      int rb = r - BM;
      int n;
      if (DUAL) {
        // rows [0, BN/2) of the weight tile come from w1, [BN/2, BN) from w3
        n = n0 + (rb < BN / 2 ? rb : rb - BN / 2);
        if (n < N) p = (rb < BN / 2 ? w.w0 : w.w1) + (int64_t)n * K;
      } else {
        n = n0 + rb;
        if (n < N) p = weight_row(w, n, K);
      }
    }
    src[i] = p ? p + c * 8 : nullptr;
  }

  bf16x8 stage[LOADS];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if (src[i] && k0 + chunk_of[i] * 8 < ke)
        stage[i] = *(const bf16x8*)(src[i] + k0);
      else
        stage[i] = bf16x8{};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      int r = row_of[i];
      smem[buf][r * CH + (chunk_of[i] ^ ((r >> 1) & 7))] = stage[i];
    }
  };

  // LDS row (within the weight tile) of this wave's MFMA tile t
  auto wrow = [&](int t) {
    if (DUAL) {
      return t < TN / 2 ? wn * (WN / 2) + t * 32 : BN / 2 + wn * (WN / 2) + (t - TN / 2) * 32;
    }
    return wn * WN + t * 32;
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x16{};

  if (nk > 0) {
    gload(kb);
    sstore(0);
  }
  __syncthreads();

  const int lrow = lane & 31, lhalf = lane >> 5;
  // (the epilogue below is shared in form with the DMA kernel's)
  constexpr int MI = 32, NV = 4;
  using acc_t = f32x16;
  const int lk = lhalf;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kb + (kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + lhalf;
      bf16x8 fa[TN], fb[TM];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        int r = BM + wrow(t) + lrow;
        fa[t] = smem[buf][r * CH + (c ^ ((r >> 1) & 7))];
      }
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        int r = wm * WM + t * 32 + lrow;
        fb[t] = smem[buf][r * CH + (c ^ ((r >> 1) & 7))];
      }
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds n = base + g*8 + lhalf*4 + {0..3} of row m = .. + lrow
#pragma unroll
  for (int b = 0; b < TM; ++b) {
    const int m = m0 + wm * WM + b * MI + lrow;
    if (m >= M) continue;
    if constexpr (DUAL) {
#pragma unroll
      for (int a = 0; a < TN / 2; ++a)
#pragma unroll
        for (int g = 0; g < NV; ++g) {
          const int n = n0 + wn * (WN / 2) + a * MI + g * 8 + lk * 4;
          if (n >= N) continue;
          f32x4 v1 = {acc[a][b][g * 4], acc[a][b][g * 4 + 1], acc[a][b][g * 4 + 2], acc[a][b][g * 4 + 3]};
          const acc_t& a3 = acc[a + TN / 2][b];
          f32x4 v3 = {a3[g * 4], a3[g * 4 + 1], a3[g * 4 + 2], a3[g * 4 + 3]};
          if (SPLIT) {
            float* p = partial + ((int64_t)blockIdx.z * M + m) * (2 * (int64_t)N);
            *(f32x4*)(p + n) = v1;
            *(f32x4*)(p + N + n) = v3;
          } else {
            epi(m, n, v1, v3);
          }
        }
    } else {
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN + a * 32 + g * 8 + lhalf * 4;
          if (n >= N) continue;
          f32x4 v = {acc[a][b][g * 4], acc[a][b][g * 4 + 1], acc[a][b][g * 4 + 2], acc[a][b][g * 4 + 3]};
          if (SPLIT) {
            *(f32x4*)(partial + ((int64_t)blockIdx.z * M + m) * (int64_t)N + n) = v;
          } else {
            epi(m, n, v);
          }
        }
    }
  }
}

// ------------------------------------------------------------------ bf16 MFMA kernel, LDS DMA pipeline
// BM x BN output tile (256 x 256 for large M; 32 or 64 rows for decode-sized
// M), BK-deep k-tiles (32 or 64) in an NS-stage ring of LDS tiles filled by
// global_load_lds_dwordx4 (global memory straight into LDS, no staging
// registers), so NS-1 k-tiles are in flight while one is consumed.  Each DMA
// instruction writes 1 KiB = 64 lanes x 16 bytes, RPB = 1024 / (2 BK) tile rows:
// lane l fetches row l / CH of its block (CH = BK / 8 chunks per row), 16-byte
// chunk (l % CH) ^ swz(row).  The XOR swizzle makes the 16 lanes of each
// ds_read_b128 phase (16 consecutive rows, one chunk) hit 16 distinct 16-byte
// bank groups.  Rows past M or N read a clamped (valid) row whose products land
// only in discarded outputs; K must be a multiple of BK.
// Schedule per k-tile: KS = BK / KM MFMA steps (KM = 16 or 32 deep).  The
// fragments of each step are read from LDS while the previous step's MFMAs run,
// the next k-tile's first fragments are read right after the single s_barrier,
// and the DMA refill of the ring slot just consumed is issued after that
// barrier.  The vmcnt waits are explicit: the compiler cannot see the LDS
// writes of the DMA.
#define LLAMA_LDS __attribute__((address_space(3)))

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  // s_waitcnt simm16 on gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(63 | (7 << 4) | (0 << 8) | (3 << 14)); }

template <int BM, int BN, int BK, int WAVES_M, int NS, bool DUAL, bool SPLIT, class Epi, int NW, int MI>
__global__ void __launch_bounds__(NW * 64)
gemm_bf16_dma(const bf16* __restrict__ A, int64_t lda, WeightRows<bf16> w, int M, int N, int K, int k_per_split,
              Epi epi, float* __restrict__ partial) {
  constexpr int CH = BK / 8;                  // 16-byte chunks per tile row
  constexpr int RPB = 64 / CH;                // tile rows per 1 KiB DMA block
  constexpr int WAVES_N = NW / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  // MFMA shape: MI x MI outputs, KM deep (32x32x16 or 16x16x32); a fragment is
  // MI rows x KM k, lane l holding 8 consecutive k of row l % MI (k block l / MI)
  constexpr int KM = MI == 32 ? 16 : 32;
  constexpr int LG = 64 / MI;                 // k blocks of 8 per fragment
  constexpr int NV = MI == 32 ? 4 : 1;        // groups of 4 consecutive rows per accumulator
  using acc_t = typename std::conditional<MI == 32, f32x16, f32x4>::type;
  static_assert(MI == 32 || MI == 16, "MFMA shape");
  constexpr int TM = WM / MI, TN = WN / MI;
  constexpr int ROWS = BM + BN;               // rows x 2*BK bytes per stage
  constexpr int BLOCKS = ROWS / RPB;          // 1 KiB DMA blocks per stage
  constexpr int LOADS = BLOCKS / NW;          // per wave (and per lane) per stage
  constexpr int BN_OUT = DUAL ? BN / 2 : BN;
  constexpr int RD = TN + TM;                 // fragment reads per KM-deep step
  constexpr int MF = TN * TM;                 // MFMAs per step
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(NS >= 2 && BLOCKS % NW == 0 && TM >= 1 && TN >= 1 && (!DUAL || TN % 2 == 0), "shape");
  static_assert(WAVES_M * WAVES_N == NW, "waves");
  __shared__ bf16x8 smem[NS][ROWS * CH];

  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar block bases
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN_OUT - 1) / BN_OUT;
  // Unsplit large tiles run on a resident grid (as many workgroups as the CUs
  // hold at once), each walking the tiles with a stride of the grid size, in
  // the logical order one workgroup per tile would take: every XCD keeps its
  // range of tiles, and no workgroup launch or set-up separates two tiles.
  constexpr bool kResident = kResidentLargeTiles && BM > 64 && !SPLIT;
  auto tile = [&](int vt) __attribute__((always_inline)) {
  // On the resident grid the thread's coordinates are derived per tile from the
  // thread id and an opaque zero: the compiler then cannot hoist them out of
  // the tile loop and keep them live through the epilogue, where the
  // accumulators need every VGPR.
  uint32_t zero = 0;
  if constexpr (kResident) asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
  const int tid = (int)(threadIdx.x ^ zero), lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn, vt);
  const int m0 = tm * BM, n0 = tn * BN_OUT;
  const int kb = blockIdx.z * k_per_split;
  const int nk = (min(K, kb + k_per_split) - kb) / BK;
  // Small-M tiles walk their k-tiles in a rotated order, starting at k-tile
  // tn % nk: weight rows a power of two apart (K = 4096, 8192) read at the same
  // k offset by every concurrent workgroup fall on few HBM channels (a probe of
  // this read pattern over 16 KiB rows: 4.3 TB/s in step, 5.4 TB/s rotated).
  const int krot = (BM <= 64 && nk > 0) ? tn % nk : 0;

  // bank-group swizzle of the 16-byte chunks: a ds_read_b128 phase reads one
  // chunk of 16 consecutive rows, which must hit 16 distinct bank groups
  auto swz = [](int r) { return BK == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7); };
  // Small-M tiles read every weight element exactly once: their weight blocks
  // carry the non-temporal hint.  The hint is an immediate of the instruction,
  // so there the blocks are dealt i-major (block i * NW + wave): the first
  // A_LOADS loads of every wave are activation rows, the rest weight rows.
  constexpr bool kStreamW = BM <= 64;
  constexpr int A_LOADS = kStreamW ? (BM / RPB) / NW : 0;
  static_assert(!kStreamW || (BM / RPB) % NW == 0, "activation rows must fill whole load slots");
  auto blk_of = [&](int i) { return kStreamW ? i * NW + wave_u : wave_u * LOADS + i; };
  // Source of each DMA block: a block is RPB consecutive rows of one operand
  // tensor (the QKV row map switches tensors at multiples of 8 rows, checked on
  // the host), so its base pointer is uniform and lives in scalar registers,
  // and a lane adds a 32-bit byte offset (its row within the block's 256-row
  // tile panel, the split's first k and its chunk); each copy adds the k-tile.
  const char* sbase[LOADS];
  uint32_t voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int blk = blk_of(i);
    const int r0 = blk * RPB;                 // the block's first tile row (uniform)
    const int r = r0 + lane / CH;
    const int c = (lane % CH) ^ swz(r);
    int64_t row;                              // this lane's row relative to the base
    int64_t ld;
    if (r0 < BM) {
      sbase[i] = (const char*)(A + (int64_t)m0 * lda);
      row = min(m0 + r, M - 1) - m0;
      ld = lda;
    } else {
      const int rb0 = r0 - BM, rb = r - BM;
      int nb, n;
      const bf16* t;
      if (DUAL) {
        nb = min(n0 + (rb0 & (BN / 2 - 1)), N - 1);
        n = min(n0 + (rb & (BN / 2 - 1)), N - 1);
        t = (rb0 < BN / 2 ? w.w0 : w.w1) + (int64_t)nb * K;
      } else {
        nb = min(n0 + rb0, N - 1);
        n = min(n0 + rb, N - 1);
        t = weight_row(w, nb, K);
      }
      sbase[i] = (const char*)t;
      row = n - nb;
      ld = K;
    }
    voff[i] = (uint32_t)((row * ld + kb + c * 8) * 2);
  }
  // DMA of k-tile kt into ring slot kt % NS (kt is clamped to the last tile so the
  // refill at the end of the loop stays branch-free; those copies are never read)
  auto issue = [&](int kt) {
    const int st = kt % NS;
    int kc = min(kt, nk - 1) + krot;
    kc = kc >= nk ? kc - nk : kc;
    const uint32_t kbyte = (uint32_t)(kc * BK * 2);
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      LLAMA_LDS void* dst = (LLAMA_LDS void*)&smem[st][blk_of(i) * 64];
      __builtin_amdgcn_global_load_lds((const void*)(sbase[i] + (voff[i] + kbyte)), dst, 16, 0, 0);
    }
#pragma unroll
    for (int i = A_LOADS; i < LOADS; ++i) {
      LLAMA_LDS void* dst = (LLAMA_LDS void*)&smem[st][blk_of(i) * 64];
      __builtin_amdgcn_global_load_lds((const void*)(sbase[i] + (voff[i] + kbyte)), dst, 16, 0,
                                       kStreamW ? kCpolNT : 0);
    }
  };
  auto wrow = [&](int t) {
    if (DUAL) return t < TN / 2 ? wn * (WN / 2) + t * MI : BN / 2 + wn * (WN / 2) + (t - TN / 2) * MI;
    return wn * WN + t * MI;
  };
  const int lrow = lane % MI, lk = lane / MI;
  auto read_half = [&](int st, int kk, bf16x8* fa, bf16x8* fb) {
    const int c = kk * LG + lk;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int r = BM + wrow(t) + lrow;
      fa[t] = smem[st][r * CH + (c ^ swz(r))];
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int r = wm * WM + t * MI + lrow;
      fb[t] = smem[st][r * CH + (c ^ swz(r))];
    }
  };

  acc_t acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = acc_t{};
  auto mfma_half = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        if constexpr (MI == 32)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
        else
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
      }
  };
  // the RD fragment reads for the next step go out one after each of the first
  // MFMAs, leaving the last MF - RD MFMAs (if any) to cover their latency
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < (MF > RD ? MF : RD); ++i) {
      if (i < MF) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  constexpr int KS = BK / KM;                 // MFMA steps per k-tile
  // (the fragment double buffer alternates per step and restarts at buffer 0
  // on every k-tile, which takes an even step count)
  static_assert(KS % 2 == 0, "MFMA steps per k-tile");
  bf16x8 fa[2][TN], fb[2][TM];
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);
  wait_vmcnt<(NS - 2) * LOADS>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  issue(NS - 1);
  read_half(0, 0, fa[0], fb[0]);

  for (int kt = 0; kt < nk - 1; ++kt) {
    const int st = kt % NS;
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      read_half(st, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      mfma_half(fa[ks & 1], fb[ks & 1]);
      interleave();
    }
    // tile kt+1 landed (NS-2 later tiles may still be in flight); our reads of slot st are done
    wait_vmcnt<(NS - 2) * LOADS>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(kt + NS);
    // Large tiles: the waves leaving the barrier take issue priority while they
    // read the new tile's first fragments and run the MFMAs that cover those
    // reads, so the matrix pipe restarts before the other wave of the SIMD
    // competes (measured +0.9 % on the 7B-shaped block prefill, +0.2 % on 8B).
    if constexpr (BM > 64) __builtin_amdgcn_s_setprio(1);
    read_half((kt + 1) % NS, 0, fa[KS & 1], fb[KS & 1]);
    mfma_half(fa[(KS - 1) & 1], fb[(KS - 1) & 1]);
    interleave();
    if constexpr (BM > 64) __builtin_amdgcn_s_setprio(0);
  }
#pragma unroll
  for (int ks = 0; ks < KS - 1; ++ks) {
    read_half((nk - 1) % NS, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
    mfma_half(fa[ks & 1], fb[ks & 1]);
    interleave();
  }
  mfma_half(fa[(KS - 1) & 1], fb[(KS - 1) & 1]);
  // no DMA may still be writing LDS when the workgroup retires
  wait_vmcnt<0>();

  // Accumulator element g*4 + i of acc[a][b] is output row m = (b * MI + lrow)
  // and column n = a * MI + g * 8 + lk * 4 + i of the wave's tile.  The lane's
  // coordinates are recomputed here instead of being kept live through the
  // k-loop, which needs every VGPR (kept, a few of them spilled to scratch).
  {
    const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int lrow = lane % MI, lk = lane / MI;
    const int wm = wave_u % WAVES_M, wn = wave_u / WAVES_M;
    using pre_t = decltype(epi_pre(epi, epi_row(epi, 0), 0));
    using row_t = decltype(epi_row(epi, 0));
    // Interior tiles of the 16x16x32 kernel whose rows are 16-byte aligned: the
    // lane rows trade halves of two 16-column accumulator tiles (lane-row pairs
    // 0/1 and 2/3, v_permlane16_swap), so that every lane holds 8 consecutive
    // columns of its output row and stores them as 16 bytes.  Half the store
    // instructions, each writing 64 contiguous bytes per row instead of 32
    // (measured on plain products at M = 131072: 2-3 us less per tile).
    constexpr bool kVec8 = MI == 16 && NV == 1 && !SPLIT && (DUAL ? (TN / 2) % 2 == 0 : TN % 2 == 0);
    bool vec8_done = false;
    if constexpr (kVec8) {
      if (m0 + BM <= M && n0 + BN_OUT <= N && epi_vec8_ok(epi)) {
        vec8_done = true;
        const int lrow4 = lane >> 4;                                 // lane row
        const int ncol = (lrow4 & 1) * MI + (lrow4 >> 1) * 8;         // its 8 columns within a tile pair
        if constexpr (DUAL) {
          float rsc8[TM];
#pragma unroll
          for (int b = 0; b < TM; ++b) rsc8[b] = epi.row_scale(m0 + wm * WM + b * MI + lrow);
#pragma unroll
          for (int b = 0; b < TM; ++b) {
            const int m = m0 + wm * WM + b * MI + lrow;
#pragma unroll
            for (int p = 0; p < TN / 2; p += 2) {
              f32x4 a1lo, a1hi, a3lo, a3hi;
              pair_transpose16(acc[p][b], acc[p + 1][b], a1lo, a1hi);
              pair_transpose16(acc[TN / 2 + p][b], acc[TN / 2 + p + 1][b], a3lo, a3hi);
              epi.apply8(m, n0 + wn * (WN / 2) + p * MI + ncol, a1lo, a1hi, a3lo, a3hi, rsc8[b]);
            }
          }
        } else {
          using pre8_t = decltype(epi_pre8(epi, epi_row(epi, 0), 0));
          constexpr bool kNoPre8 = std::is_same<pre8_t, NoPre>::value;
          constexpr int HB = (!kNoPre8 && sizeof(pre8_t) <= 16 && TM > 2) ? TM / 4 : 1;
#pragma unroll
          for (int b0 = 0; b0 < TM; b0 += HB) {
            pre8_t pre[HB][TN / 2];
            row_t rows[HB];
#pragma unroll
            for (int bb = 0; bb < HB; ++bb) {
              rows[bb] = epi_row(epi, m0 + wm * WM + (b0 + bb) * MI + lrow);
#pragma unroll
              for (int p = 0; p < TN / 2; ++p)
                pre[bb][p] = epi_pre8(epi, rows[bb], n0 + wn * WN + 2 * p * MI + ncol);
            }
#pragma unroll
            for (int bb = 0; bb < HB; ++bb) {
#pragma unroll
              for (int p = 0; p < TN / 2; ++p) {
                f32x4 lo, hi;
                pair_transpose16(acc[2 * p][b0 + bb], acc[2 * p + 1][b0 + bb], lo, hi);
                epi_apply8(epi, rows[bb], n0 + wn * WN + 2 * p * MI + ncol, lo, hi, pre[bb][p]);
              }
            }
          }
        }
      }
    }
    if (!vec8_done) {
    // Epilogues with pre-loads (the residual, the RoPE table) fetch them for a
    // batch of the wave's rows before any of those rows' stores: the stores may
    // alias the loads (in-place residual), so the compiler would otherwise wait
    // out one load round trip per store (residual).  A quarter of the rows per
    // batch for 8-byte pre-loads, one row for the 16-byte (cos, sin) pairs:
    // more next to the accumulators spill VGPRs.  Rows past M and columns past
    // N load a clamped, valid element.
    constexpr bool kBatched = !DUAL && !SPLIT && !std::is_same<pre_t, NoPre>::value;
    if constexpr (kBatched) {
      constexpr int HB = (sizeof(pre_t) <= 8 && TM > 2) ? TM / 4 : 1;
#pragma unroll
      for (int b0 = 0; b0 < TM; b0 += HB) {
        pre_t pre[HB][TN][NV];
        row_t rows[HB];
#pragma unroll
        for (int bb = 0; bb < HB; ++bb) {
          const int m = min(m0 + wm * WM + (b0 + bb) * MI + lrow, M - 1);
          rows[bb] = epi_row(epi, m);
#pragma unroll
          for (int a = 0; a < TN; ++a)
#pragma unroll
            for (int g = 0; g < NV; ++g) {
              const int n = n0 + wn * WN + a * MI + g * 8 + lk * 4;
              pre[bb][a][g] = epi_pre(epi, rows[bb], min(n, N - 4));
            }
        }
#pragma unroll
        for (int bb = 0; bb < HB; ++bb) {
          const int b = b0 + bb;
          const int m = m0 + wm * WM + b * MI + lrow;
          if (m >= M) continue;
#pragma unroll
          for (int a = 0; a < TN; ++a)
#pragma unroll
            for (int g = 0; g < NV; ++g) {
              const int n = n0 + wn * WN + a * MI + g * 8 + lk * 4;
              if (n >= N) continue;
              f32x4 v = {acc[a][b][g * 4], acc[a][b][g * 4 + 1], acc[a][b][g * 4 + 2], acc[a][b][g * 4 + 3]};
              epi_apply(epi, rows[bb], n, v, pre[bb][a][g]);
            }
        }
      }
    }
    // the dual epilogue's per-row factors, all fetched before the first store
    float rsc[DUAL && !SPLIT ? TM : 1];
    if constexpr (DUAL && !SPLIT) {
#pragma unroll
      for (int b = 0; b < TM; ++b) rsc[b] = epi.row_scale(min(m0 + wm * WM + b * MI + lrow, M - 1));
    }
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      if constexpr (kBatched) break;
      const int m = m0 + wm * WM + b * MI + lrow;
      if (m >= M) continue;
      if constexpr (DUAL) {
#pragma unroll
        for (int a = 0; a < TN / 2; ++a)
#pragma unroll
          for (int g = 0; g < NV; ++g) {
            const int n = n0 + wn * (WN / 2) + a * MI + g * 8 + lk * 4;
            if (n >= N) continue;
            f32x4 v1 = {acc[a][b][g * 4], acc[a][b][g * 4 + 1], acc[a][b][g * 4 + 2], acc[a][b][g * 4 + 3]};
            const acc_t& a3 = acc[a + TN / 2][b];
            f32x4 v3 = {a3[g * 4], a3[g * 4 + 1], a3[g * 4 + 2], a3[g * 4 + 3]};
            if constexpr (SPLIT) {
              float* p = partial + ((int64_t)blockIdx.z * M + m) * (2 * (int64_t)N);
              *(f32x4*)(p + n) = v1;
              *(f32x4*)(p + N + n) = v3;
            } else {
              epi.apply(m, n, v1, v3, rsc[b]);
            }
          }
      } else if constexpr (SPLIT) {
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
          for (int g = 0; g < NV; ++g) {
            const int n = n0 + wn * WN + a * MI + g * 8 + lk * 4;
            if (n >= N) continue;
            f32x4 v = {acc[a][b][g * 4], acc[a][b][g * 4 + 1], acc[a][b][g * 4 + 2], acc[a][b][g * 4 + 3]};
            *(f32x4*)(partial + ((int64_t)blockIdx.z * M + m) * (int64_t)N + n) = v;
          }
      } else {
        // row-dependent parts once, then the fragment's epilogue loads, then its stores
        const auto row = epi_row(epi, m);
        decltype(epi_pre(epi, row, 0)) pre[TN][NV];
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
          for (int g = 0; g < NV; ++g) {
            const int n = n0 + wn * WN + a * MI + g * 8 + lk * 4;
            pre[a][g] = epi_pre(epi, row, min(n, N - 4));
          }
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
          for (int g = 0; g < NV; ++g) {
            const int n = n0 + wn * WN + a * MI + g * 8 + lk * 4;
            if (n >= N) continue;
            f32x4 v = {acc[a][b][g * 4], acc[a][b][g * 4 + 1], acc[a][b][g * 4 + 2], acc[a][b][g * 4 + 3]};
            epi_apply(epi, row, n, v, pre[a][g]);
          }
      }
    }
    }  // !vec8_done
  }
  };
  if constexpr (kResident) {
    const int ntile = tiles_m * tiles_n;
    for (int vt = blockIdx.x; vt < ntile; vt += (int)gridDim.x) {
      // every wave is past the previous tile's reads of the ring
      if (vt != (int)blockIdx.x) __builtin_amdgcn_s_barrier();
      tile(vt);
    }
  } else {
    tile((int)blockIdx.x);
  }
}

// ------------------------------------------------------------------ fp32 FMA kernel
// 64 x 64 output tile, BK = 16; each thread owns a 4 (m) x 4 (n) block with
// 4 consecutive columns per row, matching the epilogue interface.
template <bool DUAL, bool SPLIT, class Epi>
__global__ void __launch_bounds__(kThreads)
gemm_f32_fma(const float* __restrict__ A, int64_t lda, WeightRows<float> w, int M, int N, int K,
             int k_per_split, Epi epi, float* __restrict__ partial) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Ws[DUAL ? 2 : 1][BK][BN + 4];
  const int tid = threadIdx.x;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn, (int)blockIdx.x);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb = blockIdx.z * k_per_split, ke = min(K, kb + k_per_split);
  const int tx = tid % 16, ty = tid / 16;  // n block tx*4, m block ty*4
  float acc[DUAL ? 2 : 1][4][4] = {};
  // each thread stages 4 elements of A and 4 (x2) of W per k-tile; the next
  // tile's global loads are issued into registers before the current tile's
  // products, so their latency overlaps the arithmetic
  constexpr int EPT = BM * BK / kThreads;
  static_assert(EPT * kThreads == BM * BK && BM == BN, "staging");
  float ra[EPT], rw[DUAL ? 2 : 1][EPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + i * kThreads, r = e / BK, c = e % BK;
      const int m = m0 + r, n = n0 + r, k = k0 + c;
      ra[i] = (m < M && k < ke) ? A[(int64_t)m * lda + k] : 0.f;
      if (DUAL) {
        rw[0][i] = (n < N && k < ke) ? w.w0[(int64_t)n * K + k] : 0.f;
        rw[DUAL ? 1 : 0][i] = (n < N && k < ke) ? w.w1[(int64_t)n * K + k] : 0.f;
      } else {
        rw[0][i] = (n < N && k < ke) ? weight_row(w, n, K)[k] : 0.f;
      }
    }
  };
  if (kb < ke) gload(kb);
  for (int k0 = kb; k0 < ke; k0 += BK) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + i * kThreads, r = e / BK, c = e % BK;
      As[c][r] = ra[i];
#pragma unroll
      for (int d = 0; d < (DUAL ? 2 : 1); ++d) Ws[d][c][r] = rw[d][i];
    }
    __syncthreads();
    if (k0 + BK < ke) gload(k0 + BK);
#pragma unroll
    for (int c = 0; c < BK; ++c) {
      float a[4], b[DUAL ? 2 : 1][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[c][ty * 4 + i];
#pragma unroll
      for (int d = 0; d < (DUAL ? 2 : 1); ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) b[d][j] = Ws[d][c][tx * 4 + j];
#pragma unroll
      for (int d = 0; d < (DUAL ? 2 : 1); ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[d][i][j] = fmaf(a[i], b[d][j], acc[d][i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = m0 + ty * 4 + i, n = n0 + tx * 4;
    if (m >= M || n >= N) continue;
    f32x4 v = {acc[0][i][0], acc[0][i][1], acc[0][i][2], acc[0][i][3]};
    if (DUAL) {
      f32x4 v3 = {acc[DUAL ? 1 : 0][i][0], acc[DUAL ? 1 : 0][i][1], acc[DUAL ? 1 : 0][i][2],
                  acc[DUAL ? 1 : 0][i][3]};
      if (SPLIT) {
        float* p = partial + ((int64_t)blockIdx.z * M + m) * (2 * (int64_t)N);
        *(f32x4*)(p + n) = v;
        *(f32x4*)(p + N + n) = v3;
      } else {
        if constexpr (DUAL) epi(m, n, v, v3);
      }
    } else {
      if (SPLIT)
        *(f32x4*)(partial + ((int64_t)blockIdx.z * M + m) * (int64_t)N + n) = v;
      else if constexpr (!DUAL)
        epi(m, n, v);
    }
  }
}

// ------------------------------------------------------------------ split-K reduce
// Z lanes share one output group (4 columns of one row): lane z sums the splits
// z, z+Z, ... (independent loads in flight), xor-shuffles combine the Z partial
// sums and lane 0 applies the epilogue (Z chosen by launch_reduce).
template <bool DUAL, int Z, class Epi>
__global__ void __launch_bounds__(kThreads)
splitk_reduce(const float* __restrict__ partial, int splits, int M, int N, Epi epi) {
  const int64_t groups = (int64_t)M * (N / 4);
  const int zl = threadIdx.x % Z;
  for (int64_t gi = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / Z; gi < groups;
       gi += (int64_t)gridDim.x * (kThreads / Z)) {
    const int m = (int)(gi / (N / 4));
    const int n = (int)(gi % (N / 4)) * 4;
    const int64_t row = DUAL ? 2 * (int64_t)N : (int64_t)N;
    const int64_t stride = (int64_t)M * row;
    const float* p = partial + (int64_t)m * row + n;
    f32x4 s = {}, s3 = {};
#pragma unroll 4
    for (int z = zl; z < splits; z += Z) {
      s += *(const f32x4*)(p + z * stride);
      if (DUAL) s3 += *(const f32x4*)(p + z * stride + N);
    }
#pragma unroll
    for (int off = 1; off < Z; off <<= 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] += __shfl_xor(s[i], off, 64);
        if (DUAL) s3[i] += __shfl_xor(s3[i], off, 64);
      }
    }
    if (zl == 0) {
      if constexpr (DUAL)
        epi(m, n, s, s3);
      else
        epi(m, n, s);
    }
  }
}

// Split-K reduction fused with the residual add and the next RMSNorm, one
// 1024-thread workgroup per token row: y = r + sum_z partial[z] (rounded to the
// output type), then yn = y * g and rscale[m] = rsqrt(mean(y^2) + eps) from the
// rounded y, as the normalisation kernel would compute them from y in memory.
// Every lane issues its splits' loads four at a time (clamped to the last
// split, weighted 0 past the end).
__global__ void __launch_bounds__(1024)
reduce_residual_norm(const float* __restrict__ partial, int splits, int M, int N, const bf16* r, bf16* y,
                     const bf16* __restrict__ g, bf16* __restrict__ yn, float* __restrict__ rscale, float eps) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  const int64_t row = (int64_t)m * N;
  float ss = 0.f;
  for (int n = threadIdx.x * 4; n < N; n += 1024 * 4) {
    f32x4 s = load4(r + row + n);
    for (int z0 = 0; z0 < splits; z0 += 4) {
      f32x4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = *(const f32x4*)(partial + ((int64_t)min(z0 + i, splits - 1) * M + m) * N + n);
#pragma unroll
      for (int i = 0; i < 4; ++i) s += z0 + i < splits ? v[i] : f32x4{};
    }
    const bf16x4 yb = {(bf16)s[0], (bf16)s[1], (bf16)s[2], (bf16)s[3]};
    *(bf16x4*)(y + row + n) = yb;
    const f32x4 gv = load4(g + n);
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = (float)yb[i];
      ss += f * f;
      o[i] = f * gv[i];
    }
    store4(yn + row + n, o);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) tot += red[i];
    rscale[m] = 1.0f / sqrtf(tot / (float)N + eps);
  }
}

// ------------------------------------------------------------------ launch
template <bool DUAL, class Epi>
hipError_t launch_reduce(const float* partial, int splits, int M, int N, Epi epi, hipStream_t st) {
  const int64_t groups = (int64_t)M * (N / 4);
  // lanes per group: eight when the groups are few (one token: the latency of
  // the split walk dominates), two for decode-sized outputs (measured over whole
  // 32-layer batch-64 decode steps: 6.61 ms with eight, 6.55 with one or four,
  // 6.48 with two), one for prefill-sized outputs, which run at HBM speed
  if (groups < 32768) {
    const int blocks = (int)((groups * 8 + kThreads - 1) / kThreads);
    splitk_reduce<DUAL, 8, Epi><<<blocks, kThreads, 0, st>>>(partial, splits, M, N, epi);
  } else if (groups < (1 << 20)) {
    const int blocks = (int)((groups * 2 + kThreads - 1) / kThreads);
    splitk_reduce<DUAL, 2, Epi><<<blocks, kThreads, 0, st>>>(partial, splits, M, N, epi);
  } else {
    const int blocks = (int)((groups + kThreads - 1) / kThreads);
    splitk_reduce<DUAL, 1, Epi><<<blocks < 16384 ? blocks : 16384, kThreads, 0, st>>>(partial, splits, M, N, epi);
  }
  return hipGetLastError();
}

// Workgroups of `kernel` resident at once on the current device (CUs x blocks per
// CU), or 0 if the runtime cannot say.  The CU count is read once per process.
int resident_blocks(const void* kernel, int threads) {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    return n;
  }();
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess) return 0;
  return cus * per;
}

template <int BM, int BN, int BK, int WAVES_M, int NS, bool DUAL, int NW, int MI = 32, class Epi>
hipError_t launch_dma(const bf16* A, int64_t lda, WeightRows<bf16> w, int M, int N, int K, Epi epi, int splits,
                      float* partial, hipStream_t st) {
  const int bn_out = DUAL ? BN / 2 : BN;
  const int tiles = ((M + BM - 1) / BM) * ((N + bn_out - 1) / bn_out);
  int kps = (K + splits - 1) / splits;
  kps = (kps + BK - 1) / BK * BK;
  // every split must own at least one whole k-tile
  if (K % BK != 0 || K < BK || (int64_t)(splits - 1) * kps >= K) return hipErrorInvalidValue;
  dim3 grid(tiles, 1, splits);
  if (splits > 1) {
    gemm_bf16_dma<BM, BN, BK, WAVES_M, NS, DUAL, true, Epi, NW, MI>
        <<<grid, NW * 64, 0, st>>>(A, lda, w, M, N, K, kps, epi, partial);
  } else {
    auto* kern = gemm_bf16_dma<BM, BN, BK, WAVES_M, NS, DUAL, false, Epi, NW, MI>;
    if (kResidentLargeTiles && BM > 64) {
      const int res = resident_blocks((const void*)kern, NW * 64);
      if (res <= 0) return hipErrorInvalidDeviceFunction;
      grid.x = (unsigned)std::min(tiles, res);
    }
    kern<<<grid, NW * 64, 0, st>>>(A, lda, w, M, N, K, kps, epi, partial);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits <= 1) return e;
  return launch_reduce<DUAL, Epi>(partial, splits, M, N, epi, st);
}
template <int BM, int BN, int WM_, int WN_, bool DUAL, class Epi>
hipError_t launch_mfma(const bf16* A, int64_t lda, WeightRows<bf16> w, int M, int N, int K, Epi epi,
                       int splits, float* partial, hipStream_t st) {
  constexpr int BK = 64;
  const int bn_out = DUAL ? BN / 2 : BN;
  const int tiles = ((M + BM - 1) / BM) * ((N + bn_out - 1) / bn_out);
  int kps = (K + splits - 1) / splits;
  kps = (kps + BK - 1) / BK * BK;
  dim3 grid(tiles, 1, splits);
  if (splits > 1)
    gemm_bf16_mfma<BM, BN, BK, WM_, WN_, DUAL, true, Epi>
        <<<grid, kThreads, 0, st>>>(A, lda, w, M, N, K, kps, epi, partial);
  else
    gemm_bf16_mfma<BM, BN, BK, WM_, WN_, DUAL, false, Epi>
        <<<grid, kThreads, 0, st>>>(A, lda, w, M, N, K, kps, epi, partial);
  return hipGetLastError();
}

template <bool DUAL, class Epi>
hipError_t launch_bf16(const bf16* A, int64_t lda, WeightRows<bf16> w, int M, int N, int K, Epi epi,
                       int splits, float* partial, hipStream_t st) {
  // the DMA-pipelined kernels need K (and each split's K range) in whole k-tiles
  // (BK = kSkinnyBK for small M, kBigBK otherwise), 16-byte aligned rows, the
  // row map's tensor boundaries on multiples of 8 rows (one tensor per DMA
  // block) and 32-bit byte offsets within a 256-row panel
  const bool one_tensor = w.n1 >= N && w.n2 >= N;
  const bool dma_ok = lda % 8 == 0 && (one_tensor || (w.n1 % 8 == 0 && w.n2 % 8 == 0)) &&
                      (int64_t)256 * (lda > K ? lda : K) * 2 < ((int64_t)1 << 32);
  if (dma_ok && M <= 64 && K % kSkinnyBK == 0) {
    if (M <= 32) {
      if constexpr (DUAL)
        return launch_dma<32, 256, kSkinnyBK, 1, kSkinnyStages, DUAL, 4>(A, lda, w, M, N, K, epi, splits,
                                                                           partial, st);
      else
        return launch_dma<32, 128, kSkinnyBK, 1, kSkinnyStages, DUAL, 4>(A, lda, w, M, N, K, epi, splits,
                                                                           partial, st);
    }
    if constexpr (DUAL)
      return launch_dma<64, 128, kSkinnyBK, 2, kSkinnyStages, DUAL, 4>(A, lda, w, M, N, K, epi, splits,
                                                                       partial, st);
    else
      return launch_dma<64, 128, kSkinnyBK, 2, kSkinnyStages64, DUAL, 4>(A, lda, w, M, N, K, epi, splits,
                                                                         partial, st);
  }
  if (dma_ok && M > 64 && K % kBigBK == 0)
    return launch_dma<256, 256, kBigBK, 2, kBigStages, DUAL, kBigWaves, kBigMI>(A, lda, w, M, N, K, epi, splits, partial,
                                                                        st);
  hipError_t e;
  if (M <= 32) {
    if constexpr (DUAL)
      e = launch_mfma<32, 256, 1, 4, DUAL>(A, lda, w, M, N, K, epi, splits, partial, st);
    else
      e = launch_mfma<32, 128, 1, 4, DUAL>(A, lda, w, M, N, K, epi, splits, partial, st);
  } else if (M <= 64) {
    e = launch_mfma<64, 256, 2, 2, DUAL>(A, lda, w, M, N, K, epi, splits, partial, st);
  } else {
    e = launch_mfma<256, 256, 2, 2, DUAL>(A, lda, w, M, N, K, epi, splits, partial, st);
  }
  if (e != hipSuccess || splits <= 1) return e;
  return launch_reduce<DUAL, Epi>(partial, splits, M, N, epi, st);
}

template <bool DUAL, class Epi>
hipError_t launch_f32(const float* A, int64_t lda, WeightRows<float> w, int M, int N, int K, Epi epi,
                      int splits, float* partial, hipStream_t st) {
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  int kps = (K + splits - 1) / splits;
  kps = (kps + 15) / 16 * 16;
  dim3 grid(tiles, 1, splits);
  if (splits > 1)
    gemm_f32_fma<DUAL, true, Epi><<<grid, kThreads, 0, st>>>(A, lda, w, M, N, K, kps, epi, partial);
  else
    gemm_f32_fma<DUAL, false, Epi><<<grid, kThreads, 0, st>>>(A, lda, w, M, N, K, kps, epi, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits <= 1) return e;
  return launch_reduce<DUAL, Epi>(partial, splits, M, N, epi, st);
}

}  // namespace

bool gemm_residual_norm_fits(int M, int N, int K, int64_t lda) {
  return M > kGemvMaxM && M <= 64 && N % 4 == 0 && lda % 8 == 0 && K % kSkinnyBK == 0 &&
         (int64_t)256 * (lda > K ? lda : K) * 2 < ((int64_t)1 << 32) &&
         gemm_pick_splits(M, N, K, false, true) > 1;
}

hipError_t gemm_residual_norm_launch(const bf16* A, int64_t lda, const bf16* w, int M, int N, int K, bf16* y,
                                     const bf16* r, const bf16* g, bf16* yn, float* rscale, float eps,
                                     float* partial, hipStream_t st) {
  if (!gemm_residual_norm_fits(M, N, K, lda)) return hipErrorInvalidValue;
  const int splits = gemm_pick_splits(M, N, K, false, true);
  WeightRows<bf16> wr{w, nullptr, nullptr, N, N};
  EpiResidual<bf16> epi{y, r, N};   // (type only: the splits write partials)
  const int tiles = (N + 127) / 128;
  int kps = (K + splits - 1) / splits;
  kps = (kps + kSkinnyBK - 1) / kSkinnyBK * kSkinnyBK;
  if ((int64_t)(splits - 1) * kps >= K) return hipErrorInvalidValue;
  dim3 grid(tiles, 1, splits);
  if (M <= 32)
    gemm_bf16_dma<32, 128, kSkinnyBK, 1, kSkinnyStages, false, true, EpiResidual<bf16>, 4, 32>
        <<<grid, 256, 0, st>>>(A, lda, wr, M, N, K, kps, epi, partial);
  else
    gemm_bf16_dma<64, 128, kSkinnyBK, 2, kSkinnyStages64, false, true, EpiResidual<bf16>, 4, 32>
        <<<grid, 256, 0, st>>>(A, lda, wr, M, N, K, kps, epi, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  reduce_residual_norm<<<M, 1024, 0, st>>>(partial, splits, M, N, r, y, g, yn, rscale, eps);
  return hipGetLastError();
}

int gemm_pick_splits(int M, int N, int K, bool dual, bool is_bf16) {
  if (M > 64) {
    // 256 x 256 tiles: split K only when the tiles would leave at least half the
    // CUs idle (a 2048-token chunk's wo and w2 make 128 tiles), each split keeping
    // at least 8 k-tiles of pipeline; otherwise one pass over K
    if (!is_bf16 || K % kBigBK != 0) return 1;
    const int tiles = ((M + 255) / 256) * ((N + (dual ? 127 : 255)) / (dual ? 128 : 256));
    if (tiles > kCUs / 2) return 1;
    const int nkt = K / kBigBK;
    const int s = min(kCUs / tiles, nkt / 8);
    if (s <= 1) return 1;
    const int per = (nkt + s - 1) / s;
    return (nkt + per - 1) / per;
  }
  // up to four tokens: the weight-streaming kernel, one pass over K
  // (gemm_launch sends the problem there when its shapes allow)
  if (is_bf16 ? gemv_fits<bf16>(M, N, K, K) : gemv_fits<float>(M, N, K, K)) return 1;
  // small token count: the weights stream from HBM once; split K so that the
  // grid covers the CUs
  if (is_bf16 && K % kSkinnyBK == 0) {
    // LDS-DMA kernel: aim at one workgroup per CU (fewer splits measured faster
    // than oversubscribing, also with rings small enough for two per CU: every
    // split adds an fp32 partial tile and shortens the pipeline), each split
    // keeping at least a ring's depth of k-tiles
    const int bn_out = dual ? (M <= 32 ? 128 : 64) : 128;
    const int stages = (M <= 32 || dual) ? kSkinnyStages : kSkinnyStages64;
    const int tiles = (N + bn_out - 1) / bn_out;
    const int nkt = K / kSkinnyBK;
    int s = tiles >= kCUs ? 1 : kCUs / tiles;
    s = min(s, max(1, nkt / stages));
    // every split must own at least one k-tile: use the count the rounding yields
    const int per = (nkt + s - 1) / s;
    return (nkt + per - 1) / per;
  }
  int bn, bk;
  if (is_bf16) {                         // register-staged kernel
    bn = (dual || M <= 32) ? 128 : 256;
    bk = 64;
  } else {
    bn = 64;
    bk = 16;
  }
  const int tiles = (N + bn - 1) / bn;
  const int max_splits = K / (bk * 4);
  int s = 1;
  while (tiles * s < 1024 && s * 2 <= max_splits && s < 32) s *= 2;
  return s;
}

template <typename T, class Epi>
hipError_t gemm_launch(const T* A, int64_t lda, WeightRows<T> w, int M, int N, int K, Epi epi,
                       int splits, float* partial, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (gemv_fits<T>(M, N, K, lda) && w.n1 % 4 == 0 && w.n2 % 4 == 0)
    return gemv_launch<T, Epi>(A, lda, w, M, N, K, nullptr, 0.0f, epi, st);
  if constexpr (sizeof(T) == 2)
    return launch_bf16<false>(A, lda, w, M, N, K, epi, splits, partial, st);
  else
    return launch_f32<false>(A, lda, w, M, N, K, epi, splits, partial, st);
}

template <typename T, class Epi>
hipError_t gemm_dual_launch(const T* A, int64_t lda, const T* w1, const T* w3, int M, int N, int K,
                            Epi epi, int splits, float* partial, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  WeightRows<T> w{w1, w3, nullptr, N, N};
  if (gemv_fits<T>(M, N, K, lda)) return gemv_dual_launch<T, Epi>(A, lda, w1, w3, M, N, K, nullptr, 0.0f, epi, st);
  if constexpr (sizeof(T) == 2)
    return launch_bf16<true>(A, lda, w, M, N, K, epi, splits, partial, st);
  else
    return launch_f32<true>(A, lda, w, M, N, K, epi, splits, partial, st);
}

#define LLAMA_GEMM_INST(T)                                                                      \
  template hipError_t gemm_launch<T, EpiStore<T>>(const T*, int64_t, WeightRows<T>, int, int, int, \
                                                  EpiStore<T>, int, float*, hipStream_t);       \
  template hipError_t gemm_launch<T, EpiResidual<T>>(const T*, int64_t, WeightRows<T>, int, int,   \
                                                     int, EpiResidual<T>, int, float*,          \
                                                     hipStream_t);                              \
  template hipError_t gemm_launch<T, EpiQKV<T>>(const T*, int64_t, WeightRows<T>, int, int, int,   \
                                                EpiQKV<T>, int, float*, hipStream_t);           \
  template hipError_t gemm_launch<T, EpiF32>(const T*, int64_t, WeightRows<T>, int, int, int,      \
                                             EpiF32, int, float*, hipStream_t);                 \
  template hipError_t gemm_dual_launch<T, EpiSwiGLU<T>>(const T*, int64_t, const T*, const T*, int, \
                                                        int, int, EpiSwiGLU<T>, int, float*,     \
                                                        hipStream_t);

LLAMA_GEMM_INST(bf16)
LLAMA_GEMM_INST(float)

}  // namespace llama
