// Dense linears of the block: Y = op(A) W^T with fused epilogues (store,
// float32 store, erf-form GELU, gated residual x += gate[seg] * y).
//
// The gating and residual chain is fused into the producing GEMM (blog
// close-reading 2.2(3): norm, RoPE, gating and residual chains are fused so
// intermediates stay on chip).  Three kernels:
//   gemm_mfma_kernel   bf16, MFMA 32x32x16, LDS double buffer, grouped over
//                      up to two problems (image and text streams) per launch;
//                      the 256x256 tile runs 4 waves on an explicitly
//                      pipelined mainloop (mma_tile_pipe)
//   gemm_skinny_kernel bf16, M <= 16, K % 256 == 0 (adaLN modulation,
//                      conditioning MLP):
//                      weight-streaming MFMA 16x16x32 with split-K over waves
//   gemm_simt_kernel   float32 (and any shape the MFMA kernels reject)
#include "common.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#ifndef MMDIT_PERSIST_DEFAULT
#define MMDIT_PERSIST_DEFAULT 1
#endif

namespace mmdit {

namespace {

struct GemmProb {
  const void* A;
  const void* W;
  void* Y;
  const float* gate;
  const int32_t* seg;
  void* aux;            // [M, N] dense (kEpi*Aux outputs, kEpiGeluBwd input; [M, 2H] for kEpiQkRopeAux)
  const float* rope_cs; // kEpiQkRope*: [M][D/2] (cos, sin) per row and rotation pair (NULL: no rotation)
  const float* g_q;     // kEpiQkRope*: QK-norm gains [D]
  const float* g_k;
  const bf16* xt_e;     // noised A staging (SITE 2): eps, per-sample t, per-row sample and position, z_t copy
  const float* xt_t;
  const int32_t* xt_seg;
  const int32_t* xt_pos;
  bf16* xt_zt;
  int64_t lda, ldy, gate_stride, M;
  int32_t N, K;
  int32_t tiles_n;
  int32_t tile_begin;
};

struct QkDims {
  int32_t heads, D;
  float eps;
};

struct GemmBatch {
  GemmProb p[2];
  int32_t nprob;
  const char* tag;
  int32_t site;
  int32_t xcd_remap;   // renumber tiles per XCD (off when grouped problems differ in K)
  int32_t splitk;      // > 1: blockIdx.y takes 1/splitk of K and writes float32 partials
  float* partial;      // [splitk][M][N] (single problem)
  int64_t partial_elems;
  int32_t tail_begin;   // > 0: blocks from here on share the tiles tail_begin.. (last-round fill)
  int32_t tail_chunks;  // blocks (sub-tiles) per last-round tile: 2, 4 or 8
  // > 0: the whole 256x256 tiles of the pipelined 4-wave shape are run by
  // `persist` blocks (one per CU), block b taking tiles b, b + persist, ...
  // of the XCD-renumbered order; last-round sub-tile blocks follow them
  int32_t persist;
  int32_t ntiles;       // whole tiles of the launch (persistent form)
  QkDims qk;            // kEpiQkRope*: heads, head dim, eps
  // split last round (gemm_sk_part_kernel): tiles sk_full.. are cut along k
  // into sk_S parts of sk_P 64-deep steps whose float32 partial tiles
  // gemm_sk_fixup_kernel sums in k order
  int32_t sk_full, sk_tail, sk_S, sk_P;
  float* sk_partial;    // [sk_tail][sk_S][256][256]
  // split-K reduction of a bf16 store that also sums the flow-matching
  // squared residuals of each row (row_sse non-NULL)
  const bf16* sse_z;
  const bf16* sse_e;
  const int32_t* sse_row;
  float* row_sse;
  int32_t* sse_done;
};

__device__ __forceinline__ const GemmProb& pick(const GemmBatch& bt, int& tile) {
  if (bt.nprob > 1 && tile >= bt.p[1].tile_begin) {
    tile -= bt.p[1].tile_begin;
    return bt.p[1];
  }
  return bt.p[0];
}

template <typename T, int EPI>
__device__ __forceinline__ void epi_store(const GemmProb& P, int64_t m, int n, float acc) {
  if constexpr (EPI == MMDIT_EPI_STORE_F32) {
    static_cast<float*>(P.Y)[m * P.ldy + n] = acc;
  } else if constexpr (EPI == MMDIT_EPI_STORE) {
    static_cast<T*>(P.Y)[m * P.ldy + n] = from_f<T>(acc);
  } else if constexpr (EPI == MMDIT_EPI_GELU) {
    static_cast<T*>(P.Y)[m * P.ldy + n] = from_f<T>(gelu_f(acc));
  } else if constexpr (EPI == kEpiGeluAux) {
    static_cast<T*>(P.Y)[m * P.ldy + n] = from_f<T>(gelu_f(acc));
    static_cast<T*>(P.aux)[m * P.N + n] = from_f<T>(acc);
  } else if constexpr (EPI == kEpiGeluBwd) {
    const float x = to_f(static_cast<const T*>(P.aux)[m * P.N + n]);
    static_cast<T*>(P.Y)[m * P.ldy + n] = from_f<T>(acc * gelu_grad_f(x));
  } else if constexpr (EPI == kEpiQkRope || EPI == kEpiQkRopeAux) {
    // QK-RMSNorm + RoPE needs whole head rows: only the 256x256 LDS epilogue
    // applies it, and linear() launches these epilogues on that tile alone
    static_cast<T*>(P.Y)[m * P.ldy + n] = from_f<T>(acc);
  } else {
    T* y = static_cast<T*>(P.Y) + m * P.ldy + n;
    const float g = P.gate[(int64_t)P.seg[m] * P.gate_stride + n];
    *y = from_f<T>(to_f(*y) + g * acc);
    if constexpr (EPI == kEpiGatedResAux) static_cast<T*>(P.aux)[m * P.N + n] = from_f<T>(acc);
  }
}

// ------------------------------------------------------------------ SIMT
template <typename T, int EPI, bool SILU>
__global__ void __launch_bounds__(256) gemm_simt_kernel(GemmBatch bt) {
  int tile = blockIdx.x;
  const GemmProb& P = pick(bt, tile);
  const int64_t m0 = (int64_t)(tile / P.tiles_n) * 64;
  const int n0 = (tile % P.tiles_n) * 64;
  __shared__ float As[16][68], Ws[16][68];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const T* A = static_cast<const T*>(P.A);
  const T* W = static_cast<const T*>(P.W);
  float acc[4][4] = {};
  const int lr = threadIdx.x >> 2, lk = (threadIdx.x & 3) * 4;
  for (int k0 = 0; k0 < P.K; k0 += 16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = k0 + lk + e;
      const int64_t m = m0 + lr;
      float a = (m < P.M && k < P.K) ? to_f(A[m * P.lda + k]) : 0.f;
      if (SILU) a = silu_f(a);
      As[lk + e][lr] = a;
      const int n = n0 + lr;
      Ws[lk + e][lr] = (n < P.N && k < P.K) ? to_f(W[(int64_t)n * P.K + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        w[i] = Ws[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= P.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < P.N) epi_store<T, EPI>(P, m, n, acc[i][j]);
    }
  }
}

__device__ __forceinline__ bf16x8 silu8(bf16x8 x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)silu_f((float)x[i]);
  return r;
}

// ---------------------------------------------------------------- skinny
// One block per 16 * NG output columns (NG MFMA column groups sharing each A
// fragment, so A is read once per 16 * NG weight rows); 8 waves split K into
// 8 contiguous ranges (K % 256 == 0), each keeping U A loads and U * NG
// weight loads (16 B each) in flight before its MFMAs; fixed-order reduction
// of the 8 partial tiles through LDS.  NG = 4 for wide outputs, NG = 1 when
// that would leave too few blocks to fill the chip.
template <int EPI, bool SILU, int NG>
__global__ void __launch_bounds__(512) gemm_skinny_kernel(GemmBatch bt) {
  constexpr int U = NG == 1 ? 8 : 4;
  int tile = blockIdx.x;
  const GemmProb& P = pick(bt, tile);
  const int n0 = tile * 16 * NG;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kq = P.K >> 3;
  const int kbeg = wave * kq;
  const int r16 = lane & 15, kofs = (lane >> 4) * 8;
  const bf16* A = static_cast<const bf16*>(P.A) + (int64_t)r16 * P.lda + kofs + kbeg;
  const bf16* W = static_cast<const bf16*>(P.W) + (int64_t)(n0 + r16) * P.K + kofs + kbeg;
  const int64_t gstride = (int64_t)16 * P.K;   // next column group's weight rows
  const bool arow = r16 < P.M;
  f32x4 acc[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nit = kq >> 5;
  int it = 0;
  for (; it + U <= nit; it += U) {
    bf16x8 b[U][NG], a[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < NG; ++g) b[u][g] = *reinterpret_cast<const bf16x8*>(W + g * gstride + (it + u) * 32);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = bf16x8{};
      if (arow) a[u] = *reinterpret_cast<const bf16x8*>(A + (it + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (SILU) a[u] = silu8(a[u]);
#pragma unroll
      for (int g = 0; g < NG; ++g) acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u][g], acc[g], 0, 0, 0);
    }
  }
  for (; it < nit; ++it) {
    bf16x8 a = {};
    if (arow) {
      a = *reinterpret_cast<const bf16x8*>(A + it * 32);
      if (SILU) a = silu8(a);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(W + g * gstride + it * 32);
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[g], 0, 0, 0);
    }
  }
  __shared__ f32x4 red[8][NG][64];
#pragma unroll
  for (int g = 0; g < NG; ++g) red[wave][g][lane] = acc[g];
  __syncthreads();
  for (int g = wave; g < NG; g += 8) {
    f32x4 s = red[0][g][lane];
#pragma unroll
    for (int w = 1; w < 8; ++w) s += red[w][g][lane];
    // D[i][j]: j = lane % 16 (output column), i = 4 * (lane / 16) + v (row)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * (lane >> 4) + v;
      if (m < P.M) epi_store<bf16, EPI>(P, m, n0 + g * 16 + r16, s[v]);
    }
  }
}

// ------------------------------------------------------------------ MFMA
// Tile BM x BN x 64, WM x WN waves, each wave (BM/WM) x (BN/WN) built from
// 32x32x16 MFMA tiles.  Operands go global -> LDS directly
// (global_load_lds_dwordx4: each wave instruction fills 1 KB = 8 rows of 64
// bf16), double-buffered with one barrier per 64-deep k step.  LDS rows are
// 8 chunks of 16 B; chunk c of row r sits at position c ^ swz8(r), which the
// loads realise by choosing each lane's global chunk, so the 16-B fragment
// reads of the MFMA operands are free of bank conflicts.
__device__ __forceinline__ int swz8(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ int64_t cdiv_d(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Renumber so that each XCD receives one contiguous range of tiles.
__device__ __forceinline__ int xcd_tile(int hw, int total) {
  const int per = total >> 3, rem = total & 7;
  const int xcd = hw & 7, local = hw >> 3;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Tiles ordered in groups of 8 tile-rows, down the rows first: the tiles an
// XCD runs together share a few A row-blocks and a few W column-blocks.
__device__ __forceinline__ void grouped_tile(int tile, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = tile / per_group;
  const int first = group * GM;
  const int gsize = min(tiles_m - first, GM);
  const int r = tile - group * per_group;
  tm = first + r % gsize;
  tn = r / gsize;
}


// acc[TM][TN] += A[m0:m0+BM, K-steps kt0 .. kt0+nkt) W[n0:n0+BN, ...]^T for one
// tile.  Operands go global -> LDS directly (global_load_lds_dwordx4: one wave
// instruction fills 1 KB), NS-stage ring with one barrier per BK-deep step.
// Ends with a barrier, so the caller may reuse the LDS right away.
//
// XT: A is z and a second tile of the noise eps is staged beside it (after
// the W stages); each A fragment is z_t = (1 - t) z + t eps of its row (t =
// its sample's t on frame-0 rows, else 0), rounded to bf16, and the first
// column tile's wn == 0 waves also store it to xt_zt.
template <int BM, int BN, int WM, int WN, bool SILU, int BK, int NS, bool XT = false>
__device__ __forceinline__ void mma_tile(const GemmProb& P, int64_t m0, int n0, int kt0, int nkt, bf16* smem,
                                         f32x16 (&acc)[BM / WM / 32][BN / WN / 32]) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  constexpr int CPR = BK / 8;            // 16-B chunks per LDS row
  constexpr int RPB = 64 / CPR;          // rows per 1-KB block (one wave instruction)
  constexpr int ABLK = BM / RPB, BBLK = BN / RPB;
  static_assert(ABLK % NW == 0 && BBLK % NW == 0, "tile / wave mismatch");
  constexpr int LPS = (XT ? 2 : 1) * (ABLK / NW) + BBLK / NW;   // direct loads per stage per wave
  static_assert(NS <= 4 && 2 * LPS < 64, "vmcnt range");
  bf16* As = smem;                    // [NS][BM*BK]
  bf16* Bs = smem + NS * BM * BK;     // [NS][BN*BK]
  bf16* Es = Bs + NS * BN * BK;       // XT: [NS][BM*BK]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const bf16* A = static_cast<const bf16*>(P.A);
  const bf16* W = static_cast<const bf16*>(P.W);
  auto swz = [](int r) { return CPR == 16 ? (r & 15) : CPR == 8 ? swz8(r) : ((r >> 2) & 3); };

  // per-lane source of each 1-KB block this wave fills: row rr = lane / CPR of
  // the block, LDS chunk position p = lane % CPR holds global chunk p ^ swz(row)
  const int rr = lane / CPR, pp = lane % CPR;
  const bf16* asrc[ABLK / NW];
  const bf16* esrc[ABLK / NW];
  const bf16* bsrc[BBLK / NW];
#pragma unroll
  for (int i = 0; i < ABLK / NW; ++i) {
    const int row = (wave + i * NW) * RPB + rr;
    int64_t m = m0 + row;
    if (m >= P.M) m = P.M - 1;        // rows past M load a valid row; never stored
    asrc[i] = A + m * P.lda + ((pp ^ swz(row)) << 3);
    if constexpr (XT) esrc[i] = P.xt_e + m * P.lda + ((pp ^ swz(row)) << 3);
  }
#pragma unroll
  for (int i = 0; i < BBLK / NW; ++i) {
    const int row = (wave + i * NW) * RPB + rr;
    bsrc[i] = W + (int64_t)(n0 + row) * P.K + ((pp ^ swz(row)) << 3);
  }
  auto issue = [&](int kt) {
    const int st = kt % NS, ke = (kt0 + kt) * BK;
#pragma unroll
    for (int i = 0; i < ABLK / NW; ++i)
      load_lds16(asrc[i] + ke, As + st * BM * BK + (wave + i * NW) * 512);
    if constexpr (XT) {
#pragma unroll
      for (int i = 0; i < ABLK / NW; ++i)
        load_lds16(esrc[i] + ke, Es + st * BM * BK + (wave + i * NW) * 512);
    }
#pragma unroll
    for (int i = 0; i < BBLK / NW; ++i)
      load_lds16(bsrc[i] + ke, Bs + st * BN * BK + (wave + i * NW) * 512);
  };
  // wait until at most c stages of this wave's loads are still in flight
  auto wait_stages = [&](int c) {
    if (c <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (c == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LPS) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * LPS) : "memory");
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nkt) issue(s);
  wait_stages(min(NS - 1, nkt) - 1);
  __syncthreads();
  const int l32 = lane & 31, g = lane >> 5;
  // XT: each fragment row's t, and whether this wave stores z_t
  float tx[TM];
  if constexpr (XT) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + wm * TM * 32 + i * 32 + l32;
      tx[i] = (m < P.M && P.xt_pos[3 * m] == 0) ? P.xt_t[P.xt_seg[m]] : 0.0f;
    }
  }
  const bool zt_out = XT && P.xt_zt != nullptr && n0 == 0 && wn == 0;
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + NS - 1 < nkt) issue(kt + NS - 1);
    const bf16* as = As + (kt % NS) * BM * BK;
    const bf16* bs = Bs + (kt % NS) * BN * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[TM], bfr[TN];
      const int ch = kk * 2 + g;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * TM * 32 + i * 32 + l32;
        af[i] = *reinterpret_cast<const bf16x8*>(as + r * BK + ((ch ^ swz(r)) << 3));
        if (SILU) af[i] = silu8(af[i]);
        if constexpr (XT) {
          const bf16* es = Es + (kt % NS) * BM * BK;
          const bf16x8 ef = *reinterpret_cast<const bf16x8*>(es + r * BK + ((ch ^ swz(r)) << 3));
#pragma unroll
          for (int e = 0; e < 8; ++e) af[i][e] = (bf16)rf_xt((float)af[i][e], (float)ef[e], tx[i]);
          if (zt_out && m0 + r < P.M)
            *reinterpret_cast<bf16x8*>(P.xt_zt + (m0 + r) * P.lda + (int64_t)(kt0 + kt) * BK + ch * 8) = af[i];
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * TN * 32 + j * 32 + l32;
        bfr[j] = *reinterpret_cast<const bf16x8*>(bs + r * BK + ((ch ^ swz(r)) << 3));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    // stage kt + 1 must have landed (for every wave) before the next step
    wait_stages(min(nkt - 1, kt + NS - 1) - kt - 1);
    __syncthreads();
  }
}

// 256x256 tile on 4 waves (2x2, 128x128 each, accumulators in AGPRs) with an
// explicitly pipelined schedule.  Per BK=64 step a wave issues 64 MFMAs in
// four k-slices of 16; the fragments of slice kk+1 are read from LDS while
// the MFMAs of slice kk issue, each slice starting with MFMAs so its reads
// have a whole slice to land.  The stage switch (own loads landed, then a
// barrier) sits after the first quarter of the last slice; right after it the
// next stage's first fragments are read and the 16 direct-to-LDS loads of the
// stage after next issue (into the buffer just finished), between the rest of
// that slice's MFMAs, so the loads have a whole step to land.
// The order of the MFMAs on each accumulator is the same as mma_tile's.
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) char lds_char;

// One BK=64 step of mma_tile_pipe.  NEXT: a next stage exists and the step
// ends by switching to it.  LOAD2: stage kt + 2 exists; its loads issue right
// after that switch's barrier, into the buffer of stage kt, which every wave
// has finished reading by then (a whole step of MFMAs for them to land), and
// are followed by two 4-byte direct loads that touch every 128-byte row
// segment of stage kt + 3 (into a scratch strip past the stages) so that its
// loads find the rows in L2.
template <bool NEXT, bool LOAD2>
__device__ __forceinline__ void pipe_step(rsrc_t ra, rsrc_t rb, const uint32_t (&offa)[8],
                                          const uint32_t (&offb)[8], int kt, int KT, uint32_t pfa, uint32_t pfb,
                                          bf16* smem, const lds_char* lsm,
                                          const uint32_t (&aoff)[4], const uint32_t (&boff)[4],
                                          bf16x8 (&fa)[2][4], bf16x8 (&fb)[2][4], f32x16 (&acc)[4][4]) {
  constexpr int BM = 256, BK = 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int st = kt & 1;
  auto read_slice = [&](int s, int kk, int buf) {
    const uint32_t so = s * BM * BK * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[buf][j] = *reinterpret_cast<const lds_bf16x8*>(lsm + boff[(j & 1) ? (kk ^ 2) : kk] + so + j * 4096);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[buf][i] = *reinterpret_cast<const lds_bf16x8*>(lsm + aoff[(i & 1) ? (kk ^ 2) : kk] + so + i * 4096);
  };
  auto mma_rows = [&](int buf, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
  };
  __builtin_amdgcn_sched_barrier(0);
  // slices 0..2: MFMAs on one fragment buffer while the next slice is read
  // into the other; each slice starts with MFMAs
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    read_slice(st, kk + 1, (kk + 1) & 1);
    mma_rows(kk & 1, 0, 4);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // slice 3: a quarter of its MFMAs, the stage switch, then the next stage's
  // slice 0 and the loads of stage kt + 2 while the rest issue
  mma_rows(1, 0, 1);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NEXT) {
    // vmcnt(0) lgkmcnt(0): this wave's loads of stage kt + 1 have landed and
    // its reads of stage kt are done; after the barrier the same holds for
    // every wave.  The touch of stage kt + 2 was issued after those loads
    // (when stage kt + 2 exists, i.e. LOAD2), and loads complete in issue
    // order, so vmcnt(2) waits for the stage's loads only.
    if constexpr (LOAD2) __builtin_amdgcn_s_waitcnt(0x0072);
    else __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_slice(st ^ 1, 0, 0);
    if constexpr (LOAD2) {
      // stage kt + 2 into the buffer every wave has just finished (stage kt),
      // then the touch of stage kt + 3 (past the last stage it repeats the
      // last one): the 18 direct loads go between the 12 remaining MFMAs of
      // the slice, two after each of the first eight, one after each of the
      // next two, each fenced so the compiler keeps them there (grouped, they
      // held the matrix cores idle for the whole burst); buffer loads: the
      // tile's base in a scalar resource, the lane offset 32-bit, the k
      // offset scalar
      const uint32_t ks = (uint32_t)(kt + 2) * BK * 2;
      const int kt3 = kt + 3 < KT ? kt + 3 : KT - 1;
      const uint32_t ks3 = (uint32_t)kt3 * BK * 2;
      bf16* junk = smem + 2 * 2 * BM * BK + wave * 128;
#pragma unroll
      for (int q = 0; q < 12; ++q) {
        const int i = 1 + q / 4, j = q % 4;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1][i], fb[1][j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (q < 8) {
          buf_lds<16>(ra, offa[q], ks, smem + st * BM * BK + (wave + q * 4) * 512);
          buf_lds<16>(rb, offb[q], ks, smem + 2 * BM * BK + st * BM * BK + (wave + q * 4) * 512);
        } else if (q == 8) {
          buf_lds<4>(ra, pfa, ks3, junk);
        } else if (q == 9) {
          buf_lds<4>(rb, pfb, ks3, junk);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
  }
  mma_rows(1, 1, 4);
  if constexpr (NEXT) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (LOAD2) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// acc += A[m0:m0+256, k] W[n0:n0+256, k]^T over the 64-deep k steps
// kt0 .. kt0+nkt (all of K when nkt < 0; K % 64 == 0).  256 threads; smem
// holds two stages of both operands (128 KB).  Ends with a barrier, so the
// caller may reuse the LDS right away.
__device__ __forceinline__ void mma_tile_pipe(const GemmProb& P, int64_t m0, int n0, bf16* smem,
                                              f32x16 (&acc)[4][4], int kt0 = 0, int nkt = -1, int tid_in = -1) {
  constexpr int BM = 256, BK = 64;
  const int tid = tid_in >= 0 ? tid_in : (int)threadIdx.x, lane = tid & 63,
            wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int rr = lane >> 3, pp = lane & 7;
  const int row0 = wave * 8 + rr;
  const bf16* atile =
      reinterpret_cast<const bf16*>(uniform_ptr(static_cast<const bf16*>(P.A) + m0 * P.lda + (int64_t)kt0 * BK));
  const bf16* btile =
      reinterpret_cast<const bf16*>(uniform_ptr(static_cast<const bf16*>(P.W) + (int64_t)n0 * P.K + (int64_t)kt0 * BK));
  // per-lane byte offsets of the 8 one-KB blocks this wave fills per operand
  // and stage (rows past M load row M-1; never stored)
  uint32_t offa[8], offb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = row0 + i * 32;
    const int64_t m = (m0 + row < P.M) ? row : P.M - 1 - m0;
    offa[i] = (uint32_t)((m * P.lda + ((pp ^ swz8(row)) << 3)) * 2);
    offb[i] = (uint32_t)(((int64_t)row * P.K + ((pp ^ swz8(row)) << 3)) * 2);
  }
  const lds_char* lsm = (const lds_char*)(smem);
  const int l32 = lane & 31, g = lane >> 5;
  const int ra = wm * 128 + l32, rb = wn * 128 + l32;
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    aoff[kk] = ra * 128 + (((kk * 2 + g) ^ swz8(ra)) << 4);
    boff[kk] = 2 * BM * BK * 2 + rb * 128 + (((kk * 2 + g) ^ swz8(rb)) << 4);
  }
  bf16x8 fa[2][4], fb[2][4];
  const int KT = nkt < 0 ? P.K / BK : nkt;
  const rsrc_t rsa = make_rsrc(atile), rsb = make_rsrc(btile);
  auto issue = [&](int k) {
    const int s2 = k & 1;
    const uint32_t ks = (uint32_t)k * BK * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      buf_lds<16>(rsa, offa[i], ks, smem + s2 * BM * BK + (wave + i * 4) * 512);
      buf_lds<16>(rsb, offb[i], ks, smem + 2 * BM * BK + s2 * BM * BK + (wave + i * 4) * 512);
    }
  };
  // per-lane row of the L2 touches: A rows (wave 64 + lane), B rows likewise
  const int prow = wave * 64 + lane;
  const int64_t pm = (m0 + prow < P.M) ? prow : P.M - 1 - m0;
  const uint32_t pfa = (uint32_t)(pm * P.lda * 2), pfb = (uint32_t)((int64_t)prow * P.K * 2);
  // stages 0 and 1, then the touch of stage 2 (stage 3 on is touched by the
  // mainloop)
  issue(0);
  if (KT > 1) issue(1);
  if (KT > 2) {
    bf16* junk = smem + 2 * 2 * BM * BK + wave * 128;
    buf_lds<4>(rsa, pfa, 2 * BK * 2, junk);
    buf_lds<4>(rsb, pfb, 2 * BK * 2, junk);
    __builtin_amdgcn_s_waitcnt(0x4F72);   // vmcnt(18): stage 0 landed
  } else if (KT == 2) {
    __builtin_amdgcn_s_waitcnt(0x4F70);   // vmcnt(16)
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j)
    fb[0][j] = *reinterpret_cast<const lds_bf16x8*>(lsm + boff[(j & 1) ? 2 : 0] + j * 4096);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    fa[0][i] = *reinterpret_cast<const lds_bf16x8*>(lsm + aoff[(i & 1) ? 2 : 0] + i * 4096);
  int kt = 0;
  for (; kt + 2 < KT; ++kt)
    pipe_step<true, true>(rsa, rsb, offa, offb, kt, KT, pfa, pfb, smem, lsm, aoff, boff, fa, fb, acc);
  if (KT >= 2) {
    pipe_step<true, false>(rsa, rsb, offa, offb, kt, KT, pfa, pfb, smem, lsm, aoff, boff, fa, fb, acc);
    ++kt;
  }
  pipe_step<false, false>(rsa, rsb, offa, offb, kt, KT, pfa, pfb, smem, lsm, aoff, boff, fa, fb, acc);
  __syncthreads();
}

// Epilogue of one tile.  D[i][j] of a 32x32 MFMA tile: j = lane % 32,
// i = 8 * (v / 4) + 4 * (lane / 32) + v % 4.
template <int BM, int BN, int WM, int WN, int EPI>
__device__ __forceinline__ void store_tile(const GemmProb& P, int64_t m0, int n0,
                                           const f32x16 (&acc)[BM / WM / 32][BN / WN / 32], float* partial) {
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN, l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t m = m0 + wm * TM * 32 + i * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      if (m >= P.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * TN * 32 + j * 32 + l32;
        if (partial)
          partial[m * P.N + n] = acc[i][j][v];
        else
          epi_store<bf16, EPI>(P, m, n, acc[i][j][v]);
      }
    }
}

// Epilogue of the 4-wave 256x256 tile through LDS: each half of the tile
// (128 rows, float32, 128 KB) is written to LDS by the two waves that own it,
// then all 256 threads apply the epilogue to 8 consecutive columns at a time,
// so every global access (the output, and for the gated residual the x row
// and the gate vector) is a 16- or 32-byte vector access instead of a 2- or
// 4-byte one per element.  Same per-element arithmetic as epi_store.
//
// The QKV projection's epilogue (kEpiQkRope*) also normalises and rotates
// the q and k heads here (hyper.ai 2607.19064 方法 and blog close-reading
// 2.2(2): RoPE per sample with a frame axis for editing; 2.2(3): norm and
// RoPE chains fused): a tile's 256 columns lie in one of Q, K, V and hold
// 256 / D whole heads, and the 32 threads of a row take 8 consecutive
// columns each, so a head's sum of squares is a reduction over D / 8
// neighbouring lanes.  The arithmetic is the qk_norm_rope kernel's on the
// bf16-rounded products (same lane-to-dimension map, reduction tree, gain
// and rotation expressions), so the result has the same bits as the plain
// projection followed by that kernel.
template <int EPI>
__device__ __forceinline__ void store_tile_lds(const GemmProb& P, int64_t m0, int n0, const f32x16 (&acc)[4][4],
                                               bf16* smem, const QkDims& qk, int tid_in = -1) {
  float* T = reinterpret_cast<float*>(smem);   // [128][256]
  const int tid = tid_in >= 0 ? tid_in : (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, g = lane >> 5;
  // the problem's fields in registers once (the compiler would otherwise
  // reload them after every store, which it cannot prove does not alias them)
  void* const Yp = P.Y;
  void* const auxp = P.aux;
  const float* const gatep = P.gate;
  const int32_t* const segp = P.seg;
  const int64_t ldy = P.ldy, M = P.M, gs = P.gate_stride;
  const int N = P.N;
  const int ch = tid & 31, r0 = tid >> 5, n = n0 + ch * 8;
  // QK epilogue: per-thread gains, rotation-pair frequencies and axes
  constexpr bool QK = EPI == kEpiQkRope || EPI == kEpiQkRopeAux;
  bool rot_tile = false;
  int32_t Hq = 0, Dh = 0;
  float qk_eps = 0.f, gn[8];
  const float* csp = nullptr;   // this thread's 4 pairs of row 0 in the (cos, sin) table
  if constexpr (QK) {
    Dh = qk.D;
    Hq = qk.heads * Dh;
    qk_eps = qk.eps;
    rot_tile = n0 < 2 * Hq;
    const int dcol = (ch * 8) & (Dh - 1);
    if (P.rope_cs) csp = P.rope_cs + dcol;
    Vec8<float>::load((n0 < Hq ? P.g_q : P.g_k) + dcol, gn);
  }
  constexpr bool GATED = EPI == MMDIT_EPI_GATED_RES || EPI == kEpiGatedResAux;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int64_t mb = m0 + half * 128 + r0;
    const int nrow = (int)min<int64_t>(16, (M - mb + 7) >> 3);   // rows of this thread that exist (may be <= 0)
    lds_barrier();
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = i * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
            T[r * 256 + wn * 128 + j * 32 + l32] = acc[i][j][v];
          }
    }
    lds_barrier();
    // The row operands of the epilogue are read for all of the thread's rows
    // at once (one memory latency instead of one per few rows): the gated
    // residual's x rows and samples (the gate vector once when those rows
    // belong to one sample), the GELU backward's saved pre-activations, the
    // RoPE rows' (cos, sin) pairs.
    bf16x8 xr[GATED || EPI == kEpiGeluBwd ? 16 : 1];
    int32_t sg[GATED ? 16 : 1];
    f32x4 cq[QK ? 16 : 1][2];
    float g0[8];
    int32_t s0 = 0;
    if constexpr (GATED) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < nrow) {
          xr[i] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(Yp) + (mb + 8 * i) * ldy + n);
          sg[i] = segp[mb + 8 * i];
        }
      if (nrow > 0) {
        s0 = sg[0];
        Vec8<float>::load(gatep + (int64_t)s0 * gs + n, g0);
      }
    } else if constexpr (EPI == kEpiGeluBwd) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < nrow) xr[i] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(auxp) + (mb + 8 * i) * N + n);
    } else if constexpr (QK) {
      if (rot_tile && csp) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i < nrow) {
            cq[i][0] = *reinterpret_cast<const f32x4*>(csp + (mb + 8 * i) * Dh);
            cq[i][1] = *reinterpret_cast<const f32x4*>(csp + (mb + 8 * i) * Dh + 4);
          }
      }
    }
    // thread tid takes columns n..n+7 of rows r0, r0 + 8, ..., r0 + 120
    auto chunk = [&](int i) {
      const int64_t m = mb + 8 * i;
      const float* t = T + (r0 + 8 * i) * 256 + ch * 8;
      float a[8];
      *reinterpret_cast<f32x4*>(a) = *reinterpret_cast<const f32x4*>(t);
      *reinterpret_cast<f32x4*>(a + 4) = *reinterpret_cast<const f32x4*>(t + 4);
      if constexpr (EPI == MMDIT_EPI_STORE_F32) {
        float* y = static_cast<float*>(Yp) + m * ldy + n;
        *reinterpret_cast<f32x4*>(y) = *reinterpret_cast<const f32x4*>(a);
        *reinterpret_cast<f32x4*>(y + 4) = *reinterpret_cast<const f32x4*>(a + 4);
      } else if constexpr (QK) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = (float)(bf16)a[k];   // the stored product
        if (rot_tile) {
          if constexpr (EPI == kEpiQkRopeAux) Vec8<bf16>::store(static_cast<bf16*>(auxp) + m * 2 * Hq + n, v);
          const float ss = qk_head_sum(qk_sumsq8(v), Dh >> 3);
          const float r = qk_inv_rms(ss, (float)Dh, qk_eps);
          float cs[4], sn[4];
          if (csp) {
            const f32x4 c0 = cq[i][0], c1 = cq[i][1];
            cs[0] = c0[0], sn[0] = c0[1], cs[1] = c0[2], sn[1] = c0[3];
            cs[2] = c1[0], sn[2] = c1[1], cs[3] = c1[2], sn[3] = c1[3];
          }
          qk_apply8(v, r, gn, csp != nullptr, cs, sn);
        }
        Vec8<bf16>::store(static_cast<bf16*>(Yp) + m * ldy + n, v);
      } else {
        bf16* y = static_cast<bf16*>(Yp) + m * ldy + n;
        float o[8];
        if constexpr (EPI == MMDIT_EPI_STORE) {
#pragma unroll
          for (int k = 0; k < 8; ++k) o[k] = a[k];
        } else if constexpr (EPI == MMDIT_EPI_GELU || EPI == kEpiGeluAux) {
#pragma unroll
          for (int k = 0; k < 8; ++k) o[k] = gelu_f(a[k]);
          if constexpr (EPI == kEpiGeluAux) Vec8<bf16>::store(static_cast<bf16*>(auxp) + m * N + n, a);
        } else if constexpr (EPI == kEpiGeluBwd) {
          float xv[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) xv[k] = (float)xr[i][k];
#pragma unroll
          for (int k = 0; k < 8; ++k) o[k] = a[k] * gelu_grad_f(xv[k]);
        } else {
          float xv[8], gv[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) xv[k] = (float)xr[i][k];
          if (sg[i] == s0) {
#pragma unroll
            for (int k = 0; k < 8; ++k) gv[k] = g0[k];
          } else {
            Vec8<float>::load(gatep + (int64_t)sg[i] * gs + n, gv);
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) o[k] = xv[k] + gv[k] * a[k];
          if constexpr (EPI == kEpiGatedResAux) Vec8<bf16>::store(static_cast<bf16*>(auxp) + m * N + n, a);
        }
        Vec8<bf16>::store(y, o);
      }
    };
    if (nrow == 16) {   // all 16 rows of this thread exist
#pragma unroll GATED || QK || EPI == kEpiGeluBwd ? 16 : 4
      for (int i = 0; i < 16; ++i) chunk(i);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < nrow) chunk(i);
    }
  }
}

// Whole 256x256 tiles of a persistent launch: block hw runs the virtual
// block ids hw, hw + persist, ... below `full` (the same XCD as hw, persist
// being a multiple of 8), each a whole tile in the order of the
// one-block-per-tile grid, so every tile takes the same arithmetic as there.
// (Written out in each kernel: behind a shared function taking the launch's
// argument block by reference, the compiler copied that block to scratch.)
#define MMDIT_PERSIST_TILES(hw_, full_)                                           \
  do {                                                                          \
    const int phw = (hw_), pfull = (full_);                                         \
    for (int vid = phw; vid < pfull; vid += bt.persist) {                         \
      /* the previous tile's epilogue has read its last LDS staging */          \
      if (vid != phw) lds_barrier();                                             \
      int t = bt.xcd_remap ? xcd_tile(vid, pfull) : vid;                         \
      const GemmProb& P = pick(bt, t);                                          \
      int tm, tn;                                                               \
      grouped_tile(t, (int)cdiv_d(P.M, 256), P.tiles_n, tm, tn);                \
      f32x16 acc[4][4];                                                         \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                             \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                           \
          _Pragma("unroll") for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;    \
      /* the thread index through an opaque move each tile, so that the       \
         per-thread offsets are recomputed per tile instead of held live      \
         across the loop (hoisted, they spill) */                             \
      int tid = threadIdx.x;                                                    \
      asm volatile("" : "+v"(tid));                                             \
      mma_tile_pipe(P, (int64_t)tm * 256, tn * 256, smem, acc, 0, -1, tid);     \
      store_tile_lds<EPI>(P, (int64_t)tm * 256, tn * 256, acc, smem, bt.qk, tid); \
    }                                                                           \
  } while (0)

// SITE 1 only separates the MLP down projection's instantiation from the
// output projection's (same epilogue) so profiles can tell the two apart;
// SITE 2 is the image embedding with the noising in its A staging (XT).
// PERSIST: the launch's first bt.persist blocks walk the whole tiles
// (MMDIT_PERSIST_TILES), any blocks after them take the last-round sub-tiles;
// a separate instantiation, so the one-block-per-tile kernels keep their own
// register allocation.
template <int BM, int BN, int WM, int WN, int EPI, bool SILU, int SITE = 0, int BK = 64, int NS = 2,
          bool PERSIST = false>
__global__ void __launch_bounds__(WM * WN * 64) gemm_mfma_kernel(GemmBatch bt) {
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  extern __shared__ __attribute__((aligned(1024))) bf16 smem[];
  constexpr bool PIPE = BM == 256 && BN == 256 && WM == 2 && WN == 2 && !SILU && BK == 64 && NS == 2 && SITE != 2;
  int hw = blockIdx.x;
  if constexpr (PIPE && PERSIST) {
    // persistent blocks first, then the last-round sub-tile blocks
    if (hw < bt.persist) {
      MMDIT_PERSIST_TILES(hw, bt.tail_begin > 0 ? bt.tail_begin : bt.ntiles);
      return;
    }
    hw = hw - bt.persist + bt.tail_begin;
  }
  int tile, chunk = -1;
  if (bt.tail_begin > 0 && hw >= bt.tail_begin) {
    const int u = hw - bt.tail_begin;
    tile = bt.tail_begin + u / bt.tail_chunks;
    chunk = u % bt.tail_chunks;
  } else {
    const int full = bt.tail_begin > 0 ? bt.tail_begin : (int)gridDim.x;
    tile = bt.xcd_remap ? xcd_tile(hw, full) : hw;
  }
  const GemmProb& P = pick(bt, tile);
  int tm, tn;
  grouped_tile(tile, (int)cdiv_d(P.M, BM), P.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  if constexpr (BM == 256 && BN == 256 && WM == 2 && (WN == 4 || WN == 2)) {
    if (chunk >= 0) {
      // last-round fill by sub-tiles: each block takes a 256x128, 128x128 or
      // 64x128 part of the tile over the whole K (same per-element k order as
      // a full tile, so the result does not depend on which round a row is in).
      // The two smaller ones step 128 deep in k when K allows (half the
      // barriers, the same k order), otherwise a 4-stage ring of 64-deep
      // steps, in the same 128 KB of LDS.
      static_assert(NS * (BM + BN) * BK >= 4 * (128 + 128) * BK, "LDS of the sub-tile ring");
      constexpr int T2 = 128 / WN / 32;   // 128-wide sub-tiles: MFMA columns per wave
      const int KT = P.K / BK;
      if (bt.tail_chunks == 2) {
        f32x16 a2[4][T2];
        for (int i = 0; i < 4; ++i)
          for (int j = 0; j < T2; ++j)
            for (int v = 0; v < 16; ++v) a2[i][j][v] = 0.f;
        mma_tile<256, 128, WM, WN, SILU, BK, NS>(P, m0, n0 + chunk * 128, 0, KT, smem, a2);
        store_tile<256, 128, WM, WN, EPI>(P, m0, n0 + chunk * 128, a2, nullptr);
      } else if (bt.tail_chunks == 4) {
        const int64_t sm0 = m0 + (chunk >> 1) * 128;
        if (sm0 >= P.M) return;
        f32x16 a4[2][T2];
        for (int i = 0; i < 2; ++i)
          for (int j = 0; j < T2; ++j)
            for (int v = 0; v < 16; ++v) a4[i][j][v] = 0.f;
        if (P.K % 128 == 0)
          mma_tile<128, 128, WM, WN, SILU, 128, 2>(P, sm0, n0 + (chunk & 1) * 128, 0, P.K / 128, smem, a4);
        else
          mma_tile<128, 128, WM, WN, SILU, BK, 4>(P, sm0, n0 + (chunk & 1) * 128, 0, KT, smem, a4);
        store_tile<128, 128, WM, WN, EPI>(P, sm0, n0 + (chunk & 1) * 128, a4, nullptr);
      } else {
        const int64_t sm0 = m0 + (chunk >> 1) * 64;
        if (sm0 >= P.M) return;
        f32x16 a8[1][T2];
        for (int j = 0; j < T2; ++j)
          for (int v = 0; v < 16; ++v) a8[0][j][v] = 0.f;
        // 128-deep k steps (half the barriers) when K allows; same k order
        if (P.K % 128 == 0)
          mma_tile<64, 128, WM, WN, SILU, 128, 2>(P, sm0, n0 + (chunk & 1) * 128, 0, P.K / 128, smem, a8);
        else
          mma_tile<64, 128, WM, WN, SILU, BK, 4>(P, sm0, n0 + (chunk & 1) * 128, 0, KT, smem, a8);
        store_tile<64, 128, WM, WN, EPI>(P, sm0, n0 + (chunk & 1) * 128, a8, nullptr);
      }
      return;
    }
  }
  if constexpr (PIPE) {
    // whole K, explicitly pipelined 4-wave mainloop (no split-K on this shape)
    mma_tile_pipe(P, m0, n0, smem, acc);
    store_tile_lds<EPI>(P, m0, n0, acc, smem, bt.qk);
    return;
  }
  // this block's k steps (all of K unless split-K)
  const int KT = P.K / BK / bt.splitk;
  mma_tile<BM, BN, WM, WN, SILU, BK, NS, SITE == 2>(P, m0, n0, blockIdx.y * KT, KT, smem, acc);
  store_tile<BM, BN, WM, WN, EPI>(P, m0, n0, acc,
                                  bt.splitk > 1 ? bt.partial + (int64_t)blockIdx.y * P.M * P.N : nullptr);
}

// Split last round of the 256x256 pipelined tile.  When the tiles fill a
// few rounds of the CUs and leave the last one more than half full, the full
// rounds run as whole tiles (gemm_mfma_kernel over the first sk_full tiles)
// and each remaining tile is cut along k into sk_S equal parts of sk_P
// 64-deep steps, one block per part (gemm_sk_part_kernel): the last round
// then takes ceil(tail * S / CUs) part-times instead of a whole tile time.
// Parts are numbered part-major (part j of every remaining tile, then part
// j + 1) and handed to the XCDs in contiguous runs, so the blocks running
// together on an XCD read the same k range of neighbouring tiles and share
// their operand blocks in L2.  Each part writes its float32 partial tile
// (row-major [256][256], through the LDS epilogue); gemm_sk_fixup_kernel sums
// a tile's parts in k order and applies the epilogue.  The split depends on
// the launch's shape only, so results are bitwise reproducible; a row in a
// split tile rounds its k sum at the part boundaries, so its bits differ from
// the same row in a whole tile (within float32 rounding).
template <int SITE>
__global__ void __launch_bounds__(256) gemm_sk_part_kernel(GemmBatch bt) {
  extern __shared__ __attribute__((aligned(1024))) bf16 smem[];
  const int u = xcd_tile((int)blockIdx.x, (int)gridDim.x);
  const int t = u % bt.sk_tail, j = u / bt.sk_tail;
  const int KT = bt.p[0].K / 64;
  const int k0 = j * bt.sk_P;
  const int nk = min(bt.sk_P, KT - k0);
  int tile = bt.sk_full + t;
  const GemmProb& P = pick(bt, tile);
  int tm, tn;
  grouped_tile(tile, (int)cdiv_d(P.M, 256), P.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * 256;
  const int n0 = tn * 256;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;
  mma_tile_pipe(P, m0, n0, smem, acc, k0, nk);
  // the part's float32 tile, row-major [256][256]
  GemmProb Q;
  memset(&Q, 0, sizeof(Q));
  Q.Y = bt.sk_partial + ((int64_t)t * bt.sk_S + j) * 256 * 256;
  Q.ldy = 256;
  Q.M = 256;
  Q.N = 256;
  QkDims none = {0, 0, 0.f};
  store_tile_lds<MMDIT_EPI_STORE_F32>(Q, 0, 0, acc, smem, none);
}

// Sum of a split tile's parts in k order, then the gated-residual epilogue
// (x += gate[seg] * sum, and with Aux the sum kept in aux), 8 columns per
// thread with vector accesses.
template <int EPI>
__global__ void __launch_bounds__(256) gemm_sk_fixup_kernel(GemmBatch bt) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 8-column chunk of a split tile
  const int t = (int)(e >> 13);                                // 256 rows x 32 chunks per tile
  if (t >= bt.sk_tail) return;
  const int r = (int)((e >> 5) & 255), c = (int)(e & 31) * 8;
  int tile = bt.sk_full + t;
  const GemmProb& P = pick(bt, tile);
  int tm, tn;
  grouped_tile(tile, (int)cdiv_d(P.M, 256), P.tiles_n, tm, tn);
  const int64_t m = (int64_t)tm * 256 + r;
  if (m >= P.M) return;
  const int n = tn * 256 + c;
  // the residual row and its sample first, so their loads are in flight with the parts'
  bf16* y = static_cast<bf16*>(P.Y) + m * P.ldy + n;
  const bf16x8 xr = *reinterpret_cast<const bf16x8*>(y);
  const int32_t sgm = P.seg[m];
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* src = bt.sk_partial + (int64_t)t * bt.sk_S * 65536 + r * 256 + c;
#pragma unroll 4
  for (int j = 0; j < bt.sk_S; ++j) {
    float v[8];
    Vec8<float>::load(src + (int64_t)j * 65536, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] += v[k];
  }
  float xv[8], gv[8], o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) xv[k] = (float)xr[k];
  Vec8<float>::load(P.gate + (int64_t)sgm * P.gate_stride + n, gv);
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = xv[k] + gv[k] * a[k];
  if constexpr (EPI == kEpiGatedResAux) Vec8<bf16>::store(static_cast<bf16*>(P.aux) + m * P.N + n, a);
  Vec8<bf16>::store(y, o);
}

// Sums the split-K partials in a fixed order and applies the epilogue.
template <int EPI>
__global__ void splitk_reduce_kernel(GemmBatch bt) {
  const GemmProb& P = bt.p[0];
  const int64_t total = P.M * P.N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < bt.splitk; ++s) acc += bt.partial[s * total + i];
    epi_store<bf16, EPI>(P, i / P.N, (int)(i % P.N), acc);
  }
}

// Split-K reduction of a bf16 store whose rows are also the flow-matching
// velocity: 16 lanes per row, 8 columns per lane step, the partials summed in
// split order (as splitk_reduce_kernel), Y stored, and the row's squared
// residuals against z - eps summed in the same lane layout and order as the
// loss's own row-sum kernel (so the same bits).
__global__ void splitk_reduce_sse_kernel(GemmBatch bt) {
  const GemmProb& P = bt.p[0];
  const int64_t total = P.M * P.N;
  const int C = P.N;
  const int lane16 = threadIdx.x & 15;
  const int64_t row0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int64_t rstep = ((int64_t)gridDim.x * blockDim.x) >> 4;
  bf16* Y = static_cast<bf16*>(P.Y);
  for (int64_t row = row0; row < P.M; row += rstep) {
    float acc = 0.f;
    const int64_t src = bt.sse_row[row];
    for (int c8 = lane16; c8 < (C >> 3); c8 += 16) {
      float o[8], zv[8], ev[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a = 0.f;
        for (int sp = 0; sp < bt.splitk; ++sp) a += bt.partial[sp * total + row * C + c8 * 8 + i];
        o[i] = (float)(bf16)a;
      }
      Vec8<bf16>::store(Y + row * P.ldy + c8 * 8, o);
      Vec8<bf16>::load(bt.sse_z + src * C + c8 * 8, zv);
      Vec8<bf16>::load(bt.sse_e + src * C + c8 * 8, ev);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = rf_sq_acc(o[i], zv[i], ev[i], acc);
    }
    acc = group_sum(acc, 16);
    if (lane16 == 0) bt.row_sse[row] = acc;
  }
}

int persist_blocks(int whole_tiles);

template <int BM, int BN, int WM, int WN, int EPI, bool SILU, int SITE = 0, int BK = 64, int NS = 2>
mmdit_status launch_mfma_cfg(GemmBatch& bt, hipStream_t s) {
  int tiles = 0;
  for (int i = 0; i < bt.nprob; ++i) {
    bt.p[i].tiles_n = bt.p[i].N / BN;
    bt.p[i].tile_begin = tiles;
    tiles += (int)(cdiv(bt.p[i].M, BM) * bt.p[i].tiles_n);
  }
  if (tiles == 0) return MMDIT_OK;
  // the 4-wave pipelined 256x256 tile also keeps a 1 KB strip for its L2 touches
  constexpr bool pipe = BM == 256 && BN == 256 && WM == 2 && WN == 2 && !SILU && BK == 64 && NS == 2;
  const size_t lds = (size_t)NS * (BM + BN + (SITE == 2 ? BM : 0)) * BK * sizeof(bf16) + (pipe ? 1024 : 0);
  auto kern = gemm_mfma_kernel<BM, BN, WM, WN, EPI, SILU, SITE, BK, NS>;
  static bool attr_set = false;
  if (!attr_set) {
    MMDIT_TRY(hip_check(hipFuncSetAttribute((const void*)kern,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds),
                        "hipFuncSetAttribute(gemm_mfma_kernel)"));
    attr_set = true;
  }
  bool persistent = false;
  if constexpr (pipe && SITE != 2) {
    if (bt.splitk <= 1 && bt.tail_begin == 0) {
      bt.persist = persist_blocks(tiles);
      bt.ntiles = tiles;
      persistent = bt.persist > 0;
    }
  }
  if constexpr (pipe && SITE != 2) {
    if (persistent) {
      auto pk = gemm_mfma_kernel<BM, BN, WM, WN, EPI, SILU, SITE, BK, NS, true>;
      static bool pattr = false;
      if (!pattr) {
        MMDIT_TRY(hip_check(hipFuncSetAttribute((const void*)pk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds),
                            "hipFuncSetAttribute(gemm_mfma_kernel)"));
        pattr = true;
      }
      MMDIT_LAUNCH(pk, dim3(bt.persist), dim3(256), lds, s, bt);
    }
  }
  if (!persistent) MMDIT_LAUNCH(kern, dim3(tiles, bt.splitk), dim3(WM * WN * 64), lds, s, bt);
  static char name[80];
  if (!name[0])
    snprintf(name, sizeof(name), "gemm_mfma_kernel<%d,%d,%d,%d,epi%d%s%s,bk%d,s%d>", BM, BN, WM, WN, EPI,
             SILU ? ",silu" : "", SITE == 1 ? ",down" : SITE == 2 ? ",xt" : "", BK, NS);
  MMDIT_TRY(launch_check(bt.tag ? bt.tag : name, s));
  if (bt.splitk > 1) {
    if (EPI == MMDIT_EPI_STORE && bt.row_sse && bt.p[0].N % 8 == 0) {
      const int64_t nb = cdiv(bt.p[0].M * 16, 256);
      const int blocks = (int)(nb < 4096 ? nb : 4096);
      MMDIT_LAUNCH(splitk_reduce_sse_kernel, dim3(blocks), dim3(256), 0, s, bt);
      MMDIT_TRY(launch_check("splitk_reduce_sse_kernel", s));
      *bt.sse_done = 1;
      return MMDIT_OK;
    }
    const int64_t total = bt.p[0].M * bt.p[0].N;
    const int64_t nb = cdiv(total, 256);
    const int blocks = (int)(nb < 4096 ? nb : 4096);
    MMDIT_LAUNCH(splitk_reduce_kernel<EPI>, dim3(blocks), dim3(256), 0, s, bt);
    MMDIT_TRY(launch_check("splitk_reduce_kernel", s));
  }
  return MMDIT_OK;
}

int tile_override() {
  static int v = -2;
  if (v == -2) {
    const char* e = getenv("MMDIT_GEMM_TILE");
    v = e ? atoi(e) : -1;
  }
  return v;
}

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = -1;
  }
  return n;
}

// Persistent blocks for the whole tiles of the pipelined 256x256 shape: one
// block per CU (a multiple of 8, so each keeps its XCD) when the whole tiles
// fill at least two rounds; env MMDIT_GEMM_PERSIST=0 turns it off.
int persist_blocks(int whole_tiles) {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("MMDIT_GEMM_PERSIST");
    v = e ? atoi(e) : MMDIT_PERSIST_DEFAULT;
  }
  const int nb = cu_count() & ~7;
  if (v == 0 || nb <= 0 || whole_tiles < 2 * nb) return 0;
  return nb;
}

// The 256x256 tile: 4 = 4 waves with the pipelined mainloop (default; it
// measured ahead of or level with the 8-wave tile at every block shape),
// 3 = 8 waves with the plain ring (env MMDIT_GEMM_BIG=3).
int big_tile_cfg(int /*epi*/) {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("MMDIT_GEMM_BIG");
    v = (e && atoi(e) == 3) ? 3 : 4;
  }
  return v;
}

// env MMDIT_TAILSPLIT=0 turns the last-round sub-tiling off
bool tailsplit_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("MMDIT_TAILSPLIT");
    v = e ? atoi(e) : 1;
  }
  return v != 0;
}

// env MMDIT_STREAMK=0 turns the stream-K last round off
bool streamk_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("MMDIT_STREAMK");
    v = e ? atoi(e) : 1;
  }
  return v != 0;
}

// Split-last-round plan of a launch of 256x256 tiles over problems of M[i]
// rows, N columns and depth K: the whole rounds of the CUs, then the rest of
// the tiles cut along k into S parts.  Taken for long K (>= 64 k steps) when
// at least one round is full and the last one more than half (a last round
// at most half full takes the sub-tile split instead), with the S in 2..4
// that gives the fewest part-rounds per tile time, ceil(tail S / CUs) / S,
// if that saves at least a fifth of the last round.
struct SkPlan {
  int full, tail, S, P;
  size_t bytes;
};

bool sk_plan(const int64_t* M, int nprob, int N, int K, SkPlan& pl) {
  const int nb = cu_count();
  if (!streamk_enabled() || nb <= 0 || N % 256 || K % 64 || K / 64 < 64 || tile_override() >= 0 ||
      big_tile_cfg(0) != 4)
    return false;
  int64_t T = 0;
  for (int i = 0; i < nprob; ++i) T += cdiv(M[i], 256) * (N / 256);
  const int64_t full = (T / nb) * nb, tail = T - full;
  if (full < nb || tail * 2 <= nb) return false;
  int best = 1;
  double cost = 1.0;
  for (int S = 2; S <= 4; ++S) {
    const double c = (double)cdiv(tail * S, nb) / S;
    if (c < cost - 1e-9) {
      cost = c;
      best = S;
    }
  }
  if (best == 1 || cost > 0.8) return false;
  const int KT = K / 64;
  pl.full = (int)full;
  pl.tail = (int)tail;
  pl.S = best;
  pl.P = (int)cdiv(KT, best);
  pl.bytes = (size_t)tail * best * 256 * 256 * sizeof(float);
  return true;
}

template <int EPI, int SITE>
mmdit_status launch_sk(GemmBatch& bt, const SkPlan& pl, hipStream_t s) {
  int tiles = 0;
  for (int i = 0; i < bt.nprob; ++i) {
    bt.p[i].tiles_n = bt.p[i].N / 256;
    bt.p[i].tile_begin = tiles;
    tiles += (int)(cdiv(bt.p[i].M, 256) * bt.p[i].tiles_n);
  }
  bt.sk_full = pl.full;
  bt.sk_tail = pl.tail;
  bt.sk_S = pl.S;
  bt.sk_P = pl.P;
  bt.sk_partial = bt.partial;
  const size_t lds = 2 * (256 + 256) * 64 * sizeof(bf16) + 1024;
  auto whole = gemm_mfma_kernel<256, 256, 2, 2, EPI, false, SITE>;
  static bool attr_set = false;
  if (!attr_set) {
    MMDIT_TRY(hip_check(hipFuncSetAttribute((const void*)whole, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds),
                        "hipFuncSetAttribute(gemm_mfma_kernel)"));
    MMDIT_TRY(hip_check(hipFuncSetAttribute((const void*)gemm_sk_part_kernel<SITE>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds),
                        "hipFuncSetAttribute(gemm_sk_part_kernel)"));
    attr_set = true;
  }
  const bool down = bt.tag && strcmp(bt.tag, "mlp_down_gated") == 0;
  // whole tiles of the full rounds (the launch covers tiles 0 .. full-1)
  bt.persist = persist_blocks(pl.full);
  bt.ntiles = pl.full;
  if (bt.persist > 0) {
    auto pk = gemm_mfma_kernel<256, 256, 2, 2, EPI, false, SITE, 64, 2, true>;
    static bool pattr = false;
    if (!pattr) {
      MMDIT_TRY(hip_check(hipFuncSetAttribute((const void*)pk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds),
                          "hipFuncSetAttribute(gemm_mfma_kernel)"));
      pattr = true;
    }
    MMDIT_LAUNCH(pk, dim3(bt.persist), dim3(256), lds, s, bt);
  } else {
    MMDIT_LAUNCH(whole, dim3(pl.full), dim3(256), lds, s, bt);
  }
  bt.persist = 0;
  MMDIT_TRY(launch_check(bt.tag ? bt.tag : "gemm_mfma_kernel<256,256,2,2,sk>", s));
  MMDIT_LAUNCH(gemm_sk_part_kernel<SITE>, dim3(pl.tail * pl.S), dim3(256), lds, s, bt);
  MMDIT_TRY(launch_check(down ? "mlp_down_sk" : "gemm_sk_part_kernel", s));
  MMDIT_LAUNCH(gemm_sk_fixup_kernel<EPI>, dim3(pl.tail * 32), dim3(256), 0, s, bt);
  return launch_check(down ? "mlp_down_fixup" : "gemm_sk_fixup_kernel", s);
}

// Last-round fill: when the 256x256 tiles leave the last round of CUs at
// most half busy, each tile of that round is shared by S = 2, 4 or 8 blocks,
// each computing a sub-tile over the whole K.
template <int EPI, int SITE, int WN>
mmdit_status launch_tailsplit(GemmBatch& bt, int tiles, int nb, hipStream_t s) {
  const int rounds = tiles / nb;
  const int tail = tiles - rounds * nb;
  static int smax = -1;
  if (smax < 0) {
    const char* e = getenv("MMDIT_TAIL_MAXS");
    smax = e ? atoi(e) : 8;
  }
  int S = 1;
  for (int c = 2; c <= smax && c <= 8; c *= 2)
    if (tail * c <= nb) S = c;
  if (S == 1) S = 2;
  bt.tail_begin = rounds * nb;
  bt.tail_chunks = S;
  const size_t lds = 2 * (256 + 256) * 64 * sizeof(bf16) + (WN == 2 ? 1024 : 0);
  auto kern = gemm_mfma_kernel<256, 256, 2, WN, EPI, false, SITE>;
  auto kernp = gemm_mfma_kernel<256, 256, 2, WN, EPI, false, SITE, 64, 2, true>;
  static bool attr_set = false;
  if (!attr_set) {
    MMDIT_TRY(hip_check(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds),
                        "hipFuncSetAttribute(gemm_mfma_kernel)"));
    MMDIT_TRY(hip_check(hipFuncSetAttribute((const void*)kernp, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds),
                        "hipFuncSetAttribute(gemm_mfma_kernel)"));
    attr_set = true;
  }
  if (WN == 2) {
    bt.persist = persist_blocks(bt.tail_begin);
    bt.ntiles = tiles;
  }
  if (bt.persist > 0)
    MMDIT_LAUNCH(kernp, dim3(bt.persist + tail * S), dim3(2 * WN * 64), lds, s, bt);
  else
    MMDIT_LAUNCH(kern, dim3(bt.tail_begin + tail * S), dim3(2 * WN * 64), lds, s, bt);
  static char name[80];
  if (!name[0]) snprintf(name, sizeof(name), "gemm_mfma_kernel<256,256,2,%d,epi%d%s,tailsplit>", WN, EPI, SITE ? ",down" : "");
  return launch_check(bt.tag ? bt.tag : name, s);
}

// Worth it when the 256x256 tiles fill at least one round of CUs and the last
// round is at most half occupied.
bool want_tailsplit(int64_t t256, bool n256, int& nb) {
  nb = cu_count();
  if (!tailsplit_enabled() || !n256 || nb <= 0) return false;
  const int64_t tail = t256 % nb;
  return t256 >= nb && tail > 0 && tail * 2 <= nb;
}

// Tile configuration of an MFMA launch (a function of the shapes, the CU count
// and the MMDIT_GEMM_* overrides only): cfg as in launch_mfma's switch, and
// whether the last round is filled by sub-tiles (tail_ok: the epilogue allows it).
struct MfmaPlan {
  int cfg;
  bool tail;
  int nb;
};

MfmaPlan mfma_plan(const GemmBatch& bt, bool tail_ok) {
  bool n256 = true, n128 = true;
  int64_t t256 = 0;
  int kmax = 0;
  for (int i = 0; i < bt.nprob; ++i) {
    kmax = bt.p[i].K > kmax ? bt.p[i].K : kmax;
    n256 = n256 && (bt.p[i].N % 256 == 0);
    n128 = n128 && (bt.p[i].N % 128 == 0);
    t256 += cdiv(bt.p[i].M, 256) * (bt.p[i].N / 256);
  }
  int cfg = tile_override();
  bool thin = true;
  for (int i = 0; i < bt.nprob; ++i) thin = thin && bt.p[i].N <= 256 && bt.p[i].N % 128 == 0 && bt.p[i].K >= 1024;
  if (cfg < 0) {
    // measured on MI355X: a 128x128 tile (two per CU) runs at about 0.64 of
    // the 256x256 tile's time per round of the chip, so the big tile wins
    // unless the 128x128 grid needs clearly fewer rounds: from 1.5 rounds of
    // 256 CUs up (1.5-2 rounds: 2 big rounds against 4 small ones), for one
    // round at least 70% full, and for short K (where the epilogue dominates)
    // at any count.  From one round up to 1.5 the last-round split below
    // applies where the epilogue allows it.
    if (thin) cfg = 6;
    else if (!n128) cfg = 0;
    else if (n256 && (2 * t256 > 3 * cu_count() || kmax <= 256 ||
                      (t256 * 10 >= cu_count() * 7 && t256 <= cu_count())))
      cfg = big_tile_cfg(0);
    else cfg = 1;
  }
  MfmaPlan pl;
  pl.nb = 0;
  pl.tail = tail_ok && tile_override() < 0 && want_tailsplit(t256, n256, pl.nb);
  if ((cfg == 3 || cfg == 4) && !n256) cfg = 2;
  if (cfg >= 1 && !n128) cfg = 0;
  pl.cfg = cfg;
  return pl;
}

template <int EPI, bool SILU>
mmdit_status launch_mfma(GemmBatch& bt, hipStream_t s) {
  if constexpr (!SILU && (EPI == MMDIT_EPI_GATED_RES || EPI == kEpiGatedResAux)) {
    // the MLP down projection: stream-K last round where it pays and the
    // caller gave the partial-tile workspace
    bool same = true;
    int64_t M[2];
    for (int i = 0; i < bt.nprob; ++i) {
      M[i] = bt.p[i].M;
      same = same && bt.p[i].N == bt.p[0].N && bt.p[i].K == bt.p[0].K;
    }
    SkPlan sk;
    if (bt.site == 1 && same && bt.partial && sk_plan(M, bt.nprob, bt.p[0].N, bt.p[0].K, sk) &&
        (size_t)bt.partial_elems * sizeof(float) >= sk.bytes)
      return launch_sk<EPI, 1>(bt, sk, s);
  }
  const MfmaPlan pl = mfma_plan(bt, !SILU && EPI != MMDIT_EPI_STORE_F32);
  int cfg = pl.cfg;
  if constexpr (!SILU && EPI != MMDIT_EPI_STORE_F32) {
    if (pl.tail) {
      int tiles = 0;
      for (int i = 0; i < bt.nprob; ++i) {
        bt.p[i].tiles_n = bt.p[i].N / 256;
        bt.p[i].tile_begin = tiles;
        tiles += (int)(cdiv(bt.p[i].M, 256) * bt.p[i].tiles_n);
      }
      const bool w4 = big_tile_cfg(EPI) == 4;
      if (EPI == MMDIT_EPI_GATED_RES && bt.site == 1)
        return w4 ? launch_tailsplit<EPI, 1, 2>(bt, tiles, pl.nb, s) : launch_tailsplit<EPI, 1, 4>(bt, tiles, pl.nb, s);
      return w4 ? launch_tailsplit<EPI, 0, 2>(bt, tiles, pl.nb, s) : launch_tailsplit<EPI, 0, 4>(bt, tiles, pl.nb, s);
    }
  }
  if constexpr (EPI == MMDIT_EPI_GATED_RES && !SILU) {
    if (bt.site == 1) switch (cfg) {
      case 6: return launch_mfma_cfg<32, 128, 1, 4, EPI, SILU, 1>(bt, s);
      case 5: return launch_mfma_cfg<256, 128, 2, 2, EPI, SILU, 1>(bt, s);
      case 4: return launch_mfma_cfg<256, 256, 2, 2, EPI, SILU, 1>(bt, s);
      case 3: return launch_mfma_cfg<256, 256, 2, 4, EPI, SILU, 1>(bt, s);
      case 2: return launch_mfma_cfg<256, 128, 2, 4, EPI, SILU, 1>(bt, s);
      case 1: return launch_mfma_cfg<128, 128, 2, 2, EPI, SILU, 1>(bt, s);
      default: return launch_mfma_cfg<128, 64, 2, 2, EPI, SILU, 1>(bt, s);
    }
  }
  if (cfg == 6 && bt.partial && bt.nprob == 1) {
    // thin tiles alone cannot fill the chip: split K, partials summed in a
    // fixed order.  The split depends on K (and the partial buffer, sized per
    // row) only, never on M, so a row's result does not depend on how many
    // rows share the launch.
    const int KT = bt.p[0].K / 64;
    int sk = 1;
    for (int c = 2; c <= 8; ++c)
      if (KT % c == 0 && (int64_t)c * bt.p[0].M * bt.p[0].N <= bt.partial_elems) sk = c;
    bt.splitk = sk;
  }
  switch (cfg) {
    case 6: return launch_mfma_cfg<32, 128, 1, 4, EPI, SILU>(bt, s);
    case 5: return launch_mfma_cfg<256, 128, 2, 2, EPI, SILU>(bt, s);
    case 4: return launch_mfma_cfg<256, 256, 2, 2, EPI, SILU>(bt, s);
    case 3: return launch_mfma_cfg<256, 256, 2, 4, EPI, SILU>(bt, s);
    case 2: return launch_mfma_cfg<256, 128, 2, 4, EPI, SILU>(bt, s);
    case 1: return launch_mfma_cfg<128, 128, 2, 2, EPI, SILU>(bt, s);
    default: return launch_mfma_cfg<128, 64, 2, 2, EPI, SILU>(bt, s);
  }
}

template <int EPI, bool SILU>
mmdit_status launch_skinny(GemmBatch& bt, hipStream_t s) {
  int64_t ncols = 0;
  bool n64 = true;
  for (int i = 0; i < bt.nprob; ++i) {
    ncols += bt.p[i].N;
    n64 = n64 && bt.p[i].N % 64 == 0;
  }
  const int ng = (n64 && ncols >= 32768) ? 4 : 1;
  int tiles = 0;
  for (int i = 0; i < bt.nprob; ++i) {
    bt.p[i].tiles_n = bt.p[i].N / (16 * ng);
    bt.p[i].tile_begin = tiles;
    tiles += bt.p[i].tiles_n;
  }
  if (tiles == 0) return MMDIT_OK;
  if (ng == 4)
    MMDIT_LAUNCH((gemm_skinny_kernel<EPI, SILU, 4>), dim3(tiles), dim3(512), 0, s, bt);
  else
    MMDIT_LAUNCH((gemm_skinny_kernel<EPI, SILU, 1>), dim3(tiles), dim3(512), 0, s, bt);
  static char name[64];
  if (!name[0]) snprintf(name, sizeof(name), "gemm_skinny_kernel<epi%d%s>", EPI, SILU ? ",silu" : "");
  return launch_check(bt.tag ? bt.tag : name, s);
}

template <typename T, int EPI, bool SILU>
mmdit_status launch_simt(GemmBatch& bt, hipStream_t s) {
  int tiles = 0;
  for (int i = 0; i < bt.nprob; ++i) {
    bt.p[i].tiles_n = (int)cdiv(bt.p[i].N, 64);
    bt.p[i].tile_begin = tiles;
    tiles += (int)(cdiv(bt.p[i].M, 64) * bt.p[i].tiles_n);
  }
  if (tiles == 0) return MMDIT_OK;
  MMDIT_LAUNCH((gemm_simt_kernel<T, EPI, SILU>), dim3(tiles), dim3(256), 0, s, bt);
  return launch_check(bt.tag ? bt.tag : "gemm_simt_kernel", s);
}

enum class Path { SIMT, SKINNY, MFMA };

template <int EPI, bool SILU>
mmdit_status dispatch(mmdit_dtype dt, Path path, GemmBatch& bt, hipStream_t s) {
  if (dt == MMDIT_F32) return launch_simt<float, EPI, SILU>(bt, s);
  switch (path) {
    case Path::SKINNY: return launch_skinny<EPI, SILU>(bt, s);
    case Path::MFMA: return launch_mfma<EPI, SILU>(bt, s);
    default: return launch_simt<bf16, EPI, SILU>(bt, s);
  }
}

bool force_simt() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("MMDIT_GEMM");
    v = (e && strcmp(e, "simt") == 0) ? 1 : 0;
  }
  return v == 1;
}

// The QKV projection with QK-RMSNorm + RoPE: fused into the 256x256 tile's
// LDS epilogue when every tile of the launch takes it, otherwise the plain
// projection followed by the separate kernel (and, with Aux, a copy of the
// q, k columns before the norm); the two give the same bits.
mmdit_status linear_qk(mmdit_dtype dt, Path path, GemmBatch& bt, const LinearArgs* pa, int nprob, int epi,
                       hipStream_t s) {
  const QkEpilogue& q = *pa[0].qk;
  bt.qk.heads = q.heads;
  bt.qk.D = q.D;
  bt.qk.eps = q.eps;
  const int32_t H = q.heads * q.D;
  bool fuse = dt == MMDIT_BF16 && path == Path::MFMA && H % 256 == 0 && (q.D == 64 || q.D == 128);
  for (int i = 0; i < bt.nprob; ++i) fuse = fuse && bt.p[i].N == 3 * H && bt.p[i].ldy == 3 * H;
  if (fuse) {
    const MfmaPlan pl = mfma_plan(bt, true);
    fuse = !pl.tail && pl.cfg == 4;
  }
  if (fuse) {
    if (epi == kEpiQkRopeAux) return launch_mfma_cfg<256, 256, 2, 2, kEpiQkRopeAux, false>(bt, s);
    return launch_mfma_cfg<256, 256, 2, 2, kEpiQkRope, false>(bt, s);
  }
  MMDIT_TRY((dispatch<MMDIT_EPI_STORE, false>(dt, path, bt, s)));
  const size_t es = dt == MMDIT_BF16 ? 2 : 4;
  QkArgs qa[2];
  int k = 0;
  for (int i = 0; i < nprob; ++i) {
    const LinearArgs& a = pa[i];
    if (a.M == 0) continue;
    if (epi == kEpiQkRopeAux)
      MMDIT_TRY(hip_check(hipMemcpy2DAsync(a.aux, 2 * (size_t)H * es, a.Y, (size_t)a.ldy * es, 2 * (size_t)H * es,
                                           (size_t)a.M, hipMemcpyDeviceToDevice, s),
                          "hipMemcpy2DAsync"));
    qa[k].qkv = a.Y;
    qa[k].pos = a.pos;
    qa[k].g_q = a.g_q;
    qa[k].g_k = a.g_k;
    qa[k].n_rows = a.M;
    ++k;
  }
  return qk_norm_rope2_impl(dt, q.heads, q.D, q.widths, q.theta, q.eps, qa, k, s);
}

}  // namespace

size_t gemm_sk_partial_bytes(int64_t m0, int64_t m1, int32_t N, int32_t K) {
  const int64_t M[2] = {m0, m1};
  const int np = m1 > 0 ? 2 : 1;
  SkPlan pl;
  if (m0 <= 0 || !sk_plan(M, np, N, K, pl)) return 0;
  return pl.bytes;
}

mmdit_status linear(mmdit_dtype dt, const LinearArgs* pa, int nprob, hipStream_t s) {
  if (nprob < 1 || nprob > 2) {
    set_error("linear: nprob=%d", nprob);
    return MMDIT_E_INVALID;
  }
  GemmBatch bt;
  memset(&bt, 0, sizeof(bt));
  int n = 0;
  const int epi = pa[0].epilogue, silu = pa[0].a_silu;
  bool skinny = true, mfma = true;
  for (int i = 0; i < nprob; ++i) {
    const LinearArgs& a = pa[i];
    if (a.epilogue != epi || a.a_silu != silu) {
      set_error("linear: grouped problems must share the epilogue");
      return MMDIT_E_INVALID;
    }
    if (a.lda >= (1 << 22) || a.K >= (1 << 22)) {
      set_error("linear: lda=%lld K=%d: both must stay below 2^22 (32-bit tile offsets)", (long long)a.lda, a.K);
      return MMDIT_E_UNSUPPORTED;
    }
    if (a.M < 0 || a.N <= 0 || a.K <= 0 || a.lda < a.K || a.ldy < a.N) {
      set_error("linear: bad shape M=%lld N=%d K=%d lda=%lld ldy=%lld", (long long)a.M, a.N, a.K,
                (long long)a.lda, (long long)a.ldy);
      return MMDIT_E_INVALID;
    }
    if (a.M == 0) continue;
    const bool gated = epi == MMDIT_EPI_GATED_RES || epi == kEpiGatedResAux;
    const bool with_aux = epi == kEpiGeluAux || epi == kEpiGatedResAux || epi == kEpiGeluBwd || epi == kEpiQkRopeAux;
    const bool qk = epi == kEpiQkRope || epi == kEpiQkRopeAux;
    if (!a.A || !a.W || !a.Y || (gated && (!a.gate || !a.seg)) || (with_aux && !a.aux) ||
        (qk && (!a.qk || !a.g_q || !a.g_k || (a.pos != nullptr) != (a.rope_cs != nullptr)))) {
      set_error("linear: NULL pointer");
      return MMDIT_E_INVALID;
    }
    GemmProb& p = bt.p[n++];
    p.A = a.A;
    p.W = a.W;
    p.Y = a.Y;
    p.gate = a.gate;
    p.seg = a.seg;
    p.aux = a.aux;
    p.rope_cs = a.rope_cs;
    p.g_q = a.g_q;
    p.g_k = a.g_k;
    p.lda = a.lda;
    p.ldy = a.ldy;
    p.gate_stride = a.gate_stride;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    skinny = skinny && a.M <= 16 && a.K % 256 == 0 && a.N % 16 == 0 && a.lda % 8 == 0;
    mfma = mfma && a.K % 64 == 0 && a.N % 64 == 0 && a.lda % 8 == 0;
  }
  bt.nprob = n;
  bt.tag = pa[0].tag;
  bt.site = pa[0].site;
  bt.xcd_remap = (n < 2 || bt.p[0].K == bt.p[1].K) ? 1 : 0;
  bt.splitk = 1;
  bt.partial = pa[0].partial;
  bt.partial_elems = pa[0].partial_elems;
  bt.tail_begin = 0;
  bt.tail_chunks = 1;
  if (pa[0].row_sse && dt == MMDIT_BF16 && epi == MMDIT_EPI_STORE && nprob == 1) {
    if (!pa[0].sse_z || !pa[0].sse_e || !pa[0].sse_row || !pa[0].sse_done) {
      set_error("linear: NULL pointer (row sums)");
      return MMDIT_E_INVALID;
    }
    bt.sse_z = static_cast<const bf16*>(pa[0].sse_z);
    bt.sse_e = static_cast<const bf16*>(pa[0].sse_e);
    bt.sse_row = pa[0].sse_row;
    bt.row_sse = pa[0].row_sse;
    bt.sse_done = pa[0].sse_done;
  }

  if (n == 0) return MMDIT_OK;
  Path path = force_simt() ? Path::SIMT : skinny ? Path::SKINNY : mfma ? Path::MFMA : Path::SIMT;
  if (epi == kEpiQkRope || epi == kEpiQkRopeAux) {
    if (silu) {
      set_error("linear: the QK epilogue takes no SiLU on A");
      return MMDIT_E_INVALID;
    }
    return linear_qk(dt, path, bt, pa, nprob, epi, s);
  }
  switch (epi * 2 + (silu ? 1 : 0)) {
    case MMDIT_EPI_STORE * 2: return dispatch<MMDIT_EPI_STORE, false>(dt, path, bt, s);
    case MMDIT_EPI_STORE * 2 + 1: return dispatch<MMDIT_EPI_STORE, true>(dt, path, bt, s);
    case MMDIT_EPI_STORE_F32 * 2: return dispatch<MMDIT_EPI_STORE_F32, false>(dt, path, bt, s);
    case MMDIT_EPI_STORE_F32 * 2 + 1: return dispatch<MMDIT_EPI_STORE_F32, true>(dt, path, bt, s);
    case MMDIT_EPI_GELU * 2: return dispatch<MMDIT_EPI_GELU, false>(dt, path, bt, s);
    case MMDIT_EPI_GATED_RES * 2: return dispatch<MMDIT_EPI_GATED_RES, false>(dt, path, bt, s);
    case kEpiGeluAux * 2: return dispatch<kEpiGeluAux, false>(dt, path, bt, s);
    case kEpiGatedResAux * 2: return dispatch<kEpiGatedResAux, false>(dt, path, bt, s);
    case kEpiGeluBwd * 2: return dispatch<kEpiGeluBwd, false>(dt, path, bt, s);
    default:
      set_error("linear: unsupported epilogue %d (a_silu=%d)", epi, silu);
      return MMDIT_E_UNSUPPORTED;
  }
}

mmdit_status linear_xt(const LinearArgs& a, const XtArgs& x, hipStream_t s) {
  if (a.M < 0 || a.N <= 0 || a.K <= 0 || a.K % 64 || a.N % 128 || a.lda != a.K || a.ldy < a.N ||
      a.K >= (1 << 22) || a.epilogue != MMDIT_EPI_STORE || a.a_silu) {
    set_error("linear_xt: unsupported shape M=%lld N=%d K=%d", (long long)a.M, a.N, a.K);
    return MMDIT_E_UNSUPPORTED;
  }
  if (a.M == 0) return MMDIT_OK;
  if (!a.A || !a.W || !a.Y || !x.eps || !x.t || !x.seg || !x.pos) {
    set_error("linear_xt: NULL pointer");
    return MMDIT_E_INVALID;
  }
  GemmBatch bt;
  memset(&bt, 0, sizeof(bt));
  GemmProb& p = bt.p[0];
  p.A = a.A;
  p.W = a.W;
  p.Y = a.Y;
  p.xt_e = static_cast<const bf16*>(x.eps);
  p.xt_t = x.t;
  p.xt_seg = x.seg;
  p.xt_pos = x.pos;
  p.xt_zt = static_cast<bf16*>(x.zt);
  p.lda = a.lda;
  p.ldy = a.ldy;
  p.M = a.M;
  p.N = a.N;
  p.K = a.K;
  bt.nprob = 1;
  bt.tag = a.tag;
  bt.xcd_remap = 1;
  bt.splitk = 1;
  bt.tail_chunks = 1;
  return launch_mfma_cfg<128, 128, 2, 2, MMDIT_EPI_STORE, false, 2>(bt, s);
}

}  // namespace mmdit
