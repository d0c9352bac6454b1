// Block-diagonal varlen joint attention.
//
// Every sample of the pack attends over its own [text; image] tokens only
// (blog close-reading 2.2(2): a varlen attention kernel confines attention to
// each sample; 5 "MMDiT": text and image attend jointly).  Storage is
// modality-major, so joint position j of sample b is text row cu_txt[b] + j
// for j < T_b and image row cu_img[b] + j - T_b after it; q, k, v are read in
// place from the two [rows, 3H] QKV buffers (two-segment addressing) and the
// output goes to the two [rows, H] buffers.
//
// attn_mfma_kernel (bf16): 128 queries per block (4 waves x 32), 64-key tiles
// staged in LDS, online softmax in float32.  The score tile is computed
// transposed, S^T = K Q^T, so each lane owns one query: its row maximum and
// sum are lane-local (one cross-half exchange), and the probabilities feed
// O^T = V^T P^T straight from registers; V is transposed while it is staged.
// Software-pipelined by one tile: the softmax of tile i (vector ALU) runs
// while the scores of tile i + 1 issue on the matrix cores.
// attn_simt_kernel (float32, or any head_dim): 64 queries per block, four
// lanes per query, per-key online softmax.
#include "common.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <type_traits>

namespace mmdit {

namespace {

struct AttnArgs {
  const void* qkv_img;
  const void* qkv_txt;
  void* o_img;
  void* o_txt;
  const int32_t* cu_img;
  const int32_t* cu_txt;
  int32_t heads, H;
  float scale_log2;  // log2(e) / sqrt(head_dim)
  float* lse;        // optional [heads][njp] float32: log2 of each query's softmax denominator
  int32_t njp;       // padded joint length of the lse rows (samples start at multiples of 64)
  int32_t nq;        // query blocks (32 x waves each) per (sample, head) of the MFMA forward grid
  int32_t nB;        // samples
};

// The MFMA forward's 1-D grid is numbered so that each XCD (workgroups go to
// the 8 XCDs round-robin by id) takes a contiguous range of (query block,
// head, sample) items, query blocks fastest: the blocks sharing a head's K
// and V run on one XCD and share its L2.  False for the padding ids.
__device__ __forceinline__ bool attn_item(const AttnArgs& a, int& qb, int& head, int& b) {
  const int total = a.nq * a.heads * a.nB;
  const int per = (total + 7) / 8;
  const int id = blockIdx.x;
  const int item = (id & 7) * per + (id >> 3);
  if (item >= total) return false;
  qb = item % a.nq;
  head = (item / a.nq) % a.heads;
  b = item / (a.nq * a.heads);
  return true;
}

template <typename T>
__device__ __forceinline__ const T* joint_row(const AttnArgs& a, int32_t j, int32_t Tb, int32_t t0,
                                              int32_t i0) {
  const int64_t H3 = 3 * (int64_t)a.H;
  return j < Tb ? static_cast<const T*>(a.qkv_txt) + (int64_t)(t0 + j) * H3
                : static_cast<const T*>(a.qkv_img) + (int64_t)(i0 + j - Tb) * H3;
}
template <typename T>
__device__ __forceinline__ T* out_row(const AttnArgs& a, int32_t j, int32_t Tb, int32_t t0, int32_t i0) {
  return j < Tb ? static_cast<T*>(a.o_txt) + (int64_t)(t0 + j) * a.H
                : static_cast<T*>(a.o_img) + (int64_t)(i0 + j - Tb) * a.H;
}

// Start of sample b in the 64-padded joint axis of the V^T buffer.
__device__ __forceinline__ int32_t padded_start(const AttnArgs& a, int b) {
  const int lane = threadIdx.x & 63;
  int32_t acc = 0;
  for (int i = lane; i < b; i += 64) {
    const int32_t L = (a.cu_txt[i + 1] - a.cu_txt[i]) + (a.cu_img[i + 1] - a.cu_img[i]);
    acc += (L + 63) & ~63;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  return acc;
}

// ------------------------------------------------------------------- SIMT
template <typename T, int D>
__global__ void __launch_bounds__(256) attn_simt_kernel(AttnArgs a) {
  constexpr int DQ = D / 4;   // dims per lane
  constexpr int KB = 32;      // keys per LDS tile
  const int b = blockIdx.z, head = blockIdx.y;
  const int32_t t0 = a.cu_txt[b], i0 = a.cu_img[b];
  const int32_t Tb = a.cu_txt[b + 1] - t0;
  const int32_t L = Tb + a.cu_img[b + 1] - i0;
  const int32_t qbase = blockIdx.x * 64;
  if (qbase >= L) return;
  __shared__ float Ks[KB][D + 1], Vs[KB][D + 1];
  const int sub = threadIdx.x & 3;
  const int32_t j = qbase + (threadIdx.x >> 2);
  const bool valid = j < L;
  float q[DQ], acc[DQ];
  if (valid) {
    const T* r = joint_row<T>(a, j, Tb, t0, i0) + head * D + sub * DQ;
#pragma unroll
    for (int e = 0; e < DQ; ++e) q[e] = to_f(r[e]) * a.scale_log2;
  } else {
#pragma unroll
    for (int e = 0; e < DQ; ++e) q[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < DQ; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int32_t kv0 = 0; kv0 < L; kv0 += KB) {
    for (int idx = threadIdx.x; idx < KB * D; idx += 256) {
      const int r = idx / D, c = idx % D;
      const int32_t key = kv0 + r;
      float kv = 0.f, vv = 0.f;
      if (key < L) {
        const T* p = joint_row<T>(a, key, Tb, t0, i0);
        kv = to_f(p[a.H + head * D + c]);
        vv = to_f(p[2 * a.H + head * D + c]);
      }
      Ks[r][c] = kv;
      Vs[r][c] = vv;
    }
    __syncthreads();
    const int nk = min(KB, L - kv0);
    for (int kk = 0; kk < nk; ++kk) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) s = fmaf(q[e], Ks[kk][sub * DQ + e], s);
      s = group_sum(s, 4);
      const float mn = fmaxf(m, s);
      const float corr = exp2f(m - mn);
      const float p = exp2f(s - mn);
      l = l * corr + p;
#pragma unroll
      for (int e = 0; e < DQ; ++e) acc[e] = acc[e] * corr + p * Vs[kk][sub * DQ + e];
      m = mn;
    }
    __syncthreads();
  }
  if (valid) {
    T* o = out_row<T>(a, j, Tb, t0, i0) + head * D + sub * DQ;
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < DQ; ++e) o[e] = from_f<T>(acc[e] * inv);
  }
  if (a.lse) {
    const int32_t pstart = padded_start(a, b);
    if (valid && sub == 0) a.lse[(int64_t)head * a.njp + pstart + j] = m + log2f(l);
  }
}

// ------------------------------------------------------------------- MFMA

// V^T[head][d][padded joint token] (bf16) from the v columns of the QKV
// buffers; tokens past the end of a sample are written as zeros.
template <int D>
__global__ void __launch_bounds__(256) v_transpose_kernel(AttnArgs a, bf16* __restrict__ vt, int32_t njp) {
  __shared__ bf16 t[64][D + 2];
  const int b = blockIdx.z, head = blockIdx.y;
  const int32_t t0 = a.cu_txt[b], i0 = a.cu_img[b];
  const int32_t Tb = a.cu_txt[b + 1] - t0;
  const int32_t L = Tb + a.cu_img[b + 1] - i0;
  const int32_t kv0 = blockIdx.x * 64;
  if (kv0 >= L) return;
  const int32_t pstart = padded_start(a, b);
  constexpr int DCH = D / 8;
  for (int q = threadIdx.x; q < 64 * DCH; q += 256) {
    const int r = q / DCH, c = q % DCH;
    bf16x8 v = {};
    if (kv0 + r < L) v = *reinterpret_cast<const bf16x8*>(joint_row<bf16>(a, kv0 + r, Tb, t0, i0) + 2 * a.H + head * D + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) t[r][c * 8 + e] = v[e];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < D * 8; q += 256) {
    const int d = q >> 3, c = q & 7;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t[c * 8 + e][d];
    *reinterpret_cast<bf16x8*>(vt + ((int64_t)head * D + d) * njp + pstart + kv0 + c * 8) = v;
  }
}

// K rows are D bf16 = D/8 chunks of 16 B; chunk c of key row r sits at c ^ ksw(r).
template <int D>
__device__ __forceinline__ int ksw(int r) {
  if constexpr (D == 128) return r & 15;
  else return (r ^ (r >> 3)) & 7;
}
// V^T rows are 64 keys = 8 chunks of 16 B; chunk c of row d sits at c ^ vsw(d).
__device__ __forceinline__ int vsw(int d) { return (d >> 1) & 7; }

// S^T row i of a 32-key tile is loaded from key row perm(i), which swaps bits 2
// and 3: then the 8 probabilities a lane holds for each 16-key PV step are 8
// consecutive keys, so the matching V^T operand is one 16-byte LDS read.
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// max and sum of a lane's value with that of lane l ^ 32 (v_permlane32_swap:
// the two outputs hold, in every lane, its own value and the other half's)
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// NW waves of 32 queries per block.  Every query takes the same keys in the
// same tile order whatever NW is, so the output does not depend on it.  Eight
// waves share each K / V^T tile between twice the queries (half the tile
// traffic), which pays on long samples; four give twice the blocks on short
// ones.
template <int D, int NW>
__global__ void __launch_bounds__(64 * NW, 2) attn_mfma_kernel(AttnArgs a, const bf16* __restrict__ vt, int32_t njp) {
  constexpr int BKV = 64;
  constexpr int DT = D / 32;             // 32-wide d tiles of O^T
  constexpr int QS = D / 16;             // 16-deep k steps of S^T
  constexpr int KROWS = 512 / D;         // K rows per 1-KB block
  constexpr int KB = BKV / KROWS / NW;   // K blocks per wave per tile
  constexpr int VB = D / 8 / NW;         // V^T blocks (8 rows) per wave per tile
  static_assert(KB >= 1 && VB >= 1, "tile split");
  extern __shared__ __attribute__((aligned(1024))) bf16 smem[];

  int qb, head, b;
  if (!attn_item(a, qb, head, b)) return;
  const int32_t t0 = a.cu_txt[b], i0 = a.cu_img[b];
  const int32_t Tb = a.cu_txt[b + 1] - t0;
  const int32_t L = Tb + a.cu_img[b + 1] - i0;
  const int32_t qbase = qb * 32 * NW;
  if (qbase >= L) return;
  const int32_t pstart = padded_start(a, b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  const int32_t jq = qbase + wave * 32 + l32;
  bf16x8 qf[QS];
  if (jq < L) {
    const bf16* r = joint_row<bf16>(a, jq, Tb, t0, i0) + head * D + g * 8;
#pragma unroll
    for (int s = 0; s < QS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(r + s * 16);
  } else {
#pragma unroll
    for (int s = 0; s < QS; ++s) qf[s] = bf16x8{};
  }

  // per-lane sources of the 1-KB blocks this wave fills.  V^T: byte offsets
  // from the buffer's start (below 2^32: checked on the host), the tile's key
  // offset scalar.
  const int kr = lane / (D / 8), kp = lane % (D / 8);     // row in block, chunk position
  const rsrc_t rvt = make_rsrc(vt);
  uint32_t voff[VB];
#pragma unroll
  for (int i = 0; i < VB; ++i) {
    const int d = (wave + NW * i) * 8 + (lane >> 3);
    voff[i] = (uint32_t)((((int64_t)head * D + d) * njp + pstart + (((lane & 7) ^ vsw(d)) << 3)) * 2);
  }
  // K row of joint key j: text row t0 + j for j < Tb, image row i0 + j - Tb
  // after it; both bases are offset so that base + j * 3H addresses key j
  // (byte offsets fit 32 bits: checked on the host).  The chunk swizzle of
  // this lane's K rows does not depend on the tile.
  const uint32_t rowb = 3u * (uint32_t)a.H * 2u;
  const char* ktxt = reinterpret_cast<const char*>(static_cast<const bf16*>(a.qkv_txt) + (int64_t)t0 * 3 * a.H + a.H + head * D);
  const char* kimg = reinterpret_cast<const char*>(static_cast<const bf16*>(a.qkv_img) + ((int64_t)i0 - Tb) * 3 * a.H + a.H + head * D);
  const rsrc_t rtxt = make_rsrc(uniform_ptr(ktxt)), rimg = make_rsrc(uniform_ptr(kimg));
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  uint32_t kswc[KB], koff[KB];
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    kswc[i] = ((kp ^ ksw<D>((wave + NW * i) * KROWS + kr)) << 4);
    koff[i] = (uint32_t)((wu + NW * i) * KROWS + kr) * rowb + kswc[i];
  }
  // K tiles in two stages at smem + s BKV D, V^T tiles in two stages after
  // them.  A whole K tile inside the text or inside the image rows loads
  // through one segment's resource with the tile's offset scalar; a tile that
  // straddles the two or runs past L (keys past L load key L - 1 and are
  // masked in the scores) takes per-lane addresses.
  auto issue_k = [&](int32_t kv0, int st) {
    bf16* ks = smem + st * BKV * D;
    if (kv0 + BKV <= L && (kv0 + BKV <= Tb || kv0 >= Tb)) {
      const rsrc_t r = kv0 < Tb ? rtxt : rimg;
#pragma unroll
      for (int i = 0; i < KB; ++i) buf_lds16(r, koff[i], (uint32_t)kv0 * rowb, ks + (wu + NW * i) * 512);
    } else {
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const int blk = wu + NW * i;
        const int32_t key = min(kv0 + blk * KROWS + kr, L - 1);
        load_lds16((key < Tb ? ktxt : kimg) + ((uint32_t)key * rowb + kswc[i]), ks + blk * 512);
      }
    }
  };
  auto issue_v = [&](int32_t kv0, int st) {
    bf16* vs = smem + (2 + st) * BKV * D;
#pragma unroll
    for (int i = 0; i < VB; ++i) buf_lds16(rvt, voff[i], (uint32_t)kv0 * 2, vs + (wu + NW * i) * 512);
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[t][v] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  const int ntile = (L + BKV - 1) / BKV;
  const int prow = (l32 & 16) | kperm(l32 & 15);
  const int r0 = prow, r1 = 32 + prow;
  auto kfrag = [&](const bf16* ks, int r, int s) {
    return *reinterpret_cast<const bf16x8*>(ks + r * D + (((s * 2 + g) ^ ksw<D>(r)) << 3));
  };
  // S^T of the 64 keys in K stage kst, the two 32-key halves' k steps
  // interleaved (independent accumulators back to back), the K fragments read
  // two steps ahead
  auto scores = [&](int kst, f32x16 (&sc)[2]) {
    const bf16* ks = smem + kst * BKV * D;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[kt][v] = 0.f;
    bf16x8 kf[3][2];
    kf[0][0] = kfrag(ks, r0, 0);
    kf[0][1] = kfrag(ks, r1, 0);
    kf[1][0] = kfrag(ks, r0, 1);
    kf[1][1] = kfrag(ks, r1, 1);
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      if (s + 2 < QS) {
        kf[(s + 2) % 3][0] = kfrag(ks, r0, s + 2);
        kf[(s + 2) % 3][1] = kfrag(ks, r1, s + 2);
      }
      sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % 3][0], qf[s], sc[0], 0, 0, 0);
      sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % 3][1], qf[s], sc[1], 0, 0, 0);
    }
  };

  // One 64-key tile it, whose scores sc were computed by the previous step:
  // the loads of K tile it + 2 and V^T tile it + 1 issue first (their stages
  // were freed by the last barrier); then the softmax of tile it (vector ALU)
  // runs while the scores of tile it + 1 (NEXT) go into sn on the matrix
  // cores; then O^T += V^T P^T for tile it.  Register v of score tile kt holds
  // key kv0 + 32 kt + 16 (v / 8) + 8 g + v % 8.
  auto tile = [&](int it, f32x16 (&sc)[2], f32x16 (&sn)[2], auto next_c) {
    constexpr bool NEXT = decltype(next_c)::value;
    const int st = it & 1;
    const int32_t kv0 = it * BKV;
    if (NEXT) issue_v(kv0 + BKV, st ^ 1);
    if (it + 2 < ntile) issue_k(kv0 + 2 * BKV, st);
    if (kv0 + BKV > L) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int32_t key = kv0 + kt * 32 + 16 * (v >> 3) + 8 * g + (v & 7);
          if (key >= L) sc[kt][v] = -INFINITY;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) scores(st ^ 1, sn);
    // row maximum: four independent chains, then the other half's lanes (the
    // same query's other keys) through a lane-half swap
    float mq[4] = {sc[0][0], sc[0][1], sc[0][2], sc[0][3]};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = kt == 0 ? 4 : 0; v < 16; ++v) mq[v & 3] = fmaxf(mq[v & 3], sc[kt][v]);
    const float mx = half_swap_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3])));
    // softmax in the log2 domain: p = 2^(s * log2(e)/sqrt(d) - m).  The
    // reference m moves only when the tile's maximum exceeds it by more than
    // 8 (p <= 256 otherwise, exact in float32 and in the bf16 operand's
    // exponent range), so the rescale of O and the sum is rare after the
    // first tiles; m is the same for both lanes of a query.
    const float cand = mx * a.scale_log2;
    const float mn = cand > m + 8.0f ? cand : m;
    const float corr = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[kt][v] = __builtin_amdgcn_exp2f(fmaf(sc[kt][v], a.scale_log2, -mn));
    // P as the bf16 operand of the PV product, four 16-key steps; the row sum
    // takes the same bf16-rounded P, two at a time (v_dot2 against (1, 1)), so
    // the normaliser matches the weights
    bf16x8 pf[4];
    float ps = 0.f;
    const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
#pragma unroll
      for (int u = 0; u < 8; ++u) pf[ks2][u] = (bf16)sc[ks2 >> 1][8 * (ks2 & 1) + u];
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[ks2], pf[ks2], 0, 1), one2, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[ks2], pf[ks2], 2, 3), one2, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[ks2], pf[ks2], 4, 5), one2, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[ks2], pf[ks2], 6, 7), one2, ps, false);
    }
    if constexpr (NEXT) {
      // the scores' K reads and MFMAs with the softmax's vector work between them
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        if (s + 2 < QS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (__any(corr != 1.0f)) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[t][v] *= corr;
    }
    // O^T[d][query] += V^T[d][keys] P^T[keys][query]; step ks2 covers keys
    // 16 ks2 .. 16 ks2 + 15, this lane's 8 of them being 16 ks2 + 8 g + 0..7
    const bf16* vs = smem + (2 + st) * BKV * D;
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
      const int c = 2 * ks2 + g;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int d = t * 32 + l32;
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vs + d * BKV + ((c ^ vsw(d)) << 3));
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks2], oacc[t], 0, 0, 0);
      }
    }
    lsum = lsum * corr + ps;
    // V^T tile it + 1 and K tile it + 2 have landed for every wave
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // K tiles 0 and 1 and V^T tile 0, the scores of tile 0, then a barrier so
  // that K stage 0 may be refilled
  issue_k(0, 0);
  issue_v(0, 0);
  if (ntile > 1) issue_k(BKV, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x16 sa[2], sb[2];
  scores(0, sa);
  __syncthreads();
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  int it = 0;
  for (; it + 2 < ntile; it += 2) {
    tile(it, sa, sb, yes{});
    tile(it + 1, sb, sa, yes{});
  }
  if (ntile - it == 2) {
    tile(it, sa, sb, yes{});
    tile(it + 1, sb, sa, no{});
  } else {
    tile(it, sa, sb, no{});
  }
  lsum = half_swap_sum(lsum);
  if (a.lse && jq < L && g == 0) a.lse[(int64_t)head * a.njp + pstart + jq] = m + log2f(lsum);
  if (jq < L) {
    bf16* o = out_row<bf16>(a, jq, Tb, t0, i0) + head * D;
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        // rows d = 32t + 8vg + 4g + 0..3 of O^T hold this lane's query
        bf16x4 w = {(bf16)(oacc[t][4 * vg] * inv), (bf16)(oacc[t][4 * vg + 1] * inv),
                    (bf16)(oacc[t][4 * vg + 2] * inv), (bf16)(oacc[t][4 * vg + 3] * inv)};
        *reinterpret_cast<bf16x4*>(o + t * 32 + 8 * vg + 4 * g) = w;
      }
  }
}

// --------------------------------------------------------------- backward
// Gradients of o = softmax(q k^T / sqrt(d)) v, per sample and head, from the
// forward's log2 softmax denominators: with s2 = q.k log2(e)/sqrt(d) and
// P = 2^(s2 - lse),  D_i = dO_i . O_i,  dP = dO V^T,  dS = P (dP - D_i),
// dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dV = P^T dO.
// Deterministic: dQ is summed over keys by the query's own lanes and dK, dV
// over queries by the key's own lanes (no atomics).
struct AttnBwdArgs {
  AttnArgs f;           // q, k, v after QK-norm and RoPE; o; lse (input)
  const void* do_img;   // [rows, H] gradient of o
  const void* do_txt;
  void* dqkv_img;       // [rows, 3H] output: dq | dk | dv (head-contiguous, like qkv)
  void* dqkv_txt;
  float* dsum;          // [heads][njp] D_i
  float inv_sqrt_d;
};

template <typename T>
__device__ __forceinline__ const T* grad_row(const AttnBwdArgs& a, int32_t j, int32_t Tb, int32_t t0, int32_t i0) {
  return j < Tb ? static_cast<const T*>(a.do_txt) + (int64_t)(t0 + j) * a.f.H
                : static_cast<const T*>(a.do_img) + (int64_t)(i0 + j - Tb) * a.f.H;
}
template <typename T>
__device__ __forceinline__ T* dqkv_row(const AttnBwdArgs& a, int32_t j, int32_t Tb, int32_t t0, int32_t i0) {
  const int64_t H3 = 3 * (int64_t)a.f.H;
  return j < Tb ? static_cast<T*>(a.dqkv_txt) + (int64_t)(t0 + j) * H3
                : static_cast<T*>(a.dqkv_img) + (int64_t)(i0 + j - Tb) * H3;
}

// D_i = dO_i . O_i for every query (four lanes per query).
template <typename T, int D>
__global__ void __launch_bounds__(256) attn_bwd_dsum_kernel(AttnBwdArgs a) {
  constexpr int DQ = D / 4;
  const int b = blockIdx.z, head = blockIdx.y;
  const int32_t t0 = a.f.cu_txt[b], i0 = a.f.cu_img[b];
  const int32_t Tb = a.f.cu_txt[b + 1] - t0;
  const int32_t L = Tb + a.f.cu_img[b + 1] - i0;
  const int32_t qbase = blockIdx.x * 64;
  if (qbase >= L) return;
  const int32_t pstart = padded_start(a.f, b);
  const int sub = threadIdx.x & 3;
  const int32_t j = qbase + (threadIdx.x >> 2);
  float acc = 0.f;
  if (j < L) {
    const T* go = grad_row<T>(a, j, Tb, t0, i0) + head * D + sub * DQ;
    const T* o = out_row<T>(a.f, j, Tb, t0, i0) + head * D + sub * DQ;
#pragma unroll
    for (int e = 0; e < DQ; ++e) acc = fmaf(to_f(go[e]), to_f(o[e]), acc);
  }
  acc = group_sum(acc, 4);
  if (j < L && sub == 0) a.dsum[(int64_t)head * a.f.njp + pstart + j] = acc;
}

// dQ: 64 queries per block, four lanes per query, keys streamed through LDS.
template <typename T, int D>
__global__ void __launch_bounds__(256) attn_bwd_dq_simt_kernel(AttnBwdArgs a) {
  constexpr int DQ = D / 4;
  constexpr int KB = 32;
  const int b = blockIdx.z, head = blockIdx.y;
  const int32_t t0 = a.f.cu_txt[b], i0 = a.f.cu_img[b];
  const int32_t Tb = a.f.cu_txt[b + 1] - t0;
  const int32_t L = Tb + a.f.cu_img[b + 1] - i0;
  const int32_t qbase = blockIdx.x * 64;
  if (qbase >= L) return;
  const int32_t pstart = padded_start(a.f, b);
  __shared__ float Ks[KB][D + 1], Vs[KB][D + 1];
  const int sub = threadIdx.x & 3;
  const int32_t j = qbase + (threadIdx.x >> 2);
  const bool valid = j < L;
  float q[DQ], go[DQ], dq[DQ];
  float lse = 0.f, dsum = 0.f;
  if (valid) {
    const T* r = joint_row<T>(a.f, j, Tb, t0, i0) + head * D + sub * DQ;
    const T* g = grad_row<T>(a, j, Tb, t0, i0) + head * D + sub * DQ;
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
      q[e] = to_f(r[e]) * a.f.scale_log2;
      go[e] = to_f(g[e]);
    }
    lse = a.f.lse[(int64_t)head * a.f.njp + pstart + j];
    dsum = a.dsum[(int64_t)head * a.f.njp + pstart + j];
  } else {
#pragma unroll
    for (int e = 0; e < DQ; ++e) q[e] = go[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < DQ; ++e) dq[e] = 0.f;
  for (int32_t kv0 = 0; kv0 < L; kv0 += KB) {
    for (int idx = threadIdx.x; idx < KB * D; idx += 256) {
      const int r = idx / D, c = idx % D;
      const int32_t key = kv0 + r;
      float kv = 0.f, vv = 0.f;
      if (key < L) {
        const T* p = joint_row<T>(a.f, key, Tb, t0, i0);
        kv = to_f(p[a.f.H + head * D + c]);
        vv = to_f(p[2 * a.f.H + head * D + c]);
      }
      Ks[r][c] = kv;
      Vs[r][c] = vv;
    }
    __syncthreads();
    const int nk = min(KB, L - kv0);
    for (int kk = 0; kk < nk; ++kk) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        s = fmaf(q[e], Ks[kk][sub * DQ + e], s);
        dp = fmaf(go[e], Vs[kk][sub * DQ + e], dp);
      }
      s = group_sum(s, 4);
      dp = group_sum(dp, 4);
      const float ds = exp2f(s - lse) * (dp - dsum);
#pragma unroll
      for (int e = 0; e < DQ; ++e) dq[e] = fmaf(ds, Ks[kk][sub * DQ + e], dq[e]);
    }
    __syncthreads();
  }
  if (valid) {
    T* o = dqkv_row<T>(a, j, Tb, t0, i0) + head * D + sub * DQ;
#pragma unroll
    for (int e = 0; e < DQ; ++e) o[e] = from_f<T>(dq[e] * a.inv_sqrt_d);
  }
}

// dK and dV: 64 keys per block, four lanes per key, queries streamed through LDS.
template <typename T, int D>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_simt_kernel(AttnBwdArgs a) {
  constexpr int DQ = D / 4;
  constexpr int QB = 32;
  const int b = blockIdx.z, head = blockIdx.y;
  const int32_t t0 = a.f.cu_txt[b], i0 = a.f.cu_img[b];
  const int32_t Tb = a.f.cu_txt[b + 1] - t0;
  const int32_t L = Tb + a.f.cu_img[b + 1] - i0;
  const int32_t kbase = blockIdx.x * 64;
  if (kbase >= L) return;
  const int32_t pstart = padded_start(a.f, b);
  __shared__ float Qs[QB][D + 1], Gs[QB][D + 1], Ls[QB], Ds[QB];
  const int sub = threadIdx.x & 3;
  const int32_t j = kbase + (threadIdx.x >> 2);
  const bool valid = j < L;
  float k[DQ], v[DQ], dk[DQ], dv[DQ];
  if (valid) {
    const T* r = joint_row<T>(a.f, j, Tb, t0, i0) + head * D + sub * DQ;
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
      k[e] = to_f(r[a.f.H + e]);
      v[e] = to_f(r[2 * a.f.H + e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < DQ; ++e) k[e] = v[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < DQ; ++e) dk[e] = dv[e] = 0.f;
  for (int32_t q0 = 0; q0 < L; q0 += QB) {
    for (int idx = threadIdx.x; idx < QB * D; idx += 256) {
      const int r = idx / D, c = idx % D;
      const int32_t qi = q0 + r;
      float qv = 0.f, gv = 0.f;
      if (qi < L) {
        qv = to_f(joint_row<T>(a.f, qi, Tb, t0, i0)[head * D + c]);
        gv = to_f(grad_row<T>(a, qi, Tb, t0, i0)[head * D + c]);
      }
      Qs[r][c] = qv;
      Gs[r][c] = gv;
    }
    if (threadIdx.x < QB) {
      const int32_t qi = q0 + threadIdx.x;
      Ls[threadIdx.x] = qi < L ? a.f.lse[(int64_t)head * a.f.njp + pstart + qi] : 0.f;
      Ds[threadIdx.x] = qi < L ? a.dsum[(int64_t)head * a.f.njp + pstart + qi] : 0.f;
    }
    __syncthreads();
    const int nq = min(QB, L - q0);
    for (int qq = 0; qq < nq; ++qq) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        s = fmaf(Qs[qq][sub * DQ + e], k[e], s);
        dp = fmaf(Gs[qq][sub * DQ + e], v[e], dp);
      }
      s = group_sum(s, 4);
      dp = group_sum(dp, 4);
      const float p = exp2f(s * a.f.scale_log2 - Ls[qq]);
      const float ds = p * (dp - Ds[qq]);
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        dv[e] = fmaf(p, Gs[qq][sub * DQ + e], dv[e]);
        dk[e] = fmaf(ds, Qs[qq][sub * DQ + e], dk[e]);
      }
    }
    __syncthreads();
  }
  if (valid) {
    T* o = dqkv_row<T>(a, j, Tb, t0, i0) + head * D + sub * DQ;
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
      o[a.f.H + e] = from_f<T>(dk[e] * a.inv_sqrt_d);
      o[2 * a.f.H + e] = from_f<T>(dv[e]);
    }
  }
}

// ------------------------------------------------------ backward (MFMA)
// bf16 path.  A pre-pass writes D_i and the transposes Q^T, K^T, dO^T
// ([head][d][padded joint token], zeros past a sample's end); then
//   attn_bwd_dq_kernel   the forward's shape: 4 waves x 32 queries, q and dO
//                        in registers, 32-key tiles of K, V, K^T staged in LDS;
//                        S^T = K Q^T and dP^T = V dO^T per tile, then
//                        dQ^T += K^T dS^T with dS^T straight from registers
//   attn_bwd_dkdv_kernel the transpose roles: 4 waves x 32 keys, k (and v) in
//                        registers, 32-query tiles in LDS; S = Q K^T, then
//                        either dV^T += dO^T P (tiles Q, dO^T, lse) or, with
//                        dP = dO V^T, dK^T += Q^T dS (tiles Q, dO, Q^T, lse, D).
//                        Two launches: S is computed twice, but each kernel
//                        fits two waves per SIMD without spilling.
// The rows of the 32-row A operands are read in the order kperm (bits 2 and 3
// swapped) so that each lane's 8 values of a 16-deep k-step are 8 consecutive
// tokens and the matching transposed operand is one 16-byte LDS read.

// 64-byte rows (32 tokens): chunk c of row d sits at c ^ tsw(d).
__device__ __forceinline__ int tsw(int d) { return (d >> 1) & 3; }

template <int D>
__global__ void __launch_bounds__(256) attn_bwd_prep_kernel(AttnBwdArgs a, bf16* __restrict__ qt, bf16* __restrict__ kt,
                                                            bf16* __restrict__ gt) {
  __shared__ bf16 t[64][D + 2];
  const int b = blockIdx.z, head = blockIdx.y;
  const int32_t t0 = a.f.cu_txt[b], i0 = a.f.cu_img[b];
  const int32_t Tb = a.f.cu_txt[b + 1] - t0;
  const int32_t L = Tb + a.f.cu_img[b + 1] - i0;
  const int32_t kv0 = blockIdx.x * 64;
  if (kv0 >= L) return;
  const int32_t pstart = padded_start(a.f, b);
  constexpr int DCH = D / 8;
  // D_i = dO_i . O_i, four lanes per token
  {
    const int sub = threadIdx.x & 3, r = threadIdx.x >> 2;
    const int32_t j = kv0 + r;
    float acc = 0.f;
    if (j < L) {
      const bf16* go = grad_row<bf16>(a, j, Tb, t0, i0) + head * D + sub * (D / 4);
      const bf16* o = out_row<bf16>(a.f, j, Tb, t0, i0) + head * D + sub * (D / 4);
#pragma unroll
      for (int e = 0; e < D / 4; ++e) acc = fmaf((float)go[e], (float)o[e], acc);
    }
    acc = group_sum(acc, 4);
    if (sub == 0) a.dsum[(int64_t)head * a.f.njp + pstart + j] = j < L ? acc : 0.f;
  }
  for (int which = 0; which < 3; ++which) {
    __syncthreads();
    for (int q = threadIdx.x; q < 64 * DCH; q += 256) {
      const int r = q / DCH, c = q % DCH;
      bf16x8 v = {};
      const int32_t j = kv0 + r;
      if (j < L) {
        const bf16* src = which == 2 ? grad_row<bf16>(a, j, Tb, t0, i0) + head * D
                                     : joint_row<bf16>(a.f, j, Tb, t0, i0) + which * a.f.H + head * D;
        v = *reinterpret_cast<const bf16x8*>(src + c * 8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) t[r][c * 8 + e] = v[e];
    }
    __syncthreads();
    bf16* dst = which == 0 ? qt : which == 1 ? kt : gt;
    for (int q = threadIdx.x; q < D * 8; q += 256) {
      const int d = q >> 3, c = q & 7;
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = t[c * 8 + e][d];
      *reinterpret_cast<bf16x8*>(dst + ((int64_t)head * D + d) * a.f.njp + pstart + kv0 + c * 8) = v;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(256, 2) attn_bwd_dq_kernel(AttnBwdArgs a, const bf16* __restrict__ kt) {
  constexpr int BK = 32;                 // keys per stage
  constexpr int DT = D / 32, QS = D / 16;
  constexpr int KROWS = 512 / D;         // rows of a row-major tile per 1-KB block
  constexpr int RB = D / 64;             // 1-KB blocks per wave per tile
  constexpr int TILE = BK * D;
  constexpr int STAGE = 3 * TILE;        // K, V, K^T
  extern __shared__ __attribute__((aligned(1024))) bf16 smem[];

  const int b = blockIdx.z, head = blockIdx.y;
  const int32_t t0 = a.f.cu_txt[b], i0 = a.f.cu_img[b];
  const int32_t Tb = a.f.cu_txt[b + 1] - t0;
  const int32_t L = Tb + a.f.cu_img[b + 1] - i0;
  const int32_t qbase = blockIdx.x * 128;
  if (qbase >= L) return;
  const int32_t pstart = padded_start(a.f, b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int32_t jq = qbase + wave * 32 + l32;
  bf16x8 qf[QS], gf[QS];
  float lse = 0.f, dsum = 0.f;
  if (jq < L) {
    const bf16* r = joint_row<bf16>(a.f, jq, Tb, t0, i0) + head * D + g * 8;
    const bf16* gr = grad_row<bf16>(a, jq, Tb, t0, i0) + head * D + g * 8;
#pragma unroll
    for (int s2 = 0; s2 < QS; ++s2) {
      qf[s2] = *reinterpret_cast<const bf16x8*>(r + s2 * 16);
      gf[s2] = *reinterpret_cast<const bf16x8*>(gr + s2 * 16);
    }
    lse = a.f.lse[(int64_t)head * a.f.njp + pstart + jq];
    dsum = a.dsum[(int64_t)head * a.f.njp + pstart + jq];
  } else {
#pragma unroll
    for (int s2 = 0; s2 < QS; ++s2) qf[s2] = gf[s2] = bf16x8{};
  }

  const int kr = lane / (D / 8), kp = lane % (D / 8);
  const uint32_t rowb = 3u * (uint32_t)a.f.H * 2u;
  const char* ktxt = reinterpret_cast<const char*>(static_cast<const bf16*>(a.f.qkv_txt) + (int64_t)t0 * 3 * a.f.H + a.f.H + head * D);
  const char* kimg = reinterpret_cast<const char*>(static_cast<const bf16*>(a.f.qkv_img) + ((int64_t)i0 - Tb) * 3 * a.f.H + a.f.H + head * D);
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  // whole tiles inside the text or the image rows load through one segment's
  // buffer resource (the tile offset scalar, 32-bit lane offsets; the K^T
  // buffer likewise, below 2^32 bytes: checked on the host); a straddling or
  // ragged tile takes per-lane addresses
  const rsrc_t rtxt = make_rsrc(uniform_ptr(ktxt)), rimg = make_rsrc(uniform_ptr(kimg)), rkt = make_rsrc(kt);
  uint32_t kswc[RB], koff[RB], toff[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    kswc[i] = ((kp ^ ksw<D>((wave + 4 * i) * KROWS + kr)) << 4);
    koff[i] = (uint32_t)((wu + 4 * i) * KROWS + kr) * rowb + kswc[i];
    const int d = (wave + 4 * i) * 16 + (lane >> 2);
    toff[i] = (uint32_t)((((int64_t)head * D + d) * a.f.njp + pstart + (((lane & 3) ^ tsw(d)) << 3)) * 2);
  }
  auto issue = [&](int32_t kv0, int st) {
    bf16* ks = smem + st * STAGE;
    bf16* vs = ks + TILE;
    bf16* ts = vs + TILE;
    if (kv0 + BK <= L && (kv0 + BK <= Tb || kv0 >= Tb)) {
      const rsrc_t r = kv0 < Tb ? rtxt : rimg;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int blk = wu + 4 * i;
        buf_lds16(r, koff[i], (uint32_t)kv0 * rowb, ks + blk * 512);
        buf_lds16(r, koff[i] + (uint32_t)a.f.H * 2u, (uint32_t)kv0 * rowb, vs + blk * 512);
        buf_lds16(rkt, toff[i], (uint32_t)kv0 * 2, ts + blk * 512);
      }
    } else {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int blk = wu + 4 * i;
        const int32_t key = min(kv0 + blk * KROWS + kr, L - 1);   // keys past L are masked
        const char* kb = (key < Tb ? ktxt : kimg) + ((uint32_t)key * rowb + kswc[i]);
        load_lds16(kb, ks + blk * 512);
        load_lds16(kb + a.f.H * 2, vs + blk * 512);
        buf_lds16(rkt, toff[i], (uint32_t)kv0 * 2, ts + blk * 512);
      }
    }
  };

  f32x16 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) dq[t][v] = 0.f;
  const int ntile = (L + BK - 1) / BK;
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int prow = (l32 & 16) | kperm(l32 & 15);
  for (int it = 0; it < ntile; ++it) {
    const int st = it & 1;
    const int32_t kv0 = it * BK;
    if (it + 1 < ntile) issue(kv0 + BK, st ^ 1);
    const bf16* ks = smem + st * STAGE;
    const bf16* vs = ks + TILE;
    const bf16* ts = vs + TILE;
    f32x16 sc, dp;
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] = dp[v] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < QS; ++s2) {
      const int off = prow * D + (((s2 * 2 + g) ^ ksw<D>(prow)) << 3);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(ks + off), qf[s2], sc, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(vs + off), gf[s2], dp, 0, 0, 0);
    }
    // register v holds key kv0 + 16 (v / 8) + 8 g + v % 8 of this lane's query
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int32_t key = kv0 + 16 * (v >> 3) + 8 * g + (v & 7);
      const float p = key < L ? __builtin_amdgcn_exp2f(fmaf(sc[v], a.f.scale_log2, -lse)) : 0.f;
      sc[v] = p * (dp[v] - dsum);
    }
    // dQ^T[d][query] += K^T[d][keys] dS^T[keys][query]
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      bf16x8 pf;
#pragma unroll
      for (int u = 0; u < 8; ++u) pf[u] = (bf16)sc[8 * ks2 + u];
      const int c = 2 * ks2 + g;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int d = t * 32 + l32;
        const bf16x8 kv = *reinterpret_cast<const bf16x8*>(ts + d * BK + ((c ^ tsw(d)) << 3));
        dq[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, pf, dq[t], 0, 0, 0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  if (jq < L) {
    bf16* o = dqkv_row<bf16>(a, jq, Tb, t0, i0) + head * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        bf16x4 w = {(bf16)(dq[t][4 * vg] * a.inv_sqrt_d), (bf16)(dq[t][4 * vg + 1] * a.inv_sqrt_d),
                    (bf16)(dq[t][4 * vg + 2] * a.inv_sqrt_d), (bf16)(dq[t][4 * vg + 3] * a.inv_sqrt_d)};
        *reinterpret_cast<bf16x4*>(o + t * 32 + 8 * vg + 4 * g) = w;
      }
  }
}

template <int D, bool DK, int KS>
__global__ void __launch_bounds__(256, 2) attn_bwd_dkdv_kernel(AttnBwdArgs a, const bf16* __restrict__ qt,
                                                               const bf16* __restrict__ gt) {
  constexpr int BQ = 32;                 // queries per stage
  constexpr int DT = D / 32, QS = D / 16;
  constexpr int KROWS = 512 / D;
  constexpr int RB = D / 64;
  constexpr int TILE = BQ * D;
  // Q, then dO and Q^T (dK) or dO^T (dV), then lse and D (float)
  constexpr int NT = DK ? 3 : 2;
  constexpr int STAGE = NT * TILE + 2 * BQ * 2;
  extern __shared__ __attribute__((aligned(1024))) bf16 smem[];

  const int b = blockIdx.z, head = blockIdx.y;
  const int32_t t0 = a.f.cu_txt[b], i0 = a.f.cu_img[b];
  const int32_t Tb = a.f.cu_txt[b + 1] - t0;
  const int32_t L = Tb + a.f.cu_img[b + 1] - i0;
  const int32_t kbase = blockIdx.x * 128 * KS;
  if (kbase >= L) return;
  const int32_t pstart = padded_start(a.f, b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  // this wave's KS x 32 keys: key subtile ks holds keys kbase + (wave * KS + ks) * 32 + 0..31
  int32_t jk[KS];
  bf16x8 kf[KS][QS], vf[KS][DK ? QS : 1];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    jk[ks] = kbase + (wave * KS + ks) * 32 + l32;
    if (jk[ks] < L) {
      const bf16* r = joint_row<bf16>(a.f, jk[ks], Tb, t0, i0) + head * D + g * 8;
#pragma unroll
      for (int s2 = 0; s2 < QS; ++s2) {
        kf[ks][s2] = *reinterpret_cast<const bf16x8*>(r + a.f.H + s2 * 16);
        if constexpr (DK) vf[ks][s2] = *reinterpret_cast<const bf16x8*>(r + 2 * a.f.H + s2 * 16);
      }
    } else {
#pragma unroll
      for (int s2 = 0; s2 < QS; ++s2) {
        kf[ks][s2] = bf16x8{};
        if constexpr (DK) vf[ks][s2] = bf16x8{};
      }
    }
  }

  const int kr = lane / (D / 8), kp = lane % (D / 8);
  const uint32_t rowq = 3u * (uint32_t)a.f.H * 2u, rowg = (uint32_t)a.f.H * 2u;
  const char* qtxt = reinterpret_cast<const char*>(static_cast<const bf16*>(a.f.qkv_txt) + (int64_t)t0 * 3 * a.f.H + head * D);
  const char* qimg = reinterpret_cast<const char*>(static_cast<const bf16*>(a.f.qkv_img) + ((int64_t)i0 - Tb) * 3 * a.f.H + head * D);
  const char* gtxt = reinterpret_cast<const char*>(static_cast<const bf16*>(a.do_txt) + (int64_t)t0 * a.f.H + head * D);
  const char* gimg = reinterpret_cast<const char*>(static_cast<const bf16*>(a.do_img) + ((int64_t)i0 - Tb) * a.f.H + head * D);
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const bf16* tsrc = DK ? qt : gt;   // the transposed operand: Q^T (dK) or dO^T (dV)
  // whole query tiles inside the text or the image rows load through buffer
  // resources with the tile offset scalar (as in attn_bwd_dq_kernel)
  const rsrc_t rqt = make_rsrc(uniform_ptr(qtxt)), rqi = make_rsrc(uniform_ptr(qimg));
  const rsrc_t rgt = make_rsrc(uniform_ptr(gtxt)), rgi = make_rsrc(uniform_ptr(gimg)), rts = make_rsrc(tsrc);
  uint32_t kswc[RB], qoff[RB], goff[RB], toff[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    kswc[i] = ((kp ^ ksw<D>((wave + 4 * i) * KROWS + kr)) << 4);
    qoff[i] = (uint32_t)((wu + 4 * i) * KROWS + kr) * rowq + kswc[i];
    goff[i] = (uint32_t)((wu + 4 * i) * KROWS + kr) * rowg + kswc[i];
    const int d = (wave + 4 * i) * 16 + (lane >> 2);
    toff[i] = (uint32_t)((((int64_t)head * D + d) * a.f.njp + pstart + (((lane & 3) ^ tsw(d)) << 3)) * 2);
  }
  const float* lse_g = a.f.lse + (int64_t)head * a.f.njp + pstart;
  const float* ds_g = a.dsum + (int64_t)head * a.f.njp + pstart;
  auto issue = [&](int32_t q0, int st) {
    bf16* qs = smem + st * STAGE;
    bf16* gs = qs + TILE;                  // dO (dK only)
    bf16* ts = qs + (NT - 1) * TILE;       // the transposed tile
    float* lf = reinterpret_cast<float*>(qs + NT * TILE);
    if (q0 + BQ <= L && (q0 + BQ <= Tb || q0 >= Tb)) {
      const bool txt = q0 < Tb;
      const rsrc_t rq = txt ? rqt : rqi;
      const rsrc_t rg = txt ? rgt : rgi;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int blk = wu + 4 * i;
        buf_lds16(rq, qoff[i], (uint32_t)q0 * rowq, qs + blk * 512);
        if constexpr (DK) buf_lds16(rg, goff[i], (uint32_t)q0 * rowg, gs + blk * 512);
        buf_lds16(rts, toff[i], (uint32_t)q0 * 2, ts + blk * 512);
      }
    } else {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int blk = wu + 4 * i;
        const int32_t q = min(q0 + blk * KROWS + kr, L - 1);   // queries past L are masked
        load_lds16((q < Tb ? qtxt : qimg) + ((uint32_t)q * rowq + kswc[i]), qs + blk * 512);
        if constexpr (DK) load_lds16((q < Tb ? gtxt : gimg) + ((uint32_t)q * rowg + kswc[i]), gs + blk * 512);
        buf_lds16(rts, toff[i], (uint32_t)q0 * 2, ts + blk * 512);
      }
    }
    // lse (and D) of the tile's 32 queries by direct loads too: a plain load
    // into registers would make the LDS store wait for every load in flight,
    // this stage's tiles included (padded positions hold values the mask
    // never uses)
    if (wu == 0 && lane < (DK ? 16 : 8))
      load_lds16((lane < 8 ? lse_g + q0 + lane * 4 : ds_g + q0 + (lane - 8) * 4), lf);
  };

  f32x16 acc[KS][DT];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ks][t][v] = 0.f;
  const int ntile = (L + BQ - 1) / BQ;
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int prow = (l32 & 16) | kperm(l32 & 15);
  for (int it = 0; it < ntile; ++it) {
    const int st = it & 1;
    const int32_t q0 = it * BQ;
    if (it + 1 < ntile) issue(q0 + BQ, st ^ 1);
    const bf16* qs = smem + st * STAGE;
    const bf16* gs = qs + TILE;
    const bf16* ts = qs + (NT - 1) * TILE;
    const float* lf = reinterpret_cast<const float*>(qs + NT * TILE);
    f32x16 sc[KS], dp[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[ks][v] = dp[ks][v] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < QS; ++s2) {
      const int off = prow * D + (((s2 * 2 + g) ^ ksw<D>(prow)) << 3);
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qs + off);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sc[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks][s2], sc[ks], 0, 0, 0);
      if constexpr (DK) {
        const bf16x8 ga = *reinterpret_cast<const bf16x8*>(gs + off);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) dp[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[ks][s2], dp[ks], 0, 0, 0);
      }
    }
    // register v holds query q0 + 16 (v / 8) + 8 g + v % 8 of this lane's key
    bf16x8 pf[KS][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float lv[8], dv8[8];
      const int qi = 16 * h + 8 * g;
      *reinterpret_cast<f32x4*>(lv) = *reinterpret_cast<const f32x4*>(lf + qi);
      *reinterpret_cast<f32x4*>(lv + 4) = *reinterpret_cast<const f32x4*>(lf + qi + 4);
      if constexpr (DK) {
        *reinterpret_cast<f32x4*>(dv8) = *reinterpret_cast<const f32x4*>(lf + BQ + qi);
        *reinterpret_cast<f32x4*>(dv8 + 4) = *reinterpret_cast<const f32x4*>(lf + BQ + qi + 4);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int v = 8 * h + u;
          const float p = (q0 + qi + u < L) ? __builtin_amdgcn_exp2f(fmaf(sc[ks][v], a.f.scale_log2, -lv[u])) : 0.f;
          pf[ks][h][u] = DK ? (bf16)(p * (dp[ks][v] - dv8[u])) : (bf16)p;
        }
    }
    // dV^T[d][key] += dO^T[d][queries] P[queries][key], or dK^T += Q^T dS
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const int c = 2 * ks2 + g;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int d = t * 32 + l32;
        const bf16x8 ta = *reinterpret_cast<const bf16x8*>(ts + d * BQ + ((c ^ tsw(d)) << 3));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc[ks][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, pf[ks][ks2], acc[ks][t], 0, 0, 0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (jk[ks] >= L) continue;
    bf16* o = dqkv_row<bf16>(a, jk[ks], Tb, t0, i0) + head * D + (DK ? a.f.H : 2 * a.f.H);
    const float sc = DK ? a.inv_sqrt_d : 1.0f;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        bf16x4 w = {(bf16)(acc[ks][t][4 * vg] * sc), (bf16)(acc[ks][t][4 * vg + 1] * sc),
                    (bf16)(acc[ks][t][4 * vg + 2] * sc), (bf16)(acc[ks][t][4 * vg + 3] * sc)};
        *reinterpret_cast<bf16x4*>(o + t * 32 + 8 * vg + 4 * g) = w;
      }
  }
}

// key subtiles (of 32) per wave of the dK and dV kernels
constexpr int DKS = 1, DVS = 1;

template <int D>
mmdit_status launch_attn_bwd_mfma(const AttnBwdArgs& a, const mmdit_pack_t* pk, bf16* qt, bf16* kt, bf16* gt,
                                  hipStream_t s) {
  const int heads = a.f.heads;
  MMDIT_LAUNCH(attn_bwd_prep_kernel<D>, dim3((unsigned)cdiv(pk->max_joint, 64), heads, pk->B), dim3(256), 0, s, a, qt,
               kt, gt);
  MMDIT_TRY(launch_check("attn_bwd_prep_kernel", s));
  const size_t lds_dq = 2 * 3 * 32 * D * sizeof(bf16);
  const size_t lds_dk = 2 * (3 * 32 * D * sizeof(bf16) + 2 * 32 * sizeof(float));
  const size_t lds_dv = 2 * (2 * 32 * D * sizeof(bf16) + 2 * 32 * sizeof(float));
  static bool attr = false;
  if (!attr) {
    MMDIT_TRY(hip_check(hipFuncSetAttribute((const void*)attn_bwd_dq_kernel<D>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dq),
                        "hipFuncSetAttribute(attn_bwd_dq_kernel)"));
    MMDIT_TRY(hip_check(hipFuncSetAttribute((const void*)attn_bwd_dkdv_kernel<D, true, DKS>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dk),
                        "hipFuncSetAttribute(attn_bwd_dk_kernel)"));
    MMDIT_TRY(hip_check(hipFuncSetAttribute((const void*)attn_bwd_dkdv_kernel<D, false, DVS>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dv),
                        "hipFuncSetAttribute(attn_bwd_dv_kernel)"));
    attr = true;
  }
  dim3 grid((unsigned)cdiv(pk->max_joint, 128), heads, pk->B);
  MMDIT_LAUNCH(attn_bwd_dq_kernel<D>, grid, dim3(256), lds_dq, s, a, kt);
  MMDIT_TRY(launch_check("attn_bwd_dq_kernel", s));
  dim3 gk((unsigned)cdiv(pk->max_joint, 128 * DKS), heads, pk->B);
  MMDIT_LAUNCH((attn_bwd_dkdv_kernel<D, true, DKS>), gk, dim3(256), lds_dk, s, a, qt, gt);
  MMDIT_TRY(launch_check("attn_bwd_dk_kernel", s));
  dim3 gv((unsigned)cdiv(pk->max_joint, 128 * DVS), heads, pk->B);
  MMDIT_LAUNCH((attn_bwd_dkdv_kernel<D, false, DVS>), gv, dim3(256), lds_dv, s, a, qt, gt);
  return launch_check("attn_bwd_dv_kernel", s);
}

template <typename T, int D>
mmdit_status launch_attn_bwd(const AttnBwdArgs& a, dim3 grid, hipStream_t s) {
  MMDIT_LAUNCH((attn_bwd_dsum_kernel<T, D>), grid, dim3(256), 0, s, a);
  MMDIT_TRY(launch_check("attn_bwd_dsum_kernel", s));
  MMDIT_LAUNCH((attn_bwd_dq_simt_kernel<T, D>), grid, dim3(256), 0, s, a);
  MMDIT_TRY(launch_check("attn_bwd_dq_kernel", s));
  MMDIT_LAUNCH((attn_bwd_dkdv_simt_kernel<T, D>), grid, dim3(256), 0, s, a);
  return launch_check("attn_bwd_dkdv_kernel", s);
}

}  // namespace

int64_t attention_vt_elems(const mmdit_pack_t* pk, int32_t H) {
  int64_t njp = 0;
  for (int b = 0; b < pk->B; ++b) {
    const int64_t L = (pk->h_cu_txt[b + 1] - pk->h_cu_txt[b]) + (pk->h_cu_img[b + 1] - pk->h_cu_img[b]);
    njp += (L + 63) & ~(int64_t)63;
  }
  return njp * H;
}

mmdit_status attention_impl(mmdit_dtype dt, const mmdit_pack_t* pk, int32_t heads, int32_t D,
                            const void* qkv_img, const void* qkv_txt, void* o_img, void* o_txt,
                            void* ws, size_t ws_bytes, hipStream_t s, float* lse) {
  if (pk->B == 0 || pk->max_joint == 0) return MMDIT_OK;
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.lse = lse;
  a.njp = (int32_t)(attention_vt_elems(pk, heads * D) / (heads * D));
  a.qkv_img = qkv_img;
  a.qkv_txt = qkv_txt;
  a.o_img = o_img;
  a.o_txt = o_txt;
  a.cu_img = pk->cu_img;
  a.cu_txt = pk->cu_txt;
  a.heads = heads;
  a.H = heads * D;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  if (dt == MMDIT_BF16) {
    const int64_t vt_elems = attention_vt_elems(pk, a.H);
    if (!ws || ws_bytes < (size_t)vt_elems * 2) {
      set_error("mmdit_attention: workspace needs %zu bytes, got %zu", (size_t)vt_elems * 2, ws_bytes);
      return MMDIT_E_WORKSPACE;
    }
    if (vt_elems / a.H > INT32_MAX || (double)pk->max_joint * 3.0 * a.H * 2.0 >= 2147483648.0 ||
        (double)vt_elems * 2.0 >= 4294967296.0) {
      set_error("mmdit_attention: sample too long (joint length x 3 x hidden x 2 bytes must be < 2^31, "
                "the V^T staging < 2^32 bytes)");
      return MMDIT_E_UNSUPPORTED;
    }
    const int32_t njp = (int32_t)(vt_elems / a.H);
    bf16* vt = static_cast<bf16*>(ws);
    dim3 tgrid((unsigned)cdiv(pk->max_joint, 64), heads, pk->B);
    if (D == 128)
      MMDIT_LAUNCH(v_transpose_kernel<128>, tgrid, dim3(256), 0, s, a, vt, njp);
    else
      MMDIT_LAUNCH(v_transpose_kernel<64>, tgrid, dim3(256), 0, s, a, vt, njp);
    MMDIT_TRY(launch_check("v_transpose_kernel", s));
    // 4-wave blocks (128 queries): with the pipelined loop as fast as the
    // 8-wave ones at 33k tokens per sample and 4-9% faster at 4k-8k;
    // MMDIT_ATTN_WAVES=8 selects 256-query blocks (the same bits)
    const char* we = getenv("MMDIT_ATTN_WAVES");
    const int nw = (we && atoi(we) == 8) ? 8 : 4;
    a.nq = (int32_t)cdiv(pk->max_joint, 32 * nw);
    a.nB = pk->B;
    dim3 grid((unsigned)(8 * cdiv((int64_t)a.nq * heads * pk->B, 8)));
    const size_t lds = (2 + 2) * 64 * D * sizeof(bf16);   // two K stages, two V^T stages
    const void* fn = D == 128 ? (nw == 8 ? (const void*)attn_mfma_kernel<128, 8> : (const void*)attn_mfma_kernel<128, 4>)
                              : (nw == 8 ? (const void*)attn_mfma_kernel<64, 8> : (const void*)attn_mfma_kernel<64, 4>);
    static bool attr[4] = {false, false, false, false};
    const int ai = (D == 128 ? 2 : 0) + (nw == 8 ? 1 : 0);
    if (!attr[ai]) {
      MMDIT_TRY(hip_check(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds),
                          "hipFuncSetAttribute(attn_mfma_kernel)"));
      attr[ai] = true;
    }
    if (D == 128 && nw == 8)
      MMDIT_LAUNCH((attn_mfma_kernel<128, 8>), grid, dim3(512), lds, s, a, vt, njp);
    else if (D == 128)
      MMDIT_LAUNCH((attn_mfma_kernel<128, 4>), grid, dim3(256), lds, s, a, vt, njp);
    else if (nw == 8)
      MMDIT_LAUNCH((attn_mfma_kernel<64, 8>), grid, dim3(512), lds, s, a, vt, njp);
    else
      MMDIT_LAUNCH((attn_mfma_kernel<64, 4>), grid, dim3(256), lds, s, a, vt, njp);
    return launch_check("attn_mfma_kernel", s);
  }
  dim3 grid((unsigned)cdiv(pk->max_joint, 64), heads, pk->B);
  if (D == 128)
    MMDIT_LAUNCH((attn_simt_kernel<float, 128>), grid, dim3(256), 0, s, a);
  else
    MMDIT_LAUNCH((attn_simt_kernel<float, 64>), grid, dim3(256), 0, s, a);
  return launch_check("attn_simt_kernel", s);
}

size_t attention_bwd_ws_bytes(const mmdit_pack_t* pk, int32_t heads, int32_t D) {
  // D_i (float32) + Q^T, K^T, dO^T (bf16), all over the padded joint axis
  const size_t njp_h = (size_t)(attention_vt_elems(pk, heads * D) / D);   // heads x njp
  return ((njp_h * sizeof(float) + 255) & ~(size_t)255) + 3 * njp_h * D * sizeof(bf16);
}

mmdit_status attention_bwd_impl(mmdit_dtype dt, const mmdit_pack_t* pk, int32_t heads, int32_t D,
                                const void* qkv_img, const void* qkv_txt, const void* o_img, const void* o_txt,
                                const float* lse, const void* do_img, const void* do_txt, void* dqkv_img,
                                void* dqkv_txt, void* ws, size_t ws_bytes, hipStream_t s) {
  if (pk->B == 0 || pk->max_joint == 0) return MMDIT_OK;
  AttnBwdArgs a;
  memset(&a, 0, sizeof(a));
  a.f.qkv_img = qkv_img;
  a.f.qkv_txt = qkv_txt;
  a.f.o_img = const_cast<void*>(o_img);
  a.f.o_txt = const_cast<void*>(o_txt);
  a.f.cu_img = pk->cu_img;
  a.f.cu_txt = pk->cu_txt;
  a.f.heads = heads;
  a.f.H = heads * D;
  a.f.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  a.f.lse = const_cast<float*>(lse);
  a.f.njp = (int32_t)(attention_vt_elems(pk, heads * D) / (heads * D));
  a.do_img = do_img;
  a.do_txt = do_txt;
  a.dqkv_img = dqkv_img;
  a.dqkv_txt = dqkv_txt;
  a.inv_sqrt_d = (float)(1.0 / sqrt((double)D));
  const size_t need = attention_bwd_ws_bytes(pk, heads, D);
  if (!ws || ws_bytes < need) {
    set_error("attention backward: workspace needs %zu bytes, got %zu", need, ws_bytes);
    return MMDIT_E_WORKSPACE;
  }
  const size_t njp_h = (size_t)(attention_vt_elems(pk, heads * D) / D);
  a.dsum = static_cast<float*>(ws);
  if (dt == MMDIT_BF16) {
    if ((double)pk->max_joint * 3.0 * a.f.H * 2.0 >= 2147483648.0 || (double)njp_h * D * 2.0 >= 4294967296.0) {
      set_error("attention backward: sample too long (joint length x 3 x hidden x 2 bytes must be < 2^31, "
                "each transposed operand < 2^32 bytes)");
      return MMDIT_E_UNSUPPORTED;
    }
    bf16* qt = reinterpret_cast<bf16*>(static_cast<char*>(ws) + ((njp_h * sizeof(float) + 255) & ~(size_t)255));
    bf16* kt = qt + njp_h * D;
    bf16* gt = kt + njp_h * D;
    return D == 128 ? launch_attn_bwd_mfma<128>(a, pk, qt, kt, gt, s) : launch_attn_bwd_mfma<64>(a, pk, qt, kt, gt, s);
  }
  dim3 grid((unsigned)cdiv(pk->max_joint, 64), heads, pk->B);
  return D == 128 ? launch_attn_bwd<float, 128>(a, grid, s) : launch_attn_bwd<float, 64>(a, grid, s);
}

}  // namespace mmdit
