// Elementwise and reduction kernels of the block's backward pass.
//
// The block's gradients follow from its forward definition by the chain rule
// (the pages train the backbone with the rectified-flow objective on packed
// samples: hyper.ai 2607.19064, 方法; blog close-reading, 2.2(2)).  The dense
// products of the backward run on the GEMM kernels; this file holds what
// surrounds them:
//   transpose_kernel      [n, C] -> [C, n padded to 64] (optionally GELU of the
//                         input, or rows scaled by a per-sample gate with the
//                         scaled rows also written), the K-major operands of
//                         the weight-gradient GEMMs and the transposed weights
//   colsum_kernel         per-sample column sums of up to three row products,
//                         in fixed row chunks that never straddle two samples
//   colsum_finalize_kernel  the chunk sums of each sample added in chunk order
//   norm_bwd_kernel       through h = rms(x)(1 + scale) + shift:
//                         dx = dres + (dn - n mean(dn n)) / rms, dn = dh (1 + scale)
//   qk_bwd_kernel         through q' = RoPE(g * rms(q)) per head: inverse
//                         rotation, gain gradient partials, norm backward
//   outer_kernel          dW = dy^T f(x) over the sample axis (adaLN, conditioning)
//   vecmat_part_kernel, vecmat_finalize_kernel
//                         dx += (dy W) * f'(x), over row chunks of W, the
//                         chunk products added in chunk order
// All sums run in a fixed order: results do not depend on scheduling.
#include "common.h"

#include <string.h>

namespace mmdit {

namespace {

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i, bool f32) {
  return f32 ? static_cast<const float*>(p)[i] : to_f(static_cast<const T*>(p)[i]);
}

// ------------------------------------------------------------- transpose
struct TrProb {
  const void* x;        // [n, C], row stride ldx
  void* y;              // [C, npad]
  void* y_rows;         // op 2, optional: the scaled rows [n, C]
  const float* gate;    // op 2: scale gate[seg[m] * gate_stride + c]
  const int32_t* seg;
  int64_t ldx, n, npad, gate_stride;
  int32_t C;
};
struct TrBatch {
  TrProb p[2];
  int32_t op;           // 0 copy, 1 GELU, 2 gate scale
};

template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(TrBatch bt) {
  __shared__ float t[64][65];
  const TrProb& P = bt.p[blockIdx.z];
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  if (m0 >= P.npad || c0 >= P.C) return;
  const T* x = static_cast<const T*>(P.x);
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    const int64_t m = m0 + r;
    float v = 0.f;
    if (m < P.n && c0 + c < P.C) {
      v = to_f(x[m * P.ldx + c0 + c]);
      if (bt.op == 1) {
        v = gelu_f(v);
      } else if (bt.op == 2) {
        v *= P.gate[(int64_t)P.seg[m] * P.gate_stride + c0 + c];
        if (P.y_rows) static_cast<T*>(P.y_rows)[m * P.C + c0 + c] = from_f<T>(v);
      }
    }
    t[r][c] = v;
  }
  __syncthreads();
  T* y = static_cast<T*>(P.y);
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int c = i >> 6, r = i & 63;
    if (c0 + c < P.C && m0 + r < P.npad) y[(int64_t)(c0 + c) * P.npad + m0 + r] = from_f<T>(t[r][c]);
  }
}

// bf16, C % 8 == 0: 16-byte loads along c and 16-byte stores along m through
// a 64 x 64 tile in LDS.
__global__ void __launch_bounds__(256) transpose_bf16_kernel(TrBatch bt) {
  __shared__ bf16 t[64][64 + 8];
  const TrProb& P = bt.p[blockIdx.z];
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  if (m0 >= P.npad || c0 >= P.C) return;
  const bf16* x = static_cast<const bf16*>(P.x);
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int r = i >> 3, ch = i & 7;
    const int64_t m = m0 + r;
    const int c = c0 + ch * 8;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (m < P.n && c < P.C) {
      Vec8<bf16>::load(x + m * P.ldx + c, v);
      if (bt.op == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = gelu_f(v[e]);
      } else if (bt.op == 2) {
        float g8[8];
        Vec8<float>::load(P.gate + (int64_t)P.seg[m] * P.gate_stride + c, g8);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= g8[e];
        if (P.y_rows) Vec8<bf16>::store(static_cast<bf16*>(P.y_rows) + m * P.C + c, v);
      }
    }
    bf16x8 w;
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = (bf16)v[e];
    *reinterpret_cast<bf16x8*>(&t[r][ch * 8]) = w;
  }
  __syncthreads();
  bf16* y = static_cast<bf16*>(P.y);
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int cc = i >> 3, mch = i & 7;
    const int c = c0 + cc;
    const int64_t m = m0 + mch * 8;
    if (c >= P.C || m >= P.npad) continue;
    bf16x8 w;
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = t[mch * 8 + e][cc];
    *reinterpret_cast<bf16x8*>(y + (int64_t)c * P.npad + m) = w;
  }
}

// ------------------------------------------------------- per-sample sums
struct ColTerm {
  const void* a;        // [n, H]
  const void* b;        // [n, H] or NULL (row b_map[r] when b_map is set)
  const float* rs;      // [n] row scale or NULL
  const int32_t* b_map;
  int32_t a_f32, b_f32;
};
struct ColsumArgs {
  ColTerm t[3];
  int32_t nterms;
  const int32_t* cu;    // [B + 1] first row of every sample
  int32_t B, H, rc;     // rows per chunk
  float* partial;       // [chunks][nterms][H]
  float* out;           // finalize: out[b * out_stride + out_off[k] + c]
  int64_t out_stride;
  int32_t out_off[3];
};

// chunk ci -> sample b and its row range [r0, r1); false past the last chunk
__device__ __forceinline__ bool chunk_rows(const ColsumArgs& a, int ci, int& b, int32_t& r0, int32_t& r1) {
  int acc = 0;
  for (int s = 0; s < a.B; ++s) {
    const int32_t n = a.cu[s + 1] - a.cu[s];
    const int ch = (n + a.rc - 1) / a.rc;
    if (ci < acc + ch) {
      b = s;
      r0 = a.cu[s] + (ci - acc) * a.rc;
      r1 = min(r0 + a.rc, a.cu[s + 1]);
      return true;
    }
    acc += ch;
  }
  return false;
}

template <typename T>
__device__ __forceinline__ void ld8(const void* p, int64_t i, bool f32, float* v) {
  if (f32) Vec8<float>::load(static_cast<const float*>(p) + i, v);
  else Vec8<T>::load(static_cast<const T*>(p) + i, v);
}

template <typename T>
__device__ __forceinline__ void term8(const ColTerm& t, int32_t r, int c, int H, float* v) {
  ld8<T>(t.a, (int64_t)r * H + c, t.a_f32, v);
  if (t.b) {
    float w[8];
    ld8<T>(t.b, (int64_t)(t.b_map ? t.b_map[r] : r) * H + c, t.b_f32, w);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= w[e];
  }
  if (t.rs) {
    const float q = t.rs[r];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= q;
  }
}

template <typename T>
__device__ __forceinline__ float term(const ColTerm& t, int32_t r, int c, int H) {
  float v = ld<T>(t.a, (int64_t)r * H + c, t.a_f32);
  if (t.b) v *= ld<T>(t.b, (int64_t)(t.b_map ? t.b_map[r] : r) * H + c, t.b_f32);
  if (t.rs) v *= t.rs[r];
  return v;
}

// Every term in one pass over the chunk's rows (rows in order, so each sum
// has a fixed order), several rows' loads in flight.
template <typename T>
__global__ void __launch_bounds__(256) colsum_kernel(ColsumArgs a) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int ci = blockIdx.y;
  int b;
  int32_t r0, r1;
  if (!chunk_rows(a, ci, b, r0, r1) || c >= a.H) return;
  float s[3] = {0.f, 0.f, 0.f};
  int32_t r = r0;
  for (; r + 4 <= r1; r += 4) {
    float v[3][4];
#pragma unroll
    for (int k = 0; k < 3; ++k)
      if (k < a.nterms)
#pragma unroll
        for (int u = 0; u < 4; ++u) v[k][u] = term<T>(a.t[k], r + u, c, a.H);
#pragma unroll
    for (int k = 0; k < 3; ++k)
      if (k < a.nterms)
#pragma unroll
        for (int u = 0; u < 4; ++u) s[k] += v[k][u];
  }
  for (; r < r1; ++r)
#pragma unroll
    for (int k = 0; k < 3; ++k)
      if (k < a.nterms) s[k] += term<T>(a.t[k], r, c, a.H);
#pragma unroll
  for (int k = 0; k < 3; ++k)
    if (k < a.nterms) a.partial[((int64_t)ci * a.nterms + k) * a.H + c] = s[k];
}

// 8 columns per thread (16-byte loads), rows in order: the same per-column
// sums as colsum_kernel.
template <typename T>
__global__ void __launch_bounds__(256) colsum8_kernel(ColsumArgs a) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 8;
  const int ci = blockIdx.y;
  int b;
  int32_t r0, r1;
  if (!chunk_rows(a, ci, b, r0, r1) || c >= a.H) return;
  float s[3][8];
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) s[k][e] = 0.f;
#pragma unroll 4
  for (int32_t r = r0; r < r1; ++r) {
#pragma unroll
    for (int k = 0; k < 3; ++k)
      if (k < a.nterms) {
        float v[8];
        term8<T>(a.t[k], r, c, a.H, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[k][e] += v[e];
      }
  }
#pragma unroll
  for (int k = 0; k < 3; ++k)
    if (k < a.nterms) Vec8<float>::store(a.partial + ((int64_t)ci * a.nterms + k) * a.H + c, s[k]);
}

__global__ void __launch_bounds__(256) colsum_finalize_kernel(ColsumArgs a) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y, k = blockIdx.z;
  if (c >= a.H) return;
  int first = 0;
  for (int s = 0; s < b; ++s) first += (a.cu[s + 1] - a.cu[s] + a.rc - 1) / a.rc;
  const int ch = (a.cu[b + 1] - a.cu[b] + a.rc - 1) / a.rc;
  // eight interleaved running sums combined in a fixed tree: a fixed order
  float p[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < ch; ++i) p[i & 7] += a.partial[((int64_t)(first + i) * a.nterms + k) * a.H + c];
  a.out[(int64_t)b * a.out_stride + a.out_off[k] + c] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

// ------------------------------------------------------------ norm bwd
struct NormBwdProb {
  const int32_t* row_map;   // optional: x, seg and dx rows are row_map[row]
  const void* x;        // [n, H] norm input
  const void* dh;       // [n, H] gradient of rms(x)(1 + scale) + shift
  const float* mod;     // scale at mod[seg * mod_stride + scale_off]
  const int32_t* seg;
  const void* dres;     // [n, H] gradient reaching x along the residual, or NULL
  void* dx;             // [n, H] output (may alias dres)
  float* inv_r;         // [n] output: 1 / rms(x)
  const float* gate;    // optional: dgated = gate[seg * mod_stride + gate_off] * dx
  void* dgated;
  int64_t n, mod_stride;
  int32_t scale_off, gate_off, dres_f32, dx_f32;
};
struct NormBwdBatch {
  NormBwdProb p[2];
  int64_t split;        // blocks of problem 0
  int32_t H;
  float eps;
};

// One wave per row, 8 rows per block; two passes over the row (statistics,
// then the gradient), the row staying in L2 between them.
template <typename T>
__global__ void __launch_bounds__(512) norm_bwd_kernel(NormBwdBatch bt) {
  int64_t blk = blockIdx.x;
  const NormBwdProb& P = blk < bt.split ? bt.p[0] : bt.p[1];
  if (blk >= bt.split) blk -= bt.split;
  const int64_t row = blk * 8 + (threadIdx.x >> 6);
  if (row >= P.n) return;
  const int lane = threadIdx.x & 63;
  const int H = bt.H;
  const int64_t xr = P.row_map ? (int64_t)P.row_map[row] : row;   // row of x, seg and dx
  const int32_t sg = P.seg[xr];
  const float* sc = P.mod + (int64_t)sg * P.mod_stride + P.scale_off;
  const T* x = static_cast<const T*>(P.x) + xr * H;
  const T* dh = static_cast<const T*>(P.dh) + row * H;
  float ss = 0.f, sd = 0.f;
  for (int c = lane * 8; c < H; c += 512) {
    float xv[8], dv[8], s8[8];
    Vec8<T>::load(x + c, xv);
    Vec8<T>::load(dh + c, dv);
    Vec8<float>::load(sc + c, s8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ss += xv[e] * xv[e];
      sd += dv[e] * (1.0f + s8[e]) * xv[e];
    }
  }
  ss = wave_sum(ss);
  sd = wave_sum(sd);
  const float r = 1.0f / sqrtf(ss / (float)H + bt.eps);
  const float cm = r * sd / (float)H;            // mean(dn * n)
  if (lane == 0) P.inv_r[row] = r;
  const float* gt = P.gate ? P.mod + (int64_t)sg * P.mod_stride + P.gate_off : nullptr;
  for (int c = lane * 8; c < H; c += 512) {
    float xv[8], dv[8], s8[8], rv[8], o[8];
    Vec8<T>::load(x + c, xv);
    Vec8<T>::load(dh + c, dv);
    Vec8<float>::load(sc + c, s8);
    if (!P.dres) {
#pragma unroll
      for (int e = 0; e < 8; ++e) rv[e] = 0.f;
    } else if (P.dres_f32) {
      Vec8<float>::load(static_cast<const float*>(P.dres) + row * H + c, rv);
    } else {
      Vec8<T>::load(static_cast<const T*>(P.dres) + row * H + c, rv);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = rv[e] + (dv[e] * (1.0f + s8[e]) - xv[e] * r * cm) * r;
    if (P.dx_f32) Vec8<float>::store(static_cast<float*>(P.dx) + xr * H + c, o);
    else Vec8<T>::store(static_cast<T*>(P.dx) + xr * H + c, o);
    if (gt) {
      float g8[8];
      Vec8<float>::load(gt + c, g8);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= g8[e];
      Vec8<T>::store(static_cast<T*>(P.dgated) + row * H + c, o);
    }
  }
}

// ------------------------------------------------------- QK-norm + RoPE bwd
typedef RopeTable RopeTabB;
struct QkBwdProb {
  void* dqkv;           // [n, 3H] in: dq', dk' (and dv); out: dq, dk in place
  const void* raw;      // [n, 2H] q, k before the norm
  const int32_t* pos;   // NULL: no rotation (text rows)
  const float* g_q;
  const float* g_k;
  float* gpart;         // [blocks][2][D] per-block gain-gradient partials
  int64_t n;
};
struct QkBwdBatch {
  QkBwdProb p[2];
  int64_t split;        // blocks of problem 0
  int32_t heads;
  float eps;
};

constexpr int kQkRows = 32;   // rows per block (8 per wave)

template <typename T, int D>
__global__ void __launch_bounds__(256) qk_bwd_kernel(QkBwdBatch bt, RopeTabB tab) {
  constexpr int LPH = D / 8;
  constexpr int HPS = 64 / LPH;
  __shared__ float red[4][64][16];
  int64_t blk = blockIdx.x;
  const QkBwdProb& P = blk < bt.split ? bt.p[0] : bt.p[1];
  if (blk >= bt.split) blk -= bt.split;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPH, hv0 = lane / LPH;
  const int heads = bt.heads;
  const int64_t H = (int64_t)heads * D;
  float gq[8], gk[8], aq[8], ak[8];
  Vec8<float>::load(P.g_q + sub * 8, gq);
  Vec8<float>::load(P.g_k + sub * 8, gk);
#pragma unroll
  for (int e = 0; e < 8; ++e) aq[e] = ak[e] = 0.f;
  for (int rr = 0; rr < kQkRows / 4; ++rr) {
    const int64_t row = blk * kQkRows + wave * (kQkRows / 4) + rr;
    if (row >= P.n) break;
    float cs[4], sn[4];
    if (P.pos) {
      const int32_t p3[3] = {P.pos[3 * row], P.pos[3 * row + 1], P.pos[3 * row + 2]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pr = sub * 4 + j;
        sincosf((float)p3[tab.axis[pr]] * tab.inv_freq[pr], &sn[j], &cs[j]);
      }
    }
    T* g = static_cast<T*>(P.dqkv) + row * 3 * H + sub * 8;
    const T* x = static_cast<const T*>(P.raw) + row * 2 * H + sub * 8;
    for (int hv = hv0; hv < 2 * heads; hv += HPS) {
      float dv[8], xv[8];
      Vec8<T>::load(g + hv * D, dv);
      Vec8<T>::load(x + hv * D, xv);
      if (P.pos) {   // the rotation's transpose: turn the gradient back
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = dv[2 * j], b = dv[2 * j + 1];
          dv[2 * j] = a * cs[j] + b * sn[j];
          dv[2 * j + 1] = -a * sn[j] + b * cs[j];
        }
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += xv[e] * xv[e];
      ss = group_sum(ss, LPH);
      const float r = 1.0f / sqrtf(ss / (float)D + bt.eps);
      const bool isq = hv < heads;
      const float* gg = isq ? gq : gk;
      float* acc = isq ? aq : ak;
      float dn[8], sd = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[e] += dv[e] * xv[e] * r;         // gain gradient: d(g n) . n
        dn[e] = dv[e] * gg[e];
        sd += dn[e] * xv[e];
      }
      sd = group_sum(sd, LPH) * r / (float)D;   // mean(dn * n)
#pragma unroll
      for (int e = 0; e < 8; ++e) dv[e] = (dn[e] - xv[e] * r * sd) * r;
      Vec8<T>::store(g + hv * D, dv);
    }
  }
  // block partial of the gain gradients, summed in a fixed order
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[wave][lane][e] = aq[e];
    red[wave][lane][8 + e] = ak[e];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * D; i += 256) {
    const int which = i / D, dd = i % D;
    const int sb = dd / 8, e = dd % 8;
    float s = 0.f;
    for (int w = 0; w < 4; ++w)
      for (int h0 = 0; h0 < HPS; ++h0) s += red[w][h0 * LPH + sb][which * 8 + e];
    P.gpart[(blk * 2 + which) * D + dd] = s;
  }
}

// One wave per gain element: lane l adds the partials of blocks l, l + 64,
// ... in order, then a fixed butterfly over the lanes (a fixed order).
__global__ void __launch_bounds__(64) qk_gain_finalize_kernel(const float* gpart, int64_t blocks, int32_t D,
                                                              float* dg_q, float* dg_k) {
  const int i = blockIdx.x;
  const int which = i / D, dd = i % D;
  float s = 0.f;
  for (int64_t b = threadIdx.x; b < blocks; b += 64) s += gpart[(b * 2 + which) * D + dd];
  s = wave_sum(s);
  if (threadIdx.x == 0) (which ? dg_k : dg_q)[dd] = s;
}

// ------------------------------------------- products over the sample axis
// For a linear y = W f(x) applied to one vector per sample (adaLN, the
// conditioning MLP): dW = dy^T f(x) and df(x) = dy W, both sums over samples
// or rows in a fixed order.

// f(X) and f'(X) [B, cols] float32: SiLU (mode 0) or the identity (mode 1).
template <typename T>
__global__ void __launch_bounds__(256) act_pair_kernel(const void* __restrict__ x, int32_t x_f32, int32_t mode,
                                                       float* __restrict__ f, float* __restrict__ df, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = ld<T>(x, i, x_f32);
  if (mode == 1) {
    f[i] = v;
    df[i] = 1.0f;
    return;
  }
  const float sg = 1.0f / (1.0f + __expf(-v));
  f[i] = v * sg;
  df[i] = sg * (1.0f + v * (1.0f - sg));
}

// dW[i][j] = sum_b dy[b][i] f[b][j] ([rows, cols] float32): 16 rows of 256
// columns per block (rows a multiple of 16).
__global__ void __launch_bounds__(256) outer_kernel(const float* __restrict__ dy, const float* __restrict__ f,
                                                    float* __restrict__ dw, int32_t B, int32_t cols, int32_t rows) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int i0 = blockIdx.y * 16;
  if (j >= cols) return;
  float acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int b = 0; b < B; ++b) {
    const float x = f[(int64_t)b * cols + j];
    const float* dm = dy + (int64_t)b * rows + i0;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = fmaf(dm[r], x, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) dw[(int64_t)(i0 + r) * cols + j] = acc[r];
}

// Partial products part[kc][b][j] = sum over the rows i of chunk kc (chunks
// of kr rows; stream 0's chunks, then stream 1's) of dy[b][i] W[i][j];
// dy of 16 samples x 128 rows staged in LDS.
template <typename T>
__global__ void __launch_bounds__(256) vecmat_part_kernel(const float* __restrict__ dy0, const float* __restrict__ dy1,
                                                          const T* __restrict__ w0, const T* __restrict__ w1,
                                                          float* __restrict__ part, int32_t B, int32_t cols,
                                                          int32_t rows, int32_t kr, int32_t kch) {
  __shared__ float sd[16][128];
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int kc = blockIdx.y;
  const int b0 = blockIdx.z * 16;
  const int st = kc >= kch;
  const float* dm = st ? dy1 : dy0;
  const T* w = st ? w1 : w0;
  const int i0 = (kc - st * kch) * kr;
  const int i1 = min(i0 + kr, rows);
  float acc[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) acc[u] = 0.f;
  for (int ib = i0; ib < i1; ib += 128) {
    const int n = min(128, i1 - ib);
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * 128; e += 256) {
      const int u = e >> 7, ii = e & 127;
      sd[u][ii] = (b0 + u < B && ii < n) ? dm[(int64_t)(b0 + u) * rows + ib + ii] : 0.f;
    }
    __syncthreads();
    if (j < cols)
      for (int ii = 0; ii < n; ++ii) {
        const float wv = to_f(w[(int64_t)(ib + ii) * cols + j]);
#pragma unroll
        for (int u = 0; u < 16; ++u) acc[u] = fmaf(sd[u][ii], wv, acc[u]);
      }
  }
  if (j >= cols) return;
#pragma unroll
  for (int u = 0; u < 16; ++u)
    if (b0 + u < B) part[((int64_t)kc * B + b0 + u) * cols + j] = acc[u];
}

// dx[b][j] += f'(x[b][j]) * sum over the chunks, in chunk order.
__global__ void __launch_bounds__(256) vecmat_finalize_kernel(const float* __restrict__ part, const float* __restrict__ df,
                                                              float* __restrict__ dx, int64_t n, int32_t nk) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k = 0; k < nk; ++k) s += part[(int64_t)k * n + i];
  dx[i] += s * df[i];
}

}  // namespace

// ------------------------------------------------------------- launchers
mmdit_status transpose2_impl(mmdit_dtype dt, const TransposeArgs* t, int n, int op, hipStream_t s) {
  TrBatch bt;
  memset(&bt, 0, sizeof(bt));
  bt.op = op;
  int64_t npad = 0;
  int32_t C = 0;
  for (int i = 0; i < n; ++i) {
    TrProb& p = bt.p[i];
    p.x = t[i].x;
    p.y = t[i].y;
    p.y_rows = t[i].y_rows;
    p.gate = t[i].gate;
    p.seg = t[i].seg;
    p.ldx = t[i].ldx;
    p.n = t[i].n;
    p.npad = t[i].npad;
    p.gate_stride = t[i].gate_stride;
    p.C = t[i].C;
    npad = p.npad > npad ? p.npad : npad;
    C = p.C > C ? p.C : C;
  }
  if (npad == 0 || C == 0) return MMDIT_OK;
  dim3 grid((unsigned)cdiv(npad, 64), (unsigned)cdiv(C, 64), n);
  bool vec = dt == MMDIT_BF16;
  for (int i = 0; i < n; ++i) vec = vec && t[i].C % 8 == 0 && t[i].ldx % 8 == 0 && t[i].npad % 8 == 0;
  if (vec) MMDIT_LAUNCH(transpose_bf16_kernel, grid, dim3(256), 0, s, bt);
  else if (dt == MMDIT_BF16) MMDIT_LAUNCH(transpose_kernel<bf16>, grid, dim3(256), 0, s, bt);
  else MMDIT_LAUNCH(transpose_kernel<float>, grid, dim3(256), 0, s, bt);
  return launch_check("transpose_kernel", s);
}

int64_t colsum_chunks(const int32_t* h_cu, int32_t B, int32_t rc) {
  int64_t c = 0;
  for (int b = 0; b < B; ++b) c += cdiv(h_cu[b + 1] - h_cu[b], rc);
  return c;
}

mmdit_status seg_colsum_impl(mmdit_dtype dt, const ColsumSpec& sp, hipStream_t s) {
  ColsumArgs a;
  memset(&a, 0, sizeof(a));
  a.nterms = sp.nterms;
  for (int k = 0; k < sp.nterms; ++k) {
    a.t[k].a = sp.a[k];
    a.t[k].b = sp.b[k];
    a.t[k].b_map = sp.b_map[k];
    a.t[k].rs = sp.rs[k];
    a.t[k].a_f32 = sp.a_f32[k];
    a.t[k].b_f32 = sp.b_f32[k];
    a.out_off[k] = sp.out_off[k];
  }
  a.cu = sp.cu;
  a.B = sp.B;
  a.H = sp.H;
  a.rc = kColsumRows;
  a.partial = sp.partial;
  a.out = sp.out;
  a.out_stride = sp.out_stride;
  const int64_t chunks = colsum_chunks(sp.h_cu, sp.B, kColsumRows);
  if (sp.B == 0) return MMDIT_OK;
  if (chunks > 0) {
    if (sp.H % 8 == 0) {
      dim3 grid((unsigned)cdiv(sp.H / 8, 256), (unsigned)chunks);
      if (dt == MMDIT_BF16) MMDIT_LAUNCH(colsum8_kernel<bf16>, grid, dim3(256), 0, s, a);
      else MMDIT_LAUNCH(colsum8_kernel<float>, grid, dim3(256), 0, s, a);
    } else {
      dim3 grid((unsigned)cdiv(sp.H, 256), (unsigned)chunks);
      if (dt == MMDIT_BF16) MMDIT_LAUNCH(colsum_kernel<bf16>, grid, dim3(256), 0, s, a);
      else MMDIT_LAUNCH(colsum_kernel<float>, grid, dim3(256), 0, s, a);
    }
    MMDIT_TRY(launch_check("colsum_kernel", s));
  }
  MMDIT_LAUNCH(colsum_finalize_kernel, dim3((unsigned)cdiv(sp.H, 256), sp.B, sp.nterms), dim3(256), 0, s, a);
  return launch_check("colsum_finalize_kernel", s);
}

mmdit_status norm_bwd2_impl(mmdit_dtype dt, int32_t H, float eps, const NormBwdSpec* p, int n, hipStream_t s) {
  NormBwdBatch bt;
  memset(&bt, 0, sizeof(bt));
  bt.H = H;
  bt.eps = eps;
  int64_t blocks[2] = {0, 0};
  for (int i = 0; i < n; ++i) {
    NormBwdProb& q = bt.p[i];
    q.row_map = p[i].row_map;
    q.x = p[i].x;
    q.dh = p[i].dh;
    q.mod = p[i].mod;
    q.seg = p[i].seg;
    q.dres = p[i].dres;
    q.dx = p[i].dx;
    q.inv_r = p[i].inv_r;
    q.gate = p[i].gate;
    q.dgated = p[i].dgated;
    q.n = p[i].n;
    q.mod_stride = p[i].mod_stride;
    q.scale_off = p[i].scale_off;
    q.gate_off = p[i].gate_off;
    q.dres_f32 = p[i].dres_f32;
    q.dx_f32 = p[i].dx_f32;
    blocks[i] = cdiv(q.n, 8);
  }
  bt.split = blocks[0];
  const int64_t total = blocks[0] + blocks[1];
  if (total == 0) return MMDIT_OK;
  if (dt == MMDIT_BF16) MMDIT_LAUNCH(norm_bwd_kernel<bf16>, dim3((unsigned)total), dim3(512), 0, s, bt);
  else MMDIT_LAUNCH(norm_bwd_kernel<float>, dim3((unsigned)total), dim3(512), 0, s, bt);
  return launch_check("norm_bwd_kernel", s);
}

int64_t qk_bwd_blocks(int64_t n_rows) { return cdiv(n_rows, kQkRows); }

mmdit_status qk_bwd2_impl(mmdit_dtype dt, int32_t heads, int32_t D, const int32_t* widths, float theta, float eps,
                          const QkBwdSpec* p, int n, hipStream_t s) {
  QkBwdBatch bt;
  memset(&bt, 0, sizeof(bt));
  bt.heads = heads;
  bt.eps = eps;
  int64_t blocks[2] = {0, 0};
  for (int i = 0; i < n; ++i) {
    QkBwdProb& q = bt.p[i];
    q.dqkv = p[i].dqkv;
    q.raw = p[i].raw;
    q.pos = p[i].pos;
    q.g_q = p[i].g_q;
    q.g_k = p[i].g_k;
    q.gpart = p[i].gpart;
    q.n = p[i].n;
    blocks[i] = qk_bwd_blocks(q.n);
  }
  bt.split = blocks[0];
  RopeTabB tab;
  rope_table(&tab, widths, theta);
  const int64_t total = blocks[0] + blocks[1];
  if (total > 0) {
    dim3 g((unsigned)total), b(256);
    if (dt == MMDIT_BF16) {
      if (D == 128) MMDIT_LAUNCH((qk_bwd_kernel<bf16, 128>), g, b, 0, s, bt, tab);
      else MMDIT_LAUNCH((qk_bwd_kernel<bf16, 64>), g, b, 0, s, bt, tab);
    } else {
      if (D == 128) MMDIT_LAUNCH((qk_bwd_kernel<float, 128>), g, b, 0, s, bt, tab);
      else MMDIT_LAUNCH((qk_bwd_kernel<float, 64>), g, b, 0, s, bt, tab);
    }
    MMDIT_TRY(launch_check("qk_bwd_kernel", s));
  }
  for (int i = 0; i < n; ++i) {
    MMDIT_LAUNCH(qk_gain_finalize_kernel, dim3((unsigned)(2 * D)), dim3(64), 0, s, p[i].gpart, blocks[i], D,
                 p[i].dg_q, p[i].dg_k);
    MMDIT_TRY(launch_check("qk_gain_finalize_kernel", s));
  }
  return MMDIT_OK;
}

// chunks per stream of the vector-matrix partial products: enough blocks to
// fill the chip, partials bounded to about 64 MB
int32_t outer_vecmat_chunks(int32_t B, int32_t rows, int32_t cols) {
  int64_t kch = rows / 128;
  const int64_t cap = (int64_t)16 * 1024 * 1024 / ((int64_t)2 * (B > 0 ? B : 1) * cols);
  if (kch > cap) kch = cap;
  return (int32_t)(kch < 1 ? 1 : kch);
}

size_t outer_vecmat_ws_bytes(int32_t B, int32_t rows, int32_t cols) {
  return (size_t)2 * B * cols * 4 + (size_t)2 * outer_vecmat_chunks(B, rows, cols) * B * cols * 4;
}

mmdit_status outer_vecmat_impl(mmdit_dtype dt, int32_t B, int32_t rows, int32_t cols, int ns, const float* const* dy,
                               const void* const* w, const void* x, int32_t x_f32, int32_t mode, float* const* dw,
                               float* dx, void* ws, size_t ws_bytes, hipStream_t s) {
  if (B == 0) return MMDIT_OK;
  if (rows % 16 || ns < 1 || ns > 2) {
    set_error("outer/vector-matrix product: rows %d must be a multiple of 16, streams %d in 1..2", rows, ns);
    return MMDIT_E_UNSUPPORTED;
  }
  if (!ws || ws_bytes < outer_vecmat_ws_bytes(B, rows, cols)) {
    set_error("outer/vector-matrix product: workspace needs %zu bytes, got %zu", outer_vecmat_ws_bytes(B, rows, cols),
              ws_bytes);
    return MMDIT_E_WORKSPACE;
  }
  float* f = static_cast<float*>(ws);
  float* df = f + (size_t)B * cols;
  float* part = df + (size_t)B * cols;
  const int64_t n = (int64_t)B * cols;
  if (dt == MMDIT_BF16)
    MMDIT_LAUNCH(act_pair_kernel<bf16>, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, x, x_f32, mode, f, df, n);
  else
    MMDIT_LAUNCH(act_pair_kernel<float>, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, x, x_f32, mode, f, df, n);
  MMDIT_TRY(launch_check("act_pair_kernel", s));
  for (int st = 0; st < ns; ++st) {
    MMDIT_LAUNCH(outer_kernel, dim3((unsigned)cdiv(cols, 256), (unsigned)(rows / 16)), dim3(256), 0, s, dy[st], f,
                 dw[st], B, cols, rows);
    MMDIT_TRY(launch_check("outer_kernel", s));
  }
  if (!dx) return MMDIT_OK;
  const int32_t kch = outer_vecmat_chunks(B, rows, cols);
  const int32_t kr = (int32_t)cdiv(rows, kch);
  dim3 g((unsigned)cdiv(cols, 256), (unsigned)(ns * kch), (unsigned)cdiv(B, 16));
  const void* w1 = ns > 1 ? w[1] : w[0];
  const float* dy1 = ns > 1 ? dy[1] : dy[0];
  if (dt == MMDIT_BF16)
    MMDIT_LAUNCH(vecmat_part_kernel<bf16>, g, dim3(256), 0, s, dy[0], dy1, static_cast<const bf16*>(w[0]),
                 static_cast<const bf16*>(w1), part, B, cols, rows, kr, kch);
  else
    MMDIT_LAUNCH(vecmat_part_kernel<float>, g, dim3(256), 0, s, dy[0], dy1, static_cast<const float*>(w[0]),
                 static_cast<const float*>(w1), part, B, cols, rows, kr, kch);
  MMDIT_TRY(launch_check("vecmat_part_kernel", s));
  MMDIT_LAUNCH(vecmat_finalize_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, part, df, dx, n, ns * kch);
  return launch_check("vecmat_finalize_kernel", s);
}

}  // namespace mmdit
