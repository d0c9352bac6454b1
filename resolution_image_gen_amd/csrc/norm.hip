// Fused per-token chains of the block: RMSNorm + adaLN modulate, and
// QK-RMSNorm + 3-axis RoPE (blog close-reading 2.2(3): the norm / RoPE /
// gating / residual chains are the memory-bound ones and are fused; 2.2(2) and
// hyper.ai 2607.19064 方法: per-sample 2D RoPE plus a frame axis for editing).
// Both are HBM-bound: one read and one write of every element, statistics in
// registers, one wave per row.
#include "common.h"

#include <math.h>
#include <string.h>

namespace mmdit {

namespace {

// ------------------------------------------------ RMSNorm + adaLN modulate
// y[i] = x[src] / sqrt(mean(x[src]^2) + eps) * (1 + scale[s]) + shift[s],
// src = row_map ? row_map[i] : i, s = seg[src].  NCH = 8-element chunks per
// lane.  Up to two problems (image and text streams) share one launch.
struct RmsProb {
  const void* x;
  const int32_t* row_map;
  const int32_t* seg;
  const float* mod;
  void* y;
  int64_t n_rows, mod_stride, shift_off, scale_off;
};
struct RmsBatch {
  RmsProb p[2];
  int64_t split;     // rows of problem 0
  int64_t bsplit;    // blocks of problem 0 (= ceil(split / kRmsRows))
  int32_t H;
  float eps;
};

// A block of 4 waves handles 4 consecutive rows of one problem, one row per
// wave; each wave reads its row's (scale, shift) float32 vectors straight
// from memory (a sample's vectors stay in L2 across its rows).  Staging them
// once per block in LDS was measured slower at the 1024^2 pack (8 rows per
// block with staging: 25.8 us; 4 rows without: 23.1 us for 8,704 x 3,072).
constexpr int kRmsRows = 4;

template <typename T, int NCH>
__global__ void __launch_bounds__(64 * kRmsRows) rms_modulate_kernel(RmsBatch bt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t blk = blockIdx.x;
  const bool second = blk >= bt.bsplit;
  const RmsProb& P = second ? bt.p[1] : bt.p[0];
  if (second) blk -= bt.bsplit;
  const int64_t i = blk * kRmsRows + wave;
  if (i >= P.n_rows) return;
  const int H = bt.H;
  const int nch = H >> 3;
  const T* x = static_cast<const T*>(P.x);
  T* y = static_cast<T*>(P.y);
  const int64_t src = P.row_map ? (int64_t)P.row_map[i] : i;
  float v[NCH][8];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) Vec8<T>::load(x + src * H + c * 8, v[j]);
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
    }
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + bt.eps);
  const float* mrow = P.mod + (int64_t)P.seg[src] * P.mod_stride;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
      float sc1[8], sh[8], o[8];
      Vec8<float>::load(mrow + P.shift_off + c * 8, sh);
      Vec8<float>::load(mrow + P.scale_off + c * 8, sc1);
#pragma unroll
      for (int e = 0; e < 8; ++e) sc1[e] = 1.0f + sc1[e];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = v[j][e] * r * sc1[e] + sh[e];
      Vec8<T>::store(y + i * H + c * 8, o);
    }
  }
}

template <typename T>
mmdit_status launch_rms(RmsBatch& bt, int64_t total, hipStream_t s) {
  bt.bsplit = cdiv(bt.split, kRmsRows);
  const int64_t blocks = bt.bsplit + cdiv(total - bt.split, kRmsRows);
  dim3 g((unsigned)blocks), b(64 * kRmsRows);
  const size_t shm = 0;
  const int nch = bt.H / 8;
  if (nch <= 64)
    MMDIT_LAUNCH((rms_modulate_kernel<T, 1>), g, b, shm, s, bt);
  else if (nch <= 128)
    MMDIT_LAUNCH((rms_modulate_kernel<T, 2>), g, b, shm, s, bt);
  else if (nch <= 256)
    MMDIT_LAUNCH((rms_modulate_kernel<T, 4>), g, b, shm, s, bt);
  else if (nch <= 384)
    MMDIT_LAUNCH((rms_modulate_kernel<T, 6>), g, b, shm, s, bt);
  else
    MMDIT_LAUNCH((rms_modulate_kernel<T, 16>), g, b, shm, s, bt);
  return launch_check("rms_modulate_kernel", s);
}

// ------------------------------------------------------ QK-RMSNorm + RoPE
// Lane layout: D/8 lanes per head vector, 8 consecutive dims (4 rotation
// pairs) per lane, 64/(D/8) head vectors per wave step; q heads then k heads.
typedef RopeTable RopeTab;

struct QkProb {
  void* qkv;
  const int32_t* pos;   // NULL: no rotation (text rows)
  const float* g_q;
  const float* g_k;
  int64_t n_rows;
};
struct QkBatch {
  QkProb p[2];
  int64_t split;
  int32_t heads;
  float eps;
};

template <typename T, int D>
__global__ void __launch_bounds__(256) qk_norm_rope_kernel(QkBatch bt, RopeTab tab) {
  constexpr int LPH = D / 8;      // lanes per head vector
  constexpr int HPS = 64 / LPH;   // head vectors per wave step
  const int lane = threadIdx.x & 63;
  int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const QkProb& P = row < bt.split ? bt.p[0] : bt.p[1];
  if (row >= bt.split) row -= bt.split;
  if (row >= P.n_rows) return;
  const int heads = bt.heads;
  const int32_t* pos = P.pos;
  const int sub = lane % LPH;
  const int hv0 = lane / LPH;
  float cs[4], sn[4];
  if (pos) {
    const int32_t p3[3] = {pos[3 * row], pos[3 * row + 1], pos[3 * row + 2]};
    int ax[4];
    float invf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ax[j] = tab.axis[sub * 4 + j];
      invf[j] = tab.inv_freq[sub * 4 + j];
    }
    qk_sincos4(p3, ax, invf, cs, sn);
  }
  float gq[8], gk[8];
  Vec8<float>::load(P.g_q + sub * 8, gq);
  Vec8<float>::load(P.g_k + sub * 8, gk);
  const int64_t H3 = 3 * (int64_t)heads * D;
  T* base = static_cast<T*>(P.qkv) + row * H3 + sub * 8;
  for (int hv = hv0; hv < 2 * heads; hv += HPS) {
    float v[8];
    Vec8<T>::load(base + hv * D, v);
    const float ss = qk_head_sum(qk_sumsq8(v), LPH);
    const float r = qk_inv_rms(ss, (float)D, bt.eps);
    qk_apply8(v, r, hv < heads ? gq : gk, pos != nullptr, cs, sn);
    Vec8<T>::store(base + hv * D, v);
  }
}

// cos and sin of every rotation pair of every row: out[row][pair] = (cos,
// sin) of pos[row][axis(pair)] * inv_freq(pair), float32, D / 2 pairs per
// row, computed exactly as the QK kernel computes them (qk_sincos4), so a
// consumer of the table rotates with the same values.  One thread per 4 pairs.
__global__ void __launch_bounds__(256) rope_cs_kernel(const int32_t* __restrict__ pos, int64_t n, int32_t D,
                                                      RopeTab tab, float* __restrict__ out) {
  const int32_t qpr = D >> 3;   // 4-pair groups per row
  const int64_t total = n * qpr;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = u / qpr;
    const int sub = (int)(u - row * qpr);
    const int32_t p3[3] = {pos[3 * row], pos[3 * row + 1], pos[3 * row + 2]};
    int ax[4];
    float invf[4], cs[4], sn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ax[j] = tab.axis[sub * 4 + j];
      invf[j] = tab.inv_freq[sub * 4 + j];
    }
    qk_sincos4(p3, ax, invf, cs, sn);
    float* o = out + row * D + sub * 8;
    *reinterpret_cast<f32x4*>(o) = f32x4{cs[0], sn[0], cs[1], sn[1]};
    *reinterpret_cast<f32x4*>(o + 4) = f32x4{cs[2], sn[2], cs[3], sn[3]};
  }
}

template <typename T>
mmdit_status launch_qk(const QkBatch& bt, int64_t total, int32_t D, const RopeTab& tab, hipStream_t s) {
  dim3 g((unsigned)cdiv(total, 4)), b(256);
  if (D == 128)
    MMDIT_LAUNCH((qk_norm_rope_kernel<T, 128>), g, b, 0, s, bt, tab);
  else
    MMDIT_LAUNCH((qk_norm_rope_kernel<T, 64>), g, b, 0, s, bt, tab);
  return launch_check("qk_norm_rope_kernel", s);
}

// ---------------------------------------------------- timestep embedding
// emb[b] = [cos(1000 t f_k), sin(1000 t f_k)], f_k = 10000^(-k/half); double
// precision for the argument (up to 1000 rad) and the trig functions.
template <typename T>
__global__ void temb_kernel(int32_t B, int32_t half, const float* __restrict__ t, T* __restrict__ emb) {
  const int b = blockIdx.x;
  for (int k = threadIdx.x; k < half; k += blockDim.x) {
    const double f = exp(-log(10000.0) * (double)k / (double)half);
    const double a = 1000.0 * (double)t[b] * f;
    emb[(int64_t)b * 2 * half + k] = from_f<T>((float)cos(a));
    emb[(int64_t)b * 2 * half + half + k] = from_f<T>((float)sin(a));
  }
}

}  // namespace

mmdit_status rms_modulate2_impl(mmdit_dtype dt, int32_t H, float eps, const RmsArgs* a, int n, hipStream_t s) {
  if (H % 8 || H > 8192 || H <= 0) {
    set_error("rms_modulate: hidden=%d must be a multiple of 8 and <= 8192", H);
    return MMDIT_E_UNSUPPORTED;
  }
  RmsBatch bt;
  memset(&bt, 0, sizeof(bt));
  int k = 0;
  for (int i = 0; i < n; ++i) {
    if (a[i].n_rows == 0) continue;
    RmsProb& p = bt.p[k++];
    p.x = a[i].x;
    p.row_map = a[i].row_map;
    p.seg = a[i].seg;
    p.mod = a[i].mod;
    p.y = a[i].y;
    p.n_rows = a[i].n_rows;
    p.mod_stride = a[i].mod_stride;
    p.shift_off = a[i].shift_off;
    p.scale_off = a[i].scale_off;
  }
  if (k == 0) return MMDIT_OK;
  bt.split = bt.p[0].n_rows;
  bt.H = H;
  bt.eps = eps;
  const int64_t total = bt.p[0].n_rows + (k > 1 ? bt.p[1].n_rows : 0);
  return dt == MMDIT_BF16 ? launch_rms<bf16>(bt, total, s) : launch_rms<float>(bt, total, s);
}

mmdit_status rms_modulate_impl(mmdit_dtype dt, int64_t n, int32_t H, const void* x,
                               const int32_t* map, const int32_t* seg, const float* mod,
                               int64_t ms, int64_t so, int64_t co, void* y, float eps, hipStream_t s) {
  RmsArgs a = {x, map, seg, mod, y, n, ms, so, co};
  return rms_modulate2_impl(dt, H, eps, &a, 1, s);
}

mmdit_status rope_cs_impl(const int32_t* pos, int64_t n, int32_t D, const RopeTable& tab, float* out,
                          hipStream_t s) {
  if (n == 0) return MMDIT_OK;
  int64_t g = cdiv(n * (D >> 3), 256);
  if (g > 1 << 16) g = 1 << 16;
  MMDIT_LAUNCH(rope_cs_kernel, dim3((unsigned)g), dim3(256), 0, s, pos, n, D, tab, out);
  return launch_check("rope_cs_kernel", s);
}

void rope_table(RopeTable* t, const int32_t* widths, float theta) {
  int p = 0;
  for (int ax = 0; ax < 3; ++ax)
    for (int j = 0; j < widths[ax] / 2 && p < 64; ++j, ++p) {
      t->axis[p] = ax;
      t->inv_freq[p] = (float)pow((double)theta, -2.0 * j / (double)widths[ax]);
    }
  for (; p < 64; ++p) {
    t->axis[p] = 0;
    t->inv_freq[p] = 0.f;
  }
}

mmdit_status qk_norm_rope2_impl(mmdit_dtype dt, int32_t heads, int32_t D, const int32_t* widths, float theta,
                                float eps, const QkArgs* a, int n, hipStream_t s) {
  if (D != 64 && D != 128) {
    set_error("qk_norm_rope: head_dim=%d unsupported (64 or 128)", D);
    return MMDIT_E_UNSUPPORTED;
  }
  QkBatch bt;
  memset(&bt, 0, sizeof(bt));
  int k = 0;
  for (int i = 0; i < n; ++i) {
    if (a[i].n_rows == 0) continue;
    QkProb& p = bt.p[k++];
    p.qkv = a[i].qkv;
    p.pos = a[i].pos;
    p.g_q = a[i].g_q;
    p.g_k = a[i].g_k;
    p.n_rows = a[i].n_rows;
  }
  if (k == 0) return MMDIT_OK;
  bt.split = bt.p[0].n_rows;
  bt.heads = heads;
  bt.eps = eps;
  RopeTab tab;
  rope_table(&tab, widths, theta);
  const int64_t total = bt.p[0].n_rows + (k > 1 ? bt.p[1].n_rows : 0);
  return dt == MMDIT_BF16 ? launch_qk<bf16>(bt, total, D, tab, s) : launch_qk<float>(bt, total, D, tab, s);
}

mmdit_status qk_norm_rope_impl(mmdit_dtype dt, int64_t n, int32_t heads, int32_t D, const int32_t* widths,
                               void* qkv, const int32_t* pos, const float* gq, const float* gk, float theta,
                               float eps, hipStream_t s) {
  QkArgs a = {qkv, pos, gq, gk, n};
  return qk_norm_rope2_impl(dt, heads, D, widths, theta, eps, &a, 1, s);
}

mmdit_status temb_impl(mmdit_dtype dt, int32_t B, int32_t t_dim, const float* t, void* emb,
                       hipStream_t s) {
  if (B == 0) return MMDIT_OK;
  if (dt == MMDIT_BF16)
    MMDIT_LAUNCH(temb_kernel<bf16>, dim3(B), dim3(128), 0, s, B, t_dim / 2, t, (bf16*)emb);
  else
    MMDIT_LAUNCH(temb_kernel<float>, dim3(B), dim3(128), 0, s, B, t_dim / 2, t, (float*)emb);
  return launch_check("temb_kernel", s);
}

}  // namespace mmdit
