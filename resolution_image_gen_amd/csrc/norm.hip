// Fused per-token chains of the block: RMSNorm + adaLN modulate, and
// QK-RMSNorm + 3-axis RoPE (blog close-reading 2.2(3): the norm / RoPE /
// gating / residual chains are the memory-bound ones and are fused; 2.2(2) and
// hyper.ai 2607.19064 方法: per-sample 2D RoPE plus a frame axis for editing).
// Both are HBM-bound: one read and one write of every element, statistics in
// registers, one wave per row.
#include "common.h"

#include <math.h>

namespace mmdit {

namespace {

// ------------------------------------------------ RMSNorm + adaLN modulate
// y[i] = x[src] / sqrt(mean(x[src]^2) + eps) * (1 + scale[s]) + shift[s],
// src = row_map ? row_map[i] : i, s = seg[src].  NCH = 8-element chunks per lane.
template <typename T, int NCH>
__global__ void __launch_bounds__(256) rms_modulate_kernel(
    int64_t n_rows, int32_t H, const T* __restrict__ x, const int32_t* __restrict__ row_map,
    const int32_t* __restrict__ seg, const float* __restrict__ mod, int64_t mod_stride,
    int64_t shift_off, int64_t scale_off, T* __restrict__ y, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= n_rows) return;
  const int64_t src = row_map ? (int64_t)row_map[i] : i;
  const int nch = H >> 3;
  float v[NCH][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
      Vec8<T>::load(x + src * H + c * 8, v[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
    }
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  const float* mrow = mod + (int64_t)seg[src] * mod_stride;
  const float* shift = mrow + shift_off;
  const float* scale = mrow + scale_off;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
      float sh[8], sc[8], o[8];
      Vec8<float>::load(shift + c * 8, sh);
      Vec8<float>::load(scale + c * 8, sc);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = v[j][e] * r * (1.0f + sc[e]) + sh[e];
      Vec8<T>::store(y + i * H + c * 8, o);
    }
  }
}

template <typename T>
mmdit_status launch_rms(int64_t n, int32_t H, const void* x, const int32_t* map, const int32_t* seg,
                        const float* mod, int64_t ms, int64_t so, int64_t co, void* y, float eps,
                        hipStream_t s) {
  dim3 g((unsigned)cdiv(n, 4)), b(256);
  const T* xp = static_cast<const T*>(x);
  T* yp = static_cast<T*>(y);
  const int nch = H / 8;
  if (nch <= 64)
    MMDIT_LAUNCH((rms_modulate_kernel<T, 1>), g, b, 0, s, n, H, xp, map, seg, mod, ms, so, co, yp, eps);
  else if (nch <= 128)
    MMDIT_LAUNCH((rms_modulate_kernel<T, 2>), g, b, 0, s, n, H, xp, map, seg, mod, ms, so, co, yp, eps);
  else if (nch <= 256)
    MMDIT_LAUNCH((rms_modulate_kernel<T, 4>), g, b, 0, s, n, H, xp, map, seg, mod, ms, so, co, yp, eps);
  else if (nch <= 384)
    MMDIT_LAUNCH((rms_modulate_kernel<T, 6>), g, b, 0, s, n, H, xp, map, seg, mod, ms, so, co, yp, eps);
  else
    MMDIT_LAUNCH((rms_modulate_kernel<T, 16>), g, b, 0, s, n, H, xp, map, seg, mod, ms, so, co, yp, eps);
  return launch_check("rms_modulate_kernel", s);
}

// ------------------------------------------------------ QK-RMSNorm + RoPE
// Lane layout: D/8 lanes per head vector, 8 consecutive dims (4 rotation
// pairs) per lane, 64/(D/8) head vectors per wave step; q heads then k heads.
struct RopeTab {
  float inv_freq[64];  // per rotation pair: theta^(-2j/width of its band)
  int32_t axis[64];    // 0 frame, 1 row, 2 col
};

template <typename T, int D>
__global__ void __launch_bounds__(256) qk_norm_rope_kernel(int64_t n_rows, int32_t heads,
                                                           T* __restrict__ qkv,
                                                           const int32_t* __restrict__ pos,
                                                           const float* __restrict__ g_q,
                                                           const float* __restrict__ g_k,
                                                           RopeTab tab, float eps) {
  constexpr int LPH = D / 8;      // lanes per head vector
  constexpr int HPS = 64 / LPH;   // head vectors per wave step
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int sub = lane % LPH;
  const int hv0 = lane / LPH;
  float cs[4], sn[4];
  if (pos) {
    const int32_t p3[3] = {pos[3 * row], pos[3 * row + 1], pos[3 * row + 2]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pr = sub * 4 + j;
      const float ang = (float)p3[tab.axis[pr]] * tab.inv_freq[pr];
      sincosf(ang, &sn[j], &cs[j]);
    }
  }
  float gq[8], gk[8];
  Vec8<float>::load(g_q + sub * 8, gq);
  Vec8<float>::load(g_k + sub * 8, gk);
  const int64_t H3 = 3 * (int64_t)heads * D;
  T* base = qkv + row * H3 + sub * 8;
  for (int hv = hv0; hv < 2 * heads; hv += HPS) {
    float v[8];
    Vec8<T>::load(base + hv * D, v);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    ss = group_sum(ss, LPH);
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
    const float* g = hv < heads ? gq : gk;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * r * g[e];
    if (pos) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = v[2 * j], b = v[2 * j + 1];
        v[2 * j] = a * cs[j] - b * sn[j];
        v[2 * j + 1] = a * sn[j] + b * cs[j];
      }
    }
    Vec8<T>::store(base + hv * D, v);
  }
}

template <typename T>
mmdit_status launch_qk(int64_t n, int32_t heads, int32_t D, void* qkv, const int32_t* pos,
                       const float* gq, const float* gk, const RopeTab& tab, float eps, hipStream_t s) {
  dim3 g((unsigned)cdiv(n, 4)), b(256);
  if (D == 128)
    MMDIT_LAUNCH((qk_norm_rope_kernel<T, 128>), g, b, 0, s, n, heads, (T*)qkv, pos, gq, gk, tab, eps);
  else
    MMDIT_LAUNCH((qk_norm_rope_kernel<T, 64>), g, b, 0, s, n, heads, (T*)qkv, pos, gq, gk, tab, eps);
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

mmdit_status rms_modulate_impl(mmdit_dtype dt, int64_t n, int32_t H, const void* x,
                               const int32_t* map, const int32_t* seg, const float* mod,
                               int64_t ms, int64_t so, int64_t co, void* y, float eps, hipStream_t s) {
  if (n == 0) return MMDIT_OK;
  if (H % 8 || H > 8192 || H <= 0) {
    set_error("rms_modulate: hidden=%d must be a multiple of 8 and <= 8192", H);
    return MMDIT_E_UNSUPPORTED;
  }
  return dt == MMDIT_BF16 ? launch_rms<bf16>(n, H, x, map, seg, mod, ms, so, co, y, eps, s)
                          : launch_rms<float>(n, H, x, map, seg, mod, ms, so, co, y, eps, s);
}

mmdit_status qk_norm_rope_impl(mmdit_dtype dt, int64_t n, int32_t heads, int32_t D, void* qkv,
                               const int32_t* pos, const float* gq, const float* gk, float theta,
                               float eps, hipStream_t s) {
  if (n == 0) return MMDIT_OK;
  if (D != 64 && D != 128) {
    set_error("qk_norm_rope: head_dim=%d unsupported (64 or 128)", D);
    return MMDIT_E_UNSUPPORTED;
  }
  // bands (frame, row, col) = (D/4, 3D/8, 3D/8) dims = (D/8, 3D/16, 3D/16) pairs
  RopeTab tab;
  const int widths[3] = {D / 4, 3 * D / 8, 3 * D / 8};
  int p = 0;
  for (int a = 0; a < 3; ++a)
    for (int j = 0; j < widths[a] / 2; ++j, ++p) {
      tab.axis[p] = a;
      tab.inv_freq[p] = (float)pow((double)theta, -2.0 * j / (double)widths[a]);
    }
  for (; p < 64; ++p) {
    tab.axis[p] = 0;
    tab.inv_freq[p] = 0.f;
  }
  return dt == MMDIT_BF16 ? launch_qk<bf16>(n, heads, D, qkv, pos, gq, gk, tab, eps, s)
                          : launch_qk<float>(n, heads, D, qkv, pos, gq, gk, tab, eps, s);
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
