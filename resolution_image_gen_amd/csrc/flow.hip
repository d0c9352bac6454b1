// Rectified-flow wrapper kernels: noising, loss, CFG combine + Euler step.
//
// hyper.ai 2607.19064, 方法 (and blog close-reading 2.2(2), same equation):
// z_t = (1 - t) z + t eps and the matching loss || v - (z - eps) ||^2.  Editing
// scores the target latent only.  Sampling integrates the velocity ODE from
// noise to data (blog close-reading, 5); packed CFG combines the cond and
// uncond predictions of one packed forward (hyper.ai 2607.19064, 实验).
// All are HBM-bound streaming kernels over [rows, C] with 16-byte accesses.
#include "common.h"

#include <mutex>

namespace mmdit {

// Scratch of rf_loss_noalloc: the per-row sums of up to kNoAllocMaxRows
// target rows (16 MiB + 16 B of float32 per device, held until the process
// ends).  In host code `scratch` only names the symbol: kernels receive the
// device address that hipGetSymbolAddress returns for the current device.
constexpr int64_t kNoAllocMaxRows = int64_t(1) << 22;
static __device__ __align__(256) float scratch[kNoAllocMaxRows + 4];

namespace {

int grid_for(int64_t work, int threads) {
  int64_t g = cdiv(work, threads);
  if (g < 1) g = 1;
  if (g > 1 << 20) g = 1 << 20;
  return (int)g;
}

// One thread per 8 channels of an image row.
template <typename T>
__global__ void make_xt_kernel(int64_t n_img, int32_t C, const T* __restrict__ z,
                               const T* __restrict__ eps, const float* __restrict__ t,
                               const int32_t* __restrict__ seg, const int32_t* __restrict__ pos,
                               T* __restrict__ zt) {
  const int32_t upr = C >> 3;
  const int64_t n_units = n_img * upr;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = u / upr;
    const int64_t off = row * C + (u - row * upr) * 8;
    float zv[8];
    Vec8<T>::load(z + off, zv);
    if (pos[3 * row] == 0) {  // frame 0: target rows are noised
      const float tb = t[seg[row]];
      float ev[8];
      Vec8<T>::load(eps + off, ev);
#pragma unroll
      for (int i = 0; i < 8; ++i) zv[i] = rf_xt(zv[i], ev[i], tb);
    }
    Vec8<T>::store(zt + off, zv);
  }
}

// Per-target-row sum of squared residuals; 16 lanes per row, 8 channels per
// lane-step; the 16-lane groups stride over the rows with the grid (whose
// size the host caps).
template <typename T>
__global__ void row_sse_kernel(int64_t n_tgt, int32_t C, const T* __restrict__ v,
                               const T* __restrict__ z, const T* __restrict__ eps,
                               const int32_t* __restrict__ tgt_row, float* __restrict__ row_sse) {
  const int lane16 = threadIdx.x & 15;
  const int64_t row0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int64_t rstep = ((int64_t)gridDim.x * blockDim.x) >> 4;
  // every lane of a 16-lane group shares `row`, so the group runs the loop together
  for (int64_t row = row0; row < n_tgt; row += rstep) {
    float acc = 0.f;
    const int64_t src = tgt_row[row];
    for (int c8 = lane16; c8 < (C >> 3); c8 += 16) {
      float vv[8], zv[8], ev[8];
      Vec8<T>::load(v + row * C + c8 * 8, vv);
      Vec8<T>::load(z + src * C + c8 * 8, zv);
      Vec8<T>::load(eps + src * C + c8 * 8, ev);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = rf_sq_acc(vv[i], zv[i], ev[i], acc);
    }
    acc = group_sum(acc, 16);
    if (lane16 == 0) row_sse[row] = acc;
  }
}

// Per-target-row value of the negative-aware loss (blog close-reading,
// 2.2(4), the Diffusion-NFT objective): r_b ||v+ - (z - eps)||^2 +
// (1 - r_b) ||v- - (z - eps)||^2 over the row, r_b the reward of the row's
// sample.  The same lane layout and summation order as row_sse_kernel, so
// r_b = 1 gives exactly row_sse_kernel's value for v = v+.
template <typename T>
__global__ void row_nft_kernel(int64_t n_tgt, int32_t C, const T* __restrict__ vp, const T* __restrict__ vn,
                               const T* __restrict__ z, const T* __restrict__ eps, const float* __restrict__ r,
                               const int32_t* __restrict__ seg, const int32_t* __restrict__ tgt_row,
                               float* __restrict__ row_val) {
  const int lane16 = threadIdx.x & 15;
  const int64_t row0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int64_t rstep = ((int64_t)gridDim.x * blockDim.x) >> 4;
  for (int64_t row = row0; row < n_tgt; row += rstep) {
    float ap = 0.f, an = 0.f;
    const int64_t src = tgt_row[row];
    for (int c8 = lane16; c8 < (C >> 3); c8 += 16) {
      float pv[8], nv[8], zv[8], ev[8];
      Vec8<T>::load(vp + row * C + c8 * 8, pv);
      Vec8<T>::load(vn + row * C + c8 * 8, nv);
      Vec8<T>::load(z + src * C + c8 * 8, zv);
      Vec8<T>::load(eps + src * C + c8 * 8, ev);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ap = rf_sq_acc(pv[i], zv[i], ev[i], ap);
        an = rf_sq_acc(nv[i], zv[i], ev[i], an);
      }
    }
    ap = group_sum(ap, 16);
    an = group_sum(an, 16);
    const float rb = r[seg[src]];
    if (lane16 == 0) row_val[row] = rb * ap + (1.0f - rb) * an;
  }
}

// dL/dv of the loss mean_b SSE_b / (tgt_len_b C): 2 (v - (z - eps)) / (B tgt_len_b C)
// on every target row (one thread per 8 channels).
template <typename T>
__global__ void loss_grad_kernel(int64_t n_tgt, int32_t C, int32_t B, const T* __restrict__ v,
                                 const T* __restrict__ z, const T* __restrict__ eps,
                                 const int32_t* __restrict__ tgt_row, const int32_t* __restrict__ seg,
                                 const int32_t* __restrict__ tgt_len, T* __restrict__ dv) {
  const int32_t upr = C >> 3;
  const int64_t n_units = n_tgt * upr;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = u / upr;
    const int64_t c8 = (u - row * upr) * 8;
    const int64_t src = tgt_row[row];
    const float k = 2.0f / ((float)B * (float)tgt_len[seg[src]] * (float)C);
    float vv[8], zv[8], ev[8];
    Vec8<T>::load(v + row * C + c8, vv);
    Vec8<T>::load(z + src * C + c8, zv);
    Vec8<T>::load(eps + src * C + c8, ev);
#pragma unroll
    for (int i = 0; i < 8; ++i) vv[i] = k * (vv[i] - (zv[i] - ev[i]));
    Vec8<T>::store(dv + row * C + c8, vv);
  }
}

// Target rows from which the loss's per-sample sums take one block per sample.
constexpr int64_t kLossBlocksRows = 131072;

// One block of 16 waves.  Wave w takes samples w, w + 16, ...: its lanes sum
// the sample's rows r0 + lane, r0 + lane + 64, ... and the wave reduces them
// (a fixed order that depends only on the sample's rows, so the result is
// deterministic and independent of the other samples).  Then one thread
// forms the mean loss over the samples in order.
__global__ void __launch_bounds__(1024) loss_finalize_kernel(int32_t B, int32_t C,
                                                             const int32_t* __restrict__ cu_tgt,
                                                             const float* __restrict__ row_sse,
                                                             float* __restrict__ sse,
                                                             float* __restrict__ loss) {
  __shared__ float sh[MMDIT_MAX_SAMPLES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int b = wave; b < B; b += 16) {
    const int32_t r0 = cu_tgt[b], r1 = cu_tgt[b + 1];
    // the 16-byte-aligned middle of the sample's rows as float4, lane-strided,
    // eight loads in flight per lane (eight accumulators, summed in a fixed
    // tree); the up to 3 + 3 rows outside it go to lanes 0..5
    const int32_t a0 = min((r0 + 3) & ~3, r1), a1 = max(r1 & ~3, a0);
    const f32x4* mid = reinterpret_cast<const f32x4*>(row_sse + a0);
    const int32_t nv = (a1 - a0) >> 2;
    f32x4 s8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) s8[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    int32_t j = lane;
    for (; j + 7 * 64 < nv; j += 8 * 64) {
#pragma unroll
      for (int k = 0; k < 8; ++k) s8[k] += mid[j + k * 64];
    }
    for (int k = 0; j < nv; j += 64, ++k) s8[k] += mid[j];
#pragma unroll
    for (int k = 0; k < 4; ++k) s8[k] += s8[k + 4];
    s8[0] += s8[2];
    s8[1] += s8[3];
    s8[0] += s8[1];
    float acc = (s8[0][0] + s8[0][1]) + (s8[0][2] + s8[0][3]);
    if (lane < 3 && r0 + lane < a0) acc += row_sse[r0 + lane];
    if (lane >= 3 && lane < 6 && a1 + lane - 3 < r1) acc += row_sse[a1 + lane - 3];
    acc = wave_sum(acc);
    if (lane == 0) {
      sse[b] = acc;
      sh[b] = acc;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float total = 0.f;
    for (int b = 0; b < B; ++b)
      total += sh[b] / ((float)(cu_tgt[b + 1] - cu_tgt[b]) * (float)C);
    loss[0] = B > 0 ? total / (float)B : 0.f;
  }
}

// For large packs (from kLossBlocksRows target rows) the per-sample sums
// instead take one block of 256 threads per sample (blockIdx.x), so the
// reduction spreads over the CUs (one wave per sample reads a few hundred
// GB/s at most).  The
// 16-byte-aligned middle of the sample's rows is read as float4, thread t
// taking j = t, t + 256, ... with four loads in flight (four accumulators,
// summed in a fixed tree); the up to 3 + 3 rows outside it go to threads
// 0..5; each wave reduces its threads, then thread 0 adds the four waves in
// order.  The order depends only on the sample's rows, so the result is
// deterministic and independent of the other samples.
__global__ void __launch_bounds__(256) loss_sample_sums_kernel(const int32_t* __restrict__ cu_tgt,
                                                               const float* __restrict__ row_val,
                                                               float* __restrict__ sse) {
  __shared__ float wsum[4];
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int32_t r0 = cu_tgt[b], r1 = cu_tgt[b + 1];
  const int32_t a0 = min((r0 + 3) & ~3, r1), a1 = max(r1 & ~3, a0);
  const f32x4* mid = reinterpret_cast<const f32x4*>(row_val + a0);
  const int32_t nv = (a1 - a0) >> 2;
  f32x4 s4[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) s4[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  int32_t j = t;
  for (; j + 3 * 256 < nv; j += 4 * 256) {
#pragma unroll
    for (int k = 0; k < 4; ++k) s4[k] += mid[j + k * 256];
  }
  for (int k = 0; j < nv; j += 256, ++k) s4[k] += mid[j];
  s4[0] += s4[2];
  s4[1] += s4[3];
  s4[0] += s4[1];
  float acc = (s4[0][0] + s4[0][1]) + (s4[0][2] + s4[0][3]);
  if (t < 3 && r0 + t < a0) acc += row_val[r0 + t];
  if (t >= 3 && t < 6 && a1 + t - 3 < r1) acc += row_val[a1 + t - 3];
  acc = wave_sum(acc);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (t == 0) sse[b] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// The mean loss over the samples, in sample order: one thread.
__global__ void loss_mean_kernel(int32_t B, int32_t C, const int32_t* __restrict__ cu_tgt,
                                 const float* __restrict__ sse, float* __restrict__ loss) {
  if (threadIdx.x != 0) return;
  float total = 0.f;
  for (int b = 0; b < B; ++b) total += sse[b] / ((float)(cu_tgt[b + 1] - cu_tgt[b]) * (float)C);
  loss[0] = B > 0 ? total / (float)B : 0.f;
}

// z (float32 [n, C]) += dt * (v_u + g (v_c - v_u)); optionally writes z into two target row ranges.
template <typename T>
__global__ void euler_kernel(int64_t n, int32_t C, const T* __restrict__ v_c,
                             const T* __restrict__ v_u, float g, float dt, float* __restrict__ z,
                             T* __restrict__ zt_a, T* __restrict__ zt_b) {
  const int64_t n_units = n * (C >> 3);
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t off = u * 8;
    float vc[8], zz[8];
    Vec8<T>::load(v_c + off, vc);
    Vec8<float>::load(z + off, zz);
    if (v_u) {
      float vu[8];
      Vec8<T>::load(v_u + off, vu);
#pragma unroll
      for (int i = 0; i < 8; ++i) zz[i] += dt * (vu[i] + g * (vc[i] - vu[i]));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) zz[i] += dt * vc[i];
    }
    Vec8<float>::store(z + off, zz);
    if (zt_a) Vec8<T>::store(zt_a + off, zz);
    if (zt_b) Vec8<T>::store(zt_b + off, zz);
  }
}

template <typename T>
__global__ void pack_latent_kernel(int64_t n, int32_t C, const float* __restrict__ z,
                                   T* __restrict__ zt_a, T* __restrict__ zt_b) {
  const int64_t n_units = n * (C >> 3);
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units;
       u += (int64_t)gridDim.x * blockDim.x) {
    float zz[8];
    Vec8<float>::load(z + u * 8, zz);
    Vec8<T>::store(zt_a + u * 8, zz);
    if (zt_b) Vec8<T>::store(zt_b + u * 8, zz);
  }
}

mmdit_status check_pack(const mmdit_pack_t* pk, const char* who) {
  if (!pk || pk->B < 0 || pk->B > MMDIT_MAX_SAMPLES || pk->n_img < 0 || pk->n_txt < 0 ||
      pk->n_tgt < 0 || pk->h_cu_img[pk->B] != pk->n_img || pk->h_cu_txt[pk->B] != pk->n_txt ||
      pk->h_cu_tgt[pk->B] != pk->n_tgt) {
    set_error("%s: pack is invalid or was not built by mmdit_pack", who);
    return MMDIT_E_INVALID;
  }
  return MMDIT_OK;
}

mmdit_status check_c(int32_t C, const char* who) {
  if (C <= 0 || C % 8) {
    set_error("%s: C=%d must be a positive multiple of 8", who, C);
    return MMDIT_E_UNSUPPORTED;
  }
  return MMDIT_OK;
}

}  // namespace

mmdit_status make_xt_impl(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* z,
                          const void* eps, const float* t, void* zt, hipStream_t s) {
  MMDIT_TRY(check_pack(pk, "rf_make_xt"));
  MMDIT_TRY(check_c(C, "rf_make_xt"));
  if (pk->n_img == 0) return MMDIT_OK;
  if (!z || !eps || !t || !zt || !pk->seg_img || !pk->pos_img) {
    set_error("rf_make_xt: NULL pointer");
    return MMDIT_E_INVALID;
  }
  int g = grid_for(pk->n_img * (C / 8), 256);
  if (dt == MMDIT_BF16)
    MMDIT_LAUNCH(make_xt_kernel<bf16>, dim3(g), dim3(256), 0, s, pk->n_img, C,
                       (const bf16*)z, (const bf16*)eps, t, pk->seg_img, pk->pos_img, (bf16*)zt);
  else
    MMDIT_LAUNCH(make_xt_kernel<float>, dim3(g), dim3(256), 0, s, pk->n_img, C,
                       (const float*)z, (const float*)eps, t, pk->seg_img, pk->pos_img, (float*)zt);
  return launch_check("make_xt_kernel", s);
}

mmdit_status loss_grad_impl(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* v, const void* z,
                            const void* eps, void* dv, hipStream_t s) {
  MMDIT_TRY(check_pack(pk, "rf_loss_grad"));
  MMDIT_TRY(check_c(C, "rf_loss_grad"));
  if (pk->n_tgt == 0) return MMDIT_OK;
  if (!v || !z || !eps || !dv || !pk->tgt_row || !pk->tgt_len) {
    set_error("rf_loss_grad: NULL pointer");
    return MMDIT_E_INVALID;
  }
  const int g = grid_for(pk->n_tgt * (C >> 3), 256);
  if (dt == MMDIT_BF16)
    MMDIT_LAUNCH(loss_grad_kernel<bf16>, dim3(g), dim3(256), 0, s, pk->n_tgt, C, pk->B, (const bf16*)v,
                 (const bf16*)z, (const bf16*)eps, pk->tgt_row, pk->seg_img, pk->tgt_len, (bf16*)dv);
  else
    MMDIT_LAUNCH(loss_grad_kernel<float>, dim3(g), dim3(256), 0, s, pk->n_tgt, C, pk->B, (const float*)v,
                 (const float*)z, (const float*)eps, pk->tgt_row, pk->seg_img, pk->tgt_len, (float*)dv);
  return launch_check("loss_grad_kernel", s);
}

mmdit_status row_sse_impl(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* v, const void* z,
                          const void* eps, float* row_sse, hipStream_t s) {
  if (pk->n_tgt == 0) return MMDIT_OK;
  const int g = grid_for(pk->n_tgt * 16, 256);
  if (dt == MMDIT_BF16)
    MMDIT_LAUNCH(row_sse_kernel<bf16>, dim3(g), dim3(256), 0, s, pk->n_tgt, C, (const bf16*)v, (const bf16*)z,
                 (const bf16*)eps, pk->tgt_row, row_sse);
  else
    MMDIT_LAUNCH(row_sse_kernel<float>, dim3(g), dim3(256), 0, s, pk->n_tgt, C, (const float*)v, (const float*)z,
                 (const float*)eps, pk->tgt_row, row_sse);
  return launch_check("row_sse_kernel", s);
}

mmdit_status loss_finalize_impl(const mmdit_pack_t* pk, int32_t C, const float* row_sse, float* sse, float* loss,
                                hipStream_t s) {
  // a function of the pack's size only, so every call on a pack takes the
  // same reduction order
  if (pk->n_tgt < kLossBlocksRows) {
    MMDIT_LAUNCH(loss_finalize_kernel, dim3(1), dim3(1024), 0, s, pk->B, C, pk->cu_tgt, row_sse, sse, loss);
    return launch_check("loss_finalize_kernel", s);
  }
  if (pk->B > 0) {
    MMDIT_LAUNCH(loss_sample_sums_kernel, dim3((unsigned)pk->B), dim3(256), 0, s, pk->cu_tgt, row_sse, sse);
    MMDIT_TRY(launch_check("loss_sample_sums_kernel", s));
  }
  MMDIT_LAUNCH(loss_mean_kernel, dim3(1), dim3(64), 0, s, pk->B, C, pk->cu_tgt, sse, loss);
  return launch_check("loss_mean_kernel", s);
}

mmdit_status loss_impl(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* v,
                       const void* z, const void* eps, float* sse, float* loss, void* ws,
                       size_t ws_bytes, hipStream_t s) {
  MMDIT_TRY(check_pack(pk, "rf_loss"));
  MMDIT_TRY(check_c(C, "rf_loss"));
  if (!sse && pk->B > 0) {
    set_error("rf_loss: sse is NULL");
    return MMDIT_E_INVALID;
  }
  if (!loss || (pk->n_tgt > 0 && (!v || !z || !eps || !pk->tgt_row))) {
    set_error("rf_loss: NULL pointer");
    return MMDIT_E_INVALID;
  }
  if (!ws || ws_bytes < (size_t)pk->n_tgt * 4 + 4) {
    set_error("rf_loss: workspace needs %zu bytes, got %zu", (size_t)pk->n_tgt * 4 + 4, ws_bytes);
    return MMDIT_E_WORKSPACE;
  }
  if (((uintptr_t)ws & 15) != 0) {
    set_error("rf_loss: workspace is not 16-byte aligned");
    return MMDIT_E_UNSUPPORTED;
  }
  float* row_sse = static_cast<float*>(ws);
  MMDIT_TRY(row_sse_impl(pk, dt, C, v, z, eps, row_sse, s));
  return loss_finalize_impl(pk, C, row_sse, sse, loss, s);
}

mmdit_status nft_loss_impl(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* vp, const void* vn,
                           const void* z, const void* eps, const float* r, float* sse, float* loss, void* ws,
                           size_t ws_bytes, hipStream_t s) {
  MMDIT_TRY(check_pack(pk, "rf_nft_loss"));
  MMDIT_TRY(check_c(C, "rf_nft_loss"));
  if (!sse && pk->B > 0) {
    set_error("rf_nft_loss: sse is NULL");
    return MMDIT_E_INVALID;
  }
  if (!loss || (pk->n_tgt > 0 && (!vp || !vn || !z || !eps || !r || !pk->tgt_row || !pk->seg_img))) {
    set_error("rf_nft_loss: NULL pointer");
    return MMDIT_E_INVALID;
  }
  if (!ws || ws_bytes < (size_t)pk->n_tgt * 4 + 4) {
    set_error("rf_nft_loss: workspace needs %zu bytes, got %zu", (size_t)pk->n_tgt * 4 + 4, ws_bytes);
    return MMDIT_E_WORKSPACE;
  }
  if (((uintptr_t)ws & 15) != 0) {
    set_error("rf_nft_loss: workspace is not 16-byte aligned");
    return MMDIT_E_UNSUPPORTED;
  }
  float* row_val = static_cast<float*>(ws);
  if (pk->n_tgt > 0) {
    int g = grid_for(pk->n_tgt * 16, 256);
    if (dt == MMDIT_BF16)
      MMDIT_LAUNCH(row_nft_kernel<bf16>, dim3(g), dim3(256), 0, s, pk->n_tgt, C, (const bf16*)vp, (const bf16*)vn,
                   (const bf16*)z, (const bf16*)eps, r, pk->seg_img, pk->tgt_row, row_val);
    else
      MMDIT_LAUNCH(row_nft_kernel<float>, dim3(g), dim3(256), 0, s, pk->n_tgt, C, (const float*)vp,
                   (const float*)vn, (const float*)z, (const float*)eps, r, pk->seg_img, pk->tgt_row, row_val);
    MMDIT_TRY(launch_check("row_nft_kernel", s));
  }
  return loss_finalize_impl(pk, C, row_val, sse, loss, s);
}

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];   // device address of `scratch` per device
}  // namespace

// The current device's address of `scratch`, looked up once per device (with
// that device current) and kept.
static mmdit_status scratch_address(void** out, const char* who) {
  int dev = -1;
  MMDIT_TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kScratchDevices) {
    set_error("%s: device %d beyond the %d devices the scratch table holds", who, dev, kScratchDevices);
    return MMDIT_E_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    MMDIT_TRY(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!p) {
      set_error("%s: hipGetSymbolAddress returned NULL for the scratch array", who);
      return MMDIT_E_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MMDIT_OK;
}

mmdit_status loss_noalloc_impl(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* v, const void* z,
                               const void* eps, float* sse, float* loss, hipStream_t s) {
  MMDIT_TRY(check_pack(pk, "rf_loss_noalloc"));
  if (pk->n_tgt > kNoAllocMaxRows) {
    set_error("rf_loss_noalloc: %lld target rows exceed the scratch limit of %lld rows (use rf_loss with a "
              "workspace)", (long long)pk->n_tgt, (long long)kNoAllocMaxRows);
    return MMDIT_E_UNSUPPORTED;
  }
  void* ws = nullptr;
  MMDIT_TRY(scratch_address(&ws, "rf_loss_noalloc"));
  // every row sum the reduction reads is written by this call first, so the
  // previous call's contents need no clearing
  return loss_impl(pk, dt, C, v, z, eps, sse, loss, ws, (size_t)(kNoAllocMaxRows + 4) * sizeof(float), s);
}

static mmdit_status check_target_sample(const mmdit_pack_t* pk, int32_t b, const char* who) {
  if (b < 0 || b >= pk->B) {
    set_error("%s: sample index %d out of range [0, %d)", who, b, pk->B);
    return MMDIT_E_INVALID;
  }
  return MMDIT_OK;
}

mmdit_status euler_impl(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* v,
                        int32_t cb, int32_t ub, float g, float t_cur, float t_next, float* z,
                        void* zt_next, hipStream_t s) {
  MMDIT_TRY(check_pack(pk, "rf_euler_step"));
  MMDIT_TRY(check_c(C, "rf_euler_step"));
  MMDIT_TRY(check_target_sample(pk, cb, "rf_euler_step"));
  const int64_t n = pk->h_cu_tgt[cb + 1] - pk->h_cu_tgt[cb];
  if (ub >= 0) {
    MMDIT_TRY(check_target_sample(pk, ub, "rf_euler_step"));
    if (pk->h_cu_tgt[ub + 1] - pk->h_cu_tgt[ub] != n) {
      set_error("rf_euler_step: cond and uncond samples have different target sizes");
      return MMDIT_E_INVALID;
    }
  }
  if (!v || !z) {
    set_error("rf_euler_step: NULL pointer");
    return MMDIT_E_INVALID;
  }
  const size_t es = dt == MMDIT_BF16 ? 2 : 4;
  const char* vb = static_cast<const char*>(v);
  const void* vc = vb + (size_t)pk->h_cu_tgt[cb] * C * es;
  const void* vu = ub >= 0 ? vb + (size_t)pk->h_cu_tgt[ub] * C * es : nullptr;
  // target rows of sample b are the first h*w image rows of the sample
  char* ztb = static_cast<char*>(zt_next);
  void* za = zt_next ? ztb + (size_t)pk->h_cu_img[cb] * C * es : nullptr;
  void* zb = (zt_next && ub >= 0) ? ztb + (size_t)pk->h_cu_img[ub] * C * es : nullptr;
  const float dtv = t_cur - t_next;
  if (n == 0) return MMDIT_OK;
  int gr = grid_for(n * (C / 8), 256);
  if (dt == MMDIT_BF16)
    MMDIT_LAUNCH(euler_kernel<bf16>, dim3(gr), dim3(256), 0, s, n, C, (const bf16*)vc,
                       (const bf16*)vu, g, dtv, z, (bf16*)za, (bf16*)zb);
  else
    MMDIT_LAUNCH(euler_kernel<float>, dim3(gr), dim3(256), 0, s, n, C, (const float*)vc,
                       (const float*)vu, g, dtv, z, (float*)za, (float*)zb);
  return launch_check("euler_kernel", s);
}

mmdit_status pack_latent_impl(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const float* z,
                              int32_t b0, int32_t b1, void* zt, hipStream_t s) {
  MMDIT_TRY(check_pack(pk, "rf_pack_latent"));
  MMDIT_TRY(check_c(C, "rf_pack_latent"));
  MMDIT_TRY(check_target_sample(pk, b0, "rf_pack_latent"));
  const int64_t n = pk->h_cu_tgt[b0 + 1] - pk->h_cu_tgt[b0];
  if (b1 >= 0) {
    MMDIT_TRY(check_target_sample(pk, b1, "rf_pack_latent"));
    if (pk->h_cu_tgt[b1 + 1] - pk->h_cu_tgt[b1] != n) {
      set_error("rf_pack_latent: samples have different target sizes");
      return MMDIT_E_INVALID;
    }
  }
  if (!z || !zt) {
    set_error("rf_pack_latent: NULL pointer");
    return MMDIT_E_INVALID;
  }
  const size_t es = dt == MMDIT_BF16 ? 2 : 4;
  char* ztb = static_cast<char*>(zt);
  void* za = ztb + (size_t)pk->h_cu_img[b0] * C * es;
  void* zb = b1 >= 0 ? ztb + (size_t)pk->h_cu_img[b1] * C * es : nullptr;
  if (n == 0) return MMDIT_OK;
  int gr = grid_for(n * (C / 8), 256);
  if (dt == MMDIT_BF16)
    MMDIT_LAUNCH(pack_latent_kernel<bf16>, dim3(gr), dim3(256), 0, s, n, C, z, (bf16*)za,
                       (bf16*)zb);
  else
    MMDIT_LAUNCH(pack_latent_kernel<float>, dim3(gr), dim3(256), 0, s, n, C, z, (float*)za,
                       (float*)zb);
  return launch_check("pack_latent_kernel", s);
}

}  // namespace mmdit
