// Packing: plan on the host, per-row ids and gathers on the device.
//
// Native-resolution packing (hyper.ai 2607.19064, 方法: latent grids flattened
// to variable-length token sequences and packed under a fixed token budget,
// text packed the same way; blog close-reading 2.2(2): cumulative offsets,
// attention kept inside each sample, own 2D RoPE per sample, frame index for
// editing).  Layout: modality-major buffers; image row cu_img[b] + k*h*w +
// r*w + c carries (k, r, c) with k = 0 target, 1 source; text rows carry 0.
#include "common.h"

namespace mmdit {

namespace {

constexpr int kChunk = 64;  // samples per launch (kernel arguments by value)

struct PackChunk {
  int32_t b0, nb;
  int32_t img0[kChunk + 1], txt0[kChunk + 1], tgt0[kChunk + 1];
  int32_t h[kChunk], w[kChunk];
  int32_t write_last;  // write the closing entry cu_*[B]
};

__device__ __forceinline__ int find_sample(const int32_t* off, int nb, int32_t row) {
  // largest b with off[b] <= row (off strictly covers [off[0], off[nb]))
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void pack_ids_kernel(PackChunk ck, int32_t* cu_txt, int32_t* cu_img, int32_t* cu_joint,
                                int32_t* cu_tgt, int32_t* tgt_len, int32_t* seg_img,
                                int32_t* seg_txt, int32_t* pos_img, int32_t* tgt_row) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int nb = ck.nb;
  if (tid <= nb) {
    int i = (int)tid;
    if (i < nb || ck.write_last) {
      int b = ck.b0 + i;
      cu_txt[b] = ck.txt0[i];
      cu_img[b] = ck.img0[i];
      cu_joint[b] = ck.txt0[i] + ck.img0[i];
      cu_tgt[b] = ck.tgt0[i];
      if (i < nb) tgt_len[b] = ck.h[i] * ck.w[i];
    }
  }
  const int32_t n_img = ck.img0[nb] - ck.img0[0];
  const int32_t n_txt = ck.txt0[nb] - ck.txt0[0];
  for (int64_t r = tid; r < (int64_t)n_img + n_txt; r += stride) {
    if (r < n_img) {
      int32_t row = ck.img0[0] + (int32_t)r;
      int b = find_sample(ck.img0, nb, row);
      int32_t local = row - ck.img0[b];
      int32_t hw = ck.h[b] * ck.w[b];
      int32_t k = local / hw, rem = local - k * hw;
      int32_t rr = rem / ck.w[b], cc = rem - rr * ck.w[b];
      seg_img[row] = ck.b0 + b;
      pos_img[3 * (int64_t)row + 0] = k;
      pos_img[3 * (int64_t)row + 1] = rr;
      pos_img[3 * (int64_t)row + 2] = cc;
      if (k == 0) tgt_row[ck.tgt0[b] + local] = row;
    } else {
      int32_t row = ck.txt0[0] + (int32_t)(r - n_img);
      seg_txt[row] = ck.b0 + find_sample(ck.txt0, nb, row);
    }
  }
}

struct GatherChunk {
  int32_t nb;
  int32_t dst0[kChunk + 1];
  const uint8_t* src[kChunk];
};

// Copies 16-byte units; row_bytes % 16 == 0.  A sample's rows are contiguous
// in its source and in the packed buffer, so each sample is one flat copy:
// blockIdx.y picks the sample (a uniform index into the argument block), the
// x blocks stride over its units (no per-unit search or division).
__global__ void __launch_bounds__(256) gather_kernel(GatherChunk ck, int32_t row_bytes, uint8_t* dst) {
  const int b = blockIdx.y;
  const int64_t n_units = (int64_t)(ck.dst0[b + 1] - ck.dst0[b]) * (row_bytes >> 4);
  const u32x4* s = reinterpret_cast<const u32x4*>(ck.src[b]);
  u32x4* d = reinterpret_cast<u32x4*>(dst + (int64_t)ck.dst0[b] * row_bytes);
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units;
       u += (int64_t)gridDim.x * blockDim.x)
    d[u] = s[u];
}

int grid_for(int64_t work, int threads) {
  int64_t g = cdiv(work, threads);
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

}  // namespace

mmdit_status plan_impl(const mmdit_sample* s, int32_t n, int64_t img_budget, int64_t joint_budget,
                       int32_t* n_taken, int64_t* n_img, int64_t* n_txt, int32_t* max_joint) {
  if (n < 0 || (n > 0 && !s) || img_budget <= 0 || joint_budget < 0) {
    set_error("mmdit_pack_plan: invalid arguments (n=%d, img_budget=%lld, joint_budget=%lld)", n,
              (long long)img_budget, (long long)joint_budget);
    return MMDIT_E_INVALID;
  }
  int64_t ti = 0, tt = 0;
  int32_t taken = 0, mj = 0;
  for (int32_t i = 0; i < n && taken < MMDIT_MAX_SAMPLES; ++i) {
    const mmdit_sample& x = s[i];
    if (x.h < 1 || x.w < 1 || (x.frames != 1 && x.frames != 2) || x.txt_len < 0) {
      set_error("mmdit_pack_plan: invalid sample %d (h=%d w=%d frames=%d txt_len=%d)", i, x.h, x.w,
                x.frames, x.txt_len);
      return MMDIT_E_INVALID;
    }
    int64_t img = (int64_t)x.frames * x.h * x.w;
    int64_t joint = img + x.txt_len;
    if (img > img_budget || (joint_budget > 0 && joint > joint_budget)) {
      if (taken == 0) {
        set_error("mmdit_pack_plan: sample %d (%lld image + %d text tokens) exceeds the budget", i,
                  (long long)img, x.txt_len);
        return MMDIT_E_BUDGET;
      }
      break;
    }
    if (ti + img > img_budget) break;
    if (joint_budget > 0 && ti + tt + joint > joint_budget) break;
    ti += img;
    tt += x.txt_len;
    if (joint > mj) mj = (int32_t)joint;
    ++taken;
  }
  if (ti + tt > INT32_MAX) {
    set_error("mmdit_pack_plan: pack exceeds 2^31 tokens");
    return MMDIT_E_UNSUPPORTED;
  }
  if (n_taken) *n_taken = taken;
  if (n_img) *n_img = ti;
  if (n_txt) *n_txt = tt;
  if (max_joint) *max_joint = mj;
  return MMDIT_OK;
}

mmdit_status pack_impl(const mmdit_sample* s, int32_t n, mmdit_pack_t* io, hipStream_t stream) {
  if (!io || n < 0 || n > MMDIT_MAX_SAMPLES || (n > 0 && !s)) {
    set_error("mmdit_pack: invalid arguments (n=%d, max %d)", n, MMDIT_MAX_SAMPLES);
    return MMDIT_E_INVALID;
  }
  int64_t ti = 0, tt = 0, tg = 0;
  int32_t mj = 0;
  io->h_cu_txt[0] = io->h_cu_img[0] = io->h_cu_tgt[0] = 0;
  for (int32_t i = 0; i < n; ++i) {
    const mmdit_sample& x = s[i];
    if (x.h < 1 || x.w < 1 || (x.frames != 1 && x.frames != 2) || x.txt_len < 0) {
      set_error("mmdit_pack: invalid sample %d", i);
      return MMDIT_E_INVALID;
    }
    int64_t img = (int64_t)x.frames * x.h * x.w;
    ti += img;
    tt += x.txt_len;
    tg += (int64_t)x.h * x.w;
    if (ti + tt > INT32_MAX) {
      set_error("mmdit_pack: pack exceeds 2^31 tokens");
      return MMDIT_E_UNSUPPORTED;
    }
    io->h_cu_img[i + 1] = (int32_t)ti;
    io->h_cu_txt[i + 1] = (int32_t)tt;
    io->h_cu_tgt[i + 1] = (int32_t)tg;
    io->h_frames[i] = x.frames;
    if (img + x.txt_len > mj) mj = (int32_t)(img + x.txt_len);
  }
  if (!io->cu_txt || !io->cu_img || !io->cu_joint || !io->cu_tgt || (n > 0 && !io->tgt_len) ||
      (ti > 0 && (!io->seg_img || !io->pos_img || !io->tgt_row)) || (tt > 0 && !io->seg_txt)) {
    set_error("mmdit_pack: a device array pointer of the pack is NULL");
    return MMDIT_E_INVALID;
  }
  io->B = n;
  io->max_joint = mj;
  io->n_img = ti;
  io->n_txt = tt;
  io->n_tgt = tg;
  for (int32_t b0 = 0; b0 < n || (n == 0 && b0 == 0); b0 += kChunk) {
    PackChunk ck;
    ck.b0 = b0;
    ck.nb = n - b0 < kChunk ? n - b0 : kChunk;
    ck.write_last = (b0 + ck.nb == n);
    for (int i = 0; i <= ck.nb; ++i) {
      ck.img0[i] = io->h_cu_img[b0 + i];
      ck.txt0[i] = io->h_cu_txt[b0 + i];
      ck.tgt0[i] = io->h_cu_tgt[b0 + i];
    }
    for (int i = 0; i < ck.nb; ++i) {
      ck.h[i] = s[b0 + i].h;
      ck.w[i] = s[b0 + i].w;
    }
    int64_t rows = (int64_t)(ck.img0[ck.nb] - ck.img0[0]) + (ck.txt0[ck.nb] - ck.txt0[0]) + ck.nb + 1;
    MMDIT_LAUNCH(pack_ids_kernel, dim3(grid_for(rows, 256)), dim3(256), 0, stream, ck,
                       io->cu_txt, io->cu_img, io->cu_joint, io->cu_tgt, io->tgt_len, io->seg_img,
                       io->seg_txt, io->pos_img, io->tgt_row);
    MMDIT_TRY(launch_check("pack_ids_kernel", stream));
    if (n == 0) break;
  }
  return MMDIT_OK;
}

mmdit_status gather_impl(const mmdit_pack_t* pk, int32_t which, const void* const* src,
                         int32_t width, mmdit_dtype dt, void* dst, hipStream_t stream) {
  if (!pk || which < 0 || which > 2 || width <= 0 || width % 8 || !dst || (pk->B > 0 && !src)) {
    set_error("mmdit_pack_gather: invalid arguments (which=%d, width=%d)", which, width);
    return MMDIT_E_INVALID;
  }
  const int32_t* off = which == 0 ? pk->h_cu_img : which == 1 ? pk->h_cu_txt : pk->h_cu_tgt;
  const int32_t row_bytes = width * (dt == MMDIT_BF16 ? 2 : 4);
  for (int32_t b0 = 0; b0 < pk->B; b0 += kChunk) {
    GatherChunk ck;
    ck.nb = pk->B - b0 < kChunk ? pk->B - b0 : kChunk;
    for (int i = 0; i <= ck.nb; ++i) ck.dst0[i] = off[b0 + i];
    for (int i = 0; i < ck.nb; ++i) {
      if (!src[b0 + i] && off[b0 + i + 1] > off[b0 + i]) {
        set_error("mmdit_pack_gather: source pointer of sample %d is NULL", b0 + i);
        return MMDIT_E_INVALID;
      }
      ck.src[i] = static_cast<const uint8_t*>(src[b0 + i]);
    }
    int64_t units = 0;   // the largest sample's 16-byte units
    for (int i = 0; i < ck.nb; ++i) {
      const int64_t u = (int64_t)(ck.dst0[i + 1] - ck.dst0[i]) * (row_bytes / 16);
      units = u > units ? u : units;
    }
    if (units == 0) continue;
    const int gx = grid_for(units, 256) < 1024 ? grid_for(units, 256) : 1024;
    MMDIT_LAUNCH(gather_kernel, dim3(gx, ck.nb), dim3(256), 0, stream, ck, row_bytes,
                 static_cast<uint8_t*>(dst));
    MMDIT_TRY(launch_check("gather_kernel", stream));
  }
  return MMDIT_OK;
}

}  // namespace mmdit
