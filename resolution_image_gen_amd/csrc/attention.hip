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
// attn_simt_kernel (float32, or any head_dim): 64 queries per block, four
// lanes per query, per-key online softmax.
#include "common.h"

#include <math.h>

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
};

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
}

// ------------------------------------------------------------------- MFMA
template <int D>
__device__ __forceinline__ int kswz(int key) {
  // K rows are D bf16 = D/8 chunks of 16 B; chunk c of key r stored at c ^ kswz(r)
  if constexpr (D == 128) return key & 15;
  else return (key ^ (key >> 3)) & 7;
}

template <int D>
__global__ void __launch_bounds__(256) attn_mfma_kernel(AttnArgs a) {
  constexpr int BKV = 64;
  constexpr int DCH = D / 8;             // 16-B chunks per K/V row
  constexpr int KPT = BKV * DCH / 256;   // keys staged per thread (consecutive)
  constexpr int VLD = BKV + 4;           // padded row of V^T in LDS (bf16)
  constexpr int DT = D / 32;             // 32-wide d tiles of O^T
  constexpr int QS = D / 16;             // 16-deep k steps of S^T
  __shared__ __attribute__((aligned(16))) bf16 Ks[BKV * D];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * VLD];

  const int b = blockIdx.z, head = blockIdx.y;
  const int32_t t0 = a.cu_txt[b], i0 = a.cu_img[b];
  const int32_t Tb = a.cu_txt[b + 1] - t0;
  const int32_t L = Tb + a.cu_img[b + 1] - i0;
  const int32_t qbase = blockIdx.x * 128;
  if (qbase >= L) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  // this lane's query (column of S^T and O^T)
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
  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[t][v] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  // staging map: chunk ch of keys kg*KPT .. kg*KPT + KPT-1
  const int ch = tid % DCH, kg = tid / DCH;
  for (int32_t kv0 = 0; kv0 < L; kv0 += BKV) {
    bf16x8 kr[KPT], vr[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int32_t key = kv0 + kg * KPT + i;
      if (key < L) {
        const bf16* p = joint_row<bf16>(a, key, Tb, t0, i0) + head * D + ch * 8;
        kr[i] = *reinterpret_cast<const bf16x8*>(p + a.H);
        vr[i] = *reinterpret_cast<const bf16x8*>(p + 2 * a.H);
      } else {
        kr[i] = bf16x8{};
        vr[i] = bf16x8{};
      }
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int r = kg * KPT + i;
      *reinterpret_cast<bf16x8*>(Ks + r * D + ((ch ^ kswz<D>(r)) << 3)) = kr[i];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (KPT == 4) {
        bf16x4 t = {vr[0][e], vr[1][e], vr[2][e], vr[3][e]};
        *reinterpret_cast<bf16x4*>(Vt + (ch * 8 + e) * VLD + kg * 4) = t;
      } else {
#pragma unroll
        for (int i = 0; i < KPT; ++i) Vt[(ch * 8 + e) * VLD + kg * KPT + i] = vr[i][e];
      }
    }
    __syncthreads();

    // S^T[key][query] for two 32-key tiles
    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) st[kt][v] = 0.f;
      const int r = kt * 32 + l32;
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + r * D + (((s * 2 + g) ^ kswz<D>(r)) << 3));
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[kt], 0, 0, 0);
      }
    }
    // online softmax over this lane's 32 keys (+ the other half's 32 via one exchange)
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int32_t key = kv0 + kt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        const float x = key < L ? st[kt][v] * a.scale_log2 : -INFINITY;
        st[kt][v] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float corr = exp2f(m - mn);
    m = mn;
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = exp2f(st[kt][v] - mn);
        st[kt][v] = p;
        ps += p;
      }
    lsum = lsum * corr + ps;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[t][v] *= corr;
    // O^T[d][query] += V^T[d][keys] P^T[keys][query], 16 keys per step.  Lane
    // supplies keys {16ks + 4g + 0..3, 16ks + 8 + 4g + 0..3}: the P registers
    // 8*(ks%2) .. +7 of tile ks/2, and the matching V^T entries.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 pf;
#pragma unroll
      for (int u = 0; u < 8; ++u) pf[u] = (bf16)st[ks >> 1][8 * (ks & 1) + u];
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16* vp = Vt + (t * 32 + l32) * VLD + ks * 16 + 4 * g;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vp);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vp + 8);
        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  lsum += __shfl_xor(lsum, 32, 64);
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

}  // namespace

mmdit_status attention_impl(mmdit_dtype dt, const mmdit_pack_t* pk, int32_t heads, int32_t D,
                            const void* qkv_img, const void* qkv_txt, void* o_img, void* o_txt,
                            hipStream_t s) {
  if (pk->B == 0 || pk->max_joint == 0) return MMDIT_OK;
  AttnArgs a;
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
    dim3 grid((unsigned)cdiv(pk->max_joint, 128), heads, pk->B);
    if (D == 128)
      MMDIT_LAUNCH(attn_mfma_kernel<128>, grid, dim3(256), 0, s, a);
    else
      MMDIT_LAUNCH(attn_mfma_kernel<64>, grid, dim3(256), 0, s, a);
    return launch_check("attn_mfma_kernel", s);
  }
  dim3 grid((unsigned)cdiv(pk->max_joint, 64), heads, pk->B);
  if (D == 128)
    MMDIT_LAUNCH((attn_simt_kernel<float, 128>), grid, dim3(256), 0, s, a);
  else
    MMDIT_LAUNCH((attn_simt_kernel<float, 64>), grid, dim3(256), 0, s, a);
  return launch_check("attn_simt_kernel", s);
}

}  // namespace mmdit
