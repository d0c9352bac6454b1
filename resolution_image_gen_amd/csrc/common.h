// Shared device/host helpers of the HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "../../include/mmdit.h"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace mmdit {

// ---------------------------------------------------------------- errors
void set_error(const char* fmt, ...);
mmdit_status hip_check(hipError_t e, const char* what);
// Checks the launch just made (and synchronises the stream when MMDIT_SYNC=1).
mmdit_status launch_check(const char* kernel, hipStream_t s);

// Every kernel launch goes through MMDIT_LAUNCH followed by launch_check(name, stream):
// when kernel timing is enabled the pair brackets the launch with hipEvents.
void timing_begin(hipStream_t s);
#define MMDIT_LAUNCH(kernel, grid, block, shm, stream, ...)                 \
  do {                                                                      \
    ::mmdit::timing_begin(stream);                                          \
    hipLaunchKernelGGL(kernel, grid, block, shm, stream, __VA_ARGS__);      \
  } while (0)

#define MMDIT_TRY(expr)                         \
  do {                                          \
    mmdit_status _st = (expr);                  \
    if (_st != MMDIT_OK) return _st;            \
  } while (0)

// ------------------------------------------------------------ conversions
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// 8-element vector load/store in either storage type, widened to float.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  __device__ __forceinline__ static void load(const bf16* p, float* v) {
    bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
  }
  __device__ __forceinline__ static void store(bf16* p, const float* v) {
    bf16x8 x;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (bf16)v[i];
    *reinterpret_cast<bf16x8*>(p) = x;
  }
};
template <> struct Vec8<float> {
  __device__ __forceinline__ static void load(const float* p, float* v) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  __device__ __forceinline__ static void store(float* p, const float* v) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
    *reinterpret_cast<f32x4*>(p) = a;
    *reinterpret_cast<f32x4*>(p + 4) = b;
  }
};

// Workgroup barrier ordering LDS accesses only: the fences are limited to the
// local address space, so global loads in flight stay in flight across it
// (a plain __syncthreads waits for every outstanding global access too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// --------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// x sigmoid(x) with the hardware reciprocal (v_rcp_f32, 1 ulp) instead of an
// IEEE division (a ten-instruction sequence); 1 + exp(-x) >= 1 is never denormal.
__device__ __forceinline__ float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
// Rectified-flow noising of one element, z_t = (1 - t) z + t eps, with its
// multiply-add written out: the noising kernel and the image embedding's
// fused A staging give the same bits.
__device__ __forceinline__ float rf_xt(float z, float e, float t) { return fmaf(t, e, (1.0f - t) * z); }
// One squared residual of the flow-matching loss added to a sum, written out
// (the loss kernels and the final layer's fused row sums give the same bits).
__device__ __forceinline__ float rf_sq_acc(float v, float z, float e, float acc) {
  const float d = v - (z - e);
  return fmaf(d, d, acc);
}
// GELU in its erf form, 0.5 x (1 + erf(x / sqrt 2)), with erf by Abramowitz &
// Stegun, Handbook of Mathematical Functions, formula 7.1.26: for z >= 0,
// erfc(z) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2), t = 1 / (1 + p z),
// absolute error <= 1.5e-7.  With z = |x| / sqrt 2, 0.5 erfc(z) = Q e where
// Q = t (b1 + t (b2 + ...)), b = a / 2, and e = exp(-x^2 / 2), so
// Phi(x) = 1 - Q e for x >= 0 and Q e below, and
//   GELU(x) = x Phi(x) = max(x, 0) - |x| Q e
// (0.5 x + 0.5 |x| absorbs the sign): no 1 + erf cancellation in the negative
// tail.  The derivative Phi(x) + x phi(x), phi(x) = e / sqrt(2 pi), reuses e:
// one hardware reciprocal (1 ulp; its argument is >= 1) and one exponential.
__device__ __forceinline__ void gelu_qe(float x, float& q, float& e) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(ax, 0.3275911f * 0.70710678118654752f, 1.0f));
  q = t * (0.127414796f + t * (-0.142248368f + t * (0.7107068705f + t * (-0.7265760135f + t * 0.5307027145f))));
  e = __builtin_amdgcn_exp2f(x * (x * -0.72134752044448170f));   // exp(-x^2 / 2)
}
__device__ __forceinline__ float gelu_f(float x) {
  float q, e;
  gelu_qe(x, q, e);
  // max(x, 0) as a clamp to [0, FLT_MAX]: one v_med3 (fmaxf would first quiet x)
  return fmaf(-fabsf(x) * q, e, __builtin_amdgcn_fmed3f(x, 0.0f, 3.402823466e38f));
}
__device__ __forceinline__ float gelu_grad_f(float x) {
  float q, e;
  gelu_qe(x, q, e);
  const float qe = q * e;
  return fmaf(x * 0.39894228040143268f, e, x >= 0.0f ? 1.0f - qe : qe);
}

// QK-RMSNorm + RoPE of the 8 consecutive dimensions (4 rotation pairs) of a
// head vector that one lane holds.  Shared by the QK kernel and the QKV
// projection's epilogue, with every fused multiply-add written out, so the
// two give the same bits.
__device__ __forceinline__ float qk_sumsq8(const float* v) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = fmaf(v[e], v[e], s);
  return s;
}
// Sum of a head's per-lane partial sums over its `lanes` (8 or 16)
// neighbouring lanes, aligned: DPP steps within rows of 16 lanes (pair swap,
// quad swap, half-row mirror, row mirror), one VALU add each.  Every lane of
// the group ends with the same value (each step adds two equal-shaped
// partial sums, and addition commutes).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float qk_head_sum(float v, int lanes) {
  v += dpp_f<0xB1>(v);                   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);                   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);                  // row_half_mirror
  if (lanes > 8) v += dpp_f<0x140>(v);   // row_mirror
  return v;
}
// 1 / sqrt(mean square + eps) from the head's sum of squares over D dims
// (hardware reciprocal square root, 1 ulp).
__device__ __forceinline__ float qk_inv_rms(float ss, float D, float eps) {
  return __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
}
// cos and sin of the 4 pairs' angles pos[axis[j]] * inv_freq[j].
__device__ __forceinline__ void qk_sincos4(const int32_t* p3, const int* axis, const float* invf, float* cs,
                                           float* sn) {
#pragma unroll
  for (int j = 0; j < 4; ++j) sincosf((float)p3[axis[j]] * invf[j], &sn[j], &cs[j]);
}
// v <- rotate(v * r * g) (rot false: no rotation).
__device__ __forceinline__ void qk_apply8(float* v, float r, const float* g, bool rot, const float* cs,
                                          const float* sn) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (v[e] * r) * g[e];
  if (rot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = v[2 * j], b = v[2 * j + 1];
      v[2 * j] = fmaf(a, cs[j], -(b * sn[j]));
      v[2 * j + 1] = fmaf(a, sn[j], b * cs[j]);
    }
  }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------ internal API
// RoPE rotation table: per rotation pair of a head, its axis (0 frame, 1 row,
// 2 col) and frequency theta^(-2j/w) for pair j of a band of width w; bands
// (frame, row, col) of the given widths from dimension 0.
struct RopeTable {
  float inv_freq[64];
  int32_t axis[64];
};
void rope_table(RopeTable* t, const int32_t* widths, float theta);
// out [n][D / 2][2] float32: (cos, sin) of every rotation pair of every row
// at positions pos [n][3], the values the QK kernel rotates by.
mmdit_status rope_cs_impl(const int32_t* pos, int64_t n, int32_t D, const RopeTable& tab, float* out,
                          hipStream_t s);

// QK-RMSNorm + RoPE applied by the QKV projection's epilogue (shared by the
// problems of a grouped launch).
struct QkEpilogue {
  RopeTable tab;
  int32_t heads, D;
  float eps, theta;
  int32_t widths[3];
};

// Dense linear y = op(A) W^T: A [M, K] (row stride lda), W [N, K], fp32 accumulation.
struct LinearArgs {
  int64_t M;
  int32_t N, K;
  const void* A;
  int64_t lda;
  const void* W;
  void* Y;                 // [M, N] (row stride ldy) output or in/out residual
  int64_t ldy;
  int32_t epilogue;        // mmdit_epilogue
  int32_t a_silu;          // apply SiLU to A elements on load
  const float* gate;       // gated residual: gate[seg[m] * gate_stride + n]
  int64_t gate_stride;
  const int32_t* seg;      // [M] sample of each row (gated residual)
  const char* tag;         // kernel-timing name of the launch (NULL: generic name)
  int32_t site;            // 1: MLP down projection (own kernel instantiation for profiling)
  float* partial;          // optional float32 workspace for split-K (single problem)
  int64_t partial_elems;
  void* aux;               // [M, N] dense, model dtype: second output or input of the epilogues below
                           // ([M, 2 H] for kEpiQkRopeAux)
  const int32_t* pos;      // kEpiQkRope*: [M][3] positions of the rows (NULL: text rows, no rotation)
  const float* rope_cs;    // kEpiQkRope*: their (cos, sin) table from rope_cs_impl (NULL iff pos is NULL)
  const float* g_q;        // kEpiQkRope*: QK-norm gains [D]
  const float* g_k;
  const QkEpilogue* qk;    // kEpiQkRope*: dims and rotation table
  // MMDIT_EPI_STORE, bf16: when the product runs split-K, its reduction also
  // writes row_sse[r] = sum_c (Y[r][c] - (z - eps)[sse_row[r]][c])^2 (z, eps
  // [rows, N] model dtype) and sets *sse_done = 1; otherwise *sse_done stays.
  const void* sse_z;
  const void* sse_e;
  const int32_t* sse_row;
  float* row_sse;
  int32_t* sse_done;
};
// The noising of the image embedding's A operand (linear_xt): A holds z and
// eps [M, K] the noise; row m is noised with t[seg[m]] when pos[3 m] == 0 (a
// frame-0, i.e. target, row) and taken as z otherwise; zt [M, K] (optional)
// receives the bf16 z_t.
struct XtArgs {
  const void* eps;
  const float* t;
  const int32_t* seg;
  const int32_t* pos;
  void* zt;
};
mmdit_status linear_xt(const LinearArgs& a, const XtArgs& x, hipStream_t s);
// Epilogues used inside the library only (the public ones are mmdit_epilogue):
constexpr int kEpiGeluAux = 4;      // Y = GELU(acc) and aux = acc (the pre-activation kept for backward)
constexpr int kEpiGatedResAux = 5;  // Y += gate[seg] * acc and aux = acc (the branch kept for backward)
constexpr int kEpiGeluBwd = 6;      // Y = acc * GELU'(aux), aux the saved pre-activation
// The QKV projection (Y [M, 3H] = [Q | K | V]) with QK-RMSNorm + RoPE of the q
// and k heads applied to the bf16-rounded products, the same arithmetic as
// the separate qk_norm_rope kernel on the stored Y (so the same bits); with
// Aux the bf16 q and k before their norm also go to aux [M, 2H].  Where the
// launch's tiles do not all take the 256x256 LDS epilogue, linear() runs the
// plain projection and then that kernel instead.
constexpr int kEpiQkRope = 7;
constexpr int kEpiQkRopeAux = 8;
mmdit_status linear(mmdit_dtype dt, const LinearArgs* probs, int nprob, hipStream_t s);
// Bytes of float32 partial tiles the MLP down projection (site 1) needs for
// its stream-K last round over problems of m0 and m1 rows (N columns, depth
// K) on the current device; 0 when that launch takes no stream-K round.
size_t gemm_sk_partial_bytes(int64_t m0, int64_t m1, int32_t N, int32_t K);

// RMSNorm + adaLN modulate of up to two row sets in one launch.
struct RmsArgs {
  const void* x;
  const int32_t* row_map;
  const int32_t* seg;
  const float* mod;
  void* y;
  int64_t n_rows, mod_stride, shift_off, scale_off;
};
mmdit_status rms_modulate2_impl(mmdit_dtype dt, int32_t H, float eps, const RmsArgs* a, int n, hipStream_t s);

// QK-RMSNorm + RoPE of up to two row sets in one launch.
struct QkArgs {
  void* qkv;
  const int32_t* pos;
  const float* g_q;
  const float* g_k;
  int64_t n_rows;
};
// widths: the RoPE band widths (frame, row, col), even, summing to D.
mmdit_status qk_norm_rope2_impl(mmdit_dtype dt, int32_t heads, int32_t D, const int32_t* widths, float theta,
                                float eps, const QkArgs* a, int n, hipStream_t s);

// ---------------------------------------------------------------- backward
// [n, C] (row stride ldx) -> [C, npad] with zero columns n..npad; op 0 copy,
// 1 GELU of the input, 2 rows scaled by gate[seg[m] * gate_stride + c] (the
// scaled rows also written to y_rows [n, C] when it is not NULL).
struct TransposeArgs {
  const void* x;
  void* y;
  void* y_rows;
  const float* gate;
  const int32_t* seg;
  int64_t ldx, n, npad, gate_stride;
  int32_t C;
};
mmdit_status transpose2_impl(mmdit_dtype dt, const TransposeArgs* t, int n, int op, hipStream_t s);

// Per-sample column sums out[b][out_off[k] + c] = sum over the rows of sample
// b of a_k[r][c] * b_k[r][c] * rs_k[r] (b_k, rs_k optional), in row chunks of
// kColsumRows summed in a fixed order.  partial: [chunks][nterms][H] floats.
constexpr int kColsumRows = 64;
struct ColsumSpec {
  const void* a[3];
  const void* b[3];
  const int32_t* b_map[3];   // optional: b's row is b_map[r]
  const float* rs[3];
  int32_t a_f32[3], b_f32[3], out_off[3];
  int32_t nterms;
  const int32_t* cu;     // device [B + 1]
  const int32_t* h_cu;   // host copy
  int32_t B, H;
  float* partial;
  float* out;
  int64_t out_stride;
};
int64_t colsum_chunks(const int32_t* h_cu, int32_t B, int32_t rc);
mmdit_status seg_colsum_impl(mmdit_dtype dt, const ColsumSpec& sp, hipStream_t s);

// Backward of h = rms(x)(1 + scale) + shift for up to two row sets:
// dx = dres + (dn - n mean(dn n)) / rms(x) with dn = dh (1 + scale); also
// 1/rms per row and, optionally, dgated = gate * dx.
struct NormBwdSpec {
  const int32_t* row_map;   // optional: x, seg and dx rows are row_map[row]; dh, inv_r rows are row
  const void* x;
  const void* dh;
  const float* mod;
  const int32_t* seg;
  const void* dres;
  void* dx;
  float* inv_r;
  const float* gate;
  void* dgated;
  int64_t n, mod_stride;
  int32_t scale_off, gate_off, dres_f32, dx_f32;
};
mmdit_status norm_bwd2_impl(mmdit_dtype dt, int32_t H, float eps, const NormBwdSpec* p, int n, hipStream_t s);

// Backward of q' = RoPE(g_q * rms(q)) (and k) per head, in place on the q, k
// columns of dqkv [n, 3H]; raw [n, 2H] holds q, k before the norm.  The gain
// gradients go to dg_q, dg_k [D] (float32) through per-block partials gpart.
struct QkBwdSpec {
  void* dqkv;
  const void* raw;
  const int32_t* pos;
  const float* g_q;
  const float* g_k;
  float* gpart;
  float* dg_q;
  float* dg_k;
  int64_t n;
};
int64_t qk_bwd_blocks(int64_t n_rows);
mmdit_status qk_bwd2_impl(mmdit_dtype dt, int32_t heads, int32_t D, const int32_t* widths, float theta, float eps,
                          const QkBwdSpec* p, int n, hipStream_t s);

// dW_mod = d_mod^T SiLU(c) per stream ([6H, H] float32) and
// dc += (d_mod W_mod) * SiLU'(c) summed over both streams.
// For y = W f(x), one vector per sample (b < B): dw[s] = dy[s]^T f(x)
// ([rows, cols] float32, s < ns streams sharing x) and, when dx is not NULL,
// dx += f'(x) * sum_s dy[s] W[s]  ([B, cols] float32).  W [rows, cols] in the
// model dtype; x [B, cols] in the model dtype or float32 (x_f32); f is SiLU
// (mode 0) or the identity (mode 1).  rows % 16 == 0.
size_t outer_vecmat_ws_bytes(int32_t B, int32_t rows, int32_t cols);
mmdit_status outer_vecmat_impl(mmdit_dtype dt, int32_t B, int32_t rows, int32_t cols, int ns, const float* const* dy,
                               const void* const* w, const void* x, int32_t x_f32, int32_t mode, float* const* dw,
                               float* dx, void* ws, size_t ws_bytes, hipStream_t s);

// Attention backward over a pack (see attention.hip); ws >= attention_bwd_ws_bytes.
size_t attention_bwd_ws_bytes(const mmdit_pack_t* pk, int32_t heads, int32_t D);
mmdit_status attention_bwd_impl(mmdit_dtype dt, const mmdit_pack_t* pk, int32_t heads, int32_t D,
                                const void* qkv_img, const void* qkv_txt, const void* o_img, const void* o_txt,
                                const float* lse, const void* do_img, const void* do_txt, void* dqkv_img,
                                void* dqkv_txt, void* ws, size_t ws_bytes, hipStream_t s);

// Direct global -> LDS loads: each lane's 16 bytes land at lds_block + 16 *
// lane (the LDS address of the wave instruction is wave-uniform).
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

__device__ __forceinline__ void load_lds16(const void* g, void* lds_block) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)lds_block, 16, 0, 0);
}

// Raw buffer resource over a wave-uniform base (no range clamp: every caller
// keeps its offsets below 2^32 and checks that on the host).
// Direct-to-LDS loads through it take a 32-bit lane offset and a scalar
// offset, so no 64-bit address arithmetic per load.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
template <int BYTES>
__device__ __forceinline__ void buf_lds(rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  static_assert(BYTES == 16 || BYTES == 4, "16- or 4-byte loads");
  if constexpr (BYTES == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voff, soff, 0, 0);
}

// A wave-uniform pointer held in scalar registers, so that base + 32-bit lane
// offset addresses a direct load without 64-bit vector arithmetic per load.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void buf_lds16(rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  buf_lds<16>(r, voff, soff, lds);
}

}  // namespace mmdit
