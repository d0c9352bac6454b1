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
// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
// t = 1 / (1 + p x), for x >= 0 (odd for x < 0); absolute error <= 1.5e-7.
// About a dozen instructions, against the several-branch library erff; t
// takes the hardware reciprocal (1 ulp; its argument is >= 1).
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  return copysignf(1.0f - poly * __expf(-ax * ax), x);
}
// GELU in its erf form, 0.5 x (1 + erf(x / sqrt 2)).
__device__ __forceinline__ float gelu_f(float x) { return 0.5f * x * (1.0f + erf_as(x * 0.70710678118654752f)); }
// Its derivative Phi(x) + x phi(x), with the same erf.
__device__ __forceinline__ float gelu_grad_f(float x) {
  return 0.5f * (1.0f + erf_as(x * 0.70710678118654752f)) + x * 0.39894228040143268f * __expf(-0.5f * x * x);
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------ internal API
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
};
// Epilogues used inside the library only (the public ones are mmdit_epilogue):
constexpr int kEpiGeluAux = 4;      // Y = GELU(acc) and aux = acc (the pre-activation kept for backward)
constexpr int kEpiGatedResAux = 5;  // Y += gate[seg] * acc and aux = acc (the branch kept for backward)
constexpr int kEpiGeluBwd = 6;      // Y = acc * GELU'(aux), aux the saved pre-activation
mmdit_status linear(mmdit_dtype dt, const LinearArgs* probs, int nprob, hipStream_t s);

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
mmdit_status qk_norm_rope2_impl(mmdit_dtype dt, int32_t heads, int32_t D, float theta, float eps, const QkArgs* a,
                                int n, hipStream_t s);

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
mmdit_status qk_bwd2_impl(mmdit_dtype dt, int32_t heads, int32_t D, float theta, float eps, const QkBwdSpec* p,
                          int n, hipStream_t s);

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

}  // namespace mmdit
