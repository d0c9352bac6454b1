// C ABI of libmmdit: argument validation, workspace layout and the launch
// sequence of the block, the conditioning and the rectified-flow wrapper.
#include <map>
#include <string>
#include <vector>

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"

namespace mmdit {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

mmdit_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return MMDIT_OK;
  set_error("%s: %s", what, hipGetErrorString(e));
  return MMDIT_E_HIP;
}

static bool sync_mode() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("MMDIT_SYNC");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

// ------------------------------------------------------- kernel timing
// While enabled, MMDIT_LAUNCH records an event before each launch and
// launch_check one after it; the report sums the elapsed times per kernel
// name.  Single-threaded use; not for use under stream capture.
namespace {
struct TimingRec {
  const char* name;
  int a, b;
};
bool g_timing = false;
std::vector<hipEvent_t> g_events;
size_t g_used = 0;
int g_pending = -1;
std::vector<TimingRec> g_recs;

int next_event() {
  if (g_used == g_events.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return -1;
    g_events.push_back(e);
  }
  return (int)g_used++;
}
}  // namespace

void timing_begin(hipStream_t s) {
  if (!g_timing) return;
  g_pending = next_event();
  if (g_pending >= 0) (void)hipEventRecord(g_events[g_pending], s);
}

mmdit_status launch_check(const char* kernel, hipStream_t s) {
  MMDIT_TRY(hip_check(hipGetLastError(), kernel));
  if (g_timing && g_pending >= 0) {
    int e = next_event();
    if (e >= 0) {
      (void)hipEventRecord(g_events[e], s);
      g_recs.push_back({kernel, g_pending, e});
    }
    g_pending = -1;
  }
  if (sync_mode()) MMDIT_TRY(hip_check(hipStreamSynchronize(s), kernel));
  return MMDIT_OK;
}

// implemented next to their kernels
mmdit_status plan_impl(const mmdit_sample*, int32_t, int64_t, int64_t, int32_t*, int64_t*, int64_t*, int32_t*);
mmdit_status pack_impl(const mmdit_sample*, int32_t, mmdit_pack_t*, hipStream_t);
mmdit_status gather_impl(const mmdit_pack_t*, int32_t, const void* const*, int32_t, mmdit_dtype, void*, hipStream_t);
mmdit_status make_xt_impl(const mmdit_pack_t*, mmdit_dtype, int32_t, const void*, const void*, const float*, void*, hipStream_t);
mmdit_status loss_impl(const mmdit_pack_t*, mmdit_dtype, int32_t, const void*, const void*, const void*, float*, float*, void*, size_t, hipStream_t);
mmdit_status row_sse_impl(const mmdit_pack_t*, mmdit_dtype, int32_t, const void*, const void*, const void*, float*, hipStream_t);
mmdit_status loss_finalize_impl(const mmdit_pack_t*, int32_t, const float*, float*, float*, hipStream_t);
mmdit_status loss_noalloc_impl(const mmdit_pack_t*, mmdit_dtype, int32_t, const void*, const void*, const void*, float*, float*, hipStream_t);
mmdit_status nft_loss_impl(const mmdit_pack_t*, mmdit_dtype, int32_t, const void*, const void*, const void*, const void*, const float*, float*, float*, void*, size_t, hipStream_t);
mmdit_status loss_grad_impl(const mmdit_pack_t*, mmdit_dtype, int32_t, const void*, const void*, const void*, void*, hipStream_t);
mmdit_status euler_impl(const mmdit_pack_t*, mmdit_dtype, int32_t, const void*, int32_t, int32_t, float, float, float, float*, void*, hipStream_t);
mmdit_status pack_latent_impl(const mmdit_pack_t*, mmdit_dtype, int32_t, const float*, int32_t, int32_t, void*, hipStream_t);
mmdit_status rms_modulate_impl(mmdit_dtype, int64_t, int32_t, const void*, const int32_t*, const int32_t*, const float*, int64_t, int64_t, int64_t, void*, float, hipStream_t);
mmdit_status qk_norm_rope_impl(mmdit_dtype, int64_t, int32_t, int32_t, const int32_t*, void*, const int32_t*, const float*, const float*, float, float, hipStream_t);
mmdit_status temb_impl(mmdit_dtype, int32_t, int32_t, const float*, void*, hipStream_t);
mmdit_status attention_impl(mmdit_dtype, const mmdit_pack_t*, int32_t, int32_t, const void*, const void*, void*, void*, void*, size_t, hipStream_t, float* lse = nullptr);
int64_t attention_vt_elems(const mmdit_pack_t*, int32_t);

namespace {

size_t esize(mmdit_dtype d) { return d == MMDIT_BF16 ? 2 : 4; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

mmdit_status check_dims(const mmdit_dims* d, const char* who) {
  if (!d) {
    set_error("%s: dims is NULL", who);
    return MMDIT_E_INVALID;
  }
  if (d->dtype != MMDIT_F32 && d->dtype != MMDIT_BF16) {
    set_error("%s: unknown dtype %d", who, (int)d->dtype);
    return MMDIT_E_INVALID;
  }
  if (d->heads <= 0 || d->hidden != d->heads * d->head_dim || d->mlp <= 0 || d->c_lat <= 0 ||
      d->d_txt <= 0 || d->t_dim <= 0 || !(d->eps > 0.f) || !(d->rope_theta > 0.f)) {
    set_error("%s: inconsistent dims (hidden=%d heads=%d head_dim=%d mlp=%d c_lat=%d d_txt=%d t_dim=%d)",
              who, d->hidden, d->heads, d->head_dim, d->mlp, d->c_lat, d->d_txt, d->t_dim);
    return MMDIT_E_INVALID;
  }
  if ((d->head_dim != 64 && d->head_dim != 128) || d->hidden % 64 || d->mlp % 64 || d->c_lat % 64 ||
      d->d_txt % 64 || d->t_dim % 16 || d->hidden > 8192) {
    set_error("%s: unsupported dims (head_dim in {64,128}; hidden, mlp, c_lat, d_txt multiples of 64, "
              "hidden <= 8192; t_dim multiple of 16)", who);
    return MMDIT_E_UNSUPPORTED;
  }
  const int32_t* rd = d->rope_dims;
  if (rd[0] < 0 || rd[1] < 0 || rd[2] < 0 || (rd[0] | rd[1] | rd[2]) & 1 || rd[0] + rd[1] + rd[2] != d->head_dim) {
    set_error("%s: rope_dims (%d, %d, %d) must be even and sum to head_dim=%d", who, rd[0], rd[1], rd[2],
              d->head_dim);
    return MMDIT_E_UNSUPPORTED;
  }
  return MMDIT_OK;
}

mmdit_status check_pack(const mmdit_pack_t* pk, const char* who) {
  if (!pk || pk->B < 0 || pk->B > MMDIT_MAX_SAMPLES || pk->h_cu_img[pk->B] != pk->n_img ||
      pk->h_cu_txt[pk->B] != pk->n_txt || pk->h_cu_tgt[pk->B] != pk->n_tgt) {
    set_error("%s: pack is invalid or was not built by mmdit_pack", who);
    return MMDIT_E_INVALID;
  }
  if (!pk->cu_txt || !pk->cu_img || (pk->n_img > 0 && (!pk->seg_img || !pk->pos_img || !pk->tgt_row)) ||
      (pk->n_txt > 0 && !pk->seg_txt)) {
    set_error("%s: a device array of the pack is NULL", who);
    return MMDIT_E_INVALID;
  }
  return MMDIT_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// scalar-read arrays (timesteps) only need their element alignment
mmdit_status need4(const void* p, const char* who, const char* name) {
  if (!p) {
    set_error("%s: %s is NULL", who, name);
    return MMDIT_E_INVALID;
  }
  if ((uintptr_t)p & 3) {
    set_error("%s: %s is not 4-byte aligned", who, name);
    return MMDIT_E_UNSUPPORTED;
  }
  return MMDIT_OK;
}

mmdit_status need(const void* p, const char* who, const char* name) {
  if (!p) {
    set_error("%s: %s is NULL", who, name);
    return MMDIT_E_INVALID;
  }
  if (!aligned16(p)) {
    set_error("%s: %s is not 16-byte aligned", who, name);
    return MMDIT_E_UNSUPPORTED;
  }
  return MMDIT_OK;
}

struct Layout {
  size_t mod_img, mod_txt, h, qkv, o, u, vt, rope, sk, end;
};

Layout block_layout(const mmdit_dims* d, const mmdit_pack_t* pk) {
  const size_t es = esize(d->dtype);
  const size_t N = (size_t)(pk->n_img + pk->n_txt);
  const size_t H = d->hidden;
  Layout L;
  size_t o = 0;
  L.mod_img = o; o = align256(o + (size_t)pk->B * 6 * H * 4);
  L.mod_txt = o; o = align256(o + (size_t)pk->B * 6 * H * 4);
  L.h = o;       o = align256(o + N * H * es);
  L.qkv = o;     o = align256(o + N * 3 * H * es);
  L.o = o;       o = align256(o + N * H * es);
  L.u = o;       o = align256(o + N * (size_t)d->mlp * es);
  L.vt = o;      o = align256(o + (size_t)attention_vt_elems(pk, d->hidden) * es);
  L.rope = o;    o = align256(o + (size_t)pk->n_img * d->head_dim * 4);   // (cos, sin) per image row and pair
  // partial tiles of the MLP down projection's stream-K last round (bf16 MFMA path only)
  L.sk = o;
  if (d->dtype == MMDIT_BF16)
    o = align256(o + gemm_sk_partial_bytes(pk->n_img > 0 ? pk->n_img : pk->n_txt,
                                           pk->n_img > 0 ? pk->n_txt : 0, d->hidden, d->mlp));
  L.end = o;
  return L;
}

// final layer: adaLN vectors, modulated target rows, split-K partials (up to 8)
size_t final_ws(const mmdit_dims* d, const mmdit_pack_t* pk) {
  return align256((size_t)pk->B * 2 * d->hidden * 4) + align256((size_t)pk->n_tgt * d->hidden * esize(d->dtype)) +
         align256((size_t)8 * pk->n_tgt * d->c_lat * 4);
}

LinearArgs mk(int64_t M, int32_t N, int32_t K, const void* A, const void* W, void* Y, int epi) {
  LinearArgs a;
  memset(&a, 0, sizeof(a));
  a.M = M;
  a.N = N;
  a.K = K;
  a.A = A;
  a.lda = K;
  a.W = W;
  a.Y = Y;
  a.ldy = N;
  a.epilogue = epi;
  return a;
}

mmdit_status check_stream_w(const mmdit_stream_w& w, const char* who) {
  MMDIT_TRY(need(w.w_mod, who, "w_mod"));
  MMDIT_TRY(need(w.w_qkv, who, "w_qkv"));
  MMDIT_TRY(need(w.g_q, who, "g_q"));
  MMDIT_TRY(need(w.g_k, who, "g_k"));
  MMDIT_TRY(need(w.w_o, who, "w_o"));
  MMDIT_TRY(need(w.w_up, who, "w_up"));
  MMDIT_TRY(need(w.w_down, who, "w_down"));
  return MMDIT_OK;
}

}  // namespace
}  // namespace mmdit

using namespace mmdit;

extern "C" {

const char* mmdit_last_error(void) { return g_err; }

mmdit_status mmdit_timing_enable(int32_t on) {
  g_timing = on != 0;
  g_used = 0;
  g_pending = -1;
  g_recs.clear();
  return MMDIT_OK;
}

int32_t mmdit_timing_report(int32_t max_entries, char* names, double* total_ms, int64_t* count) {
  if (hip_check(hipDeviceSynchronize(), "mmdit_timing_report") != MMDIT_OK) return -1;
  std::map<std::string, std::pair<double, int64_t>> agg;
  std::vector<std::string> order;
  for (const TimingRec& r : g_recs) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_events[r.a], g_events[r.b]) != hipSuccess) continue;
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      order.push_back(r.name);
      agg[r.name] = {ms, 1};
    } else {
      it->second.first += ms;
      it->second.second += 1;
    }
  }
  int32_t n = 0;
  for (const std::string& k : order) {
    if (n >= max_entries) break;
    if (names) {
      strncpy(names + 64 * n, k.c_str(), 63);
      names[64 * n + 63] = 0;
    }
    if (total_ms) total_ms[n] = agg[k].first;
    if (count) count[n] = agg[k].second;
    ++n;
  }
  return n;
}
const char* mmdit_version(void) { return "mmdit-gfx950 0.1"; }

mmdit_status mmdit_pack_plan(const mmdit_sample* s, int32_t n, int64_t img_budget, int64_t joint_budget,
                             int32_t* n_taken, int64_t* n_img, int64_t* n_txt, int32_t* max_joint) {
  return plan_impl(s, n, img_budget, joint_budget, n_taken, n_img, n_txt, max_joint);
}

mmdit_status mmdit_pack(const mmdit_sample* s, int32_t n, mmdit_pack_t* io, mmdit_stream stream) {
  return pack_impl(s, n, io, (hipStream_t)stream);
}

mmdit_status mmdit_pack_gather(const mmdit_pack_t* pk, int32_t which, const void* const* src,
                               int32_t width, mmdit_dtype dt, void* dst, mmdit_stream stream) {
  MMDIT_TRY(check_pack(pk, "mmdit_pack_gather"));
  return gather_impl(pk, which, src, width, dt, dst, (hipStream_t)stream);
}

size_t mmdit_workspace_size(const mmdit_dims* d, const mmdit_pack_t* pk) {
  if (check_dims(d, "mmdit_workspace_size") != MMDIT_OK || check_pack(pk, "mmdit_workspace_size") != MMDIT_OK)
    return 0;
  size_t w = block_layout(d, pk).end;
  size_t l = align256((size_t)pk->n_tgt * 4 + 4);
  size_t f = final_ws(d, pk) + l;   // rf_final_loss: the final layer's and the row sums
  size_t c = align256((size_t)pk->B * (d->t_dim + d->hidden) * esize(d->dtype) + 256);
  if (f > w) w = f;
  if (l > w) w = l;
  if (c > w) w = c;
  return w;
}

int32_t mmdit_workspace_layout(const mmdit_dims* d, const mmdit_pack_t* pk, size_t* out) {
  if (!out || check_dims(d, "mmdit_workspace_layout") != MMDIT_OK ||
      check_pack(pk, "mmdit_workspace_layout") != MMDIT_OK)
    return 0;
  Layout L = block_layout(d, pk);
  out[0] = L.mod_img;
  out[1] = L.mod_txt;
  out[2] = L.h;
  out[3] = L.qkv;
  out[4] = L.o;
  out[5] = L.u;
  return 6;
}

mmdit_status mmdit_cond(const mmdit_dims* d, const void* w_t1, const void* w_t2, const float* t, int32_t B,
                        void* c, void* ws, size_t ws_bytes, mmdit_stream stream) {
  const char* who = "mmdit_cond";
  MMDIT_TRY(check_dims(d, who));
  if (B < 0) {
    set_error("%s: B=%d", who, B);
    return MMDIT_E_INVALID;
  }
  if (B == 0) return MMDIT_OK;
  MMDIT_TRY(need(w_t1, who, "w_t1"));
  MMDIT_TRY(need(w_t2, who, "w_t2"));
  MMDIT_TRY(need4(t, who, "t"));
  MMDIT_TRY(need(c, who, "c"));
  const size_t es = esize(d->dtype);
  const size_t emb_b = align256((size_t)B * d->t_dim * es);
  const size_t need_b = emb_b + (size_t)B * d->hidden * es;
  if (!ws || ws_bytes < need_b) {
    set_error("%s: workspace needs %zu bytes, got %zu", who, need_b, ws_bytes);
    return MMDIT_E_WORKSPACE;
  }
  hipStream_t s = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  void* emb = w;
  void* h1 = w + emb_b;
  MMDIT_TRY(temb_impl(d->dtype, B, d->t_dim, t, emb, s));
  LinearArgs a = mk(B, d->hidden, d->t_dim, emb, w_t1, h1, MMDIT_EPI_STORE);
  a.tag = "cond_mlp1";
  MMDIT_TRY(linear(d->dtype, &a, 1, s));
  LinearArgs b = mk(B, d->hidden, d->hidden, h1, w_t2, c, MMDIT_EPI_STORE);
  b.a_silu = 1;
  b.tag = "cond_mlp2";
  return linear(d->dtype, &b, 1, s);
}

mmdit_status mmdit_modulation(const mmdit_dims* d, const void* w, int32_t chunks, int32_t B, const void* c,
                              float* mod, mmdit_stream stream) {
  const char* who = "mmdit_modulation";
  MMDIT_TRY(check_dims(d, who));
  if (chunks <= 0 || B < 0) {
    set_error("%s: chunks=%d B=%d", who, chunks, B);
    return MMDIT_E_INVALID;
  }
  if (B == 0) return MMDIT_OK;
  MMDIT_TRY(need(w, who, "w"));
  MMDIT_TRY(need(c, who, "c"));
  MMDIT_TRY(need(mod, who, "mod"));
  LinearArgs a = mk(B, chunks * d->hidden, d->hidden, c, w, mod, MMDIT_EPI_STORE_F32);
  a.a_silu = 1;
  return linear(d->dtype, &a, 1, (hipStream_t)stream);
}

mmdit_status mmdit_embed(const mmdit_dims* d, const void* w_in, const void* w_txt, const mmdit_pack_t* pk,
                         const void* zt, const void* tau, void* x_img, void* x_txt, mmdit_stream stream) {
  const char* who = "mmdit_embed";
  MMDIT_TRY(check_dims(d, who));
  MMDIT_TRY(check_pack(pk, who));
  LinearArgs a[2];
  int n = 0;
  if (pk->n_txt > 0) {
    MMDIT_TRY(need(w_txt, who, "w_txt"));
    MMDIT_TRY(need(tau, who, "tau"));
    MMDIT_TRY(need(x_txt, who, "x_txt"));
    a[n++] = mk(pk->n_txt, d->hidden, d->d_txt, tau, w_txt, x_txt, MMDIT_EPI_STORE);
  }
  if (pk->n_img > 0) {
    MMDIT_TRY(need(w_in, who, "w_in"));
    MMDIT_TRY(need(zt, who, "zt"));
    MMDIT_TRY(need(x_img, who, "x_img"));
    a[n++] = mk(pk->n_img, d->hidden, d->c_lat, zt, w_in, x_img, MMDIT_EPI_STORE);
  }
  if (n == 0) return MMDIT_OK;
  // two launches: the long-K text GEMM and the short-K (epilogue-bound) image
  // GEMM each get their own tile configuration
  for (int i = 0; i < n; ++i) {
    a[i].tag = a[i].K == d->c_lat && a[i].Y == x_img ? "embed_img" : "embed_txt";
    MMDIT_TRY(linear(d->dtype, &a[i], 1, (hipStream_t)stream));
  }
  return MMDIT_OK;
}

mmdit_status mmdit_rms_modulate(const mmdit_dims* d, int64_t n_rows, const void* x, const int32_t* row_map,
                                const int32_t* seg, const float* mod, int64_t mod_stride, int64_t shift_off,
                                int64_t scale_off, void* y, mmdit_stream stream) {
  const char* who = "mmdit_rms_modulate";
  MMDIT_TRY(check_dims(d, who));
  if (n_rows < 0 || mod_stride < 0 || shift_off < 0 || scale_off < 0 ||
      (mod_stride > 0 && (shift_off + d->hidden > mod_stride || scale_off + d->hidden > mod_stride)) ||
      (shift_off | scale_off | mod_stride) % 4) {
    set_error("%s: bad sizes (n_rows=%lld mod_stride=%lld shift_off=%lld scale_off=%lld)", who,
              (long long)n_rows, (long long)mod_stride, (long long)shift_off, (long long)scale_off);
    return MMDIT_E_INVALID;
  }
  if (n_rows == 0) return MMDIT_OK;
  MMDIT_TRY(need(x, who, "x"));
  MMDIT_TRY(need(seg, who, "seg"));
  MMDIT_TRY(need(mod, who, "mod"));
  MMDIT_TRY(need(y, who, "y"));
  return rms_modulate_impl(d->dtype, n_rows, d->hidden, x, row_map, seg, mod, mod_stride, shift_off, scale_off,
                           y, d->eps, (hipStream_t)stream);
}

mmdit_status mmdit_qk_norm_rope(const mmdit_dims* d, int64_t n_rows, void* qkv, const int32_t* pos,
                                const float* g_q, const float* g_k, mmdit_stream stream) {
  const char* who = "mmdit_qk_norm_rope";
  MMDIT_TRY(check_dims(d, who));
  if (n_rows < 0) {
    set_error("%s: n_rows < 0", who);
    return MMDIT_E_INVALID;
  }
  if (n_rows == 0) return MMDIT_OK;
  MMDIT_TRY(need(qkv, who, "qkv"));
  MMDIT_TRY(need(g_q, who, "g_q"));
  MMDIT_TRY(need(g_k, who, "g_k"));
  return qk_norm_rope_impl(d->dtype, n_rows, d->heads, d->head_dim, d->rope_dims, qkv, pos, g_q, g_k, d->rope_theta, d->eps,
                           (hipStream_t)stream);
}

size_t mmdit_attention_workspace_size(const mmdit_dims* d, const mmdit_pack_t* pk) {
  if (check_dims(d, "mmdit_attention_workspace_size") != MMDIT_OK ||
      check_pack(pk, "mmdit_attention_workspace_size") != MMDIT_OK)
    return 0;
  return d->dtype == MMDIT_BF16 ? (size_t)attention_vt_elems(pk, d->hidden) * 2 : 0;
}

mmdit_status mmdit_attention(const mmdit_dims* d, const mmdit_pack_t* pk, const void* qkv_img,
                             const void* qkv_txt, void* o_img, void* o_txt, void* ws, size_t ws_bytes,
                             mmdit_stream stream) {
  const char* who = "mmdit_attention";
  MMDIT_TRY(check_dims(d, who));
  MMDIT_TRY(check_pack(pk, who));
  if (pk->n_img > 0) {
    MMDIT_TRY(need(qkv_img, who, "qkv_img"));
    MMDIT_TRY(need(o_img, who, "o_img"));
  }
  if (pk->n_txt > 0) {
    MMDIT_TRY(need(qkv_txt, who, "qkv_txt"));
    MMDIT_TRY(need(o_txt, who, "o_txt"));
  }
  if (d->dtype == MMDIT_BF16) MMDIT_TRY(need(ws, who, "ws"));
  return attention_impl(d->dtype, pk, d->heads, d->head_dim, qkv_img, qkv_txt, o_img, o_txt, ws, ws_bytes,
                        (hipStream_t)stream);
}

mmdit_status mmdit_linear(mmdit_dtype dt, int64_t M, int32_t N, int32_t K, const void* A, const void* W,
                          void* Y, int32_t epilogue, const float* gate, int64_t gate_stride,
                          const int32_t* seg, int32_t a_silu, mmdit_stream stream) {
  const char* who = "mmdit_linear";
  if (dt != MMDIT_F32 && dt != MMDIT_BF16) {
    set_error("%s: unknown dtype", who);
    return MMDIT_E_INVALID;
  }
  if (epilogue < MMDIT_EPI_STORE || epilogue > MMDIT_EPI_GATED_RES || M < 0 || N <= 0 || K <= 0) {
    set_error("%s: bad arguments (M=%lld N=%d K=%d epilogue=%d)", who, (long long)M, N, K, epilogue);
    return MMDIT_E_INVALID;
  }
  if (M == 0) return MMDIT_OK;
  MMDIT_TRY(need(A, who, "A"));
  MMDIT_TRY(need(W, who, "W"));
  MMDIT_TRY(need(Y, who, "Y"));
  if (epilogue == MMDIT_EPI_GATED_RES) {
    MMDIT_TRY(need(gate, who, "gate"));
    MMDIT_TRY(need(seg, who, "seg"));
    if (gate_stride < N) {
      set_error("%s: gate_stride %lld < N %d", who, (long long)gate_stride, N);
      return MMDIT_E_INVALID;
    }
    // the epilogues read the gate as 16-byte vectors at gate + seg * gate_stride + n
    if (gate_stride % 4) {
      set_error("%s: gate_stride %lld is not a multiple of 4 floats", who, (long long)gate_stride);
      return MMDIT_E_UNSUPPORTED;
    }
  }
  LinearArgs a = mk(M, N, K, A, W, Y, epilogue);
  a.gate = gate;
  a.gate_stride = gate_stride;
  a.seg = seg;
  a.a_silu = a_silu ? 1 : 0;
  return linear(dt, &a, 1, (hipStream_t)stream);
}

namespace {

// Saved intermediates of one block for its backward, image rows then text rows
// in every buffer (all in the model dtype except mod and lse, float32).
struct SavedLayout {
  size_t mod_img, mod_txt, x_in, h1, qkv, qk_raw, o, a, x_mid, h2, u_pre, dmlp, lse, end;
};

SavedLayout saved_layout(const mmdit_dims* d, const mmdit_pack_t* pk) {
  const size_t es = esize(d->dtype);
  const size_t N = (size_t)(pk->n_img + pk->n_txt);
  const size_t H = d->hidden;
  SavedLayout S;
  size_t o = 0;
  S.mod_img = o; o = align256(o + (size_t)pk->B * 6 * H * 4);
  S.mod_txt = o; o = align256(o + (size_t)pk->B * 6 * H * 4);
  S.x_in = o;    o = align256(o + N * H * es);
  S.h1 = o;      o = align256(o + N * H * es);
  S.qkv = o;     o = align256(o + N * 3 * H * es);
  S.qk_raw = o;  o = align256(o + N * 2 * H * es);
  S.o = o;       o = align256(o + N * H * es);
  S.a = o;       o = align256(o + N * H * es);
  S.x_mid = o;   o = align256(o + N * H * es);
  S.h2 = o;      o = align256(o + N * H * es);
  S.u_pre = o;   o = align256(o + N * (size_t)d->mlp * es);
  S.dmlp = o;    o = align256(o + N * H * es);
  S.lse = o;     o = align256(o + (size_t)(attention_vt_elems(pk, d->hidden) / d->head_dim) * 4);
  S.end = o;
  return S;
}

mmdit_status copy_rows(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (bytes == 0) return MMDIT_OK;
  return hip_check(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s), "hipMemcpyAsync");
}

mmdit_status check_block_args(const mmdit_dims* d, const mmdit_block_w* w, const mmdit_pack_t* pk, const void* c,
                              void* x_img, void* x_txt, void* ws, size_t ws_bytes, const char* who) {
  MMDIT_TRY(check_dims(d, who));
  MMDIT_TRY(check_pack(pk, who));
  if (!w) {
    set_error("%s: weights are NULL", who);
    return MMDIT_E_INVALID;
  }
  if (pk->B == 0) return MMDIT_OK;
  MMDIT_TRY(check_stream_w(w->img, who));
  MMDIT_TRY(check_stream_w(w->txt, who));
  MMDIT_TRY(need(c, who, "c"));
  if (pk->n_img > 0) MMDIT_TRY(need(x_img, who, "x_img"));
  if (pk->n_txt > 0) MMDIT_TRY(need(x_txt, who, "x_txt"));
  const Layout L = block_layout(d, pk);
  if (!ws || ws_bytes < L.end) {
    set_error("%s: workspace needs %zu bytes, got %zu", who, L.end, ws_bytes);
    return MMDIT_E_WORKSPACE;
  }
  return need(ws, who, "ws");
}

// adaLN vectors of both streams of a block in one grouped launch:
// mod = W_mod SiLU(c), float32 [B][6H] each.
mmdit_status block_modulation_impl(const mmdit_dims* d, const mmdit_block_w* w, int32_t B, const void* c,
                                   float* mod_i, float* mod_t, hipStream_t s) {
  const int32_t H = d->hidden;
  LinearArgs a[2] = {mk(B, 6 * H, H, c, w->img.w_mod, mod_i, MMDIT_EPI_STORE_F32),
                     mk(B, 6 * H, H, c, w->txt.w_mod, mod_t, MMDIT_EPI_STORE_F32)};
  a[0].a_silu = a[1].a_silu = 1;
  a[0].tag = "adaln_mod";
  return linear(d->dtype, a, 2, s);
}

// The block's launch sequence.  With sv (training) every intermediate the
// backward needs is kept in sv (layout S); the arithmetic is the same.
mmdit_status block_forward_impl(const mmdit_dims* d, const mmdit_block_w* w, const mmdit_pack_t* pk, const void* c,
                                void* x_img, void* x_txt, void* ws, char* sv, const SavedLayout* S,
                                hipStream_t s, const float* premod = nullptr) {
  const Layout L = block_layout(d, pk);
  const mmdit_dtype dt = d->dtype;
  const size_t es = esize(dt);
  const int32_t H = d->hidden;
  const int64_t ni = pk->n_img, nt = pk->n_txt;
  char* base = static_cast<char*>(ws);
  float* mod_i = reinterpret_cast<float*>(sv ? sv + S->mod_img : base + L.mod_img);
  float* mod_t = reinterpret_cast<float*>(sv ? sv + S->mod_txt : base + L.mod_txt);
  char* h = sv ? sv + S->h1 : base + L.h;
  char* qkv = sv ? sv + S->qkv : base + L.qkv;
  char* o = sv ? sv + S->o : base + L.o;
  char* u = base + L.u;
  char* h_t = h + ni * H * es;
  char* qkv_t = qkv + ni * 3 * H * es;
  char* o_t = o + ni * H * es;
  char* u_t = u + ni * (int64_t)d->mlp * es;
  if (sv) {
    MMDIT_TRY(copy_rows(sv + S->x_in, x_img, ni * H * es, s));
    MMDIT_TRY(copy_rows(sv + S->x_in + ni * H * es, x_txt, nt * H * es, s));
  }

  // adaLN vectors of both streams: mod = W_mod SiLU(c), unless the caller
  // computed them beforehand (mmdit_block_modulation; read only from here on)
  if (premod) {
    mod_i = const_cast<float*>(premod);
    mod_t = const_cast<float*>(premod) + (size_t)pk->B * 6 * H;
  } else {
    MMDIT_TRY(block_modulation_impl(d, w, pk->B, c, mod_i, mod_t, s));
  }
  // h = rms(x)(1 + scale1) + shift1   (both streams, one launch)
  {
    RmsArgs r[2] = {{x_img, nullptr, pk->seg_img, mod_i, h, ni, 6 * H, 0, H},
                    {x_txt, nullptr, pk->seg_txt, mod_t, h_t, nt, 6 * H, 0, H}};
    MMDIT_TRY(rms_modulate2_impl(dt, H, d->eps, r, 2, s));
  }
  // qkv = h W_qkv^T, then QK-RMSNorm + RoPE of q and k (image rows at their
  // (frame, row, col), text rows at the origin) in the projection's epilogue;
  // training also keeps q and k before their norm
  {
    QkEpilogue qe;
    qe.heads = d->heads;
    qe.D = d->head_dim;
    qe.eps = d->eps;
    qe.theta = d->rope_theta;
    for (int i = 0; i < 3; ++i) qe.widths[i] = d->rope_dims[i];
    rope_table(&qe.tab, d->rope_dims, d->rope_theta);
    const int epi = sv ? kEpiQkRopeAux : kEpiQkRope;
    float* rope_cs = reinterpret_cast<float*>(base + L.rope);
    MMDIT_TRY(rope_cs_impl(pk->pos_img, ni, d->head_dim, qe.tab, rope_cs, s));
    LinearArgs a[2] = {mk(ni, 3 * H, H, h, w->img.w_qkv, qkv, epi), mk(nt, 3 * H, H, h_t, w->txt.w_qkv, qkv_t, epi)};
    a[0].pos = pk->pos_img;
    a[0].rope_cs = rope_cs;
    a[1].pos = nullptr;
    a[1].rope_cs = nullptr;
    a[0].g_q = w->img.g_q;
    a[0].g_k = w->img.g_k;
    a[1].g_q = w->txt.g_q;
    a[1].g_k = w->txt.g_k;
    a[0].qk = a[1].qk = &qe;
    if (sv) {
      a[0].aux = sv + S->qk_raw;
      a[1].aux = sv + S->qk_raw + ni * 2 * (size_t)H * es;
    }
    a[0].tag = "qkv_proj";
    MMDIT_TRY(linear(dt, a, 2, s));
  }
  // o = block-diagonal joint attention
  MMDIT_TRY(attention_impl(dt, pk, d->heads, d->head_dim, qkv, qkv_t, o, o_t, base + L.vt, L.rope - L.vt, s,
                           sv ? reinterpret_cast<float*>(sv + S->lse) : nullptr));
  // x += gate1 * (o W_o^T)
  {
    LinearArgs a[2] = {mk(ni, H, H, o, w->img.w_o, x_img, sv ? kEpiGatedResAux : MMDIT_EPI_GATED_RES),
                       mk(nt, H, H, o_t, w->txt.w_o, x_txt, sv ? kEpiGatedResAux : MMDIT_EPI_GATED_RES)};
    a[0].gate = mod_i + 2 * H;
    a[1].gate = mod_t + 2 * H;
    a[0].gate_stride = a[1].gate_stride = 6 * H;
    a[0].seg = pk->seg_img;
    a[1].seg = pk->seg_txt;
    a[0].tag = "out_proj_gated";
    if (sv) {
      a[0].aux = sv + S->a;
      a[1].aux = sv + S->a + ni * H * es;
    }
    MMDIT_TRY(linear(dt, a, 2, s));
  }
  if (sv) {
    MMDIT_TRY(copy_rows(sv + S->x_mid, x_img, ni * H * es, s));
    MMDIT_TRY(copy_rows(sv + S->x_mid + ni * H * es, x_txt, nt * H * es, s));
    h = sv + S->h2;
    h_t = h + ni * H * es;
  }
  // h = rms(x)(1 + scale2) + shift2
  {
    RmsArgs r[2] = {{x_img, nullptr, pk->seg_img, mod_i, h, ni, 6 * H, 3 * H, 4 * H},
                    {x_txt, nullptr, pk->seg_txt, mod_t, h_t, nt, 6 * H, 3 * H, 4 * H}};
    MMDIT_TRY(rms_modulate2_impl(dt, H, d->eps, r, 2, s));
  }
  // u = GELU(h W_up^T)
  {
    LinearArgs a[2] = {mk(ni, d->mlp, H, h, w->img.w_up, u, sv ? kEpiGeluAux : MMDIT_EPI_GELU),
                       mk(nt, d->mlp, H, h_t, w->txt.w_up, u_t, sv ? kEpiGeluAux : MMDIT_EPI_GELU)};
    a[0].tag = "mlp_up_gelu";
    if (sv) {
      a[0].aux = sv + S->u_pre;
      a[1].aux = sv + S->u_pre + ni * (int64_t)d->mlp * es;
    }
    MMDIT_TRY(linear(dt, a, 2, s));
  }
  // x += gate2 * (u W_down^T)
  {
    LinearArgs a[2] = {mk(ni, H, d->mlp, u, w->img.w_down, x_img, sv ? kEpiGatedResAux : MMDIT_EPI_GATED_RES),
                       mk(nt, H, d->mlp, u_t, w->txt.w_down, x_txt, sv ? kEpiGatedResAux : MMDIT_EPI_GATED_RES)};
    a[0].gate = mod_i + 5 * H;
    a[1].gate = mod_t + 5 * H;
    a[0].gate_stride = a[1].gate_stride = 6 * H;
    a[0].seg = pk->seg_img;
    a[1].seg = pk->seg_txt;
    a[0].tag = "mlp_down_gated";
    a[0].site = 1;
    a[0].partial = reinterpret_cast<float*>(base + L.sk);
    a[0].partial_elems = (int64_t)((L.end - L.sk) / sizeof(float));
    if (sv) {
      a[0].aux = sv + S->dmlp;
      a[1].aux = sv + S->dmlp + ni * H * es;
    }
    MMDIT_TRY(linear(dt, a, 2, s));
  }
  return MMDIT_OK;
}

}  // namespace

mmdit_status mmdit_block_fwd(const mmdit_dims* d, const mmdit_block_w* w, const mmdit_pack_t* pk, const void* c,
                             void* x_img, void* x_txt, void* ws, size_t ws_bytes, mmdit_stream stream) {
  MMDIT_TRY(check_block_args(d, w, pk, c, x_img, x_txt, ws, ws_bytes, "mmdit_block_fwd"));
  if (pk->B == 0) return MMDIT_OK;
  return block_forward_impl(d, w, pk, c, x_img, x_txt, ws, nullptr, nullptr, (hipStream_t)stream);
}

mmdit_status mmdit_block_modulation(const mmdit_dims* d, const mmdit_block_w* w, int32_t B, const void* c,
                                    float* mod, mmdit_stream stream) {
  const char* who = "mmdit_block_modulation";
  MMDIT_TRY(check_dims(d, who));
  if (!w) {
    set_error("%s: weights are NULL", who);
    return MMDIT_E_INVALID;
  }
  if (B < 0 || B > MMDIT_MAX_SAMPLES) {
    set_error("%s: B = %d outside [0, %d]", who, B, MMDIT_MAX_SAMPLES);
    return MMDIT_E_INVALID;
  }
  if (B == 0) return MMDIT_OK;
  MMDIT_TRY(need(w->img.w_mod, who, "img.w_mod"));
  MMDIT_TRY(need(w->txt.w_mod, who, "txt.w_mod"));
  MMDIT_TRY(need(c, who, "c"));
  MMDIT_TRY(need(mod, who, "mod"));
  return block_modulation_impl(d, w, B, c, mod, mod + (size_t)B * 6 * d->hidden, (hipStream_t)stream);
}

mmdit_status mmdit_block_fwd_mod(const mmdit_dims* d, const mmdit_block_w* w, const mmdit_pack_t* pk,
                                 const float* mod, void* x_img, void* x_txt, void* ws, size_t ws_bytes,
                                 mmdit_stream stream) {
  MMDIT_TRY(check_block_args(d, w, pk, mod, x_img, x_txt, ws, ws_bytes, "mmdit_block_fwd_mod"));
  if (pk->B == 0) return MMDIT_OK;
  return block_forward_impl(d, w, pk, nullptr, x_img, x_txt, ws, nullptr, nullptr, (hipStream_t)stream, mod);
}

size_t mmdit_block_saved_size(const mmdit_dims* d, const mmdit_pack_t* pk) {
  if (check_dims(d, "mmdit_block_saved_size") != MMDIT_OK || check_pack(pk, "mmdit_block_saved_size") != MMDIT_OK)
    return 0;
  return saved_layout(d, pk).end;
}

mmdit_status mmdit_block_fwd_train(const mmdit_dims* d, const mmdit_block_w* w, const mmdit_pack_t* pk,
                                   const void* c, void* x_img, void* x_txt, void* saved, size_t saved_bytes,
                                   void* ws, size_t ws_bytes, mmdit_stream stream) {
  const char* who = "mmdit_block_fwd_train";
  MMDIT_TRY(check_block_args(d, w, pk, c, x_img, x_txt, ws, ws_bytes, who));
  if (pk->B == 0) return MMDIT_OK;
  const SavedLayout S = saved_layout(d, pk);
  if (!saved || saved_bytes < S.end) {
    set_error("%s: saved buffer needs %zu bytes, got %zu", who, S.end, saved_bytes);
    return MMDIT_E_WORKSPACE;
  }
  MMDIT_TRY(need(saved, who, "saved"));
  return block_forward_impl(d, w, pk, c, x_img, x_txt, ws, static_cast<char*>(saved), &S, (hipStream_t)stream);
}

namespace {

int64_t pad64(int64_t n) { return (n + 63) & ~(int64_t)63; }

// Workspace of the block backward.
struct BwdLayout {
  size_t wt_down, wt_up, wt_o, wt_qkv, dd, ddT, guT, du, duT, h2T, dh2, dxmid, inv_r, da, daT, oT, dO, dqkv, dqkvT,
      h1T, dh1, dmod, partial, gpart, modg, attn, end;
};

BwdLayout bwd_layout(const mmdit_dims* d, const mmdit_pack_t* pk) {
  const size_t es = esize(d->dtype);
  const size_t N = (size_t)(pk->n_img + pk->n_txt);
  const size_t NP = (size_t)(pad64(pk->n_img) + pad64(pk->n_txt));
  const size_t H = d->hidden, M = d->mlp;
  BwdLayout Lb;
  size_t o = 0;
  Lb.wt_down = o; o = align256(o + 2 * M * H * es);
  Lb.wt_up = o;   o = align256(o + 2 * M * H * es);
  Lb.wt_o = o;    o = align256(o + 2 * H * H * es);
  Lb.wt_qkv = o;  o = align256(o + 2 * 3 * H * H * es);
  Lb.dd = o;      o = align256(o + N * H * es);
  Lb.ddT = o;     o = align256(o + H * NP * es);
  Lb.guT = o;     o = align256(o + M * NP * es);
  Lb.du = o;      o = align256(o + N * M * es);
  Lb.duT = o;     o = align256(o + M * NP * es);
  Lb.h2T = o;     o = align256(o + H * NP * es);
  Lb.dh2 = o;     o = align256(o + N * H * es);
  Lb.dxmid = o;   o = align256(o + N * H * 4);
  Lb.inv_r = o;   o = align256(o + N * 4);
  Lb.da = o;      o = align256(o + N * H * es);
  Lb.daT = o;     o = align256(o + H * NP * es);
  Lb.oT = o;      o = align256(o + H * NP * es);
  Lb.dO = o;      o = align256(o + N * H * es);
  Lb.dqkv = o;    o = align256(o + N * 3 * H * es);
  Lb.dqkvT = o;   o = align256(o + 3 * H * NP * es);
  Lb.h1T = o;     o = align256(o + H * NP * es);
  Lb.dh1 = o;     o = align256(o + N * H * es);
  Lb.dmod = o;    o = align256(o + 2 * (size_t)pk->B * 6 * H * 4);
  const int64_t ch = colsum_chunks(pk->h_cu_img, pk->B, kColsumRows) + colsum_chunks(pk->h_cu_txt, pk->B, kColsumRows);
  Lb.partial = o; o = align256(o + (size_t)ch * 3 * H * 4);
  Lb.gpart = o;   o = align256(o + (size_t)(qk_bwd_blocks(pk->n_img) + qk_bwd_blocks(pk->n_txt)) * 2 * d->head_dim * 4);
  Lb.modg = o;    o = align256(o + outer_vecmat_ws_bytes(pk->B, 6 * d->hidden, d->hidden));
  Lb.attn = o;    o = align256(o + attention_bwd_ws_bytes(pk, d->heads, d->head_dim));
  Lb.end = o;
  return Lb;
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

mmdit_status fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return MMDIT_OK;
  const int64_t blocks = cdiv(n, 256) < 4096 ? cdiv(n, 256) : 4096;
  MMDIT_LAUNCH(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return launch_check("fill_zero_kernel", s);
}

mmdit_status check_grads(const mmdit_stream_grad& g, const char* who) {
  const float* p[7] = {g.w_mod, g.w_qkv, g.g_q, g.g_k, g.w_o, g.w_up, g.w_down};
  const char* n[7] = {"dw_mod", "dw_qkv", "dg_q", "dg_k", "dw_o", "dw_up", "dw_down"};
  for (int i = 0; i < 7; ++i) MMDIT_TRY(need(p[i], who, n[i]));
  return MMDIT_OK;
}

// Weight gradient dW [out, in] = sum over rows of dY[r, out] X[r, in] for both
// streams: A = dY^T [out, rows padded], W = X^T [in, rows padded], float32 out.
// A stream without rows gets a zero gradient.
mmdit_status weight_grad(mmdit_dtype dt, int32_t out, int32_t in, const int64_t np[2], const char* dyT[2],
                         const char* xT[2], float* dw[2], const char* tag, hipStream_t s) {
  LinearArgs a[2];
  int n = 0;
  for (int i = 0; i < 2; ++i) {
    if (np[i] == 0) {
      MMDIT_TRY(fill_zero(dw[i], (int64_t)out * in, s));
      continue;
    }
    a[n] = mk(out, in, (int32_t)np[i], dyT[i], xT[i], dw[i], MMDIT_EPI_STORE_F32);
    a[n].tag = tag;
    ++n;
  }
  return n ? linear(dt, a, n, s) : MMDIT_OK;
}

}  // namespace

size_t mmdit_block_bwd_workspace_size(const mmdit_dims* d, const mmdit_pack_t* pk) {
  if (check_dims(d, "mmdit_block_bwd_workspace_size") != MMDIT_OK ||
      check_pack(pk, "mmdit_block_bwd_workspace_size") != MMDIT_OK)
    return 0;
  return bwd_layout(d, pk).end;
}

namespace {

// Fork / join events of the two-stream block backward (no timing), created
// once per device on first use and reused by every call.
hipEvent_t bwd_event(int k) {
  constexpr int kDev = 64, kEv = 8;
  static hipEvent_t ev[kDev][kEv] = {};
  int dev = 0;
  if (k < 0 || k >= kEv || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDev) return nullptr;
  if (!ev[dev][k] && hipEventCreateWithFlags(&ev[dev][k], hipEventDisableTiming) != hipSuccess) {
    ev[dev][k] = nullptr;
    return nullptr;
  }
  return ev[dev][k];
}

mmdit_status block_bwd_impl(const mmdit_dims* d, const mmdit_block_w* w, const mmdit_pack_t* pk, const void* c,
                            const void* saved, size_t saved_bytes, void* dx_img, void* dx_txt,
                            const mmdit_block_grad* g, float* dc, void* ws, size_t ws_bytes,
                            mmdit_stream stream, mmdit_stream stream_w, const char* who) {
  MMDIT_TRY(check_dims(d, who));
  MMDIT_TRY(check_pack(pk, who));
  if (!w || !g) {
    set_error("%s: weights or gradients are NULL", who);
    return MMDIT_E_INVALID;
  }
  MMDIT_TRY(check_stream_w(w->img, who));
  MMDIT_TRY(check_stream_w(w->txt, who));
  MMDIT_TRY(check_grads(g->img, who));
  MMDIT_TRY(check_grads(g->txt, who));
  if (pk->B == 0) return MMDIT_OK;
  MMDIT_TRY(need(c, who, "c"));
  MMDIT_TRY(need(dc, who, "dc"));
  if (pk->n_img > 0) MMDIT_TRY(need(dx_img, who, "dx_img"));
  if (pk->n_txt > 0) MMDIT_TRY(need(dx_txt, who, "dx_txt"));
  const SavedLayout S = saved_layout(d, pk);
  if (!saved || saved_bytes < S.end) {
    set_error("%s: saved buffer needs %zu bytes, got %zu", who, S.end, saved_bytes);
    return MMDIT_E_WORKSPACE;
  }
  MMDIT_TRY(need(saved, who, "saved"));
  const BwdLayout Lb = bwd_layout(d, pk);
  if (!ws || ws_bytes < Lb.end) {
    set_error("%s: workspace needs %zu bytes, got %zu", who, Lb.end, ws_bytes);
    return MMDIT_E_WORKSPACE;
  }
  MMDIT_TRY(need(ws, who, "ws"));
  hipStream_t s = (hipStream_t)stream;
  // weight gradients (their transposes and GEMMs) on sw: each group forks
  // from s once its inputs exist there and sw joins s at the end.  Nothing sw
  // reads is written again by s within the call, and every region is its own.
  hipStream_t sw = stream_w ? (hipStream_t)stream_w : s;
  const bool two = sw != s;
  int nfork = 0;
  auto fork = [&]() -> mmdit_status {
    if (!two) return MMDIT_OK;
    hipEvent_t e = bwd_event(nfork++);
    if (!e) {
      set_error("%s: could not create a stream event", who);
      return MMDIT_E_HIP;
    }
    MMDIT_TRY(hip_check(hipEventRecord(e, s), "hipEventRecord"));
    return hip_check(hipStreamWaitEvent(sw, e, 0), "hipStreamWaitEvent");
  };
  const mmdit_dtype dt = d->dtype;
  const size_t es = esize(dt);
  const int32_t H = d->hidden, M = d->mlp, D = d->head_dim;
  const int64_t ni = pk->n_img, nt = pk->n_txt;
  const int64_t np[2] = {pad64(ni), pad64(nt)};
  const int64_t nr[2] = {ni, nt};
  const char* sv = static_cast<const char*>(saved);
  char* base = static_cast<char*>(ws);
  const float* mod[2] = {reinterpret_cast<const float*>(sv + S.mod_img), reinterpret_cast<const float*>(sv + S.mod_txt)};
  const int32_t* seg[2] = {pk->seg_img, pk->seg_txt};
  const mmdit_stream_w* ws_w[2] = {&w->img, &w->txt};
  const mmdit_stream_grad* gr[2] = {&g->img, &g->txt};
  void* dx[2] = {dx_img, dx_txt};
  // row offset (in elements of width C) of stream i in a rows-major buffer, and
  // in a transposed buffer with padded row counts
  auto rows = [&](size_t off, int i, int64_t C) { return base + off + (i ? ni * C * (int64_t)es : 0); };
  auto srows = [&](size_t off, int i, int64_t C) { return sv + off + (i ? ni * C * (int64_t)es : 0); };
  auto trows = [&](size_t off, int i, int64_t C) { return base + off + (i ? C * np[0] * (int64_t)es : 0); };
  auto wt = [&](size_t off, int i, int64_t elems) { return base + off + (i ? elems * (int64_t)es : 0); };
  float* dmod[2] = {reinterpret_cast<float*>(base + Lb.dmod),
                    reinterpret_cast<float*>(base + Lb.dmod) + (size_t)pk->B * 6 * H};

  // transposed weights: W_down^T [M, H], W_up^T [H, M], W_o^T [H, H], W_qkv^T [H, 3H]
  {
    const struct { size_t off; int wi; int32_t O, I; } tw[4] = {
        {Lb.wt_down, 6, H, M}, {Lb.wt_up, 5, M, H}, {Lb.wt_o, 4, H, H}, {Lb.wt_qkv, 1, 3 * H, H}};
    for (const auto& t : tw) {
      TransposeArgs ta[2];
      memset(ta, 0, sizeof(ta));
      for (int i = 0; i < 2; ++i) {
        const void* src = t.wi == 6 ? ws_w[i]->w_down : t.wi == 5 ? ws_w[i]->w_up : t.wi == 4 ? ws_w[i]->w_o
                                                                                              : ws_w[i]->w_qkv;
        ta[i] = {src, wt(t.off, i, (int64_t)t.O * t.I), nullptr, nullptr, nullptr, t.I, t.O, t.O, 0, t.I};
      }
      MMDIT_TRY(transpose2_impl(dt, ta, 2, 0, s));
    }
  }
  // MLP branch: dd = gate2 * dy (and dd^T), du = (dd W_down) * GELU'(u_pre)
  {
    TransposeArgs ta[2];
    for (int i = 0; i < 2; ++i)
      ta[i] = {dx[i], trows(Lb.ddT, i, H), rows(Lb.dd, i, H), mod[i] + 5 * H, seg[i], H, nr[i], np[i], 6 * H, H};
    MMDIT_TRY(transpose2_impl(dt, ta, 2, 2, s));
  }
  MMDIT_TRY(fork());   // dd^T ready
  {
    TransposeArgs ta[2];
    memset(ta, 0, sizeof(ta));
    for (int i = 0; i < 2; ++i) ta[i] = {srows(S.u_pre, i, M), trows(Lb.guT, i, M), nullptr, nullptr, nullptr, M, nr[i], np[i], 0, M};
    MMDIT_TRY(transpose2_impl(dt, ta, 2, 1, sw));
    const char* A[2] = {trows(Lb.ddT, 0, H), trows(Lb.ddT, 1, H)};
    const char* X[2] = {trows(Lb.guT, 0, M), trows(Lb.guT, 1, M)};
    float* dw[2] = {gr[0]->w_down, gr[1]->w_down};
    MMDIT_TRY(weight_grad(dt, H, M, np, A, X, dw, "bwd_mlp_down_dw", sw));
  }
  {
    LinearArgs a[2] = {mk(ni, M, H, rows(Lb.dd, 0, H), wt(Lb.wt_down, 0, 0), rows(Lb.du, 0, M), kEpiGeluBwd),
                       mk(nt, M, H, rows(Lb.dd, 1, H), wt(Lb.wt_down, 1, (int64_t)M * H), rows(Lb.du, 1, M), kEpiGeluBwd)};
    a[0].aux = const_cast<char*>(srows(S.u_pre, 0, M));
    a[1].aux = const_cast<char*>(srows(S.u_pre, 1, M));
    a[0].tag = "bwd_mlp_down_dx";
    MMDIT_TRY(linear(dt, a, 2, s));
  }
  MMDIT_TRY(fork());   // du ready
  {
    TransposeArgs ta[2];
    memset(ta, 0, sizeof(ta));
    for (int i = 0; i < 2; ++i) ta[i] = {rows(Lb.du, i, M), trows(Lb.duT, i, M), nullptr, nullptr, nullptr, M, nr[i], np[i], 0, M};
    MMDIT_TRY(transpose2_impl(dt, ta, 2, 0, sw));
    for (int i = 0; i < 2; ++i) ta[i] = {srows(S.h2, i, H), trows(Lb.h2T, i, H), nullptr, nullptr, nullptr, H, nr[i], np[i], 0, H};
    MMDIT_TRY(transpose2_impl(dt, ta, 2, 0, sw));
    const char* A[2] = {trows(Lb.duT, 0, M), trows(Lb.duT, 1, M)};
    const char* X[2] = {trows(Lb.h2T, 0, H), trows(Lb.h2T, 1, H)};
    float* dw[2] = {gr[0]->w_up, gr[1]->w_up};
    MMDIT_TRY(weight_grad(dt, M, H, np, A, X, dw, "bwd_mlp_up_dw", sw));
  }
  {
    LinearArgs a[2] = {mk(ni, H, M, rows(Lb.du, 0, M), wt(Lb.wt_up, 0, 0), rows(Lb.dh2, 0, H), MMDIT_EPI_STORE),
                       mk(nt, H, M, rows(Lb.du, 1, M), wt(Lb.wt_up, 1, (int64_t)M * H), rows(Lb.dh2, 1, H), MMDIT_EPI_STORE)};
    a[0].tag = "bwd_mlp_up_dx";
    MMDIT_TRY(linear(dt, a, 2, s));
  }
  // pre-MLP norm: dx_mid = dy + rms backward; da = gate1 * dx_mid
  float* dxmid = reinterpret_cast<float*>(base + Lb.dxmid);
  float* inv_r = reinterpret_cast<float*>(base + Lb.inv_r);
  {
    NormBwdSpec nb[2];
    for (int i = 0; i < 2; ++i)
      nb[i] = {nullptr, srows(S.x_mid, i, H), rows(Lb.dh2, i, H), mod[i], seg[i], dx[i], dxmid + (i ? ni * H : 0),
               inv_r + (i ? ni : 0), mod[i], rows(Lb.da, i, H), nr[i], 6 * H, 4 * H, 2 * H, 0, 1};
    MMDIT_TRY(norm_bwd2_impl(dt, H, d->eps, nb, 2, s));
  }
  float* partial = reinterpret_cast<float*>(base + Lb.partial);
  auto colsums = [&](int i, int nterms, const void* const* A, const void* const* Bm, const float* const* rs,
                     const int32_t* af, const int32_t* bf, const int32_t* off) -> mmdit_status {
    ColsumSpec sp;
    memset(&sp, 0, sizeof(sp));
    sp.nterms = nterms;
    for (int k = 0; k < nterms; ++k) {
      sp.a[k] = A[k];
      sp.b[k] = Bm[k];
      sp.rs[k] = rs[k];
      sp.a_f32[k] = af[k];
      sp.b_f32[k] = bf[k];
      sp.out_off[k] = off[k];
    }
    sp.cu = i ? pk->cu_txt : pk->cu_img;
    sp.h_cu = i ? pk->h_cu_txt : pk->h_cu_img;
    sp.B = pk->B;
    sp.H = H;
    sp.partial = partial;
    sp.out = dmod[i];
    sp.out_stride = 6 * H;
    return seg_colsum_impl(dt, sp, s);
  };
  for (int i = 0; i < 2; ++i) {
    // d shift2 = sum dh2, d scale2 = sum dh2 * rms(x_mid), d gate2 = sum dy * mlp_out
    const void* A[3] = {rows(Lb.dh2, i, H), rows(Lb.dh2, i, H), dx[i]};
    const void* Bm[3] = {nullptr, srows(S.x_mid, i, H), srows(S.dmlp, i, H)};
    const float* rs[3] = {nullptr, inv_r + (i ? ni : 0), nullptr};
    const int32_t af[3] = {0, 0, 0}, bf[3] = {0, 0, 0}, off[3] = {3 * H, 4 * H, 5 * H};
    MMDIT_TRY(colsums(i, 3, A, Bm, rs, af, bf, off));
    // d gate1 = sum dx_mid * attn_out
    const void* A1[1] = {dxmid + (i ? ni * H : 0)};
    const void* B1[1] = {srows(S.a, i, H)};
    const float* r1[1] = {nullptr};
    const int32_t af1[1] = {1}, bf1[1] = {0}, off1[1] = {2 * H};
    MMDIT_TRY(colsums(i, 1, A1, B1, r1, af1, bf1, off1));
  }
  // attention output projection: dO = da W_o, dW_o = da^T o
  {
    LinearArgs a[2] = {mk(ni, H, H, rows(Lb.da, 0, H), wt(Lb.wt_o, 0, 0), rows(Lb.dO, 0, H), MMDIT_EPI_STORE),
                       mk(nt, H, H, rows(Lb.da, 1, H), wt(Lb.wt_o, 1, (int64_t)H * H), rows(Lb.dO, 1, H), MMDIT_EPI_STORE)};
    MMDIT_TRY(fork());   // da ready
    a[0].tag = "bwd_out_proj_dx";
    MMDIT_TRY(linear(dt, a, 2, s));
    TransposeArgs ta[2];
    memset(ta, 0, sizeof(ta));
    for (int i = 0; i < 2; ++i) ta[i] = {rows(Lb.da, i, H), trows(Lb.daT, i, H), nullptr, nullptr, nullptr, H, nr[i], np[i], 0, H};
    MMDIT_TRY(transpose2_impl(dt, ta, 2, 0, sw));
    for (int i = 0; i < 2; ++i) ta[i] = {srows(S.o, i, H), trows(Lb.oT, i, H), nullptr, nullptr, nullptr, H, nr[i], np[i], 0, H};
    MMDIT_TRY(transpose2_impl(dt, ta, 2, 0, sw));
    const char* A[2] = {trows(Lb.daT, 0, H), trows(Lb.daT, 1, H)};
    const char* X[2] = {trows(Lb.oT, 0, H), trows(Lb.oT, 1, H)};
    float* dw[2] = {gr[0]->w_o, gr[1]->w_o};
    MMDIT_TRY(weight_grad(dt, H, H, np, A, X, dw, "bwd_out_proj_dw", sw));
  }
  // joint attention, then QK-norm + RoPE
  MMDIT_TRY(attention_bwd_impl(dt, pk, d->heads, D, srows(S.qkv, 0, 3 * H), srows(S.qkv, 1, 3 * H), srows(S.o, 0, H),
                               srows(S.o, 1, H), reinterpret_cast<const float*>(sv + S.lse), rows(Lb.dO, 0, H),
                               rows(Lb.dO, 1, H), rows(Lb.dqkv, 0, 3 * H), rows(Lb.dqkv, 1, 3 * H), base + Lb.attn,
                               Lb.end - Lb.attn, s));
  {
    float* gp = reinterpret_cast<float*>(base + Lb.gpart);
    QkBwdSpec q[2] = {{rows(Lb.dqkv, 0, 3 * H), srows(S.qk_raw, 0, 2 * H), pk->pos_img, w->img.g_q, w->img.g_k, gp,
                       g->img.g_q, g->img.g_k, ni},
                      {rows(Lb.dqkv, 1, 3 * H), srows(S.qk_raw, 1, 2 * H), nullptr, w->txt.g_q, w->txt.g_k,
                       gp + qk_bwd_blocks(ni) * 2 * D, g->txt.g_q, g->txt.g_k, nt}};
    MMDIT_TRY(qk_bwd2_impl(dt, d->heads, D, d->rope_dims, d->rope_theta, d->eps, q, 2, s));
  }
  // QKV projection: dW_qkv = dqkv^T h1, dh1 = dqkv W_qkv
  {
    MMDIT_TRY(fork());   // dqkv final (after the QK-norm backward)
    TransposeArgs ta[2];
    memset(ta, 0, sizeof(ta));
    for (int i = 0; i < 2; ++i) ta[i] = {rows(Lb.dqkv, i, 3 * H), trows(Lb.dqkvT, i, 3 * H), nullptr, nullptr, nullptr, 3 * H, nr[i], np[i], 0, 3 * H};
    MMDIT_TRY(transpose2_impl(dt, ta, 2, 0, sw));
    for (int i = 0; i < 2; ++i) ta[i] = {srows(S.h1, i, H), trows(Lb.h1T, i, H), nullptr, nullptr, nullptr, H, nr[i], np[i], 0, H};
    MMDIT_TRY(transpose2_impl(dt, ta, 2, 0, sw));
    const char* A[2] = {trows(Lb.dqkvT, 0, 3 * H), trows(Lb.dqkvT, 1, 3 * H)};
    const char* X[2] = {trows(Lb.h1T, 0, H), trows(Lb.h1T, 1, H)};
    float* dw[2] = {gr[0]->w_qkv, gr[1]->w_qkv};
    MMDIT_TRY(weight_grad(dt, 3 * H, H, np, A, X, dw, "bwd_qkv_dw", sw));
    LinearArgs a[2] = {mk(ni, H, 3 * H, rows(Lb.dqkv, 0, 3 * H), wt(Lb.wt_qkv, 0, 0), rows(Lb.dh1, 0, H), MMDIT_EPI_STORE),
                       mk(nt, H, 3 * H, rows(Lb.dqkv, 1, 3 * H), wt(Lb.wt_qkv, 1, (int64_t)3 * H * H), rows(Lb.dh1, 1, H),
                          MMDIT_EPI_STORE)};
    a[0].tag = "bwd_qkv_dx";
    MMDIT_TRY(linear(dt, a, 2, s));
  }
  // pre-attention norm: dx_in = dx_mid + rms backward (written over dy)
  {
    NormBwdSpec nb[2];
    for (int i = 0; i < 2; ++i)
      nb[i] = {nullptr, srows(S.x_in, i, H), rows(Lb.dh1, i, H), mod[i], seg[i], dxmid + (i ? ni * H : 0), dx[i],
               inv_r + (i ? ni : 0), nullptr, nullptr, nr[i], 6 * H, H, 0, 1, 0};
    MMDIT_TRY(norm_bwd2_impl(dt, H, d->eps, nb, 2, s));
  }
  for (int i = 0; i < 2; ++i) {
    // d shift1 = sum dh1, d scale1 = sum dh1 * rms(x_in)
    const void* A[2] = {rows(Lb.dh1, i, H), rows(Lb.dh1, i, H)};
    const void* Bm[2] = {nullptr, srows(S.x_in, i, H)};
    const float* rs[2] = {nullptr, inv_r + (i ? ni : 0)};
    const int32_t af[2] = {0, 0}, bf[2] = {0, 0}, off[2] = {0, H};
    MMDIT_TRY(colsums(i, 2, A, Bm, rs, af, bf, off));
  }
  // adaLN: dW_mod = d_mod^T SiLU(c), dc += (d_mod W_mod) SiLU'(c)
  const float* dm[2] = {dmod[0], dmod[1]};
  const void* wm[2] = {w->img.w_mod, w->txt.w_mod};
  float* dwm[2] = {g->img.w_mod, g->txt.w_mod};
  MMDIT_TRY(outer_vecmat_impl(dt, pk->B, 6 * H, H, 2, dm, wm, c, 0, 0, dwm, dc, base + Lb.modg, Lb.attn - Lb.modg, s));
  if (two) {   // s waits for every weight gradient
    hipEvent_t e = bwd_event(nfork);
    if (!e) {
      set_error("%s: could not create a stream event", who);
      return MMDIT_E_HIP;
    }
    MMDIT_TRY(hip_check(hipEventRecord(e, sw), "hipEventRecord"));
    MMDIT_TRY(hip_check(hipStreamWaitEvent(s, e, 0), "hipStreamWaitEvent"));
  }
  return MMDIT_OK;
}

}  // namespace

mmdit_status mmdit_block_bwd(const mmdit_dims* d, const mmdit_block_w* w, const mmdit_pack_t* pk, const void* c,
                             const void* saved, size_t saved_bytes, void* dx_img, void* dx_txt,
                             const mmdit_block_grad* g, float* dc, void* ws, size_t ws_bytes,
                             mmdit_stream stream) {
  return block_bwd_impl(d, w, pk, c, saved, saved_bytes, dx_img, dx_txt, g, dc, ws, ws_bytes, stream, nullptr,
                        "mmdit_block_bwd");
}

mmdit_status mmdit_block_bwd2(const mmdit_dims* d, const mmdit_block_w* w, const mmdit_pack_t* pk, const void* c,
                              const void* saved, size_t saved_bytes, void* dx_img, void* dx_txt,
                              const mmdit_block_grad* g, float* dc, void* ws, size_t ws_bytes,
                              mmdit_stream stream, mmdit_stream stream_w) {
  return block_bwd_impl(d, w, pk, c, saved, saved_bytes, dx_img, dx_txt, g, dc, ws, ws_bytes, stream, stream_w,
                        "mmdit_block_bwd2");
}

namespace {

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// bytes % 4 == 0; a kernel rather than a memset so the call can be captured in a graph
mmdit_status zero_bytes(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n <= 0) return MMDIT_OK;
  const int64_t blocks = cdiv(n, 256) < 4096 ? cdiv(n, 256) : 4096;
  MMDIT_LAUNCH(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), n);
  return launch_check("zero_words_kernel", s);
}

// Workspace of the final-layer and embedding backward calls.
struct WrapLayout {
  size_t modf, hf, dhf, inv_r, dvT, hfT, woT, partial, dmodf, ov, dxiT, ztT, dxtT, tauT, end;
};

WrapLayout wrap_layout(const mmdit_dims* d, const mmdit_pack_t* pk) {
  const size_t es = esize(d->dtype);
  const size_t H = d->hidden, C = d->c_lat, B = pk->B;
  const size_t ntp = pad64(pk->n_tgt), nip = pad64(pk->n_img), nxp = pad64(pk->n_txt);
  WrapLayout W;
  size_t o = 0;
  W.modf = o;    o = align256(o + B * 2 * H * 4);
  W.hf = o;      o = align256(o + (size_t)pk->n_tgt * H * es);
  W.dhf = o;     o = align256(o + (size_t)pk->n_tgt * H * es);
  W.inv_r = o;   o = align256(o + (size_t)pk->n_tgt * 4);
  W.dvT = o;     o = align256(o + C * ntp * es);
  W.hfT = o;     o = align256(o + H * ntp * es);
  W.woT = o;     o = align256(o + H * C * es);
  W.partial = o; o = align256(o + (size_t)colsum_chunks(pk->h_cu_tgt, pk->B, kColsumRows) * 2 * H * 4);
  W.dmodf = o;   o = align256(o + B * 2 * H * 4);
  size_t ov = outer_vecmat_ws_bytes(pk->B, 2 * d->hidden, d->hidden);
  W.ov = o;      o = align256(o + ov);
  W.dxiT = o;    o = align256(o + H * nip * es);
  W.ztT = o;     o = align256(o + C * nip * es);
  W.dxtT = o;    o = align256(o + H * nxp * es);
  W.tauT = o;    o = align256(o + (size_t)d->d_txt * nxp * es);
  W.end = o;
  return W;
}

mmdit_status check_ws(void* ws, size_t ws_bytes, size_t need_b, const char* who) {
  if (!ws || ws_bytes < need_b) {
    set_error("%s: workspace needs %zu bytes, got %zu", who, need_b, ws_bytes);
    return MMDIT_E_WORKSPACE;
  }
  return need(ws, who, "ws");
}

}  // namespace

mmdit_status rf_loss_grad(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* v, const void* z,
                          const void* eps, void* dv, mmdit_stream stream) {
  return loss_grad_impl(pk, dt, C, v, z, eps, dv, (hipStream_t)stream);
}

size_t mmdit_wrap_bwd_workspace_size(const mmdit_dims* d, const mmdit_pack_t* pk) {
  if (check_dims(d, "mmdit_wrap_bwd_workspace_size") != MMDIT_OK ||
      check_pack(pk, "mmdit_wrap_bwd_workspace_size") != MMDIT_OK)
    return 0;
  return wrap_layout(d, pk).end;
}

mmdit_status mmdit_final_bwd(const mmdit_dims* d, const void* w_fmod, const void* w_out, const mmdit_pack_t* pk,
                             const void* c, const void* x_img, const void* dv, void* dx_img, float* dw_fmod,
                             float* dw_out, float* dc, void* ws, size_t ws_bytes, mmdit_stream stream) {
  const char* who = "mmdit_final_bwd";
  MMDIT_TRY(check_dims(d, who));
  MMDIT_TRY(check_pack(pk, who));
  const void* req[] = {w_fmod, w_out, dw_fmod, dw_out};
  const char* nm[] = {"w_fmod", "w_out", "dw_fmod", "dw_out"};
  for (int i = 0; i < 4; ++i) MMDIT_TRY(need(req[i], who, nm[i]));
  const WrapLayout W = wrap_layout(d, pk);
  MMDIT_TRY(check_ws(ws, ws_bytes, W.end, who));
  hipStream_t s = (hipStream_t)stream;
  const mmdit_dtype dt = d->dtype;
  const int32_t H = d->hidden, C = d->c_lat;
  const int64_t nt = pk->n_tgt, ntp = pad64(pk->n_tgt);
  char* base = static_cast<char*>(ws);
  if (pk->n_img > 0) {
    MMDIT_TRY(need(dx_img, who, "dx_img"));
    MMDIT_TRY(zero_bytes(dx_img, (size_t)pk->n_img * H * esize(dt), s));
  }
  if (nt == 0 || pk->B == 0) {
    MMDIT_TRY(fill_zero(dw_out, (int64_t)C * H, s));
    return fill_zero(dw_fmod, (int64_t)2 * H * H, s);
  }
  MMDIT_TRY(need(c, who, "c"));
  MMDIT_TRY(need(dc, who, "dc"));
  MMDIT_TRY(need(x_img, who, "x_img"));
  MMDIT_TRY(need(dv, who, "dv"));
  float* modf = reinterpret_cast<float*>(base + W.modf);
  // recompute [shift, scale] = W_fmod SiLU(c) and h = rms(x_tgt)(1 + scale) + shift
  LinearArgs a = mk(pk->B, 2 * H, H, c, w_fmod, modf, MMDIT_EPI_STORE_F32);
  a.a_silu = 1;
  a.tag = "final_mod";
  MMDIT_TRY(linear(dt, &a, 1, s));
  MMDIT_TRY(rms_modulate_impl(dt, nt, H, x_img, pk->tgt_row, pk->seg_img, modf, 2 * H, 0, H, base + W.hf, d->eps, s));
  // dW_out = dv^T h, dh = dv W_out
  {
    TransposeArgs ta[1];
    memset(ta, 0, sizeof(ta));
    ta[0] = {dv, base + W.dvT, nullptr, nullptr, nullptr, C, nt, ntp, 0, C};
    MMDIT_TRY(transpose2_impl(dt, ta, 1, 0, s));
    ta[0] = {base + W.hf, base + W.hfT, nullptr, nullptr, nullptr, H, nt, ntp, 0, H};
    MMDIT_TRY(transpose2_impl(dt, ta, 1, 0, s));
    ta[0] = {w_out, base + W.woT, nullptr, nullptr, nullptr, H, C, C, 0, H};
    MMDIT_TRY(transpose2_impl(dt, ta, 1, 0, s));
    LinearArgs g = mk(C, H, (int32_t)ntp, base + W.dvT, base + W.hfT, dw_out, MMDIT_EPI_STORE_F32);
    g.tag = "bwd_final_out_dw";
    MMDIT_TRY(linear(dt, &g, 1, s));
    LinearArgs x = mk(nt, H, C, dv, base + W.woT, base + W.dhf, MMDIT_EPI_STORE);
    x.tag = "bwd_final_out_dx";
    MMDIT_TRY(linear(dt, &x, 1, s));
  }
  // through the norm of the target rows into dx_img; adaLN sums per sample
  float* inv_r = reinterpret_cast<float*>(base + W.inv_r);
  {
    NormBwdSpec nb = {pk->tgt_row, x_img, base + W.dhf, modf, pk->seg_img, nullptr, dx_img, inv_r, nullptr, nullptr,
                      nt, 2 * H, H, 0, 0, 0};
    MMDIT_TRY(norm_bwd2_impl(dt, H, d->eps, &nb, 1, s));
  }
  float* dmodf = reinterpret_cast<float*>(base + W.dmodf);
  {
    ColsumSpec sp;
    memset(&sp, 0, sizeof(sp));
    sp.nterms = 2;
    sp.a[0] = base + W.dhf;
    sp.a[1] = base + W.dhf;
    sp.b[1] = x_img;
    sp.b_map[1] = pk->tgt_row;
    sp.rs[1] = inv_r;
    sp.out_off[0] = 0;
    sp.out_off[1] = H;
    sp.cu = pk->cu_tgt;
    sp.h_cu = pk->h_cu_tgt;
    sp.B = pk->B;
    sp.H = H;
    sp.partial = reinterpret_cast<float*>(base + W.partial);
    sp.out = dmodf;
    sp.out_stride = 2 * H;
    MMDIT_TRY(seg_colsum_impl(dt, sp, s));
  }
  const float* dm[1] = {dmodf};
  const void* wm[1] = {w_fmod};
  float* dwm[1] = {dw_fmod};
  return outer_vecmat_impl(dt, pk->B, 2 * H, H, 1, dm, wm, c, 0, 0, dwm, dc, base + W.ov, W.dxiT - W.ov, s);
}

mmdit_status mmdit_embed_bwd(const mmdit_dims* d, const mmdit_pack_t* pk, const void* zt, const void* tau,
                             const void* dx_img, const void* dx_txt, float* dw_in, float* dw_txt, void* ws,
                             size_t ws_bytes, mmdit_stream stream) {
  const char* who = "mmdit_embed_bwd";
  MMDIT_TRY(check_dims(d, who));
  MMDIT_TRY(check_pack(pk, who));
  MMDIT_TRY(need(dw_in, who, "dw_in"));
  MMDIT_TRY(need(dw_txt, who, "dw_txt"));
  const WrapLayout W = wrap_layout(d, pk);
  MMDIT_TRY(check_ws(ws, ws_bytes, W.end, who));
  hipStream_t s = (hipStream_t)stream;
  const mmdit_dtype dt = d->dtype;
  const int32_t H = d->hidden, C = d->c_lat, T = d->d_txt;
  const int64_t ni = pk->n_img, nx = pk->n_txt, nip = pad64(ni), nxp = pad64(nx);
  char* base = static_cast<char*>(ws);
  LinearArgs a[2];
  int n = 0;
  if (ni > 0) {
    MMDIT_TRY(need(zt, who, "zt"));
    MMDIT_TRY(need(dx_img, who, "dx_img"));
    TransposeArgs ta[1];
    ta[0] = {dx_img, base + W.dxiT, nullptr, nullptr, nullptr, H, ni, nip, 0, H};
    MMDIT_TRY(transpose2_impl(dt, ta, 1, 0, s));
    ta[0] = {zt, base + W.ztT, nullptr, nullptr, nullptr, C, ni, nip, 0, C};
    MMDIT_TRY(transpose2_impl(dt, ta, 1, 0, s));
    a[n++] = mk(H, C, (int32_t)nip, base + W.dxiT, base + W.ztT, dw_in, MMDIT_EPI_STORE_F32);
  } else {
    MMDIT_TRY(fill_zero(dw_in, (int64_t)H * C, s));
  }
  if (nx > 0) {
    MMDIT_TRY(need(tau, who, "tau"));
    MMDIT_TRY(need(dx_txt, who, "dx_txt"));
    TransposeArgs ta[1];
    ta[0] = {dx_txt, base + W.dxtT, nullptr, nullptr, nullptr, H, nx, nxp, 0, H};
    MMDIT_TRY(transpose2_impl(dt, ta, 1, 0, s));
    ta[0] = {tau, base + W.tauT, nullptr, nullptr, nullptr, T, nx, nxp, 0, T};
    MMDIT_TRY(transpose2_impl(dt, ta, 1, 0, s));
    a[n++] = mk(H, T, (int32_t)nxp, base + W.dxtT, base + W.tauT, dw_txt, MMDIT_EPI_STORE_F32);
  } else {
    MMDIT_TRY(fill_zero(dw_txt, (int64_t)H * T, s));
  }
  if (n == 0) return MMDIT_OK;
  a[0].tag = "bwd_embed_dw";
  return linear(dt, a, n, s);
}

mmdit_status mmdit_cond_bwd(const mmdit_dims* d, const void* w_t1, const void* w_t2, const float* t, int32_t B,
                            const float* dc, float* dw_t1, float* dw_t2, void* ws, size_t ws_bytes,
                            mmdit_stream stream) {
  const char* who = "mmdit_cond_bwd";
  MMDIT_TRY(check_dims(d, who));
  if (B < 0 || B > MMDIT_MAX_SAMPLES) {
    set_error("%s: B=%d", who, B);
    return MMDIT_E_INVALID;
  }
  const void* req[] = {w_t1, w_t2, dw_t1, dw_t2};
  const char* nm[] = {"w_t1", "w_t2", "dw_t1", "dw_t2"};
  for (int i = 0; i < 4; ++i) MMDIT_TRY(need(req[i], who, nm[i]));
  hipStream_t s = (hipStream_t)stream;
  const int32_t H = d->hidden;
  if (B == 0) {
    MMDIT_TRY(fill_zero(dw_t1, (int64_t)H * d->t_dim, s));
    return fill_zero(dw_t2, (int64_t)H * H, s);
  }
  MMDIT_TRY(need4(t, who, "t"));
  MMDIT_TRY(need(dc, who, "dc"));
  const size_t es = esize(d->dtype);
  size_t ov = outer_vecmat_ws_bytes(B, H, H);
  const size_t ov3 = outer_vecmat_ws_bytes(B, H, d->t_dim);
  ov = align256(ov > ov3 ? ov : ov3);
  const size_t o_emb = ov, o_h1 = o_emb + align256((size_t)B * d->t_dim * es), o_dh = o_h1 + align256((size_t)B * H * es);
  MMDIT_TRY(check_ws(ws, ws_bytes, o_dh + (size_t)B * H * 4, who));
  char* base = static_cast<char*>(ws);
  // recompute emb(t) and h1 = W_t1 emb exactly as the forward
  MMDIT_TRY(temb_impl(d->dtype, B, d->t_dim, t, base + o_emb, s));
  LinearArgs a = mk(B, H, d->t_dim, base + o_emb, w_t1, base + o_h1, MMDIT_EPI_STORE);
  a.tag = "cond_mlp1";
  MMDIT_TRY(linear(d->dtype, &a, 1, s));
  float* dh = reinterpret_cast<float*>(base + o_dh);
  MMDIT_TRY(fill_zero(dh, (int64_t)B * H, s));
  // c = W_t2 SiLU(h1): dW_t2 = dc^T SiLU(h1), dh1 = (dc W_t2) SiLU'(h1); then dW_t1 = dh1^T emb
  const float* dy[1] = {dc};
  const void* w2[1] = {w_t2};
  float* dw2[1] = {dw_t2};
  MMDIT_TRY(outer_vecmat_impl(d->dtype, B, H, H, 1, dy, w2, base + o_h1, 0, 0, dw2, dh, base, ov, s));
  const float* dy1[1] = {dh};
  const void* w1[1] = {w_t1};
  float* dw1[1] = {dw_t1};
  return outer_vecmat_impl(d->dtype, B, H, d->t_dim, 1, dy1, w1, base + o_emb, 0, 1, dw1, nullptr, base, ov, s);
}

size_t mmdit_cond_bwd_workspace_size(const mmdit_dims* d, int32_t B) {
  if (check_dims(d, "mmdit_cond_bwd_workspace_size") != MMDIT_OK || B < 0) return 0;
  const size_t es = esize(d->dtype);
  size_t ov = outer_vecmat_ws_bytes(B, d->hidden, d->hidden);
  const size_t ov3 = outer_vecmat_ws_bytes(B, d->hidden, d->t_dim);
  ov = align256(ov > ov3 ? ov : ov3);
  return ov + align256((size_t)B * d->t_dim * es) + align256((size_t)B * d->hidden * es) + (size_t)B * d->hidden * 4;
}

namespace {

// Final layer after its modulation: h = rms(x)(1 + scale_f) + shift_f on the
// target rows, v = h W_out^T.  modf float32 [B][2H] (shift, scale).
mmdit_status final_rest_impl(const mmdit_dims* d, const void* w_out, const mmdit_pack_t* pk, const float* modf,
                             const void* x_img, void* v, void* ws, hipStream_t s, const void* sse_z = nullptr,
                             const void* sse_e = nullptr, float* row_sse = nullptr, int32_t* sse_done = nullptr) {
  const int32_t H = d->hidden;
  void* hf = static_cast<char*>(ws) + align256((size_t)pk->B * 2 * H * 4);
  MMDIT_TRY(rms_modulate_impl(d->dtype, pk->n_tgt, H, x_img, pk->tgt_row, pk->seg_img, modf, 2 * H, 0, H, hf,
                              d->eps, s));
  LinearArgs b = mk(pk->n_tgt, d->c_lat, H, hf, w_out, v, MMDIT_EPI_STORE);
  b.tag = "final_out";
  b.partial = reinterpret_cast<float*>(static_cast<char*>(hf) + align256((size_t)pk->n_tgt * H * esize(d->dtype)));
  b.partial_elems = (int64_t)8 * pk->n_tgt * d->c_lat;
  if (row_sse) {
    b.sse_z = sse_z;
    b.sse_e = sse_e;
    b.sse_row = pk->tgt_row;
    b.row_sse = row_sse;
    b.sse_done = sse_done;
  }
  return linear(d->dtype, &b, 1, s);
}

mmdit_status final_modulation_impl(const mmdit_dims* d, const void* w_fmod, int32_t B, const void* c, float* modf,
                                   hipStream_t s) {
  LinearArgs a = mk(B, 2 * d->hidden, d->hidden, c, w_fmod, modf, MMDIT_EPI_STORE_F32);
  a.a_silu = 1;
  a.tag = "final_mod";
  return linear(d->dtype, &a, 1, s);
}

mmdit_status check_final_args(const mmdit_dims* d, const void* w_out, const mmdit_pack_t* pk, const void* x_img,
                              void* v, void* ws, size_t ws_bytes, const char* who) {
  MMDIT_TRY(check_dims(d, who));
  MMDIT_TRY(check_pack(pk, who));
  if (pk->n_tgt == 0) return MMDIT_OK;
  MMDIT_TRY(need(w_out, who, "w_out"));
  MMDIT_TRY(need(x_img, who, "x_img"));
  MMDIT_TRY(need(v, who, "v"));
  const size_t need_b = final_ws(d, pk);
  if (!ws || ws_bytes < need_b) {
    set_error("%s: workspace needs %zu bytes, got %zu", who, need_b, ws_bytes);
    return MMDIT_E_WORKSPACE;
  }
  return need(ws, who, "ws");
}

}  // namespace

mmdit_status mmdit_final(const mmdit_dims* d, const void* w_fmod, const void* w_out, const mmdit_pack_t* pk,
                         const void* c, const void* x_img, void* v, void* ws, size_t ws_bytes, mmdit_stream stream) {
  const char* who = "mmdit_final";
  MMDIT_TRY(check_final_args(d, w_out, pk, x_img, v, ws, ws_bytes, who));
  if (pk->n_tgt == 0) return MMDIT_OK;
  MMDIT_TRY(need(w_fmod, who, "w_fmod"));
  MMDIT_TRY(need(c, who, "c"));
  hipStream_t s = (hipStream_t)stream;
  float* modf = static_cast<float*>(ws);
  MMDIT_TRY(final_modulation_impl(d, w_fmod, pk->B, c, modf, s));
  return final_rest_impl(d, w_out, pk, modf, x_img, v, ws, s);
}

mmdit_status mmdit_final_mod(const mmdit_dims* d, const void* w_out, const mmdit_pack_t* pk, const float* modf,
                             const void* x_img, void* v, void* ws, size_t ws_bytes, mmdit_stream stream) {
  const char* who = "mmdit_final_mod";
  MMDIT_TRY(check_final_args(d, w_out, pk, x_img, v, ws, ws_bytes, who));
  if (pk->n_tgt == 0) return MMDIT_OK;
  MMDIT_TRY(need(modf, who, "modf"));
  return final_rest_impl(d, w_out, pk, modf, x_img, v, ws, (hipStream_t)stream);
}

mmdit_status rf_make_xt(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* z, const void* eps,
                        const float* t, void* zt, mmdit_stream stream) {
  return make_xt_impl(pk, dt, C, z, eps, t, zt, (hipStream_t)stream);
}

mmdit_status rf_embed(const mmdit_dims* d, const void* w_in, const void* w_txt, const mmdit_pack_t* pk,
                      const void* z, const void* eps, const float* t, const void* tau, void* x_img, void* x_txt,
                      void* zt, mmdit_stream stream) {
  const char* who = "rf_embed";
  MMDIT_TRY(check_dims(d, who));
  MMDIT_TRY(check_pack(pk, who));
  hipStream_t s = (hipStream_t)stream;
  if (pk->n_txt > 0) {
    MMDIT_TRY(need(w_txt, who, "w_txt"));
    MMDIT_TRY(need(tau, who, "tau"));
    MMDIT_TRY(need(x_txt, who, "x_txt"));
    LinearArgs a = mk(pk->n_txt, d->hidden, d->d_txt, tau, w_txt, x_txt, MMDIT_EPI_STORE);
    a.tag = "embed_txt";
    MMDIT_TRY(linear(d->dtype, &a, 1, s));
  }
  if (pk->n_img == 0) return MMDIT_OK;
  MMDIT_TRY(need(w_in, who, "w_in"));
  MMDIT_TRY(need(z, who, "z"));
  MMDIT_TRY(need(eps, who, "eps"));
  MMDIT_TRY(need(t, who, "t"));
  MMDIT_TRY(need(x_img, who, "x_img"));
  MMDIT_TRY(need(zt, who, "zt"));
  if (d->dtype == MMDIT_BF16 && d->c_lat % 64 == 0 && d->hidden % 128 == 0) {
    // the noising in the A staging of the embedding GEMM (which also writes zt)
    LinearArgs a = mk(pk->n_img, d->hidden, d->c_lat, z, w_in, x_img, MMDIT_EPI_STORE);
    a.tag = "embed_img_xt";
    XtArgs x = {eps, t, pk->seg_img, pk->pos_img, zt};
    return linear_xt(a, x, s);
  }
  MMDIT_TRY(make_xt_impl(pk, d->dtype, d->c_lat, z, eps, t, zt, s));
  LinearArgs a = mk(pk->n_img, d->hidden, d->c_lat, zt, w_in, x_img, MMDIT_EPI_STORE);
  a.tag = "embed_img";
  return linear(d->dtype, &a, 1, s);
}

mmdit_status rf_final_loss(const mmdit_dims* d, const void* w_out, const mmdit_pack_t* pk, const float* modf,
                           const void* x_img, const void* z, const void* eps, void* v, float* sse, float* loss,
                           void* ws, size_t ws_bytes, mmdit_stream stream) {
  const char* who = "rf_final_loss";
  MMDIT_TRY(check_dims(d, who));
  MMDIT_TRY(check_pack(pk, who));
  MMDIT_TRY(need(loss, who, "loss"));
  if (pk->B > 0) MMDIT_TRY(need(sse, who, "sse"));
  const size_t fb = final_ws(d, pk), lb = align256((size_t)pk->n_tgt * 4 + 4);
  if (!ws || ws_bytes < fb + lb) {
    set_error("%s: workspace needs %zu bytes, got %zu", who, fb + lb, ws_bytes);
    return MMDIT_E_WORKSPACE;
  }
  hipStream_t s = (hipStream_t)stream;
  float* row_sse = reinterpret_cast<float*>(static_cast<char*>(ws) + fb);
  if (pk->n_tgt > 0) {
    MMDIT_TRY(check_final_args(d, w_out, pk, x_img, v, ws, ws_bytes, who));
    MMDIT_TRY(need(modf, who, "modf"));
    MMDIT_TRY(need(z, who, "z"));
    MMDIT_TRY(need(eps, who, "eps"));
    // the row sums ride in the final GEMM's split-K reduction when it has one
    int32_t done = 0;
    MMDIT_TRY(final_rest_impl(d, w_out, pk, modf, x_img, v, ws, s, z, eps, row_sse, &done));
    if (!done) MMDIT_TRY(row_sse_impl(pk, d->dtype, d->c_lat, v, z, eps, row_sse, s));
  }
  return loss_finalize_impl(pk, d->c_lat, row_sse, sse, loss, s);
}

mmdit_status rf_loss(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* v, const void* z,
                     const void* eps, float* sse, float* loss, void* ws, size_t ws_bytes, mmdit_stream stream) {
  return loss_impl(pk, dt, C, v, z, eps, sse, loss, ws, ws_bytes, (hipStream_t)stream);
}

mmdit_status rf_loss_noalloc(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* v, const void* z,
                             const void* eps, float* sse, float* loss, mmdit_stream stream) {
  return loss_noalloc_impl(pk, dt, C, v, z, eps, sse, loss, (hipStream_t)stream);
}

mmdit_status rf_nft_loss(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* v_pos, const void* v_neg,
                         const void* z, const void* eps, const float* r, float* sse, float* loss, void* ws,
                         size_t ws_bytes, mmdit_stream stream) {
  return nft_loss_impl(pk, dt, C, v_pos, v_neg, z, eps, r, sse, loss, ws, ws_bytes, (hipStream_t)stream);
}

mmdit_status rf_euler_step(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const void* v, int32_t cond_b,
                           int32_t uncond_b, float guidance, float t_cur, float t_next, float* z, void* zt_next,
                           mmdit_stream stream) {
  return euler_impl(pk, dt, C, v, cond_b, uncond_b, guidance, t_cur, t_next, z, zt_next, (hipStream_t)stream);
}

mmdit_status rf_pack_latent(const mmdit_pack_t* pk, mmdit_dtype dt, int32_t C, const float* z, int32_t b0,
                            int32_t b1, void* zt, mmdit_stream stream) {
  return pack_latent_impl(pk, dt, C, z, b0, b1, zt, (hipStream_t)stream);
}

}  // extern "C"
