// C ABI of libattnbwd.so (declared in include/attn_bwd.h): argument
// validation, translation to the kernels' parameter block, and dispatch.
//
// Validation happens before any HIP call; a call that fails validation has
// no effect on the device.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/attn_bwd.h"
#include "kernels.h"

using attn::Params;

// Device scratch of attn_bwd_static: the partial dK / dV sums of split key
// blocks (or query-head parts) that attn_bwd keeps in a caller workspace.
// Each GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` is only a stand-in for the symbol: its device
// address on a GPU comes from hipGetSymbolAddress with that GPU current
// (static_scratch below), and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[ATTN_STATIC_SCRATCH_BYTES];

namespace {

// Per-device address of `scratch`, looked up once per device.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The scratch of the device that `stream` runs on (the current device for
// the null stream), looked up with that device current.
attn_status_t static_scratch(void* stream, void** out) {
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return ATTN_EHIP;
  dev = cur;
  if (stream != nullptr && hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return ATTN_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_EUNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev, cur]() {
    void* ptr = nullptr;
    hipError_t e = dev == cur ? hipSuccess : hipSetDevice(dev);
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess && e == hipSuccess) e = hipErrorInvalidDevice;
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return ATTN_EHIP;
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

constexpr int kMaxHeadDim = 512;

bool strides_ok(const int64_t* s) { return s[0] >= 0 && s[1] >= 0 && s[2] >= 0; }

// Shape / mask checks shared by the forward and the backward.
attn_status_t check_problem(const attn_problem_t* p) {
  if (!p) return ATTN_EINVAL;
  if (p->B < 0 || p->Hq <= 0 || p->Hk <= 0 || p->Sq < 0 || p->Sk < 0) return ATTN_EINVAL;
  if (p->Hq % p->Hk != 0) return ATTN_EINVAL;
  if (p->Dqk <= 0 || p->Dv <= 0 || p->Dqk > kMaxHeadDim || p->Dv > kMaxHeadDim) return ATTN_EINVAL;
  if (!(p->scale > 0.f) || !isfinite(p->scale)) return ATTN_EINVAL;
  if (p->in_dtype != ATTN_F32 && p->in_dtype != ATTN_BF16) return ATTN_EINVAL;
  if (p->o_dtype != ATTN_F32 && p->o_dtype != ATTN_BF16) return ATTN_EINVAL;
  if (p->mask != ATTN_MASK_NONE && p->mask != ATTN_MASK_TOP_LEFT && p->mask != ATTN_MASK_BOTTOM_RIGHT)
    return ATTN_EINVAL;
  if (p->window_left < -1 || p->window_right < 0 || p->num_sink_tokens < 0) return ATTN_EINVAL;
  if (p->mask == ATTN_MASK_NONE && (p->window_left != -1 || p->window_right != 0 || p->num_sink_tokens != 0))
    return ATTN_EINVAL;
  if (p->q_offset < 0 || p->k_offset < 0 || p->sq_total < 0 || p->sk_total < 0) return ATTN_EINVAL;
  const int64_t sq_t = p->sq_total ? p->sq_total : p->Sq;
  const int64_t sk_t = p->sk_total ? p->sk_total : p->Sk;
  if (p->q_offset + p->Sq > sq_t || p->k_offset + p->Sk > sk_t) return ATTN_EINVAL;
  // the kernels evaluate the mask in 32-bit global indices
  if (sq_t >= (int64_t(1) << 30) || sk_t >= (int64_t(1) << 30)) return ATTN_EUNSUPPORTED;
  if ((p->cu_seqlens_q == nullptr) != (p->cu_seqlens_k == nullptr)) return ATTN_EINVAL;
  if (p->cu_seqlens_q) {
    if (p->q_offset || p->k_offset || p->sq_total || p->sk_total) return ATTN_EINVAL;
    if (p->total_q < 0 || p->total_k < 0) return ATTN_EINVAL;
    if (p->total_q >= (int64_t(1) << 31) || p->total_k >= (int64_t(1) << 31)) return ATTN_EUNSUPPORTED;
  }
  return ATTN_OK;
}

bool packed(const attn_problem_t* p) { return p->cu_seqlens_q != nullptr; }

// dbias is written through the bias strides: its rows (and heads) must not
// overlap, or two query rows (heads) would write one element -- a broadcast
// (stride 0) bias is fine to read but has no room for its gradient.
bool dbias_strides_ok(const attn_problem_t* p) {
  const int64_t row_span = (p->Sq > 0 ? (int64_t)(p->Sq - 1) * p->bias_str[1] : 0) + p->Sk;
  if (p->Sq > 1 && p->bias_str[1] < p->Sk) return false;
  if (p->Hq > 1 && p->bias_str[0] < row_span) return false;
  return true;
}

bool aligned16(const void* x) { return ((uintptr_t)x & 15u) == 0; }

Params make_params(const attn_problem_t* p) {
  Params k{};
  k.B = p->B; k.Hq = p->Hq; k.Hk = p->Hk; k.G = p->Hq / p->Hk;
  k.Sq = p->Sq; k.Sk = p->Sk; k.Dqk = p->Dqk; k.Dv = p->Dv;
  k.scale = p->scale;
  const int64_t sq_t = p->sq_total ? p->sq_total : p->Sq;
  const int64_t sk_t = p->sk_total ? p->sk_total : p->Sk;
  k.mask.kind = p->mask;
  k.mask.wl = p->window_left;
  k.mask.wr = p->window_right;
  k.mask.n_sink = p->num_sink_tokens;
  k.mask.q_off = p->q_offset;
  k.mask.k_off = p->k_offset;
  k.mask.diag = (p->mask == ATTN_MASK_BOTTOM_RIGHT) ? (sk_t - sq_t) : 0;
  for (int i = 0; i < 3; ++i) {
    k.q_str[i] = p->q_str[i]; k.k_str[i] = p->k_str[i]; k.v_str[i] = p->v_str[i];
    k.o_str[i] = p->o_str[i]; k.do_str[i] = p->do_str[i]; k.dq_str[i] = p->dq_str[i];
    k.dk_str[i] = p->dk_str[i]; k.dv_str[i] = p->dv_str[i];
  }
  k.bias_str[0] = p->bias_str[0];
  k.bias_str[1] = p->bias_str[1];
  k.cu_q = p->cu_seqlens_q;
  k.cu_k = p->cu_seqlens_k;
  k.tot_q = p->total_q;
  k.tot_k = p->total_k;
  return k;
}

// dK / dV (or any k-side tensor) as rows to zero: [B, H, Sk] dense, or the
// packed rows [total_k] of a variable-length batch.
attn::ZeroRows ksite_rows(const attn_problem_t* p, float* x, int D, const int64_t* str) {
  if (packed(p)) return attn::ZeroRows{x, 1, p->Hk, (int)p->total_k, D, {0, str[1], str[2]}};
  return attn::ZeroRows{x, p->B, p->Hk, p->Sk, D, {str[0], str[1], str[2]}};
}

attn_status_t hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_EHIP; }

// k and v name the same tensor: one pointer, one set of strides
bool same_kv(const attn_problem_t* p, const void* k, const void* v) {
  return k == v && p->k_str[0] == p->v_str[0] && p->k_str[1] == p->v_str[1] && p->k_str[2] == p->v_str[2];
}

// attn_bwd with one tensor as keys and values (ATTN_SHARED_KV): head dim 512,
// bf16, no bias; dk receives the gradient of the shared tensor.
attn_status_t bwd_shared_kv(const attn_problem_t* p, const void* q, const void* k, const void* v,
                            const void* dout, const float* lse, const float* delta, const float* bias,
                            float* dq, float* dk, float* dv, float* dbias, uint32_t flags, void* stream,
                            bool launch) {
  if (!(flags & ATTN_SHARED_KV) || p->Dqk != attn::kSharedKvD || p->Dv != attn::kSharedKvD ||
      p->in_dtype != ATTN_BF16 || bias || dbias)
    return ATTN_EUNSUPPORTED;
  if (dv || !same_kv(p, k, v)) return ATTN_EINVAL;
  if (!strides_ok(p->q_str) || !strides_ok(p->k_str) || !strides_ok(p->do_str) || !strides_ok(p->dq_str) ||
      !strides_ok(p->dk_str))
    return ATTN_EINVAL;
  const bool no_rows = p->B == 0 || p->Sq == 0;
  const bool no_keys = p->B == 0 || p->Sk == 0;
  if (!no_rows && (!q || !dout || !lse || !delta || !dq)) return ATTN_EINVAL;
  if (!no_keys && (!k || !dk)) return ATTN_EINVAL;
  Params kp = make_params(p);
  if (!attn::mla_supported(kp) || (!no_rows && (!aligned16(q) || !aligned16(dout) || !aligned16(dq))) ||
      (!no_keys && (!aligned16(k) || !aligned16(dk))))
    return ATTN_EUNSUPPORTED;
  if (no_rows && no_keys) return ATTN_OK;
  if (!launch) return ATTN_OK;
  attn::BwdArgs a{q, k, k, dout, lse, delta, nullptr, dq, dk, nullptr, nullptr,
                  (flags & ATTN_ACCUMULATE_DQ) ? 1 : 0, (flags & ATTN_DETERMINISTIC) ? 1 : 0,
                  (flags & ATTN_ACCUMULATE_DKDV) ? 1 : 0, 0};
  a.workspace = p->workspace_bytes > 0 ? p->workspace : nullptr;
  a.workspace_bytes = p->workspace_bytes;
  return hip_status(attn::launch_bwd512(kp, a, (hipStream_t)stream));
}

// attn_bwd: validation, then (when `launch`) the kernels.  With launch false
// the call only validates: no HIP call is made.
attn_status_t bwd_impl(const attn_problem_t* p, const void* q, const void* k, const void* v,
                       const void* dout, const float* lse, const float* delta, const float* bias,
                       float* dq, float* dk, float* dv, float* dbias, uint32_t flags, void* stream,
                       bool launch) {
  attn_status_t st = check_problem(p);
  if (st != ATTN_OK) return st;
  if ((flags & ~(uint32_t)(ATTN_DETERMINISTIC | ATTN_ACCUMULATE_DQ | ATTN_ACCUMULATE_DKDV | ATTN_SHARED_KV)) != 0)
    return ATTN_EINVAL;
  if ((flags & ATTN_SHARED_KV) || p->Dqk == attn::kSharedKvD || p->Dv == attn::kSharedKvD)
    return bwd_shared_kv(p, q, k, v, dout, lse, delta, bias, dq, dk, dv, dbias, flags, stream, launch);
  if (!strides_ok(p->q_str) || !strides_ok(p->k_str) || !strides_ok(p->v_str) || !strides_ok(p->do_str) ||
      !strides_ok(p->dq_str) || !strides_ok(p->dk_str) || !strides_ok(p->dv_str))
    return ATTN_EINVAL;
  if (dbias && !bias) return ATTN_EINVAL;
  if (bias && (p->bias_str[0] < 0 || p->bias_str[1] < 0)) return ATTN_EINVAL;
  if (dbias && !dbias_strides_ok(p)) return ATTN_EINVAL;
  const bool no_rows = p->B == 0 || p->Sq == 0;
  const bool no_keys = p->B == 0 || p->Sk == 0;
  if (!no_rows && (!q || !dout || !lse || !delta || !dq)) return ATTN_EINVAL;
  if (!no_keys && (!k || !v || !dk || !dv)) return ATTN_EINVAL;
  if (p->in_dtype == ATTN_F32 && (p->Dqk > attn::kSimtMaxD || p->Dv > attn::kSimtMaxD))
    return ATTN_EUNSUPPORTED;

  Params kp = make_params(p);
  attn::BwdArgs a{q, k, v, dout, lse, delta, bias, dq, dk, dv, dbias,
                  (flags & ATTN_ACCUMULATE_DQ) ? 1 : 0, (flags & ATTN_DETERMINISTIC) ? 1 : 0,
                  (flags & ATTN_ACCUMULATE_DKDV) ? 1 : 0};
  a.workspace = p->workspace_bytes > 0 ? p->workspace : nullptr;
  a.workspace_bytes = p->workspace_bytes;
  hipStream_t s = (hipStream_t)stream;
  if (p->in_dtype == ATTN_BF16) {
    if (!attn::mfma_bwd_supported(kp)) {
      if (p->Dqk > attn::kSimtMaxD || p->Dv > attn::kSimtMaxD) return ATTN_EUNSUPPORTED;
    }
  }
  // a packed batch runs on the matrix-core kernels only
  if (packed(p) && (bias || p->in_dtype != ATTN_BF16 || !attn::mfma_bwd_supported(kp) || !aligned16(q) ||
                    !aligned16(k) || !aligned16(v) || !aligned16(dout)))
    return ATTN_EUNSUPPORTED;
  if (no_rows && no_keys) return ATTN_OK;
  if (!launch) return ATTN_OK;
  if (p->in_dtype == ATTN_BF16 && attn::mfma_bwd_supported(kp))
    return hip_status(attn::launch_bwd_mfma(kp, a, s));
  // fp32 inputs (and bf16 shapes the matrix-core kernels do not cover)
  if (no_keys) {  // no keys: dK/dV are empty, dQ gets nothing added
    if (!a.accumulate_dq) return hip_status(attn::launch_zero_rows(dq, p->B, p->Hq, p->Sq, p->Dqk, p->dq_str, s));
    return ATTN_OK;
  }
  return hip_status(attn::launch_bwd_simt(kp, a, p->in_dtype == ATTN_BF16, s));
}

}  // namespace

extern "C" {

void attn_problem_init(attn_problem_t* p, int32_t B, int32_t Hq, int32_t Hk, int32_t Sq, int32_t Sk,
                       int32_t Dqk, int32_t Dv) {
  if (!p) return;
  *p = attn_problem_t{};
  p->B = B; p->Hq = Hq; p->Hk = Hk; p->Sq = Sq; p->Sk = Sk; p->Dqk = Dqk; p->Dv = Dv;
  p->scale = Dqk > 0 ? 1.0f / sqrtf((float)Dqk) : 0.f;
  p->in_dtype = ATTN_BF16;
  p->o_dtype = ATTN_F32;
  p->mask = ATTN_MASK_NONE;
  p->window_left = -1;
  p->window_right = 0;
  p->num_sink_tokens = 0;
  auto fill = [](int64_t* s, int64_t H, int64_t S, int64_t D) { s[0] = H * S * D; s[1] = S * D; s[2] = D; };
  fill(p->q_str, Hq, Sq, Dqk);
  fill(p->o_str, Hq, Sq, Dv);
  fill(p->do_str, Hq, Sq, Dv);
  fill(p->dq_str, Hq, Sq, Dqk);
  fill(p->k_str, Hk, Sk, Dqk);
  fill(p->dk_str, Hk, Sk, Dqk);
  fill(p->v_str, Hk, Sk, Dv);
  fill(p->dv_str, Hk, Sk, Dv);
  p->bias_str[0] = (int64_t)Sq * Sk;
  p->bias_str[1] = Sk;
}

const char* attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported problem";
    case ATTN_EHIP: return "HIP runtime error";
    case ATTN_ENOSCRATCH: return "problem needs more device scratch than attn_bwd_static holds";
  }
  return "unknown status";
}

attn_status_t attn_fwd_lse(const attn_problem_t* p, const void* q, const void* k, const void* v,
                           const float* bias, const float* sinks, void* o, float* lse, void* stream) {
  attn_status_t st = check_problem(p);
  if (st != ATTN_OK) return st;
  if (!strides_ok(p->q_str) || !strides_ok(p->k_str) || !strides_ok(p->v_str) || !strides_ok(p->o_str))
    return ATTN_EINVAL;
  const bool empty = p->B == 0 || p->Sq == 0;
  if (!empty && (!q || !o || !lse)) return ATTN_EINVAL;
  if (!empty && p->Sk > 0 && (!k || !v)) return ATTN_EINVAL;
  if (bias && (p->bias_str[0] < 0 || p->bias_str[1] < 0)) return ATTN_EINVAL;
  const bool o_bf16 = p->o_dtype == ATTN_BF16;
  if (p->Dqk == attn::kSharedKvD || p->Dv == attn::kSharedKvD) {
    // head dim 512: one tensor as keys and values, bf16, no bias
    if (p->Dqk != p->Dv || p->in_dtype != ATTN_BF16 || bias || !same_kv(p, k, v)) return ATTN_EUNSUPPORTED;
    Params kp = make_params(p);
    if (!attn::mla_supported(kp) || !aligned16(q) || !aligned16(k) || ((uintptr_t)o & (o_bf16 ? 7u : 15u)))
      return ATTN_EUNSUPPORTED;
    if (empty) return ATTN_OK;
    attn::FwdArgs a{q, k, v, bias, sinks, o, lse};
    return hip_status(attn::launch_fwd512(kp, a, o_bf16, (hipStream_t)stream));
  }
  if (p->Dqk > attn::kSimtMaxD || p->Dv > attn::kSimtMaxD) return ATTN_EUNSUPPORTED;
  if (empty) return ATTN_OK;
  Params kp = make_params(p);
  attn::FwdArgs a{q, k, v, bias, sinks, o, lse};
  const bool mfma = p->in_dtype == ATTN_BF16 && attn::mfma_fwd_supported(kp, a, o_bf16);
  if (packed(p) && (!mfma || bias)) return ATTN_EUNSUPPORTED;
  if (mfma) return hip_status(attn::launch_fwd_mfma(kp, a, o_bf16, (hipStream_t)stream));
  return hip_status(attn::launch_fwd_simt(kp, a, p->in_dtype == ATTN_BF16, o_bf16, (hipStream_t)stream));
}

attn_status_t attn_bwd_preprocess(const attn_problem_t* p, const void* o, const void* dout,
                                  const float* lse, const float* sinks, float* delta, float* dsinks,
                                  float* dq_zero, float* dk_zero, float* dv_zero, void* stream) {
  attn_status_t st = check_problem(p);
  if (st != ATTN_OK) return st;
  if (!strides_ok(p->o_str) || !strides_ok(p->do_str)) return ATTN_EINVAL;
  if (dq_zero && !strides_ok(p->dq_str)) return ATTN_EINVAL;
  if ((dk_zero && !strides_ok(p->dk_str)) || (dv_zero && !strides_ok(p->dv_str))) return ATTN_EINVAL;
  if ((sinks == nullptr) != (dsinks == nullptr)) return ATTN_EINVAL;
  const bool empty = p->B == 0 || p->Sq == 0;
  if (!empty && (!o || !dout || !delta)) return ATTN_EINVAL;
  if (sinks && !empty && !lse) return ATTN_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const attn::Packed pk{p->cu_seqlens_q, p->total_q};
  if (!empty) {
    hipError_t e = attn::launch_delta(o, p->o_dtype == ATTN_BF16, dout, p->in_dtype == ATTN_BF16, delta,
                                      p->B, p->Hq, p->Sq, p->Dv, p->o_str, p->do_str, dq_zero, p->Dqk,
                                      p->dq_str, pk, s);
    if (e != hipSuccess) return ATTN_EHIP;
  }
  if (dk_zero || dv_zero) {
    attn::ZeroRows z[2];
    int nz = 0;
    if (dk_zero) z[nz++] = ksite_rows(p, dk_zero, p->Dqk, p->dk_str);
    if (dv_zero) z[nz++] = ksite_rows(p, dv_zero, p->Dv, p->dv_str);
    if (attn::launch_zero_multi(z, nz, s) != hipSuccess) return ATTN_EHIP;
  }
  if (sinks) return hip_status(attn::launch_dsinks(lse, delta, sinks, dsinks, p->B, p->Hq, p->Sq, pk, s));
  return ATTN_OK;
}

attn_status_t attn_bwd(const attn_problem_t* p, const void* q, const void* k, const void* v,
                       const void* dout, const float* lse, const float* delta, const float* bias,
                       float* dq, float* dk, float* dv, float* dbias, uint32_t flags, void* stream) {
  return bwd_impl(p, q, k, v, dout, lse, delta, bias, dq, dk, dv, dbias, flags, stream, true);
}

attn_status_t attn_bwd_static(const attn_problem_t* p, const void* q, const void* k, const void* v,
                              const void* dout, const float* lse, const float* delta, const float* bias,
                              float* dq, float* dk, float* dv, float* dbias, uint32_t flags, void* stream) {
  // every host-side check first: no HIP call for an invalid or oversized problem
  attn_status_t st = bwd_impl(p, q, k, v, dout, lse, delta, bias, dq, dk, dv, dbias, flags, stream, false);
  if (st != ATTN_OK) return st;
  int64_t need = 0;
  st = attn_bwd_workspace_size(p, flags, &need);
  if (st != ATTN_OK) return st;
  if (need > (int64_t)ATTN_STATIC_SCRATCH_BYTES) return ATTN_ENOSCRATCH;
  attn_problem_t ps = *p;
  ps.workspace = nullptr;
  ps.workspace_bytes = 0;
  if (need > 0) {
    // every slot a call reads is stored by that call first: no zeroing
    st = static_scratch(stream, &ps.workspace);
    if (st != ATTN_OK) return st;
    ps.workspace_bytes = (int64_t)ATTN_STATIC_SCRATCH_BYTES;
  }
  return bwd_impl(&ps, q, k, v, dout, lse, delta, bias, dq, dk, dv, dbias, flags, stream, true);
}

attn_status_t attn_bwd_workspace_size(const attn_problem_t* p, uint32_t flags, int64_t* bytes) {
  if (!bytes) return ATTN_EINVAL;
  *bytes = 0;
  attn_status_t st = check_problem(p);
  if (st != ATTN_OK) return st;
  if ((flags & ~(uint32_t)(ATTN_DETERMINISTIC | ATTN_ACCUMULATE_DQ | ATTN_ACCUMULATE_DKDV | ATTN_SHARED_KV)) != 0)
    return ATTN_EINVAL;
  // the bf16 matrix-core paths of attn_bwd keep partial sums
  const Params kp = make_params(p);
  if ((flags & ATTN_SHARED_KV) || p->Dqk == attn::kSharedKvD || p->Dv == attn::kSharedKvD) {
    if ((flags & ATTN_SHARED_KV) && p->in_dtype == ATTN_BF16 && p->Dqk == attn::kSharedKvD &&
        p->Dv == attn::kSharedKvD && attn::mla_supported(kp))
      *bytes = attn::bwd512_workspace_bytes(kp, (flags & ATTN_DETERMINISTIC) != 0,
                                            (flags & ATTN_ACCUMULATE_DKDV) != 0);
    return ATTN_OK;
  }
  if (p->in_dtype != ATTN_BF16 || !attn::mfma_bwd_supported(kp)) return ATTN_OK;
  *bytes = attn::bwd_workspace_bytes(kp, (flags & ATTN_ACCUMULATE_DKDV) != 0, (flags & ATTN_DETERMINISTIC) != 0);
  return ATTN_OK;
}

attn_status_t attn_lse_merge(int32_t B, int32_t H, int32_t Sq, int32_t Dv, float* o_acc, float* lse_acc,
                             const float* o_part, const float* lse_part, void* stream) {
  if (B < 0 || H < 0 || Sq < 0 || Dv <= 0) return ATTN_EINVAL;
  const int64_t rows = (int64_t)B * H * Sq;
  if (rows == 0) return ATTN_OK;
  if (!o_acc || !lse_acc || !o_part || !lse_part) return ATTN_EINVAL;
  return hip_status(attn::launch_lse_merge(rows, Dv, o_acc, lse_acc, o_part, lse_part, (hipStream_t)stream));
}

}  // extern "C"
