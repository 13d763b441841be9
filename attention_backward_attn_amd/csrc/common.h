// Shared device-side definitions of the attention kernels: launch parameter
// block, mask predicate and row / key ranges, bf16 helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

enum MaskKind : int { kMaskNone = 0, kMaskTopLeft = 1, kMaskBottomRight = 2 };

// The mask in global coordinates (CK FMHA example 22 masks; bottom-right
// alignment of the CANN sparse_flash_mla_grad example).  For local row i and
// key j: i' = i + q_off, j' = j + k_off; allowed when
//   i' + diag - wl <= j' <= i' + diag + wr  (wl < 0: no lower bound)  or  j' < n_sink.
struct Mask {
  int kind;
  int wl, wr, n_sink;
  int64_t q_off, k_off, diag;

  __host__ __device__ inline bool allowed(int64_t i, int64_t j) const {
    if (kind == kMaskNone) return true;
    const int64_t ig = i + q_off, jg = j + k_off;
    bool ok = jg <= ig + diag + wr;
    if (wl >= 0) ok = ok && (jg >= ig + diag - wl);
    return ok || (jg < n_sink);
  }

  // Local rows [lo, hi) that have at least one allowed key in local keys [j0, j1).
  __host__ __device__ inline void rows_for_keys(int64_t j0, int64_t j1, int64_t Sq, int64_t* lo,
                                                int64_t* hi) const {
    if (kind == kMaskNone || j0 + k_off < n_sink) { *lo = 0; *hi = Sq; return; }
    int64_t a = j0 + k_off - diag - wr - q_off;                 // first row that reaches j0
    int64_t b = (wl >= 0) ? (j1 - 1 + k_off - diag + wl - q_off + 1) : Sq;
    a = a < 0 ? 0 : a;
    b = b > Sq ? Sq : b;
    *lo = a;
    *hi = b > a ? b : a;
  }

  // Local keys allowed for at least one row of local rows [i0, i1): the sink
  // range [0, s_hi) and the band [b_lo, b_hi) (either may be empty).
  __host__ __device__ inline void keys_for_rows(int64_t i0, int64_t i1, int64_t Sk, int64_t* s_hi,
                                                int64_t* b_lo, int64_t* b_hi) const {
    if (kind == kMaskNone) { *s_hi = 0; *b_lo = 0; *b_hi = Sk; return; }
    int64_t s = n_sink - k_off;
    s = s < 0 ? 0 : (s > Sk ? Sk : s);
    *s_hi = s;
    int64_t hi = i1 - 1 + q_off + diag + wr - k_off + 1;
    int64_t lo = (wl >= 0) ? (i0 + q_off + diag - wl - k_off) : 0;
    lo = lo < 0 ? 0 : lo;
    hi = hi > Sk ? Sk : hi;
    *b_lo = lo;
    *b_hi = hi > lo ? hi : lo;
  }

  // True when every pair of rows [i0,i1) x keys [j0,j1) is allowed.
  __host__ __device__ inline bool tile_full(int64_t i0, int64_t i1, int64_t j0, int64_t j1) const {
    if (kind == kMaskNone) return true;
    if (j1 - 1 + k_off < n_sink) return true;
    // band: the worst corners are (i0, j1-1) for the upper bound and (i1-1, j0) for the lower
    bool up = (j1 - 1 + k_off) <= (i0 + q_off + diag + wr);
    bool low = (wl < 0) || ((j0 + k_off) >= (i1 - 1 + q_off + diag - wl));
    return up && low;
  }
};

// Launch parameters shared by the backward / forward kernels.
struct Params {
  int B, Hq, Hk, G, Sq, Sk, Dqk, Dv;
  float scale;
  Mask mask;
  int64_t q_str[3], k_str[3], v_str[3], o_str[3], do_str[3], dq_str[3], dk_str[3], dv_str[3];
  int64_t bias_str[2];
  // variable-length packed batch (null: dense): prefix sums of the rows of
  // each sequence along the s index, and the packed row counts
  const int* cu_q;
  const int* cu_k;
  int64_t tot_q, tot_k;
};

// Sequence b of the batch: where its query rows and keys start along the s
// index (dense batch: 0, with the b strides locating it), its lengths, and
// the mask with its own bottom-right offset.  Packed offsets and lengths are
// clamped to the packed row counts and to the maxima Sq / Sk, so no access
// leaves the tensors whatever the prefix sums hold.
struct SeqView {
  int64_t q_row0, k_row0;
  int Sq, Sk;
  bool packed;
  Mask mask;

  // element offset of the sequence's (head 0, row 0) in a q-side / k-side tensor
  __device__ inline int64_t q_off(const int64_t* str, int b) const { return packed ? q_row0 * str[2] : b * str[0]; }
  __device__ inline int64_t k_off(const int64_t* str, int b) const { return packed ? k_row0 * str[2] : b * str[0]; }
};

__device__ inline SeqView seq_view(const Params& p, int b) {
  SeqView s;
  s.mask = p.mask;
  s.packed = p.cu_q != nullptr;
  if (!s.packed) {
    s.q_row0 = 0;
    s.k_row0 = 0;
    s.Sq = p.Sq;
    s.Sk = p.Sk;
    return s;
  }
  int64_t q0 = p.cu_q[b], q1 = p.cu_q[b + 1], k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
  q0 = q0 < 0 ? 0 : (q0 > p.tot_q ? p.tot_q : q0);
  k0 = k0 < 0 ? 0 : (k0 > p.tot_k ? p.tot_k : k0);
  q1 = q1 < q0 ? q0 : (q1 > p.tot_q ? p.tot_q : q1);
  k1 = k1 < k0 ? k0 : (k1 > p.tot_k ? p.tot_k : k1);
  s.q_row0 = q0;
  s.k_row0 = k0;
  s.Sq = (int)(q1 - q0 < p.Sq ? q1 - q0 : p.Sq);
  s.Sk = (int)(k1 - k0 < p.Sk ? k1 - k0 : p.Sk);
  if (s.mask.kind == kMaskBottomRight) s.mask.diag = s.Sk - s.Sq;
  return s;
}

__device__ inline float bf16_to_f32(unsigned short u) {
  return __uint_as_float(((unsigned int)u) << 16);
}

// Round to nearest even (inputs are finite).
__device__ inline unsigned short f32_to_bf16_rne(float f) {
  unsigned int u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

template <typename T>
__device__ inline float load_elem(const T* p, int64_t i);
template <>
__device__ inline float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ inline float load_elem<unsigned short>(const unsigned short* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

template <typename T>
__device__ inline void store_elem(T* p, int64_t i, float v);
template <>
__device__ inline void store_elem<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ inline void store_elem<unsigned short>(unsigned short* p, int64_t i, float v) {
  p[i] = f32_to_bf16_rne(v);
}

__device__ inline float atomic_add_f32(float* p, float v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace attn
