// Plain fp32-arithmetic attention kernels (vector ALU, no matrix cores).
//
// They cover every input dtype and head dims up to kSimtMaxD: the forward
// that produces (O, LSE) for all workloads, and the backward of fp32 inputs,
// where bf16 matrix-core operands would not meet fp32 accuracy.
//
// Tiles are 32 query rows x 32 keys with 128 threads; thread t owns row (or
// key) t / 4 and the columns c = t % 4 + 4 n, so the four lanes of a row sit
// in one wavefront and reduce with cross-lane shuffles.
#include "kernels.h"

namespace attn {

constexpr int kT = 32;       // rows / keys per tile
constexpr int kThreads = 128;
constexpr int kPad = kSimtMaxD + 1;
constexpr int kCols = kSimtMaxD / 4;

template <typename IT>
__device__ inline void load_tile(float (*dst)[kPad], const IT* base, int64_t row_stride, int64_t r0,
                                 int64_t r_end, int D) {
  for (int e = threadIdx.x; e < kT * D; e += kThreads) {
    const int rr = e / D, d = e - rr * D;
    const int64_t r = r0 + rr;
    dst[rr][d] = (r < r_end) ? load_elem(base, r * row_stride + d) : 0.f;
  }
}

__device__ inline float dot_row(const float* a, const float* b, int D) {
  float acc = 0.f;
  for (int d = 0; d < D; ++d) acc += a[d] * b[d];
  return acc;
}

// ---------------------------------------------------------------------------
// Forward: online softmax over the allowed keys of each row, with bias and
// the per-head sink logit in the normaliser.  O = P V, LSE = m + log(l).
// (CK FMHA example 34 cpu_fwd_with_intermediates, example 28
// cpu_attention_fwd_bias, example 22 cpu_attention_fwd_masked; the sink
// normaliser of CANN sparse_flash_mla_grad Phase 3.)
// Grid: (ceil(Sq / 32), Hq, B).
// ---------------------------------------------------------------------------
template <typename IT, typename OT>
__global__ __launch_bounds__(kThreads) void k_fwd_simt(Params p, FwdArgs a) {
  __shared__ float Qs[kT][kPad];
  __shared__ float Ks[kT][kPad];
  __shared__ float Vs[kT][kPad];
  __shared__ float Ps[kT][kT + 1];
  const int t = threadIdx.x, r = t >> 2, s = t & 3;
  const int i0 = blockIdx.x * kT, h = blockIdx.y, b = blockIdx.z, g = h / p.G;
  const IT* q = (const IT*)a.q + b * p.q_str[0] + h * p.q_str[1];
  const IT* k = (const IT*)a.k + b * p.k_str[0] + g * p.k_str[1];
  const IT* v = (const IT*)a.v + b * p.v_str[0] + g * p.v_str[1];
  const int i1 = min(i0 + kT, p.Sq);
  const int i = i0 + r;
  load_tile(Qs, q, p.q_str[2], i0, i1, p.Dqk);

  float m = -INFINITY, l = 0.f;
  float acc[kCols];
#pragma unroll
  for (int n = 0; n < kCols; ++n) acc[n] = 0.f;

  int64_t s_hi, b_lo, b_hi;
  p.mask.keys_for_rows(i0, i1, p.Sk, &s_hi, &b_lo, &b_hi);
  for (int part = 0; part < 2; ++part) {
    const int64_t j_begin = part == 0 ? 0 : max(b_lo, s_hi);
    const int64_t j_end = part == 0 ? s_hi : b_hi;
    for (int64_t j0 = j_begin; j0 < j_end; j0 += kT) {
      __syncthreads();
      load_tile(Ks, k, p.k_str[2], j0, j_end, p.Dqk);
      load_tile(Vs, v, p.v_str[2], j0, j_end, p.Dv);
      __syncthreads();
      float sv[kT / 4];
      float tmax = -INFINITY;
#pragma unroll
      for (int mm = 0; mm < kT / 4; ++mm) {
        const int jj = s + 4 * mm;
        const int64_t j = j0 + jj;
        float x = -INFINITY;
        if (i < i1 && j < j_end && p.mask.allowed(i, j)) {
          x = p.scale * dot_row(Qs[r], Ks[jj], p.Dqk);
          if (a.bias) x += a.bias[h * p.bias_str[0] + (int64_t)i * p.bias_str[1] + j];
        }
        sv[mm] = x;
        tmax = fmaxf(tmax, x);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 1, 4));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 2, 4));
      const float m_new = fmaxf(m, tmax);
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
      float psum = 0.f;
#pragma unroll
      for (int mm = 0; mm < kT / 4; ++mm) {
        const float pv = (sv[mm] == -INFINITY) ? 0.f : expf(sv[mm] - m_new);
        Ps[r][s + 4 * mm] = pv;
        psum += pv;
      }
      psum += __shfl_xor(psum, 1, 4);
      psum += __shfl_xor(psum, 2, 4);
      l = l * alpha + psum;
      m = m_new;
      __syncthreads();
#pragma unroll
      for (int n = 0; n < kCols; ++n) {
        const int c = s + 4 * n;
        if (c < p.Dv) {
          float o = acc[n] * alpha;
          for (int jj = 0; jj < kT; ++jj) o += Ps[r][jj] * Vs[jj][c];
          acc[n] = o;
        }
      }
    }
  }
  if (a.sinks) {
    const float sk = a.sinks[h];
    const float mf = fmaxf(m, sk);
    const float corr = (m == -INFINITY) ? 0.f : expf(m - mf);
    l = l * corr + expf(sk - mf);
#pragma unroll
    for (int n = 0; n < kCols; ++n) acc[n] *= corr;
    m = mf;
  }
  if (i < i1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    OT* o = (OT*)a.o + b * p.o_str[0] + h * p.o_str[1] + (int64_t)i * p.o_str[2];
#pragma unroll
    for (int n = 0; n < kCols; ++n) {
      const int c = s + 4 * n;
      if (c < p.Dv) store_elem(o, c, acc[n] * inv);
    }
    if (s == 0) a.lse[((int64_t)b * p.Hq + h) * p.Sq + i] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

// P and dS of one pair: P = exp(S - LSE), dS = P (dP - delta) (CK FMHA
// example 34 cpu_bwd_gqa; CANN sparse_flash_mla_grad Phase 2).
__device__ inline void pair_p_ds(const Params& p, const BwdArgs& a, int h, const float* qrow,
                                 const float* dorow, const float* krow, const float* vrow, int64_t i,
                                 int64_t j, float lse, float dl, float* pv, float* dsv) {
  float x = p.scale * dot_row(qrow, krow, p.Dqk);
  if (a.bias) x += a.bias[h * p.bias_str[0] + i * p.bias_str[1] + j];
  const float pp = expf(x - lse);
  const float dp = dot_row(dorow, vrow, p.Dv);
  *pv = pp;
  *dsv = pp * (dp - dl);
}

// ---------------------------------------------------------------------------
// dK / dV: one block per (key tile, KV head[, batch]); loops over the query
// heads of the group and the query rows that can see the tile, accumulating
// dK = scale dS^T Q and dV = P^T dO in registers (CK FMHA example 34
// cpu_bwd_gqa, dK/dV summed over each KV head's group).
// With dbias the block also loops over the batch and adds dS into dbias in
// batch order (example 28 cpu_attention_bwd_dbias: dbias = sum_b dS).
// Grid: (ceil(Sk / 32), Hk, b_loop ? 1 : B).
// ---------------------------------------------------------------------------
template <typename IT>
__global__ __launch_bounds__(kThreads) void k_dkdv_simt(Params p, BwdArgs a, int b_loop) {
  __shared__ float Ks[kT][kPad];
  __shared__ float Vs[kT][kPad];
  __shared__ float Qs[kT][kPad];
  __shared__ float dOs[kT][kPad];
  __shared__ float Ps[kT][kT + 1];
  __shared__ float dSs[kT][kT + 1];
  __shared__ float Ls[kT], Dl[kT];
  const int t = threadIdx.x, r = t >> 2, s = t & 3;
  const int j0 = blockIdx.x * kT, hk = blockIdx.y;
  const int j1 = min(j0 + kT, p.Sk);
  const int b_begin = b_loop ? 0 : blockIdx.z;
  const int b_end = b_loop ? p.B : b_begin + 1;
  int64_t lo, hi;
  p.mask.rows_for_keys(j0, j1, p.Sq, &lo, &hi);

  for (int b = b_begin; b < b_end; ++b) {
    const IT* k = (const IT*)a.k + b * p.k_str[0] + hk * p.k_str[1];
    const IT* v = (const IT*)a.v + b * p.v_str[0] + hk * p.v_str[1];
    __syncthreads();
    load_tile(Ks, k, p.k_str[2], j0, j1, p.Dqk);
    load_tile(Vs, v, p.v_str[2], j0, j1, p.Dv);
    float dk[kCols], dv[kCols];
#pragma unroll
    for (int n = 0; n < kCols; ++n) { dk[n] = 0.f; dv[n] = 0.f; }

    for (int h = hk * p.G; h < (hk + 1) * p.G; ++h) {
      const IT* q = (const IT*)a.q + b * p.q_str[0] + h * p.q_str[1];
      const IT* dout = (const IT*)a.dout + b * p.do_str[0] + h * p.do_str[1];
      const float* lse = a.lse + ((int64_t)b * p.Hq + h) * p.Sq;
      const float* delta = a.delta + ((int64_t)b * p.Hq + h) * p.Sq;
      for (int64_t i0 = lo; i0 < hi; i0 += kT) {
        __syncthreads();
        load_tile(Qs, q, p.q_str[2], i0, hi, p.Dqk);
        load_tile(dOs, dout, p.do_str[2], i0, hi, p.Dv);
        if (t < kT) {
          Ls[t] = (i0 + t < hi) ? lse[i0 + t] : -INFINITY;
          Dl[t] = (i0 + t < hi) ? delta[i0 + t] : 0.f;
        }
        __syncthreads();
        const int64_t i = i0 + r;
#pragma unroll
        for (int mm = 0; mm < kT / 4; ++mm) {
          const int jj = s + 4 * mm;
          const int64_t j = j0 + jj;
          float pv = 0.f, dsv = 0.f;
          if (i < hi && j < j1 && Ls[r] != -INFINITY && p.mask.allowed(i, j))
            pair_p_ds(p, a, h, Qs[r], dOs[r], Ks[jj], Vs[jj], i, j, Ls[r], Dl[r], &pv, &dsv);
          Ps[r][jj] = pv;
          dSs[r][jj] = dsv;
          if (a.dbias && i < hi && j < j1)
            a.dbias[h * p.bias_str[0] + i * p.bias_str[1] + j] += dsv;
        }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < kCols; ++n) {
          const int c = s + 4 * n;
          float accv = dv[n], acck = dk[n];
          if (c < p.Dv)
            for (int rr = 0; rr < kT; ++rr) accv += Ps[rr][r] * dOs[rr][c];
          if (c < p.Dqk)
            for (int rr = 0; rr < kT; ++rr) acck += dSs[rr][r] * Qs[rr][c];
          dv[n] = accv;
          dk[n] = acck;
        }
      }
    }
    const int64_t j = j0 + r;  // this thread's key for the accumulators
    if (j < j1) {
      float* dkp = a.dk + b * p.dk_str[0] + hk * p.dk_str[1] + j * p.dk_str[2];
      float* dvp = a.dv + b * p.dv_str[0] + hk * p.dv_str[1] + j * p.dv_str[2];
#pragma unroll
      for (int n = 0; n < kCols; ++n) {
        const int c = s + 4 * n;
        if (c < p.Dqk) dkp[c] = (a.accumulate_dkdv ? dkp[c] : 0.f) + dk[n] * p.scale;
        if (c < p.Dv) dvp[c] = (a.accumulate_dkdv ? dvp[c] : 0.f) + dv[n];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ = scale dS K: one block per (query tile, query head, batch); loops over
// the sink keys and the band of keys visible to the tile, accumulating in
// registers (no atomics).  Grid: (ceil(Sq / 32), Hq, B).
// ---------------------------------------------------------------------------
template <typename IT>
__global__ __launch_bounds__(kThreads) void k_dq_simt(Params p, BwdArgs a) {
  __shared__ float Qs[kT][kPad];
  __shared__ float dOs[kT][kPad];
  __shared__ float Ks[kT][kPad];
  __shared__ float Vs[kT][kPad];
  __shared__ float dSs[kT][kT + 1];
  __shared__ float Ls[kT], Dl[kT];
  const int t = threadIdx.x, r = t >> 2, s = t & 3;
  const int i0 = blockIdx.x * kT, h = blockIdx.y, b = blockIdx.z, g = h / p.G;
  const int i1 = min(i0 + kT, p.Sq);
  const IT* q = (const IT*)a.q + b * p.q_str[0] + h * p.q_str[1];
  const IT* dout = (const IT*)a.dout + b * p.do_str[0] + h * p.do_str[1];
  const IT* k = (const IT*)a.k + b * p.k_str[0] + g * p.k_str[1];
  const IT* v = (const IT*)a.v + b * p.v_str[0] + g * p.v_str[1];
  const float* lse = a.lse + ((int64_t)b * p.Hq + h) * p.Sq;
  const float* delta = a.delta + ((int64_t)b * p.Hq + h) * p.Sq;
  load_tile(Qs, q, p.q_str[2], i0, i1, p.Dqk);
  load_tile(dOs, dout, p.do_str[2], i0, i1, p.Dv);
  if (t < kT) {
    Ls[t] = (i0 + t < i1) ? lse[i0 + t] : -INFINITY;
    Dl[t] = (i0 + t < i1) ? delta[i0 + t] : 0.f;
  }
  float dq[kCols];
#pragma unroll
  for (int n = 0; n < kCols; ++n) dq[n] = 0.f;
  const int64_t i = i0 + r;

  int64_t s_hi, b_lo, b_hi;
  p.mask.keys_for_rows(i0, i1, p.Sk, &s_hi, &b_lo, &b_hi);
  for (int part = 0; part < 2; ++part) {
    const int64_t j_begin = part == 0 ? 0 : max(b_lo, s_hi);
    const int64_t j_end = part == 0 ? s_hi : b_hi;
    for (int64_t j0 = j_begin; j0 < j_end; j0 += kT) {
      __syncthreads();
      load_tile(Ks, k, p.k_str[2], j0, j_end, p.Dqk);
      load_tile(Vs, v, p.v_str[2], j0, j_end, p.Dv);
      __syncthreads();
#pragma unroll
      for (int mm = 0; mm < kT / 4; ++mm) {
        const int jj = s + 4 * mm;
        const int64_t j = j0 + jj;
        float pv = 0.f, dsv = 0.f;
        if (i < i1 && j < j_end && Ls[r] != -INFINITY && p.mask.allowed(i, j))
          pair_p_ds(p, a, h, Qs[r], dOs[r], Ks[jj], Vs[jj], i, j, Ls[r], Dl[r], &pv, &dsv);
        dSs[r][jj] = dsv;
      }
      __syncthreads();
#pragma unroll
      for (int n = 0; n < kCols; ++n) {
        const int c = s + 4 * n;
        if (c < p.Dqk) {
          float accq = dq[n];
          for (int jj = 0; jj < kT; ++jj) accq += dSs[r][jj] * Ks[jj][c];
          dq[n] = accq;
        }
      }
    }
  }
  if (i < i1) {
    float* dqp = a.dq + b * p.dq_str[0] + h * p.dq_str[1] + i * p.dq_str[2];
#pragma unroll
    for (int n = 0; n < kCols; ++n) {
      const int c = s + 4 * n;
      if (c < p.Dqk) dqp[c] = (a.accumulate_dq ? dqp[c] : 0.f) + dq[n] * p.scale;
    }
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_fwd_simt(const Params& p, const FwdArgs& a, int in_bf16, int o_bf16, hipStream_t st) {
  if (p.Sq == 0 || p.B == 0 || p.Hq == 0) return hipSuccess;
  const dim3 grid((p.Sq + kT - 1) / kT, p.Hq, p.B);
  if (in_bf16 && o_bf16)
    hipLaunchKernelGGL((k_fwd_simt<unsigned short, unsigned short>), grid, dim3(kThreads), 0, st, p, a);
  else if (in_bf16)
    hipLaunchKernelGGL((k_fwd_simt<unsigned short, float>), grid, dim3(kThreads), 0, st, p, a);
  else if (o_bf16)
    hipLaunchKernelGGL((k_fwd_simt<float, unsigned short>), grid, dim3(kThreads), 0, st, p, a);
  else
    hipLaunchKernelGGL((k_fwd_simt<float, float>), grid, dim3(kThreads), 0, st, p, a);
  return hipGetLastError();
}

hipError_t launch_bwd_simt(const Params& p, const BwdArgs& a, int in_bf16, hipStream_t st) {
  // dbias is summed into (every batch entry adds its dS)
  if (a.dbias && p.Sq > 0 && p.Sk > 0 && p.B > 0) {
    hipError_t e = launch_zero_bias(a.dbias, p.Hq, p.Sq, p.Sk, p.bias_str, st);
    if (e != hipSuccess) return e;
  }
  if (p.Sk > 0 && p.B > 0) {
    const int b_loop = a.dbias != nullptr;
    const dim3 grid((p.Sk + kT - 1) / kT, p.Hk, b_loop ? 1 : p.B);
    if (in_bf16)
      hipLaunchKernelGGL((k_dkdv_simt<unsigned short>), grid, dim3(kThreads), 0, st, p, a, b_loop);
    else
      hipLaunchKernelGGL((k_dkdv_simt<float>), grid, dim3(kThreads), 0, st, p, a, b_loop);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_dq_simt(p, a, in_bf16, st);
}

hipError_t launch_dq_simt(const Params& p, const BwdArgs& a, int in_bf16, hipStream_t st) {
  if (p.Sq > 0 && p.B > 0) {
    const dim3 grid((p.Sq + kT - 1) / kT, p.Hq, p.B);
    if (in_bf16)
      hipLaunchKernelGGL((k_dq_simt<unsigned short>), grid, dim3(kThreads), 0, st, p, a);
    else
      hipLaunchKernelGGL((k_dq_simt<float>), grid, dim3(kThreads), 0, st, p, a);
  }
  return hipGetLastError();
}

}  // namespace attn
