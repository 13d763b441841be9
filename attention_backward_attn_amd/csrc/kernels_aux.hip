// Memory-bound helper kernels: the backward preprocess (delta = rowsum(dO*O)
// and the sink-logit gradient), zero fills, and the log-sum-exp merge.
#include "kernels.h"
#include "mfma_util.h"

namespace attn {

// Length and first packed row of sequence b (clamped as in seq_view).
__device__ inline int packed_seq(const Packed& pk, int b, int Smax, int64_t* row0) {
  int64_t q0 = pk.cu[b], q1 = pk.cu[b + 1];
  q0 = q0 < 0 ? 0 : (q0 > pk.tot ? pk.tot : q0);
  q1 = q1 < q0 ? q0 : (q1 > pk.tot ? pk.tot : q1);
  *row0 = q0;
  return (int)(q1 - q0 < Smax ? q1 - q0 : Smax);
}


// ---------------------------------------------------------------------------
// delta[b,h,i] = sum_d dO[b,h,i,d] * O[b,h,i,d]
// (CK FMHA example 34 cpu_bwd_gqa "D"; CANN sparse_flash_mla_grad Phase 2
// SoftmaxGrad(dO, O)).  Each row is read by a group of TPR lanes, each lane
// holding 8 contiguous elements; the group reduces with cross-lane shuffles.
// ---------------------------------------------------------------------------
// When dq is non-null the same lanes also zero dQ's row (Dqk floats).
template <typename OT, typename DT, int TPR>
__global__ __launch_bounds__(256) void k_delta_vec(const OT* __restrict__ o,
                                                   const DT* __restrict__ dout,
                                                   float* __restrict__ delta, int B, int H, int Sq,
                                                   int Dv, int64_t ob, int64_t oh, int64_t os,
                                                   int64_t db, int64_t dh, int64_t ds,
                                                   float* __restrict__ dq, int Dqk, int64_t qb,
                                                   int64_t qh, int64_t qs, Packed pk) {
  const int64_t rows = (int64_t)B * H * Sq;
  const int lane_in_row = threadIdx.x % TPR;
  const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) / TPR;
  float acc = 0.f;
  bool live = idx < rows;
  // Walk the rows in memory order: positions fastest when a head's rows are
  // contiguous ([B, H, S, D]), heads fastest when the heads of a position are
  // ([T, H, D] packed).
  const bool h_fast = oh < os;
  const int i = !live ? 0 : (h_fast ? (int)((idx / H) % Sq) : (int)(idx % Sq));
  const int h = !live ? 0 : (h_fast ? (int)(idx % H) : (int)((idx / Sq) % H));
  const int b = live ? (int)(idx / ((int64_t)Sq * H)) : 0;
  const int64_t row = ((int64_t)b * H + h) * Sq + i;   // delta index
  // dense: (b, i) through the b stride; packed: packed row r0 + i of sequence b
  int64_t ro = 0, rd = 0, rq = 0;
  if (live) {
    if (pk.cu) {
      int64_t r0;
      live = i < packed_seq(pk, b, Sq, &r0);
      ro = (r0 + i) * os; rd = (r0 + i) * ds; rq = (r0 + i) * qs;
    } else {
      ro = b * ob + i * os; rd = b * db + i * ds; rq = b * qb + i * qs;
    }
  }
  if (live) {
    const OT* orow = o + ro + h * oh;
    const DT* drow = dout + rd + h * dh;
    for (int d0 = lane_in_row * 8; d0 < Dv; d0 += TPR * 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += load_elem(orow, d0 + e) * load_elem(drow, d0 + e);
    }
    if (dq) {
      float* qrow = dq + rq + h * qh;
      for (int d = lane_in_row; d < Dqk; d += TPR) qrow[d] = 0.f;
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (idx < rows && lane_in_row == 0) delta[row] = acc;   // 0 past a packed sequence's length
}

// Scalar fallback for Dv not a multiple of 8: one thread per row.
template <typename OT, typename DT>
__global__ __launch_bounds__(256) void k_delta_scalar(const OT* __restrict__ o,
                                                      const DT* __restrict__ dout,
                                                      float* __restrict__ delta, int B, int H,
                                                      int Sq, int Dv, int64_t ob, int64_t oh,
                                                      int64_t os, int64_t db, int64_t dh,
                                                      int64_t ds, float* __restrict__ dq, int Dqk,
                                                      int64_t qb, int64_t qh, int64_t qs, Packed pk) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= (int64_t)B * H * Sq) return;
  const int i = (int)(row % Sq);
  const int h = (int)((row / Sq) % H);
  const int b = (int)(row / ((int64_t)Sq * H));
  int64_t ro = b * ob + i * os, rd = b * db + i * ds, rq = b * qb + i * qs;
  if (pk.cu) {
    int64_t r0;
    if (i >= packed_seq(pk, b, Sq, &r0)) {
      delta[row] = 0.f;
      return;
    }
    ro = (r0 + i) * os; rd = (r0 + i) * ds; rq = (r0 + i) * qs;
  }
  float acc = 0.f;
  for (int d = 0; d < Dv; ++d) acc += load_elem(o + ro + h * oh, d) * load_elem(dout + rd + h * dh, d);
  delta[row] = acc;
  if (dq)
    for (int d = 0; d < Dqk; ++d) dq[rq + h * qh + d] = 0.f;
}

// dsinks[h] = -sum_{b,i} exp(sink_h - lse[b,h,i]) * delta[b,h,i]
// (CANN sparse_flash_mla_grad Phase 3 dSinks reduced over rows and batch).
// One block of DS_NT threads per head; each thread sums the rows
// i = t + DS_NT k in a fixed order, with DS_U rows' loads in flight before
// their use, then a fixed tree adds the threads' sums: the result does not
// depend on scheduling.
constexpr int DS_NT = 1024, DS_U = 4;
__global__ __launch_bounds__(DS_NT) void k_dsinks(const float* __restrict__ lse,
                                                  const float* __restrict__ delta,
                                                  const float* __restrict__ sinks,
                                                  float* __restrict__ dsinks, int B, int H, int Sq,
                                                  Packed pk) {
  __shared__ float red[DS_NT];
  const int h = blockIdx.x, t = threadIdx.x;
  const float s = sinks[h];
  float acc = 0.f;
  for (int b = 0; b < B; ++b) {
    const float* l = lse + ((int64_t)b * H + h) * Sq;
    const float* d = delta + ((int64_t)b * H + h) * Sq;
    int64_t r0;
    const int n = pk.cu ? packed_seq(pk, b, Sq, &r0) : Sq;   // rows of this sequence
    for (int i0 = t; i0 < n; i0 += DS_NT * DS_U) {
      float lv[DS_U], dv[DS_U];
#pragma unroll
      for (int u = 0; u < DS_U; ++u) {
        const int i = i0 + DS_NT * u;
        lv[u] = i < n ? l[i] : -INFINITY;
        dv[u] = i < n ? d[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < DS_U; ++u)
        if (lv[u] != -INFINITY) acc += expf(s - lv[u]) * dv[u];
    }
  }
  red[t] = acc;
  __syncthreads();
  for (int w = DS_NT / 2; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) dsinks[h] = -red[0];
}

static unsigned fill_blocks(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (unsigned)(b > 16384 ? 16384 : (b < 1 ? 1 : b));
}

// Zero rows of a strided [B, H, S, D] fp32 tensor (D contiguous).
__global__ __launch_bounds__(256) void k_zero_rows(float* __restrict__ x, int B, int H, int S, int D,
                                                   int64_t sb, int64_t sh, int64_t ss) {
  const int64_t n = (int64_t)B * H * S * D;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int d = (int)(e % D);
    const int64_t r = e / D;
    const int i = (int)(r % S);
    const int h = (int)((r / S) % H);
    const int b = (int)(r / ((int64_t)S * H));
    x[b * sb + h * sh + i * ss + d] = 0.f;
  }
}

__global__ __launch_bounds__(256) void k_zero_multi(ZeroMulti m) {
  zero_multi_range(m, 0, m.off[m.n], blockIdx.x * 256 + threadIdx.x, gridDim.x * 256);
}

ZeroMulti make_zero_multi(const ZeroRows* z, int n) {
  ZeroMulti m{};
  int k = 0;
  m.off[0] = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t rows = (int64_t)z[i].B * z[i].H * z[i].S;
    if (rows == 0 || z[i].D == 0) continue;
    m.z[k] = z[i];
    const bool aligned = ((uintptr_t)z[i].p % 16 == 0) && z[i].str[0] % 4 == 0 && z[i].str[1] % 4 == 0 &&
                         z[i].str[2] % 4 == 0;
    m.vec[k] = (z[i].D % 4 == 0 && aligned) ? 1 : 0;
    // dense: the (size, stride) pairs of the B, H, S indices (size-1 ones
    // dropped), in increasing stride, tile the memory after the D floats of a row
    int64_t dims[3][2] = {{z[i].B, z[i].str[0]}, {z[i].H, z[i].str[1]}, {z[i].S, z[i].str[2]}};
    for (int a = 0; a < 3; ++a)
      for (int b = a + 1; b < 3; ++b)
        if (dims[b][1] < dims[a][1]) {
          int64_t t0 = dims[a][0], t1 = dims[a][1];
          dims[a][0] = dims[b][0]; dims[a][1] = dims[b][1];
          dims[b][0] = t0; dims[b][1] = t1;
        }
    int64_t expect = z[i].D;
    bool dense = true;
    for (int a = 0; a < 3; ++a) {
      if (dims[a][0] == 1) continue;
      if (dims[a][1] != expect) dense = false;
      expect *= dims[a][0];
    }
    m.dense[k] = dense ? 1 : 0;
    m.off[k + 1] = m.off[k] + rows * (m.vec[k] ? z[i].D / 4 : z[i].D);
    ++k;
  }
  m.n = k;
  return m;
}

hipError_t launch_zero_multi(const ZeroRows* z, int n, hipStream_t st) {
  const ZeroMulti m = make_zero_multi(z, n);
  if (m.n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_multi, dim3(fill_blocks(m.off[m.n])), dim3(256), 0, st, m);
  return hipGetLastError();
}

// Zero a strided [H, Sq, Sk] fp32 tensor (Sk contiguous).
__global__ __launch_bounds__(256) void k_zero_bias(float* __restrict__ x, int H, int Sq, int Sk,
                                                   int64_t sh, int64_t si) {
  const int64_t n = (int64_t)H * Sq * Sk;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int j = (int)(e % Sk);
    const int64_t r = e / Sk;
    x[(r / Sq) * sh + (r % Sq) * si + j] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// In-place merge of a partial (o, lse) into an accumulator ("Ring attention
// for PyTorch", _ring_fwd): lse = logaddexp(lse_a, lse_b),
// o = o_a e^{lse_a - lse} + o_b e^{lse_b - lse}; both empty -> o = 0, lse = -inf.
// One block per row; every lane reads both lse values before lane 0 writes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void k_lse_merge(float* __restrict__ o_acc,
                                                   float* __restrict__ lse_acc,
                                                   const float* __restrict__ o_part,
                                                   const float* __restrict__ lse_part, int Dv) {
  const int64_t row = blockIdx.x;
  const float la = lse_acc[row], lb = lse_part[row];
  const float mx = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, l = -INFINITY;
  if (mx != -INFINITY) {
    const float ea = expf(la - mx), eb = expf(lb - mx);
    const float sum = ea + eb;
    l = mx + logf(sum);
    wa = ea / sum;
    wb = eb / sum;
  }
  float* oa = o_acc + row * Dv;
  const float* ob = o_part + row * Dv;
  for (int d = threadIdx.x; d < Dv; d += 128) {
    const float a = (wa != 0.f) ? oa[d] * wa : 0.f;
    const float b = (wb != 0.f) ? ob[d] * wb : 0.f;
    oa[d] = a + b;
  }
  __syncthreads();
  if (threadIdx.x == 0) lse_acc[row] = l;
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
template <typename OT, typename DT>
static hipError_t launch_delta_t(const void* o, const void* dout, float* delta, int B, int H, int Sq,
                                 int Dv, const int64_t* os, const int64_t* ds, float* dq, int Dqk,
                                 const int64_t* qs, Packed pk, hipStream_t st) {
  const int64_t rows = (int64_t)B * H * Sq;
  if (Dv % 8 == 0) {
    // lanes per row: 8 elements each (one 16-byte load per tensor for head
    // dims up to 512, so a row's loads are all in flight at once)
    const int tpr = Dv >= 512 ? 64 : (Dv >= 256 ? 32 : (Dv >= 128 ? 16 : (Dv >= 64 ? 8 : (Dv >= 32 ? 4 : (Dv >= 16 ? 2 : 1)))));
    const int64_t blocks = (rows * tpr + 255) / 256;
#define ATTN_DELTA_LAUNCH(T)                                                                     \
  hipLaunchKernelGGL((k_delta_vec<OT, DT, T>), dim3((unsigned)blocks), dim3(256), 0, st,           \
                     (const OT*)o, (const DT*)dout, delta, B, H, Sq, Dv, os[0], os[1], os[2],      \
                     ds[0], ds[1], ds[2], dq, Dqk, qs[0], qs[1], qs[2], pk)
    switch (tpr) {
      case 64: ATTN_DELTA_LAUNCH(64); break;
      case 32: ATTN_DELTA_LAUNCH(32); break;
      case 16: ATTN_DELTA_LAUNCH(16); break;
      case 8: ATTN_DELTA_LAUNCH(8); break;
      case 4: ATTN_DELTA_LAUNCH(4); break;
      case 2: ATTN_DELTA_LAUNCH(2); break;
      default: ATTN_DELTA_LAUNCH(1); break;
    }
#undef ATTN_DELTA_LAUNCH
  } else {
    hipLaunchKernelGGL((k_delta_scalar<OT, DT>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                       st, (const OT*)o, (const DT*)dout, delta, B, H, Sq, Dv, os[0], os[1], os[2],
                       ds[0], ds[1], ds[2], dq, Dqk, qs[0], qs[1], qs[2], pk);
  }
  return hipGetLastError();
}

hipError_t launch_delta(const void* o, int o_bf16, const void* dout, int do_bf16, float* delta, int B,
                        int H, int Sq, int Dv, const int64_t* os, const int64_t* ds, float* dq_zero,
                        int Dqk, const int64_t* qs, Packed pk, hipStream_t st) {
  if (o_bf16 && do_bf16)
    return launch_delta_t<unsigned short, unsigned short>(o, dout, delta, B, H, Sq, Dv, os, ds, dq_zero,
                                                          Dqk, qs, pk, st);
  if (o_bf16)
    return launch_delta_t<unsigned short, float>(o, dout, delta, B, H, Sq, Dv, os, ds, dq_zero, Dqk, qs, pk, st);
  if (do_bf16)
    return launch_delta_t<float, unsigned short>(o, dout, delta, B, H, Sq, Dv, os, ds, dq_zero, Dqk, qs, pk, st);
  return launch_delta_t<float, float>(o, dout, delta, B, H, Sq, Dv, os, ds, dq_zero, Dqk, qs, pk, st);
}

hipError_t launch_dsinks(const float* lse, const float* delta, const float* sinks, float* dsinks,
                         int B, int H, int Sq, Packed pk, hipStream_t st) {
  hipLaunchKernelGGL(k_dsinks, dim3(H), dim3(DS_NT), 0, st, lse, delta, sinks, dsinks, B, H, Sq, pk);
  return hipGetLastError();
}

hipError_t launch_zero_rows(float* x, int B, int H, int S, int D, const int64_t* str, hipStream_t st) {
  const int64_t n = (int64_t)B * H * S * D;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_rows, dim3(fill_blocks(n)), dim3(256), 0, st, x, B, H, S, D, str[0],
                     str[1], str[2]);
  return hipGetLastError();
}

hipError_t launch_zero_bias(float* x, int H, int Sq, int Sk, const int64_t* str, hipStream_t st) {
  const int64_t n = (int64_t)H * Sq * Sk;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_bias, dim3(fill_blocks(n)), dim3(256), 0, st, x, H, Sq, Sk, str[0],
                     str[1]);
  return hipGetLastError();
}

hipError_t launch_lse_merge(int64_t rows, int Dv, float* o_acc, float* lse_acc, const float* o_part,
                            const float* lse_part, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_lse_merge, dim3((unsigned)rows), dim3(128), 0, st, o_acc, lse_acc, o_part,
                     lse_part, Dv);
  return hipGetLastError();
}

}  // namespace attn
