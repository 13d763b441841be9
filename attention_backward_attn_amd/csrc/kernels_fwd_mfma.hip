// bf16 matrix-core (gfx950 MFMA) attention forward with the row log-sum-exp.
//
// Math (ring-attention gist, _flash_fwd returning (out, lse); CK FMHA
// example 34 cpu_fwd_with_intermediates; CK FMHA example 22
// cpu_attention_fwd_masked, with the sink logit added to the normaliser):
//   S = scale Q K^T (+ bias),  LSE_i = log(sum_j exp S_ij + exp sink),
//   O = exp(S - LSE) V.  Rows with no allowed key and no sink: O = 0,
//   LSE = -inf.
//
// Kernel k_fwd: one workgroup per (128-row query block, query head, batch);
// wave w owns rows [32 w, 32 w + 32).  Per tile of KT keys, S^T = K Q^T
// with the wave's Q fragments in registers as the B operand and K rows from
// LDS as the A operand, so each lane holds one query row (and the lane
// l ^ 32 holds the row's other keys).  Online softmax in log2 units: the
// running row maximum is shared by the two lanes of a row with one shuffle
// and raised only when a tile's exceeds it by more than 8 (P < 2^8, rare O
// rescales); each lane keeps its own share of the normaliser, added up once
// at the end.
// O^T += V^T P^T uses the P values straight from the S^T accumulator as the
// B operand (reduction slots in accumulator order) and V^T from transposing
// LDS reads in the same slot order, so O^T's accumulator also has one query
// row per lane and the per-row rescale is a per-lane scalar.
#include <algorithm>

#include "kernels.h"
#include "mfma_util.h"

namespace attn {
namespace {

using namespace mfma_util;

constexpr int NTF = 256;   // threads per workgroup
constexpr int BQF = 128;   // query rows per workgroup

template <int D, int KT, bool BIAS>
struct SmemFwd {
  unsigned short kr[2][KT * Lay<D>::R];   // K tile, row copy (A of S^T = K Q^T)
  unsigned short vt[2][KT * Lay<D>::T];   // V tile, tr copy  (A of O^T += V^T P^T)
  float bias[BIAS ? 2 : 1][BIAS ? BQF * (KT + 4) : 1];   // bias[h][i0 + r][j0 + c], padded rows
};

// Staging of one KT-key K / V tile (16-byte chunks dealt round-robin, 16
// consecutive lanes on one row) and, with a bias, of the [128 x KT] fp32
// bias tile (16-byte chunks along the keys).  Keys past the end load the
// last key (finite; masked to P = 0); rows past the end load the last row.
template <int D, int KT, bool BIAS>
struct StageFwd {
  static constexpr int NCR = D / 8;
  static constexpr int NR = 2 * KT * NCR / NTF;
  static constexpr int NBI = BIAS ? BQF * KT / 4 / NTF : 0;
  static constexpr int BS = KT + 4;
  static_assert(2 * KT * NCR % NTF == 0, "tile chunks per thread");
  u16x8 v[NR];
  f32x4 bv[BIAS ? NBI : 1];

  __device__ inline void load(const unsigned short* k, const unsigned short* vv, int64_t ks, int64_t vs,
                              int64_t j0, int Sk, const float* bias_h, int64_t bstr, int i0, int Sq) {
    const int t = threadIdx.x;
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int idx = t + NTF * m;
      const int tensor = idx / (KT * NCR), rem = idx % (KT * NCR);
      const int row = rem / NCR, c = rem % NCR;
      const int64_t j = min(j0 + row, (int64_t)Sk - 1);
      v[m] = *(const u16x8*)((tensor == 0 ? k + j * ks : vv + j * vs) + 8 * c);
    }
    if (BIAS) {
#pragma unroll
      for (int m = 0; m < NBI; ++m) {
        const int idx = t + NTF * m;
        const int row = idx / (KT / 4), c4 = idx % (KT / 4);
        const int64_t i = min(i0 + row, Sq - 1);
        const int64_t j = min(j0 + 4 * c4, (int64_t)Sk - 4);   // Sk % 4 == 0 on this path
        bv[m] = *(const f32x4*)(bias_h + i * bstr + j);
      }
    }
  }

  __device__ inline void store(SmemFwd<D, KT, BIAS>& sm, int buf) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int idx = t + NTF * m;
      const int tensor = idx / (KT * NCR), rem = idx % (KT * NCR);
      const int row = rem / NCR, c = rem % NCR;
      if (tensor == 0)
        *(u16x8*)(sm.kr[buf] + row * Lay<D>::R + 8 * c) = v[m];
      else
        *(u16x8*)(sm.vt[buf] + row * Lay<D>::T + 8 * c) = v[m];
    }
    if (BIAS) {
#pragma unroll
      for (int m = 0; m < NBI; ++m) {
        const int idx = t + NTF * m;
        const int row = idx / (KT / 4), c4 = idx % (KT / 4);
        *(f32x4*)&sm.bias[buf][row * BS + 4 * c4] = bv[m];
      }
    }
  }
};

__device__ inline void store4(float* p, const float* v) { *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]}; }
__device__ inline void store4(unsigned short* p, const float* v) {
  *(u16x4*)p = u16x4{f32_to_bf16_rne(v[0]), f32_to_bf16_rne(v[1]), f32_to_bf16_rne(v[2]),
                     f32_to_bf16_rne(v[3])};
}

template <int D, int KT, bool BIAS, typename OT>
__global__ __launch_bounds__(NTF, 2) void k_fwd(Params p, FwdArgs a) {
  constexpr int NS = D / 16, NB = D / 32, NH = KT / 32;
  constexpr int R = Lay<D>::R, T = Lay<D>::T, BS = KT + 4;
  __shared__ __attribute__((aligned(16))) SmemFwd<D, KT, BIAS> sm;

  const int tid = threadIdx.x, l = tid & 63, lr = l & 31, lg = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const BlockXYZ blk = a.xmajor ? xcd_block_xmajor() : xcd_block();
  // under a causal mask later row blocks see more keys: deal them first
  const bool heavy_last = p.mask.kind != kMaskNone && p.mask.wl < 0;
  const int i0 = (heavy_last ? (int)gridDim.x - 1 - blk.x : blk.x) * BQF;
  const int h = blk.y, b = blk.z, g = h / p.G;
  const SeqView sv = seq_view(p, b);   // this batch entry (or packed sequence)
  const Mask& msk = sv.mask;
  const int Sq = sv.Sq, Sk = sv.Sk;
  if (i0 >= Sq) return;   // past this sequence's rows (uniform across the workgroup)
  const int irow = i0 + 32 * w + lr;   // this lane's query row
  const float scale_log2 = p.scale * kLog2e;
  const int rowA = lr * R + 8 * lg;
  const int trV = tr_base(l, T);

  const unsigned short* q = (const unsigned short*)a.q + sv.q_off(p.q_str, b) + h * p.q_str[1];
  const unsigned short* kp = (const unsigned short*)a.k + sv.k_off(p.k_str, b) + g * p.k_str[1];
  const unsigned short* vp = (const unsigned short*)a.v + sv.k_off(p.v_str, b) + g * p.v_str[1];

  bf16x8 qB[NS];
  {
    const int64_t ic = min(irow, Sq - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) qB[s] = as_bf16x8(*(const u16x8*)(q + ic * p.q_str[2] + 16 * s + 8 * lg));
  }
  // running row maximum (log2 units) and this lane's share of the normaliser;
  // the sink contributes exp2(sink - m) = 1 at m = sink, counted once per row
  float m = -INFINITY, lsum = 0.f;
  if (a.sinks) {
    m = a.sinks[h] * kLog2e;
    lsum = lg == 0 ? 1.f : 0.f;
  }
  wait_vm_loads();

  // key tiles: the sink tiles, then the band tiles of the block's rows
  int64_t s_hi, b_lo, b_hi;
  const int i1 = min(i0 + BQF, Sq);
  msk.keys_for_rows(i0, i1, Sk, &s_hi, &b_lo, &b_hi);
  const int a1 = (int)((s_hi + KT - 1) / KT);
  int a2 = (int)(b_lo / KT);
  const int a3 = b_hi > b_lo ? (int)((b_hi + KT - 1) / KT) : a2;
  if (a2 < a1) a2 = a1;
  const int n1 = a1, n2 = a3 > a2 ? a3 - a2 : 0;
  const int n_it = (i0 < Sq && Sk > 0) ? n1 + n2 : 0;
  auto tile_of = [&](int it) { return (int64_t)KT * (it < n1 ? it : a2 + (it - n1)); };
  const bool no_mask = msk.kind == kMaskNone;
  const int lo_t = msk.wl < 0 ? -0x3fffffff : -msk.wl;
  const int wr_t = msk.wr;

  f32x16 o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = zero16();

  const float* bias_h = BIAS ? a.bias + h * p.bias_str[0] : nullptr;
  StageFwd<D, KT, BIAS> stg;
  if (n_it > 0) {
    stg.load(kp, vp, p.k_str[2], p.v_str[2], tile_of(0), Sk, bias_h, p.bias_str[1], i0, Sq);
    stg.store(sm, 0);
    __syncthreads();
  }
  for (int it = 0; it < n_it; ++it) {
    const int cur = it & 1;
    const int j0 = (int)tile_of(it);
    if (it + 1 < n_it) stg.load(kp, vp, p.k_str[2], p.v_str[2], tile_of(it + 1), Sk, bias_h, p.bias_str[1], i0, Sq);

    f32x16 sacc[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      sacc[hh] = zero16();
#pragma unroll
      for (int s = 0; s < NS; ++s)
        sacc[hh] = mfma(lds_b128(sm.kr[cur], rowA + 32 * hh * R + 16 * s), qB[s], sacc[hh]);
    }
    const bool full = (j0 + KT <= Sk) && msk.tile_full(i0 + 32 * w, i0 + 32 * w + 32, j0, j0 + KT);
    // t = j' - i' - diag for key j0 + 4 lg + c
    const int tb = j0 + (int)msk.k_off + 4 * lg - (irow + (int)msk.q_off) - (int)msk.diag;
    float mt = -INFINITY;
    // x: the logit in log2 units with a bias; the raw S without one (the
    // scale, positive, is applied in the exponential's fma and to the tile
    // maximum)
    auto elem = [&](int hh, int r, bool masked) {
      const int c = 32 * hh + 8 * (r >> 2) + (r & 3);
      float x = sacc[hh][r];
      if (BIAS) x = fmaf(sm.bias[cur][(32 * w + lr) * BS + 4 * lg + c], kLog2e, x * scale_log2);
      if (masked) {
        const int j = j0 + 4 * lg + c;
        const int t = tb + c;
        const bool ok = (j < Sk) & (no_mask | ((t <= wr_t) & (t >= lo_t)) | ((j + (int)msk.k_off) < msk.n_sink));
        x = ok ? x : -INFINITY;
      }
      sacc[hh][r] = x;
      mt = fmaxf(mt, x);
    };
    if (full) {
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int r = 0; r < 16; ++r) elem(hh, r, false);
    } else {
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int r = 0; r < 16; ++r) elem(hh, r, true);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    if (!BIAS) mt *= scale_log2;
    // The running maximum is raised only when the tile's exceeds it by more
    // than 8 (log2 units): P stays below 2^8 and the O rescale is rare.
    const bool raise = mt > m + 8.f;   // (m = -inf: any allowed key)
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float mn = raise ? mt : m;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m - mn) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[n][r] *= alpha;
      m = mn;
    }
    const float mu = m == -INFINITY ? 0.f : m;   // no finite logit yet: every P is 0
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[r] = __builtin_amdgcn_exp2f(BIAS ? sacc[hh][r] - mu : fmaf(sacc[hh][r], scale_log2, -mu));
        lsum += pv[r];
      }
      const bf16x8 p0 = pack8(pv), p1 = pack8(pv + 8);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        o[n] = mfma(lds_trB(sm.vt[cur], trV, 32 * hh, 32 * n, T), p0, o[n]);
        o[n] = mfma(lds_trB(sm.vt[cur], trV, 32 * hh + 16, 32 * n, T), p1, o[n]);
      }
    }
    if (it + 1 < n_it) stg.store(sm, cur ^ 1);
    __syncthreads();
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (irow < Sq) {
    const bool live = ltot > 0.f;
    const float inv = live ? 1.f / ltot : 0.f;
    OT* op = (OT*)a.o + sv.q_off(p.o_str, b) + h * p.o_str[1] + (int64_t)irow * p.o_str[2];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        float v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = o[n][4 * qd + e] * inv;
        store4(op + 32 * n + 8 * qd + 4 * lg, v4);
      }
    }
    if (lg == 0)
      a.lse[((int64_t)b * p.Hq + h) * p.Sq + irow] =
          live ? (m + log2f(ltot)) * 0.6931471805599453f : -INFINITY;
  }
}

template <int D, int KT, bool BIAS>
hipError_t launch_fwd_d(const Params& p, const FwdArgs& a, bool o_bf16, hipStream_t st) {
  const dim3 grid((p.Sq + BQF - 1) / BQF, p.Hq, p.B);
  if (o_bf16)
    hipLaunchKernelGGL((k_fwd<D, KT, BIAS, unsigned short>), grid, dim3(NTF), 0, st, p, a);
  else
    hipLaunchKernelGGL((k_fwd<D, KT, BIAS, float>), grid, dim3(NTF), 0, st, p, a);
  return hipGetLastError();
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

}  // namespace

bool mfma_fwd_supported(const Params& p, const FwdArgs& a, bool o_bf16) {
  if (p.Dqk != p.Dv || (p.Dqk != 64 && p.Dqk != 128)) return false;
  const int64_t* s[] = {p.q_str, p.k_str, p.v_str};
  for (const int64_t* x : s)
    for (int i = 0; i < 3; ++i)
      if (x[i] % 8 != 0) return false;
  if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v)) return false;
  // O is written four elements at a time
  for (int i = 0; i < 3; ++i)
    if (p.o_str[i] % 4 != 0) return false;
  if (((uintptr_t)a.o & (o_bf16 ? 7u : 15u)) != 0) return false;
  // bias tiles are staged 16 bytes at a time
  if (a.bias && (!aligned16(a.bias) || p.Sk % 4 != 0 || p.bias_str[0] % 4 != 0 || p.bias_str[1] % 4 != 0))
    return false;
  return true;
}

hipError_t launch_fwd_mfma(const Params& p, const FwdArgs& a0, bool o_bf16, hipStream_t st) {
  if (p.Sq == 0 || p.B == 0 || p.Hq == 0) return hipSuccess;
  FwdArgs a = a0;
  a.xmajor = xmajor_fits(p, p.Hq, p.B) ? 1 : 0;   // grid (row blocks, Hq, B)
  const bool bias = a.bias != nullptr;
  if (p.Dqk == 64)
    return bias ? launch_fwd_d<64, 32, true>(p, a, o_bf16, st) : launch_fwd_d<64, 64, false>(p, a, o_bf16, st);
  return bias ? launch_fwd_d<128, 32, true>(p, a, o_bf16, st) : launch_fwd_d<128, 64, false>(p, a, o_bf16, st);
}

}  // namespace attn
