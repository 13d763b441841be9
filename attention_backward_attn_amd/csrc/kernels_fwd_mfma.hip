// bf16 matrix-core (gfx950 MFMA) attention forward with the row log-sum-exp.
//
// Math (ring-attention gist, _flash_fwd returning (out, lse); CK FMHA
// example 34 cpu_fwd_with_intermediates; CK FMHA example 22
// cpu_attention_fwd_masked, with the sink logit added to the normaliser):
//   S = scale Q K^T (+ bias),  LSE_i = log(sum_j exp S_ij + exp sink),
//   O = exp(S - LSE) V.  Rows with no allowed key and no sink: O = 0,
//   LSE = -inf.
//
// Without a bias the forward runs k_fwd2 (below: buffer-to-LDS tiles in one
// swizzled copy, the S chain among the previous tile's O products); k_fwd
// serves problems with a bias.
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

// ---------------------------------------------------------------------------
// Kernel k_fwd2 (no bias): the forward on the dQ pass's staging.  One
// workgroup of four waves per (128-row block, query head, batch), two per
// CU; wave w owns rows [32 w, 32 w + 32) with its Q fragments in registers.
// 32-key K / V tiles come straight from global memory into four LDS buffers
// (one swizzled copy per tile: row reads of K for S^T = K Q^T, transposing
// reads of V for O^T += V^T P^T), two tiles ahead.  Per tile t (one
// barrier) the S^T chain of tile t runs among the O^T products of tile
// t - 1; then the online softmax of tile t (running maximum raised only by
// more than 8, O rescaled then, per-lane normaliser shares) forms P(t) as
// the B operand of the next tile's products.
// ---------------------------------------------------------------------------
constexpr int NBF = 4;    // K / V tile buffers (k_fwd2)
constexpr int KTF = 32;   // keys per tile (k_fwd2)

template <int D>
struct __attribute__((aligned(1024))) SmemFwd2 {
  unsigned char k[NBF][KTF * 2 * D];   // K tile, swizzled
  unsigned char v[NBF][KTF * 2 * D];   // V tile, swizzled
};

template <int D, typename OT>
__global__ __launch_bounds__(NTF, 2) void k_fwd2(Params p, FwdArgs a) {
  constexpr int NS = D / 16;   // k-steps of S^T over the head dim
  constexpr int NB = D / 32;   // 32-column blocks of O (rows of O^T)
  constexpr int RB = Swz<D>::RB, CR = Swz<D>::CR;
  constexpr int TS = KTF * 2 * D;          // tile bytes
  constexpr int PER_T = KTF * CR / 64;     // 1 KB loads per tile
  constexpr int NI = 2 * PER_T / 4;        // loads per wave per K + V tile pair
  static_assert(NI >= 1 && PER_T % NI == 0, "loads per wave");
  __shared__ SmemFwd2<D> sm;

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
  const unsigned short* q = (const unsigned short*)a.q + sv.q_off(p.q_str, b) + h * p.q_str[1];
  const unsigned short* kp = (const unsigned short*)a.k + sv.k_off(p.k_str, b) + g * p.k_str[1];
  const unsigned short* vp = (const unsigned short*)a.v + sv.k_off(p.v_str, b) + g * p.v_str[1];

  // key tiles: the sink tiles [0, a1), then the band tiles [a2, a3)
  int64_t s_hi, b_lo, b_hi;
  msk.keys_for_rows(i0, min(i0 + BQF, Sq), Sk, &s_hi, &b_lo, &b_hi);
  const int a1 = (int)((s_hi + KTF - 1) / KTF);
  int a2 = (int)(b_lo / KTF);
  const int a3 = b_hi > b_lo ? (int)((b_hi + KTF - 1) / KTF) : a2;
  if (a2 < a1) a2 = a1;
  const int n1 = a1, n2 = a3 > a2 ? a3 - a2 : 0;
  const int n_it = Sk > 0 ? n1 + n2 : 0;
  auto tile_of = [&](int it) { return KTF * (it < n1 ? it : a2 + (it - n1)); };
  // masked tiles: key j is allowed for this lane's row when it is inside the
  // problem and  j + k_off - (irow + q_off) - diag  lies in [lo_l, lo_l + span]
  // (or it is a sink)
  const bool no_mask = msk.kind == kMaskNone;
  int lo_l = msk.wl < 0 ? -0x3fffffff : -msk.wl, span = msk.wr - lo_l;
  if (no_mask) { lo_l = -0x3fffffff; span = 0x7ffffffe; }
  const int tq = (int)msk.k_off - (irow + (int)msk.q_off) - (int)msk.diag + 4 * lg - lo_l;
  const int sink_lim = (int)min<int64_t>(max<int64_t>(msk.n_sink - msk.k_off, 0), 0x3fffffff);
  // a tile is full for this wave when every key is inside the problem and
  // allowed for all 32 of its rows
  const int wr0 = i0 + 32 * w;
  auto clamp_i = [](int64_t x) { return (int)max<int64_t>(min<int64_t>(x, 0x3fffffff), -0x3fffffff); };
  const int64_t band = (int64_t)wr0 + msk.q_off + msk.diag - msk.k_off;
  const int fl_hi = no_mask ? 0x3fffffff : clamp_i(band + msk.wr - 31);
  const int fl_lo = (no_mask || msk.wl < 0) ? -0x3fffffff : clamp_i(band + 31 - msk.wl);
  const int fl_sink = no_mask ? -0x3fffffff : clamp_i((int64_t)msk.n_sink - 31 - msk.k_off);
  auto tile_full = [&](int j0) { return (j0 + KTF <= Sk) & ((j0 < fl_sink) | ((j0 <= fl_hi) & (j0 >= fl_lo))); };

  // staging: wave w issues NI 1 KB loads of the K (waves 0, 1) or V tile
  const int k_rb = 2 * (int)p.k_str[2], v_rb = 2 * (int)p.v_str[2];
  const bool ld_v = w * NI >= PER_T;
  const unsigned int sm_base = __builtin_amdgcn_readfirstlane(lds_addr(&sm));
  int voff[NI];
  unsigned int dst0[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int slot = (w * NI + k) % PER_T;
    const int row = (64 * slot + l) / CR;
    voff[k] = row * (ld_v ? v_rb : k_rb) + 16 * ((l % CR) ^ Swz<D>::f(row));
    dst0[k] = sm_base + (ld_v ? offsetof(SmemFwd2<D>, v) : offsetof(SmemFwd2<D>, k)) + 1024 * slot;
  }
  const unsigned short* const src0 = ld_v ? vp : kp;
  const int64_t src_str = ld_v ? p.v_str[2] : p.k_str[2];
  const int src_rb = ld_v ? v_rb : k_rb;
  int ld_it = 0, ld_j0 = tile_of(0);
  const unsigned short* ld_src = src0 + (int64_t)ld_j0 * src_str;
  auto issue = [&](int buf) {
    const int keys = min(Sk - ld_j0, KTF);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(ld_src, keys * src_rb);
#pragma unroll
    for (int k = 0; k < NI; ++k) lds_dma16(rs, __builtin_amdgcn_readfirstlane(dst0[k] + buf * TS), voff[k]);
    if (++ld_it == n1) {
      ld_j0 = KTF * a2;
      ld_src = src0 + (int64_t)ld_j0 * src_str;
    } else {
      ld_j0 += KTF;
      ld_src += KTF * src_str;
    }
  };

  // running row maximum (log2 units) and this lane's share of the
  // normaliser; the sink contributes exp2(sink - m) = 1 at m = sink, counted
  // once per row
  float m = -INFINITY, lsum = 0.f;
  if (a.sinks) {
    m = a.sinks[h] * kLog2e;
    lsum = lg == 0 ? 1.f : 0.f;
  }
  f32x16 o[NB];   // O^T: this lane's row, head-dim columns 32 n + crow(r, lg)
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = zero16();

  if (n_it > 0) {
    // tiles 0 and 1 and the Q fragments (B operands) in flight together
    issue(0);
    if (n_it > 1) issue(1);
    bf16x8 qB[NS];
    {
      const int64_t ic = min(irow, Sq - 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) qB[s] = as_bf16x8(*(const u16x8*)(q + ic * p.q_str[2] + 16 * s + 8 * lg));
    }
    wait_vm_loads();

    // operand lane addresses in tile buffer 0: K rows (A of S^T, chain step s
    // at ka ^ 32 s) and V^T by transposing reads (A of O^T: head-dim block n,
    // keys 16 kk ..)
    const int a_lane = Swz<D>::a_lane(l), t_lane = Swz<D>::t_lane(l);
    const unsigned int k_t0 = sm_base + offsetof(SmemFwd2<D>, k), v_t0 = sm_base + offsetof(SmemFwd2<D>, v);
    const unsigned int ka = k_t0 + a_lane;
    unsigned int br[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) br[n] = v_t0 + (t_lane ^ (64 * n));
    auto read_k = [&](int j, int s) { return lds_b128_at((ka ^ (32 * s)) + j * TS); };
    auto read_vt = [&](int j, int i) {
      const int n = i % NB, r0 = 16 * (i / NB);
      return cat44(lds_tr4_at(br[n] + j * TS + r0 * RB), lds_tr4_at((br[n] ^ 32) + j * TS + (r0 + 8) * RB));
    };
    constexpr int AHEAD = 2;
    // P of the previous tile (B operands of its O^T products); zeros before
    // the first tile, against V tile buffer NBF - 1, zeroed here
    bf16x8 P0 = as_bf16x8(u16x8{0, 0, 0, 0, 0, 0, 0, 0}), P1 = P0;
#pragma unroll
    for (int k = 0; k < TS / (16 * NTF); ++k) *(u16x8*)&sm.v[NBF - 1][16 * (tid + NTF * k)] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};

    // tile t in buffer j: the S^T chain of tile t among the O^T products of
    // tile t - 1 (buffer jp), then the softmax of tile t
    auto tile = [&](auto jc, bool full, int j0) {
      constexpr int j = decltype(jc)::value, jp = (j + NBF - 1) % NBF;
      // Issue priority low over the products, raised over the softmax: the
      // two waves sharing a SIMD come from different workgroups and run in
      // any phase, and the one in its softmax then issues first while the
      // other's products keep the matrix pipe busy (measured on GQA 32:8,
      // S = 4096, D = 128, causal: 0.156 -> 0.154 ms).
      __builtin_amdgcn_s_setprio(0);
      f32x16 sacc = zero16();
      {
        bf16x8 xk[NS], bv[NS];
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) { xk[i] = read_k(j, i); bv[i] = read_vt(jp, i); }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          sacc = mfma(xk[i], qB[i], sacc);
          o[i % NB] = mfma(bv[i], i < NB ? P0 : P1, o[i % NB]);
          if (i + AHEAD < NS) { xk[i + AHEAD] = read_k(j, i + AHEAD); bv[i + AHEAD] = read_vt(jp, i + AHEAD); }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(1);
      // softmax of tile t: masked logits to -inf, the tile maximum over the
      // row's two lanes, the running maximum raised (and O rescaled) only by
      // more than 8, then P = 2^(S scale log2(e) - m)
      if (!full) {
        const int tb = tq + j0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 8 * (r >> 2) + (r & 3);
          const int jj = j0 + 4 * lg + c;
          const bool ok = (jj < Sk) & (((unsigned int)(tb + c) <= (unsigned int)span) | (jj < sink_lim));
          sacc[r] = ok ? sacc[r] : -INFINITY;
        }
      }
      float mt = sacc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * scale_log2;
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
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, -mu));
        lsum += pv[r];
      }
      P0 = pack8(pv);
      P1 = pack8(pv + 8);
    };
    int cur_it = 0, cur_j0 = tile_of(0);
    auto step = [&](int t, auto jc) {
      constexpr int j = decltype(jc)::value;
      __syncthreads();   // tile t complete; tile t - 2's buffer free
      const bool more = t + 2 < n_it;
      if (more) issue((j + 2) % NBF);
      tile(jc, tile_full(cur_j0), cur_j0);
      if (++cur_it == n1) cur_j0 = KTF * a2;
      else cur_j0 += KTF;
      wait_vm_keep<NI>(more);   // tile t + 1 complete before the next barrier
    };
    int t = 0;
    for (; t + NBF <= n_it; t += NBF) {
      step(t, std::integral_constant<int, 0>{});
      step(t + 1, std::integral_constant<int, 1>{});
      step(t + 2, std::integral_constant<int, 2>{});
      step(t + 3, std::integral_constant<int, 3>{});
    }
    if (t < n_it) step(t, std::integral_constant<int, 0>{});
    if (t + 1 < n_it) step(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 < n_it) step(t + 2, std::integral_constant<int, 2>{});
    // the O^T products of the last tile
    {
      const unsigned int jb = ((n_it - 1) % NBF) * TS;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int n = i % NB, r0 = 16 * (i / NB);
        const bf16x8 bv = cat44(lds_tr4_at(br[n] + jb + r0 * RB), lds_tr4_at((br[n] ^ 32) + jb + (r0 + 8) * RB));
        o[n] = mfma(bv, i < NB ? P0 : P1, o[n]);
      }
    }
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
  if (!BIAS) {
    if (o_bf16)
      hipLaunchKernelGGL((k_fwd2<D, unsigned short>), grid, dim3(NTF), 0, st, p, a);
    else
      hipLaunchKernelGGL((k_fwd2<D, float>), grid, dim3(NTF), 0, st, p, a);
    return hipGetLastError();
  }
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
