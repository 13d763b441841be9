// bf16 matrix-core kernels for head dim 512 with one tensor serving as both
// keys and values (the shared-KV layout of the CANN sparse_flash_mla_grad
// page: "Formula", sliding-window case, where the selected KV is the
// original KV).  Three kernels:
//   k_fwd512  O, LSE                       (online softmax; the producer)
//   k_dq512   dQ = scale * dS KV           (query-parallel, no atomics)
//   k_dkv512  dKV = scale * dS^T Q + P^T dO (key-parallel; dK and dV of the
//             shared tensor summed, per that page's Phase 3)
// All use v_mfma_f32_16x16x32_bf16 at one wave per SIMD.  At D = 512 a wave
// keeps 16 rows (or keys) of fragments and a 16 x 512 fp32 accumulator in
// registers; the other operand streams through LDS in padded 1 KB rows.
//
// MFMA 16x16x32 bf16 operand layout (lane l, g = l / 16, r = 0..3):
//   A[m][k]: lane holds m = l % 16, k = 8 g + 0..7
//   B[k][n]: lane holds n = l % 16, k = 8 g + 0..7
//   C[m][n]: lane holds n = l % 16, m = 4 g + r
// Products whose reduction runs over 32 keys (or rows) use the slot order of
// two 16-row accumulator halves: slot 8 g + e is key 4 g + e for e < 4 and
// 16 + 4 g + (e - 4) otherwise, on both operands.
#include <stddef.h>

#include "kernels.h"
#include "mfma_util.h"

namespace attn {
namespace {

using namespace mfma_util;

constexpr int XD = 512;          // head dim
constexpr int XRB = 2 * XD;      // row bytes (bf16)
constexpr int XNT = 256;         // threads per workgroup (4 waves)
constexpr int XNS = XD / 32;     // k-steps over the head dim (16)
constexpr int XNC = XD / 16;     // 16-column blocks of the head dim (32)
constexpr int XBK = 32;          // keys per tile (forward, dQ)
constexpr int XBQ = 64;          // query rows per workgroup (forward, dQ)
constexpr int XTS = XBK * (XRB + 32);   // key tile bytes (32 padded rows)
constexpr int XNB = 4;           // key tile buffers (forward, dQ)
constexpr int YBK = 64;          // keys per workgroup (dKV)
constexpr int YBQ = 32;          // query rows per tile (dKV)
constexpr int YTS = YBQ * (XRB + 32);   // Q or dO tile bytes (32 padded rows)

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// LDS rows of 1 KB padded to 1056 bytes.  Measured on gfx950 with the two
// operand read patterns below (in-bounds probe), this stride serves both at
// full speed -- ds_read_b128 of one 16-byte chunk of 16 consecutive rows at
// 2.7 cycles per wave instruction per CU, ds_read_b64_tr_b16 of 4 x 8 bytes
// of 16 consecutive rows at 1.67 -- while unpadded 1 KB rows with chunks
// XOR-permuted per row run the row reads at 4.5.  Every operand address is
// then a lane base plus a constant.
constexpr int XRS = XRB + 32;      // LDS row stride (bytes)
constexpr int XHS = 16 * XRS;      // second 16-row half of a tile
// row-read lane base: row l % 16, chunk l / 16 (k-step s at + 64 s)
__device__ inline int a_lane_of(int l) { return (l & 15) * XRS + 16 * (l >> 4); }
// transposing-read lane base: lane 4 e + q of 16-lane group g addresses row
// 4 g + e, columns 4 q .. 4 q + 3 (column block nb at + 32 nb)
__device__ inline int t_lane_of(int l) { return (4 * (l >> 4) + ((l & 15) >> 2)) * XRS + 8 * (l & 3); }

// Per-lane read addresses of one tile: row reads and transposing reads.
struct TileAddr {
  unsigned int a, t;
  __device__ inline void set(unsigned int tile, int a_lane, int t_lane) {
    a = tile + a_lane;
    t = tile + t_lane;
  }
  // A operand: rows 16 h + l % 16, head-dim step s
  __device__ inline bf16x8 row(int h, int s) const { return lds_b128_at(a + 64 * s + XHS * h); }
  // transposed operand of column block nb over the tile's 32 rows in slot order
  __device__ inline bf16x8 tr(int nb) const {
    const unsigned int x = t + 32 * nb;
    return cat44(lds_tr4_at(x), lds_tr4_at(x + XHS));
  }
};

// Pack the two halves of a 32-key (or 32-row) accumulator pair into an
// operand in slot order.
__device__ inline bf16x8 pack_halves(const float* v) {   // v[0..3]: half 0, v[4..7]: half 1
  return pack8(v);
}

// Direct loads of a tile of rows (1 KB each) into padded LDS rows: one load
// per row, lane l bringing its 16-byte chunk l.  Rows past `rows` (the buffer
// resource's extent) arrive as zeros.
__device__ inline void stage_rows(const unsigned short* src, int64_t row_str, int rows, unsigned int lds_tile,
                                  int r0, int nrows, int l) {
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(src, rows * (int)(2 * row_str));
  for (int k = 0; k < nrows; ++k) {
    const int r = r0 + k;
    lds_dma16(rs, __builtin_amdgcn_readfirstlane(lds_tile + r * XRS), r * (int)(2 * row_str) + 16 * l);
  }
}

// Key tiles seen by a block of query rows: the sink tiles [0, a1) and the
// band tiles [a2, a3) (keys_for_rows), in 32-key units.
struct KeyTiles {
  int n1, a2, n_it;
  __device__ inline int j0(int it) const { return XBK * (it < n1 ? it : a2 + (it - n1)); }
};

__device__ inline KeyTiles key_tiles(const Mask& msk, int i0, int i1, int Sk) {
  int64_t s_hi, b_lo, b_hi;
  msk.keys_for_rows(i0, i1, Sk, &s_hi, &b_lo, &b_hi);
  const int a1 = (int)((s_hi + XBK - 1) / XBK);
  int a2 = (int)(b_lo / XBK);
  const int a3 = b_hi > b_lo ? (int)((b_hi + XBK - 1) / XBK) : a2;
  if (a2 < a1) a2 = a1;
  KeyTiles kt;
  kt.n1 = a1;
  kt.a2 = a2;
  kt.n_it = a1 + (a3 > a2 ? a3 - a2 : 0);
  return kt;
}

// Per-lane mask of a 32-key tile for one query row (the lane's), keys
// j0 + 16 h + 4 g + r: allowed when the window offset lies in [lo, lo + span]
// or the key is a sink, and the key exists.
struct RowMask {
  int tq, span, sink_lim, Sk;
  // 16 rows starting at wr0: tile [j0, j0 + 32) fully allowed
  int fl_hi, fl_lo, fl_sink;
  __device__ inline void init(const Mask& msk, int irow, int wr0, int g, int Sk_) {
    Sk = Sk_;
    const bool no_mask = msk.kind == kMaskNone;
    int lo = msk.wl < 0 ? -0x3fffffff : -msk.wl;
    span = msk.wr - lo;
    if (no_mask) { lo = -0x3fffffff; span = 0x7ffffffe; }
    tq = (int)msk.k_off - (irow + (int)msk.q_off) - (int)msk.diag + 4 * g - lo;
    sink_lim = (int)min<int64_t>(max<int64_t>(msk.n_sink - msk.k_off, 0), 0x3fffffff);
    auto clamp_i = [](int64_t x) { return (int)max<int64_t>(min<int64_t>(x, 0x3fffffff), -0x3fffffff); };
    const int64_t band = (int64_t)wr0 + msk.q_off + msk.diag - msk.k_off;
    fl_hi = no_mask ? 0x3fffffff : clamp_i(band + msk.wr - (XBK - 1));
    fl_lo = (no_mask || msk.wl < 0) ? -0x3fffffff : clamp_i(band + 15 - msk.wl);
    fl_sink = no_mask ? -0x3fffffff : clamp_i((int64_t)msk.n_sink - (XBK - 1) - msk.k_off);
  }
  __device__ inline bool full(int j0) const {
    return (j0 + XBK <= Sk) & ((j0 < fl_sink) | ((j0 <= fl_hi) & (j0 >= fl_lo)));
  }
  // element (h, r) of the tile at j0 for lane group g
  __device__ inline bool ok(int j0, int g, int h, int r) const {
    const int jj = j0 + 16 * h + 4 * g + r;
    const int tb = tq + j0 + 16 * h + r;
    return (jj < Sk) & (((unsigned int)tb <= (unsigned int)span) | (jj < sink_lim));
  }
};

// ---------------------------------------------------------------------------
// k_fwd512: one workgroup of four waves per (64 query rows, query head,
// batch entry); wave w owns rows 16 w .. 16 w + 15 with their Q fragments in
// registers.  Per 32-key tile: S^T = KV Q^T (one query row per lane), online
// softmax in log2 units, O^T += KV^T P^T -- so O also has one row per lane
// and the rescale is a per-lane scalar.  The running maximum is raised only
// when a tile exceeds it by more than 8 (P <= 256 stays exact enough in
// bf16 and fp32), so the rescale of O is rare.  Sink logits start the
// maximum and the normaliser (the sink term of the CK sink example's
// softmax and of that page's SimpleSoftmax(sinks, lse)).
// ---------------------------------------------------------------------------
struct __attribute__((aligned(1024))) SmemX {
  unsigned char k[XNB][XTS];
};

template <bool OBF16>
__global__ __launch_bounds__(XNT, 1) void k_fwd512(Params p, FwdArgs a) {
  __shared__ SmemX sm;
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const BlockXYZ blk = a.xmajor ? xcd_block_xmajor() : xcd_block();
  const bool heavy_last = p.mask.kind != kMaskNone && p.mask.wl < 0;
  const int i0 = (heavy_last ? (int)gridDim.x - 1 - blk.x : blk.x) * XBQ;
  const int h = blk.y, b = blk.z, hk = h / p.G;
  const SeqView sv = seq_view(p, b);
  const Mask& msk = sv.mask;
  const int Sq = sv.Sq, Sk = sv.Sk;
  if (i0 >= Sq) return;
  const int irow = i0 + 16 * w + lr;
  const float scale_log2 = p.scale * kLog2e;

  const unsigned short* q = (const unsigned short*)a.q + sv.q_off(p.q_str, b) + h * p.q_str[1];
  const unsigned short* kv = (const unsigned short*)a.k + sv.k_off(p.k_str, b) + hk * p.k_str[1];
  const KeyTiles kt = key_tiles(msk, i0, min(i0 + XBQ, Sq), Sk);
  RowMask rm;
  rm.init(msk, irow, i0 + 16 * w, g, Sk);
  const unsigned int sm_base = __builtin_amdgcn_readfirstlane(lds_addr(&sm));
  const int a_lane = a_lane_of(l), t_lane = t_lane_of(l);
  auto issue = [&](int it) {
    const int j0 = kt.j0(it);
    stage_rows(kv + (int64_t)j0 * p.k_str[2], p.k_str[2], min(Sk - j0, XBK), sm_base + (it % XNB) * XTS, 8 * w, 8, l);
  };

  const int n_it = kt.n_it;
  // key tiles 0 and 1 in flight before the fragment loads
  if (n_it > 0) issue(0);
  if (n_it > 1) issue(1);
  bf16x8 qB[XNS];
  {
    const int64_t ic = min(irow, Sq - 1);
#pragma unroll
    for (int s = 0; s < XNS; ++s) qB[s] = as_bf16x8(*(const u16x8*)(q + ic * p.q_str[2] + 32 * s + 8 * g));
  }
  // running maximum (log2 units) and this lane's part of the normaliser
  float m_run = -INFINITY, l_run = 0.f;
  if (a.sinks) {
    m_run = a.sinks[h] * kLog2e;
    l_run = g == 0 ? 1.f : 0.f;
  }

  wait_vm_loads();   // fragments and both key tiles

  f32x4 o[XNC];
#pragma unroll
  for (int n = 0; n < XNC; ++n) o[n] = zero4();
  bf16x8 Pb = as_bf16x8(u16x8{0, 0, 0, 0, 0, 0, 0, 0});
  if (n_it > 0) {
    // One tile step: the S^T chains of tile t (when HC) among the O^T
    // products of tile t - 1 (when HP), operands two product steps ahead,
    // then the online softmax of tile t.  First and last steps peeled.
    auto step = [&](int t, auto hc_, auto hp_) {
      constexpr bool HC = decltype(hc_)::value, HP = decltype(hp_)::value;
      constexpr int AH = 3;
      __syncthreads();   // tile t complete; tile t - 3's buffer free
      if (t + 2 < n_it) issue(t + 2);
      TileAddr cur, prv;
      if (HC) cur.set(sm_base + (t % XNB) * XTS, a_lane, t_lane);
      if (HP) prv.set(sm_base + ((t + XNB - 1) % XNB) * XTS, a_lane, t_lane);
      f32x4 sacc[2] = {zero4(), zero4()};
      bf16x8 k0[XNS], k1[XNS], bt[XNC];
#pragma unroll
      for (int i = 0; i < AH; ++i) {
        if (HC) { k0[i] = cur.row(0, i); k1[i] = cur.row(1, i); }
        if (HP) { bt[2 * i] = prv.tr(2 * i); bt[2 * i + 1] = prv.tr(2 * i + 1); }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < XNS; ++s) {
        if (HC) sacc[0] = mfma16(k0[s], qB[s], sacc[0]);
        if (HP) o[2 * s] = mfma16(bt[2 * s], Pb, o[2 * s]);
        if (HC) sacc[1] = mfma16(k1[s], qB[s], sacc[1]);
        if (HP) o[2 * s + 1] = mfma16(bt[2 * s + 1], Pb, o[2 * s + 1]);
        if (s + AH < XNS) {
          if (HC) { k0[s + AH] = cur.row(0, s + AH); k1[s + AH] = cur.row(1, s + AH); }
          if (HP) { bt[2 * (s + AH)] = prv.tr(2 * (s + AH)); bt[2 * (s + AH) + 1] = prv.tr(2 * (s + AH) + 1); }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (HC) {
        const int j0 = kt.j0(t);
        float sv8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sv8[e] = sacc[e >> 2][e & 3] * scale_log2;
        if (!rm.full(j0)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) sv8[e] = rm.ok(j0, g, e >> 2, e & 3) ? sv8[e] : -INFINITY;
        }
        float mt = sv8[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sv8[e]);
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const bool raise = mt > m_run + 8.f;   // (m_run = -inf: any allowed key)
        if (__builtin_amdgcn_ballot_w64(raise)) {
          const float m_new = raise ? mt : m_run;
          const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
          l_run *= alpha;
#pragma unroll
          for (int n = 0; n < XNC; ++n) o[n] *= alpha;
          m_run = m_new;
        }
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = sv8[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv8[e] - m_run);
          l_run += pv[e];
        }
        Pb = pack_halves(pv);
      }
      if (t + 1 < n_it) wait_vm_keep<8>(t + 2 < n_it);   // tile t + 1 complete before the next barrier
    };
    step(0, std::true_type{}, std::false_type{});
    for (int t = 1; t < n_it; ++t) step(t, std::true_type{}, std::true_type{});
    step(n_it, std::false_type{}, std::true_type{});
  }
  // normaliser of the row over its four lane groups
  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (irow < Sq) {
    char* ob = (char*)a.o + (sv.q_off(p.o_str, b) + h * p.o_str[1] + (int64_t)irow * p.o_str[2]) * (OBF16 ? 2 : 4);
#pragma unroll
    for (int n = 0; n < XNC; ++n) {
      const int c = 16 * n + 4 * g;
      if (OBF16) {
        unsigned short u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = f32_to_bf16_rne(o[n][r] * inv);
        *(u16x4*)(ob + 2 * c) = u16x4{u[0], u[1], u[2], u[3]};
      } else {
        *(f32x4*)(ob + 4 * c) = o[n] * inv;
      }
    }
    if (g == 0)
      a.lse[((int64_t)b * p.Hq + h) * p.Sq + irow] = lt > 0.f ? (m_run + __builtin_amdgcn_logf(lt)) * 0.6931471805599453f : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// k_dq512: the dQ pass.  Workgroup and row ownership as k_fwd512; wave w
// keeps Q and dO fragments of its 16 rows.  Per 32-key tile t (one barrier):
// S^T = KV Q^T and dP^T = KV dO^T as four chains sharing each KV row read,
// among the dQ^T products of tile t - 1; then P = exp2(S - LSE) and
// dS = P (dP - delta) (scale folded in) for tile t, published in LDS.  The
// products split the head dim: wave w accumulates dQ^T columns
// 128 w .. 128 w + 127 of all 64 rows, from the four waves' dS -- so each
// KV^T block is read once per workgroup rather than once per wave.
// ---------------------------------------------------------------------------
struct __attribute__((aligned(1024))) SmemXD {
  unsigned char k[XNB][XTS];
  bf16x8 ds[2][4][64];   // dS operands of the previous two tiles, per wave and lane
};

__global__ __launch_bounds__(XNT, 1) void k_dq512(Params p, BwdArgs a) {
  __shared__ SmemXD sm;
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const BlockXYZ blk = a.xmajor ? xcd_block_xmajor() : xcd_block();
  const bool heavy_last = p.mask.kind != kMaskNone && p.mask.wl < 0;
  const int i0 = (heavy_last ? (int)gridDim.x - 1 - blk.x : blk.x) * XBQ;
  const int h = blk.y, b = blk.z, hk = h / p.G;
  const SeqView sv = seq_view(p, b);
  const Mask& msk = sv.mask;
  const int Sq = sv.Sq, Sk = sv.Sk;
  if (i0 >= Sq) return;
  const int irow = i0 + 16 * w + lr;
  const float scale = p.scale, scale_log2 = p.scale * kLog2e;

  const unsigned short* q = (const unsigned short*)a.q + sv.q_off(p.q_str, b) + h * p.q_str[1];
  const unsigned short* dout = (const unsigned short*)a.dout + sv.q_off(p.do_str, b) + h * p.do_str[1];
  const unsigned short* kv = (const unsigned short*)a.k + sv.k_off(p.k_str, b) + hk * p.k_str[1];
  const KeyTiles kt = key_tiles(msk, i0, min(i0 + XBQ, Sq), Sk);
  RowMask rm;
  rm.init(msk, irow, i0 + 16 * w, g, Sk);
  const unsigned int sm_base = __builtin_amdgcn_readfirstlane(lds_addr(&sm));
  const int a_lane = a_lane_of(l), t_lane = t_lane_of(l);
  auto issue = [&](int it) {
    const int j0 = kt.j0(it);
    stage_rows(kv + (int64_t)j0 * p.k_str[2], p.k_str[2], min(Sk - j0, XBK), sm_base + (it % XNB) * XTS, 8 * w, 8, l);
  };

  const int n_it = kt.n_it;
  // key tiles 0 and 1 in flight before the fragment loads, so that their
  // latencies overlap
  if (n_it > 0) issue(0);
  if (n_it > 1) issue(1);
  bf16x8 qB[XNS], doB[XNS];
  {
    const int64_t ic = min(irow, Sq - 1);
#pragma unroll
    for (int s = 0; s < XNS; ++s) {
      qB[s] = as_bf16x8(*(const u16x8*)(q + ic * p.q_str[2] + 32 * s + 8 * g));
      doB[s] = as_bf16x8(*(const u16x8*)(dout + ic * p.do_str[2] + 32 * s + 8 * g));
    }
  }
  float lse2 = INFINITY, dls = 0.f;
  if (irow < Sq) {
    const float lv = a.lse[((int64_t)b * p.Hq + h) * p.Sq + irow];
    lse2 = lv == -INFINITY ? INFINITY : lv * kLog2e;
    dls = a.delta[((int64_t)b * p.Hq + h) * p.Sq + irow] * scale;
  }

  wait_vm_loads();   // fragments, LSE / delta and both key tiles

  // dQ^T of columns 128 w + 16 c + 4 g + r for rows 16 rb + lane % 16:
  // dq[4 c + rb], c = 0..7, rb = 0..3
  constexpr int NCW = XNC / 4;   // 16-column blocks per wave
  f32x4 dq[4 * NCW];
#pragma unroll
  for (int n = 0; n < 4 * NCW; ++n) dq[n] = zero4();
  const unsigned int ds_base = sm_base + offsetof(SmemXD, ds);
  if (n_it > 0) {
    // One tile step: the S^T / dP^T chains of tile t (when HC) among the
    // first half of the dQ^T products of tile t - 1 (when HP), then the
    // second half among the exponentials and dS arithmetic of tile t.
    // Operands are read ahead; the first and last steps are peeled, so the
    // main loop has no branches.
    auto step = [&](int t, auto hc_, auto hp_) {
      constexpr bool HC = decltype(hc_)::value, HP = decltype(hp_)::value;
      constexpr int AH = 3;
      __syncthreads();   // tile t complete, dS of tile t - 1 published; tile t - 3's buffer free
      if (t + 2 < n_it) issue(t + 2);
      TileAddr cur, prv;
      if (HC) cur.set(sm_base + (t % XNB) * XTS, a_lane, t_lane);
      // (transposing reads of this wave's column blocks: base offset to block NCW w)
      if (HP) prv.set(sm_base + ((t + XNB - 1) % XNB) * XTS, a_lane, t_lane + 32 * NCW * w);
      f32x4 sacc[2] = {zero4(), zero4()}, pacc[2] = {zero4(), zero4()};
      bf16x8 k0[XNS], k1[XNS], kt_[NCW], dsb[4];
      const unsigned int dsp = ds_base + ((t + 1) & 1) * (4 * 64 * 16) + 16 * l;   // dS of tile t - 1
#pragma unroll
      for (int i = 0; i < AH; ++i)
        if (HC) { k0[i] = cur.row(0, i); k1[i] = cur.row(1, i); }
      if (HP) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) dsb[rb] = lds_b128_at(dsp + rb * 64 * 16);
        kt_[0] = prv.tr(0);
        kt_[1] = prv.tr(1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // dQ^T product n = 4 c + rb (column block c, row block rb); the K^T
      // operand of block c + 2 is read when block c starts
      auto product = [&](int n) {
        if ((n & 3) == 0 && (n >> 2) + 2 < NCW) kt_[(n >> 2) + 2] = prv.tr((n >> 2) + 2);
        dq[n] = mfma16(kt_[n >> 2], dsb[n & 3], dq[n]);
      };
      // region 1: 64 chain products among dQ^T products 0 .. XNS - 3 (the
      // first two steps wait only for their own rows' reads)
      constexpr int D1 = 2;
#pragma unroll
      for (int s = 0; s < XNS; ++s) {
        if (HC) {
          sacc[0] = mfma16(k0[s], qB[s], sacc[0]);
          pacc[0] = mfma16(k0[s], doB[s], pacc[0]);
        }
        if (HP && s >= D1) product(s - D1);
        if (HC) {
          sacc[1] = mfma16(k1[s], qB[s], sacc[1]);
          pacc[1] = mfma16(k1[s], doB[s], pacc[1]);
        }
        if (HC && s + AH < XNS) { k0[s + AH] = cur.row(0, s + AH); k1[s + AH] = cur.row(1, s + AH); }
        __builtin_amdgcn_sched_barrier(0);
      }
      // region 2: the remaining dQ^T products among the exponentials and dS
      // of tile t
      float pv[8], dsv[8];
#pragma unroll
      for (int i = 0; i < XNC - (XNS - D1); ++i) {
        if (HP) product(XNS - D1 + i);
        if (HC && i < 16) {
          if (i < 8) pv[i] = __builtin_amdgcn_exp2f(fmaf(sacc[i >> 2][i & 3], scale_log2, -lse2));
          else dsv[i - 8] = pv[i - 8] * fmaf(pacc[(i - 8) >> 2][(i - 8) & 3], scale, -dls);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (HC) {
        const int j0 = kt.j0(t);
        if (!rm.full(j0)) {   // (the branch touches dS only)
#pragma unroll
          for (int e = 0; e < 8; ++e) dsv[e] = rm.ok(j0, g, e >> 2, e & 3) ? dsv[e] : 0.f;
        }
        // publish dS of tile t (read by every wave in the next step)
        *(lds_u16x8*)(size_t)(ds_base + (t & 1) * (4 * 64 * 16) + w * 64 * 16 + 16 * l) =
            __builtin_bit_cast(u16x8, pack_halves(dsv));
      }
      if (t + 1 < n_it) wait_vm_keep<8>(t + 2 < n_it);   // tile t + 1 complete before the next barrier
    };
    step(0, std::true_type{}, std::false_type{});
    for (int t = 1; t < n_it; ++t) step(t, std::true_type{}, std::true_type{});
    step(n_it, std::false_type{}, std::true_type{});
  }
  // dQ rows i0 + 16 rb + lane % 16, columns 128 w + 16 c + 4 g .. + 3
  float* dqp = a.dq + sv.q_off(p.dq_str, b) + h * p.dq_str[1];
  if (a.accumulate_dq) {   // every load ahead of the adds (in flight together)
    f32x4 old[4 * NCW];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int i = i0 + 16 * rb + lr;
#pragma unroll
      for (int c = 0; c < NCW; ++c)
        old[4 * c + rb] = i < Sq ? *(const f32x4*)(dqp + (int64_t)i * p.dq_str[2] + 128 * w + 16 * c + 4 * g)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int x = 0; x < 4 * NCW; ++x) dq[x] = old[x] + dq[x];
  }
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int i = i0 + 16 * rb + lr;
    if (i < Sq) {
#pragma unroll
      for (int c = 0; c < NCW; ++c)
        *(f32x4*)(dqp + (int64_t)i * p.dq_str[2] + 128 * w + 16 * c + 4 * g) = dq[4 * c + rb];
    }
  }
}

// ---------------------------------------------------------------------------
// k_dkv512: the dKV pass.  One workgroup of four waves per (64-key block,
// part of a KV head's query group, batch entry); wave w owns keys
// 16 w .. 16 w + 15 with their KV fragments, and a 64 x 128 fp32 slice of
// dKV^T in registers.  The workgroup walks the
// part's (head, 32-row tile) iterations; Q and dO tiles come straight into
// two padded LDS buffers, one tile ahead.  Per tile: S = Q KV^T and
// dP = dO KV^T for the wave's keys (one key per lane), P and dS, published
// in LDS; in the next step dKV^T += dO^T P + Q^T (scale dS) runs under the
// next tile's S / dP, split over the head dim: wave w accumulates columns
// 128 w .. 128 w + 127 for all 64 keys, from the four waves' P and dS, with
// its dO^T / Q^T operands read into registers during the tile's own step.
// The reduction over the tile's rows uses the accumulators' slot order.
// Several parts add into zeroed dKV.
// ---------------------------------------------------------------------------
struct __attribute__((aligned(1024))) SmemY {
  unsigned char q[2][YTS];
  unsigned char d[2][YTS];
  bf16x8 px[2][2][4][64];   // [tile parity][P, dS][wave][lane]: B operands of the dKV^T products
  float lse[2][64];   // raw LSE / delta rows (a wave-wide load fills 64 entries)
  float dl[2][64];
};

enum : int { kStoreX = 0, kAddIntoX = 1, kAtomicAddX = 2 };

// slots: with partial sums, part q >= 1 stores its dKV into slots + (q - 1)
// slot_elems, at the element offsets dKV has from a.dk (nullptr: none)
__global__ __launch_bounds__(XNT, 1) void k_dkv512(Params p, BwdArgs a, int parts, int out_mode, float* slots,
                                                    int64_t slot_elems) {
  __shared__ SmemY sm;
  const int tid = threadIdx.x, l = tid & 63, lr = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const BlockXYZ blk = xcd_block();
  const int kb = blk.x, hk = blk.y / parts, part = blk.y % parts, b = blk.z;
  const SeqView sv = seq_view(p, b);
  const Mask& msk = sv.mask;
  const int Sq = sv.Sq, Sk = sv.Sk;
  const int k0 = kb * YBK;
  if (k0 >= Sk) return;
  const int key = k0 + 16 * w + lr;   // this lane's key
  const float scale = p.scale, scale_log2 = p.scale * kLog2e;
  const int G = p.G, hp = G / parts;
  const int h_begin = hk * G + part * hp;

  const unsigned short* kv = (const unsigned short*)a.k + sv.k_off(p.k_str, b) + hk * p.k_str[1];
  bf16x8 kB[XNS];
  {
    const int64_t kc = min(key, Sk - 1);
#pragma unroll
    for (int s = 0; s < XNS; ++s) kB[s] = as_bf16x8(*(const u16x8*)(kv + kc * p.k_str[2] + 32 * s + 8 * g));
  }
  wait_vm_loads();

  // query rows that see this key block, in 32-row tiles aligned to 32
  int64_t lo, hi;
  msk.rows_for_keys(k0, min(k0 + YBK, Sk), Sq, &lo, &hi);
  const int lo_al = (int)(lo / YBQ) * YBQ;
  const int nqb = hi > lo ? (int)((hi - lo_al + YBQ - 1) / YBQ) : 0;
  const int n_it = hp * nqb;

  // per-lane mask of the tile rows 16 h + 4 g + r for this lane's key:
  // allowed when key + k_off - (row + q_off) - diag lies in [lo_w, lo_w + span]
  const bool no_mask = msk.kind == kMaskNone;
  int lo_w = msk.wl < 0 ? -0x3fffffff : -msk.wl, span = msk.wr - lo_w;
  if (no_mask) { lo_w = -0x3fffffff; span = 0x7ffffffe; }
  const bool sink_key = !no_mask && (int64_t)key + msk.k_off < msk.n_sink;
  if (no_mask || sink_key) { lo_w = -0x3fffffff; span = 0x7ffffffe; }
  const bool key_ok = key < Sk;
  const int tb0 = key + (int)msk.k_off - (int)msk.q_off - (int)msk.diag - 4 * g - lo_w;
  // tile rows [i0, i0 + 32) allowed for all 64 keys of the block
  auto clamp_i = [](int64_t x) { return (int)max<int64_t>(min<int64_t>(x, 0x3fffffff), -0x3fffffff); };
  int full_a = -0x3fffffff, full_c = 0x3fffffff;
  if (k0 + YBK > Sk) {
    full_a = 0x3fffffff;
  } else if (!no_mask && k0 + YBK - 1 + msk.k_off >= msk.n_sink) {
    const int64_t base = (int64_t)k0 + msk.k_off - msk.q_off - msk.diag;
    full_a = clamp_i(base + YBK - 1 - msk.wr);
    if (msk.wl >= 0) full_c = clamp_i(base + msk.wl);
  }

  const unsigned int sm_base = __builtin_amdgcn_readfirstlane(lds_addr(&sm));
  const int a_lane = a_lane_of(l), t_lane = t_lane_of(l);
  const int64_t lrow = (int64_t)p.Sq;   // rows per (batch, head) of LSE / delta
  // tile walk of the loads: heads outer, 32-row tiles inner; pointers to the
  // next tile's Q, dO, LSE and delta rows advance by one tile, and wrap to
  // the next head after the last row tile
  int ld_i0 = lo_al, cur_i0 = lo_al;
  const int i_end = lo_al + YBQ * nqb;
  const unsigned short* ld_q = (const unsigned short*)a.q + sv.q_off(p.q_str, b) + h_begin * p.q_str[1] + (int64_t)lo_al * p.q_str[2];
  const unsigned short* ld_d = (const unsigned short*)a.dout + sv.q_off(p.do_str, b) + h_begin * p.do_str[1] + (int64_t)lo_al * p.do_str[2];
  const int64_t rb0 = ((int64_t)b * p.Hq + h_begin) * lrow + lo_al;
  const float* ld_l = a.lse + rb0;
  const float* ld_dl = a.delta + rb0;
  const int64_t q_step = YBQ * p.q_str[2], d_step = YBQ * p.do_str[2];
  const int64_t q_wrap = p.q_str[1] - nqb * q_step, d_wrap = p.do_str[1] - nqb * d_step;
  const int64_t l_wrap = lrow - (int64_t)nqb * YBQ;
  auto issue = [&](int it) {
    const int i0 = ld_i0;
    const int rows = min(Sq - i0, YBQ);
    const int buf = it & 1;
    stage_rows(ld_q, p.q_str[2], rows, sm_base + offsetof(SmemY, q) + buf * YTS, 8 * w, 8, l);
    stage_rows(ld_d, p.do_str[2], rows, sm_base + offsetof(SmemY, d) + buf * YTS, 8 * w, 8, l);
    if (w == 0) {
      // raw LSE and delta of the tile's rows (zeros past the end)
      const __amdgpu_buffer_rsrc_t rl = buf_rsrc(ld_l, rows * 4), rd = buf_rsrc(ld_dl, rows * 4);
      // (lanes past the tile's rows read past the resource: zeros)
      lds_dma4(rl, __builtin_amdgcn_readfirstlane(sm_base + offsetof(SmemY, lse) + buf * 256), 4 * l);
      lds_dma4(rd, __builtin_amdgcn_readfirstlane(sm_base + offsetof(SmemY, dl) + buf * 256), 4 * l);
    }
    ld_i0 += YBQ;
    ld_q += q_step;
    ld_d += d_step;
    ld_l += YBQ;
    ld_dl += YBQ;
    if (ld_i0 >= i_end) {
      ld_i0 = lo_al;
      ld_q += q_wrap;
      ld_d += d_wrap;
      ld_l += l_wrap;
      ld_dl += l_wrap;
    }
  };
  // dKV^T of columns 128 w + 16 c + 4 g + r for keys k0 + 16 kb + lane % 16:
  // acc[4 c + kb]
  constexpr int NCW = XNC / 4;   // 16-column blocks per wave
  f32x4 acc[4 * NCW];
#pragma unroll
  for (int n = 0; n < 4 * NCW; ++n) acc[n] = zero4();
  // A operands of the products (dO^T, Q^T of this wave's column blocks over
  // a tile's 32 rows, slot order): read during the step of their tile, used
  // in the next one; block c is refilled right after its last use
  bf16x8 ad[NCW], aq[NCW];
  const unsigned int px_base = sm_base + offsetof(SmemY, px);
  if (n_it > 0) {
    issue(0);
    wait_vm(0);
    // One step u: S = Q KV^T and dP = dO KV^T of tile u (when HC) among the
    // dKV^T products of tile u - 1 (when HP), which take the four waves' P
    // and dS from LDS; then P and dS of tile u, published for the next step.
    auto step = [&](int u, auto hc_, auto hp_) {
      constexpr bool HC = decltype(hc_)::value, HP = decltype(hp_)::value;
      constexpr int AH = 2, D1 = 2;
      __syncthreads();   // tile u complete; P / dS of tile u - 1 published; tile u - 1's buffer free
      if (HC && u + 1 < n_it) issue(u + 1);
      const int buf = u & 1;
      const int i0 = cur_i0;
      if (HC) {
        cur_i0 += YBQ;
        if (cur_i0 >= i_end) cur_i0 = lo_al;
      }
      // row reads of the chains; transposing reads of this wave's column
      // blocks (base offset to block NCW w)
      TileAddr tq, td, tqw, tdw;
      if (HC) {
        tq.set(sm_base + offsetof(SmemY, q) + buf * YTS, a_lane, t_lane);
        td.set(sm_base + offsetof(SmemY, d) + buf * YTS, a_lane, t_lane);
        tqw.set(sm_base + offsetof(SmemY, q) + buf * YTS, a_lane, t_lane + 32 * NCW * w);
        tdw.set(sm_base + offsetof(SmemY, d) + buf * YTS, a_lane, t_lane + 32 * NCW * w);
      }
      bf16x8 pb[4], sb[4];
      if (HP) {
        const unsigned int pxp = px_base + (buf ^ 1) * (2 * 4 * 64 * 16) + 16 * l;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          pb[kb] = lds_b128_at(pxp + kb * 64 * 16);
          sb[kb] = lds_b128_at(pxp + 4 * 64 * 16 + kb * 64 * 16);
        }
      }
      f32x4 sacc[2] = {zero4(), zero4()}, pacc[2] = {zero4(), zero4()};
      bf16x8 xq0[XNS], xq1[XNS], xd0[XNS], xd1[XNS];
      if (HC) {
#pragma unroll
        for (int i = 0; i < AH; ++i) {
          xq0[i] = tq.row(0, i); xd0[i] = td.row(0, i); xq1[i] = tq.row(1, i); xd1[i] = td.row(1, i);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // product n of tile u - 1: column block c = n / 8; n % 8 < 4: dO^T P
      // into key block n % 4, else Q^T dS; after the last product of block c
      // its operands are refilled from tile u
      auto product = [&](int n) {
        const int c = n >> 3, kb = n & 3;
        if ((n & 4) == 0) acc[4 * c + kb] = mfma16(ad[c], pb[kb], acc[4 * c + kb]);
        else acc[4 * c + kb] = mfma16(aq[c], sb[kb], acc[4 * c + kb]);
        if (HC && (n & 7) == 7) { ad[c] = tdw.tr(c); aq[c] = tqw.tr(c); }
      };
      constexpr int NP = 4 * NCW * 2;   // 64 products
      // region 1: the four chains, products 0 .. 2 (XNS - D1) - 1
#pragma unroll
      for (int s = 0; s < XNS; ++s) {
        if (HC) {
          sacc[0] = mfma16(xq0[s], kB[s], sacc[0]);
          pacc[0] = mfma16(xd0[s], kB[s], pacc[0]);
        }
        if (HP && s >= D1) product(2 * (s - D1));
        if (HC) {
          sacc[1] = mfma16(xq1[s], kB[s], sacc[1]);
          pacc[1] = mfma16(xd1[s], kB[s], pacc[1]);
        }
        if (HP && s >= D1) product(2 * (s - D1) + 1);
        if (HC && s + AH < XNS) {
          xq0[s + AH] = tq.row(0, s + AH); xd0[s + AH] = td.row(0, s + AH);
          xq1[s + AH] = tq.row(1, s + AH); xd1[s + AH] = td.row(1, s + AH);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!HP && HC) {   // first step: nothing to refill behind, read every block now
#pragma unroll
        for (int c = 0; c < NCW; ++c) { ad[c] = tdw.tr(c); aq[c] = tqw.tr(c); }
      }
      // region 2: the remaining products among P = exp2(S scale log2 e -
      // LSE log2 e) (LSE -inf: a row without keys, P = 0) and
      // dS = P (dP - delta) scale of tile u
      float pv[8], dsv[8];
      f32x4 L0, L1, D0, D1v;
      if (HC) {
        L0 = *(const f32x4*)&sm.lse[buf][4 * g];
        L1 = *(const f32x4*)&sm.lse[buf][16 + 4 * g];
        D0 = *(const f32x4*)&sm.dl[buf][4 * g];
        D1v = *(const f32x4*)&sm.dl[buf][16 + 4 * g];
      }
      constexpr int R2 = NP - 2 * (XNS - D1);   // products left for region 2
#pragma unroll
      for (int i = 0; i < R2; ++i) {
        if (HP) product(2 * (XNS - D1) + i);
        if (HC && i >= 2 && i < 10) {
          const int e = i - 2;
          const float lv = e < 4 ? L0[e & 3] : L1[e & 3];
          const float l2 = lv == -INFINITY ? INFINITY : lv * kLog2e;
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e >> 2][e & 3], scale_log2, -l2));
        }
        if (HC && i >= 10 && i < 18) {
          const int e = i - 10;
          const float dv = e < 4 ? D0[e & 3] : D1v[e & 3];
          dsv[e] = pv[e] * (pacc[e >> 2][e & 3] - dv) * scale;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (HC) {
        if (!(i0 >= full_a && i0 + YBQ - 1 <= full_c)) {   // (the branch touches P and dS only)
          const int tb = tb0 - i0;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const unsigned int tt = (unsigned int)(tb - (16 * (e >> 2) + (e & 3)));
            const bool ok = key_ok & (tt <= (unsigned int)span);
            pv[e] = ok ? pv[e] : 0.f;
            dsv[e] = ok ? dsv[e] : 0.f;
          }
        }
        // publish P and dS of tile u (read by every wave in the next step)
        const unsigned int pxw = px_base + buf * (2 * 4 * 64 * 16) + w * 64 * 16 + 16 * l;
        *(lds_u16x8*)(size_t)pxw = __builtin_bit_cast(u16x8, pack_halves(pv));
        *(lds_u16x8*)(size_t)(pxw + 4 * 64 * 16) = __builtin_bit_cast(u16x8, pack_halves(dsv));
      }
      if (HC && u + 1 < n_it) wait_vm(0);   // tile u + 1 complete before the next barrier
    };
    step(0, std::true_type{}, std::false_type{});
    for (int u = 1; u < n_it; ++u) step(u, std::true_type{}, std::true_type{});
    step(n_it, std::false_type{}, std::true_type{});
  }
  // dKV rows k0 + 16 kb + lane % 16, columns 128 w + 16 c + 4 g .. + 3
  // (a part without tiles has nothing to add to the zeroed output; a part
  // with a slot stores it, zeros included)
  const bool slot = slots != nullptr && part > 0;
  if (n_it == 0 && out_mode == kAtomicAddX && !slot) return;
  const int64_t dko = sv.k_off(p.dk_str, b) + hk * p.dk_str[1];
  float* dkp = slot ? slots + (part - 1) * slot_elems + dko : a.dk + dko;
  const int mode = slot ? kStoreX : out_mode;
  if (mode == kAddIntoX) {   // every load ahead of the adds (in flight together)
    f32x4 old[4 * NCW];
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2) {
      const int kk = k0 + 16 * kb2 + lr;
#pragma unroll
      for (int c = 0; c < NCW; ++c)
        old[4 * c + kb2] = kk < Sk ? *(const f32x4*)(dkp + (int64_t)kk * p.dk_str[2] + 128 * w + 16 * c + 4 * g)
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int x = 0; x < 4 * NCW; ++x) acc[x] = old[x] + acc[x];
  }
#pragma unroll
  for (int kb2 = 0; kb2 < 4; ++kb2) {
    const int kk = k0 + 16 * kb2 + lr;
    if (kk < Sk) {
#pragma unroll
      for (int c = 0; c < NCW; ++c) {
        float* d = dkp + (int64_t)kk * p.dk_str[2] + 128 * w + 16 * c + 4 * g;
        const f32x4 v = acc[4 * c + kb2];
        if (mode == kAtomicAddX) {
#pragma unroll
          for (int r = 0; r < 4; ++r) atomic_add_f32(d + r, v[r]);
        } else {
          *(f32x4*)d = v;
        }
      }
    }
  }
}

// dKV (+)= the slots of parts 1 .. nslot, in slot order: 128 threads per
// 512-float row, rows r of [tot_k, Hk] (packed) or [B, Hk, Sk] (dense).
__global__ __launch_bounds__(256) void k_slot_sum512(Params p, float* dk, const float* slots, int64_t slot_elems,
                                                     int nslot) {
  const bool pk = p.cu_k != nullptr;
  const int64_t rows = pk ? p.tot_k * p.Hk : (int64_t)p.B * p.Hk * p.Sk;
  const int c = threadIdx.x & 127;
  for (int64_t r = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7); r < rows; r += (int64_t)gridDim.x * 2) {
    int64_t off;
    if (pk) {
      off = (r / p.Hk) * p.dk_str[2] + (r % p.Hk) * p.dk_str[1];
    } else {
      const int64_t i = r % p.Sk, bh = r / p.Sk;
      off = (bh / p.Hk) * p.dk_str[0] + (bh % p.Hk) * p.dk_str[1] + i * p.dk_str[2];
    }
    float* d = dk + off + 4 * c;
    f32x4 v = *(const f32x4*)d;
    for (int q = 0; q < nslot; ++q) v += *(const f32x4*)(slots + q * slot_elems + off + 4 * c);
    *(f32x4*)d = v;
  }
}

}  // namespace

bool mla_supported(const Params& p) {
  if (p.Dqk != XD || p.Dv != XD) return false;
  for (int i = 0; i < 3; ++i) {
    if (p.q_str[i] % 8 || p.k_str[i] % 8 || p.do_str[i] % 8 || p.o_str[i] % 4 || p.dq_str[i] % 4 ||
        p.dk_str[i] % 4)
      return false;
  }
  // byte offsets of tiles and rows fit the 32-bit buffer addressing
  return 2 * p.k_str[2] * (int64_t)XBK < (int64_t(1) << 31) && 2 * p.q_str[2] * (int64_t)YBQ < (int64_t(1) << 31) &&
         2 * p.do_str[2] * (int64_t)YBQ < (int64_t(1) << 31);
}

hipError_t launch_fwd512(const Params& p, const FwdArgs& a0, bool o_bf16, hipStream_t st) {
  const dim3 grid((p.Sq + XBQ - 1) / XBQ, p.Hq, p.B);
  FwdArgs a = a0;
  a.xmajor = xmajor_fits(p, grid.y, grid.z);
  if (o_bf16)
    hipLaunchKernelGGL(k_fwd512<true>, grid, dim3(XNT), 0, st, p, a);
  else
    hipLaunchKernelGGL(k_fwd512<false>, grid, dim3(XNT), 0, st, p, a);
  return hipGetLastError();
}

// Parts per KV head's query group: split the group until the grid covers the
// chip (a part must divide the group).  Atomic parts: at most two when the
// result must be deterministic (one when adding into existing values);
// parts that keep partial sums are summed in a fixed order, at most 16.
static int dkv512_parts(const Params& p, bool deterministic, bool accumulate, bool partials) {
  const int nkb = (p.Sk + YBK - 1) / YBK;
  const int64_t units = (int64_t)nkb * p.Hk * p.B;
  const int max_parts = partials ? 16 : deterministic ? (accumulate ? 1 : 2) : 64;
  int parts = 1;
  while (units * parts < 256 && parts * 2 <= max_parts && p.G % (parts * 2) == 0) parts *= 2;
  return parts;
}

// Elements of the dKV tensor's extent (one slot of partial sums).
static int64_t dkv512_extent(const Params& p) {
  if (p.cu_k) return (p.tot_k - 1) * p.dk_str[2] + (p.Hk - 1) * p.dk_str[1] + p.Dqk;
  return (int64_t)(p.B - 1) * p.dk_str[0] + (p.Hk - 1) * p.dk_str[1] + (int64_t)(p.Sk - 1) * p.dk_str[2] + p.Dqk;
}

int64_t bwd512_workspace_bytes(const Params& p, bool deterministic, bool accumulate) {
  if (p.Sk <= 0 || p.B <= 0 || (p.cu_k && p.tot_k <= 0)) return 0;
  const int parts = dkv512_parts(p, deterministic, accumulate, true);
  const int atomic_parts = dkv512_parts(p, deterministic, accumulate, false);
  // partial sums when they split further or keep a fixed order where atomics could not
  if (parts < 2 || (parts <= 2 && atomic_parts == parts && !(deterministic && accumulate))) return 0;
  return (int64_t)(parts - 1) * dkv512_extent(p) * (int64_t)sizeof(float);
}

hipError_t launch_bwd512(const Params& p, const BwdArgs& a0, hipStream_t st) {
  BwdArgs a = a0;
  if (p.Sk > 0) {
    const bool det = a.deterministic != 0, acc = a.accumulate_dkdv != 0;
    const int64_t need = bwd512_workspace_bytes(p, det, acc);
    if (need > 0 && a.workspace != nullptr && ((uintptr_t)a.workspace & 15u) == 0 && a.workspace_bytes >= need) {
      // parts >= 1 store slots of partial sums that are then added in order
      const int parts = dkv512_parts(p, det, acc, true);
      const int64_t ext = dkv512_extent(p);
      float* slots = (float*)a.workspace;
      const dim3 grid((p.Sk + YBK - 1) / YBK, p.Hk * parts, p.B);
      hipLaunchKernelGGL(k_dkv512, grid, dim3(XNT), 0, st, p, a, parts, acc ? kAddIntoX : kStoreX, slots, ext);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_slot_sum512, dim3(1024), dim3(256), 0, st, p, a.dk, slots, ext, parts - 1);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else {
      const int parts = dkv512_parts(p, det, acc, false);
      int mode = kStoreX;
      if (parts > 1) {
        mode = kAtomicAddX;
        if (!acc) {
          ZeroRows z{a.dk, p.B, p.Hk, p.Sk, p.Dqk, {p.dk_str[0], p.dk_str[1], p.dk_str[2]}};
          if (p.cu_k) {   // packed: every row of the packed tensor
            z.B = 1;
            z.S = (int)p.tot_k;
            z.str[0] = 0;
          }
          hipError_t e = launch_zero_multi(&z, 1, st);
          if (e != hipSuccess) return e;
        }
      } else if (acc) {
        mode = kAddIntoX;
      }
      const dim3 grid((p.Sk + YBK - 1) / YBK, p.Hk * parts, p.B);
      hipLaunchKernelGGL(k_dkv512, grid, dim3(XNT), 0, st, p, a, parts, mode, (float*)nullptr, (int64_t)0);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (p.Sq > 0) {
    const dim3 grid((p.Sq + XBQ - 1) / XBQ, p.Hq, p.B);
    a.xmajor = xmajor_fits(p, grid.y, grid.z);
    hipLaunchKernelGGL(k_dq512, grid, dim3(XNT), 0, st, p, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace attn
