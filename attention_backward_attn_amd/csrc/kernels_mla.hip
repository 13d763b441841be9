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
      if (t + 1 < n_it) wait_vm(t + 2 < n_it ? 8 : 0);   // tile t + 1 complete before the next barrier
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
// dS = P (dP - delta) (scale folded in) for tile t.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(XNT, 1) void k_dq512(Params p, BwdArgs a) {
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

  f32x4 dq[XNC];
#pragma unroll
  for (int n = 0; n < XNC; ++n) dq[n] = zero4();
  bf16x8 Db = as_bf16x8(u16x8{0, 0, 0, 0, 0, 0, 0, 0});
  if (n_it > 0) {
    // One tile step: the S^T / dP^T chains of tile t (when HC) among the dQ^T
    // products of tile t - 1 (when HP, first half of the columns), then the
    // second half of those products among the exponentials and dS arithmetic
    // of tile t.  Operands are read two product steps ahead.  The first and
    // last steps are peeled, so the main loop has no branches.
    auto step = [&](int t, auto hc_, auto hp_) {
      constexpr bool HC = decltype(hc_)::value, HP = decltype(hp_)::value;
      // read-ahead: three steps of the chains; ten dQ product operands in
      // flight when the second region (one product per step) starts
      constexpr int AH = 3, BAH = 10, XTRA = BAH - AH;
      __syncthreads();   // tile t complete; tile t - 3's buffer free
      if (t + 2 < n_it) issue(t + 2);
      TileAddr cur, prv;
      if (HC) cur.set(sm_base + (t % XNB) * XTS, a_lane, t_lane);
      if (HP) prv.set(sm_base + ((t + XNB - 1) % XNB) * XTS, a_lane, t_lane);
      f32x4 sacc[2] = {zero4(), zero4()}, pacc[2] = {zero4(), zero4()};
      bf16x8 k0[XNS], k1[XNS], bt[XNC];
#pragma unroll
      for (int i = 0; i < AH; ++i) {
        if (HC) { k0[i] = cur.row(0, i); k1[i] = cur.row(1, i); }
        if (HP) bt[i] = prv.tr(i);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < XNS; ++s) {
        if (HC) {
          sacc[0] = mfma16(k0[s], qB[s], sacc[0]);
          pacc[0] = mfma16(k0[s], doB[s], pacc[0]);
        }
        if (HP) dq[s] = mfma16(bt[s], Db, dq[s]);
        if (HC) {
          sacc[1] = mfma16(k1[s], qB[s], sacc[1]);
          pacc[1] = mfma16(k1[s], doB[s], pacc[1]);
        }
        if (HC && s + AH < XNS) { k0[s + AH] = cur.row(0, s + AH); k1[s + AH] = cur.row(1, s + AH); }
        if (HP) bt[s + AH] = prv.tr(s + AH);
        if (HP && s >= XNS - XTRA) bt[XNS + AH + s - (XNS - XTRA)] = prv.tr(XNS + AH + s - (XNS - XTRA));
        __builtin_amdgcn_sched_barrier(0);
      }
      float pv[8], dsv[8];
#pragma unroll
      for (int i = 0; i < XNC - XNS; ++i) {
        const int nb = XNS + i;
        if (HP) dq[nb] = mfma16(bt[nb], Db, dq[nb]);
        if (HC) {
          if (i < 8) pv[i] = __builtin_amdgcn_exp2f(fmaf(sacc[i >> 2][i & 3], scale_log2, -lse2));
          else dsv[i - 8] = pv[i - 8] * fmaf(pacc[(i - 8) >> 2][(i - 8) & 3], scale, -dls);
        }
        if (HP && nb + BAH < XNC) bt[nb + BAH] = prv.tr(nb + BAH);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (HC) {
        const int j0 = kt.j0(t);
        if (!rm.full(j0)) {   // (the branch touches dS only)
#pragma unroll
          for (int e = 0; e < 8; ++e) dsv[e] = rm.ok(j0, g, e >> 2, e & 3) ? dsv[e] : 0.f;
        }
        Db = pack_halves(dsv);
      }
      if (t + 1 < n_it) wait_vm(t + 2 < n_it ? 8 : 0);   // tile t + 1 complete before the next barrier
    };
    step(0, std::true_type{}, std::false_type{});
    for (int t = 1; t < n_it; ++t) step(t, std::true_type{}, std::true_type{});
    step(n_it, std::false_type{}, std::true_type{});
  }
  if (irow < Sq) {
    float* dst = a.dq + sv.q_off(p.dq_str, b) + h * p.dq_str[1] + (int64_t)irow * p.dq_str[2];
#pragma unroll
    for (int n = 0; n < XNC; ++n) {
      f32x4* d4 = (f32x4*)(dst + 16 * n + 4 * g);
      *d4 = a.accumulate_dq ? *d4 + dq[n] : dq[n];
    }
  }
}

// ---------------------------------------------------------------------------
// k_dkv512: the dKV pass.  One workgroup of four waves per (64-key block,
// part of a KV head's query group, batch entry); wave w owns keys
// 16 w .. 16 w + 15 with their KV fragments and a 16 x 512 fp32 dKV^T
// accumulator (one key per lane) in registers.  The workgroup walks the
// part's (head, 32-row tile) iterations; Q and dO tiles come straight into
// two padded LDS buffers, one tile ahead.  Per tile: S = Q KV^T and
// dP = dO KV^T (one key per lane), P and dS, then
// dKV^T += dO^T P + Q^T (scale dS), whose reduction over the tile's rows
// uses the accumulators' slot order.  Several parts add into zeroed dKV.
// ---------------------------------------------------------------------------
struct __attribute__((aligned(1024))) SmemY {
  unsigned char q[2][YTS];
  unsigned char d[2][YTS];
  float lse[2][64];   // raw LSE / delta rows (a wave-wide load fills 64 entries)
  float dl[2][64];
};

enum : int { kStoreX = 0, kAddIntoX = 1, kAtomicAddX = 2 };

__global__ __launch_bounds__(XNT, 1) void k_dkv512(Params p, BwdArgs a, int parts, int out_mode) {
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
  auto tile_rows = [&](int it, int* hh, int* i0) {
    *hh = h_begin + it / nqb;
    *i0 = lo_al + YBQ * (it % nqb);
  };
  auto issue = [&](int it) {
    int hh, i0;
    tile_rows(it, &hh, &i0);
    const int rows = min(Sq - i0, YBQ);
    const int buf = it & 1;
    const unsigned short* qs = (const unsigned short*)a.q + sv.q_off(p.q_str, b) + hh * p.q_str[1] + (int64_t)i0 * p.q_str[2];
    const unsigned short* ds = (const unsigned short*)a.dout + sv.q_off(p.do_str, b) + hh * p.do_str[1] + (int64_t)i0 * p.do_str[2];
    stage_rows(qs, p.q_str[2], rows, sm_base + offsetof(SmemY, q) + buf * YTS, 8 * w, 8, l);
    stage_rows(ds, p.do_str[2], rows, sm_base + offsetof(SmemY, d) + buf * YTS, 8 * w, 8, l);
    if (w == 0) {
      // raw LSE and delta of the tile's rows (zeros past the end)
      const int64_t rb = ((int64_t)b * p.Hq + hh) * lrow + i0;
      const __amdgpu_buffer_rsrc_t rl = buf_rsrc(a.lse + rb, rows * 4), rd = buf_rsrc(a.delta + rb, rows * 4);
      // (lanes past the tile's rows read past the resource: zeros)
      lds_dma4(rl, __builtin_amdgcn_readfirstlane(sm_base + offsetof(SmemY, lse) + buf * 256), 4 * l);
      lds_dma4(rd, __builtin_amdgcn_readfirstlane(sm_base + offsetof(SmemY, dl) + buf * 256), 4 * l);
    }
  };
  f32x4 acc[XNC];
#pragma unroll
  for (int n = 0; n < XNC; ++n) acc[n] = zero4();
  if (n_it > 0) {
    issue(0);
    wait_vm(0);
    for (int t = 0; t < n_it; ++t) {
      __syncthreads();   // tile t complete; tile t - 1's buffer free
      if (t + 1 < n_it) issue(t + 1);
      const int buf = t & 1;
      int hh, i0;
      tile_rows(t, &hh, &i0);
      TileAddr tq, td;
      tq.set(sm_base + offsetof(SmemY, q) + buf * YTS, a_lane, t_lane);
      td.set(sm_base + offsetof(SmemY, d) + buf * YTS, a_lane, t_lane);
      // rows 16 h + 4 g + r of the tile: raw LSE and delta
      const f32x4 L0 = *(const f32x4*)&sm.lse[buf][4 * g], L1 = *(const f32x4*)&sm.lse[buf][16 + 4 * g];
      const f32x4 D0 = *(const f32x4*)&sm.dl[buf][4 * g], D1 = *(const f32x4*)&sm.dl[buf][16 + 4 * g];
      // S = Q KV^T and dP = dO KV^T: four chains, operands two steps ahead;
      // the products' first operands are read during the last steps
      constexpr int AH = 3, AHB = 2 * AH;
      f32x4 sacc[2] = {zero4(), zero4()}, pacc[2] = {zero4(), zero4()};
      bf16x8 xq0[XNS], xq1[XNS], xd0[XNS], xd1[XNS], bd[XNC], bq[XNC];
#pragma unroll
      for (int i = 0; i < AH; ++i) {
        xq0[i] = tq.row(0, i); xd0[i] = td.row(0, i); xq1[i] = tq.row(1, i); xd1[i] = td.row(1, i);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < XNS; ++s) {
        sacc[0] = mfma16(xq0[s], kB[s], sacc[0]);
        pacc[0] = mfma16(xd0[s], kB[s], pacc[0]);
        sacc[1] = mfma16(xq1[s], kB[s], sacc[1]);
        pacc[1] = mfma16(xd1[s], kB[s], pacc[1]);
        if (s + AH < XNS) {
          xq0[s + AH] = tq.row(0, s + AH); xd0[s + AH] = td.row(0, s + AH);
          xq1[s + AH] = tq.row(1, s + AH); xd1[s + AH] = td.row(1, s + AH);
        } else {
          const int n = s + AH - XNS;   // 0 .. AH - 1
          bd[n] = td.tr(n); bq[n] = tq.tr(n);
          if (AHB > AH) { bd[n + AH] = td.tr(n + AH); bq[n + AH] = tq.tr(n + AH); }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // P = exp2(S scale log2 e - LSE log2 e) (LSE -inf: a row without keys,
      // P = 0); dS = P (dP - delta) scale
      float pv[8], dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float lv = e < 4 ? L0[e & 3] : L1[e & 3];
        const float l2 = lv == -INFINITY ? INFINITY : lv * kLog2e;
        pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e >> 2][e & 3], scale_log2, -l2));
      }
      if (!(i0 >= full_a && i0 + YBQ - 1 <= full_c)) {
        const int tb = tb0 - i0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const unsigned int tt = (unsigned int)(tb - (16 * (e >> 2) + (e & 3)));
          pv[e] = (key_ok & (tt <= (unsigned int)span)) ? pv[e] : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dv = e < 4 ? D0[e & 3] : D1[e & 3];
        dsv[e] = pv[e] * (pacc[e >> 2][e & 3] - dv) * scale;
      }
      const bf16x8 Pb = pack_halves(pv), Sb = pack_halves(dsv);
      __builtin_amdgcn_sched_barrier(0);
      // dKV^T += dO^T P + Q^T (scale dS), operands four steps ahead
#pragma unroll
      for (int n = 0; n < XNC; ++n) {
        acc[n] = mfma16(bd[n], Pb, acc[n]);
        acc[n] = mfma16(bq[n], Sb, acc[n]);
        if (n + AHB < XNC) { bd[n + AHB] = td.tr(n + AHB); bq[n + AHB] = tq.tr(n + AHB); }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (t + 1 < n_it) wait_vm(0);
    }
  }
  if (key < Sk) {
    float* dst = a.dk + sv.k_off(p.dk_str, b) + hk * p.dk_str[1] + (int64_t)key * p.dk_str[2];
#pragma unroll
    for (int n = 0; n < XNC; ++n) {
      float* d = dst + 16 * n + 4 * g;
      if (out_mode == kAtomicAddX) {
#pragma unroll
        for (int r = 0; r < 4; ++r) atomic_add_f32(d + r, acc[n][r]);
      } else if (out_mode == kAddIntoX) {
        *(f32x4*)d = *(const f32x4*)d + acc[n];
      } else {
        *(f32x4*)d = acc[n];
      }
    }
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
// chip (a part must divide the group); at most two when the result must be
// deterministic.
static int dkv512_parts(const Params& p, bool deterministic, bool accumulate) {
  const int nkb = (p.Sk + YBK - 1) / YBK;
  const int64_t units = (int64_t)nkb * p.Hk * p.B;
  const int max_parts = deterministic ? (accumulate ? 1 : 2) : 64;
  int parts = 1;
  while (units * parts < 256 && parts * 2 <= max_parts && p.G % (parts * 2) == 0) parts *= 2;
  return parts;
}

hipError_t launch_bwd512(const Params& p, const BwdArgs& a0, hipStream_t st) {
  BwdArgs a = a0;
  if (p.Sk > 0) {
    const int parts = dkv512_parts(p, a.deterministic != 0, a.accumulate_dkdv != 0);
    int mode = kStoreX;
    if (parts > 1) {
      mode = kAtomicAddX;
      if (!a.accumulate_dkdv) {
        ZeroRows z{a.dk, p.B, p.Hk, p.Sk, p.Dqk, {p.dk_str[0], p.dk_str[1], p.dk_str[2]}};
        if (p.cu_k) {   // packed: every row of the packed tensor
          z.B = 1;
          z.S = (int)p.tot_k;
          z.str[0] = 0;
        }
        hipError_t e = launch_zero_multi(&z, 1, st);
        if (e != hipSuccess) return e;
      }
    } else if (a.accumulate_dkdv) {
      mode = kAddIntoX;
    }
    const dim3 grid((p.Sk + YBK - 1) / YBK, p.Hk * parts, p.B);
    hipLaunchKernelGGL(k_dkv512, grid, dim3(XNT), 0, st, p, a, parts, mode);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
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
