// bf16 matrix-core (gfx950 MFMA) attention backward.
//
// Math (CK FMHA example 34 "Backward Pass with GQA", cpu_bwd_gqa and its
// docstring; CANN sparse_flash_mla_grad "Formula" Phase 2 / 3; CK FMHA
// example 28 cpu_attention_bwd_dbias):
//   S = scale Q K^T (+ bias),  P = exp(S - LSE),  dP = dO V^T,
//   dS = P (dP - delta),  dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K,
//   dbias = sum_b dS.
//
// The backward runs as two passes, neither with atomic dQ updates:
//   * dK / dV by key blocks: one workgroup per (128-key block, KV head,
//     batch) loops over the G query heads of the group and the query tiles
//     that can see the block, keeping dK and dV for its keys in registers
//     (GQA group sums without atomics).  k_dkdv3 (head dim 128) and k_dkdv2
//     (head dim 64, also with a bias) split each 32-key slice between a pair
//     of waves on one SIMD (two waves per SIMD), on 64-row and 32-row query
//     tiles respectively; k_dkdv, one wave per 32 keys,
//     serves a bias at head dim 128 and walks the batch when dbias is asked,
//     so that dbias is summed in a fixed order.
//   * dQ by query blocks: k_dq2 (k_dq with a bias), one workgroup per
//     (128-row block, query head, batch), recomputes S and dP per key tile
//     and keeps dQ in registers.  k_dq2 may run first and also zero the
//     dK / dV that the split key-block parts add into.  With a bias and
//     dbias at head dim 64, k_dqb forms dQ and dbias together, walking the
//     batch inside the workgroup (dbias summed in a fixed order, written
//     once per group of entries).
// In the 32x32 kernels S (or S^T) comes out of v_mfma_f32_32x32x16_bf16 with
// one row or key per lane, and that accumulator layout is used directly as
// the operand of the next product once the reduction index is permuted the
// same way on both operands; the other operand is read from row-major LDS
// tiles, with the gfx950 transposing read ds_read_b64_tr_b16 where the tile
// row is the reduction index.  k_dqb does the same with
// v_mfma_f32_16x16x32_bf16.
//
// MFMA 32x32x16 bf16 operand layout (lane l, r = 0..15):
//   A[m][k]: lane holds m = l % 32, k = 8 (l / 32) + 0..7
//   B[k][n]: lane holds n = l % 32, k = 8 (l / 32) + 0..7
//   C[m][n]: lane holds n = l % 32, m = 8 (r / 4) + 4 (l / 32) + r % 4
#include <algorithm>
#include <type_traits>

#include "kernels.h"
#include "mfma_util.h"

namespace attn {
namespace {

using namespace mfma_util;

constexpr int BK = 128;       // keys per workgroup (k_dkdv)
#ifndef ATTN_MIN_WORKGROUPS
#define ATTN_MIN_WORKGROUPS 256
#endif
constexpr int64_t kMinWorkgroups = ATTN_MIN_WORKGROUPS;   // split target of the dK/dV grid
constexpr int BQ = 32;        // query rows per iteration (k_dkdv)
constexpr int NT = 256;       // threads per workgroup


template <int D>
struct SmemDKDV {
  unsigned short qr[2][BQ * Lay<D>::R];   // Q tile, row copy  (A of S = Q K^T)
  unsigned short dr[2][BQ * Lay<D>::R];   // dO tile, row copy (A of dP = dO V^T)
  unsigned short qt[2][BQ * Lay<D>::T];   // Q tile, tr copy   (B of dK += dS^T Q)
  unsigned short dt[2][BQ * Lay<D>::T];   // dO tile, tr copy  (B of dV += P^T dO)
  float lse2[2][BQ];                      // LSE * log2(e); +inf for rows without keys
  float dls[2][BQ];                       // delta * scale
};

// Per-thread staging of one 32-row Q / dO tile: the 2 x 32 x (D / 8)
// 16-byte chunks are dealt round-robin to the threads (16 consecutive lanes
// load one row's consecutive chunks); the last 32 threads carry the tile's
// LSE and delta.  load() only issues the global loads (rows clamped into
// range, so no branches and no use of the values) and store() writes both
// LDS copies.  Rows past the end hold a copy of the last row: finite, and
// their LSE of +inf makes every P (and dS) of the row zero.
template <int D>
struct Stage {
  static constexpr int NCR = D / 8;               // chunks per row
  static constexpr int NCH = 2 * BQ * NCR;        // chunks per Q + dO tile
  static constexpr int NR = NCH / NT;             // chunks per thread
  u16x8 v[NR];
  float lse, dl;

  __device__ inline void load(const unsigned short* q, const unsigned short* dout, int64_t qs, int64_t ds,
                              const float* lse_p, const float* dl_p, int i0, int Sq) {
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int idx = t + NT * k;
      const int tensor = idx / (BQ * NCR), rem = idx % (BQ * NCR);
      const int row = rem / NCR, c = rem % NCR;
      const int64_t i = min(i0 + row, Sq - 1);
      v[k] = *(const u16x8*)((tensor == 0 ? q + i * qs : dout + i * ds) + 8 * c);
    }
    if (t >= NT - BQ) {
      const int64_t i = min(i0 + (t - (NT - BQ)), Sq - 1);
      lse = lse_p[i];
      dl = dl_p[i];
    }
  }

  __device__ inline void store(SmemDKDV<D>& sm, int buf, int i0, int Sq, float scale) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int idx = t + NT * k;
      const int tensor = idx / (BQ * NCR), rem = idx % (BQ * NCR);
      const int row = rem / NCR, c = rem % NCR;
      *(u16x8*)((tensor == 0 ? sm.qr[buf] : sm.dr[buf]) + row * Lay<D>::R + 8 * c) = v[k];
      *(u16x8*)((tensor == 0 ? sm.qt[buf] : sm.dt[buf]) + row * Lay<D>::T + 8 * c) = v[k];
    }
    if (t >= NT - BQ) {
      const int r = t - (NT - BQ);
      const bool ok = i0 + r < Sq;
      sm.lse2[buf][r] = (!ok || lse == -INFINITY) ? INFINITY : lse * kLog2e;
      sm.dls[buf][r] = ok ? dl * scale : 0.f;
    }
  }
};

// How a dK/dV accumulator reaches global memory.
enum : int { kStore = 0, kAtomicAdd = 1, kAddInto = 2 };

// How the key blocks of a KV head are dealt to workgroups.
//
// A unit is one key block of one KV head; its work is the list of
// (query head of the group, 32-row query tile) iterations that can see it.
// Pairing: under a causal mask the number of query rows that see key block
// kb falls linearly with kb, so block kb and block nkb-1-kb together cost the
// same for every pair -- one pair per workgroup balances the grid.
// Splitting: a unit's iteration list may be cut into `nsplit` contiguous
// parts handled by separate workgroups.  With partials (k_dkdv3 / k_dkdv2
// without a bias on dense problems, more than two parts) part 0 writes dK/dV and the other parts
// their own slots, which the dQ pass adds in slot order afterwards
// (deterministic for any split); otherwise every part adds atomically into
// zeroed outputs (with exactly two addends onto zero the fp32 result does
// not depend on their order).
// Sink block: with sink tokens under a sliding window, key block 0 is seen by
// every query row while the others see only a band; it gets `nsplit0` parts,
// dealt first (logical block x < nsplit0).
struct DkdvGrid {
  int pair;      // complementary key blocks per workgroup
  int nsplit;    // parts per unit (logical block y = hk * nsplit + part)
  int nsplit0;   // parts of key block 0 (1 = no separate treatment)
  int out_mode;  // kStore / kAtomicAdd / kAddInto (part 0 with partials)
  Partials pt;   // slots of parts >= 1 (pt.base nullptr: none)
};

// Kernel k_dkdv (problems with a bias): four waves, wave w owns keys
// [32 w, 32 w + 32) of the block with K / V fragments and dK / dV
// accumulators in registers; per tile S and dP with the fragments as the B
// operand, the bias added to S, P and dS elementwise, then dV += P^T dO and
// dK += dS^T Q.  With dbias the workgroup walks the batch: the first entry
// stores dS, later ones add to it, so the sum over the batch has a fixed
// order.
template <int D, bool BIAS, bool BLOOP>
__global__ __launch_bounds__(NT, 1) void k_dkdv(Params p, BwdArgs a, DkdvGrid gd) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int NS = D / 16;          // k-steps over the head dim
  constexpr int NB = D / 32;          // 32-column blocks of the head dim
  constexpr int R = Lay<D>::R, T = Lay<D>::T;
  __shared__ __attribute__((aligned(16))) SmemDKDV<D> sm;

  const int tid = threadIdx.x, l = tid & 63, lr = l & 31, lg = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int Sq = p.Sq, Sk = p.Sk;
  const int nkb = (Sk + BK - 1) / BK;
  const BlockXYZ blk = xcd_block();
  const int hk = blk.y / gd.nsplit;
  int part = blk.y % gd.nsplit, nparts = gd.nsplit;
  int kbx = blk.x;
  if (gd.nsplit0 > 1) {
    if (kbx < gd.nsplit0) {
      part = kbx * gd.nsplit + part;
      nparts = gd.nsplit0 * gd.nsplit;
      kbx = 0;
    } else {
      kbx -= gd.nsplit0 - 1;
    }
  }
  const int h_begin = hk * p.G;
  const float scale = p.scale, scale_log2 = p.scale * kLog2e;
  const int n_units = (gd.pair && nkb - 1 - kbx != kbx) ? 2 : 1;
  const int out_mode = gd.out_mode;
  const bool no_mask = p.mask.kind == kMaskNone;
  // mask as t = j' - i' - diag:  allowed <=> lo_t <= t <= wr, or j' < n_sink
  const int lo_t = p.mask.wl < 0 ? -0x3fffffff : -p.mask.wl;
  const int wr_t = p.mask.wr;
  // per-lane LDS bases
  const int rowA = lr * R + 8 * lg;            // row-copy A operands: + 16 s
  const int trQ = tr_base(l, T);               // tr-copy B operands

  const int b_begin = BLOOP ? 0 : blk.z;
  const int b_end = BLOOP ? p.B : b_begin + 1;
  for (int b = b_begin; b < b_end; ++b) {
    for (int u = 0; u < n_units; ++u) {
      const int kb = u == 0 ? kbx : nkb - 1 - kbx;
      const int k0 = kb * BK;
      const int kw = k0 + 32 * w;     // first key of this wave
      const int jkey = kw + lr;       // this lane's key (accumulator column of S / dP)
      const bool wave_keys_in = kw + 32 <= Sk;
      const bool key_ok = jkey < Sk;
      const int jg = jkey + (int)p.mask.k_off;
      const bool sink_key = jg < p.mask.n_sink;
      int64_t lo64, hi64;
      p.mask.rows_for_keys(k0, min(k0 + BK, Sk), Sq, &lo64, &hi64);
      const int lo = (int)lo64, hi = (int)hi64;
      const int lo_al = lo & ~(BQ - 1);
      const int nqb = hi > lo ? (hi - lo_al + BQ - 1) / BQ : 0;
      // this part's slice [it_lo, it_hi) of the unit's G * nqb iterations
      const int n_all = p.G * nqb;
      const int it_lo = (int)((int64_t)n_all * part / nparts);
      const int n_it = (int)((int64_t)n_all * (part + 1) / nparts) - it_lo;

      const unsigned short* kp = (const unsigned short*)a.k + b * p.k_str[0] + hk * p.k_str[1];
      const unsigned short* vp = (const unsigned short*)a.v + b * p.v_str[0] + hk * p.v_str[1];
      // K / V fragments of this wave's keys (B operands of S and dP); keys
      // past the end read the last key (finite; their P is forced to 0).
      bf16x8 kB[NS], vB[NS];
      {
        const int64_t jc = min(jkey, Sk - 1);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          kB[s] = as_bf16x8(*(const u16x8*)(kp + jc * p.k_str[2] + 16 * s + 8 * lg));
          vB[s] = as_bf16x8(*(const u16x8*)(vp + jc * p.v_str[2] + 16 * s + 8 * lg));
        }
      }
      __syncthreads();  // readers of the previous unit's LDS tiles are done
      f32x16 dk[NB], dv[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) { dk[n] = zero16(); dv[n] = zero16(); }
      wait_vm_loads();

      Stage<D> stg;
      auto issue = [&](int h, int i0) {
        stg.load((const unsigned short*)a.q + b * p.q_str[0] + h * p.q_str[1],
                 (const unsigned short*)a.dout + b * p.do_str[0] + h * p.do_str[1], p.q_str[2], p.do_str[2],
                 a.lse + ((int64_t)b * p.Hq + h) * Sq, a.delta + ((int64_t)b * p.Hq + h) * Sq, i0, Sq);
      };
      // (head, row-tile) of the current iteration, advanced incrementally
      int h = h_begin + (nqb > 0 ? it_lo / nqb : 0), qb = nqb > 0 ? it_lo % nqb : 0;
      if (n_it > 0) {
        issue(h, lo_al + BQ * qb);
        stg.store(sm, 0, lo_al + BQ * qb, Sq, scale);
        __syncthreads();
      }

      for (int it = 0; it < n_it; ++it) {
        const int cur = it & 1;
        const int i0 = lo_al + BQ * qb;
        int hn = h, qbn = qb + 1;
        if (qbn == nqb) { qbn = 0; ++hn; }
        if (it + 1 < n_it) issue(hn, lo_al + BQ * qbn);
        // bias (and, past the first batch entry, the running dbias) of this
        // lane's 16 pairs: loads issued now, used after the products below
        float bpre[BIAS ? 16 : 1], dbpre[BIAS ? 16 : 1];
        if (BIAS) {
          const int64_t jc = min(jkey, Sk - 1);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t i = min(i0 + crow(r, lg), Sq - 1);
            bpre[r] = a.bias[h * p.bias_str[0] + i * p.bias_str[1] + jc];
          }
          if (BLOOP && a.dbias && b > b_begin) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int64_t i = min(i0 + crow(r, lg), Sq - 1);
              dbpre[r] = a.dbias[h * p.bias_str[0] + i * p.bias_str[1] + jc];
            }
          }
        }

        // S = Q K^T and dP = dO V^T for rows i0..i0+31, this wave's 32 keys.
        // The A operands are read from LDS in bulk ahead of the products, so
        // the read latency is paid once rather than once per product.
        f32x16 sacc = zero16(), dpacc = zero16();
        {
          bf16x8 qa[NS], da[NS];
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            qa[s] = lds_b128(sm.qr[cur], rowA + 16 * s);
            da[s] = lds_b128(sm.dr[cur], rowA + 16 * s);
          }
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            sacc = mfma(qa[s], kB[s], sacc);
            dpacc = mfma(da[s], vB[s], dpacc);
          }
        }
        // B operands of dV += P^T dO and dK += dS^T Q for the first two
        // head-dim blocks (independent of P): their reads overlap the
        // elementwise step below; the rest are read while those multiply.
        constexpr int NPF = NB < 2 ? NB : 2;
        bf16x8 oB[NB][2], qB[NB][2];
#pragma unroll
        for (int n = 0; n < NPF; ++n) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            oB[n][hf] = lds_trB(sm.dt[cur], trQ, 16 * hf, 32 * n, T);
            qB[n][hf] = lds_trB(sm.qt[cur], trQ, 16 * hf, 32 * n, T);
          }
        }
        // LSE (log2 units) and delta * scale of this lane's 16 rows: rows 8 m + 4 lg + 0..3
        f32x4 L4[4], D4[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          L4[m] = *(const f32x4*)&sm.lse2[cur][8 * m + 4 * lg];
          D4[m] = *(const f32x4*)&sm.dls[cur][8 * m + 4 * lg];
        }

        // P = exp(S - LSE) on allowed pairs; dS = P (dP - delta), carried
        // pre-multiplied by the softmax scale (the factor of dK and dQ).
        // Tiles that are entirely allowed (the bulk under causal masks) skip
        // the mask.
        const bool full = wave_keys_in && p.mask.tile_full(i0, i0 + BQ, kw, kw + 32);
        float pv[16], dsv[16];
        if (full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = fmaf(sacc[r], scale_log2, -L4[r >> 2][r & 3]);
            if (BIAS) x = fmaf(bpre[r], kLog2e, x);
            pv[r] = __builtin_amdgcn_exp2f(x);
            dsv[r] = pv[r] * fmaf(dpacc[r], scale, -D4[r >> 2][r & 3]);
          }
        } else {
          const int tb = jg - (i0 + (int)p.mask.q_off) - (int)p.mask.diag - 4 * lg;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 8 * (r >> 2) + (r & 3);
            const int t = tb - c;
            const bool ok = key_ok & (no_mask | ((t <= wr_t) & (t >= lo_t)) | sink_key);
            float x = fmaf(sacc[r], scale_log2, -L4[r >> 2][r & 3]);
            if (BIAS) x = fmaf(bpre[r], kLog2e, x);
            const float ex = __builtin_amdgcn_exp2f(x);
            pv[r] = ok ? ex : 0.f;
            dsv[r] = pv[r] * fmaf(dpacc[r], scale, -D4[r >> 2][r & 3]);
          }
        }
        if (BIAS && a.dbias) {
          // dbias takes the unscaled dS; with the batch loop the first entry
          // stores (rows and keys inside the problem) and later ones add
          const float inv_scale = 1.f / scale;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = i0 + crow(r, lg);
            if (i < Sq && key_ok) {
              float* dst = a.dbias + h * p.bias_str[0] + (int64_t)i * p.bias_str[1] + jkey;
              if (BLOOP)
                *dst = (b > b_begin ? dbpre[r] : 0.f) + dsv[r] * inv_scale;
              else if (pv[r] != 0.f)
                atomic_add_f32(dst, dsv[r] * inv_scale);
            }
          }
        }
        const bf16x8 pa0 = pack8(pv), pa1 = pack8(pv + 8);
        const bf16x8 sa0 = pack8(dsv), sa1 = pack8(dsv + 8);

        // dV += P^T dO and dK += dS^T Q (reduction over the 32 rows, permuted
        // consistently with the accumulator layout of S).
#pragma unroll
        for (int n = NPF; n < NB; ++n) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            oB[n][hf] = lds_trB(sm.dt[cur], trQ, 16 * hf, 32 * n, T);
            qB[n][hf] = lds_trB(sm.qt[cur], trQ, 16 * hf, 32 * n, T);
          }
        }
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          dv[n] = mfma(pa0, oB[n][0], dv[n]);
          dk[n] = mfma(sa0, qB[n][0], dk[n]);
          dv[n] = mfma(pa1, oB[n][1], dv[n]);
          dk[n] = mfma(sa1, qB[n][1], dk[n]);
        }

        if (it + 1 < n_it) stg.store(sm, cur ^ 1, lo_al + BQ * qbn, Sq, scale);
        __syncthreads();
        h = hn;
        qb = qbn;
      }

      // Epilogue: dK (scaled through dS) and dV for this wave's keys.
      float* dkp = a.dk + b * p.dk_str[0] + hk * p.dk_str[1];
      float* dvp = a.dv + b * p.dv_str[0] + hk * p.dv_str[1];
      if (out_mode == kAddInto) {
        add_loaded<NB>(dk, dkp, p.dk_str[2], kw, Sk, lg, lr);
        add_loaded<NB>(dv, dvp, p.dv_str[2], kw, Sk, lg, lr);
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t j = kw + crow(r, lg);
          if (j < Sk) {
            float* pk = dkp + j * p.dk_str[2] + 32 * n + lr;
            float* pvv = dvp + j * p.dv_str[2] + 32 * n + lr;
            if (out_mode == kAtomicAdd) {
              atomic_add_f32(pk, dk[n][r]);
              atomic_add_f32(pvv, dv[n][r]);
            } else {
              *pk = dk[n][r];
              *pvv = dv[n][r];
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel k_dkdv2: dK / dV without dQ (dQ from k_dq), two waves per SIMD.
// One workgroup of eight waves per unit.  Waves w and w + 4 form a pair on
// one SIMD that owns keys [32 (w % 4), 32 (w % 4) + 32) of the block: the
// "S" wave keeps the keys' K fragments, forms S = Q K^T and P and
// accumulates all of dV; the "dP" wave keeps V, forms dP = dO V^T and
// dS = P (dP - delta) and accumulates all of dK.  P (bf16, in the
// accumulator's own lane order) is the only value handed across, through
// LDS.  One barrier per 32-row query tile: before barrier t the S wave
// publishes P(t) and the dP wave has formed dP(t); after it the S wave adds
// P(t)^T dO(t) into dV and goes on to S(t + 1), while the dP wave forms
// dS(t), adds dS(t)^T Q(t) into dK and goes on to dP(t + 1) -- so each
// wave's exponentials or dS arithmetic run under its partner's products.
// Q / dO tiles are staged through three LDS buffers: the tile stored after
// barrier t is first read after barrier t + 1, and the buffer it replaces
// was last read before barrier t.
// ---------------------------------------------------------------------------
constexpr int NT2 = 512;
constexpr int NB2 = 5;   // Q / dO tile buffers

template <int D>
struct __attribute__((aligned(1024))) SmemDKDV2 {
  unsigned char q[NB2][BQ * 2 * D];   // Q tile, swizzled (A of S = Q K^T; tr B of dK += dS^T Q)
  unsigned char d[NB2][BQ * 2 * D];   // dO tile, swizzled (A of dP = dO V^T; tr B of dV += P^T dO)
  float lse[NB2][2 * BQ];             // LSE of the tile's rows (second half: padding)
  float dl[NB2][2 * BQ];              // delta of the tile's rows (second half: padding)
  f32x4 px[2][4][4][64];              // P (fp32) by tile parity, pair w % 4: [4 values][lane]
};

// With a bias (head dim 64): the bias tile [32 rows][128 keys] (fp32) of each
// buffer, after the members above (the S wave adds it to S).
template <int D>
struct __attribute__((aligned(1024))) SmemDKDV2B : SmemDKDV2<D> {
  float bias[NB2][BQ * BK];
};

// Staging of one 32-row Q / dO tile straight from global memory into LDS:
// wave w issues CR / 8 64-lane loads, each filling 1 KB (64 / CR rows) of
// one tensor's tile in the swizzled layout, so every lane has one fixed
// source offset per load; wave 0 also loads the tile's LSE and delta.  The
// buffer resources span the tile's rows inside the problem: rows past the
// end arrive as zeros.
template <int D>
struct StageDma {
  static constexpr int CR = D / 8;
  static constexpr int NI = CR / 8;   // Q / dO loads per wave per tile
  static_assert(NI >= 1 && (2 * BQ * CR) % (64 * NI) == 0, "loads per wave");
  int voff[NI];
  unsigned int dst0[NI];   // LDS byte offset of each load in buffer 0
  bool is_d;               // this wave loads dO (else Q)
  bool rows_too;           // wave 0: also the LSE / delta rows

  __device__ inline void init(int w, int l, int q_rb, int d_rb) {
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int gi = w * NI + k;   // load index over both tiles
      is_d = gi >= BQ * CR / 64;
      const int slot = gi % (BQ * CR / 64);
      const int row = (64 * slot + l) / CR;
      voff[k] = row * (is_d ? d_rb : q_rb) + 16 * ((l % CR) ^ Swz<D>::f(row));
      dst0[k] = (is_d ? offsetof(SmemDKDV2<D>, d) : offsetof(SmemDKDV2<D>, q)) + 1024 * slot;
    }
    rows_too = w == 0;
  }

  // q_t / d_t / l_t / dl_t: the tile's first row; rows: rows inside the problem
  // Wave 0 issues the two small row loads first, so that every wave can
  // wait for "at most NI loads in flight" to see a whole tile complete.
  __device__ inline void issue(unsigned int sm_base, int buf, const unsigned short* q_t, const unsigned short* d_t,
                               int q_rb, int d_rb, const float* l_t, const float* dl_t, int rows, int l) {
    if (rows_too) {
      lds_dma4(buf_rsrc(l_t, rows * 4),
               __builtin_amdgcn_readfirstlane(sm_base + offsetof(SmemDKDV2<D>, lse) + buf * (8 * BQ)), 4 * l);
      lds_dma4(buf_rsrc(dl_t, rows * 4),
               __builtin_amdgcn_readfirstlane(sm_base + offsetof(SmemDKDV2<D>, dl) + buf * (8 * BQ)), 4 * l);
    }
    const __amdgpu_buffer_rsrc_t rs = is_d ? buf_rsrc(d_t, rows * d_rb) : buf_rsrc(q_t, rows * q_rb);
#pragma unroll
    for (int k = 0; k < NI; ++k)
      lds_dma16(rs, __builtin_amdgcn_readfirstlane(sm_base + dst0[k] + buf * (BQ * 2 * D)), voff[k]);
  }
};

// Walk over the (query head, 32-row tile) sequence of one unit part, with
// running tile pointers: a step adds one tile's rows, a head change adds the
// head stride less the rows walked.
struct TileWalk {
  const unsigned short *q, *d;
  const float *l, *dl;
  const float* bz;   // bias of the tile's first row and the block's first key (with a bias)
  int qb, nqb, i0, lo_al;
  int64_t q_step, d_step, q_wrap, d_wrap, l_wrap, b_step, b_wrap;

  __device__ inline void next() {
    q += q_step;
    d += d_step;
    l += BQ;
    dl += BQ;
    bz += b_step;
    i0 += BQ;
    if (++qb == nqb) {
      qb = 0;
      i0 = lo_al;
      q += q_wrap;
      d += d_wrap;
      l += l_wrap;
      dl += l_wrap;
      bz += b_wrap;
    }
  }
};

// BIAS (head dim 64): S gets the elementwise bias [Hq, Sq, Sk] (shared over
// the batch), staged per tile into LDS next to Q / dO; the S wave adds it
// before the exponentials.  No dbias here (the dQ pass sums it).
template <int D, bool BIAS>
__global__ __launch_bounds__(NT2) void k_dkdv2(Params p, BwdArgs a, DkdvGrid gd) {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(!BIAS || D == 64, "the bias tiles fit LDS at head dim 64");
  constexpr int NS = D / 16;          // k-steps over the head dim
  constexpr int NC = D / 32;          // 32-column blocks of dK / dV
  constexpr int RB = Swz<D>::RB;
  constexpr int NIW = StageDma<D>::NI + (BIAS ? 2 : 0);   // loads per wave per tile
  constexpr int BIAS_OFF = (int)sizeof(SmemDKDV2<D>);      // byte offset of the bias tiles
  constexpr int BTS = BQ * BK * 4;                         // bias tile bytes
  __shared__ std::conditional_t<BIAS, SmemDKDV2B<D>, SmemDKDV2<D>> sm;

  const int tid = threadIdx.x, l = tid & 63, lr = l & 31, lg = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int pr = w & 3;               // pair: keys [32 pr, 32 pr + 32) of the block
  const bool sw = w < 4;              // S wave (else dP wave)
  // with a bias (shared over the batch) the batch entries of a unit run side
  // by side, so each bias tile comes from HBM about once
  const BlockXYZ blk = BIAS ? xcd_block_zfast() : xcd_block();
  // a packed batch takes its sequences by decreasing work (query rows x
  // keys, ties by index): each XCD walks its logical blocks with the key
  // blocks fastest, then the batch index, so the longest sequences' units
  // start first and the short ones fill the end (batch index z stands for
  // the sequence of rank z; the P exchange area, unused until the first
  // tile, holds the prefix sums meanwhile)
  int b = blk.z;
  if (p.cu_k != nullptr && p.B <= NT2) {
    int* cu = (int*)&sm.px;   // cu_q[0 .. B], cu_k[0 .. B], the answer
    for (int i = tid; i <= p.B; i += NT2) {
      cu[i] = p.cu_q[i];
      cu[p.B + 1 + i] = p.cu_k[i];
    }
    __syncthreads();
    if (tid < p.B) {
      auto work = [&](int s_) {
        const int lq = min(max(cu[s_ + 1] - cu[s_], 0), p.Sq);
        const int lk = min(max(cu[p.B + 2 + s_] - cu[p.B + 1 + s_], 0), p.Sk);
        return (int64_t)lq * lk;
      };
      const int64_t wt = work(tid);
      int rank = 0;
      for (int s_ = 0; s_ < p.B; ++s_) {
        const int64_t ws = work(s_);
        rank += (ws > wt) | ((ws == wt) & (s_ < tid));
      }
      if (rank == blk.z) cu[2 * p.B + 2] = tid;
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(cu[2 * p.B + 2]);
    __syncthreads();   // every wave has read it before the area is reused
  }
  const SeqView sv = seq_view(p, b);   // this batch entry (or packed sequence)
  const Mask& msk = sv.mask;
  const int Sq = sv.Sq, Sk = sv.Sk;
  const int nkb = (Sk + BK - 1) / BK;
  const int hk = blk.y / gd.nsplit;
  int part = blk.y % gd.nsplit, nparts = gd.nsplit;
  int kbx = blk.x;
  if (gd.nsplit0 > 1) {
    if (kbx < gd.nsplit0) {
      part = kbx * gd.nsplit + part;
      nparts = gd.nsplit0 * gd.nsplit;
      kbx = 0;
    } else {
      kbx -= gd.nsplit0 - 1;
    }
  }
  const int h_begin = hk * p.G;
  const float scale = p.scale, scale_log2 = p.scale * kLog2e;
  // key blocks of this sequence (a packed batch's grid covers the longest)
  const bool unit_in = gd.pair ? 2 * kbx < nkb : kbx < nkb;
  const int n_units = !unit_in ? 0 : ((gd.pair && nkb - 1 - kbx != kbx) ? 2 : 1);
  const int out_mode = gd.out_mode;
  const bool no_mask = msk.kind == kMaskNone;
  const int lo_t = msk.wl < 0 ? -0x3fffffff : -msk.wl;
  const int wr_t = msk.wr;
  const int a_lane = Swz<D>::a_lane(l), t_lane = Swz<D>::t_lane(l);
  const int q_rb = 2 * (int)p.q_str[2], d_rb = 2 * (int)p.do_str[2];
  StageDma<D> stg;
  stg.init(w, l, q_rb, d_rb);
  const unsigned int sm_base = lds_addr(&sm);

  for (int u = 0; u < n_units; ++u) {
    const int kb = u == 0 ? kbx : nkb - 1 - kbx;
    const int k0 = kb * BK;
    const int kw = k0 + 32 * pr;
    const int jkey = kw + lr;
    const bool key_ok = jkey < Sk;
    const int jg = jkey + (int)msk.k_off;
    const bool sink_key = jg < msk.n_sink;
    int64_t lo64, hi64;
    msk.rows_for_keys(k0, min(k0 + BK, Sk), Sq, &lo64, &hi64);
    const int lo = (int)lo64, hi = (int)hi64;
    const int lo_al = lo & ~(BQ - 1);
    const int nqb = hi > lo ? (hi - lo_al + BQ - 1) / BQ : 0;
    const int n_all = p.G * nqb;
    const int it_lo = (int)((int64_t)n_all * part / nparts);
    const int n_it = (int)((int64_t)n_all * (part + 1) / nparts) - it_lo;
    // tiles [i0, i0 + 32) in which every row sees all 32 keys of this wave:
    // i0 >= full_a and i0 + 31 <= full_c
    int full_a = -0x3fffffff, full_c = 0x3fffffff;
    if (kw + 32 > Sk) {
      full_a = 0x3fffffff;
    } else if (!no_mask && kw + 31 + msk.k_off >= msk.n_sink) {
      const int64_t base = (int64_t)kw + msk.k_off - msk.q_off - msk.diag;
      full_a = (int)max<int64_t>(min<int64_t>(base + 31 - msk.wr, 0x3fffffff), -0x3fffffff);
      if (msk.wl >= 0) full_c = (int)max<int64_t>(min<int64_t>(base + msk.wl, 0x3fffffff), -0x3fffffff);
    }

    // K (S wave) or V (dP wave) fragments of this pair's keys: B operands
    bf16x8 fB[NS];
    {
      const unsigned short* src = sw ? (const unsigned short*)a.k + sv.k_off(p.k_str, b) + hk * p.k_str[1]
                                     : (const unsigned short*)a.v + sv.k_off(p.v_str, b) + hk * p.v_str[1];
      const int64_t rs = sw ? p.k_str[2] : p.v_str[2];
      const int64_t jc = min(jkey, Sk - 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) fB[s] = as_bf16x8(*(const u16x8*)(src + jc * rs + 16 * s + 8 * lg));
    }
    // where this wave's dV (S wave) or dK (dP wave) rows go: dK / dV, or for
    // part >= 1 of a split unit with partials the part's slot (rows j - k0,
    // the dK columns then the dV ones)
    const bool slot = gd.pt.base != nullptr && part > 0;
    float* op;
    int64_t os, jr;
    if (slot) {
      const int rw = p.Dqk + p.Dv;
      op = gd.pt.base + (((int64_t)b * p.Hk + hk) * gd.pt.nslot + partial_slot(gd.pt, kb, part)) * BK * rw +
           (sw ? p.Dqk : 0);
      os = rw;
      jr = k0;
    } else {
      op = sw ? a.dv + sv.k_off(p.dv_str, b) + hk * p.dv_str[1] : a.dk + sv.k_off(p.dk_str, b) + hk * p.dk_str[1];
      os = sw ? p.dv_str[2] : p.dk_str[2];
      jr = 0;
    }
    const int mode = slot ? kStore : out_mode;
    __syncthreads();  // readers of the previous unit's LDS tiles are done
    if (n_it <= 0) {
      // no query row reaches this part: stored rows get zeros (rows that
      // are added into keep their values)
      if (mode == kStore) {
#pragma unroll
        for (int n = 0; n < NC; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t j = kw + crow(r, lg);
            if (j < Sk) op[(j - jr) * os + 32 * n + lr] = 0.f;
          }
      }
      continue;
    }

    // tile walks: `ld` runs ahead with the loads, `fr` is the tile whose
    // S / dP is formed next
    TileWalk ld;
    {
      const int h0 = h_begin + it_lo / nqb, qb0 = it_lo % nqb;
      const int i00 = lo_al + BQ * qb0;
      ld.q = (const unsigned short*)a.q + sv.q_off(p.q_str, b) + h0 * p.q_str[1] + (int64_t)i00 * p.q_str[2];
      ld.d = (const unsigned short*)a.dout + sv.q_off(p.do_str, b) + h0 * p.do_str[1] +
             (int64_t)i00 * p.do_str[2];
      const int64_t rb = ((int64_t)b * p.Hq + h0) * p.Sq + i00;
      ld.l = a.lse + rb;
      ld.dl = a.delta + rb;
      ld.qb = qb0;
      ld.nqb = nqb;
      ld.i0 = i00;
      ld.lo_al = lo_al;
      ld.q_step = BQ * p.q_str[2];
      ld.d_step = BQ * p.do_str[2];
      ld.q_wrap = p.q_str[1] - nqb * ld.q_step;
      ld.d_wrap = p.do_str[1] - nqb * ld.d_step;
      ld.l_wrap = (int64_t)p.Sq - (int64_t)nqb * BQ;
      ld.bz = BIAS ? a.bias + h0 * p.bias_str[0] + (int64_t)i00 * p.bias_str[1] + k0 : nullptr;
      ld.b_step = BIAS ? BQ * p.bias_str[1] : 0;
      ld.b_wrap = BIAS ? p.bias_str[0] - nqb * ld.b_step : 0;
    }
    int fr_i0 = ld.i0, fr_qb = ld.qb;   // tile whose P the S wave forms next
    auto fr_next = [&]() {
      fr_i0 += BQ;
      if (++fr_qb == nqb) { fr_qb = 0; fr_i0 = lo_al; }
    };
    // bias tile: wave w loads rows 4 w .. 4 w + 3 (two 1 KB loads of two rows each);
    // the resource ends at the tile's last valid element (rows past the end read zeros)
    const int b_rb = BIAS ? 4 * (int)p.bias_str[1] : 0, bkeys = min(Sk - k0, BK);
    auto issue = [&](int buf) {
      const int rows = min(Sq - ld.i0, BQ);
      stg.issue(sm_base, buf, ld.q, ld.d, q_rb, d_rb, ld.l, ld.dl, rows, l);
      if (BIAS) {
        const __amdgpu_buffer_rsrc_t rb_ = buf_rsrc(ld.bz, (rows - 1) * b_rb + 4 * bkeys);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int g = 2 * w + k;   // rows 2 g, 2 g + 1
          lds_dma16(rb_, __builtin_amdgcn_readfirstlane(sm_base + BIAS_OFF + buf * BTS + 1024 * g),
                    (2 * g + (l >> 5)) * b_rb + 16 * (l & 31));
        }
      }
      ld.next();
    };
    // Prologue: tiles 0..3 in flight together with the K / V fragments, all
    // complete before the first barrier.
    issue(0);
#pragma unroll
    for (int j = 1; j < NB2 - 1; ++j)
      if (n_it > j) issue(j);
    wait_vm_loads();
    __syncthreads();
    // Wave 0 turns the raw LSE / delta rows of a complete tile into
    // LSE * log2(e) (+inf for a row without keys) and delta * scale, in place.
    // Rows past the end hold zeros (P = 1 there, against zero Q / dO rows).
    auto prep_rows = [&](int buf) {
      if (w == 0) {
        float* x = (l < BQ ? sm.lse[buf] : sm.dl[buf]) + (l & (BQ - 1));
        const float v = *x;
        *x = l < BQ ? (v == -INFINITY ? INFINITY : v * kLog2e) : v * scale;
      }
    };
    prep_rows(0);
    if (n_it > 1) prep_rows(1);
    __syncthreads();

    // Per-lane key window of the masked exponentials: key lane jg is allowed
    // for row i when  jg - i - q_off - diag  lies in [lo_l, lo_l + span]
    // (all offsets for a sink key or no mask, none for a key past the end).
    int lo_l = lo_t, span = wr_t - lo_t;
    if (no_mask | sink_key) { lo_l = -0x3fffffff; span = 0x7ffffffe; }
    if (!key_ok) { lo_l = 0x3fffffff; span = 0; }
    const int tb0 = jg - (int)msk.q_off - (int)msk.diag - 4 * lg - lo_l;

    constexpr int TS = BQ * 2 * D;   // tile bytes
    // LSE * log2(e) or delta * scale of the rows this lane holds in the accumulator
    auto row_vals = [&](f32x4* x, const float* v) {
#pragma unroll
      for (int m = 0; m < 4; ++m) x[m] = *(const f32x4*)&v[8 * m + 4 * lg];
    };
    // bias (log2 units) of the 16 pairs this lane holds for the tile in
    // buffer j: rows crow(r, lg), key 32 pr + lane of the block
    const unsigned int b_lane = sm_base + BIAS_OFF + (4 * lg) * (BK * 4) + (32 * pr + lr) * 4;
    auto bias_vals = [&](float* bv, int j) {
      if (BIAS) {
        typedef __attribute__((address_space(3))) const float lds_f32;
        const unsigned int base = b_lane + j * BTS;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          bv[r] = *(lds_f32*)(size_t)(base + (8 * (r >> 2) + (r & 3)) * (BK * 4)) * kLog2e;
      }
    };
    // exponent (log2 units) of P = exp(S scale + bias - LSE)
    auto expo = [&](float s_, float l2, float b2) {
      const float x = fmaf(s_, scale_log2, -l2);
      return BIAS ? x + b2 : x;
    };
    constexpr int EPS = 16 / NS;   // accumulator elements handled per chain step
    constexpr int AHEAD = 2;       // chain steps whose operands are in flight

    // Each role runs its own copy of the loop, so that its accumulators never
    // cross a branch.  Per query tile t (one barrier):
    //   S wave:  dV += P(t)^T dO(t);  S(t + 2) = Q K^T;  P(t + 1) = exp2(S(t + 1) - LSE)
    //   dP wave: dS(t) = P(t) (dP(t) - delta);  dP(t + 1) = dO V^T;  dK += dS(t)^T Q(t)
    // The exponentials and dS arithmetic run between the products of the
    // same wave; P(t + 1) (fp32) is published before barrier t + 1.  The
    // loop is unrolled over the tile buffers, so every operand read is a
    // per-lane register plus a constant offset.
    auto run = [&](auto role) {
      constexpr bool SW = decltype(role)::value;
      f32x16 og[NC];   // dV (S wave) or dK (dP wave), columns 32 n + lane
#pragma unroll
      for (int n = 0; n < NC; ++n) og[n] = zero16();
      // operand read addresses in tile buffer 0
      const unsigned int a_t0 = sm_base + (SW ? offsetof(SmemDKDV2<D>, q) : offsetof(SmemDKDV2<D>, d));
      const unsigned int b_t0 = sm_base + (SW ? offsetof(SmemDKDV2<D>, d) : offsetof(SmemDKDV2<D>, q));
      unsigned int ar[NS], br[NC];
#pragma unroll
      for (int s = 0; s < NS; ++s) ar[s] = a_t0 + (a_lane ^ (32 * s));
#pragma unroll
      for (int n = 0; n < NC; ++n) br[n] = b_t0 + (t_lane ^ (64 * n));
      // A of chain step s, and B of dV / dK product i (accumulator i % NC,
      // tile rows 16 (i / NC) ...), in tile buffer j (a constant)
      auto read_a = [&](int j, int s) { return lds_b128_at(ar[s] + j * TS); };
      auto read_b = [&](int j, int i) {
        const int n = i % NC, r0 = 16 * (i / NC);
        // (tile buffers are 1 KB aligned: the XOR only touches address bits 5..7)
        return cat44(lds_tr4_at(br[n] + j * TS + r0 * RB), lds_tr4_at((br[n] ^ 32) + j * TS + (r0 + 8) * RB));
      };
      auto chain = [&](int j) {   // S or dP of the tile in buffer j, in one go
        bf16x8 xa[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) xa[s] = read_a(j, s);
        f32x16 c = zero16();
#pragma unroll
        for (int s = 0; s < NS; ++s) c = mfma(xa[s], fB[s], c);
        return c;
      };
      f32x16 acc = chain(0);   // S(0) / dP(0)
      bf16x8 pa0, pa1;         // S wave: P of the current tile
      float pv[16];
      // S wave: mask P of tile fr (in pv), keep it as operands, publish it
      auto publish = [&](int pbuf) {
        const int i0 = fr_i0;
        if (!(i0 >= full_a && i0 + BQ - 1 <= full_c)) {
          const int tb = tb0 - i0;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const unsigned int tt = (unsigned int)(tb - (8 * (r >> 2) + (r & 3)));
            pv[r] = tt <= (unsigned int)span ? pv[r] : 0.f;
          }
        }
        pa0 = pack8(pv);
        pa1 = pack8(pv + 8);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          sm.px[pbuf][pr][k][l] = f32x4{pv[4 * k], pv[4 * k + 1], pv[4 * k + 2], pv[4 * k + 3]};
      };
      if (SW) {
        f32x4 L4[4];
        row_vals(L4, sm.lse[0]);
        float bv[16];
        bias_vals(bv, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pv[r] = __builtin_amdgcn_exp2f(expo(acc[r], L4[r >> 2][r & 3], bv[r]));
        publish(0);
        fr_next();
        acc = chain(1);   // S(1) (stale when there is no tile 1; then unused)
      }

      // one tile: t the tile index, j = t % NB2 (a constant)
      // Operands of the next tile read before its barrier, from buffers that
      // are complete (and not rewritten) since an earlier one: B of its
      // dV / dK products and, for the dP wave, A of its dP chain.  Their
      // latency then overlaps the end of the current tile.
      bf16x8 bq_n[AHEAD], xa_n[AHEAD];
      auto prefetch = [&](auto jc) {   // jc: buffer of the next tile
        constexpr int j = decltype(jc)::value, j1 = (j + 1) % NB2;
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) bq_n[i] = read_b(j, i);
        if (!SW) {
#pragma unroll
          for (int i = 0; i < AHEAD; ++i) xa_n[i] = read_a(j1, i);
        }
      };
      prefetch(std::integral_constant<int, 0>{});
      auto tile = [&](int t, auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int j1 = (j + 1) % NB2, j2 = (j + 2) % NB2;
        __syncthreads();  // P(t) published; tile t + 2 complete, its rows prepared; tile t - 1's buffer free
        const bool more = t + NB2 - 1 < n_it;
        if (more) issue((j + NB2 - 1) % NB2);
        if (t + 2 < n_it) prep_rows(j2);   // complete since the barrier; first read after the next one
        bf16x8 bq[NS], xa[NS];
        f32x16 accn = zero16();
        if (SW) {
          // region: dV(t) products, S(t + 2) chain, exponentials of S(t + 1)
          f32x4 L4[4];
          row_vals(L4, sm.lse[j1]);
          float bv[16];
          bias_vals(bv, j1);
#pragma unroll
          for (int i = 0; i < AHEAD; ++i) { bq[i] = bq_n[i]; xa[i] = read_a(j2, i); }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            og[i % NC] = mfma(i < NC ? pa0 : pa1, bq[i], og[i % NC]);
            accn = mfma(xa[i], fB[i], accn);
#pragma unroll
            for (int e = 0; e < EPS; ++e) {
              const int r = EPS * i + e;
              pv[r] = __builtin_amdgcn_exp2f(expo(acc[r], L4[r >> 2][r & 3], bv[r]));
            }
            if (i + AHEAD < NS) { bq[i + AHEAD] = read_b(j, i + AHEAD); xa[i + AHEAD] = read_a(j2, i + AHEAD); }
            __builtin_amdgcn_sched_barrier(0);
          }
          // (unconditional, so the exponentials stay among the products; past
          // the last tile it writes an unread P buffer)
          publish((t + 1) & 1);
          fr_next();
        } else {
          // region: dS(t) arithmetic, dP(t + 1) chain, dK(t) products
          f32x4 D4[4], P4[4];
          row_vals(D4, sm.dl[j]);
#pragma unroll
          for (int k = 0; k < 4; ++k) P4[k] = sm.px[t & 1][pr][k][l];
#pragma unroll
          for (int i = 0; i < AHEAD; ++i) { bq[i] = bq_n[i]; xa[i] = xa_n[i]; }
          __builtin_amdgcn_sched_barrier(0);
          float dsv[16];
          bf16x8 A0, A1;
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            accn = mfma(xa[i], fB[i], accn);
            if (i >= NS / 2) og[(i - NS / 2) % NC] = mfma(A0, bq[i - NS / 2], og[(i - NS / 2) % NC]);
#pragma unroll
            for (int e = 0; e < EPS; ++e) {
              const int r = EPS * i + e;
              dsv[r] = P4[r >> 2][r & 3] * fmaf(acc[r], scale, -D4[r >> 2][r & 3]);
            }
            if (i == NS / 2 - 1) A0 = pack8(dsv);
            if (i + AHEAD < NS) { bq[i + AHEAD] = read_b(j, i + AHEAD); xa[i + AHEAD] = read_a(j1, i + AHEAD); }
            __builtin_amdgcn_sched_barrier(0);
          }
          A1 = pack8(dsv + 8);
#pragma unroll
          for (int i = NS / 2; i < NS; ++i) og[i % NC] = mfma(A1, bq[i], og[i % NC]);
        }
        acc = accn;
        prefetch(std::integral_constant<int, j1>{});   // (past the last tile: stale, unused)
        // tile t + 3 complete before the next barrier (tile t + 4 may stay in flight)
        wait_vm_keep<NIW>(more);
      };
      static_assert(NB2 == 5, "tile loop unrolled over five buffers");
      for (int t0 = 0; t0 < n_it; t0 += NB2) {
        tile(t0, std::integral_constant<int, 0>{});
        if (t0 + 1 >= n_it) break;
        tile(t0 + 1, std::integral_constant<int, 1>{});
        if (t0 + 2 >= n_it) break;
        tile(t0 + 2, std::integral_constant<int, 2>{});
        if (t0 + 3 >= n_it) break;
        tile(t0 + 3, std::integral_constant<int, 3>{});
        if (t0 + 4 >= n_it) break;
        tile(t0 + 4, std::integral_constant<int, 4>{});
      }

      // Epilogue: dV (S wave) or dK (dP wave, scaled through dS) of this pair's keys.
#pragma unroll
      for (int n = 0; n < NC; ++n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t j = kw + crow(r, lg);
          if (j < Sk) {
            float* po = op + (j - jr) * os + 32 * n + lr;
            if (mode == kAtomicAdd) atomic_add_f32(po, og[n][r]);
            else if (mode == kAddInto) *po += og[n][r];
            else *po = og[n][r];
          }
        }
      }
    };
    if (sw) run(std::true_type{});
    else run(std::false_type{});
  }
}

// ---------------------------------------------------------------------------
// Kernel k_dkdv3 (dK / dV on 64-row query tiles: head dim 128 without a
// bias, head dim 64 with one): the wave pairs of k_dkdv2 on 64-row tiles.
// Per tile each wave issues two independent S (or dP) chains over the head
// dim (8 products each at head dim 128) and the dV (or dK) products (16),
// twice what a 32-row tile gives it, so the barrier, the hand-over of P and
// the operand reads that follow the barrier are paid once per 64 rows, and
// no wave waits on a single dependent chain.
// LDS (130 KB at head dim 128): the Q and dO tiles in three swizzled
// buffers each, loaded two tiles ahead; the rows' LSE and delta in four
// buffers, loaded three tiles ahead and prepared in place (LSE * log2(e),
// delta * scale) by wave 0 two tiles before their use; P handed from the S
// wave to the dP wave as the bf16 operand registers the S wave itself
// multiplies with, in two buffers by tile parity.  With a bias (head dim 64,
// 146 KB) the [64 rows x 128 keys] fp32 bias tile of each Q / dO tile comes
// into LDS beside it (two buffers) and the S wave adds it to S before the
// exponentials.  Every wave issues its share of a tile's loads one 1 KB
// slot at a time among its first products.  Per tile t, one barrier:
//   S wave:  S(t + 1) = Q K^T as two chains (rows 0..31 and 32..63,
//            alternating), then dV += P(t)^T dO(t) with the exponentials,
//            masking and bf16 rounding of P(t + 1) = exp2(S - LSE) among
//            those products; P(t + 1) published before the next barrier.
//   dP wave: dP(t + 1) = dO V^T as two alternating chains, with
//            dS(t) = P(t) (dP(t) scale - delta scale) of rows 0..31 among
//            the first half; dK += dS(t)^T Q(t) for rows 0..31 among the
//            second half (with the dS of rows 32..63), then for rows 32..63.
// ---------------------------------------------------------------------------
constexpr int BQ4 = 64;   // query rows per tile (k_dkdv3)
constexpr int NB4 = 3;    // Q / dO tile buffers
constexpr int NL4 = 4;    // LSE / delta row buffers

template <int D>
struct __attribute__((aligned(1024))) SmemDKDV3 {
  unsigned char q[NB4][BQ4 * 2 * D];   // Q tile, swizzled (A of S = Q K^T; tr B of dK += dS^T Q)
  unsigned char d[NB4][BQ4 * 2 * D];   // dO tile, swizzled (A of dP = dO V^T; tr B of dV += P^T dO)
  u16x8 px[2][4][4][64];               // P as bf16 operands: [tile % 2][pair][operand][lane]
  float lse[NL4][BQ4];                 // LSE of the tile's rows, then LSE * log2(e) (+inf: no keys)
  float dl[NL4][BQ4];                  // delta of the tile's rows, then delta * scale
};

// With a bias: the bias tile [64 rows][128 keys] (fp32) of Q / dO tile t in
// buffer t % 2, after the members above.
template <int D>
struct __attribute__((aligned(1024))) SmemDKDV3B : SmemDKDV3<D> {
  float bias[2][BQ4 * BK];
};

// Walk over the (query head, 64-row tile) sequence of a unit part: Q / dO
// tile pointers, or LSE / delta row pointers, one tile at a time.
struct Walk64 {
  const void *x, *y, *z;   // Q, dO and bias (bytes), or LSE and delta (floats)
  int qb, i0;
  __device__ inline void next(int nqb, int lo_al, int64_t x_step, int64_t y_step, int64_t x_wrap, int64_t y_wrap,
                              int64_t z_step = 0, int64_t z_wrap = 0) {
    x = (const char*)x + x_step;
    y = (const char*)y + y_step;
    z = (const char*)z + z_step;
    i0 += BQ4;
    if (++qb == nqb) {
      qb = 0;
      i0 = lo_al;
      x = (const char*)x + x_wrap;
      y = (const char*)y + y_wrap;
      z = (const char*)z + z_wrap;
    }
  }
};

template <int D, bool BIAS>
__global__ __launch_bounds__(NT2) void k_dkdv3(Params p, BwdArgs a, DkdvGrid gd) {
  static_assert((D == 128 && !BIAS) || (D == 64 && BIAS), "head dim 128 without a bias, 64 with one");
  constexpr int NS = D / 16;                   // k-steps over the head dim
  constexpr int NC = D / 32;                   // 32-column blocks of dK / dV
  constexpr int NVT = 4 * NC;                  // dV (or dK) products per tile
  constexpr int RB = Swz<D>::RB, CR = Swz<D>::CR;
  constexpr int TS = BQ4 * RB;                 // tile bytes
  constexpr int SLW = BQ4 * CR / 64 / 8;       // 1 KB slots of each tile loaded per wave
  constexpr int HB = 32 * RB;                  // byte offset of rows 32..63
  constexpr int NDMA = 2 * SLW + (BIAS ? 4 : 0);   // 1 KB loads per wave per tile
  constexpr int BIAS_OFF = (int)sizeof(SmemDKDV3<D>);   // byte offset of the bias tiles
  constexpr int BTS = BQ4 * BK * 4;                      // bias tile bytes
  __shared__ std::conditional_t<BIAS, SmemDKDV3B<D>, SmemDKDV3<D>> sm;

  const int tid = threadIdx.x, l = tid & 63, lr = l & 31, lg = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int pr = w & 3;               // pair: keys [32 pr, 32 pr + 32) of the block
  const bool sw = w < 4;              // S wave (else dP wave)
  // with a bias (shared over the batch) the batch entries of a unit run side
  // by side, so each bias tile comes from HBM about once
  const BlockXYZ blk = BIAS ? xcd_block_zfast() : xcd_block();
  // packed batch: batch index z stands for the sequence of rank z by work
  // (query rows x keys, ties by index), longest first (as in k_dkdv2)
  int b = blk.z;
  if (p.cu_k != nullptr && p.B <= NT2) {
    int* cu = (int*)&sm.px;   // cu_q[0 .. B], cu_k[0 .. B], the answer
    for (int i = tid; i <= p.B; i += NT2) {
      cu[i] = p.cu_q[i];
      cu[p.B + 1 + i] = p.cu_k[i];
    }
    __syncthreads();
    if (tid < p.B) {
      auto work = [&](int s_) {
        const int lq = min(max(cu[s_ + 1] - cu[s_], 0), p.Sq);
        const int lk = min(max(cu[p.B + 2 + s_] - cu[p.B + 1 + s_], 0), p.Sk);
        return (int64_t)lq * lk;
      };
      const int64_t wt = work(tid);
      int rank = 0;
      for (int s_ = 0; s_ < p.B; ++s_) {
        const int64_t ws = work(s_);
        rank += (ws > wt) | ((ws == wt) & (s_ < tid));
      }
      if (rank == blk.z) cu[2 * p.B + 2] = tid;
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(cu[2 * p.B + 2]);
    __syncthreads();   // every wave has read it before the area is reused
  }
  const SeqView sv = seq_view(p, b);
  const Mask& msk = sv.mask;
  const int Sq = sv.Sq, Sk = sv.Sk;
  const int nkb = (Sk + BK - 1) / BK;
  const int hk = blk.y / gd.nsplit;
  int part = blk.y % gd.nsplit, nparts = gd.nsplit;
  int kbx = blk.x;
  if (gd.nsplit0 > 1) {
    if (kbx < gd.nsplit0) {
      part = kbx * gd.nsplit + part;
      nparts = gd.nsplit0 * gd.nsplit;
      kbx = 0;
    } else {
      kbx -= gd.nsplit0 - 1;
    }
  }
  const int h_begin = hk * p.G;
  const float scale = p.scale, scale_log2 = p.scale * kLog2e;
  const bool unit_in = gd.pair ? 2 * kbx < nkb : kbx < nkb;
  const int n_units = !unit_in ? 0 : ((gd.pair && nkb - 1 - kbx != kbx) ? 2 : 1);
  const int out_mode = gd.out_mode;
  const bool no_mask = msk.kind == kMaskNone;
  const int lo_t = msk.wl < 0 ? -0x3fffffff : -msk.wl;
  const int wr_t = msk.wr;
  const int a_lane = Swz<D>::a_lane(l), t_lane = Swz<D>::t_lane(l);
  const int q_rb = 2 * (int)p.q_str[2], d_rb = 2 * (int)p.do_str[2];
  const unsigned int sm_base = __builtin_amdgcn_readfirstlane(lds_addr(&sm));
  // staging: wave w fills the 1 KB slots SLW w .. SLW w + SLW - 1 (rows
  // 4 slot .. 4 slot + 3) of each Q and dO tile; one fixed source offset per
  // lane and slot, the chunk order swizzled
  int qv[SLW], dv_[SLW];
#pragma unroll
  for (int k = 0; k < SLW; ++k) {
    const int slot = SLW * w + k, row = (64 * slot + l) / CR, c = l % CR;
    qv[k] = row * q_rb + 16 * (c ^ Swz<D>::f(row));
    dv_[k] = row * d_rb + 16 * (c ^ Swz<D>::f(row));
  }

  for (int u = 0; u < n_units; ++u) {
    const int kb = u == 0 ? kbx : nkb - 1 - kbx;
    const int k0 = kb * BK;
    const int kw = k0 + 32 * pr;
    const int jkey = kw + lr;
    const bool key_ok = jkey < Sk;
    const int jg = jkey + (int)msk.k_off;
    const bool sink_key = jg < msk.n_sink;
    int64_t lo64, hi64;
    msk.rows_for_keys(k0, min(k0 + BK, Sk), Sq, &lo64, &hi64);
    const int lo = (int)lo64, hi = (int)hi64;
    const int lo_al = lo & ~(BQ4 - 1);
    const int nqb = hi > lo ? (hi - lo_al + BQ4 - 1) / BQ4 : 0;
    const int n_all = p.G * nqb;
    const int it_lo = (int)((int64_t)n_all * part / nparts);
    const int n_it = (int)((int64_t)n_all * (part + 1) / nparts) - it_lo;
    // 32-row halves [i, i + 32) in which every row sees all 32 keys of this
    // wave: i >= full_a and i + 31 <= full_c
    int full_a = -0x3fffffff, full_c = 0x3fffffff;
    if (kw + 32 > Sk) {
      full_a = 0x3fffffff;
    } else if (!no_mask && kw + 31 + msk.k_off >= msk.n_sink) {
      const int64_t base = (int64_t)kw + msk.k_off - msk.q_off - msk.diag;
      full_a = (int)max<int64_t>(min<int64_t>(base + 31 - msk.wr, 0x3fffffff), -0x3fffffff);
      if (msk.wl >= 0) full_c = (int)max<int64_t>(min<int64_t>(base + msk.wl, 0x3fffffff), -0x3fffffff);
    }

    // K (S wave) or V (dP wave) fragments of this pair's keys: B operands
    bf16x8 fB[NS];
    {
      const unsigned short* src = sw ? (const unsigned short*)a.k + sv.k_off(p.k_str, b) + hk * p.k_str[1]
                                     : (const unsigned short*)a.v + sv.k_off(p.v_str, b) + hk * p.v_str[1];
      const int64_t rs = sw ? p.k_str[2] : p.v_str[2];
      const int64_t jc = min(jkey, Sk - 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) fB[s] = as_bf16x8(*(const u16x8*)(src + jc * rs + 16 * s + 8 * lg));
    }
    // where this wave's dV (S wave) or dK (dP wave) rows go (as in k_dkdv2)
    const bool slot = gd.pt.base != nullptr && part > 0;
    float* op;
    int64_t os, jr;
    if (slot) {
      const int rw = p.Dqk + p.Dv;
      op = gd.pt.base + (((int64_t)b * p.Hk + hk) * gd.pt.nslot + partial_slot(gd.pt, kb, part)) * BK * rw +
           (sw ? p.Dqk : 0);
      os = rw;
      jr = k0;
    } else {
      op = sw ? a.dv + sv.k_off(p.dv_str, b) + hk * p.dv_str[1] : a.dk + sv.k_off(p.dk_str, b) + hk * p.dk_str[1];
      os = sw ? p.dv_str[2] : p.dk_str[2];
      jr = 0;
    }
    const int mode = slot ? kStore : out_mode;
    __syncthreads();  // readers of the previous unit's LDS tiles are done
    if (n_it <= 0) {
      if (mode == kStore) {
#pragma unroll
        for (int n = 0; n < NC; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t j = kw + crow(r, lg);
            if (j < Sk) op[(j - jr) * os + 32 * n + lr] = 0.f;
          }
      }
      continue;
    }

    // tile walks: `wqd` issues the Q / dO tiles (two ahead), `wl` the LSE /
    // delta rows (three ahead)
    Walk64 wqd, wl;
    const int64_t q_step = (int64_t)BQ4 * p.q_str[2] * 2, d_step = (int64_t)BQ4 * p.do_str[2] * 2;
    const int64_t q_wrap = p.q_str[1] * 2 - nqb * q_step, d_wrap = p.do_str[1] * 2 - nqb * d_step;
    const int64_t l_step = BQ4 * 4, l_wrap = ((int64_t)p.Sq - (int64_t)nqb * BQ4) * 4;
    // bias rows of a tile (bytes): the tile's first row, the block's first key
    const int64_t z_step = BIAS ? (int64_t)BQ4 * p.bias_str[1] * 4 : 0;
    const int64_t z_wrap = BIAS ? (p.bias_str[0] - (int64_t)nqb * BQ4 * p.bias_str[1]) * 4 : 0;
    const int b_rb = BIAS ? 4 * (int)p.bias_str[1] : 0, bkeys = min(Sk - k0, BK);
    {
      const int h0 = h_begin + it_lo / nqb, qb0 = it_lo % nqb;
      const int i00 = lo_al + BQ4 * qb0;
      wqd.x = (const unsigned short*)a.q + sv.q_off(p.q_str, b) + h0 * p.q_str[1] + (int64_t)i00 * p.q_str[2];
      wqd.y = (const unsigned short*)a.dout + sv.q_off(p.do_str, b) + h0 * p.do_str[1] + (int64_t)i00 * p.do_str[2];
      const int64_t rb = ((int64_t)b * p.Hq + h0) * p.Sq + i00;
      wl.x = a.lse + rb;
      wl.y = a.delta + rb;
      wqd.z = BIAS ? a.bias + h0 * p.bias_str[0] + (int64_t)i00 * p.bias_str[1] + k0 : nullptr;
      wl.z = nullptr;
      wqd.qb = wl.qb = qb0;
      wqd.i0 = wl.i0 = i00;
    }
    int fr_i0 = wqd.i0, fr_qb = wqd.qb;   // first row of the tile whose P the S wave forms next
    auto fr_next = [&]() {
      fr_i0 += BQ4;
      if (++fr_qb == nqb) { fr_qb = 0; fr_i0 = lo_al; }
    };
    // bias tile slot g (1 KB: rows 2 g, 2 g + 1) of wave w: g = 4 w + k
    auto bias_dma = [&](__amdgpu_buffer_rsrc_t rz, int bbuf, int k) {
      const int g = 4 * w + k;
      lds_dma16(rz, sm_base + BIAS_OFF + bbuf * BTS + 1024 * g, (2 * g + (l >> 5)) * b_rb + 16 * (l & 31));
    };
    auto issue_qd = [&](int buf, int bbuf) {
      const int rows = min(Sq - wqd.i0, BQ4);
      const __amdgpu_buffer_rsrc_t rq = buf_rsrc(wqd.x, rows * q_rb), rd = buf_rsrc(wqd.y, rows * d_rb);
      const unsigned int mq = sm_base + offsetof(SmemDKDV3<D>, q) + buf * TS + 1024 * SLW * w;
      const unsigned int md = sm_base + offsetof(SmemDKDV3<D>, d) + buf * TS + 1024 * SLW * w;
#pragma unroll
      for (int k = 0; k < SLW; ++k) lds_dma16(rq, mq + 1024 * k, qv[k]);
#pragma unroll
      for (int k = 0; k < SLW; ++k) lds_dma16(rd, md + 1024 * k, dv_[k]);
      if (BIAS) {
        // (the resource ends at the tile's last valid element: rows past the end read zeros)
        const __amdgpu_buffer_rsrc_t rz = buf_rsrc(wqd.z, (rows - 1) * b_rb + 4 * bkeys);
#pragma unroll
        for (int k = 0; k < 4; ++k) bias_dma(rz, bbuf, k);
      }
      wqd.next(nqb, lo_al, q_step, d_step, q_wrap, d_wrap, z_step, z_wrap);
    };
    auto issue_l = [&](int lb) {
      if (w == 0) {
        const int rows = min(Sq - wl.i0, BQ4);
        lds_dma4(buf_rsrc(wl.x, rows * 4), sm_base + offsetof(SmemDKDV3<D>, lse) + lb * (4 * BQ4), 4 * l);
        lds_dma4(buf_rsrc(wl.y, rows * 4), sm_base + offsetof(SmemDKDV3<D>, dl) + lb * (4 * BQ4), 4 * l);
      }
      wl.next(nqb, lo_al, l_step, l_step, l_wrap, l_wrap);
    };
    // wave 0 turns the raw rows of a complete buffer into LSE * log2(e)
    // (+inf for a row without keys) and delta * scale; rows past the end
    // hold zeros (P = 1 there, against zero Q / dO rows)
    auto prep = [&](int lb) {
      if (w == 0) {
        const float x = sm.lse[lb][l], y = sm.dl[lb][l];
        sm.lse[lb][l] = x == -INFINITY ? INFINITY : x * kLog2e;
        sm.dl[lb][l] = y * scale;
      }
    };
    // Prologue: Q / dO tiles 0, 1 and LSE / delta rows 0..2 in flight
    // together with the K / V fragments, all complete before the barrier.
    issue_qd(0, 0);
    if (n_it > 1) issue_qd(1, 1);
    issue_l(0);
    if (n_it > 1) issue_l(1);
    if (n_it > 2) issue_l(2);
    wait_vm_loads();
    __syncthreads();
    prep(0);
    if (n_it > 1) prep(1);
    __syncthreads();

    // Per-lane key window of the masked exponentials (as in k_dkdv2).
    int lo_l = lo_t, span = wr_t - lo_t;
    if (no_mask | sink_key) { lo_l = -0x3fffffff; span = 0x7ffffffe; }
    if (!key_ok) { lo_l = 0x3fffffff; span = 0; }
    const int tb0 = jg - (int)msk.q_off - (int)msk.diag - 4 * lg - lo_l;

    // The loads of Q / dO tile t + 2 (into the buffer of tile t - 1), set up
    // at barrier t and issued one 1 KB slot at a time among the wave's first
    // products: issued together right after the barrier, the eight waves'
    // loads queue for the vector memory unit and hold up every wave's
    // products behind them.  Past the last tile they load nothing (zeros).
    struct DmaSet {
      __amdgpu_buffer_rsrc_t rq, rd, rz;
      unsigned int mq, md;
      int bbuf;
    };
    auto dma_set = [&](int t, int buf) {
      DmaSet d;
      const bool on = t + 2 < n_it;
      const int rows = on ? min(Sq - wqd.i0, BQ4) : 0;
      d.rq = buf_rsrc(wqd.x, rows * q_rb);
      d.rd = buf_rsrc(wqd.y, rows * d_rb);
      d.rz = buf_rsrc(wqd.z, on && BIAS ? (rows - 1) * b_rb + 4 * bkeys : 0);
      d.mq = sm_base + offsetof(SmemDKDV3<D>, q) + buf * TS + 1024 * SLW * w;
      d.md = sm_base + offsetof(SmemDKDV3<D>, d) + buf * TS + 1024 * SLW * w;
      d.bbuf = t & 1;   // tile t + 2's bias buffer
      if (on) wqd.next(nqb, lo_al, q_step, d_step, q_wrap, d_wrap, z_step, z_wrap);
      return d;
    };
    // k < SLW: Q slot k; k < 2 SLW: dO slot k - SLW; then the bias slots
    auto dma_one = [&](const DmaSet& d, int k) {
      if (k < SLW) lds_dma16(d.rq, d.mq + 1024 * k, qv[k]);
      else if (k < 2 * SLW) lds_dma16(d.rd, d.md + 1024 * (k - SLW), dv_[k - SLW]);
      else if (BIAS) bias_dma(d.rz, d.bbuf, k - 2 * SLW);
    };
    // one tile's common start: barrier t, the loads of the rows of tile
    // t + 3, the rows of tile t + 2 prepared
    auto tile_head = [&](int t) {
      __syncthreads();  // P(t) published; tile t + 1 and rows t + 2 complete; tile t - 1's buffers free
      if (t + 3 < n_it) issue_l((t + 3) & 3);
      if (t + 2 < n_it) prep((t + 2) & 3);
    };

    if (sw) {
      // ------------------------------------------------------------------ S wave
      f32x16 og[NC];   // dV, columns 32 n + lane
#pragma unroll
      for (int n = 0; n < NC; ++n) og[n] = zero16();
      unsigned int ar[NS], br[NC];
#pragma unroll
      for (int s = 0; s < NS; ++s) ar[s] = sm_base + offsetof(SmemDKDV3<D>, q) + (a_lane ^ (32 * s));
#pragma unroll
      for (int n = 0; n < NC; ++n) br[n] = sm_base + offsetof(SmemDKDV3<D>, d) + (t_lane ^ (64 * n));
      // chain step c of S: rows 32 (c % 2) .., k-step c / 2
      auto read_a = [&](int j, int c) { return lds_b128_at(ar[c >> 1] + j * TS + (c & 1) * HB); };
      // dV product i: accumulator i % NC, tile rows 16 (i / NC) .. (reduction slots)
      auto read_v = [&](int j, int i) {
        const int n = i % NC, r0 = 16 * (i / NC);
        return cat44(lds_tr4_at(br[n] + j * TS + r0 * RB), lds_tr4_at((br[n] ^ 32) + j * TS + (r0 + 8) * RB));
      };
      // exponent, mask and bf16 rounding of half h of S (rows 32 h ..) of the
      // tile whose first row is i0, with the prepared LSE rows lrow
      auto lse_vals = [&](f32x4* L4, const float* lrow, int h) {
#pragma unroll
        for (int m = 0; m < 4; ++m) L4[m] = *(const f32x4*)&lrow[32 * h + 8 * m + 4 * lg];
      };
      // bias of the four-element group g (rows 32 (g / 4) + 8 (g % 4) + 4 lg
      // + 0..3, this lane's key) of the tile in bias buffer bbuf
      typedef __attribute__((address_space(3))) const float lds_f32;
      const unsigned int b_lane = sm_base + BIAS_OFF + (4 * lg) * (BK * 4) + (32 * pr + lr) * 4;
      auto bias4 = [&](int g, int bbuf) {
        f32x4 v{0.f, 0.f, 0.f, 0.f};
        if (BIAS) {
          const unsigned int base = b_lane + bbuf * BTS + (32 * (g >> 2) + 8 * (g & 3)) * (BK * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = *(lds_f32*)(size_t)(base + e * (BK * 4));
        }
        return v;
      };
      // exponent (log2 units) of P = exp(S scale + bias - LSE)
      auto expo = [&](float s_, float l2, float bz) {
        const float x = fmaf(s_, scale_log2, -l2);
        return BIAS ? fmaf(bz, kLog2e, x) : x;
      };
      auto mask_pack = [&](float* pv, int i0h, bf16x8* dst2) {
        if (!(i0h >= full_a && i0h + 31 <= full_c)) {
          const int tb = tb0 - i0h;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const unsigned int tt = (unsigned int)(tb - (8 * (r >> 2) + (r & 3)));
            pv[r] = tt <= (unsigned int)span ? pv[r] : 0.f;
          }
        }
        dst2[0] = pack8(pv);
        dst2[1] = pack8(pv + 8);
      };
      auto publish = [&](const bf16x8* pn, int par) {
#pragma unroll
        for (int k = 0; k < 4; ++k) sm.px[par][pr][k][l] = __builtin_bit_cast(u16x8, pn[k]);
      };
      bf16x8 pa[4];   // P(t) as dV operands: rows 16 k .. 16 k + 15 in slot order
      {
        // P(0): both chains on Q tile 0, then the exponentials
        f32x16 s0 = zero16(), s1 = zero16();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          s0 = mfma(read_a(0, 2 * s), fB[s], s0);
          s1 = mfma(read_a(0, 2 * s + 1), fB[s], s1);
        }
        f32x4 L4[4], B4[4];
        float pv[16];
        lse_vals(L4, sm.lse[0], 0);
#pragma unroll
        for (int m = 0; m < 4; ++m) B4[m] = bias4(m, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = __builtin_amdgcn_exp2f(expo(s0[r], L4[r >> 2][r & 3], B4[r >> 2][r & 3]));
        mask_pack(pv, fr_i0, pa);
        lse_vals(L4, sm.lse[0], 1);
#pragma unroll
        for (int m = 0; m < 4; ++m) B4[m] = bias4(4 + m, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = __builtin_amdgcn_exp2f(expo(s1[r], L4[r >> 2][r & 3], B4[r >> 2][r & 3]));
        mask_pack(pv, fr_i0 + 32, pa + 2);
        publish(pa, 0);
        fr_next();
      }
      constexpr int VPRE = 2;   // dV operands read before the barrier
      bf16x8 vn[VPRE];
#pragma unroll
      for (int i = 0; i < VPRE; ++i) vn[i] = read_v(0, i);
      constexpr int AH = 2;     // operand reads in flight ahead of their product
      auto tile = [&](int t, auto jc) {
        constexpr int j = decltype(jc)::value, j1 = (j + 1) % NB4;
        tile_head(t);
        const DmaSet dma = dma_set(t, (j + 2) % NB4);
        const float* lrow = sm.lse[(t + 1) & 3];
        f32x16 s0 = zero16(), s1 = zero16();
        bf16x8 xa[2 * NS], bv[NVT];
#pragma unroll
        for (int i = 0; i < VPRE; ++i) bv[i] = vn[i];
#pragma unroll
        for (int c = 0; c < AH; ++c) xa[c] = read_a(j1, c);
        __builtin_amdgcn_sched_barrier(0);
        // dV products 0, 1 (operands already here) cover the first reads
#pragma unroll
        for (int i = 0; i < VPRE; ++i) og[i % NC] = mfma(pa[i / NC], bv[i], og[i % NC]);
#pragma unroll
        for (int i = VPRE; i < VPRE + AH; ++i) bv[i] = read_v(j, i);
        __builtin_amdgcn_sched_barrier(0);
        // the two S chains, alternating
#pragma unroll
        for (int c = 0; c < 2 * NS; ++c) {
          if (c & 1) s1 = mfma(xa[c], fB[c >> 1], s1);
          else s0 = mfma(xa[c], fB[c >> 1], s0);
          if (c + AH < 2 * NS) xa[c + AH] = read_a(j1, c + AH);
          if constexpr (NS == 8) {
            if (c % 3 == 0 && c / 3 < NDMA) dma_one(dma, c / 3);
          } else {
#pragma unroll
            for (int q_ = (c * NDMA) / (2 * NS); q_ < ((c + 1) * NDMA) / (2 * NS); ++q_) dma_one(dma, q_);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // the remaining dV products, among the exponentials of both halves
        // (element r: half r / 16, its LSE in the four-row group r / 4,
        // read one product ahead of the group's first exponential)
        float pv[32];
        constexpr int NV = NVT - VPRE;         // products in this region
        auto r_lo = [](int k) { return (32 * k + NV - 1) / NV; };   // first element of product k
        auto lse4 = [&](int g) {   // rows of four-element group g
          return *(const f32x4*)&lrow[32 * (g >> 2) + 8 * (g & 3) + 4 * lg];
        };
        const int bbuf = (t + 1) & 1;   // bias of tile t + 1
        f32x4 L4[8], B4[8];
#pragma unroll
        for (int g = 0; g < 8; ++g)   // the groups that product 0 starts
          if (4 * g < r_lo(1)) {
            L4[g] = lse4(g);
            B4[g] = bias4(g, bbuf);
          }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          const int i = VPRE + k;
          og[i % NC] = mfma(pa[i / NC], bv[i], og[i % NC]);
#pragma unroll
          for (int r = r_lo(k); r < r_lo(k + 1); ++r) {
            const float sv_ = r < 16 ? s0[r] : s1[r - 16];
            pv[r] = __builtin_amdgcn_exp2f(expo(sv_, L4[r >> 2][r & 3], B4[r >> 2][r & 3]));
            // (kept here: otherwise the compiler sinks them below the products)
            asm volatile("" : "+v"(pv[r]));
          }
#pragma unroll
          for (int g = 1; g < 8; ++g)
            if (4 * g >= r_lo(k + 1) && 4 * g < r_lo(k + 2)) {
              L4[g] = lse4(g);
              B4[g] = bias4(g, bbuf);
            }
          if (i + AH < NVT) bv[i + AH] = read_v(j, i + AH);
          __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 pn[4];
        mask_pack(pv, fr_i0, pn);
        mask_pack(pv + 16, fr_i0 + 32, pn + 2);
        // (unconditional: past the last tile it writes an unread buffer)
        publish(pn, (t + 1) & 1);
        fr_next();
#pragma unroll
        for (int k = 0; k < 4; ++k) pa[k] = pn[k];
        // dV operands of tile t + 1 (complete since barrier t)
#pragma unroll
        for (int i = 0; i < VPRE; ++i) vn[i] = read_v(j1, i);
        wait_vm_loads();   // this wave's loads of tile t + 2 done before the next barrier
      };
      for (int t0 = 0; t0 < n_it; t0 += NB4) {
        tile(t0, std::integral_constant<int, 0>{});
        if (t0 + 1 >= n_it) break;
        tile(t0 + 1, std::integral_constant<int, 1>{});
        if (t0 + 2 >= n_it) break;
        tile(t0 + 2, std::integral_constant<int, 2>{});
      }
#pragma unroll
      for (int n = 0; n < NC; ++n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t j = kw + crow(r, lg);
          if (j < Sk) {
            float* po = op + (j - jr) * os + 32 * n + lr;
            if (mode == kAtomicAdd) atomic_add_f32(po, og[n][r]);
            else if (mode == kAddInto) *po += og[n][r];
            else *po = og[n][r];
          }
        }
      }
    } else {
      // ----------------------------------------------------------------- dP wave
      f32x16 og[NC];   // dK, columns 32 n + lane (scaled through dS)
#pragma unroll
      for (int n = 0; n < NC; ++n) og[n] = zero16();
      unsigned int ar[NS], br[NC];
#pragma unroll
      for (int s = 0; s < NS; ++s) ar[s] = sm_base + offsetof(SmemDKDV3<D>, d) + (a_lane ^ (32 * s));
#pragma unroll
      for (int n = 0; n < NC; ++n) br[n] = sm_base + offsetof(SmemDKDV3<D>, q) + (t_lane ^ (64 * n));
      auto read_a = [&](int j, int c) { return lds_b128_at(ar[c >> 1] + j * TS + (c & 1) * HB); };
      auto read_k = [&](int j, int i) {
        const int n = i % NC, r0 = 16 * (i / NC);
        return cat44(lds_tr4_at(br[n] + j * TS + r0 * RB), lds_tr4_at((br[n] ^ 32) + j * TS + (r0 + 8) * RB));
      };
      // dP(0): both chains on dO tile 0
      f32x16 p0 = zero16(), p1 = zero16();
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        p0 = mfma(read_a(0, 2 * s), fB[s], p0);
        p1 = mfma(read_a(0, 2 * s + 1), fB[s], p1);
      }
      constexpr int AH = 2;
      // dS of one half: P (bf16 operands k0, k0 + 1 of the published P) times
      // dP scale - delta scale, rounded to the bf16 operands of dK
      auto ds_half = [&](const u32x4* pw, const f32x16& acc, const f32x4* D4, int r, float* dsv) {
        const unsigned int wd = pw[r >> 3][(r & 7) >> 1];
        const float pval = __uint_as_float((r & 1) ? (wd & 0xffff0000u) : (wd << 16));
        dsv[r] = pval * fmaf(acc[r], scale, -D4[r >> 2][r & 3]);
      };
      auto tile = [&](int t, auto jc) {
        constexpr int j = decltype(jc)::value, j1 = (j + 1) % NB4;
        tile_head(t);
        const DmaSet dma = dma_set(t, (j + 2) % NB4);
        const int par = t & 1;
        const float* drow = sm.dl[t & 3];
        // P(t) as bf16 pairs and the delta rows; at head dim 128 those of
        // rows 32..63 (and part of rows 0..31) are read during the products
        constexpr bool LATE = NS == 8;
        u32x4 pw[4];
        f32x4 Da[4], Db[4];
#pragma unroll
        for (int k = 0; k < (LATE ? 2 : 4); ++k) pw[k] = __builtin_bit_cast(u32x4, sm.px[par][pr][k][l]);
#pragma unroll
        for (int m = 0; m < (LATE ? 2 : 4); ++m) Da[m] = *(const f32x4*)&drow[8 * m + 4 * lg];
        if (!LATE) {
#pragma unroll
          for (int m = 0; m < 4; ++m) Db[m] = *(const f32x4*)&drow[32 + 8 * m + 4 * lg];
        }
        f32x16 n0 = zero16(), n1 = zero16();
        bf16x8 xa[2 * NS], bk[NVT];
#pragma unroll
        for (int c = 0; c < AH; ++c) xa[c] = read_a(j1, c);
        __builtin_amdgcn_sched_barrier(0);
        float dsv[32];
        bf16x8 ds[4];
        // chain steps 0..7 among the dS of rows 0..31
        constexpr int EP = 2;   // dS elements per product
#pragma unroll
        for (int c = 0; c < NS; ++c) {
          if (c & 1) n1 = mfma(xa[c], fB[c >> 1], n1);
          else n0 = mfma(xa[c], fB[c >> 1], n0);
          if (c >= 2) {   // (P arrives after the first products)
            // elements of step c: 3 a step at head dim 128, else spread evenly
            constexpr int ES = LATE ? EP + 1 : (16 + NS - 3) / (NS - 2);
#pragma unroll
            for (int e = 0; e < ES; ++e) {
              const int r = ES * (c - 2) + e;
              if (r < 16) ds_half(pw, p0, Da, r, dsv);
            }
          }
          if (LATE && c == 2) {
#pragma unroll
            for (int m = 2; m < 4; ++m) Da[m] = *(const f32x4*)&drow[8 * m + 4 * lg];
          }
          if (LATE && c == 5) {
#pragma unroll
            for (int k = 2; k < 4; ++k) pw[k] = __builtin_bit_cast(u32x4, sm.px[par][pr][k][l]);
#pragma unroll
            for (int m = 0; m < 2; ++m) Db[m] = *(const f32x4*)&drow[32 + 8 * m + 4 * lg];
          }
          if (c + AH < 2 * NS) xa[c + AH] = read_a(j1, c + AH);
          if (c >= NS - AH) bk[c - (NS - AH)] = read_k(j, c - (NS - AH));
          if constexpr (LATE) {
            if ((c & 1) == 0 && c / 2 < NDMA) dma_one(dma, c / 2);
          } else {
#pragma unroll
            for (int q_ = (c * NDMA) / NS; q_ < ((c + 1) * NDMA) / NS; ++q_) dma_one(dma, q_);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        ds[0] = pack8(dsv);
        ds[1] = pack8(dsv + 8);
        // chain steps 8..15 among the dK products of rows 0..31 and the dS of rows 32..63
#pragma unroll
        for (int c = NS; c < 2 * NS; ++c) {
          const int i = c - NS;   // dK product 0..7
          og[i % NC] = mfma(ds[i / NC], bk[i], og[i % NC]);
          if (c & 1) n1 = mfma(xa[c], fB[c >> 1], n1);
          else n0 = mfma(xa[c], fB[c >> 1], n0);
          constexpr int EB = 16 / NS;   // dS elements of rows 32..63 per step
#pragma unroll
          for (int e = 0; e < EB; ++e) {
            const int r = EB * i + e;
            const unsigned int wd = pw[2 + (r >> 3)][(r & 7) >> 1];
            const float pval = __uint_as_float((r & 1) ? (wd & 0xffff0000u) : (wd << 16));
            dsv[16 + r] = pval * fmaf(p1[r], scale, -Db[r >> 2][r & 3]);
          }
          if (LATE && i == 1) {
#pragma unroll
            for (int m = 2; m < 4; ++m) Db[m] = *(const f32x4*)&drow[32 + 8 * m + 4 * lg];
          }
          if (c + AH < 2 * NS) xa[c + AH] = read_a(j1, c + AH);
          if (i + AH < NVT) bk[i + AH] = read_k(j, i + AH);
          __builtin_amdgcn_sched_barrier(0);
        }
        ds[2] = pack8(dsv + 16);
        ds[3] = pack8(dsv + 24);
        // dK products of rows 32..63
#pragma unroll
        for (int i = NS; i < NVT; ++i) {
          og[i % NC] = mfma(ds[i / NC], bk[i], og[i % NC]);
          if (i + AH < NVT) bk[i + AH] = read_k(j, i + AH);
          __builtin_amdgcn_sched_barrier(0);
        }
        p0 = n0;
        p1 = n1;
        wait_vm_loads();
      };
      for (int t0 = 0; t0 < n_it; t0 += NB4) {
        tile(t0, std::integral_constant<int, 0>{});
        if (t0 + 1 >= n_it) break;
        tile(t0 + 1, std::integral_constant<int, 1>{});
        if (t0 + 2 >= n_it) break;
        tile(t0 + 2, std::integral_constant<int, 2>{});
      }
#pragma unroll
      for (int n = 0; n < NC; ++n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t j = kw + crow(r, lg);
          if (j < Sk) {
            float* po = op + (j - jr) * os + 32 * n + lr;
            if (mode == kAtomicAdd) atomic_add_f32(po, og[n][r]);
            else if (mode == kAddInto) *po += og[n][r];
            else *po = og[n][r];
          }
        }
      }
    }
  }
}

// Grid shape of k_dkdv for a problem (host side).
struct DkdvPlan {
  DkdvGrid g;
  dim3 grid;
};

// partials: split parts write slots that the dQ pass adds (no bias, dense
// problems); otherwise they add atomically.
DkdvPlan plan_dkdv(const Params& p, bool bloop, bool accumulate_dkdv, bool deterministic, bool partials) {
  DkdvPlan pl{};
  const int nkb = (p.Sk + BK - 1) / BK;
  const Mask& m = p.mask;
  // causal-like masks (no lower window bound): work per key block decreases
  // monotonically, so complementary blocks pair up evenly
  pl.g.pair = (m.kind != kMaskNone && m.wl < 0 && nkb > 1) ? 1 : 0;
  const int xblocks = pl.g.pair ? (nkb + 1) / 2 : nkb;
  const int64_t units = (int64_t)xblocks * p.Hk * (bloop ? 1 : p.B);
  // Atomic partial dK/dV go onto zeroed outputs: never with the batch loop
  // (its dbias is ordered), and only two-way when the result must be
  // deterministic -- two partials into existing values would not be.  Slot
  // partials are summed in a fixed order, so any split is deterministic.
  const bool can_split = !bloop && (partials || !(accumulate_dkdv && deterministic));
  const int max_parts = (deterministic && !partials) ? 2 : 16;
  // Split until the grid covers the chip once (one workgroup per CU at one
  // wave per SIMD), keeping at least a few iterations per part; more parts
  // cost more dK/dV atomics than they gain in balance.
  int64_t lo, hi;
  m.rows_for_keys(0, std::min(BK, p.Sk), p.Sq, &lo, &hi);
  const int64_t iters = (int64_t)p.G * ((hi - lo + BQ - 1) / BQ + 1);   // about one unit's, paired or not
  int ns = 1;
  if (can_split)
    while (ns < max_parts && units * ns < kMinWorkgroups && iters >= 8 * 2 * ns) ns *= 2;
  pl.g.nsplit = ns;
  // the sink key block under a sliding window sees every row
  const bool sink_block = m.kind != kMaskNone && m.wl >= 0 && m.n_sink > m.k_off && nkb > 1;
  pl.g.nsplit0 = 1;
  if (can_split && sink_block) {
    int64_t lo1, hi1;
    m.rows_for_keys(BK, std::min(2 * BK, p.Sk), p.Sq, &lo1, &hi1);
    const int64_t ratio = (hi1 > lo1) ? (hi - lo + (hi1 - lo1) - 1) / (hi1 - lo1) : 1;
    int ns0 = 1;
    while (ns0 * pl.g.nsplit < max_parts && ns0 < ratio) ns0 *= 2;
    pl.g.nsplit0 = ns0;
  }
  const int nparts_max = pl.g.nsplit * pl.g.nsplit0;
  pl.g.out_mode = (nparts_max > 1 && !partials) ? kAtomicAdd : (accumulate_dkdv ? kAddInto : kStore);
  // slots per (batch entry, KV head) when parts write partials (base set by the launcher)
  pl.g.pt = Partials{nullptr, 0, nparts_max, pl.g.nsplit};
  if (partials && nparts_max > 1) pl.g.pt.nslot = (nparts_max - 1) + (nkb - 1) * (pl.g.nsplit - 1);
  pl.grid = dim3(xblocks + pl.g.nsplit0 - 1, p.Hk * pl.g.nsplit, bloop ? 1 : p.B);
  return pl;
}

template <int D, bool BIAS, bool BLOOP>
hipError_t launch_dkdv(const Params& p, const BwdArgs& a, const DkdvPlan& pl, hipStream_t st) {
  hipLaunchKernelGGL((k_dkdv<D, BIAS, BLOOP>), pl.grid, dim3(NT), 0, st, p, a, pl.g);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_dkdv(const Params& p, const BwdArgs& a, const DkdvPlan& pl, bool bias, bool bloop,
                         hipStream_t st) {
  if (!bias) {
    if constexpr (D == 128)
      hipLaunchKernelGGL((k_dkdv3<128, false>), pl.grid, dim3(NT2), 0, st, p, a, pl.g);
    else
      hipLaunchKernelGGL((k_dkdv2<D, false>), pl.grid, dim3(NT2), 0, st, p, a, pl.g);
    return hipGetLastError();
  }
  if constexpr (D == 64) {   // with a bias, head dim 64 always takes k_dkdv3 (dbias comes from k_dqb)
    hipLaunchKernelGGL((k_dkdv3<64, true>), pl.grid, dim3(NT2), 0, st, p, a, pl.g);
    return hipGetLastError();
  } else {
    return bloop ? launch_dkdv<D, true, true>(p, a, pl, st) : launch_dkdv<D, true, false>(p, a, pl, st);
  }
}

// ---------------------------------------------------------------------------
// Kernel k_dq (dQ): one workgroup per (128-row query block,
// query head, batch).  Wave w owns rows [32 w, 32 w + 32) and keeps Q and dO
// as B-operand fragments in registers; per 32-key tile it forms
// S^T = K Q^T and dP^T = V dO^T (keys on accumulator rows, one query row per
// lane), so dS^T's accumulator layout is directly the A operand of
// dQ = dS K with K^T from a transposed LDS copy.  dQ accumulates in registers
// over every key tile the block can see -- no atomics.
// ---------------------------------------------------------------------------
constexpr int BQ3 = 128;   // query rows per workgroup (k_dq)
constexpr int BK3 = 32;    // keys per iteration (k_dq)

constexpr int BSTR = BK3 + 4;   // bias tile row stride (floats): 16 lanes reading 16 rows hit distinct banks

template <int D, bool BIAS>
struct SmemDQ {
  unsigned short kr[2][BK3 * Lay<D>::R];   // K tile, row copy (A of S^T = K Q^T)
  unsigned short vr[2][BK3 * Lay<D>::R];   // V tile, row copy (A of dP^T = V dO^T)
  unsigned short kt[2][BK3 * Lay<D>::T];   // K tile, tr copy  (B of dQ += dS K)
  float bias[BIAS ? 2 : 1][BIAS ? BQ3 * BSTR : 1];   // bias[h][i0 + r][j0 + c], row-major padded
};

// Staging of one 32-key K / V tile and, with a bias, of the [128 rows x 32
// keys] fp32 bias tile (8 lanes per row, 16 bytes each: coalesced along the
// keys).  Fixed per-thread 16-byte slots fetched with buffer loads whose
// resource ends at the tile's last valid element: keys (and bias rows) past
// the end read as zero and are masked to P = 0.
template <int D, bool BIAS>
struct StageKV {
  static constexpr int NCR = D / 8;
  static constexpr int NCH = 2 * BK3 * NCR;
  static constexpr int NR = NCH / NT;
  static constexpr int NBI = BIAS ? BQ3 * BK3 / 4 / NT : 0;   // float4 bias chunks per thread
  static_assert((BK3 * NCR) % NT == 0, "one tensor per chunk slot");
  u16x8 v[NR];
  f32x4 bv[BIAS ? NBI : 1];
  int voff[NR], lrow[NR], ltr[NR];
  int boff[BIAS ? NBI : 1], bl[BIAS ? NBI : 1];

  static constexpr bool is_v(int m) { return (NT * m) / (BK3 * NCR) != 0; }

  __device__ inline void init(int k_rb, int v_rb, int b_rb) {
    const int t = threadIdx.x;
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int rem = (t + NT * m) % (BK3 * NCR);
      const int row = rem / NCR, c = rem % NCR;
      voff[m] = row * (is_v(m) ? v_rb : k_rb) + 16 * c;
      lrow[m] = row * Lay<D>::R + 8 * c;
      ltr[m] = row * Lay<D>::T + 8 * c;
    }
    if (BIAS) {
#pragma unroll
      for (int m = 0; m < NBI; ++m) {
        const int idx = t + NT * m;
        const int row = idx / (BK3 / 4), c4 = idx % (BK3 / 4);
        boff[m] = row * b_rb + 16 * c4;
        bl[m] = row * BSTR + 4 * c4;
      }
    }
  }

  // k_t / v_t: first key of the tile; keys = keys inside the problem;
  // b_t: bias of (first row, first key), b_bytes: bytes up to its last valid element
  __device__ inline void load(const unsigned short* k_t, const unsigned short* v_t, int k_rb, int v_rb, int keys,
                              const float* b_t, int b_bytes) {
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(k_t, keys * k_rb);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(v_t, keys * v_rb);
#pragma unroll
    for (int m = 0; m < NR; ++m) v[m] = buf_load16(is_v(m) ? rv : rk, voff[m]);
    if (BIAS) {
      const __amdgpu_buffer_rsrc_t rb = buf_rsrc(b_t, b_bytes);
#pragma unroll
      for (int m = 0; m < NBI; ++m)
        bv[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, boff[m], 0, 0));
    }
  }

  __device__ inline void store(SmemDQ<D, BIAS>& sm, int buf) const {
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      if (is_v(m)) {
        *(u16x8*)(sm.vr[buf] + lrow[m]) = v[m];
      } else {
        *(u16x8*)(sm.kr[buf] + lrow[m]) = v[m];
        *(u16x8*)(sm.kt[buf] + ltr[m]) = v[m];
      }
    }
    if (BIAS) {
#pragma unroll
      for (int m = 0; m < NBI; ++m) *(f32x4*)&sm.bias[buf][bl[m]] = bv[m];
    }
  }
};

template <int D, bool BIAS>
__global__ __launch_bounds__(NT, 2) void k_dq(Params p, BwdArgs a) {
  constexpr int NS = D / 16;
  constexpr int NB = D / 32;
  constexpr int R = Lay<D>::R, T = Lay<D>::T;
  __shared__ __attribute__((aligned(16))) SmemDQ<D, BIAS> sm;

  const int tid = threadIdx.x, l = tid & 63, lr = l & 31, lg = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const BlockXYZ blk = a.xmajor ? xcd_block_xmajor() : xcd_block();
  // under a causal mask later row blocks see more keys: deal them first
  const bool heavy_last = p.mask.kind != kMaskNone && p.mask.wl < 0;
  const int i0 = (heavy_last ? (int)gridDim.x - 1 - blk.x : blk.x) * BQ3;
  const int h = blk.y, b = blk.z, g = h / p.G;
  const SeqView sv = seq_view(p, b);   // this batch entry (or packed sequence)
  const Mask& msk = sv.mask;
  const int Sq = sv.Sq, Sk = sv.Sk;
  if (i0 >= Sq) return;   // past this sequence's rows (uniform across the workgroup)
  const int irow = i0 + 32 * w + lr;           // this lane's query row
  const float scale = p.scale, scale_log2 = p.scale * kLog2e;
  const int rowA = lr * R + 8 * lg;
  const int trK = tr_base(l, T);

  const unsigned short* q = (const unsigned short*)a.q + sv.q_off(p.q_str, b) + h * p.q_str[1];
  const unsigned short* dout = (const unsigned short*)a.dout + sv.q_off(p.do_str, b) + h * p.do_str[1];
  const unsigned short* kp = (const unsigned short*)a.k + sv.k_off(p.k_str, b) + g * p.k_str[1];
  const unsigned short* vp = (const unsigned short*)a.v + sv.k_off(p.v_str, b) + g * p.v_str[1];

  bf16x8 qB[NS], doB[NS];
  {
    const int64_t ic = min(irow, Sq - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qB[s] = as_bf16x8(*(const u16x8*)(q + ic * p.q_str[2] + 16 * s + 8 * lg));
      doB[s] = as_bf16x8(*(const u16x8*)(dout + ic * p.do_str[2] + 16 * s + 8 * lg));
    }
  }
  float lse2 = INFINITY, dls = 0.f;
  if (irow < Sq) {
    const float lv = a.lse[((int64_t)b * p.Hq + h) * p.Sq + irow];
    lse2 = (lv == -INFINITY) ? INFINITY : lv * kLog2e;
    dls = a.delta[((int64_t)b * p.Hq + h) * p.Sq + irow] * scale;
  }
  wait_vm_loads();

  // key tiles: the sink tiles [0, a1) and the band tiles [a2, a3)
  int64_t s_hi, b_lo, b_hi;
  const int i1 = min(i0 + BQ3, Sq);
  msk.keys_for_rows(i0, i1, Sk, &s_hi, &b_lo, &b_hi);
  const int a1 = (int)((s_hi + BK3 - 1) / BK3);
  int a2 = (int)(b_lo / BK3);
  const int a3 = b_hi > b_lo ? (int)((b_hi + BK3 - 1) / BK3) : a2;
  if (a2 < a1) a2 = a1;
  const int n1 = a1, n2 = a3 > a2 ? a3 - a2 : 0;
  const int n_it = i0 < Sq ? n1 + n2 : 0;
  auto tile_of = [&](int it) { return (int64_t)BK3 * (it < n1 ? it : a2 + (it - n1)); };
  const bool no_mask = msk.kind == kMaskNone;
  const int lo_t = msk.wl < 0 ? -0x3fffffff : -msk.wl;
  const int wr_t = msk.wr;

  f32x16 dq[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) dq[n] = zero16();

  const float* bias_h = BIAS ? a.bias + h * p.bias_str[0] : nullptr;
  const int k_rb = 2 * (int)p.k_str[2], v_rb = 2 * (int)p.v_str[2], b_rb = 4 * (int)p.bias_str[1];
  const int brows = min(Sq - i0, BQ3);
  StageKV<D, BIAS> stg;
  stg.init(k_rb, v_rb, b_rb);
  auto issue = [&](int it) {
    const int j0 = (int)tile_of(it);
    const int keys = min(Sk - j0, BK3);
    stg.load(kp + (int64_t)j0 * p.k_str[2], vp + (int64_t)j0 * p.v_str[2], k_rb, v_rb, keys,
             BIAS ? bias_h + (int64_t)i0 * p.bias_str[1] + j0 : nullptr, (brows - 1) * b_rb + 4 * keys);
  };
  if (n_it > 0) {
    issue(0);
    stg.store(sm, 0);
    __syncthreads();
  }
  for (int it = 0; it < n_it; ++it) {
    const int cur = it & 1;
    const int j0 = (int)tile_of(it);
    if (it + 1 < n_it) issue(it + 1);

    // S^T = K Q^T and dP^T = V dO^T: keys on accumulator rows, this lane's row on the column
    f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      sacc = mfma(lds_b128(sm.kr[cur], rowA + 16 * s), qB[s], sacc);
      dpacc = mfma(lds_b128(sm.vr[cur], rowA + 16 * s), doB[s], dpacc);
    }
    const bool full = (j0 + BK3 <= Sk) && msk.tile_full(i0 + 32 * w, i0 + 32 * w + 32, j0, j0 + BK3);
    // t = j' - i' - diag for key j0 + 4 lg + c
    const int tb = j0 + (int)msk.k_off + 4 * lg - (irow + (int)msk.q_off) - (int)msk.diag;
    float dsv[16];
    auto elem = [&](int r, bool masked) {
      const int c = 8 * (r >> 2) + (r & 3);
      float x = fmaf(sacc[r], scale_log2, -lse2);
      if (BIAS) x = fmaf(sm.bias[cur][(32 * w + lr) * BSTR + 4 * lg + c], kLog2e, x);
      float pp = __builtin_amdgcn_exp2f(x);
      if (masked) {
        const int j = j0 + 4 * lg + c;
        const int t = tb + c;
        const bool ok = (j < Sk) & (no_mask | ((t <= wr_t) & (t >= lo_t)) | ((j + (int)msk.k_off) < msk.n_sink));
        pp = ok ? pp : 0.f;
      }
      dsv[r] = pp * fmaf(dpacc[r], scale, -dls);
    };
    if (full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) elem(r, false);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) elem(r, true);
    }
    const bf16x8 sa0 = pack8(dsv), sa1 = pack8(dsv + 8);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      dq[n] = mfma(sa0, lds_trB(sm.kt[cur], trK, 0, 32 * n, T), dq[n]);
      dq[n] = mfma(sa1, lds_trB(sm.kt[cur], trK, 16, 32 * n, T), dq[n]);
    }
    if (it + 1 < n_it) stg.store(sm, cur ^ 1);
    __syncthreads();
  }

  // dQ rows i0 + 32 w + crow(r, lg), columns 32 n + lr (already scaled through dS).
  float* dqp = a.dq + sv.q_off(p.dq_str, b) + h * p.dq_str[1];
  if (a.accumulate_dq) add_loaded<NB>(dq, dqp, p.dq_str[2], i0 + 32 * w, Sq, lg, lr);
#pragma unroll
  for (int n = 0; n < NB; ++n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t i = i0 + 32 * w + crow(r, lg);
      if (i < Sq) dqp[i * p.dq_str[2] + 32 * n + lr] = dq[n][r];
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel k_dq2 (dQ without a bias): one workgroup of four waves per
// (128-row query block, query head, batch), two workgroups per CU.  Wave w
// owns rows [32 w, 32 w + 32) and keeps Q and dO as B-operand fragments in
// registers.  The 32-key K / V tiles come straight from global memory into
// four LDS buffers (XOR-swizzled, one copy per tile serving the row reads of
// S^T = K Q^T, dP^T = V dO^T and the transposing reads of dQ += dS K), two
// tiles ahead of use.  Per key tile t (one barrier): the S^T / dP^T chains
// of tile t + 1 run between the exponentials and dS arithmetic of tile t,
// then dS(t) K(t) goes into dQ; the loop is unrolled over the buffers so
// every operand read is a lane register plus a constant offset.
// ---------------------------------------------------------------------------
constexpr int NBQ = 4;   // K / V tile buffers (k_dq2)

// Rows of a PartialSum that have partials: those of every key when the
// blocks are split (nsplit > 1), else those of key block 0 only.
__host__ __device__ inline int partial_rows_per_head(const PartialSum& ps) {
  return ps.pt.nsplit > 1 ? ps.Sk : (ps.Sk < BK ? ps.Sk : BK);
}

// Rows [r0, r1) (r = (b Hk + h) nrow + i, nrow from partial_rows_per_head)
// of a PartialSum, thread t of nt (nt a multiple of (Dk + Dv) / 4): the
// dK / dV row of key i gets the partials of its block's parts >= 1 added in
// slot order.  A thread takes one float4 column of every (nt / w)-th row,
// U rows at a time with the loads of up to MS slots of each in flight
// together (further slots follow one at a time); row and element counts fit
// in 32 bits.
__device__ inline void partial_sum_rows(const PartialSum& ps, int r0, int r1, int t, int nt) {
  constexpr int U = 2, MS = 8;
  const int w = (ps.Dk + ps.Dv) / 4, wk = ps.Dk / 4, rw = ps.Dk + ps.Dv;
  const int c = t % w, rstep = nt / w, nrow = partial_rows_per_head(ps);
  for (int rb = r0 + t / w; rb < r1; rb += U * rstep) {
    float4 v[U], y[U][MS];
    float* dst[U];
    const float* src[U];
    int parts[U], kbv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + u * rstep;
      parts[u] = 0;
      if (r < r1) {
        const int bh = r / nrow, i = r - bh * nrow;
        const int b = bh / ps.Hk, h = bh - b * ps.Hk;
        kbv[u] = i / BK;
        parts[u] = kbv[u] == 0 ? ps.pt.nparts0 : ps.pt.nsplit;
        dst[u] = c < wk ? ps.dk + b * ps.dk_str[0] + h * ps.dk_str[1] + i * ps.dk_str[2] + 4 * c
                        : ps.dv + b * ps.dv_str[0] + h * ps.dv_str[1] + i * ps.dv_str[2] + 4 * (c - wk);
        src[u] = ps.pt.base + ((int64_t)bh * ps.pt.nslot * BK + (i - kbv[u] * BK)) * rw + 4 * c;
        if (parts[u] >= 2) {
          v[u] = *(const float4*)dst[u];
#pragma unroll
          for (int q = 1; q <= MS; ++q)
            if (q < parts[u]) y[u][q - 1] = *(const float4*)(src[u] + (int64_t)partial_slot(ps.pt, kbv[u], q) * BK * rw);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (parts[u] < 2) continue;
#pragma unroll
      for (int q = 1; q <= MS; ++q) {
        if (q < parts[u]) {
          v[u].x += y[u][q - 1].x;
          v[u].y += y[u][q - 1].y;
          v[u].z += y[u][q - 1].z;
          v[u].w += y[u][q - 1].w;
        }
      }
      for (int q = MS + 1; q < parts[u]; ++q) {
        const float4 z = *(const float4*)(src[u] + (int64_t)partial_slot(ps.pt, kbv[u], q) * BK * rw);
        v[u].x += z.x;
        v[u].y += z.y;
        v[u].z += z.z;
        v[u].w += z.w;
      }
      *(float4*)dst[u] = v[u];
    }
  }
}

// The sums alone (when no dQ pass follows the key-block pass).
__global__ __launch_bounds__(256) void k_partial_sum(PartialSum ps) {
  const int rows = ps.B * ps.Hk * partial_rows_per_head(ps);
  const int per = (rows + (int)gridDim.x - 1) / (int)gridDim.x;
  const int r0 = blockIdx.x * per;
  partial_sum_rows(ps, r0, min(rows, r0 + per), threadIdx.x, 256);
}

template <int D>
struct __attribute__((aligned(1024))) SmemDQ2 {
  unsigned char k[NBQ][BK3 * 2 * D];   // K tile, swizzled
  unsigned char v[NBQ][BK3 * 2 * D];   // V tile, swizzled
};

template <int D, bool PRIO>
__global__ __launch_bounds__(NT, 2) void k_dq2(Params p, BwdArgs a, ZeroMulti zm, PartialSum ps) {
  constexpr int NS = D / 16;   // k-steps over the head dim
  constexpr int NC = D / 32;   // 32-column blocks of dQ
  constexpr int RB = Swz<D>::RB, CR = Swz<D>::CR;
  constexpr int TS = BK3 * 2 * D;   // tile bytes
  constexpr int PER_T = BK3 * CR / 64;   // 1 KB loads per tile
  constexpr int NI = 2 * PER_T / 4;      // loads per wave per K + V tile pair
  static_assert(NI >= 1 && PER_T % NI == 0, "loads per wave");
  __shared__ SmemDQ2<D> sm;

  const int tid = threadIdx.x, l = tid & 63, lr = l & 31, lg = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  // Side duties for the key-block pass, an even share per workgroup once its
  // own work is done (the memory traffic then overlaps other workgroups'
  // products): the tensors that a key-block pass launched after this one
  // adds into (its split parts) are zeroed ...
  auto zero_share = [&]() {
    if (zm.n > 0) {
      const int64_t nwg = (int64_t)gridDim.x * gridDim.y * gridDim.z;
      const int64_t wg = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
      const int64_t total = zm.off[zm.n], per = (total + nwg - 1) / nwg;
      zero_multi_range(zm, wg * per, min(total, (wg + 1) * per), tid, NT);
    }
    // ... and the partial dK / dV that the key-block pass launched before
    // this one left in slots are added into dK / dV
    if (ps.pt.base != nullptr) {
      const int nwg = (int)(gridDim.x * gridDim.y * gridDim.z);
      const int wg = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
      const int rows = ps.B * ps.Hk * partial_rows_per_head(ps), per = (rows + nwg - 1) / nwg;
      partial_sum_rows(ps, wg * per, min(rows, (wg + 1) * per), tid, NT);
    }
  };
  const BlockXYZ blk = a.xmajor ? xcd_block_xmajor() : xcd_block();
  // under a causal mask later row blocks see more keys: deal them first
  const bool heavy_last = p.mask.kind != kMaskNone && p.mask.wl < 0;
  const int i0 = (heavy_last ? (int)gridDim.x - 1 - blk.x : blk.x) * BQ3;
  const int h = blk.y, b = blk.z, g = h / p.G;
  const SeqView sv = seq_view(p, b);   // this batch entry (or packed sequence)
  const Mask& msk = sv.mask;
  const int Sq = sv.Sq, Sk = sv.Sk;
  if (i0 >= Sq) {   // past this sequence's rows (uniform across the workgroup)
    zero_share();
    return;
  }
  // key tiles: the sink tiles [0, a1) and the band tiles [a2, a3)
  int64_t s_hi, b_lo, b_hi;
  const int i1 = min(i0 + BQ3, Sq);
  msk.keys_for_rows(i0, i1, Sk, &s_hi, &b_lo, &b_hi);
  const int a1 = (int)((s_hi + BK3 - 1) / BK3);
  int a2 = (int)(b_lo / BK3);
  const int a3 = b_hi > b_lo ? (int)((b_hi + BK3 - 1) / BK3) : a2;
  if (a2 < a1) a2 = a1;
  const int n1 = a1, n2 = a3 > a2 ? a3 - a2 : 0;
  const int n_it = n1 + n2;
  if (n_it == 0 && a.accumulate_dq) {   // no key reaches these rows: dQ keeps its values
    zero_share();
    return;
  }
  const int irow = i0 + 32 * w + lr;           // this lane's query row
  const float scale = p.scale, scale_log2 = p.scale * kLog2e;

  const unsigned short* q = (const unsigned short*)a.q + sv.q_off(p.q_str, b) + h * p.q_str[1];
  const unsigned short* dout = (const unsigned short*)a.dout + sv.q_off(p.do_str, b) + h * p.do_str[1];
  const unsigned short* kp = (const unsigned short*)a.k + sv.k_off(p.k_str, b) + g * p.k_str[1];
  const unsigned short* vp = (const unsigned short*)a.v + sv.k_off(p.v_str, b) + g * p.v_str[1];

  // Q / dO fragments (B operands) and the row's LSE and delta: loaded after
  // the first K / V tiles are issued, so that all arrive in one round trip
  bf16x8 qB[NS], doB[NS];
  float lse2 = INFINITY, dls = 0.f;

  auto tile_of = [&](int it) { return BK3 * (it < n1 ? it : a2 + (it - n1)); };
  // this wave's rows: a tile [j0, j0 + 32) is full when every key is
  // allowed for all 32 rows
  const int wr0 = i0 + 32 * w;
  // per-lane key window of the masked tiles: key j is allowed for this
  // lane's row when  j + k_off - (irow + q_off) - diag  lies in [lo_l, lo_l + span]
  const bool no_mask = msk.kind == kMaskNone;
  int lo_l = msk.wl < 0 ? -0x3fffffff : -msk.wl, span = msk.wr - lo_l;
  if (no_mask) { lo_l = -0x3fffffff; span = 0x7ffffffe; }
  const int tq = (int)msk.k_off - (irow + (int)msk.q_off) - (int)msk.diag + 4 * lg - lo_l;
  const int sink_lim = (int)min<int64_t>(max<int64_t>(msk.n_sink - msk.k_off, 0), 0x3fffffff);   // keys below are sinks
  // tile [j0, j0 + 32) full for this wave's 32 rows: every key inside the
  // problem and allowed for every row (all sinks, or inside the band)
  auto clamp_i = [](int64_t x) { return (int)max<int64_t>(min<int64_t>(x, 0x3fffffff), -0x3fffffff); };
  const int64_t band = (int64_t)wr0 + msk.q_off + msk.diag - msk.k_off;
  const int fl_hi = no_mask ? 0x3fffffff : clamp_i(band + msk.wr - 31);
  const int fl_lo = (no_mask || msk.wl < 0) ? -0x3fffffff : clamp_i(band + 31 - msk.wl);
  const int fl_sink = no_mask ? -0x3fffffff : clamp_i((int64_t)msk.n_sink - 31 - msk.k_off);
  auto tile_full = [&](int j0) { return (j0 + BK3 <= Sk) & ((j0 < fl_sink) | ((j0 <= fl_hi) & (j0 >= fl_lo))); };

  // staging: wave w issues NI 1 KB loads of the K (waves 0, 1) or V tile
  const int k_rb = 2 * (int)p.k_str[2], v_rb = 2 * (int)p.v_str[2];
  const bool ld_v = w * NI >= PER_T;
  int voff[NI];
  unsigned int dst0[NI];
  const unsigned int sm_base = __builtin_amdgcn_readfirstlane(lds_addr(&sm));
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int slot = (w * NI + k) % PER_T;
    const int row = (64 * slot + l) / CR;
    voff[k] = row * (ld_v ? v_rb : k_rb) + 16 * ((l % CR) ^ Swz<D>::f(row));
    dst0[k] = sm_base + (ld_v ? offsetof(SmemDQ2<D>, v) : offsetof(SmemDQ2<D>, k)) + 1024 * slot;
  }
  // tile walk: the next tile to load (its first key and this wave's K or V
  // pointer) and the tile being formed, advanced one tile at a time (the
  // step from the last sink tile to the first band tile jumps)
  const unsigned short* const src0 = ld_v ? vp : kp;
  const int64_t src_str = ld_v ? p.v_str[2] : p.k_str[2];
  const int src_rb = ld_v ? v_rb : k_rb;
  int ld_it = 0, ld_j0 = tile_of(0);
  const unsigned short* ld_src = src0 + (int64_t)ld_j0 * src_str;
  auto issue = [&](int buf) {
    const int keys = min(Sk - ld_j0, BK3);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(ld_src, keys * src_rb);
#pragma unroll
    for (int k = 0; k < NI; ++k) lds_dma16(rs, __builtin_amdgcn_readfirstlane(dst0[k] + buf * TS), voff[k]);
    if (++ld_it == n1) {
      ld_j0 = BK3 * a2;
      ld_src = src0 + (int64_t)ld_j0 * src_str;
    } else {
      ld_j0 += BK3;
      ld_src += BK3 * src_str;
    }
  };
  int cur_it = 0, cur_j0 = tile_of(0);
  auto advance_cur = [&]() {
    if (++cur_it == n1) cur_j0 = BK3 * a2;
    else cur_j0 += BK3;
  };

  f32x16 dq[NC];
#pragma unroll
  for (int n = 0; n < NC; ++n) dq[n] = zero16();

  if (n_it > 0) {
    // K tile buffer 3 zeroed (read by the zero dQ products ahead of tile 0)
#pragma unroll
    for (int k = 0; k < TS / (16 * NT); ++k) *(u16x8*)&sm.k[NBQ - 1][16 * (tid + NT * k)] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    // tiles 0 and 1, the Q / dO fragments, LSE and delta in flight together,
    // all complete before the first barrier
    issue(0);
    if (n_it > 1) issue(1);
    {
      const int64_t ic = min(irow, Sq - 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        qB[s] = as_bf16x8(*(const u16x8*)(q + ic * p.q_str[2] + 16 * s + 8 * lg));
        doB[s] = as_bf16x8(*(const u16x8*)(dout + ic * p.do_str[2] + 16 * s + 8 * lg));
      }
    }
    if (irow < Sq) {
      const float lv = a.lse[((int64_t)b * p.Hq + h) * p.Sq + irow];
      lse2 = (lv == -INFINITY) ? INFINITY : lv * kLog2e;
      dls = a.delta[((int64_t)b * p.Hq + h) * p.Sq + irow] * scale;
    }
    wait_vm_loads();

    // operand read addresses in tile buffer 0
    const int a_lane = Swz<D>::a_lane(l), t_lane = Swz<D>::t_lane(l);
    const unsigned int k_t0 = sm_base + offsetof(SmemDQ2<D>, k), v_t0 = sm_base + offsetof(SmemDQ2<D>, v);
    unsigned int br[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) br[n] = k_t0 + (t_lane ^ (64 * n));
    const unsigned int ka = k_t0 + a_lane, va = v_t0 + a_lane;
    // K / V rows of chain step s and K^T of dQ product i in tile buffer j (a
    // constant; the buffers are 1 KB aligned, so the XOR stays in the row)
    auto read_k = [&](int j, int s) { return lds_b128_at((ka ^ (32 * s)) + j * TS); };
    auto read_v = [&](int j, int s) { return lds_b128_at((va ^ (32 * s)) + j * TS); };
    auto read_kt = [&](int j, int i) {
      const int n = i % NC, r0 = 16 * (i / NC);
      return cat44(lds_tr4_at(br[n] + j * TS + r0 * RB), lds_tr4_at((br[n] ^ 32) + j * TS + (r0 + 8) * RB));
    };
    constexpr int AHEAD = 2;
    // dS of the previous tile (dQ operands); before the first tile zeros,
    // against the K tile buffer 3 zeroed in the prologue
    bf16x8 A0 = as_bf16x8(u16x8{0, 0, 0, 0, 0, 0, 0, 0}), A1 = A0;
    // P (masked) and dP^T of the previous tile: its dS is formed while the
    // next tile's chains run; zeros before the first tile (dS = 0)
    float pp[16], pc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) { pp[r] = 0.f; pc[r] = 0.f; }
    auto ds_prev = [&]() {
      float dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) dsv[r] = pp[r] * fmaf(pc[r], scale, -dls);
      A0 = pack8(dsv);
      A1 = pack8(dsv + 8);
    };

    // tile t in buffer j: dS of tile t - 1, the S^T / dP^T chains of tile t
    // among the dQ products of tile t - 1, then the exponentials of tile t
    auto tile = [&](int t, int j, bool full, int j0) {
      const int jp = (j + NBQ - 1) % NBQ;
      ds_prev();
      constexpr bool DQ = true;
      bf16x8 xk[NS], xv[NS], bq[NS];
      f32x16 sacc = zero16(), pacc = zero16();
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) {
        xk[i] = read_k(j, i);
        xv[i] = read_v(j, i);
        if (DQ) bq[i] = read_kt(jp, i);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        sacc = mfma(xk[i], qB[i], sacc);
        if (DQ) dq[i % NC] = mfma(i < NC ? A0 : A1, bq[i], dq[i % NC]);
        pacc = mfma(xv[i], doB[i], pacc);
        if (i + AHEAD < NS) {
          xk[i + AHEAD] = read_k(j, i + AHEAD);
          xv[i + AHEAD] = read_v(j, i + AHEAD);
          if (DQ) bq[i + AHEAD] = read_kt(jp, i + AHEAD);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const int tb = tq + j0;   // window offset of key j0 + 4 lg for this lane's row
#pragma unroll
      for (int r = 0; r < 16; ++r) pp[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, -lse2));
      if (!full) {   // (the branch touches P only)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 8 * (r >> 2) + (r & 3);
          const int jj = j0 + 4 * lg + c;
          const bool ok = (jj < Sk) & (((unsigned int)(tb + c) <= (unsigned int)span) | (jj < sink_lim));
          pp[r] = ok ? pp[r] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) pc[r] = pacc[r];
    };
    auto step = [&](int t) {
      const int j = t % NBQ;
      __syncthreads();  // tile t complete; tile t - 2's buffer free
      const bool more = t + 2 < n_it;
      if (more) issue((j + 2) % NBQ);
      tile(t, j, tile_full(cur_j0), cur_j0);
      advance_cur();
      // tile t + 1 complete before the next barrier (tile t + 2 may stay in flight)
      wait_vm_keep<NI>(more);
    };
    auto tilec = [&](int t, auto jc, bool full, int j0) {
      constexpr int j = decltype(jc)::value, jp = (j + NBQ - 1) % NBQ;
      constexpr int EPS = 16 / NS;   // accumulator elements per chain step
      // Issue priority: low over region 1, raised from region 2 to the end of
      // the tile.  The two waves sharing a SIMD come from different
      // workgroups and run in any phase; when both are ready, the one among
      // its exponentials and independent dQ products issues first, and the
      // other's dependent chain products fill the matrix pipe behind it
      // (measured on GQA 32:8, S = 4096, D = 128, causal: 199 -> 188 us;
      // raised over region 1 instead, 197 us).  Only when the launch holds
      // two workgroups per CU (PRIO): alone on its SIMD a wave lost 3 % to it.
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
      // region 1: the S^T / dP^T chains of tile t (two independent chains)
      // among the dS arithmetic of tile t - 1
      f32x16 sacc = zero16(), pacc = zero16();
      {
        bf16x8 xk[NS], xv[NS];
        float dsv[16];
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) { xk[i] = read_k(j, i); xv[i] = read_v(j, i); }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          sacc = mfma(xk[i], qB[i], sacc);
          pacc = mfma(xv[i], doB[i], pacc);
#pragma unroll
          for (int e = 0; e < EPS; ++e) {
            const int r = EPS * i + e;
            dsv[r] = pp[r] * fmaf(pc[r], scale, -dls);
          }
          if (i == NS / 2 - 1) A0 = pack8(dsv);
          if (i + AHEAD < NS) { xk[i + AHEAD] = read_k(j, i + AHEAD); xv[i + AHEAD] = read_v(j, i + AHEAD); }
          __builtin_amdgcn_sched_barrier(0);
        }
        A1 = pack8(dsv + 8);
      }
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
      // region 2: the dQ products of tile t - 1 among the exponentials of tile t
      {
        bf16x8 bq[NS];
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) bq[i] = read_kt(jp, i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          dq[i % NC] = mfma(i < NC ? A0 : A1, bq[i], dq[i % NC]);
#pragma unroll
          for (int e = 0; e < EPS; ++e) {
            const int r = EPS * i + e;
            pp[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, -lse2));
          }
          if (i + AHEAD < NS) bq[i + AHEAD] = read_kt(jp, i + AHEAD);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (!full) {   // (the branch touches P only)
        const int tb = tq + j0;   // window offset of key j0 + 4 lg for this lane's row
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 8 * (r >> 2) + (r & 3);
          const int jj = j0 + 4 * lg + c;
          const bool ok = (jj < Sk) & (((unsigned int)(tb + c) <= (unsigned int)span) | (jj < sink_lim));
          pp[r] = ok ? pp[r] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) pc[r] = pacc[r];
    };
    auto stepc = [&](int t, auto jc) {
      constexpr int j = decltype(jc)::value;
      __syncthreads();  // tile t complete; tile t - 2's buffer free
      const bool more = t + 2 < n_it;
      if (more) issue((j + 2) % NBQ);
      tilec(t, jc, tile_full(cur_j0), cur_j0);
      advance_cur();
      // tile t + 1 complete before the next barrier (tile t + 2 may stay in flight)
      wait_vm_keep<NI>(more);
    };
    // main loop unrolled over the four buffers (constant read offsets), then
    // the remaining tiles
    int t = 0;
    for (; t + NBQ <= n_it; t += NBQ) {
      stepc(t, std::integral_constant<int, 0>{});
      stepc(t + 1, std::integral_constant<int, 1>{});
      stepc(t + 2, std::integral_constant<int, 2>{});
      stepc(t + 3, std::integral_constant<int, 3>{});
    }
    for (; t < n_it; ++t) step(t);
    // the dS and dQ products of the last tile
    ds_prev();
    {
      const unsigned int jb = ((n_it - 1) % NBQ) * TS;
      bf16x8 bq[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int n = i % NC, r0 = 16 * (i / NC);
        bq[i] = cat44(lds_tr4_at(br[n] + jb + r0 * RB), lds_tr4_at((br[n] ^ 32) + jb + (r0 + 8) * RB));
      }
#pragma unroll
      for (int i = 0; i < NS; ++i) dq[i % NC] = mfma(i < NC ? A0 : A1, bq[i], dq[i % NC]);
    }
  }

  // dQ rows i0 + 32 w + crow(r, lg), columns 32 n + lr (already scaled through dS).
  float* dqp = a.dq + sv.q_off(p.dq_str, b) + h * p.dq_str[1];
  if (a.accumulate_dq) add_loaded<NC>(dq, dqp, p.dq_str[2], i0 + 32 * w, Sq, lg, lr);
#pragma unroll
  for (int n = 0; n < NC; ++n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t i = i0 + 32 * w + crow(r, lg);
      if (i < Sq) dqp[i * p.dq_str[2] + 32 * n + lr] = dq[n][r];
    }
  }
  zero_share();
}

// ---------------------------------------------------------------------------
// Kernel k_dqb (dQ and dbias, head dim 64): one workgroup of eight waves per
// (128-row block, query head), two waves per SIMD; wave w owns rows
// 16 w .. 16 w + 15 for every batch entry.  The batch is walked innermost,
// in groups of up to BGB entries.  For each 32-key tile the workgroup stages
// the group's K / V tiles and the [128 x 32] fp32 bias tile (one copy for all
// entries: the bias is shared over the batch) straight into LDS, two tiles
// ahead, and each wave, entry by entry, forms S^T = K Q^T (16x16x32 products;
// the chain starts from bias / scale) and dP^T = V dO^T (keys on accumulator
// rows, one query row per lane, the Q / dO fragments of the group's entries
// in registers), P, dS, dQ += dS K, and adds dS into a register dbias tile,
// which it stores (the first group) or adds to dbias (later groups) once per
// tile: dbias = sum_b dS is written once per group, in a fixed order.  A
// lane holds keys 4 g + 0..3 and 16 + 4 g + 0..3 (g = lane / 16) of its row:
// two 16-byte chunks of the bias and dbias rows, and directly the eight
// reduction slots of its dQ = dS K operand.  A group with fewer than BGB
// entries fills the rest with copies of its last entry whose P is zero.
// ---------------------------------------------------------------------------
constexpr int BGB = 4;     // batch entries per group (k_dqb)
constexpr int NQB = 3;     // tile buffers (k_dqb)
constexpr int NTB = 512;   // threads per workgroup (k_dqb)
struct DbTile {   // a lane's two dbias chunks of a tile
  f32x4 c0, c1;
};

template <int D>
struct __attribute__((aligned(1024))) SmemDQB {
  unsigned char kv[NQB][BGB][2][BK3 * 2 * D];   // K then V tile of each entry, swizzled
  float bias[NQB][BQ3 * BK3];                   // bias[i0 + r][j0 + c] / scale, 16-byte chunks swizzled by row
};
static_assert(sizeof(SmemDQB<64>) <= 160 * 1024, "k_dqb LDS");

template <int D>
__global__ __launch_bounds__(NTB, 1) void k_dqb(Params p, BwdArgs a) {
  static_assert(D == 64, "head dim 64");
  constexpr int RB = Swz<D>::RB, CR = Swz<D>::CR;
  constexpr int TS = BK3 * 2 * D;            // K or V tile bytes
  constexpr int PER_T = BK3 * CR / 64;       // 1 KB loads per K or V tile
  constexpr int BUF_B = BGB * 2 * TS;        // one buffer of K / V tiles
  constexpr int BTB = BQ3 * BK3 * 4;         // bias tile bytes
  constexpr int BIAS_OFF = (int)offsetof(SmemDQB<D>, bias);
  constexpr int NI = PER_T + 2;              // loads per wave per tile
  static_assert(PER_T == 4 && BTB == 16384 && RB == 128, "one K or V tile and 16 bias rows per wave");
  __shared__ SmemDQB<D> sm;

  const int tid = threadIdx.x, l = tid & 63, j = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const BlockXYZ blk = xcd_block();
  const int i0 = blk.x * BQ3, h = blk.y, hk = h / p.G;
  const Mask& msk = p.mask;
  const int Sq = p.Sq, Sk = p.Sk;
  if (i0 >= Sq) return;
  const int irow = i0 + 16 * w + j;   // this lane's query row
  const bool row_ok = irow < Sq;
  const float scale = p.scale, scale_log2 = p.scale * kLog2e, inv_scale = 1.f / p.scale;

  // key tiles: the sink tiles [0, a1) and the band tiles [a2, a3)
  int64_t s_hi, b_lo, b_hi;
  msk.keys_for_rows(i0, min(i0 + BQ3, Sq), Sk, &s_hi, &b_lo, &b_hi);
  const int a1 = (int)((s_hi + BK3 - 1) / BK3);
  int a2 = (int)(b_lo / BK3);
  const int a3 = b_hi > b_lo ? (int)((b_hi + BK3 - 1) / BK3) : a2;
  if (a2 < a1) a2 = a1;
  const int n1 = a1, n2 = a3 > a2 ? a3 - a2 : 0, n_it = n1 + n2;
  auto tile_of = [&](int it) { return BK3 * (it < n1 ? it : a2 + (it - n1)); };
  const bool no_mask = msk.kind == kMaskNone;
  int lo_l = msk.wl < 0 ? -0x3fffffff : -msk.wl, span = msk.wr - lo_l;
  if (no_mask) { lo_l = -0x3fffffff; span = 0x7ffffffe; }
  // window offset of key 4 g (+ 16 mt + i) of a tile for this lane's row
  const int tq = (int)msk.k_off - (irow + (int)msk.q_off) - (int)msk.diag + 4 * g - lo_l;
  const int sink_lim = (int)min<int64_t>(max<int64_t>(msk.n_sink - msk.k_off, 0), 0x3fffffff);
  // a tile is full for this wave when every key is inside the problem and
  // allowed for all 16 of its rows
  const int wr0 = i0 + 16 * w;
  auto clamp_i = [](int64_t x) { return (int)max<int64_t>(min<int64_t>(x, 0x3fffffff), -0x3fffffff); };
  const int64_t band = (int64_t)wr0 + msk.q_off + msk.diag - msk.k_off;
  const int fl_hi = no_mask ? 0x3fffffff : clamp_i(band + msk.wr - 31);
  const int fl_lo = (no_mask || msk.wl < 0) ? -0x3fffffff : clamp_i(band + 15 - msk.wl);
  const int fl_sink = no_mask ? -0x3fffffff : clamp_i((int64_t)msk.n_sink - 31 - msk.k_off);
  auto tile_full = [&](int j0) { return (j0 + BK3 <= Sk) & ((j0 < fl_sink) | ((j0 <= fl_hi) & (j0 >= fl_lo))); };

  const unsigned int sm_base = __builtin_amdgcn_readfirstlane(lds_addr(&sm));
  const int b_rb = 4 * (int)p.bias_str[1];
  const int brows = min(Sq - i0, BQ3);
  const float* bias_h = a.bias + h * p.bias_str[0] + (int64_t)i0 * p.bias_str[1];
  // staging: wave w loads the K (w < 4) or V tile of entry w % 4 of the group
  // (four 1 KB loads; a group with fewer entries loads its last entry's
  // instead) and bias rows 16 w .. 16 w + 15 (two 1 KB loads of 8 rows;
  // 16-byte chunk c of row r lands at chunk c ^ ((r / 2) % 8): a 128-byte row
  // covers half the banks, row parity picks the half, and the 16 rows that one
  // read serves at a time fall on distinct banks)
  const int we = w & 3, wkv = w >> 2;
  const int64_t* kv_str = wkv == 0 ? p.k_str : p.v_str;
  const int kv_rb = 2 * (int)kv_str[2];
  const unsigned char* kv_head =
      (const unsigned char*)((wkv == 0 ? (const unsigned short*)a.k : (const unsigned short*)a.v) + hk * kv_str[1]);
  const int64_t kv_bbytes = 2 * kv_str[0];
  const unsigned int kv_dst = sm_base + (we * 2 + wkv) * TS;
  // K / V tiles: 16-byte chunk c of row r sits at chunk c ^ fq(r).  LDS
  // serves these reads 32 lanes at a time from 64 banks of 8 bytes
  // (measured), so a 128-byte row covers 16 banks and rows r, r + 4, r + 8,
  // r + 12 share them: fq gives those four rows distinct chunk pairs, and
  // both read patterns -- one chunk of 16 consecutive rows (the A operands)
  // and two chunks of 8 consecutive rows (the transposing reads of dQ's B
  // operand) -- fall on distinct banks.
  auto fq = [](int r) { return 2 * ((r >> 2) & 3) + ((r >> 1) & 1); };
  const unsigned char* kv_grp = kv_head;   // the group's entry w % 4 (or its last)
  struct DmaB {
    __amdgpu_buffer_rsrc_t rs, rb;
    int buf;
  };
  auto dma_set = [&](int it, int buf, bool on) {
    DmaB d;
    const int j0 = tile_of(on ? it : 0);
    const int keys = on ? min(Sk - j0, BK3) : 0;
    d.rs = buf_rsrc(kv_grp + j0 * kv_rb, keys * kv_rb);
    d.rb = buf_rsrc(bias_h + j0, on ? (brows - 1) * b_rb + 4 * keys : 0);
    d.buf = buf;
    return d;
  };
  // A tile's loads are set up at the barrier and issued two at a time after
  // the first entries' products: issued together right after the barrier,
  // the eight waves' 48 KB queue for the vector memory unit and hold up the
  // products behind them.  With `on` false they load nothing (zeros into a
  // buffer no later tile reads).
  auto dma_one = [&](const DmaB& d, int k) {   // k < PER_T: K / V slot k, else bias rows
    if (k < PER_T) {
      const int row = (64 * k + l) / CR, c = (l % CR) ^ fq(row);
      lds_dma16(d.rs, __builtin_amdgcn_readfirstlane(kv_dst + d.buf * BUF_B + 1024 * k), row * kv_rb + 16 * c);
    } else {
      const int kb = k - PER_T;
      const int row = 16 * w + 8 * kb + (l >> 3), c = (l & 7) ^ ((row >> 1) & 7);
      lds_dma16(d.rb, __builtin_amdgcn_readfirstlane(sm_base + BIAS_OFF + d.buf * BTB + (16 * w + 8 * kb) * 128),
                row * b_rb + 16 * c);
    }
  };
  auto issue = [&](int it, int buf) {
    const DmaB d = dma_set(it, buf, true);
#pragma unroll
    for (int k = 0; k < NI; ++k) dma_one(d, k);
  };
  // bias / scale in place: each wave scales the 16 rows it loaded itself
  // (complete once its own loads are; only this wave reads them)
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  auto scale_bias = [&](int buf) {
    const unsigned int o = sm_base + BIAS_OFF + buf * BTB + 16 * w * 128 + 16 * l;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      lds_f32x4* x = (lds_f32x4*)(size_t)(o + 1024 * k);
      *x = *x * inv_scale;
    }
  };

  // operand lane addresses (buffer 0, entry 0's K tile; tiles are reached by
  // immediate offsets):
  //  * A of S^T / dP^T: K / V row 16 mt + j, chunk g + 4 s  ->  (a16 ^ 64 s) + 2048 mt
  //  * B of dQ (transposing reads): lane 4 r + cc of group g addresses K row
  //    16 h + 4 g + r, columns 16 nt + 4 cc ..  ->  (tb16 ^ 32 nt) + 2048 h
  //  * bias row 16 w + j, chunk 4 mt + g  ->  bb ^ 64 mt
  const unsigned int a16 = sm_base + j * RB + 16 * (g ^ fq(j));
  const int tr = j >> 2, tc = j & 3;
  const int ftr = fq(4 * g + tr);
  const unsigned int tb16 = sm_base + (4 * g + tr) * RB + 16 * ((tc >> 1) ^ ftr) + 8 * (tc & 1);
  unsigned int ta[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) ta[nt] = tb16 ^ (32 * nt);
  const unsigned int aa[2] = {a16, a16 ^ 64};
  const int brow = 16 * w + j;
  const unsigned int bb = sm_base + BIAS_OFF + brow * 128 + 16 * (g ^ ((brow >> 1) & 7));
  const unsigned int bl[2] = {bb, bb ^ 64};

  float* dbias_h = a.dbias + h * p.bias_str[0] + (int64_t)i0 * p.bias_str[1];
  const int db_off = brow * b_rb + 16 * g;   // this lane's row, keys 4 g + 0..3 of a tile
  for (int b0 = 0; b0 < p.B; b0 += BGB) {
    const int nb = min(BGB, p.B - b0);
    const bool first = b0 == 0;
    // the group's Q / dO fragments (B operands: row j, head-dim columns
    // 8 g + 32 s ..), LSE * log2(e) and -delta of this lane's row
    bf16x8 qB[BGB][2], doB[BGB][2];
    float lse2[BGB], ndl[BGB];
    f32x4 dq[BGB][4];
#pragma unroll
    for (int e = 0; e < BGB; ++e) {
      const int b = b0 + min(e, nb - 1);
      const int64_t ic = min(irow, Sq - 1);
      const unsigned short* q = (const unsigned short*)a.q + b * p.q_str[0] + h * p.q_str[1] + ic * p.q_str[2];
      const unsigned short* d = (const unsigned short*)a.dout + b * p.do_str[0] + h * p.do_str[1] + ic * p.do_str[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        qB[e][s] = as_bf16x8(*(const u16x8*)(q + 32 * s + 8 * g));
        doB[e][s] = as_bf16x8(*(const u16x8*)(d + 32 * s + 8 * g));
      }
      lse2[e] = INFINITY;   // P = 0: rows past the end and the filler entries
      ndl[e] = 0.f;
      if (row_ok && e < nb) {
        const float lv = a.lse[((int64_t)b * p.Hq + h) * p.Sq + irow];
        lse2[e] = (lv == -INFINITY) ? INFINITY : lv * kLog2e;
        ndl[e] = -a.delta[((int64_t)b * p.Hq + h) * p.Sq + irow];
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) dq[e][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    kv_grp = kv_head + (b0 + min(we, nb - 1)) * kv_bbytes;
    wait_vm_loads();
    __syncthreads();   // the previous group's readers of the tile buffers are done
    if (n_it > 0) {
      issue(0, 0);
      if (n_it > 1) issue(1, 1);
    }
    if (n_it > 1) wait_vm_c<NI>();
    else wait_vm_c<0>();
    if (n_it > 0) scale_bias(0);

    // the products and arithmetic of one tile in buffer J; full: no key of
    // the tile is masked for this wave's rows.  A masked pair starts its S^T
    // chain from -inf instead of bias / scale: the products are finite, so the
    // chain ends at -inf and P = 0 for every entry (LSE is never -inf here).
    // The mask is applied once per tile, before any product, and the entries
    // form one straight block.
    auto body = [&](int j0, auto Jc, bool full, const DmaB& dm) {
      constexpr int J = decltype(Jc)::value;
      const int tb = tq + j0;
      f32x4 bz[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) bz[mt] = *(const lds_f32x4*)(size_t)(bl[mt] + J * BTB);
      if (!full) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int c = 16 * (r >> 2) + (r & 3);   // key 4 g + c of the tile
          const int jj = j0 + 4 * g + c;
          const bool ok = (jj < Sk) & (((unsigned int)(tb + c) <= (unsigned int)span) | (jj < sink_lim));
          bz[r >> 2][r & 3] = ok ? bz[r >> 2][r & 3] : -INFINITY;
        }
      }
      f32x4 db[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int e = 0; e < BGB; ++e) {
        const int kt = J * BUF_B + e * 2 * TS, vt = kt + TS;
        // S^T starts from bias / scale, so it ends at (S scale + bias) / scale
        f32x4 sacc[2] = {bz[0], bz[1]};
        f32x4 pacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = mfma16(lds_b128_at(aa[s] + kt + 2048 * mt), qB[e][s], sacc[mt]);
            pacc[mt] = mfma16(lds_b128_at(aa[s] + vt + 2048 * mt), doB[e][s], pacc[mt]);
          }
        }
        // P, then dS = P (dP - delta), unscaled (dQ takes the scale once at the end)
        float dsv[8];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) dsv[4 * mt + i] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][i], scale_log2, -lse2[e]));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dsv[4 * mt + i] *= pacc[mt][i] + ndl[e];
            db[mt][i] += dsv[4 * mt + i];
          }
        const bf16x8 A = pack8(dsv);
        // two of the next-but-one tile's loads after each of the first entries
        if (2 * e < NI) dma_one(dm, 2 * e);
        if (2 * e + 1 < NI) dma_one(dm, 2 * e + 1);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const bf16x8 bq = cat44(lds_tr4_at(ta[nt] + kt), lds_tr4_at(ta[nt] + kt + 2048));
          dq[e][nt] = mfma16(A, bq, dq[e][nt]);
        }
      }
      return DbTile{db[0], db[1]};
    };

    // tile t in buffer J
    auto tile = [&](int t, auto Jc) {
      constexpr int J = decltype(Jc)::value;
      __syncthreads();   // tile t complete for every wave; tile t - 1's buffer free
      const DmaB dm = dma_set(t + 2, (J + 2) % NQB, t + 2 < n_it);
      const int j0 = tile_of(t);
      const DbTile dbt = body(j0, Jc, tile_full(j0), dm);
      const f32x4 db[2] = {dbt.c0, dbt.c1};
      // dbias of this tile (unscaled dS summed over the group): this lane's
      // row, keys j0 + 16 mt + 4 g + 0..3.  A whole key tile is stored by two
      // buffer stores from every lane (rows past the end fall outside the
      // resource and are dropped), so the count of memory operations is the
      // same in every wave; the ragged last tile stores the chunks inside the
      // problem only.
      const bool whole = j0 + BK3 <= Sk;
      const __amdgpu_buffer_rsrc_t rd = buf_rsrc(dbias_h + j0, (brows - 1) * b_rb + 4 * min(BK3, Sk - j0));
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        if (whole || (row_ok && j0 + 16 * mt + 4 * g < Sk)) {
          f32x4 v = db[mt];
          if (!first) v += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, db_off + 64 * mt, 0, 0));
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rd, db_off + 64 * mt, 0, 0);
        }
      }
      // Tile t + 1 complete before the next barrier (tile t + 2 may stay in
      // flight).  Behind tile t + 1's loads come the dbias stores of tile
      // t - 1, then tile t + 2's loads and this tile's dbias stores (vector
      // memory operations complete in issue order).  Only the last tile can
      // be ragged, so tile t - 1 was whole here.
      if (t + 2 < n_it && whole && first) {
        if (t > 0) wait_vm_c<NI + 4>();
        else wait_vm_c<NI + 2>();
      } else {
        wait_vm_c<0>();
      }
      if (t + 1 < n_it) scale_bias((J + 1) % NQB);   // (own rows of tile t + 1, complete)
    };
    int t = 0;
    for (; t + NQB <= n_it; t += NQB) {
      tile(t, std::integral_constant<int, 0>{});
      tile(t + 1, std::integral_constant<int, 1>{});
      tile(t + 2, std::integral_constant<int, 2>{});
    }
    if (t < n_it) tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < n_it) tile(t + 1, std::integral_constant<int, 1>{});

    // dQ of the group's entries: rows i0 + 16 w + 4 g + i, columns 16 nt + j
#pragma unroll
    for (int e = 0; e < BGB; ++e) {
      if (e >= nb) break;
      float* dqp = a.dq + (b0 + e) * p.dq_str[0] + h * p.dq_str[1];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dq[e][nt][i] *= scale;
      }
      if (a.accumulate_dq) {   // every load ahead of the adds (in flight together)
        f32x4 old[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t r = i0 + 16 * w + 4 * g + i;
            old[nt][i] = r < Sq ? dqp[r * p.dq_str[2] + 16 * nt + j] : 0.f;
          }
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) dq[e][nt] = old[nt] + dq[e][nt];
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t r = i0 + 16 * w + 4 * g + i;
          if (r < Sq) dqp[r * p.dq_str[2] + 16 * nt + j] = dq[e][nt][i];
        }
      }
    }
  }
}

// zm / ps: tensors to zero, partials to sum on the way (k_dq2 only: none
// with a bias)
template <int D>
hipError_t launch_dq(const Params& p, const BwdArgs& a0, const ZeroMulti& zm, const PartialSum& ps,
                     hipStream_t st) {
  const dim3 grid((p.Sq + BQ3 - 1) / BQ3, p.Hq, p.B);
  BwdArgs a = a0;
  a.xmajor = xmajor_fits(p, grid.y, grid.z) ? 1 : 0;
  if (a.bias && a.dbias && D == 64)   // dQ and dbias, the batch walked inside
    hipLaunchKernelGGL((k_dqb<64>), dim3(grid.x, grid.y, 1), dim3(NTB), 0, st, p, a);
  else if (a.bias)
    hipLaunchKernelGGL((k_dq<D, true>), grid, dim3(NT), 0, st, p, a);
  else if ((int64_t)grid.x * grid.y * grid.z >= 2 * 256)   // two workgroups per CU: issue priorities
    hipLaunchKernelGGL((k_dq2<D, true>), grid, dim3(NT), 0, st, p, a, zm, ps);
  else
    hipLaunchKernelGGL((k_dq2<D, false>), grid, dim3(NT), 0, st, p, a, zm, ps);
  return hipGetLastError();
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

}  // namespace

bool mfma_bwd_supported(const Params& p) {
  if (p.Dqk != p.Dv || (p.Dqk != 64 && p.Dqk != 128)) return false;
  // 16-byte row loads need every row stride to be a multiple of 8 elements
  const int64_t* s[] = {p.q_str, p.k_str, p.v_str, p.do_str};
  for (const int64_t* x : s)
    for (int i = 0; i < 3; ++i)
      if (x[i] % 8 != 0) return false;
  return true;
}

bool xmajor_fits(const Params& p, int ny, int nz) {
  const int U = ny * nz;
  if (U % 8 != 0) return false;
  const int per = U / 8;   // units of XCD 0: unit u is head u / nz, batch entry u % nz
  int pairs = 0, last_z = -1, last_g = -1;
  for (int u = 0; u < per; ++u) {
    const int z = u % nz, g = (u / nz) / p.G;
    if (z != last_z || g != last_g) ++pairs;   // consecutive units share a K / V head when both match
    last_z = z;
    last_g = g;
  }
  // distinct (batch entry, KV head) pairs are at most `pairs` (runs of equal ones counted once)
  const double bytes = (double)pairs * p.Sk * (p.Dqk + p.Dv) * 2.0;
  return bytes <= 3.0 * 1024 * 1024;
}

// Partial sums are kept for dense problems whose row and element counts
// fit in 32 bits.
static bool partials_fit(const Params& p) {
  return p.cu_k == nullptr && (int64_t)p.B * p.Hk * p.Sk * ((p.Dqk + p.Dv) / 4) < ((int64_t)1 << 31);
}

// The key-block plan of a call: with partial sums when `partials` allows
// them and a unit splits into more than two parts (or into two added into
// existing values in deterministic mode); otherwise with atomic parts,
// which for at most two parts onto zeroed outputs cost no more (measured)
// and stay deterministic.
static DkdvPlan plan_bwd(const Params& p, bool bloop, bool accumulate_dkdv, bool deterministic, bool partials) {
  DkdvPlan pl = plan_dkdv(p, bloop, accumulate_dkdv, deterministic, partials);
  if (partials && pl.g.pt.nparts0 <= 2 && pl.g.nsplit <= 2 && !(deterministic && accumulate_dkdv))
    pl = plan_dkdv(p, bloop, accumulate_dkdv, deterministic, false);
  return pl;
}

static int64_t partial_bytes(const Params& p, const DkdvPlan& pl) {
  return (int64_t)p.B * p.Hk * pl.g.pt.nslot * BK * (p.Dqk + p.Dv) * (int64_t)sizeof(float);
}

hipError_t launch_bwd_mfma(const Params& p, const BwdArgs& a, hipStream_t st) {
  if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v) || !aligned16(a.dout))
    return launch_bwd_simt(p, a, 1, st);
  // bias tiles are staged 16 bytes at a time
  if (a.bias && (!aligned16(a.bias) || p.Sk % 4 != 0 || p.bias_str[0] % 4 != 0 || p.bias_str[1] % 4 != 0))
    return launch_bwd_simt(p, a, 1, st);
  const bool bias = a.bias != nullptr;
  // dbias: the first batch entry stores the dS of every tile it visits;
  // without a mask every tile is visited, so only masked problems need the
  // tiles that no key block reaches zeroed first
  if (a.dbias && p.mask.kind != kMaskNone && p.Sq > 0 && p.Sk > 0 && p.B > 0) {
    hipError_t e = launch_zero_bias(a.dbias, p.Hq, p.Sq, p.Sk, p.bias_str, st);
    if (e != hipSuccess) return e;
  }
  // dK / dV by key blocks (k_dkdv3 / k_dkdv2; k_dkdv with a bias, where dbias is
  // summed over the batch in a fixed order by one workgroup per key block
  // walking the batch) and dQ by query blocks (k_dq2; k_dq with a bias): no
  // dQ atomics.  Units of dense problems without a bias split into more than
  // two parts leave the partial dK / dV of their parts >= 1 in the caller's
  // workspace, and the dQ pass, run second, adds them in slot order.  Otherwise split
  // parts add atomically into zeroed dK / dV; those are zeroed by the dQ
  // pass, run first, when it is k_dq2 and reads its K / V mostly from L2
  // (the stores then cost it little), else by a zero kernel ahead of the
  // key-block pass.
  // head dim 64: k_dkdv3 takes the bias (dbias, if asked, comes from k_dqb);
  // head dim 128: k_dkdv, walking the batch when dbias is asked
  const bool bloop = a.dbias != nullptr && p.Dqk != 64;
  const bool run_dq = p.Sq > 0 && p.B > 0, run_kv = p.Sk > 0 && p.B > 0;
  auto dq = [&](const ZeroMulti& zm, const PartialSum& ps) {
    return p.Dqk == 64 ? launch_dq<64>(p, a, zm, ps, st) : launch_dq<128>(p, a, zm, ps, st);
  };
  auto dkdv = [&](const DkdvPlan& pl) {
    return p.Dqk == 64 ? dispatch_dkdv<64>(p, a, pl, bias, bloop, st) : dispatch_dkdv<128>(p, a, pl, bias, bloop, st);
  };
  const bool vec_ok = aligned16(a.dk) && aligned16(a.dv) && p.dk_str[0] % 4 == 0 && p.dk_str[1] % 4 == 0 &&
                      p.dk_str[2] % 4 == 0 && p.dv_str[0] % 4 == 0 && p.dv_str[1] % 4 == 0 && p.dv_str[2] % 4 == 0;
  const bool partials_ok = !bias && vec_ok && partials_fit(p);
  DkdvPlan pl = plan_bwd(p, bloop, a.accumulate_dkdv != 0, a.deterministic != 0, partials_ok);
  if (pl.g.pt.nslot > 0 && run_kv) {
    if (a.workspace != nullptr && aligned16(a.workspace) && a.workspace_bytes >= partial_bytes(p, pl)) {
      pl.g.pt.base = (float*)a.workspace;
      PartialSum ps{pl.g.pt, a.dk, a.dv, {p.dk_str[0], p.dk_str[1], p.dk_str[2]},
                    {p.dv_str[0], p.dv_str[1], p.dv_str[2]}, p.B, p.Hk, p.Sk, p.Dqk, p.Dv};
      hipError_t e = dkdv(pl);
      if (e != hipSuccess) return e;
      if (run_dq) return dq(ZeroMulti{}, ps);
      hipLaunchKernelGGL(k_partial_sum, dim3(1024), dim3(256), 0, st, ps);
      return hipGetLastError();
    }
    // no (or too small a) workspace: the parts add atomically
    pl = plan_dkdv(p, bloop, a.accumulate_dkdv != 0, a.deterministic != 0, false);
  }
  const bool dq_first = run_dq && !bias && xmajor_fits(p, p.Hq, p.B);
  ZeroMulti zm{};
  if (pl.g.out_mode == kAtomicAdd && !a.accumulate_dkdv && p.Sk > 0) {
    // dense [B, Hk, Sk] or the packed rows of a variable-length batch
    const bool pk = p.cu_k != nullptr;
    const int zb = pk ? 1 : p.B, zs = pk ? (int)p.tot_k : p.Sk;
    ZeroRows z[2] = {ZeroRows{a.dk, zb, p.Hk, zs, p.Dqk, {pk ? 0 : p.dk_str[0], p.dk_str[1], p.dk_str[2]}},
                     ZeroRows{a.dv, zb, p.Hk, zs, p.Dv, {pk ? 0 : p.dv_str[0], p.dv_str[1], p.dv_str[2]}}};
    zm = make_zero_multi(z, 2);
    if (!dq_first && zm.n > 0) {
      hipError_t e = launch_zero_multi(z, 2, st);
      if (e != hipSuccess) return e;
    }
  }
  if (dq_first) {
    hipError_t e = dq(zm, PartialSum{});
    if (e != hipSuccess) return e;
  }
  if (run_kv) {
    hipError_t e = dkdv(pl);
    if (e != hipSuccess) return e;
  }
  if (run_dq && !dq_first) return dq(ZeroMulti{}, PartialSum{});
  return hipSuccess;
}

int64_t bwd_workspace_bytes(const Params& p, bool accumulate_dkdv, bool deterministic) {
  if (p.Sk <= 0 || p.B <= 0 || !partials_fit(p)) return 0;
  const DkdvPlan pl = plan_bwd(p, false, accumulate_dkdv, deterministic, true);
  return pl.g.pt.nslot > 0 ? partial_bytes(p, pl) : 0;
}

}  // namespace attn
