// Host-side launch entry points of the attention kernels (internal to the
// library; the public ABI is include/attn_bwd.h).
#pragma once

#include "common.h"

namespace attn {

// Extra device pointers handed to the forward / backward kernels.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* bias;   // nullable [Hq, Sq, Sk]
  const float* sinks;  // nullable [Hq]
  void* o;
  float* lse;
  int xmajor;           // set by the launcher: walk row blocks heaviest first per XCD
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* delta;
  const float* bias;  // nullable
  float* dq;
  float* dk;
  float* dv;
  float* dbias;       // nullable
  int accumulate_dq;    // add into dq instead of overwriting
  int deterministic;
  int accumulate_dkdv;  // add into dk / dv instead of overwriting
  int xmajor;           // set by the launcher: walk row blocks heaviest first per XCD
  void* workspace;      // caller scratch for partial dK / dV sums (nullable)
  int64_t workspace_bytes;
};

// Whether the query-block kernels may walk each XCD's (head, batch) units
// row-block-major (heaviest blocks first): only when the K / V rows those
// units read at once fit well within the XCD's 4 MiB L2.
bool xmajor_fits(const Params& p, int ny, int nz);

// A strided [B, H, S, D] fp32 tensor (D contiguous) to be zeroed.
struct ZeroRows {
  float* p;
  int B, H, S, D;
  int64_t str[3];
};

// Query rows of a variable-length packed batch (cu == nullptr: dense):
// prefix sums of the sequences' rows along the s index and their count.
struct Packed {
  const int* cu;
  int64_t tot;
};

// delta = rowsum(dO * O); when dq_zero is non-null its rows are zeroed in the
// same pass.  Packed batch: delta rows past a sequence's length are 0.
hipError_t launch_delta(const void* o, int o_bf16, const void* dout, int do_bf16, float* delta, int B,
                        int H, int Sq, int Dv, const int64_t* os, const int64_t* ds, float* dq_zero,
                        int Dqk, const int64_t* dqs, Packed pk, hipStream_t st);
hipError_t launch_dsinks(const float* lse, const float* delta, const float* sinks, float* dsinks,
                         int B, int H, int Sq, Packed pk, hipStream_t st);
hipError_t launch_zero_rows(float* x, int B, int H, int S, int D, const int64_t* str, hipStream_t st);
// Partial dK / dV sums of split key-block units.  Part 0 of a unit writes
// dK / dV itself; part p >= 1 writes the slot partial_slot(kb, p) of its
// (batch entry, KV head): 128 keys x (Dqk + Dv) floats, the dK row of a key
// then its dV row.  Key block 0 has nparts0 parts, every other block nsplit.
struct Partials {
  float* base;   // nullptr: no partials (parts add atomically, or no split)
  int nslot;     // slots per (batch entry, KV head)
  int nparts0, nsplit;
};
__host__ __device__ inline int partial_slot(const Partials& pt, int kb, int part) {
  return (kb == 0 ? 0 : pt.nparts0 - 1 + (kb - 1) * (pt.nsplit - 1)) + part - 1;
}

// dK / dV of a dense [B, Hk, Sk, D] problem (strided rows) and the partials
// still to be added into them, in slot order.
struct PartialSum {
  Partials pt;
  float* dk;
  float* dv;
  int64_t dk_str[3], dv_str[3];
  int B, Hk, Sk, Dk, Dv;
};


// Up to three strided row tensors zeroed as one flat range: tensor k covers
// the elements [off[k], off[k + 1]), counted in 4-float groups where vec[k].
struct ZeroMulti {
  ZeroRows z[3];
  int64_t off[4];
  int vec[3];
  int dense[3];   // the tensor is one gap-free block from z.p (zeroed flat)
  int n;          // tensors (0: nothing to zero)
};
// The tensors z[0 .. n) with the empty ones dropped.
ZeroMulti make_zero_multi(const ZeroRows* z, int n);
// Zero up to three tensors in one launch (n == 0: nothing is launched).
hipError_t launch_zero_multi(const ZeroRows* z, int n, hipStream_t st);
hipError_t launch_zero_bias(float* x, int H, int Sq, int Sk, const int64_t* str, hipStream_t st);
hipError_t launch_lse_merge(int64_t rows, int Dv, float* o_acc, float* lse_acc, const float* o_part,
                            const float* lse_part, hipStream_t st);

// Plain fp32-arithmetic (no matrix cores) kernels: every dtype, head dims up
// to kSimtMaxD.  The fp32 path, and the forward for every dtype.
constexpr int kSimtMaxD = 128;
hipError_t launch_fwd_simt(const Params& p, const FwdArgs& a, int in_bf16, int o_bf16, hipStream_t st);
hipError_t launch_bwd_simt(const Params& p, const BwdArgs& a, int in_bf16, hipStream_t st);
// dQ alone (query-parallel, no atomics); ACCUMULATE adds into dq.
hipError_t launch_dq_simt(const Params& p, const BwdArgs& a, int in_bf16, hipStream_t st);

// bf16 matrix-core forward (gfx950 MFMA), head dims 64 and 128 (Dqk == Dv),
// 16-byte aligned operands; O in fp32 or bf16.
bool mfma_fwd_supported(const Params& p, const FwdArgs& a, bool o_bf16);
hipError_t launch_fwd_mfma(const Params& p, const FwdArgs& a, bool o_bf16, hipStream_t st);

// bf16 matrix-core backward (gfx950 MFMA), head dims 64 and 128.
bool mfma_bwd_supported(const Params& p);
hipError_t launch_bwd_mfma(const Params& p, const BwdArgs& a, hipStream_t st);
// Workspace bytes with which launch_bwd_mfma keeps split parts' partial
// sums (0: none used); host-only.
int64_t bwd_workspace_bytes(const Params& p, bool accumulate_dkdv, bool deterministic);

// bf16 matrix-core kernels for head dim 512 with one tensor as keys and
// values (k == v): forward, and the backward whose dk output is the gradient
// of the shared tensor (dK + dV).  Row strides multiples of 8 elements,
// 16-byte aligned operands.
constexpr int kSharedKvD = 512;
bool mla_supported(const Params& p);
hipError_t launch_fwd512(const Params& p, const FwdArgs& a, bool o_bf16, hipStream_t st);
hipError_t launch_bwd512(const Params& p, const BwdArgs& a, hipStream_t st);
// Workspace bytes with which launch_bwd512 keeps its head-split parts'
// partial sums (0: none used); host-only.
int64_t bwd512_workspace_bytes(const Params& p, bool deterministic, bool accumulate);

}  // namespace attn
