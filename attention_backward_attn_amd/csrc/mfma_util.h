// Matrix-core building blocks shared by the gfx950 MFMA kernels: the
// v_mfma_f32_32x32x16_bf16 wrapper, bf16 operand packing, and the padded LDS
// tile layouts with their plain and transposing operand reads.
//
// MFMA 32x32x16 bf16 operand layout (lane l, r = 0..15):
//   A[m][k]: lane holds m = l % 32, k = 8 (l / 32) + 0..7
//   B[k][n]: lane holds n = l % 32, k = 8 (l / 32) + 0..7
//   C[m][n]: lane holds n = l % 32, m = 8 (r / 4) + 4 (l / 32) + r % 4
#pragma once

#include "kernels.h"

namespace attn {
namespace mfma_util {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32: lane l holds A[l % 16][8 (l / 16) + 0..7], B[8 (l / 16) + 0..7][l % 16]
// and C[4 (l / 16) + 0..3][l % 16].
__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline bf16x8 cat44(u16x4 lo, u16x4 hi) {
  u16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return as_bf16x8(v);
}

// 8 fp32 accumulator values -> bf16x8 operand (round to nearest even).
__device__ inline bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
  return r;
}

// Wait for every outstanding vector-memory load (vmcnt = 0; expcnt and
// lgkmcnt left at their maxima).  Issued once after the register-resident
// fragments are loaded, ahead of a loop: otherwise the compiler's wait
// counting carries those loads into the loop body, and each use there waits
// for the vmcnt of older operations -- including the previous iteration's
// dQ atomics.
__device__ inline void wait_vm_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row (within a 32-row accumulator block) held by lane group lg in register r.
__device__ inline int crow(int r, int lg) { return 8 * (r >> 2) + 4 * lg + (r & 3); }

// Accumulating epilogue of N 32 x 32 accumulator blocks: acc[n][r] += the
// fp32 value at base[(row0 + crow(r, lg)) stride + 32 n + lr] for the rows
// below nrows, ahead of the stores.  The loads of a block are issued
// together; written as one load-add-store per element, every store must
// stay ahead of the next load (their addresses may alias), and each load's
// full memory latency is paid in turn.
template <int N>
__device__ inline void add_loaded(f32x16 (&acc)[N], const float* base, int64_t stride, int64_t row0,
                                  int64_t nrows, int lg, int lr) {
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t i = row0 + crow(r, lg);
      v[r] = i < nrows ? base[i * stride + 32 * n + lr] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] += v[r];
  }
}

// LDS layouts.  Every tile is row-major bf16 with a padded row stride, and
// each access pattern gets a copy whose padding makes it bank-conflict-free
// with per-lane addresses of the form  lane_base + compile-time offset:
//   * "row" copies, stride D + 8: 16 lanes read 16 bytes of the same columns
//     of 16 consecutive rows (A operands, ds_read_b128) -- consecutive rows
//     start 4 banks apart;
//   * "tr" copies, stride D + 32: 32 lanes read 4 consecutive rows x 64 bytes
//     with the transposing ds_read_b64_tr_b16 (B operands whose reduction
//     index is the tile row) -- consecutive rows start 16 banks apart.
template <int D>
struct Lay {
  static constexpr int R = D + 8;    // row-copy stride (elements)
  static constexpr int T = D + 32;   // tr-copy stride (elements)
};

__device__ inline bf16x8 lds_b128(const unsigned short* tile, int off) {
  return as_bf16x8(*(const u16x8*)(tile + off));
}

__device__ inline u16x4 lds_tr4(const unsigned short* tile, int off) {
  const auto* b = (__attribute__((address_space(3))) const unsigned short*)tile;
  return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + off)));
}

// Transposing-read lane base for a tile of stride `stride`: ds_read_b64_tr_b16
// hands lane j of each 16-lane group element j % 4 of the 8-byte chunk
// addressed by lane 4 r + j / 4 of that group.  Lane l therefore addresses
// row 4 (l / 32) + (l % 16) / 4, column 16 ((l / 16) % 2) + 4 (l % 4); the
// read at  base + r0 * stride + n0  (and + 8 rows) yields the B operand of a
// 32x32x16 MFMA whose reduction slots are tile rows
// r0 + {4 lg + 0..3, 8 + 4 lg + 0..3} -- the slot order of the S / dS
// accumulators -- and whose output column is n0 + l % 32.
__device__ inline int tr_base(int l, int stride) {
  const int j = l & 15;
  return (4 * (l >> 5) + (j >> 2)) * stride + 16 * ((l >> 4) & 1) + 4 * (j & 3);
}

__device__ inline bf16x8 lds_trB(const unsigned short* tile, int base, int r0, int n0, int stride) {
  return cat44(lds_tr4(tile, base + r0 * stride + n0), lds_tr4(tile, base + (r0 + 8) * stride + n0));
}

// The same LDS address passed through a register the compiler cannot see
// into: reads at  opaque(p) + constant  then keep one address register and
// fold the constant into the instruction's offset field, instead of one
// hoisted address register per constant.
__device__ inline const unsigned short* lds_opaque(const unsigned short* p) {
  const auto* p3 = (__attribute__((address_space(3))) const unsigned short*)p;
  unsigned int a = (unsigned int)(size_t)p3;
  asm volatile("" : "+v"(a));
  return (const unsigned short*)(__attribute__((address_space(3))) const unsigned short*)(size_t)a;
}

// Swizzled tile layout: rows of D bf16 with no padding, and the 16-byte
// chunk c of row r stored at chunk position c ^ swz(r).  For both operand
// read patterns -- one chunk of 16 consecutive rows (ds_read_b128) and four
// chunks of four consecutive rows (ds_read_b64_tr_b16) -- the units read
// together fall into distinct bank groups, so one copy of a tile serves both
// (measured on gfx950 at the speed of the best padded layout of each
// pattern).  For r0 a multiple of 8, swz(r0 + r) = swz(r) ^ ((r0 / 4) % 4),
// which keeps every operand address a lane base XOR a constant.
template <int D>
struct Swz {
  static constexpr int RB = 2 * D;   // row bytes
  static constexpr int CR = D / 8;   // 16-byte chunks per row
  __host__ __device__ static constexpr int f(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
  __host__ __device__ static constexpr int off(int r, int c) { return r * RB + ((c ^ f(r)) << 4); }
  // A-operand lane base: row l % 32, chunk l / 32 (k-step s reads base ^ 32 s)
  __device__ static int a_lane(int l) { return off(l & 31, l >> 5); }
  // transposing-read lane base (see tr_base): row 4 (l / 32) + (l % 16) / 4,
  // chunk 2 ((l / 16) % 2) + (l % 4) / 2, byte 8 (l % 2) of the chunk.
  // Rows r0..r0+3 (r0 a multiple of 8) of 32-column block n0 read at
  // (base ^ 16 K) + r0 RB with K = n0 / 8 ^ (r0 / 4) % 4.
  __device__ static int t_lane(int l) {
    const int r = 4 * (l >> 5) + ((l & 15) >> 2);
    return off(r, 2 * ((l >> 4) & 1) + ((l & 3) >> 1)) + 8 * (l & 1);
  }
};

typedef __attribute__((address_space(3))) u16x8 lds_u16x8;

__device__ inline bf16x8 lds_b128_at(unsigned int addr) {
  return as_bf16x8(*(const lds_u16x8*)(size_t)addr);
}

__device__ inline u16x4 lds_tr4_at(unsigned int addr) {
  return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)addr));
}

// Byte address of an LDS object, opaque to the compiler (see lds_opaque).
__device__ inline unsigned int lds_addr(const void* p) {
  unsigned int a = (unsigned int)(size_t)(const __attribute__((address_space(3))) char*)p;
  asm volatile("" : "+v"(a));
  return a;
}

// 16-byte (dwordx4) or 4-byte (dword) load from a buffer straight into LDS:
// lane l writes to lds + size * l (lds: wave-uniform byte address in M0).
// Issued as inline assembly, which the compiler does not count: the caller
// waits for completion (vmcnt) itself.  The compiler would otherwise make
// every transposing LDS read wait for all such loads in flight.
// The compiler's hazard checks do not look inside inline assembly, so the
// wait states that the hardware needs before a vector memory instruction
// reads an SGPR just written by a VALU instruction (5: the compiler may
// restore the resource from a VGPR lane with v_readlane right before) and
// before an LDS DMA reads M0 just written (1) are inserted here.
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t r, unsigned int lds, int voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(lds) : "memory");
}
__device__ inline void lds_dma4(__amdgpu_buffer_rsrc_t r, unsigned int lds, int voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(lds) : "memory");
}

// Wait until at most n vector-memory operations of this wave are in flight
// (vmcnt; expcnt and lgkmcnt left at their maxima).
__device__ inline void wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    case 15: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

// wait_vm with a compile-time count: one instruction, no branch.
template <int N>
__device__ inline void wait_vm_c() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
// wait_vm_c for counts up to 63 (the count's two high bits sit in bits 15:14
// of the s_waitcnt immediate).
template <int N>
__device__ inline void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Either N or 0 in flight, chosen at run time by `keep` (two fixed waits).
template <int N>
__device__ inline void wait_vm_keep(bool keep) {
  if (keep) wait_vm_c<N>();
  else wait_vm_c<0>();
}

// The hardware deals a launch's workgroups to the eight XCDs round-robin by
// linear workgroup id.  Renumbering them so that each XCD receives one
// contiguous range of logical ids (x fastest, then z, then y) keeps the
// workgroups of one head -- which share its K / V or Q / dO rows -- on one
// XCD and in its L2, while every XCD gets a share of every batch entry (or
// packed sequence, whose sizes may differ) so the XCDs stay balanced.
struct BlockXYZ {
  int x, y, z;
};

__device__ inline BlockXYZ xcd_block() {
  const int nx = gridDim.x, ny = gridDim.y, nz = gridDim.z;
  const int n = nx * ny * nz;
  const int id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const int q = n >> 3, r = n & 7, k = id & 7;
  const int L = k * q + min(k, r) + (id >> 3);
  const int zy = L / nx;
  return {L - zy * nx, zy / nz, zy % nz};
}

// As xcd_block, with the logical order batch (z) fastest, then x, then y:
// the batch entries of one (x, y) unit run side by side on one XCD, so
// tensors broadcast over the batch (a bias) are read from its L2 by all of
// them at about the same time.
__device__ inline BlockXYZ xcd_block_zfast() {
  const int nx = gridDim.x, ny = gridDim.y, nz = gridDim.z;
  const int n = nx * ny * nz;
  const int id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const int q = n >> 3, r = n & 7, k = id & 7;
  const int L = k * q + min(k, r) + (id >> 3);
  const int xy = L / nz;
  return {xy % nx, xy / nx, L - xy * nz};
}

// As xcd_block, for grids whose x index ranks the blocks by work (heaviest
// first): when the (y, z) units divide evenly over the XCDs, XCD k takes
// units [k U / 8, (k + 1) U / 8) (their K / V stay in its L2) and walks them
// x-major, so every XCD starts its heaviest blocks first.
__device__ inline BlockXYZ xcd_block_xmajor() {
  const int nx = gridDim.x, ny = gridDim.y, nz = gridDim.z;
  const int U = ny * nz;
  if (U % 8 != 0) return xcd_block();
  const int id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const int k = id & 7, i = id >> 3, per = U / 8;
  const int unit = k * per + i % per;
  return {i / per, unit / nz, unit % nz};
}

// Raw buffer resource over [base, base + bytes): a load at an offset past the
// end returns zero without touching memory, so ragged tiles need no clamping.
__device__ inline __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ inline u16x8 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ inline float buf_load_f32(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

}  // namespace mfma_util
// Thread t of nt zeroes the flat elements [e0, e1) of m (consecutive
// threads on consecutive elements).
__device__ inline void zero_multi_range(const ZeroMulti& m, int64_t e0, int64_t e1, int t, int nt) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (k >= m.n) break;
    const ZeroRows& z = m.z[k];
    const int64_t lo = e0 > m.off[k] ? e0 : m.off[k], hi = e1 < m.off[k + 1] ? e1 : m.off[k + 1];
    const int w = m.vec[k] ? z.D / 4 : z.D;
    if (m.dense[k]) {   // flat: no index arithmetic
      if (m.vec[k]) {
        float4* q = (float4*)z.p;
        for (int64_t e = lo + t; e < hi; e += nt) q[e - m.off[k]] = make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        for (int64_t e = lo + t; e < hi; e += nt) z.p[e - m.off[k]] = 0.f;
      }
      continue;
    }
    for (int64_t e = lo + t; e < hi; e += nt) {
      const int64_t x = e - m.off[k];
      const int d = (int)(x % w);
      const int64_t r = x / w;
      const int i = (int)(r % z.S);
      const int h = (int)((r / z.S) % z.H);
      const int b = (int)(r / ((int64_t)z.S * z.H));
      float* row = z.p + b * z.str[0] + h * z.str[1] + i * z.str[2];
      if (m.vec[k])
        *(float4*)(row + 4 * d) = make_float4(0.f, 0.f, 0.f, 0.f);
      else
        row[d] = 0.f;
    }
  }
}

}  // namespace attn
