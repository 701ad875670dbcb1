// Tile machinery shared by the bf16 MFMA kernels of the forward and the
// backward (gfx950): direct global->LDS staging of 64-row tiles, the two LDS
// block layouts, and the two MFMA products every kernel is built from.
//
// v_mfma_f32_32x32x16_bf16 operand layouts (lane l, element e, register r):
//   A (32 x 16): lane l holds A[l % 32][8 (l / 32) + e]
//   B (16 x 32): lane l holds B[8 (l / 32) + e][l % 32]
//   C (32 x 32): lane l, register r holds C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
//
// "evidence" is a product C = X . Z^T with X read row-wise from an LDS tile
// (A operand) and the rows of Z held in registers (B operand): C[x][z] puts one
// z per lane (column l % 32) and 16 x values in registers.
// "transport" is O^T[d][z] += X^T[d][x] . W[x][z] with X^T read transposed from
// an LDS tile and W taken from the registers of an evidence tile C[x][z]
// (converted to bf16 pairs). The contraction index x is permuted the same way
// on both sides (the x order of the C layout), which the sum does not see.
#pragma once

#include <hip/hip_runtime.h>

namespace rel {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileRows = 64;               // rows per LDS tile
constexpr int kBufFlags = 0x00020000;       // raw buffer descriptor word 3 (gfx9)
constexpr int kOutOfRange = 0x7ffffff0;     // buffer offset past every head's range (reads 0)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS tiles are filled by direct global->LDS loads (buffer_load ... lds): one
// wave instruction writes 64 lanes x 16 bytes to 1 KB of consecutive LDS, so a
// tile is stored as blocks of 8 rows x 8 sixteen-byte chunks (8 x 128 bytes of
// global memory per instruction). The order inside a block and the block
// stride make every operand read a lane base plus an immediate and free of
// bank conflicts:
//   row layout (evidence reads): position rr + 8 cc (chunk-major), block
//             stride 1152 bytes, so the two 8-row blocks read by 16 lanes sit
//             128 bytes apart in the bank space;
//   transposed layout (transport reads): position 8 rr + (cc ^ 4 ((rr >> 1) & 1))
//             (row-major, chunk bit 2 flipped on every other row pair), block
//             stride 1024 bytes.
// Block k of a tile holds rows 8 (k % 8) .. +7 and chunks 8 (k / 8) .. +7.
template <int D>
struct TileLayout {
  static constexpr int kChunks = D / 8;              // 16-byte chunks per row
  static constexpr int kBlocks = kChunks;            // 8x8-chunk blocks per 64-row tile
  static constexpr int kKBlock = 1152;               // row-layout block stride
  static constexpr int kVBlock = 1024;               // transposed-layout block stride
  static constexpr int kKBytes = kBlocks * kKBlock;  // one row-layout tile
  static constexpr int kVBytes = kBlocks * kVBlock;  // one transposed-layout tile
  static constexpr int kDs = D / 16;                 // evidence MFMA k-steps
  static constexpr int kDb = D / 32;                 // 32-row blocks of O^T
  // Byte offset of evidence operand (32-row block kb, k-step ds) from the lane base.
  static constexpr int k_imm(int kb, int ds) { return 8 * kKBlock * (ds / 4) + 4 * kKBlock * kb + 256 * (ds % 4); }
  // Byte offset of the 8-row group `half` of transport operand (kb, ks, db).
  static constexpr int v_imm(int kb, int ks, int db, int half) {
    return kVBlock * (8 * (db >> 1) + 4 * kb + 2 * ks + half);
  }
  // Global byte offset (within a tile) that lane `lane` fetches for block k.
  __device__ static int row_src(int k, int lane) {
    return (8 * (k % 8) + (lane & 7)) * (D * 2) + 16 * (8 * (k / 8) + (lane >> 3));
  }
  __device__ static int tr_src(int k, int lane) {
    const int rr = lane >> 3;
    return (8 * (k % 8) + rr) * (D * 2) + 16 * (8 * (k / 8) + ((lane & 7) ^ (4 * ((rr >> 1) & 1))));
  }
  // The same for rows of DR <= D elements in memory (DR a multiple of 16):
  // chunks past the row's end get an offset past any buffer's range, so the
  // direct load writes zeros there.
  template <int DR>
  __device__ static int row_src_real(int k, int lane) {
    if constexpr (DR == D) return row_src(k, lane);
    const int cc = 8 * (k / 8) + (lane >> 3);
    return cc < DR / 8 ? (8 * (k % 8) + (lane & 7)) * (DR * 2) + 16 * cc : kOutOfRange;
  }
  template <int DR>
  __device__ static int tr_src_real(int k, int lane) {
    if constexpr (DR == D) return tr_src(k, lane);
    const int rr = lane >> 3;
    const int cc = 8 * (k / 8) + ((lane & 7) ^ (4 * ((rr >> 1) & 1)));
    return cc < DR / 8 ? (8 * (k % 8) + rr) * (DR * 2) + 16 * cc : kOutOfRange;
  }
  // Lane read base of the row layout: operand rows (lane % 32, chunk lane / 32).
  __device__ static int row_base(int lane) {
    const int lq = lane & 31, hf = lane >> 5;
    return kKBlock * (lq >> 3) + 16 * (lq & 7) + 128 * hf;
  }
  // Lane read bases of the transposed layout (16-lane group g supplies rows
  // 4 (g / 2) + i / 4 and columns 16 (g % 2) + 4 (i % 4) of each 16-row half,
  // i = lane % 16), for even and odd 32-row blocks db of O^T.
  __device__ static int tr_base(int lane, bool odd) {
    const int tg = lane >> 4, ti = lane & 15;
    const int vrr = 4 * (tg >> 1) + (ti >> 2), vcc = 2 * (tg & 1) + ((ti & 3) >> 1), vsw = (vrr >> 1) & 1;
    return 16 * (8 * vrr + 4 * (odd ? (vsw ^ 1) : vsw) + vcc) + 8 * (ti & 1);
  }
};

// Lane read bases of one transposed-layout tile: transport operands of even /
// odd 32-row O^T blocks (db) differ in the flipped chunk bit.
struct VBase {
  const char* even;
  const char* odd;
};

// s_waitcnt vmcnt(VM) lgkmcnt(LGKM), expcnt unconstrained (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int VM, int LGKM>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

// Raw buffer descriptor as four words (base, stride 0, num_records, flags) for
// use in inline assembly. Loads at offsets >= bytes return zeros.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, int bytes) {
  const unsigned long long a = (unsigned long long)base;
  return u32x4{(unsigned)a, (unsigned)(a >> 32) & 0xffffu, (unsigned)(bytes > 0 ? bytes : 0), (unsigned)kBufFlags};
}

// One direct global->LDS load: lane l's 16 bytes at voffset go to LDS byte
// address lds + 16 l (M0 holds lds). Written as inline assembly so that the
// compiler does not guard every later LDS read with a wait for all
// outstanding loads; kernels wait for them explicitly before the barrier
// that publishes the tile.
// The compiler's hazard checks do not look inside inline assembly: the
// descriptor SGPRs may have just been written by a VALU instruction (e.g.
// restored from spill lanes by v_readlane), and a VMEM instruction that
// reads a VALU-written SGPR needs 5 wait states on this architecture (an
// SALU write of M0 before an LDS-DMA needs 1); s_nop 4 provides them.
__device__ __forceinline__ void dma16(const u32x4& r, const char* lds, int voffset) {
  const unsigned m0 = (unsigned)(size_t)(const __attribute__((address_space(3))) char*)lds;
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voffset), "s"(r), "{m0}"(m0) : "memory");
}

// dma16 with the non-temporal hint, for data read exactly once.
__device__ __forceinline__ void dma16_nt(const u32x4& r, const char* lds, int voffset) {
  const unsigned m0 = (unsigned)(size_t)(const __attribute__((address_space(3))) char*)lds;
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" : : "v"(voffset), "s"(r), "{m0}"(m0) : "memory");
}

// Cache-policy operand of the buffer store builtins: non-temporal (gfx950).
constexpr int kCachePolicyNT = 2;

__device__ __forceinline__ float lane_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x4 lds_tr_read(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, long long bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufFlags);
}

// Two values as one packed bf16 pair (round to nearest even).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}

// Evidence of one 32-row block kb of a row-layout tile: C = X[kb] . Z^T with
// z[ds] the lane's B operands (row l % 32 of Z, columns 16 ds + 8 (l / 32) + e).
template <int D>
__device__ __forceinline__ f32x16 evidence_block(const char* kl, int kb, const bf16x8 (&z)[D / 16]) {
  using L = TileLayout<D>;
  f32x16 s;
#pragma unroll
  for (int ds = 0; ds < L::kDs; ++ds) {
    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + L::k_imm(kb, ds));
    if (ds == 0) {
      const f32x16 zero = {};
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, z[0], zero, 0, 0, 0);
    } else {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, z[ds], s, 0, 0, 0);
    }
  }
  return s;
}

// As evidence_block, with the accumulator starting at `init` instead of 0.
template <int D>
__device__ __forceinline__ f32x16 evidence_block_from(const char* kl, int kb, const bf16x8 (&z)[D / 16],
                                                      const f32x16& init) {
  using L = TileLayout<D>;
  f32x16 s = init;
#pragma unroll
  for (int ds = 0; ds < L::kDs; ++ds) {
    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + L::k_imm(kb, ds));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, z[ds], s, 0, 0, 0);
  }
  return s;
}

// Transposed operand of transport MFMA i = (block kb, k-step ks, O^T block db);
// the row order inside an MFMA k-step matches the register order of the
// evidence tile.
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const VBase& vb, int i) {
  using L = TileLayout<D>;
  const int kb = i / (2 * L::kDb), ks = (i / L::kDb) % 2, db = i % L::kDb;
  const char* p = (db & 1) ? vb.odd : vb.even;
  bf16x8 vf;
  vf.lo = lds_tr_read(p + L::v_imm(kb, ks, db, 0));
  vf.hi = lds_tr_read(p + L::v_imm(kb, ks, db, 1));
  return vf;
}

// Transport of one 32-row block kb: O^T[d][z] += X^T[d][x] W[x][z], W given as
// packed bf16 pairs pf[ks] (register r of the evidence tile -> operand r / 8,
// element r % 8).
template <int D>
__device__ __forceinline__ void transport_block(const VBase& vl, int kb, const u32x4 (&pf)[2],
                                                f32x16 (&o)[D / 32]) {
  using L = TileLayout<D>;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int db = 0; db < L::kDb; ++db) {
      const bf16x8 vf = v_operand<D>(vl, kb * 2 * L::kDb + ks * L::kDb + db);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, pf[ks]), o[db], 0, 0, 0);
    }
  }
}

}  // namespace mfma
}  // namespace rel
