// The 16-bit MFMA GEMM kernel (main loop and register epilogue), included by
// one translation unit per operand type.
#pragma once

#include "muon_gemm_common.h"

namespace muon {

// ---------------------------------------------------------------------------
// 16-bit MFMA kernel on packed operands.
//
// Block tile 256 (i) x BN (j) with BN = 256 or 128 (TileCfg below), 4 waves;
// wave w owns rows i0 + 64 w .. + 64 against all BN columns (2 x BN/32 MFMA
// 32x32x16 blocks, 2 BN accumulator registers).  k runs in slabs of 64 (4
// MFMA k-steps):
//  * the P rows of a wave are private to it, so its P fragments go straight
//    from global memory (L2) into registers with one contiguous 1 KB load per
//    fragment, three slabs ahead in four register slab buffers (BN = 256) or
//    one slab ahead in two (BN = 128, whose register budget is half);
//  * the Q tile is shared by all waves: it is streamed into a 4-stage LDS
//    ring with buffer_load ... lds (1 KB per instruction, lane l landing at
//    byte 16 l), three slabs ahead, and each fragment is read back with one
//    contiguous, conflict-free 16-byte-per-lane LDS read.
// One barrier per slab, half-way through the fourth k-step: by then every
// wave has read the whole slab into registers (the reads of the last k-step's
// fragments were issued a k-step earlier), so its stage can take the slab
// four ahead, and the MFMAs already issued keep the matrix pipe busy through
// the wait.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;
// The per-wave epilogue staging area, typed as LDS so its accesses are
// ds_read / ds_write rather than flat instructions.
typedef __attribute__((address_space(3))) float lds_f32;
__device__ __forceinline__ float4 lds_load4(const lds_f32* p) {
  const gf32x4_t v = *(const __attribute__((address_space(3))) gf32x4_t*)p;
  return make_float4(v.x, v.y, v.z, v.w);
}

template <int OP>
__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
  if constexpr (OP == kOpBF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

constexpr int kBM = kMfmaTile, kBK = 64;
constexpr int kNW = 4, kNT = 64 * kNW;
constexpr int kFM = kBM / kNW / 32;   // MFMA row blocks per wave (2)
constexpr int kKS = kBK / 16;         // k-steps per slab (4)
constexpr int kStages = 4;            // LDS ring depth for Q
constexpr int kLoadsA = kFM * kKS;    // P loads per wave and slab

// The block tile is 256 rows by BN columns.  BN = 256: one block per compute
// unit, 2 x 8 MFMA blocks (256 accumulator registers) per wave, P three slabs
// ahead in four register buffers.  BN = 128: two blocks per compute unit (two
// waves per SIMD, so one wave's waits and barrier are covered by the other's
// MFMAs), 2 x 4 MFMA blocks (128 accumulator registers) per wave, P two slabs
// ahead in three buffers; used for symmetric products with k = n (short), where
// the finer tiles also fill the last round better, and for the last product
// (k = n), where one block's update of W overlaps the other block's MFMAs.
template <int BN>
struct TileCfg {
  static constexpr int kFN = BN / 32;          // MFMA column blocks per wave
  static constexpr int kRBW = BN / 32 / kNW;   // Q row blocks each wave streams in per slab
  static constexpr int kLoadsB = kRBW * kKS;   // Q loads per wave and slab
  static constexpr int kStageBytes = BN * kBK * 2;
  // a stage also holds one wave's 32-row staging block of the last product (rows of BN + 4 floats)
  static constexpr int kStageAlloc = kStageBytes < 32 * (BN + 4) * 4 ? 32 * (BN + 4) * 4 : kStageBytes;
  static constexpr int kPBufs = BN == 256 ? 4 : 3;
  // Loads a wave issues after its part of Q slab kt + 1 and before the
  // barrier of slab kt: three P slab groups (issued at the starts of slabs
  // kt - 2 .. kt: slabs kt + 1 .. kt + 3 with P three slabs ahead, kt .. kt + 2
  // with P two ahead) and Q slabs kt + 2, kt + 3.
  static constexpr int kWaitBarrier = 3 * kLoadsA + 2 * kLoadsB;
};

// s_waitcnt immediate for gfx9: vmcnt in bits [3:0] and [15:14], expcnt [6:4]
// (7 = no wait), lgkmcnt [11:8] (15 = no wait).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (((vm >> 4) & 3) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// A buffer resource for `bytes` bytes at `base` (a block-uniform address;
// readfirstlane states that to the compiler, so the descriptor stays in
// scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes);
  const uint64_t u = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u & 0xffffffffu)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u >> 32)));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), static_cast<short>(0),
                                           __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// The P fragments of slab kt for this wave: kFM row blocks x kKS k-steps.
__device__ __forceinline__ void load_a_slab(uint4 (&buf)[kFM][kKS], __amdgpu_buffer_rsrc_t r, int voff,
                                            int sbase, int rb_stride, int kt) {
#pragma unroll
  for (int f = 0; f < kFM; ++f)
#pragma unroll
    for (int s = 0; s < kKS; ++s)
      buf[f][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
          r, voff, __builtin_amdgcn_readfirstlane(sbase + f * rb_stride + kt * 4096 + s * 1024), 0));
}

// The P fragments of k-step s of slab kt for this wave (kFM loads).
__device__ __forceinline__ void load_a_part(uint4 (&buf)[kFM][kKS], __amdgpu_buffer_rsrc_t r, int voff, int sbase,
                                            int rb_stride, int kt, int s) {
#pragma unroll
  for (int f = 0; f < kFM; ++f)
    buf[f][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
        r, voff, __builtin_amdgcn_readfirstlane(sbase + f * rb_stride + kt * 4096 + s * 1024), 0));
}

// The Q slab kt into LDS stage `stage`: this wave's row blocks x 4 fragments.
template <int BN>
__device__ __forceinline__ void load_b_slab(uint4* stage, __amdgpu_buffer_rsrc_t r, int voff, int sbase,
                                            int rb_stride, int kt, int wave) {
  constexpr int RBW = TileCfg<BN>::kRBW;
#pragma unroll
  for (int f = 0; f < RBW; ++f) {
    const int rb = wave * RBW + f;
    // the 4 fragments of a row block are 1 KB apart both in memory and in
    // the stage, so they share the LDS base (M0) and the scalar offset and
    // differ only in the immediate offset, which applies to both addresses
    lds_ptr_t dst = (lds_ptr_t)(stage + rb * kKS * 64);
    const int so = __builtin_amdgcn_readfirstlane(sbase + rb * rb_stride + kt * 4096);
    static_assert(kKS == 4, "four fragments per row block and slab");
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, so, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, so, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, so, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, so, 3072, 0);
  }
}

// MFMAs of one k-step with the Q fragments of the next k-step read in between.
template <int OP, int FN>
__device__ __forceinline__ void kstep(f32x16_t (&acc)[kFM][FN], const uint4 (&a)[kFM][kKS], int s,
                                      const uint4 (&bcur)[FN], uint4 (&bnext)[FN], const uint4* next_frags,
                                      bool read_next, int lane) {
  if (read_next) {
#pragma unroll
    for (int y = 0; y < FN; ++y) bnext[y] = next_frags[y * kKS * 64 + lane];
  }
#pragma unroll
  for (int y = 0; y < FN; ++y)
#pragma unroll
    for (int x = 0; x < kFM; ++x) acc[x][y] = mfma32<OP>(a[x][s], bcur[y], acc[x][y]);
  if (read_next) {
#pragma unroll
    for (int g = 0; g < FN; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
    }
  }
}

// Half a k-step: the MFMAs of columns Y0 .. Y0 + 3 with the reads of the
// next k-step's fragments Y0 .. Y0 + 3 in between.
template <int OP, int FN, int Y0>
__device__ __forceinline__ void kstep_half(f32x16_t (&acc)[kFM][FN], const uint4 (&a)[kFM][kKS], int s,
                                           const uint4 (&bcur)[FN], uint4 (&bnext)[FN], const uint4* next_frags,
                                           int lane) {
#pragma unroll
  for (int y = Y0; y < Y0 + FN / 2; ++y) bnext[y] = next_frags[y * kKS * 64 + lane];
#pragma unroll
  for (int y = Y0; y < Y0 + FN / 2; ++y)
#pragma unroll
    for (int x = 0; x < kFM; ++x) acc[x][y] = mfma32<OP>(a[x][s], bcur[y], acc[x][y]);
#pragma unroll
  for (int g = 0; g < FN / 2; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
  }
}

// One slab: k-steps 0..3 of slab kt from registers `a` and LDS stage `cur`,
// reading ahead into bf; the barrier and the ring refill (slab kt + 4 into
// `cur`) sit half-way through k-step 3.  Loads are issued unconditionally, also past
// the last slab: buffer loads are range-checked against the descriptor and
// the data is never used, and straight-line code lets the compiler count
// outstanding loads exactly.
template <int OP, int BN>
__device__ __forceinline__ void slab(f32x16_t (&acc)[kFM][TileCfg<BN>::kFN], const uint4 (&a)[kFM][kKS],
                                     uint4 (&bf)[2][TileCfg<BN>::kFN], uint4* cur, const uint4* nxt,
                                     __amdgpu_buffer_rsrc_t rQ, int voff, int sQ, int qstride, int kt, int wave,
                                     int lane) {
  constexpr int kFN = TileCfg<BN>::kFN;
  kstep<OP, kFN>(acc, a, 0, bf[0], bf[1], cur + 1 * 64, true, lane);
  kstep<OP, kFN>(acc, a, 1, bf[1], bf[0], cur + 2 * 64, true, lane);
  kstep<OP, kFN>(acc, a, 2, bf[0], bf[1], cur + 3 * 64, true, lane);
  kstep_half<OP, kFN, 0>(acc, a, 3, bf[1], bf[0], nxt, lane);
  // This wave's reads of slab kt (all older than the 4 reads of `nxt` just
  // issued) have landed and its part of slab kt + 1 is in LDS (the 5 load
  // groups issued after it may still be in flight); after the barrier the
  // whole slab kt + 1 is visible and nobody reads `cur`.
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(TileCfg<BN>::kWaitBarrier, kFN / 2));
  block_barrier();
  __builtin_amdgcn_sched_barrier(0);
  load_b_slab<BN>(cur, rQ, voff, sQ, qstride, kt + kStages, wave);
  kstep_half<OP, kFN, kFN / 2>(acc, a, 3, bf[1], bf[0], nxt, lane);
}

// slab() with the P fragments of slab ktp loaded into `anext` a k-step at a
// time (all before the barrier, so the barrier's count is unchanged).
template <int OP, int BN>
__device__ __forceinline__ void slab_spread(f32x16_t (&acc)[kFM][TileCfg<BN>::kFN], const uint4 (&a)[kFM][kKS],
                                            uint4 (&bf)[2][TileCfg<BN>::kFN], uint4* cur, const uint4* nxt,
                                            uint4 (&anext)[kFM][kKS], __amdgpu_buffer_rsrc_t rP, int sP, int pstride,
                                            int ktp, __amdgpu_buffer_rsrc_t rQ, int voff, int sQ, int qstride, int kt,
                                            int wave, int lane) {
  constexpr int kFN = TileCfg<BN>::kFN;
  load_a_part(anext, rP, voff, sP, pstride, ktp, 0);
  kstep<OP, kFN>(acc, a, 0, bf[0], bf[1], cur + 1 * 64, true, lane);
  load_a_part(anext, rP, voff, sP, pstride, ktp, 1);
  kstep<OP, kFN>(acc, a, 1, bf[1], bf[0], cur + 2 * 64, true, lane);
  load_a_part(anext, rP, voff, sP, pstride, ktp, 2);
  kstep<OP, kFN>(acc, a, 2, bf[0], bf[1], cur + 3 * 64, true, lane);
  load_a_part(anext, rP, voff, sP, pstride, ktp, 3);
  kstep_half<OP, kFN, 0>(acc, a, 3, bf[1], bf[0], nxt, lane);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(TileCfg<BN>::kWaitBarrier, kFN / 2));
  block_barrier();
  __builtin_amdgcn_sched_barrier(0);
  load_b_slab<BN>(cur, rQ, voff, sQ, qstride, kt + kStages, wave);
  kstep_half<OP, kFN, kFN / 2>(acc, a, 3, bf[1], bf[0], nxt, lane);
}

// ---------------------------------------------------------------------------
// Register epilogue of the MFMA kernel.
//
// For the 32 x 32 MFMA block at rows ib.., columns jb.. a lane holds 16
// values in the accumulator arrangement "A": lane l, register r is element
//   (ib + 8 (r / 4) + 4 (l / 32) + r % 4,  jb + l % 32).
// Exchanging registers 4..7 of the lower half-wave with registers 0..3 of the
// upper half-wave (and 12..15 with 8..11) by v_permlane32_swap gives "N":
// lane l, register 8 h + e is (ib + 16 h + 8 (l / 32) + e, jb + l % 32), so a
// lane holds 8 consecutive rows of one column: in the packed operand layout
// that is this lane's 16 bytes of a fragment of C^T (row j, k = i).  Using
// such a fragment as the MFMA A operand against an identity B fragment gives
// the block transposed, exactly (products with 1 and sums with 0), in
// arrangement "T": lane l, register 8 h + e is (ib + l % 32, jb + 16 h +
// 8 (l / 32) + e), a fragment of C itself (row i, k = j).  Both C and C^T are
// thus written as whole 1 KB fragments from registers, and the 16-bit
// epilogue input is read as fragments of E^T (E is symmetric, or E = X read
// from X^T).
//
// Exchange the upper half-wave of x with the lower half-wave of y.
__device__ __forceinline__ void xchg_halves(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}

template <int OP>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return OP == kOpBF16 ? f32x2_to_bf16x2(lo, hi) : f32x2_to_f16x2(lo, hi);
}

// 16 values in arrangement A -> two 16-bit fragments in arrangement N.
template <int OP>
__device__ __forceinline__ void a_to_n16(const float (&v)[16], uint4 (&f)[2]) {
  uint32_t d[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) d[k] = pack2<OP>(v[2 * k], v[2 * k + 1]);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    xchg_halves(d[4 * h], d[4 * h + 2]);
    xchg_halves(d[4 * h + 1], d[4 * h + 3]);
  }
  f[0] = make_uint4(d[0], d[1], d[2], d[3]);
  f[1] = make_uint4(d[4], d[5], d[6], d[7]);
}

// Two 16-bit fragments in arrangement N -> 16 fp32 values in arrangement A.
template <int OP>
__device__ __forceinline__ void n16_to_a(const uint4& f0, const uint4& f1, float (&v)[16]) {
  uint32_t d[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    xchg_halves(d[4 * h], d[4 * h + 2]);
    xchg_halves(d[4 * h + 1], d[4 * h + 3]);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    v[2 * k] = OpT<OP>::to_f(static_cast<uint16_t>(d[k] & 0xffffu));
    v[2 * k + 1] = OpT<OP>::to_f(static_cast<uint16_t>(d[k] >> 16));
  }
}

// B fragment h of the 32 x 32 identity: lane l holds B[k][n] for n = l % 32,
// k = 8 (l / 32) + e, equal to 1 where n == 16 h + k.
template <int OP>
__device__ __forceinline__ uint4 ident_frag(int h, int lane) {
  const uint32_t one = OP == kOpBF16 ? 0x3F80u : 0x3C00u;
  const int e = (lane & 31) - 16 * h - 8 * (lane >> 5);
  uint32_t d[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) d[k] = (e >= 0 && (e >> 1) == k) ? one << (16 * (e & 1)) : 0u;
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// Fragments in arrangement N -> the transposed block in arrangement T.
template <int OP>
__device__ __forceinline__ void transpose16(const uint4 (&n)[2], const uint4 (&id)[2], uint4 (&t)[2]) {
  f32x16_t d;
#pragma unroll
  for (int r = 0; r < 16; ++r) d[r] = 0.0f;
  d = mfma32<OP>(n[0], id[0], d);
  d = mfma32<OP>(n[1], id[1], d);
  float dv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) dv[r] = d[r];
  a_to_n16<OP>(dv, t);
}

// Diagonal block of a symmetric product: N and T fragments address the same
// elements (p, q) = (l % 32, 16 h + 8 (l / 32) + e); keep the owned value
// C[max][min], which is T where p >= q and N elsewhere.
__device__ __forceinline__ uint4 sym_select(const uint4& t, const uint4& n, int h, int lane) {
  const int p = lane & 31, q0 = 16 * h + 8 * (lane >> 5);
  const uint32_t tv[4] = {t.x, t.y, t.z, t.w}, nv[4] = {n.x, n.y, n.z, n.w};
  uint32_t r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t m = (p >= q0 + 2 * k ? 0x0000ffffu : 0u) | (p >= q0 + 2 * k + 1 ? 0xffff0000u : 0u);
    r[k] = (tv[k] & m) | (nv[k] & ~m);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

template <int OP>
__device__ __forceinline__ void store_frag(void* base, int64_t off, int lane, const uint4& f) {
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off + 8 * lane) = f;
}

// Four consecutive user elements of dtype D (kF32 or kBF16) at byte offset
// off of p, aligned to four elements.
template <int D>
__device__ __forceinline__ float4 ld4(void* p, int64_t off) {
  return D == kF32 ? gload_f32x4(p, off) : gload_bf16x4(p, off);
}
template <int D>
__device__ __forceinline__ void st4(void* p, int64_t off, const float4& v) {
  if constexpr (D == kF32) {
    gstore_f32x4(p, off, v);
  } else {
    gstore_bf16x4(p, off, v);
  }
}

// The final update for a staged 32 x BW block of O (BW = 256 or 128) that
// lies wholly inside the user's matrix, whose rows are aligned to four
// elements: W of dtype WD and O of dtype OD (-1: absent).  Loads of W for R
// rows (or columns) are issued together; there are no per-element range
// checks.
template <int WD, int OD, int LDE, int BW>
__device__ __forceinline__ void final_rows_fast(const GemmArgs& a, const EpiState& st, const lds_f32* ep, int i0, int j0,
                                                int lane) {
  constexpr int R = BW == 256 ? 16 : 8;
  constexpr int LPR = BW / 4, RS = 64 / LPR;  // lanes per row of the block, rows per step
  constexpr int wsz = WD == kF32 ? 4 : 2, osz = OD == kF32 ? 4 : 2;
  void* w = st.w;
  void* o = st.o;
  const int64_t ld = a.user_ld;
  const float lr = a.lr, wd = a.wd, os = a.oscale;
  auto update = [&](float4& nw, const float4& ov) {
    nw.x -= lr * (os * ov.x + wd * nw.x);
    nw.y -= lr * (os * ov.y + wd * nw.y);
    nw.z -= lr * (os * ov.z + wd * nw.z);
    nw.w -= lr * (os * ov.w + wd * nw.w);
  };
  if (!a.transposed) {  // W[i][j .. j + 3], lane -> columns j0 + 4 (lane % LPR) of rows RS r + lane / LPR
    const int sub = lane / LPR, cl = 4 * (lane % LPR);
    const int64_t base = static_cast<int64_t>(i0 + sub) * ld + j0 + cl;
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += R * RS) {
      float4 wv[R];
      if constexpr (WD >= 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) wv[r] = ld4<WD>(w, (base + (r0 + RS * r) * ld) * wsz);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float4 ov = lds_load4(ep + (r0 + RS * r + sub) * LDE + cl);
        if constexpr (OD >= 0) st4<OD>(o, (base + (r0 + RS * r) * ld) * osz, ov);
        if constexpr (WD >= 0) {
          update(wv[r], ov);
          st4<WD>(w, (base + (r0 + RS * r) * ld) * wsz, wv[r]);
        }
      }
    }
  } else {  // W[j][i .. i + 3], lane -> rows i0 + r4 .. + 3 of columns j0 + c
    const int r4 = (lane & 7) * 4;
    const int64_t base = static_cast<int64_t>(j0 + (lane >> 3)) * ld + i0 + r4;
#pragma unroll
    for (int c0 = 0; c0 < BW; c0 += 8 * R) {
      float4 wv[R];
      if constexpr (WD >= 0) {
#pragma unroll
        for (int t = 0; t < R; ++t) wv[t] = ld4<WD>(w, (base + (c0 + 8 * t) * ld) * wsz);
      }
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const int c = c0 + 8 * t + (lane >> 3);
        const float4 ov = make_float4(ep[(r4 + 0) * LDE + c], ep[(r4 + 1) * LDE + c], ep[(r4 + 2) * LDE + c],
                                      ep[(r4 + 3) * LDE + c]);
        if constexpr (OD >= 0) st4<OD>(o, (base + (c0 + 8 * t) * ld) * osz, ov);
        if constexpr (WD >= 0) {
          update(wv[t], ov);
          st4<WD>(w, (base + (c0 + 8 * t) * ld) * wsz, wv[t]);
        }
      }
    }
  }
}

// Whether final_rows_fast may take this 32 x BW block: inside the matrix and
// with rows of W and O aligned to four elements.
template <int BW>
__device__ __forceinline__ bool final_fast_ok(const GemmArgs& a, const EpiState& st, int i0, int j0) {
  if (i0 + 32 > a.n_real || j0 + BW > a.m_real || (a.user_ld & 3) != 0) return false;
  const uintptr_t wal = a.w_dtype == kF32 ? 15 : 7, oal = a.o_dtype == kF32 ? 15 : 7;
  return (reinterpret_cast<uintptr_t>(st.w) & wal) == 0 && (reinterpret_cast<uintptr_t>(st.o) & oal) == 0;
}

template <int LDE, int BW>
__device__ __forceinline__ void final_rows_any(const GemmArgs& a, const EpiState& st, const lds_f32* ep, int i0, int j0,
                                               int lane);

// The update of one staged 32 x BW block: the fast form for the dtype pair,
// or the general one (ragged edges, unaligned rows).
template <int LDE, int BW>
__device__ __forceinline__ void final_block(const GemmArgs& a, const EpiState& st, const lds_f32* ep, int i0, int j0,
                                            int lane) {
  if (final_fast_ok<BW>(a, st, i0, j0)) {
    const int wdt = st.w != nullptr ? a.w_dtype : -1, odt = st.o != nullptr ? a.o_dtype : -1;
#define MUON_FAST(WD, OD)                                               \
  if (wdt == WD && odt == OD) {                                         \
    final_rows_fast<WD, OD, LDE, BW>(a, st, ep, i0, j0, lane);          \
    return;                                                             \
  }
    MUON_FAST(kF32, -1) MUON_FAST(kBF16, -1) MUON_FAST(-1, kF32) MUON_FAST(-1, kBF16)
    MUON_FAST(kF32, kF32) MUON_FAST(kF32, kBF16) MUON_FAST(kBF16, kF32) MUON_FAST(kBF16, kBF16)
#undef MUON_FAST
  }
  final_rows_any<LDE, BW>(a, st, ep, i0, j0, lane);
}

// The fast update of a staged 32 x 128 block split in two, so that the loads
// of W can go out before O is staged: final_load_w128 issues the 16
// four-element loads of W that final_rows_fast<WD, OD, LDE, 128> makes for
// this lane (rows 2 r + lane / 32, or columns 8 r + lane / 8, r < 16), and
// final_apply128 then updates and stores them with the staged O (and stores
// O itself when OD >= 0), element for element as final_rows_fast does.
template <int WD>
__device__ __forceinline__ void final_load_w128(const GemmArgs& a, const EpiState& st, int i0, int j0, int lane,
                                                float4 (&wv)[16]) {
  constexpr int wsz = WD == kF32 ? 4 : 2;
  const int64_t ld = a.user_ld;
  if (!a.transposed) {
    const int64_t base = static_cast<int64_t>(i0 + (lane >> 5)) * ld + j0 + 4 * (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[r] = ld4<WD>(st.w, (base + 2 * r * ld) * wsz);
  } else {
    const int64_t base = static_cast<int64_t>(j0 + (lane >> 3)) * ld + i0 + (lane & 7) * 4;
#pragma unroll
    for (int t = 0; t < 16; ++t) wv[t] = ld4<WD>(st.w, (base + 8 * t * ld) * wsz);
  }
}

template <int WD, int OD, int LDE>
__device__ __forceinline__ void final_apply128(const GemmArgs& a, const EpiState& st, const lds_f32* ep, int i0, int j0,
                                               int lane, float4 (&wv)[16]) {
  constexpr int wsz = WD == kF32 ? 4 : 2, osz = OD == kF32 ? 4 : 2;
  const int64_t ld = a.user_ld;
  const float lr = a.lr, wd = a.wd, os = a.oscale;
  auto update = [&](float4& nw, const float4& ov) {
    nw.x -= lr * (os * ov.x + wd * nw.x);
    nw.y -= lr * (os * ov.y + wd * nw.y);
    nw.z -= lr * (os * ov.z + wd * nw.z);
    nw.w -= lr * (os * ov.w + wd * nw.w);
  };
  if (!a.transposed) {
    const int sub = lane >> 5, cl = 4 * (lane & 31);
    const int64_t base = static_cast<int64_t>(i0 + sub) * ld + j0 + cl;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float4 ov = lds_load4(ep + (2 * r + sub) * LDE + cl);
      if constexpr (OD >= 0) st4<OD>(st.o, (base + 2 * r * ld) * osz, ov);
      update(wv[r], ov);
      st4<WD>(st.w, (base + 2 * r * ld) * wsz, wv[r]);
    }
  } else {
    const int r4 = (lane & 7) * 4;
    const int64_t base = static_cast<int64_t>(j0 + (lane >> 3)) * ld + i0 + r4;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int c = 8 * t + (lane >> 3);
      const float4 ov = make_float4(ep[(r4 + 0) * LDE + c], ep[(r4 + 1) * LDE + c], ep[(r4 + 2) * LDE + c],
                                    ep[(r4 + 3) * LDE + c]);
      if constexpr (OD >= 0) st4<OD>(st.o, (base + 8 * t * ld) * osz, ov);
      update(wv[t], ov);
      st4<WD>(st.w, (base + 8 * t * ld) * wsz, wv[t]);
    }
  }
}

// Final product, general form (ragged edges, unaligned rows): W <- W -
// lr (O + wd W) and the optional store of O, for rows i0 .. i0 + 31 and
// columns j0 .. j0 + BW - 1 of O staged in LDS (row-major, LDE floats per
// row), with per-element range checks.
template <int LDE, int BW>
__device__ __forceinline__ void final_rows_any(const GemmArgs& a, const EpiState& st, const lds_f32* ep, int i0, int j0,
                                               int lane) {
  constexpr int R = BW == 256 ? 16 : 8;
  constexpr int LPR = BW / 4, RS = 64 / LPR;  // lanes per row of the block, rows per step
  if (!a.transposed) {  // W is n x m: lane -> columns j .. j + 3 of rows RS r + lane / LPR
    const int sub = lane / LPR, cl = 4 * (lane % LPR);
    const int j = j0 + cl;
    const int valid = a.m_real - j;
    for (int r0 = 0; r0 < 32; r0 += R * RS) {
      float4 w[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int i = i0 + r0 + RS * r + sub;
        w[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (st.w != nullptr && i < a.n_real && valid > 0)
          w[r] = user_load4(st.w, static_cast<int64_t>(i) * a.user_ld + j, a.w_dtype, valid);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int i = i0 + r0 + RS * r + sub;
        if (i < a.n_real)
          final_update4(a, st, static_cast<int64_t>(i) * a.user_ld + j, valid,
                        lds_load4(ep + (r0 + RS * r + sub) * LDE + cl), w[r]);
      }
    }
  } else {  // W is m x n: lane -> W[j][i .. i + 3] for 32 columns j of O
    const int r4 = (lane & 7) * 4;
    const int i = i0 + r4;
    const int valid = a.n_real - i;
    for (int c0 = 0; c0 < BW; c0 += 8 * R) {
      float4 w[R];
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const int j = j0 + c0 + 8 * t + (lane >> 3);
        w[t] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (st.w != nullptr && j < a.m_real && valid > 0)
          w[t] = user_load4(st.w, static_cast<int64_t>(j) * a.user_ld + i, a.w_dtype, valid);
      }
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const int c = c0 + 8 * t + (lane >> 3);
        if (j0 + c < a.m_real) {
          const float4 o = make_float4(ep[(r4 + 0) * LDE + c], ep[(r4 + 1) * LDE + c], ep[(r4 + 2) * LDE + c],
                                       ep[(r4 + 3) * LDE + c]);
          final_update4(a, st, static_cast<int64_t>(j0 + c) * a.user_ld + i, valid, o, w[t]);
        }
      }
    }
  }
}

struct EpiSpec {
  bool sym, fin, q;
  bool e;  // an epilogue input E, read as 16-bit fragments of E^T
};

constexpr EpiSpec epi_spec(int k) {
  return k == kEpiSym       ? EpiSpec{true, false, false, false}
         : k == kEpiSymE16  ? EpiSpec{true, false, false, true}
         : k == kEpiSymE16Q ? EpiSpec{true, false, true, true}
         : k == kEpiGen     ? EpiSpec{false, false, false, false}
         : k == kEpiGenE16  ? EpiSpec{false, false, false, true}
         : k == kEpiFin     ? EpiSpec{false, true, false, false}
                            : EpiSpec{false, true, false, true};
}

// This wave's output and input addresses, in elements, at MFMA block (0, 0)
// of its 64 x BN sub-tile (rows ib0 = 256 I + 64 w, columns jb0 = BN J).
// In the packed layout the fragments of block (x, y), half h, sit at
//   T (rows i, k = j):  t16 + x rs_t + 2048 (y / 2) + 512 (2 (y % 2) + h)
//   N (rows j, k = i):  n16 + y rs_n + 512 (2 x + h)
// and the fragments of E^T for block (x, y) at e16 + y rs_e16 + 512 (2 x + h).
struct EpiPtrs {
  uint16_t *t16, *n16, *tq, *nq;
  const uint16_t* e16;
  int64_t rs_t, rs_n, rs_e16;
};

template <int KIND, int BN>
__device__ __forceinline__ EpiPtrs epi_ptrs(const GemmArgs& a, int b, int I, int J, int wave) {
  constexpr EpiSpec S = epi_spec(KIND);
  EpiPtrs p{};
  const int64_t ib5 = (I * kBM + wave * (kBM / kNW)) >> 5, ib6 = ib5 >> 1;
  const int64_t jb5 = (J * BN) >> 5, jb6 = jb5 >> 1;
  const int64_t bO = static_cast<int64_t>(b) * a.sO;
  if constexpr (!S.fin) {
    uint16_t* o16 = static_cast<uint16_t*>(a.out16) + bO;
    p.rs_t = static_cast<int64_t>(a.ldo >> 6) * 2048;
    p.t16 = o16 + (ib5 * (a.ldo >> 6) + jb6) * 2048;
    if constexpr (S.sym) {
      p.rs_n = p.rs_t;
      p.n16 = o16 + (jb5 * (a.ldo >> 6) + ib6) * 2048;
    } else {
      uint16_t* oT = static_cast<uint16_t*>(a.outT16) + static_cast<int64_t>(b) * a.sOT;
      p.rs_n = static_cast<int64_t>(a.ldot >> 6) * 2048;
      p.n16 = oT + (jb5 * (a.ldot >> 6) + ib6) * 2048;
    }
    if constexpr (S.q) {
      uint16_t* q16 = static_cast<uint16_t*>(a.q16) + bO;
      p.tq = q16 + (ib5 * (a.ldo >> 6) + jb6) * 2048;
      p.nq = q16 + (jb5 * (a.ldo >> 6) + ib6) * 2048;
    }
  }
  if constexpr (S.e) {
    p.rs_e16 = static_cast<int64_t>(a.lde >> 6) * 2048;
    p.e16 = static_cast<const uint16_t*>(a.E16) + static_cast<int64_t>(b) * a.sE + (jb5 * (a.lde >> 6) + ib6) * 2048;
  }
  return p;
}

// The epilogue input of block (x, y): its two 16-bit fragments of E^T.
template <int KIND>
__device__ __forceinline__ void load_ein(const EpiPtrs& p, int x, int y, int lane, uint4 (&ein)[2]) {
  if constexpr (epi_spec(KIND).e) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      ein[h] = *reinterpret_cast<const uint4*>(p.e16 + y * p.rs_e16 + 512 * (2 * x + h) + 8 * lane);
  }
}

// Both 16-bit copies of one block: T at (i, j) and N at (j, i) (symmetric),
// or X and X^T (general).  On a diagonal block the two address the same
// elements and both get the owned values.
template <int OP, bool SYMDIAG>
__device__ __forceinline__ void store_tn(uint16_t* t, uint16_t* n, const float (&v)[16], int lane, const uint4 (&id)[2],
                                         bool dblk) {
  uint4 n16[2], t16[2];
  a_to_n16<OP>(v, n16);
  transpose16<OP>(n16, id, t16);
  if constexpr (SYMDIAG) {
    if (dblk) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        t16[h] = sym_select(t16[h], n16[h], h, lane);
        n16[h] = t16[h];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    *reinterpret_cast<uint4*>(t + 512 * h + 8 * lane) = t16[h];
    *reinterpret_cast<uint4*>(n + 512 * h + 8 * lane) = n16[h];
  }
}

// Epilogue of MFMA block (x, y) of the wave (rows ib.., columns jb..):
// v = alpha C + beta E + gamma [i == j < n_real] in arrangement A, then its
// stores and partial sums.  MAYDIAG: the tile is on the diagonal of a
// symmetric product and dblk says whether this block is (ib == jb).  Final
// kinds write v to the wave's LDS staging area ep (row-major, BN + 4 floats per
// row) for the update of W.
template <int OP, int KIND, bool MAYDIAG, int FN>
__device__ __forceinline__ void epi_block(const GemmArgs& a, EpiState& st, const EpiPtrs& p, const f32x16_t& c,
                                          const uint4 (&ein)[2], int x, int y, int ib, bool dblk, int lane,
                                          const uint4 (&id)[2], lds_f32* ep) {
  constexpr EpiSpec S = epi_spec(KIND);
  const int jr = lane & 31, ir0 = 4 * (lane >> 5);
  float v[16];
  if constexpr (S.e) {
    float e[16];
    n16_to_a<OP>(ein[0], ein[1], e);
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = st.alpha * c[r] + st.beta * e[r];
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = st.alpha * c[r];
  }
  if constexpr (MAYDIAG) {
    if (dblk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ir = 8 * (r >> 2) + ir0 + (r & 3);
        if (ir == jr && ib + ir < a.n_real) v[r] += st.gamma;
      }
    }
  }
  if constexpr (S.fin) {
#pragma unroll
    for (int r = 0; r < 16; ++r) ep[(8 * (r >> 2) + ir0 + (r & 3)) * (32 * FN + 4) + 32 * y + jr] = v[r];
    return;
  }
  if constexpr (S.sym) {
    if (a.part_out != nullptr) {  // an off-diagonal value stands for two
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ir = 8 * (r >> 2) + ir0 + (r & 3);
        const double xv = v[r];
        if (!MAYDIAG || !dblk || ir > jr) {
          st.ss += 2.0 * xv * xv;
        } else if (ir == jr) {
          st.ss += xv * xv;
          st.tr += xv;
        }
      }
    }
  }
  uint16_t* t = p.t16 + x * p.rs_t + 2048 * (y >> 1) + 512 * (2 * (y & 1));
  uint16_t* n = p.n16 + y * p.rs_n + 512 * (2 * x);
  store_tn<OP, S.sym && MAYDIAG>(t, n, v, lane, id, dblk);
  if constexpr (S.q) {  // a fresh Q = v + a' I; it differs from v on diagonal blocks only
    uint16_t* tq = p.tq + x * p.rs_t + 2048 * (y >> 1) + 512 * (2 * (y & 1));
    uint16_t* nq = p.nq + y * p.rs_t + 512 * (2 * x);
    if (MAYDIAG && dblk) {
      float q[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ir = 8 * (r >> 2) + ir0 + (r & 3);
        q[r] = (ir == jr && ib + ir < a.n_real) ? v[r] + st.ap : v[r];
      }
      store_tn<OP, true>(tq, nq, q, lane, id, true);
    } else {
      store_tn<OP, false>(tq, nq, v, lane, id, false);
    }
  }
}

// Block BLK + U of a group (see epi_run); recursion keeps every block index a
// compile-time constant.
// dg = (first column block of the tile) - (first row block of the tile), in
// 32-wide MFMA blocks; on tiles that meet the diagonal, block (x, y) of wave
// w is a diagonal block when dg + y == 2 w + x and lies above the diagonal
// (the mirror of an owned block, skipped) when dg + y > 2 w + x.
template <int OP, int KIND, bool MAYDIAG, int FN, int G, int BLK, int U>
__device__ __forceinline__ void epi_unit(const GemmArgs& a, EpiState& st, const EpiPtrs& p,
                                         const f32x16_t (&acc)[kFM][FN], const uint4 (&cur)[G][2], int I, int dg,
                                         int wave, int lane, const uint4 (&id)[2], lds_f32* ep) {
  constexpr int x = (BLK + U) / FN, y = (BLK + U) % FN;
  const int rel = dg + y - (2 * wave + x);
  if (!MAYDIAG || rel <= 0)
    epi_block<OP, KIND, MAYDIAG, FN>(a, st, p, acc[x][y], cur[U], x, y, I * kBM + wave * (kBM / kNW) + 32 * x,
                                 MAYDIAG && rel == 0, lane, id, ep);
  if constexpr (U + 1 < G)
    epi_unit<OP, KIND, MAYDIAG, FN, G, BLK, U + 1>(a, st, p, acc, cur, I, dg, wave, lane, id, ep);
}

// Blocks BLK .. BLK + G - 1 (block index FN x + y) of the wave's register
// epilogue with their inputs in `cur`; the inputs of the next group are
// loaded first, so their latency overlaps this group's work.  All blocks are
// named by template arguments: the accumulators stay in registers.
template <int OP, int KIND, bool MAYDIAG, int FN, int G, int BLK, int END>
__device__ __forceinline__ void epi_run(const GemmArgs& a, EpiState& st, const EpiPtrs& p,
                                        const f32x16_t (&acc)[kFM][FN], uint4 (&cur)[G][2], int I, int dg, int wave,
                                        int lane, const uint4 (&id)[2], lds_f32* ep) {
  uint4 nxt[G][2];
  if constexpr (BLK + G < END) {
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int x = (BLK + G + u) / FN, y = (BLK + G + u) % FN;
      if (!MAYDIAG || dg + y <= 2 * wave + x) load_ein<KIND>(p, x, y, lane, nxt[u]);
    }
  }
  epi_unit<OP, KIND, MAYDIAG, FN, G, BLK, 0>(a, st, p, acc, cur, I, dg, wave, lane, id, ep);
  if constexpr (BLK + G < END)
    epi_run<OP, KIND, MAYDIAG, FN, G, BLK + G, END>(a, st, p, acc, nxt, I, dg, wave, lane, id, ep);
}

template <int OP, int KIND, bool MAYDIAG, int FN, int BEGIN, int END>
__device__ __forceinline__ void epi_range(const GemmArgs& a, EpiState& st, const EpiPtrs& p,
                                          const f32x16_t (&acc)[kFM][FN], int I, int dg, int wave, int lane,
                                          const uint4 (&id)[2], lds_f32* ep) {
  constexpr int G = FN >= 8 ? 4 : 2;  // blocks per prefetch group (fewer registers with two blocks per CU)
  uint4 cur[G][2];
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const int x = (BEGIN + u) / FN, y = (BEGIN + u) % FN;
    if (!MAYDIAG || dg + y <= 2 * wave + x) load_ein<KIND>(p, x, y, lane, cur[u]);
  }
  epi_run<OP, KIND, MAYDIAG, FN, G, BEGIN, END>(a, st, p, acc, cur, I, dg, wave, lane, id, ep);
}

// The last product's epilogue for a 256 x 128 tile wholly inside the matrix
// (every 32 x 128 block passes final_fast_ok): as the general sequence
// (stage half 0, update it, stage half 1, update it; three block barriers),
// with each half's W loads issued before that half is staged.
template <int OP, int KIND, int WD, int OD>
__device__ __forceinline__ void fin_prefetched(const GemmArgs& a, EpiState& st, const EpiPtrs& p,
                                               const f32x16_t (&acc)[kFM][TileCfg<kHalfTile>::kFN], int I, int J,
                                               int wave, int lane, const uint4 (&id)[2], lds_f32* ep) {
  constexpr int FN = TileCfg<kHalfTile>::kFN, NB = kFM * FN, LDE = kHalfTile + 4;
  const int i0 = I * kBM + wave * (kBM / kNW), j0 = J * kHalfTile;
  float4 wv[16];
  final_load_w128<WD>(a, st, i0, j0, lane, wv);
  epi_range<OP, KIND, false, FN, 0, FN>(a, st, p, acc, I, 0, wave, lane, id, ep);
  __syncthreads();
  final_apply128<WD, OD, LDE>(a, st, ep, i0, j0, lane, wv);
  final_load_w128<WD>(a, st, i0 + 32, j0, lane, wv);
  __syncthreads();
  epi_range<OP, KIND, false, FN, FN, NB>(a, st, p, acc, I, 0, wave, lane, id, ep);
  __syncthreads();
  final_apply128<WD, OD, LDE>(a, st, ep, i0 + 32, j0, lane, wv);
}

// The register epilogue of the wave's 64 x BN sub-tile; the last product
// stages O through LDS one 32-row block (32 x BN) at a time so
// that the user's row-major W is read and written along its rows.
template <int OP, int KIND, int BN>
__device__ __forceinline__ void epilogue_mfma(const GemmArgs& a, EpiState& st,
                                              const f32x16_t (&acc)[kFM][TileCfg<BN>::kFN], int b, int I, int J,
                                              int wave, int lane, lds_f32* ep) {
  constexpr int FN = TileCfg<BN>::kFN, NB = kFM * FN;
  constexpr EpiSpec S = epi_spec(KIND);
  const EpiPtrs p = epi_ptrs<KIND, BN>(a, b, I, J, wave);
  if constexpr (S.fin) {
    const uint4 id[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};  // no transposes here
    if constexpr (BN == kHalfTile && KIND == kEpiFin) {
      // a tile wholly inside the matrix with a W to update: the W loads of
      // each 32-row half go out before that half of O is staged (not with a
      // 16-bit epilogue input, whose prefetch leaves no registers for them)
      if (st.w != nullptr && final_fast_ok<BN>(a, st, I * kBM, J * BN) &&
          final_fast_ok<BN>(a, st, I * kBM + kBM - 32, J * BN)) {
        const int odt = st.o != nullptr ? a.o_dtype : -1;
#define MUON_PREFETCHED(WD, OD)                                                         \
  if (a.w_dtype == WD && odt == OD) {                                                   \
    fin_prefetched<OP, KIND, WD, OD>(a, st, p, acc, I, J, wave, lane, id, ep);          \
    return;                                                                             \
  }
        MUON_PREFETCHED(kF32, -1) MUON_PREFETCHED(kBF16, -1) MUON_PREFETCHED(kF32, kF32)
        MUON_PREFETCHED(kF32, kBF16) MUON_PREFETCHED(kBF16, kF32) MUON_PREFETCHED(kBF16, kBF16)
#undef MUON_PREFETCHED
      }
    }
    epi_range<OP, KIND, false, FN, 0, FN>(a, st, p, acc, I, 0, wave, lane, id, ep);
    __syncthreads();
    final_block<BN + 4, BN>(a, st, ep, I * kBM + wave * (kBM / kNW), J * BN, lane);
    __syncthreads();
    epi_range<OP, KIND, false, FN, FN, NB>(a, st, p, acc, I, 0, wave, lane, id, ep);
    __syncthreads();
    final_block<BN + 4, BN>(a, st, ep, I * kBM + wave * (kBM / kNW) + 32, J * BN, lane);
  } else {
    const uint4 id[2] = {ident_frag<OP>(0, lane), ident_frag<OP>(1, lane)};
    // a symmetric tile meets the diagonal when its column range overlaps its
    // row range: tile J == I of the 256-wide tiles (dg = 0), tiles J == 2 I
    // and 2 I + 1 of the 128-wide ones (dg = 0 and 4)
    if constexpr (BN == kMfmaTile) {
      if (S.sym && I == J)
        epi_range<OP, KIND, S.sym, FN, 0, NB>(a, st, p, acc, I, 0, wave, lane, id, ep);
      else
        epi_range<OP, KIND, false, FN, 0, NB>(a, st, p, acc, I, 0, wave, lane, id, ep);
    } else {
      if (S.sym && J >= 2 * I)
        epi_range<OP, KIND, S.sym, FN, 0, NB>(a, st, p, acc, I, 4 * (J - 2 * I), wave, lane, id, ep);
      else
        epi_range<OP, KIND, false, FN, 0, NB>(a, st, p, acc, I, 0, wave, lane, id, ep);
    }
  }
}

// The kernel's argument block, loaded again from the kernel argument segment
// through a pointer the compiler cannot follow (so it cannot reuse values
// loaded before the main loop).
__device__ __forceinline__ GemmArgs reload_args() {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef const __attribute__((address_space(4))) GemmArgs* kargs_ptr;
  kargs_ptr p = (kargs_ptr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  GemmArgs r;
  __builtin_memcpy(&r, (const __attribute__((address_space(4))) void*)p, sizeof(GemmArgs));
  return r;
#else
  return GemmArgs{};  // device code only
#endif
}

// This block's work: matrix b, tile (I, J) and slabs [k0, k1), and for a
// piece of a split tail tile its tail index and piece number (piece = -1 for
// a whole tile).  Consecutive block ids go to different XCDs (round-robin),
// so within the whole-tile range and within the tail range the ids are
// renumbered such that each XCD works through a contiguous range; tiles of a
// general product are ordered in groups of 8 tile-rows for L2 reuse.
struct WorkItem {
  int b, tile, I, J, k0, k1, tail, piece;
};

__device__ __forceinline__ int xcd_contiguous(int id, int n) {
  const int q = n >> 3, rem = n & 7, x = id & 7, slot = id >> 3;
  return (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + slot;
}

// Tile t of the lower triangle in 256 x 128 tiles: row I (256 rows) holds
// the tiles J = 0 .. 2 I + 1 (128 columns each), rows in order.
__device__ __forceinline__ void tri_tile_half(int t, int& I, int& J) {
  int i = static_cast<int>((sqrtf(4.0f * static_cast<float>(t) + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) <= t) ++i;
  while (i * (i + 1) > t) --i;
  I = i;
  J = t - i * (i + 1);
}

template <int BN>
__device__ __forceinline__ WorkItem work_item(const GemmArgs& a) {
  WorkItem w;
  const int hw = blockIdx.x, nfull = a.full_blocks;
  const int nk = a.K / kBK;
  int t;
  if (hw < nfull) {
    t = xcd_contiguous(hw, nfull);
    w.k0 = 0;
    w.k1 = nk;
    w.tail = -1;
    w.piece = -1;
  } else {
    const int p = xcd_contiguous(hw - nfull, static_cast<int>(gridDim.x) - nfull);
    w.tail = p / a.kpieces;
    w.piece = p - w.tail * a.kpieces;
    t = nfull + w.tail;
    const int units = nk >> 2;  // k in units of 4 slabs, shared out as evenly as possible
    w.k0 = 4 * ((units * w.piece) / a.kpieces);
    w.k1 = 4 * ((units * (w.piece + 1)) / a.kpieces);
  }
  w.b = t / a.ntiles;
  const int tile = t - w.b * a.ntiles;
  w.tile = tile;
  if (a.sym) {
    if constexpr (BN == kMfmaTile) {
      tri_tile(tile, w.I, w.J);
    } else {
      tri_tile_half(tile, w.I, w.J);
    }
  } else {
    const int ntm = a.Mdim / kBM, ntn = a.Ndim / BN;
    constexpr int G = 8;
    const int grp = tile / (G * ntn);
    const int first = grp * G;
    const int rows = ntm - first < G ? ntm - first : G;
    const int in = tile - grp * G * ntn;
    w.I = first + in % rows;
    w.J = in / rows;
  }
  return w;
}

// A piece of a split tail tile: store this block's fp32 partial tile, and
// return true for the last piece to finish, which then holds the sum of all
// pieces, added in piece order (so the result does not depend on which piece
// finishes last), in acc.  Partials are kept per wave as [x][y][g][lane]
// float4 records (1 KB per store).  All threads of the block call this.
template <int kFN>
__device__ __forceinline__ bool tail_reduce(const GemmArgs& a, const WorkItem& w, f32x16_t (&acc)[kFM][kFN], int wave,
                                            int lane, int* flag) {
  constexpr int64_t kWaveFloats = kFM * kFN * 16 * 64;
  auto part = [&](int piece) {
    return a.part32 + (static_cast<int64_t>(w.tail) * a.kpieces + piece) * kPartFloats + wave * kWaveFloats +
           4 * lane;
  };
  float* mine = part(w.piece);
#pragma unroll
  for (int x = 0; x < kFM; ++x)
#pragma unroll
    for (int y = 0; y < kFN; ++y)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(mine + ((x * kFN + y) * 4 + g) * 256) =
            make_float4(acc[x][y][4 * g], acc[x][y][4 * g + 1], acc[x][y][4 * g + 2], acc[x][y][4 * g + 3]);
  // Release: this piece's partial is written back to memory before the
  // counter moves.  Only the last piece acquires (invalidates its caches), so
  // the other pieces leave the cached operands of their neighbours alone.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) *flag = atomicAdd(a.counters + w.tail, 1);
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(*flag) != a.kpieces - 1) return false;  // uniform over the block
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (threadIdx.x == 0) a.counters[w.tail] = 0;  // ready for the next launch
#pragma unroll
  for (int x = 0; x < kFM; ++x)
#pragma unroll
    for (int y = 0; y < kFN; ++y) {
      const f32x16_t own = acc[x][y];
      f32x16_t sum;
      for (int p = 0; p < a.kpieces; ++p) {
        f32x16_t v;
        if (p == w.piece) {
          v = own;
        } else {
          const float* src = part(p) + (x * kFN + y) * 4 * 256;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 q = *reinterpret_cast<const float4*>(src + g * 256);
            v[4 * g] = q.x;
            v[4 * g + 1] = q.y;
            v[4 * g + 2] = q.z;
            v[4 * g + 3] = q.w;
          }
        }
        if (p == 0) {
          sum = v;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) sum[r] += v[r];
        }
      }
      acc[x][y] = sum;
    }
  return true;
}

template <int OP, int KIND, int BN>
__global__ __launch_bounds__(kNT, BN == kMfmaTile ? 1 : 2) void gemm_nt_mfma(GemmArgs a) {
  using C = TileCfg<BN>;
  constexpr int kFN = C::kFN;
  // The Q ring is four separate arrays, each named statically at every access,
  // so the compiler's wait for an LDS read covers only the DMA into that stage.
  __shared__ uint4 stg0[C::kStageAlloc / 16], stg1[C::kStageAlloc / 16], stg2[C::kStageAlloc / 16],
      stg3[C::kStageAlloc / 16];
  __shared__ double red[2 * kNW];
  __shared__ int tail_flag;
  const WorkItem w = work_item<BN>(a);
  const int b = w.b, tile = w.tile, I = w.I, J = w.J;
  EpiState st;
  block_init<kNT>(a, b, tile, red, st);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint16_t* Pm = static_cast<const uint16_t*>(a.P) + static_cast<int64_t>(b) * a.sP;
  const uint16_t* Qm = static_cast<const uint16_t*>(a.Q) + static_cast<int64_t>(b) * a.sQ;
  // In a 256 x 128 symmetric tile at J = 2 I + 1 the rows of waves 0 and 1
  // lie wholly above the diagonal, so none of their values is stored.  Their
  // P descriptor covers nothing: the loads return zeros without a memory
  // access, and their MFMAs (the same count, so the block's schedule and
  // barriers are unchanged) run on zero operands, which draws less power.
  const bool above_diag = BN == kHalfTile && a.sym != 0 && J == 2 * I + 1 && wave < 2;
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(Pm, above_diag ? 0 : static_cast<int64_t>(a.Mdim) * a.ldp * 2);
  const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Qm, static_cast<int64_t>(a.Ndim) * a.ldq * 2);
  const int voff = lane * 16;
  // byte offset of a row block = (row / 32) * (K / 64) * 4 KB
  const int pstride = (a.ldp >> 6) * 4096, qstride = (a.ldq >> 6) * 4096;
  const int sP = __builtin_amdgcn_readfirstlane((I * (kBM / 32) + wave * kFM) * pstride);
  const int sQ = __builtin_amdgcn_readfirstlane(J * (BN / 32) * qstride);

  f32x16_t acc[kFM][kFN];
#pragma unroll
  for (int x = 0; x < kFM; ++x)
#pragma unroll
    for (int y = 0; y < kFN; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;

  // slabs k0 .. k1 - 1 (a multiple of 4 of them: every operand dimension is a
  // multiple of 256 and tail pieces are cut at multiples of 4 slabs)
  const int k0 = w.k0, k1 = w.k1;
  uint4 bf[2][kFN];
  if constexpr (C::kPBufs == 4) {
    uint4 abuf0[kFM][kKS], abuf1[kFM][kKS], abuf2[kFM][kKS], abuf3[kFM][kKS];
    // prologue: Q slabs k0 .. k0 + 3 into the ring, P slabs k0 .. k0 + 2 into
    // registers, issued in the order the loop itself issues them (P slab j + 3
    // at the start of slab j, Q slab j + 4 in its middle), so the outstanding
    // loads at the loop head look the same on entry and on every trip and the
    // compiler's waits for the P registers stay exact.
    load_b_slab<BN>(stg0, rQ, voff, sQ, qstride, k0, wave);
    load_a_slab(abuf0, rP, voff, sP, pstride, k0);
    load_b_slab<BN>(stg1, rQ, voff, sQ, qstride, k0 + 1, wave);
    load_a_slab(abuf1, rP, voff, sP, pstride, k0 + 1);
    load_b_slab<BN>(stg2, rQ, voff, sQ, qstride, k0 + 2, wave);
    load_a_slab(abuf2, rP, voff, sP, pstride, k0 + 2);
    load_b_slab<BN>(stg3, rQ, voff, sQ, qstride, k0 + 3, wave);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(3 * kLoadsA + 3 * C::kLoadsB, 15));  // Q slab 0 landed
    block_barrier();
#pragma unroll
    for (int y = 0; y < kFN; ++y) bf[0][y] = stg0[y * kKS * 64 + lane];

    // 4 slabs per trip (the 4 LDS stages and the 4 P register buffers, which
    // are loaded three slabs ahead).
#define MUON_SLAB(U, BUF, NEXTBUF, CUR, NXT)                                                           \
  load_a_slab(NEXTBUF, rP, voff, sP, pstride, kt + U + 3);                                             \
  slab<OP, BN>(acc, BUF, bf, CUR, NXT, rQ, voff, sQ, qstride, kt + U, wave, lane);
    for (int kt = k0; kt < k1; kt += 4) {
      MUON_SLAB(0, abuf0, abuf3, stg0, stg1)
      MUON_SLAB(1, abuf1, abuf0, stg1, stg2)
      MUON_SLAB(2, abuf2, abuf1, stg2, stg3)
      MUON_SLAB(3, abuf3, abuf2, stg3, stg0)
    }
#undef MUON_SLAB
  } else {
    uint4 abuf0[kFM][kKS], abuf1[kFM][kKS], abuf2[kFM][kKS];
    // prologue: Q slabs k0 .. k0 + 3 and P slabs k0, k0 + 1, in the order the
    // loop issues them (P slab j + 2 at the start of slab j, Q slab j + 4 in
    // its middle), so the compiler's waits for the P registers stay exact
    load_b_slab<BN>(stg0, rQ, voff, sQ, qstride, k0, wave);
    load_b_slab<BN>(stg1, rQ, voff, sQ, qstride, k0 + 1, wave);
    load_a_slab(abuf0, rP, voff, sP, pstride, k0);
    load_b_slab<BN>(stg2, rQ, voff, sQ, qstride, k0 + 2, wave);
    load_a_slab(abuf1, rP, voff, sP, pstride, k0 + 1);
    load_b_slab<BN>(stg3, rQ, voff, sQ, qstride, k0 + 3, wave);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kLoadsA + 3 * C::kLoadsB, 15));  // Q slab 0 landed
    block_barrier();
#pragma unroll
    for (int y = 0; y < kFN; ++y) bf[0][y] = stg0[y * kKS * 64 + lane];

    // 12 slabs per trip (the 4 LDS stages against the 3 P buffers, loaded two
    // slabs ahead); the slab count is a multiple of 4, so the trip may end
    // after its 4th or 8th slab
#define MUON_SLAB(U, BUF, NEXTBUF, CUR, NXT)                                                           \
  slab_spread<OP, BN>(acc, BUF, bf, CUR, NXT, NEXTBUF, rP, sP, pstride, kt + U + 2, rQ, voff, sQ, qstride,      \
                      kt + U, wave, lane);
    for (int kt = k0;; kt += 12) {
      MUON_SLAB(0, abuf0, abuf2, stg0, stg1)
      MUON_SLAB(1, abuf1, abuf0, stg1, stg2)
      MUON_SLAB(2, abuf2, abuf1, stg2, stg3)
      MUON_SLAB(3, abuf0, abuf2, stg3, stg0)
      if (kt + 4 >= k1) break;
      MUON_SLAB(4, abuf1, abuf0, stg0, stg1)
      MUON_SLAB(5, abuf2, abuf1, stg1, stg2)
      MUON_SLAB(6, abuf0, abuf2, stg2, stg3)
      MUON_SLAB(7, abuf1, abuf0, stg3, stg0)
      if (kt + 8 >= k1) break;
      MUON_SLAB(8, abuf2, abuf1, stg0, stg1)
      MUON_SLAB(9, abuf0, abuf2, stg1, stg2)
      MUON_SLAB(10, abuf1, abuf0, stg2, stg3)
      MUON_SLAB(11, abuf2, abuf1, stg3, stg0)
      if (kt + 12 >= k1) break;
    }
#undef MUON_SLAB
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  block_barrier();
  if constexpr (BN == kMfmaTile) {
    if (w.piece >= 0 && !tail_reduce<kFN>(a, w, acc, wave, lane, &tail_flag)) return;
  }

  // The epilogue runs from registers; the last product stages O through this
  // wave's LDS stage.  It reads the launch arguments afresh, so they are not
  // held in scalar registers through the main loop.
  const GemmArgs ea = reload_args();
  lds_f32* ep = (lds_f32*)(wave == 0 ? stg0 : (wave == 1 ? stg1 : (wave == 2 ? stg2 : stg3)));
  epilogue_mfma<OP, KIND, BN>(ea, st, acc, b, I, J, wave, lane, ep);
  block_partials<kNT>(ea, b, tile, red, st);
}

template <int OP>
hipError_t launch_gemm_mfma(const GemmArgs& a, int batch, int kind, hipStream_t s) {
  const int64_t tiles = static_cast<int64_t>(a.ntiles) * batch;
  const dim3 grid(static_cast<unsigned>(a.full_blocks + (tiles - a.full_blocks) * a.kpieces)), block(kNT);
  if (a.bn == kHalfTile) {  // short symmetric products and last products, without the tail split
    if (a.kpieces != 1) return hipErrorInvalidValue;
    const bool fin = kind == kEpiFin || kind == kEpiFinE16;
    if (fin ? a.sym != 0 : a.sym == 0) return hipErrorInvalidValue;
    switch (kind) {
      case kEpiSym: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiSym, kHalfTile>), grid, block, 0, s, a); break;
      case kEpiSymE16: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiSymE16, kHalfTile>), grid, block, 0, s, a); break;
      case kEpiSymE16Q: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiSymE16Q, kHalfTile>), grid, block, 0, s, a); break;
      case kEpiFin: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiFin, kHalfTile>), grid, block, 0, s, a); break;
      case kEpiFinE16: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiFinE16, kHalfTile>), grid, block, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (a.bn != kMfmaTile) return hipErrorInvalidValue;
  switch (kind) {
    case kEpiSym: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiSym, kMfmaTile>), grid, block, 0, s, a); break;
    case kEpiSymE16: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiSymE16, kMfmaTile>), grid, block, 0, s, a); break;
    case kEpiSymE16Q: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiSymE16Q, kMfmaTile>), grid, block, 0, s, a); break;
    case kEpiGen: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiGen, kMfmaTile>), grid, block, 0, s, a); break;
    case kEpiGenE16: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiGenE16, kMfmaTile>), grid, block, 0, s, a); break;
    case kEpiFin: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiFin, kMfmaTile>), grid, block, 0, s, a); break;
    case kEpiFinE16: hipLaunchKernelGGL((gemm_nt_mfma<OP, kEpiFinE16, kMfmaTile>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace muon
