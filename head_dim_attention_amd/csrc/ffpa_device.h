// Device-side building blocks shared by the gfx950 attention kernels.
//
// Conventions used by every kernel in this library:
//  * A workgroup is 4 or 8 wave64s (8, two per SIMD, where a wave's state fits 256 registers).
//    Waves are arranged NR x NC: NR row groups of stationary rows
//    (queries in the forward and dQ kernels, keys in the dK/dV kernel) and NC column groups that
//    each own DW = NDB*32 of the (padded) head dim. Partial sums over the head dim are combined
//    across the NC waves of a row group through LDS.
//  * Matrix products use v_mfma_f32_32x32x16_{bf16,f16}. Lane l = 32*h + n holds, for an A
//    operand, row (l%32) and k = 8h..8h+7; for a B operand, column (l%32) and the same k; the
//    16 fp32 results of a C block sit at row 8*(r/4) + 4h + (r%4), column l%32.
//  * Streamed tiles are 32 rows x RS bytes in LDS, row-major, with the 16-byte chunks of each row
//    permuted by an XOR swizzle so that both the row reads (ds_read_b128) and the transposed reads
//    (ds_read_b64_tr_b16) touch distinct banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ffpa_params.h"

namespace ffpa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) char lds_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct BF16 {};
struct FP16 {};

template <class T> struct Elt;

template <> struct Elt<BF16> {
  static __device__ __forceinline__ f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // Round two fp32 values to nearest-even bf16 and pack (lo in bits 0..15).
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float to_f32(uint16_t x) {
    return __builtin_bit_cast(float, (uint32_t)x << 16);
  }
  static __device__ __forceinline__ void unpack2(uint32_t x, float& lo, float& hi) {
    lo = __builtin_bit_cast(float, x << 16);
    hi = __builtin_bit_cast(float, x & 0xffff0000u);
  }
};

template <> struct Elt<FP16> {
  static __device__ __forceinline__ f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t);
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float to_f32(uint16_t x) {
    return (float)__builtin_bit_cast(_Float16, x);
  }
  static __device__ __forceinline__ void unpack2(uint32_t x, float& lo, float& hi) {
    const f16x2_t v = __builtin_bit_cast(f16x2_t, x);
    lo = (float)v.x;
    hi = (float)v.y;
  }
};

// XOR applied to the 16-byte chunk index of LDS row `row`. Within any 16 consecutive rows it is
// a bijection onto 0..15 (row reads of 16 lanes hit 16 distinct chunks), and for 4 consecutive
// rows starting at a multiple of 4 it yields 4 distinct multiples of 4 (transposed reads of a
// 16-lane group hit distinct chunks).
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// MFMA row m of a streamed A operand is loaded from tile row row_perm(m), which exchanges bits 2
// and 3 of m. With that order, C-block register r of a lane in half h holds tile row
// c_row(r, h) = 16*(r/8) + 8h + 4*((r/4)%2) + r%4, so registers 8kb..8kb+7 cover the consecutive
// tile rows 16kb + 8h + 0..7: exactly the k-slots of a B operand for k-step kb. A C block of
// scores can then feed the next product as a B operand without moving data between lanes.
__device__ __forceinline__ int row_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
__device__ __forceinline__ int c_row(int r, int h) { return 16 * (r >> 3) + 8 * h + 4 * ((r >> 2) & 1) + (r & 3); }

__device__ __forceinline__ u32x4_t lds_read_b128(const lds_t* base, int byte_off) {
  return *(const __attribute__((address_space(3))) u32x4_t*)(base + byte_off);
}

__device__ __forceinline__ void lds_write_b128(lds_t* base, int byte_off, u32x4_t v) {
  *(__attribute__((address_space(3))) u32x4_t*)(base + byte_off) = v;
}

__device__ __forceinline__ f32x4_t lds_read_f4(const lds_t* base, int byte_off) {
  return *(const __attribute__((address_space(3))) f32x4_t*)(base + byte_off);
}

__device__ __forceinline__ void lds_write_f4(lds_t* base, int byte_off, f32x4_t v) {
  *(__attribute__((address_space(3))) f32x4_t*)(base + byte_off) = v;
}

// Transposed read (ds_read_b64_tr_b16). Within each 16-lane group, source lane s supplies the
// address of 4 consecutive 16-bit elements ("row s"); lane i receives element i%4 of rows
// i/4, i/4+4, i/4+8, i/4+12.
__device__ __forceinline__ s16x4_t lds_read_tr16(const lds_t* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(base + byte_off));
}

// Reads at a raw LDS byte address (for addresses formed by XOR from a per-lane base).
__device__ __forceinline__ uint32_t lds_addr(const lds_t* p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ u32x4_t lds_read_b128_at(uint32_t a) {
  return *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)a;
}
__device__ __forceinline__ s16x4_t lds_read_tr16_at(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(uintptr_t)a);
}

__device__ __forceinline__ u32x4_t join_tr(s16x4_t lo, s16x4_t hi) {
  u32x2_t a = __builtin_bit_cast(u32x2_t, lo);
  u32x2_t b = __builtin_bit_cast(u32x2_t, hi);
  return (u32x4_t){a.x, a.y, b.x, b.y};
}

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource descriptor over [base, base + bytes) for raw (unformatted) 32-bit accesses:
// base address in words 0-1 (stride 0), size in word 2, data format 32 in word 3.
// The descriptor is wave-uniform; readfirstlane keeps it in scalar registers.
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  return (i32x4_t){__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)b),
                   __builtin_amdgcn_readfirstlane((int32_t)((b >> 32) & 0xffff)),
                   __builtin_amdgcn_readfirstlane((int32_t)bytes), 0x00020000};
}

// Asynchronous 16-byte copy through a buffer resource: lane l reads base + voff(lane) + soff and
// writes LDS bytes [lds + 16 l, lds + 16 l + 16) (buffer_load_dwordx4 ... lds, LDS address in M0).
// It is issued as inline asm on purpose: the compiler then does not track it, and so does not wait
// for an in-flight prefetch of the next tile before reading the current one. Callers make copied
// data visible explicitly: wait_vmcnt() in every issuing wave, then lds_barrier().
// M0 is saved and restored around the copy, so its value is unchanged for the compiler.
__device__ __forceinline__ void dma16_buf(i32x4_t r, int voff, int soff, lds_t* lds) {
  // All scalar operands are wave-uniform by construction; readfirstlane makes that explicit for
  // the LDS address and row offset (r comes from make_rsrc, already scalar).
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  soff = __builtin_amdgcn_readfirstlane(soff);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(soff), "s"(m)
      : "memory");
}

// dma16_buf with the non-temporal hint, for blocks each workgroup reads once: they are not kept
// in L2 at the expense of the rows that neighbouring workgroups read again.
__device__ __forceinline__ void dma16_buf_nt(i32x4_t r, int voff, int soff, lds_t* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  soff = __builtin_amdgcn_readfirstlane(soff);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(soff), "s"(m)
      : "memory");
}

// Scheduling pin for a run of N MFMAs fed by LDS reads in the current scheduling region: the
// reads of the first AHEAD MFMAs first, then alternately one MFMA and the reads of a later one,
// then the last AHEAD MFMAs. Each MFMA then finds its operand already loaded instead of waiting
// for the full LDS latency. R = LDS reads per MFMA. (Mask bits: 0x008 MFMA, 0x100 LDS read.)
template <int N, int AHEAD, int R>
__device__ __forceinline__ void pin_lds_mfma_pipeline() {
  static_assert(AHEAD >= 1 && AHEAD <= N, "pipeline depth");
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * R, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// Asynchronous 4-byte copy through a buffer resource: lane l reads base + voff(lane) and writes
// LDS bytes [lds + 4 l, lds + 4 l + 4). Same tracking rules as dma16_buf.
__device__ __forceinline__ void dma4_buf(i32x4_t r, int voff, lds_t* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dword %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(m)
      : "memory");
}

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// Wait until at most N vector-memory loads of this wave are outstanding. Issued through the
// builtin so the compiler accounts for it in its own wait tracking.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 15));
}

// Wait for every outstanding memory operation of this wave.
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0)); }

// Workgroup barrier that orders LDS accesses only. __syncthreads() adds a release fence that also
// waits for every outstanding global load, including asynchronous global->LDS prefetches of the
// next tile, which would expose their full latency at every exchange. Prefetched tiles are made
// visible separately: wait_vmcnt() in every issuing wave, then this barrier. The empty asm
// statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Combine the values of lanes l and l ^ 32 (the two halves of a wave). v_permlane32_swap
// exchanges the upper half of one register with the lower half of another in the VALU (no LDS
// round trip); applied to two copies of x it leaves lane l with x of lanes l % 32 and 32 + l % 32,
// so every lane combines the same two operands in the same order and gets the same bits.
__device__ __forceinline__ void wave_halves(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_max(float x) {
  float lo, hi;
  wave_halves(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float half_sum(float x) {
  float lo, hi;
  wave_halves(x, lo, hi);
  return lo + hi;
}

// Opaque register definition (empty asm): the value is not known to the compiler past this point,
// so nothing derived from it is hoisted out of a loop (it is recomputed where it is used instead
// of holding registers across the loop).
__device__ __forceinline__ int opaque_v(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Opaque scalar (wave-uniform) value: like opaque_v, for values kept in scalar registers.
__device__ __forceinline__ uint32_t opaque_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// This lane's index in its wave, read from the hardware at this point (not a value the compiler
// may keep in a register across a loop).
__device__ __forceinline__ int fresh_lane_id() {
  int x;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
  return x;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Work item of workgroup L among items ordered (sequence, head, inner index), `inner` items per
// head. Workgroup ids go round-robin over the 8 XCDs (L mod 8). Dense: XCD x takes the contiguous
// eighth [x grid / 8, (x + 1) grid / 8) of the list -- whole heads, so a head's K/V tiles are
// shared in one XCD's L2. Varlen sequences differ in length and contiguous eighths would hand
// whole sequences to one XCD; there XCD x takes heads x, x + 8, ... of every sequence (each XCD
// the same share of every sequence, a head's items still on one XCD) when the head count is a
// multiple of 8, else the items round-robin. Needs grid = total rounded up to a multiple of 8.
// Building with -DFFPA_XCD_ORDER=0 hands out items in launch order instead (workgroup L takes
// item L), which is only useful to measure what the mapping saves in L2 traffic.
#ifndef FFPA_XCD_ORDER
#define FFPA_XCD_ORDER 1
#endif
__device__ __forceinline__ int xcd_item(int L, int grid, bool varlen, int heads, int inner) {
  if (!FFPA_XCD_ORDER) return L;
  if (!varlen) return (L & 7) * (grid >> 3) + (L >> 3);
  if ((heads & 7) != 0) return L;
  const int r = L >> 3, hpx = heads >> 3;
  const int t = r % inner, q = r / inner;
  return ((q / hpx) * heads + (L & 7) + 8 * (q % hpx)) * inner + t;
}

// Epilogue store of a workgroup's output block through LDS, so that each global store writes 1 KB
// of one row (64 lanes x 16 bytes) rather than 8- or 16-byte pieces of 32 rows; the store path
// takes a piece per cache line and cycle, so the scattered form costs about 32 cycles an
// instruction. The 8 waves hold the block as NRG row groups x NCG column groups: wave (rg, cg)
// has RB x NDB fp32 C blocks, block (b, db) covering rows 32 (RB rg + b) + (lane % 32) and columns
// 32 (NDB cg + db) + 8 i4 + 4 h + 0..3 in registers 4 i4 .. 4 i4 + 3 of lane half h. The values
// (times the lane's `scale`) go out as T (rounded once) or, with F32, as fp32. A pass stages the
// rows of RGP row groups for one b in LDS rows of RS bytes (16-byte chunk c of stage row s at
// chunk c ^ (s % 16)); after a barrier the 8 waves copy them to dst (block row 0, column 0; row
// stride in elements). Rows at or past `rows` and columns at or past `cols` (a multiple of 8)
// are not stored. Called by all 8 waves after their last LDS read and DMA wait of the main loop;
// uses store_block_lds<..., LDSB>() bytes of LDS at `stage`, at most LDSB (RGP is the largest
// power of two of row groups whose stage fits in LDSB and 128 KB).
template <bool F32, int NCG, int NDB>
struct BlockStore {
  static constexpr int ES = F32 ? 4 : 2;                 // bytes per stored element
  static constexpr int ROWB = NCG * NDB * 32 * ES;       // bytes of a block row
  static constexpr int RS = ROWB <= 1024 ? 1024 : ROWB <= 2048 ? 2048 : 4096;
};
template <bool F32, int NRG, int NCG, int NDB, int LDSB>
constexpr int store_block_rgp() {
  constexpr int RS = BlockStore<F32, NCG, NDB>::RS;
  int r = NRG;
  while (r > 1 && (32 * r * RS > LDSB || 32 * r * RS > 131072)) r /= 2;
  return r;
}
template <bool F32, int NRG, int NCG, int NDB, int LDSB = 163840>
constexpr int store_block_lds() {
  return 32 * store_block_rgp<F32, NRG, NCG, NDB, LDSB>() * BlockStore<F32, NCG, NDB>::RS;
}
template <class T, bool F32, int NRG, int NCG, int RB, int NDB, int LDSB = 163840>
__device__ __forceinline__ void store_block_rows(lds_t* stage, const f32x16_t (&acc)[RB][NDB], float scale,
                                                 void* dst, long long row_stride, int rows, int cols) {
  using S = BlockStore<F32, NCG, NDB>;
  constexpr int RGP = store_block_rgp<F32, NRG, NCG, NDB, LDSB>();
  static_assert(NRG * NCG == 8 && NRG % RGP == 0 && 32 * RGP * S::RS <= LDSB, "8 waves; whole row groups per pass");
  constexpr int SROWS = 32 * RGP;       // stage rows per pass
  constexpr int PER_WAVE = SROWS / 8;   // stage rows each wave copies out
  constexpr int PARTS = S::RS / 1024;   // 1 KB store instructions per stage row
  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int rg = w / NCG;
  const int cg = w % NCG;
  lds_barrier();  // every wave is past its last read of the streamed tiles
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int pr = 0; pr < NRG / RGP; ++pr) {
      if (rg / RGP == pr) {
        const int srow = 32 * (rg % RGP) + l32;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const f32x16_t& a = acc[b][db];
            if constexpr (F32) {
              const int chunk = (NDB * cg + db) * 8 + 2 * i4 + hh;
              lds_write_f4(stage, srow * S::RS + ((chunk ^ (srow & 15)) << 4),
                           (f32x4_t){a[4 * i4] * scale, a[4 * i4 + 1] * scale, a[4 * i4 + 2] * scale,
                                     a[4 * i4 + 3] * scale});
            } else {
              const int chunk = (NDB * cg + db) * 4 + i4;
              const u32x2_t pk = {Elt<T>::pack2(a[4 * i4] * scale, a[4 * i4 + 1] * scale),
                                  Elt<T>::pack2(a[4 * i4 + 2] * scale, a[4 * i4 + 3] * scale)};
              *(__attribute__((address_space(3))) u32x2_t*)(stage + srow * S::RS + ((chunk ^ (srow & 15)) << 4) +
                                                            8 * hh) = pk;
            }
          }
      }
      lds_barrier();
#pragma unroll
      for (int rr = 0; rr < PER_WAVE; ++rr) {
        const int srow = PER_WAVE * w + rr;
        const int brow = 32 * (RB * (RGP * pr + srow / 32) + b) + (srow & 31);
#pragma unroll
        for (int part = 0; part < PARTS; ++part) {
          const int chunk = 64 * part + lane;
          if (brow < rows && chunk * (16 / S::ES) < cols) {
            const u32x4_t x = lds_read_b128(stage, srow * S::RS + ((chunk ^ (srow & 15)) << 4));
            *(u32x4_t*)((char*)dst + (brow * row_stride + chunk * (16 / S::ES)) * S::ES) = x;
          }
        }
      }
      if (b + 1 < RB || pr + 1 < NRG / RGP) lds_barrier();  // the stage is rewritten by the next pass
    }
}

// Tile item -> (sequence or batch s, query head h, tile t). Dense grids put the G query heads of
// a KV head side by side, item = ((s Hkv + kvh) ntiles + t) G + (h - kvh G): they sweep the same
// keys at the same time, so a tile's K/V lines serve all of them from L2. Varlen keeps
// item = (s Hq + h) ntiles + t (its XCD mapping hands out whole heads by index).
struct HeadTile {
  int s, h, t;
};
__device__ __forceinline__ HeadTile head_tile(int item, int ntiles, int hq, int group, bool dense) {
  HeadTile r;
  if (dense) {
    const int hg = item % group;
    const int rest = item / group;
    r.t = rest % ntiles;
    const int ks = rest / ntiles;
    const int hkv = hq / group;
    r.h = (ks % hkv) * group + hg;
    r.s = ks / hkv;
  } else {
    r.t = item % ntiles;
    const int hs = item / ntiles;
    r.h = hs % hq;
    r.s = hs / hq;
  }
  return r;
}

// Geometry of one (batch or sequence) slice, resolved from dense strides or cu_seqlens.
struct SeqView {
  long long q_off, k_off, lse_off, v_off, o_off;
  int lq, lk;
};

// Resolve slice s: a dense batch entry (strides) or a packed sequence (cu_seqlens).
__device__ __forceinline__ SeqView seq_view(const AttnParams& p, int s) {
  SeqView v;
  if (p.cu_q != nullptr) {
    const int q0 = p.cu_q[s], k0 = p.cu_k[s];
    v.lq = p.cu_q[s + 1] - q0;
    v.lk = p.cu_k[s + 1] - k0;
    v.q_off = (long long)q0 * p.q_row;
    v.k_off = (long long)k0 * p.k_row;
    v.v_off = (long long)k0 * p.v_row;
    v.o_off = (long long)q0 * p.o_row;
    v.lse_off = q0;
  } else {
    v.lq = p.nq;
    v.lk = p.nkv;
    v.q_off = (long long)s * p.q_batch;
    v.k_off = (long long)s * p.k_batch;
    v.v_off = (long long)s * p.v_batch;
    v.o_off = (long long)s * p.o_batch;
    v.lse_off = (long long)s * p.lse_batch;
  }
  return v;
}

// Stored P/dS geometry of slice s (blocks stored transposed, one row per key): element offset of
// (s, head 0, key 0, query 0), the head stride and the row stride (queries padded to a multiple of
// 8 elements, so 16-byte pieces stay aligned).
struct DsView {
  long long base, head;
  int row;
};

__device__ __forceinline__ int round_up8(int x) { return (x + 7) & ~7; }

__device__ __forceinline__ DsView ds_view(const AttnParams& p, int s, const SeqView& sv) {
  DsView v;
  if (p.cu_q != nullptr) {
    long long pre = 0;
    for (int t = 0; t < s; ++t) pre += (long long)(p.cu_k[t + 1] - p.cu_k[t]) * round_up8(p.cu_q[t + 1] - p.cu_q[t]);
    v.row = round_up8(sv.lq);
    v.head = (long long)sv.lk * v.row;
    v.base = pre * p.hq;
  } else {
    v.row = p.ds_row;
    v.head = p.ds_head;
    v.base = (long long)s * p.ds_batch;
  }
  return v;
}

// attn_mask of 8 consecutive keys key0 .. key0 + 7 (key0 a multiple of 8) of the mask row at
// element offset rowoff, in two steps so that the load can be issued well before its use.
// mask_raw8 returns the raw bits: additive, eight 16-bit values (all four words); boolean, eight
// bytes (.x, .y); a key-broadcast mask (m_key == 0), its one element in .x. With a contiguous key
// dim the row offset is a multiple of 8 and the base is aligned, so a piece is one aligned 16-byte
// (bias) or 8-byte (boolean) load. A piece that reaches past the row's last key lk - 1 is read
// as the row's last whole aligned piece instead (the one holding key lk - 1: an aligned piece
// never crosses a memory page, so the read stays in mapped memory); the terms of keys at or past
// lk are then meaningless and the caller drops those keys by the key bound. lk >= 1.
template <class T>
__device__ __forceinline__ u32x4_t mask_raw8(const AttnParams& p, long long rowoff, int key0, int lk) {
  const int k = p.m_key == 0 ? 0 : min(key0, max(lk - 1, 0) & ~7);
  if (p.mask_kind == 1) {
    const uint16_t* m = (const uint16_t*)p.mask + rowoff + k;
    if (p.m_key == 0) return (u32x4_t){(uint32_t)m[0], 0u, 0u, 0u};
    return *(const u32x4_t*)m;
  }
  const uint8_t* m = (const uint8_t*)p.mask + rowoff + k;
  if (p.m_key == 0) return (u32x4_t){(uint32_t)m[0], 0u, 0u, 0u};
  const u32x2_t v = *(const u32x2_t*)m;
  return (u32x4_t){v.x, v.y, 0u, 0u};
}

// The mask terms of those eight keys, in units of the raw scores: bias / scale for an additive
// mask, 0 (kept) or -inf (dropped) for a boolean one.
template <class T>
__device__ __forceinline__ void mask_apply8(const AttnParams& p, u32x4_t raw, float (&out)[8]) {
  if (p.mask_kind == 1) {
    if (p.m_key == 0) {
      const float x = Elt<T>::to_f32((uint16_t)raw.x) * p.inv_scale;
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = x;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float lo, hi;
        Elt<T>::unpack2(raw[e], lo, hi);
        out[2 * e] = lo * p.inv_scale;
        out[2 * e + 1] = hi * p.inv_scale;
      }
    }
  } else if (p.m_key == 0) {
    const float x = (raw.x & 0xffu) != 0 ? 0.f : -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = x;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = ((e < 4 ? raw.x : raw.y) >> (8 * (e & 3))) & 0xffu ? 0.f : -INFINITY;
  }
}

// The same 8 keys as one load in every form (used where the load is issued long before its use
// and copies are issued in between: a form that also writes zero words after its load makes the
// compiler wait for that load, and so for the copies, before the registers are reused).
// mask_block loads the aligned 16-byte block that holds the first needed element: with a
// contiguous key dim the row offset is a multiple of 8 and the base is aligned, so an additive
// piece is the whole block and a boolean piece one half of it; a key-broadcast mask (m_key == 0)
// has its one element somewhere in the block. An aligned block never crosses a memory page, so the
// read stays in mapped memory. A piece that reaches past the row's last key lk - 1 is read as the
// row's last whole aligned piece instead (the one holding key lk - 1); the terms of keys at or
// past lk are then meaningless and the caller drops those keys by the key bound. lk >= 1.
// (Pointer arithmetic on the mask pointer throughout, so that the loads stay global loads.)
__device__ __forceinline__ const char* mask_addr(const AttnParams& p, long long rowoff, int key0, int lk) {
  const int k = p.m_key == 0 ? 0 : min(key0, max(lk - 1, 0) & ~7);
  return (const char*)p.mask + ((rowoff + k) << (p.mask_kind == 1 ? 1 : 0));
}
__device__ __forceinline__ u32x4_t mask_block(const AttnParams& p, long long rowoff, int key0, int lk) {
  const char* a = mask_addr(p, rowoff, key0, lk);
  return *(const u32x4_t*)(a - ((uintptr_t)a & 15));
}

// The mask terms of those eight keys from mask_block's bits (same rowoff, key0, lk), in units of
// the raw scores: bias / scale for an additive mask, 0 (kept) or -inf (dropped) for a boolean one.
template <class T>
__device__ __forceinline__ void mask_apply8_block(const AttnParams& p, u32x4_t blk, long long rowoff, int key0,
                                                  int lk, float (&out)[8]) {
  if (p.m_key == 0) {
    const int at = (int)((uintptr_t)mask_addr(p, rowoff, key0, lk) & 15);  // byte offset of the element
    const uint32_t word = at < 8 ? (at < 4 ? blk.x : blk.y) : (at < 12 ? blk.z : blk.w);
    const uint32_t e = word >> (8 * (at & 3));
    const float x = p.mask_kind == 1 ? Elt<T>::to_f32((uint16_t)e) * p.inv_scale : ((e & 0xffu) != 0 ? 0.f : -INFINITY);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = x;
  } else if (p.mask_kind == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lo, hi;
      Elt<T>::unpack2(blk[i], lo, hi);
      out[2 * i] = lo * p.inv_scale;
      out[2 * i + 1] = hi * p.inv_scale;
    }
  } else {
    const bool upper = ((uintptr_t)mask_addr(p, rowoff, key0, lk) & 8) != 0;
    const uint32_t w0 = upper ? blk.z : blk.x, w1 = upper ? blk.w : blk.y;
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = ((i < 4 ? w0 : w1) >> (8 * (i & 3))) & 0xffu ? 0.f : -INFINITY;
  }
}

// Element offset of the attn_mask row of (slice s, query head h, query i).
__device__ __forceinline__ long long mask_row(const AttnParams& p, int s, int h, int i) {
  return (long long)s * p.m_batch + (long long)h * p.m_head + (long long)i * p.m_row;
}

}  // namespace ffpa
