// FP8 forward for large head dims on gfx950 (the ffpa-attn user guide, "Backends Overview":
// backend table and notes -- FP8 attention is a forward-only path that takes fp16/bf16
// activations and quantizes Q, K and V inside the library).
//
// The guide's FP8 page (scale granularity, formats) is not part of the pages; the reading taken
// here is the plainest one that the rest supports:
//   * OCP e4m3 (the gfx950 MFMA format, max 448) for Q, K, V and P;
//   * one scale per (batch, head) and tensor: x8 = e4m3(x * (448 / amax)), rounded to nearest
//     even from fp32, with amax the largest |x| of that head's rows (0 gives a zero tensor);
//   * S = (Q8 K8^T) * amax_q * amax_k / 448^2 (times the softmax scale); the softmax keeps an exact
//     running row max, so P = exp(S - max) is in [0, 1] and P8 = e4m3(P * 448);
//   * O = (sum_j P8_ij V8_j) * amax_v / 448^2 / l_i with l_i = sum_j P_ij (fp32, unquantized), and
//     LSE = max + log l, both as in the bf16/fp16 forward.
//
// Pipeline: a pre-pass finds the per-head amax of Q, K and V (one atomic max per block on the fp32
// bits, which order like the values for non-negative floats) and writes K8 row-major and V8
// transposed (one row per head-dim column, keys contiguous, padded to 64) into a caller
// workspace. The forward kernel then streams 64-key tiles of K8 and V8^T (32 KB each at D = 512,
// the LDS of a 32-key bf16 tile) and runs v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales.
// It splits KEYS, not the head dim, between the two waves of a pair: each wave holds its 32
// queries' Q8 for the whole head dim in registers (64 VGPRs at D = 512) and forms S for one
// 32-key half of the tile with no partial-sum exchange; the pair shares the tile max (one float
// per query through LDS) and its P8 halves (1 KB per wave), and each wave then multiplies P V for
// its half of the head dim. Waves 0-3 and 4-7 run one slot apart (one multiplies while the other
// does the softmax), as in the bf16/fp16 forward. Above D = 512 Q8 of the whole head dim no longer
// fits beside a wave's share of O, and a second kernel (below) splits S over head-dim halves.
#include "ffpa_device.h"
#include "ffpa_params.h"

namespace ffpa {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Two fp32 values to OCP e4m3 (round to nearest even) in bytes 0 and 1 of the result.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  return e4m3x2(a, b) | (e4m3x2(c, d) << 16);
}

// ---- pre-pass -------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) ffpa_fp8_amax_init_kernel(float* amax, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) amax[i] = 0.f;
}

// amax[head] = max |x| over a head's n * d values: grid (chunks of 256K values, heads); each thread
// keeps four 16-byte loads in flight, then one atomic max per workgroup (the fp32 bits of
// non-negative values order like the values).
constexpr int kAmaxChunk = 1 << 18;
template <class T>
__global__ void __launch_bounds__(256) ffpa_fp8_amax_kernel(const uint16_t* x, long long head_elems, float* amax) {
  __shared__ float wmax[4];
  const int head = blockIdx.y;
  const long long beg = (long long)blockIdx.x * kAmaxChunk;
  const long long end = min(beg + kAmaxChunk, head_elems);
  const uint16_t* base = x + (long long)head * head_elems;
  float m = 0.f;
  for (long long i = beg + 8 * threadIdx.x; i < end; i += 4 * 8 * 256) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long long iu = i + (long long)u * 8 * 256;
      v[u] = iu < end ? *(const u32x4_t*)(base + iu) : (u32x4_t){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float lo, hi;
        Elt<T>::unpack2(v[u][e], lo, hi);
        m = fmaxf(m, fmaxf(fabsf(lo), fabsf(hi)));
      }
  }
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax((unsigned int*)(amax + head), __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
}

__device__ __forceinline__ float quant_factor(float amax) { return amax > 0.f ? 448.0f / amax : 0.f; }

// K8[head][row][d] = e4m3(K * 448 / amax): 16 values per thread.
template <class T>
__global__ void __launch_bounds__(256) ffpa_fp8_quant_rows_kernel(const uint16_t* x, uint8_t* x8, const float* amax,
                                                                  long long head_elems) {
  const int head = blockIdx.y;
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 16;
  if (i >= head_elems) return;
  const float f = quant_factor(amax[head]);
  const uint16_t* src = x + (long long)head * head_elems + i;
  uint32_t w[4];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const u32x4_t v = *(const u32x4_t*)(src + 8 * half);
    float a[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) Elt<T>::unpack2(v[e], a[2 * e], a[2 * e + 1]);
    w[2 * half] = e4m3x4(a[0] * f, a[1] * f, a[2] * f, a[3] * f);
    w[2 * half + 1] = e4m3x4(a[4] * f, a[5] * f, a[6] * f, a[7] * f);
  }
  *(u32x4_t*)(x8 + (long long)head * head_elems + i) = (u32x4_t){w[0], w[1], w[2], w[3]};
}

// V8T[head][d][key] = e4m3(V[head][key][d] * 448 / amax) for keys < rows, 0 up to the padded row
// length np (a multiple of 64): one 64-key x 64-column tile per block, transposed through LDS.
template <class T>
__global__ void __launch_bounds__(256) ffpa_fp8_quant_vt_kernel(const uint16_t* v, uint8_t* v8t, const float* amax,
                                                                int rows, int d, int np) {
  __shared__ uint8_t t[64][64 + 4];
  const int head = blockIdx.z;
  const int k0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  const float f = quant_factor(amax[head]);
  const uint16_t* src = v + (long long)head * rows * d;
  // load: thread (key kr, 16-column group cq) converts 16 values
  {
    const int kr = threadIdx.x >> 2, cq = threadIdx.x & 3;
    const int key = k0 + kr;
    const int dc = d0 + 16 * cq;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (key < rows && dc < d) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const u32x4_t x = *(const u32x4_t*)(src + (long long)key * d + dc + 8 * half);
        float a[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) Elt<T>::unpack2(x[e], a[2 * e], a[2 * e + 1]);
        w[2 * half] = e4m3x4(a[0] * f, a[1] * f, a[2] * f, a[3] * f);
        w[2 * half + 1] = e4m3x4(a[4] * f, a[5] * f, a[6] * f, a[7] * f);
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) t[kr][16 * cq + e] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
  }
  __syncthreads();
  // store: thread (column dr, 16-key group kq) writes 16 keys of one column row
  {
    const int dr = threadIdx.x >> 2, kq = threadIdx.x & 3;
    const int dcol = d0 + dr;
    if (dcol < d) {
      uint32_t w[4];
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        w[e4] = (uint32_t)t[16 * kq + 4 * e4][dr] | ((uint32_t)t[16 * kq + 4 * e4 + 1][dr] << 8) |
                ((uint32_t)t[16 * kq + 4 * e4 + 2][dr] << 16) | ((uint32_t)t[16 * kq + 4 * e4 + 3][dr] << 24);
      *(u32x4_t*)(v8t + ((long long)head * d + dcol) * np + k0 + 16 * kq) = (u32x4_t){w[0], w[1], w[2], w[3]};
    }
  }
}

// ---- forward kernel -------------------------------------------------------------------------
template <int NDB>
struct Fp8Cfg {
  static constexpr int NW = 8;
  static constexpr int DW = NDB * 32;          // head-dim columns of O per wave (half the head)
  static constexpr int DPAD = 2 * DW;          // padded head dim (multiple of 64)
  static constexpr int KS = DPAD / 64;         // 64-wide k-steps of S over the head dim
  static constexpr int KT = 64;                // keys per tile
  static constexpr int KROW = 512;             // K8 tile row stride in LDS (bytes)
  static constexpr int KTILE = KT * KROW;      // 32 KB
  static constexpr int VROWS = DPAD;           // V8^T tile rows (copies of 16 rows x 4 waves)
  static constexpr int VTILE = VROWS * KT;     // V8^T tile: VROWS rows x 64 keys
  static constexpr int P8_OFF = 2 * KTILE + 2 * VTILE;
  static constexpr int XM_OFF = P8_OFF + NW * 1024;  // per wave: 32 queries x 32 keys of P8
  static constexpr int LDS = XM_OFF + NW * 32 * 4;   // per wave: tile max, then l, per query
  static constexpr int KCOPY4 = KTILE / 1024 / 4;  // 1 KB copies per wave of the copying group
  static constexpr int VCOPY4 = VTILE / 1024 / 4;
  static_assert(DPAD <= 512 && LDS <= 160 * 1024 && VTILE % 4096 == 0, "LDS budget");
};

// Scheduling pin for N MFMAs with R LDS reads each, after PRE other LDS reads: the PRE reads and
// those of the first AHEAD MFMAs, then one MFMA and the reads of a later one alternately, then the
// last AHEAD MFMAs (mask bits: 0x008 MFMA, 0x100 LDS read).
template <int N, int AHEAD, int R, int PRE>
__device__ __forceinline__ void pin_fp8_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, PRE + AHEAD * R, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// LDS operand reads issued ahead of their MFMA in the product runs.
constexpr int FP8_AHEAD = 2;

// Opaque register use (empty asm): the value is materialised here (see opaque_v for the other
// direction).
__device__ __forceinline__ void keep_here(const f32x16_t& x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ f32x16_t mma_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  // unit block scales (E8M0 127 = 2^0); A and B in OCP e4m3 (format 0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <class T, int NDB>
__global__ void __launch_bounds__(512, 2) ffpa_fwd_fp8_kernel(AttnParams p, const float* amax_q,
                                                              const float* amax_k, const float* amax_v,
                                                              const uint8_t* k8, const uint8_t* v8t, int np) {
  using C = Fp8Cfg<NDB>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  lds_t* smem = (lds_t*)smem_raw;
  auto kbuf = [&](int b) { return smem + b * C::KTILE; };
  auto vbuf = [&](int b) { return smem + 2 * C::KTILE + b * C::VTILE; };
  lds_t* const p8buf = smem + C::P8_OFF;
  lds_t* const xmbuf = smem + C::XM_OFF;

  const int L = blockIdx.x;
  const int item = xcd_item(L, gridDim.x, false, 0, 0);
  if (item >= p.total) return;
  const HeadTile ht = head_tile(item, p.ntiles, p.hq, p.group, true);
  int t = ht.t;
  const int h = ht.h;
  const int s = ht.s;
  if (p.causal) t = p.ntiles - 1 - t;
  const int qt0 = t * 128;
  if (qt0 >= p.nq) return;
  const int kvh = h / p.group;
  const int hq_flat = s * p.hq + h, hk_flat = s * p.hkv + kvh;

  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int rg = w >> 1;
  const int cg = w & 1;
  const int qw0 = qt0 + rg * 32;
  const int off = p.nkv - p.nq;
  int kend = p.nkv;
  if (p.causal) kend = min(kend, qt0 + 128 + off);
  const int ntk = kend > 0 ? (kend + C::KT - 1) / C::KT : 0;

  const float fq = quant_factor(amax_q[hq_flat]);
  const float ak = amax_k[hk_flat], av = amax_v[hk_flat];
  // S in log2 units from the e4m3 products: times amax_q amax_k / 448^2, the scale and log2(e).
  const float sdq = p.scale_log2 * (amax_q[hq_flat] / 448.0f) * (ak / 448.0f);

  // Q8 of this lane's query for the whole head dim: k-step kb, lane half h holds logical dims
  // 64 kb + 32 h .. + 31 (the same assignment as the K8 A operand, so the MFMA pairs them).
  i32x8_t q8[C::KS];
  {
    const int qi = min(qw0 + l32, p.nq - 1);
    const uint16_t* qrow = (const uint16_t*)p.q + ((long long)s * p.hq + h) * p.q_head + (long long)qi * p.q_row;
#pragma unroll
    for (int kb = 0; kb < C::KS; ++kb) {
      uint32_t wv[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = 64 * kb + 32 * hh + 8 * g;
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (dim < p.d) {
          const u32x4_t x = *(const u32x4_t*)(qrow + dim);
#pragma unroll
          for (int e = 0; e < 4; ++e) Elt<T>::unpack2(x[e], a[2 * e], a[2 * e + 1]);
        }
        wv[2 * g] = e4m3x4(a[0] * fq, a[1] * fq, a[2] * fq, a[3] * fq);
        wv[2 * g + 1] = e4m3x4(a[4] * fq, a[5] * fq, a[6] * fq, a[7] * fq);
      }
      q8[kb] = (i32x8_t){(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3], (int)wv[4], (int)wv[5], (int)wv[6], (int)wv[7]};
    }
  }

  // ---- copies. K8 tile: 64 rows x D bytes into 512-byte LDS rows, 16-byte chunk c of row r at
  // physical chunk c ^ (r & 15) (chunks past the head dim clamped); one 1 KB copy = two rows.
  // V8^T tile: VROWS rows x 64 keys, chunk c of row r at c ^ ((r >> 2) & 3) (rows past the head
  // dim clamped); one copy = 16 rows. Each copy is split over the four waves of one group.
  const int grp = w >> 2, wg = w & 3;
  const int dch = p.d >> 4;
  const long long k8_head = (long long)hk_flat * p.nkv * p.d;
  const long long v8_head = (long long)hk_flat * p.d * np;
  const i32x4_t krs = make_rsrc(k8 + k8_head, (uint32_t)min((long long)p.nkv * p.d, (long long)0xFFFFFFF0));
  const i32x4_t vrs = make_rsrc(v8t + v8_head, (uint32_t)min((long long)p.d * np, (long long)0xFFFFFFF0));
  // rows 2 (wg + 4 c) + h: the swizzle (row & 15) takes two values, for even and odd c
  const int kch0 = min(l32 ^ (2 * wg + hh), dch - 1) << 4;
  const int kch1 = min(l32 ^ (2 * wg + hh + 8), dch - 1) << 4;
  // copy tile j into the buffer of tile jb
  // (kb0/kb1 are laundered per slot by the caller, so the compiler does not keep one offset per
  // copy live across the loop)
  auto copy_k = [&](int j, int jb, int c, int kb0, int kb1) {
    const int r0 = 2 * (wg + 4 * c);
    const int key = min(j * C::KT + r0 + hh, p.nkv - 1);
    dma16_buf(krs, key * p.d + ((c & 1) ? kb1 : kb0), 0, kbuf(jb & 1) + r0 * C::KROW);
  };
  // rows 16 (wg + 4 c) + lane / 4: the swizzle ((row >> 2) & 3) is (lane >> 4) & 3 for every c
  const int vch = ((lane & 3) ^ ((lane >> 4) & 3)) << 4;
  auto copy_v = [&](int j, int jb, int c, int vr, int vc) {
    const int r0 = 16 * (wg + 4 * c);
    const int row = min(r0 + vr, p.d - 1);
    dma16_buf(vrs, row * np + vc + j * C::KT, 0, vbuf(jb & 1) + r0 * C::KT);
  };

  // ---- operand addresses
  // S^T block of this wave: keys 32 cg + row_perm(n) of the tile (A rows), so C register r holds key
  // 32 cg + c_row(r, h); lane reads 32 bytes = chunks 4 kb + 2 h, + 1 of its key row.
  // The row base is a multiple of 512, so the swizzled chunk is one per-lane base XOR a constant.
  const int krow = 32 * cg + row_perm(l32);
  // (the lane half's chunk offset 2 h is folded into the lane base; the tile base is a multiple of
  // 512, so adding it and XOR-ing the chunk commute, and the per-read XOR is an immediate)
  const uint32_t klane = krow * C::KROW + (((krow & 15) ^ (2 * hh)) << 4);
  auto k_addr = [&](uint32_t tile_lane, int kb, int part) -> uint32_t {
    return tile_lane ^ ((4 * kb + part) << 4);
  };
  // V8^T (A of O^T += V^T P^T): row d = cg DW + 32 db + n, keys 32 h .. + 31 = chunks 2 h, + 1; the
  // swizzle depends on n only.
  // Per lane two byte offsets (part 0 and 1); the column block adds an immediate.
  const int vsw = (l32 >> 2) & 3;
  const int vlane0 = (cg * C::DW + l32) * C::KT + (((2 * hh) ^ vsw) << 4);
  const int vlane1 = (cg * C::DW + l32) * C::KT + (((2 * hh + 1) ^ vsw) << 4);
  // P8 of wave (rg, c): [query n][32 keys], 32-byte rows whose two chunks swap for n & 8.
  auto p8_off = [&](int wave, int n, int key) -> int {
    return wave * 1024 + n * 32 + ((((key >> 4) ^ ((n >> 3) & 1))) << 4) + (key & 15);
  };
  auto rd8 = [&](uint32_t a0, uint32_t a1) -> i32x8_t {
    const u32x4_t x = lds_read_b128_at(a0), y = lds_read_b128_at(a1);
    return (i32x8_t){(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = (f32x16_t){};
  f32x16_t sacc = (f32x16_t){};
  float mref = -INFINITY, lsum = 0.f, mw = -INFINITY;
  const int qi = qw0 + l32;
  const int lim_row = p.causal ? min(qi + off, p.nkv - 1) : p.nkv - 1;

  // Multiply slot of step j: S^T of tile j and O^T += V8^T P8^T of tile j - 1, alternating so that
  // no two dependent MFMAs are adjacent; then (group 0) the copy of K of tile j + 1, and the scale,
  // mask and tile max of this wave's 32 keys, written for the partner. At j = 0 the P8 slots and
  // the second V buffer hold zeros, so the P V product adds exact zeros; at j = ntk the scores are
  // formed (on a stale tile) but not used.
  auto m_slot = [&](int j) {
    // opaque per slot, so the per-read addresses are formed at their use instead of being kept
    // live across the loop
    const uint32_t kt = (uint32_t)opaque_v((int)(lds_addr(kbuf(j & 1)) + klane));
    const lds_t* const vt0 = vbuf((j + 1) & 1) + opaque_v(vlane0);
    const lds_t* const vt1 = vbuf((j + 1) & 1) + opaque_v(vlane1);
    // P8^T B operand: lane (h, n) = query n, keys 32 h .. + 31 of tile j - 1, i.e. the P8 row of
    // wave (rg, h); the V8^T A operand holds the same keys in the same byte order.
    const uint32_t pb = lds_addr(p8buf) + p8_off(2 * rg + hh, l32, 0);
    const i32x8_t bop = rd8(pb, pb ^ 16);
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
      const u32x4_t x = lds_read_b128(vt0, 32 * i * C::KT), y = lds_read_b128(vt1, 32 * i * C::KT);
      const i32x8_t a = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      oacc[i] = mma_fp8(a, bop, oacc[i]);
    }
    pin_fp8_pipeline<NDB, FP8_AHEAD, 2, 2>();
    // opaque uses: the products stay in this slot (otherwise they are sunk towards their next use,
    // past the barrier, where their operands occupy registers the softmax needs)
#pragma unroll
    for (int i = 0; i < NDB; ++i) keep_here(oacc[i]);
    __builtin_amdgcn_sched_barrier(0);
    sacc = (f32x16_t){};
#pragma unroll
    for (int i = 0; i < NDB; ++i) sacc = mma_fp8(rd8(k_addr(kt, i, 0), k_addr(kt, i, 1)), q8[i], sacc);
    pin_fp8_pipeline<NDB, FP8_AHEAD, 2, 0>();
    keep_here(sacc);
    if (grp == 0) {
      const int jn = min(j + 1, ntk - 1);
      const int kb0 = opaque_v(kch0), kb1 = opaque_v(kch1);
#pragma unroll
      for (int c = 0; c < C::KCOPY4; ++c) copy_k(jn, j + 1, c, kb0, kb1);
    }
    // key of register r: j KT + 32 cg + c_row(r, h), and c_row(r, h) = c_row(r, 0) + 8 h, so one
    // per-lane bound against immediates
    const int klim = lim_row - (j * C::KT + 32 * cg + 8 * hh);
    mw = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = sacc[r] * sdq;
      if (c_row(r, 0) > klim) v = -INFINITY;
      sacc[r] = v;
      mw = fmaxf(mw, v);
    }
    mw = half_max(mw);
    if (hh == 0) *(__attribute__((address_space(3))) float*)(xmbuf + (w * 32 + l32) * 4) = mw;
  };

  // Softmax slot of step j: (group 1) the copy of V of tile j + 1; the pair's tile max, the exact
  // running max (rescaling O and l when it grows), P = exp2(S - max) in [0, 1] and
  // P8 = e4m3(448 P) for the partner.
  auto e_slot = [&](int j) {
    if (grp == 1) {
      const int jn = min(j + 1, ntk - 1);
      const int vr = opaque_v(lane >> 2), vc = opaque_v(vch);
#pragma unroll
      for (int c = 0; c < C::VCOPY4; ++c) copy_v(jn, j + 1, c, vr, vc);
    }
    const float mpart = *(const __attribute__((address_space(3))) float*)(xmbuf + ((w ^ 1) * 32 + l32) * 4);
    // the pair's tile max: the same commutative max in both waves
    const float mt = cg == 0 ? fmaxf(mw, mpart) : fmaxf(mpart, mw);
    const float mnew = fmaxf(mref, mt);
    if (__any(mnew > mref)) {
      const float alpha = mnew > mref ? (mref == -INFINITY ? 0.f : fast_exp2(mref - mnew)) : 1.0f;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      mref = mnew;
    }
    // a row with no finite score yet keeps P = 0
    const float mu = mref == -INFINITY ? 0.f : mref;
    // keys 8 h + 0..7 (registers 0..7) and 16 + 8 h + 0..7 (8..15) of this wave's 32 as bytes
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t wd[2];
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4) {
        float e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          e[u] = fast_exp2(sacc[8 * half + 4 * q4 + u] - mu);
          lsum += e[u];
        }
        wd[q4] = e4m3x4(e[0] * 448.f, e[1] * 448.f, e[2] * 448.f, e[3] * 448.f);
      }
      *(__attribute__((address_space(3))) u32x2_t*)(p8buf + p8_off(w, l32, 16 * half + 8 * hh)) =
          (u32x2_t){wd[0], wd[1]};
    }
  };

  // Two-group schedule. Waves 0-3 (row groups 0, 1) and 4-7 (row groups 2, 3) run one slot apart,
  // so in every slot one wave of each SIMD multiplies while the other does the softmax:
  //   slot 2j:     group 0 multiplies (S_j, P_{j-1} V_{j-1}) | group 1 softmax of tile j - 1
  //   slot 2j + 1: group 0 softmax of tile j                  | group 1 multiplies (S_j, P_{j-1} V_{j-1})
  // for j = 0 .. ntk (group 1's slot 0 only copies). Buffers (two each): K_{j+1} replaces K_{j-1}
  // (last read in slot 2j - 1) and is copied by group 0 in slot 2j; V_j replaces V_{j-2} (last read
  // in slot 2j - 1) and is copied by group 1 in slot 2j. The copying waves complete their copies
  // before the barrier that ends slot 2j + 1. Past the last tile the copies repeat tile ntk - 1
  // into the free buffer, so every slot has the same shape. A wave's tile max and P8 are read by
  // its partner (same group) in the next slot and rewritten two slots later.
  if (ntk > 0) {
    // zero P8 slots and the second V buffer (read by the first multiply slot), then K_0
    {
      const u32x4_t z = {0u, 0u, 0u, 0u};
      for (int o = threadIdx.x * 16; o < C::VTILE; o += 512 * 16) lds_write_b128(vbuf(1), o, z);
      lds_write_b128(p8buf, threadIdx.x * 16, z);
    }
    if (grp == 0) {
#pragma unroll
      for (int c = 0; c < C::KCOPY4; ++c) copy_k(0, 0, c, kch0, kch1);
    }
    wait_vmcnt<0>();
    lds_barrier();
    if (grp == 1) {
#pragma unroll
      for (int c = 0; c < C::VCOPY4; ++c) copy_v(0, 0, c, lane >> 2, vch);
      lds_barrier();
    }
    // (the scheduling barriers keep each slot's MFMAs on its side of the workgroup barrier)
    for (int j = 0; j < ntk; ++j) {
      m_slot(j);
      if (grp == 1) wait_vmcnt<0>();  // V_j
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      e_slot(j);
      if (grp == 0) wait_vmcnt<0>();  // K_{j+1}
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    m_slot(ntk);
    wait_vmcnt<0>();
    lds_barrier();
    if (grp == 0) {
      wait_vmcnt<0>();
      lds_barrier();
    }
  }

  // ---- epilogue: the pair's l (each wave summed its own keys), O = O^T * amax_v / 448^2 / l.
  // Both groups have passed the same number of barriers; the partner read this wave's exchange
  // slot (its last tile max) before the last one.
  const float lw = half_sum(lsum);
  if (hh == 0) *(__attribute__((address_space(3))) float*)(xmbuf + (w * 32 + l32) * 4) = lw;
  lds_barrier();
  const float lp = *(const __attribute__((address_space(3))) float*)(xmbuf + ((w ^ 1) * 32 + l32) * 4);
  const float lt = cg == 0 ? lw + lp : lp + lw;
  const float inv = lt > 0.f ? (av / (448.0f * 448.0f)) / lt : 0.f;
  // O through LDS, whole rows per store (the block: 4 row groups x 2 head-dim halves)
  wait_vmcnt<0>();
  store_block_rows<T, false, 4, 2, 1, NDB, C::LDS>(
      smem, reinterpret_cast<const f32x16_t(&)[1][NDB]>(oacc), inv,
      (uint16_t*)p.o + ((long long)s * p.hq + h) * p.o_head + (long long)qt0 * p.o_row, p.o_row, p.nq - qt0, p.d);
  if (qi < p.nq && cg == 0 && hh == 0)
    p.lse[(long long)s * p.lse_batch + (long long)h * p.lse_head + qi] =
        lt > 0.f ? (mref + fast_log2(lt)) * kLn2 : -INFINITY;
}

// ---- forward kernel for D > 512 --------------------------------------------------------------
// The same FP8 algorithm at head dims 544..1024, where a wave can no longer hold Q8 for the whole
// head dim beside half of O. Eight waves (two per SIMD) own 64 queries as 2 row groups x 4; within
// a row group, wave (kb, dh) forms the partial S^T of key block kb (32 of the tile's 64 keys) over
// head-dim half dh (Q8 of that half in registers: 64 registers at D = 1024) and owns a quarter of
// O^T (128 registers). The two halves of a key block are combined by a reduce-scatter (the A rows
// of half dh are rotated by 16 dh, so registers 0..7 hold the 16 keys the wave finishes), the four
// waves share their 16-key maxima for the exact running max, and each writes the e4m3 P of its keys
// into the row group's P8 block, from which every wave multiplies its quarter: O^T += V8^T P8^T
// over all 64 keys. K8 (64 keys x 1 KB rows, the two head-dim halves at 0 and 512 bytes) and V8^T
// (D rows x 64 keys) tiles are 64 KB each and single-buffered; every step runs, all waves in step:
//   S partials (V_j copies spread over them) | partner's keys out | barrier | own keys in, maxima
//   out | barrier | running max, P8 out | wait V_j, barrier | O^T += V8^T P8^T (K_{j+1} copies)
template <int NQ>
struct Fp8WideCfg {
  static constexpr int NW = 8;
  static constexpr int DQW = NQ * 32;          // head-dim columns of O per wave (a quarter)
  static constexpr int DPAD = 4 * DQW;         // padded head dim (multiple of 128)
  static constexpr int DH = DPAD / 2;          // head-dim half of the S partials
  static constexpr int KSH = DH / 64;          // 64-wide k-steps over a half (= NQ)
  static constexpr int KT = 64;                // keys per tile
  static constexpr int KROW = 1024;            // K8 row in LDS: half 0 at byte 0, half 1 at 512
  static constexpr int KTILE = KT * KROW;      // 64 KB
  static constexpr int VTILE = DPAD * KT;      // V8^T tile: DPAD rows x 64 keys
  static constexpr int XS_OFF = KTILE + VTILE;       // S partials: per wave 2 KB (the partner's keys)
  static constexpr int P8_OFF = XS_OFF + NW * 2048;  // per row group: 32 queries x 64 keys of P8
  static constexpr int XM_OFF = P8_OFF + 2 * 2048;   // per wave: 16-key maximum, then l, per query
  static constexpr int LDS = XM_OFF + NW * 32 * 4;
  static constexpr int KCOPY = KTILE / 1024 / NW;    // 1 KB copies per wave of a K8 tile (one row each)
  static constexpr int VCOPY = VTILE / 1024 / NW;    // of a V8^T tile (16 rows each)
  static_assert(DPAD > 512 && DPAD <= 1024 && DH <= 512 && LDS <= 160 * 1024 && KSH == NQ, "LDS budget");
};

template <class T, int NQ>
__global__ void __launch_bounds__(512, 2) ffpa_fwd_fp8_wide_kernel(AttnParams p, const float* amax_q,
                                                                   const float* amax_k, const float* amax_v,
                                                                   const uint8_t* k8, const uint8_t* v8t, int np) {
  using C = Fp8WideCfg<NQ>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  lds_t* smem = (lds_t*)smem_raw;
  lds_t* const kbuf = smem;
  lds_t* const vbuf = smem + C::KTILE;
  lds_t* const xsbuf = smem + C::XS_OFF;
  lds_t* const p8buf = smem + C::P8_OFF;
  lds_t* const xmbuf = smem + C::XM_OFF;

  const int L = blockIdx.x;
  const int item = xcd_item(L, gridDim.x, false, 0, 0);
  if (item >= p.total) return;
  const HeadTile ht = head_tile(item, p.ntiles, p.hq, p.group, true);
  int t = ht.t;
  const int h = ht.h;
  const int s = ht.s;
  if (p.causal) t = p.ntiles - 1 - t;
  const int qt0 = t * 64;
  if (qt0 >= p.nq) return;
  const int kvh = h / p.group;
  const int hq_flat = s * p.hq + h, hk_flat = s * p.hkv + kvh;

  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int rg = w >> 2;
  const int kb = (w >> 1) & 1;  // key block of the tile
  const int dh = w & 1;         // head-dim half of the S partials
  const int oq = w & 3;         // O quarter
  const int qw0 = qt0 + rg * 32;
  const int off = p.nkv - p.nq;
  int kend = p.nkv;
  if (p.causal) kend = min(kend, qt0 + 64 + off);
  const int ntk = kend > 0 ? (kend + C::KT - 1) / C::KT : 0;

  const float fq = quant_factor(amax_q[hq_flat]);
  const float av = amax_v[hk_flat];
  const float sdq = p.scale_log2 * (amax_q[hq_flat] / 448.0f) * (amax_k[hk_flat] / 448.0f);

  // Q8 of this lane's query over head-dim half dh: k-step kk, lane half h holds dims
  // dh DH + 64 kk + 32 h .. + 31.
  i32x8_t q8[C::KSH];
  {
    const int qi = min(qw0 + l32, p.nq - 1);
    const uint16_t* qrow = (const uint16_t*)p.q + ((long long)s * p.hq + h) * p.q_head + (long long)qi * p.q_row;
#pragma unroll
    for (int kk = 0; kk < C::KSH; ++kk) {
      uint32_t wv[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = dh * C::DH + 64 * kk + 32 * hh + 8 * g;
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (dim < p.d) {
          const u32x4_t x = *(const u32x4_t*)(qrow + dim);
#pragma unroll
          for (int e = 0; e < 4; ++e) Elt<T>::unpack2(x[e], a[2 * e], a[2 * e + 1]);
        }
        wv[2 * g] = e4m3x4(a[0] * fq, a[1] * fq, a[2] * fq, a[3] * fq);
        wv[2 * g + 1] = e4m3x4(a[4] * fq, a[5] * fq, a[6] * fq, a[7] * fq);
      }
      q8[kk] = (i32x8_t){(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3], (int)wv[4], (int)wv[5], (int)wv[6], (int)wv[7]};
    }
  }

  // ---- copies. K8 row r: 64 physical 16-byte chunks; physical chunk pc holds logical chunk
  // u = pc ^ (r & 15), i.e. chunk u % 32 of head-dim half u / 32 (padding and chunks past the head
  // dim hold clamped duplicates); copy c of wave w is row w + 8 c. V8^T rows r0 .. r0 + 15
  // (r0 = 16 (w + 8 c)), chunk c of row r at c ^ ((r >> 2) & 3), rows past the head dim clamped.
  const int dch = p.d >> 4;
  const long long k8_head = (long long)hk_flat * p.nkv * p.d;
  const long long v8_head = (long long)hk_flat * p.d * np;
  const i32x4_t krs = make_rsrc(k8 + k8_head, (uint32_t)min((long long)p.nkv * p.d, (long long)0xFFFFFFF0));
  const i32x4_t vrs = make_rsrc(v8t + v8_head, (uint32_t)min((long long)p.d * np, (long long)0xFFFFFFF0));
  auto copy_k = [&](int j, int c) {
    const int r = w + C::NW * c;
    const int key = min(j * C::KT + r, p.nkv - 1);
    const int u = fresh_lane_id() ^ (r & 15);
    const int ch = min((u >> 5) * (C::DH / 16) + min(u & 31, C::DH / 16 - 1), dch - 1) << 4;
    lds_t* d = (lds_t*)(uintptr_t)opaque_s((uint32_t)(uintptr_t)(kbuf + r * C::KROW));
    dma16_buf(krs, key * p.d + ch, 0, d);
  };
  auto copy_v = [&](int j, int c) {
    const int r0 = 16 * (w + C::NW * c);
    const int ln = fresh_lane_id();
    const int row = min(r0 + (ln >> 2), p.d - 1);
    const int vc = ((ln & 3) ^ ((ln >> 4) & 3)) << 4;
    lds_t* d = (lds_t*)(uintptr_t)opaque_s((uint32_t)(uintptr_t)(vbuf + r0 * C::KT));
    dma16_buf(vrs, row * np + vc + j * C::KT, 0, d);
  };
  auto spread_k = [](int n, int c) { return (c * n) / C::KCOPY; };
  auto spread_v = [](int n, int c) { return (c * n) / C::VCOPY; };

  // ---- operand addresses. S^T A rows: tile row 32 kb + (row_perm(n) ^ 16 dh); lane reads 32
  // bytes of its half's chunks 32 dh + 4 kk + 2 h, + 1 (the half's base is 16-chunk aligned, so
  // the swizzle is one per-lane base XOR a constant).
  const int krow = 32 * kb + (row_perm(l32) ^ (16 * dh));
  const uint32_t klane = krow * C::KROW + ((32 * dh) << 4) + (((krow & 15) ^ (2 * hh)) << 4);
  auto k_addr = [&](uint32_t tile_lane, int kk, int part) -> uint32_t { return tile_lane ^ ((4 * kk + part) << 4); };
  // V8^T (A of O^T += V8^T P8^T): row d = oq DQW + 32 i + n, keys 32 h .. + 31 = chunks 2 h, + 1.
  const int vsw = (l32 >> 2) & 3;
  const int vlane0 = (oq * C::DQW + l32) * C::KT + (((2 * hh) ^ vsw) << 4);
  const int vlane1 = (oq * C::DQW + l32) * C::KT + (((2 * hh + 1) ^ vsw) << 4);
  // P8 block of the row group: [query n][64 keys], the 16-byte chunk index XOR-ed with (n >> 1) & 3.
  auto p8_off = [&](int n, int key) -> int { return rg * 2048 + n * 64 + ((((key >> 4) ^ (n >> 1)) & 3) << 4) + (key & 15); };
  auto rd8 = [&](uint32_t a0, uint32_t a1) -> i32x8_t {
    const u32x4_t x = lds_read_b128_at(a0), y = lds_read_b128_at(a1);
    return (i32x8_t){(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  };

  f32x16_t oacc[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) oacc[i] = (f32x16_t){};
  float mref = -INFINITY, lsum = 0.f;
  const int qi = qw0 + l32;
  const int lim_row = p.causal ? min(qi + off, p.nkv - 1) : p.nkv - 1;
  // This lane's 8 keys of the tile: 32 kb + 16 dh + 8 h + 0..7.
  const int kown = 32 * kb + 16 * dh + 8 * hh;

  if (ntk > 0) {
#pragma unroll
    for (int c = 0; c < C::KCOPY; ++c) copy_k(0, c);
  }
  wait_all();  // Q8's loads and K_0
  lds_barrier();

  for (int j = 0; j < ntk; ++j) {
    if (j > 0) {
      wait_vmcnt<0>();  // K_j (copied during the products of step j - 1)
      lds_barrier();    // every wave has finished step j - 1 (V_{j-1}, the P8 and exchange slots are free)
    }
    const uint32_t kt = (uint32_t)opaque_v((int)(lds_addr(kbuf) + klane));
    f32x16_t sacc = (f32x16_t){};
#pragma unroll
    for (int kk = 0; kk < C::KSH; ++kk) {
      sacc = mma_fp8(rd8(k_addr(kt, kk, 0), k_addr(kt, kk, 1)), q8[kk], sacc);
#pragma unroll
      for (int c = 0; c < C::VCOPY; ++c)
        if (kk == spread_v(C::KSH, c)) copy_v(j, c);
    }
    pin_fp8_pipeline<C::KSH, FP8_AHEAD, 2, 0>();
    // The partner's keys (registers 8..15) to its slot.
    lds_t* const xs_partner = xsbuf + (w ^ 1) * 2048;
    lds_write_f4(xs_partner, lane * 16, (f32x4_t){sacc[8], sacc[9], sacc[10], sacc[11]});
    lds_write_f4(xs_partner, 1024 + lane * 16, (f32x4_t){sacc[12], sacc[13], sacc[14], sacc[15]});
    lds_barrier();  // partial sums visible; K_j released
    const lds_t* const xs_mine = xsbuf + w * 2048;
    const f32x4_t pa = lds_read_f4(xs_mine, lane * 16), pb4 = lds_read_f4(xs_mine, 1024 + lane * 16);
    float sv[8];
    const int klim = lim_row - (j * C::KT + kown);
    float mw = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = (sacc[e] + (e < 4 ? pa[e] : pb4[e - 4])) * sdq;
      if (e > klim) v = -INFINITY;
      sv[e] = v;
      mw = fmaxf(mw, v);
    }
    mw = half_max(mw);
    if (hh == 0) *(__attribute__((address_space(3))) float*)(xmbuf + (w * 32 + l32) * 4) = mw;
    lds_barrier();  // the row group's 16-key maxima visible
    // Tile max over the four waves of the row group, in wave order (bit-identical in all four), the
    // exact running max (rescaling O and l when it grows), P = exp2(S - max) and P8 = e4m3(448 P).
    float mt = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c) mt = fmaxf(mt, *(const __attribute__((address_space(3))) float*)(xmbuf + ((4 * rg + c) * 32 + l32) * 4));
    const float mnew = fmaxf(mref, mt);
    if (__any(mnew > mref)) {
      const float alpha = mnew > mref ? (mref == -INFINITY ? 0.f : fast_exp2(mref - mnew)) : 1.0f;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < NQ; ++i) oacc[i] *= alpha;
      mref = mnew;
    }
    const float mu = mref == -INFINITY ? 0.f : mref;
    uint32_t wd[2];
#pragma unroll
    for (int q4 = 0; q4 < 2; ++q4) {
      float e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        e[u] = fast_exp2(sv[4 * q4 + u] - mu);
        lsum += e[u];
      }
      wd[q4] = e4m3x4(e[0] * 448.f, e[1] * 448.f, e[2] * 448.f, e[3] * 448.f);
    }
    *(__attribute__((address_space(3))) u32x2_t*)(p8buf + p8_off(l32, kown)) = (u32x2_t){wd[0], wd[1]};
    wait_vmcnt<0>();  // V_j
    lds_barrier();    // the row group's P8 visible
    // O^T += V8^T P8^T over the tile's 64 keys (lane half h: keys 32 h .. + 31), K_{j+1} copies
    // spread over the products (past the last tile: clamped, into a buffer no longer read).
    const uint32_t pbase = lds_addr(p8buf);
    const i32x8_t bop = rd8(pbase + p8_off(l32, 32 * hh), pbase + p8_off(l32, 32 * hh + 16));
    const lds_t* const vt0 = vbuf + opaque_v(vlane0);
    const lds_t* const vt1 = vbuf + opaque_v(vlane1);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const u32x4_t x = lds_read_b128(vt0, 32 * i * C::KT), y = lds_read_b128(vt1, 32 * i * C::KT);
      const i32x8_t a = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      oacc[i] = mma_fp8(a, bop, oacc[i]);
#pragma unroll
      for (int c = 0; c < C::KCOPY; ++c)
        if (i == spread_k(NQ, c)) copy_k(j + 1, c);
    }
    pin_fp8_pipeline<NQ, FP8_AHEAD, 2, 2>();
  }
  wait_vmcnt<0>();

  // ---- epilogue: l = the row group's four per-wave sums (wave order), O = O^T * amax_v / 448^2 / l.
  lds_barrier();  // every wave has read the row group's last maxima
  const float lw = half_sum(lsum);
  if (hh == 0) *(__attribute__((address_space(3))) float*)(xmbuf + (w * 32 + l32) * 4) = lw;
  lds_barrier();
  float lt = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) lt += *(const __attribute__((address_space(3))) float*)(xmbuf + ((4 * rg + c) * 32 + l32) * 4);
  const float inv = lt > 0.f ? (av / (448.0f * 448.0f)) / lt : 0.f;
  // O through LDS, whole rows per store (the block: 2 row groups x 4 head-dim quarters)
  wait_vmcnt<0>();
  store_block_rows<T, false, 2, 4, 1, NQ, C::LDS>(
      smem, reinterpret_cast<const f32x16_t(&)[1][NQ]>(oacc), inv,
      (uint16_t*)p.o + ((long long)s * p.hq + h) * p.o_head + (long long)qt0 * p.o_row, p.o_row, p.nq - qt0, p.d);
  if (qi < p.nq && oq == 0 && hh == 0)
    p.lse[(long long)s * p.lse_batch + (long long)h * p.lse_head + qi] =
        lt > 0.f ? (mref + fast_log2(lt)) * kLn2 : -INFINITY;
}

// Workspace: amax of Q (B Hq floats), K and V (B Hkv each), then K8 (B Hkv Nkv D bytes), then V8^T
// (B Hkv D np bytes, np = Nkv rounded up to 64); each part 256-byte aligned.
struct Fp8Layout {
  size_t amax, k8, v8t, total;
  int np;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Fp8Layout fp8_layout(int batch, int hq, int hkv, int nkv, int d) {
  Fp8Layout l{};
  l.np = (nkv + 63) / 64 * 64;
  l.amax = 0;
  l.k8 = align256((size_t)(batch * hq + 2 * batch * hkv) * 4);
  l.v8t = l.k8 + align256((size_t)batch * hkv * nkv * d);
  l.total = l.v8t + align256((size_t)batch * hkv * d * l.np);
  return l;
}

template <class T, int NDB>
static hipError_t launch_fp8_cfg(AttnParams p, char* ws, hipStream_t st) {
  const Fp8Layout lay = fp8_layout(p.batch, p.hq, p.hkv, p.nkv, p.d);
  float* amax_q = (float*)(ws + lay.amax);
  float* amax_k = amax_q + p.batch * p.hq;
  float* amax_v = amax_k + p.batch * p.hkv;
  uint8_t* k8 = (uint8_t*)(ws + lay.k8);
  uint8_t* v8t = (uint8_t*)(ws + lay.v8t);
  const int nam = p.batch * (p.hq + 2 * p.hkv);
  hipLaunchKernelGGL(ffpa_fp8_amax_init_kernel, dim3((nam + 255) / 256), dim3(256), 0, st, amax_q, nam);
  const long long qelems = (long long)p.nq * p.d, kvelems = (long long)p.nkv * p.d;
  hipLaunchKernelGGL(ffpa_fp8_amax_kernel<T>, dim3((unsigned)((qelems + kAmaxChunk - 1) / kAmaxChunk), p.batch * p.hq),
                     dim3(256), 0, st, (const uint16_t*)p.q, qelems, amax_q);
  hipLaunchKernelGGL(ffpa_fp8_amax_kernel<T>, dim3((unsigned)((kvelems + kAmaxChunk - 1) / kAmaxChunk), p.batch * p.hkv),
                     dim3(256), 0, st, (const uint16_t*)p.k, kvelems, amax_k);
  hipLaunchKernelGGL(ffpa_fp8_amax_kernel<T>, dim3((unsigned)((kvelems + kAmaxChunk - 1) / kAmaxChunk), p.batch * p.hkv),
                     dim3(256), 0, st, (const uint16_t*)p.v, kvelems, amax_v);
  hipLaunchKernelGGL(ffpa_fp8_quant_rows_kernel<T>, dim3((unsigned)((kvelems / 16 + 255) / 256), p.batch * p.hkv),
                     dim3(256), 0, st, (const uint16_t*)p.k, k8, amax_k, kvelems);
  hipLaunchKernelGGL(ffpa_fp8_quant_vt_kernel<T>, dim3(lay.np / 64, (p.d + 63) / 64, p.batch * p.hkv), dim3(256), 0,
                     st, (const uint16_t*)p.v, v8t, amax_v, p.nkv, p.d, lay.np);
  if constexpr (NDB <= 8) {
    p.ntiles = (p.nq + 127) / 128;
    p.total = p.batch * p.hq * p.ntiles;
    const int grid = (p.total + 7) & ~7;
    hipLaunchKernelGGL((ffpa_fwd_fp8_kernel<T, NDB>), dim3(grid), dim3(64 * Fp8Cfg<NDB>::NW), 0, st, p, amax_q, amax_k,
                       amax_v, k8, v8t, lay.np);
  } else {
    // D in 544..1024 (NDB = ceil(D / 64) rounded up to even): each wave owns a quarter of the
    // padded head dim, NQ = NDB / 2 blocks of 32 columns
    static_assert(NDB % 2 == 0, "D > 512 takes even block counts");
    constexpr int NQ = NDB / 2;
    p.ntiles = (p.nq + 63) / 64;
    p.total = p.batch * p.hq * p.ntiles;
    const int grid = (p.total + 7) & ~7;
    hipLaunchKernelGGL((ffpa_fwd_fp8_wide_kernel<T, NQ>), dim3(grid), dim3(64 * Fp8WideCfg<NQ>::NW), 0, st, p, amax_q,
                       amax_k, amax_v, k8, v8t, lay.np);
  }
  return hipGetLastError();
}

template <class T>
static hipError_t launch_fp8_t(const AttnParams& p, char* ws, hipStream_t st) {
  switch ((p.d + 63) / 64) {
    case 5: return launch_fp8_cfg<T, 5>(p, ws, st);
    case 6: return launch_fp8_cfg<T, 6>(p, ws, st);
    case 7: return launch_fp8_cfg<T, 7>(p, ws, st);
    case 8: return launch_fp8_cfg<T, 8>(p, ws, st);
    case 9:
    case 10: return launch_fp8_cfg<T, 10>(p, ws, st);
    case 11:
    case 12: return launch_fp8_cfg<T, 12>(p, ws, st);
    case 13:
    case 14: return launch_fp8_cfg<T, 14>(p, ws, st);
    default: return launch_fp8_cfg<T, 16>(p, ws, st);
  }
}

size_t fp8_workspace_bytes(int batch, int hq, int hkv, int nkv, int d) {
  return fp8_layout(batch, hq, hkv, nkv, d).total;
}

hipError_t launch_fwd_fp8(const AttnParams& p, int fp16, void* ws, hipStream_t st) {
  return fp16 ? launch_fp8_t<FP16>(p, (char*)ws, st) : launch_fp8_t<BF16>(p, (char*)ws, st);
}

}  // namespace ffpa
