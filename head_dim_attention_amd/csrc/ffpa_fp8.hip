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
// its half of the head dim.
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

// amax[head] = max |x| over the head's rows: grid (heads, row blocks of 64 rows); 8 bf16/fp16
// values per thread and step.
template <class T>
__global__ void __launch_bounds__(256) ffpa_fp8_amax_kernel(const uint16_t* x, long long head_elems, int rows,
                                                            int d, float* amax) {
  const int head = blockIdx.x;
  const int r0 = blockIdx.y * 64;
  const uint16_t* base = x + (long long)head * head_elems;
  const int per_row = d >> 3;
  float m = 0.f;
  for (int idx = threadIdx.x; idx < 64 * per_row; idx += 256) {
    const int r = r0 + idx / per_row;
    if (r < rows) {
      const u32x4_t v = *(const u32x4_t*)(base + (long long)r * d + 8 * (idx % per_row));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float lo, hi;
        Elt<T>::unpack2(v[e], lo, hi);
        m = fmaxf(m, fmaxf(fabsf(lo), fabsf(hi)));
      }
    }
  }
  // wave max, then one atomic per wave (the fp32 bits of non-negative values order like them)
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) atomicMax((unsigned int*)(amax + head), __float_as_uint(m));
}

__device__ __forceinline__ float quant_factor(float amax) { return amax > 0.f ? 448.0f / amax : 0.f; }

// K8[head][row][d] = e4m3(K * 448 / amax): 16 values per thread.
template <class T>
__global__ void __launch_bounds__(256) ffpa_fp8_quant_rows_kernel(const uint16_t* x, uint8_t* x8, const float* amax,
                                                                  long long head_elems, int d) {
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
  static constexpr int VROWS = (DPAD + 127) / 128 * 128;  // V8^T tile rows (copies of 16 rows x 8 waves)
  static constexpr int VTILE = VROWS * KT;     // V8^T tile: VROWS rows x 64 keys
  static constexpr int P8_OFF = 2 * KTILE + 2 * VTILE;
  static constexpr int XM_OFF = P8_OFF + NW * 1024;  // per wave: 32 queries x 32 keys of P8
  static constexpr int LDS = XM_OFF + NW * 32 * 4;   // per wave: tile max, then l, per query
  static constexpr int KCOPY = KTILE / 1024 / NW;
  static constexpr int VCOPY = VTILE / 1024 / NW;
  static_assert(DPAD <= 512 && LDS <= 160 * 1024 && VTILE % (1024 * NW) == 0, "LDS budget");
};

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
  const int item = (L & 7) * (gridDim.x >> 3) + (L >> 3);
  if (item >= p.total) return;
  int t = item % p.ntiles;
  const int hs = item / p.ntiles;
  const int h = hs % p.hq;
  const int s = hs / p.hq;
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

  // ---- copies of tile j: K8 rows (64 x D bytes into 512-byte LDS rows; 16-byte chunk c of row r
  // at physical chunk c ^ (r & 15), chunks past the head dim clamped) and V8^T rows (DPAD x 64
  // bytes; chunk c of row r at c ^ ((r >> 2) & 3), rows past the head dim clamped).
  const int dch = p.d >> 4;
  const long long k8_head = (long long)hk_flat * p.nkv * p.d;
  const long long v8_head = (long long)hk_flat * p.d * np;
  const i32x4_t krs = make_rsrc(k8 + k8_head, (uint32_t)min((long long)p.nkv * p.d, (long long)0xFFFFFFF0));
  const i32x4_t vrs = make_rsrc(v8t + v8_head, (uint32_t)min((long long)p.d * np, (long long)0xFFFFFFF0));
  int kvoff[C::KCOPY], vvoff[C::VCOPY], vrow[C::VCOPY];
#pragma unroll
  for (int c = 0; c < C::KCOPY; ++c) {
    const int r = 2 * (w + C::NW * c) + hh;  // 2 rows per 1 KB copy
    kvoff[c] = min(l32 ^ (r & 15), dch - 1) << 4;
  }
#pragma unroll
  for (int c = 0; c < C::VCOPY; ++c) {
    const int r = 16 * (w + C::NW * c) + (lane >> 2);  // 16 rows per copy
    vrow[c] = min(r, p.d - 1);
    vvoff[c] = vrow[c] * np + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
  }
  auto copy_tile = [&](int j, int b) {
#pragma unroll
    for (int c = 0; c < C::KCOPY; ++c) {
      const int r = 2 * (w + C::NW * c);
      const int key = min(j * C::KT + r + hh, p.nkv - 1);
      // the row offset is per lane here (two rows per instruction): fold it into voffset
      dma16_buf(krs, key * p.d + kvoff[c], 0, kbuf(b) + r * C::KROW);
    }
#pragma unroll
    for (int c = 0; c < C::VCOPY; ++c)
      dma16_buf(vrs, vvoff[c] + j * C::KT, 0, vbuf(b) + (16 * (w + C::NW * c)) * C::KT);
  };

  // ---- operand addresses
  // S^T block of this wave: keys 32 cg + row_perm(n) of the tile (A rows), so C register r holds key
  // 32 cg + c_row(r, h); lane reads 32 bytes = chunks 4 kb + 2 h, + 1 of its key row.
  // The row base is a multiple of 512, so the swizzled chunk is one per-lane base XOR a constant.
  const int krow = 32 * cg + row_perm(l32);
  const uint32_t klane = krow * C::KROW + ((krow & 15) << 4);
  auto k_addr = [&](uint32_t tile, int kb, int part) -> uint32_t {
    return (tile + klane) ^ ((4 * kb + 2 * hh + part) << 4);
  };
  // V8^T (A of O^T += V^T P^T): row d = cg DW + 32 db + n, keys 32 h .. + 31 = chunks 2 h, + 1; the
  // swizzle depends on n only.
  const uint32_t vlane = (cg * C::DW + l32) * C::KT;
  const int vsw = (l32 >> 2) & 3;
  auto v_addr = [&](uint32_t tile, int db, int part) -> uint32_t {
    return tile + vlane + 32 * db * C::KT + (((2 * hh + part) ^ vsw) << 4);
  };
  // P8 of wave (rg, c): [query n][32 keys], 32-byte rows whose two chunks swap for n & 8.
  auto p8_off = [&](int wave, int n, int key) -> int {
    return wave * 1024 + n * 32 + ((((key >> 4) ^ ((n >> 3) & 1))) << 4) + (key & 15);
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = (f32x16_t){};
  float mref = -INFINITY, lsum = 0.f;

  if (ntk > 0) copy_tile(0, 0);
  wait_all();
  const int qi = qw0 + l32;
  for (int j = 0; j < ntk; ++j) {
    wait_vmcnt<0>();
    lds_barrier();  // tile j visible; every wave has finished tile j - 1
    const uint32_t kt = lds_addr(kbuf(j & 1)), vt = lds_addr(vbuf(j & 1));
    if (j + 1 < ntk) copy_tile(j + 1, (j + 1) & 1);

    // S^T for this wave's 32 keys over the whole head dim
    f32x16_t sacc = (f32x16_t){};
#pragma unroll
    for (int kb = 0; kb < C::KS; ++kb) {
      const u32x4_t a0 = lds_read_b128_at(k_addr(kt, kb, 0));
      const u32x4_t a1 = lds_read_b128_at(k_addr(kt, kb, 1));
      const i32x8_t a = (i32x8_t){(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      sacc = mma_fp8(a, q8[kb], sacc);
    }
    // log2-domain scores, masked; tile max of this wave's keys per query
    const int key0 = j * C::KT + 32 * cg;
    const int lim = p.causal ? min(qi + off, p.nkv - 1) : p.nkv - 1;
    float mw = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = sacc[r] * sdq;
      if (key0 + c_row(r, hh) > lim) v = -INFINITY;
      sacc[r] = v;
      mw = fmaxf(mw, v);
    }
    mw = half_max(mw);
    if (hh == 0) *(__attribute__((address_space(3))) float*)(xmbuf + (w * 32 + l32) * 4) = mw;
    lds_barrier();
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
    // P in [0, 1] against the running max (a row with no finite score yet keeps P = 0), P8
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
    lds_barrier();
    // P8^T B operand: lane (h, n) = query n, keys 32 h .. + 31 of the tile, i.e. the P8 row of wave
    // (rg, h); the V8^T A operand holds the same keys in the same byte order.
    const int pw = 2 * rg + hh;
    const u32x4_t b0 = lds_read_b128(p8buf, p8_off(pw, l32, 0));
    const u32x4_t b1 = lds_read_b128(p8buf, p8_off(pw, l32, 16));
    const i32x8_t bop = (i32x8_t){(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x4_t a0 = lds_read_b128_at(v_addr(vt, db, 0));
      const u32x4_t a1 = lds_read_b128_at(v_addr(vt, db, 1));
      const i32x8_t a = (i32x8_t){(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      oacc[db] = mma_fp8(a, bop, oacc[db]);
    }
  }
  wait_vmcnt<0>();

  // ---- epilogue: the pair's l (each wave summed its own keys), O = O^T * amax_v / 448^2 / l
  lds_barrier();
  const float lw = half_sum(lsum);
  if (hh == 0) *(__attribute__((address_space(3))) float*)(xmbuf + (w * 32 + l32) * 4) = lw;
  lds_barrier();
  const float lp = *(const __attribute__((address_space(3))) float*)(xmbuf + ((w ^ 1) * 32 + l32) * 4);
  const float lt = cg == 0 ? lw + lp : lp + lw;
  const float inv = lt > 0.f ? (av / (448.0f * 448.0f)) / lt : 0.f;
  if (qi < p.nq) {
    uint16_t* orow = (uint16_t*)p.o + ((long long)s * p.hq + h) * p.o_head + (long long)qi * p.o_row;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = cg * C::DW + 32 * db + 8 * i4 + 4 * hh;
        if (d < p.d) {
          const f32x16_t& o = oacc[db];
          *(u32x2_t*)(orow + d) = (u32x2_t){Elt<T>::pack2(o[4 * i4] * inv, o[4 * i4 + 1] * inv),
                                            Elt<T>::pack2(o[4 * i4 + 2] * inv, o[4 * i4 + 3] * inv)};
        }
      }
    if (cg == 0 && hh == 0)
      p.lse[(long long)s * p.lse_batch + (long long)h * p.lse_head + qi] =
          lt > 0.f ? (mref + fast_log2(lt)) * kLn2 : -INFINITY;
  }
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
  using C = Fp8Cfg<NDB>;
  const Fp8Layout lay = fp8_layout(p.batch, p.hq, p.hkv, p.nkv, p.d);
  float* amax_q = (float*)(ws + lay.amax);
  float* amax_k = amax_q + p.batch * p.hq;
  float* amax_v = amax_k + p.batch * p.hkv;
  uint8_t* k8 = (uint8_t*)(ws + lay.k8);
  uint8_t* v8t = (uint8_t*)(ws + lay.v8t);
  const int nam = p.batch * (p.hq + 2 * p.hkv);
  hipLaunchKernelGGL(ffpa_fp8_amax_init_kernel, dim3((nam + 255) / 256), dim3(256), 0, st, amax_q, nam);
  hipLaunchKernelGGL(ffpa_fp8_amax_kernel<T>, dim3(p.batch * p.hq, (p.nq + 63) / 64), dim3(256), 0, st,
                     (const uint16_t*)p.q, (long long)p.nq * p.d, p.nq, p.d, amax_q);
  hipLaunchKernelGGL(ffpa_fp8_amax_kernel<T>, dim3(p.batch * p.hkv, (p.nkv + 63) / 64), dim3(256), 0, st,
                     (const uint16_t*)p.k, (long long)p.nkv * p.d, p.nkv, p.d, amax_k);
  hipLaunchKernelGGL(ffpa_fp8_amax_kernel<T>, dim3(p.batch * p.hkv, (p.nkv + 63) / 64), dim3(256), 0, st,
                     (const uint16_t*)p.v, (long long)p.nkv * p.d, p.nkv, p.d, amax_v);
  const long long kelems = (long long)p.nkv * p.d;
  hipLaunchKernelGGL(ffpa_fp8_quant_rows_kernel<T>, dim3((unsigned)((kelems / 16 + 255) / 256), p.batch * p.hkv),
                     dim3(256), 0, st, (const uint16_t*)p.k, k8, amax_k, kelems, p.d);
  hipLaunchKernelGGL(ffpa_fp8_quant_vt_kernel<T>, dim3(lay.np / 64, (p.d + 63) / 64, p.batch * p.hkv), dim3(256), 0,
                     st, (const uint16_t*)p.v, v8t, amax_v, p.nkv, p.d, lay.np);
  p.ntiles = (p.nq + 127) / 128;
  p.total = p.batch * p.hq * p.ntiles;
  const int grid = (p.total + 7) & ~7;
  hipLaunchKernelGGL((ffpa_fwd_fp8_kernel<T, NDB>), dim3(grid), dim3(64 * C::NW), 0, st, p, amax_q, amax_k, amax_v,
                     k8, v8t, lay.np);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_fp8_t(const AttnParams& p, char* ws, hipStream_t st) {
  switch ((p.d + 63) / 64) {
    case 5: return launch_fp8_cfg<T, 5>(p, ws, st);
    case 6: return launch_fp8_cfg<T, 6>(p, ws, st);
    case 7: return launch_fp8_cfg<T, 7>(p, ws, st);
    default: return launch_fp8_cfg<T, 8>(p, ws, st);
  }
}

size_t fp8_workspace_bytes(int batch, int hq, int hkv, int nkv, int d) {
  return fp8_layout(batch, hq, hkv, nkv, d).total;
}

hipError_t launch_fwd_fp8(const AttnParams& p, int fp16, void* ws, hipStream_t st) {
  return fp16 ? launch_fp8_t<FP16>(p, (char*)ws, st) : launch_fp8_t<BF16>(p, (char*)ws, st);
}

}  // namespace ffpa
