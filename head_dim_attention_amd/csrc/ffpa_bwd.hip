// Backward kernels for large-head-dim attention on gfx950.
//
// The backward of L = sum(dO * O) runs in four stages, as the ffpa-attn user guide describes for
// its D=512 Blackwell path ("CuTe-DSL Backend", "Blackwell status": preprocess, dV, dK, dQ, split
// because one unsplit dK/dV tile does not fit on chip). On gfx950 the same split keeps every
// kernel's register-resident state at or below two operand blocks plus one fp32 accumulator:
//
//   preprocess  Delta_i = sum_d dO_id O_id                           (HBM-bound streaming)
//   dV          dV_j += sum_i P_ij dO_i,  P = exp(scale S - LSE)     (keys stationary)
//   dK          dK_j += scale sum_i dS_ij Q_i, dS = P (dP - Delta), dP = dO V^T (keys stationary)
//   dQ          dQ_i += scale sum_j dS_ij K_j                         (queries stationary)
//
// All accumulation is fp32 in registers over the whole sweep (no atomics, deterministic); GQA
// key/value gradients are summed over the query heads of their group inside the same workgroup
// ("CuTe-DSL Backend", "Hard constraints": zero-stride broadcast). Rows whose LSE is -inf (no legal
// key) get P = 0 and so contribute nothing and receive zero gradient.
//
// The dV/dK/dQ kernels share one skeleton with the forward kernel: NW wave64s as NR x NC, the
// stationary rows' operands in registers as MFMA B operands, the other side streamed through LDS
// in 32-row tiles (buffer_load...lds), partial head-dim products combined through LDS, scores in a
// C-block layout whose registers feed the accumulating product directly as B operands, and the
// accumulating product's A operand read transposed from the streamed tile (ds_read_b64_tr_b16).
// For D <= 512, dV runs 8 waves (NC = 2) and dK/dQ run the 8-wave reduce-scatter variant below
// (NC = 4), both at two waves per SIMD; larger head dims use 4 waves (NC = 4), one per SIMD.
#include "ffpa_device.h"
#include "ffpa_params.h"

namespace ffpa {
// MFMAs whose LDS operands are requested ahead of the one issuing (see pin_lds_mfma_pipeline).
#ifndef BWD_AHEAD
#define BWD_AHEAD 2
#endif

// ------------------------------------------------------------------------------------------------
// Stage 1: Delta = rowsum(dO * O) in fp32 from the stored (rounded) O.
// One wave per row, 8 elements (16 bytes) per lane per step, 4 rows per wave.
// ------------------------------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ float dot8(u32x4_t a, u32x4_t b) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float a0, a1, b0, b1;
    Elt<T>::unpack2(a[e], a0, a1);
    Elt<T>::unpack2(b[e], b0, b1);
    s += a0 * b0;
    s += a1 * b1;
  }
  return s;
}

template <class T>
__global__ void __launch_bounds__(256) ffpa_bwd_preprocess_kernel(AttnParams p, int nrows, int varlen_total) {
  constexpr int RPW = 4;
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const long long row0 = ((long long)blockIdx.x * 4 + wv) * RPW;
  float acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    acc[r] = 0.f;
    const long long row = row0 + r;
    if (row < nrows) {
      const uint16_t* o = (const uint16_t*)p.o_in + row * p.d;
      const uint16_t* g = (const uint16_t*)p.dout + row * p.d;
      for (int c = lane * 8; c < p.d; c += 512) acc[r] += dot8<T>(*(const u32x4_t*)(o + c), *(const u32x4_t*)(g + c));
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc[r] += __shfl_xor(acc[r], m);
    const long long row = row0 + r;
    if (lane == 0 && row < nrows) {
      // Dense rows are ordered (b, h, n) like Delta; packed rows are (t, h) and Delta is [H, T].
      const long long idx = varlen_total > 0 ? (row % p.hq) * varlen_total + row / p.hq : row;
      p.delta[idx] = acc[r];
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Stages 2-4: dV, dK, dQ.
// ------------------------------------------------------------------------------------------------
enum BwdMode { kDQ = 0, kDK = 1, kDV = 2 };

template <int NC, int NDB, int NBUF, int NX, int NW>
struct BwdCfg {
  static constexpr int NR = NW / NC;
  static constexpr int DW = NDB * 32;
  static constexpr int DPAD = NC * DW;
  static constexpr int RS = DPAD <= 512 ? 1024 : 2048;
  static constexpr int BOWN = NR * 32;                 // stationary rows per workgroup
  static constexpr int TILE = 32 * RS;
  static constexpr int XBYTES = NW * NX * 16 * 64 * 4;  // NX partial C blocks per wave
  static constexpr int LDS = NBUF * 2 * TILE + XBYTES;
  static constexpr int NINSTR = TILE / 1024 / NW;
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <class T, int MODE, int NC, int NDB, int NBUF, int NW>
__global__ void __launch_bounds__(64 * NW, NW / 4) ffpa_bwd_kernel(AttnParams p) {
  constexpr bool OWN_Q = MODE == kDQ;   // stationary rows are queries (dQ) or keys (dK, dV)
  constexpr bool HAS_DP = MODE != kDV;  // dK and dQ need dP = dO V^T
  constexpr int NX = HAS_DP ? 2 : 1;
  using C = BwdCfg<NC, NDB, NBUF, NX, NW>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  lds_t* smem = (lds_t*)smem_raw;

  const int L = blockIdx.x;
  const int item = (L & 7) * (gridDim.x >> 3) + (L >> 3);
  if (item >= p.total) return;
  const int heads = OWN_Q ? p.hq : p.hkv;
  int t = item % p.ntiles;
  const int hs = item / p.ntiles;
  const int hd = hs % heads;
  const int s = hs / heads;
  if (OWN_Q && p.causal) t = p.ntiles - 1 - t;  // heaviest causal tiles first

  const SeqView sv = seq_view(p, s);
  const int own_len = OWN_Q ? sv.lq : sv.lk;
  const int o0 = t * C::BOWN;
  if (o0 >= own_len) return;

  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int rg = w / NC;
  const int cg = w % NC;
  const int ow0 = o0 + rg * 32;
  const int off = sv.lk - sv.lq;

  // ---- stationary operands: lane (h, n) holds own row n, dims 16 kb + 8 h + 0..7
  const int own_row = OWN_Q ? p.q_row : p.k_row;
  const long long own_base = OWN_Q ? sv.q_off + (long long)hd * p.q_head : sv.k_off + (long long)hd * p.k_head;
  const uint16_t* r1src = (const uint16_t*)(OWN_Q ? p.q : p.k) + own_base;
  const uint16_t* r2src = (const uint16_t*)(OWN_Q ? p.dout : p.v) + own_base;
  u32x4_t r1[2 * NDB];
  u32x4_t r2[HAS_DP ? 2 * NDB : 1];
  {
    const long long oi = min(ow0 + l32, own_len - 1);
#pragma unroll
    for (int kb = 0; kb < 2 * NDB; ++kb) {
      const int dim = cg * C::DW + kb * 16 + hh * 8;
      const bool in = dim < p.d;
      r1[kb] = in ? *(const u32x4_t*)(r1src + oi * own_row + dim) : (u32x4_t){0u, 0u, 0u, 0u};
      if constexpr (HAS_DP)
        r2[kb] = in ? *(const u32x4_t*)(r2src + oi * own_row + dim) : (u32x4_t){0u, 0u, 0u, 0u};
    }
  }

  // dQ: the query's LSE (log2 units; +inf for an empty row makes P = 0) and Delta are per lane.
  float lse2_own = 0.f, dlt_own = 0.f;
  if constexpr (OWN_Q) {
    const long long qi = sv.lse_off + (long long)hd * p.lse_head + min(ow0 + l32, sv.lq - 1);
    const float l = p.lse_in[qi];
    lse2_own = l == -INFINITY ? INFINITY : l * kLog2e;
    dlt_own = p.delta[qi];
  }

  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = (f32x16_t){};

  // ---- streamed side
  const int str_len = OWN_Q ? sv.lk : sv.lq;
  const int str_row = OWN_Q ? p.k_row : p.q_row;
  const int row_bytes = str_row * 2;
  int nsteps, nqt = 1, qt_first = 0;
  if constexpr (OWN_Q) {
    int kend = sv.lk;
    if (p.causal) kend = min(kend, o0 + C::BOWN + off);
    nsteps = kend > 0 ? (kend + 31) >> 5 : 0;
  } else {
    const int qfirst = p.causal ? max(0, o0 - off) : 0;
    qt_first = qfirst >> 5;
    nqt = sv.lq > qfirst ? ((sv.lq + 31) >> 5) - qt_first : 0;
    nsteps = p.group * nqt;
  }
  auto step_head = [&](int st) { return OWN_Q ? hd / p.group : hd * p.group + st / nqt; };
  auto step_row0 = [&](int st) { return OWN_Q ? st * 32 : (qt_first + st % nqt) * 32; };
  auto str_base = [&](int head) {
    return OWN_Q ? sv.k_off + (long long)head * p.k_head : sv.q_off + (long long)head * p.q_head;
  };
  const uint32_t span = (uint32_t)min((long long)max(str_len, 1) * row_bytes, (long long)0xFFFFFFF0);

  constexpr int IPR = C::RS / 1024;
  const int dch = p.d >> 3;
  int voff[C::NINSTR];
#pragma unroll
  for (int ii = 0; ii < C::NINSTR; ++ii) {
    const int i = w + NW * ii;
    const int R = i / IPR;
    const int pc = (i % IPR) * 64 + lane;
    voff[ii] = min(pc ^ swz(R), dch - 1) << 4;
  }
  // Tile 1 feeds the scores (K for dQ, Q for dK/dV); tile 2 feeds dP (V for dQ, dO for dK) or the
  // dV product (dO).
  // A step index past the end is clamped to the last step (its copies then land in a buffer that
  // is not read again).
  struct StepSrc {
    i32x4_t r1, r2;
    int row0;
  };
  auto step_src = [&](int st) {
    st = min(st, nsteps - 1);
    const long long base = str_base(step_head(st));
    StepSrc x;
    x.r1 = make_rsrc((const uint16_t*)(OWN_Q ? p.k : p.q) + base, span);
    x.r2 = make_rsrc((const uint16_t*)(OWN_Q ? p.v : p.dout) + base, span);
    x.row0 = step_row0(st);
    return x;
  };
  // Copy ii of tile `which` (1 or 2) of a step into buffer buf.
  auto copy1 = [&](const StepSrc& x, int buf, int which, int ii) {
    const int i = w + NW * ii;
    const int row = min(x.row0 + i / IPR, str_len - 1);
    dma16_buf(which == 1 ? x.r1 : x.r2, voff[ii], row * row_bytes,
              smem + buf * 2 * C::TILE + (which - 1) * C::TILE + i * 1024);
  };
  auto issue = [&](int st, int buf) {
    const StepSrc x = step_src(st);
#pragma unroll
    for (int ii = 0; ii < C::NINSTR; ++ii) {
      copy1(x, buf, 1, ii);
      copy1(x, buf, 2, ii);
    }
  };
  // With two buffers, the copies of step st + 1 are spread over the partial products of step st
  // (both of its buffers were released at the barrier that opens step st): the copy path moves
  // about 64 B per clock per CU, so a whole step issued at once would hold every wave at the issue.
  // Copy c of the 2 * NINSTR of a step is issued after MFMA spread_at(n, c) of a run of n.
  auto spread_at = [](int n, int c) { return (c * n) / (2 * C::NINSTR); };

  const int krow = row_perm(l32);
  const int kswz = swz(krow);
  const int g16 = lane >> 4;
  const int r16 = lane & 15;
  const int cbase = cg * C::DW >> 3;  // first 16-byte chunk of this wave's head-dim columns
  lds_t* xbuf = smem + NBUF * 2 * C::TILE;

  // LDS byte addresses of this lane's operands in a tile at LDS address `tile`. When the wave's
  // first chunk is a multiple of 16, the swizzle (an XOR on the low 4 bits of the 16-byte chunk
  // index) touches only address bits 4-7, which are zero in the row, column-group and tile bases:
  // every operand address is then one per-lane base XOR a compile-time constant, plus a constant.
  constexpr bool kAligned = (C::DW % 128) == 0;
  // Streamed rows as A operand of the partial products: tile row row_perm(m), chunk cbase + 2 kb + h.
  const uint32_t alane = krow * C::RS + (cbase << 4) + ((hh ^ kswz) << 4);
  auto a_addr = [&](uint32_t tile, int kb) -> uint32_t {
    if constexpr (kAligned) return ((tile + alane) ^ ((kb & 7) << 5)) + ((kb >> 3) << 8);
    return tile + krow * C::RS + (((cbase + 2 * kb + hh) ^ kswz) << 4);
  };
  // Transposed reads of the streamed tile (A operand of the accumulating product): tile row
  // k = 16 kb2 + 8 h + 4 half + r16/4, head-dim column cg DW + 32 db + 16 (g16 % 2) + 4 (r16 % 4),
  // i.e. chunk cbase + 4 db + tclo. swz(k) does not depend on kb2.
  const int tclo = 2 * (g16 & 1) + ((r16 & 3) >> 1);
  const int twithin = ((4 * (r16 & 3)) & 7) << 1;
  uint32_t tlane[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int k = 8 * hh + 4 * half + (r16 >> 2);
    tlane[half] = k * C::RS + (cbase << 4) + ((tclo ^ swz(k)) << 4) + twithin;
  }
  auto t_addr = [&](uint32_t tile, int db, int kb2, int half) -> uint32_t {
    if constexpr (kAligned)
      return ((tile + tlane[half]) ^ ((db & 3) << 6)) + ((db >> 2) << 8) + kb2 * 16 * C::RS;
    const int k = 16 * kb2 + 8 * hh + 4 * half + (r16 >> 2);
    return tile + k * C::RS + (((cbase + 4 * db + tclo) ^ swz(k)) << 4) + twithin;
  };

  // dK/dV: LSE (log2 units; +inf for an empty row makes P = 0) and Delta of streamed query row
  // row0 + l % 32, loaded one step ahead and after that step's tile copy, so the wait that makes
  // the tile visible covers them too.
  // The raw values are kept until use so that no instruction waits on the loads early.
  float lse_next = 0.f, dlt_next = 0.f;
  auto load_row_stats = [&](int st) {
    if constexpr (!OWN_Q) {
      const long long li = sv.lse_off + (long long)step_head(st) * p.lse_head + min(step_row0(st) + l32, sv.lq - 1);
      lse_next = p.lse_in[li];
      dlt_next = p.delta[li];
    }
  };

  if (nsteps > 0) {
    issue(0, 0);
    load_row_stats(0);
  }
  // Stationary operands, row statistics and tile 0 are complete before the loop.
  wait_all();

  for (int st = 0; st < nsteps; ++st) {
    const int buf = NBUF == 2 ? (st & 1) : 0;
    wait_vmcnt<0>();
    lds_barrier();
    const float lse2_cur = lse_next == -INFINITY ? INFINITY : lse_next * kLog2e;
    const float dlt_cur = dlt_next;
    if (NBUF == 2 && st + 1 < nsteps) load_row_stats(st + 1);
    const StepSrc xn = step_src(st + 1);
    const lds_t* t1 = smem + buf * 2 * C::TILE;
    const lds_t* t2 = t1 + C::TILE;
    const int row0 = step_row0(st);

    // ---- partial S (and dP) over this wave's head-dim columns: C[streamed row][own row]
    f32x16_t sacc = (f32x16_t){}, dpacc = (f32x16_t){};
    constexpr int KSTEPS = 2 * NDB;
#pragma unroll
    for (int kb = 0; kb < KSTEPS; ++kb) {
      sacc = Elt<T>::mma(lds_read_b128_at(a_addr(lds_addr(t1), kb)), r1[kb], sacc);
      if constexpr (HAS_DP) dpacc = Elt<T>::mma(lds_read_b128_at(a_addr(lds_addr(t2), kb)), r2[kb], dpacc);
      if constexpr (NBUF == 2) {
#pragma unroll
        for (int c = 0; c < 2 * C::NINSTR; ++c)
          if (kb == spread_at(KSTEPS, c)) copy1(xn, buf ^ 1, 1 + (c & 1), c >> 1);
      }
    }
    pin_lds_mfma_pipeline<KSTEPS * (HAS_DP ? 2 : 1), BWD_AHEAD, 1>();
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      lds_write_f4(xbuf, (((w * NX + 0) * 4 + r4) * 64 + lane) * 16,
                   (f32x4_t){sacc[4 * r4], sacc[4 * r4 + 1], sacc[4 * r4 + 2], sacc[4 * r4 + 3]});
      if constexpr (HAS_DP)
        lds_write_f4(xbuf, (((w * NX + 1) * 4 + r4) * 64 + lane) * 16,
                     (f32x4_t){dpacc[4 * r4], dpacc[4 * r4 + 1], dpacc[4 * r4 + 2], dpacc[4 * r4 + 3]});
    }
    lds_barrier();
    // Fixed commutative combination (bit-identical in every wave of the row group).
    auto combine = [&](f32x16_t& v, int m) {
      const int base = rg * NC;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        auto rd = [&](int wv) { return lds_read_f4(xbuf, (((wv * NX + m) * 4 + r4) * 64 + lane) * 16); };
        f32x4_t mine = (f32x4_t){v[4 * r4], v[4 * r4 + 1], v[4 * r4 + 2], v[4 * r4 + 3]};
        mine = mine + rd(base + (cg ^ 1));
        if constexpr (NC == 4) {
          const int o1 = base + ((cg & 2) ^ 2);
          mine = mine + (rd(o1) + rd(o1 + 1));
        }
        v[4 * r4] = mine.x; v[4 * r4 + 1] = mine.y; v[4 * r4 + 2] = mine.z; v[4 * r4 + 3] = mine.w;
      }
    };
    combine(sacc, 0);
    if constexpr (HAS_DP) combine(dpacc, 1);

    // ---- P (and dS) for the 16 (streamed, own) pairs of this lane
    // dK/dV: the streamed rows are queries; lane l holds LSE/Delta of query row0 + l % 32 and the
    // values of the 16 rows c_row(r, h) a lane needs are broadcast with ds_bpermute.
    const float lse2_lane = OWN_Q ? lse2_own : lse2_cur;
    const float dlt_lane = OWN_Q ? dlt_own : dlt_cur;
    const int bp_base = (8 * hh) << 2;  // byte address of lane 8h for ds_bpermute
    auto row_val = [&](float x, int r) -> float {
      if constexpr (OWN_Q) return x;
      const int c = 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3);  // c_row(r, h) - 8h
      return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(bp_base + 4 * c, __builtin_bit_cast(int, x)));
    };
    // Masking is needed only on tiles that cross the causal diagonal or the end of either side.
    const int oi = ow0 + l32;
    bool need_mask;
    if constexpr (OWN_Q) {
      need_mask = (row0 + 32 > sv.lk) || (p.causal && row0 + 31 > ow0 + off);
    } else {
      need_mask = (row0 + 32 > sv.lq) || (p.causal && ow0 + 31 > row0 + off);
    }
    uint32_t bop[2][4];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float v2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int rr = r + u;
        const float lse2 = row_val(lse2_lane, rr);
        float pv = fast_exp2(sacc[rr] * p.scale_log2 - lse2);
        if (need_mask) {
          const int si = row0 + c_row(rr, hh);
          const int qi = OWN_Q ? oi : si;
          const int ki = OWN_Q ? si : oi;
          const bool legal = ki < sv.lk && qi < sv.lq && (!p.causal || ki <= qi + off);
          pv = legal ? pv : 0.f;
        }
        if constexpr (HAS_DP) pv = pv * (dpacc[rr] - row_val(dlt_lane, rr));
        v2[u] = pv;
      }
      bop[r >> 3][(r & 7) >> 1] = Elt<T>::pack2(v2[0], v2[1]);
    }

    // ---- acc^T[d][own] += A[d][streamed] * B[streamed][own], A read transposed from the tile
    const lds_t* tt = MODE == kDV ? t2 : t1;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const s16x4_t lo = lds_read_tr16_at(t_addr(lds_addr(tt), db, kb2, 0));
        const s16x4_t hi = lds_read_tr16_at(t_addr(lds_addr(tt), db, kb2, 1));
        const u32x4_t bv = {bop[kb2][0], bop[kb2][1], bop[kb2][2], bop[kb2][3]};
        acc[db] = Elt<T>::mma(join_tr(lo, hi), bv, acc[db]);
      }
    }
    pin_lds_mfma_pipeline<2 * NDB, BWD_AHEAD, 2>();

    if constexpr (NBUF == 1) {
      lds_barrier();
      if (st + 1 < nsteps) {
        issue(st + 1, 0);
        load_row_stats(st + 1);
      }
    }
  }
  // Copies issued during the last step land in LDS that the next workgroup may own.
  wait_vmcnt<0>();

  // ---- epilogue: scale, round once to the storage dtype, store own rows
  const float osc = MODE == kDV ? 1.0f : p.scale;
  const int oi = ow0 + l32;
  if (oi < own_len) {
    uint16_t* dst = (uint16_t*)(MODE == kDQ ? p.dq : (MODE == kDK ? p.dk : p.dv)) + own_base + (long long)oi * own_row;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = cg * C::DW + 32 * db + 8 * i4 + 4 * hh;
        if (d < p.d) {
          const f32x16_t& a = acc[db];
          const u32x2_t pk = {Elt<T>::pack2(a[4 * i4] * osc, a[4 * i4 + 1] * osc),
                              Elt<T>::pack2(a[4 * i4 + 2] * osc, a[4 * i4 + 3] * osc)};
          *(u32x2_t*)(dst + d) = pk;
        }
      }
  }
}

// ------------------------------------------------------------------------------------------------
// dK and dQ for D <= 512 with two waves per SIMD.
//
// Eight waves form NR = 2 row groups of NC = 4; a wave holds 32 stationary rows x D/4 head-dim
// columns of both stationary operands and of the fp32 accumulator, which fits 256 registers.
// The four partial score blocks of a row group are combined by a reduce-scatter: wave cg
// finishes only the 8 streamed rows of register quarter cg (registers 4cg..4cg+3 of the C block),
// computes dS for them, and the bf16 dS quarters are then all-gathered, so each wave does a
// quarter of the softmax-gradient arithmetic and exchanges half the partial-sum bytes of a full
// all-reduce. The tile read only by the partial products (dO for dK, V for dQ) has one buffer
// and is refilled as soon as every wave has passed the exchange barrier; the tile also read by
// the accumulating product is double-buffered. dK's per-query LSE and Delta come with the query
// tile into LDS and are read by broadcast.
// ------------------------------------------------------------------------------------------------
template <int NDB>
struct RsCfg {
  static constexpr int NC = 4, NW = 8, NR = 2;
  static constexpr int DW = NDB * 32;
  static constexpr int RS = 1024;                // LDS row stride (bytes), padded head dim <= 512
  static constexpr int BOWN = NR * 32;           // stationary rows per workgroup
  static constexpr int TILE = 32 * RS;
  static constexpr int PIECE = 64 * 16;          // one f32x4 per lane
  static constexpr int T2_OFF = 2 * TILE;        // single-buffered tile
  static constexpr int X_OFF = 3 * TILE;         // [wave][3 partner quarters][S, dP] pieces
  static constexpr int G_OFF = X_OFF + NW * 3 * 2 * PIECE;  // [wave] packed dS quarter, 8 B/lane
  static constexpr int ST_OFF = G_OFF + NW * 64 * 8;        // [buffer][LSE, Delta] x 64 floats
  static constexpr int LDS = ST_OFF + 2 * 2 * 256;
  static constexpr int NINSTR = TILE / 1024 / NW;
  static_assert(4 * DW <= 512 && LDS <= 160 * 1024, "LDS budget");
};

template <class T, int MODE, int NDB>
__global__ void __launch_bounds__(512, 2) ffpa_bwd_rs_kernel(AttnParams p) {
  static_assert(MODE == kDQ || MODE == kDK, "dK and dQ only");
  constexpr bool OWN_Q = MODE == kDQ;
  using C = RsCfg<NDB>;
  constexpr int NC = C::NC, NW = C::NW;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  lds_t* smem = (lds_t*)smem_raw;

  const int L = blockIdx.x;
  const int item = (L & 7) * (gridDim.x >> 3) + (L >> 3);
  if (item >= p.total) return;
  const int heads = OWN_Q ? p.hq : p.hkv;
  int t = item % p.ntiles;
  const int hs = item / p.ntiles;
  const int hd = hs % heads;
  const int s = hs / heads;
  if (OWN_Q && p.causal) t = p.ntiles - 1 - t;  // heaviest causal tiles first

  const SeqView sv = seq_view(p, s);
  const int own_len = OWN_Q ? sv.lq : sv.lk;
  const int o0 = t * C::BOWN;
  if (o0 >= own_len) return;

  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int rg = w / NC;
  const int cg = w % NC;
  const int ow0 = o0 + rg * 32;
  const int off = sv.lk - sv.lq;

  // ---- stationary operands: lane (h, n) holds own row n, dims 16 kb + 8 h + 0..7
  const int own_row = OWN_Q ? p.q_row : p.k_row;
  const long long own_base = OWN_Q ? sv.q_off + (long long)hd * p.q_head : sv.k_off + (long long)hd * p.k_head;
  const uint16_t* r1src = (const uint16_t*)(OWN_Q ? p.q : p.k) + own_base;
  const uint16_t* r2src = (const uint16_t*)(OWN_Q ? p.dout : p.v) + own_base;
  u32x4_t r1[2 * NDB], r2[2 * NDB];
  {
    const long long oi = min(ow0 + l32, own_len - 1);
#pragma unroll
    for (int kb = 0; kb < 2 * NDB; ++kb) {
      const int dim = cg * C::DW + kb * 16 + hh * 8;
      const bool in = dim < p.d;
      r1[kb] = in ? *(const u32x4_t*)(r1src + oi * own_row + dim) : (u32x4_t){0u, 0u, 0u, 0u};
      r2[kb] = in ? *(const u32x4_t*)(r2src + oi * own_row + dim) : (u32x4_t){0u, 0u, 0u, 0u};
    }
  }
  // dQ: the query's LSE (log2 units; +inf for an empty row makes P = 0) and Delta are per lane.
  float lse2_own = 0.f, dlt_own = 0.f;
  if constexpr (OWN_Q) {
    const long long qi = sv.lse_off + (long long)hd * p.lse_head + min(ow0 + l32, sv.lq - 1);
    const float l = p.lse_in[qi];
    lse2_own = l == -INFINITY ? INFINITY : l * kLog2e;
    dlt_own = p.delta[qi];
  }

  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = (f32x16_t){};

  // ---- streamed side
  const int str_len = OWN_Q ? sv.lk : sv.lq;
  const int row_bytes = (OWN_Q ? p.k_row : p.q_row) * 2;
  int nsteps, nqt = 1, qt_first = 0;
  if constexpr (OWN_Q) {
    int kend = sv.lk;
    if (p.causal) kend = min(kend, o0 + C::BOWN + off);
    nsteps = kend > 0 ? (kend + 31) >> 5 : 0;
  } else {
    const int qfirst = p.causal ? max(0, o0 - off) : 0;
    qt_first = qfirst >> 5;
    nqt = sv.lq > qfirst ? ((sv.lq + 31) >> 5) - qt_first : 0;
    nsteps = p.group * nqt;
  }
  auto step_head = [&](int st) { return OWN_Q ? hd / p.group : hd * p.group + st / nqt; };
  auto step_row0 = [&](int st) { return OWN_Q ? st * 32 : (qt_first + st % nqt) * 32; };
  auto str_base = [&](int head) {
    return OWN_Q ? sv.k_off + (long long)head * p.k_head : sv.q_off + (long long)head * p.q_head;
  };
  const uint32_t span = (uint32_t)min((long long)max(str_len, 1) * row_bytes, (long long)0xFFFFFFF0);
  const int dch = p.d >> 3;
  int voff[C::NINSTR];
#pragma unroll
  for (int ii = 0; ii < C::NINSTR; ++ii) voff[ii] = min(lane ^ swz(w + NW * ii), dch - 1) << 4;

  // Copies of step st: tile 1 (K for dQ, Q for dK) into buffer buf, tile 2 (V for dQ, dO for dK)
  // into its single buffer, and dK's row statistics. A step index past the end is clamped to the
  // last step (its copies then land in buffers that are not read again).
  struct StepSrc {
    i32x4_t r1, r2;
    int row0, head;
  };
  auto step_src = [&](int st) {
    st = min(st, nsteps - 1);
    StepSrc x;
    x.head = step_head(st);
    x.row0 = step_row0(st);
    x.r1 = make_rsrc((const uint16_t*)(OWN_Q ? p.k : p.q) + str_base(x.head), span);
    x.r2 = make_rsrc((const uint16_t*)(OWN_Q ? p.v : p.dout) + str_base(x.head), span);
    return x;
  };
  auto copy_t1 = [&](const StepSrc& x, int buf, int ii) {
    const int i = w + NW * ii;
    dma16_buf(x.r1, voff[ii], min(x.row0 + i, str_len - 1) * row_bytes, smem + buf * C::TILE + i * 1024);
  };
  auto copy_t2 = [&](const StepSrc& x, int ii) {
    const int i = w + NW * ii;
    dma16_buf(x.r2, voff[ii], min(x.row0 + i, str_len - 1) * row_bytes, smem + C::T2_OFF + i * 1024);
  };
  auto copy_stats = [&](const StepSrc& x, int buf) {
    if constexpr (!OWN_Q) {
      if (w == 0) {
        const long long li = sv.lse_off + (long long)x.head * p.lse_head;
        const uint32_t bytes = (uint32_t)max(sv.lq, 1) * 4;
        const int vo = min(x.row0 + l32, sv.lq - 1) * 4;
        lds_t* sd = smem + C::ST_OFF + buf * 512;
        dma4_buf(make_rsrc(p.lse_in + li, bytes), vo, sd);
        dma4_buf(make_rsrc(p.delta + li, bytes), vo, sd + 256);
      }
    }
  };
  // MFMA index (of a run of n) after which copy ii is issued: the copy path moves about 64 B per
  // clock per CU, so a whole tile issued at once would hold every wave at the issue.
  auto spread_at = [](int n, int ii) { return (ii * n) / C::NINSTR; };

  // Register quarter i of the C block (registers 4i..4i+3) covers tile rows 16 (i/2) + 8 h +
  // 4 (i%2) + 0..3. Wave cg reads its A operand with the quarter bits of the row index (bits 4
  // and 2) rotated by cg, so register quarter i holds the rows of quarter (i + cg) % 4: the quarter
  // the wave finishes is always registers 0..3 and the partners' quarters are registers 4..15.
  auto rot_quarter = [&](int row) {
    const int q = (((row >> 4) & 1) << 1 | ((row >> 2) & 1)) + cg;
    return (row & ~0x14) | (((q >> 1) & 1) << 4) | ((q & 1) << 2);
  };
  const int krow = rot_quarter(row_perm(l32));
  const int kswz = swz(krow);
  const int g16 = lane >> 4;
  const int r16 = lane & 15;
  const int cbase = cg * C::DW >> 3;
  // LDS operand addresses (see the forward kernel): with a 16-chunk-aligned column base every
  // address is one per-lane base XOR a constant, plus a constant.
  constexpr bool kAligned = (C::DW % 128) == 0;
  const uint32_t alane = krow * C::RS + (cbase << 4) + ((hh ^ kswz) << 4);
  auto a_addr = [&](uint32_t tile, int kb) -> uint32_t {
    if constexpr (kAligned) return ((tile + alane) ^ ((kb & 7) << 5)) + ((kb >> 3) << 8);
    return tile + krow * C::RS + (((cbase + 2 * kb + hh) ^ kswz) << 4);
  };
  const int tclo = 2 * (g16 & 1) + ((r16 & 3) >> 1);
  const int twithin = ((4 * (r16 & 3)) & 7) << 1;
  uint32_t tlane[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int k = 8 * hh + 4 * half + (r16 >> 2);
    tlane[half] = k * C::RS + (cbase << 4) + ((tclo ^ swz(k)) << 4) + twithin;
  }
  auto t_addr = [&](uint32_t tile, int db, int kb2, int half) -> uint32_t {
    if constexpr (kAligned)
      return ((tile + tlane[half]) ^ ((db & 3) << 6)) + ((db >> 2) << 8) + kb2 * 16 * C::RS;
    const int k = 16 * kb2 + 8 * hh + 4 * half + (r16 >> 2);
    return tile + k * C::RS + (((cbase + 4 * db + tclo) ^ swz(k)) << 4) + twithin;
  };
  lds_t* const xbuf = smem + C::X_OFF;
  lds_t* const gbuf = smem + C::G_OFF;
  // Rows of this wave's register quarter, relative to the tile: 16 (cg/2) + 8 h + 4 (cg%2) + 0..3.
  const int qrow = 16 * (cg >> 1) + 8 * hh + 4 * (cg & 1);

  if (nsteps > 0) {
    const StepSrc x0 = step_src(0);
    copy_stats(x0, 0);
#pragma unroll
    for (int ii = 0; ii < C::NINSTR; ++ii) {
      copy_t1(x0, 0, ii);
      copy_t2(x0, ii);
    }
  }
  wait_all();  // stationary operands, dQ's row statistics and the first tiles

  // The copies of step st + 1 are issued during step st: its statistics after barrier A, tile 1
  // spread over the partial products (its other buffer was released at barrier A), tile 2 right
  // after barrier B, which releases its single buffer (as early as possible, so that it lands
  // before step st + 1). All are waited for before barrier A of step st + 1.
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    wait_vmcnt<0>();
    lds_barrier();  // (A) this step's tiles are visible; every wave has finished the last step
    const StepSrc xn = step_src(st + 1);
    copy_stats(xn, buf ^ 1);
    const uint32_t t1 = lds_addr(smem + buf * C::TILE);
    const uint32_t t2 = lds_addr(smem + C::T2_OFF);
    const int row0 = step_row0(st);

    // ---- partial S and dP over this wave's head-dim columns: C[streamed row][own row]
    f32x16_t sacc = (f32x16_t){}, dpacc = (f32x16_t){};
#pragma unroll
    for (int kb = 0; kb < 2 * NDB; ++kb) {
      sacc = Elt<T>::mma(lds_read_b128_at(a_addr(t1, kb)), r1[kb], sacc);
      dpacc = Elt<T>::mma(lds_read_b128_at(a_addr(t2, kb)), r2[kb], dpacc);
#pragma unroll
      for (int ii = 0; ii < C::NINSTR; ++ii)
        if (kb == spread_at(2 * NDB, ii)) copy_t1(xn, buf ^ 1, ii);
    }
    pin_lds_mfma_pipeline<4 * NDB, 2, 1>();
    // Partner quarters to the exchange: slot j holds register quarter j + 1, i.e. quarter
    // (cg + 1 + j) % 4.
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int q = j + 1;
      const int base = ((w * 3 + j) * 2) * C::PIECE + lane * 16;
      lds_write_f4(xbuf, base, (f32x4_t){sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]});
      lds_write_f4(xbuf, base + C::PIECE,
                   (f32x4_t){dpacc[4 * q], dpacc[4 * q + 1], dpacc[4 * q + 2], dpacc[4 * q + 3]});
    }
    lds_barrier();  // (B) partial sums visible; every wave has finished reading tile 2
#pragma unroll
    for (int ii = 0; ii < C::NINSTR; ++ii) copy_t2(xn, ii);

    // ---- reduce this wave's quarter: own part + partners in a fixed order
    f32x4_t sq = (f32x4_t){sacc[0], sacc[1], sacc[2], sacc[3]};
    f32x4_t dq = (f32x4_t){dpacc[0], dpacc[1], dpacc[2], dpacc[3]};
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      const int pc = (cg + i) & 3;            // partner column group
      const int j = ((cg - pc) & 3) - 1;      // its slot holding quarter cg
      const int base = (((rg * NC + pc) * 3 + j) * 2) * C::PIECE + lane * 16;
      sq = sq + lds_read_f4(xbuf, base);
      dq = dq + lds_read_f4(xbuf, base + C::PIECE);
    }

    // ---- P and dS for the 4 (streamed, own) pairs of this lane's quarter
    f32x4_t lse2q, dltq;
    if constexpr (OWN_Q) {
      lse2q = (f32x4_t){lse2_own, lse2_own, lse2_own, lse2_own};
      dltq = (f32x4_t){dlt_own, dlt_own, dlt_own, dlt_own};
    } else {
      const lds_t* sd = smem + C::ST_OFF + buf * 512;
      const f32x4_t lr = lds_read_f4(sd, qrow * 4);
      dltq = lds_read_f4(sd, 256 + qrow * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) lse2q[i] = lr[i] == -INFINITY ? INFINITY : lr[i] * kLog2e;
    }
    const int oi = ow0 + l32;
    bool need_mask;
    if constexpr (OWN_Q) {
      need_mask = (row0 + 32 > sv.lk) || (p.causal && row0 + 31 > ow0 + off);
    } else {
      need_mask = (row0 + 32 > sv.lq) || (p.causal && ow0 + 31 > row0 + off);
    }
    float ds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float pv = fast_exp2(sq[i] * p.scale_log2 - lse2q[i]);
      if (need_mask) {
        const int si = row0 + qrow + i;
        const int qi = OWN_Q ? oi : si;
        const int ki = OWN_Q ? si : oi;
        const bool legal = ki < sv.lk && qi < sv.lq && (!p.causal || ki <= qi + off);
        pv = legal ? pv : 0.f;
      }
      ds[i] = pv * (dq[i] - dltq[i]);
    }
    const u32x2_t mine = {Elt<T>::pack2(ds[0], ds[1]), Elt<T>::pack2(ds[2], ds[3])};
    *(__attribute__((address_space(3))) u32x2_t*)(gbuf + w * 512 + lane * 8) = mine;
    lds_barrier();  // (C) dS quarters visible

    // ---- all-gather dS: quarter q gives B-operand words 2 (q % 2), +1 of k-block q / 2
    uint32_t bop[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x2_t v = mine;
      if (q != cg) v = *(const __attribute__((address_space(3))) u32x2_t*)(gbuf + (rg * NC + q) * 512 + lane * 8);
      bop[q >> 1][2 * (q & 1)] = v.x;
      bop[q >> 1][2 * (q & 1) + 1] = v.y;
    }

    // ---- acc^T[d][own] += A[d][streamed] * dS[streamed][own], A read transposed from tile 1
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const s16x4_t lo = lds_read_tr16_at(t_addr(t1, db, kb2, 0));
        const s16x4_t hi = lds_read_tr16_at(t_addr(t1, db, kb2, 1));
        const u32x4_t bv = {bop[kb2][0], bop[kb2][1], bop[kb2][2], bop[kb2][3]};
        acc[db] = Elt<T>::mma(join_tr(lo, hi), bv, acc[db]);
      }
    }
    pin_lds_mfma_pipeline<2 * NDB, 2, 2>();
  }
  // Copies issued during the last step land in LDS that the next workgroup may own.
  wait_vmcnt<0>();

  // ---- epilogue: scale, round once to the storage dtype, store own rows
  const int oi = ow0 + l32;
  if (oi < own_len) {
    uint16_t* dst = (uint16_t*)(OWN_Q ? p.dq : p.dk) + own_base + (long long)oi * own_row;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = cg * C::DW + 32 * db + 8 * i4 + 4 * hh;
        if (d < p.d) {
          const f32x16_t& a = acc[db];
          const u32x2_t pk = {Elt<T>::pack2(a[4 * i4] * p.scale, a[4 * i4 + 1] * p.scale),
                              Elt<T>::pack2(a[4 * i4 + 2] * p.scale, a[4 * i4 + 3] * p.scale)};
          *(u32x2_t*)(dst + d) = pk;
        }
      }
  }
}

template <class T, int MODE, int NDB>
static hipError_t launch_bwd_rs(AttnParams p, hipStream_t st) {
  using C = RsCfg<NDB>;
  p.ntiles = ((MODE == kDQ ? p.nq : p.nkv) + C::BOWN - 1) / C::BOWN;
  p.total = p.batch * (MODE == kDQ ? p.hq : p.hkv) * p.ntiles;
  if (p.total == 0) return hipSuccess;
  const int grid = (p.total + 7) & ~7;
  hipLaunchKernelGGL((ffpa_bwd_rs_kernel<T, MODE, NDB>), dim3(grid), dim3(64 * C::NW), 0, st, p);
  return hipGetLastError();
}

template <class T, int MODE, int NC, int NDB>
static hipError_t launch_bwd_cfg(AttnParams p, hipStream_t st) {
  constexpr int NX = MODE != kDV ? 2 : 1;
  // Two waves per SIMD where the per-wave state fits 256 registers (dV for D <= 512), else one.
  constexpr int NW = (MODE == kDV && NC == 2) ? 8 : 4;
  using C1 = BwdCfg<NC, NDB, 1, NX, NW>;
  constexpr int NBUF = (2 * 2 * C1::TILE + C1::XBYTES) <= 160 * 1024 ? 2 : 1;
  using C = BwdCfg<NC, NDB, NBUF, NX, NW>;
  const bool own_q = MODE == kDQ;
  p.ntiles = ((own_q ? p.nq : p.nkv) + C::BOWN - 1) / C::BOWN;
  p.total = p.batch * (own_q ? p.hq : p.hkv) * p.ntiles;
  if (p.total == 0) return hipSuccess;
  const int grid = (p.total + 7) & ~7;
  hipLaunchKernelGGL((ffpa_bwd_kernel<T, MODE, NC, NDB, NBUF, NW>), dim3(grid), dim3(64 * NW), 0, st, p);
  return hipGetLastError();
}

template <class T, int MODE>
static hipError_t launch_bwd_mode(const AttnParams& p, hipStream_t st) {
  if constexpr (MODE != kDV) {
    if (p.d <= 512) {
      if (p.d > 384) return launch_bwd_rs<T, MODE, 4>(p, st);
      return launch_bwd_rs<T, MODE, 3>(p, st);
    }
  }
  if (p.d <= 512) {
    switch ((p.d + 63) / 64) {
      case 5: return launch_bwd_cfg<T, MODE, 2, 5>(p, st);
      case 6: return launch_bwd_cfg<T, MODE, 2, 6>(p, st);
      case 7: return launch_bwd_cfg<T, MODE, 2, 7>(p, st);
      default: return launch_bwd_cfg<T, MODE, 2, 8>(p, st);
    }
  }
  switch ((p.d + 127) / 128) {
    case 5: return launch_bwd_cfg<T, MODE, 4, 5>(p, st);
    case 6: return launch_bwd_cfg<T, MODE, 4, 6>(p, st);
    case 7: return launch_bwd_cfg<T, MODE, 4, 7>(p, st);
    default: return launch_bwd_cfg<T, MODE, 4, 8>(p, st);
  }
}

template <class T>
static hipError_t launch_stage_t(int stage, const AttnParams& p, int nrows, int varlen_total, hipStream_t st) {
  switch (stage) {
    case 0:
      if (nrows > 0) {
        const int blocks = (nrows + 15) / 16;
        hipLaunchKernelGGL(ffpa_bwd_preprocess_kernel<T>, dim3(blocks), dim3(256), 0, st, p, nrows, varlen_total);
        return hipGetLastError();
      }
      return hipSuccess;
    case 1: return launch_bwd_mode<T, kDV>(p, st);
    case 2: return launch_bwd_mode<T, kDK>(p, st);
    default: return launch_bwd_mode<T, kDQ>(p, st);
  }
}

// Stage 0 = preprocess, 1 = dV, 2 = dK, 3 = dQ; -1 runs all four in order.
hipError_t launch_bwd(const AttnParams& p, int fp16, int nrows, int varlen_total, hipStream_t st, int stage) {
  for (int s = stage < 0 ? 0 : stage; s <= (stage < 0 ? 3 : stage); ++s) {
    const hipError_t e = fp16 ? launch_stage_t<FP16>(s, p, nrows, varlen_total, st)
                              : launch_stage_t<BF16>(s, p, nrows, varlen_total, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ffpa
