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
// Two paths. With a caller's P/dS workspace, one kernel forms P and dS for every (query, key) pair
// and stores them (8 waves; D <= 512 in two head-dim halves, above in four quarters), and dK, dV
// and dQ become plain products of the stored blocks (8 waves each, or one launch of all three for
// small grids). Without it, the stages recompute: for D <= 512 dV runs 8 waves (NC = 2) and dK/dQ
// the 8-wave reduce-scatter variant (NC = 4), at two waves per SIMD; larger head dims use 4 waves
// (NC = 4), one per SIMD.
#include <algorithm>

#include "ffpa_device.h"
#include "ffpa_params.h"

namespace ffpa {
// Fixed pipelining and cache-policy constants of the backward kernels (measured choices).
// MFMAs whose LDS operands are requested ahead of the one issuing (see pin_lds_mfma_pipeline).
constexpr int kBwdAhead = 2;
// Cache policy of the dS and P stores (written once, read once by the dQ and dV passes):
// non-temporal, system scope (nt sc1), the fastest of the policies measured for this pattern.
constexpr int kDsStoreCpol = 18;
// LDS reads requested ahead of the MFMA issuing in the dQ-from-dS and dV-from-P products (each
// A operand is two transposed reads used by two MFMAs).
constexpr int kProdAhead = 6;
// Depth of the product passes' tile rings (copies are issued kProdNbuf - 1 steps ahead).
constexpr int kProdNbuf = 3;
// Same as kBwdAhead, for the two MFMA phases of the two-group dK/dQ kernel, whose MFMA phases run
// one wave per SIMD at a time.
constexpr int kPpAheadM1 = 2;
constexpr int kPpAheadM2 = 2;

// ------------------------------------------------------------------------------------------------
// Stage 1: Delta = rowsum(dO * O) in fp32 from the stored (rounded) O, minus the gradient of the
// returned LSE when there is one: d LSE_i / d S_ij = P_ij, so a loss term g_i LSE_i adds g_i P_ij to
// dS = P (dP - Delta), which is the same as Delta_i - g_i in place of Delta_i.
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
      p.delta[idx] = p.dlse != nullptr ? acc[r] - p.dlse[idx] : acc[r];
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

// The O(N)-memory form (no P/dS workspace; the attn_mask backward always uses the workspace).
template <class T, int MODE, int NC, int NDB, int NBUF, int NW>
__global__ void __launch_bounds__(64 * NW, NW / 4) ffpa_bwd_kernel(AttnParams p) {
  constexpr bool OWN_Q = MODE == kDQ;   // stationary rows are queries (dQ) or keys (dK, dV)
  constexpr bool HAS_DP = MODE != kDV;  // dK and dQ need dP = dO V^T
  constexpr int NX = HAS_DP ? 2 : 1;
  using C = BwdCfg<NC, NDB, NBUF, NX, NW>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  lds_t* smem = (lds_t*)smem_raw;

  const int L = blockIdx.x;
  const int heads = OWN_Q ? p.hq : p.hkv;
  const int item = xcd_item(L, gridDim.x, p.cu_q != nullptr, heads, p.ntiles);
  if (item >= p.total) return;
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
  // dK/dV: query tiles from the last down, each for every head of the group (the workgroups of a
  // causal grid then start at the same tile and sweep the same query rows together, as in the
  // products from the stored blocks).
  auto step_head = [&](int st) { return OWN_Q ? hd / p.group : hd * p.group + st % p.group; };
  auto step_row0 = [&](int st) { return OWN_Q ? st * 32 : (qt_first + nqt - 1 - st / p.group) * 32; };
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
    pin_lds_mfma_pipeline<KSTEPS * (HAS_DP ? 2 : 1), kBwdAhead, 1>();
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
    pin_lds_mfma_pipeline<2 * NDB, kBwdAhead, 2>();

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
// dK and dQ for D <= 512 with two waves per SIMD, as a two-group ping-pong.
//
// Eight waves form two row groups of NC = 4; a wave holds 32 stationary rows x D/4 head-dim
// columns of both stationary operands and of the fp32 accumulator, which fits 256 registers.
// One step over 32 streamed rows is four phases per wave:
//   M1a, M1b  partial S and dP over the wave's head-dim columns (split in two runs of MFMAs), then
//             the partner quarters go to the exchange buffer;
//   V1        reduce-scatter: wave cg finishes the 8 streamed rows of register quarter cg, computes
//             dS for them and writes its bf16 dS quarter (a quarter of the softmax-gradient work
//             per wave, half the partial-sum bytes of a full all-reduce);
//   M2        all-gather of the dS quarters, then the accumulating product with its A operand read
//             transposed from tile 1.
// The second row group runs two phases behind the first, and every phase ends at a workgroup
// barrier. The two waves of a SIMD (one per group) are then always in different phases: while one
// does the exchange and the exponentials (V1) or issues the gather, the other keeps the SIMD's
// matrix core busy, instead of both waiting on the same exchange at the same time.
//
//   slot:     0              1               2              3
//   group 0:  M1a(st)        M1b(st)         V1(st)         M2(st)
//   group 1:  V1(st-1)       M2(st-1)        M1a(st)        M1b(st)
//
// Buffers: tiles 1 and 2 are double-buffered; the exchange and dS-gather buffers are shared by the
// two groups (a group writes them in one slot and reads them in the next, while the other group
// is between its own write and read). Copies of step st + 1: tile 2 by group 0 during M1a(st),
// tile 1 by group 1 during M1a(st) (after group 1's M2(st-1) released that buffer), dK's row
// statistics by wave 0 at M1b(st); all complete before slot 0 of step st + 1.
// ------------------------------------------------------------------------------------------------
template <int NDB>
struct PpCfg {
  static constexpr int NC = 4, NW = 8;
  static constexpr int DW = NDB * 32;
  static constexpr int RS = 1024;                // LDS row stride (bytes), padded head dim <= 512
  static constexpr int BOWN = 2 * 32;            // stationary rows per workgroup
  static constexpr int TILE = 32 * RS;
  static constexpr int PIECE = 64 * 16;          // one f32x4 per lane
  static constexpr int T1_OFF = 0;               // [2] tile 1
  static constexpr int T2_OFF = 2 * TILE;        // [2] tile 2
  static constexpr int X_OFF = 4 * TILE;         // [cg][3 partner quarters][S, dP] pieces
  static constexpr int G_OFF = X_OFF + NC * 3 * 2 * PIECE;  // [cg] packed dS quarter, 8 B/lane
  static constexpr int ST_OFF = G_OFF + NC * 64 * 8;        // [buffer][LSE, Delta] x 64 floats
  static constexpr int LDS = ST_OFF + 2 * 2 * 256;
  static constexpr int NCOPY = TILE / 1024 / 4;  // copies per wave of a tile (one group copies it)
  static constexpr int KSTEPS = 2 * NDB;         // k-steps of the partial products
  static constexpr int KA = (3 * KSTEPS) / 4;    // k-steps in M1a (M1b shares its slot with M2)
  static_assert(4 * DW <= 512 && LDS <= 160 * 1024, "LDS budget");
};

template <class T, int MODE, int NDB>
__global__ void __launch_bounds__(512, 2) ffpa_bwd_pp_kernel(AttnParams p) {
  static_assert(MODE == kDQ || MODE == kDK, "dK and dQ only");
  constexpr bool OWN_Q = MODE == kDQ;
  using C = PpCfg<NDB>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  lds_t* smem = (lds_t*)smem_raw;

  const int L = blockIdx.x;
  const int heads = OWN_Q ? p.hq : p.hkv;
  const int item = xcd_item(L, gridDim.x, p.cu_q != nullptr, heads, p.ntiles);
  if (item >= p.total) return;
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
  const int grp = w >> 2;  // 0: leading row group, 1: trailing row group
  const int cg = w & 3;
  const int ow0 = o0 + grp * 32;
  const int off = sv.lk - sv.lq;

  // ---- stationary operands: lane (h, n) holds own row n, dims 16 kb + 8 h + 0..7
  const int own_row = OWN_Q ? p.q_row : p.k_row;
  const long long own_base = OWN_Q ? sv.q_off + (long long)hd * p.q_head : sv.k_off + (long long)hd * p.k_head;
  const uint16_t* r1src = (const uint16_t*)(OWN_Q ? p.q : p.k) + own_base;
  const uint16_t* r2src = (const uint16_t*)(OWN_Q ? p.dout : p.v) + own_base;
  u32x4_t r1[C::KSTEPS], r2[C::KSTEPS];
  {
    const long long oi = min(ow0 + l32, own_len - 1);
#pragma unroll
    for (int kb = 0; kb < C::KSTEPS; ++kb) {
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
  // dK/dV: query tiles from the last down, each for every head of the group (the workgroups of a
  // causal grid then start at the same tile and sweep the same query rows together, as in the
  // products from the stored blocks).
  auto step_head = [&](int st) { return OWN_Q ? hd / p.group : hd * p.group + st % p.group; };
  auto step_row0 = [&](int st) { return OWN_Q ? st * 32 : (qt_first + nqt - 1 - st / p.group) * 32; };
  auto str_base = [&](int head) {
    return OWN_Q ? sv.k_off + (long long)head * p.k_head : sv.q_off + (long long)head * p.q_head;
  };
  const uint32_t span = (uint32_t)min((long long)max(str_len, 1) * row_bytes, (long long)0xFFFFFFF0);
  const int dch = p.d >> 3;
  // Copy ii of this wave fills tile row i = cg + 4 ii; lane l writes physical chunk l, holding
  // logical chunk l ^ swz(i) (clamped into the head dim). swz(i) depends on ii % 4 only.
  int voff[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) voff[ii] = min(lane ^ swz(cg + 4 * ii), dch - 1) << 4;

  // Source of step st (clamped to the last step: copies past the end land in buffers that are not
  // read again). This group's tile: tile 2 for group 0, tile 1 for group 1.
  struct StepSrc {
    i32x4_t rs;
    int row0, head;
  };
  auto step_src = [&](int st) {
    st = min(st, nsteps - 1);
    StepSrc x;
    x.head = step_head(st);
    x.row0 = step_row0(st);
    const uint16_t* src = grp == 0 ? (const uint16_t*)(OWN_Q ? p.v : p.dout) : (const uint16_t*)(OWN_Q ? p.k : p.q);
    x.rs = make_rsrc(src + str_base(x.head), span);
    return x;
  };
  auto copy_tile = [&](const StepSrc& x, int buf, int ii) {
    const int i = cg + 4 * ii;
    lds_t* dst = smem + (grp == 0 ? C::T2_OFF : C::T1_OFF) + buf * C::TILE + i * 1024;
    dma16_buf(x.rs, voff[ii & 3], min(x.row0 + i, str_len - 1) * row_bytes, dst);
  };
  auto copy_stats = [&](int st, int buf) {
    if constexpr (!OWN_Q) {
      st = min(st, nsteps - 1);
      const long long li = sv.lse_off + (long long)step_head(st) * p.lse_head;
      const uint32_t bytes = (uint32_t)max(sv.lq, 1) * 4;
      const int vo = min(step_row0(st) + l32, sv.lq - 1) * 4;
      lds_t* sd = smem + C::ST_OFF + buf * 512;
      dma4_buf(make_rsrc(p.lse_in + li, bytes), vo, sd);
      dma4_buf(make_rsrc(p.delta + li, bytes), vo, sd + 256);
    }
  };

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
  auto t1_addr = [&](int st) { return lds_addr(smem + C::T1_OFF + (st & 1) * C::TILE); };
  auto t2_addr = [&](int st) { return lds_addr(smem + C::T2_OFF + (st & 1) * C::TILE); };
  // MFMA index (of a run of n) after which copy ii is issued: the copy path moves about 64 B per
  // clock per CU, so a whole tile issued at once would hold the waves at the issue.
  auto spread_at = [](int n, int ii) { return (ii * n) / C::NCOPY; };

  f32x16_t sacc, dpacc;
  f32x4_t sq_own, dq_own;  // this wave's own quarter of the partial S and dP, kept for V1
  uint32_t bop[2][4];

  // ---- phase M1a: first KA k-steps of the partial products, with this group's copies of st + 1
  auto m1a = [&](int st) {
    const uint32_t t1 = t1_addr(st), t2 = t2_addr(st);
    const StepSrc xn = step_src(st + 1);
    const int nb = (st + 1) & 1;
    sacc = (f32x16_t){};
    dpacc = (f32x16_t){};
#pragma unroll
    for (int kb = 0; kb < C::KA; ++kb) {
      sacc = Elt<T>::mma(lds_read_b128_at(a_addr(t1, kb)), r1[kb], sacc);
      dpacc = Elt<T>::mma(lds_read_b128_at(a_addr(t2, kb)), r2[kb], dpacc);
#pragma unroll
      for (int ii = 0; ii < C::NCOPY; ++ii)
        if (kb == spread_at(C::KA, ii)) copy_tile(xn, nb, ii);
    }
    pin_lds_mfma_pipeline<2 * C::KA, kPpAheadM1, 1>();
  };
  // ---- phase M1b: remaining k-steps, then the partner quarters to the exchange buffer
  auto m1b = [&](int st) {
    if (grp == 0 && w == 0) copy_stats(st + 1, (st + 1) & 1);
    const uint32_t t1 = t1_addr(st), t2 = t2_addr(st);
#pragma unroll
    for (int kb = C::KA; kb < C::KSTEPS; ++kb) {
      sacc = Elt<T>::mma(lds_read_b128_at(a_addr(t1, kb)), r1[kb], sacc);
      dpacc = Elt<T>::mma(lds_read_b128_at(a_addr(t2, kb)), r2[kb], dpacc);
    }
    pin_lds_mfma_pipeline<2 * (C::KSTEPS - C::KA), (kPpAheadM1 < 2 * (C::KSTEPS - C::KA) ? kPpAheadM1 : 2 * (C::KSTEPS - C::KA)), 1>();
    // Slot j holds register quarter j + 1, i.e. quarter (cg + 1 + j) % 4.
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int q = j + 1;
      const int base = ((cg * 3 + j) * 2) * C::PIECE + lane * 16;
      lds_write_f4(xbuf, base, (f32x4_t){sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]});
      lds_write_f4(xbuf, base + C::PIECE,
                   (f32x4_t){dpacc[4 * q], dpacc[4 * q + 1], dpacc[4 * q + 2], dpacc[4 * q + 3]});
    }
    sq_own = (f32x4_t){sacc[0], sacc[1], sacc[2], sacc[3]};
    dq_own = (f32x4_t){dpacc[0], dpacc[1], dpacc[2], dpacc[3]};
  };
  // ---- phase V1: reduce this wave's quarter (own part + partners in a fixed order), P and dS
  u32x2_t mine;
  auto v1 = [&](int st) {
    f32x4_t sq = sq_own, dq = dq_own;
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      const int pc = (cg + i) & 3;        // partner column group
      const int j = ((cg - pc) & 3) - 1;  // its slot holding quarter cg
      const int base = ((pc * 3 + j) * 2) * C::PIECE + lane * 16;
      sq = sq + lds_read_f4(xbuf, base);
      dq = dq + lds_read_f4(xbuf, base + C::PIECE);
    }
    f32x4_t lse2q, dltq;
    if constexpr (OWN_Q) {
      lse2q = (f32x4_t){lse2_own, lse2_own, lse2_own, lse2_own};
      dltq = (f32x4_t){dlt_own, dlt_own, dlt_own, dlt_own};
    } else {
      const lds_t* sd = smem + C::ST_OFF + (st & 1) * 512;
      const f32x4_t lr = lds_read_f4(sd, qrow * 4);
      dltq = lds_read_f4(sd, 256 + qrow * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) lse2q[i] = lr[i] == -INFINITY ? INFINITY : lr[i] * kLog2e;
    }
    const int row0 = step_row0(st);
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
    mine = (u32x2_t){Elt<T>::pack2(ds[0], ds[1]), Elt<T>::pack2(ds[2], ds[3])};
    *(__attribute__((address_space(3))) u32x2_t*)(gbuf + cg * 512 + lane * 8) = mine;
  };
  // ---- phase M2: all-gather dS (quarter q gives B-operand words 2 (q % 2), +1 of k-block q / 2),
  // then acc^T[d][own] += A[d][streamed] * dS[streamed][own], A read transposed from tile 1
  auto m2 = [&](int st) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x2_t v = mine;
      if (q != cg) v = *(const __attribute__((address_space(3))) u32x2_t*)(gbuf + q * 512 + lane * 8);
      bop[q >> 1][2 * (q & 1)] = v.x;
      bop[q >> 1][2 * (q & 1) + 1] = v.y;
    }
    const uint32_t t1 = t1_addr(st);
    // k-block outer, head-dim block inner: consecutive MFMAs use different accumulators (two
    // dependent MFMAs in a row issue 44 instead of 32 cycles apart, and here only one wave per
    // SIMD is multiplying).
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const s16x4_t lo = lds_read_tr16_at(t_addr(t1, db, kb2, 0));
        const s16x4_t hi = lds_read_tr16_at(t_addr(t1, db, kb2, 1));
        const u32x4_t bv = {bop[kb2][0], bop[kb2][1], bop[kb2][2], bop[kb2][3]};
        acc[db] = Elt<T>::mma(join_tr(lo, hi), bv, acc[db]);
      }
    }
    pin_lds_mfma_pipeline<2 * NDB, kPpAheadM2, 2>();
  };

  if (nsteps > 0) {
    const StepSrc x0 = step_src(0);
#pragma unroll
    for (int ii = 0; ii < C::NCOPY; ++ii) copy_tile(x0, 0, ii);
    if (w == 0) copy_stats(0, 0);
  }
  wait_all();  // stationary operands, dQ's row statistics and the tiles of step 0
  lds_barrier();

  // Each group runs its own straight-line loop of four phases per step, so that its accumulators
  // stay in place; both run 4 nsteps + 2 barriers, group 1 two slots later than group 0. Every
  // copy of step st + 1 has been issued by the end of slot 3 of step st (group 0 in its M1a,
  // group 1 in its M1a two slots later): each wave completes its own before that barrier.
  if (nsteps > 0) {
    if (grp == 0) {
      for (int st = 0; st < nsteps; ++st) {
        m1a(st);
        lds_barrier();
        m1b(st);
        lds_barrier();
        v1(st);
        lds_barrier();
        m2(st);
        wait_vmcnt<0>();  // the tile copies (M1a) and the row statistics (M1b)
        lds_barrier();
      }
      lds_barrier();
      lds_barrier();
    } else {
      lds_barrier();
      lds_barrier();
      for (int st = 0; st < nsteps; ++st) {
        m1a(st);
        lds_barrier();
        m1b(st);
        wait_vmcnt<0>();
        lds_barrier();
        v1(st);
        lds_barrier();
        m2(st);
        lds_barrier();
      }
    }
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
static hipError_t launch_bwd_pp(AttnParams p, hipStream_t st) {
  using C = PpCfg<NDB>;
  p.ntiles = ((MODE == kDQ ? p.nq : p.nkv) + C::BOWN - 1) / C::BOWN;
  p.total = p.batch * (MODE == kDQ ? p.hq : p.hkv) * p.ntiles;
  if (p.total == 0) return hipSuccess;
  const int grid = (p.total + 7) & ~7;
  hipLaunchKernelGGL((ffpa_bwd_pp_kernel<T, MODE, NDB>), dim3(grid), dim3(64 * C::NW), 0, st, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// P and dS for the stored-P/dS backward (D <= 512): P = exp(scale S - LSE) and dS = P (dP - Delta)
// of every (query, key) pair, rounded to the storage dtype, with dP = dO V^T. No accumulator: the
// gradients are products of the stored blocks (dK = scale dS^T Q, dV = P^T dO, dQ = scale dS K).
//
// The layout is the forward kernel's: a workgroup owns 128 queries of one head as 4 row groups x
// 2 head-dim halves (8 waves, two per SIMD); each wave keeps its 32 queries' Q and dO columns in
// registers (B operands) and forms the partial S^T = K Q^T and dP^T = V dO^T over its half from
// K and V tiles (32 keys x 1 KB, XOR-swizzled) streamed through LDS. The two halves are combined by
// a reduce-scatter: the A operand rows of the wave with head-dim half c are rotated by 16 c, so
// its registers 0..7 hold keys 16 c + 8 h + 0..7 of the tile (the keys it finishes) and registers
// 8..15 the partner's, which go to the exchange buffer. After the exchange, lane (h, query n)
// holds 8 consecutive keys of its query. P and dS are stored transposed (one row per key, queries
// contiguous), so that the two waves of a group that share a head-dim half complete whole 128-byte
// lines of a key row in the same slot: each wave turns its 32 queries x 16 keys into 16-byte pieces
// of 8 queries of one key with one LDS write and two transposed reads per block. LSE and Delta are
// per lane (one query per lane).
//
// Two-group schedule (as in the forward): waves 0-3 and 4-7 run half a step apart, so in every
// slot one wave of each SIMD multiplies while the other exchanges, exponentiates and stores.
//   slot 2j:     group 0 multiplies tile j   | group 1 finishes tile j - 1 and copies tile j + 1
//   slot 2j + 1: group 0 finishes tile j     | group 1 multiplies tile j
// Tile j + 1 goes into the buffer of tile j - 1, which group 1 last read in slot 2j - 1, and group
// 1 completes the copies before the barrier that ends slot 2j + 1. All copies are issued by the
// finishing group: the multiplying waves issue nothing but LDS reads and MFMAs. (j counts the
// item's steps; with a key-range split, step j covers key tile split + j nsplit.)
// ------------------------------------------------------------------------------------------------
// Stationary B operands of a P/dS wave (its 32 queries x one head-dim part of at most 512 bytes),
// staged through 16 KB of LDS so that the copies read whole rows: copy i brings rows 2 i and
// 2 i + 1 (lane (h', c): row 2 i + h', 16-byte chunk c ^ row of the part, so that the reads below
// hit distinct banks), then lane (h, n) reads query n, columns col0 + 16 kb + 8 h + 0..7. Loading
// the B layout directly reads 32 rows x 32 bytes per instruction, which takes about twice as long
// per workgroup. Rows at or past lq repeat row lq - 1; columns at or past the head dim are zero.
// Only the calling wave touches `stage`; it waits for its own reads before returning.
template <int KSTEPS>
__device__ __forceinline__ void stage_b_operand(const uint16_t* head, long long row_elems, int row0, int lq,
                                                int col0, int d, lds_t* stage, u32x4_t (&dst)[KSTEPS]) {
  constexpr int NCH = 2 * KSTEPS;  // 16-byte chunks of the part
  static_assert(NCH <= 32, "at most 512 bytes of columns per wave");
  const int lane = threadIdx.x & 63, hh = lane >> 5, l32 = lane & 31;
  const uint32_t span = (uint32_t)min(((long long)(lq - 1) * row_elems + d) * 2, (long long)0xFFFFFFF0);
  const i32x4_t rs = make_rsrc(head, span);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 2 * i + hh;
    const long long row = min(row0 + r, lq - 1);
    const int col = min(col0 + min(l32 ^ r, NCH - 1) * 8, d - 8);
    dma16_buf(rs, (int)(uint32_t)((row * row_elems + col) * 2), 0, stage + i * 1024);
  }
  wait_vmcnt<0>();
#pragma unroll
  for (int kb = 0; kb < KSTEPS; ++kb) {
    const u32x4_t x = lds_read_b128(stage, l32 * 512 + (((2 * kb + hh) ^ l32) << 4));
    dst[kb] = col0 + kb * 16 + hh * 8 < d ? x : (u32x4_t){0u, 0u, 0u, 0u};
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));  // the reads are done: `stage` may be rewritten
}

// LDS operands requested ahead in the P/dS kernel's score products.
constexpr int kPdsAhead = 2;
template <int NDB>
struct PdsCfg {
  static constexpr int NW = 8;
  static constexpr int DW = NDB * 32;              // head-dim columns per wave (half the head)
  static constexpr int KSTEPS = 2 * NDB;           // 16-wide k-steps over them
  static constexpr int RS = 1024;                  // LDS row stride (bytes)
  static constexpr int BQ = 4 * 32;                // queries per workgroup
  static constexpr int TILE = 32 * RS;
  static constexpr int XWAVE = 4 * 64 * 16;        // per wave: the partner's half of S and dP
  static constexpr int LDS = 4 * TILE + 8 * XWAVE;  // [buffer][K, V] tiles, exchange
  static constexpr int GCOPY = TILE / 1024 / 4;    // 1 KB copies per wave of a tile (one group)
  // Each head-dim half owns a 32-chunk (512-byte) slot of an LDS row, its WCH chunks first, so its
  // operands start on a 16-chunk boundary and every operand address is one per-lane base XOR a
  // constant (the row swizzle flips only address bits 4-7).
  static constexpr int WCH = NDB * 4;
  static constexpr int SLOT = 32;
  static_assert(2 * DW <= 512 && LDS <= 160 * 1024 && WCH <= SLOT && 2 * SLOT * 16 == RS, "LDS budget");
};

template <class T, int NDB, bool MASK>
__global__ void __launch_bounds__(512, 2) ffpa_pds_kernel(AttnParams p) {
  using C = PdsCfg<NDB>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  lds_t* smem = (lds_t*)smem_raw;
  auto kbuf = [&](int b) { return smem + (2 * b) * C::TILE; };
  auto vbuf = [&](int b) { return smem + (2 * b + 1) * C::TILE; };
  lds_t* const xbuf = smem + 4 * C::TILE;

  // Work item (sequence, query head, query tile, key range): grids too small to fill the GPU
  // split each tile's key tiles into p.nsplit interleaved sets (P and dS of different keys are
  // independent).
  const int L = blockIdx.x;
  const int item = xcd_item(L, gridDim.x, p.cu_q != nullptr, p.hq, p.ntiles * p.nsplit);
  if (item >= p.total) return;
  const int split = item % p.nsplit;
  const HeadTile ht = head_tile(item / p.nsplit, p.ntiles, p.hq, p.group, p.cu_q == nullptr);
  int t = ht.t;
  const int h = ht.h;
  const int s = ht.s;
  if (p.causal) t = p.ntiles - 1 - t;  // heaviest causal tiles first

  const SeqView sv = seq_view(p, s);
  const int qt0 = t * C::BQ;
  if (qt0 >= sv.lq) return;
  const DsView dsv = ds_view(p, s, sv);
  const int kvh = h / p.group;

  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int grp = w >> 2;
  const int wg = w & 3;
  const int rg = w >> 1;
  const int cg = w & 1;
  const int qw0 = qt0 + rg * 32;
  const int off = sv.lk - sv.lq;

  const int row_bytes = p.k_row * 2;
  const long long kv_off = sv.k_off + (long long)kvh * p.k_head;
  const uint32_t span = (uint32_t)min((long long)max(sv.lk, 1) * row_bytes, (long long)0xFFFFFFF0);
  const i32x4_t krs = make_rsrc((const uint16_t*)p.k + kv_off, span);
  const i32x4_t vrs = make_rsrc((const uint16_t*)p.v + kv_off, span);
  int kend = sv.lk;
  if (p.causal) kend = min(kend, qt0 + C::BQ + off);
  const int ntk = kend > 0 ? (kend + 31) >> 5 : 0;
  // This item's key tiles: every nsplit-th of the query tile's own range, from tile `split` on
  // (step jj covers key tile split + jj nsplit). Interleaved, not contiguous, so that the ranges
  // of all the grid's items start at the first key tiles and sweep the keys together (shared K/V
  // lines in L2).
  const int nsteps = split < ntk ? (ntk - split + p.nsplit - 1) / p.nsplit : 0;
  auto tile_of = [&](int jj) { return split + jj * p.nsplit; };
  if (nsteps == 0 && split > 0) return;

  // The query's LSE in log2 units (+inf for a row without a legal key makes P = 0) and Delta.
  const int qi = qw0 + l32;
  const long long li = sv.lse_off + (long long)h * p.lse_head + min(qi, sv.lq - 1);
  const float lse_raw = p.lse_in[li];
  const float lse2 = lse_raw == -INFINITY ? INFINITY : lse_raw * kLog2e;
  const float dlt = p.delta[li];
  // Q and dO columns of this wave as B operands: lane (h, n) holds query n, dims 16 kb + 8 h + 0..7,
  // staged through the tile buffers (16 KB per wave) before the first tile is copied.
  u32x4_t qreg[C::KSTEPS], oreg[C::KSTEPS];
  {
    const long long hq0 = sv.q_off + (long long)h * p.q_head;
    lds_t* const stage = smem + w * 16384;
    stage_b_operand<C::KSTEPS>((const uint16_t*)p.q + hq0, p.q_row, qw0, sv.lq, cg * C::DW, p.d, stage, qreg);
    stage_b_operand<C::KSTEPS>((const uint16_t*)p.dout + hq0, p.q_row, qw0, sv.lq, cg * C::DW, p.d, stage, oreg);
  }
  lds_barrier();  // every wave has read its staged operands: the tile buffers are free

  // The head's P and dS blocks (Lk rows of round_up(Lq, 8) queries).
  const long long hoff = dsv.base + (long long)h * dsv.head;
  const int nrec = (int)((long long)sv.lk * dsv.row * 2);
  const __amdgpu_buffer_rsrc_t ds_rs = __builtin_amdgcn_make_buffer_rsrc((uint16_t*)p.ds + hoff, 0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t p_rs = __builtin_amdgcn_make_buffer_rsrc((uint16_t*)p.pst + hoff, 0, nrec, 0x00020000);

  // Copies: instruction ii of a wave of a group fills tile row i = wg + 4 ii of that group's tile;
  // lane l writes physical chunk l, whose un-swizzled index u = l ^ swz(i) is chunk u % SLOT of
  // half u / SLOT (padding and chunks past the head dim hold clamped, finite duplicates).
  const int dch = p.d >> 3;
  auto src_chunk = [&](int u) { return min((u / C::SLOT) * C::WCH + min(u % C::SLOT, C::WCH - 1), dch - 1); };
  int gvoff[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) gvoff[ii] = src_chunk(lane ^ swz(wg + 4 * ii)) << 4;
  auto gcopy = [&](const i32x4_t& rs, lds_t* tile, int j, int ii) {
    const int i = wg + 4 * ii;
    dma16_buf(rs, gvoff[ii & 3], min(j * 32 + i, sv.lk - 1) * row_bytes, tile + i * 1024);
  };

  // K and V rows (A operands): MFMA row m reads tile row row_perm(m) ^ 16 cg (see above).
  const int krow = row_perm(l32) ^ (16 * cg);
  const int kswz = swz(krow);
  const int cbase = cg * C::SLOT;
  const uint32_t klane = krow * C::RS + (cbase << 4) + ((hh ^ kswz) << 4);
  auto a_addr = [&](uint32_t tile, int kb) -> uint32_t {
    return ((tile + klane) ^ ((kb & 7) << 5)) + ((kb >> 3) << 8);
  };

  f32x16_t sacc, pacc;
  // attn_mask bits of this lane's 8 keys of tile j: requested when the tile's products start (the
  // multiplying phase issues no copies), used after the exchange.
  const long long mrow = MASK ? mask_row(p, s, h, min(qi, sv.lq - 1)) : 0;
  u32x4_t mraw;
  // Partial S^T and dP^T of step jj (key tile j) over this wave's half; the partner's rows go to
  // the exchange.
  auto m_phase = [&](int jj) {
    const int j = tile_of(jj);
    const uint32_t kt = lds_addr(kbuf(jj & 1)), vt = lds_addr(vbuf(jj & 1));
    if constexpr (MASK) {
      mraw = mask_block(p, mrow, j * 32 + 16 * cg + 8 * hh, sv.lk);
      __builtin_amdgcn_sched_barrier(0);  // issued here, not sunk behind the products
    }
    sacc = (f32x16_t){};
    pacc = (f32x16_t){};
#pragma unroll
    for (int kb = 0; kb < C::KSTEPS; ++kb) {
      sacc = Elt<T>::mma(lds_read_b128_at(a_addr(kt, kb)), qreg[kb], sacc);
      pacc = Elt<T>::mma(lds_read_b128_at(a_addr(vt, kb)), oreg[kb], pacc);
    }
    pin_lds_mfma_pipeline<2 * C::KSTEPS, kPdsAhead, 1>();
#pragma unroll
    for (int r4 = 0; r4 < 2; ++r4) {
      lds_write_f4(xbuf, ((w * 4 + r4) * 64 + lane) * 16,
                   (f32x4_t){sacc[8 + 4 * r4], sacc[9 + 4 * r4], sacc[10 + 4 * r4], sacc[11 + 4 * r4]});
      lds_write_f4(xbuf, ((w * 4 + 2 + r4) * 64 + lane) * 16,
                   (f32x4_t){pacc[8 + 4 * r4], pacc[9 + 4 * r4], pacc[10 + 4 * r4], pacc[11 + 4 * r4]});
    }
  };
  // Full S and dP of this lane's 8 keys (own half + partner's), then P, dS and their stores.
  auto e_phase = [&](int jj, auto&& copies) {
    const int j = tile_of(jj);
    const int pw = w ^ 1;
    float sf[8], df[8];
#pragma unroll
    for (int r4 = 0; r4 < 2; ++r4) {
      const f32x4_t a = lds_read_f4(xbuf, ((pw * 4 + r4) * 64 + lane) * 16);
      const f32x4_t b = lds_read_f4(xbuf, ((pw * 4 + 2 + r4) * 64 + lane) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sf[4 * r4 + i] = sacc[4 * r4 + i] + a[i];
        df[4 * r4 + i] = pacc[4 * r4 + i] + b[i];
      }
    }
    if constexpr (MASK) {
      // attn_mask terms of this lane's 8 keys (added to the scores before P). The empty asm keeps
      // the sums, and so the wait for the mask load, ahead of the copies issued next.
      float mb[8];
      mask_apply8_block<T>(p, mraw, mrow, j * 32 + 16 * cg + 8 * hh, sv.lk, mb);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sf[e] += mb[e];
        asm volatile("" ::"v"(sf[e]));
      }
    }
    copies();
    const int key0 = j * 32 + 16 * cg + 8 * hh;
    const bool need_mask = (j * 32 + 32 > sv.lk) || (p.causal && j * 32 + 31 > qw0 + off);
    const int lim = p.causal ? min(qi + off, sv.lk - 1) : sv.lk - 1;
    uint32_t pk[4], dk[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      float pv[2], dv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * e2 + u;
        float pe = fast_exp2(sf[e] * p.scale_log2 - lse2);
        if (need_mask) pe = key0 + e <= lim ? pe : 0.f;
        pv[u] = pe;
        dv[u] = pe * (df[e] - dlt);
      }
      pk[e2] = Elt<T>::pack2(pv[0], pv[1]);
      dk[e2] = Elt<T>::pack2(dv[0], dv[1]);
    }
    // Transpose through this wave's inbox, free once read: lane (h, n) writes the 16 keys of query
    // n as a 32-byte row (its half at 16 h); in 16-lane group g, source lane s = 4 e + t points at
    // query row 8 g + e (+ 4 in the second read), keys 4 t .. 4 t + 3, so lane i receives key i and
    // queries 8 g + 0..7.
    lds_t* const tb = xbuf + (w ^ 1) * C::XWAVE;
    const int wo = l32 * 32 + hh * 16;
    lds_write_b128(tb, wo, (u32x4_t){pk[0], pk[1], pk[2], pk[3]});
    lds_write_b128(tb, 1024 + wo, (u32x4_t){dk[0], dk[1], dk[2], dk[3]});
    const int s16 = lane & 15, g = lane >> 4;
    const int ro = (8 * g + (s16 >> 2)) * 32 + 8 * (s16 & 3);
    const u32x4_t pt = join_tr(lds_read_tr16(tb, ro), lds_read_tr16(tb, ro + 128));
    const u32x4_t dt = join_tr(lds_read_tr16(tb, 1024 + ro), lds_read_tr16(tb, 1024 + ro + 128));
    // Pieces of keys at or past Lk, or starting at or past the padded row end, get an offset past
    // the block, which the buffer range check discards.
    const int key = j * 32 + 16 * cg + s16;
    const int q8 = qw0 + 8 * g;
    const bool ok = key < sv.lk && q8 < dsv.row;
    const uint32_t boff = ok ? (uint32_t)(((long long)key * dsv.row + q8) * 2) : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, pt), p_rs, (int)boff, 0, kDsStoreCpol);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, dt), ds_rs, (int)boff, 0, kDsStoreCpol);
  };

  if (nsteps > 0) {
    // The first step's tile by all waves (rows w + 8 ii of K and V).
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = w + 8 * ii;
      const int row = min(tile_of(0) * 32 + i, sv.lk - 1) * row_bytes;
      const int vo = src_chunk(lane ^ swz(i)) << 4;
      dma16_buf(krs, vo, row, kbuf(0) + i * 1024);
      dma16_buf(vrs, vo, row, vbuf(0) + i * 1024);
    }
  }
  wait_all();  // the stationary operands, LSE, Delta and tile 0
  lds_barrier();

  if (nsteps > 0) {
    if (grp == 0) {
      // Only stores leave this group's waves inside the loop; they are not waited for.
      for (int jj = 0; jj < nsteps; ++jj) {
        m_phase(jj);
        lds_barrier();
        e_phase(jj, [] {});
        lds_barrier();
      }
      lds_barrier();
    } else {
#pragma unroll
      for (int ii = 0; ii < C::GCOPY; ++ii) {
        gcopy(krs, kbuf(1), tile_of(1), ii);
        gcopy(vrs, vbuf(1), tile_of(1), ii);
      }
      lds_barrier();
      for (int jj = 0; jj < nsteps; ++jj) {
        m_phase(jj);
        // The next step's tile (copied in the prologue, or in the finishing phase of the step
        // before, followed there by that step's two stores and then this step's mask load, which
        // may stay in flight).
        if (jj == 0) wait_vmcnt<0>(); else wait_vmcnt<MASK ? 3 : 2>();
        lds_barrier();
        e_phase(jj, [&] {
#pragma unroll
          for (int ii = 0; ii < C::GCOPY; ++ii) {
            gcopy(krs, kbuf(jj & 1), tile_of(jj + 2), ii);
            gcopy(vrs, vbuf(jj & 1), tile_of(jj + 2), ii);
          }
        });
        lds_barrier();
      }
    }
  }
  // Copies issued during the last steps land in LDS that the next workgroup may own.
  wait_vmcnt<0>();
}

template <class T, int NDB>
static hipError_t launch_pds(AttnParams p, hipStream_t st) {
  using C = PdsCfg<NDB>;
  p.ntiles = (p.nq + C::BQ - 1) / C::BQ;
  // Fewer than two workgroups per compute unit (of 256): split the key tiles of each query tile
  // into up to 8 interleaved sets of at least 4 tiles, which also spreads the heavy tiles of a causal grid.
  const long long base = (long long)p.batch * p.hq * p.ntiles;
  const int ktiles = (p.nkv + 31) / 32;
  p.nsplit = (int)std::max(1LL, std::min({8LL, (512 + base - 1) / std::max(base, 1LL), (long long)ktiles / 4}));
  p.total = p.batch * p.hq * p.ntiles * p.nsplit;
  if (p.total == 0) return hipSuccess;
  const int grid = (p.total + 7) & ~7;
  if (p.mask_kind != 0)
    hipLaunchKernelGGL((ffpa_pds_kernel<T, NDB, true>), dim3(grid), dim3(64 * C::NW), 0, st, p);
  else
    hipLaunchKernelGGL((ffpa_pds_kernel<T, NDB, false>), dim3(grid), dim3(64 * C::NW), 0, st, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// P and dS for D > 512 (the stored-P/dS backward's P/dS stage at large head dims).
//
// The forward's D > 512 layout: a workgroup owns 64 queries of one head as 2 row groups x 4
// head-dim quarters (8 waves, two per SIMD); each wave keeps its 32 queries' Q and dO columns of
// its quarter in registers (B operands, 2 x 64 registers at D = 1024) and forms partial
// S^T = K Q^T and dP^T = V dO^T from K and V tiles (32 keys x 2 KB, single-buffered: 64 KB each)
// streamed through LDS. The four quarters are combined by a reduce-scatter: register group
// r4 = c of a C block (4 registers: keys 16 (c / 2) + 8 h + 4 (c % 2) + 0..3 of lane half h)
// belongs to the wave with quarter c, which receives the three partners' partial sums of it
// through its LDS inbox, forms P = exp(scale S - LSE) and dS = P (dP - Delta) for those 8 keys x 32
// queries, and stores them transposed (one row per key, 8 queries per 16-byte piece) after a
// transposition through its own inbox slot. Per step (32 keys):
//   wait K_j | S products (V_j copies spread over them) | S partials out | wait V_j, barrier |
//   S partials in | dP products (K_{j+1} copies spread over them) | P | barrier | dP partials out |
//   barrier | dP partials in, dS, transposition, stores
// so each tile copy overlaps the other tile's products, and the exchange moves 3 register groups
// per wave instead of the forward's all-reduce of 4 x 3.
// ------------------------------------------------------------------------------------------------
template <int NDB>
struct PdsWideCfg {
  static constexpr int NW = 8;
  static constexpr int NC = 4;                      // head-dim quarters
  static constexpr int DW = NDB * 32;               // head-dim columns per wave
  static constexpr int KSTEPS = 2 * NDB;            // 16-wide k-steps over them
  static constexpr int RS = 2048;                   // LDS row stride (bytes)
  static constexpr int BQ = 2 * 32;                 // queries per workgroup
  static constexpr int TILE = 32 * RS;              // one 32-key K or V tile
  static constexpr int WCH = NDB * 4;               // 16-byte chunks of one wave's columns
  static constexpr int SLOT = RS / 16 / NC;         // chunks per wave slot of an LDS row
  static constexpr int XSLOT = 64 * 16;             // one register group of one wave
  static constexpr int XBYTES = NW * NC * XSLOT;    // inbox[wave][source quarter]
  static constexpr int LDS = 2 * TILE + XBYTES;
  static constexpr int NINSTR = TILE / 1024 / NW;   // 1 KB copies per wave per tile
  static_assert(NC * DW <= 1024 && WCH <= SLOT && SLOT % 16 == 0 && LDS <= 160 * 1024, "LDS budget");
};

// MASK adds the attn_mask term of each owned (query, key) pair to its score before P, as in the
// forward (the tile's mask bits are requested when its score products start).
template <class T, int NDB, bool MASK>
__global__ void __launch_bounds__(512, 2) ffpa_pds_wide_kernel(AttnParams p) {
  using C = PdsWideCfg<NDB>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  lds_t* const kbuf = (lds_t*)smem_raw;
  lds_t* const vbuf = kbuf + C::TILE;
  lds_t* const xbuf = kbuf + 2 * C::TILE;

  const int L = blockIdx.x;
  const int item = xcd_item(L, gridDim.x, p.cu_q != nullptr, p.hq, p.ntiles * p.nsplit);
  if (item >= p.total) return;
  const int split = item % p.nsplit;
  const HeadTile ht = head_tile(item / p.nsplit, p.ntiles, p.hq, p.group, p.cu_q == nullptr);
  int t = ht.t;
  const int h = ht.h;
  const int s = ht.s;
  if (p.causal) t = p.ntiles - 1 - t;  // heaviest causal tiles first

  const SeqView sv = seq_view(p, s);
  const int qt0 = t * C::BQ;
  if (qt0 >= sv.lq) return;
  const DsView dsv = ds_view(p, s, sv);
  const int kvh = h / p.group;

  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int rg = w / C::NC;
  const int cg = w % C::NC;
  const int qw0 = qt0 + rg * 32;
  const int off = sv.lk - sv.lq;

  const int row_bytes = p.k_row * 2;
  const long long kv_off = sv.k_off + (long long)kvh * p.k_head;
  const uint32_t span = (uint32_t)min((long long)max(sv.lk, 1) * row_bytes, (long long)0xFFFFFFF0);
  const i32x4_t krs = make_rsrc((const uint16_t*)p.k + kv_off, span);
  const i32x4_t vrs = make_rsrc((const uint16_t*)p.v + kv_off, span);
  int kend = sv.lk;
  if (p.causal) kend = min(kend, qt0 + C::BQ + off);
  const int ntk = kend > 0 ? (kend + 31) >> 5 : 0;
  // This item's key tiles [jb, je): an equal share of the query tile's own range.
  const int per = (ntk + p.nsplit - 1) / p.nsplit;
  const int jb = min(split * per, ntk), je = min(jb + per, ntk);
  if (jb >= je && split > 0) return;

  // The query's LSE in log2 units (+inf for a row without a legal key makes P = 0) and Delta.
  const int qi = qw0 + l32;
  const long long li = sv.lse_off + (long long)h * p.lse_head + min(qi, sv.lq - 1);
  const float lse_raw = p.lse_in[li];
  const float lse2 = lse_raw == -INFINITY ? INFINITY : lse_raw * kLog2e;
  const float dlt = p.delta[li];
  // Q and dO columns of this wave's quarter as B operands: lane (h, n) holds query n, dims
  // 16 kb + 8 h + 0..7 of the quarter, staged through the K and V tiles (16 KB per wave) before
  // the first tile is copied.
  u32x4_t qreg[C::KSTEPS], oreg[C::KSTEPS];
  {
    const long long hq0 = sv.q_off + (long long)h * p.q_head;
    lds_t* const stage = kbuf + w * 16384;
    stage_b_operand<C::KSTEPS>((const uint16_t*)p.q + hq0, p.q_row, qw0, sv.lq, cg * C::DW, p.d, stage, qreg);
    stage_b_operand<C::KSTEPS>((const uint16_t*)p.dout + hq0, p.q_row, qw0, sv.lq, cg * C::DW, p.d, stage, oreg);
  }
  lds_barrier();  // every wave has read its staged operands: the tile buffers are free

  // The head's P and dS blocks (Lk rows of round_up(Lq, 8) queries).
  const long long hoff = dsv.base + (long long)h * dsv.head;
  const int nrec = (int)((long long)sv.lk * dsv.row * 2);
  const __amdgpu_buffer_rsrc_t ds_rs = __builtin_amdgcn_make_buffer_rsrc((uint16_t*)p.ds + hoff, 0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t p_rs = __builtin_amdgcn_make_buffer_rsrc((uint16_t*)p.pst + hoff, 0, nrec, 0x00020000);

  // Copies: instruction ii of wave w fills LDS bytes [1024 i, 1024 i + 1024) of a tile,
  // i = w + 8 ii, i.e. tile row R = i / 2; lane l writes physical chunk pc = (i % 2) 64 + l, whose
  // un-swizzled index u = pc ^ swz(R) is chunk u % SLOT of quarter u / SLOT (padding and chunks
  // past the head dim hold clamped, finite duplicates). Offsets and LDS addresses are rebuilt at
  // each copy (no registers held across the loop for them).
  const int dch = p.d >> 3;
  auto src_chunk = [&](int u) { return min((u / C::SLOT) * C::WCH + min(u % C::SLOT, C::WCH - 1), dch - 1); };
  auto copy1 = [&](const i32x4_t& rs, lds_t* tile, int j, int ii) {
    const int i = w + C::NW * ii;
    const int row = min(j * 32 + (i >> 1), sv.lk - 1);
    const int vo = src_chunk((((i & 1) << 6) + fresh_lane_id()) ^ swz(i >> 1)) << 4;
    lds_t* d = (lds_t*)(uintptr_t)opaque_s((uint32_t)(uintptr_t)(tile + i * 1024));
    dma16_buf(rs, vo, row * row_bytes, d);
  };
  auto spread_at = [](int n, int ii) { return (ii * n) / C::NINSTR; };

  // K and V rows (A operands): MFMA row m reads tile row row_perm(m), chunk cbase + 2 kb + h.
  const int krow = row_perm(l32);
  const int kswz = swz(krow);
  const uint32_t klane = krow * C::RS + ((cg * C::SLOT) << 4) + ((hh ^ kswz) << 4);
  auto a_addr = [&](uint32_t tile, int kb) -> uint32_t {
    return ((tile + klane) ^ ((kb & 7) << 5)) + ((kb >> 3) << 8);
  };
  // Inbox slot of wave `dst` for partial sums from quarter `src`; a wave's own slot (src = its
  // quarter) holds its P and dS transposition.
  auto inbox = [&](int dst, int src) { return xbuf + (dst * C::NC + src) * C::XSLOT; };
  const int w0 = rg * C::NC;
  // Owned keys: register group cg, keys 16 (cg / 2) + 4 (cg % 2) + 8 h + 0..3 of the tile.
  const int kown = 16 * (cg >> 1) + 4 * (cg & 1);

  auto send = [&](const f32x16_t& acc) {
#pragma unroll
    for (int c = 0; c < C::NC; ++c)
      if (c != cg)
        lds_write_f4(inbox(w0 + c, cg), lane * 16, (f32x4_t){acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]});
  };
  // Own register group plus the three partners' partial sums, in quarter order (deterministic).
  auto receive = [&](const f32x16_t& acc) {
    f32x4_t r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      const f32x4_t x = c == cg ? (f32x4_t){acc[4 * cg], acc[4 * cg + 1], acc[4 * cg + 2], acc[4 * cg + 3]}
                                : lds_read_f4(inbox(w, c), lane * 16);
      r = c == 0 ? x : r + x;
    }
    return r;
  };

  if (je > jb) {
#pragma unroll
    for (int ii = 0; ii < C::NINSTR; ++ii) copy1(krs, kbuf, jb, ii);
  }
  wait_all();  // the stationary operands, LSE, Delta and K_jb
  lds_barrier();

  f32x16_t sacc, pacc;
  // attn_mask: the aligned 8-key block that holds this lane's 4 owned keys of the tile.
  const long long mrow = MASK ? mask_row(p, s, h, min(qi, sv.lq - 1)) : 0;
  u32x4_t mraw;
  for (int j = jb; j < je; ++j) {
    // K_j landed (copied during the dP products of step j - 1; the two stores of that step may
    // still be in flight).
    if (j > jb) {
      wait_vmcnt<2>();
      lds_barrier();
    }
    if constexpr (MASK) {
      mraw = mask_block(p, mrow, j * 32 + 16 * (cg >> 1) + 8 * hh, sv.lk);
      __builtin_amdgcn_sched_barrier(0);  // issued here, not sunk behind the products
    }
    const uint32_t kt = (uint32_t)opaque_v((int)lds_addr(kbuf)), vt = (uint32_t)opaque_v((int)lds_addr(vbuf));
    sacc = (f32x16_t){};
#pragma unroll
    for (int kb = 0; kb < C::KSTEPS; ++kb) {
      sacc = Elt<T>::mma(lds_read_b128_at(a_addr(kt, kb)), qreg[kb], sacc);
#pragma unroll
      for (int ii = 0; ii < C::NINSTR; ++ii)
        if (kb == spread_at(C::KSTEPS, ii)) copy1(vrs, vbuf, j, ii);
    }
    pin_lds_mfma_pipeline<C::KSTEPS, kPdsAhead, 1>();
    send(sacc);
    wait_vmcnt<0>();  // V_j (and the stores of step j - 1)
    lds_barrier();    // S partials visible; K_j released
    const f32x4_t s4 = receive(sacc);
    pacc = (f32x16_t){};
#pragma unroll
    for (int kb = 0; kb < C::KSTEPS; ++kb) {
      pacc = Elt<T>::mma(lds_read_b128_at(a_addr(vt, kb)), oreg[kb], pacc);
#pragma unroll
      for (int ii = 0; ii < C::NINSTR; ++ii)
        if (kb == spread_at(C::KSTEPS, ii)) copy1(krs, kbuf, j + 1, ii);  // past the last tile: clamped, unused
    }
    pin_lds_mfma_pipeline<C::KSTEPS, kPdsAhead, 1>();
    // P of the owned keys (0 past the key bound and, on diagonal tiles, above the causal limit).
    const int key0 = j * 32 + kown + 8 * hh;
    const bool need_mask = (j * 32 + 32 > sv.lk) || (p.causal && j * 32 + 31 > qw0 + off);
    const int lim = p.causal ? min(qi + off, sv.lk - 1) : sv.lk - 1;
    float sown[4] = {s4[0], s4[1], s4[2], s4[3]};
    if constexpr (MASK) {
      float mb[8];
      mask_apply8_block<T>(p, mraw, mrow, j * 32 + 16 * (cg >> 1) + 8 * hh, sv.lk, mb);
#pragma unroll
      for (int e = 0; e < 4; ++e) sown[e] += mb[4 * (cg & 1) + e];
    }
    float pe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = fast_exp2(sown[e] * p.scale_log2 - lse2);
      pe[e] = need_mask && key0 + e > lim ? 0.f : x;
    }
    lds_barrier();  // every wave has read its S partials: the inboxes take the dP partials
    send(pacc);
    lds_barrier();
    const f32x4_t d4 = receive(pacc);
    // Transposition through the own slot: P at [key kk][query n] (8 rows of 64 bytes), dS 512
    // bytes further; lane (h, n) owns keys kk = 4 h + e.
    lds_t* const tb = inbox(w, cg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t pk = Elt<T>::pack2(pe[e], pe[e] * (d4[e] - dlt));
      const int o = (4 * hh + e) * 64 + 2 * l32;
      *(__attribute__((address_space(3))) uint16_t*)(tb + o) = (uint16_t)(pk & 0xffffu);
      *(__attribute__((address_space(3))) uint16_t*)(tb + 512 + o) = (uint16_t)(pk >> 16);
    }
    // Lane l stores one 16-byte piece: P for l < 32, dS for l >= 32; key kk = (l % 32) / 4,
    // queries qw0 + 8 ((l % 4)) + 0..7. Pieces of keys at or past Lk, or starting at or past the
    // padded row end, get an offset past the block, which the buffer range check discards.
    const int kk = l32 >> 2, g = l32 & 3;
    const u32x4_t piece = lds_read_b128(tb, hh * 512 + kk * 64 + g * 16);
    const int key = j * 32 + 16 * (cg >> 1) + 4 * (cg & 1) + 8 * (kk >> 2) + (kk & 3);
    const int q8 = qw0 + 8 * g;
    const bool ok = key < sv.lk && q8 < dsv.row;
    const uint32_t boff = ok ? (uint32_t)(((long long)key * dsv.row + q8) * 2) : 0xFFFFFFF0u;
    if (hh == 0)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, piece), p_rs, (int)boff, 0, kDsStoreCpol);
    else
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, piece), ds_rs, (int)boff, 0, kDsStoreCpol);
  }
  // Copies issued during the last step land in LDS that the next workgroup may own.
  wait_vmcnt<0>();
}

template <class T, int NDB>
static hipError_t launch_pds_wide(AttnParams p, hipStream_t st) {
  using C = PdsWideCfg<NDB>;
  p.ntiles = (p.nq + C::BQ - 1) / C::BQ;
  const long long base = (long long)p.batch * p.hq * p.ntiles;
  const int ktiles = (p.nkv + 31) / 32;
  p.nsplit = (int)std::max(1LL, std::min({8LL, (512 + base - 1) / std::max(base, 1LL), (long long)ktiles / 4}));
  p.total = p.batch * p.hq * p.ntiles * p.nsplit;
  if (p.total == 0) return hipSuccess;
  const int grid = (p.total + 7) & ~7;
  if (p.mask_kind != 0)
    hipLaunchKernelGGL((ffpa_pds_wide_kernel<T, NDB, true>), dim3(grid), dim3(64 * C::NW), 0, st, p);
  else
    hipLaunchKernelGGL((ffpa_pds_wide_kernel<T, NDB, false>), dim3(grid), dim3(64 * C::NW), 0, st, p);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_pds_t(const AttnParams& p, hipStream_t st) {
  if (p.d > 512) {
    switch ((p.d + 127) / 128) {
      case 5: return launch_pds_wide<T, 5>(p, st);
      case 6: return launch_pds_wide<T, 6>(p, st);
      case 7: return launch_pds_wide<T, 7>(p, st);
      default: return launch_pds_wide<T, 8>(p, st);
    }
  }
  switch ((p.d + 63) / 64) {
    case 5: return launch_pds<T, 5>(p, st);
    case 6: return launch_pds<T, 6>(p, st);
    case 7: return launch_pds<T, 7>(p, st);
    default: return launch_pds<T, 8>(p, st);
  }
}

// ------------------------------------------------------------------------------------------------
// dQ from a stored dS: dQ_i = scale * sum_j dS_ij K_j (fp32 accumulation, one rounding).
//
// With dS written by the P/dS kernel (the rounded value the dK product uses too), the dQ stage is
// a plain product instead of a recomputation of S, P, dP and dS: 2 D flops per legal pair instead
// of 6 D, for dense B * Hq * Nq * Nkv dS elements of HBM workspace. A workgroup owns 128 queries of
// one head and one chunk of up to 512 head-dim columns; its 8 waves are 2 query groups x 4 column
// groups, each wave 64 queries (two 32-row MFMA blocks) x DW columns of fp32 accumulators. Per
// step of 32 keys the K rows of the chunk (32 x 1 KB, swizzled as elsewhere) and the dS block
// (stored transposed: 32 keys x 128 queries, 256-byte rows whose 64-byte blocks are XOR-swizzled
// by the row index mod 4) are copied into LDS, triple-buffered: the copies of step j + 2 are
// spread over the MFMAs of step j, so each has a whole step to land. acc^T[d][q] += K^T[d][k]
// dS^T[k][q]: K^T is read transposed (ds_read_b64_tr_b16) and used for both query blocks; dS^T,
// 8 consecutive keys of one query, is read transposed from the key rows (the swizzle keeps a
// half-wave's transposed reads on distinct banks). Causal and ragged tiles mask dS to 0 where the
// key is not legal (those entries were not written by the P/dS kernel).
// ------------------------------------------------------------------------------------------------
template <int NDB>
struct DqCfg {
  static constexpr int NW = 8;
  static constexpr int QB = 2;                 // 32-query MFMA blocks per wave
  static constexpr int DW = NDB * 32;          // head-dim columns per wave
  static constexpr int DWG = 4 * DW;           // head-dim columns per workgroup (one chunk)
  static constexpr int BQ = 2 * QB * 32;       // queries per workgroup
  static constexpr int RS = 1024;              // K tile row stride (bytes)
  static constexpr int KTILE = 32 * RS;
  static constexpr int STILE = 32 * BQ * 2;    // dS block: 32 key rows x BQ queries x 2 bytes
  static constexpr int SROW = BQ * 2;
  static constexpr int STAGE = KTILE + STILE;
  static constexpr int NBUF = kProdNbuf;
  static constexpr int LDS = NBUF * STAGE;
  static constexpr int KCOPY = KTILE / 1024 / NW;  // K copies per wave per step
  static constexpr int SCOPY = STILE / 1024 / NW;  // dS copies per wave per step
  static_assert(DWG <= 512 && SCOPY == 1 && SROW == 256 && LDS <= 160 * 1024, "tile budget");
};

// Work item `item` of the dQ pass: ((sequence, query head), chunk, query tile), `ntiles` query
// tiles per head; a causal grid takes its heaviest tiles (the last queries) first.
template <class T, int NDB>
__device__ __forceinline__ void dq_from_ds_body(const AttnParams& p, int nchunk, int ntiles, int item, lds_t* smem) {
  using C = DqCfg<NDB>;
  // item = (head-tile slice * nchunk + chunk) * (ntiles G) + head_tile's index within the slice:
  // dense, the G query heads of a KV head side by side (head_tile); varlen, item = ((s Hq + h)
  // nchunk + chunk) ntiles + t.
  const bool dense = p.cu_q == nullptr;
  const int per_chunk = dense ? ntiles * p.group : ntiles;
  const int chunk = (item / per_chunk) % nchunk;
  const HeadTile ht = head_tile((item / (per_chunk * nchunk)) * per_chunk + item % per_chunk, ntiles, p.hq,
                                p.group, dense);
  int qt = ht.t;
  const int h = ht.h;
  const int s = ht.s;
  if (p.causal) qt = ntiles - 1 - qt;

  const SeqView sv = seq_view(p, s);
  const int q0 = qt * C::BQ;
  if (q0 >= sv.lq) return;
  const DsView dsv = ds_view(p, s, sv);
  const int kvh = h / p.group;
  const int d0 = chunk * C::DWG;

  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int qg = w >> 2;
  const int dg = w & 3;
  const int off = sv.lk - sv.lq;

  int kend = sv.lk;
  if (p.causal) kend = min(kend, q0 + C::BQ + off);
  const int nsteps = kend > 0 ? (kend + 31) >> 5 : 0;

  f32x16_t acc[C::QB][NDB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = (f32x16_t){};

  // ---- copies. K rows of this chunk: copy ii of wave w fills tile row i = w + 8 ii; lane l writes
  // physical chunk l, holding logical chunk l ^ swz(i) of the chunk (clamped into the head dim).
  const char* kbase = (const char*)p.k + 2 * (sv.k_off + (long long)kvh * p.k_head);
  const int krow_bytes = p.k_row * 2;
  const i32x4_t krs = make_rsrc(kbase, (uint32_t)min((long long)max(sv.lk, 1) * krow_bytes, (long long)0xFFFFFFF0));
  const int dch = p.d >> 3;
  int kvoff[C::KCOPY];
#pragma unroll
  for (int ii = 0; ii < C::KCOPY; ++ii) kvoff[ii] = min((d0 >> 3) + (lane ^ swz(w + 8 * ii)), dch - 1) << 4;
  // dS rows (one per key): the copy of wave w fills block rows 4 w .. 4 w + 3; lane l writes row
  // 4 w + l / 16 (key 32 j + row, clamped to the last key), physical chunk l % 16, holding logical
  // chunk (l % 16) ^ (4 (row % 4)) (queries q0 + 8 * logical chunk). The whole byte offset goes in
  // the per-lane operand, which the buffer range check covers: pieces past the head's block read
  // as 0. The block size is a multiple of 16 bytes, so no piece straddles its end.
  const uint16_t* dsh = (const uint16_t*)p.ds + dsv.base + (long long)h * dsv.head;
  const i32x4_t srs = make_rsrc(dsh, (uint32_t)((long long)sv.lk * dsv.row * 2));
  const int srow_l = 4 * w + (lane >> 4);
  const int sqoff = q0 + 8 * ((lane & 15) ^ (4 * (srow_l & 3)));
  auto copy = [&](int j, int buf, int c) {
    lds_t* stage = smem + buf * C::STAGE;
    if (c < C::KCOPY) {
      const int i = w + 8 * c;
      dma16_buf(krs, kvoff[c], min(j * 32 + i, sv.lk - 1) * krow_bytes, stage + i * 1024);
    } else {
      const int key = min(j * 32 + srow_l, sv.lk - 1);
      dma16_buf_nt(srs, (key * dsv.row + sqoff) * 2, 0, stage + C::KTILE + w * 1024);
    }
  };
  constexpr int NCOPY = C::KCOPY + C::SCOPY;
  constexpr int NMMA = 2 * NDB * C::QB;
  auto spread_at = [](int c) { return (c * NMMA) / NCOPY; };

  // ---- operand addresses. K^T (A operand) by transposed reads as in the other kernels; the
  // chunk's column base inside the tile is dg * DW (tile columns are chunk-relative).
  const int g16 = lane >> 4;
  const int r16 = lane & 15;
  const int cbase = dg * C::DW >> 3;
  const int tclo = 2 * (g16 & 1) + ((r16 & 3) >> 1);
  const int twithin = ((4 * (r16 & 3)) & 7) << 1;
  constexpr bool kAligned = (C::DW % 128) == 0;
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
  // dS^T (B operand): lane (h, query n) needs keys 16 kb2 + 8 h + 0..7 of query 64 qg + 32 qb + n.
  // In 16-lane group g16 source lane s = t + 4 m points at key row 16 kb2 + 8 h + 4 half + m,
  // queries 64 qg + 32 qb + 16 (g16 % 2) + 4 t + 0..3, so lane i receives query 16 (g16 % 2) + i
  // of the 32-query block and keys + 0..3 (half 0) or + 4..7 (half 1).
  auto s_addr = [&](uint32_t tile, int qb, int kb2, int half) -> uint32_t {
    const int m = r16 >> 2, t = r16 & 3;
    const int row = 16 * kb2 + 8 * hh + 4 * half + m;
    const int byte = (64 * qg + 32 * qb + 16 * (g16 & 1) + 4 * t) * 2;
    return tile + C::KTILE + row * C::SROW + ((((byte >> 4) ^ (4 * (row & 3))) << 4) | (byte & 15));
  };

  constexpr int NB = C::NBUF;
  if (nsteps > 0) {
#pragma unroll
    for (int b = 0; b < NB - 1; ++b)
#pragma unroll
      for (int c = 0; c < NCOPY; ++c) copy(min(b, nsteps - 1), b, c);
  }
  wait_all();

  int buf = 0;  // j % NB
  for (int j = 0; j < nsteps; ++j) {
    // In flight: the copies of step j (issued during step j - NB + 1) and then those of the NB - 2
    // steps after it.
    wait_vmcnt<(NB - 2) * NCOPY>();
    lds_barrier();  // step j's tiles are visible; every wave has finished step j - 1
    const uint32_t tile = lds_addr(smem + buf * C::STAGE);
    // Step j + NB - 1 goes into the buffer of step j - 1 (released by the barrier above); past the
    // end the last step is copied again into a buffer that is not read any more.
    const int jn = min(j + NB - 1, nsteps - 1);
    const int bn = buf == 0 ? NB - 1 : buf - 1;

    // dS^T operands of both query blocks; masked where the key is not legal.
    u32x4_t bs[C::QB][2];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
        bs[qb][kb2] = join_tr(lds_read_tr16_at(s_addr(tile, qb, kb2, 0)), lds_read_tr16_at(s_addr(tile, qb, kb2, 1)));
    const bool need_mask = (j * 32 + 32 > sv.lk) || (p.causal && j * 32 + 31 > q0 + 64 * qg + off);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        const int qi = q0 + 64 * qg + 32 * qb + l32;
        const int lim = p.causal ? min(qi + off, sv.lk - 1) : sv.lk - 1;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k0 = j * 32 + 16 * kb2 + 8 * hh + 2 * e;
            uint32_t x = bs[qb][kb2][e];
            if (k0 > lim) x &= 0xffff0000u;
            if (k0 + 1 > lim) x &= 0x0000ffffu;
            bs[qb][kb2][e] = x;
          }
      }
    }
    int mi = 0;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const s16x4_t lo = lds_read_tr16_at(t_addr(tile, db, kb2, 0));
        const s16x4_t hi = lds_read_tr16_at(t_addr(tile, db, kb2, 1));
        const u32x4_t a = join_tr(lo, hi);
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) {
          acc[qb][db] = Elt<T>::mma(a, bs[qb][kb2], acc[qb][db]);
#pragma unroll
          for (int c = 0; c < NCOPY; ++c)
            if (mi == spread_at(c)) copy(jn, bn, c);
          ++mi;
        }
      }
    }
    pin_lds_mfma_pipeline<NMMA, kProdAhead, 1>();
    buf = buf == NB - 1 ? 0 : buf + 1;
  }
  // Copies issued during the last step land in LDS that the next workgroup may own.
  wait_vmcnt<0>();

  // ---- epilogue: scale, round once, store rows < lq and columns < D (whole rows, through LDS)
  uint16_t* dqh = (uint16_t*)p.dq + sv.q_off + (long long)h * p.q_head;
  store_block_rows<T, false, 2, 4, C::QB, NDB, C::LDS>(smem, acc, p.scale, dqh + (long long)q0 * p.q_row + d0, p.q_row,
                                               sv.lq - q0, min(C::DWG, p.d - d0));
}

template <class T, int NDB>
__global__ void __launch_bounds__(512, 2) ffpa_dq_from_ds_kernel(AttnParams p, int nchunk) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[DqCfg<NDB>::LDS];
  const int item = xcd_item(blockIdx.x, gridDim.x, p.cu_q != nullptr, p.hq, nchunk * p.ntiles);
  if (item >= p.total) return;
  dq_from_ds_body<T, NDB>(p, nchunk, p.ntiles, item, (lds_t*)smem_raw);
}

template <class T, int NDB>
static hipError_t launch_dq_from_ds(AttnParams p, int nchunk, hipStream_t st) {
  using C = DqCfg<NDB>;
  p.ntiles = (p.nq + C::BQ - 1) / C::BQ;
  p.total = p.batch * p.hq * nchunk * p.ntiles;
  if (p.total == 0) return hipSuccess;
  const int grid = (p.total + 7) & ~7;
  hipLaunchKernelGGL((ffpa_dq_from_ds_kernel<T, NDB>), dim3(grid), dim3(64 * C::NW), 0, st, p, nchunk);
  return hipGetLastError();
}

// Head-dim chunking of the dQ-from-dS pass: chunks of at most 512 columns, each covered by four
// waves of 96 or 128 columns.
template <class T>
static hipError_t launch_dq_ds_t(const AttnParams& p, hipStream_t st) {
  const int nchunk = (p.d + 511) / 512;
  const int per = (p.d + nchunk - 1) / nchunk;
  if (per <= 384) return launch_dq_from_ds<T, 3>(p, nchunk, st);
  return launch_dq_from_ds<T, 4>(p, nchunk, st);
}

// ------------------------------------------------------------------------------------------------
// dV from a stored P: dV_j = sum over the query heads h of the group and queries i of P_hij dO_hi,
// and with DK the same product dK_j = scale sum dS_hij Q_hi (fp32 accumulation, one rounding).
//
// Same tiling as the dQ pass with keys as the output rows: a workgroup owns 128 keys of one KV head
// and one chunk of up to 512 head-dim columns; its 8 waves are 2 key groups x 4 column groups, each
// wave 64 keys (two 32-row MFMA blocks) x DW columns. The streamed side is 32 queries of one query
// head of the group per step (all the group's heads in turn; causal steps start at the first
// query that sees a key of the block). acc^T[d][j] += dO^T[d][i] P[i][j]: dO^T is read transposed
// from the dO rows (as K^T in the dQ pass); P is stored transposed (one row per key), so P[i][j]
// for 8 consecutive queries i of key j is one 16-byte read from the block in LDS (128 keys x 32
// queries, 64-byte rows whose 16-byte chunks are XOR-swizzled by bits 2-3 of the row).
// Triple-buffered copies as in the dQ pass. P is masked to 0 for queries at or past Lq (padding or
// the next row's values) and for pairs that are not legal (not written by the P/dS kernel).
// ------------------------------------------------------------------------------------------------
// SQ = queries per step: 32 (triple-buffered) or 64 (double-buffered), i.e. block rows of 64 or
// 128 bytes per key; whole 128-byte rows keep the stored blocks' HBM reads at full lines.
constexpr int kDvSq = 64;
template <int NDB, int SQ = kDvSq>
struct DvCfg {
  static constexpr int NW = 8;
  static constexpr int KB = 2;                 // 32-key MFMA blocks per wave
  static constexpr int KB2 = SQ / 16;          // 16-query k-steps per step
  static constexpr int DW = NDB * 32;
  static constexpr int DWG = 4 * DW;
  static constexpr int BK = 2 * KB * 32;       // keys per workgroup
  static constexpr int RS = 1024;              // dO tile row stride (bytes)
  static constexpr int OTILE = SQ * RS;
  static constexpr int PROW = SQ * 2;          // P block row: one key, SQ queries x 2 bytes
  static constexpr int PCH = PROW / 16;        // 16-byte chunks per P row
  static constexpr int PTILE = BK * PROW;
  static constexpr int STAGE = OTILE + PTILE;
  static constexpr int NBUF = SQ == 32 ? kProdNbuf : 2;
  static constexpr int LDS = NBUF * STAGE;
  static constexpr int OCOPY = OTILE / 1024 / NW;
  static constexpr int PCOPY = PTILE / 1024 / NW;
  static_assert((SQ == 32 || SQ == 64) && DWG <= 512 && PCOPY * NW * 1024 == PTILE && LDS <= 160 * 1024,
                "tile budget");
  // XOR on the chunk index of P row r: 16 consecutive rows read by a half-wave at one logical
  // chunk land on 16 distinct 16-byte bank groups.
  static __device__ __forceinline__ int pswz(int r) { return PCH == 4 ? (r >> 2) & 3 : (r >> 1) & 7; }
};

// Work item `item` of the dV (or dK) pass: ((sequence, KV head), chunk, key tile), `ntiles` key
// tiles per head (the first keys, the heaviest of a causal grid, first).
template <class T, int NDB, bool DK>
__device__ __forceinline__ void dv_from_p_body(const AttnParams& p, int nchunk, int ntiles, int item, lds_t* smem) {
  using C = DvCfg<NDB>;
  // dV = P^T dO, or (DK) dK = scale dS^T Q: the same product of a stored block and query rows.
  const void* const rows_src = DK ? p.q : p.dout;
  const void* const blk_src = DK ? p.ds : p.pst;
  const int kt = item % ntiles;
  const int rest = item / ntiles;
  const int chunk = rest % nchunk;
  const int hs = rest / nchunk;
  const int kvh = hs % p.hkv;
  const int s = hs / p.hkv;

  const SeqView sv = seq_view(p, s);
  const int k0 = kt * C::BK;
  if (k0 >= sv.lk) return;
  const DsView dsv = ds_view(p, s, sv);
  const int d0 = chunk * C::DWG;

  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int kg = w >> 2;
  const int dg = w & 3;
  const int off = sv.lk - sv.lq;

  // Streamed steps: SQ-query tiles, from the last one down to the first that sees a key of the
  // block, each for every query head of the group in turn. Every workgroup of a causal grid then
  // starts at the same (last) tile and the workgroups sweep the same query rows at the same time,
  // whatever their key block, so the rows they read are shared in L2 (in ascending order each
  // would start at its own first query and the sweeps would drift apart).
  constexpr int SQ = C::KB2 * 16;
  const int qfirst = p.causal ? max(0, k0 - off) : 0;
  const int qt_first = qfirst / SQ;
  const int nqt = sv.lq > qfirst ? (sv.lq + SQ - 1) / SQ - qt_first : 0;
  const int nsteps = p.group * nqt;
  auto step_head = [&](int st) { return kvh * p.group + st % p.group; };
  auto step_row0 = [&](int st) { return (qt_first + nqt - 1 - st / p.group) * SQ; };

  f32x16_t acc[C::KB][NDB];
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[kb][db] = (f32x16_t){};

  // ---- copies. dO rows of the chunk: copy ii of wave w fills tile row i = w + 8 ii (as in dQ).
  const int orow_bytes = p.q_row * 2;
  const uint32_t ospan = (uint32_t)min((long long)max(sv.lq, 1) * orow_bytes, (long long)0xFFFFFFF0);
  const int dch = p.d >> 3;
  int ovoff[C::OCOPY];
#pragma unroll
  for (int ii = 0; ii < C::OCOPY; ++ii) ovoff[ii] = min((d0 >> 3) + (lane ^ swz(w + 8 * ii)), dch - 1) << 4;
  // P rows (one per key): copy c of wave w fills 1 KB of the block, rows (PCOPY w + c) * 1024 /
  // PROW + l / PCH for lane l (key k0 + row, clamped to the last key), physical chunk l % PCH,
  // holding logical chunk (l % PCH) ^ pswz(row) (queries row0 + 8 * logical chunk). The whole
  // byte offset is per lane (range-checked; the block is a multiple of 16 bytes).
  int pkey[C::PCOPY], pchunk[C::PCOPY];
#pragma unroll
  for (int c = 0; c < C::PCOPY; ++c) {
    const int r = (C::PCOPY * w + c) * (1024 / C::PROW) + lane / C::PCH;
    pkey[c] = min(k0 + r, sv.lk - 1);
    pchunk[c] = (lane % C::PCH) ^ C::pswz(r);
  }
  const uint32_t pspan = (uint32_t)((long long)sv.lk * dsv.row * 2);
  struct StepSrc {
    i32x4_t ors, prs;
    int row0;
  };
  auto step_src = [&](int st) {
    st = min(st, nsteps - 1);
    StepSrc x;
    const int h = step_head(st);
    x.row0 = step_row0(st);
    x.ors = make_rsrc((const uint16_t*)rows_src + sv.q_off + (long long)h * p.q_head, ospan);
    x.prs = make_rsrc((const uint16_t*)blk_src + dsv.base + (long long)h * dsv.head, pspan);
    return x;
  };
  auto copy = [&](const StepSrc& x, int buf, int c) {
    lds_t* stage = smem + buf * C::STAGE;
    if (c < C::OCOPY) {
      const int i = w + 8 * c;
      dma16_buf(x.ors, ovoff[c], min(x.row0 + i, sv.lq - 1) * orow_bytes, stage + i * 1024);
    } else {
      const int pc = c - C::OCOPY;
      dma16_buf_nt(x.prs, (pkey[pc] * dsv.row + x.row0 + 8 * pchunk[pc]) * 2, 0,
                stage + C::OTILE + (C::PCOPY * w + pc) * 1024);
    }
  };
  constexpr int NCOPY = C::OCOPY + C::PCOPY;
  constexpr int NMMA = C::KB2 * NDB * C::KB;
  auto spread_at = [](int c) { return (c * NMMA) / NCOPY; };

  // ---- operand addresses. dO^T (A operand): transposed reads as K^T in the dQ pass.
  const int g16 = lane >> 4;
  const int r16 = lane & 15;
  const int cbase = dg * C::DW >> 3;
  const int tclo = 2 * (g16 & 1) + ((r16 & 3) >> 1);
  const int twithin = ((4 * (r16 & 3)) & 7) << 1;
  constexpr bool kAligned = (C::DW % 128) == 0;
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
  // P (B operand): lane (h, key n) reads block row r = 64 kg + 32 kb + n, queries 16 kb2 + 8 h + 0..7,
  // i.e. logical chunk 2 kb2 + h of the row.
  auto p_addr = [&](uint32_t tile, int kb, int kb2) -> uint32_t {
    const int r = 64 * kg + 32 * kb + l32;
    return tile + C::OTILE + r * C::PROW + (((2 * kb2 + hh) ^ C::pswz(r)) << 4);
  };

  constexpr int NB = C::NBUF;
  if (nsteps > 0) {
#pragma unroll
    for (int b = 0; b < NB - 1; ++b) {
      const StepSrc xb = step_src(b);
#pragma unroll
      for (int c = 0; c < NCOPY; ++c) copy(xb, b, c);
    }
  }
  wait_all();

  int buf = 0;  // st % NB
  for (int st = 0; st < nsteps; ++st) {
    // In flight: the copies of step st (issued during step st - NB + 1) and then those of the
    // NB - 2 steps after it.
    wait_vmcnt<(NB - 2) * NCOPY>();
    lds_barrier();  // step st's tiles are visible; every wave has finished step st - 1
    const uint32_t tile = lds_addr(smem + buf * C::STAGE);
    const int bn = buf == 0 ? NB - 1 : buf - 1;  // the buffer of step st - 1
    const StepSrc xn = step_src(st + NB - 1);
    const int row0 = step_row0(st);

    u32x4_t bp[C::KB][C::KB2];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int kb2 = 0; kb2 < C::KB2; ++kb2)
        bp[kb][kb2] = lds_read_b128_at(p_addr(tile, kb, kb2));
    const int kw0 = k0 + 64 * kg;
    const bool need_mask = (row0 + SQ > sv.lq) || (kw0 + 64 > sv.lk) || (p.causal && kw0 + 63 > row0 + off);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const int kj = kw0 + 32 * kb + l32;
#pragma unroll
        for (int kb2 = 0; kb2 < C::KB2; ++kb2)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int q = row0 + 16 * kb2 + 8 * hh + 2 * e;
            auto legal = [&](int qi) { return qi < sv.lq && kj < sv.lk && (!p.causal || kj <= qi + off); };
            uint32_t x = bp[kb][kb2][e];
            if (!legal(q)) x &= 0xffff0000u;
            if (!legal(q + 1)) x &= 0x0000ffffu;
            bp[kb][kb2][e] = x;
          }
      }
    }
    int mi = 0;
#pragma unroll
    for (int kb2 = 0; kb2 < C::KB2; ++kb2) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const s16x4_t lo = lds_read_tr16_at(t_addr(tile, db, kb2, 0));
        const s16x4_t hi = lds_read_tr16_at(t_addr(tile, db, kb2, 1));
        const u32x4_t a = join_tr(lo, hi);
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
          acc[kb][db] = Elt<T>::mma(a, bp[kb][kb2], acc[kb][db]);
#pragma unroll
          for (int c = 0; c < NCOPY; ++c)
            if (mi == spread_at(c)) copy(xn, bn, c);
          ++mi;
        }
      }
    }
    pin_lds_mfma_pipeline<NMMA, kProdAhead, 1>();
    buf = buf == NB - 1 ? 0 : buf + 1;
  }
  // Copies issued during the last steps land in LDS that the next workgroup may own.
  wait_vmcnt<0>();

  // ---- epilogue: round once, store keys < Lk and columns < D (whole rows, through LDS)
  uint16_t* dvh = (uint16_t*)(DK ? p.dk : p.dv) + sv.k_off + (long long)kvh * p.k_head;
  store_block_rows<T, false, 2, 4, C::KB, NDB, C::LDS>(smem, acc, DK ? p.scale : 1.0f, dvh + (long long)k0 * p.k_row + d0,
                                               p.k_row, sv.lk - k0, min(C::DWG, p.d - d0));
}

template <class T, int NDB, bool DK>
__global__ void __launch_bounds__(512, 2) ffpa_dv_from_p_kernel(AttnParams p, int nchunk) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[DvCfg<NDB>::LDS];
  const int item = xcd_item(blockIdx.x, gridDim.x, p.cu_q != nullptr, p.hkv, nchunk * p.ntiles);
  if (item >= p.total) return;
  dv_from_p_body<T, NDB, DK>(p, nchunk, p.ntiles, item, (lds_t*)smem_raw);
}

template <class T, int NDB, bool DK>
static hipError_t launch_dv_from_p(AttnParams p, int nchunk, hipStream_t st) {
  using C = DvCfg<NDB>;
  p.ntiles = (p.nkv + C::BK - 1) / C::BK;
  p.total = p.batch * p.hkv * nchunk * p.ntiles;
  if (p.total == 0) return hipSuccess;
  const int grid = (p.total + 7) & ~7;
  hipLaunchKernelGGL((ffpa_dv_from_p_kernel<T, NDB, DK>), dim3(grid), dim3(64 * C::NW), 0, st, p, nchunk);
  return hipGetLastError();
}

template <class T, bool DK>
static hipError_t launch_dv_p_t(const AttnParams& p, hipStream_t st) {
  const int nchunk = (p.d + 511) / 512;
  const int per = (p.d + nchunk - 1) / nchunk;
  if (per <= 384) return launch_dv_from_p<T, 3, DK>(p, nchunk, st);
  return launch_dv_from_p<T, 4, DK>(p, nchunk, st);
}

// ------------------------------------------------------------------------------------------------
// attn_mask gradient ("Triton Backend", "Feature support": the backward reduces the bias gradient
// back to the mask's original shape): dBias = dS summed over the dimensions the bias broadcasts,
// read from the stored (transposed) dS block. Pairs that are not legal (causal, or queries past Lq)
// are not all written there and count as 0. The output has dims DB, DH, DQ, DK (1 where the bias
// broadcasts), packed row-major in q's dtype, summed in fp32 and rounded once.
//
// Full query and key dims (the bias may broadcast over batch and heads): a workgroup owns a 64-key
// x 64-query tile of one output (b', h'), adds the stored 16-byte pieces of every (batch, head) of
// its set (4 lanes per key row, so each row's 128 bytes are one coalesced read), transposes
// through LDS and writes 64 consecutive keys per instruction. A bias broadcast over queries or
// keys uses one thread per output element looping over its whole set.
// ------------------------------------------------------------------------------------------------
struct DbiasDims {
  int db, dh, dq, dk;
};

template <class T>
__global__ void __launch_bounds__(256) ffpa_dbias_tile_kernel(AttnParams p, DbiasDims od) {
  __shared__ float tile[64][65];
  const int nit = (p.nq + 63) / 64, njt = (p.nkv + 63) / 64;
  int item = blockIdx.x;
  const int jt = item % njt;
  item /= njt;
  const int it = item % nit;
  item /= nit;
  const int ho = item % od.dh;
  const int bo = item / od.dh;
  const int i0 = it * 64, j0 = jt * 64;
  const int tid = threadIdx.x;
  const int off = p.nkv - p.nq;

  // Phase A: thread (key row jr, query chunk c) sums queries i0 + 16 c + 0..15 of key j0 + jr.
  const int jr = tid >> 2, c = tid & 3;
  const int key = j0 + jr;
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  if (key < p.nkv) {
    for (int b = od.db == 1 ? 0 : bo; b < (od.db == 1 ? p.batch : bo + 1); ++b)
      for (int h = od.dh == 1 ? 0 : ho; h < (od.dh == 1 ? p.hq : ho + 1); ++h) {
        const uint16_t* row = (const uint16_t*)p.ds + (long long)b * p.ds_batch + (long long)h * p.ds_head +
                              (long long)key * p.ds_row;
#pragma unroll
        for (int pc = 0; pc < 2; ++pc) {
          const int q8 = i0 + 16 * c + 8 * pc;
          if (q8 < p.ds_row) {
            const u32x4_t v = *(const u32x4_t*)(row + q8);
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
              float lo, hi;
              Elt<T>::unpack2(v[e2], lo, hi);
              const int qa = q8 + 2 * e2;
              const bool la = qa < p.nq && (!p.causal || key <= qa + off);
              const bool lb = qa + 1 < p.nq && (!p.causal || key <= qa + 1 + off);
              acc[8 * pc + 2 * e2] += la ? lo : 0.f;
              acc[8 * pc + 2 * e2 + 1] += lb ? hi : 0.f;
            }
          }
        }
      }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) tile[16 * c + e][jr] = acc[e];
  __syncthreads();
  // Phase B: thread (key j, row group g) writes rows 16 g + 0..15 of the tile at key j0 + j.
  const int j = tid & 63, g = tid >> 6;
  if (j0 + j < p.nkv) {
    uint16_t* out = (uint16_t*)p.dmask + ((long long)bo * od.dh + ho) * od.dq * (long long)od.dk + j0 + j;
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
      const int qi = i0 + 16 * g + r;
      if (qi < p.nq) {
        const uint32_t pk = Elt<T>::pack2(tile[16 * g + r][j], 0.f);
        out[(long long)qi * od.dk] = (uint16_t)(pk & 0xffffu);
      }
    }
  }
}

template <class T>
__global__ void __launch_bounds__(256) ffpa_dbias_any_kernel(AttnParams p, DbiasDims od, long long total) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  long long r = idx;
  const int jo = (int)(r % od.dk);
  r /= od.dk;
  const int io = (int)(r % od.dq);
  r /= od.dq;
  const int ho = (int)(r % od.dh);
  const int bo = (int)(r / od.dh);
  const int off = p.nkv - p.nq;
  float acc = 0.f;
  for (int b = od.db == 1 ? 0 : bo; b < (od.db == 1 ? p.batch : bo + 1); ++b)
    for (int h = od.dh == 1 ? 0 : ho; h < (od.dh == 1 ? p.hq : ho + 1); ++h) {
      const uint16_t* blk = (const uint16_t*)p.ds + (long long)b * p.ds_batch + (long long)h * p.ds_head;
      for (int j = od.dk == 1 ? 0 : jo; j < (od.dk == 1 ? p.nkv : jo + 1); ++j)
        for (int i = od.dq == 1 ? 0 : io; i < (od.dq == 1 ? p.nq : io + 1); ++i)
          if (!p.causal || j <= i + off) acc += Elt<T>::to_f32(blk[(long long)j * p.ds_row + i]);
    }
  ((uint16_t*)p.dmask)[idx] = (uint16_t)(Elt<T>::pack2(acc, 0.f) & 0xffffu);
}

template <class T>
static hipError_t launch_dbias_t(const AttnParams& p, hipStream_t st) {
  const DbiasDims od{p.m_batch ? p.batch : 1, p.m_head ? p.hq : 1, p.m_row ? p.nq : 1, p.m_key ? p.nkv : 1};
  if (od.dq == p.nq && od.dk == p.nkv && p.nq > 1 && p.nkv > 1) {
    const long long blocks = (long long)od.db * od.dh * ((p.nq + 63) / 64) * ((p.nkv + 63) / 64);
    hipLaunchKernelGGL(ffpa_dbias_tile_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, st, p, od);
  } else {
    const long long total = (long long)od.db * od.dh * od.dq * od.dk;
    hipLaunchKernelGGL(ffpa_dbias_any_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, p, od,
                       total);
  }
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
      if (p.d > 384) return launch_bwd_pp<T, MODE, 4>(p, st);
      return launch_bwd_pp<T, MODE, 3>(p, st);
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

// ------------------------------------------------------------------------------------------------
// dK, dV and dQ from the stored blocks in one launch, for dense grids too small to fill the GPU.
// Each product pass alone runs one workgroup per compute unit or fewer, and a causal grid's
// heaviest tile (first keys for dK/dV, last queries for dQ) takes about twice the average tile's
// time. The three passes' items share one grid, in an order that lets the dispatcher balance
// them: a slice is one (batch, KV head, head-dim chunk) with its dK and dV key tiles and its
// dQ query tiles (G heads); rank r of a slice is its r-th heaviest dK, dV and dQ tiles; the list
// runs rank by rank (r = 0 first), and within a rank slice by slice. Every compute unit that
// finishes early then takes the heaviest item left (longest-processing-time order), so the
// launch ends close to the average load instead of a heavy item started last.
// XCDs: with a multiple of 8 slices, XCD x runs the ranks of its own slices (one slice's rows in
// one L2); otherwise the whole list goes round-robin over the XCDs (L mod 8), which still hands
// each XCD a heaviest-first sequence.
// ------------------------------------------------------------------------------------------------
struct ProductsGrid {
  int nchunk, ktiles, qtiles, nk, nq;  // nk: dK (and dV) items, nq: dQ items
  int nslice;                          // (batch, KV head, chunk) slices
  int per_xcd;                         // slices per XCD (nslice % 8 == 0), else 0
};

template <int NDB>
constexpr int products_lds() { return DvCfg<NDB>::LDS > DqCfg<NDB>::LDS ? DvCfg<NDB>::LDS : DqCfg<NDB>::LDS; }

template <class T, int NDB>
__global__ void __launch_bounds__(512, 2) ffpa_products_kernel(AttnParams p, ProductsGrid g) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[products_lds<NDB>()];
  lds_t* const smem = (lds_t*)smem_raw;
  const int L = blockIdx.x;
  // i: position in the rank-ordered list of nsl slices starting at slice sl0
  int i = L, nsl = g.nslice, sl0 = 0;
  if (g.per_xcd > 0) {
    i = L >> 3;
    nsl = g.per_xcd;
    sl0 = (L & 7) * g.per_xcd;
  }
  // Ranks below min(ktiles, qtiles) hold 2 + G items per slice (dK, dV, then dQ of each query
  // head); past it only the longer side's items remain (2 or G per slice).
  const int m = min(g.ktiles, g.qtiles);
  const int gs = 2 + p.group;
  int r, sl, j;  // j = 0: dK, 1: dV, 2 + hg: dQ of query head hg of the group
  if (i < m * nsl * gs) {
    r = i / (nsl * gs);
    const int rem = i % (nsl * gs);
    sl = rem / gs;
    j = rem % gs;
  } else {
    const bool keys = g.ktiles > g.qtiles;
    const int gs2 = keys ? 2 : p.group;
    const int i2 = i - m * nsl * gs;
    r = m + i2 / (nsl * gs2);
    const int rem = i2 % (nsl * gs2);
    sl = rem / gs2;
    j = rem % gs2 + (keys ? 0 : 2);
  }
  if (r >= max(g.ktiles, g.qtiles)) return;  // padding of the grid to a multiple of 8
  sl += sl0;
  if (j == 0)
    dv_from_p_body<T, NDB, true>(p, g.nchunk, g.ktiles, sl * g.ktiles + r, smem);
  else if (j == 1)
    dv_from_p_body<T, NDB, false>(p, g.nchunk, g.ktiles, sl * g.ktiles + r, smem);
  else
    dq_from_ds_body<T, NDB>(p, g.nchunk, g.qtiles, (sl * g.qtiles + r) * p.group + (j - 2), smem);
}

static ProductsGrid products_grid(const AttnParams& p) {
  ProductsGrid g{};
  g.nchunk = (p.d + 511) / 512;
  g.ktiles = (p.nkv + DvCfg<4>::BK - 1) / DvCfg<4>::BK;
  g.qtiles = (p.nq + DqCfg<4>::BQ - 1) / DqCfg<4>::BQ;
  g.nslice = p.batch * p.hkv * g.nchunk;
  g.nk = g.nslice * g.ktiles;
  g.nq = g.nslice * p.group * g.qtiles;
  g.per_xcd = g.nslice % 8 == 0 ? g.nslice / 8 : 0;
  return g;
}

// Dense grids whose product passes would each give fewer than two workgroups per compute unit (of
// 256) take the one-launch form.
bool fused_products(const AttnParams& p) {
  if (p.cu_q != nullptr) return false;
  const ProductsGrid g = products_grid(p);
  return std::max(g.nk, g.nq) < 512;
}

template <class T>
static hipError_t launch_products_t(const AttnParams& p, hipStream_t st) {
  const ProductsGrid g = products_grid(p);
  const long long total = 2LL * g.nk + g.nq;
  if (total == 0) return hipSuccess;
  const int grid = (int)((total + 7) & ~7LL);
  const int per = (p.d + g.nchunk - 1) / g.nchunk;
  if (per <= 384)
    hipLaunchKernelGGL((ffpa_products_kernel<T, 3>), dim3(grid), dim3(512), 0, st, p, g);
  else
    hipLaunchKernelGGL((ffpa_products_kernel<T, 4>), dim3(grid), dim3(512), 0, st, p, g);
  return hipGetLastError();
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
    // With a workspace, stage 4 stores P and dS and dK, dV, dQ are products of them.
    case 4: return p.ds != nullptr ? launch_pds_t<T>(p, st) : hipSuccess;
    case 1: {
      const hipError_t e = p.ds != nullptr ? launch_dv_p_t<T, true>(p, st) : launch_bwd_mode<T, kDK>(p, st);
      // The attn_mask gradient, once dS is stored (stage 4 for D <= 512, the dK kernel above otherwise).
      if (e != hipSuccess || p.dmask == nullptr) return e;
      return launch_dbias_t<T>(p, st);
    }
    case 2: return p.pst != nullptr ? launch_dv_p_t<T, false>(p, st) : launch_bwd_mode<T, kDV>(p, st);
    case 5: {
      // dK, dV and dQ in one launch (needs the workspace), then the attn_mask gradient.
      if (p.ds == nullptr) return hipErrorInvalidValue;
      const hipError_t e = launch_products_t<T>(p, st);
      if (e != hipSuccess || p.dmask == nullptr) return e;
      return launch_dbias_t<T>(p, st);
    }
    default: return p.ds != nullptr ? launch_dq_ds_t<T>(p, st) : launch_bwd_mode<T, kDQ>(p, st);
  }
}

// Stage 0 = preprocess, 4 = P and dS, 1 = dK, 2 = dV, 3 = dQ, 5 = dK, dV and dQ in one launch
// (workspace only). -1 runs 0, 4, 1, 2, 3, or 0, 4, 5 when the workspace is there and the dense grid
// is small (fused_products).
hipError_t launch_bwd(const AttnParams& p, int fp16, int nrows, int varlen_total, hipStream_t st, int stage) {
  auto run = [&](int s) {
    return fp16 ? launch_stage_t<FP16>(s, p, nrows, varlen_total, st) : launch_stage_t<BF16>(s, p, nrows, varlen_total, st);
  };
  if (stage >= 0) return run(stage);
  static const int kOrder[5] = {0, 4, 1, 2, 3};
  static const int kFused[3] = {0, 4, 5};
  const bool fused = p.ds != nullptr && fused_products(p);
  const int* order = fused ? kFused : kOrder;
  const int n = fused ? 3 : 5;
  for (int i = 0; i < n; ++i) {
    const hipError_t e = run(order[i]);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ffpa
