// Forward kernel: split-D online-softmax attention for large head dims on gfx950.
//
// What it computes (ffpa-attn user guide): O = softmax(scale * Q K^T) V with the SDPA contract
// ("Backends Overview", "Automatic SDPA fallback"), bottom-right causal masking and GQA head
// broadcast ("Triton Backend", "Feature support"; "CuTe-DSL Backend", "Hard constraints"), rows
// without a legal key giving O = 0 and LSE = -inf, and an fp32 natural-log LSE
// ("CuTe-DSL Backend", "Varlen (packed THD) API").
//
// How it maps to gfx950:
//  * One workgroup of NW = 8 wave64s (two per SIMD) owns BQ = NR*QB*32 queries of one head: 128
//    for D <= 512 (4 row groups x 2 head-dim halves), 64 above (2 x 4 quarters; the masked form
//    above D = 896 keeps 4 waves and 32 queries), so each K/V tile copied into LDS serves that
//    many queries. Each wave keeps QB*32 queries x DW head-dim columns of Q in registers (B
//    operand of S^T = K Q^T) and the matching O^T block as fp32 MFMA accumulators ("O
//    accumulator held per D chunk").
//  * K and V stream through LDS in 32-key tiles, copied straight from global memory with 16-byte
//    global_load_lds (no VGPR staging), double-buffered when a tile pair fits twice in the 160 KB.
//  * Scores are formed transposed (keys x queries): each lane owns one query column, so the row
//    max/sum over keys is an in-lane reduction plus one exchange between the two wave halves.
//    The C block of scores is, with the key permutation described in ffpa_device.h, already the B
//    operand of O^T += V^T P^T; V^T comes from LDS with ds_read_b64_tr_b16.
//  * The NC waves sharing a query block each hold part of the head dim; their partial scores are
//    added through LDS in a fixed commutative pattern so every wave gets bit-identical S.
//  * Softmax runs in the exp2 domain with a lazily updated reference max: O and l are rescaled
//    only when a row max grows by more than 2^8, which leaves the result unchanged (the same
//    reference is used for numerator and denominator) and removes the per-tile O rescale.
#include <algorithm>

#include "ffpa_device.h"
#include "ffpa_params.h"

namespace ffpa {
// MFMAs whose LDS operands are requested ahead of the one issuing (see pin_lds_mfma_pipeline):
// three for the two-wave head-dim split at D = 384 and 448 (1-2% faster there), two otherwise
// (three is 3.5% slower at D = 512 and no faster at D = 320).
template <int NC, int NDB>
constexpr int fwd_ahead() { return NC == 2 && (NDB == 6 || NDB == 7) ? 3 : 2; }


template <int NC, int NDB, int QB, int NBUF, int NW>
struct FwdCfg {
  static constexpr int NR = NW / NC;                     // query row groups
  static constexpr int DW = NDB * 32;                    // head-dim columns per wave
  static constexpr int DPAD = NC * DW;                   // padded head dim
  static constexpr int RS = DPAD <= 512 ? 1024 : 2048;   // LDS row stride (bytes), power of two
  // An LDS row gives each wave's head-dim columns a slot of SLOT 16-byte chunks, of which the
  // first WCH hold its columns; the rest are padding. Every wave's operands then start on a
  // 16-chunk boundary, where the row swizzle (an XOR on the low 4 bits of the chunk index) makes
  // each operand address one per-lane base XOR a constant.
  static constexpr int WCH = NDB * 4;                    // 16-byte chunks of one wave's columns
  static constexpr int SLOT = RS / 16 / NC;              // chunks per wave slot
  static_assert(WCH <= SLOT && SLOT % 16 == 0, "one 16-chunk-aligned slot per wave in an LDS row");
  static constexpr int BQ = NR * QB * 32;                // queries per workgroup
  static constexpr int TILE = 32 * RS;                   // one 32-row K or V tile in LDS
  static constexpr int XBYTES = NW * QB * 16 * 64 * 4;   // partial scores of all waves
  static constexpr int LDS = NBUF * 2 * TILE + XBYTES;
  static constexpr int NINSTR = TILE / 1024 / NW;        // 1 KB DMA instructions per wave per tile
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// DEC selects the split-KV decode form (one 32-row block of (query head, query) rows of a KV
// group, one range of key tiles, partial results to a workspace); see the decode section below.
// MASK adds an attn_mask to the scores ("Triton Backend", "Feature support": boolean or additive,
// broadcast in any dimension): the combined scores of each tile get bias / scale, or -inf where a
// boolean mask drops the key, before the row max; a row that ends with no finite score is empty.
// SPL splits the key tiles of each query tile into p.nsplit ranges (work item = (sequence, head,
// query tile, range)) and writes, per row and range, the normalised fp32 O and the log2-domain
// LSE to part_o / part_lse as the decode form does; the same merge pass combines them. It serves
// grids too small to fill the GPU (a causal grid's heavy tiles are split as well).
template <class T, int NC, int NDB, int QB, int NBUF, int NW, bool DEC = false, bool MASK = false, bool SPL = false>
__global__ void __launch_bounds__(64 * NW, NW / 4) ffpa_fwd_kernel(AttnParams p) {
  using C = FwdCfg<NC, NDB, QB, NBUF, NW>;
  static_assert(!DEC || (QB == 1 && NW == NC), "decode: one 32-row block per workgroup");
  static_assert(!SPL || (QB == 1 && !DEC), "key-range split: one query block per wave, prefill form");
  // LDS: K and V tiles of buffer 0, those of buffer 1 (double-buffered forms), the exchange of
  // partial scores; the epilogue reuses the tile space to write whole rows of O.
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  lds_t* const smem = (lds_t*)smem_raw;
  auto kbuf = [&](int b) { return smem + (b ? 2 * C::TILE : 0); };
  auto vbuf = [&](int b) { return smem + (b ? 3 * C::TILE : C::TILE); };

  // Work item: XCD-aware decode (xcd_item): each XCD runs whole heads, so the tiles of one KV head
  // share that XCD's L2.
  const int L = blockIdx.x;
  const int item = DEC ? xcd_item(L, gridDim.x, false, p.hkv, p.nsplit * p.nrb)
                       : xcd_item(L, gridDim.x, p.cu_q != nullptr, p.hq, SPL ? p.ntiles * p.nsplit : p.ntiles);
  if (item >= p.total) return;
  int t, h, s, kvh, split = 0;
  if constexpr (DEC) {
    // item = ((s * Hkv + kvh) * nsplit + split) * nrb + row block: the row blocks of one key range
    // are neighbours (same XCD, shared K/V lines in its L2).
    t = item % p.nrb;
    int rest = item / p.nrb;
    split = rest % p.nsplit;
    rest /= p.nsplit;
    kvh = rest % p.hkv;
    s = rest / p.hkv;
    h = kvh * p.group;
  } else {
    const int tile_item = SPL ? item / p.nsplit : item;
    if constexpr (SPL) split = item % p.nsplit;
    const HeadTile ht = head_tile(tile_item, p.ntiles, p.hq, p.group, p.cu_q == nullptr);
    t = ht.t;
    h = ht.h;
    s = ht.s;
    kvh = h / p.group;
    if (p.causal) t = p.ntiles - 1 - t;  // heaviest causal tiles first
  }

  const SeqView sv = seq_view(p, s);
  const int qt0 = DEC ? 0 : t * C::BQ;
  if (qt0 >= sv.lq) return;

  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int rg = w / NC;
  const int cg = w % NC;
  const int qw0 = qt0 + rg * QB * 32;
  // Head and query of this lane's row (query column n of the MFMA blocks). Decode: row
  // R = 32 t + n of the block is query R % Nq of query head kvh * G + R / Nq (rows at or past
  // G * Nq repeat the last row and are not stored).
  int hl = h, qi_l = qw0 + l32;
  bool row_ok = true;
  if constexpr (SPL) row_ok = qi_l < sv.lq;
  if constexpr (DEC) {
    const int r = t * 32 + l32;
    row_ok = r < p.rows;
    const int rc = min(r, p.rows - 1);
    hl = h + rc / sv.lq;
    qi_l = rc % sv.lq;
  }
  const int q_lo = DEC ? 0 : qw0;  // smallest query index of the wave's rows
  // Eight waves with double-buffered 1 KB-row tiles run the two-group schedule below.
  constexpr bool kPingPong = NW == 8 && NBUF == 2 && NC == 2 && C::RS == 1024;

  const uint16_t* qh = (const uint16_t*)p.q + sv.q_off + (long long)hl * p.q_head;
  // K and V of the KV head: buffer resource over the head's rows and the row stride in bytes
  // (K and V may have different strides, e.g. slices of one fused QKV tensor).
  struct Src {
    i32x4_t rs;
    int rb;
  };
  auto stream_src = [&](const void* base, long long off, int row) {
    const int rb = row * 2;
    const uint32_t span = (uint32_t)min((long long)max(sv.lk, 1) * rb, (long long)0xFFFFFFF0);
    return Src{make_rsrc((const uint16_t*)base + off, span), rb};
  };
  const Src ksrc = stream_src(p.k, sv.k_off + (long long)kvh * p.k_head, p.k_row);
  const Src vsrc = stream_src(p.v, sv.v_off + (long long)kvh * p.v_head, p.v_row);

  const int off = sv.lk - sv.lq;  // tail alignment of the causal mask
  int kend = sv.lk;
  if (p.causal && !DEC) kend = min(kend, qt0 + C::BQ + off);
  const int ntk = kend > 0 ? (kend + 31) >> 5 : 0;
  // Key tiles of this workgroup: all of them, or (decode) this split's range.
  int jbeg = 0, jend = ntk;
  if constexpr (DEC) {
    jbeg = split * p.split_tiles;
    jend = min(jbeg + p.split_tiles, ntk);
  }
  if constexpr (SPL) {
    // an equal share of this query tile's own key tiles (empty ranges give O = 0, LSE = -inf)
    const int per = (ntk + p.nsplit - 1) / p.nsplit;
    jbeg = min(split * per, ntk);
    jend = min(jbeg + per, ntk);
  }

  // Q block of this wave as B operands: lane (h, n) holds query n, dims 16 kb + 8 h + 0..7.
  u32x4_t qreg[QB][2 * NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = DEC ? qi_l : min(qw0 + qb * 32 + l32, sv.lq - 1);
    const uint16_t* qrow = qh + (long long)qi * p.q_row;
#pragma unroll
    for (int kb = 0; kb < 2 * NDB; ++kb) {
      const int dim = cg * C::DW + kb * 16 + hh * 8;
      qreg[qb][kb] = dim < p.d ? *(const u32x4_t*)(qrow + dim) : (u32x4_t){0u, 0u, 0u, 0u};
    }
  }

  f32x16_t oacc[QB][NDB];
  float mref[QB], lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mref[qb] = -INFINITY;
    lsum[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[qb][db] = (f32x16_t){};
  }

  lds_t* const xbuf = smem + NBUF * 2 * C::TILE;

  // DMA: instruction ii of this wave fills LDS bytes [1024 i, 1024 i + 1024) of a tile, i = w + 4 ii,
  // i.e. tile row R = i / (RS / 1024) (uniform per instruction). Lane l writes physical chunk
  // pc = (i % (RS/1024)) * 64 + l; un-swizzled, u = pc ^ swz(R) is chunk u % SLOT of wave slot
  // u / SLOT, i.e. head-dim chunk (u / SLOT) WCH + u % SLOT. Padding chunks and chunks past the head dim
  // hold finite duplicates (clamped indices) that never reach a result. The column offset is
  // loop-invariant (VGPR); the row offset, clamped to the last key, is scalar.
  constexpr int IPR = C::RS / 1024;  // DMA instructions per LDS row
  const int dch = p.d >> 3;
  auto src_chunk = [&](int u) { return min((u / C::SLOT) * C::WCH + min(u % C::SLOT, C::WCH - 1), dch - 1); };
  int voff[C::NINSTR];
#pragma unroll
  for (int ii = 0; ii < C::NINSTR; ++ii) {
    const int i = w + NW * ii;
    const int R = i / IPR;
    const int pc = (i % IPR) * 64 + lane;
    voff[ii] = src_chunk(pc ^ swz(R)) << 4;
  }
  // Single-buffered eight-wave tiles: the column offsets are rebuilt from the hardware lane index
  // at each copy instead of holding NINSTR registers across the loop.
  constexpr bool kFreshOff = NBUF == 1 && NW == 8;
  auto issue1 = [&](const Src& x, int j, lds_t* dst, int ii) {
    const int i = w + NW * ii;
    const int row = min(j * 32 + i / IPR, sv.lk - 1);
    const int vo = kFreshOff ? src_chunk(((i % IPR) * 64 + fresh_lane_id()) ^ swz(i / IPR)) << 4 : voff[ii];
    lds_t* d = dst + i * 1024;
    if constexpr (kFreshOff) d = (lds_t*)(uintptr_t)opaque_s((uint32_t)(uintptr_t)d);
    dma16_buf(x.rs, vo, row * x.rb, d);
  };
  auto issue = [&](const Src& x, int j, lds_t* dst) {
#pragma unroll
    for (int ii = 0; ii < C::NINSTR; ++ii) issue1(x, j, dst, ii);
  };
  // With two buffers, the copies of tile j + 1 are spread over the MFMAs of step j (K during the
  // scores, V during P V): the copy path moves about 64 B per clock per CU, so a whole tile issued
  // at once would hold every wave at the issue for hundreds of cycles. They are issued for every
  // step, the last one included (rows clamped, into a buffer no longer read), so that no branch
  // splits the MFMA sequence; the kernel waits for them before it exits.
  // MFMA index after which copy ii of a run of N MFMAs is issued.
  auto spread_at = [](int n, int ii) { return (ii * n) / C::NINSTR; };

  const int krow = row_perm(l32);
  const int kswz = swz(krow);
  const int g16 = lane >> 4;
  const int r16 = lane & 15;
  const int cbase = cg * C::SLOT;  // first physical 16-byte chunk of this wave's slot

  // LDS byte addresses of this lane's operands in a tile at LDS address `tile`. The wave's slot
  // starts on a multiple of 16 chunks, so the swizzle (an XOR on the low 4 bits of the 16-byte
  // chunk index) touches only address bits 4-7, which are zero in the row, slot and tile bases:
  // every operand address is one per-lane base XOR a compile-time constant, plus a constant.
  // K rows (A operand of S^T): tile row row_perm(m), chunk cbase + 2 kb + h.
  const uint32_t klane = krow * C::RS + (cbase << 4) + ((hh ^ kswz) << 4);
  auto k_addr = [&](uint32_t tile, int kb) -> uint32_t {
    return ((tile + klane) ^ ((kb & 7) << 5)) + ((kb >> 3) << 8);
  };
  // V^T (A operand of O^T += V^T P^T) via transposed reads: key row
  // k = 16 kb2 + 8 h + 4 half + r16/4, head-dim column d = cg DW + 32 db + 16 (g16 % 2) + 4 (r16 % 4),
  // i.e. chunk cbase + 4 db + vclo. swz(k) does not depend on kb2.
  const int vclo = 2 * (g16 & 1) + ((r16 & 3) >> 1);
  const int vwithin = ((4 * (r16 & 3)) & 7) << 1;
  uint32_t vlane[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int k = 8 * hh + 4 * half + (r16 >> 2);
    vlane[half] = k * C::RS + (cbase << 4) + ((vclo ^ swz(k)) << 4) + vwithin;
  }
  auto v_addr = [&](uint32_t tile, int db, int kb2, int half) -> uint32_t {
    return ((tile + vlane[half]) ^ ((db & 3) << 6)) + ((db >> 2) << 8) + kb2 * 16 * C::RS;
  };

  // ---- pipeline pieces (each runs the same barriers in every wave) --------------------------
  // Start of a step: K_j has landed (in flight behind it: V_j, which is waited for later).
  auto top = [&]() {
    wait_vmcnt<C::NINSTR>();
    lds_barrier();
  };

  // attn_mask: this lane's mask rows and the raw bits of one tile (mask_fetch). The two-group
  // schedule requests tile j + 1's bits during the P V products of tile j (no copies are issued
  // there, and the score registers are free) and starts the scores of one wave of each row group
  // from the mask terms, so that the combined sum holds them once; the other schedules request
  // them when a tile's score products start and add them to the combined scores.
  // The row address is rebuilt at each fetch from the lane index (a few ALU operations) rather
  // than held in registers across the loop.
  u32x4_t mraw[QB][2];
  auto mask_fetch = [&](int j) {
    const int ln = fresh_lane_id();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      int hm = h, qm = min(qw0 + qb * 32 + (ln & 31), sv.lq - 1);
      if constexpr (DEC) {
        const int rc = min(t * 32 + (ln & 31), p.rows - 1);
        hm = h + rc / sv.lq;
        qm = rc % sv.lq;
      }
      const long long row = mask_row(p, s, hm, qm);
#pragma unroll
      for (int half = 0; half < 2; ++half)
        mraw[qb][half] = mask_raw8<T>(p, row, j * 32 + 16 * half + 8 * (ln >> 5), sv.lk);
    }
  };
  // Registers 0..7 of a score block hold keys 8 h + 0..7 of the tile, registers 8..15 keys
  // 16 + 8 h + 0..7.
  auto mask_terms = [&](int qb, f32x16_t& acc, bool add) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float mb[8];
      mask_apply8<T>(p, mraw[qb][half], mb);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[8 * half + e] = add ? acc[8 * half + e] + mb[e] : mb[e];
    }
  };

  // Partial S^T (keys x queries) of tile j over this wave's head-dim columns, written to the
  // exchange buffer; copy_at(kb) issues the tile copies assigned to k-step kb.
  auto s_partial = [&](int j, f32x16_t (&sacc)[QB], auto&& copy_at) {
    const lds_t* kt = kbuf(NBUF == 2 ? (j & 1) : 0);
    // (single-buffered eight waves: an opaque base, so that the constant operand addresses are
    // formed at each use instead of held in registers across the loop)
    const uint32_t kta = kFreshOff ? (uint32_t)opaque_v((int)lds_addr(kt)) : lds_addr(kt);
    if constexpr (MASK && kPingPong) {
      if (cg == 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) mask_terms(qb, sacc[qb], false);
      } else {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb] = (f32x16_t){};
      }
    } else {
      if constexpr (MASK) mask_fetch(j);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[qb] = (f32x16_t){};
    }
#pragma unroll
    for (int kb = 0; kb < 2 * NDB; ++kb) {
      const u32x4_t a = lds_read_b128_at(k_addr(kta, kb));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[qb] = Elt<T>::mma(a, qreg[qb][kb], sacc[qb]);
      copy_at(kb);
    }
    if constexpr (QB == 1) pin_lds_mfma_pipeline<2 * NDB, fwd_ahead<NC, NDB>(), 1>();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        lds_write_f4(xbuf, (((w * QB + qb) * 4 + r4) * 64 + lane) * 16,
                     (f32x4_t){sacc[qb][4 * r4], sacc[qb][4 * r4 + 1], sacc[qb][4 * r4 + 2], sacc[qb][4 * r4 + 3]});
  };

  // Full S^T of tile j (after the barrier that makes the partners' partial sums visible), masked.
  auto s_combine = [&](int j, f32x16_t (&sacc)[QB]) {
    // Add the partial sums of the row group's waves in a fixed commutative pattern, so that
    // every wave of the row group ends with bit-identical scores.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int base = rg * NC;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        auto rd = [&](int wv) { return lds_read_f4(xbuf, (((wv * QB + qb) * 4 + r4) * 64 + lane) * 16); };
        f32x4_t mine = (f32x4_t){sacc[qb][4 * r4], sacc[qb][4 * r4 + 1], sacc[qb][4 * r4 + 2], sacc[qb][4 * r4 + 3]};
        mine = mine + rd(base + (cg ^ 1));
        if constexpr (NC == 4) {
          const int o0 = base + ((cg & 2) ^ 2);
          mine = mine + (rd(o0) + rd(o0 + 1));
        }
        // Eight single-buffered waves: the sums of each half of the block are complete before
        // the next half's partner reads are issued (all twelve reads at once would need 48
        // registers the wave does not have).
        if constexpr (kFreshOff) {
          if (r4 & 1) asm volatile("" : "+v"(mine) : : "memory");
        }
        sacc[qb][4 * r4] = mine.x; sacc[qb][4 * r4 + 1] = mine.y;
        sacc[qb][4 * r4 + 2] = mine.z; sacc[qb][4 * r4 + 3] = mine.w;
      }
    }
    if constexpr (MASK && !kPingPong) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mask_terms(qb, sacc[qb], true);
    }
    // Mask tail keys and the causal diagonal (only on tiles that need it).
    const bool need_mask = (j * 32 + 32 > sv.lk) || (p.causal && j * 32 + 31 > q_lo + off);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = DEC ? qi_l : qw0 + qb * 32 + l32;
        const int lim = p.causal ? min(qi + off, sv.lk - 1) : sv.lk - 1;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (j * 32 + c_row(r, hh) > lim) sacc[qb][r] = -INFINITY;
      }
    }
  };

  // Full S^T of tile j, all eight waves in step (the loop without the two-group schedule).
  auto scores = [&](int j, f32x16_t (&sacc)[QB]) {
    s_partial(j, sacc, [&](int kb) {
      if constexpr (NBUF == 2) {
#pragma unroll
        for (int ii = 0; ii < C::NINSTR; ++ii)
          if (kb == spread_at(2 * NDB, ii)) issue1(ksrc, j + 1, kbuf((j + 1) & 1), ii);
      }
    });
    // In flight: V_j (issued during P V of step j - 1), then K_{j+1}. V_j is needed after this
    // barrier.
    if constexpr (NBUF == 2) wait_vmcnt<C::NINSTR>();
    lds_barrier();
    if constexpr (NBUF == 1) {
      if (j + 1 < jend) issue(ksrc, j + 1, kbuf(0));
    }
    s_combine(j, sacc);
  };

  // P = exp2(S * scale*log2e - mref), l += rowsum P, packed as B operands.
  auto make_p = [&](f32x16_t (&sacc)[QB], uint32_t (&pb)[QB][2][4]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mu = mref[qb] == -INFINITY ? 0.f : mref[qb];
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(sacc[qb][r] * p.scale_log2 - mu);
        sacc[qb][r] = pv;
        rs += pv;
      }
      lsum[qb] += rs;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pb[qb][kb2][e] = Elt<T>::pack2(sacc[qb][8 * kb2 + 2 * e], sacc[qb][8 * kb2 + 2 * e + 1]);
    }
  };

  // Row maxima of the tile in log2 units.
  auto tile_max = [&](const f32x16_t (&sacc)[QB], float (&mt)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = sacc[qb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) m = fmaxf(m, sacc[qb][r]);
      mt[qb] = half_max(m) * p.scale_log2;
    }
  };

  // O^T += V^T P^T for tile j; copy_at(m) issues the copies assigned to MFMA m.
  auto pv_mma = [&](int j, const uint32_t (&pb)[QB][2][4], auto&& copy_at) {
    const lds_t* vt = vbuf(NBUF == 2 ? (j & 1) : 0);
    const uint32_t vta = kFreshOff ? (uint32_t)opaque_v((int)lds_addr(vt)) : lds_addr(vt);
    // keys 0..15 of the tile (P registers 0..7) for every column block first, so the first half
    // of the products needs only the first half of P
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const s16x4_t lo = lds_read_tr16_at(v_addr(vta, db, kb2, 0));
        const s16x4_t hi = lds_read_tr16_at(v_addr(vta, db, kb2, 1));
        const u32x4_t a = join_tr(lo, hi);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const u32x4_t bop = {pb[qb][kb2][0], pb[qb][kb2][1], pb[qb][kb2][2], pb[qb][kb2][3]};
          oacc[qb][db] = Elt<T>::mma(a, bop, oacc[qb][db]);
        }
        copy_at(NDB * kb2 + db);
      }
    }
    if constexpr (QB == 1) pin_lds_mfma_pipeline<2 * NDB, fwd_ahead<NC, NDB>(), 2>();
  };
  auto pv = [&](int j, const uint32_t (&pb)[QB][2][4]) {
    if constexpr (NBUF == 1) {
      if (j + 1 < jend) wait_vmcnt<C::NINSTR>(); else wait_vmcnt<0>();  // V_j has landed
      lds_barrier();
    }
    pv_mma(j, pb, [&](int m) {
      if constexpr (NBUF == 2) {
#pragma unroll
        for (int ii = 0; ii < C::NINSTR; ++ii)
          if (m == spread_at(2 * NDB, ii)) issue1(vsrc, j + 1, vbuf((j + 1) & 1), ii);
      }
    });
    if constexpr (NBUF == 1) {
      lds_barrier();
      if (j + 1 < jend) issue(vsrc, j + 1, vbuf(0));
    }
  };

  if (jend > jbeg) {
    issue(ksrc, jbeg, kbuf(NBUF == 2 ? (jbeg & 1) : 0));
    // (single-buffered eight waves copy V_j during the step's score products)
    if constexpr (!kFreshOff) issue(vsrc, jbeg, vbuf(NBUF == 2 ? (jbeg & 1) : 0));
  }
  // The Q operands (and tile 0) are complete before the loop, so the loop never waits for them.
  wait_all();

  f32x16_t sacc[QB];
  if constexpr (kPingPong) {
    // Two-group schedule (eight waves, double-buffered K and V). Waves 0-3 (query row groups 0 and
    // 1) and waves 4-7 (row groups 2 and 3) form two groups; the two waves of a SIMD belong to
    // different groups. Each step is two slots separated by barriers:
    //   slot 0: group 0 forms partial scores of tile j | group 1 finishes tile j - 1 (exchange,
    //           softmax, P V)
    //   slot 1: group 0 finishes tile j                 | group 1 forms partial scores of tile j
    // so in every slot one wave of each SIMD multiplies scores while the other does the softmax
    // and then multiplies P V. Group 0 copies K of tile j + 1 after its score MFMAs (K_{j-1},
    // last read in slot 1 of step j - 1, has been released) and completes it before slot 0 of
    // step j + 1; group 1 copies V of tile j + 1 after its score MFMAs (V_{j-1}, last read in
    // slot 0 of step j, has been released) and completes it before slot 1 of step j + 1. Every
    // wave keeps its own exchange slot, which its partner reads in the next slot.
    const int grp = w >> 2, wg = w & 3;
    constexpr int GCOPY = 2 * C::NINSTR;  // 1 KB copies per wave of the group's tile
    int gvoff[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) gvoff[ii] = src_chunk(lane ^ swz(wg + 4 * ii)) << 4;
    const Src gsrc = grp == 0 ? ksrc : vsrc;
    auto gcopy = [&](int j, int ii) {
      const int i = wg + 4 * ii;
      lds_t* dst = (grp == 0 ? kbuf(j & 1) : vbuf(j & 1)) + i * 1024;
      dma16_buf(gsrc.rs, gvoff[ii & 3], min(j * 32 + i, sv.lk - 1) * gsrc.rb, dst);
    };
    // The group's copies go after its score products (and their exchange writes), not between
    // them: a wave held at a copy issue then no longer holds back its own MFMAs, which are in the
    // pipe, and the partner's P V products have the pipe to themselves (4.40 -> 4.06 ms at the
    // headline shape). The tile has the rest of this slot and the next one to land.
    auto s_phase = [&](int j) {
      s_partial(j, sacc, [&](int) {});
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ii = 0; ii < GCOPY; ++ii) gcopy(j + 1, ii);
    };
    // Without a mask, the V^T operand of the first P V product is requested ahead of the exchange
    // reads, so that its LDS latency overlaps the wait for the partner's partial scores (0.9% at
    // the headline shape; the masked form has no registers to spare for it).
    const uint32_t vta0 = lds_addr(vbuf(0)), vta1 = lds_addr(vbuf(1));
    auto p_phase = [&](int j) {
      const uint32_t vta = (j & 1) ? vta1 : vta0;
      auto vread = [&](int m) {
        const int kb2 = m / NDB, db = m % NDB;
        return join_tr(lds_read_tr16_at(v_addr(vta, db, kb2, 0)), lds_read_tr16_at(v_addr(vta, db, kb2, 1)));
      };
      u32x4_t a0 = {};
      if constexpr (!MASK) {
        a0 = vread(0);
        __builtin_amdgcn_sched_barrier(0);
      }
      s_combine(j, sacc);
      // Online softmax with a lazily updated reference max: a row's reference is its first finite
      // tile max, raised (with the matching rescale of O and l) only when a tile max exceeds it
      // by more than 2^8; exp2 then stays below 256.
      float mt[QB];
      tile_max(sacc, mt);
      bool grow = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (mref[qb] == -INFINITY) mref[qb] = mt[qb];
        grow |= mt[qb] > mref[qb] + 8.0f;
      }
      if (__any(grow)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const bool nd = mt[qb] > mref[qb] + 8.0f;
          const float alpha = nd ? fast_exp2(mref[qb] - mt[qb]) : 1.0f;
          if (nd) mref[qb] = mt[qb];
          lsum[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[qb][db] *= alpha;
        }
      }
      uint32_t pb[QB][2][4];
      make_p(sacc, pb);
      if constexpr (MASK) {
        if (cg == 0) mask_fetch(j + 1);  // past the last tile: clamped to the row, unused
        pv_mma(j, pb, [](int) {});
      } else {
        // keys-first order as in pv_mma; operand m = NDB kb2 + db, the first one already read
        static_assert(QB == 1, "one query block per wave");
#pragma unroll
        for (int m = 0; m < 2 * NDB; ++m) {
          const int kb2 = m / NDB, db = m % NDB;
          const u32x4_t a = m == 0 ? a0 : vread(m);
          const u32x4_t bop = {pb[0][kb2][0], pb[0][kb2][1], pb[0][kb2][2], pb[0][kb2][3]};
          oacc[0][db] = Elt<T>::mma(a, bop, oacc[0][db]);
        }
        // the operand reads run AHEAD MFMAs ahead, as in pin_lds_mfma_pipeline, the first operand
        // already read
        constexpr int AHEAD = fwd_ahead<NC, NDB>();
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (AHEAD - 1), 0);
#pragma unroll
        for (int i = 0; i < 2 * NDB - AHEAD; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
      }
    };
    if constexpr (MASK) {
      if (cg == 0) mask_fetch(jbeg);
    }
    lds_barrier();
    if (jend > jbeg) {
      if (grp == 0) {
        for (int j = jbeg; j < jend; ++j) {
          s_phase(j);
          lds_barrier();
          p_phase(j);
          wait_vmcnt<0>();  // K_{j+1}
          lds_barrier();
        }
        lds_barrier();
      } else {
        lds_barrier();
        for (int j = jbeg; j < jend; ++j) {
          s_phase(j);
          lds_barrier();
          p_phase(j);
          wait_vmcnt<0>();  // V_{j+1}
          lds_barrier();
        }
      }
    }
  } else {

  if constexpr (kFreshOff) {
    // Eight waves, single-buffered K and V tiles (64 KB each). The copies are spread over the
    // MFMAs (a burst of them would hold every wave at the copy issue, which drains at about 64
    // bytes per clock per CU): V_j during the score products of step j (V_{j-1} was last read
    // before the barrier that opens the step) and K_{j+1} during the P V products of step j (K_j
    // was last read before the exchange barrier). K_{j+1} is issued on the last step too (rows
    // clamped, into a buffer no longer read) so that no branch splits the MFMA sequence. One loop
    // with the lazily updated reference max (rescale only when a tile max exceeds the reference
    // by more than 2^8), as in the two-group schedule.
    for (int j = jbeg; j < jend; ++j) {
      wait_vmcnt<0>();  // K_j: the only copies in flight
      lds_barrier();
      s_partial(j, sacc, [&](int kb) {
#pragma unroll
        for (int ii = 0; ii < C::NINSTR; ++ii)
          if (kb == spread_at(2 * NDB, ii)) issue1(vsrc, j, vbuf(0), ii);
      });
      lds_barrier();  // partial sums visible; K_j released
      s_combine(j, sacc);
      float mt[QB];
      tile_max(sacc, mt);
      bool grow = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (mref[qb] == -INFINITY) mref[qb] = mt[qb];
        grow |= mt[qb] > mref[qb] + 8.0f;
      }
      if (__any(grow)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const bool nd = mt[qb] > mref[qb] + 8.0f;
          const float alpha = nd ? fast_exp2(mref[qb] - mt[qb]) : 1.0f;
          if (nd) mref[qb] = mt[qb];
          lsum[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[qb][db] *= alpha;
        }
      }
      uint32_t pb[QB][2][4];
      make_p(sacc, pb);
      wait_vmcnt<0>();  // V_j (and any mask bits of the tile)
      lds_barrier();
      pv_mma(j, pb, [&](int m) {
#pragma unroll
        for (int ii = 0; ii < C::NINSTR; ++ii)
          if (m == spread_at(2 * NDB, ii)) issue1(ksrc, j + 1, kbuf(0), ii);
      });
    }
  } else {
  // ---- fast loop: the reference max of a row is fixed at its first finite tile max. The loop
  // leaves (per wave) as soon as a tile max exceeds the reference by more than 2^8, so O never
  // needs rescaling here and exp2 stays below 256.
  int j = jbeg;
  for (; j < jend; ++j) {
    top();
    scores(j, sacc);
    float mt[QB];
    tile_max(sacc, mt);
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (mref[qb] == -INFINITY) mref[qb] = mt[qb];
      grow |= mt[qb] > mref[qb] + 8.0f;
    }
    if (__any(grow)) break;
    uint32_t pb[QB][2][4];
    make_p(sacc, pb);
    pv(j, pb);
  }

  // ---- rescaling loop (entered only after a large growth of a row max): standard online
  // softmax with a lazily updated reference. Tile j's scores are already in sacc.
  for (bool fresh = false; j < jend; ++j, fresh = true) {
    if (fresh) {
      top();
      scores(j, sacc);
    }
    float mt[QB];
    tile_max(sacc, mt);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const bool nd = mt[qb] > mref[qb] + 8.0f;
      const float alpha = nd ? fast_exp2(mref[qb] - mt[qb]) : 1.0f;
      if (nd) mref[qb] = mt[qb];
      lsum[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[qb][db] *= alpha;
    }
    uint32_t pb[QB][2][4];
    make_p(sacc, pb);
    pv(j, pb);
  }
  }  // !kFreshOff
  }  // !kPingPong

  // Copies issued during the last step land in LDS that the next workgroup may own.
  wait_vmcnt<0>();

  // Eight-wave prefill forms write O through LDS, whole rows per store (store_block_rows).
  constexpr bool kRowStore = NW == 8 && !DEC;
  if constexpr (DEC || SPL) {
    // ---- decode / split epilogue: this key range's normalised O (fp32) and its LSE in log2 units
    // (-inf and 0 when no key of the range is legal for the row), for the combine pass.
    const float lt = half_sum(lsum[0]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    if constexpr (kRowStore) {
      const long long prow0 = ((long long)s * p.hq + h) * sv.lq + qt0;
      store_block_rows<T, true, NW / NC, NC, 1, NDB, C::LDS>(smem, oacc, inv, p.part_o + (prow0 * p.nsplit + split) * p.d,
                                                     (long long)p.nsplit * p.d, sv.lq - qt0, p.d);
      if (row_ok && cg == 0 && hh == 0)
        p.part_lse[((prow0 + 32 * rg + l32) * p.nsplit) + split] = lt > 0.f ? mref[0] + fast_log2(lt) : -INFINITY;
      return;
    }
    if (row_ok) {
      const long long prow = ((long long)s * p.hq + hl) * sv.lq + qi_l;
      float* orow = p.part_o + (prow * p.nsplit + split) * p.d;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = cg * C::DW + 32 * db + 8 * i4 + 4 * hh;
          if (d < p.d) {
            const f32x16_t& o = oacc[0][db];
            *(f32x4_t*)(orow + d) = (f32x4_t){o[4 * i4] * inv, o[4 * i4 + 1] * inv, o[4 * i4 + 2] * inv,
                                              o[4 * i4 + 3] * inv};
          }
        }
      if (cg == 0 && hh == 0) p.part_lse[prow * p.nsplit + split] = lt > 0.f ? mref[0] + fast_log2(lt) : -INFINITY;
    }
    return;
  }

  // ---- epilogue: O = O^T / l, LSE = ln(2) * (mref + log2 l); empty rows give 0 and -inf
  if constexpr (kRowStore) {
    static_assert(QB == 1, "one query block per wave");
    const float lt = half_sum(lsum[0]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    store_block_rows<T, false, NW / NC, NC, 1, NDB, C::LDS>(smem, oacc, inv,
                                                    (uint16_t*)p.o + sv.o_off + (long long)h * p.o_head +
                                                        (long long)qt0 * p.o_row,
                                                    p.o_row, sv.lq - qt0, p.d);
    const int qi = qw0 + l32;
    if (qi < sv.lq && cg == 0 && hh == 0)
      p.lse[sv.lse_off + (long long)h * p.lse_head + qi] = lt > 0.f ? (mref[0] + fast_log2(lt)) * kLn2 : -INFINITY;
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = half_sum(lsum[qb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int qi = qw0 + qb * 32 + l32;
    if (qi < sv.lq) {
      uint16_t* orow = (uint16_t*)p.o + sv.o_off + (long long)h * p.o_head + (long long)qi * p.o_row;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = cg * C::DW + 32 * db + 8 * i4 + 4 * hh;
          if (d < p.d) {
            const f32x16_t& o = oacc[qb][db];
            const u32x2_t pk = {Elt<T>::pack2(o[4 * i4] * inv, o[4 * i4 + 1] * inv),
                                Elt<T>::pack2(o[4 * i4 + 2] * inv, o[4 * i4 + 3] * inv)};
            *(u32x2_t*)(orow + d) = pk;
          }
        }
      if (cg == 0 && hh == 0)
        p.lse[sv.lse_off + (long long)h * p.lse_head + qi] =
            lt > 0.f ? (mref[qb] + fast_log2(lt)) * kLn2 : -INFINITY;
    }
  }
}

template <class T, int NC, int NDB, int NW, bool MASK>
static hipError_t launch_fwd_nw(AttnParams p, hipStream_t st) {
  constexpr int QB = 1;
  using C1 = FwdCfg<NC, NDB, QB, 1, NW>;
  constexpr int NBUF = (2 * 2 * C1::TILE + C1::XBYTES) <= 160 * 1024 ? 2 : 1;
  using C = FwdCfg<NC, NDB, QB, NBUF, NW>;
  p.ntiles = (p.nq + C::BQ - 1) / C::BQ;
  p.total = p.batch * p.hq * p.ntiles;
  if (p.total == 0) return hipSuccess;
  const int grid = (p.total + 7) & ~7;
  hipLaunchKernelGGL((ffpa_fwd_kernel<T, NC, NDB, QB, NBUF, NW, false, MASK>), dim3(grid), dim3(64 * NW), 0, st, p);
  return hipGetLastError();
}

// Eight waves (two per SIMD): 128 queries per workgroup for D <= 512 (two head-dim halves,
// double-buffered 32 KB tiles), 64 for D > 512 (four head-dim quarters, single-buffered 64 KB K and
// V tiles: each copied K/V byte then feeds twice the queries of a four-wave workgroup). The masked
// form above D = 896 keeps four waves (32 queries): its mask registers do not fit beside the
// 256-column operands in the 256 registers of a two-wave SIMD.
template <class T, int NC, int NDB>
static hipError_t launch_fwd_cfg(AttnParams p, hipStream_t st) {
  static_assert(NC == 2 || NC == 4, "head-dim split");
  if (p.mask_kind != 0) return launch_fwd_nw<T, NC, NDB, (NC == 4 && NDB == 8) ? 4 : 8, true>(p, st);
  return launch_fwd_nw<T, NC, NDB, 8, false>(p, st);
}

// Merge of the key-range split forward: many rows, few ranges. One wave per output row (four rows
// per workgroup); lane l covers columns 8 l .. + 7 of each 512-column chunk and loops over the
// ranges in order: LSE = log2 sum_s exp2(LSE_s), O = sum_s exp2(LSE_s - LSE) O_s, the same formula
// as the decode merge in a fixed order.
template <class T>
__global__ void __launch_bounds__(256) ffpa_split_combine_kernel(AttnParams p, int nrows) {
  const int row = blockIdx.x * 4 + wave_id();
  if (row >= nrows) return;
  const int lane = threadIdx.x & 63;
  const int i = row % p.nq;
  const int bh = row / p.nq;
  const int h = bh % p.hq;
  const int b = bh / p.hq;
  const float* lp = p.part_lse + (long long)row * p.nsplit;
  const float* po = p.part_o + (long long)row * p.nsplit * p.d;
  float m = -INFINITY;
  for (int sp = 0; sp < p.nsplit; ++sp) m = fmaxf(m, lp[sp]);
  float l = 0.f;
  if (m != -INFINITY)
    for (int sp = 0; sp < p.nsplit; ++sp) l += fast_exp2(lp[sp] - m);  // 0 for a range without a legal key
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  uint16_t* orow = (uint16_t*)p.o + (long long)b * p.o_batch + (long long)h * p.o_head + (long long)i * p.o_row;
  for (int d0 = 8 * lane; d0 < p.d; d0 += 512) {
    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    if (m != -INFINITY)
      for (int sp = 0; sp < p.nsplit; ++sp) {
        const float wgt = fast_exp2(lp[sp] - m);
        const float* src = po + (long long)sp * p.d + d0;
        // Read once: non-temporal loads, so that the partials do not stay in the caches at the
        // expense of the next launch's operands (the P/dS pass after a split forward ran about 35%
        // slower with ordinary loads here).
        a0 += wgt * __builtin_nontemporal_load((const f32x4_t*)src);
        a1 += wgt * __builtin_nontemporal_load((const f32x4_t*)(src + 4));
      }
    *(u32x4_t*)(orow + d0) = (u32x4_t){Elt<T>::pack2(a0.x * inv, a0.y * inv), Elt<T>::pack2(a0.z * inv, a0.w * inv),
                                       Elt<T>::pack2(a1.x * inv, a1.y * inv), Elt<T>::pack2(a1.z * inv, a1.w * inv)};
  }
  if (lane == 0)
    p.lse[(long long)b * p.lse_batch + (long long)h * p.lse_head + i] = l > 0.f ? (m + fast_log2(l)) * kLn2 : -INFINITY;
}

// Key-range split count of a dense forward: 1 when the grid gives at least two workgroups per
// compute unit (of 256), else enough ranges for that, up to 8 and with at least 4 key tiles each.
int fwd_split_count(int batch, int hq, int nq, int nkv, int d) {
  const int bq = d <= 512 ? 128 : 64;  // queries per workgroup of the forward configurations
  const long long base = (long long)batch * hq * ((nq + bq - 1) / bq);
  const long long ktiles = (nkv + 31) / 32;
  if (base <= 0 || base >= 512) return 1;
  return (int)std::max(1LL, std::min({8LL, (512 + base - 1) / base, ktiles / 4}));
}

template <class T, int NC, int NDB>
static hipError_t launch_fwd_split_cfg(AttnParams p, int nsplit, float* ws, hipStream_t st) {
  constexpr int QB = 1;
  constexpr int NW = 8;
  using C1 = FwdCfg<NC, NDB, QB, 1, NW>;
  constexpr int NBUF = (2 * 2 * C1::TILE + C1::XBYTES) <= 160 * 1024 ? 2 : 1;
  using C = FwdCfg<NC, NDB, QB, NBUF, NW>;
  p.ntiles = (p.nq + C::BQ - 1) / C::BQ;
  p.nsplit = nsplit;
  const long long nrows = (long long)p.batch * p.hq * p.nq;
  p.part_o = ws;
  p.part_lse = ws + nrows * nsplit * p.d;
  p.total = p.batch * p.hq * p.ntiles * nsplit;
  if (p.total == 0) return hipSuccess;
  const int grid = (p.total + 7) & ~7;
  hipLaunchKernelGGL((ffpa_fwd_kernel<T, NC, NDB, QB, NBUF, NW, false, false, true>), dim3(grid), dim3(64 * NW), 0, st,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ffpa_split_combine_kernel<T>, dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, st, p, (int)nrows);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_fwd_split_t(const AttnParams& p, int nsplit, float* ws, hipStream_t st) {
  if (p.d <= 512) {
    switch ((p.d + 63) / 64) {
      case 5: return launch_fwd_split_cfg<T, 2, 5>(p, nsplit, ws, st);
      case 6: return launch_fwd_split_cfg<T, 2, 6>(p, nsplit, ws, st);
      case 7: return launch_fwd_split_cfg<T, 2, 7>(p, nsplit, ws, st);
      default: return launch_fwd_split_cfg<T, 2, 8>(p, nsplit, ws, st);
    }
  }
  switch ((p.d + 127) / 128) {
    case 5: return launch_fwd_split_cfg<T, 4, 5>(p, nsplit, ws, st);
    case 6: return launch_fwd_split_cfg<T, 4, 6>(p, nsplit, ws, st);
    case 7: return launch_fwd_split_cfg<T, 4, 7>(p, nsplit, ws, st);
    default: return launch_fwd_split_cfg<T, 4, 8>(p, nsplit, ws, st);
  }
}

hipError_t launch_fwd_split(const AttnParams& p, int fp16, int nsplit, void* ws, hipStream_t st) {
  return fp16 ? launch_fwd_split_t<FP16>(p, nsplit, (float*)ws, st) : launch_fwd_split_t<BF16>(p, nsplit, (float*)ws, st);
}

template <class T>
static hipError_t launch_fwd_t(const AttnParams& p, hipStream_t st) {
  if (p.d <= 512) {
    switch ((p.d + 63) / 64) {
      case 5: return launch_fwd_cfg<T, 2, 5>(p, st);
      case 6: return launch_fwd_cfg<T, 2, 6>(p, st);
      case 7: return launch_fwd_cfg<T, 2, 7>(p, st);
      default: return launch_fwd_cfg<T, 2, 8>(p, st);
    }
  }
  switch ((p.d + 127) / 128) {
    case 5: return launch_fwd_cfg<T, 4, 5>(p, st);
    case 6: return launch_fwd_cfg<T, 4, 6>(p, st);
    case 7: return launch_fwd_cfg<T, 4, 7>(p, st);
    default: return launch_fwd_cfg<T, 4, 8>(p, st);
  }
}

hipError_t launch_fwd(const AttnParams& p, int fp16, hipStream_t st) {
  return fp16 ? launch_fwd_t<FP16>(p, st) : launch_fwd_t<BF16>(p, st);
}

// ------------------------------------------------------------------------------------------------
// Split-KV decode ("Triton Backend", "Feature support": decode as a two-stage split-KV path;
// "Backends Overview", "Automatic SDPA fallback": the native decode path serves Nq in [1, 8)).
//
// With a handful of queries the forward grid above has one small workgroup per (head, 128
// queries) that streams all of K and V: a few dozen workgroups for the whole GPU, and each KV
// head read once per query head of its group. The decode form instead gives every workgroup one
// KV head, one 32-row block of (query head of the group, query) rows -- all G * Nq rows of the
// group share each K/V tile -- and one range of key tiles; the key ranges of a row are
// independent (partial O normalised by its own sum, plus its LSE) and a second pass merges them:
//   LSE = log sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s,
// which is exactly the softmax over the union of the ranges (the merge: one workgroup per output
// row and 256 columns, its four waves taking every fourth range). The work is HBM-bound (each K/V
// byte is read once per row block): the split count fills the GPU with about two workgroups per
// compute unit while keeping at least four tiles per range. Four waves split the head dim
// (NC = 4); K and V tiles are double-buffered for D <= 512.
// ------------------------------------------------------------------------------------------------
template <class T>
__global__ void __launch_bounds__(256) ffpa_decode_combine_kernel(AttnParams p, int nrows) {
  // Workgroup = (output row (b, h, i) = ((b * Hq + h) * Nq + i), 256-column chunk); lane l covers
  // columns 256 chunk + 4 l .. + 3, and wave w the key ranges w, w + 4, ...; the four partial sums
  // are added through LDS in a fixed order. Every wave forms the same max and weight sum.
  __shared__ f32x4_t part[3][64];
  const int nchunk = (p.d + 255) / 256;
  const int row = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  if (row >= nrows) return;
  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int i = row % p.nq;
  const int bh = row / p.nq;
  const int h = bh % p.hq;
  const int b = bh / p.hq;
  const float* lp = p.part_lse + (long long)row * p.nsplit;
  const float* po = p.part_o + (long long)row * p.nsplit * p.d;
  float m = -INFINITY;
  for (int sp = 0; sp < p.nsplit; ++sp) m = fmaxf(m, lp[sp]);
  float l = 0.f;
  if (m != -INFINITY)
    for (int sp = 0; sp < p.nsplit; ++sp) l += fast_exp2(lp[sp] - m);  // 0 for a range without a legal key
  const int d = 256 * chunk + 4 * lane;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (m != -INFINITY && d < p.d)
    for (int sp = w; sp < p.nsplit; sp += 4) acc += fast_exp2(lp[sp] - m) * *(const f32x4_t*)(po + (long long)sp * p.d + d);
  if (w > 0) part[w - 1][lane] = acc;
  __syncthreads();
  if (w != 0) return;
  acc = ((acc + part[0][lane]) + part[1][lane]) + part[2][lane];
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  uint16_t* orow = (uint16_t*)p.o + (long long)b * p.o_batch + (long long)h * p.o_head + (long long)i * p.o_row;
  if (d < p.d)
    *(u32x2_t*)(orow + d) = (u32x2_t){Elt<T>::pack2(acc.x * inv, acc.y * inv), Elt<T>::pack2(acc.z * inv, acc.w * inv)};
  if (lane == 0 && chunk == 0)
    p.lse[(long long)b * p.lse_batch + (long long)h * p.lse_head + i] = l > 0.f ? (m + fast_log2(l)) * kLn2 : -INFINITY;
}

template <class T, int NDB>
static hipError_t launch_decode_cfg(AttnParams p, hipStream_t st) {
  constexpr int NC = 4, NW = 4, QB = 1;
  using C1 = FwdCfg<NC, NDB, QB, 1, NW>;
  constexpr int NBUF = (2 * 2 * C1::TILE + C1::XBYTES) <= 160 * 1024 ? 2 : 1;
  p.total = p.batch * p.hkv * p.nsplit * p.nrb;
  if (p.total == 0) return hipSuccess;
  const int grid = (p.total + 7) & ~7;
  if (p.mask_kind != 0)
    hipLaunchKernelGGL((ffpa_fwd_kernel<T, NC, NDB, QB, NBUF, NW, true, true>), dim3(grid), dim3(64 * NW), 0, st, p);
  else
    hipLaunchKernelGGL((ffpa_fwd_kernel<T, NC, NDB, QB, NBUF, NW, true>), dim3(grid), dim3(64 * NW), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nrows = p.batch * p.hq * p.nq;
  hipLaunchKernelGGL(ffpa_decode_combine_kernel<T>, dim3(nrows * ((p.d + 255) / 256)), dim3(256), 0, st, p, nrows);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_decode_t(const AttnParams& p, hipStream_t st) {
  switch ((p.d + 127) / 128) {
    case 3: return launch_decode_cfg<T, 3>(p, st);
    case 4: return launch_decode_cfg<T, 4>(p, st);
    case 5: return launch_decode_cfg<T, 5>(p, st);
    case 6: return launch_decode_cfg<T, 6>(p, st);
    case 7: return launch_decode_cfg<T, 7>(p, st);
    default: return launch_decode_cfg<T, 8>(p, st);
  }
}

hipError_t launch_decode(const AttnParams& p, int fp16, hipStream_t st) {
  return fp16 ? launch_decode_t<FP16>(p, st) : launch_decode_t<BF16>(p, st);
}

}  // namespace ffpa
