// Launch parameters shared by the host dispatcher and the kernels (plain data, no HIP types).
#pragma once

#include <stdint.h>

namespace ffpa {

struct AttnParams {
  // Tensors. o/dout/dq share q's strides; v/dk/dv share k's strides; lse/delta share lse strides.
  const void* q;
  const void* k;
  const void* v;
  const void* o_in;     // backward: forward output O
  const void* dout;     // backward: dO
  void* o;              // forward output
  float* lse;           // forward output
  const float* lse_in;  // backward input
  const float* dlse;    // backward: gradient of the returned LSE (lse layout), or NULL for zero
  float* delta;         // backward: Delta = rowsum(dO * O)
  void* dq;
  void* dk;
  void* dv;
  const int32_t* cu_q;  // varlen: [batch+1]; NULL for dense
  const int32_t* cu_k;
  // Stored dS (same dtype as q), or NULL, transposed: row (b or sequence s, query head h, key j)
  // holds queries 0..nq-1 padded to ds_row = round_up(nq, 8) elements. Dense: element offset
  // b * ds_batch + h * ds_head + j * ds_row + i. Varlen: sequence s starts at hq * P_s with
  // P_s = sum over earlier sequences of Lk * round_up(Lq, 8), head h at + h * Lk_s * round_up(Lq_s, 8).
  void* ds;
  void* pst;  // stored P (same geometry as ds), or NULL
  long long ds_batch, ds_head;
  int ds_row;
  // Dense strides in elements (unused for varlen except row/head strides). The forward reads V
  // and writes O with their own strides (v_*, o_*); every other kernel uses q's strides for
  // o/dout/dq and k's for v/dk/dv, and the backward entry points set v_* = k_*, o_* = q_*.
  long long q_batch, k_batch, lse_batch, v_batch, o_batch;
  int q_row, q_head, k_row, k_head, lse_head, v_row, v_head, o_row, o_head;
  // Problem.
  int batch, hq, hkv, group;  // group = hq / hkv
  int nq, nkv;                // dense lengths, or max lengths for varlen
  int d, causal;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  // Grid decode.
  int ntiles;  // row tiles per (sequence, head)
  int total;   // work items = batch * heads * ntiles
  // Split-KV decode: rows = G * nq (query head in group, query) rows per KV head in nrb blocks of
  // 32; nsplit key ranges of split_tiles 32-key tiles; per (row, range) a normalised fp32 O
  // (part_o [B, Hq, Nq, nsplit, D]) and its log2-domain LSE (part_lse [B, Hq, Nq, nsplit]).
  int rows, nrb, nsplit, split_tiles;
  float* part_o;
  float* part_lse;
  // attn_mask (dense entry points): kind 0 none, 1 additive bias (q's dtype, added to the scaled
  // scores), 2 boolean (one byte per element, nonzero keeps the key). Element (b, h, i, j) sits at
  // b * m_batch + h * m_head + i * m_row + j * m_key (stride 0 broadcasts; m_key is 0 or 1).
  // dmask: the bias gradient (q's dtype), packed in the shape with a 1 for every 0-stride dim.
  const void* mask;
  void* dmask;
  int mask_kind;
  long long m_batch, m_head;
  int m_row, m_key;
  float inv_scale;  // 1 / scale: the bias in units of the raw scores
};

}  // namespace ffpa
