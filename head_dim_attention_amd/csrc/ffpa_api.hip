// Host side of libffpa.so: argument validation, launch geometry and the C ABI (include/ffpa.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/ffpa.h"
#include "ffpa_params.h"

namespace ffpa {
hipError_t launch_fwd(const AttnParams& p, int fp16, hipStream_t st);
hipError_t launch_decode(const AttnParams& p, int fp16, hipStream_t st);
hipError_t launch_fwd_fp8(const AttnParams& p, int fp16, void* ws, hipStream_t st);
hipError_t launch_fwd_split(const AttnParams& p, int fp16, int nsplit, void* ws, hipStream_t st);
int fwd_split_count(int batch, int hq, int nq, int nkv, int d);
size_t fp8_workspace_bytes(int batch, int hq, int hkv, int nkv, int d);
hipError_t launch_bwd(const AttnParams& p, int fp16, int nrows, int varlen_total, hipStream_t st, int stage);
bool fused_products(const AttnParams& p);
}  // namespace ffpa

using ffpa::AttnParams;

// Fixed device scratch of ffpa_decode_fwd_noalloc (partial O and LSE of the split-KV decode). In
// host code `scratch` is only a stand-in for the symbol: its device address, per device, comes
// from hipGetSymbolAddress and is the only form passed to kernels.
static __device__ __align__(256) char scratch[FFPA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device (with that device
// current); NULL on failure.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

bool bad_dtype(int dtype) { return dtype != FFPA_DTYPE_BF16 && dtype != FFPA_DTYPE_FP16; }

// Shared checks of every entry point; NOT_SUPPORTED is reported only for otherwise valid calls.
ffpa_status_t check_common(int hq, int hkv, int d, int dtype, float scale, int causal) {
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return FFPA_ERR_INVALID_ARGUMENT;
  if (bad_dtype(dtype)) return FFPA_ERR_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return FFPA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FFPA_ERR_INVALID_ARGUMENT;
  if (d < 320 || d > 1024 || d % 32 != 0) return FFPA_ERR_NOT_SUPPORTED;
  return FFPA_OK;
}

AttnParams dense_params(int batch, int hq, int hkv, int nq, int nkv, int d, float scale, int causal) {
  AttnParams p{};
  p.q_row = d;
  p.q_head = nq * d;
  p.q_batch = (long long)hq * nq * d;
  p.k_row = d;
  p.k_head = nkv * d;
  p.k_batch = (long long)hkv * nkv * d;
  p.lse_head = nq;
  p.lse_batch = (long long)hq * nq;
  p.v_row = p.k_row;
  p.v_head = p.k_head;
  p.v_batch = p.k_batch;
  p.o_row = p.q_row;
  p.o_head = p.q_head;
  p.o_batch = p.q_batch;
  p.batch = batch;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.nq = nq;
  p.nkv = nkv;
  p.d = d;
  p.causal = causal;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  return p;
}

AttnParams varlen_params(int batch, int max_q, int max_k, int total_q, int hq, int hkv, int d, float scale,
                         int causal, const int32_t* cu_q, const int32_t* cu_k) {
  AttnParams p{};
  p.q_row = hq * d;
  p.q_head = d;
  p.k_row = hkv * d;
  p.k_head = d;
  p.lse_head = total_q;
  p.v_row = p.k_row;
  p.v_head = p.k_head;
  p.o_row = p.q_row;
  p.o_head = p.q_head;
  p.cu_q = cu_q;
  p.cu_k = cu_k != nullptr ? cu_k : cu_q;
  p.batch = batch;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.nq = max_q;
  p.nkv = max_k;
  p.d = d;
  p.causal = causal;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  return p;
}

ffpa_status_t to_status(hipError_t e) { return e == hipSuccess ? FFPA_OK : FFPA_ERR_HIP; }

// Sizes in elements must stay addressable with the kernels' 32-bit row/head arithmetic.
bool too_big_dense(int batch, int h, int n, int d) {
  const long long per_head = (long long)n * d;
  return per_head > (1LL << 31) - 1 || (long long)batch * h * per_head > (1LL << 46);
}

long long round_up8(long long x) { return (x + 7) & ~7LL; }

// Bytes of one head's stored dS (or P) block, transposed: nkv rows of round_up8(nq) elements; the
// kernels address it with 32-bit byte offsets, so larger blocks use the recomputing kernels.
bool ds_block_ok(long long nq, long long nkv) { return nkv * round_up8(nq) * 2 <= (1LL << 31) - 4096; }

// The workspace holds two equal blocks: dS, then P.
size_t dense_ds_bytes(int batch, int hq, int nq, int nkv) {
  if (batch < 1 || hq < 1 || nq < 1 || nkv < 1 || !ds_block_ok(nq, nkv)) return 0;
  return 2 * (size_t)batch * hq * nkv * round_up8(nq) * 2;
}

// Sequence s needs Lk_s * round_up8(Lq_s) elements per head and block, at most
// Lk_s * round_up8(max_q); the sum over sequences is at most total_k * round_up8(max_q).
size_t varlen_ds_bytes(int hq, int total_q, int total_k, int max_q, int max_k) {
  if (hq < 1 || total_q < 1 || total_k < 1 || max_q < 1 || max_k < 1 || !ds_block_ok(max_q, max_k)) return 0;
  return 2 * (size_t)hq * total_k * round_up8(max_q) * 2;
}

// Host copies of cu_seqlens (k NULL: the q ones) that follow the rules of the varlen entry points
// for these totals and max lengths: batch + 1 entries from 0, non-decreasing, ending at the totals,
// every length at most the max length.
bool host_cu_ok(int batch, const int32_t* cu, int total, int max_len) {
  if (cu == nullptr || batch < 1 || cu[0] != 0 || cu[batch] != total) return false;
  for (int s = 0; s < batch; ++s)
    if (cu[s + 1] < cu[s] || cu[s + 1] - cu[s] > max_len) return false;
  return true;
}

// Exact P/dS workspace of these sequences: two blocks of hq * sum_s Lk_s * round_up8(Lq_s)
// elements (the layout the kernels address, sequence by sequence), or 0 when not available.
size_t varlen_ds_bytes_exact(int hq, int batch, const int32_t* cu_q, const int32_t* cu_k, int total_q, int total_k,
                             int max_q, int max_k) {
  if (cu_k == nullptr) cu_k = cu_q;
  if (hq < 1 || total_q < 1 || total_k < 1 || max_q < 1 || max_k < 1 || !ds_block_ok(max_q, max_k)) return 0;
  if (!host_cu_ok(batch, cu_q, total_q, max_q) || !host_cu_ok(batch, cu_k, total_k, max_k)) return 0;
  if (cu_k == cu_q && total_k != total_q) return 0;
  long long elems = 0;
  for (int s = 0; s < batch; ++s) elems += (long long)(cu_k[s + 1] - cu_k[s]) * round_up8(cu_q[s + 1] - cu_q[s]);
  return elems == 0 ? 0 : 2 * (size_t)hq * (size_t)elems * 2;
}

// Strided forward layouts: strides[12] = {q, k, v, o} x {batch, head, row} in elements (the head
// dim is contiguous). Rows must stay 16-byte aligned (strides multiples of 8 elements, 16-byte
// aligned base pointers), strides non-negative, and one head's rows addressable with the kernels'
// 32-bit row arithmetic.
ffpa_status_t apply_strides(AttnParams& p, const int64_t* st, const void* q, const void* k, const void* v, const void* o,
                  int nq, int nkv, int d) {
  if (st == nullptr) return FFPA_ERR_INVALID_ARGUMENT;
  for (const void* ptr : {q, k, v, o})
    if ((uintptr_t)ptr % 16 != 0) return FFPA_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < 12; ++i)
    if (st[i] < 0 || st[i] % 8 != 0) return FFPA_ERR_INVALID_ARGUMENT;
  const long long lim = (1LL << 31) - 1;
  // {q, k, v, o}: rows per head and the row/head strides must fit the int fields; the last row of a
  // head must end below 2^31 bytes from the head's first row.
  const int rows[4] = {nq, nkv, nkv, nq};
  for (int t = 0; t < 4; ++t) {
    const long long hs = st[3 * t + 1], rs = st[3 * t + 2];
    if (hs > lim || rs > lim) return FFPA_ERR_INVALID_ARGUMENT;
    if (((long long)(rows[t] - 1) * rs + d) * 2 > lim) return FFPA_ERR_INVALID_ARGUMENT;
  }
  p.q_batch = st[0];
  p.q_head = (int)st[1];
  p.q_row = (int)st[2];
  p.k_batch = st[3];
  p.k_head = (int)st[4];
  p.k_row = (int)st[5];
  p.v_batch = st[6];
  p.v_head = (int)st[7];
  p.v_row = (int)st[8];
  p.o_batch = st[9];
  p.o_head = (int)st[10];
  p.o_row = (int)st[11];
  return FFPA_OK;
}

// attn_mask arguments: kind 1 additive (2-byte elements), 2 boolean (1 byte); strides[4] =
// (batch, head, query, key) in elements, non-negative, key stride 0 or 1; with a contiguous key
// dim the other strides are multiples of 8 and the pointer is 16-byte (additive) or 8-byte
// (boolean) aligned, so that 8 keys are one aligned load.
ffpa_status_t apply_mask(AttnParams& p, const void* mask, int kind, const int64_t* st, float scale) {
  if (mask == nullptr || st == nullptr || (kind != FFPA_MASK_ADDITIVE && kind != FFPA_MASK_BOOL))
    return FFPA_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < 4; ++i)
    if (st[i] < 0) return FFPA_ERR_INVALID_ARGUMENT;
  if (st[3] != 0 && st[3] != 1) return FFPA_ERR_INVALID_ARGUMENT;
  if (st[3] == 1) {
    if (st[0] % 8 != 0 || st[1] % 8 != 0 || st[2] % 8 != 0) return FFPA_ERR_INVALID_ARGUMENT;
    if ((uintptr_t)mask % (kind == FFPA_MASK_ADDITIVE ? 16 : 8) != 0) return FFPA_ERR_INVALID_ARGUMENT;
  }
  if (st[2] > (1LL << 31) - 1) return FFPA_ERR_INVALID_ARGUMENT;
  p.mask = mask;
  p.mask_kind = kind;
  p.m_batch = st[0];
  p.m_head = st[1];
  p.m_row = (int)st[2];
  p.m_key = (int)st[3];
  p.inv_scale = 1.0f / scale;
  return FFPA_OK;
}

// Split-KV decode geometry: rows = G * nq rows per KV head in blocks of 32, and the key ranges.
// About two workgroups per compute unit (256 CUs), at least four 32-key tiles per range, at most
// 256 ranges; the tile count per range is then evened out so that no range is empty.
struct DecodeGeom {
  int rows, nrb, nsplit, split_tiles;
};

DecodeGeom decode_geom(int batch, int hq, int hkv, int nq, int nkv) {
  DecodeGeom g{};
  g.rows = (hq / hkv) * nq;
  g.nrb = (g.rows + 31) / 32;
  const long long ntk = ((long long)nkv + 31) / 32;
  const long long base = (long long)batch * hkv * g.nrb;
  long long want = (512 + base - 1) / base;
  const long long cap = std::max(1LL, std::min(256LL, ntk / 4));
  want = std::max(1LL, std::min(want, cap));
  g.split_tiles = (int)((ntk + want - 1) / want);
  g.nsplit = (int)((ntk + g.split_tiles - 1) / g.split_tiles);
  return g;
}

// Workspace of the decode path: per (b, h, query, range) a normalised fp32 O row, then the LSEs.
size_t decode_ws_bytes(int batch, int hq, int hkv, int nq, int nkv, int d) {
  if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || nq < 1 || nkv < 1 || d < 1) return 0;
  const DecodeGeom g = decode_geom(batch, hq, hkv, nq, nkv);
  return (size_t)batch * hq * nq * g.nsplit * ((size_t)d + 1) * 4;
}

// Attach a caller workspace for dS and P. NULL selects the recomputing dV and dQ kernels; a
// workspace smaller than `need` is an invalid argument; need == 0 (not available for these sizes)
// ignores it.
ffpa_status_t attach_ds(AttnParams& p, void* ws, size_t ws_bytes, size_t need) {
  if (ws == nullptr || need == 0) return FFPA_OK;
  if (ws_bytes < need) return FFPA_ERR_INVALID_ARGUMENT;
  p.ds = ws;
  p.pst = (char*)ws + need / 2;
  return FFPA_OK;
}

}  // namespace

extern "C" {

static ffpa_status_t dense_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int hq, int hkv,
                     int nq, int nkv, int d, const int64_t* strides, int dtype, float scale, int causal,
                     hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FFPA_ERR_INVALID_ARGUMENT;
  if (batch < 1 || nq < 1 || nkv < 1) return FFPA_ERR_INVALID_ARGUMENT;
  const ffpa_status_t st = check_common(hq, hkv, d, dtype, scale, causal);
  if (st != FFPA_OK) return st;
  if (too_big_dense(batch, hq, nq, d) || too_big_dense(batch, hkv, nkv, d)) return FFPA_ERR_INVALID_ARGUMENT;
  AttnParams p = dense_params(batch, hq, hkv, nq, nkv, d, scale, causal);
  if (strides != nullptr) {
    const ffpa_status_t sst = apply_strides(p, strides, q, k, v, o, nq, nkv, d);
    if (sst != FFPA_OK) return sst;
  }
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  return to_status(ffpa::launch_fwd(p, dtype == FFPA_DTYPE_FP16, stream));
}

ffpa_status_t ffpa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int hq, int hkv,
             int nq, int nkv, int d, ffpa_dtype_t dtype, float scale, int causal, hipStream_t stream) {
  return dense_fwd(q, k, v, o, lse, batch, hq, hkv, nq, nkv, d, nullptr, dtype, scale, causal, stream);
}

// Workspace of the key-range split forward: per row and range a normalised fp32 O and a log2 LSE;
// 0 when the grid fills the GPU without a split (or the sizes are invalid).
static size_t fwd_split_ws_bytes(int batch, int hq, int hkv, int nq, int nkv, int d) {
  if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || nq < 1 || nkv < 1 || d < 320 || d > 1024 || d % 32 != 0)
    return 0;
  const int ns = ffpa::fwd_split_count(batch, hq, nq, nkv, d);
  return ns > 1 ? (size_t)batch * hq * nq * ns * ((size_t)d + 1) * 4 : 0;
}

size_t ffpa_fwd_split_workspace_bytes(int batch, int hq, int hkv, int nq, int nkv, int d) {
  return fwd_split_ws_bytes(batch, hq, hkv, nq, nkv, d);
}

ffpa_status_t ffpa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int hq, int hkv,
                   int nq, int nkv, int d, ffpa_dtype_t dtype, float scale, int causal, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  const size_t need = fwd_split_ws_bytes(batch, hq, hkv, nq, nkv, d);
  if (need == 0) return dense_fwd(q, k, v, o, lse, batch, hq, hkv, nq, nkv, d, nullptr, dtype, scale, causal, stream);
  if (!q || !k || !v || !o || !lse || !workspace) return FFPA_ERR_INVALID_ARGUMENT;
  const ffpa_status_t st = check_common(hq, hkv, d, dtype, scale, causal);
  if (st != FFPA_OK) return st;
  if (too_big_dense(batch, hq, nq, d) || too_big_dense(batch, hkv, nkv, d)) return FFPA_ERR_INVALID_ARGUMENT;
  if ((long long)batch * hq * nq > (1LL << 31) - 1) return FFPA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return FFPA_ERR_INVALID_ARGUMENT;
  AttnParams p = dense_params(batch, hq, hkv, nq, nkv, d, scale, causal);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  return to_status(ffpa::launch_fwd_split(p, dtype == FFPA_DTYPE_FP16,
                                          ffpa::fwd_split_count(batch, hq, nq, nkv, d), workspace, stream));
}

ffpa_status_t ffpa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int hq, int hkv,
                    int nq, int nkv, int d, const void* mask, ffpa_mask_kind_t mask_kind, const int64_t* mask_strides,
                    ffpa_dtype_t dtype, float scale, int causal, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FFPA_ERR_INVALID_ARGUMENT;
  if (batch < 1 || nq < 1 || nkv < 1) return FFPA_ERR_INVALID_ARGUMENT;
  const ffpa_status_t st = check_common(hq, hkv, d, dtype, scale, causal);
  if (st != FFPA_OK) return st;
  if (too_big_dense(batch, hq, nq, d) || too_big_dense(batch, hkv, nkv, d)) return FFPA_ERR_INVALID_ARGUMENT;
  AttnParams p = dense_params(batch, hq, hkv, nq, nkv, d, scale, causal);
  const ffpa_status_t ms = apply_mask(p, mask, mask_kind, mask_strides, scale);
  if (ms != FFPA_OK) return ms;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  return to_status(ffpa::launch_fwd(p, dtype == FFPA_DTYPE_FP16, stream));
}

size_t ffpa_fwd_fp8_workspace_bytes(int batch, int hq, int hkv, int nq, int nkv, int d) {
  if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || nq < 1 || nkv < 1 || d < 320 || d > 1024 || d % 32 != 0)
    return 0;
  return ffpa::fp8_workspace_bytes(batch, hq, hkv, nkv, d);
}

ffpa_status_t ffpa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int hq, int hkv,
                 int nq, int nkv, int d, ffpa_dtype_t dtype, float scale, int causal, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return FFPA_ERR_INVALID_ARGUMENT;
  if (batch < 1 || nq < 1 || nkv < 1) return FFPA_ERR_INVALID_ARGUMENT;
  const ffpa_status_t st = check_common(hq, hkv, d, dtype, scale, causal);
  if (st != FFPA_OK) return st;
  // (the quantizing passes put batch x heads in one grid dimension)
  if ((long long)batch * hq > 65535) return FFPA_ERR_NOT_SUPPORTED;
  if (too_big_dense(batch, hq, nq, d) || too_big_dense(batch, hkv, nkv, d)) return FFPA_ERR_INVALID_ARGUMENT;
  // The fp8 copies of one head (K8 rows, V8^T rows of nkv rounded up to 64) use 32-bit offsets.
  if ((long long)(nkv + 63) / 64 * 64 * d > (1LL << 31) - 1) return FFPA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < ffpa::fp8_workspace_bytes(batch, hq, hkv, nkv, d)) return FFPA_ERR_INVALID_ARGUMENT;
  AttnParams p = dense_params(batch, hq, hkv, nq, nkv, d, scale, causal);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  return to_status(ffpa::launch_fwd_fp8(p, dtype == FFPA_DTYPE_FP16, workspace, stream));
}

ffpa_status_t ffpa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int hq, int hkv,
                     int nq, int nkv, int d, const int64_t* strides, ffpa_dtype_t dtype, float scale, int causal,
                     hipStream_t stream) {
  if (strides == nullptr) return FFPA_ERR_INVALID_ARGUMENT;
  return dense_fwd(q, k, v, o, lse, batch, hq, hkv, nq, nkv, d, strides, dtype, scale, causal, stream);
}

ffpa_status_t ffpa_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                    int total_k, int hq, int hkv, int d, ffpa_dtype_t dtype, float scale, int causal, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q) return FFPA_ERR_INVALID_ARGUMENT;
  if (batch < 1 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return FFPA_ERR_INVALID_ARGUMENT;
  if (max_seqlen_q > total_q || max_seqlen_k > total_k) return FFPA_ERR_INVALID_ARGUMENT;
  // Keys share the query offsets: both sides must have the same total.
  if (cu_seqlens_k == nullptr && total_k != total_q) return FFPA_ERR_INVALID_ARGUMENT;
  const ffpa_status_t st = check_common(hq, hkv, d, dtype, scale, causal);
  if (st != FFPA_OK) return st;
  if ((long long)total_q * hq * d > (1LL << 31) - 1 || (long long)total_k * hkv * d > (1LL << 31) - 1)
    return FFPA_ERR_INVALID_ARGUMENT;
  if (total_q == 0 || max_seqlen_q == 0) return FFPA_OK;
  AttnParams p = varlen_params(batch, max_seqlen_q, max_seqlen_k, total_q, hq, hkv, d, scale, causal,
                               cu_seqlens_q, cu_seqlens_k);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  return to_status(ffpa::launch_fwd(p, dtype == FFPA_DTYPE_FP16, stream));
}

static ffpa_status_t dense_bwd(int stage, const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, const float* dlse, float* delta, void* dq, void* dk, void* dv, int batch, int hq, int hkv,
                     int nq, int nkv, int d, int dtype, float scale, int causal, void* workspace,
                     size_t workspace_bytes, hipStream_t stream, const void* mask = nullptr, int mask_kind = 0,
                     const int64_t* mask_strides = nullptr, void* dmask = nullptr) {
  if (stage < -1 || stage > 5) return FFPA_ERR_INVALID_ARGUMENT;
  if (!q || !k || !v || !o || !dout || !lse || !delta || !dq || !dk || !dv) return FFPA_ERR_INVALID_ARGUMENT;
  if (batch < 1 || nq < 1 || nkv < 1) return FFPA_ERR_INVALID_ARGUMENT;
  const ffpa_status_t st = check_common(hq, hkv, d, dtype, scale, causal);
  if (st != FFPA_OK) return st;
  if (too_big_dense(batch, hq, nq, d) || too_big_dense(batch, hkv, nkv, d)) return FFPA_ERR_INVALID_ARGUMENT;
  const long long nrows = (long long)batch * hq * nq;
  if (nrows > (1LL << 31) - 1) return FFPA_ERR_INVALID_ARGUMENT;
  AttnParams p = dense_params(batch, hq, hkv, nq, nkv, d, scale, causal);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o_in = o;
  p.dout = dout;
  p.lse_in = lse;
  p.dlse = dlse;
  p.delta = delta;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  const ffpa_status_t ws = attach_ds(p, workspace, workspace_bytes, dense_ds_bytes(batch, hq, nq, nkv));
  if (ws != FFPA_OK) return ws;
  if (mask != nullptr || mask_kind != 0) {
    const ffpa_status_t ms = apply_mask(p, mask, mask_kind, mask_strides, scale);
    if (ms != FFPA_OK) return ms;
    p.dmask = dmask;
  }
  if (stage == 5 && p.ds == nullptr) return FFPA_ERR_INVALID_ARGUMENT;  // the one-launch products need P and dS
  p.ds_row = (int)round_up8(nq);
  p.ds_head = (long long)nkv * p.ds_row;
  p.ds_batch = (long long)hq * p.ds_head;
  return to_status(ffpa::launch_bwd(p, dtype == FFPA_DTYPE_FP16, (int)nrows, 0, stream, stage));
}

size_t ffpa_bwd_workspace_bytes(int batch, int hq, int nq, int nkv) { return dense_ds_bytes(batch, hq, nq, nkv); }

int ffpa_bwd_fused_products(int batch, int hq, int hkv, int nq, int nkv, int d) {
  if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || nq < 1 || nkv < 1 || d < 320 || d > 1024 || d % 32 != 0)
    return 0;
  if (dense_ds_bytes(batch, hq, nq, nkv) == 0) return 0;
  return ffpa::fused_products(dense_params(batch, hq, hkv, nq, nkv, d, 1.0f, 0)) ? 1 : 0;
}

size_t ffpa_decode_workspace_bytes(int batch, int hq, int hkv, int nq, int nkv, int d) {
  return decode_ws_bytes(batch, hq, hkv, nq, nkv, d);
}

static ffpa_status_t decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int hq, int hkv,
                      int nq, int nkv, int d, const int64_t* strides, int dtype, float scale, int causal,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return FFPA_ERR_INVALID_ARGUMENT;
  if (batch < 1 || nq < 1 || nkv < 1) return FFPA_ERR_INVALID_ARGUMENT;
  const ffpa_status_t st = check_common(hq, hkv, d, dtype, scale, causal);
  if (st != FFPA_OK) return st;
  if (too_big_dense(batch, hq, nq, d) || too_big_dense(batch, hkv, nkv, d)) return FFPA_ERR_INVALID_ARGUMENT;
  if ((long long)batch * hq * nq > (1LL << 31) - 1) return FFPA_ERR_INVALID_ARGUMENT;
  const size_t need = decode_ws_bytes(batch, hq, hkv, nq, nkv, d);
  if (workspace_bytes < need) return FFPA_ERR_INVALID_ARGUMENT;
  AttnParams p = dense_params(batch, hq, hkv, nq, nkv, d, scale, causal);
  if (strides != nullptr) {
    const ffpa_status_t sst = apply_strides(p, strides, q, k, v, o, nq, nkv, d);
    if (sst != FFPA_OK) return sst;
  }
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  const DecodeGeom g = decode_geom(batch, hq, hkv, nq, nkv);
  p.rows = g.rows;
  p.nrb = g.nrb;
  p.nsplit = g.nsplit;
  p.split_tiles = g.split_tiles;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)workspace + (size_t)batch * hq * nq * g.nsplit * d;
  return to_status(ffpa::launch_decode(p, dtype == FFPA_DTYPE_FP16, stream));
}

ffpa_status_t ffpa_decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int hq, int hkv,
                    int nq, int nkv, int d, ffpa_dtype_t dtype, float scale, int causal, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return decode_fwd(q, k, v, o, lse, batch, hq, hkv, nq, nkv, d, nullptr, dtype, scale, causal, workspace,
                    workspace_bytes, stream);
}

ffpa_status_t ffpa_decode_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int hq,
                            int hkv, int nq, int nkv, int d, const int64_t* strides, ffpa_dtype_t dtype, float scale,
                            int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (strides == nullptr) return FFPA_ERR_INVALID_ARGUMENT;
  return decode_fwd(q, k, v, o, lse, batch, hq, hkv, nq, nkv, d, strides, dtype, scale, causal, workspace,
                    workspace_bytes, stream);
}

ffpa_status_t ffpa_decode_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                                      int hq, int hkv, int nq, int nkv, int d, ffpa_dtype_t dtype, float scale,
                                      int causal, hipStream_t stream) {
  // Every argument check of ffpa_decode_fwd first (a stand-in workspace pointer that is never
  // dereferenced), then the size against the fixed scratch; only then the scratch address.
  if (!q || !k || !v || !o || !lse) return FFPA_ERR_INVALID_ARGUMENT;
  if (batch < 1 || nq < 1 || nkv < 1) return FFPA_ERR_INVALID_ARGUMENT;
  const ffpa_status_t st = check_common(hq, hkv, d, dtype, scale, causal);
  if (st != FFPA_OK) return st;
  if (too_big_dense(batch, hq, nq, d) || too_big_dense(batch, hkv, nkv, d)) return FFPA_ERR_INVALID_ARGUMENT;
  if ((long long)batch * hq * nq > (1LL << 31) - 1) return FFPA_ERR_INVALID_ARGUMENT;
  if (decode_ws_bytes(batch, hq, hkv, nq, nkv, d) > FFPA_NOALLOC_SCRATCH_BYTES) return FFPA_ERR_TOO_LARGE;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return FFPA_ERR_HIP;
  return decode_fwd(q, k, v, o, lse, batch, hq, hkv, nq, nkv, d, nullptr, dtype, scale, causal, ws,
                    FFPA_NOALLOC_SCRATCH_BYTES, stream);
}

size_t ffpa_varlen_bwd_workspace_bytes(int hq, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k) {
  return varlen_ds_bytes(hq, total_q, total_k, max_seqlen_q, max_seqlen_k);
}

ffpa_status_t ffpa_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    const float* dlse, float* delta, void* dq, void* dk, void* dv, int batch, int hq, int hkv, int nq, int nkv, int d,
                    const void* mask, ffpa_mask_kind_t mask_kind, const int64_t* mask_strides, void* dmask, ffpa_dtype_t dtype,
                    float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (workspace == nullptr) return FFPA_ERR_INVALID_ARGUMENT;
  if (dense_ds_bytes(batch, hq, nq, nkv) == 0 && batch >= 1 && hq >= 1 && nq >= 1 && nkv >= 1)
    return FFPA_ERR_NOT_SUPPORTED;  // a head's P/dS block is too large for the stored path
  if (dmask != nullptr && mask_kind != FFPA_MASK_ADDITIVE) return FFPA_ERR_INVALID_ARGUMENT;
  return dense_bwd(-1, q, k, v, o, dout, lse, dlse, delta, dq, dk, dv, batch, hq, hkv, nq, nkv, d, dtype, scale,
                   causal, workspace, workspace_bytes, stream, mask, mask_kind, mask_strides, dmask);
}

ffpa_status_t ffpa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             const float* dlse, float* delta, void* dq, void* dk, void* dv, int batch, int hq, int hkv, int nq, int nkv, int d,
             ffpa_dtype_t dtype, float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return dense_bwd(-1, q, k, v, o, dout, lse, dlse, delta, dq, dk, dv, batch, hq, hkv, nq, nkv, d, dtype, scale,
                   causal, workspace, workspace_bytes, stream);
}

ffpa_status_t ffpa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, const float* dlse, float* delta, void* dq, void* dk, void* dv, int batch, int hq, int hkv, int nq,
                   int nkv, int d, ffpa_dtype_t dtype, float scale, int causal, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  if (stage < 0 || stage > 5) return FFPA_ERR_INVALID_ARGUMENT;
  return dense_bwd(stage, q, k, v, o, dout, lse, dlse, delta, dq, dk, dv, batch, hq, hkv, nq, nkv, d, dtype, scale,
                   causal, workspace, workspace_bytes, stream);
}

size_t ffpa_varlen_bwd_workspace_bytes_exact(int hq, int batch, const int32_t* cu_seqlens_q_host,
                                             const int32_t* cu_seqlens_k_host, int total_q, int total_k,
                                             int max_seqlen_q, int max_seqlen_k) {
  return varlen_ds_bytes_exact(hq, batch, cu_seqlens_q_host, cu_seqlens_k_host, total_q, total_k, max_seqlen_q,
                               max_seqlen_k);
}

ffpa_status_t ffpa_varlen_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, const float* dlse, float* delta, void* dq, void* dk, void* dv,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host, int batch,
                              int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int hq, int hkv, int d,
                              ffpa_dtype_t dtype, float scale, int causal, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  if (!q || !k || !v || !o || !dout || !lse || !delta || !dq || !dk || !dv || !cu_seqlens_q)
    return FFPA_ERR_INVALID_ARGUMENT;
  if (batch < 1 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return FFPA_ERR_INVALID_ARGUMENT;
  if (max_seqlen_q > total_q || max_seqlen_k > total_k) return FFPA_ERR_INVALID_ARGUMENT;
  if (cu_seqlens_k == nullptr && total_k != total_q) return FFPA_ERR_INVALID_ARGUMENT;
  if (cu_seqlens_k_host != nullptr && cu_seqlens_q_host == nullptr) return FFPA_ERR_INVALID_ARGUMENT;
  if (cu_seqlens_q_host != nullptr) {
    // Host copies are checked here; the device contents must equal them.
    if (!host_cu_ok(batch, cu_seqlens_q_host, total_q, max_seqlen_q)) return FFPA_ERR_INVALID_ARGUMENT;
    if (!host_cu_ok(batch, cu_seqlens_k_host != nullptr ? cu_seqlens_k_host : cu_seqlens_q_host, total_k,
                    max_seqlen_k))
      return FFPA_ERR_INVALID_ARGUMENT;
  }
  const ffpa_status_t st = check_common(hq, hkv, d, dtype, scale, causal);
  if (st != FFPA_OK) return st;
  if ((long long)total_q * hq * d > (1LL << 31) - 1 || (long long)total_k * hkv * d > (1LL << 31) - 1)
    return FFPA_ERR_INVALID_ARGUMENT;
  if (total_k == 0 || max_seqlen_k == 0) {
    // No keys at all: dK and dV are empty, every query row is empty and gets dQ = 0.
    if (total_q > 0) {
      const hipError_t e = hipMemsetAsync(dq, 0, (size_t)total_q * hq * d * 2, stream);
      if (e != hipSuccess) return FFPA_ERR_HIP;
    }
    return FFPA_OK;
  }
  AttnParams p = varlen_params(batch, max_seqlen_q, max_seqlen_k, total_q, hq, hkv, d, scale, causal,
                               cu_seqlens_q, cu_seqlens_k);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o_in = o;
  p.dout = dout;
  p.lse_in = lse;
  p.dlse = dlse;
  p.delta = delta;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  // With host copies the workspace needs only the exact size of these sequences; the P block
  // then starts at half of that size (both blocks are equal).
  const size_t need = cu_seqlens_q_host != nullptr
                          ? varlen_ds_bytes_exact(hq, batch, cu_seqlens_q_host, cu_seqlens_k_host, total_q, total_k,
                                                  max_seqlen_q, max_seqlen_k)
                          : varlen_ds_bytes(hq, total_q, total_k, max_seqlen_q, max_seqlen_k);
  const ffpa_status_t ws = attach_ds(p, workspace, workspace_bytes, need);
  if (ws != FFPA_OK) return ws;
  return to_status(ffpa::launch_bwd(p, dtype == FFPA_DTYPE_FP16, total_q * hq, total_q, stream, -1));
}

const char* ffpa_status_string(ffpa_status_t status) {
  switch (status) {
    case FFPA_OK: return "FFPA_OK";
    case FFPA_ERR_INVALID_ARGUMENT: return "FFPA_ERR_INVALID_ARGUMENT: invalid argument";
    case FFPA_ERR_NOT_SUPPORTED: return "FFPA_ERR_NOT_SUPPORTED: head dim must be a multiple of 32 in [320, 1024]";
    case FFPA_ERR_HIP: return "FFPA_ERR_HIP: a HIP launch or runtime call failed";
    case FFPA_ERR_TOO_LARGE:
      return "FFPA_ERR_TOO_LARGE: the sizes need more than the fixed decode scratch (use ffpa_decode_fwd with a workspace)";
    default: return "FFPA_ERR_UNKNOWN: unknown status code";
  }
}

}  // extern "C"
