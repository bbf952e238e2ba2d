// C ABI of libsas: argument validation, workspace sizing and kernel dispatch.
// Every entry point validates on the host first and reports argument errors
// before anything is enqueued; kernels are then enqueued on the caller's
// stream.  No exception crosses the ABI; the only mutable state is the
// thread-local error message.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "../../include/sas.h"
#include "sas_internal.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int32_t ok() {
  g_last_error.clear();
  return SAS_OK;
}

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(SAS_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Validate the problem and build the kernel-side shape.
int32_t validate(const sas_problem* p, int32_t sel_cap, bool need_cap, sas::Shape* s) {
  if (p == nullptr) return fail(SAS_E_INVALID, "problem pointer is NULL");
  if (p->batch < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1 || p->seq_len < 1 ||
      p->head_dim < 1 || p->block_size < 1)
    return fail(SAS_E_INVALID, "batch, heads, seq_len, head_dim and block_size must be >= 1");
  if (p->n_q_heads % p->n_kv_heads != 0)
    return fail(SAS_E_INVALID, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                p->n_q_heads, p->n_kv_heads);
  if (p->budget_k < 0) return fail(SAS_E_INVALID, "budget_k must be >= 0 (got %d)", p->budget_k);
  if (p->dtype != SAS_BF16 && p->dtype != SAS_FP32)
    return fail(SAS_E_INVALID, "dtype %d is not a sas_dtype", p->dtype);
  if (p->o_dtype != SAS_BF16 && p->o_dtype != SAS_FP32)
    return fail(SAS_E_INVALID, "o_dtype %d is not a sas_dtype", p->o_dtype);
  if (p->dtype == SAS_FP32 && p->o_dtype != SAS_FP32)
    return fail(SAS_E_INVALID, "o_dtype must be SAS_FP32 when dtype is SAS_FP32");
  if (isnan(p->sm_scale) || isinf(p->sm_scale))
    return fail(SAS_E_INVALID, "sm_scale must be finite");
  if (p->gate_act != SAS_GATE_SOFTMAX && p->gate_act != SAS_GATE_SIGMOID &&
      p->gate_act != SAS_GATE_RAW)
    return fail(SAS_E_INVALID, "gate_act %d is not a sas_gate_act", p->gate_act);
  if (p->gate_pos != SAS_GATE_INNER && p->gate_pos != SAS_GATE_OUTER)
    return fail(SAS_E_INVALID, "gate_pos %d is not a sas_gate_pos", p->gate_pos);
  if (p->n_score_heads != 0 && p->n_score_heads != p->n_kv_heads &&
      p->n_score_heads != p->n_q_heads)
    return fail(SAS_E_INVALID, "n_score_heads %d must be 0, n_kv_heads or n_q_heads",
                p->n_score_heads);
  if (p->cu_seqlens != nullptr) {
    if (p->seq_lens != nullptr)
      return fail(SAS_E_INVALID, "seq_lens and cu_seqlens are exclusive (packed batches take "
                  "their lengths from cu_seqlens)");
    if (p->total_tokens < 1 || p->total_tokens > (long long)p->batch * p->seq_len)
      return fail(SAS_E_INVALID, "total_tokens %lld must lie in [1, batch * seq_len = %lld]",
                  (long long)p->total_tokens, (long long)p->batch * p->seq_len);
  }
  if (p->gate_rank != SAS_GATE_SOFT && p->gate_rank != SAS_GATE_HARD_STE)
    return fail(SAS_E_INVALID, "gate_rank %d is not a sas_gate_rank", p->gate_rank);
  if (p->gate_rank == SAS_GATE_HARD_STE &&
      (p->gate_act != SAS_GATE_SOFTMAX || p->gate_pos != SAS_GATE_INNER))
    return fail(SAS_E_UNSUPPORTED, "hard Top-K gates need the softmax activation and the "
                "inner gate position");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SAS_E_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", p->head_dim);
  if (p->block_size != 16 && p->block_size != 32 && p->block_size != 64)
    return fail(SAS_E_UNSUPPORTED, "block_size %d unsupported (16, 32 or 64)", p->block_size);
  if (p->seq_len % p->block_size != 0)
    return fail(SAS_E_UNSUPPORTED, "seq_len %d is not a multiple of block_size %d (ragged "
                "blocks are not supported)", p->seq_len, p->block_size);
  const int C = p->seq_len / p->block_size;
  if (C > 8192) return fail(SAS_E_UNSUPPORTED, "%d blocks per sequence exceeds 8192", C);
  if ((long long)p->batch * p->n_q_heads > 65535)
    return fail(SAS_E_UNSUPPORTED, "batch * n_q_heads exceeds 65535");
  if (need_cap) {
    const int need = p->budget_k < C - 1 ? p->budget_k : C - 1;
    if (sel_cap < 1 || sel_cap < need)
      return fail(SAS_E_INVALID, "sel_cap %d is smaller than min(budget_k, C-1) = %d (and "
                  "must be >= 1)", sel_cap, need);
  }
  s->B = p->batch;
  s->Hq = p->n_q_heads;
  s->Hkv = p->n_kv_heads;
  s->G = p->n_q_heads / p->n_kv_heads;
  s->N = p->seq_len;
  s->D = p->head_dim;
  s->blk = p->block_size;
  s->C = C;
  s->K = p->budget_k;
  s->cap = sel_cap;
  s->fp32 = p->dtype == SAS_FP32;
  s->o_fp32 = p->o_dtype == SAS_FP32;
  s->scale = p->sm_scale > 0.0f ? p->sm_scale : 1.0f / sqrtf((float)p->head_dim);
  s->act = p->gate_act;
  s->outer = p->gate_pos == SAS_GATE_OUTER;
  s->hard = p->gate_rank == SAS_GATE_HARD_STE;
  s->Hs = p->n_score_heads == 0 ? p->n_kv_heads : p->n_score_heads;
  s->lens = p->seq_lens;
  s->cu = p->cu_seqlens;
  s->T = p->cu_seqlens != nullptr ? (long long)p->total_tokens : 0;
  return SAS_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace sas {

bool mfma_path(const Shape& s) {
  return !s.fp32 && s.D == 128 && s.blk == 64;
}

BwdWorkspace bwd_workspace_layout(const Shape& s) {
  BwdWorkspace w{};
  const long long nrow = (long long)s.B * s.Hs * s.C;   // gate-table rows
  const long long ncol = (long long)s.B * s.Hkv * s.C;  // key-major columns
  const int nsh = s.Hs / s.Hkv;                         // score heads per kv head
  // largest possible number of (row, selected block) entries
  long long per_seq = 0;
  for (int i = 0; i < s.C; ++i) per_seq += (i < s.cap ? i : s.cap);
  const long long emax = per_seq * s.B * s.Hs;
  w.words = (int)(((long long)s.C * nsh + 31) / 32);   // a column's bits: (query block, score head)
  size_t off = 0;
  w.delta = off;    off = align256(off + sizeof(float) * (size_t)s.B * s.Hq * s.N);
  if (mfma_path(s)) {
    w.lsen = off;     off = align256(off + sizeof(float) * (size_t)s.B * s.Hq * s.N);
    w.colmask = off;  off = align256(off + sizeof(uint32_t) * (size_t)ncol * w.words);
    w.collen = off;   off = align256(off + sizeof(int32_t) * (size_t)ncol);
    w.coloff = off;   off = align256(off + sizeof(int32_t) * (size_t)(ncol + 1));
    w.chunkoff = off; off = align256(off + sizeof(int32_t) * (size_t)(ncol + 1));
    w.collist = off;  off = align256(off + sizeof(int32_t) * (size_t)(emax + nrow));
    // chunks of at most cc entries: sum over columns of ceil(L / cc) with
    // sum L = emax + nrow (each column also holds one diagonal entry per
    // score head)
    const int cc = col_chunk(s);
    w.max_chunks = (emax + nrow + (long long)ncol * (cc - 1)) / cc;
    w.partial = off;  off = align256(off + sizeof(float) * 2 * 64 * 128 * (size_t)w.max_chunks);
    w.chunk_rank = off;  off = align256(off + sizeof(int32_t) * (size_t)w.max_chunks);
    w.chunk_hist = off;  off = align256(off + sizeof(int32_t) * (size_t)(ncol + 1));
    w.chunk_desc = off; off = align256(off + 4 * sizeof(int32_t) * (size_t)w.max_chunks);
  }
  w.total = off;
  return w;
}

}  // namespace sas

extern "C" {

int32_t sas_abi_version(void) { return SAS_ABI_VERSION; }

const char* sas_last_error(void) { return g_last_error.c_str(); }

int32_t sas_gate_threshold(const sas_problem* p, const float* scores, float* log_gate, float* tau,
                           int32_t* sel_idx, int32_t* sel_cnt, int32_t sel_cap, int32_t* d_status,
                           void* stream) {
  sas::Shape s;
  int32_t rc = validate(p, sel_cap, true, &s);
  if (rc != SAS_OK) return rc;
  if (!scores || !log_gate || !tau || !sel_idx || !sel_cnt)
    return fail(SAS_E_INVALID, "sas_gate_threshold: a required pointer is NULL");
  hipError_t e = sas::launch_threshold(s, scores, log_gate, tau, sel_idx, sel_cnt, d_status,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sas_gate_threshold launch");
  return ok();
}

int32_t sas_gated_attn_fwd(const sas_problem* p, const void* q, const void* k, const void* v,
                           const float* log_gate, const int32_t* sel_idx, const int32_t* sel_cnt,
                           int32_t sel_cap, void* o, float* lse, void* stream) {
  sas::Shape s;
  int32_t rc = validate(p, sel_cap, true, &s);
  if (rc != SAS_OK) return rc;
  if (!q || !k || !v || !log_gate || !sel_idx || !sel_cnt || !o || !lse)
    return fail(SAS_E_INVALID, "sas_gated_attn_fwd: a required pointer is NULL");
  hipError_t e = sas::mfma_path(s)
                     ? sas::launch_fwd_mfma(s, q, k, v, log_gate, sel_idx, sel_cnt, o, lse,
                                            (hipStream_t)stream)
                     : sas::launch_fwd_generic(s, q, k, v, log_gate, sel_idx, sel_cnt, o, lse,
                                               (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sas_gated_attn_fwd launch");
  return ok();
}

size_t sas_gated_attn_bwd_workspace_size(const sas_problem* p, int32_t sel_cap) {
  sas::Shape s;
  if (validate(p, sel_cap, true, &s) != SAS_OK) return 0;
  g_last_error.clear();
  return sas::bwd_workspace_layout(s).total;
}

}  // extern "C"

namespace {

enum BwdStage { kStageDq = 1, kStageDkdv = 2 };

int32_t run_bwd(const char* name, int stages, const sas_problem* p, const sas::BwdPtrs& ptr,
                int32_t sel_cap, void* workspace, size_t workspace_bytes, void* stream) {
  sas::Shape s;
  int32_t rc = validate(p, sel_cap, true, &s);
  if (rc != SAS_OK) return rc;
  bool missing = !ptr.q || !ptr.k || !ptr.v || !ptr.d_o || !ptr.lse || !ptr.log_gate ||
                 !ptr.sel_idx || !ptr.sel_cnt;
  if (stages & kStageDq) missing = missing || !ptr.o || !ptr.dq;
  if (stages & kStageDkdv) missing = missing || !ptr.dk || !ptr.dv || !ptr.dlog_gate;
  if (missing) return fail(SAS_E_INVALID, "%s: a required pointer is NULL", name);
  const sas::BwdWorkspace wl = sas::bwd_workspace_layout(s);
  if (workspace == nullptr || workspace_bytes < wl.total)
    return fail(SAS_E_WORKSPACE, "%s: workspace of %zu bytes given, %zu required", name,
                workspace == nullptr ? (size_t)0 : workspace_bytes, wl.total);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(SAS_E_WORKSPACE, "%s: workspace must be 256-byte aligned", name);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const bool mf = sas::mfma_path(s);
  hipError_t e = hipSuccess;
  if (stages & kStageDq)
    e = mf ? sas::launch_bwd_dq_mfma(s, ptr, ws, wl, st)
           : sas::launch_bwd_dq_generic(s, ptr, ws, wl, st);
  if (e == hipSuccess && (stages & kStageDkdv))
    e = mf ? sas::launch_bwd_dkdv_mfma(s, ptr, ws, wl, st)
           : sas::launch_bwd_dkdv_generic(s, ptr, ws, wl, st);
  if (e != hipSuccess) return hip_fail(e, name);
  return ok();
}

}  // namespace

extern "C" {

int32_t sas_gated_attn_bwd(const sas_problem* p, const void* q, const void* k, const void* v,
                           const void* o, const void* d_o, const float* lse, const float* log_gate,
                           const int32_t* sel_idx, const int32_t* sel_cnt, int32_t sel_cap,
                           void* dq, void* dk, void* dv, float* dlog_gate, float* dscores,
                           void* workspace, size_t workspace_bytes, void* stream) {
  const sas::BwdPtrs ptr{q, k, v, o, d_o, lse, log_gate, sel_idx, sel_cnt,
                         dq, dk, dv, dlog_gate, dscores};
  return run_bwd("sas_gated_attn_bwd", kStageDq | kStageDkdv, p, ptr, sel_cap, workspace,
                 workspace_bytes, stream);
}

int32_t sas_gated_attn_bwd_dq(const sas_problem* p, const void* q, const void* k, const void* v,
                              const void* o, const void* d_o, const float* lse,
                              const float* log_gate, const int32_t* sel_idx,
                              const int32_t* sel_cnt, int32_t sel_cap, void* dq, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const sas::BwdPtrs ptr{q, k, v, o, d_o, lse, log_gate, sel_idx, sel_cnt,
                         dq, nullptr, nullptr, nullptr, nullptr};
  return run_bwd("sas_gated_attn_bwd_dq", kStageDq, p, ptr, sel_cap, workspace, workspace_bytes,
                 stream);
}

int32_t sas_gated_attn_bwd_dkdv(const sas_problem* p, const void* q, const void* k,
                                const void* v, const void* d_o, const float* lse,
                                const float* log_gate, const int32_t* sel_idx,
                                const int32_t* sel_cnt, int32_t sel_cap, void* dk, void* dv,
                                float* dlog_gate, float* dscores, void* workspace,
                                size_t workspace_bytes, void* stream) {
  const sas::BwdPtrs ptr{q, k, v, nullptr, d_o, lse, log_gate, sel_idx, sel_cnt,
                         nullptr, dk, dv, dlog_gate, dscores};
  return run_bwd("sas_gated_attn_bwd_dkdv", kStageDkdv, p, ptr, sel_cap, workspace,
                 workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// sparse decode
// ---------------------------------------------------------------------------
namespace {

int32_t validate_decode(const sas_decode_problem* p, int32_t sel_cap, sas::DecodeShape* s) {
  if (p == nullptr) return fail(SAS_E_INVALID, "decode problem pointer is NULL");
  if (p->batch < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1 || p->head_dim < 1 ||
      p->block_size < 1 || p->max_blocks < 1 || p->pool_blocks < 1)
    return fail(SAS_E_INVALID, "batch, heads, head_dim, block_size, max_blocks and pool_blocks "
                "must be >= 1");
  if (p->n_q_heads % p->n_kv_heads != 0)
    return fail(SAS_E_INVALID, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                p->n_q_heads, p->n_kv_heads);
  if (p->budget_k < 0) return fail(SAS_E_INVALID, "budget_k must be >= 0 (got %d)", p->budget_k);
  if (p->dtype != SAS_BF16 && p->dtype != SAS_FP32)
    return fail(SAS_E_INVALID, "dtype %d is not a sas_dtype", p->dtype);
  if (isnan(p->sm_scale) || isinf(p->sm_scale))
    return fail(SAS_E_INVALID, "sm_scale must be finite");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SAS_E_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", p->head_dim);
  if (p->block_size != 16 && p->block_size != 32 && p->block_size != 64)
    return fail(SAS_E_UNSUPPORTED, "block_size %d unsupported (16, 32 or 64)", p->block_size);
  if (p->max_blocks > 16384)
    return fail(SAS_E_UNSUPPORTED, "max_blocks %d exceeds 16384", p->max_blocks);
  if ((long long)p->max_blocks * p->block_size > 0x7fffffffLL)
    return fail(SAS_E_UNSUPPORTED, "max_blocks * block_size overflows int32");
  const int G = p->n_q_heads / p->n_kv_heads;
  if (G > 64) return fail(SAS_E_UNSUPPORTED, "more than 64 query heads per kv head");
  if ((long long)p->batch * p->n_q_heads > 0x7fffffffLL / 128)
    return fail(SAS_E_UNSUPPORTED, "batch * n_q_heads too large");
  const int need = p->budget_k < p->max_blocks - 1 ? p->budget_k : p->max_blocks - 1;
  if (sel_cap < 1 || sel_cap < need || sel_cap > 65534)
    return fail(SAS_E_INVALID, "sel_cap %d must lie in [max(1, min(budget_k, max_blocks-1)) = %d, "
                "65534]", sel_cap, need < 1 ? 1 : need);
  s->B = p->batch;
  s->Hq = p->n_q_heads;
  s->Hkv = p->n_kv_heads;
  s->G = G;
  s->D = p->head_dim;
  s->blk = p->block_size;
  s->cmax = p->max_blocks;
  s->pool = p->pool_blocks;
  s->K = p->budget_k;
  s->cap = sel_cap;
  s->fp32 = p->dtype == SAS_FP32;
  s->scale = p->sm_scale > 0.0f ? p->sm_scale : 1.0f / sqrtf((float)p->head_dim);
  return SAS_OK;
}

size_t decode_ws_bytes(const sas::DecodeShape& s) {
  return align256(sizeof(float) * (size_t)s.B * s.Hkv * (s.cap + 1) * s.G * (s.D + 2));
}

}  // namespace

extern "C" {

int32_t sas_decode_select(const sas_decode_problem* p, const float* scores,
                          const int32_t* seq_lens, float* tau, int32_t* sel_idx, int32_t* sel_cnt,
                          int32_t sel_cap, int32_t* d_status, void* stream) {
  sas::DecodeShape s;
  int32_t rc = validate_decode(p, sel_cap, &s);
  if (rc != SAS_OK) return rc;
  if (!scores || !seq_lens || !sel_idx || !sel_cnt)
    return fail(SAS_E_INVALID, "sas_decode_select: a required pointer is NULL");
  hipError_t e = sas::launch_decode_select(s, scores, seq_lens, tau, sel_idx, sel_cnt, d_status,
                                           (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sas_decode_select launch");
  return ok();
}

size_t sas_decode_workspace_size(const sas_decode_problem* p, int32_t sel_cap) {
  sas::DecodeShape s;
  if (validate_decode(p, sel_cap, &s) != SAS_OK) return 0;
  g_last_error.clear();
  return decode_ws_bytes(s);
}

int32_t sas_decode_attn(const sas_decode_problem* p, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* sel_idx, const int32_t* sel_cnt, int32_t sel_cap, void* o,
                        float* lse, void* workspace, size_t workspace_bytes, int32_t* d_status,
                        void* stream) {
  sas::DecodeShape s;
  int32_t rc = validate_decode(p, sel_cap, &s);
  if (rc != SAS_OK) return rc;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !sel_idx || !sel_cnt || !o || !lse)
    return fail(SAS_E_INVALID, "sas_decode_attn: a required pointer is NULL");
  const size_t need = decode_ws_bytes(s);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SAS_E_WORKSPACE, "sas_decode_attn: workspace of %zu bytes given, %zu required",
                workspace == nullptr ? (size_t)0 : workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(SAS_E_WORKSPACE, "sas_decode_attn: workspace must be 256-byte aligned");
  if (sas::decode_attn_lds_bytes(s) > 160 * 1024)
    return fail(SAS_E_UNSUPPORTED, "sas_decode_attn: too many query heads per kv head");
  hipError_t e = sas::launch_decode_attn(s, q, k_pool, v_pool, block_table, seq_lens, sel_idx,
                                         sel_cnt, o, lse, (float*)workspace, d_status,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sas_decode_attn launch");
  return ok();
}

int32_t sas_decode_attn_noalloc(const sas_decode_problem* p, const void* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* sel_idx,
                                const int32_t* sel_cnt, int32_t sel_cap, void* o, float* lse,
                                int32_t* d_status, void* stream) {
  sas::DecodeShape s;
  int32_t rc = validate_decode(p, sel_cap, &s);
  if (rc != SAS_OK) return rc;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !sel_idx || !sel_cnt || !o || !lse)
    return fail(SAS_E_INVALID, "sas_decode_attn_noalloc: a required pointer is NULL");
  const size_t need = decode_ws_bytes(s);
  if (need > sas::kDecodeScratchBytes)
    return fail(SAS_E_WORKSPACE, "sas_decode_attn_noalloc: the problem needs %zu bytes of scratch "
                "(batch * n_kv_heads * (sel_cap + 1) * G * (head_dim + 2) floats); the fixed "
                "scratch holds %zu", need, sas::kDecodeScratchBytes);
  if (sas::decode_attn_lds_bytes(s) > 160 * 1024)
    return fail(SAS_E_UNSUPPORTED, "sas_decode_attn_noalloc: too many query heads per kv head");
  void* scratch = nullptr;
  hipError_t e = sas::decode_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "sas_decode_attn_noalloc scratch lookup");
  e = sas::launch_decode_attn(s, q, k_pool, v_pool, block_table, seq_lens, sel_idx, sel_cnt, o,
                              lse, (float*)scratch, d_status, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sas_decode_attn_noalloc launch");
  return ok();
}

}  // extern "C"
