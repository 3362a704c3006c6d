// C ABI of libmsa (declared in include/msa.h): argument validation, dispatch
// to the gfx950 kernels, host-side schedule introspection, error reporting.
// No entry point allocates device memory or keeps state between calls.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <limits>
#include <string>

#include "msa_internal.hpp"
#include "msa_plan.hpp"

namespace {

thread_local std::string g_last_error;

msa_status fail(msa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

msa_status fail(msa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

msa_status ok() {
  g_last_error.clear();
  return MSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

msa_status check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(MSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(MSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MSA_OK;
}

msa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MSA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// Shape checks shared by pooling, prefill and the prefill plan queries.
msa_status check_attn_shape(const msa_attn_desc* d, bool need_heads_q) {
  if (d == nullptr) return fail(MSA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 0 || d->seq_len < 0 || d->heads_kv < 1)
    return fail(MSA_ERR_INVALID_ARG, "batch=%d seq_len=%d heads_kv=%d: need batch>=0, seq_len>=0, heads_kv>=1",
                d->batch, d->seq_len, d->heads_kv);
  if (need_heads_q && (d->heads_q < 1 || d->heads_q % d->heads_kv != 0))
    return fail(MSA_ERR_INVALID_ARG, "heads_q=%d must be a positive multiple of heads_kv=%d", d->heads_q,
                d->heads_kv);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(MSA_ERR_UNSUPPORTED, "head_dim=%d: supported values are 64 and 128", d->head_dim);
  if (d->in_dtype != MSA_DTYPE_F32 && d->in_dtype != MSA_DTYPE_BF16)
    return fail(MSA_ERR_INVALID_ARG, "in_dtype=%d is not a msa_dtype", d->in_dtype);
  if (d->num_landmarks < 0) return fail(MSA_ERR_INVALID_ARG, "num_landmarks=%d < 0", d->num_landmarks);
  if (d->num_landmarks > 0 && d->seq_len % d->num_landmarks != 0)
    return fail(MSA_ERR_INVALID_ARG, "num_landmarks=%d does not divide seq_len=%d", d->num_landmarks,
                d->seq_len);
  return MSA_OK;
}

msa_status check_attn(const msa_attn_desc* d) {
  msa_status s = check_attn_shape(d, true);
  if (s != MSA_OK) return s;
  if (d->window < 1) return fail(MSA_ERR_INVALID_ARG, "window=%d must be >= 1", d->window);
  if (d->window > (1 << 30)) return fail(MSA_ERR_INVALID_ARG, "window=%d too large (max 2^30)", d->window);
  if (!isfinite(d->scale) || !(d->scale > 0.f))
    return fail(MSA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (d->out_dtype != MSA_DTYPE_F32 && d->out_dtype != MSA_DTYPE_BF16)
    return fail(MSA_ERR_INVALID_ARG, "out_dtype=%d is not a msa_dtype", d->out_dtype);
  if (d->in_dtype == MSA_DTYPE_F32 && d->out_dtype != MSA_DTYPE_F32)
    return fail(MSA_ERR_UNSUPPORTED, "float32 inputs write float32 output only");
  const long long wgs = (long long)d->batch * d->heads_q * ((d->seq_len + 63) / 64);
  if (wgs > (1LL << 31) - 1) return fail(MSA_ERR_UNSUPPORTED, "problem too large for one launch");
  if (d->in_dtype == MSA_DTYPE_BF16 && (long long)d->seq_len * d->head_dim * 2 >= (1LL << 31))
    return fail(MSA_ERR_UNSUPPORTED, "seq_len=%d: one head's K or V must be < 2 GiB", d->seq_len);
  return MSA_OK;
}

msa_status check_decode_shape(const msa_decode_desc* d) {
  if (d == nullptr) return fail(MSA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 0 || d->ctx_len < 1 || d->heads_kv < 1 || d->heads_q < 1 || d->heads_q % d->heads_kv != 0)
    return fail(MSA_ERR_INVALID_ARG,
                "batch=%d ctx_len=%d heads_q=%d heads_kv=%d: need batch>=0, ctx_len>=1, heads_q a multiple of heads_kv",
                d->batch, d->ctx_len, d->heads_q, d->heads_kv);
  if (d->heads_q / d->heads_kv > 16)
    return fail(MSA_ERR_UNSUPPORTED, "heads_q/heads_kv=%d: at most 16 query heads per KV head",
                d->heads_q / d->heads_kv);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(MSA_ERR_UNSUPPORTED, "head_dim=%d: supported values are 64 and 128", d->head_dim);
  if (d->window < 1 || d->window > (1 << 30)) return fail(MSA_ERR_INVALID_ARG, "window=%d out of range", d->window);
  if (d->num_landmarks < 0 || (d->num_landmarks > 0 && d->ctx_len % d->num_landmarks != 0))
    return fail(MSA_ERR_INVALID_ARG, "num_landmarks=%d must be >= 0 and divide ctx_len=%d", d->num_landmarks,
                d->ctx_len);
  if (d->num_splits < 1) return fail(MSA_ERR_INVALID_ARG, "num_splits=%d must be >= 1", d->num_splits);
  if (d->schedule != MSA_DECODE_AUTO && d->schedule != MSA_DECODE_SPLIT && d->schedule != MSA_DECODE_FUSED)
    return fail(MSA_ERR_INVALID_ARG, "schedule=%d is not a msa_decode_schedule", d->schedule);
  if (!isfinite(d->scale) || !(d->scale > 0.f))
    return fail(MSA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (d->in_dtype != MSA_DTYPE_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "decode reads bf16 caches only (in_dtype=%d)", d->in_dtype);
  if (d->out_dtype != MSA_DTYPE_F32 && d->out_dtype != MSA_DTYPE_BF16)
    return fail(MSA_ERR_INVALID_ARG, "out_dtype=%d is not a msa_dtype", d->out_dtype);
  const long long wgs = (long long)d->batch * d->heads_kv * d->num_splits;
  if (wgs > (1LL << 31) - 1) return fail(MSA_ERR_UNSUPPORTED, "problem too large for one launch");
  return MSA_OK;
}

// Contiguous caches additionally keep one head's cache under 2 GiB.
msa_status check_decode(const msa_decode_desc* d) {
  msa_status s = check_decode_shape(d);
  if (s != MSA_OK) return s;
  if ((long long)d->ctx_len * d->head_dim * 2 >= (1LL << 31))
    return fail(MSA_ERR_UNSUPPORTED, "ctx_len=%d: one head's cache must be < 2 GiB", d->ctx_len);
  return MSA_OK;
}

// Shape checks of the append entry points (the caches' layout is checked
// by each caller).
msa_status check_append_shape(const msa_decode_desc* desc) {
  if (desc == nullptr) return fail(MSA_ERR_INVALID_ARG, "desc is NULL");
  if (desc->batch < 0 || desc->ctx_len < 1 || desc->heads_kv < 1)
    return fail(MSA_ERR_INVALID_ARG, "batch=%d ctx_len=%d heads_kv=%d: need batch>=0, ctx_len>=1, heads_kv>=1",
                desc->batch, desc->ctx_len, desc->heads_kv);
  if (desc->head_dim != 64 && desc->head_dim != 128)
    return fail(MSA_ERR_UNSUPPORTED, "head_dim=%d: supported values are 64 and 128", desc->head_dim);
  if (desc->num_landmarks < 0 || (desc->num_landmarks > 0 && desc->ctx_len % desc->num_landmarks != 0))
    return fail(MSA_ERR_INVALID_ARG, "num_landmarks=%d must be >= 0 and divide ctx_len=%d", desc->num_landmarks,
                desc->ctx_len);
  if (desc->in_dtype != MSA_DTYPE_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "the cache is bf16 only (in_dtype=%d)", desc->in_dtype);
  if (2LL * desc->batch * desc->heads_kv > (1LL << 31) - 1)
    return fail(MSA_ERR_UNSUPPORTED, "problem too large for one launch");
  return MSA_OK;
}

// Paging arguments shared by the paged entry points.
msa_status check_paging(const msa_decode_desc* d, int32_t page_size, int32_t num_pages, const int32_t* table,
                        msa::DecodePaging* out) {
  if (page_size < 32 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
    return fail(MSA_ERR_INVALID_ARG, "page_size=%d must be a power of two in [32, 2^20]", page_size);
  if (d->ctx_len % page_size != 0)
    return fail(MSA_ERR_INVALID_ARG, "ctx_len=%d (the capacity) must be a multiple of page_size=%d", d->ctx_len,
                page_size);
  if (num_pages < 1) return fail(MSA_ERR_INVALID_ARG, "num_pages=%d must be >= 1", num_pages);
  if (table == nullptr || (reinterpret_cast<uintptr_t>(table) & 3u) != 0)
    return fail(MSA_ERR_INVALID_ARG, "block_table is NULL or not 4-byte aligned");
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  *out = msa::DecodePaging{table, shift, d->ctx_len / page_size, num_pages};
  return MSA_OK;
}

msa_status check_bwd(const msa_attn_desc* d) {
  msa_status s = check_attn(d);
  if (s != MSA_OK) return s;
  if (d->in_dtype != MSA_DTYPE_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "the backward takes bf16 inputs only (in_dtype=%d)", d->in_dtype);
  const long long rows = (long long)d->batch * d->heads_q * (((long long)d->seq_len + 127) / 128 * 128);
  if ((rows + 15) / 16 > (1LL << 31) - 1) return fail(MSA_ERR_UNSUPPORTED, "problem too large for one launch");
  return MSA_OK;
}

size_t decode_ws_bytes(const msa_decode_desc* d) {
  return (size_t)d->num_splits * d->batch * d->heads_q * (d->head_dim + 1) * sizeof(float);
}

}  // namespace

extern "C" {

int32_t msa_abi_version(void) { return MSA_ABI_VERSION; }

const char* msa_status_string(msa_status s) {
  switch (s) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported";
    case MSA_ERR_WORKSPACE: return "workspace too small";
    case MSA_ERR_HIP: return "HIP runtime error";
    case MSA_ERR_CAPACITY: return "output capacity too small";
  }
  return "unknown status";
}

const char* msa_last_error(void) { return g_last_error.c_str(); }

msa_status msa_pool_landmarks(const msa_attn_desc* desc, const void* K, const void* V, void* Kbar, void* Vbar,
                              void* stream) {
  msa_status s = check_attn_shape(desc, false);
  if (s != MSA_OK) return s;
  if (desc->num_landmarks == 0 || desc->batch == 0) return ok();
  if ((s = check_ptr(K, "K")) || (s = check_ptr(V, "V")) || (s = check_ptr(Kbar, "Kbar")) ||
      (s = check_ptr(Vbar, "Vbar")))
    return s;
  const long long wgs = 2LL * desc->batch * desc->heads_kv * desc->num_landmarks;
  if (wgs > (1LL << 31) - 1) return fail(MSA_ERR_UNSUPPORTED, "problem too large for one launch");
  return hip_status(msa::launch_pool(*desc, K, V, Kbar, Vbar, static_cast<hipStream_t>(stream)),
                    "pool launch");
}

msa_status msa_attn_fwd(const msa_attn_desc* desc, const void* Q, const void* K, const void* V, const void* Kbar,
                        const void* Vbar, void* O, float* LSE, void* stream) {
  msa_status s = check_attn(desc);
  if (s != MSA_OK) return s;
  if (desc->batch == 0 || desc->seq_len == 0) return ok();
  if ((s = check_ptr(Q, "Q")) || (s = check_ptr(K, "K")) || (s = check_ptr(V, "V")) || (s = check_ptr(O, "O")))
    return s;
  if (desc->num_landmarks > 0 && ((s = check_ptr(Kbar, "Kbar")) || (s = check_ptr(Vbar, "Vbar")))) return s;
  if (LSE != nullptr && !aligned16(LSE)) return fail(MSA_ERR_INVALID_ARG, "LSE is not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = desc->in_dtype == MSA_DTYPE_BF16
                           ? msa::launch_attn_bf16(*desc, Q, K, V, Kbar, Vbar, O, LSE, st)
                           : msa::launch_attn_f32(*desc, Q, K, V, Kbar, Vbar, O, LSE, st);
  return hip_status(e, "attention launch");
}

msa_status msa_attn_fwd_blocksparse(const msa_attn_desc* desc, const int32_t* block_counts,
                                   const int32_t* block_indices, int32_t max_blocks, int32_t causal, const void* Q,
                                   const void* K, const void* V, void* O, float* LSE, void* stream) {
  if (desc == nullptr) return fail(MSA_ERR_INVALID_ARG, "desc is NULL");
  msa_attn_desc d = *desc;
  d.window = 1;         // not read by this entry point
  d.num_landmarks = 0;  // not read by this entry point
  msa_status s = check_attn(&d);
  if (s != MSA_OK) return s;
  if (d.in_dtype != MSA_DTYPE_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "block-sparse lists take bf16 inputs only (in_dtype=%d)", d.in_dtype);
  if (max_blocks < 0) return fail(MSA_ERR_INVALID_ARG, "max_blocks=%d < 0", max_blocks);
  if (causal != 0 && causal != 1) return fail(MSA_ERR_INVALID_ARG, "causal=%d must be 0 or 1", causal);
  if (d.batch == 0 || d.seq_len == 0) return ok();
  if ((s = check_ptr(Q, "Q")) || (s = check_ptr(K, "K")) || (s = check_ptr(V, "V")) || (s = check_ptr(O, "O")))
    return s;
  if (block_counts == nullptr || (reinterpret_cast<uintptr_t>(block_counts) & 3u) != 0)
    return fail(MSA_ERR_INVALID_ARG, "block_counts is NULL or not 4-byte aligned");
  if (max_blocks > 0 && (block_indices == nullptr || (reinterpret_cast<uintptr_t>(block_indices) & 3u) != 0))
    return fail(MSA_ERR_INVALID_ARG, "block_indices is NULL or not 4-byte aligned");
  if (LSE != nullptr && !aligned16(LSE)) return fail(MSA_ERR_INVALID_ARG, "LSE is not 16-byte aligned");
  return hip_status(msa::launch_attn_list_bf16(d, block_counts, block_indices, max_blocks, causal, Q, K, V, O, LSE,
                                               static_cast<hipStream_t>(stream)),
                    "block-sparse attention launch");
}

msa_status msa_attn_bwd_workspace_size(const msa_attn_desc* desc, size_t* bytes) {
  msa_status s = check_bwd(desc);
  if (s != MSA_OK) return s;
  if (bytes == nullptr) return fail(MSA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = msa::bwd_layout(*desc).bytes;
  return ok();
}

msa_status msa_attn_bwd(const msa_attn_desc* desc, const void* Q, const void* K, const void* V, const void* Kbar,
                        const void* Vbar, const void* O, const float* LSE, const void* dO, void* workspace,
                        size_t workspace_bytes, void* dQ, void* dK, void* dV, void* stream) {
  msa_status s = check_bwd(desc);
  if (s != MSA_OK) return s;
  if (desc->batch == 0 || desc->seq_len == 0) return ok();
  if ((s = check_ptr(Q, "Q")) || (s = check_ptr(K, "K")) || (s = check_ptr(V, "V")) || (s = check_ptr(O, "O")) ||
      (s = check_ptr(LSE, "LSE")) || (s = check_ptr(dO, "dO")) || (s = check_ptr(workspace, "workspace")) ||
      (s = check_ptr(dQ, "dQ")) || (s = check_ptr(dK, "dK")) || (s = check_ptr(dV, "dV")))
    return s;
  if (desc->num_landmarks > 0 && ((s = check_ptr(Kbar, "Kbar")) || (s = check_ptr(Vbar, "Vbar")))) return s;
  const size_t need = msa::bwd_layout(*desc).bytes;
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return hip_status(msa::launch_attn_bwd(*desc, Q, K, V, Kbar, Vbar, O, LSE, dO, workspace, dQ, dK, dV,
                                         static_cast<hipStream_t>(stream)),
                    "backward launch");
}

msa_status msa_decode_workspace_size(const msa_decode_desc* desc, size_t* bytes) {
  msa_status s = check_decode_shape(desc);  // the size does not depend on the caches' layout
  if (s != MSA_OK) return s;
  if (bytes == nullptr) return fail(MSA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = decode_ws_bytes(desc);
  return ok();
}

msa_status msa_decode_fwd(const msa_decode_desc* desc, const void* q, const void* Kcache, const void* Vcache,
                          const void* Kbar, const void* Vbar, void* workspace, size_t workspace_bytes, void* O,
                          float* LSE, void* stream) {
  msa_status s = check_decode(desc);
  if (s != MSA_OK) return s;
  if (desc->batch == 0) return ok();
  if ((s = check_ptr(q, "q")) || (s = check_ptr(Kcache, "Kcache")) || (s = check_ptr(Vcache, "Vcache")) ||
      (s = check_ptr(O, "O")) || (s = check_ptr(workspace, "workspace")))
    return s;
  if (desc->num_landmarks > 0 && ((s = check_ptr(Kbar, "Kbar")) || (s = check_ptr(Vbar, "Vbar")))) return s;
  if (LSE != nullptr && !aligned16(LSE)) return fail(MSA_ERR_INVALID_ARG, "LSE is not 16-byte aligned");
  const size_t need = decode_ws_bytes(desc);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  float* ws_o = static_cast<float*>(workspace);
  float* ws_lse = ws_o + (size_t)desc->num_splits * desc->batch * desc->heads_q * desc->head_dim;
  return hip_status(msa::launch_decode(*desc, q, Kcache, Vcache, Kbar, Vbar, nullptr, nullptr, ws_o, ws_lse, O, LSE,
                                       static_cast<hipStream_t>(stream)),
                    "decode launch");
}

msa_status msa_decode_fwd_noalloc(const msa_decode_desc* desc, const void* q, const void* Kcache,
                                  const void* Vcache, const void* Kbar, const void* Vbar, void* O, float* LSE,
                                  void* stream) {
  msa_status s = check_decode(desc);
  if (s != MSA_OK) return s;
  if (desc->batch == 0) return ok();
  if ((s = check_ptr(q, "q")) || (s = check_ptr(Kcache, "Kcache")) || (s = check_ptr(Vcache, "Vcache")) ||
      (s = check_ptr(O, "O")))
    return s;
  if (desc->num_landmarks > 0 && ((s = check_ptr(Kbar, "Kbar")) || (s = check_ptr(Vbar, "Vbar")))) return s;
  if (LSE != nullptr && !aligned16(LSE)) return fail(MSA_ERR_INVALID_ARG, "LSE is not 16-byte aligned");
  const size_t need = decode_ws_bytes(desc);
  if (desc->schedule != MSA_DECODE_FUSED && need > msa::kNoallocScratchBytes && msa::decode_uses_split(*desc))
    return fail(MSA_ERR_WORKSPACE, "the split schedule needs %zu bytes of partials, more than the %zu of the "
                                   "library's array (use msa_decode_fwd with a workspace)",
                need, (size_t)msa::kNoallocScratchBytes);
  float* ws = nullptr;
  hipError_t e = msa::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "scratch address");
  float* ws_lse = ws + (size_t)desc->num_splits * desc->batch * desc->heads_q * desc->head_dim;
  return hip_status(msa::launch_decode(*desc, q, Kcache, Vcache, Kbar, Vbar, nullptr, nullptr, ws, ws_lse, O, LSE,
                                       static_cast<hipStream_t>(stream)),
                    "decode launch");
}

msa_status msa_decode_fwd_varlen(const msa_decode_desc* desc, const int32_t* ctx_lens, const void* q,
                                 const void* Kcache, const void* Vcache, const void* Kbar, const void* Vbar,
                                 void* workspace, size_t workspace_bytes, void* O, float* LSE, void* stream) {
  msa_status s = check_decode(desc);
  if (s != MSA_OK) return s;
  if (desc->batch == 0) return ok();
  if (ctx_lens == nullptr) return fail(MSA_ERR_INVALID_ARG, "ctx_lens is NULL");
  if ((reinterpret_cast<uintptr_t>(ctx_lens) & 3u) != 0)
    return fail(MSA_ERR_INVALID_ARG, "ctx_lens is not 4-byte aligned");
  if ((s = check_ptr(q, "q")) || (s = check_ptr(Kcache, "Kcache")) || (s = check_ptr(Vcache, "Vcache")) ||
      (s = check_ptr(O, "O")) || (s = check_ptr(workspace, "workspace")))
    return s;
  if (desc->num_landmarks > 0 && ((s = check_ptr(Kbar, "Kbar")) || (s = check_ptr(Vbar, "Vbar")))) return s;
  if (LSE != nullptr && !aligned16(LSE)) return fail(MSA_ERR_INVALID_ARG, "LSE is not 16-byte aligned");
  const size_t need = decode_ws_bytes(desc);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  float* ws_o = static_cast<float*>(workspace);
  float* ws_lse = ws_o + (size_t)desc->num_splits * desc->batch * desc->heads_q * desc->head_dim;
  return hip_status(msa::launch_decode(*desc, q, Kcache, Vcache, Kbar, Vbar, ctx_lens, nullptr, ws_o, ws_lse, O, LSE,
                                       static_cast<hipStream_t>(stream)),
                    "decode launch");
}

msa_status msa_append_kv(const msa_decode_desc* desc, const int32_t* positions, const void* k_new,
                         const void* v_new, void* Kcache, void* Vcache, void* Kbar, void* Vbar, void* stream) {
  msa_status s0 = check_append_shape(desc);
  if (s0 != MSA_OK) return s0;
  if ((long long)desc->ctx_len * desc->head_dim * 2 >= (1LL << 31))
    return fail(MSA_ERR_UNSUPPORTED, "ctx_len=%d: one head's cache must be < 2 GiB", desc->ctx_len);
  if (desc->batch == 0) return ok();
  if (positions == nullptr) return fail(MSA_ERR_INVALID_ARG, "positions is NULL");
  if ((reinterpret_cast<uintptr_t>(positions) & 3u) != 0)
    return fail(MSA_ERR_INVALID_ARG, "positions is not 4-byte aligned");
  msa_status s;
  if ((s = check_ptr(k_new, "k_new")) || (s = check_ptr(v_new, "v_new")) || (s = check_ptr(Kcache, "Kcache")) ||
      (s = check_ptr(Vcache, "Vcache")))
    return s;
  if (desc->num_landmarks > 0 && ((s = check_ptr(Kbar, "Kbar")) || (s = check_ptr(Vbar, "Vbar")))) return s;
  return hip_status(msa::launch_append(*desc, positions, nullptr, k_new, v_new, Kcache, Vcache, Kbar, Vbar,
                                       static_cast<hipStream_t>(stream)),
                    "append launch");
}

msa_status msa_decode_fwd_paged(const msa_decode_desc* desc, int32_t page_size, int32_t num_pages,
                                const int32_t* block_table, const int32_t* ctx_lens, const void* q,
                                const void* Kpages, const void* Vpages, const void* Kbar, const void* Vbar,
                                void* workspace, size_t workspace_bytes, void* O, float* LSE, void* stream) {
  msa_status s = check_decode_shape(desc);
  if (s != MSA_OK) return s;
  if (desc->batch == 0) return ok();
  msa::DecodePaging pg;
  if ((s = check_paging(desc, page_size, num_pages, block_table, &pg)) != MSA_OK) return s;
  if (ctx_lens == nullptr || (reinterpret_cast<uintptr_t>(ctx_lens) & 3u) != 0)
    return fail(MSA_ERR_INVALID_ARG, "ctx_lens is NULL or not 4-byte aligned");
  if ((s = check_ptr(q, "q")) || (s = check_ptr(Kpages, "Kpages")) || (s = check_ptr(Vpages, "Vpages")) ||
      (s = check_ptr(O, "O")) || (s = check_ptr(workspace, "workspace")))
    return s;
  if (desc->num_landmarks > 0 && ((s = check_ptr(Kbar, "Kbar")) || (s = check_ptr(Vbar, "Vbar")))) return s;
  if (LSE != nullptr && !aligned16(LSE)) return fail(MSA_ERR_INVALID_ARG, "LSE is not 16-byte aligned");
  const size_t need = decode_ws_bytes(desc);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  float* ws_o = static_cast<float*>(workspace);
  float* ws_lse = ws_o + (size_t)desc->num_splits * desc->batch * desc->heads_q * desc->head_dim;
  return hip_status(msa::launch_decode(*desc, q, Kpages, Vpages, Kbar, Vbar, ctx_lens, &pg, ws_o, ws_lse, O, LSE,
                                       static_cast<hipStream_t>(stream)),
                    "paged decode launch");
}

msa_status msa_append_kv_paged(const msa_decode_desc* desc, int32_t page_size, int32_t num_pages,
                               const int32_t* block_table, const int32_t* positions, const void* k_new,
                               const void* v_new, void* Kpages, void* Vpages, void* Kbar, void* Vbar,
                               void* stream) {
  msa_status s = check_append_shape(desc);
  if (s != MSA_OK) return s;
  if (desc->batch == 0) return ok();
  msa::DecodePaging pg;
  if ((s = check_paging(desc, page_size, num_pages, block_table, &pg)) != MSA_OK) return s;
  if (positions == nullptr || (reinterpret_cast<uintptr_t>(positions) & 3u) != 0)
    return fail(MSA_ERR_INVALID_ARG, "positions is NULL or not 4-byte aligned");
  if ((s = check_ptr(k_new, "k_new")) || (s = check_ptr(v_new, "v_new")) || (s = check_ptr(Kpages, "Kpages")) ||
      (s = check_ptr(Vpages, "Vpages")))
    return s;
  if (desc->num_landmarks > 0 && ((s = check_ptr(Kbar, "Kbar")) || (s = check_ptr(Vbar, "Vbar")))) return s;
  return hip_status(msa::launch_append(*desc, positions, &pg, k_new, v_new, Kpages, Vpages, Kbar, Vbar,
                                       static_cast<hipStream_t>(stream)),
                    "paged append launch");
}

msa_status msa_plan_rows(const msa_attn_desc* desc, int32_t* win_lo, int32_t* lm_count) {
  msa_status s = check_attn(desc);
  if (s != MSA_OK) return s;
  if (desc->seq_len > 0 && (win_lo == nullptr || lm_count == nullptr))
    return fail(MSA_ERR_INVALID_ARG, "output array is NULL");
  const int n = desc->seq_len, w = desc->window, G = desc->num_landmarks;
  const int L = G > 0 ? n / G : 1;
  for (int i = 0; i < n; ++i) {
    win_lo[i] = msa::win_lo(i, w);
    lm_count[i] = msa::lm_count(i, w, G, L);
  }
  return ok();
}

msa_status msa_plan_tiles(const msa_attn_desc* desc, int32_t* out, int64_t capacity, int64_t* count, int32_t* bm,
                          int32_t* bn) {
  msa_status s = check_attn(desc);
  if (s != MSA_OK) return s;
  if (count == nullptr || bm == nullptr || bn == nullptr) return fail(MSA_ERR_INVALID_ARG, "output is NULL");
  const bool bf = desc->in_dtype == MSA_DTYPE_BF16;
  const int BM = bf ? msa::kBM_BF16 : msa::kBM_F32;
  const int BN = bf ? msa::kBN_BF16 : msa::kBN_F32;
  const int n = desc->seq_len, w = desc->window, G = desc->num_landmarks;
  const int L = G > 0 ? n / G : 1;
  const int T = (n + BM - 1) / BM;
  int64_t total = 0;
  for (int t = 0; t < T; ++t) {
    const msa::TileRange r = msa::tile_range(t, BM, BN, n, w, G, L);
    total += r.n_lm_tiles + (r.kt_hi - r.kt_lo + 1);
  }
  *count = total;
  *bm = BM;
  *bn = BN;
  if (out == nullptr) return ok();
  if (capacity < total) return fail(MSA_ERR_CAPACITY, "capacity %lld < %lld tiles", (long long)capacity, (long long)total);
  int64_t k = 0;
  for (int t = 0; t < T; ++t) {
    const msa::TileRange r = msa::tile_range(t, BM, BN, n, w, G, L);
    for (int lt = 0; lt < r.n_lm_tiles; ++lt, ++k) {
      out[4 * k + 0] = t;
      out[4 * k + 1] = 0;
      out[4 * k + 2] = lt;
      out[4 * k + 3] = msa::lm_tile_interior(lt, BN, r.lm_lo) ? 1 : 0;
    }
    for (int kt = r.kt_lo; kt <= r.kt_hi; ++kt, ++k) {
      out[4 * k + 0] = t;
      out[4 * k + 1] = 1;
      out[4 * k + 2] = kt;
      out[4 * k + 3] = msa::win_tile_interior(kt, BN, r.r0, r.r1, w) ? 1 : 0;
    }
  }
  return ok();
}

msa_status msa_plan_decode(const msa_decode_desc* desc, int32_t* chunk_bounds, int32_t* lm_visible,
                           int32_t* entries) {
  msa_status s = check_decode(desc);
  if (s != MSA_OK) return s;
  if (chunk_bounds == nullptr || lm_visible == nullptr || entries == nullptr)
    return fail(MSA_ERR_INVALID_ARG, "output is NULL");
  const msa::DecodePlan p = msa::decode_plan(desc->ctx_len, desc->window, desc->num_landmarks, desc->num_splits);
  for (int c = 0; c <= desc->num_splits; ++c) {
    const long long b = (long long)c * p.chunk;
    chunk_bounds[c] = (int32_t)(b < p.entries ? b : p.entries);
  }
  *lm_visible = p.lm;
  *entries = p.entries;
  return ok();
}

msa_status msa_plan_decode_varlen(const msa_decode_desc* desc, int32_t ctx, int32_t* chunk_bounds,
                                  int32_t* lm_visible, int32_t* entries) {
  msa_status s = check_decode(desc);
  if (s != MSA_OK) return s;
  if (ctx < 0 || ctx > desc->ctx_len)
    return fail(MSA_ERR_INVALID_ARG, "ctx=%d outside [0, ctx_len=%d]", ctx, desc->ctx_len);
  if (chunk_bounds == nullptr || lm_visible == nullptr || entries == nullptr)
    return fail(MSA_ERR_INVALID_ARG, "output is NULL");
  const int G = desc->num_landmarks;
  const msa::DecodePlan p =
      msa::decode_plan_fixed(ctx, desc->window, G, G > 0 ? desc->ctx_len / G : 1, desc->num_splits);
  for (int c = 0; c <= desc->num_splits; ++c) {
    const long long b = (long long)c * p.chunk;
    chunk_bounds[c] = (int32_t)(b < p.entries ? b : p.entries);
  }
  *lm_visible = p.lm;
  *entries = p.entries;
  return ok();
}

}  // extern "C"
