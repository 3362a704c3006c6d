// Launchers of the gfx950 kernels, called by the C ABI layer after it has
// validated every argument.  Each returns the HIP error of its launch.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/msa.h"

namespace msa {

hipError_t launch_pool(const msa_attn_desc& d, const void* K, const void* V, void* Kbar, void* Vbar,
                       hipStream_t stream);

hipError_t launch_attn_bf16(const msa_attn_desc& d, const void* Q, const void* K, const void* V,
                            const void* Kbar, const void* Vbar, void* O, float* LSE,
                            hipStream_t stream);

// Attention over per-(batch, query head, 128-row query tile) lists of
// 64-key blocks (arguments validated; lists in device memory).
hipError_t launch_attn_list_bf16(const msa_attn_desc& d, const int32_t* counts, const int32_t* indices,
                                 int max_blocks, int causal, const void* Q, const void* K, const void* V, void* O,
                                 float* LSE, hipStream_t stream);

hipError_t launch_attn_f32(const msa_attn_desc& d, const void* Q, const void* K, const void* V,
                           const void* Kbar, const void* Vbar, void* O, float* LSE,
                           hipStream_t stream);

// Backward workspace layout (bytes) for a prefill problem.
struct BwdLayout {
  int n_pad, seg, nseg;
  size_t ld_off, part_off, lmg_off, bytes;
};
BwdLayout bwd_layout(const msa_attn_desc& d);

// Gradients dQ, dK, dV of the bf16 prefill (arguments validated).
hipError_t launch_attn_bwd(const msa_attn_desc& d, const void* Q, const void* K, const void* V, const void* Kbar,
                           const void* Vbar, const void* O, const float* LSE, const void* dO, void* workspace,
                           void* dQ, void* dK, void* dV, hipStream_t stream);

// Paged caches: pools [num_pages][Hkv][1 << page_shift][d]; sequence b's
// logical page p is physical page table[b * max_pages + p].
struct DecodePaging {
  const int32_t* table;
  int page_shift, max_pages, num_pages;
};

// lens: per-sequence lengths in device memory, or null for ctx_len each;
// paging: null for contiguous caches [B][Hkv][ctx_len][d].
hipError_t launch_decode(const msa_decode_desc& d, const void* q, const void* Kc, const void* Vc,
                         const void* Kbar, const void* Vbar, const int32_t* lens, const DecodePaging* paging,
                         float* ws_o, float* ws_lse, void* O, float* LSE, hipStream_t stream);

// Whether the decode of d runs the split schedule (per-chunk partials in
// the workspace) rather than the fused one.
bool decode_uses_split(const msa_decode_desc& d);

// The allocation-free decode's partials: a static device array of
// kNoallocScratchBytes; *ptr receives its address on the current device
// (looked up once per device).
constexpr size_t kNoallocScratchBytes = MSA_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(float** ptr);

// Write one token's K/V row per sequence at positions[b] (skipped outside
// [0, ctx_len)) and re-pool the landmark block that row completes.
hipError_t launch_append(const msa_decode_desc& d, const int32_t* positions, const DecodePaging* paging,
                         const void* k_new, const void* v_new, void* Kc, void* Vc, void* Kbar, void* Vbar,
                         hipStream_t stream);

}  // namespace msa
