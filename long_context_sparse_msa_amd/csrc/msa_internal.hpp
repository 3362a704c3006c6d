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

hipError_t launch_attn_f32(const msa_attn_desc& d, const void* Q, const void* K, const void* V,
                           const void* Kbar, const void* Vbar, void* O, float* LSE,
                           hipStream_t stream);

hipError_t launch_decode(const msa_decode_desc& d, const void* q, const void* Kc, const void* Vc,
                         const void* Kbar, const void* Vbar, float* ws_o, float* ws_lse, void* O,
                         float* LSE, hipStream_t stream);

}  // namespace msa
