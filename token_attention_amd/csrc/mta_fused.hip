// Fused forward: shape dispatch. The kernel template is in mta_fused_impl.h; each
// (dtype, head size) pair is instantiated in its own translation unit.
#include "mta_internal.h"

namespace mta {

hipError_t launch_fused_f32_d16(const Problem& p, hipStream_t stream);
hipError_t launch_fused_f32_d32(const Problem& p, hipStream_t stream);
hipError_t launch_fused_f32_d64(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d32(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d64(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d96(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d128(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d32_split(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d64_split(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d96_split(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d128_split(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d32_split_postconv(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d64_split_postconv(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d96_split_postconv(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d128_split_postconv(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d32_postconv(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d64_postconv(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d96_postconv(const Problem& p, hipStream_t stream);
hipError_t launch_fused_bf16_d128_postconv(const Problem& p, hipStream_t stream);

bool fused_supported(const Problem& p) {
  const int ch = p.mix ? p.c_h : 1;
  if (ch != 1 && ch != 2 && ch != 4) return false;
  if (p.kq && (p.c_q < 1 || p.c_q > 8 || p.c_k < 1 || p.c_k > 17 || p.c_k % 2 == 0)) return false;
  if (p.fp32 && p.split_mode) return false;
  if (p.fp32) return p.d == 16 || p.d == 32 || p.d == 64;
  return p.d == 32 || p.d == 64 || p.d == 96 || p.d == 128;
}

hipError_t launch_fused(const Problem& p, hipStream_t stream, bool* unsupported) {
  *unsupported = false;
  if (!fused_supported(p)) {
    *unsupported = true;
    return hipSuccess;
  }
  if (p.fp32) {
    switch (p.d) {
      case 16: return launch_fused_f32_d16(p, stream);
      case 32: return launch_fused_f32_d32(p, stream);
      case 64: return launch_fused_f32_d64(p, stream);
    }
  } else if (p.split_mode) {  // one chunk of a split key range
    const bool post = (p.kq & KQ_POST) != 0;
    switch (p.d) {
      case 32: return post ? launch_fused_bf16_d32_split_postconv(p, stream) : launch_fused_bf16_d32_split(p, stream);
      case 64: return post ? launch_fused_bf16_d64_split_postconv(p, stream) : launch_fused_bf16_d64_split(p, stream);
      case 96: return post ? launch_fused_bf16_d96_split_postconv(p, stream) : launch_fused_bf16_d96_split(p, stream);
      case 128:
        return post ? launch_fused_bf16_d128_split_postconv(p, stream) : launch_fused_bf16_d128_split(p, stream);
    }
  } else if (p.kq & KQ_POST) {
    switch (p.d) {
      case 32: return launch_fused_bf16_d32_postconv(p, stream);
      case 64: return launch_fused_bf16_d64_postconv(p, stream);
      case 96: return launch_fused_bf16_d96_postconv(p, stream);
      case 128: return launch_fused_bf16_d128_postconv(p, stream);
    }
  } else {
    switch (p.d) {
      case 32: return launch_fused_bf16_d32(p, stream);
      case 64: return launch_fused_bf16_d64(p, stream);
      case 96: return launch_fused_bf16_d96(p, stream);
      case 128: return launch_fused_bf16_d128(p, stream);
    }
  }
  *unsupported = true;
  return hipSuccess;
}

}  // namespace mta
