// Flash-attention forward instantiations (fp16, bf16; head dimension 128) and launcher.
#include "attention.hpp"

namespace dg {

int launch_attn(const AttnLaunch& l, void* stream) {
  AttnArgs a;
  a.Q = l.Q;
  a.K = l.K;
  a.V = l.V;
  a.O = l.O;
  a.BH = (int)l.BH;
  a.Sq = (int)l.Sq;
  a.Sk = (int)l.Sk;
  a.bytesQ = (uint32_t)(l.BH * l.Sq * l.D * 2);
  a.bytesKV = (uint32_t)(l.BH * l.Sk * l.D * 2);
  a.scale_log2 = (float)((double)l.scale * 1.4426950408889634);  // log2(e)
  a.q_blocks = (int)((l.Sq + 255) / 256);
  const dim3 grid((unsigned)(l.BH * a.q_blocks));
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool neg = l.scale < 0.f;
  if (l.dtype == DT_F16) {
    if (neg) hipLaunchKernelGGL((attn_fwd_kernel<F16T, true>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<F16T, false>), grid, dim3(512), 0, s, a);
  } else {
    if (neg) hipLaunchKernelGGL((attn_fwd_kernel<BF16T, true>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<BF16T, false>), grid, dim3(512), 0, s, a);
  }
  return (int)hipGetLastError();
}

}  // namespace dg
