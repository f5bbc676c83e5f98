// Log-sum-exp merge of split-K partials.
//
// A sequence longer than one partition was reduced per partition p to
// (m_p = reference maximum in log2 units, l_p = sum of 2^(s - m_p),
// acc_p = sum of 2^(s - m_p) * v).  With M = max_p m_p the result is
//     out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,
// which equals softmax attention over the whole sequence.  One workgroup per
// (sequence, query head); partitions are spread over the threads' groups and
// combined in LDS.  Sequences held by one partition were finished by the
// partition pass and are skipped.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

template <class T, int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
  using bits = typename T::bits;
  constexpr int NGP = 256 / D;  // partition groups
  __shared__ float red_l[NGP];
  __shared__ float red_o[NGP][D];

  const int64_t row = blockIdx.x;  // seq * Hq + q head
  const int seq = int(row / a.num_q_heads);
  const int ctx = min(max(a.ctx[seq], 0), a.max_ctx);
  const int np = (ctx + a.part - 1) / a.part;
  if (np <= 1) return;
  const float* m = a.ws_m + row * a.pmax;
  const float* l = a.ws_l + row * a.pmax;
  const float* acc = a.ws_acc + row * a.pmax * D;

  float M = kNegInf;
  for (int p = 0; p < np; ++p) M = fmaxf(M, m[p]);

  const int g = threadIdx.x / D, d = threadIdx.x % D;
  float L = 0.f, O = 0.f;
  for (int p = g; p < np; p += NGP) {
    const float e = fast_exp2(m[p] - M);
    L = __builtin_fmaf(e, l[p], L);
    O = __builtin_fmaf(e, acc[int64_t(p) * D + d], O);
  }
  red_o[g][d] = O;
  if (d == 0) red_l[g] = L;
  __syncthreads();
  if (g == 0) {
    float Lt = 0.f, Ot = 0.f;
#pragma unroll
    for (int i = 0; i < NGP; ++i) {
      Lt += red_l[i];
      Ot += red_o[i][d];
    }
    const float val = Ot / Lt;
    if (a.out_f32) static_cast<float*>(a.out)[row * D + d] = val;
    else static_cast<bits*>(a.out)[row * D + d] = static_cast<bits>(T::from_f32(val));
  }
}

template <class T>
static hipError_t launch_t(const DecodeArgs& a, int d, hipStream_t stream) {
  dim3 grid(static_cast<uint32_t>(int64_t(a.num_seqs) * a.num_q_heads)), block(256);
  switch (d) {
    case 64: hipLaunchKernelGGL((merge_kernel<T, 64>), grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL((merge_kernel<T, 128>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs& a, int32_t dtype, int32_t d, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_t<F32>(a, d, stream);
    case 1: return launch_t<F16>(a, d, stream);
    case 2: return launch_t<BF16>(a, d, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
