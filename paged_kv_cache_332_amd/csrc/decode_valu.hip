// Paged decode attention, vector-ALU kernel (every dtype and group size;
// the matrix-core kernel takes 16-bit caches with grouped heads).
//
// The kernel follows each sequence's block table instead of assuming the
// sequence is contiguous ("Paged Attention: Virtual Memory for the KV Cache",
// §The fix borrowed from operating systems; glossary "What is Paged
// Attention?") and computes plain softmax attention of one query per head.
//
// Work item = (sequence, kv head, head group, partition of `part` tokens),
// one 256-thread workgroup; its four waves take consecutive runs of blocks
// and keep separate running-max softmax states that are merged through LDS.
// Per block tile the 64 lanes map as follows (E = element bytes, X = 16/E):
//   K tile [D/X][BS][X]: load m, lane l reads bytes (64m + l)*16 = token
//       l % BS, chunk (l / BS) + (64/BS)*m -> dot products need a sum over
//       the 64/BS lane groups only (xor partners, bits log2(BS)..5);
//   V tile [D][BS]: load m, lane l reads bytes (64m + l)*16 = row
//       d = (64m + l) / CR, tokens (l % CR)*X .. +X (CR = BS*E/16 chunks per
//       row) -> each lane accumulates whole rows, weights come from LDS.
// Every load is one contiguous 1 KiB wave access; a tile is read once.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

template <class T, int D, int BS, int GH>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  using bits = typename T::bits;
  constexpr int E = T::kBytes;
  constexpr int X = 16 / E;
  constexpr int NG = 64 / BS;
  constexpr int NL = D * E * BS / 1024;
  constexpr int CR = BS * E / 16;
  constexpr int LBS = ilog2<BS>::value;
  constexpr int LCR = ilog2<CR>::value;
  static_assert(NL >= 1 && CR >= 1 && BS >= 8 && BS <= 32, "unsupported tile");

  __shared__ float lds_p[4][2][GH][BS];
  __shared__ float lds_m[4][GH];
  __shared__ float lds_l[4][GH];
  __shared__ float lds_acc[4][GH][D];

  const int G = a.num_q_heads / a.num_kv_heads;
  const int groups = G / GH;
  const int64_t total = int64_t(a.num_kv_heads) * groups * a.pmax * a.num_seqs;
  const int64_t rank = xcd_rank(total);
  if (rank >= total) return;
  const int seq = int(rank % a.num_seqs);
  int64_t r = rank / a.num_seqs;
  const int part = int(r % a.pmax);
  r /= a.pmax;
  const int kvh = int(r / groups);
  const int hg = int(r % groups);
  const int ctx = min(max(a.ctx[seq], 0), a.max_ctx);
  const int p0 = part * a.part;
  if (part > 0 && p0 >= ctx) return;
  const int p1 = min(ctx, p0 + a.part);
  const int nparts = max(1, (ctx + a.part - 1) / a.part);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = lane % BS;
  const int grp = lane / BS;
  const int cr = lane % CR;
  const int qh0 = kvh * G + hg * GH;

  // query chunks this lane multiplies: chunk grp + NG*m of each head
  u32x4 qreg[GH][NL];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const bits*>(a.q) +
                                                     (int64_t(seq) * a.num_q_heads + qh0) * D);
#pragma unroll
    for (int j = 0; j < GH; ++j)
#pragma unroll
      for (int m = 0; m < NL; ++m) qreg[j][m] = qp[j * (D / X) + grp + NG * m];
  }

  float m_ref[GH], l_lane[GH], acc[GH][NL];
#pragma unroll
  for (int j = 0; j < GH; ++j) {
    m_ref[j] = kNegInf;
    l_lane[j] = 0.f;
#pragma unroll
    for (int m = 0; m < NL; ++m) acc[j][m] = 0.f;
  }

  const int tpw = a.part / BS / 4;
  const int b_begin = p0 / BS + wave * tpw;
  const int b_end = min(b_begin + tpw, (p1 + BS - 1) / BS);
  const int32_t* trow = a.tables + int64_t(seq) * a.table_stride;
  const bits* kpool = static_cast<const bits*>(a.k);
  const bits* vpool = static_cast<const bits*>(a.v);
  constexpr int64_t kTile = int64_t(BS) * D;
  int buf = 0;

  for (int b = b_begin; b < b_end; ++b) {
    const int64_t tile = (int64_t(trow[b]) * a.num_kv_heads + kvh) * kTile;
    const u32x4* kt = reinterpret_cast<const u32x4*>(kpool + tile);
    const u32x4* vt = reinterpret_cast<const u32x4*>(vpool + tile);
    u32x4 kr[NL], vr[NL];
#pragma unroll
    for (int m = 0; m < NL; ++m) kr[m] = kt[64 * m + lane];
#pragma unroll
    for (int m = 0; m < NL; ++m) vr[m] = vt[64 * m + lane];

    const bool valid = b * BS + t < ctx;
    float p[GH];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < NL; ++m) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (E == 4) {
            s = __builtin_fmaf(__uint_as_float(qreg[j][m][w]), __uint_as_float(kr[m][w]), s);
          } else {
            s = T::dot2(qreg[j][m][w], kr[m][w], s);
          }
        }
      }
      s = reduce_high_bits<OpSum, LBS>(s);
      s = valid ? s * a.scale_log2 : kNegInf;
      float mt = reduce_low_bits<OpMax, LBS>(s);
      mt = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mt)));
      if (mt > m_ref[j] + 8.f) {
        // new reference maximum; a stale one within 2^8 is kept, which only
        // scales every term of this head alike
        const float alpha = m_ref[j] == kNegInf ? 0.f : fast_exp2(m_ref[j] - mt);
        l_lane[j] *= alpha;
#pragma unroll
        for (int m = 0; m < NL; ++m) acc[j][m] *= alpha;
        m_ref[j] = mt;
      }
      p[j] = fast_exp2(s - m_ref[j]);
      l_lane[j] += p[j];
    }

    if (grp == 0) {
#pragma unroll
      for (int j = 0; j < GH; ++j) lds_p[wave][buf][j][t] = p[j];
    }
    wave_lds_fence();

    const bool partial = (b + 1) * BS > ctx;
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      float pw[X];
#pragma unroll
      for (int x = 0; x < X; x += 4) {
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(&lds_p[wave][buf][j][cr * X + x]);
        pw[x] = v4[0];
        pw[x + 1] = v4[1];
        pw[x + 2] = v4[2];
        pw[x + 3] = v4[3];
      }
#pragma unroll
      for (int m = 0; m < NL; ++m) {
        float sum = acc[j][m];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (E == 4) {
            float v = __uint_as_float(vr[m][w]);
            if (partial && b * BS + cr * X + w >= ctx) v = 0.f;
            sum = __builtin_fmaf(pw[w], v, sum);
          } else {
            float v0 = T::lo(vr[m][w]), v1 = T::hi(vr[m][w]);
            if (partial) {
              const int tok = b * BS + cr * X + 2 * w;
              if (tok >= ctx) v0 = 0.f;
              if (tok + 1 >= ctx) v1 = 0.f;
            }
            sum = __builtin_fmaf(pw[2 * w], v0, sum);
            sum = __builtin_fmaf(pw[2 * w + 1], v1, sum);
          }
        }
        acc[j][m] = sum;
      }
    }
    buf ^= 1;
  }

  // per-wave totals
#pragma unroll
  for (int j = 0; j < GH; ++j) {
    l_lane[j] = reduce_low_bits<OpSum, LBS>(l_lane[j]);
#pragma unroll
    for (int m = 0; m < NL; ++m) acc[j][m] = reduce_low_bits<OpSum, LCR>(acc[j][m]);
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      lds_m[wave][j] = m_ref[j];
      lds_l[wave][j] = l_lane[j];
    }
  }
  if (cr == 0) {
#pragma unroll
    for (int j = 0; j < GH; ++j)
#pragma unroll
      for (int m = 0; m < NL; ++m) lds_acc[wave][j][m * (64 / CR) + lane / CR] = acc[j][m];
  }
  __syncthreads();

  // merge the four waves; write the result or this partition's partials
  for (int idx = threadIdx.x; idx < GH * D; idx += blockDim.x) {
    const int j = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, lds_m[w][j]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = lds_m[w][j];
      if (mw != kNegInf) {
        const float e = fast_exp2(mw - M);
        L = __builtin_fmaf(e, lds_l[w][j], L);
        O = __builtin_fmaf(e, lds_acc[w][j][d], O);
      }
    }
    const int64_t row = int64_t(seq) * a.num_q_heads + qh0 + j;
    if (nparts == 1) {
      const float val = L > 0.f ? O / L : 0.f;
      if (a.out_f32) static_cast<float*>(a.out)[row * D + d] = val;
      else static_cast<bits*>(a.out)[row * D + d] = static_cast<bits>(T::from_f32(val));
    } else {
      const int64_t slot = row * a.pmax + part;
      a.ws_acc[slot * D + d] = O;
      if (d == 0) {
        a.ws_m[slot] = M;
        a.ws_l[slot] = L;
      }
    }
  }
}

template <class T, int D, int BS>
static hipError_t launch_g(const DecodeArgs& a, int group, hipStream_t stream) {
  const int gh = group >= 4 ? 4 : group;
  const int64_t total = int64_t(a.num_kv_heads) * (group / gh) * a.pmax * a.num_seqs;
  dim3 grid(static_cast<uint32_t>(xcd_grid(total))), block(256);
  switch (gh) {
    case 1: hipLaunchKernelGGL((decode_valu_kernel<T, D, BS, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_valu_kernel<T, D, BS, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_valu_kernel<T, D, BS, 4>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_bs(const DecodeArgs& a, int bs, int group, hipStream_t stream) {
  switch (bs) {
    case 8: return launch_g<T, D, 8>(a, group, stream);
    case 16: return launch_g<T, D, 16>(a, group, stream);
    case 32: return launch_g<T, D, 32>(a, group, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class T>
static hipError_t launch_d(const DecodeArgs& a, int d, int bs, int group, hipStream_t stream) {
  switch (d) {
    case 64: return launch_bs<T, 64>(a, bs, group, stream);
    case 128: return launch_bs<T, 128>(a, bs, group, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_valu(const DecodeArgs& a, int32_t dtype, int32_t d, int32_t bs,
                              int32_t group, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_d<F32>(a, d, bs, group, stream);
    case 1: return launch_d<F16>(a, d, bs, group, stream);
    case 2: return launch_d<BF16>(a, d, bs, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
