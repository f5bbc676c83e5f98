// Paged decode attention on the gfx950 matrix cores, for 16-bit caches with
// grouped query heads (several query heads share one kv head, "Paged
// Attention: Virtual Memory for the KV Cache", §What it does not fix): the g
// query rows of a kv head against a 16-token tile form a small dense product.
//
// Work item = (sequence, kv head, partition), one 256-thread workgroup whose
// four waves take consecutive 16-token tiles and keep separate softmax states
// merged through LDS.  Per tile, with lane l = 16*q + c (q = l/16, c = l%16):
//   S^T[16 tok][16 heads] = K[16 tok][D] . Q^T[D][16 heads]
//       v_mfma_f32_16x16x32 over D/32 slices; A = K: lane l holds token c,
//       d-chunk 4m+q (8 elements = 16 bytes at (chunk*BS + token)*16 in the
//       K tile [D/8][BS][8]); B = Q^T: lane l holds head c (zero past g).
//       Result: lane l holds scores of head c for tokens 4q..4q+3.
//   O^T[D][16 heads] += V^T[D][16 tok] . P^T[16 tok][16 heads]
//       v_mfma_f32_16x16x16 per 16 rows of D; A = V^T: lane l holds row
//       d = 16n + c, tokens 4q..4q+3 (8 contiguous bytes of the V tile
//       [D][BS]); B = P^T: exactly the four probabilities lane l computed
//       from its S^T registers, so no data moves between the two products.
//       P is split into a bf16 (or f16) high part and the rounded remainder,
//       two products, so the weights keep ~16 significant bits.
// Softmax state (running reference max, sum) lives in the lanes of head c;
// the tile max needs two cross-row exchanges (lane bits 4 and 5).
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

template <class T>
struct Mfma;

template <>
struct Mfma<BF16> {
  using v8 = bf16x8;
  using v4 = bf16x4;
  using e = __bf16;
  __device__ static f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b),
                                                   c, 0, 0, 0);
  }
  __device__ static f32x4 pv(u32x2 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4, a), b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<F16> {
  using v8 = f16x8;
  using v4 = f16x4;
  using e = _Float16;
  __device__ static f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c,
                                                  0, 0, 0);
  }
  __device__ static f32x4 pv(u32x2 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4, a), b, c, 0, 0, 0);
  }
};

template <class T, int D, int BS, int GMAX>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  using bits = typename T::bits;
  using MF = Mfma<T>;
  using v4 = typename MF::v4;
  using el = typename MF::e;
  constexpr int NS = D / 32;  // QK slices
  constexpr int NT = D / 16;  // PV row tiles
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");

  __shared__ float lds_m[4][16];
  __shared__ float lds_l[4][16];
  __shared__ float lds_acc[4][GMAX][D + 4];

  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t total = int64_t(a.num_kv_heads) * a.pmax * a.num_seqs;
  const int64_t rank = xcd_rank(total);
  if (rank >= total) return;
  const int seq = int(rank % a.num_seqs);
  int64_t r = rank / a.num_seqs;
  const int part = int(r % a.pmax);
  const int kvh = int(r / a.pmax);
  const int ctx = min(max(a.ctx[seq], 0), a.max_ctx);
  const int p0 = part * a.part;
  if (part > 0 && p0 >= ctx) return;
  const int p1 = min(ctx, p0 + a.part);
  const int nparts = max(1, (ctx + a.part - 1) / a.part);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int c = lane & 15;

  // Q^T operand: head c, d-chunk 4m + q
  u32x4 qop[NS];
  {
    const int hq = kvh * G + min(c, G - 1);  // lanes past the group read a valid row, then zero it
    const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const bits*>(a.q) +
                                                     (int64_t(seq) * a.num_q_heads + hq) * D);
#pragma unroll
    for (int m = 0; m < NS; ++m) {
      const u32x4 v = qp[4 * m + q];
      qop[m] = c < G ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf, l_lane = 0.f;

  const int tpw = a.part / 64;  // 16-token tiles per wave
  const int k_begin = p0 / 16 + wave * tpw;
  const int k_end = min(k_begin + tpw, (p1 + 15) / 16);
  const int32_t* trow = a.tables + int64_t(seq) * a.table_stride;
  const bits* kpool = static_cast<const bits*>(a.k);
  const bits* vpool = static_cast<const bits*>(a.v);
  constexpr int64_t kTile = int64_t(BS) * D;
  const int64_t head_off = int64_t(kvh) * kTile;
  const int64_t blk_stride = int64_t(a.num_kv_heads) * kTile;

  // element offsets of this lane's K and V operands for tile k
  auto tile_offsets = [&](int k, int64_t& koff, int64_t& voff) {
    const int t0 = 16 * k;
    if constexpr (BS >= 16) {
      const int64_t base = int64_t(trow[t0 / BS]) * blk_stride + head_off;
      koff = base + (int64_t(q) * BS + (t0 % BS) + c) * 8;
      voff = base + int64_t(c) * BS + (t0 % BS) + 4 * q;
    } else {
      // a tile spans two 8-token blocks; the second is only read when it
      // holds a token of the context (its table entry exists)
      const int b0 = t0 / 8;
      const int64_t base0 = int64_t(trow[b0]) * blk_stride + head_off;
      const int64_t base1 = t0 + 8 < ctx ? int64_t(trow[b0 + 1]) * blk_stride + head_off : base0;
      koff = (c < 8 ? base0 : base1) + (int64_t(q) * 8 + (c & 7)) * 8;
      voff = (q < 2 ? base0 : base1) + int64_t(c) * 8 + 4 * (q & 1);
    }
  };
  // chunk stride between slices m: 4 chunks of BS tokens; row stride between
  // row tiles n: 16 rows of BS tokens
  auto load = [&](int k, u32x4 (&ko)[NS], u32x2 (&vo)[NT]) {
    int64_t koff, voff;
    tile_offsets(k, koff, voff);
#pragma unroll
    for (int m = 0; m < NS; ++m)
      ko[m] = *reinterpret_cast<const u32x4*>(kpool + koff + int64_t(m) * 4 * BS * 8);
#pragma unroll
    for (int n = 0; n < NT; ++n)
      vo[n] = *reinterpret_cast<const u32x2*>(vpool + voff + int64_t(n) * 16 * BS);
  };

  auto compute = [&](int k, const u32x4 (&ko)[NS], u32x2 (&vo)[NT]) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NS; ++m) s = MF::qk(ko[m], qop[m], s);
    const int tok0 = 16 * k + 4 * q;
    const bool partial = 16 * k + 16 > ctx;
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (!partial || tok0 + i < ctx) ? s[i] * a.scale_log2 : kNegInf;
    float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mt = xor16<OpMax>(mt);
    mt = xor32<OpMax>(mt);
    const bool need = mt > m_ref + 8.f;
    if (__builtin_amdgcn_ballot_w64(need)) {
      // a new reference maximum for the heads that need it; one within 2^8
      // of the stale reference is kept (every term of a head scales alike)
      const float alpha = need ? (m_ref == kNegInf ? 0.f : fast_exp2(m_ref - mt)) : 1.f;
      m_ref = need ? mt : m_ref;
      l_lane *= alpha;
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - m_ref);
    l_lane += (p[0] + p[1]) + (p[2] + p[3]);
    v4 phi, plo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const el h = static_cast<el>(p[i]);
      phi[i] = h;
      plo[i] = static_cast<el>(p[i] - static_cast<float>(h));
    }
    if (partial) {
      // tokens past the context may hold anything (NaN poison included):
      // select zeros instead of multiplying by a zero weight
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        uint32_t w0 = vo[n][0], w1 = vo[n][1];
        if (tok0 + 0 >= ctx) w0 &= 0xFFFF0000u;
        if (tok0 + 1 >= ctx) w0 &= 0x0000FFFFu;
        if (tok0 + 2 >= ctx) w1 &= 0xFFFF0000u;
        if (tok0 + 3 >= ctx) w1 &= 0x0000FFFFu;
        vo[n] = u32x2{w0, w1};
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      acc[n] = MF::pv(vo[n], phi, acc[n]);
      acc[n] = MF::pv(vo[n], plo, acc[n]);
    }
  };

  if (k_begin < k_end) {
    u32x4 kA[NS], kB[NS];
    u32x2 vA[NT], vB[NT];
    load(k_begin, kA, vA);
    int k = k_begin;
    for (; k + 1 < k_end; k += 2) {
      load(k + 1, kB, vB);
      compute(k, kA, vA);
      if (k + 2 < k_end) load(k + 2, kA, vA);
      compute(k + 1, kB, vB);
    }
    if (k < k_end) compute(k, kA, vA);
  }

  // per-wave totals: sum of the four token quarters of each head
  l_lane = xor16<OpSum>(l_lane);
  l_lane = xor32<OpSum>(l_lane);
  if (q == 0) {
    lds_m[wave][c] = m_ref;
    lds_l[wave][c] = l_lane;
  }
  if (c < G) {
#pragma unroll
    for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(&lds_acc[wave][c][16 * n + 4 * q]) = acc[n];
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
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
    const int64_t row = int64_t(seq) * a.num_q_heads + kvh * G + j;
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
static hipError_t launch_gm(const DecodeArgs& a, int group, hipStream_t stream) {
  const int64_t total = int64_t(a.num_kv_heads) * a.pmax * a.num_seqs;
  dim3 grid(static_cast<uint32_t>(xcd_grid(total))), block(256);
  if (group <= 4)
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, BS, 4>), grid, block, 0, stream, a);
  else if (group <= 8)
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, BS, 8>), grid, block, 0, stream, a);
  else if (group <= 16)
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, BS, 16>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_bs(const DecodeArgs& a, int bs, int group, hipStream_t stream) {
  switch (bs) {
    case 8: return launch_gm<T, D, 8>(a, group, stream);
    case 16: return launch_gm<T, D, 16>(a, group, stream);
    case 32: return launch_gm<T, D, 32>(a, group, stream);
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

hipError_t launch_decode_mfma(const DecodeArgs& a, int32_t dtype, int32_t d, int32_t bs,
                              int32_t group, hipStream_t stream) {
  switch (dtype) {
    case 1: return launch_d<F16>(a, d, bs, group, stream);
    case 2: return launch_d<BF16>(a, d, bs, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
