// Paged prefill attention for 16-bit caches (gfx950): the step before decode.
//
// A chunk of a sequence's new tokens attends causally over the sequence's
// whole context -- its earlier tokens and the chunk itself, whose keys and
// values were written through the slots first -- read through the block
// table like decode ("Paged Attention as a Memory Manager", §How the Kernel
// Executes Paged Attention: at prefill each new sequence gets its logical
// blocks in order; "Paged Attention: Virtual Memory for the KV Cache", §The
// fix borrowed from operating systems).  Query token t of a chunk of L tokens
// in a context of P sits at position P - L + t and sees positions 0 .. its
// own: textbook causal attention (the pages give no formula), i.e. for each
// token exactly the decode result at that length.
//
// Work decomposition.  One workgroup per (sequence, kv head, block of
// 64 CB / group query tokens); its four waves each own CB blocks of 16
// matrix-core columns, the (query token, query head) pairs of 16 / group
// tokens of the kv head's group per block.  The workgroup streams the
// 16-token K/V tiles of the positions its tokens can see through a 6-slot LDS
// ring filled by direct global->LDS loads, each wave loading a quarter of
// every tile, so every K/V byte read serves 64 CB columns (CB = 2 for long
// chunks: twice the flops per byte streamed; CB = 1 keeps short chunks
// spread over many workgroups).  Per tile, wave and column block:
// S^T = K Q^T with v_mfma_f32_16x16x32 (the K operand read once for all
// blocks), a causal limit per column (skipped where every key of the tiles
// is visible to every column of the block), an online softmax over a lazy
// reference maximum (the exponent folds the scale in as one fma; the
// reference is raised to the column's exact maximum only when a lane's terms
// of a step sum past 2^16, which leaves no maximum on the common path), P
// split into a 16-bit high part and the rounded remainder for two P V
// products into O^T; a block none of whose columns sees the tiles skips
// them.  No split of the context: a workgroup covers its tokens' whole
// prefix, and many workgroups run at once.
//
// Tiles go in pairs: one softmax step covers 32 keys (one cross-lane
// reduction and one rescale check per 32 keys), and P V is one
// v_mfma_f32_16x16x32 per 16 value dims over both tiles (on gfx950 twice the
// rate of the 16x16x16 form over one tile): key k = 8 q + i of the product
// is key 4 q + i of the first tile for i < 4, of the second for i >= 4, in
// both operands.  Registers are held to two waves per SIMD.
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

// LDS reads of the ring and the block ids.  As volatile LDS accesses the
// compiler keeps them where they are (after the explicit waits and the
// barrier) and does not add a wait for every direct load still in flight.
template <class V>
__device__ __forceinline__ V ring_read(const uint8_t* p) {
  return *(const volatile __attribute__((address_space(3))) V*)(p);
}

// Wait until this wave's loads of the oldest tiles in flight have landed,
// when k newer tiles (LPW loads each) may stay in flight (k uniform, at most
// KMAX).
template <int LPW, int KMAX>
__device__ __forceinline__ void wait_oldest_tile(int k) {
  if constexpr (KMAX > 0) {
    if (k >= KMAX) {
      vm_wait<KMAX * LPW>();
      return;
    }
    wait_oldest_tile<LPW, KMAX - 1>(k);
  } else {
    vm_wait<0>();
  }
}

template <class T, int D, int BS, int G, int CB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(PrefillArgs a) {
  using bits = typename T::bits;
  using MF = MfmaOps<T>;
  using v8 = typename MF::v8;
  using el = typename MF::e;
  constexpr int TB = 16 / G;           // query tokens per column block
  constexpr int TQ = CB * TB;          // per wave
  constexpr int TQW = 4 * TQ;          // per workgroup
  constexpr int NS = D / 32;           // QK slices of 32 dims
  constexpr int NT = D / 16;           // PV row tiles of 16 dims
  constexpr int KI = D / 32;           // 1 KiB loads per K (and per V) tile
  constexpr int LPW = 2 * KI / 4;      // loads per wave per tile
  constexpr int NSL = 6;               // ring slots: three pairs of tiles
  constexpr int IDCAP = 512;           // tiles whose block ids are staged at once
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(LPW >= 1 && LPW * (NSL - 1) < 64, "loads per wave");
  // the ring is the dynamic LDS array, a separate object from the block ids,
  // so the compiler can tell that its direct loads never write s_ids; reads
  // of a landed slot are ordered by the explicit waits below
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  constexpr int SLOT = 2 * KI * 1024;
  __shared__ int2 s_ids[IDCAP];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int c = lane & 15;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int s = blockIdx.y / Hkv;
  const int h = blockIdx.y % Hkv;
  const int qs = a.query_start[s];
  const int P = min(max(a.ctx[s], 0), a.max_ctx);
  const int L = min(max(a.query_start[s + 1] - qs, 0), P);
  const int tq0 = blockIdx.x * TQW;
  if (tq0 >= L) return;                          // (whole workgroup)
  const int p0 = P - L;                          // position of the chunk's first token
  const int kmax = p0 + min(L, tq0 + TQW);       // positions the workgroup's tokens see
  const int nt = (kmax + 15) / 16;

  // this lane's column in block cb: token cb TB + j of the wave, head gc of
  // the group
  const int tw0 = tq0 + wave * TQ;
  const int j = c / G, gc = c % G;
  bool col_valid[CB];
  int lim[CB];                                   // causal limit of the column (exclusive)
  int64_t qrow[CB];
  u32x4 qop[CB][NS];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    col_valid[cb] = tw0 + cb * TB + j < L;
    const int tok = min(tw0 + cb * TB + j, L - 1);  // (a spare column repeats the last token)
    lim[cb] = p0 + tok + 1;
    qrow[cb] = (int64_t(qs) + tok) * Hq + int64_t(h) * G + gc;
    const bits* qp = static_cast<const bits*>(a.q) + qrow[cb] * D;
#pragma unroll
    for (int m = 0; m < NS; ++m) qop[cb][m] = *reinterpret_cast<const u32x4*>(qp + (4 * m + q) * 8);
  }
  // the last position any column of block cb sees, and the causal limit of
  // its first column, below which no key of the block is masked (both
  // uniform over the wave)
  int blk_last[CB], blk_open[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    blk_last[cb] = uniform(p0 + min(L, tw0 + (cb + 1) * TB) - 1);
    blk_open[cb] = uniform(p0 + min(tw0 + cb * TB, L - 1) + 1);
  }
  // scores are taken raw and scaled inside the exponent, which needs a
  // positive factor: a negative scale flips the sign of q (exact), a zero
  // one zeroes q and scales by 1 (every score is 0 either way)
  const float sraw = a.scale_log2;
  const uint32_t qflip = sraw < 0.f ? 0x80008000u : 0u;
  const uint32_t qkeep = sraw == 0.f ? 0u : 0xFFFFFFFFu;
  const float sf = sraw == 0.f ? 1.f : fabsf(sraw);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int m = 0; m < NS; ++m)
#pragma unroll
      for (int w = 0; w < 4; ++w) qop[cb][m][w] = (qop[cb][m][w] & qkeep) ^ qflip;
  // the query loads complete here, in a wait the compiler knows about
  // (vmcnt 0; expcnt and lgkmcnt at their maxima): otherwise it waits for
  // every load in flight before each tile's first product
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const int32_t* row = a.tables + int64_t(s) * a.table_stride;
  const bits* kpool = static_cast<const bits*>(a.k);
  const bits* vpool = static_cast<const bits*>(a.v);
  // block ids of tiles [from, from + IDCAP) (the whole workgroup)
  int id_base = 0;
  auto stage_ids = [&](int from) {
    const int n = min(IDCAP, nt - from);
    for (int i = threadIdx.x; i < n; i += 256) {
      const int t = from + i;
      int2 ids;
      if constexpr (BS == 16) {
        ids.x = ids.y = row[t];
      } else if constexpr (BS == 32) {
        ids.x = ids.y = row[t >> 1];
      } else {
        ids.x = row[2 * t];
        ids.y = 16 * t + 8 < kmax ? row[2 * t + 1] : ids.x;
      }
      s_ids[i] = ids;
    }
    id_base = from;
  };
  // this wave's quarter of the loads of tile t into its slot
  auto issue = [&](int t) {
    uint8_t* sl = ring + (t % NSL) * SLOT;
    const int b0 = uniform(ring_read<int32_t>(reinterpret_cast<const uint8_t*>(&s_ids[t - id_base].x)));
    const int b1 = uniform(ring_read<int32_t>(reinterpret_cast<const uint8_t*>(&s_ids[t - id_base].y)));
#pragma unroll
    for (int ii = 0; ii < LPW; ++ii) {
      const int i = wave * LPW + ii;             // load i of the tile's 2 KI
      if (i < KI) {
        const int u = i * 64 + lane;
        const int jj = u >> 4, tt = u & 15;
        int blk, tk;
        if constexpr (BS == 16) {
          blk = b0;
          tk = tt;
        } else if constexpr (BS == 32) {
          blk = b0;
          tk = 16 * (t & 1) + tt;
        } else {
          blk = tt < 8 ? b0 : b1;
          tk = tt & 7;
        }
        const int64_t e = ((int64_t(blk) * Hkv + h) * (D / 8) + jj) * (BS * 8) + tk * 8;
        dma16(kpool + e, sl + i * 1024);
      } else {
        const int u = (i - KI) * 64 + lane;
        const int d = u >> 1, hh = u & 1;
        int blk, tk0;
        if constexpr (BS == 16) {
          blk = b0;
          tk0 = 8 * hh;
        } else if constexpr (BS == 32) {
          blk = b0;
          tk0 = 16 * (t & 1) + 8 * hh;
        } else {
          blk = hh ? b1 : b0;
          tk0 = 0;
        }
        const int64_t e = ((int64_t(blk) * Hkv + h) * D + d) * BS + tk0;
        dma16(vpool + e, sl + i * 1024);
      }
    }
  };

  f32x4 acc[CB][NT];
  float m_ref[CB], l_lane[CB];                   // (reference maximum: scaled, log2 units)
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[cb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref[cb] = kNegInf;
    l_lane[cb] = 0.f;
  }

  // one softmax step over tiles t, t + 1 (OPEN: every key of the pair is
  // visible to every column of the wave, and the reference maxima are finite)
  auto pair_step = [&](int t, auto open_tag) __attribute__((always_inline)) {
    constexpr bool OPEN = decltype(open_tag)::value;
    const uint8_t* sa = ring + (t % NSL) * SLOT;
    const uint8_t* sb = ring + ((t + 1) % NSL) * SLOT;
    const int kp0 = 16 * t + 4 * q;              // keys kp0 .. + 3 (tile t), kp0 + 16 .. + 19 (tile t + 1)
    f32x4 sc[CB][2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const uint8_t* sl = h2 ? sb : sa;
      u32x4 kr[NS];
#pragma unroll
      for (int m = 0; m < NS; ++m) kr[m] = ring_read<u32x4>(sl + ((4 * m + q) * 16 + c) * 16);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        sc[cb][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (!OPEN) {
          if (16 * t > blk_last[cb]) continue;
        }
#pragma unroll
        for (int m = 0; m < NS; ++m) sc[cb][h2] = MF::qk(kr[m], qop[cb][m], sc[cb][h2]);
      }
    }
    // V rows of both tiles, 8 keys per lane (k = 8 q + i: key kp0 + i of
    // tile t for i < 4, of tile t + 1 for i >= 4), zeros past the
    // workgroup's last position (which may hold anything, NaN poison
    // included)
    u32x4 vr[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const u32x2 va = ring_read<u32x2>(sa + KI * 1024 + (16 * n + c) * 32 + 8 * q);
      const u32x2 vb = ring_read<u32x2>(sb + KI * 1024 + (16 * n + c) * 32 + 8 * q);
      vr[n] = u32x4{va[0], va[1], vb[0], vb[1]};
    }
    if constexpr (OPEN) {
      // exponents against the reference maxima as they stand; a column's
      // reference is raised to its exact maximum only when one of its terms
      // would pass 2^13 (or is not a number)
      float x[CB][8], xm[CB];
      bool over = false;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[cb][i] = __builtin_fmaf(sc[cb][0][i], sf, -m_ref[cb]);
          x[cb][4 + i] = __builtin_fmaf(sc[cb][1][i], sf, -m_ref[cb]);
        }
        xm[cb] = fmaxf(fmaxf(fmaxf(x[cb][0], x[cb][1]), fmaxf(x[cb][2], x[cb][3])),
                       fmaxf(fmaxf(x[cb][4], x[cb][5]), fmaxf(x[cb][6], x[cb][7])));
        over = over || !(xm[cb] <= 13.f);
      }
      if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          float cm = xor16<OpMax>(xm[cb]);
          cm = xor32<OpMax>(cm);
          const bool up = cm > 0.f;
          const float mn = up ? m_ref[cb] + cm : m_ref[cb];
          const float d = mn - m_ref[cb];
          const float alpha = fast_exp2(-d);
          m_ref[cb] = mn;
          l_lane[cb] *= alpha;
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[cb][n] *= alpha;
#pragma unroll
          for (int i = 0; i < 8; ++i) x[cb][i] -= d;
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(x[cb][i]);
        l_lane[cb] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
        v8 phi, plo;
        MF::split(pv, phi, plo);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          acc[cb][n] = MF::pv32(vr[n], phi, acc[cb][n]);
          acc[cb][n] = MF::pv32(vr[n], plo, acc[cb][n]);
        }
      }
    } else {
      if (16 * t + 32 > kmax) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) {
            const int k0 = kp0 + (w2 >> 1) * 16 + 2 * (w2 & 1);   // the two keys of 32-bit word w2
            uint32_t x = vr[n][w2];
            if (k0 >= kmax) x &= 0xFFFF0000u;
            if (k0 + 1 >= kmax) x &= 0x0000FFFFu;
            vr[n][w2] = x;
          }
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        // (tile 0 holds position 0, which every column sees, so no block
        // skips the first pair: m_ref is finite from then on and masked terms
        // give exp2(-inf) = 0)
        if (16 * t > blk_last[cb]) continue;
        float sv[8];
        if (16 * t + 32 <= blk_open[cb]) {
          // every key of the pair is visible to every column of the block
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[i] = sc[cb][0][i];
            sv[4 + i] = sc[cb][1][i];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[i] = kp0 + i < lim[cb] ? sc[cb][0][i] : kNegInf;
            sv[4 + i] = kp0 + 16 + i < lim[cb] ? sc[cb][1][i] : kNegInf;
          }
        }
        // exponents against the column's reference maximum as it stands; it
        // is raised (to the column's exact maximum, over its four lanes) only
        // when a lane's eight terms sum past 2^16 or are not finite (the first
        // step, whose reference is -inf): no maximum at all on the common path
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = fast_exp2(__builtin_fmaf(sv[i], sf, -m_ref[cb]));
        float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        if (__builtin_amdgcn_ballot_w64(!(ps <= 65536.f))) {
          float cm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                           fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
          cm = xor16<OpMax>(cm);
          cm = xor32<OpMax>(cm);
          const float mn = cm * sf;
          const bool up = mn > m_ref[cb];
          const float alpha = up ? (m_ref[cb] == kNegInf ? 0.f : fast_exp2(m_ref[cb] - mn)) : 1.f;
          m_ref[cb] = up ? mn : m_ref[cb];
          l_lane[cb] *= alpha;
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[cb][n] *= alpha;
#pragma unroll
          for (int i = 0; i < 8; ++i) p[i] = fast_exp2(__builtin_fmaf(sv[i], sf, -m_ref[cb]));
          ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        }
        l_lane[cb] += ps;
        v8 phi, plo;
        MF::split(p, phi, plo);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          acc[cb][n] = MF::pv32(vr[n], phi, acc[cb][n]);
          acc[cb][n] = MF::pv32(vr[n], plo, acc[cb][n]);
        }
      }
    }
  };

  stage_ids(0);
  __syncthreads();
  // tiles go in pairs (32 keys per softmax step): pair p computes from slots
  // 2p, 2p + 1 (mod NSL) while pair p + 1 is in flight and pair p + 2 fills
  // the slots of pair p - 1
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < nt) issue(i);
  // one pair: wait for its tiles, refill the slots of the pair before it,
  // compute
  auto advance = [&](int t, auto open_tag) __attribute__((always_inline)) {
    // this wave's loads of tiles t and t + 1 have landed once at most its
    // loads of the newer tiles are outstanding; the barrier then covers every
    // wave's share (and every wave is done with the previous pair, whose
    // slots are refilled next)
    wait_oldest_tile<LPW, 2>(min(nt - 1, t + 3) - min(nt - 1, t + 1));
    wg_barrier();
#pragma unroll
    for (int i = 4; i < 6; ++i) {
      const int tn = t + i;
      if (tn < nt) {
        if (tn >= id_base + IDCAP) {
          // next window of block ids (every slot's loads have landed: the
          // compiler waits for the table reads before the LDS writes)
          stage_ids(tn);
          lgkm_wait0();
          wg_barrier();
        }
        issue(tn);
      }
    }
    pair_step(t, open_tag);
  };
  // Pairs past the first whose keys every column of the wave sees (those
  // before the wave's first causal limit) take the open path: no causal
  // mask, no skipped block, no zeroed values, and one rescale check for all
  // blocks, so that each phase is one straight run of code in which the
  // matrix products of one block overlap the vector work of the next.  The
  // first pair (where the reference maxima are set) and those from the
  // diagonal on take the general path: a causal limit per column, blocks
  // past their last position skipped, and a missing tile t + 1 read from a
  // stale slot with every score masked and every value selected to zero.
  const int open_end = max(2, (blk_open[0] - 32) / 16 + 1);   // first t (even or odd) not open
  int t = 0;
  advance(t, std::false_type{});
  for (t = 2; t < open_end; t += 2) advance(t, std::true_type{});
  for (; t < nt; t += 2) advance(t, std::false_type{});

#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    float l = xor16<OpSum>(l_lane[cb]);
    l = xor32<OpSum>(l);
    if (col_valid[cb]) {
      const float inv = 1.f / l;
      const int64_t o = qrow[cb] * D + 4 * q;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const f32x4 v = acc[cb][n] * inv;
        if (a.out_f32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o + 16 * n) = v;
        } else {
          const uint32_t lo = T::from_f32(v[0]) | (T::from_f32(v[1]) << 16);
          const uint32_t hi = T::from_f32(v[2]) | (T::from_f32(v[3]) << 16);
          *reinterpret_cast<u32x2*>(static_cast<bits*>(a.out) + o + 16 * n) = u32x2{lo, hi};
        }
      }
    }
  }
}

template <class T, int D, int BS, int G>
hipError_t launch_g(const PrefillArgs& a, int32_t max_query_len, hipStream_t stream) {
  const int cb = prefill_column_blocks(G, max_query_len, a.num_seqs, a.num_kv_heads);
  const int tpw = 4 * cb * (16 / G);
  const size_t lds = 6 * 2 * (D / 32) * 1024;   // the tile ring: 6 slots of K and V
  dim3 grid((max_query_len + tpw - 1) / tpw, a.num_seqs * a.num_kv_heads), block(256);
  if (cb == 3) hipLaunchKernelGGL((prefill_kernel<T, D, BS, G, 3>), grid, block, lds, stream, a);
  else if (cb == 2) hipLaunchKernelGGL((prefill_kernel<T, D, BS, G, 2>), grid, block, lds, stream, a);
  else hipLaunchKernelGGL((prefill_kernel<T, D, BS, G, 1>), grid, block, lds, stream, a);
  return hipGetLastError();
}

template <class T, int D, int BS>
hipError_t launch_b(const PrefillArgs& a, int32_t group, int32_t max_query_len, hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<T, D, BS, 1>(a, max_query_len, stream);
    case 2: return launch_g<T, D, BS, 2>(a, max_query_len, stream);
    case 4: return launch_g<T, D, BS, 4>(a, max_query_len, stream);
    case 8: return launch_g<T, D, BS, 8>(a, max_query_len, stream);
    case 16: return launch_g<T, D, BS, 16>(a, max_query_len, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class T, int D>
hipError_t launch_d(const PrefillArgs& a, int32_t bs, int32_t group, int32_t max_query_len, hipStream_t stream) {
  switch (bs) {
    case 8: return launch_b<T, D, 8>(a, group, max_query_len, stream);
    case 16: return launch_b<T, D, 16>(a, group, max_query_len, stream);
    case 32: return launch_b<T, D, 32>(a, group, max_query_len, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class T>
hipError_t launch_t(const PrefillArgs& a, int32_t d, int32_t bs, int32_t group, int32_t max_query_len,
                    hipStream_t stream) {
  switch (d) {
    case 64: return launch_d<T, 64>(a, bs, group, max_query_len, stream);
    case 128: return launch_d<T, 128>(a, bs, group, max_query_len, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int32_t dtype, int32_t d, int32_t bs, int32_t group,
                          int32_t max_query_len, hipStream_t stream) {
  if (max_query_len <= 0 || a.num_seqs <= 0) return hipSuccess;
  switch (dtype) {
    case 1: return launch_t<F16>(a, d, bs, group, max_query_len, stream);
    case 2: return launch_t<BF16>(a, d, bs, group, max_query_len, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
