// Extend attention: prefill of each request's unmatched suffix over its reused prefix.
//
// The RadixAttention explainer's point is that the matched prefix needs no recompute and
// only the rest of the prompt is prefilled.  For request r with p reused tokens and e new
// ones, query row j (token position i = p + j) attends over K/V of positions 0..i, gathered
// through the request's slot row: full over the prefix, causal over the suffix.  Query head
// h reads kv head h / (hq/hkv).
//
// Work items come from a host plan: (request, first extend row of a query tile), longest
// context first.  blockIdx.x = item * hkv + g, so consecutive workgroups cycle through the
// kv heads and each kv head's K/V stays in one XCD's L2 when hkv = 8.
//
// Three kernels:
//  - extend_dma (bf16 q/o, bf16 pool, d = 128) and extend_mfma (bf16 q/o, fp8 E4M3 pool,
//    d = 128) share the per-tile arithmetic (WaveAttn below): one workgroup = 4 waves = 128
//    query rows = (128/G tokens) x (G heads of one GQA group), so every K/V tile staged in LDS
//    is shared by the whole group.  Per 64-token K/V tile and wave (32 query rows):
//      S^T = K . Q^T  (A = K rows from LDS, B = Q^T held in registers), 32 MFMA 16x16x32;
//      online softmax in the log2 domain with a lazily moved reference max;
//      O^T += V^T . P^T (A = V^T from LDS, B = P^T straight from the S^T registers), 32 MFMA,
//      and the row sums with 4 more MFMA against a row of ones.
//    The S^T row order inside each 16-row MFMA block is permuted so that each lane's four
//    S^T values of two neighbouring blocks are 8 consecutive kv tokens, which is exactly the
//    B-operand slice of P^T for the PV product.  Tiles are double-buffered in LDS (one barrier
//    per tile).  extend_dma stages them with global-to-LDS loads (no registers, no LDS store
//    instructions) in a token-row layout and reads V^T with the transposing LDS read of gfx950;
//    extend_mfma gathers fp8 codes into registers, decodes them to bf16 (exact) and stores
//    K row-major and V transposed; the per-head scales are folded into the float32 logits and
//    output.  The slot table is read with buffer loads one tile ahead of the K/V records it
//    addresses, so a gathered row waits on no dependent load; rows are addressed in 64 bits
//    (slot * slot bytes), so pools beyond 4 GiB work.
//  - extend_vec (f32 q/o with an f32 pool at d 64 or 128, and bf16 q/o with a bf16 or fp8
//    pool at d 64): one wave per (tile, q head), VALU only; it serves the small fp32 case and
//    the head dim the MFMA kernels are not built for.

#include <math.h>

#include <algorithm>
#include <new>
#include <type_traits>

#include "device.h"

namespace pkv {
namespace {

// ------------------------------------------------------------------------------------------
// VALU path (fp32, and head dim 64 for bf16 q/o)
// ------------------------------------------------------------------------------------------

constexpr int kF32Tile = 16;   // query tokens per work item
constexpr int kF32Kv = 64;     // kv tokens per iteration (one per lane)

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) x += __shfl_xor(x, off);
  return x;
}

// one pool or q element as a float (fp8 codes decoded exactly; their scale is applied by the caller)
__device__ __forceinline__ float elem_f(float x) { return x; }
__device__ __forceinline__ float elem_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float elem_f(uint8_t x) { return e4m3x2_to_f32<false>((uint32_t)x).x; }
__device__ __forceinline__ void put_f(float* p, float x) { *p = x; }
__device__ __forceinline__ void put_f(bf16* p, float x) { *p = (bf16)x; }

// QT: q/o element type; PT: pool element type (float, bf16, or uint8_t E4M3 codes with
// per-kv-head scales kscale / vscale)
template <typename QT, typename PT, int D>
__global__ __launch_bounds__(64) void extend_vec(const QT* __restrict__ q, QT* __restrict__ o,
                                                 const PT* __restrict__ kpool, const PT* __restrict__ vpool,
                                                 const float* __restrict__ kscale, const float* __restrict__ vscale,
                                                 const int32_t* __restrict__ r2t, int64_t stride,
                                                 const int32_t* __restrict__ prefix_lens,
                                                 const int32_t* __restrict__ extend_lens,
                                                 const int32_t* __restrict__ qo_indptr,
                                                 const int32_t* __restrict__ work, int hq, int hkv,
                                                 float scale_log2, uint32_t max_slot) {
  constexpr int PER = D / 64;
  constexpr bool kFp8 = std::is_same<PT, uint8_t>::value;
  __shared__ float qs[kF32Tile][D];
  __shared__ float ps[kF32Kv];
  __shared__ int32_t sl[kF32Kv];
  const int lane = threadIdx.x;
  const int h = blockIdx.x % hq;
  const int w = blockIdx.x / hq;
  const int req = work[2 * w], j0 = work[2 * w + 1];
  const int p = prefix_lens[req], e = extend_lens[req];
  const int nq = min(kF32Tile, e - j0);
  const int g = h / (hq / hkv);
  const float kmul = kFp8 ? scale_log2 * kscale[g] : scale_log2;
  const float vmul = kFp8 ? vscale[g] : 1.f;
  const int64_t qrow0 = (int64_t)qo_indptr[req] + j0;
  for (int x = lane; x < kF32Tile * D; x += 64) {
    const int t = x / D, dd = x - t * D;
    qs[t][dd] = t < nq ? elem_f(q[((qrow0 + t) * hq + h) * D + dd]) : 0.f;
  }
  float m[kF32Tile], l[kF32Tile], acc[kF32Tile][PER];
#pragma unroll
  for (int t = 0; t < kF32Tile; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[t][i] = 0.f;
  }
  const int ctx = p + j0 + nq;
  const int32_t* row = r2t + (int64_t)req * stride;
  __syncthreads();
  for (int kv0 = 0; kv0 < ctx; kv0 += kF32Kv) {
    const int k = kv0 + lane;
    const bool kin = k < ctx;
    const int64_t slot = min((uint32_t)row[kin ? k : 0], max_slot);   // a slot past the pool reads the last one
    sl[lane] = (int32_t)slot;
    const PT* krow = kpool + (slot * hkv + g) * D;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kF32Tile; ++t) {
      if (t < nq) {  // uniform across the wave
        const int pos = p + j0 + t;
        float dot = 0.f;
        for (int dd = 0; dd < D; ++dd) dot = fmaf(qs[t][dd], elem_f(krow[dd]), dot);
        const float s = (kin && k <= pos) ? dot * kmul : -INFINITY;
        const float mn = fmaxf(m[t], wave_max64(s));   // finite: kv 0 is visible to every row
        const float alpha = exp2f(m[t] - mn);
        const float pk = exp2f(s - mn);
        l[t] = l[t] * alpha + wave_sum64(pk);
        ps[lane] = pk;
        __syncthreads();
        const int nk = min(kF32Kv, ctx - kv0);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          float a = acc[t][i] * alpha;
          for (int kk = 0; kk < nk; ++kk)
            a = fmaf(ps[kk], elem_f(vpool[((int64_t)sl[kk] * hkv + g) * D + lane + 64 * i]), a);
          acc[t][i] = a;
        }
        m[t] = mn;
        __syncthreads();
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kF32Tile; ++t) {
    if (t < nq) {
      const float inv = vmul / l[t];
#pragma unroll
      for (int i = 0; i < PER; ++i) put_f(o + ((qrow0 + t) * hq + h) * D + lane + 64 * i, acc[t][i] * inv);
    }
  }
}

// ------------------------------------------------------------------------------------------
// bf16 MFMA paths (d = 128)
// ------------------------------------------------------------------------------------------

constexpr int kD = 128;
constexpr int kBN = 64;                 // kv tokens per tile
constexpr int kRows = 128;              // query rows per workgroup (tokens x heads)

// kv token (tile-local) held in row rho of 16-row MFMA block mb of S^T.
__device__ __forceinline__ int sigma(int mb, int rho) {
  return 32 * (mb >> 1) + 8 * (rho >> 2) + 4 * (mb & 1) + (rho & 3);
}

// Buffer loads of the slot table: a raw buffer with range checking (the table stays below
// 2 GB), so an entry past the table reads as slot 0.  K/V rows of a bf16 pool of at most
// 2 GiB are gathered as structured-buffer records (PoolGather below); larger pools, and the
// fp8 path, use 64-bit addresses (slot * slot bytes + column), since a buffer offset is 32 bits.
__device__ u32x4 buf_load_raw_x4(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset,
                                 int aux) __asm("llvm.amdgcn.raw.ptr.buffer.load.v4i32");
__device__ u32x2 buf_load_raw_x2(__amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset,
                                 int aux) __asm("llvm.amdgcn.raw.ptr.buffer.load.v2i32");
constexpr int kBufWord3 = 0x00020000;   // 32-bit data format, no swizzle

__device__ __forceinline__ __amdgpu_buffer_rsrc_t table_rsrc(const void* p, int table_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, table_bytes, kBufWord3);
}

// Lazy rescaling: a row's reference max only moves when a tile's max exceeds it by more than
// this many log2 units, so P = 2^(s - m) stays <= 2^8 (fine for bf16 and fp32 sums) and the
// 64-register output rescale runs on the first tile and almost never after.
constexpr float kRescaleSlack = 8.f;

// One wave's 32 query rows (two 16-row MFMA blocks nb) and their online-softmax state.
//
// S^T comes out of the products exactly (bf16 x bf16 products, float32 sums); the softmax
// scale (log2 units, times the K scale for fp8 pools) and the reference max are applied in
// float32 by one fused multiply-add per value before the exponential, so no logit carries a
// rounding of a scaled operand.  Row sums come from one more MFMA per 32 tokens against a row
// of ones (the same bf16 P values the PV product uses): the matrix cores have room where the
// vector ALU has none.
// A tile is processed in two halves that the tile loop places in different iterations:
//   probs(S) -> P (exponentials, conversions, row sums), then qk(next tile) into the same S
//   registers block by block (each block's products start once its exponentials are done),
//   pv(P) (MFMA) beside the lane maxima of the next S (vector max; the rare rescale, which
//   must follow the products, comes after them),
// so each wave always has independent vector and matrix work to interleave.
template <int G>
struct WaveAttn {
  static constexpr int BT = kRows / G;   // query tokens per work item
  int ln, lg;
  int qt[2], qh[2];      // this lane's query token (in the item) and head, per row block
  int vis[2];            // last visible kv position of this lane's rows
  bf16x8 qf[2][4];       // Q^T as B operand: d = 32 ks + 8 lg .. +7 of the lane's query row
  floatx4 oacc[2][8];    // O^T, d block db
  floatx4 lsum[2];       // (ones row) . P^T: element 0 of lanes 0..15 holds the row sum
  float m[2];            // reference max (log2 units)
  float sc;              // softmax scale in log2 units (times the K scale for fp8 pools)
  bf16x8 ones_row;
  int qpos0;             // earliest visible position of any row of the wave

  __device__ __forceinline__ void load_q(const bf16* qp, bool ok, int nb) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 v = ok ? *(const u32x4*)(qp + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
      qf[nb][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  __device__ __forceinline__ void reset(int nb) {
    lsum[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[nb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
    m[nb] = 0.f;
    const bf16 one = (bf16)(ln == 0 ? 1.f : 0.f);
    ones_row = bf16x8{one, one, one, one, one, one, one, one};
  }

  __device__ __forceinline__ void init(const bf16* q, int64_t qrow0, int hq, int g, int wave, int lane, int nq,
                                       int p, int j0, int ctx, float scale) {
    ln = lane & 15;
    lg = lane >> 4;
    sc = scale;
    qpos0 = p + j0;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int r0 = 32 * wave + 16 * nb;
      qh[nb] = g * G + r0 / BT;
      qt[nb] = r0 % BT + ln;
      vis[nb] = min(qpos0 + qt[nb], ctx - 1);   // padded rows see the whole context
      const bool ok = qt[nb] < nq;
      load_q(q + ((qrow0 + (ok ? qt[nb] : 0)) * hq + qh[nb]) * kD + 8 * lg, ok, nb);
      reset(nb);
    }
  }

  // Rows of a decode item instead of extend rows: row r of the workgroup is the newest token
  // of sequence members[m0 + r / G] at head g * G + r % G (nm real members, so rows 0 ..
  // nm G - 1 are real and a wave whose 32 rows start at or past nm G has none), which sees
  // positions 0 .. seq_lens[b] - 1 (and none at or past kv_end, the end of the item's chunks).
  // A shared item's chunks lie inside every member's context, so its tiles never reach the mask;
  // a one-member item over a sequence's own last chunk masks the positions past its newest token.
  __device__ __forceinline__ void init_shared(const bf16* q, const int32_t* members, const int32_t* seq_lens, int m0,
                                              int nm, int batch, int hq, int g, int wave, int lane, float scale,
                                              int kv_end) {
    ln = lane & 15;
    lg = lane >> 4;
    sc = scale;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int r = 32 * wave + 16 * nb + ln;
      qh[nb] = g * G + r % G;
      qt[nb] = r / G;
      vis[nb] = kv_end - 1;   // padding rows see the whole item
      int b = qt[nb] < nm ? members[m0 + qt[nb]] : -1;
      const bool ok = b >= 0 && b < batch;   // a member index outside the batch is a padding row
      if (!ok) {
        b = 0;
        qt[nb] = BT;   // never stored
      } else {
        vis[nb] = min(seq_lens[b], kv_end) - 1;
      }
      load_q(q + ((int64_t)b * hq + qh[nb]) * kD + 8 * lg, ok, nb);
      reset(nb);
    }
    // the wave's earliest newest-token position: tiles ending at or before it need no mask
    int v = min(vis[0], vis[1]);
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) v = min(v, __shfl_xor(v, off));
    qpos0 = v;
  }

  // S^T = K . Q^T for one 64-token tile; kop(mb, ks) returns the K operand (tokens of S^T
  // block mb, d = 32 ks + 8 lg .. +7) read from LDS
  template <class KOp>
  __device__ __forceinline__ void qk(floatx4 (&s)[4][2], KOp kop) const {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const bf16x8 a = kop(mb, ks);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          s[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[nb][ks], ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f}
                                                                                      : s[mb][nb], 0, 0, 0);
      }
    }
  }

  // causal / context mask of the tile at kv0 (branch-free; callers use it on the tiles that
  // reach past the earliest visible position)
  __device__ __forceinline__ void mask(floatx4 (&s)[4][2], int kv0) const {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int lim = vis[nb] - kv0 - 8 * lg;   // visible iff token offset - 8 lg <= lim
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int off = 32 * (mb >> 1) + 4 * (mb & 1) + i;
          s[mb][nb][i] = off <= lim ? s[mb][nb][i] : -INFINITY;
        }
    }
  }

  // this lane's max over its 16 raw values of each row, in log2 units relative to the
  // reference max (three-input maxes in a shallow tree, then one fused multiply-add)
  __device__ __forceinline__ void lane_max(const floatx4 (&s)[4][2], float (&mt)[2]) const {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float a = fmaxf(fmaxf(s[0][nb][0], s[0][nb][1]), s[0][nb][2]);
      const float b = fmaxf(fmaxf(s[0][nb][3], s[1][nb][0]), s[1][nb][1]);
      const float c = fmaxf(fmaxf(s[1][nb][2], s[1][nb][3]), s[2][nb][0]);
      const float d = fmaxf(fmaxf(s[2][nb][1], s[2][nb][2]), s[2][nb][3]);
      const float e = fmaxf(fmaxf(s[3][nb][0], s[3][nb][1]), s[3][nb][2]);
      const float x = fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), s[3][nb][3]));
      mt[nb] = fmaf(x, sc, -m[nb]);
    }
  }

  // the row max across the four lanes that hold a query row (lanes ln, ln+16, ln+32, ln+48)
  static __device__ __forceinline__ float row_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
  }

  // move the reference max of each row up by d (log2 units, >= 0): the output and the row
  // sums follow
  __device__ __forceinline__ void shift(int nb, float d) {
    const float alpha = __builtin_amdgcn_exp2f(-d);   // 1 for rows that keep their max
    lsum[nb] *= alpha;
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[nb][db] *= alpha;
    m[nb] += d;
  }

  // first tile (reference 0, nothing accumulated yet): the reference max becomes the row max
  __device__ __forceinline__ void first_max(const floatx4 (&s)[4][2]) {
    float mt[2];
    lane_max(s, mt);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) m[nb] = row_max(mt[nb]);
  }

  // later tiles, from the lane maxima: only where some lane's value exceeds the reference by
  // more than the slack (one wave-uniform test, rare after the first tile) is the row max
  // formed and the row moved
  __device__ __forceinline__ void later_shift(const float (&mt)[2]) {
    if (__any(mt[0] > kRescaleSlack || mt[1] > kRescaleSlack)) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float x = row_max(mt[nb]);
        shift(nb, x > kRescaleSlack ? x : 0.f);
      }
    }
  }

  // P = 2^(sc S^T - m) as the bf16 B operand of the PV product (each lane's 8 values of a
  // block pair are 8 consecutive kv tokens)
  __device__ __forceinline__ void probs(const floatx4 (&s)[4][2], bf16x8 (&pf)[2][2]) const {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float nm = -m[nb];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[2 * kk][nb][i], sc, nm));
          pv[4 + i] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[2 * kk + 1][nb][i], sc, nm));
        }
        pf[nb][kk] = pv;
      }
    }
  }

  // O^T += V^T . P^T, and the row sums; vop(kk, db) returns the V^T operand (d = 16 db + ln,
  // tokens 32 kk + 8 lg .. +7) read from LDS.  Issued at raised wave priority: on a SIMD
  // shared with a wave in its vector work, the products go first.  pre() runs in the same
  // region, so its vector work (independent of the products) can fill their gaps.
  template <class VOp, class Pre>
  __device__ __forceinline__ void pv(const bf16x8 (&pf)[2][2], VOp vop, Pre pre) {
    __builtin_amdgcn_s_setprio(1);
    pre();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        lsum[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_row, pf[nb][kk], lsum[nb], 0, 0, 0);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const bf16x8 a = vop(kk, db);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          oacc[nb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[nb][kk], oacc[nb][db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // the row sum sits in element 0 of lane ln (row 0 of the ones product)
  __device__ __forceinline__ float row_sum(int nb) const { return __shfl(lsum[nb][0], ln); }

  // Split partials of a shared-prefix decode item, in the split phase's layout: for member b
  // and head h, partial p = (b * hq + h) * max_splits + s holds (reference max, row sum) at
  // ws_ml[2p], ws_ml[2p + 1] and the unnormalised output row (times omul) at ws_acc[p * d].
  // An item spanning chunks s .. s + span - 1 marks the later ones empty (max -inf, sum 0;
  // the reduce skips them without reading their output row).
  __device__ __forceinline__ void store_partial(float* ws_ml, float* ws_acc, const int32_t* members, int m0, int nm,
                                                int hq, int max_splits, int s, int span, float omul) const {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float lt = row_sum(nb);
      if (qt[nb] >= nm) continue;
      const int64_t part = ((int64_t)members[m0 + qt[nb]] * hq + qh[nb]) * max_splits + s;
      float* ap = ws_acc + part * kD + 4 * lg;
#pragma unroll
      for (int db = 0; db < 8; ++db) *(floatx4*)(ap + 16 * db) = oacc[nb][db] * omul;
      if (lg == 0) *(float2*)(ws_ml + 2 * part) = float2{m[nb], lt};
      for (int j = 1 + lg; j < span; j += 4) *(float2*)(ws_ml + 2 * (part + j)) = float2{-INFINITY, 0.f};
    }
  }

  // O = O^T / row sum (times the V scale for fp8 pools), bf16, for the item's real rows
  __device__ __forceinline__ void store(bf16* o, int64_t qrow0, int hq, int nq, float omul) const {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float lt = row_sum(nb);
      if (qt[nb] >= nq) continue;
      const float inv = omul / lt;
      bf16* op = o + ((qrow0 + qt[nb]) * hq + qh[nb]) * kD + 4 * lg;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const uint32_t w0 = f32_to_bf16_bits(oacc[nb][db][0] * inv) | (f32_to_bf16_bits(oacc[nb][db][1] * inv) << 16);
        const uint32_t w1 = f32_to_bf16_bits(oacc[nb][db][2] * inv) | (f32_to_bf16_bits(oacc[nb][db][3] * inv) << 16);
        *(u32x2*)(op + 16 * db) = u32x2{w0, w1};
      }
    }
  }
};

// The tile loop shared by every MFMA kernel.  Tile t's K is consumed one iteration before its
// V: iteration t runs the exponentials of tile t beside the S^T products of tile t + 1, then
// tile t's PV products beside tile t + 1's max.  K and V tiles are double-buffered in LDS
// (K(t) in kbuf[t & 1], V(t) in vbuf[t & 1]); iteration t stages K(t + 2) into kbuf[t & 1] and
// V(t + 1) into vbuf[(t + 1) & 1], whose readers (tile t's products, tile t - 1's PV) all
// passed the barrier that ends iteration t - 1, and ends with its own barrier.  The loop runs
// the tiles that need no mask two per trip with the buffers and S^T arrays fixed by the
// unrolling (so the compiler can tell the buffers apart), then the rest with the mask; the
// step after the last tile multiplies a tile past the context that the mask hides entirely.
// Stage must provide:
//   kMaxBesidePV       whether the next tile's lane maxima are formed beside the PV products
//                      (the register-staged fp8 path keeps them after: beside the products they
//                      push its register count past the limit)
//   prologue()         tiles K(0), V(0), K(1) staged and visible, then nothing in flight
//   issue(t, kd, vd)   start staging K(t + 2) into kd and V(t + 1) into vd
//   finish()           this thread's staging of iteration t complete (before the barrier)
// kop(buf, mb, ks) / vop(buf, kk, db) read operands from a K / V buffer.
template <int G, class Stage, class KOp, class VOp>
__device__ __forceinline__ void tile_loop(WaveAttn<G>& wa, Stage& st, int kv_begin, int n_tiles, int n_plain,
                                          bool active, char* k0, char* k1, char* v0, char* v1, KOp kop, VOp vop) {
  floatx4 s[4][2];   // S^T of the tile being exponentiated, then of the next one
  bf16x8 pf[2][2];
  st.prologue();
  __syncthreads();
  if (active) {
    wa.qk(s, [&](int mb, int ks) { return kop(k0, mb, ks); });
    wa.mask(s, kv_begin);
    wa.first_max(s);
  }
  __syncthreads();   // K(0)'s buffer takes K(2) next
  auto step = [&](auto mask_next, int t, const char* kr, const char* vr, char* kd, char* vd) {
    st.issue(t, kd, vd);
    if (active) {   // wave-uniform; with one head per item a wave of only padding tokens just stages
      wa.probs(s, pf);
      wa.qk(s, [&](int mb, int ks) { return kop(kr, mb, ks); });
      __builtin_amdgcn_sched_barrier(0);   // keep the PV operand reads out of the S^T half
      float mt[2];
      if constexpr (Stage::kMaxBesidePV) {
        wa.pv(pf, [&](int kk, int db) { return vop(vr, kk, db); }, [&]() {
          if constexpr (decltype(mask_next)::value) wa.mask(s, kv_begin + (t + 1) * kBN);
          wa.lane_max(s, mt);
        });
      } else {
        wa.pv(pf, [&](int kk, int db) { return vop(vr, kk, db); }, [] {});
        if constexpr (decltype(mask_next)::value) wa.mask(s, kv_begin + (t + 1) * kBN);
        wa.lane_max(s, mt);
      }
      wa.later_shift(mt);
    }
    st.finish();
    __syncthreads();
  };
  using Plain = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  int t = 0;
  // iteration t needs no mask when tile t + 1 is an unmasked tile
  for (; t + 2 < n_plain; t += 2) {
    step(Plain{}, t, k1, v0, k0, v1);
    step(Plain{}, t + 1, k0, v1, k1, v0);
  }
  // t is even here: the rest two per trip too, then possibly one more
  for (; t + 1 < n_tiles; t += 2) {
    step(Masked{}, t, k1, v0, k0, v1);
    step(Masked{}, t + 1, k0, v1, k1, v0);
  }
  if (t < n_tiles) step(Masked{}, t, k1, v0, k0, v1);
}

// ------------------------------------------------------------------------------------------
// bf16 pools: tiles staged by global-to-LDS loads
// ------------------------------------------------------------------------------------------
//
// LDS layout of a 64-token K (or V) tile: 16 blocks of 4 token rows (256 B each), block
// stride 1040 B, so block j starts 4 banks after block j - 1.  Token t (bits t0..t5) sits in
// block 2 t0 + 4 t1 + t4 + 8 t3, row t2 + 2 t5.  A global-to-LDS load writes 16 bytes per lane
// at consecutive addresses, so one load fills one block, 16 lanes per token row, which keeps
// the global reads of a row contiguous.  The 16 tokens of one S^T operand read differ in bits
// t0, t1, t3, t4 and so lie in 16 different blocks (16 different bank groups), and the 4
// tokens x 2 chunks of a 16-lane transposing V^T read cover 8 different bank groups.  All
// operand reads are at immediate offsets from a few per-lane bases.
constexpr int kBlk = 1040;
constexpr int kTileBytes = 16 * kBlk;
__device__ __forceinline__ int kv_off(int t) {
  const int blk = 2 * (t & 1) + 4 * ((t >> 1) & 1) + ((t >> 4) & 1) + 8 * ((t >> 3) & 1);
  const int row = ((t >> 2) & 1) + 2 * ((t >> 5) & 1);
  return blk * kBlk + row * 256;
}
// token in row r of block j (the inverse of the placement above)
__device__ __forceinline__ int kv_tok(int j, int r) {
  return ((j >> 1) & 1) + 2 * ((j >> 2) & 1) + 4 * (r & 1) + 8 * ((j >> 3) & 1) + 16 * (j & 1) + 32 * (r >> 1);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glob_void;

// Eight bf16 of one column of a row-major tile: two transposing reads.  In each 16-lane
// group, ds_read_b64_tr_b16 hands lane i element i of the 4 rows addressed by lanes
// 4j + i/4 (j = 0..3), i.e. lane k supplies the address of row k/4, columns 4(k%4) .. +3.
__device__ __forceinline__ bf16x8 lds_read_tr2(const char* p0, const char* p1) {
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p1);
  const v4i16 ab[2] = {a, b};
  return __builtin_bit_cast(bf16x8, ab);
}

// Gathers of one tile's rows into LDS (16 bytes per lane, one 4-row block per load).  NARROW:
// the pool is read as a raw buffer whose range check covers it (offset slot * slot bytes +
// column, one multiply-add per row; a slot past the pool reads zero); its 32-bit offsets
// reach 2 GiB of pool.  Otherwise 64-bit addresses, a slot past the pool clamped to the last.
template <bool NARROW>
struct PoolGather {
  const uint8_t *kcol, *vcol;   // pool + this lane's byte column
  __amdgpu_buffer_rsrc_t kp, vp;
  uint32_t slot_bytes, max_slot;
  int col;
  __device__ __forceinline__ PoolGather(const uint8_t* kpool, const uint8_t* vpool, int hkv, int num_slots, int col_)
      : kcol(kpool + col_), vcol(vpool + col_), slot_bytes((uint32_t)(hkv * 2 * kD)),
        max_slot((uint32_t)(num_slots - 1)), col(col_) {
    if constexpr (NARROW) {
      const int bytes = (int)((int64_t)num_slots * hkv * 2 * kD);
      kp = __builtin_amdgcn_make_buffer_rsrc((void*)kpool, (short)0, bytes, kBufWord3);
      vp = __builtin_amdgcn_make_buffer_rsrc((void*)vpool, (short)0, bytes, kBufWord3);
    }
  }
  __device__ __forceinline__ void k(uint32_t slot, char* d) const {
    if constexpr (NARROW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kp, (lds_void*)d, 16, (int)(slot * slot_bytes + col), 0, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((glob_void*)(kcol + (uint64_t)min(slot, max_slot) * slot_bytes), (lds_void*)d,
                                       16, 0, 0);
  }
  __device__ __forceinline__ void v(uint32_t slot, char* d) const {
    if constexpr (NARROW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vp, (lds_void*)d, 16, (int)(slot * slot_bytes + col), 0, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((glob_void*)(vcol + (uint64_t)min(slot, max_slot) * slot_bytes), (lds_void*)d,
                                       16, 0, 0);
  }
};
// pools up to this size are gathered through buffer offsets
constexpr int64_t kNarrowPoolBytes = (int64_t)1 << 31;

// Staging of a bf16 pool's tiles by global-to-LDS loads.  Wave w fills blocks 4w + i
// (i = 0..3) of a tile; lane l writes row l / 16 (token kv_tok(4w + i, l / 16)), byte column
// 16 (l % 16) of kv head g.  Those tokens are t, t + 16, t + 1, t + 17 for i = 0..3: two
// 8-byte slot-table reads per tile.  The slot table is read one tile ahead of the rows it
// addresses (each tile's slots serve its K at one iteration and its V at the next).  Tiles at
// or past the last one are staged as the last one (into buffers nobody reads after).
template <bool NARROW>
struct DmaStage {
  static constexpr bool kMaxBesidePV = true;
  const PoolGather<NARROW>& gather;
  __amdgpu_buffer_rsrc_t tab;
  int row_bytes, kv_begin, last, tok0, wave;
  char *k0, *v0, *k1;
  u32x2 s_k[2], s_v[2];   // slots of the next K tile to stage (t + 2) and of the next V tile (t + 1)
  __device__ __forceinline__ void slots(int tile, u32x2* sl) const {
    // the whole byte offset goes in the vector offset, which the buffer's range check covers
    const int kv0 = kv_begin + min(tile, last) * kBN;
    sl[0] = buf_load_raw_x2(tab, row_bytes + 4 * (kv0 + tok0), 0, 0);
    sl[1] = buf_load_raw_x2(tab, row_bytes + 4 * (kv0 + tok0 + 16), 0, 0);
  }
  __device__ __forceinline__ void stage_k(char* d, const u32x2* sl) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) gather.k(sl[i & 1][i >> 1], d + kBlk * (4 * wave + i));
  }
  __device__ __forceinline__ void stage_v(char* d, const u32x2* sl) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) gather.v(sl[i & 1][i >> 1], d + kBlk * (4 * wave + i));
  }
  __device__ __forceinline__ void prologue() {
    slots(0, s_v);
    slots(1, s_k);
    stage_k(k0, s_v);
    stage_v(v0, s_v);
    stage_k(k1, s_k);
    s_v[0] = s_k[0];
    s_v[1] = s_k[1];
    slots(2, s_k);
    // this wave's global-to-LDS loads are complete (vmcnt(0): the table loads issued after
    // them are waited for too); then the caller's barrier publishes the tiles
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  // iteration t: K(t + 2) with the slots read one iteration ago, V(t + 1) with those of K(t + 1);
  // then the slots of K(t + 3), which finish() waits for
  __device__ __forceinline__ void issue(int t, char* kd, char* vd) {
    stage_k(kd, s_k);
    stage_v(vd, s_v);
    s_v[0] = s_k[0];
    s_v[1] = s_k[1];
    slots(t + 3, s_k);
  }
  __device__ __forceinline__ void finish() const { __builtin_amdgcn_s_waitcnt(0x0F70); }
};

// K operand of S^T block mb at chunk ks, and the V^T operand of (kk, db), from a DMA-staged
// tile at per-lane bases: K row sigma(mb, ln) at chunk lg (+ 4 ks); V rows 32 kk + 8 lg + 4 h +
// ln / 4 at d = 4 (ln % 4) (+ 16 db)
struct DmaOperands {
  int kb[4], vb[2][2];
  __device__ __forceinline__ DmaOperands(int ln, int lg) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) kb[mb] = kv_off(sigma(mb, ln)) + 16 * lg;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h) vb[kk][h] = kv_off(32 * kk + 8 * lg + 4 * h + (ln >> 2)) + 8 * (ln & 3);
  }
  __device__ __forceinline__ bf16x8 k(const char* K, int mb, int ks) const {
    return *(const bf16x8*)(K + kb[mb] + 64 * ks);
  }
  __device__ __forceinline__ bf16x8 v(const char* V, int kk, int db) const {
    return lds_read_tr2(V + vb[kk][0] + 32 * db, V + vb[kk][1] + 32 * db);
  }
};

// tiles of an item before the first one that reaches past position `first_visible` (they
// need no mask)
__device__ __forceinline__ int plain_tiles(int kv_begin, int first_visible, int n_tiles) {
  const int n = (first_visible + 1 - kv_begin) / kBN;   // tiles ending at or before first_visible + 1
  return max(0, min(n, n_tiles));
}

template <int G, bool NARROW>
__global__ __launch_bounds__(256, 2) void extend_dma(const bf16* __restrict__ q, bf16* __restrict__ o,
                                                     const uint8_t* __restrict__ kpool,
                                                     const uint8_t* __restrict__ vpool,
                                                     const int32_t* __restrict__ r2t, int64_t stride,
                                                     const int32_t* __restrict__ prefix_lens,
                                                     const int32_t* __restrict__ extend_lens,
                                                     const int32_t* __restrict__ qo_indptr,
                                                     const int32_t* __restrict__ work, int hkv,
                                                     float scale_log2, int num_slots, int table_bytes) {
  // two buffers of K and V tiles, as separate arrays so that the loads into one buffer and the
  // reads of the other are known not to overlap (no wait for the loads before those reads)
  __shared__ __attribute__((aligned(16))) char k0s[kTileBytes], v0s[kTileBytes], k1s[kTileBytes], v1s[kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int g = blockIdx.x % hkv;
  const int w = blockIdx.x / hkv;
  const int req = work[2 * w], j0 = work[2 * w + 1];
  const int p = prefix_lens[req], e = extend_lens[req];
  const int nq = min(WaveAttn<G>::BT, e - j0);
  const int ctx = p + j0 + nq;
  const int hq = hkv * G;
  const int64_t qrow0 = (int64_t)qo_indptr[req] + j0;

  const PoolGather<NARROW> gather(kpool, vpool, hkv, num_slots, g * kD * 2 + 16 * ln);
  const int n_tiles = (ctx + kBN - 1) / kBN;
  DmaStage<NARROW> st{gather, table_rsrc(r2t, table_bytes), (int)((int64_t)req * stride * 4), 0, n_tiles - 1,
                      kv_tok(4 * wave, lg), wave, k0s, v0s, k1s};

  WaveAttn<G> wa;
  wa.init(q, qrow0, hq, g, wave, lane, nq, p, j0, ctx, scale_log2);
  // only for G = 1 (a wave's rows are 32 consecutive tokens): is any of them a real query?
  const bool active = G != 1 || 32 * wave < nq;
  const DmaOperands ops(ln, lg);
  // the item's first query token is the earliest visible position of every wave
  tile_loop<G>(wa, st, 0, n_tiles, plain_tiles(0, p + j0, n_tiles), active, k0s, k1s, v0s, v1s,
               [&](const char* K, int mb, int ks) { return ops.k(K, mb, ks); },
               [&](const char* V, int kk, int db) { return ops.v(V, kk, db); });
  wa.store(o, qrow0, hq, nq, 1.f);
}

// ------------------------------------------------------------------------------------------
// fp8 E4M3 pools: tiles gathered into registers, decoded to bf16, stored to LDS
// ------------------------------------------------------------------------------------------

constexpr int kKStride = kD + 8;        // bf16 elements per K row in LDS (272 B)
constexpr int kVStride = kBN + 8;       // bf16 elements per V^T row in LDS (144 B)
constexpr int kFp8KBytes = kBN * kKStride * 2;
constexpr int kFp8VBytes = kD * kVStride * 2;

// LDS row of kv token t in the K tile.  With a 272 B row stride a row starts at bank 4*row
// (mod 64), and one MFMA block reads tokens {0-3, 8-11, 16-19, 24-27} (+4, +32): flipping
// bit 2 of the row for the upper half of each 32-token group makes those 16 rows start on
// 16 different banks.
__device__ __forceinline__ int krow(int t) { return t ^ (((t >> 4) & 1) << 2); }

// four E4M3 codes -> four bf16 (exact: every E4M3 value is a bf16 value), with gfx950's
// packed conversion (scale 1)
__device__ __forceinline__ u32x2 dec4(uint32_t c) {
  return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.f, true))};
}

// Staging of an fp8 pool's tiles: global -> registers -> decoded -> LDS.
//   K: 64 rows x 128 B = 512 chunks of 16 B, 2 per thread (rows 2*(tid/8), +1, chunk tid%8).
//   V: thread -> 4 consecutive tokens (4*(tid%16) .. +3) x 8 d (8*(tid/16) .. +7), stored
//      transposed (V^T [d][token]).
// Iteration t stores K(t + 2) and V(t + 1) from the registers they were loaded into during
// iteration t - 1, then loads K(t + 3) and V(t + 2).  The slot-table entries run one more
// tile ahead.  Tokens at or past the context read whatever slot the table holds there (or
// zero past the table's end), rows past the pool the last slot; they are masked later.
struct Fp8Stage {
  static constexpr bool kMaxBesidePV = false;
  __amdgpu_buffer_rsrc_t tab;
  const uint8_t *kc, *vc;    // pool + this thread's byte column of kv head g
  uint32_t slot_bytes, max_slot;
  int row_bytes, kv_begin, last, tid;
  char *k0, *v0, *k1;
  u32x4 kr0, kr1;            // K codes of 2 tokens (16 B each), in flight
  u32x2 vr[4];               // V codes of 4 tokens (8 B each), in flight
  u32x2 sk;                  // slots of the next K tile to load
  u32x4 sv;                  // slots of the next V tile to load
  __device__ __forceinline__ u32x2 kslots(int tile) const {
    return buf_load_raw_x2(tab, row_bytes + 4 * (kv_begin + min(tile, last) * kBN) + 8 * (tid >> 3), 0, 0);
  }
  __device__ __forceinline__ u32x4 vslots(int tile) const {
    return buf_load_raw_x4(tab, row_bytes + 4 * (kv_begin + min(tile, last) * kBN) + 16 * (tid & 15), 0, 0);
  }
  __device__ __forceinline__ uint64_t off(uint32_t slot) const { return (uint64_t)min(slot, max_slot) * slot_bytes; }
  __device__ __forceinline__ void load_k(u32x2 s) {
    kr0 = *(const u32x4*)(kc + off(s[0]));
    kr1 = *(const u32x4*)(kc + off(s[1]));
  }
  __device__ __forceinline__ void load_v(u32x4 s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = *(const u32x2*)(vc + off(s[i]));
  }
  static __device__ __forceinline__ void store_k16(bf16* dst, u32x4 c) {
    const u32x2 a = dec4(c[0]), b = dec4(c[1]), d = dec4(c[2]), e = dec4(c[3]);
    *(u32x4*)dst = u32x4{a[0], a[1], b[0], b[1]};
    *(u32x4*)(dst + 8) = u32x4{d[0], d[1], e[0], e[1]};
  }
  __device__ __forceinline__ void store_k(char* Kd) const {
    bf16* Ks = (bf16*)Kd;
    const int r = 2 * (tid >> 3);   // tokens r, r+1
    bf16* kd = Ks + (tid & 7) * 16;
    store_k16(kd + krow(r) * kKStride, kr0);
    store_k16(kd + krow(r + 1) * kKStride, kr1);
  }
  // 4 tokens x 8 d (token-major in registers) to V^T [d][token]; one byte permute builds each
  // pair of 16-bit values
  __device__ __forceinline__ void store_v(char* Vd) const {
    bf16* Vt = (bf16*)Vd;
    u32x4 w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x2 lo = dec4(vr[j][0]), hi = dec4(vr[j][1]);
      w[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};   // token j, d = d0 .. d0 + 7 as bf16 pairs
    }
    const int d0 = 8 * (tid >> 4), t0 = 4 * (tid & 15);
    bf16* base = Vt + d0 * kVStride + t0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // d = d0 + 2i (low halves) and d0 + 2i + 1 (high halves) of tokens 0..3
      const u32x2 lo = {__builtin_amdgcn_perm(w[1][i], w[0][i], 0x05040100u),
                        __builtin_amdgcn_perm(w[3][i], w[2][i], 0x05040100u)};
      const u32x2 hi = {__builtin_amdgcn_perm(w[1][i], w[0][i], 0x07060302u),
                        __builtin_amdgcn_perm(w[3][i], w[2][i], 0x07060302u)};
      *(u32x2*)(base + (2 * i) * kVStride) = lo;
      *(u32x2*)(base + (2 * i + 1) * kVStride) = hi;
    }
  }
  __device__ __forceinline__ void prologue() {
    // K(0), V(0), K(1) to LDS; K(2), V(1) into registers; slots of K(3), V(2) in flight
    load_k(kslots(0));
    load_v(vslots(0));
    store_k(k0);
    store_v(v0);
    load_k(kslots(1));
    store_k(k1);
    load_k(kslots(2));
    load_v(vslots(1));
    sk = kslots(3);
    sv = vslots(2);
  }
  __device__ __forceinline__ void issue(int t, char* kd, char* vd) {
    store_k(kd);          // K(t + 2)
    store_v(vd);          // V(t + 1)
    load_k(sk);           // K(t + 3)
    load_v(sv);           // V(t + 2)
    sk = kslots(t + 4);
    sv = vslots(t + 3);
  }
  __device__ __forceinline__ void finish() const {}
};

struct Fp8Operands {
  int ln, lg;
  __device__ __forceinline__ bf16x8 k(const char* K, int mb, int ks) const {
    return *(const bf16x8*)((const bf16*)K + krow(sigma(mb, ln)) * kKStride + 32 * ks + 8 * lg);
  }
  __device__ __forceinline__ bf16x8 v(const char* V, int kk, int db) const {
    return *(const bf16x8*)((const bf16*)V + (16 * db + ln) * kVStride + 32 * kk + 8 * lg);
  }
};

template <int G>
__global__ __launch_bounds__(256, 2) void extend_mfma(const bf16* __restrict__ q, bf16* __restrict__ o,
                                                      const uint8_t* __restrict__ kpool,
                                                      const uint8_t* __restrict__ vpool,
                                                      const float* __restrict__ kscale,
                                                      const float* __restrict__ vscale,
                                                      const int32_t* __restrict__ r2t, int64_t stride,
                                                      const int32_t* __restrict__ prefix_lens,
                                                      const int32_t* __restrict__ extend_lens,
                                                      const int32_t* __restrict__ qo_indptr,
                                                      const int32_t* __restrict__ work, int hkv,
                                                      float scale_log2, int num_slots, int table_bytes) {
  // two K (row-major) / V^T tile buffers each
  __shared__ __attribute__((aligned(16))) char k0s[kFp8KBytes], k1s[kFp8KBytes], v0s[kFp8VBytes], v1s[kFp8VBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int g = blockIdx.x % hkv;
  const int w = blockIdx.x / hkv;
  const int req = work[2 * w], j0 = work[2 * w + 1];
  const int p = prefix_lens[req], e = extend_lens[req];
  const int nq = min(WaveAttn<G>::BT, e - j0);
  const int ctx = p + j0 + nq;
  const int hq = hkv * G;
  const int64_t qrow0 = (int64_t)qo_indptr[req] + j0;
  const int n_tiles = (ctx + kBN - 1) / kBN;

  Fp8Stage st;
  st.tab = table_rsrc(r2t, table_bytes);
  st.kc = kpool + g * kD + (tid & 7) * 16;
  st.vc = vpool + g * kD + (tid >> 4) * 8;
  st.slot_bytes = (uint32_t)(hkv * kD);
  st.max_slot = (uint32_t)(num_slots - 1);
  st.row_bytes = (int)((int64_t)req * stride * 4);
  st.kv_begin = 0;
  st.last = n_tiles - 1;
  st.tid = tid;
  st.k0 = k0s;
  st.v0 = v0s;
  st.k1 = k1s;

  WaveAttn<G> wa;
  wa.init(q, qrow0, hq, g, wave, lane, nq, p, j0, ctx, scale_log2 * kscale[g]);
  const bool active = G != 1 || 32 * wave < nq;
  const Fp8Operands ops{ln, lg};
  tile_loop<G>(wa, st, 0, n_tiles, plain_tiles(0, p + j0, n_tiles), active, k0s, k1s, v0s, v1s,
               [&](const char* K, int mb, int ks) { return ops.k(K, mb, ks); },
               [&](const char* V, int kk, int db) { return ops.v(V, kk, db); });
  wa.store(o, qrow0, hq, nq, vscale[g]);
}

// ------------------------------------------------------------------------------------------
// Shared-prefix decode: one chunk of context held in the same slots by several sequences
// ------------------------------------------------------------------------------------------
//
// A decode step reads each sequence's whole context once for a single query token.  Where
// several sequences of the batch hold a chunk of context in the same slots (a prefix the
// radix tree shares), their newest tokens are stacked as the query rows of one extend-style
// workgroup: the chunk's K/V tiles are staged once and multiplied against up to 128 query
// rows with MFMA, instead of being gathered once per sequence by the split phase.  An item
// (host plan) is (first member, member count <= 128 / G, first chunk s, span): one workgroup
// per (item, kv head), blockIdx.x = item * hkv + g, reads chunks s .. s + span - 1 (their
// slots from the first member's row).  The output is the split phase's partial at chunk s of
// every member (chunks s + 1 .. marked empty), which the reduce then merges with the other
// chunks.  Same tile loop as extend_dma / extend_mfma.

// the item's earliest newest-token position over all its members (the same in every wave):
// tiles ending before it need no mask
__device__ __forceinline__ int item_first_visible(const int32_t* members, const int32_t* seq_lens, int m0, int nm,
                                                  int batch, int kv_end, int lane) {
  int v = kv_end - 1;
  for (int i = lane; i < nm; i += 64) {
    const int b = members[m0 + i];
    if (b >= 0 && b < batch) v = min(v, seq_lens[b] - 1);
  }
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) v = min(v, __shfl_xor(v, off));
  return v;
}

// an item outside the batch or the workspace is ignored (the whole workgroup leaves)
__device__ __forceinline__ bool bad_item(int m0, int nm, int rows, int batch, int s, int span, int max_splits) {
  return m0 < 0 || nm <= 0 || nm > rows || m0 > batch - nm || s < 0 || span <= 0 || s > max_splits - span;
}

template <int G, bool NARROW>
__global__ __launch_bounds__(256, 2) void decode_shared_dma(const bf16* __restrict__ q,
                                                            const uint8_t* __restrict__ kpool,
                                                            const uint8_t* __restrict__ vpool,
                                                            const int32_t* __restrict__ r2t, int64_t stride,
                                                            const int32_t* __restrict__ members,
                                                            const int32_t* __restrict__ seq_lens,
                                                            const int32_t* __restrict__ items, int chunk,
                                                            int max_splits, int hkv, float scale_log2, int num_slots,
                                                            int table_bytes, int batch, float* __restrict__ ws_ml,
                                                            float* __restrict__ ws_acc) {
  __shared__ __attribute__((aligned(16))) char k0s[kTileBytes], v0s[kTileBytes], k1s[kTileBytes], v1s[kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int g = blockIdx.x % hkv;
  const int it = blockIdx.x / hkv;
  const int m0 = items[4 * it], nm = items[4 * it + 1], s = items[4 * it + 2], span = items[4 * it + 3];
  if (bad_item(m0, nm, WaveAttn<G>::BT, batch, s, span, max_splits)) return;
  const int hq = hkv * G;
  const int kv_begin = s * chunk;
  const int n_tiles = span * chunk / kBN;

  const PoolGather<NARROW> gather(kpool, vpool, hkv, num_slots, g * kD * 2 + 16 * ln);
  DmaStage<NARROW> st{gather, table_rsrc(r2t, table_bytes), (int)((int64_t)members[m0] * stride * 4), kv_begin,
                      n_tiles - 1, kv_tok(4 * wave, lg), wave, k0s, v0s, k1s};

  WaveAttn<G> wa;
  wa.init_shared(q, members, seq_lens, m0, nm, batch, hq, g, wave, lane, scale_log2, kv_begin + n_tiles * kBN);
  const bool active = 32 * wave < nm * G;   // a wave of only padding rows just stages
  const DmaOperands ops(ln, lg);
  const int first = item_first_visible(members, seq_lens, m0, nm, batch, kv_begin + n_tiles * kBN, lane);
  tile_loop<G>(wa, st, kv_begin, n_tiles, plain_tiles(kv_begin, first, n_tiles), active, k0s, k1s, v0s, v1s,
               [&](const char* K, int mb, int ks) { return ops.k(K, mb, ks); },
               [&](const char* V, int kk, int db) { return ops.v(V, kk, db); });
  wa.store_partial(ws_ml, ws_acc, members, m0, nm, hq, max_splits, s, span, 1.f);
}

template <int G>
__global__ __launch_bounds__(256, 2) void decode_shared_fp8(const bf16* __restrict__ q,
                                                            const uint8_t* __restrict__ kpool,
                                                            const uint8_t* __restrict__ vpool,
                                                            const float* __restrict__ kscale,
                                                            const float* __restrict__ vscale,
                                                            const int32_t* __restrict__ r2t, int64_t stride,
                                                            const int32_t* __restrict__ members,
                                                            const int32_t* __restrict__ seq_lens,
                                                            const int32_t* __restrict__ items, int chunk,
                                                            int max_splits, int hkv, float scale_log2, int num_slots,
                                                            int table_bytes, int batch, float* __restrict__ ws_ml,
                                                            float* __restrict__ ws_acc) {
  __shared__ __attribute__((aligned(16))) char k0s[kFp8KBytes], k1s[kFp8KBytes], v0s[kFp8VBytes], v1s[kFp8VBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int g = blockIdx.x % hkv;
  const int it = blockIdx.x / hkv;
  const int m0 = items[4 * it], nm = items[4 * it + 1], s = items[4 * it + 2], span = items[4 * it + 3];
  if (bad_item(m0, nm, WaveAttn<G>::BT, batch, s, span, max_splits)) return;
  const int hq = hkv * G;
  const int kv_begin = s * chunk;
  const int n_tiles = span * chunk / kBN;

  Fp8Stage st;
  st.tab = table_rsrc(r2t, table_bytes);
  st.kc = kpool + g * kD + (tid & 7) * 16;
  st.vc = vpool + g * kD + (tid >> 4) * 8;
  st.slot_bytes = (uint32_t)(hkv * kD);
  st.max_slot = (uint32_t)(num_slots - 1);
  st.row_bytes = (int)((int64_t)members[m0] * stride * 4);
  st.kv_begin = kv_begin;
  st.last = n_tiles - 1;
  st.tid = tid;
  st.k0 = k0s;
  st.v0 = v0s;
  st.k1 = k1s;

  WaveAttn<G> wa;
  wa.init_shared(q, members, seq_lens, m0, nm, batch, hq, g, wave, lane, scale_log2 * kscale[g],
                 kv_begin + n_tiles * kBN);
  const bool active = 32 * wave < nm * G;   // a wave of only padding rows just stages
  const Fp8Operands ops{ln, lg};
  const int first = item_first_visible(members, seq_lens, m0, nm, batch, kv_begin + n_tiles * kBN, lane);
  tile_loop<G>(wa, st, kv_begin, n_tiles, plain_tiles(kv_begin, first, n_tiles), active, k0s, k1s, v0s, v1s,
               [&](const char* K, int mb, int ks) { return ops.k(K, mb, ks); },
               [&](const char* V, int kk, int db) { return ops.v(V, kk, db); });
  wa.store_partial(ws_ml, ws_acc, members, m0, nm, hq, max_splits, s, span, vscale[g]);
}

int mfma_tile(int G) { return kRows / G; }

}  // namespace

int launch_decode_shared(const void* q, int32_t pool_dtype, const void* k_pool, const void* v_pool,
                         const float* k_scale, const float* v_scale, int64_t num_slots, const int32_t* r2t,
                         int64_t stride, int32_t batch, const int32_t* seq_lens, const int32_t* members,
                         const int32_t* items, int64_t n_items,
                         int chunk, int max_splits, int hq, int hkv, float sc_log2, float* ws_ml, float* ws_acc,
                         hipStream_t st) {
  const int G = hq / hkv;
  const int64_t slot_bytes = (int64_t)hkv * (pool_dtype == PKV_FP8_E4M3 ? 128 : 256);
  const int64_t table_bytes = (int64_t)batch * stride * 4;
  if (slot_bytes > 16383) return fail(PKV_ERR_UNSUPPORTED, "decode: a slot of %lld bytes is too wide", (long long)slot_bytes);
  if (table_bytes > 0x7FFFFFFFLL || num_slots > 0x7FFFFFFFLL)
    return fail(PKV_ERR_UNSUPPORTED, "decode: slot table or pool too large for 32-bit buffer offsets");
  if (n_items * hkv > 0x7FFFFFFFLL) return fail(PKV_ERR_INVAL, "decode: too many shared items");
  const dim3 grid((unsigned)(n_items * hkv));
  const bool narrow = num_slots * slot_bytes <= kNarrowPoolBytes;
#define PKV_SHARED_CASE(GG)                                                                                      \
  if (G == GG) {                                                                                                 \
    if (pool_dtype == PKV_BF16 && narrow)                                                                        \
      hipLaunchKernelGGL((decode_shared_dma<GG, true>), grid, dim3(256), 0, st, (const bf16*)q,                 \
                         (const uint8_t*)k_pool, (const uint8_t*)v_pool, r2t, stride, members, seq_lens, items, chunk, \
                         max_splits, hkv, sc_log2, (int)num_slots, (int)table_bytes, batch, ws_ml, ws_acc);      \
    else if (pool_dtype == PKV_BF16)                                                                             \
      hipLaunchKernelGGL((decode_shared_dma<GG, false>), grid, dim3(256), 0, st, (const bf16*)q,                \
                         (const uint8_t*)k_pool, (const uint8_t*)v_pool, r2t, stride, members, seq_lens, items, chunk, \
                         max_splits, hkv, sc_log2, (int)num_slots, (int)table_bytes, batch, ws_ml, ws_acc);      \
    else                                                                                                         \
      hipLaunchKernelGGL((decode_shared_fp8<GG>), grid, dim3(256), 0, st, (const bf16*)q, (const uint8_t*)k_pool, \
                         (const uint8_t*)v_pool, k_scale, v_scale, r2t, stride, members, seq_lens, items, chunk, \
                         max_splits, hkv, sc_log2, (int)num_slots, (int)table_bytes, batch, ws_ml, ws_acc);      \
    return hip_check(hipGetLastError(), "decode_shared launch");                                                 \
  }
  PKV_SHARED_CASE(1)
  PKV_SHARED_CASE(2)
  PKV_SHARED_CASE(4)
  PKV_SHARED_CASE(8)
#undef PKV_SHARED_CASE
  return fail(PKV_ERR_UNSUPPORTED, "decode: no shared-prefix kernel for group %d", G);
}

}  // namespace pkv

using namespace pkv;

extern "C" int32_t pkv_extend_tile(int32_t qo_dtype, int32_t pool_dtype, int32_t hq, int32_t hkv, int32_t d) {
  if (hq <= 0 || hkv <= 0 || hq % hkv) return PKV_ERR_INVAL;
  const int G = hq / hkv;
  if (qo_dtype == PKV_F32 && pool_dtype == PKV_F32 && (d == 64 || d == 128)) return kF32Tile;
  if (qo_dtype == PKV_BF16 && (pool_dtype == PKV_BF16 || pool_dtype == PKV_FP8_E4M3) && d == 64) return kF32Tile;
  if (qo_dtype == PKV_BF16 && (pool_dtype == PKV_BF16 || pool_dtype == PKV_FP8_E4M3) && d == 128 &&
      (G == 1 || G == 2 || G == 4 || G == 8))
    return mfma_tile(G);
  return PKV_ERR_UNSUPPORTED;
}

extern "C" int64_t pkv_extend_plan_size(const int32_t* extend_lens, int32_t num_reqs, int32_t tile) {
  if (num_reqs < 0 || tile <= 0 || (num_reqs > 0 && !extend_lens)) return fail(PKV_ERR_INVAL, "plan: bad arguments");
  int64_t n = 0;
  for (int32_t r = 0; r < num_reqs; ++r) {
    if (extend_lens[r] < 0) return fail(PKV_ERR_INVAL, "plan: negative extend length");
    n += (extend_lens[r] + tile - 1) / tile;
  }
  return n;
}

extern "C" int64_t pkv_extend_plan(const int32_t* prefix_lens, const int32_t* extend_lens, int32_t num_reqs,
                                   int32_t tile, int32_t* out_work, int64_t work_cap) {
  const int64_t n = pkv_extend_plan_size(extend_lens, num_reqs, tile);
  if (n < 0) return n;
  if (n > 0 && (!prefix_lens || !out_work)) return fail(PKV_ERR_INVAL, "plan: null pointer");
  if (work_cap < n) return fail(PKV_ERR_INVAL, "plan: needs %lld items", (long long)n);
  // (context length of the tile's last query, request, tile start): longest first, then by
  // request and tile so the order is deterministic
  struct Item {
    int64_t ctx;
    int32_t req, j0;
  };
  Item* items = new (std::nothrow) Item[(size_t)n + 1];
  if (!items) return fail(PKV_ERR_INTERNAL, "plan: host allocation failed");
  int64_t k = 0;
  for (int32_t r = 0; r < num_reqs; ++r)
    for (int32_t j0 = 0; j0 < extend_lens[r]; j0 += tile) {
      const int32_t nq = extend_lens[r] - j0 < tile ? extend_lens[r] - j0 : tile;
      items[k++] = Item{(int64_t)prefix_lens[r] + j0 + nq, r, j0};
    }
  std::stable_sort(items, items + n, [](const Item& a, const Item& b) { return a.ctx > b.ctx; });
  for (int64_t i = 0; i < n; ++i) {
    out_work[2 * i] = items[i].req;
    out_work[2 * i + 1] = items[i].j0;
  }
  delete[] items;
  return n;
}

extern "C" int pkv_extend_attention(const void* q, void* o, int32_t qo_dtype, const void* k_pool, const void* v_pool,
                                    int32_t pool_dtype, int64_t num_slots, const float* k_scale,
                                    const float* v_scale, const int32_t* req_to_token, int64_t stride,
                                    const int32_t* prefix_lens, const int32_t* extend_lens,
                                    const int32_t* qo_indptr, int32_t num_reqs, const int32_t* work,
                                    int64_t n_work, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                                    void* stream) {
  if (num_reqs < 0 || n_work < 0 || hq <= 0 || hkv <= 0 || hq % hkv || stride <= 0 || num_slots <= 0)
    return fail(PKV_ERR_INVAL, "extend: bad sizes");
  if (n_work == 0) return PKV_OK;
  if (!q || !o || !k_pool || !v_pool || !req_to_token || !prefix_lens || !extend_lens || !qo_indptr || !work)
    return fail(PKV_ERR_INVAL, "extend: null pointer");
  if (pkv_extend_tile(qo_dtype, pool_dtype, hq, hkv, d) < 0)
    return fail(PKV_ERR_UNSUPPORTED, "extend: qo dtype %d, pool dtype %d, hq %d, hkv %d, d %d", qo_dtype,
                pool_dtype, hq, hkv, d);
  if (pool_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return fail(PKV_ERR_INVAL, "extend: fp8 pool needs scales");
  if (!(sm_scale > 0.f)) return fail(PKV_ERR_INVAL, "extend: sm_scale must be positive");
  if ((int64_t)n_work * (qo_dtype == PKV_F32 || d == 64 ? hq : hkv) > 0x7FFFFFFFLL)
    return fail(PKV_ERR_INVAL, "extend: grid too large");
  hipStream_t st = (hipStream_t)stream;
  const float sc = sm_scale * kLog2e;
  const int G = hq / hkv;
  if (qo_dtype == PKV_F32 || d == 64) {
    if (num_slots > 0x7FFFFFFFLL) return fail(PKV_ERR_UNSUPPORTED, "extend: pool beyond int32 slots");
    const uint32_t mslot = (uint32_t)(num_slots - 1);
    const dim3 grid((unsigned)(n_work * hq));
    if (qo_dtype == PKV_F32 && d == 64)
      hipLaunchKernelGGL((extend_vec<float, float, 64>), grid, dim3(64), 0, st, (const float*)q, (float*)o,
                         (const float*)k_pool, (const float*)v_pool, k_scale, v_scale, req_to_token, stride,
                         prefix_lens, extend_lens, qo_indptr, work, hq, hkv, sc, mslot);
    else if (qo_dtype == PKV_F32)
      hipLaunchKernelGGL((extend_vec<float, float, 128>), grid, dim3(64), 0, st, (const float*)q, (float*)o,
                         (const float*)k_pool, (const float*)v_pool, k_scale, v_scale, req_to_token, stride,
                         prefix_lens, extend_lens, qo_indptr, work, hq, hkv, sc, mslot);
    else if (pool_dtype == PKV_BF16)
      hipLaunchKernelGGL((extend_vec<bf16, bf16, 64>), grid, dim3(64), 0, st, (const bf16*)q, (bf16*)o,
                         (const bf16*)k_pool, (const bf16*)v_pool, k_scale, v_scale, req_to_token, stride,
                         prefix_lens, extend_lens, qo_indptr, work, hq, hkv, sc, mslot);
    else
      hipLaunchKernelGGL((extend_vec<bf16, uint8_t, 64>), grid, dim3(64), 0, st, (const bf16*)q, (bf16*)o,
                         (const uint8_t*)k_pool, (const uint8_t*)v_pool, k_scale, v_scale, req_to_token, stride,
                         prefix_lens, extend_lens, qo_indptr, work, hq, hkv, sc, mslot);
    return hip_check(hipGetLastError(), "extend_vec launch");
  }
  const int64_t slot_bytes = (int64_t)hkv * (pool_dtype == PKV_FP8_E4M3 ? 128 : 256);
  const int64_t table_bytes = (int64_t)num_reqs * stride * 4;
  if (slot_bytes > 16383) return fail(PKV_ERR_UNSUPPORTED, "extend: a slot of %lld bytes is too wide", (long long)slot_bytes);
  if (table_bytes > 0x7FFFFFFFLL || num_slots > 0x7FFFFFFFLL)
    return fail(PKV_ERR_UNSUPPORTED, "extend: slot table or pool too large for 32-bit buffer offsets");
  const dim3 grid((unsigned)(n_work * hkv));
#define PKV_EXTEND_CASE(PP, GG)                                                                                  \
  if (pool_dtype == PP && G == GG) {                                                                             \
    hipLaunchKernelGGL((extend_mfma<GG>), grid, dim3(256), 0, st, (const bf16*)q, (bf16*)o,                      \
                       (const uint8_t*)k_pool, (const uint8_t*)v_pool, k_scale, v_scale, req_to_token, stride,   \
                       prefix_lens, extend_lens, qo_indptr, work, hkv, sc, (int)num_slots, (int)table_bytes);     \
    return hip_check(hipGetLastError(), "extend_mfma launch");                                                   \
  }
  const bool narrow = num_slots * slot_bytes <= kNarrowPoolBytes;
#define PKV_EXTEND_DMA(GG)                                                                                       \
  if (pool_dtype == PKV_BF16 && G == GG) {                                                                       \
    if (narrow)                                                                                                  \
      hipLaunchKernelGGL((extend_dma<GG, true>), grid, dim3(256), 0, st, (const bf16*)q, (bf16*)o,               \
                         (const uint8_t*)k_pool, (const uint8_t*)v_pool, req_to_token, stride, prefix_lens,      \
                         extend_lens, qo_indptr, work, hkv, sc, (int)num_slots, (int)table_bytes);               \
    else                                                                                                         \
      hipLaunchKernelGGL((extend_dma<GG, false>), grid, dim3(256), 0, st, (const bf16*)q, (bf16*)o,              \
                         (const uint8_t*)k_pool, (const uint8_t*)v_pool, req_to_token, stride, prefix_lens,      \
                         extend_lens, qo_indptr, work, hkv, sc, (int)num_slots, (int)table_bytes);               \
    return hip_check(hipGetLastError(), "extend_dma launch");                                                    \
  }
  PKV_EXTEND_DMA(1)
  PKV_EXTEND_DMA(2)
  PKV_EXTEND_DMA(4)
  PKV_EXTEND_DMA(8)
#undef PKV_EXTEND_DMA
  PKV_EXTEND_CASE(PKV_FP8_E4M3, 1)
  PKV_EXTEND_CASE(PKV_FP8_E4M3, 2)
  PKV_EXTEND_CASE(PKV_FP8_E4M3, 4)
  PKV_EXTEND_CASE(PKV_FP8_E4M3, 8)
#undef PKV_EXTEND_CASE
  return fail(PKV_ERR_UNSUPPORTED, "extend: no kernel for group %d", G);
}
