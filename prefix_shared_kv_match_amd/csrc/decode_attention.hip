// Split-K decode attention over K/V gathered through slot rows, then a log-sum-exp reduce.
//
// Decode is the `gen` step of the pages (one new token per sequence per step, attending
// over its whole cached context, the newest token's own K/V included).  The context of
// sequence b is cut into chunks; for each chunk s a workgroup streams the chunk's K and V
// rows and keeps a running max / running sum / unnormalised output for the G = hq/hkv
// query heads that share a kv head, so every gathered row is read once for the whole GQA
// group.  The reduce merges the chunks: M = max_s m_s, o = sum_s 2^(m_s-M) acc_s /
// sum_s 2^(m_s-M) l_s.
//
// Layout on gfx950: a 256-thread workgroup is 16 rows of 16 lanes.  A 16-lane row owns one
// token at a time and covers the head dim (d/16 values per lane), so each K or V row
// (256 B for bf16 d=128, 128 B for fp8) is one coalesced access per row of lanes.  Dot
// products are reduced inside the row with DPP (no LDS).  Each row runs its own online
// softmax over a token sub-stream; rows of one head are merged once at the end.  Work is
// HBM-bound (about 4 FLOP per gathered byte for bf16 GQA-4), so no MFMA is used.
//  - decode_split_slot (hkv 2, 4 or 8, or any multiple of 8 in groups of 8 heads, e.g.
//    multi-head attention): one workgroup per (sequence, chunk, head group), so a token's
//    slot row (or its 8-head part) is read at once; blockIdx.x = (b * ns_odd + s - s0) *
//    groups + group over chunks s0 .. s0 + ns - 1 (s0 > 0 when a shared-prefix pass has
//    covered every sequence's first s0 chunks).  The chunk count per sequence is padded to an
//    odd number (the extra workgroup leaves at once): with the XCD of a workgroup being
//    blockIdx.x mod 8, chunk s of consecutive sequences then lands on different XCDs, and the
//    XCDs get equal work whatever the spread of context lengths (an even count would pin a
//    chunk index to one or a few XCDs, and only long sequences have late chunks).
//  - decode_split (other hkv, and the short private tails left after a shared-prefix pass):
//    one workgroup per (sequence, chunk, kv head), 16 token streams; blockIdx.x =
//    (b * ns + s - s0) * hkv + g, so consecutive workgroups cycle through the kv heads.

#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "device.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;

// K/V rows are read once per step, so their loads are nontemporal: they stream past the
// caches instead of evicting lines that are reused (1.71 -> 1.58 ms on the 512-sequence bf16
// decode batch).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));

// VEC consecutive pool values of one (slot, head) row as loaded (raw bytes), so a group of
// tokens in flight costs only its loaded registers; the consumer decodes them once per token
// (floats, or bf16 pairs for packed dot products) and reuses them for every q head.
template <int POOL, int VEC>
struct RowChunk;

template <int VEC>
struct RowChunk<PKV_F32, VEC> {
  static constexpr int kBytes = VEC * 4;
  f32x4_nt r[VEC / 4];
  __device__ __forceinline__ void load(const uint8_t* p) {
#pragma unroll
    for (int i = 0; i < VEC / 4; ++i) r[i] = __builtin_nontemporal_load((const f32x4_nt*)p + i);
  }
  __device__ __forceinline__ void floats(float* f) const {
#pragma unroll
    for (int i = 0; i < VEC; ++i) f[i] = r[i / 4][i & 3];
  }
};

template <int VEC>
struct RowChunk<PKV_BF16, VEC> {
  static constexpr int kBytes = VEC * 2;
  uint32_t w[VEC / 2];
  __device__ __forceinline__ void load(const uint8_t* p) {
    if constexpr (VEC == 8) {
      const u32x4_nt v = __builtin_nontemporal_load((const u32x4_nt*)p);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
      const u32x2_nt v = __builtin_nontemporal_load((const u32x2_nt*)p);
      w[0] = v.x; w[1] = v.y;
    }
  }
  __device__ __forceinline__ void floats(float* f) const {
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  }
  __device__ __forceinline__ void pairs(bf16x2* p) const {
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) p[i] = __builtin_bit_cast(bf16x2, w[i]);
  }
};

template <int VEC>
struct RowChunk<PKV_FP8_E4M3, VEC> {
  static constexpr int kBytes = VEC;
  uint32_t w[VEC / 4];
  __device__ __forceinline__ void load(const uint8_t* p) {
    if constexpr (VEC == 8) {
      const u32x2_nt v = __builtin_nontemporal_load((const u32x2_nt*)p);
      w[0] = v.x; w[1] = v.y;
    } else {
      w[0] = __builtin_nontemporal_load((const uint32_t*)p);
    }
  }
  // hardware E4M3 conversion, two codes per instruction
  __device__ __forceinline__ void floats(float* f) const {
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) {
      const float2 a = e4m3x2_to_f32<false>(w[j]), b = e4m3x2_to_f32<true>(w[j]);
      f[4 * j] = a.x; f[4 * j + 1] = a.y; f[4 * j + 2] = b.x; f[4 * j + 3] = b.y;
    }
  }
  // every E4M3 value is a bf16 value, so the pairs are exact
  __device__ __forceinline__ void pairs(bf16x2* p) const {
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) {
      p[2 * j] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.f, false);
      p[2 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.f, true);
    }
  }
};

template <typename QT>
__device__ __forceinline__ float load_q(const QT* p, int i);
template <>
__device__ __forceinline__ float load_q<float>(const float* p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float load_q<bf16>(const bf16* p, int i) { return (float)p[i]; }

__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float m2, float l2, const float* acc2,
                                            int n) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  const float a = exp2f(m - mn), b = exp2f(m2 - mn);
  l = l * a + l2 * b;
  for (int i = 0; i < n; ++i) acc[i] = acc[i] * a + acc2[i] * b;
  m = mn;
}

// The online-softmax state of one 16-lane row for the G q heads of its kv head, over a stream
// of tokens first, first + STRIDE, ... of [t0, t1).  Lane li covers values li*VEC .. +VEC-1 of
// the head dim; dot products are reduced over the row with DPP.  With bf16 q and a bf16 or
// fp8 pool, q.k runs as packed bf16 dot products (float32 accumulation).
template <typename QT, int POOL, int VEC, int G>
struct HeadStream {
  using Chunk = RowChunk<POOL, VEC>;
  static constexpr bool kDot2 = sizeof(QT) == 2 && POOL != PKV_F32;
  float qf[kDot2 ? 1 : G][VEC];
  bf16x2 q2[G][VEC / 2];
  float m[G], l[G], acc[G][VEC];
  float kmul;

  // qp: this lane's values of the group's first q head; heads are D = 16 * VEC apart
  __device__ __forceinline__ void init(const QT* qp, float kmul_) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const QT* qh = qp + h * 16 * VEC;
      if constexpr (kDot2) {
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i)
          q2[h][i] = bf16x2{(bf16)load_q<QT>(qh, 2 * i), (bf16)load_q<QT>(qh, 2 * i + 1)};
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) qf[h][i] = load_q<QT>(qh, i);
      }
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[h][i] = 0.f;
    }
    kmul = kmul_;
  }

  // one group: tokens base + STRIDE*u, u < kUnroll (those at or past t1 are masked)
  template <int STRIDE>
  __device__ __forceinline__ void consume(int base, int t1, const Chunk* kc, const Chunk* vc) {
    float sc[kUnroll][G];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool valid = base + STRIDE * u < t1;
      if constexpr (kDot2) {
        bf16x2 kp[VEC / 2];
        kc[u].pairs(kp);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float part = 0.f;
#pragma unroll
          for (int i = 0; i < VEC / 2; ++i) part = __builtin_amdgcn_fdot2_f32_bf16(q2[h][i], kp[i], part, false);
          sc[u][h] = valid ? row16_sum(part) * kmul : -INFINITY;
        }
      } else {
        float kf[VEC];
        kc[u].floats(kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float part = 0.f;
#pragma unroll
          for (int i = 0; i < VEC; ++i) part = fmaf(qf[h][i], kf[i], part);
          sc[u][h] = valid ? row16_sum(part) * kmul : -INFINITY;
        }
      }
    }
    float vf[kUnroll][VEC];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) vc[u].floats(vf[u]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mt = sc[0][h];
#pragma unroll
      for (int u = 1; u < kUnroll; ++u) mt = fmaxf(mt, sc[u][h]);
      const float mn = fmaxf(m[h], mt);
      if (mn == -INFINITY) continue;  // this row has not seen a token yet (uniform within the row)
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
      float pr[kUnroll];
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        pr[u] = __builtin_amdgcn_exp2f(sc[u][h] - mn);  // masked: 2^-inf = 0
        psum += pr[u];
      }
      l[h] = l[h] * alpha + psum;
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        float a = acc[h][i] * alpha;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) a = fmaf(pr[u], vf[u][i], a);
        acc[h][i] = a;
      }
      m[h] = mn;
    }
  }

  // Tokens first, first + STRIDE, ... < t1 in groups of kUnroll, the next group's K/V rows in
  // flight while one is consumed.  With SLOTS_AHEAD the slot numbers are read a group earlier
  // still, so that the next group's row fetch does not wait on a fresh slot lookup (loads
  // complete in issue order, and each group's slots are issued before the previous group's
  // rows): this pays where a workgroup streams few tokens and latency dominates (the short
  // private tails); on long bandwidth-bound streams the plain order is as fast and needs
  // fewer registers.  Past t1 the slot of token t0 is re-read (and masked).
  template <int STRIDE, bool SLOTS_AHEAD>
  __device__ __forceinline__ void run(const int32_t* row, int t0, int t1, int first, const uint8_t* kpool,
                                      const uint8_t* vpool, int64_t slot_bytes, int64_t head_off,
                                      uint32_t max_slot) {
    constexpr int kStep = STRIDE * kUnroll;
    auto slots = [&](int base, uint32_t* sl) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int t = base + STRIDE * u;
        sl[u] = min((uint32_t)row[t < t1 ? t : t0], max_slot);   // a slot past the pool reads the last one
      }
    };
    auto fetch = [&](const uint32_t* sl, Chunk* kc, Chunk* vc) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        kc[u].load(kpool + (int64_t)sl[u] * slot_bytes + head_off);
        vc[u].load(vpool + (int64_t)sl[u] * slot_bytes + head_off);
      }
    };
    if constexpr (!SLOTS_AHEAD) {
      if (first >= t1) return;
      uint32_t sl[kUnroll];
      Chunk ka[kUnroll], va[kUnroll], kb[kUnroll], vb[kUnroll];
      int base = first;
      slots(base, sl);
      fetch(sl, ka, va);
      while (true) {
        slots(base + kStep, sl);
        fetch(sl, kb, vb);
        consume<STRIDE>(base, t1, ka, va);
        base += kStep;
        if (base >= t1) break;
        slots(base + kStep, sl);
        fetch(sl, ka, va);
        consume<STRIDE>(base, t1, kb, vb);
        base += kStep;
        if (base >= t1) break;
      }
    } else {
      if (first >= t1) return;
      uint32_t sa[kUnroll], sb[kUnroll];
      Chunk ka[kUnroll], va[kUnroll], kb[kUnroll], vb[kUnroll];
      int base = first;
      slots(base, sa);
      slots(base + kStep, sb);
      fetch(sa, ka, va);
      while (true) {
        slots(base + 2 * kStep, sa);
        fetch(sb, kb, vb);
        consume<STRIDE>(base, t1, ka, va);
        base += kStep;
        if (base >= t1) break;
        slots(base + 2 * kStep, sb);
        fetch(sa, ka, va);
        consume<STRIDE>(base, t1, kb, vb);
        base += kStep;
        if (base >= t1) break;
      }
    }
  }
};

template <typename QT, int POOL, int D, int G>
__global__ __launch_bounds__(256) void decode_split(const QT* __restrict__ q, const uint8_t* __restrict__ kpool,
                                                    const uint8_t* __restrict__ vpool, const float* __restrict__ kscale,
                                                    const float* __restrict__ vscale,
                                                    const int32_t* __restrict__ r2t, int64_t stride,
                                                    const int32_t* __restrict__ seq_lens, int hkv, int chunk,
                                                    int max_splits, float qk_scale_log2, float* __restrict__ ws_ml,
                                                    float* __restrict__ ws_acc, const int32_t* __restrict__ skip,
                                                    int s0, int ns, uint32_t max_slot) {
  constexpr int VEC = D / 16;
  using Chunk = RowChunk<POOL, VEC>;
  constexpr int ROWB = D * Chunk::kBytes / VEC;  // bytes of one (slot, head) row
  __shared__ float sm_ml[kWaves][G][2];
  __shared__ float sm_acc[kWaves][G][D];

  const int g = blockIdx.x % hkv;
  const int rest = blockIdx.x / hkv;
  const int s = s0 + rest % ns;
  const int b = rest / ns;
  const int L = seq_lens[b];
  const int t0 = s * chunk;
  if (t0 >= L) return;  // the whole workgroup leaves together
  if (skip && s < skip[b]) return;  // chunk computed by the shared-prefix pass
  const int t1 = min(t0 + chunk, L);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, li = lane & 15;
  const int hq = hkv * G;

  float kmul = qk_scale_log2;
  if constexpr (POOL == PKV_FP8_E4M3) kmul *= kscale[g];
  HeadStream<QT, POOL, VEC, G> hs;
  hs.init(q + ((int64_t)b * hq + (int64_t)g * G) * D + li * VEC, kmul);
  const int64_t slot_bytes = (int64_t)hkv * ROWB;
  const int64_t head_off = (int64_t)g * ROWB + li * Chunk::kBytes;
  hs.template run<16, true>(r2t + (int64_t)b * stride, t0, t1, t0 + wave * 4 + grp, kpool, vpool, slot_bytes, head_off,
                      max_slot);
  auto& m = hs.m;
  auto& l = hs.l;
  auto& acc = hs.acc;

  // merge the four 16-lane rows of the wave (lanes li, li+16, li+32, li+48 cover the same d)
#pragma unroll
  for (int off = 16; off <= 32; off *= 2) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m2 = __shfl_xor(m[h], off);
      const float l2 = __shfl_xor(l[h], off);
      float a2[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) a2[i] = __shfl_xor(acc[h][i], off);
      merge_state(m[h], l[h], acc[h], m2, l2, a2, VEC);
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) sm_acc[wave][h][li * VEC + i] = acc[h][i];
      if (li == 0) {
        sm_ml[wave][h][0] = m[h];
        sm_ml[wave][h][1] = l[h];
      }
    }
  }
  __syncthreads();
  const float vmul = POOL == PKV_FP8_E4M3 ? vscale[g] : 1.f;
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int h = e / D, dd = e - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_ml[w][h][0]);
    float a = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_ml[w][h][0];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
      a += f * sm_acc[w][h][dd];
      lsum += f * sm_ml[w][h][1];
    }
    const int64_t part = ((int64_t)b * hq + (int64_t)g * G + h) * max_splits + s;
    ws_acc[part * D + dd] = a * vmul;
    if (dd == 0) {
      ws_ml[part * 2 + 0] = M;
      ws_ml[part * 2 + 1] = lsum;
    }
  }
}

// All kv heads of a sequence in one workgroup: 16 rows of 16 lanes = HKV heads x (16/HKV)
// token streams.  Every token's K (and V) slot row of HKV*d values is then read as one
// contiguous run by the HKV rows of a stream, instead of HKV separate 256-byte pieces
// fetched by different workgroups at different times.  Each stream keeps the next group of
// kUnroll tokens in flight (two register buffers) while it consumes the current one; with a
// bf16 pool the q.k products are packed bf16 dot products.  Streams of one head are merged
// in LDS at the end.  blockIdx.x = (b * ns_odd + s - s0) * groups + group (chunks s0 .. s0 + ns - 1,
// ns_odd = ns rounded up to an odd count).
template <typename QT, int POOL, int D, int G, int HKV>
__global__ __launch_bounds__(256, (G >= 8 ? 2 : 3)) void decode_split_slot(const QT* __restrict__ q, const uint8_t* __restrict__ kpool,
                                                         const uint8_t* __restrict__ vpool,
                                                         const float* __restrict__ kscale,
                                                         const float* __restrict__ vscale,
                                                         const int32_t* __restrict__ r2t, int64_t stride,
                                                         const int32_t* __restrict__ seq_lens, int chunk,
                                                         int max_splits, float qk_scale_log2,
                                                         float* __restrict__ ws_ml, float* __restrict__ ws_acc,
                                                         int hkv_total, const int32_t* __restrict__ skip, int s0,
                                                         int ns, int ns_odd, uint32_t max_slot) {
  constexpr int VEC = D / 16;
  constexpr int STREAMS = 16 / HKV;
  using Chunk = RowChunk<POOL, VEC>;
  constexpr int ROWB = D * Chunk::kBytes / VEC;
  __shared__ float sm_ml[(STREAMS - 1) * HKV][G][2];
  __shared__ float sm_acc[(STREAMS - 1) * HKV][G][D];

  // kv heads in groups of HKV: blockIdx.x = (b * ns_odd + s - s0) * groups + group
  const int groups = hkv_total / HKV;
  const int group = blockIdx.x % groups;
  const int j = (blockIdx.x / groups) % ns_odd;
  const int b = blockIdx.x / groups / ns_odd;
  if (j >= ns) return;  // the padding chunk of an even count
  const int s = s0 + j;
  const int L = seq_lens[b];
  const int t0 = s * chunk;
  if (t0 >= L) return;  // the whole workgroup leaves together
  if (skip && s < skip[b]) return;  // chunk computed by the shared-prefix pass
  const int t1 = min(t0 + chunk, L);
  const int r = threadIdx.x >> 4, li = threadIdx.x & 15;
  const int gl = r % HKV, stream = r / HKV;   // this row's head within the group, token stream
  const int g = group * HKV + gl;
  const int hq = hkv_total * G;

  float kmul = qk_scale_log2;
  if constexpr (POOL == PKV_FP8_E4M3) kmul *= kscale[g];
  HeadStream<QT, POOL, VEC, G> hs;
  hs.init(q + ((int64_t)b * hq + (int64_t)g * G) * D + li * VEC, kmul);
  const int64_t slot_bytes = (int64_t)hkv_total * ROWB;
  const int64_t head_off = (int64_t)g * ROWB + li * Chunk::kBytes;
  hs.template run<STREAMS, false>(r2t + (int64_t)b * stride, t0, t1, t0 + stream, kpool, vpool, slot_bytes, head_off,
                           max_slot);
  auto& m = hs.m;
  auto& l = hs.l;
  auto& acc = hs.acc;

  // merge the streams of each head into stream 0
  if (stream > 0) {
    const int slot_r = (stream - 1) * HKV + gl;
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) sm_acc[slot_r][h][li * VEC + i] = acc[h][i];
      if (li == 0) {
        sm_ml[slot_r][h][0] = m[h];
        sm_ml[slot_r][h][1] = l[h];
      }
    }
  }
  __syncthreads();
  if (stream == 0) {
    const float vmul = POOL == PKV_FP8_E4M3 ? vscale[g] : 1.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      for (int st = 1; st < STREAMS; ++st) {
        const int slot_r = (st - 1) * HKV + gl;
        float a2[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) a2[i] = sm_acc[slot_r][h][li * VEC + i];
        merge_state(m[h], l[h], acc[h], sm_ml[slot_r][h][0], sm_ml[slot_r][h][1], a2, VEC);
      }
      const int64_t part = ((int64_t)b * hq + (int64_t)g * G + h) * max_splits + s;
#pragma unroll
      for (int i = 0; i < VEC; ++i) ws_acc[part * D + li * VEC + i] = acc[h][i] * vmul;
      if (li == 0) {
        ws_ml[part * 2 + 0] = m[h];
        ws_ml[part * 2 + 1] = l[h];
      }
    }
  }
}

template <typename OT>
__device__ __forceinline__ void store_o(OT* p, float v);
template <>
__device__ __forceinline__ void store_o<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_o<bf16>(bf16* p, float v) { *p = (bf16)v; }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) x += __shfl_xor(x, off);
  return x;
}

// One wave per (sequence, q head): merge that head's chunk partials.  A partial with running
// max -inf is empty (a later chunk of a shared-prefix span): it has no weight and its row,
// never written, is not read.  The (m, l) pairs of the first 64 R chunks come in with R loads
// per lane, all in flight together, and stay in registers; the rows of the partials that
// carry weight (found with a ballot per 64 chunks) are then gathered U at a time with all U
// loads in flight, so a sequence with many chunks, most of them empty, costs a few round
// trips rather than one per group of chunks.
// U and R are template parameters: a launch whose sequences have at most 64 chunks takes
// (U, R) = (8, 1), so the registers of the long-context gathers do not cost it occupancy.
template <typename OT, int D, int U, int R>
__global__ __launch_bounds__(256) void decode_reduce(const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
                                                     const int32_t* __restrict__ seq_lens, int batch, int hq,
                                                     int chunk, int max_splits, OT* __restrict__ o) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (idx >= batch * hq) return;
  const int b = idx / hq;
  const int ns = min((seq_lens[b] + chunk - 1) / chunk, max_splits);
  const float* ml = ws_ml + (int64_t)idx * max_splits * 2;
  const float* acc = ws_acc + (int64_t)idx * max_splits * D + lane * PER;
  float mr[R], lr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int s = lane + 64 * r;
    const float2 v = s < ns ? *(const float2*)(ml + 2 * s) : float2{-INFINITY, 0.f};
    mr[r] = v.x;
    lr[r] = v.y;
  }
  float M = mr[0];
#pragma unroll
  for (int r = 1; r < R; ++r) M = fmaxf(M, mr[r]);
  for (int s = lane + 64 * R; s < ns; s += 64) M = fmaxf(M, ml[2 * s]);
  M = wave_max(M);
  float lsum = 0.f;
  float out[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) out[i] = 0.f;
  for (int s0 = 0, r = 0; s0 < ns; s0 += 64, ++r) {
    const int s = s0 + lane;
    float m, l;
    if (r < R) {   // the same in every lane
      m = mr[0];
      l = lr[0];
#pragma unroll
      for (int k = 1; k < R; ++k)
        if (r == k) {
          m = mr[k];
          l = lr[k];
        }
    } else {
      m = s < ns ? ml[2 * s] : -INFINITY;
      l = s < ns ? ml[2 * s + 1] : 0.f;
    }
    const bool used = m != -INFINITY;
    const float w = used ? exp2f(m - M) : 0.f;
    if (used) lsum = fmaf(w, l, lsum);
    uint64_t mask = __ballot(used);   // the same in every lane
    // U rows at a time: many partials in 32s, the last few in 8s
    auto gather = [&](auto uu) {
      constexpr int UU = decltype(uu)::value;
      const int j0 = __builtin_ctzll(mask);
      int js[UU];
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        js[u] = mask ? __builtin_ctzll(mask) : -1;   // -1: padding, weight 0, re-reads chunk j0
        mask &= mask - 1;
      }
      float av[UU][PER];
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        const int j = js[u] < 0 ? j0 : js[u];
#pragma unroll
        for (int i = 0; i < PER; ++i) av[u][i] = acc[(int64_t)(s0 + j) * D + i];
      }
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        const float wu = js[u] < 0 ? 0.f : __shfl(w, js[u]);
#pragma unroll
        for (int i = 0; i < PER; ++i) out[i] = fmaf(wu, av[u][i], out[i]);
      }
    };
    if constexpr (U > 8)
      while (__builtin_popcountll(mask) > 8) gather(std::integral_constant<int, U>{});
    while (mask) gather(std::integral_constant<int, 8>{});
  }
  lsum = wave_sum(lsum);
  const float inv = 1.f / lsum;
#pragma unroll
  for (int i = 0; i < PER; ++i) store_o<OT>(o + (int64_t)idx * D + lane * PER + i, out[i] * inv);
}

template <typename QT, int POOL, int D, int HKV>
int launch_slot(int G, int batch, int s0, int ns, hipStream_t st, const void* q, const void* kp, const void* vp,
                const float* ks, const float* vs, const int32_t* r2t, int64_t stride, const int32_t* lens, int chunk,
                int max_splits, float sc, float* ml, float* acc, int hkv_total, const int32_t* skip,
                uint32_t max_slot) {
  const int ns_odd = ns | 1;
  const dim3 grid((unsigned)((int64_t)batch * ns_odd * (hkv_total / HKV)));
#define PKV_SLOT_CASE(GG)                                                                                        \
  case GG:                                                                                                       \
    hipLaunchKernelGGL((decode_split_slot<QT, POOL, D, GG, HKV>), grid, dim3(256), 0, st, (const QT*)q,          \
                       (const uint8_t*)kp, (const uint8_t*)vp, ks, vs, r2t, stride, lens, chunk, max_splits, sc, \
                       ml, acc, hkv_total, skip, s0, ns, ns_odd, max_slot);                                      \
    return PKV_OK;
  switch (G) {
    PKV_SLOT_CASE(1)
    PKV_SLOT_CASE(2)
    PKV_SLOT_CASE(4)
    PKV_SLOT_CASE(8)
    default:
      return fail(PKV_ERR_UNSUPPORTED, "decode: group size %d", G);
  }
#undef PKV_SLOT_CASE
}

template <typename QT, int POOL, int D>
int launch_split(int G, int batch, int s0, int ns, bool per_head, hipStream_t st, const void* q, const void* kp,
                 const void* vp, const float* ks, const float* vs, const int32_t* r2t, int64_t stride,
                 const int32_t* lens, int hkv, int chunk, int max_splits, float sc, float* ml, float* acc,
                 const int32_t* skip, uint32_t max_slot) {
#define PKV_DECODE_CASE(GG)                                                                                    \
  case GG:                                                                                                     \
    hipLaunchKernelGGL((decode_split<QT, POOL, D, GG>), dim3((unsigned)((int64_t)batch * ns * hkv)), dim3(256), 0, \
                       st, (const QT*)q, (const uint8_t*)kp, (const uint8_t*)vp, ks, vs, r2t, stride, lens, hkv,  \
                       chunk, max_splits, sc, ml, acc, skip, s0, ns, max_slot);                                \
    return PKV_OK;
  // all heads of a slot row per workgroup for 2, 4 or 8 kv heads; groups of 8 heads for
  // any multiple of 8 (multi-head attention)
  if (!per_head) {
    if (hkv == 8) return launch_slot<QT, POOL, D, 8>(G, batch, s0, ns, st, q, kp, vp, ks, vs, r2t, stride, lens, chunk,
                                                    max_splits, sc, ml, acc, hkv, skip, max_slot);
    if (hkv == 4) return launch_slot<QT, POOL, D, 4>(G, batch, s0, ns, st, q, kp, vp, ks, vs, r2t, stride, lens, chunk,
                                                    max_splits, sc, ml, acc, hkv, skip, max_slot);
    if (hkv == 2) return launch_slot<QT, POOL, D, 2>(G, batch, s0, ns, st, q, kp, vp, ks, vs, r2t, stride, lens, chunk,
                                                    max_splits, sc, ml, acc, hkv, skip, max_slot);
    if (hkv % 8 == 0)
      return launch_slot<QT, POOL, D, 8>(G, batch, s0, ns, st, q, kp, vp, ks, vs, r2t, stride, lens, chunk,
                                         max_splits, sc, ml, acc, hkv, skip, max_slot);
  }
  switch (G) {
    PKV_DECODE_CASE(1)
    PKV_DECODE_CASE(2)
    PKV_DECODE_CASE(4)
    PKV_DECODE_CASE(8)
    default:
      return fail(PKV_ERR_UNSUPPORTED, "decode: group size %d", G);
  }
#undef PKV_DECODE_CASE
}

int splits_for(int max_seq_len, int chunk) { return (max_seq_len + chunk - 1) / chunk; }

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int32_t pkv_decode_chunk(int32_t batch, int32_t hkv, int32_t max_seq_len) {
  // workgroups per (sequence, chunk): one for all kv heads when hkv is 2, 4 or 8, else one per head
  const int64_t per_chunk = (hkv == 2 || hkv == 4 || hkv == 8) ? 1 : (hkv % 8 == 0 ? hkv / 8 : hkv);
  int chunk = 1024;
  while (chunk > 128 && (int64_t)batch * per_chunk * splits_for(max_seq_len, chunk) < 2048) chunk /= 2;
  return chunk;
}

extern "C" size_t pkv_decode_workspace_bytes(int32_t batch, int32_t hq, int32_t d, int32_t max_seq_len,
                                             int32_t chunk) {
  if (batch <= 0 || hq <= 0 || d <= 0 || max_seq_len <= 0) return 0;
  if (chunk <= 0) chunk = 1024;
  const size_t parts = (size_t)batch * hq * splits_for(max_seq_len, chunk);
  return parts * (2 + (size_t)d) * sizeof(float);
}

extern "C" int32_t pkv_decode_shared_rows(int32_t qo_dtype, int32_t pool_dtype, int32_t hq, int32_t hkv, int32_t d) {
  if (hq <= 0 || hkv <= 0 || hq % hkv) return PKV_ERR_INVAL;
  const int G = hq / hkv;
  if (qo_dtype == PKV_BF16 && (pool_dtype == PKV_BF16 || pool_dtype == PKV_FP8_E4M3) && d == 128 &&
      (G == 1 || G == 2 || G == 4 || G == 8) && hkv * (pool_dtype == PKV_FP8_E4M3 ? 128 : 256) <= 16383)
    return 128 / G;
  return PKV_ERR_UNSUPPORTED;
}

namespace {

int decode_impl(const void* q, void* o, int32_t qo_dtype, const void* k_pool, const void* v_pool, int32_t pool_dtype,
                int64_t num_slots, const float* k_scale, const float* v_scale, const int32_t* req_to_token,
                int64_t stride, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, int32_t hq, int32_t hkv,
                int32_t d, float sm_scale, int32_t chunk, const int32_t* members, const int32_t* skip,
                const int32_t* items, int64_t n_items, int32_t first_split, void* workspace, size_t ws_bytes,
                void* stream) {
  if (batch < 0 || hq <= 0 || hkv <= 0 || hq % hkv || max_seq_len <= 0 || max_seq_len > stride || num_slots <= 0)
    return fail(PKV_ERR_INVAL, "decode: bad sizes (batch %d hq %d hkv %d max_seq_len %d stride %lld)", batch, hq,
                hkv, max_seq_len, (long long)stride);
  if (batch == 0) return PKV_OK;
  if (!q || !o || !k_pool || !v_pool || !req_to_token || !seq_lens || !workspace)
    return fail(PKV_ERR_INVAL, "decode: null pointer");
  if (chunk == 0) chunk = pkv_decode_chunk(batch, hkv, max_seq_len);
  if (chunk < 64 || chunk % 64) return fail(PKV_ERR_INVAL, "decode: chunk %d is not a positive multiple of 64", chunk);
  if (ws_bytes < pkv_decode_workspace_bytes(batch, hq, d, max_seq_len, chunk))
    return fail(PKV_ERR_INVAL, "decode: workspace of %zu bytes is too small", ws_bytes);
  if (pool_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return fail(PKV_ERR_INVAL, "decode: fp8 pool needs scales");
  const int G = hq / hkv;
  const int max_splits = splits_for(max_seq_len, chunk);
  if ((int64_t)batch * (max_splits | 1) * hkv > 0x7FFFFFFFLL)
    return fail(PKV_ERR_UNSUPPORTED, "decode: %d sequences x %d chunks x %d kv heads is beyond one launch", batch,
                max_splits, hkv);
  float* ml = (float*)workspace;
  float* acc = ml + (size_t)batch * hq * max_splits * 2;
  hipStream_t st = (hipStream_t)stream;
  const float sc = sm_scale * kLog2e;
  // split phase over chunks s0 .. max_splits - 1.  After a shared-prefix pass only short
  // private tails may be left: when the all-heads kernel would then launch too few
  // workgroups to fill the GPU (counting its head groups), the per-head kernel (16 token
  // streams each) takes them.
  // A plan whose items cover every chunk (first_split >= max_splits) leaves no split phase.
  const int s0 = skip ? std::min(std::max(first_split, 0), max_splits - 1) : 0;
  const int ns = max_splits - s0;
  const int slot_groups = (hkv == 2 || hkv == 4 || hkv == 8) ? 1 : (hkv % 8 == 0 ? hkv / 8 : 0);
  const bool per_head = skip && (int64_t)batch * ns * slot_groups < 1024;
  const bool split_phase = !skip || first_split < max_splits;
  if (num_slots > 0x7FFFFFFFLL) return fail(PKV_ERR_INVAL, "decode: num_slots beyond int32");
  const uint32_t mslot = (uint32_t)(num_slots - 1);
  int rc = PKV_OK;
  if (!split_phase)
    rc = PKV_OK;
  else if (qo_dtype == PKV_F32 && pool_dtype == PKV_F32 && d == 64)
    rc = launch_split<float, PKV_F32, 64>(G, batch, s0, ns, per_head, st, q, k_pool, v_pool, k_scale, v_scale, req_to_token, stride,
                                          seq_lens, hkv, chunk, max_splits, sc, ml, acc, skip, mslot);
  else if (qo_dtype == PKV_F32 && pool_dtype == PKV_F32 && d == 128)
    rc = launch_split<float, PKV_F32, 128>(G, batch, s0, ns, per_head, st, q, k_pool, v_pool, k_scale, v_scale, req_to_token, stride,
                                           seq_lens, hkv, chunk, max_splits, sc, ml, acc, skip, mslot);
  else if (qo_dtype == PKV_BF16 && pool_dtype == PKV_BF16 && d == 64)
    rc = launch_split<bf16, PKV_BF16, 64>(G, batch, s0, ns, per_head, st, q, k_pool, v_pool, k_scale, v_scale, req_to_token, stride,
                                          seq_lens, hkv, chunk, max_splits, sc, ml, acc, skip, mslot);
  else if (qo_dtype == PKV_BF16 && pool_dtype == PKV_FP8_E4M3 && d == 64)
    rc = launch_split<bf16, PKV_FP8_E4M3, 64>(G, batch, s0, ns, per_head, st, q, k_pool, v_pool, k_scale, v_scale, req_to_token,
                                              stride, seq_lens, hkv, chunk, max_splits, sc, ml, acc, skip, mslot);
  else if (qo_dtype == PKV_BF16 && pool_dtype == PKV_BF16 && d == 128)
    rc = launch_split<bf16, PKV_BF16, 128>(G, batch, s0, ns, per_head, st, q, k_pool, v_pool, k_scale, v_scale, req_to_token, stride,
                                           seq_lens, hkv, chunk, max_splits, sc, ml, acc, skip, mslot);
  else if (qo_dtype == PKV_BF16 && pool_dtype == PKV_FP8_E4M3 && d == 128)
    rc = launch_split<bf16, PKV_FP8_E4M3, 128>(G, batch, s0, ns, per_head, st, q, k_pool, v_pool, k_scale, v_scale, req_to_token,
                                               stride, seq_lens, hkv, chunk, max_splits, sc, ml, acc, skip, mslot);
  else
    return fail(PKV_ERR_UNSUPPORTED, "decode: qo dtype %d, pool dtype %d, d %d", qo_dtype, pool_dtype, d);
  if (rc < 0) return rc;
  if (split_phase) {
    rc = hip_check(hipGetLastError(), "decode split launch");
    if (rc < 0) return rc;
  }
  if (n_items > 0) {
    rc = launch_decode_shared(q, pool_dtype, k_pool, v_pool, k_scale, v_scale, num_slots, req_to_token, stride, batch,
                              seq_lens, members, items, n_items, chunk, max_splits, hq, hkv, sc, ml, acc, st);
    if (rc < 0) return rc;
  }
  const dim3 rgrid((unsigned)(((int64_t)batch * hq + kWaves - 1) / kWaves));
  const bool few = max_splits <= 64;
#define PKV_REDUCE(OT, DD)                                                                                     \
  if (few)                                                                                                   \
    hipLaunchKernelGGL((decode_reduce<OT, DD, 8, 1>), rgrid, dim3(256), 0, st, ml, acc, seq_lens, batch, hq, chunk, \
                       max_splits, (OT*)o);                                                                  \
  else                                                                                                       \
    hipLaunchKernelGGL((decode_reduce<OT, DD, 32, 4>), rgrid, dim3(256), 0, st, ml, acc, seq_lens, batch, hq,     \
                       chunk, max_splits, (OT*)o);
  if (qo_dtype == PKV_F32 && d == 64) {
    PKV_REDUCE(float, 64)
  } else if (qo_dtype == PKV_F32) {
    PKV_REDUCE(float, 128)
  } else if (d == 64) {
    PKV_REDUCE(bf16, 64)
  } else {
    PKV_REDUCE(bf16, 128)
  }
#undef PKV_REDUCE
  return hip_check(hipGetLastError(), "decode reduce launch");
}

}  // namespace

extern "C" int pkv_decode_attention(const void* q, void* o, int32_t qo_dtype, const void* k_pool, const void* v_pool,
                                    int32_t pool_dtype, int64_t num_slots, const float* k_scale, const float* v_scale,
                                    const int32_t* req_to_token, int64_t stride, const int32_t* seq_lens,
                                    int32_t batch, int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d,
                                    float sm_scale, int32_t chunk, void* workspace, size_t ws_bytes, void* stream) {
  return decode_impl(q, o, qo_dtype, k_pool, v_pool, pool_dtype, num_slots, k_scale, v_scale, req_to_token, stride,
                     seq_lens, batch, max_seq_len, hq, hkv, d, sm_scale, chunk, nullptr, nullptr, nullptr, 0, 0,
                     workspace, ws_bytes, stream);
}

extern "C" int pkv_decode_attention_shared(const void* q, void* o, int32_t qo_dtype, const void* k_pool,
                                           const void* v_pool, int32_t pool_dtype, int64_t num_slots,
                                           const float* k_scale, const float* v_scale, const int32_t* req_to_token,
                                           int64_t stride, const int32_t* seq_lens, int32_t batch,
                                           int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                                           int32_t chunk, const int32_t* members, const int32_t* skip,
                                           const int32_t* items, int64_t n_items, int32_t first_split,
                                           void* workspace, size_t ws_bytes, void* stream) {
  if (n_items < 0) return fail(PKV_ERR_INVAL, "decode: n_items %lld", (long long)n_items);
  if (n_items > 0 && batch > 0) {
    if (!members || !skip || !items) return fail(PKV_ERR_INVAL, "decode: null shared-prefix plan");
    if (chunk <= 0) return fail(PKV_ERR_INVAL, "decode: a shared-prefix plan needs the chunk it was made for");
    if (pkv_decode_shared_rows(qo_dtype, pool_dtype, hq, hkv, d) < 0)
      return fail(PKV_ERR_UNSUPPORTED, "decode: no shared-prefix kernel for qo dtype %d, pool dtype %d, hq %d, hkv %d, d %d",
                  qo_dtype, pool_dtype, hq, hkv, d);
  }
  return decode_impl(q, o, qo_dtype, k_pool, v_pool, pool_dtype, num_slots, k_scale, v_scale, req_to_token, stride,
                     seq_lens, batch, max_seq_len, hq, hkv, d, sm_scale, chunk, members, n_items > 0 ? skip : nullptr,
                     items, n_items, first_split, workspace, ws_bytes, stream);
}

// ------------------------------------------------------------------------------------------
// Decode without a caller workspace: the split partials go to a file-scope device array.
// ------------------------------------------------------------------------------------------
//
// For callers that cannot allocate (code under graph capture, tight serving loops): the
// partials of pkv_decode_attention_shared live in `scratch`, one copy per GPU, held until the
// process ends.  In host code the array's name is only a stand-in, so its device address is
// taken once per device with hipGetSymbolAddress (with that device current) and that address
// is what the kernels get.  Every call on a GPU shares its array: calls that overlap on one GPU
// race.  Nothing needs clearing between calls: every partial the reduce reads is written by
// the split phase or a plan item of the same call (the array keeps the last call's partials).

static __device__ __align__(256) char scratch[PKV_DECODE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
int g_scratch_rc[kMaxDevices];

int scratch_for_current_device(void** out) {
  int dev = 0;
  if (int rc = hip_check(hipGetDevice(&dev), "decode (static): hipGetDevice")) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "decode (static): device %d", dev);
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_rc[dev] = e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
    g_scratch_ptr[dev] = e == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_rc[dev] != PKV_OK || !g_scratch_ptr[dev])
    return fail(PKV_ERR_HIP, "decode (static): hipGetSymbolAddress of the scratch array failed on device %d", dev);
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_decode_attention_static(const void* q, void* o, int32_t qo_dtype, const void* k_pool,
                                           const void* v_pool, int32_t pool_dtype, int64_t num_slots,
                                           const float* k_scale, const float* v_scale, const int32_t* req_to_token,
                                           int64_t stride, const int32_t* seq_lens, int32_t batch,
                                           int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                                           int32_t chunk, const int32_t* members, const int32_t* skip,
                                           const int32_t* items, int64_t n_items, int32_t first_split,
                                           void* stream) {
  if (batch < 0 || hq <= 0 || hkv <= 0 || max_seq_len <= 0)
    return fail(PKV_ERR_INVAL, "decode (static): bad sizes (batch %d hq %d hkv %d max_seq_len %d)", batch, hq, hkv,
                max_seq_len);
  if (batch == 0) return PKV_OK;
  if (chunk == 0) {
    // the automatic chunk; for a plain decode (no plan, whose items and first split are tied to
    // its chunk) doubled while the partials would not fit the array
    chunk = pkv_decode_chunk(batch, hkv, max_seq_len);
    while (n_items == 0 && first_split == 0 &&
           pkv_decode_workspace_bytes(batch, hq, d, max_seq_len, chunk) > (size_t)PKV_DECODE_STATIC_SCRATCH_BYTES &&
           chunk < max_seq_len)
      chunk *= 2;
  }
  const size_t need = pkv_decode_workspace_bytes(batch, hq, d, max_seq_len, chunk);
  if (need > (size_t)PKV_DECODE_STATIC_SCRATCH_BYTES)
    return fail(PKV_ERR_INVAL,
                "decode (static): %d sequences x %d q heads over %d tokens in chunks of %d need %zu bytes of partials, "
                "more than the %lld-byte static scratch array",
                batch, hq, max_seq_len, chunk, need, (long long)PKV_DECODE_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int rc = scratch_for_current_device(&ws)) return rc;
  return pkv_decode_attention_shared(q, o, qo_dtype, k_pool, v_pool, pool_dtype, num_slots, k_scale, v_scale,
                                     req_to_token, stride, seq_lens, batch, max_seq_len, hq, hkv, d, sm_scale, chunk,
                                     members, skip, items, n_items, first_split, ws,
                                     (size_t)PKV_DECODE_STATIC_SCRATCH_BYTES, stream);
}
