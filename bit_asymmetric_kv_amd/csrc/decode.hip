// Decode-step attention read directly from the packed low-bit cache.
//
// Decode reads the whole cache at every step; the pages describe it as bound by
// memory traffic ("Read What Matters", the NOVA-KV and RDKV abstracts; "KV cache
// quantization: putting the bits in the cached vectors", the KIVI abstract on the
// compute core idling while the cache loads). On gfx950 this kernel is bound by
// instruction issue instead: per 32-token group a wave spends 64 code conversions
// and 16 MFMAs on 3 KB of cache. Scores over the quantized groups and over the FP16
// residual are combined inside one attention computation (same page, full-text-skim
// notes on KIVI's grouped/residual split).
//
// Work split (flash-decoding style): one workgroup per (sequence split of whole
// groups, kv-head, sequence) plus, per (kv-head, sequence), the FP16 window's
// workgroups (four 32-token chunks each, one per wave); each writes partial (max,
// sum, unnormalized output) per query head, and a second kernel merges them.
//
// Inside a split each wave streams whole 32-token groups straight into registers,
// issued three groups ahead of the group whose value side runs (two ahead of its
// key side). Every group block is read from HBM once and serves all query heads of
// the kv-head:
//  * scores: an MFMA 16x16x32 f16 contraction over channels with the key codes as
//    A (converted exactly to f16 by the scaled fp4/fp8 conversions) and, as B, the
//    query multiplied by the group's per-channel key scale, split into fp16 high and
//    low parts (two columns per head, so the product keeps ~21 bits); the key
//    zero-points enter through q.z, computed once per group per head;
//  * values: an MFMA contraction over the group's tokens with the value codes as A
//    and, as B, the softmax weight times the per-token value scale (again high/low
//    columns); the value zero-points enter through sum_t p_t z_t per channel group.
#include <cstddef>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kD = kHeadDim;
constexpr int kG = kGroup;
constexpr int kWaves = 4;
// Headroom of the split kernel's softmax reference above the running maximum, in
// log2 units (a factor of 4).
constexpr float kRefSlack = 2.0f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

struct DecodeArgs {
  GroupStore store;  // packed group blocks (contiguous or paged)
  __half* ringk;  // written only by a folded append, for its new window tokens
  __half* ringv;
  const SeqDesc* seq;
  const __half* q;
  float* part;
  int B, Hkv, Hq, W, gps, rotate;
  int RS, sink;  // ring slots per (sequence, kv-head): W, plus slot W for an attention sink
  int wblocks;   // FP16-window workgroups per (sequence, kv-head)
  SplitPlan plan;  // split workgroups per sequence and the partial slots per query head
  AppendArgs app;  // an append folded into this launch (app.pending)
  float scale_log2;
  // Pre-RoPE keys: cos / sin of the rotary angles at every group start position
  // o + 32 g ([g][cos 64 | sin 64] fp32) and at the in-group offsets i = 0..31
  // ([i][cos 64 | sin 64]); null without RoPE.
  const float* rope_tab;
  const float* rope_in;
};

// 8 two-bit codes of one MFMA operand: `m` holds them in bits 0-1 and 4-5 of each
// byte (the other bits already masked off). As fp4 (e2m1) a nibble 00cc is c/2, so
// the scaled conversion with scale 2 returns c exactly.
__device__ inline half8 codes2_to_half8(uint32_t m) {
  half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 0);
  half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 1);
  half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 2);
  half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 3);
  half8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 8 four-bit codes in one word (slot s at bit 8*(s%4) + 4*(s/4)). A byte holding
// c in 0..15 reads as fp8 e4m3 c * 2^-9; the scaled conversion with 512 returns c.
__device__ inline half8 codes4_to_half8(uint32_t w) {
  uint32_t m0 = w & 0x0F0F0F0Fu, m1 = (w >> 4) & 0x0F0F0F0Fu;
  half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m0, 512.0f, false);
  half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m0, 512.0f, true);
  half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m1, 512.0f, false);
  half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m1, 512.0f, true);
  half8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Operand o (0..7) of a lane's code section.
template <int BITS>
__device__ inline half8 code_operand(const uint4& w0, const uint4& w1, int o) {
  if constexpr (BITS == 2) {
    uint32_t w = (o / 2 == 0) ? w0.x : (o / 2 == 1) ? w0.y : (o / 2 == 2) ? w0.z : w0.w;
    return codes2_to_half8((w >> (2 * (o % 2))) & 0x33333333u);
  } else if constexpr (BITS == 3) {
    // bits 0-1 from the 2-bit plane (w0), bit 2 from the 1-bit plane (w1.x, w1.y);
    // both in the 4-bit nibble order, so the 4-bit conversion finishes the job
    const uint32_t w = (o / 2 == 0) ? w0.x : (o / 2 == 1) ? w0.y : (o / 2 == 2) ? w0.z : w0.w;
    const uint32_t hw = o < 4 ? w1.x : w1.y;
    const uint32_t lo = (w >> (2 * (o % 2))) & 0x33333333u;
    const uint32_t hi = (hw >> (o % 4)) & 0x11111111u;
    return codes4_to_half8(lo | (hi << 2));
  } else {
    const uint4& v = o < 4 ? w0 : w1;
    uint32_t w = (o % 4 == 0) ? v.x : (o % 4 == 1) ? v.y : (o % 4 == 2) ? v.z : v.w;
    return codes4_to_half8(w);
  }
}

// Value held by the lane of the paired column inside a block of U columns, for the
// mirror layout u <-> U - 1 - u (u = lane % U) used to pair high and low parts.
template <int U>
__device__ inline float partner(float x) {
  const int xi = __builtin_bit_cast(int, x);
  int r;
  if constexpr (U == 2) r = __builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, false);        // quad_perm 1,0,3,2
  else if constexpr (U == 4) r = __builtin_amdgcn_update_dpp(0, xi, 0x1B, 0xF, 0xF, false);   // quad_perm 3,2,1,0
  else if constexpr (U == 8) r = __builtin_amdgcn_update_dpp(0, xi, 0x141, 0xF, 0xF, false);  // row_half_mirror
  else r = __builtin_amdgcn_update_dpp(0, xi, 0x140, 0xF, 0xF, false);                         // row_mirror
  return __builtin_bit_cast(float, r);
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ inline float wave_max_rows(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float wave_sum_rows(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Max over the four quads of a 16-lane row for lanes with equal lane % 4.
__device__ inline float row_max_stride4(float x) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false)));
  return x;
}

// Max / sum over the lanes of a 16-lane row with equal lane % (16 / NR) (DPP row
// rotations by 2, 4 and 8).
template <int CTRL>
__device__ inline float row_rot(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int NR>
__device__ inline float row_class_max(float x) {
  if constexpr (NR >= 8) x = fmaxf(x, row_rot<0x122>(x));
  if constexpr (NR >= 4) x = fmaxf(x, row_rot<0x124>(x));
  if constexpr (NR >= 2) x = fmaxf(x, row_rot<0x128>(x));
  return x;
}
template <int NR>
__device__ inline float row_class_sum(float x) {
  if constexpr (NR >= 8) x += row_rot<0x122>(x);
  if constexpr (NR >= 4) x += row_rot<0x124>(x);
  if constexpr (NR >= 2) x += row_rot<0x128>(x);
  return x;
}

// Sum over the four quads of a 16-lane row for lanes with equal lane % 4
// (DPP row rotations by 4 and 8).
__device__ inline float row_sum_stride4(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
  return x;
}

// (hi, lo) fp16 operand pair of the products x_i = a[i] * s[i], i = 0..7, with
// hi + lo = x to about 21 bits: hi = fp16(ah[i] * s[i]) with ah an fp16 copy of a
// (packed fp16 multiply), lo = fp16(a[i] * s[i] - hi[i]) with the residual formed by
// one fused fp32 operation (so hi may be any nearby fp16 value). Mixed-precision
// fused forms that round straight to fp16 are several times slower on this hardware
// than these; the empty asm keeps the compiler from forming them.
__device__ inline void split_products(const float* a, const half8& ah, const half8& s, half8& hi, half8& lo) {
  hi = ah * s;
  for (int i = 0; i < 8; i += 2) {
    const float l0 = __builtin_fmaf(a[i], float(s[i]), -float(hi[i]));
    const float l1 = __builtin_fmaf(a[i + 1], float(s[i + 1]), -float(hi[i + 1]));
    float m0 = l0, m1 = l1;
    asm("" : "+v"(m0), "+v"(m1));
    lo[i] = _Float16(m0);
    lo[i + 1] = _Float16(m1);
  }
}

// Low parts round to nearest even: their rounding errors, unlike those of a
// truncation, do not share a sign and so do not add up over many tokens.
__device__ inline half8 to_half8_rne(const float* a) {
  half8 r;
  for (int i = 0; i < 8; i += 2) {
    float m0 = a[i], m1 = a[i + 1];
    asm("" : "+v"(m0), "+v"(m1));  // keeps the conversion a plain packed one
    r[i] = _Float16(m0);
    r[i + 1] = _Float16(m1);
  }
  return r;
}

// fp16 copies that serve as high parts (of q, p, rotated keys), rounded toward zero
// by the one-instruction packed conversion: whatever the high part misses, the low
// part computed from it carries.
__device__ inline half8 to_half8(const float* a) {
  half8 r;
  for (int i = 0; i < 8; i += 2) {
    const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(a[i], a[i + 1]));
    r[i] = h[0];
    r[i + 1] = h[1];
  }
  return r;
}

__device__ inline half8 load_half8(const uint8_t* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(half8, u);
}

// Group-block bytes are read once per decode call: non-temporal loads, so that they
// do not displace what is reused (the query, the arguments, the partials). Measured
// 1-3 % faster than plain loads over the 128K, 1M, 32K-batch and ragged workloads.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 stream_load16(const uint8_t* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ inline half8 stream_half8(const uint8_t* p) { return __builtin_bit_cast(half8, stream_load16(p)); }
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ inline uint2 stream_load8(const uint8_t* p) {
  return __builtin_bit_cast(uint2, __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)));
}

// Query preparation shared by all workgroups of one (kv-head, sequence): load the
// HG query rows, rotate (normalized Walsh-Hadamard, fp32) if the cache rotates,
// fold in softmax_scale * log2(e), and scale each head by a power of two 2^-e so
// that its largest entry is below 1 (keeps the fp16 high/low parts in range).
template <int HG>
__device__ void prepare_query(const DecodeArgs& a, int b, int h, float (*qf)[kD], float* expo) {
  for (int e = threadIdx.x; e < HG * kD; e += blockDim.x) {
    int hh = e / kD, d = e % kD;
    qf[hh][d] = __half2float(a.q[(size_t(b) * a.Hq + h * HG + hh) * kD + d]);
  }
  __syncthreads();
  if (a.rotate) {
    for (int hs = 1; hs < kD; hs <<= 1) {
      for (int p = threadIdx.x; p < HG * kD / 2; p += blockDim.x) {
        int hh = p / (kD / 2), j = p % (kD / 2);
        int ia = (j / hs) * (2 * hs) + (j % hs);
        float x = qf[hh][ia], y = qf[hh][ia + hs];
        qf[hh][ia] = x + y;
        qf[hh][ia + hs] = x - y;
      }
      __syncthreads();
    }
  }
  const float post = a.scale_log2 * (a.rotate ? 0x1.6a09e6p-4f : 1.0f);
  for (int e = threadIdx.x; e < HG * kD; e += blockDim.x) qf[e / kD][e % kD] *= post;
  __syncthreads();
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int hh = wave; hh < HG; hh += kWaves) {
    float m = fmaxf(fabsf(qf[hh][lane]), fabsf(qf[hh][lane + 64]));
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    int ex = 0;
    if (m > 0.0f) frexpf(m, &ex);
    qf[hh][lane] = ldexpf(qf[hh][lane], -ex);
    qf[hh][lane + 64] = ldexpf(qf[hh][lane + 64], -ex);
    if (lane == 0) expo[hh] = ldexpf(1.0f, ex);
  }
  __syncthreads();
}

// Split workgroups of each kv-head of sequence b.
__device__ inline int splits_of(const SplitPlan& p, int b) {
  return p.use_prefix ? p.count[b] : p.uniform;
}

// Partial of one query head: running max m (log2 domain), sum l, output o[128].
__device__ inline float* partial_ptr(const DecodeArgs& a, int b, int hq, int split) {
  return a.part + ((size_t(b) * a.Hq + hq) * size_t(a.plan.pstride) + split) * kPartialStride;
}

// Per-wave partials (m, l, o[128] per head) in shared memory; wave w's block starts
// at base + w * stride floats.
struct WaveParts {
  float* base;
  int stride;
  __device__ float& at(int w, int hh, int c) const { return base[w * stride + hh * kPartialStride + c]; }
};

// exp2 of a non-positive argument (a softmax weight or rescale factor): the hardware
// instruction; -inf gives 0, and results below the fp32 normal range, which it may
// flush, are negligible next to the weight 1 of the maximum.
__device__ inline float exp2_nonpos(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge the per-wave partials and write the workgroup's partial. The factor
// 2^(m_w - M) of wave w is formed once per query head; a wave without tokens (m_w =
// -inf) has no o entries and is skipped.
template <int HG>
__device__ void merge_and_store(const DecodeArgs& a, int b, int h, int split, const WaveParts& wp) {
  __shared__ float fac[HG][kWaves + 1];  // per head: the waves' factors, then M
  __syncthreads();
  if (threadIdx.x < HG) {
    const int hh = threadIdx.x;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; w++) M = fmaxf(M, wp.at(w, hh, 0));
    for (int w = 0; w < kWaves; w++) {
      const float mw = wp.at(w, hh, 0);
      fac[hh][w] = mw == -INFINITY ? 0.0f : exp2_nonpos(mw - M);
    }
    fac[hh][kWaves] = M;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < HG * kPartialStride; idx += blockDim.x) {
    const int hh = idx / kPartialStride, c = idx % kPartialStride;
    float r = 0.0f;
    if (c == 0) {
      r = fac[hh][kWaves];
    } else {
      for (int w = 0; w < kWaves; w++) {
        const float f = fac[hh][w];
        if (wp.at(w, hh, 0) != -INFINITY) r = __builtin_fmaf(wp.at(w, hh, c), f, r);
      }
    }
    partial_ptr(a, b, h * HG + hh, split)[c] = r;
  }
}

// Attention of the HG query heads over one chunk of at most 32 FP16 tokens,
// tokens [t0, t0 + cnt), computed by one wave; the wave's partial (m, l, o) goes to
// its slot of `wp`. Token t0 + i sits in ring slot s0 + i, less W once that reaches
// `wlim` (W for the window, whose token t is in slot t % W; W + 1 for the attention
// sink, in slot W). All loads of the chunk are issued first. Scores: lane l takes
// token l % 32 and channel half l / 32. Weighted values: lane l accumulates
// channels 2l and 2l + 1 over the chunk's tokens.
// With an append folded into the launch (caches without rotation), tokens
// t >= t_old come from the appended rows and are written to the ring.
// With pre-RoPE keys (ROPE), the keys of a chunk starting at a group start position
// (rope_entry >= 0: the position's entry in a.rope_tab) are rotated after loading:
// lane l pairs its channel with the same token's channel 64 away, held by lane l^32.
// Row stride (floats) of the in-group rotary table in shared memory: one 16-byte
// pad per row moves consecutive rows to different banks (lanes read one column of
// 16 different rows at once).
constexpr int kRopeRow = kD + 4;

template <int HG, bool ROPE>
__device__ void window_chunk(const DecodeArgs& a, int b, int h, int t0, int cnt, int s0, int wlim, int t_old,
                             const float (*qf)[kD], const float* expo, const WaveParts& wp, int wave, int lane,
                             int rope_entry, const float* ropein) {
  if (cnt <= 0) {
    if (lane < HG) {
      wp.at(wave, lane, 0) = -INFINITY;
      wp.at(wave, lane, 1) = 0.0f;
    }
    return;
  }
  const size_t row0 = (size_t(b) * a.Hkv + h) * size_t(a.RS);
  const int tl = lane % 32, hf = lane / 32;
  const bool kval = tl < cnt;
  const bool pend = a.app.pending != 0;
  const __half* kin = static_cast<const __half*>(a.app.k);
  const __half* vin = static_cast<const __half*>(a.app.v);
  // Appended token t of this (b, h): row (b, t - t_old, h) of k / v.
  auto in_row = [&](int t) { return ((size_t(b) * a.app.n_max + (t - t_old)) * a.Hkv + h) * kD; };
  const int tk = t0 + (kval ? tl : 0);
  const bool knew = pend && tk >= t_old;
  int kslot = s0 + (kval ? tl : 0);
  if (kslot >= wlim) kslot -= a.W;
  uint4 kr[8];
  {
    const __half* src = knew ? kin + in_row(tk) : a.ringk + (row0 + kslot) * kD;
    const uint4* krow = reinterpret_cast<const uint4*>(src + 64 * hf);
    for (int i = 0; i < 8; i++) kr[i] = krow[i];
  }
  uint32_t vr[kG];
  for (int t = 0; t < kG; t++) {
    const int tt = t0 + (t < cnt ? t : 0);
    int slot = s0 + (t < cnt ? t : 0);
    if (slot >= wlim) slot -= a.W;
    const __half* src = pend && tt >= t_old ? vin + in_row(tt) : a.ringv + (row0 + slot) * kD;
    vr[t] = *reinterpret_cast<const uint32_t*>(src + 2 * lane);
  }

  float kf[64];
  for (int i = 0; i < 8; i++) {
    const half8 k8 = __builtin_bit_cast(half8, kr[i]);
    for (int e = 0; e < 8; e++) kf[8 * i + e] = float(k8[e]);
  }
  if constexpr (ROPE) {
    if (rope_entry >= 0) {
      // angle (t0 + tl) theta_f = base angle of t0 plus in-group angle of tl
      const float* bt = a.rope_tab + size_t(rope_entry) * kD;
      const float* it = ropein + tl * kRopeRow;
      for (int d = 0; d < 64; d++) {
        const float xp = __shfl_xor(kf[d], 32);
        const float c = bt[d] * it[d] - bt[64 + d] * it[64 + d];
        const float sn = bt[64 + d] * it[d] + bt[d] * it[64 + d];
        kf[d] = hf == 0 ? kf[d] * c - xp * sn : kf[d] * c + xp * sn;
      }
    }
  }
  if (pend && t0 + cnt > t_old) {
    // Appended tokens in this chunk: write their keys and values to the ring.
    if (knew && kval) {
      uint4* dst = reinterpret_cast<uint4*>(a.ringk + (row0 + kslot) * kD + 64 * hf);
      for (int i = 0; i < 8; i++) dst[i] = kr[i];
    }
    for (int t = max(0, t_old - t0); t < cnt; t++) {
      int slot = s0 + t;
      if (slot >= wlim) slot -= a.W;
      *reinterpret_cast<uint32_t*>(a.ringv + (row0 + slot) * kD + 2 * lane) = vr[t];
    }
  }
  float p[HG];
  for (int hh = 0; hh < HG; hh++) {
    float x = 0.0f;
    for (int d = 0; d < 64; d++) x = __builtin_fmaf(qf[hh][64 * hf + d], kf[d], x);
    x += __shfl_xor(x, 32);
    const float sc = kval ? x * expo[hh] : -INFINITY;
    float m = sc;
    for (int off = 16; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    p[hh] = kval ? exp2_nonpos(sc - m) : 0.0f;
    float l = p[hh];
    for (int off = 16; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) {
      wp.at(wave, hh, 0) = m;
      wp.at(wave, hh, 1) = l;
    }
  }
  float o0[HG], o1[HG];
  for (int hh = 0; hh < HG; hh++) o0[hh] = o1[hh] = 0.0f;
  for (int t = 0; t < kG; t++) {
    if (t < cnt) {
      const half2v vv = __builtin_bit_cast(half2v, vr[t]);
      const float v0 = float(vv[0]), v1 = float(vv[1]);
      for (int hh = 0; hh < HG; hh++) {
        const float pt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p[hh]), t));
        o0[hh] = __builtin_fmaf(pt, v0, o0[hh]);
        o1[hh] = __builtin_fmaf(pt, v1, o1[hh]);
      }
    }
  }
  for (int hh = 0; hh < HG; hh++) {
    wp.at(wave, hh, 2 + 2 * lane) = o0[hh];
    wp.at(wave, hh, 3 + 2 * lane) = o1[hh];
  }
}

// Kernel-argument lines read at the start of a split workgroup. The fields that
// place the workgroup (the plan's scalars, split counts and order, the sequence
// records, the store) lie in six 64-byte lines of the arguments, and the compiler's
// own scalar reads follow the dependences between them, so that each line's first
// read waits for the one before. One read of each line, all issued together, brings
// them into the scalar cache in one memory round trip (128K-token decode about 2 %
// shorter). The loads complete inside the asm block.
__device__ inline void warm_argument_lines() {
  constexpr unsigned kPlan = offsetof(DecodeArgs, plan), kApp = offsetof(DecodeArgs, app);
  const auto kp = __builtin_amdgcn_kernarg_segment_ptr();
  int t0, t1, t2, t3, t4, t5;
  asm volatile(
      "s_load_dword %0, %6, 0x0\n\t"
      "s_load_dword %1, %6, 0x40\n\t"
      "s_load_dword %2, %6, %7\n\t"
      "s_load_dword %3, %6, %8\n\t"
      "s_load_dword %4, %6, %9\n\t"
      "s_load_dword %5, %6, %10\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=s"(t0), "=s"(t1), "=s"(t2), "=s"(t3), "=s"(t4), "=s"(t5)
      : "s"(kp), "i"(kPlan + offsetof(SplitPlan, seq)), "i"(kPlan + offsetof(SplitPlan, count)),
        "i"(kPlan + offsetof(SplitPlan, use_prefix)),
        "i"(kApp + offsetof(AppendArgs, seq) + offsetof(SeqArgs, inl_valid)));
}

// The bytes of one group block that a lane uses.
template <int BITS, int NJ>
struct GroupRegs {
  uint4 kc0, kc1, vc0, vc1;  // key / value code words (kc1, vc1: 4-bit second half, 3-bit high-bit plane)
  half8 ks, kz;              // key scale / zero of this lane's 8-channel block
  half8 vs[NJ], vz[NJ];      // value scale / zero of this lane's 8 tokens per channel group
};

template <int BITS, int HG, bool ROPE>
// Two waves per SIMD for every instantiation: the 8-head and 4-bit pre-RoPE ones
// would take more than 256 registers and run one wave per SIMD; bounded, the
// compiler fits them in 256 (spilling at most 22 registers at 4 bits, 8 heads),
// which measured 9-21 % faster at 128K tokens.
__global__ __launch_bounds__(256, ((BITS == 4 && ROPE) || HG == 8) ? 2 : 1) void decode_split_kernel(DecodeArgs a) {
  // MFMA columns. Key side: U = 2 * HG column kinds, the fp16 high part of head u at
  // u < HG and the low part of head U - 1 - u at u >= HG (u = column % U), repeated
  // over the 16 columns; the two parts of a score are added across the paired
  // columns. Value side: the same column kinds; each lane computes the high and low
  // parts of p * s_value for its head and one channel group j (j from the column's
  // copy), and the MFMA of a 16-channel block reads, through shared memory, the B
  // operand of that block's channel group. The high and low columns accumulate apart
  // and are added across the pair once, at the end.
  constexpr int U = 2 * HG;
  constexpr int NCOPY = 16 / HG;                // columns per head
  constexpr int NJ = NCOPY >= 4 ? 1 : 4 / NCOPY;  // value channel groups handled per lane
  constexpr int ITEMS = (HG + 3) / 4;         // key-side operand items per lane
  constexpr int NR = 16 / U;                  // column blocks of U (copies of a column kind)
  constexpr int SP = 8 / NR;                  // score slots whose softmax weight a lane computes

  __shared__ float wpart_mem[kWaves * HG * kPartialStride];  // per-wave partials
  __shared__ float qf[HG][kD];
  __shared__ float expo[HG];
  __shared__ union {
    struct {
      // key-side B operands per wave: [kc][k-block][column kind, rotated by
      // (U / 2) * k-block so that neither the writes nor the reads collide in banks]
      half8 b[4][4][U];
    } bk[kWaves];
  } sh;
  // value-side B operands per wave: [k-block][channel group j][column kind, rotated
  // by j so that the eight lanes of a write hit eight different 16-byte bank groups];
  // kind 2 hd + part holds the high (part 0) or low (part 1) half of p * s_value of
  // head hd
  __shared__ half8 vstage[kWaves][4][4][U];
  // softmax weights per wave: [k-block][head][8 slots]; the NR copies of a column
  // kind each compute SP of the 8 and read the rest from here
  __shared__ float pstage[NR > 1 ? kWaves : 1][4][HG][8];
  // Pre-RoPE keys: in-group rotary cos / sin [32][128], and per wave the current
  // group's key scales / zero-points (512 B) and base-angle cos / sin (512 B).
  __shared__ float ropein[ROPE ? kG * kRopeRow : 1];
  __shared__ uint4 ropew[ROPE ? kWaves * 64 : 1];
  const WaveParts wp{wpart_mem, HG * kPartialStride};
  warm_argument_lines();

  // 1-D grid: the split workgroups first, sequence by sequence in the plan's order
  // (each sequence's n_b splits for each kv-head), then wblocks FP16-window
  // workgroups per (sequence, kv-head), which fill the gaps the splits leave.
  const int nsplit_total = a.plan.use_prefix ? a.plan.prefix[a.B] : a.B * a.plan.uniform;
  const int wbase = nsplit_total * a.Hkv;
  const bool tail = int(blockIdx.x) >= wbase;
  int b, h, split, nsb;
  if (tail) {
    const int bh = (int(blockIdx.x) - wbase) / a.wblocks;
    b = bh / a.Hkv;
    h = bh % a.Hkv;
    nsb = splits_of(a.plan, b);
    split = nsb + (int(blockIdx.x) - wbase) % a.wblocks;
  } else {
    const int idx = int(blockIdx.x);
    if (a.plan.older_weight > 0.0f) {
      // split-major: equal split counts for every sequence (one round)
      nsb = a.plan.use_prefix ? a.plan.count[a.plan.seq[0]] : a.plan.uniform;
      const int bh = idx % (a.B * a.Hkv);
      split = idx / (a.B * a.Hkv);
      b = a.plan.use_prefix ? a.plan.seq[bh / a.Hkv] : bh / a.Hkv;
      h = bh % a.Hkv;
    } else if (!a.plan.use_prefix) {
      nsb = a.plan.uniform;
      b = idx / (a.Hkv * nsb);
      const int rem = idx - b * a.Hkv * nsb;
      h = rem / nsb;
      split = rem % nsb;
    } else {
      int lo = 0, hi = a.B;  // largest position p with Hkv * prefix[p] <= idx
      while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (a.Hkv * a.plan.prefix[mid] <= idx) lo = mid;
        else hi = mid;
      }
      b = a.plan.seq[lo];
      nsb = a.plan.prefix[lo + 1] - a.plan.prefix[lo];
      const int rem = idx - a.Hkv * a.plan.prefix[lo];
      h = rem / nsb;
      split = rem % nsb;
    }
  }
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  // Small batches pass every sequence's record in the arguments (the host mirror of
  // the lengths this launch sees), so no workgroup waits on a record load before
  // its first group loads go out.
  const SeqDesc sd = seq_record(a.app.seq, a.seq, b);
  const int T = sd.t_old + sd.n_new, Q = sd.q_new;
  const int ng = Q / kG;

  // This wave's groups.
  int g0 = split * a.gps, g1 = min(ng, g0 + a.gps);
  if (a.plan.older_weight > 0.0f && !tail) {
    // splits [0, nold) take older_weight times the groups of splits [nold, nsb)
    const int nold = (nsb + 1) / 2;
    const float w = a.plan.older_weight;
    const float x = float(ng) / (float(nold) + float(nsb - nold) / w);
    auto bound = [&](int sp) {
      const float v = sp <= nold ? float(sp) * x : float(nold) * x + float(sp - nold) * (x / w);
      return min(ng, int(v + 0.5f));
    };
    g0 = bound(split);
    g1 = split == nsb - 1 ? ng : bound(split + 1);
  }
  const int len = tail ? 0 : max(0, g1 - g0);
  // The waves take the split's groups in turn (wave w: groups g0 + w, g0 + w + 4,
  // ...), so their counts differ by at most one and they reach the partial merge
  // together. Wave-uniform (kept in scalar registers: a paged cache's table entries
  // are then scalar loads, and the loop's waits branch on scalars).
  const int wg0 = __builtin_amdgcn_readfirstlane(g0 + wave);
  const int n = __builtin_amdgcn_readfirstlane(max(0, (len - wave + kWaves - 1) / kWaves));
  auto group_of = [&](int r) { return wg0 + kWaves * r; };  // r-th group of this wave

  // Group r's bytes of this lane, loaded straight into registers.
  auto load_group = [&](int r, GroupRegs<BITS, NJ>& G) {
    const uint8_t* blk = a.store.at(b, h, group_of(r));
    constexpr int CB = kG * kD * BITS / 8;
    G.kc0 = stream_load16(blk + 16 * lane);
    G.vc0 = stream_load16(blk + CB + 16 * lane);
    if constexpr (BITS == 4) {
      G.kc1 = stream_load16(blk + 1024 + 16 * lane);
      G.vc1 = stream_load16(blk + CB + 1024 + 16 * lane);
    } else if constexpr (BITS == 3) {  // the lane's 8 bytes of the 1-bit plane
      const uint2 kh = stream_load8(blk + 1024 + 8 * lane);
      const uint2 vh = stream_load8(blk + CB + 1024 + 8 * lane);
      G.kc1 = make_uint4(kh.x, kh.y, 0u, 0u);
      G.vc1 = make_uint4(vh.x, vh.y, 0u, 0u);
    }
    if constexpr (ROPE) {
      // lanes 0-31: the key scale / zero-point region; lanes 32-63: the rotary
      // cos / sin of the group's start position
      G.ks = lane < 32 ? stream_half8(blk + 2 * CB + 16 * lane)
                       : load_half8(reinterpret_cast<const uint8_t*>(a.rope_tab + size_t(group_of(r)) * kD) +
                                    16 * (lane - 32));
    } else {
      G.ks = stream_half8(blk + 2 * CB + 16 * (lane / 4));
      G.kz = stream_half8(blk + 2 * CB + 256 + 16 * (lane / 4));
    }
    const int kb_ = lane / 16, col_ = lane % 16, u_ = col_ % (2 * HG);
    const int kcopy_ = 2 * (col_ / (2 * HG)) + (u_ < HG ? 0 : 1);
    const int jbase_ = (kcopy_ % (4 / NJ)) * NJ;
    for (int jr = 0; jr < NJ; jr++) {
      G.vs[jr] = stream_half8(blk + 2 * CB + 512 + 16 * (kb_ * 4 + jbase_ + jr));
      G.vz[jr] = stream_half8(blk + 2 * CB + 768 + 16 * (kb_ * 4 + jbase_ + jr));
    }
  };
  // The query entries this lane needs go out first (a few hundred bytes that every
  // workgroup of the kv-head reads, so mostly cache hits), then the first three
  // groups' loads: the query can be prepared as soon as it arrives and the first
  // group computed as soon as its own loads land.
  half8 qraw[ITEMS];
  if (!tail && !a.rotate) {
    for (int it = 0; it < ITEMS; it++)
      qraw[it] = load_half8(reinterpret_cast<const uint8_t*>(
          a.q + (size_t(b) * a.Hq + h * HG + (lane % 4) % HG + 4 * it) * kD + 8 * (lane / 4)));
  }
  GroupRegs<BITS, NJ> R0, R1, R2, R3;
  if (n > 0) {
    load_group(0, R0);
    load_group(min(1, n - 1), R1);
    load_group(min(2, n - 1), R2);
  }

  if constexpr (ROPE) {
    for (int e = threadIdx.x; e < kG * kD / 4; e += blockDim.x)
      reinterpret_cast<float4*>(ropein)[(e / (kD / 4)) * (kRopeRow / 4) + e % (kD / 4)] =
          reinterpret_cast<const float4*>(a.rope_in)[e];
    __syncthreads();
  }

  // The FP16-window workgroup and rotated queries use the shared-memory query
  // preparation; otherwise each wave prepares what its lanes need on its own.
  if (tail || a.rotate) prepare_query<HG>(a, b, h, qf, expo);

  if (tail) {
    // Window workgroup wsub takes chunk 4 * wsub + wave: with an attention sink,
    // chunk 0 is the sink (token 0, ring slot W) and chunk c >= 1 holds tokens
    // [o + Q + 32 (c - 1), ...) of the window; without one, chunk c holds
    // [Q + 32 c, ...). Window token t is in ring slot t % W.
    const int chunk = (split - nsb) * kWaves + wave;
    if (a.sink && chunk == 0) {  // position 0: no rotation
      window_chunk<HG, ROPE>(a, b, h, 0, min(1, T), a.W, a.W + 1, sd.t_old, qf, expo, wp, wave, lane, -1, ropein);
    } else {
      const int t0 = a.sink + Q + (chunk - a.sink) * kG;  // start of group Q / 32 + chunk - sink
      window_chunk<HG, ROPE>(a, b, h, t0, min(kG, T - t0), t0 % a.W, a.W, sd.t_old, qf, expo, wp, wave, lane,
                             Q / kG + chunk - a.sink, ropein);
    }
    // A folded append with inline records: store them as the sequence's state.
    if (a.app.pending && a.app.seq.inl_valid && h == 0 && split == nsb && threadIdx.x == 0)
      a.app.seq.state[b] = sd;
    merge_and_store<HG>(a, b, h, split, wp);
    return;
  }

  // MFMA lane roles: column col = lane % 16, k-block or row block kb = lane / 16.
  const int col = lane % 16, kb = lane / 16;
  const int u = col % U;
  const bool ishi = u < HG;
  const int hd = ishi ? u : U - 1 - u;                  // query head of this column
  const int kcopy = 2 * (col / U) + (ishi ? 0 : 1);     // which copy of the head (0..NCOPY-1)
  const int role = col / U;                             // block of U columns (0..NR-1)
  const int jbase = (kcopy % (4 / NJ)) * NJ;            // first value channel group of the column
  // Key-side operand preparation: channel block cb = lane / 4 (8 channels) and head
  // (lane % 4) % HG + 4 * it. With this mapping the q . z_key sum of a head ends up
  // in exactly the lanes whose MFMA column belongs to that head.
  const int cb = lane / 4, hh0 = (lane % 4) % HG;
  const bool bwriter = (lane % 4) < HG;

  // qreg: this lane's 8 channels of its heads, times softmax_scale * log2(e) and a
  // power of two 2^-e per head that brings the head's largest entry below 1;
  // ex = 2^e of the head of this lane's column.
  float qreg[ITEMS][8];
  float ex;
  if (a.rotate) {
    for (int it = 0; it < ITEMS; it++)
      for (int s = 0; s < 8; s++) qreg[it][s] = qf[hh0 + 4 * it][8 * cb + s];
    ex = expo[hd];
  } else {
    float exo[ITEMS];
    for (int it = 0; it < ITEMS; it++) {
      const half8 qh = qraw[it];
      float m = 0.0f;
      for (int s = 0; s < 8; s++) {
        qreg[it][s] = float(qh[s]) * a.scale_log2;
        m = fmaxf(m, fabsf(qreg[it][s]));
      }
      m = wave_max_rows(row_max_stride4(m));
      int e = 0;
      if (m > 0.0f) frexpf(m, &e);
      for (int s = 0; s < 8; s++) qreg[it][s] = ldexpf(qreg[it][s], -e);
      exo[it] = ldexpf(1.0f, e);
    }
    // High-part columns own their head's exponent (lane % 4 matches); low-part
    // columns take it from the paired column.
    float exh;
    if constexpr (ITEMS == 1) exh = exo[0];
    else exh = hd >= 4 ? exo[1] : exo[0];
    const float exp_ = partner<U>(exh);
    ex = ishi ? exh : exp_;
  }
  // Pre-RoPE keys at up to 4 query heads per kv-head: q of the channel 64 away
  // (lane ^ 32), negated on the lanes that hold the upper channel of a rotary pair.
  // (At 8 heads the query stays unrotated and the keys take the whole angle: the
  // per-group query rotation would not fit in two waves' registers.)
  constexpr bool QROT = ROPE && ITEMS == 1;
  float qpair[8];
  if constexpr (QROT) {
    for (int e = 0; e < 8; e++) {
      const float x = __shfl_xor(qreg[0][e], 32);
      qpair[e] = cb < 8 ? x : -x;
    }
  }
  // q = qh16 + ql16 to about 21 bits (fp16 high part and fp16 residual); the
  // residual is kept for one query item per lane only (two would not fit in two
  // waves' registers, and their low parts come from the fp32 query instead)
  half8 qh16[ITEMS], ql16[ITEMS == 1 ? 1 : 1];
  for (int it = 0; it < ITEMS; it++) qh16[it] = to_half8(qreg[it]);
  if constexpr (ITEMS == 1)
    for (int e = 0; e < 8; e++) ql16[0][e] = _Float16(qreg[0][e] - float(qh16[0][e]));

  float4v oacc[8];
  for (int t = 0; t < 8; t++) oacc[t] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;
  bool started = false;  // wave-uniform: a group's softmax has run
  // Softmax reference with headroom: when a score passes the running reference, the
  // reference moves kRefSlack log2 units above the new maximum, so every weight stays
  // at most 1, the maximum's at least 2^-kRefSlack, and the sums are rescaled only
  // when a score passes the reference again (in the prescaled units of this lane's
  // head: ex is a power of two, so the quotient is exact).
  const float ref_slack = kRefSlack / ex;
  float zacc[NJ];
  for (int jr = 0; jr < NJ; jr++) zacc[jr] = 0.0f;

  // The group loop is software-pipelined: while group r's softmax and value side run,
  // group r+1's key-side scores are computed (its bytes are already in registers)
  // and group r+2's bytes are on their way, so the dependency chains overlap.
  float4v s0, s1;  // key-side scores of the group whose value side runs next

  // Key side, first half: q' = q * s_key per channel as fp16 high + low parts, to
  // shared memory in the MFMA B layout, and q . z_key per head (returned for this
  // lane's column). Issued one group ahead so that its shared-memory round trips
  // overlap the previous group's value side.
  auto key_prep = [&](const GroupRegs<BITS, NJ>& g) -> float {
    float qz[ITEMS];
    for (int it = 0; it < ITEMS; it++) {
      const int hh = hh0 + 4 * it;
      half8 hi, lo;
      if constexpr (ITEMS == 1) {
        // hi = fp16(qh * s); qh * s - hi is exact in fp16 (the rounding error of a
        // product), so one fused fp16 operation forms it and a second adds ql * s
        hi = qh16[it] * g.ks;
        lo = __builtin_elementwise_fma(qh16[it], g.ks, -hi);
        lo = __builtin_elementwise_fma(ql16[0], g.ks, lo);
      } else {
        split_products(qreg[it], qh16[it], g.ks, hi, lo);
      }
      float z = 0.0f;
      for (int s = 0; s < 8; s++) z = __builtin_fmaf(qreg[it][s], float(g.kz[s]), z);
      qz[it] = wave_sum_rows(row_sum_stride4(z));
      if (bwriter) {
        const int rot = (U / 2) * (cb % 4);
        sh.bk[wave].b[cb / 4][cb % 4][(hh + rot) % U] = hi;
        sh.bk[wave].b[cb / 4][cb % 4][(U - 1 - hh + rot) % U] = lo;
      }
    }
    float qzc;
    if constexpr (ITEMS == 1) qzc = qz[0];
    else qzc = hd >= 4 ? qz[1] : qz[0];
    return ishi ? qzc : 0.0f;  // q . z_key enters once, through the high-part column
  };
  // Key side, second half: the high- or low-part sums of the scores of the group's
  // 32 tokens (rows 4*kb + i of token tiles 0 and 1), by column kind.
  auto key_mfma = [&](const GroupRegs<BITS, NJ>& g, float qzc, float4v& r0, float4v& r1) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    r0 = float4v{qzc, qzc, qzc, qzc};
    r1 = r0;
    for (int kc = 0; kc < 4; kc++) {
      const half8 bk = sh.bk[wave].b[kc][kb][(u + (U / 2) * kb) % U];
      r0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(code_operand<BITS>(g.kc0, g.kc1, 2 * kc), bk, r0, 0, 0, 0);
      r1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(code_operand<BITS>(g.kc0, g.kc1, 2 * kc + 1), bk, r1, 0, 0, 0);
    }
  };

  // Pre-RoPE keys: scores of the group's 32 tokens from the dequantized keys
  // z + s * c rotated at their positions n0 + i (n0 = the group's start). The
  // rotation by n0 moves to the query: q . R(n0 + i) k = (R(-n0) q) . R(i) k, so B
  // is R(-n0) q (fp16 high / low columns, staged per group like the plain key
  // operand) and the keys turn by the in-group angles i * theta only, read from the
  // workgroup's table. Lane (token i, k-block kb) holds channels 32 kc + 8 kb + slot
  // for kc = 0..3, so the rotary pair (f, f + 64) of its channel f < 64 sits in
  // operand kc + 2 of the same lane and slot. The rotated key is split into fp16
  // high and low parts, two MFMAs each. The group's scale / zero-point region and
  // its start angle's cos / sin come through this wave's shared memory.
  auto key_rope = [&](const GroupRegs<BITS, NJ>& g, float4v& r0, float4v& r1) {
    // The low parts' residuals x - hi come from one mixed-precision fused operation
    // (fp16 hi times -1 plus the fp32 x; exact, since hi is x truncated to fp16); the
    // opaque -1 keeps the compiler from rewriting it as a conversion and a subtraction.
    float neg1 = -1.0f;
    asm("" : "+v"(neg1));
    uint4* wl = ropew + wave * 64;
    wl[lane] = __builtin_bit_cast(uint4, g.ks);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint8_t* wb = reinterpret_cast<const uint8_t*>(wl);
    const float* bcs = reinterpret_cast<const float*>(wb + 512);  // cos[64] | sin[64] of the start
    if constexpr (QROT) {
      // R(-n0) q on this lane's key-operand slots: channel 8 cb + s pairs with the
      // channel 64 away (held by lane ^ 32, whose q is qpair, sign folded in)
      const int fq = 8 * (cb % 8);
      const float4 c0 = *reinterpret_cast<const float4*>(bcs + fq);
      const float4 c1 = *reinterpret_cast<const float4*>(bcs + fq + 4);
      const float4 n0 = *reinterpret_cast<const float4*>(bcs + 64 + fq);
      const float4 n1 = *reinterpret_cast<const float4*>(bcs + 64 + fq + 4);
      const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float sn[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
      for (int it = 0; it < ITEMS; it++) {
        const int hh = hh0 + 4 * it;
        float qr[8], rr[8];
        for (int e = 0; e < 8; e++) qr[e] = __builtin_fmaf(qpair[e], sn[e], qreg[it][e] * cs[e]);
        const half8 hi = to_half8(qr);
        for (int e = 0; e < 8; e++) rr[e] = __builtin_fmaf(float(hi[e]), neg1, qr[e]);
        const half8 lo = to_half8_rne(rr);
        if (bwriter) {
          const int rot = (U / 2) * (cb % 4);
          sh.bk[wave].b[cb / 4][cb % 4][(hh + rot) % U] = hi;
          sh.bk[wave].b[cb / 4][cb % 4][(U - 1 - hh + rot) % U] = lo;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    r0 = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    r1 = r0;
    for (int kc = 0; kc < 2; kc++) {
      const half8 sa = *reinterpret_cast<const half8*>(wb + 64 * kc + 16 * kb);
      const half8 za = *reinterpret_cast<const half8*>(wb + 256 + 64 * kc + 16 * kb);
      const half8 sb = *reinterpret_cast<const half8*>(wb + 64 * (kc + 2) + 16 * kb);
      const half8 zb = *reinterpret_cast<const half8*>(wb + 256 + 64 * (kc + 2) + 16 * kb);
      const int f0 = 32 * kc + 8 * kb;  // frequency of slot 0
      const half8 bka = sh.bk[wave].b[kc][kb][(u + (U / 2) * kb) % U];
      const half8 bkb = sh.bk[wave].b[kc + 2][kb][(u + (U / 2) * kb) % U];
      for (int tile = 0; tile < 2; tile++) {
        const float* it = ropein + (16 * tile + lane % 16) * kRopeRow;
        const half8 ca = code_operand<BITS>(g.kc0, g.kc1, 2 * kc + tile);
        const half8 cb = code_operand<BITS>(g.kc0, g.kc1, 2 * (kc + 2) + tile);
        float ya[8], yb[8];
        for (int s2 = 0; s2 < 8; s2++) {
          const float ci = it[f0 + s2], si = it[64 + f0 + s2];
          float c = ci, sn = si;  // in-group angle; with QROT the start angle is in B
          if constexpr (!QROT) {
            const float bc = bcs[f0 + s2], bs = bcs[64 + f0 + s2];
            c = bc * ci - bs * si;
            sn = bs * ci + bc * si;
          }
          const float xa = __builtin_fmaf(float(ca[s2]), float(sa[s2]), float(za[s2]));
          const float xb = __builtin_fmaf(float(cb[s2]), float(sb[s2]), float(zb[s2]));
          ya[s2] = xa * c - xb * sn;
          yb[s2] = xb * c + xa * sn;
        }
        // fp16 high parts (round toward zero) and the fp32 residuals as low parts
        const half8 ah = to_half8(ya), bh = to_half8(yb);
        float ra[8], rb[8];
        for (int s2 = 0; s2 < 8; s2++) {
          ra[s2] = __builtin_fmaf(float(ah[s2]), neg1, ya[s2]);
          rb[s2] = __builtin_fmaf(float(bh[s2]), neg1, yb[s2]);
        }
        const half8 al = to_half8_rne(ra), bl = to_half8_rne(rb);
        float4v r = tile == 0 ? r0 : r1;
        r = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bka, r, 0, 0, 0);
        r = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bka, r, 0, 0, 0);
        r = __builtin_amdgcn_mfma_f32_16x16x32_f16(bh, bkb, r, 0, 0, 0);
        r = __builtin_amdgcn_mfma_f32_16x16x32_f16(bl, bkb, r, 0, 0, 0);
        if (tile == 0) r0 = r;
        else r1 = r;
      }
    }
  };

  // Value side, first half: online softmax of the group's scores, B = p * s_value as
  // fp16 high and low parts to shared memory, sum p * z_value.
  auto value_prep = [&](const GroupRegs<BITS, NJ>& g, const float4v& r0, const float4v& r1) {
    // This lane's score slots SP * role + i (slot k: row k % 4 of tile k / 4), the
    // high and low parts added across the paired columns (the pair shares the role).
    float x[SP];
    for (int i = 0; i < SP; i++) {
      float v = i < 4 ? r0[i] : r1[i - 4];
      for (int rr = 1; rr < NR; rr++) {
        const int k = SP * rr + i;
        v = role == rr ? (k < 4 ? r0[k] : r1[k - 4]) : v;
      }
      x[i] = v + partner<U>(v);
    }
    // Online softmax. Scores stay in the prescaled units S (log2 units are ex * S);
    // the running reference m_run (at least every score so far) is kept in the same
    // units. The cross-lane max is only formed when some score exceeds it.
    float mloc = x[0];
    for (int i = 1; i < SP; i++) mloc = fmaxf(mloc, x[i]);
    if (__ballot(mloc > m_run)) {
      const float hmax = row_class_max<NR>(wave_max_rows(mloc));
      const float m_new = hmax > m_run ? hmax + ref_slack : m_run;
      if (started) {  // before the first group the sums are zero
        const float alpha = exp2_nonpos(ex * (m_run - m_new));
        for (int t = 0; t < 8; t++) oacc[t] *= alpha;
        l_run *= alpha;
        for (int jr = 0; jr < NJ; jr++) zacc[jr] *= alpha;
      }
      m_run = m_new;
    }
    started = true;
    const float negm = -ex * m_run;
    float p[8];
    if constexpr (NR == 1) {
      for (int i = 0; i < 8; i++) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], ex, negm));
        l_run += p[i];
      }
    } else {
      // each copy computes SP weights; all 8 come back through shared memory
      float pl[SP];
      for (int i = 0; i < SP; i++) {
        pl[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], ex, negm));
        l_run += pl[i];
      }
      float* ps = &pstage[wave][kb][hd][0];
      if (ishi) {  // the low-part column of the pair holds the same weights
        if constexpr (SP == 4) *reinterpret_cast<float4*>(ps + 4 * role) = make_float4(pl[0], pl[1], pl[2], pl[3]);
        else if constexpr (SP == 2) *reinterpret_cast<float2*>(ps + 2 * role) = make_float2(pl[0], pl[1]);
        else ps[role] = pl[0];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float4 pa = *reinterpret_cast<const float4*>(ps), pb = *reinterpret_cast<const float4*>(ps + 4);
      p[0] = pa.x; p[1] = pa.y; p[2] = pa.z; p[3] = pa.w;
      p[4] = pb.x; p[5] = pb.y; p[6] = pb.z; p[7] = pb.w;
    }
    // B = p * s_value (fp16 high + low parts) of this lane's head and channel
    // groups, plus sum p * z_value.
    const half8 ph = to_half8(p);
    for (int jr = 0; jr < NJ; jr++) {
      half8 bvh, bvl;
      split_products(p, ph, g.vs[jr], bvh, bvl);
      const int j = jbase + jr;
      vstage[wave][kb][j][(2 * hd + j) % U] = bvh;
      vstage[wave][kb][j][(2 * hd + 1 + j) % U] = bvl;
      float z = zacc[jr];
      for (int s = 0; s < 8; s++) z = __builtin_fmaf(p[s], float(g.vz[jr][s]), z);
      zacc[jr] = z;
    }
  };
  // Value side, second half: one MFMA per 16-channel block t against the B operand of
  // its channel group t / 2; high- and low-part columns accumulate apart and are
  // added across the paired columns at the end.
  auto value_mfma = [&](const GroupRegs<BITS, NJ>& g) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int kind = 2 * hd + (ishi ? 0 : 1);
    for (int t = 0; t < 8; t++) {
      const int j = t / 2;
      const half8 bv = vstage[wave][kb][j][(kind + j) % U];
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(code_operand<BITS>(g.vc0, g.vc1, t), bv, oacc[t], 0, 0, 0);
    }
  };
  auto value_side = [&](const GroupRegs<BITS, NJ>& g, const float4v& r0, const float4v& r1) {
    value_prep(g, r0, r1);
    value_mfma(g);
  };

  // Four register sets R0..R3 take the roles (group r, r+1, r+2, r+3) in turn, so nothing
  // is copied between them: the loads of group r+3, issued in stage r, are first
  // used in stage r+2 and have two stages to land. Loads past the last group
  // re-read the last group (same bytes; always issued, so the count of loads in
  // flight is the same in every stage).
  auto stage = [&](int r, const GroupRegs<BITS, NJ>& Gr, const GroupRegs<BITS, NJ>& Gr1,
                   GroupRegs<BITS, NJ>& Gr3) {
    load_group(min(r + 3, n - 1), Gr3);
    if constexpr (ROPE) {
      value_prep(Gr, s0, s1);
      key_rope(Gr1, s0, s1);
      value_mfma(Gr);
    } else {
      const float qzn = key_prep(Gr1);
      value_prep(Gr, s0, s1);
      key_mfma(Gr1, qzn, s0, s1);
      value_mfma(Gr);
    }
  };
  if constexpr (ROPE && !QROT) {
    // B = q for every group: the high / low split of q times a unit scale.
    GroupRegs<BITS, NJ> unit;
    for (int e = 0; e < 8; e++) {
      unit.ks[e] = _Float16(1.0f);
      unit.kz[e] = _Float16(0.0f);
    }
    (void)key_prep(unit);
  }
  if (n > 0) {
    if constexpr (ROPE) key_rope(R0, s0, s1);
    else key_mfma(R0, key_prep(R0), s0, s1);
    int r = 0;
    for (; r + 4 < n; r += 4) {
      stage(r, R0, R1, R3);
      stage(r + 1, R1, R2, R0);
      stage(r + 2, R2, R3, R1);
      stage(r + 3, R3, R0, R2);
    }
    // n - 1 - r (0 to 3) stages remain; the last group's value side closes.
    if (r + 1 < n) {
      stage(r, R0, R1, R3);
      if (r + 2 < n) {
        stage(r + 1, R1, R2, R0);
        if (r + 3 < n) {
          stage(r + 2, R2, R3, R1);
          value_side(R3, s0, s1);
        } else {
          value_side(R2, s0, s1);
        }
      } else {
        value_side(R1, s0, s1);
      }
    } else {
      value_side(R0, s0, s1);
    }
  }

  // Wave partial: sums over the four row blocks.
  const float l_tot = row_class_sum<NR>(wave_sum_rows(l_run));
  float zs[NJ];
  for (int jr = 0; jr < NJ; jr++) zs[jr] = wave_sum_rows(zacc[jr]);
  if (kb == 0 && kcopy == 0) {
    wp.at(wave, hd, 0) = m_run == -INFINITY ? -INFINITY : ex * m_run;
    wp.at(wave, hd, 1) = l_tot;
  }
  for (int t = 0; t < 8; t++) {
    float o[4];
    for (int i = 0; i < 4; i++) o[i] = oacc[t][i] + partner<U>(oacc[t][i]);  // high + low columns
    if (kcopy == (t / 2) / NJ)
      for (int i = 0; i < 4; i++) wp.at(wave, hd, 2 + 16 * t + 4 * kb + i) = o[i] + zs[(t / 2) % NJ];
  }
  merge_and_store<HG>(a, b, h, split, wp);
}

// out[b][hq][d] = sum_i o_i[d] 2^(m_i - M) / sum_i l_i 2^(m_i - M) over the
// partials of one (sequence, query head), M = max_i m_i. One workgroup per (query
// head, sequence, 16-channel slice): 16 slices of 16 threads each merge a strided
// subset of the partials with a running maximum (all of a thread's loads are
// independent, so the partials are read in one memory round trip), then the slices
// are merged in shared memory.
// The same for the combine: the lines holding the partial and output pointers, row
// b's split count and the plan's scalars, read together. The plan follows the
// pointers and Hq in the parameter list. Split counts exist for the first
// kInlineSeqs sequences only (larger batches use the plan's uniform count), so the
// read stays inside the arguments for any b.
constexpr unsigned kCombinePlanOffset = 2 * sizeof(void*) + sizeof(int);
__device__ inline void warm_combine_lines(int b) {
  typedef __attribute__((address_space(4))) const char* karg_t;
  const karg_t kp = (karg_t)__builtin_amdgcn_kernarg_segment_ptr();
  int t0, t1, t2;
  asm volatile(
      "s_load_dword %0, %3, 0x0\n\t"
      "s_load_dword %1, %4, 0x0\n\t"
      "s_load_dword %2, %3, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=s"(t0), "=s"(t1), "=s"(t2)
      : "s"(kp), "s"(kp + kCombinePlanOffset + offsetof(SplitPlan, count) + 4 * min(b, kInlineSeqs - 1)),
        "i"(kCombinePlanOffset + offsetof(SplitPlan, use_prefix)));
}

constexpr int kCombineThreads = 256;
constexpr int kCombineChannels = 16;
constexpr int kCombineSlices = kCombineThreads / kCombineChannels;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ part,
                                                                  float* __restrict__ out, int Hq,
                                                                  const SplitPlan plan, int wblocks) {
  __shared__ float sm[kCombineSlices], sl[kCombineSlices];
  __shared__ float so[kCombineSlices][kCombineChannels];
  const int hq = blockIdx.x, b = blockIdx.y, d0 = blockIdx.z * kCombineChannels, tid = threadIdx.x;
  warm_combine_lines(b);
  const int dl = tid % kCombineChannels, slice = tid / kCombineChannels;
  const int nparts = splits_of(plan, b) + wblocks;
  const float* p = part + (size_t(b) * Hq + hq) * size_t(plan.pstride) * kPartialStride;

  // Batches of kBatch partials per thread: all loads of a batch are issued before
  // any of them is used, and the merge is branch-free (empty partials have m = -inf).
  constexpr int kBatch = 8;
  float m = -INFINITY, l = 0.0f, o = 0.0f;
  for (int i0 = slice; i0 < nparts; i0 += kCombineSlices * kBatch) {
    float mi[kBatch], li[kBatch], oi[kBatch];
    for (int u = 0; u < kBatch; u++) {
      const int i = i0 + u * kCombineSlices;
      const float* pi = p + size_t(i < nparts ? i : 0) * kPartialStride;
      mi[u] = i < nparts ? pi[0] : -INFINITY;
      li[u] = pi[1];
      oi[u] = pi[2 + d0 + dl];
    }
    for (int u = 0; u < kBatch; u++) {
      const float mn = fmaxf(m, mi[u]);
      const float a = m == -INFINITY ? 0.0f : exp2_nonpos(m - mn);
      const float c = mi[u] == -INFINITY ? 0.0f : exp2_nonpos(mi[u] - mn);
      l = l * a + li[u] * c;
      o = o * a + oi[u] * c;
      m = mn;
    }
  }
  if (dl == 0) {
    sm[slice] = m;
    sl[slice] = l;
  }
  so[slice][dl] = o;
  __syncthreads();
  if (slice == 0) {
    float M = -INFINITY;
    for (int s2 = 0; s2 < kCombineSlices; s2++) M = fmaxf(M, sm[s2]);
    float L = 0.0f, acc = 0.0f;
    for (int s2 = 0; s2 < kCombineSlices; s2++) {
      if (sm[s2] == -INFINITY) continue;
      const float w = exp2_nonpos(sm[s2] - M);
      L += sl[s2] * w;
      acc += so[s2][dl] * w;
    }
    out[(size_t(b) * Hq + hq) * kD + d0 + dl] = acc / L;
  }
}

// Many (sequence, query head) rows with few partials each (large batches): one wave
// merges one row over all 128 channels (two per lane, 8-byte loads), four rows per
// workgroup, so the whole merge is one round of workgroups instead of one workgroup
// per 16-channel slice of every row.
constexpr int kRowWaves = 4;
// Rows from which the one-wave-per-row merge is used.
constexpr int kRowsCombineMin = 512;

__global__ __launch_bounds__(64 * kRowWaves) void combine_rows_kernel(const float* __restrict__ part,
                                                                      float* __restrict__ out, int Hq, int rows,
                                                                      const SplitPlan plan, int wblocks) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int row = int(blockIdx.x) * kRowWaves + wave;  // b * Hq + hq
  if (row >= rows) return;
  const int nparts = splits_of(plan, row / Hq) + wblocks;
  const float* p = part + size_t(row) * size_t(plan.pstride) * kPartialStride;
  constexpr int kBatch = 8;
  float m = -INFINITY, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int i0 = 0; i0 < nparts; i0 += kBatch) {
    float mi[kBatch], li[kBatch];
    float2 oi[kBatch];
    for (int u = 0; u < kBatch; u++) {
      const int i = i0 + u;
      const float* pi = p + size_t(i < nparts ? i : 0) * kPartialStride;
      mi[u] = i < nparts ? pi[0] : -INFINITY;
      li[u] = pi[1];
      oi[u] = *reinterpret_cast<const float2*>(pi + 2 + 2 * lane);
    }
    for (int u = 0; u < kBatch; u++) {
      const float mn = fmaxf(m, mi[u]);
      const float a = m == -INFINITY ? 0.0f : exp2_nonpos(m - mn);
      const float c = mi[u] == -INFINITY ? 0.0f : exp2_nonpos(mi[u] - mn);
      l = l * a + li[u] * c;
      o0 = o0 * a + oi[u].x * c;
      o1 = o1 * a + oi[u].y * c;
      m = mn;
    }
  }
  *reinterpret_cast<float2*>(out + size_t(row) * kD + 2 * lane) = make_float2(o0 / l, o1 / l);
}

template <int BITS, int HG, bool ROPE>
int resident_blocks_of() {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<BITS, HG, ROPE>, 256, 0) !=
      hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return per_cu;
}

// With profiling events the launch goes through hipExtLaunchKernelGGL, which sets the
// events to the kernel's own start and end timestamps (those of its dispatch packet,
// as a kernel trace reports them). Events recorded on the stream around the launch
// would instead take their start stamp as soon as the previous kernel was dispatched,
// so the interval would include the tail of that kernel.
template <int BITS, int HG, bool ROPE>
hipError_t launch_split(const DecodeArgs& a, int B, hipStream_t stream, hipEvent_t prof_start,
                        hipEvent_t prof_stop) {
  const int nsplit_total = a.plan.use_prefix ? a.plan.prefix[B] : B * a.plan.uniform;
  const dim3 grid((nsplit_total + B * a.wblocks) * a.Hkv);
  if (prof_start || prof_stop)
    hipExtLaunchKernelGGL((decode_split_kernel<BITS, HG, ROPE>), grid, dim3(256), 0, stream, prof_start, prof_stop, 0,
                          a);
  else
    hipLaunchKernelGGL((decode_split_kernel<BITS, HG, ROPE>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Rotary cos / sin tables of a pre-RoPE cache, computed once in fp64 and stored in
// fp32: entry g holds cos(p theta_f), sin(p theta_f) at the group start position
// p = o + 32 g, and the in-group table holds them at p = i, i = 0..31, with
// theta_f = base^(-f / 64), f = 0..63 (the standard rotary embedding over the
// channel pairs f, f + 64).
__global__ void rope_table_kernel(float* __restrict__ tab, float* __restrict__ in_tab, int entries, int o,
                                  double base) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int f = idx % 64;
  const double theta = pow(base, -double(f) / 64.0);
  if (idx < entries * 64) {
    const int g = idx / 64;
    const double ang = double(o + kG * g) * theta;
    tab[size_t(g) * kD + f] = float(cos(ang));
    tab[size_t(g) * kD + 64 + f] = float(sin(ang));
  } else if (idx < entries * 64 + kG * 64) {
    const int i = (idx - entries * 64) / 64;
    const double ang = double(i) * theta;
    in_tab[i * kD + f] = float(cos(ang));
    in_tab[i * kD + 64 + f] = float(sin(ang));
  }
}

hipError_t launch_rope_tables(const Layout& L, uint8_t* base, double rope_base, hipStream_t stream) {
  const int total = L.rope_entries * 64 + kG * 64;
  hipLaunchKernelGGL(rope_table_kernel, dim3((total + 255) / 256), dim3(256), 0, stream,
                     reinterpret_cast<float*>(base + L.rope_off), reinterpret_cast<float*>(base + L.ropein_off),
                     L.rope_entries, L.sink, rope_base);
  return hipGetLastError();
}

template <bool ROPE>
int resident_blocks_for(int bits, int hg) {
  if (bits == 2)
    return hg == 1 ? resident_blocks_of<2, 1, ROPE>() : hg == 2 ? resident_blocks_of<2, 2, ROPE>()
           : hg == 4 ? resident_blocks_of<2, 4, ROPE>() : resident_blocks_of<2, 8, ROPE>();
  if (bits == 3)
    return hg == 1 ? resident_blocks_of<3, 1, ROPE>() : hg == 2 ? resident_blocks_of<3, 2, ROPE>()
           : hg == 4 ? resident_blocks_of<3, 4, ROPE>() : resident_blocks_of<3, 8, ROPE>();
  return hg == 1 ? resident_blocks_of<4, 1, ROPE>() : hg == 2 ? resident_blocks_of<4, 2, ROPE>()
         : hg == 4 ? resident_blocks_of<4, 4, ROPE>() : resident_blocks_of<4, 8, ROPE>();
}

int decode_blocks_per_cu(int bits, int hg, int rope) {
  return rope ? resident_blocks_for<true>(bits, hg) : resident_blocks_for<false>(bits, hg);
}

int device_compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return cus;
}

template <int BITS, bool ROPE>
hipError_t launch_split_hg(const DecodeArgs& a, int hg, int B, hipStream_t stream, hipEvent_t ps, hipEvent_t pe) {
  return hg == 1   ? launch_split<BITS, 1, ROPE>(a, B, stream, ps, pe)
         : hg == 2 ? launch_split<BITS, 2, ROPE>(a, B, stream, ps, pe)
         : hg == 4 ? launch_split<BITS, 4, ROPE>(a, B, stream, ps, pe)
                   : launch_split<BITS, 8, ROPE>(a, B, stream, ps, pe);
}

template <bool ROPE>
hipError_t launch_split_for(const DecodeArgs& a, int bits, int hg, int B, hipStream_t stream, hipEvent_t ps,
                            hipEvent_t pe) {
  return bits == 2   ? launch_split_hg<2, ROPE>(a, hg, B, stream, ps, pe)
         : bits == 3 ? launch_split_hg<3, ROPE>(a, hg, B, stream, ps, pe)
                     : launch_split_hg<4, ROPE>(a, hg, B, stream, ps, pe);
}

hipError_t launch_decode(const Layout& L, uint8_t* base, const SeqDesc* seq, const AppendArgs& app, const void* q,
                         float* out, int32_t groups_per_split, const SplitPlan& plan, float scale_log2, int rotate,
                         hipStream_t stream,
                         hipEvent_t prof_start, hipEvent_t prof_stop) {
  DecodeArgs a;
  a.store = group_store(L, base);
  a.ringk = reinterpret_cast<__half*>(base + L.ringk_off);
  a.ringv = reinterpret_cast<__half*>(base + L.ringv_off);
  a.seq = seq;
  a.q = static_cast<const __half*>(q);
  a.part = reinterpret_cast<float*>(base + L.part_off);
  a.Hkv = L.Hkv;
  a.Hq = L.Hq;
  a.W = L.W;
  a.RS = L.RS;
  a.sink = L.sink;
  a.gps = groups_per_split;
  a.plan = plan;
  a.app = app;
  a.wblocks = L.win_blocks;
  a.B = L.B;
  a.rotate = rotate;
  a.scale_log2 = scale_log2;
  a.rope_tab = L.rope ? reinterpret_cast<const float*>(base + L.rope_off) : nullptr;
  a.rope_in = L.rope ? reinterpret_cast<const float*>(base + L.ropein_off) : nullptr;
  const int hg = L.Hq / L.Hkv;
  hipError_t e;
  e = L.rope ? launch_split_for<true>(a, L.bits, hg, L.B, stream, prof_start, prof_stop)
             : launch_split_for<false>(a, L.bits, hg, L.B, stream, prof_start, prof_stop);
  if (e != hipSuccess) return e;
  return launch_combine(a.part, out, L.Hq, L.B, plan, L.win_blocks, stream);
}

hipError_t launch_combine(const float* part, float* out, int Hq, int B, const SplitPlan& plan, int wblocks,
                          hipStream_t stream) {
  const int64_t rows = int64_t(B) * Hq;
  if (rows >= kRowsCombineMin && rows <= INT32_MAX)
    hipLaunchKernelGGL(combine_rows_kernel, dim3(unsigned((rows + kRowWaves - 1) / kRowWaves)), dim3(64 * kRowWaves),
                       0, stream, part, out, Hq, int(rows), plan, wblocks);
  else
    hipLaunchKernelGGL(combine_kernel, dim3(Hq, B, kD / kCombineChannels), dim3(kCombineThreads), 0, stream, part,
                       out, Hq, plan, wblocks);
  return hipGetLastError();
}

}  // namespace kvq
